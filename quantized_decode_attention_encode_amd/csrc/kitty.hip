// kitty.hip - Kitty caches ("Changelog" v0.11.0, Kitty): key channels ranked by their running
// variance, the top n_hi quantized at 4 bits and the rest at 2 bits in KIVI's per-channel
// groups of 32 tokens, values kept in fp16 ("Algorithm Overview": Kitty stores fp16 values).
//
// Encode (five launches over the records a prefill, encode or window flush adds):
//   kitty_stats_kernel   one wave per record: each channel's exact sums over the record's
//                        32 tokens, s1 = sum X and s2 = sum X^2 with X = x * 2^24 (an integer
//                        for every finite fp16 x; |X| < 2^40, so over the at most 2^22 tokens
//                        of a Kitty sequence s1 fits int64, s2 and n * s2 uint128), staged in
//                        the record's value area.
//   kitty_seg/top/fix    running sums up to each record's end (the sequence's stored sums plus
//                        every earlier group) written back over the staged group sums, and the
//                        new totals into the sequence's state: segment totals, one walk over
//                        them per (b, h), then every segment's records (a two-level scan; the
//                        integer sums are exact in any order).
//   kitty_encode_kernel  one wave per record: n * s2 - s1^2 (n^2 times the variance, exact in
//                        128 bits) ranks the channels (the larger first, the lower index on
//                        ties; compared through order-preserving fp32 images, exactly where the
//                        images are equal); the top n_hi take 4-bit groups, the rest 2-bit ones, by KIVI's
//                        min/max rule (quant.h); codes, params and the slot table are written,
//                        then the fp16 value rows over the staging.
// Decode: kitty_decode_kernel, split-K over the records and window units of each (b, h_kv) with
// an fp32 online softmax in base-2 units; the last split of each (b, h_kv) to finish merges the
// splits' partials (merge_splits of the KIVI decode).
//   key lanes   lane (t = l/2, half = l%2): token t, the code chunks k = 2j + half; each code
//               multiplies q~[slot] = q[channel] * scale[slot] (formed once per record in LDS);
//               the zero terms add up to beta = q . zero, one number per record and head.
//   value lanes lane (octet o, token subset): 16-byte loads of 8 fp16 values of the tokens
//               tg, tg + 64/(D/8), ...; the subsets meet at the end of the wave.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "decode_kernel.h"  // dpp, wave_sync, split-partial stores and the in-kernel merge
#include "kernels.h"
#include "layout.h"
#include "quant.h"

namespace kvq {
namespace {

typedef unsigned __int128 u128;
constexpr int kHB = 4, kLB = 2;  // high and low key widths
constexpr int kDecWaves = 4;

// x * 2^24 for the finite fp16 x with bits hb, exactly
__device__ __forceinline__ int64_t fp16_fixed(uint32_t hb) {
  const int ex = (hb >> 10) & 31;
  const int64_t man = hb & 1023;
  const int64_t mag = ex ? ((man | 1024) << (ex - 1)) : man;
  return (hb & 0x8000) ? -mag : mag;
}

__device__ __forceinline__ u128 square(int64_t x) {
  const uint64_t a = uint64_t(x < 0 ? -x : x);
  return u128(a) * a;
}

// An fp32 image of a non-negative 128-bit integer that keeps its order: the leading 24 bits,
// truncated, at the leading bit's power of two. x < y gives f(x) <= f(y), so f(x) < f(y) decides
// x < y, and only equal images need the exact comparison.
__device__ __forceinline__ float order_image(u128 x) {
  const uint64_t hi = uint64_t(x >> 64), lo = uint64_t(x);
  if ((hi | lo) == 0) return 0.0f;
  const int top = hi ? 127 - __clzll(hi) : 63 - __clzll(lo);  // the leading one's bit
  const uint32_t m = uint32_t(top >= 23 ? (x >> (top - 23)) : (x << (23 - top)));  // 24 bits, bit 23 set
  return __uint_as_float((uint32_t(top + 127) << 23) | (m & 0x7FFFFFu));
}

__device__ __forceinline__ uint64_t* staging(uint8_t* buf, const Layout& L, int b, int h, int j) {
  return reinterpret_cast<uint64_t*>(buf + L.record(b, h, j) + kitty_off_values(L.D, L.nhi));
}

// Reductions over the wave in every lane, without LDS: DPP inside each 16-lane row, then the
// gfx950 row swaps (with both operands equal, permlane32_swap yields rows (0,1,0,1) and
// (2,3,2,3), permlane16_swap rows (0,0,2,2) and (1,1,3,3)).
__device__ __forceinline__ float wave_sum_all(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kRowRor8>(v);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ float wave_max_all(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kRowRor8>(v));
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}


// ---------------------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------------------
// seq.a = first record, seq.b = records, seq.c = token of K[b][h] where the first one starts.
template <int D>
__global__ __launch_bounds__(64) void kitty_stats_kernel(uint8_t* __restrict__ buf, Layout L,
                                                         const __half* __restrict__ K, int64_t ld_tok, PerSeq seq) {
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (x >= seq.b[b]) return;
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(K) +
                        ((int64_t(b) * L.Hkv + h) * ld_tok + seq.c[b] + int64_t(x) * kGroup) * D + lane * E;
  int64_t s1[E];
  u128 s2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s1[e] = 0;
    s2[e] = 0;
  }
#pragma unroll 8
  for (int t = 0; t < kGroup; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t X = fp16_fixed(src[t * D + e]);
      s1[e] += X;
      s2[e] += square(X);
    }
  uint64_t* st = staging(buf, L, b, h, seq.a[b] + x);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    st[c] = uint64_t(s1[e]);
    st[D + c] = uint64_t(s2[e]);
    st[2 * D + c] = uint64_t(s2[e] >> 64);
  }
}

// Running sums, in three launches (integer sums are exact in any order): each segment of
// kSeg records sums its records' group sums (kitty_seg_kernel, the total staged after the group
// sums of the segment's first record); one wave per (b, h) turns the totals into exclusive
// prefixes, starting from the sequence's stored sums (none before its first record: a
// sequence's first encode starts from zero, whatever the buffer held), and stores the new
// totals (kitty_top_kernel); each segment then rewrites its records' staged group sums as
// running sums up to their ends (kitty_fix_kernel).
constexpr int kSeg = 16;

__device__ __forceinline__ void load_sums(const uint64_t* p, int c, int D, int64_t& s1, u128& s2) {
  s1 = int64_t(p[c]);
  s2 = u128(p[D + c]) | (u128(p[2 * D + c]) << 64);
}
__device__ __forceinline__ void store_sums(uint64_t* p, int c, int D, int64_t s1, u128 s2) {
  p[c] = uint64_t(s1);
  p[D + c] = uint64_t(s2);
  p[2 * D + c] = uint64_t(s2 >> 64);
}

template <int D>
__global__ __launch_bounds__(64) void kitty_seg_kernel(uint8_t* __restrict__ buf, Layout L, PerSeq seq) {
  const int sg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = seq.b[b], x0 = sg * kSeg;
  if (x0 >= n) return;
  constexpr int E = D / 64;
  const int lane = threadIdx.x, j0 = seq.a[b], x1 = min(n, x0 + kSeg);
  int64_t t1[E];
  u128 t2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    t1[e] = 0;
    t2[e] = 0;
  }
#pragma unroll 4
  for (int x = x0; x < x1; ++x) {
    const uint64_t* p = staging(buf, L, b, h, j0 + x);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int64_t a1;
      u128 a2;
      load_sums(p, lane * E + e, D, a1, a2);
      t1[e] += a1;
      t2[e] += a2;
    }
  }
  uint64_t* tot = staging(buf, L, b, h, j0 + x0) + 3 * D;
#pragma unroll
  for (int e = 0; e < E; ++e) store_sums(tot, lane * E + e, D, t1[e], t2[e]);
}

template <int D>
__global__ __launch_bounds__(64) void kitty_top_kernel(uint8_t* __restrict__ buf, Layout L, PerSeq seq) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = seq.b[b];
  if (n == 0) return;
  constexpr int E = D / 64;
  const int lane = threadIdx.x, j0 = seq.a[b];
  uint64_t* base = reinterpret_cast<uint64_t*>(buf + L.kstats(b, h));
  int64_t r1[E];
  u128 r2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (j0 == 0) {
      r1[e] = 0;
      r2[e] = 0;
    } else {
      load_sums(base, lane * E + e, D, r1[e], r2[e]);
    }
  }
#pragma unroll 4
  for (int x0 = 0; x0 < n; x0 += kSeg) {
    uint64_t* tot = staging(buf, L, b, h, j0 + x0) + 3 * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int64_t a1;
      u128 a2;
      load_sums(tot, lane * E + e, D, a1, a2);
      store_sums(tot, lane * E + e, D, r1[e], r2[e]);  // the segment's exclusive prefix
      r1[e] += a1;
      r2[e] += a2;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) store_sums(base, lane * E + e, D, r1[e], r2[e]);
}

template <int D>
__global__ __launch_bounds__(64) void kitty_fix_kernel(uint8_t* __restrict__ buf, Layout L, PerSeq seq) {
  const int sg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = seq.b[b], x0 = sg * kSeg;
  if (x0 >= n) return;
  constexpr int E = D / 64;
  const int lane = threadIdx.x, j0 = seq.a[b], x1 = min(n, x0 + kSeg);
  const uint64_t* pre = staging(buf, L, b, h, j0 + x0) + 3 * D;
  int64_t r1[E];
  u128 r2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) load_sums(pre, lane * E + e, D, r1[e], r2[e]);
#pragma unroll 4
  for (int x = x0; x < x1; ++x) {
    uint64_t* p = staging(buf, L, b, h, j0 + x);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int64_t a1;
      u128 a2;
      load_sums(p, lane * E + e, D, a1, a2);
      r1[e] += a1;
      r2[e] += a2;
      store_sums(p, lane * E + e, D, r1[e], r2[e]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void kitty_encode_kernel(uint8_t* __restrict__ buf, Layout L,
                                                          const __half* __restrict__ K, const __half* __restrict__ V,
                                                          int64_t ld_tok, PerSeq seq) {
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (x >= seq.b[b]) return;
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const int j = seq.a[b] + x;
  const int nhi = L.nhi, nhc = nhi / 16, W = kitty_words(D, nhi);
  uint8_t* rec = buf + L.record(b, h, j);
  const int64_t row0 = ((int64_t(b) * L.Hkv + h) * ld_tok + seq.c[b] + int64_t(x) * kGroup) * D;
  __shared__ u128 key[D];
  __shared__ float fkey[D];
  __shared__ uint8_t cb[kGroup][D];  // codes by (token, slot)

  // the key tile: the lane's channels over the 32 tokens
  float kx[kGroup][E];
#pragma unroll
  for (int t = 0; t < kGroup; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) kx[t][e] = __half2float(K[row0 + int64_t(t) * D + lane * E + e]);
  // n * s2 - s1^2 from the running sums at the group's end (staged in the value area)
  const uint64_t* st = reinterpret_cast<const uint64_t*>(rec + kitty_off_values(D, nhi));
  const uint64_t n = uint64_t(j + 1) * kGroup;
  u128 my[E];
  float myf[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    const int64_t s1 = int64_t(st[c]);
    const u128 s2 = u128(st[D + c]) | (u128(st[2 * D + c]) << 64);
    my[e] = s2 * n - square(s1);
    myf[e] = order_image(my[e]);
    key[c] = my[e];
    fkey[c] = myf[e];
  }
  __syncthreads();
  // rank: channels of larger spread, or of equal spread and lower index, come first (the fp32
  // images decide unless they are equal)
  bool hi[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    int r = 0;
    bool tie = false;
    for (int c2 = 0; c2 < D; ++c2) {
      const float f2 = fkey[c2];
      r += f2 > myf[e] ? 1 : 0;
      tie = tie || (f2 == myf[e] && c2 != c);
    }
    if (tie) {
      for (int c2 = 0; c2 < D; ++c2) {
        if (fkey[c2] != myf[e]) continue;
        const u128 k2 = key[c2];
        r += (k2 > my[e] || (k2 == my[e] && c2 < c)) ? 1 : 0;
      }
    }
    hi[e] = r < nhi;
  }
  // high channels below each of the lane's channels, from the wave's votes (channel
  // lane*E + e votes in mask e)
  uint64_t vote[E];
#pragma unroll
  for (int e = 0; e < E; ++e) vote[e] = __ballot(hi[e]);
  const uint64_t below_lane = lane ? (~0ull >> (64 - lane)) : 0ull;
  // slots: the high channels first, each set in ascending channel order
  uint32_t* params = reinterpret_cast<uint32_t*>(rec + kitty_off_params(D, nhi));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    int below = 0;  // high channels c2 < c: c2 = lane' * E + e' with lane' < lane, or lane' = lane and e' < e
#pragma unroll
    for (int e2 = 0; e2 < E; ++e2) below += __popcll(vote[e2] & (e2 < e ? (below_lane | (1ull << lane)) : below_lane));
    const int slot = hi[e] ? below : nhi + (c - below);
    rec[kitty_off_table(D, nhi) + slot] = uint8_t(c);
    float mn = kx[0][e], mx = kx[0][e];
#pragma unroll
    for (int t = 1; t < kGroup; ++t) {
      mn = fminf(mn, kx[t][e]);
      mx = fmaxf(mx, kx[t][e]);
    }
    if (hi[e]) {
      const GroupParams p = group_params<kHB>(mn, mx);
      params[slot] = p.packed;
#pragma unroll
      for (int t = 0; t < kGroup; ++t) cb[t][slot] = uint8_t(code_of<kHB>(kx[t][e], p));
    } else {
      const GroupParams p = group_params<kLB>(mn, mx);
      params[slot] = p.packed;
#pragma unroll
      for (int t = 0; t < kGroup; ++t) cb[t][slot] = uint8_t(code_of<kLB>(kx[t][e], p));
    }
  }
  __syncthreads();
  // code words: token t, word w: a high chunk's half (8 slots x 4 bits) or a low chunk
  // (16 slots x 2 bits)
  uint32_t* cw = reinterpret_cast<uint32_t*>(rec);
  for (int w = lane; w < kGroup * W; w += 64) {
    const int t = w / W, wt = w % W;
    uint32_t v = 0;
    if (wt < 2 * nhc) {
      const int s0 = (wt >> 1) * 16 + (wt & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) v |= uint32_t(cb[t][s0 + i]) << (kHB * i);
    } else {
      const int s0 = (wt - nhc) * 16;
#pragma unroll
      for (int i = 0; i < 16; ++i) v |= uint32_t(cb[t][s0 + i]) << (kLB * i);
    }
    cw[w] = v;
  }
  // value rows, over the staging (read above, before the barriers)
  const uint4* vs = reinterpret_cast<const uint4*>(V + row0);
  uint4* vd = reinterpret_cast<uint4*>(rec + kitty_off_values(D, nhi));
  for (int i = lane; i < kGroup * D / 8; i += 64) vd[i] = vs[i];
}

// ---------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct KittyLds {
  float qc[G][D];       // query by channel (base-2 units)
  float qt[G][D];       // query times key scale, by slot
  float p[G][kGroup];   // softmax weights of the unit's tokens
};

// One record's loads for one lane: its token's code words (key lanes), its slots' params and
// table entries, and its value octet of its tokens (value lanes; rows past the window's valid
// ones are clamped, their weights are 0).
template <int D>
struct RecRegs {
  uint32_t w0[D / 32], w1[D / 32], pr[D / 64];
  int tb[D / 64];
  uint4 vv[kGroup / (64 / (D / 8))];
};

template <int D>
__device__ __forceinline__ void load_rec(const uint8_t* __restrict__ rec, int nhc, int Wd, int nhi, int tk, int hh,
                                         int lane, int o, RecRegs<D>& r) {
  constexpr int E = D / 64, NO = D / 8, NTG = 64 / NO, TPL = kGroup / NTG, NJ = D / 32;
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(rec) + tk * Wd;
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int k = 2 * jj + hh;
    const int a = k + min(k, nhc);
    r.w0[jj] = cw[a];
    r.w1[jj] = cw[a + 1];  // the second word of a high chunk (unused otherwise; inside the record)
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    r.pr[e] = reinterpret_cast<const uint32_t*>(rec + kitty_off_params(D, nhi))[lane * E + e];
    r.tb[e] = rec[kitty_off_table(D, nhi) + lane * E + e];
  }
  // the value rows (most of the record, read once per step, each load a contiguous 1 KiB across
  // the wave): non-temporal loads, which stream them in faster than the default policy (the
  // 64K-token, 32-head decode: 119 -> 107 us); the key words (4-byte loads, token-strided) keep it
  const uint4* vs = reinterpret_cast<const uint4*>(rec + kitty_off_values(D, nhi));
#pragma unroll
  for (int k = 0; k < TPL; ++k)
    r.vv[k] = load_nt4(reinterpret_cast<const uint32_t*>(vs + (lane / NO + NTG * k) * NO + lane % NO));
}

template <int D, int G>
__global__ __launch_bounds__(64 * kDecWaves) void kitty_decode_kernel(const uint8_t* __restrict__ buf, Layout L,
                                                                       DecodeShape ds, const __half* __restrict__ q,
                                                                       float* __restrict__ ws, uint32_t* __restrict__ sync,
                                                                       void* __restrict__ out) {
  constexpr int E = D / 64, NO = D / 8, NTG = 64 / NO, TPL = kGroup / NTG, NJ = D / 32;
  __shared__ KittyLds<D, G> lw[kDecWaves];
  __shared__ float res[kDecWaves][G][D + 2];
  __shared__ float mrg[3][64 * kDecWaves];
  __shared__ int sh_last;
  const int sigma = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t* len = reinterpret_cast<const int32_t*>(buf + L.lengths(b, h));
  const int nq = max(0, min(len[0], L.max_groups * kGroup));
  const int nr = max(0, min(len[1], L.R));
  const int ngroups = nq / kGroup;
  const int nunits = ngroups + (nr + kGroup - 1) / kGroup;
  const int u0 = sigma * ds.chunk;
  if (u0 >= nunits) return;  // uniform over the workgroup
  const int u1 = min(u0 + ds.chunk, nunits);
  KittyLds<D, G>& W = lw[wave];
  const int nhi = L.nhi, nhc = nhi / 16, Wd = kitty_words(D, nhi);
  // Multi-query attend (ds.nqry > 1): row i is query i % nqry of its head, the cache's token
  // S - nqry + i % nqry; it sees the positions below lim[i] (kMaskScore above, as in the KIVI
  // decode: a wave or split that sees only a row's future merges with weight 0).
  int lim[G];
#pragma unroll
  for (int i = 0; i < G; ++i) lim[i] = nq + nr - (ds.nqry - 1 - i % ds.nqry);
  const int tk = lane >> 1, hh = lane & 1;  // key lanes
  const int o = lane % NO, tg = lane / NO;  // value lanes
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = lane * E + e;
      W.qc[i][c] = __half2float(q[(int64_t(b) * ds.n_q_heads + h * G + i) * D + c]) * ds.qscale;
    }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
  }
  wave_sync();
  // One record ahead is requested while the current one is computed (G <= 4; at G = 8 the
  // registers would spill). The prefetch index is clamped to the split's last
  // record, so the load is unconditional (a wave's last prefetch re-reads a record).
  constexpr bool kPrefetch = G <= 4;
  const int ulast = max(min(u1, ngroups) - 1, 0);
  RecRegs<D> cur, nxt;
  if (u0 + wave < min(u1, ngroups)) load_rec<D>(buf + L.record(b, h, u0 + wave), nhc, Wd, nhi, tk, hh, lane, o, cur);
  for (int u = u0 + wave; u < u1; u += kDecWaves) {
    float s[G];
    const uint4* vsrc = nullptr;
    int nvalid;
    uint4 vv[TPL];
    if (u < ngroups) {
      if constexpr (kPrefetch)
        load_rec<D>(buf + L.record(b, h, min(u + kDecWaves, ulast)), nhc, Wd, nhi, tk, hh, lane, o, nxt);
      else if (u != u0 + wave)
        load_rec<D>(buf + L.record(b, h, u), nhc, Wd, nhi, tk, hh, lane, o, cur);
      nvalid = kGroup;
#pragma unroll
      for (int k = 0; k < TPL; ++k) vv[k] = cur.vv[k];
      float beta[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float bp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float qv = W.qc[i][cur.tb[e]];
          W.qt[i][lane * E + e] = qv * lo_f(cur.pr[e]);
          bp = __builtin_fmaf(qv, hi_f(cur.pr[e]), bp);
        }
        beta[i] = wave_sum_all(bp);
      }
      wave_sync();
      // each code is converted once and serves every query head
      float a[G];
#pragma unroll
      for (int i = 0; i < G; ++i) a[i] = 0.f;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int k = 2 * jj + hh;
        if (k < nhc) {
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) {
            const uint32_t w = ii < 8 ? cur.w0[jj] : cur.w1[jj];
            const float c = float((w >> (kHB * (ii & 7))) & 15u);
#pragma unroll
            for (int i = 0; i < G; ++i) a[i] = __builtin_fmaf(W.qt[i][16 * k + ii], c, a[i]);
          }
        } else {
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) {
            const float c = float((cur.w0[jj] >> (kLB * ii)) & 3u);
#pragma unroll
            for (int i = 0; i < G; ++i) a[i] = __builtin_fmaf(W.qt[i][16 * k + ii], c, a[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < G; ++i) s[i] = a[i] + dpp<kQuadXor1>(a[i]) + beta[i];  // lanes (t, 0), (t, 1) are adjacent
      if (ds.nqry > 1 && u * kGroup + kGroup > lim[0]) {  // wave-uniform: a record that reaches a query
#pragma unroll
        for (int i = 0; i < G; ++i)
          if (u * kGroup + tk >= lim[i]) s[i] = kMaskScore;
      }
      if constexpr (kPrefetch) cur = nxt;
    } else {
      const int tbase = (u - ngroups) * kGroup;
      nvalid = min(kGroup, nr - tbase);
      const __half* wk = reinterpret_cast<const __half*>(buf + L.wk_off + L.window(b, h)) + tbase * D;
      vsrc = reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(buf + L.wv_off + L.window(b, h)) + tbase * D);
      const int tc = min(tk, nvalid - 1);
      const uint4* kr = reinterpret_cast<const uint4*>(wk + tc * D + hh * (D / 2));
      uint4 kk[D / 16];
#pragma unroll
      for (int i = 0; i < D / 16; ++i) kk[i] = kr[i];
#pragma unroll
      for (int k = 0; k < TPL; ++k) vv[k] = vsrc[min(tg + NTG * k, nvalid - 1) * NO + o];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float* qh = &W.qc[i][hh * (D / 2)];
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < D / 16; ++r) {
          const uint32_t wv[4] = {kk[r].x, kk[r].y, kk[r].z, kk[r].w};
#pragma unroll
          for (int z = 0; z < 4; ++z) {
            a = __builtin_fmaf(qh[8 * r + 2 * z], lo_f(wv[z]), a);
            a = __builtin_fmaf(qh[8 * r + 2 * z + 1], hi_f(wv[z]), a);
          }
        }
        s[i] = a + dpp<kQuadXor1>(a);
        if (nq + tbase + tk >= lim[i]) s[i] = kMaskScore;
        if (tk >= nvalid) s[i] = -INFINITY;
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float mx = wave_max_all(s[i]);
      if (mx > m[i]) {  // uniform
        const float alpha = __builtin_amdgcn_exp2f(m[i] - mx);
        l[i] *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] *= alpha;
        m[i] = mx;
      }
      const float p = __builtin_amdgcn_exp2f(s[i] - m[i]);
      if (hh == 0) {
        l[i] += p;
        W.p[i][tk] = p;
      }
    }
    wave_sync();
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const uint32_t wv[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
      float vf[8];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        vf[2 * z] = lo_f(wv[z]);
        vf[2 * z + 1] = hi_f(wv[z]);
      }
      const int t = tg + NTG * k;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float a = W.p[i][t];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(a, vf[c], acc[i][c]);
      }
    }
    wave_sync();
  }
  // the wave's partial: l over its lanes, acc over the token subsets of each octet
#pragma unroll
  for (int i = 0; i < G; ++i) {
    l[i] = wave_sum_all(l[i]);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int msk = NO; msk < 64; msk <<= 1) acc[i][c] += __shfl_xor(acc[i][c], msk, 64);
    if (lane < NO)
#pragma unroll
      for (int c = 0; c < 8; ++c) res[wave][i][8 * o + c] = acc[i][c];
    if (lane == 0) {
      res[wave][i][D] = m[i];
      res[wave][i][D + 1] = l[i];
    }
  }
  __syncthreads();
  // the workgroup's partial per query head (acc[D], m, l), or the output when it is the
  // sequence's only split; the last split of (b, h_kv) to finish merges the partials (the
  // protocol of the KIVI decode: device-scope partial stores, a device-scope counter)
  const int nvalid = min(ds.n_split, (nunits + ds.chunk - 1) / ds.chunk);
  const int64_t row0 = int64_t(b) * ds.n_q_heads + h * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kDecWaves) {
    const int i = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, res[w][i][D]);
    float A = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = res[w][i][D];
      if (mw == -INFINITY) continue;  // a wave with no unit
      const float f = __builtin_amdgcn_exp2f(mw - M);
      A = __builtin_fmaf(f, res[w][i][c], A);
      Ls = __builtin_fmaf(f, res[w][i][D + 1], Ls);
    }
    if (nvalid == 1) {
      store_out(out, ds.out_fp32, (row0 + i) * D + c, A / Ls);
      continue;
    }
    float* p = ws + ((row0 + i) * ds.n_split + sigma) * (D + 4);
    put_partial(p + c, A);
    if (c == 0) {
      put_partial(p + D, M);
      put_partial(p + D + 1, Ls);
    }
  }
  if (nvalid == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* cnt = sync + (int64_t(b) * L.Hkv + h);
  if (threadIdx.x == 0) sh_last = atomicAdd(cnt, 1u) + 1u == uint32_t(nvalid);
  __syncthreads();
  if (!sh_last) return;
  merge_splits<D, G>(ws, row0, ds.n_split, nvalid, mrg, out, ds.out_fp32);
  if (threadIdx.x == 0) atomicExch(cnt, 0u);
}

template <int D>
hipError_t kitty_encode_d(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                          const PerSeq& seq, int max_records, hipStream_t s) {
  const dim3 grid(max_records, L.Hkv, L.B);
  const __half* kh = static_cast<const __half*>(K);
  const __half* vh = static_cast<const __half*>(V);
  const dim3 segs((max_records + kSeg - 1) / kSeg, L.Hkv, L.B);
  hipLaunchKernelGGL(kitty_stats_kernel<D>, grid, dim3(64), 0, s, buf, L, kh, ld_tok, seq);
  hipLaunchKernelGGL(kitty_seg_kernel<D>, segs, dim3(64), 0, s, buf, L, seq);
  hipLaunchKernelGGL(kitty_top_kernel<D>, dim3(L.Hkv, L.B), dim3(64), 0, s, buf, L, seq);
  hipLaunchKernelGGL(kitty_fix_kernel<D>, segs, dim3(64), 0, s, buf, L, seq);
  hipLaunchKernelGGL(kitty_encode_kernel<D>, grid, dim3(64), 0, s, buf, L, kh, vh, ld_tok, seq);
  return hipGetLastError();
}

template <int D, int G>
hipError_t kitty_decode_t(uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q, float* ws, void* out,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(ds.n_split, L.Hkv, L.B);
  const uint8_t* cb = buf;
  uint32_t* sync = reinterpret_cast<uint32_t*>(buf + L.sync_off);
  const __half* qh = static_cast<const __half*>(q);
  if (e0 || e1)
    hipExtLaunchKernelGGL((kitty_decode_kernel<D, G>), grid, dim3(64 * kDecWaves), 0, s, e0, e1, 0, cb, L, ds, qh, ws,
                          sync, out);
  else
    hipLaunchKernelGGL((kitty_decode_kernel<D, G>), grid, dim3(64 * kDecWaves), 0, s, cb, L, ds, qh, ws, sync, out);
  return hipGetLastError();
}

template <int D>
hipError_t kitty_decode_d(uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q, float* ws, void* out,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (ds.G) {
    case 1: return kitty_decode_t<D, 1>(buf, L, ds, q, ws, out, s, e0, e1);
    case 2: return kitty_decode_t<D, 2>(buf, L, ds, q, ws, out, s, e0, e1);
    case 4: return kitty_decode_t<D, 4>(buf, L, ds, q, ws, out, s, e0, e1);
    case 8: return kitty_decode_t<D, 8>(buf, L, ds, q, ws, out, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_kitty_encode(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                               const PerSeq& seq, int max_records, hipStream_t s) {
  if (max_records <= 0) return hipSuccess;
  if (L.D == 128) return kitty_encode_d<128>(buf, L, K, V, ld_tok, seq, max_records, s);
  if (L.D == 64) return kitty_encode_d<64>(buf, L, K, V, ld_tok, seq, max_records, s);
  return hipErrorInvalidValue;
}

hipError_t launch_kitty_decode(uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q, float* ws,
                               void* out, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (L.D == 128) return kitty_decode_d<128>(buf, L, ds, q, ws, out, s, e0, e1);
  if (L.D == 64) return kitty_decode_d<64>(buf, L, ds, q, ws, out, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace kvq
