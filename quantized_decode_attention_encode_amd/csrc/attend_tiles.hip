// attend_tiles.hip - multi-query attend over the quantized cache on the matrix cores: chunked
// prefill, where many query rows share every key and value they read.
//
// What is computed (the decode attention of "Changelog" v0.42.0 "Added", for several queries at
// once, the multi-token companion the pages pair with their fused decode in v0.40.0 "Added"):
// the newest n_query tokens of each sequence attend causally over every cached token, query j of
// a head seeing the first S - (n_query - 1 - j) tokens; k_hat = code * scale + zero per key group,
// v_hat likewise per value group; softmax in fp32 with an online running max.
//
// Work split: grid (n_split, row blocks, B * H_kv); a workgroup of 8 wavefronts takes 256 query
// rows of one KV head (rows = its query heads x n_query, in q's order) and `chunk` consecutive
// units of the sequence (a unit is one 32-token record, or up to 32 window tokens). Per unit the
// workgroup rebuilds k_hat and v_hat once into LDS as fp16 pairs (high part, and the low part
// k_hat - high, so that high + low is k_hat within 2^-20 of it; keys by the first 256 threads,
// values by the next 256), and every wave runs its two 16-row tiles through
// v_mfma_f32_16x16x32_f16, each LDS fragment of k_hat or v_hat serving both tiles:
//   S^T[token][row] = K_hat[token][:] . q[row][:]   (A = K_hat high / low, B = q^T, exact fp16)
//   O^T[ch][row]   += V_hat^T[ch][token] . P^T[token][row]   (V_hat and P as high + low pairs:
//                     V_hi P_hi + V_hi P_lo + V_lo P_hi)
// With keys and values on the M side and rows on N, a lane's accumulator column (its row) is the
// same row whose softmax state it keeps, and the eight scores a lane receives from the key
// product are exactly the eight tokens it contributes to the value product's B operand.
// Splits write (acc[D], m, l) partials and a second kernel merges them.
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"

namespace kvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kTW = 8;                        // wavefronts per workgroup
constexpr int kNT = 2;                        // 16-row tiles per wavefront
constexpr int kBlockRows = 16 * kNT * kTW;    // query rows per workgroup
constexpr float kMaskScore = -1.0e30f;        // a visible-later token: weight 0 once a real one is seen
constexpr int kKPad = 8, kVPad = 8;           // LDS row padding (halves)

template <int D>
struct TileLds {
  _Float16 kh[32][D + kKPad], kl[32][D + kKPad];  // k_hat [token][channel], high and low parts
  _Float16 vh[D][32 + kVPad], vl[D][32 + kVPad];  // v_hat [channel][token slot], see vslot()
};

// Token order of the value product's K index: slot 8g + i holds token 4g + i and slot 8g + 4 + i
// token 16 + 4g + i (g = lane / 16, i < 4): the tokens whose scores a lane gets from the key
// product (rows 4g + i of its two 16-token output tiles).
__device__ __forceinline__ int vslot(int t) { return t < 16 ? (t >> 2) * 8 + (t & 3) : ((t - 16) >> 2) * 8 + 4 + (t & 3); }

// fp16 high and low parts of two fp32 values, packed: hi = x rounded toward zero, lo = x - hi
// (exact in fp32) rounded toward zero again; hi + lo = x within 2^-20 |x|.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
  const auto l = __builtin_amdgcn_cvt_pkrtz(x0 - (float)h[0], x1 - (float)h[1]);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Maximum over the lanes c, c + 16, c + 32, c + 48 (the four rows of the wave at one position),
// through the gfx950 row swaps.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// A record's raw bytes as one thread holds them between the fetch and the rebuild: a key thread's
// 16 codes of its (token, 16-channel chunk) and the (scale, zero) of those 16 channels, or a value
// thread's 16 codes of its (channel, 16-token half) and the (scale, zero) of those 16 tokens'
// value group.
constexpr int kValueThread0 = 256;  // threads [0, 256) rebuild keys, [256, 512) values

template <int BK, int BV>
struct RawUnit {
  uint32_t w[(BK > BV ? BK : BV) / 2];
  uint32_t prm[16];
};

template <int D, int BK, int BV>
__device__ __forceinline__ void fetch_record(const uint8_t* __restrict__ rec, RawUnit<BK, BV>& r) {
  constexpr int NKC = D / 16;       // 16-channel chunks of a key row
  constexpr int WQ = D * BK / 128;  // key code words per (token, quarter)
  constexpr int KW = BK / 2, VW = BV / 2, NKG = D / 32;
  const int tid = threadIdx.x;
  if (tid < 32 * NKC) {
    const int kt = tid / NKC, kj = tid % NKC;
    const int ch0 = kj * 16, Q = ch0 / (D / 4), c0 = ch0 % (D / 4);
    const uint32_t* p = reinterpret_cast<const uint32_t*>(rec) + (((kt >> 1) * 4 + Q) * 2 + (kt & 1)) * WQ + (c0 / 16) * KW;
#pragma unroll
    for (int w = 0; w < KW; ++w) r.w[w] = p[w];
    const uint4* pp = reinterpret_cast<const uint4*>(rec + rec_off_kparams(D, BK, BV)) + kj * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = pp[i];
      r.prm[4 * i] = v.x; r.prm[4 * i + 1] = v.y; r.prm[4 * i + 2] = v.z; r.prm[4 * i + 3] = v.w;
    }
  }
  const int vt = tid - kValueThread0;
  if (vt >= 0 && vt < 2 * D) {
    const int vd = vt >> 1, vh = vt & 1, k = vd / 32;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + rec_off_vcodes(D, BK)) + vd * BV + vh * VW;
#pragma unroll
    for (int w = 0; w < VW; ++w) r.w[w] = p[w];
    // tokens 16 vh + 2 j + tp: dwords [8 vh + j][k][tp], a pair per j
    const uint2* pp = reinterpret_cast<const uint2*>(rec + rec_off_vparams(D, BK, BV));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint2 v = pp[(8 * vh + j) * NKG + k];
      r.prm[2 * j] = v.x; r.prm[2 * j + 1] = v.y;
    }
  }
}

__device__ __forceinline__ float h_lo(uint32_t w, uint32_t mask = 0xFFFF) {
  return (float)__builtin_bit_cast(_Float16, uint16_t(w & mask));
}
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, uint16_t(w >> 16)); }

// Rebuild a fetched record into LDS: keys as (token, 16-channel chunk) by the threads below 256,
// values as (channel, 16-token half) by the threads from 256 on.
template <int D, int BK, int BV>
__device__ __forceinline__ void build_record(TileLds<D>& sh, const RawUnit<BK, BV>& r) {
  constexpr int NKC = D / 16;
  const int tid = threadIdx.x;
  if (tid < 32 * NKC) {
    const int kt = tid / NKC, kj = tid % NKC;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int c = 0; c < 16; c += 2) {
      float x[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int bit = (c + d) * BK;
        const uint32_t code = (r.w[bit >> 5] >> (bit & 31)) & ((1u << BK) - 1);
        x[d] = __builtin_fmaf(h_lo(r.prm[c + d]), float(code), h_hi(r.prm[c + d]));
      }
      split2(x[0], x[1], hi[c >> 1], lo[c >> 1]);
    }
    uint4* dh = reinterpret_cast<uint4*>(&sh.kh[kt][kj * 16]);
    uint4* dl = reinterpret_cast<uint4*>(&sh.kl[kt][kj * 16]);
    dh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    dh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    dl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    dl[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
  }
  const int vt = tid - kValueThread0;
  if (vt >= 0 && vt < 2 * D) {
    const int vd = vt >> 1, vh = vt & 1;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {  // tokens 16 vh + 4 q4 + i sit in slots 8 q4 + 4 vh + i
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bit = (q4 * 4 + i) * BV;
        const uint32_t code = (r.w[bit >> 5] >> (bit & 31)) & ((1u << BV) - 1);
        const uint32_t prm = r.prm[q4 * 4 + i];
        x[i] = __builtin_fmaf(h_lo(prm, 0x7FFF), float(code), h_hi(prm));  // bit 15: sink marker
      }
      uint2 hi, lo;
      split2(x[0], x[1], hi.x, lo.x);
      split2(x[2], x[3], hi.y, lo.y);
      *reinterpret_cast<uint2*>(&sh.vh[vd][8 * q4 + 4 * vh]) = hi;
      *reinterpret_cast<uint2*>(&sh.vl[vd][8 * q4 + 4 * vh]) = lo;
    }
  }
}

// A window unit: its fp16 rows themselves (low parts 0), zeros past the last valid token.
template <int D>
__device__ __forceinline__ void build_window(TileLds<D>& sh, const __half* __restrict__ wk,
                                             const __half* __restrict__ wv, int nvalid) {
  const int tid = threadIdx.x;
  for (int e = tid; e < 32 * D / 8; e += 64 * kTW) {  // keys: 8 channels per item
    const int t = e / (D / 8), c8 = (e % (D / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < nvalid) v = *reinterpret_cast<const uint4*>(wk + t * D + c8);
    *reinterpret_cast<uint4*>(&sh.kh[t][c8]) = v;
    *reinterpret_cast<uint4*>(&sh.kl[t][c8]) = make_uint4(0, 0, 0, 0);
  }
  for (int e = tid; e < 32 * D; e += 64 * kTW) {  // values: one element per item, transposed
    const int t = e / D, d = e % D;
    const _Float16 v = t < nvalid ? __builtin_bit_cast(_Float16, wv[t * D + d]) : (_Float16)0.0f;
    sh.vh[d][vslot(t)] = v;
    sh.vl[d][vslot(t)] = (_Float16)0.0f;
  }
}

template <int D, int BK, int BV>
__global__ __launch_bounds__(64 * kTW) void attend_tiles_kernel(const uint8_t* __restrict__ buf, Layout L, TileShape ts,
                                                                PerSeq seq, const __half* __restrict__ q,
                                                                float* __restrict__ ws, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) TileLds<D> shb[2];  // unit u in shb[(u - u0) & 1]
  const int sigma = blockIdx.x, rb = blockIdx.y;
  const int b = blockIdx.z / L.Hkv, h = blockIdx.z % L.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4;  // lane group: k-group of the operands, row group of the outputs
  const int nq = max(0, min(seq.a[b], L.max_groups * kGroup)), nr = max(0, min(seq.b[b], L.R));
  const int ngroups = nq / kGroup;
  const int nunits = ngroups + (nr + kGroup - 1) / kGroup;
  const int u0 = sigma * ts.chunk;
  if (u0 >= nunits) return;  // the whole workgroup: an idle split of a shorter sequence
  const int u1 = min(u0 + ts.chunk, nunits);
  const int NR = ts.G * ts.nqry;  // query rows of this KV head
  const int S = nq + nr;
  const int tile0 = rb * kBlockRows + wave * 16 * kNT;  // first row of the wave's tiles
  const int ntl = max(0, min(kNT, (NR - tile0 + 15) / 16));  // live tiles of the wave (wave-uniform)
  // per tile: the lane's row, its visibility limit and its q^T fragments (channels 32 ks + 8 g .. + 8)
  int lim[kNT];
  bool row_ok[kNT];
  int64_t qrow[kNT];
  h8 qb[kNT][D / 32];
#pragma unroll
  for (int tt = 0; tt < kNT; ++tt) {
    const int r = tile0 + tt * 16 + (lane & 15);
    row_ok[tt] = r < NR;
    lim[tt] = S - (ts.nqry - 1 - (r % ts.nqry));  // positions below it are visible to the row
    qrow[tt] = (int64_t(b) * ts.n_q_heads + h * ts.G) * ts.nqry + r;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      if (row_ok[tt]) {
        const uint4 v = *reinterpret_cast<const uint4*>(q + qrow[tt] * D + ks * 32 + 8 * g);
        qb[tt][ks] = __builtin_bit_cast(h8, v);
      } else {
        qb[tt][ks] = h8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  float m[kNT], lsum[kNT];
  f4 o[kNT][D / 16];
#pragma unroll
  for (int tt = 0; tt < kNT; ++tt) {
    m[tt] = kMaskScore;
    lsum[tt] = 0.0f;
#pragma unroll
    for (int mc = 0; mc < D / 16; ++mc) o[tt][mc] = f4{0.f, 0.f, 0.f, 0.f};
  }

  const uint8_t* rec0 = buf + L.record(b, h, 0);
  const __half* wk0 = reinterpret_cast<const __half*>(buf + L.wk_off + L.window(b, h));
  const __half* wv0 = reinterpret_cast<const __half*>(buf + L.wv_off + L.window(b, h));
  // Software pipeline over the units: unit u is in shb[(u - u0) & 1] while unit u + 1 is rebuilt
  // into the other buffer (its fetch issued one unit earlier still), between the key products and
  // the softmax of unit u; one barrier per unit.
  auto build = [&](int v, TileLds<D>& dst, RawUnit<BK, BV>& raw) {
    if (v < ngroups) {
      build_record<D, BK, BV>(dst, raw);
      if (v + 1 < min(u1, ngroups)) fetch_record<D, BK, BV>(rec0 + uint64_t(v + 1) * L.rec_bytes, raw);
    } else {
      const int tb = (v - ngroups) * kGroup;
      build_window<D>(dst, wk0 + tb * D, wv0 + tb * D, min(kGroup, nr - tb));
    }
  };
  RawUnit<BK, BV> raw;
  if (u0 < ngroups) fetch_record<D, BK, BV>(rec0 + uint64_t(u0) * L.rec_bytes, raw);
  build(u0, shb[0], raw);
  __syncthreads();
  for (int u = u0; u < u1; ++u) {
    const bool is_rec = u < ngroups;
    const int tbase = is_rec ? 0 : (u - ngroups) * kGroup;
    const int nvalid = is_rec ? kGroup : min(kGroup, nr - tbase);
    const int pos0 = is_rec ? u * kGroup : nq + tbase;
    TileLds<D>& sh = shb[(u - u0) & 1];
    // no row sees past S - (nqry - 1) - ... : a unit ending below every row's limit needs no mask
    const bool masked = !is_rec || pos0 + kGroup > S - (ts.nqry - 1);
    if (ntl == 0) {  // no rows here: only the rebuild of the next unit
      if (u + 1 < u1) build(u + 1, shb[(u - u0 + 1) & 1], raw);
      __syncthreads();
      continue;
    }

    // ---- scores: two 16-token tiles x high and low key parts, every k_hat fragment for all tiles
    f4 acc[kNT][2];
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) acc[tt][0] = acc[tt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const h8 ah = *reinterpret_cast<const h8*>(&sh.kh[mt * 16 + (lane & 15)][ks * 32 + 8 * g]);
        const h8 al = *reinterpret_cast<const h8*>(&sh.kl[mt * 16 + (lane & 15)][ks * 32 + 8 * g]);
#pragma unroll
        for (int tt = 0; tt < kNT; ++tt) {
          if (tt >= ntl) break;
          acc[tt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qb[tt][ks], acc[tt][mt], 0, 0, 0);
          acc[tt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qb[tt][ks], acc[tt][mt], 0, 0, 0);
        }
      }
    // ---- the next unit's rebuild (VALU and LDS writes) while the key products run
    if (u + 1 < u1) build(u + 1, shb[(u - u0 + 1) & 1], raw);
    h8 ph[kNT], pl[kNT];
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
      if (tt >= ntl) break;
      float s[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[mt * 4 + i] = acc[tt][mt][i] * ts.qscale;
      if (masked) {  // wave-uniform: a window unit, or a unit holding some row's future
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = mt * 16 + 4 * g + i;
            if (pos0 + t >= lim[tt]) s[mt * 4 + i] = kMaskScore;
            if (t >= nvalid) s[mt * 4 + i] = -INFINITY;
          }
      }
      // ---- online softmax of the lane's row: its 32 scores sit in lanes l, l^16, l^32, l^48
      float mx = s[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) mx = fmaxf(mx, s[k]);
      mx = max_over_rows(mx);
      if (__any(mx > m[tt])) {  // wave-uniform: some row's maximum moves
        const float mn = fmaxf(m[tt], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[tt] - mn);
        m[tt] = mn;
        lsum[tt] *= alpha;
#pragma unroll
        for (int mc = 0; mc < D / 16; ++mc) o[tt][mc] *= alpha;
      }
      uint32_t phw[4], plw[4];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[k] - m[tt]), p1 = __builtin_amdgcn_exp2f(s[k + 1] - m[tt]);
        lsum[tt] += p0 + p1;
        split2(p0, p1, phw[k >> 1], plw[k >> 1]);
      }
      ph[tt] = __builtin_bit_cast(h8, make_uint4(phw[0], phw[1], phw[2], phw[3]));
      pl[tt] = __builtin_bit_cast(h8, make_uint4(plw[0], plw[1], plw[2], plw[3]));
    }
    // ---- values: O^T += V^T P^T, channel tiles of 16, every v_hat fragment for all tiles
#pragma unroll
    for (int mc = 0; mc < D / 16; ++mc) {
      const h8 vh = *reinterpret_cast<const h8*>(&sh.vh[mc * 16 + (lane & 15)][8 * g]);
      const h8 vl = *reinterpret_cast<const h8*>(&sh.vl[mc * 16 + (lane & 15)][8 * g]);
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) {
        if (tt >= ntl) break;
        o[tt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, ph[tt], o[tt][mc], 0, 0, 0);
        o[tt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pl[tt], o[tt][mc], 0, 0, 0);
        o[tt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, ph[tt], o[tt][mc], 0, 0, 0);
      }
    }
    __syncthreads();  // unit u + 1 is built; every read of unit u is done
  }
  const int nvs = min(ts.n_split, (nunits + ts.chunk - 1) / ts.chunk);  // splits of this sequence
#pragma unroll
  for (int tt = 0; tt < kNT; ++tt) {
    if (tt >= ntl) break;
    float ls = lsum[tt];
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (!row_ok[tt]) continue;
    if (nvs == 1) {
      const float inv = 1.0f / ls;
#pragma unroll
      for (int mc = 0; mc < D / 16; ++mc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t idx = qrow[tt] * D + mc * 16 + 4 * g + i;
          if (ts.out_fp32) static_cast<float*>(out)[idx] = o[tt][mc][i] * inv;
          else static_cast<__half*>(out)[idx] = __float2half_rn(o[tt][mc][i] * inv);
        }
      continue;
    }
    float* dst = ws + (qrow[tt] * ts.n_split + sigma) * (D + 4);
#pragma unroll
    for (int mc = 0; mc < D / 16; ++mc) *reinterpret_cast<f4*>(dst + mc * 16 + 4 * g) = o[tt][mc];
    if (g == 0) {
      dst[D] = m[tt];
      dst[D + 1] = ls;
    }
  }
}

// Merge the split partials of every query row: one workgroup of D threads per row.
template <int D>
__global__ __launch_bounds__(D) void tiles_merge_kernel(Layout L, TileShape ts, PerSeq seq, const float* __restrict__ ws,
                                                        void* __restrict__ out) {
  const int64_t qrow = blockIdx.x;  // (b * H_q + head) * nqry + query
  const int b = int(qrow / (int64_t(ts.n_q_heads) * ts.nqry));
  const int nq = max(0, min(seq.a[b], L.max_groups * kGroup)), nr = max(0, min(seq.b[b], L.R));
  const int nunits = nq / kGroup + (nr + kGroup - 1) / kGroup;
  const int nvs = min(ts.n_split, (nunits + ts.chunk - 1) / ts.chunk);
  if (nvs <= 1) return;  // written directly by the split kernel
  const int ch = threadIdx.x;
  const float* base = ws + qrow * ts.n_split * (D + 4);
  float M = -INFINITY;
  for (int sg = 0; sg < nvs; ++sg) M = fmaxf(M, base[sg * (D + 4) + D]);
  float O = 0.f, Ls = 0.f;
  for (int sg = 0; sg < nvs; ++sg) {
    const float w = __builtin_amdgcn_exp2f(base[sg * (D + 4) + D] - M);
    O = __builtin_fmaf(w, base[sg * (D + 4) + ch], O);
    Ls = __builtin_fmaf(w, base[sg * (D + 4) + D + 1], Ls);
  }
  const int64_t idx = qrow * D + ch;
  if (ts.out_fp32) static_cast<float*>(out)[idx] = O / Ls;
  else static_cast<__half*>(out)[idx] = __float2half_rn(O / Ls);
}

template <int D, int BK, int BV>
hipError_t launch_t(const uint8_t* buf, const Layout& L, const TileShape& ts, const PerSeq& seq, const void* q, float* ws,
                    void* out, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(ts.n_split, ts.row_blocks, L.B * L.Hkv);
  const __half* qh = static_cast<const __half*>(q);
  const bool merge = ts.n_split > 1;
  if (e0 || e1)
    hipExtLaunchKernelGGL((attend_tiles_kernel<D, BK, BV>), grid, dim3(64 * kTW), 0, s, e0, merge ? nullptr : e1, 0, buf,
                          L, ts, seq, qh, ws, out);
  else
    hipLaunchKernelGGL((attend_tiles_kernel<D, BK, BV>), grid, dim3(64 * kTW), 0, s, buf, L, ts, seq, qh, ws, out);
  if (merge) {
    const dim3 g2(L.B * ts.n_q_heads * ts.nqry);
    if (e1)
      hipExtLaunchKernelGGL((tiles_merge_kernel<D>), g2, dim3(D), 0, s, nullptr, e1, 0, L, ts, seq,
                            static_cast<const float*>(ws), out);
    else
      hipLaunchKernelGGL((tiles_merge_kernel<D>), g2, dim3(D), 0, s, L, ts, seq, static_cast<const float*>(ws), out);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const uint8_t* buf, const Layout& L, const TileShape& ts, const PerSeq& seq, const void* q, float* ws,
                    void* out, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (L.bk * 16 + L.bv) {
    case 0x22: return launch_t<D, 2, 2>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x24: return launch_t<D, 2, 4>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x28: return launch_t<D, 2, 8>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x42: return launch_t<D, 4, 2>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x44: return launch_t<D, 4, 4>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x48: return launch_t<D, 4, 8>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x82: return launch_t<D, 8, 2>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x84: return launch_t<D, 8, 4>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    case 0x88: return launch_t<D, 8, 8>(buf, L, ts, seq, q, ws, out, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attend_tiles(const uint8_t* buf, const Layout& L, const TileShape& ts, const PerSeq& seq, const void* q,
                               float* ws, void* out, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (L.method != kMethodKivi || L.NS != 0) return hipErrorInvalidValue;
  if (L.D == 128) return launch_d<128>(buf, L, ts, seq, q, ws, out, s, e0, e1);
  if (L.D == 64) return launch_d<64>(buf, L, ts, seq, q, ws, out, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace kvq
