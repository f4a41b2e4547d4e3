// attend_tiles.hip - multi-query attend over the quantized cache on the matrix cores: chunked
// prefill, where many query rows share every key and value they read.
//
// What is computed (the decode attention of "Changelog" v0.42.0 "Added", for several queries at
// once, the multi-token companion the pages pair with their fused decode in v0.40.0 "Added"):
// the newest n_query tokens of each sequence attend causally over every cached token, query j of
// a head seeing the first S - (n_query - 1 - j) tokens; k_hat = code * scale + zero per key group,
// v_hat likewise per value group; softmax in fp32 with an online running max.
//
// Work split: grid (n_split, row blocks, B * H_kv); a workgroup of 4 wavefronts takes 64 query
// rows of one KV head (rows = its query heads x n_query, in q's order) and `chunk` consecutive
// units of the sequence (a unit is one 32-token record, or up to 32 window tokens). Per unit the
// workgroup rebuilds k_hat and v_hat once into LDS as fp16 pairs (high part, and the low part
// k_hat - high, so that high + low carries 22 significant bits), and every wave runs its own
// 16-row tile through v_mfma_f32_16x16x32_f16:
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

constexpr int kTW = 4;                        // wavefronts per workgroup, one 16-row tile each
constexpr int kBlockRows = 16 * kTW;          // query rows per workgroup
constexpr float kMaskScore = -1.0e30f;        // a visible-later token: weight 0 once a real one is seen
constexpr int kKPad = 8, kVPad = 8;           // LDS row padding (halves)

template <int D>
struct TileLds {
  _Float16 kh[32][D + kKPad], kl[32][D + kKPad];  // k_hat [token][channel], high and low parts
  _Float16 vh[D][32 + kVPad], vl[D][32 + kVPad];  // v_hat [channel][token slot], see vslot()
  uint32_t kp[D];                                  // the record's key params (scale | zero << 16)
  uint32_t vp[D];                                  // its value params [t/2][group][t%2]
};

// Token order of the value product's K index: slot 8g + i holds token 4g + i and slot 8g + 4 + i
// token 16 + 4g + i (g = lane / 16, i < 4): the tokens whose scores a lane gets from the key
// product (rows 4g + i of its two 16-token output tiles).
__device__ __forceinline__ int vslot(int t) { return t < 16 ? (t >> 2) * 8 + (t & 3) : ((t - 16) >> 2) * 8 + 4 + (t & 3); }

__device__ __forceinline__ void split_hl(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// Rebuild one unit into LDS. Records: 256 threads, keys as (token, 16-channel chunk) and values as
// (channel, 16-token half), both in the record's code layout (layout.h). Window units: the fp16
// rows themselves (low parts 0), zeros past the last valid token.
template <int D, int BK, int BV>
__device__ __forceinline__ void load_unit(TileLds<D>& sh, const uint8_t* __restrict__ rec, const __half* __restrict__ wk,
                                          const __half* __restrict__ wv, int nvalid, bool is_rec) {
  constexpr int NKC = D / 16;               // 16-channel chunks of a key row
  constexpr int WQ = D * BK / 128;          // key code words per (token, quarter)
  constexpr int KW = BK / 2;                // words holding 16 key codes
  constexpr int VW = BV / 2;                // words holding 16 value codes
  constexpr int NKG = D / 32;
  const int tid = threadIdx.x;
  if (is_rec) {
    // params to LDS, codes to registers
    const uint32_t* kpg = reinterpret_cast<const uint32_t*>(rec + rec_off_kparams(D, BK, BV));
    const uint32_t* vpg = reinterpret_cast<const uint32_t*>(rec + rec_off_vparams(D, BK, BV));
    if (tid < D) sh.kp[tid] = kpg[tid];
    else if (tid < 2 * D) sh.vp[tid - D] = vpg[tid - D];
    uint32_t kw[KW], vw[VW];
    const int kt = tid / NKC, kj = tid % NKC;  // key work item (valid for tid < 32 * NKC)
    const int vd = tid >> 1, vh = tid & 1;     // value work item (valid for tid < 2 * D)
    if (tid < 32 * NKC) {
      const int P = kt >> 1, tp = kt & 1;
      const int ch0 = kj * 16, Q = ch0 / (D / 4), c0 = ch0 % (D / 4);
      const uint32_t* p = reinterpret_cast<const uint32_t*>(rec) + ((P * 4 + Q) * 2 + tp) * WQ + (c0 / 16) * KW;
#pragma unroll
      for (int w = 0; w < KW; ++w) kw[w] = p[w];
    }
    if (tid < 2 * D) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + rec_off_vcodes(D, BK)) + vd * BV + vh * VW;
#pragma unroll
      for (int w = 0; w < VW; ++w) vw[w] = p[w];
    }
    __syncthreads();  // params visible
    if (tid < 32 * NKC) {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int bit = c * BK;
        const uint32_t code = (kw[bit >> 5] >> (bit & 31)) & ((1u << BK) - 1);
        const uint32_t prm = sh.kp[kj * 16 + c];
        const float s = (float)__builtin_bit_cast(_Float16, uint16_t(prm & 0xFFFF));
        const float z = (float)__builtin_bit_cast(_Float16, uint16_t(prm >> 16));
        split_hl(__builtin_fmaf(s, float(code), z), sh.kh[kt][kj * 16 + c], sh.kl[kt][kj * 16 + c]);
      }
    }
    if (tid < 2 * D) {
      const int k = vd / 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = vh * 16 + i, bit = i * BV;
        const uint32_t code = (vw[bit >> 5] >> (bit & 31)) & ((1u << BV) - 1);
        const uint32_t prm = sh.vp[((t >> 1) * NKG + k) * 2 + (t & 1)];
        const float s = (float)__builtin_bit_cast(_Float16, uint16_t(prm & 0x7FFF));  // bit 15: sink marker
        const float z = (float)__builtin_bit_cast(_Float16, uint16_t(prm >> 16));
        split_hl(__builtin_fmaf(s, float(code), z), sh.vh[vd][vslot(t)], sh.vl[vd][vslot(t)]);
      }
    }
  } else {
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
}

template <int D, int BK, int BV>
__global__ __launch_bounds__(64 * kTW) void attend_tiles_kernel(const uint8_t* __restrict__ buf, Layout L, TileShape ts,
                                                                PerSeq seq, const __half* __restrict__ q,
                                                                float* __restrict__ ws, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) TileLds<D> sh;
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
  const int r = rb * kBlockRows + wave * 16 + (lane & 15);  // this lane's row
  const bool row_ok = r < NR;
  const bool tile_live = rb * kBlockRows + wave * 16 < NR;  // wave-uniform
  const int lim = S - (ts.nqry - 1 - (r % ts.nqry));  // positions below it are visible to the row
  const int64_t qrow = (int64_t(b) * ts.n_q_heads + h * ts.G) * ts.nqry + r;

  // q^T fragments of the key product: channels 32 ks + 8 g .. + 8 of the lane's row
  h8 qb[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    if (row_ok) {
      const uint4 v = *reinterpret_cast<const uint4*>(q + qrow * D + ks * 32 + 8 * g);
      qb[ks] = __builtin_bit_cast(h8, v);
    } else {
      qb[ks] = h8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float m = kMaskScore, lsum = 0.0f;
  f4 o[D / 16];
#pragma unroll
  for (int mc = 0; mc < D / 16; ++mc) o[mc] = f4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* rec0 = buf + L.record(b, h, 0);
  const __half* wk0 = reinterpret_cast<const __half*>(buf + L.wk_off + L.window(b, h));
  const __half* wv0 = reinterpret_cast<const __half*>(buf + L.wv_off + L.window(b, h));
  for (int u = u0; u < u1; ++u) {
    const bool is_rec = u < ngroups;
    const int tbase = is_rec ? 0 : (u - ngroups) * kGroup;
    const int nvalid = is_rec ? kGroup : min(kGroup, nr - tbase);
    const int pos0 = is_rec ? u * kGroup : nq + tbase;
    __syncthreads();  // the previous unit's readers are done with the LDS
    load_unit<D, BK, BV>(sh, rec0 + uint64_t(u) * L.rec_bytes, wk0 + tbase * D, wv0 + tbase * D, nvalid, is_rec);
    __syncthreads();
    if (!tile_live) continue;

    // ---- scores: two 16-token tiles, high and low key parts
    float s[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const h8 ah = *reinterpret_cast<const h8*>(&sh.kh[mt * 16 + (lane & 15)][ks * 32 + 8 * g]);
        const h8 al = *reinterpret_cast<const h8*>(&sh.kl[mt * 16 + (lane & 15)][ks * 32 + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qb[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qb[ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * g + i;
        float x = acc[i] * ts.qscale;
        if (pos0 + t >= lim) x = kMaskScore;
        if (t >= nvalid) x = -INFINITY;
        s[mt * 4 + i] = x;
      }
    }
    // ---- online softmax of the lane's row: its 32 scores sit in lanes l, l^16, l^32, l^48
    float mx = s[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, s[k]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__any(mx > m)) {  // wave-uniform: some row's maximum moves
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int mc = 0; mc < D / 16; ++mc) o[mc] *= alpha;
    }
    h8 ph, pl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = __builtin_amdgcn_exp2f(s[k] - m);
      lsum += p;
      const _Float16 hi = (_Float16)p;
      ph[k] = hi;
      pl[k] = (_Float16)(p - (float)hi);
    }
    // ---- values: O^T += V^T P^T, channel tiles of 16
#pragma unroll
    for (int mc = 0; mc < D / 16; ++mc) {
      const h8 vh = *reinterpret_cast<const h8*>(&sh.vh[mc * 16 + (lane & 15)][8 * g]);
      const h8 vl = *reinterpret_cast<const h8*>(&sh.vl[mc * 16 + (lane & 15)][8 * g]);
      o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, ph, o[mc], 0, 0, 0);
      o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pl, o[mc], 0, 0, 0);
      o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, ph, o[mc], 0, 0, 0);
    }
  }
  if (!tile_live) return;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (!row_ok) return;
  const int nvs = min(ts.n_split, (nunits + ts.chunk - 1) / ts.chunk);  // splits of this sequence
  if (nvs == 1) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int mc = 0; mc < D / 16; ++mc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t idx = qrow * D + mc * 16 + 4 * g + i;
        if (ts.out_fp32) static_cast<float*>(out)[idx] = o[mc][i] * inv;
        else static_cast<__half*>(out)[idx] = __float2half_rn(o[mc][i] * inv);
      }
    return;
  }
  float* dst = ws + (qrow * ts.n_split + sigma) * (D + 4);
#pragma unroll
  for (int mc = 0; mc < D / 16; ++mc)
    *reinterpret_cast<f4*>(dst + mc * 16 + 4 * g) = o[mc];
  if (g == 0) {
    dst[D] = m;
    dst[D + 1] = lsum;
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
