// decode.hip - decode attention straight over the quantized cache (split-K + merge).
//
// What is computed ("Changelog" v0.42.0 "Added": fused group-affine decode + attention):
//   out = softmax(sm_scale * q . K_hat^T) V_hat over every quantized and window token,
//   k_hat = code * scale + zero per key group, v_hat likewise per value group, with the
//   reconstruction done in registers inside an online softmax accumulated in fp32.
//
// Algebra used to avoid rebuilding k_hat / v_hat element by element:
//   score_t = sum_d q_d * (s_{j,d} c_{t,d} + z_{j,d})
//           = sum_d (q_d s_{j,d}) c_{t,d} + sum_d q_d z_{j,d}
//   so per key group (32 tokens) the scaled query q~_d = q_d s_{j,d} and the offset
//   beta_j = q . z_j are formed once, and each token costs one multiply-add per channel.
//   out_d  = sum_t p_t (s_{t,k} c_{t,d} + z_{t,k})
//          = sum_t (p_t s_{t,k}) c_{t,d} + sum_t p_t z_{t,k}
//   so each (token, value group) weight a_{t,k} = p_t s_{t,k} is formed once and the zero
//   terms collapse into one bias per value group.
// Scores are carried in base-2 units (q is pre-multiplied by sm_scale * log2 e) so the
// softmax uses exp2.
//
// Work split: grid (n_split, H_kv, B); workgroup = 4 wavefronts; a workgroup owns `chunk`
// consecutive units of one (b, h_kv) (unit = one 32-token record, or up to 32 window
// tokens), its waves take every 4th unit, and it writes one (m, l, acc[D]) partial per
// query head. The merge kernel combines the partials of a (b, h_q).
//
// Lane roles inside a wave for one record (they match the record layout in layout.h):
//   q~ producer   lane l: channels l*D/64 .. (D/64 of them), i.e. quarter l/16
//   key consumer  lane (P = l/4, Q = l%4): tokens 2P, 2P+1 x channels of quarter Q
//   a producer    lane (P, Q): value params of tokens 2P, 2P+1 (D/64 entries)
//   value consumer lane l: channels l*D/64 .., the 32 tokens of the record
// The quarter partial scores are summed with two DPP quad butterflies.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"

namespace kvq {

__device__ __forceinline__ float qxor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float qxor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); __builtin_amdgcn_wave_barrier(); }

__device__ __forceinline__ float lo_f(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w & 0xFFFF))); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w >> 16))); }

template <int N>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t* out) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[i];
      out[2 * i] = v.x; out[2 * i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = p[i];
  }
}

template <int D, int G>
struct WaveLds {
  float qt[G][4][D / 4 + 4];  // scaled query per quarter (padded rows)
  float beta[G][4];           // quarter offsets q . z
  float a[G][D / 32][32];     // value weights per (value group, token)
  float red[G][64];
};

template <int D, int BK, int BV, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(const uint8_t* __restrict__ buf, Layout L,
                                                           DecodeShape ds, const __half* __restrict__ q,
                                                           float* __restrict__ ws) {
  constexpr int E = D / 64;       // channels per lane (producer / value consumer)
  constexpr int DQ = D / 4;       // channels per key quarter
  constexpr int NKG = D / 32;     // value groups
  constexpr int WQ = D * BK / 128;
  constexpr int KW = 2 * WQ;      // key-code words per key-consumer lane
  constexpr int VW = E * BV;      // value-code words per value-consumer lane
  constexpr uint32_t KMASK = (1u << BK) - 1, VMASK = (1u << BV) - 1;
  constexpr int KPW = 32 / BK, VPW = 32 / BV;  // codes per word

  __shared__ union {
    WaveLds<D, G> w[4];
    float res[4][G][D + 4];
  } sh;

  const int sigma = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t* len = reinterpret_cast<const int32_t*>(buf + L.lengths(b, h));
  const int nq = max(0, min(len[0], L.max_groups * kGroup));
  const int nr = max(0, min(len[1], L.R));
  const int ngroups = nq / kGroup;
  const int nunits = ngroups + (nr + kGroup - 1) / kGroup;
  const int u0 = sigma * ds.chunk;
  if (u0 >= nunits) return;
  const int u1 = min(u0 + ds.chunk, nunits);

  WaveLds<D, G>& W = sh.w[wave];
  const int P = lane >> 2, Q = lane & 3;
  const int kprod = ((lane * E) >> 1) % NKG;
  const int kcons = (lane * E) / 32;

  float qp[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e)
      qp[i][e] = __half2float(q[(int64_t(b) * ds.n_q_heads + h * G + i) * D + lane * E + e]) * ds.qscale;

  float m[G], l[G], bias[G], acc[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
    bias[i] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[i][e] = 0.f;
  }

  for (int u = u0 + wave; u < u1; u += 4) {
    const bool quant = u < ngroups;
    uint32_t kc[KW], vc[VW], kp[E], vp[E];
    const __half* wk = nullptr;
    const __half* wv = nullptr;
    int nvalid = kGroup;
    if (quant) {
      const uint8_t* rec = buf + L.record(b, h, u);
      load_words<KW>(reinterpret_cast<const uint32_t*>(rec) + lane * KW, kc);
      load_words<VW>(reinterpret_cast<const uint32_t*>(rec + rec_off_vcodes(D, BK)) + lane * VW, vc);
      load_words<E>(reinterpret_cast<const uint32_t*>(rec + rec_off_kparams(D, BK, BV)) + lane * E, kp);
      load_words<E>(reinterpret_cast<const uint32_t*>(rec + rec_off_vparams(D, BK, BV)) + lane * E, vp);
    } else {
      // window tokens are plain fp16: scale 1.0 (0x3C00), zero 0
#pragma unroll
      for (int e = 0; e < E; ++e) kp[e] = vp[e] = 0x3C00u;
      const int tbase = (u - ngroups) * kGroup;
      nvalid = min(kGroup, nr - tbase);
      wk = reinterpret_cast<const __half*>(buf + L.wk_off + L.window(b, h)) + tbase * D;
      wv = reinterpret_cast<const __half*>(buf + L.wv_off + L.window(b, h)) + tbase * D;
    }

    // ---- scaled query and quarter offsets
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float bp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int ch = lane * E + e;
        const float s = lo_f(kp[e]);
        const float z = hi_f(kp[e]);
        W.qt[i][ch / DQ][ch % DQ] = qp[i][e] * s;
        bp += qp[i][e] * z;
      }
      bp += __shfl_xor(bp, 1, 64);
      bp += __shfl_xor(bp, 2, 64);
      bp += __shfl_xor(bp, 4, 64);
      bp += __shfl_xor(bp, 8, 64);
      if ((lane & 15) == 0) W.beta[i][lane >> 4] = bp;
    }
    wave_sync();

    // ---- scores of tokens 2P, 2P+1, online softmax, value weights
    const int t0 = 2 * P, t1 = 2 * P + 1;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float s0 = W.beta[i][Q], s1 = s0;
      if (quant) {
#pragma unroll
        for (int c = 0; c < DQ; ++c) {
          const float qv = W.qt[i][Q][c];
          const uint32_t c0 = (kc[(c * BK) / 32] >> ((c % KPW) * BK)) & KMASK;
          const uint32_t c1 = (kc[WQ + (c * BK) / 32] >> ((c % KPW) * BK)) & KMASK;
          s0 += qv * float(c0);
          s1 += qv * float(c1);
        }
      } else {
#pragma unroll 8
        for (int c = 0; c < DQ; ++c) {
          const float qv = W.qt[i][Q][c];
          const float k0 = t0 < nvalid ? __half2float(wk[t0 * D + Q * DQ + c]) : 0.f;
          const float k1 = t1 < nvalid ? __half2float(wk[t1 * D + Q * DQ + c]) : 0.f;
          s0 += qv * k0;
          s1 += qv * k1;
        }
      }
      s0 += qxor1(s0);
      s0 += qxor2(s0);
      s1 += qxor1(s1);
      s1 += qxor2(s1);
      if (t0 >= nvalid) s0 = -INFINITY;
      if (t1 >= nvalid) s1 = -INFINITY;

      float mx = fmaxf(s0, s1);
      mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m[i], mx);
      const float alpha = exp2f(m[i] - mnew);
      m[i] = mnew;
      l[i] *= alpha;
      bias[i] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[i][e] *= alpha;
      const float p0 = exp2f(s0 - mnew), p1 = exp2f(s1 - mnew);
      l[i] += p0 + p1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int idx = lane * E + e;
        const int tp = idx & 1, k = (idx >> 1) % NKG;
        const float p = tp ? p1 : p0;
        const float sv = lo_f(vp[e]);
        const float zv = hi_f(vp[e]);
        W.a[i][k][2 * P + tp] = p * sv;
        bias[i] += p * zv;
      }
    }
    wave_sync();

    // ---- weighted sum of the value codes
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float sacc = 0.f;
        if (quant) {
#pragma unroll
          for (int t = 0; t < kGroup; ++t) {
            const uint32_t c = (vc[e * BV + t / VPW] >> ((t % VPW) * BV)) & VMASK;
            sacc += W.a[i][kcons][t] * float(c);
          }
        } else {
          const int ch = lane * E + e;
          for (int t = 0; t < nvalid; ++t) sacc += W.a[i][kcons][t] * __half2float(wv[t * D + ch]);
        }
        acc[i][e] += sacc;
      }
    }
    wave_sync();
  }

  // ---- finish the wave: l counted once per quad, bias summed over its producers
  float lt[G], o[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float v = (Q == 0) ? l[i] : 0.f;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) v += __shfl_xor(v, msk, 64);
    lt[i] = v;
    W.red[i][lane] = bias[i];
  }
  wave_sync();
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float bsum = 0.f;
    for (int j = 0; j < 64; ++j)
      if (((j * E) >> 1) % NKG == kcons) bsum += W.red[i][j];
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = acc[i][e] + bsum;
  }
  (void)kprod;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < G; ++i) {
#pragma unroll
    for (int e = 0; e < E; ++e) sh.res[wave][i][lane * E + e] = o[i][e];
    if (lane == 0) {
      sh.res[wave][i][D] = m[i];
      sh.res[wave][i][D + 1] = lt[i];
    }
  }
  __syncthreads();

  // ---- combine the 4 waves and write the partial of each query head
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int i = idx / D, ch = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.res[w][i][D]);
    float O = 0.f, Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sh.res[w][i][D];
      if (mw != -INFINITY) {
        const float wgt = exp2f(mw - M);
        O += wgt * sh.res[w][i][ch];
        Lsum += wgt * sh.res[w][i][D + 1];
      }
    }
    float* dst = ws + ((int64_t(b) * ds.n_q_heads + h * G + i) * ds.n_split + sigma) * (D + 4);
    dst[ch] = O;
    if (ch == 0) {
      dst[D] = M;
      dst[D + 1] = Lsum;
    }
  }
}

// Combine the split partials of one (b, h_q) into the output row.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const uint8_t* __restrict__ buf, Layout L, DecodeShape ds,
                                                          const float* __restrict__ ws, void* __restrict__ out) {
  constexpr int E = D / 64;
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int h = hq / ds.G;
  const int32_t* len = reinterpret_cast<const int32_t*>(buf + L.lengths(b, h));
  const int nq = max(0, min(len[0], L.max_groups * kGroup));
  const int nr = max(0, min(len[1], L.R));
  const int nunits = nq / kGroup + (nr + kGroup - 1) / kGroup;
  const int nvalid = min(ds.n_split, (nunits + ds.chunk - 1) / ds.chunk);
  const float* base = ws + (int64_t(b) * ds.n_q_heads + hq) * ds.n_split * (D + 4);
  float M = -INFINITY;
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, base[s * (D + 4) + D]);
  float Lsum = 0.f, O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  for (int s = 0; s < nvalid; ++s) {
    const float ms = base[s * (D + 4) + D];
    if (ms == -INFINITY) continue;
    const float wgt = exp2f(ms - M);
    Lsum += wgt * base[s * (D + 4) + D + 1];
#pragma unroll
    for (int e = 0; e < E; ++e) O[e] += wgt * base[s * (D + 4) + lane * E + e];
  }
  const float inv = 1.f / Lsum;
  const int64_t row = (int64_t(b) * ds.n_q_heads + hq) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = O[e] * inv;
    if (ds.out_fp32)
      static_cast<float*>(out)[row + lane * E + e] = v;
    else
      static_cast<__half*>(out)[row + lane * E + e] = __float2half_rn(v);
  }
}

// ------------------------------------------------------------------------------------
template <int D, int BK, int BV, int G>
static hipError_t launch_split_t(const uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q,
                                 float* ws, hipStream_t s) {
  dim3 grid(ds.n_split, L.Hkv, L.B);
  hipLaunchKernelGGL((decode_split_kernel<D, BK, BV, G>), grid, dim3(256), 0, s, buf, L, ds,
                     static_cast<const __half*>(q), ws);
  return hipGetLastError();
}

template <int D, int BK, int BV>
static hipError_t launch_split_g(const uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q,
                                 float* ws, hipStream_t s) {
  switch (ds.G) {
    case 1: return launch_split_t<D, BK, BV, 1>(buf, L, ds, q, ws, s);
    case 2: return launch_split_t<D, BK, BV, 2>(buf, L, ds, q, ws, s);
    case 4: return launch_split_t<D, BK, BV, 4>(buf, L, ds, q, ws, s);
    case 8: return launch_split_t<D, BK, BV, 8>(buf, L, ds, q, ws, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t launch_split_d(const uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q,
                                 float* ws, hipStream_t s) {
  switch (L.bk * 16 + L.bv) {
    case 0x22: return launch_split_g<D, 2, 2>(buf, L, ds, q, ws, s);
    case 0x24: return launch_split_g<D, 2, 4>(buf, L, ds, q, ws, s);
    case 0x28: return launch_split_g<D, 2, 8>(buf, L, ds, q, ws, s);
    case 0x42: return launch_split_g<D, 4, 2>(buf, L, ds, q, ws, s);
    case 0x44: return launch_split_g<D, 4, 4>(buf, L, ds, q, ws, s);
    case 0x48: return launch_split_g<D, 4, 8>(buf, L, ds, q, ws, s);
    case 0x82: return launch_split_g<D, 8, 2>(buf, L, ds, q, ws, s);
    case 0x84: return launch_split_g<D, 8, 4>(buf, L, ds, q, ws, s);
    case 0x88: return launch_split_g<D, 8, 8>(buf, L, ds, q, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_split(const uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q,
                               float* ws, hipStream_t s) {
  if (L.D == 128) return launch_split_d<128>(buf, L, ds, q, ws, s);
  if (L.D == 64) return launch_split_d<64>(buf, L, ds, q, ws, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const uint8_t* buf, const Layout& L, const DecodeShape& ds, const float* ws,
                               void* out, hipStream_t s) {
  dim3 grid(ds.n_q_heads, L.B);
  if (L.D == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, s, buf, L, ds, ws, out);
  else if (L.D == 64)
    hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, s, buf, L, ds, ws, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
