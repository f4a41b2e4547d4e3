// encode.hip - group quantization kernels: prefill/encode, residual-window append + flush.
//
// The quantizer ("Changelog" v0.8.0 KIVI; v0.42.0 codes + per-group (scale, zero);
// v0.30.0 lo/scale and fp16 metadata):
//   key group   = 32 consecutive tokens of one channel,
//   value group = 32 consecutive channels of one token,
//   lo = min + 0, hi = max + 0 (turns -0 into +0),
//   scale16 = fp16_rne((hi - lo) / (2^b - 1)), zero16 = lo,
//   inv = 1 / float(scale16)  (0 when the stored scale is 0),
//   code = clamp(rint((x - lo) * inv), 0, 2^b - 1).
// Every step is one IEEE fp32 operation rounded to nearest even; this translation unit is
// built with -ffp-contract=off and correctly rounded fp32 division, so the codes and
// parameters are bit-identical to any other IEEE implementation of the same steps.
//
// One wavefront quantizes one record (32 tokens x D channels of K and of V); the prefill
// kernel runs two independent waves per workgroup:
//   * the 32 x D fp16 tile is loaded with non-temporal 16-byte loads, lane = (row r, 8-channel
//     chunk c8), and stays in its fp16 words;
//   * key min/max: packed fp16 pairs, lane-local over the lane's tokens, then the cross-row
//     exchanges (DPP row rotate, permlane16/32 swaps) leave every channel's range in all
//     lanes of its chunk;
//   * value min/max: packed fp16 pairs over the lane's 8 channels, then DPP quad butterflies
//     (quad_perm) across the 4 chunks of a 32-channel value group;
//   * codes: fma-mix subtract from the fp16 half, multiply, and a round-and-clamp on the bits
//     of t + 1.5 * 2^23 (biased_code); key codes are ORed into their pieces, value codes into
//     words that three halving lane exchanges complete;
//   * the record image is assembled in LDS and leaves with coalesced 16-byte stores.
//
// Sink tokens ("Changelog" v0.9.0, KIVI-Sink): the tokens of largest key L2 norm (squares
// added in fp32, channel 0 first, earlier token on equal norms), chosen once per
// (sequence, KV head) among the tokens of the first step that quantizes any. They keep
// their fp16 rows in the sink regions, are left out of their key groups' min/max, and their
// value scales are stored with the sign bit set so that decode skips their quantized slots.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"
#include "quant.h"

namespace kvq {

template <int D, int BK, int BV>
struct EncodeLds {
  static constexpr int kRecWords = D * (BK + BV + 2);
  uint32_t rec[kRecWords];       // record image
  // value codes one byte each, [d][t]: only where a word holds fewer tokens than one load's rows
  uint8_t vbytes[64 / (D / 8) > 32 / BV ? D * kGroup : 4];
  float2 kpar[D];                // (lo, inv) of each channel's key group
};

__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
}
// Value of quad lane Q (quad_perm [Q,Q,Q,Q]) in every lane of the quad.
template <int Q>
__device__ __forceinline__ float dpp_quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Q | (Q << 2) | (Q << 4) | (Q << 6), 0xF, 0xF, false));
}

// 16 bytes of a row that is read once: a non-temporal load (streaming cache policy), which
// streams the K and V rows in at a higher rate than the default policy.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 load_streaming(const __half* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Packed fp16 pairs: the min / max of two fp16 values is one of them, so taking it in fp16
// gives the same value as in fp32.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b)));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b)));
}
template <int HI>
__device__ __forceinline__ float half_of(uint32_t w) {
  return __half2float(__ushort_as_half(uint16_t(HI ? w >> 16 : w & 0xFFFFu)));
}

// Min and max (of fp16 pairs) over the lanes that hold the same 8 channels of a row-major
// tile with CH 16-byte chunks per row: lanes l, l ^ CH, l ^ 2 CH, ... (CH = 8: first the other
// half of the 16-lane row by DPP row_ror 8); then the gfx950 row swaps: with both operands
// equal, permlane16_swap returns rows (0,0,2,2) / (1,1,3,3) and permlane32_swap rows
// (0,1,0,1) / (2,3,2,3), lane positions within a row kept. Min and max do not care which is which.
template <int CH>
__device__ __forceinline__ void column_minmax(uint32_t& mn, uint32_t& mx) {
  if constexpr (CH == 8) {
    mn = pk_min(mn, uint32_t(__builtin_amdgcn_mov_dpp(int(mn), 0x128, 0xF, 0xF, false)));
    mx = pk_max(mx, uint32_t(__builtin_amdgcn_mov_dpp(int(mx), 0x128, 0xF, 0xF, false)));
  }
  const auto a = __builtin_amdgcn_permlane16_swap(mn, mn, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
  mn = pk_min(a[0], a[1]);
  mx = pk_max(b[0], b[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(mn, mn, false, false);
  const auto d = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
  mn = pk_min(c[0], c[1]);
  mx = pk_max(d[0], d[1]);
}

// The quantization code of x, the fp16 in half HI of w, as the bits of an fp32 in
// [1.5 * 2^23, 1.5 * 2^23 + L]: kCodeBias + clamp(rint((x - lo) * inv), 0, L).
//  * x - lo is one fma-mix (fp16 x times 1, plus -lo): a single rounding of the exact
//    difference, the same fp32 value as converting x and subtracting;
//  * adding 1.5 * 2^23 to t = (x - lo) * inv leaves an fp32 of unit spacing wherever
//    |t| < 2^22, so its rounding is rint's (to nearest, ties to even) and its bits are
//    kCodeBias + rint(t); further out the clamp decides alone, and fp32 bits read as signed
//    integers are ordered like the values, so the clamp is an integer median on the bits.
// The low 22 bits of kCodeBias are clear: the code sits alone in the low byte, and a code
// shifted left by s bits keeps the bias at bit 22 + s and up.
constexpr int32_t kCodeBias = 0x4B400000;  // 1.5 * 2^23
template <int B, int HI>
__device__ __forceinline__ uint32_t biased_code(uint32_t w, float lo, float inv) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(lo));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(lo));
  const float t = d * inv;
  const int32_t b = __float_as_int(t + 12582912.0f);
  return uint32_t(min(max(b, kCodeBias), kCodeBias + (1 << B) - 1));
}
template <int B>
__device__ __forceinline__ uint32_t biased_code(uint32_t w, int hi, float lo, float inv) {
  return hi ? biased_code<B, 1>(w, lo, inv) : biased_code<B, 0>(w, lo, inv);
}
// Low bytes of four words, b0 in byte 0 (v_perm_b32 selectors: 0-3 bytes of the second
// operand, 4-7 of the first, 12 a zero byte).
__device__ __forceinline__ uint32_t low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  return __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
}

// v[sel] for a lane-dependent sel < N (N a power of two) as a tree of selects on the bits of
// sel. (A chain of `sel == k` selects is folded back into an indexed read of the array, which a
// lane-dependent index sends through scratch memory.)
template <int N>
__device__ __forceinline__ float pick(const float (&v)[N], int sel) {
  static_assert((N & (N - 1)) == 0, "N must be a power of two");
  float level[N];
#pragma unroll
  for (int k = 0; k < N; ++k) level[k] = v[k];
#pragma unroll
  for (int bit = 0, n = N; n > 1; ++bit, n >>= 1) {
    const bool hi = (sel >> bit) & 1;
#pragma unroll
    for (int k = 0; k < n / 2; ++k) level[k] = hi ? level[2 * k + 1] : level[2 * k];
  }
  return level[0];
}

// LDS hand-off between the lanes of one wave: a wave's LDS accesses are performed in the
// order it issues them, so keeping the compiler from moving them across this point is all
// the ordering a single-wave exchange needs.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Quantize the 32-token tile (rows ks[0..31], vs[0..31], row stride D elements) into the
// record at `rec_out`. Called by all 64 lanes of one wave, which owns `lds`. Bit t of
// sink_mask (wave-uniform) marks token t as a sink.
template <int D, int BK, int BV>
__device__ __forceinline__ void encode_record(const __half* __restrict__ ks, const __half* __restrict__ vs,
                              uint32_t* __restrict__ rec_out, EncodeLds<D, BK, BV>& lds,
                              uint32_t sink_mask = 0) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / CH;   // rows covered by one load instruction
  constexpr int NI = kGroup / RPI;
  constexpr int DQ = D / 4;      // channels per key-code quarter
  constexpr int WQ = D * BK / 128;  // words per (token, quarter)
  constexpr int NKG = D / kGroup;   // value groups per token
  constexpr uint32_t KC_W = 0;
  constexpr uint32_t VC_W = D * BK;
  constexpr uint32_t KP_W = D * (BK + BV);
  constexpr uint32_t VP_W = KP_W + D;
  const int lane = threadIdx.x & 63;
  const int c8 = lane % CH, r = lane / CH;

  // fp16 pairs: channels 8*c8 + 2w, + 1 of token r + RPI*i. Every key row is requested before
  // any value row (the scheduling barriers keep the order), so that the key groups can be
  // computed while the value rows are still arriving.
  uint32_t kw[NI][4], vw[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = r + RPI * i;
    const u32x4 kr = load_streaming(ks + t * D + 8 * c8);
#pragma unroll
    for (int w = 0; w < 4; ++w) kw[i][w] = kr[w];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = r + RPI * i;
    const u32x4 vr = load_streaming(vs + t * D + 8 * c8);
#pragma unroll
    for (int w = 0; w < 4; ++w) vw[i][w] = vr[w];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- keys: one group per channel over the 32 tokens. Every lane of a chunk column ends up
  // with the column's min/max; each of the RPI lanes of the column then computes the
  // parameters of 8/RPI of its channels, and they meet in LDS.
  constexpr int EK = 8 / RPI;  // key groups whose parameters this lane computes
  float kmn[8], kmx[8];
  {
    uint32_t mn2[4], mx2[4];
    if (sink_mask == 0) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mn2[w] = kw[0][w];
        mx2[w] = kw[0][w];
#pragma unroll
        for (int i = 1; i < NI; ++i) {
          mn2[w] = pk_min(mn2[w], kw[i][w]);
          mx2[w] = pk_max(mx2[w], kw[i][w]);
        }
      }
    } else {  // sinks stay out of the min/max (every group keeps at least 32 - 16 tokens)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mn2[w] = 0x7C007C00u;  // +inf, +inf
        mx2[w] = 0xFC00FC00u;  // -inf, -inf
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const bool skip = (sink_mask >> (r + RPI * i)) & 1u;
          mn2[w] = pk_min(mn2[w], skip ? 0x7C007C00u : kw[i][w]);
          mx2[w] = pk_max(mx2[w], skip ? 0xFC00FC00u : kw[i][w]);
        }
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      column_minmax<CH>(mn2[w], mx2[w]);
      kmn[2 * w] = half_of<0>(mn2[w]);
      kmn[2 * w + 1] = half_of<1>(mn2[w]);
      kmx[2 * w] = half_of<0>(mx2[w]);
      kmx[2 * w + 1] = half_of<1>(mx2[w]);
    }
  }
#pragma unroll
  for (int j = 0; j < EK; ++j) {
    float mn8[8 / EK], mx8[8 / EK];  // candidates e = k * EK + j, k = the lane's row
#pragma unroll
    for (int k = 0; k < 8 / EK; ++k) {
      mn8[k] = kmn[k * EK + j];
      mx8[k] = kmx[k * EK + j];
    }
    const GroupParams g = group_params<BK>(pick(mn8, r), pick(mx8, r));
    const int ch = 8 * c8 + r * EK + j;
    lds.kpar[ch] = make_float2(g.lo, g.inv);
    lds.rec[KP_W + ch] = g.packed;
  }
  wave_lds_sync();
  GroupParams kp[8];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float4 v = *reinterpret_cast<const float4*>(&lds.kpar[8 * c8 + e]);
    kp[e].lo = v.x;
    kp[e].inv = v.y;
    kp[e + 1].lo = v.z;
    kp[e + 1].inv = v.w;
  }
  {
    const int ch0 = 8 * c8;
    const int Q = ch0 / DQ, cq = ch0 % DQ;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = r + RPI * i;
      const int P = t >> 1, tp = t & 1;
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = biased_code<BK>(kw[i][e >> 1], e & 1, kp[e].lo, kp[e].inv);
      const uint32_t word = KC_W + ((P * 4 + Q) * 2 + tp) * WQ + (cq * BK) / 32;
      const int bit = (cq * BK) % 32;
      uint8_t* base = reinterpret_cast<uint8_t*>(&lds.rec[word]) + bit / 8;
      if constexpr (BK == 2) {  // the bias stays above the 16 bits kept
        uint32_t piece = c[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) piece |= c[e] << (2 * e);
        *reinterpret_cast<uint16_t*>(base) = uint16_t(piece);
      } else if constexpr (BK == 4) {  // code pairs in the low byte, then the four bytes
        uint32_t pr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pr[k] = c[2 * k] | (c[2 * k + 1] << 4);
        *reinterpret_cast<uint32_t*>(base) = low_bytes(pr[0], pr[1], pr[2], pr[3]);
      } else {
        reinterpret_cast<uint32_t*>(base)[0] = low_bytes(c[0], c[1], c[2], c[3]);
        reinterpret_cast<uint32_t*>(base)[1] = low_bytes(c[4], c[5], c[6], c[7]);
      }
    }
  }

  // ---- values: one group per (token, 32 channels) = 4 adjacent chunks of the same row, i.e.
  // the 4 lanes of a quad. Each quad lane computes the parameters of NI/4 of its rows'
  // groups; DPP quad broadcasts hand them to the other three.
  constexpr int NQ = NI / 4;  // value groups whose parameters this lane computes
  const int q = c8 & 3;
  float vmn[NI], vmx[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t mn2 = pk_min(pk_min(vw[i][0], vw[i][1]), pk_min(vw[i][2], vw[i][3]));
    const uint32_t mx2 = pk_max(pk_max(vw[i][0], vw[i][1]), pk_max(vw[i][2], vw[i][3]));
    float mn = fminf(half_of<0>(mn2), half_of<1>(mn2));
    float mx = fmaxf(half_of<0>(mx2), half_of<1>(mx2));
    mn = fminf(mn, dpp_xor1(mn));
    mx = fmaxf(mx, dpp_xor1(mx));
    mn = fminf(mn, dpp_xor2(mn));
    mx = fmaxf(mx, dpp_xor2(mx));
    vmn[i] = mn;
    vmx[i] = mx;
  }
  float own_lo[NQ], own_inv[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    float mn4[4], mx4[4];  // candidates: rows i = k * NQ + j, k = this lane's quad position
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mn4[k] = vmn[k * NQ + j];
      mx4[k] = vmx[k * NQ + j];
    }
    const GroupParams g = group_params<BV>(pick(mn4, q), pick(mx4, q));
    own_lo[j] = g.lo;
    own_inv[j] = g.inv;
    const int t = r + RPI * (q * NQ + j);
    lds.rec[VP_W + ((t >> 1) * NKG + c8 / 4) * 2 + (t & 1)] = g.packed | (((sink_mask >> t) & 1u) << 15);
  }
  // Row i's parameters live in quad lane i / NQ, slot i % NQ.
  auto value_params = [&](int i) {
    GroupParams vp;
    switch (i / NQ) {
      case 0: vp.lo = dpp_quad_bcast<0>(own_lo[i % NQ]); vp.inv = dpp_quad_bcast<0>(own_inv[i % NQ]); break;
      case 1: vp.lo = dpp_quad_bcast<1>(own_lo[i % NQ]); vp.inv = dpp_quad_bcast<1>(own_inv[i % NQ]); break;
      case 2: vp.lo = dpp_quad_bcast<2>(own_lo[i % NQ]); vp.inv = dpp_quad_bcast<2>(own_inv[i % NQ]); break;
      default: vp.lo = dpp_quad_bcast<3>(own_lo[i % NQ]); vp.inv = dpp_quad_bcast<3>(own_inv[i % NQ]); break;
    }
    return vp;
  };

  // ---- value codes: word (channel d, sub-word sw) holds tokens sw*PER_WORD .. at bit t*BV
  constexpr int PER_WORD = 32 / BV;
  if constexpr (RPI <= PER_WORD) {
    // In registers. The lane's 8 channels own T = 8*BV consecutive words of the record, and
    // every one of them takes codes from the RPI lanes of the chunk column (lanes c8 + CH*r):
    // the lane places its own codes at their final bits (token t = r + RPI*i sits at bit
    // BV*(r + RPI*(i % CPW)) of sub-word i / CPW), then halving exchanges across the column
    // (lane distance 32, 16, then 8) OR the words together while each lane keeps half of
    // what is left, until lane r holds the M complete words T/RPI*r .. and stores them.
    constexpr int CPW = PER_WORD / RPI;  // codes of one lane in a word
    constexpr int T = 8 * BV;
    constexpr int M = T / RPI;
    uint32_t cd[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const GroupParams vp = value_params(i);
#pragma unroll
      for (int e = 0; e < 8; ++e) cd[i][e] = biased_code<BV>(vw[i][e >> 1], e & 1, vp.lo, vp.inv);
    }
    uint32_t wd[T];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int sw = 0; sw < BV; ++sw) {
        const int i0 = sw * CPW;
        uint32_t x;
        if constexpr (CPW == 4) x = low_bytes(cd[i0][e], cd[i0 + 1][e], cd[i0 + 2][e], cd[i0 + 3][e]);
        else if constexpr (CPW == 2) x = __builtin_amdgcn_perm(cd[i0 + 1][e], cd[i0][e], 0x0c040c00u);
        else x = cd[i0][e] & 0xFFu;
        wd[e * BV + sw] = x << (BV * r);
      }
    }
    // lane bit 5 (lanes 32..63 keep the upper half of the words)
#pragma unroll
    for (int k = 0; k < T / 2; ++k) {
      const auto x = __builtin_amdgcn_permlane32_swap(wd[k], wd[k + T / 2], false, false);
      wd[k] = x[0] | x[1];
    }
    // lane bit 4 (odd rows of 16 lanes keep the upper half)
#pragma unroll
    for (int k = 0; k < T / 4; ++k) {
      const auto x = __builtin_amdgcn_permlane16_swap(wd[k], wd[k + T / 4], false, false);
      wd[k] = x[0] | x[1];
    }
    if constexpr (RPI == 8) {  // lane bit 3 (lanes 8..15 of each row keep the upper half)
      const bool up = (lane >> 3) & 1;
#pragma unroll
      for (int k = 0; k < M; ++k) {
        const uint32_t send = up ? wd[k] : wd[k + M];
        const uint32_t keep = up ? wd[k + M] : wd[k];
        wd[k] = keep | uint32_t(__builtin_amdgcn_mov_dpp(int(send), 0x128, 0xF, 0xF, false));  // row_ror 8
      }
    }
    uint32_t* dst = &lds.rec[VC_W + T * c8 + M * r];
    if constexpr (M % 4 == 0) {
#pragma unroll
      for (int k = 0; k < M; k += 4)
        *reinterpret_cast<uint4*>(dst + k) = make_uint4(wd[k], wd[k + 1], wd[k + 2], wd[k + 3]);
    } else {
      static_assert(M == 2, "two words per lane");
      *reinterpret_cast<uint2*>(dst) = make_uint2(wd[0], wd[1]);
    }
    wave_lds_sync();
  } else {
    // Fewer tokens per word than rows per load (D = 64, 8-bit values): one byte per code
    // in LDS, then one lane per word gathers them.
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = r + RPI * i;
      const GroupParams vp = value_params(i);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        lds.vbytes[(8 * c8 + e) * kGroup + t] = uint8_t(biased_code<BV>(vw[i][e >> 1], e & 1, vp.lo, vp.inv));
    }
    wave_lds_sync();
    for (int w = lane; w < D * BV; w += 64) {
      const int d = w / BV, sw = w % BV;
      const uint8_t* src = &lds.vbytes[d * kGroup + sw * PER_WORD];
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < PER_WORD; ++n) word |= uint32_t(src[n]) << (n * BV);
      lds.rec[VC_W + w] = word;
    }
    wave_lds_sync();
  }

  // ---- copy the record out, 16 bytes per lane per step
  constexpr int NV4 = EncodeLds<D, BK, BV>::kRecWords / 4;
  const uint4* src4 = reinterpret_cast<const uint4*>(lds.rec);
  uint4* dst4 = reinterpret_cast<uint4*>(rec_out);
  for (int v = lane; v < NV4; v += 64) dst4[v] = src4[v];
  wave_lds_sync();
}

// ------------------------------------------------------------------------------------
// SKVQ-adapted ("Changelog" v0.30.0): per-token groups of 32 permuted channels for keys and
// values, each group's window [lo, hi] shrunk to [lo + d, hi - d], d = (hi - lo) * c, with c
// the fixed fraction (1 - alpha) / 2 or, with the search, the c_k = k / 40 (k = 0..10) whose
// reconstruction has the smallest fp32 sum of squared errors (taken in group order; the
// smaller k on ties). Channels are permuted by ascending range over the first chunk (stable).
// ------------------------------------------------------------------------------------
constexpr int kClipCandidates = 11;

template <int D, int BK, int BV>
struct SkvqLds {
  static constexpr int kRecWords = D * (BK + BV + 2);
  uint32_t rec[kRecWords];
  uint8_t vbytes[D * kGroup];      // value codes [permuted channel][token]
  __half tile[2][kGroup][D + 8];   // K and V rows of the record (padded)
  uint8_t perm[2][D];
};

// Codes (packed little-endian, B bits each, 32 of them) and (scale16 | zero16 << 16) of one
// group with the clip search over `ncand` candidates (fixed fraction `cfix` when ncand = 1).
template <int B>
__device__ __forceinline__ void clip_quant_group(const float (&x)[kGroup], int ncand, float cfix,
                                                 uint32_t (&best_codes)[B], uint32_t& best_params) {
  constexpr float L = float((1 << B) - 1);
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < kGroup; ++i) {
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
  lo = lo + 0.0f;
  hi = hi + 0.0f;
  // the search keeps the error only; the winner's codes are formed once afterwards
  float best_err = 0.0f, bs = 0.0f, bz = 0.0f;
  for (int k = 0; k < ncand; ++k) {
    const float c = ncand > 1 ? float(k) / 40.0f : cfix;
    const float d = (hi - lo) * c;
    const float lo_c = lo + d, hi_c = hi - d;
    const __half s16 = __float2half_rn((hi_c - lo_c) / L);
    const __half z16 = __float2half_rn(lo_c);
    const float s = __half2float(s16), z = __half2float(z16);
    const float inv = (s != 0.0f) ? 1.0f / s : 0.0f;
    float err = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float cf = fminf(fmaxf(rintf((x[i] - z) * inv), 0.0f), L);
      const float xh = cf * s + z;  // no contraction in this file: a multiply, then an add
      const float diff = x[i] - xh;
      err = err + diff * diff;
    }
    if (k == 0 || err < best_err) {
      best_err = err;
      bs = s;
      bz = z;
      best_params = uint32_t(__half_as_ushort(s16)) | (uint32_t(__half_as_ushort(z16)) << 16);
    }
  }
  const float binv = (bs != 0.0f) ? 1.0f / bs : 0.0f;
#pragma unroll
  for (int w = 0; w < B; ++w) best_codes[w] = 0;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float cf = fminf(fmaxf(rintf((x[i] - bz) * binv), 0.0f), L);
    best_codes[(i * B) / 32] |= uint32_t(cf) << ((i * B) % 32);
  }
}

// Channel permutation of one tile of n rows (row stride D) by ascending range, stable:
// perm[rank(c)] = c (the identity when `reorder` is 0). Called by `nthreads` threads of the
// workgroup, each taking channels tid, tid + nthreads, ...; rng is D floats of LDS.
template <int D>
__device__ __forceinline__ void range_permutation(const __half* __restrict__ rows, int n, float* rng,
                                                  uint8_t* __restrict__ perm_out, int tid, int nthreads, int reorder) {
  if (!reorder) {
    for (int c = tid; c < D; c += nthreads) perm_out[c] = uint8_t(c);
    return;
  }
  for (int c = tid; c < D; c += nthreads) {
    float mn = __half2float(rows[c]), mx = mn;
    for (int t = 1; t < n; ++t) {
      const float x = __half2float(rows[int64_t(t) * D + c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    rng[c] = mx - mn;
  }
  __syncthreads();
  for (int c = tid; c < D; c += nthreads) {
    const float r = rng[c];
    int rank = 0;
    for (int o = 0; o < D; ++o) rank += (rng[o] < r || (rng[o] == r && o < c)) ? 1 : 0;
    perm_out[rank] = uint8_t(c);
  }
  __syncthreads();
}

// Quantize 32 tokens (rows ks[0..31], vs[0..31], row stride D) into the SKVQ record at
// rec_out; perm_k / perm_v are the sequence's permutations (global), or null when the rows
// are stored permuted already (a window flushed after the first chunk). One wave.
template <int D, int BK, int BV>
__device__ __forceinline__ void skvq_encode_record(const __half* __restrict__ ks, const __half* __restrict__ vs,
                                                   const uint8_t* __restrict__ perm_k,
                                                   const uint8_t* __restrict__ perm_v, int ncand, float cfix,
                                                   uint32_t* __restrict__ rec_out, SkvqLds<D, BK, BV>& lds) {
  constexpr int NKG = D / kGroup;             // groups per token
  constexpr int DQ = D / 4;                   // channels per key-code quarter
  constexpr int QPG = kGroup / DQ;            // quarters per group (1 at D = 128, 2 at D = 64)
  constexpr int WQ = D * BK / 128;            // key-code words per (token, quarter)
  constexpr uint32_t VC_W = D * BK;
  constexpr uint32_t KP_W = D * (BK + BV);
  constexpr uint32_t VP_W = KP_W + D;
  constexpr int PAIRS = kGroup * NKG;         // (token, group) pairs per tensor
  const int lane = threadIdx.x & 63;
  // rows and permutations into LDS
  for (int i = lane; i < kGroup * D / 8; i += 64) {
    const int t = i / (D / 8), c = i % (D / 8);
    *reinterpret_cast<uint4*>(&lds.tile[0][t][8 * c]) = reinterpret_cast<const uint4*>(ks + t * D)[c];
    *reinterpret_cast<uint4*>(&lds.tile[1][t][8 * c]) = reinterpret_cast<const uint4*>(vs + t * D)[c];
  }
  for (int i = lane; i < D; i += 64) {
    lds.perm[0][i] = perm_k ? perm_k[i] : uint8_t(i);
    lds.perm[1][i] = perm_v ? perm_v[i] : uint8_t(i);
  }
  __syncthreads();
  for (int p = lane; p < PAIRS; p += 64) {
    const int t = p / NKG, k = p % NKG;
    const int P = t >> 1, tp = t & 1;
    float x[kGroup];
    // keys
#pragma unroll
    for (int i = 0; i < kGroup; ++i) x[i] = __half2float(lds.tile[0][t][lds.perm[0][k * kGroup + i]]);
    uint32_t cw[BK], par;
    clip_quant_group<BK>(x, ncand, cfix, cw, par);
#pragma unroll
    for (int qq = 0; qq < QPG; ++qq)
#pragma unroll
      for (int w = 0; w < WQ; ++w) lds.rec[((P * 4 + k * QPG + qq) * 2 + tp) * WQ + w] = cw[qq * WQ + w];
    lds.rec[KP_W + (P * NKG + k) * 2 + tp] = par;
    // values
#pragma unroll
    for (int i = 0; i < kGroup; ++i) x[i] = __half2float(lds.tile[1][t][lds.perm[1][k * kGroup + i]]);
    uint32_t vw[BV], vpar;
    clip_quant_group<BV>(x, ncand, cfix, vw, vpar);
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      lds.vbytes[(k * kGroup + i) * kGroup + t] = uint8_t((vw[(i * BV) / 32] >> ((i * BV) % 32)) & ((1u << BV) - 1));
    lds.rec[VP_W + (P * NKG + k) * 2 + tp] = vpar;
  }
  __syncthreads();
  constexpr int PER_WORD = 32 / BV;
  for (int w = lane; w < D * BV; w += 64) {
    const int d = w / BV, sw = w % BV;
    const uint8_t* src = &lds.vbytes[d * kGroup + sw * PER_WORD];
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < PER_WORD; ++n) word |= uint32_t(src[n]) << (n * BV);
    lds.rec[VC_W + w] = word;
  }
  __syncthreads();
  constexpr int NV4 = SkvqLds<D, BK, BV>::kRecWords / 4;
  const uint4* src4 = reinterpret_cast<const uint4*>(lds.rec);
  uint4* dst4 = reinterpret_cast<uint4*>(rec_out);
  for (int v = lane; v < NV4; v += 64) dst4[v] = src4[v];
  __syncthreads();
}

__device__ __forceinline__ int clip_candidates(const Layout& L) { return L.clip < 0.0f ? kClipCandidates : 1; }

// SKVQ records: record seq.a[b] + blockIdx.x of (b, h) from tokens seq.c[b] + 32 blockIdx.x of
// K, V [B][H_kv][ld_tok][D]: the caller's tokens at a prefill (channel order), or the cache's
// windows at a flush (rows_permuted: stored in permuted order already).
template <int D, int BK, int BV>
__global__ __launch_bounds__(64) void skvq_encode_kernel(uint8_t* __restrict__ buf, Layout L,
                                                         const __half* __restrict__ K,
                                                         const __half* __restrict__ V, int64_t ld_tok,
                                                         PerSeq seq, int rows_permuted) {
  __shared__ SkvqLds<D, BK, BV> lds;
  const int jl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (jl >= seq.b[b]) return;
  const int j = seq.a[b] + jl;
  if (j >= L.max_groups) return;
  const int64_t row0 = ((int64_t(b) * L.Hkv + h) * ld_tok + seq.c[b] + int64_t(kGroup) * jl) * D;
  const uint8_t* pm = buf + L.perm(b, h);
  skvq_encode_record<D, BK, BV>(K + row0, V + row0, rows_permuted ? nullptr : pm, rows_permuted ? nullptr : pm + D,
                                clip_candidates(L), L.clip, reinterpret_cast<uint32_t*>(buf + L.record(b, h, j)),
                                lds);
}

// SKVQ first flush (seq.b[b] > 0): the window's R rows and the sink rows of (b, h), in channel
// order so far, are rewritten in permuted order (the permutations have just been computed).
template <int D>
__global__ __launch_bounds__(64) void skvq_permute_rows_kernel(uint8_t* __restrict__ buf, Layout L, PerSeq seq) {
  constexpr int RB = 8;  // rows per pass
  __shared__ __half rows[2][RB][D];
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  if (seq.b[b] <= 0) return;
  const uint8_t* pk = buf + L.perm(b, h);
  const uint8_t* pv = pk + D;
  for (int region = 0; region < 2; ++region) {
    const int n = region == 0 ? L.R : L.NS;
    __half* rk = reinterpret_cast<__half*>(buf + (region == 0 ? L.wk_off + L.window(b, h) : L.sink_k(b, h)));
    __half* rv = reinterpret_cast<__half*>(buf + (region == 0 ? L.wv_off + L.window(b, h) : L.sink_v(b, h)));
    for (int r0 = 0; r0 < n; r0 += RB) {
      const int nb = min(RB, n - r0);
      for (int i = lane; i < nb * D; i += 64) {
        rows[0][i / D][i % D] = rk[r0 * D + i];
        rows[1][i / D][i % D] = rv[r0 * D + i];
      }
      __syncthreads();
      for (int i = lane; i < nb * D; i += 64) {
        rk[r0 * D + i] = rows[0][i / D][pk[i % D]];
        rv[r0 * D + i] = rows[1][i / D][pv[i % D]];
      }
      __syncthreads();
    }
  }
}

// SKVQ permutations from the first chunk: R tokens from token seq.c[b] (seq.b[b] > 0 only).
template <int D>
__global__ __launch_bounds__(128) void skvq_perm_kernel(uint8_t* __restrict__ buf, Layout L,
                                                        const __half* __restrict__ K,
                                                        const __half* __restrict__ V, int64_t ld_tok, PerSeq seq) {
  __shared__ float rng[D];
  const int h = blockIdx.x, b = blockIdx.y;
  if (seq.b[b] <= 0) return;
  const int64_t row0 = ((int64_t(b) * L.Hkv + h) * ld_tok + seq.c[b]) * D;
  uint8_t* pm = buf + L.perm(b, h);
  range_permutation<D>(K + row0, L.R, rng, pm, threadIdx.x, blockDim.x, L.reorder);
  range_permutation<D>(V + row0, L.R, rng, pm + D, threadIdx.x, blockDim.x, L.reorder);
}

// Prefill / encode: wave w of workgroup x quantizes record j0[b] + jl, jl = kEncodeWaves*x + w,
// of (b = blockIdx.z, h = blockIdx.y) from tokens 32*jl .. of the caller's K, V
// [B][H_kv][ld_tok][D]. The waves of a workgroup share nothing.
constexpr int kEncodeWaves = 2;
template <int D, int BK, int BV>
__global__ __launch_bounds__(64 * kEncodeWaves) void encode_kernel(uint8_t* __restrict__ buf, Layout L,
                                                                   const __half* __restrict__ K,
                                                                   const __half* __restrict__ V, int64_t ld_tok,
                                                                   PerSeq seq /* a: first record, b: records */) {
  __shared__ EncodeLds<D, BK, BV> lds_w[kEncodeWaves];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  EncodeLds<D, BK, BV>& lds = lds_w[wave];
  const int jl = blockIdx.x * kEncodeWaves + wave, h = blockIdx.y, b = blockIdx.z;
  if (jl >= seq.b[b]) return;
  const int j = seq.a[b] + jl;
  if (j >= L.max_groups) return;
  const int64_t row0 = ((int64_t(b) * L.Hkv + h) * ld_tok + int64_t(kGroup) * jl) * D;
  // sinks of (b, h) inside this record (they are chosen before any record is encoded, and
  // only the records of that first step can hold them)
  uint32_t mask = 0;
  const int32_t* sp = reinterpret_cast<const int32_t*>(buf + L.sink_pos(b, h));
  for (int k = 0; k < L.NS; ++k) {
    const int p = sp[k];
    if ((p >> 5) == j) mask |= 1u << (p & 31);
  }
  encode_record<D, BK, BV>(K + row0, V + row0, reinterpret_cast<uint32_t*>(buf + L.record(b, h, j)), lds, mask);
}

// Squared L2 norm of one fp16 row of D channels: fp32, channel 0 first, each square rounded
// to fp32 before it is added (this file is built without contraction into fused multiply-adds).
template <int D>
__device__ __forceinline__ float row_norm_sq(const __half* __restrict__ row) {
  float acc = 0.0f;
#pragma unroll 4
  for (int c = 0; c < D / 8; ++c) {
    const uint4 w = reinterpret_cast<const uint4*>(row)[c];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = __half2float(__ushort_as_half(uint16_t(ww[e] & 0xFFFF)));
      const float x1 = __half2float(__ushort_as_half(uint16_t(ww[e] >> 16)));
      acc = acc + x0 * x0;
      acc = acc + x1 * x1;
    }
  }
  return acc;
}

// (norm, position) order of the sink choice: the larger norm first, the earlier token on ties.
__device__ __forceinline__ bool sink_before(float n1, int t1, float n2, int t2) {
  return n1 > n2 || (n1 == n2 && t1 < t2);
}

// Sinks of the sequences whose first quantizing step is a prefill or an encode: among
// tokens 0 .. seq.b[b] - 1 of K[b][h] (0 = the sequence chooses nothing now), which are then
// also its token positions. Two kernels: every workgroup takes a chunk of 2048 tokens and
// writes its best NS (norm, position) pairs; a second pass per (b, h) picks the best NS of
// those, writes sink_pos (ascending) and copies the sinks' K, V rows. The chunk lists are
// staged in the sequence's record area, which the encode that follows overwrites (the
// first step quantizes every token the lists come from: 8 * NS bytes per chunk of 64
// records).
constexpr int kSelTPT = 8;                // tokens per thread
constexpr int kSelChunk = 256 * kSelTPT;  // tokens per workgroup

// The (norm, position) pair that comes first among the 256 threads' candidates, in every thread.
__device__ __forceinline__ void block_best(float& n, int& t, float* sn, int* st) {
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) {
    const float on = __shfl_xor(n, msk, 64);
    const int ot = __shfl_xor(t, msk, 64);
    if (sink_before(on, ot, n, t)) {
      n = on;
      t = ot;
    }
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();  // the previous round's readers are done
  if ((threadIdx.x & 63) == 0) {
    sn[w] = n;
    st[w] = t;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (sink_before(sn[k], st[k], n, t)) {
      n = sn[k];
      t = st[k];
    }
}

template <int D>
__global__ __launch_bounds__(256) void sink_chunk_kernel(uint8_t* __restrict__ buf, Layout L,
                                                         const __half* __restrict__ K, int64_t ld_tok, PerSeq seq) {
  __shared__ float sn[4];
  __shared__ int st[4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = seq.b[b], t0 = c * kSelChunk;
  if (t0 >= T) return;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t(b) * L.Hkv + h) * ld_tok * D;
  float nrm[kSelTPT];  // norms are >= 0; -1 = no token, -2 = already chosen
#pragma unroll
  for (int k = 0; k < kSelTPT; ++k) {
    const int t = t0 + tid + 256 * k;
    nrm[k] = t < T ? row_norm_sq<D>(K + base + int64_t(t) * D) : -1.0f;
  }
  float2* lists = reinterpret_cast<float2*>(buf + L.record(b, h, 0)) + int64_t(c) * L.NS;
  for (int r = 0; r < L.NS; ++r) {
    float n = -1.0f;
    int t = 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < kSelTPT; ++k)
      if (nrm[k] >= 0.0f && sink_before(nrm[k], t0 + tid + 256 * k, n, t)) {
        n = nrm[k];
        t = t0 + tid + 256 * k;
      }
    block_best(n, t, sn, st);
#pragma unroll
    for (int k = 0; k < kSelTPT; ++k)
      if (t0 + tid + 256 * k == t) nrm[k] = -2.0f;
    if (tid == 0) lists[r] = make_float2(n, __int_as_float(t));
  }
}

template <int D>
__global__ __launch_bounds__(256) void sink_merge_kernel(uint8_t* __restrict__ buf, Layout L,
                                                         const __half* __restrict__ K,
                                                         const __half* __restrict__ V, int64_t ld_tok, PerSeq seq) {
  __shared__ float sn[4];
  __shared__ int st[4];
  __shared__ int win[kMaxSinks];
  const int h = blockIdx.x, b = blockIdx.y;
  const int T = seq.b[b], NS = L.NS;
  if (T <= 0) return;
  const int tid = threadIdx.x;
  const int n_entries = (T + kSelChunk - 1) / kSelChunk * NS;
  const float2* lists = reinterpret_cast<const float2*>(buf + L.record(b, h, 0));
  for (int r = 0; r < NS; ++r) {
    float n = -1.0f;
    int t = 0x7FFFFFFF;
    for (int e = tid; e < n_entries; e += 256) {
      const float2 v = lists[e];
      const int et = __float_as_int(v.y);
      bool taken = false;
      for (int k = 0; k < r; ++k) taken = taken || win[k] == et;
      if (!taken && v.x >= 0.0f && sink_before(v.x, et, n, t)) {
        n = v.x;
        t = et;
      }
    }
    block_best(n, t, sn, st);
    if (tid == 0) win[r] = t;
    __syncthreads();
  }
  if (tid == 0) {  // ascending positions
    for (int i = 1; i < NS; ++i)
      for (int k = i; k > 0 && win[k - 1] > win[k]; --k) {
        const int x = win[k];
        win[k] = win[k - 1];
        win[k - 1] = x;
      }
    int32_t* sp = reinterpret_cast<int32_t*>(buf + L.sink_pos(b, h));
    for (int k = 0; k < NS; ++k) sp[k] = win[k];
  }
  __syncthreads();
  const int64_t base = (int64_t(b) * L.Hkv + h) * ld_tok * D;
  uint4* sk = reinterpret_cast<uint4*>(buf + L.sink_k(b, h));
  uint4* sv = reinterpret_cast<uint4*>(buf + L.sink_v(b, h));
  for (int i = tid; i < NS * (D / 8); i += 256) {
    const int k = i / (D / 8), c = i % (D / 8);
    const int64_t row = base + int64_t(win[k]) * D;
    sk[i] = reinterpret_cast<const uint4*>(K + row)[c];
    sv[i] = reinterpret_cast<const uint4*>(V + row)[c];
  }
}

constexpr int kMaxResidual = 256;  // largest window the host accepts

// masks[m] for a wave-uniform m < R/32, without a dynamically indexed register array
__device__ __forceinline__ uint32_t pick_mask(const uint32_t (&masks)[kMaxResidual / kGroup], int m) {
  uint32_t r = masks[0];
#pragma unroll
  for (int k = 1; k < kMaxResidual / kGroup; ++k) r = (m == k) ? masks[k] : r;
  return r;
}

// A sequence's first flush: choose its sinks among the R window tokens (one wave; R <= 256,
// so at most 4 candidates per lane), write their positions and fp16 rows, and set the bits
// of the flushed records' sink masks.
template <int D>
__device__ void select_window_sinks(uint8_t* __restrict__ buf, const Layout& L, int b, int h,
                                    const __half* __restrict__ wk, const __half* __restrict__ wv,
                                    uint32_t (&masks)[kMaxResidual / kGroup]) {
  const int lane = threadIdx.x & 63;
  constexpr int PL = kMaxResidual / 64;
  float nrm[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) {
    const int t = lane + 64 * k;
    nrm[k] = t < L.R ? row_norm_sq<D>(wk + t * D) : -1.0f;  // norms are >= 0; -1 = none
  }
  int pos[kMaxSinks];
#pragma unroll
  for (int r = 0; r < kMaxSinks; ++r) {
    pos[r] = 0x7FFFFFFF;
    if (r >= L.NS) continue;
    float bn = -1.0f;
    int bt = 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < PL; ++k)
      if (sink_before(nrm[k], lane + 64 * k, bn, bt)) {
        bn = nrm[k];
        bt = lane + 64 * k;
      }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
      const float on = __shfl_xor(bn, msk, 64);
      const int ot = __shfl_xor(bt, msk, 64);
      if (sink_before(on, ot, bn, bt)) {
        bn = on;
        bt = ot;
      }
    }
    pos[r] = bt;  // the same in every lane
#pragma unroll
    for (int k = 0; k < PL; ++k)
      if (lane + 64 * k == bt) nrm[k] = -2.0f;  // taken
  }
  // ascending positions (unused entries hold INT_MAX and stay last)
#pragma unroll
  for (int i = 1; i < kMaxSinks; ++i)
#pragma unroll
    for (int k = i; k > 0; --k) {
      const int lo = min(pos[k - 1], pos[k]), hi = max(pos[k - 1], pos[k]);
      pos[k - 1] = lo;
      pos[k] = hi;
    }
  int32_t* sp = reinterpret_cast<int32_t*>(buf + L.sink_pos(b, h));
  __half* sk = reinterpret_cast<__half*>(buf + L.sink_k(b, h));
  __half* sv = reinterpret_cast<__half*>(buf + L.sink_v(b, h));
  constexpr int HPL = D / 64;
#pragma unroll
  for (int r = 0; r < kMaxSinks; ++r) {
    if (r >= L.NS) break;
    if (lane == 0) sp[r] = pos[r];
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      sk[r * D + lane * HPL + e] = wk[pos[r] * D + lane * HPL + e];
      sv[r * D + lane * HPL + e] = wv[pos[r] * D + lane * HPL + e];
    }
#pragma unroll
    for (int m = 0; m < kMaxResidual / kGroup; ++m)
      if ((pos[r] >> 5) == m) masks[m] |= 1u << (pos[r] & 31);
  }
}

// Append one token per (b, h); a full window is flushed first (R/32 records). seq holds every
// sequence's lengths before the append (the host's mirror of the device lengths), so the
// token's loads and the flush decision wait for no device read.
// SKVQ caches: the first NS tokens of a sequence (seq.c = sinks present) go to the sink
// region; after them the window rule holds. Their full windows are flushed by the host's
// launches before this kernel (seq then holds the lengths after the flush).
template <int D, int BK, int BV>
__global__ __launch_bounds__(64) void append_kernel(uint8_t* __restrict__ buf, Layout L,
                                                    const __half* __restrict__ k_tok,
                                                    const __half* __restrict__ v_tok, PerSeq seq) {
  __shared__ EncodeLds<D, BK, BV> lds;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  constexpr int HPL = D / 64;  // halves per lane
  const int64_t src = (int64_t(b) * L.Hkv + h) * D;
  __half kt[HPL], vt[HPL];
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    kt[e] = k_tok[src + lane * HPL + e];
    vt[e] = v_tok[src + lane * HPL + e];
  }
  int nq = seq.a[b], nr = seq.b[b];
  __half* wk = reinterpret_cast<__half*>(buf + L.wk_off + L.window(b, h));
  __half* wv = reinterpret_cast<__half*>(buf + L.wv_off + L.window(b, h));
  if (L.method == kMethodSkvq) {
    const int nsp = seq.c[b];
    if (nsp < L.NS) {  // a sink: lengths unchanged
      __half* sk = reinterpret_cast<__half*>(buf + L.sink_k(b, h)) + nsp * D;
      __half* sv = reinterpret_cast<__half*>(buf + L.sink_v(b, h)) + nsp * D;
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        sk[lane * HPL + e] = kt[e];
        sv[lane * HPL + e] = vt[e];
      }
      if (lane == 0) reinterpret_cast<int32_t*>(buf + L.sink_pos(b, h))[nsp] = nsp;
      return;
    }
    if (nq > 0) {  // the token in permuted channel order
      const uint8_t* pm = buf + L.perm(b, h);
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        kt[e] = k_tok[src + pm[lane * HPL + e]];
        vt[e] = v_tok[src + pm[D + lane * HPL + e]];
      }
    }
  } else if (nr >= L.R) {  // uniform over the workgroup
    const int j0 = nq / kGroup;
    uint32_t masks[kMaxResidual / kGroup];  // sinks per flushed record
#pragma unroll
    for (int m = 0; m < kMaxResidual / kGroup; ++m) masks[m] = 0;
    if (L.NS > 0 && nq == 0) select_window_sinks<D>(buf, L, b, h, wk, wv, masks);
    for (int m = 0; m < L.R / kGroup; ++m) {
      if (j0 + m < L.max_groups)
        encode_record<D, BK, BV>(wk + m * kGroup * D, wv + m * kGroup * D,
                                 reinterpret_cast<uint32_t*>(buf + L.record(b, h, j0 + m)), lds,
                                 pick_mask(masks, m));
    }
    nq += L.R;
    nr = 0;
    __syncthreads();  // every lane has read the window before slot 0 is overwritten
  }
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    wk[nr * D + lane * HPL + e] = kt[e];
    wv[nr * D + lane * HPL + e] = vt[e];
  }
  if (lane == 0) {
    int32_t* len = reinterpret_cast<int32_t*>(buf + L.lengths(b, h));
    len[0] = nq;
    len[1] = nr + 1;
  }
}

// Prefill tail: copy tokens [t0, t0 + n_r) of K, V into window slots 0.. and set the lengths
// of (b, h) to (n_q, n_r); seq.a = n_q, seq.b = n_r, seq.c = t0 (n_q, or for SKVQ the sinks
// present plus n_q: its sinks, tokens 0 .. t0 - n_q - 1, are copied too). Sink slots that stay
// empty are marked -1 (KIVI-Sink: all of them while nothing is quantized).
template <int D>
__global__ __launch_bounds__(64) void window_fill_kernel(uint8_t* __restrict__ buf, Layout L,
                                                         const __half* __restrict__ K,
                                                         const __half* __restrict__ V,
                                                         int64_t ld_tok, PerSeq seq) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int nq = seq.a[b], nr = seq.b[b], t0 = seq.c[b];
  __half* wk = reinterpret_cast<__half*>(buf + L.wk_off + L.window(b, h));
  __half* wv = reinterpret_cast<__half*>(buf + L.wv_off + L.window(b, h));
  const int64_t row0 = ((int64_t(b) * L.Hkv + h) * ld_tok + t0) * D;
  constexpr int HPL = D / 64;
  // SKVQ rows are stored in permuted channel order once the sequence has a permutation
  // (its first chunk is quantized): slot c of a key row holds channel pk[c]
  const bool permuted = L.method == kMethodSkvq && nq > 0;
  const uint8_t* pk = buf + L.perm(b, h);
  const uint8_t* pv = pk + D;
  if (L.NS > 0) {
    int32_t* sp = reinterpret_cast<int32_t*>(buf + L.sink_pos(b, h));
    if (L.method == kMethodSkvq) {
      const int ns = t0 - nq;
      const int64_t s0 = (int64_t(b) * L.Hkv + h) * ld_tok * D;
      __half* sk = reinterpret_cast<__half*>(buf + L.sink_k(b, h));
      __half* sv = reinterpret_cast<__half*>(buf + L.sink_v(b, h));
      for (int t = 0; t < ns; ++t)
        for (int e = 0; e < HPL; ++e) {
          const int c = lane * HPL + e;
          sk[t * D + c] = K[s0 + int64_t(t) * D + (permuted ? pk[c] : c)];
          sv[t * D + c] = V[s0 + int64_t(t) * D + (permuted ? pv[c] : c)];
        }
      if (lane < L.NS) sp[lane] = lane < ns ? lane : -1;
    } else if (nq == 0 && lane < L.NS) {
      sp[lane] = -1;
    }
  }
  int ck[HPL], cv[HPL];  // source channel of each of the lane's slots
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    const int c = lane * HPL + e;
    ck[e] = permuted ? pk[c] : c;
    cv[e] = permuted ? pv[c] : c;
  }
  constexpr int TB = 8;  // rows in flight
  for (int t0 = 0; t0 < nr; t0 += TB) {
    __half kx[TB][HPL], vx[TB][HPL];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const int64_t r = row0 + int64_t(min(t0 + k, nr - 1)) * D;
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        kx[k][e] = K[r + ck[e]];
        vx[k][e] = V[r + cv[e]];
      }
    }
#pragma unroll
    for (int k = 0; k < TB; ++k)
      if (t0 + k < nr)
#pragma unroll
        for (int e = 0; e < HPL; ++e) {
          wk[(t0 + k) * D + lane * HPL + e] = kx[k][e];
          wv[(t0 + k) * D + lane * HPL + e] = vx[k][e];
        }
  }
  if (lane == 0) {
    int32_t* len = reinterpret_cast<int32_t*>(buf + L.lengths(b, h));
    len[0] = nq;
    len[1] = nr;
    *reinterpret_cast<uint32_t*>(buf + L.sync(b, h)) = 0;  // decode split counter starts at zero
  }
}

// Stateless encode of one fp16 block X [n_tok][D] (the kvq_encode_block test hook): one
// thread per group, with the same min/max, parameters and codes as the record encoder.
// per_channel: groups of `group` consecutive tokens of a channel (keys), scales [n_tok/group][D];
// else groups of `group` consecutive channels of a token (values), scales [n_tok][D/group].
// codes: one byte per element of X.
template <int B>
__global__ __launch_bounds__(64) void encode_block_kernel(const __half* __restrict__ X, int n_tok, int D, int group,
                                                          int per_channel, uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ zeros) {
  const int64_t gi = int64_t(blockIdx.x) * 64 + threadIdx.x;
  const int64_t ngroups = per_channel ? int64_t(n_tok / group) * D : int64_t(n_tok) * (D / group);
  if (gi >= ngroups) return;
  int64_t base, stride;
  if (per_channel) {
    base = (gi / D) * group * D + gi % D;
    stride = D;
  } else {
    base = (gi / (D / group)) * D + (gi % (D / group)) * group;
    stride = 1;
  }
  float mn = __half2float(X[base]), mx = mn;
  for (int j = 1; j < group; ++j) {
    const float x = __half2float(X[base + j * stride]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  const GroupParams p = group_params<B>(mn, mx);
  scales[gi] = uint16_t(p.packed & 0xFFFF);
  zeros[gi] = uint16_t(p.packed >> 16);
  for (int j = 0; j < group; ++j)
    codes[base + j * stride] = uint8_t(code_of<B>(__half2float(X[base + j * stride]), p));
}

// Set the lengths of every (b, h) to (seq.a[b], seq.b[b]); with clear_sinks also mark every
// sink slot empty (-1).
__global__ __launch_bounds__(64) void lengths_fill_kernel(uint8_t* __restrict__ buf, Layout L, PerSeq seq,
                                                          int clear_sinks) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= L.B * L.Hkv) return;
  const int b = i / L.Hkv;
  int32_t* len = reinterpret_cast<int32_t*>(buf + L.len_off) + 2 * i;
  len[0] = seq.a[b];
  len[1] = seq.b[b];
  reinterpret_cast<uint32_t*>(buf + L.sync_off)[i] = 0;  // decode split counters start at zero
  if (clear_sinks)
    for (int k = 0; k < L.NS; ++k) reinterpret_cast<int32_t*>(buf + L.sp_off)[int64_t(i) * L.NS + k] = -1;
}

// ------------------------------------------------------------------------------------
// Host-side launchers
// ------------------------------------------------------------------------------------
template <int D, int BK, int BV>
static hipError_t launch_encode_t(uint8_t* buf, const Layout& L, const void* K, const void* V,
                                  int64_t ld_tok, const PerSeq& seq, int max_records, hipStream_t s) {
  dim3 grid((max_records + kEncodeWaves - 1) / kEncodeWaves, L.Hkv, L.B);
  hipLaunchKernelGGL((encode_kernel<D, BK, BV>), grid, dim3(64 * kEncodeWaves), 0, s, buf, L,
                     static_cast<const __half*>(K), static_cast<const __half*>(V), ld_tok, seq);
  return hipGetLastError();
}

template <int D, int BK, int BV>
static hipError_t launch_append_t(uint8_t* buf, const Layout& L, const void* k, const void* v, const PerSeq& seq,
                                  hipStream_t s) {
  dim3 grid(L.Hkv, L.B);
  hipLaunchKernelGGL((append_kernel<D, BK, BV>), grid, dim3(64), 0, s, buf, L,
                     static_cast<const __half*>(k), static_cast<const __half*>(v), seq);
  return hipGetLastError();
}

#define KVQ_DISPATCH_BITS(D, FN, ...)                                     \
  switch (L.bk * 16 + L.bv) {                                             \
    case 0x22: return FN<D, 2, 2>(__VA_ARGS__);                           \
    case 0x24: return FN<D, 2, 4>(__VA_ARGS__);                           \
    case 0x28: return FN<D, 2, 8>(__VA_ARGS__);                           \
    case 0x42: return FN<D, 4, 2>(__VA_ARGS__);                           \
    case 0x44: return FN<D, 4, 4>(__VA_ARGS__);                           \
    case 0x48: return FN<D, 4, 8>(__VA_ARGS__);                           \
    case 0x82: return FN<D, 8, 2>(__VA_ARGS__);                           \
    case 0x84: return FN<D, 8, 4>(__VA_ARGS__);                           \
    case 0x88: return FN<D, 8, 8>(__VA_ARGS__);                           \
    default: return hipErrorInvalidValue;                                 \
  }

hipError_t launch_encode(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                         const PerSeq& seq, int max_records, hipStream_t s) {
  if (L.D == 128) { KVQ_DISPATCH_BITS(128, launch_encode_t, buf, L, K, V, ld_tok, seq, max_records, s) }
  if (L.D == 64) { KVQ_DISPATCH_BITS(64, launch_encode_t, buf, L, K, V, ld_tok, seq, max_records, s) }
  return hipErrorInvalidValue;
}

hipError_t launch_append(uint8_t* buf, const Layout& L, const void* k, const void* v, const PerSeq& seq,
                         hipStream_t s) {
  if (L.D == 128) { KVQ_DISPATCH_BITS(128, launch_append_t, buf, L, k, v, seq, s) }
  if (L.D == 64) { KVQ_DISPATCH_BITS(64, launch_append_t, buf, L, k, v, seq, s) }
  return hipErrorInvalidValue;
}

hipError_t launch_window_fill(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                              const PerSeq& seq, hipStream_t s) {
  dim3 grid(L.Hkv, L.B);
  if (L.D == 128)
    hipLaunchKernelGGL(window_fill_kernel<128>, grid, dim3(64), 0, s, buf, L, static_cast<const __half*>(K),
                       static_cast<const __half*>(V), ld_tok, seq);
  else if (L.D == 64)
    hipLaunchKernelGGL(window_fill_kernel<64>, grid, dim3(64), 0, s, buf, L, static_cast<const __half*>(K),
                       static_cast<const __half*>(V), ld_tok, seq);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_sink_select(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                              const PerSeq& seq, hipStream_t s) {
  if (L.NS < 1 || L.NS > kMaxSinks) return hipErrorInvalidValue;
  int max_t = 0;
  for (int b = 0; b < L.B; ++b) max_t = seq.b[b] > max_t ? seq.b[b] : max_t;
  if (max_t == 0) return hipSuccess;
  const dim3 g1((max_t + kSelChunk - 1) / kSelChunk, L.Hkv, L.B), g2(L.Hkv, L.B);
  const __half* k = static_cast<const __half*>(K);
  const __half* v = static_cast<const __half*>(V);
  if (L.D == 128) {
    hipLaunchKernelGGL(sink_chunk_kernel<128>, g1, dim3(256), 0, s, buf, L, k, ld_tok, seq);
    hipLaunchKernelGGL(sink_merge_kernel<128>, g2, dim3(256), 0, s, buf, L, k, v, ld_tok, seq);
  } else if (L.D == 64) {
    hipLaunchKernelGGL(sink_chunk_kernel<64>, g1, dim3(256), 0, s, buf, L, k, ld_tok, seq);
    hipLaunchKernelGGL(sink_merge_kernel<64>, g2, dim3(256), 0, s, buf, L, k, v, ld_tok, seq);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lengths_fill(uint8_t* buf, const Layout& L, const PerSeq& seq, hipStream_t s, int clear_sinks) {
  const int n = L.B * L.Hkv;
  hipLaunchKernelGGL(lengths_fill_kernel, dim3((n + 63) / 64), dim3(64), 0, s, buf, L, seq, clear_sinks);
  return hipGetLastError();
}

template <int D, int BK, int BV>
static hipError_t launch_skvq_encode_t(uint8_t* buf, const Layout& L, const void* K, const void* V,
                                       int64_t ld_tok, const PerSeq& seq, int max_records, int rows_permuted,
                                       hipStream_t s) {
  dim3 grid(max_records, L.Hkv, L.B);
  hipLaunchKernelGGL((skvq_encode_kernel<D, BK, BV>), grid, dim3(64), 0, s, buf, L,
                     static_cast<const __half*>(K), static_cast<const __half*>(V), ld_tok, seq, rows_permuted);
  return hipGetLastError();
}

hipError_t launch_skvq_encode(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                              const PerSeq& seq, int max_records, int rows_permuted, hipStream_t s) {
  if (L.D == 128) {
    KVQ_DISPATCH_BITS(128, launch_skvq_encode_t, buf, L, K, V, ld_tok, seq, max_records, rows_permuted, s)
  }
  if (L.D == 64) {
    KVQ_DISPATCH_BITS(64, launch_skvq_encode_t, buf, L, K, V, ld_tok, seq, max_records, rows_permuted, s)
  }
  return hipErrorInvalidValue;
}

hipError_t launch_skvq_permute_rows(uint8_t* buf, const Layout& L, const PerSeq& seq, hipStream_t s) {
  dim3 grid(L.Hkv, L.B);
  if (L.D == 128)
    hipLaunchKernelGGL(skvq_permute_rows_kernel<128>, grid, dim3(64), 0, s, buf, L, seq);
  else if (L.D == 64)
    hipLaunchKernelGGL(skvq_permute_rows_kernel<64>, grid, dim3(64), 0, s, buf, L, seq);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_skvq_perm(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                            const PerSeq& seq, hipStream_t s) {
  dim3 grid(L.Hkv, L.B);
  const __half* k = static_cast<const __half*>(K);
  const __half* v = static_cast<const __half*>(V);
  if (L.D == 128)
    hipLaunchKernelGGL(skvq_perm_kernel<128>, grid, dim3(128), 0, s, buf, L, k, v, ld_tok, seq);
  else if (L.D == 64)
    hipLaunchKernelGGL(skvq_perm_kernel<64>, grid, dim3(128), 0, s, buf, L, k, v, ld_tok, seq);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_encode_block(const void* X, int n_tok, int D, int bits, int group, int per_channel, void* codes,
                               void* scales, void* zeros, hipStream_t s) {
  const int64_t ngroups = per_channel ? int64_t(n_tok / group) * D : int64_t(n_tok) * (D / group);
  if (ngroups == 0) return hipSuccess;
  const dim3 grid(unsigned((ngroups + 63) / 64));
  const __half* x = static_cast<const __half*>(X);
  uint8_t* c = static_cast<uint8_t*>(codes);
  uint16_t* sc = static_cast<uint16_t*>(scales);
  uint16_t* z = static_cast<uint16_t*>(zeros);
  switch (bits) {
    case 2: hipLaunchKernelGGL(encode_block_kernel<2>, grid, dim3(64), 0, s, x, n_tok, D, group, per_channel, c, sc, z); break;
    case 4: hipLaunchKernelGGL(encode_block_kernel<4>, grid, dim3(64), 0, s, x, n_tok, D, group, per_channel, c, sc, z); break;
    case 8: hipLaunchKernelGGL(encode_block_kernel<8>, grid, dim3(64), 0, s, x, n_tok, D, group, per_channel, c, sc, z); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
