// decode_kernel.h - decode attention straight over the quantized cache (split-K, merged in-kernel).
// Included by decode.hip (plain caches) and decode_sink.hip (caches with sink tokens), which
// instantiate the kernel for SK = false and SK = true and compile in parallel.
//
// What is computed ("Changelog" v0.42.0 "Added": fused group-affine decode + attention):
//   out = softmax(sm_scale * q . K_hat^T) V_hat over every quantized and window token,
//   k_hat = code * scale + zero per key group, v_hat likewise per value group, with the
//   reconstruction done in registers inside an online softmax accumulated in fp32; no
//   dequantized K/V is written anywhere.
//
// Algebra used so that each cached code costs one multiply-add:
//   score_t = sum_d q_d (s_{j,d} c_{t,d} + z_{j,d}) = sum_d q~_d c_{t,d} + beta_j,
//     q~_d = q_d s_{j,d} and beta_j = q . z_j formed once per key group (32 tokens);
//   out_d  = sum_t p_t (s_{t,k} c_{t,d} + z_{t,k}) = sum_t a_{t,k} c_{t,d} + sum_t p_t z_{t,k},
//     a_{t,k} = p_t s_{t,k} formed once per (token, value group); the zero terms collapse
//     into one bias per value group.
//
// Code -> float conversion: a b-bit code c sitting at bits [o, o+b) of a 16-bit half, with
// o + b <= 10, becomes the exact fp16 number 1 + c * 2^(o-10) by OR-ing the exponent bits of
// 1.0 (0x3C00) into that half. One v_and_or_b32 (mask, magic held in VGPRs) turns two codes
// into such a pair, and v_fma_mix_f32 consumes either half directly as an fp32 operand. The
// factor 2^(10-o) is folded into the partner operand (q~ or a) and the constant "1" terms
// are removed exactly through beta and the value bias:
//   sum_c x'_c (1 + c 2^(o_c-10)) - sum_c x'_c = sum_c x_c c,   x'_c = x_c 2^(10-o_c).
// Codes not already at a usable bit position are first brought there by one shift per word
// shared by every code it moves (two shifts per 16 two-bit codes).
//
// Scores are kept in base-2 units (q is pre-multiplied by sm_scale * log2 e): exp2 softmax.
//
// Work split: grid (n_split, H_kv, B); workgroup = 4 wavefronts; a workgroup owns `chunk`
// consecutive units of one (b, h_kv) (unit = one 32-token record, or up to 32 window
// tokens), its waves take every 4th unit and prefetch their next record while computing
// the current one, and the workgroup writes one (acc[D], m, l) partial per query head. The
// last workgroup of a (b, h_kv) to finish (a counter in the cache buffer decides) merges the
// partials of that KV head's query heads into the output; a lone split writes it directly.
//
// Lane roles for a record (they follow the record layout, see layout.h):
//   q~ producer    lane l: channels l*D/64 .. (D/64 of them) = quarter l/16
//   key consumer   lane (P = l/4, Q = l%4): tokens 2P, 2P+1 x the channels of quarter Q
//   a producer     lane (P, Q): value params of tokens 2P, 2P+1 (D/64 entries)
//   value consumer lane l: channels l*D/64 .., all 32 tokens of the record
// Quarter partial scores meet through two DPP quad butterflies.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"

namespace kvq {

// ---------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {  // old = 0: lets the compiler fuse the move into the consumer
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Lane bits that a producer lane j can flip without leaving its value group ((j E) >> 1) % NKG
// (E channels per lane, NKG value groups): 0b111100 at D = 128, 0b111101 at D = 64.
__host__ __device__ constexpr int value_group_keep_mask(int E, int NKG) {
  int m = 0;
  for (int bit = 0; bit < 6; ++bit) {
    bool keep = true;
    for (int j = 0; j < 64; ++j)
      keep = keep && ((j * E) >> 1) % NKG == (((j ^ (1 << bit)) * E) >> 1) % NKG;
    if (keep) m |= 1 << bit;
  }
  return m;
}

// The zero-term bias of the output channels of this lane: v summed over the producer lanes of
// the value group that holds channels lane E .. lane E + E - 1 (a butterfly over the bits that
// keep the group, then a read from the first lane of the wanted group, 2 kc / E).
template <int D>
__device__ __forceinline__ float value_group_bias(float v, int lane) {
  constexpr int E = D / 64, NKG = D / 32, KEEP = value_group_keep_mask(E, NKG);
#pragma unroll
  for (int bit = 0; bit < 6; ++bit)
    if (KEEP & (1 << bit)) v += __shfl_xor(v, 1 << bit, 64);
  const int kc = (lane * E) / 32;
  return __shfl(v, (2 * kc) / E, 64);
}
static_assert(value_group_keep_mask(2, 4) == 0x3C && value_group_keep_mask(1, 2) == 0x3D, "value group lanes");

__device__ __forceinline__ float row_sum16(float v) {  // sum over the 16 lanes of a row, in every lane
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kRowRor8>(v);
  return v;
}
// Max over the wave when the 4 lanes of each quad hold equal values: row_ror 4 / 8 inside a
// row, then the gfx950 row swaps: with both operands equal, permlane32_swap returns rows
// (0,1,0,1) and (2,3,2,3), permlane16_swap rows (0,0,2,2) and (1,1,3,3).
__device__ __forceinline__ float wave_max_of_quads(float v) {
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kRowRor8>(v));
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float lo_f(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xFFFF))); }
__device__ __forceinline__ float hi_f(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16))); }

// A value the compiler must keep in a VGPR (so v_and_or_b32 can take it; gfx9 VOP3 has no literals).
template <uint32_t C>
__device__ __forceinline__ uint32_t vconst() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(C));
  return r;
}
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// Non-temporal loads (streaming cache policy) for record words that are read once per step.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt4(const uint32_t* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// N words from p; NT: with the non-temporal policy.
template <int N, bool NT = false>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t* out) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = NT ? load_nt4(p + 4 * i) : reinterpret_cast<const uint4*>(p)[i];
      out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0 && NT) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p) + i);
      out[2 * i] = v[0]; out[2 * i + 1] = v[1];
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[i];
      out[2 * i] = v.x; out[2 * i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = NT ? __builtin_nontemporal_load(p + i) : p[i];
  }
}

// Where each code of a word goes before the OR with 1.0: in-half position j (bit j*B) is
// shifted by sh(j) bits (left positive) to bit od(j) = j*B + sh(j), with od(j) + B <= 10.
template <int B>
struct Magic {
  static constexpr int NH = 16 / B;  // codes per 16-bit half
  static constexpr int NC = 32 / B;  // codes per word
  __host__ __device__ static constexpr int sh(int j) {
    return B == 2 ? (j < 2 ? 4 : (j < 5 ? 0 : -6))
         : B == 4 ? (j == 0 ? 6 : (j == 1 ? 0 : (j == 2 ? -2 : -6)))
                  : (j == 0 ? 2 : -6);
  }
  __host__ __device__ static constexpr int od(int j) { return j * B + sh(j); }
  // factor 2^(10 - od) folded into the partner operand of the code at word position p
  __host__ __device__ static constexpr float fold(int p) {
    return float(1 << (10 - od(p % NH)));
  }
};

// The NH fp16 pairs of one word: pair j holds the codes at positions j (low half) and
// j + NH (high half). MATRIX: the pairs feed matrix-core instructions. The compiler does not see
// what an asm statement writes, so it would not insert the wait states an MFMA needs after a VALU
// write of its source registers; there the and-or is written as plain code (the compiler still
// forms v_and_or_b32 from it, with the hazard known).
template <int B, bool MATRIX = false>
struct Unpacker {
  uint32_t magic, mk[10];  // mk[o]: the code bits at [o, o+B) of both halves
  __device__ __forceinline__ void init() {
    magic = vconst<0x3C003C00u>();
#pragma unroll
    for (int j = 0; j < Magic<B>::NH; ++j) {
      const int o = Magic<B>::od(j);
      const uint32_t m = ((1u << B) - 1) << o;
      uint32_t r;
      asm("v_mov_b32 %0, %1" : "=v"(r) : "v"(m | (m << 16)));
      mk[o] = r;
    }
  }
  __device__ __forceinline__ void run(uint32_t w, uint32_t* out) const { run_n<Magic<B>::NH>(w, out); }
  // the first N pairs only
  template <int N>
  __device__ __forceinline__ void run_n(uint32_t w, uint32_t* out) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int s = Magic<B>::sh(j);
      const uint32_t v = s > 0 ? (w << s) : (s < 0 ? (w >> -s) : w);
      out[j] = MATRIX ? ((v & mk[Magic<B>::od(j)]) | magic) : and_or(v, mk[Magic<B>::od(j)], magic);
    }
  }
};

// Value weights travel as fp16: A_t = fp16(p_t * s_t * 2^(10-o_t) * kVScale), with p <= 1 the
// softmax weight relative to the running max, s the token's value-group scale and 2^(10-o) <= F
// the fold factor (F = 64 at 2/4 bits, 256 at 8 bits). kVScale = 2^6 keeps the weights of a long
// context normal fp16 (relative rounding <= 2^-11) down to p ~ 2^-23 at unit-sized scales; it is
// safe while s * F * 2^6 <= 65504, i.e. every value scale of the record is at most kBigScale<B>.
// A record holding a larger scale (a wave vote decides) forms its weights at 2^-6 instead (safe
// for every fp16 scale: s <= 43669 at 2 bits), sums them on their own and adds that sum times
// 2^12, so the accumulators always carry kVScale units.
constexpr float kVScale = 64.0f;
constexpr float kVScaleBig = 1.0f / 64.0f;
constexpr float kVBigRatio = kVScale / kVScaleBig;  // 2^12
// fp16 bit pattern of the largest value scale a record may hold for the kVScale weights: 15.5
// (15.5 * 64 * 64 < 65504) at 2/4 bits, 3.875 (3.875 * 256 * 64 < 65504) at 8 bits
template <int BV>
__device__ __forceinline__ constexpr uint32_t big_scale_bits() { return BV == 8 ? 0x43C0u : 0x4BC0u; }

template <int D, int G>
struct WaveLds {
  float qt[G][4][D / 4 + 4];      // scaled, folded query per quarter (padded rows)
  float beta[G][4];               // quarter offsets (q . z minus the fold constant)
  float qsum[G][4];               // per-token key groups: the query summed over each quarter
  uint32_t A[G][D / 32][16 + 4];  // fp16 value weights per (value group, token pair), see kVScale
  float pw[G][32 + 4];            // window tokens: softmax weights
};

template <int D, int BK, int BV>
struct RecordRegs {
  uint32_t kc[2 * (D * BK / 128)];
  uint32_t vc[(D / 64) * BV];
  uint32_t kp[D / 64 < 2 ? 2 : D / 64];  // two words at D = 64 with per-token key groups
  uint32_t vp[D / 64];
};

// A record is read once per step: non-temporal loads (streaming cache policy), which stream the
// records in at a higher rate than the default policy while a lane's words of each record part
// come in at most two 16-byte loads (2- and 4-bit codes). With 8-bit codes a lane reads its 64
// contiguous bytes of a part in four loads, each of which touches every line of the part, and
// the streaming policy then measured much slower (2/8 bits at S = 64K: 98.6 against 72.6 us):
// those keep the default policy.
template <int D, int BK, int BV>
constexpr bool stream_records() {
  return 2 * (D * BK / 128) <= 8 && (D / 64) * BV <= 8;
}

// KT (per-token key groups): lane (P, Q) takes the key params of its tokens 2P, 2P+1 for the
// group of its quarter, two adjacent words at [P][group][t%2].
template <int D, int BK, int BV, bool KT = false>
__device__ __forceinline__ void load_record(const uint8_t* __restrict__ rec, int lane, RecordRegs<D, BK, BV>& r) {
  constexpr int E = D / 64, KW = 2 * (D * BK / 128), VW = E * BV;
  constexpr bool NT = stream_records<D, BK, BV>();
  load_words<KW, NT>(reinterpret_cast<const uint32_t*>(rec) + lane * KW, r.kc);
  load_words<VW, NT>(reinterpret_cast<const uint32_t*>(rec + rec_off_vcodes(D, BK)) + lane * VW, r.vc);
  if constexpr (KT) {
    constexpr int NKG = D / 32;
    const int kg = ((lane & 3) * (D / 4)) / 32;
    load_words<2, NT>(
        reinterpret_cast<const uint32_t*>(rec + rec_off_kparams(D, BK, BV)) + ((lane >> 2) * NKG + kg) * 2, r.kp);
  } else {
    load_words<E, NT>(reinterpret_cast<const uint32_t*>(rec + rec_off_kparams(D, BK, BV)) + lane * E, r.kp);
  }
  load_words<E, NT>(reinterpret_cast<const uint32_t*>(rec + rec_off_vparams(D, BK, BV)) + lane * E, r.vp);
}

// Wavefronts per decode workgroup; each takes every kWaves-th unit of the workgroup's chunk.
constexpr int kWaves = 4;

// State of one wavefront across the units it visits.
template <int D, int G>
struct WaveState {
  float m[G], l[G], bias[G], acc[G][D / 64];
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax step for one head: new scores s0, s1 (base-2 units) of tokens 2P, 2P+1.
// With SK, keep0 / keep1 (1 or 0) drop the weights of skipped slots (sinks' quantized copies).
template <int D, int G, bool SK = false>
__device__ __forceinline__ void softmax_step(WaveState<D, G>& st, int i, float s0, float s1, float& p0, float& p1,
                                             float keep0 = 1.0f, float keep1 = 1.0f) {
  // The running max only moves when some lane holds a larger score; a wave vote finds out
  // with one comparison, so the reduction and the rescale run only then.
  if (__any(fmaxf(s0, s1) > st.m[i])) {  // wave-uniform
    const float mx = wave_max_of_quads(fmaxf(s0, s1));
    const float alpha = fast_exp2(st.m[i] - mx);
    st.m[i] = mx;
    st.l[i] *= alpha;
    st.bias[i] *= alpha;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) st.acc[i][e] *= alpha;
  }
  p0 = fast_exp2(s0 - st.m[i]);
  p1 = fast_exp2(s1 - st.m[i]);
  if constexpr (SK) {
    p0 *= keep0;
    p1 *= keep1;
  }
  st.l[i] += p0 + p1;
}

// Multi-query decode: virtual head i sees the positions below lim[i] (query i % S_q of its
// head is the cache's token S - S_q + i % S_q). A masked score becomes kMaskScore, a finite
// value so far below any real score that its weight vanishes once a visible token is seen
// (in the same wave, across waves and across splits alike); -inf could leave a running max
// of -inf, and exp2(-inf - -inf) is not 0.
constexpr float kMaskScore = -1.0e30f;
template <int G>
struct Causal {
  int lim[G];
  int lim_min;  // no position below it is masked for any head
};

// One 32-token record of (b, h_kv), all G query heads. With SK, slots whose value scale
// carries the sign bit (sinks, attended from their fp16 rows instead) get no weight.
template <int D, int BK, int BV, int G, bool SK, bool KT>
__device__ __forceinline__ void process_record(const RecordRegs<D, BK, BV>& cur, WaveLds<D, G>& W, WaveState<D, G>& st,
                                               const Unpacker<BK>& upk, const Unpacker<BV>& upv,
                                               const float (&qs)[G][D / 64], const float (&qf)[G][D / 64],
                                               float vf0, float vf1, int lane, const Causal<G>& cz, int tok0) {
  constexpr int E = D / 64, DQ = D / 4, WQ = D * BK / 128, NKG = D / 32;
  using MK = Magic<BK>;
  using MV = Magic<BV>;
  const int P = lane >> 2, Q = lane & 3;
  const int kcons = (lane * E) / 32;
  float keep0 = 1.0f, keep1 = 1.0f;
  if constexpr (SK) {
    // value-param entry e of this lane belongs to token 2P + ((lane * E + e) & 1): with E >= 2
    // the lane holds both of its tokens, with E = 1 the other one sits in lane ^ 1
    if constexpr (E >= 2) {
      keep0 = (cur.vp[0] & 0x8000u) ? 0.0f : 1.0f;
      keep1 = (cur.vp[1] & 0x8000u) ? 0.0f : 1.0f;
    } else {
      const uint32_t own = cur.vp[0] & 0x8000u;
      const uint32_t other = uint32_t(__builtin_amdgcn_mov_dpp(int(own), kQuadXor1, 0xF, 0xF, false));
      const uint32_t f0 = (lane & 1) ? other : own, f1 = (lane & 1) ? own : other;
      keep0 = f0 ? 0.0f : 1.0f;
      keep1 = f1 ? 0.0f : 1.0f;
    }
  }

  // value scales beyond big_scale_bits (the sign bit is the sink marker, not the scale's):
  // this record's weights are formed at kVScaleBig (wave-uniform)
  bool bigv;
  {
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) mx = max(mx, cur.vp[e] & 0x7FFFu);
    bigv = __any(mx > big_scale_bits<BV>());
  }
  const float vw0 = bigv ? vf0 * (1.0f / kVBigRatio) : vf0, vw1 = bigv ? vf1 * (1.0f / kVBigRatio) : vf1;
  const float amul = bigv ? kVBigRatio : 1.0f;

  // ---- producer: folded scaled query and quarter offsets (per-token key groups: set once
  // per launch, nothing to do per record)
#pragma unroll
  for (int i = 0; i < G && !KT; ++i) {
    float bp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int ch = lane * E + e;
      const float qt = qf[i][e] * lo_f(cur.kp[e]);
      W.qt[i][ch / DQ][ch % DQ] = qt;
      bp += qs[i][e] * hi_f(cur.kp[e]) - qt;
    }
    bp = row_sum16(bp);
    if ((lane & 15) == 0) W.beta[i][lane >> 4] = bp;
  }
  wave_sync();

  // ---- keys
  float s[G][2];
#pragma unroll
  for (int i = 0; i < G; ++i) s[i][0] = s[i][1] = KT ? 0.0f : W.beta[i][Q];
  if constexpr (G == 1) {
    // word by word: few live registers
#pragma unroll
    for (int w = 0; w < WQ; ++w) {
      uint32_t k0[MK::NH], k1[MK::NH];
      upk.run(cur.kc[w], k0);
      upk.run(cur.kc[WQ + w], k1);
      float qv[MK::NC];
#pragma unroll
      for (int c = 0; c < MK::NC; c += 4) {
        const float4 t4 = *reinterpret_cast<const float4*>(&W.qt[0][Q][w * MK::NC + c]);
        qv[c] = t4.x; qv[c + 1] = t4.y; qv[c + 2] = t4.z; qv[c + 3] = t4.w;
      }
#pragma unroll
      for (int j = 0; j < MK::NH; ++j) {
        s[0][0] = __builtin_fmaf(qv[j], lo_f(k0[j]), s[0][0]);
        s[0][1] = __builtin_fmaf(qv[j], lo_f(k1[j]), s[0][1]);
        s[0][0] = __builtin_fmaf(qv[j + MK::NH], hi_f(k0[j]), s[0][0]);
        s[0][1] = __builtin_fmaf(qv[j + MK::NH], hi_f(k1[j]), s[0][1]);
      }
    }
  } else {
    // unpack the whole quarter once; every head reuses it
    uint32_t kr[2][WQ][MK::NH];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int w = 0; w < WQ; ++w) upk.run(cur.kc[tp * WQ + w], kr[tp][w]);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float qv[DQ];
#pragma unroll
      for (int c = 0; c < DQ; c += 4) {
        const float4 t4 = *reinterpret_cast<const float4*>(&W.qt[i][Q][c]);
        qv[c] = t4.x; qv[c + 1] = t4.y; qv[c + 2] = t4.z; qv[c + 3] = t4.w;
      }
#pragma unroll
      for (int w = 0; w < WQ; ++w)
#pragma unroll
        for (int j = 0; j < MK::NH; ++j) {
          const int c = w * MK::NC + j;
          s[i][0] = __builtin_fmaf(qv[c], lo_f(kr[0][w][j]), s[i][0]);
          s[i][1] = __builtin_fmaf(qv[c], lo_f(kr[1][w][j]), s[i][1]);
          s[i][0] = __builtin_fmaf(qv[c + MK::NH], hi_f(kr[0][w][j]), s[i][0]);
          s[i][1] = __builtin_fmaf(qv[c + MK::NH], hi_f(kr[1][w][j]), s[i][1]);
        }
    }
  }

  if constexpr (KT) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      // quarter partial sum_c q~_c (1 + c_code 2^(o-10)) minus the fold constant, times the
      // token's group scale, plus its zero times the quarter's query sum
      const float fq = W.beta[i][Q], qsm = W.qsum[i][Q];
      s[i][0] = __builtin_fmaf(lo_f(cur.kp[0]), s[i][0] - fq, hi_f(cur.kp[0]) * qsm);
      s[i][1] = __builtin_fmaf(lo_f(cur.kp[1]), s[i][1] - fq, hi_f(cur.kp[1]) * qsm);
    }
  }
  // one query row per KV head (G = 1) means one query: nothing is ever masked
  if (G > 1 && tok0 + kGroup > cz.lim_min) {  // wave-uniform: a record holding some query's future
    // a masked quarter partial makes the whole score at least this far below any real one
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (tok0 + 2 * P >= cz.lim[i]) s[i][0] = kMaskScore;
      if (tok0 + 2 * P + 1 >= cz.lim[i]) s[i][1] = kMaskScore;
    }
  }

#pragma unroll
  for (int i = 0; i < G; ++i) {
    float s0 = s[i][0], s1 = s[i][1];
    s0 += dpp<kQuadXor1>(s0);
    s1 += dpp<kQuadXor1>(s1);
    s0 += dpp<kQuadXor2>(s0);
    s1 += dpp<kQuadXor2>(s1);
    float p0, p1;
    softmax_step<D, G, SK>(st, i, s0, s1, p0, p1, keep0, keep1);
    // ---- producer: fp16 folded value weights and the zero-term bias (in kVScale units), the
    // record's part summed on its own first
    float br = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // entry e of this lane: token t, value group k (the value-param dword lane*E + e)
      const int idx = lane * E + e;
      const int tp = idx & 1, k = (idx >> 1) % NKG, t = 2 * P + tp;
      const float p = tp ? p1 : p0;
      const float vfold = (tp ? vw1 : vw0);  // 2^(10-o_t) * kVScale, or * kVScaleBig
      const __half a16 = __float2half_rn((p * vfold) * lo_f(cur.vp[e]));
      br = __builtin_fmaf(-__half2float(a16), amul, __builtin_fmaf(p * kVScale, hi_f(cur.vp[e]), br));
      const int dw = (t / MV::NC) * MV::NH + (t % MV::NC) % MV::NH, hf = (t % MV::NC) / MV::NH;
      reinterpret_cast<__half*>(&W.A[i][k][dw])[hf] = a16;
    }
    st.bias[i] += br;
  }
  wave_sync();

  // ---- values: v_dot2_f32_f16 of (weight pair) x (code pair); a word = NC tokens of a channel
  // (x: the chains' accumulators, st.acc itself, or zeros for a record with kVScaleBig weights)
  using h2 = _Float16 __attribute__((ext_vector_type(2)));
  auto values = [&](float (&x)[G][E]) {
    if constexpr (G == 1) {
#pragma unroll
      for (int w = 0; w < BV; ++w) {
        uint32_t vr[E][MV::NH];
#pragma unroll
        for (int e = 0; e < E; ++e) upv.run(cur.vc[e * BV + w], vr[e]);
        uint32_t av[MV::NH];
#pragma unroll
        for (int j = 0; j < MV::NH; j += (MV::NH >= 4 ? 4 : 2)) {
          if constexpr (MV::NH >= 4) {
            const uint4 t4 = *reinterpret_cast<const uint4*>(&W.A[0][kcons][w * MV::NH + j]);
            av[j] = t4.x; av[j + 1] = t4.y; av[j + 2] = t4.z; av[j + 3] = t4.w;
          } else {
            const uint2 t2 = *reinterpret_cast<const uint2*>(&W.A[0][kcons][w * MV::NH + j]);
            av[j] = t2.x; av[j + 1] = t2.y;
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int j = 0; j < MV::NH; ++j)
            x[0][e] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, av[j]), __builtin_bit_cast(h2, vr[e][j]), x[0][e],
                                             false);
      }
    } else {
      uint32_t vr[E][BV][MV::NH];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int w = 0; w < BV; ++w) upv.run(cur.vc[e * BV + w], vr[e][w]);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        uint32_t av[16];
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const uint4 t4 = *reinterpret_cast<const uint4*>(&W.A[i][kcons][j]);
          av[j] = t4.x; av[j + 1] = t4.y; av[j + 2] = t4.z; av[j + 3] = t4.w;
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int w = 0; w < BV; ++w)
#pragma unroll
            for (int j = 0; j < MV::NH; ++j)
              x[i][e] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, av[w * MV::NH + j]),
                                               __builtin_bit_cast(h2, vr[e][w][j]), x[i][e], false);
      }
    }
  };
  // Each record is summed from zero and joins the running sums once: the converted codes carry
  // their constant 1 (up to 64 times the code's own part, removed only at the end through the
  // bias), so a running sum is much larger than the value it stands for, and adding every code
  // pair to it directly would round away the low bits of small weights.
  {
    float x[G][E];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) x[i][e] = 0.0f;
    values(x);
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[i][e] = __builtin_fmaf(x[i][e], amul, st.acc[i][e]);
  }
  wave_sync();
}

// Up to 32 fp16 window tokens (tokens tbase .. tbase + nvalid - 1 of the window).
// Token tnew of the unit (when 0 <= tnew < nvalid) is the one this launch appends: its rows
// come from kn / vn instead of the window.
// With KT the query and the accumulators run in permuted channel order, like the stored window
// and sink rows; only the token this launch appends (kn, vn, in channel order) is read through
// the permutations pk, pv.
template <int D, int G, bool KT = false>
__device__ __forceinline__ void process_window(const __half* __restrict__ wk, const __half* __restrict__ wv, int nvalid,
                                               int tnew, const __half* kn, const __half* vn,
                                               WaveLds<D, G>& W, WaveState<D, G>& st, const float (&qs)[G][D / 64],
                                               int lane, const Causal<G>& cz, int tok0,
                                               const int32_t* __restrict__ pos, const uint8_t* __restrict__ pk = nullptr,
                                               const uint8_t* __restrict__ pv = nullptr) {
  // token t of the unit is at position pos[t] (sinks chosen by norm), else tok0 + t
  constexpr int E = D / 64, DQ = D / 4;
  const int P = lane >> 2, Q = lane & 3;
  const int kcons = (lane * E) / 32;
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int ch = lane * E + e;
      W.qt[i][ch / DQ][ch % DQ] = qs[i][e];
    }
  wave_sync();
  const int t0 = 2 * P, t1 = 2 * P + 1;
  const int t0c = min(t0, nvalid - 1), t1c = min(t1, nvalid - 1);
  const uint32_t* k0p = reinterpret_cast<const uint32_t*>((t0c == tnew ? kn : wk + t0c * D) + Q * DQ);
  const uint32_t* k1p = reinterpret_cast<const uint32_t*>((t1c == tnew ? kn : wk + t1c * D) + Q * DQ);
  uint32_t k0w[DQ / 2], k1w[DQ / 2];
#pragma unroll
  for (int c = 0; c < DQ / 2; ++c) {
    k0w[c] = k0p[c];
    k1w[c] = k1p[c];
  }
  if (KT && (t0c == tnew || t1c == tnew)) {  // the appended token, gathered into permuted order
    const uint16_t* rn = reinterpret_cast<const uint16_t*>(kn);
#pragma unroll
    for (int c = 0; c < DQ / 2; ++c) {
      const uint32_t w = uint32_t(rn[pk[Q * DQ + 2 * c]]) | (uint32_t(rn[pk[Q * DQ + 2 * c + 1]]) << 16);
      if (t0c == tnew) k0w[c] = w;
      if (t1c == tnew) k1w[c] = w;
    }
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int c = 0; c < DQ / 2; ++c) {
      const float qa = W.qt[i][Q][2 * c], qb = W.qt[i][Q][2 * c + 1];
      s0 = __builtin_fmaf(qa, lo_f(k0w[c]), s0);
      s0 = __builtin_fmaf(qb, hi_f(k0w[c]), s0);
      s1 = __builtin_fmaf(qa, lo_f(k1w[c]), s1);
      s1 = __builtin_fmaf(qb, hi_f(k1w[c]), s1);
    }
    s0 += dpp<kQuadXor1>(s0);
    s0 += dpp<kQuadXor2>(s0);
    s1 += dpp<kQuadXor1>(s1);
    s1 += dpp<kQuadXor2>(s1);
    if constexpr (G > 1) {
      const int a0 = pos ? pos[t0c] : tok0 + t0, a1 = pos ? pos[t1c] : tok0 + t1;
      if (a0 >= cz.lim[i]) s0 = kMaskScore;
      if (a1 >= cz.lim[i]) s1 = kMaskScore;
    }
    if (t0 >= nvalid) s0 = -INFINITY;
    if (t1 >= nvalid) s1 = -INFINITY;
    float p0, p1;
    softmax_step<D, G>(st, i, s0, s1, p0, p1);
    if (Q == 0) *reinterpret_cast<float2*>(&W.pw[i][2 * P]) = make_float2(p0 * kVScale, p1 * kVScale);
  }
  wave_sync();
  // values: 8 rows in flight at a time, each loaded once for all G heads. Rows past nvalid are
  // clamped to the last valid one; their weights are 0 (their scores were -inf).
  constexpr int VB = 8;
  for (int tb = 0; tb < nvalid; tb += VB) {
    float v[VB][E];
#pragma unroll
    for (int k = 0; k < VB; ++k) {
      const int t = min(tb + k, nvalid - 1);
      const __half* vrow = t == tnew ? vn : wv + t * D;
      if (KT && t == tnew) {  // the appended token, gathered into permuted order
#pragma unroll
        for (int e = 0; e < E; ++e) v[k][e] = __half2float(vrow[pv[lane * E + e]]);
      } else if constexpr (E == 2) {
        const uint32_t vw = reinterpret_cast<const uint32_t*>(vrow)[lane];
        v[k][0] = lo_f(vw);
        v[k][1] = hi_f(vw);
      } else {
        v[k][0] = __half2float(vrow[lane]);
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int k = 0; k < VB; ++k) {
        const float a = W.pw[i][tb + k];
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[i][e] = __builtin_fmaf(a, v[k][e], st.acc[i][e]);
      }
  }
  wave_sync();
}

// Split partials cross workgroups (and XCDs, each with its own L2) inside one launch. They are
// written and read with device-scope relaxed atomics, which the hardware performs coherently
// across the XCDs (cache-policy bit sc1) without writing back or invalidating a whole L2, which
// a device-scope fence would do in every wave.
__device__ __forceinline__ void put_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_out(void* out, int out_fp32, int64_t idx, float v) {
  if (out_fp32)
    static_cast<float*>(out)[idx] = v;
  else
    static_cast<__half*>(out)[idx] = __float2half_rn(v);
}

// Merge the nv split partials (acc[D], m, l) of the G query heads row0 .. row0+G-1 into the
// output, by one workgroup of NT threads: T threads per output element each fold a strided
// share of the splits (batches of 8 loads in flight), then meet through LDS.
// pv (per-token key groups): partial channel ch is output channel pv[ch].
template <int D, int G, int NT = 64 * kWaves>
__device__ __forceinline__ void merge_splits(const float* __restrict__ ws, int64_t row0, int n_split, int nv,
                                             float (*mrg)[NT], void* out, int out_fp32,
                                             const uint8_t* __restrict__ pv = nullptr) {
  constexpr int NOUT = G * D;
  constexpr int T = NOUT >= NT ? 1 : NT / NOUT;
  constexpr int NO = NOUT >= NT ? NT : NOUT;  // output elements per pass
  const int tid = threadIdx.x, r = tid / NO;
  for (int oi = tid % NO; oi < NOUT; oi += NO) {
    const int i = oi / D, ch = oi % D;
    const float* base = ws + (row0 + i) * n_split * (D + 4);
    float M = -INFINITY, Ls = 0.f, O = 0.f;
    for (int s0 = r; s0 < nv; s0 += 8 * T) {
      float m[8], l[8], o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sk = s0 + k * T;
        const float* p = base + min(sk, nv - 1) * (D + 4);  // clamped: every load in bounds
        const float mv = get_partial(p + D);
        m[k] = sk < nv ? mv : -INFINITY;
        l[k] = get_partial(p + D + 1);
        o[k] = get_partial(p + ch);
      }
      float mx = M;
#pragma unroll
      for (int k = 0; k < 8; ++k) mx = fmaxf(mx, m[k]);
      const float sc = fast_exp2(M - mx);  // 0 while M is still -inf
      O *= sc;
      Ls *= sc;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = fast_exp2(m[k] - mx);
        O = __builtin_fmaf(w, o[k], O);
        Ls = __builtin_fmaf(w, l[k], Ls);
      }
      M = mx;
    }
    if constexpr (T == 1) {
      store_out(out, out_fp32, (row0 + i) * D + (pv ? pv[ch] : ch), O / Ls);
    } else {
      mrg[0][tid] = M;
      mrg[1][tid] = Ls;
      mrg[2][tid] = O;
    }
  }
  if constexpr (T > 1) {
    __syncthreads();
    if (tid < NO) {
      float M = -INFINITY;
#pragma unroll
      for (int j = 0; j < T; ++j) M = fmaxf(M, mrg[0][tid + j * NO]);
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const float w = fast_exp2(mrg[0][tid + j * NO] - M);  // a share with no split: 0
        Ls = __builtin_fmaf(w, mrg[1][tid + j * NO], Ls);
        O = __builtin_fmaf(w, mrg[2][tid + j * NO], O);
      }
      store_out(out, out_fp32, (row0 + tid / D) * D + (pv ? pv[tid % D] : tid % D), O / Ls);
    }
  }
}

// The identity permutation, used by SKVQ sequences before their first chunk fixes theirs.
__device__ const uint8_t kIdentityPerm[128] = {
    0,   1,   2,   3,   4,   5,   6,   7,   8,   9,   10,  11,  12,  13,  14,  15,  16,  17,  18,  19,  20,  21,
    22,  23,  24,  25,  26,  27,  28,  29,  30,  31,  32,  33,  34,  35,  36,  37,  38,  39,  40,  41,  42,  43,
    44,  45,  46,  47,  48,  49,  50,  51,  52,  53,  54,  55,  56,  57,  58,  59,  60,  61,  62,  63,  64,  65,
    66,  67,  68,  69,  70,  71,  72,  73,  74,  75,  76,  77,  78,  79,  80,  81,  82,  83,  84,  85,  86,  87,
    88,  89,  90,  91,  92,  93,  94,  95,  96,  97,  98,  99,  100, 101, 102, 103, 104, 105, 106, 107, 108, 109,
    110, 111, 112, 113, 114, 115, 116, 117, 118, 119, 120, 121, 122, 123, 124, 125, 126, 127};

// SK: the cache has sink slots (the sinks present are the leading non-negative positions);
// KT: SKVQ records (per-token key groups, permuted channels, see layout.h).
template <int D, int BK, int BV, int G, bool SK, bool KT>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(G == 1 ? 4 : (G <= 4 ? 2 : 1))))
void decode_split_kernel(const uint8_t* __restrict__ buf, Layout L, DecodeShape ds, PerSeq seq,
                         const __half* __restrict__ q, float* __restrict__ ws, uint32_t* __restrict__ sync,
                         void* __restrict__ out, const __half* __restrict__ k_app, const __half* __restrict__ v_app,
                         uint8_t* bufw) {
  constexpr int E = D / 64, DQ = D / 4, NKG = D / 32;
  using MK = Magic<BK>;
  using MV = Magic<BV>;

  __shared__ __attribute__((aligned(16))) union {
    WaveLds<D, G> w[kWaves];
    float res[kWaves][G][D + 4];
    float mrg[3][64 * kWaves];
  } sh;
  __shared__ int sh_last;

  int sigma = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (ds.n_hi > 0) {  // split-major: workgroup id = (split * B + sequence) * H_kv + KV head
    const int id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int pairs = L.Hkv * L.B;
    sigma = id / pairs;
    h = id % L.Hkv;
    b = (id % pairs) / L.Hkv;
  }
  // the wave index is wave-uniform: record indices and addresses stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // The plan comes from the host's lengths (seq: quantized tokens, window tokens before this
  // launch's append, sinks present), never from the device copy: with an append, the split that
  // finishes last rewrites the device window length inside this launch, and a split that read
  // it afterwards would see a different number of units than its siblings.
  const int nq = max(0, min(seq.a[b], L.max_groups * kGroup));
  const int nr_old = max(0, min(seq.b[b], L.R));
  const int nr = min(nr_old + ds.append, L.R);  // with an append: the new token is window slot nr_old
  const int ngroups = nq / kGroup;
  // with sinks one more unit, the last: their fp16 rows
  const int nsink = SK ? max(0, min(seq.c[b], L.NS)) : 0;
  const bool sinks = nsink > 0;
  // positions: SKVQ sinks are tokens 0 .. nsink - 1 and its records start after them
  const int pos0 = KT ? nsink : 0;
  Causal<G> cz;
  {
    const int S = pos0 + nq + nr;
#pragma unroll
    for (int i = 0; i < G; ++i) cz.lim[i] = S - (ds.nqry - 1 - i % ds.nqry);
    cz.lim_min = S - (ds.nqry - 1);
  }
  const int nunits = ngroups + (nr + kGroup - 1) / kGroup + (sinks ? 1 : 0);
  const int hi_units = ds.n_hi * ds.chunk_hi;  // units of the first n_hi splits
  auto split_start = [&](int sg) {
    return sg <= ds.n_hi ? sg * ds.chunk_hi : hi_units + (sg - ds.n_hi) * ds.chunk;
  };
  const int u0 = split_start(sigma);
  if (u0 >= nunits) return;
  const int u1 = min(split_start(sigma + 1), nunits);
  const int uq = min(u1, ngroups);  // end of the quantized units of this split

  WaveLds<D, G>& W = sh.w[wave];
  const int P = lane >> 2, Q = lane & 3;
  const int kcons = (lane * E) / 32;

  Unpacker<BK> upk;
  Unpacker<BV> upv;
  upk.init();
  upv.init();

  // KT: the query in permuted channel order (channel ch of the records is pk[ch]); a sequence
  // with no chunk quantized yet has no permutation of its own (any one is consistent for its
  // fp16 rows): the identity
  const uint8_t* pk = KT ? (nq > 0 ? buf + L.perm(b, h) : kIdentityPerm) : nullptr;
  const uint8_t* pv = KT ? (nq > 0 ? pk + D : kIdentityPerm) : nullptr;
  float qs[G][E], qf[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int ch = lane * E + e;
      qs[i][e] = __half2float(q[(int64_t(b) * ds.n_q_heads + h * G + i) * D + (KT ? pk[ch] : ch)]) * ds.qscale;
      qf[i][e] = qs[i][e] * MK::fold((ch % DQ) % MK::NC);
    }
  if constexpr (KT) {
    // no per-channel key scale: the folded query, its fold constant and its plain sum per
    // quarter are the same for every record
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float fq = 0.f, qsm = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int ch = lane * E + e;
        W.qt[i][ch / DQ][ch % DQ] = qf[i][e];
        fq += qf[i][e];
        qsm += qs[i][e];
      }
      fq = row_sum16(fq);
      qsm = row_sum16(qsm);
      if ((lane & 15) == 0) {
        W.beta[i][lane >> 4] = fq;
        W.qsum[i][lane >> 4] = qsm;
      }
    }
    wave_sync();
  }
  const float vf0 = MV::fold((2 * P) % MV::NC) * kVScale, vf1 = MV::fold((2 * P + 1) % MV::NC) * kVScale;

  WaveState<D, G> st;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.f;
    st.bias[i] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[i][e] = 0.f;
  }

  // Quantized records, the next one loaded while the current one is computed. Prefetch loads
  // are unconditional (their record index is clamped into the buffer: the last one of a
  // wave re-reads a record it never uses) so that the compiler's memory-counter waits stay
  // exact: a conditional load at a control-flow merge makes it wait for the prefetch too.
  // With streamed records each register set is loaded in one place of the loop (the second set
  // where the loop begins): with a second load site ahead of the loop, the two sites of a set
  // were given different registers, and the copy between them waited for every load in flight.
  // Up to 4 rows per KV head the two sets fit the registers; beyond that (and with 8-bit codes
  // at more than one row) the next record goes to one set that is copied into the current one.
  const uint8_t* rec0 = buf + L.record(b, h, 0);
  const uint64_t rb = L.rec_bytes;
  const int ulast = max(uq - 1, 0);
  int u = u0 + wave;
  if constexpr (G == 1 || (G <= 4 && stream_records<D, BK, BV>())) {
    RecordRegs<D, BK, BV> ra, rbuf;
    if (u < uq) {
      load_record<D, BK, BV, KT>(rec0 + u * rb, lane, ra);
      if constexpr (!stream_records<D, BK, BV>())
        load_record<D, BK, BV, KT>(rec0 + min(u + kWaves, ulast) * rb, lane, rbuf);
      while (true) {
        if constexpr (stream_records<D, BK, BV>())
          load_record<D, BK, BV, KT>(rec0 + min(u + kWaves, ulast) * rb, lane, rbuf);
        process_record<D, BK, BV, G, SK, KT>(ra, W, st, upk, upv, qs, qf, vf0, vf1, lane, cz, pos0 + u * kGroup);
        u += kWaves;
        if (u >= uq) break;
        load_record<D, BK, BV, KT>(rec0 + min(u + kWaves, ulast) * rb, lane, ra);
        process_record<D, BK, BV, G, SK, KT>(rbuf, W, st, upk, upv, qs, qf, vf0, vf1, lane, cz, pos0 + u * kGroup);
        u += kWaves;
        if (u >= uq) break;
        if constexpr (!stream_records<D, BK, BV>())
          load_record<D, BK, BV, KT>(rec0 + min(u + kWaves, ulast) * rb, lane, rbuf);
      }
    }
  } else {
    RecordRegs<D, BK, BV> cur, nxt;
    if (u < uq) {
      load_record<D, BK, BV, KT>(rec0 + u * rb, lane, cur);
      for (; u < uq; u += kWaves) {
        load_record<D, BK, BV, KT>(rec0 + min(u + kWaves, ulast) * rb, lane, nxt);
        process_record<D, BK, BV, G, SK, KT>(cur, W, st, upk, upv, qs, qf, vf0, vf1, lane, cz, pos0 + u * kGroup);
        cur = nxt;
      }
    }
  }
  // window units, then the sink unit
  for (; u < u1; u += kWaves) {
    const bool sink_unit = sinks && u == nunits - 1;
    const int tbase = (u - ngroups) * kGroup;
    const int nvalid = sink_unit ? nsink : min(kGroup, nr - tbase);
    const __half* wk = sink_unit ? reinterpret_cast<const __half*>(buf + L.sink_k(b, h))
                                 : reinterpret_cast<const __half*>(buf + L.wk_off + L.window(b, h)) + tbase * D;
    const __half* wv = sink_unit ? reinterpret_cast<const __half*>(buf + L.sink_v(b, h))
                                 : reinterpret_cast<const __half*>(buf + L.wv_off + L.window(b, h)) + tbase * D;
    // the appended token in this unit, if 0 <= tnew < nvalid
    const int tnew = (ds.append && !sink_unit) ? nr_old - tbase : -1;
    const int64_t tok = (int64_t(b) * L.Hkv + h) * D;
    const __half* kn = ds.append ? k_app + tok : nullptr;
    const __half* vn = ds.append ? v_app + tok : nullptr;
    const int32_t* sink_pos = (sink_unit && !KT) ? reinterpret_cast<const int32_t*>(buf + L.sink_pos(b, h)) : nullptr;
    process_window<D, G, KT>(wk, wv, nvalid, tnew, kn, vn, W, st, qs, lane, cz,
                             sink_unit ? 0 : pos0 + nq + tbase, sink_pos, pk, pv);
    if (tnew >= 0 && tnew < nvalid) {  // store the appended token in its slot (no read of it here)
      __half* dk = reinterpret_cast<__half*>(bufw + L.wk_off + L.window(b, h)) + nr_old * D;
      __half* dv = reinterpret_cast<__half*>(bufw + L.wv_off + L.window(b, h)) + nr_old * D;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = lane * E + e;
        dk[c] = kn[KT ? pk[c] : c];
        dv[c] = vn[KT ? pv[c] : c];
      }
    }
  }

  // ---- finish the wave: l counted once per quad, bias summed over its producer lanes
  float lt[G], o[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float v = (Q == 0) ? st.l[i] : 0.f;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) v += __shfl_xor(v, msk, 64);
    lt[i] = v;
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float bsum = value_group_bias<D>(st.bias[i], lane);
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = (st.acc[i][e] + bsum) * (1.0f / kVScale);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < G; ++i) {
#pragma unroll
    for (int e = 0; e < E; ++e) sh.res[wave][i][lane * E + e] = o[i][e];
    if (lane == 0) {
      sh.res[wave][i][D] = st.m[i];
      sh.res[wave][i][D + 1] = lt[i];
    }
  }
  __syncthreads();

  // ---- combine the waves: the partial of each query head, or the output when this
  // workgroup is the sequence's only split
  const int nvalid = min(ds.n_split, nunits <= hi_units ? (nunits + ds.chunk_hi - 1) / ds.chunk_hi
                                                       : ds.n_hi + (nunits - hi_units + ds.chunk - 1) / ds.chunk);
  const int64_t row0 = int64_t(b) * ds.n_q_heads + h * G;  // first query head of this KV head
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kWaves) {
    const int i = idx / D, ch = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh.res[w][i][D]);
    float O = 0.f, Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sh.res[w][i][D];
      if (mw != -INFINITY) {
        const float wgt = fast_exp2(mw - M);
        O += wgt * sh.res[w][i][ch];
        Lsum += wgt * sh.res[w][i][D + 1];
      }
    }
    if (nvalid == 1) {
      store_out(out, ds.out_fp32, (row0 + i) * D + (KT ? pv[ch] : ch), O / Lsum);
      continue;
    }
    float* dst = ws + ((row0 + i) * ds.n_split + sigma) * (D + 4);
    put_partial(dst + ch, O);
    if (ch == 0) {
      put_partial(dst + D, M);
      put_partial(dst + D + 1, Lsum);
    }
  }
  // With an append, the split that finishes (b, h_kv) last advances its device lengths: every
  // split of (b, h_kv) has read them by then.
  int32_t* len_w = reinterpret_cast<int32_t*>(bufw + L.lengths(b, h));
  if (nvalid == 1) {
    if (ds.append && threadIdx.x == 0) len_w[1] = nr;
    return;
  }

  // ---- the last split of (b, h_kv) to finish merges every partial. Each wave waits until its
  // partial stores are acknowledged at device scope, the workgroup meets, and only then does
  // one thread move the counter (a device-scope atomic, performed coherently); the workgroup
  // that brings it to nvalid reads every partial back the same coherent way, then clears the
  // counter for the next call.
  // Why this orders the partials without release/acquire fences: every partial store and load
  // is a device-scope atomic, so it is performed at the device's coherence point (past the
  // eight XCD L2s; no line of it stays in a non-coherent cache). s_waitcnt(0) returns only once
  // this wave's stores are acknowledged there, the barrier extends that to the workgroup, and
  // the counter increment is issued after it, also at the coherence point. A split that reads
  // the count nvalid therefore increments after every other split's partials were performed,
  // and its atomic loads read them from that same point. A fence would add an L2 writeback and
  // invalidate in every wave (measured 204 us per long decode), which nothing here needs.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* cnt = sync + (int64_t(b) * L.Hkv + h);
  if (threadIdx.x == 0) sh_last = atomicAdd(cnt, 1u) + 1u == uint32_t(nvalid);
  __syncthreads();
  if (!sh_last) return;
  merge_splits<D, G>(ws, row0, ds.n_split, nvalid, sh.mrg, out, ds.out_fp32, pv);
  if (threadIdx.x == 0) {
    if (ds.append) len_w[1] = nr;
    atomicExch(cnt, 0u);
  }
}

// ------------------------------------------------------------------------------------
template <int D, int BK, int BV, int G, bool SK, bool KT>
static hipError_t launch_split_t(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq,
                                 const void* q, float* ws, void* out, const void* ka, const void* va, hipStream_t s,
                                 hipEvent_t e0, hipEvent_t e1) {
  dim3 grid(ds.n_split, L.Hkv, L.B);
  uint32_t* sync = reinterpret_cast<uint32_t*>(buf + L.sync_off);
  const __half* qh = static_cast<const __half*>(q);
  const __half* kh = static_cast<const __half*>(ka);
  const __half* vh = static_cast<const __half*>(va);
  if (e0 || e1)
    hipExtLaunchKernelGGL((decode_split_kernel<D, BK, BV, G, SK, KT>), grid, dim3(64 * kWaves), 0, s, e0, e1, 0,
                          static_cast<const uint8_t*>(buf), L, ds, seq, qh, ws, sync, out, kh, vh, buf);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, BK, BV, G, SK, KT>), grid, dim3(64 * kWaves), 0, s,
                       static_cast<const uint8_t*>(buf), L, ds, seq, qh, ws, sync, out, kh, vh, buf);
  return hipGetLastError();
}

template <int D, int BK, int BV, bool SK, bool KT>
static hipError_t launch_split_g(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq,
                                 const void* q, float* ws, void* out, const void* ka, const void* va, hipStream_t s,
                                 hipEvent_t e0, hipEvent_t e1) {
  switch (ds.G) {
    case 1: return launch_split_t<D, BK, BV, 1, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 2: return launch_split_t<D, BK, BV, 2, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 4: return launch_split_t<D, BK, BV, 4, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 8: return launch_split_t<D, BK, BV, 8, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool SK, bool KT>
static hipError_t launch_split_d(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq,
                                 const void* q, float* ws, void* out, const void* ka, const void* va, hipStream_t s,
                                 hipEvent_t e0, hipEvent_t e1) {
  switch (L.bk * 16 + L.bv) {
    case 0x22: return launch_split_g<D, 2, 2, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x24: return launch_split_g<D, 2, 4, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x28: return launch_split_g<D, 2, 8, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x42: return launch_split_g<D, 4, 2, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x44: return launch_split_g<D, 4, 4, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x48: return launch_split_g<D, 4, 8, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x82: return launch_split_g<D, 8, 2, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x84: return launch_split_g<D, 8, 4, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    case 0x88: return launch_split_g<D, 8, 8, SK, KT>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
