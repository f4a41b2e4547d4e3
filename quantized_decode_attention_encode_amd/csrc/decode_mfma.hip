// decode_mfma.hip - decode attention for 4 or 8 query rows per KV head (GQA groups, or a few
// queries per head) with both per-record products on the matrix cores.
//
// The decode of decode_kernel.h spends one VALU op per (key code, query row) and one per
// (value code pair, row): at 4 rows it is VALU-bound. Here, per 32-token record and wave:
//   scores  S[r][token] = sum_c A[r][c] * code'[c][token] on v_mfma_f32_16x16x32_f16: A = the
//           folded scaled query q~'[row][c] = q s_c 2^(10-o) split into an fp16 high part (A row
//           2 row) and low part (row 2 row + 1), formed per record in LDS; B = the record's key
//           codes as exact fp16 numbers 1 + c 2^(o-10) (the exponent-OR of decode_kernel.h). The
//           constant "1" terms and the zeros leave through beta per row (the accumulator's start),
//           as in the VALU decode; each lane adds its high and low rows, so lanes 16 g .. 16 g + 15
//           hold the scores of query rows 2 g and 2 g + 1.
//   values  O^T[ch][row] += sum_t vcode'[ch][t] * A_w[t][row]: A = the value codes as exact fp16
//           numbers, B = the fp16 folded weights p s 2^(10-o) kVScale per (row, value group),
//           written by the weight producers in exactly the token order of the converted codes.
// The key chunks are loaded lane = token pair + 16 x quarter (a permutation of the VALU decode's
// lane = 4 x pair + quarter), which makes each lane's converted key words its B fragments: column
// m of a 16-token tile is token pair m, and k-group g is quarter g. The value codes reach their
// A layout (a channel per lane, 8 tokens per k-group) through an LDS staging copy.
// Window and sink units go through process_window of decode_kernel.h with its own running state,
// merged with the matrix-core state at the end of the wave. Split partials and the in-kernel
// merge are the VALU decode's.
#include "decode_kernel.h"

namespace kvq {
namespace {

typedef _Float16 h8m __attribute__((ext_vector_type(8)));
typedef float f4m __attribute__((ext_vector_type(4)));
typedef _Float16 h2m __attribute__((ext_vector_type(2)));
constexpr h2m kNegOnes2 = {(_Float16)-1.0f, (_Float16)-1.0f};  // subtracts both halves in a dot product

// LDS of one wave, on top of the VALU decode's (used by the window units and the weights).
template <int D, int NR, int BV>
struct MfmaLds {
  // q~' A fragments [k-step][k-group][row (17: padding)][4 dwords of fp16 pairs]: a producer lane
  // writes row 2 i + h of its own (k-step, k-group), so (k-step, k-group) blocks 68 dwords apart
  // (4 mod 32) put 8 consecutive lanes' 16-byte writes on distinct banks
  uint32_t qb[D / 32][4][17][4];
  float beta[NR];                 // per row: q . z minus the fold constant, this record
  float pbuf[NR][32 + 4];         // softmax weights of the record per row (token order)
  uint32_t vcs[D][BV];            // the record's value codes [channel][words]
  // fp16 value weights, row r (B column) at r * kWaRow: [value group][token pairs] (20 dwords
  // each), rows padded to an odd multiple of 4 dwords so 8 consecutive columns' 16-byte reads
  // fall on distinct banks
  uint32_t wa[16 * (D / 32 * 20 + 4)];  // rows past NR stay zero
};

// Maximum over the 16 lanes of a row, in every lane.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kRowRor8>(v));
  return v;
}

// Sum over the N consecutive lanes (N = 8 or 16, aligned) holding one row's key producers.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  if constexpr (N == 8) {
    v += dpp<0x141>(v);  // row_half_mirror: lane x with 7 - x of its half-row
  } else {
    v += dpp<kRowRor4>(v);
    v += dpp<kRowRor8>(v);
  }
  return v;
}

template <int D, int BK>
struct KeyCombo {
  // producer combo c -> (row, k-step, k-group): 8 channels of quarter g (the channels of the
  // A fragment of k-step ks), for one row
  static constexpr int KS = D / 32;
  __device__ static int row(int c) { return c / (4 * KS); }
  __device__ static int ks(int c) { return (c / 4) % KS; }
  __device__ static int g(int c) { return c % 4; }
};

// Channel (within the head) of element e (0..7) of the key A fragment for k-step ks and k-group
// (= quarter) g: element e is half e % 2 of converted dword e / 2 of the fragment's words.
template <int D, int BK>
__device__ __forceinline__ int key_channel(int ks, int g, int e) {
  using MK = Magic<BK>;
  constexpr int DQ = D / 4;
  constexpr int WQ = D * BK / 128;       // words per (token, quarter)
  constexpr int FPW = MK::NH / 4;        // fragments per word (2, 1) or words per fragment (BK = 8: 2)
  int word, j;
  if constexpr (BK == 8) {               // a fragment spans two words of 2 dwords
    word = 2 * ks + (e >> 2);
    j = (e >> 1) & 1;
  } else {
    word = ks / FPW;
    j = (ks % FPW) * 4 + (e >> 1);
  }
  (void)WQ;
  const int pos = j + (e & 1) * MK::NH;  // code position within the word
  return g * DQ + word * MK::NC + pos;
}

// Element e of a key B fragment within its two 4-channel runs (run 0 then run 1): BK 2 and 4
// alternate the runs (a converted dword pairs positions j and j + NH), BK = 8 takes run 0 then 1.
template <int BK>
__host__ __device__ constexpr int key_param_slot(int e) {
  return BK == 8 ? (e >> 2) * 4 + ((e >> 1) & 1) + 2 * (e & 1) : (e & 1) * 4 + (e >> 1);
}

template <int D, int BK>
__device__ __forceinline__ float key_fold(int ks, int e) {
  using MK = Magic<BK>;
  int j;
  if constexpr (BK == 8) j = (e >> 1) & 1;
  else j = (ks % (MK::NH / 4)) * 4 + (e >> 1);
  return MK::fold(j);  // fold of code position j (or j + NH: same in-half position)
}

// Waves per workgroup: one workgroup fills a CU at two waves per SIMD.
constexpr int kMW = 8;

template <int D, int BK, int BV, int NR>
__global__ __launch_bounds__(64 * kMW) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_kernel(const uint8_t* __restrict__ buf, Layout L, DecodeShape ds, PerSeq seq, SplitPlan plan,
                        const __half* __restrict__ q, float* __restrict__ ws, uint32_t* __restrict__ sync,
                        void* __restrict__ out, const __half* __restrict__ k_app, const __half* __restrict__ v_app,
                        uint8_t* bufw) {
  constexpr int E = D / 64, DQ = D / 4, NKG = D / 32, KS = D / 32;
  constexpr int WQ = D * BK / 128;
  using MK = Magic<BK>;
  using MV = Magic<BV>;
  constexpr int NCOMBO = NR * KS * 4;               // key producer combos per record
  constexpr int kWaRow = D / 32 * 20 + 4;           // dwords per weight row in LDS
  constexpr int PL = (NCOMBO + 63) / 64;            // combos per lane
  static_assert(NR == 4 || NR == 8, "4 or 8 query rows per KV head");

  // per wave: the matrix-core arrays while records are computed, then the VALU decode's arrays for
  // the window units (which come after every record of the wave)
  union PerWave {
    MfmaLds<D, NR, BV> m;
    WaveLds<D, NR> w;
  };
  __shared__ __attribute__((aligned(16))) union {
    PerWave pw[kMW];
    float res[kMW][2][NR][D + 4];
    float mrg[3][64 * kMW];
  } sh;
  __shared__ int sh_last;
  __shared__ int sh_prog[kMW];  // records each wave has computed
  __shared__ int sh_simd[kMW];  // the SIMD each wave runs on

  // this workgroup's (sequence, KV head, split) from the plan
  const int item = blockIdx.x / L.Hkv, h = blockIdx.x % L.Hkv;
  int k = 0;  // the plan's sequence: first[k] <= item < first[k + 1]
  {
    int hi = L.B;
    while (hi - k > 1) {
      const int mid = (k + hi) >> 1;
      if (plan.first(mid) <= item) k = mid;
      else hi = mid;
    }
  }
  const int b = plan.order[k];
  const int nsp = plan.first(k + 1) - plan.first(k), sigma = item - plan.first(k);
  // wave-uniform: record indices and addresses stay in scalar registers, the loops' branches uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nq = max(0, min(seq.a[b], L.max_groups * kGroup));
  const int nr_old = max(0, min(seq.b[b], L.R));
  const int nr = min(nr_old + ds.append, L.R);
  const int ngroups = nq / kGroup;
  Causal<NR> cz;
  {
    const int S = nq + nr;
#pragma unroll
    for (int i = 0; i < NR; ++i) cz.lim[i] = S - (ds.nqry - 1 - i % ds.nqry);
    cz.lim_min = S - (ds.nqry - 1);
  }
  const int nunits = ngroups + (nr + kGroup - 1) / kGroup;
  const int chunk = (nunits + nsp - 1) / nsp;
  const int u0 = sigma * chunk;
  if (u0 >= nunits) return;
  const int u1 = min(u0 + chunk, nunits);
  const int uq = min(u1, ngroups);
  // hardware wave id register, bits 5:4: the SIMD of this wave
  const int simd = int((__builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11)) >> 4) & 3);
  if (lane == 0) {
    sh_prog[wave] = 0;
    sh_simd[wave] = simd;
  }

  WaveLds<D, NR>& W = sh.pw[wave].w;
  MfmaLds<D, NR, BV>& M = sh.pw[wave].m;
  const int P = lane >> 2, Q = lane & 3;  // the VALU decode's lane roles (weights, window)
  const int g = lane >> 4, col = lane & 15;  // MFMA roles: k-group / row group, column

  Unpacker<BK, true> upk;  // their pairs are matrix-core operands
  Unpacker<BV, true> upv;
  upk.init();
  upv.init();

  // query: VALU layout (window units) and the key producers' folded channels
  float qs[NR][E];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e)
      qs[i][e] = __half2float(q[(int64_t(b) * ds.n_q_heads + h * NR + i) * D + lane * E + e]) * ds.qscale;
  float pq[PL][8], pqf[PL][8];  // per combo: q (scaled) and q * fold of its 8 channels
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int c = min(lane + 64 * j, NCOMBO - 1);
    const int i = KeyCombo<D, BK>::row(c), ks = KeyCombo<D, BK>::ks(c), gg = KeyCombo<D, BK>::g(c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = key_channel<D, BK>(ks, gg, e);
      pq[j][e] = __half2float(q[(int64_t(b) * ds.n_q_heads + h * NR + i) * D + ch]) * ds.qscale;
      pqf[j][e] = pq[j][e] * key_fold<D, BK>(ks, e);
    }
  }
  // fold of token t's converted value code: at 2 bits the matrix-core path converts each k-group's
  // 4 + 4 codes from word positions t % 4 (the word shifted by 8 bits for the upper four), else
  // from their own word position
  auto vfold = [](int t) { return BV == 2 ? MV::fold(t % 4) : MV::fold(t % MV::NC); };
  const float vf0 = vfold(2 * P) * kVScale, vf1 = vfold(2 * P + 1) * kVScale;

  // matrix-core running state: column col's row (col / 2) softmax; value sums O^T for row col
  // matrix-core softmax state: lanes 16 g .. 16 g + 15 hold query rows 2 g and 2 g + 1 (g < NR / 2)
  const bool rowok = g < NR / 2;
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  int lim2[2];  // causal limits of those rows
#pragma unroll
  for (int j = 0; j < 2; ++j) lim2[j] = nq + nr - (ds.nqry - 1 - (2 * g + j) % ds.nqry);
  f4m o[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) o[mt] = f4m{0.f, 0.f, 0.f, 0.f};
  float bias[NR];  // weight producers: zero-term bias per row
#pragma unroll
  for (int i = 0; i < NR; ++i) bias[i] = 0.0f;
  // window / sink units: the VALU decode's running state
  WaveState<D, NR> stw;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    stw.m[i] = -INFINITY;
    stw.l[i] = 0.f;
    stw.bias[i] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) stw.acc[i][e] = 0.f;
  }
  __syncthreads();  // sh_prog, sh_simd are set
  // window units first (their loads wait while the other waves compute records), on the last
  // waves, which hold the fewest records: the VALU decode's path and state
  for (int u = max(u0, ngroups) + (kMW - 1 - wave); u < u1; u += kMW) {
    const int tbase = (u - ngroups) * kGroup;
    const int nvalid = min(kGroup, nr - tbase);
    const __half* wk = reinterpret_cast<const __half*>(buf + L.wk_off + L.window(b, h)) + tbase * D;
    const __half* wv = reinterpret_cast<const __half*>(buf + L.wv_off + L.window(b, h)) + tbase * D;
    const int tnew = ds.append ? nr_old - tbase : -1;
    const int64_t tok = (int64_t(b) * L.Hkv + h) * D;
    const __half* kn = ds.append ? k_app + tok : nullptr;
    const __half* vn = ds.append ? v_app + tok : nullptr;
    process_window<D, NR, false>(wk, wv, nvalid, tnew, kn, vn, W, stw, qs, lane, cz, nq + tbase, nullptr);
    if (tnew >= 0 && tnew < nvalid) {
      __half* dk = reinterpret_cast<__half*>(bufw + L.wk_off + L.window(b, h)) + nr_old * D;
      __half* dv = reinterpret_cast<__half*>(bufw + L.wv_off + L.window(b, h)) + nr_old * D;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dk[lane * E + e] = kn[lane * E + e];
        dv[lane * E + e] = vn[lane * E + e];
      }
    }
  }

  // A rows of q~' past 2 NR and weight columns past NR stay zero
  for (int x = lane; x < KS * 4 * 17 * 4; x += 64) (&M.qb[0][0][0][0])[x] = 0u;
  for (int x = NR * kWaRow + lane; x < 16 * kWaRow; x += 64) M.wa[x] = 0u;
  wave_sync();
  int partner = -1;  // the other wave of this workgroup on this SIMD, if any
#pragma unroll
  for (int w = 0; w < kMW; ++w)
    if (w != wave && sh_simd[w] == simd) partner = w;

  const uint8_t* rec0 = buf + L.record(b, h, 0);
  const uint64_t rb = L.rec_bytes;
  // the record's words as this lane loads them
  struct Regs {
    uint32_t kc[2 * WQ];       // tokens 2 col, 2 col + 1 of quarter g (permuted chunk)
    uint32_t kp[PL][8];        // key params of the lane's producer channels
    uint32_t vc[E * BV];       // value codes of channels lane * E ..
    uint32_t vp[E];            // value params (the VALU decode's producer entries)
  };
  // Records are read once per step: non-temporal loads (streaming cache policy), which stream
  // them in at a higher rate here than the default policy. Scheduling barriers keep a record's
  // loads in one fixed order wherever it is loaded, so that the compiler's memory-counter waits
  // at the loop head, which merge the paths into it, need not assume another order.
  auto load = [&](int u, Regs& r) {
    const uint8_t* rec = rec0 + uint64_t(u) * rb;
    load_words<2 * WQ, true>(reinterpret_cast<const uint32_t*>(rec) + (4 * col + g) * 2 * WQ, r.kc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      // the 8 channels are two runs of 4 consecutive ones: two 16-byte loads
      const int c = min(lane + 64 * j, NCOMBO - 1);
      const int ks = KeyCombo<D, BK>::ks(c), gg = KeyCombo<D, BK>::g(c);
      const uint32_t* kpg = reinterpret_cast<const uint32_t*>(rec + rec_off_kparams(D, BK, BV));
      const uint4 r0 = load_nt4(kpg + key_channel<D, BK>(ks, gg, 0));
      __builtin_amdgcn_sched_barrier(0);
      const uint4 r1 = load_nt4(kpg + key_channel<D, BK>(ks, gg, BK == 8 ? 4 : 1));
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t w8[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) r.kp[j][e] = w8[key_param_slot<BK>(e)];
    }
    load_words<E * BV, true>(reinterpret_cast<const uint32_t*>(rec + rec_off_vcodes(D, BK)) + lane * E * BV, r.vc);
    __builtin_amdgcn_sched_barrier(0);
    load_words<E, true>(reinterpret_cast<const uint32_t*>(rec + rec_off_vparams(D, BK, BV)) + lane * E, r.vp);
    __builtin_amdgcn_sched_barrier(0);
  };

  auto process = [&](const Regs& cur, int tok0) {
    // ---- key producers: B fragments (fp16 high / low columns) and beta per row
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int c = lane + 64 * j;
      float bp = 0.f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        // q~' as fp16 high + low parts; beta takes out exactly what the matrix cores will see
        // (high + low, not q~' itself), so the converted codes' constant 1 (times a fold factor up
        // to 64) cancels to fp32 accuracy and only the codes' own part carries the split error.
        // The product with a -0 addend is the plain product (one rounding); the parts leave beta
        // through dot products with (-1, -1), exact products summed in fp32, with no conversion.
        const float x0 = __builtin_fmaf(pqf[j][e], lo_f(cur.kp[j][e]), -0.0f);
        const float x1 = __builtin_fmaf(pqf[j][e + 1], lo_f(cur.kp[j][e + 1]), -0.0f);
        const auto hh = __builtin_amdgcn_cvt_pkrtz(x0, x1);
        const auto ll = __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf(pqf[j][e], lo_f(cur.kp[j][e]), -(float)hh[0]),
                                                   __builtin_fmaf(pqf[j][e + 1], lo_f(cur.kp[j][e + 1]), -(float)hh[1]));
        bp = __builtin_fmaf(pq[j][e], hi_f(cur.kp[j][e]), bp);
        bp = __builtin_fmaf(pq[j][e + 1], hi_f(cur.kp[j][e + 1]), bp);
        bp = __builtin_amdgcn_fdot2(hh, kNegOnes2, bp, false);
        bp = __builtin_amdgcn_fdot2(ll, kNegOnes2, bp, false);
        hi[e >> 1] = __builtin_bit_cast(uint32_t, hh);
        lo[e >> 1] = __builtin_bit_cast(uint32_t, ll);
      }
      bp = group_sum<4 * KS>(bp);  // the 4 KS combos of one row are consecutive lanes
      if (c < NCOMBO) {
        const int i = KeyCombo<D, BK>::row(c), ks = KeyCombo<D, BK>::ks(c), gg = KeyCombo<D, BK>::g(c);
        *reinterpret_cast<uint4*>(&M.qb[ks][gg][2 * i][0]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(&M.qb[ks][gg][2 * i + 1][0]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        if (c % (4 * KS) == 0) M.beta[i] = bp;
      }
    }
    // ---- value codes to their A layout
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int w = 0; w < BV; ++w) M.vcs[lane * E + e][w] = cur.vc[e * BV + w];
    // ---- key A fragments: the lane's two tokens x its quarter, converted
    h8m ka[2][KS];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      uint32_t cv[WQ][MK::NH];
#pragma unroll
      for (int w = 0; w < WQ; ++w) upk.run(cur.kc[tp * WQ + w], cv[w]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint32_t f[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          if constexpr (BK == 8) f[d] = cv[2 * ks + (d >> 1)][d & 1];
          else f[d] = cv[ks / (MK::NH / 4)][(ks % (MK::NH / 4)) * 4 + d];
        }
        ka[tp][ks] = __builtin_bit_cast(h8m, make_uint4(f[0], f[1], f[2], f[3]));
      }
    }
    wave_sync();
    // ---- scores on the matrix cores, S = q~' x codes^T: A = the q~' fragments (row 2 i + h: query
    // row i, high or low part), B = the converted key codes (column m: token pair m of tile tp),
    // beta entering as the accumulator's start in the high rows
    float b0 = 0.f, b1 = 0.f;
    if (rowok) {
      b0 = M.beta[2 * g];
      b1 = M.beta[2 * g + 1];
    }
    f4m acc[2] = {f4m{b0, 0.f, b1, 0.f}, f4m{b0, 0.f, b1, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const h8m aq = __builtin_bit_cast(h8m, *reinterpret_cast<const uint4*>(&M.qb[ks][g][col][0]));
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) acc[tp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, ka[tp][ks], acc[tp], 0, 0, 0);
    }
    // lane (g, m): token 2 m + tp of query rows 2 g + j (high + low parts)
    float s[2][2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int j = 0; j < 2; ++j) s[tp][j] = acc[tp][2 * j] + acc[tp][2 * j + 1];
    if (NR > 1 && tok0 + kGroup > cz.lim_min) {  // some row's future is in this record
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (tok0 + 2 * col + tp >= lim2[j]) s[tp][j] = kMaskScore;
    }
    float mx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) mx[j] = row_max16(fmaxf(s[0][j], s[1][j]));
    if (__any(rowok && (mx[0] > mrow[0] || mx[1] > mrow[1]))) {  // some row's maximum moves
      float a[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float mn = fmaxf(mrow[j], mx[j]);
        a[j] = fast_exp2(mrow[j] - mn);
        mrow[j] = mn;
        lrow[j] *= a[j];
      }
      // every row's factor, wave-uniform (row 2 g + j lives in lanes 16 g ..)
      float al[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i)
        al[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[i % 2]), 16 * (i / 2)));
      float ao = 1.0f;
#pragma unroll
      for (int i = 0; i < NR; ++i) ao = col == i ? al[i] : ao;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) o[mt] *= ao;
#pragma unroll
      for (int i = 0; i < NR; ++i) bias[i] *= al[i];
    }
    if (rowok) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float p0 = fast_exp2(s[0][j] - mrow[j]), p1 = fast_exp2(s[1][j] - mrow[j]);
        lrow[j] += p0 + p1;
        *reinterpret_cast<float2*>(&M.pbuf[2 * g + j][2 * col]) = make_float2(p0, p1);
      }
    }
    wave_sync();
    // ---- weight producers (the VALU decode's lanes): fp16 folded weights, zero-term bias
    bool bigv;
    {
      uint32_t mxs = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) mxs = max(mxs, cur.vp[e] & 0x7FFFu);
      bigv = __any(mxs > big_scale_bits<BV>());
    }
    const float vw0 = bigv ? vf0 * (1.0f / kVBigRatio) : vf0, vw1 = bigv ? vf1 * (1.0f / kVBigRatio) : vf1;
    const float amul = bigv ? kVBigRatio : 1.0f;
    float2 pw[NR];  // every row's weights first: the LDS reads need not wait for the writes below
#pragma unroll
    for (int i = 0; i < NR; ++i) pw[i] = *reinterpret_cast<const float2*>(&M.pbuf[i][2 * P]);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float2 pp = pw[i];
      float br = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int idx = lane * E + e;
        const int tp = idx & 1, k = (idx >> 1) % NKG, t = 2 * P + tp;
        const float pv = tp ? pp.y : pp.x;
        const __half a16 = __float2half_rn((pv * (tp ? vw1 : vw0)) * lo_f(cur.vp[e]));
        br = __builtin_fmaf(-__half2float(a16), amul, __builtin_fmaf(pv * kVScale, hi_f(cur.vp[e]), br));
        const int dw = (t / MV::NC) * MV::NH + (t % MV::NC) % MV::NH, hf = (t % MV::NC) / MV::NH;
        reinterpret_cast<__half*>(&M.wa[i * kWaRow + k * 20 + dw])[hf] = a16;
      }
      bias[i] += br;
    }
    wave_sync();
    // ---- values on the matrix cores: A = the codes of channel 16 mt + col, k-group g, accumulated
    // into o (one rounding per record and element, as a separate per-record sum would take); a
    // record with weights at kVScaleBig meets o scaled down by kVBigRatio, exactly (a power of 2)
    if (bigv) {
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) o[mt] *= 1.0f / kVBigRatio;
    }
#pragma unroll
    for (int k = 0; k < NKG; ++k) {
      const h8m bw = __builtin_bit_cast(h8m, *reinterpret_cast<const uint4*>(&M.wa[col * kWaRow + k * 20 + 4 * g]));
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        const int mt = 2 * k + mh;
        uint32_t f[4];
        if constexpr (BV == 8) {
#pragma unroll
          for (int w2 = 0; w2 < 2; ++w2) {
            uint32_t cv[MV::NH];
            upv.run(M.vcs[mt * 16 + col][2 * g + w2], cv);
            f[2 * w2] = cv[0];
            f[2 * w2 + 1] = cv[1];
          }
        } else if constexpr (BV == 2) {
          // k-group g: word positions 4 (g % 2) .. + 3 and 8 + the same, shifted down to 0 .. 3
          // and 8 .. 11 (a runtime pick among the converted pairs would cost selects)
          upv.template run_n<4>(M.vcs[mt * 16 + col][g >> 1] >> (8 * (g & 1)), f);
        } else {
          upv.run(M.vcs[mt * 16 + col][g], f);  // 4 bits: a word is one fragment
        }
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8m, make_uint4(f[0], f[1], f[2], f[3])),
                                                       bw, o[mt], 0, 0, 0);
      }
    }
    if (bigv) {
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) o[mt] *= kVBigRatio;
    }
    wave_sync();
  };

  // quantized records [u0, uq): wave w takes u0 + w, u0 + w + kMW, ... (a fixed assignment keeps
  // the sums in a fixed order). The two waves of a SIMD would not progress alike (the arbiter
  // serves the older one first when both are ready), so each wave compares its record count with
  // its SIMD partner's after every record and takes the higher issue priority while it is not
  // ahead: both finish together. Two of a wave's records are in flight, the older computed while
  // the newer arrives. The second register set is loaded only where the loop begins, the first
  // ahead of the loop and after its record is computed, each record's loads in one fixed order:
  // with both sets loaded ahead of the loop, the compiler copied registers of a set still in
  // flight on the back edge, behind a wait for every load. A ring of three sets (tried at 4 rows)
  // measured slower (GQA batch 42.0 against 40.6 us): the compiler's first wait of each round
  // covered two of its records.
  int u = u0 + wave;
  if (u < uq) {
    const int ulast = uq - 1;
    int done = 0;
    auto progress = [&]() {
      ++done;
      if (lane == 0) sh_prog[wave] = done;
      if (partner >= 0) {
        const int theirs = sh_prog[partner];
        if (done <= theirs) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
    };
    Regs ra, rbf;
    load(u, ra);
    while (true) {
      load(min(u + kMW, ulast), rbf);
      process(ra, u * kGroup);
      u += kMW;
      if (u >= uq) break;
      load(min(u + kMW, ulast), ra);
      progress();
      process(rbf, u * kGroup);
      u += kMW;
      if (u >= uq) break;
      progress();
    }
    __builtin_amdgcn_s_setprio(0);
  }
  // ---- finish the wave: both states to LDS as (acc[D], m, l) per row, in output units
  // matrix-core state: l per row summed over its 4 row groups, bias per (row, value group)
  float lt[2];  // l of rows 2 g + j, over the 16 lanes of the row group
#pragma unroll
  for (int j = 0; j < 2; ++j) lt[j] = row_sum16(lrow[j]);
  float ltw[NR], bsum[NR], bsumw[NR];  // window l per row; the bias of this lane's value group
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float v = (Q == 0) ? stw.l[i] : 0.f;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) v += __shfl_xor(v, msk, 64);
    ltw[i] = v;
    bsum[i] = value_group_bias<D>(bias[i], lane);
    bsumw[i] = value_group_bias<D>(stw.bias[i], lane);
  }
  __syncthreads();  // the union switches from the per-wave arrays to res
  // matrix-core O^T: lane (g, col) holds channels 16 mt + 4 g + r of row col
  if (col < NR) {
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.res[wave][0][col][mt * 16 + 4 * g + r] = o[mt][r];
  }
  if (col == 0 && rowok) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sh.res[wave][0][2 * g + j][D] = mrow[j];
      sh.res[wave][0][2 * g + j][D + 1] = lt[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    // the bias joins the matrix-core sums (its weights' zero terms); both states in output units
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int ch = lane * E + e;
      sh.res[wave][0][i][ch] = (sh.res[wave][0][i][ch] + bsum[i]) * (1.0f / kVScale);
      sh.res[wave][1][i][ch] = (stw.acc[i][e] + bsumw[i]) * (1.0f / kVScale);
    }
    if (lane == 0) {
      sh.res[wave][1][i][D] = stw.m[i];
      sh.res[wave][1][i][D + 1] = ltw[i];
    }
  }
  __syncthreads();

  // ---- combine the 2 x kMW states per row: the partial of each row, or the output
  const int nvs = (nunits + chunk - 1) / chunk;  // splits of (b, h_kv) that hold units
  const int64_t row0 = int64_t(b) * ds.n_q_heads + h * NR;
  for (int idx = threadIdx.x; idx < NR * D; idx += 64 * kMW) {
    const int i = idx / D, ch = idx % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMW; ++w)
#pragma unroll
      for (int z = 0; z < 2; ++z) Mx = fmaxf(Mx, sh.res[w][z][i][D]);
    float O = 0.f, Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kMW; ++w)
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float mw = sh.res[w][z][i][D];
        if (mw != -INFINITY) {
          const float wgt = fast_exp2(mw - Mx);
          O += wgt * sh.res[w][z][i][ch];
          Lsum += wgt * sh.res[w][z][i][D + 1];
        }
      }
    if (nvs == 1) {
      store_out(out, ds.out_fp32, (row0 + i) * D + ch, O / Lsum);
      continue;
    }
    float* dst = ws + ((row0 + i) * ds.n_split + sigma) * (D + 4);
    put_partial(dst + ch, O);
    if (ch == 0) {
      put_partial(dst + D, Mx);
      put_partial(dst + D + 1, Lsum);
    }
  }
  int32_t* len_w = reinterpret_cast<int32_t*>(bufw + L.lengths(b, h));
  if (nvs == 1) {
    if (ds.append && threadIdx.x == 0) len_w[1] = nr;
    return;
  }
  // the last split of (b, h_kv) merges, as in the VALU decode (see decode_split_kernel)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* cnt = sync + (int64_t(b) * L.Hkv + h);
  if (threadIdx.x == 0) sh_last = atomicAdd(cnt, 1u) + 1u == uint32_t(nvs);
  __syncthreads();
  if (!sh_last) return;
  merge_splits<D, NR, 64 * kMW>(ws, row0, ds.n_split, nvs, sh.mrg, out, ds.out_fp32);
  if (threadIdx.x == 0) {
    if (ds.append) len_w[1] = nr;
    atomicExch(cnt, 0u);
  }
}

template <int D, int BK, int BV, int NR>
hipError_t launch_t(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const SplitPlan& plan,
                    const void* q, float* ws, void* out, const void* ka, const void* va, hipStream_t s, hipEvent_t e0,
                    hipEvent_t e1) {
  const dim3 grid(unsigned(plan.first(L.B)) * unsigned(L.Hkv));
  uint32_t* sync = reinterpret_cast<uint32_t*>(buf + L.sync_off);
  const __half* qh = static_cast<const __half*>(q);
  const __half* kh = static_cast<const __half*>(ka);
  const __half* vh = static_cast<const __half*>(va);
  if (e0 || e1)
    hipExtLaunchKernelGGL((decode_mfma_kernel<D, BK, BV, NR>), grid, dim3(64 * kMW), 0, s, e0, e1, 0,
                          static_cast<const uint8_t*>(buf), L, ds, seq, plan, qh, ws, sync, out, kh, vh, buf);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, BK, BV, NR>), grid, dim3(64 * kMW), 0, s,
                       static_cast<const uint8_t*>(buf), L, ds, seq, plan, qh, ws, sync, out, kh, vh, buf);
  return hipGetLastError();
}

template <int D, int BK, int BV>
hipError_t launch_r(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const SplitPlan& plan,
                    const void* q, float* ws, void* out, const void* ka, const void* va, hipStream_t s, hipEvent_t e0,
                    hipEvent_t e1) {
  if (ds.G == 4) return launch_t<D, BK, BV, 4>(buf, L, ds, seq, plan, q, ws, out, ka, va, s, e0, e1);
  if (ds.G == 8) return launch_t<D, BK, BV, 8>(buf, L, ds, seq, plan, q, ws, out, ka, va, s, e0, e1);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const SplitPlan& plan,
                    const void* q, float* ws, void* out, const void* ka, const void* va, hipStream_t s, hipEvent_t e0,
                    hipEvent_t e1) {
#define KVQ_MFMA_CASE(BK, BV) \
  case BK * 16 + BV: return launch_r<D, BK, BV>(buf, L, ds, seq, plan, q, ws, out, ka, va, s, e0, e1);
  switch (L.bk * 16 + L.bv) {
    KVQ_MFMA_CASE(2, 2) KVQ_MFMA_CASE(2, 4) KVQ_MFMA_CASE(2, 8)
    KVQ_MFMA_CASE(4, 2) KVQ_MFMA_CASE(4, 4) KVQ_MFMA_CASE(4, 8)
    KVQ_MFMA_CASE(8, 2) KVQ_MFMA_CASE(8, 4) KVQ_MFMA_CASE(8, 8)
    default: return hipErrorInvalidValue;
  }
#undef KVQ_MFMA_CASE
}

}  // namespace

hipError_t launch_decode_mfma(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq,
                              const SplitPlan& plan, const void* q, float* ws, void* out, const void* ka,
                              const void* va, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (L.method != kMethodKivi || L.NS != 0) return hipErrorInvalidValue;
  if (plan.first(0) != 0 || plan.first(L.B) == 0) return hipErrorInvalidValue;
  if (L.D == 128) return launch_d<128>(buf, L, ds, seq, plan, q, ws, out, ka, va, s, e0, e1);
  if (L.D == 64) return launch_d<64>(buf, L, ds, seq, plan, q, ws, out, ka, va, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace kvq
