// layout.h - byte layout of the quantized cache in HBM (host and device).
//
// One cache buffer per layer:
//   lengths  int32 [B][H_kv][2]                 (quantized tokens, window tokens)
//   sync     uint32 [B][H_kv]                   decode split counters (zero between calls)
//   records  [B][H_kv][max_tokens/32][record]   one record per group of 32 quantized tokens
//   window_k fp16  [B][H_kv][R][D]              the newest tokens, unquantized
//   window_v fp16  [B][H_kv][R][D]
//   sink_pos int32 [B][H_kv][NS]                sink token positions, ascending (NS = n_sink)
//   sink_k   fp16  [B][H_kv][NS][D]             the sinks' key and value rows, unquantized
//   sink_v   fp16  [B][H_kv][NS][D]
//   perm     uint8 [B][H_kv][2][D]              SKVQ only: channel permutations of K and V
//   kstats   [B][H_kv] x (int64 s1[D], uint64 s2lo[D], uint64 s2hi[D])
//                                               Kitty only: exact running key sums per channel
// Every region but sync starts on a 256-byte boundary (sync follows lengths directly). With
// NS = 0 the three sink regions are empty and the buffer is the plain KIVI cache. A sink
// position of -1 marks an empty slot: the sinks present are the leading non-negative entries.
//
// SKVQ-adapted caches ("Changelog" v0.30.0) use the same records with per-token key groups:
// the key codes hold the permuted channels (channel c' of a quarter is permuted channel
// Q*D/4 + c'), and the key params use the value-param layout [t/2][k][t%2], group k being
// the permuted channels 32k .. 32k+31 of token t. Value codes and params hold permuted
// channels too. Their sinks are the first NS tokens of the sequence. Once a sequence has
// quantized tokens (and so its permutations), its window and sink rows are stored permuted as
// well: slot c of a key row holds channel perm_k[c], of a value row channel perm_v[c].
//
// Kitty caches ("Changelog" v0.11.0) use records of their own (kitty_* below): per token the
// key codes of the slots, slot s holding channel table[s]: slots 0 .. nhi-1 are the high-width
// channels in ascending order at HB = 4 bits, the rest the low-width ones at LB = 2 bits; in
// chunks of 16 slots, a high chunk taking two u32 words and a low chunk one, chunk k at word
// k + min(k, nhi/16) of the token, slot 16k+i at bit i*bits of its chunk (little-endian across a
// high chunk's two words); then the key params [slot] (scale | zero << 16), the slot table
// (uint8 [D]) and the fp16 value rows [32][D] (values are not quantized). Before a record is
// encoded its value area stages the key sums of its group (s1[D] int64, s2 lo[D], s2 hi[D]
// uint64), and then the running sums up to the group's end.
//
// A record holds everything decode needs for 32 tokens, so one group streams from one
// contiguous 4*D*(bk+bv+2)-byte block (3 KiB at D=128, 2/2 bits):
//   key codes    4*D*bk bytes  u32 words [P=t/2 : 16][Q : 4][tp=t%2 : 2][D*bk/128 words]
//                the words of (P, Q, tp) carry the codes of token t = 2P+tp for channels
//                Q*D/4 .. Q*D/4 + D/4 - 1, channel c' (within the quarter) at bit c'*bk
//                (little-endian across the words). A decode lane (P, Q) reads its two
//                tokens' quarter as one contiguous 8*D*bk/64-byte piece, and the 64 lanes
//                of a wave read the whole block contiguously.
//   value codes  4*D*bv bytes  u32 words [d : D][bv words]: the 32 tokens of channel d,
//                token t at bit t*bv. A lane owning channels d..d+D/64-1 reads one
//                contiguous piece.
//   key params   D dwords      [d]: (scale fp16 in bits 0-15, zero fp16 in bits 16-31)
//                of the key group (32 tokens) of channel d.
//   value params D dwords      [t/2][k : D/32][t%2]: (scale, zero) of value group k
//                (channels 32k..32k+31) of token t. The scale of a sink token carries the
//                sign bit: decode skips that slot (the sink's fp16 rows stand in for it).
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define KVQ_HD __host__ __device__
#else
#define KVQ_HD
#endif

namespace kvq {

constexpr int kGroup = 32;     // tokens per key group == channels per value group
constexpr int kMaxBatch = 256;
constexpr int kMaxSinks = 16;  // sink tokens per (sequence, KV head)
constexpr int kMethodKivi = 0, kMethodSkvq = 1, kMethodKitty = 2;

KVQ_HD constexpr uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

KVQ_HD constexpr uint64_t key_code_bytes(int D, int bk) { return 4ull * D * bk; }
KVQ_HD constexpr uint64_t value_code_bytes(int D, int bv) { return 4ull * D * bv; }
KVQ_HD constexpr uint64_t param_bytes(int D) { return 4ull * D; }
KVQ_HD constexpr uint64_t record_bytes(int D, int bk, int bv) { return 4ull * D * (bk + bv + 2); }
KVQ_HD constexpr uint64_t rec_off_vcodes(int D, int bk) { return key_code_bytes(D, bk); }
KVQ_HD constexpr uint64_t rec_off_kparams(int D, int bk, int bv) {
  return key_code_bytes(D, bk) + value_code_bytes(D, bv);
}
KVQ_HD constexpr uint64_t rec_off_vparams(int D, int bk, int bv) {
  return rec_off_kparams(D, bk, bv) + param_bytes(D);
}

// Kitty records (HB = 4, LB = 2): u32 code words per token, and the offsets inside a record.
KVQ_HD constexpr int kitty_words(int D, int nhi) { return D / 16 + nhi / 16; }
KVQ_HD constexpr uint64_t kitty_off_params(int D, int nhi) { return 128ull * kitty_words(D, nhi); }
KVQ_HD constexpr uint64_t kitty_off_table(int D, int nhi) { return kitty_off_params(D, nhi) + 4ull * D; }
KVQ_HD constexpr uint64_t kitty_off_values(int D, int nhi) { return (kitty_off_table(D, nhi) + D + 15) & ~15ull; }
KVQ_HD constexpr uint64_t kitty_record_bytes(int D, int nhi) {
  return (kitty_off_values(D, nhi) + 64ull * D + 127) & ~127ull;
}

// Offsets of the regions of one cache buffer.
struct Layout {
  int B, Hkv, D, bk, bv, R, max_groups, NS, method, reorder;
  float clip;  // SKVQ: the fixed clip fraction (1 - alpha) / 2, or < 0 for the search
  int nhi;     // Kitty: high-width key channels (a multiple of 16)
  uint64_t len_off, sync_off, rec_off, rec_bytes, wk_off, wv_off, sp_off, sk_off, sv_off, pm_off, ks_off, total;

  KVQ_HD void init(int B_, int Hkv_, int D_, int bk_, int bv_, int R_, int max_tokens, int NS_, int method_ = 0,
                   float clip_ = -1.0f, int reorder_ = 1, int nhi_ = 0) {
    B = B_; Hkv = Hkv_; D = D_; bk = bk_; bv = bv_; R = R_; NS = NS_; method = method_; clip = clip_;
    reorder = reorder_;
    nhi = nhi_;
    max_groups = max_tokens / kGroup;
    rec_bytes = method == kMethodKitty ? kitty_record_bytes(D, nhi) : record_bytes(D, bk, bv);
    len_off = 0;
    sync_off = uint64_t(B) * Hkv * 2 * sizeof(int32_t);
    rec_off = align256(sync_off + uint64_t(B) * Hkv * sizeof(uint32_t));
    wk_off = align256(rec_off + uint64_t(B) * Hkv * max_groups * rec_bytes);
    uint64_t wbytes = uint64_t(B) * Hkv * R * D * 2;
    wv_off = align256(wk_off + wbytes);
    sp_off = align256(wv_off + wbytes);
    sk_off = align256(sp_off + uint64_t(B) * Hkv * NS * sizeof(int32_t));
    const uint64_t sbytes = uint64_t(B) * Hkv * NS * D * 2;
    sv_off = align256(sk_off + sbytes);
    pm_off = align256(sv_off + sbytes);
    ks_off = align256(pm_off + (method == kMethodSkvq ? uint64_t(B) * Hkv * 2 * D : 0));
    total = align256(ks_off + (method == kMethodKitty ? uint64_t(B) * Hkv * 24 * D : 0));
  }
  // record j of (b, h)
  KVQ_HD uint64_t record(int b, int h, int j) const {
    return rec_off + ((uint64_t(b) * Hkv + h) * max_groups + j) * rec_bytes;
  }
  // first window slot of (b, h), in bytes from the buffer start (K; V at wv_off)
  KVQ_HD uint64_t window(int b, int h) const { return (uint64_t(b) * Hkv + h) * R * D * 2; }
  KVQ_HD uint64_t lengths(int b, int h) const { return len_off + (uint64_t(b) * Hkv + h) * 8; }
  KVQ_HD uint64_t sync(int b, int h) const { return sync_off + (uint64_t(b) * Hkv + h) * 4; }
  // sinks of (b, h): positions (int32), key rows and value rows (fp16 [NS][D])
  KVQ_HD uint64_t sink_pos(int b, int h) const { return sp_off + (uint64_t(b) * Hkv + h) * NS * 4; }
  KVQ_HD uint64_t sink_k(int b, int h) const { return sk_off + (uint64_t(b) * Hkv + h) * NS * D * 2; }
  KVQ_HD uint64_t sink_v(int b, int h) const { return sv_off + (uint64_t(b) * Hkv + h) * NS * D * 2; }
  // SKVQ: permutation of K (D bytes) then of V: permuted channel j is channel perm[j]
  KVQ_HD uint64_t perm(int b, int h) const { return pm_off + (uint64_t(b) * Hkv + h) * 2 * D; }
  // Kitty: running key sums of (b, h): s1 int64 [D], s2 low words uint64 [D], s2 high words [D]
  KVQ_HD uint64_t kstats(int b, int h) const { return ks_off + (uint64_t(b) * Hkv + h) * 24 * D; }
};

}  // namespace kvq
