// kernels.h - launchers of the HIP kernels, called by the C ABI in kvq.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace kvq {

// Three per-sequence int32 arrays passed by value as a kernel argument (3 KiB).
struct PerSeq {
  int32_t a[kMaxBatch];
  int32_t b[kMaxBatch];
  int32_t c[kMaxBatch];
};

// Split plan of the matrix-core decode: the k-th sequence of the plan, b = order[k], is cut into
// first[k + 1] - first[k] splits of ceil(units / splits) units each; workgroup x of the
// one-dimensional grid takes split x / H_kv - first[k] of that sequence (the k with
// first[k] <= x / H_kv < first[k + 1]) and KV head x % H_kv.
struct SplitPlan {
  uint8_t order[kMaxBatch];            // sequences, the largest splits first
  uint32_t first2[kMaxBatch / 2 + 1];  // first[i] in the 16-bit half i % 2 of word i / 2
  KVQ_HD int first(int i) const { return int((first2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu); }
  KVQ_HD void set(int i, int v) {
    first2[i >> 1] = (first2[i >> 1] & ~(0xFFFFu << (16 * (i & 1)))) | (uint32_t(v) << (16 * (i & 1)));
  }
};

// Decode launch geometry: gridDim.x = n_split workgroups per (b, h_kv), each covering
// `chunk` consecutive units (a unit is one 32-token record, or up to 32 window tokens).
struct DecodeShape {
  int n_split;
  int chunk;
  // Skewed splits: with n_hi > 0 the first n_hi splits of every (sequence, KV head) take
  // chunk_hi units each and the others chunk, and the workgroups run split-major (the linear
  // workgroup id counts the (KV head, sequence) pairs first), so that the splits dispatched
  // first, which share their CUs with later ones and win the SIMD arbiter over them, are the
  // longer ones. n_hi = 0: every split takes chunk units, split-minor order.
  int n_hi;
  int chunk_hi;
  int G;            // query heads per KV head
  int n_q_heads;
  float qscale;     // sm_scale * log2(e): scores are kept in base-2 units
  int out_fp32;
  int append;       // 1: the launch also appends one token per (b, h) (no window is full)
  int nqry;         // queries per head: the newest nqry tokens, causal among themselves (G
                    // and n_q_heads count query rows: heads x nqry)
};

// Multi-query attend on the matrix cores (attend_tiles.hip): grid (n_split, row_blocks, B * H_kv),
// 256 query rows (query heads x queries of one KV head) per workgroup, `chunk` units per split.
struct TileShape {
  int n_split;
  int chunk;
  int G;           // query heads per KV head
  int n_q_heads;   // H_q
  int nqry;        // queries per head (the newest nqry tokens of each sequence)
  int row_blocks;  // 256-row blocks per KV head
  float qscale;    // sm_scale * log2(e)
  int out_fp32;
};

hipError_t launch_encode(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                         const PerSeq& seq, int max_records, hipStream_t s);
// seq: every sequence's lengths before the append (a = quantized, b = window tokens).
hipError_t launch_append(uint8_t* buf, const Layout& L, const void* k, const void* v, const PerSeq& seq, hipStream_t s);
hipError_t launch_window_fill(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                              const PerSeq& seq, hipStream_t s);
hipError_t launch_encode_block(const void* X, int n_tok, int D, int bits, int group, int per_channel, void* codes,
                               void* scales, void* zeros, hipStream_t s);
// clear_sinks: also mark every sink slot empty (a reset, or the first use of a buffer).
hipError_t launch_lengths_fill(uint8_t* buf, const Layout& L, const PerSeq& seq, hipStream_t s, int clear_sinks);
// SKVQ permutations of the sequences with seq.b[b] > 0, from the R tokens of K[b][h] and V[b][h]
// that start at token seq.c[b] (the first chunk).
hipError_t launch_skvq_perm(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                            const PerSeq& seq, hipStream_t s);
// SKVQ records seq.a[b] + x (x < seq.b[b]) of every (b, h) from tokens seq.c[b] + 32 x on;
// rows_permuted: the rows are stored in permuted channel order (a window flush).
hipError_t launch_skvq_encode(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                              const PerSeq& seq, int max_records, int rows_permuted, hipStream_t s);
// SKVQ first flush of the sequences with seq.b[b] > 0: their window and sink rows rewritten in
// permuted order.
hipError_t launch_skvq_permute_rows(uint8_t* buf, const Layout& L, const PerSeq& seq, hipStream_t s);
// Sinks of the sequences with seq.b[b] > 0: chosen among tokens 0 .. seq.b[b]-1 of K[b][h]
// (the sequence's first quantized tokens), positions and fp16 K, V rows written (L.NS >= 1).
hipError_t launch_sink_select(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                              const PerSeq& seq, hipStream_t s);

// Decode attention: split-K kernel whose last split per (b, h_kv) merges the partials into
// `out`. start/stop, when not null, are stamped by the kernel's own dispatch (its execution
// time).
// seq: the host's lengths of every sequence (a = quantized tokens, b = window tokens before the
// launch's append, c = sinks present); the launch is planned from them, not from the device copy.
// With ds.append, k_tok / v_tok (fp16 [B][H_kv][D]) are the appended tokens: the launch attends
// over the window plus them, stores them in their window slots and advances the device lengths.
hipError_t launch_decode(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const void* q, float* ws,
                         void* out, const void* k_tok, const void* v_tok, hipStream_t s,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// The same for SKVQ caches and for KIVI caches with sink tokens (L.NS > 0); launch_decode
// forwards to them.
hipError_t launch_decode_skvq(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const void* q, float* ws,
                              void* out, const void* k_tok, const void* v_tok, hipStream_t s, hipEvent_t start,
                              hipEvent_t stop);
// The decode for 4 or 8 query rows per KV head of KIVI caches without sinks, both per-record
// products on the matrix cores (decode_mfma.hip); the same arguments and results.
hipError_t launch_decode_mfma(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq,
                              const SplitPlan& plan, const void* q,
                              float* ws, void* out, const void* k_tok, const void* v_tok, hipStream_t s,
                              hipEvent_t start, hipEvent_t stop);
hipError_t launch_decode_sink(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const void* q, float* ws,
                              void* out, const void* k_tok, const void* v_tok, hipStream_t s, hipEvent_t start,
                              hipEvent_t stop);

// Multi-query attend over a KIVI cache without sinks: split kernel, then (n_split > 1) a merge
// kernel; seq: the host's lengths (a = quantized tokens, b = window tokens). start/stop bracket
// both launches.
hipError_t launch_attend_tiles(const uint8_t* buf, const Layout& L, const TileShape& ts, const PerSeq& seq,
                               const void* q, float* ws, void* out, hipStream_t s, hipEvent_t start, hipEvent_t stop);

// Kitty records seq.a[b] + x (x < seq.b[b]) of every (b, h) from tokens seq.c[b] + 32 x on of
// K[b][h], V[b][h] (row stride D, ld_tok rows per (b, h)): group sums, running sums (those of
// record 0 start from zero, later ones from the sequence's stored sums, which end updated), then
// ranking and encoding.
hipError_t launch_kitty_encode(uint8_t* buf, const Layout& L, const void* K, const void* V, int64_t ld_tok,
                               const PerSeq& seq, int max_records, hipStream_t s);
// Kitty decode: split kernel whose last split per (b, h_kv) merges the partials (ws) into out.
// start/stop as above.
hipError_t launch_kitty_decode(uint8_t* buf, const Layout& L, const DecodeShape& ds, const void* q, float* ws,
                               void* out, hipStream_t s, hipEvent_t start, hipEvent_t stop);

}  // namespace kvq
