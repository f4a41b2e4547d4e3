/*
 * kvq.h - C ABI of libkvq: a KIVI-style quantized KV cache with decode attention that
 * reads the quantized cache directly, for AMD Instinct MI355X (gfx950).
 *
 * The method (VeloxQuant-MLX documentation pages):
 *  - "Changelog", v0.8.0 "New" (KIVI): asymmetric group quantization, keys grouped per
 *    channel and values per token, no codebook, no rotation, an fp16 residual window of
 *    the newest tokens; group size 32 by default ("veloxquant_mlx.cache package",
 *    KVCacheConfig.kivi_group_size).
 *  - "Changelog", v0.42.0 "Added": decode attention straight over b-bit codes plus a
 *    per-group (scale, zero); k_hat / v_hat are rebuilt in registers inside an online
 *    softmax accumulated in fp32, so no dequantized K/V is ever written to memory.
 *  - "Changelog", v0.30.0 "New" / "Honest scope": parameters kept as low end and step,
 *    integer bit widths, fp16 metadata.  "Changelog", v0.28.0: the residual window is
 *    flushed through the quantizer one whole chunk at a time.
 *  - "Changelog", v0.9.0 "New" (KIVI-Sink): tokens with an outstanding key L2 norm stay in
 *    fp16 and are left out of the statistics their groups' parameters come from;
 *    n_sink_tokens = 0 is plain KIVI (kvq_config.n_sink).
 *
 * Conventions shared by every call:
 *  - Tensor arguments are DEVICE pointers owned by the caller. The library never allocates
 *    or frees device memory; the cache state lives in one caller-allocated device buffer
 *    of kvq_cache_bytes() bytes and decode scratch in a caller buffer of
 *    kvq_workspace_bytes() bytes.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call
 *    that takes a stream is asynchronous and ordered on that stream; the caller keeps
 *    the buffers alive until the work is done.
 *  - Every call validates its arguments on the host before anything is launched and
 *    returns a kvq_status; on failure nothing was enqueued and kvq_last_error() returns a
 *    thread-local message. No C++ exception crosses the ABI.
 *  - fp16 tensors are IEEE binary16. Layouts are row-major with the last index fastest.
 *  - A kvq_cache handle is not thread safe; calls on one handle must come from one thread
 *    (they may use any stream, but calls on different streams are not ordered).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;
#define KVQ_OK 0
#define KVQ_E_INVALID (-1)     /* bad argument, shape or state */
#define KVQ_E_UNSUPPORTED (-2) /* valid in principle, not built (e.g. group != 32) */
#define KVQ_E_CAPACITY (-3)    /* a sequence would exceed max_tokens */
#define KVQ_E_WORKSPACE (-4)   /* workspace too small */
#define KVQ_E_NODEVICE (-5)    /* no gfx950 device visible */
#define KVQ_E_HIP (-6)         /* a HIP runtime call failed */

#define KVQ_MAX_BATCH 256

/* Shape and precision of one layer's cache. */
typedef struct kvq_config {
  int32_t batch;      /* B sequences, 1..KVQ_MAX_BATCH */
  int32_t n_kv_heads; /* H_kv >= 1 */
  int32_t n_q_heads;  /* H_q = G * H_kv with G in {1, 2, 4, 8}; query head h reads KV head h / G */
  int32_t head_dim;   /* D in {64, 128} */
  int32_t key_bits;   /* b_k in {2, 4, 8} */
  int32_t value_bits; /* b_v in {2, 4, 8} */
  int32_t group;      /* g, must be 32 (the pages' default group size) */
  int32_t residual;   /* R, fp16 window capacity: a multiple of 32, at most 256 */
  int32_t max_tokens; /* per-sequence capacity in tokens, a positive multiple of 32 */
  int32_t n_sink;     /* sink tokens per (sequence, KV head), 0..16 (KIVI-Sink); 0 = plain KIVI,
                         and then the buffer is byte for byte the KIVI cache. The sinks are the
                         n_sink tokens of largest key norm (squares added in fp32, channel 0
                         first; the earlier token on equal norms) among the tokens quantized by
                         the first call that quantizes any token of the sequence (a prefill or
                         encode, or the first window flush); they never change afterwards. Their
                         fp16 key and value rows are kept, they take no part in their key
                         groups' min/max, and attention uses their fp16 rows in place of their
                         quantized slots. With method = KVQ_METHOD_SKVQ: the first n_sink tokens
                         of each sequence, kept in fp16 (the SKVQ sink filter). */
  int32_t method;           /* KVQ_METHOD_KIVI (0) or KVQ_METHOD_SKVQ (1) */
  int32_t skvq_reorder;     /* SKVQ: 1 = permute channels by range over the first chunk, 0 = identity */
  int32_t skvq_clip_search; /* SKVQ: 1 = per-group search over alpha = 1 - k/20 (k = 0..10),
                               0 = the fixed skvq_clip_alpha */
  float skvq_clip_alpha;    /* SKVQ with the search off: alpha in (0, 1] (1 = no clipping) */
  int32_t kitty_n_hi;       /* KITTY: key channels at the high width, a multiple of 16 in [0, head_dim]
                               (32 of 128 at the pages' quarter) */
  int32_t kitty_hi_bits;    /* KITTY: the high key width, 4 (key_bits is the low width, 2) */
} kvq_config;

/* Methods ("Changelog" v0.8.0 KIVI, v0.9.0 KIVI-Sink through n_sink; v0.30.0 SKVQ-adapted):
 * SKVQ quantizes keys and values in per-token groups of 32 channels taken in the order of a
 * per-(sequence, KV head) permutation (ascending channel range over the first flushed chunk
 * of R tokens, fp32 max - min, stable), each group's [min, max] window shrunk around its
 * centre to [lo + d, hi - d], d = (hi - lo)(1 - alpha)/2, with alpha picked per group by the
 * smallest fp32 sum of squared reconstruction errors (alpha = 1 on ties, fp32 operations in
 * group order), and the chosen window stored as its fp16 (scale, zero). The window rule
 * applies to the tokens after the n_sink sinks; a prefill equals the same tokens appended one
 * by one. */
#define KVQ_METHOD_KIVI 0
#define KVQ_METHOD_SKVQ 1
/* Kitty ("Changelog" v0.11.0; "Algorithm Overview", Kitty: values in fp16): every key group
 * (32 tokens of a channel) is quantized by KIVI's min/max rule at kitty_hi_bits when its channel
 * is among the kitty_n_hi channels of largest variance over all key tokens of the sequence up to
 * the end of that group (the exact population variance of the fp16 values, computed from integer
 * running sums; the lower channel index first on equal variances), else at key_bits. Values are
 * stored as their fp16 inputs (value_bits = 16). The window rule is KIVI's; a flush ranks each of
 * its groups with the sums at its own end, so a prefill equals the same tokens appended one by
 * one. n_sink must be 0; max_tokens is at most 2^22, which keeps the integer sums exact for every
 * finite fp16 key. */
#define KVQ_METHOD_KITTY 2

/* Byte offsets of the regions inside the cache buffer (see the layout description in the
 * design notes; all offsets but sync_offset are multiples of 256). */
typedef struct kvq_layout_info {
  uint64_t lengths_offset;  /* int32 [B][H_kv][2]: (quantized tokens, window tokens) */
  uint64_t records_offset;  /* [B][H_kv][max_tokens/32] group records */
  uint64_t record_bytes;    /* 4*D*(b_k + b_v + 2) */
  uint64_t rec_key_codes;   /* offset of the key codes inside a record (4*D*b_k bytes) */
  uint64_t rec_value_codes; /* value codes (4*D*b_v bytes) */
  uint64_t rec_key_params;  /* key (scale, zero) fp16 pairs, D dwords */
  uint64_t rec_value_params;/* value (scale, zero) fp16 pairs, D dwords */
  uint64_t window_k_offset; /* fp16 [B][H_kv][R][D] */
  uint64_t window_v_offset; /* fp16 [B][H_kv][R][D] */
  uint64_t total_bytes;     /* == kvq_cache_bytes() */
  uint64_t sync_offset;     /* uint32 [B][H_kv] decode split counters, right after the lengths;
                               zero between calls (decode's last split of a sequence clears its
                               counter; every lengths update zeroes them) */
  uint64_t sink_pos_offset; /* int32 [B][H_kv][n_sink]: sink token positions, ascending */
  uint64_t sink_k_offset;   /* fp16 [B][H_kv][n_sink][D]: sink key rows */
  uint64_t sink_v_offset;   /* fp16 [B][H_kv][n_sink][D]: sink value rows. The sinks present are
                               the leading non-negative positions (-1 = empty slot); in KIVI
                               records a sink's value scales carry the sign bit (decode skips
                               that slot). */
  uint64_t perm_offset;     /* SKVQ: uint8 [B][H_kv][2][D], the K and V channel permutations
                               (permuted channel j is channel perm[j]); == total_bytes for KIVI */
  uint64_t rec_slot_table;  /* KITTY records: uint8 [D], the channel of each key slot (slots
                               0 .. n_hi-1 the high-width channels, ascending, then the others);
                               rec_key_codes: per token (D + n_hi)/16 u32 words, 16-slot chunks,
                               chunk k at word k + min(k, n_hi/16), a high chunk two words of
                               4-bit codes, a low one a word of 2-bit codes; rec_key_params:
                               (scale, zero) per slot; rec_value_codes: fp16 values [32][D];
                               rec_value_params: unused (0). 0 for other methods */
  uint64_t kstats_offset;   /* KITTY: per (b, h_kv) the running key sums over the quantized
                               tokens, int64 s1[D] then uint64 s2_lo[D], s2_hi[D] (X = x * 2^24);
                               == total_bytes for other methods */
} kvq_layout_info;

typedef struct kvq_cache kvq_cache; /* opaque host handle */

/* Capability probe, the counterpart of the capability probe and the auto/require backend
 * flag of "Changelog" v0.5.1 "New": *has_gfx950 = 1 when a gfx950 device is visible to the
 * HIP runtime, else 0. Returns KVQ_OK, or KVQ_E_INVALID for a NULL pointer; never fails
 * for lack of a device. There is no CPU fallback behind it: every other call needs the GPU. */
kvq_status kvq_probe(int32_t* has_gfx950);

/* Validate a configuration (the pages' QuantizerConfigError checks). */
kvq_status kvq_config_check(const kvq_config* cfg);

/* Kitty's channel count from its fraction ("veloxquant_mlx.cache package", KVCacheConfig: the
 * share of key channels kept at the high width, a quarter by default): *n_hi = round(hi_fraction
 * * head_dim), halves rounded up, the value to put in kvq_config.kitty_n_hi. Returns KVQ_OK, or
 * KVQ_E_INVALID (and *n_hi untouched) for a NULL pointer, head_dim < 1, or a fraction that is not
 * a finite number in [0, 1]. A count that is not a multiple of 16 is accepted here and refused
 * by kvq_config_check. */
kvq_status kvq_kitty_n_hi(int32_t head_dim, double hi_fraction, int32_t* n_hi);

/* Device bytes the caller allocates for one cache (0 if cfg is invalid). The counterpart of the
 * standalone caches' memory_bytes() ("veloxquant_mlx.cache package", e.g.
 * PolarQuantKVCache.memory_bytes: bytes held for the cached tokens), taken here at full
 * capacity (max_tokens per sequence) plus the lengths, window and sink regions. */
size_t kvq_cache_bytes(const kvq_config* cfg);

/* Region offsets of the cache buffer. */
kvq_status kvq_layout(const kvq_config* cfg, kvq_layout_info* out);

/* Device bytes of decode scratch for up to n_split splits per sequence (n_split = 0: the
 * largest split count kvq_decode_attend picks by itself). 0 if cfg is invalid. */
size_t kvq_workspace_bytes(const kvq_config* cfg, int32_t n_split);

/* Create a host handle over a caller-owned device buffer of at least kvq_cache_bytes(cfg)
 * bytes (256-byte aligned). Host-only: nothing is launched here; the first call that takes
 * a stream zeroes the lengths on the device before its own work. The buffer's contents are
 * otherwise left as they are. */
kvq_status kvq_cache_create(const kvq_config* cfg, void* dev_buf, size_t bytes, kvq_cache** out);

/* Free the host handle only (never the device buffer). NULL is ignored. */
void kvq_cache_destroy(kvq_cache* cache);

/* Empty every sequence (device lengths zeroed with a fill kernel on `stream`). */
kvq_status kvq_reset(kvq_cache* cache, void* stream);

/* Host mirror of the lengths: n_quantized[b], n_window[b] (arrays of `batch` entries,
 * either may be NULL). Exact without a device sync: every length change is decided on the
 * host before it is enqueued. */
kvq_status kvq_cache_lengths(const kvq_cache* cache, int32_t* n_quantized, int32_t* n_window);

/* North-star call 1 ("Changelog" v0.8.0 quantizer; v0.42.0 codes + (scale, zero)).
 * Quantize n_tok[b] new tokens of every sequence b after its quantized region:
 *   K, V: fp16 [B][H_kv][ld_tok][D]; tokens 0..n_tok[b]-1 of sequence b are encoded.
 *   n_tok: HOST array of B entries, each a multiple of 32 (KVQ_E_INVALID otherwise); 0 skips
 *   the sequence. A sequence with a non-empty window is KVQ_E_INVALID (its window tokens
 *   are older than the new ones). Over capacity is KVQ_E_CAPACITY.
 * Key groups: 32 consecutive tokens of one channel; value groups: 32 consecutive channels
 * of one token. Per group: zero = min, scale = fp16((max - min) / (2^b - 1)) (fp32 ops),
 * codes = clamp(rint((x - zero) * (1/scale)), 0, 2^b - 1) with the stored scale, all
 * codes 0 when the stored scale is 0. Results are bit-identical on every run.
 * With n_sink > 0, a sequence that had no quantized token first chooses its sinks among
 * the n_tok[b] tokens (see kvq_config.n_sink); they stay out of their key groups' min/max.
 * SKVQ caches (whose sinks and chunks follow from the token stream) return
 * KVQ_E_UNSUPPORTED: fill them with kvq_prefill and kvq_append. */
kvq_status kvq_encode(kvq_cache* cache, const void* K, const void* V, int64_t ld_tok,
                      const int32_t* n_tok, void* stream);

/* Stateless form of the same quantizer, for checking it element by element ("Changelog"
 * v0.8.0 KIVI: per-channel keys, per-token values; v0.42.0 codes + per-group (scale, zero)).
 * Quantizes one fp16 block X [n_tok][D] (device, row-major) to `bits`-bit codes in groups of
 * `group` elements:
 *   per_channel != 0: a group is `group` consecutive tokens of one channel (the key rule);
 *     n_tok % group == 0; scales and zeros are fp16 [n_tok/group][D];
 *   per_channel == 0: a group is `group` consecutive channels of one token (the value rule);
 *     D % group == 0; scales and zeros are fp16 [n_tok][D/group].
 *   codes: uint8 [n_tok][D], one unpacked code per element.
 * bits in {2, 4, 8}, group == 32 (KVQ_E_UNSUPPORTED otherwise); n_tok >= 0, 1 <= D <= 4096
 * (KVQ_E_INVALID otherwise). All buffers are caller-owned device memory; nothing is
 * allocated. The arithmetic is exactly kvq_encode's, so codes, scales and zeros equal the
 * record contents bit for bit. Asynchronous on `stream`. */
kvq_status kvq_encode_block(const void* X, int32_t n_tok, int32_t D, int32_t bits, int32_t group,
                            int32_t per_channel, void* codes, void* scales, void* zeros, void* stream);

/* Fill an EMPTY cache with seq_len[b] tokens per sequence following the window rule of the
 * residual window ("Changelog" v0.8.0, v0.28.0): the first S - n_r tokens are quantized and
 * the last n_r = ((S - 1) mod R) + 1 stay fp16 (S = 0 leaves the sequence empty).
 * K, V as in kvq_encode; seq_len is a HOST array of B entries. A sequence that is not
 * empty is KVQ_E_INVALID; S > max_tokens is KVQ_E_CAPACITY. With n_sink > 0 the sinks are
 * chosen among the S - n_r quantized tokens (none when that is 0). */
kvq_status kvq_prefill(kvq_cache* cache, const void* K, const void* V, int64_t ld_tok,
                       const int32_t* seq_len, void* stream);

/* North-star call 2 (residual window and chunk flush, "Changelog" v0.8.0 / v0.28.0).
 * Append one token to every sequence: k_tok, v_tok fp16 [B][H_kv][D]. A sequence whose
 * window is full first quantizes all R window tokens (R/32 key groups, R value tokens)
 * exactly as kvq_encode would, then stores the new token as window slot 0 (with n_sink > 0,
 * a sequence's first flush chooses its sinks among the R window tokens).
 * KVQ_E_CAPACITY if any sequence would exceed max_tokens (nothing is enqueued). */
kvq_status kvq_append(kvq_cache* cache, const void* k_tok, const void* v_tok, void* stream);

/* North-star call 3 (fused decode + attention, "Changelog" v0.42.0).
 * out[b][h] = softmax(sm_scale * q[b][h] . K_hat[b][h/G]^T) V_hat[b][h/G] over all
 * quantized and window tokens of sequence b, with K_hat / V_hat rebuilt in registers from
 * the codes and fp16 (scale, zero) and never written out; fp32 scores and accumulation.
 *   q:   fp16 [B][H_q][D];  out: fp16 [B][H_q][D], or fp32 when out_fp32 != 0.
 *   workspace: at least kvq_workspace_bytes(cfg, n_split) device bytes (KVQ_E_WORKSPACE).
 *   n_split: maximum splits per sequence along the tokens (0 = chosen from the lengths).
 * Every sequence must hold at least one token (KVQ_E_INVALID otherwise). Sink tokens
 * (n_sink > 0) enter with their fp16 rows, and their quantized slots are skipped.
 * One kernel: splits along the tokens write (acc, m, l) partials to the workspace and the
 * last split of each sequence and KV head merges them (counted in the cache's sync region).
 * Calls on one cache must therefore be ordered (one stream, or synchronised streams). */
kvq_status kvq_decode_attend(kvq_cache* cache, const void* q, void* out, int32_t out_fp32,
                             float sm_scale, void* workspace, size_t ws_bytes, int32_t n_split,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kvq_decode_attend without a caller workspace. The
 * split partials go to a file-scope device array of KVQ_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; nothing is allocated or freed by this
 * call (no hipMalloc / hipFree, no allocating library routine), and no profiling events are
 * created or recorded.
 *   Arguments, layout, ordering and errors as kvq_decode_attend; a call whose partials
 *   (B * H_q * n_splits * (D + 4) * 4 bytes for the split count the call uses) exceed
 *   KVQ_NOALLOC_SCRATCH_BYTES is KVQ_E_WORKSPACE, with nothing enqueued.
 * All calls on one GPU share that GPU's array, and it keeps the last call's contents (nothing
 * in it needs to start at zero: every partial a call reads, the same call wrote). Calls that
 * overlap on one GPU (unordered streams, or several host threads) race on it: order them. */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)
kvq_status kvq_decode_attend_noalloc(kvq_cache* cache, const void* q, void* out, int32_t out_fp32,
                                     float sm_scale, int32_t n_split, void* stream);

/* Multi-query attend: speculative decoding (a few new tokens scored at once) and chunked prefill
 * (hundreds), the multi-token work the pages pair with their fused decode ("Changelog" v0.40.0
 * "Added": a matrix-tiled prefill / cross-attention companion for large S_q; v0.42.0 "Added" for
 * the decode attention itself). The newest n_query tokens of every sequence (already appended)
 * each attend, causally, over the cache up to and including themselves: query j (0-based) of
 * head h of sequence b sees the first S_b - (n_query - 1 - j) tokens, S_b being all the tokens
 * the sequence holds (sinks, quantized and window, in token order). n_query = 1 is
 * kvq_decode_attend.
 *   q:   fp16 [B][H_q][n_query][D];  out: fp16 (or fp32) [B][H_q][n_query][D].
 *   n_query: 1 .. max_tokens; every sequence holds at least n_query tokens (KVQ_E_INVALID).
 *   workspace: at least n_query x kvq_workspace_bytes(cfg, n_split) bytes.
 * Two kernels serve it, by the query rows per KV head (G x n_query, G = H_q / H_kv):
 *  - at most 8 rows and n_query a power of two: the decode kernel of kvq_decode_attend, the rows
 *    sharing every code it unpacks; every method and sink setting;
 *  - otherwise the matrix-core kernel (KIVI caches without sinks; KVQ_E_UNSUPPORTED for others):
 *    256 rows per workgroup, k_hat / v_hat rebuilt once per 32 tokens as fp16 high + low pairs
 *    (within 2^-20 relative) and multiplied on v_mfma_f32_16x16x32_f16 tiles with fp32
 *    accumulation; splits along the tokens are merged by a second kernel.
 * Masked scores take a large negative finite value, so a split that sees only a query's future
 * contributes nothing to it. */
kvq_status kvq_decode_attend_multi(kvq_cache* cache, const void* q, void* out, int32_t n_query, int32_t out_fp32,
                                   float sm_scale, void* workspace, size_t ws_bytes, int32_t n_split,
                                   void* stream);

/* North-star calls 2 and 3 in one ("Changelog" v0.8.0 / v0.28.0 window and chunk flush, v0.42.0
 * fused decode): exactly kvq_append(cache, k_tok, v_tok) followed by
 * kvq_decode_attend(cache, q, ...) on the same stream, same arguments and errors, same cache
 * state and output. When no window is full (31 appends in 32 at R = 32) it is one kernel
 * launch: the decode reads each new token from k_tok / v_tok, stores it in its window slot and
 * advances the device lengths. Otherwise the window is flushed by the append kernel first. */
kvq_status kvq_append_decode_attend(kvq_cache* cache, const void* k_tok, const void* v_tok, const void* q,
                                    void* out, int32_t out_fp32, float sm_scale, void* workspace,
                                    size_t ws_bytes, int32_t n_split, void* stream);

/* Timing hook for benchmarks: while enabled, kvq_decode_attend launches its split pass (the
 * dominant kernel) with a pair of HIP events that the kernel's own dispatch stamps at its start
 * and end (hipExtLaunchKernelGGL), so each pair brackets that kernel's execution on the
 * caller's stream and nothing else. enable = n > 0 turns this on and creates the events of
 * min(n, 4096) launches up front (so that timed launches create none); 0 turns it off.
 * kvq_profile_read waits for the recorded events and returns their total elapsed
 * milliseconds and count, then clears them. At most 4096 pairs are kept (KVQ_E_INVALID past
 * that). */
kvq_status kvq_profile_enable(kvq_cache* cache, int32_t enable);
kvq_status kvq_profile_read(kvq_cache* cache, double* total_ms, int64_t* count);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* kvq_last_error(void);

/* Name of a status code. */
const char* kvq_status_string(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
