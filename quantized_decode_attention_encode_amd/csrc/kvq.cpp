// kvq.cpp - host side of the C ABI declared in include/kvq.h.
//
// Validation happens here, on the host, before any launch; lengths are mirrored on the
// host (every change is decided here) so capacity checks and decode geometry never need a
// device synchronisation. The decode and append kernels take the mirror as kernel arguments
// (their loads then wait for nothing, and a decode that also appends never plans from lengths
// it rewrites itself); the device copy is kept for the other kernels and readers. Each call
// is planned from the mirror at enqueue time, so a captured graph of these calls replays
// that plan: it is valid only for the lengths it was captured at.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kvq.h"  // include/ is on the include path
#include "kernels.h"
#include "layout.h"

using kvq::Layout;
using kvq::PerSeq;

struct kvq_cache {
  kvq_config cfg;
  Layout L;
  uint8_t* buf;
  size_t bytes;
  std::vector<int32_t> nq, nr;  // host mirror of the lengths, per sequence
  std::vector<int32_t> nsp;     // SKVQ: sinks present per sequence (the first tokens)
  bool dev_ready;               // device lengths have been written at least once
  bool profiling;
  std::vector<hipEvent_t> ev;   // begin/end pairs
  size_t ev_used;
};

namespace {

constexpr int kMaxDevices = 64;
thread_local std::string g_err;

kvq_status fail(kvq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kvq_status fail(kvq_status st, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  g_err = msg;
  return st;
}

kvq_status ok() {
  g_err.clear();
  return KVQ_OK;
}

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxResidual = 256;
constexpr int kMaxProfilePairs = 4096;

kvq_status check_config(const kvq_config* c) {
  if (!c) return fail(KVQ_E_INVALID, "config is NULL");
  if (c->batch < 1 || c->batch > KVQ_MAX_BATCH)
    return fail(KVQ_E_INVALID, "batch must be in [1, %d], got %d", KVQ_MAX_BATCH, c->batch);
  if (c->n_kv_heads < 1) return fail(KVQ_E_INVALID, "n_kv_heads must be >= 1");
  if (c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads)
    return fail(KVQ_E_INVALID, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(KVQ_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8, got %d", G);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVQ_E_UNSUPPORTED, "head_dim must be 64 or 128, got %d", c->head_dim);
  if (c->method == KVQ_METHOD_KITTY) {
    if (c->key_bits != 2 || c->kitty_hi_bits != 4)
      return fail(KVQ_E_UNSUPPORTED, "Kitty key widths must be 2 (key_bits) and 4 (kitty_hi_bits), got %d and %d",
                  c->key_bits, c->kitty_hi_bits);
    if (c->value_bits != 16) return fail(KVQ_E_INVALID, "Kitty keeps values in fp16: value_bits must be 16, got %d", c->value_bits);
    if (c->kitty_n_hi < 0 || c->kitty_n_hi > c->head_dim || c->kitty_n_hi % 16)
      return fail(KVQ_E_UNSUPPORTED, "kitty_n_hi must be a multiple of 16 in [0, head_dim], got %d", c->kitty_n_hi);
    if (c->n_sink != 0) return fail(KVQ_E_UNSUPPORTED, "Kitty caches take no sink tokens (n_sink = %d)", c->n_sink);
    // the running key sums stay exact for every finite fp16 key up to 2^22 tokens: |sum X| <
    // 2^22 * 2^40 fits int64, and n * sum X^2 < 2^44 * 2^80 fits 128 bits
    if (c->max_tokens > (1 << 22))
      return fail(KVQ_E_UNSUPPORTED, "Kitty caches hold at most 2^22 tokens per sequence, got max_tokens %d", c->max_tokens);
  } else {
    for (int bits : {c->key_bits, c->value_bits})
      if (bits != 2 && bits != 4 && bits != 8)
        return fail(KVQ_E_UNSUPPORTED, "bit widths must be 2, 4 or 8, got %d", bits);
  }
  if (c->group != kvq::kGroup) return fail(KVQ_E_UNSUPPORTED, "group size must be 32, got %d", c->group);
  if (c->residual < kvq::kGroup || c->residual > kMaxResidual || c->residual % kvq::kGroup)
    return fail(KVQ_E_INVALID, "residual must be a multiple of 32 in [32, %d], got %d", kMaxResidual, c->residual);
  if (c->max_tokens < kvq::kGroup || c->max_tokens % kvq::kGroup)
    return fail(KVQ_E_INVALID, "max_tokens must be a positive multiple of 32, got %d", c->max_tokens);
  if (c->max_tokens > (1 << 26)) return fail(KVQ_E_INVALID, "max_tokens above 2^26");
  if (c->n_sink < 0 || c->n_sink > kvq::kMaxSinks)
    return fail(KVQ_E_INVALID, "n_sink must be in [0, %d], got %d", kvq::kMaxSinks, c->n_sink);
  if (c->method != KVQ_METHOD_KIVI && c->method != KVQ_METHOD_SKVQ && c->method != KVQ_METHOD_KITTY)
    return fail(KVQ_E_UNSUPPORTED, "method must be KVQ_METHOD_KIVI, KVQ_METHOD_SKVQ or KVQ_METHOD_KITTY, got %d",
                c->method);
  if (c->method == KVQ_METHOD_SKVQ) {
    if ((c->skvq_reorder != 0 && c->skvq_reorder != 1) || (c->skvq_clip_search != 0 && c->skvq_clip_search != 1))
      return fail(KVQ_E_INVALID, "skvq_reorder and skvq_clip_search must be 0 or 1");
    if (!c->skvq_clip_search && !(c->skvq_clip_alpha > 0.0f && c->skvq_clip_alpha <= 1.0f))
      return fail(KVQ_E_INVALID, "skvq_clip_alpha must be in (0, 1], got %g", double(c->skvq_clip_alpha));
  }
  return ok();
}

bool is_skvq(const kvq_config& c) { return c.method == KVQ_METHOD_SKVQ; }
bool is_kitty(const kvq_config& c) { return c.method == KVQ_METHOD_KITTY; }

Layout make_layout(const kvq_config* c) {
  Layout L;
  const bool sk = c->method == KVQ_METHOD_SKVQ;
  const bool kt = c->method == KVQ_METHOD_KITTY;
  // the fixed clip fraction in fp32 operations, or -1 for the search
  const float clip = (sk && !c->skvq_clip_search) ? (1.0f - c->skvq_clip_alpha) * 0.5f : -1.0f;
  // Kitty: (bk, bv) = (2, 2) selects the append kernel instance, which only stores tokens for
  // these caches (their windows are flushed by the Kitty encode launches)
  L.init(c->batch, c->n_kv_heads, c->head_dim, c->key_bits, kt ? c->key_bits : c->value_bits, c->residual,
         c->max_tokens, c->n_sink, c->method, clip, sk ? c->skvq_reorder : 1, kt ? c->kitty_n_hi : 0);
  return L;
}

// Decode units of a sequence: its records, its window in 32-token pieces, and its sinks (one
// unit, present when any sink is: KIVI-Sink once tokens are quantized, SKVQ from the first token).
int units_of(int nq, int nr, bool sinks) {
  return nq / kvq::kGroup + (nr + kvq::kGroup - 1) / kvq::kGroup + (sinks ? 1 : 0);
}

bool has_sinks(const kvq_cache* c, int b) {
  return c->cfg.n_sink > 0 && (is_skvq(c->cfg) ? c->nsp[b] > 0 : c->nq[b] > 0);
}

// Largest split count the automatic choice can produce.
int max_auto_splits(const kvq_config* c) {
  const int units_cap = c->max_tokens / kvq::kGroup + c->residual / kvq::kGroup + (c->n_sink > 0 ? 1 : 0);
  return (units_cap + 3) / 4;
}

// Device check: the current HIP device must be a gfx950. The verdict and the CU count are kept
// per device id (querying the properties costs far more than a kernel launch).
int g_cus[kMaxDevices];  // CUs of each checked gfx950 device

kvq_status check_device(int* cus = nullptr) {
  static std::atomic<int8_t> verdict[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_E_NODEVICE, "no HIP device: %s", hipGetErrorString(e));
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && verdict[dev].load(std::memory_order_acquire) == 1) {
    if (cus) *cus = g_cus[dev];
    return ok();
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(KVQ_E_NODEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  const bool good = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (!good) {
    if (cached) verdict[dev].store(-1, std::memory_order_release);
    return fail(KVQ_E_NODEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (cached) {
    g_cus[dev] = prop.multiProcessorCount;
    verdict[dev].store(1, std::memory_order_release);
  }
  if (cus) *cus = prop.multiProcessorCount;
  return ok();
}

// A ragged batch: its longest sequence holds more than 1.5 x the mean units.
bool ragged_batch(int max_units, int64_t total_units, int64_t seq_heads) {
  return double(max_units) * double(seq_heads) > 1.5 * double(total_units);
}
// Workgroups the automatic split aims for: two per CU when the sequences are about equally
// long, three when they are ragged (max > 1.5 x mean units), where smaller chunks fill the
// gaps the short sequences leave. Both were the fastest of 2, 3 and 4 per CU on the uniform
// (one 64K-token sequence; 8 x 32K tokens, 4 query heads per KV head) and ragged (16
// sequences of 1K..16K tokens) workloads.
int target_workgroups(int cus, int max_units, int64_t total_units, int64_t seq_heads) {
  return std::max(1, cus) * (ragged_batch(max_units, total_units, seq_heads) ? 3 : 2);
}

// Skewed splits for the vector-ALU decode at two workgroups per CU: the workgroups dispatched
// first (split-major order: the first half of every sequence's splits) share their CUs with
// the second half and win the SIMD arbiter over them; with equal chunks they finish about a
// sixth sooner. The first n_hi = n_split / 2 splits therefore take kSkew times the units of
// the others, which evens the pair's finish (on the 64K-token, 32-head cache: kSkew 1.2, 1.3,
// 1.35, 1.4 and 1.5 gave 40.1, 39.7, 39.6, 39.3 and 40.1 us, against 41.2-41.7 us with equal
// splits). KIVI caches only: the SKVQ decode (per-token key groups, its longer window)
// measured slower with it (44.8 -> 50.2 us on the same cache).
constexpr double kSkew = 1.4;
void skew_splits(int max_units, int n_split, kvq::DecodeShape& ds) {
  ds.n_hi = 0;
  ds.chunk_hi = 0;
  if (n_split < 2 || ds.chunk < 24) return;  // short chunks: launch-bound, nothing to even out
  const int n_hi = n_split / 2;
  const int lo = int(std::ceil(double(max_units) / (kSkew * n_hi + (n_split - n_hi))));
  const int hi = int(std::ceil(kSkew * lo));
  if (lo < 1 || int64_t(n_hi) * hi + int64_t(n_split - n_hi) * lo < max_units) return;
  ds.n_hi = n_hi;
  ds.chunk_hi = hi;
  ds.chunk = lo;
}

// Split plan of the matrix-core decode, whose workgroups fill a CU each. With n_split > 0,
// sequence b gets ceil(units_b / chunk) splits, chunk = ceil(max_units / n_split). Otherwise, for
// a number of workgroups per KV head (first cus / H_kv: one wave of workgroups), the smallest
// per-split load c such that sum_b min(limit_b, ceil(units_b / c)) splits fit, each sequence then
// cut into that many equal splits; limit_b keeps 16 units (two records per wave) per split and
// the workspace's split count. The largest splits are launched first. Returns the largest split
// count.
constexpr int kMfmaMinUnits = 16;
int plan_mfma(const int* units, int B, int Hkv, int n_split, int cus, int max_splits, kvq::SplitPlan& plan) {
  int max_units = 1;
  for (int b = 0; b < B; ++b) max_units = std::max(max_units, units[b]);
  int ns[kvq::kMaxBatch];
  if (n_split > 0) {
    const int cap = std::max(1, std::min(n_split, 65535 / B));  // the plan's 16-bit prefix
    const int chunk = (max_units + cap - 1) / cap;
    for (int b = 0; b < B; ++b) ns[b] = (units[b] + chunk - 1) / chunk;
  } else {
    auto splits = [&](int b, int c) {
      const int lim = std::max(1, std::min(max_splits, units[b] / kMfmaMinUnits));
      return std::min(lim, (units[b] + c - 1) / c);
    };
    const int per_head = std::max(1, cus / std::max(1, Hkv));
    int lo = 1, hi = max_units;  // the smallest c whose splits fit per_head workgroups
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      int64_t n = 0;
      for (int b = 0; b < B; ++b) n += splits(b, mid);
      if (n <= per_head) hi = mid;
      else lo = mid + 1;
    }
    for (int b = 0; b < B; ++b) ns[b] = splits(b, lo);
  }
  // sequences by split size, largest first (ties: lower index first)
  int idx[kvq::kMaxBatch];
  for (int b = 0; b < B; ++b) idx[b] = b;
  std::stable_sort(idx, idx + B, [&](int x, int y) {
    return (units[x] + ns[x] - 1) / ns[x] > (units[y] + ns[y] - 1) / ns[y];
  });
  int most = 1, first = 0;
  plan.set(0, 0);
  for (int k = 0; k < B; ++k) {
    const int b = idx[k];
    plan.order[k] = uint8_t(b);
    most = std::max(most, ns[b]);
    first += ns[b];
    plan.set(k + 1, first);
  }
  return most;
}

kvq_status ensure_ready(kvq_cache* c, hipStream_t s) {
  kvq_status st = check_device();
  if (st != KVQ_OK) return st;
  if (!c->dev_ready) {
    PerSeq z;
    memset(&z, 0, sizeof z);
    hipError_t e = kvq::launch_lengths_fill(c->buf, c->L, z, s, 1);
    if (e != hipSuccess) return hip_fail(e, "zeroing lengths");
    c->dev_ready = true;
  }
  return ok();
}

}  // namespace

namespace {

// Multi-query attend on the matrix cores: 256-row blocks of each KV head's query rows, splits along
// the units so that the grid holds about one workgroup per CU (or n_split when given).
kvq_status tiles_enqueue(kvq_cache* c, const void* q, void* out, int32_t out_fp32, float sm_scale, void* workspace,
                         size_t ws_bytes, int32_t n_split, void* stream, int32_t n_query, bool allow_profile) {
  const kvq_config& cfg = c->cfg;
  const int G = cfg.n_q_heads / cfg.n_kv_heads;
  int max_units = 0;
  for (int b = 0; b < cfg.batch; ++b) {
    const int held = c->nq[b] + c->nr[b];
    if (held < n_query)
      return fail(KVQ_E_INVALID, "sequence %d holds %d tokens, fewer than the %d queries", b, held, n_query);
    max_units = std::max(max_units, units_of(c->nq[b], c->nr[b], false));
  }
  kvq::TileShape ts;
  ts.G = G;
  ts.n_q_heads = cfg.n_q_heads;
  ts.nqry = n_query;
  ts.row_blocks = (G * n_query + 255) / 256;
  ts.qscale = sm_scale * 1.4426950408889634f;
  ts.out_fp32 = out_fp32 ? 1 : 0;
  int chunk;
  if (n_split > 0) {
    chunk = (max_units + n_split - 1) / n_split;
  } else {
    int cus = 0;
    kvq_status dst = check_device(&cus);
    if (dst != KVQ_OK) return dst;
    const int64_t blocks = int64_t(cfg.batch) * cfg.n_kv_heads * ts.row_blocks;
    // splits per sequence (one 8-wave workgroup per CU), within what kvq_workspace_bytes(cfg, 0)
    // provides for
    const int64_t want = std::min<int64_t>((int64_t(std::max(1, cus)) + blocks - 1) / blocks, max_auto_splits(&cfg));
    chunk = int((max_units + want - 1) / want);
  }
  chunk = std::max(1, chunk);
  ts.chunk = chunk;
  ts.n_split = (max_units + chunk - 1) / chunk;
  const size_t need = ts.n_split > 1
      ? size_t(cfg.batch) * cfg.n_q_heads * n_query * ts.n_split * (cfg.head_dim + 4) * sizeof(float) : 0;
  if (ws_bytes < need) return fail(KVQ_E_WORKSPACE, "workspace holds %zu bytes, this call needs %zu", ws_bytes, need);
  if (need && !workspace) return fail(KVQ_E_WORKSPACE, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq_status st = ensure_ready(c, s);
  if (st != KVQ_OK) return st;
  PerSeq seq;
  memset(&seq, 0, sizeof seq);
  for (int b = 0; b < cfg.batch; ++b) {
    seq.a[b] = c->nq[b];
    seq.b[b] = c->nr[b];
  }
  const bool prof = c->profiling && allow_profile;
  if (prof && c->ev_used + 2 > c->ev.size()) {
    if (c->ev.size() >= size_t(2 * kMaxProfilePairs)) return fail(KVQ_E_INVALID, "profile buffer full; call kvq_profile_read");
    for (int i = 0; i < 2; ++i) {
      hipEvent_t ev;
      hipError_t e = hipEventCreate(&ev);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
      c->ev.push_back(ev);
    }
  }
  hipError_t e = kvq::launch_attend_tiles(c->buf, c->L, ts, seq, q, static_cast<float*>(workspace), out, s,
                                          prof ? c->ev[c->ev_used] : nullptr, prof ? c->ev[c->ev_used + 1] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "multi-query attend launch");
  if (prof) c->ev_used += 2;
  return ok();
}

// Plan and enqueue one decode launch. With k_tok / v_tok set, the launch also appends one token
// per sequence (the caller has checked that no window is full): it attends over the window
// plus that token, stores the token in its slot and advances the device lengths.
// n_query > 1: that many queries per head, the cache's newest tokens (causal among themselves).
kvq_status decode_enqueue(kvq_cache* c, const void* q, void* out, int32_t out_fp32, float sm_scale,
                          void* workspace, size_t ws_bytes, int32_t n_split, void* stream,
                          const void* k_tok, const void* v_tok, int32_t n_query = 1, bool allow_profile = true) {
  if (!q || !out) return fail(KVQ_E_INVALID, "q or out is NULL");
  if (!workspace) return fail(KVQ_E_WORKSPACE, "workspace is NULL");
  if (n_split < 0) return fail(KVQ_E_INVALID, "n_split must be >= 0");
  if (!std::isfinite(sm_scale)) return fail(KVQ_E_INVALID, "sm_scale is not finite");
  const kvq_config& cfg = c->cfg;
  const int add = k_tok ? 1 : 0;  // window tokens the launch appends
  const int G = cfg.n_q_heads / cfg.n_kv_heads;
  if (is_kitty(cfg) && k_tok) return fail(KVQ_E_UNSUPPORTED, "Kitty caches append before the decode launch");
  if (n_query < 1) return fail(KVQ_E_INVALID, "n_query = %d must be >= 1", n_query);
  if (n_query > cfg.max_tokens) return fail(KVQ_E_INVALID, "n_query = %d exceeds max_tokens %d", n_query, cfg.max_tokens);
  // More query rows per KV head than the decode kernel holds (8), or a count that is not a power
  // of two: the matrix-core kernel, for KIVI caches without sinks.
  if (G * n_query > 8 || (n_query & (n_query - 1))) {
    if (cfg.method != KVQ_METHOD_KIVI || cfg.n_sink != 0)
      return fail(KVQ_E_UNSUPPORTED, "n_query = %d with %d query heads per KV head (more than 8 rows, or not a power of "
                  "two) is built for KIVI caches without sinks", n_query, G);
    return tiles_enqueue(c, q, out, out_fp32, sm_scale, workspace, ws_bytes, n_split, stream, n_query, allow_profile);
  }
  int max_units = 0;
  int64_t total_units = 0;
  int units[kvq::kMaxBatch];
  for (int b = 0; b < cfg.batch; ++b) {
    const int held = c->nq[b] + c->nr[b] + c->nsp[b] + add;
    if (held == 0) return fail(KVQ_E_INVALID, "sequence %d is empty", b);
    if (held < n_query)
      return fail(KVQ_E_INVALID, "sequence %d holds %d tokens, fewer than the %d queries", b, held, n_query);
    const int u = units_of(c->nq[b], c->nr[b] + add, has_sinks(c, b));
    units[b] = u;
    max_units = std::max(max_units, u);
    total_units += int64_t(u) * cfg.n_kv_heads;
  }
  // 4 or 8 query rows per KV head of a KIVI cache without sinks: both per-record products on the
  // matrix cores, with a split plan of its own
  const bool mfma = cfg.method == KVQ_METHOD_KIVI && cfg.n_sink == 0 && (G * n_query == 4 || G * n_query == 8);
  kvq::SplitPlan plan;
  memset(&plan, 0, sizeof plan);
  int chunk = 0, ns;
  if (mfma) {
    int cus = 0;
    if (n_split == 0) {
      kvq_status dst = check_device(&cus);
      if (dst != KVQ_OK) return dst;
    }
    ns = plan_mfma(units, cfg.batch, cfg.n_kv_heads, n_split, cus, max_auto_splits(&cfg), plan);
  } else if (n_split > 0) {
    chunk = (max_units + n_split - 1) / n_split;
  } else {
    int cus = 0;
    kvq_status dst = check_device(&cus);
    if (dst != KVQ_OK) return dst;
    const int64_t target = target_workgroups(cus, max_units, total_units, int64_t(cfg.batch) * cfg.n_kv_heads);
    chunk = int((total_units + target - 1) / target);
    chunk = std::max(4, (chunk + 3) / 4 * 4);
  }
  if (!mfma) ns = (max_units + chunk - 1) / chunk;
  const size_t need = size_t(cfg.batch) * cfg.n_q_heads * n_query * ns * (cfg.head_dim + 4) * sizeof(float);
  if (ws_bytes < need) return fail(KVQ_E_WORKSPACE, "workspace holds %zu bytes, this call needs %zu", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq_status st = ensure_ready(c, s);
  if (st != KVQ_OK) return st;
  kvq::DecodeShape ds;
  ds.n_split = ns;
  ds.chunk = chunk;
  ds.n_hi = 0;
  ds.chunk_hi = 0;
  if (!mfma && cfg.method == KVQ_METHOD_KIVI && n_split == 0 &&
      !ragged_batch(max_units, total_units, int64_t(cfg.batch) * cfg.n_kv_heads))
    skew_splits(max_units, ns, ds);
  ds.G = G * n_query;  // query rows per KV head
  ds.n_q_heads = cfg.n_q_heads * n_query;
  ds.nqry = n_query;
  ds.qscale = sm_scale * 1.4426950408889634f;
  ds.out_fp32 = out_fp32 ? 1 : 0;
  ds.append = add;
  PerSeq seq;  // the plan's lengths: the host mirror before this launch's append
  memset(&seq, 0, sizeof seq);
  for (int b = 0; b < cfg.batch; ++b) {
    seq.a[b] = c->nq[b];
    seq.b[b] = c->nr[b];
    seq.c[b] = is_skvq(cfg) ? c->nsp[b] : (has_sinks(c, b) ? cfg.n_sink : 0);
  }
  float* ws = static_cast<float*>(workspace);
  hipError_t e;
  const bool prof = c->profiling && allow_profile;
  if (prof) {
    if (c->ev_used + 2 > c->ev.size()) {
      if (c->ev.size() >= size_t(2 * kMaxProfilePairs)) return fail(KVQ_E_INVALID, "profile buffer full; call kvq_profile_read");
      for (int i = 0; i < 2; ++i) {
        hipEvent_t ev;
        e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        c->ev.push_back(ev);
      }
    }
  }
  // With profiling on, the events are stamped by the kernel's own dispatch packet, so their
  // interval is its execution time (no queue or launch latency).
  if (is_kitty(cfg))
    e = kvq::launch_kitty_decode(c->buf, c->L, ds, q, ws, out, s, prof ? c->ev[c->ev_used] : nullptr,
                                 prof ? c->ev[c->ev_used + 1] : nullptr);
  else if (mfma)
    e = kvq::launch_decode_mfma(c->buf, c->L, ds, seq, plan, q, ws, out, k_tok, v_tok, s,
                                prof ? c->ev[c->ev_used] : nullptr, prof ? c->ev[c->ev_used + 1] : nullptr);
  else
    e = kvq::launch_decode(c->buf, c->L, ds, seq, q, ws, out, k_tok, v_tok, s, prof ? c->ev[c->ev_used] : nullptr,
                           prof ? c->ev[c->ev_used + 1] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (prof) c->ev_used += 2;
  if (add)
    for (int b = 0; b < cfg.batch; ++b) c->nr[b] += 1;
  return ok();
}

}  // namespace

// Split partials of kvq_decode_attend_noalloc: a file-scope device array, so that the call needs
// no caller workspace and allocates nothing. Every GPU the library runs on holds its own copy
// (KVQ_NOALLOC_SCRATCH_BYTES) until the process ends; in host code `scratch` only names the
// symbol, and its device address is looked up once per device and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

kvq_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_E_NODEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_E_NODEVICE, "device %d is beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(KVQ_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ok();
}

}  // namespace

extern "C" {

kvq_status kvq_probe(int32_t* has_gfx950) {
  if (!has_gfx950) return fail(KVQ_E_INVALID, "has_gfx950 is NULL");
  *has_gfx950 = 0;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) {
    (void)hipGetLastError();
    return ok();
  }
  for (int d = 0; d < n; ++d) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, d) == hipSuccess && strncmp(prop.gcnArchName, "gfx950", 6) == 0) {
      *has_gfx950 = 1;
      break;
    }
  }
  return ok();
}

kvq_status kvq_config_check(const kvq_config* cfg) { return check_config(cfg); }

kvq_status kvq_kitty_n_hi(int32_t head_dim, double hi_fraction, int32_t* n_hi) {
  if (!n_hi) return fail(KVQ_E_INVALID, "kvq_kitty_n_hi: n_hi is NULL");
  if (head_dim < 1) return fail(KVQ_E_INVALID, "kvq_kitty_n_hi: head_dim must be positive");
  if (!(hi_fraction >= 0.0 && hi_fraction <= 1.0))
    return fail(KVQ_E_INVALID, "kvq_kitty_n_hi: the fraction must be a number in [0, 1]");
  *n_hi = int32_t(std::floor(hi_fraction * double(head_dim) + 0.5));
  return ok();
}

size_t kvq_cache_bytes(const kvq_config* cfg) {
  if (check_config(cfg) != KVQ_OK) return 0;
  return size_t(make_layout(cfg).total);
}

kvq_status kvq_layout(const kvq_config* cfg, kvq_layout_info* out) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_E_INVALID, "out is NULL");
  const Layout L = make_layout(cfg);
  out->lengths_offset = L.len_off;
  out->records_offset = L.rec_off;
  out->record_bytes = L.rec_bytes;
  out->rec_key_codes = 0;
  out->rec_value_codes = kvq::rec_off_vcodes(L.D, L.bk);
  out->rec_key_params = kvq::rec_off_kparams(L.D, L.bk, L.bv);
  out->rec_value_params = kvq::rec_off_vparams(L.D, L.bk, L.bv);
  out->window_k_offset = L.wk_off;
  out->window_v_offset = L.wv_off;
  out->total_bytes = L.total;
  out->sync_offset = L.sync_off;
  out->sink_pos_offset = L.sp_off;
  out->sink_k_offset = L.sk_off;
  out->sink_v_offset = L.sv_off;
  out->perm_offset = L.pm_off;
  out->rec_slot_table = 0;
  out->kstats_offset = L.ks_off;
  if (is_kitty(*cfg)) {
    out->rec_key_codes = 0;
    out->rec_key_params = kvq::kitty_off_params(L.D, L.nhi);
    out->rec_slot_table = kvq::kitty_off_table(L.D, L.nhi);
    out->rec_value_codes = kvq::kitty_off_values(L.D, L.nhi);
    out->rec_value_params = 0;
  }
  return ok();
}

size_t kvq_workspace_bytes(const kvq_config* cfg, int32_t n_split) {
  if (check_config(cfg) != KVQ_OK || n_split < 0) return 0;
  const int ns = n_split > 0 ? n_split : max_auto_splits(cfg);
  return size_t(cfg->batch) * cfg->n_q_heads * ns * (cfg->head_dim + 4) * sizeof(float);
}

kvq_status kvq_cache_create(const kvq_config* cfg, void* dev_buf, size_t bytes, kvq_cache** out) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!dev_buf) return fail(KVQ_E_INVALID, "device buffer is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % 256) return fail(KVQ_E_INVALID, "device buffer must be 256-byte aligned");
  const Layout L = make_layout(cfg);
  if (bytes < L.total)
    return fail(KVQ_E_INVALID, "device buffer holds %zu bytes, the cache needs %llu", bytes,
                (unsigned long long)L.total);
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return fail(KVQ_E_INVALID, "out of host memory");
  c->cfg = *cfg;
  c->L = L;
  c->buf = static_cast<uint8_t*>(dev_buf);
  c->bytes = bytes;
  c->nq.assign(cfg->batch, 0);
  c->nr.assign(cfg->batch, 0);
  c->nsp.assign(cfg->batch, 0);
  c->dev_ready = false;
  c->profiling = false;
  c->ev_used = 0;
  *out = c;
  return ok();
}

void kvq_cache_destroy(kvq_cache* cache) {
  if (!cache) return;
  for (hipEvent_t e : cache->ev) (void)hipEventDestroy(e);
  delete cache;
}

kvq_status kvq_reset(kvq_cache* c, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  kvq_status st = check_device();
  if (st != KVQ_OK) return st;
  PerSeq z;
  memset(&z, 0, sizeof z);
  hipError_t e = kvq::launch_lengths_fill(c->buf, c->L, z, static_cast<hipStream_t>(stream), 1);
  if (e != hipSuccess) return hip_fail(e, "reset");
  std::fill(c->nq.begin(), c->nq.end(), 0);
  std::fill(c->nr.begin(), c->nr.end(), 0);
  std::fill(c->nsp.begin(), c->nsp.end(), 0);
  c->dev_ready = true;
  return ok();
}

kvq_status kvq_cache_lengths(const kvq_cache* c, int32_t* n_quantized, int32_t* n_window) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  for (int b = 0; b < c->cfg.batch; ++b) {
    if (n_quantized) n_quantized[b] = c->nq[b];
    if (n_window) n_window[b] = c->nr[b];
  }
  return ok();
}

kvq_status kvq_encode(kvq_cache* c, const void* K, const void* V, int64_t ld_tok, const int32_t* n_tok,
                      void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (!n_tok) return fail(KVQ_E_INVALID, "n_tok is NULL");
  if (is_skvq(c->cfg)) return fail(KVQ_E_UNSUPPORTED, "kvq_encode does not apply to SKVQ caches: use kvq_prefill / kvq_append");
  int max_rec = 0, max_tok = 0;
  for (int b = 0; b < c->cfg.batch; ++b) {
    const int n = n_tok[b];
    if (n < 0 || n % kvq::kGroup)
      return fail(KVQ_E_INVALID, "n_tok[%d] = %d is not a non-negative multiple of 32", b, n);
    if (n && c->nr[b]) return fail(KVQ_E_INVALID, "sequence %d has %d window tokens; encode needs an empty window", b, c->nr[b]);
    if (int64_t(c->nq[b]) + n > c->cfg.max_tokens)
      return fail(KVQ_E_CAPACITY, "sequence %d: %d + %d tokens exceed max_tokens %d", b, c->nq[b], n, c->cfg.max_tokens);
    max_rec = std::max(max_rec, n / kvq::kGroup);
    max_tok = std::max(max_tok, n);
  }
  if (max_tok == 0) return ok();
  if (!K || !V) return fail(KVQ_E_INVALID, "K or V is NULL");
  if (ld_tok < max_tok) return fail(KVQ_E_INVALID, "ld_tok %lld is below the longest block %d", (long long)ld_tok, max_tok);
  if ((reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) % 16)
    return fail(KVQ_E_INVALID, "K and V must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq_status st = ensure_ready(c, s);
  if (st != KVQ_OK) return st;
  PerSeq enc, len, sel;
  memset(&enc, 0, sizeof enc);
  memset(&len, 0, sizeof len);
  memset(&sel, 0, sizeof sel);
  bool select = false;
  for (int b = 0; b < c->cfg.batch; ++b) {
    enc.a[b] = c->nq[b] / kvq::kGroup;
    enc.b[b] = n_tok[b] / kvq::kGroup;
    len.a[b] = c->nq[b] + n_tok[b];
    len.b[b] = c->nr[b];
    sel.b[b] = (c->cfg.n_sink > 0 && c->nq[b] == 0) ? n_tok[b] : 0;  // first quantized tokens
    select = select || sel.b[b] > 0;
  }
  hipError_t e;
  if (select) {
    e = kvq::launch_sink_select(c->buf, c->L, K, V, ld_tok, sel, s);
    if (e != hipSuccess) return hip_fail(e, "sink selection launch");
  }
  if (is_kitty(c->cfg))
    e = kvq::launch_kitty_encode(c->buf, c->L, K, V, ld_tok, enc, max_rec, s);  // enc.c = 0: blocks start at token 0
  else
    e = kvq::launch_encode(c->buf, c->L, K, V, ld_tok, enc, max_rec, s);
  if (e != hipSuccess) return hip_fail(e, "encode launch");
  e = kvq::launch_lengths_fill(c->buf, c->L, len, s, 0);
  if (e != hipSuccess) return hip_fail(e, "lengths launch");
  for (int b = 0; b < c->cfg.batch; ++b) c->nq[b] += n_tok[b];
  return ok();
}

kvq_status kvq_encode_block(const void* X, int32_t n_tok, int32_t D, int32_t bits, int32_t group,
                            int32_t per_channel, void* codes, void* scales, void* zeros, void* stream) {
  if (bits != 2 && bits != 4 && bits != 8) return fail(KVQ_E_UNSUPPORTED, "bits = %d; supported: 2, 4, 8", bits);
  if (group != kvq::kGroup) return fail(KVQ_E_UNSUPPORTED, "group = %d; supported: %d", group, kvq::kGroup);
  if (n_tok < 0) return fail(KVQ_E_INVALID, "n_tok = %d is negative", n_tok);
  if (D < 1 || D > 4096) return fail(KVQ_E_INVALID, "D = %d is outside [1, 4096]", D);
  if (per_channel && n_tok % group)
    return fail(KVQ_E_INVALID, "per-channel groups need n_tok %% %d == 0 (n_tok = %d)", group, n_tok);
  if (!per_channel && D % group) return fail(KVQ_E_INVALID, "per-token groups need D %% %d == 0 (D = %d)", group, D);
  if (n_tok == 0) return ok();
  if (!X || !codes || !scales || !zeros) return fail(KVQ_E_INVALID, "NULL buffer");
  kvq_status st = check_device();
  if (st != KVQ_OK) return st;
  hipError_t e = kvq::launch_encode_block(X, n_tok, D, bits, group, per_channel ? 1 : 0, codes, scales, zeros,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "encode_block launch");
  return ok();
}

kvq_status kvq_prefill(kvq_cache* c, const void* K, const void* V, int64_t ld_tok, const int32_t* seq_len,
                       void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (!seq_len) return fail(KVQ_E_INVALID, "seq_len is NULL");
  const int R = c->cfg.residual;
  const bool sk = is_skvq(c->cfg);
  int max_rec = 0, max_S = 0;
  PerSeq enc, win, sel;
  memset(&enc, 0, sizeof enc);
  memset(&win, 0, sizeof win);
  memset(&sel, 0, sizeof sel);
  std::vector<int32_t> nsp(c->cfg.batch, 0);
  for (int b = 0; b < c->cfg.batch; ++b) {
    const int S = seq_len[b];
    if (S < 0) return fail(KVQ_E_INVALID, "seq_len[%d] = %d is negative", b, S);
    if (c->nq[b] || c->nr[b] || c->nsp[b])
      return fail(KVQ_E_INVALID, "sequence %d is not empty; prefill needs an empty cache", b);
    // SKVQ: the first n_sink tokens are the sinks and the window rule covers the rest
    const int ns = sk ? std::min(S, c->cfg.n_sink) : 0;
    if (S - ns > c->cfg.max_tokens)
      return fail(KVQ_E_CAPACITY, "seq_len[%d] = %d exceeds max_tokens %d", b, S, c->cfg.max_tokens);
    const int nr = S > ns ? (S - ns - 1) % R + 1 : 0;
    const int nq = S - ns - nr;
    nsp[b] = ns;
    enc.a[b] = 0;
    enc.b[b] = nq / kvq::kGroup;
    enc.c[b] = ns;  // first quantized token
    win.a[b] = nq;
    win.b[b] = nr;
    win.c[b] = ns + nq;  // first window token
    if (sk) {
      sel.b[b] = nq > 0 ? 1 : 0;  // permutations from the first chunk, tokens ns .. ns + R - 1
      sel.c[b] = ns;
    } else {
      sel.b[b] = c->cfg.n_sink > 0 ? nq : 0;  // sinks among the quantized part
    }
    max_rec = std::max(max_rec, nq / kvq::kGroup);
    max_S = std::max(max_S, S);
  }
  if (max_S && (!K || !V)) return fail(KVQ_E_INVALID, "K or V is NULL");
  if (ld_tok < max_S) return fail(KVQ_E_INVALID, "ld_tok %lld is below the longest sequence %d", (long long)ld_tok, max_S);
  if ((reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) % 16)
    return fail(KVQ_E_INVALID, "K and V must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq_status st = check_device();
  if (st != KVQ_OK) return st;
  if (max_rec && sk) {
    hipError_t e = kvq::launch_skvq_perm(c->buf, c->L, K, V, ld_tok, sel, s);
    if (e != hipSuccess) return hip_fail(e, "permutation launch");
    e = kvq::launch_skvq_encode(c->buf, c->L, K, V, ld_tok, enc, max_rec, 0, s);
    if (e != hipSuccess) return hip_fail(e, "encode launch");
  } else if (max_rec && is_kitty(c->cfg)) {
    hipError_t e = kvq::launch_kitty_encode(c->buf, c->L, K, V, ld_tok, enc, max_rec, s);
    if (e != hipSuccess) return hip_fail(e, "encode launch");
  } else if (max_rec) {
    hipError_t e;
    if (c->cfg.n_sink > 0) {
      e = kvq::launch_sink_select(c->buf, c->L, K, V, ld_tok, sel, s);
      if (e != hipSuccess) return hip_fail(e, "sink selection launch");
    }
    e = kvq::launch_encode(c->buf, c->L, K, V, ld_tok, enc, max_rec, s);
    if (e != hipSuccess) return hip_fail(e, "encode launch");
  }
  hipError_t e = kvq::launch_window_fill(c->buf, c->L, K, V, ld_tok, win, s);  // also writes every length
  if (e != hipSuccess) return hip_fail(e, "window launch");
  c->dev_ready = true;
  for (int b = 0; b < c->cfg.batch; ++b) {
    c->nq[b] = win.a[b];
    c->nr[b] = win.b[b];
    c->nsp[b] = nsp[b];
  }
  return ok();
}

kvq_status kvq_append(kvq_cache* c, const void* k_tok, const void* v_tok, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (!k_tok || !v_tok) return fail(KVQ_E_INVALID, "k_tok or v_tok is NULL");
  for (int b = 0; b < c->cfg.batch; ++b)
    if (int64_t(c->nq[b]) + c->nr[b] + 1 > c->cfg.max_tokens)
      return fail(KVQ_E_CAPACITY, "sequence %d is full (%d tokens)", b, c->cfg.max_tokens);
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq_status st = ensure_ready(c, s);
  if (st != KVQ_OK) return st;
  PerSeq len;  // lengths before the append: the host mirror of the device lengths
  for (int b = 0; b < c->cfg.batch; ++b) {
    len.a[b] = c->nq[b];
    len.b[b] = c->nr[b];
    len.c[b] = c->nsp[b];
  }
  if (is_skvq(c->cfg)) {
    // SKVQ windows are flushed here, one wave per record (the clip search is the costly part):
    // a first flush computes the permutations from the window and rewrites the window and sink
    // rows in permuted order; every flush then encodes the (permuted) window rows
    PerSeq first, fl;
    memset(&first, 0, sizeof first);
    memset(&fl, 0, sizeof fl);
    bool any = false, any_first = false;
    for (int b = 0; b < c->cfg.batch; ++b) {
      if (c->nsp[b] < c->cfg.n_sink || c->nr[b] < c->cfg.residual) continue;
      any = true;
      fl.a[b] = c->nq[b] / kvq::kGroup;
      fl.b[b] = c->cfg.residual / kvq::kGroup;
      if (c->nq[b] == 0) {
        first.b[b] = 1;
        any_first = true;
      }
      len.a[b] = c->nq[b] + c->cfg.residual;  // the append kernel then sees an empty window
      len.b[b] = 0;
    }
    const void* wk = c->buf + c->L.wk_off;
    const void* wv = c->buf + c->L.wv_off;
    hipError_t e;
    if (any_first) {
      e = kvq::launch_skvq_perm(c->buf, c->L, wk, wv, c->cfg.residual, first, s);
      if (e != hipSuccess) return hip_fail(e, "permutation launch");
      e = kvq::launch_skvq_permute_rows(c->buf, c->L, first, s);
      if (e != hipSuccess) return hip_fail(e, "row permutation launch");
    }
    if (any) {
      e = kvq::launch_skvq_encode(c->buf, c->L, wk, wv, c->cfg.residual, fl, c->cfg.residual / kvq::kGroup, 1, s);
      if (e != hipSuccess) return hip_fail(e, "flush launch");
    }
  }
  if (is_kitty(c->cfg)) {
    // full windows are quantized by the Kitty encode launches (their window rows are the source);
    // the append kernel then sees an empty window
    PerSeq fl;
    memset(&fl, 0, sizeof fl);
    bool any = false;
    for (int b = 0; b < c->cfg.batch; ++b) {
      if (c->nr[b] < c->cfg.residual) continue;
      any = true;
      fl.a[b] = c->nq[b] / kvq::kGroup;
      fl.b[b] = c->cfg.residual / kvq::kGroup;
      len.a[b] = c->nq[b] + c->cfg.residual;
      len.b[b] = 0;
    }
    if (any) {
      hipError_t e = kvq::launch_kitty_encode(c->buf, c->L, c->buf + c->L.wk_off, c->buf + c->L.wv_off,
                                              c->cfg.residual, fl, c->cfg.residual / kvq::kGroup, s);
      if (e != hipSuccess) return hip_fail(e, "flush launch");
    }
  }
  hipError_t e = kvq::launch_append(c->buf, c->L, k_tok, v_tok, len, s);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  for (int b = 0; b < c->cfg.batch; ++b) {
    if (is_skvq(c->cfg) && c->nsp[b] < c->cfg.n_sink) {  // the token became a sink
      c->nsp[b] += 1;
      continue;
    }
    if (c->nr[b] == c->cfg.residual) {
      c->nq[b] += c->cfg.residual;
      c->nr[b] = 0;
    }
    c->nr[b] += 1;
  }
  return ok();
}

kvq_status kvq_decode_attend(kvq_cache* c, const void* q, void* out, int32_t out_fp32, float sm_scale,
                             void* workspace, size_t ws_bytes, int32_t n_split, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  return decode_enqueue(c, q, out, out_fp32, sm_scale, workspace, ws_bytes, n_split, stream, nullptr, nullptr);
}

kvq_status kvq_decode_attend_noalloc(kvq_cache* c, const void* q, void* out, int32_t out_fp32, float sm_scale,
                                     int32_t n_split, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  kvq_status st = check_device();
  if (st != KVQ_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != KVQ_OK) return st;
  st = decode_enqueue(c, q, out, out_fp32, sm_scale, ws, KVQ_NOALLOC_SCRATCH_BYTES, n_split, stream, nullptr,
                      nullptr, 1, false);
  if (st == KVQ_E_WORKSPACE)
    return fail(KVQ_E_WORKSPACE, "kvq_decode_attend_noalloc: %s (the static scratch holds %u bytes; pass a smaller "
                "n_split, or use kvq_decode_attend with a workspace)", kvq_last_error(), unsigned(KVQ_NOALLOC_SCRATCH_BYTES));
  return st;
}

kvq_status kvq_decode_attend_multi(kvq_cache* c, const void* q, void* out, int32_t n_query, int32_t out_fp32,
                                   float sm_scale, void* workspace, size_t ws_bytes, int32_t n_split, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  return decode_enqueue(c, q, out, out_fp32, sm_scale, workspace, ws_bytes, n_split, stream, nullptr, nullptr,
                        n_query);
}

kvq_status kvq_append_decode_attend(kvq_cache* c, const void* k_tok, const void* v_tok, const void* q, void* out,
                                    int32_t out_fp32, float sm_scale, void* workspace, size_t ws_bytes,
                                    int32_t n_split, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (!k_tok || !v_tok) return fail(KVQ_E_INVALID, "k_tok or v_tok is NULL");
  if (!q || !out) return fail(KVQ_E_INVALID, "q or out is NULL");
  if (!workspace) return fail(KVQ_E_WORKSPACE, "workspace is NULL");
  if (n_split < 0) return fail(KVQ_E_INVALID, "n_split must be >= 0");
  if (!std::isfinite(sm_scale)) return fail(KVQ_E_INVALID, "sm_scale is not finite");
  bool flush = false;
  for (int b = 0; b < c->cfg.batch; ++b) {
    if (int64_t(c->nq[b]) + c->nr[b] + 1 > c->cfg.max_tokens)
      return fail(KVQ_E_CAPACITY, "sequence %d is full (%d tokens)", b, c->cfg.max_tokens);
    flush = flush || c->nr[b] == c->cfg.residual;
    // an SKVQ token that becomes a sink is the append kernel's work too
    flush = flush || (is_skvq(c->cfg) && c->nsp[b] < c->cfg.n_sink);
  }
  flush = flush || is_kitty(c->cfg);  // Kitty decode reads no appended token: append first
  if (flush) {  // some window is full: the append kernel quantizes it, then a plain decode
    kvq_status st = kvq_append(c, k_tok, v_tok, stream);
    if (st != KVQ_OK) return st;
    return decode_enqueue(c, q, out, out_fp32, sm_scale, workspace, ws_bytes, n_split, stream, nullptr, nullptr);
  }
  return decode_enqueue(c, q, out, out_fp32, sm_scale, workspace, ws_bytes, n_split, stream, k_tok, v_tok);
}

kvq_status kvq_profile_enable(kvq_cache* c, int32_t enable) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (enable < 0) return fail(KVQ_E_INVALID, "enable must be >= 0");
  c->profiling = enable != 0;
  // Create the events of `enable` launches now, so that timed launches create none.
  const size_t want = size_t(2) * std::min(enable, kMaxProfilePairs);
  while (c->ev.size() < want) {
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    c->ev.push_back(ev);
  }
  return ok();
}

kvq_status kvq_profile_read(kvq_cache* c, double* total_ms, int64_t* count) {
  if (!c || !total_ms || !count) return fail(KVQ_E_INVALID, "NULL argument");
  double tot = 0;
  for (size_t i = 0; i + 1 < c->ev_used; i += 2) {
    hipError_t e = hipEventSynchronize(c->ev[i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0;
    e = hipEventElapsedTime(&ms, c->ev[i], c->ev[i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot += ms;
  }
  *total_ms = tot;
  *count = int64_t(c->ev_used / 2);
  c->ev_used = 0;
  return ok();
}

const char* kvq_last_error(void) { return g_err.c_str(); }

const char* kvq_status_string(kvq_status st) {
  switch (st) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_E_INVALID: return "KVQ_E_INVALID";
    case KVQ_E_UNSUPPORTED: return "KVQ_E_UNSUPPORTED";
    case KVQ_E_CAPACITY: return "KVQ_E_CAPACITY";
    case KVQ_E_WORKSPACE: return "KVQ_E_WORKSPACE";
    case KVQ_E_NODEVICE: return "KVQ_E_NODEVICE";
    case KVQ_E_HIP: return "KVQ_E_HIP";
    default: return "KVQ_E_UNKNOWN";
  }
}

}  // extern "C"
