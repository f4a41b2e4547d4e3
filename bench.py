"""Benchmark of the quantized KV-cache hot path on one MI355X.

Workload (default "long"): B=1, H=32 (MHA), D=128, S_kv=65536, 2-bit keys and values,
g=32, fp16 window of 32 tokens; seeded synthetic K/V (N(0,1), 8 outlier key channels x10).
A step is one decode step of the cache through kvq_append_decode_attend: one token per
sequence appended and one query per head attended, in one kernel launch (split-K, the last
split of each sequence and KV head merging the partials), except on the 1 step in 32 per
cache whose append flushes a full window through the quantizer (the append kernel runs
first). The same steps through the separate kvq_append + kvq_decode_attend calls are timed
too and reported as step_separate_calls_us.
Steps rotate over 4 cache replicas (4 x 202 MB) so the 256 MB Infinity Cache cannot hold
the working set. Inputs are resident in HBM before timing. Before the warmup steps, 0.5 s of
attend-only calls (which change no cache) let the GPU clocks settle, before the prefill
encode is timed and again before the warmup steps.

Printed: one JSON line with the step time, the decode kernel's achieved HBM bandwidth
against the 8 TB/s peak (algorithmic bytes / kernel time from HIP events that the decode
kernel's own dispatch stamps, on its stream), the prefill-encode rate, and the CPU oracle
timed on a bounded sample of the same workload.

With --n-sink N the caches keep N sink tokens per (sequence, KV head) in fp16 (KIVI-Sink,
"Changelog" v0.9.0): the prefill then also chooses them, and every decode attends them as one
more fp16 unit and skips their quantized slots. With --method skvq the caches are
SKVQ-adapted ("Changelog" v0.30.0: per-token groups of range-sorted channels, per-group clip
search, the first --n-sink tokens in fp16; window --window, the pages' defaults 128 and 5).

With --method kitty the caches are Kitty ("Changelog" v0.11.0: per key group, the
--kitty-hi-fraction of channels with the largest running variance at 4 bits, the rest at 2 bits;
values in fp16): the step is kvq_append then the Kitty decode kernel (split-K, merged in-kernel).

With --n-query N > 1 a step appends N tokens per sequence and then scores them with one causal
multi-query attend (kvq_decode_attend_multi: speculative decoding's verification step).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long] [--n-sink 0]
                  [--method kivi|skvq|kitty] [--window R] [--n-query 1] [--kitty-hi-fraction 0.25]
                  [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_FP16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak (no sparsity)

# HBM bytes per decode launch (KIVI, no sinks, default window and splits) from two rocprofv3 --pmc
# runs (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, factors from a 1 GiB device copy; see
# profiles/*_counters.md), valid only for the decode kernel and split-plan sources they were
# taken on (their hash over TRAFFIC_SOURCES).
MEASURED_TRAFFIC = {
    "long": {"src_sha256_16": "811827841dc9b543", "bytes": 202966744},
    "gqa": {"src_sha256_16": "811827841dc9b543", "bytes": 132473269},
    "full32": {"src_sha256_16": "811827841dc9b543", "bytes": 204043793},
}
TRAFFIC_SOURCES = ("decode_kernel.h", "decode.hip", "decode_mfma.hip", "kvq.cpp")


def cache_compression(wl, n_q, n_r):
    """Bytes per cached token and KV head (a 32-token record: codes and fp16 (scale, zero) per
    group), and the compression against fp16 keys and values, without and with the fp16 window."""
    D = wl.head_dim
    key = (32 * D * wl.key_bits // 8 + 4 * D) / 32  # codes + per-channel (scale, zero) of 32 tokens
    val = (32 * D * wl.value_bits // 8 + 4 * D) / 32  # codes + per-token (scale, zero) per 32 channels
    fp16 = 2 * D
    toks = sum(n_q) + sum(n_r)
    stored = sum(n_q) * (key + val) + sum(n_r) * 2 * fp16
    return {"bytes_per_token_key": key, "bytes_per_token_value": val,
            "key_vs_fp16": round(fp16 / key, 3), "kv_vs_fp16": round(2 * fp16 / (key + val), 3),
            "kv_vs_fp16_with_window": round(toks * 2 * fp16 / stored, 3),
            "pages": "KIVI-2bit: about 5.8x key, 4x full KV (Changelog v0.8.0)"}


def kitty_record_bytes(D, n_hi):
    """Algorithmic bytes of a Kitty record (32 tokens): 4-bit codes of n_hi channels and 2-bit
    codes of the rest, an fp16 (scale, zero) and a slot-table byte per channel, fp16 values."""
    return 32 * (4 * n_hi + 2 * (D - n_hi)) // 8 + 4 * D + D + 32 * D * 2


def algorithmic_decode_bytes(wl, n_q, n_r, n_sink=0, kitty_n_hi=None):
    """Bytes one decode launch must move: every record once per KV head (GQA query heads share
    it), the fp16 window and sink rows, q and out. n_q, n_r: per-sequence lengths."""
    D = wl.head_dim
    rec = 4 * D * (wl.key_bits + wl.value_bits + 2)  # per 32 quantized tokens
    if kitty_n_hi is not None:
        rec = kitty_record_bytes(D, kitty_n_hi)
    kv = sum((nq // 32) * rec + (nr + (n_sink if nq else 0)) * D * 2 * 2
             for nq, nr in zip(n_q, n_r)) * wl.n_kv_heads
    return kv + 2 * wl.batch * wl.n_q_heads * D * 2


def attend_flops(wl, n_q, n_r, n_query):
    """Useful flops of one causal multi-query attend: per query head and query j, a dot product
    and a weighted sum over its visible tokens (S - (n_query - 1 - j)), 2 flops per element each."""
    total = 0
    for b in range(wl.batch):
        S = n_q[b] + n_r[b]
        visible = sum(S - (n_query - 1 - j) for j in range(n_query))
        total += 4 * wl.head_dim * wl.n_q_heads * visible
    return total


def algorithmic_encode_bytes(wl, n_q_tokens, n_sink=0, kitty_n_hi=None):
    """Prefill encode: read fp16 K and V once, write codes and parameters once (and the sink rows)."""
    D = wl.head_dim
    rec = 4 * D * (wl.key_bits + wl.value_bits + 2)
    if kitty_n_hi is not None:
        rec = kitty_record_bytes(D, kitty_n_hi)
    return sum(nq * D * 2 * 2 + (nq // 32) * rec + (n_sink * D * 2 * 2 if nq else 0)
               for nq in n_q_tokens) * wl.n_kv_heads


def cpu_baseline(wl, draw, budget_s=12.0, n_sink=0, method="kivi", window=32, kitty_n_hi=0):
    """The oracle's decode (reconstruct K_hat/V_hat, fp64 softmax attention) on a sample of the
    KV heads of sequence 0, scaled by tokens to the whole step (every sequence, head and layer)."""
    import numpy as np  # noqa: F401

    from oracle import kitty, kivi, skvq

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t_dec = 0.0
    heads = 0
    t_enc = 0.0
    H = wl.n_kv_heads
    G = wl.n_q_heads // H
    S0 = draw.seq_lens[0]
    for h in range(H):
        if method == "skvq":
            s = skvq.SkvqSequence(wl.head_dim, wl.key_bits, wl.value_bits, 32, window, n_sink)
        elif method == "kitty":
            s = kitty.KittySequence(wl.head_dim, kitty_n_hi, 4, wl.key_bits, 32, window)
        else:
            s = kivi.KiviSequence(wl.head_dim, wl.key_bits, wl.value_bits, 32, window, n_sink)
        t0 = time.perf_counter()
        s.prefill(draw.K[0][h], draw.V[0][h])
        t1 = time.perf_counter()
        kh, vh = s.keys_hat(), s.values_hat()
        for hq in range(h * G, h * G + G):
            kivi.attend(draw.q[0, hq], kh, vh)
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        heads += 1
        if t_dec + t_enc > budget_s:
            break
    head_tokens = sum(draw.seq_lens) * H * wl.layers  # (KV head, token) pairs of one step
    scale = head_tokens / (heads * S0)
    return {
        "value": t_dec * scale * 1e6, "unit": "us/step (decode-attend)", "cores": int(threads), "kind": "oracle",
        "sample": f"{heads} of {H} KV heads of sequence 0 ({S0} tokens), scaled by tokens x{scale:g} to every "
                  f"sequence, head and layer; oracle decode = dequantize to fp64 + softmax attention; host "
                  f"os.cpu_count()={os.cpu_count()}",
        "encode_tokens_per_s": (heads * S0) / (t_enc * H) if t_enc else None,
    }


def device_record(torch):
    """What the run was measured on: the GPU's properties as HIP reports them, and the versions."""
    p = torch.cuda.get_device_properties(0)
    rec = {k: getattr(p, k) for k in ("name", "gcnArchName", "multi_processor_count", "total_memory",
                                      "L2_cache_size", "clock_rate", "memory_clock_rate", "memory_bus_width")
           if hasattr(p, k)}
    rec["hip"] = torch.version.hip
    rec["torch"] = torch.__version__
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--encode-reps", type=int, default=5)
    ap.add_argument("--n-split", type=int, default=0, help="splits per sequence (0 = the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=0.5, help="seconds of attend-only calls before the warmup")
    ap.add_argument("--n-sink", type=int, default=None,
                    help="sink tokens per (sequence, KV head): KIVI-Sink by key norm (default 0 = KIVI), SKVQ the first "
                         "tokens (default 5)")
    ap.add_argument("--method", default="kivi", choices=("kivi", "skvq", "kitty"))
    ap.add_argument("--kitty-hi-fraction", type=float, default=0.25, help="Kitty: key channels at 4 bits")
    ap.add_argument("--window", type=int, default=None, help="fp16 window (default: the workload's, 128 for skvq)")
    ap.add_argument("--n-query", type=int, default=1, help="queries per head per step (causal multi-query attend)")
    args = ap.parse_args()
    if args.n_sink is None:
        args.n_sink = 5 if args.method == "skvq" else 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path shards by "
              "(sequence, KV head) with no exchange, so N GPUs run N independent copies.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_decode_attention_encode_amd import (KVQCache, kvq_append, kvq_decode_attend, kvq_prefill,
                                                       make_config, workloads)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    wl = workloads.WORKLOADS[args.workload]
    R = args.window or (128 if args.method == "skvq" else wl.residual)
    # Single-layer workloads rotate over `replicas` copies of one cache (one cache per step);
    # the multi-layer workload keeps one cache per layer and a step visits every layer.
    multi = wl.layers > 1
    n_caches = wl.layers if multi else args.replicas
    draw = workloads.Draw(wl)  # multi-layer: layer 0's K/V fill every layer (costs do not depend on values)
    K, V, lens = draw.padded()
    # warmup, then three passes of `steps` steps each: the timed steps through the one call (no
    # instrumentation), the same through the two separate calls, and a pass through the one call
    # with the decode kernel's dispatch-stamped events on (the kernel's execution time; the
    # events themselves lengthen a step, so that pass is not the step time)
    n_steps_total = args.warmup + 3 * args.steps
    per_cache = n_steps_total if multi else (n_steps_total + n_caches - 1) // n_caches
    NQ = args.n_query
    cap = (max(lens) + per_cache * NQ + R + 64 + 31) // 32 * 32
    cfg = make_config(wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.key_bits, wl.value_bits, 32,
                      R, cap, n_sink=args.n_sink, method=args.method, kitty_hi_fraction=args.kitty_hi_fraction)
    kitty_n_hi = cfg.kitty_n_hi if args.method == "kitty" else None
    Kt, Vt = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    del K, V
    stream = torch.cuda.current_stream()

    # ---- every cache prefilled (the prefill encode rate is timed below, once the clocks settled)
    caches = [KVQCache(cfg, device=dev) for _ in range(n_caches)]
    for c in caches:
        kvq_prefill(c, Kt, Vt, lens)
    torch.cuda.synchronize()
    q = torch.from_numpy(draw.q).to(dev)
    outs = [torch.empty(tuple(q.shape), dtype=torch.float16, device=dev) for _ in caches]
    wss = [c.workspace(args.n_split) for c in caches]

    # Settle the GPU clocks first (they ramp up over the first ~0.1 s of sustained work, and a
    # kernel timed before that reads up to 10% slow): attend-only calls, which leave every
    # cache as it is, for at least `settle_s` seconds.
    def settle():
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle_s:
            for _ in range(20):
                for c, o, w in zip(caches, outs, wss):
                    kvq_decode_attend(c, q, out=o, workspace=w, n_split=args.n_split, stream=stream)
            torch.cuda.synchronize()

    settle()

    # ---- prefill encode rate (reset + prefill of cache 0, the prefill timed alone)
    enc_ms = []
    for r in range(args.encode_reps):
        c = caches[0]
        c.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq_prefill(c, Kt, Vt, lens)
        e1.record(stream)
        torch.cuda.synchronize()
        enc_ms.append(e0.elapsed_time(e1))
    enc_t = statistics.median(enc_ms) / 1e3
    n_q0, n_r0 = (list(x) for x in caches[0].lengths())
    enc_tokens_per_s = sum(lens) / enc_t
    enc_gbs = algorithmic_encode_bytes(wl, n_q0, args.n_sink, kitty_n_hi) / enc_t / 1e9

    # ---- device-resident inputs of the decode steps
    toks = [draw.next_token() for _ in range(n_steps_total * NQ)]
    kt = torch.from_numpy(np.stack([t[0] for t in toks])).to(dev)
    vt = torch.from_numpy(np.stack([t[1] for t in toks])).to(dev)
    del Kt, Vt
    torch.cuda.synchronize()

    # The timed loop makes exactly the C-ABI calls of a step, with every argument prepared
    # beforehand (the checked Python wrappers cost more host time than the GPU work of a step).
    from quantized_decode_attention_encode_amd import _lib
    import ctypes
    lib = _lib.lib
    sp = ctypes.c_void_p(stream.cuda_stream)
    kp = [ctypes.c_void_p(kt[i].data_ptr()) for i in range(n_steps_total * NQ)]
    vp = [ctypes.c_void_p(vt[i].data_ptr()) for i in range(n_steps_total * NQ)]
    dec_args = [(c.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(o.data_ptr()), 0, 1.0,
                 ctypes.c_void_p(w.data_ptr()), w.numel(), args.n_split, sp) for c, o, w in zip(caches, outs, wss)]
    visits = (lambda i: range(n_caches)) if multi else (lambda i: (i % n_caches,))

    fused_args = [(c.handle, None, None) + a[1:] for c, a in zip(caches, dec_args)]
    if NQ > 1:  # q [B, H_q, NQ, D] for the multi-query steps
        qm = torch.from_numpy((np.random.default_rng(wl.seed + 1000).standard_normal(
            (wl.batch, wl.n_q_heads, NQ, wl.head_dim)) / math.sqrt(wl.head_dim)).astype(np.float16)).to(dev)
        outm = [torch.empty(tuple(qm.shape), dtype=torch.float16, device=dev) for _ in caches]
        wsm = [c.workspace(args.n_split, NQ).clone() for c in caches]
        multi_args = [(c.handle, ctypes.c_void_p(qm.data_ptr()), ctypes.c_void_p(o.data_ptr()), NQ, 0, 1.0,
                       ctypes.c_void_p(w.data_ptr()), w.numel(), args.n_split, sp) for c, o, w in zip(caches, outm, wsm)]

    def step(i):  # one decode step of the hot path: append + attend, one call
        for r in visits(i):
            if NQ > 1:
                st = 0
                for k in range(NQ):
                    st = st or lib.kvq_append(caches[r].handle, kp[i * NQ + k], vp[i * NQ + k], sp)
                st = st or lib.kvq_decode_attend_multi(*multi_args[r])
            else:
                a = fused_args[r]
                st = lib.kvq_append_decode_attend(a[0], kp[i], vp[i], *a[3:])
            if st:
                _lib.check(st)

    def step_separate(i):  # the same step through kvq_append, then kvq_decode_attend
        if NQ > 1:
            return step(i)
        for r in visits(i):
            st = lib.kvq_append(caches[r].handle, kp[i], vp[i], sp)
            st = st or lib.kvq_decode_attend(*dec_args[r])
            if st:
                _lib.check(st)

    # lengths each decode sees, replayed from the window rule (one appended token per visit)
    lens_now = [c.lengths() for c in caches]
    settle()  # again: the host work since the prefill timing left the GPU idle
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_ev0, t_ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_ev0.record(stream)
    wall0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    t_ev1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    s_ev0, s_ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev0.record(stream)
    for i in range(args.warmup + args.steps, args.warmup + 2 * args.steps):
        step_separate(i)
    s_ev1.record(stream)
    torch.cuda.synchronize()
    step_sep_ms = s_ev0.elapsed_time(s_ev1) / args.steps
    for c in caches:
        c.profile_enable(True, launches=args.steps if multi else (args.steps + n_caches - 1) // n_caches)
    first, last = args.warmup + 2 * args.steps, n_steps_total  # the pass the roofline is taken over
    for i in range(first, last):
        step(i)
    torch.cuda.synchronize()
    bytes_per_launch, flops_per_launch = [], []
    for i in range(n_steps_total):
        for r in visits(i):
            nq, nr = lens_now[r]
            for _ in range(NQ):
                for b in range(wl.batch):
                    if nr[b] == R:
                        nq[b] += R
                        nr[b] = 0
                    nr[b] += 1
            if first <= i < last:  # (the extra queries add their q and out rows)
                bytes_per_launch.append(algorithmic_decode_bytes(wl, nq, nr, args.n_sink, kitty_n_hi)
                                        + (NQ - 1) * 2 * wl.batch * wl.n_q_heads * wl.head_dim * 2)
                flops_per_launch.append(attend_flops(wl, nq, nr, NQ))
    for r, c in enumerate(caches):
        assert tuple(map(list, lens_now[r])) == tuple(map(list, c.lengths())), "length replay disagrees"
    step_ms = t_ev0.elapsed_time(t_ev1) / args.steps
    split_ms, split_n = 0.0, 0
    for c in caches:
        ms, n = c.profile_read()
        c.profile_enable(False)
        split_ms += ms
        split_n += n
    split_avg_ms = split_ms / split_n
    alg_bytes = statistics.mean(bytes_per_launch)
    achieved = alg_bytes / (split_avg_ms / 1e3) / 1e9
    # more query rows per KV head than the decode kernel holds: the matrix-core kernel, whose
    # bound is its fp16 MFMA rate (useful flops; the fp16 high + low operands cost 2.5x that)
    G_rows = (wl.n_q_heads // wl.n_kv_heads) * NQ
    tiles = NQ > 1 and (G_rows > 8 or (NQ & (NQ - 1)))
    alg_flops = statistics.mean(flops_per_launch)
    tflops = alg_flops / (split_avg_ms / 1e3) / 1e12

    # ---- achievable HBM bandwidth for context: a plain device copy, 1 GiB each way
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b

    traffic = None
    csrc = os.path.join(ROOT, "quantized_decode_attention_encode_amd", "csrc")
    measured = MEASURED_TRAFFIC.get(args.workload)
    if (measured and args.n_split == 0 and args.n_sink == 0 and args.method == "kivi" and R == wl.residual
            and NQ == 1):
        import hashlib

        h = hashlib.sha256()
        for name in TRAFFIC_SOURCES:  # the decode kernels and the host's split plan
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] == measured["src_sha256_16"]:
            traffic = measured["bytes"]
    G = wl.n_q_heads // wl.n_kv_heads
    if kitty_n_hi is not None:
        decode_kernel = "kitty_decode_kernel"
    elif args.method == "kivi" and args.n_sink == 0 and G * NQ in (4, 8):
        decode_kernel = "decode_mfma_kernel"
    else:
        decode_kernel = "decode_split_kernel"

    result = {
        "metric": "decode-attend us/step + achieved HBM GB/s (% peak) at S_kv=64K; encode tokens/s",
        "value": round(step_ms * 1e3, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.describe()}",
            "step": ("every layer: " if multi else "")
            + ("kvq_append_decode_attend (Kitty: the append kernel, then the decode kernel; the "
               "1 step in 32 that flushes a full window runs the Kitty encode launches first)"
               if kitty_n_hi is not None else
               "kvq_append_decode_attend (append + attend in one decode kernel; on the 1 step in 32 that "
               "flushes a full window, the append kernel runs first)" if NQ == 1 else
               f"{NQ} x kvq_append, then kvq_decode_attend_multi over the {NQ} new tokens (causal)"),
            "caches": f"{n_caches} layer caches" if multi else f"{n_caches} replicas of one cache, one per step",
            "codes": (f"{wl.key_bits}-bit keys / {wl.value_bits}-bit values, fp16 (scale, zero), fp32 softmax"
                      if kitty_n_hi is None else
                      f"{kitty_n_hi} of {wl.head_dim} key channels at 4 bits (running variance), the rest at "
                      f"{wl.key_bits} bits, fp16 (scale, zero); fp16 values; fp32 softmax"),
            "sinks": args.n_sink,
            "method": args.method,
            "window": R,
            "n_query": NQ,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": decode_kernel,
            "kernel_avg_us": round(split_avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(alg_bytes),
        } if not tiles else {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_FP16_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_FP16_MFMA_TFLOPS, 4),
            "traffic": None,
            "kernel": "attend_tiles_kernel (+ tiles_merge_kernel when split)",
            "kernel_avg_us": round(split_avg_ms * 1e3, 3),
            "algorithmic_flops_per_launch": int(alg_flops),
            "hbm": {"achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": int(alg_bytes)},
        },
        "cache_compression": (cache_compression(wl, n_q0, n_r0) if kitty_n_hi is None and args.method == "kivi"
                              else None),
        "decode_split_us": round(split_avg_ms * 1e3, 3),
        "decode_gbps": round(achieved, 1),
        "decode_frac_of_copy_bw": round(achieved / copy_gbs, 4),
        "copy_gbps_measured": round(copy_gbs, 1),
        "encode_tokens_per_s": round(enc_tokens_per_s, 1),
        "encode_gbps": round(enc_gbs, 1),
        "encode_prefill_us": round(enc_t * 1e6, 2),
        "wall_s_timed": round(wall1 - wall0, 3),
        "step_separate_calls_us": round(step_sep_ms * 1e3, 3),
        "device": device_record(torch),
    }
    if multi:
        result["encode_all_layers_us"] = round(enc_t * 1e6 * wl.layers, 1)
        result["decode_launches_per_step"] = wl.layers
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, draw, n_sink=args.n_sink, method=args.method, window=R,
                                              kitty_n_hi=kitty_n_hi or 0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
