"""GPU parity for sink tokens ("Changelog" v0.9.0, KIVI-Sink) through the C ABI.

The cache state (records with the sinks left out of their key groups and marked in their
value scales, sink positions and fp16 rows) must equal the oracle's bit for bit after
prefill, encode and appends across the first flush; attention must be within the tolerance
of the fp64 oracle for every split count, with and without the fused append. A few tokens
of every (sequence, KV head) get keys scaled by 6 so that the sinks are real outliers.
"""
import numpy as np
import pytest
import torch

from oracle import kivi
from quantized_decode_attention_encode_amd import (KVQCache, kvq_append, kvq_append_decode_attend,
                                                   kvq_decode_attend, kvq_encode, kvq_prefill, make_config,
                                                   workloads)
from tests.gpu_helpers import assert_close, assert_state_equal, host_buffer, oracle_attend, oracle_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Hq, Hkv, D, bk, bv, ragged lengths, n_sink
    ("d128-b22-s5", 3, 4, 4, 128, 2, 2, (1, 400), 5),
    ("d64-b22-s1", 2, 4, 4, 64, 2, 2, (33, 300), 1),
    ("d128-b24-gqa4-s16", 2, 8, 2, 128, 2, 4, (1, 500), 16),
    ("d64-b48-gqa2-s3", 2, 4, 2, 64, 4, 8, (1, 260), 3),
    ("d128-b88-gqa8-s7", 2, 8, 1, 128, 8, 8, (40, 300), 7),
]


def plant(draw, seed, n=4):
    """Scale the keys of n random tokens of every (b, h) by 6 (in fp16)."""
    rng = np.random.default_rng(seed)
    for b, Kb in enumerate(draw.K):
        for h in range(Kb.shape[0]):
            S = Kb.shape[1]
            if S:
                t = rng.choice(S, min(n, S), replace=False)
                Kb[h, t] = (Kb[h, t].astype(np.float32) * 6).astype(np.float16)


def make(case, seed=21, seq_lens=None, max_tokens=1024):
    name, B, Hq, Hkv, D, bk, bv, rag, ns = case
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=bk, value_bits=bv,
                          n_outlier=2, seed=seed, ragged=rag)
    draw = workloads.Draw(wl, seq_lens=seq_lens)
    plant(draw, seed + 1000)
    cfg = make_config(B, Hkv, Hq, D, bk, bv, 32, 32, max_tokens, n_sink=ns)
    return wl, draw, cfg


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sink_prefill_state_and_decode(case):
    wl, draw, cfg = make(case)
    say("case", case, "lens", draw.seq_lens)
    cache = KVQCache(cfg, device=DEV)
    K, V, lens = draw.padded()
    kvq_prefill(cache, torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), lens)
    torch.cuda.synchronize()
    seqs = oracle_prefill(draw, 32, n_sink=cfg.n_sink)
    assert_state_equal(host_buffer(cache), cfg, seqs, case[0])
    assert any(s.sink_pos.size for s in seqs.values())
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    q = torch.from_numpy(draw.q).to(DEV)
    for n_split in (0, 1, 3, 50):
        out = kvq_decode_attend(cache, q, out_fp32=True, n_split=n_split)
        err = assert_close(out.cpu().numpy(), ref, f"{case[0]} n_split={n_split}")
        say("  n_split", n_split, "err", err)


def test_sink_encode_chooses_once():
    # two encode calls: the first chooses the sinks among its tokens, the second leaves them
    case = CASES[0]
    wl, draw, cfg = make(case, seed=22, seq_lens=[192, 128, 64])
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    cache = KVQCache(cfg, device=DEV)
    first = [64, 64, 32]
    kvq_encode(cache, Kt, Vt, first)
    rest = [192 - 64, 128 - 64, 64 - 32]
    Kr = torch.stack([Kt[b, :, first[b]:first[b] + 128] for b in range(3)]).contiguous()
    Vr = torch.stack([Vt[b, :, first[b]:first[b] + 128] for b in range(3)]).contiguous()
    kvq_encode(cache, Kr, Vr, rest)
    torch.cuda.synchronize()
    seqs = {}
    for b in range(3):
        for h in range(wl.n_kv_heads):
            s = kivi.KiviSequence(wl.head_dim, wl.key_bits, wl.value_bits, 32, 32, cfg.n_sink)
            s.encode(draw.K[b][h][:first[b]], draw.V[b][h][:first[b]])
            s.encode(draw.K[b][h][first[b]:first[b] + rest[b]], draw.V[b][h][first[b]:first[b] + rest[b]])
            seqs[(b, h)] = s
            assert np.all(s.sink_pos < first[b])
    assert_state_equal(host_buffer(cache), cfg, seqs, "encode twice")
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    out = kvq_decode_attend(cache, torch.from_numpy(draw.q).to(DEV), out_fp32=True)
    assert_close(out.cpu().numpy(), ref, "encode twice")


@pytest.mark.parametrize("fused", [False, True])
def test_sinks_chosen_by_the_first_flush(fused):
    # sequences that grow by appends only: the first window flush chooses the sinks among the
    # R flushed tokens; a sequence already past it keeps its prefill sinks
    case = CASES[3]
    n_steps = 75
    lens0 = [5, 100]  # sequence 0 flushes first at step 27; sequence 1 has prefill sinks
    wl, draw, cfg = make(case, seed=23, seq_lens=[lens0[0] + n_steps, lens0[1] + n_steps])
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    cache = KVQCache(cfg, device=DEV)
    kvq_prefill(cache, Kt, Vt, lens0)
    seqs = {}
    for b in range(2):
        for h in range(wl.n_kv_heads):
            s = kivi.KiviSequence(wl.head_dim, wl.key_bits, wl.value_bits, 32, 32, cfg.n_sink)
            s.prefill(draw.K[b][h][:lens0[b]], draw.V[b][h][:lens0[b]])
            seqs[(b, h)] = s
    q = torch.from_numpy(draw.q).to(DEV)
    for t in range(n_steps):
        k = torch.stack([Kt[b, :, lens0[b] + t] for b in range(2)]).contiguous()
        v = torch.stack([Vt[b, :, lens0[b] + t] for b in range(2)]).contiguous()
        for b in range(2):
            for h in range(wl.n_kv_heads):
                seqs[(b, h)].append(draw.K[b][h][lens0[b] + t], draw.V[b][h][lens0[b] + t])
        if fused:
            out = kvq_append_decode_attend(cache, k, v, q, out_fp32=True, n_split=2)
        else:
            kvq_append(cache, k, v)
            out = kvq_decode_attend(cache, q, out_fp32=True, n_split=2)
        if t % 9 == 0 or t == n_steps - 1:
            torch.cuda.synchronize()
            assert_state_equal(host_buffer(cache), cfg, seqs, f"step {t}")
            ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
            assert_close(out.cpu().numpy(), ref, f"step {t}")
    assert seqs[(0, 0)].sink_pos.size == cfg.n_sink and np.all(seqs[(0, 0)].sink_pos < 32)


# ---------------------------------------------------------------------------------------------
# Long prefills: the sink choice runs over several 2048-token chunks whose candidate lists are
# merged, so the winners can come from any chunk and ties can straddle a chunk boundary.
TIE = (2047, 2048, 4095, 4096)  # one identical key row: an exact norm tie across two boundaries

MULTI = [
    # name, B, Hq, Hkv, D, bk, bv, sequence lengths, n_sink
    ("d128-b22-s1", 3, 4, 4, 128, 2, 2, (5000, 9000, 6150), 1),
    ("d64-b24-gqa2-s5", 3, 4, 2, 64, 2, 4, (8999, 5031, 7000), 5),
    ("d128-b44-gqa4-s16", 2, 8, 2, 128, 4, 4, (6400, 9000), 16),
]


def plant_multichunk(draw, n_sink, seed):
    """Per (b, h): n_sink - 1 keys of distinct, large norms at random positions of the quantized
    part (spread over its chunks), and the TIE tokens sharing one key row whose norm ranks just
    below them; so the sinks are those n_sink - 1 tokens and token 2047, the earliest of the tie.
    Returns the expected sink positions per (b, h)."""
    rng = np.random.default_rng(seed)
    D, R = draw.wl.head_dim, draw.wl.residual
    expect = {}
    for b, Kb in enumerate(draw.K):
        n_q, _ = kivi.window_split(Kb.shape[1], R)
        assert n_q > max(TIE)
        for h in range(Kb.shape[0]):
            u = rng.standard_normal(D, np.float32).astype(np.float16)
            tie = (u.astype(np.float32) * 8).astype(np.float16)  # a power of two: exact, norm 64 |u|^2
            for t in TIE:
                Kb[h, t] = tie
            top = rng.choice(np.setdiff1d(np.arange(n_q), TIE), n_sink - 1, replace=False)
            for t in top:  # norms ~ 256 * chi2(128): far above the tie, distinct from each other
                Kb[h, t] = (rng.standard_normal(D, np.float32) * 16).astype(np.float16)
            expect[(b, h)] = sorted(int(t) for t in top) + [2047]
            expect[(b, h)].sort()
    return expect


@pytest.mark.parametrize("start", ["prefill", "encode"])
@pytest.mark.parametrize("case", MULTI, ids=[c[0] for c in MULTI])
def test_sink_choice_over_many_chunks(case, start):
    name, B, Hq, Hkv, D, bk, bv, lens, ns = case
    if start == "encode":  # kvq_encode takes whole groups and leaves the window empty
        lens = tuple(s // 32 * 32 for s in lens)
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=bk, value_bits=bv,
                          n_outlier=2, seed=70 + ns, ragged=(1, 2))
    draw = workloads.Draw(wl, seq_lens=list(lens))
    expect = plant_multichunk(draw, ns, 80 + ns)
    say("case", name, start, "lens", draw.seq_lens)
    cfg = make_config(B, Hkv, Hq, D, bk, bv, 32, 32, 9216, n_sink=ns)
    cache = KVQCache(cfg, device=DEV)
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    if start == "prefill":
        kvq_prefill(cache, Kt, Vt, list(lens))
    else:
        kvq_encode(cache, Kt, Vt, list(lens))
    torch.cuda.synchronize()
    seqs = {}
    for b in range(B):
        for h in range(Hkv):
            s = kivi.KiviSequence(D, bk, bv, 32, 32, ns)
            (s.prefill if start == "prefill" else s.encode)(draw.K[b][h], draw.V[b][h])
            assert s.sink_pos.tolist() == expect[(b, h)], (b, h)  # the oracle picks the planted ones
            seqs[(b, h)] = s
    assert_state_equal(host_buffer(cache), cfg, seqs, f"{name} {start}")
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    q = torch.from_numpy(draw.q).to(DEV)
    for n_split in (0, 5):
        out = kvq_decode_attend(cache, q, out_fp32=True, n_split=n_split)
        err = assert_close(out.cpu().numpy(), ref, f"{name} {start} n_split={n_split}")
        say("  n_split", n_split, "err", err)
    # appends across a window flush keep the sinks, fused with the decode
    for t in range(40):
        k, v = draw.next_token()
        kt, vt = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
        for (b, h), s in seqs.items():
            s.append(k[b, h], v[b, h])
        out = kvq_append_decode_attend(cache, kt, vt, q, out_fp32=True)
    torch.cuda.synchronize()
    assert_state_equal(host_buffer(cache), cfg, seqs, f"{name} {start} appended")
    assert_close(out.cpu().numpy(), oracle_attend(draw.q.astype(np.float64), seqs, wl), f"{name} {start} appended")


def test_long_workload_with_five_sinks():
    # the bench's sink configuration at full size (65504 quantized tokens: 32 chunks per head),
    # bit-exact state and attention on sampled heads
    wl = workloads.WORKLOADS["long"]
    say(f"long with 5 sinks: {wl.describe()}")
    draw = workloads.Draw(wl)
    cfg = make_config(wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.key_bits, wl.value_bits, 32,
                      wl.residual, 65536, n_sink=5)
    cache = KVQCache(cfg, device=DEV)
    K, V, lens = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    del K, V
    kvq_prefill(cache, Kt, Vt, lens)
    out = kvq_decode_attend(cache, torch.from_numpy(draw.q).to(DEV)).float().cpu().numpy()
    buf = host_buffer(cache)
    del Kt, Vt
    pairs = {(0, 0), (0, 17), (0, 31)}
    seqs = oracle_prefill(draw, wl.residual, pairs=pairs, n_sink=5)
    chunks = {(b, h): sorted({int(p) // 2048 for p in s.sink_pos}) for (b, h), s in seqs.items()}
    say("  sink chunks per sampled head", chunks)
    assert_state_equal(buf, cfg, seqs, "long n_sink=5")
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl, heads=pairs)
    err = assert_close(out, ref, "long n_sink=5")
    say("  long n_sink=5: attention max abs / row rel", err)
