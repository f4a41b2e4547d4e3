"""GPU parity for Kitty caches ("Changelog" v0.11.0, Kitty) through the C ABI.

The cache state (per key group the high-width channel set, the 4- and 2-bit codes and their
fp16 (scale, zero), the fp16 values, the window and the exact running key sums) must equal the
oracle's bit for bit after prefill, after encode calls and after appends across window flushes;
attention must be within the tolerance of the fp64 oracle for several split counts. Cases cover
D = 64 and 128, no / a quarter / half / all channels at 4 bits, query-head groups 1..8, empty,
one-token and window-only sequences.
"""
import numpy as np
import pytest
import torch

from oracle import kitty
from quantized_decode_attention_encode_amd import (KVQCache, kvq_append, kvq_append_decode_attend, kvq_decode_attend,
                                                   kvq_encode, kvq_prefill, make_config, workloads)
from tests import kvq_unpack
from tests.gpu_helpers import assert_close, host_buffer, oracle_attend, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Hq, Hkv, D, hi_fraction, lengths, R
    ("d128-quarter-mha", 2, 4, 4, 128, 0.25, [700, 133], 32),
    ("d64-quarter-gqa2", 3, 4, 2, 64, 0.25, [300, 1, 36], 32),
    ("d128-none-gqa4-R64", 2, 8, 2, 128, 0.0, [400, 64], 64),
    ("d128-all-gqa8", 2, 8, 1, 128, 1.0, [330, 90], 32),
    ("d128-half-R64", 2, 2, 2, 128, 0.5, [250, 17], 64),
    ("d64-quarter-gqa8-R128", 2, 8, 1, 64, 0.25, [500, 140], 128),
    ("d128-eighth-gqa2-long", 1, 2, 1, 128, 0.125, [1000], 32),
]


def make(case, seed=41, lens=None):
    name, B, Hq, Hkv, D, frac, lengths, R = case
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=2, value_bits=2,
                          n_outlier=3, seed=seed, residual=R, ragged=(1, 2))
    draw = workloads.Draw(wl, seq_lens=lens if lens is not None else lengths)
    cfg = make_config(B, Hkv, Hq, D, 2, 16, 32, R, 1024, method="kitty", kitty_hi_fraction=frac)
    return wl, draw, cfg


def oracle_seq(wl, cfg):
    return kitty.KittySequence(wl.head_dim, cfg.kitty_n_hi, 4, 2, 32, cfg.residual)


def assert_kitty_state(buf, cfg, seqs, what=""):
    cd = {"B": cfg.batch, "Hkv": cfg.n_kv_heads, "D": cfg.head_dim, "R": cfg.residual, "max_tokens": cfg.max_tokens,
          "n_hi": cfg.kitty_n_hi}
    for (b, h), s in seqs.items():
        got = kvq_unpack.unpack_kitty_sequence(buf, cd, b, h)
        assert (got["n_q"], got["n_r"]) == (s.n_q, s.n_r), f"{what} lengths of {(b, h)}"
        for name, ref in (("kc", s.kc), ("ks", s.ks), ("kz", s.kz), ("khi", s.khi), ("vq", s.vq), ("wk", s.wk),
                          ("wv", s.wv)):
            g = got[name]
            assert g.shape == ref.shape, f"{what} {name} shape {g.shape} vs {ref.shape} at {(b, h)}"
            if not np.array_equal(g.view(np.uint8), ref.view(np.uint8)):
                bad = np.argwhere(g.view(np.uint8).reshape(g.shape[0], -1) != ref.view(np.uint8).reshape(ref.shape[0], -1))
                raise AssertionError(f"{what} {name} differs at {(b, h)}: first mismatches {bad[:5].tolist()}")
        if s.n_q:  # the running sums exist once a group is quantized
            assert got["s1"] == s.mom.s1 and got["s2"] == s.mom.s2, f"{what} running sums of {(b, h)}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kitty_prefill_state_and_decode(case):
    wl, draw, cfg = make(case)
    say("case", case[0], "lens", draw.seq_lens, "n_hi", cfg.kitty_n_hi)
    cache = KVQCache(cfg, device=DEV)
    K, V, lens = draw.padded()
    kvq_prefill(cache, torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), lens)
    torch.cuda.synchronize()
    seqs = {}
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            s = oracle_seq(wl, cfg)
            s.prefill(draw.K[b][h], draw.V[b][h])
            seqs[(b, h)] = s
    assert_kitty_state(host_buffer(cache), cfg, seqs, case[0])
    if 0 < cfg.kitty_n_hi < cfg.head_dim:  # the ranking moves between groups on this data
        assert any(len({tuple(r) for r in s.khi}) > 1 for s in seqs.values() if s.n_q > 32)
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    q = torch.from_numpy(draw.q).to(DEV)
    for n_split in (0, 1, 3, 40):
        out = kvq_decode_attend(cache, q, out_fp32=True, n_split=n_split)
        err = assert_close(out.cpu().numpy(), ref, f"{case[0]} n_split={n_split}")
        say("  n_split", n_split, "err", err)
    out16 = kvq_decode_attend(cache, q).float().cpu().numpy()  # fp16 output
    assert_close(out16, ref, f"{case[0]} fp16 out")


@pytest.mark.parametrize("fused", [False, True])
def test_kitty_appends_through_flushes(fused):
    case = CASES[1]
    n_steps = 80
    lens0 = [0, 5, 40]  # empty, window only, a group and a window
    wl, draw, cfg = make(case, seed=42, lens=[s + n_steps for s in lens0])
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    cache = KVQCache(cfg, device=DEV)
    kvq_prefill(cache, Kt, Vt, lens0)
    seqs = {}
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            s = oracle_seq(wl, cfg)
            s.prefill(draw.K[b][h][:lens0[b]], draw.V[b][h][:lens0[b]])
            seqs[(b, h)] = s
    q = torch.from_numpy(draw.q).to(DEV)
    for t in range(n_steps):
        k = torch.stack([Kt[b, :, lens0[b] + t] for b in range(wl.batch)]).contiguous()
        v = torch.stack([Vt[b, :, lens0[b] + t] for b in range(wl.batch)]).contiguous()
        for b in range(wl.batch):
            for h in range(wl.n_kv_heads):
                seqs[(b, h)].append(draw.K[b][h][lens0[b] + t], draw.V[b][h][lens0[b] + t])
        if fused:
            out = kvq_append_decode_attend(cache, k, v, q, out_fp32=True, n_split=2)
        else:
            kvq_append(cache, k, v)
            out = kvq_decode_attend(cache, q, out_fp32=True, n_split=2)
        if t % 11 == 0 or t == n_steps - 1:
            torch.cuda.synchronize()
            assert_kitty_state(host_buffer(cache), cfg, seqs, f"step {t}")
            ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
            assert_close(out.cpu().numpy(), ref, f"step {t}")


def test_kitty_flush_of_a_long_window():
    case = CASES[5]  # R = 128: each flush quantizes 4 groups, each ranked with its own sums
    n_steps = 140
    lens0 = [130, 3]
    wl, draw, cfg = make(case, seed=45, lens=[s + n_steps for s in lens0])
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    cache = KVQCache(cfg, device=DEV)
    kvq_prefill(cache, Kt, Vt, lens0)
    seqs = {}
    for b in range(wl.batch):
        s = oracle_seq(wl, cfg)
        s.prefill(draw.K[b][0][:lens0[b]], draw.V[b][0][:lens0[b]])
        seqs[(b, 0)] = s
    q = torch.from_numpy(draw.q).to(DEV)
    for t in range(n_steps):
        k = torch.stack([Kt[b, :, lens0[b] + t] for b in range(wl.batch)]).contiguous()
        v = torch.stack([Vt[b, :, lens0[b] + t] for b in range(wl.batch)]).contiguous()
        for b in range(wl.batch):
            seqs[(b, 0)].append(draw.K[b][0][lens0[b] + t], draw.V[b][0][lens0[b] + t])
        kvq_append(cache, k, v)
    torch.cuda.synchronize()
    assert seqs[(0, 0)].n_q == 256 and seqs[(1, 0)].n_q == 128  # flushes happened
    assert_kitty_state(host_buffer(cache), cfg, seqs, "after the flushes")
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    out = kvq_decode_attend(cache, q, out_fp32=True, n_split=3)
    assert_close(out.cpu().numpy(), ref, "after the flushes")


def test_kitty_prefill_equals_appends_on_the_device():
    case = CASES[0]
    wl, draw, cfg = make(case, seed=43, lens=[200, 131])
    K, V, lens = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    a = KVQCache(cfg, device=DEV)
    kvq_prefill(a, Kt, Vt, lens)
    b_ = KVQCache(cfg, device=DEV)
    lens0 = [70, 33]
    kvq_prefill(b_, Kt, Vt, lens0)
    for t in range(max(x - y for x, y in zip(lens, lens0))):
        # both sequences take the same number of appends here: pad the shorter one's source
        k = torch.stack([Kt[b, :, min(lens0[b] + t, Kt.shape[2] - 1)] for b in range(2)]).contiguous()
        v = torch.stack([Vt[b, :, min(lens0[b] + t, Vt.shape[2] - 1)] for b in range(2)]).contiguous()
        kvq_append(b_, k, v)
    torch.cuda.synchronize()
    cd = {"B": 2, "Hkv": wl.n_kv_heads, "D": wl.head_dim, "R": cfg.residual, "max_tokens": cfg.max_tokens,
          "n_hi": cfg.kitty_n_hi}
    ba, bb = host_buffer(a), host_buffer(b_)
    # sequence 0 took exactly 130 appends (200 - 70), the same tokens as the prefill
    for h in range(wl.n_kv_heads):
        x = kvq_unpack.unpack_kitty_sequence(ba, cd, 0, h)
        y = kvq_unpack.unpack_kitty_sequence(bb, cd, 0, h)
        for name in ("kc", "ks", "kz", "khi", "vq", "wk", "wv"):
            assert np.array_equal(x[name].view(np.uint8), y[name].view(np.uint8)), (name, h)
        assert x["s1"] == y["s1"] and x["s2"] == y["s2"]


def test_kitty_encode_calls():
    case = CASES[3]
    wl, draw, cfg = make(case, seed=44, lens=[160, 160])
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    cache = KVQCache(cfg, device=DEV)
    kvq_encode(cache, Kt[:, :, :64].contiguous(), Vt[:, :, :64].contiguous(), [64, 32])
    kvq_encode(cache, Kt[:, :, 64:160].contiguous(), Vt[:, :, 64:160].contiguous(), [96, 64])
    torch.cuda.synchronize()
    seqs = {}
    for b, (n0, n1) in enumerate([(64, 96), (32, 64)]):
        for h in range(wl.n_kv_heads):
            s = oracle_seq(wl, cfg)
            s.encode(draw.K[b][h][:n0], draw.V[b][h][:n0])
            s.encode(draw.K[b][h][64:64 + n1], draw.V[b][h][64:64 + n1])
            seqs[(b, h)] = s
    assert_kitty_state(host_buffer(cache), cfg, seqs, "encode")
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    out = kvq_decode_attend(cache, torch.from_numpy(draw.q).to(DEV), out_fp32=True)
    assert_close(out.cpu().numpy(), ref, "after encode")


def test_kitty_ranking_ties_on_the_device():
    """Spreads that tie exactly at the top-n_hi boundary (copies of a channel, and a copy
    shifted by an exactly representable constant; 17 constant channels) are decided by the
    lower channel index (equal fp32 images, then the exact 128-bit comparison and the index), and
    a near-tie (one value moved by 2^-6) by the spreads, on the device as in the oracle."""
    D, R, T = 128, 32, 244
    sign = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)
    K = np.zeros((T, D))
    for d in range(D):
        K[:, d] = sign * (1.0 + d / 256.0)  # small distinct spreads
    for d in range(98, 128):
        K[:, d] = sign * (10.0 + d - 98)  # the 30 largest spreads
    for d in (5, 9, 50):
        K[:, d] = sign * 5.0  # tied for ranks 32..35 with channel 70
    K[:, 70] = sign * 5.0 + 8.0  # the same values shifted: the same spread, exactly
    K[:, 7] = sign * 5.0
    K[3, 7] += 2.0 ** -6  # a near-tie just below them (token 3 holds -5: its magnitude shrinks)
    const = [0, 1, 2, 3, 4, 6, 8, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19]
    K[:, const] = 0.75  # spread 0: 17 channels tied at the bottom
    K = K.astype(np.float16)
    rng = np.random.default_rng(46)
    V = rng.standard_normal((T, D)).astype(np.float16)
    expect = {0.25: [5, 9] + list(range(98, 128)), 0.875: None}  # 5 and 9: the lower indices of the tie
    for frac in (0.25, 0.875):
        cfg = make_config(1, 1, 1, D, 2, 16, 32, R, 1024, method="kitty", kitty_hi_fraction=frac)
        cache = KVQCache(cfg, device=DEV)
        kvq_prefill(cache, torch.from_numpy(K[None, None]).to(DEV), torch.from_numpy(V[None, None]).to(DEV), [T])
        torch.cuda.synchronize()
        s = kitty.KittySequence(D, cfg.kitty_n_hi, 4, 2, 32, R)
        s.prefill(K, V)
        if expect[frac] is not None:
            assert all(np.flatnonzero(r).tolist() == expect[frac] for r in s.khi)
        else:  # every channel but 16 of the constants: the lowest-index constant gets in
            assert all(r[0] and not r[1:20][[c - 1 for c in const[1:]]].any() for r in s.khi)
        assert_kitty_state(host_buffer(cache), cfg, {(0, 0): s}, f"ties, fraction {frac}")


@pytest.mark.parametrize("name,pairs", [("long", {(0, 0), (0, 13), (0, 31)}), ("gqa", {(0, 0), (5, 3), (15, 7)})])
def test_kitty_full_size(name, pairs):
    """The long (64K tokens, 32 heads) and ragged GQA-batch workloads as Kitty caches, in the
    launch configuration bench.py times (automatic split count, fp16 output): sampled (b, h)
    pairs bit-exact against the oracle and their query heads' outputs within tolerance."""
    wl = workloads.WORKLOADS[name]
    draw = workloads.Draw(wl)
    cap = (max(draw.seq_lens) + 31) // 32 * 32
    cfg = make_config(wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.key_bits, 16, 32, wl.residual, cap,
                      method="kitty", kitty_hi_fraction=0.25)
    say(f"kitty {name}: {wl.describe()}, n_hi {cfg.kitty_n_hi}")
    cache = KVQCache(cfg, device=DEV)
    K, V, lens = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    del K, V
    kvq_prefill(cache, Kt, Vt, lens)
    out = kvq_decode_attend(cache, torch.from_numpy(draw.q).to(DEV)).float().cpu().numpy()
    buf = host_buffer(cache)
    del Kt, Vt
    seqs = {}
    for (b, h) in pairs:
        s = oracle_seq(wl, cfg)
        s.prefill(draw.K[b][h], draw.V[b][h])
        seqs[(b, h)] = s
    assert_kitty_state(buf, cfg, seqs, name)
    G = wl.n_q_heads // wl.n_kv_heads
    heads = {(b, hq) for (b, h) in pairs for hq in range(G * h, G * h + G)}
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl, heads=heads)
    err = assert_close(out, ref, f"kitty {name}")
    say(f"  kitty {name}: state bit-exact on {len(pairs)} (b, h); attention max abs {err[0]:.2e}")
