"""GPU parity for SKVQ-adapted caches ("Changelog" v0.30.0) through the C ABI.

The cache state (records with per-token groups of permuted channels and the clip search's
parameters, the channel permutations, the first-token sinks and the window) must equal the
oracle's bit for bit after prefill and after appends across the sinks and the first flush;
attention must be within the tolerance of the fp64 oracle for every split count, with and
without the fused append. Lengths include sequences that are all sinks, and all window.
"""
import numpy as np
import pytest
import torch

from oracle import skvq
from quantized_decode_attention_encode_amd import (KVQCache, kvq_append, kvq_append_decode_attend,
                                                   kvq_decode_attend, kvq_prefill, make_config, workloads)
from tests.gpu_helpers import assert_close, assert_state_equal, host_buffer, oracle_attend, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Hq, Hkv, D, bk, bv, lengths, R, n_sink, reorder, search, alpha
    ("d128-b22-R128-s5", 4, 4, 4, 128, 2, 2, [700, 133, 3, 140], 128, 5, True, True, 1.0),
    ("d64-b42-R32-s3-gqa2", 3, 4, 2, 64, 4, 2, [300, 1, 36], 32, 3, True, True, 1.0),
    ("d128-b24-R64-s0-gqa4", 2, 8, 2, 128, 2, 4, [400, 64], 64, 0, True, True, 1.0),
    ("d128-b88-R32-s16-fixed", 2, 2, 2, 128, 8, 8, [250, 17], 32, 16, False, False, 0.8),
    ("d64-b28-R64-s5-gqa8", 2, 8, 1, 64, 2, 8, [330, 90], 64, 5, True, True, 1.0),
]


def make(case, seed=31, lens=None):
    name, B, Hq, Hkv, D, bk, bv, lengths, R, ns, reorder, search, alpha = case
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=bk, value_bits=bv,
                          n_outlier=3, seed=seed, residual=R, ragged=(1, 2))
    draw = workloads.Draw(wl, seq_lens=lens if lens is not None else lengths)
    cfg = make_config(B, Hkv, Hq, D, bk, bv, 32, R, 1024, n_sink=ns, method="skvq", skvq_reorder=reorder,
                      skvq_clip_search=search, skvq_clip_alpha=alpha)
    return wl, draw, cfg


def oracle_seq(wl, cfg):
    return skvq.SkvqSequence(wl.head_dim, wl.key_bits, wl.value_bits, 32, cfg.residual, cfg.n_sink,
                             bool(cfg.skvq_reorder), bool(cfg.skvq_clip_search), cfg.skvq_clip_alpha)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_skvq_prefill_state_and_decode(case):
    wl, draw, cfg = make(case)
    say("case", case[0], "lens", draw.seq_lens)
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
    assert_state_equal(host_buffer(cache), cfg, seqs, case[0])
    if cfg.skvq_clip_search:
        assert any((s.kk > 0).any() for s in seqs.values() if s.n_q)  # the search clipped something
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
    q = torch.from_numpy(draw.q).to(DEV)
    for n_split in (0, 1, 3, 40):
        out = kvq_decode_attend(cache, q, out_fp32=True, n_split=n_split)
        err = assert_close(out.cpu().numpy(), ref, f"{case[0]} n_split={n_split}")
        say("  n_split", n_split, "err", err)


@pytest.mark.parametrize("fused", [False, True])
def test_skvq_appends_through_sinks_and_flushes(fused):
    case = CASES[1]
    n_steps = 80
    lens0 = [0, 2, 40]  # empty, inside the sinks, past the sinks
    wl, draw, cfg = make(case, seed=32, lens=[s + n_steps for s in lens0])
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
            assert_state_equal(host_buffer(cache), cfg, seqs, f"step {t}")
            ref = oracle_attend(draw.q.astype(np.float64), seqs, wl)
            assert_close(out.cpu().numpy(), ref, f"step {t}")
    assert seqs[(0, 0)].n_q > 0 and seqs[(1, 0)].n_q > 0  # both flushed at least once


def test_skvq_prefill_equals_appends_on_the_gpu():
    # the page's claim, on the device: the same tokens through prefill or through appends give
    # the same cache bytes (records, permutations, sinks, window, lengths)
    case = CASES[0]
    S = [5 + 128 * 2 + 7, 9]
    wl, draw, cfg = make(case, seed=33, lens=S + [1, 1])
    K, V, _ = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    a, b_ = KVQCache(cfg, device=DEV), KVQCache(cfg, device=DEV)
    kvq_prefill(a, Kt, Vt, S + [1, 1])
    kvq_prefill(b_, Kt, Vt, [0, 0, 0, 0])
    for t in range(max(S)):
        # sequences shorter than t + 1 would grow past their prefill length: give them their own
        # tokens too and compare only the sequences' common prefix below
        k = torch.stack([Kt[bb, :, min(t, Kt.shape[2] - 1)] for bb in range(4)]).contiguous()
        v = torch.stack([Vt[bb, :, min(t, Vt.shape[2] - 1)] for bb in range(4)]).contiguous()
        kvq_append(b_, k, v)
        if t + 1 == S[1]:
            torch.cuda.synchronize()
            cmp_seq(a, b_, cfg, 1)
    torch.cuda.synchronize()
    cmp_seq(a, b_, cfg, 0)


def cmp_seq(a, b_, cfg, b):
    from tests import kvq_unpack
    from tests.gpu_helpers import cfg_dict
    cd = cfg_dict(cfg)
    ba, bb = host_buffer(a), host_buffer(b_)
    for h in range(cfg.n_kv_heads):
        ua = kvq_unpack.unpack_sequence(ba, cd, b, h)
        ub = kvq_unpack.unpack_sequence(bb, cd, b, h)
        assert ua.keys() == ub.keys()
        for key in ua:
            va, vb = np.asarray(ua[key]), np.asarray(ub[key])
            if va.ndim == 0:
                assert va == vb, (b, h, key)
            else:
                assert va.shape == vb.shape and np.array_equal(va.view(np.uint8), vb.view(np.uint8)), (b, h, key)
