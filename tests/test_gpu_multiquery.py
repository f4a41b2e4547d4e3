"""GPU parity for multi-query attend (kvq_decode_attend_multi): the newest n_query tokens of each
sequence attend causally over the quantized cache, against the fp64 oracle's causal prefix
attention. Lengths are chosen so that masked tokens fall in the window, in the last record
(a window of 1..2 tokens) and among the sinks (short sequences), for KIVI, KIVI-Sink, SKVQ and
Kitty caches, every split count; n_query = 1 must equal kvq_decode_attend bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import kitty, kivi, skvq
from quantized_decode_attention_encode_amd import (KVQCache, kvq_decode_attend, kvq_decode_attend_multi,
                                                   kvq_prefill, make_config, workloads)
from tests.gpu_helpers import assert_close, oracle_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Hq, Hkv, D, bk, bv, lengths, n_query, method, n_sink, R
    ("kivi-d128-g1-q4", 4, 4, 4, 128, 2, 2, [321, 322, 96, 4], 4, "kivi", 0, 32),
    ("kivi-d64-g2-q4", 3, 4, 2, 64, 2, 4, [65, 200, 7], 4, "kivi", 0, 32),
    ("kivi-d128-g4-q2", 2, 8, 2, 128, 4, 2, [129, 33], 2, "kivi", 0, 32),
    ("sink-d128-g1-q8", 3, 2, 2, 128, 2, 2, [40, 300, 8], 8, "kivi", 5, 32),
    ("skvq-d64-g2-q2", 3, 4, 2, 64, 2, 2, [3, 140, 6], 2, "skvq", 3, 64),
    ("skvq-d128-g1-q4", 2, 2, 2, 128, 4, 4, [133, 4], 4, "skvq", 2, 128),
    ("kitty-d128-g1-q4", 3, 2, 2, 128, 2, 16, [321, 96, 4], 4, "kitty", 0, 32),
    ("kitty-d64-g2-q4", 2, 4, 2, 64, 2, 16, [200, 7], 4, "kitty", 0, 64),
    ("kitty-d128-g4-q2", 2, 8, 2, 128, 2, 16, [129, 33], 2, "kitty", 0, 32),
]


def setup(case, seed=41):
    name, B, Hq, Hkv, D, bk, bv, lens, nqry, method, ns, R = case
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=bk, value_bits=bv,
                          n_outlier=2, seed=seed, residual=R, ragged=(1, 2))
    draw = workloads.Draw(wl, seq_lens=lens)
    cfg = make_config(B, Hkv, Hq, D, bk, bv, 32, R, 1024, n_sink=ns, method=method)
    cache = KVQCache(cfg, device=DEV)
    K, V, _ = draw.padded()
    kvq_prefill(cache, torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), lens)
    if method in ("skvq", "kitty"):
        seqs = {}
        for b in range(B):
            for h in range(Hkv):
                if method == "skvq":
                    s = skvq.SkvqSequence(D, bk, bv, 32, R, ns)
                else:
                    s = kitty.KittySequence(D, cfg.kitty_n_hi, 4, bk, 32, R)
                s.prefill(draw.K[b][h], draw.V[b][h])
                seqs[(b, h)] = s
    else:
        seqs = oracle_prefill(draw, R, n_sink=ns)
    rng = np.random.default_rng(seed + 7)
    q = (rng.standard_normal((B, Hq, nqry, D)) / np.sqrt(D)).astype(np.float16)
    ref = np.zeros((B, Hq, nqry, D))
    for b in range(B):
        for hq in range(Hq):
            s = seqs[(b, kivi.kv_head_of(hq, Hq, Hkv))]
            ref[b, hq] = kivi.attend_causal(q[b, hq], s.keys_hat(), s.values_hat())
    return cache, q, ref


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_multi_query_causal_attend(case):
    cache, q, ref = setup(case)
    say("case", case[0])
    qt = torch.from_numpy(q).to(DEV)
    B, Hq, S_q, D = q.shape
    for n_split in (0, 1, 3, 64):
        out = kvq_decode_attend_multi(cache, qt, out_fp32=True, n_split=n_split).cpu().numpy()
        err = assert_close(out.reshape(B, Hq * S_q, D), ref.reshape(B, Hq * S_q, D), f"{case[0]} n_split={n_split}")
        say("  n_split", n_split, "err", err)


def test_one_query_is_decode_attend():
    cache, q, _ = setup(CASES[0])
    qt = torch.from_numpy(q[:, :, -1:]).to(DEV).contiguous()
    for n_split in (0, 2):
        a = kvq_decode_attend_multi(cache, qt, out_fp32=True, n_split=n_split)
        b = kvq_decode_attend(cache, qt[:, :, 0].contiguous(), out_fp32=True, n_split=n_split)
        assert torch.equal(a[:, :, 0], b)
