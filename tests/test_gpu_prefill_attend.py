"""GPU parity for chunked-prefill attend on the matrix cores (kvq_decode_attend_multi with more
query rows per KV head than the decode kernel holds): the newest n_query tokens of each sequence
attend causally over the quantized cache, against the fp64 oracle's causal prefix attention
(oracle.kivi.attend_causal). Ragged caches put the queries' own tokens in records and in the
window; row counts that are not multiples of the 16-row tiles or 64-row blocks leave partial
tiles; split counts from 1 to more than the units of the shortest sequence.
"""
import numpy as np
import pytest
import torch

from oracle import kivi
from quantized_decode_attention_encode_amd import (KVQCache, KVQError, kvq_decode_attend_multi, kvq_prefill,
                                                   make_config, workloads)
from tests.gpu_helpers import assert_close, oracle_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Hq, Hkv, D, bk, bv, lengths, n_query
    ("d128-g1-q16", 3, 4, 4, 128, 2, 2, [40, 700, 16], 16),
    ("d64-g4-q16", 2, 8, 2, 64, 2, 4, [333, 97], 16),
    ("d128-g4-q64", 2, 8, 2, 128, 2, 4, [1000, 130], 64),
    ("d64-g1-q64", 3, 2, 2, 64, 4, 8, [64, 480, 900], 64),
    ("d128-g1-q256", 2, 2, 2, 128, 2, 2, [1500, 257], 256),
    ("d128-g4-q256", 1, 8, 2, 128, 8, 4, [2100], 256),
    ("d64-g4-q256", 2, 4, 1, 64, 2, 2, [300, 1024], 256),
    ("d128-g2-q24", 2, 4, 2, 128, 4, 2, [500, 31], 24),
    ("d128-g1-q100", 2, 4, 4, 128, 2, 4, [100, 645], 100),
]


def setup(case, seed=91):
    name, B, Hq, Hkv, D, bk, bv, lens, nqry = case
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=bk, value_bits=bv,
                          n_outlier=2, seed=seed, ragged=(1, 2))
    draw = workloads.Draw(wl, seq_lens=lens)
    cfg = make_config(B, Hkv, Hq, D, bk, bv, 32, 32, 2304)
    cache = KVQCache(cfg, device=DEV)
    K, V, _ = draw.padded()
    kvq_prefill(cache, torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), lens)
    seqs = oracle_prefill(draw, 32)
    rng = np.random.default_rng(seed + 3)
    q = (rng.standard_normal((B, Hq, nqry, D)) / np.sqrt(D)).astype(np.float16)
    ref = np.zeros((B, Hq, nqry, D))
    for b in range(B):
        for hq in range(Hq):
            s = seqs[(b, kivi.kv_head_of(hq, Hq, Hkv))]
            ref[b, hq] = kivi.attend_causal(q[b, hq], s.keys_hat(), s.values_hat())
    return cache, q, ref


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_attend_matches_oracle(case):
    cache, q, ref = setup(case)
    say("case", case[0])
    qt = torch.from_numpy(q).to(DEV)
    B, Hq, S_q, D = q.shape
    for n_split in (0, 1, 3, 40):
        out = kvq_decode_attend_multi(cache, qt, out_fp32=True, n_split=n_split).cpu().numpy()
        err = assert_close(out.reshape(B, Hq * S_q, D), ref.reshape(B, Hq * S_q, D), f"{case[0]} n_split={n_split}")
        say("  n_split", n_split, "err", err)
    o16 = kvq_decode_attend_multi(cache, qt).float().cpu().numpy()
    assert_close(o16.reshape(B, Hq * S_q, D), ref.reshape(B, Hq * S_q, D), f"{case[0]} fp16 out")


def test_prefill_attend_on_a_reused_workspace_and_poisoned_output():
    cache, q, ref = setup(CASES[2], seed=92)
    qt = torch.from_numpy(q).to(DEV)
    B, Hq, S_q, D = q.shape
    ws = cache.workspace(0, S_q)
    ws.view(torch.uint8).fill_(0xFF)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    kvq_decode_attend_multi(cache, qt, out=out, out_fp32=True, workspace=ws)
    assert torch.isfinite(out).all()
    assert_close(out.cpu().numpy().reshape(B, Hq * S_q, D), ref.reshape(B, Hq * S_q, D), "reused")


def test_prefill_attend_rejects_caches_it_is_not_built_for():
    cfg = make_config(1, 2, 2, 64, 2, 2, 32, 32, 256, n_sink=2)
    c = KVQCache(cfg, device=DEV)
    K = torch.randn(1, 2, 200, 64, device=DEV).half()
    kvq_prefill(c, K, K, [200])
    with pytest.raises(KVQError) as e:
        kvq_decode_attend_multi(c, torch.zeros(1, 2, 16, 64, dtype=torch.float16, device=DEV))
    assert e.value.status == -2
    with pytest.raises(KVQError) as e:  # more queries than tokens
        cfg2 = make_config(1, 2, 2, 64, 2, 2, 32, 32, 256)
        c2 = KVQCache(cfg2, device=DEV)
        kvq_prefill(c2, K[:, :, :10].contiguous(), K[:, :, :10].contiguous(), [10])
        kvq_decode_attend_multi(c2, torch.zeros(1, 2, 16, 64, dtype=torch.float16, device=DEV))
    assert e.value.status == -1
