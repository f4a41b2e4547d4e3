"""kvq_decode_attend_noalloc (no caller workspace: the split partials live in the library's
static device scratch) against kvq_decode_attend on the same cache, through the C ABI.

Two calls in a row, the second with a smaller input, each equal to the workspace entry point's
output bit for bit (the same kernel and plan) and within the oracle's tolerance; a call whose
partials exceed the scratch is rejected before anything runs.
"""
import numpy as np
import pytest
import torch

from quantized_decode_attention_encode_amd import (KVQCache, KVQError, kvq_decode_attend, kvq_decode_attend_noalloc,
                                                   kvq_prefill, make_config, workloads)
from quantized_decode_attention_encode_amd._lib import KVQ_E_WORKSPACE, KVQ_NOALLOC_SCRATCH_BYTES
from tests.gpu_helpers import assert_close, oracle_attend, oracle_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def filled(name, B, Hq, Hkv, D, bk, bv, rag, seed, max_tokens):
    wl = workloads.custom(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, key_bits=bk, value_bits=bv,
                          n_outlier=2, seed=seed, ragged=rag)
    draw = workloads.Draw(wl)
    cfg = make_config(B, Hkv, Hq, D, bk, bv, 32, 32, max_tokens)
    cache = KVQCache(cfg, device=DEV)
    K, V, lens = draw.padded()
    kvq_prefill(cache, torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), lens)
    return wl, draw, cfg, cache


def check_one(wl, draw, cfg, cache, n_split, fp32):
    q = torch.from_numpy(draw.q).to(DEV)
    odt = torch.float32 if fp32 else torch.float16
    ref = kvq_decode_attend(cache, q, out_fp32=fp32, n_split=n_split)
    out = torch.full(tuple(q.shape), float("nan"), dtype=odt, device=DEV)
    kvq_decode_attend_noalloc(cache, q, out, out_fp32=fp32, n_split=n_split)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"{wl.name} n_split={n_split} fp32={fp32}"
    seqs = oracle_prefill(draw, cfg.residual)
    assert_close(out.float().cpu().numpy(), oracle_attend(draw.q.astype(np.float64), seqs, wl), wl.name)


def test_noalloc_equals_workspace_entry_then_a_smaller_call():
    big = filled("noalloc-big", 4, 16, 4, 128, 2, 4, (1, 3000), 90, 3072)
    small = filled("noalloc-small", 1, 4, 4, 64, 2, 2, (40, 100), 91, 128)
    for n_split in (0, 7):
        say("noalloc big then small, n_split", n_split)
        check_one(*big, n_split, True)
        check_one(*small, n_split, False)
    check_one(*big, 0, False)  # and back to the larger one: the array keeps nothing a call needs


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 64 sequences of 97..128 tokens (3 records + a window unit each), 64 query heads: with 4
    # splits the partials take 64 x 64 x 4 x 132 floats = 8.65 MB > 8 MiB
    wl, draw, cfg, cache = filled("noalloc-huge", 64, 64, 8, 128, 2, 2, (97, 128), 92, 160)
    need = 64 * 64 * 4 * (128 + 4) * 4
    assert need > KVQ_NOALLOC_SCRATCH_BYTES
    q = torch.from_numpy(draw.q).to(DEV)
    out = torch.zeros(tuple(q.shape), dtype=torch.float16, device=DEV)
    with pytest.raises(KVQError) as e:
        kvq_decode_attend_noalloc(cache, q, out, n_split=4)
    assert e.value.status == KVQ_E_WORKSPACE
    kvq_decode_attend_noalloc(cache, q, out, n_split=1)  # 64 x 64 x 1 x 132 floats fit
    assert torch.equal(out, kvq_decode_attend(cache, q, n_split=1))
