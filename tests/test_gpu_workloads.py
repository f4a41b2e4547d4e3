"""GPU parity at the full sizes of the five workloads, in the launch configuration the bench
times (automatic split count, fp16 output).

tiny / short: every head bit-exact and every output row checked. long: every output row,
encode bit-exact on sampled heads. gqa (ragged B=16, 32q/8kv, 2/4 bits): every head and
row. full32: one layer per run of sampled (b, h) pairs (layers 0 and 31), encode bit-exact
and the query heads of those KV heads.
"""
import numpy as np
import pytest
import torch

from quantized_decode_attention_encode_amd import KVQCache, kvq_decode_attend, kvq_prefill, make_config, workloads
from tests.gpu_helpers import assert_close, assert_state_equal, host_buffer, oracle_attend, oracle_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(name, layer=0, pairs=None, heads=None):
    wl = workloads.WORKLOADS[name]
    say(f"workload {name} layer {layer}: {wl.describe()}")
    draw = workloads.Draw(wl, layer=layer)
    S_max = max(draw.seq_lens)
    cap = (S_max + 31) // 32 * 32
    cfg = make_config(wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.key_bits, wl.value_bits, 32,
                      wl.residual, cap)
    cache = KVQCache(cfg, device=DEV)
    K, V, lens = draw.padded()
    Kt, Vt = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    del K, V
    kvq_prefill(cache, Kt, Vt, lens)
    q = torch.from_numpy(draw.q).to(DEV)
    out = kvq_decode_attend(cache, q).float().cpu().numpy()
    buf = host_buffer(cache)
    del Kt, Vt
    say("  gpu done; oracle ...")
    seqs = oracle_prefill(draw, wl.residual, pairs=pairs)
    bitexact = seqs if pairs is None else seqs
    assert_state_equal(buf, cfg, bitexact, name)
    ref = oracle_attend(draw.q.astype(np.float64), seqs, wl, heads=heads)
    err = assert_close(out, ref, name)
    say(f"  {name}: state bit-exact on {len(bitexact)} (b, h); attention max abs {err[0]:.2e}, row rel {err[1]:.2e}")
    return err


def test_tiny():
    run("tiny")


def test_short():
    run("short")


def test_long():
    # every output row; the oracle reconstructs all 32 heads
    run("long")


def test_gqa_ragged_batch():
    run("gqa")


@pytest.mark.parametrize("layer", [0, 31])
def test_full32_layer(layer):
    pairs = {(0, 0), (3, 5), (7, 7)}
    heads = {(b, hq) for (b, h) in pairs for hq in range(4 * h, 4 * h + 4)}
    run("full32", layer=layer, pairs=pairs, heads=heads)
