"""kvq_encode_block against the oracle quantizer, element by element (bit-exact codes, scale
and zero bits), on adversarial groups: ties, signed zeros, constant and near-constant groups,
subnormal-range ranges, outliers and wide ranges, for every bit width and both group rules."""
import numpy as np
import pytest
import torch

from oracle import kivi
from quantized_decode_attention_encode_amd import kvq_encode_block

pytestmark = pytest.mark.gpu
DEV = "cuda"
F16 = np.float16


def adversarial_groups(n_groups: int, bits: int, seed: int) -> np.ndarray:
    """[n_groups, 32] fp16 groups cycling through the kinds listed in the module docstring."""
    rng = np.random.default_rng(seed)
    L = 2 ** bits - 1
    out = np.empty((n_groups, 32), F16)
    for i in range(n_groups):
        kind = i % 8
        if kind == 0:
            g = rng.standard_normal(32)
        elif kind == 1:  # half-integer grid 0 .. L with both ends present: many exact ties
            g = rng.integers(0, 2 * L + 1, 32) / 2.0
            g[0], g[1] = 0.0, L
        elif kind == 2:  # signed zeros only
            g = np.where(rng.random(32) < 0.5, -0.0, 0.0)
        elif kind == 3:  # constant
            g = np.full(32, rng.standard_normal())
        elif kind == 4:  # one ulp apart
            base = F16(rng.standard_normal())
            g = np.where(rng.random(32) < 0.5, base, np.nextafter(base, F16(np.inf)))
        elif kind == 5:  # range inside the fp16 subnormals: subnormal or zero scale
            g = rng.standard_normal(32) * 2e-6
        elif kind == 6:  # one outlier
            g = rng.standard_normal(32)
            g[rng.integers(32)] *= 100.0
        else:  # wide range, near the fp16 limits
            g = rng.uniform(-60000.0, 60000.0, 32)
        out[i] = np.asarray(g).astype(F16)
    return out


def oracle_block(X: np.ndarray, bits: int, per_channel: bool):
    n_tok, D = X.shape
    if per_channel:
        g = X.reshape(n_tok // 32, 32, D).transpose(0, 2, 1)  # [n_tok/32, D, 32]
        c, s, z = kivi.quantize_groups(np.ascontiguousarray(g), bits)
        return c.transpose(0, 2, 1).reshape(n_tok, D), s, z
    c, s, z = kivi.quantize_groups(X.reshape(n_tok, D // 32, 32), bits)
    return c.reshape(n_tok, D), s, z


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("per_channel,n_tok,D", [(True, 64, 40), (True, 96, 128), (False, 37, 64), (False, 5, 128)])
def test_block_encode_matches_oracle_bit_for_bit(bits, per_channel, n_tok, D):
    n_groups = (n_tok // 32) * D if per_channel else n_tok * (D // 32)
    groups = adversarial_groups(n_groups, bits, seed=1000 + bits + n_tok + D)
    if per_channel:
        X = groups.reshape(n_tok // 32, D, 32).transpose(0, 2, 1).reshape(n_tok, D)
    else:
        X = groups.reshape(n_tok, D)
    X = np.ascontiguousarray(X)
    codes, scale, zero = kvq_encode_block(torch.from_numpy(X).to(DEV), bits, per_channel)
    rc, rs, rz = oracle_block(X, bits, per_channel)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scale.cpu().numpy().view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(zero.cpu().numpy().view(np.uint16), rz.view(np.uint16))


def test_block_encode_agrees_with_the_record_encoder():
    # the same values through kvq_encode_block and through a cache's records give the same
    # codes and parameters (both follow one arithmetic)
    from quantized_decode_attention_encode_amd import KVQCache, kvq_encode, make_config
    from tests.gpu_helpers import cfg_dict, host_buffer
    from tests.kvq_unpack import unpack_sequence
    rng = np.random.default_rng(5)
    D, T = 128, 64
    K = (rng.standard_normal((1, 1, T, D)) * 3).astype(F16)
    V = rng.standard_normal((1, 1, T, D)).astype(F16)
    cfg = make_config(1, 1, 1, D, 4, 2, 32, 32, 128)
    c = KVQCache(cfg, device=DEV)
    kvq_encode(c, torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), [T])
    st = unpack_sequence(host_buffer(c), cfg_dict(cfg), 0, 0)
    assert (st["n_q"], st["n_r"]) == (T, 0)
    kc, ks, kz = kvq_encode_block(torch.from_numpy(K[0, 0]).to(DEV), 4, True)
    vc, vs, vz = kvq_encode_block(torch.from_numpy(V[0, 0]).to(DEV), 2, False)
    assert np.array_equal(kc.cpu().numpy(), st["kc"]) and np.array_equal(vc.cpu().numpy(), st["vc"])
    for got, want in ((ks, st["ks"]), (kz, st["kz"]), (vs, st["vs"]), (vz, st["vz"])):
        assert np.array_equal(got.cpu().numpy().view(np.uint16), np.asarray(want, F16).view(np.uint16))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bk,bv", [(k, v) for k in (2, 4, 8) for v in (2, 4, 8)])
def test_record_encoder_on_adversarial_groups(D, bk, bv):
    # the record encoder (packed fp16 min/max, biased codes, lane-exchanged value words) on the
    # adversarial groups above: key groups (32 tokens of a channel) and value groups (32
    # channels of a token) each cycle through ties, signed zeros, constant, one-ulp,
    # subnormal-range, outlier and wide-range groups; codes, scales and zeros bit for bit
    from quantized_decode_attention_encode_amd import KVQCache, kvq_encode, make_config
    from tests.gpu_helpers import cfg_dict, host_buffer
    from tests.kvq_unpack import unpack_sequence
    T = 96
    kg = adversarial_groups((T // 32) * D, bk, seed=2000 + D + 10 * bk + bv)
    K = np.ascontiguousarray(kg.reshape(T // 32, D, 32).transpose(0, 2, 1).reshape(T, D))
    V = np.ascontiguousarray(adversarial_groups(T * (D // 32), bv, seed=3000 + D + 10 * bk + bv).reshape(T, D))
    cfg = make_config(1, 1, 1, D, bk, bv, 32, 32, 128)
    c = KVQCache(cfg, device=DEV)
    kvq_encode(c, torch.from_numpy(K[None, None]).to(DEV), torch.from_numpy(V[None, None]).to(DEV), [T])
    st = unpack_sequence(host_buffer(c), cfg_dict(cfg), 0, 0)
    assert (st["n_q"], st["n_r"]) == (T, 0)
    for name, X, bits, per_channel, got in (("keys", K, bk, True, ("kc", "ks", "kz")),
                                            ("values", V, bv, False, ("vc", "vs", "vz"))):
        rc, rs, rz = oracle_block(X, bits, per_channel)
        assert np.array_equal(np.asarray(st[got[0]]), rc), f"{name} codes"
        assert np.array_equal(np.asarray(st[got[1]], F16).view(np.uint16), rs.view(np.uint16)), f"{name} scales"
        assert np.array_equal(np.asarray(st[got[2]], F16).view(np.uint16), rz.view(np.uint16)), f"{name} zeros"
