"""Pins for the SKVQ-adapted oracle ("Changelog" v0.30.0, SKVQ-adapted), checked against
things other than itself:

* with the clip search off at alpha = 1 and no reordering it is the plain per-token group
  quantizer, which the KIVI oracle implements independently (bit for bit);
* the brute-force twin (pure Python, explicit binary32/binary16 rounding) for the clip search
  and the permutation, on adversarial groups;
* hand-derived cases: the grid, the clip of a group with one far outlier, the channel order;
* invariants: the search never loses to alpha = 1 under its own error; 8-bit codes of
  integer ramps reproduce the input exactly after the inverse permutation; reordered groups
  hold channels of non-overlapping range bands; prefill equals token-by-token appends (the
  page's claim); sinks and window rows are exact; attention matches the brute-force loop.
"""
import numpy as np
import pytest

from oracle import brute, kivi, skvq

F16 = np.float16
F32 = np.float32


def test_grid_contains_alpha_one_and_is_k_over_40():
    c = skvq.clip_fractions()
    assert len(c) == 11 and c[0] == 0.0
    assert [float(x) for x in c] == [float(F32(k) / F32(40)) for k in range(11)]
    assert float(c[4]) == float(F32(0.1))  # alpha = 0.8 shrinks each end by a tenth of the range
    assert skvq.fixed_clip_fraction(1.0) == [0.0]
    assert skvq.fixed_clip_fraction(0.6)[0] == (F32(1) - F32(0.6)) * F32(0.5)  # fp32 ops, not 0.2


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_no_clip_no_reorder_is_the_plain_per_token_quantizer(bits):
    rng = np.random.default_rng(bits)
    X = (rng.standard_normal((40, 64)) * rng.uniform(0.1, 8, 64)).astype(F16)
    c, s, z, k = skvq.encode_block(X, np.arange(64), bits, skvq.fixed_clip_fraction(1.0))
    c0, s0, z0 = kivi.encode_values(X, bits, 32)
    assert np.array_equal(c, c0) and np.array_equal(s.view(np.uint16), s0.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), z0.view(np.uint16)) and not k.any()


def test_one_far_outlier_is_clipped():
    # 31 values spread over [0, 3] and one at 60: at alpha = 1 the 2-bit step is 20 and the 31
    # small values all round to 0; clipping saturates the outlier and resolves the rest.
    x = np.concatenate([np.linspace(0, 3, 31), [60]]).astype(F16)[None]
    c, s, z, k = skvq.clipped_group_quant(x, 2, skvq.clip_fractions())
    assert k[0] > 0
    _, s1, _, _ = skvq.clipped_group_quant(x, 2, skvq.fixed_clip_fraction(1.0))
    assert float(s[0]) < float(s1[0])
    assert c[0, -1] == 3  # the outlier saturates at the top code


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("bits", [2, 4])
def test_clip_search_matches_brute_force(seed, bits):
    rng = np.random.default_rng(100 + seed)
    G = rng.standard_normal((6, 32)).astype(np.float32)
    G[0, 5] = 40  # far outlier
    G[1] = np.round(G[1] * 4) / 4  # ties
    G[2] = 1.5  # constant group
    G[3, :16] = -0.0
    G[3, 16:] = 0.0
    G[4] *= 1e-5  # subnormal-range scales
    G = G.astype(F16)
    fr = skvq.clip_fractions()
    c, s, z, k = skvq.clipped_group_quant(G, bits, fr)
    for i in range(G.shape[0]):
        bc, bs, bz, bk = brute.clipped_group_quant([float(v) for v in G[i]], bits, [float(f) for f in fr])
        assert c[i].tolist() == bc, i
        assert s[i].view(np.uint16) == np.array(bs, F16).view(np.uint16), i
        assert z[i].view(np.uint16) == np.array(bz, F16).view(np.uint16), i
        assert k[i] == bk, i


def test_search_never_loses_to_alpha_one():
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((200, 32)) * 2).astype(F16)
    X[::7, 3] = F16(30)
    err = lambda c, s, z: ((X.astype(np.float64) - (c * s.astype(np.float64)[:, None] + z.astype(np.float64)[:, None])) ** 2).sum(1)
    c, s, z, k = skvq.clipped_group_quant(X, 2, skvq.clip_fractions())
    c1, s1, z1, _ = skvq.clipped_group_quant(X, 2, skvq.fixed_clip_fraction(1.0))
    assert np.all(err(c, s, z) <= err(c1, s1, z1) * (1 + 1e-6))
    assert (k > 0).any()


def test_channel_permutation_hand_case_and_brute_force():
    X = np.zeros((4, 6), F16)
    X[:, 0] = [0, 5, 0, 0]  # range 5
    X[:, 1] = [1, 2, 1, 1]  # range 1
    X[:, 2] = [-3, 3, 0, 0]  # range 6
    X[:, 3] = [2, 3, 2, 2]  # range 1 (tie with channel 1: stays after it)
    # channels 4, 5: range 0
    assert skvq.channel_permutation(X).tolist() == [4, 5, 1, 3, 0, 2]
    rng = np.random.default_rng(3)
    Y = (rng.standard_normal((128, 64)) * rng.uniform(0.5, 5, 64)).astype(F16)
    Y[:, 10] = Y[:, 20]  # a tie
    rows = [[float(v) for v in r] for r in Y]
    assert skvq.channel_permutation(Y).tolist() == brute.channel_permutation(rows)


def test_reordered_groups_hold_range_bands():
    rng = np.random.default_rng(4)
    spread = np.exp(rng.uniform(0, np.log(300), 128))  # 2.5 decades of channel scales
    X = (rng.standard_normal((128, 128)) * spread).astype(F16)
    perm = skvq.channel_permutation(X)
    r = X.astype(np.float32).max(0) - X.astype(np.float32).min(0)
    bands = r[perm].reshape(4, 32)
    assert np.all(bands[:-1].max(1) <= bands[1:].min(1))


def test_eight_bit_integer_ramps_round_trip_through_the_permutation():
    rng = np.random.default_rng(5)
    D = 64
    perm = rng.permutation(D)
    X = np.zeros((3, D), F16)
    for t in range(3):
        ramp = np.arange(32, dtype=np.float32) * 255 / 31  # 0 .. 255 inside each group
        vals = np.concatenate([np.round(ramp), np.round(ramp[::-1])]) + 100 * t
        X[t, perm] = vals.astype(F16)  # permuted group k holds an exact 0..255 span
    c, s, z, k = skvq.encode_block(X, perm, 8, skvq.fixed_clip_fraction(1.0))
    assert np.all(s == 1)
    assert np.array_equal(skvq.decode_block(c, s, z, perm), X.astype(np.float64))


def _toks(rng, S, D):
    K = (rng.standard_normal((S, D)) * rng.uniform(0.3, 6, D)).astype(F16)
    V = rng.standard_normal((S, D)).astype(F16)
    return K, V


@pytest.mark.parametrize("R,ns,S", [(128, 5, 5 + 128 * 2 + 40), (64, 0, 64 * 3 + 1), (32, 3, 2), (32, 16, 20 + 97)])
def test_prefill_equals_appends(R, ns, S):
    rng = np.random.default_rng(R + ns)
    K, V = _toks(rng, S, 64)
    a = skvq.SkvqSequence(64, 2, 2, 32, R, ns)
    a.prefill(K, V)
    b = skvq.SkvqSequence(64, 2, 2, 32, R, ns)
    for t in range(S):
        b.append(K[t], V[t])
    for f in ("kc", "vc", "ks", "kz", "vs", "vz", "wk", "wv", "sink_k", "sink_v"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8)), f
    if a.n_q:
        assert np.array_equal(a.perm_k, b.perm_k) and np.array_equal(a.perm_v, b.perm_v)
    n_q, n_r = kivi.window_split(max(S - ns, 0), R)
    assert (a.n_q, a.n_r, a.sink_k.shape[0]) == (n_q, n_r, min(ns, S))


def test_permutation_comes_from_the_first_chunk_only():
    rng = np.random.default_rng(6)
    K, V = _toks(rng, 5 + 128 * 3 + 1, 64)
    seq = skvq.SkvqSequence(64, 2, 2, 32, 128, 5)
    seq.prefill(K, V)
    assert np.array_equal(seq.perm_k, skvq.channel_permutation(K[5:133]))
    assert np.array_equal(seq.perm_v, skvq.channel_permutation(V[5:133]))
    off = skvq.SkvqSequence(64, 2, 2, 32, 128, 5, reorder=False)
    off.prefill(K, V)
    assert np.array_equal(off.perm_k, np.arange(64))


def test_attention_over_skvq_matches_brute_force():
    rng = np.random.default_rng(8)
    D, R, ns = 32, 32, 3
    S = ns + 64 + 10
    K, V = _toks(rng, S, D)
    q = (rng.standard_normal(D) / np.sqrt(D)).astype(F16)
    seq = skvq.SkvqSequence(D, 2, 2, 32, R, ns)
    seq.prefill(K, V)
    out = kivi.attend(q, seq.keys_hat(), seq.values_hat())
    # brute: own permutation and clip search on the 64 quantized tokens
    rows = lambda A: [[float(v) for v in r] for r in A]
    fr = [float(f) for f in skvq.clip_fractions()]
    keys, vals = rows(K[:ns]), rows(V[:ns])
    for X, out_rows in ((K, keys), (V, vals)):
        perm = brute.channel_permutation(rows(X[ns:ns + R]))
        for t in range(ns, ns + 64):
            xp = [float(X[t, p]) for p in perm]
            c, s, z, _ = brute.clipped_group_quant(xp, 2, fr)
            row = [0.0] * D
            for j, p in enumerate(perm):
                row[p] = c[j] * s + z
            out_rows.append(row)
    keys += rows(K[ns + 64:])
    vals += rows(V[ns + 64:])
    ref = brute.attend([float(v) for v in q], keys, vals)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
