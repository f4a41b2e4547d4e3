"""Pins for the oracle's sink tokens ("Changelog" v0.9.0, KIVI-Sink), checked against things
other than the oracle itself:

* a hand-derived case where the fp32 channel-by-channel norm decides differently from the
  exact norm (pins the summation order and precision);
* the brute-force twin (pure Python, explicit binary32 rounding) for the selection and for
  the key groups with sinks left out, bit for bit;
* invariants: sink rows are reproduced exactly, the remaining rows' groups take their range
  from the remaining rows only, plain value parameters, the first-step rule;
* the page's own claims: n_sink_tokens = 0 is plain KIVI, and keeping a high-norm token out
  of the statistics lowers the other tokens' key error.
"""
import numpy as np
import pytest

from oracle import brute, kivi

F16 = np.float16


def rows(a):
    return [[float(x) for x in r] for r in np.asarray(a, np.float32)]


def test_norm_is_an_fp32_sum_in_channel_order():
    # Row 0 = [4096, 1, 1]: 4096^2 = 2^24; 2^24 + 1 rounds back to 2^24 (ties to even) twice.
    # Row 1 = [1, 1, 4096]: 1 + 1 = 2, then 2 + 2^24 is exact. Exact norms are equal
    # (2^24 + 2), so the exact rule would pick row 0 (earlier); the fp32 channel-order rule
    # picks row 1.
    K = np.array([[4096, 1, 1], [1, 1, 4096], [0, 0, 0]], F16)
    assert kivi.key_norms_sq(K).tolist() == [2.0 ** 24, 2.0 ** 24 + 2, 0.0]
    assert kivi.select_sinks(K, 1).tolist() == [1]
    # equal norms: the earlier row wins
    K2 = np.array([[3, 4], [4, 3], [0, 5], [1, 1]], F16)
    assert kivi.select_sinks(K2, 2).tolist() == [0, 1]
    assert kivi.select_sinks(K2, 3).tolist() == [0, 1, 2]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_selection_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((70, 32)).astype(F16)
    K[[5, 40]] *= F16(8)  # two planted high-norm rows
    K[17] = K[3]  # an exact tie
    for n in (1, 2, 5, 9):
        assert kivi.select_sinks(K, n).tolist() == brute.select_sinks(rows(K), n)
    assert set(kivi.select_sinks(K, 2).tolist()) == {5, 40}


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_key_groups_without_sinks_match_brute_force(bits):
    rng = np.random.default_rng(10 + bits)
    K = rng.standard_normal((64, 32)).astype(F16)
    K[[3, 35, 36]] *= F16(20)
    sinks = [3, 35, 36]
    c, s, z = kivi.encode_keys(K, bits, 32, sinks)
    bc, bs, bz = brute.encode_keys(rows(K), bits, 32, set(sinks))
    assert np.array_equal(c, np.array(bc, np.uint8))
    assert np.array_equal(s.view(np.uint16), np.array(bs, F16).view(np.uint16))
    assert np.array_equal(z.view(np.uint16), np.array(bz, F16).view(np.uint16))


def test_group_range_comes_from_the_other_tokens():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((64, 64)).astype(F16)
    K[7] = F16(100)
    c, s, z = kivi.encode_keys(K, 2, 32, [7])
    keep = np.ones(32, bool)
    keep[7] = False
    assert np.array_equal(z[0], K[:32][keep].min(axis=0))  # zero = min of the 31 others
    assert np.all(c[7] == 3)  # the sink is above every other key: clamped to the top code
    c0, s0, _ = kivi.encode_keys(K, 2, 32)
    assert np.all(s[0] < s0[0])  # the range shrank in every channel
    assert np.array_equal(s[1], s0[1]) and np.array_equal(c[32:], c0[32:])  # group 1 untouched


def test_sink_values_are_quantized_like_any_row():
    # a value group is one token's channels: choosing sinks changes no value parameter, and the
    # sink's own value rows reach attention exact (fp16) in place of their quantized slot
    rng = np.random.default_rng(4)
    K = rng.standard_normal((64, 64)).astype(F16)
    K[[2, 40]] = (K[[2, 40]].astype(np.float32) * 8).astype(F16)
    V = rng.standard_normal((64, 64)).astype(F16)
    plain, sink = kivi.KiviSequence(64, 2, 4, n_sink=0), kivi.KiviSequence(64, 2, 4, n_sink=2)
    plain.encode(K, V)
    sink.encode(K, V)
    assert sink.sink_pos.tolist() == [2, 40]
    for f in ("vc", "vs", "vz"):
        assert np.array_equal(getattr(plain, f).view(np.uint8), getattr(sink, f).view(np.uint8)), f
    assert np.all(sink.vs.view(np.uint16) < 0x8000)  # plain non-negative scales
    vh = sink.values_hat()
    assert np.array_equal(vh[[2, 40]], V[[2, 40]].astype(np.float64))
    others = np.setdiff1d(np.arange(64), [2, 40])
    assert np.array_equal(vh[others], plain.values_hat()[others])


def _sink_seq(K, V, n_sink, R=32, bits=(2, 2)):
    seq = kivi.KiviSequence(K.shape[1], *bits, R=R, n_sink=n_sink)
    seq.prefill(K, V)
    return seq


def test_zero_sinks_is_kivi():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((200, 64)).astype(F16)
    V = rng.standard_normal((200, 64)).astype(F16)
    a, b = _sink_seq(K, V, 0), _sink_seq(K, V, 0)
    b0 = kivi.KiviSequence(64, 2, 2)
    b0.prefill(K, V)
    for f in ("kc", "ks", "kz", "vc", "vs", "vz", "wk", "wv"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b0, f).view(np.uint8))
    assert a.sink_pos.size == 0 and b.sink_k.shape == (0, 64)


def test_sink_rows_are_exact_and_chosen_from_the_quantized_part():
    rng = np.random.default_rng(6)
    S, D = 150, 64  # n_q = 128, window 22
    K = rng.standard_normal((S, D)).astype(F16)
    V = rng.standard_normal((S, D)).astype(F16)
    K[[10, 70, 140]] *= F16(30)  # 140 is a window token: not a candidate
    seq = _sink_seq(K, V, 3)
    assert seq.n_q == 128 and seq.n_r == 22
    expect = brute.select_sinks(rows(K[:128]), 3)
    assert seq.sink_pos.tolist() == expect and {10, 70} <= set(expect)
    kh, vh = seq.keys_hat(), seq.values_hat()
    assert np.array_equal(kh[seq.sink_pos], K[seq.sink_pos].astype(np.float64))
    assert np.array_equal(vh[seq.sink_pos], V[seq.sink_pos].astype(np.float64))
    assert np.array_equal(kh[128:], K[128:].astype(np.float64))  # window rows


def test_sinks_are_chosen_once_at_the_first_flush():
    rng = np.random.default_rng(7)
    D = 32
    toks = rng.standard_normal((100, 2, D)).astype(F16)
    toks[[4, 50]] *= F16(25)  # 50 arrives after the first flush: never a sink
    seq = kivi.KiviSequence(D, 2, 2, R=32, n_sink=2)
    for t in range(100):
        seq.append(toks[t, 0], toks[t, 1])
        if t < 32:
            assert seq.sink_pos.size == 0  # nothing quantized yet
    assert seq.n_q == 96
    first = brute.select_sinks(rows(toks[:32, 0]), 2)
    assert seq.sink_pos.tolist() == first and 4 in first
    # the later groups were quantized without any exclusion
    c, s, z = kivi.encode_keys(np.ascontiguousarray(toks[32:96, 0]), 2, 32)
    assert np.array_equal(seq.kc[32:], c) and np.array_equal(seq.ks[1:].view(np.uint16), s.view(np.uint16))


def test_attention_over_sinks_matches_brute_force():
    rng = np.random.default_rng(8)
    S, D = 90, 32  # n_q = 64, window 26
    K = rng.standard_normal((S, D)).astype(F16)
    V = rng.standard_normal((S, D)).astype(F16)
    K[[1, 33]] *= F16(12)
    q = (rng.standard_normal(D) / np.sqrt(D)).astype(F16)
    seq = _sink_seq(K, V, 2)
    out = kivi.attend(q, seq.keys_hat(), seq.values_hat())
    # brute: own encode with the sinks left out, own reconstruction, fp16 rows at the sinks
    sinks = brute.select_sinks(rows(K[:64]), 2)
    kc, ks, kz = brute.encode_keys(rows(K[:64]), 2, 32, set(sinks))
    vc, vs, vz = brute.encode_values(rows(V[:64]), 2, 32)
    keys = [[kc[t][d] * ks[t // 32][d] + kz[t // 32][d] for d in range(D)] for t in range(64)]
    vals = [[vc[t][d] * vs[t][d // 32] + vz[t][d // 32] for d in range(D)] for t in range(64)]
    for t in sinks:
        keys[t] = [float(x) for x in K[t]]
        vals[t] = [float(x) for x in V[t]]
    keys += rows(K[64:])
    vals += rows(V[64:])
    ref = brute.attend([float(x) for x in q], keys, vals)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_a_high_norm_token_out_of_the_statistics_lowers_the_others_error():
    # the page's claim for KIVI-Sink: a sink outlier no longer inflates its groups' scale
    rng = np.random.default_rng(9)
    S, D = 256 + 1, 128
    K = rng.standard_normal((S, D)).astype(F16)
    V = rng.standard_normal((S, D)).astype(F16)
    K[[0, 100]] *= F16(40)
    plain, sink = _sink_seq(K, V, 0), _sink_seq(K, V, 2)
    assert sink.sink_pos.tolist() == [0, 100]
    others = np.setdiff1d(np.arange(256), [0, 100])
    err = lambda s: np.mean((s.keys_hat()[others] - K[others].astype(np.float64)) ** 2)
    assert err(sink) < 0.2 * err(plain)
