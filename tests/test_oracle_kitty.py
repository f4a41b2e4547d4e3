"""Pins for the Kitty oracle ("Changelog" v0.11.0, Kitty), checked against things other than
itself:

* the brute-force twin (pure Python): variances recomputed from scratch for every group in
  exact rational arithmetic (mean, then mean squared deviation) instead of the oracle's
  running integer sums, the ranking, and the binary32/binary16 group quantizer;
* special cases that reduce to the independently pinned KIVI key quantizer: all channels
  high (n_hi = D) is KIVI at hi_bits, none (n_hi = 0) is KIVI at lo_bits;
* hand-derived rankings: channels of known spread, equal spreads (lower index wins), a
  channel whose variance overtakes another's only after later groups;
* invariants: 2.5 average key bits at the default quarter, values stored exactly, high
  channels reconstruct better than low ones, prefill equals token-by-token appends, the
  running sums equal a direct sum.
"""
import numpy as np
import pytest

from oracle import brute, kitty, kivi

F16 = np.float16


def draw(T, D, seed, spread=True):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, D)) * (rng.uniform(0.2, 6.0, D) if spread else 1.0)
    V = rng.standard_normal((T, D))
    return K.astype(F16), V.astype(F16)


def test_n_hi_of_fraction():
    assert kitty.n_hi_of(0.25, 128) == 32 and kitty.n_hi_of(0.25, 64) == 16
    assert kitty.n_hi_of(0.0, 128) == 0 and kitty.n_hi_of(1.0, 128) == 128
    with pytest.raises(ValueError):
        kitty.n_hi_of(1.5, 128)


def test_key_ints_are_exact():
    x = np.array([0.0, -0.0, 2.0 ** -24, -(2.0 ** -24), 1.0, 65504.0, -65504.0, 0.333], F16)
    X = kitty.key_ints(x[:, None])[:, 0]
    assert X.tolist()[:7] == [0, 0, 1, -1, 2 ** 24, 65504 * 2 ** 24, -65504 * 2 ** 24]
    assert X[7] == int(float(x[7]) * 2 ** 24) and float(X[7]) / 2 ** 24 == float(x[7])


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("D,n_hi", [(32, 8), (64, 16), (32, 0), (32, 32)])
def test_matches_brute_force(seed, D, n_hi):
    K, V = draw(96, D, seed)
    K[:, 3] = K[0, 3]  # a constant channel (variance 0)
    K[:, 5] = K[:, 6]  # two channels of equal variance: the lower index ranks first
    s = kitty.KittySequence(D, n_hi, 4, 2, 32, 32)
    s.encode(K, V)
    c, sc, z, hi = brute.kitty_encode_keys(K.astype(float).tolist(), n_hi, 4, 2, 32)
    assert np.array_equal(s.kc, np.array(c, np.uint8))
    assert np.array_equal(s.ks, np.array(sc, F16)) and np.array_equal(s.kz, np.array(z, F16))
    assert np.array_equal(s.khi, np.array(hi, bool))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_all_or_no_channels_high_is_kivi(bits):
    K, V = draw(64, 64, 7)
    for n_hi, hb, lb in ((64, bits, 2), (0, 4, bits)):
        s = kitty.KittySequence(64, n_hi, hb, lb, 32, 32)
        s.encode(K, V)
        c0, s0, z0 = kivi.encode_keys(K, bits, 32)
        assert np.array_equal(s.kc, c0)
        assert np.array_equal(s.ks.view(np.uint16), s0.view(np.uint16))
        assert np.array_equal(s.kz.view(np.uint16), z0.view(np.uint16))


def test_hand_ranking_by_spread_and_ties():
    # channel d takes the values +-d (alternating): variance d^2, so the top channels are the
    # highest indices; channel 12 is made a copy of channel 11, so the two tie for the fourth
    # place and the lower index, 11, takes it.
    T, D = 32, 16
    sign = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)
    K = (sign[:, None] * np.arange(D)[None, :]).astype(F16)
    K[:, 12] = K[:, 11]
    s = kitty.KittySequence(D, 4, 4, 2, 32, 32)
    s.encode(K, K)
    assert np.flatnonzero(s.khi[0]).tolist() == [11, 13, 14, 15]
    # a mean shift does not change a variance
    K2 = K.astype(np.float32)
    K2[:, 0] += 512.0
    s2 = kitty.KittySequence(D, 4, 4, 2, 32, 32)
    s2.encode(K2.astype(F16), K)
    assert np.flatnonzero(s2.khi[0]).tolist() == [11, 13, 14, 15]


def test_ranking_uses_every_token_up_to_the_group():
    # channel 0 is quiet in group 0 and loud in group 1; channel 1 the other way round. At
    # group 1 the running variances are (over 64 tokens) 0: 1^2/2 + 8^2/2 + ... -> channel 0
    # leads only once its loud group is counted, while group 0 is ranked on group 0 alone.
    T, D = 64, 4
    sign = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)
    K = np.zeros((T, D))
    K[:32, 0], K[32:, 0] = sign[:32] * 1.0, sign[32:] * 8.0
    K[:32, 1], K[32:, 1] = sign[:32] * 4.0, sign[32:] * 4.0
    K[:, 2] = sign * 0.5
    K[:, 3] = sign * 0.25
    s = kitty.KittySequence(D, 1, 4, 2, 32, 32)
    s.encode(K.astype(F16), K.astype(F16))
    assert np.flatnonzero(s.khi[0]).tolist() == [1]  # 16 > 1
    assert np.flatnonzero(s.khi[1]).tolist() == [0]  # (1 + 64)/2 = 32.5 > 16


def test_running_sums_equal_direct_sums():
    K, V = draw(128, 32, 3)
    s = kitty.KittySequence(32, 8, 4, 2, 32, 32)
    s.encode(K, V)
    X = K.astype(float) * 2 ** 24
    for d in range(32):
        col = [int(x) for x in X[:, d]]
        assert s.mom.s1[d] == sum(col) and s.mom.s2[d] == sum(x * x for x in col)
    assert s.mom.n == 128


def test_average_key_bits_and_exact_values():
    s = kitty.KittySequence(128, kitty.n_hi_of(0.25, 128), 4, 2, 32, 32)
    assert s.key_bits_per_element() == 2.5
    K, V = draw(100, 128, 4)
    s.prefill(K, V)
    assert np.array_equal(s.values_hat(), V.astype(np.float64))


def test_high_channels_reconstruct_better():
    K, V = draw(256, 64, 5, spread=False)
    s = kitty.KittySequence(64, 16, 4, 2, 32, 32)
    s.encode(K, V)
    err = (s.keys_hat() - K.astype(np.float64)) ** 2
    hi = np.repeat(s.khi, 32, axis=0)
    rel = err / np.maximum(np.repeat(s.ks.astype(np.float64), 32, axis=0), 1e-30) ** 2
    assert err[hi].mean() < err[~hi].mean()
    assert rel.max() <= 0.25 + 1e-6  # |x - x_hat| <= scale / 2 in every group


@pytest.mark.parametrize("S0", [1, 31, 32, 33, 64, 70])
def test_prefill_equals_appends(S0):
    K, V = draw(160, 64, 6)
    a = kitty.KittySequence(64, 16, 4, 2, 32, 64)
    a.prefill(K, V)
    b = kitty.KittySequence(64, 16, 4, 2, 32, 64)
    b.prefill(K[:S0], V[:S0])
    for t in range(S0, 160):
        b.append(K[t], V[t])
    for name in ("kc", "ks", "kz", "khi", "vq", "wk", "wv"):
        assert np.array_equal(getattr(a, name).view(np.uint8), getattr(b, name).view(np.uint8)), name
    assert a.mom.s1 == b.mom.s1 and a.mom.s2 == b.mom.s2 and (a.n_q, a.n_r) == (128, 32)


def test_attention_matches_brute_force_loop():
    K, V = draw(80, 32, 8)
    s = kitty.KittySequence(32, 8, 4, 2, 32, 32)
    s.prefill(K, V)
    q = np.random.default_rng(9).standard_normal(32) / np.sqrt(32)
    ref = brute.attend(q.tolist(), s.keys_hat().tolist(), s.values_hat().tolist())
    assert np.allclose(kivi.attend(q, s.keys_hat(), s.values_hat()), ref, atol=1e-12)
