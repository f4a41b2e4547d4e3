"""Pins for the oracle's encoder, checked against things other than itself.

* hand-derived closed forms (which axis a group runs along, round-half-even ties,
  parameters of a known ramp);
* the brute-force twin (pure Python, binary64 with explicit rounding) on tiny adversarial
  inputs, bit for bit;
* invariants every min/max group quantizer must satisfy (code range, end points, constant
  groups, round-trip bound, signed zeros).

Passages: "Changelog" v0.8.0 (KIVI: keys per channel, values per token, group size 32),
v0.42.0 (codes plus per-group (scale, zero) from min/max), v0.30.0 (lo/scale, fp16 metadata).
"""
import numpy as np
import pytest

from oracle import brute, kivi

F16 = np.float16


def f16bits(a):
    return np.asarray(a, F16).view(np.uint16)


# ---------------------------------------------------------------------------------------
# Closed forms derived by hand
# ---------------------------------------------------------------------------------------
def test_key_groups_run_along_tokens_and_value_groups_along_channels():
    # K[t, 0] = t (a ramp over tokens), K[t, 1] = 5 (constant over tokens).
    # Per-channel key groups: channel 0 spans 0..31, channel 1 is constant.
    T, D = 32, 32
    K = np.zeros((T, D), F16)
    K[:, 0] = np.arange(T)
    K[:, 1] = 5
    codes, scale, zero = kivi.encode_keys(K, bits=2, g=32)
    # scale = 31/3 = 10.3333..., rounded to fp16: spacing 2**-7 in [8, 16),
    # 10.3333/2**-7 = 1322.67 -> 1323 * 2**-7 = 10.3359375.
    assert scale[0, 0] == F16(10.3359375)
    assert zero[0, 0] == 0
    # code boundaries at t/10.3359375 = 0.5, 1.5, 2.5  ->  t = 5.17, 15.5, 25.84
    expect = np.array([0] * 6 + [1] * 10 + [2] * 10 + [3] * 6, np.uint8)
    assert np.array_equal(codes[:, 0], expect)
    # constant channel: scale 0, zero 5, all codes 0
    assert f16bits(scale[0, 1]) == 0 and zero[0, 1] == 5 and not codes[:, 1].any()
    # the same matrix as values: every token is [t, 5, 0, 0, ...] -> per-token range is
    # max(t, 5) - 0; token 0 has range 5 -> scale 5/3 rounded to fp16.
    vc, vs, vz = kivi.encode_values(K, bits=2, g=32)
    assert vs.shape == (T, 1)
    assert vs[0, 0] == F16(5.0 / 3.0)
    assert vs[31, 0] == F16(31.0 / 3.0)


def test_value_groups_of_32_channels():
    # V[t, d] = d for d < 64: group k covers channels 32k..32k+31 -> lo = 32k, hi = 32k+31
    V = np.tile(np.arange(64, dtype=F16), (4, 1))
    codes, scale, zero = kivi.encode_values(V, bits=2, g=32)
    assert scale.shape == (4, 2)
    assert np.all(zero[:, 0] == 0) and np.all(zero[:, 1] == 32)
    assert np.all(scale == F16(10.3359375))
    # within each group the codes follow the same ramp as the key test
    ramp = np.array([0] * 6 + [1] * 10 + [2] * 10 + [3] * 6, np.uint8)
    assert np.array_equal(codes[0], np.concatenate([ramp, ramp]))


def test_ties_round_half_to_even():
    # lo = 0, hi = 3, b = 2 -> scale exactly 1, inv exactly 1; x = 0.5, 1.5, 2.5 sit on ties.
    xs = np.zeros((32, 1), F16)
    xs[:8, 0] = [0, 3, 0.5, 1.5, 2.5, 1, 2, 0.25]
    codes, scale, zero = kivi.encode_keys(xs, bits=2, g=32)
    assert scale[0, 0] == 1 and zero[0, 0] == 0
    # half to even: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2 (half-up would give 1, 2, 3)
    assert list(codes[:8, 0]) == [0, 3, 0, 2, 2, 1, 2, 0]


def test_eight_bit_identity_on_integers():
    # values 0..255 spread over a group of 32 with min 0 and max 255 -> scale 1, codes = values
    rng = np.random.default_rng(0)
    v = rng.integers(0, 256, size=32).astype(F16)
    v[0], v[1] = 0, 255
    codes, scale, zero = kivi.quantize_groups(v[None, :], 8)
    assert scale[0] == 1 and zero[0] == 0
    assert np.array_equal(codes[0], v.astype(np.uint8))


def test_signed_zero_group_has_zero_parameter_bits():
    x = np.array([[-0.0, 0.0] * 16], F16)
    codes, scale, zero = kivi.quantize_groups(x, 2)
    assert f16bits(scale)[0] == 0 and f16bits(zero)[0] == 0 and not codes.any()
    x = np.array([[-0.0] * 32], F16)
    codes, scale, zero = kivi.quantize_groups(x, 4)
    assert f16bits(zero)[0] == 0  # -0 canonicalised to +0


# ---------------------------------------------------------------------------------------
# Brute-force twin, bit for bit
# ---------------------------------------------------------------------------------------
def adversarial_block(rng, T, D):
    """fp16 [T, D] mixing normal data, outliers, subnormals, ties, zeros and constants."""
    kind = rng.integers(0, 7)
    if kind == 0:
        x = rng.standard_normal((T, D)).astype(np.float32)
    elif kind == 1:
        x = rng.standard_normal((T, D)).astype(np.float32) * np.float32(2.0 ** rng.integers(-20, 12))
    elif kind == 2:  # subnormal range
        x = rng.integers(-40, 40, size=(T, D)).astype(np.float32) * np.float32(2.0 ** -24)
    elif kind == 3:  # small integers: exact scales, many ties
        x = rng.integers(-6, 7, size=(T, D)).astype(np.float32) * np.float32(0.5)
    elif kind == 4:  # near-constant
        x = np.float32(rng.standard_normal()) + rng.integers(0, 2, size=(T, D)).astype(np.float32) * np.float32(2 ** -10)
    elif kind == 5:  # extremes
        x = rng.choice(np.array([-65504, -1, -0.0, 0.0, 1, 65504], np.float32), size=(T, D))
    else:  # outlier channels
        x = rng.standard_normal((T, D)).astype(np.float32)
        x[:, rng.integers(0, D, 3)] *= 10
    return x.astype(F16)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_twin_bit_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    g = 32
    T = g * int(rng.integers(1, 4))
    D = int(rng.choice([32, 64]))
    X = adversarial_block(rng, T, D)
    for bits in (2, 3, 4, 8):
        kc, ks, kz = kivi.encode_keys(X, bits, g)
        bc, bs, bz = brute.encode_keys(X.astype(np.float64).tolist(), bits, g)
        assert np.array_equal(kc, np.array(bc, np.uint8))
        assert np.array_equal(f16bits(ks), f16bits(np.array(bs)))
        assert np.array_equal(f16bits(kz), f16bits(np.array(bz)))
        vc, vs, vz = kivi.encode_values(X, bits, g)
        bc, bs, bz = brute.encode_values(X.astype(np.float64).tolist(), bits, g)
        assert np.array_equal(vc, np.array(bc, np.uint8))
        assert np.array_equal(f16bits(vs), f16bits(np.array(bs)))
        assert np.array_equal(f16bits(vz), f16bits(np.array(bz)))


# ---------------------------------------------------------------------------------------
# Invariants of a min/max group quantizer
# ---------------------------------------------------------------------------------------
def random_groups(n=20000, g=32, seed=5):
    rng = np.random.default_rng(seed)
    parts = [
        rng.standard_normal((n, g)),
        rng.standard_normal((n // 4, g)) * 10,
        rng.integers(-30, 30, size=(n // 4, g)) * 2.0 ** -24,  # subnormal range
        rng.standard_normal((n // 4, 1)) + rng.integers(0, 3, size=(n // 4, g)) * 2.0 ** -11,
        rng.integers(-4, 5, size=(n // 4, g)) * 0.25,  # exact ties
    ]
    return np.concatenate([p.astype(np.float32).astype(F16) for p in parts])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_group_invariants(bits):
    x = random_groups()
    L = 2 ** bits - 1
    codes, scale, zero = kivi.quantize_groups(x, bits)
    assert codes.max() <= L
    x32 = x.astype(np.float64)
    lo = x32.min(1)
    hi = x32.max(1)
    s = scale.astype(np.float64)
    nonconst = s > 0
    # zero is the exact group minimum
    assert np.array_equal(zero.astype(np.float64), lo)
    # the minimum element always maps to code 0
    amin = x32.argmin(1)
    assert np.all(codes[np.arange(len(x)), amin][nonconst] == 0)
    # the maximum maps to L whenever the stored scale is a normal fp16 (>= 2**-14)
    amax = x32.argmax(1)
    normal = s >= 2.0 ** -14
    assert np.all(codes[np.arange(len(x)), amax][normal] == L)
    # constant groups reconstruct exactly
    const = hi == lo
    xhat = kivi.dequantize_groups(codes, scale, zero)
    assert np.array_equal(xhat[const], x32[const])
    # round-trip bound: half a step + clamp slack from rounding the scale to fp16
    # + a few ulps of the fp32 arithmetic
    err = np.abs(xhat - x32)
    slack = np.maximum(0.0, (hi - lo) - L * s)
    bound = s / 2 + slack + 2.0 ** -22 * np.maximum(np.abs(lo), np.abs(hi))
    assert np.all(err <= bound[:, None] * (1 + 1e-12))


def test_round_trip_within_half_step_for_normal_data():
    # the pages' own invariant stated without the rounding slack: for N(0,1) data the
    # reconstruction is within scale/2 (plus a relative 2**-11 of the range)
    x = np.random.default_rng(9).standard_normal((4096, 32)).astype(np.float32).astype(F16)
    codes, scale, zero = kivi.quantize_groups(x, 2)
    xhat = kivi.dequantize_groups(codes, scale, zero)
    s = scale.astype(np.float64)[:, None]
    assert np.all(np.abs(xhat - x.astype(np.float64)) <= s / 2 + s * 3 * 2.0 ** -11)
