"""Pins for the oracle's window state machine and decode attention.

* attention: a library routine (torch's scaled_dot_product_attention in float64 on the CPU)
  on the same reconstructed K/V, the brute-force loop twin, and closed forms (q = 0 gives
  the mean of the values; one dominant key returns its value);
* the all-fp16 special case (S <= R): no quantization at all, so the result is exact
  attention over the raw fp16 K/V;
* the window rule: known splits, path independence of prefill versus appends;
* GQA: a grouped cache equals a per-head cache with replicated KV heads;
* near-lossless at 8 bits, with an error that shrinks like the quantization step.

Passages: "Changelog" v0.42.0 (dequantize-then-attend equivalence of the fused kernel),
v0.8.0 (fp16 residual window), v0.28.0 (whole-chunk flush), "veloxquant_mlx.cache package"
(KVCacheConfig residual_length, kivi_group_size).
"""
import numpy as np
import pytest
import torch

from oracle import brute, kivi

F16 = np.float16


def sdpa64(q, k, v, scale=1.0):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, 0, 0].numpy()


def rand_seq(rng, S, D=64, bk=2, bv=2, R=32, outliers=2):
    K = rng.standard_normal((S, D)).astype(np.float32)
    K[:, :outliers] *= 10
    V = rng.standard_normal((S, D)).astype(np.float32)
    seq = kivi.KiviSequence(D, bk, bv, 32, R)
    seq.prefill(K.astype(F16), V.astype(F16))
    return seq, K.astype(F16), V.astype(F16)


def test_window_split_known_values():
    assert kivi.window_split(256, 32) == (224, 32)  # tiny workload: 224 quantized + 32 fp16
    assert kivi.window_split(512, 32) == (480, 32)
    assert kivi.window_split(65536, 32) == (65504, 32)
    assert kivi.window_split(1, 32) == (0, 1)
    assert kivi.window_split(32, 32) == (0, 32)
    assert kivi.window_split(33, 32) == (32, 1)
    assert kivi.window_split(0, 32) == (0, 0)
    assert kivi.window_split(200, 128) == (128, 72)
    for S in range(1, 300):
        nq, nr = kivi.window_split(S, 32)
        assert nq % 32 == 0 and 1 <= nr <= 32 and nq + nr == S


@pytest.mark.parametrize("R", [32, 64])
def test_prefill_equals_prefill_plus_appends(R):
    rng = np.random.default_rng(3)
    D = 64
    K = rng.standard_normal((300, D)).astype(F16)
    V = rng.standard_normal((300, D)).astype(F16)
    for S0 in (1, 31, 32, 33, 100):
        a = kivi.KiviSequence(D, 2, 4, 32, R)
        a.prefill(K, V)
        b = kivi.KiviSequence(D, 2, 4, 32, R)
        b.prefill(K[:S0], V[:S0])
        for t in range(S0, 300):
            b.append(K[t], V[t])
        for name in ("kc", "ks", "kz", "vc", "vs", "vz", "wk", "wv"):
            x, y = getattr(a, name), getattr(b, name)
            assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8)), name


def test_encode_then_appends_follows_window_rule():
    rng = np.random.default_rng(4)
    D = 32
    K = rng.standard_normal((96, D)).astype(F16)
    V = rng.standard_normal((96, D)).astype(F16)
    a = kivi.KiviSequence(D, 2, 2)
    a.encode(K[:64], V[:64])
    assert (a.n_q, a.n_r) == (64, 0)
    for t in range(64, 96):
        a.append(K[t], V[t])
    assert (a.n_q, a.n_r) == (64, 32)
    a.append(K[0], V[0])
    assert (a.n_q, a.n_r) == (96, 1)
    with pytest.raises(ValueError):
        a.encode(K[:32], V[:32])  # window not empty


def test_all_fp16_window_is_exact_attention():
    rng = np.random.default_rng(5)
    for S in (1, 7, 32):
        seq, K, V = rand_seq(rng, S)
        assert seq.n_q == 0
        q = (rng.standard_normal(64) / 8).astype(F16)
        out = kivi.attend(q, seq.keys_hat(), seq.values_hat())
        ref = sdpa64(q, K.astype(np.float64), V.astype(np.float64))
        assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("S,bk,bv", [(100, 2, 2), (257, 2, 4), (640, 4, 8)])
def test_attend_matches_library_sdpa_on_reconstruction(S, bk, bv):
    rng = np.random.default_rng(S)
    seq, _, _ = rand_seq(rng, S, bk=bk, bv=bv)
    q = (rng.standard_normal(64) / 8).astype(F16)
    kh, vh = seq.keys_hat(), seq.values_hat()
    for scale in (1.0, 0.37):
        out = kivi.attend(q, kh, vh, scale)
        assert np.max(np.abs(out - sdpa64(q, kh, vh, scale))) < 1e-12


def test_attend_matches_brute_loops():
    rng = np.random.default_rng(6)
    seq, _, _ = rand_seq(rng, 70, D=32)
    q = rng.standard_normal(32).astype(F16)
    kh, vh = seq.keys_hat(), seq.values_hat()
    ref = brute.attend(q.astype(np.float64).tolist(), kh.tolist(), vh.tolist(), 0.5)
    assert np.max(np.abs(kivi.attend(q, kh, vh, 0.5) - np.array(ref))) < 1e-12


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(7)
    seq, _, _ = rand_seq(rng, 200)
    out = kivi.attend(np.zeros(64, F16), seq.keys_hat(), seq.values_hat())
    assert np.max(np.abs(out - seq.values_hat().mean(0))) < 1e-12


def test_dominant_key_returns_its_value():
    rng = np.random.default_rng(8)
    D, S = 64, 96
    K = np.zeros((S, D), F16)
    K[:, 0] = 0.5  # every key scores 0.5 * q0 ...
    K[40, 0] = 100.0  # ... except token 40, which scores 100 * q0
    V = rng.standard_normal((S, D)).astype(F16)
    seq = kivi.KiviSequence(D, 8, 8)
    seq.prefill(K, V)
    q = np.zeros(D, F16)
    q[0] = 0.5  # score gap 49.75: the others carry a total weight below 95 * e**-49.75
    out = kivi.attend(q, seq.keys_hat(), seq.values_hat())
    assert np.max(np.abs(out - seq.values_hat()[40])) < 1e-18 + 95 * np.exp(-49.75) * 10


def test_gqa_equals_mha_with_replicated_kv():
    rng = np.random.default_rng(9)
    D, Hkv, G, S = 64, 2, 4, 150
    seqs_gqa = [[rand_seq(rng, S)[0] for _ in range(Hkv)]]
    seqs_mha = [[seqs_gqa[0][h // G] for h in range(Hkv * G)]]
    q = (rng.standard_normal((1, Hkv * G, D)) / 8).astype(F16)
    a = kivi.decode_attend(q, seqs_gqa)
    b = kivi.decode_attend(q, seqs_mha)
    assert np.array_equal(a, b)
    assert kivi.kv_head_of(5, 8, 2) == 1 and kivi.kv_head_of(3, 8, 2) == 0


def test_eight_bits_near_lossless_and_error_shrinks_with_step():
    rng = np.random.default_rng(10)
    D, S = 128, 2048
    K = rng.standard_normal((S, D)).astype(np.float32)
    K[:, :8] *= 10
    K = K.astype(F16)
    V = rng.standard_normal((S, D)).astype(F16)
    qs = (rng.standard_normal((16, D)) / np.sqrt(D)).astype(F16)
    Kd, Vd = K.astype(np.float64), V.astype(np.float64)
    exact = np.stack([sdpa64(q, Kd, Vd) for q in qs])
    err = {}
    for b in (2, 4, 8):
        seq = kivi.KiviSequence(D, b, b)
        seq.prefill(K, V)
        k_hat, v_hat = seq.keys_hat(), seq.values_hat()
        out = np.stack([kivi.attend(q, k_hat, v_hat) for q in qs])
        err[b] = np.linalg.norm(out - exact, axis=1) / np.linalg.norm(exact, axis=1)
        # every element's step: its key group's scale (32 tokens of a channel) or its value
        # group's (32 channels of a token); the window rows are exact
        nq = seq.n_q
        sk = np.zeros((S, D))
        sv = np.zeros((S, D))
        sk[:nq] = np.repeat(seq.ks.astype(np.float64), 32, axis=0)[:nq]
        sv[:nq] = np.repeat(seq.vs.astype(np.float64), 32, axis=1)[:nq]
        # rounding to the nearest code leaves every element within half its step (the fp32
        # subtract and multiply before the rounding add at most a few 2^-24 of the step)
        assert np.all(np.abs(k_hat - Kd) <= 0.5 * sk * (1 + 1e-3)), b
        assert np.all(np.abs(v_hat - Vd) <= 0.5 * sv * (1 + 1e-3)), b
        # the output error the steps imply: with the rounding errors spread evenly over their
        # half steps (variance step^2 / 12 each) and independent, the first-order error of
        # output channel c is a sum over tokens with standard deviation
        #   sigma_c = sqrt(sum_t p_t^2 (sv_tc^2 / 12 + (v_tc - o_c)^2 sum_d q_d^2 sk_td^2 / 12))
        # (value rounding, and the score perturbation moving the weights); the errors are
        # required to have that size: none beyond 6 sigma, and a median near a normal
        # deviate's 0.67 (a wrong step, a bias or a missing rounding moves it far off)
        z = []
        for q, o, oh in zip(qs, exact, out):
            qd = q.astype(np.float64)
            s = Kd @ qd
            p = np.exp(s - s.max())
            p /= p.sum()
            var_s = (qd ** 2 * sk ** 2).sum(axis=1) / 12
            sigma = np.sqrt((p[:, None] ** 2 * (sv ** 2 / 12 + (Vd - o) ** 2 * var_s[:, None])).sum(axis=0))
            z.append(np.abs(oh - o) / sigma)
        z = np.concatenate(z)
        assert z.max() <= 6.0, (b, z.max())
        assert 0.4 <= np.median(z) <= 1.0, (b, np.median(z))
    # near-lossless read as: median per-row relative L2 error below 1e-2 at 8 bits
    assert np.median(err[8]) <= 1e-2
    # the step shrinks by (2**4 - 1)/(2**2 - 1) = 5 and (2**8 - 1)/(2**4 - 1) = 17
    r24 = np.median(err[2]) / np.median(err[4])
    r48 = np.median(err[4]) / np.median(err[8])
    assert 5 / 2 <= r24 <= 5 * 2, r24
    assert 17 / 2 <= r48 <= 17 * 2, r48


# ---------------------------------------------------------------------------------------
# Multi-query (causal) attend: query j of S_q sees the cache up to its own token
# ---------------------------------------------------------------------------------------
def test_causal_multi_query_against_brute_force_prefixes():
    rng = np.random.default_rng(21)
    T, D, S_q = 45, 32, 4
    k = rng.standard_normal((T, D))
    v = rng.standard_normal((T, D))
    q = rng.standard_normal((S_q, D)).astype(np.float16)
    out = kivi.attend_causal(q, k, v, 0.7)
    for j in range(S_q):
        n = T - (S_q - 1 - j)
        ref = brute.attend([float(x) for x in q[j]], k[:n].tolist(), v[:n].tolist(), 0.7)
        assert np.allclose(out[j], ref, rtol=0, atol=1e-12)
    # one query: plain decode attention; the newest query sees every row
    assert np.allclose(kivi.attend_causal(q[-1:], k, v), kivi.attend(q[-1], k, v), rtol=0, atol=0)
    assert np.allclose(out[-1], kivi.attend(q[-1], k, v, 0.7), rtol=0, atol=0)
    # a key that only the last query can see changes only the last output
    k2 = k.copy()
    k2[-1] *= 50
    out2 = kivi.attend_causal(q, k2, v, 0.7)
    assert np.array_equal(out2[:-1], out[:-1]) and not np.allclose(out2[-1], out[-1])
