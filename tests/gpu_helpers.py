"""Shared pieces of the GPU parity tests: run the HIP path and the CPU oracle on the same
seeded inputs and compare them (codes/params bit for bit, attention within tolerance).

Tolerance for attention (fp32 kernel arithmetic vs the fp64 oracle): max |out - ref| <= 2e-3
and, per (b, h) row, ||out - ref||_2 / ||ref||_2 <= 1e-2.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import kivi
from tests import kvq_unpack

ATOL = 2e-3
RTOL_ROW = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cfg_dict(c):
    return {"B": c.batch, "Hkv": c.n_kv_heads, "D": c.head_dim, "bk": c.key_bits, "bv": c.value_bits,
            "R": c.residual, "max_tokens": c.max_tokens, "NS": c.n_sink, "method": c.method}


def oracle_prefill(draw, R, pairs=None, n_sink=0):
    """KiviSequence per (b, h) for the drawn K/V (optionally only the given (b, h) pairs)."""
    wl = draw.wl
    seqs = {}
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            if pairs is not None and (b, h) not in pairs:
                continue
            s = kivi.KiviSequence(wl.head_dim, wl.key_bits, wl.value_bits, 32, R, n_sink)
            s.prefill(draw.K[b][h], draw.V[b][h])
            seqs[(b, h)] = s
    return seqs


def host_buffer(cache):
    return cache.buffer.cpu().numpy()


def assert_state_equal(buf, c, seqs, what=""):
    """Bit-exact comparison of the device cache state with oracle sequences."""
    cd = cfg_dict(c)
    for (b, h), s in seqs.items():
        got = kvq_unpack.unpack_sequence(buf, cd, b, h)
        assert (got["n_q"], got["n_r"]) == (s.n_q, s.n_r), f"{what} lengths of {(b, h)}"
        fields = [("kc", s.kc), ("vc", s.vc), ("ks", s.ks), ("kz", s.kz), ("vs", s.vs), ("vz", s.vz),
                  ("wk", s.wk), ("wv", s.wv), ("sink_k", s.sink_k), ("sink_v", s.sink_v)]
        if hasattr(s, "sink_pos"):
            fields.append(("sink_pos", s.sink_pos))
            # the device's slot marker: exactly the sinks' quantized slots
            mark = np.zeros(s.n_q, bool)
            mark[s.sink_pos] = True
            fields.append(("vmark", mark))
        else:  # SKVQ: the first tokens, and the permutations once a chunk is quantized
            fields.append(("sink_pos", np.arange(s.sink_k.shape[0], dtype=np.int64)))
            fields.append(("vmark", np.zeros(s.n_q, bool)))  # its sinks have no quantized slot
            if s.n_q:
                fields += [("perm_k", np.asarray(s.perm_k, np.int64)), ("perm_v", np.asarray(s.perm_v, np.int64))]
        for name, ref in fields:
            g = got[name]
            assert g.shape == ref.shape, f"{what} {name} shape {g.shape} vs {ref.shape} at {(b, h)}"
            if not np.array_equal(g.view(np.uint8), ref.view(np.uint8)):
                bad = np.argwhere(g.view(np.uint8).reshape(g.shape[0], -1) != ref.view(np.uint8).reshape(ref.shape[0], -1))
                raise AssertionError(f"{what} {name} differs at {(b, h)}: first mismatches {bad[:5].tolist()}")


def oracle_attend(q, seqs, wl, sm_scale=1.0, heads=None):
    """fp64 reference [B, H_q, D] (rows not in `heads` are NaN)."""
    B, Hq, D = q.shape
    G = Hq // wl.n_kv_heads
    out = np.full((B, Hq, D), np.nan)
    cache = {}
    for b in range(B):
        for hq in range(Hq):
            h = kivi.kv_head_of(hq, Hq, wl.n_kv_heads)
            if (b, h) not in seqs or (heads is not None and (b, hq) not in heads):
                continue
            if (b, h) not in cache:
                cache[(b, h)] = (seqs[(b, h)].keys_hat(), seqs[(b, h)].values_hat())
            out[b, hq] = kivi.attend(q[b, hq], *cache[(b, h)], sm_scale)
    assert G >= 1
    return out


def assert_close(out, ref, what=""):
    out = np.asarray(out, np.float64)
    mask = ~np.isnan(ref[..., 0])
    assert np.all(np.isfinite(out[mask])), f"{what}: non-finite output"
    err = np.abs(out[mask] - ref[mask])
    rel = np.linalg.norm(out[mask] - ref[mask], axis=-1) / np.maximum(np.linalg.norm(ref[mask], axis=-1), 1e-30)
    assert err.max() <= ATOL, f"{what}: max abs err {err.max():.3e} > {ATOL}"
    assert rel.max() <= RTOL_ROW, f"{what}: max row rel err {rel.max():.3e} > {RTOL_ROW}"
    return float(err.max()), float(rel.max())
