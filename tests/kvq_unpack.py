"""Test-side reader of the cache buffer: raw device bytes -> logical arrays.

Written from the layout description (records of 32 tokens; key codes as
[P=t/2][quarter][t%2][words] with channel c' of the quarter at bit c'*bk, value codes as
[channel][words] with token t at bit t*bv, key params [channel], value params
[t/2][value group][t%2], fp16 (scale, zero) pairs with the scale in the low half, whose sign
bit marks a sink's quantized slot (stripped here and returned as "vmark"); then the
sink regions: positions int32 [B][H_kv][NS], key and value rows fp16 [B][H_kv][NS][D], and for
SKVQ caches the channel permutations uint8 [B][H_kv][2][D]; SKVQ records keep their key params
in the value-param layout, one (scale, zero) per token and group of permuted channels, and their
window and sink rows are stored permuted once the permutations exist; Kitty records hold per
token the key codes of the slots in 16-slot chunks, two words for a 4-bit chunk and one for a
2-bit chunk, then the (scale, zero) per slot, the slot-to-channel table and the fp16 values,
and a Kitty buffer ends with the running key sums per (b, h)). It shares no code with the HIP
library; parity tests compare its output with the CPU oracle.
"""
from __future__ import annotations

import numpy as np


def align256(x: int) -> int:
    return (x + 255) // 256 * 256


def kitty_record(D: int, n_hi: int) -> dict:
    """Offsets inside a Kitty record: (D + n_hi)/16 code words per token, then (scale, zero) per
    slot, the slot table, and the fp16 value rows [32][D] (16-byte aligned); 128-byte records."""
    W = D // 16 + n_hi // 16
    o = {"words": W, "params": 128 * W}
    o["table"] = o["params"] + 4 * D
    o["values"] = (o["table"] + D + 15) // 16 * 16
    o["bytes"] = (o["values"] + 64 * D + 127) // 128 * 128
    return o


def offsets(B, Hkv, D, bk, bv, R, max_tokens, NS=0, skvq=False, kitty_n_hi=None):
    max_groups = max_tokens // 32
    rec = 4 * D * (bk + bv + 2) if kitty_n_hi is None else kitty_record(D, kitty_n_hi)["bytes"]
    o = {"lengths": 0, "sync": B * Hkv * 2 * 4}
    o["records"] = align256(o["sync"] + B * Hkv * 4)
    o["record_bytes"] = rec
    o["rec_key_codes"] = 0
    o["rec_value_codes"] = 4 * D * bk
    o["rec_key_params"] = 4 * D * (bk + bv)
    o["rec_value_params"] = 4 * D * (bk + bv) + 4 * D
    o["window_k"] = align256(o["records"] + B * Hkv * max_groups * rec)
    wbytes = B * Hkv * R * D * 2
    o["window_v"] = align256(o["window_k"] + wbytes)
    o["sink_pos"] = align256(o["window_v"] + wbytes)
    o["sink_k"] = align256(o["sink_pos"] + B * Hkv * NS * 4)
    o["sink_v"] = align256(o["sink_k"] + B * Hkv * NS * D * 2)
    o["perm"] = align256(o["sink_v"] + B * Hkv * NS * D * 2)
    o["kstats"] = align256(o["perm"] + (B * Hkv * 2 * D if skvq else 0))
    o["total"] = align256(o["kstats"] + (B * Hkv * 24 * D if kitty_n_hi is not None else 0))
    o["max_groups"] = max_groups
    o["NS"] = NS
    return o


def _fields(u8: np.ndarray, nbits: int) -> np.ndarray:
    """Little-endian bit strings along the last axis (bytes) -> unsigned nbits-wide fields."""
    bits = np.unpackbits(u8, axis=-1, bitorder="little")
    bits = bits.reshape(*bits.shape[:-1], bits.shape[-1] // nbits, nbits).astype(np.uint16)
    return (bits << np.arange(nbits, dtype=np.uint16)).sum(-1).astype(np.uint8)


def unpack_records(recs: np.ndarray, D: int, bk: int, bv: int, skvq: bool = False):
    """Records as bytes [n, record_bytes] -> logical arrays covering their 32*n tokens."""
    n = recs.shape[0]
    o_vc = 4 * D * bk
    o_kp = o_vc + 4 * D * bv
    o_vp = o_kp + 4 * D
    # key codes [P][Q][tp][quarter bytes] -> [n, P, Q, tp, D/4]
    kc = _fields(recs[:, :o_vc].reshape(n, 16, 4, 2, D * bk // 32), bk)
    kc = kc.transpose(0, 1, 3, 2, 4).reshape(n * 32, D)  # token 2P+tp, channel Q*D/4 + c
    # value codes [d][bytes of 32 tokens] -> [n, d, 32]
    vc = _fields(recs[:, o_vc:o_kp].reshape(n, D, 4 * bv), bv).transpose(0, 2, 1).reshape(n * 32, D)
    NKG = D // 32
    if skvq:  # per-token key groups, value-param layout
        kp = np.ascontiguousarray(recs[:, o_kp:o_vp]).view("<u2").reshape(n, 16, NKG, 2, 2)
        kp = kp.transpose(0, 1, 3, 2, 4).reshape(n * 32, NKG, 2)
        ks, kz = kp[..., 0].view(np.float16), kp[..., 1].view(np.float16)
    else:
        kp = np.ascontiguousarray(recs[:, o_kp:o_vp]).view("<u2").reshape(n, D, 2)
        ks = kp[..., 0].view(np.float16).reshape(n, D)
        kz = kp[..., 1].view(np.float16).reshape(n, D)
    vp = np.ascontiguousarray(recs[:, o_vp:o_vp + 4 * D]).view("<u2").reshape(n, 16, NKG, 2, 2)
    vp = vp.transpose(0, 1, 3, 2, 4).reshape(n * 32, NKG, 2)  # token 2P+tp
    # The device marks the quantized slot of a KIVI-Sink token (attended from its fp16 rows
    # instead) with the sign bit of each of its value scales; a stored scale is never negative.
    # The marker is stripped here and returned on its own: "vmark" per token (every group of
    # the token agrees, or the record is malformed).
    sign = (vp[..., 0] & 0x8000) != 0
    vmark = sign.any(axis=-1)
    if np.any(sign.any(axis=-1) != sign.all(axis=-1)):
        raise ValueError("a token's value groups disagree on the sink marker")
    vs = (vp[..., 0] & 0x7FFF).view(np.float16)
    vz = vp[..., 1].view(np.float16)
    out = {"kc": kc, "ks": ks, "kz": kz, "vc": vc, "vs": vs, "vz": vz, "vmark": vmark}
    return {k: np.ascontiguousarray(v) for k, v in out.items()}


def unpack_kitty_records(recs: np.ndarray, D: int, n_hi: int):
    """Kitty records as bytes [n, record_bytes] -> channel-order logical arrays: key codes
    [32n, D], scale / zero [n, D] (fp16), the high-width mask [n, D] and the fp16 values [32n, D]."""
    n = recs.shape[0]
    o = kitty_record(D, n_hi)
    W, nhc = o["words"], n_hi // 16
    words = np.ascontiguousarray(recs[:, :128 * W]).view("<u4").reshape(n, 32, W).astype(np.uint64)
    slot = np.zeros((n, 32, D), np.uint8)
    for k in range(D // 16):
        if k < nhc:  # 16 4-bit codes over words 2k, 2k+1
            w = words[..., 2 * k] | (words[..., 2 * k + 1] << np.uint64(32))
            bits = 4
        else:  # 16 2-bit codes in word k + nhc
            w = words[..., k + nhc]
            bits = 2
        for i in range(16):
            slot[..., 16 * k + i] = ((w >> np.uint64(bits * i)) & np.uint64((1 << bits) - 1)).astype(np.uint8)
    table = recs[:, o["table"]:o["table"] + D].astype(np.int64)
    prm = np.ascontiguousarray(recs[:, o["params"]:o["params"] + 4 * D]).view("<u2").reshape(n, D, 2)
    kc = np.zeros((n, 32, D), np.uint8)
    ks = np.zeros((n, D), np.uint16)
    kz = np.zeros((n, D), np.uint16)
    hi = np.zeros((n, D), bool)
    for r in range(n):
        kc[r][:, table[r]] = slot[r]
        ks[r, table[r]] = prm[r, :, 0]
        kz[r, table[r]] = prm[r, :, 1]
        hi[r, table[r]] = np.arange(D) < n_hi
    vq = np.ascontiguousarray(recs[:, o["values"]:o["values"] + 64 * D]).view(np.float16).reshape(n * 32, D)
    return {"kc": kc.reshape(n * 32, D), "ks": ks.view(np.float16), "kz": kz.view(np.float16), "khi": hi,
            "vq": vq.copy(), "table": table}


def unpack_kitty_sequence(buf: np.ndarray, cfg: dict, b: int, h: int):
    """Kitty (b, h): records, window and the running key sums (Python ints) from the buffer."""
    B, Hkv, D, R, n_hi = (cfg[k] for k in ("B", "Hkv", "D", "R", "n_hi"))
    o = offsets(B, Hkv, D, 2, 2, R, cfg["max_tokens"], 0, False, n_hi)
    L = lengths(buf, B, Hkv)
    n_q, n_r = int(L[b, h, 0]), int(L[b, h, 1])
    ng = n_q // 32
    start = o["records"] + (b * Hkv + h) * o["max_groups"] * o["record_bytes"]
    recs = buf[start:start + ng * o["record_bytes"]].reshape(ng, o["record_bytes"])
    cat = unpack_kitty_records(recs, D, n_hi)
    w0 = ((b * Hkv + h) * R) * D * 2
    cat["wk"] = buf[o["window_k"] + w0:o["window_k"] + w0 + R * D * 2].view(np.float16).reshape(R, D)[:n_r].copy()
    cat["wv"] = buf[o["window_v"] + w0:o["window_v"] + w0 + R * D * 2].view(np.float16).reshape(R, D)[:n_r].copy()
    st = buf[o["kstats"] + (b * Hkv + h) * 24 * D:o["kstats"] + (b * Hkv + h + 1) * 24 * D]
    s1 = st[:8 * D].view("<i8")
    lo = st[8 * D:16 * D].view("<u8")
    hi = st[16 * D:].view("<u8")
    cat["s1"] = [int(v) for v in s1]
    cat["s2"] = [int(a) + (int(c) << 64) for a, c in zip(lo, hi)]
    cat["n_q"], cat["n_r"] = n_q, n_r
    return cat


def unpack_record(rec: np.ndarray, D: int, bk: int, bv: int):
    return unpack_records(rec.reshape(1, -1), D, bk, bv)


def lengths(buf: np.ndarray, B: int, Hkv: int) -> np.ndarray:
    return buf[: B * Hkv * 8].view("<i4").reshape(B, Hkv, 2).copy()


def unpack_sequence(buf: np.ndarray, cfg: dict, b: int, h: int, n_q: int | None = None, n_r: int | None = None):
    """Logical arrays of (b, h): codes/params of the quantized region plus the window.

    ``buf`` is the whole cache buffer as uint8 on the host; cfg has B, Hkv, D, bk, bv, R,
    max_tokens (and NS, default 0). Lengths default to the ones stored in the buffer. The
    sinks (positions, fp16 rows) are returned when the sequence has quantized tokens.
    """
    B, Hkv, D, bk, bv, R = (cfg[k] for k in ("B", "Hkv", "D", "bk", "bv", "R"))
    NS = cfg.get("NS", 0)
    skvq = cfg.get("method", 0) == 1
    o = offsets(B, Hkv, D, bk, bv, R, cfg["max_tokens"], NS, skvq)
    L = lengths(buf, B, Hkv)
    n_q = int(L[b, h, 0]) if n_q is None else n_q
    n_r = int(L[b, h, 1]) if n_r is None else n_r
    ng = n_q // 32
    start = o["records"] + (b * Hkv + h) * o["max_groups"] * o["record_bytes"]
    recs = buf[start:start + ng * o["record_bytes"]].reshape(ng, o["record_bytes"])
    cat = unpack_records(recs, D, bk, bv, skvq)
    w0 = ((b * Hkv + h) * R) * D * 2
    wk = buf[o["window_k"] + w0:o["window_k"] + w0 + R * D * 2].view(np.float16).reshape(R, D)[:n_r]
    wv = buf[o["window_v"] + w0:o["window_v"] + w0 + R * D * 2].view(np.float16).reshape(R, D)[:n_r]
    cat["wk"] = wk.copy()
    cat["wv"] = wv.copy()
    i = b * Hkv + h
    pos = buf[o["sink_pos"] + i * NS * 4:o["sink_pos"] + (i + 1) * NS * 4].view("<i4")
    ns = 0  # the sinks present: the leading non-negative positions
    while ns < NS and pos[ns] >= 0:
        ns += 1
    if skvq and n_q > 0:  # fixed by the first quantized chunk
        pm = buf[o["perm"] + i * 2 * D:o["perm"] + (i + 1) * 2 * D]
        cat["perm_k"], cat["perm_v"] = pm[:D].astype(np.int64), pm[D:].astype(np.int64)
    cat["sink_pos"] = buf[o["sink_pos"] + i * NS * 4:o["sink_pos"] + (i * NS + ns) * 4].view("<i4").astype(np.int64)
    cat["sink_k"] = buf[o["sink_k"] + i * NS * D * 2:o["sink_k"] + (i * NS + ns) * D * 2].view(np.float16).reshape(ns, D).copy()
    cat["sink_v"] = buf[o["sink_v"] + i * NS * D * 2:o["sink_v"] + (i * NS + ns) * D * 2].view(np.float16).reshape(ns, D).copy()
    if "perm_k" in cat:  # SKVQ rows are stored permuted once the permutations exist: back to channel order
        for key, pm_ in (("wk", cat["perm_k"]), ("sink_k", cat["perm_k"]), ("wv", cat["perm_v"]), ("sink_v", cat["perm_v"])):
            nat = np.empty_like(cat[key])
            nat[:, pm_] = cat[key]
            cat[key] = nat
    cat["n_q"], cat["n_r"] = n_q, n_r
    return cat
