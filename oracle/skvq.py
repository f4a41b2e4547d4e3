"""Plain CPU oracle: SKVQ-adapted quantized KV cache (channel reordering + clipped groups).

TEST INFRASTRUCTURE ONLY, under the same rule as ``oracle/kivi.py``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import or call
it. numpy ``float32``/``float16`` arithmetic (IEEE, round-to-nearest-even, one rounding per
operation, no fused multiply-add) for the encoder; attention reuses ``oracle.kivi.attend``
(fp64, the plain softmax definition).

What it follows (VeloxQuant-MLX documentation pages):

* "Changelog", v0.30.0 "New" (SKVQ-adapted): keys and values both quantized in per-token
  groups of channels; the head-dim channels are first permuted so that channels of similar
  dynamic range share a group (one permutation per head, sorted by range, fixed by the first
  flushed chunk; identity when reordering is off); each group's min/max window is shrunk by a
  clip factor alpha picked per group from a grid that contains alpha = 1, by reconstruction
  error, and folded into the stored low end and step (nothing else is stored); a sliding fp16
  window flushed a chunk at a time; the first few tokens kept in fp16 (the sink filter); a
  prefill gives the same cache as the same tokens appended one by one.
* "Changelog", v0.30.0 "Honest scope": first-chunk statistics and a per-group
  reconstruction-MSE grid search stand in for calibration; integer bit widths, fp16 metadata.
* "veloxquant_mlx.cache package", ``KVCacheConfig``: skvq_bits_key / skvq_bits_value 2,
  skvq_group_size 32, skvq_window 128, skvq_n_sink 5, skvq_reorder True, skvq_clip_search
  True, skvq_clip_alpha 1.0.

Readings taken where the pages leave a step open:

* sinks are the first n_sink tokens of the sequence; the window rule applies to the tokens
  after them: with S' = S - n_sink >= 1 of those, the window holds ((S' - 1) mod R) + 1 and
  the rest are quantized; a full window is flushed whole when the next token arrives, and
  its R tokens are the chunk;
* the permutation of K (and separately of V) is a stable ascending sort of the channels by
  their range over the first chunk, range = fp32(max) - fp32(min) (one rounding);
* a group is 32 consecutive permuted channels of one token: group k holds channels
  perm[32k], ..., perm[32k + 31], in that order;
* "shrunk by alpha" keeps the window's centre: with c = (1 - alpha) / 2 and
  d = (hi - lo) * c, the clipped window is [lo + d, hi - d]; the grid is alpha = 1 - k/20,
  k = 0..10, i.e. c_k = fp32(k) / fp32(40); with the search off, c = (1 - alpha) * 0.5 in
  fp32 for the configured alpha;
* per candidate: scale16 = fp16((hi' - lo') / L), zero16 = fp16(lo'), codes from the stored
  values exactly as in KIVI (inv = 1/scale once, clamp(rint((x - zero) * inv), 0, L), all
  zero when the stored scale is 0); the error is the fp32 sum over the group's 32 elements,
  in group order, of (x - (code * scale + zero))^2, each operation rounded; the candidate with
  the smallest error wins and ties go to the smaller k (alpha = 1 first).
"""
from __future__ import annotations

import numpy as np

from oracle.kivi import F16, F32, F64, window_split

N_CLIP = 11


def clip_fractions() -> list:
    """c_k = (1 - alpha_k) / 2 for the grid alpha_k = 1 - k/20: fp32(k) / fp32(40)."""
    return [F32(k) / F32(40) for k in range(N_CLIP)]


def fixed_clip_fraction(alpha: float) -> list:
    return [(F32(1.0) - F32(alpha)) * F32(0.5)]


def channel_permutation(X: np.ndarray) -> np.ndarray:
    """Channels of fp16 ``X[T, D]`` in ascending order of their range over the T rows
    (fp32 max minus fp32 min, one rounding); equal ranges keep channel order."""
    x = X.astype(F32)
    rng = x.max(axis=0) - x.min(axis=0)
    return np.argsort(rng, kind="stable")


def clipped_group_quant(x: np.ndarray, bits: int, fracs) -> tuple:
    """Quantize every group along the last axis of fp16 ``x`` with the clip search.

    Returns ``(codes uint8, scale fp16, zero fp16, k)`` where ``k`` is the index of the chosen
    candidate in ``fracs`` per group.
    """
    if x.dtype != F16:
        raise TypeError("clipped_group_quant expects float16 input")
    levels = F32(2 ** bits - 1)
    x32 = x.astype(F32)
    lo = x32.min(axis=-1) + F32(0.0)
    hi = x32.max(axis=-1) + F32(0.0)
    best = None
    for k, c in enumerate(fracs):
        d = (hi - lo) * F32(c)
        lo_c = lo + d
        hi_c = hi - d
        scale16 = ((hi_c - lo_c) / levels).astype(F16)
        zero16 = lo_c.astype(F16)
        s = scale16.astype(F32)
        z = zero16.astype(F32)
        nonzero = s != F32(0.0)
        inv = np.zeros_like(s)
        inv[nonzero] = F32(1.0) / s[nonzero]
        t = (x32 - z[..., None]) * inv[..., None]
        codes = np.clip(np.rint(t), F32(0.0), levels)
        codes = np.where(nonzero[..., None], codes, F32(0.0))
        xh = codes * s[..., None] + z[..., None]
        err = np.zeros(x.shape[:-1], F32)
        for i in range(x.shape[-1]):
            diff = x32[..., i] - xh[..., i]
            err = err + diff * diff
        if best is None:
            best = [codes, scale16, zero16, np.zeros(x.shape[:-1], np.int64), err]
            continue
        better = err < best[4]
        best[0] = np.where(better[..., None], codes, best[0])
        best[1] = np.where(better, scale16, best[1])
        best[2] = np.where(better, zero16, best[2])
        best[3] = np.where(better, k, best[3])
        best[4] = np.where(better, err, best[4])
    return best[0].astype(np.uint8), best[1].astype(F16), best[2].astype(F16), best[3]


def encode_block(X: np.ndarray, perm: np.ndarray, bits: int, fracs, g: int = 32):
    """Per-token groups of g permuted channels of fp16 ``X[T, D]``: codes [T, D] in permuted
    channel order, scale and zero [T, D/g], chosen clip index [T, D/g]."""
    T, D = X.shape
    if D % g:
        raise ValueError("head dim must be a multiple of the group size")
    Xp = np.ascontiguousarray(X[:, perm])
    c, s, z, k = clipped_group_quant(Xp.reshape(T, D // g, g), bits, fracs)
    return c.reshape(T, D), s, z, k


def decode_block(codes, scale, zero, perm, g: int = 32) -> np.ndarray:
    """x_hat [T, D] in the original channel order, fp64."""
    T, D = codes.shape
    xp = codes.astype(F64).reshape(T, D // g, g) * scale.astype(F64)[..., None] + zero.astype(F64)[..., None]
    out = np.empty((T, D), F64)
    out[:, perm] = xp.reshape(T, D)
    return out


class SkvqSequence:
    """One (sequence, KV head) cache: fp16 sinks, quantized chunks, fp16 window."""

    def __init__(self, D: int, key_bits: int, value_bits: int, g: int = 32, R: int = 128, n_sink: int = 5,
                 reorder: bool = True, clip_search: bool = True, clip_alpha: float = 1.0):
        if R % g or D % g:
            raise ValueError("R and D must be multiples of g")
        self.D, self.bk, self.bv, self.g, self.R, self.n_sink = D, key_bits, value_bits, g, R, n_sink
        self.reorder = reorder
        self.fracs = clip_fractions() if clip_search else fixed_clip_fraction(clip_alpha)
        self.sink_k = np.zeros((0, D), F16)
        self.sink_v = np.zeros((0, D), F16)
        self.perm_k = self.perm_v = None
        self.kc = np.zeros((0, D), np.uint8)
        self.vc = np.zeros((0, D), np.uint8)
        self.ks = np.zeros((0, D // g), F16)
        self.kz = np.zeros((0, D // g), F16)
        self.vs = np.zeros((0, D // g), F16)
        self.vz = np.zeros((0, D // g), F16)
        self.kk = np.zeros((0, D // g), np.int64)  # chosen clip indices (for the pins)
        self.vk = np.zeros((0, D // g), np.int64)
        self.wk = np.zeros((0, D), F16)
        self.wv = np.zeros((0, D), F16)

    @property
    def n_q(self) -> int:
        return self.kc.shape[0]

    @property
    def n_r(self) -> int:
        return self.wk.shape[0]

    def _quantize(self, K: np.ndarray, V: np.ndarray):
        if self.perm_k is None:
            first_k, first_v = K[:self.R], V[:self.R]  # the first chunk fixes the permutations
            ident = np.arange(self.D)
            self.perm_k = channel_permutation(first_k) if self.reorder else ident
            self.perm_v = channel_permutation(first_v) if self.reorder else ident
        c, s, z, k = encode_block(K, self.perm_k, self.bk, self.fracs, self.g)
        self.kc, self.ks, self.kz, self.kk = (np.concatenate([a, b]) for a, b in
                                              ((self.kc, c), (self.ks, s), (self.kz, z), (self.kk, k)))
        c, s, z, k = encode_block(V, self.perm_v, self.bv, self.fracs, self.g)
        self.vc, self.vs, self.vz, self.vk = (np.concatenate([a, b]) for a, b in
                                              ((self.vc, c), (self.vs, s), (self.vz, z), (self.vk, k)))

    def prefill(self, K: np.ndarray, V: np.ndarray):
        if self.n_q or self.n_r or self.sink_k.shape[0]:
            raise ValueError("prefill needs an empty cache")
        K, V = K.astype(F16), V.astype(F16)
        ns = min(self.n_sink, K.shape[0])
        self.sink_k, self.sink_v = K[:ns].copy(), V[:ns].copy()
        n_q, _ = window_split(K.shape[0] - ns, self.R)
        if n_q:
            self._quantize(K[ns:ns + n_q], V[ns:ns + n_q])
        self.wk, self.wv = K[ns + n_q:].copy(), V[ns + n_q:].copy()

    def append(self, k: np.ndarray, v: np.ndarray):
        k, v = k.astype(F16)[None], v.astype(F16)[None]
        if self.sink_k.shape[0] < self.n_sink:
            self.sink_k = np.concatenate([self.sink_k, k])
            self.sink_v = np.concatenate([self.sink_v, v])
            return
        if self.n_r == self.R:
            self._quantize(self.wk, self.wv)
            self.wk, self.wv = self.wk[:0], self.wv[:0]
        self.wk = np.concatenate([self.wk, k])
        self.wv = np.concatenate([self.wv, v])

    def keys_hat(self) -> np.ndarray:
        kq = decode_block(self.kc, self.ks, self.kz, self.perm_k, self.g) if self.n_q else np.zeros((0, self.D))
        return np.concatenate([self.sink_k.astype(F64), kq, self.wk.astype(F64)])

    def values_hat(self) -> np.ndarray:
        vq = decode_block(self.vc, self.vs, self.vz, self.perm_v, self.g) if self.n_q else np.zeros((0, self.D))
        return np.concatenate([self.sink_v.astype(F64), vq, self.wv.astype(F64)])
