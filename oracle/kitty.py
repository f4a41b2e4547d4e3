"""Plain CPU oracle: Kitty mixed-precision key channels over a KIVI-style cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything under ``oracle/``. It is deliberately slow and plain.

What it follows (VeloxQuant-MLX documentation pages):

* "Changelog", v0.11.0 "New" (Kitty): key channels are ranked by their online (running)
  per-channel variance; the top quarter of them is quantized to 4 bits and the rest to 2
  bits with asymmetric group quantization; values stay in fp16; no calibration.
* "Algorithm Overview", the method list (Kitty: dynamic channel-wise mixed precision,
  2.5-bit effective key precision) and the method table (Kitty: values fp16).
* "veloxquant_mlx.cache package", ``KVCacheConfig``: ``kitty_hi_fraction = 0.25``,
  ``kitty_hi_bit = 4``, ``kitty_lo_bit = 2``, ``kitty_group_size = 32``.
* "Changelog", v0.42.0 "Added": the fused group-affine decode serves the Kitty family too,
  with codes plus a per-group (scale, zero); attention is the plain softmax over the
  reconstructed keys (``oracle.kivi.attend``).

Readings taken where the pages leave a step open:

* a key group is g = 32 consecutive tokens of one channel (KIVI's per-channel key groups);
  it is quantized by KIVI's min/max rule (``oracle.kivi.quantize_groups``) at the bit width
  its channel holds for that group;
* which channels hold the high width is decided once per key group, when the group is
  quantized, from the variance of every channel over all key tokens of the sequence up to
  the end of that group (the running accumulator): the n_hi channels of largest variance get
  hi_bits, the others lo_bits; between equal variances the lower channel index wins;
* the variance is the exact population variance of the fp16 key values. It is kept as two
  exact integer sums per channel, s1 = sum X and s2 = sum X^2 with X = x * 2^24 (an integer
  for every finite fp16 x), and channels are compared by n * s2 - s1^2 = n^2 * variance;
* n_hi = round(hi_fraction * D) channels (32 of 128 at the default quarter);
* values are stored as their fp16 inputs;
* the fp16 residual window and its flush follow KIVI's window rule (``oracle.kivi``); a
  flush of R tokens quantizes R/g groups, each ranked with the accumulator at its own end,
  so a prefill equals the same tokens appended one by one.
"""
from __future__ import annotations

import numpy as np

from oracle import kivi

F16 = np.float16
F64 = np.float64
X_SHIFT = 24  # fp16 values are integer multiples of 2^-24


def n_hi_of(hi_fraction: float, D: int) -> int:
    """Channels at the high width for a fraction of D (half rounds up)."""
    if not 0.0 <= hi_fraction <= 1.0:
        raise ValueError("hi_fraction must be in [0, 1]")
    return int(np.floor(hi_fraction * D + 0.5))


def key_ints(K: np.ndarray) -> np.ndarray:
    """Exact integers X = x * 2^24 of fp16 ``K`` (|X| < 2^40), as int64."""
    if K.dtype != F16:
        raise TypeError("key_ints expects float16 input")
    x = K.astype(F64) * F64(2.0 ** X_SHIFT)  # exact: an fp16 value times a power of two
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite key")
    return x.astype(np.int64)


class RunningMoments:
    """Exact running sums of X and X^2 per channel over the key tokens seen so far."""

    def __init__(self, D: int):
        self.n = 0
        self.s1 = [0] * D
        self.s2 = [0] * D

    def add(self, K: np.ndarray):
        X = key_ints(K).astype(object)  # Python integers: no overflow
        self.n += K.shape[0]
        for d in range(K.shape[1]):
            col = X[:, d]
            self.s1[d] += int(col.sum())
            self.s2[d] += int((col * col).sum())

    def spread(self) -> list[int]:
        """n * s2 - s1^2 per channel: n^2 times the population variance, exactly."""
        return [self.n * a - b * b for a, b in zip(self.s2, self.s1)]


def rank_hi(spread: list[int], n_hi: int) -> np.ndarray:
    """Boolean mask of the n_hi channels of largest spread (lower index first on ties)."""
    D = len(spread)
    order = sorted(range(D), key=lambda d: (-spread[d], d))
    mask = np.zeros(D, bool)
    mask[order[:n_hi]] = True
    return mask


def encode_key_group(Kg: np.ndarray, hi: np.ndarray, hi_bits: int, lo_bits: int):
    """One key group ``Kg[g, D]`` (fp16): channel d quantized over its g tokens at hi_bits
    where ``hi[d]``, else lo_bits. Returns codes [g, D] (uint8), scale [D], zero [D] (fp16)."""
    g, D = Kg.shape
    codes = np.zeros((g, D), np.uint8)
    scale = np.zeros(D, F16)
    zero = np.zeros(D, F16)
    for sel, bits in ((hi, hi_bits), (~hi, lo_bits)):
        if not sel.any():
            continue
        c, s, z = kivi.quantize_groups(np.ascontiguousarray(Kg[:, sel].T), bits)  # groups along tokens
        codes[:, sel] = c.T
        scale[sel] = s
        zero[sel] = z
    return codes, scale, zero


class KittySequence:
    """One (sequence, KV head) cache: Kitty key groups, fp16 values, the fp16 window."""

    def __init__(self, D: int, n_hi: int, hi_bits: int = 4, lo_bits: int = 2, g: int = 32, R: int = 32):
        if R % g:
            raise ValueError("R must be a multiple of g")
        if not 0 <= n_hi <= D:
            raise ValueError("n_hi must be in [0, D]")
        self.D, self.n_hi, self.hb, self.lb, self.g, self.R = D, n_hi, hi_bits, lo_bits, g, R
        self.mom = RunningMoments(D)  # over the quantized tokens
        self.kc = np.zeros((0, D), np.uint8)
        self.ks = np.zeros((0, D), F16)
        self.kz = np.zeros((0, D), F16)
        self.khi = np.zeros((0, D), bool)
        self.vq = np.zeros((0, D), F16)
        self.wk = np.zeros((0, D), F16)
        self.wv = np.zeros((0, D), F16)

    @property
    def n_q(self) -> int:
        return self.kc.shape[0]

    @property
    def n_r(self) -> int:
        return self.wk.shape[0]

    def _quantize(self, K: np.ndarray, V: np.ndarray):
        g = self.g
        if K.shape[0] % g:
            raise ValueError("a quantized block is a whole number of groups")
        for j in range(K.shape[0] // g):
            Kg = K[j * g:(j + 1) * g]
            self.mom.add(Kg)  # the accumulator at the end of this group
            hi = rank_hi(self.mom.spread(), self.n_hi)
            c, s, z = encode_key_group(Kg, hi, self.hb, self.lb)
            self.kc = np.concatenate([self.kc, c])
            self.ks = np.concatenate([self.ks, s[None]])
            self.kz = np.concatenate([self.kz, z[None]])
            self.khi = np.concatenate([self.khi, hi[None]])
        self.vq = np.concatenate([self.vq, V])

    def encode(self, K: np.ndarray, V: np.ndarray):
        """Quantize a block of tokens (a multiple of g) after the quantized region."""
        if self.n_r:
            raise ValueError("encode needs an empty window")
        self._quantize(K.astype(F16), V.astype(F16))

    def prefill(self, K: np.ndarray, V: np.ndarray):
        if self.n_q or self.n_r:
            raise ValueError("prefill needs an empty cache")
        n_q, _ = kivi.window_split(K.shape[0], self.R)
        self._quantize(K[:n_q].astype(F16), V[:n_q].astype(F16))
        self.wk = K[n_q:].astype(F16).copy()
        self.wv = V[n_q:].astype(F16).copy()

    def append(self, k: np.ndarray, v: np.ndarray):
        if self.n_r == self.R:
            self._quantize(self.wk, self.wv)
            self.wk = self.wk[:0]
            self.wv = self.wv[:0]
        self.wk = np.concatenate([self.wk, k.astype(F16)[None]])
        self.wv = np.concatenate([self.wv, v.astype(F16)[None]])

    def keys_hat(self) -> np.ndarray:
        """Every cached key as attention sees it: code * scale + zero per key group, then the
        window rows."""
        kq = kivi.dequantize_keys(self.kc, self.ks, self.kz, self.g) if self.n_q else np.zeros((0, self.D))
        return np.concatenate([kq, self.wk.astype(F64)])

    def values_hat(self) -> np.ndarray:
        return np.concatenate([self.vq.astype(F64), self.wv.astype(F64)])

    def key_bits_per_element(self) -> float:
        """Average stored key code width (parameters not counted)."""
        return (self.n_hi * self.hb + (self.D - self.n_hi) * self.lb) / self.D
