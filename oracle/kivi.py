"""Plain CPU oracle: KIVI-style group-affine KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything under ``oracle/``. It is deliberately slow and plain:
numpy ``float32``/``float16`` arithmetic (IEEE, round-to-nearest-even, one rounding per
operation, no fused multiply-add) for the encoder, and ``float64`` for attention.

What it follows (VeloxQuant-MLX documentation pages):

* "Changelog", v0.8.0 "New" (KIVI): asymmetric group quantization with no codebook and no
  rotation; keys are grouped per channel, values per token; the cache keeps an fp16
  residual window of recent tokens.
* "Changelog", v0.42.0 "Added" (fused group-affine decode + attention): codes plus a
  per-group (scale, zero) taken from the group minimum and maximum; k_hat / v_hat are
  rebuilt from them and attended with an online softmax that accumulates in fp32, giving the
  same result as dequantize-then-SDPA.
* "Changelog", v0.30.0 "New" and "Honest scope" (SKVQ): the group parameters are stored as a
  low end and a step ("lo/scale"); bit widths are integers and metadata is fp16.
* "Changelog", v0.28.0 "New" (NSNQuant): the residual buffer is flushed through the
  quantizer a whole chunk at a time, which the page calls KIVI's idiom.
* "Algorithm Overview", "Method families / Zero-calibration methods": KIVI shares the plain
  min/max group quantizer.
* "veloxquant_mlx.cache package", ``KVCacheConfig``: ``kivi_group_size`` defaults to 32 and
  the cache has a ``residual_length`` window; the standalone ``attend(q)`` returns fp16.
* "Changelog", v0.9.0 "New" (KIVI-Sink): tokens whose key L2 norm stands out are kept in
  fp16 and left out of the statistics the quantization parameters come from;
  ``n_sink_tokens = 0`` is plain KIVI.

Readings taken where the pages leave a step open:

* zero = group minimum, stored fp16 (exact, it is an fp16 input value);
* scale = (max - min) / (2**b - 1), fp32 subtract then fp32 divide, rounded once to fp16;
* codes use the *stored* fp16 scale: inv = 1/scale (fp32 divide, once per group), then
  c = clamp(rint((x - zero) * inv), 0, 2**b - 1), sub then mul, ties to even;
* a group whose stored scale is 0 (constant group, or a range that underflows fp16)
  gets all-zero codes;
* min and max are canonicalised with ``+ 0.0`` so that -0 becomes +0;
* key groups run along tokens from token 0 of the quantized region, value groups along
  channels from channel 0;
* window rule: with S tokens seen (S >= 1) the window holds ((S - 1) mod R) + 1 tokens and
  the rest are quantized; a full window is flushed whole on the next append.
* sinks (KIVI-Sink): the n tokens of largest key norm, chosen per (sequence, KV head) once,
  by the first step that quantizes tokens of it (a prefill or encode with a quantized part,
  or the first window flush), among the tokens that step quantizes; the squared norm is an
  fp32 sum of fp32 squares taken channel by channel in order; equal norms go to the earlier
  token. A sink keeps its fp16 key and value rows; its quantized slot stays in the cache
  (codes from the group parameters, clamped) but attention uses the fp16 rows in its place.
  How a device marks that slot is a storage choice of the device layout, not part of what
  the method computes: the oracle's value parameters are the plain ones, and the sinks are
  its list of positions.
"""
from __future__ import annotations

import numpy as np

F16 = np.float16
F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------------------
# Group quantizer (one group = the last axis of the input)
# ----------------------------------------------------------------------------------------
def quantize_groups(x: np.ndarray, bits: int, exclude: np.ndarray | None = None):
    """Quantize every group along the last axis of fp16 array ``x`` to ``bits``-bit codes.

    Follows the min/max group quantizer of "Changelog" v0.8.0 (KIVI) and v0.42.0 (codes
    plus per-group (scale, zero)), with zero stored as the group low end ("Changelog"
    v0.30.0, lo/scale) in fp16 metadata ("Changelog" v0.30.0, Honest scope).

    ``exclude`` (boolean, x's shape) marks elements left out of the min and max ("Changelog"
    v0.9.0, KIVI-Sink); they are still given codes from the group's parameters. Every group
    must keep at least one element.

    Returns ``(codes uint8 with x's shape, scale fp16, zero fp16)``; the parameter arrays
    have x's shape without its last axis.
    """
    if x.dtype != F16:
        raise TypeError("quantize_groups expects float16 input")
    if bits not in (2, 3, 4, 5, 6, 7, 8):
        # b = 1 is excluded: a range of up to 2 * 65504 would overflow an fp16 scale
        raise ValueError("bits must be an integer in [2, 8]")
    levels = F32(2 ** bits - 1)
    x32 = x.astype(F32)  # exact widening
    if exclude is None:
        lo = x32.min(axis=-1) + F32(0.0)  # + 0.0 turns -0 into +0
        hi = x32.max(axis=-1) + F32(0.0)
    else:
        if np.any(np.all(exclude, axis=-1)):
            raise ValueError("a group with every element excluded has no range")
        lo = np.where(exclude, F32(np.inf), x32).min(axis=-1) + F32(0.0)
        hi = np.where(exclude, F32(-np.inf), x32).max(axis=-1) + F32(0.0)
    s32 = (hi - lo) / levels  # fp32 subtract, fp32 divide
    scale16 = s32.astype(F16)  # one RNE rounding, subnormals kept
    zero16 = lo.astype(F16)  # exact: lo is an fp16 value
    s = scale16.astype(F32)
    nonzero = s != F32(0.0)
    inv = np.zeros_like(s)
    inv[nonzero] = F32(1.0) / s[nonzero]  # fp32 IEEE divide, once per group
    t = (x32 - lo[..., None]) * inv[..., None]  # fp32 subtract, then fp32 multiply
    c = np.clip(np.rint(t), F32(0.0), levels)  # rint: round half to even
    c = np.where(nonzero[..., None], c, F32(0.0))
    return c.astype(np.uint8), scale16, zero16


def dequantize_groups(codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray) -> np.ndarray:
    """x_hat = code * scale + zero, in float64 (exact for fp16 parameters and codes < 256)."""
    return codes.astype(F64) * scale16.astype(F64)[..., None] + zero16.astype(F64)[..., None]


# ----------------------------------------------------------------------------------------
# Keys per channel, values per token ("Changelog" v0.8.0, KIVI)
# ----------------------------------------------------------------------------------------
def encode_keys(K: np.ndarray, bits: int, g: int = 32, sinks=()):
    """Per-channel key quantization of an fp16 block ``K[T, D]`` with T a multiple of g.

    A group is g consecutive tokens of one channel. Rows listed in ``sinks`` (positions in
    the block) take no part in their groups' min/max ("Changelog" v0.9.0, KIVI-Sink).
    Returns ``codes[T, D]`` (uint8), ``scale[T/g, D]`` and ``zero[T/g, D]`` (fp16).
    """
    T, D = K.shape
    if T % g:
        raise ValueError("key block length must be a multiple of the group size")
    blk = K.reshape(T // g, g, D).transpose(0, 2, 1)  # [T/g, D, g]: group along tokens
    exclude = None
    if len(sinks):
        rows = np.zeros(T, bool)
        rows[np.asarray(sinks)] = True
        exclude = np.broadcast_to(rows.reshape(T // g, 1, g), blk.shape)
    c, s, z = quantize_groups(np.ascontiguousarray(blk), bits, exclude)
    return np.ascontiguousarray(c.transpose(0, 2, 1).reshape(T, D)), s, z


def encode_values(V: np.ndarray, bits: int, g: int = 32):
    """Per-token value quantization of an fp16 block ``V[T, D]`` with D a multiple of g.

    A group is g consecutive channels of one token, so a sink token ("Changelog" v0.9.0,
    KIVI-Sink) changes no value group's statistics: its own groups are quantized like any
    other row. Returns ``codes[T, D]`` (uint8), ``scale[T, D/g]`` and ``zero[T, D/g]`` (fp16).
    """
    T, D = V.shape
    if D % g:
        raise ValueError("head dim must be a multiple of the group size")
    c, s, z = quantize_groups(V.reshape(T, D // g, g), bits)
    return c.reshape(T, D), s, z


# ----------------------------------------------------------------------------------------
# Sink tokens ("Changelog" v0.9.0, KIVI-Sink)
# ----------------------------------------------------------------------------------------
def key_norms_sq(K: np.ndarray) -> np.ndarray:
    """Squared L2 norm of every row of fp16 ``K[T, D]``: in fp32, channel 0 first, each
    square rounded to fp32 and then added (one rounding per operation, no fused multiply-add)."""
    acc = np.zeros(K.shape[0], F32)
    for d in range(K.shape[1]):
        x = K[:, d].astype(F32)
        acc = acc + x * x
    return acc


def select_sinks(K: np.ndarray, n: int) -> np.ndarray:
    """Row positions (ascending) of the ``n`` rows of ``K`` with the largest key norm;
    between equal norms the earlier row wins."""
    n = min(int(n), K.shape[0])
    if n <= 0:
        return np.zeros(0, np.int64)
    nrm = key_norms_sq(K)
    order = np.lexsort((np.arange(len(nrm)), -nrm.astype(F64)))  # by -norm, then by position
    return np.sort(order[:n]).astype(np.int64)


def dequantize_keys(codes, scale, zero, g: int = 32) -> np.ndarray:
    T, D = codes.shape
    blk = codes.reshape(T // g, g, D).transpose(0, 2, 1)  # [T/g, D, g]
    x = dequantize_groups(blk, scale, zero)
    return x.transpose(0, 2, 1).reshape(T, D)


def dequantize_values(codes, scale, zero, g: int = 32) -> np.ndarray:
    T, D = codes.shape
    return dequantize_groups(codes.reshape(T, D // g, g), scale, zero).reshape(T, D)


# ----------------------------------------------------------------------------------------
# Window rule (fp16 residual window, chunk flush)
# ----------------------------------------------------------------------------------------
def window_split(S: int, R: int) -> tuple[int, int]:
    """(quantized tokens, window tokens) after S tokens, for a window of capacity R.

    The window keeps the newest tokens in fp16 ("Changelog" v0.8.0, KIVI) and is flushed a
    whole chunk at a time ("Changelog" v0.28.0); a flush happens when a token arrives at a
    full window, so after S >= 1 tokens the window holds ((S - 1) mod R) + 1 of them.
    """
    if S < 0 or R < 1:
        raise ValueError("bad sizes")
    if S == 0:
        return 0, 0
    n_r = (S - 1) % R + 1
    return S - n_r, n_r


class KiviSequence:
    """One (sequence, KV head) cache: quantized groups plus the fp16 window.

    The state machine is the plain reading of the pages: ``prefill`` of S tokens quantizes
    the first S - n_r tokens and keeps the rest in the window; ``append`` flushes a full
    window (all R tokens, R/g key groups) through the quantizer before storing the new token.
    """

    def __init__(self, D: int, key_bits: int, value_bits: int, g: int = 32, R: int = 32, n_sink: int = 0):
        if R % g or D % g:
            raise ValueError("R and D must be multiples of g")
        if not 0 <= n_sink < g:
            raise ValueError("n_sink must be in [0, g)")
        self.D, self.bk, self.bv, self.g, self.R = D, key_bits, value_bits, g, R
        self.n_sink = n_sink
        self.sink_pos = np.zeros(0, np.int64)  # token positions, ascending
        self.sink_k = np.zeros((0, D), F16)
        self.sink_v = np.zeros((0, D), F16)
        self.kc = np.zeros((0, D), np.uint8)
        self.ks = np.zeros((0, D), F16)
        self.kz = np.zeros((0, D), F16)
        self.vc = np.zeros((0, D), np.uint8)
        self.vs = np.zeros((0, D // g), F16)
        self.vz = np.zeros((0, D // g), F16)
        self.wk = np.zeros((0, D), F16)
        self.wv = np.zeros((0, D), F16)

    @property
    def n_q(self) -> int:
        return self.kc.shape[0]

    @property
    def n_r(self) -> int:
        return self.wk.shape[0]

    def _quantize(self, K: np.ndarray, V: np.ndarray):
        local = ()
        if self.n_q == 0 and self.n_sink and K.shape[0]:
            # the first step that quantizes tokens chooses the sinks among them
            local = select_sinks(K, self.n_sink)
            self.sink_pos = local.copy()  # nothing is quantized yet: block rows = positions
            self.sink_k = K[local].copy()
            self.sink_v = V[local].copy()
        c, s, z = encode_keys(K, self.bk, self.g, local)
        self.kc = np.concatenate([self.kc, c])
        self.ks = np.concatenate([self.ks, s])
        self.kz = np.concatenate([self.kz, z])
        c, s, z = encode_values(V, self.bv, self.g)
        self.vc = np.concatenate([self.vc, c])
        self.vs = np.concatenate([self.vs, s])
        self.vz = np.concatenate([self.vz, z])

    def encode(self, K: np.ndarray, V: np.ndarray):
        """Quantize a block of tokens (a multiple of g) after the quantized region."""
        if self.n_r:
            raise ValueError("encode needs an empty window")
        self._quantize(K.astype(F16), V.astype(F16))

    def prefill(self, K: np.ndarray, V: np.ndarray):
        if self.n_q or self.n_r:
            raise ValueError("prefill needs an empty cache")
        n_q, _ = window_split(K.shape[0], self.R)
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
        """Every cached key as attention sees it: reconstructed, except sinks and window rows."""
        kq = dequantize_keys(self.kc, self.ks, self.kz, self.g) if self.n_q else np.zeros((0, self.D))
        kq[self.sink_pos] = self.sink_k.astype(F64)
        return np.concatenate([kq, self.wk.astype(F64)])

    def values_hat(self) -> np.ndarray:
        vq = dequantize_values(self.vc, self.vs, self.vz, self.g) if self.n_q else np.zeros((0, self.D))
        vq[self.sink_pos] = self.sink_v.astype(F64)
        return np.concatenate([vq, self.wv.astype(F64)])


# ----------------------------------------------------------------------------------------
# Decode attention over the reconstructed cache, in float64
# ----------------------------------------------------------------------------------------
def attend(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, sm_scale: float = 1.0) -> np.ndarray:
    """softmax(sm_scale * k_hat @ q) @ v_hat for one query vector, in float64.

    This is the plain definition the fused kernel of "Changelog" v0.42.0 reproduces with
    an online softmax: scores over every cached token, max-subtracted softmax, weighted sum.
    """
    if k_hat.shape[0] == 0:
        raise ValueError("attention over an empty cache is undefined")
    s = (k_hat @ q.astype(F64)) * F64(sm_scale)
    s = s - s.max()
    p = np.exp(s)
    return (p @ v_hat) / p.sum()


def attend_causal(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, sm_scale: float = 1.0) -> np.ndarray:
    """S_q queries ``q[S_q, D]`` that are the cache's newest S_q tokens (rows in token order):
    query j sees the first T - (S_q - 1 - j) rows, so its own token and everything before it.

    Multi-query attend over the quantized cache (speculative decode; the pages pair the fused
    decode kernel with multi-token work in "Changelog" v0.40.0 "Added", RaBitQ): each query is
    the plain decode attention of ``attend`` over its causal prefix.
    """
    S_q, T = q.shape[0], k_hat.shape[0]
    if S_q > T:
        raise ValueError("more queries than cached tokens")
    out = np.zeros((S_q, v_hat.shape[1]), F64)
    for j in range(S_q):
        lim = T - (S_q - 1 - j)
        out[j] = attend(q[j], k_hat[:lim], v_hat[:lim], sm_scale)
    return out


def kv_head_of(h_q: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Query head h_q reads KV head floor(h_q * H_kv / H_q) (contiguous GQA blocks)."""
    return (h_q * n_kv_heads) // n_q_heads


def decode_attend(q: np.ndarray, seqs, sm_scale: float = 1.0) -> np.ndarray:
    """Attention for a batch: ``q[B, H_q, D]``, ``seqs[b][h_kv]`` KiviSequence objects."""
    B, Hq, D = q.shape
    Hkv = len(seqs[0])
    out = np.zeros((B, Hq, D), F64)
    for b in range(B):
        cache = {}
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            if hk not in cache:
                cache[hk] = (seqs[b][hk].keys_hat(), seqs[b][hk].values_hat())
            out[b, h] = attend(q[b, h], *cache[hk], sm_scale)
    return out
