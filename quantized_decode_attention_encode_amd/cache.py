"""Python binding of the C ABI: argument marshalling only.

Every step of the hot path runs in the HIP kernels of libkvq.so. PyTorch supplies device
memory (tensors) and the stream; this module checks shapes and dtypes, passes raw device
pointers, and turns status codes into KVQError.

The functions carry the C names (kvq_encode, kvq_prefill, kvq_append, kvq_decode_attend,
...); KVQCache bundles a cache buffer, its handle and a decode workspace.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import KVQ_OK, Config, KVQError, LayoutInfo, check, lib

__all__ = ["KVQCache", "KVQError", "make_config", "kvq_probe", "kvq_cache_bytes", "kvq_layout",
           "kvq_workspace_bytes", "kvq_encode", "kvq_prefill", "kvq_append", "kvq_decode_attend",
           "kvq_decode_attend_multi", "kvq_decode_attend_noalloc"]


def make_config(batch, n_kv_heads, n_q_heads, head_dim, key_bits=2, value_bits=2, group=32, residual=32,
                max_tokens=4096, n_sink=0, method="kivi", skvq_reorder=True, skvq_clip_search=True,
                skvq_clip_alpha=1.0, kitty_hi_fraction=0.25, kitty_hi_bits=4) -> Config:
    """method "kivi" (n_sink > 0: KIVI-Sink, that many high key-norm tokens per (sequence, KV head)
    kept in fp16), "skvq" (SKVQ-adapted: per-token groups of range-sorted channels with a
    per-group clip search; n_sink first tokens in fp16; residual is its window, 128 by default
    on the pages) or "kitty" (the round(kitty_hi_fraction * head_dim) key channels of largest
    running variance at kitty_hi_bits, the rest at key_bits; values in fp16, so value_bits is
    16 whatever is passed)."""
    methods = {"kivi": _lib.METHOD_KIVI, "skvq": _lib.METHOD_SKVQ, "kitty": _lib.METHOD_KITTY}
    if method not in methods:
        raise ValueError(f"method must be one of {sorted(methods)}, got {method!r}")
    n_hi = 0
    if method == "kitty":
        hi = ctypes.c_int32(0)
        check(lib.kvq_kitty_n_hi(int(head_dim), float(kitty_hi_fraction), ctypes.byref(hi)))
        n_hi = hi.value
        value_bits = 16
    return Config(batch, n_kv_heads, n_q_heads, head_dim, key_bits, value_bits, group, residual, max_tokens,
                  n_sink, methods[method], int(bool(skvq_reorder)), int(bool(skvq_clip_search)),
                  float(skvq_clip_alpha), n_hi, int(kitty_hi_bits))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _i32(values) -> ctypes.Array:
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * len(vals))(*vals)


def _dev(t: torch.Tensor, name: str, dtype=torch.float16) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise KVQError(-1, f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise KVQError(-1, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise KVQError(-1, f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def kvq_probe() -> bool:
    has = ctypes.c_int32(0)
    check(lib.kvq_probe(ctypes.byref(has)))
    return bool(has.value)


def kvq_cache_bytes(cfg: Config) -> int:
    n = lib.kvq_cache_bytes(ctypes.byref(cfg))
    if n == 0:
        check(lib.kvq_config_check(ctypes.byref(cfg)))
    return n


def kvq_layout(cfg: Config) -> LayoutInfo:
    info = LayoutInfo()
    check(lib.kvq_layout(ctypes.byref(cfg), ctypes.byref(info)))
    return info


def kvq_workspace_bytes(cfg: Config, n_split: int = 0) -> int:
    n = lib.kvq_workspace_bytes(ctypes.byref(cfg), int(n_split))
    if n == 0:
        check(lib.kvq_config_check(ctypes.byref(cfg)))
    return n


class KVQCache:
    """One layer's quantized KV cache in a caller-owned (torch) device buffer."""

    def __init__(self, cfg: Config, device="cuda", buffer: torch.Tensor | None = None):
        self.cfg = cfg
        nbytes = kvq_cache_bytes(cfg)
        if buffer is None:
            buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.buffer = buffer
        self.handle = ctypes.c_void_p()
        check(lib.kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(buffer.data_ptr()), buffer.numel(),
                                   ctypes.byref(self.handle)))
        self._ws = None

    def close(self):
        if self.handle:
            lib.kvq_cache_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lengths(self):
        nq = (ctypes.c_int32 * self.cfg.batch)()
        nr = (ctypes.c_int32 * self.cfg.batch)()
        check(lib.kvq_cache_lengths(self.handle, nq, nr))
        return list(nq), list(nr)

    def reset(self, stream=None):
        check(lib.kvq_reset(self.handle, _stream(stream)))

    def workspace(self, n_split: int = 0, n_query: int = 1) -> torch.Tensor:
        need = kvq_workspace_bytes(self.cfg, n_split) * n_query
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.buffer.device)
        return self._ws

    def profile_enable(self, on: bool = True, launches: int = 1):
        """Time each decode kernel with dispatch-stamped events; events for `launches` calls are
        created up front."""
        check(lib.kvq_profile_enable(self.handle, max(1, int(launches)) if on else 0))

    def profile_read(self):
        ms = ctypes.c_double(0)
        n = ctypes.c_int64(0)
        check(lib.kvq_profile_read(self.handle, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value


def _kv_shape_check(cache: KVQCache, K: torch.Tensor, V: torch.Tensor):
    c = cache.cfg
    if K.dim() != 4 or K.shape[0] != c.batch or K.shape[1] != c.n_kv_heads or K.shape[3] != c.head_dim:
        raise KVQError(-1, f"K must be [B={c.batch}, H_kv={c.n_kv_heads}, T, D={c.head_dim}], got {tuple(K.shape)}")
    if V.shape != K.shape:
        raise KVQError(-1, f"V shape {tuple(V.shape)} differs from K shape {tuple(K.shape)}")


def kvq_encode(cache: KVQCache, K: torch.Tensor, V: torch.Tensor, n_tok, stream=None) -> None:
    """Quantize n_tok[b] tokens of K, V [B, H_kv, T, D] fp16 after each sequence's quantized region."""
    _kv_shape_check(cache, K, V)
    check(lib.kvq_encode(cache.handle, _dev(K, "K"), _dev(V, "V"), K.shape[2], _i32(n_tok), _stream(stream)))


def kvq_encode_block(X: torch.Tensor, bits: int, per_channel: bool, group: int = 32, stream=None):
    """Quantize one fp16 block X [n_tok, D] in groups of `group` (per_channel: along tokens, the
    key rule; else along channels, the value rule). Returns (codes uint8 [n_tok, D], scale fp16,
    zero fp16) with scale/zero [n_tok/group, D] or [n_tok, D/group]."""
    if X.dim() != 2:
        raise KVQError(-1, "X must be [n_tok, D]")
    n_tok, D = X.shape
    pshape = (n_tok // group, D) if per_channel else (n_tok, D // group)
    codes = torch.empty((n_tok, D), dtype=torch.uint8, device=X.device)
    scale = torch.empty(pshape, dtype=torch.float16, device=X.device)
    zero = torch.empty(pshape, dtype=torch.float16, device=X.device)
    check(lib.kvq_encode_block(_dev(X, "X"), n_tok, D, int(bits), int(group), 1 if per_channel else 0,
                               _dev(codes, "codes", torch.uint8), _dev(scale, "scale"), _dev(zero, "zero"),
                               _stream(stream)))
    return codes, scale, zero


def kvq_prefill(cache: KVQCache, K: torch.Tensor, V: torch.Tensor, seq_len, stream=None) -> None:
    """Fill an empty cache with seq_len[b] tokens per sequence (window rule applied)."""
    _kv_shape_check(cache, K, V)
    check(lib.kvq_prefill(cache.handle, _dev(K, "K"), _dev(V, "V"), K.shape[2], _i32(seq_len), _stream(stream)))


def kvq_append(cache: KVQCache, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
    """Append one token per sequence: k, v fp16 [B, H_kv, D]."""
    c = cache.cfg
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (c.batch, c.n_kv_heads, c.head_dim):
            raise KVQError(-1, f"{name} must be [B, H_kv, D] = {(c.batch, c.n_kv_heads, c.head_dim)}")
    check(lib.kvq_append(cache.handle, _dev(k, "k"), _dev(v, "v"), _stream(stream)))


def kvq_decode_attend(cache: KVQCache, q: torch.Tensor, out: torch.Tensor | None = None, sm_scale: float = 1.0,
                      n_split: int = 0, out_fp32: bool = False, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Attention of q [B, H_q, D] fp16 over the quantized cache; returns out [B, H_q, D]."""
    c = cache.cfg
    if tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
        raise KVQError(-1, f"q must be [B, H_q, D] = {(c.batch, c.n_q_heads, c.head_dim)}")
    odt = torch.float32 if out_fp32 else torch.float16
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=odt, device=q.device)
    if tuple(out.shape) != tuple(q.shape):
        raise KVQError(-1, "out must have q's shape")
    if workspace is None:
        workspace = cache.workspace(n_split)
    st = lib.kvq_decode_attend(cache.handle, _dev(q, "q"), _dev(out, "out", odt), 1 if out_fp32 else 0,
                               float(sm_scale), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                               int(n_split), _stream(stream))
    if st != KVQ_OK:
        check(st)
    return out


def kvq_decode_attend_noalloc(cache: KVQCache, q: torch.Tensor, out: torch.Tensor, sm_scale: float = 1.0,
                              n_split: int = 0, out_fp32: bool = False, stream=None) -> torch.Tensor:
    """kvq_decode_attend with no workspace: the split partials live in the library's static
    device scratch. The caller passes q [B, H_q, D] fp16 and a preallocated out of q's shape."""
    c = cache.cfg
    if tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
        raise KVQError(-1, f"q must be [B, H_q, D] = {(c.batch, c.n_q_heads, c.head_dim)}")
    odt = torch.float32 if out_fp32 else torch.float16
    if out is None or tuple(out.shape) != tuple(q.shape):
        raise KVQError(-1, "out must be a preallocated tensor of q's shape")
    st = lib.kvq_decode_attend_noalloc(cache.handle, _dev(q, "q"), _dev(out, "out", odt), 1 if out_fp32 else 0,
                                       float(sm_scale), int(n_split), _stream(stream))
    if st != KVQ_OK:
        check(st)
    return out


def kvq_decode_attend_multi(cache: KVQCache, q: torch.Tensor, out: torch.Tensor | None = None, sm_scale: float = 1.0,
                            n_split: int = 0, out_fp32: bool = False, workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Causal attention of the newest n_query tokens' queries q [B, H_q, n_query, D] fp16 over the
    cache (query j sees the tokens up to and including its own); returns out of q's shape."""
    c = cache.cfg
    if q.dim() != 4 or tuple(q.shape[:2]) != (c.batch, c.n_q_heads) or q.shape[3] != c.head_dim:
        raise KVQError(-1, f"q must be [B, H_q, n_query, D] with B, H_q, D = {(c.batch, c.n_q_heads, c.head_dim)}")
    n_query = int(q.shape[2])
    odt = torch.float32 if out_fp32 else torch.float16
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=odt, device=q.device)
    if tuple(out.shape) != tuple(q.shape):
        raise KVQError(-1, "out must have q's shape")
    if workspace is None:
        workspace = cache.workspace(n_split, n_query)
    st = lib.kvq_decode_attend_multi(cache.handle, _dev(q, "q"), _dev(out, "out", odt), n_query, 1 if out_fp32 else 0,
                                     float(sm_scale), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                     int(n_split), _stream(stream))
    if st != KVQ_OK:
        check(st)
    return out


def kvq_append_decode_attend(cache: KVQCache, k_tok: torch.Tensor, v_tok: torch.Tensor, q: torch.Tensor,
                             out: torch.Tensor | None = None, sm_scale: float = 1.0, n_split: int = 0,
                             out_fp32: bool = False, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_append(k_tok, v_tok) then kvq_decode_attend(q) as one call (one launch unless a window
    is full)."""
    c = cache.cfg
    for name, t in (("k_tok", k_tok), ("v_tok", v_tok)):
        if tuple(t.shape) != (c.batch, c.n_kv_heads, c.head_dim):
            raise KVQError(-1, f"{name} must be [B, H_kv, D] = {(c.batch, c.n_kv_heads, c.head_dim)}")
    if tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
        raise KVQError(-1, f"q must be [B, H_q, D] = {(c.batch, c.n_q_heads, c.head_dim)}")
    odt = torch.float32 if out_fp32 else torch.float16
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=odt, device=q.device)
    if tuple(out.shape) != tuple(q.shape):
        raise KVQError(-1, "out must have q's shape")
    if workspace is None:
        workspace = cache.workspace(n_split)
    st = lib.kvq_append_decode_attend(cache.handle, _dev(k_tok, "k_tok"), _dev(v_tok, "v_tok"), _dev(q, "q"),
                                      _dev(out, "out", odt), 1 if out_fp32 else 0, float(sm_scale),
                                      _dev(workspace, "workspace", torch.uint8), workspace.numel(), int(n_split),
                                      _stream(stream))
    if st != KVQ_OK:
        check(st)
    return out
