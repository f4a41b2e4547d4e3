"""CPU-side checks of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments on the host before anything is launched (no GPU needed).

Validation mirrors the pages' fail-loudly configuration errors ("veloxquant_mlx.cache
package", KVCacheBuilder / KVCacheFactory raising QuantizerConfigError).
"""
import ctypes
import os
import re
import subprocess

import pytest

from quantized_decode_attention_encode_amd import _lib
from quantized_decode_attention_encode_amd._lib import (KVQ_E_CAPACITY, KVQ_E_INVALID, KVQ_E_NODEVICE,
                                                        KVQ_E_UNSUPPORTED, KVQ_E_WORKSPACE, KVQ_OK, Config,
                                                        KVQError, LayoutInfo, lib)
from tests import kvq_unpack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

torch_cuda = False
try:
    import torch

    torch_cuda = torch.cuda.is_available()
except Exception:  # pragma: no cover
    pass


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def cfg(**kw):
    base = dict(batch=2, n_kv_heads=4, n_q_heads=8, head_dim=128, key_bits=2, value_bits=4, group=32,
                residual=32, max_tokens=1024, n_sink=0, method=0, skvq_reorder=1, skvq_clip_search=1,
                skvq_clip_alpha=1.0, kitty_n_hi=0, kitty_hi_bits=4)
    base.update(kw)
    return Config(*(base[f] for f, _ in Config._fields_))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kvq_encode", "kvq_append", "kvq_decode_attend"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvq_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)
    assert set(names) == set(_lib.EXPORTED)


def test_probe_without_gpu_reports_absence():
    has = ctypes.c_int32(7)
    assert lib.kvq_probe(ctypes.byref(has)) == KVQ_OK
    if not torch_cuda:
        assert has.value == 0
    assert lib.kvq_probe(None) == KVQ_E_INVALID


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, KVQ_E_INVALID), ("batch", 257, KVQ_E_INVALID), ("n_kv_heads", 0, KVQ_E_INVALID),
    ("n_q_heads", 6, KVQ_E_INVALID), ("n_q_heads", 12, KVQ_E_UNSUPPORTED), ("head_dim", 96, KVQ_E_UNSUPPORTED),
    ("key_bits", 3, KVQ_E_UNSUPPORTED), ("value_bits", 1, KVQ_E_UNSUPPORTED), ("group", 64, KVQ_E_UNSUPPORTED),
    ("residual", 48, KVQ_E_INVALID), ("residual", 0, KVQ_E_INVALID), ("residual", 288, KVQ_E_INVALID),
    ("max_tokens", 1000, KVQ_E_INVALID), ("max_tokens", 0, KVQ_E_INVALID),
    ("n_sink", -1, KVQ_E_INVALID), ("n_sink", 17, KVQ_E_INVALID), ("method", 3, KVQ_E_UNSUPPORTED),
])
def test_config_validation(field, value, status):
    c = cfg(**{field: value})
    assert lib.kvq_config_check(ctypes.byref(c)) == status
    assert lib.kvq_last_error()  # a message is set
    assert lib.kvq_cache_bytes(ctypes.byref(c)) == 0
    assert lib.kvq_workspace_bytes(ctypes.byref(c), 0) == 0


@pytest.mark.parametrize("D,bk,bv,R,B,H,NS", [(128, 2, 2, 32, 1, 32, 0), (64, 2, 2, 32, 1, 8, 0),
                                              (128, 2, 4, 32, 16, 8, 0), (128, 8, 4, 64, 3, 2, 5),
                                              (64, 4, 8, 128, 5, 3, 16), (128, 2, 2, 32, 2, 4, 1)])
def test_layout_matches_independent_formula(D, bk, bv, R, B, H, NS):
    c = cfg(batch=B, n_kv_heads=H, n_q_heads=H, head_dim=D, key_bits=bk, value_bits=bv, residual=R, max_tokens=2048,
            n_sink=NS)
    info = LayoutInfo()
    assert lib.kvq_layout(ctypes.byref(c), ctypes.byref(info)) == KVQ_OK
    o = kvq_unpack.offsets(B, H, D, bk, bv, R, 2048, NS)
    assert info.lengths_offset == o["lengths"] and info.records_offset == o["records"]
    assert info.record_bytes == o["record_bytes"] == 4 * D * (bk + bv + 2)
    assert (info.rec_key_codes, info.rec_value_codes, info.rec_key_params, info.rec_value_params) == (
        o["rec_key_codes"], o["rec_value_codes"], o["rec_key_params"], o["rec_value_params"])
    assert info.window_k_offset == o["window_k"] and info.window_v_offset == o["window_v"]
    assert info.total_bytes == o["total"] == lib.kvq_cache_bytes(ctypes.byref(c))
    assert info.sync_offset == o["sync"]
    assert (info.sink_pos_offset, info.sink_k_offset, info.sink_v_offset) == (o["sink_pos"], o["sink_k"], o["sink_v"])
    for off in (info.records_offset, info.window_k_offset, info.window_v_offset, info.sink_pos_offset,
                info.sink_k_offset, info.sink_v_offset, info.total_bytes):
        assert off % 256 == 0
    if NS == 0:  # no sink regions: the plain KIVI buffer
        assert info.sink_pos_offset == info.sink_k_offset == info.sink_v_offset == info.total_bytes


@pytest.mark.parametrize("alpha,search,reorder,status", [
    (1.0, 1, 1, KVQ_OK), (0.0, 0, 1, KVQ_E_INVALID), (1.5, 0, 1, KVQ_E_INVALID), (0.8, 0, 0, KVQ_OK),
    (0.8, 2, 1, KVQ_E_INVALID), (0.8, 1, 3, KVQ_E_INVALID)])
def test_skvq_config_validation_and_layout(alpha, search, reorder, status):
    c = cfg(method=1, n_sink=5, residual=128, skvq_clip_alpha=alpha, skvq_clip_search=search, skvq_reorder=reorder)
    assert lib.kvq_config_check(ctypes.byref(c)) == status
    if status != KVQ_OK:
        return
    info = LayoutInfo()
    assert lib.kvq_layout(ctypes.byref(c), ctypes.byref(info)) == KVQ_OK
    o = kvq_unpack.offsets(2, 4, 128, 2, 4, 128, 1024, 5, skvq=True)
    assert (info.perm_offset, info.total_bytes) == (o["perm"], o["total"])
    assert info.total_bytes - info.perm_offset >= 2 * 4 * 2 * 128


@pytest.mark.parametrize("kw,status", [
    (dict(), KVQ_OK), (dict(kitty_n_hi=0), KVQ_OK), (dict(kitty_n_hi=128), KVQ_OK),
    (dict(kitty_n_hi=24), KVQ_E_UNSUPPORTED), (dict(kitty_n_hi=144), KVQ_E_UNSUPPORTED),
    (dict(kitty_n_hi=-16), KVQ_E_UNSUPPORTED), (dict(value_bits=2), KVQ_E_INVALID),
    (dict(key_bits=4), KVQ_E_UNSUPPORTED), (dict(kitty_hi_bits=8), KVQ_E_UNSUPPORTED),
    (dict(n_sink=2), KVQ_E_UNSUPPORTED), (dict(max_tokens=1 << 22), KVQ_OK),
    (dict(max_tokens=(1 << 22) + 32), KVQ_E_UNSUPPORTED)])
def test_kitty_config_validation(kw, status):
    base = dict(method=2, value_bits=16, kitty_n_hi=32)
    base.update(kw)
    c = cfg(**base)
    assert lib.kvq_config_check(ctypes.byref(c)) == status


@pytest.mark.parametrize("D,n_hi,B,H,R", [(128, 32, 1, 32, 32), (64, 16, 3, 2, 64), (128, 0, 2, 4, 32),
                                          (128, 128, 2, 1, 32)])
def test_kitty_layout_matches_independent_formula(D, n_hi, B, H, R):
    c = cfg(method=2, value_bits=16, kitty_n_hi=n_hi, head_dim=D, batch=B, n_kv_heads=H, n_q_heads=H, residual=R,
            max_tokens=2048)
    info = LayoutInfo()
    assert lib.kvq_layout(ctypes.byref(c), ctypes.byref(info)) == KVQ_OK
    o = kvq_unpack.offsets(B, H, D, 2, 2, R, 2048, 0, False, n_hi)
    r = kvq_unpack.kitty_record(D, n_hi)
    assert info.record_bytes == o["record_bytes"] == r["bytes"]
    assert (info.rec_key_codes, info.rec_key_params, info.rec_slot_table, info.rec_value_codes) == (
        0, r["params"], r["table"], r["values"])
    assert (info.kstats_offset, info.total_bytes) == (o["kstats"], o["total"])
    assert info.total_bytes == lib.kvq_cache_bytes(ctypes.byref(c))
    assert info.total_bytes - info.kstats_offset >= B * H * 24 * D


def test_kitty_record_at_the_headline_shape():
    # D = 128, 32 channels at 4 bits: 40 B of key codes per token (2.5 bits a channel), 512 B of
    # key params, 128 B of slot table, 8 KiB of fp16 values
    r = kvq_unpack.kitty_record(128, 32)
    assert (r["words"] * 4, r["params"], r["table"], r["values"], r["bytes"]) == (40, 1280, 1792, 1920, 10112)


def test_skvq_cache_rejects_encode():
    c = cfg(method=1, n_sink=5, residual=128)
    cache = ctypes.c_void_p()
    buf = ctypes.c_void_p(FAKE)
    assert lib.kvq_cache_create(ctypes.byref(c), buf, lib.kvq_cache_bytes(ctypes.byref(c)), ctypes.byref(cache)) == KVQ_OK
    n_tok = (ctypes.c_int32 * 2)(32, 32)
    assert lib.kvq_encode(cache, buf, buf, 64, n_tok, None) == KVQ_E_UNSUPPORTED
    lib.kvq_cache_destroy(cache)


def test_record_is_three_kib_at_the_headline_shape():
    # D=128, 2-bit keys and values: 1 KiB key codes + 1 KiB value codes + 512 B + 512 B params
    assert kvq_unpack.offsets(1, 32, 128, 2, 2, 32, 65536)["record_bytes"] == 3072


def test_workspace_bytes():
    c = cfg()
    assert lib.kvq_workspace_bytes(ctypes.byref(c), 5) == 2 * 8 * 5 * (128 + 4) * 4
    assert lib.kvq_workspace_bytes(ctypes.byref(c), 0) >= lib.kvq_workspace_bytes(ctypes.byref(c), 9)
    assert lib.kvq_workspace_bytes(ctypes.byref(c), -1) == 0


FAKE = 0x7F0000000000  # never dereferenced: every call below fails before any launch


def make_handle(c):
    h = ctypes.c_void_p()
    nbytes = lib.kvq_cache_bytes(ctypes.byref(c))
    assert lib.kvq_cache_create(ctypes.byref(c), ctypes.c_void_p(FAKE), nbytes, ctypes.byref(h)) == KVQ_OK
    return h


def i32(*v):
    return (ctypes.c_int32 * len(v))(*v)


def test_create_rejects_bad_buffers():
    c = cfg()
    h = ctypes.c_void_p()
    n = lib.kvq_cache_bytes(ctypes.byref(c))
    assert lib.kvq_cache_create(ctypes.byref(c), None, n, ctypes.byref(h)) == KVQ_E_INVALID
    assert lib.kvq_cache_create(ctypes.byref(c), ctypes.c_void_p(FAKE + 8), n, ctypes.byref(h)) == KVQ_E_INVALID
    assert lib.kvq_cache_create(ctypes.byref(c), ctypes.c_void_p(FAKE), n - 1, ctypes.byref(h)) == KVQ_E_INVALID
    assert not h.value
    lib.kvq_cache_destroy(None)


def test_host_side_errors_before_any_launch():
    c = cfg(batch=2, max_tokens=256)
    h = make_handle(c)
    P = ctypes.c_void_p(FAKE)
    try:
        # encode: n_tok not a multiple of 32, negative, over capacity, ld_tok too small
        assert lib.kvq_encode(h, P, P, 64, i32(32, 33), None) == KVQ_E_INVALID
        assert lib.kvq_encode(h, P, P, 64, i32(-32, 0), None) == KVQ_E_INVALID
        assert lib.kvq_encode(h, P, P, 512, i32(288, 0), None) == KVQ_E_CAPACITY
        assert lib.kvq_encode(h, P, P, 16, i32(32, 0), None) == KVQ_E_INVALID
        assert lib.kvq_encode(h, None, P, 64, i32(32, 0), None) == KVQ_E_INVALID
        assert lib.kvq_encode(h, P, P, 64, None, None) == KVQ_E_INVALID
        # nothing to do is fine without a device
        assert lib.kvq_encode(h, P, P, 64, i32(0, 0), None) == KVQ_OK
        # prefill: negative, over capacity, short ld_tok
        assert lib.kvq_prefill(h, P, P, 64, i32(-1, 3), None) == KVQ_E_INVALID
        assert lib.kvq_prefill(h, P, P, 300, i32(257, 3), None) == KVQ_E_CAPACITY
        assert lib.kvq_prefill(h, P, P, 10, i32(11, 3), None) == KVQ_E_INVALID
        # decode on an empty cache
        ws = ctypes.c_void_p(FAKE)
        assert lib.kvq_decode_attend(h, P, P, 0, 1.0, ws, 1 << 30, 0, None) == KVQ_E_INVALID
        assert b"empty" in lib.kvq_last_error()
        # multi-query: n_query >= 1 and at most max_tokens; here every sequence is empty, so both
        # the decode-kernel path (G * n_query <= 8, a power of two; G = 2) and the matrix-core
        # path (3, 8) reject it before any launch
        for nq_bad in (0, 257, 3, 8, 4):
            assert lib.kvq_decode_attend_multi(h, P, P, nq_bad, 0, 1.0, ws, 1 << 30, 0, None) == KVQ_E_INVALID
        assert lib.kvq_decode_attend(h, P, P, 0, 1.0, None, 1 << 30, 0, None) == KVQ_E_WORKSPACE
        assert lib.kvq_decode_attend(h, P, P, 0, float("nan"), ws, 1 << 30, 0, None) == KVQ_E_INVALID
        assert lib.kvq_decode_attend(h, P, P, 0, 1.0, ws, 1 << 30, -2, None) == KVQ_E_INVALID
        assert lib.kvq_append(h, None, P, None) == KVQ_E_INVALID
        # fused append + decode: the same argument checks, before any launch
        assert lib.kvq_append_decode_attend(h, None, P, P, P, 0, 1.0, ws, 1 << 30, 0, None) == KVQ_E_INVALID
        assert lib.kvq_append_decode_attend(h, P, P, None, P, 0, 1.0, ws, 1 << 30, 0, None) == KVQ_E_INVALID
        assert lib.kvq_append_decode_attend(h, P, P, P, P, 0, 1.0, None, 1 << 30, 0, None) == KVQ_E_WORKSPACE
        assert lib.kvq_append_decode_attend(h, P, P, P, P, 0, float("inf"), ws, 1 << 30, 0, None) == KVQ_E_INVALID
        assert lib.kvq_append_decode_attend(h, P, P, P, P, 0, 1.0, ws, 1 << 30, -1, None) == KVQ_E_INVALID
        # lengths mirror
        nq, nr = (ctypes.c_int32 * 2)(), (ctypes.c_int32 * 2)()
        assert lib.kvq_cache_lengths(h, nq, nr) == KVQ_OK and list(nq) == [0, 0] and list(nr) == [0, 0]
    finally:
        lib.kvq_cache_destroy(h)
    # the matrix-core multi-query kernel is built for KIVI caches without sinks
    for kw in (dict(n_sink=2), dict(method=1), dict(method=2, value_bits=16, kitty_n_hi=32)):
        h = make_handle(cfg(batch=2, max_tokens=256, **kw))
        try:
            assert lib.kvq_decode_attend_multi(h, P, P, 8, 0, 1.0, ctypes.c_void_p(FAKE), 1 << 30, 0, None) == \
                KVQ_E_UNSUPPORTED, kw
        finally:
            lib.kvq_cache_destroy(h)


def test_encode_block_validates_on_the_host():
    P = ctypes.c_void_p(FAKE)
    # bit width and group size outside the supported set
    assert lib.kvq_encode_block(P, 32, 64, 3, 32, 1, P, P, P, None) == KVQ_E_UNSUPPORTED
    assert lib.kvq_encode_block(P, 32, 64, 2, 16, 1, P, P, P, None) == KVQ_E_UNSUPPORTED
    # key rule needs 32 | n_tok, value rule needs 32 | D; D and n_tok ranges; NULL buffers
    assert lib.kvq_encode_block(P, 33, 64, 2, 32, 1, P, P, P, None) == KVQ_E_INVALID
    assert lib.kvq_encode_block(P, 33, 40, 2, 32, 0, P, P, P, None) == KVQ_E_INVALID
    assert lib.kvq_encode_block(P, 32, 0, 2, 32, 1, P, P, P, None) == KVQ_E_INVALID
    assert lib.kvq_encode_block(P, 32, 4097, 2, 32, 1, P, P, P, None) == KVQ_E_INVALID
    assert lib.kvq_encode_block(P, -32, 64, 2, 32, 1, P, P, P, None) == KVQ_E_INVALID
    assert lib.kvq_encode_block(P, 32, 64, 2, 32, 1, P, None, P, None) == KVQ_E_INVALID
    # an empty block needs no device
    assert lib.kvq_encode_block(None, 0, 64, 4, 32, 0, None, None, None, None) == KVQ_OK


@pytest.mark.skipif(torch_cuda, reason="checks the no-device path")
def test_device_calls_fail_cleanly_without_a_gpu():
    c = cfg(batch=1, n_kv_heads=1, n_q_heads=1, max_tokens=256)
    h = make_handle(c)
    P = ctypes.c_void_p(FAKE)
    try:
        assert lib.kvq_append(h, P, P, None) == KVQ_E_NODEVICE
        assert lib.kvq_encode(h, P, P, 64, i32(32), None) == KVQ_E_NODEVICE
        assert lib.kvq_prefill(h, P, P, 64, i32(40), None) == KVQ_E_NODEVICE
        assert lib.kvq_reset(h, None) == KVQ_E_NODEVICE
        # the host mirror did not move
        nq, nr = (ctypes.c_int32 * 1)(), (ctypes.c_int32 * 1)()
        lib.kvq_cache_lengths(h, nq, nr)
        assert (nq[0], nr[0]) == (0, 0)
    finally:
        lib.kvq_cache_destroy(h)


def test_status_strings():
    for st, name in [(KVQ_OK, "KVQ_OK"), (KVQ_E_INVALID, "KVQ_E_INVALID"), (KVQ_E_CAPACITY, "KVQ_E_CAPACITY"),
                     (KVQ_E_NODEVICE, "KVQ_E_NODEVICE"), (-99, "KVQ_E_UNKNOWN")]:
        assert lib.kvq_status_string(st).decode() == name


def test_kitty_config_from_python():
    from quantized_decode_attention_encode_amd import make_config

    c = make_config(1, 2, 2, 128, 2, 2, 32, 32, 1024, method="kitty")  # the pages' quarter
    assert (c.method, c.kitty_n_hi, c.kitty_hi_bits, c.value_bits) == (2, 32, 4, 16)
    assert lib.kvq_config_check(ctypes.byref(c)) == KVQ_OK
    assert make_config(1, 1, 1, 64, method="kitty", kitty_hi_fraction=0.25).kitty_n_hi == 16
    assert make_config(1, 1, 1, 128, method="kitty", kitty_hi_fraction=1.0).kitty_n_hi == 128
    odd = make_config(1, 1, 1, 128, method="kitty", kitty_hi_fraction=0.3)  # 38 channels: not built
    assert odd.kitty_n_hi == 38 and lib.kvq_config_check(ctypes.byref(odd)) == KVQ_E_UNSUPPORTED
    with pytest.raises(KVQError):
        make_config(1, 1, 1, 128, method="kitty", kitty_hi_fraction=1.5)
    with pytest.raises(ValueError):
        make_config(1, 1, 1, 128, method="polar")


def test_kitty_fraction_to_channel_count_in_the_library():
    """kvq_kitty_n_hi: round(fraction * head_dim), halves up; refuses NULL, head_dim < 1 and
    fractions outside [0, 1] (NaN included) without touching the output."""
    out = ctypes.c_int32(-7)
    for d, f, want in ((128, 0.25, 32), (64, 0.25, 16), (128, 0.0, 0), (128, 1.0, 128),
                       (128, 0.3, 38), (128, 0.125, 16), (96, 1 / 6, 16), (10, 0.25, 3), (10, 0.05, 1)):
        assert lib.kvq_kitty_n_hi(d, f, ctypes.byref(out)) == KVQ_OK
        assert out.value == want, (d, f, out.value)
    out.value = -7
    for d, f in ((128, -0.01), (128, 1.01), (128, float("nan")), (128, float("inf")), (0, 0.25), (-4, 0.5)):
        assert lib.kvq_kitty_n_hi(d, f, ctypes.byref(out)) == KVQ_E_INVALID
        assert out.value == -7
    assert lib.kvq_kitty_n_hi(128, 0.25, None) == KVQ_E_INVALID
