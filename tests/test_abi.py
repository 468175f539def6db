"""CPU tests of the C ABI: the library loads, exports every declared entry
point, reports closed-form buffer sizes, and rejects bad arguments on the
host before anything is launched (no compute call needs a GPU here)."""

import ctypes
import os

import pytest

from quantized_kv_cache_kvq_amd import lib


@pytest.fixture(scope="module")
def L():
    return lib.load()


def _layer(B=1, Hkv=8, cap=1024, N=0, kc="q8_0", vc="q4_0", T=0):
    d = lib.kvq_layer()
    d.batch, d.n_kv_heads, d.head_dim, d.capacity, d.tail_len, d.n_tokens = B, Hkv, 128, cap, N, T
    d.k.codec, d.v.codec = lib.CODEC_ID[kc], lib.CODEC_ID[vc]
    fake = 0x1000
    for p in (d.k, d.v):
        p.codes = p.scales = p.mins = p.tail = fake
    return d


def _status(L, fn, *args):
    return getattr(L, fn)(*args)


def test_exports_every_declared_symbol(L):
    names = lib.header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert L.kvq_abi_version() == 2
    assert L.kvq_status_string(3) == b"KVQ_ERR_CAPACITY"


def test_plane_bytes_closed_forms(L):
    d = _layer(B=2, Hkv=8, cap=1024, N=128)
    codes, scales, mins, tail = lib.plane_bytes(d, 0)            # K q8_0
    assert codes == 2 * 8 * 1024 * 128 and scales == 2 * 8 * 1024 * 4 * 2 and mins == 0
    assert tail == 2 * 8 * 128 * 256
    codes, scales, mins, _ = lib.plane_bytes(d, 1)               # V q4_0
    assert codes == 2 * 8 * 1024 * 64 and scales == 2 * 8 * 1024 * 8
    d = _layer(kc="q3_1", vc="f16")
    c, s, m, t = lib.plane_bytes(d, 0)
    assert (c, s, m, t) == (8 * 1024 * 48, 8 * 1024 * 8, 8 * 1024 * 8, 0)
    c, s, m, _ = lib.plane_bytes(d, 1)
    assert (c, s, m) == (8 * 1024 * 256, 0, 0)


def test_lowrank_plane_bytes(L):
    d = _layer(Hkv=8, cap=64)
    table = [(128, 1), (64, 2), (32, 4), (16, 4), (64, 3), (128, 1), (32, 2), (64, 3)]
    ranks = (ctypes.c_int32 * 8)(*[r for r, _ in table])
    codecs = (ctypes.c_int32 * 8)(*[lib.CODEC_ID["q%d_1" % b] for _, b in table])
    for p in (d.k, d.v):
        p.basis = 2
        p.rank = ctypes.cast(ranks, ctypes.POINTER(ctypes.c_int32))
        p.head_codec = ctypes.cast(codecs, ctypes.POINTER(ctypes.c_int32))
        p.proj = 0x1000
    c, s, m, _ = lib.plane_bytes(d, 0)
    assert c == 64 * 128 and s == 64 * 17 * 2 and m == 64 * 17 * 2


def test_host_validation_rejects_before_launch(L):
    null = ctypes.c_void_p(0)
    assert L.kvq_quantize_append(None, null, null, 1, null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer()
    d.head_dim = 64
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_UNSUPPORTED
    d = _layer(cap=100)
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
    assert b"capacity" in L.kvq_last_error()
    d = _layer(cap=64, T=60)
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 5, null) == lib.KVQ_ERR_CAPACITY
    d = _layer()
    d.k.codec = 99
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer(N=128)
    d.k.tail = 0
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer(kc="q4_1")
    d.k.mins = 0
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer()
    d.k.basis = 1                                            # hadamard without w
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer()
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 0, null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer(N=64)
    d.tail_format = 2                                        # not a kvq_tail_format
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
    assert b"tail_format" in L.kvq_last_error()
    s, dd = _layer(N=64, T=64), _layer(N=64, T=64)
    dd.tail_format = 1                                       # transcode shares the tails
    assert L.kvq_transcode_layer(ctypes.byref(s), ctypes.byref(dd), null) == lib.KVQ_ERR_INVALID_ARG
    d = _layer(T=0)
    assert L.kvq_dequantize(ctypes.byref(d), 0, null, null) == lib.KVQ_OK   # nothing to write
    d = _layer(T=64)
    assert L.kvq_dequantize(ctypes.byref(d), 2, 1, null) == lib.KVQ_ERR_INVALID_ARG
    assert L.kvq_dequantize(ctypes.byref(d), 0, null, null) == lib.KVQ_ERR_INVALID_ARG


def test_capacity_above_maximum_rejected(L):
    """Layers beyond KVQ_MAX_CAPACITY (32-bit in-plane offsets) are refused
    by every compute entry point before anything is enqueued."""
    import re
    hdr = open(os.path.join(os.path.dirname(lib.HERE), "include", "kvq.h")).read()
    m = re.search(r"#define KVQ_MAX_CAPACITY \(1 << (\d+)\)", hdr)
    assert m and lib.KVQ_MAX_CAPACITY == 1 << int(m.group(1))
    null = ctypes.c_void_p(0)
    big = lib.KVQ_MAX_CAPACITY + 64
    for d in (_layer(cap=big, T=10), _layer(cap=1024, N=big, T=10)):
        assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, null) == lib.KVQ_ERR_INVALID_ARG
        assert b"KVQ_MAX_CAPACITY" in L.kvq_last_error()
        assert L.kvq_dequantize(ctypes.byref(d), 0, 1, null) == lib.KVQ_ERR_INVALID_ARG
        assert L.kvq_transcode_layer(ctypes.byref(d), ctypes.byref(d), null) == lib.KVQ_ERR_INVALID_ARG
        ws = (1, 32, ctypes.c_float(1.0), 1, 1, ctypes.c_size_t(1 << 30), null)
        assert L.kvq_decode_attention(ctypes.byref(d), *ws) == lib.KVQ_ERR_INVALID_ARG
        assert L.kvq_append_decode(ctypes.byref(d), 1, 1, 1, 32, ctypes.c_float(1.0), 1, 1,
                                   ctypes.c_size_t(1 << 30), null) == lib.KVQ_ERR_INVALID_ARG


def test_decode_validation(L):
    d = _layer(T=0)
    args = (1, 32, ctypes.c_float(1.0), 1, 1, ctypes.c_size_t(1 << 30), ctypes.c_void_p(0))
    assert L.kvq_decode_attention(ctypes.byref(d), *args) == lib.KVQ_ERR_INVALID_ARG   # empty
    d = _layer(T=10)
    bad = (1, 30, ctypes.c_float(1.0), 1, 1, ctypes.c_size_t(1 << 30), ctypes.c_void_p(0))
    assert L.kvq_decode_attention(ctypes.byref(d), *bad) == lib.KVQ_ERR_INVALID_ARG    # 30 % 8
    need = lib.decode_workspace_bytes(d, 32)
    assert need > 0
    small = (1, 32, ctypes.c_float(1.0), 1, 1, ctypes.c_size_t(64), ctypes.c_void_p(0))
    assert L.kvq_decode_attention(ctypes.byref(d), *small) == lib.KVQ_ERR_WORKSPACE
    nows = (1, 32, ctypes.c_float(1.0), 1, None, ctypes.c_size_t(need), ctypes.c_void_p(0))
    assert L.kvq_decode_attention(ctypes.byref(d), *nows) == lib.KVQ_ERR_WORKSPACE
    d = _layer(kc="q5_0", vc="q2_1", T=10)                      # no compiled path
    assert L.kvq_decode_attention(ctypes.byref(d), *args) == lib.KVQ_ERR_UNSUPPORTED
    assert lib.decode_workspace_bytes(_layer(cap=4096), 32) > lib.decode_workspace_bytes(_layer(cap=1024), 32)


def test_lowrank_and_transcode_validation(L):
    d = _layer(Hkv=2, T=4)
    ranks = (ctypes.c_int32 * 2)(48, 16)
    codecs = (ctypes.c_int32 * 2)(lib.CODEC_ID["q2_1"], lib.CODEC_ID["q2_1"])
    for p in (d.k, d.v):
        p.basis, p.proj = 2, 0x1000
        p.rank = ctypes.cast(ranks, ctypes.POINTER(ctypes.c_int32))
        p.head_codec = ctypes.cast(codecs, ctypes.POINTER(ctypes.c_int32))
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, None) == lib.KVQ_ERR_INVALID_ARG
    ranks[0] = 32
    vr = (ctypes.c_int32 * 2)(32, 32)
    d.v.rank = ctypes.cast(vr, ctypes.POINTER(ctypes.c_int32))
    assert L.kvq_quantize_append(ctypes.byref(d), 1, 1, 1, None) == lib.KVQ_ERR_UNSUPPORTED
    d.v.rank = d.k.rank
    e = _layer(Hkv=2, T=4)
    assert L.kvq_transcode_layer(ctypes.byref(d), ctypes.byref(d), None) == lib.KVQ_ERR_UNSUPPORTED
    a, b = _layer(T=5), _layer(T=5)
    assert L.kvq_transcode_layer(ctypes.byref(a), ctypes.byref(b), None) == lib.KVQ_ERR_INVALID_ARG  # alias
    b.capacity = 2048
    b.k.codes = b.v.codes = 0x2000
    assert L.kvq_transcode_layer(ctypes.byref(a), ctypes.byref(b), None) == lib.KVQ_ERR_INVALID_ARG
    del e


def test_timing_hook_host_side(L):
    """The measurement hook rejects bad capacities before touching a device,
    and ending a session that recorded nothing reports zero launches."""
    assert L.kvq_timing_begin(0) == lib.KVQ_ERR_INVALID_ARG
    assert L.kvq_timing_begin((1 << 20) + 1) == lib.KVQ_ERR_INVALID_ARG
    ms, n = ctypes.c_double(-1.0), ctypes.c_int32(-1)
    assert L.kvq_timing_end(ctypes.byref(ms), ctypes.byref(n)) == lib.KVQ_OK
    assert n.value == 0 and ms.value == 0.0
