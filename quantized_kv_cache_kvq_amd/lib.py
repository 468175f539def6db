"""ctypes binding of libkvq.so: the C structs and entry points of
``include/kvq.h`` with the same names.  Argument marshalling only; every step
of the computation runs in the library's HIP kernels.

``load()`` raises if the library has not been built: there is no fallback.
"""

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kvq.h")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = range(6)
KVQ_MAX_CAPACITY = 1 << 24     # include/kvq.h: largest capacity / tail_len per plane

CODECS = ["f16", "q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0",
          "q8_1", "q6_1", "q5_1", "q4_1", "q3_1", "q2_1", "q1_1"]
CODEC_ID = {n: i for i, n in enumerate(CODECS)}
BASIS_ID = {"plain": 0, "hadamard": 1, "lowrank": 2}
HEAD_DIM = 128
TILE = 64


class kvq_plane(ctypes.Structure):
    _fields_ = [
        ("codec", ctypes.c_int32),
        ("basis", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("mins", ctypes.c_void_p),
        ("tail", ctypes.c_void_p),
        ("w", ctypes.c_void_p),
        ("proj", ctypes.c_void_p),
        ("rank", ctypes.POINTER(ctypes.c_int32)),
        ("head_codec", ctypes.POINTER(ctypes.c_int32)),
    ]


class kvq_layer(ctypes.Structure):
    _fields_ = [
        ("k", kvq_plane),
        ("v", kvq_plane),
        ("batch", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("tail_len", ctypes.c_int32),
        ("n_tokens", ctypes.c_int32),
        ("tail_format", ctypes.c_int32),
        ("seq_tokens", ctypes.c_void_p),
    ]


TAIL_FORMATS = ("f16", "bf16")       # kvq_tail_format order


class KvqError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, status), detail))


_STATUS_NAMES = {0: "KVQ_OK", 1: "KVQ_ERR_INVALID_ARG", 2: "KVQ_ERR_UNSUPPORTED",
                 3: "KVQ_ERR_CAPACITY", 4: "KVQ_ERR_WORKSPACE", 5: "KVQ_ERR_HIP"}

_lib = None

_SIGS = {
    "kvq_plane_bytes": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                                       ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "kvq_quantize_append": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_void_p]),
    "kvq_transcode_layer": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.POINTER(kvq_layer),
                                           ctypes.c_void_p]),
    "kvq_dequantize": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]),
    "kvq_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(kvq_layer), ctypes.c_int32]),
    "kvq_append_decode": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]),
    "kvq_append_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                                 ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "kvq_decode_attention": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "kvq_decode_attention_splits": (ctypes.c_int, [ctypes.POINTER(kvq_layer), ctypes.c_void_p,
                                                   ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                                   ctypes.c_void_p]),
    "kvq_vbr_bytes": (ctypes.c_longlong, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]),
    "kvq_vbr_plan": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32)]),
    "kvq_cobra_allocate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                          ctypes.c_longlong, ctypes.c_double,
                                          ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]),
    "kvq_timing_begin": (ctypes.c_int, [ctypes.c_int32]),
    "kvq_timing_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]),
    "kvq_timing_durations": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32)]),
    "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_abi_version": (ctypes.c_int32, []),
    "kvq_source_hash": (ctypes.c_char_p, []),
}


def load(path=LIB_PATH):
    """Load libkvq.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libkvq.so is not built (%s); run __graft_entry__.build() or "
                           "python -m quantized_kv_cache_kvq_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.kvq_abi_version() != 2:
        raise RuntimeError("libkvq.so ABI version mismatch")
    from .build import source_hash
    built, now = lib.kvq_source_hash().decode(), source_hash()
    if built != now:
        raise RuntimeError("libkvq.so was built from other sources (library %s, sources %s); "
                           "rebuild with __graft_entry__.build()" % (built, now))
    _lib = lib
    return lib


def header_functions(path=HEADER):
    """Names of the entry points declared in include/kvq.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def check(status):
    """Raise KvqError for a non-zero kvq_status."""
    if status != KVQ_OK:
        detail = load().kvq_last_error().decode()
        raise KvqError(status, detail)


def plane_bytes(layer, which):
    lib = load()
    sizes = [ctypes.c_size_t() for _ in range(4)]
    check(lib.kvq_plane_bytes(ctypes.byref(layer), which, *[ctypes.byref(s) for s in sizes]))
    return tuple(s.value for s in sizes)


def quantize_append(layer, k_new_ptr, v_new_ptr, n_new, stream):
    check(load().kvq_quantize_append(ctypes.byref(layer), k_new_ptr, v_new_ptr, n_new, stream))


def transcode_layer(src, dst, stream):
    check(load().kvq_transcode_layer(ctypes.byref(src), ctypes.byref(dst), stream))


def dequantize(layer, which, out_ptr, stream):
    check(load().kvq_dequantize(ctypes.byref(layer), which, out_ptr, stream))


def decode_workspace_bytes(layer, n_q_heads):
    return load().kvq_decode_workspace_bytes(ctypes.byref(layer), n_q_heads)


def append_decode(layer, k_ptr, v_ptr, q_ptr, n_q_heads, sm_scale, out_ptr, ws_ptr, ws_bytes, stream):
    check(load().kvq_append_decode(ctypes.byref(layer), k_ptr, v_ptr, q_ptr, n_q_heads,
                                   ctypes.c_float(sm_scale), out_ptr, ws_ptr, ws_bytes, stream))


def append_decode_noalloc(layer, k_ptr, v_ptr, q_ptr, n_q_heads, sm_scale, out_ptr, stream):
    """The one-call step with the library's fixed scratch as its workspace."""
    check(load().kvq_append_decode_noalloc(ctypes.byref(layer), k_ptr, v_ptr, q_ptr, n_q_heads,
                                           ctypes.c_float(sm_scale), out_ptr, stream))


def decode_attention(layer, q_ptr, n_q_heads, sm_scale, out_ptr, ws_ptr, ws_bytes, stream,
                     body_splits=0):
    check(load().kvq_decode_attention_splits(ctypes.byref(layer), q_ptr, n_q_heads,
                                             ctypes.c_float(sm_scale), out_ptr, ws_ptr, ws_bytes,
                                             body_splits, stream))


def timing_begin(capacity):
    """Start recording event pairs around the split-K decode kernel."""
    check(load().kvq_timing_begin(capacity))


def timing_durations(capacity):
    """Per-launch kernel durations (milliseconds) recorded so far."""
    buf = (ctypes.c_float * max(1, capacity))()
    n = ctypes.c_int32()
    check(load().kvq_timing_durations(buf, capacity, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def timing_end():
    """(summed milliseconds, number of recorded launches); stops recording."""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    check(load().kvq_timing_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class kvq_vbr_policy(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("ladder", ctypes.POINTER(ctypes.c_int32)),
                ("ladder_len", ctypes.c_int32), ("floor", ctypes.c_int32),
                ("order", ctypes.POINTER(ctypes.c_int32)), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("tail_len", ctypes.c_int32),
                ("budget_bytes", ctypes.c_longlong)]


def _i32(values):
    return (ctypes.c_int32 * max(1, len(values)))(*values)


def vbr_policy(ladder, floor, order, batch, n_kv_heads, tail_len, budget_bytes):
    """Policy descriptor; ladder: codec names best first, floor: a ladder
    index, order: degrade order (layer indices)."""
    lad = _i32([CODECS.index(c) for c in ladder])
    ordr = _i32(list(order))
    pol = kvq_vbr_policy(len(order), lad, len(ladder), floor, ordr, batch, n_kv_heads, tail_len,
                         budget_bytes)
    pol._keep = (lad, ordr)
    return pol


def vbr_bytes(pol, level, n_tokens):
    return load().kvq_vbr_bytes(ctypes.byref(pol), _i32(level), n_tokens)


def vbr_plan(pol, n_tokens, level, max_steps=4096):
    """(status, new levels, steps [(layer, from codec name, to codec name)])."""
    lv = _i32(level)
    steps = (ctypes.c_int32 * (3 * max_steps))()
    n = ctypes.c_int32()
    st = load().kvq_vbr_plan(ctypes.byref(pol), n_tokens, lv, steps, max_steps, ctypes.byref(n))
    out = [(steps[3 * i], CODECS[steps[3 * i + 1]], CODECS[steps[3 * i + 2]]) for i in range(n.value)]
    return st, [lv[i] for i in range(len(level))], out


def cobra_allocate(spectra, ranks, bits, budget_bits, gamma=4.0 / 3.0):
    """Per-head (rank, bits) for spectra [H, 128] (largest first).
    Returns (list of (rank, bits), C2 rounds, total error)."""
    import numpy as np

    sp = np.ascontiguousarray(spectra, dtype=np.float64)
    H = sp.shape[0]
    r_out, b_out = (ctypes.c_int32 * H)(), (ctypes.c_int32 * H)()
    rounds, tot = ctypes.c_int32(), ctypes.c_double()
    check(load().kvq_cobra_allocate(sp.ctypes.data, H, _i32(ranks), len(ranks), _i32(bits), len(bits),
                                    budget_bits, gamma, r_out, b_out, ctypes.byref(rounds),
                                    ctypes.byref(tot)))
    return [(r_out[h], b_out[h]) for h in range(H)], rounds.value, tot.value
