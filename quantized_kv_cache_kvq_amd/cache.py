"""A layer of the packed KV cache held in PyTorch device memory.

PyTorch provides the device buffers and the stream; the library's kernels do
all the work.  The object keeps the host bookkeeping the C ABI leaves to the
caller: the token count, the per-head tables of the low-rank basis and the
decode workspace.
"""

import ctypes
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

from . import lib


@dataclass
class PlaneSpec:
    """How K or V of a layer is stored."""
    codec: str = "q8_0"
    basis: str = "plain"                      # "plain" | "hadamard" | "lowrank"
    w: Optional[torch.Tensor] = None          # hadamard: [Hkv, 128] float32, 1/sigma
    proj: Optional[torch.Tensor] = None       # lowrank: [Hkv, 128, 128] float16
    ranks: Sequence[int] = field(default_factory=tuple)
    head_codecs: Sequence[str] = field(default_factory=tuple)


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


class LayerCache:
    def __init__(self, batch, n_kv_heads, capacity, tail_len, kspec: PlaneSpec,
                 vspec: PlaneSpec, device="cuda", share_tail_with=None, tail_format="f16"):
        self.device = torch.device(device)
        self.batch, self.n_kv_heads = batch, n_kv_heads
        self.capacity, self.tail_len = capacity, tail_len
        self.kspec, self.vspec = kspec, vspec
        self.desc = lib.kvq_layer()
        self.desc.batch, self.desc.n_kv_heads = batch, n_kv_heads
        self.desc.head_dim, self.desc.capacity = lib.HEAD_DIM, capacity
        self.desc.tail_len, self.desc.n_tokens = tail_len, 0
        if tail_format not in lib.TAIL_FORMATS:
            raise ValueError("tail_format must be one of %s" % (lib.TAIL_FORMATS,))
        self.tail_format = tail_format
        self.desc.tail_format = lib.TAIL_FORMATS.index(tail_format)
        self._keep = []
        self.bufs = {}
        for which, name, spec in ((0, "k", kspec), (1, "v", vspec)):
            plane = self.desc.k if which == 0 else self.desc.v
            self._fill_spec(plane, spec)
            codes, scales, mins, tail = lib.plane_bytes(self.desc, which)
            b = {
                "codes": torch.zeros(max(codes, 1), dtype=torch.uint8, device=self.device),
                "scales": torch.zeros(scales, dtype=torch.uint8, device=self.device) if scales else None,
                "mins": torch.zeros(mins, dtype=torch.uint8, device=self.device) if mins else None,
            }
            if tail:
                b["tail"] = (share_tail_with.bufs[name]["tail"] if share_tail_with is not None
                             else torch.zeros(tail, dtype=torch.uint8, device=self.device))
            else:
                b["tail"] = None
            plane.codes = _ptr(b["codes"]).value
            plane.scales = _ptr(b["scales"]).value
            plane.mins = _ptr(b["mins"]).value
            plane.tail = _ptr(b["tail"]).value
            self.bufs[name] = b
        self._ws = None
        self.seq_tokens = None

    def set_seq_tokens(self, seq):
        """Ragged batch: seq is a device int32 tensor [B] of per-sequence token
        counts (each <= n_tokens, which is their maximum), or None.  append()
        advances it with n_tokens."""
        if seq is None:
            self.seq_tokens, self.desc.seq_tokens = None, None
            return
        if seq.dtype != torch.int32 or tuple(seq.shape) != (self.batch,) or seq.device != self.device:
            raise ValueError("seq must be int32 [batch] on the layer's device")
        self.seq_tokens = seq.contiguous()
        self.desc.seq_tokens = self.seq_tokens.data_ptr()

    def _fill_spec(self, plane, spec):
        plane.basis = lib.BASIS_ID[spec.basis]
        plane.codec = lib.CODEC_ID[spec.codec] if spec.basis != "lowrank" else 0
        if spec.basis == "hadamard":
            w = spec.w.to(self.device, torch.float32).contiguous()
            self._keep.append(w)
            plane.w = w.data_ptr()
        if spec.basis == "lowrank":
            P = spec.proj.to(self.device, torch.float16).contiguous()
            self._keep.append(P)
            plane.proj = P.data_ptr()
            ranks = (ctypes.c_int32 * self.n_kv_heads)(*spec.ranks)
            hc = (ctypes.c_int32 * self.n_kv_heads)(*[lib.CODEC_ID[c] for c in spec.head_codecs])
            self._keep += [ranks, hc]
            plane.rank = ctypes.cast(ranks, ctypes.POINTER(ctypes.c_int32))
            plane.head_codec = ctypes.cast(hc, ctypes.POINTER(ctypes.c_int32))

    @property
    def n_tokens(self):
        return self.desc.n_tokens

    @n_tokens.setter
    def n_tokens(self, t):
        self.desc.n_tokens = t

    def append(self, k_new, v_new, stream=None):
        """k_new, v_new: float32 [B, n, Hkv, 128] on the device."""
        k_new = k_new.contiguous()
        v_new = v_new.contiguous()
        if k_new.dtype != torch.float32 or k_new.shape != v_new.shape or k_new.dim() != 4:
            raise ValueError("k_new/v_new must be float32 [B, n, Hkv, 128] of equal shape")
        if k_new.shape[0] != self.batch or k_new.shape[2] != self.n_kv_heads or k_new.shape[3] != 128:
            raise ValueError("k_new shape %s does not match the layer" % (tuple(k_new.shape),))
        n = k_new.shape[1]
        lib.quantize_append(self.desc, _ptr(k_new), _ptr(v_new), n, _stream(self.device, stream))
        self.desc.n_tokens += n
        if self.seq_tokens is not None:
            if stream is None:
                self.seq_tokens.add_(n)
            else:
                with torch.cuda.stream(stream):
                    self.seq_tokens.add_(n)

    def workspace(self, n_q_heads, stream=None):
        """The layer's decode workspace for n_q_heads query heads (allocated
        and zero-filled on first use, on the stream that will use it)."""
        need = lib.decode_workspace_bytes(self.desc, n_q_heads)
        if self._ws is None or self._ws.numel() < need:
            st = stream if stream is not None else torch.cuda.current_stream(self.device)
            if self._ws is not None:
                # the old buffer may still be in use on its stream
                self._ws.record_stream(st)
            with torch.cuda.stream(st):
                # zero once: the library keeps its completion counters zero
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def bind_step(self, k_new, v_new, q, sm_scale, out, stream=None):
        """A decode step bound to fixed buffers: checks the arguments and
        reserves the workspace once, then each call of the returned object
        enqueues kvq_append_decode with the pre-built arguments and advances
        n_tokens (and seq_tokens).  For serving loops that reuse the same
        input and output buffers every step."""
        return BoundStep(self, k_new, v_new, q, sm_scale, out, stream)

    def decode(self, q, sm_scale, out=None, body_splits=0, stream=None, ws=None):
        """q: float32 [B, Hq, 128] -> out float32 [B, Hq, 128]."""
        q = q.contiguous()
        if q.dtype != torch.float32 or q.dim() != 3 or q.shape[0] != self.batch or q.shape[2] != 128:
            raise ValueError("q must be float32 [B, Hq, 128]")
        Hq = q.shape[1]
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(Hq, stream) if ws is None else ws
        lib.decode_attention(self.desc, _ptr(q), Hq, float(sm_scale), _ptr(out), _ptr(ws),
                             ws.numel(), _stream(self.device, stream), body_splits)
        return out

    def dequantize(self, which, out=None, stream=None):
        """The K (which="k") or V ("v") vectors decode attends over, raw
        basis: float32 [B, n_tokens, Hkv, 128] on the device."""
        shape = (self.batch, self.n_tokens, self.n_kv_heads, lib.HEAD_DIM)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be contiguous float32 %s" % (shape,))
        lib.dequantize(self.desc, {"k": 0, "v": 1}[which], _ptr(out), _stream(self.device, stream))
        return out

    def append_decode(self, k_new, v_new, q, sm_scale, out=None, stream=None, ws=None):
        """One decode step: append k_new, v_new (float32 [B, 1, Hkv, 128]) and
        decode q (float32 [B, Hq, 128]) over the cache with the new token, in
        one launch where the library can fuse them.  Advances n_tokens (and
        seq_tokens)."""
        k_new = k_new.contiguous()
        v_new = v_new.contiguous()
        if (k_new.dtype != torch.float32 or k_new.shape != v_new.shape
                or tuple(k_new.shape) != (self.batch, 1, self.n_kv_heads, 128)):
            raise ValueError("k_new/v_new must be float32 [B, 1, Hkv, 128]")
        q = q.contiguous()
        if q.dtype != torch.float32 or q.dim() != 3 or q.shape[0] != self.batch or q.shape[2] != 128:
            raise ValueError("q must be float32 [B, Hq, 128]")
        Hq = q.shape[1]
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(Hq, stream) if ws is None else ws
        st = _stream(self.device, stream)
        lib.append_decode(self.desc, _ptr(k_new), _ptr(v_new), _ptr(q), Hq, float(sm_scale), _ptr(out),
                          _ptr(ws), ws.numel(), st)
        self.desc.n_tokens += 1
        if self.seq_tokens is not None:
            if stream is None:
                self.seq_tokens.add_(1)
            else:
                with torch.cuda.stream(stream):
                    self.seq_tokens.add_(1)
        return out

    def transcode(self, kcodec, vcodec, stream=None):
        """A new layer with K and V re-encoded; shares this layer's tails."""
        ks = PlaneSpec(kcodec, self.kspec.basis, self.kspec.w)
        vs = PlaneSpec(vcodec, self.vspec.basis, self.vspec.w)
        dst = LayerCache(self.batch, self.n_kv_heads, self.capacity, self.tail_len, ks, vs,
                         self.device, share_tail_with=self, tail_format=self.tail_format)
        dst.n_tokens = self.n_tokens
        lib.transcode_layer(self.desc, dst.desc, _stream(self.device, stream))
        return dst

    def transcode_into(self, dst, stream=None):
        """Re-encode into an existing layer ``dst`` (same shapes and token count)."""
        dst.n_tokens = self.n_tokens
        lib.transcode_layer(self.desc, dst.desc, _stream(self.device, stream))
        return dst


class BoundStep:
    """One layer's decode step (append the new token, attend) with every
    argument of kvq_append_decode marshalled once.  Calling it enqueues the
    step on the bound stream and advances the layer's token count; the
    bound tensors must keep their storage (their contents may change)."""

    def __init__(self, layer, k_new, v_new, q, sm_scale, out, stream=None):
        B, Hkv = layer.batch, layer.n_kv_heads
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if (t.dtype != torch.float32 or not t.is_contiguous()
                    or tuple(t.shape) != (B, 1, Hkv, 128) or t.device != layer.device):
                raise ValueError("%s must be contiguous float32 [B, 1, Hkv, 128] on the layer's device" % name)
        if (q.dtype != torch.float32 or not q.is_contiguous() or q.dim() != 3 or q.shape[0] != B
                or q.shape[2] != 128 or q.device != layer.device):
            raise ValueError("q must be contiguous float32 [B, Hq, 128] on the layer's device")
        if out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be contiguous float32 shaped like q")
        Hq = q.shape[1]
        self.layer = layer
        self.stream = stream if stream is not None else torch.cuda.current_stream(layer.device)
        ws = layer.workspace(Hq, self.stream)
        self._keep = (k_new, v_new, q, out, ws)
        self._fn = lib.load().kvq_append_decode
        self._args = (ctypes.byref(layer.desc), _ptr(k_new), _ptr(v_new), _ptr(q), Hq,
                      ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(ws), ws.numel(),
                      ctypes.c_void_p(self.stream.cuda_stream))
        self.out = out

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            lib.check(st)
        layer = self.layer
        layer.desc.n_tokens += 1
        if layer.seq_tokens is not None:
            with torch.cuda.stream(self.stream):
                layer.seq_tokens.add_(1)
        return self.out
