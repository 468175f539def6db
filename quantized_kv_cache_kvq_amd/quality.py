"""Quality of the packed cache on synthetic data, per codec, tail length and
basis: how far decode attention over the packed cache is from exact
attention over the unquantised rows.

This mirrors the shape of the precision-tail KLD table of the BeeLlama.cpp
v0.4.0 release notes (codecs q2_0 .. q8_0 and their KVarN counterparts at
tails 0, 1024 and 2048, 64k context) without a model: the divergence here is
between one query's attention weights over exact and over packed keys, not
between a model's output distributions, so only the trends compare.

Tails are binary16 or bfloat16 (the release notes allow either).

Per configuration, on the device: the layer is built by the library's append
(one call over the whole context), the outputs come from the library's
decode, and the keys attended over are the library's read-back
(kvq_dequantize).  The exact attention over the unquantised binary32 rows and
the metrics are computed with PyTorch in float64.  Metrics per (query, batch
entry, query head): KL(p || p_hat) of the softmax weights in nats and the
relative L2 error of the output; a configuration reports median and mean.
"""

import math

import torch

from . import calib
from .cache import LayerCache, PlaneSpec

CODECS = ("q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0")
TAILS = (0, 1024, 2048)
BASES = ("plain", "hadamard")


def bits_per_value(codec):
    """Stored bits per coordinate: codes plus binary16 scale (and min) per
    32-coordinate block."""
    if codec == "f16":
        return 16.0
    b = int(codec[1])
    return b + (32.0 if codec.endswith("_1") else 16.0) / 32.0


def _exact(q, K, V, G, sm_scale):
    """fp64 weights log p [B, Hq, T] and outputs [B, Hq, 128]; K, V are
    [B, T, Hkv, 128] float64, q [B, Hq, 128]."""
    Kq = K.repeat_interleave(G, dim=2)                      # [B, T, Hq, 128]
    Vq = V.repeat_interleave(G, dim=2)
    s = torch.einsum("bhd,bthd->bht", q.double(), Kq) * sm_scale
    logp = torch.log_softmax(s, dim=-1)
    o = torch.einsum("bht,bthd->bhd", logp.exp(), Vq)
    return logp, o


def kl_nats(logp, logp_h):
    """KL(p || p_hat) in nats over the last axis, from log-weights."""
    return (logp.exp() * (logp - logp_h)).sum(-1)


def measure(layer, q_all, K, V, sm_scale):
    """Metrics of one built layer over queries q_all [n, B, Hq, 128]."""
    G = q_all.shape[2] // K.shape[2]
    Kh = layer.dequantize("k").double()
    Vh = layer.dequantize("v").double()
    kls, errs, cons = [], [], 0.0
    for q in q_all:
        logp, o = _exact(q, K, V, G, sm_scale)
        logp_h, o_h = _exact(q, Kh, Vh, G, sm_scale)
        out = layer.decode(q, sm_scale).double()
        kl = kl_nats(logp, logp_h)                          # [B, Hq]
        err = (out - o).norm(dim=-1) / o.norm(dim=-1)
        kls.append(kl.flatten())
        errs.append(err.flatten())
        cons = max(cons, float((out - o_h).abs().max()))
    kl = torch.cat(kls)
    err = torch.cat(errs)
    return {"kl_median": float(kl.median()), "kl_mean": float(kl.mean()),
            "err_median": float(err.median()), "err_mean": float(err.mean()),
            "decode_vs_readback_maxabs": cons}


def sweep(k, v, q_all, sm_scale, codecs=CODECS, tails=TAILS, bases=BASES, calib_tokens=4096,
          tail_formats=("f16", "bf16"), log=None):
    """k, v: [B, T, Hkv, 128] float32 on the device; q_all [n, B, Hq, 128].
    Returns one dict per (basis, codec, tail, tail format); tail 0 has one
    row (format "-")."""
    B, T, Hkv, _ = k.shape
    capacity = (T + 63) // 64 * 64
    K, V = k.double(), v.double()
    n_cal = min(calib_tokens, T)
    w = {"k": calib.kvarn_weights(k[0, :n_cal].permute(1, 0, 2).cpu()),
         "v": calib.kvarn_weights(v[0, :n_cal].permute(1, 0, 2).cpu())}
    rows = []
    for basis in bases:
        for codec in codecs:
            for tail in tails:
                for fmt in (tail_formats if tail > 0 else ("f16",)):
                    ks = PlaneSpec(codec, basis, w["k"] if basis == "hadamard" else None)
                    vs = PlaneSpec(codec, basis, w["v"] if basis == "hadamard" else None)
                    layer = LayerCache(B, Hkv, capacity, tail, ks, vs, k.device, tail_format=fmt)
                    layer.append(k, v)
                    r = {"basis": basis, "codec": codec, "bits": bits_per_value(codec), "tail": tail,
                         "tail_format": fmt if tail > 0 else "-"}
                    r.update(measure(layer, q_all, K, V, sm_scale))
                    rows.append(r)
                    if log:
                        log(r)
                    del layer
    return rows


def entropy_nats(q_all, k, sm_scale):
    """Median entropy of the exact attention weights (how peaked the
    synthetic attention is)."""
    K = k.double()
    G = q_all.shape[2] // k.shape[2]
    ents = []
    for q in q_all:
        logp, _ = _exact(q, K, K, G, sm_scale)
        ents.append(-(logp.exp() * logp).sum(-1).flatten())
    e = torch.cat(ents)
    return float(e.median()), math.log(k.shape[1])
