"""Seeded synthetic workloads for the packed KV cache.

Shared by the tests, the smoke check and the benchmark.  This module draws
random numbers and arranges them into tensors; it holds none of the codec,
rotation, projection or attention arithmetic.  Every chunk (one batch entry,
one kv head, one of K/V/q, one layer) has its own seed derived from the
workload seed and the chunk's key, so any chunk can be regenerated alone.
Chunks regenerate identically on the same device type (torch's host and
GPU generators differ): tests that generate on the device hand the device's
values to the oracle.

The five workloads stand in for the pages' own (a 27B model's 64k-context
cache, an 8-KV-head 32-layer Llama-class cache, Wikitext/LongBench text),
which are not available here; sizes follow the layers those models have.
"""

import hashlib
import math
from dataclasses import dataclass, field, replace

import torch

D = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hkv: int
    Hq: int
    T: int
    N: int                      # precision tail length
    kcodec: str
    vcodec: str
    basis: str                  # "plain" | "hadamard" | "lowrank"
    sm_scale: float
    q_scale: float = 1.0
    layers: int = 1
    seed: int = 0
    lowrank: tuple = ()         # ((rank, bits), ...) per kv head
    layer_codecs: tuple = ()    # per-layer codec names (VBR)

    def with_(self, **kw):
        return replace(self, **kw)


INV_SQRT_D = 1.0 / math.sqrt(D)
COBRA_TABLE = ((128, 1), (64, 2), (32, 4), (16, 4), (64, 3), (128, 1), (32, 2), (64, 3))
VBR_CODECS = ("f16", "q8_0", "q4_0", "q2_0")

WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hkv=1, Hq=1, T=256, N=0, kcodec="q4_0", vcodec="q4_0",
                     basis="plain", sm_scale=INV_SQRT_D),
    "gqa4_q8k_q4v_tail1024": Workload("gqa4_q8k_q4v_tail1024", B=1, Hkv=8, Hq=32, T=32768,
                                      N=1024, kcodec="q8_0", vcodec="q4_0", basis="plain",
                                      sm_scale=1.0, q_scale=INV_SQRT_D),
    "kvarn_q3_tail2048": Workload("kvarn_q3_tail2048", B=4, Hkv=8, Hq=48, T=65536, N=2048,
                                  kcodec="q3_0", vcodec="q3_0", basis="hadamard",
                                  sm_scale=INV_SQRT_D),
    "vbr_32layer": Workload("vbr_32layer", B=1, Hkv=8, Hq=32, T=131072, N=0, kcodec="f16",
                            vcodec="f16", basis="plain", sm_scale=INV_SQRT_D, layers=32),
    "lowrank_1bpd": Workload("lowrank_1bpd", B=8, Hkv=8, Hq=32, T=131072, N=0, kcodec="",
                             vcodec="", basis="lowrank", sm_scale=INV_SQRT_D,
                             lowrank=COBRA_TABLE),
}
ORDER = ["tiny", "gqa4_q8k_q4v_tail1024", "kvarn_q3_tail2048", "vbr_32layer", "lowrank_1bpd"]


def chunk_seed(seed, *key):
    h = hashlib.sha256(repr((seed,) + tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, *key):
    g = torch.Generator(device=device)
    g.manual_seed(chunk_seed(seed, *key))
    return g


def _normal(shape, device, seed, *key):
    return torch.randn(shape, generator=_gen(device, seed, *key), device=device,
                       dtype=torch.float32)


def _student_t4(shape, device, seed, *key):
    g = _gen(device, seed, *key)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    u1 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float64)
    u2 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float64)
    chi2 = -2.0 * (torch.log(u1) + torch.log(u2))          # chi-square, 4 dof
    return (z / torch.sqrt(chi2 / 4.0)).to(torch.float32)


def vbr_schedule(wl):
    """Per-layer codec: a seeded permutation of layers/4 copies of each codec."""
    n = wl.layers
    base = [VBR_CODECS[i % 4] for i in range(n)]
    g = _gen("cpu", wl.seed, "vbr-schedule")
    perm = torch.randperm(n, generator=g).tolist()
    return tuple(base[p] for p in perm)


def channel_scales(wl, layer, which, h):
    """Per-channel multipliers of head h (host tensor [128], fp64)."""
    if wl.name.startswith("gqa4") and which == "k" or wl.name.startswith("vbr"):
        return torch.exp(_normal((D,), "cpu", wl.seed, "chscale", layer, which, h)).double()
    if wl.name == "tiny":
        s = torch.ones(D, dtype=torch.float64)
        s[3] = s[77] = 20.0
        return s
    if wl.name.startswith("kvarn") and which == "k":
        g = _gen("cpu", wl.seed, "outliers", layer, h)
        s = torch.ones(D, dtype=torch.float64)
        s[torch.randperm(D, generator=g)[:4]] = 30.0
        return s
    return torch.ones(D, dtype=torch.float64)


def basis(wl, layer, h):
    """Seeded orthonormal 128x128 basis of head h (stand-in for a per-head SVD)."""
    g = _gen("cpu", wl.seed, "basis", layer, h)
    Z = torch.randn((D, D), generator=g, dtype=torch.float64)
    Q, R = torch.linalg.qr(Z)
    return Q * torch.sign(torch.diagonal(R))[None, :]


def _lowrank_alpha(rank):
    return {16: 2.0, 32: 1.0, 64: 0.5, 128: 0.25}[rank]


def head_rows(wl, layer, which, b, h, T, device="cpu", t0=0):
    """Rows [T, 128] (binary32) of K ("k") or V ("v") for (layer, b, h),
    tokens t0 .. t0+T-1 of that chunk's stream (generated in 4096-token
    pieces so any token range regenerates identically)."""
    piece = 4096
    out = torch.empty((T, D), dtype=torch.float32, device=device)
    p0, p1 = t0 // piece, (t0 + T + piece - 1) // piece
    for p in range(p0, p1):
        rows = _piece(wl, layer, which, b, h, p, piece, device)
        lo, hi = max(t0, p * piece), min(t0 + T, (p + 1) * piece)
        out[lo - t0: hi - t0] = rows[lo - p * piece: hi - p * piece]
    return out


def _piece(wl, layer, which, b, h, p, n, device):
    key = ("rows", layer, which, b, h, p)
    if wl.basis == "lowrank" and which == "k":
        rank = wl.lowrank[h][0]
        lam = torch.arange(1, D + 1, dtype=torch.float64) ** (-_lowrank_alpha(rank))
        Z = _normal((n, D), device, wl.seed, *key).double()
        U = basis(wl, layer, h).to(device)
        return ((Z * lam.to(device).sqrt()[None, :]) @ U.T * 3.0).to(torch.float32)
    if wl.name.startswith("kvarn") and which == "k":
        x = _student_t4((n, D), device, wl.seed, *key)
    else:
        x = _normal((n, D), device, wl.seed, *key)
    s = channel_scales(wl, layer, which, h).to(device=device, dtype=torch.float32)
    return x * s[None, :]


def layer_rows(wl, layer, which, T=None, device="cpu", t0=0):
    """K or V of one layer: [B, T, Hkv, 128] binary32."""
    T = wl.T if T is None else T
    out = torch.empty((wl.B, T, wl.Hkv, D), dtype=torch.float32, device=device)
    for b in range(wl.B):
        for h in range(wl.Hkv):
            out[b, :, h, :] = head_rows(wl, layer, which, b, h, T, device, t0)
    return out


def queries(wl, layer, device="cpu", step=0):
    """q: [B, Hq, 128] binary32."""
    return _normal((wl.B, wl.Hq, D), device, wl.seed, "q", layer, step) * wl.q_scale


def kvarn_normalizers(wl, layer, which, calib_tokens=4096):
    """w = 1/sigma per (kv head, channel), sigma the population std of the
    channel over the first ``calib_tokens`` tokens of batch entry 0 (a
    calibration prefix).  Returns [Hkv, 128] binary32 (host)."""
    n = min(calib_tokens, wl.T)
    w = torch.empty((wl.Hkv, D), dtype=torch.float32)
    for h in range(wl.Hkv):
        x = head_rows(wl, layer, which, 0, h, n).double()
        sigma = x.std(dim=0, unbiased=False)
        w[h] = (1.0 / sigma).to(torch.float32)
    return w


def peaked_queries(wl, k, n, device="cpu", layer=0, recent=1024, targets=(6, 2), strength=9.0,
                   step=0):
    """Queries that attend to a few tokens (the quality sweep's stand-in for a
    model's attention).  For each (query, batch entry, query head), `targets`
    = (a, b) tokens are drawn among the newest `recent` and among the older
    ones; with s the channel scales of the kv head's keys and z_j = k_j / s,
    q = strength * sqrt(128) * sum_j (z_j / s) / |z_j|^2 + N(0, 1) / sqrt(128):
    a target's own term in q . k_j / sqrt(128) is `strength`, and the
    channels the scales blow up (outliers) weigh no more than the others.
    k: [B, T, Hkv, 128] (the keys, on `device`).  Returns [n, B, Hq, 128]."""
    B, T, Hkv, _ = k.shape
    G = wl.Hq // Hkv
    g = _gen("cpu", wl.seed, "peaked", step)
    out = torch.empty((n, B, wl.Hq, D), dtype=torch.float32, device=device)
    scales = [channel_scales(wl, layer, "k", h).to(device) for h in range(Hkv)]
    a, b = targets
    lo = max(0, T - recent)
    for i in range(n):
        for bb in range(B):
            for hq in range(wl.Hq):
                idx = []
                if T - lo > 0 and a > 0:
                    idx += (lo + torch.randint(0, T - lo, (a,), generator=g)).tolist()
                if lo > 0 and b > 0:
                    idx += torch.randint(0, lo, (b,), generator=g).tolist()
                s = scales[hq // G]
                z = k[bb, idx, hq // G, :].double() / s
                dirs = (z / s) / (z * z).sum(-1, keepdim=True)
                noise = torch.randn((D,), generator=g, dtype=torch.float64).to(device) * INV_SQRT_D
                out[i, bb, hq] = (strength * math.sqrt(D) * dirs.sum(0) + noise).to(torch.float32)
    return out
