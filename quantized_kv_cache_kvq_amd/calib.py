"""Host-side calibration helpers: the frozen per-head settings a cache is
built with.

* KVarN normalisers: ``w = 1/sigma`` per (kv head, channel) from a
  calibration sample (BeeLlama v0.4.0 notes, KVarN section: variance
  normalisation before quantising).
* Low-rank projections: ``P_h = RN16(U_h[:, :r] H_r / sqrt(r))`` (KV-COBRA
  explainer: keep the top-r directions of a per-head basis and fuse a
  Hadamard rotation into the same matrix so the kept coordinates have even
  variances).  Stored as [Hkv, 128, 128] binary16 with columns >= r_h zero.
"""

import numpy as np
import torch


def sylvester(n):
    """Order-n Sylvester Hadamard matrix with +-1 entries (n a power of two)."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.concatenate([np.concatenate([H, H], 1), np.concatenate([H, -H], 1)], 0)
    return H


def lowrank_projection(U, rank):
    """Binary16 [128, 128]: the fused projection of basis U (128 x 128,
    orthonormal columns, strongest first) at ``rank``, zero beyond it."""
    U = np.asarray(U, dtype=np.float64)
    P = U[:, :rank] @ sylvester(rank) / np.sqrt(rank)
    out = np.zeros((U.shape[0], U.shape[0]), dtype=np.float16)
    out[:, :rank] = P.astype(np.float16)
    return out


def lowrank_projections(bases, ranks):
    return torch.from_numpy(np.stack([lowrank_projection(U, r) for U, r in zip(bases, ranks)]))


def kvarn_weights(samples):
    """w = 1/sigma per channel from samples [..., n, 128] (population std)."""
    x = torch.as_tensor(samples, dtype=torch.float64)
    sigma = x.reshape(-1, x.shape[-2], x.shape[-1]).std(dim=1, unbiased=False)
    return (1.0 / sigma).to(torch.float32)


def head_spectra(keys):
    """Variances of each head's key directions, largest first: eigenvalues of
    the second-moment matrix of calibration keys [T, Hkv, 128] (the input of
    the per-head rank/bit allocation).  Returns [Hkv, 128] float64 (host)."""
    x = torch.as_tensor(keys, dtype=torch.float64, device="cpu")
    out = []
    for h in range(x.shape[1]):
        xh = x[:, h, :]
        ev = torch.linalg.eigvalsh(xh.T @ xh / xh.shape[0])
        out.append(torch.clamp(ev.flip(0), min=0.0))
    return torch.stack(out)
