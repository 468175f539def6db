"""Single-query decode attention, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: the forum thread on decode memory bandwidth (second post) describes
the computation: the newest token's query is dotted with every cached key,
the scores go through a softmax, and the resulting weights average the cached
values.  Grouped-query attention (the KV-COBRA explainer notes the method
composes with it) lets ``G = Hq / Hkv`` query heads share one KV head;
reading: query head ``h`` uses KV head ``h // G``.
"""

import numpy as np


def attend(q, K, V, sm_scale):
    """One query per head against a cache.

    q: [Hq, D]; K: [T, Hkv, D]; V: [T, Hkv, Dv]; returns [Hq, Dv] (fp64).
    ``s_t = sm_scale <q_h, k_t>``, ``p = exp(s - max s) / sum``,
    ``o_h = sum_t p_t v_t``.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq = q.shape[0]
    T, Hkv = K.shape[0], K.shape[1]
    if T == 0:
        raise ValueError("attention over an empty cache is undefined")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // Hkv
    out = np.empty((Hq, V.shape[2]), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = sm_scale * (K[:, g, :] @ q[h])
        p = np.exp(s - np.max(s))
        p /= np.sum(p)
        out[h] = p @ V[:, g, :]
    return out


def attend_batch(q, K, V, sm_scale):
    """Batched form.  q: [B, Hq, D]; K, V: [B, T, Hkv, D]."""
    return np.stack([attend(q[b], K[b], V[b], sm_scale) for b in range(q.shape[0])])
