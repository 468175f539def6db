"""The quality sweep's metrics, pinned on the CPU.

The sweep (``bench.py --quality``) reports KL(p || p_hat) between one query's
exact attention weights and those over the packed keys, and the relative
error of the output.  Its fp64 attention (``quality._exact``) is checked here
against the oracle's attention (``oracle.attention``: the forum post's
score / softmax / weighted sum), its log-weights against SciPy's
``log_softmax``, the KL sum against ``scipy.special.rel_entr`` and against
the closed form for two distributions that differ on a known set of tokens,
and the bit accounting against the oracle's.  The device half of the sweep
(append, decode, read-back) is covered by the GPU parity tests.
"""

import numpy as np
import pytest
import torch
from scipy.special import log_softmax, rel_entr

import oracle.attention as OA
import oracle.budget as OB
from quantized_kv_cache_kvq_amd import quality as Q


def _case(seed, B=2, T=37, Hkv=2, G=3):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, T, Hkv, 128))
    V = rng.standard_normal((B, T, Hkv, 128))
    q = rng.standard_normal((B, Hkv * G, 128))
    return q, K, V, G


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_attention_equals_oracle(seed):
    q, K, V, G = _case(seed)
    sm = 128 ** -0.5
    logp, o = Q._exact(torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V), G, sm)
    ref = OA.attend_batch(q, K, V, sm)
    assert np.max(np.abs(o.numpy() - ref)) < 1e-12
    # log-weights: SciPy's log_softmax of the same scores, head h on kv head h // G
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            s = sm * (K[b, :, h // G, :] @ q[b, h])
            assert np.max(np.abs(logp[b, h].numpy() - log_softmax(s))) < 1e-12


def test_kl_matches_rel_entr_and_is_zero_on_equal_weights():
    rng = np.random.default_rng(7)
    s, sh = rng.standard_normal((4, 50)), rng.standard_normal((4, 50))
    lp, lph = torch.from_numpy(log_softmax(s, axis=-1)), torch.from_numpy(log_softmax(sh, axis=-1))
    kl = Q.kl_nats(lp, lph).numpy()
    ref = rel_entr(np.exp(lp.numpy()), np.exp(lph.numpy())).sum(-1)
    assert np.max(np.abs(kl - ref)) < 1e-12
    assert np.all(kl > 0)                                   # Gibbs' inequality, p != p_hat
    assert np.max(np.abs(Q.kl_nats(lp, lp).numpy())) == 0.0


def test_kl_closed_form_two_level():
    # p uniform over n tokens; p_hat puts weight a/k on k of them and
    # (1-a)/(n-k) on the rest: KL = (k/n) log(k/(n a)) + ((n-k)/n) log((n-k)/(n(1-a)))
    n, k, a = 64, 8, 0.3
    p = np.full(n, 1.0 / n)
    ph = np.concatenate([np.full(k, a / k), np.full(n - k, (1 - a) / (n - k))])
    kl = float(Q.kl_nats(torch.from_numpy(np.log(p)), torch.from_numpy(np.log(ph))))
    closed = (k / n) * np.log(k / (n * a)) + ((n - k) / n) * np.log((n - k) / (n * (1 - a)))
    assert abs(kl - closed) < 1e-14


@pytest.mark.parametrize("codec", ["q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0",
                                   "q8_1", "q4_1", "q2_1", "q1_1", "f16"])
def test_bits_per_value_matches_oracle_accounting(codec):
    assert Q.bits_per_value(codec) == OB.bits_per_value(codec)
