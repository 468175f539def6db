"""Quality sweep on the GPU path (codec x tail x plain/KVarN), small context.

What the pages report qualitatively, checked on synthetic data (outlier-heavy
Student-t keys, normal values, queries that attend to a few recent and a few
older tokens):
 - fewer bits, larger divergence (the codec ladder of the release notes' KLD
   table is monotone at every tail length);
 - the variance-normalised rotation (KVarN) beats the plain codec at equal
   bits when keys have outlier channels (release notes, KVarN section and
   KLD table);
 - a precision tail never hurts on average (mean KL at tail 1024 and 2048 is
   at most the tail-0 value), in binary16 and in bfloat16;
 - the decode kernel agrees with plain attention over the library's own
   read-back of the cache (the decode contract, 2e-3 max-abs)."""

import pytest

import synth
from quantized_kv_cache_kvq_amd import quality as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rows(gpu):
    wl = synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=1, Hq=32, T=8192)
    k = synth.layer_rows(wl, 0, "k", device=gpu)
    v = synth.layer_rows(wl, 0, "v", device=gpu)
    q_all = synth.peaked_queries(wl, k, 2, device=gpu)
    out = Q.sweep(k, v, q_all, wl.sm_scale, codecs=("q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0"))
    return {(r["basis"], r["codec"], r["tail"], r["tail_format"]): r for r in out}


def test_divergence_grows_as_bits_shrink(rows):
    ladder = ("q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0")
    for basis in Q.BASES:
        for tail in Q.TAILS:
            kl = [rows[(basis, c, tail, "-" if tail == 0 else "f16")]["kl_mean"] for c in ladder]
            assert all(a < b for a, b in zip(kl, kl[1:])), (basis, tail, kl)


def test_kvarn_beats_plain_at_equal_bits(rows):
    for codec in ("q8_0", "q6_0", "q5_0", "q4_0", "q3_0"):
        for tail in Q.TAILS:
            f = "-" if tail == 0 else "f16"
            assert rows[("hadamard", codec, tail, f)]["kl_mean"] < rows[("plain", codec, tail, f)]["kl_mean"], \
                (codec, tail)


def test_tail_never_hurts_on_average(rows):
    for basis in Q.BASES:
        for codec in ("q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0"):
            k0 = rows[(basis, codec, 0, "-")]["kl_mean"]
            for tail in (1024, 2048):
                for fmt in ("f16", "bf16"):
                    assert rows[(basis, codec, tail, fmt)]["kl_mean"] <= k0 * (1 + 1e-6), (basis, codec, tail, fmt)


def test_decode_matches_attention_over_readback(rows):
    for key, r in rows.items():
        assert r["decode_vs_readback_maxabs"] <= 2e-3, (key, r["decode_vs_readback_maxabs"])
