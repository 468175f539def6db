"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the prefix of T - 1 tokens appended by the library, then
one decode step through the one-call entry point (append of the last token
and decode in the same launch, default split plan).

Inputs are device-generated; the oracle then checks, after the step:

* 32k GQA workload: every K/V code, scale and tail byte of all 8 kv heads
  bit-exact against the oracle's encoding of the same inputs, and all 32
  query heads' outputs against the oracle's decode of that cache;
* the other workloads (too large to re-encode whole on the host at once):
  every (batch, kv head) unit, one at a time over its whole context: stored codes
  under the tie rule of tests/helpers.py, and the unit's query heads'
  outputs against the oracle's attention over the unit's device cache;
* the VBR workload: one layer per codec of the schedule at full context,
  every kv head's codes bit-exact and every unit's outputs checked, and the
  per-step f16 -> q8_0 transcode of a full layer (every head bit-exact).

Each test prints what it checked; inputs are seeded (synth) and generated
on the device (chunks regenerate identically on the same device type)."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
from oracle import attention
from oracle.codecs import CODECS
from oracle.layout import untile_plane, unpack_rows
from oracle.rounding import f16_from_bits
import synth
from tests import helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _build(gpu, wl, layer=0, codec=None):
    """Device cache of one layer after one decode step: T-1 tokens appended,
    then the one-call step (append token T-1 + decode).  Returns the step's
    output as float64 numpy [B][Hq][128] with the cache."""
    gk, gv, ok_, ov = H.specs(wl, layer, kcodec=codec, vcodec=codec)
    capacity = (wl.T + 63) // 64 * 64
    cache = H.new_cache(wl, capacity, gk, gv, gpu)
    k = synth.layer_rows(wl, layer, "k", device=gpu)
    v = synth.layer_rows(wl, layer, "v", device=gpu)
    q = synth.queries(wl, layer, device=gpu)
    cache.append(k[:, : wl.T - 1], v[:, : wl.T - 1])
    out = cache.append_decode(k[:, wl.T - 1:].contiguous(), v[:, wl.T - 1:].contiguous(), q, wl.sm_scale)
    torch.cuda.synchronize()
    assert cache.n_tokens == wl.T
    return cache, k, v, ok_, ov, out.cpu().numpy().astype(np.float64), q.cpu().numpy()


def _head_slice_offsets(spec, B, Hkv, capacity, b, h):
    co = so = 0
    for bb in range(B):
        for hh in range(Hkv):
            if (bb, hh) == (b, h):
                return co, so
            co += capacity * OL.head_row_bytes(spec, hh)
            so += capacity * OL.head_nblk(spec, hh)
    raise AssertionError


def _unpack_head(cache, name, spec, b, h, T):
    """Device encoding of one (b, kv head) over its first T rows."""
    buf = cache.bufs[name]
    codec = spec.codec_of(h)
    R = OL.head_row_bytes(spec, h)
    co, so = _head_slice_offsets(spec, cache.batch, cache.n_kv_heads, cache.capacity, b, h)
    rows = untile_plane(buf["codes"][co: co + cache.capacity * R].cpu().numpy(), R)[:T]
    vals = unpack_rows(rows, codec, spec.width(h), spec.block_len(h))
    if CODECS[codec][0] == "f16":
        return {"values": vals}
    nb = OL.head_nblk(spec, h)
    sc = buf["scales"].view(torch.int16)[so: so + cache.capacity * nb].cpu().numpy().view(np.uint16)
    out = {"codes": vals, "scales": f16_from_bits(sc.reshape(cache.capacity, nb)[:T]), "mins": None}
    if CODECS[codec][0] == "1":
        mn = buf["mins"].view(torch.int16)[so: so + cache.capacity * nb].cpu().numpy().view(np.uint16)
        out["mins"] = f16_from_bits(mn.reshape(cache.capacity, nb)[:T])
    return out


def _tail_rows(cache, name, b, h):
    """Device tail ring of (b, h): binary16 [N, 128]."""
    N = cache.tail_len
    plane = b * cache.n_kv_heads + h
    raw = cache.bufs[name]["tail"][plane * N * 256: (plane + 1) * N * 256].cpu().numpy()
    rows = untile_plane(raw, 256)
    return unpack_rows(rows, "f16", 128, 128).astype(np.float16)


def _unit_outputs(wl, kenc, venc, ktail, vtail, kspec, vspec, h, qb):
    """Oracle outputs of kv head h's query heads over one unit's cache."""
    T, N = wl.T, wl.N
    K = OL.dequant_head(kenc, kspec, h)[:T]
    V = OL.dequant_head(venc, vspec, h)[:T]
    if N > 0:
        for t in range(max(0, T - N), T):
            K[t] = ktail[t % N].astype(np.float64)
            V[t] = vtail[t % N].astype(np.float64)
    G = wl.Hq // wl.Hkv
    return attention.attend(qb[h * G:(h + 1) * G], K[:, None, :], V[:, None, :], wl.sm_scale)


def _check_units(wl, cache, k, v, ok_, ov, out, qh, units, rotated):
    G = wl.Hq // wl.Hkv
    worst = 0.0
    for (b, h) in units:
        xk = k[b, :, h, :].cpu().numpy()
        xv = v[b, :, h, :].cpu().numpy()
        kenc = _unpack_head(cache, "k", ok_, b, h, wl.T)
        venc = _unpack_head(cache, "v", ov, b, h, wl.T)
        for x, enc, spec in ((xk, kenc, ok_), (xv, venc, ov)):
            if rotated:
                H.check_rotated_head(x, enc, spec, h)
            else:
                ref = OL.encode_head(x, spec, h)
                for key in ("codes", "scales", "mins"):
                    if ref.get(key) is not None:
                        assert np.array_equal(enc[key], ref[key]), (b, h, key)
        kt = vt = None
        if wl.N > 0:
            kt, vt = _tail_rows(cache, "k", b, h), _tail_rows(cache, "v", b, h)
            ring_k = OL.tail_ring(xk[None, :, None, :], wl.N)[0, 0]
            ring_v = OL.tail_ring(xv[None, :, None, :], wl.N)[0, 0]
            assert np.array_equal(kt.view(np.uint16), ring_k.view(np.uint16))
            assert np.array_equal(vt.view(np.uint16), ring_v.view(np.uint16))
        ref = _unit_outputs(wl, kenc, venc, kt, vt, ok_, ov, h, qh[b])
        err = float(np.max(np.abs(out[b, h * G:(h + 1) * G] - ref)))
        worst = max(worst, err)
        assert err <= H.ATOL, (wl.name, b, h, err)
        bound = H.unit_bound(qh[b, h * G:(h + 1) * G], kenc, venc, kt, vt, ok_, ov, h, wl.T, wl.N,
                             wl.sm_scale)
        H.check_precision(out[b, h * G:(h + 1) * G], ref, bound, "%s unit (%d, %d)" % (wl.name, b, h))
    print("%s: %d units over T=%d, worst max-abs %.3g" % (wl.name, len(units), wl.T, worst))


def test_gqa4_32k_all_heads(gpu):
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"]
    cache, k, v, ok_, ov, out, qh = _build(gpu, wl)
    kx, vx = k.cpu().numpy(), v.cpu().numpy()
    for name, x, spec in (("k", kx, ok_), ("v", vx, ov)):
        _, packed, tail = H.oracle_layer_bytes(x, spec, cache.capacity, wl.N)
        dev = H.download(cache, name)
        assert np.array_equal(dev["codes"][: packed["codes"].size], packed["codes"]), name
        assert np.array_equal(dev["scales"], packed["scales"]), name
        assert np.array_equal(dev["tail"], tail), name
    units = [(0, h) for h in range(wl.Hkv)]
    _check_units(wl, cache, k, v, ok_, ov, out, qh, units, rotated=False)


@pytest.mark.parametrize("entries", [(0, 1), (2, 3)])
def test_kvarn_q3_64k_all_units(gpu, entries):
    # every kv head of these batch entries (two tests, each well inside the
    # per-test limit)
    wl = synth.WORKLOADS["kvarn_q3_tail2048"]
    cache, k, v, ok_, ov, out, qh = _build(gpu, wl)
    units = [(b, h) for b in entries for h in range(wl.Hkv)]
    _check_units(wl, cache, k, v, ok_, ov, out, qh, units, rotated=True)


@pytest.mark.parametrize("entries", [(0, 1, 2, 3), (4, 5, 6, 7)])
def test_lowrank_128k_all_units(gpu, entries):
    # every kv head (every rank and bit width of the table) of these batch
    # entries; two tests so that each stays well inside the per-test limit
    wl = synth.WORKLOADS["lowrank_1bpd"]
    cache, k, v, ok_, ov, out, qh = _build(gpu, wl)
    units = [(b, h) for b in entries for h in range(wl.Hkv)]
    _check_units(wl, cache, k, v, ok_, ov, out, qh, units, rotated=True)


@pytest.mark.parametrize("codec", ["f16", "q8_0", "q4_0", "q2_0"])
def test_vbr_128k_layer_all_heads(gpu, codec):
    """The first layer of each codec in the 32-layer schedule: codes of every
    kv head bit-exact, every unit's outputs against the oracle; for the f16
    layer, the f16 -> q8_0 transcode of every head bit-exact."""
    wl = synth.WORKLOADS["vbr_32layer"]
    layer = list(synth.vbr_schedule(wl)).index(codec)
    cache, k, v, ok_, ov, out, qh = _build(gpu, wl, layer, codec)
    G = wl.Hq // wl.Hkv
    worst = 0.0
    for h in range(wl.Hkv):
        xk, xv = k[0, :, h, :].cpu().numpy(), v[0, :, h, :].cpu().numpy()
        kenc = _unpack_head(cache, "k", ok_, 0, h, wl.T)
        venc = _unpack_head(cache, "v", ov, 0, h, wl.T)
        rk, rv = OL.encode_head(xk, ok_, h), OL.encode_head(xv, ov, h)
        for enc, ref in ((kenc, rk), (venc, rv)):
            for key in ("codes", "scales", "mins", "values"):
                if ref.get(key) is not None:
                    assert np.array_equal(enc[key], ref[key]), (codec, h, key)
        ref = _unit_outputs(wl, kenc, venc, None, None, ok_, ov, h, qh[0])
        err = float(np.max(np.abs(out[0, h * G:(h + 1) * G] - ref)))
        worst = max(worst, err)
        assert err <= H.ATOL, (codec, h, err)
        bound = H.unit_bound(qh[0, h * G:(h + 1) * G], kenc, venc, None, None, ok_, ov, h, wl.T, 0,
                             wl.sm_scale)
        H.check_precision(out[0, h * G:(h + 1) * G], ref, bound, "vbr %s head %d" % (codec, h))
    if codec == "f16":
        dst = cache.transcode("q8_0", "q8_0")
        torch.cuda.synchronize()
        _, _, okd, ovd = H.specs(wl, layer, kcodec="q8_0", vcodec="q8_0")
        for h in range(wl.Hkv):
            for name, spec_s, spec_d in (("k", ok_, okd), ("v", ov, ovd)):
                src = _unpack_head(cache, name, spec_s, 0, h, wl.T)
                got = _unpack_head(dst, name, spec_d, 0, h, wl.T)
                ref = OL.transcode_head(src, spec_s, spec_d, h)
                for key in ("codes", "scales"):
                    assert np.array_equal(got[key], ref[key]), ("transcode", name, h, key)
    print("vbr layer %d (%s): %d heads, worst max-abs %.3g" % (layer, codec, wl.Hkv, worst))
    del cache, k, v
    torch.cuda.empty_cache()
