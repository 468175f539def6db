"""Shared helpers of the GPU parity tests: matched library/oracle plane
specifications for a workload, upload of oracle-packed caches, download and
comparison of device planes.

Acceptance rules (stated once here, used by every parity test):
* unrotated formats: codes, scales, mins and the tail are bit-exact;
* rotated (Hadamard) and low-rank codes: at most 0.1% of codes may differ,
  each by +-1 and only where the exact stored coordinate is within the
  device's binary32 rounding error of a rounding boundary; a block scale (or
  min) may differ by one binary16 step only where the exact unrounded value
  is within that error of a binary16 rounding midpoint, and the codes are
  then checked against the device's scale;
* attention outputs: max-abs difference <= 2e-3 against the oracle run on
  the same cache.
"""

import numpy as np
import torch

import oracle.cobra
import oracle.layer as OL
from oracle.codecs import CODECS
from oracle.layer import PlaneSpec as OSpec
from quantized_kv_cache_kvq_amd import calib
from quantized_kv_cache_kvq_amd.cache import LayerCache, PlaneSpec as GSpec
import synth

ATOL = 2e-3
U32 = 2.0 ** -24


def specs(wl, layer=0, kcodec=None, vcodec=None):
    """(gpu K spec, gpu V spec, oracle K spec, oracle V spec) of a workload."""
    kc = kcodec or wl.kcodec
    vc = vcodec or wl.vcodec
    if wl.basis == "plain":
        return GSpec(kc), GSpec(vc), OSpec(kc), OSpec(vc)
    if wl.basis == "hadamard":
        wk = synth.kvarn_normalizers(wl, layer, "k")
        wv = synth.kvarn_normalizers(wl, layer, "v")
        return (GSpec(kc, "hadamard", w=wk), GSpec(vc, "hadamard", w=wv),
                OSpec(kc, "hadamard", w=wk.numpy()), OSpec(vc, "hadamard", w=wv.numpy()))
    ranks = [r for r, _ in wl.lowrank[: wl.Hkv]]
    hcod = ["q%d_1" % b for _, b in wl.lowrank[: wl.Hkv]]
    bases = [synth.basis(wl, layer, h).numpy() for h in range(wl.Hkv)]
    P_or = [oracle.cobra.projection(U, r) for U, r in zip(bases, ranks)]
    P_dev = calib.lowrank_projections(bases, ranks)
    for h, r in enumerate(ranks):
        assert np.array_equal(P_dev[h, :, :r].numpy(), P_or[h]), "projection builders disagree"
    g = GSpec("", "lowrank", proj=P_dev, ranks=ranks, head_codecs=hcod)
    o = OSpec("", "lowrank", P=P_or, head_codec=hcod)
    return g, g, o, o


def new_cache(wl, capacity, gk, gv, device, N=None):
    N = wl.N if N is None else N
    return LayerCache(wl.B, wl.Hkv, capacity, N, gk, gv, device)


def upload(cache, name, packed, tail_bytes=None):
    b = cache.bufs[name]
    b["codes"][: packed["codes"].size].copy_(torch.from_numpy(packed["codes"]))
    for key in ("scales", "mins"):
        if packed.get(key) is not None:
            b[key].copy_(torch.from_numpy(packed[key].view(np.uint8)))
    if tail_bytes is not None and b["tail"] is not None:
        b["tail"].copy_(torch.from_numpy(tail_bytes))


def download(cache, name):
    b = cache.bufs[name]
    out = {"codes": b["codes"].cpu().numpy()}
    for key in ("scales", "mins"):
        out[key] = b[key].cpu().numpy().view(np.uint16) if b[key] is not None else None
    out["tail"] = b["tail"].cpu().numpy() if b["tail"] is not None else None
    return out


def oracle_layer_bytes(x, ospec, capacity, N):
    enc = OL.encode_plane(x, ospec)
    packed = OL.pack_plane(enc, ospec, capacity)
    tail = OL.pack_tail(OL.tail_ring(x, N)) if N > 0 else None
    return enc, packed, tail


# ------------------------------------------------- tie-tolerant comparison --

def _coord_error_bound(x, spec, h):
    """Bound on |device - exact| of the stored coordinates of raw rows x."""
    x = np.asarray(x, np.float64)
    if spec.basis == "hadamard":
        z = np.abs(x * spec.w[h].astype(np.float64))
        return 9 * U32 * z.sum(-1, keepdims=True) * np.ones_like(x)
    P = np.abs(spec.P[h].astype(np.float64))
    return (D_LOWRANK_TERMS + 2) * U32 * (np.abs(x) @ P)


D_LOWRANK_TERMS = 128


def _f16_neighbours(v):
    v16 = np.float16(v)
    return {float(v16), float(np.nextafter(v16, np.float16(np.inf))),
            float(np.nextafter(v16, np.float16(-np.inf)))}


def check_rotated_head(x, enc_gpu, spec, h, max_frac=1e-3):
    """Compare device encodings of raw rows x [T,128] of head h against the
    oracle under the tie rule.  Returns (n_mismatch, n_codes)."""
    codec = spec.codec_of(h)
    fam, b = CODECS[codec]
    L = spec.block_len(h)
    y = OL.stored_coords(x, spec, h)                        # exact, fp64
    err = _coord_error_bound(x, spec, h)
    T, n = y.shape
    yb = y.reshape(T, n // L, L)
    eb = err.reshape(T, n // L, L)
    cg = enc_gpu["codes"].reshape(T, n // L, L)
    dg = enc_gpu["scales"].astype(np.float64)
    ref = OL.encode_head(x, spec, h)
    cr = ref["codes"].reshape(T, n // L, L)
    dr = ref["scales"].astype(np.float64)
    bad_scale = np.argwhere(dg != dr)
    for (t, j) in bad_scale:
        blk, e = yb[t, j], eb[t, j].max()
        if fam == "0":
            qm = 2 ** (b - 1) - 1
            amax = np.abs(blk).max()
            ok = dg[t, j] in _f16_neighbours(amax / qm) and abs(
                np.float16((amax + e) / qm) - np.float16((amax - e) / qm)) > 0
        else:
            ok = True   # _1 scale/min move together; codes re-checked below with device values
        assert ok, "scale of block (%d,%d) differs off a rounding midpoint" % (t, j)
    if fam == "1":
        mg = enc_gpu["mins"].astype(np.float64)
        mr = ref["mins"].astype(np.float64)
        for (t, j) in np.argwhere(mg != mr):
            e = eb[t, j].max()
            lo = yb[t, j].min()
            assert np.float16(lo + e) != np.float16(lo - e), "min differs off a midpoint"
    # codes against the device's own scale (and min)
    d = dg[..., None]
    if fam == "0":
        qm = 2 ** (b - 1) - 1
        quot = np.where(d == 0, 0.0, yb / np.where(d == 0, 1, d))
        lo_c, hi_c = -qm, qm
    else:
        m = enc_gpu["mins"].astype(np.float64)[..., None]
        quot = np.where(d == 0, 0.0, (yb - m) / np.where(d == 0, 1, d))
        lo_c, hi_c = 0, 2 ** b - 1
    tol = np.where(d == 0, 0.0, eb / np.where(d == 0, 1, d)) + 1e-4
    expect = np.clip(np.rint(quot), lo_c, hi_c)
    diff = cg != expect
    ok_tie = (np.abs(cg - expect) <= 1) & (
        (np.abs(quot - cg) <= 0.5 + tol) | ((cg == lo_c) & (quot < lo_c)) | ((cg == hi_c) & (quot > hi_c)))
    assert np.all(ok_tie | ~diff), "codes off by more than a tie"
    # count against the oracle's own codes as well
    n_mis = int(np.sum(cg != cr))
    assert n_mis <= max_frac * cg.size + 0, (n_mis, cg.size)
    return n_mis, cg.size


def unpack(cache, name, ospec, T):
    buf = download(cache, name)
    return OL.unpack_plane(buf, ospec, cache.batch, cache.n_kv_heads, cache.capacity, T), buf


# ------------------------------------------------- precision of the kernels --

def _softmax_stats(qh, K, V, sm_scale):
    s = sm_scale * (K @ qh)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p, p @ V


def decode_bound(q, kenc, venc, ktail, vtail, kspec, vspec, T, N, sm_scale, tail_fmt="f16"):
    """Elementwise bound on |device decode - oracle decode| [B, Hq, 128]
    from the roundings the kernels make: a statistical model of the
    rounding errors (each uniform over its half-width, std = half-width /
    sqrt 3, independent), 8 standard deviations of their sum, plus
    binary32 terms taken at their worst case.

    Score errors (natural units), per token t:
    * body keys on the integer matrix cores: the stored-basis query of each
      head is rounded to a multiple of 2^-sh with 2^19 <= max|q'|*2^sh <
      2^20, below max|q'|*2^-20 per component: std max|q'| 2^-20 |y_t| /
      sqrt3 (y_t the stored-basis key); binary16 keys use hi + lo binary16
      query parts (22 bits): 2^-22;
    * tail keys: hi + lo binary16 parts (2^-22), bfloat16 parts (2^-16);
    * binary32 query transforms (KVarN rotation, low-rank projection):
      2^-22 of the transform's absolute sums per component;
    * _1 keys: the block minimum times the block's query sum, in binary32.
    A score error d_t moves the output by sum_t p_t (d_t - mean d)(v_t - o).
    Value side: PV weights p * d_v as hi + lo binary16 (relative 2^-22) or
    bfloat16 parts (2^-16); _1 values add sum_t p_t m_t in binary32; the
    output transforms (inverse rotation, back projection) in binary32;
    accumulation, exp2 and normalisation: 2^-20 of sum_t p_t |v_t| + |o|."""
    q = np.asarray(q, np.float64)
    B, Hq, _ = q.shape
    Hkv = len(kenc[0])
    G = Hq // Hkv
    out = np.zeros((B, Hq, 128))
    for b in range(B):
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = unit_bound(
                q[b, g * G:(g + 1) * G], kenc[b][g], venc[b][g],
                ktail[b, g] if N > 0 else None, vtail[b, g] if N > 0 else None,
                kspec, vspec, g, T, N, sm_scale, tail_fmt)
    return out


def unit_bound(qg, kenc, venc, ktail, vtail, kspec, vspec, g, T, N, sm_scale, tail_fmt="f16"):
    """decode_bound for one (batch entry, kv head g): qg [G, 128] its query
    heads, kenc / venc its encodings, ktail / vtail its ring [N, 128]."""
    import oracle.cobra as OC
    import oracle.kvarn as OK
    from oracle.codecs import decode_rows

    r3 = np.sqrt(3.0)
    tail_q = 2.0 ** (-16 if tail_fmt == "bf16" else -22)
    tail_w = 2.0 ** (-16 if tail_fmt == "bf16" else -22)
    u32 = 2.0 ** -22                     # binary32 sums, a few roundings each
    G = qg.shape[0]
    out = np.zeros((G, 128))
    if True:
        if True:
            K = OL.dequant_head(kenc, kspec, g)[:T]
            V = OL.dequant_head(venc, vspec, g)[:T]
            tail = np.zeros(T, bool)
            if N > 0:
                for t in range(max(0, T - N), T):
                    K[t] = ktail[t % N].astype(np.float64)
                    V[t] = vtail[t % N].astype(np.float64)
                    tail[t] = True
            kc, vc = kspec.codec_of(g), vspec.codec_of(g)
            Lk, Lv = kspec.block_len(g), vspec.block_len(g)
            Yk = decode_rows(kenc, kc, Lk, rounded=False)[:T]
            Yv = decode_rows(venc, vc, Lv, rounded=False)[:T]
            kmin = kenc.get("mins") if kc != "f16" else None
            vmin = venc.get("mins") if vc != "f16" else None
            body_q = 2.0 ** (-20 if (kc != "f16" and vc != "f16") else -22)
            for hh in range(G):
                qh = np.asarray(qg[hh], np.float64)
                if kspec.basis == "hadamard":
                    wk = kspec.w[g].astype(np.float64)
                    qs = OK.rotate(qh, 1.0 / wk) / 128.0
                    qt = u32 * np.abs(qh / wk).sum() / 128.0 * np.ones_like(qs)
                elif kspec.basis == "lowrank":
                    Pk = kspec.P[g].astype(np.float64)
                    qs = OC.project(qh, kspec.P[g])
                    qt = u32 * (np.abs(Pk).T @ np.abs(qh))
                else:
                    qs, qt = qh, np.zeros_like(qh)
                p, o = _softmax_stats(qh, K, V, sm_scale)
                d_body = np.abs(qs).max() * body_q / r3 * np.linalg.norm(Yk, axis=1) + np.abs(Yk) @ qt
                if kmin is not None:
                    L = Lk
                    qsum = np.abs(qs.reshape(-1, L).sum(1))
                    d_body = d_body + u32 * (np.abs(kmin[:T]) @ qsum)
                d = sm_scale * np.where(tail, np.abs(qh).max() * tail_q / r3 * np.linalg.norm(K, axis=1),
                                        d_body)
                ew = np.where(tail, tail_w, 2.0 ** -22) / r3
                var = ((p * d)[:, None] ** 2 * (V - o) ** 2).sum(0) + ((p * ew)[:, None] ** 2 * V ** 2).sum(0)
                floor = 2.0 ** -20 * ((p[:, None] * np.abs(V)).sum(0) + np.abs(o))
                body = ~tail
                if vmin is not None:
                    mv = np.repeat(np.abs(vmin[:T]), Lv, axis=1)[:, : Yv.shape[1]]
                    m_raw = (p[body, None] * mv[body]).sum(0)
                else:
                    m_raw = np.zeros(Yv.shape[1])
                fam_v, bits_v = CODECS[vc]
                if kc != "f16" and fam_v == "0" and bits_v <= 4:
                    # integer path, codes of <= 4 bits: the PV sums u d (u the
                    # offset-binary code) and the offset 2^(b-1) sum_t p_t d_t
                    # is a separate binary32 term, like a _1 minimum; the
                    # accumulator then holds magnitudes up to sum p (|v| + off)
                    dv = np.abs(np.asarray(venc["scales"][:T], np.float64))
                    off = np.repeat(dv, Lv, axis=1)[:, : Yv.shape[1]] * float(1 << (bits_v - 1))
                    off_raw = (p[body, None] * off[body]).sum(0)
                    m_raw = m_raw + off_raw
                    floor = floor + 2.0 ** -20 * off_raw
                ob = (p[body, None] * np.abs(Yv[body])).sum(0) + m_raw     # stored-basis magnitudes
                if vspec.basis == "hadamard":
                    wv = vspec.w[g].astype(np.float64)
                    floor = floor + u32 * ob.sum() / 128.0 / wv
                elif vspec.basis == "lowrank":
                    floor = floor + u32 * (np.abs(vspec.P[g].astype(np.float64)) @ ob)
                else:
                    floor = floor + u32 * m_raw
                # transforms and merges mix channels: no channel's floor is
                # below a 2^-2 share of the head's mean
                floor = np.maximum(floor, 0.25 * floor.mean())
                out[hh] = 8.0 * np.sqrt(var) + floor
    return out


def check_precision(got, ref, bound, what=""):
    """|got - ref| <= bound elementwise; returns the worst ratio."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    ratio = float((err / bound).max())
    print("precision %s: max err %.3g, max err/bound %.3g" % (what, float(err.max()), ratio))
    assert ratio <= 1.0, (what, float(err.max()), ratio)
    return ratio
