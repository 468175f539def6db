#!/usr/bin/env python3
"""Decode-step benchmark of the packed KV cache on one MI355X.

A step is one pass of the hot path over one synthetic batch: append the new
token's K and V to every layer (quantise, pack, tail copy) and decode
attention of every query head over the whole cache -- one kvq_append_decode
call per layer, a single launch where the library fuses the two -- and, for
the mixed-codec workload, one layer transcode.  Inputs are resident in HBM before timing starts.  To
keep the step honest about HBM (the 256 MB Infinity Cache would otherwise
hold a 57 MB cache), consecutive steps rotate over replicas of the cache
whose total size exceeds the Infinity Cache.

Prints one JSON line (rank 0, one GPU):
  value = algorithmic packed-KV bytes read per step / step time  (GB/s)
  roofline = the decode kernels' achieved bytes/s against 8 TB/s
  cpu_baseline = the fp64 oracle decoding a bounded sample on the host.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import synth  # noqa: E402
from quantized_kv_cache_kvq_amd import calib, lib  # noqa: E402
from quantized_kv_cache_kvq_amd.cache import LayerCache, PlaneSpec  # noqa: E402

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
DEFAULT = "gqa4_q8k_q4v_tail1024"
BITS = {c: (16 if c == "f16" else int(c[1])) for c in lib.CODECS}


def row_total_bytes(codec, n=128):
    """Codes + scales (+ mins) of one token of one head."""
    if codec == "f16":
        return 2 * n
    L = min(32, n)
    side = (2 if codec.endswith("_0") else 4) * (n // L)
    return n * BITS[codec] // 8 + side


def layer_bytes(wl, kc, vc, T):
    """Algorithmic bytes one decode of a layer reads at T cached tokens."""
    N = min(wl.N, T)
    body = T - N
    per_head = 0
    if wl.basis == "lowrank":
        for r, b in wl.lowrank[: wl.Hkv]:
            per_head += 2 * row_total_bytes("q%d_1" % b, r)
        per_tok = per_head
    else:
        per_tok = wl.Hkv * (row_total_bytes(kc) + row_total_bytes(vc))
    return wl.B * (body * per_tok + N * wl.Hkv * 2 * 256)


def plane_specs(wl, layer, codec=None):
    if wl.basis == "plain":
        c = codec or wl.kcodec
        return PlaneSpec(c), PlaneSpec(codec or wl.vcodec)
    if wl.basis == "hadamard":
        return (PlaneSpec(wl.kcodec, "hadamard", w=synth.kvarn_normalizers(wl, layer, "k")),
                PlaneSpec(wl.vcodec, "hadamard", w=synth.kvarn_normalizers(wl, layer, "v")))
    ranks = [r for r, _ in wl.lowrank[: wl.Hkv]]
    hc = ["q%d_1" % b for _, b in wl.lowrank[: wl.Hkv]]
    P = calib.lowrank_projections([synth.basis(wl, layer, h).numpy() for h in range(wl.Hkv)], ranks)
    s = PlaneSpec("", "lowrank", proj=P, ranks=ranks, head_codecs=hc)
    return s, s


def build_layer(wl, layer, codec, dev, capacity):
    ks, vs = plane_specs(wl, layer, codec)
    cache = LayerCache(wl.B, wl.Hkv, capacity, wl.N, ks, vs, dev)
    k = synth.layer_rows(wl, layer, "k", device=dev)
    v = synth.layer_rows(wl, layer, "v", device=dev)
    cache.append(k[:, : wl.T - 1], v[:, : wl.T - 1])
    new = (k[:, wl.T - 1:].contiguous(), v[:, wl.T - 1:].contiguous())
    del k, v
    return cache, new


def clone_layer(src):
    dst = LayerCache(src.batch, src.n_kv_heads, src.capacity, src.tail_len, src.kspec,
                     src.vspec, src.device, tail_format=src.tail_format)
    for name in ("k", "v"):
        for key, t in src.bufs[name].items():
            if t is not None:
                dst.bufs[name][key].copy_(t)
    dst.n_tokens = src.n_tokens
    return dst


def setup(wl, dev, replicas):
    """Layer caches (per replica, per layer), new-token inputs and queries."""
    capacity = math.ceil(wl.T / 64) * 64
    codecs = synth.vbr_schedule(wl) if wl.layers > 1 else (None,)
    base, news = [], []
    for layer, codec in enumerate(codecs):
        c, new = build_layer(wl, layer, codec, dev, capacity)
        base.append(c)
        news.append(new)
    reps = [base] + [[clone_layer(c) for c in base] for _ in range(replicas - 1)]
    qs = [synth.queries(wl, layer, device=dev) for layer in range(len(codecs))]
    return reps, news, qs, codecs


def _oracle_specs(wl, layer, codec):
    """Oracle plane descriptions (K, V) of one layer of the workload."""
    import oracle.cobra
    import oracle.layer as OL

    if wl.basis == "plain":
        return OL.PlaneSpec(codec or wl.kcodec), OL.PlaneSpec(codec or wl.vcodec)
    if wl.basis == "hadamard":
        return (OL.PlaneSpec(wl.kcodec, "hadamard", w=synth.kvarn_normalizers(wl, layer, "k").numpy()),
                OL.PlaneSpec(wl.vcodec, "hadamard", w=synth.kvarn_normalizers(wl, layer, "v").numpy()))
    ranks = [r for r, _ in wl.lowrank[: wl.Hkv]]
    P = [oracle.cobra.projection(synth.basis(wl, layer, h).numpy(), r) for h, r in enumerate(ranks)]
    s = OL.PlaneSpec("", "lowrank", P=P, head_codec=["q%d_1" % b for _, b in wl.lowrank[: wl.Hkv]])
    return s, s


def _baseline_units(wl, codecs):
    """Decode units (layer, batch entry, kv head) of one step, ordered so
    that any prefix samples the layers' codecs in proportion."""
    by_codec = {}
    for layer, c in enumerate(codecs):
        by_codec.setdefault(c, []).append(layer)
    order = []
    for i in range(max(len(v) for v in by_codec.values())):
        for c in sorted(by_codec, key=str):
            if i < len(by_codec[c]):
                order.append(by_codec[c][i])
    return [(layer, b, h) for h in range(wl.Hkv) for b in range(wl.B) for layer in order]


def cpu_baseline(wl, codecs, budget_s=12.0):
    """The oracle (as it stands) decoding a bounded sample of the step on the
    host: whole (layer, batch entry, kv head) units -- fp64 dequantisation of
    the unit's K and V (body codes, binary16 tail) and softmax attention of
    its query heads -- as many as fit the budget, on a thread pool of the
    GPU's share of host cores (BLAS pinned to one thread per worker).  The
    step time is scaled from the sampled units to all of the step's units."""
    import concurrent.futures

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle.layer as OL
    from oracle import attention

    host_cpus = len(os.sched_getaffinity(0))
    cores = min(16, host_cpus)          # one GPU's share of the machine's CPUs
    G = wl.Hq // wl.Hkv
    N, T = wl.N, wl.T
    units = _baseline_units(wl, codecs)
    specs = {}

    def prepare(u):
        layer, b, h = u
        if layer not in specs:
            specs[layer] = _oracle_specs(wl, layer, codecs[layer])
        ks, vs = specs[layer]
        xk = synth.head_rows(wl, layer, "k", b, h, T).numpy()
        xv = synth.head_rows(wl, layer, "v", b, h, T).numpy()
        ring = (OL.tail_ring(xk[None, :, None, :], N)[0, 0], OL.tail_ring(xv[None, :, None, :], N)[0, 0]) \
            if N else (None, None)
        q = synth.queries(wl, layer).numpy()[b, h * G:(h + 1) * G]
        return (u, OL.encode_head(xk, ks, h), OL.encode_head(xv, vs, h), ring, q)

    def decode_unit(prep):
        (layer, b, h), ke, ve, (kt, vt), q = prep
        ks, vs = specs[layer]
        with threadpool_limits(1):
            K = OL.dequant_head(ke, ks, h)[:T]
            V = OL.dequant_head(ve, vs, h)[:T]
            for t in range(max(0, T - N), T):
                K[t] = kt[t % N]
                V[t] = vt[t % N]
            return attention.attend(q, K[:, None, :], V[:, None, :], wl.sm_scale)

    # encode a pool of units once (setup), then time whole decode passes over
    # it until the budget is spent
    n_prep = min(len(units), cores)
    for u in units[:n_prep]:            # specs first, outside the threads
        if u[0] not in specs:
            specs[u[0]] = _oracle_specs(wl, u[0], codecs[u[0]])
    with concurrent.futures.ThreadPoolExecutor(cores) as ex:
        with threadpool_limits(1):
            pool = list(ex.map(prepare, units[:n_prep]))
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < budget_s or done == 0:
            list(ex.map(decode_unit, pool))
            done += len(pool)
        dt = time.perf_counter() - t0
    step_s = dt * len(units) / done
    nbytes = sum(layer_bytes(wl, c or wl.kcodec, c or wl.vcodec, T) for c in codecs)
    frac = "all" if n_prep == len(units) else "%d of the step's %d" % (n_prep, len(units))
    return {"value": nbytes / step_s / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%s (layer, batch entry, kv head) decode units (codec mix of the step), each "
                      "fp64 dequantisation of K and V over %d tokens + softmax attention of %d query "
                      "heads, decoded %d times in %.1f s wall on %d threads (the GPU's share of a "
                      "%d-CPU host); step time scaled to all units, bytes of the whole step"
                      % (frac, T, G, done, dt, cores, host_cpus),
            "host_cpus": host_cpus, "seconds_per_step": step_s}


def kernel_source_hash():
    """Hash of the library's sources (comments ignored), as compiled into it."""
    from quantized_kv_cache_kvq_amd.build import source_hash
    return source_hash()


def measured_traffic(workload):
    """HBM bytes per split-K attention launch from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    factor), or None when that summary is missing, covers another workload,
    or was taken on kernels whose sources have changed since."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_%s_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes, reps):
    """A plain device-to-device copy of nbytes, reps times: the reference
    kernel whose FETCH_SIZE / WRITE_SIZE calibrate the counter scale."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def prefill(args, dev):
    """Prefill-scale append and transcode (the survey's next-row workload):
    append the whole context of one layer in one call into an empty cache,
    and transcode a full binary16 layer to q8_0.  Reports each kernel's
    bytes moved (inputs read + packed rows, scales, mins and tail written;
    transcode: source read + destination written) per second against the
    8 TB/s HBM peak."""
    wl = synth.WORKLOADS[args.workload]
    kc, vc = (wl.kcodec, wl.vcodec) if wl.layers == 1 else ("q8_0", "q8_0")
    ks, vs = plane_specs(wl, 0, None if wl.layers == 1 else kc)
    capacity = math.ceil(wl.T / 64) * 64
    k = synth.layer_rows(wl, 0, "k", device=dev)
    v = synth.layer_rows(wl, 0, "v", device=dev)
    reps = 3
    caches = [LayerCache(wl.B, wl.Hkv, capacity, wl.N, ks, vs, dev) for _ in range(reps)]

    def plane_out(c):
        tot = 0
        for name in ("k", "v"):
            for key, t in c.bufs[name].items():
                if t is not None and not (key == "tail" and c.tail_len == 0):
                    tot += t.numel() * t.element_size()
        return tot

    out_bytes = plane_out(caches[0]) * wl.T / capacity
    in_bytes = 2 * k.numel() * 4
    stream = torch.cuda.current_stream(dev)
    for c in caches:
        c.n_tokens = 0
        c.append(k, v)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(3, args.steps // 20)
    e0.record(stream)
    for i in range(n):
        c = caches[i % reps]
        c.n_tokens = 0
        c.append(k, v)
    e1.record(stream)
    torch.cuda.synchronize()
    app_ms = e0.elapsed_time(e1) / n
    app_gbs = (in_bytes + out_bytes) / (app_ms * 1e-3) / 1e9
    del caches
    tr = None
    if wl.basis != "lowrank":
        tr = transcode_rate(wl, ks, vs, capacity, k, v, plane_out, n, dev, stream)
    line = {
        "metric": "prefill append and layer transcode GB/s (bytes read + written)",
        "append": {"value": round(app_gbs, 1), "unit": "GB/s", "ms": round(app_ms, 4),
                   "bytes": int(in_bytes + out_bytes), "frac_of_hbm_peak": round(app_gbs / HBM_PEAK_GBS, 4),
                   "tokens_per_s": round(wl.B * wl.T / (app_ms * 1e-3), 1)},
        "transcode_f16_to_q8_0": tr,
        "config": {"workload": wl.name, "batch": wl.B, "kv_heads": wl.Hkv, "context": wl.T,
                   "tail": wl.N, "k_codec": kc or "per-head", "v_codec": vc or "per-head",
                   "basis": wl.basis},
        "n_gpus": 1, "data": "synthetic (seeded), resident in HBM",
    }
    print(json.dumps(line), flush=True)


def transcode_rate(wl, ks, vs, capacity, k, v, plane_out, n, dev, stream):
    """Full binary16 layer re-encoded to q8_0 (the degrade step) n times."""
    src = LayerCache(wl.B, wl.Hkv, capacity, 0, PlaneSpec("f16", ks.basis, ks.w),
                     PlaneSpec("f16", vs.basis, vs.w), dev)
    src.append(k, v)
    dst = LayerCache(wl.B, wl.Hkv, capacity, 0, PlaneSpec("q8_0", ks.basis, ks.w),
                     PlaneSpec("q8_0", vs.basis, vs.w), dev)
    src.transcode_into(dst)
    torch.cuda.synchronize()
    tr_bytes = (plane_out(src) + plane_out(dst)) * wl.T / capacity
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        src.transcode_into(dst)
    e1.record(stream)
    torch.cuda.synchronize()
    tr_ms = e0.elapsed_time(e1) / n
    tr_gbs = tr_bytes / (tr_ms * 1e-3) / 1e9
    return {"value": round(tr_gbs, 1), "unit": "GB/s", "ms": round(tr_ms, 4), "bytes": int(tr_bytes),
            "frac_of_hbm_peak": round(tr_gbs / HBM_PEAK_GBS, 4)}


def quality(args, dev):
    """Quality sweep (codec x tail x plain/KVarN) on the rotated-3-bit
    workload's key and value statistics (Student-t keys with outlier
    channels, normal values) at one batch entry, 8 kv heads, 32 query heads
    and the given context; queries attend to a few recent and a few older
    tokens.  Prints one JSON line per configuration, then a summary line."""
    from quantized_kv_cache_kvq_amd import quality as Q
    wl = synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=1, Hq=32, T=args.quality_tokens)
    k = synth.layer_rows(wl, 0, "k", device=dev)
    v = synth.layer_rows(wl, 0, "v", device=dev)
    q_all = synth.peaked_queries(wl, k, args.quality_queries, device=dev)
    ent, ent_max = Q.entropy_nats(q_all, k, wl.sm_scale)
    print(json.dumps({"quality_setup": {"T": wl.T, "Hkv": wl.Hkv, "Hq": wl.Hq,
                                        "queries": args.quality_queries,
                                        "median_attention_entropy_nats": round(ent, 3),
                                        "uniform_entropy_nats": round(ent_max, 3)}}), flush=True)
    t0 = time.time()
    rows = Q.sweep(k, v, q_all, wl.sm_scale,
                   log=lambda r: print(json.dumps(r), flush=True))
    print(json.dumps({"quality_rows": len(rows), "seconds": round(time.time() - t0, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT, choices=synth.ORDER)
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP graph replays of the step instead of eager launches")
    ap.add_argument("--prefill", action="store_true",
                    help="measure prefill-scale append and layer transcode instead")
    ap.add_argument("--quality", action="store_true",
                    help="run the quality sweep (codec x tail x basis) instead")
    ap.add_argument("--quality-tokens", type=int, default=65536)
    ap.add_argument("--quality-queries", type=int, default=4)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe, max(1, args.steps))
        return
    lib.load()
    dev = torch.device("cuda:0")
    if args.prefill:
        prefill(args, dev)
        return
    if args.quality:
        quality(args, dev)
        return
    wl = synth.WORKLOADS[args.workload]
    if wl.name == "tiny":
        wl = wl.with_(T=256)
    codecs = synth.vbr_schedule(wl) if wl.layers > 1 else (wl.kcodec,)
    step_bytes = sum(layer_bytes(wl, c if wl.layers > 1 else wl.kcodec,
                                 c if wl.layers > 1 else wl.vcodec, wl.T) for c in codecs)
    replicas = args.replicas or max(1, math.ceil(2 * MALL_BYTES / max(step_bytes, 1)))
    replicas = min(replicas, 16)
    print("setting up %s: %d layer(s), %d replica(s), %.1f MB read per step"
          % (wl.name, len(codecs), replicas, step_bytes / 1e6), file=sys.stderr, flush=True)
    reps, news, qs, layer_codecs = setup(wl, dev, replicas)
    outs = [torch.empty_like(q) for q in qs]
    stream = torch.cuda.current_stream(dev)
    # Every layer's step is bound once, before any timing: arguments
    # marshalled, workspaces allocated and zeroed.  A step then costs the
    # host one library call per layer.
    bound = [[c.bind_step(news[li][0], news[li][1], qs[li], wl.sm_scale, outs[li], stream)
              for li, c in enumerate(layers)] for layers in reps]
    transcode_args = None
    if wl.layers > 1:
        import ctypes
        src = [i for i, c in enumerate(codecs) if c == "f16"][0]
        s0 = reps[0][src]
        dst = LayerCache(s0.batch, s0.n_kv_heads, s0.capacity, s0.tail_len, PlaneSpec("q8_0"),
                         PlaneSpec("q8_0"), dev, share_tail_with=s0, tail_format=s0.tail_format)
        dst.n_tokens = wl.T           # the source holds T tokens after the step's append
        st = ctypes.c_void_p(stream.cuda_stream)
        transcode_args = [(ctypes.byref(layers[src].desc), ctypes.byref(dst.desc), st) for layers in reps]
        transcode_fn = lib.load().kvq_transcode_layer
    t_prev = wl.T - 1

    def step(i):
        r = i % len(reps)
        for b in bound[r]:
            b.layer.desc.n_tokens = t_prev
            b()
        if transcode_args is not None:
            st = transcode_fn(*transcode_args[r])
            if st:
                lib.check(st)

    def step_unbound(i):
        # the same step through the per-call path, on torch's current stream
        # (graph capture switches it)
        layers = reps[i % len(reps)]
        for li, c in enumerate(layers):
            c.n_tokens = t_prev
            c.append_decode(news[li][0], news[li][1], qs[li], wl.sm_scale, out=outs[li])
        if transcode_args is not None:
            layers[src].transcode_into(dst)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # --graph: the step replayed as a HIP graph (one graph per cache
    # replica, captured after the warm-up), as a serving loop that captures
    # its step would run it.  The step's kernels allocate nothing and record
    # no memset, so a replay does exactly what the eager step does.
    graphs = None
    if args.graph:
        graphs = []
        for r in range(len(reps)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_unbound(r)
            graphs.append(g)
        for i in range(max(args.warmup, len(reps))):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is not None:
            graphs[i % len(graphs)].replay()
        else:
            step(i)

    # timed region: exactly K whole steps between two events, synchronised
    # on both sides
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        run_step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # outside the timed region: K more steps with an event after each (the
    # per-step median), then K eager steps with every split-K attention
    # launch stamped by HIP events of its own dispatch (hipExtLaunchKernel)
    # for the kernel's duration
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        run_step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    lib.timing_begin(args.steps * len(codecs))
    for i in range(args.steps):
        step(i)
    kern = lib.timing_durations(args.steps * len(codecs))
    lib.timing_end()

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ctx_tok_s = wl.B * wl.T * len(codecs) / (ms_per_step * 1e-3)
    roof = None
    if kern:
        # algorithmic bytes per launch: the packed cache one layer's decode
        # reads (codes, scales, mins, 16-bit tail), averaged over layers
        per_launch = step_bytes / len(codecs)
        avg_ms = sum(kern) / len(kern)
        ach = per_launch / (avg_ms * 1e-3) / 1e9
        ks = sorted(kern)
        traffic = measured_traffic(wl.name)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "traffic_source": ("rocprofv3 FETCH_SIZE/WRITE_SIZE summary committed under profiles/ "
                                   "for these kernel sources (not measured in this run)")
                if traffic is not None else None,
                "kernel": "split-K decode attention (kvq::decode_kernel / decode_lowrank_kernel)",
                "avg_launch_us": round(avg_ms * 1e3, 2),
                "median_launch_us": round(ks[len(ks) // 2] * 1e3, 2), "launches": len(kern),
                "algorithmic_bytes_per_launch": per_launch}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, layer_codecs if wl.layers > 1 else (None,))
        if cpu is not None:
            cpu.pop("seconds_per_step", None)
    line = {
        "metric": "decode-attention packed-KV GB/s and % of 8 TB/s HBM peak; context tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": arithmetic_label(wl),
        "data": "synthetic (seeded), resident in HBM; %d cache replicas rotated per step; %s"
                % (replicas, "eager launches" if graphs is None else "step replayed as a HIP graph"),
        "config": {"workload": wl.name, "batch": wl.B, "kv_heads": wl.Hkv, "q_heads": wl.Hq,
                   "context": wl.T, "tail": wl.N, "k_codec": wl.kcodec or "per-head",
                   "v_codec": wl.vcodec or "per-head", "basis": wl.basis, "layers": len(codecs),
                   "bytes_per_step": step_bytes},
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "context_tokens_per_s": round(ctx_tok_s, 1),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 5),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kld_context": kld_context(wl, codecs),
    }
    print(json.dumps(line), flush=True)


def arithmetic_label(wl):
    """What the decode computes in, for the line's dtype field."""
    if wl.basis == "lowrank":
        return ("i8 MFMA QK on 1-4 bit codes (query in 21-bit integer digits), f16 hi+lo MFMA PV, "
                "f32 accumulate; f32 MFMA query projection")
    if wl.layers > 1:
        return ("mixed per layer: i8 MFMA QK (21-bit query digits) + f16 hi+lo MFMA PV on q8_0/q4_0/"
                "q2_0 layers, f16 hi+lo MFMA QK and PV on f16 layers; f32 accumulate")
    tail = "; 16-bit tail: f16 hi+lo MFMA QK and PV" if wl.N else ""
    return ("i8 MFMA QK (query in 21-bit integer digits), f16 hi+lo MFMA PV (22-bit weights), "
            "f32 accumulate" + tail)


def kld_context(wl, codecs):
    """The pages' median-KLD row(s) for this workload's codecs (another model
    and another machine: context only, not compared)."""
    path = os.path.join(ROOT, "tests", "golden", "kld_table.json")
    if not os.path.exists(path):
        return None
    tab = json.load(open(path))
    names = set()
    for c in (codecs if wl.layers > 1 else (wl.kcodec, wl.vcodec)):
        if c and c != "f16":
            names.add(("kvarn" + c[1]) if wl.basis == "hadamard" else c)
    rows = {n: dict(zip(["tail_%d" % t for t in tab["tails"]], tab["median_kld"][n]))
            for n in sorted(names) if n in tab["median_kld"]}
    if not rows:
        return None
    return {"source": "BeeLlama.cpp v0.4.0 release notes, Qwen 3.6 27B Q5_K_S 64k-context KLD table "
                      "(median KLD against an unquantised cache); another model and machine, context only",
            "median_kld": rows}


if __name__ == "__main__":
    main()
