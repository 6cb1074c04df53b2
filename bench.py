"""Benchmark of the fused MoE expert-FFN forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME[:T1/T2],...]
                    [--tokens 8,64,256] [--no-cpu-baseline]

A step is one whole forward on one batch: the planner (moe_align) and the
fused expert FFN (gather, gate/up GEMM, SwiGLU + requantization, down GEMM,
top-k weighted combine), inputs resident in HBM, on synthetic seeded data of
the workload's shapes (random-init weights; no trained checkpoint exists
here).  By default two workloads run: blockwise FP8 K=4096, I=2048, E=256,
top-6 at T = 8, 64 and 256 (the weight-stream-bound decode sizes), then
blockwise FP8 K=4096, I=2048, E=288, top-8 at T = 8192, the largest
single-GPU configuration, whose throughput, configuration and roofline make
the JSON line's headline (``value``, ``config``, ``roofline``); ``sweep``
lists every point.

Throughput: algorithmic FLOPs 6 * R * K * I per step (R = routes to local
experts; padding rows do not count) over the step time.  Roofline, per point
and for the headline: the dominant kernel (the gate/up kernel in split mode,
``k_up`` streaming or ``k_up_t`` LDS-tiled; the fused kernel in fused mode;
the persistent kernel in ring mode) is timed with HIP events recorded around
it on its own stream; its algorithmic FLOPs (4 * R * K * I for the gate/up
GEMM) and HBM bytes (weights and scales of the experts it reads once, the
token rows, its outputs) give its binding roof max(F / MFMA peak, B / HBM
peak), and t_roof / t_measured is the fraction of that roof reached.  The
whole step gets the same figure from its own FLOPs and bytes.

Per token count the sweep also holds per-call distributions (median, p10,
p90 of event pairs around each call): the whole call and the forward alone
(planner outputs reused), back to back ("warm"), and the whole call with a
1 GiB read before each call outside its events ("cold": L2 and the 256 MB
MALL hold other, clean lines), and the whole call captured once in a HIP
graph and replayed ("graph_warm": launch gaps gone, as in a decode loop).  The line records the GPU clocks (from sysfs) and two
measured reference ceilings beside the spec peaks: a plain device copy, a
read-only sum, and a large e4m3 GEMM through the vendor BLAS.

The CPU baseline runs the fp64 oracle on a bounded sample of the headline
workload (a few tokens of its batch) on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense MFMA peaks; an e4m3 x e2m1 product issues at the e4m3 rate
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8_blockwise": 5000.0, "mxfp8": 5000.0, "mxfp4": 5000.0}
DTYPE_NAME = {"bf16": "bf16", "fp8_blockwise": "e4m3/fp32-blockwise", "mxfp8": "e4m3/e8m0-mx",
              "mxfp4": "e2m1/e8m0-mx weights x e4m3/e8m0-mx activations"}
METRIC = ("fused MoE fwd µs and TFLOP/s (% FP8 MFMA / % HBM roofline) vs tokens T")
CSRC = "mixture_experts_ffn_moe_amd/csrc"
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(os.path.join(ROOT, CSRC))
                        if f.endswith((".hip", ".h")))


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its stream)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def kernel_source_hash():
    """Hash of the kernel sources' code: comments removed and whitespace
    collapsed, so that an edit of a comment keeps the counters current."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            t = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()[:16]


def byte_model(kind, K, I, E_act, T, R, split):
    """Algorithmic HBM bytes: (step total, dominant kernel)."""
    N = 2 * I
    es = 2 if kind == "bf16" else 1
    if kind == "bf16":
        w1e, w2e = N * K * 2, K * I * 2
    elif kind == "mxfp4":
        w1e = N * K // 2 + N * (K // 32)
        w2e = K * I // 2 + K * (I // 32)
    elif kind == "fp8_blockwise":
        w1e = N * K + (N // 128) * (K // 128) * 4
        w2e = K * I + (K // 128) * (I // 128) * 4
    else:
        w1e = N * K + N * (K // 32)
        w2e = K * I + K * (I // 32)
    xs = 0 if kind == "bf16" else (T * (K // 128) * 4 if kind == "fp8_blockwise" else T * (K // 32))
    x_b = T * K * es + xs
    out_b = T * K * 2
    route_b = R * 8
    step = E_act * (w1e + w2e) + x_b + out_b + route_b
    hs = 0 if kind == "bf16" else (R * (I // 128) * 4 if kind == "fp8_blockwise" else R * (I // 32))
    if split == 2:
        # persistent ring kernel: both GEMMs, H written and read back, bf16 route rows
        dom = E_act * (w1e + w2e) + x_b + 2 * (R * I * es + hs) + R * K * 2
    elif split:
        dom = E_act * w1e + x_b + R * I * es + hs          # gate/up kernel: w1, x, H write
    else:
        dom = E_act * (w1e + w2e) + x_b + 2 * T * K * 4    # fused: weights, x, fp32 acc r/w
    return step, dom


def load_traffic(workload, T, kernel_name):
    """HBM traffic per launch from a committed rocprofv3 counter summary, or
    None when absent or taken on another revision of the kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    e = d.get("entries", {}).get(f"{workload}/T={T}/{kernel_name}")
    return None if e is None else e.get("bytes_per_launch")


# Counter runs of the traffic measurement: (directory tag, workload, tokens,
# kernels).  Each run is a short bench.py of that workload and token count
# under `rocprofv3 --pmc FETCH_SIZE` and, separately, `--pmc WRITE_SIZE`; the
# fused-mode run forces the fused mode.
COUNTER_RUNS = [
    ("up", "fp8-k4096-i2048-e256-top6", 256, ("k_up", "k_down")),
    ("fused", "fp8-k4096-i2048-e256-top6", 8, ("k_fused",)),
    ("up4", "mxfp4-k4096-i2048-e256-top6", 256, ("k_up", "k_down")),
    ("tiled", "fp8-k4096-i2048-e288-top8", 8192, ("k_up_t", "k_down_t")),
]


def summarize_counters(root):
    """Turn the rocprofv3 counter runs of the traffic measurement into
    profiles/hbm_traffic.json.  `root` holds one directory per run, named
    pmc_{copy,<tag>}_{FETCH_SIZE,WRITE_SIZE} for the tags of COUNTER_RUNS (see
    the command lists in profiles/hbm_traffic_*.md), each with the profiler's
    *_counter_collection.csv."""
    import csv
    import glob

    def values(run, counter, kernel_sub=None):
        out = []
        for f in glob.glob(os.path.join(root, f"pmc_{run}_{counter}", "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                if kernel_sub and kernel_sub not in r["Kernel_Name"]:
                    continue
                out.append(float(r["Counter_Value"]))
        if not out:
            raise SystemExit(f"no {counter} values for {run} {kernel_sub or ''} under {root}")
        return out

    # the copy kernel moves exactly n bytes each way per launch; the largest
    # dispatches are the copies (torch's fill of the source is a write only)
    n = 1024 << 20
    fetch_copy = max(values("copy", "FETCH_SIZE"))
    write_copy = max(values("copy", "WRITE_SIZE"))
    fetch_factor = n / (fetch_copy * 1024)
    write_factor = n / (write_copy * 1024)
    entries = {}
    for tag, workload, T, kernels in COUNTER_RUNS:
        for kname in kernels:
            sub = f"::{kname}<"
            fk = values(tag, "FETCH_SIZE", sub)
            wk = values(tag, "WRITE_SIZE", sub)
            f_raw, w_raw = sum(fk) / len(fk), sum(wk) / len(wk)
            fb, wb = f_raw * 1024 * fetch_factor, w_raw * 1024 * write_factor
            entries[f"{workload}/T={T}/{kname}"] = {
                "fetch_kib_raw": f_raw, "write_kib_raw": w_raw, "fetch_bytes": fb,
                "write_bytes": wb, "bytes_per_launch": fb + wb, "dispatches": len(fk)}
    d = {"kernel_source_hash": kernel_source_hash(),
         "calibration": {"copy_bytes_read": n, "copy_bytes_written": n,
                         "fetch_kib_per_copy": fetch_copy, "write_kib_per_copy": write_copy,
                         "fetch_factor": fetch_factor, "write_factor": write_factor},
         "entries": entries}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d, indent=1))


def cpu_baseline(case, n_tokens, K, I):
    import numpy as np

    import datagen
    from oracle.moe import moe_ref
    tokens = np.arange(min(n_tokens, case.T))
    ids = case.topk_ids.cpu().numpy()[tokens]
    experts = sorted(set(int(e) for e in np.unique(ids) if 0 <= e < case.E))
    d = datagen.to_numpy(case, experts=experts)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    moe_ref(d["kind"], d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"],
            d["topk_ids"], d["topk_weights"], tokens=tokens)
    dt = time.perf_counter() - t0
    R = int(((ids >= 0) & (ids < case.E)).sum())
    flops = 6.0 * R * K * I
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{len(tokens)} tokens ({R} routes, {len(experts)} experts dequantized) of "
                       f"the T={case.T} batch; fp64 numpy oracle, {dt:.2f} s"),
            "seconds": dt}


def shared_leg(torch, moe, datagen, case, shared_w, calls, stream):
    """One shared expert at this token count: one call that runs it with the
    routed experts (planner + forward, split mode) against the routed call
    followed by the shared expert as a call of its own (every token routed to
    it with weight 1) and an add of the two outputs (median of per-call event
    pairs, back to back)."""
    import dataclasses
    sw, cat = shared_w
    T, E, k = case.T, case.E, case.top_k
    both = dataclasses.replace(case, w1=cat[0], w1_scale=cat[1], w2=cat[2], w2_scale=cat[3],
                               n_shared=1)
    alone = dataclasses.replace(case, w1=sw[0], w1_scale=sw[1], w2=sw[2], w2_scale=sw[3], E=1,
                                top_k=1, topk_ids=torch.zeros_like(case.topk_ids[:, :1]),
                                topk_weights=torch.ones_like(case.topk_weights[:, :1]))
    bm_both = moe.moe_select_block_m(T, k + 1, E + 1, case.kind, case.K)
    bm_r = moe.moe_select_block_m(T, k, E, case.kind, case.K)
    bm_s = moe.moe_select_block_m(T, 1, 1, case.kind, case.K)
    out = torch.empty(T, case.K, dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out)
    ws = {}

    def run(c, bm, o):
        key = id(c)
        if key not in ws:
            need = moe.moe_workspace_size(c.kind, T, c.K, 2 * c.I, c.E + c.n_shared,
                                          c.top_k + c.n_shared, bm, 1)
            ws[key] = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        moe.run_case(c, block_m=bm, split=1, workspace=ws[key], out=o)

    def fused():
        run(both, bm_both, out)

    def separate():
        run(case, bm_r, out)
        run(alone, bm_s, out2)
        out.add_(out2)

    res = {}
    for name, fn in (("routed_and_shared_one_call", fused),
                     ("routed_then_shared_then_add", separate)):
        fn()
        res[name] = per_call(torch, fn, calls, stream)["median_us"]
    return res


def router_leg(torch, moe, datagen, spec, workload, T, bm, calls, stream):
    """The router step to the left of the planner at this token count, on the
    workload's router logits: the fused router + planner launch against
    torch's softmax / topk / renormalization followed by the planner launch,
    and the planner alone (median of per-call event pairs, back to back)."""
    E, k = spec["E"], spec["top_k"]
    kw = {key: spec[key] for key in ("n_masked", "zipf_s") if key in spec}
    logits = datagen.make_router_logits(T, E, k, spec["routing"], device="cuda",
                                        tag=workload, **kw)
    ids, w, sid, eid, ntp = moe.moe_route_align(logits, k, bm)
    outs = (ids, w, sid, eid, ntp)

    def fused():
        moe.moe_route_align(logits, k, bm, out=outs)

    def separate():
        p = torch.softmax(logits, dim=1)
        tw, ti = torch.topk(p, k, dim=1)
        tw = tw / tw.sum(dim=1, keepdim=True)
        moe.moe_align(ti.to(torch.int32), E, bm, out=(sid, eid, ntp))

    def planner():
        moe.moe_align(ids, E, bm, out=(sid, eid, ntp))

    res = {}
    for name, fn in (("route_align_fused", fused), ("torch_router_then_planner", separate),
                     ("planner_alone", planner)):
        fn()
        res[name] = per_call(torch, fn, calls, stream)["median_us"]
    return res


def percentiles(v):
    v = sorted(v)
    def at(q):
        x = q / 100.0 * (len(v) - 1)
        i = int(x)
        return v[i] if i + 1 >= len(v) else v[i] + (x - i) * (v[i + 1] - v[i])
    return {"n": len(v), "median_us": at(50), "p10_us": at(10), "p90_us": at(90),
            "mean_us": sum(v) / len(v)}


def per_call(torch, fn, n, stream, flush=None):
    """Event pair around each of n calls on ``stream`` (the flush, when given,
    runs before each call, outside its pair)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return percentiles([a.elapsed_time(b) * 1e3 for a, b in evs])


def graph_leg(torch, step, calls, stream):
    """The whole call (planner + forward) captured once in a HIP graph
    (torch.cuda.CUDAGraph over the same C ABI calls, which allocate nothing
    and never synchronize) and replayed: per-replay event pairs.  What a
    decode loop that replays a captured step pays per call."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    res = per_call(torch, g.replay, calls, stream)
    del g
    return res


def gpu_clocks():
    """Current shader and memory clocks from the amdgpu sysfs DPM tables (the
    level marked with '*'); None where the files are absent.  Read directly:
    this process has initialised the GPU, and starting rocm-smi would exec."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        res = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [ln.split(":", 1)[1].strip(" *\n") for ln in f if ln.rstrip().endswith("*")]
            except (OSError, IndexError):
                continue
            if cur:
                res[name[7:]] = cur[0]
        if res:
            return res
    return None


def measured_ceilings(torch):
    """Reference ceilings measured on this GPU beside the spec peaks: a plain
    device copy (bytes read + written per second), a read-only sum, and a
    large e4m3 GEMM through torch._scaled_mm (the vendor BLAS), each the best
    of 6."""
    res = {}
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        best = t if best is None else min(best, t)
    res["copy_gbs"] = 2 * n / (best * 1e-3) / 1e9
    del dst
    f = src.view(torch.float32)
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.sum(f, dim=0, out=sink)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        best = t if best is None else min(best, t)
    res["read_gbs"] = n / (best * 1e-3) / 1e9
    del src, f, sink
    try:
        m = 8192
        x = torch.randn(m, m, device="cuda").to(torch.float8_e4m3fn)
        w = torch.randn(m, m, device="cuda").to(torch.float8_e4m3fn).t()
        one = torch.ones((), device="cuda")
        best = None
        for _ in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch._scaled_mm(x, w, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        res["fp8_gemm_tflops"] = 2.0 * m ** 3 / (best * 1e-3) / 1e12
        res["fp8_gemm_shape"] = [m, m, m]
    except Exception as exc:  # the vendor GEMM is a reference only
        res["fp8_gemm_tflops"] = None
        res["fp8_gemm_error"] = str(exc)[:200]
    return res


DEFAULT_WORKLOADS = "fp8-k4096-i2048-e256-top6,fp8-k4096-i2048-e288-top8:8192"


def parse_workloads(arg, tokens):
    """'name[:T1/T2..],..' -> [(name, [T..])]; --tokens overrides every list."""
    import datagen
    out = []
    for part in arg.split(","):
        name, _, ts = part.partition(":")
        if tokens:
            ts_list = [int(t) for t in tokens.split(",")]
        elif ts:
            ts_list = [int(t) for t in ts.split("/")]
        else:
            ts_list = list(datagen.WORKLOADS[name]["tokens"])
        out.append((name, ts_list))
    return out


def dominant(kind, bm, split, K, I):
    """Name and kind of the kernel that streams the gate/up weights."""
    if split == 0:
        return "k_fused"
    if split == 2:
        return "k_ring"
    tiled = kind in ("fp8_blockwise", "mxfp8") and bm >= 64 and K % 256 == 0 and I % 128 == 0
    return "k_up_t" if tiled else "k_up"


def roof(flops, nbytes, us, kind):
    """Binding roof of a kernel or step: (bound, t_roof us, frac = t_roof / t)."""
    t_mfma = flops / (MFMA_PEAK_TFLOPS[kind] * 1e12) * 1e6
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    bound = "mfma" if t_mfma > t_hbm else "hbm"
    t = max(t_mfma, t_hbm)
    return bound, t, t / us


def run_workload(args, torch, moe, datagen, name, tokens, dev, stream):
    spec = datagen.WORKLOADS[name]
    kind, K, I, E, k = spec["kind"], spec["K"], spec["I"], spec["E"], spec["top_k"]
    N = 2 * I
    print(f"[bench] generating {name} weights on the GPU", file=sys.stderr, flush=True)
    weights = datagen.make_weights(kind, K, I, E, device=dev, tag=name, w_std=spec.get("w_std"))
    torch.cuda.synchronize()
    # one shared expert of the same format, stored after the routed ones
    shared_w = None
    if args.calls:
        sw = datagen.make_weights(kind, K, I, 1, device=dev, tag=name + "/shared",
                                  w_std=spec.get("w_std"))
        shared_w = (sw, [None if a is None else torch.cat([a, b]) for a, b in zip(weights, sw)])
        torch.cuda.synchronize()
    sweep = []
    case = None
    for T in tokens:
        case = datagen.make_workload_case(name, T, device=dev, weights=weights)
        ids = case.topk_ids
        valid = (ids >= 0) & (ids < E)
        R = int(valid.sum().item())
        E_act = int(torch.unique(ids[valid]).numel())
        # block size from the routing at hand: routes per active expert
        bm = args.block_m or moe.moe_select_block_m_routed(T, k, E, E_act, kind, K)
        split = args.split if args.split >= 0 else moe.moe_select_split(kind, T, K, N, E, k, bm)
        rows, blocks = moe.moe_align_capacity(T, k, E, bm)
        align_out = (torch.empty(rows, dtype=torch.int32, device=dev),
                     torch.empty(blocks, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
        ws = torch.empty(max(moe.moe_workspace_size(kind, T, K, N, E, k, bm, split), 256),
                         dtype=torch.uint8, device=dev)
        out = torch.empty(T, K, dtype=torch.bfloat16, device=dev)

        def step():
            moe.run_case(case, block_m=bm, split=split, workspace=ws, out=out, align_out=align_out)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        hev = HipEvents(2 * args.steps)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            moe.moe_set_timing_events(hev.ev[2 * i], hev.ev[2 * i + 1], 1)
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        moe.moe_set_timing_events(None, None)
        ms = t0.elapsed_time(t1) / args.steps
        kms = sum(hev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)) / args.steps
        hev.close()
        flops = 6.0 * R * K * I
        step_bytes, dom_bytes = byte_model(kind, K, I, E_act, T, R, split)
        kname = dominant(kind, bm, split, K, I)
        dom_flops = flops if split != 1 else 4.0 * R * K * I    # gate/up GEMM alone
        mode = {0: "fused", 1: "split", 2: "ring"}[split]
        s_bound, s_troof, s_frac = roof(flops, step_bytes, ms * 1e3, kind)
        d_bound, d_troof, d_frac = roof(dom_flops, dom_bytes, kms * 1e3, kind)
        sweep.append({
            "workload": name, "T": T, "routes": R, "active_experts": E_act, "block_m": bm,
            "mode": mode,
            "us_per_step": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12,
            "pct_mfma_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[kind],
            "step_gbs": step_bytes / (ms * 1e-3) / 1e9,
            "pct_hbm_peak": 100.0 * step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "step_roof": {"bound": s_bound, "t_roof_us": s_troof, "t_roof_over_t": s_frac},
            "dominant_kernel": kname, "dominant_us": kms * 1e3,
            "dominant_bytes": dom_bytes, "dominant_flops": dom_flops,
            "dominant_gbs": dom_bytes / (kms * 1e-3) / 1e9,
            "dominant_tflops": dom_flops / (kms * 1e-3) / 1e12,
            "dominant_roof": {"bound": d_bound, "t_roof_us": d_troof, "t_roof_over_t": d_frac},
        })
        print(f"[bench] {name} T={T} bm={bm} {mode}: {ms*1e3:.1f} us/step "
              f"({100 * s_frac:.0f}% of its {s_bound} roof), {kname} {kms*1e3:.1f} us "
              f"({100 * d_frac:.0f}% of its {d_bound} roof)", file=sys.stderr, flush=True)
        # per-call distributions: the whole call (planner + forward) and the
        # forward alone, warm (back to back), then cold (a 1 GiB read before
        # each call, outside its event pair: evicts L2 and the 256 MB MALL)
        prot = {}

        def op_only():
            moe.run_case(case, block_m=bm, split=split, workspace=ws, out=out,
                         align_out=align_out, skip_align=True)

        if args.calls:
            prot["full_warm"] = per_call(torch, step, args.calls, stream)
            prot["op_warm"] = per_call(torch, op_only, args.calls, stream)
            prot["graph_warm"] = graph_leg(torch, step, args.calls, stream)
        if args.cold_calls:
            # a read, not a write: written scratch would leave the caches
            # dirty, and the call would pay for writing it back
            scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
            sink = torch.empty((), dtype=torch.float32, device=dev)
            prot["full_cold"] = per_call(torch, step, args.cold_calls, stream,
                                         flush=lambda: torch.sum(scratch, dim=0, out=sink))
            del scratch, sink
        sweep[-1]["per_call"] = prot
        if args.calls:
            sweep[-1]["router"] = router_leg(torch, moe, datagen, spec, name, T, bm,
                                             args.calls, stream)
            sweep[-1]["shared"] = shared_leg(torch, moe, datagen, case, shared_w, args.calls,
                                             stream)
        del ws
    del weights, shared_w
    return sweep, case


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOADS,
                    help="comma list of name[:T1/T2..]; the last token count of the last "
                         "workload is the headline")
    ap.add_argument("--tokens", default=None, help="comma list for every workload")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--split", type=int, default=-1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=24)
    ap.add_argument("--calls", type=int, default=200,
                    help="per-call timed calls (warm) for the median / p10 / p90")
    ap.add_argument("--cold-calls", type=int, default=50,
                    help="per-call timed calls with a 1 GiB read before each (cold caches)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR",
                    help="only write profiles/hbm_traffic.json from the counter runs under DIR")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the fused MoE forward here runs on one GPU's local "
              "experts with no collectives; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        # a plain copy of known size: each launch reads and writes exactly
        # MIB MiB, which calibrates the HBM byte counters of a profiler
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return

    import datagen
    import mixture_experts_ffn_moe_amd as moe

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    moe.lib()
    stream = torch.cuda.current_stream()
    sweep = []
    last_case = None
    for name, tokens in parse_workloads(args.workload, args.tokens):
        part, last_case = run_workload(args, torch, moe, datagen, name, tokens, dev, stream)
        sweep += part
        torch.cuda.empty_cache()

    head = sweep[-1]
    spec = datagen.WORKLOADS[head["workload"]]
    kind, K, I, E, k = spec["kind"], spec["K"], spec["I"], spec["E"], spec["top_k"]
    dr = head["dominant_roof"]
    if dr["bound"] == "hbm":
        achieved, peak, unit = head["dominant_gbs"], HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = head["dominant_tflops"], MFMA_PEAK_TFLOPS[kind], "TFLOP/s"
    roof_line = {"bound": dr["bound"], "achieved": achieved, "peak": peak, "unit": unit,
                 "frac": achieved / peak,
                 "traffic": load_traffic(head["workload"], head["T"], head["dominant_kernel"]),
                 "kernel": head["dominant_kernel"], "bytes_per_launch": head["dominant_bytes"],
                 "flops_per_launch": head["dominant_flops"], "us_per_launch": head["dominant_us"],
                 "t_roof_us": dr["t_roof_us"],
                 "mfma_frac": head["dominant_tflops"] / MFMA_PEAK_TFLOPS[kind],
                 "hbm_frac": head["dominant_gbs"] / HBM_PEAK_GBS}
    result = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["us_per_step"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[kind], "data": "synthetic (seeded random weights, tokens, routing)",
        "config": {"workload": head["workload"], "tokens": head["T"], "hidden": K,
                   "intermediate": I, "experts": E, "top_k": k, "block_m": head["block_m"],
                   "mode": head["mode"], "parallelism": "single GPU, all experts local"},
        "roofline": roof_line,
        "step_roofline": head["step_roof"],
        "sweep": sweep,
        "kernel_source_hash": kernel_source_hash(),
    }
    result["clocks"] = gpu_clocks()
    result["measured_ceilings"] = measured_ceilings(torch)
    result["spec_peaks"] = {"hbm_gbs": HBM_PEAK_GBS, "mfma_tflops": MFMA_PEAK_TFLOPS[kind]}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(last_case, args.cpu_tokens, K, I)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
