"""Benchmark of the fused EXL3 routed-experts layer on one MI355X.

A step is one full layer forward (route pack, rotations, gate/up GEMM +
SwiGLU, down GEMM, ordered combine) over one batch of synthetic input that is
already resident in HBM. The headline workload is the mixed-width prefill
layer (192 experts, top-8, hidden 6144, intermediate 2048, K per expert in
{3,4,5,6,8}, 3072 rows, Zipf(1.2) routing, capacity 2048 pairs). The decode
layer (128 experts, top-8, hidden 4096, intermediate 1536, K=4) at 1, 8 and 32
rows is reported alongside, timed by hipGraph replay over rotating routings,
and so are the additive layer (256 experts, base K=3 plus a K=2 residual
stage, 128 rows) and the plain 4096 -> 4096 linear at K = 2, 3, 4, 8 and 1,
32, 2048 rows, both with cold weights.

Prints one JSON line. ``--gpus N`` with N > 1 is refused: this build runs on
one GPU.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer µs and tokens/sec at M=1/32/3072; % HBM peak (decode), "
          "% MFMA (prefill)")
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _kernel_stats(records):
    st = {}
    for name, ms in records:
        s = st.setdefault(name, [0, 0.0])
        s[0] += 1
        s[1] += ms
    return {k: {"launches": n, "total_ms": t, "avg_us": 1000.0 * t / n}
            for k, (n, t) in st.items()}


def check_status(ws, dropped, what):
    """The library's status words of the last call on this workspace (ctrl[0]
    pairs left out, ctrl[1] skipped stage entries, ctrl[2] device waits that
    gave up) must read (dropped, 0, 0): otherwise the timed result is not a
    valid layer output."""
    import torch
    torch.cuda.synchronize()
    c = [int(v) for v in ws[:12].view(torch.int32).cpu()]
    if c != [dropped, 0, 0]:
        raise RuntimeError("%s: status words %s, expected [%d, 0, 0]" % (what, c, dropped))


def prefill_step_flops(wl):
    """Algorithmic flops of one layer: 2 per multiply-add of every kept pair
    through gate and up (H x 2I) and down (I x H). With 128-row tiles the two
    run in one launch per pass (gemm_experts)."""
    P = int(np.sum((wl.ids >= 0) & (wl.ids < wl.num_experts)))
    H, I = wl.hidden, wl.intermediate
    gu, dn = 2.0 * P * H * 2 * I, 2.0 * P * I * H
    return {"gemm_gateup": gu, "gemm_down": dn, "gemm_experts": gu + dn}


def run_prefill(args, torch, exl3, synth, **over):
    _log("prefill %s: drawing inputs" % (over or ""))
    t0 = time.time()
    wl = synth.moe_workload("prefill", materialize=False, **over)
    gate, up, down = (exl3.DeviceProj(p, "cuda", words_fn=synth.realize_words)
                      for p in (wl.gate, wl.up, wl.down))
    x, ids, w = exl3.device_inputs(wl, "cuda")
    out = torch.empty(wl.rows, wl.hidden, dtype=torch.float16, device="cuda")
    need = exl3.moe_workspace_size(wl.rows, wl.topk, wl.num_experts, wl.hidden,
                                   wl.intermediate, wl.capacity)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    _log("prefill: inputs resident in %.1f s (trellis %.2f GB)" % (
        time.time() - t0, sum(p.buffer.numel() for p in (gate, up, down)) / 1e9))

    def step():
        exl3.exl3_moe_forward(x, ids, w, gate, up, down, wl.capacity, out=out, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _log("prefill: warmup done")
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    # per-kernel durations measured live over the timed steps (events on the
    # stream the library launches on)
    with exl3.Profile(max_launches=64 * args.steps) as prof:
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(args.steps):
            step()
        t_stop.record()
        torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_stop) / args.steps
    check_status(ws, int(np.sum((wl.ids < 0) | (wl.ids >= wl.num_experts))), "prefill")
    _log("prefill: %.1f us per layer" % (1000 * ms))
    kstats = _kernel_stats(prof.records)
    flops = prefill_step_flops(wl)
    dom = max((k for k in ("gemm_experts", "gemm_gateup", "gemm_down") if k in kstats),
              key=lambda k: kstats[k]["total_ms"])
    per_launch_flops = flops[dom] / (kstats[dom]["launches"] / args.steps)
    achieved = per_launch_flops / (kstats[dom]["avg_us"] * 1e-6) / 1e12
    layer_tflops = flops["gemm_experts"] / (ms * 1e-3) / 1e12
    res = {
        "ms": ms, "tokens_per_s": wl.rows / (ms * 1e-3), "kernels": kstats,
        "dominant": dom, "per_launch_flops": per_launch_flops,
        "achieved_tflops": achieved, "layer_tflops": layer_tflops,
        "layer_mfma_frac": layer_tflops / MFMA_F16_PEAK_TFLOPS,
        "passes": exl3.moe_layout(wl.rows, wl.topk, wl.num_experts, wl.hidden,
                                  wl.intermediate, wl.capacity).passes,
    }
    return wl, res


def run_decode(args, torch, exl3, synth, M, groups=16, **over):
    """The decode layer (128 experts, top-8, hidden 4096, intermediate 1536,
    K=4) at M rows. `groups` routings are drawn; one captured graph holds one
    layer call per routing, so a replay streams the experts of 16 different
    routings (together about all 1.2 GB of weights, far more than the 256 MB
    MALL) and the host's cost per graph replay is spread over 16 layers.
    Layer time = replay time / 16. Per-kernel durations come from eager calls
    over the same routings (HIP events around each launch)."""
    wl = synth.moe_workload("decode", rows=M, **over)
    gate, up, down = (exl3.DeviceProj(p, "cuda") for p in (wl.gate, wl.up, wl.down))
    x, _, _ = exl3.device_inputs(wl, "cuda")
    routings = []
    for gi in range(groups):
        ids, wb = synth.routes("uniform", 1000 + gi, M, wl.num_experts, wl.topk, "bf16")
        it = torch.from_numpy(ids.astype(np.int64)).cuda()
        wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).cuda()
        routings.append((ids, it, wt))
    out = torch.empty(M, wl.hidden, dtype=torch.float16, device="cuda")
    need = exl3.moe_workspace_size(M, wl.topk, wl.num_experts, wl.hidden, wl.intermediate,
                                   M * wl.topk)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call(r):
        exl3.exl3_moe_forward(x, r[1], r[2], gate, up, down, M * wl.topk, out=out, ws=ws)

    for r in routings:
        call(r)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        for r in routings:
            call(r)
    torch.cuda.synchronize()
    reps = max(4, args.steps)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * groups)
    check_status(ws, 0, "decode M=%d" % M)
    # per-kernel durations from eager launches over the same routings
    with exl3.Profile(max_launches=16 * groups * 4) as prof:
        for _ in range(4):
            for r in routings:
                call(r)
        torch.cuda.synchronize()
    kst = _kernel_stats(prof.records)
    # algorithmic HBM bytes: the trellis of every active expert's gate, up and
    # down projection (each read once), the input rows, the rotated inputs
    # x~ (written and read), a~ (written and read), d (written and read) and
    # the output
    per_tensor = wl.hidden * wl.intermediate * 4 // 8
    act = [len(np.unique(r[0])) for r in routings]
    P = M * wl.topk
    trellis = np.mean([3 * per_tensor * n for n in act])
    acts = (M * wl.hidden * 2 + P * (2 * wl.hidden * 2) * 2 + P * wl.intermediate * 2 * 2
            + P * wl.hidden * 4 * 2 + M * wl.hidden * 2)
    layer_bytes = trellis + acts
    res = {
        "rows": M, "us": 1000 * ms, "tokens_per_s": M / (ms * 1e-3),
        "graph": "%d layer calls per replay, %d replays" % (groups, reps),
        "kernels": kst, "algorithmic_bytes": layer_bytes, "trellis_bytes": trellis,
        "layer_GBps": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    if "gemm_experts" in kst:
        res["gemm_experts_GBps"] = trellis / (kst["gemm_experts"]["avg_us"] * 1e-6) / 1e9
    return res


def run_linear(args, torch, exl3, synth, Ks=(2, 3, 4, 8), Ms=(1, 32, 2048), reps=48):
    """The plain linear 4096 -> 4096 (exl3_linear: rotation + GEMM launch) at
    each width K and row count M, weights cold: calls rotate over enough
    copies of the trellis (>= 600 MB) that none is cache-resident. Bytes are
    the trellis plus fp16 rows in and out; flops 2 x M x in x out."""
    res = {}
    for K in Ks:
        p, x = synth.linear_workload(K, max(Ms))
        tbytes = p.in_features * p.out_features * K // 8
        ncopy = max(2, -(-600_000_000 // tbytes))
        copies = [exl3.DeviceProj(p, "cuda") for _ in range(ncopy)]
        xd = exl3.f16_tensor(x)
        for M in Ms:
            out = torch.empty(M, p.out_features, dtype=torch.float16, device="cuda")
            ws = torch.empty(max(256, exl3.linear_workspace_size(M, p.in_features,
                                                                 p.out_features)),
                             dtype=torch.uint8, device="cuda")
            for c in copies[:4]:
                exl3.exl3_linear(xd[:M], c, out=out, ws=ws)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(reps):
                exl3.exl3_linear(xd[:M], copies[i % ncopy], out=out, ws=ws)
            b.record()
            torch.cuda.synchronize()
            us = 1000.0 * a.elapsed_time(b) / reps
            nbytes = tbytes + M * (p.in_features + p.out_features) * 2
            flops = 2.0 * M * p.in_features * p.out_features
            res["K%d_M%d" % (K, M)] = {
                "us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
                "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                "tflops": flops / (us * 1e-6) / 1e12,
                "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS}
        del copies
        torch.cuda.empty_cache()
    return res


def run_additive(args, torch, exl3, synth, reps=20):
    """The additive layer (256 experts, top-8, 4096/2048, 128 rows, base K=3
    plus one K=2 residual stage per projection, 30% of the residual scales
    zero): exl3_moe_additive on a route pack made once. Its trellis (over
    3 GB) exceeds every cache. Bytes are the trellis of the stages that run
    (active experts, nonzero scales) plus rows in, a~ and d traffic."""
    wl = synth.moe_workload("additive", materialize=False)
    gate, up, down = (exl3.DeviceProj(p, "cuda", words_fn=synth.realize_words)
                      for p in (wl.gate, wl.up, wl.down))
    x, ids, w = exl3.device_inputs(wl, "cuda")
    meta = exl3.exl3_route_pack(ids, w, wl.num_experts)
    cap = wl.rows * wl.topk
    out = torch.empty(wl.rows, wl.hidden, dtype=torch.float16, device="cuda")
    ws = torch.empty(exl3.moe_workspace_size(wl.rows, wl.topk, wl.num_experts, wl.hidden,
                                             wl.intermediate, cap),
                     dtype=torch.uint8, device="cuda")

    def call():
        exl3.exl3_moe_additive(x, wl.topk, meta, gate, up, down, cap, out=out, ws=ws)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = 1000.0 * a.elapsed_time(b) / reps
    check_status(ws, int((meta["pos_of_pair"][:wl.rows * wl.topk] < 0).sum()), "additive")
    with exl3.Profile(max_launches=8 * 4) as prof:
        for _ in range(4):
            call()
        torch.cuda.synchronize()
    kst = _kernel_stats(prof.records)
    active = np.unique(wl.ids[(wl.ids >= 0) & (wl.ids < wl.num_experts)])
    tbytes = 0
    for pr in (wl.gate, wl.up, wl.down):
        for t in range(len(pr.words)):
            for e in active:
                if float(pr.scale[t][e]) != 0.0:
                    tbytes += pr.in_features * pr.out_features * int(pr.bits[t][e]) // 8
    P = int(np.sum((wl.ids >= 0) & (wl.ids < wl.num_experts)))
    nbytes = tbytes + wl.rows * wl.hidden * 2 + P * (wl.intermediate * 2 * 2 + wl.hidden * 4 * 2)
    return {"rows": wl.rows, "us": us, "tokens_per_s": wl.rows / (us * 1e-6),
            "kernels": kst, "algorithmic_bytes": nbytes, "trellis_bytes": tbytes,
            "layer_GBps": nbytes / (us * 1e-6) / 1e9,
            "layer_hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


# ------------------------------------------------------------- CPU baseline
# The float64 oracle, as it stands, timed on the host's cores: a process pool
# (spawned workers, BLAS limited to one thread each) over a bounded sample of
# each workload. The unit of work is one routed pair (MoE layers: gate and up,
# SwiGLU, down; expert dequantisation included) or one row (linear); a
# worker's pairs are grouped by expert so each dequantises an expert once.

_CPU_WL = {}


def _cpu_workload(key):
    from trellis_quantized_moe_amd import synth
    if key not in _CPU_WL:
        if key[0] == "moe":
            _CPU_WL[key] = synth.moe_workload(key[1], rows=key[2], materialize=False)
        else:
            _CPU_WL[key] = synth.linear_workload(key[1], key[2])
    return _CPU_WL[key]


def _cpu_warm(keys):
    """Worker start-up, outside the timed region: imports, the workloads'
    inputs and the BLAS description."""
    import numpy  # noqa: F401
    from threadpoolctl import threadpool_info

    import oracle.moe  # noqa: F401
    for k in keys:
        _cpu_workload(k)
    return [(i.get("internal_api"), i.get("version")) for i in threadpool_info()]


def _cpu_task(task):
    """One worker's share of a sample; returns its busy seconds."""
    from threadpoolctl import threadpool_limits

    from oracle import linear as olin
    from oracle import moe as omoe
    from oracle.linear import WeightCache
    from trellis_quantized_moe_amd import synth
    key, items = task
    with threadpool_limits(limits=1):
        if key[0] == "moe":
            wl = _cpu_workload(key)
            experts = {e for _, _, e in items}
            views = [synth.materialized_view(p, experts) for p in (wl.gate, wl.up, wl.down)]
            t0 = time.perf_counter()
            cache = WeightCache()
            for r, j, e in items:
                at = omoe.stage1(wl.x[r:r + 1].astype(np.float64), e, *views, "R", cache)
                omoe.down_output(at, e, views[2], cache)
        else:
            proj, x = _cpu_workload(key)
            t0 = time.perf_counter()
            olin.linear(x[list(items)].astype(np.float64), proj, "R", WeightCache())
        return time.perf_counter() - t0


def _cpu_samples(synth):
    """(name, key, tokens, work items) of each sampled workload."""
    out = []
    # (workload, its rows, the sampled rows); decode: the 32-row layer
    for name, nrows, rows in (("prefill", 3072, range(16)), ("decode", 32, range(4)),
                              ("additive", 128, range(4))):
        wl = synth.moe_workload(name, rows=nrows, materialize=False)
        pairs = [(r, j, int(wl.ids[r, j])) for r in rows for j in range(wl.topk)
                 if 0 <= int(wl.ids[r, j]) < wl.num_experts]
        out.append((name, ("moe", name, nrows), len(rows), pairs))
    out.append(("linear_K4", ("linear", 4, 64), 64, list(range(64))))
    return out


def cpu_pool():
    """The worker pool of the CPU baseline, started (and its workers warmed
    up) before this process touches the GPU: its workers are new
    interpreters, and a process that has initialised the GPU starts no new
    program. Returns (pool, warm-up future list, worker count)."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    from trellis_quantized_moe_amd import synth
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    keys = [k for _, k, _, _ in _cpu_samples(synth)]
    ex = ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("spawn"))
    warm = [ex.submit(_cpu_warm, keys) for _ in range(workers)]
    return ex, warm, workers


def cpu_baseline(synth, pool):
    """The oracle over the host's cores (see above, at most 16 workers) on
    bounded samples: 16 prefill rows (128 pairs), 4 rows of the 32-row decode
    layer, 4 additive rows, 64 rows of the 4096 -> 4096 K = 4 linear. Returns
    the prefill figure (the headline workload) with the others under
    'per_workload'. pool: cpu_pool()."""
    import platform

    ex, warm, workers = pool
    samples = _cpu_samples(synth)
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    res = {}
    with ex:
        blas = [f.result() for f in warm][0]
        for name, key, tokens, items in samples:
            if key[0] == "moe":
                items = sorted(items, key=lambda t: (t[2], t[0], t[1]))
            n = min(workers, len(items))
            tasks = [(key, items[len(items) * i // n:len(items) * (i + 1) // n]) for i in range(n)]
            t0 = time.perf_counter()
            busy = list(ex.map(_cpu_task, tasks))
            wall = time.perf_counter() - t0
            res[name] = {"value": tokens / wall, "unit": "tokens/s", "cores": n,
                         "wall_s": wall, "busy_s": sum(busy),
                         "sample": "%d tokens, %d %s over %d worker processes" % (
                             tokens, len(items), "pairs" if key[0] == "moe" else "rows", n)}
    head = res["prefill"]
    return {"value": head["value"], "unit": "tokens/s", "cores": head["cores"], "kind": "oracle",
            "sample": "prefill workload, rows 0-15 with all their routed pairs (%s) through the "
                      "float64 oracle, expert dequantisation included; %.1f s wall"
                      % (head["sample"], head["wall_s"]),
            "host": {"cpu": model, "threads_available": len(os.sched_getaffinity(0)),
                     "numpy": np.__version__, "blas": blas},
            "per_workload": res}


KERNEL_SOURCES = ("gemm_wide.hip", "gemm_shared.hpp", "common.hpp", "kernels.hpp",
                  "rotate_dev.hpp", "combine_dev.hpp", "route_pack.hip", "host.cpp")


def kernel_source_sha():
    """SHA-256 over the sources of the 128-row GEMM (the prefill's dominant
    kernel), its plan builder and the host code that decides what one launch
    holds: a committed counter summary applies only to this exact code."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "trellis_quantized_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_probe(torch, gib=1.0, reps=5):
    """Plain device copy of known size, used to calibrate HBM counters."""
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode extras")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-tp", action="store_true",
                    help="skip the 4-way tensor-parallel shard shapes (intermediate / 4)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--only", default="",
                    help="comma-separated parts to run, for profiling: prefill, decode1, "
                         "decode8, decode32, additive, linear (no JSON line)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="JSON with measured HBM bytes per launch of the dominant kernel")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    # the CPU baseline's workers start now, before the GPU is touched
    pool = cpu_pool() if not (args.no_cpu or args.only or args.copy_probe) else None

    import torch

    from trellis_quantized_moe_amd import exl3, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    exl3.lib()
    if args.copy_probe:
        copy_probe(torch)
        return

    if args.only:
        parts = set(args.only.split(","))
        res = {}
        if "prefill" in parts:
            res["prefill"] = run_prefill(args, torch, exl3, synth)[1]
        for M in (1, 8, 32):
            if "decode%d" % M in parts:
                res["decode_M%d" % M] = run_decode(args, torch, exl3, synth, M)
        if "additive" in parts:
            res["additive"] = run_additive(args, torch, exl3, synth)
        if "linear" in parts:
            res["linear"] = run_linear(args, torch, exl3, synth)
        print(json.dumps({"only": sorted(parts), "results": res}), flush=True)
        return

    wl, pre = run_prefill(args, torch, exl3, synth)
    extra = {"prefill": pre}
    if not args.no_decode:
        for M in (1, 8, 32):
            _log("decode M=%d" % M)
            extra["decode_M%d" % M] = run_decode(args, torch, exl3, synth, M)
        _log("additive layer")
        extra["additive"] = run_additive(args, torch, exl3, synth)
        _log("linear 4096 -> 4096")
        extra["linear"] = run_linear(args, torch, exl3, synth)
    if not args.no_tp:
        # one GPU's share under 4-way tensor parallelism: intermediate / 4
        _log("tp4 shard: decode M=32, intermediate 384")
        extra["tp4_shard_decode_M32"] = run_decode(args, torch, exl3, synth, 32, I=384)
        _log("tp4 shard: prefill, intermediate 512")
        extra["tp4_shard_prefill"] = run_prefill(args, torch, exl3, synth, I=512)[1]

    dom = pre["dominant"]
    # HBM bytes per launch of the dominant kernel from the committed rocprofv3
    # counter summary, only while the kernel source is the one measured
    traffic = None
    if os.path.exists(args.traffic):
        import hashlib
        with open(args.traffic) as f:
            t = json.load(f)
        sha = kernel_source_sha()
        if (t.get("kernel") == dom and t.get("workload") == "prefill"
                and t.get("source_sha256") == sha):
            traffic = t.get("bytes_per_launch")
    roof = {"bound": "mfma", "kernel": dom, "achieved": pre["achieved_tflops"],
            "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": pre["achieved_tflops"] / MFMA_F16_PEAK_TFLOPS, "traffic": traffic,
            "per_launch": "%.4g flops: the layer's 2 x pairs x in x out over gate, up "
                          "and down, divided by its launches of this kernel" % pre["per_launch_flops"]}
    cpu = None
    if not args.no_cpu:
        _log("cpu baseline (oracle)")
        cpu = cpu_baseline(synth, pool)

    line = {
        "metric": METRIC, "value": pre["tokens_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": pre["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "prefill MoE layer: 192 experts, top-8, hidden 6144, "
                               "intermediate 2048, K per expert in {3,4,5,6,8}, 3072 rows, "
                               "Zipf(1.2) routing, capacity 2048 pairs",
                   "global_batch": wl.rows, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
