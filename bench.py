"""Benchmark of the local MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one moe_forward call (route -> dispatch -> SwiGLU experts ->
combine) over one batch of synthetic inputs already resident in HBM; for the
``grouped`` workload, one moe_forward_sigmoid_grouped call (group-limited
sigmoid routing in place of the softmax).  The default workload is the
largest single-GPU layer, the fine-grained many-expert bf16 layer (T=8192,
H=7168, I=2048, E=64, top-8, renormalised, per-expert logit bias so some
experts get no token); ``--workload mixtral``, ``decode32``, ``decode256``
and ``grouped`` select the others.  W untimed steps, then K timed steps bracketed by
device synchronisation; one JSON line on stdout.

In the timed steps the library records HIP events (moe_set_timing_events)
only around the gate+up grouped GEMM with the SwiGLU epilogue, the dominant
kernel the roofline object describes, on the forward's stream: each
recorded mark costs a few microseconds of GPU time.  A second, untimed pass
of K steps records all 8 marks for the per-stage durations ("stages",
averaged) and step_gpu_ms (median and minimum GPU time of one step, first
kernel start to last kernel end, marks included).  The CPU baseline times
the oracle (numpy) on a few tokens of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("MoE forward tokens/sec + grouped-GEMM MFMA util; "
          "route/dispatch/combine HBM GB/s")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# The forward's stages between its timing marks.  Its dispatch writes only
# the mapping where the gate+up GEMM gathers the token rows from x, else it
# also scatters them (forward_gathers).
KERNELS = ["route", "dispatch_count", "dispatch_scan", "dispatch",
           "gateup_gemm", "down_gemm", "combine"]


def forward_gathers(wl):
    """Whether moe_forward reads the token rows in place for this workload
    (the library's rule: the MFMA paths, except prefill-sized segments with
    more than 32 gate+up column blocks of 256, where the scatter is cheaper)."""
    N, E, I = wl["T"] * wl["k"], wl["E"], wl["I"]
    if wl["fmt"] == "f32":
        return False
    prefill = N >= 96 * E
    return not (prefill and 2 * I > 32 * 256)


def mark_cost_ms(dev):
    """Median interval between two events recorded back to back on the
    stream: what a timing mark with no kernel after it measures."""
    import torch
    stream = torch.cuda.current_stream(dev)
    t = []
    for _ in range(16):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        torch.cuda.synchronize(dev)
        t.append(a.elapsed_time(b))
    return sorted(t)[len(t) // 2]


def fuse_stages(per, alg, empty_ms):
    """(names, per-stage ms, algorithmic work) with the route and count
    stages merged when the count ran inside the routing launch: the count
    interval then holds no kernel (shorter than `empty_ms`, a bound on
    what two marks recorded back to back measure) and the two are reported
    as one, "route+dispatch_count"."""
    names = list(KERNELS)
    per, alg = dict(per), dict(alg)
    if per["dispatch_count"] < empty_ms:
        name = "route+dispatch_count"
        per[name] = per.pop("route") + per.pop("dispatch_count")
        alg[name] = dict(bytes=alg["route"]["bytes"]
                         + alg["dispatch_count"]["bytes"])
        names = [name] + names[2:]
    return names, per, alg

WORKLOADS = {
    "mixtral": ("mixtral", None),
    "fine": ("fine", None),
    "decode32": ("decode", 32),
    "decode256": ("decode", 256),
    "grouped": ("grouped", None),
}
CPU_SAMPLE_MAX_TOKENS = 256
CPU_SAMPLE_SECONDS = 15.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="fine", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run one plain device copy of COPY_BYTES (for "
                        "scaling the FETCH_SIZE/WRITE_SIZE counters)")
    p.add_argument("--record-traffic", nargs=2, metavar=("PROF_DIR", "COPY_DIR"),
                   help="no GPU work: read the rocprofv3 FETCH_SIZE and "
                        "WRITE_SIZE runs under PROF_DIR/{fetch,write} (this "
                        "workload) and COPY_DIR/{fetch,write} (the copy "
                        "calibration), update profiles/traffic.json and print "
                        "a markdown table")
    p.add_argument("--route-sweep", action="store_true",
                   help="extension, not the benchmark: time moe_route and "
                        "moe_route_sigmoid_grouped alone at T = 2^16, 2^18, "
                        "2^20 (bf16 logits, the cases listed in ROUTE_SWEEP) "
                        "with the Infinity Cache flushed before each call; "
                        "one JSON line per case")
    p.add_argument("--router-weights-sweep", action="store_true",
                   help="extension, not the benchmark: time "
                        "moe_selected_router_weights and "
                        "moe_selected_router_backward alone at T = 2^16, "
                        "2^18, 2^20; one JSON line per case")
    p.add_argument("--train", action="store_true",
                   help="extension, not the benchmark: time one first-order "
                        "training step (forward and the backward chain) of "
                        "the workload; one JSON line")
    p.add_argument("--clipped", action="store_true",
                   help="extension, not the benchmark: time the expert stage "
                        "with the plain and the clipped SwiGLU epilogue")
    p.add_argument("--vendor-reference", action="store_true",
                   help="extension, not the benchmark: the expert stage "
                        "beside hipBLASLt (torch.mm) running the same "
                        "per-expert GEMMs")
    p.add_argument("--cold-cache", action="store_true",
                   help="extension, not the benchmark: the forward with the "
                        "Infinity Cache flushed before every step; per-kernel "
                        "HBM rates")
    p.add_argument("--graph", action="store_true",
                   help="also time the forward captured once in a HIP graph "
                        "and replayed per step (an extension field 'graph'; "
                        "the headline value stays the eager forward)")
    p.add_argument("--summarize-counters", metavar="PMC_DIR",
                   help="print a table of a rocprofv3 --pmc run's counters "
                        "per library kernel (no GPU work)")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="no GPU work: print the kernel statistics of a "
                        "rocprofv3 --kernel-trace --stats run as markdown")
    return p.parse_args()


COPY_BYTES = 4 << 30  # 4 GiB: far beyond the 256 MB Infinity Cache


def copy_calibration():
    """One plain copy of COPY_BYTES between two fresh buffers, after a
    write that evicts the source from the Infinity Cache."""
    import torch
    n = COPY_BYTES // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    flush = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda")
    flush.fill_(0.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


def algorithmic(wl, counts):
    """Algorithmic work of each kernel for one forward (bytes moved or
    FLOP), from the sizes and the routing histogram."""
    T, H, I, E, k = wl["T"], wl["H"], wl["I"], wl["E"], wl["k"]
    s = 2 if wl["fmt"] != "f32" else 4
    sl = s
    N = T * k
    touched = int((counts > 0).sum())
    w_gu = 2 * touched * I * H * s
    w_d = touched * H * I * s
    return {
        "route": dict(bytes=T * E * sl + N * (4 + sl)
                      + (E * 4 if wl.get("bias") is not None else 0)),
        "dispatch_count": dict(bytes=N * 4 * 2),
        "dispatch_scan": dict(bytes=(E + 1) * 4),
        # idx and ranks read, token_row / row_expert / row_token written;
        # with the scatter also every token row read and its k copies written
        "dispatch": dict(bytes=N * 4 * 5 + (0 if forward_gathers(wl)
                                            else T * H * s + N * H * s)),
        "gateup_gemm": dict(flop=4 * N * H * I,
                            bytes=N * H * s + w_gu + N * I * s),
        "down_gemm": dict(flop=2 * N * H * I,
                          bytes=N * I * s + w_d + N * H * s),
        "combine": dict(bytes=N * H * s + N * (4 + sl) + T * H * s),
        "touched_experts": touched,
    }


TRAFFIC_SOURCES = [
    "mixture_experts_layer_28_amd/csrc/gemm_big.hip",
    "mixture_experts_layer_28_amd/csrc/gemm_common.h",
    "mixture_experts_layer_28_amd/csrc/device_common.h",
    "mixture_experts_layer_28_amd/csrc/gemm.hip",
]
# kernel-name fragments of each timed kernel whose traffic is recorded
# (prefill and decode-sized forms)
TRAFFIC_KERNELS = {"gateup_gemm": ("gemm_big_kernel<2, true",
                                   "gemm_mfma_kernel<2, 32, 128, 1, true"),
                   "down_gemm": ("gemm_big_kernel<2, false",
                                 "gemm_mfma_kernel<2, 32, 128, 1, false")}


def _counter_rows(run_dir):
    """{dispatch id: (kernel name, summed counter value)} of one rocprofv3
    --pmc run with a single counter (values summed over its instances)."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                d = int(r["Dispatch_Id"])
                name, v = out.get(d, (r["Kernel_Name"], 0.0))
                out[d] = (name, v + float(r["Counter_Value"]))
    return out


def _sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def record_traffic(workload, prof_dir, copy_dir):
    """Scale the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of the
    timed kernels by what the same counters read for the plain copy of
    COPY_BYTES, and store the per-launch HBM bytes in profiles/traffic.json."""
    def last_value(run):
        rows = _counter_rows(run)
        return rows[max(rows)][1]
    cf, cw = last_value(os.path.join(copy_dir, "fetch")), last_value(
        os.path.join(copy_dir, "write"))
    fetch_factor = COPY_BYTES / 1024.0 / cf
    write_factor = COPY_BYTES / 1024.0 / cw
    fetch = _counter_rows(os.path.join(prof_dir, "fetch"))
    write = _counter_rows(os.path.join(prof_dir, "write"))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        doc = {}
    doc["about"] = (
        "HBM traffic per launch of the dominant kernels, from two rocprofv3 "
        "--pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) of "
        "bench.py, each scaled by what the same counter reads for a plain "
        "4 GiB device copy (bench.py --copy-calibration).  Written by "
        "bench.py --record-traffic; bench.py reports a kernel's traffic only "
        "while the sha256 of the listed sources still matches.")
    doc["sources"] = TRAFFIC_SOURCES
    doc["copy_calibration"] = dict(copy_bytes=COPY_BYTES, fetch_kib=cf,
                                   write_kib=cw,
                                   fetch_factor=round(fetch_factor, 4),
                                   write_factor=round(write_factor, 4))
    doc.setdefault("kernels", {})
    sha = _sources_sha256()
    lines = ["| kernel | FETCH_SIZE KiB per dispatch | WRITE_SIZE KiB per "
             "dispatch | scaled traffic per launch |", "|---|---|---|---|"]
    for key, frags in TRAFFIC_KERNELS.items():
        fk = [v for d, (n, v) in sorted(fetch.items())
              if any(f in n for f in frags)]
        wk = [v for d, (n, v) in sorted(write.items())
              if any(f in n for f in frags)]
        if not fk or not wk:
            continue
        traffic = int(round(sum(fk) / len(fk) * 1024 * fetch_factor +
                            sum(wk) / len(wk) * 1024 * write_factor))
        doc["kernels"]["%s/%s" % (workload, key)] = dict(
            source_sha256=sha, fetch_kib=fk, write_kib=wk,
            traffic_bytes_per_launch=traffic)
        lines.append("| %s | %s | %s | %.3f GB |" % (
            key, ", ".join("%.0f" % v for v in fk),
            ", ".join("%.0f" % v for v in wk), traffic / 1e9))
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print("Calibration: the %d-byte copy reads FETCH_SIZE = %.0f KiB and "
          "WRITE_SIZE = %.0f KiB: fetch x %.4f, write x %.4f.\n" % (
              COPY_BYTES, cf, cw, fetch_factor, write_factor))
    print("\n".join(lines))


# (router, E, top_k, groups, selected_groups); the sigmoid cases keep the top
# two of each group's scores
ROUTE_SWEEP = [("softmax", 8, 2, 0, 0), ("softmax", 64, 8, 0, 0),
               ("softmax", 128, 8, 0, 0), ("softmax", 256, 8, 0, 0),
               ("sigmoid", 64, 8, 8, 4), ("sigmoid", 256, 8, 8, 4)]


def route_sweep():
    """Streaming efficiency of the routing kernels on their own at large T
    (the benchmark workloads hold at most 1.5 MB of logits, far below where
    HBM bandwidth decides).  Bytes: T*E logits read + T*k*(4 + 2) written
    (+ 4*E of bias for the sigmoid router)."""
    import statistics
    import torch
    import mixture_experts_layer_28_amd as moe
    flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)
    for kind, E, k, groups, sel in ROUTE_SWEEP:
        bias = torch.randn(E, device="cuda", generator=gen) * 0.25
        for T in (1 << 16, 1 << 18, 1 << 20):
            lg = torch.randn(T, E, device="cuda", generator=gen).to(
                torch.bfloat16)
            idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
            w = torch.empty(T, k, dtype=torch.bfloat16, device="cuda")

            def call():
                if kind == "softmax":
                    moe.moe_route(lg, k, True, idx, w)
                else:
                    moe.moe_route_sigmoid_grouped(
                        lg, k, groups, sel, bias=bias, group_top_two=True,
                        renormalize=True, scale=2.5, idx=idx, weights=w)

            call()
            torch.cuda.synchronize()
            ts = []
            for _ in range(7):
                flush.fill_(1)  # evicts the 256 MB Infinity Cache
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            ms = statistics.median(ts)
            nbytes = T * E * 2 + T * k * 6 + (E * 4 if kind != "softmax"
                                              else 0)
            print(json.dumps({"extension": "route_sweep", "router": kind,
                              "E": E, "top_k": k, "groups": groups,
                              "selected_groups": sel, "T": T,
                              "us": round(ms * 1e3, 1),
                              "GB/s": round(nbytes / ms / 1e6, 1),
                              "hbm_frac": round(nbytes / ms / 1e6 /
                                                PEAK_HBM_GBS, 4)}),
                  flush=True)


ROUTER_WEIGHTS_SWEEP = [(64, 8), (256, 8)]  # (E, top_k), int64 indices


def router_weights_sweep():
    """The router-weight kernels of a fixed selection (weights, then the
    logits gradient) on their own at large T, bf16 logits, softmax scoring,
    renormalised, Infinity Cache flushed before each call.  Algorithmic
    bytes: weights T*E*2 logits + T*k*8 indices read, T*k*4 written;
    backward the same reads plus T*k*4 grad_weights, T*E*2 written."""
    import statistics
    import torch
    import mixture_experts_layer_28_amd as moe
    flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(11)
    for E, k in ROUTER_WEIGHTS_SWEEP:
        for T in (1 << 16, 1 << 18, 1 << 20):
            lg = torch.randn(T, E, device="cuda", generator=gen).to(
                torch.bfloat16)
            ind = torch.topk(lg.float(), k, dim=1).indices.contiguous()
            g = torch.randn(T, k, device="cuda", generator=gen)
            w = torch.empty(T, k, device="cuda")
            dx = torch.empty(T, E, device="cuda", dtype=torch.bfloat16)
            calls = {
                "weights": (lambda: moe.moe_selected_router_weights(
                    lg, ind, "softmax", True, 1.0, out=w),
                    T * E * 2 + T * k * 8 + T * k * 4),
                "backward": (lambda: moe.moe_selected_router_backward(
                    lg, ind, g, "softmax", True, 1.0, out=dx),
                    T * E * 2 + T * k * 12 + T * E * 2),
            }
            for name, (call, nbytes) in calls.items():
                call()
                torch.cuda.synchronize()
                ts = []
                for _ in range(7):
                    flush.fill_(1)
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    call()
                    b.record()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                ms = statistics.median(ts)
                print(json.dumps({"extension": "router_weights_sweep",
                                  "kernel": name, "E": E, "top_k": k,
                                  "T": T, "us": round(ms * 1e3, 1),
                                  "GB/s": round(nbytes / ms / 1e6, 1),
                                  "hbm_frac": round(nbytes / ms / 1e6 /
                                                    PEAK_HBM_GBS, 4)}),
                      flush=True)


TRAIN_STAGES = ["route", "router_weights", "dispatch", "experts_fwd",
                "combine", "combine_bwd", "experts_bwd", "dispatch_bwd",
                "router_bwd"]
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector


def train_step_bench(args):
    """Extension, not the benchmark: one first-order training step of the
    MoE layer for a fixed output gradient -- softmax route, FP32 router
    weights of the choice, dispatch, training forward, combine, then the
    backward chain (combine, experts, dispatch, router).  Per-stage times
    from torch events on the one stream every call is enqueued on."""
    import torch

    import mixture_experts_layer_28_amd as moe
    from mixture_experts_layer_28_amd import workloads

    dev = torch.device("cuda:0")
    base, T = WORKLOADS[args.workload]
    wl = workloads.make(base, T=T, device=dev)
    T, H, I, E, k = wl["T"], wl["H"], wl["I"], wl["E"], wl["k"]
    x, logits = wl["x"], wl["logits"]
    wg, wu, wd = wl["w_gate"], wl["w_up"], wl["w_down"]
    gen = torch.Generator(device=dev).manual_seed(5)
    dout = torch.randn((T, H), generator=gen, device=dev).to(x.dtype)
    N = T * k
    ws = torch.empty(moe.moe_experts_backward_workspace_size(
        N, H, I, E, x.dtype), dtype=torch.uint8, device=dev)

    def step(ev=None):
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        mark(0)
        idx, _ = moe.moe_route(logits, k, wl["renorm"])
        mark(1)
        w = moe.moe_selected_router_weights(logits, idx, "softmax",
                                            wl["renorm"], index_type="u32")
        mark(2)
        d = moe.moe_dispatch(x, idx, E)
        mark(3)
        cache = moe.moe_experts_forward_training(d["xd"], d["offsets"], wg,
                                                 wu, wd)
        mark(4)
        moe.moe_combine(cache["y"], w, d["token_row"])
        mark(5)
        dexp, dw = moe.moe_combine_backward(cache["y"], w, d["token_row"],
                                            dout)
        mark(6)
        b = moe.moe_experts_backward(d["xd"], d["offsets"], wg, wu, wd, cache,
                                     dexp, workspace=ws)
        mark(7)
        moe.moe_dispatch_backward(b["grad_xd"], d["token_row"])
        mark(8)
        moe.moe_selected_router_backward(logits, idx, dw, "softmax",
                                         wl["renorm"], index_type="u32")
        mark(9)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(10)]
             for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i])
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    per = {name: sum(m[j].elapsed_time(m[j + 1]) for m in marks) / args.steps
           for j, name in enumerate(TRAIN_STAGES)}
    # 6 N H I FLOP forward (three products), 12 N H I backward (six)
    flop = 18 * N * H * I
    ms_step = elapsed / args.steps * 1e3
    print(json.dumps({
        "extension": "train_step", "metric": "MoE training step tokens/sec",
        "value": round(T * args.steps / elapsed, 1), "unit": "tokens/s",
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "tflops_per_step": round(flop / (ms_step * 1e-3) / 1e12, 1),
        "config": {"workload": base, "T": T, "H": H, "I": I, "E": E,
                   "top_k": k},
        "stages_ms": {n: round(v, 4) for n, v in per.items()},
        "experts_bwd_tflops": round(12 * N * H * I /
                                    (per["experts_bwd"] * 1e-3) / 1e12, 1),
        "experts_fwd_tflops": round(6 * N * H * I /
                                    (per["experts_fwd"] * 1e-3) / 1e12, 1),
        # the expert backward as a whole (its GEMMs, transposes and
        # elementwise kernels) against the dense bf16 MFMA peak
        "roofline": {"bound": "mfma", "kernel": "experts_bwd",
                     "achieved": round(12 * N * H * I /
                                       (per["experts_bwd"] * 1e-3) / 1e12, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(12 * N * H * I /
                                   (per["experts_bwd"] * 1e-3) / 1e12 /
                                   PEAK_BF16_TFLOPS, 4)}}),
        flush=True)


def clipped_bench(args):
    """Extension, not the benchmark: the expert stage of the workload with
    the plain and with the clipped SwiGLU epilogue (alpha 1.702, limit 7) on
    the same dispatched rows, alternating, torch events around each call."""
    import statistics
    import torch

    import mixture_experts_layer_28_amd as moe
    from mixture_experts_layer_28_amd import workloads

    base, T = WORKLOADS[args.workload]
    wl = workloads.make(base, T=T, device="cuda")
    idx, _ = moe.moe_route(wl["logits"], wl["k"], wl["renorm"])
    d = moe.moe_dispatch(wl["x"], idx, wl["E"])
    N, H, I = d["xd"].shape[0], wl["H"], wl["I"]
    act = torch.empty((N, I), dtype=d["xd"].dtype, device="cuda")
    y = torch.empty((N, H), dtype=d["xd"].dtype, device="cuda")
    calls = {
        "plain": lambda: moe.moe_experts_forward(
            d["xd"], d["offsets"], wl["w_gate"], wl["w_up"], wl["w_down"],
            act=act, y=y),
        "clipped": lambda: moe.moe_experts_forward_clipped(
            d["xd"], d["offsets"], wl["w_gate"], wl["w_up"], wl["w_down"],
            1.702, 7.0, act=act, y=y),
    }
    times = {name: [] for name in calls}
    for _ in range(args.warmup):
        for call in calls.values():
            call()
    for _ in range(args.steps):
        for name, call in calls.items():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            times[name].append(a.elapsed_time(b))
    flop = 6 * N * H * I
    out = {"extension": "clipped_swiglu", "workload": base, "N": N}
    for name, ts in times.items():
        ms = statistics.median(ts)
        out[name] = {"ms": round(ms, 4),
                     "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    print(json.dumps(out), flush=True)


def vendor_reference_bench(args):
    """Extension, not the benchmark: the expert stage's two grouped GEMMs
    beside the vendor library on the same work.  The reference runs, per
    expert with rows, hipBLASLt (through torch.mm, bf16, FP32 accumulation)
    on that expert's dispatched rows: xd_e . [W_gate; W_up]_e^T (one product
    of 2I columns) and act_e . W_down_e^T, weights pre-transposed to
    contiguous [K, N] outside the timed region; no SwiGLU (GEMMs only), so
    the library's gate+up epilogue is extra work on its side.  Both run in
    one process, alternating, torch events around each.  A third line runs
    the same FLOPs ungrouped (all rows against the first expert's weights,
    two dense products): what the library reaches on a plain GEMM of that
    size, for scale."""
    import statistics
    import torch

    import mixture_experts_layer_28_amd as moe
    from mixture_experts_layer_28_amd import workloads

    base, T = WORKLOADS[args.workload]
    wl = workloads.make(base, T=T, device="cuda")
    idx, _ = moe.moe_route(wl["logits"], wl["k"], wl["renorm"])
    d = moe.moe_dispatch(wl["x"], idx, wl["E"])
    xd = d["xd"]
    N, H, I, E = xd.shape[0], wl["H"], wl["I"], wl["E"]
    off = d["offsets"].cpu().numpy().astype("int64")
    segs = [(e, int(off[e]), int(off[e + 1])) for e in range(E)
            if off[e + 1] > off[e]]
    act = torch.empty((N, I), dtype=xd.dtype, device="cuda")
    y = torch.empty((N, H), dtype=xd.dtype, device="cuda")
    # [K, N] row-major copies of the weights for torch.mm (no transposed views)
    wgu_t = [torch.cat([wl["w_gate"][e], wl["w_up"][e]], 0).t().contiguous()
             for e, _, _ in segs]
    wd_t = [wl["w_down"][e].t().contiguous() for e, _, _ in segs]
    gu = torch.empty((N, 2 * I), dtype=xd.dtype, device="cuda")
    yv = torch.empty((N, H), dtype=xd.dtype, device="cuda")

    def vendor():
        for (e, lo, hi), wg, wd in zip(segs, wgu_t, wd_t):
            torch.mm(xd[lo:hi], wg, out=gu[lo:hi])
            torch.mm(act[lo:hi], wd, out=yv[lo:hi])

    def vendor_dense():
        # the same FLOPs with no grouping: every row against one expert's
        # weights, two dense products (the library's best case)
        torch.mm(xd, wgu_t[0], out=gu)
        torch.mm(act, wd_t[0], out=yv)

    calls = {
        "library": lambda: moe.moe_experts_forward(
            xd, d["offsets"], wl["w_gate"], wl["w_up"], wl["w_down"],
            act=act, y=y),
        "hipblaslt_per_expert": vendor,
        "hipblaslt_dense_one_expert": vendor_dense,
    }
    times = {name: [] for name in calls}
    for _ in range(args.warmup):
        for call in calls.values():
            call()
    for _ in range(args.steps):
        for name, call in calls.items():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            times[name].append(a.elapsed_time(b))
    flop = 6 * N * H * I
    out = {"extension": "vendor_reference", "workload": base, "N": N,
           "experts_with_rows": len(segs)}
    for name, ts in times.items():
        ms = statistics.median(ts)
        out[name] = {"ms": round(ms, 4),
                     "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    print(json.dumps(out), flush=True)


def cold_cache_bench(args):
    """Extension, not the benchmark: the forward with the 256 MB Infinity
    Cache flushed before every step (a 1 GB fill, outside the events), so
    each kernel's bytes come from HBM; per-kernel times from the library's
    timing events, rates against the algorithmic bytes."""
    import numpy as np
    import torch

    import mixture_experts_layer_28_amd as moe
    from mixture_experts_layer_28_amd import _lib, workloads

    dev = torch.device("cuda:0")
    base, T = WORKLOADS[args.workload]
    wl = workloads.make(base, T=T, device=dev)
    T, H, I, E, k = wl["T"], wl["H"], wl["I"], wl["E"], wl["k"]
    x, logits = wl["x"], wl["logits"]
    idx, _ = moe.moe_route(logits, k, wl["renorm"])
    d = moe.moe_dispatch(x, idx, E)
    counts = np.diff(d["offsets"].cpu().numpy().astype(np.int64))
    del d, idx
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I, E, k, x.dtype),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=x.dtype, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    L = _lib.lib()
    per = {name: [] for name in KERNELS}
    for i in range(args.warmup + args.steps):
        flush.fill_(i & 0xff)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        stream = torch.cuda.current_stream(dev)
        for ev in evs:
            ev.record(stream)
        handles = (_lib.ctypes.c_void_p * 8)(*[ev.cuda_event for ev in evs])
        _lib.check(L.moe_set_timing_events(handles, 8))
        moe.moe_forward(x, logits, wl["w_gate"], wl["w_up"], wl["w_down"], k,
                        wl["renorm"], out=out, workspace=ws)
        _lib.check(L.moe_set_timing_events(None, 0))
        torch.cuda.synchronize(dev)
        if i >= args.warmup:
            for j, name in enumerate(KERNELS):
                per[name].append(evs[j].elapsed_time(evs[j + 1]))
    med = {name: sorted(v)[len(v) // 2] for name, v in per.items()}
    names, med, alg = fuse_stages(med, algorithmic(wl, counts),
                                  1.5 * mark_cost_ms(dev))
    stages = {}
    for name in names:
        ms = med[name]
        st = {"ms": round(ms, 5),
              "gbs": round(alg[name]["bytes"] / (ms * 1e-3) / 1e9, 1)}
        st["hbm_frac"] = round(st["gbs"] / PEAK_HBM_GBS, 4)
        if "flop" in alg[name]:
            st["tflops"] = round(alg[name]["flop"] / (ms * 1e-3) / 1e12, 1)
        stages[name] = st
    step_ms = sum(st["ms"] for st in stages.values())
    print(json.dumps({"extension": "cold_cache", "workload": base, "T": T,
                      "step_gpu_ms_sum_of_medians": round(step_ms, 4),
                      "stages": stages}), flush=True)


def summarize_trace(trace_dir):
    """Markdown table of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"),
                      recursive=True)
    print("| kernel | calls | total us | average us | min us | max us | % |")
    print("|---|---|---|---|---|---|---|")
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Name"].replace("(anonymous namespace)::", "")
                name = name.replace("void ", "").split("(")[0]
                if not name.startswith("moe::"):
                    continue  # the input generator's kernels
                print("| %s | %s | %.1f | %.1f | %.1f | %.1f | %.1f |" % (
                    name, r["Calls"], float(r["TotalDurationNs"]) / 1e3,
                    float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3, float(r["Percentage"])))


CUS = 256        # MI355X: 256 compute units
SIMDS = CUS * 4  # ... of 4 SIMDs each
XCDS = 8         # ... in 8 XCDs


def summarize_counters(run_dir):
    """Markdown table of one rocprofv3 --pmc run: per library kernel, the
    mean over its dispatches of each counter as rocprofv3 reports it (one
    value per dispatch, summed over the counter's dimensions: GRBM_ counters
    over the 8 XCDs, so GRBM_GUI_ACTIVE / 8 is the kernel's active cycles),
    the mean dispatch duration from the same run's timestamps, and where the
    counters allow it the MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
    the active cycles times the SIMDs), the bf16 MFMA FLOP
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) with its rate, the clock (active
    cycles over the duration), and FETCH_SIZE / WRITE_SIZE in MB as counted
    (KiB x 1024, before any copy calibration)."""
    import csv
    import glob
    vals, meta = {}, {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                d, c = int(r["Dispatch_Id"]), r["Counter_Name"]
                vals.setdefault((d, c), []).append(float(r["Counter_Value"]))
                meta[d] = (r["Kernel_Name"], int(r["End_Timestamp"]) -
                           int(r["Start_Timestamp"]))
    per = {}
    for (d, c), v in vals.items():
        name = meta[d][0].replace("(anonymous namespace)::", "")
        name = name.replace("void ", "").split("(")[0]
        if not name.startswith("moe::"):
            continue
        x = sum(v)
        k = per.setdefault(name, {"_d": {}})
        k.setdefault(c, {})[d] = x
        k["_d"][d] = meta[d][1]
    counters = sorted({c for k in per.values() for c in k if c != "_d"})
    derived = []
    if {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"} <= set(counters):
        derived.append("MFMA busy %")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in counters:
        derived += ["bf16 MFMA TFLOP", "TFLOP/s"]
    if "GRBM_GUI_ACTIVE" in counters:
        derived.append("GHz")
    if {"SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"} <= set(counters):
        derived.append("LDS busy %")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in counters:
            derived.append(c + " MB")
    # wave-state counters over SQ_WAVE_CYCLES (all in quad-cycles summed
    # over the SIMDs): the share of the waves' resident time spent so
    shares = [c for c in WAVE_SHARES if c in counters]
    if "SQ_WAVE_CYCLES" in counters:
        derived += ["%s %%" % WAVE_SHARES[c] for c in shares]
    cols = ["kernel", "dispatches", "mean us"] + counters + derived
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for name, k in sorted(per.items(), key=lambda kv: -sum(kv[1]["_d"].values())):
        n = len(k["_d"])
        us = sum(k["_d"].values()) / n / 1e3
        mean = {c: sum(k[c].values()) / len(k[c]) for c in counters if c in k}
        row = [name, str(n), "%.1f" % us] + ["%.4g" % mean[c] if c in mean
                                             else "" for c in counters]
        if "MFMA busy %" in derived:
            row.append("%.1f" % (100.0 * mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0)
                                 / (mean["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)))
        if "TFLOP/s" in derived:
            fl = mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512
            row += ["%.4g" % (fl / 1e12), "%.0f" % (fl / (us * 1e-6) / 1e12)]
        if "GHz" in derived:
            row.append("%.2f" % (mean["GRBM_GUI_ACTIVE"] / XCDS / (us * 1e3)))
        if "LDS busy %" in derived:
            # cycles a CU's LDS serves indexed (ds_*) accesses, summed over
            # the CUs, over the active cycles times the CUs
            row.append("%.1f" % (100.0 * mean.get("SQ_LDS_IDX_ACTIVE", 0)
                                 / (mean["GRBM_GUI_ACTIVE"] / XCDS * CUS)))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c + " MB" in derived:
                row.append("%.1f" % (mean.get(c, 0) * 1024 / 1e6))
        if "SQ_WAVE_CYCLES" in counters:
            wc = mean.get("SQ_WAVE_CYCLES", 0)
            row += ["%.1f" % (100.0 * mean.get(c, 0) / wc) if wc else ""
                    for c in shares]
        print("| " + " | ".join(row) + " |")


# counter -> column label of its share of SQ_WAVE_CYCLES
WAVE_SHARES = {"SQ_WAIT_ANY": "waiting", "SQ_WAIT_INST_ANY": "waiting on a dependency",
               "SQ_ACTIVE_INST_ANY": "issuing", "SQ_ACTIVE_INST_VMEM": "issuing VMEM",
               "SQ_ACTIVE_INST_LDS": "issuing LDS", "SQ_WAIT_INST_LDS": "waiting to issue LDS"}


def recorded_traffic(key):
    """HBM bytes per launch recorded in profiles/traffic.json for `key`, if
    the kernel sources still hash to what they were when the counters were
    taken; None otherwise (the kernel has changed since)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
        rec = doc["kernels"][key]
        if doc["sources"] != TRAFFIC_SOURCES:
            return None
        sha = _sources_sha256()
    except (OSError, KeyError, ValueError):
        return None
    if sha != rec["source_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


def cpu_baseline(wl):
    """The oracle, untuned, on a bounded sample of the workload's tokens:
    tokens drawn at random are pushed through the oracle one at a time
    until about CPU_SAMPLE_SECONDS have passed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from mixture_experts_layer_28_amd import workloads
    from oracle.grouped import forward_sigmoid_tokens
    from oracle.moe import forward_tokens

    fmt = wl["fmt"]
    host = {key: workloads.to_numpy(wl[key], fmt)
            for key in ("x", "logits", "w_gate", "w_up", "w_down")}
    grouped = "groups" in wl
    bias = wl["bias"].cpu().numpy() if wl.get("bias") is not None else None
    rng = np.random.default_rng(123)
    order = rng.permutation(wl["T"])[:CPU_SAMPLE_MAX_TOKENS].tolist()
    tokens = 0
    t0 = time.perf_counter()
    for t in order:
        if grouped:
            forward_sigmoid_tokens(
                host["x"], host["logits"], bias, host["w_gate"],
                host["w_up"], host["w_down"], wl["k"], wl["groups"],
                wl["selected_groups"], wl["group_top_two"], wl["renorm"],
                wl["scale"], fmt, [t])
        else:
            forward_tokens(host["x"], host["logits"], host["w_gate"],
                           host["w_up"], host["w_down"], wl["k"],
                           wl["renorm"], fmt, [t])
        tokens += 1
        if time.perf_counter() - t0 >= CPU_SAMPLE_SECONDS:
            break
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": model,
            "sample": "%d of %d tokens (route, k experts, combine per token; "
                      "numpy float64), %.1f s" % (tokens, wl["T"], dt)}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.route_sweep:
        route_sweep()
        return
    if args.router_weights_sweep:
        router_weights_sweep()
        return
    if args.train:
        train_step_bench(args)
        return
    if args.clipped:
        clipped_bench(args)
        return
    if args.cold_cache:
        cold_cache_bench(args)
        return
    if args.vendor_reference:
        vendor_reference_bench(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (expert/data parallelism is described, not built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_28_amd as moe
    from mixture_experts_layer_28_amd import _lib, workloads

    dev = torch.device("cuda:0")
    base, T = WORKLOADS[args.workload]
    wl = workloads.make(base, T=T, device=dev)
    T, H, I, E, k = wl["T"], wl["H"], wl["I"], wl["E"], wl["k"]
    x, logits = wl["x"], wl["logits"]
    wg, wu, wd = wl["w_gate"], wl["w_up"], wl["w_down"]

    grouped = base == "grouped"
    if grouped:
        gargs = (k, wl["groups"], wl["selected_groups"])
        gopts = dict(bias=wl["bias"], group_top_two=wl["group_top_two"],
                     renormalize=wl["renorm"], scale=wl["scale"])

    # routing histogram (outside the timed region): touched experts
    if grouped:
        idx, _ = moe.moe_route_sigmoid_grouped(logits, *gargs, **gopts)
    else:
        idx, _ = moe.moe_route(logits, k, wl["renorm"])
    d = moe.moe_dispatch(x, idx, E)
    off = d["offsets"].cpu().numpy().astype(np.int64)
    counts = np.diff(off)
    del d, idx

    ws_bytes = moe.moe_forward_workspace_size(T, H, I, E, k, x.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=x.dtype, device=dev)

    def step():
        if grouped:
            moe.moe_forward_sigmoid_grouped(x, logits, wg, wu, wd, *gargs,
                                            out=out, workspace=ws, **gopts)
        else:
            moe.moe_forward(x, logits, wg, wu, wd, k, wl["renorm"], out=out,
                            workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    stream = torch.cuda.current_stream(dev)
    nev = _lib.lib()

    def events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for ev in evs:
            ev.record(stream)  # materialise the handles
        return evs

    def install(evs_by_mark):
        h = [None] * 8
        for j, ev in evs_by_mark.items():
            h[j] = ev.cuda_event
        _lib.check(nev.moe_set_timing_events((_lib.ctypes.c_void_p * 8)(*h), 8))

    # Timed region: each recorded mark costs a few microseconds of GPU time,
    # so only the gate+up GEMM (the roofline's kernel) is bracketed here,
    # by the library's marks 4 and 5 on the stream it launches on.
    gu = [events(2) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        install({4: gu[i][0], 5: gu[i][1]})
        step()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    _lib.check(nev.moe_set_timing_events(None, 0))
    g_ms = sum(a.elapsed_time(b) for a, b in gu) / args.steps

    # Per-stage pass (after the timed region, not part of `value`): all 8
    # marks; an interval holding no kernel measures one mark's own cost.
    marks = [events(8) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    for i in range(args.steps):
        install(dict(enumerate(marks[i])))
        step()
    torch.cuda.synchronize(dev)
    _lib.check(nev.moe_set_timing_events(None, 0))
    per_kernel = {name: 0.0 for name in KERNELS}
    for evs in marks:
        for j, name in enumerate(KERNELS):
            per_kernel[name] += evs[j].elapsed_time(evs[j + 1])
    per_kernel = {n: v / args.steps for n, v in per_kernel.items()}  # ms
    # GPU time of each step (with the marks), first kernel start to last end
    step_gpu = sorted(evs[0].elapsed_time(evs[7]) for evs in marks)
    names, per_kernel, alg = fuse_stages(per_kernel, algorithmic(wl, counts),
                                         1.5 * mark_cost_ms(dev))
    stages = {}
    for name in names:
        ms = per_kernel[name]
        st = {"ms": round(ms, 5)}
        a = alg[name]
        if "flop" in a:
            st["tflops"] = round(a["flop"] / (ms * 1e-3) / 1e12, 2)
        st["gbs"] = round(a["bytes"] / (ms * 1e-3) / 1e9, 1)
        stages[name] = st

    ms_step = elapsed / args.steps * 1e3
    g = alg["gateup_gemm"]
    if base == "decode":
        ach = g["bytes"] / (g_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(args.workload + "/gateup_gemm"),
                "kernel": "gateup_gemm"}
    else:
        ach = g["flop"] / (g_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(args.workload + "/gateup_gemm"),
                "kernel": "gateup_gemm"}

    graph = None
    if args.graph:
        # the library enqueues only kernels, so the whole forward captures
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize(dev)
        t1 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize(dev)
        g_el = time.perf_counter() - t1
        graph = {"value": round(T * args.steps / g_el, 1),
                 "ms_per_step": round(g_el / args.steps * 1e3, 4)}
        del g

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    line = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_gpu_ms": {"p50": round(step_gpu[len(step_gpu) // 2], 4),
                        "min": round(step_gpu[0], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl["fmt"] == "bf16" else wl["fmt"],
        "data": "synthetic",
        "config": {"workload": "%s bf16 T=%d H=%d I=%d E=%d top_k=%d "
                               "renormalize=%s%s" % (
                                   base, T, H, I, E, k, wl["renorm"],
                                   " sigmoid groups=%d selected=%d "
                                   "top_two=%s scale=%g bias" % (
                                       wl["groups"], wl["selected_groups"],
                                       wl["group_top_two"], wl["scale"])
                                   if grouped else ""),
                   "T": T, "H": H, "I": I, "E": E, "top_k": k,
                   "touched_experts": alg["touched_experts"],
                   "flop_per_step": 6 * T * k * H * I},
        "tflops_per_step": round(6 * T * k * H * I / (ms_step * 1e-3) / 1e12,
                                 1),
        "roofline": roof,
        "stages": stages,
        "cpu_baseline": cpu,
    }
    if graph is not None:
        line["graph"] = graph
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
