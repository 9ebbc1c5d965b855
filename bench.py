"""Benchmark of the LaCT fast-weight layer forward (update + apply) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--backward]

One step = one whole layer forward over the workload's sequence (every chunk:
forward products, SwiGLU backward epilogue, weight-gradient contraction,
optimiser + renorm, apply), inputs resident in HBM.  The default workload is
the largest language configuration, the 3B-LM-shaped layer: 6 heads,
d = dh = 512, 32,768 tokens in chunks of 4,096, bf16 q/k/v, fp32 fast
weights, Muon (5 Newton-Schulz steps) + row renormalisation,
apply-then-update.  Prints one JSON line.

Every step starts from the same initial state: the fast weights (and the
momentum buffer) are restored by device copies between steps, outside the
per-step HIP events that time the layer calls.

--backward measures the layer's backward pass instead (lact_layer_backward:
gradients of q, k, v, lr, beta and the initial state for a seeded output
cotangent; one step = one whole backward call, which replays the forward
state trajectory and sweeps the chunks in reverse).  Its products run as
bf16 MFMA passes over fp32 operands split into bf16 planes, so they are
priced against the bf16 peak, algorithmically and (from committed counters)
as executed MFMA work.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16 = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12         # bytes/s
RIDGE = PEAK_BF16 / PEAK_HBM   # flop per byte where the bf16 MFMA and HBM roofs meet


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload id 1..10 (default: the 3B LM layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work to sample")
    ap.add_argument("--backward", action="store_true", help="measure the layer's backward pass")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain device copy of known size (PMC counter calibration)")
    return ap.parse_args()


def kernel_flops(wl, lact):
    """Algorithmic FLOPs per step, per kernel class."""
    from test_layers_amd import workloads as W
    D, Dh, n = wl.D, wl.dh, wl.n_inst
    upd = sum(b - a for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags) if f & W.UPDATE)
    app = sum(b - a for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags) if f & W.APPLY)
    n_upd = sum(1 for f in wl.flags if f & W.UPDATE)
    return {
        lact.K_UPD: 6.0 * upd * D * Dh * n,                 # K W1^T, K W3^T, V W2
        lact.K_APP: 4.0 * app * D * Dh * n,                 # Q W1^T, Q W3^T
        lact.K_OUT: 2.0 * app * D * Dh * n,                 # Hq W2^T
        lact.K_DW: 6.0 * upd * D * Dh * n,                  # three contractions over tokens
        lact.K_OPT: 0.0,
        lact.K_NS: (30.0 * D ** 3 * 3 * n * n_upd) if wl.opt in (W.OPT_MUON, W.OPT_MUON_MOMENTUM) else 0.0,
        lact.K_SNAP: 0.0,
        lact.K_PREP: 0.0,
        lact.K_NSRED: 0.0,
    }


def kernel_bytes(wl, lact, fused):
    """Algorithmic HBM bytes per step, per kernel class: what each kernel must
    read or write at least -- inputs read once, layer outputs and the state
    written once, the weights a product reads once per launch -- with the
    intermediates that a fused path keeps on chip (update terms, gated
    hidden, split partials, Newton-Schulz operands) counted as zero.
    `fused` names the classes whose work runs inside another class's kernel
    ('app_in_upd', 'dw_in_upd', 'out_in_app')."""
    from test_layers_amd import workloads as W
    D, Dh, n = wl.D, wl.dh, wl.n_inst
    io = 2 if wl.io_dtype == W.DTYPE_BF16 else 4
    snap = 2 if wl.io_dtype == W.DTYPE_BF16 else 4
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    upd = sum(b - a for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags) if f & W.UPDATE)
    app = sum(b - a for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags) if f & W.APPLY)
    n_upd = sum(1 for f in wl.flags if f & W.UPDATE)
    n_app = sum(1 for f in wl.flags if f & W.APPLY)
    mat = D * Dh
    b = {c: 0.0 for c in lact.K_NAMES}
    b[lact.K_UPD] = n * upd * (2 * D * io + 12 + (4 if mom else 0)) + n_upd * n * 3 * mat * snap
    if "app_in_upd" in fused:
        b[lact.K_UPD] += n * app * D * io
    b[lact.K_APP] = n * app * D * io + n_app * n * 2 * mat * snap
    b[lact.K_OUT] = n * app * D * io + n_app * n * mat * snap
    if "out_in_app" in fused:
        b[lact.K_APP] += b[lact.K_OUT]
    b[lact.K_DW] = n * upd * 2 * D * io
    b[lact.K_OPT] = n_upd * n * 3 * mat * 4 * (4 if wl.opt == W.OPT_MOMENTUM else 2)
    b[lact.K_SNAP] = n * 3 * mat * 4
    b[lact.K_PREP] = (n * app * D * io * 2 + n * upd * D * io * 2) if wl.layer_qk_prep else 0.0
    # the Newton-Schulz input reduction: the momentum state read and written
    # (its partials and outputs are intermediates)
    b[lact.K_NSRED] = n_upd * n * 3 * mat * 4 * 2 if wl.opt == W.OPT_MUON_MOMENTUM else 0.0
    return b


def ns_flops_per_matrix(D, Dh, iters=5):
    """Newton-Schulz forward per matrix: per iteration X X^T (2 m^2 k), A A
    (2 m^3), B X (2 m^2 k), with m = min(d, dh), k = max(d, dh)."""
    m, k = min(D, Dh), max(D, Dh)
    return iters * (4.0 * m * m * k + 2.0 * m ** 3)


def backward_kernel_flops(wl, lact):
    """FLOPs per backward call, per kernel class.  The call replays the
    forward state trajectory (update chunks only: update forward, the
    contractions and Newton-Schulz run on the forward's kernels) and then
    runs the reverse sweep on its own products:
      per update token 36 d dh (recomputed k W1^T, k W3^T, v W2 and the three
      direction contractions, 12; k gU1^T, k gU3^T, v gU2, 6; dk and dv from
      the update terms, 6, and through W, 6; dW contractions, 6),
      per apply token 16 d dh (q W1^T, q W3^T, dO W2, 6; three dW
      contractions, 6; dq, 4),
      Newton-Schulz per matrix and update: its forward again plus, per
      iteration, gX X^T, gP A, A gP, P g, Q X (6 m^2 k + 4 m^3)."""
    from test_layers_amd import workloads as W
    D, Dh, n = wl.D, wl.dh, wl.n_inst
    upd = sum(b - a for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags) if f & W.UPDATE)
    app = sum(b - a for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags) if f & W.APPLY)
    n_upd = sum(1 for f in wl.flags if f & W.UPDATE)
    ns = wl.opt in (W.OPT_MUON, W.OPT_MUON_MOMENTUM)
    m, k = min(D, Dh), max(D, Dh)
    f = {c: 0.0 for c in lact.K_NAMES}
    f[lact.K_UPD] = 6.0 * upd * D * Dh * n
    f[lact.K_DW] = 6.0 * upd * D * Dh * n
    f[lact.K_NS] = ns_flops_per_matrix(D, Dh) * 3 * n * n_upd if ns else 0.0
    f[lact.K_BWD_GEMM] = (36.0 * upd + 16.0 * app) * D * Dh * n
    if ns:
        f[lact.K_BWD_GEMM] += 3 * n * n_upd * (ns_flops_per_matrix(D, Dh) + 5 * (6.0 * m * m * k + 4.0 * m ** 3))
    return f


def host_info():
    """The host the oracle is timed on: CPU model, logical CPUs, the CPUs this
    process may run on, and the BLAS library numpy's threads come from."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")} for d in threadpool_info()]
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas}


def cpu_baseline_backward(wl, inp, dO, budget):
    """The backward oracle as it stands, on a bounded sample (whole instances
    over the whole sequence until about `budget` seconds of work)."""
    from oracle import lact_backward as OB
    from test_layers_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < budget:
        i = done % wl.n_inst
        OB.backward_instance(inp.q[i], inp.k[i], inp.v[i], inp.lr[i], inp.beta[i] if mom else None,
                             inp.W1[i], inp.W2[i], inp.W3[i], wl.bounds, wl.flags, wl.order, wl.opt, dO[i],
                             qk_prep=wl.layer_qk_prep, oz=inp.oz[i] if wl.out_scale else None)
        done += 1
    dt = time.perf_counter() - t0
    tokens = wl.tokens * done / wl.n_inst
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} instance backward passes (heads, cycling over the {wl.n_inst} of the workload), "
                      f"whole {wl.L}-token sequence each, {dt:.1f} s, numpy fp64", "host": host_info()}


def cpu_baseline(wl, inp, budget):
    """The oracle as it stands, on a bounded sample of the same workload:
    whole instances (heads), each over the whole sequence, until about
    `budget` seconds of CPU work have been done."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < budget:
        i = done % wl.n_inst
        O.forward_instance(inp.q[i], inp.k[i], inp.v[i], inp.lr[i],
                           None if inp.beta is None else inp.beta[i],
                           inp.W1[i], inp.W2[i], inp.W3[i], wl.bounds, wl.flags, wl.order, wl.opt,
                           qk_prep=wl.layer_qk_prep, oz=inp.oz[i] if wl.out_scale else None)
        done += 1
    dt = time.perf_counter() - t0
    tokens = wl.tokens * done / wl.n_inst
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} instance passes (heads, cycling over the {wl.n_inst} of the workload), "
                      f"whole {wl.L}-token sequence each, {dt:.1f} s, numpy fp64", "host": host_info()}


SRC_FILES = ("lact.hip", "lact_device.hpp", "lact_kernels.hpp", "lact_direct.hpp", "lact_planes.hpp", "lact_backward.hpp",
             "lact_backward_host.hpp")


def source_sha():
    """Hash of the kernel sources; counter-derived traffic is reported only
    for the exact sources the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    here = os.path.dirname(os.path.abspath(__file__))
    for f in SRC_FILES:
        with open(os.path.join(here, "test_layers_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def pmc_entry(kernel, workload, fname="pmc_traffic.json"):
    """The committed counter summary of one kernel class on one workload
    (HBM bytes from FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's
    reading; MFMA work where recorded), or None when absent or taken on
    other sources."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", fname)
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    w = t.get("workloads", {}).get(workload)
    if not w or w.get("source_sha") != source_sha():
        return None
    return w.get("kernels", {}).get(kernel)


def pmc_traffic(kernel, workload, fname="pmc_traffic.json"):
    k = pmc_entry(kernel, workload, fname)
    if not k:
        return None
    return k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from test_layers_amd import lact
    from test_layers_amd import workloads as W

    if args.copy_calib:
        # plain copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE counters
        nbytes = 1 << 30
        a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": nbytes, "launches": 5}))
        return

    wl = W.WORKLOADS[args.config]
    inp = W.generate(wl, threads=16)
    dev = lambda x: None if x is None else (
        torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() if x.dtype == np.uint16
        else torch.from_numpy(np.ascontiguousarray(x)).cuda())
    q, k, v, lr, beta = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.lr), dev(inp.beta)
    oz = dev(inp.oz) if wl.out_scale else None
    Ws = [dev(inp.W1), dev(inp.W2), dev(inp.W3)]
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    bounds, flags = list(wl.bounds), list(wl.flags)
    stream = torch.cuda.current_stream()

    if args.backward:
        # seeded output cotangent in the io dtype
        rng = np.random.default_rng([0, 77])
        dO_np = rng.standard_normal((wl.n_inst, wl.L, wl.D)).astype(np.float32)
        if wl.io_dtype == W.DTYPE_BF16:
            dO_np = W.f32_to_bf16_bits(dO_np)
        dO = dev(dO_np)
        p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, 3, dh=wl.dh, qk_prep=wl.layer_qk_prep)
        ws = torch.empty(lact.backward_workspace_size(p, wl.L, 0, wl.order, bounds, flags), dtype=torch.uint8,
                         device="cuda")
        box = {"out": None}

        def step():
            box["out"] = lact.layer_backward(q, k, v, lr, beta if mom else None, *Ws, *Ms, dO=dO, order=wl.order,
                                             opt=wl.opt, bounds=bounds, flags=flags, qk_prep=wl.layer_qk_prep,
                                             oz=oz, out=box["out"], workspace=ws, stream=stream)
        kf = backward_kernel_flops(wl, lact)
        peak, peak_name = PEAK_BF16, "bf16"
        metric = ("LaCT layer backward tokens/sec (gradients of q, k, v, lr, beta and the initial state; "
                  "fp32-grade), 1xMI355X")
        dtype = "f32"
    else:
        o = torch.zeros_like(q)
        W0 = [w.clone() for w in Ws]
        M0 = [None if m is None else m.clone() for m in Ms]
        p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, wl.rec_planes, dh=wl.dh,
                         qk_prep=wl.layer_qk_prep)
        ws = torch.empty(lact.workspace_size(p, wl.L, 0, wl.order, bounds, flags), dtype=torch.uint8,
                         device="cuda")

        def step():
            lact.layer_forward(q, k, v, lr, beta, *Ws, *Ms, o, order=wl.order, opt=wl.opt,
                               bounds=bounds, flags=flags, rec_planes=wl.rec_planes,
                               qk_prep=wl.layer_qk_prep, oz=oz, workspace=ws, stream=stream)
        kf = kernel_flops(wl, lact)
        peak, peak_name = PEAK_BF16, "bf16"
        metric = "LaCT layer tokens/sec (update+apply) and % bf16 MFMA peak, 1xMI355X"
        dtype = "bf16" if wl.io_dtype == W.DTYPE_BF16 else "f32"

    def restore():
        # the forward overwrites the state in place: every step starts from W0 (M0)
        if not args.backward:
            for w, w0 in zip(Ws, W0):
                w.copy_(w0)
            for m, m0 in zip(Ms, M0):
                if m is not None:
                    m.copy_(m0)

    for _ in range(args.warmup):
        restore()
        step()
    # one pair of events on the layer's stream around each layer call (no
    # host sync inside the timed loop); the state restores sit between them
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        restore()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [starts[i].elapsed_time(ends[i]) for i in range(args.steps)]
    ms_per_step = sum(step_ms) / args.steps
    step_ms.sort()
    tokens = wl.tokens
    value = tokens / (ms_per_step * 1e-3)
    flops = sum(kf.values()) if args.backward else W.algorithmic_flops(wl)["total"]

    # per-kernel HIP-event timing over the same number of steps
    for kc in lact.K_NAMES:
        lact.timing_enable(kc, True)
    for _ in range(args.steps):
        restore()
        step()
    torch.cuda.synchronize()
    per = {}
    for kc, name in lact.K_NAMES.items():
        ms, nl = lact.timing_read(kc)
        lact.timing_enable(kc, False)
        if nl:
            per[name] = {"ms_per_step": ms / args.steps, "launches_per_step": nl / args.steps,
                         "avg_launch_us": ms / nl * 1e3, "kc": kc}
    fused = set()
    if "apply_out" not in per and "apply_fwd" in per:
        # the fused apply kernel also runs the output product
        kf[lact.K_APP] += kf[lact.K_OUT]
        fused.add("out_in_app")
    elif "apply_fwd" not in per and "apply_out" in per:
        # every apply-then-update chunk's query products ran in its update
        # forward tile (plain bf16, the same snapshot); the workloads here
        # fuse all of their applies or none
        kf[lact.K_UPD] += kf[lact.K_APP]
        fused.add("app_in_upd")
    if "dw" not in per and "update_fwd" in per:
        # the fused update kernel also runs the weight-gradient contraction
        kf[lact.K_UPD] += kf[lact.K_DW]
        fused.add("dw_in_upd")
    kb = kernel_bytes(wl, lact, fused)
    traffic_file = "pmc_traffic_backward.json" if args.backward else "pmc_traffic.json"
    dom = max(per.items(), key=lambda kv: kv[1]["ms_per_step"])
    dname, d = dom
    fl = kf.get(d["kc"], 0.0)
    nbytes = kb.get(d["kc"], 0.0)
    # the roof that bounds the kernel: MFMA when its algorithmic arithmetic
    # intensity reaches the ridge point, else HBM
    intensity = fl / nbytes if nbytes > 0 else float("inf")
    t_launch = d["avg_launch_us"] * 1e-6
    if fl > 0 and intensity >= RIDGE:
        per_launch = fl / d["launches_per_step"]
        achieved = per_launch / t_launch
        roof = {"kernel": dname, "bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak, "traffic": pmc_traffic(dname, wl.name, traffic_file),
                "flops_per_launch": per_launch, "avg_launch_us": d["avg_launch_us"], "peak_dtype": peak_name,
                "intensity_flop_per_byte": intensity if nbytes > 0 else None}
        ent = pmc_entry(dname, wl.name, traffic_file)
        if ent and ent.get("mfma_flops_per_launch"):
            # MFMA work the kernel executes (plane passes, padding and
            # symmetric tiles included), from the committed counters
            roof["executed_flops_per_launch"] = ent["mfma_flops_per_launch"]
            roof["executed_frac"] = ent["mfma_flops_per_launch"] / t_launch / peak
    else:
        per_launch = nbytes / d["launches_per_step"]
        achieved = per_launch / t_launch
        roof = {"kernel": dname, "bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": achieved / PEAK_HBM, "traffic": pmc_traffic(dname, wl.name, traffic_file),
                "bytes_per_launch": per_launch, "avg_launch_us": d["avg_launch_us"],
                "intensity_flop_per_byte": intensity,
                "flops_per_launch": fl / d["launches_per_step"]}
    kernels = {k: {kk: round(vv, 4) for kk, vv in v.items() if kk != "kc"} for k, v in per.items()}

    out = {
        "metric": metric,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0], "max": step_ms[-1]},
        "timing": ("HIP events around each layer call on its stream; mean over the timed steps"
                   + ("" if args.backward else "; W0 (and M0) restored by device copies between steps, "
                      "outside the events")),
        "wall_ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded generator; no dataset, random-init fast weights)",
        "config": {"workload": wl.name, "n_inst": wl.n_inst, "d": wl.D, "dh": wl.dh, "seq_len": wl.L,
                   "max_chunk": wl.max_chunk, "n_chunks": wl.n_chunks,
                   "opt": ["gd", "momentum", "muon", "muon_momentum"][wl.opt],
                   "order": ["apply_then_update", "update_then_apply"][wl.order],
                   "rec_planes": 3 if args.backward else wl.rec_planes, "layer_qk_prep": wl.layer_qk_prep,
                   "output_scale": wl.out_scale, "pass": "backward" if args.backward else "forward",
                   "global_batch": 1},
        "algorithmic_tflop_per_step": flops / 1e12,
        "roofline": roof,
        "kernels": kernels,
    }
    out["layer_frac_bf16_peak"] = flops / (ms_per_step * 1e-3) / PEAK_BF16
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_backward(wl, inp, dO_np, args.cpu_budget) if args.backward
                               else cpu_baseline(wl, inp, args.cpu_budget))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
