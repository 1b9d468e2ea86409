"""Benchmark of the GRPO loss hot path on one MI355X.

One step = the whole loss with its gradients over one batch of synthetic inputs already
resident in HBM: advantages, row compaction, the forward GEMMs with their online
logsumexp for policy and reference, the KL / advantage epilogue and loss, onehot - softmax
and dX (and dW for the trainable-head workload).

  single-pass (timed for `value`): grpo_advantages + grpo_loss_fwd_bwd, which keeps the
      policy forward's softmax terms per chunk of rows instead of recomputing the logits;
  two-pass (reported as `two_pass`): grpo_advantages + grpo_loss_fwd + grpo_loss_bwd, the
      backward recomputing each chunk's logits.

The roofline is that of the forward kernel, timed with HIP events around each two-pass
grpo_loss_fwd call (one fwd_kernel launch covering both sides, plus the row compaction
and merge, which take well under 0.1% of it).

Prints ONE JSON line.  Default workload: the long-context Llama-3.1-8B shape
(G = 8, L = 20480, H = 4096, V = 128256, bf16, frozen head).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path P]
                  [--no-two-pass] [--no-fp8] [--no-offload] [--no-graph] [--small-chunk ROWS]
                  [--no-cpu-baseline]
                  [--cpu-rows R] [--calibrate-copy-gib X]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GRPO loss fwd+bwd completion tokens/sec; % bf16 MFMA peak; extra GB"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense, published
HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3.1-8b-long-bf16")
    ap.add_argument("--path", choices=["single", "two"], default="single",
                    help="path timed for value; the other one is reported beside it")
    ap.add_argument("--no-two-pass", action="store_true",
                    help="time only the path given by --path")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the single-pass leg with fp8 (e4m3) logits")
    ap.add_argument("--small-chunk", type=int, default=0,
                    help="rows per backward chunk of an extra single-pass leg that trades "
                         "speed for workspace (0: no such leg)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the single-pass leg with the gradients offloaded to host memory")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the single-pass leg replayed from a captured HIP graph")
    ap.add_argument("--no-trace", action="store_true",
                    help="no kernel event brackets (no roofline block)")
    ap.add_argument("--cpu-rows", type=int, default=256, help="oracle rows per sequence")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="run one device-to-device copy of this many GiB first, so a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a known size")
    return ap.parse_args()


# counter summaries under profiles/ are named for the kernel they cover
TRAFFIC_FILES = {"fwd_all": "fwd_kernel_all_rows", "fwd_chunk": "fwd_kernel_chunk",
                 "dx": "dx_kernel", "dw": "dw_kernel", "recompute": "recompute_kernel"}


def measured_traffic(workload, kind):
    """HBM-side bytes per launch of one GEMM kernel from the committed counter summary, or
    None when there is none for this kernel and workload or the kernel source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{TRAFFIC_FILES[kind]}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("kernel_source_sha256", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    src = b"".join(open(os.path.join(ROOT, "grpo_loss_amd", "csrc", f), "rb").read()
                   for f in ("mfma.hip", "common.h"))
    if fields.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"])


def cpu_baseline(wl, inp, adv_host, rows_per_seq):
    """Time the fp64 oracle, as it stands, on a stratified sample of loss rows."""
    import oracle
    from synth.generate import hidden_rows
    mask = inp.mask.numpy()
    rng = np.random.default_rng(1234)
    rows = []
    for s in range(wl.S):
        nz = np.nonzero(mask[s * wl.L:(s + 1) * wl.L])[0] + s * wl.L
        if len(nz):
            rows += sorted(rng.choice(nz, size=min(rows_per_seq, len(nz)), replace=False).tolist())
    rows = np.array(rows, dtype=np.int64)
    xq = hidden_rows(wl, "q", rows)
    xp = hidden_rows(wl, "p", rows)
    t0 = time.perf_counter()
    f = oracle.forward(xq, xp, inp.W, inp.targets.numpy(), mask, adv_host, wl.L, wl.beta,
                       rows=rows)
    oracle.backward(xq, inp.W, inp.targets.numpy(), mask, f, grad_loss=wl.loss_scale,
                    loss_scale=wl.loss_scale, rows=rows)
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas, blas_threads = "unknown", None
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            blas_threads = info[0].get("num_threads")
    except ImportError:
        pass
    return {"value": len(rows) / dt, "unit": "completion tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": _cpu_model(), "blas": blas,
            "blas_threads": blas_threads,
            "sample": f"{len(rows)} loss rows ({rows_per_seq} per sequence, seeded), fp64 "
                      f"forward + backward incl. full-vocabulary logits, {dt:.1f} s"}


def _cpu_model():
    """The host CPU's model name, with its family and model numbers (a virtual machine may
    report only the vendor's brand)."""
    f = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                f.setdefault(k.strip(), v.strip())
            if not line.strip() and f:
                break
    except OSError:
        return "unknown"
    return (f"{f.get('model name', 'unknown')} (family {f.get('cpu family', '?')}, "
            f"model {f.get('model', '?')}, {f.get('vendor_id', '?')})")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the benchmark measures the kernels of one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch

    import grpo_loss_amd as g
    from synth import generate, workload_by_name
    from synth.device import to_device

    wl = workload_by_name(args.workload)
    inp = generate(wl)
    n_tok = int(inp.mask.sum())
    torch.cuda.set_device(0)
    d = to_device(inp)
    del inp.xq, inp.xp  # host copies no longer needed
    dt = d["xq"].dtype
    need_dW = wl.need_dW
    # Kernel timing inside the timed steps: each timed step of the leg reported as `value`
    # has the library bracket every launch of one GEMM kernel with a pair of HIP events of
    # its own, recorded on the stream the kernel runs on; the steps take the kernels in
    # turn, and all events are read after the timed region.
    kinds = {"single": ["fwd_all", "fwd_chunk", "dx"] + (["dw"] if need_dW else []),
             "two": ["fwd_all", "recompute", "dx"] + (["dw"] if need_dW else [])}
    max_launches = -(-wl.N // 256) + 1        # chunks of at least 256 rows
    step_traces = []
    if not args.no_trace:
        for i in range(args.steps):
            k = kinds[args.path][i % len(kinds[args.path])]
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * max_launches)]
            for e in evs:
                e.record()   # creates the HIP event
            step_traces.append(g.KernelTrace(k, evs))
        torch.cuda.synchronize()

    # inputs and outputs first: everything allocated after this point is extra memory
    dX = torch.empty_like(d["xq"])
    dW = torch.empty(wl.V, wl.H, dtype=torch.float32, device="cuda") if need_dW else None
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    grad = torch.full((1,), wl.loss_scale, dtype=torch.float32, device="cuda")
    adv = torch.empty(wl.S, dtype=torch.float32, device="cuda")
    g.grpo_advantages(d["rewards"], wl.eps, out=adv)  # the library's code object loaded
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    base_reserved = torch.cuda.memory_reserved()
    base_free = torch.cuda.mem_get_info()[0]   # hipMemGetInfo: the device's own count
    torch.cuda.reset_peak_memory_stats()
    ws_bytes = g.grpo_workspace_bytes(wl.S, wl.L, wl.H, wl.V, dt, need_dW)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    if args.calibrate_copy_gib > 0:
        # a known-size copy whose source is not cache resident: fill it, stream an
        # unrelated 2 GiB buffer through the caches, then copy
        nb = int(args.calibrate_copy_gib * 2 ** 30)
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        flush = torch.zeros(2 * 2 ** 30, dtype=torch.uint8, device="cuda")
        flush.add_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()

    opts = {"v": None}

    def with_trace(step_no):
        base = opts["v"]
        if step_no is None or not step_traces:
            return base
        o = g.options() if base is None else g.GRPOOptions.from_buffer_copy(base)
        return step_traces[step_no].attach(o)

    def step_two(step_no):
        g.grpo_advantages(d["rewards"], wl.eps, out=adv)
        o = with_trace(step_no)
        f = g.grpo_loss_fwd(d["xq"], d["xp"], d["W"], d["targets"], d["mask"], adv, wl.beta,
                            wl.L, workspace=ws, want_terms=False, opts=o)
        if o is not None and o.trace_kernel == g.TRACE_KERNELS["fwd_all"]:
            o = opts["v"]   # the forward's brackets are taken; the backward has none of it
        g.grpo_loss_bwd(d["xq"], d["W"], d["targets"], d["mask"], f["saved"], wl.L, grad,
                        wl.loss_scale, dW=dW, found_inf=found, workspace=ws, dXq=dX, opts=o)
        return f

    def step_single(step_no):
        g.grpo_advantages(d["rewards"], wl.eps, out=adv)
        return g.grpo_loss_fwd_bwd(d["xq"], d["xp"], d["W"], d["targets"], d["mask"], adv,
                                   wl.beta, wl.L, grad, wl.loss_scale, dW=dW, found_inf=found,
                                   workspace=ws, dXq=dX, want_terms=False,
                                   opts=with_trace(step_no))

    def timed(step, trace=False):
        for _ in range(args.warmup):
            step(None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            f = step(i if trace else None)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3, f

    gemm_eq = 2.0 * n_tok * wl.H * wl.V
    dtn = wl.dtype
    peak = PEAK_TFLOPS[dtn]
    # GEMM-equivalents executed per step: policy and reference forward, dX, dW if trainable,
    # plus the recompute in the two-pass path.  The survey's method count (4 or 5) always
    # includes the recompute, which the single pass does not execute: reported beside,
    # labelled as a recompute-equivalent rate.
    n_exec = {"single": 3 + need_dW, "two": 4 + need_dW}
    n_method = 4 + need_dW
    flops_kind = {("single", "fwd_all"): gemm_eq, ("single", "fwd_chunk"): gemm_eq,
                  ("single", "dx"): gemm_eq, ("single", "dw"): gemm_eq,
                  ("two", "fwd_all"): 2 * gemm_eq, ("two", "recompute"): gemm_eq,
                  ("two", "dx"): gemm_eq, ("two", "dw"): gemm_eq}
    kernel_names = {"fwd_all": {"single": "fwd_kernel<E, E, 1> (reference side, all loss rows)",
                                "two": "fwd_kernel<E, E, 0> (both sides, all loss rows)"},
                    "fwd_chunk": {"single": "fwd_kernel<E, E, 3> (policy side, one chunk, "
                                            "softmax terms kept)"},
                    "recompute": {"two": "recompute_kernel (one chunk)"},
                    "dx": {"single": "dx_kernel (one chunk)", "two": "dx_kernel (one chunk)"},
                    "dw": {"single": "dw_kernel (one chunk)", "two": "dw_kernel (one chunk)"}}
    legs = {}
    kernels = {}
    order = [args.path]
    if not args.no_two_pass:
        order.append("two" if args.path == "single" else "single")
    for path in order:
        step = step_single if path == "single" else step_two
        ms, f = timed(step, trace=bool(step_traces) and path == args.path)
        legs[path] = {"value": n_tok / (ms * 1e-3), "ms_per_step": ms,
                      "mfma_peak_frac": n_exec[path] * gemm_eq / (ms * 1e-3) / (peak * 1e12),
                      "recompute_equiv_frac": n_method * gemm_eq / (ms * 1e-3) / (peak * 1e12),
                      "status": int(f["status"].item()), "found_inf": int(found.item())}
        f = None  # the result holds a reference to the workspace
    per_kind = {}
    for tr in step_traces:
        launches = tr.launch_ms()
        if launches:
            per_kind.setdefault(tr.kernel, []).append(launches)
    names = {v: k for k, v in g.TRACE_KERNELS.items()}
    for kid, steps in per_kind.items():
        k = names[kid]
        n = len(steps[0])
        tot = float(np.mean([np.sum(x) for x in steps]))       # ms per step
        # launches that did work: a chunk past the loss-row count is launched too (the host
        # never reads the count) and exits within microseconds
        nw = float(np.mean([sum(1 for t in x if t > 0.05) for x in steps]))
        kernels[k] = {"kernel": kernel_names[k][args.path], "launches_per_step": n,
                      "working_launches_per_step": nw,
                      "ms_per_step": tot, "launch_ms": tot / nw,
                      "flop_per_launch": flops_kind[(args.path, k)] / nw,
                      "tflops": flops_kind[(args.path, k)] / (tot * 1e-3) / 1e12,
                      "steps_traced": len(steps)}
        kernels[k]["frac"] = kernels[k]["tflops"] / peak
    peak_extra = torch.cuda.max_memory_allocated() - base_mem
    # cross-check against the device: the free memory it lost over the timed legs, and how
    # much of that torch's caching allocator does not account for (anything the library or
    # the runtime took outside torch)
    torch.cuda.synchronize()
    dev_delta = base_free - torch.cuda.mem_get_info()[0]
    untracked = dev_delta - (torch.cuda.memory_reserved() - base_reserved)
    main_leg = legs[args.path]
    out = {
        "metric": METRIC,
        "value": main_leg["value"],
        "unit": "completion tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtn,
        "data": "synthetic",
        "config": {"workload": wl.name, "G": wl.G, "L": wl.L, "H": wl.H, "V": wl.V,
                   "completion_tokens": n_tok, "trainable_head": need_dW,
                   "path": "single-pass" if args.path == "single" else "two-pass"},
        "mfma_peak_frac": main_leg["mfma_peak_frac"],
        "recompute_equiv_frac": main_leg["recompute_equiv_frac"],
        "extra_gib": peak_extra / 2 ** 30,
        "device_free_drop_gib": dev_delta / 2 ** 30,
        "untracked_by_torch_gib": untracked / 2 ** 30,
        "workspace_gib": ws_bytes / 2 ** 30,
        "materialized_logits_gib": 2 * 2 * wl.S * wl.L * wl.V / 2 ** 30,
    }
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        kd = kernels[dom]
        out["roofline"] = {"bound": "mfma", "kernel": kd["kernel"], "achieved": kd["tflops"],
                           "peak": peak, "unit": "TFLOP/s", "frac": kd["frac"],
                           "traffic": measured_traffic(wl.name, dom),
                           "launch_ms": kd["launch_ms"], "flop_per_launch": kd["flop_per_launch"],
                           "launches_per_step": kd["launches_per_step"],
                           "working_launches_per_step": kd["working_launches_per_step"]}
        out["kernels"] = kernels
    other = [p for p in legs if p != args.path]
    if other:
        out["two_pass" if other[0] == "two" else "single_pass"] = legs[other[0]]
    out["status"] = main_leg["status"]
    out["found_inf"] = main_leg["found_inf"]
    if not args.no_graph and args.path == "single":
        # the same single-pass step (advantages and grpo_loss_fwd_bwd) captured once in a
        # HIP graph and replayed: the gaps between its launches (about 800 per headline
        # step, 440 of them the vocabulary split's gated fallbacks) close up.  Reported
        # beside the eager `value`, never as it.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_single(None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fg = step_single(None)

        def step_graph(step_no):
            graph.replay()
            return fg

        ms, f = timed(step_graph)
        out["graph_replay"] = {
            "value": n_tok / (ms * 1e-3), "ms_per_step": ms,
            "step_gain_frac": 1.0 - ms / legs["single"]["ms_per_step"],
            "status": int(f["status"].item())}
        f = fg = None
        del graph
        torch.cuda.synchronize()
    if args.small_chunk and args.path == "single":
        # the same single-pass step with a smaller backward chunk: less workspace, more and
        # smaller launches (reported beside the default, never as `value`)
        oc = g.options(chunk_rows=args.small_chunk)
        del ws
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        wsc_bytes = g.grpo_workspace_bytes(wl.S, wl.L, wl.H, wl.V, dt, need_dW, oc)
        ws = torch.empty(wsc_bytes, dtype=torch.uint8, device="cuda")
        opts["v"] = oc
        ms, f = timed(step_single)
        out[f"chunk_{args.small_chunk}"] = {
            "value": n_tok / (ms * 1e-3), "ms_per_step": ms,
            "recompute_equiv_frac": n_method * gemm_eq / (ms * 1e-3) / (peak * 1e12),
            "extra_gib": (torch.cuda.max_memory_allocated() - base_mem) / 2 ** 30,
            "workspace_gib": wsc_bytes / 2 ** 30, "status": int(f["status"].item())}
        f = None
        opts["v"] = None
    if not args.no_offload and args.path == "single":
        # the single pass with its gradients kept in pinned host memory between forward and
        # backward: each chunk's dX rows are copied out by the copy engines while the next
        # chunks compute, and grpo_grad_restore brings them back (kernels reading host
        # memory over PCIe, which the step waits for).  Reported beside the default, never
        # as `value`.
        del ws
        torch.cuda.empty_cache()
        cs = g.offload_stream()
        dx_host = torch.empty(wl.N, wl.H, dtype=dt, pin_memory=True)
        dw_host = (torch.empty(wl.V, wl.H, dtype=torch.float32, pin_memory=True) if need_dW
                   else None)
        oo = g.options()
        oo.dx_host, oo.copy_stream = dx_host.data_ptr(), cs.cuda_stream
        wso_bytes = g.grpo_workspace_bytes(wl.S, wl.L, wl.H, wl.V, dt, need_dW, oo)
        ws = torch.empty(wso_bytes, dtype=torch.uint8, device="cuda")
        rws = torch.empty(g.grpo_restore_workspace_bytes(wl.N), dtype=torch.uint8,
                          device="cuda")

        def step_offload_fwd(step_no):
            g.grpo_advantages(d["rewards"], wl.eps, out=adv)
            return g.grpo_loss_fwd_bwd(d["xq"], d["xp"], d["W"], d["targets"], d["mask"], adv,
                                       wl.beta, wl.L, grad, wl.loss_scale, dW=dW,
                                       found_inf=found, workspace=ws, want_terms=False,
                                       dx_host=dx_host, dw_host=dw_host, copy_stream=cs)

        def step_offload(step_no):
            f = step_offload_fwd(step_no)
            g.grpo_grad_restore(d["mask"], dx_host, dw_host, None, 1.0, dXq=dX, dW=dW,
                                found_inf=found, workspace=rws)
            return f

        ms_fwd, f = timed(step_offload_fwd)
        ms, f = timed(step_offload)
        single_ms = legs["single"]["ms_per_step"]
        held = wl.N * wl.H * d["xq"].element_size() + (wl.V * wl.H * 4 if need_dW else 0)
        ring = wso_bytes - g.grpo_workspace_bytes(wl.S, wl.L, wl.H, wl.V, dt, need_dW)
        out["offload"] = {
            "value": n_tok / (ms * 1e-3), "ms_per_step": ms,
            "fwd_bwd_ms": ms_fwd, "restore_ms": ms - ms_fwd,
            "step_overhead_frac": ms / single_ms - 1.0,
            "fwd_bwd_overhead_frac": ms_fwd / single_ms - 1.0,
            "held_device_gib_saved": (held - ring) / 2 ** 30,
            "host_gib": held / 2 ** 30, "status": int(f["status"].item()),
            "found_inf": int(found.item())}
        f = None
        del ws, rws, dx_host, dw_host
        torch.cuda.empty_cache()
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    if not args.no_fp8 and dtn != "f32":
        # the same single-pass step with both sides' logits from per-row e4m3 copies (a
        # lower-precision variant, reported beside the 16-bit result, never as `value`)
        o8 = g.options(fp8_logits=True)
        del ws
        torch.cuda.empty_cache()
        ws8_bytes = g.grpo_workspace_bytes(wl.S, wl.L, wl.H, wl.V, dt, need_dW, o8)
        ws = torch.empty(ws8_bytes, dtype=torch.uint8, device="cuda")
        opts["v"] = o8
        ms, f = timed(step_single)
        out["fp8_logits"] = {"value": n_tok / (ms * 1e-3), "ms_per_step": ms,
                             "workspace_gib": ws8_bytes / 2 ** 30,
                             "status": int(f["status"].item())}
    if not args.no_cpu_baseline:
        import oracle
        adv_host = oracle.group_advantages(inp.rewards.numpy(), wl.eps)
        out["cpu_baseline"] = cpu_baseline(wl, inp, adv_host, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
