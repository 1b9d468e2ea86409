"""Benchmark of the GRPO loss hot path on one MI355X.

One step = grpo_advantages + grpo_loss_fwd + grpo_loss_bwd over one batch of synthetic
inputs already resident in HBM: advantages, row compaction, the fused forward GEMM with
its online logsumexp for policy and reference, the KL / advantage epilogue and loss,
the backward recompute of onehot - softmax, dX (and dW for the trainable-head workload).

Prints ONE JSON line.  Default workload: the long-context Llama-3.1-8B shape
(G = 8, L = 20480, H = 4096, V = 128256, bf16, frozen head).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--cpu-rows R] [--calibrate-copy-gib X]
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=256, help="oracle rows per sequence")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="run one device-to-device copy of this many GiB first, so a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a known size")
    return ap.parse_args()


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
    return {"value": len(rows) / dt, "unit": "completion tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(rows)} loss rows ({rows_per_seq} per sequence, seeded), fp64 "
                      f"forward + backward incl. full-vocabulary logits, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this build measures the single-GPU kernel path)", file=sys.stderr)
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
    # inputs and outputs first: everything allocated after this point is extra memory
    dX = torch.empty_like(d["xq"])
    dW = torch.empty(wl.V, wl.H, dtype=torch.float32, device="cuda") if need_dW else None
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    grad = torch.full((1,), wl.loss_scale, dtype=torch.float32, device="cuda")
    adv = torch.empty(wl.S, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
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

    ev = []

    def step(record):
        g.grpo_advantages(d["rewards"], wl.eps, out=adv)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        f = g.grpo_loss_fwd(d["xq"], d["xp"], d["W"], d["targets"], d["mask"], adv, wl.beta,
                            wl.L, workspace=ws, want_terms=False)
        e1.record()
        g.grpo_loss_bwd(d["xq"], d["W"], d["targets"], d["mask"], f["saved"], wl.L, grad,
                        wl.loss_scale, dW=dW, found_inf=found, workspace=ws, dXq=dX)
        if record:
            ev.append((e0, e1))
        return f

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        f = step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    peak_extra = torch.cuda.max_memory_allocated() - base_mem
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms = elapsed / args.steps * 1e3
    gemm_eq = 2.0 * n_tok * wl.H * wl.V
    method_flops = (5 if need_dW else 4) * gemm_eq
    dtn = wl.dtype
    peak = PEAK_TFLOPS[dtn]
    fwd_tflops = 2 * gemm_eq / (fwd_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": n_tok / (ms * 1e-3),
        "unit": "completion tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtn,
        "data": "synthetic",
        "config": {"workload": wl.name, "G": wl.G, "L": wl.L, "H": wl.H, "V": wl.V,
                   "completion_tokens": n_tok, "trainable_head": need_dW},
        "mfma_peak_frac": method_flops / (ms * 1e-3) / (peak * 1e12),
        "extra_gib": peak_extra / 2 ** 30,
        "workspace_gib": ws_bytes / 2 ** 30,
        "materialized_logits_gib": 2 * 2 * wl.S * wl.L * wl.V / 2 ** 30,
        "roofline": {"bound": "mfma", "kernel": "fwd_kernel (policy + reference logits, "
                                                  "online logsumexp)",
                     "achieved": fwd_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": fwd_tflops / peak, "traffic": None,
                     "fwd_call_ms": fwd_ms},
        "status": int(f["status"].item()),
        "found_inf": int(found.item()),
    }
    if not args.no_cpu_baseline:
        import oracle
        adv_host = oracle.group_advantages(inp.rewards.numpy(), wl.eps)
        out["cpu_baseline"] = cpu_baseline(wl, inp, adv_host, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
