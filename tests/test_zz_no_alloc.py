"""grpo_loss_fwd_noalloc (the forward with the library's fixed per-GPU scratch array in
place of a workspace) against grpo_loss_fwd, through the C ABI: equal outputs bit for bit
(same kernels, same order), on two calls in a row whose second has fewer rows, so the
second call reads a scratch array the first one left filled."""

import dataclasses

import numpy as np
import pytest
import torch

from synth import generate, workload_by_name
from synth.device import to_device

pytestmark = pytest.mark.gpu


def _inputs(name, **kw):
    wl = dataclasses.replace(workload_by_name(name), **kw)
    return wl, to_device(generate(wl))


def _host(out):
    return {k: out[k].cpu().numpy() for k in ("loss", "saved", "logp", "ref_logp", "kl",
                                               "status")}


def _compare(a, b, tag):
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (tag, k)


@pytest.mark.parametrize("name,big,small", [
    ("qwen2.5-1.5b-bf16", dict(G=8, L=512, prefix=64, comp_min=64, comp_max=448),
     dict(G=4, L=96, prefix=16, comp_min=8, comp_max=80)),
    ("phi4-f16", dict(G=4, L=384, prefix=32, comp_min=64, comp_max=352),
     dict(G=2, L=80, prefix=16, comp_min=16, comp_max=64)),
    ("tiny-f32", dict(), dict(G=2, L=40, prefix=8, comp_min=8, comp_max=32)),
])
def test_noalloc_forward_matches_workspace_forward(name, big, small):
    import grpo_loss_amd as g
    cases = [_inputs(name, **big), _inputs(name, **small)]
    print(f"[no-alloc] {name}: N = {[w.N for w, _ in cases]}", flush=True)
    got = []
    for wl, d in cases:  # two no-alloc calls in a row, the second smaller
        adv = g.grpo_advantages(d["rewards"], wl.eps)
        got.append((adv, g.grpo_loss_fwd_noalloc(d["xq"], d["xp"], d["W"], d["targets"],
                                                 d["mask"], adv, wl.beta, wl.L)))
    torch.cuda.synchronize()
    got = [_host(o) for _, o in got]
    for (wl, d), nb in zip(cases, got):
        adv = g.grpo_advantages(d["rewards"], wl.eps)
        ref = g.grpo_loss_fwd(d["xq"], d["xp"], d["W"], d["targets"], d["mask"], adv, wl.beta,
                              wl.L)
        torch.cuda.synchronize()
        ref = _host(ref)
        assert int(ref["status"][0]) == 0 and np.isfinite(ref["loss"][0])
        _compare(nb, ref, (name, wl.N))


def test_noalloc_rejects_what_does_not_fit():
    """The long-context forward needs more than the fixed array: GRPO_ERR_SCRATCH, and
    nothing is enqueued (the pointers are never dereferenced)."""
    import grpo_loss_amd as g
    lib = g.load_library()
    import ctypes
    p = ctypes.c_void_p(256)
    rc = lib.grpo_loss_fwd_noalloc(p, p, p, 1, p, p, p, 8, 20480, 4096, 128256,
                                   ctypes.c_float(0.04), p, p, None, None, None, p, None, None)
    assert rc == -9
