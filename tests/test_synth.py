"""The seeded input generator: determinism, row regeneration, layout and distributions."""

import dataclasses

import numpy as np
import torch

from synth import WORKLOADS, generate, workload_by_name
from synth.generate import hidden_rows, make_mask, make_rewards, make_targets


def _small(name, **kw):
    wl = workload_by_name(name)
    return dataclasses.replace(wl, **kw)


def test_five_workloads_shapes():
    names = [w.name for w in WORKLOADS]
    assert len(set(names)) == 5
    wl = workload_by_name("llama3.1-8b-long-bf16")
    assert (wl.G, wl.L, wl.H, wl.V, wl.dtype) == (8, 20480, 4096, 128256, "bf16")
    m = make_mask(wl)
    assert m.sum() == 8 * 20224 and m[:, :256].sum() == 0


def test_generation_is_deterministic_and_row_addressable():
    wl = _small("phi4-f16", L=80, H=64, V=300, prefix=8, comp_min=10, comp_max=60)
    a = generate(wl)
    b = generate(wl)
    assert torch.equal(a.xq, b.xq) and torch.equal(a.W, b.W) and torch.equal(a.mask, b.mask)
    assert a.xq.dtype == torch.float16 and a.xq.shape == (wl.N, wl.H)
    rows = np.array([0, 5, 257, wl.N - 1, 300])
    assert torch.equal(hidden_rows(wl, "q", rows), a.xq[torch.from_numpy(rows)])
    assert torch.equal(hidden_rows(wl, "p", rows), a.xp[torch.from_numpy(rows)])
    assert not torch.equal(a.xq, a.xp)


def test_outliers_and_scale():
    wl = _small("phi4-f16", L=512, H=256, V=64, prefix=8, comp_min=10, comp_max=60)
    x = generate(wl, with_weight=False).xq.float()
    frac = (x.abs() == 30).float().mean().item()
    assert 0.0005 < frac < 0.0015
    core = x[x.abs() != 30]
    assert abs(core.std().item() - 1.5) < 0.02


def test_rounding_is_nearest_even():
    wl = _small("qwen2.5-1.5b-bf16", L=16, H=64, V=64, prefix=4, comp_min=4, comp_max=8)
    x = generate(wl).xq
    assert x.dtype == torch.bfloat16
    # every stored value is a bf16 value: low 16 bits of the fp32 pattern are zero
    bits = x.float().numpy().view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_mask_targets_rewards():
    wl = workload_by_name("llama3.1-8b-train-bf16")
    m = make_mask(wl)
    lens = m.sum(1)
    assert np.all((lens >= 512) & (lens <= 3840))
    for s in range(wl.S):   # one contiguous span starting after the prompt
        nz = np.nonzero(m[s])[0]
        assert nz[0] == 256 and nz[-1] == 256 + lens[s] - 1
    y = make_targets(wl)
    assert y.min() >= 0 and y.max() < wl.V
    counts = np.bincount(y.reshape(-1), minlength=4)
    assert counts[0] > counts[1] > counts[2] > counts[3]   # Zipf: rank order
    r = make_rewards(wl)
    assert r.shape == (1, 8, 1) and r.dtype == np.float32 and r.min() >= 0 and r.max() <= 3
    r1 = make_rewards(workload_by_name("tiny-f32"))
    assert set(np.unique(r1)).issubset({0.0, 1.0, 2.0})
