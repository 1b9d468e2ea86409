"""Seeded generation of the loss inputs.

Every tensor is drawn with NumPy's Philox generator.  Hidden-state rows and
vocabulary rows are drawn in fixed blocks of ``ROW_BLOCK`` rows, each block from
its own key, so any subset of rows can be regenerated on its own (the oracle
uses that to check sampled rows of the large workloads without holding every
input twice).  Values are drawn in float32 and rounded to the storage type with
round-to-nearest-even.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np
import torch

from .workloads import Workload

ROW_BLOCK = 256

_XQ, _XP, _W, _MASK, _TARGET, _REWARD = 1, 2, 3, 4, 5, 6

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _rng(seed: int, tensor_id: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[seed, (tensor_id << 40) | block]))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _dense_block(wl: Workload, tensor_id: int, block: int, rows: int, cols: int,
                 std: float) -> np.ndarray:
    g = _rng(wl.seed, tensor_id, block)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(std)
    if tensor_id in (_XQ, _XP) and wl.outlier_p > 0.0:
        hit = g.random((rows, cols), dtype=np.float32) < np.float32(wl.outlier_p)
        sign = g.integers(0, 2, size=(rows, cols), dtype=np.int8)
        x[hit] = np.where(sign[hit] == 1, np.float32(wl.outlier_val),
                          np.float32(-wl.outlier_val))
    return x


def _matrix_rows(wl: Workload, tensor_id: int, nrows: int, cols: int, std: float,
                 rows: np.ndarray | None) -> torch.Tensor:
    """Rows of a [nrows, cols] matrix in storage dtype; all rows if ``rows`` is None."""
    dt = _TORCH_DTYPE[wl.dtype]
    if rows is None:
        nblk = (nrows + ROW_BLOCK - 1) // ROW_BLOCK
        out = torch.empty((nrows, cols), dtype=dt)

        def work(b):
            r0 = b * ROW_BLOCK
            r1 = min(nrows, r0 + ROW_BLOCK)
            out[r0:r1] = torch.from_numpy(_dense_block(wl, tensor_id, b, r1 - r0, cols, std)).to(dt)

        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = torch.empty((len(rows), cols), dtype=dt)
    for b in np.unique(rows // ROW_BLOCK):
        r0 = int(b) * ROW_BLOCK
        r1 = min(nrows, r0 + ROW_BLOCK)
        blk = torch.from_numpy(_dense_block(wl, tensor_id, int(b), r1 - r0, cols, std)).to(dt)
        sel = np.nonzero(rows // ROW_BLOCK == b)[0]
        out[torch.from_numpy(sel)] = blk[torch.from_numpy(rows[sel] - r0)]
    return out


def make_mask(wl: Workload) -> np.ndarray:
    """uint8 [S, L]: 1 on each sequence's completion span, 0 on prompt and padding."""
    g = _rng(wl.seed, _MASK)
    lengths = g.integers(wl.comp_min, wl.comp_max + 1, size=wl.S)
    m = np.zeros((wl.S, wl.L), dtype=np.uint8)
    for s, n in enumerate(lengths):
        end = min(wl.L, wl.prefix + int(n))
        m[s, wl.prefix:end] = 1
    return m


def make_targets(wl: Workload) -> np.ndarray:
    """int64 [S, L] token ids in [0, V), for every position (masked ones too)."""
    g = _rng(wl.seed, _TARGET)
    if wl.targets == "uniform":
        return g.integers(0, wl.V, size=(wl.S, wl.L), dtype=np.int64)
    if wl.targets == "zipf":
        w = np.arange(1, wl.V + 1, dtype=np.float64) ** (-wl.zipf_s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = g.random(size=(wl.S, wl.L))
        y = np.searchsorted(cdf, u, side="right")
        return np.minimum(y, wl.V - 1).astype(np.int64)
    raise ValueError(wl.targets)


def make_rewards(wl: Workload) -> np.ndarray:
    """float32 [B, G, K] scores from K reward functions."""
    g = _rng(wl.seed, _REWARD)
    shape = (wl.B, wl.G, wl.K)
    if wl.rewards == "int012":
        r = g.integers(0, 3, size=shape).astype(np.float64)
    elif wl.rewards == "uniform03":
        r = g.uniform(0.0, 3.0, size=shape)
    elif wl.rewards == "bern_noise":
        r = (g.random(size=shape) < 0.3).astype(np.float64) + g.normal(0.0, np.sqrt(0.1), size=shape)
    else:
        raise ValueError(wl.rewards)
    return r.astype(np.float32)


@dataclass
class Inputs:
    wl: Workload
    xq: torch.Tensor        # [N, H] storage dtype, row t = (sequence t // L, position t % L)
    xp: torch.Tensor        # [N, H]
    W: torch.Tensor         # [V, H]
    targets: torch.Tensor   # int64 [N]
    mask: torch.Tensor      # uint8 [N]
    rewards: torch.Tensor   # float32 [B, G, K]


def generate(wl: Workload, with_hidden: bool = True, with_weight: bool = True) -> Inputs:
    """All inputs of a workload as CPU tensors (hidden states / weight optional)."""
    xq = _matrix_rows(wl, _XQ, wl.N, wl.H, wl.x_std, None) if with_hidden else None
    xp = _matrix_rows(wl, _XP, wl.N, wl.H, wl.x_std, None) if with_hidden else None
    W = _matrix_rows(wl, _W, wl.V, wl.H, wl.w_std, None) if with_weight else None
    return Inputs(wl, xq, xp, W,
                  torch.from_numpy(make_targets(wl).reshape(-1)),
                  torch.from_numpy(make_mask(wl).reshape(-1)),
                  torch.from_numpy(make_rewards(wl)))


def hidden_rows(wl: Workload, which: str, rows) -> torch.Tensor:
    """Selected rows of X_q (``which == "q"``) or X_p (``"p"``), storage dtype."""
    tid = {"q": _XQ, "p": _XP}[which]
    return _matrix_rows(wl, tid, wl.N, wl.H, wl.x_std, np.asarray(rows))


def weight(wl: Workload) -> torch.Tensor:
    return _matrix_rows(wl, _W, wl.V, wl.H, wl.w_std, None)


def materialized_logits_bytes(G: int, L: int, V: int, elem_bytes: int = 2,
                              copies: int = 2) -> int:
    """Bytes of the (G, L, V) logits a plain implementation builds for policy and
    reference: copies x elem_bytes x G x L x V [Long-context GRPO, §2]."""
    return copies * elem_bytes * G * L * V
