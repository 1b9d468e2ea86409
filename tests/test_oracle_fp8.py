"""Pins of the oracle's fp8-logits variant (an e4m3 lm_head path; [Long-context GRPO, §3]
notes that naive fp8 breaks, hence the per-row scales).

* e4m3 rounding and byte codes against torch's float8_e4m3fn cast;
* per-row quantisation: the row maximum maps to 448, the error bound of 3 fraction bits;
* inputs already on a scaled e4m3 grid quantise losslessly, so the fp8 loss and
  gradients equal the default ones;
* the fp8 forward's log-probs against torch: per-row scales, torch's fp8 cast, a
  float64 matmul and torch's log_softmax;
* the fp8 backward against torch's cross-entropy gradient of the fp8 logits, carried to
  X through the original W (beta = 0, A = 1).

``test_planted_fp8_mistakes_are_caught`` plants mistakes into this code of the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.grpo_oracle as og

BETA = 0.04
V8 = oracle.Variant(fp8_logits=True)


def _values(seed, n=20000):
    g = np.random.default_rng(seed)
    mag = 2.0 ** g.uniform(-12, np.log2(448.0), size=n)
    v = (mag * g.choice([-1.0, 1.0], size=n)).astype(np.float32)
    # exact ties between neighbours in both ranges, and the range ends
    ties = np.array([1.0 + 1 / 16, 1.0 + 3 / 16, 2 ** -7 + 2 ** -10, 3 * 2 ** -10, 448.0,
                     -448.0, 2 ** -6, 2 ** -9, 2 ** -10, 0.0, -0.0, -2 ** -11], np.float32)
    return np.concatenate([v, ties])


def pin_e4m3_round_matches_torch():
    for seed in (1, 2):
        v = _values(seed)
        t8 = torch.from_numpy(v).to(torch.float8_e4m3fn)
        ref = t8.to(torch.float64).numpy()
        got = oracle.e4m3_round(v)
        assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:5]
        assert np.array_equal(oracle.e4m3_codes(got), t8.view(torch.uint8).numpy())


def _case(seed, S=2, L=6, H=32, V=40):
    g = np.random.default_rng(seed)
    N = S * L
    xq = g.standard_normal((N, H)).astype(np.float32)
    xp = (xq + 0.3 * g.standard_normal((N, H))).astype(np.float32)
    W = (0.3 * g.standard_normal((V, H))).astype(np.float32)
    y = g.integers(0, V, size=N)
    m = (g.random(N) < 0.8).astype(np.int64)
    m[0] = 1
    adv = g.standard_normal(S).astype(np.float32)
    return xq, xp, W, y, m, adv, L


def pin_quantize_rows_bounds():
    xq, _, W, *_ = _case(3)
    for x in (xq, W):
        q, codes, s = oracle.quantize_e4m3_rows(x)
        assert np.all(np.abs(q).max(axis=1) == 448.0)
        xh = q * s.astype(np.float64)[:, None]
        err = np.abs(xh - x)
        # 3 fraction bits: half a step is 2^-4 relative for normals, 2^-10 s below 2^-6 s
        assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s[:, None]) * 1.0001)
        assert codes.dtype == np.uint8 and codes.shape == x.shape


def _grid_case(seed, S=2, L=5, H=16, V=24):
    """Rows of e4m3 values times a power of two, each row's maximum exactly 448 * 2^k."""
    g = np.random.default_rng(seed)
    grid = np.unique(np.abs(oracle.e4m3_round(g.uniform(-448, 448, 4000))))

    def rows(n, k):
        r = g.choice(grid, size=(n, H)) * g.choice([-1.0, 1.0], size=(n, H))
        r[:, 0] = 448.0
        return (r * 2.0 ** k[:, None]).astype(np.float32)
    N = S * L
    xq = rows(N, g.integers(-9, -5, size=N))
    xp = rows(N, g.integers(-9, -5, size=N))
    W = rows(V, g.integers(-11, -8, size=V))
    y = g.integers(0, V, size=N)
    m = (g.random(N) < 0.8).astype(np.int64)
    m[0] = 1
    adv = g.standard_normal(S).astype(np.float32)
    return xq, xp, W, y, m, adv, L


def pin_lossless_grid():
    xq, xp, W, y, m, adv, L = _grid_case(5)
    assert np.array_equal(oracle.dequantize_e4m3_rows(W), W.astype(np.float64))
    f0 = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    f8 = oracle.forward(xq, xp, W, y, m, adv, L, BETA, variant=V8)
    for k in ("logp", "ref_logp", "kl"):
        assert np.array_equal(f0[k], f8[k]), k
    # g: the same value by the general variant formula (last-bit rounding differences)
    assert np.allclose(f0["g"], f8["g"], rtol=1e-14, atol=0)
    b0 = oracle.backward(xq, W, y, m, f0, need_dW=True)
    b8 = oracle.backward(xq, W, y, m, f8, need_dW=True)
    for k in ("dX", "dW"):
        assert np.abs(b0[k] - b8[k]).max() <= 1e-13 * np.abs(b0[k]).max(), k


def _torch_fp8_rows(x):
    x = torch.from_numpy(np.asarray(x, np.float32))
    amax = x.abs().amax(dim=1)
    inv = torch.where(amax > 0, 448.0 / amax, torch.ones_like(amax))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (x * inv[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
    return q * s.to(torch.float64)[:, None]


def pin_fp8_forward_against_torch():
    xq, xp, W, y, m, adv, L = _case(7)
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA, variant=V8)
    Wh = _torch_fp8_rows(W)
    rows = np.nonzero(m)[0]
    for x, key in ((xq, "logp"), (xp, "ref_logp")):
        lp = torch.log_softmax(_torch_fp8_rows(x[rows]) @ Wh.T, dim=1)
        ref = lp[torch.arange(len(rows)), torch.from_numpy(y[rows])].numpy()
        assert np.allclose(f[key][rows], ref, rtol=0, atol=1e-12), key
    f0 = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    assert np.abs(f["logp"] - f0["logp"]).max() > 1e-6      # the variant is not a no-op


def pin_fp8_backward_against_torch_ce():
    xq, xp, W, y, m, _, L = _case(11)
    adv = np.ones(2, np.float32)
    f = oracle.forward(xq, xp, W, y, m, adv, L, 0.0, variant=V8)
    b = oracle.backward(xq, W, y, m, f, need_dW=True)
    rows = np.nonzero(m)[0]
    Z = (_torch_fp8_rows(xq[rows]) @ _torch_fp8_rows(W).T).detach().requires_grad_(True)
    torch.nn.functional.cross_entropy(Z, torch.from_numpy(y[rows])).backward()
    dZ = Z.grad
    dX = (dZ @ torch.from_numpy(W.astype(np.float64))).numpy()
    dW = (dZ.T @ torch.from_numpy(xq[rows].astype(np.float64))).numpy()
    assert np.allclose(b["dX"], dX, rtol=0, atol=1e-13)
    assert np.allclose(b["dW"], dW, rtol=0, atol=1e-13)


PINS = [pin_e4m3_round_matches_torch, pin_quantize_rows_bounds, pin_lossless_grid,
        pin_fp8_forward_against_torch, pin_fp8_backward_against_torch_ce]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------- teeth

_REAL = {k: getattr(og, k) for k in ("e4m3_round", "quantize_e4m3_rows", "dequantize_e4m3_rows")}


def _mut_round_truncate(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    quantum = np.where(e < -6, 2.0 ** -9, 2.0 ** (e - 3))
    return np.sign(y) * np.floor(a / quantum) * quantum


def _mut_round_no_subnormals(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    quantum = 2.0 ** (e - 3)
    return np.sign(y) * np.rint(a / quantum) * quantum


def _mut_quantize_240(x, codes=True):
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    inv = (np.float32(240.0) / amax).astype(np.float32)
    s = (amax / np.float32(240.0)).astype(np.float32)
    q = _REAL["e4m3_round"]((x * inv[:, None]).astype(np.float32))
    return q, og.e4m3_codes(q), s


_calls = {"n": 0}


def _mut_dequant_first_call_only(x):
    # quantises the first call (W in the forward) and passes later ones (X rows) through
    _calls["n"] += 1
    if _calls["n"] == 1:
        return _REAL["dequantize_e4m3_rows"](x)
    return np.asarray(x, dtype=np.float64)


MUTATIONS = {
    "round_truncates": ("e4m3_round", _mut_round_truncate),
    "round_without_subnormals": ("e4m3_round", _mut_round_no_subnormals),
    "scale_to_240": ("quantize_e4m3_rows", _mut_quantize_240),
    "only_W_quantised": ("dequantize_e4m3_rows", _mut_dequant_first_call_only),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_fp8_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    _calls["n"] = 0
    monkeypatch.setattr(og, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        _calls["n"] = 0
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} slipped past every pin"
