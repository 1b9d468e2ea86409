"""Pins of the CPU oracle against what the pages and mathematics fix.

Each ``pin_*`` function raises AssertionError on failure.  The tests run every
pin on the oracle as written, and ``test_planted_mistakes_are_caught`` plants
plausible mistakes into the oracle (on the CPU) and checks that at least one
pin fails for each, so the pins are known to have teeth.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.grpo_oracle as og
from synth import materialized_logits_bytes
from tests._brute import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BETA = 0.04


def _case(seed, S=2, L=3, H=4, V=5, x_std=1.0, w_std=0.5, full_mask=False):
    g = np.random.default_rng(seed)
    N = S * L
    xq = g.standard_normal((N, H))
    xp = g.standard_normal((N, H))
    W = g.standard_normal((V, H)) * w_std
    y = g.integers(0, V, size=N)
    m = np.ones(N, dtype=np.int64) if full_mask else (g.random(N) < 0.7).astype(np.int64)
    if m.sum() == 0:
        m[0] = 1
    adv = g.standard_normal(S).astype(np.float32)
    return xq * x_std, xp * x_std, W, y, m, adv, L


# ----------------------------------------------------------------------------- advantages

def pin_advantages_equal_rewards():
    """Equal scores whose fp32 sum is exact (1.5 * 8) give exactly zero advantage.  When the
    sum rounds (1.7 * 8), the mean is off by under an ulp of the score and the std is
    about that size too, so |A| stays below ulp(score) / eps."""
    A = oracle.group_advantages(np.full((3, 8, 1), 1.5, np.float32))
    assert np.all(A == 0.0), A
    A = oracle.group_advantages(np.full((1, 8, 1), 1.7, np.float32))
    assert np.all(np.abs(A) < 2 * np.spacing(np.float32(1.7)) / 1e-4), A


def pin_advantages_two_closed_form():
    """G = 2, scores (0, 1): mean 1/2, unbiased std sqrt(1/2), A = -+(1/2)/(sqrt(1/2)+1e-4)."""
    A = oracle.group_advantages(np.array([[[0.0], [1.0]]], np.float32), eps=1e-4)
    exact = 0.5 / (math.sqrt(0.5) + 1e-4)
    assert abs(float(A[1]) - exact) <= 2 * np.spacing(np.float32(exact)), (A, exact)
    assert float(A[0]) == -float(A[1])


def pin_advantages_match_torch_std():
    """Against torch's unbiased std (a library routine) in fp64: agreement to fp32 rounding,
    including the sum over K reward functions before normalising."""
    g = np.random.default_rng(7)
    r = g.uniform(0, 3, size=(5, 8, 3)).astype(np.float32)
    A = oracle.group_advantages(r, eps=1e-4).reshape(5, 8)
    t = torch.from_numpy(r.astype(np.float64)).sum(-1)
    ref = (t - t.mean(1, keepdim=True)) / (t.std(1, unbiased=True, keepdim=True) + 1e-4)
    assert np.allclose(A, ref.numpy(), rtol=3e-6, atol=3e-6), np.abs(A - ref.numpy()).max()


def pin_advantages_moments():
    """mean(A) = 0 and the unbiased std of A is sd / (sd + eps)."""
    g = np.random.default_rng(3)
    r = g.normal(0, 1, size=(1, 16, 1)).astype(np.float32)
    A = oracle.group_advantages(r, eps=1e-4).astype(np.float64)
    sd = float(np.std(r.astype(np.float64), ddof=1))
    assert abs(A.mean()) < 1e-6
    assert abs(np.std(A, ddof=1) - sd / (sd + 1e-4)) < 1e-5


def pin_advantages_sequential_order():
    """The fixed order is a left-to-right fp32 sum.  Scores (1e8, 1, -1e8, 1): left to right
    the 1 is absorbed by 1e8 (fp32 spacing there is 8), so the sum is 1 and the mean is
    0.25; a pairwise order would give mean 0.  A[1] = 0.75 / (std + eps) tells them apart."""
    r = np.array([[[1e8], [1.0], [-1e8], [1.0]]], np.float32)
    A = oracle.group_advantages(r, eps=1e-4)
    sd = math.sqrt(2e16 / 3.0)
    assert abs(float(A[1]) * sd - 0.75) < 1e-3, float(A[1]) * sd
    assert float(A[1]) == float(A[3])


# ----------------------------------------------------------------------------- per token

def pin_logsoftmax_normalised():
    """exp(log-softmax) sums to 1 per row; with W = 0 every log-prob is exactly -log V."""
    g = np.random.default_rng(11)
    z = g.standard_normal((6, 1000)) * 30.0
    lp, lse = oracle.log_softmax_rows(z)
    assert np.allclose(np.exp(lp).sum(1), 1.0, atol=1e-12)
    assert np.allclose(lse, np.log(np.exp(z).sum(1)), rtol=1e-13)
    xq, xp, W, y, m, adv, L = _case(12, V=1000, H=8)
    f = oracle.forward(xq, xp, np.zeros_like(W), y, m, adv, L, BETA)
    assert np.allclose(f["logp"][m == 1], -math.log(1000), rtol=0, atol=1e-14)


def pin_kl_direction_exact_expectation():
    """Under y ~ Q the estimator averages to the reverse KL(Q||P), not KL(P||Q): the exact
    expectation, summed over a small vocabulary."""
    g = np.random.default_rng(5)
    for _ in range(4):
        Q = g.dirichlet(np.ones(7))
        P = g.dirichlet(np.ones(7))
        est = float(np.sum(Q * oracle.reverse_kl_k3(np.log(Q), np.log(P))))
        rev = float(np.sum(Q * np.log(Q / P)))
        fwd = float(np.sum(P * np.log(P / Q)))
        assert abs(est - rev) < 1e-12, (est, rev)
        assert abs(est - fwd) > 1e-3
    # the estimator is >= 0 pointwise and 0 only at q = ref
    d = np.linspace(-5, 5, 101)
    k = oracle.reverse_kl_k3(np.zeros_like(d), d)
    assert np.all(k >= 0) and k[50] == 0.0


def pin_policy_equals_reference():
    """X_p = X_q: KL = 0 exactly, loss = -sum(m*A)/N_tok, g = -m*A/N_tok."""
    xq, _, W, y, m, adv, L = _case(21, S=4, L=6, H=5, V=9)
    f = oracle.forward(xq, xq, W, y, m, adv, L, BETA)
    a_tok = adv[np.arange(len(m)) // L].astype(np.float64)
    n = m.sum()
    assert np.all(f["kl"] == 0.0)
    assert abs(f["loss"] - (-(m * a_tok).sum() / n)) < 1e-15
    assert np.allclose(f["g"], -m * a_tok / n, rtol=0, atol=1e-16)


def pin_brute_force():
    """Scalar loops (no BLAS) against the oracle on tiny shapes."""
    for seed, shp in enumerate([(2, 3, 4, 5), (3, 4, 2, 7), (1, 5, 3, 3), (2, 2, 6, 11)]):
        S, L, H, V = shp
        xq, xp, W, y, m, adv, L = _case(100 + seed, S, L, H, V)
        f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
        b = oracle.backward(xq, W, y, m, f, need_dW=True)
        bb = brute(xq.tolist(), xp.tolist(), W.tolist(), y.tolist(), m.tolist(),
                   adv.astype(np.float64).tolist(), L, BETA)
        assert abs(f["loss"] - bb["loss"]) < 1e-12
        assert np.allclose(f["logp"], bb["logp"], atol=1e-12)
        assert np.allclose(f["ref_logp"], bb["ref"], atol=1e-12)
        assert np.allclose(f["kl"], bb["kl"], atol=1e-12)
        assert np.allclose(f["g"], bb["g"], atol=1e-13)
        dX = np.zeros_like(xq)
        dX[b["rows"]] = b["dX"]
        assert np.allclose(dX, np.array(bb["dX"]), atol=1e-12)
        assert np.allclose(b["dW"], np.array(bb["dW"]), atol=1e-12)


def pin_g_matches_surrogate_fd():
    """g = d loss/dq equals central differences of -A*exp(q-q0) + beta*KL(q, ref) at q0.
    (Differencing the loss value instead would miss the -A term: the ratio's value is 1.)"""
    xq, xp, W, y, m, adv, L = _case(31, S=3, L=4, H=6, V=13)
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    q0, ref = f["logp"].copy(), f["ref_logp"]
    a_tok = adv[np.arange(len(m)) // L].astype(np.float64)
    h = 1e-6
    for t in np.nonzero(m)[0]:
        qp, qm = q0.copy(), q0.copy()
        qp[t] += h
        qm[t] -= h
        fd = (oracle.surrogate_objective(qp, q0, ref, a_tok, m, BETA)
              - oracle.surrogate_objective(qm, q0, ref, a_tok, m, BETA)) / (2 * h)
        assert abs(fd - f["g"][t]) < 1e-8, (t, fd, f["g"][t])


def pin_dx_dw_finite_differences():
    """dX_q and dW against central differences of the surrogate through q(X_q, W), with the
    reference log-probs and q0 held fixed (only the policy path is differentiated)."""
    xq, xp, W, y, m, adv, L = _case(41, S=2, L=4, H=3, V=6)
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    b = oracle.backward(xq, W, y, m, f, need_dW=True)
    q0, ref = f["logp"].copy(), f["ref_logp"]
    a_tok = adv[np.arange(len(m)) // L].astype(np.float64)

    def F(Xq, Wm):
        lp, _ = oracle.log_softmax_rows(Xq @ Wm.T)
        q = lp[np.arange(len(y)), y]
        return oracle.surrogate_objective(q, q0, ref, a_tok, m, BETA)

    h = 1e-6
    dX = np.zeros_like(xq)
    dX[b["rows"]] = b["dX"]
    for t in range(xq.shape[0]):
        for j in range(xq.shape[1]):
            P, M = xq.copy(), xq.copy()
            P[t, j] += h
            M[t, j] -= h
            assert abs((F(P, W) - F(M, W)) / (2 * h) - dX[t, j]) < 1e-8
    # dW whole, and one vocabulary row at a time from the loss rows alone
    rows = np.nonzero(m)[0]
    dWr = oracle.dw_rows(xq[rows], W, y, m, f, np.arange(W.shape[0])[::-1])[::-1]
    for v in range(W.shape[0]):
        for j in range(W.shape[1]):
            P, M = W.copy(), W.copy()
            P[v, j] += h
            M[v, j] -= h
            fd = (F(xq, P) - F(xq, M)) / (2 * h)
            assert abs(fd - b["dW"][v, j]) < 1e-8
            assert abs(fd - dWr[v, j]) < 1e-8


def pin_cross_entropy_reduction():
    """beta = 0 and A = 1: the loss is -1 and dX_q, dW equal the gradients of the mean
    cross-entropy over loss tokens, as computed by torch's cross_entropy autograd (fp64)."""
    xq, xp, W, y, m, _, L = _case(51, S=3, L=5, H=7, V=17)
    adv = np.ones(3, np.float32)
    f = oracle.forward(xq, xp, W, y, m, adv, L, 0.0)
    b = oracle.backward(xq, W, y, m, f, need_dW=True)
    assert abs(f["loss"] + 1.0) < 1e-15
    rows = np.nonzero(m)[0]
    X = torch.tensor(xq[rows], dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(X @ Wt.T, torch.tensor(y[rows]))
    ce.backward()
    assert np.allclose(b["dX"], X.grad.numpy(), atol=1e-14)
    assert np.allclose(b["dW"], Wt.grad.numpy(), atol=1e-14)


def pin_loss_scale_cancels():
    """The fp16 convention: grad_loss = loss_scale = S returns the unscaled gradient."""
    xq, xp, W, y, m, adv, L = _case(61, S=2, L=4, H=3, V=6)
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    b1 = oracle.backward(xq, W, y, m, f, need_dW=True)
    b2 = oracle.backward(xq, W, y, m, f, grad_loss=65536.0, loss_scale=65536.0, need_dW=True)
    assert np.allclose(b1["dX"], b2["dX"], rtol=1e-15) and np.allclose(b1["dW"], b2["dW"])


def pin_naive_fp16_overflow():
    """The mixed-precision diagnostic, by hand: W = 0 makes every softmax uniform, so with
    V = 2 and target 0 the logit gradient row is (1/2, -1/2); X_p = X_q makes KL = 0, so
    g_t = -A_t / N_tok, here -+2 / 2.  A naive path forming grad_loss * g * (onehot - P) then
    peaks at grad_loss / 2 (over tau: the temperature divides it), and it overflows fp16
    exactly when that reaches 65520, the first magnitude that rounds to inf."""
    xq = np.array([[0.3], [-1.1]])
    W = np.zeros((2, 1))
    y = np.array([0, 0])
    m = np.array([1, 1])
    adv = np.array([2.0, -2.0], np.float32)
    f = oracle.forward(xq, xq.copy(), W, y, m, adv, 1, BETA)
    assert np.array_equal(f["g"], [-1.0, 1.0]), f["g"]
    for grad_loss, over in ((131040.0, True), (131038.0, False)):
        b = oracle.backward(xq, W, y, m, f, grad_loss=grad_loss, loss_scale=grad_loss)
        assert b["naive_max_abs"] == grad_loss / 2 and b["naive_fp16_overflow"] is over
    with np.errstate(over="ignore"):
        assert float(np.float16(65520.0)) == np.inf and float(np.float16(65519.0)) == 65504.0
    fv = oracle.forward(xq, xq.copy(), W, y, m, adv, 1, BETA, variant=og.Variant(temperature=2.0))
    b = oracle.backward(xq, W, y, m, fv, grad_loss=131040.0, loss_scale=131040.0)
    assert b["naive_max_abs"] == 131040.0 / 4 and not b["naive_fp16_overflow"]


PINS = [pin_advantages_equal_rewards, pin_advantages_two_closed_form,
        pin_advantages_match_torch_std, pin_advantages_moments,
        pin_advantages_sequential_order, pin_logsoftmax_normalised,
        pin_kl_direction_exact_expectation, pin_policy_equals_reference, pin_brute_force,
        pin_g_matches_surrogate_fd, pin_dx_dw_finite_differences,
        pin_cross_entropy_reduction, pin_loss_scale_cancels, pin_naive_fp16_overflow]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------- edges

def test_masked_rows_not_read():
    """A NaN in a masked-out row neither reaches any output nor sets the non-finite flag."""
    xq, xp, W, y, m, adv, L = _case(71, S=2, L=5, H=4, V=8)
    m[1] = 0
    xq[1] = np.nan
    xp[1] = np.inf
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    b = oracle.backward(xq, W, y, m, f, need_dW=True)
    assert np.isfinite(f["loss"]) and not oracle.found_inf(f, b)
    assert f["logp"][1] == 0.0 and f["g"][1] == 0.0
    xq[2] = np.nan
    m[2] = 1
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    assert oracle.found_inf(f, None)


def test_no_loss_tokens():
    """N_tok = 0: the denominator is clamped to 1, loss and gradients are 0."""
    xq, xp, W, y, m, adv, L = _case(81)
    m[:] = 0
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    b = oracle.backward(xq, W, y, m, f, need_dW=True)
    assert f["loss"] == 0.0 and f["n_tok"] == 0
    assert np.all(b["dW"] == 0.0) and b["dX"].size == 0


def test_sampled_rows_match_full():
    """Sampled mode (rows given explicitly) reproduces the full computation row by row."""
    xq, xp, W, y, m, adv, L = _case(91, S=3, L=6, H=5, V=11)
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    b = oracle.backward(xq, W, y, m, f)
    rows = np.array([4, 0, 17, 9])
    fs = oracle.forward(xq[rows], xp[rows], W, y, m, adv, L, BETA, rows=rows)
    bs = oracle.backward(xq[rows], W, y, m, fs, rows=rows)
    for k in ("logp", "ref_logp", "kl", "g", "lse_q"):
        assert np.array_equal(fs[k][rows], f[k][rows])
    full = np.zeros_like(xq)
    full[b["rows"]] = b["dX"]
    assert np.allclose(bs["dX"], full[rows], atol=1e-15)
    assert fs["loss"] is None


@pytest.mark.parametrize("variant", [og.Variant(), og.Variant(temperature=0.6),
                                     og.Variant(kl="forward", norm="sequences")],
                         ids=["default", "temperature", "forward-seq"])
def test_dw_rows_match_backward(variant):
    """Selected vocabulary rows of dW from the loss rows alone equal the same rows of the
    full dW (pinned by finite differences), for any row order and with a loss scale."""
    xq, xp, W, y, m, adv, L = _case(97, S=3, L=6, H=5, V=23)
    f = oracle.forward(xq, xp, W, y, m, adv, L, BETA, variant=variant)
    b = oracle.backward(xq, W, y, m, f, grad_loss=3.0, loss_scale=2.0, need_dW=True)
    vr = np.array([22, 0, 7, int(y[np.nonzero(m)[0][0]]), 13])
    got = oracle.dw_rows(xq[np.nonzero(m)[0]], W, y, m, f, vr, grad_loss=3.0, loss_scale=2.0,
                         block=4)
    assert np.allclose(got, b["dW"][vr], rtol=1e-12, atol=1e-15)


def test_memory_figures_golden():
    """The pages' memory arithmetic for the long-context shape: two 16-bit (G, L, V) logits
    tensors are 78.3 GiB; one generation's share (1/8) is the 9.8 GiB the efficient loss
    still needs; the difference is the 68.5 GiB saved, a factor of more than 8."""
    gold = json.load(open(os.path.join(GOLDEN, "memory_figures.json")))
    b = materialized_logits_bytes(gold["G"], gold["L"], gold["V"], gold["bytes_per_element"],
                                  gold["copies"])
    gib = b / 2 ** 30
    assert round(gib, 1) == gold["materialized_logits_GB_printed"]
    assert round(gib / gold["G"], 1) == gold["efficient_extra_GB_printed"]
    assert round(gib - gib / gold["G"], 1) == gold["saved_GB_printed"]
    assert gib / (gib / gold["G"]) >= gold["reduction_factor_printed"]


# ----------------------------------------------------------------------------- teeth

def _mut_forward_kl(q, ref):
    d = np.asarray(q, float) - np.asarray(ref, float)
    return np.expm1(d) - d


def _mut_kl_no_minus_one(q, ref):
    d = np.asarray(ref, float) - np.asarray(q, float)
    return np.exp(d) - d


def _mut_kl_extra_q_factor(q, ref):
    d = np.asarray(ref, float) - np.asarray(q, float)
    return np.exp(np.asarray(q, float)) * (np.expm1(d) - d)


def _mut_grad_sign(adv, q, ref, beta, n):
    return (adv - beta * np.expm1(ref - q)) / n


def _mut_grad_no_kl(adv, q, ref, beta, n):
    return -adv / n


def _mut_grad_no_detach(adv, q, ref, beta, n):   # ratio without stop-gradient: zero A-term
    return (-beta * np.expm1(ref - q)) / n


def _mut_loss_plus_a(kl, adv, beta):
    return beta * kl + adv


def _mut_logit_grad_sign(lp, y):
    T = np.exp(lp)
    T[np.arange(len(y)), y] -= 1.0
    return T


def _mut_logit_grad_offby1(lp, y):
    T = -np.exp(lp)
    T[np.arange(len(y)), (y + 1) % lp.shape[1]] += 1.0
    return T


def _mut_lse_no_shift(z):
    z = np.asarray(z, float)
    lse = np.log(np.exp(z).sum(axis=1))
    return z - lse[:, None] * 0.999, lse


def _mut_adv_population(rewards, eps=1e-4, unbiased=True):
    return _REAL_ADV(rewards, eps, unbiased=False)


def _mut_adv_eps_in_var(rewards, eps=1e-4, unbiased=True):
    r = np.asarray(rewards, np.float64)
    r = r if r.ndim == 3 else r[:, :, None]
    s = r.sum(-1)
    A = (s - s.mean(1, keepdims=True)) / np.sqrt(s.var(1, ddof=1, keepdims=True) + eps)
    return A.astype(np.float32).reshape(-1)


def _mut_adv_pairwise(rewards, eps=1e-4, unbiased=True):
    """Same formula, tree-order sums ((r0 + r1) + (r2 + r3)) ... instead of left to right."""
    f = np.float32
    r = np.asarray(rewards, f)
    r = r if r.ndim == 3 else r[:, :, None]

    def tree(v):
        v = list(v)
        while len(v) > 1:
            v = [f(v[i] + v[i + 1]) if i + 1 < len(v) else v[i] for i in range(0, len(v), 2)]
        return v[0]

    out = []
    for b in range(r.shape[0]):
        s = [tree(r[b, g]) for g in range(r.shape[1])]
        mean = f(tree(s) / f(len(s)))
        sd = f(np.sqrt(f(tree([f(f(x - mean) * f(x - mean)) for x in s]) / f(len(s) - 1))))
        out += [f(f(x - mean) / f(sd + f(eps))) for x in s]
    return np.array(out, f)


_REAL_ADV = og.group_advantages
_REAL_DW_ROWS = og.dw_rows


def _mut_dw_rows_no_onehot(xq, W, targets, mask, fwd, vrows, **kw):
    # the softmax part only: as if every target were outside the selected rows
    return _REAL_DW_ROWS(xq, W, np.full_like(np.asarray(targets), -1), mask, fwd, vrows, **kw)

MUTATIONS = {
    "forward_kl": ("reverse_kl_k3", _mut_forward_kl),
    "kl_without_minus_one": ("reverse_kl_k3", _mut_kl_no_minus_one),
    "kl_extra_q_factor": ("reverse_kl_k3", _mut_kl_extra_q_factor),
    "grad_sign_of_A": ("policy_grad", _mut_grad_sign),
    "grad_missing_kl": ("policy_grad", _mut_grad_no_kl),
    "grad_no_detach": ("policy_grad", _mut_grad_no_detach),
    "loss_sign_of_A": ("token_loss", _mut_loss_plus_a),
    "logit_grad_sign": ("logit_grad", _mut_logit_grad_sign),
    "logit_grad_wrong_index": ("logit_grad", _mut_logit_grad_offby1),
    "lse_wrong": ("log_softmax_rows", _mut_lse_no_shift),
    "adv_population_std": ("group_advantages", _mut_adv_population),
    "adv_eps_in_variance": ("group_advantages", _mut_adv_eps_in_var),
    "adv_other_sum_order": ("group_advantages", _mut_adv_pairwise),
    "dw_rows_no_onehot": ("dw_rows", _mut_dw_rows_no_onehot),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(og, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} slipped past every pin"
