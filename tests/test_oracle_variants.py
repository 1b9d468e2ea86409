"""Pins of the oracle's loss variants [Long-context GRPO, §4 (the KL, ratio and
normalisation experiments)] against what mathematics fixes independently of the oracle.

* forward estimator: its exact expectation under P is KL(P||Q), by scipy's rel_entr;
* reverse estimator with the Q factor: summed over the vocabulary it is KL(Q||P);
* each estimator's gradient: central differences of its value;
* sequence mean: hand-computed weights, and the reduction to independent one-sequence
  problems (where the token mean is the sequence mean) averaged over sequences;
* temperature tau: the same loss as the default with the head W / tau, so dX matches
  and dW is the default's divided by tau;
* ratio without stop-gradient: with beta = 0 its gradient vanishes;
* every variant's dX, dW: central differences of the surrogate through q(X, W).

``test_planted_variant_mistakes_are_caught`` plants mistakes into the variant code of
the oracle and checks that a pin fails for each.
"""

import numpy as np
import pytest
from scipy.special import rel_entr

import oracle
import oracle.grpo_oracle as og

BETA = 0.04
V_ = oracle.Variant


def _case(seed, S=3, L=4, H=5, V=11, w_std=0.7):
    g = np.random.default_rng(seed)
    N = S * L
    xq = g.standard_normal((N, H))
    xp = xq + 0.3 * g.standard_normal((N, H))
    W = g.standard_normal((V, H)) * w_std
    y = g.integers(0, V, size=N)
    m = (g.random(N) < 0.7).astype(np.int64)
    m[0] = 1
    adv = g.standard_normal(S).astype(np.float32)
    return xq, xp, W, y, m, adv, L


VARIANTS = [V_(kl="forward"), V_(kl="reverse_q"), V_(detach=False), V_(norm="sequences"),
            V_(temperature=0.7), V_(kl="forward", detach=False, norm="sequences",
                                    temperature=1.6)]


def pin_forward_kl_exact_expectation():
    g = np.random.default_rng(3)
    for _ in range(4):
        Q = g.dirichlet(np.ones(9))
        P = g.dirichlet(np.ones(9))
        est = float(np.sum(P * oracle.forward_kl_k3(np.log(Q), np.log(P))))
        assert abs(est - rel_entr(P, Q).sum()) < 1e-12
        assert abs(est - rel_entr(Q, P).sum()) > 1e-3


def pin_reverse_q_full_vocabulary_sum():
    g = np.random.default_rng(4)
    for _ in range(4):
        Q = g.dirichlet(np.ones(9))
        P = g.dirichlet(np.ones(9))
        tot = float(np.sum(oracle.reverse_kl_q(np.log(Q), np.log(P))))
        assert abs(tot - rel_entr(Q, P).sum()) < 1e-12


def pin_kl_gradients_fd():
    g = np.random.default_rng(5)
    q = -np.abs(g.standard_normal(20)) - 0.1
    ref = q + 0.5 * g.standard_normal(20)
    h = 1e-6
    for kl in ("reverse", "forward", "reverse_q"):
        v = V_(kl=kl)
        fd = (oracle.kl_value(v, q + h, ref) - oracle.kl_value(v, q - h, ref)) / (2 * h)
        assert np.allclose(fd, oracle.kl_grad_q(v, q, ref), rtol=1e-7, atol=1e-9), kl


def pin_sequence_weights_closed_form():
    m = np.array([1, 1, 0, 0,   0, 0, 0, 0,   1, 1, 1, 1,   0, 1, 0, 0])
    w = oracle.token_weights(m, 4, "sequences")
    # three non-empty sequences with 2, 4 and 1 loss tokens
    want = np.array([1 / 6, 1 / 6, 0, 0, 0, 0, 0, 0, 1 / 12, 1 / 12, 1 / 12, 1 / 12,
                     0, 1 / 3, 0, 0])
    assert np.allclose(w, want, rtol=1e-15, atol=0)
    assert np.allclose(oracle.token_weights(m, 4, "tokens"), m / 7, rtol=1e-15, atol=0)


def pin_sequence_mean_is_mean_of_sequences():
    xq, xp, W, y, m, adv, L = _case(11, S=4, L=5)
    m[5:10] = 0                                   # one empty sequence
    for kl in ("reverse", "forward"):
        v = V_(kl=kl, norm="sequences")
        f = oracle.forward(xq, xp, W, y, m, adv, L, BETA, variant=v)
        b = oracle.backward(xq, W, y, m, f, need_dW=True)
        nonempty = [s for s in range(4) if m[s * L:(s + 1) * L].sum() > 0]
        loss, g, dW = 0.0, np.zeros(len(m)), 0.0
        for s in nonempty:
            sl = slice(s * L, (s + 1) * L)
            fs = oracle.forward(xq[sl], xp[sl], W, y[sl], m[sl], adv[s:s + 1], L, BETA,
                                variant=V_(kl=kl))
            bs = oracle.backward(xq[sl], W, y[sl], m[sl], fs, need_dW=True)
            loss += fs["loss"] / len(nonempty)
            g[sl] = fs["g"] / len(nonempty)
            dW = dW + bs["dW"] / len(nonempty)
        assert abs(f["loss"] - loss) < 1e-14
        assert np.allclose(f["g"], g, rtol=1e-13, atol=1e-16)
        assert np.allclose(b["dW"], dW, rtol=1e-12, atol=1e-15)


def pin_temperature_is_a_scaled_head():
    xq, xp, W, y, m, adv, L = _case(13)
    for tau in (0.5, 1.7):
        for kl in ("reverse", "reverse_q"):
            f = oracle.forward(xq, xp, W, y, m, adv, L, BETA,
                               variant=V_(kl=kl, temperature=tau))
            f1 = oracle.forward(xq, xp, W / tau, y, m, adv, L, BETA, variant=V_(kl=kl))
            for k in ("logp", "ref_logp", "kl", "g"):
                assert np.allclose(f[k], f1[k], rtol=1e-12, atol=1e-15), (tau, k)
            assert abs(f["loss"] - f1["loss"]) < 1e-13
            b = oracle.backward(xq, W, y, m, f, need_dW=True)
            b1 = oracle.backward(xq, W / tau, y, m, f1, need_dW=True)
            assert np.allclose(b["dX"], b1["dX"], rtol=1e-11, atol=1e-15)
            assert np.allclose(b["dW"], b1["dW"] / tau, rtol=1e-11, atol=1e-15)


def pin_no_detach_without_kl_has_no_gradient():
    xq, xp, W, y, m, adv, L = _case(17)
    f = oracle.forward(xq, xp, W, y, m, adv, L, 0.0, variant=V_(detach=False))
    f0 = oracle.forward(xq, xp, W, y, m, adv, L, 0.0)
    b = oracle.backward(xq, W, y, m, f, need_dW=True)
    assert np.all(f["g"] == 0.0) and np.all(b["dX"] == 0.0) and np.all(b["dW"] == 0.0)
    assert f["loss"] == f0["loss"]
    assert np.any(f0["g"] != 0.0)


def pin_variant_dx_dw_fd():
    xq, xp, W, y, m, adv, L = _case(19, S=2, L=3, H=3, V=6)
    a_tok = adv[np.arange(len(m)) // L].astype(np.float64)
    h = 1e-6
    for v in VARIANTS:
        f = oracle.forward(xq, xp, W, y, m, adv, L, BETA, variant=v)
        b = oracle.backward(xq, W, y, m, f, need_dW=True)
        q0, ref = f["logp"].copy(), f["ref_logp"]

        def F(Xq, Wm):
            z = Xq @ Wm.T / v.temperature
            z = z - z.max(1, keepdims=True)
            lp = z - np.log(np.exp(z).sum(1, keepdims=True))
            q = lp[np.arange(len(y)), y]
            return oracle.surrogate_objective(q, q0, ref, a_tok, m, BETA, v, L)

        dX = np.zeros_like(xq)
        dX[b["rows"]] = b["dX"]
        for t in range(xq.shape[0]):
            for j in range(xq.shape[1]):
                P, M = xq.copy(), xq.copy()
                P[t, j] += h
                M[t, j] -= h
                assert abs((F(P, W) - F(M, W)) / (2 * h) - dX[t, j]) < 1e-8, v
        for vv in range(W.shape[0]):
            for j in range(W.shape[1]):
                P, M = W.copy(), W.copy()
                P[vv, j] += h
                M[vv, j] -= h
                assert abs((F(xq, P) - F(xq, M)) / (2 * h) - b["dW"][vv, j]) < 1e-8, v
        # the loss value is the surrogate at q = q0
        assert abs(F(xq, W) - f["loss"]) < 1e-12, v


PINS = [pin_forward_kl_exact_expectation, pin_reverse_q_full_vocabulary_sum,
        pin_kl_gradients_fd, pin_sequence_weights_closed_form,
        pin_sequence_mean_is_mean_of_sequences, pin_temperature_is_a_scaled_head,
        pin_no_detach_without_kl_has_no_gradient, pin_variant_dx_dw_fd]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_default_variant_matches_plain_call():
    xq, xp, W, y, m, adv, L = _case(23)
    a = oracle.forward(xq, xp, W, y, m, adv, L, BETA)
    b = oracle.forward(xq, xp, W, y, m, adv, L, BETA, variant=V_())
    for k in ("logp", "kl", "g"):
        assert np.array_equal(a[k], b[k])


# ----------------------------------------------------------------------------- teeth

_REAL = {k: getattr(og, k) for k in ("forward_kl_k3", "reverse_kl_k3", "kl_grad_q",
                                     "token_weights", "logits", "grad_factor",
                                     "advantage_term")}


def _mut_kl_grad(sign_kl):
    def f(v, q, ref):
        g = _REAL["kl_grad_q"](v, q, ref)
        return -g if v.kl == sign_kl else g
    return f


def _mut_weights_no_nseq(mask, L, norm):
    if norm != "sequences":
        return _REAL["token_weights"](mask, L, norm)
    m = np.asarray(mask).reshape(-1).astype(np.float64)
    per = m.reshape(-1, L).sum(1)
    w = np.zeros_like(m)
    rows = np.nonzero(m)[0]
    w[rows] = 1.0 / per[rows // L]
    return w


def _mut_weights_by_L(mask, L, norm):
    if norm != "sequences":
        return _REAL["token_weights"](mask, L, norm)
    m = np.asarray(mask).reshape(-1).astype(np.float64)
    nseq = max(1.0, float((m.reshape(-1, L).sum(1) > 0).sum()))
    return m / (L * nseq)


MUTATIONS = {
    "forward_kl_roles_not_swapped": ("forward_kl_k3", lambda q, ref: _REAL["reverse_kl_k3"](q, ref)),
    "reverse_q_without_q_factor": ("reverse_q", None),
    "forward_kl_grad_sign": ("kl_grad_q", _mut_kl_grad("forward")),
    "reverse_q_grad_sign": ("kl_grad_q", _mut_kl_grad("reverse_q")),
    "sequence_weights_without_count": ("token_weights", _mut_weights_no_nseq),
    "sequence_weights_over_L": ("token_weights", _mut_weights_by_L),
    "temperature_ignored_in_logits": ("logits", lambda x, W, tau=1.0: _REAL["logits"](x, W)),
    "temperature_ignored_in_backward": ("grad_factor",
                                        lambda gl, ls, tau: _REAL["grad_factor"](gl, ls, 1.0)),
    "ratio_always_detached": ("advantage_term", lambda a, d: _REAL["advantage_term"](a, True)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_variant_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    if attr == "reverse_q":
        attr, fn = "reverse_kl_q", lambda q, ref: _REAL["reverse_kl_k3"](q, ref)
    monkeypatch.setattr(og, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} slipped past every pin"
