"""fp64 NumPy oracle for the memory-efficient linear GRPO loss (test infrastructure).

What the pages fix, restated (the formulas on the pages were images and did not
survive; the prose and the one surviving code fragment carry the method):

* GRPO scores each sampled response of a group and compares it with the group
  mean; better-than-average responses are reinforced [Train your own R1
  reasoning model with Unsloth, §3 "GRPO + aha moment"].  The advantage A
  takes every reward function into account [Long-context GRPO, §4].
* The KL term is the reverse KL between the trained policy Q and the frozen
  reference P, estimated per token without an extra Q factor, scaled by
  beta = 0.04 [Long-context GRPO, §3 and §4].
* The advantage is multiplied by exp(q - stopgrad(q)): a factor whose value is 1
  but whose gradient flows through the policy log-prob q [Long-context GRPO, §4].
* Log-probs come from the logsumexp trick [Long-context GRPO, §4], and the
  memory-efficient algorithm never stores the (G, L, V) logits
  [Long-context GRPO, §2 and §3].  Chunking and an online logsumexp reach the
  same numbers as the dense definition, so this oracle is the dense definition:
  it materialises each row's full vocabulary of logits in fp64.

Readings where the pages are silent (each one is pinned by a test):
* loss = sum_t m_t * l_t / N_tok, a masked mean over all completion tokens,
  with N_tok = sum_t m_t clamped to at least 1;
* l_t = beta * KL_t - A_s (the value of -(ratio * A - beta * KL), ratio = 1);
* KL_t = exp(ref - q) - (ref - q) - 1, written expm1(d) - d with d = ref - q;
* A_s = (r_s - mean) / (std + eps) with the unbiased std and eps = 1e-4, rewards
  of the K reward functions summed first, in the fixed fp32 order below;
* one lm_head W serves policy and reference; only the policy path is
  differentiated, so X_p and the reference log-probs get no gradient;
* rows with mask 0 are never read; their outputs are 0.

Loss variants (the experiments of [Long-context GRPO, §4], see Variant): the KL
estimator with the roles of P and Q swapped (forward KL), the reverse estimator
with the extra Q(y) factor, the ratio without its stop-gradient, a mean over
sequences instead of tokens, and a softmax temperature.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------------------
# Advantages
# --------------------------------------------------------------------------------------

def group_advantages(rewards, eps: float = 1e-4, unbiased: bool = True) -> np.ndarray:
    """Group-relative advantages in fp32, in one fixed order of operations.

    For each prompt b: each response's score is the sum of its K reward-function
    scores (k ascending); mean = (sum over g ascending) / G; the squared
    deviations are summed g ascending with no fused multiply-add; std is the
    correctly rounded sqrt of that sum / (G - 1) (G with ``unbiased=False``);
    A = (r - mean) / (std + eps).  Every step rounds to fp32 nearest-even, so a
    GPU that performs the same operations in the same order matches bit for bit.
    [Train your own R1 reasoning model with Unsloth, §3; Long-context GRPO, §4]

    Pinned by tests/test_oracle_pins.py::test_advantages_* (closed forms, torch.std,
    exact zero for equal rewards, K-sum).
    """
    r = np.asarray(rewards, dtype=F32)
    if r.ndim == 2:
        r = r[:, :, None]
    B, G, K = r.shape
    if G < 1 or K < 1 or (unbiased and G < 2):
        raise ValueError("need G >= 2 for the unbiased std and K >= 1")
    e = F32(eps)
    out = np.empty(B * G, dtype=F32)
    for b in range(B):
        score = []
        for g in range(G):
            acc = r[b, g, 0]
            for k in range(1, K):
                acc = F32(acc + r[b, g, k])
            score.append(acc)
        total = F32(0.0)
        for g in range(G):
            total = F32(total + score[g])
        mean = F32(total / F32(G))
        sq = F32(0.0)
        for g in range(G):
            d = F32(score[g] - mean)
            sq = F32(sq + F32(d * d))
        var = F32(sq / F32(G - 1 if unbiased else G))
        std = F32(np.sqrt(var))
        den = F32(std + e)
        for g in range(G):
            out[b * G + g] = F32(F32(score[g] - mean) / den)
    return out


# --------------------------------------------------------------------------------------
# Per-token pieces
# --------------------------------------------------------------------------------------

def log_softmax_rows(z: np.ndarray):
    """Row-wise log-softmax of fp64 logits by the logsumexp trick: subtract the
    row max before exponentiating [Long-context GRPO, §4].  Returns
    (log-probs, lse).  Pinned by test_logsoftmax_normalised and the brute force."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    return z - lse[:, None], lse


def reverse_kl_k3(q: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-token estimator of KL(Q || P) from the sampled token's log-probs under
    the policy (q) and the reference (ref): exp(ref - q) - (ref - q) - 1, with no
    extra Q factor [Long-context GRPO, §3 and §4].  Its expectation under y ~ Q is
    the reverse KL.  Pinned by test_kl_direction_exact_expectation."""
    d = np.asarray(ref, dtype=np.float64) - np.asarray(q, dtype=np.float64)
    return np.expm1(d) - d


def forward_kl_k3(q: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """The same estimator with the roles of policy and reference swapped,
    exp(q - ref) - (q - ref) - 1: its expectation under y ~ P is the forward KL(P || Q)
    (the "forward KL instead" experiment of [Long-context GRPO, §4]).  Pinned by
    test_forward_kl_exact_expectation."""
    d = np.asarray(q, dtype=np.float64) - np.asarray(ref, dtype=np.float64)
    return np.expm1(d) - d


def reverse_kl_q(q: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """The reverse estimator multiplied by the policy probability of the sampled token,
    Q(y) * (exp(ref - q) - (ref - q) - 1): the reading implemented for the "full reverse KL
    with the extra Q term" experiment of [Long-context GRPO, §4], whose formula did not
    survive.  Its gradient is pinned by finite differences."""
    return np.exp(np.asarray(q, dtype=np.float64)) * reverse_kl_k3(q, ref)


def logits(x, W, tau: float = 1.0) -> np.ndarray:
    """Softmax argument of the rows x: x W^T / tau."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T / tau


def advantage_term(a, detach: bool):
    """The advantage's contribution to d loss / d q: -A through exp(q - sg(q)), whose
    gradient is the ratio times dq; nothing through exp(q - q), which is constant."""
    return -np.asarray(a, dtype=np.float64) if detach else np.zeros_like(a, dtype=np.float64)


def grad_factor(grad_loss: float, loss_scale: float, tau: float) -> float:
    """Per-row factor of the backward: grad_loss / loss_scale times the 1 / tau that
    d(z / tau)/dz contributes."""
    return float(grad_loss) / float(loss_scale) / float(tau)


E4M3_MAX = 448.0


def e4m3_round(y) -> np.ndarray:
    """Round to the nearest fp8 e4m3 (fn) value, ties to even, for |y| <= 448: 3 fraction
    bits for |y| >= 2^-6, steps of 2^-9 below.  Pinned against torch's float8_e4m3fn cast
    by test_e4m3_round_matches_torch."""
    y = np.asarray(y)
    if y.dtype != np.float32:
        y = y.astype(np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX):
        raise ValueError("value outside the e4m3 range")
    # a = m 2^e with m in [0.5, 1): the step is 2^(max(e - 1, -6) - 3); every operation
    # below is exact, the rounding is the one rint
    _, e = np.frexp(a)
    step = np.maximum(e - 1, -6) - 3
    q = np.ldexp(np.rint(np.ldexp(a, -step)), step)
    return np.copysign(q, y).astype(np.float64)     # the sign of zero is kept


def e4m3_codes(v) -> np.ndarray:
    """Byte codes of e4m3 (fn) values (sign, 4 exponent bits with bias 7, 3 fraction bits;
    exponent field 0 holds the subnormals k 2^-9; a negative value that rounds to zero is
    -0, code 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)   # -0 keeps its sign
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    sub = a < 2.0 ** -6
    code_sub = np.rint(a * 512.0).astype(np.int64)
    frac = np.rint((a / 2.0 ** e - 1.0) * 8.0).astype(np.int64)
    code_norm = ((e + 7) << 3) | frac
    return (sign | np.where(sub, code_sub, code_norm)).astype(np.uint8)


def quantize_e4m3_rows(x, codes: bool = True):
    """Per-row fp8 quantisation: amax = max |x| of the row (fp32), inv = 448 / amax and
    s = amax / 448 (fp32 divisions; 1 and 1 for an all-zero row), q = e4m3_round(x * inv)
    with the product rounded to fp32.  Returns (q as float64 values, codes uint8 [rows, H]
    or None, s float32 [rows]); the dequantised row is q * s."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    one = np.float32(1.0)
    inv = np.where(nz, np.float32(E4M3_MAX) / np.where(nz, amax, one), one).astype(np.float32)
    s = np.where(nz, amax / np.float32(E4M3_MAX), one).astype(np.float32)
    y = (x * inv[:, None]).astype(np.float32)
    q = e4m3_round(np.copysign(np.minimum(np.abs(y), np.float32(E4M3_MAX)), y))
    return q, (e4m3_codes(q) if codes else None), s


def dequantize_e4m3_rows(x, block: int = 128) -> np.ndarray:
    """x rounded through the per-row fp8 quantisation, as float64 (rows in blocks)."""
    x = np.asarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    for i in range(0, x.shape[0], block):
        q, _, s = quantize_e4m3_rows(x[i:i + block], codes=False)
        out[i:i + block] = q * s.astype(np.float64)[:, None]
    return out


@dataclass(frozen=True)
class Variant:
    """Loss variant: KL estimator ("reverse", "forward", "reverse_q"), whether the ratio's
    stop-gradient is kept, normalisation ("tokens" or "sequences"), the temperature the
    logits are divided by, and fp8 logits (both sides' logits from per-row e4m3 copies of
    X and W; the gradients' products use the original X and W, the straight-through
    reading).  The default is the loss of [Long-context GRPO, §4]."""
    kl: str = "reverse"
    detach: bool = True
    norm: str = "tokens"
    temperature: float = 1.0
    fp8_logits: bool = False


DEFAULT = Variant()


def kl_value(v: Variant, q, ref):
    return {"reverse": reverse_kl_k3, "forward": forward_kl_k3, "reverse_q": reverse_kl_q}[v.kl](q, ref)


def kl_grad_q(v: Variant, q, ref):
    """d KL / d q of the chosen estimator (written out from its definition)."""
    q = np.asarray(q, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if v.kl == "reverse":
        return -np.expm1(ref - q)
    if v.kl == "forward":
        return np.expm1(q - ref)
    if v.kl == "reverse_q":     # d/dq [e^q (e^(ref-q) - (ref-q) - 1)] = (q - ref) e^q
        return (q - ref) * np.exp(q)
    raise ValueError(v.kl)


def token_weights(mask, L: int, norm: str) -> np.ndarray:
    """Weight of each loss token in the loss: 1 / N_tok for the token mean; for the
    sequence mean 1 / (n_s * S'), n_s the loss tokens of the row's sequence and S' the
    sequences that have any.  Zero for masked rows."""
    m = np.asarray(mask).reshape(-1).astype(np.float64)
    if norm == "tokens":
        return m / max(1.0, m.sum())
    if norm == "sequences":
        per = m.reshape(-1, L).sum(1)
        nseq = max(1.0, float((per > 0).sum()))
        w = np.zeros_like(m)
        rows = np.nonzero(m)[0]
        w[rows] = 1.0 / (per[rows // L] * nseq)
        return w
    raise ValueError(norm)


def token_loss(kl: np.ndarray, adv_tok: np.ndarray, beta: float) -> np.ndarray:
    """Per-token loss value beta * KL - A: the value of -(exp(q - sg(q)) * A - beta * KL)
    with the ratio equal to 1 [Long-context GRPO, §4].  Pinned by
    test_policy_equals_reference and the brute force."""
    return beta * kl - adv_tok


def policy_grad(adv_tok: np.ndarray, q: np.ndarray, ref: np.ndarray, beta: float,
                n_tok: float) -> np.ndarray:
    """d loss / d q per loss token: (-A - beta * (exp(ref - q) - 1)) / N_tok.  The
    ratio contributes A * dq (its value is 1, its gradient is not zero) and the
    estimator contributes beta * (1 - exp(ref - q)) [Long-context GRPO, §4].
    Pinned by test_g_matches_surrogate_fd and the brute force."""
    return (-adv_tok - beta * np.expm1(ref - q)) / n_tok


def logit_grad(logp: np.ndarray, y: np.ndarray) -> np.ndarray:
    """d q / d z for the sampled token y of each row: onehot(y) - softmax(z).
    Pinned by test_dx_dw_finite_differences and test_cross_entropy_reduction."""
    T = -np.exp(logp)
    T[np.arange(len(y)), y] += 1.0
    return T


def surrogate_objective(q, q0, ref, adv_tok, mask, beta: float, variant: Variant = DEFAULT,
                        L: int | None = None) -> float:
    """The GRPO objective as autograd sees it: sum over loss tokens of
    w_t * (-A * ratio + beta * KL(q, ref)), with ratio = exp(q - q0) and q0 a frozen copy of
    q (or exp(q - q) = 1 without the stop-gradient), w_t the token weights.  At q = q0 its
    value is the loss; its gradient in q is the policy gradient.  [Long-context GRPO, §4]
    Used by the finite-difference pins."""
    q = np.asarray(q, dtype=np.float64)
    m = np.asarray(mask, dtype=np.float64)
    if variant.norm == "tokens":
        w = m / max(1.0, float(m.sum()))
    else:
        w = token_weights(m, L, variant.norm)
    ratio = np.exp(q - np.asarray(q0, dtype=np.float64)) if variant.detach else np.ones_like(q)
    terms = -np.asarray(adv_tok, dtype=np.float64) * ratio + beta * kl_value(variant, q, ref)
    return float((w * terms).sum())


# --------------------------------------------------------------------------------------
# Forward and backward, materialising full rows of logits
# --------------------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: promote exactly via float64
        import torch
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _finite(a) -> bool:
    return bool(np.all(np.isfinite(a)))


def forward(xq, xp, W, targets, mask, adv, L: int, beta: float = 0.04, rows=None,
            block: int = 256, variant: Variant = DEFAULT) -> dict:
    """Loss and per-token terms.

    Arguments: xq, xp hidden states [N, H] (or only the rows listed in ``rows``,
    in that order); W [V, H]; targets int [N]; mask {0,1} [N]; adv fp32 [S] (one
    per sequence, broadcast over its L tokens); L positions per sequence;
    ``variant`` the loss variant (default: the loss of [Long-context GRPO, §4]).

    Returns per-row arrays of length N (zero for masked rows and, in sampled
    mode, for rows not listed): ``lse_q``, ``logp`` (q), ``ref_logp``, ``kl``,
    ``ell`` (beta*KL - A), ``g`` (d loss / d q); plus ``n_tok``, ``loss`` (None in
    sampled mode), ``rows`` (the rows computed) and ``inputs_finite``.
    """
    targets = np.asarray(targets).reshape(-1)
    mask = np.asarray(mask).reshape(-1).astype(np.int64)
    N = mask.shape[0]
    adv = np.asarray(adv, dtype=F32).reshape(-1)
    Wd = _f64(W)
    V = Wd.shape[0]
    n_tok = int(mask.sum())
    wts = token_weights(mask, L, variant.norm)
    tau = float(variant.temperature)
    Wl = dequantize_e4m3_rows(Wd) if variant.fp8_logits else Wd
    loss_rows = np.nonzero(mask)[0]
    if rows is None:
        rows = loss_rows
        xq_rows = _f64(xq)[rows]
        xp_rows = _f64(xp)[rows]
        full = True
    else:
        rows = np.asarray(rows, dtype=np.int64)
        xq_rows, xp_rows = _f64(xq), _f64(xp)
        assert xq_rows.shape[0] == len(rows)
        full = False
    out = {k: np.zeros(N) for k in ("lse_q", "logp", "ref_logp", "kl", "ell", "g")}
    finite = _finite(Wd) and _finite(adv)
    for i0 in range(0, len(rows), block):
        sel = slice(i0, i0 + block)
        r = rows[sel]
        keep = mask[r] == 1                     # masked rows are not read
        r = r[keep]
        if len(r) == 0:
            continue
        y = targets[r]
        if np.any((y < 0) | (y >= V)):
            raise ValueError("target id outside [0, V) on a loss token")
        xq_b = xq_rows[sel][keep]
        xp_b = xp_rows[sel][keep]
        finite = finite and _finite(xq_b) and _finite(xp_b)
        if variant.fp8_logits:
            xq_b, xp_b = dequantize_e4m3_rows(xq_b), dequantize_e4m3_rows(xp_b)
        lp_q, lse_q = log_softmax_rows(logits(xq_b, Wl, tau))
        lp_p, _ = log_softmax_rows(logits(xp_b, Wl, tau))
        q = lp_q[np.arange(len(r)), y]
        ref = lp_p[np.arange(len(r)), y]
        kl = kl_value(variant, q, ref)
        a = adv[r // L].astype(np.float64)
        out["lse_q"][r] = lse_q
        out["logp"][r] = q
        out["ref_logp"][r] = ref
        out["kl"][r] = kl
        out["ell"][r] = token_loss(kl, a, beta)
        if variant == DEFAULT:
            out["g"][r] = policy_grad(a, q, ref, beta, float(max(1, n_tok)))
        else:
            out["g"][r] = wts[r] * (advantage_term(a, variant.detach)
                                    + beta * kl_grad_q(variant, q, ref))
    out["n_tok"] = n_tok
    out["rows"] = rows
    if not full:
        out["loss"] = None
    elif variant.norm == "tokens":
        out["loss"] = float(out["ell"][loss_rows].sum() / max(1, n_tok))
    else:
        out["loss"] = float((wts[loss_rows] * out["ell"][loss_rows]).sum())
    out["variant"] = variant
    out["inputs_finite"] = finite
    return out


def backward(xq, W, targets, mask, fwd: dict, grad_loss: float = 1.0,
             loss_scale: float = 1.0, need_dW: bool = False, rows=None,
             block: int = 256) -> dict:
    """Gradients of the loss with respect to X_q (and W), from ``forward``'s g.

    dX_q[t] = c * g_t * (onehot(y_t) - P_t) @ W and dW = sum_t c * g_t *
    (onehot(y_t) - P_t)^T x_q[t], where P_t is the softmax of row t's policy
    logits and c = grad_loss / loss_scale (an fp16 caller back-propagates the
    loss scaled by S and passes S for both, so the gradients come back
    unscaled).  Rows with mask 0 get zero.  ``rows``/``xq`` follow ``forward``'s
    convention; dW needs every loss row.

    Also reports ``naive_fp16_overflow``: whether a path that formed the scaled
    logit gradient grad_loss * g_t * (onehot - P) in fp16 would overflow (any
    magnitude >= 65520) — the mixed-precision hazard [Long-context GRPO, §3].
    """
    targets = np.asarray(targets).reshape(-1)
    mask = np.asarray(mask).reshape(-1).astype(np.int64)
    Wd = _f64(W)
    V, H = Wd.shape
    variant = fwd.get("variant", DEFAULT)
    tau = float(variant.temperature)
    # dq/dz = (onehot - softmax(z / tau)) / tau: the 1/tau joins the per-row factor
    c = grad_factor(grad_loss, loss_scale, tau)
    Wl = dequantize_e4m3_rows(Wd) if variant.fp8_logits else Wd
    if rows is None:
        rows = np.nonzero(mask)[0]
        xq_rows = _f64(xq)[rows]
        full = True
    else:
        rows = np.asarray(rows, dtype=np.int64)
        xq_rows = _f64(xq)
        full = False
    if need_dW and not full:
        raise ValueError("dW needs every loss row")
    dX = np.zeros((len(rows), H))
    dW = np.zeros((V, H)) if need_dW else None
    worst = 0.0
    for i0 in range(0, len(rows), block):
        sel = slice(i0, i0 + block)
        r = rows[sel]
        keep = np.nonzero(mask[r] == 1)[0]
        if len(keep) == 0:
            continue
        rk = r[keep]
        x = xq_rows[sel][keep]
        xl = dequantize_e4m3_rows(x) if variant.fp8_logits else x
        lp, _ = log_softmax_rows(logits(xl, Wl, tau))
        T = logit_grad(lp, targets[rk])
        gt = fwd["g"][rk]
        worst = max(worst, float(np.max(np.abs(gt * float(grad_loss) / tau)[:, None] * np.abs(T))))
        dX[i0 + keep] = (c * gt)[:, None] * (T @ Wd)
        if need_dW:
            dW += ((c * gt)[:, None] * T).T @ x
    finite = _finite(dX) and (dW is None or _finite(dW))
    return {"dX": dX, "dW": dW, "rows": rows, "outputs_finite": finite,
            "naive_fp16_overflow": worst >= 65520.0, "naive_max_abs": worst}


def dw_rows(xq, W, targets, mask, fwd: dict, vrows, grad_loss: float = 1.0,
            loss_scale: float = 1.0, block: int = 1024) -> np.ndarray:
    """Rows ``vrows`` of dW = sum_t c * g_t * (onehot(y_t) - P_t)^T x_q[t], summed over
    every loss row t, without forming the other rows of dW: P_tv = exp(z_tv / tau - lse_t)
    needs only the selected vocabulary columns of each row's logits once lse_t is known,
    and ``fwd``'s lse_q holds it from the row's full vocabulary.  The same definition as
    ``backward``'s dW, read one row of W at a time, for vocabulary sizes where the full
    [V, H] product is too slow to check.  xq: the loss rows in ascending order (the rows
    ``fwd`` computed); c = grad_loss / loss_scale / tau.  Returns [len(vrows), H] fp64.
    Pinned by test_pin[pin_dx_dw_finite_differences] and test_dw_rows_match_backward.
    """
    targets = np.asarray(targets).reshape(-1)
    mask = np.asarray(mask).reshape(-1).astype(np.int64)
    vrows = np.asarray(vrows, dtype=np.int64)
    variant = fwd.get("variant", DEFAULT)
    tau = float(variant.temperature)
    c = grad_factor(grad_loss, loss_scale, tau)
    Wd = _f64(W)
    Wv = Wd[vrows]
    Wl = dequantize_e4m3_rows(Wd)[vrows] if variant.fp8_logits else Wv
    rows = np.nonzero(mask)[0]
    X = _f64(xq)
    if X.shape[0] != len(rows):
        raise ValueError("xq must hold the loss rows, in order")
    out = np.zeros((len(vrows), Wd.shape[1]))
    for i0 in range(0, len(rows), block):
        r = rows[i0:i0 + block]
        x = X[i0:i0 + block]
        xl = dequantize_e4m3_rows(x) if variant.fp8_logits else x
        z = logits(xl, Wl, tau)                                   # [rows, len(vrows)]
        T = (targets[r][:, None] == vrows[None, :]).astype(np.float64)
        T -= np.exp(z - fwd["lse_q"][r][:, None])
        out += (T * (c * fwd["g"][r])[:, None]).T @ x
    return out


def found_inf(fwd: dict, bwd: dict | None = None) -> bool:
    """The non-finite predicate a mixed-precision caller needs: anything read on a
    loss row, the loss, g, dX or dW is inf/NaN."""
    ok = fwd["inputs_finite"] and _finite(fwd["g"])
    if fwd["loss"] is not None:
        ok = ok and np.isfinite(fwd["loss"])
    if bwd is not None:
        ok = ok and bwd["outputs_finite"]
    return not ok
