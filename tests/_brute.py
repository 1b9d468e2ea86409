"""Scalar brute force of the GRPO loss for tiny shapes: plain Python loops and the
math module, no BLAS and no NumPy, written independently of the oracle so the
two can pin each other.  Everything follows the definitions: logits are dot
products, log-probs subtract a max-shifted logsumexp, the KL estimator is
exp(ref - q) - (ref - q) - 1, the per-token loss is beta * KL - A, the loss is the
mean over loss tokens, and the gradients differentiate -A * exp(q - q0) +
beta * KL at q = q0 [Long-context GRPO, §4]."""

import math


def brute(xq, xp, W, y, m, adv, L, beta, need_dW=True):
    N = len(xq)
    H = len(xq[0]) if N else 0
    V = len(W)
    n_tok = sum(1 for t in range(N) if m[t])
    denom = float(max(1, n_tok))
    res = {"logp": [0.0] * N, "ref": [0.0] * N, "kl": [0.0] * N, "g": [0.0] * N,
           "dX": [[0.0] * H for _ in range(N)], "dW": [[0.0] * H for _ in range(V)]}
    total = 0.0
    for t in range(N):
        if not m[t]:
            continue

        def logits(x):
            return [sum(x[h] * W[v][h] for h in range(H)) for v in range(V)]

        zq, zp = logits(xq[t]), logits(xp[t])
        mq, mp = max(zq), max(zp)
        lse_q = mq + math.log(sum(math.exp(z - mq) for z in zq))
        lse_p = mp + math.log(sum(math.exp(z - mp) for z in zp))
        q = zq[y[t]] - lse_q
        ref = zp[y[t]] - lse_p
        kl = math.exp(ref - q) - (ref - q) - 1.0
        a = adv[t // L]
        total += beta * kl - a
        g = (-a + beta * (1.0 - math.exp(ref - q))) / denom
        res["logp"][t], res["ref"][t], res["kl"][t], res["g"][t] = q, ref, kl, g
        for v in range(V):
            tv = (1.0 if v == y[t] else 0.0) - math.exp(zq[v] - lse_q)
            for h in range(H):
                res["dX"][t][h] += g * tv * W[v][h]
                if need_dW:
                    res["dW"][v][h] += g * tv * xq[t][h]
    res["loss"] = total / denom
    res["n_tok"] = n_tok
    return res
