"""CPU fp64 oracle of the LaCT layer's backward pass (reverse mode through the
chunk recurrence).

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What is differentiated is exactly the forward computation of
`lact_oracle.forward_instance` (same sources: [LaCT-DPSHK] §2.1 update and
apply phases, eqs. 2 and 4-5; §2.2.1 L2 weight normalisation, eq. 8, and the
Newton-Schulz orthogonalisation, eqs. 9-10; [LaCT-GSYQ] §1.2 momentum with a
per-token beta; [LaCT-IPLEX] the apply/update orders).  The pages train the
layer end to end (the throughput figures of [LaCT-IPLEX] "语言模型的质量与吞吐量"
are training rates) but print no backward formulas: every derivative below
is the ordinary chain rule applied to those forward steps, written out by
hand.

The scalar being differentiated is
    J = sum(dO * o) + sum_j sum(gW_j * W_j(final)) + sum_j sum(gM_j * M_j(final))
over o's APPLY rows, so the results are the vector-Jacobian products of the
layer with the cotangents dO (output) and gW, gM (final state).  Gradients
are returned for q, k, v, lr, beta and the initial state W0, M0.

Everything is float64.  Pinned by tests/test_oracle_backward.py: central
finite differences of J in random directions for every input, optimiser,
order and renorm setting (including rectangular Newton-Schulz in both
orientations), and closed forms of the linear-attention special case.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

from .lact_oracle import (APPLY, APPLY_THEN_UPDATE, NS_COEFFS, NS_EPS, OPT_GD, OPT_MOMENTUM, OPT_MUON,
                          OPT_MUON_MOMENTUM, UPDATE, UPDATE_THEN_APPLY, chunk_grads, f64, forward_instance,
                          momentum_step, newton_schulz5, qk_preprocess, sigmoid, silu, silu_prime, update_step)


def silu_second(x):
    """d^2/dx^2 [x sigmoid(x)] = s (1 - s) (2 + x (1 - 2 s)), s = sigmoid(x)."""
    s = sigmoid(x)
    return s * (1.0 - s) * (2.0 + x * (1.0 - 2.0 * s))


# ------------------------------------------------------------ apply (eq. 2)

def apply_vjp(W1, W2, W3, X, dO):
    """Cotangents of X and (W1, W2, W3) for O = (silu(X W1^T) * (X W3^T)) W2^T."""
    A = X @ W1.T
    B = X @ W3.T
    S = silu(A)
    H = S * B
    dH = dO @ W2
    gW2 = dO.T @ H
    dA = dH * B * silu_prime(A)
    dB = dH * S
    dX = dA @ W1 + dB @ W3
    return dX, [dA.T @ X, gW2, dB.T @ X]


# ------------------------------------------------------------ update terms (eqs. 4-5)

def chunk_grads_vjp(W1, W2, W3, K, V, lr, gU):
    """Cotangents of (W1, W2, W3), K, V and lr for the chunk's descent
    directions U1 = E1^T K, U3 = E3^T K, U2 = V^T H2 with A = K W1^T,
    B = K W3^T, G = V W2, E1 = lr1 G B silu'(A), E3 = lr3 G silu(A),
    H2 = lr2 silu(A) B (the terms of `lact_oracle.chunk_grads`).
    gU = (gU1, gU2, gU3)."""
    gU1, gU2, gU3 = gU
    A = K @ W1.T
    B = K @ W3.T
    G = V @ W2
    S, Sp, Spp = silu(A), silu_prime(A), silu_second(A)
    e1, e2, e3 = lr[:, 0:1], lr[:, 1:2], lr[:, 2:3]
    E1 = e1 * G * B * Sp
    E3 = e3 * G * S
    H2 = e2 * S * B
    # through the contractions over the chunk's tokens
    gE1 = K @ gU1.T
    gE3 = K @ gU3.T
    gH2 = V @ gU2
    dK = E1 @ gU1 + E3 @ gU3
    dV = H2 @ gU2.T
    # through the elementwise terms
    gA = gE1 * e1 * G * B * Spp + gE3 * e3 * G * Sp + gH2 * e2 * B * Sp
    gB = gE1 * e1 * G * Sp + gH2 * e2 * S
    gG = gE1 * e1 * B * Sp + gE3 * e3 * S
    dlr = np.stack([np.sum(gE1 * G * B * Sp, axis=1), np.sum(gH2 * S * B, axis=1),
                    np.sum(gE3 * G * S, axis=1)], axis=1)
    # through A = K W1^T, B = K W3^T, G = V W2
    dK = dK + gA @ W1 + gB @ W3
    dV = dV + gG @ W2.T
    return [gA.T @ K, V.T @ gG, gB.T @ K], dK, dV, dlr


# ------------------------------------------------------------ optimisers

def newton_schulz5_vjp(G, gY, steps: int = 5, coeffs=NS_COEFFS, eps: float = NS_EPS):
    """Cotangent of G for Y = newton_schulz5(G) given the cotangent gY.

    Forward per iteration: A = X X^T, P = b A + c A A, X' = a X + P X.
    Reverse: gP = gX' X^T, gA = b gP + c (gP A + A gP) (A and P are
    symmetric), gX = a gX' + P gX' + (gA + gA^T) X.  Normalisation
    X0 = G / (||G|| + eps): gG = gX0 / (||G|| + eps) - G <gX0, G> /
    ((||G|| + eps)^2 ||G||)."""
    a, b, c = coeffs
    nG = float(np.linalg.norm(G))
    X = G / (nG + eps)
    tr = X.shape[0] > X.shape[1]
    if tr:
        X = X.T
        gY = gY.T
    xs = [X]
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
        xs.append(X)
    g = gY
    for i in range(steps - 1, -1, -1):
        X = xs[i]
        A = X @ X.T
        P = b * A + c * (A @ A)
        gP = g @ X.T
        gA = b * gP + c * (gP @ A + A @ gP)
        g = a * g + P @ g + (gA + gA.T) @ X
    if tr:
        g = g.T
    gG = g / (nG + eps)
    if nG > 0:
        gG = gG - G * (float(np.sum(g * G)) / ((nG + eps) ** 2 * nG))
    return gG


def renorm_rows_vjp(W_new, W_old, gY):
    """Cotangents of (W_new, W_old) for Y = W_new * ||W_old_r|| / ||W_new_r||
    row by row: with s = ||W_old_r|| / ||W_new_r|| and w = W_new_r /
    ||W_new_r||, gW_new = s (gY - (gY . w) w) and gW_old = (gY . w) W_old_r /
    ||W_old_r||."""
    n_old = np.linalg.norm(W_old, axis=1, keepdims=True)
    n_new = np.linalg.norm(W_new, axis=1, keepdims=True)
    w = W_new / n_new
    dot = np.sum(gY * w, axis=1, keepdims=True)
    return (n_old / n_new) * (gY - dot * w), dot * W_old / n_old


def update_vjp(W, M, K, V, lr, beta, opt, renorm, gWn, gMn, ns_steps=5):
    """Reverse of `lact_oracle.update_step`: cotangents of the chunk's input
    state (W, M), K, V, lr and beta from those of its output state."""
    W1, W2, W3 = W
    U = chunk_grads(W1, W2, W3, K, V, lr)
    bm = float(np.mean(beta)) if opt in (OPT_MOMENTUM, OPT_MUON_MOMENTUM) else 0.0
    # the pre-normalisation step W' of each matrix
    if opt == OPT_GD:
        Wp = [w + u for w, u in zip(W, U)]
    elif opt == OPT_MOMENTUM:
        Mn = [momentum_step(m, u, bm) for m, u in zip(M, U)]
        Wp = [w - m for w, m in zip(W, Mn)]
    elif opt == OPT_MUON:
        Wp = [w + newton_schulz5(u, ns_steps) for w, u in zip(W, U)]
    elif opt == OPT_MUON_MOMENTUM:
        Mn = [momentum_step(m, u, bm) for m, u in zip(M, U)]
        Wp = [w - newton_schulz5(m, ns_steps) for w, m in zip(W, Mn)]
    else:
        raise ValueError(f"unknown optimiser {opt}")
    # renorm (eq. 8): W_next = renorm(W', W)
    if renorm:
        pairs = [renorm_rows_vjp(wp, w, g) for wp, w, g in zip(Wp, W, gWn)]
        gWp = [p[0] for p in pairs]
        gW = [p[1] + p[0] for p in pairs]          # W' = W +- step: the step term passes gWp to W
    else:
        gWp = [g.copy() for g in gWn]
        gW = [g.copy() for g in gWn]
    dbeta = None
    if opt == OPT_GD:
        gU = gWp
        gM = gMn
    elif opt == OPT_MUON:
        gU = [newton_schulz5_vjp(u, g, ns_steps) for u, g in zip(U, gWp)]
        gM = gMn
    else:
        if opt == OPT_MOMENTUM:
            gMt = [gm - g for gm, g in zip(gMn, gWp)]               # W' = W - M_next
        else:
            gMt = [gm - newton_schulz5_vjp(m, g, ns_steps) for gm, m, g in zip(gMn, Mn, gWp)]
        gM = [bm * g for g in gMt]                                 # M_next = bm M - U
        gbm = float(sum(np.sum(g * m) for g, m in zip(gMt, M)))
        gU = [-g for g in gMt]
        dbeta = np.full(K.shape[0], gbm / K.shape[0])              # bm = mean of the chunk's beta
    gWu, dK, dV, dlr = chunk_grads_vjp(W1, W2, W3, K, V, lr, gU)
    gW = [a + b for a, b in zip(gW, gWu)]
    return gW, gM, dK, dV, dlr, dbeta


# ------------------------------------------------------------ input / output scaling

def qk_preprocess_vjp(x, g):
    """Cotangent of the raw x for x_hat = silu(x) / ||silu(x)|| (per token,
    over d) given the cotangent g of x_hat: with s = silu(x), n = ||s||,
    s_hat = s / n: dx = silu'(x) (g - s_hat (s_hat . g)) / n."""
    x = f64(x)
    s = silu(x)
    n = np.sqrt(np.sum(s * s, axis=-1, keepdims=True))
    sh = s / n
    return silu_prime(x) * (g - sh * np.sum(sh * g, axis=-1, keepdims=True)) / n


# ------------------------------------------------------------ layer

def backward_instance(q, k, v, lr, beta, W1, W2, W3, bounds: Sequence[int], flags: Sequence[int], order: int,
                      opt: int, dO, gW=None, gM=None, renorm=True, M=None, ns_steps=5, qk_prep=False,
                      oz=None) -> Dict[str, np.ndarray]:
    """Reverse mode through one instance's chunk schedule.  dO [L, D] is the
    output cotangent (rows of non-APPLY chunks are ignored); gW, gM the
    cotangents of the final state (None: zero).  qk_prep: q and k are raw
    and the layer pre-processes them; oz [L]: the output rows are scaled by
    silu(oz) (both as in `lact_oracle.forward_instance`).  Returns dq, dk, dv
    [L, D] (of the raw q, k when qk_prep), dlr [L, 3], dbeta [L] (zeros
    without momentum), dW1, dW2, dW3, dM1, dM2, dM3 (cotangents of the
    initial state) and doz [L] (only with oz)."""
    q, k, v, lr, dO = f64(q), f64(k), f64(v), f64(lr), f64(dO)
    q_raw, k_raw = q, k
    if qk_prep:
        q, k = qk_preprocess(q_raw), qk_preprocess(k_raw)
    doz = None
    if oz is not None:
        # o_s = o * silu(z): d z_t = silu'(z_t) <dO_t, o_t>, and o sees dO * silu(z)
        z = f64(oz)
        # the unscaled output of every APPLY row (zero elsewhere), from the forward
        o = forward_instance(q, k, v, lr, beta, W1, W2, W3, bounds, flags, order, opt, renorm, M=M,
                             ns_steps=ns_steps)["o"]
        doz = silu_prime(z) * np.sum(dO * o, axis=1)
        dO = dO * silu(z)[:, None]
    beta = None if beta is None else f64(beta)
    W = [f64(W1), f64(W2), f64(W3)]
    M = [np.zeros_like(w) for w in W] if M is None else [f64(m) for m in M]
    L, D = q.shape
    # forward, keeping the state before every chunk
    states = []
    for c in range(len(flags)):
        states.append((W, M))
        a, b = int(bounds[c]), int(bounds[c + 1])
        if int(flags[c]) & UPDATE:
            bt = None if beta is None else beta[a:b]
            W, M = update_step(W, M, k[a:b], v[a:b], lr[a:b], bt, opt, renorm, ns_steps)
    states.append((W, M))
    gWc = [np.zeros_like(w) for w in W] if gW is None else [f64(g).copy() for g in gW]
    gMc = [np.zeros_like(w) for w in W] if gM is None else [f64(g).copy() for g in gM]
    dq, dk, dv = np.zeros((L, D)), np.zeros((L, D)), np.zeros((L, D))
    dlr, dbeta = np.zeros((L, 3)), np.zeros(L)
    for c in range(len(flags) - 1, -1, -1):
        a, b = int(bounds[c]), int(bounds[c + 1])
        f = int(flags[c])
        Wc, Mc = states[c]
        if (f & APPLY) and (f & UPDATE) and order == UPDATE_THEN_APPLY:
            # o read the state after this chunk's update
            dX, gWa = apply_vjp(*states[c + 1][0], q[a:b], dO[a:b])
            dq[a:b] = dX
            gWc = [g + h for g, h in zip(gWc, gWa)]
        if f & UPDATE:
            bt = None if beta is None else beta[a:b]
            gWc, gMc, dK, dV, dL, dB = update_vjp(Wc, Mc, k[a:b], v[a:b], lr[a:b], bt, opt, renorm, gWc, gMc,
                                                  ns_steps)
            dk[a:b], dv[a:b], dlr[a:b] = dK, dV, dL
            if dB is not None:
                dbeta[a:b] = dB
        if (f & APPLY) and (order == APPLY_THEN_UPDATE or not (f & UPDATE)):
            dX, gWa = apply_vjp(*Wc, q[a:b], dO[a:b])
            dq[a:b] = dX
            gWc = [g + h for g, h in zip(gWc, gWa)]
    if qk_prep:
        dq = qk_preprocess_vjp(q_raw, dq)
        dk = qk_preprocess_vjp(k_raw, dk)
    out = {"dq": dq, "dk": dk, "dv": dv, "dlr": dlr, "dbeta": dbeta,
           "dW1": gWc[0], "dW2": gWc[1], "dW3": gWc[2], "dM1": gMc[0], "dM2": gMc[1], "dM3": gMc[2]}
    if doz is not None:
        out["doz"] = doz
    return out



def layer_backward(q, k, v, lr, beta, W1, W2, W3, bounds, flags, order, opt, dO, gW=None, gM=None, renorm=True,
                   M=None, ns_steps=5, qk_prep=False, oz=None) -> Dict[str, np.ndarray]:
    """All instances ([n, L, D] inputs, [n, ...] state and cotangents)."""
    n = q.shape[0]
    outs = []
    for i in range(n):
        pick = lambda xs: None if xs is None else [x[i] for x in xs]
        outs.append(backward_instance(q[i], k[i], v[i], lr[i], None if beta is None else beta[i],
                                      W1[i], W2[i], W3[i], bounds, flags, order, opt, dO[i],
                                      pick(gW), pick(gM), renorm, pick(M), ns_steps, qk_prep,
                                      None if oz is None else oz[i]))
    return {key: np.stack([o[key] for o in outs]) for key in outs[0]}
