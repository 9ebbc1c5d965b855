"""CPU fp64 oracle of the LaCT fast-weight layer forward (update + apply).

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Sources (page title, then the labelled part of the page):
  [LaCT-IPLEX] "LaCT：以大分块更新人工智能的临时记忆" (iplexlaw.co.kr blog):
      "局部注意力与非线性记忆相互补充" -- the memory is a three-matrix SwiGLU
      MLP; its loss is the negative inner product of the network output on
      the key with the value; per-token learning rates weight a gradient
      summed over the chunk; queries read the fast weights; GD, momentum and
      Muon (Newton-Schulz) are the update rules; the weights are
      L2-normalised after the update.
      "更新顺序必须遵守信息可见范围" -- language models apply the memory of
      earlier chunks to the current chunk before updating with it; posed
      image sets update first, then read target views; video updates only
      from clean chunks, noisy chunks read what was accumulated before.
  [LaCT-DPSHK] "大块测试时训练（LaCT）技术解析" (dpshk.com):
      §2.1 -- update phase sums the gradient over the whole chunk (eqs. 4-5),
      apply phase runs the updated weights on all queries (eq. 2);
      §2.2.1 -- L2 weight normalisation (eq. 8) and Muon via an approximate
      orthogonalisation of the gradient (eqs. 9-10).
  [LaCT-GSYQ] "LaCT架构核心思想解析" (gsyq.cn):
      §1.2 -- three fast-weight matrices per layer; momentum with a per-token
      beta: M is scaled by the chunk mean of beta and the gradient is added,
      then W <- L2norm(W - M); q and k pass through silu and are divided by
      their norm over d before use; §2.1 -- lr is [b, l, 3 * nh] rearranged
      to [(b nh), l, 3]; the layer output is multiplied per head and token by
      silu of a linear projection of the input (one scalar per token).

Conventions (readings where the pages are silent; each is listed in the
design notes):
  * per instance, W1, W3 are [dh, d] and W2 is [d, dh];
    f_W(x) = W2 (silu(W1 x) * (W3 x));
  * lr column j-1 scales the gradient of W_j;
  * U_j = -sum_i lr_ij dl_i/dW_j with l_i = -<f_W(k_i), v_i>  (a sum over the
    chunk, not a mean);
  * GD: W' = W + U.  Momentum: M <- mean_chunk(beta) M - U, W' = W - M.
    Muon: W' = W + NS5(U) with the quintic coefficients published with the
    Muon optimiser (3.4445, -4.7750, 2.0315), X0 = U / (||U||_F + 1e-7), five
    iterations, no extra step scale;
  * renorm: each row of W' (one output unit's fan-in vector: rows of the
    stored matrices) is rescaled to the norm that row had before the update;
  * order: apply-then-update (shifted block-causal) or update-then-apply;
    chunks flagged apply-only read the current weights; the last chunk's
    update is still performed and returned as state.

Everything is float64; inputs are first decoded exactly (bf16 bit patterns
given as uint16 are widened).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

UPDATE = 1
APPLY = 2
APPLY_THEN_UPDATE = 0
UPDATE_THEN_APPLY = 1
OPT_GD = 0
OPT_MOMENTUM = 1
OPT_MUON = 2
OPT_MUON_MOMENTUM = 3

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7


def f64(x) -> np.ndarray:
    """Exact float64 value of an input array (uint16 means bf16 bits)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ------------------------------------------------------------ activations

def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def silu_prime(x):
    """d/dx [x sigmoid(x)] = sigmoid(x) (1 + x (1 - sigmoid(x)))."""
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# ------------------------------------------------------------ apply (eq. 2)

def apply(W1, W2, W3, X):
    """Run the fast-weight SwiGLU MLP on the rows of X ([T, d] -> [T, d]).
    [LaCT-DPSHK] §2.1 apply phase; [LaCT-IPLEX] SwiGLU memory."""
    A = X @ W1.T
    B = X @ W3.T
    return (silu(A) * B) @ W2.T


# ------------------------------------------------------------ update (eqs. 4-5)

def chunk_grads(W1, W2, W3, K, V, lr):
    """Chunk-summed, lr-weighted descent directions U1, U2, U3.

    U_j = -sum_i lr[i, j-1] * d l_i / d W_j,  l_i = -<f_W(k_i), v_i>.
    With A = K W1^T, B = K W3^T, G = V W2 (row i is W2^T v_i):
        U1 = (lr1 * G * B * silu'(A))^T K      [dh, d]
        U3 = (lr3 * G * silu(A))^T K           [dh, d]
        U2 = (lr2 * V)^T (silu(A) * B)         [d, dh]
    [LaCT-DPSHK] §2.1 (sum over the chunk); [LaCT-IPLEX] loss and per-token lr.
    """
    A = K @ W1.T
    B = K @ W3.T
    G = V @ W2
    S = silu(A)
    H = S * B
    e1, e2, e3 = lr[:, 0:1], lr[:, 1:2], lr[:, 2:3]
    U1 = (e1 * G * B * silu_prime(A)).T @ K
    U3 = (e3 * G * S).T @ K
    U2 = (e2 * V).T @ H
    return U1, U2, U3


# ------------------------------------------------------------ optimisers

def newton_schulz5(G, steps: int = 5, coeffs=NS_COEFFS, eps: float = NS_EPS):
    """Muon's quintic Newton-Schulz map ([LaCT-DPSHK] §2.2.1, eqs. 9-10):
    X <- G / (||G||_F + eps); repeat: A = X X^T, B = b A + c A A,
    X <- a X + B X.  Works on the transpose when G has more rows than
    columns, so that X X^T is the smaller Gram matrix."""
    a, b, c = coeffs
    X = G / (np.linalg.norm(G) + eps)
    tr = X.shape[0] > X.shape[1]
    if tr:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tr else X


def momentum_step(M, U, beta_mean):
    """M <- mean(beta) M + g with g = -U ([LaCT-GSYQ] §1.2); returns new M,
    which is also the step: W' = W - M."""
    return beta_mean * M - U


def renorm_rows(W_new, W_old):
    """Row-wise L2 weight normalisation ([LaCT-DPSHK] §2.2.1, eq. 8;
    [LaCT-GSYQ] §1.2): every row of W_new gets the norm its row had in
    W_old, so row norms are invariant across updates."""
    n_old = np.linalg.norm(W_old, axis=1, keepdims=True)
    n_new = np.linalg.norm(W_new, axis=1, keepdims=True)
    return W_new * (n_old / n_new)


def update_step(W, M, K, V, lr, beta, opt, renorm=True, ns_steps=5):
    """One chunk update of the state (W1, W2, W3), (M1, M2, M3)."""
    W1, W2, W3 = W
    U = chunk_grads(W1, W2, W3, K, V, lr)
    if opt == OPT_GD:
        Wn = [w + u for w, u in zip(W, U)]
        Mn = M
    elif opt == OPT_MOMENTUM:
        bm = float(np.mean(beta))
        Mn = [momentum_step(m, u, bm) for m, u in zip(M, U)]
        Wn = [w - m for w, m in zip(W, Mn)]
    elif opt == OPT_MUON:
        Wn = [w + newton_schulz5(u, ns_steps) for w, u in zip(W, U)]
        Mn = M
    elif opt == OPT_MUON_MOMENTUM:
        # momentum with per-token beta ([LaCT-GSYQ] §1.2) whose buffer is then
        # orthogonalised ([LaCT-DPSHK] §2.2.1, eqs. 9-10) -- the two options
        # combined by orthogonalising the momentum buffer (reading: the
        # pages list the options separately; this composition reduces to
        # Muon when beta = 0)
        bm = float(np.mean(beta))
        Mn = [momentum_step(m, u, bm) for m, u in zip(M, U)]
        Wn = [w - newton_schulz5(m, ns_steps) for w, m in zip(W, Mn)]
    else:
        raise ValueError(f"unknown optimiser {opt}")
    if renorm:
        Wn = [renorm_rows(wn, w) for wn, w in zip(Wn, W)]
    return Wn, Mn


# ------------------------------------------------------------ input / output scaling

def qk_preprocess(x):
    """[LaCT-GSYQ] §1.2: silu, then each token's vector divided by its L2
    norm over d (no epsilon is printed; none is added)."""
    s = silu(f64(x))
    return s / np.sqrt(np.sum(s * s, axis=-1, keepdims=True))


def output_scale(o, z):
    """[LaCT-GSYQ] §2.1: per-token output scale silu(z) of a given
    pre-activation z [L] (the projection itself is outside the layer)."""
    return o * silu(f64(z))[:, None]


# ------------------------------------------------------------ layer

def forward_instance(q, k, v, lr, beta, W1, W2, W3, bounds: Sequence[int],
                     flags: Sequence[int], order: int, opt: int, renorm=True,
                     M=None, ns_steps=5, qk_prep=False, oz=None):
    """One instance ([L, D] inputs) through the chunk schedule.  qk_prep: q
    and k are raw and pre-processed first; oz: per-token output-scale
    pre-activation [L] (or None).

    Returns dict(o [L, D] float64 with zeros on rows of non-APPLY chunks,
    o_mask [L] bool, W1, W2, W3, M1, M2, M3 (final state))."""
    q, k, v, lr = f64(q), f64(k), f64(v), f64(lr)
    if qk_prep:
        q, k = qk_preprocess(q), qk_preprocess(k)
    beta = None if beta is None else f64(beta)
    W = [f64(W1), f64(W2), f64(W3)]
    if M is None:
        M = [np.zeros_like(w) for w in W]
    else:
        M = [f64(m) for m in M]
    L, D = q.shape
    o = np.zeros((L, D))
    mask = np.zeros(L, dtype=bool)
    for c in range(len(flags)):
        a, b = int(bounds[c]), int(bounds[c + 1])
        f = int(flags[c])
        if (f & APPLY) and (order == APPLY_THEN_UPDATE or not (f & UPDATE)):
            o[a:b] = apply(W[0], W[1], W[2], q[a:b])
            mask[a:b] = True
        if f & UPDATE:
            bt = None if beta is None else beta[a:b]
            W, M = update_step(W, M, k[a:b], v[a:b], lr[a:b], bt, opt, renorm, ns_steps)
        if (f & APPLY) and order == UPDATE_THEN_APPLY and (f & UPDATE):
            o[a:b] = apply(W[0], W[1], W[2], q[a:b])
            mask[a:b] = True
    if oz is not None:
        o = output_scale(o, oz)
    return {"o": o, "o_mask": mask, "W1": W[0], "W2": W[1], "W3": W[2],
            "M1": M[0], "M2": M[1], "M3": M[2]}


def layer_forward(q, k, v, lr, beta, W1, W2, W3, bounds, flags, order, opt,
                  renorm=True, M=None, ns_steps=5) -> Dict[str, np.ndarray]:
    """All instances ([n, L, D] inputs); instances are independent."""
    n = q.shape[0]
    outs = []
    for i in range(n):
        Mi = None if M is None else [m[i] for m in M]
        outs.append(forward_instance(q[i], k[i], v[i], lr[i],
                                     None if beta is None else beta[i],
                                     W1[i], W2[i], W3[i], bounds, flags, order, opt,
                                     renorm, Mi, ns_steps))
    return {key: np.stack([o[key] for o in outs]) for key in outs[0]}
