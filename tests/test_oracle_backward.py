"""Pins of the fp64 backward oracle against things other than itself:

* central finite differences of the forward oracle's scalar
  J = sum(dO * o) + sum(gW * W_final) + sum(gM * M_final) in random
  directions, for every input, optimiser, order and renorm setting, with
  square and rectangular (both Newton-Schulz orientations) fast weights and
  a schedule holding update+apply, apply-only and update-only chunks;
* the linear-attention special case (GD, no renorm, lr1 = lr3 = 0, one
  update-then-apply chunk), whose gradients have a closed form in the
  kernel matrix of h(x) = silu(W1 x) * (W3 x);
* the two building blocks alone (Newton-Schulz and row renorm).
"""

import numpy as np
import pytest

from oracle import lact_backward as B
from oracle import lact_oracle as O

BOUNDS = [0, 4, 7, 10, 13]
FLAGS = [O.UPDATE | O.APPLY, O.APPLY, O.UPDATE, O.UPDATE | O.APPLY]


def make(seed, D, Dh, L=13):
    rng = np.random.default_rng(seed)
    x = {
        "q": rng.standard_normal((L, D)),
        "k": rng.standard_normal((L, D)) / np.sqrt(D),
        "v": rng.standard_normal((L, D)),
        "lr": 0.05 + 0.3 * rng.random((L, 3)),
        "beta": rng.random(L),
        "W1": rng.standard_normal((Dh, D)) / np.sqrt(D),
        "W2": rng.standard_normal((D, Dh)) / np.sqrt(Dh),
        "W3": rng.standard_normal((Dh, D)) / np.sqrt(D),
        "M1": 0.1 * rng.standard_normal((Dh, D)),
        "M2": 0.1 * rng.standard_normal((D, Dh)),
        "M3": 0.1 * rng.standard_normal((Dh, D)),
    }
    cot = {
        "dO": rng.standard_normal((L, D)),
        "gW": [rng.standard_normal(x[n].shape) for n in ("W1", "W2", "W3")],
        "gM": [rng.standard_normal(x[n].shape) for n in ("M1", "M2", "M3")],
    }
    return x, cot


def objective(x, cot, order, opt, renorm, bounds=BOUNDS, flags=FLAGS, qk_prep=False):
    r = O.forward_instance(x["q"], x["k"], x["v"], x["lr"], x["beta"], x["W1"], x["W2"], x["W3"], bounds, flags,
                           order, opt, renorm, M=[x["M1"], x["M2"], x["M3"]], qk_prep=qk_prep, oz=x.get("oz"))
    J = float(np.sum(cot["dO"] * r["o"]))
    J += sum(float(np.sum(g * r[n])) for g, n in zip(cot["gW"], ("W1", "W2", "W3")))
    J += sum(float(np.sum(g * r[n])) for g, n in zip(cot["gM"], ("M1", "M2", "M3")))
    return J


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "lr": "dlr", "beta": "dbeta", "W1": "dW1", "W2": "dW2", "W3": "dW3",
           "M1": "dM1", "M2": "dM2", "M3": "dM3"}


def check_fd(x, cot, order, opt, renorm, seed, h=1e-5, tol=1e-6, bounds=BOUNDS, flags=FLAGS, qk_prep=False):
    """Directional derivative of J in a random direction per input against
    the oracle's gradient.  Central differences at h and h / 2 combined by
    Richardson extrapolation (the h^2 error term cancels; Newton-Schulz makes
    J curved enough that plain central differences need h ~ 1e-7)."""
    g = B.backward_instance(x["q"], x["k"], x["v"], x["lr"], x["beta"], x["W1"], x["W2"], x["W3"], bounds,
                            flags, order, opt, cot["dO"], cot["gW"], cot["gM"], renorm,
                            M=[x["M1"], x["M2"], x["M3"]], qk_prep=qk_prep, oz=x.get("oz"))
    rng = np.random.default_rng(1000 + seed)
    names = dict(GRAD_OF, **({"oz": "doz"} if "oz" in x else {}))
    for name, gname in names.items():
        d = rng.standard_normal(x[name].shape)

        def central(step):
            xp = dict(x)
            xm = dict(x)
            xp[name] = x[name] + step * d
            xm[name] = x[name] - step * d
            return (objective(xp, cot, order, opt, renorm, bounds, flags, qk_prep)
                    - objective(xm, cot, order, opt, renorm, bounds, flags, qk_prep)) / (2 * step)
        fd = (4 * central(h / 2) - central(h)) / 3
        an = float(np.sum(g[gname] * d))
        scale = max(abs(fd), abs(an), 1e-3)
        assert abs(fd - an) <= tol * scale, (name, fd, an)


SHAPES = [(4, 4), (4, 6), (6, 4)]


@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MOMENTUM, O.OPT_MUON, O.OPT_MUON_MOMENTUM])
@pytest.mark.parametrize("order", [O.APPLY_THEN_UPDATE, O.UPDATE_THEN_APPLY])
@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_finite_differences(opt, order, renorm, shape):
    D, Dh = shape
    seed = 17 * opt + 5 * order + 3 * int(renorm) + D + 7 * Dh
    x, cot = make(seed, D, Dh)
    check_fd(x, cot, order, opt, renorm, seed)


@pytest.mark.parametrize("opt", [O.OPT_MOMENTUM, O.OPT_MUON])
@pytest.mark.parametrize("order", [O.APPLY_THEN_UPDATE, O.UPDATE_THEN_APPLY])
def test_finite_differences_raw_qk_and_output_scale(opt, order):
    """q and k raw (the layer applies silu and the per-token L2 norm) and
    the output scaled by silu(oz): gradients of the raw q, k and of oz."""
    x, cot = make(40 + opt + order, 5, 5)
    x["oz"] = np.random.default_rng(41).standard_normal(x["q"].shape[0])
    check_fd(x, cot, order, opt, True, 40, qk_prep=True)


def test_qk_preprocess_vjp_alone():
    rng = np.random.default_rng(12)
    X, gY = rng.standard_normal((6, 7)), rng.standard_normal((6, 7))
    gX = B.qk_preprocess_vjp(X, gY)
    for _ in range(3):
        d = rng.standard_normal((6, 7))
        h = 1e-6
        fd = (np.sum(gY * O.qk_preprocess(X + h * d)) - np.sum(gY * O.qk_preprocess(X - h * d))) / (2 * h)
        assert abs(fd - np.sum(gX * d)) <= 1e-7 * max(1.0, abs(fd))


def test_finite_differences_single_chunk_and_apply_only_tail():
    """Schedules at the edges: one chunk covering everything, and an
    apply-only chunk after the last update."""
    for bounds, flags in [([0, 9], [O.UPDATE | O.APPLY]),
                          ([0, 5, 9], [O.UPDATE | O.APPLY, O.APPLY])]:
        for order in (O.APPLY_THEN_UPDATE, O.UPDATE_THEN_APPLY):
            x, cot = make(3 + order, 5, 5, L=9)
            check_fd(x, cot, order, O.OPT_MOMENTUM, True, 3, bounds=bounds, flags=flags)


def test_linear_attention_closed_form():
    """GD, no renorm, lr1 = lr3 = 0, one update-then-apply chunk:
    o_t = W2 h(q_t) + sum_i lr2_i <h(k_i), h(q_t)> v_i, so with the kernel
    matrix Km[i, t] = <h(k_i), h(q_t)>:
      dv_i = lr2_i sum_t Km[i, t] dO_t,
      dlr2_i = sum_t Km[i, t] <v_i, dO_t>,
      dW2 = sum_t dO_t h(q_t)^T,  dlr1 = dlr3 = 0 is not implied (W1, W3
      still move W2's input) -- only the listed closed forms are checked."""
    rng = np.random.default_rng(5)
    D, Dh, L = 5, 7, 11
    q, k, v = rng.standard_normal((L, D)), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    lr = np.zeros((L, 3))
    lr[:, 1] = rng.random(L)
    W1 = rng.standard_normal((Dh, D)) / np.sqrt(D)
    W3 = rng.standard_normal((Dh, D)) / np.sqrt(D)
    W2 = rng.standard_normal((D, Dh)) / np.sqrt(Dh)
    dO = rng.standard_normal((L, D))
    g = B.backward_instance(q, k, v, lr, None, W1, W2, W3, [0, L], [O.UPDATE | O.APPLY], O.UPDATE_THEN_APPLY,
                            O.OPT_GD, dO, renorm=False)
    h = lambda X: O.silu(X @ W1.T) * (X @ W3.T)
    Km = h(k) @ h(q).T
    KdO = Km @ dO
    np.testing.assert_allclose(g["dv"], lr[:, 1:2] * KdO, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dlr"][:, 1], np.sum(KdO * v, axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dW2"], dO.T @ h(q), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", [(5, 5), (3, 6), (6, 3)])
def test_newton_schulz_vjp(shape):
    rng = np.random.default_rng(shape[0] * 10 + shape[1])
    G = rng.standard_normal(shape)
    gY = rng.standard_normal(shape)
    gG = B.newton_schulz5_vjp(G, gY)
    for _ in range(3):
        d = rng.standard_normal(shape)
        h = 1e-6
        fd = (np.sum(gY * O.newton_schulz5(G + h * d)) - np.sum(gY * O.newton_schulz5(G - h * d))) / (2 * h)
        assert abs(fd - np.sum(gG * d)) <= 1e-7 * max(1.0, abs(fd))


def test_renorm_vjp():
    rng = np.random.default_rng(2)
    Wn, Wo, gY = rng.standard_normal((4, 6)), rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    gn, go = B.renorm_rows_vjp(Wn, Wo, gY)
    for _ in range(3):
        dn, do = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
        h = 1e-6
        f = lambda a, b: np.sum(gY * O.renorm_rows(a, b))
        fd = (f(Wn + h * dn, Wo + h * do) - f(Wn - h * dn, Wo - h * do)) / (2 * h)
        assert abs(fd - np.sum(gn * dn) - np.sum(go * do)) <= 1e-7 * max(1.0, abs(fd))


def test_state_only_cotangent_without_updates_passes_through():
    """With no UPDATE chunk the state is the identity map: dW0 = gW, dM0 = gM,
    and dk = dv = dlr = 0."""
    x, cot = make(9, 4, 4, L=6)
    g = B.backward_instance(x["q"], x["k"], x["v"], x["lr"], x["beta"], x["W1"], x["W2"], x["W3"], [0, 6],
                            [O.APPLY], O.APPLY_THEN_UPDATE, O.OPT_MOMENTUM, np.zeros((6, 4)), cot["gW"], cot["gM"],
                            M=[x["M1"], x["M2"], x["M3"]])
    for i, n in enumerate(("dW1", "dW2", "dW3")):
        np.testing.assert_array_equal(g[n], cot["gW"][i])
    for i, n in enumerate(("dM1", "dM2", "dM3")):
        np.testing.assert_array_equal(g[n], cot["gM"][i])
    assert not np.any(g["dk"]) and not np.any(g["dv"]) and not np.any(g["dlr"])
