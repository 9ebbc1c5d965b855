"""Pins of the CPU oracle against facts fixed outside the oracle itself.

The pages print no worked numeric example, so every pin here is a property
that the mathematics or the pages' semantics fix: finite differences of an
independently written loss, causality of the two update/apply orders, the
order-shift equivalence, row-norm invariance, the closed form of the quintic
Newton-Schulz map via an SVD, special cases that reduce to textbook formulas
(plain SwiGLU MLP, un-normalised linear attention, GD), the geometric sum of
momentum, sum-over-chunk scaling, resume and instance permutation.
"""
import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(12345)


def rand_state(D, scale=None, rng=RNG):
    s = 1.0 / np.sqrt(D) if scale is None else scale
    return [rng.standard_normal((D, D)) * s for _ in range(3)]


def rand_chunk(C, D, rng=RNG, lr_scale=0.1):
    K = rng.standard_normal((C, D))
    V = rng.standard_normal((C, D))
    lr = rng.uniform(0.2, 1.0, size=(C, 3)) * lr_scale
    return K, V, lr


# ---------------------------------------------------------------- independent forward
def f_token(W1, W2, W3, x):
    """Textbook SwiGLU MLP on one vector: W2 (silu(W1 x) * (W3 x))."""
    a = W1 @ x
    b = W3 @ x
    s = a / (1.0 + np.exp(-a))
    return W2 @ (s * b)


def weighted_loss(W, K, V, lr, j):
    """sum_i lr[i, j] * l_i with l_i = -<f_W(k_i), v_i> (token loop)."""
    tot = 0.0
    for i in range(K.shape[0]):
        tot += lr[i, j] * -(f_token(W[0], W[1], W[2], K[i]) @ V[i])
    return tot


@pytest.mark.parametrize("D,C", [(3, 5), (5, 5), (8, 5)])
def test_grads_match_finite_differences(D, C):
    rng = np.random.default_rng(D * 100 + C)
    W = rand_state(D, 0.7, rng)
    K, V, lr = rand_chunk(C, D, rng, lr_scale=1.0)
    U = O.chunk_grads(W[0], W[1], W[2], K, V, lr)
    h = 1e-6
    for j in range(3):
        fd = np.zeros((D, D))
        for r in range(D):
            for c in range(D):
                Wp = [w.copy() for w in W]
                Wm = [w.copy() for w in W]
                Wp[j][r, c] += h
                Wm[j][r, c] -= h
                fd[r, c] = (weighted_loss(Wp, K, V, lr, j) - weighted_loss(Wm, K, V, lr, j)) / (2 * h)
        # U_j is the negative lr-weighted gradient
        err = np.max(np.abs(-fd - U[j])) / np.max(np.abs(U[j]))
        assert err <= 1e-7, (j, err)


def test_grad_is_a_sum_over_the_chunk():
    D, C = 6, 7
    W = rand_state(D)
    K, V, lr = rand_chunk(C, D)
    U = O.chunk_grads(*W, K, V, lr)
    U2x = O.chunk_grads(*W, np.vstack([K, K]), np.vstack([V, V]), np.vstack([lr, lr]))
    for a, b in zip(U, U2x):
        np.testing.assert_allclose(b, 2 * a, rtol=1e-13, atol=1e-15)


def test_lr_columns_map_to_matrices():
    """lr column j-1 only moves W_j (GD, no renorm)."""
    D, C = 5, 6
    W = rand_state(D)
    K, V, lr = rand_chunk(C, D)
    for j in range(3):
        lj = np.zeros_like(lr)
        lj[:, j] = lr[:, j]
        Wn, _ = O.update_step(W, [np.zeros((D, D))] * 3, K, V, lj, None, O.OPT_GD, renorm=False)
        for jj in range(3):
            same = np.array_equal(Wn[jj], W[jj])
            assert same == (jj != j), (j, jj)


# ---------------------------------------------------------------- schedule semantics
def make_seq(n_chunks, C, D, rng):
    L = n_chunks * C
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    lr = rng.uniform(0.0, 0.05, size=(L, 3))
    beta = rng.uniform(0.5, 0.99, size=L)
    W = rand_state(D, rng=rng)
    b = list(range(0, L + 1, C))
    return q, k, v, lr, beta, W, b


@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MOMENTUM, O.OPT_MUON, O.OPT_MUON_MOMENTUM])
def test_causality_apply_then_update(opt):
    rng = np.random.default_rng(7)
    n, C, D = 4, 6, 5
    q, k, v, lr, beta, W, b = make_seq(n, C, D, rng)
    fl = [O.UPDATE | O.APPLY] * n
    ref = O.forward_instance(q, k, v, lr, beta, *W, b, fl, O.APPLY_THEN_UPDATE, opt)
    c = 1
    sl = slice(b[c + 1], b[c + 2])
    for name in ["q", "k", "v", "lr", "beta"]:
        arrs = dict(q=q.copy(), k=k.copy(), v=v.copy(), lr=lr.copy(), beta=beta.copy())
        arrs[name][sl] += 0.5
        out = O.forward_instance(arrs["q"], arrs["k"], arrs["v"], arrs["lr"], arrs["beta"],
                                 *W, b, fl, O.APPLY_THEN_UPDATE, opt)
        # chunks <= c and chunk c+1 itself never see chunk c+1's keys
        assert np.array_equal(out["o"][: b[c + 1]], ref["o"][: b[c + 1]]), name
        if name == "q":
            assert not np.array_equal(out["o"][sl], ref["o"][sl])
            assert np.array_equal(out["o"][b[c + 2]:], ref["o"][b[c + 2]:])
        elif name in ("k", "v", "lr") or (name == "beta" and opt in (O.OPT_MOMENTUM, O.OPT_MUON_MOMENTUM)):
            assert np.array_equal(out["o"][sl], ref["o"][sl]), name
            assert not np.array_equal(out["o"][b[c + 2]:], ref["o"][b[c + 2]:]), name


@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MUON])
def test_causality_update_then_apply(opt):
    rng = np.random.default_rng(8)
    n, C, D = 4, 6, 5
    q, k, v, lr, beta, W, b = make_seq(n, C, D, rng)
    fl = [O.UPDATE | O.APPLY] * n
    ref = O.forward_instance(q, k, v, lr, beta, *W, b, fl, O.UPDATE_THEN_APPLY, opt)
    c = 1
    k2 = k.copy()
    k2[b[c + 1]:b[c + 2]] += 0.5
    out = O.forward_instance(q, k2, v, lr, beta, *W, b, fl, O.UPDATE_THEN_APPLY, opt)
    assert np.array_equal(out["o"][: b[c + 1]], ref["o"][: b[c + 1]])
    # chunk c+1 reads the weights it was just updated with
    assert not np.array_equal(out["o"][b[c + 1]:b[c + 2]], ref["o"][b[c + 1]:b[c + 2]])


def test_order_shift_equivalence():
    """Apply-then-update output of chunk c equals update-then-apply output of
    chunk c-1 when the queries are shifted back by one chunk."""
    rng = np.random.default_rng(9)
    n, C, D = 5, 4, 6
    q, k, v, lr, beta, W, b = make_seq(n, C, D, rng)
    fl = [O.UPDATE | O.APPLY] * n
    atu = O.forward_instance(q, k, v, lr, beta, *W, b, fl, O.APPLY_THEN_UPDATE, O.OPT_MOMENTUM)
    qs = np.roll(q, -C, axis=0)
    uta = O.forward_instance(qs, k, v, lr, beta, *W, b, fl, O.UPDATE_THEN_APPLY, O.OPT_MOMENTUM)
    for c in range(1, n):
        assert np.array_equal(atu["o"][b[c]:b[c + 1]], uta["o"][b[c - 1]:b[c]]), c
    for key in ["W1", "W2", "W3", "M1", "M2", "M3"]:
        assert np.array_equal(atu[key], uta[key])


def test_video_schedule_noisy_chunks_only_read():
    """Apply-only (noisy) chunks never write the state, and read the weights
    the following clean chunk reads."""
    rng = np.random.default_rng(10)
    C, D, n_clean = 4, 5, 4
    flags = [O.UPDATE | O.APPLY]
    for _ in range(n_clean - 1):
        flags += [O.APPLY, O.UPDATE | O.APPLY]
    L = C * len(flags)
    b = list(range(0, L + 1, C))
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    lr = rng.uniform(0, 0.05, (L, 3))
    W = rand_state(D, rng=rng)
    ref = O.forward_instance(q, k, v, lr, None, *W, b, flags, O.APPLY_THEN_UPDATE, O.OPT_MUON)
    k2, v2 = k.copy(), v.copy()
    for c, f in enumerate(flags):
        if f == O.APPLY:
            k2[b[c]:b[c + 1]] += 1.0
            v2[b[c]:b[c + 1]] -= 1.0
    out = O.forward_instance(q, k2, v2, lr, None, *W, b, flags, O.APPLY_THEN_UPDATE, O.OPT_MUON)
    for key in ["o", "W1", "W2", "W3"]:
        assert np.array_equal(out[key], ref[key])
    # noisy chunk N_j (index 2j-1) and clean chunk C_j (index 2j) share weights:
    # same queries give the same outputs
    q3 = q.copy()
    q3[b[1]:b[2]] = q3[b[2]:b[3]]
    out3 = O.forward_instance(q3, k, v, lr, None, *W, b, flags, O.APPLY_THEN_UPDATE, O.OPT_MUON)
    assert np.array_equal(out3["o"][b[1]:b[2]], out3["o"][b[2]:b[3]])


# ---------------------------------------------------------------- renorm
@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MOMENTUM, O.OPT_MUON, O.OPT_MUON_MOMENTUM])
def test_row_norms_invariant(opt):
    rng = np.random.default_rng(11)
    D, C = 7, 9
    W0 = rand_state(D, rng=rng)
    W = W0
    M = [np.zeros((D, D))] * 3
    n0 = [np.linalg.norm(w, axis=1) for w in W0]
    for _ in range(6):
        K, V, lr = rand_chunk(C, D, rng, lr_scale=2.0)
        W, M = O.update_step(W, M, K, V, lr, rng.uniform(0.5, 1, C), opt)
        for w, n in zip(W, n0):
            np.testing.assert_allclose(np.linalg.norm(w, axis=1), n, rtol=1e-12)
    # without renorm the norms do move (the pin above is not vacuous)
    Wn, _ = O.update_step(W0, M, K, V, lr, rng.uniform(0.5, 1, C), opt, renorm=False)
    assert np.max(np.abs(np.linalg.norm(Wn[0], axis=1) - n0[0])) > 1e-3


# ---------------------------------------------------------------- Newton-Schulz
def ns_closed_form(G, steps=5, eps=1e-7):
    a, b, c = 3.4445, -4.7750, 2.0315
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    x = s / (np.sqrt(np.sum(s * s)) + eps)
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x) @ Vt, s / (np.sqrt(np.sum(s * s)) + eps)


@pytest.mark.parametrize("shape", [(8, 8), (16, 16), (12, 7), (5, 9)])
def test_ns5_closed_form(shape):
    rng = np.random.default_rng(sum(shape))
    G = rng.standard_normal(shape) @ np.diag(np.logspace(-1, 1, shape[1]))
    X = O.newton_schulz5(G)
    ref, _ = ns_closed_form(G)
    assert np.max(np.abs(X - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_ns5_singular_value_band():
    """Five quintic steps send every normalised singular value to at most
    1.2024; those at or above 1.6e-3 land in [0.68, 1.2024]."""
    rng = np.random.default_rng(3)
    for _ in range(5):
        D = 24
        G = rng.standard_normal((D, D)) @ np.diag(np.logspace(-3, 0, D)) @ rng.standard_normal((D, D))
        X = O.newton_schulz5(G)
        sv = np.linalg.svd(X, compute_uv=False)
        _, sn = ns_closed_form(G)
        assert sv.max() <= 1.2024
        big = np.sort(sn)[::-1] >= 1.6e-3
        sv_sorted = np.sort(sv)[::-1]
        # singular values keep their order where the map is monotone enough; compare sets
        inband = sv_sorted[(sv_sorted >= 0.68) & (sv_sorted <= 1.2024)]
        assert len(inband) >= big.sum()
    assert np.array_equal(O.newton_schulz5(np.zeros((6, 6))), np.zeros((6, 6)))


# ---------------------------------------------------------------- special cases
@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MOMENTUM, O.OPT_MUON, O.OPT_MUON_MOMENTUM])
@pytest.mark.parametrize("order", [O.APPLY_THEN_UPDATE, O.UPDATE_THEN_APPLY])
def test_zero_lr_is_a_plain_swiglu_mlp(opt, order):
    rng = np.random.default_rng(5)
    q, k, v, lr, beta, W, b = make_seq(3, 5, 6, rng)
    out = O.forward_instance(q, k, v, np.zeros_like(lr), beta, *W, b, [3] * 3, order, opt)
    for j, key in enumerate(["W1", "W2", "W3"]):
        assert np.array_equal(out[key], W[j])
    ref = np.stack([f_token(*W, x) for x in q])
    assert np.max(np.abs(out["o"] - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_w2_only_update_is_linear_attention():
    """lr1 = lr3 = 0, GD, no renorm, one chunk, update-then-apply:
    o(q) = W2 h(q) + sum_i lr2_i <h(k_i), h(q)> v_i with h(x) = silu(W1 x)*(W3 x)."""
    rng = np.random.default_rng(6)
    C, D = 9, 6
    q = rng.standard_normal((C, D))
    k = rng.standard_normal((C, D))
    v = rng.standard_normal((C, D))
    lr = np.zeros((C, 3))
    lr[:, 1] = rng.uniform(0.1, 1.0, C)
    W = rand_state(D, rng=rng)
    out = O.forward_instance(q, k, v, lr, None, *W, [0, C], [3], O.UPDATE_THEN_APPLY,
                             O.OPT_GD, renorm=False)

    def h(X):
        a = X @ W[0].T
        return a / (1 + np.exp(-a)) * (X @ W[2].T)
    kern = h(q) @ h(k).T                        # [Cq, Ck] feature-map kernel
    ref = h(q) @ W[1].T + (kern * lr[:, 1][None, :]) @ v
    assert np.max(np.abs(out["o"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_momentum_zero_beta_is_gd():
    rng = np.random.default_rng(4)
    q, k, v, lr, beta, W, b = make_seq(4, 5, 6, rng)
    fl = [3] * 4
    gd = O.forward_instance(q, k, v, lr, None, *W, b, fl, O.APPLY_THEN_UPDATE, O.OPT_GD)
    mo = O.forward_instance(q, k, v, lr, np.zeros_like(beta), *W, b, fl,
                            O.APPLY_THEN_UPDATE, O.OPT_MOMENTUM)
    for key in ["o", "W1", "W2", "W3"]:
        assert np.array_equal(gd[key], mo[key])


def test_momentum_geometric_sum():
    rng = np.random.default_rng(2)
    D, steps, bm = 5, 6, 0.83
    Us = [rng.standard_normal((D, D)) for _ in range(steps)]
    M = np.zeros((D, D))
    for c, U in enumerate(Us):
        M = O.momentum_step(M, U, bm)
        ref = -sum(bm ** (c - s) * Us[s] for s in range(c + 1))
        np.testing.assert_allclose(M, ref, rtol=1e-12, atol=1e-13)


def test_momentum_uses_chunk_mean_of_beta():
    """A chunk whose betas average to b behaves like a constant-b chunk."""
    rng = np.random.default_rng(1)
    q, k, v, lr, beta, W, b = make_seq(3, 4, 5, rng)
    fl = [3] * 3
    beta2 = beta.copy()
    for c in range(3):
        sl = slice(b[c], b[c + 1])
        beta2[sl] = np.mean(beta[sl])
    r1 = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, O.OPT_MOMENTUM)
    r2 = O.forward_instance(q, k, v, lr, beta2, *W, b, fl, 0, O.OPT_MOMENTUM)
    for key in ["o", "W1", "M2"]:
        np.testing.assert_allclose(r1[key], r2[key], rtol=1e-12, atol=1e-14)
    r3 = O.forward_instance(q, k, v, lr, beta * 0.5, *W, b, fl, 0, O.OPT_MOMENTUM)
    assert not np.allclose(r1["o"][b[2]:], r3["o"][b[2]:])


# ---------------------------------------------------------------- state carry
@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MOMENTUM, O.OPT_MUON, O.OPT_MUON_MOMENTUM])
def test_resume_equals_single_call(opt):
    rng = np.random.default_rng(13)
    n, C, D = 5, 4, 6
    q, k, v, lr, beta, W, b = make_seq(n, C, D, rng)
    fl = [3] * n
    full = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, opt)
    cut = 2
    s = b[cut]
    first = O.forward_instance(q[:s], k[:s], v[:s], lr[:s], beta[:s], *W, b[: cut + 1],
                               fl[:cut], 0, opt)
    rest_b = [x - s for x in b[cut:]]
    second = O.forward_instance(q[s:], k[s:], v[s:], lr[s:], beta[s:], first["W1"],
                                first["W2"], first["W3"], rest_b, fl[cut:], 0, opt,
                                M=[first["M1"], first["M2"], first["M3"]])
    assert np.array_equal(np.vstack([first["o"], second["o"]]), full["o"])
    for key in ["W1", "W2", "W3", "M1", "M2", "M3"]:
        assert np.array_equal(second[key], full[key])


def test_instance_permutation():
    rng = np.random.default_rng(14)
    n, L, D = 3, 8, 5
    arr = lambda *s: rng.standard_normal(s)
    q, k, v = arr(n, L, D), arr(n, L, D), arr(n, L, D)
    lr = rng.uniform(0, 0.1, (n, L, 3))
    W = [arr(n, D, D) / np.sqrt(D) for _ in range(3)]
    b, fl = [0, 4, 8], [3, 3]
    ref = O.layer_forward(q, k, v, lr, None, *W, b, fl, 0, O.OPT_GD)
    p = np.array([2, 0, 1])
    out = O.layer_forward(q[p], k[p], v[p], lr[p], None, *[w[p] for w in W], b, fl, 0, O.OPT_GD)
    for key in ["o", "W1", "W2", "W3"]:
        assert np.array_equal(out[key], ref[key][p])


def test_bf16_decoding_is_exact():
    bits = np.array([0x3F80, 0xBF00, 0x4049, 0x0000, 0x3C00], dtype=np.uint16)
    np.testing.assert_array_equal(O.f64(bits), [1.0, -0.5, 3.140625, 0.0, 2.0 ** -7])


def fd_grad(W, K, V, lr, j, h=1e-6):
    D = W[j].shape[0]
    g = np.zeros_like(W[j])
    for r in range(D):
        for c in range(W[j].shape[1]):
            Wp = [w.copy() for w in W]
            Wm = [w.copy() for w in W]
            Wp[j][r, c] += h
            Wm[j][r, c] -= h
            g[r, c] = (weighted_loss(Wp, K, V, lr, j) - weighted_loss(Wm, K, V, lr, j)) / (2 * h)
    return g


def test_muon_step_is_ns_of_the_descent_direction():
    """Without renorm, the Muon step on W_j is the quintic Newton-Schulz map
    (closed form via SVD) of minus the finite-difference gradient, and it
    decreases the lr-weighted loss to first order."""
    rng = np.random.default_rng(21)
    D, C = 6, 5
    W = rand_state(D, 0.7, rng)
    K, V, lr = rand_chunk(C, D, rng, lr_scale=1.0)
    Wn, _ = O.update_step(W, [np.zeros((D, D))] * 3, K, V, lr, None, O.OPT_MUON, renorm=False)
    for j in range(3):
        g = fd_grad(W, K, V, lr, j)
        ref, _ = ns_closed_form(-g)
        step = Wn[j] - W[j]
        assert np.max(np.abs(step - ref)) <= 1e-5 * np.max(np.abs(ref)), j
        assert np.sum(g * step) < 0


def test_muon_momentum_with_zero_beta_is_muon():
    """Momentum + Muon with beta = 0: the buffer is minus this chunk's
    direction and the step equals Muon's, bitwise (NS5 is exactly odd)."""
    rng = np.random.default_rng(31)
    D, C = 7, 9
    W = rand_state(D, 0.8, rng)
    K, V, lr = rand_chunk(C, D, rng, lr_scale=0.3)
    M0 = [rng.standard_normal((D, D)) for _ in range(3)]
    for renorm in (True, False):
        Wa, Ma = O.update_step(W, M0, K, V, lr, np.zeros(C), O.OPT_MUON_MOMENTUM, renorm=renorm)
        Wb, _ = O.update_step(W, M0, K, V, lr, None, O.OPT_MUON, renorm=renorm)
        U = O.chunk_grads(*W, K, V, lr)
        for j in range(3):
            assert np.array_equal(Wa[j], Wb[j]), (renorm, j)
            assert np.array_equal(Ma[j], -U[j]), (renorm, j)


def test_muon_momentum_orthogonalises_the_momentum_buffer():
    """Two chunks, constant beta, no renorm: the buffer is the geometric sum
    of finite-difference gradients and each step is the SVD closed form of
    the quintic map of that buffer, subtracted from W."""
    rng = np.random.default_rng(32)
    D, C, b = 5, 6, 0.7
    W0 = rand_state(D, 0.7, rng)
    K1, V1, lr1 = rand_chunk(C, D, rng, lr_scale=0.5)
    K2, V2, lr2 = rand_chunk(C, D, rng, lr_scale=0.5)
    beta = np.full(C, b)
    M0 = [np.zeros((D, D))] * 3
    W1, M1 = O.update_step(W0, M0, K1, V1, lr1, beta, O.OPT_MUON_MOMENTUM, renorm=False)
    W2, M2 = O.update_step(W1, M1, K2, V2, lr2, beta, O.OPT_MUON_MOMENTUM, renorm=False)
    for j in range(3):
        g1 = fd_grad(W0, K1, V1, lr1, j)
        m1 = g1                                   # b * 0 + g1
        w1 = W0[j] - ns_closed_form(m1)[0]
        assert np.max(np.abs(M1[j] - m1)) <= 1e-6 * np.max(np.abs(m1)), j
        assert np.max(np.abs(W1[j] - w1)) <= 1e-5 * np.max(np.abs(w1)), j
        g2 = fd_grad(W1, K2, V2, lr2, j)
        m2 = b * M1[j] + g2
        w2 = W1[j] - ns_closed_form(m2)[0]
        assert np.max(np.abs(M2[j] - m2)) <= 1e-6 * np.max(np.abs(m2)), j
        assert np.max(np.abs(W2[j] - w2)) <= 1e-5 * np.max(np.abs(w2)), j


# ---------------------------------------------------------------- q/k pre-processing, output scale
def test_qk_preprocess_is_unit_norm_along_silu():
    """Each pre-processed token vector has unit norm and points along the
    element-wise silu of the raw vector (silu checked against the library
    logistic function)."""
    from scipy.special import expit
    rng = np.random.default_rng(41)
    for scale in (0.1, 1.0, 8.0):
        x = rng.standard_normal((17, 9)) * scale
        y = O.qk_preprocess(x)
        assert np.max(np.abs(np.linalg.norm(y, axis=1) - 1.0)) <= 1e-14
        s = x * expit(x)
        ratio = s / y
        assert np.max(np.abs(ratio / ratio[:, :1] - 1.0)) <= 1e-12
        assert np.all(ratio > 0)
    # silu(0) = 0 and silu(x) -> x for large x
    y = O.qk_preprocess(np.array([[0.0, 40.0, 30.0]]))
    assert y[0, 0] == 0.0
    assert np.allclose(y[0, 1:], np.array([40.0, 30.0]) / 50.0, rtol=1e-12, atol=0)


def test_layer_on_raw_qk_equals_layer_on_preprocessed_inputs():
    """The layer with in-layer q/k pre-processing equals the layer fed the
    generator's independently pre-processed q, k (fp64, no rounding)."""
    from test_layers_amd import workloads as Wk
    rng = np.random.default_rng(42)
    n, C, D = 3, 5, 6
    q, k, v, lr, beta, W, b = make_seq(n, C, D, rng)
    fl = [3] * n
    raw = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, O.OPT_MOMENTUM, qk_prep=True)
    pre = O.forward_instance(Wk._qk_prep(q), Wk._qk_prep(k), v, lr, beta, *W, b, fl, 0, O.OPT_MOMENTUM)
    for key in ("o", "W1", "W2", "W3", "M1", "M2", "M3"):
        assert np.max(np.abs(raw[key] - pre[key])) <= 1e-12 * max(1.0, np.max(np.abs(pre[key]))), key


def test_output_scale_special_values():
    """silu(0) = 0 zeroes every row; a pre-activation of 40 (logistic rounds
    to exactly 1 in fp64) scales by exactly 40; it touches no state."""
    rng = np.random.default_rng(43)
    n, C, D = 3, 4, 5
    q, k, v, lr, beta, W, b = make_seq(n, C, D, rng)
    fl = [3] * n
    base = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, O.OPT_GD)
    z0 = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, O.OPT_GD, oz=np.zeros(n * C))
    z40 = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, O.OPT_GD, oz=np.full(n * C, 40.0))
    zm = rng.standard_normal(n * C)
    zr = O.forward_instance(q, k, v, lr, beta, *W, b, fl, 0, O.OPT_GD, oz=zm)
    assert np.all(z0["o"] == 0.0)
    assert np.array_equal(z40["o"], 40.0 * base["o"])
    for t in range(n * C):   # one scalar per token
        r = zr["o"][t] / base["o"][t]
        assert np.max(np.abs(r - r[0])) <= 1e-12 * abs(r[0])
    for key in ("W1", "W2", "W3"):
        assert np.array_equal(zr[key], base[key])


# ---------------------------------------------------------------- rectangular fast weights (d != dh)
def rand_rect(d, dh, rng, scale=None):
    """W1, W3 [dh, d] (fan-in d) and W2 [d, dh] (fan-in dh)."""
    s1 = 1.0 / np.sqrt(d) if scale is None else scale
    s2 = 1.0 / np.sqrt(dh) if scale is None else scale
    return [rng.standard_normal((dh, d)) * s1, rng.standard_normal((d, dh)) * s2,
            rng.standard_normal((dh, d)) * s1]


@pytest.mark.parametrize("d,dh", [(4, 7), (6, 3)])
def test_rectangular_grads_match_finite_differences(d, dh):
    rng = np.random.default_rng(10 * d + dh)
    W = rand_rect(d, dh, rng, 0.7)
    K, V, lr = rand_chunk(5, d, rng, lr_scale=1.0)
    U = O.chunk_grads(W[0], W[1], W[2], K, V, lr)
    for j in range(3):
        assert U[j].shape == W[j].shape
    h = 1e-6
    for j in range(3):
        fd = np.zeros(W[j].shape)
        for r in range(W[j].shape[0]):
            for c in range(W[j].shape[1]):
                Wp = [w.copy() for w in W]
                Wm = [w.copy() for w in W]
                Wp[j][r, c] += h
                Wm[j][r, c] -= h
                fd[r, c] = (weighted_loss(Wp, K, V, lr, j) - weighted_loss(Wm, K, V, lr, j)) / (2 * h)
        err = np.max(np.abs(-fd - U[j])) / np.max(np.abs(U[j]))
        assert err <= 1e-7, (j, err)


@pytest.mark.parametrize("opt", [O.OPT_GD, O.OPT_MOMENTUM, O.OPT_MUON, O.OPT_MUON_MOMENTUM])
def test_rectangular_row_norms_invariant(opt):
    """Rows are fan-in vectors: length d for W1, W3 and dh for W2."""
    rng = np.random.default_rng(21)
    d, dh, C = 5, 8, 9
    W0 = rand_rect(d, dh, rng)
    W, M = W0, [np.zeros_like(w) for w in W0]
    n0 = [np.linalg.norm(w, axis=1) for w in W0]
    for _ in range(4):
        K, V, lr = rand_chunk(C, d, rng, lr_scale=2.0)
        W, M = O.update_step(W, M, K, V, lr, rng.uniform(0.5, 1, C), opt)
        for w, w0, n in zip(W, W0, n0):
            assert w.shape == w0.shape
            np.testing.assert_allclose(np.linalg.norm(w, axis=1), n, rtol=1e-12)


def test_rectangular_w2_only_update_is_linear_attention():
    """As the square case, with a feature map h of dh features on d-wide tokens."""
    rng = np.random.default_rng(16)
    C, d, dh = 9, 5, 11
    q = rng.standard_normal((C, d))
    k = rng.standard_normal((C, d))
    v = rng.standard_normal((C, d))
    lr = np.zeros((C, 3))
    lr[:, 1] = rng.uniform(0.1, 1.0, C)
    W = rand_rect(d, dh, rng)
    out = O.forward_instance(q, k, v, lr, None, *W, [0, C], [3], O.UPDATE_THEN_APPLY,
                             O.OPT_GD, renorm=False)

    def h(X):
        a = X @ W[0].T
        return a / (1 + np.exp(-a)) * (X @ W[2].T)
    ref = h(q) @ W[1].T + ((h(q) @ h(k).T) * lr[:, 1][None, :]) @ v
    assert out["o"].shape == (C, d)
    assert np.max(np.abs(out["o"] - ref)) <= 1e-12 * np.max(np.abs(ref))
