"""The oracle's pins are not vacuous: each plausible mistake planted in a copy
of the oracle (on the CPU) must make tests/test_oracle_pins.py fail."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "silu_prime_dropped": ("return s * (1.0 + x * (1.0 - s))", "return s"),
    "U2_sign": ("U2 = (e2 * V).T @ H", "U2 = -(e2 * V).T @ H"),
    "U1_transposed": ("U1 = (e1 * G * B * silu_prime(A)).T @ K",
                      "U1 = ((e1 * G * B * silu_prime(A)).T @ K).T"),
    "G_transposed_W2": ("G = V @ W2\n", "G = V @ W2.T\n"),
    "mean_not_sum": ("U2 = (e2 * V).T @ H", "U2 = (e2 * V).T @ H / K.shape[0]"),
    "lr_columns_swapped": ("e1, e2, e3 = lr[:, 0:1], lr[:, 1:2], lr[:, 2:3]",
                           "e1, e2, e3 = lr[:, 2:3], lr[:, 1:2], lr[:, 0:1]"),
    "renorm_over_columns": ("n_old = np.linalg.norm(W_old, axis=1, keepdims=True)\n"
                            "    n_new = np.linalg.norm(W_new, axis=1, keepdims=True)",
                            "n_old = np.linalg.norm(W_old, axis=0, keepdims=True)\n"
                            "    n_new = np.linalg.norm(W_new, axis=0, keepdims=True)"),
    "renorm_to_unit": ("return W_new * (n_old / n_new)", "return W_new / n_new"),
    "ns_coefficient": ("NS_COEFFS = (3.4445, -4.7750, 2.0315)", "NS_COEFFS = (3.4445, -4.7750, 2.0)"),
    "ns_product_order": ("X = a * X + B @ X", "X = a * X + X @ B"),
    "momentum_sign": ("return beta_mean * M - U", "return beta_mean * M + U"),
    "momentum_last_beta": ("bm = float(np.mean(beta))\n        Mn = [momentum_step(m, u, bm) for m, u in zip(M, U)]\n"
                           "        Wn = [w - m for w, m in zip(W, Mn)]",
                           "bm = float(beta[-1])\n        Mn = [momentum_step(m, u, bm) for m, u in zip(M, U)]\n"
                           "        Wn = [w - m for w, m in zip(W, Mn)]"),
    "order_swapped": ("if (f & APPLY) and (order == APPLY_THEN_UPDATE or not (f & UPDATE)):",
                      "if (f & APPLY) and (order == UPDATE_THEN_APPLY or not (f & UPDATE)):"),
    "gd_sign": ("Wn = [w + u for w, u in zip(W, U)]", "Wn = [w - u for w, u in zip(W, U)]"),
    "muon_sign": ("Wn = [w + newton_schulz5(u, ns_steps) for w, u in zip(W, U)]",
                  "Wn = [w - newton_schulz5(u, ns_steps) for w, u in zip(W, U)]"),
    "apply_W1_for_W3": ("B = X @ W3.T\n    return", "B = X @ W1.T\n    return"),
    "apply_only_chunk_updates": ("if f & UPDATE:\n            bt", "if True:\n            bt"),
    "muon_momentum_orthogonalises_U": ("Wn = [w - newton_schulz5(m, ns_steps) for w, m in zip(W, Mn)]",
                                       "Wn = [w + newton_schulz5(u, ns_steps) for w, u in zip(W, U)]"),
    "qk_prep_no_norm": ("return s / np.sqrt(np.sum(s * s, axis=-1, keepdims=True))", "return s"),
    "output_scale_sigmoid": ("return o * silu(f64(z))[:, None]", "return o * sigmoid(f64(z))[:, None]"),
    "muon_momentum_plus": ("Wn = [w - newton_schulz5(m, ns_steps) for w, m in zip(W, Mn)]",
                           "Wn = [w + newton_schulz5(m, ns_steps) for w, m in zip(W, Mn)]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    a, b = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "lact_oracle.py")).read()
    assert src.count(a) == 1, f"mutation anchor for {name} not found exactly once"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    (pkg / "lact_oracle.py").write_text(src.replace(a, b))
    env = dict(os.environ, PYTHONPATH=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c",
                        "import sys; sys.path.insert(0, %r); import oracle; "
                        "assert oracle.__file__.startswith(%r); "
                        "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
                        % (str(tmp_path), str(tmp_path), os.path.join(ROOT, "tests", "test_oracle_pins.py"))],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"{name} not caught:\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"


# plausible mistakes in the backward oracle; each must make
# tests/test_oracle_backward.py fail
BWD_MUTATIONS = {
    "silu_second_dropped": ("gA = gE1 * e1 * G * B * Spp", "gA = gE1 * e1 * G * B * Sp"),
    "dK_update_term_dropped": ("dK = E1 @ gU1 + E3 @ gU3", "dK = E1 @ gU1"),
    "dV_forward_term_dropped": ("dV = dV + gG @ W2.T", "dV = dV"),
    "gB_lr_dropped": ("gB = gE1 * e1 * G * Sp + gH2 * e2 * S", "gB = gE1 * G * Sp + gH2 * e2 * S"),
    "dlr_columns_swapped": ("dlr = np.stack([np.sum(gE1 * G * B * Sp, axis=1), np.sum(gH2 * S * B, axis=1),\n"
                            "                    np.sum(gE3 * G * S, axis=1)], axis=1)",
                            "dlr = np.stack([np.sum(gE3 * G * S, axis=1), np.sum(gH2 * S * B, axis=1),\n"
                            "                    np.sum(gE1 * G * B * Sp, axis=1)], axis=1)"),
    "renorm_projection_sign": ("(gY - dot * w), dot * W_old / n_old", "(gY + dot * w), dot * W_old / n_old"),
    "renorm_old_norm_term_dropped": ("gW = [p[1] + p[0] for p in pairs]", "gW = [p[0] for p in pairs]"),
    "ns_gram_not_symmetrised": ("g = a * g + P @ g + (gA + gA.T) @ X", "g = a * g + P @ g + gA @ X"),
    "ns_normalisation_term_dropped": ("    if nG > 0:\n        gG = gG -", "    if False:\n        gG = gG -"),
    "momentum_beta_grad_dropped": ("gbm = float(sum(np.sum(g * m) for g, m in zip(gMt, M)))", "gbm = 0.0"),
    "momentum_state_grad_unscaled": ("gM = [bm * g for g in gMt]", "gM = [g for g in gMt]"),
    "apply_vjp_W1_for_W3": ("dX = dA @ W1 + dB @ W3", "dX = dA @ W1 + dB @ W1"),
    "update_then_apply_reads_old_state": ("dX, gWa = apply_vjp(*states[c + 1][0], q[a:b], dO[a:b])",
                                          "dX, gWa = apply_vjp(*states[c][0], q[a:b], dO[a:b])"),
    "qk_prep_vjp_projection_dropped": ("(g - sh * np.sum(sh * g, axis=-1, keepdims=True)) / n", "g / n"),
    "output_scale_grad_silu_not_derivative": ("doz = silu_prime(z) * np.sum(dO * o, axis=1)",
                                              "doz = silu(z) * np.sum(dO * o, axis=1)"),
    "output_scale_not_on_cotangent": ("dO = dO * silu(z)[:, None]", "dO = dO"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_planted_backward_mistake_is_caught(name, tmp_path):
    a, b = BWD_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "lact_backward.py")).read()
    assert src.count(a) == 1, f"mutation anchor for {name} not found exactly once"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    shutil.copy(os.path.join(ROOT, "oracle", "lact_oracle.py"), pkg / "lact_oracle.py")
    (pkg / "lact_backward.py").write_text(src.replace(a, b))
    env = dict(os.environ, PYTHONPATH=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c",
                        "import sys; sys.path.insert(0, %r); import oracle.lact_backward as ob; "
                        "assert ob.__file__.startswith(%r); "
                        "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
                        % (str(tmp_path), str(tmp_path), os.path.join(ROOT, "tests", "test_oracle_backward.py"))],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"{name} not caught:\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
