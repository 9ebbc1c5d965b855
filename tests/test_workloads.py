"""Seeded input generator: shapes, schedules, rounding and reproducibility."""
import numpy as np
import torch

from test_layers_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 0.0], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_schedules():
    c = W.WORKLOADS
    assert c[1].bounds == (0, 256, 512, 768, 1024) and c[1].flags == (3, 3, 3, 3)
    assert c[2].n_chunks == 16 and c[3].n_chunks == 8
    assert c[4].bounds == (0, 196608, 200704) and c[4].flags == (W.UPDATE, W.APPLY)
    assert c[5].n_chunks == 23 and c[5].L == 107640
    assert c[5].flags[:4] == (3, W.APPLY, 3, W.APPLY) and c[5].flags[-1] == 3
    assert sum(1 for f in c[5].flags if f & W.UPDATE) == 12
    # schedule variants: view-set prefill also applies to the inputs; the
    # noisy-first video schedule has 12 noisy + 12 clean chunks (112,320 tokens)
    assert c[6].bounds == c[4].bounds and c[6].flags == (W.UPDATE | W.APPLY, W.APPLY)
    assert c[6].order == W.UPDATE_THEN_APPLY
    assert c[7].L == 24 * 4680 == 112320 and c[7].n_chunks == 24
    assert c[7].flags[:4] == (W.APPLY, 3, W.APPLY, 3) and c[7].flags[-1] == 3
    assert sum(1 for f in c[7].flags if f & W.UPDATE) == 12
    assert W.uniform_schedule(10, 4) == ((0, 4, 8, 10), (3, 3, 3))


def test_generator_reproducible_per_instance():
    wl = W.WORKLOADS[2].scaled(n_inst=3, L=64, chunk=32)
    a = W.generate(wl)
    b = W.generate_instance(wl, 2)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.lr, b.lr), (a.beta, b.beta), (a.W2, b.W2)]:
        np.testing.assert_array_equal(x[2], y[0])
    assert a.q.dtype == np.uint16 and a.lr.dtype == np.float32 and a.W1.dtype == np.float32
    # q, k are unit-norm after the silu + L2 recipe (up to bf16 rounding)
    n = np.linalg.norm(W.to_f64(a.k), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all(a.lr > 0) and np.all((a.beta > 0) & (a.beta < 1))
    wl1 = W.WORKLOADS[1]
    g = W.generate(wl1)
    assert g.q.dtype == np.float32 and g.beta is None and g.q.shape == (1, 1024, 64)


def test_flop_counts():
    f = W.algorithmic_flops(W.WORKLOADS[2])
    assert abs(f["total"] - 0.348e12) / 0.348e12 < 0.01
    f = W.algorithmic_flops(W.WORKLOADS[3])
    assert abs(f["total"] - 1.508e12) / 1.508e12 < 0.01


def test_rectangular_fast_weights():
    """dh != d: W1, W3 [dh, d], W2 [d, dh], each ~ N(0, 1/fan-in); the square
    workloads keep their draws (same shapes, same order)."""
    wl = W.WORKLOADS[10].scaled(n_inst=2, L=64, chunk=32)
    assert wl.D == 384 and wl.dh == 768
    g = W.generate(wl)
    assert g.W1.shape == (2, 768, 384) and g.W3.shape == (2, 768, 384) and g.W2.shape == (2, 384, 768)
    assert g.q.shape == (2, 64, 384)
    assert abs(np.std(g.W1) * np.sqrt(384) - 1) < 0.02 and abs(np.std(g.W2) * np.sqrt(768) - 1) < 0.02
    sq = W.WORKLOADS[2].scaled(n_inst=1, L=64, chunk=32)
    assert sq.dh == sq.D
    f = W.algorithmic_flops(W.WORKLOADS[10])
    assert f["total"] == 2 * W.algorithmic_flops(W.WORKLOADS[2])["total"]
