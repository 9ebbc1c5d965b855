"""bench.py's host-side logic (no GPU): the one-GPU guard, the per-kernel
flop split that the roofline divides by, and the host record of the oracle
baseline."""
import os
import subprocess
import sys

import pytest

import bench
from test_layers_amd import lact
from test_layers_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert not r.stdout.strip()   # no JSON line for a configuration that was not measured


@pytest.mark.parametrize("cid", sorted(W.WORKLOADS))
def test_per_kernel_flops_add_up_to_the_algorithmic_total(cid):
    wl = W.WORKLOADS[cid]
    kf = bench.kernel_flops(wl, lact)
    alg = W.algorithmic_flops(wl)
    parts = kf[lact.K_UPD] + kf[lact.K_DW] + kf[lact.K_APP] + kf[lact.K_OUT]
    assert parts == pytest.approx(alg["update"] + alg["apply"], rel=1e-12)
    if wl.D == wl.dh:
        assert kf[lact.K_NS] == pytest.approx(alg["total"] - alg["update"] - alg["apply"], rel=1e-12, abs=0.0)


def test_host_record():
    h = bench.host_info()
    assert set(h) == {"cpu_model", "os_cpu_count", "affinity_cpus", "blas"}
    assert h["os_cpu_count"] >= h["affinity_cpus"] >= 1


@pytest.mark.parametrize("cid", sorted(W.WORKLOADS))
def test_roofline_bound_follows_the_arithmetic_intensity(cid):
    """The roofline picks the HBM roof for kernels below the ridge point:
    the fused apply at d = dh = 128 (6 d dh flop against 4 d bytes per query:
    1.5 dh = 192 flop/B) is HBM-bound, the update products at d = 512 are
    not, and Newton-Schulz has no algorithmic HBM traffic at all."""
    wl = W.WORKLOADS[cid]
    kf = bench.kernel_flops(wl, lact)
    kb = bench.kernel_bytes(wl, lact, {"out_in_app"})
    app_ai = (kf[lact.K_APP] + kf[lact.K_OUT]) / kb[lact.K_APP] if kb[lact.K_APP] else None
    if wl.D == wl.dh == 128 and wl.io_dtype == W.DTYPE_BF16 and app_ai is not None:
        assert app_ai < bench.RIDGE
    if wl.D == wl.dh == 512:
        assert kf[lact.K_UPD] / kb[lact.K_UPD] > bench.RIDGE
    assert kb[lact.K_NS] == 0.0


def test_default_workload_is_the_largest_language_layer():
    import bench as B
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = B.parse()
    finally:
        sys.argv = old
    wl = W.WORKLOADS[args.config]
    assert wl.name == "lm3b_d512_bf16_muon"
    lm = [w for w in W.WORKLOADS.values() if w.name.startswith("lm")]
    assert all(bench.kernel_flops(w, lact)[lact.K_UPD] <= bench.kernel_flops(wl, lact)[lact.K_UPD] for w in lm)
