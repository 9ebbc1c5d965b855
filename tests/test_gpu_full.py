"""GPU parity at the full workload sizes (the launch configuration the
benchmark times), every output compared with the fp64 oracle."""
import time

import pytest

from test_layers_amd import workloads as W
from parity_util import compare, log, run_gpu

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lact():
    from test_layers_amd import lact as L
    return L


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
def test_full_size_config(lact, cid):
    wl = W.WORKLOADS[cid]
    t = time.time()
    log(f"full cfg{cid} {wl.name}: n={wl.n_inst} D={wl.D} L={wl.L} chunks={wl.n_chunks} "
        f"rec_planes={wl.rec_planes}")
    inp = W.generate(wl, threads=16)
    log(f"  generated in {time.time() - t:.1f}s; running the HIP layer")
    gpu = run_gpu(wl, inp, torch, lact)
    log(f"  gpu done; oracle over {wl.n_inst} instances")
    t = time.time()
    fro = {}
    errs = compare(wl, inp, gpu, fro=fro)
    log(f"  oracle {time.time() - t:.1f}s errs={ {k: f'{v:.2e}' for k, v in errs.items()} } gate={wl.tol}")
    log(f"  frobenius ratios { {k: f'{v:.2e}' for k, v in fro.items()} }")
    assert max(errs.values()) <= wl.tol, errs
