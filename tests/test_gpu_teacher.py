"""Teacher-forced per-chunk parity at the full workload sizes.

The GPU advances its own state chunk by chunk through the chunk-level ABI
(lact_chunk_update, lact_apply); before every chunk the oracle is handed the
GPU's current state exactly (fp32 values read as fp64) and performs that one
chunk's apply and update.  Comparing the two isolates the kernels' accuracy
for one chunk from the recurrence's sensitivity to accumulated rounding
(the end-to-end tests cover the latter).  Same metric and gates as the
end-to-end tests; the oracle runs on two instances (first and last)."""
import time

import numpy as np
import pytest

import oracle as O
from test_layers_amd import workloads as W
from parity_util import fro_ratio, log, rel_err, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lact():
    from test_layers_amd import lact as L
    return L


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 3, 5, 8, 10])
def test_teacher_forced_chunks(lact, cid):
    wl = W.WORKLOADS[cid]
    assert wl.order == W.APPLY_THEN_UPDATE
    n, L, D = wl.n_inst, wl.L, wl.D
    inst = sorted({0, n - 1})
    log(f"teacher-forced cfg{cid} {wl.name}: n={n} D={D} chunks={wl.n_chunks} rec_planes={wl.rec_planes}")
    inp = W.generate(wl, threads=16)
    q, k, v, lr = to_dev(inp.q, torch), to_dev(inp.k, torch), to_dev(inp.v, torch), to_dev(inp.lr, torch)
    beta = to_dev(inp.beta, torch)
    Ws = [to_dev(inp.W1, torch).clone(), to_dev(inp.W2, torch).clone(), to_dev(inp.W3, torch).clone()]
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    o = torch.zeros_like(q)
    p = lact.problem(n, D, wl.io_dtype, wl.opt, wl.rec_planes, dh=wl.dh)
    esz = q.element_size()
    C = wl.max_chunk
    ws = torch.empty(max(lact.workspace_size(p, C, C), 256), dtype=torch.uint8, device="cuda")
    ptr = lambda t: 0 if t is None else t.data_ptr()
    worst = {"o": 0.0, "W": 0.0, "M": 0.0}
    worst_fro = {"o": 0.0, "W": 0.0, "M": 0.0}
    t_or = 0.0
    for c, f in enumerate(wl.flags):
        t0, t1 = wl.bounds[c], wl.bounds[c + 1]
        Lc = t1 - t0
        Wc = [[_f64(w[i]) for w in Ws] for i in inst]
        Mc = [[_f64(m[i]) for m in Ms] if mom else [np.zeros_like(w) for w in Wc[j]] for j, i in enumerate(inst)]
        if f & W.APPLY:   # apply-then-update: the chunk's queries read the weights before its update
            lact.check(lact.apply_ptr(p, q.data_ptr() + t0 * D * esz, Lc, L, *[w.data_ptr() for w in Ws],
                                      o.data_ptr() + t0 * D * esz, ws.data_ptr(), ws.numel(),
                                      torch.cuda.current_stream().cuda_stream))
        if f & W.UPDATE:
            lact.check(lact.chunk_update_ptr(
                p, k.data_ptr() + t0 * D * esz, v.data_ptr() + t0 * D * esz, lr.data_ptr() + t0 * 3 * 4,
                0 if beta is None else beta.data_ptr() + t0 * 4, Lc, L, *[w.data_ptr() for w in Ws],
                *[ptr(m) for m in Ms], ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        t = time.time()
        for j, i in enumerate(inst):
            if f & W.APPLY:
                ref = O.apply(*Wc[j], O.f64(inp.q[i][t0:t1]))
                g = _f64(o[i, t0:t1])
                worst["o"] = max(worst["o"], rel_err(g, ref))
                worst_fro["o"] = max(worst_fro["o"], fro_ratio(g, ref))
            if f & W.UPDATE:
                b = None if inp.beta is None else O.f64(inp.beta[i][t0:t1])
                Wn, Mn = O.update_step(Wc[j], Mc[j], O.f64(inp.k[i][t0:t1]), O.f64(inp.v[i][t0:t1]),
                                       O.f64(inp.lr[i][t0:t1]), b, wl.opt)
                for m in range(3):
                    g = _f64(Ws[m][i])
                    worst["W"] = max(worst["W"], rel_err(g, Wn[m]))
                    worst_fro["W"] = max(worst_fro["W"], fro_ratio(g, Wn[m]))
                    if mom:
                        g = _f64(Ms[m][i])
                        worst["M"] = max(worst["M"], rel_err(g, Mn[m]))
                        worst_fro["M"] = max(worst_fro["M"], fro_ratio(g, Mn[m]))
        t_or += time.time() - t
    log(f"  oracle {t_or:.1f}s per-chunk worst errs={ {k: f'{v:.2e}' for k, v in worst.items()} } "
        f"frobenius={ {k: f'{v:.2e}' for k, v in worst_fro.items()} } gate={wl.tol}")
    assert max(worst.values()) <= wl.tol, worst
