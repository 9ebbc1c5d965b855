"""The allocation-free entry point lact_layer_forward_noalloc, called through
the C ABI, against lact_layer_forward with a caller workspace: two calls in
a row on the device's shared scratch array (the second on a smaller problem,
so stale contents of the first are still in the array), each bitwise equal to
the existing entry point (same kernels, fixed-order reductions) and within the
bf16 gate of the fp64 oracle."""
import numpy as np
import pytest

from test_layers_amd import workloads as W
from parity_util import compare, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lact():
    from test_layers_amd import lact as L
    return L


def _inputs(wl, seed):
    inp = W.generate(wl, seed=seed)
    dev = {name: to_dev(getattr(inp, name), torch) for name in ("q", "k", "v", "lr", "beta")}
    return inp, dev


def _state(inp, wl):
    Ws = [to_dev(inp.W1, torch).clone(), to_dev(inp.W2, torch).clone(), to_dev(inp.W3, torch).clone()]
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    return Ws, Ms


def _noalloc(lact, wl, dev, Ws, Ms, o):
    p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, wl.rec_planes, dh=wl.dh)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lact.layer_forward_noalloc_ptr(p, ptr(dev["q"]), ptr(dev["k"]), ptr(dev["v"]), ptr(dev["lr"]),
                                        ptr(dev["beta"]), wl.L, 0, wl.order, list(wl.bounds), list(wl.flags),
                                        *[ptr(w) for w in Ws], *[ptr(m) for m in Ms], ptr(o),
                                        torch.cuda.current_stream().cuda_stream)
    lact.check(st)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cid,sizes", [
    (2, [(3, 1536, 512), (2, 700, 256)]),    # momentum, plain bf16 (second: ragged last chunk)
    (3, [(2, 1024, 512), (1, 512, 256)]),    # Muon, two-plane recurrence
    (5, [(4, 1400, 280), (2, 560, 280)]),    # d = 128 Muon, three-plane recurrence
    (5, [(3, 2400, 1200), (2, 1100, 1100)]),  # ... in chunks long enough for the fused update
])
def test_noalloc_matches_the_workspace_entry_point(lact, cid, sizes):
    for n, L, chunk in sizes:
        wl = W.WORKLOADS[cid].scaled(n_inst=n, L=L, chunk=chunk)
        p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, wl.rec_planes, dh=wl.dh)
        need = lact.workspace_size(p, wl.L, 0, wl.order, list(wl.bounds), list(wl.flags))
        assert need <= lact.NOALLOC_SCRATCH_BYTES
        log(f"noalloc cfg{cid} n={n} L={L} chunk={chunk} workspace {need} bytes")
        inp, dev = _inputs(wl, seed=31 + n)
        Wa, Ma = _state(inp, wl)
        oa = torch.full_like(dev["q"], 3.0)
        lact.layer_forward(dev["q"], dev["k"], dev["v"], dev["lr"], dev["beta"], *Wa, *Ma, oa, order=wl.order,
                           opt=wl.opt, bounds=list(wl.bounds), flags=list(wl.flags), rec_planes=wl.rec_planes)
        Wb, Mb = _state(inp, wl)
        ob = torch.full_like(dev["q"], 3.0)
        _noalloc(lact, wl, dev, Wb, Mb, ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob)
        for x, y in zip(Wa + Ma, Wb + Mb):
            if x is not None:
                assert torch.equal(x, y)
        gpu = {"o": ob, "W1": Wb[0], "W2": Wb[1], "W3": Wb[2], "M1": Mb[0], "M2": Mb[1], "M3": Mb[2]}
        errs = compare(wl, inp, gpu)
        log(f"  oracle errs { {k: f'{v:.2e}' for k, v in errs.items()} }")
        assert max(errs.values()) <= wl.tol, errs


def test_noalloc_rejects_a_problem_beyond_its_scratch(lact):
    wl = W.WORKLOADS[3]   # the 3B-LM layer needs far more than the scratch array
    p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, wl.rec_planes, dh=wl.dh)
    assert lact.workspace_size(p, wl.L, wl.max_chunk) > lact.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, dtype=torch.float32, device="cuda")   # never dereferenced: rejected before device work
    a = x.data_ptr()
    st = lact.layer_forward_noalloc_ptr(p, a, a, a, a, None, wl.L, wl.max_chunk, 0, None, None, a, a, a,
                                        None, None, None, a, None)
    assert st == lact.ERR_WORKSPACE_TOO_SMALL
    assert "LACT_NOALLOC_SCRATCH_BYTES" in lact.last_error()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cid,n,L,chunk", [(2, 2, 1736, 512), (3, 2, 2348, 1024)])
def test_noalloc_replays_in_a_hip_graph(lact, cid, n, L, chunk):
    """The callers the allocation-free entry point is for may capture it: a
    HIP graph of one call (the 3B-LM shape forks its orthogonalisation to the
    helper streams and joins them) replays three times, with eager work and
    synchronisations between the replays, each bitwise equal to the
    workspace entry point's eager call."""
    wl = W.WORKLOADS[cid].scaled(n_inst=n, L=L, chunk=chunk)
    inp, dev = _inputs(wl, seed=41 + cid)
    Wa, Ma = _state(inp, wl)
    oa = torch.zeros_like(dev["q"])
    lact.layer_forward(dev["q"], dev["k"], dev["v"], dev["lr"], dev["beta"], *Wa, *Ma, oa, order=wl.order,
                       opt=wl.opt, bounds=list(wl.bounds), flags=list(wl.flags), rec_planes=wl.rec_planes)
    W0, _ = _state(inp, wl)
    Wb, Mb = _state(inp, wl)
    ob = torch.zeros_like(dev["q"])

    def call():
        for w, w0 in zip(Wb, W0):
            w.copy_(w0)
        for m in Mb:
            if m is not None:
                m.zero_()
        _noalloc(lact, wl, dev, Wb, Mb, ob)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        ob.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, oa), rep
        for x, y in zip(Wa + Ma, Wb + Mb):
            if x is not None:
                assert torch.equal(x, y), rep
        _ = float((ob.float() * 2).sum())   # eager work between replays
    log(f"  noalloc cfg{cid}: 3 graph replays equal the workspace entry point")
