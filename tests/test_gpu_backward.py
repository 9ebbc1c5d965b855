"""GPU parity of the layer's backward pass (lact_layer_backward) with the fp64
backward oracle, element by element on the same seeded inputs.

err = max|gpu - ref| / max|ref| per output and instance (maximum over
instances).  The forward state trajectory is replayed fp32-grade; the
backward products take fp32 operands as three bf16 planes (fp32 grade) for
the Newton-Schulz optimisers and two (16-bit significands) for GD and
momentum, bf16 inputs exact in one plane, all with fp32 accumulation.  The
gate is the fp32 one, 1e-4 (two-plane cases measure up to 3.2e-5).

Exception, the Newton-Schulz optimisers at full workload length: the Muon
recurrence amplifies rounding (each chunk's step is a quintic polynomial of
the normalised gradient), so even a plain float32 evaluation of the oracle's
own arithmetic differs from float64 by E32 = 2.0e-4 on the 3B-LM workload
(d = 512, 8 chunks of 4,096; max over its 6 instances), 7.4e-5 with
momentum + Muon on the same shape, and 1.2e-2 on the video workload
(d = 128, 12 Muon chunks; instances 0, 13, 27, 39).  Their full-size gate
is 5 x E32, capped at the bf16-input gate of the forward (2e-2).
"""
import dataclasses

import numpy as np
import pytest

from oracle import lact_backward as OB
from test_layers_amd import workloads as W
from parity_util import log, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = 1e-4
# full-size gates of the Newton-Schulz workloads (5 x the plain-fp32 error, capped at 2e-2)
TOL_NS_FULL = {3: 1e-3, 5: 2e-2, 8: 4e-4}
OUTS = ("dq", "dk", "dv", "dlr", "dbeta", "doz", "dW1", "dW2", "dW3", "dM1", "dM2", "dM3")


@pytest.fixture(scope="module")
def lact():
    from test_layers_amd import lact as L
    return L


def cotangents(wl, seed, state_cot):
    """dO in the io dtype (bf16 as uint16 bits), final-state cotangents fp32."""
    rng = np.random.default_rng([seed, 77])
    dO = rng.standard_normal((wl.n_inst, wl.L, wl.D)).astype(np.float32)
    if wl.io_dtype == W.DTYPE_BF16:
        dO = W.f32_to_bf16_bits(dO)
    shapes = [(wl.n_inst, wl.dh, wl.D), (wl.n_inst, wl.D, wl.dh), (wl.n_inst, wl.dh, wl.D)]
    gW = [0.1 * rng.standard_normal(s).astype(np.float32) for s in shapes] if state_cot else None
    gM = [0.1 * rng.standard_normal(s).astype(np.float32) for s in shapes] if state_cot else None
    return dO, gW, gM


def run_case(lact, wl, seed=0, order=None, renorm=True, state_cot=True, M0_scale=0.0, instances=None):
    """Run the GPU backward on every instance; compare `instances` (default:
    all) with the oracle."""
    order = wl.order if order is None else order
    inp = W.generate(wl, seed=seed, threads=16)
    dO, gW, gM = cotangents(wl, seed, state_cot)
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    rng = np.random.default_rng([seed, 78])
    M0 = [(M0_scale * rng.standard_normal(w.shape)).astype(np.float32) for w in (inp.W1, inp.W2, inp.W3)]
    dev = lambda x: to_dev(x, torch)
    out = lact.layer_backward(
        dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.lr), dev(inp.beta) if mom else None,
        dev(inp.W1), dev(inp.W2), dev(inp.W3), *([dev(m) for m in M0] if mom else [None] * 3),
        dO=dev(dO), gW=None if gW is None else [dev(g) for g in gW],
        gM=None if gM is None else [dev(g) for g in gM], order=order, opt=wl.opt,
        bounds=list(wl.bounds), flags=list(wl.flags), renorm=renorm, qk_prep=wl.layer_qk_prep,
        oz=dev(inp.oz) if wl.out_scale else None)
    torch.cuda.synchronize()
    idx = list(range(wl.n_inst)) if instances is None else list(instances)
    pick = lambda x: None if x is None else x[idx]
    ref = OB.layer_backward(pick(inp.q), pick(inp.k), pick(inp.v), pick(inp.lr), pick(inp.beta) if mom else None,
                            pick(inp.W1), pick(inp.W2), pick(inp.W3), wl.bounds, wl.flags, order, wl.opt,
                            pick(dO), None if gW is None else [pick(g) for g in gW],
                            None if gM is None else [pick(g) for g in gM], renorm,
                            M=[pick(m) for m in M0] if mom else None, qk_prep=wl.layer_qk_prep,
                            oz=pick(inp.oz) if wl.out_scale else None)
    errs = {}
    for key in OUTS:
        g = out.get(key)
        if g is None:
            continue
        g = g.float().cpu().numpy().astype(np.float64)[idx]
        r = ref[key]
        e = 0.0
        for i in range(len(idx)):
            den = np.max(np.abs(r[i]))
            e = max(e, float(np.max(np.abs(g[i] - r[i])) / den) if den > 0 else float(np.max(np.abs(g[i]))))
        errs[key] = e
    if not mom:
        # GD / Muon: the momentum state passes through: dM = gM
        assert out["dM1"] is None and out["dbeta"] is None
    return errs


CASES = {
    # fp32 io, GD, three uniform chunks
    "f32_gd": W.WORKLOADS[1].scaled(n_inst=2, L=640, chunk=256),
    # bf16 io, momentum, ragged tail
    "bf16_momentum": W.WORKLOADS[2].scaled(n_inst=2, L=3 * 256 + 100, chunk=256),
    # bf16 io, Muon at d = 512 (3B-LM shape, reduced)
    "bf16_muon_d512": W.WORKLOADS[3].scaled(n_inst=2, L=2 * 512 + 64, chunk=512),
    # bf16 io, momentum + Muon
    "bf16_muon_momentum": W.WORKLOADS[8].scaled(n_inst=2, L=2 * 256 + 64, chunk=256),
    # view set: one update-only chunk then an apply-only chunk (update-then-apply)
    "viewset": dataclasses.replace(W.WORKLOADS[4], n_inst=2, L=1500, bounds=(0, 1200, 1500),
                                   flags=(W.UPDATE, W.APPLY)),
    # video: clean chunks update+apply, noisy chunks apply only
    "video": dataclasses.replace(W.WORKLOADS[5], n_inst=2, L=W.video_schedule(3, 200)[0][-1],
                                 bounds=W.video_schedule(3, 200)[0], flags=W.video_schedule(3, 200)[1]),
    # rectangular fast weights, dh > d, momentum
    "rect_dh_gt_d": W.WORKLOADS[10].scaled(n_inst=2, L=2 * 256 + 30, chunk=256),
    # raw q / k (pre-processed by the layer) and the per-token output scale
    "raw_qk_scaled": W.WORKLOADS[9].scaled(n_inst=2, L=3 * 256 + 100, chunk=256),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(lact, name):
    wl = CASES[name]
    log(f"backward {name}: n={wl.n_inst} d={wl.D} dh={wl.dh} L={wl.L} chunks={wl.n_chunks} opt={wl.opt}")
    errs = run_case(lact, wl, seed=1)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("opt", [W.OPT_GD, W.OPT_MOMENTUM, W.OPT_MUON, W.OPT_MUON_MOMENTUM])
@pytest.mark.parametrize("order", [W.APPLY_THEN_UPDATE, W.UPDATE_THEN_APPLY])
def test_backward_optimisers_orders_renorm(lact, opt, order):
    """Every optimiser x order, with and without renorm, nonzero initial
    momentum, fp32 io."""
    base = W.WORKLOADS[1].scaled(n_inst=2, L=3 * 128 + 40, chunk=128)
    wl = dataclasses.replace(base, opt=opt)
    for renorm in (True, False):
        errs = run_case(lact, wl, seed=2 + opt, order=order, renorm=renorm, M0_scale=0.05)
        log(f"  opt={opt} order={order} renorm={renorm}: errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
        assert max(errs.values()) <= TOL, (renorm, errs)


@pytest.mark.parametrize("shape", [(128, 64), (64, 192)])
@pytest.mark.parametrize("opt", [W.OPT_MUON, W.OPT_MUON_MOMENTUM])
def test_backward_rectangular_newton_schulz(lact, shape, opt):
    """d != dh in both orientations: the Newton-Schulz backward transposes the
    tall matrices, as the forward map does."""
    D, Dh = shape
    wl = dataclasses.replace(W.WORKLOADS[1].scaled(n_inst=2, L=2 * 128 + 20, chunk=128), D=D, Dh=Dh, opt=opt)
    errs = run_case(lact, wl, seed=5, M0_scale=0.05)
    log(f"  d={D} dh={Dh} opt={opt}: errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("order", [W.APPLY_THEN_UPDATE, W.UPDATE_THEN_APPLY])
def test_backward_raw_qk_output_scale_muon_fp32(lact, order):
    """Raw q / k and the output scale with fp32 inputs and Muon, both orders."""
    base = W.WORKLOADS[9].scaled(n_inst=2, L=3 * 128 + 40, chunk=128)
    wl = dataclasses.replace(base, D=64, io_dtype=W.DTYPE_F32, opt=W.OPT_MUON)
    errs = run_case(lact, wl, seed=8, order=order)
    log(f"  order={order}: errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert "doz" in errs and max(errs.values()) <= TOL, errs


def test_backward_without_state_cotangents(lact):
    """gW = gM = NULL means zero cotangents of the final state."""
    wl = W.WORKLOADS[2].scaled(n_inst=2, L=2 * 256, chunk=256)
    errs = run_case(lact, wl, seed=4, state_cot=False)
    assert max(errs.values()) <= TOL, errs


def test_backward_no_update_passes_state_cotangent_through(lact):
    """Apply-only schedule: dW = gW + the apply's weight gradients, dk = dv =
    dlr = 0 exactly, dM = gM exactly."""
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=2, L=300, chunk=300), bounds=(0, 300), flags=(W.APPLY,))
    errs = run_case(lact, wl, seed=6)
    assert max(errs.values()) <= TOL, errs


# ----------------------------------------------------------------- full workload sizes
FULL = {1: None, 2: None, 3: None, 4: None, 5: (0, 13, 27, 39), 8: None, 9: None, 10: None}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", sorted(FULL))
def test_backward_full_size(lact, cid):
    """The backward at the full workload sizes (every instance on the GPU;
    the oracle on all of them, or on a spread sample for the 40-head video
    workload)."""
    wl = W.WORKLOADS[cid]
    log(f"backward full cfg{cid} {wl.name}: n={wl.n_inst} d={wl.D} dh={wl.dh} L={wl.L} chunks={wl.n_chunks}")
    errs = run_case(lact, wl, seed=0, instances=FULL[cid])
    tol = TOL_NS_FULL[cid] if wl.opt in (W.OPT_MUON, W.OPT_MUON_MOMENTUM) else TOL
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} } gate={tol}")
    assert max(errs.values()) <= tol, errs


@pytest.mark.parametrize("opt", [W.OPT_MOMENTUM, W.OPT_MUON])
def test_backward_maximum_width(lact, opt):
    """d = dh = 1024, the widest the library takes (Newton-Schulz on
    1024 x 1024 matrices for Muon)."""
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=1, L=2 * 64 + 16, chunk=64), D=1024, opt=opt)
    errs = run_case(lact, wl, seed=9)
    log(f"  d=1024 opt={opt}: errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= TOL, errs


def test_backward_empty_sequence(lact):
    """L = 0: no chunk, so dW = gW and dM = gM exactly."""
    dev = "cuda"
    n, D = 2, 128
    g = torch.Generator(device="cpu").manual_seed(3)
    Ws = [torch.randn(n, D, D, generator=g).to(dev) for _ in range(3)]
    gW = [torch.randn(n, D, D, generator=g).to(dev) for _ in range(3)]
    gM = [torch.randn(n, D, D, generator=g).to(dev) for _ in range(3)]
    empty = torch.empty(n, 0, D, dtype=torch.bfloat16, device=dev)
    out = lact.layer_backward(empty, empty, empty, torch.empty(n, 0, 3, device=dev), torch.empty(n, 0, device=dev),
                              *Ws, *[torch.zeros_like(w) for w in Ws], dO=empty, gW=gW, gM=gM, chunk=64,
                              opt=W.OPT_MOMENTUM)
    torch.cuda.synchronize()
    for j in range(3):
        assert torch.equal(out[f"dW{j + 1}"], gW[j])
        assert torch.equal(out[f"dM{j + 1}"], gM[j])


def test_backward_single_token_chunk(lact):
    """A one-token last chunk (the shortest a chunk can be)."""
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=2, L=257, chunk=256))
    errs = run_case(lact, wl, seed=10)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("opt", [W.OPT_MOMENTUM, W.OPT_MUON])
def test_backward_replays_in_a_hip_graph(lact, opt):
    """The backward only enqueues kernels and device-to-device copies on the
    caller's stream (no allocation, memset or host synchronisation), so a HIP
    graph can capture it; every replay, with eager work and synchronisations
    between replays, equals the eager call bitwise and rewrites every
    output."""
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=2, L=2 * 256 + 40, chunk=256), opt=opt)
    inp = W.generate(wl, seed=23)
    dO, gW, gM = cotangents(wl, 23, True)
    dev = lambda x: to_dev(x, torch)
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ws = [dev(inp.W1), dev(inp.W2), dev(inp.W3)]
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    kw = dict(dO=dev(dO), gW=[dev(g) for g in gW], gM=[dev(g) for g in gM], order=wl.order, opt=wl.opt,
              bounds=list(wl.bounds), flags=list(wl.flags))
    q, k, v, lr = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.lr)
    beta = dev(inp.beta) if mom else None
    ref = lact.layer_backward(q, k, v, lr, beta, *Ws, *Ms, **kw)
    p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, 3)
    ws = torch.empty(lact.backward_workspace_size(p, wl.L, 0, wl.order, list(wl.bounds), list(wl.flags)),
                     dtype=torch.uint8, device="cuda")
    out = {key: (None if t is None else torch.empty_like(t)) for key, t in ref.items()}

    def call():
        lact.layer_backward(q, k, v, lr, beta, *Ws, *Ms, out=out, workspace=ws, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                        # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for t in out.values():
            if t is not None:
                t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for key, t in out.items():
            if t is not None:
                assert torch.equal(t, ref[key]), (rep, key)
        _ = float(out["dq"].sum())    # eager work between replays
    log(f"  opt={opt}: 3 graph replays of the backward equal the eager call")


@pytest.mark.parametrize("name", ["bf16_momentum", "bf16_muon_momentum", "raw_qk_scaled", "viewset"])
def test_backward_is_deterministic(lact, name):
    """Two backward calls on the same inputs give bitwise-identical
    gradients (split-K partials and every reduction summed in fixed order)."""
    wl = CASES[name]
    inp = W.generate(wl, seed=12)
    dO, gW, gM = cotangents(wl, 12, True)
    dev = lambda x: to_dev(x, torch)
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ws = [dev(inp.W1), dev(inp.W2), dev(inp.W3)]
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    call = lambda: lact.layer_backward(
        dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.lr), dev(inp.beta) if mom else None, *Ws, *Ms, dO=dev(dO),
        gW=[dev(g) for g in gW], gM=[dev(g) for g in gM], order=wl.order, opt=wl.opt, bounds=list(wl.bounds),
        flags=list(wl.flags), qk_prep=wl.layer_qk_prep, oz=dev(inp.oz) if wl.out_scale else None)
    a, b = call(), call()
    torch.cuda.synchronize()
    for key, t in a.items():
        if t is not None:
            assert torch.equal(t, b[key]), key
