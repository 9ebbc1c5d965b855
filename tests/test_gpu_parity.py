"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on
the same seeded inputs.  Gates: max|gpu - ref| / max|ref| <= 1e-4 for fp32
inputs and <= 2e-2 for bf16 inputs, per instance, on the APPLY rows of o and
on the final state."""
import numpy as np
import pytest

import oracle as O
from test_layers_amd import workloads as W
from parity_util import compare, from_dev, log, rel_err, run_gpu, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lact():
    from test_layers_amd import lact as L
    return L


def _gate(io):
    return 1e-4 if io == W.DTYPE_F32 else 2e-2


def _rand_inputs(n, L, D, io, seed, raw=False):
    wl = W.Workload(99, "unit", n, D, L, (0, L), (3,), 0, W.OPT_GD, io, not raw, 1, _gate(io))
    return W.generate(wl, seed=seed)


# ------------------------------------------------------------------ apply alone
@pytest.mark.parametrize("D", [64, 128, 384])
@pytest.mark.parametrize("io", [W.DTYPE_F32, W.DTYPE_BF16])
def test_apply_matches_oracle(lact, D, io):
    log(f"apply D={D} io={io}")
    n, L = 2, 300
    inp = _rand_inputs(n, L, D, io, seed=D + io)
    q = to_dev(inp.q, torch)
    Ws = [to_dev(w, torch) for w in (inp.W1, inp.W2, inp.W3)]
    o = lact.apply(q, *Ws)
    torch.cuda.synchronize()
    g = from_dev(o, torch)
    err = 0.0
    for i in range(n):
        ref = O.apply(O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i]), O.f64(inp.q[i]))
        err = max(err, rel_err(g[i], ref))
    log(f"  err={err:.3e}")
    assert err <= _gate(io)


def test_apply_respects_seq_stride_and_leaves_other_rows(lact):
    n, S, Lq, D = 2, 400, 257, 128
    inp = _rand_inputs(n, S, D, W.DTYPE_BF16, seed=5)
    q = to_dev(inp.q, torch)
    Ws = [to_dev(w, torch) for w in (inp.W1, inp.W2, inp.W3)]
    o = torch.full_like(q, 7.0)
    lact.apply(q, *Ws, o, Lq=Lq)
    torch.cuda.synchronize()
    g = from_dev(o, torch)
    assert np.all(g[:, Lq:] == 7.0)
    for i in range(n):
        ref = O.apply(O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i]), O.f64(inp.q[i][:Lq]))
        assert rel_err(g[i, :Lq], ref) <= 2e-2


# ------------------------------------------------------------------ one chunk update
@pytest.mark.parametrize("opt", [W.OPT_GD, W.OPT_MOMENTUM, W.OPT_MUON, W.OPT_MUON_MOMENTUM])
@pytest.mark.parametrize("io,planes", [(W.DTYPE_F32, 3), (W.DTYPE_BF16, 1), (W.DTYPE_BF16, 2),
                                       (W.DTYPE_BF16, 3)])
@pytest.mark.parametrize("D", [64, 128])
def test_chunk_update_matches_oracle(lact, opt, io, planes, D):
    log(f"chunk_update opt={opt} io={io} planes={planes} D={D}")
    n, Lc = 2, 300
    inp = _rand_inputs(n, Lc, D, io, seed=10 * D + opt)
    rng = np.random.default_rng(1)
    beta = rng.uniform(0.5, 0.99, (n, Lc)).astype(np.float32)
    M0 = [rng.standard_normal((n, D, D)).astype(np.float32) * 0.01 for _ in range(3)]
    k, v, lr = to_dev(inp.k, torch), to_dev(inp.v, torch), to_dev(inp.lr, torch)
    Ws = [to_dev(w, torch).clone() for w in (inp.W1, inp.W2, inp.W3)]
    mom = opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [to_dev(m, torch).clone() for m in M0] if mom else [None] * 3
    lact.chunk_update(k, v, lr, to_dev(beta, torch) if mom else None,
                      *Ws, *Ms, opt=opt, rec_planes=planes)
    torch.cuda.synchronize()
    errs = {}
    for i in range(n):
        Wr, Mr = O.update_step([O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i])],
                               [O.f64(m[i]) for m in M0], O.f64(inp.k[i]), O.f64(inp.v[i]),
                               O.f64(inp.lr[i]), O.f64(beta[i]), opt)
        for j, nm in enumerate(["W1", "W2", "W3"]):
            errs[nm] = max(errs.get(nm, 0), rel_err(from_dev(Ws[j], torch)[i], Wr[j]))
            if mom:
                errs["M" + nm[1]] = max(errs.get("M" + nm[1], 0), rel_err(from_dev(Ms[j], torch)[i], Mr[j]))
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    gate = _gate(io) if planes == 1 or io == W.DTYPE_F32 else 1e-3
    assert max(errs.values()) <= gate, errs


# ------------------------------------------------------------------ layer at reduced sizes
SMALL = {
    1: W.WORKLOADS[1],
    2: W.WORKLOADS[2].scaled(n_inst=2, L=3 * 512 + 200, chunk=512),
    3: W.WORKLOADS[3].scaled(n_inst=2, L=2 * 1024 + 300, chunk=1024),
}


def _small_viewset():
    c = W.WORKLOADS[4]
    b, f = (0, 4000, 4500), (W.UPDATE, W.APPLY)
    import dataclasses
    return dataclasses.replace(c, n_inst=2, L=4500, bounds=b, flags=f)


def _small_video():
    c = W.WORKLOADS[5]
    import dataclasses
    b, f = W.video_schedule(3, 700)
    return dataclasses.replace(c, n_inst=3, L=b[-1], bounds=b, flags=f)


def _small_prefill():
    c = W.WORKLOADS[6]
    b, f = (0, 4000, 4500), (W.UPDATE | W.APPLY, W.APPLY)
    import dataclasses
    return dataclasses.replace(c, n_inst=2, L=4500, bounds=b, flags=f)


def _small_video_noisy_first():
    c = W.WORKLOADS[7]
    import dataclasses
    b, f = W.video_schedule_noisy_first(3, 700)
    return dataclasses.replace(c, n_inst=3, L=b[-1], bounds=b, flags=f)


def _small_video_fused(noisy_first=False):
    """Video schedule with clean chunks of 1,100 tokens: long enough for the
    fused multi-plane update (17 token tiles of 64, the last one ragged)."""
    import dataclasses
    c = W.WORKLOADS[7 if noisy_first else 5]
    sched = W.video_schedule_noisy_first if noisy_first else W.video_schedule
    b, f = sched(3, 1100)
    return dataclasses.replace(c, n_inst=3, L=b[-1], bounds=b, flags=f)


SMALL[4] = _small_viewset()
SMALL[5] = _small_video()
SMALL[6] = _small_prefill()
SMALL[7] = _small_video_noisy_first()
SMALL[8] = W.WORKLOADS[8].scaled(n_inst=2, L=2 * 1024 + 300, chunk=1024)
SMALL[9] = W.WORKLOADS[9].scaled(n_inst=2, L=3 * 512 + 200, chunk=512)
SMALL[10] = W.WORKLOADS[10].scaled(n_inst=2, L=3 * 512 + 200, chunk=512)


SMALL["video_fused"] = _small_video_fused()
SMALL["video_noisy_first_fused"] = _small_video_fused(noisy_first=True)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, "video_fused", "video_noisy_first_fused"])
def test_layer_reduced_size(lact, cid):
    wl = SMALL[cid]
    log(f"layer reduced cfg{cid}: n={wl.n_inst} D={wl.D} L={wl.L} chunks={wl.n_chunks}")
    inp = W.generate(wl)
    gpu = run_gpu(wl, inp, torch, lact)
    errs = compare(wl, inp, gpu)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= wl.tol, errs


@pytest.mark.parametrize("order", [W.APPLY_THEN_UPDATE, W.UPDATE_THEN_APPLY])
def test_layer_orders_and_no_renorm(lact, order):
    wl = W.WORKLOADS[2].scaled(n_inst=2, L=1000, chunk=384)
    inp = W.generate(wl, seed=3)
    for renorm in (True, False):
        log(f"order={order} renorm={renorm}")
        gpu = run_gpu(wl, inp, torch, lact, order=order, renorm=renorm)
        errs = compare(wl, inp, gpu, order=order, renorm=renorm)
        log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
        assert max(errs.values()) <= wl.tol, errs


MIXED = {
    # ragged last update+apply chunk (333 tokens)
    "ragged": ((0, 512, 700, 1212, 1724, 2057),
               (W.UPDATE | W.APPLY, W.APPLY, W.UPDATE | W.APPLY, W.UPDATE, W.UPDATE | W.APPLY)),
    # a one-token update+apply chunk last, after an apply-only chunk at the start
    "one_token": ((0, 100, 612, 1124, 1125),
                  (W.APPLY, W.UPDATE | W.APPLY, W.UPDATE | W.APPLY, W.UPDATE | W.APPLY)),
}


@pytest.mark.parametrize("sched", sorted(MIXED))
@pytest.mark.parametrize("order", [W.APPLY_THEN_UPDATE, W.UPDATE_THEN_APPLY])
def test_layer_mixed_schedule_plain_bf16(lact, order, sched):
    """Plain bf16 at d = 384 on schedules that mix update+apply chunks
    (apply-then-update: their queries run in the update forward tile) with
    apply-only chunks that merge into the next step's apply range, an
    update-only chunk, and ragged or one-token last chunks."""
    import dataclasses
    b, f = MIXED[sched]
    wl = dataclasses.replace(W.WORKLOADS[2], n_inst=2, L=b[-1], bounds=b, flags=f)
    inp = W.generate(wl, seed=5)
    log(f"mixed schedule order={order}: bounds={b}")
    gpu = run_gpu(wl, inp, torch, lact, order=order)
    errs = compare(wl, inp, gpu, order=order)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= wl.tol, errs


# d = dh = 128: update chunks long enough for the fused update (>= 4,096
# tokens with one weight plane, >= 1,024 with planes) beside shorter ones that
# run the separate update forward and contraction, in one call
FUSED_MIXED = {
    "planes": (5, 3, (0, 1100, 1400, 2700, 3000), (W.UPDATE | W.APPLY, W.UPDATE | W.APPLY, W.APPLY,
                                                     W.UPDATE | W.APPLY)),
    "plain": (4, 1, (0, 4200, 4700, 5000), (W.UPDATE | W.APPLY, W.UPDATE | W.APPLY, W.UPDATE | W.APPLY)),
}


@pytest.mark.parametrize("case", sorted(FUSED_MIXED))
def test_layer_fused_and_separate_updates_in_one_call(lact, case):
    """A schedule mixing fused and separate update steps at d = dh = 128 (the
    workspace then holds the update-term buffer the separate steps need):
    three-plane Muon (the video recipe) and plain bf16 GD (the view-set
    recipe)."""
    import dataclasses
    cid, planes, b, f = FUSED_MIXED[case]
    wl = dataclasses.replace(W.WORKLOADS[cid], n_inst=2, L=b[-1], bounds=b, flags=f, rec_planes=planes,
                             order=W.APPLY_THEN_UPDATE)
    inp = W.generate(wl, seed=12)
    log(f"fused and separate updates ({case}): bounds={b}")
    gpu = run_gpu(wl, inp, torch, lact)
    errs = compare(wl, inp, gpu)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= wl.tol, errs


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, "fused_update", "video_fused"])
def test_layer_is_deterministic(lact, cid):
    """Every workload (reduced) run twice gives bitwise-identical outputs and
    state: no atomics, every reduction in a fixed order.  "fused_update": the
    view-set layer with a 4,608-token update chunk (the fused update kernel)."""
    import dataclasses
    if cid == "fused_update":
        wl = dataclasses.replace(W.WORKLOADS[4], n_inst=2, L=4608 + 512, bounds=(0, 4608, 4608 + 512),
                                 flags=(W.UPDATE, W.APPLY))
    else:
        wl = SMALL[cid]
    inp = W.generate(wl, seed=4)
    a = run_gpu(wl, inp, torch, lact)
    b = run_gpu(wl, inp, torch, lact)
    for key in ["o", "W1", "W2", "W3", "M1", "M2", "M3"]:
        if a[key] is not None:
            assert torch.equal(a[key], b[key]), key


def test_resume_equals_single_call(lact):
    """Chunks [0, c) then [c, n) with the state carried equal one call (bitwise:
    every kernel reduces in a fixed order)."""
    wl = W.WORKLOADS[2].scaled(n_inst=2, L=1536, chunk=512)
    inp = W.generate(wl, seed=6)
    full = run_gpu(wl, inp, torch, lact)
    q, k, v = to_dev(inp.q, torch), to_dev(inp.k, torch), to_dev(inp.v, torch)
    lr, beta = to_dev(inp.lr, torch), to_dev(inp.beta, torch)
    Ws = [to_dev(w, torch).clone() for w in (inp.W1, inp.W2, inp.W3)]
    Ms = [torch.zeros_like(w) for w in Ws]
    o = torch.zeros_like(q)
    s = 1024
    sl = lambda t: t[:, :s].contiguous()
    o1 = lact.layer_forward(sl(q), sl(k), sl(v), sl(lr), sl(beta), *Ws, *Ms, chunk=512,
                            opt=W.OPT_MOMENTUM)
    tl = lambda t: t[:, s:].contiguous()
    o2 = lact.layer_forward(tl(q), tl(k), tl(v), tl(lr), tl(beta), *Ws, *Ms, chunk=512,
                            opt=W.OPT_MOMENTUM)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), full["o"])
    for j, key in enumerate(["W1", "W2", "W3"]):
        assert torch.equal(Ws[j], full[key])


@pytest.mark.parametrize("opt", [W.OPT_MOMENTUM, W.OPT_MUON])
def test_layer_empty_sequence_leaves_the_state(lact, opt):
    """L = 0 on the device: the call succeeds, launches nothing that touches
    the state, and W (and M) come back bit-identical."""
    n, D = 2, 128
    rng = np.random.default_rng(21)
    Ws = [torch.from_numpy((rng.standard_normal((n, D, D)) / 8).astype(np.float32)).cuda() for _ in range(3)]
    Ms = [torch.from_numpy((rng.standard_normal((n, D, D)) / 64).astype(np.float32)).cuda() for _ in range(3)]
    W0, M0 = [w.clone() for w in Ws], [m.clone() for m in Ms]
    empty = torch.empty(n, 0, D, dtype=torch.bfloat16, device="cuda")
    o = lact.layer_forward(empty, empty, empty, torch.empty(n, 0, 3, device="cuda"),
                           torch.empty(n, 0, device="cuda"), *Ws, *Ms, chunk=64, opt=opt)
    torch.cuda.synchronize()
    assert o.shape == (n, 0, D)
    for a, b in zip(Ws + Ms, W0 + M0):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ raw q/k and the output scale
@pytest.mark.parametrize("io,planes,opt", [(W.DTYPE_F32, 3, W.OPT_GD), (W.DTYPE_BF16, 1, W.OPT_MOMENTUM),
                                           (W.DTYPE_BF16, 2, W.OPT_MUON),
                                           (W.DTYPE_BF16, 3, W.OPT_MUON_MOMENTUM)])
def test_layer_raw_qk_and_output_scale_every_profile(lact, io, planes, opt):
    """Every precision profile (the fp32 one scales inside the generic output
    GEMM, the bf16 ones inside the apply tile), with tokens whose scale
    pre-activation is 0 or far negative (silu = 0: the row must vanish)."""
    import dataclasses
    wl = dataclasses.replace(W.WORKLOADS[9].scaled(n_inst=2, L=900, chunk=256), io_dtype=io,
                             rec_planes=planes, opt=opt, tol=_gate(io))
    log(f"raw qk + scale io={io} planes={planes} opt={opt}")
    inp = W.generate(wl, seed=11)
    inp.oz[:, 5] = 0.0
    inp.oz[:, 6] = -200.0
    inp.oz[:, 7] = 60.0
    gpu = run_gpu(wl, inp, torch, lact)
    o = from_dev(gpu["o"], torch)
    assert np.all(o[:, 5:7] == 0.0)
    errs = compare(wl, inp, gpu)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= wl.tol, errs


@pytest.mark.parametrize("io", [W.DTYPE_F32, W.DTYPE_BF16])
def test_chunk_entry_points_with_raw_qk_and_stride(lact, io):
    """lact_chunk_update / lact_apply with LACT_QK_PREP and seq_stride > the
    tokens used: the pre-processed copies are packed while v, lr and o keep
    the caller's stride."""
    n, S, Lc, D = 2, 700, 531, 128
    inp = _rand_inputs(n, S, D, io, seed=21, raw=True)
    k, v, lr, q = (to_dev(x, torch) for x in (inp.k, inp.v, inp.lr, inp.q))
    Ws = [to_dev(w, torch).clone() for w in (inp.W1, inp.W2, inp.W3)]
    lact.chunk_update(k, v, lr, None, *Ws, Lc=Lc, qk_prep=True)
    o = torch.full_like(q, 3.0)
    lact.apply(q, *Ws, o, Lq=Lc, qk_prep=True)
    torch.cuda.synchronize()
    g = from_dev(o, torch)
    assert np.all(g[:, Lc:] == 3.0)
    ew, eo = 0.0, 0.0
    for i in range(n):
        kh = O.qk_preprocess(inp.k[i][:Lc])
        qh = O.qk_preprocess(inp.q[i][:Lc])
        Wr, _ = O.update_step([O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i])], [None] * 3,
                              kh, O.f64(inp.v[i][:Lc]), O.f64(inp.lr[i][:Lc]), None, W.OPT_GD)
        for j in range(3):
            ew = max(ew, rel_err(from_dev(Ws[j], torch)[i], Wr[j]))
        # the apply reads the GPU's updated weights: compare against the
        # oracle's apply on exactly those
        Wg = [from_dev(w, torch)[i] for w in Ws]
        eo = max(eo, rel_err(g[i, :Lc], O.apply(Wg[0], Wg[1], Wg[2], qh)))
    log(f"  io={io} W err={ew:.2e} o err={eo:.2e}")
    assert max(ew, eo) <= _gate(io)


# ------------------------------------------------------------------ rectangular fast weights (d != dh)
def _rect_inputs(n, L, d, dh, io, seed):
    import dataclasses
    wl = dataclasses.replace(W.Workload(99, "unit", n, d, L, (0, L), (3,), 0, W.OPT_GD, io, True, 1,
                                        _gate(io)), Dh=dh)
    return W.generate(wl, seed=seed)


@pytest.mark.parametrize("d,dh", [(128, 256), (384, 192), (64, 128), (256, 128), (384, 128)])
@pytest.mark.parametrize("io", [W.DTYPE_F32, W.DTYPE_BF16])
def test_apply_rectangular(lact, d, dh, io):
    log(f"apply d={d} dh={dh} io={io}")
    n, L = 2, 300
    inp = _rect_inputs(n, L, d, dh, io, seed=d + dh + io)
    q = to_dev(inp.q, torch)
    Ws = [to_dev(w, torch) for w in (inp.W1, inp.W2, inp.W3)]
    o = lact.apply(q, *Ws)
    torch.cuda.synchronize()
    g = from_dev(o, torch)
    assert g.shape == (n, L, d)
    err = max(rel_err(g[i], O.apply(O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i]), O.f64(inp.q[i])))
              for i in range(n))
    log(f"  err={err:.3e}")
    assert err <= _gate(io)


# Newton-Schulz in one bf16 plane is not part of this grid: the quintic map's
# slope near a zero singular value is a^5 ~ 487, so the bf16 rounding of its
# products is amplified to 1.6-2.1e-2 on 128 x 256 matrices (at the 2e-2
# gate); the Muon workloads run two or three planes.
RECT_CASES = [(opt, io, planes) for opt in (W.OPT_GD, W.OPT_MOMENTUM, W.OPT_MUON, W.OPT_MUON_MOMENTUM)
              for io, planes in ((W.DTYPE_F32, 3), (W.DTYPE_BF16, 1), (W.DTYPE_BF16, 2), (W.DTYPE_BF16, 3))
              if not (planes == 1 and opt in (W.OPT_MUON, W.OPT_MUON_MOMENTUM))]


@pytest.mark.parametrize("opt,io,planes", RECT_CASES)
@pytest.mark.parametrize("d,dh", [(128, 256), (192, 64)])
def test_chunk_update_rectangular(lact, opt, io, planes, d, dh):
    log(f"chunk_update d={d} dh={dh} opt={opt} io={io} planes={planes}")
    n, Lc = 2, 300
    inp = _rect_inputs(n, Lc, d, dh, io, seed=7 * d + dh + opt)
    rng = np.random.default_rng(3)
    beta = rng.uniform(0.5, 0.99, (n, Lc)).astype(np.float32)
    M0 = [(rng.standard_normal(w.shape) * 0.01).astype(np.float32) for w in (inp.W1, inp.W2, inp.W3)]
    k, v, lr = to_dev(inp.k, torch), to_dev(inp.v, torch), to_dev(inp.lr, torch)
    Ws = [to_dev(w, torch).clone() for w in (inp.W1, inp.W2, inp.W3)]
    mom = opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [to_dev(m, torch).clone() for m in M0] if mom else [None] * 3
    lact.chunk_update(k, v, lr, to_dev(beta, torch) if mom else None, *Ws, *Ms, opt=opt, rec_planes=planes)
    torch.cuda.synchronize()
    errs = {}
    for i in range(n):
        Wr, Mr = O.update_step([O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i])],
                               [O.f64(m[i]) for m in M0], O.f64(inp.k[i]), O.f64(inp.v[i]),
                               O.f64(inp.lr[i]), O.f64(beta[i]), opt)
        for j, nm in enumerate(["W1", "W2", "W3"]):
            errs[nm] = max(errs.get(nm, 0), rel_err(from_dev(Ws[j], torch)[i], Wr[j]))
            if mom:
                errs["M" + nm[1]] = max(errs.get("M" + nm[1], 0), rel_err(from_dev(Ms[j], torch)[i], Mr[j]))
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    gate = _gate(io) if planes == 1 or io == W.DTYPE_F32 else 1e-3
    assert max(errs.values()) <= gate, errs


@pytest.mark.parametrize("io,planes,opt", [(W.DTYPE_F32, 3, W.OPT_MOMENTUM), (W.DTYPE_BF16, 1, W.OPT_MOMENTUM),
                                           (W.DTYPE_BF16, 2, W.OPT_MOMENTUM), (W.DTYPE_F32, 3, W.OPT_MUON_MOMENTUM),
                                           (W.DTYPE_BF16, 2, W.OPT_MUON_MOMENTUM),
                                           (W.DTYPE_BF16, 3, W.OPT_MUON)])
def test_layer_rectangular_every_profile(lact, io, planes, opt):
    """The full layer with dh < d and dh > d (ragged last chunk), every profile."""
    import dataclasses
    for d, dh in [(128, 64), (64, 192)]:
        wl = dataclasses.replace(W.WORKLOADS[10].scaled(n_inst=2, L=700, chunk=256), D=d, Dh=dh, io_dtype=io,
                                 rec_planes=planes, opt=opt, tol=_gate(io))
        log(f"layer d={d} dh={dh} io={io} planes={planes} opt={opt}")
        inp = W.generate(wl, seed=5)
        gpu = run_gpu(wl, inp, torch, lact)
        errs = compare(wl, inp, gpu)
        log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
        assert max(errs.values()) <= wl.tol, errs


# ------------------------------------------------------------------ the largest widths
@pytest.mark.parametrize("d,dh,io,planes,opt", [
    (1024, 1024, W.DTYPE_BF16, 1, W.OPT_MOMENTUM),
    (1024, 1024, W.DTYPE_BF16, 2, W.OPT_MUON),
    (1024, 1024, W.DTYPE_F32, 3, W.OPT_GD),
    (1024, 128, W.DTYPE_BF16, 1, W.OPT_MOMENTUM),   # fused apply, eight output blocks
    (64, 1024, W.DTYPE_BF16, 2, W.OPT_MUON_MOMENTUM),
])
def test_layer_maximum_width(lact, d, dh, io, planes, opt):
    """The largest widths the library accepts (1024), ragged chunks."""
    import dataclasses
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=1, L=700, chunk=256), D=d, Dh=dh, io_dtype=io,
                             rec_planes=planes, opt=opt, tol=_gate(io))
    log(f"layer d={d} dh={dh} io={io} planes={planes} opt={opt}")
    inp = W.generate(wl, seed=9)
    gpu = run_gpu(wl, inp, torch, lact)
    errs = compare(wl, inp, gpu)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= wl.tol, errs


# ------------------------------------------------------------------ degenerate inputs
@pytest.mark.parametrize("opt", [W.OPT_GD, W.OPT_MOMENTUM, W.OPT_MUON, W.OPT_MUON_MOMENTUM])
def test_zero_learning_rates_leave_the_state_unchanged(lact, opt):
    """lr = 0: U = 0, NS5(0) = 0 and the renorm ratio is exactly 1, so W (and
    M = 0) come back bit-identical, and every output row is the plain SwiGLU
    MLP of the initial weights."""
    import dataclasses
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=2, L=700, chunk=256), D=128, opt=opt, rec_planes=2)
    inp = W.generate(wl, seed=13)
    inp.lr[:] = 0.0
    gpu = run_gpu(wl, inp, torch, lact)
    for j, key in enumerate(["W1", "W2", "W3"]):
        assert torch.equal(gpu[key], to_dev(getattr(inp, key), torch)), key
        if gpu["M" + key[1]] is not None:
            assert not torch.any(gpu["M" + key[1]]), "M"
    g = from_dev(gpu["o"], torch)
    err = max(rel_err(g[i], O.apply(O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i]), O.f64(inp.q[i])))
              for i in range(wl.n_inst))
    log(f"  opt={opt} o err={err:.2e}")
    assert err <= wl.tol


# ------------------------------------------------------------------ fused update (long chunks, d = dh = 128, bf16)
@pytest.mark.parametrize("n,Lc,opt", [(2, 4096 + 77, W.OPT_GD), (6, 9000, W.OPT_MOMENTUM), (6, 6000, W.OPT_MUON),
                                      (3, 20000, W.OPT_MUON_MOMENTUM)])
def test_long_chunk_update_fused(lact, n, Lc, opt):
    """Chunks of >= 4,096 tokens at d = dh = 128 in plain bf16 run the update
    forward and the contraction as one kernel (several token tiles per split,
    ragged last tile, beta partial sums for momentum); seq_stride > Lc."""
    log(f"fused update n={n} Lc={Lc} opt={opt}")
    D, S = 128, Lc + 50
    inp = _rand_inputs(n, S, D, W.DTYPE_BF16, seed=Lc + opt)
    rng = np.random.default_rng(8)
    beta = rng.uniform(0.5, 0.99, (n, S)).astype(np.float32)
    M0 = [(rng.standard_normal((n, D, D)) * 0.01).astype(np.float32) for _ in range(3)]
    k, v, lr = to_dev(inp.k, torch), to_dev(inp.v, torch), to_dev(inp.lr, torch)
    Ws = [to_dev(w, torch).clone() for w in (inp.W1, inp.W2, inp.W3)]
    mom = opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [to_dev(m, torch).clone() for m in M0] if mom else [None] * 3
    lact.chunk_update(k, v, lr, to_dev(beta, torch) if mom else None, *Ws, *Ms, Lc=Lc, opt=opt, rec_planes=1)
    torch.cuda.synchronize()
    errs = {}
    for i in range(n):
        Wr, Mr = O.update_step([O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i])],
                               [O.f64(m[i]) for m in M0], O.f64(inp.k[i][:Lc]), O.f64(inp.v[i][:Lc]),
                               O.f64(inp.lr[i][:Lc]), O.f64(beta[i][:Lc]), opt)
        for j, nm in enumerate(["W1", "W2", "W3"]):
            errs[nm] = max(errs.get(nm, 0), rel_err(from_dev(Ws[j], torch)[i], Wr[j]))
            if mom:
                errs["M" + nm[1]] = max(errs.get("M" + nm[1], 0), rel_err(from_dev(Ms[j], torch)[i], Mr[j]))
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= 2e-2, errs


@pytest.mark.parametrize("n,Lc,opt,planes", [(2, 1024, W.OPT_GD, 3), (3, 1024 + 77, W.OPT_MOMENTUM, 3),
                                             (3, 4680, W.OPT_MUON, 3), (2, 3000 + 5, W.OPT_MUON_MOMENTUM, 3),
                                             (5, 2100, W.OPT_MUON, 2), (2, 1500 + 33, W.OPT_MOMENTUM, 2)])
def test_long_chunk_update_fused_planes(lact, n, Lc, opt, planes):
    """Chunks of >= 1,024 tokens at d = dh = 128 with two or three weight
    planes run the fused multi-plane update (update terms split into planes
    in LDS, several token tiles per split, ragged last tile, beta partial
    sums for momentum); seq_stride > Lc."""
    log(f"fused plane update n={n} Lc={Lc} opt={opt} planes={planes}")
    D, S = 128, Lc + 40
    inp = _rand_inputs(n, S, D, W.DTYPE_BF16, seed=Lc + 7 * opt + planes)
    rng = np.random.default_rng(9)
    beta = rng.uniform(0.5, 0.99, (n, S)).astype(np.float32)
    M0 = [(rng.standard_normal((n, D, D)) * 0.01).astype(np.float32) for _ in range(3)]
    k, v, lr = to_dev(inp.k, torch), to_dev(inp.v, torch), to_dev(inp.lr, torch)
    Ws = [to_dev(w, torch).clone() for w in (inp.W1, inp.W2, inp.W3)]
    mom = opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [to_dev(m, torch).clone() for m in M0] if mom else [None] * 3
    lact.chunk_update(k, v, lr, to_dev(beta, torch) if mom else None, *Ws, *Ms, Lc=Lc, opt=opt,
                      rec_planes=planes)
    torch.cuda.synchronize()
    errs = {}
    for i in range(n):
        Wr, Mr = O.update_step([O.f64(inp.W1[i]), O.f64(inp.W2[i]), O.f64(inp.W3[i])],
                               [O.f64(m[i]) for m in M0], O.f64(inp.k[i][:Lc]), O.f64(inp.v[i][:Lc]),
                               O.f64(inp.lr[i][:Lc]), O.f64(beta[i][:Lc]), opt)
        for j, nm in enumerate(["W1", "W2", "W3"]):
            errs[nm] = max(errs.get(nm, 0), rel_err(from_dev(Ws[j], torch)[i], Wr[j]))
            if mom:
                errs["M" + nm[1]] = max(errs.get("M" + nm[1], 0), rel_err(from_dev(Ms[j], torch)[i], Mr[j]))
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= 1e-3, errs


def test_layer_d128_fused_apply_with_output_scale(lact):
    """d = dh = 128 in bf16: the fused apply (Hq kept in LDS) with the
    per-token output scale in its epilogue and raw q, k, over several apply
    groups and instances."""
    import dataclasses
    wl = dataclasses.replace(W.WORKLOADS[9].scaled(n_inst=3, L=6000, chunk=1000), D=128, opt=W.OPT_GD)
    log(f"fused apply with output scale n={wl.n_inst} L={wl.L} chunks={wl.n_chunks}")
    inp = W.generate(wl, seed=17)
    gpu = run_gpu(wl, inp, torch, lact)
    errs = compare(wl, inp, gpu)
    log(f"  errs={ {k: f'{v:.2e}' for k, v in errs.items()} }")
    assert max(errs.values()) <= wl.tol, errs


# ------------------------------------------------------------------ HIP graph capture
@pytest.mark.parametrize("cid", [2, 4, 3, "video_fused"])
def test_layer_replays_in_a_hip_graph(lact, cid):
    """The layer only enqueues kernels on the caller's stream (no allocation,
    memset, copy or host synchronisation), so a HIP graph can capture a whole
    layer forward; every replay, with eager work and synchronisations between
    replays, equals the eager call bitwise.  The Newton-Schulz layers (3:
    d = 512, the orthogonalisation on two helper streams; video_fused:
    d = 128, the fused update and the applies on a helper stream) fork from
    and join the caller's stream, which the capture follows."""
    wl = W.WORKLOADS[2].scaled(n_inst=2, L=1500, chunk=512) if cid == 2 else SMALL[cid]
    inp = W.generate(wl, seed=21)
    ref = run_gpu(wl, inp, torch, lact)
    q, k, v, lr, beta = (to_dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.lr, inp.beta))
    W0 = [to_dev(w, torch) for w in (inp.W1, inp.W2, inp.W3)]
    Ws = [w.clone() for w in W0]
    mom = wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    o = torch.zeros_like(q)
    p = lact.problem(wl.n_inst, wl.D, wl.io_dtype, wl.opt, wl.rec_planes)
    ws = torch.empty(lact.workspace_size(p, wl.L, 0, wl.order, list(wl.bounds), list(wl.flags)),
                     dtype=torch.uint8, device="cuda")

    def layer():
        for w, w0 in zip(Ws, W0):
            w.copy_(w0)
        for m in Ms:
            if m is not None:
                m.zero_()
        lact.layer_forward(q, k, v, lr, beta, *Ws, *Ms, o, order=wl.order, opt=wl.opt, bounds=list(wl.bounds),
                           flags=list(wl.flags), rec_planes=wl.rec_planes, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    applied = torch.zeros(wl.L, dtype=torch.bool, device="cuda")   # rows the schedule writes
    for c, f in enumerate(wl.flags):
        if f & W.APPLY:
            applied[wl.bounds[c]:wl.bounds[c + 1]] = True
    for rep in range(3):
        o.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o[:, applied], ref["o"][:, applied]), rep
        assert bool((o[:, ~applied] == -1.0).all()), rep      # rows of non-APPLY chunks untouched
        for j, key in enumerate(["W1", "W2", "W3"]):
            assert torch.equal(Ws[j], ref[key]), (rep, key)
            if mom:
                assert torch.equal(Ms[j], ref["M" + key[1]]), (rep, key)
        _ = float((o.float() * 2).sum())   # eager work between replays
    log(f"  cfg{cid}: 3 graph replays equal the eager layer")
