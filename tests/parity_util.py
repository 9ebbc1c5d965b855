"""Helpers shared by the GPU parity tests: upload generated inputs, run the
HIP layer through the C ABI, run the oracle instance by instance, and measure
err = max|gpu - ref| / max|ref| per instance (maximum over instances)."""
import sys
import time

import numpy as np

import oracle as O
from test_layers_amd import workloads as W


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x, torch):
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_dev(t, torch):
    """Device tensor -> float64 numpy (exact for fp32 and bf16)."""
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(wl: W.Workload, inp: W.Inputs, torch, lact, rec_planes=None, order=None,
            renorm=True, o_init=None):
    q, k, v = to_dev(inp.q, torch), to_dev(inp.k, torch), to_dev(inp.v, torch)
    lr = to_dev(inp.lr, torch)
    beta = to_dev(inp.beta, torch)
    Ws = [to_dev(inp.W1, torch).clone(), to_dev(inp.W2, torch).clone(), to_dev(inp.W3, torch).clone()]
    Ms = [None] * 3
    if wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM):
        Ms = [torch.zeros_like(w) for w in Ws]
    o = torch.zeros_like(q) if o_init is None else o_init
    oz = to_dev(inp.oz, torch) if wl.out_scale else None
    lact.layer_forward(q, k, v, lr, beta, *Ws, *Ms, o, order=wl.order if order is None else order,
                       opt=wl.opt, bounds=list(wl.bounds), flags=list(wl.flags),
                       rec_planes=wl.rec_planes if rec_planes is None else rec_planes, renorm=renorm,
                       qk_prep=wl.layer_qk_prep, oz=oz)
    torch.cuda.synchronize()
    return {"o": o, "W1": Ws[0], "W2": Ws[1], "W3": Ws[2], "M1": Ms[0], "M2": Ms[1], "M3": Ms[2]}


def rel_err(x, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / den) if den > 0 else float(np.max(np.abs(x)))


def fro_ratio(x, ref):
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def compare(wl: W.Workload, inp: W.Inputs, gpu, order=None, renorm=True, instances=None, fro=None):
    """Oracle instance by instance; returns {tensor: max over instances of err}.
    If `fro` is a dict it receives the Frobenius ratios ||gpu - ref|| / ||ref||
    (max over instances) as well."""
    keys = ["o", "W1", "W2", "W3"] + (["M1", "M2", "M3"] if wl.opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM) else [])
    errs = {k: 0.0 for k in keys}
    idx = range(wl.n_inst) if instances is None else instances
    for i in idx:
        ref = O.forward_instance(inp.q[i], inp.k[i], inp.v[i], inp.lr[i],
                                 None if inp.beta is None else inp.beta[i],
                                 inp.W1[i], inp.W2[i], inp.W3[i], wl.bounds, wl.flags,
                                 wl.order if order is None else order, wl.opt, renorm=renorm,
                                 qk_prep=wl.layer_qk_prep,
                                 oz=inp.oz[i] if wl.out_scale else None)
        mask = ref["o_mask"]
        for key in keys:
            g = gpu[key][i]
            g = g.float().cpu().numpy().astype(np.float64)
            r = ref[key]
            if key == "o":
                g, r = g[mask], r[mask]
            errs[key] = max(errs[key], rel_err(g, r))
            if fro is not None:
                fro[key] = max(fro.get(key, 0.0), fro_ratio(g, r))
    return errs
