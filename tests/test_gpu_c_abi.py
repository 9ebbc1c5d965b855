"""The layer through the C ABI alone: tests/c_layer_run (plain C: hipMalloc,
a stream of its own, lact_layer_forward then lact_layer_backward, no torch)
on seeded inputs written to files.  Its results must equal, bitwise, those
of the torch binding on the same inputs (same library, deterministic
kernels; the C program zero-fills its workspace where torch leaves it
uninitialised, so this also shows no kernel reads workspace it has not
written), and match the fp64 oracle at the gates."""
import os
import subprocess

import numpy as np
import pytest

from oracle import lact_backward as OB
import oracle as O
from test_layers_amd import workloads as W
from parity_util import log, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_layer_run")


def _read(path, dtype, shape):
    return np.fromfile(path, dtype=dtype).reshape(shape)


@pytest.mark.parametrize("opt,planes", [(W.OPT_MOMENTUM, 1), (W.OPT_MUON, 2)])
def test_layer_through_the_c_abi_alone(tmp_path, opt, planes):
    import dataclasses
    if not os.path.exists(EXE):
        pytest.skip("tests/c_layer_run is not built (__graft_entry__.build() builds it)")
    from test_layers_amd import lact
    wl = dataclasses.replace(W.WORKLOADS[2].scaled(n_inst=2, L=2 * 512 + 160, chunk=512), opt=opt)
    inp = W.generate(wl, seed=31)
    mom = opt in (W.OPT_MOMENTUM, W.OPT_MUON_MOMENTUM)
    rng = np.random.default_rng([31, 77])
    dO = W.f32_to_bf16_bits(rng.standard_normal((wl.n_inst, wl.L, wl.D)).astype(np.float32))
    files = {"q": inp.q, "k": inp.k, "v": inp.v, "dO": dO, "lr": inp.lr, "W1": inp.W1, "W2": inp.W2, "W3": inp.W3}
    if mom:
        files["beta"] = inp.beta
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(str(tmp_path / f"{name}.bin"))
    cmd = [EXE, str(tmp_path), str(wl.n_inst), str(wl.D), str(wl.dh), str(wl.L), "512", str(wl.io_dtype), str(opt),
           str(planes)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    n, L, D = wl.n_inst, wl.L, wl.D
    shapes = {"W1": (n, wl.dh, D), "W2": (n, D, wl.dh), "W3": (n, wl.dh, D)}
    c = {"o": _read(tmp_path / "o.bin", np.uint16, (n, L, D))}
    for key in ("W1", "W2", "W3"):
        c[key] = _read(tmp_path / f"{key}o.bin", np.float32, shapes[key])
        c["d" + key] = _read(tmp_path / f"d{key}.bin", np.float32, shapes[key])
    for key in ("dq", "dk", "dv"):
        c[key] = _read(tmp_path / f"{key}.bin", np.float32, (n, L, D))
    c["dlr"] = _read(tmp_path / "dlr.bin", np.float32, (n, L, 3))
    if mom:
        c["dbeta"] = _read(tmp_path / "dbeta.bin", np.float32, (n, L))

    # the same calls through the torch binding
    dev = lambda x: to_dev(x, torch)
    Ws = [dev(inp.W1).clone(), dev(inp.W2).clone(), dev(inp.W3).clone()]
    Ms = [torch.zeros_like(w) for w in Ws] if mom else [None] * 3
    o = lact.layer_forward(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.lr), dev(inp.beta) if mom else None, *Ws,
                           *Ms, chunk=512, opt=opt, rec_planes=planes)
    g = lact.layer_backward(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.lr), dev(inp.beta) if mom else None,
                            dev(inp.W1), dev(inp.W2), dev(inp.W3), *([torch.zeros_like(w) for w in Ws] if mom else
                                                                     [None] * 3),
                            dO=dev(dO), chunk=512, opt=opt)
    torch.cuda.synchronize()
    t = {"o": o.view(torch.int16).cpu().numpy().view(np.uint16), "W1": Ws[0].cpu().numpy(),
         "W2": Ws[1].cpu().numpy(), "W3": Ws[2].cpu().numpy()}
    for key in ("dq", "dk", "dv", "dlr", "dW1", "dW2", "dW3") + (("dbeta",) if mom else ()):
        t[key] = g[key].cpu().numpy()
    for key, val in c.items():
        assert np.array_equal(val, t[key]), f"{key}: the C program and the torch binding differ"

    # and the oracle
    ref = O.layer_forward(inp.q, inp.k, inp.v, inp.lr, inp.beta if mom else None, inp.W1, inp.W2, inp.W3,
                          wl.bounds, wl.flags, wl.order, opt)
    worst = max(float(np.max(np.abs(W.bf16_bits_to_f32(c["o"]).astype(np.float64) - ref["o"]))
                      / np.max(np.abs(ref["o"]))),
                *[float(np.max(np.abs(c[k].astype(np.float64) - ref[k])) / np.max(np.abs(ref[k])))
                  for k in ("W1", "W2", "W3")])
    gref = OB.layer_backward(inp.q, inp.k, inp.v, inp.lr, inp.beta if mom else None, inp.W1, inp.W2, inp.W3,
                             wl.bounds, wl.flags, wl.order, opt, dO)
    gworst = max(float(np.max(np.abs(c[k].astype(np.float64) - gref[k])) / np.max(np.abs(gref[k])))
                 for k in ("dq", "dk", "dv", "dlr", "dW1", "dW2", "dW3"))
    log(f"  opt={opt}: C program == torch binding bitwise; forward err {worst:.2e}, backward err {gworst:.2e}")
    assert worst <= 2e-2 and gworst <= 1e-4, (worst, gworst)
