"""C-ABI checks that need no GPU: the library loads, exports every function
include/lact.h declares, the header is valid C11, and every validation path
returns its error code before any device work."""
import ctypes
import functools
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lact.h")

lact = pytest.importorskip("test_layers_amd.lact", reason="liblact.so not built")

# An aligned non-null address.  Validation never dereferences it, but an
# argument set that passes validation goes on to enqueue kernels on it if a
# device is visible: such calls are made only under @device_free.
FAKE = 1 << 20

_CHILD_FLAG = "LACT_ABI_DEVICE_FREE_CHILD"


def _device_visible() -> bool:
    try:
        import torch
    except ImportError:
        return True   # cannot tell: treat as visible
    return torch.cuda.device_count() > 0


def device_free(fn):
    """For tests whose calls pass validation with fake pointers: run the body
    only in a process that sees no device, where such a call stops at the
    device check.  Without a visible device the body runs here; otherwise
    this test runs again in a child interpreter with every device hidden,
    and if the child still sees one the body is skipped there, never run."""
    @functools.wraps(fn)
    def wrapper(*args, **kw):
        if not _device_visible():
            return fn(*args, **kw)
        if os.environ.get(_CHILD_FLAG) == "1":
            pytest.skip("a device is still visible: fake-pointer calls are not made")
        env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
        env[_CHILD_FLAG] = "1"
        node = f"{os.path.abspath(__file__)}::{fn.__name__}"
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", node],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        if "1 passed" not in r.stdout:
            pytest.skip("no device-free child available: " + r.stdout.strip().splitlines()[-1])
    return wrapper


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lact_\w+)\s*\(", txt)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(lact.EXPORTS)
    L = lact.lib()
    for nm in names:
        assert hasattr(L, nm), nm


def test_header_is_c11(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "lact.h"\nint main(void){lact_problem p; (void)p; '
                   'return (int)LACT_OK + LACT_CHUNK_APPLY;}\n')
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    L = lact.lib()
    for s in [0, -1, -2, -3, -4, -5]:
        assert len(L.lact_status_str(s)) > 0
    assert L.lact_status_str(7) == b"unknown status"


def P(**kw):
    base = dict(n_inst=2, d=128, io_dtype=lact.DTYPE_BF16, opt=lact.OPT_GD)
    base.update(kw)
    return lact.problem(**base)


def fwd(p, L=512, chunk=128, order=0, bounds=None, flags=None, ws_bytes=None, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lr=FAKE, beta=FAKE, W1=FAKE, W2=FAKE, W3=FAKE,
             M1=FAKE, M2=FAKE, M3=FAKE, o=FAKE, ws=FAKE)
    a.update(ptrs)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lact.layer_forward_ptr(p, a["q"], a["k"], a["v"], a["lr"], a["beta"], L, chunk, order,
                                  bounds, flags, a["W1"], a["W2"], a["W3"], a["M1"], a["M2"], a["M3"],
                                  a["o"], a["ws"], ws_bytes, None)


def test_null_problem():
    st = lact.lib().lact_layer_forward(None, None, None, None, None, None, 0, 1, 0, None, None, 0,
                                       None, None, None, None, None, None, None, None, 0, None)
    assert st == lact.ERR_INVALID_ARG
    assert "problem" in lact.last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(d=128, dh=96), lact.ERR_UNSUPPORTED),
    (dict(d=128, dh=2048), lact.ERR_UNSUPPORTED),
    (dict(d=96), lact.ERR_UNSUPPORTED),
    (dict(d=32), lact.ERR_UNSUPPORTED),
    (dict(d=2048), lact.ERR_UNSUPPORTED),
    (dict(io_dtype=5), lact.ERR_INVALID_ARG),
    (dict(opt=9), lact.ERR_INVALID_ARG),
    (dict(opt=lact.OPT_MUON, ns_iters=0), lact.ERR_INVALID_ARG),
    (dict(opt=lact.OPT_MUON_MOMENTUM, ns_iters=17), lact.ERR_INVALID_ARG),
    (dict(opt=4), lact.ERR_INVALID_ARG),
    (dict(rec_planes=4), lact.ERR_INVALID_ARG),
    (dict(n_inst=-1), lact.ERR_INVALID_ARG),
])
def test_bad_problem(kw, code):
    assert fwd(P(**kw)) == code
    assert lact.last_error() != ""


def test_bad_flags_field():
    p = P()
    p.flags = 0x10
    assert fwd(p) == lact.ERR_INVALID_ARG


@pytest.mark.parametrize("args", [
    dict(order=2),
    dict(chunk=0),
    dict(L=-1),
    dict(bounds=[0, 100, 512], flags=None),
    dict(bounds=[1, 100, 512], flags=[3, 3]),
    dict(bounds=[0, 100, 100, 512], flags=[3, 3, 3]),
    dict(bounds=[0, 300, 200, 512], flags=[3, 3, 3]),
    dict(bounds=[0, 100, 500], flags=[3, 3]),
    dict(bounds=[0, 100, 512], flags=[3, 4]),
])
def test_bad_schedule(args):
    assert fwd(P(), **args) == lact.ERR_INVALID_ARG


@pytest.mark.parametrize("ptrs,opt", [
    (dict(q=None), lact.OPT_GD),
    (dict(o=None), lact.OPT_GD),
    (dict(k=None), lact.OPT_GD),
    (dict(v=None), lact.OPT_GD),
    (dict(lr=None), lact.OPT_GD),
    (dict(W2=None), lact.OPT_GD),
    (dict(beta=None), lact.OPT_MOMENTUM),
    (dict(M3=None), lact.OPT_MOMENTUM),
    (dict(beta=None), lact.OPT_MUON_MOMENTUM),
    (dict(M1=None), lact.OPT_MUON_MOMENTUM),
    (dict(k=FAKE + 2), lact.OPT_GD),
    (dict(W1=FAKE + 4), lact.OPT_GD),
    (dict(ws=FAKE + 16), lact.OPT_GD),
])
def test_bad_pointers(ptrs, opt):
    assert fwd(P(opt=opt), **ptrs) == lact.ERR_INVALID_ARG


@device_free
def test_pointers_not_needed_by_the_schedule_may_be_null():
    # update-only schedule: q and o are never touched; GD: beta and M unused
    p = P()
    st = fwd(p, L=256, bounds=[0, 256], flags=[lact.CHUNK_UPDATE], q=None, o=None, beta=None,
             M1=None, M2=None, M3=None)
    assert st == lact.ERR_NO_DEVICE, lact.last_error()


def test_workspace_too_small():
    p = P()
    need = lact.workspace_size(p, 512, 128)
    assert fwd(p, ws_bytes=need - 1) == lact.ERR_WORKSPACE_TOO_SMALL


def test_noop_calls_need_no_device():
    assert fwd(P(n_inst=0)) == lact.OK
    assert fwd(P(), L=0, chunk=16) == lact.OK
    assert lact.chunk_update_ptr(P(), FAKE, FAKE, FAKE, None, 0, 0, FAKE, FAKE, FAKE,
                                 None, None, None, FAKE, 1 << 30, None) == lact.OK
    assert lact.apply_ptr(P(), FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == lact.OK


def test_chunk_update_and_apply_validation():
    p = P()
    assert lact.chunk_update_ptr(p, FAKE, FAKE, FAKE, None, 64, 32, FAKE, FAKE, FAKE,
                                 None, None, None, FAKE, 1 << 30, None) == lact.ERR_INVALID_ARG
    assert lact.chunk_update_ptr(P(opt=lact.OPT_MOMENTUM), FAKE, FAKE, FAKE, None, 64, 64, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == lact.ERR_INVALID_ARG
    assert lact.apply_ptr(p, None, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == lact.ERR_INVALID_ARG
    assert lact.apply_ptr(p, FAKE, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == lact.ERR_WORKSPACE_TOO_SMALL


def test_workspace_size_properties():
    p = P()
    a = lact.workspace_size(p, 512, 128)
    b = lact.workspace_size(p, 4096, 1024)
    assert 0 < a < b
    m = lact.workspace_size(P(opt=lact.OPT_MUON), 512, 128)
    assert m > a
    with pytest.raises(lact.LactError):
        lact.workspace_size(P(d=96), 512, 128)
    # explicit schedule equal to the uniform one gives the same size
    assert lact.workspace_size(p, 512, 128, 0, [0, 128, 256, 384, 512], [3, 3, 3, 3]) == a
    # the view-set schedule: one long update chunk, then the targets; its
    # update is the fused kernel, whose update terms never leave the chip, so
    # no buffer for them is sized
    v = lact.workspace_size(P(n_inst=6, d=128), 200704, 0, 1, [0, 196608, 200704], [1, 2])
    assert 0 < v < 6 * 196608 * 3 * 128 * 2
    # 2,048-token chunks at d = 384 (separate update forward and contraction):
    # one chunk's update terms are sized
    u = lact.workspace_size(P(n_inst=4, d=384), 32768, 2048)
    assert u > 4 * 2048 * 3 * 384 * 2


@device_free
def test_valid_call_without_gpu_reports_no_device():
    assert fwd(P()) == lact.ERR_NO_DEVICE


def fwd_scaled(p, oz=FAKE, L=512, chunk=128, ws_bytes=1 << 40, bounds=None, flags=None, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lr=FAKE, beta=FAKE, W1=FAKE, W2=FAKE, W3=FAKE,
             M1=FAKE, M2=FAKE, M3=FAKE, o=FAKE, ws=FAKE)
    a.update(ptrs)
    return lact.layer_forward_scaled_ptr(p, a["q"], a["k"], a["v"], a["lr"], a["beta"], oz, L, chunk,
                                         0, bounds, flags, a["W1"], a["W2"], a["W3"], a["M1"], a["M2"],
                                         a["M3"], a["o"], a["ws"], ws_bytes, None)


def test_qk_prep_flag_accepted_and_sized():
    p = P(qk_prep=True)
    assert p.flags == lact.QK_PREP
    base = lact.workspace_size(P(), 512, 128)
    prep = lact.workspace_size(p, 512, 128)
    # one pre-processed copy of q and one of k: [n, L, D] bf16 each
    assert prep - base == 2 * 2 * 512 * 128 * 2
    # an update-only schedule keeps only the k copy
    b1 = lact.workspace_size(P(), 512, 0, 0, [0, 512], [1])
    p1 = lact.workspace_size(p, 512, 0, 0, [0, 512], [1])
    assert p1 - b1 == 2 * 512 * 128 * 2
    both = P(qk_prep=True, renorm=False)
    assert both.flags == lact.QK_PREP | lact.NO_RENORM
    assert fwd(both, ws_bytes=prep - 1) == lact.ERR_WORKSPACE_TOO_SMALL


@device_free
def test_scaled_entry_validation():
    assert fwd_scaled(P(), oz=None) == lact.ERR_INVALID_ARG
    assert "oz" in lact.last_error()
    assert fwd_scaled(P(), oz=FAKE + 2) == lact.ERR_INVALID_ARG
    # no APPLY chunk: the scale is never read, so NULL is allowed
    st = fwd_scaled(P(), oz=None, L=256, chunk=0, bounds=[0, 256], flags=[1], q=None, o=None)
    assert st == lact.ERR_NO_DEVICE, lact.last_error()
    assert fwd_scaled(P(n_inst=0), oz=None) == lact.OK
    assert fwd_scaled(P(), ws_bytes=10) == lact.ERR_WORKSPACE_TOO_SMALL
    assert fwd_scaled(P()) == lact.ERR_NO_DEVICE


@device_free
def test_rectangular_fast_weights_accepted_and_sized():
    """d != dh (multiples of 64) is accepted for every optimiser; the
    workspace grows with dh where the hidden width is stored."""
    for dh in (64, 256):
        p = P(d=128, dh=dh)
        assert p.dh == dh
        assert fwd(p) == lact.ERR_NO_DEVICE, lact.last_error()
        for opt in (lact.OPT_MOMENTUM, lact.OPT_MUON, lact.OPT_MUON_MOMENTUM):
            assert fwd(P(d=128, dh=dh, opt=opt)) == lact.ERR_NO_DEVICE, lact.last_error()
    a = lact.workspace_size(P(d=128, dh=128), 512, 128)
    b = lact.workspace_size(P(d=128, dh=256), 512, 128)
    assert b > a


def test_single_hip_runtime_in_process():
    """Importing the binding before torch must not pull in a second HIP
    runtime: torch's bundled one has to be the only one mapped, or the
    library's calls see no device."""
    code = ("import test_layers_amd.lact, torch\n"
            "m = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in m if 'libamdhip64' in l}))\n")
    r = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs


# ----------------------------------------------------------------- backward entry point
def bwd(p, L=512, chunk=128, order=0, bounds=None, flags=None, ws_bytes=None, **ptrs):
    names = ["q", "k", "v", "lr", "beta", "oz", "W1", "W2", "W3", "M1", "M2", "M3", "dO", "gW1", "gW2", "gW3",
             "gM1", "gM2", "gM3", "dq", "dk", "dv", "dlr", "dbeta", "doz", "dW1", "dW2", "dW3", "dM1", "dM2", "dM3",
             "ws"]
    a = {n: FAKE for n in names}
    a.update(ptrs)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lact.layer_backward_ptr(p, a["q"], a["k"], a["v"], a["lr"], a["beta"], a["oz"], L, chunk, order, bounds,
                                   flags, a["W1"], a["W2"], a["W3"], a["M1"], a["M2"], a["M3"], a["dO"], a["gW1"],
                                   a["gW2"], a["gW3"], a["gM1"], a["gM2"], a["gM3"], a["dq"], a["dk"], a["dv"],
                                   a["dlr"], a["dbeta"], a["doz"], a["dW1"], a["dW2"], a["dW3"], a["dM1"], a["dM2"],
                                   a["dM3"], a["ws"], ws_bytes, None)


@device_free
def test_backward_takes_raw_qk_and_output_scale():
    # raw q / k and an output scale pass validation (the workspace grows by the fp32 copies)
    p = P(qk_prep=True)
    assert bwd(p) == lact.ERR_NO_DEVICE, lact.last_error()
    assert lact.backward_workspace_size(p, 512, 128) > lact.backward_workspace_size(P(), 512, 128)
    assert bwd(P(), doz=None) == lact.ERR_INVALID_ARG          # oz given, doz missing
    assert bwd(P(), oz=None, doz=None) == lact.ERR_NO_DEVICE, lact.last_error()
    assert bwd(P(), oz=FAKE + 2) == lact.ERR_INVALID_ARG


@pytest.mark.parametrize("ptrs,opt", [
    (dict(dW1=None), lact.OPT_GD),
    (dict(dq=None), lact.OPT_GD),
    (dict(dO=None), lact.OPT_GD),
    (dict(dlr=None), lact.OPT_GD),
    (dict(dbeta=None), lact.OPT_MOMENTUM),
    (dict(M2=None), lact.OPT_MOMENTUM),
    (dict(gW1=FAKE + 4), lact.OPT_GD),
    (dict(dk=FAKE + 2), lact.OPT_GD),
    (dict(ws=FAKE + 16), lact.OPT_GD),
])
def test_backward_bad_pointers(ptrs, opt):
    assert bwd(P(opt=opt), **ptrs) == lact.ERR_INVALID_ARG, lact.last_error()


@device_free
def test_backward_optional_pointers_may_be_null():
    # GD: beta, M, dbeta and dM unused; state cotangents optional
    st = bwd(P(), beta=None, M1=None, M2=None, M3=None, dbeta=None, dM1=None, dM2=None, dM3=None, gW1=None,
             gW2=None, gW3=None, gM1=None, gM2=None, gM3=None)
    assert st == lact.ERR_NO_DEVICE, lact.last_error()


def test_backward_workspace():
    for opt in (lact.OPT_GD, lact.OPT_MOMENTUM, lact.OPT_MUON, lact.OPT_MUON_MOMENTUM):
        p = P(opt=opt)
        need = lact.backward_workspace_size(p, 512, 128)
        assert need >= lact.workspace_size(p, 512, 128)
        assert bwd(p, ws_bytes=need - 1) == lact.ERR_WORKSPACE_TOO_SMALL
    # more chunks keep more states
    p = P(opt=lact.OPT_MOMENTUM)
    assert lact.backward_workspace_size(p, 1024, 128) > lact.backward_workspace_size(p, 512, 128)
    with pytest.raises(lact.LactError):
        lact.backward_workspace_size(P(d=96), 512, 128)


def test_binding_rejects_mis_shaped_tensors():
    """The binding checks every tensor's shape before any library call (the
    library sees raw pointers only)."""
    torch = pytest.importorskip("torch")
    n, L, D = 2, 64, 128
    q = torch.zeros(n, L, D)
    W = [torch.zeros(n, D, D) for _ in range(3)]
    with pytest.raises(ValueError, match="lr has shape"):
        lact.layer_forward(q, q, q, torch.zeros(n, L, 2), None, *W)
    with pytest.raises(ValueError, match="W2 has shape"):
        lact.layer_forward(q, q, q, torch.zeros(n, L, 3), None, W[0], torch.zeros(n, D, 64), W[2])
    with pytest.raises(ValueError, match="dO has shape"):
        lact.layer_backward(q, q, q, torch.zeros(n, L, 3), None, *W, dO=torch.zeros(n, L - 1, D))
    with pytest.raises(ValueError, match=r"out\[dq\] has shape"):
        lact.layer_backward(q, q, q, torch.zeros(n, L, 3), None, *W, dO=q, out={"dq": torch.zeros(1)})
    with pytest.raises(ValueError, match="v has shape"):
        lact.chunk_update(q, torch.zeros(n, L + 1, D), torch.zeros(n, L, 3), None, *W)
    with pytest.raises(ValueError, match="o has shape"):
        lact.apply(q, *W, o=torch.zeros(n, L, 64))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without liblact.so the binding raises; there is no other implementation
    to fall back to."""
    monkeypatch.setattr(lact, "_lib", None)
    monkeypatch.setattr(lact, "LIB_PATH", str(tmp_path / "liblact.so"))
    with pytest.raises(ImportError, match="not built"):
        lact.lib()
    with pytest.raises(ImportError):
        lact.workspace_size(lact.problem(1, 64, 0, 0, 1), 128, 0, 0, None, None)


def test_newton_schulz_default_precision_is_fp32_grade():
    """rec_planes = 0 with a Newton-Schulz optimiser selects the fp32-grade
    recurrence (three planes; one plane lets the rounding grow about x2 per
    chunk), visible in the workspace: its update terms are stored in fp32, not
    bf16.  GD and momentum keep plain bf16 by default."""
    for opt in (lact.OPT_MUON, lact.OPT_MUON_MOMENTUM):
        d0 = lact.workspace_size(P(opt=opt, rec_planes=0), 4096, 1024)
        assert d0 == lact.workspace_size(P(opt=opt, rec_planes=3), 4096, 1024)
        assert d0 > lact.workspace_size(P(opt=opt, rec_planes=1), 4096, 1024)
    for opt in (lact.OPT_GD, lact.OPT_MOMENTUM):
        assert (lact.workspace_size(P(opt=opt, rec_planes=0), 4096, 1024)
                == lact.workspace_size(P(opt=opt, rec_planes=1), 4096, 1024))


@pytest.mark.parametrize("bounds,flags", [
    ([0, 256], [3, 3]),            # one bound short: the library would read past the array
    ([0, 128, 256, 384], [3, 3]),  # one bound too many
    ([0, 256], [259]),             # does not fit a uint8 (would wrap to 3)
    ([0, 256], [-1]),
])
def test_binding_rejects_inconsistent_schedule_arrays(bounds, flags):
    with pytest.raises(ValueError):
        lact.workspace_size(P(), 256, 0, 0, bounds, flags)
    with pytest.raises(ValueError):
        fwd(P(), L=256, bounds=bounds, flags=flags)


def test_binding_schedule_cache_keys_on_values():
    """The binding keeps converted schedules keyed by their values: a
    repeated schedule gives the same answer, a changed one (even with the
    same length) is converted afresh, and a bad one is still rejected after a
    good one of the same length was cached."""
    b, f = [0, 256, 640, 1000], [3, 3, 3]
    a1 = lact.workspace_size(P(), 1000, 0, 0, b, f)
    assert lact.workspace_size(P(), 1000, 0, 0, list(b), list(f)) == a1
    assert lact.workspace_size(P(), 1000, 0, 0, tuple(b), tuple(f)) == a1
    # a longer first chunk needs more workspace (the update terms scale with it)
    b2 = [0, 900, 950, 1000]
    assert lact.workspace_size(P(), 1000, 0, 0, b2, f) > a1
    with pytest.raises(ValueError):
        lact.workspace_size(P(), 1000, 0, 0, b, [3, 3, 300])
    for i in range(200):   # more schedules than the cache keeps
        assert lact.workspace_size(P(), 1000, 0, 0, [0, 256 + i, 640 + i, 1000], f) > 0
    assert lact.workspace_size(P(), 1000, 0, 0, b, f) == a1


def test_binding_workspace_must_be_bytes():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="uint8"):
        lact._workspace(1024, torch.zeros(1024, dtype=torch.float32), "cpu")


def noalloc(p, L=512, chunk=128, order=0, bounds=None, flags=None, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lr=FAKE, beta=FAKE, W1=FAKE, W2=FAKE, W3=FAKE,
             M1=FAKE, M2=FAKE, M3=FAKE, o=FAKE)
    a.update(ptrs)
    return lact.layer_forward_noalloc_ptr(p, a["q"], a["k"], a["v"], a["lr"], a["beta"], L, chunk, order,
                                          bounds, flags, a["W1"], a["W2"], a["W3"], a["M1"], a["M2"], a["M3"],
                                          a["o"], None)


def test_noalloc_validation():
    """The allocation-free entry point validates like lact_layer_forward and
    rejects, before any device work, a problem whose workspace exceeds its
    scratch array."""
    assert noalloc(P(n_inst=0)) == lact.OK
    assert noalloc(P(d=96)) == lact.ERR_UNSUPPORTED
    assert noalloc(P(), k=FAKE + 2) == lact.ERR_INVALID_ARG
    big = P(n_inst=6, d=512, opt=lact.OPT_MUON, rec_planes=2)
    assert lact.workspace_size(big, 32768, 4096) > lact.NOALLOC_SCRATCH_BYTES
    assert noalloc(big, L=32768, chunk=4096) == lact.ERR_WORKSPACE_TOO_SMALL
    assert "LACT_NOALLOC_SCRATCH_BYTES" in lact.last_error()


@device_free
def test_noalloc_valid_call_reports_no_device():
    assert lact.workspace_size(P(), 512, 128) <= lact.NOALLOC_SCRATCH_BYTES
    assert noalloc(P()) == lact.ERR_NO_DEVICE


def test_noalloc_scratch_size_matches_the_header():
    txt = open(HEADER).read()
    m = re.search(r"#define LACT_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == lact.NOALLOC_SCRATCH_BYTES
