"""Thin ctypes binding of liblact (include/lact.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Torch tensors supply device memory (data_ptr) and the current HIP
stream; nothing here computes any part of the layer.  If liblact.so is
missing the import fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblact.so")

# values mirror include/lact.h
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE_TOO_SMALL = -3
ERR_NO_DEVICE = -4
ERR_HIP = -5

DTYPE_F32 = 0
DTYPE_BF16 = 1
OPT_GD = 0
OPT_MOMENTUM = 1
OPT_MUON = 2
OPT_MUON_MOMENTUM = 3
APPLY_THEN_UPDATE = 0
UPDATE_THEN_APPLY = 1
CHUNK_UPDATE = 1
CHUNK_APPLY = 2
NO_RENORM = 1
QK_PREP = 2

K_UPD, K_APP, K_OUT, K_DW, K_OPT, K_NS, K_SNAP, K_PREP, K_BWD_GEMM, K_BWD_ELEM, K_NSRED = range(11)
K_NAMES = {K_UPD: "update_fwd", K_APP: "apply_fwd", K_OUT: "apply_out", K_DW: "dw", K_OPT: "opt",
           K_NS: "newton_schulz", K_SNAP: "snapshot", K_PREP: "qk_prep", K_BWD_GEMM: "bwd_gemm",
           K_BWD_ELEM: "bwd_elem", K_NSRED: "ns_reduce"}

EXPORTS = ["lact_workspace_size", "lact_chunk_update", "lact_apply", "lact_layer_forward",
           "lact_layer_forward_scaled", "lact_layer_forward_noalloc", "lact_backward_workspace_size",
           "lact_layer_backward", "lact_status_str", "lact_last_error", "lact_timing_enable", "lact_timing_read"]

NOALLOC_SCRATCH_BYTES = 128 << 20   # LACT_NOALLOC_SCRATCH_BYTES


class LactError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"liblact status {status}: {detail}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("n_inst", ctypes.c_int32), ("d", ctypes.c_int32), ("dh", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("opt", ctypes.c_int32), ("ns_iters", ctypes.c_int32),
                ("rec_planes", ctypes.c_int32), ("flags", ctypes.c_uint32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m test_layers_amd.build` "
                          "(the LaCT layer has no non-HIP implementation)")
    # torch ships its own HIP runtime, reached through the unversioned name
    # libamdhip64.so.  If liblact were loaded first, its dependency
    # libamdhip64.so.7 would resolve to the system runtime and the process
    # would hold two HIP (and HSA) runtimes; the second one to open the GPU
    # sees no device.  Loading torch first makes liblact bind to the runtime
    # that owns the tensors it is given.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(Problem)
    L.lact_workspace_size.restype = sz
    L.lact_workspace_size.argtypes = [P, i64, i64, i32, vp, vp, i32]
    L.lact_chunk_update.restype = i32
    L.lact_chunk_update.argtypes = [P, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lact_apply.restype = i32
    L.lact_apply.argtypes = [P, vp, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    L.lact_layer_forward.restype = i32
    L.lact_layer_forward.argtypes = [P, vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, i32,
                                     vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lact_layer_forward_scaled.restype = i32
    L.lact_layer_forward_scaled.argtypes = [P, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, i32,
                                            vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lact_layer_forward_noalloc.restype = i32
    L.lact_layer_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, i32,
                                             vp, vp, vp, vp, vp, vp, vp, vp]
    L.lact_backward_workspace_size.restype = sz
    L.lact_backward_workspace_size.argtypes = [P, i64, i64, i32, vp, vp, i32]
    L.lact_layer_backward.restype = i32
    L.lact_layer_backward.argtypes = ([P, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, i32]
                                      + [vp] * 6 + [vp] + [vp] * 6 + [vp] * 6 + [vp] * 6 + [vp, sz, vp])
    L.lact_status_str.restype = ctypes.c_char_p
    L.lact_status_str.argtypes = [i32]
    L.lact_last_error.restype = ctypes.c_char_p
    L.lact_last_error.argtypes = []
    L.lact_timing_enable.restype = i32
    L.lact_timing_enable.argtypes = [i32, i32]
    L.lact_timing_read.restype = i32
    L.lact_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    _lib = L
    return L


def last_error() -> str:
    return lib().lact_last_error().decode()


def check(status: int) -> None:
    if status != OK:
        raise LactError(status, f"{lib().lact_status_str(status).decode()}: {last_error()}")


def problem(n_inst: int, d: int, io_dtype: int, opt: int, rec_planes: int = 0, ns_iters: int = 5,
            renorm: bool = True, dh: Optional[int] = None, qk_prep: bool = False) -> Problem:
    return Problem(n_inst, d, d if dh is None else dh, io_dtype, opt, ns_iters, rec_planes,
                   (0 if renorm else NO_RENORM) | (QK_PREP if qk_prep else 0))


# ----------------------------------------------------------------- raw-pointer calls
_SCHED_CACHE = {}


def _sched(bounds, flags):
    # either may be None: the library reports a half-given schedule itself.
    # Both given: the library reads n_chunks + 1 bounds and n_chunks flags,
    # so their lengths must agree, and flags must fit the uint8 they become.
    # A layer call marshals its schedule twice (workspace size, then the
    # call), and callers repeat schedules: the converted arrays of recent
    # schedules are kept (they are read by the library only during a call).
    if bounds is None and flags is None:
        return None, None, 0, None
    key = (None if bounds is None else tuple(bounds), None if flags is None else tuple(flags))
    hit = _SCHED_CACHE.get(key)
    if hit is not None:
        return hit
    res = _sched_convert(bounds, flags)
    if len(_SCHED_CACHE) >= 64:
        _SCHED_CACHE.clear()
    _SCHED_CACHE[key] = res
    return res


def _sched_convert(bounds, flags):
    if bounds is not None and flags is not None and len(bounds) != len(flags) + 1:
        raise ValueError(f"schedule has {len(bounds)} bounds for {len(flags)} chunks (need chunks + 1)")
    if flags is not None and any(not 0 <= int(x) <= 255 for x in flags):
        raise ValueError("schedule flags must lie in 0..255")
    b = None if bounds is None else (ctypes.c_int64 * len(bounds))(*[int(x) for x in bounds])
    f = None if flags is None else (ctypes.c_uint8 * len(flags))(*[int(x) for x in flags])
    nc = len(flags) if flags is not None else len(bounds) - 1
    cast = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
    return cast(b), cast(f), nc, (b, f)


def workspace_size(p: Problem, L: int, chunk: int = 0, order: int = 0,
                   bounds: Optional[Sequence[int]] = None, flags: Optional[Sequence[int]] = None) -> int:
    bp, fp, nc, _keep = _sched(bounds, flags)
    n = lib().lact_workspace_size(ctypes.byref(p), L, chunk, order, bp, fp, nc)
    if n == 0:
        raise LactError(ERR_INVALID_ARG, last_error())
    return n


def layer_forward_ptr(p: Problem, q, k, v, lr, beta, L, chunk, order, bounds, flags,
                      W1, W2, W3, M1, M2, M3, o, ws, ws_bytes, stream) -> int:
    bp, fp, nc, _keep = _sched(bounds, flags)
    return lib().lact_layer_forward(ctypes.byref(p), q, k, v, lr, beta, L, chunk, order, bp, fp, nc,
                                    W1, W2, W3, M1, M2, M3, o, ws, ws_bytes, stream)


def layer_forward_scaled_ptr(p: Problem, q, k, v, lr, beta, oz, L, chunk, order, bounds, flags,
                             W1, W2, W3, M1, M2, M3, o, ws, ws_bytes, stream) -> int:
    bp, fp, nc, _keep = _sched(bounds, flags)
    return lib().lact_layer_forward_scaled(ctypes.byref(p), q, k, v, lr, beta, oz, L, chunk, order,
                                           bp, fp, nc, W1, W2, W3, M1, M2, M3, o, ws, ws_bytes, stream)


def layer_forward_noalloc_ptr(p: Problem, q, k, v, lr, beta, L, chunk, order, bounds, flags,
                              W1, W2, W3, M1, M2, M3, o, stream) -> int:
    bp, fp, nc, _keep = _sched(bounds, flags)
    return lib().lact_layer_forward_noalloc(ctypes.byref(p), q, k, v, lr, beta, L, chunk, order, bp, fp, nc,
                                            W1, W2, W3, M1, M2, M3, o, stream)


def backward_workspace_size(p: Problem, L: int, chunk: int = 0, order: int = 0,
                            bounds: Optional[Sequence[int]] = None, flags: Optional[Sequence[int]] = None) -> int:
    bp, fp, nc, _keep = _sched(bounds, flags)
    n = lib().lact_backward_workspace_size(ctypes.byref(p), L, chunk, order, bp, fp, nc)
    if n == 0:
        raise LactError(ERR_INVALID_ARG, last_error())
    return n


def layer_backward_ptr(p: Problem, q, k, v, lr, beta, oz, L, chunk, order, bounds, flags, W1, W2, W3, M1, M2, M3,
                       dO, gW1, gW2, gW3, gM1, gM2, gM3, dq, dk, dv, dlr, dbeta, doz, dW1, dW2, dW3, dM1, dM2, dM3,
                       ws, ws_bytes, stream) -> int:
    bp, fp, nc, _keep = _sched(bounds, flags)
    return lib().lact_layer_backward(ctypes.byref(p), q, k, v, lr, beta, oz, L, chunk, order, bp, fp, nc,
                                     W1, W2, W3, M1, M2, M3, dO, gW1, gW2, gW3, gM1, gM2, gM3,
                                     dq, dk, dv, dlr, dbeta, doz, dW1, dW2, dW3, dM1, dM2, dM3, ws, ws_bytes,
                                     stream)


def chunk_update_ptr(p: Problem, k, v, lr, beta, Lc, seq_stride, W1, W2, W3, M1, M2, M3,
                     ws, ws_bytes, stream) -> int:
    return lib().lact_chunk_update(ctypes.byref(p), k, v, lr, beta, Lc, seq_stride, W1, W2, W3,
                                   M1, M2, M3, ws, ws_bytes, stream)


def apply_ptr(p: Problem, q, Lq, seq_stride, W1, W2, W3, o, ws, ws_bytes, stream) -> int:
    return lib().lact_apply(ctypes.byref(p), q, Lq, seq_stride, W1, W2, W3, o, ws, ws_bytes, stream)


def timing_enable(kclass: int, on: bool = True) -> None:
    check(lib().lact_timing_enable(kclass, 1 if on else 0))


def timing_read(kclass: int):
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    check(lib().lact_timing_read(kclass, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ----------------------------------------------------------------- torch-tensor calls
def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _check_shapes(**named):
    """Every given tensor must have exactly the expected shape: the library
    receives raw pointers and cannot detect a mis-sized buffer itself."""
    for name, (t, shape) in named.items():
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _w_shapes(n, D, Dh):
    return (n, Dh, D), (n, D, Dh), (n, Dh, D)


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise ValueError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes, workspace, device):
    torch = _torch()
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not workspace.is_cuda:
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace smaller than the {nbytes} bytes needed")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def layer_forward(q, k, v, lr, beta, W1, W2, W3, M1=None, M2=None, M3=None, o=None, *,
                  chunk: int = 0, order: int = APPLY_THEN_UPDATE, opt: int = OPT_GD,
                  bounds=None, flags=None, rec_planes: int = 0, ns_iters: int = 5,
                  renorm: bool = True, qk_prep: bool = False, oz=None, workspace=None,
                  stream=None):
    """q, k, v [n, L, d] (fp32 or bf16), lr [n, L, 3] fp32, beta [n, L] fp32
    (momentum) or None, W1, W3 [n, dh, d] and W2 [n, d, dh] fp32 (updated in
    place; dh is read from W1's shape), M1..M3
    (momentum state, updated in place).  qk_prep: q and k are raw (the library
    applies silu and the per-token L2 normalisation).  oz [n, L] fp32: the
    output rows are scaled by silu(oz) (lact_layer_forward_scaled).  Returns o
    [n, L, D] (allocated with torch.zeros if not given; rows of non-APPLY
    chunks keep their values)."""
    torch = _torch()
    if q.dim() != 3 or W1.dim() != 3:
        raise ValueError("q must be [n, L, d] and W1 [n, dh, d]")
    n, L, D = q.shape
    Dh = W1.shape[1]
    s1, s2, s3 = _w_shapes(n, D, Dh)
    _check_shapes(k=(k, (n, L, D)), v=(v, (n, L, D)), lr=(lr, (n, L, 3)), beta=(beta, (n, L)), W1=(W1, s1),
                  W2=(W2, s2), W3=(W3, s3), M1=(M1, s1), M2=(M2, s2), M3=(M3, s3), o=(o, (n, L, D)),
                  oz=(oz, (n, L)))
    io = _io_dtype(q)
    p = problem(n, D, io, opt, rec_planes, ns_iters, renorm, dh=Dh, qk_prep=qk_prep)
    if o is None:
        o = torch.zeros_like(q)
    need = workspace_size(p, L, chunk, order, bounds, flags)
    ws = _workspace(need, workspace, q.device)
    f32 = torch.float32
    head = (p, _ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"),
            _ptr(lr, f32, "lr"), _ptr(beta, f32, "beta"))
    tail = (L, chunk, order, bounds, flags,
            _ptr(W1, f32, "W1"), _ptr(W2, f32, "W2"), _ptr(W3, f32, "W3"),
            _ptr(M1, f32, "M1"), _ptr(M2, f32, "M2"), _ptr(M3, f32, "M3"),
            _ptr(o, q.dtype, "o"), ws.data_ptr(), ws.numel(), _stream(stream))
    if oz is None:
        st = layer_forward_ptr(*head, *tail)
    else:
        st = layer_forward_scaled_ptr(*head, _ptr(oz, f32, "oz"), *tail)
    check(st)
    return o


def chunk_update(k, v, lr, beta, W1, W2, W3, M1=None, M2=None, M3=None, *, Lc: Optional[int] = None,
                 opt: int = OPT_GD, rec_planes: int = 0, ns_iters: int = 5, renorm: bool = True,
                 qk_prep: bool = False, workspace=None, stream=None):
    torch = _torch()
    if k.dim() != 3 or W1.dim() != 3:
        raise ValueError("k must be [n, S, d] and W1 [n, dh, d]")
    n, S, D = k.shape
    s1, s2, s3 = _w_shapes(n, D, W1.shape[1])
    _check_shapes(v=(v, (n, S, D)), lr=(lr, (n, S, 3)), beta=(beta, (n, S)), W2=(W2, s2), W3=(W3, s3),
                  M1=(M1, s1), M2=(M2, s2), M3=(M3, s3))
    Lc = S if Lc is None else Lc
    p = problem(n, D, _io_dtype(k), opt, rec_planes, ns_iters, renorm, dh=W1.shape[1], qk_prep=qk_prep)
    ws = _workspace(workspace_size(p, Lc, max(Lc, 1)), workspace, k.device)
    f32 = torch.float32
    check(chunk_update_ptr(p, _ptr(k, k.dtype, "k"), _ptr(v, k.dtype, "v"), _ptr(lr, f32, "lr"),
                           _ptr(beta, f32, "beta"), Lc, S, _ptr(W1, f32, "W1"), _ptr(W2, f32, "W2"),
                           _ptr(W3, f32, "W3"), _ptr(M1, f32, "M1"), _ptr(M2, f32, "M2"),
                           _ptr(M3, f32, "M3"), ws.data_ptr(), ws.numel(), _stream(stream)))


def apply(q, W1, W2, W3, o=None, *, Lq: Optional[int] = None, qk_prep: bool = False,
          workspace=None, stream=None):
    torch = _torch()
    if q.dim() != 3 or W1.dim() != 3:
        raise ValueError("q must be [n, S, d] and W1 [n, dh, d]")
    n, S, D = q.shape
    s1, s2, s3 = _w_shapes(n, D, W1.shape[1])
    _check_shapes(W2=(W2, s2), W3=(W3, s3), o=(o, (n, S, D)))
    Lq = S if Lq is None else Lq
    p = problem(n, D, _io_dtype(q), OPT_GD, dh=W1.shape[1], qk_prep=qk_prep)
    if o is None:
        o = torch.zeros_like(q)
    ws = _workspace(workspace_size(p, Lq, max(Lq, 1)), workspace, q.device)
    f32 = torch.float32
    check(apply_ptr(p, _ptr(q, q.dtype, "q"), Lq, S, _ptr(W1, f32, "W1"), _ptr(W2, f32, "W2"),
                    _ptr(W3, f32, "W3"), _ptr(o, q.dtype, "o"), ws.data_ptr(), ws.numel(),
                    _stream(stream)))
    return o


def layer_backward(q, k, v, lr, beta, W1, W2, W3, M1=None, M2=None, M3=None, *, dO, gW=None, gM=None,
                   chunk: int = 0, order: int = APPLY_THEN_UPDATE, opt: int = OPT_GD, bounds=None, flags=None,
                   ns_iters: int = 5, renorm: bool = True, qk_prep: bool = False, oz=None, out=None,
                   workspace=None, stream=None):
    """Backward of layer_forward (lact_layer_backward).  Inputs as for
    layer_forward with W1..W3, M1..M3 the INITIAL state (read only); dO
    [n, L, d] in q's dtype (the cotangent of the scaled output when oz is
    given); gW, gM: None or 3-tuples of cotangents of the final state.
    Returns a dict of fp32 gradients dq, dk, dv (of the raw q, k with
    qk_prep), dlr, dbeta (momentum optimisers, else None), doz (with oz, else
    None), dW1..dW3, dM1..dM3 (momentum optimisers, else None); `out` (such a
    dict from an earlier call with the same shapes) is filled instead of
    allocating."""
    torch = _torch()
    if q.dim() != 3 or W1.dim() != 3:
        raise ValueError("q must be [n, L, d] and W1 [n, dh, d]")
    n, L, D = q.shape
    Dh = W1.shape[1]
    ws_ = _w_shapes(n, D, Dh)
    _check_shapes(k=(k, (n, L, D)), v=(v, (n, L, D)), lr=(lr, (n, L, 3)), beta=(beta, (n, L)), W2=(W2, ws_[1]),
                  W3=(W3, ws_[2]), M1=(M1, ws_[0]), M2=(M2, ws_[1]), M3=(M3, ws_[2]), dO=(dO, (n, L, D)),
                  oz=(oz, (n, L)))
    for name, gs in (("gW", gW), ("gM", gM)):
        for j, g in enumerate(gs or ()):
            _check_shapes(**{f"{name}{j + 1}": (g, ws_[j])})
    if out is not None:
        expect = {"dq": (n, L, D), "dk": (n, L, D), "dv": (n, L, D), "dlr": (n, L, 3), "dbeta": (n, L),
                  "doz": (n, L), "dW1": ws_[0], "dW2": ws_[1], "dW3": ws_[2], "dM1": ws_[0], "dM2": ws_[1],
                  "dM3": ws_[2]}
        _check_shapes(**{f"out[{key}]": (out.get(key), shape) for key, shape in expect.items()})
    io = _io_dtype(q)
    p = problem(n, D, io, opt, 3, ns_iters, renorm, dh=Dh, qk_prep=qk_prep)
    mom = opt in (OPT_MOMENTUM, OPT_MUON_MOMENTUM)
    f32 = torch.float32
    if out is None:
        e = lambda *shape: torch.empty(*shape, dtype=f32, device=q.device)
        out = {"dq": e(n, L, D), "dk": e(n, L, D), "dv": e(n, L, D), "dlr": e(n, L, 3),
               "dbeta": e(n, L) if mom else None, "doz": e(n, L) if oz is not None else None}
        for j, w in enumerate((W1, W2, W3)):
            out[f"dW{j + 1}"] = torch.empty_like(w)
            out[f"dM{j + 1}"] = torch.empty_like(w) if mom else None
    gW = (None, None, None) if gW is None else gW
    gM = (None, None, None) if gM is None else gM
    need = backward_workspace_size(p, L, chunk, order, bounds, flags)
    ws = _workspace(need, workspace, q.device)
    check(layer_backward_ptr(
        p, _ptr(q, q.dtype, "q"), _ptr(k, q.dtype, "k"), _ptr(v, q.dtype, "v"), _ptr(lr, f32, "lr"),
        _ptr(beta, f32, "beta"), _ptr(oz, f32, "oz"), L, chunk, order, bounds, flags,
        _ptr(W1, f32, "W1"), _ptr(W2, f32, "W2"), _ptr(W3, f32, "W3"),
        _ptr(M1, f32, "M1"), _ptr(M2, f32, "M2"), _ptr(M3, f32, "M3"), _ptr(dO, q.dtype, "dO"),
        *[_ptr(g, f32, "gW") for g in gW], *[_ptr(g, f32, "gM") for g in gM],
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlr"]), _ptr(out["dbeta"]),
        _ptr(out.get("doz")),
        _ptr(out["dW1"]), _ptr(out["dW2"]), _ptr(out["dW3"]), _ptr(out["dM1"]), _ptr(out["dM2"]), _ptr(out["dM3"]),
        ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


lib()  # fail at import time if the library is missing
