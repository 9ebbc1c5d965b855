"""Seeded synthetic workloads for the LaCT fast-weight layer.

This module only describes and draws inputs: shapes, chunk schedules and
value distributions.  It holds none of the layer's update/apply arithmetic.
Both the HIP path and the CPU oracle consume the arrays it returns; neither
imports the other.

Workload shapes follow the pages' experiments:
  * language models at 32K tokens, 2K/4K chunks, shifted block-causal order
    ("LaCT：以大分块更新人工智能的临时记忆", section on LM quality and
    throughput; "大块测试时训练（LaCT）技术解析" §3.2 and §4.1);
  * a 48-view set of 512x512 images as one update chunk plus 4K target
    tokens (same LaCT page, view-synthesis measurement conditions, Table 2);
  * an autoregressive video sequence of clean 3-frame chunks interleaved with
    noisy chunks ("大块测试时训练（LaCT）技术解析" §3.3; LaCT page, video and
    distributed section).

Input recipe (fp64 draws, then rounded):
  * q, k ~ N(0, 1), then silu and division by the per-token L2 norm over d
    (the q/k pre-processing of "LaCT架构核心思想解析" §1.2), for the LM and
    video workloads; raw N(0, 1) for the view-set workload;
  * v ~ N(0, 1);
  * lr = softplus(N(0, 1) - 5) per token and per fast-weight matrix;
  * beta = sigmoid(N(0, 1) + 2.2) per token (momentum only);
  * W1, W2, W3 ~ N(0, 1/D).
Rounding: fp64 -> fp32 (round to nearest even), then for bf16 inputs
fp32 -> bf16 (round to nearest even).  bf16 arrays are returned as uint16
bit patterns.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

# chunk flags (same values as the C header)
UPDATE = 1
APPLY = 2

APPLY_THEN_UPDATE = 0
UPDATE_THEN_APPLY = 1

OPT_GD = 0
OPT_MOMENTUM = 1
OPT_MUON = 2
OPT_MUON_MOMENTUM = 3   # Newton-Schulz of the momentum buffer

DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    n_inst: int           # B * nh
    D: int                # d: width of q, k, v, o
    L: int                # tokens per instance
    bounds: Tuple[int, ...]   # chunk boundaries, len n_chunks + 1
    flags: Tuple[int, ...]    # per chunk: UPDATE | APPLY
    order: int
    opt: int
    io_dtype: int
    qk_prep: bool         # silu + L2 normalisation of q, k (in the generator)
    rec_planes: int       # bf16 planes used for the state recurrence on the GPU
    tol: float            # parity gate, max-abs error relative to max |ref|
    layer_qk_prep: bool = False   # q, k handed over raw; the layer pre-processes them
    out_scale: bool = False       # per-token output-scale pre-activation oz [n, L]
    Dh: Optional[int] = None      # fast-weight hidden width dh (None: dh = d)

    @property
    def dh(self) -> int:
        return self.D if self.Dh is None else self.Dh

    @property
    def n_chunks(self) -> int:
        return len(self.flags)

    @property
    def tokens(self) -> int:
        """Sequence positions the layer consumes (the throughput unit)."""
        return self.L

    @property
    def max_chunk(self) -> int:
        return max(b - a for a, b in zip(self.bounds[:-1], self.bounds[1:]))

    def scaled(self, n_inst: Optional[int] = None, L: Optional[int] = None,
               chunk: Optional[int] = None) -> "Workload":
        """Same recipe at a smaller size (uniform chunks, all U+A unless the
        schedule is the view-set one)."""
        n = self.n_inst if n_inst is None else n_inst
        if L is None and chunk is None:
            return dataclasses.replace(self, n_inst=n)
        L = self.L if L is None else L
        chunk = self.max_chunk if chunk is None else chunk
        bounds, flags = uniform_schedule(L, chunk)
        return dataclasses.replace(self, n_inst=n, L=L, bounds=bounds, flags=flags)


def uniform_schedule(L: int, chunk: int) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """Uniform chunks of `chunk` tokens, the last one taking the remainder."""
    b = list(range(0, L, chunk)) + [L]
    return tuple(b), tuple([UPDATE | APPLY] * (len(b) - 1))


def video_schedule(n_clean: int, chunk: int) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """[C1, N2, C2, N3, C3, ..., N_n, C_n]: clean chunks update and apply,
    noisy chunks only apply (they read the weights that the following clean
    chunk also reads)."""
    flags = [UPDATE | APPLY]
    for _ in range(n_clean - 1):
        flags += [APPLY, UPDATE | APPLY]
    b = [i * chunk for i in range(len(flags) + 1)]
    return tuple(b), tuple(flags)


def video_schedule_noisy_first(n_clean: int, chunk: int) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """[N1, C1, N2, C2, ..., N_n, C_n]: every clean chunk preceded by a noisy
    one that reads the weights the clean chunk reads."""
    flags = [APPLY, UPDATE | APPLY] * n_clean
    b = [i * chunk for i in range(len(flags) + 1)]
    return tuple(b), tuple(flags)


def _viewset_schedule(prefill: bool = False):
    """Posed-view set: update on the 48 x 64 x 64 = 196,608 input tokens, then
    apply to 4,096 target tokens; with prefill, also apply to the inputs."""
    n_in = 48 * (512 // 8) * (512 // 8)   # 196,608 input tokens
    n_tgt = 4096
    return (0, n_in, n_in + n_tgt), ((UPDATE | APPLY) if prefill else UPDATE, APPLY)


def _make_workloads() -> Dict[int, Workload]:
    c = {}
    b, f = uniform_schedule(1024, 256)
    c[1] = Workload(1, "tiny_lm_d64_fp32_gd", 1, 64, 1024, b, f, APPLY_THEN_UPDATE,
                    OPT_GD, DTYPE_F32, True, 3, 1e-4)
    b, f = uniform_schedule(32768, 2048)
    c[2] = Workload(2, "lm760m_d384_bf16_momentum", 4, 384, 32768, b, f, APPLY_THEN_UPDATE,
                    OPT_MOMENTUM, DTYPE_BF16, True, 1, 2e-2)
    b, f = uniform_schedule(32768, 4096)
    c[3] = Workload(3, "lm3b_d512_bf16_muon", 6, 512, 32768, b, f, APPLY_THEN_UPDATE,
                    OPT_MUON, DTYPE_BF16, True, 2, 2e-2)
    b, f = _viewset_schedule()
    c[4] = Workload(4, "viewset_d128_bf16_gd", 6, 128, b[-1], b, f, UPDATE_THEN_APPLY,
                    OPT_GD, DTYPE_BF16, False, 1, 2e-2)
    b, f = video_schedule(12, 4680)
    c[5] = Workload(5, "video_d128_bf16_muon", 40, 128, b[-1], b, f, APPLY_THEN_UPDATE,
                    OPT_MUON, DTYPE_BF16, True, 3, 2e-2)
    # schedule variants of the same layers
    b, f = _viewset_schedule(prefill=True)
    c[6] = Workload(6, "viewset_prefill_d128_bf16_gd", 6, 128, b[-1], b, f, UPDATE_THEN_APPLY,
                    OPT_GD, DTYPE_BF16, False, 1, 2e-2)
    b, f = video_schedule_noisy_first(12, 4680)
    c[7] = Workload(7, "video_noisy_first_d128_bf16_muon", 40, 128, b[-1], b, f, APPLY_THEN_UPDATE,
                    OPT_MUON, DTYPE_BF16, True, 3, 2e-2)
    # raw q, k pre-processed by the layer, and the per-token output scale:
    # the 760M-LM layer with its input/output scaling inside the layer
    b, f = uniform_schedule(32768, 2048)
    c[9] = Workload(9, "lm760m_d384_bf16_momentum_raw_qk_scaled", 4, 384, 32768, b, f, APPLY_THEN_UPDATE,
                    OPT_MOMENTUM, DTYPE_BF16, False, 1, 2e-2, layer_qk_prep=True, out_scale=True)
    # optimiser variant: the 3B-LM layer with momentum + Muon
    b, f = uniform_schedule(32768, 4096)
    c[8] = Workload(8, "lm3b_d512_bf16_muon_momentum", 6, 512, 32768, b, f, APPLY_THEN_UPDATE,
                    OPT_MUON_MOMENTUM, DTYPE_BF16, True, 2, 2e-2)
    # fast-weight width variant: the 760M-LM layer with a hidden width dh = 2d
    b, f = uniform_schedule(32768, 2048)
    c[10] = Workload(10, "lm760m_d384_dh768_bf16_momentum", 4, 384, 32768, b, f, APPLY_THEN_UPDATE,
                     OPT_MOMENTUM, DTYPE_BF16, True, 1, 2e-2, Dh=768)
    return c


WORKLOADS: Dict[int, Workload] = _make_workloads()


# ---------------------------------------------------------------- rounding

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact fp64 value of a generated array (uint16 = bf16 bits)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- generator

@dataclasses.dataclass
class Inputs:
    q: np.ndarray      # [n, L, D]  float32 or uint16 (bf16 bits)
    k: np.ndarray
    v: np.ndarray
    lr: np.ndarray     # [n, L, 3] float32
    beta: Optional[np.ndarray]   # [n, L] float32 (momentum only)
    W1: np.ndarray     # [n, dh, d] float32
    W2: np.ndarray     # [n, d, dh] float32
    W3: np.ndarray     # [n, dh, d] float32
    oz: Optional[np.ndarray] = None   # [n, L] float32 output-scale pre-activation


def _qk_prep(x: np.ndarray) -> np.ndarray:
    # input recipe, not part of the layer: silu then per-token L2 normalisation
    x = x / (1.0 + np.exp(-x))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _draw_instance(wl: Workload, seed: int, inst: int):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.cid, inst])))
    L, D = wl.L, wl.D
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    if wl.qk_prep:
        q = _qk_prep(q)
        k = _qk_prep(k)
    zlr = rng.standard_normal((L, 3))
    lr = np.logaddexp(0.0, zlr - 5.0)            # softplus
    beta = None
    if wl.opt in (OPT_MOMENTUM, OPT_MUON_MOMENTUM):
        zb = rng.standard_normal(L)
        beta = 1.0 / (1.0 + np.exp(-(zb + 2.2)))
    # W ~ N(0, 1/fan-in): W1, W3 [dh, d] (fan-in d), W2 [d, dh] (fan-in dh)
    dh = wl.dh
    W1 = rng.standard_normal((dh, D)) / np.sqrt(D)
    W2 = rng.standard_normal((D, dh)) / np.sqrt(dh)
    W3 = rng.standard_normal((dh, D)) / np.sqrt(D)
    # output-scale pre-activation (drawn last: earlier draws are unchanged)
    oz = rng.standard_normal(L) if wl.out_scale else None

    def io(x):
        x32 = x.astype(np.float32)
        return f32_to_bf16_bits(x32) if wl.io_dtype == DTYPE_BF16 else x32

    return (io(q), io(k), io(v), lr.astype(np.float32),
            None if beta is None else beta.astype(np.float32),
            W1.astype(np.float32), W2.astype(np.float32), W3.astype(np.float32),
            None if oz is None else oz.astype(np.float32))


def generate(wl: Workload, seed: int = 0, threads: int = 8) -> Inputs:
    """Draw all instances (per-instance seeded, so any subset of instances is
    reproducible on its own)."""
    with ThreadPoolExecutor(max_workers=max(1, min(threads, wl.n_inst))) as ex:
        parts = list(ex.map(lambda i: _draw_instance(wl, seed, i), range(wl.n_inst)))
    st = lambda j: np.stack([p[j] for p in parts])
    beta = st(4) if parts[0][4] is not None else None
    oz = st(8) if parts[0][8] is not None else None
    return Inputs(st(0), st(1), st(2), st(3), beta, st(5), st(6), st(7), oz)


def generate_instance(wl: Workload, inst: int, seed: int = 0) -> Inputs:
    """One instance (n = 1 arrays), identical to row `inst` of generate()."""
    p = _draw_instance(wl, seed, inst)
    e = lambda a: None if a is None else a[None]
    return Inputs(e(p[0]), e(p[1]), e(p[2]), e(p[3]), e(p[4]), e(p[5]), e(p[6]), e(p[7]), e(p[8]))


# ---------------------------------------------------------------- work counts

def algorithmic_flops(wl: Workload) -> Dict[str, float]:
    """Work the method must do (MFMA-countable contractions only).

    update: 12 d dh per (token, instance): the three forward products on k/v
            (6 d dh) and the three weight-gradient contractions (6 d dh);
    apply:   6 d dh per (query, instance);
    Newton-Schulz (Muon, d = dh): 5 iterations x 3 products x 2 D^3 per
            matrix, three matrices per instance per update chunk.
    """
    D, dh, n = wl.D, wl.dh, wl.n_inst
    upd = app = 0
    n_upd = 0
    for (a, b), f in zip(zip(wl.bounds[:-1], wl.bounds[1:]), wl.flags):
        if f & UPDATE:
            upd += b - a
            n_upd += 1
        if f & APPLY:
            app += b - a
    fu = 12.0 * D * dh * upd * n
    fa = 6.0 * D * dh * app * n
    fns = (30.0 * D ** 3 * 3 * n_upd * n) if wl.opt in (OPT_MUON, OPT_MUON_MOMENTUM) else 0.0
    return {"update": fu, "apply": fa, "ns": fns, "total": fu + fa + fns}
