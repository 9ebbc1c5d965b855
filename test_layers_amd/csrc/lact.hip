// liblact: host side of the gfx950 LaCT fast-weight layer.
//
// Validation (before any HIP call), chunk planning, workspace layout,
// precision dispatch and kernel launches for the C ABI in include/lact.h.
// All device work is asynchronous on the caller's stream.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <dlfcn.h>

#include <algorithm>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <type_traits>
#include <vector>

#include "lact.h"
#include "lact_direct.hpp"
#include "lact_planes.hpp"
#include "lact_backward.hpp"

using namespace lact;

namespace {

thread_local std::string g_err;

lact_status fail(lact_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(LACT_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

// --------------------------------------------------------------- timing (diagnostics)
struct TimingState {
  std::mutex mu;
  bool on[LACT_K_COUNT] = {};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[LACT_K_COUNT];
};
TimingState& timing() {
  static TimingState t;
  return t;
}

// While timing is enabled for its class, a KernelTimer scope hands its two
// events to the first kernel launched inside it (LACT_LAUNCH), whose dispatch
// records them at kernel start and end: the execution time alone, the window
// a kernel trace reports, without the gap before the dispatch.
struct KernelTimer;
KernelTimer*& current_timer() {
  static thread_local KernelTimer* t = nullptr;
  return t;
}
struct KernelTimer {
  hipEvent_t a = nullptr, b = nullptr;
  int kc;
  bool launched = false;
  KernelTimer* prev;
  KernelTimer(int kclass, hipStream_t) : kc(kclass), prev(current_timer()) {
    current_timer() = this;
    TimingState& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on[kc]) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      a = b = nullptr;
    }
  }
  ~KernelTimer() {
    current_timer() = prev;
    if (!a) return;
    if (!launched) {
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
      return;
    }
    TimingState& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.ev[kc].push_back({a, b});
  }
};

#define LACT_LAUNCH(kernel, grid, block, stream, ...)                                    \
  do {                                                                                   \
    KernelTimer* kt_ = current_timer();                                                  \
    if (kt_ && kt_->a && !kt_->launched) {                                               \
      kt_->launched = true;                                                              \
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, kt_->a, kt_->b, 0, __VA_ARGS__); \
    } else {                                                                             \
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                   \
    }                                                                                    \
  } while (0)

// --------------------------------------------------------------- host trace ranges
// With LACT_TRACE=1 in the environment the library marks its host-side
// phases (each update chunk, the batched applies, the backward's replay and
// reverse chunks) as roctx ranges, which `rocprofv3 --marker-trace` records
// next to the kernels those phases enqueue.  The roctx library is opened on
// first use; without it (or without the variable) tracing is off and costs a
// pointer test.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};
const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx x;
    const char* e = getenv("LACT_TRACE");
    if (!e || strcmp(e, "1") != 0) return x;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) return x;
    x.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    x.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (!x.push || !x.pop) x.push = nullptr, x.pop = nullptr;
    return x;
  }();
  return r;
}
struct TraceRange {
  bool on;
  explicit TraceRange(const char* fmt, ...) : on(roctx().push != nullptr) {
    if (!on) return;
    char buf[128];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    roctx().push(buf);
  }
  ~TraceRange() {
    if (on) roctx().pop();
  }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

// --------------------------------------------------------------- device check
lact_status check_device() {
  static std::mutex mu;
  static std::vector<int> ok;  // per device: 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
    return fail(LACT_ERR_NO_DEVICE, "no HIP device is visible");
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(LACT_ERR_NO_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> g(mu);
  if ((int)ok.size() <= dev) ok.resize(dev + 1, 0);
  if (ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(LACT_ERR_HIP, "hipGetDeviceProperties failed");
    ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (ok[dev] < 0) return fail(LACT_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return LACT_OK;
}

// --------------------------------------------------------------- precision profiles
enum Prof { PF32 = 0, PBF16 = 1, PBF16X2 = 2, PBF16X3 = 3 };

bool uses_momentum(int opt) { return opt == LACT_OPT_MOMENTUM || opt == LACT_OPT_MUON_MOMENTUM; }
bool uses_ns(int opt) { return opt == LACT_OPT_MUON || opt == LACT_OPT_MUON_MOMENTUM; }

// rec_planes = 0 picks the default: one plane (plain bf16) for GD and
// momentum, whose recurrence keeps bf16 rounding flat over many chunks; three
// (fp32 grade) for the Newton-Schulz optimisers, whose recurrence amplifies
// the rounding of every update (about x2 per chunk with one plane)
Prof profile_of(const lact_problem& p) {
  if (p.io_dtype == LACT_DTYPE_F32) return PF32;
  int rp = p.rec_planes == 0 ? (uses_ns(p.opt) ? 3 : 1) : p.rec_planes;
  return rp == 1 ? PBF16 : rp == 2 ? PBF16X2 : PBF16X3;
}
size_t io_size(const lact_problem& p) { return p.io_dtype == LACT_DTYPE_F32 ? 4 : 2; }
// bf16 planes per Newton-Schulz operand
int ns_planes(Prof f) { return f == PBF16 ? 1 : f == PBF16X2 ? 2 : 3; }
// square matrices that fit a workgroup's LDS: the whole orthogonalisation
// of a matrix runs in one workgroup (ns_small_kernel)
bool ns_small(const lact_problem& p) { return p.d == p.dh && p.d <= 128; }
// update terms storage per element: bf16, fp32, or two / three bf16 planes
size_t rec_size(Prof f) { return f == PBF16 ? 2 : f == PBF16X3 ? 6 : 4; }
// bf16 planes of the update forward's weight operands beyond the snapshot
int weight_lo_planes(Prof f) { return f == PBF16X2 ? 1 : f == PBF16X3 ? 2 : 0; }
size_t app_size(Prof f) { return f == PF32 ? 4 : 2; }    // gated hidden of the queries

// --------------------------------------------------------------- plan
struct Step {
  int64_t app_t0 = 0, app_len = 0;
  int64_t upd_t0 = 0, upd_len = 0;
};

struct Plan {
  std::vector<Step> steps;
  int64_t max_app = 0, max_upd = 0;
};

// Group chunks into steps that all read the same fast weights: a step applies
// (possibly several adjacent chunks' queries) and then updates with one chunk.
// Apply-then-update: an UPDATE|APPLY chunk's queries join its own step.
// Update-then-apply: they join the next step (after the chunk's update).
// APPLY-only chunks read the current weights and join the pending apply range.
void build_plan(int32_t order, const std::vector<int64_t>& b, const std::vector<uint8_t>& f, Plan& plan) {
  int64_t max_chunk = 0;
  for (size_t c = 0; c + 1 < b.size(); ++c) max_chunk = std::max(max_chunk, b[c + 1] - b[c]);
  const int64_t app_cap = 2 * max_chunk;
  bool pend = false;
  int64_t pa = 0, pl = 0;
  auto add_apply = [&](int64_t a0, int64_t len) {
    if (pend && pa + pl == a0 && pl + len <= app_cap) {
      pl += len;
      return;
    }
    if (pend) {
      Step s;
      s.app_t0 = pa;
      s.app_len = pl;
      plan.steps.push_back(s);
    }
    pend = true;
    pa = a0;
    pl = len;
  };
  for (size_t c = 0; c < f.size(); ++c) {
    const int64_t a0 = b[c], len = b[c + 1] - b[c];
    const bool U = f[c] & LACT_CHUNK_UPDATE, A = f[c] & LACT_CHUNK_APPLY;
    if (A && (order == LACT_APPLY_THEN_UPDATE || !U)) add_apply(a0, len);
    if (U) {
      Step s;
      if (pend) {
        s.app_t0 = pa;
        s.app_len = pl;
        pend = false;
      }
      s.upd_t0 = a0;
      s.upd_len = len;
      plan.steps.push_back(s);
      if (A && order == LACT_UPDATE_THEN_APPLY) add_apply(a0, len);
    }
  }
  if (pend) {
    Step s;
    s.app_t0 = pa;
    s.app_len = pl;
    plan.steps.push_back(s);
  }
  for (const Step& s : plan.steps) {
    plan.max_app = std::max(plan.max_app, s.app_len);
    plan.max_upd = std::max(plan.max_upd, s.upd_len);
  }
}

// --------------------------------------------------------------- tiling heuristics
constexpr int LDS_MAX = 160 * 1024;

// workgroups of 128x128 GEMM tiles -> tile edge
// 128-wide tiles only for grids that stay several rounds deep with them
int gemm_tile(int64_t wgs128) { return wgs128 >= 4 * NCU ? 128 : 64; }

// the column-k operand tile of the contraction must not overhang D
int dw_tile(const lact_problem& p) { return p.d % 128 == 0 ? 128 : 64; }

// split of the chunk's tokens for the weight-gradient contraction; split
// lengths are multiples of 64 tokens
int64_t round128(int64_t x) { return (x + 127) / 128 * 128; }

void dw_split(const lact_problem& p, int64_t C, int& S, int64_t& kps) {
  const int bt = dw_tile(p);
  const int64_t tiles = (int64_t)((3 * p.dh + bt - 1) / bt) * (p.d / bt) * std::max(1, p.n_inst);
  // Split count: the filled fraction of the last round of (one-per-CU)
  // workgroups, minus a charge per split for the partial set it writes and
  // the optimiser (or the Newton-Schulz row reduction) re-reads: 3 d dh per
  // instance, bf16 partials in the plain-bf16 recurrence (~0.2 d / C
  // against the E and k, v traffic), fp32 otherwise (measured on the 3B-LM
  // layer's two-plane contraction: 3 splits 104 us, 2: 107, 4: 110, 6: 127,
  // i.e. ~0.5 d / C); ties go to instances x splits a multiple of the 8
  // XCDs (every XCD then receives whole (instance, split) groups).
  const int64_t n = std::max(1, p.n_inst);
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(64, C / 256));
  const bool part16 = profile_of(p) == PBF16 && !uses_ns(p.opt);
  const double charge = (part16 ? 0.2 : 0.5) * (double)p.d / (double)std::max<int64_t>(1, C);
  int64_t s = 1;
  double best = -1e9;
  for (int64_t c = 1; c <= smax; ++c) {
    const int64_t wgs = tiles * c;
    const double fill = (double)wgs / (double)(((wgs + NCU - 1) / NCU) * NCU);
    const double score = fill - charge * (double)c + ((n * c) % 8 == 0 ? 0.005 : 0.0);
    if (score > best + 1e-12) {
      best = score;
      s = c;
    }
  }
  s = std::max<int64_t>(1, std::min<int64_t>(s, 64));
  kps = round128((C + s - 1) / s);
  S = (int)((C + kps - 1) / kps);
  if (S < 1) S = 1;
}

// long chunks at d = dh = 128 run the update forward and the contraction as
// one kernel (the update terms stay in LDS): plain bf16 from 4,096 tokens,
// the multi-plane recurrence (whose update terms would cross HBM as two or
// three planes) from 1,024
bool fused_update(const lact_problem& p, int64_t C) {
  if (p.d != UDW_D || p.dh != UDW_D) return false;
  const Prof f = profile_of(p);
  if (f == PBF16) return C >= 4096;
  return (f == PBF16X2 || f == PBF16X3) && C >= 1024;
}

// its token split (32-token tiles, 128 / udp_bj hidden blocks per instance,
// one workgroup per CU by LDS), every split non-empty: the split count that
// minimises rounds of workgroups x tiles per workgroup plus the cost of the
// splits' fp32 partials (each written once and read once by the reduction,
// ~5 TB/s), in units of a tile's run time (measured: ~1.0 us with one
// plane, ~1.3 us with planes); the smaller count on ties
void udw_split(const lact_problem& p, int64_t C, int& S, int& tps) {
  const int64_t tt = (C + UDS_T - 1) / UDS_T;
  const bool plain = profile_of(p) == PBF16;
  const int64_t n = std::max(1, p.n_inst);
  const int64_t per = (UDW_D / udp_bj(plain ? 1 : 2)) * n;
  const double part_bytes = 2.0 * (double)n * 3 * UDW_D * UDW_D * sizeof(float);
  const double split_cost = part_bytes / (5e12 * (plain ? 1.0e-6 : 1.3e-6));
  double best = -1;
  int64_t bt = tt;
  for (int64_t c = 1; c <= std::min<int64_t>(tt, 32); ++c) {
    const int64_t t = (tt + c - 1) / c;
    const int64_t cs = (tt + t - 1) / t;   // splits actually used
    const double cost = (double)(((per * cs + NCU - 1) / NCU) * t) + split_cost * (double)cs;
    if (best < 0 || cost < best - 1e-9) {
      best = cost;
      bt = t;
    }
  }
  tps = (int)bt;
  S = (int)((tt + tps - 1) / tps);
}

// hidden-column block of the update forward tile: the one whose workgroup
// count fills the chip best (ties go to the wider block)
int upd_bj(const lact_problem& p, int64_t C) {
  const int64_t tt = (C + FBT - 1) / FBT;
  int best = 64;
  double best_eff = -1;
  // plain-bf16 direct-load tiles fit BJ <= 96; the multi-plane tile is
  // built for BJ = 64, and the fp32 register-path tile is free of register
  // spills only there
  const bool direct = profile_of(p) == PBF16;
  for (int bj : {128, 96, 64}) {
    if (bj == 128 || (!direct && bj != 64)) continue;
    if (p.dh % bj) continue;
    const int64_t wgs = tt * (p.dh / bj) * p.n_inst;
    const int64_t rounds = (wgs + 255) / 256;
    const double eff = (double)wgs / (double)(rounds * 256);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = bj;
    }
  }
  return best;
}


// the whole apply in one kernel with the tile's gated hidden kept in LDS:
// bf16 apply operands and a hidden width of one 128-column block (there the
// apply is bound by HBM traffic, which the fused kernel halves)
bool fused_apply(const lact_problem& p) { return profile_of(p) != PF32 && p.dh == 128 && p.d % 128 == 0; }

// --------------------------------------------------------------- workspace layout
struct Ws {
  size_t e = 0, h = 0, part = 0, bpart = 0, snap = 0, u = 0, am = 0, bm = 0, xa = 0, xb = 0, rowsq = 0, total = 0;
  size_t xp0 = 0, xp1 = 0, ap = 0, bp = 0;   // Newton-Schulz operand planes (d = dh)
  size_t wlo = 0;                            // weight operand planes 1.. of the next update
  size_t qp = 0, kp = 0;  // pre-processed q / k ([n, prep_rows, D], LACT_QK_PREP)
  int64_t prep_rows = 0;
  size_t snap_slot = 0;   // bytes per snapshot slot (W1, W2, W3, W2^T)
  int S = 1;
  int nslots = 1;
  int64_t ldE = 0;
  int64_t h_rows = 0;
  int max_tt = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Ws layout(const lact_problem& p, const Plan& plan) {
  Ws w;
  const Prof f = profile_of(p);
  const size_t n = (size_t)std::max(0, p.n_inst), D = (size_t)p.d, Dh = (size_t)p.dh;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  // the token split count is not monotone in the chunk length (rounding of
  // the split size), so size the partials for the largest count of any step
  int S = 1, nupd = 0;
  int64_t h_rows = 0, rows = 0;
  for (const Step& st : plan.steps) {
    h_rows += st.app_len;
    rows = std::max(rows, std::max(st.app_t0 + st.app_len, st.upd_t0 + st.upd_len));
    if (st.upd_len == 0) continue;
    ++nupd;
    int s_ = 1;
    int64_t kps = 0;
    dw_split(p, st.upd_len, s_, kps);
    if (fused_update(p, st.upd_len)) {
      int tps = 0;
      udw_split(p, st.upd_len, s_, tps);
    }
    S = std::max(S, s_);
  }
  w.S = S;
  w.nslots = nupd + 1;
  w.ldE = round128(plan.max_upd);
  w.h_rows = h_rows;
  // beta partial sums: one per 128-token tile, or per 32-token tile of the
  // fused update
  w.max_tt = (int)((plan.max_upd + UDS_T - 1) / UDS_T);
  const size_t snap_el = (f == PF32) ? 4 : 2;
  w.snap_slot = align256(4 * n * D * Dh * snap_el);
  bool unfused = false;   // the fused update keeps its update terms in LDS
  for (const Step& st : plan.steps)
    if (st.upd_len > 0 && !fused_update(p, st.upd_len)) unfused = true;
  w.e = take(unfused ? n * 3 * Dh * (size_t)w.ldE * rec_size(f) : 0);
  w.h = take(fused_apply(p) ? 0 : n * (size_t)h_rows * Dh * app_size(f));
  const size_t mats = n * 3 * D * Dh * sizeof(float);
  w.part = take(plan.max_upd > 0 ? (size_t)S * mats : 0);
  w.bpart = take(uses_momentum(p.opt) ? n * (size_t)w.max_tt * sizeof(float) : 0);
  w.snap = take(w.snap_slot * (size_t)w.nslots);
  w.wlo = take(plan.max_upd > 0 ? (size_t)weight_lo_planes(f) * 3 * n * D * Dh * sizeof(bf16_t) : 0);
  if (uses_ns(p.opt) && plan.max_upd > 0) {
    // larger square matrices keep U and A as planes only; small ones read U
    // in fp32 and keep everything else in LDS
    const bool small = ns_small(p);
    w.u = take(D == Dh && !small ? 0 : mats);
    w.am = take(D == Dh ? 0 : mats);
    w.bm = take(D == Dh ? 0 : mats);
    w.xa = take(mats);
    w.xb = take(small ? 0 : mats);
    w.rowsq = take(n * (2 * Dh + D) * sizeof(float));
    if (D == Dh && !small) {
      // operand planes of the square products: X (two, alternating), A, B
      const size_t pl = (size_t)ns_planes(f) * n * 3 * D * Dh * sizeof(bf16_t);
      w.xp0 = take(pl);
      w.xp1 = take(pl);
      w.ap = take(pl);
      w.bp = take(pl);
    }
  }
  if (p.flags & LACT_QK_PREP) {
    const size_t el = f == PF32 ? 4 : 2;
    w.prep_rows = rows;
    w.qp = take(plan.max_app > 0 ? n * (size_t)rows * D * el : 0);
    w.kp = take(plan.max_upd > 0 ? n * (size_t)rows * D * el : 0);
  }
  w.total = off;
  return w;
}

// --------------------------------------------------------------- validation
lact_status validate_problem(const lact_problem* p) {
  if (!p) return fail(LACT_ERR_INVALID_ARG, "problem is NULL");
  if (p->n_inst < 0) return fail(LACT_ERR_INVALID_ARG, "n_inst = %d < 0", p->n_inst);
  if (p->d < 64 || p->d > 1024 || p->d % 64 != 0)
    return fail(LACT_ERR_UNSUPPORTED, "d = %d: need a multiple of 64 in [64, 1024]", p->d);
  if (p->dh < 64 || p->dh > 1024 || p->dh % 64 != 0)
    return fail(LACT_ERR_UNSUPPORTED, "dh = %d: need a multiple of 64 in [64, 1024]", p->dh);
  if (p->io_dtype != LACT_DTYPE_F32 && p->io_dtype != LACT_DTYPE_BF16)
    return fail(LACT_ERR_INVALID_ARG, "io_dtype = %d", p->io_dtype);
  if (p->opt < LACT_OPT_GD || p->opt > LACT_OPT_MUON_MOMENTUM) return fail(LACT_ERR_INVALID_ARG, "opt = %d", p->opt);
  if (uses_ns(p->opt) && (p->ns_iters < 1 || p->ns_iters > 16))
    return fail(LACT_ERR_INVALID_ARG, "ns_iters = %d: need 1..16", p->ns_iters);
  if (p->rec_planes < 0 || p->rec_planes > 3) return fail(LACT_ERR_INVALID_ARG, "rec_planes = %d", p->rec_planes);
  if (p->flags & ~(LACT_NO_RENORM | LACT_QK_PREP)) return fail(LACT_ERR_INVALID_ARG, "unknown flags 0x%x", p->flags);
  return LACT_OK;
}

lact_status make_schedule(int64_t L, int64_t chunk, int32_t order, const int64_t* bounds,
                          const uint8_t* flags, int32_t n_chunks, std::vector<int64_t>& b,
                          std::vector<uint8_t>& f) {
  if (L < 0) return fail(LACT_ERR_INVALID_ARG, "L = %lld < 0", (long long)L);
  if (order != LACT_APPLY_THEN_UPDATE && order != LACT_UPDATE_THEN_APPLY)
    return fail(LACT_ERR_INVALID_ARG, "order = %d", order);
  if (bounds == nullptr && flags == nullptr) {
    if (chunk <= 0) return fail(LACT_ERR_INVALID_ARG, "chunk = %lld must be > 0", (long long)chunk);
    b.clear();
    for (int64_t t = 0; t < L; t += chunk) b.push_back(t);
    b.push_back(L);
    f.assign(b.size() - 1, LACT_CHUNK_UPDATE | LACT_CHUNK_APPLY);
    return LACT_OK;
  }
  if (!bounds || !flags) return fail(LACT_ERR_INVALID_ARG, "bounds and flags must both be given or both be NULL");
  if (n_chunks < 0) return fail(LACT_ERR_INVALID_ARG, "n_chunks = %d < 0", n_chunks);
  if (bounds[0] != 0) return fail(LACT_ERR_INVALID_ARG, "bounds[0] = %lld != 0", (long long)bounds[0]);
  for (int32_t c = 0; c < n_chunks; ++c) {
    if (bounds[c + 1] <= bounds[c])
      return fail(LACT_ERR_INVALID_ARG, "bounds not strictly increasing at chunk %d", c);
    if (flags[c] & ~(LACT_CHUNK_UPDATE | LACT_CHUNK_APPLY))
      return fail(LACT_ERR_INVALID_ARG, "flags[%d] = 0x%x", c, flags[c]);
  }
  if (bounds[n_chunks] != L)
    return fail(LACT_ERR_INVALID_ARG, "bounds[n_chunks] = %lld != L = %lld", (long long)bounds[n_chunks], (long long)L);
  b.assign(bounds, bounds + n_chunks + 1);
  f.assign(flags, flags + n_chunks);
  return LACT_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

#define NEED(ptr, al)                                                                         \
  do {                                                                                        \
    if ((ptr) == nullptr) return fail(LACT_ERR_INVALID_ARG, "%s is NULL", #ptr);             \
    if (!aligned((ptr), (al))) return fail(LACT_ERR_INVALID_ARG, "%s is not %d-byte aligned", #ptr, (int)(al)); \
  } while (0)

// --------------------------------------------------------------- launches
struct Ptrs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* lr = nullptr;
  const float* beta = nullptr;
  float* W1 = nullptr;
  float* W2 = nullptr;
  float* W3 = nullptr;
  float* M1 = nullptr;
  float* M2 = nullptr;
  float* M3 = nullptr;
  void* o = nullptr;
  const float* oz = nullptr;   // per-token output-scale pre-activation [n, seq]
  char* ws = nullptr;
};

// TIO/PIO: inputs; TS/PS: weight snapshots (apply, and the update forward in
// plain bf16); PWU: planes of fp32 weights in the update forward when it reads
// the master copy; TREC/PREC: update terms and Newton-Schulz operands;
// TAPP/PAPP: gated hidden of the queries.
// PL > 1: the multi-plane recurrence on direct-load tiles -- the weight
// operands of the update forward stream as stored bf16 planes (plane 0 the
// snapshot, planes 1.. written beside it by the optimiser), the update terms
// and the Newton-Schulz operands are stored as PL bf16 planes.
template <typename TIO_, int PIO_, typename TS_, int PS_, int PWU_, typename TREC_, int PREC_, typename TAPP_,
          int PAPP_, int PL_ = 0>
struct ProfT {
  using TIO = TIO_;
  using TS = TS_;
  using TREC = TREC_;
  using TAPP = TAPP_;
  static constexpr int PIO = PIO_, PS = PS_, PWU = PWU_, PREC = PREC_, PAPP = PAPP_, PL = PL_;
  static constexpr bool UPD_FROM_SNAP = (PWU_ == 0);
};
using ProfF32 = ProfT<float, 3, float, 3, 3, float, 3, float, 3>;
using ProfBF16 = ProfT<bf16_t, 1, bf16_t, 1, 0, bf16_t, 1, bf16_t, 1>;
using ProfBF16X2 = ProfT<bf16_t, 1, bf16_t, 1, 2, float, 2, bf16_t, 1, 2>;
using ProfBF16X3 = ProfT<bf16_t, 1, bf16_t, 1, 3, float, 3, bf16_t, 1, 3>;

// k-stage depth and buffering that fit the LDS
constexpr int pick_bk(int planes_sum) { return planes_sum <= 2 ? 64 : 32; }
constexpr int stage_words(int rows_a, int pa, int rows_b, int pb, int bk) { return (rows_a * pa + rows_b * pb) * (bk + 8); }
constexpr int pick_stages(int words) { return 2 * words * 2 + 4096 <= LDS_MAX ? 2 : 1; }

template <typename TA, int PA, bool CA, typename TB, int PB, bool CB, typename TC, int BM>
lact_status launch_gemm_t(const GemmArgs& g, int64_t grid, hipStream_t s) {
  if constexpr (sizeof(TA) == 2 && sizeof(TB) == 2) {
    // both operands bf16: direct-load kernel (8 waves).  A k stage of width W
    // must not cross a split boundary, and its reads past K must stay within
    // a row-k operand's zero padding (column-k operands clamp their rows)
    auto fits = [&](int64_t W) {
      return (g.splits == 1 || g.kps % W == 0) && (g.K % W == 0 || g.kpad >= (g.K + W - 1) / W * W);
    };
    // short contractions (a few stages per tile): a two-stage 64-wide ring
    // that leaves room for two workgroups per CU, so one's prologue and
    // epilogue overlap the other's main loop; long ones: 128-wide stages
    if (g.kps <= 512 && fits(64)) {
      LACT_LAUNCH((dgemm_kernel<CA, CB, TC, BM, 64, 2>), dim3((unsigned)grid), dim3(DG_THREADS), s, g);
    } else if (fits(128)) {
      LACT_LAUNCH((dgemm_kernel<CA, CB, TC, BM, 128, 2>), dim3((unsigned)grid), dim3(DG_THREADS), s, g);
    } else if (fits(64)) {
      LACT_LAUNCH((dgemm_kernel<CA, CB, TC, BM, 64, 4>), dim3((unsigned)grid), dim3(DG_THREADS), s, g);
    } else {
      return fail(LACT_ERR_UNSUPPORTED, "internal: contraction length %lld / split %lld not 64-aligned",
                  (long long)g.K, (long long)g.kps);
    }
    HIP_TRY(hipGetLastError());
    return LACT_OK;
  }
  constexpr int BKK = pick_bk(PA + PB);
  constexpr int ST = pick_stages(stage_words(BM, PA, BM, PB, BKK));
  LACT_LAUNCH((gemm_kernel<TA, PA, CA, TB, PB, CB, TC, BM, BM, BKK, ST>), dim3((unsigned)grid), dim3(NT), s,
                     g);
  HIP_TRY(hipGetLastError());
  return LACT_OK;
}

// fills in per-group tile counts and launches
template <typename TA, int PA, bool CA, typename TB, int PB, bool CB, typename TC>
lact_status launch_gemm(GemmArgs g, int tile, int kclass, hipStream_t s) {
  int64_t grid = 0;
  if (g.sym) {
    if constexpr (sizeof(TA) == 2 && sizeof(TB) == 2)
      return fail(LACT_ERR_UNSUPPORTED, "internal: symmetric products run on the register-path GEMM");
    for (int i = 0; i < g.ngroups; ++i)
      if (g.g[i].M != g.N) return fail(LACT_ERR_UNSUPPORTED, "internal: symmetric product of a non-square block");
  }
  for (int i = 0; i < g.ngroups; ++i) {
    const int64_t tt = (g.N + tile - 1) / tile;
    const int64_t t = (g.sym ? tt * (tt + 1) / 2 : (int64_t)((g.g[i].M + tile - 1) / tile) * tt) * g.batch * g.splits;
    if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    g.g[i].tiles = (int)t;
    grid += t;
  }
  if (grid <= 0) return LACT_OK;
  if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
  KernelTimer kt(kclass, s);
  if (tile == 128) return launch_gemm_t<TA, PA, CA, TB, PB, CB, TC, 128>(g, grid, s);
  return launch_gemm_t<TA, PA, CA, TB, PB, CB, TC, 64>(g, grid, s);
}

GemmArgs gemm_args() {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.ngroups = 1;
  g.splits = 1;
  g.batch = 1;
  g.alpha = 1.f;
  g.m_switch = 1 << 30;
  g.trans_from = 1 << 30;
  return g;
}

// bf16 snapshot profile: direct-load kernels
constexpr bool direct_fits(int bytes) { return bytes + 1024 <= LDS_MAX; }

template <typename PT, int BJ>
lact_status launch_upd_fwd(const UpdFwdArgs& ua, int64_t grid, hipStream_t s) {
  if constexpr (PT::PL > 1) {
    // weight planes from the snapshot, update terms stored as planes;
    // 32-wide stages: two deep for two planes (80 KB, two workgroups per
    // CU, one's prologue and epilogue beside the other's products), three
    // deep for three
    if constexpr (BJ == 64) {
      constexpr int NST = PT::PL == 2 ? 2 : 3;
      LACT_LAUNCH((dupd_fwd_kernel<64, 32, NST, false, PT::PL>), dim3((unsigned)grid), dim3(DG_THREADS), s, ua);
      HIP_TRY(hipGetLastError());
      return LACT_OK;
    } else {
      return fail(LACT_ERR_UNSUPPORTED, "internal: plane update tile of %d columns", BJ);
    }
  } else if constexpr (PT::UPD_FROM_SNAP && (BJ == 64 || BJ == 96)) {
    // with the chunk's queries the ring holds a third token tile: 32-wide
    // stages, three deep, fit the LDS
    if (ua.q != nullptr) LACT_LAUNCH((dupd_fwd_kernel<BJ, 32, 3, true>), dim3((unsigned)grid), dim3(DG_THREADS), s, ua);
    else LACT_LAUNCH((dupd_fwd_kernel<BJ, 64, 2>), dim3((unsigned)grid), dim3(DG_THREADS), s, ua);
    HIP_TRY(hipGetLastError());
    return LACT_OK;
  } else if constexpr (BJ != 64) {
    // the register-path tile is free of register spills only at 64 columns
    return fail(LACT_ERR_UNSUPPORTED, "internal: register-path update tile of %d columns", BJ);
  } else {
    using TW = typename std::conditional<PT::UPD_FROM_SNAP, typename PT::TS, float>::type;
    constexpr int PW = PT::UPD_FROM_SNAP ? PT::PS : PT::PWU;
    constexpr int BKK = pick_bk(PT::PIO + PW);
    constexpr int words = (2 * PT::PIO * FBT + 3 * PW * BJ) * (BKK + 8);
    constexpr int ST = pick_stages(words);
    LACT_LAUNCH((upd_fwd_kernel<typename PT::TIO, PT::PIO, TW, PW, typename PT::TREC, BJ, BKK, ST>),
                dim3((unsigned)grid), dim3(NT), s, ua);
    HIP_TRY(hipGetLastError());
    return LACT_OK;
  }
}

// weight-gradient contraction with the update terms as PL bf16 planes
// (second operand: the chunk's k and v, column-k)
template <int PL>
lact_status launch_dw_planes(GemmArgs g, int tile, hipStream_t s) {
  if (g.splits != 1 && g.kps % 64) return fail(LACT_ERR_UNSUPPORTED, "internal: contraction split %lld", (long long)g.kps);
  if (g.K % 64 && g.kpad < (g.K + 63) / 64 * 64) return fail(LACT_ERR_UNSUPPORTED, "internal: contraction padding");
  int64_t grid = 0;
  for (int i = 0; i < g.ngroups; ++i) {
    const int64_t t = (int64_t)((g.g[i].M + tile - 1) / tile) * ((g.N + tile - 1) / tile) * g.batch * g.splits;
    if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    g.g[i].tiles = (int)t;
    grid += t;
  }
  if (grid <= 0) return LACT_OK;
  if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
  KernelTimer kt(LACT_K_DW, s);
  constexpr int NST = PL <= 2 ? 3 : 2;   // 48 KB (two planes) or 64 KB stages at 128-wide tiles
  if (tile == 128) LACT_LAUNCH((dgemm_kernel<false, true, float, 128, 64, NST, PL>), dim3((unsigned)grid), dim3(DG_THREADS), s, g);
  else LACT_LAUNCH((dgemm_kernel<false, true, float, 64, 64, NST, PL>), dim3((unsigned)grid), dim3(DG_THREADS), s, g);
  HIP_TRY(hipGetLastError());
  return LACT_OK;
}

// o = Hq W2^T with the apply tile (bf16 operands only); returns false when
// the profile has no such path
template <typename PT, int BJ>
bool launch_app_out(const AppFwdArgs& aa, int64_t grid, hipStream_t s, lact_status* st) {
  if constexpr (sizeof(typename PT::TIO) == 2 && sizeof(typename PT::TS) == 2 && sizeof(typename PT::TAPP) == 2) {
    LACT_LAUNCH((dapp_fwd_kernel<BJ, 32, 3, true>), dim3((unsigned)grid), dim3(NT), s, aa);
    *st = hipGetLastError() == hipSuccess ? LACT_OK : fail(LACT_ERR_HIP, "output launch failed");
    return true;
  }
  return false;
}

template <typename PT, int BJ>
lact_status launch_app_fwd(const AppFwdArgs& aa, int64_t grid, hipStream_t s) {
  if constexpr (sizeof(typename PT::TIO) == 2 && sizeof(typename PT::TS) == 2) {
    LACT_LAUNCH((dapp_fwd_kernel<BJ, 32, 3>), dim3((unsigned)grid), dim3(NT), s, aa);
    HIP_TRY(hipGetLastError());
    return LACT_OK;
  } else if constexpr (BJ != 64) {
    // the register-path tile is free of register spills only at 64 columns
    return fail(LACT_ERR_UNSUPPORTED, "internal: register-path apply tile of %d columns", BJ);
  } else {
    constexpr int BKK = pick_bk(PT::PIO + PT::PS);
    constexpr int words = (PT::PIO * FBT + 2 * PT::PS * BJ) * (BKK + 8);
    constexpr int ST = pick_stages(words);
    LACT_LAUNCH((app_fwd_kernel<typename PT::TIO, PT::PIO, typename PT::TS, PT::PS, typename PT::TAPP, BJ, BKK, ST>),
                dim3((unsigned)grid), dim3(NT), s, aa);
    HIP_TRY(hipGetLastError());
    return LACT_OK;
  }
}

// --------------------------------------------------------------- helper streams
// Work off the recurrence's critical path runs on two library streams per
// device (default priority, created on first use, kept until the process
// ends): the second half of every Newton-Schulz batch, and the deferred
// applies, each chunk's as soon as the snapshot it reads exists.  They are
// tied to the caller's stream by events in both directions, so a call still
// completes, as seen from the caller's stream, when the caller's stream says
// so, and a graph captured from the caller's stream captures them too.
// The mutex is held while a call enqueues its work (host side only).
struct DevAux {
  hipStream_t ns = nullptr, app = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, ready = nullptr, done = nullptr;
};
std::mutex& aux_mutex() {
  static std::mutex m;
  return m;
}
// call with aux_mutex() held
lact_status dev_aux(DevAux** out) {
  static std::vector<DevAux> aux;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(LACT_ERR_NO_DEVICE, "hipGetDevice failed");
  if ((int)aux.size() <= dev) aux.resize(dev + 1);
  DevAux& a = aux[dev];
  if (a.ns == nullptr) {
    DevAux x;
    if (hipStreamCreateWithFlags(&x.ns, hipStreamNonBlocking) != hipSuccess ||
        hipStreamCreateWithFlags(&x.app, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&x.join, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&x.ready, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&x.done, hipEventDisableTiming) != hipSuccess)
      return fail(LACT_ERR_HIP, "creating the helper streams and events failed");
    a = x;
  }
  *out = &a;
  return LACT_OK;
}
// `to` waits for everything enqueued on `from` so far
lact_status stream_after(hipStream_t to, hipStream_t from, hipEvent_t ev) {
  HIP_TRY(hipEventRecord(ev, from));
  HIP_TRY(hipStreamWaitEvent(to, ev, 0));
  return LACT_OK;
}

// plane GEMM (lact_planes.hpp): P planes per operand; B column-k when colk;
// the result's planes stored when a group has Cp
template <int P, class S = PgSmall>
lact_status launch_pgemm(GemmArgs g, bool colk, int kclass, hipStream_t s) {
  if (g.N % S::BN || g.K % S::BK || g.splits != 1)
    return fail(LACT_ERR_UNSUPPORTED, "internal: plane product shape %d x %lld", g.N, (long long)g.K);
  int64_t grid = 0;
  const int64_t tt = g.N / S::BN;
  for (int i = 0; i < g.ngroups; ++i) {
    if (g.g[i].M % S::BM || (g.sym && g.g[i].M != g.N))
      return fail(LACT_ERR_UNSUPPORTED, "internal: plane product rows %d", g.g[i].M);
    const int64_t t = (g.sym ? tt * (tt + 1) / 2 : (g.g[i].M / S::BM) * tt) * g.batch;
    if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    g.g[i].tiles = (int)t;
    grid += t;
  }
  if (grid <= 0) return LACT_OK;
  if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
  KernelTimer kt(kclass, s);
  if (colk) LACT_LAUNCH((pgemm_kernel<P, P, true, P, S>), dim3((unsigned)grid), dim3(S::THREADS), s, g);
  else LACT_LAUNCH((pgemm_kernel<P, P, false, P, S>), dim3((unsigned)grid), dim3(S::THREADS), s, g);
  HIP_TRY(hipGetLastError());
  return LACT_OK;
}

template <typename PT>
lact_status run_steps(const lact_problem& p, const Ptrs& P, int64_t seq_stride, const Plan& plan, const Ws& w,
                      hipStream_t s) {
  using TIO = typename PT::TIO;
  using TS = typename PT::TS;
  using TREC = typename PT::TREC;
  using TAPP = typename PT::TAPP;
  const int n = p.n_inst, D = p.d, Dh = p.dh;
  if (n == 0) return LACT_OK;
  std::lock_guard<std::mutex> aux_lock(aux_mutex());
  DevAux* aux = nullptr;
  if (lact_status r = dev_aux(&aux)) return r;
  const bool part16 = PT::PREC == 1 && !uses_ns(p.opt);
  const int64_t DD = (int64_t)D * Dh;   // elements per fast-weight matrix
  const int64_t x_bs = seq_stride * D;
  char* ws = P.ws;
  const size_t snap_mat = (size_t)n * DD * sizeof(TS);
  // snapshot slot k holds the weights after k updates: W1, W2, W3, W2^T
  auto slot = [&](int k, int m) -> void* { return ws + w.snap + (size_t)k * w.snap_slot + (size_t)m * snap_mat; };

  // raw q / k: pre-processed copies, packed per instance, replace them
  const void* qx = P.q;
  const void* kx = P.k;
  int64_t q_bs = x_bs, k_bs = x_bs;
  if (p.flags & LACT_QK_PREP) {
    QkPrepArgs pa;
    memset(&pa, 0, sizeof(pa));
    int nm = 0;
    if (plan.max_app > 0) {
      pa.src[nm] = P.q;
      pa.dst[nm++] = ws + w.qp;
      qx = ws + w.qp;
      q_bs = w.prep_rows * D;
    }
    if (plan.max_upd > 0) {
      pa.src[nm] = P.k;
      pa.dst[nm++] = ws + w.kp;
      kx = ws + w.kp;
      k_bs = w.prep_rows * D;
    }
    pa.src_bs = x_bs;
    pa.rows = w.prep_rows;
    pa.total = (int64_t)nm * n * w.prep_rows;
    pa.n = n;
    pa.D = D;
    const int64_t blocks = (pa.total + NT / QP_LANES - 1) / (NT / QP_LANES);
    if (blocks > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    if (blocks > 0) {
      KernelTimer kt(LACT_K_PREP, s);
      LACT_LAUNCH(qk_prep_kernel<TIO>, dim3((unsigned)blocks), dim3(NT), s, pa);
      HIP_TRY(hipGetLastError());
    }
  }

  // weight operand planes 1.. of the multi-plane recurrence: [PL - 1][W1, W3, W2^T][n, dh, d]
  constexpr int SP = PT::PL > 1 ? PT::PL : 1;
  void* wlo = ws + w.wlo;
  const int64_t wlo_ms = (int64_t)n * DD, wlo_ps = 3 * wlo_ms;
  {
    const int64_t n4 = (int64_t)n * DD / 4;
    KernelTimer kt(LACT_K_SNAP, s);
    LACT_LAUNCH((snap_kernel<TS, SP>), dim3((unsigned)((n4 + NT - 1) / NT)), dim3(NT), s, P.W1, P.W2, P.W3,
                slot(0, 0), slot(0, 1), slot(0, 2), sizeof(TS) == 2 ? slot(0, 3) : nullptr, (int64_t)n * DD, D,
                Dh, wlo, wlo_ps, wlo_ms);
    HIP_TRY(hipGetLastError());
  }

  // Apply groups, one per step with queries, in step order: group i reads
  // the snapshot taken before its step's update.  When a step's queries are
  // the same tokens as its update (an apply-then-update chunk), the plain
  // bf16 update forward tile also computes their gated hidden (it holds the
  // same W1, W3 fragments); the apply then runs only the output product for
  // that group.
  std::vector<AppGroup> groups;
  std::vector<char> hq_done;
  std::vector<int> step_group(plan.steps.size(), -1);
  {
    int u = 0;
    int64_t h0 = 0;
    for (size_t si = 0; si < plan.steps.size(); ++si) {
      const Step& st = plan.steps[si];
      if (st.app_len > 0) {
        AppGroup ag;
        memset(&ag, 0, sizeof(ag));
        ag.t0 = st.app_t0;
        ag.len = st.app_len;
        ag.h0 = h0;
        ag.W1 = slot(u, 0);
        ag.W3 = slot(u, 2);
        ag.W2 = slot(u, 1);
        step_group[si] = (int)groups.size();
        groups.push_back(ag);
        hq_done.push_back(0);
        h0 += st.app_len;
      }
      if (st.upd_len > 0) ++u;
    }
  }

  // Applies of groups [ga, gb) on stream st (groups batched MAXG to a launch).
  auto apply_groups = [&](size_t ga, size_t gb, hipStream_t st) -> lact_status {
    if (fused_apply(p)) {
      for (size_t g0 = ga; g0 < gb; g0 += MAXG) {
        const int ng = (int)std::min<size_t>(MAXG, gb - g0);
        AppFwdArgs aa;
        memset(&aa, 0, sizeof(aa));
        aa.ngroups = ng;
        aa.q = qx;
        aa.q_bs = q_bs;
        aa.x_bs = x_bs;
        aa.o = P.o;
        aa.oz = P.oz;
        aa.oz_bs = seq_stride;
        aa.D = D;
        aa.Dh = Dh;
        int64_t grid = 0;
        for (int i = 0; i < ng; ++i) {
          aa.g[i] = groups[g0 + i];
          const int64_t t = ((aa.g[i].len + FBT - 1) / FBT) * n;
          if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
          aa.g[i].tiles = (int)t;
          grid += t;
        }
        if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
        KernelTimer kt(LACT_K_APP, st);
        LACT_LAUNCH((dapp_fused_kernel<128, 32, 2>), dim3((unsigned)grid), dim3(NT), st, aa);
        HIP_TRY(hipGetLastError());
      }
      return LACT_OK;
    }
    // the column block serves both the forward (dh columns) and the output
    // mode (d columns); the fp32 register-path apply tile spills at 128
    const int abj = (D % 128 == 0 && Dh % 128 == 0 && profile_of(p) != PF32) ? 128 : 64;
    for (size_t g0 = ga; g0 < gb; g0 += MAXG) {
      const int ng = (int)std::min<size_t>(MAXG, gb - g0);
      AppFwdArgs aa;
      memset(&aa, 0, sizeof(aa));
      aa.ngroups = ng;
      aa.q = qx;
      aa.q_bs = q_bs;
      aa.x_bs = x_bs;
      aa.oz = P.oz;
      aa.oz_bs = seq_stride;
      aa.H = ws + w.h;
      aa.h_bs = w.h_rows * Dh;
      aa.D = D;
      aa.Dh = Dh;
      // workgroups per group: token tiles x column blocks (cols wide) x instances
      auto set_tiles = [&](int cols, int64_t& grid) -> lact_status {
        grid = 0;
        for (int i = 0; i < aa.ngroups; ++i) {
          const int64_t t = ((aa.g[i].len + FBT - 1) / FBT) * (cols / abj) * n;
          if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
          aa.g[i].tiles = (int)t;
          grid += t;
        }
        if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
        return LACT_OK;
      };
      // gated hidden of the batch's groups not done by their update tile
      int nf = 0;
      for (int i = 0; i < ng; ++i)
        if (!hq_done[g0 + i]) aa.g[nf++] = groups[g0 + i];
      aa.ngroups = nf;
      int64_t grid = 0;
      if (nf > 0) {
        if (lact_status r = set_tiles(Dh, grid)) return r;
        KernelTimer kt(LACT_K_APP, st);
        lact_status r = abj == 128 ? launch_app_fwd<PT, 128>(aa, grid, st) : launch_app_fwd<PT, 64>(aa, grid, st);
        if (r) return r;
      }
      // output product over every group of the batch
      aa.ngroups = ng;
      for (int i = 0; i < ng; ++i) aa.g[i] = groups[g0 + i];
      // o[t, r] = sum_j Hq[t, j] W2[r, j]: the apply tile in output mode
      // (d column blocks), or the generic GEMM for profiles without a bf16 path
      {
        aa.o = P.o;
        if (lact_status r = set_tiles(D, grid)) return r;
        lact_status ost = LACT_OK;
        bool done;
        {
          KernelTimer kt(LACT_K_OUT, st);
          done = abj == 128 ? launch_app_out<PT, 128>(aa, grid, st, &ost) : launch_app_out<PT, 64>(aa, grid, st, &ost);
        }
        if (done) {
          if (ost) return ost;
          continue;
        }
      }
      GemmArgs g = gemm_args();
      g.ngroups = ng;
      int64_t wgs128 = 0;
      for (int i = 0; i < ng; ++i) {
        const AppGroup& ag = aa.g[i];
        g.g[i].A = static_cast<const char*>(aa.H) + (size_t)ag.h0 * Dh * app_size(profile_of(p));
        int u = 0;
        // the snapshot this group reads is the one its W1 came from
        for (int k = 0; k < w.nslots; ++k)
          if (slot(k, 0) == ag.W1) u = k;
        g.g[i].B = slot(u, 1);
        g.g[i].C = static_cast<char*>(P.o) + (size_t)ag.t0 * D * io_size(p);
        g.g[i].rs = P.oz ? P.oz + ag.t0 : nullptr;
        g.g[i].M = (int)ag.len;
        wgs128 += ((ag.len + 127) / 128) * std::max(1, D / 128) * n;
      }
      g.lda = Dh;
      g.a_bs = w.h_rows * Dh;
      g.ldb = Dh;          // W2 [d, dh]: row n = output unit n
      g.b_bs = DD;
      g.ldc = D;
      g.c_bs = x_bs;
      g.rs_bs = seq_stride;
      g.N = D;
      g.K = g.kps = Dh;
      g.batch = n;
      lact_status r =
          launch_gemm<TAPP, PT::PAPP, false, TS, PT::PS, false, TIO>(g, gemm_tile(wgs128), LACT_K_OUT, st);
      if (r) return r;
    }
    return LACT_OK;
  };
  // Every group whose snapshot (and, when its gated hidden came from its
  // update's tile, that update) is enqueued goes to the apply stream, after
  // what the caller's stream holds so far.
  size_t app_next = 0;
  bool launched_app = false;
  auto apply_upto = [&](size_t gb) -> lact_status {
    if (gb <= app_next) return LACT_OK;
    if (lact_status r = stream_after(aux->app, s, aux->ready)) return r;
    if (lact_status r = apply_groups(app_next, gb, aux->app)) return r;
    app_next = gb;
    launched_app = true;
    return LACT_OK;
  };

  // ---------------------------------------------------------------- recurrence
  int nu = 0;   // updates done so far
  for (size_t si = 0; si < plan.steps.size(); ++si) {
    const Step& st = plan.steps[si];
    if (st.upd_len == 0) continue;
    const int64_t C = st.upd_len;
    TraceRange tr("lact update %d: tokens %lld..%lld", nu, (long long)st.upd_t0, (long long)(st.upd_t0 + C));
    // forward products on k, v and the SwiGLU backward terms
    UpdFwdArgs ua;
    memset(&ua, 0, sizeof(ua));
    ua.k = kx;
    ua.v = P.v;
    ua.x_bs = x_bs;
    ua.k_bs = k_bs;
    ua.lr = P.lr;
    ua.lr_bs = seq_stride * 3;
    ua.beta = uses_momentum(p.opt) ? P.beta : nullptr;
    ua.beta_bs = seq_stride;
    ua.bpart = reinterpret_cast<float*>(ws + w.bpart);
    if (PT::UPD_FROM_SNAP || PT::PL > 1) {
      ua.W1 = slot(nu, 0);
      ua.W3 = slot(nu, 2);
      ua.W2x = slot(nu, 3);
      ua.Wlo = wlo;
      ua.wlo_ps = wlo_ps;
      ua.wlo_ms = wlo_ms;
    } else {
      ua.W1 = P.W1;
      ua.W3 = P.W3;
      ua.W2x = P.W2;
    }
    ua.E = ws + w.e;
    ua.ldE = round128(C);
    ua.e_ps = (int64_t)n * 3 * Dh * ua.ldE;   // plane stride of the update terms (multi-plane)
    ua.D = D;
    ua.Dh = Dh;
    ua.upd_t0 = st.upd_t0;
    ua.upd_len = C;
    ua.tiles_t = (int)((C + FBT - 1) / FBT);
    const bool fused = fused_update(p, C);
    int S = 1;
    int64_t kps = 0;
    if (fused) {
      // update forward + contraction in one kernel, fp32 partials per split
      if constexpr (PT::UPD_FROM_SNAP || PT::PL > 1) {
        constexpr int FP = PT::PL > 1 ? PT::PL : 1;   // weight planes
        constexpr int BJ = udp_bj(FP);
        int tps = 0;
        udw_split(p, C, S, tps);
        if (S > w.S) return fail(LACT_ERR_UNSUPPORTED, "internal: token split %d exceeds workspace plan %d", S, w.S);
        UpdDwArgs ud;
        memset(&ud, 0, sizeof(ud));
        ud.u = ua;
        ud.part = reinterpret_cast<float*>(ws + w.part);
        ud.part_ss = (int64_t)n * 3 * DD;
        ud.tps = tps;
        ud.splits = S;
        ud.nbp = (int)((C + UDS_T - 1) / UDS_T);
        const int64_t grid = (int64_t)n * S * (UDW_D / BJ);
        if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
        KernelTimer kt(LACT_K_UPD, s);
        LACT_LAUNCH((dupd_dwp_kernel<FP, BJ>), dim3((unsigned)grid), dim3(DG_THREADS), s, ud);
        HIP_TRY(hipGetLastError());
      }
    } else {
      const int bj = upd_bj(p, C);
      const int gi = step_group[si];
      if (std::is_same<PT, ProfBF16>::value && !fused_apply(p) && (bj == 64 || bj == 96) && gi >= 0 &&
          st.app_t0 == st.upd_t0 && st.app_len == C) {
        ua.q = qx;
        ua.q_bs = q_bs;
        ua.H = ws + w.h;
        ua.h_bs = w.h_rows * Dh;
        ua.h0 = groups[gi].h0;
        hq_done[gi] = 1;
      }
      const int64_t grid = (int64_t)n * ua.tiles_t * (Dh / bj);
      if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
      KernelTimer kt(LACT_K_UPD, s);
      lact_status r = bj == 128 ? launch_upd_fwd<PT, 128>(ua, grid, s)
                      : bj == 96 ? launch_upd_fwd<PT, 96>(ua, grid, s)
                                 : launch_upd_fwd<PT, 64>(ua, grid, s);
      if (r) return r;
    }
    // weight-gradient contraction over the chunk's tokens (split over tokens)
    if (!fused) dw_split(p, C, S, kps);
    if (S > w.S) return fail(LACT_ERR_UNSUPPORTED, "internal: token split %d exceeds workspace plan %d", S, w.S);
    if (!fused) {
      GemmArgs g = gemm_args();
      g.g[0].A = ws + w.e;         // (m, t) = E[m, t]: rows U1 | U3 | U2^T terms
      g.lda = ua.ldE;
      g.a_bs = 3 * Dh * ua.ldE;
      g.g[0].B = static_cast<const char*>(kx) + (size_t)st.upd_t0 * D * io_size(p);
      g.B2 = static_cast<const char*>(P.v) + (size_t)st.upd_t0 * D * io_size(p);
      g.m_switch = 2 * Dh;
      g.trans_from = 2 * Dh;       // the U2 block is stored as U2 [d, dh] (not U2^T)
      g.ldc_t = Dh;
      g.ldb = D;
      g.b_bs = k_bs;
      g.b2_bs = x_bs;
      g.g[0].C = ws + w.part;
      g.ldc = D;
      g.c_bs = 3 * DD;
      g.c_ss = (int64_t)n * 3 * DD;
      g.g[0].M = 3 * Dh;
      g.N = D;
      g.K = C;
      g.kps = kps;
      g.kpad = ua.ldE;             // the update forward zero-fills E up to ldE
      g.batch = n;
      g.splits = S;
      // the plain-bf16 recurrence keeps its token-split partials in bf16
      // (fp32 accumulation inside each split, fp32 sum of the splits)
      lact_status r;
      if constexpr (PT::PL > 1) {
        g.a_ps = ua.e_ps;
        r = launch_dw_planes<PT::PL>(g, dw_tile(p), s);
      } else {
        r = part16 ? launch_gemm<TREC, PT::PREC, false, TIO, PT::PIO, true, bf16_t>(g, dw_tile(p), LACT_K_DW, s)
                   : launch_gemm<TREC, PT::PREC, false, TIO, PT::PIO, true, float>(g, dw_tile(p), LACT_K_DW, s);
      }
      if (r) return r;
    }
    OptArgs oa;
    memset(&oa, 0, sizeof(oa));
    oa.W[0] = P.W1;
    oa.W[1] = P.W3;
    oa.W[2] = P.W2;
    oa.M[0] = P.M1;
    oa.M[1] = P.M3;
    oa.M[2] = P.M2;
    oa.mat_el = DD;
    oa.opt = p.opt;
    oa.renorm = (p.flags & LACT_NO_RENORM) ? 0 : 1;
    oa.bpart = reinterpret_cast<const float*>(ws + w.bpart);
    // beta partial sums: per 128-token tile, or per tile of the fused update
    const int nbp = fused ? (int)((C + UDS_T - 1) / UDS_T) : ua.tiles_t;
    oa.nbp = nbp;
    oa.inv_len = 1.0f / (float)C;
    oa.snap[0] = slot(nu + 1, 0);
    oa.snap[1] = slot(nu + 1, 2);
    oa.snap[2] = slot(nu + 1, 1);
    oa.snapT2 = sizeof(TS) == 2 ? slot(nu + 1, 3) : nullptr;
    oa.wlo = wlo;
    oa.wlo_ps = wlo_ps;
    oa.wlo_ms = wlo_ms;
    if (!uses_ns(p.opt)) {
      oa.src = ws + w.part;
      oa.src_ss = (int64_t)n * 3 * DD;
      oa.splits = S;
    } else {
      // Muon: U = sum of partials, then quintic Newton-Schulz on every matrix
      float* U = reinterpret_cast<float*>(ws + w.u);
      float* rowsq = reinterpret_cast<float*>(ws + w.rowsq);
      {
        KernelTimer kt(LACT_K_NSRED, s);
        const int64_t rows = (int64_t)n * (2 * Dh + D);
        // momentum + Muon: the Newton-Schulz input is the new momentum buffer
        // M' = mean(beta) M - U, also written back to the state
        RowsMomentum rm;
        memset(&rm, 0, sizeof(rm));
        if (p.opt == LACT_OPT_MUON_MOMENTUM) {
          rm.M[0] = P.M1;
          rm.M[1] = P.M3;
          rm.M[2] = P.M2;
          rm.bpart = reinterpret_cast<const float*>(ws + w.bpart);
          rm.nbp = nbp;
          rm.inv_len = 1.0f / (float)C;
        }
        // larger square matrices: U's operand planes go to the second X plane
        // set, which the first Newton-Schulz step reads
        bf16_t* up = D == Dh && !ns_small(p) ? reinterpret_cast<bf16_t*>(ws + w.xp1) : nullptr;
        const int64_t ups = (int64_t)n * 3 * DD;
        const dim3 rg((unsigned)((rows + 3) / 4));
        const float* part = reinterpret_cast<const float*>(ws + w.part);
        // (the square path keeps U as planes only)
        float* Uf = up ? nullptr : U;
        if (!up) LACT_LAUNCH(reduce_rows_kernel<0>, rg, dim3(NT), s, part, ups, S, Uf, rowsq, rows, D, Dh, rm, up, ups);
        else if (PT::PREC == 1) LACT_LAUNCH(reduce_rows_kernel<1>, rg, dim3(NT), s, part, ups, S, Uf, rowsq, rows, D, Dh, rm, up, ups);
        else if (PT::PREC == 2) LACT_LAUNCH(reduce_rows_kernel<2>, rg, dim3(NT), s, part, ups, S, Uf, rowsq, rows, D, Dh, rm, up, ups);
        else LACT_LAUNCH(reduce_rows_kernel<3>, rg, dim3(NT), s, part, ups, S, Uf, rowsq, rows, D, Dh, rm, up, ups);
        HIP_TRY(hipGetLastError());
      }
      float* Am = reinterpret_cast<float*>(ws + w.am);
      float* Bm = reinterpret_cast<float*>(ws + w.bm);
      float* X[2] = {reinterpret_cast<float*>(ws + w.xa), reinterpret_cast<float*>(ws + w.xb)};
      const float ca = 3.4445f, cb = -4.7750f, cc = 2.0315f;
      const float* Xin = U;
      if (ns_small(p)) {
        // one workgroup per matrix, the whole orthogonalisation in its LDS;
        // the applies whose snapshots exist go beside it (it occupies 3n CUs)
        size_t ready = 0;
        for (size_t sj = 0; sj <= si; ++sj)
          if (step_group[sj] >= 0) ready = (size_t)step_group[sj] + 1;
        if (lact_status r = apply_upto(ready)) return r;
        KernelTimer kt(LACT_K_NS, s);
        if (D == 64) LACT_LAUNCH((ns_small_kernel<64, PT::PREC>), dim3((unsigned)(3 * n)), dim3(NsSmall<64>::THREADS), s, U, rowsq, X[0], p.ns_iters, ca, cb, cc);
        else LACT_LAUNCH((ns_small_kernel<128, PT::PREC>), dim3((unsigned)(3 * n)), dim3(NsSmall<128>::THREADS), s, U, rowsq, X[0], p.ns_iters, ca, cb, cc);
        HIP_TRY(hipGetLastError());
        Xin = X[0];
      } else if (D == Dh) {
        // every matrix square: one batch of 3n, every product on operands
        // stored as bf16 planes by the product (or the row reduction) before.
        // The batch is cut in two halves that run on two streams: each
        // half's chain of fifteen dependent launches leaves the chip idle
        // between launches, which the other half fills.
        constexpr int PN = PT::PREC;
        const int nb = 3 * n;
        const int64_t ps = (int64_t)nb * DD;   // plane stride
        auto ns_range = [&](int b0, int nbh, hipStream_t st) -> lact_status {
          bf16_t* Xp[2] = {reinterpret_cast<bf16_t*>(ws + w.xp0) + b0 * DD, reinterpret_cast<bf16_t*>(ws + w.xp1) + b0 * DD};
          bf16_t* Ap = reinterpret_cast<bf16_t*>(ws + w.ap) + b0 * DD;
          bf16_t* Bp = reinterpret_cast<bf16_t*>(ws + w.bp) + b0 * DD;
          const bf16_t* Xpin = Xp[1];   // U's planes
          const float* rq = rowsq + (int64_t)b0 * D;
          for (int it = 0; it < p.ns_iters; ++it) {
            const bool first = it == 0, last = it + 1 == p.ns_iters;
            float* Xout = X[it & 1] + b0 * DD;
            bf16_t* Xpout = Xp[it & 1];
            GemmArgs g = gemm_args();
            g.lda = g.ldb = g.ldc = g.ldcin = D;
            g.a_bs = g.b_bs = g.c_bs = g.cin_bs = DD;
            g.a_ps = g.b_ps = g.cp_ps = ps;
            g.g[0].M = D;
            g.N = D;
            g.K = g.kps = D;
            g.batch = nbh;
            // A = X X^T (X = s U on the first step, s = 1 / (||U||_F + 1e-7)
            // from the row sums of squares); A and B are symmetric, so only
            // their upper-triangle tiles run, each also storing its mirror.
            // Every intermediate is kept as planes only (the b A and a X terms
            // read them back: exact in three planes, 16-bit significands in two,
            // the precision of the products' operands)
            g.sym = D > PgSmall::BM;
            g.g[0].A = Xpin;
            g.g[0].B = Xpin;
            g.g[0].Cp = Ap;
            if (first) {
              g.g[0].rowsq = rq;
              g.rowsq_bs = D;
              g.rowsq_n = D;
              g.alpha_pow = 2;
            }
            lact_status r = launch_pgemm<PN>(g, false, LACT_K_NS, st);
            if (r) return r;
            // B = b A + c A A   (A is symmetric: A A = A A^T); only its planes are needed
            g.g[0].rowsq = nullptr;
            g.alpha_pow = 0;
            g.g[0].A = Ap;
            g.g[0].B = Ap;
            g.g[0].Cp = Bp;
            g.g[0].Cinp = Ap;
            g.alpha = cc;
            g.beta = cb;
            r = launch_pgemm<PN>(g, false, LACT_K_NS, st);
            if (r) return r;
            // X' = a X + B X  (element (n = j, k) of the second operand is X[k, j]:
            // column-k); the last step's result is read by the optimiser in fp32
            g.sym = 0;
            g.g[0].A = Bp;
            g.g[0].B = Xpin;
            g.g[0].C = last ? Xout : nullptr;
            g.g[0].Cp = last ? nullptr : Xpout;
            g.g[0].Cinp = Xpin;
            g.alpha = 1.f;
            g.beta = ca;
            if (first) {
              g.g[0].rowsq = rq;
              g.alpha_pow = 1;
              g.beta_pow = 1;
            }
            r = launch_pgemm<PN>(g, true, LACT_K_NS, st);
            if (r) return r;
            Xpin = Xpout;
          }
          return LACT_OK;
        };
        const int nb0 = (nb + 1) / 2;
        if (lact_status r = stream_after(aux->ns, s, aux->fork)) return r;
        // the applies of the groups of steps up to this one (their snapshots
        // and gated hidden rows exist now) run beside the Newton-Schulz chain,
        // which leaves the chip partly idle between its launches
        size_t ready = 0;
        for (size_t sj = 0; sj <= si; ++sj)
          if (step_group[sj] >= 0) ready = (size_t)step_group[sj] + 1;
        if (lact_status r = apply_upto(ready)) return r;
        if (lact_status r = ns_range(0, nb0, s)) return r;
        if (nb > nb0)
          if (lact_status r = ns_range(nb0, nb - nb0, aux->ns)) return r;
        if (lact_status r = stream_after(s, aux->ns, aux->join)) return r;
        Xin = X[(p.ns_iters - 1) & 1];
        (void)Am;
      } else {
        // W1, W3 are [dh, d] and W2 is [d, dh]: every Gram matrix is the
        // smaller side, r = min(d, dh), so one group uses X X^T and
        // X' = a X + B X, the other X^T X and X' = a X + X B (the same map:
        // NS(X^T) = NS(X)^T).  Matrices sit at their offsets in each
        // instance's [U1 | U3 | U2] block; the Gram matrices at the same
        // offsets of Am, Bm.
        const int rr = std::min(D, Dh);
        struct NsPart {
          int nmat;
          int64_t off[2];
          int rows, cols;
          int rq_off[2];
        };
        const NsPart parts[2] = {{2, {0, DD}, Dh, D, {0, Dh}}, {1, {2 * DD, 0}, D, Dh, {2 * Dh, 0}}};
        const int64_t IB = 3 * DD;   // instance stride of the stacked blocks
        for (int it = 0; it < p.ns_iters; ++it) {
          const bool first = it == 0;
          float* Xout = X[it & 1];
          for (const NsPart& pt : parts) {
            const bool xxT = pt.rows <= pt.cols;   // Gram on the rows side
            const int64_t w128 = (int64_t)((rr + 127) / 128) * ((rr + 127) / 128) * n * pt.nmat;
            const int tile = gemm_tile(w128);
            GemmArgs g = gemm_args();
            g.ngroups = pt.nmat;
            g.a_bs = g.b_bs = g.c_bs = g.cin_bs = IB;
            g.batch = n;
            g.sym = rr >= 256;   // the Gram matrix and b A + c A A are symmetric
            // Gram: X X^T (rows-k reads of X) or X^T X (column-k reads of X)
            for (int i = 0; i < pt.nmat; ++i) {
              g.g[i].A = Xin + pt.off[i];
              g.g[i].B = Xin + pt.off[i];
              g.g[i].C = Am + pt.off[i];
              g.g[i].M = rr;
              if (first) g.g[i].rowsq = rowsq + pt.rq_off[i];
            }
            g.lda = g.ldb = pt.cols;
            g.ldc = rr;
            g.N = rr;
            g.K = g.kps = xxT ? pt.cols : pt.rows;
            if (first) {
              g.rowsq_bs = 2 * Dh + D;
              g.rowsq_n = pt.rows;
              g.alpha_pow = 2;
            }
            lact_status r = xxT ? launch_gemm<float, PT::PREC, false, float, PT::PREC, false, float>(g, tile, LACT_K_NS, s)
                                : launch_gemm<float, PT::PREC, true, float, PT::PREC, true, float>(g, tile, LACT_K_NS, s);
            if (r) return r;
            // B = b A + c A A   (A symmetric)
            for (int i = 0; i < pt.nmat; ++i) {
              g.g[i].A = Am + pt.off[i];
              g.g[i].B = Am + pt.off[i];
              g.g[i].C = Bm + pt.off[i];
              g.g[i].Cin = Am + pt.off[i];
              g.g[i].rowsq = nullptr;
            }
            g.alpha_pow = g.beta_pow = 0;
            g.lda = g.ldb = g.ldc = g.ldcin = rr;
            g.N = rr;
            g.K = g.kps = rr;
            g.alpha = cc;
            g.beta = cb;
            r = launch_gemm<float, PT::PREC, false, float, PT::PREC, false, float>(g, tile, LACT_K_NS, s);
            if (r) return r;
            // X' = a X + B X (rows side) or a X + X B (columns side)
            g.sym = 0;
            for (int i = 0; i < pt.nmat; ++i) {
              g.g[i].A = xxT ? Bm + pt.off[i] : Xin + pt.off[i];
              g.g[i].B = xxT ? Xin + pt.off[i] : Bm + pt.off[i];
              g.g[i].C = Xout + pt.off[i];
              g.g[i].Cin = Xin + pt.off[i];
              g.g[i].M = pt.rows;
              if (first) g.g[i].rowsq = rowsq + pt.rq_off[i];
            }
            g.lda = xxT ? rr : pt.cols;
            g.ldb = xxT ? pt.cols : rr;   // rows side: element (n = j, k) = X[k, j]; else B[n, k] = B[k, n]
            g.ldc = g.ldcin = pt.cols;
            g.N = pt.cols;
            g.K = g.kps = rr;
            g.alpha = 1.f;
            g.beta = ca;
            if (first) {
              g.alpha_pow = 1;
              g.beta_pow = 1;
            }
            r = xxT ? launch_gemm<float, PT::PREC, false, float, PT::PREC, true, float>(g, tile, LACT_K_NS, s)
                    : launch_gemm<float, PT::PREC, false, float, PT::PREC, false, float>(g, tile, LACT_K_NS, s);
            if (r) return r;
          }
          Xin = Xout;
        }
      }
      oa.src = Xin;
      oa.src_ss = 0;
      oa.splits = 1;
    }
    // one launch when the three matrices share their shape, else W1 and W3
    // (dh rows of d) and W2 (d rows of dh) separately
    const int nparts = D == Dh ? 1 : 2;
    for (int part = 0; part < nparts; ++part) {
      KernelTimer kt(LACT_K_OPT, s);
      oa.mat0 = part == 0 ? 0 : 2;
      oa.nmat = nparts == 1 ? 3 : part == 0 ? 2 : 1;
      oa.R = part == 0 ? Dh : D;
      oa.L = part == 0 ? D : Dh;
      oa.rpw = opt_rpw(oa.L);
      const dim3 og((unsigned)(n * oa.nmat * (oa.R / (4 * oa.rpw))));
      const int vpl = (oa.rpw * oa.L + 255) / 256;
      if (part16 && !fused) {
        if (vpl == 1) LACT_LAUNCH((opt_kernel<TS, 1, bf16_t>), og, dim3(NT), s, oa);
        else if (vpl == 2) LACT_LAUNCH((opt_kernel<TS, 2, bf16_t>), og, dim3(NT), s, oa);
        else if (vpl == 3) LACT_LAUNCH((opt_kernel<TS, 3, bf16_t>), og, dim3(NT), s, oa);
        else LACT_LAUNCH((opt_kernel<TS, 4, bf16_t>), og, dim3(NT), s, oa);
      } else {
        if (vpl == 1) LACT_LAUNCH((opt_kernel<TS, 1, float, SP>), og, dim3(NT), s, oa);
        else if (vpl == 2) LACT_LAUNCH((opt_kernel<TS, 2, float, SP>), og, dim3(NT), s, oa);
        else if (vpl == 3) LACT_LAUNCH((opt_kernel<TS, 3, float, SP>), og, dim3(NT), s, oa);
        else LACT_LAUNCH((opt_kernel<TS, 4, float, SP>), og, dim3(NT), s, oa);
      }
      HIP_TRY(hipGetLastError());
    }
    ++nu;
  }

  // ---------------------------------------------------------------- apply
  // the rest: on the caller's stream when no apply went beside the
  // recurrence (without Newton-Schulz there is no idle phase to fill, and
  // the grouped launches are larger), else after the others on the apply stream
  TraceRange tr_apply("lact apply (all chunks)");
  if (!launched_app) return apply_groups(0, groups.size(), s);
  if (lact_status r = apply_upto(groups.size())) return r;
  // the caller's stream completes after the applies
  return stream_after(s, aux->app, aux->done);
}

lact_status dispatch(const lact_problem& p, const Ptrs& P, int64_t seq_stride, const Plan& plan, const Ws& w,
                     hipStream_t s) {
  switch (profile_of(p)) {
    case PF32: return run_steps<ProfF32>(p, P, seq_stride, plan, w, s);
    case PBF16: return run_steps<ProfBF16>(p, P, seq_stride, plan, w, s);
    case PBF16X2: return run_steps<ProfBF16X2>(p, P, seq_stride, plan, w, s);
    default: return run_steps<ProfBF16X3>(p, P, seq_stride, plan, w, s);
  }
}

#include "lact_backward_host.hpp"

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* lact_status_str(lact_status s) {
  switch (s) {
    case LACT_OK: return "ok";
    case LACT_ERR_INVALID_ARG: return "invalid argument";
    case LACT_ERR_UNSUPPORTED: return "unsupported";
    case LACT_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LACT_ERR_NO_DEVICE: return "no device";
    case LACT_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* lact_last_error(void) { return g_err.c_str(); }

size_t lact_workspace_size(const lact_problem* p, int64_t L, int64_t chunk, int32_t order, const int64_t* bounds,
                           const uint8_t* flags, int32_t n_chunks) {
  if (validate_problem(p) != LACT_OK) return 0;
  std::vector<int64_t> b;
  std::vector<uint8_t> f;
  if (make_schedule(L, chunk, order, bounds, flags, n_chunks, b, f) != LACT_OK) return 0;
  Plan plan;
  build_plan(order, b, f, plan);
  return std::max<size_t>(layout(*p, plan).total, 256);
}

}  // extern "C"

namespace {
// ------------------------------------------------------------- allocation-free entry point
// Device scratch of lact_layer_forward_noalloc, for callers that cannot
// allocate (HIP graph capture, serving loops): one copy per device, created
// when the library's code object is loaded on that device and held until
// the process ends.  Host code never uses the array's name as an address (it
// is a host-side stand-in): the device address is taken once per device with
// hipGetSymbolAddress, with that device current, and only it is passed on.
static __device__ __align__(256) char scratch[LACT_NOALLOC_SCRATCH_BYTES];

lact_status scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;   // per device
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(LACT_ERR_NO_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> g(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || a == nullptr)
      return fail(LACT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
    addr[dev] = a;
  }
  *out = addr[dev];
  return LACT_OK;
}

// ws == nullptr with use_scratch: the workspace is the device's scratch array
lact_status layer_forward_impl(const lact_problem* p, const void* q, const void* k, const void* v, const float* lr,
                               const float* beta, const float* oz, bool scaled, int64_t L, int64_t chunk,
                               int32_t order, const int64_t* bounds, const uint8_t* flags, int32_t n_chunks,
                               float* W1, float* W2, float* W3, float* M1, float* M2, float* M3, void* o, void* ws,
                               size_t ws_bytes, void* stream, bool use_scratch = false) {
  g_err.clear();
  lact_status r = validate_problem(p);
  if (r) return r;
  std::vector<int64_t> b;
  std::vector<uint8_t> f;
  r = make_schedule(L, chunk, order, bounds, flags, n_chunks, b, f);
  if (r) return r;
  Plan plan;
  build_plan(order, b, f, plan);
  if (p->n_inst == 0 || plan.steps.empty()) return LACT_OK;
  bool any_upd = plan.max_upd > 0, any_app = plan.max_app > 0;
  NEED(W1, 16);
  NEED(W2, 16);
  NEED(W3, 16);
  if (any_app) {
    NEED(q, 16);
    NEED(o, 16);
    if (scaled) NEED(oz, 4);
  }
  if (any_upd) {
    NEED(k, 16);
    NEED(v, 16);
    NEED(lr, 4);
    if (uses_momentum(p->opt)) {
      NEED(beta, 4);
      NEED(M1, 16);
      NEED(M2, 16);
      NEED(M3, 16);
    }
  }
  Ws w = layout(*p, plan);
  if (use_scratch) {
    if (w.total > LACT_NOALLOC_SCRATCH_BYTES)
      return fail(LACT_ERR_WORKSPACE_TOO_SMALL, "the problem needs %zu bytes of workspace; the allocation-free "
                  "entry point has %zu (LACT_NOALLOC_SCRATCH_BYTES)", w.total, (size_t)LACT_NOALLOC_SCRATCH_BYTES);
  } else {
    if (w.total > 0) NEED(ws, 256);
    if (ws_bytes < w.total)
      return fail(LACT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  }
  r = check_device();
  if (r) return r;
  if (use_scratch) {
    r = scratch_address(&ws);
    if (r) return r;
  }
  Ptrs P;
  P.q = q;
  P.k = k;
  P.v = v;
  P.lr = lr;
  P.beta = beta;
  P.W1 = W1;
  P.W2 = W2;
  P.W3 = W3;
  P.M1 = M1;
  P.M2 = M2;
  P.M3 = M3;
  P.o = o;
  P.oz = any_app ? oz : nullptr;
  P.ws = static_cast<char*>(ws);
  return dispatch(*p, P, L, plan, w, static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" {

lact_status lact_layer_forward(const lact_problem* p, const void* q, const void* k, const void* v, const float* lr,
                               const float* beta, int64_t L, int64_t chunk, int32_t order, const int64_t* bounds,
                               const uint8_t* flags, int32_t n_chunks, float* W1, float* W2, float* W3, float* M1,
                               float* M2, float* M3, void* o, void* ws, size_t ws_bytes, void* stream) {
  return layer_forward_impl(p, q, k, v, lr, beta, nullptr, false, L, chunk, order, bounds, flags, n_chunks, W1, W2,
                            W3, M1, M2, M3, o, ws, ws_bytes, stream);
}

lact_status lact_layer_forward_scaled(const lact_problem* p, const void* q, const void* k, const void* v,
                                      const float* lr, const float* beta, const float* oz, int64_t L, int64_t chunk,
                                      int32_t order, const int64_t* bounds, const uint8_t* flags, int32_t n_chunks,
                                      float* W1, float* W2, float* W3, float* M1, float* M2, float* M3, void* o,
                                      void* ws, size_t ws_bytes, void* stream) {
  return layer_forward_impl(p, q, k, v, lr, beta, oz, true, L, chunk, order, bounds, flags, n_chunks, W1, W2, W3, M1,
                            M2, M3, o, ws, ws_bytes, stream);
}

lact_status lact_layer_forward_noalloc(const lact_problem* p, const void* q, const void* k, const void* v,
                                       const float* lr, const float* beta, int64_t L, int64_t chunk, int32_t order,
                                       const int64_t* bounds, const uint8_t* flags, int32_t n_chunks, float* W1,
                                       float* W2, float* W3, float* M1, float* M2, float* M3, void* o, void* stream) {
  return layer_forward_impl(p, q, k, v, lr, beta, nullptr, false, L, chunk, order, bounds, flags, n_chunks, W1, W2,
                            W3, M1, M2, M3, o, nullptr, 0, stream, true);
}

lact_status lact_chunk_update(const lact_problem* p, const void* k, const void* v, const float* lr, const float* beta,
                              int64_t Lc, int64_t seq_stride, float* W1, float* W2, float* W3, float* M1, float* M2,
                              float* M3, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  lact_status r = validate_problem(p);
  if (r) return r;
  if (Lc < 0) return fail(LACT_ERR_INVALID_ARG, "Lc = %lld < 0", (long long)Lc);
  if (seq_stride < Lc) return fail(LACT_ERR_INVALID_ARG, "seq_stride < Lc");
  if (Lc == 0 || p->n_inst == 0) return LACT_OK;
  Plan plan;
  Step st;
  st.upd_t0 = 0;
  st.upd_len = Lc;
  plan.steps.push_back(st);
  plan.max_upd = Lc;
  NEED(W1, 16);
  NEED(W2, 16);
  NEED(W3, 16);
  NEED(k, 16);
  NEED(v, 16);
  NEED(lr, 4);
  if (uses_momentum(p->opt)) {
    NEED(beta, 4);
    NEED(M1, 16);
    NEED(M2, 16);
    NEED(M3, 16);
  }
  Ws w = layout(*p, plan);
  NEED(ws, 256);
  if (ws_bytes < w.total)
    return fail(LACT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  r = check_device();
  if (r) return r;
  Ptrs P;
  P.k = k;
  P.v = v;
  P.lr = lr;
  P.beta = beta;
  P.W1 = W1;
  P.W2 = W2;
  P.W3 = W3;
  P.M1 = M1;
  P.M2 = M2;
  P.M3 = M3;
  P.ws = static_cast<char*>(ws);
  return dispatch(*p, P, seq_stride, plan, w, static_cast<hipStream_t>(stream));
}

lact_status lact_apply(const lact_problem* p, const void* q, int64_t Lq, int64_t seq_stride, const float* W1,
                       const float* W2, const float* W3, void* o, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  lact_status r = validate_problem(p);
  if (r) return r;
  if (Lq < 0) return fail(LACT_ERR_INVALID_ARG, "Lq = %lld < 0", (long long)Lq);
  if (seq_stride < Lq) return fail(LACT_ERR_INVALID_ARG, "seq_stride < Lq");
  if (Lq == 0 || p->n_inst == 0) return LACT_OK;
  Plan plan;
  Step st;
  st.app_t0 = 0;
  st.app_len = Lq;
  plan.steps.push_back(st);
  plan.max_app = Lq;
  NEED(W1, 16);
  NEED(W2, 16);
  NEED(W3, 16);
  NEED(q, 16);
  NEED(o, 16);
  Ws w = layout(*p, plan);
  NEED(ws, 256);
  if (ws_bytes < w.total)
    return fail(LACT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  r = check_device();
  if (r) return r;
  Ptrs P;
  P.q = q;
  P.W1 = const_cast<float*>(W1);
  P.W2 = const_cast<float*>(W2);
  P.W3 = const_cast<float*>(W3);
  P.o = o;
  P.ws = static_cast<char*>(ws);
  return dispatch(*p, P, seq_stride, plan, w, static_cast<hipStream_t>(stream));
}

size_t lact_backward_workspace_size(const lact_problem* p, int64_t L, int64_t chunk, int32_t order,
                                    const int64_t* bounds, const uint8_t* flags, int32_t n_chunks) {
  g_err.clear();
  if (validate_problem(p) != LACT_OK) return 0;
  std::vector<int64_t> b;
  std::vector<uint8_t> f;
  if (make_schedule(L, chunk, order, bounds, flags, n_chunks, b, f) != LACT_OK) return 0;
  return std::max<size_t>(bwd_layout(*p, b, f).total, 256);
}

lact_status lact_layer_backward(const lact_problem* p, const void* q, const void* k, const void* v, const float* lr,
                                const float* beta, const float* oz, int64_t L, int64_t chunk, int32_t order,
                                const int64_t* bounds,
                                const uint8_t* flags, int32_t n_chunks, const float* W1, const float* W2,
                                const float* W3, const float* M1, const float* M2, const float* M3, const void* dO,
                                const float* gW1, const float* gW2, const float* gW3, const float* gM1,
                                const float* gM2, const float* gM3, float* dq, float* dk, float* dv, float* dlr,
                                float* dbeta, float* doz, float* dW1, float* dW2, float* dW3, float* dM1, float* dM2,
                                float* dM3, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  lact_status r = validate_problem(p);
  if (r) return r;
  std::vector<int64_t> b;
  std::vector<uint8_t> f;
  r = make_schedule(L, chunk, order, bounds, flags, n_chunks, b, f);
  if (r) return r;
  if (p->n_inst == 0) return LACT_OK;
  bool any_upd = false, any_app = false;
  for (uint8_t x : f) {
    any_upd |= (x & LACT_CHUNK_UPDATE) != 0;
    any_app |= (x & LACT_CHUNK_APPLY) != 0;
  }
  const bool mom = uses_momentum(p->opt);
  NEED(W1, 16);
  NEED(W2, 16);
  NEED(W3, 16);
  NEED(dW1, 16);
  NEED(dW2, 16);
  NEED(dW3, 16);
  if (L > 0) {
    NEED(dq, 16);
    NEED(dk, 16);
    NEED(dv, 16);
    NEED(dlr, 4);
  }
  if (any_app) {
    NEED(q, 16);
    NEED(dO, 16);
    if (oz) NEED(doz, 4);
  }
  if (any_upd) {
    NEED(k, 16);
    NEED(v, 16);
    NEED(lr, 4);
  }
  if (mom) {
    NEED(M1, 16);
    NEED(M2, 16);
    NEED(M3, 16);
    if (any_upd) {
      NEED(beta, 4);
      NEED(dbeta, 4);
    }
  }
  if (!aligned(oz, 4)) return fail(LACT_ERR_INVALID_ARG, "oz is not 4-byte aligned");
  for (const void* g : {(const void*)gW1, (const void*)gW2, (const void*)gW3, (const void*)gM1, (const void*)gM2,
                        (const void*)gM3, (const void*)dM1, (const void*)dM2, (const void*)dM3, (const void*)dbeta})
    if (g && !aligned(g, 4)) return fail(LACT_ERR_INVALID_ARG, "misaligned optional pointer");
  if (!aligned(gW1, 16) || !aligned(gW2, 16) || !aligned(gW3, 16) || !aligned(gM1, 16) || !aligned(gM2, 16) ||
      !aligned(gM3, 16))
    return fail(LACT_ERR_INVALID_ARG, "state cotangents must be 16-byte aligned");
  const BwdWs w = bwd_layout(*p, b, f);
  NEED(ws, 256);
  if (ws_bytes < w.total)
    return fail(LACT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  r = check_device();
  if (r) return r;
  BwdPtrs P;
  P.q = any_app ? q : nullptr;
  P.k = any_upd ? k : nullptr;
  P.v = any_upd ? v : nullptr;
  P.dO = dO;
  P.lr = lr;
  P.beta = beta;
  P.oz = any_app ? oz : nullptr;
  P.doz = any_app && oz ? doz : nullptr;
  const float* Ws[3] = {W1, W2, W3};
  const float* Ms[3] = {M1, M2, M3};
  const float* gWs[3] = {gW1, gW2, gW3};
  const float* gMs[3] = {gM1, gM2, gM3};
  float* dWs[3] = {dW1, dW2, dW3};
  float* dMs[3] = {dM1, dM2, dM3};
  for (int j = 0; j < 3; ++j) {
    P.W[j] = Ws[j];
    P.M[j] = mom ? Ms[j] : nullptr;
    P.gW[j] = gWs[j];
    P.gM[j] = gMs[j];
    P.dW[j] = dWs[j];
    P.dM[j] = dMs[j];
  }
  P.dq = dq;
  P.dk = dk;
  P.dv = dv;
  P.dlr = dlr;
  P.dbeta = dbeta;
  P.ws = static_cast<char*>(ws);
  return run_backward(*p, P, L, order, b, f, w, static_cast<hipStream_t>(stream));
}

lact_status lact_timing_enable(int32_t kclass, int32_t on) {
  if (kclass < 0 || kclass >= LACT_K_COUNT) return fail(LACT_ERR_INVALID_ARG, "kernel class %d", kclass);
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.on[kclass] = on != 0;
  return LACT_OK;
}

lact_status lact_timing_read(int32_t kclass, double* total_ms, int64_t* launches) {
  if (kclass < 0 || kclass >= LACT_K_COUNT) return fail(LACT_ERR_INVALID_ARG, "kernel class %d", kclass);
  if (!total_ms || !launches) return fail(LACT_ERR_INVALID_ARG, "NULL output");
  TimingState& t = timing();
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  {
    std::lock_guard<std::mutex> g(t.mu);
    ev.swap(t.ev[kclass]);
  }
  double tot = 0;
  lact_status st = LACT_OK;
  for (auto& e : ev) {
    float ms = 0;
    if (hipEventSynchronize(e.second) != hipSuccess || hipEventElapsedTime(&ms, e.first, e.second) != hipSuccess)
      st = fail(LACT_ERR_HIP, "event timing failed");
    tot += ms;
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  *total_ms = tot;
  *launches = (int64_t)ev.size();
  return st;
}

}  // extern "C"
