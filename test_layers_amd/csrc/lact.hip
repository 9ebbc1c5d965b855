// liblact: host side of the gfx950 LaCT fast-weight layer.
//
// Validation (before any HIP call), chunk planning, workspace layout,
// precision dispatch and kernel launches for the C ABI in include/lact.h.
// All device work is asynchronous on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "lact.h"
#include "lact_kernels.hpp"

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

struct KernelTimer {
  hipEvent_t a = nullptr, b = nullptr;
  hipStream_t s;
  int kc;
  KernelTimer(int kclass, hipStream_t st) : s(st), kc(kclass) {
    TimingState& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on[kc]) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      a = b = nullptr;
      return;
    }
    (void)hipEventRecord(a, s);
  }
  ~KernelTimer() {
    if (!a) return;
    (void)hipEventRecord(b, s);
    TimingState& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.ev[kc].push_back({a, b});
  }
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

Prof profile_of(const lact_problem& p) {
  if (p.io_dtype == LACT_DTYPE_F32) return PF32;
  int rp = p.rec_planes == 0 ? 1 : p.rec_planes;
  return rp == 1 ? PBF16 : rp == 2 ? PBF16X2 : PBF16X3;
}
size_t io_size(const lact_problem& p) { return p.io_dtype == LACT_DTYPE_F32 ? 4 : 2; }
size_t rec_size(Prof f) { return f == PBF16 ? 2 : 4; }   // update terms storage
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
int gemm_tile(int64_t wgs128) { return wgs128 >= 200 ? 128 : 64; }

int dw_tile(const lact_problem& p) { return p.d >= 128 ? 128 : 64; }

// split of the chunk's tokens for the weight-gradient contraction
void dw_split(const lact_problem& p, int64_t C, int& S, int64_t& kps) {
  const int bt = dw_tile(p);
  const int64_t tiles = (int64_t)(3 * p.d / bt) * (p.d / bt) * std::max(1, p.n_inst);
  int64_t s = (512 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, C / 256));
  s = std::max<int64_t>(1, std::min<int64_t>(s, 64));
  kps = ((C + s - 1) / s + BK - 1) / BK * BK;
  if (kps <= 0) kps = BK;
  S = (int)((C + kps - 1) / kps);
  if (S < 1) S = 1;
}

// --------------------------------------------------------------- workspace layout
struct Ws {
  size_t e = 0, h = 0, part = 0, u = 0, am = 0, bm = 0, xa = 0, xb = 0, rowsq = 0, total = 0;
  int S = 1;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Ws layout(const lact_problem& p, const Plan& plan) {
  Ws w;
  const Prof f = profile_of(p);
  const size_t n = (size_t)std::max(0, p.n_inst), D = (size_t)p.d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  // the token split count is not monotone in the chunk length (rounding of
  // the split size), so size the partials for the largest count of any step
  int S = 1;
  for (const Step& st : plan.steps) {
    if (st.upd_len == 0) continue;
    int s_ = 1;
    int64_t kps = 0;
    dw_split(p, st.upd_len, s_, kps);
    S = std::max(S, s_);
  }
  w.S = S;
  w.e = take(n * (size_t)plan.max_upd * 3 * D * rec_size(f));
  w.h = take(n * (size_t)plan.max_app * D * app_size(f));
  const size_t mats = n * 3 * D * D * sizeof(float);
  w.part = take(plan.max_upd > 0 ? (size_t)S * mats : 0);
  if (p.opt == LACT_OPT_MUON && plan.max_upd > 0) {
    w.u = take(mats);
    w.am = take(mats);
    w.bm = take(mats);
    w.xa = take(mats);
    w.xb = take(mats);
    w.rowsq = take(n * 3 * D * sizeof(float));
  }
  w.total = off;
  return w;
}

// --------------------------------------------------------------- validation
lact_status validate_problem(const lact_problem* p) {
  if (!p) return fail(LACT_ERR_INVALID_ARG, "problem is NULL");
  if (p->n_inst < 0) return fail(LACT_ERR_INVALID_ARG, "n_inst = %d < 0", p->n_inst);
  if (p->d != p->dh) return fail(LACT_ERR_UNSUPPORTED, "d = %d != dh = %d", p->d, p->dh);
  if (p->d < 64 || p->d > 1024 || p->d % 64 != 0)
    return fail(LACT_ERR_UNSUPPORTED, "d = %d: need a multiple of 64 in [64, 1024]", p->d);
  if (p->io_dtype != LACT_DTYPE_F32 && p->io_dtype != LACT_DTYPE_BF16)
    return fail(LACT_ERR_INVALID_ARG, "io_dtype = %d", p->io_dtype);
  if (p->opt < LACT_OPT_GD || p->opt > LACT_OPT_MUON) return fail(LACT_ERR_INVALID_ARG, "opt = %d", p->opt);
  if (p->opt == LACT_OPT_MUON && (p->ns_iters < 1 || p->ns_iters > 16))
    return fail(LACT_ERR_INVALID_ARG, "ns_iters = %d: need 1..16", p->ns_iters);
  if (p->rec_planes < 0 || p->rec_planes > 3) return fail(LACT_ERR_INVALID_ARG, "rec_planes = %d", p->rec_planes);
  if (p->flags & ~LACT_NO_RENORM) return fail(LACT_ERR_INVALID_ARG, "unknown flags 0x%x", p->flags);
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
  char* ws = nullptr;
};

template <typename TIO_, int PIO_, int PWU_, int PWA_, typename TREC_, int PREC_, typename TAPP_, int PAPP_>
struct ProfT {
  using TIO = TIO_;
  using TREC = TREC_;
  using TAPP = TAPP_;
  static constexpr int PIO = PIO_, PWU = PWU_, PWA = PWA_, PREC = PREC_, PAPP = PAPP_;
};
using ProfF32 = ProfT<float, 3, 3, 3, float, 3, float, 3>;
using ProfBF16 = ProfT<bf16_t, 1, 1, 1, bf16_t, 1, bf16_t, 1>;
using ProfBF16X2 = ProfT<bf16_t, 1, 2, 1, float, 2, bf16_t, 1>;
using ProfBF16X3 = ProfT<bf16_t, 1, 3, 1, float, 3, bf16_t, 1>;

template <typename TA, int PA, bool CA, typename TB, int PB, bool CB, typename TC>
lact_status launch_gemm(GemmArgs g, int tile, int kclass, hipStream_t s) {
  const int64_t tiles = (int64_t)((g.M + tile - 1) / tile) * ((g.N + tile - 1) / tile);
  const int64_t grid = tiles * g.batch * g.splits;
  if (grid <= 0) return LACT_OK;
  if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
  KernelTimer kt(kclass, s);
  if (tile == 128)
    hipLaunchKernelGGL((gemm_kernel<TA, PA, CA, TB, PB, CB, TC, 128, 128>), dim3((unsigned)grid), dim3(NT), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_kernel<TA, PA, CA, TB, PB, CB, TC, 64, 64>), dim3((unsigned)grid), dim3(NT), 0, s, g);
  HIP_TRY(hipGetLastError());
  return LACT_OK;
}

GemmArgs gemm_args() {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.splits = 1;
  g.alpha = 1.f;
  g.m_switch = 1 << 30;
  return g;
}

template <typename PT>
lact_status run_steps(const lact_problem& p, const Ptrs& P, int64_t seq_stride, const Plan& plan, const Ws& w,
                      hipStream_t s) {
  using TIO = typename PT::TIO;
  using TREC = typename PT::TREC;
  using TAPP = typename PT::TAPP;
  const int n = p.n_inst, D = p.d;
  if (n == 0) return LACT_OK;
  const int64_t DD = (int64_t)D * D;
  const int64_t x_bs = seq_stride * D;
  char* ws = P.ws;
  for (const Step& st : plan.steps) {
    // ---- forward tiles (apply hidden + update terms), all on the current weights
    FwdArgs fa;
    memset(&fa, 0, sizeof(fa));
    fa.q = P.q;
    fa.k = P.k;
    fa.v = P.v;
    fa.x_bs = x_bs;
    fa.lr = P.lr;
    fa.lr_bs = seq_stride * 3;
    fa.W1 = P.W1;
    fa.W2 = P.W2;
    fa.W3 = P.W3;
    fa.E = ws + w.e;
    fa.e_bs = st.upd_len * 3 * D;
    fa.H = ws + w.h;
    fa.h_bs = st.app_len * D;
    fa.D = D;
    fa.upd_t0 = st.upd_t0;
    fa.upd_len = st.upd_len;
    fa.app_t0 = st.app_t0;
    fa.app_len = st.app_len;
    fa.upd_tiles = (int)((st.upd_len + FBT - 1) / FBT) * (D / FBJ);
    fa.app_tiles = (int)((st.app_len + FBT - 1) / FBT) * (D / FBJ);
    const int64_t fgrid = (int64_t)n * (fa.upd_tiles + fa.app_tiles);
    if (fgrid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    if (fgrid > 0) {
      KernelTimer kt(LACT_K_FWD, s);
      hipLaunchKernelGGL((fwd_kernel<TIO, PT::PIO, PT::PWU, PT::PWA, TREC, TAPP>), dim3((unsigned)fgrid), dim3(NT), 0,
                         s, fa);
      HIP_TRY(hipGetLastError());
    }
    // ---- apply output: o[t, r] = sum_j Hq[t, j] W2[r, j]
    if (st.app_len > 0) {
      GemmArgs g = gemm_args();
      g.A = ws + w.h;
      g.lda = D;
      g.a_bs = st.app_len * D;
      g.B = P.W2;
      g.ldb = D;
      g.b_bs = DD;
      g.C = static_cast<char*>(P.o) + (size_t)st.app_t0 * D * io_size(p);
      g.ldc = D;
      g.c_bs = x_bs;
      g.M = (int)st.app_len;
      g.N = D;
      g.K = D;
      g.kps = D;
      g.batch = n;
      const int64_t w128 = ((st.app_len + 127) / 128) * (D / 128 > 0 ? D / 128 : 1) * n;
      lact_status r = launch_gemm<TAPP, PT::PAPP, false, float, PT::PWA, false, TIO>(g, gemm_tile(w128), LACT_K_OUT, s);
      if (r) return r;
    }
    if (st.upd_len == 0) continue;
    // ---- weight-gradient contraction over the chunk's tokens (split over tokens)
    int S;
    int64_t kps;
    dw_split(p, st.upd_len, S, kps);
    if (S > w.S) return fail(LACT_ERR_UNSUPPORTED, "internal: token split %d exceeds workspace plan %d", S, w.S);
    {
      GemmArgs g = gemm_args();
      g.A = ws + w.e;              // (m, t) = E[t, m], m over [U1 | U3 | U2^T] rows
      g.lda = 3 * D;
      g.a_bs = st.upd_len * 3 * D;
      g.B = static_cast<const char*>(P.k) + (size_t)st.upd_t0 * D * io_size(p);
      g.B2 = static_cast<const char*>(P.v) + (size_t)st.upd_t0 * D * io_size(p);
      g.m_switch = 2 * D;
      g.ldb = D;
      g.b_bs = x_bs;
      g.C = ws + w.part;
      g.ldc = D;
      g.c_bs = 3 * DD;
      g.c_ss = (int64_t)n * 3 * DD;
      g.M = 3 * D;
      g.N = D;
      g.K = st.upd_len;
      g.kps = kps;
      g.batch = n;
      g.splits = S;
      lact_status r = launch_gemm<TREC, PT::PREC, true, TIO, PT::PIO, true, float>(g, dw_tile(p), LACT_K_DW, s);
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
    oa.D = D;
    oa.opt = p.opt;
    oa.renorm = (p.flags & LACT_NO_RENORM) ? 0 : 1;
    oa.beta = P.beta;
    oa.beta_bs = seq_stride;
    oa.beta_t0 = st.upd_t0;
    oa.beta_len = st.upd_len;
    if (p.opt != LACT_OPT_MUON) {
      oa.src = reinterpret_cast<const float*>(ws + w.part);
      oa.src_ss = (int64_t)n * 3 * DD;
      oa.splits = S;
    } else {
      // ---- Muon: U = sum of partials, then quintic Newton-Schulz on every matrix
      float* U = reinterpret_cast<float*>(ws + w.u);
      float* rowsq = reinterpret_cast<float*>(ws + w.rowsq);
      {
        KernelTimer kt(LACT_K_NS, s);
        const int64_t rows = (int64_t)n * 3 * D;
        hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(NT), 0, s,
                           reinterpret_cast<const float*>(ws + w.part), (int64_t)n * 3 * DD, S, U, rowsq, rows, D);
        HIP_TRY(hipGetLastError());
      }
      float* Am = reinterpret_cast<float*>(ws + w.am);
      float* Bm = reinterpret_cast<float*>(ws + w.bm);
      float* X[2] = {reinterpret_cast<float*>(ws + w.xa), reinterpret_cast<float*>(ws + w.xb)};
      const int nb = 3 * n;
      const int64_t w128 = (int64_t)((D + 127) / 128) * ((D + 127) / 128) * nb;
      const int tile = gemm_tile(w128);
      const float ca = 3.4445f, cb = -4.7750f, cc = 2.0315f;
      const float* Xin = U;
      for (int it = 0; it < p.ns_iters; ++it) {
        const bool first = it == 0;
        float* Xout = X[it & 1];
        GemmArgs g = gemm_args();
        g.lda = g.ldb = g.ldc = g.ldcin = D;
        g.a_bs = g.b_bs = g.c_bs = g.cin_bs = DD;
        g.M = g.N = D;
        g.K = g.kps = D;
        g.batch = nb;
        // A = X X^T (X = s U on the first step)
        g.A = Xin;
        g.B = Xin;
        g.C = Am;
        if (first) {
          g.rowsq = rowsq;
          g.rowsq_n = D;
          g.alpha_pow = 2;
        }
        lact_status r = launch_gemm<float, PT::PREC, false, float, PT::PREC, false, float>(g, tile, LACT_K_NS, s);
        if (r) return r;
        // B = b A + c A A   (A is symmetric: A A = A A^T)
        g.rowsq = nullptr;
        g.alpha_pow = 0;
        g.A = Am;
        g.B = Am;
        g.C = Bm;
        g.Cin = Am;
        g.alpha = cc;
        g.beta = cb;
        r = launch_gemm<float, PT::PREC, false, float, PT::PREC, false, float>(g, tile, LACT_K_NS, s);
        if (r) return r;
        // X' = a X + B X
        g.A = Bm;
        g.B = Xin;     // element (n = j, k) = X[k, j]: column-k source
        g.C = Xout;
        g.Cin = Xin;
        g.alpha = 1.f;
        g.beta = ca;
        if (first) {
          g.rowsq = rowsq;
          g.rowsq_n = D;
          g.alpha_pow = 1;
          g.beta_pow = 1;
        }
        r = launch_gemm<float, PT::PREC, false, float, PT::PREC, true, float>(g, tile, LACT_K_NS, s);
        if (r) return r;
        Xin = Xout;
      }
      oa.src = Xin;
      oa.src_ss = 0;
      oa.splits = 1;
    }
    {
      KernelTimer kt(LACT_K_OPT, s);
      const size_t lds = 0;
      hipLaunchKernelGGL(opt_kernel, dim3((unsigned)(n * 3 * (D / OPT_ROWS))), dim3(NT), lds, s, oa);
      HIP_TRY(hipGetLastError());
    }
  }
  return LACT_OK;
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

lact_status lact_layer_forward(const lact_problem* p, const void* q, const void* k, const void* v, const float* lr,
                               const float* beta, int64_t L, int64_t chunk, int32_t order, const int64_t* bounds,
                               const uint8_t* flags, int32_t n_chunks, float* W1, float* W2, float* W3, float* M1,
                               float* M2, float* M3, void* o, void* ws, size_t ws_bytes, void* stream) {
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
  }
  if (any_upd) {
    NEED(k, 16);
    NEED(v, 16);
    NEED(lr, 4);
    if (p->opt == LACT_OPT_MOMENTUM) {
      NEED(beta, 4);
      NEED(M1, 16);
      NEED(M2, 16);
      NEED(M3, 16);
    }
  }
  Ws w = layout(*p, plan);
  if (w.total > 0) NEED(ws, 256);
  if (ws_bytes < w.total)
    return fail(LACT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  r = check_device();
  if (r) return r;
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
  P.ws = static_cast<char*>(ws);
  return dispatch(*p, P, L, plan, w, static_cast<hipStream_t>(stream));
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
  if (p->opt == LACT_OPT_MOMENTUM) {
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
