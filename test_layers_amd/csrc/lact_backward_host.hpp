// Host side of the layer's backward pass: workspace layout, the replay of the
// forward state trajectory and the reverse sweep over the chunk schedule.
// Included by lact.hip inside its anonymous namespace, after the forward
// dispatch (it reuses the forward's validation, schedule, product launcher
// and chunk update).
//
// The reverse sweep follows the chain rule through the forward steps of
// "大块测试时训练（LaCT）技术解析" §2.1 (apply, eq. 2; update, eqs. 4-5) and
// §2.2.1 (renormalisation, eq. 8; Newton-Schulz, eqs. 9-10) and the momentum
// of "LaCT架构核心思想解析" §1.2, chunk by chunk from the last to the first:
//   apply chunk:   dq = dAq W1 + dBq W3;  dW1 += dAq^T q, dW3 += dBq^T q,
//                  dW2 += dO^T Hq   (Hq = silu(q W1^T) (q W3^T), dHq = dO W2)
//   update chunk:  renorm backward (per row), optimiser backward (momentum:
//                  linear; Muon: Newton-Schulz backward through the stored
//                  iterates), then the update terms' backward:
//                  gE1 = k gU1^T, gE3 = k gU3^T, gH2 = v gU2,
//                  dk = E1 gU1 + E3 gU3 + gA W1 + gB W3, dv = H2 gU2^T + gG W2^T,
//                  dW1 += gA^T k, dW3 += gB^T k, dW2 += v^T gG.
// Every product runs on the grouped GEMM with fp32 operands split into bf16
// planes (bf16 inputs are exact in one plane): three (fp32 grade) for the
// Newton-Schulz products and for every product of the Newton-Schulz
// optimisers, two (16-bit significands) for the others of GD and momentum.

// ----------------------------------------------------------------- products
// grid of a grid-stride elementwise kernel
inline unsigned ew_grid(int64_t total) {
  const int64_t b = (total + NT - 1) / NT;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 8 * NCU));
}

struct BOp {
  const void* p;
  int64_t ld, bs;
  bool colk;   // element (m, k) at p[k ld + m]; else at p[m ld + k]
  bool bf16;
  // an fp32 operand already split into bf16 planes: the planes of the
  // element at pl_base + e are at pl + e + q * pl_ps
  const bf16_t* pl = nullptr;
  const float* pl_base = nullptr;
  int64_t pl_ps = 0;
};
inline BOp bop(const void* p, int64_t ld, int64_t bs, bool colk, bool bf16 = false) {
  return BOp{p, ld, bs, colk, bf16};
}
inline BOp with_planes(BOp o, const bf16_t* pl, const float* base, int64_t ps) {
  o.pl = pl;
  o.pl_base = base;
  o.pl_ps = ps;
  return o;
}

template <typename TA, int PA, bool CA, typename TB, int PB, bool CB>
lact_status bgemm_t(GemmArgs& g, hipStream_t s) {
  const int64_t per = (int64_t)((g.N + 63) / 64) * g.batch * g.splits;
  int64_t t = 0;
  for (int i = 0; i < g.ngroups; ++i) {
    const int64_t ti = (int64_t)((g.g[i].M + 63) / 64) * per;
    if (ti > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    g.g[i].tiles = (int)ti;
    t += ti;
  }
  if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
  if (t == 0) return LACT_OK;
  KernelTimer kt(LACT_K_BWD_GEMM, s);
  return launch_gemm_t<TA, PA, CA, TB, PB, CB, float, 64>(g, t, s);
}

// bf16 planes per fp32 operand of a backward product: two (16-bit
// significands) or three (fp32 grade)
template <int PL>
lact_status bgemm_form(const BOp& A, const BOp& B, GemmArgs& g, hipStream_t s) {
  if (!A.bf16 && !B.bf16) {
    if (!A.colk && !B.colk) return bgemm_t<float, PL, false, float, PL, false>(g, s);
    if (!A.colk && B.colk) return bgemm_t<float, PL, false, float, PL, true>(g, s);
    if (A.colk && B.colk) return bgemm_t<float, PL, true, float, PL, true>(g, s);
  } else {
    if (A.bf16 && !B.bf16) {
      if (!A.colk && !B.colk) return bgemm_t<bf16_t, 1, false, float, PL, false>(g, s);
      if (!A.colk && B.colk) return bgemm_t<bf16_t, 1, false, float, PL, true>(g, s);
      if (A.colk && B.colk) return bgemm_t<bf16_t, 1, true, float, PL, true>(g, s);
    } else if (!A.bf16 && B.bf16) {
      if (A.colk && B.colk) return bgemm_t<float, PL, true, bf16_t, 1, true>(g, s);
    }
  }
  return fail(LACT_ERR_UNSUPPORTED, "internal: backward product form");
}

// Token split of a long contraction (K = a chunk's tokens) whose output has
// few 64 x 64 tiles: enough splits for about four workgroups per CU, at
// least 256 of K per split.
int bwd_splits(int64_t tiles, int64_t K) {
  if (K < 512 || tiles >= 4 * NCU) return 1;
  const int64_t want = (4 * NCU + tiles - 1) / tiles;
  return (int)std::max<int64_t>(1, std::min<int64_t>({64, want, K / 256}));
}

// Products with fp32 operands on the direct-load GEMM: each fp32 operand is
// split into PL bf16 planes once, in its own layout (bf16 inputs stay one
// exact plane), and the product sums the plane pairs in dgemm_kernel instead
// of splitting every tile's loads in registers (the register path).
// Scratch: `apl` holds the first operands' planes (ng x PA x batch x A.bs
// elements), `bpl` the second's.
inline lact_status bwd_split(const void* src, int64_t per, int64_t bs, int batch, int P, bf16_t* dst, int64_t ps,
                             hipStream_t s) {
  KernelTimer kt(LACT_K_BWD_ELEM, s);
  const dim3 grid(ew_grid((int64_t)batch * per / 4));
  if (P == 3) LACT_LAUNCH((bwd_planes_kernel<3>), grid, dim3(NT), s, static_cast<const float*>(src), per, bs, batch, dst, ps);
  else LACT_LAUNCH((bwd_planes_kernel<2>), grid, dim3(NT), s, static_cast<const float*>(src), per, bs, batch, dst, ps);
  HIP_TRY(hipGetLastError());
  return LACT_OK;
}

template <bool CA, bool CB, int PA, int PB>
lact_status bgemm_planes(GemmArgs& g, const BOp& A, const BOp& B, int64_t K, bf16_t* apl, bf16_t* bpl, hipStream_t s) {
  // the valid rows of each operand: k rows when read column-k, else its M (N) rows
  const int64_t a_ps = A.pl ? A.pl_ps : (int64_t)g.batch * A.bs, b_ps = B.pl ? B.pl_ps : (int64_t)g.batch * B.bs;
  for (int i = 0; i < g.ngroups; ++i) {
    if constexpr (PA > 1) {
      if (A.pl) {
        g.g[i].A = A.pl + (static_cast<const float*>(g.g[i].A) - A.pl_base);
      } else {
        bf16_t* dst = apl + (int64_t)i * PA * a_ps;
        const int64_t per = (CA ? K : (int64_t)g.g[i].M) * A.ld;
        if (lact_status r = bwd_split(g.g[i].A, per, A.bs, g.batch, PA, dst, a_ps, s)) return r;
        g.g[i].A = dst;
      }
    }
    if constexpr (PB > 1) {
      if (B.pl) {
        g.g[i].B = B.pl + (static_cast<const float*>(g.g[i].B) - B.pl_base);
      } else {
        bf16_t* dst = bpl + (int64_t)i * PB * b_ps;
        const int64_t per = (CB ? K : (int64_t)g.N) * B.ld;
        if (lact_status r = bwd_split(g.g[i].B, per, B.bs, g.batch, PB, dst, b_ps, s)) return r;
        g.g[i].B = dst;
      }
    }
  }
  g.a_ps = a_ps;
  g.b_ps = b_ps;
  int64_t grid = 0;
  for (int i = 0; i < g.ngroups; ++i) {
    const int64_t t = (int64_t)(g.g[i].M / 64) * (g.N / 64) * g.batch * g.splits;
    if (t > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
    g.g[i].tiles = (int)t;
    grid += t;
  }
  if (grid <= 0) return LACT_OK;
  if (grid > 0x7fffffff) return fail(LACT_ERR_UNSUPPORTED, "grid too large");
  KernelTimer kt(LACT_K_BWD_GEMM, s);
  constexpr int NST = PA + PB <= 3 ? 3 : 2;   // 64-wide stages: 24 KB (three planes) to 48 KB (six)
  LACT_LAUNCH((dgemm_kernel<CA, CB, float, 64, 64, NST, PA, PB>), dim3((unsigned)grid), dim3(DG_THREADS), s, g);
  HIP_TRY(hipGetLastError());
  return LACT_OK;
}

// the forms the backward's products take (layout of A and B, which are fp32)
template <int PL>
lact_status bgemm_planes_form(GemmArgs& g, const BOp& A, const BOp& B, int64_t K, bf16_t* apl, bf16_t* bpl,
                              hipStream_t s) {
  const bool fa = !A.bf16, fb = !B.bf16;
  if (fa && !fb && A.colk && B.colk) return bgemm_planes<true, true, PL, 1>(g, A, B, K, apl, bpl, s);
  if (!fa && fb && A.colk && B.colk) return bgemm_planes<true, true, 1, PL>(g, A, B, K, apl, bpl, s);
  if (!fa && fb && !A.colk && !B.colk) return bgemm_planes<false, false, 1, PL>(g, A, B, K, apl, bpl, s);
  if (!fa && fb && !A.colk && B.colk) return bgemm_planes<false, true, 1, PL>(g, A, B, K, apl, bpl, s);
  if (fa && fb && !A.colk && B.colk) return bgemm_planes<false, true, PL, PL>(g, A, B, K, apl, bpl, s);
  if (fa && fb && !A.colk && !B.colk) return bgemm_planes<false, false, PL, PL>(g, A, B, K, apl, bpl, s);
  return fail(LACT_ERR_UNSUPPORTED, "internal: backward plane product form");
}
inline bool bgemm_planes_has_form(const BOp& A, const BOp& B) {
  const bool fa = !A.bf16, fb = !B.bf16;
  return (fa && !fb && A.colk && B.colk) || (!fa && fb && A.colk && B.colk) || (!fa && fb && !A.colk && !B.colk) ||
         (!fa && fb && !A.colk && B.colk) || (fa && fb && !A.colk);
}

// one product of a group: its own A, B, C and accumulation source
struct BGrp {
  const void* A;
  const void* B;
  float* C;
  const float* Cin;
};

// For each group i < ng: C_i,b[m, n] = alpha sum_k A_i,b(m, k) B_i,b(n, k)
// + beta Cin_i,b[m, n] for b < batch (Cin has C's strides and may be C
// itself; NULL: no accumulation).  A and B give the operands' layout (their
// pointers are ignored).  Long contractions with few output tiles are split
// over K into fp32 partials in `spl` (spl_floats of scratch), summed in
// fixed order by bwd_splitsum_kernel.  With plane scratch `apl` (apl_elems
// bf16), the token contractions of bgemm_planes' form take that path.
lact_status bgemm_g(const BGrp* gs, int ng, const BOp& A, const BOp& B, int64_t ldc, int64_t c_bs, int M, int N,
                    int64_t K, int batch, float alpha, float beta, float* spl, size_t spl_floats, hipStream_t s,
                    bool fp32_grade = false, bf16_t* apl = nullptr, size_t apl_elems = 0) {
  if (M <= 0 || N <= 0 || batch <= 0 || ng <= 0) return LACT_OK;
  // fp32 operands not already split are split here: worth a launch only
  // for large ones (token buffers); small weight-shaped ones must come split
  const size_t PL = fp32_grade ? 3 : 2;
  const size_t need_a = (A.bf16 || A.pl) ? 0 : (size_t)ng * PL * (size_t)batch * (size_t)A.bs;
  const size_t need_b = (B.bf16 || B.pl) ? 0 : (size_t)ng * PL * (size_t)batch * (size_t)B.bs;
  const size_t big = (size_t)1 << 20;   // elements
  const bool cheap_a = A.bf16 || A.pl || (size_t)batch * (size_t)A.bs >= big;
  const bool cheap_b = B.bf16 || B.pl || (size_t)batch * (size_t)B.bs >= big;
  const bool planes = apl != nullptr && bgemm_planes_has_form(A, B) && cheap_a && cheap_b && M % 64 == 0 &&
                      N % 64 == 0 && K % 64 == 0 && A.ld % 4 == 0 && A.bs % 4 == 0 && B.ld % 4 == 0 && B.bs % 4 == 0 &&
                      need_a <= apl_elems / 2 && need_b <= apl_elems / 2;
  bf16_t* bpl = apl ? apl + apl_elems / 2 : nullptr;
  auto run = [&](GemmArgs& ga) -> lact_status {
    if (planes)
      return fp32_grade ? bgemm_planes_form<3>(ga, A, B, K, apl, bpl, s) : bgemm_planes_form<2>(ga, A, B, K, apl, bpl, s);
    return fp32_grade ? bgemm_form<3>(A, B, ga, s) : bgemm_form<2>(A, B, ga, s);
  };
  GemmArgs g = gemm_args();
  g.ngroups = ng;
  g.lda = A.ld;
  g.a_bs = A.bs;
  g.ldb = B.ld;
  g.b_bs = B.bs;
  g.N = N;
  g.K = g.kps = K;
  g.batch = batch;
  g.alpha = alpha;
  const int64_t tiles = (int64_t)((M + 63) / 64) * ((N + 63) / 64) * batch * ng;
  int S = spl ? bwd_splits(tiles, K) : 1;
  const int64_t mnb = (int64_t)M * N * batch;
  while (S > 1 && (size_t)S * ng * mnb > spl_floats) --S;
  if (S > 1) {
    // split boundaries on whole k stages (32 wide; 64 on the plane path)
    const int64_t kq = planes ? 64 : 32;
    g.kps = (K + S - 1) / S;
    g.kps = (g.kps + kq - 1) / kq * kq;
    S = (int)((K + g.kps - 1) / g.kps);
  }
  if (S > 1) {
    // partials [S][batch][M][N] per group
    g.splits = S;
    g.ldc = N;
    g.c_bs = (int64_t)M * N;
    g.c_ss = mnb;
    for (int i = 0; i < ng; ++i) {
      g.g[i].A = gs[i].A;
      g.g[i].B = gs[i].B;
      g.g[i].C = spl + (int64_t)i * S * mnb;
      g.g[i].Cin = nullptr;
      g.g[i].M = M;
    }
    lact_status r = run(g);
    if (r) return r;
    for (int i = 0; i < ng; ++i) {
      KernelTimer kt(LACT_K_BWD_ELEM, s);
      LACT_LAUNCH(bwd_splitsum_kernel, dim3(ew_grid(mnb)), dim3(NT), s, (const float*)(spl + (int64_t)i * S * mnb),
                  S, batch, M, N, gs[i].C, ldc, c_bs, gs[i].Cin, beta);
      HIP_TRY(hipGetLastError());
    }
    return LACT_OK;
  }
  g.ldc = ldc;
  g.c_bs = c_bs;
  g.ldcin = ldc;
  g.cin_bs = c_bs;
  g.beta = beta;
  for (int i = 0; i < ng; ++i) {
    g.g[i].A = gs[i].A;
    g.g[i].B = gs[i].B;
    g.g[i].C = gs[i].C;
    g.g[i].Cin = gs[i].Cin;
    g.g[i].M = M;
  }
  return run(g);
}

// one Newton-Schulz product (fp32 grade)
lact_status bgemm_ns(BOp A, BOp B, float* C, int64_t ldc, int64_t c_bs, int M, int N, int64_t K, int batch,
                     float alpha, const float* Cin, float beta, hipStream_t s) {
  const BGrp g1{A.p, B.p, C, Cin};
  return bgemm_g(&g1, 1, A, B, ldc, c_bs, M, N, K, batch, alpha, beta, nullptr, 0, s, true);
}

#define BWD_LAUNCH(kernel, grid, ...)                      \
  do {                                                     \
    KernelTimer kt_(LACT_K_BWD_ELEM, s);                   \
    LACT_LAUNCH(kernel, grid, dim3(NT), s, __VA_ARGS__);   \
    HIP_TRY(hipGetLastError());                            \
  } while (0)

constexpr int BWD_NB = 32;    // partial sums per matrix (Newton-Schulz reductions)
constexpr int BWD_NBM = 64;   // partial sums per (instance, matrix) (momentum)

// ----------------------------------------------------------------- layout
struct BwdWs {
  int nu = 0;                 // update chunks
  int64_t cmax = 0;           // longest chunk
  size_t stW = 0, stM = 0;    // state slots: (nu + 1) x [W1 | W2 | W3] (and M)
  size_t fws = 0, fws_bytes = 0;
  size_t tok[9] = {};         // [n, cmax, dh] fp32 token buffers
  size_t U = 0, step = 0, gWp = 0, gU = 0, gM = 0, gX = 0;
  size_t X = 0, Am = 0, Pm = 0, gP = 0, gA = 0, Qm = 0, g0 = 0, g1 = 0, nrm = 0, part = 0;
  size_t mpart = 0;
  size_t spl = 0, spl_floats = 0;   // split-K partials of the token contractions
  size_t apl = 0, apl_elems = 0;     // bf16 planes of a token contraction's fp32 operands
  size_t wpl = 0, upl = 0;           // bf16 planes of the chunk's weight set and of gU
  size_t tpl = 0;                    // bf16 planes of three consecutive token buffers
  size_t qf = 0, kf = 0, vf = 0;     // LACT_QK_PREP: fp32 q^, k^ and v [n, L, d]
  size_t total = 0;
};

// The replay of the forward state trajectory: with bf16 inputs, two bf16
// planes per fp32 weight operand for GD and momentum, three (fp32 grade) for
// the Newton-Schulz optimisers; fp32 inputs always take three.  With raw
// q / k it runs on the backward's own fp32 pre-processed copies (not rounded
// to the io dtype), so its io type is fp32.
lact_problem replay_problem(const lact_problem& p) {
  lact_problem f = p;
  f.rec_planes = uses_ns(p.opt) ? 3 : 2;
  if (p.flags & LACT_QK_PREP) f.io_dtype = LACT_DTYPE_F32;
  f.flags &= LACT_NO_RENORM;
  return f;
}

Plan single_update(int64_t t0, int64_t len) {
  Plan pl;
  Step st;
  st.upd_t0 = t0;
  st.upd_len = len;
  pl.steps.push_back(st);
  pl.max_upd = len;
  return pl;
}

BwdWs bwd_layout(const lact_problem& p, const std::vector<int64_t>& b, const std::vector<uint8_t>& f) {
  BwdWs w;
  const size_t n = (size_t)std::max(0, p.n_inst), D = (size_t)p.d, Dh = (size_t)p.dh;
  const size_t DD = D * Dh, MDB = 3 * n * DD * 4;
  const size_t m = std::min(D, Dh);
  const lact_problem pf = replay_problem(p);
  for (size_t c = 0; c < f.size(); ++c) {
    const int64_t len = b[c + 1] - b[c];
    w.cmax = std::max(w.cmax, len);
    if (f[c] & LACT_CHUNK_UPDATE) {
      ++w.nu;
      w.fws_bytes = std::max(w.fws_bytes, layout(pf, single_update(b[c], len)).total);
    }
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.stW = take((size_t)(w.nu + 1) * MDB);
  if (uses_momentum(p.opt)) w.stM = take((size_t)(w.nu + 1) * MDB);
  w.fws = take(w.fws_bytes);
  for (int i = 0; i < 9; ++i) w.tok[i] = take(n * (size_t)w.cmax * Dh * 4);
  w.U = take(MDB);
  w.step = take(MDB);
  w.gWp = take(MDB);
  w.gU = take(MDB);
  w.gM = take(MDB);
  w.gX = take(MDB);
  if (uses_ns(p.opt)) {
    const size_t it = (size_t)p.ns_iters;
    const size_t MMB = 3 * n * m * m * 4;
    w.X = take((it + 1) * MDB);
    w.Am = take(it * MMB);
    w.Pm = take(it * MMB);
    w.gP = take(MMB);
    w.gA = take(MMB);
    w.Qm = take(MMB);
    w.g0 = take(MDB);
    w.g1 = take(MDB);
    w.nrm = take(3 * n * 4);
    w.part = take(3 * n * BWD_NB * 4);
  }
  w.mpart = take(n * 3 * BWD_NBM * 4);
  {
    // the token contractions: pairs of [dh, d] outputs, single [d, dh] ones
    const int64_t tb = (int64_t)((Dh + 63) / 64) * ((D + 63) / 64) * (int64_t)n;
    const size_t s2 = (size_t)bwd_splits(2 * tb, w.cmax) * 2 * n * DD;
    const size_t s1 = (size_t)bwd_splits(tb, w.cmax) * n * DD;
    w.spl_floats = std::max(s1, s2);
    w.spl = take(w.spl_floats * 4);
    // planes of the products' fp32 operands (token buffers [n, cmax, dh] or
    // weight-shaped [n, d dh]): two groups per operand, first half for the
    // first operands, second half for the second
    const size_t opnd = std::max((size_t)w.cmax * Dh, DD) * n;
    w.apl_elems = 2 * 2 * (size_t)(uses_ns(p.opt) ? 3 : 2) * opnd;
    w.apl = take(w.apl_elems * 2);
    w.wpl = take((size_t)(uses_ns(p.opt) ? 3 : 2) * 3 * n * DD * 2);
    w.upl = take((size_t)(uses_ns(p.opt) ? 3 : 2) * 3 * n * DD * 2);
    w.tpl = take((size_t)(uses_ns(p.opt) ? 3 : 2) * 3 * n * (size_t)w.cmax * Dh * 2);
  }
  if (p.flags & LACT_QK_PREP) {
    const size_t L = (size_t)b.back();
    w.qf = take(n * L * D * 4);
    w.kf = take(n * L * D * 4);
    w.vf = take(n * L * D * 4);
  }
  w.total = off;
  return w;
}

// ----------------------------------------------------------------- the pass
struct BwdPtrs {
  const void *q, *k, *v, *dO;
  const float *lr, *beta;
  const float* oz;   // per-token output-scale pre-activation [n, L] (NULL: no scale)
  float* doz;
  const float *W[3], *M[3], *gW[3], *gM[3];
  float *dq, *dk, *dv, *dlr, *dbeta;
  float *dW[3], *dM[3];
  char* ws;
};

lact_status run_backward(const lact_problem& p, const BwdPtrs& P, int64_t L, int32_t order,
                         const std::vector<int64_t>& b, const std::vector<uint8_t>& f, const BwdWs& w,
                         hipStream_t s) {
  const int n = p.n_inst, D = p.d, Dh = p.dh;
  const int64_t DD = (int64_t)D * Dh, MD = 3 * (int64_t)n * DD;
  const int m = std::min(D, Dh), kf = std::max(D, Dh);
  const int64_t MM = (int64_t)m * m;
  const bool bf = p.io_dtype == LACT_DTYPE_BF16;
  const bool prep = (p.flags & LACT_QK_PREP) != 0;
  const int64_t x_bs = L * D;          // instance stride of q, k, v, dO, dq, dk, dv
  const int64_t buf_bs = w.cmax * Dh;  // instance stride of the token buffers
  const bool mom = uses_momentum(p.opt), ns = uses_ns(p.opt);
  const bool renorm = !(p.flags & LACT_NO_RENORM);
  char* ws = P.ws;
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  // a weight-shaped set at byte offset `off` (W1 | W2 | W3, each [n, DD])
  auto set = [&](size_t off) {
    MatP r;
    for (int j = 0; j < 3; ++j) r.p[j] = fp(off) + (int64_t)j * n * DD;
    return r;
  };
  auto cset = [](const MatP& a) {
    MatC r;
    for (int j = 0; j < 3; ++j) r.p[j] = a.p[j];
    return r;
  };
  auto slotW = [&](int u) { return set(w.stW + (size_t)u * MD * 4); };
  auto slotM = [&](int u) { return set(w.stM + (size_t)u * MD * 4); };
  float* tk[9];
  for (int i = 0; i < 9; ++i) tk[i] = fp(w.tok[i]);
  const MatP U = set(w.U), STEP = set(w.step), GWP = set(w.gWp), GU = set(w.gU), GM = set(w.gM), GX = set(w.gX);
  MatP DW;
  for (int j = 0; j < 3; ++j) DW.p[j] = P.dW[j];
  lact_status r = LACT_OK;

  // ---- the operands of the sweep: the caller's q, k, v in the io dtype, or
  // (raw q / k) fp32 pre-processed copies of q, k and an fp32 copy of v
  const void* Qs = P.q;
  const void* Ks = P.k;
  const void* Vs = P.v;
  bool bq = bf, bv = bf;
  const bool bo = bf;
  if (prep) {
    const int64_t rows = (int64_t)n * L;
    const dim3 g((unsigned)((rows + 3) / 4));
    auto conv = [&](const void* src, float* dst, int pr) -> lact_status {
      if (!src) return LACT_OK;
      if (bf) BWD_LAUNCH(bwd_prep_kernel<bf16_t>, g, static_cast<const bf16_t*>(src), dst, rows, D, pr);
      else BWD_LAUNCH(bwd_prep_kernel<float>, g, static_cast<const float*>(src), dst, rows, D, pr);
      return LACT_OK;
    };
    if ((r = conv(P.q, fp(w.qf), 1))) return r;
    if ((r = conv(P.k, fp(w.kf), 1))) return r;
    if ((r = conv(P.v, fp(w.vf), 0))) return r;
    Qs = fp(w.qf);
    Ks = fp(w.kf);
    Vs = fp(w.vf);
    bq = bv = false;
  }
  const size_t eq = bq ? 2 : 4, ev = bv ? 2 : 4, eo = bo ? 2 : 4;

  // ---- outputs start at zero (rows outside the chunks that write them stay zero)
  BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * L * D)), P.dq, (int64_t)n * L * D, 0.f);
  BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * L * D)), P.dk, (int64_t)n * L * D, 0.f);
  BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * L * D)), P.dv, (int64_t)n * L * D, 0.f);
  BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * L * 3)), P.dlr, (int64_t)n * L * 3, 0.f);
  if (P.dbeta) BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * L)), P.dbeta, (int64_t)n * L, 0.f);
  if (P.doz) BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * L)), P.doz, (int64_t)n * L, 0.f);
  // running cotangents of the state: W in the caller's dW arrays, M in the workspace
  for (int j = 0; j < 3; ++j) {
    const size_t mb = (size_t)n * DD * 4;
    if (P.gW[j]) HIP_TRY(hipMemcpyAsync(DW.p[j], P.gW[j], mb, hipMemcpyDeviceToDevice, s));
    else BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * DD)), DW.p[j], (int64_t)n * DD, 0.f);
    if (P.gM[j]) HIP_TRY(hipMemcpyAsync(GM.p[j], P.gM[j], mb, hipMemcpyDeviceToDevice, s));
    else BWD_LAUNCH(bwd_fill_kernel, dim3(ew_grid((int64_t)n * DD)), GM.p[j], (int64_t)n * DD, 0.f);
  }

  // ---- replay of the forward state trajectory: slot u = state before update u
  {
    TraceRange tr("lact backward: replay of %d updates", w.nu);
    const MatP s0 = slotW(0);
    for (int j = 0; j < 3; ++j)
      HIP_TRY(hipMemcpyAsync(s0.p[j], P.W[j], (size_t)n * DD * 4, hipMemcpyDeviceToDevice, s));
    if (mom) {
      const MatP m0 = slotM(0);
      for (int j = 0; j < 3; ++j)
        HIP_TRY(hipMemcpyAsync(m0.p[j], P.M[j], (size_t)n * DD * 4, hipMemcpyDeviceToDevice, s));
    }
    const lact_problem pf = replay_problem(p);
    int u = 0;
    for (size_t c = 0; c < f.size(); ++c) {
      if (!(f[c] & LACT_CHUNK_UPDATE)) continue;
      const MatP wa = slotW(u), wb = slotW(u + 1);
      HIP_TRY(hipMemcpyAsync(wb.p[0], wa.p[0], (size_t)MD * 4, hipMemcpyDeviceToDevice, s));
      Ptrs F;
      F.k = Ks;
      F.v = Vs;
      F.lr = P.lr;
      F.beta = P.beta;
      F.W1 = wb.p[0];
      F.W2 = wb.p[1];
      F.W3 = wb.p[2];
      if (mom) {
        const MatP ma = slotM(u), mb = slotM(u + 1);
        HIP_TRY(hipMemcpyAsync(mb.p[0], ma.p[0], (size_t)MD * 4, hipMemcpyDeviceToDevice, s));
        F.M1 = mb.p[0];
        F.M2 = mb.p[1];
        F.M3 = mb.p[2];
      }
      F.ws = ws + w.fws;
      const Plan pl = single_update(b[c], b[c + 1] - b[c]);
      r = dispatch(pf, F, L, pl, layout(pf, pl), s);
      if (r) return r;
      ++u;
    }
  }

  // ---- Newton-Schulz forward, keeping the iterates (frame layout)
  const int iters = p.ns_iters;
  auto Xi = [&](int i) { return fp(w.X) + (int64_t)i * MD; };
  auto Ai = [&](int i) { return fp(w.Am) + (int64_t)i * 3 * n * MM; };
  auto Pi = [&](int i) { return fp(w.Pm) + (int64_t)i * 3 * n * MM; };
  const float na = 3.4445f, nb = -4.7750f, nc = 2.0315f;
  const float ns_eps = 1e-7f;
  auto ns_forward = [&](const MatC& G) -> lact_status {
    MatC none;
    none.p[0] = none.p[1] = none.p[2] = nullptr;
    BWD_LAUNCH(bwd_dot_kernel, dim3(BWD_NB, 3 * n), G, none, fp(w.part), n, DD, BWD_NB);
    BWD_LAUNCH(bwd_ns_init_kernel, dim3(ew_grid(MD)), G, (const float*)fp(w.part), BWD_NB, Xi(0), fp(w.nrm), n, D,
               Dh, ns_eps);
    for (int i = 0; i < iters; ++i) {
      lact_status q;
      // A = X X^T ; P = c A A + b A ; X' = P X + a X
      if ((q = bgemm_ns(bop(Xi(i), kf, DD, false), bop(Xi(i), kf, DD, false), Ai(i), m, MM, m, m, kf, 3 * n, 1.f,
                     nullptr, 0.f, s)))
        return q;
      if ((q = bgemm_ns(bop(Ai(i), m, MM, false), bop(Ai(i), m, MM, false), Pi(i), m, MM, m, m, m, 3 * n, nc, Ai(i),
                     nb, s)))
        return q;
      if ((q = bgemm_ns(bop(Pi(i), m, MM, false), bop(Xi(i), kf, DD, true), Xi(i + 1), kf, DD, m, kf, m, 3 * n, 1.f,
                     Xi(i), na, s)))
        return q;
    }
    return LACT_OK;
  };
  // cotangent of G for Y = NS(G) given gY (original layout) -> out; uses the
  // iterates of the last ns_forward(G)
  auto ns_backward = [&](const MatC& G, const MatC& gY, const MatP& out) -> lact_status {
    float* g0 = fp(w.g0);
    float* g1 = fp(w.g1);
    BWD_LAUNCH(bwd_frame_in_kernel, dim3(ew_grid(MD)), gY, g0, n, D, Dh);
    for (int i = iters - 1; i >= 0; --i) {
      lact_status q;
      // gP = g X^T
      if ((q = bgemm_ns(bop(g0, kf, DD, false), bop(Xi(i), kf, DD, false), fp(w.gP), m, MM, m, m, kf, 3 * n, 1.f,
                     nullptr, 0.f, s)))
        return q;
      // gA = c gP A + b gP, then += c A gP
      if ((q = bgemm_ns(bop(fp(w.gP), m, MM, false), bop(Ai(i), m, MM, false), fp(w.gA), m, MM, m, m, m, 3 * n, nc,
                     fp(w.gP), nb, s)))
        return q;
      if ((q = bgemm_ns(bop(Ai(i), m, MM, false), bop(fp(w.gP), m, MM, true), fp(w.gA), m, MM, m, m, m, 3 * n, nc,
                     fp(w.gA), 1.f, s)))
        return q;
      BWD_LAUNCH(bwd_symadd_kernel, dim3(ew_grid(3 * n * MM)), (const float*)fp(w.gA), fp(w.Qm), m,
                 (int64_t)3 * n);
      // g' = P g + a g + (gA + gA^T) X
      if ((q = bgemm_ns(bop(Pi(i), m, MM, false), bop(g0, kf, DD, true), g1, kf, DD, m, kf, m, 3 * n, 1.f, g0, na,
                     s)))
        return q;
      if ((q = bgemm_ns(bop(fp(w.Qm), m, MM, false), bop(Xi(i), kf, DD, true), g1, kf, DD, m, kf, m, 3 * n, 1.f, g1,
                     1.f, s)))
        return q;
      std::swap(g0, g1);
    }
    // back to the original layout (into gX), then the normalisation backward
    BWD_LAUNCH(bwd_frame_out_kernel, dim3(ew_grid(MD)), (const float*)g0, GX, 1.f, n, D, Dh);
    BWD_LAUNCH(bwd_dot_kernel, dim3(BWD_NB, 3 * n), cset(GX), G, fp(w.part), n, DD, BWD_NB);
    BWD_LAUNCH(bwd_ns_finish_kernel, dim3(ew_grid(MD)), cset(GX), G, (const float*)fp(w.nrm),
               (const float*)fp(w.part), BWD_NB, out, 1.f, n, DD, ns_eps);
    return LACT_OK;
  };

  // the sweep's products: two planes per fp32 operand for GD and momentum,
  // three (fp32 grade) for the Newton-Schulz optimisers, whose backward
  // amplifies the rounding of the recomputed directions U
  const bool fp32g = ns;
  auto gemm1 = [&](BOp A, BOp B, float* C, int64_t ldc, int64_t c_bs, int M, int N, int64_t K, int batch,
                   float alpha, const float* Cin, float beta, hipStream_t st) {
    const BGrp g1{A.p, B.p, C, Cin};
    return bgemm_g(&g1, 1, A, B, ldc, c_bs, M, N, K, batch, alpha, beta, nullptr, 0, st, fp32g,
                   reinterpret_cast<bf16_t*>(ws + w.apl), w.apl_elems);
  };
  auto gemmg = [&](const BGrp* gs, int ng, const BOp& A, const BOp& B, int64_t ldc, int64_t c_bs, int M, int N,
                   int64_t K, int batch, float alpha, float beta, float* spl, size_t spl_floats, hipStream_t st) {
    return bgemm_g(gs, ng, A, B, ldc, c_bs, M, N, K, batch, alpha, beta, spl, spl_floats, st, fp32g,
                   reinterpret_cast<bf16_t*>(ws + w.apl), w.apl_elems);
  };

  // weight-shaped sets (W1 | W2 | W3 contiguous) split into bf16 planes once
  // per chunk, for the products that read them on the direct-load GEMM
  const int PLW = fp32g ? 3 : 2;
  const int64_t setps = 3 * (int64_t)n * DD;   // plane stride of a set's planes
  bf16_t* WPL = reinterpret_cast<bf16_t*>(ws + w.wpl);
  bf16_t* UPL = reinterpret_cast<bf16_t*>(ws + w.upl);
  // every product that reads these planes has the chunk's length as a
  // dimension, so a chunk whose length is not a whole number of 64-wide
  // tiles takes the register path throughout and splits nothing
  bool chunk_planes = false;
  auto contiguous = [&](const MatC& m) {
    return chunk_planes && m.p[1] == m.p[0] + (int64_t)n * DD && m.p[2] == m.p[0] + 2 * (int64_t)n * DD;
  };
  auto split_set = [&](const MatC& m, bf16_t* dst) -> lact_status {
    if (!contiguous(m)) return LACT_OK;
    return bwd_split(m.p[0], setps, setps, 1, PLW, dst, setps, s);
  };
  auto wop = [&](BOp o, const MatC& m, const bf16_t* pl) { return contiguous(m) ? with_planes(o, pl, m.p[0], setps) : o; };
  // token buffers tk[j0 .. j0 + 2] (contiguous [n, cmax, dh] each) split once
  // after their producer, read by the products that follow
  bf16_t* TPL = reinterpret_cast<bf16_t*>(ws + w.tpl);
  const int64_t tps = 3 * (int64_t)n * buf_bs;
  auto tok_contig = [&](int j0) {
    return chunk_planes && tk[j0 + 1] == tk[j0] + (int64_t)n * buf_bs && tk[j0 + 2] == tk[j0] + 2 * (int64_t)n * buf_bs;
  };
  auto split_tok = [&](int j0) -> lact_status {
    if (!tok_contig(j0)) return LACT_OK;
    return bwd_split(tk[j0], tps, tps, 1, PLW, TPL, tps, s);
  };
  auto tokop = [&](BOp o, int j0) { return tok_contig(j0) ? with_planes(o, TPL, tk[j0], tps) : o; };

  // ---- apply backward of rows [t0, t0 + C) read with weights Wa
  auto apply_bwd = [&](const MatC& Wa, int64_t t0, int64_t C) -> lact_status {
    lact_status q;
    chunk_planes = C % 64 == 0;
    if ((q = split_set(Wa, WPL))) return q;
    const char* Q = static_cast<const char*>(Qs) + (size_t)t0 * D * eq;
    const char* dO = static_cast<const char*>(P.dO) + (size_t)t0 * D * eo;
    // Aq = q W1^T, Bq = q W3^T (one launch), dHq = dO W2
    {
      const BGrp g2[2] = {{Q, Wa.p[0], tk[0], nullptr}, {Q, Wa.p[2], tk[1], nullptr}};
      if ((q = gemmg(g2, 2, bop(Q, D, x_bs, false, bq), wop(bop(nullptr, D, DD, false), Wa, WPL), Dh, buf_bs, (int)C,
                       Dh, D, n, 1.f, 0.f, nullptr, 0, s)))
        return q;
    }
    if ((q = gemm1(bop(dO, D, x_bs, false, bo), wop(bop(Wa.p[1], Dh, DD, true), Wa, WPL), tk[2], Dh, buf_bs, (int)C,
                   Dh, D, n, 1.f, nullptr, 0.f, s)))
      return q;
    // -> dAq, dBq, Hq (with an output scale: s Hq, and doz)
    if (P.oz)
      BWD_LAUNCH(bwd_app_elem_oz_kernel, dim3((unsigned)(((int64_t)n * C + 3) / 4)), tk[0], tk[1], tk[2], P.oz, L,
                 t0, P.doz, n, C, Dh, buf_bs);
    else
      BWD_LAUNCH(bwd_app_elem_kernel, dim3(ew_grid((int64_t)n * C * Dh)), tk[0], tk[1], tk[2], n, C, Dh, buf_bs);
    if ((q = split_tok(0))) return q;
    // dW2 += dO^T Hq ; dW1 += dAq^T q, dW3 += dBq^T q (one launch); split over tokens
    {
      const BGrp g1[1] = {{dO, tk[2], DW.p[1], DW.p[1]}};
      if ((q = gemmg(g1, 1, bop(dO, D, x_bs, true, bo), tokop(bop(nullptr, Dh, buf_bs, true), 0), Dh, DD, D, Dh, C, n,
                       1.f, 1.f, fp(w.spl), w.spl_floats, s)))
        return q;
      const BGrp g2[2] = {{tk[0], Q, DW.p[0], DW.p[0]}, {tk[1], Q, DW.p[2], DW.p[2]}};
      if ((q = gemmg(g2, 2, tokop(bop(nullptr, Dh, buf_bs, true), 0), bop(Q, D, x_bs, true, bq), D, DD, Dh, D, C, n,
                       1.f, 1.f, fp(w.spl), w.spl_floats, s)))
        return q;
    }
    // dq = dAq W1 + dBq W3
    float* dq = P.dq + t0 * D;
    if ((q = gemm1(tokop(bop(tk[0], Dh, buf_bs, false), 0), wop(bop(Wa.p[0], D, DD, true), Wa, WPL), dq, D, x_bs,
                   (int)C, D, Dh, n, 1.f, nullptr, 0.f, s)))
      return q;
    return gemm1(tokop(bop(tk[1], Dh, buf_bs, false), 0), wop(bop(Wa.p[2], D, DD, true), Wa, WPL), dq, D, x_bs,
                 (int)C, D, Dh, n, 1.f, dq, 1.f, s);
  };

  // ---- update backward of chunk [t0, t0 + C), update ordinal u
  auto update_bwd = [&](int u, int64_t t0, int64_t C) -> lact_status {
    lact_status q;
    const MatC Wb = cset(slotW(u));
    chunk_planes = C % 64 == 0;
    if ((q = split_set(Wb, WPL))) return q;
    const char* K = static_cast<const char*>(Ks) + (size_t)t0 * D * eq;
    const char* V = static_cast<const char*>(Vs) + (size_t)t0 * D * ev;
    float *A_ = tk[0], *B_ = tk[1], *G_ = tk[2], *E1 = tk[3], *E3 = tk[4], *H2 = tk[5], *gE1 = tk[6], *gE3 = tk[7],
          *gH2 = tk[8];
    // recompute A = k W1^T, B = k W3^T (one launch), G = v W2 and the update terms
    {
      const BGrp g2[2] = {{K, Wb.p[0], A_, nullptr}, {K, Wb.p[2], B_, nullptr}};
      if ((q = gemmg(g2, 2, bop(K, D, x_bs, false, bq), wop(bop(nullptr, D, DD, false), Wb, WPL), Dh, buf_bs, (int)C,
                       Dh, D, n, 1.f, 0.f, nullptr, 0, s)))
        return q;
    }
    if ((q = gemm1(bop(V, D, x_bs, false, bv), wop(bop(Wb.p[1], Dh, DD, true), Wb, WPL), G_, Dh, buf_bs, (int)C, Dh,
                   D, n, 1.f, nullptr, 0.f, s)))
      return q;
    BWD_LAUNCH(bwd_upd_terms_kernel, dim3(ew_grid((int64_t)n * C * Dh)), (const float*)A_, (const float*)B_,
               (const float*)G_, P.lr, L * 3, t0, E1, E3, H2, n, C, Dh, buf_bs);
    if ((q = split_tok(3))) return q;
    // U1 = E1^T k, U3 = E3^T k (one launch), U2 = v^T H2; split over tokens
    {
      const BGrp g2[2] = {{E1, K, U.p[0], nullptr}, {E3, K, U.p[2], nullptr}};
      if ((q = gemmg(g2, 2, tokop(bop(nullptr, Dh, buf_bs, true), 3), bop(K, D, x_bs, true, bq), D, DD, Dh, D, C, n,
                       1.f, 0.f, fp(w.spl), w.spl_floats, s)))
        return q;
      const BGrp g1[1] = {{V, H2, U.p[1], nullptr}};
      if ((q = gemmg(g1, 1, bop(V, D, x_bs, true, bv), tokop(bop(nullptr, Dh, buf_bs, true), 3), Dh, DD, D, Dh, C, n,
                       1.f, 0.f, fp(w.spl), w.spl_floats, s)))
        return q;
    }
    // the weight step W' = W + sgn step
    MatC step;
    float sgn = 1.f;
    const MatC Mn = mom ? cset(slotM(u + 1)) : MatC{};
    if (p.opt == LACT_OPT_GD) {
      step = cset(U);
    } else if (p.opt == LACT_OPT_MOMENTUM) {
      step = Mn;
      sgn = -1.f;
    } else {
      if ((q = ns_forward(p.opt == LACT_OPT_MUON ? cset(U) : Mn))) return q;
      BWD_LAUNCH(bwd_frame_out_kernel, dim3(ew_grid(MD)), (const float*)Xi(iters), STEP, 1.f, n, D, Dh);
      step = cset(STEP);
      if (p.opt == LACT_OPT_MUON_MOMENTUM) sgn = -1.f;
    }
    // renorm backward: dW (cotangent of the next state) -> cotangent of W
    // through the renorm; gW' -> GWP
    BWD_LAUNCH(bwd_renorm_kernel, dim3((unsigned)(((int64_t)n * (2 * Dh + D) + 3) / 4)), Wb, step, sgn, DW, GWP, n,
               D, Dh, renorm ? 1 : 0);
    // optimiser backward -> gU
    MatC gU = cset(GU);
    if (p.opt == LACT_OPT_GD) {
      gU = cset(GWP);
    } else if (p.opt == LACT_OPT_MUON) {
      if ((q = ns_backward(cset(U), cset(GWP), GU))) return q;
    } else {
      MatC gX = cset(GWP);
      if (p.opt == LACT_OPT_MUON_MOMENTUM) {
        if ((q = ns_backward(Mn, cset(GWP), GU))) return q;
        gX = cset(GU);   // consumed below before GU is overwritten element by element
      }
      BWD_LAUNCH(bwd_mom_kernel, dim3(BWD_NBM, 3, n), GM, gX, cset(slotM(u)), P.beta, L, t0, C, GU, fp(w.mpart),
                 DD, BWD_NBM);
      BWD_LAUNCH(bwd_mom_finish_kernel, dim3((unsigned)std::min<int64_t>((C + NT - 1) / NT, 64), n),
                 (const float*)fp(w.mpart), BWD_NBM, P.dbeta, L, t0, C);
    }
    // through the update terms: gE1 = k gU1^T, gE3 = k gU3^T (one launch), gH2 = v gU2
    if ((q = split_set(gU, UPL))) return q;
    {
      const BGrp g2[2] = {{K, gU.p[0], gE1, nullptr}, {K, gU.p[2], gE3, nullptr}};
      if ((q = gemmg(g2, 2, bop(K, D, x_bs, false, bq), wop(bop(nullptr, D, DD, false), gU, UPL), Dh, buf_bs, (int)C,
                       Dh, D, n, 1.f, 0.f, nullptr, 0, s)))
        return q;
    }
    if ((q = gemm1(bop(V, D, x_bs, false, bv), wop(bop(gU.p[1], Dh, DD, true), gU, UPL), gH2, Dh, buf_bs, (int)C, Dh,
                   D, n, 1.f, nullptr, 0.f, s)))
      return q;
    // dk = E1 gU1 + E3 gU3 ; dv = H2 gU2^T
    float* dk = P.dk + t0 * D;
    float* dv = P.dv + t0 * D;
    if ((q = gemm1(tokop(bop(E1, Dh, buf_bs, false), 3), wop(bop(gU.p[0], D, DD, true), gU, UPL), dk, D, x_bs, (int)C,
                   D, Dh, n, 1.f, nullptr, 0.f, s)))
      return q;
    if ((q = gemm1(tokop(bop(E3, Dh, buf_bs, false), 3), wop(bop(gU.p[2], D, DD, true), gU, UPL), dk, D, x_bs, (int)C,
                   D, Dh, n, 1.f, dk, 1.f, s)))
      return q;
    if ((q = gemm1(tokop(bop(H2, Dh, buf_bs, false), 3), wop(bop(gU.p[1], Dh, DD, false), gU, UPL), dv, D, x_bs,
                   (int)C, D, Dh, n, 1.f, nullptr, 0.f, s)))
      return q;
    // -> gA, gB, gG (in place) and dlr
    BWD_LAUNCH(bwd_upd_elem_kernel, dim3((unsigned)(((int64_t)n * C + 3) / 4)), (const float*)A_, (const float*)B_,
               (const float*)G_, P.lr, L * 3, t0, gE1, gE3, gH2, P.dlr, n, C, Dh, buf_bs);
    if ((q = split_tok(6))) return q;
    // dk += gA W1 + gB W3 ; dv += gG W2^T
    if ((q = gemm1(tokop(bop(gE1, Dh, buf_bs, false), 6), wop(bop(Wb.p[0], D, DD, true), Wb, WPL), dk, D, x_bs,
                   (int)C, D, Dh, n, 1.f, dk, 1.f, s)))
      return q;
    if ((q = gemm1(tokop(bop(gE3, Dh, buf_bs, false), 6), wop(bop(Wb.p[2], D, DD, true), Wb, WPL), dk, D, x_bs,
                   (int)C, D, Dh, n, 1.f, dk, 1.f, s)))
      return q;
    if ((q = gemm1(tokop(bop(gH2, Dh, buf_bs, false), 6), wop(bop(Wb.p[1], Dh, DD, false), Wb, WPL), dv, D, x_bs,
                   (int)C, D, Dh, n, 1.f, dv, 1.f, s)))
      return q;
    // dW1 += gA^T k, dW3 += gB^T k (one launch) ; dW2 += v^T gG; split over tokens
    const BGrp g2[2] = {{gE1, K, DW.p[0], DW.p[0]}, {gE3, K, DW.p[2], DW.p[2]}};
    if ((q = gemmg(g2, 2, tokop(bop(nullptr, Dh, buf_bs, true), 6), bop(K, D, x_bs, true, bq), D, DD, Dh, D, C, n, 1.f,
                     1.f, fp(w.spl), w.spl_floats, s)))
      return q;
    const BGrp g1[1] = {{V, gH2, DW.p[1], DW.p[1]}};
    return gemmg(g1, 1, bop(V, D, x_bs, true, bv), tokop(bop(nullptr, Dh, buf_bs, true), 6), Dh, DD, D, Dh, C, n, 1.f,
                 1.f, fp(w.spl), w.spl_floats, s);
  };

  // ---- reverse sweep
  int u = w.nu;
  for (int c = (int)f.size() - 1; c >= 0; --c) {
    const int64_t t0 = b[c], C = b[c + 1] - b[c];
    const bool U_ = f[c] & LACT_CHUNK_UPDATE, A_ = f[c] & LACT_CHUNK_APPLY;
    TraceRange tr("lact backward chunk %d: tokens %lld..%lld", c, (long long)t0, (long long)(t0 + C));
    // slot u: the state before this chunk (after its update: slot u + 1)
    if (U_) --u;
    if (A_ && U_ && order == LACT_UPDATE_THEN_APPLY)
      if ((r = apply_bwd(cset(slotW(u + 1)), t0, C))) return r;
    if (U_)
      if ((r = update_bwd(u, t0, C))) return r;
    if (A_ && (order == LACT_APPLY_THEN_UPDATE || !U_))
      if ((r = apply_bwd(cset(slotW(u)), t0, C))) return r;
  }
  // raw q / k: through the pre-processing (rows outside the chunks stay zero)
  if (prep) {
    const int64_t rows = (int64_t)n * L;
    const dim3 g((unsigned)((rows + 3) / 4));
    for (int m = 0; m < 2; ++m) {
      const void* x = m == 0 ? P.q : P.k;
      float* gx = m == 0 ? P.dq : P.dk;
      if (!x) continue;
      if (bf) BWD_LAUNCH(bwd_prep_vjp_kernel<bf16_t>, g, static_cast<const bf16_t*>(x), gx, rows, D);
      else BWD_LAUNCH(bwd_prep_vjp_kernel<float>, g, static_cast<const float*>(x), gx, rows, D);
    }
  }
  for (int j = 0; j < 3; ++j)
    if (P.dM[j]) HIP_TRY(hipMemcpyAsync(P.dM[j], GM.p[j], (size_t)n * DD * 4, hipMemcpyDeviceToDevice, s));
  return LACT_OK;
}
