// gfx950 kernels of the LaCT fast-weight layer forward.
//
// Update path (once per update chunk, on the current fast weights):
//   upd_fwd_kernel -- per (instance, 128-token block, BJ hidden columns):
//                     A = K W1^T, B = K W3^T, G = V W2 on MFMA, then the SwiGLU
//                     backward terms lr1*G*B*silu'(A), lr3*G*silu(A),
//                     lr2*silu(A)*B in registers, stored token-fastest
//                     ("大块测试时训练（LaCT）技术解析" §2.1, eqs. 4-5).
//   gemm_kernel    -- weight-gradient contraction over the chunk's tokens
//                     (split over tokens, fp32 partials), Newton-Schulz
//                     products, apply output product.
//   opt_kernel     -- sums the partials, GD / momentum step, row L2
//                     renormalisation ("大块测试时训练（LaCT）技术解析" §2.2.1
//                     eq. 8; "LaCT架构核心思想解析" §1.2), and writes the bf16
//                     snapshot of the new weights.
//   reduce_rows_kernel -- Muon: sums partials, per-row sums of squares.
// Apply path (after the recurrence, all chunks at once, each chunk on the
// snapshot of the weights it reads):
//   app_fwd_kernel -- Hq = silu(Q W1^T) * (Q W3^T);  gemm_kernel: o = Hq W2^T.
#pragma once
#include "lact_device.hpp"

namespace lact {

constexpr int NT = 256;   // threads per workgroup (4 waves, 2 x 2)

template <typename T, int P, int ROWS, int BK, bool COLK>
__device__ __forceinline__ void load_tile(typename LoaderSel<T, P, ROWS, BK, NT, COLK>::type& L, const T* base,
                                          int64_t ld, int64_t r0, int64_t rvalid, int64_t k0, int64_t kvalid,
                                          int tid) {
  if constexpr (COLK) L.load(base, ld, r0, rvalid, k0, kvalid, tid);
  else L.load(base, ld, r0, rvalid, k0, tid);
}

// =========================================================================
// update forward tiles
struct UpdFwdArgs {
  const void* k;
  const void* v;
  int64_t x_bs;          // elements between instances in v (seq_stride * D)
  int64_t k_bs;          // elements between instances in k
  const float* lr;
  int64_t lr_bs;
  const float* beta;     // momentum: per-token beta (partial sums per token block), else null
  int64_t beta_bs;
  float* bpart;          // [n, tiles_t] beta partial sums
  const void* W1;        // [n, dh, d] (bf16 snapshot or fp32 master)
  const void* W3;
  const void* W2x;       // bf16: W2^T snapshot [n, dh, d]; fp32: W2 master [n, d, dh]
  void* E;               // [n, 3 dh, ldE] update terms, token-fastest: rows U1 | U3 | U2^T terms
  int64_t ldE;
  int D;                 // d: width of k, v (the products' contraction)
  int Dh;                // dh: hidden width (the products' output columns)
  int64_t upd_t0;
  int64_t upd_len;
  int tiles_t;           // token blocks per instance
  // bf16 tile only: the same tokens' queries, applied on the same snapshot
  // (null: none); Hq rows go to H + inst * h_bs, row h0 + (t - upd_t0)
  const void* q;
  int64_t q_bs;
  void* H;
  int64_t h_bs;
  int64_t h0;
  // multi-plane recurrence (direct-load tile): weight planes 1.. and the
  // plane stride of the stored update terms
  const void* Wlo;       // [P - 1][3: W1, W3, W2^T][n, dh, d] bf16
  int64_t wlo_ps, wlo_ms;
  int64_t e_ps;
};

constexpr int FBT = 128;  // tokens per forward tile

template <typename TIO, int PIO, typename TW, int PW, typename TREC, int BJ, int BK, int STAGES>
__global__ __launch_bounds__(NT) void upd_fwd_kernel(UpdFwdArgs a) {
  // W2 operand (element (j, r) = W2[r, j]): from the transposed bf16 snapshot
  // as a row-k source, or from the fp32 master as a column-k source.
  constexpr bool W2COL = sizeof(TW) == 4;
  using GT = TileGeom<FBT, BK>;
  using GJ = TileGeom<BJ, BK>;
  constexpr int STAGE = 2 * PIO * GT::PLANE + 3 * PW * GJ::PLANE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * STAGE];
  __shared__ float s_red[2];
  constexpr int FN = BJ / 32;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int D = a.D, Dh = a.Dh;
  const int njb = Dh / BJ;
  const int per_inst = a.tiles_t * njb;
  const int lbid = xcd_remap(blockIdx.x, gridDim.x);
  const int inst = lbid / per_inst;
  const int tile = lbid % per_inst;
  const int tb = tile / njb, jb = tile % njb;
  const int64_t t0 = a.upd_t0 + (int64_t)tb * FBT;
  const int64_t tend = a.upd_t0 + a.upd_len;
  const int j0 = jb * BJ;
  const int64_t DD = (int64_t)D * Dh;
  const TIO* K = reinterpret_cast<const TIO*>(a.k) + inst * a.k_bs;
  const TIO* V = reinterpret_cast<const TIO*>(a.v) + inst * a.x_bs;
  const TW* W1 = reinterpret_cast<const TW*>(a.W1) + inst * DD;
  const TW* W3 = reinterpret_cast<const TW*>(a.W3) + inst * DD;
  const TW* W2 = reinterpret_cast<const TW*>(a.W2x) + inst * DD;

  if (a.beta != nullptr && jb == 0) {
    // partial sum of beta over this token block (for the chunk mean)
    float bsum = 0.f;
    if (tid < FBT && t0 + tid < tend) bsum = a.beta[inst * a.beta_bs + t0 + tid];
    bsum = wave_sum(bsum);
    if (lane == 0 && wave < 2) s_red[wave] = bsum;
    __syncthreads();
    if (tid == 0) a.bpart[(int64_t)inst * a.tiles_t + tb] = s_red[0] + s_red[1];
  }

  RowKLoader<TIO, PIO, FBT, BK, NT> LK[2], LV[2];
  RowKLoader<TW, PW, BJ, BK, NT> L1[2], L3[2];
  typename LoaderSel<TW, PW, BJ, BK, NT, W2COL>::type L2[2];
  f32x4 accA[4][FN], accB[4][FN], accG[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) accA[i][j] = accB[i][j] = accG[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](auto set, int kt) {
    constexpr int r = decltype(set)::value;
    const int k0 = kt * BK;
    LK[r].load(K, D, t0, tend, k0, tid);
    LV[r].load(V, D, t0, tend, k0, tid);
    L1[r].load(W1, D, j0, Dh, k0, tid);
    L3[r].load(W3, D, j0, Dh, k0, tid);
    load_tile<TW, PW, BJ, BK, W2COL>(L2[r], W2, W2COL ? Dh : D, j0, Dh, k0, D, tid);
  };
  auto put = [&](auto set, auto buf) {
    constexpr int r = decltype(set)::value;
    uint16_t* b = smem + decltype(buf)::value * STAGE;
    LK[r].store(b, tid);
    LV[r].store(b + PIO * GT::PLANE, tid);
    uint16_t* w = b + 2 * PIO * GT::PLANE;
    L1[r].store(w, tid);
    L3[r].store(w + PW * GJ::PLANE, tid);
    L2[r].store(w + 2 * PW * GJ::PLANE, tid);
  };
  auto compute = [&](auto buf) {
    const uint16_t* b = smem + decltype(buf)::value * STAGE;
    const uint16_t* lK = b;
    const uint16_t* lV = b + PIO * GT::PLANE;
    const uint16_t* w = b + 2 * PIO * GT::PLANE;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      mma_tile<PIO, PW, 4, FN, GT::STRIDE, GJ::STRIDE>(accA, lK, GT::PLANE, wm * 64, w, GJ::PLANE, wn * (BJ / 2), kk, lane);
      mma_tile<PIO, PW, 4, FN, GT::STRIDE, GJ::STRIDE>(accB, lK, GT::PLANE, wm * 64, w + PW * GJ::PLANE, GJ::PLANE,
                                                       wn * (BJ / 2), kk, lane);
      mma_tile<PIO, PW, 4, FN, GT::STRIDE, GJ::STRIDE>(accG, lV, GT::PLANE, wm * 64, w + 2 * PW * GJ::PLANE,
                                                       GJ::PLANE, wn * (BJ / 2), kk, lane);
    }
  };
  pipeline<STAGES>(D / BK, fetch, put, compute);

  // SwiGLU backward epilogue; every token of the padded row is written (zeros
  // past the chunk end) so the contraction can read whole 16-byte vectors.
  TREC* E = reinterpret_cast<TREC*>(a.E) + inst * 3 * (int64_t)Dh * a.ldE;
  const float* lr = a.lr + inst * a.lr_bs;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tq = t0 + wm * 64 + i * 16 + 4 * (lane >> 4);   // first of 4 tokens
    const int64_t trel = tq - a.upd_t0;
    if (trel >= a.ldE) continue;
    float e1[4], e2[4], e3[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = tq + r < tend;
      e1[r] = ok ? lr[(tq + r) * 3 + 0] : 0.f;
      e2[r] = ok ? lr[(tq + r) * 3 + 1] : 0.f;
      e3[r] = ok ? lr[(tq + r) * 3 + 2] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = j0 + wn * (BJ / 2) + j * 16 + (lane & 15);
      float u1[4], u3[4], u2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = accA[i][j][r], b = accB[i][j][r], g = accG[i][j][r];
        const float sg = fast_sigmoid(x);
        const float s = x * sg;
        const float sp = sg * (1.0f + x * (1.0f - sg));
        u1[r] = e1[r] * g * b * sp;
        u3[r] = e3[r] * g * s;
        u2[r] = e2[r] * s * b;
      }
      store4(E + (int64_t)col * a.ldE + trel, u1);
      store4(E + (int64_t)(Dh + col) * a.ldE + trel, u3);
      store4(E + (int64_t)(2 * Dh + col) * a.ldE + trel, u2);
    }
  }
}

// =========================================================================
// apply forward tiles, grouped by the weight snapshot they read
constexpr int MAXG = 24;

struct AppGroup {
  int64_t t0;            // first token of the group's apply range
  int64_t len;
  int64_t h0;            // row offset of the group in the Hq buffer
  const void* W1;        // snapshot [n, dh, d] (W3 alike; W2 [n, d, dh])
  const void* W3;
  const void* W2;
  int tiles;             // workgroups of this group
};

struct AppFwdArgs {
  AppGroup g[MAXG];
  int ngroups;
  const void* q;
  int64_t q_bs;          // elements between instances in q
  int64_t x_bs;          // elements between instances in o
  void* H;               // [n, h_rows, dh]
  int64_t h_bs;
  void* o;               // output mode: [n, seq, d] (x_bs per instance)
  const float* oz;       // output mode: o[t, :] *= silu(oz[t]) (NULL: no scale)
  int64_t oz_bs;
  int D;                 // d: width of q and o
  int Dh;                // dh: hidden width
};

template <typename TIO, int PIO, typename TW, int PW, typename TAPP, int BJ, int BK, int STAGES>
__global__ __launch_bounds__(NT) void app_fwd_kernel(AppFwdArgs a) {
  using GT = TileGeom<FBT, BK>;
  using GJ = TileGeom<BJ, BK>;
  constexpr int STAGE = PIO * GT::PLANE + 2 * PW * GJ::PLANE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * STAGE];
  constexpr int FN = BJ / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int D = a.D, Dh = a.Dh;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < a.ngroups && bid >= a.g[gi].tiles) bid -= a.g[gi++].tiles;
  const AppGroup& G = a.g[gi];
  const int njb = Dh / BJ;
  const int tiles_t = (int)((G.len + FBT - 1) / FBT);
  const int per_inst = tiles_t * njb;
  const int inst = bid / per_inst;
  const int tile = bid % per_inst;
  const int tb = tile / njb, jb = tile % njb;
  const int64_t t0 = G.t0 + (int64_t)tb * FBT;
  const int64_t tend = G.t0 + G.len;
  const int j0 = jb * BJ;
  const int64_t DD = (int64_t)D * Dh;
  const TIO* Q = reinterpret_cast<const TIO*>(a.q) + inst * a.q_bs;
  const TW* W1 = reinterpret_cast<const TW*>(G.W1) + inst * DD;
  const TW* W3 = reinterpret_cast<const TW*>(G.W3) + inst * DD;

  RowKLoader<TIO, PIO, FBT, BK, NT> LQ[2];
  RowKLoader<TW, PW, BJ, BK, NT> L1[2], L3[2];
  f32x4 accA[4][FN], accB[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) accA[i][j] = accB[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](auto set, int kt) {
    constexpr int r = decltype(set)::value;
    const int k0 = kt * BK;
    LQ[r].load(Q, D, t0, tend, k0, tid);
    L1[r].load(W1, D, j0, Dh, k0, tid);
    L3[r].load(W3, D, j0, Dh, k0, tid);
  };
  auto put = [&](auto set, auto buf) {
    constexpr int r = decltype(set)::value;
    uint16_t* b = smem + decltype(buf)::value * STAGE;
    LQ[r].store(b, tid);
    L1[r].store(b + PIO * GT::PLANE, tid);
    L3[r].store(b + PIO * GT::PLANE + PW * GJ::PLANE, tid);
  };
  // swapped MFMA order: each lane ends with 4 consecutive hidden columns of one token
  auto compute = [&](auto buf) {
    const uint16_t* b = smem + decltype(buf)::value * STAGE;
    const uint16_t* w = b + PIO * GT::PLANE;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      mma_tile<PIO, PW, 4, FN, GT::STRIDE, GJ::STRIDE, true>(accA, b, GT::PLANE, wm * 64, w, GJ::PLANE, wn * (BJ / 2),
                                                             kk, lane);
      mma_tile<PIO, PW, 4, FN, GT::STRIDE, GJ::STRIDE, true>(accB, b, GT::PLANE, wm * 64, w + PW * GJ::PLANE,
                                                             GJ::PLANE, wn * (BJ / 2), kk, lane);
    }
  };
  pipeline<STAGES>(D / BK, fetch, put, compute);
  TAPP* H = reinterpret_cast<TAPP*>(a.H) + inst * a.h_bs;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + wm * 64 + i * 16 + (lane & 15);
    if (t >= tend) continue;
    TAPP* Hr = H + (G.h0 + (t - G.t0)) * (int64_t)Dh;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = j0 + wn * (BJ / 2) + j * 16 + 4 * (lane >> 4);
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = accA[i][j][r];
        h[r] = x * fast_sigmoid(x) * accB[i][j][r];
      }
      store4(Hr + col, h);
    }
  }
}

// =========================================================================
// grouped batched GEMM:  C[m, n] = alpha * sum_k A(m, k) B(n, k) + beta * Cin[m, n]
//   A(m, k): row-k source A[m * lda + k]   or column-k source A[k * lda + m]
//   B(n, k): row-k source B[n * ldb + k]   or column-k source B[k * ldb + n]
// Groups share every stride and N, K; each has its own A, B, C and M.  K may
// be split: split s covers k in [s*kps, min(K, (s+1)*kps)) and writes its
// own partial C + s * c_ss.  Rows m >= trans_from are stored transposed into
// the block that starts at element trans_from * ldc, with row stride ldc_t.
struct GemmGroup {
  const void* A;
  const void* B;
  void* C;
  void* Cp;              // optional (plane GEMM): C also stored as bf16 planes, plane p at Cp + p * cp_ps
  const void* Cinp;      // optional (plane GEMM): Cin given as bf16 planes (layout of Cp) instead of fp32
  const float* rs;       // optional: row m of C is scaled by silu(rs[b * rs_bs + m])
  const float* Cin;      // optional: C += beta * Cin (batch stride cin_bs, row stride ldcin)
  const float* rowsq;    // optional Frobenius scale source (see GemmArgs), this group's first row
  int M;
  int tiles;             // workgroups of this group
};

struct GemmArgs {
  GemmGroup g[MAXG];
  int ngroups;
  int64_t lda, a_bs, ldb, b_bs, ldc, c_bs, c_ss;
  const void* B2;        // B operand for m-tiles at or beyond m_switch (group 0 only)
  int64_t b2_bs;         // its batch stride
  int64_t rs_bs;
  int m_switch;
  int trans_from;
  int64_t ldc_t;         // row stride of the transposed block
  int64_t ldcin, cin_bs;
  int N;
  int64_t K, kps;
  int64_t kpad;          // row-k operands are readable, and zero, from K up to kpad (0: no padding)
  int batch, splits;
  float alpha, beta;
  // optional scale s = 1 / (sqrt(sum of G.rowsq[b * rowsq_bs ... + rowsq_n)) + 1e-7):
  // alpha *= s^alpha_pow, beta *= s^beta_pow
  int64_t rowsq_bs;
  int rowsq_n, alpha_pow, beta_pow;
  // symmetric result (M == N, e.g. a Gram matrix X X^T or a product of
  // symmetric matrices): only tiles on or above the diagonal run, and the
  // off-diagonal ones also store their mirror image
  int sym;
  // plane GEMM: elements between the bf16 planes of A, B and of the stored C planes
  int64_t a_ps, b_ps, cp_ps;
};

template <typename TA, int PA, bool CA, typename TB, int PB, bool CB, typename TC, int BM, int BN, int BK, int STAGES>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs g) {
  using GA = TileGeom<BM, BK>;
  using GB = TileGeom<BN, BK>;
  constexpr int FM = BM / 32, FN = BN / 32;     // 2x2 waves, wave tile (BM/2) x (BN/2)
  constexpr int STAGE = PA * GA::PLANE + PB * GB::PLANE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * STAGE];
  __shared__ float s_scale;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < g.ngroups && bid >= g.g[gi].tiles) bid -= g.g[gi++].tiles;
  const GemmGroup& G = g.g[gi];
  const int M = G.M;
  const int tn_count = (g.N + BN - 1) / BN;
  const int tm_count = (M + BM - 1) / BM;
  const int tiles = g.sym ? tn_count * (tn_count + 1) / 2 : tm_count * tn_count;
  const int tile = bid % tiles;
  bid /= tiles;
  const int split = bid % g.splits;
  const int b = bid / g.splits;
  int tm = tile / tn_count, tn = tile % tn_count;
  if (g.sym) {   // upper triangle, row by row: row tm holds tiles tn = tm .. tn_count - 1
    int rem = tile;
    tm = 0;
    while (rem >= tn_count - tm) rem -= tn_count - tm++;
    tn = tm + rem;
  }
  const bool mirror = g.sym && tn != tm;
  const int m0 = tm * BM, n0 = tn * BN;

  const TA* A = reinterpret_cast<const TA*>(G.A) + b * g.a_bs;
  const bool second_b = g.B2 != nullptr && m0 >= g.m_switch;
  const TB* B = reinterpret_cast<const TB*>(second_b ? g.B2 : G.B) + b * (second_b ? g.b2_bs : g.b_bs);
  const int64_t kbeg = (int64_t)split * g.kps;
  const int64_t kend = min(g.K, kbeg + g.kps);

  typename LoaderSel<TA, PA, BM, BK, NT, CA>::type LA[2];
  typename LoaderSel<TB, PB, BN, BK, NT, CB>::type LB[2];
  auto fetch = [&](auto set, int64_t kt) {
    constexpr int r = decltype(set)::value;
    const int64_t k0 = kbeg + kt * BK;
    load_tile<TA, PA, BM, BK, CA>(LA[r], A, g.lda, m0, M, k0, kend, tid);
    load_tile<TB, PB, BN, BK, CB>(LB[r], B, g.ldb, n0, g.N, k0, kend, tid);
  };
  auto put = [&](auto set, auto buf) {
    constexpr int r = decltype(set)::value;
    uint16_t* b = smem + decltype(buf)::value * STAGE;
    LA[r].store(b, tid);
    LB[r].store(b + PA * GA::PLANE, tid);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // swapped MFMA order: each lane ends with 4 consecutive columns of one row
  auto compute = [&](auto buf) {
    const uint16_t* la = smem + decltype(buf)::value * STAGE;
    const uint16_t* lb = la + PA * GA::PLANE;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32)
      mma_tile<PA, PB, FM, FN, GA::STRIDE, GB::STRIDE, true>(acc, la, GA::PLANE, wm * (BM / 2), lb, GB::PLANE,
                                                             wn * (BN / 2), kk, lane);
  };
  const int64_t nk = kbeg < kend ? (kend - kbeg + BK - 1) / BK : 0;
  pipeline<STAGES>((int)nk, fetch, put, compute);

  float alpha = g.alpha, beta = g.beta;
  if (G.rowsq != nullptr) {
    if (wave == 0) {
      float s = 0.f;
      const float* rq = G.rowsq + (int64_t)b * g.rowsq_bs;
      for (int i = lane; i < g.rowsq_n; i += WAVE) s += rq[i];
      s = wave_sum(s);
      if (lane == 0) s_scale = 1.0f / (sqrtf(s) + 1e-7f);
    }
    __syncthreads();
    const float sc = s_scale;
    for (int i = 0; i < g.alpha_pow; ++i) alpha *= sc;
    for (int i = 0; i < g.beta_pow; ++i) beta *= sc;
  }
  TC* C = reinterpret_cast<TC*>(G.C) + b * g.c_bs + split * g.c_ss;
  const float* Cin = G.Cin ? G.Cin + b * g.cin_bs : nullptr;
  const bool trans = m0 >= g.trans_from;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * (BM / 2) + i * 16 + (lane & 15);
    if (m >= M) continue;
    const float am = G.rs ? alpha * silu(G.rs[(int64_t)b * g.rs_bs + m]) : alpha;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nq = n0 + wn * (BN / 2) + j * 16 + 4 * (lane >> 4);   // 4 columns nq .. nq+3
      if (nq >= g.N) continue;
      float val[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) val[r] = am * acc[i][j][r];
      if (Cin) {
        const float4 c = *reinterpret_cast<const float4*>(Cin + (int64_t)m * g.ldcin + nq);
        val[0] += beta * c.x;
        val[1] += beta * c.y;
        val[2] += beta * c.z;
        val[3] += beta * c.w;
      }
      if (trans) {
        // row m of the block is stored as column m - trans_from
#pragma unroll
        for (int r = 0; r < 4; ++r)
          io_traits<TC>::store(C + (int64_t)g.trans_from * g.ldc + (int64_t)(nq + r) * g.ldc_t + (m - g.trans_from),
                               val[r]);
      } else {
        store4(C + (int64_t)m * g.ldc + nq, val);
        if (mirror) {
#pragma unroll
          for (int r = 0; r < 4; ++r) io_traits<TC>::store(C + (int64_t)(nq + r) * g.ldc + m, val[r]);
        }
      }
    }
  }
}

// =========================================================================
// split-K reduction for the Muon path: U = sum_s P[s]; rowsq = per-row sum of
// squares of U.  One wave per row of the stacked blocks (2 dh + d rows per
// instance).
// momentum + Muon: the buffer M' = mean(beta) M - U replaces U as the
// Newton-Schulz input and is written back to the state (M[mat] in the order
// of the stacked blocks U1 | U3 | U2; null M: plain Muon)
struct RowsMomentum {
  float* M[3];
  const float* bpart;    // [n, nbp] beta partial sums
  int nbp;
  float inv_len;
};

// PO > 0: U is also stored as PO bf16 planes (plane p at Up + p * up_ps, the
// layout of U), the operand form of the plane products that follow; U (fp32)
// may then be null.
template <int PO>
__global__ __launch_bounds__(NT) void reduce_rows_kernel(const float* P, int64_t p_ss, int splits,
                                                        float* U, float* rowsq, int64_t rows, int D, int Dh,
                                                        RowsMomentum rm, bf16_t* Up, int64_t up_ps) {
  // per instance the stacked blocks U1 [dh, d], U3 [dh, d], U2 [d, dh]:
  // 2 dh + d rows, d long in the first two blocks and dh long in the third
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bool mom = rm.M[0] != nullptr;
  const int64_t DD = (int64_t)D * Dh;
  const int64_t rpi = 2 * (int64_t)Dh + D;
  const int64_t inst = row / rpi;
  const int r = (int)(row % rpi);
  const int mat = r < Dh ? 0 : r < 2 * Dh ? 1 : 2;
  const int len = mat < 2 ? D : Dh;
  const int64_t moff = mat < 2 ? (int64_t)(r - mat * Dh) * D : (int64_t)(r - 2 * Dh) * Dh;   // within the matrix
  const int64_t base = inst * 3 * DD + mat * DD + moff;
  float bm = 0.f;
  float* Mrow = nullptr;
  if (mom) {
    float sb = 0.f;
    for (int i = lane; i < rm.nbp; i += WAVE) sb += rm.bpart[inst * rm.nbp + i];
    bm = wave_sum(sb) * rm.inv_len;
    Mrow = rm.M[mat] + inst * DD + moff;
  }
  float ss = 0.f;
  for (int e4 = lane; e4 < len / 4; e4 += WAVE) {
    const float4* src = reinterpret_cast<const float4*>(P + base) + e4;
    float4 u = src[0];
    for (int s = 1; s < splits; ++s) {
      const float4 x = src[s * p_ss / 4];
      u.x += x.x;
      u.y += x.y;
      u.z += x.z;
      u.w += x.w;
    }
    if (mom) {
      const float4 m = reinterpret_cast<const float4*>(Mrow)[e4];
      u = make_float4(bm * m.x - u.x, bm * m.y - u.y, bm * m.z - u.z, bm * m.w - u.w);
      reinterpret_cast<float4*>(Mrow)[e4] = u;
    }
    if (U) reinterpret_cast<float4*>(U + base)[e4] = u;
    if constexpr (PO > 0) {
      const float uv[4] = {u.x, u.y, u.z, u.w};
      uint32_t h[4][PO];
#pragma unroll
      for (int r = 0; r < 4; ++r) split_planes<PO>(uv[r], h[r]);
#pragma unroll
      for (int p = 0; p < PO; ++p)
        *reinterpret_cast<uint2*>(Up + p * up_ps + base + 4 * e4) =
            make_uint2(h[0][p] | (h[1][p] << 16), h[2][p] | (h[3][p] << 16));
    }
    ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
  }
  ss = wave_sum(ss);
  if (lane == 0) rowsq[row] = ss;
}

// =========================================================================
// optimiser step + row renormalisation + snapshot of the new weights.
// src: per instance the stacked direction [U1; U3; U2] (three d x dh blocks
// in natural layouts: U1, U3 [dh, d], U2 [d, dh]) as `splits` partials
// summed in order.  One wave per row; a launch covers matrices mat0 ..
// mat0 + nmat - 1, which share their row count and length.
struct OptArgs {
  const void* src;       // partials (fp32, or bf16 in the plain-bf16 recurrence) or Muon's direction
  int64_t src_ss;        // elements between partials
  int splits;
  float* W[3];           // W1, W3, W2 (matching the stacked source blocks)
  float* M[3];
  const float* bpart;    // momentum: beta partial sums [n, nbp]
  int nbp;
  float inv_len;         // 1 / chunk length
  int R;                 // rows of each matrix handled (dh for W1, W3; d for W2)
  int L;                 // row length (d for W1, W3; dh for W2)
  int mat0, nmat;        // matrices mat0 .. mat0 + nmat - 1 of the stacked source
  int64_t mat_el;        // elements per matrix (d * dh)
  int rpw;               // rows per wave: 4 (L <= 256), 2 (L <= 512) or 1
  int opt;               // 0 GD, 1 momentum, 2 Muon, 3 momentum + Muon
  int renorm;
  // snapshot of the new weights (bf16 or fp32, natural layout) and, for
  // bf16, the transposed W2 snapshot used by the next update's forward
  void* snap[3];
  void* snapT2;
  // multi-plane recurrence: bf16 planes 1.. of the next update's weight
  // operands W1, W3, W2^T (plane 0 is the snapshot), [SP - 1][3][n, dh, d]
  void* wlo;
  int64_t wlo_ps, wlo_ms;
};

constexpr int OPT_MAXS = 4;               // partials loaded per batch

__host__ __device__ constexpr int opt_rpw(int L) { return L <= 256 ? 4 : L <= 512 ? 2 : 1; }

// Optimiser step, one matrix row block per workgroup.  A wave owns rpw
// consecutive rows, i.e. one contiguous span of rpw * L floats that its lanes
// cover with VPL float4 each (lane + 64 i); lanes past the span load its last
// float4 (always in bounds) and drop it, so every load is a plain 16-byte
// load issued before any arithmetic consumes it.  Row sums of squares are
// wave reductions per row.
template <typename TS, int VPL, typename TP = float, int SP = 1>
__global__ __launch_bounds__(NT) void opt_kernel(OptArgs a) {
  __shared__ uint16_t s_t[SP][4096];   // transposed-snapshot staging per plane: rows_wg x L bf16 (rows_wg * L <= 4096)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = a.L, R = a.R, rpw = a.rpw, rows_wg = 4 * rpw;
  const int rblocks = R / rows_wg;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int rb = bid % rblocks;
  bid /= rblocks;
  const int mat = a.mat0 + bid % a.nmat;
  const int inst = bid / a.nmat;
  const int64_t DD = a.mat_el;
  const int nv = L / 4;
  const int span = rpw * nv;
  const int row0 = rb * rows_wg + wave * rpw;
  const int64_t base4 = (int64_t)row0 * nv;
  const TP* src = reinterpret_cast<const TP*>(a.src) + inst * 3 * DD + mat * DD + base4 * 4;
  // four consecutive partial values as floats
  auto ldp = [](const TP* p) -> float4 {
    if constexpr (sizeof(TP) == 4) {
      return *reinterpret_cast<const float4*>(p);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      return make_float4(bf2f(v.x & 0xffffu), bf2f(v.x >> 16), bf2f(v.y & 0xffffu), bf2f(v.y >> 16));
    }
  };
  float4* W = reinterpret_cast<float4*>(a.W[mat] + inst * DD) + base4;
  float4* M = a.M[mat] ? reinterpret_cast<float4*>(a.M[mat] + inst * DD) + base4 : nullptr;
  TS* snap = a.snap[mat] ? reinterpret_cast<TS*>(a.snap[mat]) + inst * DD + base4 * 4 : nullptr;

  int ix[VPL], rid[VPL];
  bool ok[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int idx = lane + i * WAVE;
    ok[i] = idx < span;
    ix[i] = min(idx, span - 1);
    rid[i] = ix[i] / nv;
  }
  float4 u[VPL], w[VPL], m[VPL];
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    w[i] = W[ix[i]];
    m[i] = z4;
    u[i] = z4;
  }
  if (a.opt == 1) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) m[i] = M[ix[i]];
  }
  for (int s0 = 0; s0 < a.splits; s0 += OPT_MAXS) {
    float4 x[OPT_MAXS][VPL];
#pragma unroll
    for (int s = 0; s < OPT_MAXS; ++s) {
      if (s0 + s < a.splits) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) x[s][i] = ldp(src + (int64_t)(s0 + s) * a.src_ss + (int64_t)ix[i] * 4);
      } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) x[s][i] = z4;
      }
    }
#pragma unroll
    for (int s = 0; s < OPT_MAXS; ++s)   // fixed order: partial 0, 1, 2, ...
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        u[i].x += x[s][i].x;
        u[i].y += x[s][i].y;
        u[i].z += x[s][i].z;
        u[i].w += x[s][i].w;
      }
  }

  float bm = 0.f;
  if (a.opt == 1) {
    float sb = 0.f;
    for (int i = lane; i < a.nbp; i += WAVE) sb += a.bpart[(int64_t)inst * a.nbp + i];
    bm = wave_sum(sb) * a.inv_len;
  }
  float4 xn[VPL], mm[VPL];
  float so[4] = {0.f, 0.f, 0.f, 0.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (a.opt == 1) {
      mm[i] = make_float4(bm * m[i].x - u[i].x, bm * m[i].y - u[i].y, bm * m[i].z - u[i].z, bm * m[i].w - u[i].w);
      xn[i] = make_float4(w[i].x - mm[i].x, w[i].y - mm[i].y, w[i].z - mm[i].z, w[i].w - mm[i].w);
    } else if (a.opt == 3) {   // momentum + Muon: W - NS(M'), the buffer already advanced
      mm[i] = z4;
      xn[i] = make_float4(w[i].x - u[i].x, w[i].y - u[i].y, w[i].z - u[i].z, w[i].w - u[i].w);
    } else {
      mm[i] = z4;
      xn[i] = make_float4(w[i].x + u[i].x, w[i].y + u[i].y, w[i].z + u[i].z, w[i].w + u[i].w);
    }
    const float o2 = ok[i] ? w[i].x * w[i].x + w[i].y * w[i].y + w[i].z * w[i].z + w[i].w * w[i].w : 0.f;
    const float n2 = ok[i] ? xn[i].x * xn[i].x + xn[i].y * xn[i].y + xn[i].z * xn[i].z + xn[i].w * xn[i].w : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      so[r] += rid[i] == r ? o2 : 0.f;
      sn[r] += rid[i] == r ? n2 : 0.f;
    }
  }
  float scale[4] = {1.f, 1.f, 1.f, 1.f};
  if (a.renorm) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < rpw) scale[r] = sqrtf(wave_sum(so[r])) / sqrtf(wave_sum(sn[r]));
  }
  const bool stage_t = sizeof(TS) == 2 && mat == 2 && a.snapT2 != nullptr;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (!ok[i]) continue;
    const float sc = rid[i] == 0 ? scale[0] : rid[i] == 1 ? scale[1] : rid[i] == 2 ? scale[2] : scale[3];
    const float4 y = make_float4(xn[i].x * sc, xn[i].y * sc, xn[i].z * sc, xn[i].w * sc);
    W[ix[i]] = y;
    if (a.opt == 1) M[ix[i]] = mm[i];
    const float yy[4] = {y.x, y.y, y.z, y.w};
    if (snap) store4(snap + (int64_t)ix[i] * 4, yy);
    if constexpr (sizeof(TS) == 2) {
      uint32_t h[4][SP];
#pragma unroll
      for (int q = 0; q < 4; ++q) split_planes<SP>(yy[q], h[q]);
      if constexpr (SP > 1) {
        if (mat < 2) {
          uint16_t* lo = reinterpret_cast<uint16_t*>(a.wlo) + mat * a.wlo_ms + inst * DD + base4 * 4 + (int64_t)ix[i] * 4;
#pragma unroll
          for (int p = 1; p < SP; ++p)
            *reinterpret_cast<uint2*>(lo + (p - 1) * a.wlo_ps) = make_uint2(h[0][p] | (h[1][p] << 16), h[2][p] | (h[3][p] << 16));
        }
      }
      if (stage_t) {
        const int lrow = wave * rpw + rid[i];
        const int c = 4 * (ix[i] - rid[i] * nv);
#pragma unroll
        for (int p = 0; p < SP; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) s_t[p][(c + q) * rows_wg + lrow] = (uint16_t)h[q][p];
      }
    }
  }
  if constexpr (sizeof(TS) == 2) {
    if (stage_t) {
      // W2^T[j, r0 .. r0 + rows_wg - 1] (W2^T is [dh, d]: L rows of R):
      // rows_wg contiguous bf16 per j
      __syncthreads();
#pragma unroll
      for (int p = 0; p < SP; ++p) {
        uint16_t* T = (p == 0 ? reinterpret_cast<uint16_t*>(a.snapT2)
                              : reinterpret_cast<uint16_t*>(a.wlo) + (p - 1) * a.wlo_ps + 2 * a.wlo_ms) +
                      inst * DD + rb * rows_wg;
        const uint16_t* st = s_t[p];
        if (rows_wg == 4) {
          for (int j = tid; j < L; j += NT)
            *reinterpret_cast<uint2*>(T + (int64_t)j * R) = *reinterpret_cast<const uint2*>(st + j * 4);
        } else if (rows_wg == 8) {
          for (int j = tid; j < L; j += NT)
            *reinterpret_cast<uint4*>(T + (int64_t)j * R) = *reinterpret_cast<const uint4*>(st + j * 8);
        } else {
          for (int j = tid; j < L; j += NT) {
            *reinterpret_cast<uint4*>(T + (int64_t)j * R) = *reinterpret_cast<const uint4*>(st + j * 16);
            *reinterpret_cast<uint4*>(T + (int64_t)j * R + 8) = *reinterpret_cast<const uint4*>(st + j * 16 + 8);
          }
        }
      }
    }
  }
}

// =========================================================================
// q / k pre-processing ("LaCT架构核心思想解析" §1.2): each token's feature
// vector x [D] becomes silu(x) / ||silu(x)||_2 (no epsilon: a token whose
// silu is identically zero yields non-finite values, as the formula does).
// Matrix m reads src[m] (instance stride src_bs) and writes dst[m] packed as
// [n, rows, D].  A group of QP_LANES lanes owns one token row: lane l of the
// group takes the row's 16-byte chunks l, l + QP_LANES, ... (each group
// instruction covers 256 contiguous bytes), and the row's sum of squares is
// a butterfly over the group -- no LDS and no workgroup barrier, which
// measured faster than staging partial sums through LDS.
struct QkPrepArgs {
  const void* src[2];
  void* dst[2];
  int64_t src_bs;
  int64_t rows;          // tokens per instance
  int64_t total;         // nmat * n * rows
  int n;
  int D;
};

constexpr int QP_LANES = 16;

template <typename TIO>
__global__ __launch_bounds__(NT) void qk_prep_kernel(QkPrepArgs a) {
  constexpr int VE = 16 / (int)sizeof(TIO);            // elements per 16-byte chunk
  constexpr int MAXC = 1024 / VE / QP_LANES;           // chunks per lane at D = 1024
  const int gl = threadIdx.x & (QP_LANES - 1);
  const int64_t row = (int64_t)blockIdx.x * (NT / QP_LANES) + threadIdx.x / QP_LANES;
  if (row >= a.total) return;                          // whole groups leave together
  const int cpr = a.D / VE;
  const int64_t per_mat = (int64_t)a.n * a.rows;
  const int m = (int)(row / per_mat);
  const int64_t r = row % per_mat;
  const TIO* x = reinterpret_cast<const TIO*>(a.src[m]) + (r / a.rows) * a.src_bs + (r % a.rows) * a.D;
  TIO* y = reinterpret_cast<TIO*>(a.dst[m]) + r * a.D;
  float v[MAXC][VE];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = gl + i * QP_LANES;
    if (c < cpr) {
      load_chunk(x + c * VE, v[i]);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        v[i][e] = silu(v[i][e]);
        ss += v[i][e] * v[i][e];
      }
    }
  }
#pragma unroll
  for (int o = QP_LANES / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
  const float inv = 1.0f / sqrtf(ss);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = gl + i * QP_LANES;
    if (c < cpr) {
      float w[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) w[e] = v[i][e] * inv;
      store_chunk(y + c * VE, w);
    }
  }
}

// =========================================================================
// snapshot of caller weights: fp32 -> TS (natural) and, for bf16, W2^T
// SP > 1: also the weight operands' bf16 planes 1 .. SP - 1 (W1, W3 natural,
// W2^T) at wlo + (p - 1) * wlo_ps + m * wlo_ms, m = 0 W1, 1 W3, 2 W2^T.
template <typename TS, int SP = 1>
__global__ __launch_bounds__(NT) void snap_kernel(const float* W1, const float* W2, const float* W3, void* s1,
                                                   void* s2, void* s3, void* sT2, int64_t n_dd, int D, int Dh,
                                                   void* wlo, int64_t wlo_ps, int64_t wlo_ms) {
  const int64_t i4 = (int64_t)blockIdx.x * NT + threadIdx.x;   // float4 index
  if (i4 * 4 >= n_dd) return;
  const float* src[3] = {W1, W2, W3};
  void* dst[3] = {s1, s2, s3};
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const float4 x = reinterpret_cast<const float4*>(src[m])[i4];
    const float v[4] = {x.x, x.y, x.z, x.w};
    store4(reinterpret_cast<TS*>(dst[m]) + i4 * 4, v);
    if constexpr (sizeof(TS) == 2 && SP > 1) {
      if (m != 1) {   // W1 (plane set 0), W3 (plane set 1)
        uint32_t h[4][SP];
#pragma unroll
        for (int q = 0; q < 4; ++q) split_planes<SP>(v[q], h[q]);
        uint16_t* lo = reinterpret_cast<uint16_t*>(wlo) + (m == 0 ? 0 : wlo_ms) + i4 * 4;
#pragma unroll
        for (int p = 1; p < SP; ++p)
          *reinterpret_cast<uint2*>(lo + (p - 1) * wlo_ps) = make_uint2(h[0][p] | (h[1][p] << 16), h[2][p] | (h[3][p] << 16));
      }
    }
  }
  if constexpr (sizeof(TS) == 2) {
    if (sT2) {
      const float4 x = reinterpret_cast<const float4*>(W2)[i4];
      const float v[4] = {x.x, x.y, x.z, x.w};
      const int64_t e = i4 * 4;
      // W2 is [d, dh]; W2^T is [dh, d]
      const int64_t DD = (int64_t)D * Dh;
      const int64_t inst = e / DD, rem = e % DD;
      const int r = (int)(rem / Dh), c = (int)(rem % Dh);
      uint16_t* T = reinterpret_cast<uint16_t*>(sT2) + inst * DD;
      uint32_t h[4][SP];
#pragma unroll
      for (int q = 0; q < 4; ++q) split_planes<SP>(v[q], h[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q) T[(int64_t)(c + q) * D + r] = (uint16_t)h[q][0];
      if constexpr (SP > 1) {
        uint16_t* TL = reinterpret_cast<uint16_t*>(wlo) + 2 * wlo_ms + inst * DD;
#pragma unroll
        for (int p = 1; p < SP; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) TL[(p - 1) * wlo_ps + (int64_t)(c + q) * D + r] = (uint16_t)h[q][p];
      }
    }
  }
}

}  // namespace lact
