// gfx950 kernels of the LaCT fast-weight layer forward.
//
//   fwd_kernel   -- per (instance, 128-token block, 64-column block) tile:
//                   apply tiles compute Aq = Q W1^T, Bq = Q W3^T and store
//                   Hq = silu(Aq) * Bq; update tiles compute A = K W1^T,
//                   B = K W3^T, G = V W2 and store the SwiGLU backward terms
//                   lr1*G*B*silu'(A), lr3*G*silu(A), lr2*silu(A)*B
//                   ("大块测试时训练（LaCT）技术解析" §2.1, eqs. 2 and 4-5).
//   gemm_kernel  -- batched C = alpha*A B^T + beta*Cin with fp32 output and
//                   optional split over K (the weight-gradient contraction
//                   over the chunk's tokens, the apply output product and the
//                   Newton-Schulz products).
//   reduce_rows_kernel -- sums split-K partials, emits per-row sums of squares.
//   opt_kernel   -- GD / momentum / Muon step and row L2 renormalisation
//                   ("大块测试时训练（LaCT）技术解析" §2.2.1 eq. 8;
//                   "LaCT架构核心思想解析" §1.2).
#pragma once
#include "lact_device.hpp"

namespace lact {

constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr int BK = 32;    // k per LDS stage (one MFMA k-slice)

// =========================================================================
// fused forward tiles
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t x_bs;          // elements between instances in q/k/v (seq_stride * D)
  const float* lr;
  int64_t lr_bs;         // seq_stride * 3
  const float* W1;
  const float* W2;
  const float* W3;
  void* E;               // [n, upd_len, 3D] update terms (token rows relative to upd_t0)
  int64_t e_bs;
  void* H;               // [n, app_len, D] gated hidden of the queries
  int64_t h_bs;
  int D;
  int64_t upd_t0;
  int64_t upd_len;
  int64_t app_t0;
  int64_t app_len;
  int upd_tiles;         // per instance
  int app_tiles;
};

constexpr int FBT = 128;  // tokens per forward tile
constexpr int FBJ = 64;   // hidden columns per forward tile

template <typename TIO, int PIO, int PWU, int PWA, typename TREC, typename TAPP>
__global__ __launch_bounds__(NT) void fwd_kernel(FwdArgs a) {
  using G_T = TileGeom<FBT, BK>;
  using G_J = TileGeom<FBJ, BK>;
  constexpr int UPD_LDS = 2 * PIO * G_T::PLANE + 3 * PWU * G_J::PLANE;
  constexpr int APP_LDS = PIO * G_T::PLANE + 2 * PWA * G_J::PLANE;
  constexpr int LDS = UPD_LDS > APP_LDS ? UPD_LDS : APP_LDS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;        // 2x2 waves: 64 tokens x 32 columns each
  const int D = a.D;
  const int njb = D / FBJ;
  const int per_inst = a.upd_tiles + a.app_tiles;
  const int inst = blockIdx.x / per_inst;
  const int tile = blockIdx.x % per_inst;
  const float* W1 = a.W1 + (int64_t)inst * D * D;
  const float* W2 = a.W2 + (int64_t)inst * D * D;
  const float* W3 = a.W3 + (int64_t)inst * D * D;

  if (tile < a.upd_tiles) {
    // ------------------------------------------------------------ update tile
    const int tb = tile / njb, jb = tile % njb;
    const int64_t t0 = a.upd_t0 + (int64_t)tb * FBT;
    const int64_t tend = a.upd_t0 + a.upd_len;
    const int j0 = jb * FBJ;
    const TIO* K = reinterpret_cast<const TIO*>(a.k) + inst * a.x_bs;
    const TIO* V = reinterpret_cast<const TIO*>(a.v) + inst * a.x_bs;
    uint16_t* lK = smem;
    uint16_t* lV = lK + PIO * G_T::PLANE;
    uint16_t* l1 = lV + PIO * G_T::PLANE;
    uint16_t* l3 = l1 + PWU * G_J::PLANE;
    uint16_t* l2 = l3 + PWU * G_J::PLANE;
    RowKLoader<TIO, PIO, FBT, BK, NT> LK, LV;
    RowKLoader<float, PWU, FBJ, BK, NT> L1, L3;
    ColKLoader<float, PWU, FBJ, BK, NT> L2;
    f32x4 accA[4][2], accB[4][2], accG[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) accA[i][j] = accB[i][j] = accG[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto fetch = [&](int k0) {
      LK.load(K, D, t0, tend, k0, tid);
      LV.load(V, D, t0, tend, k0, tid);
      L1.load(W1, D, j0, D, k0, tid);
      L3.load(W3, D, j0, D, k0, tid);
      L2.load(W2, D, j0, D, k0, D, tid);   // element (j, r) = W2[r, j]
    };
    fetch(0);
    for (int k0 = 0; k0 < D; k0 += BK) {
      __syncthreads();
      LK.store(lK, tid);
      LV.store(lV, tid);
      L1.store(l1, tid);
      L3.store(l3, tid);
      L2.store(l2, tid);
      __syncthreads();
      if (k0 + BK < D) fetch(k0 + BK);
      mma_tile<PIO, PWU, 4, 2, G_T::STRIDE, G_J::STRIDE>(accA, lK, G_T::PLANE, wm * 64, l1, G_J::PLANE, wn * 32, 0, lane);
      mma_tile<PIO, PWU, 4, 2, G_T::STRIDE, G_J::STRIDE>(accB, lK, G_T::PLANE, wm * 64, l3, G_J::PLANE, wn * 32, 0, lane);
      mma_tile<PIO, PWU, 4, 2, G_T::STRIDE, G_J::STRIDE>(accG, lV, G_T::PLANE, wm * 64, l2, G_J::PLANE, wn * 32, 0, lane);
    }
    // SwiGLU backward epilogue in registers
    TREC* E = reinterpret_cast<TREC*>(a.E) + inst * a.e_bs;
    const float* lr = a.lr + inst * a.lr_bs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (t >= tend) continue;
        const float e1 = lr[t * 3 + 0], e2 = lr[t * 3 + 1], e3 = lr[t * 3 + 2];
        TREC* Er = E + (t - a.upd_t0) * (3 * (int64_t)D);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = j0 + wn * 32 + j * 16 + (lane & 15);
          const float x = accA[i][j][r], b = accB[i][j][r], g = accG[i][j][r];
          const float sg = fast_sigmoid(x);
          const float s = x * sg;
          const float sp = sg * (1.0f + x * (1.0f - sg));
          io_traits<TREC>::store(Er + col, e1 * g * b * sp);
          io_traits<TREC>::store(Er + D + col, e3 * g * s);
          io_traits<TREC>::store(Er + 2 * D + col, e2 * s * b);
        }
      }
    }
  } else {
    // ------------------------------------------------------------ apply tile
    const int at = tile - a.upd_tiles;
    const int tb = at / njb, jb = at % njb;
    const int64_t t0 = a.app_t0 + (int64_t)tb * FBT;
    const int64_t tend = a.app_t0 + a.app_len;
    const int j0 = jb * FBJ;
    const TIO* Q = reinterpret_cast<const TIO*>(a.q) + inst * a.x_bs;
    uint16_t* lQ = smem;
    uint16_t* l1 = lQ + PIO * G_T::PLANE;
    uint16_t* l3 = l1 + PWA * G_J::PLANE;
    RowKLoader<TIO, PIO, FBT, BK, NT> LQ;
    RowKLoader<float, PWA, FBJ, BK, NT> L1, L3;
    f32x4 accA[4][2], accB[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) accA[i][j] = accB[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto fetch = [&](int k0) {
      LQ.load(Q, D, t0, tend, k0, tid);
      L1.load(W1, D, j0, D, k0, tid);
      L3.load(W3, D, j0, D, k0, tid);
    };
    fetch(0);
    for (int k0 = 0; k0 < D; k0 += BK) {
      __syncthreads();
      LQ.store(lQ, tid);
      L1.store(l1, tid);
      L3.store(l3, tid);
      __syncthreads();
      if (k0 + BK < D) fetch(k0 + BK);
      mma_tile<PIO, PWA, 4, 2, G_T::STRIDE, G_J::STRIDE>(accA, lQ, G_T::PLANE, wm * 64, l1, G_J::PLANE, wn * 32, 0, lane);
      mma_tile<PIO, PWA, 4, 2, G_T::STRIDE, G_J::STRIDE>(accB, lQ, G_T::PLANE, wm * 64, l3, G_J::PLANE, wn * 32, 0, lane);
    }
    TAPP* H = reinterpret_cast<TAPP*>(a.H) + inst * a.h_bs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (t >= tend) continue;
        TAPP* Hr = H + (t - a.app_t0) * (int64_t)D;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = j0 + wn * 32 + j * 16 + (lane & 15);
          const float x = accA[i][j][r];
          io_traits<TAPP>::store(Hr + col, x * fast_sigmoid(x) * accB[i][j][r]);
        }
      }
    }
  }
}

// =========================================================================
// generic batched GEMM:  C[m, n] = alpha * sum_k A(m, k) B(n, k) + beta * Cin[m, n]
//   A(m, k): row-k source A[m * lda + k]   or column-k source A[k * lda + m]
//   B(n, k): row-k source B[n * ldb + k]   or column-k source B[k * ldb + n]
// K may be split over gridDim: split s covers k in [s*kps, min(K, (s+1)*kps))
// and writes its own partial C + s * c_ss.
struct GemmArgs {
  const void* A;
  int64_t lda, a_bs;
  const void* B;
  int64_t ldb, b_bs;
  const void* B2;        // B operand for m-tiles at or beyond m_switch (else unused)
  int m_switch;
  void* C;
  int64_t ldc, c_bs, c_ss;
  const float* Cin;
  int64_t ldcin, cin_bs;
  int M, N;
  int64_t K, kps;
  int batch, splits;
  float alpha, beta;
  // optional scale s = 1 / (sqrt(sum of rowsq[b * rowsq_n ...]) + 1e-7):
  // alpha *= s^alpha_pow, beta *= s^beta_pow
  const float* rowsq;
  int rowsq_n, alpha_pow, beta_pow;
};

template <typename TA, int PA, bool CA, typename TB, int PB, bool CB, typename TC, int BM, int BN>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs g) {
  using GA = TileGeom<BM, BK>;
  using GB = TileGeom<BN, BK>;
  constexpr int FM = BM / 32, FN = BN / 32;     // 2x2 waves, wave tile (BM/2) x (BN/2)
  __shared__ __attribute__((aligned(16))) uint16_t smem[PA * GA::PLANE + PB * GB::PLANE];
  __shared__ float s_scale;
  uint16_t* lA = smem;
  uint16_t* lB = smem + PA * GA::PLANE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn_count = (g.N + BN - 1) / BN;
  const int tm_count = (g.M + BM - 1) / BM;
  const int tiles = tm_count * tn_count;
  int bid = blockIdx.x;
  const int tile = bid % tiles;
  bid /= tiles;
  const int split = bid % g.splits;
  const int b = bid / g.splits;
  const int tm = tile / tn_count, tn = tile % tn_count;
  const int m0 = tm * BM, n0 = tn * BN;

  const TA* A = reinterpret_cast<const TA*>(g.A) + b * g.a_bs;
  const void* Bsrc = (g.B2 != nullptr && m0 >= g.m_switch) ? g.B2 : g.B;
  const TB* B = reinterpret_cast<const TB*>(Bsrc) + b * g.b_bs;
  const int64_t kbeg = (int64_t)split * g.kps;
  const int64_t kend = min(g.K, kbeg + g.kps);

  typename LoaderSel<TA, PA, BM, BK, NT, CA>::type LA;
  typename LoaderSel<TB, PB, BN, BK, NT, CB>::type LB;
  auto fetch = [&](int64_t k0) {
    if constexpr (CA) LA.load(A, g.lda, m0, g.M, k0, kend, tid);
    else LA.load(A, g.lda, m0, g.M, k0, tid);
    if constexpr (CB) LB.load(B, g.ldb, n0, g.N, k0, kend, tid);
    else LB.load(B, g.ldb, n0, g.N, k0, tid);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kbeg < kend) fetch(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    LA.store(lA, tid);
    LB.store(lB, tid);
    __syncthreads();
    if (k0 + BK < kend) fetch(k0 + BK);
    mma_tile<PA, PB, FM, FN, GA::STRIDE, GB::STRIDE>(acc, lA, GA::PLANE, wm * (BM / 2), lB, GB::PLANE,
                                                     wn * (BN / 2), 0, lane);
  }

  float alpha = g.alpha, beta = g.beta;
  if (g.rowsq != nullptr) {
    if (wave == 0) {
      float s = 0.f;
      const float* rq = g.rowsq + (int64_t)b * g.rowsq_n;
      for (int i = lane; i < g.rowsq_n; i += WAVE) s += rq[i];
      s = wave_sum(s);
      if (lane == 0) s_scale = 1.0f / (sqrtf(s) + 1e-7f);
    }
    __syncthreads();
    const float sc = s_scale;
    for (int i = 0; i < g.alpha_pow; ++i) alpha *= sc;
    for (int i = 0; i < g.beta_pow; ++i) beta *= sc;
  }
  TC* C = reinterpret_cast<TC*>(g.C) + b * g.c_bs + split * g.c_ss;
  const float* Cin = g.Cin ? g.Cin + b * g.cin_bs : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4) + r;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
        if (n >= g.N) continue;
        float val = alpha * acc[i][j][r];
        if (Cin) val += beta * Cin[(int64_t)m * g.ldcin + n];
        io_traits<TC>::store(C + (int64_t)m * g.ldc + n, val);
      }
    }
}

// =========================================================================
// split-K reduction for the Muon path: U = sum_s P[s]; rowsq = per-row sum of
// squares of U.  One wave per row of the stacked [n * 3D, D] matrix.
__global__ __launch_bounds__(NT) void reduce_rows_kernel(const float* P, int64_t p_ss, int splits,
                                                        float* U, float* rowsq, int64_t rows, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  if (row >= rows) return;
  float ss = 0.f;
  for (int e = lane; e < D; e += WAVE) {
    float u = 0.f;
    for (int s = 0; s < splits; ++s) u += P[s * p_ss + row * D + e];
    U[row * D + e] = u;
    ss += u * u;
  }
  ss = wave_sum(ss);
  if (lane == 0) rowsq[row] = ss;
}

// =========================================================================
// optimiser step + row renormalisation.
// src holds, per instance, the stacked direction [U1; U3; U2^T] ([3D, D]) as
// `splits` partials to be summed in order.  Workgroup = 16 rows of one matrix.
struct OptArgs {
  const float* src;
  int64_t src_ss;        // elements between partials
  int splits;
  float* W[3];           // W1, W3, W2 (matching the stacked source blocks)
  float* M[3];
  const float* beta;     // momentum only
  int64_t beta_bs;
  int64_t beta_t0;
  int64_t beta_len;
  int D;
  int opt;               // 0 GD, 1 momentum, 2 Muon
  int renorm;
};

constexpr int OPT_ROWS = 16;
constexpr int OPT_MAXPL = 16;   // D / 64 elements per lane, D <= 1024

__global__ __launch_bounds__(NT) void opt_kernel(OptArgs a) {
  __shared__ float s_src[1024 * (OPT_ROWS + 1)];
  __shared__ float s_red[NT / WAVE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.D;
  const int rblocks = D / OPT_ROWS;
  int bid = blockIdx.x;
  const int rb = bid % rblocks;
  bid /= rblocks;
  const int mat = bid % 3;
  const int inst = bid / 3;
  const int r0 = rb * OPT_ROWS;
  const int64_t DD = (int64_t)D * D;
  const float* src = a.src + inst * 3 * DD + mat * DD;

  float bm = 0.f;
  if (a.opt == 1) {
    const float* bt = a.beta + inst * a.beta_bs + a.beta_t0;
    float s = 0.f;
    for (int64_t i = tid; i < a.beta_len; i += NT) s += bt[i];
    s = wave_sum(s);
    if (lane == 0) s_red[wave] = s;
    __syncthreads();
    bm = (s_red[0] + s_red[1] + s_red[2] + s_red[3]) / (float)a.beta_len;
  }
  if (mat == 2) {
    // W2 row r is column r of the transposed block: stage 16 columns in LDS
    for (int idx = tid; idx < D * OPT_ROWS; idx += NT) {
      const int j = idx / OPT_ROWS, rr = idx % OPT_ROWS;
      float u = 0.f;
      for (int s = 0; s < a.splits; ++s) u += src[s * a.src_ss + (int64_t)j * D + r0 + rr];
      s_src[j * (OPT_ROWS + 1) + rr] = u;
    }
    __syncthreads();
  }
  float* W = a.W[mat] + inst * DD;
  float* M = a.M[mat] ? a.M[mat] + inst * DD : nullptr;
  for (int rr = wave; rr < OPT_ROWS; rr += NT / WAVE) {
    const int row = r0 + rr;
    float wn[OPT_MAXPL];
    float so = 0.f, sn = 0.f;
#pragma unroll
    for (int i = 0; i < OPT_MAXPL; ++i) {
      const int e = lane + i * WAVE;
      if (e >= D) continue;
      float u;
      if (mat == 2) {
        u = s_src[e * (OPT_ROWS + 1) + rr];
      } else {
        u = 0.f;
        for (int s = 0; s < a.splits; ++s) u += src[s * a.src_ss + (int64_t)row * D + e];
      }
      const float w = W[(int64_t)row * D + e];
      float x;
      if (a.opt == 1) {
        const float m = bm * M[(int64_t)row * D + e] - u;
        M[(int64_t)row * D + e] = m;
        x = w - m;
      } else {
        x = w + u;
      }
      wn[i] = x;
      so += w * w;
      sn += x * x;
    }
    float scale = 1.f;
    if (a.renorm) {
      so = wave_sum(so);
      sn = wave_sum(sn);
      scale = sqrtf(so) / sqrtf(sn);
    }
#pragma unroll
    for (int i = 0; i < OPT_MAXPL; ++i) {
      const int e = lane + i * WAVE;
      if (e < D) W[(int64_t)row * D + e] = wn[i] * scale;
    }
  }
}

}  // namespace lact
