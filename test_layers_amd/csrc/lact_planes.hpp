// Products whose fp32 operands are stored as bf16 planes.
//
// An fp32 matrix X is kept as P bf16 planes X = X_0 + X_1 (+ X_2), each plane
// the round-to-nearest-even bf16 of what the earlier planes leave (the
// precision model of lact_device.hpp).  A producer writes the planes of its
// result once, in its epilogue; every consumer then streams them with gfx950's
// direct global->LDS loads, like plain bf16 data, instead of splitting fp32
// values in registers on every load.  A product sums the plane pairs (i, j)
// with i + j < max(P_A, P_B), the pairs of smaller weight first.
//
// Used for the Newton-Schulz orthogonalisation of the chunk gradient
// ("大块测试时训练（LaCT）技术解析" §2.2.1, eqs. 9-10): per step
// A = X X^T, B = b A + c A A, X <- a X + B X, on every fast-weight matrix of
// every instance at once.
#pragma once
#include "lact_direct.hpp"

namespace lact {

// Tile shape of a plane product: BM x BN outputs per workgroup, k stages of
// BK, waves laid out WGM x WGN over the tile and KS ways over each stage's k
// (KS = 2: two waves share a quadrant, each takes half of every stage, and
// their sums meet in LDS at the end), NST-deep direct-load ring.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int KS_, int NST_>
struct PgShape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, KS = KS_, NST = NST_;
  static constexpr int NW = WGM * WGN * KS;
  static constexpr int THREADS = NW * WAVE;
  static constexpr int FM = BM / WGM / 16, FN = BN / WGN / 16;   // 16 x 16 fragments per wave
  static constexpr int KW = BK / KS;                             // k of a stage per wave
  static_assert(FM >= 1 && FN >= 1 && KW % 32 == 0, "wave tile");
};

// C[m, n] = alpha * sum_k A(m, k) B(n, k) + beta * Cin[m, n]  (GemmArgs contract)
//   A(m, k) = A[m * lda + k]: PA bf16 planes, plane p at A + p * a_ps;
//   B(n, k) = B[n * ldb + k] (row-k) or B[k * ldb + n] (CB, column-k: read
//   with transposing LDS reads), PB planes at B + p * b_ps;
//   C fp32 (optional, G.C) and its PO bf16 planes (optional, G.Cp, plane p at
//   Cp + p * cp_ps), both with row stride ldc.
// Symmetric results (g.sym): only the tiles on or above the diagonal run, and
// an off-diagonal tile also stores its mirror image, staged through LDS so
// that the mirrored rows are written as whole 16-byte pieces.  M, N are
// multiples of the tile, K of BK (the callers' square matrices); one split.
template <int PA, int PB, bool CB, int PO, class S>
__global__ __launch_bounds__(S::THREADS) void pgemm_kernel(GemmArgs g) {
  constexpr int BM = S::BM, BN = S::BN, BK = S::BK, NW = S::NW, FM = S::FM, FN = S::FN, KS = S::KS;
  using TA = DTile<BM, BK, NW>;
  using TB = typename std::conditional<CB, DTile<BK, BN, NW, true>, DTile<BN, BK, NW>>::type;
  constexpr int STAGE = PA * TA::BYTES + PB * TB::BYTES;
  constexpr int LPS = PA * TA::INSTR + PB * TB::INSTR;
  constexpr int PM = PA > PB ? PA : PB;
  constexpr int EST = BN + 4;                                  // fp32 staging row stride
  constexpr int EPI = BM * EST * 4;
  constexpr int RED = (KS > 1 ? (NW / KS) * FM * FN * 256 * 4 : 0);   // k-split reduction
  constexpr int SMEM0 = S::NST * STAGE > EPI ? S::NST * STAGE : EPI;
  constexpr int SMEM = SMEM0 > RED ? SMEM0 : RED;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ float s_scale;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quad = wave % (S::WGM * S::WGN), ks = wave / (S::WGM * S::WGN);
  const int wm = quad / S::WGN, wn = quad % S::WGN;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < g.ngroups && bid >= g.g[gi].tiles) bid -= g.g[gi++].tiles;
  const GemmGroup& G = g.g[gi];
  const int M = G.M;
  const int tn_count = g.N / BN;
  const int tiles = g.sym ? tn_count * (tn_count + 1) / 2 : (M / BM) * tn_count;
  const int tile = bid % tiles;
  const int b = bid / tiles;
  int tm = tile / tn_count, tn = tile % tn_count;
  if (g.sym) {   // upper triangle, row by row: row tm holds tiles tn = tm .. tn_count - 1
    int rem = tile;
    tm = 0;
    while (rem >= tn_count - tm) rem -= tn_count - tm++;
    tn = tm + rem;
  }
  const bool mirror = g.sym && tn != tm;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t* A = reinterpret_cast<const bf16_t*>(G.A) + b * g.a_bs;
  const bf16_t* B = reinterpret_cast<const bf16_t*>(G.B) + b * g.b_bs;
  const int nk = (int)(g.K / BK);
  typename TA::Plan pa[PA];
  typename TB::Plan pb[PB];
#pragma unroll
  for (int p = 0; p < PA; ++p) pa[p] = TA::plan(A + p * g.a_ps, g.lda, m0, M - 1, 0, wave, lane);
#pragma unroll
  for (int p = 0; p < PB; ++p)
    pb[p] = CB ? TB::plan(B + p * g.b_ps, g.ldb, 0, g.K - 1, n0, wave, lane)
               : TB::plan(B + p * g.b_ps, g.ldb, n0, g.N - 1, 0, wave, lane);
  const int64_t sa = (int64_t)BK * 2;
  const int64_t sb = CB ? (int64_t)BK * g.ldb * 2 : (int64_t)BK * 2;
  auto issue_one = [&](int s, int buf, int idx) {
    char* st = smem + buf * STAGE;
#pragma unroll
    for (int p = 0; p < PA; ++p)
#pragma unroll
      for (int i = 0; i < TA::INSTR; ++i)
        if (idx == p * TA::INSTR + i) TA::issue_one(st + p * TA::BYTES, pa[p], s * sa, wave, i);
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int i = 0; i < TB::INSTR; ++i)
        if (idx == PA * TA::INSTR + p * TB::INSTR + i)
          TB::issue_one(st + PA * TA::BYTES + p * TB::BYTES, pb[p], s * sb, wave, i);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, auto&& hook) {
    const char* st = smem + buf * STAGE;
    constexpr int NK32 = S::KW / 32;
#pragma unroll
    for (int t = 0; t < NK32; ++t) {
      const int kk = ks * S::KW + t * 32;
      bf16x8 af[PA][FM], bfr[PB][FN];
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i) af[p][i] = dfrag_row<TA>(st + p * TA::BYTES, wm * (BM / S::WGM) + i * 16, kk, lane);
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[p][j] = dfrag<TB, CB>(st + PA * TA::BYTES + p * TB::BYTES, wn * (BN / S::WGN) + j * 16, kk, lane);
      // plane pairs of smaller weight first; the next stage's loads are
      // spread over the groups of equal weight
#pragma unroll
      for (int sp = PM - 1; sp >= 0; --sp) {
#pragma unroll
        for (int p = 0; p < PA; ++p)
#pragma unroll
          for (int q = 0; q < PB; ++q)
            if (p + q == sp)
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma(bfr[q][j], af[p][i], acc[i][j]);
        hook(t * PM + PM - 1 - sp, NK32 * PM);
      }
    }
  };
  dpipeline_il<S::NST, LPS>(nk, issue_one, compute);

  if constexpr (KS > 1) {
    // sum the k slices in fixed order (slice 0 + slice 1 + ...)
    bar();
    float* red = reinterpret_cast<float*>(smem);
    for (int r = 1; r < KS; ++r) {
      if (ks == r) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            *reinterpret_cast<f32x4*>(red + ((quad * FM + i) * FN + j) * 256 + lane * 4) = acc[i][j];
      }
      bar();
      if (ks == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] += *reinterpret_cast<const f32x4*>(red + ((quad * FM + i) * FN + j) * 256 + lane * 4);
      }
      bar();
    }
  }

  float alpha = g.alpha, beta = g.beta;
  if (G.rowsq != nullptr) {
    if (wave == 0) {
      float sq = 0.f;
      const float* rq = G.rowsq + (int64_t)b * g.rowsq_bs;
      for (int i = lane; i < g.rowsq_n; i += WAVE) sq += rq[i];
      sq = wave_sum(sq);
      if (lane == 0) s_scale = 1.0f / (sqrtf(sq) + 1e-7f);
    }
    __syncthreads();
    const float sc = s_scale;
    for (int i = 0; i < g.alpha_pow; ++i) alpha *= sc;
    for (int i = 0; i < g.beta_pow; ++i) beta *= sc;
  }
  float* C = G.C ? reinterpret_cast<float*>(G.C) + b * g.c_bs : nullptr;
  bf16_t* Cp = G.Cp ? reinterpret_cast<bf16_t*>(G.Cp) + b * g.c_bs : nullptr;
  const float* Cin = G.Cin ? G.Cin + b * g.cin_bs : nullptr;
  const bf16_t* Cinp = G.Cinp ? reinterpret_cast<const bf16_t*>(G.Cinp) + b * g.cin_bs : nullptr;

  // The tile goes through LDS (fp32, row = m) so that every store covers
  // whole rows: 16 bytes of fp32 or 8 bytes per bf16 plane per lane, lanes
  // side by side along the row; a mirrored tile is read back by columns.
  if (KS == 1) bar();   // every wave is done reading the ring (KS > 1: the reduction ended with one)
  float* stg = reinterpret_cast<float*>(smem);
  if (ks == 0) {
    // swapped MFMA order: lane holds row lane % 16 of a fragment, columns 4 (lane / 16) .. +3
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int ml = wm * (BM / S::WGM) + i * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int nl = wn * (BN / S::WGN) + j * 16 + 4 * (lane >> 4);
        *reinterpret_cast<float4*>(stg + ml * EST + nl) =
            make_float4(alpha * acc[i][j][0], alpha * acc[i][j][1], alpha * acc[i][j][2], alpha * acc[i][j][3]);
      }
    }
  }
  bar();
  // v (4 consecutive values of row m, columns n .. n + 3) plus beta Cin, stored
  auto emit = [&](int64_t m, int64_t n, float (&v)[4]) {
    const int64_t off = m * g.ldc + n;
    if (Cin) {
      const float4 c = *reinterpret_cast<const float4*>(Cin + m * g.ldcin + n);
      v[0] += beta * c.x;
      v[1] += beta * c.y;
      v[2] += beta * c.z;
      v[3] += beta * c.w;
    } else if constexpr (PO > 0) {
      if (Cinp) {
        float c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = PO - 1; p >= 0; --p) {   // smaller planes first
          const uint2 h = *reinterpret_cast<const uint2*>(Cinp + p * g.cp_ps + m * g.ldcin + n);
          c[0] += bf2f(h.x & 0xffffu);
          c[1] += bf2f(h.x >> 16);
          c[2] += bf2f(h.y & 0xffffu);
          c[3] += bf2f(h.y >> 16);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += beta * c[r];
      }
    }
    if (C) store4(C + off, v);
    if constexpr (PO > 0) {
      if (Cp) {
        uint32_t h[4][PO];
#pragma unroll
        for (int r = 0; r < 4; ++r) split_planes<PO>(v[r], h[r]);
#pragma unroll
        for (int p = 0; p < PO; ++p)
          *reinterpret_cast<uint2*>(Cp + p * g.cp_ps + off) = make_uint2(h[0][p] | (h[1][p] << 16), h[2][p] | (h[3][p] << 16));
      }
    }
  };
  constexpr int QN = BN / 4, QM = BM / 4;
  for (int qd = tid; qd < BM * QN; qd += S::THREADS) {
    const int r = qd / QN, c = (qd % QN) * 4;
    const float4 x = *reinterpret_cast<const float4*>(stg + r * EST + c);
    float v[4] = {x.x, x.y, x.z, x.w};
    emit(m0 + r, n0 + c, v);
  }
  if (!mirror) return;
  // mirrored tile: C[n0 + r, m0 + c .. +3] = staged[m = c .. c + 3][n = r]
  for (int qd = tid; qd < BN * QM; qd += S::THREADS) {
    const int r = qd / QM, c = (qd % QM) * 4;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = stg[(c + e) * EST + r];
    emit(n0 + r, m0 + c, v);
  }
}

// the shapes in use
using PgSmall = PgShape<64, 64, 32, 2, 2, 1, 3>;     // 4 waves, 32 x 32 each
using PgLarge = PgShape<128, 128, 64, 2, 2, 2, 2>;   // 8 waves, 64 x 64 each over half of every stage

}  // namespace lact
