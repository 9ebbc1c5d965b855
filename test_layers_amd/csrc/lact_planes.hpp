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
  // the epilogue's input-term planes (beta Cin), loaded before the main loop
  // so that their latency hides behind it: the quads (row, 4 columns) of the
  // tile and, for a mirrored symmetric tile, of its mirror, as the epilogue
  // visits them
  constexpr int QN = BN / 4, QM = BM / 4;
  constexpr int QPT = BM * QN / S::THREADS, QPM = BN * QM / S::THREADS;
  static_assert(BM * QN % S::THREADS == 0 && BN * QM % S::THREADS == 0, "epilogue quads per thread");
  constexpr int PP = PO > 0 ? PO : 1;
  uint2 cpre[QPT][PP], cprm[QPM][PP];
  const bf16_t* Cinp =
      (PO > 0 && G.Cinp && !G.Cin) ? reinterpret_cast<const bf16_t*>(G.Cinp) + b * g.cin_bs : nullptr;
  if constexpr (PO > 0) {
    if (Cinp) {
#pragma unroll
      for (int q = 0; q < QPT; ++q) {
        const int qd = tid + q * S::THREADS;
        const int64_t off = (int64_t)(m0 + qd / QN) * g.ldcin + n0 + (qd % QN) * 4;
#pragma unroll
        for (int p = 0; p < PO; ++p) cpre[q][p] = *reinterpret_cast<const uint2*>(Cinp + p * g.cp_ps + off);
      }
      if (mirror) {
#pragma unroll
        for (int q = 0; q < QPM; ++q) {
          const int qd = tid + q * S::THREADS;
          const int64_t off = (int64_t)(n0 + qd / QM) * g.ldcin + m0 + (qd % QM) * 4;
#pragma unroll
          for (int p = 0; p < PO; ++p) cprm[q][p] = *reinterpret_cast<const uint2*>(Cinp + p * g.cp_ps + off);
        }
      }
    }
  }

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
      wait_lgkm0();   // slice r's sums are in LDS before wave set 0 reads them
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
  wait_lgkm0();   // the staged tile is in LDS before other waves read it back
  bar();
  // beta times the value held in the prefetched planes h, added to v
  auto add_planes = [&](const uint2 (&h)[PP], float (&v)[4]) {
    float c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = PO - 1; p >= 0; --p) {   // smaller planes first
      c[0] += bf2f(h[p].x & 0xffffu);
      c[1] += bf2f(h[p].x >> 16);
      c[2] += bf2f(h[p].y & 0xffffu);
      c[3] += bf2f(h[p].y >> 16);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += beta * c[r];
  };
  // v (4 consecutive values of row m, columns n .. n + 3) plus beta Cin
  // (fp32 input; plane input already added), stored
  auto emit = [&](int64_t m, int64_t n, float (&v)[4]) {
    const int64_t off = m * g.ldc + n;
    if (Cin) {
      const float4 c = *reinterpret_cast<const float4*>(Cin + m * g.ldcin + n);
      v[0] += beta * c.x;
      v[1] += beta * c.y;
      v[2] += beta * c.z;
      v[3] += beta * c.w;
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
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int qd = tid + q * S::THREADS;
    const int r = qd / QN, c = (qd % QN) * 4;
    const float4 x = *reinterpret_cast<const float4*>(stg + r * EST + c);
    float v[4] = {x.x, x.y, x.z, x.w};
    if constexpr (PO > 0)
      if (Cinp) add_planes(cpre[q], v);
    emit(m0 + r, n0 + c, v);
  }
  if (!mirror) return;
  // mirrored tile: C[n0 + r, m0 + c .. +3] = staged[m = c .. c + 3][n = r]
#pragma unroll
  for (int q = 0; q < QPM; ++q) {
    const int qd = tid + q * S::THREADS;
    const int r = qd / QM, c = (qd % QM) * 4;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = stg[(c + e) * EST + r];
    if constexpr (PO > 0)
      if (Cinp) add_planes(cprm[q], v);
    emit(n0 + r, m0 + c, v);
  }
}

// the shapes in use
using PgSmall = PgShape<64, 64, 32, 2, 2, 1, 3>;     // 4 waves, 32 x 32 each
using PgLarge = PgShape<128, 128, 64, 2, 2, 2, 2>;   // 8 waves, 64 x 64 each over half of every stage

}  // namespace lact

namespace lact {

// =========================================================================
// Newton-Schulz of small square matrices (d = dh <= 128) in one workgroup
// per matrix: the iterate X and the Gram / polynomial matrix live in LDS as
// fp32 for all ns_iters steps, so the fifteen products of a chunk's
// orthogonalisation need no launch, no global round trip and no grid-wide
// synchronisation.  Each 32-wide k slice of an operand that all waves read
// is split once into P bf16 planes in LDS (the B X product's B rows, read by
// two waves each, are split in registers by those waves); every product sums
// the plane pairs (i, j) with i + j < P, smaller pairs first (fp32 grade at
// P = 3).
//   X0 = U / (||U||_F + 1e-7);  per step:  A = X X^T,  B = b A + c A A,
//   X <- a X + B X  ("大块测试时训练（LaCT）技术解析" §2.2.1, eqs. 9-10).
// U: [nmat, D, D] fp32, rowsq: [nmat, D] per-row sums of squares of U
// (the Frobenius norm), out: [nmat, D, D] fp32.
template <int D>
struct NsSmall {
  static constexpr int NW = D == 128 ? 8 : 4;   // waves: 4 x 2 (D = 128) or 2 x 2 over the output
  static constexpr int THREADS = NW * WAVE;
  static constexpr int WGN = 2, WGM = NW / 2;
  static constexpr int FM = D / WGM / 16, FN = D / WGN / 16;
  static constexpr int PITCH = D + 4;            // fp32 row pitch (16-byte row reads conflict-free)
  static constexpr int SLOT = D * PITCH * 4;
};

// eight consecutive fp32 values as P bf16 plane fragments: each plane two
// values at a time with the packed round-to-nearest-even conversion, the
// remainder for the next plane exact (the values and their bf16 rounding
// share an exponent range), as split_planes does one value at a time
template <int P>
__device__ __forceinline__ void split8(float (&v)[8], bf16x8 (&f)[P]) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int p = 0; p < P; ++p) {
    u4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    f[p] = __builtin_bit_cast(bf16x8, w);
    if (p + 1 < P) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] -= __uint_as_float(w[q] << 16);
        v[2 * q + 1] -= __uint_as_float(w[q] & 0xffff0000u);
      }
    }
  }
}

template <int D, int P>
__global__ __launch_bounds__(NsSmall<D>::THREADS) void ns_small_kernel(const float* U, const float* rowsq, float* out,
                                                                        int iters, float ca, float cb, float cc) {
  using G = NsSmall<D>;
  using TP = DTile<D, 32, G::NW>;   // one bf16 plane of a 32-wide k slice, D rows
  static_assert(TP::CHUNKS == G::THREADS, "one 8-value chunk of a slice per thread");
  constexpr int FM = G::FM, FN = G::FN, PITCH = G::PITCH;
  __shared__ __attribute__((aligned(16))) float s0[D * PITCH];   // X
  __shared__ __attribute__((aligned(16))) float s1[D * PITCH];   // A, then B
  __shared__ __attribute__((aligned(256))) char s_pl[P * TP::BYTES];
  __shared__ float s_scale;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  const int64_t b = blockIdx.x;
  const int64_t DD = (int64_t)D * D;
  if (wave == 0) {
    float sq = 0.f;
    for (int i = lane; i < D; i += WAVE) sq += rowsq[b * D + i];
    sq = wave_sum(sq);
    if (lane == 0) s_scale = 1.0f / (sqrtf(sq) + 1e-7f);
  }
  __syncthreads();
  {
    const float sc = s_scale;
    const float* Ub = U + b * DD;
    for (int e = tid * 4; e < D * D; e += G::THREADS * 4) {
      const float4 u = *reinterpret_cast<const float4*>(Ub + e);
      *reinterpret_cast<float4*>(s0 + (e / D) * PITCH + e % D) = make_float4(sc * u.x, sc * u.y, sc * u.z, sc * u.w);
    }
  }
  __syncthreads();

  // fragment (16 rows x 8 k per lane-group) of a row-major fp32 slot, as P planes
  auto frag_rows = [&](const float* sl, int r0, int kk, bf16x8 (&f)[P]) {
    const float* src = sl + (r0 + (lane & 15)) * PITCH + kk + 8 * (lane >> 4);
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    split8<P>(v, f);
  };
  // The k slice [kk, kk + 32) of an operand that every wave reads, split
  // once into P bf16 planes of s_pl (row n, k - kk) instead of once per
  // reading wave: each thread one 8-value chunk, of a row of `sl` (ROWS) or
  // of a column (element (n, k) = sl[k][n]); lanes run along n, so both
  // kinds of fp32 reads are free of bank conflicts.
  auto fill = [&](const float* sl, int kk, auto rows) {
    constexpr bool ROWS = decltype(rows)::value;
    const int n = tid % D, c = tid / D;
    float v[8];
    if constexpr (ROWS) {
      const float4 x0 = *reinterpret_cast<const float4*>(sl + n * PITCH + kk + 8 * c);
      const float4 x1 = *reinterpret_cast<const float4*>(sl + n * PITCH + kk + 8 * c + 4);
      v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
      v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sl[(kk + 8 * c + e) * PITCH + n];
    }
    bf16x8 f[P];
    split8<P>(v, f);
#pragma unroll
    for (int p = 0; p < P; ++p) *reinterpret_cast<bf16x8*>(s_pl + p * TP::BYTES + TP::phys(n, c) * 16) = f[p];
  };
  // acc = Aop Bop^T over k, swapped MFMA order (lane holds row lane % 16 of
  // a fragment and 4 consecutive columns).  Square products (COLB = 0,
  // sa = sb): both operands are rows of sa, read from the split slice.  B X
  // (COLB = 1): Aop rows of sa split by each wave that reads them, Bop
  // element (n, k) = sb[k][n] from the split slice.
  f32x4 acc[FM][FN];
  auto product = [&](const float* sa, const float* sb, auto colb) {
    constexpr bool COLB = decltype(colb)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < D; kk += 32) {
      // the previous slice's planes are read by every wave (before the
      // first slice, the barrier that ended the last update of the slots)
      if (kk) __syncthreads();
      fill(sb, kk, IC<COLB ? 0 : 1>{});
      __syncthreads();
      bf16x8 fa[FM][P], fb[FN][P];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (COLB) frag_rows(sa, wm * (D / G::WGM) + i * 16, kk, fa[i]);
        else {
#pragma unroll
          for (int p = 0; p < P; ++p) fa[i][p] = dfrag_row<TP>(s_pl + p * TP::BYTES, wm * (D / G::WGM) + i * 16, 0, lane);
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int p = 0; p < P; ++p) fb[j][p] = dfrag_row<TP>(s_pl + p * TP::BYTES, wn * (D / G::WGN) + j * 16, 0, lane);
#pragma unroll
      for (int sp = P - 1; sp >= 0; --sp)
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int q = 0; q < P; ++q)
            if (p + q == sp)
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma(fb[j][q], fa[i][p], acc[i][j]);
    }
  };
  // v = alpha acc + beta slot (own positions), stored into `dst` after the barrier
  auto finish = [&](float alpha, const float* sin, float beta, float* dst) {
    float y[FM][FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wm * (D / G::WGM) + i * 16 + (lane & 15);
        const int c = wn * (D / G::WGN) + j * 16 + 4 * (lane >> 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sin) x = *reinterpret_cast<const float4*>(sin + r * PITCH + c);
        y[i][j][0] = alpha * acc[i][j][0] + beta * x.x;
        y[i][j][1] = alpha * acc[i][j][1] + beta * x.y;
        y[i][j][2] = alpha * acc[i][j][2] + beta * x.z;
        y[i][j][3] = alpha * acc[i][j][3] + beta * x.w;
      }
    __syncthreads();   // every read of the slot being replaced is done
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wm * (D / G::WGM) + i * 16 + (lane & 15);
        const int c = wn * (D / G::WGN) + j * 16 + 4 * (lane >> 4);
        *reinterpret_cast<float4*>(dst + r * PITCH + c) = make_float4(y[i][j][0], y[i][j][1], y[i][j][2], y[i][j][3]);
      }
    __syncthreads();
  };
  for (int it = 0; it < iters; ++it) {
    product(s0, s0, IC<0>{});         // A = X X^T
    finish(1.f, nullptr, 0.f, s1);
    product(s1, s1, IC<0>{});         // A A  (A symmetric: A A^T)
    finish(cc, s1, cb, s1);           // B = c A A + b A
    product(s1, s0, IC<1>{});         // B X: second operand element (n, k) = X[k][n]
    finish(1.f, s0, ca, s0);          // X <- B X + a X
  }
  float* ob = out + b * DD;
  for (int e = tid * 4; e < D * D; e += G::THREADS * 4)
    *reinterpret_cast<float4*>(ob + e) = *reinterpret_cast<const float4*>(s0 + (e / D) * PITCH + e % D);
}

}  // namespace lact
