// bf16 kernels built on gfx950's direct global->LDS loads.
//
// Tiles are copied from global memory into LDS with global_load_lds_dwordx4
// (16 bytes per lane, landing at the wave's LDS base + 16 * lane), so no
// staging registers are needed and several k-stages can be in flight.  LDS
// rows hold 16-byte chunks XOR-swizzled by row to keep fragment reads free of
// bank conflicts.  Operands whose k index is the slow dimension in memory (a
// token-major activation contracted over tokens) are read into MFMA
// fragments with ds_read_b64_tr_b16: in each 16-lane group, output lane i,
// element r is element (i % 4) of source lane 4r + i/4, so source lane j
// points at row 8g + j/4, columns 4(j % 4) .. +3 of the tile and two such
// reads give lane (g, i) the 8 consecutive k of column i.
#pragma once
#include "lact_kernels.hpp"

namespace lact {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt that only waits for vector-memory counts <= N (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence __syncthreads() implies (the
// fence would wait for every in-flight direct load); the empty asm keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte offset of an LDS location (generic pointer to __shared__ memory).
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One global_load_lds_dwordx4: 16 bytes per lane from g to LDS byte offset
// m0 + 16 * lane.  Issued from asm because the compiler, unable to tell ring
// buffers apart, would otherwise wait for every in-flight copy before each
// LDS read; completion is tracked with explicit vmcnt waits instead.  The
// instruction has no register outputs.
__device__ __forceinline__ void dma16(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
}

// One global_load_lds_dword: 4 bytes per lane from g to LDS byte offset
// m0 + 4 * lane (placement measured by an in-bounds probe); no register
// outputs, completion tracked with vmcnt like dma16.
__device__ __forceinline__ void dma4(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
}

// s_waitcnt for LDS traffic only (direct loads in flight are left alone)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// LDS tile of R rows x CC bf16 columns (CC = 32, 64 or 128), filled by NW
// waves.  Chunk c (16 bytes) of row r is stored at chunk swz(r, c) of that
// row.  The swizzle spreads the rows a fragment read touches over distinct
// bank groups: 8 rows x 16 B for row-k reads of 64- and 128-byte rows, and
// for 256-byte rows read with ds_read_b64_tr_b16, the 32-byte column pairs of
// rows r..r+3 and r+8..r+11 (two 16-lane groups) over all eight 32-byte slots.
template <int R, int CC, int NW = 4, bool TR = false>
struct DTile {
  static constexpr int CPR = CC / 8;
  static constexpr int BYTES = R * CC * 2;
  static constexpr int CHUNKS = R * CPR;
  static constexpr int INSTR = CHUNKS / (WAVE * NW);   // loads per wave
  static_assert(CHUNKS % (WAVE * NW) == 0, "tile must be a whole number of workgroup loads");
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "row width");
  // TR: the tile is read with ds_read_b64_tr_b16 (rows = k); otherwise with
  // 16-byte row reads (rows = the MFMA row index)
  __device__ static __forceinline__ int swz(int r, int c) {
    if constexpr (CPR == 4) return c ^ ((r >> 1) & 3);
    else if constexpr (!TR || CPR == 8) return c ^ (r & 7);
    else return c ^ ((((r & 3) | (((r >> 3) & 1) << 2))) << 1);
  }
  __device__ static __forceinline__ int phys(int row, int chunk) { return row * CPR + swz(row, chunk); }

  // Per-lane global pointers of the tile's loads for one stage: rows
  // r0 .. r0+R-1 (clamped to rmax) of a row-major bf16 matrix with row stride
  // ld elements, columns c0 .. c0+CC-1.  Later stages are reached by adding a
  // byte offset, so the address arithmetic is paid once per kernel.
  struct Plan {
    const char* p[INSTR];
  };
  __device__ static __forceinline__ Plan plan(const bf16_t* base, int64_t ld, int64_t r0, int64_t rmax, int64_t c0,
                                              int wave, int lane) {
    Plan pl;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int q = (i * NW + wave) * WAVE + lane;
      const int row = q / CPR, slot = q % CPR;
      const int c = swz(row, slot);   // swz is an involution in c
      const int64_t gr = min(r0 + row, rmax);
      pl.p[i] = reinterpret_cast<const char*>(base + gr * ld + c0 + c * 8);
    }
    return pl;
  }
  // load i of the stage (0 <= i < INSTR)
  __device__ static __forceinline__ void issue_one(char* tile, const Plan& pl, int64_t byte_off, int wave, int i) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_off(tile) + (uint32_t)((i * NW + wave) * WAVE * 16));
    dma16(pl.p[i] + byte_off, m0);
  }
  __device__ static __forceinline__ void issue_one(char* tile, const bf16_t* base, int64_t ld, int64_t r0, int64_t rmax,
                                                   int64_t c0, int wave, int lane, int i) {
    const int q = (i * NW + wave) * WAVE + lane;
    const int row = q / CPR, slot = q % CPR;
    const int64_t gr = min(r0 + row, rmax);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_off(tile) + (uint32_t)((i * NW + wave) * WAVE * 16));
    dma16(base + gr * ld + c0 + swz(row, slot) * 8, m0);
  }
  __device__ static __forceinline__ void issue(char* tile, const Plan& pl, int64_t byte_off, int wave) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_off(tile) + (uint32_t)(wave * WAVE * 16));
#pragma unroll
    for (int i = 0; i < INSTR; ++i) dma16(pl.p[i] + byte_off, m0 + (uint32_t)(i * NW * WAVE * 16));
  }
  // one-off load with full address arithmetic (ragged last stage)
  __device__ static __forceinline__ void issue(char* tile, const bf16_t* base, int64_t ld, int64_t r0, int64_t rmax,
                                               int64_t c0, int wave, int lane) {
    issue(tile, plan(base, ld, r0, rmax, c0, wave, lane), 0, wave);
  }
};

// fragment of a tile whose rows are the MFMA row index and columns are k
template <class T>
__device__ __forceinline__ bf16x8 dfrag_row(const char* tile, int row0, int kk, int lane) {
  const int row = row0 + (lane & 15);
  const int chunk = (kk >> 3) + (lane >> 4);
  return *reinterpret_cast<const bf16x8*>(tile + T::phys(row, chunk) * 16);
}

// fragment of a tile whose rows are k and columns are the MFMA row index
template <class T>
__device__ __forceinline__ bf16x8 dfrag_col(const char* tile, int n0, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = kk + 8 * g + (j >> 2);
  const int col = n0 + 4 * (j & 3);
  const int chunk = col >> 3, half = (col >> 2) & 1;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(tile + T::phys(row, chunk) * 16 + half * 8));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(tile + T::phys(row + 4, chunk) * 16 + half * 8));
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <class T, bool COLK>
__device__ __forceinline__ bf16x8 dfrag(const char* tile, int r0, int kk, int lane) {
  if constexpr (COLK) return dfrag_col<T>(tile, r0, kk, lane);
  else return dfrag_row<T>(tile, r0, kk, lane);
}

// Direct-load pipeline over nk stages with an NST-deep LDS ring: stage s is
// issued NST-1 iterations before it is consumed.  issue(s, buf) must emit
// exactly LPS global_load_lds per wave.
template <int NST, int LPS, class I, class C>
__device__ __forceinline__ void dpipeline(int nk, I&& issue, C&& compute) {
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt is complete once at most min(NST-2, nk-1-kt) later stages are in flight
    const int later = min(NST - 2, nk - 1 - kt);
    if constexpr (NST >= 4) {
      if (later >= 2) wait_vm<2 * LPS>();
      else if (later == 1) wait_vm<LPS>();
      else wait_vm<0>();
    } else if constexpr (NST == 3) {
      if (later >= 1) wait_vm<LPS>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    bar();
    if (kt + NST - 1 < nk) issue(kt + NST - 1, (kt + NST - 1) % NST);
    compute(kt % NST);
  }
}

// Same ring, but the loads of the stage being prefetched are spread over the
// MFMA groups of the stage being computed: compute(buf, hook) calls
// hook(slot, nslots) after each group, and the hook issues loads
// [slot * LPS / nslots, (slot + 1) * LPS / nslots) of the prefetched stage via
// issue_one(stage, buf, index).  A wave blocked on a full memory queue then
// stalls between MFMA groups instead of ahead of all of them.
template <int NST, int LPS, class I, class C>
__device__ __forceinline__ void dpipeline_il(int nk, I&& issue_one, C&& compute) {
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk)
#pragma unroll
      for (int i = 0; i < LPS; ++i) issue_one(s, s, i);
  for (int kt = 0; kt < nk; ++kt) {
    const int later = min(NST - 2, nk - 1 - kt);
    if constexpr (NST >= 4) {
      if (later >= 2) wait_vm<2 * LPS>();
      else if (later == 1) wait_vm<LPS>();
      else wait_vm<0>();
    } else if constexpr (NST == 3) {
      if (later >= 1) wait_vm<LPS>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    bar();
    const int ns = kt + NST - 1;
    const bool nxt = ns < nk;
    const int nb = ns % NST;
    compute(kt % NST, [&](int slot, int nslots) {
      if (nxt) {
#pragma unroll
        for (int i = 0; i < LPS; ++i)
          if (i * nslots >= slot * LPS && i * nslots < (slot + 1) * LPS) issue_one(ns, nb, i);
      }
    });
  }
}

// dpipeline_il for workgroups whose waves issue different numbers of loads
// per stage: LPS_A for waves with `wide` set, LPS_B for the others.  The
// vmcnt target of each wait is that wave's own count of later stages' loads.
template <int NST, int LPS_A, int LPS_B, class I, class C>
__device__ __forceinline__ void dpipeline_il2(int nk, bool wide, I&& issue_one, C&& compute) {
  static_assert(NST >= 2 && NST <= 4, "ring depth");
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk)
#pragma unroll
      for (int i = 0; i < LPS_A; ++i) issue_one(s, s, i);
  for (int kt = 0; kt < nk; ++kt) {
    const int later = min(NST - 2, nk - 1 - kt);
    if (later >= 2) {
      if (wide) wait_vm<2 * LPS_A>();
      else wait_vm<2 * LPS_B>();
    } else if (later == 1) {
      if (wide) wait_vm<LPS_A>();
      else wait_vm<LPS_B>();
    } else {
      wait_vm<0>();
    }
    bar();
    const int ns = kt + NST - 1;
    const bool nxt = ns < nk;
    const int nb = ns % NST;
    compute(kt % NST, [&](int slot, int nslots) {
      if (nxt) {
#pragma unroll
        for (int i = 0; i < LPS_A; ++i)
          if (i * nslots >= slot * LPS_A && i * nslots < (slot + 1) * LPS_A) issue_one(ns, nb, i);
      }
    });
  }
}

// =========================================================================
// bf16 GEMM (same contract as gemm_kernel; A, B bf16).  T x T output tile,
// 8 waves: wave w owns quadrant (w & 3) of the tile and k half (w >> 2) of
// every BKK stage (two waves per SIMD); the two k halves are summed through
// LDS at the end.  The swapped MFMA operand order leaves each lane with 4
// consecutive output columns.
constexpr int DG_THREADS = 512;

// PA > 1: the first operand is an fp32 quantity stored as PA bf16 planes
// (plane p at A + p * a_ps, lact_planes.hpp); PB > 1: the second likewise
// (plane q at B + q * b_ps).  A product sums the plane pairs (p, q) with
// p + q < max(PA, PB), the pairs of smaller weight first (with one exact
// operand: its plane products, smallest plane first).
template <bool CA, bool CB, typename TC, int T, int BKK, int NST, int PA = 1, int PB = 1>
__global__ __launch_bounds__(DG_THREADS) void dgemm_kernel(GemmArgs g) {
  constexpr int NW = 8, KH = BKK / 2, NKK = KH / 32;
  using TA = typename std::conditional<CA, DTile<BKK, T, NW, true>, DTile<T, BKK, NW>>::type;
  using TB = typename std::conditional<CB, DTile<BKK, T, NW, true>, DTile<T, BKK, NW>>::type;
  constexpr int STAGE = PA * TA::BYTES + PB * TB::BYTES;
  constexpr int LPS = PA * TA::INSTR + PB * TB::INSTR;
  constexpr int PM = PA > PB ? PA : PB;
  constexpr int FM = T / 32, FN = T / 32;                 // quadrant T/2 x T/2
  constexpr int RED = 4 * FM * FN * 256 * 4;              // k-half reduction buffer (bytes)
  constexpr int SMEM = NST * STAGE > RED ? NST * STAGE : RED;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ float s_scale;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = wave & 3, kh = wave >> 2;
  const int wm = q >> 1, wn = q & 1;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < g.ngroups && bid >= g.g[gi].tiles) bid -= g.g[gi++].tiles;
  const GemmGroup& G = g.g[gi];
  const int M = G.M;
  const int tn_count = (g.N + T - 1) / T;
  const int tm_count = (M + T - 1) / T;
  const int tiles = tm_count * tn_count;
  const int tile = bid % tiles;
  bid /= tiles;
  const int split = bid % g.splits;
  const int b = bid / g.splits;
  const int tm = tile / tn_count, tn = tile % tn_count;
  const int m0 = tm * T, n0 = tn * T;

  const bf16_t* A = reinterpret_cast<const bf16_t*>(G.A) + b * g.a_bs;
  const bool second_b = g.B2 != nullptr && m0 >= g.m_switch;
  const bf16_t* B = reinterpret_cast<const bf16_t*>(second_b ? g.B2 : G.B) + b * (second_b ? g.b2_bs : g.b_bs);
  const int64_t kbeg = (int64_t)split * g.kps;
  const int64_t kend = min(g.K, kbeg + g.kps);
  const int nk = kbeg < kend ? (int)((kend - kbeg + BKK - 1) / BKK) : 0;
  // rows past the data are clamped: for row-k operands they are outputs that
  // are never stored; for column-k operands they are k positions the other
  // operand holds as zeros (callers pad it) or that lie in the valid range
  const int64_t kmax = g.K - 1;

  // column-k operands step BKK rows per stage, row-k operands BKK columns
  typename TA::Plan pa[PA];
#pragma unroll
  for (int p = 0; p < PA; ++p)
    pa[p] = CA ? TA::plan(A + p * g.a_ps, g.lda, kbeg, kmax, m0, wave, lane)
               : TA::plan(A + p * g.a_ps, g.lda, m0, M - 1, kbeg, wave, lane);
  typename TB::Plan pb[PB];
#pragma unroll
  for (int q = 0; q < PB; ++q)
    pb[q] = CB ? TB::plan(B + q * g.b_ps, g.ldb, kbeg, kmax, n0, wave, lane)
               : TB::plan(B + q * g.b_ps, g.ldb, n0, g.N - 1, kbeg, wave, lane);
  const int64_t sa = CA ? (int64_t)BKK * g.lda * 2 : (int64_t)BKK * 2;
  const int64_t sb = CB ? (int64_t)BKK * g.ldb * 2 : (int64_t)BKK * 2;
  auto issue_one = [&](int s, int buf, int idx) {
    char* st = smem + buf * STAGE;
    const int64_t k0 = kbeg + (int64_t)s * BKK;
    const bool ragged = k0 + BKK - 1 > kmax;   // a column-k stage past the data must clamp rows
    if (idx < PA * TA::INSTR) {
#pragma unroll
      for (int p = 0; p < PA; ++p) {
        if (idx / TA::INSTR != p) continue;
        const int i = idx - p * TA::INSTR;
        if (CA && ragged) TA::issue_one(st + p * TA::BYTES, A + p * g.a_ps, g.lda, k0, kmax, m0, wave, lane, i);
        else TA::issue_one(st + p * TA::BYTES, pa[p], s * sa, wave, i);
      }
    } else {
      const int ib = idx - PA * TA::INSTR;
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        if (ib / TB::INSTR != q) continue;
        const int i = ib - q * TB::INSTR;
        char* bt = st + PA * TA::BYTES + q * TB::BYTES;
        if (CB && ragged) TB::issue_one(bt, B + q * g.b_ps, g.ldb, k0, kmax, n0, wave, lane, i);
        else TB::issue_one(bt, pb[q], s * sb, wave, i);
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, auto&& hook) {
    const char* st = smem + buf * STAGE;
#pragma unroll
    for (int t = 0; t < NKK; ++t) {
      const int kk = kh * KH + t * 32;
      bf16x8 af[PA][FM], bfr[PB][FN];
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i) af[p][i] = dfrag<TA, CA>(st + p * TA::BYTES, wm * (T / 2) + i * 16, kk, lane);
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[q][j] = dfrag<TB, CB>(st + PA * TA::BYTES + q * TB::BYTES, wn * (T / 2) + j * 16, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int sp = PM - 1; sp >= 0; --sp)
#pragma unroll
          for (int p = 0; p < PA; ++p)
#pragma unroll
            for (int q = 0; q < PB; ++q)
              if (p + q == sp)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma(bfr[q][j], af[p][i], acc[i][j]);
        hook(t * FM + i, NKK * FM);
      }
    }
  };
  dpipeline_il<NST, LPS>(nk, issue_one, compute);

  // sum the two k halves (fixed order: half 0 + half 1)
  bar();
  float* red = reinterpret_cast<float*>(smem);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        *reinterpret_cast<f32x4*>(red + ((q * FM + i) * FN + j) * 256 + lane * 4) = acc[i][j];
  }
  wait_lgkm0();   // the half-1 sums are in LDS before another wave reads them
  bar();
  if (kh == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] += *reinterpret_cast<const f32x4*>(red + ((q * FM + i) * FN + j) * 256 + lane * 4);
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
  if (kh == 1) return;
  TC* C = reinterpret_cast<TC*>(G.C) + b * g.c_bs + split * g.c_ss;
  const float* Cin = G.Cin ? G.Cin + b * g.cin_bs : nullptr;
  const bool trans = m0 >= g.trans_from;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * (T / 2) + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nq = n0 + wn * (T / 2) + j * 16 + 4 * (lane >> 4);
      if (nq >= g.N) continue;
      float val[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) val[r] = alpha * acc[i][j][r];
      if (Cin) {
        const float4 c = *reinterpret_cast<const float4*>(Cin + (int64_t)m * g.ldcin + nq);
        val[0] += beta * c.x;
        val[1] += beta * c.y;
        val[2] += beta * c.z;
        val[3] += beta * c.w;
      }
      if (trans) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          io_traits<TC>::store(C + (int64_t)g.trans_from * g.ldc + (int64_t)(nq + r) * g.ldc_t + (m - g.trans_from),
                               val[r]);
      } else {
        store4(C + (int64_t)m * g.ldc + nq, val);
      }
    }
  }
}

// =========================================================================
// bf16 update forward tile (same contract as upd_fwd_kernel with bf16
// snapshots: W2 operand from the transposed snapshot)
// waves that issue the W tile loads: the largest count that divides the tile
constexpr int upd_w_waves(int bj, int bkk) {
  return (bj * (bkk / 8)) % (WAVE * 8) == 0 ? 8 : (bj * (bkk / 8)) % (WAVE * 6) == 0 ? 6 : 4;
}

// 8 waves: wave w owns tokens 32 (w >> 1) .. +31 and hidden columns
// (BJ / 2)(w & 1) .. +BJ/2-1 of the 128 x BJ tile (two waves per SIMD keep
// the MFMA pipes fed).  K and V tiles are loaded by all eight waves, the W
// tiles by the first upd_w_waves; each wave waits on its own load count.
// WQ: the same tokens' queries are applied on the same snapshot (an
// apply-then-update chunk): a third token tile q shares the W1 and W3
// fragments, and the tile also writes its gated hidden
// Hq = silu(q W1^T) * (q W3^T) to rows h0 + (t - upd_t0) of the Hq buffer
// (swapped MFMA operands: each lane holds 4 consecutive hidden units of one
// token, stored as 8 bytes straight from registers).
// P > 1 (the multi-plane recurrence): the weights are P bf16 planes, plane 0
// the snapshot (W1, W3, W2^T as above), planes 1.. at Wlo + (p - 1) * wlo_ps
// + m * wlo_ms (m = 0 W1, 1 W3, 2 W2^T); K and V are exact, so each product
// sums P plane products, smallest plane first.  The update terms are fp32
// values stored as P bf16 planes (plane p at E + p * e_ps), the operand form
// of the contraction that follows.
// waves per SIMD the update tile is compiled for: two workgroups per CU for
// the two-plane tile on a two-stage ring (80 KB of LDS), else one
constexpr int upd_min_waves(int P, int NST) { return P == 2 && NST == 2 ? 4 : 1; }

template <int BJ, int BKK, int NST, bool WQ = false, int P = 1>
__global__ __launch_bounds__(DG_THREADS, upd_min_waves(P, NST)) void dupd_fwd_kernel(UpdFwdArgs a) {
  constexpr int NWV = DG_THREADS / WAVE;
  constexpr int WW = upd_w_waves(BJ, BKK);
  constexpr int NX = WQ ? 3 : 2;     // token tiles per stage: k, v (, q)
  using TX = DTile<FBT, BKK, NWV>;   // K, V (, Q): 128 tokens x BKK
  using TW = DTile<BJ, BKK, WW>;     // W1, W3, W2^T rows (each plane): BJ x BKK
  static_assert(!WQ || P == 1, "the queries' products run in the plain-bf16 tile only");
  constexpr int STAGE = NX * TX::BYTES + 3 * P * TW::BYTES;
  constexpr int LPS = NX * TX::INSTR + 3 * P * TW::INSTR;   // loads per stage of a W-loading wave
  constexpr int LPS_X = NX * TX::INSTR;                     // ... of the other waves
  constexpr int FM = 2, FN = BJ / 32;
  constexpr int ET_PLANE = 3 * BJ * FBT * 2;   // one plane of the tile's update terms (bf16)
  // After the main loop the ring holds the staged update terms (for
  // full-line stores) and, at its end, the tile's learning rates and beta
  // sums; all planes are staged at once when they fit, else one per pass.
  constexpr int RING = NST * STAGE;
  constexpr int LR_BYTES = FBT * 3 * 4;
  constexpr int LR_OFF = (RING - LR_BYTES - 16) & ~15;
  constexpr int PPASS = P * ET_PLANE <= LR_OFF ? P : 1;   // planes staged per pass
  static_assert(PPASS * ET_PLANE <= LR_OFF, "staging fits the ring beside the learning rates");
  __shared__ __attribute__((aligned(1024))) char smem[RING];
  float* s_lr = reinterpret_cast<float*>(smem + LR_OFF);
  float* s_red = reinterpret_cast<float*>(smem + LR_OFF + LR_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + inst * a.k_bs;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + inst * a.x_bs;
  const bf16_t* W1 = reinterpret_cast<const bf16_t*>(a.W1) + inst * DD;
  const bf16_t* W3 = reinterpret_cast<const bf16_t*>(a.W3) + inst * DD;
  const bf16_t* W2T = reinterpret_cast<const bf16_t*>(a.W2x) + inst * DD;
  const bf16_t* Q = WQ ? reinterpret_cast<const bf16_t*>(a.q) + inst * a.q_bs : K;

  // the tile's learning rates and momentum coefficients, held in registers
  // through the main loop (used by the epilogue)
  float lrv = 0.f, bval = 0.f;
  {
    const float* lr = a.lr + inst * a.lr_bs + t0 * 3;
    if (tid < FBT * 3 && t0 + tid / 3 < tend) lrv = lr[tid];
    if (a.beta != nullptr && jb == 0 && tid < FBT && t0 + tid < tend) bval = a.beta[inst * a.beta_bs + t0 + tid];
  }

  const bool wload = wave < WW;
  const typename TX::Plan pk = TX::plan(K, D, t0, tend - 1, 0, wave, lane);
  const typename TX::Plan pv = TX::plan(V, D, t0, tend - 1, 0, wave, lane);
  const typename TX::Plan pq = TX::plan(Q, D, t0, tend - 1, 0, wave, lane);
  // W1, W3 and W2^T rows: hidden units j0 .. j0 + BJ - 1 (of dh), d long;
  // W tile (m, p) of a stage sits at w + (m * P + p) * TW::BYTES.  One
  // plane: per-lane addresses planned once; several: the planes' bases
  // (uniform) kept and each load's address formed when it is issued, which
  // keeps the per-lane registers of 3 P planned addresses free.
  const bf16_t* W0[3] = {W1, W3, W2T};
  const bf16_t* wsrc[3][P];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int p = 0; p < P; ++p)
      wsrc[m][p] = p == 0 ? W0[m] : reinterpret_cast<const bf16_t*>(a.Wlo) + (p - 1) * a.wlo_ps + m * a.wlo_ms + inst * DD;
  typename TW::Plan pw[3][P == 1 ? 1 : 1];
  if constexpr (P == 1) {
#pragma unroll
    for (int m = 0; m < 3; ++m) pw[m][0] = TW::plan(wsrc[m][0], D, j0, Dh - 1, 0, wload ? wave : 0, lane);
  }
  auto issue_one = [&](int s, int buf, int idx) {
    char* st = smem + buf * STAGE;
    const int64_t off = (int64_t)s * BKK * 2;
    char* w = st + NX * TX::BYTES;
    // token tiles first (every wave issues them), then the W tiles
    if (idx < TX::INSTR) TX::issue_one(st, pk, off, wave, idx);
    else if (idx < 2 * TX::INSTR) TX::issue_one(st + TX::BYTES, pv, off, wave, idx - TX::INSTR);
    else if (WQ && idx < 3 * TX::INSTR) TX::issue_one(st + 2 * TX::BYTES, pq, off, wave, idx - 2 * TX::INSTR);
    else if (!wload) return;
    else {
      const int wi = idx - NX * TX::INSTR;
#pragma unroll
      for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (wi / TW::INSTR == m * P + p) {
            if constexpr (P == 1)
              TW::issue_one(w + m * TW::BYTES, pw[m][0], off, wave, wi % TW::INSTR);
            else
              TW::issue_one(w + (m * P + p) * TW::BYTES, wsrc[m][p], D, j0, Dh - 1, (int64_t)s * BKK, wave, lane,
                            wi % TW::INSTR);
          }
    }
  };
  f32x4 accA[FM][FN], accB[FM][FN], accG[FM][FN], accQ1[FM][FN], accQ3[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      accA[i][j] = accB[i][j] = accG[i][j] = accQ1[i][j] = accQ3[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, auto&& hook) {
    const char* st = smem + buf * STAGE;
    const char* w = st + NX * TX::BYTES;
    constexpr int NSLOT = (BKK / 32) * (P == 1 ? FM : P);
#pragma unroll
    for (int kk = 0; kk < BKK; kk += 32) {
      bf16x8 fk[FM], fv[FM], fq[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        fk[i] = dfrag_row<TX>(st, wm * 32 + i * 16, kk, lane);
        fv[i] = dfrag_row<TX>(st + TX::BYTES, wm * 32 + i * 16, kk, lane);
        if constexpr (WQ) fq[i] = dfrag_row<TX>(st + 2 * TX::BYTES, wm * 32 + i * 16, kk, lane);
      }
      if constexpr (P == 1) {
        bf16x8 f1[FN], f3[FN], f2[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          f1[j] = dfrag_row<TW>(w, wn * (BJ / 2) + j * 16, kk, lane);
          f3[j] = dfrag_row<TW>(w + TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
          f2[j] = dfrag_row<TW>(w + 2 * TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            accA[i][j] = mfma(fk[i], f1[j], accA[i][j]);
            accB[i][j] = mfma(fk[i], f3[j], accB[i][j]);
            accG[i][j] = mfma(fv[i], f2[j], accG[i][j]);
            if constexpr (WQ) {
              accQ1[i][j] = mfma(f1[j], fq[i], accQ1[i][j]);
              accQ3[i][j] = mfma(f3[j], fq[i], accQ3[i][j]);
            }
          }
          hook((kk / 32) * FM + i, NSLOT);
        }
      } else {
        // one weight plane at a time (smallest first): its fragments, then
        // its products, so only one plane's fragments are live
#pragma unroll
        for (int p = P - 1; p >= 0; --p) {
          bf16x8 f1[FN], f3[FN], f2[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            f1[j] = dfrag_row<TW>(w + p * TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
            f3[j] = dfrag_row<TW>(w + (P + p) * TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
            f2[j] = dfrag_row<TW>(w + (2 * P + p) * TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
          }
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              accA[i][j] = mfma(fk[i], f1[j], accA[i][j]);
              accB[i][j] = mfma(fk[i], f3[j], accB[i][j]);
              accG[i][j] = mfma(fv[i], f2[j], accG[i][j]);
            }
          hook((kk / 32) * P + (P - 1 - p), NSLOT);
        }
      }
    }
  };
  dpipeline_il2<NST, LPS, LPS_X>(D / BKK, wload, issue_one, compute);

  if constexpr (WQ) {
    // Hq rows of the tile's tokens inside the chunk (bf16, as the apply
    // stores them); lane: token lane & 15 of the fragment, hidden units
    // 4 (lane >> 4) .. +3
    bf16_t* H = reinterpret_cast<bf16_t*>(a.H) + inst * a.h_bs + j0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t t = t0 + wm * 32 + i * 16 + (lane & 15);
      if (t >= tend) continue;
      bf16_t* Hr = H + (a.h0 + (t - a.upd_t0)) * (int64_t)Dh;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = accQ1[i][j][r];
          h[r] = x * fast_sigmoid(x) * accQ3[i][j][r];
        }
        store4(Hr + wn * (BJ / 2) + j * 16 + 4 * (lane >> 4), h);
      }
    }
  }

  // Epilogue: SwiGLU backward terms into an LDS copy of the tile's E rows
  // (row = term x hidden column, 128 tokens = 256 bytes, 16-byte chunks
  // XOR-swizzled by row), then whole rows to global memory.
  bar();   // every wave is done reading the ring
  if (tid < FBT * 3) s_lr[tid] = lrv;
  if (a.beta != nullptr && jb == 0) {
    const float bs = wave_sum(bval);
    if (lane == 0 && wave < 2) s_red[wave] = bs;
  }
  __syncthreads();
  if (a.beta != nullptr && jb == 0 && tid == 0) a.bpart[(int64_t)inst * a.tiles_t + tb] = s_red[0] + s_red[1];
  char* et = smem;
  bf16_t* E = reinterpret_cast<bf16_t*>(a.E) + inst * 3 * (int64_t)Dh * a.ldE + (t0 - a.upd_t0);
  constexpr int ROWS = 3 * BJ;
  for (int p0 = 0; p0 < P; p0 += PPASS) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int tl = wm * 32 + i * 16 + 4 * (lane >> 4);   // tile-local token of element r = 0
      float e1[4], e2[4], e3[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e1[r] = s_lr[(tl + r) * 3 + 0];
        e2[r] = s_lr[(tl + r) * 3 + 1];
        e3[r] = s_lr[(tl + r) * 3 + 2];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wn * (BJ / 2) + j * 16 + (lane & 15);
        float u1[4], u3[4], u2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = accA[i][j][r], bb = accB[i][j][r], gg = accG[i][j][r];
          const float sg = fast_sigmoid(x);
          const float s = x * sg;
          const float sp = sg * (1.0f + x * (1.0f - sg));
          u1[r] = e1[r] * gg * bb * sp;
          u3[r] = e3[r] * gg * s;
          u2[r] = e2[r] * s * bb;
        }
        const int chunk = tl >> 3, half = (tl >> 2) & 1;
        const float* terms[3] = {u1, u3, u2};
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          const int row = m * BJ + col;
          const int off = row * (FBT * 2) + ((chunk ^ (row & 15)) << 4) + (half << 3);
          if constexpr (P == 1) {
            uint2 pk2;
            pk2.x = pack_bf16x2(terms[m][0], terms[m][1]);
            pk2.y = pack_bf16x2(terms[m][2], terms[m][3]);
            *reinterpret_cast<uint2*>(et + off) = pk2;
          } else {
            uint32_t h[4][P];
#pragma unroll
            for (int r = 0; r < 4; ++r) split_planes<P>(terms[m][r], h[r]);
#pragma unroll
            for (int pp = 0; pp < PPASS; ++pp)
              *reinterpret_cast<uint2*>(et + pp * ET_PLANE + off) =
                  make_uint2(h[0][p0 + pp] | (h[1][p0 + pp] << 16), h[2][p0 + pp] | (h[3][p0 + pp] << 16));
          }
        }
      }
    }
    __syncthreads();
    // E rows U1 | U3 | U2-terms, token-fastest (one set per plane); the
    // tile's 128 tokens lie inside the row's ldE (zero terms past the chunk end)
    for (int r0 = 0; r0 < PPASS * ROWS; r0 += 4 * NWV) {
      const int prow = r0 + wave * 4 + (lane >> 4);
      if (prow < PPASS * ROWS) {
        const int pp = prow / ROWS, row = prow % ROWS;
        const int c = lane & 15;
        const uint4 v = *reinterpret_cast<const uint4*>(et + pp * ET_PLANE + row * (FBT * 2) + ((c ^ (row & 15)) << 4));
        const int m = row / BJ, col = row % BJ;
        *reinterpret_cast<uint4*>(E + (p0 + pp) * a.e_ps + (int64_t)(m * Dh + j0 + col) * a.ldE + c * 8) = v;
      }
    }
    if (p0 + PPASS < P) __syncthreads();   // every row read before the next pass overwrites the staging
  }
}

// =========================================================================
// Arguments of the fused update (update forward + contraction in one kernel)
struct UpdDwArgs {
  UpdFwdArgs u;          // chunk, inputs, snapshot of the weights (E unused)
  float* part;           // partials [splits, n, U1 | U3 | U2]
  int64_t part_ss;       // elements between partials
  int tps;               // token tiles per split
  int splits;
  int nbp;               // beta partial sums per instance (one per token tile)
};

constexpr int UDW_D = 128;   // d = dh handled by the fused update

// =========================================================================
// Fused update at d = dh = 128: per 32-token tile, the update forward
// A = K W1^T, B = K W3^T, G = V W2 over the tile's tokens and the workgroup's
// BJ hidden units, the SwiGLU backward terms ("大块测试时训练（LaCT）技术解析"
// §2.1, eqs. 4-5) in LDS (split into P bf16 planes for the multi-plane
// recurrence), and the tile's share of U1 = E1^T K, U3 = E3^T K, U2 = V^T E2,
// accumulated in registers over the workgroup's run of tiles; one fp32
// partial per workgroup.  The update terms never reach HBM (at this width
// their write and re-read, 2 or 6 bytes per term, would be most of the
// update's traffic).  Every product sums the plane pairs (plane p of the
// weights or update terms with the single plane of k or v), smaller planes
// first.
// The waves are specialised: the four forward waves hold the weight planes
// of their hidden units in registers for the whole run (64 units per
// workgroup for plain bf16, 32 with planes) and produce the update terms of
// tile s while the four contraction waves consume those of tile s - 1, one
// barrier per step, so the forward's VALU epilogue overlaps the
// contraction's MFMA work on every SIMD (one wave of each kind per SIMD).
// K and V stream through a direct-load ring, six deep for plain bf16 and
// four with planes (tiles s + 1 .. s + NKV - 2 are in flight while tiles s
// and s - 1 are read); the update terms are double-buffered.
constexpr int UDS_T = 32;   // tokens per tile
// hidden units per workgroup: 64 for plain bf16, 32 with weight planes
constexpr int udp_bj(int P) { return P == 1 ? 64 : 32; }

template <int P, int BJ>
__global__ __launch_bounds__(DG_THREADS) void dupd_dwp_kernel(UpdDwArgs g) {
  const UpdFwdArgs& a = g.u;
  constexpr int BKK = 64;
  constexpr int NKV = P == 1 ? 6 : 4;     // K, V ring depth (what the LDS holds beside the update terms)
  constexpr int LA = NKV - 2;             // tiles loaded ahead of the one the forward waves read
  constexpr int NH = BJ / 32;             // hidden fragments per forward wave
  constexpr int CH = BJ / 16;             // hidden fragments per contraction wave
  using TT = DTile<UDS_T, BKK, 4>;        // 32 tokens x 64 d (K, V stages), loaded by the four contraction waves
  static_assert(TT::INSTR == 1 && UDW_D == 2 * BKK && DG_THREADS == 8 * WAVE && BJ % 32 == 0, "tile shapes");
  constexpr int TB = TT::BYTES;           // 4 KB
  constexpr int KVB = 4 * TB;             // K s0, K s1, V s0, V s1
  constexpr int ERB = UDS_T * 2;          // update-term row: 32 tokens of bf16 (4 chunks)
  constexpr int EPL = 3 * BJ * ERB;       // one plane: rows U1 | U3 | U2 terms
  __shared__ __attribute__((aligned(1024))) char s_kv[NKV * KVB];
  __shared__ __attribute__((aligned(1024))) char s_e[2 * P * EPL];
  __shared__ __attribute__((aligned(16))) float s_lr[NKV][128];   // 96 used (3 per token)
  __shared__ __attribute__((aligned(16))) float s_beta[NKV][64];  // 32 used

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool fwd = wave < 4;
  const int D = UDW_D;
  const int njb = UDW_D / BJ;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int jb = bid % njb;
  bid /= njb;
  const int split = bid % g.splits;
  const int inst = bid / g.splits;
  const int j0 = jb * BJ;
  const int64_t DD = (int64_t)D * D;
  const int64_t tend = a.upd_t0 + a.upd_len;
  const int ntiles = (int)((a.upd_len + UDS_T - 1) / UDS_T);
  const int tb0 = split * g.tps, tb1 = min(ntiles, tb0 + g.tps);
  const int nt = max(0, tb1 - tb0);
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + inst * a.k_bs;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + inst * a.x_bs;
  const float* LR = a.lr + inst * a.lr_bs;
  const float* BETA = a.beta != nullptr ? a.beta + inst * a.beta_bs : nullptr;

  // contraction waves: loads of local tile i into ring slot i % NKV, five per
  // wave (K, V stages, then learning rates or beta)
  const int cw = wave & 3;
  auto issue_tile = [&](int i) {
    const int64_t t0 = a.upd_t0 + (int64_t)(tb0 + i) * UDS_T;
    const int nv = (int)min((int64_t)UDS_T, tend - t0);
    char* kv = s_kv + (i % NKV) * KVB;
    TT::issue_one(kv, K, D, t0, tend - 1, 0, cw, lane, 0);
    TT::issue_one(kv + TB, K, D, t0, tend - 1, BKK, cw, lane, 0);
    TT::issue_one(kv + 2 * TB, V, D, t0, tend - 1, 0, cw, lane, 0);
    TT::issue_one(kv + 3 * TB, V, D, t0, tend - 1, BKK, cw, lane, 0);
    const float* src;
    uint32_t dst;
    if (cw < 2) {   // learning rates: 96 values over two waves (the rest land in the padding)
      src = LR + t0 * 3 + min(cw * 64 + lane, nv * 3 - 1);
      dst = lds_off(&s_lr[i % NKV][cw * 64]);
    } else if (cw == 2 && BETA != nullptr) {
      src = BETA + t0 + min(lane, nv - 1);
      dst = lds_off(&s_beta[i % NKV][0]);
    } else {        // a harmless reload, so that every wave issues five loads per tile
      src = LR + t0 * 3 + min(lane, nv * 3 - 1);
      dst = lds_off(&s_lr[i % NKV][0]);
    }
    dma4(src, __builtin_amdgcn_readfirstlane(dst));
  };

  if (fwd) {
    // ---------------------------------------------------------------- forward waves
    // tokens 16 tf .., hidden units j0 + BJ / 2 * hg + 16 h .. (h < NH)
    const int tf = wave >> 1, hg = wave & 1;
    // this wave's weight fragments, every plane: row j0 + BJ / 2 * hg + 16 h +
    // lane % 16, k = 32 kk + 8 (lane / 16) .. + 7
    bf16x8 wr[3][P][4][NH];
    {
      const bf16_t* W0[3] = {reinterpret_cast<const bf16_t*>(a.W1), reinterpret_cast<const bf16_t*>(a.W3),
                             reinterpret_cast<const bf16_t*>(a.W2x)};
      const bf16_t* Wlo = reinterpret_cast<const bf16_t*>(a.Wlo);
#pragma unroll
      for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int pl = 0; pl < P; ++pl) {
          const bf16_t* base = (pl == 0 ? W0[m] : Wlo + (pl - 1) * a.wlo_ps + m * a.wlo_ms) + inst * DD;
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            const int64_t roff = (int64_t)(j0 + BJ / 2 * hg + 16 * h + (lane & 15)) * D + 8 * (lane >> 4);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) wr[m][pl][kk][h] = *reinterpret_cast<const bf16x8*>(base + roff + 32 * kk);
          }
        }
    }
    bar();   // tile 0 has landed (the contraction waves waited for it)
    for (int s = 0; s <= nt; ++s) {
      if (s < nt) {
        const int64_t t0 = a.upd_t0 + (int64_t)(tb0 + s) * UDS_T;
        const char* kv = s_kv + (s % NKV) * KVB;
        // learning rates of this lane's four tokens (12 consecutive values),
        // read ahead of the products so that their latency is hidden
        const int tl = tf * 16 + 4 * (lane >> 4);   // tile-local token of element r = 0
        const float4* lrv = reinterpret_cast<const float4*>(s_lr[s % NKV] + tl * 3);
        const float4 l0 = lrv[0], l1 = lrv[1], l2 = lrv[2];
        f32x4 accA[NH], accB[NH], accG[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) accA[h] = accB[h] = accG[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int st = kk >> 1, kl = (kk & 1) * 32;
          const bf16x8 fk = dfrag_row<TT>(kv + st * TB, tf * 16, kl, lane);
          const bf16x8 fv = dfrag_row<TT>(kv + (2 + st) * TB, tf * 16, kl, lane);
#pragma unroll
          for (int pl = P - 1; pl >= 0; --pl)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              accA[h] = mfma(fk, wr[0][pl][kk][h], accA[h]);
              accB[h] = mfma(fk, wr[1][pl][kk][h], accB[h]);
              accG[h] = mfma(fv, wr[2][pl][kk][h], accG[h]);
            }
        }
        // beta partial sum of this tile (chunk mean), once per tile
        if (BETA != nullptr && jb == 0 && wave == 0) {
          const float bs = wave_sum(lane < UDS_T && t0 + lane < tend ? s_beta[s % NKV][lane] : 0.f);
          if (lane == 0) a.bpart[(int64_t)inst * g.nbp + tb0 + s] = bs;
        }
        // SwiGLU backward terms, split into planes, into the update-term rows of
        // buffer s % 2 (zero past the chunk end)
        const float lrr[12] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w, l2.x, l2.y, l2.z, l2.w};
        const int chunk = tl >> 3, half = (tl >> 2) & 1;
        char* eb = s_e + (s & 1) * (P * EPL);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const int col = BJ / 2 * hg + 16 * h + (lane & 15);
          float u1[4], u3[4], u2[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = t0 + tl + r < tend;
            const float e1 = ok ? lrr[r * 3 + 0] : 0.f;
            const float e2 = ok ? lrr[r * 3 + 1] : 0.f;
            const float e3 = ok ? lrr[r * 3 + 2] : 0.f;
            const float x = accA[h][r], bb = accB[h][r], gg = accG[h][r];
            const float sg = fast_sigmoid(x);
            const float sx = x * sg;
            const float sp = sg * (1.0f + x * (1.0f - sg));
            u1[r] = e1 * gg * bb * sp;
            u3[r] = e3 * gg * sx;
            u2[r] = e2 * sx * bb;
          }
          float* terms[3] = {u1, u3, u2};
#pragma unroll
          for (int m = 0; m < 3; ++m) {
            const int row = m * BJ + col;
            char* dst = eb + row * ERB + ((chunk ^ ((row >> 1) & 3)) << 4) + (half << 3);
            // planes of the four terms, two values per conversion (the same
            // round-to-nearest-even planes as split_planes)
            float* v = terms[m];
#pragma unroll
            for (int pl = 0; pl < P; ++pl) {
              const uint32_t w0 = pack_bf16x2(v[0], v[1]), w1 = pack_bf16x2(v[2], v[3]);
              *reinterpret_cast<uint2*>(dst + pl * EPL) = make_uint2(w0, w1);
              if (pl + 1 < P) {
                v[0] -= __uint_as_float(w0 << 16);
                v[1] -= __uint_as_float(w0 & 0xffff0000u);
                v[2] -= __uint_as_float(w1 << 16);
                v[3] -= __uint_as_float(w1 & 0xffff0000u);
              }
            }
          }
        }
      }
      wait_lgkm0();
      bar();   // update terms of tile s written, tile s + 1 landed
    }
    return;
  }

  // ---------------------------------------------------------------- contraction waves
  // d columns 32 cw .. + 31 (k stage cw / 2 of K, V), all BJ hidden rows:
  // U1, U3 [hidden x d] and U2 [d x hidden], 2 x CH fragments each
  // wait until at most k tiles' loads (five per tile) are in flight
  auto wait_tiles = [](int k) {
    if (k >= 3) wait_vm<15>();
    else if (k == 2) wait_vm<10>();
    else if (k == 1) wait_vm<5>();
    else wait_vm<0>();
  };
  static_assert(LA <= 4, "wait_tiles covers up to three tiles in flight");
  for (int i = 0; i < LA && i < nt; ++i) issue_tile(i);
  wait_tiles(min(LA, nt) - 1);
  bar();   // tile 0 landed
  f32x4 cu1[2][CH], cu3[2][CH], cu2[2][CH];   // [d fragment][hidden fragment]
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < CH; ++i) cu1[c][i] = cu3[c][i] = cu2[c][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int cn = 32 * (cw & 1);
  for (int s = 0; s <= nt; ++s) {
    // slot (s + LA) % NKV held tile s - 2, read by the forward waves in step
    // s - 2 and here in step s - 1
    if (s + LA < nt) issue_tile(s + LA);
    if (s >= 1) {
      const int i = s - 1;   // consume tile i
      const char* kt = s_kv + (i % NKV) * KVB + (cw >> 1) * TB;
      const char* vt = kt + 2 * TB;
      const char* eb = s_e + (i & 1) * (P * EPL);
      bf16x8 fbk[2], fbv[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        fbk[c] = dfrag_col<TT>(kt, cn + 16 * c, 0, lane);
        fbv[c] = dfrag_col<TT>(vt, cn + 16 * c, 0, lane);
      }
#pragma unroll
      for (int pl = P - 1; pl >= 0; --pl) {
        const char* ep = eb + pl * EPL;
#pragma unroll
        for (int h = 0; h < CH; ++h) {
          const int jr = 16 * h + (lane & 15);
          const int off = (((lane >> 4) ^ ((jr >> 1) & 3)) << 4);
          const bf16x8 fa1 = *reinterpret_cast<const bf16x8*>(ep + jr * ERB + off);
          const bf16x8 fa3 = *reinterpret_cast<const bf16x8*>(ep + (BJ + jr) * ERB + off);
          const bf16x8 fa2 = *reinterpret_cast<const bf16x8*>(ep + (2 * BJ + jr) * ERB + off);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            cu1[c][h] = mfma(fbk[c], fa1, cu1[c][h]);
            cu3[c][h] = mfma(fbk[c], fa3, cu3[c][h]);
            cu2[c][h] = mfma(fa2, fbv[c], cu2[c][h]);
          }
        }
      }
    }
    // tile s + 1 must have landed before the barrier (tiles s + 2 .. s + LA
    // may be in flight)
    wait_tiles(max(0, min(s + LA, nt - 1) - (s + 1)));
    wait_lgkm0();
    bar();
  }

  float* Pp = g.part + (int64_t)split * g.part_ss + (int64_t)inst * 3 * DD;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int h = 0; h < CH; ++h) {
      const int j = j0 + 16 * h + (lane & 15);
      const int cc = 32 * cw + 16 * c + 4 * (lane >> 4);
      const float y1[4] = {cu1[c][h][0], cu1[c][h][1], cu1[c][h][2], cu1[c][h][3]};
      const float y3[4] = {cu3[c][h][0], cu3[c][h][1], cu3[c][h][2], cu3[c][h][3]};
      store4(Pp + (int64_t)j * D + cc, y1);
      store4(Pp + DD + (int64_t)j * D + cc, y3);
      const int c2 = 32 * cw + 16 * c + (lane & 15);
      const int j2 = j0 + 16 * h + 4 * (lane >> 4);
      const float y2[4] = {cu2[c][h][0], cu2[c][h][1], cu2[c][h][2], cu2[c][h][3]};
      store4(Pp + 2 * DD + (int64_t)c2 * D + j2, y2);
    }
}

// =========================================================================
// bf16 apply forward tile (same contract as app_fwd_kernel)
template <int BJ, int BKK, int NST, bool OUT = false>
__global__ __launch_bounds__(NT, 2) void dapp_fwd_kernel(AppFwdArgs a) {
  // OUT = false: Hq = silu(q W1^T) * (q W3^T) into the Hq buffer.
  // OUT = true:  o = Hq W2^T, the same tiling with one product (A = Hq rows,
  //              B = W2 rows, both contracted over the hidden index).
  constexpr int NB = OUT ? 1 : 2;
  using TX = DTile<FBT, BKK>;
  using TW = DTile<BJ, BKK>;
  constexpr int STAGE = TX::BYTES + NB * TW::BYTES;
  constexpr int LPS = TX::INSTR + NB * TW::INSTR;
  constexpr int FN = BJ / 32;
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int D = a.D, Dh = a.Dh;
  // forward: contraction over d, output columns = hidden units (dh);
  // output mode: contraction over dh, output columns = o's d features
  const int KLEN = OUT ? Dh : D, NCOL = OUT ? D : Dh;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < a.ngroups && bid >= a.g[gi].tiles) bid -= a.g[gi++].tiles;
  const AppGroup& G = a.g[gi];
  const int njb = NCOL / BJ;
  const int tiles_t = (int)((G.len + FBT - 1) / FBT);
  const int per_inst = tiles_t * njb;
  const int inst = bid / per_inst;
  const int tile = bid % per_inst;
  const int tb = tile / njb, jb = tile % njb;
  const int64_t t0 = G.t0 + (int64_t)tb * FBT;
  const int64_t tend = G.t0 + G.len;
  const int j0 = jb * BJ;
  const int64_t DD = (int64_t)D * Dh;
  // A operand rows: queries (q rows t) or their gated hidden (Hq rows h0 + t - t0)
  const bf16_t* X = OUT ? reinterpret_cast<const bf16_t*>(a.H) + inst * a.h_bs
                        : reinterpret_cast<const bf16_t*>(a.q) + inst * a.q_bs;
  const int64_t xr0 = OUT ? G.h0 + (t0 - G.t0) : t0;
  const int64_t xrmax = OUT ? G.h0 + (tend - G.t0) - 1 : tend - 1;
  const bf16_t* B1 = reinterpret_cast<const bf16_t*>(OUT ? G.W2 : G.W1) + inst * DD;
  const bf16_t* B3 = reinterpret_cast<const bf16_t*>(G.W3) + inst * DD;

  const typename TX::Plan pq = TX::plan(X, KLEN, xr0, xrmax, 0, wave, lane);
  const typename TW::Plan p1 = TW::plan(B1, KLEN, j0, NCOL - 1, 0, wave, lane);
  const typename TW::Plan p3 = TW::plan(OUT ? B1 : B3, KLEN, j0, NCOL - 1, 0, wave, lane);
  auto issue_one = [&](int s, int buf, int idx) {
    char* st = smem + buf * STAGE;
    const int64_t off = (int64_t)s * BKK * 2;
    if (idx < TX::INSTR) TX::issue_one(st, pq, off, wave, idx);
    else if (idx < TX::INSTR + TW::INSTR) TW::issue_one(st + TX::BYTES, p1, off, wave, idx - TX::INSTR);
    else if constexpr (!OUT) TW::issue_one(st + TX::BYTES + TW::BYTES, p3, off, wave, idx - TX::INSTR - TW::INSTR);
  };
  f32x4 accA[4][FN], accB[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) accA[i][j] = accB[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, auto&& hook) {
    const char* st = smem + buf * STAGE;
    constexpr int NSLOT = (BKK / 32) * 4;
#pragma unroll
    for (int kk = 0; kk < BKK; kk += 32) {
      bf16x8 fq[4], f1[FN], f3[FN];
#pragma unroll
      for (int i = 0; i < 4; ++i) fq[i] = dfrag_row<TX>(st, wm * 64 + i * 16, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        f1[j] = dfrag_row<TW>(st + TX::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
        if constexpr (!OUT) f3[j] = dfrag_row<TW>(st + TX::BYTES + TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          accA[i][j] = mfma(f1[j], fq[i], accA[i][j]);   // swapped: lane owns 4 columns of one token
          if constexpr (!OUT) accB[i][j] = mfma(f3[j], fq[i], accB[i][j]);
        }
        hook((kk / 32) * 4 + i, NSLOT);
      }
    }
  };
  dpipeline_il<NST, LPS>(KLEN / BKK, issue_one, compute);

  // output rows: o rows t, or Hq rows h0 + t - t0
  bf16_t* Y = OUT ? reinterpret_cast<bf16_t*>(a.o) + inst * a.x_bs : reinterpret_cast<bf16_t*>(a.H) + inst * a.h_bs;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + wm * 64 + i * 16 + (lane & 15);
    if (t >= tend) continue;
    bf16_t* Yr = Y + (OUT ? t : G.h0 + (t - G.t0)) * (int64_t)NCOL;
    // per-token output scale (output mode only)
    const float ys = (OUT && a.oz != nullptr) ? silu(a.oz[inst * a.oz_bs + t]) : 1.f;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = j0 + wn * (BJ / 2) + j * 16 + 4 * (lane >> 4);
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = accA[i][j][r];
        h[r] = OUT ? x * ys : x * fast_sigmoid(x) * accB[i][j][r];
      }
      store4(Yr + col, h);
    }
  }
}

// =========================================================================
// Fused apply for a hidden width of one column block (dh = BJ): o = W2
// (silu(W1 q) * (W3 q)) for one 128-token tile of one apply group, the
// tile's gated hidden Hq kept in LDS and never written to HBM.  At this
// width the apply is bound by HBM traffic, and Hq's write and re-read would
// move as many bytes as q and o themselves.  Phase 1 computes Hq (the
// apply tile's forward, contraction over d) into LDS, cut into the dh / BKK
// k-stage tiles that phase 2 reads; phase 2 runs o = Hq W2^T over the
// output blocks with only the W2 tiles streamed.  The 32 KB of Hq and a
// two-stage ring leave room for two workgroups per CU.  4 waves: wave w
// owns tokens 64 (w >> 1) .. +63 and columns (BJ / 2)(w & 1) .. +BJ/2-1.
template <int BJ, int BKK, int NST>
__global__ __launch_bounds__(NT, 2) void dapp_fused_kernel(AppFwdArgs a) {
  using TX = DTile<FBT, BKK>;   // query stage tiles and the Hq k-stage tiles
  using TW = DTile<BJ, BKK>;    // W1, W3 (phase 1) and W2 (phase 2) rows
  constexpr int STAGE = TX::BYTES + 2 * TW::BYTES;
  constexpr int LPS1 = TX::INSTR + 2 * TW::INSTR;
  constexpr int LPS2 = TW::INSTR;
  constexpr int FN = BJ / 32;
  constexpr int NKH = BJ / BKK;   // k-stage tiles of Hq (dh = BJ)
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
  __shared__ __attribute__((aligned(1024))) char hq[NKH * TX::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int D = a.D;   // a.Dh == BJ
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < a.ngroups && bid >= a.g[gi].tiles) bid -= a.g[gi++].tiles;
  const AppGroup& G = a.g[gi];
  const int tiles_t = (int)((G.len + FBT - 1) / FBT);
  const int inst = bid / tiles_t, tb = bid % tiles_t;
  const int64_t t0 = G.t0 + (int64_t)tb * FBT;
  const int64_t tend = G.t0 + G.len;
  const int64_t DD = (int64_t)D * BJ;
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + inst * a.q_bs;
  const bf16_t* W1 = reinterpret_cast<const bf16_t*>(G.W1) + inst * DD;
  const bf16_t* W3 = reinterpret_cast<const bf16_t*>(G.W3) + inst * DD;
  const bf16_t* W2 = reinterpret_cast<const bf16_t*>(G.W2) + inst * DD;

  // ---- phase 1: Hq = silu(Q W1^T) * (Q W3^T) into LDS (contraction over d)
  {
    const typename TX::Plan pq = TX::plan(Q, D, t0, tend - 1, 0, wave, lane);
    const typename TW::Plan p1 = TW::plan(W1, D, 0, BJ - 1, 0, wave, lane);
    const typename TW::Plan p3 = TW::plan(W3, D, 0, BJ - 1, 0, wave, lane);
    auto issue_one = [&](int s, int buf, int idx) {
      char* st = smem + buf * STAGE;
      const int64_t off = (int64_t)s * BKK * 2;
      if (idx < TX::INSTR) TX::issue_one(st, pq, off, wave, idx);
      else if (idx < TX::INSTR + TW::INSTR) TW::issue_one(st + TX::BYTES, p1, off, wave, idx - TX::INSTR);
      else TW::issue_one(st + TX::BYTES + TW::BYTES, p3, off, wave, idx - TX::INSTR - TW::INSTR);
    };
    f32x4 accA[4][FN], accB[4][FN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) accA[i][j] = accB[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf, auto&& hook) {
      const char* st = smem + buf * STAGE;
      constexpr int NSLOT = (BKK / 32) * 4;
#pragma unroll
      for (int kk = 0; kk < BKK; kk += 32) {
        bf16x8 fq[4], f1[FN], f3[FN];
#pragma unroll
        for (int i = 0; i < 4; ++i) fq[i] = dfrag_row<TX>(st, wm * 64 + i * 16, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          f1[j] = dfrag_row<TW>(st + TX::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
          f3[j] = dfrag_row<TW>(st + TX::BYTES + TW::BYTES, wn * (BJ / 2) + j * 16, kk, lane);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            accA[i][j] = mfma(f1[j], fq[i], accA[i][j]);   // swapped: lane owns 4 columns of one token
            accB[i][j] = mfma(f3[j], fq[i], accB[i][j]);
          }
          hook((kk / 32) * 4 + i, NSLOT);
        }
      }
    };
    dpipeline_il<NST, LPS1>(D / BKK, issue_one, compute);
    // hidden columns c .. c+3 of token row tl -> k-stage tile c / BKK of Hq
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wm * 64 + i * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = wn * (BJ / 2) + j * 16 + 4 * (lane >> 4);
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = accA[i][j][r];
          h[r] = x * fast_sigmoid(x) * accB[i][j][r];
        }
        const int cc = c % BKK;
        char* dst = hq + (c / BKK) * TX::BYTES + TX::phys(tl, cc >> 3) * 16 + ((cc >> 2) & 1) * 8;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
      }
    }
  }
  __syncthreads();   // Hq visible to every wave; the ring is free

  // ---- phase 2: o[:, o0 .. o0 + BJ) = Hq W2[o0 .., :]^T (contraction over dh)
  bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + inst * a.x_bs;
  float ys[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = min(t0 + wm * 64 + i * 16 + (lane & 15), tend - 1);
    ys[i] = a.oz != nullptr ? silu(a.oz[inst * a.oz_bs + t]) : 1.f;
  }
  const int nob = D / BJ;
  for (int ob = 0; ob < nob; ++ob) {
    const int o0 = ob * BJ;
    const typename TW::Plan p2 = TW::plan(W2, BJ, o0, D - 1, 0, wave, lane);
    auto issue_one = [&](int s, int buf, int idx) {
      TW::issue_one(smem + buf * STAGE, p2, (int64_t)s * BKK * 2, wave, idx);
    };
    f32x4 acc[4][FN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int sidx = 0;
    auto compute = [&](int buf, auto&& hook) {
      const char* st = smem + buf * STAGE;
      const char* ht = hq + sidx * TX::BYTES;
      constexpr int NSLOT = (BKK / 32) * 4;
#pragma unroll
      for (int kk = 0; kk < BKK; kk += 32) {
        bf16x8 fh[4], fw[FN];
#pragma unroll
        for (int i = 0; i < 4; ++i) fh[i] = dfrag_row<TX>(ht, wm * 64 + i * 16, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fw[j] = dfrag_row<TW>(st, wn * (BJ / 2) + j * 16, kk, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma(fw[j], fh[i], acc[i][j]);
          hook((kk / 32) * 4 + i, NSLOT);
        }
      }
      ++sidx;
    };
    dpipeline_il<NST, LPS2>(NKH, issue_one, compute);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + wm * 64 + i * 16 + (lane & 15);
      if (t >= tend) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = o0 + wn * (BJ / 2) + j * 16 + 4 * (lane >> 4);
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = acc[i][j][r] * ys[i];
        store4(O + t * (int64_t)D + col, y);
      }
    }
    if (ob + 1 < nob) bar();   // every wave is done with the ring before the next block's loads
  }
}

}  // namespace lact
