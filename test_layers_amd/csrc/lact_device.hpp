// Device building blocks for the gfx950 LaCT kernels: bf16 rounding and
// plane splitting, LDS tile loaders (row-k and column-k sources), and the
// 16x16x32 bf16 MFMA fragment loop.
//
// Precision model.  Every product runs on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  An fp32 operand is split into P bf16 planes
// (x = p0 + p1 + p2, each plane the round-to-nearest-even bf16 of what the
// previous planes left); P = 3 reproduces the fp32 significand.  A product of
// a P_A-plane operand with a P_B-plane operand sums the plane pairs (i, j)
// with i + j < max(P_A, P_B): the dropped pairs are below fp32 rounding for
// P = 3, so a 3-plane product is fp32-grade, a 1-plane product is plain bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lact {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16_t { uint16_t x; };  // storage type of bf16 tensors (raw bits)

constexpr int WAVE = 64;

// float -> bf16 bits, round to nearest even (gfx950's conversion instruction)
__device__ __forceinline__ uint32_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two floats -> packed bf16 pair (lo in bits 0..15), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

template <int P>
__device__ __forceinline__ void split_planes(float x, uint32_t (&h)[P]) {
  float r = x;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    h[p] = f2bf(r);
    r = r - bf2f(h[p]);  // exact: r and its bf16 rounding share an exponent range
  }
}

template <typename T> struct io_traits;
template <> struct io_traits<float> {
  static constexpr int VE = 4;  // elements per 16-byte vector
  __device__ static float to_f(float x) { return x; }
  __device__ static void store(float* p, float x) { *p = x; }
};
template <> struct io_traits<bf16_t> {
  static constexpr int VE = 8;
  __device__ static void store(bf16_t* p, float x) { p->x = (uint16_t)f2bf(x); }
};

// four consecutive values as one vector store (16 B fp32 / 8 B bf16)
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, const float (&v)[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float (&v)[4]) {
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  v[0] = bf2f(x.x & 0xffffu);
  v[1] = bf2f(x.x >> 16);
  v[2] = bf2f(x.y & 0xffffu);
  v[3] = bf2f(x.y >> 16);
}

// one 16-byte chunk of a row as floats (4 fp32 or 8 bf16 values)
__device__ __forceinline__ void load_chunk(const float* p, float (&v)[4]) { load4(p, v); }
__device__ __forceinline__ void load_chunk(const bf16_t* p, float (&v)[8]) {
  const uint4 x = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf2f(w[i] & 0xffffu);
    v[2 * i + 1] = bf2f(w[i] >> 16);
  }
}
__device__ __forceinline__ void store_chunk(float* p, const float (&v)[4]) { store4(p, v); }
__device__ __forceinline__ void store_chunk(bf16_t* p, const float (&v)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// LDS tile: ROWS rows of BK k-values (bf16 bits), padded by 8 elements so
// that the 16-byte fragment reads of 8 consecutive rows fall in distinct bank
// groups.  Plane p of a multi-plane tile starts at p * PLANE.
template <int ROWS, int BK>
struct TileGeom {
  static constexpr int STRIDE = BK + 8;
  static constexpr int PLANE = ROWS * STRIDE;
};

// -------------------------------------------------------------------------
// Row-k source: element (row, k) at base[row * ld + k], k contiguous.
// Rows >= rows_valid read as zero.  k0 + BK must not pass the row end.
template <typename T, int P, int ROWS, int BK, int NT>
struct RowKLoader {
  static constexpr int VE = io_traits<T>::VE;
  static constexpr int VPR = BK / VE;
  static constexpr int NV = ROWS * VPR;
  static constexpr int IT = (NV + NT - 1) / NT;
  static constexpr int STRIDE = TileGeom<ROWS, BK>::STRIDE;
  static constexpr int PLANE = TileGeom<ROWS, BK>::PLANE;
  static_assert(BK % VE == 0, "BK must hold whole vectors");
  static_assert(sizeof(T) == 4 || P == 1, "bf16 sources are exact in one plane");
  uint4 r[IT];

  __device__ __forceinline__ void load(const T* base, int64_t ld, int64_t row0, int64_t rows_valid,
                                       int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      int v = tid + i * NT;
      r[i] = zero4();
      if (NV % NT == 0 || v < NV) {
        int row = v / VPR, seg = v % VPR;
        int64_t gr = row0 + row;
        if (gr < rows_valid) r[i] = *reinterpret_cast<const uint4*>(base + gr * ld + k0 + seg * VE);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      int v = tid + i * NT;
      if (NV % NT == 0 || v < NV) {
        int row = v / VPR, seg = v % VPR;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint4*>(lds + row * STRIDE + seg * 8) = r[i];
        } else {
          const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
          uint32_t h[4][P];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_planes<P>(__uint_as_float(w[e]), h[e]);
#pragma unroll
          for (int p = 0; p < P; ++p) {
            uint2 pk = make_uint2(h[0][p] | (h[1][p] << 16), h[2][p] | (h[3][p] << 16));
            *reinterpret_cast<uint2*>(lds + p * PLANE + row * STRIDE + seg * 4) = pk;
          }
        }
      }
    }
  }
};

// -------------------------------------------------------------------------
// Column-k source: element (m, k) at base[k * ld + m], m contiguous (a
// token-major activation read along tokens).  Each thread reads KB
// consecutive k-rows of one 16-byte m-vector and writes them transposed
// (KB k-values per m-row) into the k-contiguous LDS tile.  k-rows >= k_valid
// and m >= m_valid read as zero (m_valid is a multiple of the vector width).
template <typename T, int P, int ROWS, int BK, int NT>
struct ColKLoader {
  static constexpr int VE = io_traits<T>::VE;
  static constexpr int KB = 4;
  static constexpr int MB = ROWS / VE;          // m-vectors per k-row
  static constexpr int NB = (BK / KB) * MB;     // thread blocks per tile
  static constexpr int IT = (NB + NT - 1) / NT;
  static constexpr int STRIDE = TileGeom<ROWS, BK>::STRIDE;
  static constexpr int PLANE = TileGeom<ROWS, BK>::PLANE;
  static_assert(ROWS % VE == 0 && BK % KB == 0, "tile shape");
  static_assert(sizeof(T) == 4 || P == 1, "bf16 sources are exact in one plane");
  uint4 r[IT][KB];

  __device__ __forceinline__ void load(const T* base, int64_t ld, int64_t m0, int64_t m_valid,
                                       int64_t k0, int64_t k_valid, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      int b = tid + i * NT;
      // consecutive threads take consecutive k-blocks of one m-vector so that
      // their transposed LDS writes land side by side
      int kb = b % (BK / KB), mb = b / (BK / KB);
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        r[i][kk] = zero4();
        if (NB % NT == 0 || b < NB) {
          int64_t gk = k0 + kb * KB + kk, gm = m0 + mb * VE;
          if (gk < k_valid && gm < m_valid) r[i][kk] = *reinterpret_cast<const uint4*>(base + gk * ld + gm);
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      int b = tid + i * NT;
      if (!(NB % NT == 0 || b < NB)) continue;
      int kb = b % (BK / KB), mb = b / (BK / KB);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint32_t e[KB];
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            const uint32_t w[4] = {r[i][kk].x, r[i][kk].y, r[i][kk].z, r[i][kk].w};
            e[kk] = (w[m >> 1] >> ((m & 1) * 16)) & 0xFFFFu;
          }
          uint2 pk = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
          *reinterpret_cast<uint2*>(lds + (mb * 8 + m) * STRIDE + kb * KB) = pk;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint32_t h[KB][P];
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            const uint32_t w[4] = {r[i][kk].x, r[i][kk].y, r[i][kk].z, r[i][kk].w};
            split_planes<P>(__uint_as_float(w[m]), h[kk]);
          }
#pragma unroll
          for (int p = 0; p < P; ++p) {
            uint2 pk = make_uint2(h[0][p] | (h[1][p] << 16), h[2][p] | (h[3][p] << 16));
            *reinterpret_cast<uint2*>(lds + p * PLANE + (mb * 4 + m) * STRIDE + kb * KB) = pk;
          }
        }
      }
    }
  }
};

template <typename T, int P, int ROWS, int BK, int NT, bool COLK>
struct LoaderSel;
template <typename T, int P, int ROWS, int BK, int NT>
struct LoaderSel<T, P, ROWS, BK, NT, false> { using type = RowKLoader<T, P, ROWS, BK, NT>; };
template <typename T, int P, int ROWS, int BK, int NT>
struct LoaderSel<T, P, ROWS, BK, NT, true> { using type = ColKLoader<T, P, ROWS, BK, NT>; };

// -------------------------------------------------------------------------
// MFMA fragments.  For v_mfma_f32_16x16x32_bf16, lane l supplies row
// (l % 16) and k-values 8*(l/16) .. 8*(l/16)+7 of each operand, and receives
// rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16) of the 16x16 result.
template <int STRIDE>
__device__ __forceinline__ bf16x8 frag(const uint16_t* lds, int row0, int kk, int lane) {
  return *reinterpret_cast<const bf16x8*>(lds + (row0 + (lane & 15)) * STRIDE + kk + 8 * (lane >> 4));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc[i][j] += sum over plane pairs of A[i] * B[j] for one 32-wide k slice.
// Smaller plane pairs go first (they carry the low-order bits).
// SWAP = false: acc[i][j] lane l holds C rows 4*(l/16)+r, column l%16 of the
//               16x16 block (4 consecutive rows per lane);
// SWAP = true:  the operands enter the MFMA in the other order, so lane l
//               holds row l%16, columns 4*(l/16)+r (4 consecutive columns).
template <int PA, int PB, int FM, int FN, int SA, int SB, bool SWAP = false>
__device__ __forceinline__ void mma_tile(f32x4 (&acc)[FM][FN], const uint16_t* la, int pla_stride,
                                         int arow0, const uint16_t* lb, int plb_stride, int brow0,
                                         int kk, int lane) {
  constexpr int PM = PA > PB ? PA : PB;
  bf16x8 a[PA][FM], b[PB][FN];
#pragma unroll
  for (int p = 0; p < PA; ++p)
#pragma unroll
    for (int i = 0; i < FM; ++i) a[p][i] = frag<SA>(la + p * pla_stride, arow0 + i * 16, kk, lane);
#pragma unroll
  for (int p = 0; p < PB; ++p)
#pragma unroll
    for (int j = 0; j < FN; ++j) b[p][j] = frag<SB>(lb + p * plb_stride, brow0 + j * 16, kk, lane);
#pragma unroll
  for (int s = PM - 1; s >= 0; --s)
#pragma unroll
    for (int pa = 0; pa < PA; ++pa)
#pragma unroll
      for (int pb = 0; pb < PB; ++pb)
        if (pa + pb == s)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              if constexpr (SWAP) acc[i][j] = mfma(b[pb][j], a[pa][i], acc[i][j]);
              else acc[i][j] = mfma(a[pa][i], b[pb][j], acc[i][j]);
            }
}

template <int V>
using IC = std::integral_constant<int, V>;

// Software pipeline over nk k-stages.  Tiles are fetched two stages ahead
// into two alternating register sets (fetch(IC<set>, stage)), written to one
// of two LDS buffers (put(IC<set>, IC<buf>)) a full stage after their loads
// were issued, and consumed by compute(IC<buf>); one barrier per stage.  With
// LDS_STAGES = 1 the single buffer is rewritten between two barriers.
template <int LDS_STAGES, class F, class P, class C>
__device__ __forceinline__ void pipeline(int nk, F&& fetch, P&& put, C&& compute) {
  if (nk <= 0) return;
  fetch(IC<0>{}, 0);
  if (nk > 1) fetch(IC<1>{}, 1);
  if constexpr (LDS_STAGES == 2) {
    put(IC<0>{}, IC<0>{});
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      if (kt + 2 < nk) fetch(IC<0>{}, kt + 2);
      compute(IC<0>{});
      if (kt + 1 < nk) put(IC<1>{}, IC<1>{});
      __syncthreads();
      if (kt + 1 >= nk) break;
      if (kt + 3 < nk) fetch(IC<1>{}, kt + 3);
      compute(IC<1>{});
      if (kt + 2 < nk) put(IC<0>{}, IC<0>{});
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < nk; kt += 2) {
      put(IC<0>{}, IC<0>{});
      __syncthreads();
      if (kt + 2 < nk) fetch(IC<0>{}, kt + 2);
      compute(IC<0>{});
      __syncthreads();
      if (kt + 1 >= nk) break;
      put(IC<1>{}, IC<0>{});
      __syncthreads();
      if (kt + 3 < nk) fetch(IC<1>{}, kt + 3);
      compute(IC<0>{});
      __syncthreads();
    }
  }
}

// Workgroup b runs on XCD b % 8 (round-robin dispatch; each XCD has its own
// L2).  Map it to a logical index so that each XCD receives one contiguous
// block of logical indices: tiles that share operands then share an L2.
constexpr int NXCD = 8;
constexpr int NCU = 256;   // compute units (32 per XCD)
__device__ __forceinline__ int xcd_remap(int b, int nwg) {
  const int per = nwg / NXCD, rem = nwg % NXCD;
  const int x = b % NXCD, s = b / NXCD;
  return x < rem ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, WAVE);
  return x;
}

// logistic function with the hardware reciprocal (1 ulp) instead of an IEEE division
__device__ __forceinline__ float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
// x sigmoid(x) with an IEEE division (x -> -inf gives -0, x -> +inf gives x)
__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

}  // namespace lact
