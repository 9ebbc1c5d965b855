// Device kernels of the layer's backward pass (reverse sweep over the chunk
// recurrence).  The products of the sweep run on the grouped GEMM of
// lact_kernels.hpp with fp32 operands split into three bf16 planes; this file
// holds the elementwise terms, the per-row renormalisation backward, the
// momentum backward and the reductions, all in fp32.
//
// What is differentiated: the update and apply phases of "大块测试时训练
// （LaCT）技术解析" §2.1 (eqs. 2, 4-5), its §2.2.1 renormalisation (eq. 8)
// and Newton-Schulz map (eqs. 9-10), and the momentum of "LaCT架构核心思想解析"
// §1.2.  The derivatives are the chain rule through those steps:
//   S = silu(a), S' = s (1 + a (1 - s)), S'' = s (1 - s) (2 + a (1 - 2 s)),
//   s = sigmoid(a).
//
// Token buffers are [n, Cmax, Dh] fp32 (row t of instance i at
// i * buf_bs + t * Dh); only the chunk's first C rows are touched.  Weight-
// shaped sets are three arrays W1 [n, Dh, D], W2 [n, D, Dh], W3 [n, Dh, D].
#pragma once
#include "lact_kernels.hpp"

namespace lact {

struct BwdSig {
  float S, Sp, Spp;
};
__device__ __forceinline__ BwdSig bwd_sig(float a) {
  const float s = 1.0f / (1.0f + __expf(-a));
  BwdSig r;
  r.S = a * s;
  r.Sp = s * (1.0f + a * (1.0f - s));
  r.Spp = s * (1.0f - s) * (2.0f + a * (1.0f - 2.0f * s));
  return r;
}

// three weight-shaped arrays (W1, W2, W3 order)
struct MatP {
  float* p[3];
};
struct MatC {
  const float* p[3];
};

// rows of the three matrices, matrix-major: W1 has n Dh rows of D, W2 n D
// rows of Dh, W3 n Dh rows of D
__device__ __forceinline__ void mat_row(int64_t row, int n, int D, int Dh, int& mat, int64_t& off, int& len) {
  const int64_t r1 = (int64_t)n * Dh, r2 = (int64_t)n * D;
  if (row < r1) {
    mat = 0;
    off = row * D;
    len = D;
  } else if (row < r1 + r2) {
    mat = 1;
    off = (row - r1) * Dh;
    len = Dh;
  } else {
    mat = 2;
    off = (row - r1 - r2) * D;
    len = D;
  }
}

__global__ __launch_bounds__(NT) void bwd_fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] = v;
}

// Apply backward terms, in place: (Aq, Bq, dH) -> (dAq, dBq, Hq) with
// Aq = q W1^T, Bq = q W3^T, dH = dO W2: Hq = S(Aq) Bq, dAq = dH Bq S'(Aq),
// dBq = dH S(Aq).
__global__ __launch_bounds__(NT) void bwd_app_elem_kernel(float* Aq, float* Bq, float* dH, int n, int64_t C, int Dh,
                                                          int64_t buf_bs) {
  const int64_t per = C * Dh, total = per * n;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total; e += (int64_t)gridDim.x * NT) {
    const int64_t i = e / per, r = e % per;
    const int64_t o = i * buf_bs + r;
    const float a = Aq[o], b = Bq[o], g = dH[o];
    const BwdSig z = bwd_sig(a);
    Aq[o] = g * b * z.Sp;
    Bq[o] = g * z.S;
    dH[o] = z.S * b;
  }
}

// Apply backward terms with the per-token output scale o_t * silu(z_t), one
// wave per token row, in place: dH holds dO W2 for the UNSCALED cotangent;
// with s_t = silu(z_t): dAq = s_t dH Bq S'(Aq), dBq = s_t dH S(Aq), and dH
// becomes s_t Hq (so that dW2 += dO^T (s Hq)); doz_t = silu'(z_t) <dH_t, Hq_t>
// (= silu'(z_t) <dO_t, o_t>, o the unscaled output).
__global__ __launch_bounds__(NT) void bwd_app_elem_oz_kernel(float* Aq, float* Bq, float* dH, const float* oz,
                                                             int64_t oz_bs, int64_t t0, float* doz, int n, int64_t C,
                                                             int Dh, int64_t buf_bs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  if (row >= (int64_t)n * C) return;
  const int64_t i = row / C, t = row % C;
  const float z = oz[i * oz_bs + t0 + t];
  const float sg = 1.0f / (1.0f + __expf(-z));
  const float sz = z * sg, spz = sg * (1.0f + z * (1.0f - sg));
  const int64_t base = i * buf_bs + t * Dh;
  float dz = 0.f;
  for (int j = lane; j < Dh; j += WAVE) {
    const int64_t o = base + j;
    const float a = Aq[o], b = Bq[o], g = dH[o];
    const BwdSig q = bwd_sig(a);
    const float hq = q.S * b;
    dz += g * hq;
    Aq[o] = sz * g * b * q.Sp;
    Bq[o] = sz * g * q.S;
    dH[o] = sz * hq;
  }
  dz = wave_sum(dz);
  if (lane == 0) doz[i * oz_bs + t0 + t] = spz * dz;
}

__device__ __forceinline__ float bwd_ld(const float* p) { return *p; }
__device__ __forceinline__ float bwd_ld(const bf16_t* p) { return __uint_as_float((uint32_t)p->x << 16); }

// q / k pre-processing for the backward, kept in fp32 (the forward's
// "LaCT架构核心思想解析" §1.2 map x -> silu(x) / ||silu(x)|| over a token's d
// features), one wave per token row; prep = 0 copies x to fp32 unchanged.
template <typename T>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(const T* src, float* dst, int64_t rows, int D, int prep) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* x = src + row * D;
  float* y = dst + row * D;
  if (!prep) {
    for (int j = lane; j < D; j += WAVE) y[j] = bwd_ld(x + j);
    return;
  }
  float ss = 0.f;
  for (int j = lane; j < D; j += WAVE) {
    const float v = bwd_ld(x + j), sv = v / (1.0f + __expf(-v));
    ss += sv * sv;
  }
  const float inv = 1.0f / sqrtf(wave_sum(ss));
  for (int j = lane; j < D; j += WAVE) {
    const float v = bwd_ld(x + j);
    y[j] = v / (1.0f + __expf(-v)) * inv;
  }
}

// Backward of the pre-processing, in place on the cotangent g, one wave per
// row: with s = silu(x), n = ||s||: g <- silu'(x) (g - s (s . g) / n^2) / n.
template <typename T>
__global__ __launch_bounds__(NT) void bwd_prep_vjp_kernel(const T* src, float* g, int64_t rows, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* x = src + row * D;
  float* gr = g + row * D;
  float ss = 0.f, dt = 0.f;
  for (int j = lane; j < D; j += WAVE) {
    const float v = bwd_ld(x + j), sv = v / (1.0f + __expf(-v));
    ss += sv * sv;
    dt += sv * gr[j];
  }
  ss = wave_sum(ss);
  dt = wave_sum(dt);
  const float n = sqrtf(ss), c = dt / ss;
  for (int j = lane; j < D; j += WAVE) {
    const float v = bwd_ld(x + j);
    const float sg = 1.0f / (1.0f + __expf(-v));
    const float sv = v * sg, sp = sg * (1.0f + v * (1.0f - sg));
    gr[j] = sp * (gr[j] - sv * c) / n;
  }
}

// Update terms of the chunk: E1 = lr1 G B S'(A), E3 = lr3 G S(A),
// H2 = lr2 S(A) B (so U1 = E1^T K, U3 = E3^T K, U2 = V^T H2).
__global__ __launch_bounds__(NT) void bwd_upd_terms_kernel(const float* A, const float* B, const float* G,
                                                           const float* lr, int64_t lr_bs, int64_t t0, float* E1,
                                                           float* E3, float* H2, int n, int64_t C, int Dh,
                                                           int64_t buf_bs) {
  const int64_t per = C * Dh, total = per * n;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total; e += (int64_t)gridDim.x * NT) {
    const int64_t i = e / per, r = e % per;
    const int64_t t = r / Dh;
    const int64_t o = i * buf_bs + r;
    const float* l = lr + i * lr_bs + (t0 + t) * 3;
    const float a = A[o], b = B[o], g = G[o];
    const BwdSig z = bwd_sig(a);
    E1[o] = l[0] * g * b * z.Sp;
    E3[o] = l[2] * g * z.S;
    H2[o] = l[1] * z.S * b;
  }
}

// Backward of the update terms, one wave per token row, in place:
// (gE1, gE3, gH2) -> (gA, gB, gG) and the row sums dlr[t] (zeros for the
// chunk's rows are not needed: every row is written).
//   gA = gE1 lr1 G B S'' + gE3 lr3 G S' + gH2 lr2 B S'
//   gB = gE1 lr1 G S' + gH2 lr2 S
//   gG = gE1 lr1 B S' + gE3 lr3 S
//   dlr1 = sum gE1 G B S',  dlr2 = sum gH2 S B,  dlr3 = sum gE3 G S
__global__ __launch_bounds__(NT) void bwd_upd_elem_kernel(const float* A, const float* B, const float* G,
                                                          const float* lr, int64_t lr_bs, int64_t t0, float* gE1,
                                                          float* gE3, float* gH2, float* dlr, int n, int64_t C,
                                                          int Dh, int64_t buf_bs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  if (row >= (int64_t)n * C) return;
  const int64_t i = row / C, t = row % C;
  const int64_t base = i * buf_bs + t * Dh;
  const float* l = lr + i * lr_bs + (t0 + t) * 3;
  const float e1 = l[0], e2 = l[1], e3 = l[2];
  float s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int j = lane; j < Dh; j += WAVE) {
    const int64_t o = base + j;
    const float a = A[o], b = B[o], g = G[o];
    const float ge1 = gE1[o], ge3 = gE3[o], gh2 = gH2[o];
    const BwdSig z = bwd_sig(a);
    s1 += ge1 * g * b * z.Sp;
    s2 += gh2 * z.S * b;
    s3 += ge3 * g * z.S;
    gE1[o] = ge1 * e1 * g * b * z.Spp + ge3 * e3 * g * z.Sp + gh2 * e2 * b * z.Sp;
    gE3[o] = ge1 * e1 * g * z.Sp + gh2 * e2 * z.S;
    gH2[o] = ge1 * e1 * b * z.Sp + ge3 * e3 * z.S;
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  s3 = wave_sum(s3);
  if (lane == 0) {
    float* d = dlr + i * lr_bs + (t0 + t) * 3;
    d[0] = s1;
    d[1] = s2;
    d[2] = s3;
  }
}

// Renormalisation backward, one wave per row.  The step was W' = W + sgn
// step; the forward output Y = W' ||W_r|| / ||W'_r||.  In: gW = cotangent of
// Y.  Out: gWp = cotangent of W' (s (gY - (gY.w) w), s = ||W_r|| / ||W'_r||,
// w = W'_r / ||W'_r||) and gW = cotangent of W through both W' and the row's
// old norm (gWp + (gY.w) W_r / ||W_r||).  Without renorm Y = W': gWp = gY,
// gW = gY.
__global__ __launch_bounds__(NT) void bwd_renorm_kernel(MatC W, MatC step, float sgn, MatP gW, MatP gWp, int n, int D,
                                                        int Dh, int renorm) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)n * (2 * Dh + D);
  if (row >= rows) return;
  int mat, len;
  int64_t off;
  mat_row(row, n, D, Dh, mat, off, len);
  const float* w = W.p[mat] + off;
  const float* st = step.p[mat] + off;
  float* g = gW.p[mat] + off;
  float* gp = gWp.p[mat] + off;
  if (!renorm) {
    for (int j = lane; j < len; j += WAVE) gp[j] = g[j];
    return;
  }
  float so = 0.f, sn = 0.f, dt = 0.f;
  for (int j = lane; j < len; j += WAVE) {
    const float x = w[j], xp = x + sgn * st[j];
    so += x * x;
    sn += xp * xp;
    dt += g[j] * xp;
  }
  so = wave_sum(so);
  sn = wave_sum(sn);
  dt = wave_sum(dt);
  const float n_old = sqrtf(so), n_new = sqrtf(sn);
  const float s = n_old / n_new;
  const float dot = dt / n_new;          // gY . w
  const float inv_new = 1.0f / n_new, inv_old = 1.0f / n_old;
  for (int j = lane; j < len; j += WAVE) {
    const float x = w[j], xp = x + sgn * st[j];
    const float gpj = s * (g[j] - dot * xp * inv_new);
    gp[j] = gpj;
    g[j] = gpj + dot * x * inv_old;
  }
}

// Momentum backward (M_next = bbar M - U, the weight step reads M_next with
// sign -1): gMt = gM_next - gX, where gX is the cotangent reaching M_next
// through the weight step (gW' for MOMENTUM, the Newton-Schulz backward of
// gW' for MUON_MOMENTUM).  Out: gM <- bbar gMt (cotangent of the old M),
// gU = -gMt, and per-block partial sums of gMt . M_old for d(bbar).
// bbar = the mean of beta over the chunk's rows [t0, t0 + C), summed by each
// workgroup itself (C values from L2).  Grid: (nblk, 3 matrices, n).
__global__ __launch_bounds__(NT) void bwd_mom_kernel(MatP gM, MatC gX, MatC Mold, const float* beta, int64_t beta_bs,
                                                     int64_t t0, int64_t C, MatP gU, float* part, int64_t DD,
                                                     int nblk) {
  __shared__ float red[NT / WAVE];
  __shared__ float s_bb;
  const int b = blockIdx.x, mat = blockIdx.y, i = blockIdx.z;
  {
    float sb = 0.f;
    for (int64_t t = threadIdx.x; t < C; t += NT) sb += beta[i * beta_bs + t0 + t];
    sb = wave_sum(sb);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sb;
    __syncthreads();
    if (threadIdx.x == 0) {
      float tb = 0.f;
      for (int w = 0; w < NT / WAVE; ++w) tb += red[w];
      s_bb = tb / (float)C;
    }
    __syncthreads();
  }
  const float bb = s_bb;
  const int64_t per = (DD + nblk - 1) / nblk;
  const int64_t e0 = (int64_t)b * per, e1 = min(DD, e0 + per);
  float* gm = gM.p[mat] + (int64_t)i * DD;
  const float* gx = gX.p[mat] + (int64_t)i * DD;
  const float* mo = Mold.p[mat] + (int64_t)i * DD;
  float* gu = gU.p[mat] + (int64_t)i * DD;
  float s = 0.f;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += NT) {
    const float gmt = gm[e] - gx[e];
    s += gmt * mo[e];
    gm[e] = bb * gmt;
    gu[e] = -gmt;
  }
  s = wave_sum(s);
  __syncthreads();   // red[] is reused
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < NT / WAVE; ++w) t += red[w];
    part[((int64_t)i * 3 + mat) * nblk + b] = t;
  }
}

// dbeta[t] = d(bbar) / C for the chunk's rows (bbar is the chunk mean);
// part holds 3 nblk partial sums per instance
__global__ __launch_bounds__(NT) void bwd_mom_finish_kernel(const float* part, int nblk, float* dbeta, int64_t beta_bs,
                                                            int64_t t0, int64_t C) {
  __shared__ float s_g;
  const int i = blockIdx.y;
  if (threadIdx.x == 0) {
    float g = 0.f;
    for (int b = 0; b < 3 * nblk; ++b) g += part[(int64_t)i * 3 * nblk + b];
    s_g = g / (float)C;
  }
  __syncthreads();
  const float g = s_g;
  for (int64_t t = (int64_t)blockIdx.x * NT + threadIdx.x; t < C; t += (int64_t)gridDim.x * NT)
    dbeta[i * beta_bs + t0 + t] = g;
}

// fp32 -> P bf16 planes (the rounding of split_planes), same layout: batch
// entries of `per` valid elements at stride bs; plane p at out + p * ps
template <int P>
__global__ __launch_bounds__(NT) void bwd_planes_kernel(const float* x, int64_t per, int64_t bs, int batch,
                                                        bf16_t* out, int64_t ps) {
  const int64_t nq = per / 4, total = nq * batch;
  for (int64_t q = blockIdx.x * (int64_t)NT + threadIdx.x; q < total; q += (int64_t)gridDim.x * NT) {
    const int64_t off = (q / nq) * bs + (q % nq) * 4;
    const float4 v = *reinterpret_cast<const float4*>(x + off);
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t h[4][P];
#pragma unroll
    for (int r = 0; r < 4; ++r) split_planes<P>(e[r], h[r]);
#pragma unroll
    for (int pl = 0; pl < P; ++pl)
      *reinterpret_cast<uint2*>(out + pl * ps + off) = make_uint2(h[0][pl] | (h[1][pl] << 16), h[2][pl] | (h[3][pl] << 16));
  }
}

// Split-K reduction: C[b][m, n] = sum_s P[s][b][m, n] + beta Cin[b][m, n],
// partials compact ([S][batch][M][N]); Cin has C's strides and may be C.
__global__ __launch_bounds__(NT) void bwd_splitsum_kernel(const float* P, int S, int batch, int M, int N, float* C,
                                                          int64_t ldc, int64_t c_bs, const float* Cin, float beta) {
  const int64_t mn = (int64_t)M * N, tot = mn * batch;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < tot; e += (int64_t)gridDim.x * NT) {
    const int64_t b = e / mn, r = e % mn;
    const int64_t o = b * c_bs + (r / N) * ldc + r % N;
    float v = 0.f;
    for (int q = 0; q < S; ++q) v += P[(int64_t)q * tot + e];
    if (Cin) v += beta * Cin[o];
    C[o] = v;
  }
}

// ----------------------------------------------------------------- Newton-Schulz
// Working frame: every matrix of the set as X [m, k] with m = min(D, Dh) and
// k = max(D, Dh) (matrices with more rows than columns are transposed, as the
// forward map does), batch index b = mat * n + i, stride D Dh.

__device__ __forceinline__ void frame_map(int mat, int D, int Dh, int64_t x, int64_t y, int64_t& orig) {
  const int rows = mat == 1 ? D : Dh, cols = mat == 1 ? Dh : D;
  const bool tr = rows > cols;
  orig = tr ? y * cols + x : x * cols + y;   // frame (x, y) = orig (y, x) when transposed
}

// Partial sums of a.b (or a.a with b == nullptr) per (matrix, instance):
// grid (nblk, 3 n); part[(mat n + i) nblk + blk].
__global__ __launch_bounds__(NT) void bwd_dot_kernel(MatC a, MatC b, float* part, int n, int64_t DD, int nblk) {
  __shared__ float red[NT / WAVE];
  const int bi = blockIdx.y, blk = blockIdx.x;
  const int mat = bi / n, i = bi % n;
  const int64_t per = (DD + nblk - 1) / nblk;
  const int64_t e0 = (int64_t)blk * per, e1 = min(DD, e0 + per);
  const float* pa = a.p[mat] + (int64_t)i * DD;
  const float* pb = b.p[0] ? b.p[mat] + (int64_t)i * DD : pa;
  float s = 0.f;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += NT) s += pa[e] * pb[e];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < NT / WAVE; ++w) t += red[w];
    part[(int64_t)bi * nblk + blk] = t;
  }
}

// X0 (frame) = src / (||src|| + eps) per matrix; nrm[b] = ||src_b||
// (from the partial sums of squares).  Grid-stride over 3 n D Dh elements.
__global__ __launch_bounds__(NT) void bwd_ns_init_kernel(MatC src, const float* part, int nblk, float* X, float* nrm,
                                                         int n, int D, int Dh, float eps) {
  const int64_t DD = (int64_t)D * Dh, tot = 3 * n * DD;
  const int k = D > Dh ? D : Dh;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < tot; e += (int64_t)gridDim.x * NT) {
    const int64_t bi = e / DD, r = e % DD;
    const int mat = (int)(bi / n), i = (int)(bi % n);
    float ss = 0.f;
    for (int q = 0; q < nblk; ++q) ss += part[bi * nblk + q];
    const float nr = sqrtf(ss);
    if (r == 0) nrm[bi] = nr;
    int64_t o;
    frame_map(mat, D, Dh, r / k, r % k, o);
    X[e] = src.p[mat][(int64_t)i * DD + o] / (nr + eps);
  }
}

// frame -> original layout (dst = sgn frame value)
__global__ __launch_bounds__(NT) void bwd_frame_out_kernel(const float* X, MatP dst, float sgn, int n, int D, int Dh) {
  const int64_t DD = (int64_t)D * Dh, tot = 3 * n * DD;
  const int k = D > Dh ? D : Dh;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < tot; e += (int64_t)gridDim.x * NT) {
    const int64_t bi = e / DD, r = e % DD;
    const int mat = (int)(bi / n), i = (int)(bi % n);
    int64_t o;
    frame_map(mat, D, Dh, r / k, r % k, o);
    dst.p[mat][(int64_t)i * DD + o] = sgn * X[e];
  }
}

// original layout -> frame (no scale)
__global__ __launch_bounds__(NT) void bwd_frame_in_kernel(MatC src, float* X, int n, int D, int Dh) {
  const int64_t DD = (int64_t)D * Dh, tot = 3 * n * DD;
  const int k = D > Dh ? D : Dh;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < tot; e += (int64_t)gridDim.x * NT) {
    const int64_t bi = e / DD, r = e % DD;
    const int mat = (int)(bi / n), i = (int)(bi % n);
    int64_t o;
    frame_map(mat, D, Dh, r / k, r % k, o);
    X[e] = src.p[mat][(int64_t)i * DD + o];
  }
}

// Q = gA + gA^T for a batch of m x m matrices
__global__ __launch_bounds__(NT) void bwd_symadd_kernel(const float* gA, float* Q, int m, int64_t batch) {
  const int64_t mm = (int64_t)m * m, tot = mm * batch;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < tot; e += (int64_t)gridDim.x * NT) {
    const int64_t b = e / mm, r = e % mm;
    const int64_t x = r / m, y = r % m;
    Q[e] = gA[e] + gA[b * mm + y * m + x];
  }
}

// Normalisation backward: gG = g / (||G|| + eps) - G <g, G> / ((||G|| + eps)^2 ||G||)
// (the second term only for ||G|| > 0).  g and G in the original layout;
// part holds the partial sums of <g, G>.  out may alias g.
__global__ __launch_bounds__(NT) void bwd_ns_finish_kernel(MatC g, MatC G, const float* nrm, const float* part,
                                                           int nblk, MatP out, float sgn, int n, int64_t DD,
                                                           float eps) {
  const int64_t tot = 3 * n * DD;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < tot; e += (int64_t)gridDim.x * NT) {
    const int64_t bi = e / DD, r = e % DD;
    const int mat = (int)(bi / n), i = (int)(bi % n);
    float dot = 0.f;
    for (int q = 0; q < nblk; ++q) dot += part[bi * nblk + q];
    const float nr = nrm[bi], ne = nr + eps;
    const int64_t o = (int64_t)i * DD + r;
    float v = g.p[mat][o] / ne;
    if (nr > 0.f) v -= G.p[mat][o] * (dot / (ne * ne * nr));
    out.p[mat][o] = sgn * v;
  }
}

}  // namespace lact
