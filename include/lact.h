/*
 * lact.h -- C ABI of liblact, the MI355X (gfx950) LaCT fast-weight layer.
 *
 * The layer (Large-Chunk Test-Time Training) keeps, per instance
 * (batch x head), a SwiGLU fast-weight MLP
 *
 *     f_W(x) = W2 (silu(W1 x) * (W3 x)),   W1, W3: [dh x d],  W2: [d x dh],
 *
 * updates it once per large chunk of tokens from the lr-weighted gradient of
 * the loss -<f_W(k), v> summed over the chunk, and applies it to the chunk's
 * queries.  Sources, by page title and labelled part:
 *   "大块测试时训练（LaCT）技术解析" (dpshk.com) §2.1: update = gradient summed
 *       over the whole chunk (eqs. 4-5); apply = updated weights on all
 *       queries (eq. 2); §2.2.1: L2 weight normalisation (eq. 8), Muon
 *       (eqs. 9-10); §2.2.2: context-parallel gradient sum.
 *   "LaCT：以大分块更新人工智能的临时记忆" (iplexlaw.co.kr): sections
 *       "局部注意力与非线性记忆相互补充" (SwiGLU memory, negative inner-product
 *       loss, per-token lr, GD / momentum / Muon, L2 normalisation) and
 *       "更新顺序必须遵守信息可见范围" (apply-then-update for language,
 *       update-then-apply for posed image sets, video updates only on clean
 *       chunks).
 *   "LaCT架构核心思想解析" (gsyq.cn) §1.2 (three fast-weight matrices,
 *       momentum with per-token beta, W <- L2norm(W - M), silu and L2
 *       normalisation of q and k) and §2.1 (lr laid out as [(b nh), l, 3];
 *       the layer output scaled per token by silu of a projection).
 *
 * Conventions fixed by this library where the pages leave a choice:
 *   - lr[..., j-1] scales the gradient of W_j (j = 1, 2, 3).
 *   - U_j = -sum_{i in chunk} lr_ij dl_i/dW_j (a sum, not a mean).
 *     GD: W' = W + U.  MOMENTUM: M <- mean_chunk(beta) M - U, W' = W - M.
 *     MUON: W' = W + NS(U), NS = ns_iters quintic Newton-Schulz steps with
 *     (a, b, c) = (3.4445, -4.7750, 2.0315) on X0 = U / (||U||_F + 1e-7).
 *     MUON_MOMENTUM: M <- mean_chunk(beta) M - U, W' = W - NS(M) (the two
 *     options combined by orthogonalising the momentum buffer; with beta = 0
 *     it is MUON).
 *   - Renormalisation (unless LACT_NO_RENORM): every row of each updated
 *     matrix (rows of the stored [rows x cols] arrays: an output unit's
 *     fan-in) is rescaled to the L2 norm it had before the update.
 *
 * Memory: every tensor argument is a caller-owned DEVICE pointer, contiguous,
 * innermost dimension fastest; host arrays (bounds, flags) are read during
 * the call only.  The library allocates no device memory, keeps no pointer
 * after returning, and frees nothing.  All device work is enqueued
 * asynchronously, without any host synchronisation, on `stream` (a
 * hipStream_t; NULL = the legacy default stream) and on two helper streams
 * the library creates once per device (default priority, kept until the
 * process ends): the second half of each Newton-Schulz batch and the
 * deferred applies run there, ordered after the caller's stream by events
 * and joined back to it before the call's work on `stream` ends.
 * Completion is therefore observed through `stream`, and a HIP graph
 * captured from `stream` contains the helper streams' work; while such a
 * capture is in progress no other thread may call the library on the same
 * device.
 *
 * Layouts (n = n_inst, D = d, Dh = dh):
 *   q, k, v, o : [n, L, D]   io_dtype (F32 or BF16)
 *   lr         : [n, L, 3]   float32 (post-softplus learning rates)
 *   beta       : [n, L]      float32 (post-sigmoid momentum coefficients)
 *   W1, W3     : [n, Dh, D]  float32, row j = fan-in vector of hidden unit j
 *   W2         : [n, D, Dh]  float32, row r = fan-in vector of output unit r
 *   M1, M2, M3 : same shapes as W1, W2, W3 (momentum state)
 *   ws         : workspace, >= lact_workspace_size(...) bytes, 256-B aligned
 *
 * Errors: every argument is validated before any device work; on a negative
 * status other than LACT_ERR_HIP nothing was enqueued and W, M, o are
 * untouched.  LACT_ERR_HIP means a HIP call failed while enqueuing; W, M and
 * o are then undefined.  lact_last_error() returns a thread-local text for
 * the last failure on the calling thread.  No C++ exception crosses the ABI.
 * Calls that share a workspace must not overlap on the device (order them
 * on one stream).
 */
#ifndef LACT_H
#define LACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LACT_OK = 0,
    LACT_ERR_INVALID_ARG = -1,        /* null/misaligned pointer, bad size, bad schedule */
    LACT_ERR_UNSUPPORTED = -2,        /* d or dh not a multiple of 64 in [64, 1024],
                                         a flag the entry point does not take,
                                         device is not gfx950 */
    LACT_ERR_WORKSPACE_TOO_SMALL = -3,
    LACT_ERR_NO_DEVICE = -4,          /* no HIP device visible */
    LACT_ERR_HIP = -5                 /* a HIP runtime call failed */
} lact_status;

typedef enum { LACT_DTYPE_F32 = 0, LACT_DTYPE_BF16 = 1 } lact_dtype;
typedef enum {
    LACT_OPT_GD = 0,
    LACT_OPT_MOMENTUM = 1,
    LACT_OPT_MUON = 2,
    LACT_OPT_MUON_MOMENTUM = 3   /* Newton-Schulz of the momentum buffer */
} lact_opt;
typedef enum { LACT_APPLY_THEN_UPDATE = 0, LACT_UPDATE_THEN_APPLY = 1 } lact_order;

/* per-chunk schedule flags */
#define LACT_CHUNK_UPDATE 1u
#define LACT_CHUNK_APPLY 2u

/* lact_problem.flags */
#define LACT_NO_RENORM 1u
/* q and k arrive raw: before use, every token's q and k vector x becomes
 * silu(x) / ||silu(x)||_2 over its D features ("LaCT架构核心思想解析" §1.2;
 * no epsilon, so a token whose silu is identically zero gives non-finite
 * values).  The caller's q and k are not modified; the pre-processed copies
 * live in the workspace. */
#define LACT_QK_PREP 2u

typedef struct {
    int32_t n_inst;     /* B * nh independent instances (>= 0) */
    int32_t d;          /* model width per head */
    int32_t dh;         /* fast-weight hidden width (a multiple of 64 in [64, 1024]) */
    int32_t io_dtype;   /* lact_dtype of q, k, v, o */
    int32_t opt;        /* lact_opt */
    int32_t ns_iters;   /* Newton-Schulz steps for MUON, 1..16 (5 = standard) */
    int32_t rec_planes; /* bf16 planes per fp32 operand in the state
                           recurrence (update products, Newton-Schulz):
                           1 = bf16, 2 = bf16x2, 3 = bf16x3 (fp32-grade);
                           0 = default: 3 for MUON and MUON_MOMENTUM (their
                           Newton-Schulz step amplifies rounding, about x2
                           per chunk with one plane), else 1.  F32 io always
                           uses 3 planes for every product. */
    uint32_t flags;     /* LACT_NO_RENORM | LACT_QK_PREP */
} lact_problem;

/*
 * Bytes of workspace needed by lact_layer_forward with the same schedule
 * arguments.  For lact_chunk_update / lact_apply over Lc tokens pass
 * L = chunk = Lc, order = 0, bounds = flags = NULL, n_chunks = 0.
 * Returns 0 (and sets lact_last_error) if the arguments are invalid.
 */
size_t lact_workspace_size(const lact_problem* p, int64_t L, int64_t chunk, int32_t order,
                           const int64_t* bounds, const uint8_t* flags, int32_t n_chunks);

/*
 * One chunk update ("大块测试时训练（LaCT）技术解析" §2.1, eqs. 4-5: the
 * gradient of the chunk's loss summed over its tokens; optimiser and row
 * renormalisation of §2.2.1, eqs. 8-10, and momentum of
 * "LaCT架构核心思想解析" §1.2): forward products on k and v, SwiGLU backward
 * epilogue, weight-gradient contractions over the chunk, optimiser, row
 * renormalisation, for Lc tokens per instance.  k, v are [n, seq_stride, D]
 * (the first Lc tokens of each instance are used), lr [n, seq_stride, 3],
 * beta [n, seq_stride] (MOMENTUM and MUON_MOMENTUM, else may be NULL).  W1..W3
 * are read and overwritten with the updated weights; M1..M3 likewise for
 * MOMENTUM and MUON_MOMENTUM
 * (else may be NULL).  Lc == 0 is a no-op.
 */
lact_status lact_chunk_update(const lact_problem* p, const void* k, const void* v,
                              const float* lr, const float* beta, int64_t Lc,
                              int64_t seq_stride, float* W1, float* W2, float* W3,
                              float* M1, float* M2, float* M3, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * Apply the fast weights to Lq queries per instance
 * ("大块测试时训练（LaCT）技术解析" §2.1, eq. 2; the SwiGLU memory of
 * "LaCT：以大分块更新人工智能的临时记忆", "局部注意力与非线性记忆相互补充"):
 * o = W2 (silu(W1 q) * (W3 q)).  q, o are [n, seq_stride, D] (first Lq
 * tokens used).  W1..W3 are read only.
 */
lact_status lact_apply(const lact_problem* p, const void* q, int64_t Lq, int64_t seq_stride,
                       const float* W1, const float* W2, const float* W3, void* o,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * The layer over a whole sequence of L tokens per instance: chunks of it
 * updated and applied in the order that keeps information visible only where
 * it may be ("LaCT：以大分块更新人工智能的临时记忆", "更新顺序必须遵守信息可见范围";
 * "LaCT架构核心思想解析" §2.2: apply-then-update for causal language), each
 * update and apply as in lact_chunk_update and lact_apply.
 * Schedule: if bounds == NULL and flags == NULL, chunks are uniform of
 * `chunk` tokens (the last takes the remainder) and every chunk is
 * UPDATE|APPLY.  Otherwise bounds[0..n_chunks] (host array, bounds[0] = 0,
 * strictly increasing, bounds[n_chunks] = L) and flags[0..n_chunks-1]
 * (host array of LACT_CHUNK_* bits) define it.
 * Order: LACT_APPLY_THEN_UPDATE -- an UPDATE|APPLY chunk is applied with the
 * weights before its own update (shifted block-causal);
 * LACT_UPDATE_THEN_APPLY -- it is applied after its own update.  An
 * APPLY-only chunk reads the current weights; an UPDATE-only chunk writes no
 * output.  Rows of o outside APPLY chunks are left untouched.  The final
 * state is written back to W1..W3 (and M1..M3 for MOMENTUM, MUON_MOMENTUM).
 */
lact_status lact_layer_forward(const lact_problem* p, const void* q, const void* k,
                               const void* v, const float* lr, const float* beta, int64_t L,
                               int64_t chunk, int32_t order, const int64_t* bounds,
                               const uint8_t* flags, int32_t n_chunks, float* W1, float* W2,
                               float* W3, float* M1, float* M2, float* M3, void* o, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * lact_layer_forward followed by the per-token output scale of
 * "LaCT架构核心思想解析" §2.1: every written row t of o is multiplied by
 * silu(oz[t]), where oz [n, L] float32 (device) holds the pre-activation of
 * that scale (the linear projection producing it is the caller's).  oz may
 * be NULL only when no chunk is APPLY; all other arguments, the workspace
 * size and the error behaviour are those of lact_layer_forward.  The scale
 * is applied inside the output product's epilogue (no extra pass over o).
 */
lact_status lact_layer_forward_scaled(const lact_problem* p, const void* q, const void* k,
                                      const void* v, const float* lr, const float* beta,
                                      const float* oz, int64_t L, int64_t chunk, int32_t order,
                                      const int64_t* bounds, const uint8_t* flags,
                                      int32_t n_chunks, float* W1, float* W2, float* W3,
                                      float* M1, float* M2, float* M3, void* o, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * Backward pass of lact_layer_forward (same problem, schedule and order
 * arguments): vector-Jacobian products of the layer through the whole chunk
 * recurrence.  The pages train the layer end to end but print no backward
 * formulas; what is differentiated is exactly the forward map above (update
 * and apply phases of "大块测试时训练（LaCT）技术解析" §2.1, eqs. 2 and 4-5;
 * renormalisation and Newton-Schulz of §2.2.1, eqs. 8-10; momentum of
 * "LaCT架构核心思想解析" §1.2), by the chain rule.  The gradients are those of
 *
 *     J = sum(dO * o) + sum_j sum(gW_j * W_j,final) + sum_j sum(gM_j * M_j,final)
 *
 * over o's APPLY rows, with respect to q, k, v, lr, beta and the initial
 * state W1..W3, M1..M3 (as passed to lact_layer_forward, i.e. BEFORE it
 * overwrote them).
 *
 * Inputs (device): q, k, v [n, L, D] io_dtype (raw q, k with LACT_QK_PREP);
 * lr [n, L, 3]; beta [n, L] (momentum optimisers, else may be NULL); oz
 * [n, L] fp32 or NULL: the output-scale pre-activation of
 * lact_layer_forward_scaled (NULL: the unscaled layer); W1..W3 initial
 * weights, M1..M3 initial momentum (momentum optimisers, else may be NULL);
 * dO [n, L, D] io_dtype, the cotangent of the (scaled) output (rows outside
 * APPLY chunks are not read); gW1..gW3, gM1..gM3 cotangents of the final
 * state, each may be NULL (= zero).  All read only.
 * Outputs (device, float32, fully written): dq, dk, dv [n, L, D] (of the raw
 * q, k with LACT_QK_PREP; zero on rows outside APPLY, resp. UPDATE chunks);
 * dlr [n, L, 3] (zero outside UPDATE chunks); dbeta [n, L] (momentum
 * optimisers; may be NULL otherwise); doz [n, L] (with oz; zero outside
 * APPLY chunks); dW1..dW3 (shapes of W1..W3); dM1..dM3 (shapes of M1..M3;
 * may be NULL -- for GD and MUON they equal gM).  The call recomputes the
 * forward state trajectory itself (rec_planes is ignored; raw q, k are
 * pre-processed in fp32, not rounded to the io dtype).  Its products take
 * fp32 operands as bf16 planes with fp32 accumulation: three planes (fp32
 * grade) for MUON and MUON_MOMENTUM, whose Newton-Schulz backward amplifies
 * rounding, and for fp32 inputs; two (16-bit significands) for GD and
 * MOMENTUM.  Workspace:
 * lact_backward_workspace_size bytes, 256-B aligned.  Errors as for
 * lact_layer_forward; outputs are undefined after LACT_ERR_HIP.
 */
size_t lact_backward_workspace_size(const lact_problem* p, int64_t L, int64_t chunk, int32_t order,
                                    const int64_t* bounds, const uint8_t* flags, int32_t n_chunks);

lact_status lact_layer_backward(const lact_problem* p, const void* q, const void* k,
                                const void* v, const float* lr, const float* beta,
                                const float* oz, int64_t L, int64_t chunk, int32_t order,
                                const int64_t* bounds,
                                const uint8_t* flags, int32_t n_chunks, const float* W1,
                                const float* W2, const float* W3, const float* M1,
                                const float* M2, const float* M3, const void* dO,
                                const float* gW1, const float* gW2, const float* gW3,
                                const float* gM1, const float* gM2, const float* gM3, float* dq,
                                float* dk, float* dv, float* dlr, float* dbeta, float* doz,
                                float* dW1, float* dW2, float* dW3, float* dM1, float* dM2,
                                float* dM3, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free variant of lact_layer_forward, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid it.  Same arguments and semantics as
 * lact_layer_forward without the workspace: the library's own device scratch
 * array takes its place.  That array has LACT_NOALLOC_SCRATCH_BYTES bytes,
 * one copy per device (created when the library's code is loaded on the
 * device, held until the process ends); a problem whose
 * lact_workspace_size exceeds it is rejected with
 * LACT_ERR_WORKSPACE_TOO_SMALL before any device work.  The call allocates
 * and frees nothing.  Every call on a device shares that device's array:
 * calls that overlap on one device (several streams or host threads at
 * once) race and must be ordered by the caller, e.g. on one stream.  No
 * result depends on the array's previous contents.
 */
#define LACT_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
lact_status lact_layer_forward_noalloc(const lact_problem* p, const void* q, const void* k,
                                       const void* v, const float* lr, const float* beta, int64_t L,
                                       int64_t chunk, int32_t order, const int64_t* bounds,
                                       const uint8_t* flags, int32_t n_chunks, float* W1, float* W2,
                                       float* W3, float* M1, float* M2, float* M3, void* o,
                                       void* stream);

/* Static text for a status code. */
const char* lact_status_str(lact_status s);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* lact_last_error(void);

/*
 * Per-kernel timing (diagnostics; process-wide, not for concurrent use).
 * While enabled, every launch of a library kernel of class `kclass` (see
 * LACT_K_*) is bracketed by HIP events recorded on the launch stream.
 * lact_timing_read synchronises those events and returns the summed
 * milliseconds and the number of launches since the previous read.
 */
#define LACT_K_UPD 0       /* update forward: k W1^T, k W3^T, v W2 + SwiGLU backward terms
                              (bf16 inputs at d = dh = 128, chunks of >= 4,096 tokens, or of
                              >= 1,024 with weight planes: together with the weight-gradient
                              contraction, one kernel; plain bf16 apply-then-update chunks:
                              also the chunk's q W1^T, q W3^T -> gated hidden) */
#define LACT_K_APP 1       /* apply forward: q W1^T, q W3^T -> gated hidden, for applies not
                              computed in their update's kernel (bf16 q with dh = 128: the
                              whole apply, o = Hq W2^T included, in one kernel) */
#define LACT_K_OUT 2       /* apply output product o = Hq W2^T (when not fused) */
#define LACT_K_DW 3        /* weight-gradient contractions (split over tokens; when not fused) */
#define LACT_K_OPT 4       /* optimiser step + row renormalisation + weight snapshot */
#define LACT_K_NS 5        /* Newton-Schulz products */
#define LACT_K_SNAP 6      /* snapshot of the caller's weights at call start */
#define LACT_K_PREP 7      /* q / k pre-processing (LACT_QK_PREP) */
#define LACT_K_BWD_GEMM 8  /* backward: products of the reverse sweep */
#define LACT_K_BWD_ELEM 9  /* backward: elementwise, row and reduction kernels */
#define LACT_K_NSRED 10    /* Newton-Schulz input: the sum of the split partials with its row
                              sums of squares (and, with momentum, the new momentum) */
#define LACT_K_COUNT 11
lact_status lact_timing_enable(int32_t kclass, int32_t on);
lact_status lact_timing_read(int32_t kclass, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* LACT_H */
