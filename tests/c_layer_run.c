/* The LaCT layer through the C ABI alone: no Python, no torch.  Reads one
 * problem's inputs from raw little-endian files, allocates device memory
 * with hipMalloc, runs lact_layer_forward and then lact_layer_backward (from
 * the initial state, for a given output cotangent) on a stream of its own,
 * and writes the results back to files.  Used by tests/test_gpu_c_abi.py.
 *
 *   c_layer_run <dir> <n> <d> <dh> <L> <chunk> <io_dtype> <opt> <rec_planes>
 *
 * <dir> holds q.bin k.bin v.bin dO.bin ([n, L, d], io dtype), lr.bin
 * ([n, L, 3] f32), beta.bin ([n, L] f32, momentum optimisers), W1.bin W2.bin
 * W3.bin (f32); the program writes o.bin, W1o.bin W2o.bin W3o.bin (M1o..M3o
 * for momentum) and the gradients dq.bin dk.bin dv.bin dlr.bin dW1.bin
 * dW2.bin dW3.bin (dbeta.bin for momentum).  Uniform chunks, all
 * UPDATE|APPLY, apply-then-update.  Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lact.h"

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            exit(2);                                                                \
        }                                                                           \
    } while (0)
#define LACT_OK_(x)                                                                 \
    do {                                                                            \
        lact_status s_ = (x);                                                       \
        if (s_ != LACT_OK) {                                                        \
            fprintf(stderr, "%s: %s (%s)\n", #x, lact_status_str(s_), lact_last_error()); \
            exit(3);                                                                \
        }                                                                           \
    } while (0)

static const char* g_dir;

static void* load(const char* name, size_t bytes) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/%s", g_dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(4);
    }
    void* host = malloc(bytes);
    if (fread(host, 1, bytes, f) != bytes) {
        fprintf(stderr, "short read %s\n", path);
        exit(4);
    }
    fclose(f);
    void* dev = NULL;
    HIP_OK(hipMalloc(&dev, bytes ? bytes : 1));
    HIP_OK(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
    free(host);
    return dev;
}

static void* zeros(size_t bytes) {
    void* dev = NULL;
    HIP_OK(hipMalloc(&dev, bytes ? bytes : 1));
    HIP_OK(hipMemset(dev, 0, bytes));
    return dev;
}

static void save(const char* name, const void* dev, size_t bytes) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/%s", g_dir, name);
    void* host = malloc(bytes);
    HIP_OK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(host, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(4);
    }
    fclose(f);
    free(host);
}

int main(int argc, char** argv) {
    if (argc != 10) {
        fprintf(stderr, "usage: %s <dir> <n> <d> <dh> <L> <chunk> <io_dtype> <opt> <rec_planes>\n", argv[0]);
        return 1;
    }
    g_dir = argv[1];
    lact_problem p;
    memset(&p, 0, sizeof(p));
    p.n_inst = atoi(argv[2]);
    p.d = atoi(argv[3]);
    p.dh = atoi(argv[4]);
    const int64_t L = atoll(argv[5]), chunk = atoll(argv[6]);
    p.io_dtype = atoi(argv[7]);
    p.opt = atoi(argv[8]);
    p.rec_planes = atoi(argv[9]);
    p.ns_iters = 5;
    const int mom = p.opt == LACT_OPT_MOMENTUM || p.opt == LACT_OPT_MUON_MOMENTUM;
    const size_t n = (size_t)p.n_inst, es = p.io_dtype == LACT_DTYPE_BF16 ? 2 : 4;
    const size_t xb = n * (size_t)L * (size_t)p.d, wb = n * (size_t)p.d * (size_t)p.dh * 4;

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    void* q = load("q.bin", xb * es);
    void* k = load("k.bin", xb * es);
    void* v = load("v.bin", xb * es);
    void* dO = load("dO.bin", xb * es);
    float* lr = (float*)load("lr.bin", n * L * 3 * 4);
    float* beta = mom ? (float*)load("beta.bin", n * L * 4) : NULL;
    float* W0[3] = {(float*)load("W1.bin", wb), (float*)load("W2.bin", wb), (float*)load("W3.bin", wb)};
    float* W[3];
    float* M[3] = {NULL, NULL, NULL};
    float* M0[3] = {NULL, NULL, NULL};
    for (int j = 0; j < 3; ++j) {
        W[j] = (float*)zeros(wb);
        HIP_OK(hipMemcpy(W[j], W0[j], wb, hipMemcpyDeviceToDevice));
        if (mom) {
            M[j] = (float*)zeros(wb);
            M0[j] = (float*)zeros(wb);
        }
    }
    void* o = zeros(xb * es);

    /* forward: W, M updated in place, o written */
    size_t ws_bytes = lact_workspace_size(&p, L, chunk, LACT_APPLY_THEN_UPDATE, NULL, NULL, 0);
    const size_t bws = lact_backward_workspace_size(&p, L, chunk, LACT_APPLY_THEN_UPDATE, NULL, NULL, 0);
    if (ws_bytes == 0 || bws == 0) {
        fprintf(stderr, "workspace query failed: %s\n", lact_last_error());
        return 3;
    }
    if (bws > ws_bytes) ws_bytes = bws;
    void* ws = zeros(ws_bytes);
    LACT_OK_(lact_layer_forward(&p, q, k, v, lr, beta, L, chunk, LACT_APPLY_THEN_UPDATE, NULL, NULL, 0, W[0], W[1],
                                W[2], M[0], M[1], M[2], o, ws, ws_bytes, s));

    /* backward from the initial state */
    float* dq = (float*)zeros(xb * 4);
    float* dk = (float*)zeros(xb * 4);
    float* dv = (float*)zeros(xb * 4);
    float* dlr = (float*)zeros(n * L * 3 * 4);
    float* dbeta = mom ? (float*)zeros(n * L * 4) : NULL;
    float* dW[3] = {(float*)zeros(wb), (float*)zeros(wb), (float*)zeros(wb)};
    LACT_OK_(lact_layer_backward(&p, q, k, v, lr, beta, NULL, L, chunk, LACT_APPLY_THEN_UPDATE, NULL, NULL, 0, W0[0],
                                 W0[1], W0[2], M0[0], M0[1], M0[2], dO, NULL, NULL, NULL, NULL, NULL, NULL, dq, dk, dv,
                                 dlr, dbeta, NULL, dW[0], dW[1], dW[2], NULL, NULL, NULL, ws, ws_bytes, s));
    HIP_OK(hipStreamSynchronize(s));

    save("o.bin", o, xb * es);
    save("W1o.bin", W[0], wb);
    save("W2o.bin", W[1], wb);
    save("W3o.bin", W[2], wb);
    if (mom) {
        save("M1o.bin", M[0], wb);
        save("M2o.bin", M[1], wb);
        save("M3o.bin", M[2], wb);
        save("dbeta.bin", dbeta, n * L * 4);
    }
    save("dq.bin", dq, xb * 4);
    save("dk.bin", dk, xb * 4);
    save("dv.bin", dv, xb * 4);
    save("dlr.bin", dlr, n * L * 3 * 4);
    save("dW1.bin", dW[0], wb);
    save("dW2.bin", dW[1], wb);
    save("dW3.bin", dW[2], wb);
    HIP_OK(hipStreamDestroy(s));
    printf("c_layer_run: ok\n");
    return 0;
}
