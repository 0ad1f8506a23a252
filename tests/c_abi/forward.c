/*
 * A plain C caller of the layer's C ABI (include/moe.h): no Python between
 * the caller and the library. It reads one layer's inputs from a file,
 * copies them to the device, sizes the workspace with moe_workspace_bytes,
 * runs moe_forward on a stream of its own, and writes y, the top-k ids and
 * weights back to a file. It also shows the error path: a call with k > E
 * must return MOE_ERR_INVALID_ARG and enqueue nothing.
 *
 * Input file (little-endian): int32 T, H, F, E, k, dt (0 fp32, 1 bf16),
 * has_bias; float drop; then x[T*H], Wr[H*E] in dt, bias[E] fp32 when
 * has_bias, W1[E*H*F], W2[E*F*H] in dt.
 * Output file: float y[T*H], int32 ids[T*k], float w[T*k].
 *
 * usage: forward <in> <out>; exit status 0 on success.
 */
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static void* read_bytes(FILE* f, size_t n) {
    void* p = malloc(n ? n : 1);
    if (p != NULL && n > 0 && fread(p, 1, n, f) != n) {
        free(p);
        return NULL;
    }
    return p;
}

static void* to_device(const void* host, size_t n) {
    void* d = NULL;
    if (hipMalloc(&d, n ? n : 1) != hipSuccess) return NULL;
    if (n > 0 && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return d;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <in> <out>\n", argv[0]);
        return 2;
    }
    FILE* f = fopen(argv[1], "rb");
    if (f == NULL) return 2;
    int32_t hdr[7];
    float drop = 0.0f;
    if (fread(hdr, sizeof(int32_t), 7, f) != 7 || fread(&drop, sizeof(float), 1, f) != 1) return 2;
    const int T = hdr[0], H = hdr[1], F = hdr[2], E = hdr[3], k = hdr[4], has_bias = hdr[6];
    const moe_dtype_t dt = hdr[5] == 1 ? MOE_BF16 : MOE_F32;
    const size_t es = dt == MOE_BF16 ? 2 : 4;
    void* x = read_bytes(f, (size_t)T * H * es);
    void* Wr = read_bytes(f, (size_t)H * E * es);
    void* bias = has_bias ? read_bytes(f, (size_t)E * sizeof(float)) : NULL;
    void* W1 = read_bytes(f, (size_t)E * H * F * es);
    void* W2 = read_bytes(f, (size_t)E * F * H * es);
    fclose(f);
    if (x == NULL || Wr == NULL || (has_bias && bias == NULL) || W1 == NULL || W2 == NULL) return 2;

    void* dx = to_device(x, (size_t)T * H * es);
    void* dWr = to_device(Wr, (size_t)H * E * es);
    void* dbias = has_bias ? to_device(bias, (size_t)E * sizeof(float)) : NULL;
    void* dW1 = to_device(W1, (size_t)E * H * F * es);
    void* dW2 = to_device(W2, (size_t)E * F * H * es);
    if (dx == NULL || dWr == NULL || (has_bias && dbias == NULL) || dW1 == NULL || dW2 == NULL) return 1;

    float* dy = NULL;
    int32_t* dids = NULL;
    float* dw = NULL;
    HIP_OK(hipMalloc((void**)&dy, (size_t)T * H * sizeof(float)));
    HIP_OK(hipMalloc((void**)&dids, (size_t)T * k * sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&dw, (size_t)T * k * sizeof(float)));
    const size_t ws_bytes = moe_workspace_bytes(T, H, F, E, k, 0, dt);
    if (ws_bytes == 0) {
        fprintf(stderr, "moe_workspace_bytes: sizes not supported\n");
        return 1;
    }
    void* ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* the error path: nothing is enqueued and a negative status comes back */
    int st = moe_forward(dx, dWr, dbias, dW1, dW2, NULL, NULL, 0, T, H, F, E, E + 1, drop, dt, dy, MOE_F32, dids,
                         dw, NULL, NULL, ws, ws_bytes, stream);
    if (st != MOE_ERR_INVALID_ARG) {
        fprintf(stderr, "k > E: expected MOE_ERR_INVALID_ARG, got %d (%s)\n", st, moe_strerror(st));
        return 1;
    }
    printf("k > E rejected: %s\n", moe_strerror(st));

    st = moe_forward(dx, dWr, dbias, dW1, dW2, NULL, NULL, 0, T, H, F, E, k, drop, dt, dy, MOE_F32, dids, dw, NULL,
                     NULL, ws, ws_bytes, stream);
    if (st != MOE_OK) {
        fprintf(stderr, "moe_forward: %s\n", moe_strerror(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));

    float* y = (float*)malloc((size_t)T * H * sizeof(float));
    int32_t* ids = (int32_t*)malloc((size_t)T * k * sizeof(int32_t));
    float* w = (float*)malloc((size_t)T * k * sizeof(float));
    if (y == NULL || ids == NULL || w == NULL) return 1;
    HIP_OK(hipMemcpy(y, dy, (size_t)T * H * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ids, dids, (size_t)T * k * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(w, dw, (size_t)T * k * sizeof(float), hipMemcpyDeviceToHost));
    FILE* o = fopen(argv[2], "wb");
    if (o == NULL) return 1;
    fwrite(y, sizeof(float), (size_t)T * H, o);
    fwrite(ids, sizeof(int32_t), (size_t)T * k, o);
    fwrite(w, sizeof(float), (size_t)T * k, o);
    fclose(o);
    printf("moe_forward (%s, library %s): T=%d H=%d F=%d E=%d k=%d ok\n", dt == MOE_BF16 ? "bf16" : "fp32",
           moe_version(), T, H, F, E, k);

    hipStreamDestroy(stream);
    hipFree(ws);
    hipFree(dw);
    hipFree(dids);
    hipFree(dy);
    hipFree(dW2);
    hipFree(dW1);
    hipFree(dbias);
    hipFree(dWr);
    hipFree(dx);
    free(w);
    free(ids);
    free(y);
    free(W2);
    free(W1);
    free(bias);
    free(Wr);
    free(x);
    return 0;
}
