/*
 * A plain C program that runs the device calls of include/sgemv.h on the
 * GPU with the HIP runtime API only (no Python, no PyTorch): it reads q, s,
 * z, one activation row and its threshold from the directory named on the
 * command line, packs the matrix, uploads it, and runs
 *   1. sgemv_run_fused with the list written,
 *   2. sgemv_gather_indices, then sgemv_run over that list,
 *   3. sgemv_run with no list (the dense int4 GEMV),
 * each with fp32 output on the null stream, then writes y1.bin, y2.bin,
 * y3.bin, list.bin and count.bin back into the directory.  The test compares
 * them with the fp64 oracle.  Prints "ok" and returns 0 when every HIP call
 * and library call succeeded.
 *
 * usage: c_abi_device dir N K
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "sgemv.h"

#define HIP_OK(c)                                                              \
    do {                                                                       \
        hipError_t e_ = (c);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s failed: %d (line %d)\n", #c, (int)e_, __LINE__); \
            return 1;                                                          \
        }                                                                      \
    } while (0)
#define LIB_OK(c)                                                              \
    do {                                                                       \
        int s_ = (c);                                                          \
        if (s_ != SGEMV_OK) {                                                  \
            fprintf(stderr, "%s: %s (line %d)\n", #c, sgemv_strerror(s_), __LINE__); \
            return 1;                                                          \
        }                                                                      \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(n);
    const size_t r = p ? fread(p, 1, n, f) : 0;
    fclose(f);
    if (r != n) {
        free(p);
        return NULL;
    }
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const size_t w = fwrite(p, 1, n, f);
    fclose(f);
    return w == n ? 0 : 1;
}

int main(int argc, char** argv) {
    if (argc != 4) {
        fprintf(stderr, "usage: %s dir N K\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    const int32_t N = atoi(argv[2]), K = atoi(argv[3]), G = K / SGEMV_GROUP;
    uint8_t* q = read_file(dir, "q.bin", (size_t)N * K);
    uint16_t* s = read_file(dir, "s.bin", (size_t)N * G * 2);
    uint16_t* z = read_file(dir, "z.bin", (size_t)N * G * 2);
    uint16_t* x = read_file(dir, "x.bin", (size_t)K * 2);
    float* t = read_file(dir, "t.bin", sizeof(float));
    if (!q || !s || !z || !x || !t) {
        fprintf(stderr, "missing input files\n");
        return 1;
    }

    sgemv_desc d;
    LIB_OK(sgemv_pack_layout(NULL, NULL, NULL, N, K, SGEMV_GROUP, SGEMV_TILE_N, NULL, 0, &d));
    uint8_t* blob = malloc(d.total_bytes);
    LIB_OK(sgemv_pack_layout(q, s, z, N, K, SGEMV_GROUP, SGEMV_TILE_N, blob, d.total_bytes, &d));
    const size_t ws_bytes = sgemv_workspace_bytes(&d, 1);

    void *d_blob, *d_x, *d_ws, *d_y;
    int32_t *d_idx, *d_cnt;
    HIP_OK(hipMalloc(&d_blob, d.total_bytes));
    HIP_OK(hipMalloc(&d_x, (size_t)K * 2));
    HIP_OK(hipMalloc(&d_ws, ws_bytes ? ws_bytes : 256));
    HIP_OK(hipMalloc(&d_y, (size_t)N * 4));
    HIP_OK(hipMalloc((void**)&d_idx, (size_t)K * 4));
    HIP_OK(hipMalloc((void**)&d_cnt, 4));
    HIP_OK(hipMemcpy(d_blob, blob, d.total_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, (size_t)K * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_ws, 0, ws_bytes ? ws_bytes : 256));   /* once, at allocation */

    float* y = malloc((size_t)N * 4);
    int32_t* idx = malloc((size_t)K * 4);
    int32_t cnt = -1;

    /* 1. one fused launch, the list written */
    LIB_OK(sgemv_run_fused(&d, d_blob, d_x, 1, K, t, d_idx, d_cnt, d_y, N, SGEMV_OUT_F32, d_ws, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(y, d_y, (size_t)N * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&cnt, d_cnt, 4, hipMemcpyDeviceToHost));
    if (cnt < 0 || cnt > K) return 1;
    HIP_OK(hipMemcpy(idx, d_idx, (size_t)cnt * 4, hipMemcpyDeviceToHost));
    if (write_file(dir, "y1.bin", y, (size_t)N * 4) || write_file(dir, "count.bin", &cnt, 4) ||
        write_file(dir, "list.bin", idx, (size_t)cnt * 4))
        return 1;

    /* 2. the gather, then the GEMV over its list */
    LIB_OK(sgemv_gather_indices(d_x, 1, K, K, t, d_idx, d_cnt, NULL));
    LIB_OK(sgemv_run(&d, d_blob, d_x, d_idx, d_cnt, d_y, SGEMV_OUT_F32, d_ws, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(y, d_y, (size_t)N * 4, hipMemcpyDeviceToHost));
    if (write_file(dir, "y2.bin", y, (size_t)N * 4)) return 1;

    /* 3. every column */
    LIB_OK(sgemv_run(&d, d_blob, d_x, NULL, NULL, d_y, SGEMV_OUT_F32, d_ws, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(y, d_y, (size_t)N * 4, hipMemcpyDeviceToHost));
    if (write_file(dir, "y3.bin", y, (size_t)N * 4)) return 1;

    HIP_OK(hipFree(d_blob));
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_ws));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_idx));
    HIP_OK(hipFree(d_cnt));
    free(blob);
    free(y);
    free(idx);
    free(q);
    free(s);
    free(z);
    free(x);
    free(t);
    printf("ok\n");
    return 0;
}
