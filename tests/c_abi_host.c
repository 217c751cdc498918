/*
 * A plain C program against include/sgemv.h and libsgemv.so: the host-side
 * calls (packing, the header round trip, workspace sizes, argument checks)
 * from C with no Python and no GPU.  Packs a small random matrix in both
 * layout versions, writes q, s, z and both blobs into the directory named on
 * the command line (the test compares the blobs with the oracle's layout
 * specification), and checks that the device calls reject bad arguments
 * before any HIP call.  Prints "ok" and returns 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sgemv.h"

#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                              \
        }                                                          \
    } while (0)

static uint32_t lcg(uint32_t* s) { return *s = *s * 1664525u + 1013904223u; }

static int write_file(const char* path, const void* p, size_t n) {
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const size_t w = fwrite(p, 1, n, f);
    fclose(f);
    return w == n ? 0 : 1;
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s out_dir\n", argv[0]);
        return 2;
    }
    char path[4096];
    const int32_t N = 1024, K = 384, G = K / SGEMV_GROUP;
    uint8_t* q = malloc((size_t)N * K);
    uint16_t* s = malloc((size_t)N * G * 2);
    uint16_t* z = malloc((size_t)N * G * 2);
    uint32_t seed = 12345u;
    for (size_t i = 0; i < (size_t)N * K; ++i) q[i] = (uint8_t)(lcg(&seed) >> 28);
    for (size_t i = 0; i < (size_t)N * G; ++i) {
        s[i] = (uint16_t)(0x2000u + (lcg(&seed) >> 22));   /* positive normal fp16 */
        z[i] = (lcg(&seed) >> 31) ? (uint16_t)0x3C00u : (uint16_t)0u;   /* 1.0 or 0.0 */
    }
    snprintf(path, sizeof path, "%s/q.bin", argv[1]);
    CHECK(write_file(path, q, (size_t)N * K) == 0);
    snprintf(path, sizeof path, "%s/s.bin", argv[1]);
    CHECK(write_file(path, s, (size_t)N * G * 2) == 0);
    snprintf(path, sizeof path, "%s/z.bin", argv[1]);
    CHECK(write_file(path, z, (size_t)N * G * 2) == 0);

    /* size query, pack, header round trip: version 1 and version 2 */
    for (int v = 1; v <= 2; ++v) {
        int (*pack)(const uint8_t*, const uint16_t*, const uint16_t*, int32_t, int32_t, int32_t, int32_t, void*,
                    size_t, sgemv_desc*) = v == 1 ? sgemv_pack_layout : sgemv_pack_layout_z4;
        sgemv_desc d;
        memset(&d, 0, sizeof d);
        CHECK(pack(NULL, NULL, NULL, N, K, SGEMV_GROUP, SGEMV_TILE_N, NULL, 0, &d) == SGEMV_OK);
        CHECK(d.N == N && d.K == K && d.version == (uint32_t)v && d.w_bytes == (uint64_t)N * K / 2);
        uint8_t* blob = malloc(d.total_bytes);
        CHECK(pack(q, s, z, N, K, SGEMV_GROUP, SGEMV_TILE_N, blob, d.total_bytes - 1, &d) == SGEMV_ESIZE);
        CHECK(pack(q, s, z, N, K, SGEMV_GROUP, SGEMV_TILE_N, blob, d.total_bytes, &d) == SGEMV_OK);
        sgemv_desc h;
        CHECK(sgemv_desc_from_header(blob, 64, &h) == SGEMV_OK);
        CHECK(memcmp(&h, &d, sizeof d) == 0);
        snprintf(path, sizeof path, "%s/blob%d.bin", argv[1], v);
        CHECK(write_file(path, blob, d.total_bytes) == 0);
        CHECK(sgemv_workspace_bytes(&d, 1) > 0 && sgemv_workspace_bytes(&d, 16) >= sgemv_workspace_bytes(&d, 1));
        CHECK(sgemv_workspace_bytes(&d, 0) == 0 && sgemv_workspace_bytes(&d, 17) == 0);

        /* bad arguments are refused before any HIP call (no GPU needed) */
        void* fake = (void*)(uintptr_t)(1u << 20);   /* aligned, never dereferenced */
        CHECK(sgemv_run(NULL, fake, fake, NULL, NULL, fake, 0, fake, NULL) == SGEMV_EINVAL);
        CHECK(sgemv_run(&d, fake, fake, NULL, NULL, fake, 2u, fake, NULL) == SGEMV_EINVAL);
        CHECK(sgemv_run_batched(&d, fake, fake, 17, K, NULL, NULL, NULL, fake, N, 0, fake, NULL) == SGEMV_ESIZE);
        CHECK(sgemv_run_batched(&d, fake, fake, 2, K + 1, NULL, NULL, NULL, fake, N, 0, fake, NULL) == SGEMV_EALIGN);
        const float bad_t = -1.0f;
        CHECK(sgemv_run_fused(&d, fake, fake, 1, K, &bad_t, NULL, NULL, fake, N, 0, fake, NULL) == SGEMV_EINVAL);
        CHECK(sgemv_gather_indices(fake, 1, K, K, NULL, fake, fake, NULL) == SGEMV_EINVAL);
        free(blob);
    }
    CHECK(strcmp(sgemv_strerror(SGEMV_OK), sgemv_strerror(SGEMV_EINVAL)) != 0);
    CHECK(sgemv_last_hip_error() == 0);

    /* a code above 15 is refused */
    q[7] = 16;
    sgemv_desc d;
    CHECK(sgemv_pack_layout(q, s, z, N, K, SGEMV_GROUP, SGEMV_TILE_N, NULL, 0, &d) == SGEMV_OK);
    uint8_t* blob = malloc(d.total_bytes);
    CHECK(sgemv_pack_layout(q, s, z, N, K, SGEMV_GROUP, SGEMV_TILE_N, blob, d.total_bytes, &d) == SGEMV_EINVAL);
    free(blob);
    free(q);
    free(s);
    free(z);
    printf("ok\n");
    return 0;
}
