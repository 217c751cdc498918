// Host packer for the sparsity-aware int4 layout (no HIP calls).
//
// The layout answers the page's call ("Enabling Dynamic Sparsity in
// Quantized LLM Inference", Abstract) for a quantized-weight arrangement
// that agrees with activation sparsity and keeps GPU reads local.  For each
// tile of tile_n outputs, the tile_n codes of one input column k sit in one
// contiguous run of tile_n/2 bytes (even row in the low nibble), so a GEMV
// that skips inactive inputs reads whole 256-byte runs and nothing else.
// Scales and zero-points of one (tile, group) pair are one contiguous run:
// tile_n (s, z) fp16 pairs (version 1), or tile_n fp16 scales followed by
// the integer zero-points as 4-bit codes, two per byte (version 2, 37.5 %
// fewer metadata bytes for the same numbers).  Version 3 packs the other
// quantization, with groups along the outputs (one (s, z) per input column
// and 128 outputs): per 256 outputs and column, 8 contiguous bytes, so a
// column's metadata is read only with the column.  The byte formulas are
// documented in sgemv.h.
#include "sgemv.h"

#include <cstring>

namespace {

constexpr uint64_t kHeader = 256;

uint64_t roundup(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool fp16_is_finite(uint16_t b) { return (b & 0x7C00u) != 0x7C00u; }

// Value of an fp16 bit pattern when it is an integer in 0..15, else -1.
int fp16_small_int(uint16_t b) {
    if (b == 0x0000u || b == 0x8000u) return 0;
    if (b & 0x8000u) return -1;
    const int e = (b >> 10) & 0x1F;  // biased exponent
    const int m = b & 0x3FF;
    if (e < 15 || e > 18) return -1;  // value outside [1, 16)
    const int shift = 10 - (e - 15);  // mantissa bits below the binary point
    if (m & ((1 << shift) - 1)) return -1;
    return (1 << (e - 15)) | (m >> shift);
}

}  // namespace

extern "C" int sgemv_layout_fill_desc(int32_t N, int32_t K, int32_t tile_n, uint32_t version,
                                      sgemv_desc* d) {
    d->N = N;
    d->K = K;
    d->group = SGEMV_GROUP;
    d->tile_n = tile_n;
    d->w_off = kHeader;
    d->w_bytes = (uint64_t)N * (uint64_t)K / 2;
    d->m_off = d->w_off + roundup(d->w_bytes, 256);
    d->m_bytes = version == SGEMV_LAYOUT_Z4 ? (uint64_t)(K / SGEMV_GROUP) * (uint64_t)N * 5 / 2
                                            : (uint64_t)(K / SGEMV_GROUP) * (uint64_t)N * 4;
    d->total_bytes = d->m_off + roundup(d->m_bytes, 256);
    d->version = version;
    d->reserved = 0;
    return SGEMV_OK;
}

static int check_shape(int32_t N, int32_t K, int32_t group, int32_t tile_n) {
    if (group != SGEMV_GROUP) return SGEMV_EINVAL;
    if (N <= 0 || K <= 0 || K % SGEMV_GROUP || K > SGEMV_MAX_K || N > SGEMV_MAX_N)
        return SGEMV_ESIZE;
    if (tile_n < 64 || tile_n > 1024 || (tile_n & (tile_n - 1)) || N % tile_n)
        return SGEMV_ESIZE;
    return SGEMV_OK;
}

// The rows of the matrix being packed: one or more parts stacked along N
// (part p holds rows n_part[p] of its own [rows][K] codes and [rows][K/128]
// scales and zero-points, or [rows/128][K] with groups along the outputs).
struct Rows {
    int32_t parts;
    const uint8_t* const* q;
    const uint16_t* const* s;
    const uint16_t* const* z;
    const int32_t* n_part;

    // part and row within it of matrix row n
    void locate(uint64_t n, int32_t& p, uint64_t& r) const {
        p = 0;
        r = n;
        while (p + 1 < parts && r >= (uint64_t)n_part[p]) r -= (uint64_t)n_part[p++];
    }
    const uint8_t* qrow(uint64_t n, int32_t K) const {
        int32_t p; uint64_t r;
        locate(n, p, r);
        return q[p] + r * (uint64_t)K;
    }
    uint16_t scale(uint64_t n, int32_t Gk, int32_t g) const {
        int32_t p; uint64_t r;
        locate(n, p, r);
        return s[p][r * Gk + g];
    }
    uint16_t zero(uint64_t n, int32_t Gk, int32_t g) const {
        int32_t p; uint64_t r;
        locate(n, p, r);
        return z[p][r * Gk + g];
    }
    // groups along the outputs: the (s, z) of column k for the 128 outputs
    // that hold row n (parts are whole tiles of at least 256 rows)
    uint16_t scale_ng(uint64_t n, int32_t K, int32_t k) const {
        int32_t p; uint64_t r;
        locate(n, p, r);
        return s[p][(r / SGEMV_GROUP) * (uint64_t)K + k];
    }
    uint16_t zero_ng(uint64_t n, int32_t K, int32_t k) const {
        int32_t p; uint64_t r;
        locate(n, p, r);
        return z[p][(r / SGEMV_GROUP) * (uint64_t)K + k];
    }
};

static int pack(const Rows& src, int32_t N, int32_t K, int32_t group, int32_t tile_n, uint32_t version, void* out,
                size_t out_capacity, sgemv_desc* desc_out) {
    int st = check_shape(N, K, group, tile_n);
    if (st) return st;
    const bool ng = version == SGEMV_LAYOUT_NG;
    if (ng && tile_n < 2 * SGEMV_GROUP) return SGEMV_ESIZE;
    sgemv_desc d;
    sgemv_layout_fill_desc(N, K, tile_n, version, &d);
    if (!out) {  // size query
        if (desc_out) *desc_out = d;
        return SGEMV_OK;
    }
    for (int32_t p = 0; p < src.parts; ++p)
        if (!src.q[p] || !src.s[p] || !src.z[p]) return SGEMV_EINVAL;
    if (out_capacity < d.total_bytes) return SGEMV_ESIZE;

    const int32_t Gk = K / SGEMV_GROUP;
    // Validate every input before writing anything.
    for (uint64_t n = 0; n < (uint64_t)N; ++n) {
        const uint8_t* qr = src.qrow(n, K);
        for (int32_t k = 0; k < K; ++k)
            if (qr[k] > 15) return SGEMV_EINVAL;
        if (ng) {
            if (n % SGEMV_GROUP == 0)
                for (int32_t k = 0; k < K; ++k) {
                    if (!fp16_is_finite(src.scale_ng(n, K, k))) return SGEMV_EINVAL;
                    if (fp16_small_int(src.zero_ng(n, K, k)) < 0) return SGEMV_EINVAL;
                }
            continue;
        }
        for (int32_t g = 0; g < Gk; ++g) {
            if (!fp16_is_finite(src.scale(n, Gk, g))) return SGEMV_EINVAL;
            if (fp16_small_int(src.zero(n, Gk, g)) < 0) return SGEMV_EINVAL;
        }
    }

    uint8_t* blob = static_cast<uint8_t*>(out);
    std::memset(blob, 0, d.total_bytes);
    // header (little-endian host assumed: x86-64 and the GPU are both LE)
    std::memcpy(blob + 0, "SGV1", 4);
    std::memcpy(blob + 4, &version, 4);
    const int32_t hv[4] = {N, K, SGEMV_GROUP, tile_n};
    std::memcpy(blob + 8, hv, 16);
    const uint64_t ho[5] = {d.w_off, d.w_bytes, d.m_off, d.m_bytes, d.total_bytes};
    std::memcpy(blob + 24, ho, 40);

    // weights: tile t, column k -> tile_n/2 contiguous bytes
    const int32_t T = N / tile_n;
    const int32_t half = tile_n / 2;
    uint8_t* wr = blob + d.w_off;
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < half; ++j) {
            const uint8_t* r0 = src.qrow((uint64_t)t * tile_n + 2 * j, K);       // even row
            const uint8_t* r1 = src.qrow((uint64_t)t * tile_n + 2 * j + 1, K);   // odd row
            uint8_t* dst = wr + (uint64_t)t * K * half + j;
            for (int32_t k = 0; k < K; ++k)
                dst[(uint64_t)k * half] = (uint8_t)(r0[k] | (r1[k] << 4));
        }
    }
    if (ng) {
        // metadata: outputs 256 h .. 256 h + 255, column k -> (s, z) of group
        // 2 h, then (s, z) of group 2 h + 1
        uint16_t* md = reinterpret_cast<uint16_t*>(blob + d.m_off);
        const int32_t H = N / (2 * SGEMV_GROUP);
        for (int32_t h = 0; h < H; ++h)
            for (int32_t e = 0; e < 2; ++e) {
                const uint64_t n = ((uint64_t)2 * h + e) * SGEMV_GROUP;
                for (int32_t k = 0; k < K; ++k) {
                    const uint64_t o = (((uint64_t)h * K + k) * 2 + e) * 2;
                    md[o] = src.scale_ng(n, K, k);
                    md[o + 1] = src.zero_ng(n, K, k);
                }
            }
    } else if (version == SGEMV_LAYOUT_Z4) {
        // metadata: tile t, group g -> tile_n scales, then tile_n / 2 bytes of
        // 4-bit zero-points (even row in the low nibble)
        const uint64_t run = (uint64_t)tile_n * 5 / 2;
        for (int32_t t = 0; t < T; ++t)
            for (int32_t g = 0; g < Gk; ++g) {
                uint8_t* r = blob + d.m_off + ((uint64_t)t * Gk + g) * run;
                for (int32_t i = 0; i < tile_n; ++i) {
                    const uint64_t n = (uint64_t)t * tile_n + i;
                    const uint16_t sb = src.scale(n, Gk, g);
                    r[2 * i] = (uint8_t)(sb & 0xFF);
                    r[2 * i + 1] = (uint8_t)(sb >> 8);
                    const uint8_t z = (uint8_t)fp16_small_int(src.zero(n, Gk, g));
                    r[2 * tile_n + i / 2] |= (uint8_t)(z << (4 * (i & 1)));
                }
            }
    } else {
        // metadata: tile t, group g -> tile_n (s, z) pairs
        uint16_t* md = reinterpret_cast<uint16_t*>(blob + d.m_off);
        for (int32_t t = 0; t < T; ++t)
            for (int32_t i = 0; i < tile_n; ++i) {
                const uint64_t n = (uint64_t)t * tile_n + i;
                for (int32_t g = 0; g < Gk; ++g) {
                    const uint64_t o = (((uint64_t)t * Gk + g) * tile_n + i) * 2;
                    md[o] = src.scale(n, Gk, g);
                    md[o + 1] = src.zero(n, Gk, g);
                }
            }
    }
    if (desc_out) *desc_out = d;
    return SGEMV_OK;
}

extern "C" int sgemv_pack_layout(const uint8_t* q, const uint16_t* scales_f16,
                                 const uint16_t* zeros_f16, int32_t N, int32_t K,
                                 int32_t group, int32_t tile_n, void* out,
                                 size_t out_capacity, sgemv_desc* desc_out) {
    const Rows src{1, &q, &scales_f16, &zeros_f16, &N};
    return pack(src, N, K, group, tile_n, SGEMV_LAYOUT_PAIRS, out, out_capacity, desc_out);
}

extern "C" int sgemv_pack_layout_z4(const uint8_t* q, const uint16_t* scales_f16,
                                    const uint16_t* zeros_f16, int32_t N, int32_t K,
                                    int32_t group, int32_t tile_n, void* out,
                                    size_t out_capacity, sgemv_desc* desc_out) {
    const Rows src{1, &q, &scales_f16, &zeros_f16, &N};
    return pack(src, N, K, group, tile_n, SGEMV_LAYOUT_Z4, out, out_capacity, desc_out);
}

extern "C" int sgemv_pack_layout_ng(const uint8_t* q, const uint16_t* scales_f16,
                                    const uint16_t* zeros_f16, int32_t N, int32_t K,
                                    int32_t group, int32_t tile_n, void* out,
                                    size_t out_capacity, sgemv_desc* desc_out) {
    const Rows src{1, &q, &scales_f16, &zeros_f16, &N};
    return pack(src, N, K, group, tile_n, SGEMV_LAYOUT_NG, out, out_capacity, desc_out);
}

extern "C" int sgemv_pack_layout_parts(int32_t parts, const uint8_t* const* q,
                                       const uint16_t* const* scales_f16,
                                       const uint16_t* const* zeros_f16, const int32_t* n_part,
                                       int32_t K, int32_t group, int32_t tile_n, uint32_t version,
                                       void* out, size_t out_capacity, sgemv_desc* desc_out) {
    if (parts < 1 || !n_part) return SGEMV_EINVAL;
    if (version != SGEMV_LAYOUT_PAIRS && version != SGEMV_LAYOUT_Z4 && version != SGEMV_LAYOUT_NG)
        return SGEMV_EINVAL;
    if (out && (!q || !scales_f16 || !zeros_f16)) return SGEMV_EINVAL;
    int64_t N = 0;
    for (int32_t p = 0; p < parts; ++p) {
        // every part whole tiles, so that no tile mixes two parts
        if (n_part[p] <= 0 || tile_n <= 0 || n_part[p] % tile_n) return SGEMV_ESIZE;
        N += n_part[p];
    }
    if (N > SGEMV_MAX_N) return SGEMV_ESIZE;
    const Rows src{parts, q, scales_f16, zeros_f16, n_part};
    return pack(src, (int32_t)N, K, group, tile_n, version, out, out_capacity, desc_out);
}

extern "C" int sgemv_desc_from_header(const void* header, size_t bytes, sgemv_desc* desc_out) {
    if (!header || !desc_out) return SGEMV_EINVAL;
    if (bytes < 64) return SGEMV_ESIZE;
    const uint8_t* h = static_cast<const uint8_t*>(header);
    if (std::memcmp(h, "SGV1", 4) != 0) return SGEMV_EINVAL;
    uint32_t version;
    std::memcpy(&version, h + 4, 4);
    if (version != SGEMV_LAYOUT_PAIRS && version != SGEMV_LAYOUT_Z4 && version != SGEMV_LAYOUT_NG)
        return SGEMV_EINVAL;
    int32_t hv[4];
    std::memcpy(hv, h + 8, 16);
    int st = check_shape(hv[0], hv[1], hv[2], hv[3]);
    if (st) return SGEMV_EINVAL;
    if (version == SGEMV_LAYOUT_NG && hv[3] < 2 * SGEMV_GROUP) return SGEMV_EINVAL;
    uint64_t ho[5];
    std::memcpy(ho, h + 24, 40);
    sgemv_desc d;
    sgemv_layout_fill_desc(hv[0], hv[1], hv[3], version, &d);
    if (ho[0] != d.w_off || ho[1] != d.w_bytes || ho[2] != d.m_off ||
        ho[3] != d.m_bytes || ho[4] != d.total_bytes)
        return SGEMV_EINVAL;
    *desc_out = d;
    return SGEMV_OK;
}
