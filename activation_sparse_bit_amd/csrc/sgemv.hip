// Device kernels and C ABI of the dynamically sparse int4 GEMV (gfx950).
//
// What is computed follows "Enabling Dynamic Sparsity in Quantized LLM
// Inference" (Abstract): the activation vector is thresholded at run time,
// the surviving indices are gathered into a compact list, and a GEMV reads
// only the int4 weight columns (with their group-128 fp16 scale and
// zero-point) that the list names, from a layout arranged so that every
// listed column is one contiguous run of bytes.  The kernels below are our
// own CDNA4 design; the page's kernels target other GPUs and are not given.
//
// Kernels
//   k_gather   one 1024-thread workgroup: per-lane 8-element masks from
//              16-byte loads, wavefront ballots and mbcnt for in-wave ranks,
//              an LDS scan across the 16 wavefronts, ordered index writes.
//   k_run      grid = (tiles of 512 outputs) x (slices of the index list).
//              Each wavefront owns all 512 outputs of its tile (8 per lane)
//              and a run of list positions; it reads the listed columns with
//              one 4-byte load per lane (256 contiguous bytes per column),
//              dequantizes pairs of columns exactly in fp16
//              (magic-number nibble extraction, q - z in fp16) and
//              accumulates with v_dot2_f32_f16 in fp32, applying the group
//              scale once per (group, output).  Wavefronts are summed by a
//              fixed-order LDS tree, slices through a workspace by the last
//              workgroup to arrive, in slice order: the result is
//              bitwise reproducible.  No MFMA: this is a matrix-vector
//              product bound by HBM bandwidth.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "sgemv.h"

extern "C" int sgemv_layout_fill_desc(int32_t N, int32_t K, int32_t tile_n, sgemv_desc* d);

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kTileN = SGEMV_TILE_N;  // outputs per tile
constexpr int kGroup = SGEMV_GROUP;
constexpr int kChunk = 16;            // list positions a wavefront loads at once
constexpr int kColBytes = kTileN / 2; // bytes of one column within one tile

thread_local int g_last_hip_error = 0;

struct Codes {
    uint32_t w[8];  // 16 threshold codes, two per word
};

struct RunArgs {
    const uint8_t* w;        // weight region of the blob
    const uint32_t* md;      // metadata region: one (s | z << 16) word per (tile, group, row)
    const uint16_t* x;       // fp16 bits [M][ldx]
    const int32_t* idx;      // listed columns (unused when dense)
    const int32_t* count;    // number of listed columns (device)
    void* y;
    uint32_t* counters;      // one arrival counter per tile
    float* partials;         // [tile][slice][Mt][512]
    int32_t K, ldx, ldy, M;
    int32_t tiles, slices_max;
    uint32_t out_f32;
    Codes tc;
};

__device__ __forceinline__ uint32_t code_of(const Codes& c, int m) {
    return (c.w[m >> 1] >> ((m & 1) * 16)) & 0xFFFFu;
}

// |x| >= t for an fp16 bit pattern, with t given as the smallest fp16
// magnitude code whose value is >= t.  Magnitudes above 0x7C00 are NaN.
__device__ __forceinline__ bool is_active(uint32_t bits, uint32_t code) {
    const uint32_t mag = bits & 0x7FFFu;
    return mag >= code && mag <= 0x7C00u;
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// ---------------------------------------------------------------------------
// index gathering
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mask8_of(uint4 v, uint32_t code) {
    uint32_t m = 0;
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m |= (uint32_t)is_active(wv[i] & 0xFFFFu, code) << (2 * i);
        m |= (uint32_t)is_active(wv[i] >> 16, code) << (2 * i + 1);
    }
    return m;
}

// Exclusive prefix (over lower lanes) and wave total of a per-lane count in
// 0..15, from four bit-plane ballots.
__device__ __forceinline__ void wave_scan16(uint32_t c, uint32_t& prefix, uint32_t& total) {
    prefix = 0;
    total = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const unsigned long long bal = __ballot((c >> b) & 1u);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        prefix += below << b;
        total += (uint32_t)__popcll(bal) << b;
    }
}

__global__ __launch_bounds__(1024) void k_gather(const uint16_t* __restrict__ x, int M, int K, int ldx,
                                                 Codes tc, int32_t* __restrict__ idx,
                                                 int32_t* __restrict__ count) {
    __shared__ uint8_t masks[SGEMV_MAX_K / 8];
    __shared__ uint32_t wtot[16];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int Kw = K >> 4;          // elements per wavefront, a multiple of 8
    const int base = wave * Kw;

    uint32_t mytotal = 0;
    for (int s = 0; s * 512 < Kw; ++s) {
        const int off = s * 512 + lane * 8;
        uint32_t m8 = 0;
        if (off < Kw) {
            for (int m = 0; m < M; ++m) {
                const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)m * ldx + base + off);
                m8 |= mask8_of(v, code_of(tc, m));
            }
            masks[(base + off) >> 3] = (uint8_t)m8;
        }
        uint32_t pre, tot;
        wave_scan16((uint32_t)__popc(m8), pre, tot);
        mytotal += tot;
    }
    if (lane == 0) wtot[wave] = mytotal;
    __syncthreads();
    uint32_t wbase = 0, grand = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const uint32_t t = wtot[w];
        wbase += (w < wave) ? t : 0u;
        grand += t;
    }
    if (threadIdx.x == 0) *count = (int32_t)grand;

    uint32_t running = wbase;
    for (int s = 0; s * 512 < Kw; ++s) {
        const int off = s * 512 + lane * 8;
        uint32_t m8 = (off < Kw) ? masks[(base + off) >> 3] : 0u;
        uint32_t pre, tot;
        wave_scan16((uint32_t)__popc(m8), pre, tot);
        uint32_t pos = running + pre;
        while (m8) {
            const int b = __builtin_ctz(m8);
            idx[pos++] = base + off + b;
            m8 &= m8 - 1u;
        }
        running += tot;
    }
}

// ---------------------------------------------------------------------------
// sparse / dense GEMV
// ---------------------------------------------------------------------------
template <int MT>
struct WaveState {
    float y[MT][8];     // running sums per row and output (odd outputs x16)
    float acc[MT][8];   // current group's sums of (q - z) * x
    uint32_t md[8];     // current group's (s | z << 16) words
    half2_t zc[8];      // 1024 + z (even outputs) / 1024 + 16 z (odd), both halves
};

template <int MT>
__device__ __forceinline__ void fold_group(WaveState<MT>& st) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float s = (float)as_h2(st.md[r]).x;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            st.y[m][r] = __builtin_fmaf(s, st.acc[m][r], st.y[m][r]);
            st.acc[m][r] = 0.f;
        }
    }
}

template <int MT>
__device__ __forceinline__ void set_group(WaveState<MT>& st, const uint32_t (&md)[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        st.md[r] = md[r];
        const _Float16 z = as_h2(md[r]).y;
        const _Float16 zz = (r & 1) ? (_Float16)(z * (_Float16)16.0f) : z;
        st.zc[r] = (half2_t){zz, zz} + (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
    }
}

// Two listed columns A (list position 2p) and B (2p+1) of this lane's 8
// outputs.  Byte i of a column word holds outputs 2i (low nibble) and 2i+1
// (high nibble).  v_perm puts byte i of A and of B into the low bytes of the
// two halves; OR-ing 0x6400 makes each half the fp16 value 1024 + q (low
// nibble) or 1024 + 16 q (high nibble), exactly; subtracting the matching
// 1024 + z (or 1024 + 16 z) leaves q - z (or 16 (q - z)) exactly, and
// v_dot2_f32_f16 adds (q_A - z) x_A + (q_B - z) x_B to the fp32 sum.
template <int MT>
__device__ __forceinline__ void dot_pair(WaveState<MT>& st, uint32_t A, uint32_t B,
                                         const uint32_t (&xp)[MT]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t sel = (0x0Cu << 24) | ((uint32_t)i << 16) | (0x0Cu << 8) | (4u + i);
        const uint32_t R = __builtin_amdgcn_perm(A, B, sel);
        const half2_t lo = as_h2((R & 0x000F000Fu) | 0x64006400u) - st.zc[2 * i];
        const half2_t hi = as_h2((R & 0x00F000F0u) | 0x64006400u) - st.zc[2 * i + 1];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            st.acc[m][2 * i] = __builtin_amdgcn_fdot2(lo, as_h2(xp[m]), st.acc[m][2 * i], false);
            st.acc[m][2 * i + 1] = __builtin_amdgcn_fdot2(hi, as_h2(xp[m]), st.acc[m][2 * i + 1], false);
        }
    }
}

// Scale/zero words of this lane's 8 outputs for one (tile, group): the
// uniform base lives in SGPRs, the lane offset in a VGPR.
__device__ __forceinline__ void load_md(const uint32_t* __restrict__ grp, int lane, uint32_t (&md)[8]) {
    const uint4* p = reinterpret_cast<const uint4*>(grp) + lane * 2;
    const uint4 a = p[0];
    const uint4 b = p[1];
    md[0] = a.x; md[1] = a.y; md[2] = a.z; md[3] = a.w;
    md[4] = b.x; md[5] = b.y; md[6] = b.z; md[7] = b.w;
}

template <int MT, int WPW, int CHUNKS, bool DENSE, bool MASK>
__global__ __launch_bounds__(WPW * 64) void k_run(RunArgs a) {
    constexpr int kColsWave = kChunk * CHUNKS;
    constexpr int kColsWG = kColsWave * WPW;
    __shared__ uint16_t xs[WPW][MT][kChunk];
    __shared__ float red[(WPW > 1 ? WPW / 2 : 1)][MT][kTileN];

    const int tile = blockIdx.x % a.tiles;
    const int slice = blockIdx.x / a.tiles;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int K = a.K;
    const int Gk = K / kGroup;

    int count;
    if (DENSE) {
        count = K;
    } else {
        count = __builtin_amdgcn_readfirstlane(*a.count);
        count = count < 0 ? 0 : (count > K ? K : count);
    }
    const int S = count > 0 ? (count + kColsWG - 1) / kColsWG : 1;
    if (slice >= S) return;

    WaveState<MT> st;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            st.y[m][r] = 0.f;
            st.acc[m][r] = 0.f;
        }
    int gcur = -1;

    const uint8_t* __restrict__ wtile = a.w + (size_t)tile * K * kColBytes;
    const uint32_t* __restrict__ mdtile = a.md + (size_t)tile * Gk * kTileN;
    const int wbase = slice * kColsWG + wave * kColsWave;

    for (int c = 0; c < CHUNKS; ++c) {
        const int j0 = wbase + c * kChunk;
        int nv = count - j0;
        nv = nv > kChunk ? kChunk : nv;
        if (nv <= 0) break;

        // listed columns of this chunk (uniform); padding repeats the last one
        // (j0 + 16 <= K always holds, so all 16 entries are in bounds)
        int kk[kChunk];
        if (DENSE) {
#pragma unroll
            for (int i = 0; i < kChunk; ++i) kk[i] = j0 + i;
        } else {
            const int4* ip = reinterpret_cast<const int4*>(a.idx + j0);
#pragma unroll
            for (int q4 = 0; q4 < kChunk / 4; ++q4) {
                const int4 v = ip[q4];
                kk[4 * q4 + 0] = v.x; kk[4 * q4 + 1] = v.y;
                kk[4 * q4 + 2] = v.z; kk[4 * q4 + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                int k = (i == 0 || i < nv) ? kk[i] : kk[i > 0 ? i - 1 : 0];
                k = (unsigned)k < (unsigned)K ? k : K - 1;
                kk[i] = __builtin_amdgcn_readfirstlane(k);
            }
        }

        // weight words of this lane for every column (256 contiguous bytes per column)
        uint32_t wv[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const uint32_t* col = reinterpret_cast<const uint32_t*>(wtile + (size_t)kk[i] * kColBytes);
            wv[i] = __builtin_nontemporal_load(col + lane);
        }

        // scale/zero words of up to three consecutive groups from the first
        const int gA = kk[0] >> 7;
        const int gZ = kk[kChunk - 1] >> 7;
        uint32_t slot[3][8];
#pragma unroll
        for (int sidx = 0; sidx < 3; ++sidx)
            if (gA + sidx <= gZ) load_md(mdtile + (size_t)(gA + sidx) * kTileN, lane, slot[sidx]);

        // stage this chunk's activations (masked, zero for padding) in LDS
        for (int e = lane; e < MT * kChunk; e += 64) {
            const int m = e / kChunk, i = e % kChunk;
            uint32_t v = 0;
            if (m < a.M && i < nv) {
                int k = DENSE ? j0 + i : a.idx[j0 + i];
                k = (unsigned)k < (unsigned)K ? k : K - 1;
                v = a.x[(size_t)m * a.ldx + k];
                if (MASK && !is_active(v, code_of(a.tc, m))) v = 0;
            }
            xs[wave][m][i] = (uint16_t)v;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
        for (int p = 0; p < kChunk / 2; ++p) {
            uint32_t xp[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                xp[m] = reinterpret_cast<const uint32_t*>(&xs[wave][m][0])[p];
            const int ga = kk[2 * p] >> 7;
            const int gb = kk[2 * p + 1] >> 7;
            if (ga != gcur) {
                if (gcur >= 0) fold_group(st);
                const int d = ga - gA;
                if (d == 0) set_group(st, slot[0]);
                else if (d == 1) set_group(st, slot[1]);
                else if (d == 2) set_group(st, slot[2]);
                else {
                    uint32_t tmp[8];
                    load_md(mdtile + (size_t)ga * kTileN, lane, tmp);
                    set_group(st, tmp);
                }
                gcur = ga;
            }
            if (gb == ga) {
                dot_pair(st, wv[2 * p], wv[2 * p + 1], xp);
            } else {
                uint32_t xa[MT], xb[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    xa[m] = xp[m] & 0x0000FFFFu;
                    xb[m] = xp[m] & 0xFFFF0000u;
                }
                dot_pair(st, wv[2 * p], wv[2 * p + 1], xa);
                fold_group(st);
                const int d = gb - gA;
                if (d == 1) set_group(st, slot[1]);
                else if (d == 2) set_group(st, slot[2]);
                else {
                    uint32_t tmp[8];
                    load_md(mdtile + (size_t)gb * kTileN, lane, tmp);
                    set_group(st, tmp);
                }
                gcur = gb;
                dot_pair(st, wv[2 * p], wv[2 * p + 1], xb);
            }
        }
    }
    if (gcur >= 0) fold_group(st);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 1; r < 8; r += 2) st.y[m][r] *= 0.0625f;  // the 16 of the high nibbles

    // fixed-order tree over the wavefronts of the workgroup
#pragma unroll
    for (int h = WPW / 2; h >= 1; h /= 2) {
        if (wave >= h && wave < 2 * h) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float4* dst = reinterpret_cast<float4*>(&red[wave - h][m][lane * 8]);
                dst[0] = make_float4(st.y[m][0], st.y[m][1], st.y[m][2], st.y[m][3]);
                dst[1] = make_float4(st.y[m][4], st.y[m][5], st.y[m][6], st.y[m][7]);
            }
        }
        __syncthreads();
        if (wave < h) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float4* src = reinterpret_cast<const float4*>(&red[wave][m][lane * 8]);
                const float4 u = src[0], v = src[1];
                st.y[m][0] += u.x; st.y[m][1] += u.y; st.y[m][2] += u.z; st.y[m][3] += u.w;
                st.y[m][4] += v.x; st.y[m][5] += v.y; st.y[m][6] += v.z; st.y[m][7] += v.w;
            }
        }
        __syncthreads();
    }
    if (wave != 0) return;

    const int n0 = tile * kTileN + lane * 8;
    auto store_y = [&](const float (&v)[MT][8]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= a.M) break;
            if (a.out_f32) {
                float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.y) + (size_t)m * a.ldy + n0);
                dst[0] = make_float4(v[m][0], v[m][1], v[m][2], v[m][3]);
                dst[1] = make_float4(v[m][4], v[m][5], v[m][6], v[m][7]);
            } else {
                uint32_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const half2_t pr = (half2_t){(_Float16)v[m][2 * r], (_Float16)v[m][2 * r + 1]};
                    h[r] = __builtin_bit_cast(uint32_t, pr);
                }
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + (size_t)m * a.ldy + n0) =
                    make_uint4(h[0], h[1], h[2], h[3]);
            }
        }
    };

    if (S == 1) {
        store_y(st.y);
        return;
    }

    // publish this slice's sums; the last workgroup of the tile adds all
    // slices in slice order and writes y
    float* part = a.partials + ((size_t)tile * a.slices_max + slice) * MT * kTileN + lane * 8;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float4* dst = reinterpret_cast<float4*>(part + m * kTileN);
        dst[0] = make_float4(st.y[m][0], st.y[m][1], st.y[m][2], st.y[m][3]);
        dst[1] = make_float4(st.y[m][4], st.y[m][5], st.y[m][6], st.y[m][7]);
    }
    __threadfence();
    uint32_t old = 0;
    if (lane == 0) old = atomicAdd(&a.counters[tile], 1u);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(S - 1)) return;
    __threadfence();

    float tot[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 8; ++r) tot[m][r] = 0.f;
    const float* p0 = a.partials + (size_t)tile * a.slices_max * MT * kTileN + lane * 8;
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float4* src = reinterpret_cast<const float4*>(p0 + ((size_t)s * MT + m) * kTileN);
            const float4 u = src[0];
            const float4 v = src[1];
            tot[m][0] += u.x; tot[m][1] += u.y; tot[m][2] += u.z; tot[m][3] += u.w;
            tot[m][4] += v.x; tot[m][5] += v.y; tot[m][6] += v.z; tot[m][7] += v.w;
        }
    }
    store_y(tot);
    if (lane == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Shape {
    int wpw, chunks;
    int cols() const { return 16 * chunks * wpw; }
};

Shape shape_for(int mt) {
    switch (mt) {
        case 1: return {8, 2};
        case 2: return {8, 2};
        case 4: return {8, 2};
        case 8: return {8, 4};
        default: return {4, 8};
    }
}

int pow2_ceil(int m) {
    int p = 1;
    while (p < m) p <<= 1;
    return p;
}

float half_value(uint32_t b) {
    const int e = (b >> 10) & 0x1F;
    const int m = b & 0x3FF;
    if (e == 0) return std::ldexp((float)m, -24);
    if (e == 31) return INFINITY;
    return std::ldexp((float)(1024 + m), e - 25);
}

// Smallest fp16 magnitude code c in [0, 0x7C00] whose value is >= t.
uint32_t threshold_code(float t) {
    uint32_t lo = 0, hi = 0x7C00;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) / 2;
        if (half_value(mid) >= t) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

int fill_codes(const float* thr, int M, Codes& c) {
    std::memset(&c, 0, sizeof c);
    for (int m = 0; m < M; ++m) {
        const float t = thr[m];
        if (!std::isfinite(t) || t < 0.f) return SGEMV_EINVAL;
        c.w[m >> 1] |= threshold_code(t) << ((m & 1) * 16);
    }
    return SGEMV_OK;
}

int check_desc(const sgemv_desc* d) {
    if (!d) return SGEMV_EINVAL;
    if (d->group != kGroup) return SGEMV_EINVAL;
    if (d->N <= 0 || d->K <= 0 || d->K % kGroup || d->K > SGEMV_MAX_K || d->N > SGEMV_MAX_N)
        return SGEMV_ESIZE;
    if (d->tile_n < 64 || d->tile_n > 1024 || (d->tile_n & (d->tile_n - 1)) || d->N % d->tile_n)
        return SGEMV_ESIZE;
    sgemv_desc ref;
    sgemv_layout_fill_desc(d->N, d->K, d->tile_n, &ref);
    if (d->w_off != ref.w_off || d->w_bytes != ref.w_bytes || d->m_off != ref.m_off ||
        d->m_bytes != ref.m_bytes || d->total_bytes != ref.total_bytes)
        return SGEMV_EINVAL;
    if (d->tile_n != kTileN) return SGEMV_EUNSUPPORTED;
    return SGEMV_OK;
}

size_t ws_counters_bytes(int tiles) { return ((size_t)tiles * 4 + 255) / 256 * 256; }

size_t ws_bytes_for(const sgemv_desc* d, int mt) {
    const int tiles = d->N / kTileN;
    const Shape sh = shape_for(mt);
    const int smax = (d->K + sh.cols() - 1) / sh.cols();
    size_t b = ws_counters_bytes(tiles);
    if (smax > 1) b += (size_t)tiles * smax * mt * kTileN * sizeof(float);
    return b;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <int MT, bool DENSE, bool MASK>
hipError_t launch_run(const RunArgs& a, hipStream_t s) {
    constexpr Shape sh = {MT <= 8 ? 8 : 4, MT <= 4 ? 2 : MT == 8 ? 4 : 8};
    const dim3 grid((unsigned)(a.tiles * a.slices_max));
    hipLaunchKernelGGL((k_run<MT, sh.wpw, sh.chunks, DENSE, MASK>), grid, dim3(sh.wpw * 64), 0, s, a);
    return hipGetLastError();
}

template <bool DENSE, bool MASK>
hipError_t launch_mt(int mt, const RunArgs& a, hipStream_t s) {
    switch (mt) {
        case 1: return launch_run<1, DENSE, MASK>(a, s);
        case 2: return launch_run<2, DENSE, MASK>(a, s);
        case 4: return launch_run<4, DENSE, MASK>(a, s);
        case 8: return launch_run<8, DENSE, MASK>(a, s);
        default: return launch_run<16, DENSE, MASK>(a, s);
    }
}

int run_common(const sgemv_desc* d, const void* packed, const void* x, int M, int ldx,
               const float* thr, const int32_t* idx, const int32_t* count, void* y, int ldy,
               uint32_t flags, void* ws, void* stream) {
    int st = check_desc(d);
    if (st) return st;
    if (!packed || !x || !y) return SGEMV_EINVAL;
    if (idx && !count) return SGEMV_EINVAL;
    if (flags & ~SGEMV_OUT_F32) return SGEMV_EINVAL;
    if (M < 1 || M > SGEMV_MAX_BATCH) return SGEMV_ESIZE;
    if (ldx < d->K || ldy < d->N) return SGEMV_ESIZE;
    if (ldx % 8 || ldy % 8) return SGEMV_EALIGN;
    if (!aligned(packed, 256) || !aligned(x, 16) || !aligned(y, 16)) return SGEMV_EALIGN;
    if (idx && !aligned(idx, 4)) return SGEMV_EALIGN;
    if (count && !aligned(count, 4)) return SGEMV_EALIGN;

    const int mt = pow2_ceil(M);
    const Shape sh = shape_for(mt);
    RunArgs a;
    std::memset(&a, 0, sizeof a);
    if (thr) {
        st = fill_codes(thr, M, a.tc);
        if (st) return st;
    }
    a.tiles = d->N / kTileN;
    a.slices_max = (d->K + sh.cols() - 1) / sh.cols();
    if (a.slices_max > 1) {
        if (!ws) return SGEMV_EINVAL;
        if (!aligned(ws, 256)) return SGEMV_EALIGN;
    }
    const uint8_t* blob = static_cast<const uint8_t*>(packed);
    a.w = blob + d->w_off;
    a.md = reinterpret_cast<const uint32_t*>(blob + d->m_off);
    a.x = static_cast<const uint16_t*>(x);
    a.idx = idx;
    a.count = count;
    a.y = y;
    a.counters = static_cast<uint32_t*>(ws);
    a.partials = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + ws_counters_bytes(a.tiles))
                    : nullptr;
    a.K = d->K;
    a.ldx = ldx;
    a.ldy = ldy;
    a.M = M;
    a.out_f32 = (flags & SGEMV_OUT_F32) ? 1u : 0u;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const bool dense = (idx == nullptr);
    const bool mask = (thr != nullptr);
    if (dense) e = mask ? launch_mt<true, true>(mt, a, s) : launch_mt<true, false>(mt, a, s);
    else e = mask ? launch_mt<false, true>(mt, a, s) : launch_mt<false, false>(mt, a, s);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SGEMV_EHIP;
    }
    return SGEMV_OK;
}

}  // namespace

extern "C" int sgemv_gather_indices(const void* x_f16, int32_t M, int32_t K, int32_t ldx,
                                    const float* thresholds, int32_t* idx, int32_t* count,
                                    void* stream) {
    if (!x_f16 || !thresholds || !idx || !count) return SGEMV_EINVAL;
    if (M < 1 || M > SGEMV_MAX_BATCH) return SGEMV_ESIZE;
    if (K <= 0 || K % kGroup || K > SGEMV_MAX_K || ldx < K) return SGEMV_ESIZE;
    if (ldx % 8) return SGEMV_EALIGN;
    if (!aligned(x_f16, 16) || !aligned(idx, 4) || !aligned(count, 4)) return SGEMV_EALIGN;
    Codes c;
    int st = fill_codes(thresholds, M, c);
    if (st) return st;
    hipLaunchKernelGGL(k_gather, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(x_f16), (int)M, (int)K, (int)ldx, c, idx, count);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SGEMV_EHIP;
    }
    return SGEMV_OK;
}

extern "C" int sgemv_run(const sgemv_desc* d, const void* packed, const void* x_f16,
                         const int32_t* idx, const int32_t* count, void* y, uint32_t flags,
                         void* workspace, void* stream) {
    if (!d) return SGEMV_EINVAL;
    return run_common(d, packed, x_f16, 1, d->K, nullptr, idx, count, y, d->N, flags, workspace,
                      stream);
}

extern "C" int sgemv_run_batched(const sgemv_desc* d, const void* packed, const void* x_f16,
                                 int32_t M, int32_t ldx, const float* thresholds,
                                 const int32_t* idx, const int32_t* count, void* y, int32_t ldy,
                                 uint32_t flags, void* workspace, void* stream) {
    return run_common(d, packed, x_f16, M, ldx, thresholds, idx, count, y, ldy, flags, workspace,
                      stream);
}

extern "C" size_t sgemv_workspace_bytes(const sgemv_desc* d, int32_t M) {
    if (check_desc(d) != SGEMV_OK || M < 1 || M > SGEMV_MAX_BATCH) return 0;
    size_t b = 0;
    for (int mt = 1; mt <= pow2_ceil(M); mt <<= 1) {
        const size_t v = ws_bytes_for(d, mt);
        b = v > b ? v : b;
    }
    return b;
}

extern "C" const char* sgemv_strerror(int status) {
    switch (status) {
        case SGEMV_OK: return "ok";
        case SGEMV_EINVAL: return "invalid argument";
        case SGEMV_ESIZE: return "size out of range";
        case SGEMV_EALIGN: return "misaligned pointer or leading dimension";
        case SGEMV_EUNSUPPORTED: return "layout not supported by the device kernels";
        case SGEMV_EHIP: return "HIP call failed";
        default: return "unknown status";
    }
}

extern "C" int sgemv_last_hip_error(void) { return g_last_hip_error; }
