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
//   k_gather   the standalone gathering step: a few workgroups, each over
//              its own column range, with no scratch and no communication
//              (each recounts the active columns below its range from x);
//              per-lane 8-element masks from 16-byte loads (two entries per
//              packed 16-bit instruction), bit-plane ballots and mbcnt for
//              in-wave ranks, an LDS scan across the wavefronts, ordered
//              index writes.
//   k_fs, k_fs4  one or two rows, fused: threshold, compaction and GEMV in
//              one launch, one quantization group per wavefront, 8 or (one
//              row, small or short-K matrices) 4 wavefronts per workgroup
//              (k_fs4: the 8-wavefront build for grids of several rounds);
//              with every column listed, also the dense GEMV (no compaction).
//              Every layout version: groups along K with (s, z) pairs or
//              compact zero-points, or groups along N (one (s, z) per column
//              and 128 outputs, the scale folded into the activation).
//   k_fm       3 to 16 rows, fused (or over a given list): the union of the
//              rows' active columns, exact fp16 dequantization in registers
//              and v_mfma_f32_16x16x32_f16 on the matrix cores.
// The vector kernels dequantize exactly in fp16 (magic-number nibble
// extraction, q - z in fp16) and accumulate with v_dot2_f32_f16 in fp32; the
// matrix kernel feeds the same exact values to the MFMA.  The group scale is
// applied once per (group, output).  Lanes, wavefronts and workgroups are
// combined in fixed orders (the last workgroup of a half tile to arrive adds
// the others' published sums in segment order), so the result is bitwise
// reproducible.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "sgemv.h"

extern "C" int sgemv_layout_fill_desc(int32_t N, int32_t K, int32_t tile_n, uint32_t version,
                                      sgemv_desc* d);

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kTileN = SGEMV_TILE_N;  // outputs per tile
constexpr int kGroup = SGEMV_GROUP;
constexpr int kCounterStride = 64;   // uint32 words between arrival counters

thread_local int g_last_hip_error = 0;

struct Codes {
    uint32_t w[8];  // 16 threshold codes, two per word
};

struct RunArgs {
    const uint8_t* w;        // weight region of the blob
    const uint8_t* md;       // metadata region (layout version 1, 2 or 3)
    uint32_t md_z4;          // version 2: fp16 scales, then 4-bit zero-points
    const uint16_t* x;       // fp16 bits [M][ldx]
    void* y;
    uint32_t* counters;      // one arrival counter per half tile, kCounterStride words apart
    float* partials;         // [half tile][segment][M][256] segment sums
    uint32_t partial_bytes;  // size of the partials region
    int32_t K, ldx, ldy, M;
    int32_t tiles, slices;
    uint32_t out_f32;
    Codes tc;
    int32_t* idx_out;        // fused kernel: list output (optional)
    int32_t* count_out;      // fused kernel: count output (optional)
    int32_t segs;            // fused kernel: column segments
    uint32_t all_cols;       // fused kernels: every column listed (dense), rows masked unless unmasked
    uint32_t unmasked;       // fused kernels: activations used as they are (no thresholds)
    int32_t gblocks;         // many-row fused kernel: workgroups that build the list (0 without one)
    int32_t grange;          // ... columns per such workgroup (a multiple of 128)
    int32_t* gscratch;       // ... their lists, at the first column of each range ([K])
    uint32_t* gsync;         // ... [0]: arrival counter, [16 + j]: length of list j
    const int32_t* lidx;     // fused kernels over a given list (NULL: the list is computed)
    const int32_t* lcount;   // ... its length
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

// The list for rows x[0..M) by one workgroup of W wavefronts: wavefront w
// owns the K / W consecutive columns w K / W ..; pass 1 builds per-lane
// 8-column masks (kept in LDS) and counts, an LDS exchange of the
// wavefront totals gives every wavefront its base, pass 2 writes the
// columns in order.
struct GatherShared {
    uint8_t masks[SGEMV_MAX_K / 8];
    uint32_t wtot[16];
};

// Union over rows 0..M-1 of the 8-column masks at column col: the rows are
// loaded RB at a time, all in flight together (rows past M repeat row M - 1,
// whose mask is already in).  Two fp16 values per 32-bit word, decided in
// packed 16-bit arithmetic: with mag = bits & 0x7FFF, a value is inactive
// for its row's code c exactly when mag - c or 0x7C00 - mag is negative as a
// signed 16-bit number (mag < c, or a NaN; both differences lie in
// [-0x7C00, 0x7FFF]), that is the is_active rule; the sign bits are ANDed
// over the rows, and a column is in the union when its bit ends clear.
typedef short s2_t __attribute__((ext_vector_type(2)));

template <int RB>
__device__ __forceinline__ uint32_t union_mask8(const uint16_t* __restrict__ x, int M, int ldx, int col,
                                                const Codes& tc) {
    uint32_t none[4] = {~0u, ~0u, ~0u, ~0u};   // bits 15 and 31: inactive in every row so far
    const s2_t kInf = __builtin_bit_cast(s2_t, 0x7C007C00u);
    for (int m0 = 0; m0 < M; m0 += RB) {
        uint4 v[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int mr = m0 + r < M ? m0 + r : M - 1;
            v[r] = *reinterpret_cast<const uint4*>(x + (size_t)mr * ldx + col);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int mr = m0 + r < M ? m0 + r : M - 1;
            const uint32_t c = code_of(tc, mr);
            const s2_t c2 = __builtin_bit_cast(s2_t, c | (c << 16));
            const uint32_t wv[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const s2_t mag = __builtin_bit_cast(s2_t, wv[i] & 0x7FFF7FFFu);
                none[i] &= __builtin_bit_cast(uint32_t, mag - c2) | __builtin_bit_cast(uint32_t, kInf - mag);
            }
        }
    }
    uint32_t m8 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m8 |= (((none[i] >> 15) & 1u) | ((none[i] >> 30) & 2u)) << (2 * i);
    return ~m8 & 0xFFu;
}

// Wavefronts W and above of the workgroup only join the barrier.  The
// entries written are kbase + column (x points at column kbase); with COH
// the list and count are stored device-coherent (written through), for a
// workgroup on another XCD to read.
template <int W, bool COH = false>
__device__ __forceinline__ void gather_body(const uint16_t* __restrict__ x, int M, int K, int ldx, const Codes& tc,
                                            int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                            GatherShared& gs, int kbase = 0) {
    static_assert(W == 4 || W == 8 || W == 16, "K / W must stay a multiple of 8");
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int Kw = K / W;           // columns per wavefront, a multiple of 8
    const int base = wave * Kw;
    const bool work = wave < W;

    uint32_t mytotal = 0;
    for (int s = 0; work && s * 512 < Kw; ++s) {
        const int off = s * 512 + lane * 8;
        uint32_t m8 = 0;
        if (off < Kw) {
            m8 = M >= 8 ? union_mask8<8>(x, M, ldx, base + off, tc)
               : M >= 4 ? union_mask8<4>(x, M, ldx, base + off, tc)
                        : union_mask8<1>(x, M, ldx, base + off, tc);
            gs.masks[(base + off) >> 3] = (uint8_t)m8;
        }
        uint32_t pre, tot;
        wave_scan16((uint32_t)__popc(m8), pre, tot);
        mytotal += tot;
    }
    if (work && lane == 0) gs.wtot[wave] = mytotal;
    __syncthreads();
    if (!work) return;
    uint32_t wbase = 0, grand = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const uint32_t t = gs.wtot[w];
        wbase += (w < wave) ? t : 0u;
        grand += t;
    }
    if (threadIdx.x == 0) {
        if (COH) __hip_atomic_store(count, (int32_t)grand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *count = (int32_t)grand;
    }

    uint32_t running = wbase;
    for (int s = 0; s * 512 < Kw; ++s) {
        const int off = s * 512 + lane * 8;
        uint32_t m8 = (off < Kw) ? gs.masks[(base + off) >> 3] : 0u;
        uint32_t pre, tot;
        wave_scan16((uint32_t)__popc(m8), pre, tot);
        uint32_t pos = running + pre;
        while (m8) {
            const int b = __builtin_ctz(m8);
            if (COH) __hip_atomic_store(&idx[pos++], kbase + base + off + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else idx[pos++] = kbase + base + off + b;
            m8 &= m8 - 1u;
        }
        running += tot;
    }
}

// The standalone gathering step over several workgroups, with no scratch
// memory and no communication between them.  Workgroup j owns the columns
// j R .. j R + R - 1 (R = 8 x its thread count, one 8-column chunk per
// thread).  Its threads first count the union's active columns below j R
// straight from x (every earlier range is read again; x is small, and the
// loads are all in flight with the workgroup's own ones), then rank their own
// chunk's columns with bit-plane ballots and an LDS scan of the wavefront
// totals, and write them at that count plus their rank.  The last workgroup
// also writes the count.  Deterministic, and nothing past the count is
// touched.
template <int WW>
__global__ __launch_bounds__(WW * 64) void k_gather(const uint16_t* __restrict__ x, int M, int K, int ldx, Codes tc,
                                                    int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    constexpr int T = WW * 64;
    constexpr int R = 8 * T;
    __shared__ uint32_t wsum[WW], wtot[WW];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int k0 = blockIdx.x * R;
    // the chunk of this thread (columns k0 + 8 t ..), if inside K
    const int own = k0 + 8 * t;
    uint32_t m8 = 0;
    if (own < K)
        m8 = M >= 8 ? union_mask8<8>(x, M, ldx, own, tc)
           : M >= 4 ? union_mask8<4>(x, M, ldx, own, tc)
                    : union_mask8<1>(x, M, ldx, own, tc);
    // active columns below k0: chunks t, t + T, ... of [0, k0)
    uint32_t below = 0;
    for (int c = 8 * t; c < k0; c += 8 * T) {
        const uint32_t u = M >= 8 ? union_mask8<8>(x, M, ldx, c, tc)
                         : M >= 4 ? union_mask8<4>(x, M, ldx, c, tc)
                                  : union_mask8<1>(x, M, ldx, c, tc);
        below += (uint32_t)__popc(u);
    }
    // wavefront sums (butterfly over the 64 lanes), then the workgroup's
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) below += (uint32_t)__shfl_xor((int)below, d);
    uint32_t pre, tot;
    wave_scan16((uint32_t)__popc(m8), pre, tot);
    if (lane == 0) {
        wsum[wave] = below;
        wtot[wave] = tot;
    }
    __syncthreads();
    uint32_t base = 0, grand = 0;
#pragma unroll
    for (int w = 0; w < WW; ++w) {
        base += wsum[w] + (w < wave ? wtot[w] : 0u);
        grand += wtot[w];
    }
    if (blockIdx.x == gridDim.x - 1 && t == 0) {
        uint32_t all = grand;
#pragma unroll
        for (int w = 0; w < WW; ++w) all += wsum[w];
        *count = (int32_t)all;
    }
    uint32_t pos = base + pre;
    while (m8) {
        const int b = __builtin_ctz(m8);
        idx[pos++] = own + b;
        m8 &= m8 - 1u;
    }
}

// ---------------------------------------------------------------------------
// sparse / dense GEMV
// ---------------------------------------------------------------------------
//
// Every kernel works on half tiles: a workgroup owns 256 outputs, one half
// of a 512-output layout tile, whose part of every column run is 128
// contiguous bytes (one cache line).  The one- and two-row kernel and the
// many-row kernel each describe their work split below; both also run over
// a list the caller gives, which they search for each group's entries.
//
// Arithmetic.  For two listed columns a, b the two 4-bit codes of one output
// are placed in the low mantissa bits of 0x6400 (= 1024.0 in fp16), which
// makes the fp16 values 1024 + q exactly (high nibbles: 1024 + 16 q);
// subtracting 1024 + z (or 1024 + 16 z) in packed fp16 leaves q - z (or
// 16 (q - z)) exactly, and v_dot2_f32_f16 adds (q_a - z) x_a + (q_b - z) x_b
// to an fp32 sum.  The weight operands are small integers (or 16 times
// them), exact in fp16; the activations are any finite fp16 values the
// threshold admits, subnormal ones included: the dot instruction and the
// matrix cores take subnormal fp16 inputs at their value (fp16 denormals are
// on), so every product is exact in fp32.  A chunk is computed in one pass per group
// it touches, with x masked to that group's positions, so every pass uses
// one scale and one zero-point and runs without branches.  The scale is
// applied once per (pass, output); the 16 of the high nibbles at the end.
//
// Reduction.  Wavefronts are added by a fixed-order LDS tree.  Slices
// publish their sums with device-scope (sc1) stores, which write through the
// XCD's L2, wait for the stores to complete, and count themselves on a
// per-half-tile atomic counter; the workgroup that arrives last reads every
// slice's sums, adds them in slice order and writes y, then resets the
// counter.  Its loads must not return a stale L2 copy of another XCD's slice:
// the one- and two-row kernels use device-scope (sc1) loads, which miss in
// L2.  The many-row kernel, whose last read is up to 16 times larger, reads
// through L2: each of its workgroups reads its XCC id and counts itself on
// that XCD's field of the arrival word, and when every slice came from the
// last workgroup's own XCD the write-through stores went through its L2,
// which is then current; otherwise it first takes a device-scope acquire
// (dropping its XCD's L2 copies, including the weights other workgroups are
// streaming, which is why the one-row kernel does not do this).  Counting
// by XCD cost the one-row kernel more than its L2 reads saved.  The writers
// need no whole-L2 write-back (a device-scope release would cost about
// 1.7 us per call): their stores write through.  The result does not depend
// on which workgroup arrives last or where the workgroups run.

constexpr int kVTile = 256;            // outputs per workgroup (half a layout tile)
constexpr int kHalfRun = kVTile / 2;   // bytes of one column for those outputs
constexpr uint32_t kCacheSC1 = 16;     // cache policy: coherent at device scope
constexpr uint32_t kCacheSC0 = 1;      // cache policy: miss in the CU's L1, may hit in L2
constexpr int kHwRegXccId = (31 << 11) | 20;   // s_getreg operand: HW_REG_XCC_ID, 32 bits

// The XCD (XCC) this wavefront runs on: the low four bits of HW_REG_XCC_ID.
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg(kHwRegXccId) & 0xFu; }

// Counts the calling workgroup (one thread of the many-row kernel) as an
// arrival of half tile vt, whose S slices are published, and returns 0 if
// others are still to come,
// 1 for the last arrival, 2 for the last arrival when every slice was
// published from its own XCD.  The half tile's 64-bit arrival word holds the
// count in bits 0..7 and, in the 7-bit field at 8 + 7 x, the arrivals from
// XCD x (x < 8).  When the last workgroup's own field holds all S arrivals,
// every slice was written through one L2, its own, so L2 reads of them are
// current; a field that overflows (S > 127) or an id past 7 only ever gives 1.
// A workgroup's placement on the XCDs decides speed only, never the sums.
__device__ __forceinline__ uint32_t count_arrival(uint32_t* counters, int vt, int S) {
    const uint32_t x = xcc_id();
    const uint64_t add = 1ull + (x < 8u ? 1ull << (8u + 7u * x) : 0ull);
    const uint64_t old = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(&counters[vt * kCounterStride]), add,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old & 0xFFu) != (uint32_t)(S - 1)) return 0u;
    return x < 8u && (((old + add) >> (8u + 7u * x)) & 0x7Fu) == (uint64_t)S ? 2u : 1u;
}

// The last arrival leaves the arrival word at zero for the next call.
__device__ __forceinline__ void reset_arrivals(uint32_t* counters, int vt) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(&counters[vt * kCounterStride]), 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The last workgroup's view of the slices the others published, when some
// came through another XCD's L2 (before loads that may hit in its own).
__device__ __forceinline__ void acquire_slices() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Scale/zero metadata of one half tile (256 outputs), in either version of
// the layout: version 1 holds one (s, z) pair of fp16 bit patterns per output
// and group (kTileN * 4 bytes per tile and group); version 2 holds the fp16
// scales, then the integer zero-points as 4-bit codes, two per byte
// (kTileN * 5 / 2 bytes).  md_raw4 loads the 16 bytes per lane of outputs
// o .. o + 3 (o a multiple of 4) and md_cook4 turns them into the version-1
// words (s bits | z bits << 16) either way, so the kernels after it are the
// same for both.  (Version 3, groups along the outputs, has per-column
// metadata and its own loads: fs_block_ng, fs_dense_ng and k_fm<3>.)
struct MdHalf {
    const uint8_t* tile;   // the tile's metadata (group 0)
    uint32_t h;            // which half of the tile
    uint32_t z4;           // version 2
};

// The layout version is a template parameter of every kernel: the handle's
// z4 is then a constant, and the branches below fold away after inlining.
template <bool Z4>
__device__ __forceinline__ MdHalf md_half(const RunArgs& a, int t, int h) {
    const size_t run = Z4 ? (size_t)kTileN * 5 / 2 : (size_t)kTileN * 4;   // bytes per group
    return MdHalf{a.md + (size_t)t * (a.K / kGroup) * run, (uint32_t)h, Z4 ? 1u : 0u};
}

// The loads (md_raw4: version-1 words, or (four scales, four zero codes, 0)
// for version 2) and the conversion (md_cook4) are separate, so that a
// kernel can issue the loads early and convert where it uses the values.
__device__ __forceinline__ u32x4 md_raw4(const MdHalf& m, int g, int o) {
    if (!m.z4)
        return *reinterpret_cast<const u32x4*>(m.tile + ((size_t)g * (2 * kVTile) + m.h * kVTile + o) * 4);
    const uint8_t* run = m.tile + (size_t)g * (kTileN * 5 / 2);
    const int i = (int)m.h * kVTile + o;                 // row within the tile
    const uint2 sv = *reinterpret_cast<const uint2*>(run + 2 * i);
    const uint32_t zv = *reinterpret_cast<const uint16_t*>(run + 2 * kTileN + i / 2);
    return (u32x4){sv.x, sv.y, zv, 0u};
}

__device__ __forceinline__ u32x4 md_cook4(const u32x4& r, uint32_t z4) {
    if (!z4) return r;
    // zero-point z (0..15) as fp16: (1024 + z) - 1024, exactly, two per word
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const uint32_t zv = r.z;
    const uint32_t za = __builtin_bit_cast(
        uint32_t, as_h2(0x64006400u | (zv & 0xFu) | ((zv & 0xF0u) << 12)) - k1024);
    const uint32_t zb = __builtin_bit_cast(
        uint32_t, as_h2(0x64006400u | ((zv >> 8) & 0xFu) | ((zv & 0xF000u) << 4)) - k1024);
    return (u32x4){(r.x & 0xFFFFu) | (za << 16), (r.x >> 16) | (za & 0xFFFF0000u),
                   (r.y & 0xFFFFu) | (zb << 16), (r.y >> 16) | (zb & 0xFFFF0000u)};
}


// Wavefronts per workgroup: two per SIMD for few rows; four in all for
// many rows, whose accumulators fill the register file.
// (R & mask) | magic: with the magic held in a VGPR the compiler can use one
// v_and_or_b32 (a VOP3 instruction on this target takes no literal).
__device__ __forceinline__ uint32_t and_or(uint32_t r, uint32_t mask, uint32_t vmagic) {
    return (r & mask) | vmagic;
}

// ---------------------------------------------------------------------------
// pieces shared by the one- and two-row kernels
// ---------------------------------------------------------------------------
//
// Memory first.  Listed columns are scattered 128-byte runs (one per half
// tile).  On this GPU a wavefront load that fetches one such run per
// instruction (4 bytes per lane) tops out near 2 TB/s, while loads that
// fetch 16 bytes per lane from 8 different runs per instruction reach the
// HBM limit.  So each lane reads 16 bytes of one column: lane
// (c = lane / 8, o = lane % 8) reads bytes 16 o .. 16 o + 15 of the half
// tile's run of its columns, which hold its 32 outputs 32 o .. 32 o + 31,
// and one load instruction covers 8 listed columns (slot c takes column
// pairs, for v_dot2).
//
// Sums.  The 8 slots of an output are combined by a fixed reduce-scatter
// butterfly across lanes (each lane ends with 4 outputs), wavefronts by one
// LDS pass, the segments of a half tile by the last workgroup to arrive, in
// segment order: bitwise reproducible.

constexpr int kLaneOut = 32;   // outputs per lane while computing

__device__ __forceinline__ float u2f(uint32_t v) { return __uint_as_float(v); }
__device__ __forceinline__ uint32_t f2u(float v) { return __float_as_uint(v); }

// Output (within the half tile) of sum d (0..3) that lane l keeps after the
// reduce-scatter over lane bits 5, 4 and 3.
__device__ __forceinline__ int sp_out(int lane, int d) {
    return 32 * (lane & 7) + 8 * d + 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
}

// Sum over the 8 slots (lane bits 5, 4, 3) of 8 per-lane sums v[0..7]
// (outputs 8d .. 8d + 7 of the lane's block); each lane returns one output,
// sp_out(lane, d).  Lane swaps, no LDS: the halves of the wavefront
// exchange with v_permlane32_swap, rows of 16 with v_permlane16_swap, and
// lanes 8 apart with a DPP row rotation.  Fixed order, so reproducible.
__device__ __forceinline__ float sp_reduce8(const float (&v)[8], int lane) {
    float t4[4], t2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // lanes 0-31 keep output j (own + partner's), lanes 32-63 output 4 + j
        const auto r = __builtin_amdgcn_permlane32_swap(f2u(v[j]), f2u(v[4 + j]), false, false);
        t4[j] = u2f(r[0]) + u2f(r[1]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        // even rows keep the lower pair, odd rows the upper pair
        const auto r = __builtin_amdgcn_permlane16_swap(f2u(t4[j]), f2u(t4[2 + j]), false, false);
        t2[j] = u2f(r[0]) + u2f(r[1]);
    }
    const bool b3 = (lane >> 3) & 1;
    const float send = b3 ? t2[0] : t2[1];
    const float keep = b3 ? t2[1] : t2[0];
    return keep + u2f(__builtin_amdgcn_update_dpp(0u, f2u(send), 0x128 /* row_ror:8 */, 0xF, 0xF, false));
}

template <int MT, int NW>
struct SpShared {
    float red[NW][MT][kVTile];
    uint32_t flag;
};

// Sum the workgroup's NW wavefronts and write y (S == 1), or publish the
// workgroup's sums as slice `slice` of S and let the last workgroup of the
// half tile to arrive add every slice in slice order and write y.  Every
// thread of the workgroup calls it (NW >= 4 MT).  Thread t handles output
// t % 256 of row (t / 256) % MT; the NH = NW / (4 MT) groups of 256 MT
// threads split the slices of the last workgroup, whose partial sums are
// then added in group order.
template <int MT, int NW>
__device__ __forceinline__ void sp_finish(const RunArgs& a, int vt, int slice, int S, int wave, int lane,
                                          const float (&v4)[MT][4], SpShared<MT, NW>& sh) {
    static_assert(NW >= 4 * MT, "one thread per output and row");
    constexpr int NH = NW / (4 * MT);
#pragma unroll
    for (int m = 0; m < MT; ++m)
        *reinterpret_cast<float4*>(&sh.red[wave][m][4 * lane]) = make_float4(v4[m][0], v4[m][1], v4[m][2], v4[m][3]);
    __syncthreads();
    const int t = threadIdx.x;
    const int o = t % kVTile;                 // lane-major slot: lane o / 4, sum o % 4
    const int r = t / kVTile;
    const int m = MT == 1 ? 0 : r % MT;
    const int h = r / MT;                     // thread group
    const bool own = h == 0;
    float sum = 0.f;
    if (own) {
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += sh.red[w][m][o];
    }
    const size_t n = (size_t)vt * kVTile + sp_out(o >> 2, o & 3);
    if (S == 1) {
        if (own && m < a.M) {
            if (a.out_f32) static_cast<float*>(a.y)[(size_t)m * a.ldy + n] = sum;
            else static_cast<_Float16*>(a.y)[(size_t)m * a.ldy + n] = (_Float16)sum;
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(a.partials, (short)0, (int)a.partial_bytes, 0x00020000);
    const uint32_t tile_base = (uint32_t)vt * a.slices * MT * kVTile * 4u;
    if (own) {
        const uint32_t off = tile_base + (((uint32_t)slice * MT + m) * kVTile + o) * 4u;
        __builtin_amdgcn_raw_buffer_store_b32(f2u(sum), prs, off, 0, kCacheSC1);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's store acknowledged
    __syncthreads();                // ... and every thread's, before the count
    if (t == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(&a.counters[vt * kCounterStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.flag = (old == (uint32_t)(S - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (sh.flag == 0u) return;

    // last to arrive: group h adds slices s0 .. s1 - 1, 16 loads in flight
    const int per = (S + NH - 1) / NH;
    const int s0 = h * per;
    const int s1 = s0 + per < S ? s0 + per : S;
    float tot = 0.f;
    if (h < NH) {
        for (int sb = s0; sb < s1; sb += 16) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int sl = sb + i < s1 ? sb + i : sb;
                const uint32_t off = tile_base + (((uint32_t)sl * MT + m) * kVTile + o) * 4u;
                v[i] = u2f(__builtin_amdgcn_raw_buffer_load_b32(prs, off, 0, kCacheSC1));
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (sb + i < s1) tot += v[i];
        }
    }
    if constexpr (NH > 1) {  // add the other groups' sums to group 0's, in group order
        if (h >= 1 && h < NH) sh.red[h][m][o] = tot;
        __syncthreads();
        if (own) {
#pragma unroll
            for (int hh = 1; hh < NH; ++hh) tot += sh.red[hh][m][o];
        }
    }
    if (own && m < a.M) {
        if (a.out_f32) static_cast<float*>(a.y)[(size_t)m * a.ldy + n] = tot;
        else static_cast<_Float16*>(a.y)[(size_t)m * a.ldy + n] = (_Float16)tot;
    }
    if (t == 0) __hip_atomic_store(&a.counters[vt * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// a quantization group's entries in a given ascending list
// ---------------------------------------------------------------------------
//
// Entries read per lane per round (all in flight).  The window searched for a
// group holds at most ceil(count / 64) + 128 entries, so one round of 6
// covers every count up to 16384.
constexpr int kListLoads = 6;

// Sets bit k - kw of the four LDS words lm (zeroed by the caller) for every
// entry k of lidx[0 .. c) in [kw, kw + 128), with c > 0.  The wavefront reads
// 64 evenly spaced entries; those below kw are a prefix of the lanes (the list
// is ascending), nlo of them, so the group's entries (at most 128) lie after
// sample nlo - 1 and start at or before sample nlo: one window of positions.
// An unsorted list gives wrong bits, never an access outside lidx[0 .. c).
__device__ __forceinline__ void list_group_bits(const int32_t* __restrict__ lidx, int c, int kw, int lane,
                                                uint32_t* lm) {
    const int step = (c + 63) / 64;
    const int sv = lidx[lane * step < c ? lane * step : c - 1];
    const int nlo = __popcll(__ballot(sv < kw));
    const int ws = nlo > 0 ? (nlo - 1) * step : 0;
    const int we = nlo * step + kGroup < c ? nlo * step + kGroup : c;
    for (int b = ws; b < we; b += 64 * kListLoads) {
        int v[kListLoads];
#pragma unroll
        for (int i = 0; i < kListLoads; ++i) {
            const int pos = b + 64 * i + lane;
            v[i] = lidx[pos < we ? pos : we - 1];
        }
#pragma unroll
        for (int i = 0; i < kListLoads; ++i) {
            const int cc = v[i] - kw;
            if (b + 64 * i + lane < we && (unsigned)cc < (unsigned)kGroup) atomicOr(&lm[cc >> 5], 1u << (cc & 31));
        }
    }
}

// ---------------------------------------------------------------------------
// fused threshold + compact + sparse GEMV (one or two rows)
// ---------------------------------------------------------------------------
//
// Workgroup (half tile vt, segment seg) of W wavefronts owns the W groups
// seg * W .. seg * W + W - 1, and its wavefront w the 128 columns of group
// seg * W + w.  Every wavefront works on its own until the final sums, with
// no workgroup barrier:
//   1. it loads its 128 activations (two per lane and row), then its group's
//      scale/zero row for the half tile (16 bytes per lane);
//   2. thresholds them, ranks the active lanes with ballots and mbcnt, and
//      writes the active columns and their masked activations to its own
//      LDS rows;
//   3. splits its n active columns over the 8 slots, ceil(n / 16) column
//      pairs per lane, and issues all their 16-byte weight loads at once;
//   4. converts the scale/zero row, dequantizes and accumulates per lane (one
//      group: the scale is applied once per output), and sums the slots with
//      lane swaps.
// The workgroup then sums its wavefronts, and the segments of a half tile
// are added by the last workgroup to arrive (sp_finish).
//
// When the global list is asked for, one more workgroup (block 0) writes it
// with the gathering routine while the others compute; it reads only the
// activations.

constexpr int kFsCols = kGroup;                // columns per wavefront: one quantization group
constexpr int kFsW = 8;                          // wavefronts per workgroup (groups per segment)
constexpr int kFsWSmall = 4;                     // ... for one row on small matrices
// A workgroup of W wavefronts owns W groups (W * 128 columns) of a half
// tile.  W = 8 in general; small matrices take W = 4 (one row), twice the
// workgroups over the same columns, so that more CUs stream them.
template <int MT, int W>
struct FsShared {
    uint32_t zc[W][kVTile / 2];                  // per wavefront: (1024 + z, 1024 + 16 z) of output pairs
    __align__(16) float sc[W][kVTile];           // ... scale of output sp_out(l, d) at 4 l + d (1/16 folded in for odd)
    __align__(16) int k[W][kFsCols];             // ... its active columns
    __align__(16) uint16_t xs[W][MT][kFsCols];   // ... and their masked activations
    uint32_t lm[W][4];                           // ... over a given list: its listed columns
};

template <int MT, int W>
union FsLds {
    struct {
        FsShared<MT, W> f;
        SpShared<MT, W> sh;
    } g;
    GatherShared gl;
};

// Column pair (A, B) of one lane against its 8 outputs 8d .. 8d + 7:
// acc[m][r] += (q - z) x over the pair, exactly dequantized.
template <int MT>
__device__ __forceinline__ void fs_pair8(uint32_t Ad, uint32_t Bd, const uint32_t (&zc4)[4], const uint32_t (&xp)[MT],
                                         uint32_t vmagic, float (&acc)[MT][8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // byte i of the two columns into the low bytes of the two halves
        const uint32_t sel = (0x0Cu << 24) | ((uint32_t)i << 16) | (0x0Cu << 8) | (4u + i);
        const uint32_t R = __builtin_amdgcn_perm(Ad, Bd, sel);
        const half2_t z2 = as_h2(zc4[i]);   // (1024 + z, 1024 + 16 z) of outputs 2i, 2i + 1
        const half2_t lo = as_h2(and_or(R, 0x000F000Fu, vmagic)) - (half2_t){z2.x, z2.x};  // q - z
        const half2_t hi = as_h2(and_or(R, 0x00F000F0u, vmagic)) - (half2_t){z2.y, z2.y};  // 16 (q - z)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc[m][2 * i] = __builtin_amdgcn_fdot2(lo, as_h2(xp[m]), acc[m][2 * i], false);
            acc[m][2 * i + 1] = __builtin_amdgcn_fdot2(hi, as_h2(xp[m]), acc[m][2 * i + 1], false);
        }
    }
}

// The weights' arithmetic of a wavefront's NP column pairs per lane (their
// loads issued by the caller, x pairs in xp): converts the group's scale/zero
// row, dequantizes and accumulates pair by pair as the loads arrive, and
// returns in v4[m][d] the scaled sum of output sp_out(lane, d).
template <int MT, int NP, int W>
__device__ __forceinline__ void fs_compute(FsShared<MT, W>& fs, int wave, int lane, int blk, const u32x4 (&w)[2 * NP],
                                           const uint32_t (&xp)[NP][MT], const u32x4& mdv, uint32_t z4,
                                           float (&v4)[MT][4]) {
    {
        // the group row: lane l holds outputs 4l .. 4l + 3; zero codes as two
        // (even, odd) pairs, scales at the lane and sum that will own them
        // after the slot sums
        const u32x4 mw = md_cook4(mdv, z4);
        const half2_t s01 = as_h2(mw.x), s11 = as_h2(mw.y), s21 = as_h2(mw.z), s31 = as_h2(mw.w);
        const half2_t zp0 = (half2_t){(_Float16)(s01.y + (_Float16)1024.0f),
                                      (_Float16)(s11.y * (_Float16)16.0f + (_Float16)1024.0f)};
        const half2_t zp1 = (half2_t){(_Float16)(s21.y + (_Float16)1024.0f),
                                      (_Float16)(s31.y * (_Float16)16.0f + (_Float16)1024.0f)};
        *reinterpret_cast<uint2*>(&fs.zc[wave][2 * lane]) =
            make_uint2(__builtin_bit_cast(uint32_t, zp0), __builtin_bit_cast(uint32_t, zp1));
        const float sv[4] = {(float)s01.x, (float)s11.x * 0.0625f, (float)s21.x, (float)s31.x * 0.0625f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = 4 * lane + r;        // output o = 32 blk + 8 d + 4 b5 + 2 b4 + b3
            const int j = o & 7;
            const int L = (o >> 5) + 8 * (j & 1) + 16 * ((j >> 1) & 1) + 32 * (j >> 2);
            fs.sc[wave][4 * L + ((o >> 3) & 3)] = sv[r];
        }
        __builtin_amdgcn_wave_barrier();
    }
    // zero codes of the lane's 32 outputs, scales of its 4 final outputs
    uint32_t zc[16];
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(&fs.zc[wave][blk * (kLaneOut / 2)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 u = src[i];
            zc[4 * i] = u.x; zc[4 * i + 1] = u.y; zc[4 * i + 2] = u.z; zc[4 * i + 3] = u.w;
        }
    }
    const float4 s4 = *reinterpret_cast<const float4*>(&fs.sc[wave][4 * lane]);
    const float sc[4] = {s4.x, s4.y, s4.z, s4.w};
    const uint32_t vmagic = 0x64006400u | __builtin_amdgcn_mbcnt_lo(0u, 0u);  // per-lane (VGPR) copy
    if constexpr (MT == 1) {
        float acc[4][MT][8];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[d][0][r] = 0.f;
#pragma unroll
        for (int pr = 0; pr < NP; ++pr) {
            const u32x4 A = w[2 * pr], B = w[2 * pr + 1];
            const uint32_t Ad[4] = {A.x, A.y, A.z, A.w}, Bd[4] = {B.x, B.y, B.z, B.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t zc4[4] = {zc[4 * d], zc[4 * d + 1], zc[4 * d + 2], zc[4 * d + 3]};
                fs_pair8<MT>(Ad[d], Bd[d], zc4, xp[pr], vmagic, acc[d]);
            }
        }
        // slot sums, then the scale (one group per wavefront)
#pragma unroll
        for (int d = 0; d < 4; ++d) v4[0][d] = sc[d] * sp_reduce8(acc[d][0], lane);
    } else {  // two rows: 8 outputs at a time (register budget)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            float acc[MT][8];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[m][r] = 0.f;
            const uint32_t zc4[4] = {zc[4 * d], zc[4 * d + 1], zc[4 * d + 2], zc[4 * d + 3]};
#pragma unroll
            for (int pr = 0; pr < NP; ++pr) {
                const u32x4 A = w[2 * pr], B = w[2 * pr + 1];
                const uint32_t Ad = d == 0 ? A.x : d == 1 ? A.y : d == 2 ? A.z : A.w;
                const uint32_t Bd = d == 0 ? B.x : d == 1 ? B.y : d == 2 ? B.z : B.w;
                fs_pair8<MT>(Ad, Bd, zc4, xp[pr], vmagic, acc);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) v4[m][d] = sc[d] * sp_reduce8(acc[m], lane);
        }
    }
}

// A wavefront's nact active columns (nact <= 128, in its LDS rows) as NP
// column pairs per lane: slot c takes positions 2 NP c .. 2 NP c + 2 NP - 1
// (positions past nact repeat the first column with x = 0).  Issues the
// group's scale/zero row and all 16-byte weight loads, then accumulates pair
// by pair as they arrive, and returns in v4[m][d] the scaled sum of output
// sp_out(lane, d).
template <int MT, int NP, int W>
__device__ __forceinline__ void fs_block(FsShared<MT, W>& fs, int wave, int lane, int slot, int blk, int nact,
                                         int K, const uint8_t* __restrict__ wcol, const MdHalf& mdh, int g,
                                         float (&v4)[MT][4]) {
    const int kfirst = fs.k[wave][0];
    int kk[2 * NP];
    uint32_t xp[NP][MT];
    u32x4 w[2 * NP];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
        const int p = 2 * NP * slot + 2 * pr;          // even, below kFsCols: 8-byte aligned pairs
        const int2 k2 = *reinterpret_cast<const int2*>(&fs.k[wave][p]);
        const bool ok0 = p < nact, ok1 = p + 1 < nact;
        const int k0 = ok0 ? k2.x : kfirst, k1 = ok1 ? k2.y : kfirst;
        kk[2 * pr] = (unsigned)k0 < (unsigned)K ? k0 : K - 1;
        kk[2 * pr + 1] = (unsigned)k1 < (unsigned)K ? k1 : K - 1;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t x2 = *reinterpret_cast<const uint32_t*>(&fs.xs[wave][m][p]);
            xp[pr][m] = (ok0 ? (x2 & 0xFFFFu) : 0u) | (ok1 ? (x2 & 0xFFFF0000u) : 0u);
        }
    }
    // the scale/zero row just before the weights (loads complete in order,
    // and it is converted first); loading it here keeps it out of the
    // registers of the compaction
    const u32x4 mdv = md_raw4(mdh, g, 4 * lane);
#pragma unroll
    for (int j = 0; j < 2 * NP; ++j)
        w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wcol + (size_t)kk[j] * (2 * kHalfRun)) + blk);

    fs_compute<MT, NP, W>(fs, wave, lane, blk, w, xp, mdv, mdh.z4, v4);
}

// Every column of the wavefront's group (the dense GEMV): no thresholding
// pass and no compaction, so the activation pairs, the scale/zero row and all
// 16 weight loads per lane go out at once, in that order (loads complete in
// order).  Rows are masked by their thresholds unless the call is unmasked.
template <int MT, int W>
__device__ __forceinline__ void fs_dense(const RunArgs& a, FsShared<MT, W>& fs, int wave, int lane, int slot, int blk,
                                         int kw, const uint8_t* __restrict__ wcol, const MdHalf& mdh, int g,
                                         float (&v4)[MT][4]) {
    constexpr int NP = kFsCols / 16;        // 8 column pairs per lane
    const int k0 = kw + 2 * NP * slot;      // the lane's 16 consecutive columns
    uint32_t xp[NP][MT];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mr = m < a.M ? m : a.M - 1;
            xp[pr][m] = *reinterpret_cast<const uint32_t*>(a.x + (size_t)mr * a.ldx + k0 + 2 * pr);
        }
    const u32x4 mdv = md_raw4(mdh, g, 4 * lane);
    u32x4 w[2 * NP];
#pragma unroll
    for (int j = 0; j < 2 * NP; ++j)
        w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wcol + (size_t)(k0 + j) * (2 * kHalfRun)) + blk);
    if (!a.unmasked) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t code = code_of(a.tc, m < a.M ? m : a.M - 1);
#pragma unroll
            for (int pr = 0; pr < NP; ++pr) {
                const uint32_t v = xp[pr][m];
                xp[pr][m] = (is_active(v & 0xFFFFu, code) ? (v & 0xFFFFu) : 0u) |
                            (is_active(v >> 16, code) ? (v & 0xFFFF0000u) : 0u);
            }
        }
    }
    fs_compute<MT, NP, W>(fs, wave, lane, blk, w, xp, mdv, mdh.z4, v4);
}

// ---------------------------------------------------------------------------
// layout version 3: groups along the outputs
// ---------------------------------------------------------------------------
//
// One (s, z) per input column and 128 outputs; a half tile's two groups of
// column k are 8 bytes at md3[k] (md3 = the half tile's metadata row).  A
// wavefront loads the metadata of its listed positions lane and lane + 64
// (both loads unconditional: positions past the list re-read the first
// column), issued before its weight loads, and keeps it in the LDS rows that
// version 1's scales would use.  Lane (slot c, block o) then takes, for each
// column pair, the (s, z) of its outputs' group (o / 4): it folds the scales
// into the activations (s * x, rounded once to fp16) and subtracts
// 1024 + z (1024 + 16 z for high nibbles) from the magic-number codes, so
// q - z stays exact and each pair is one v_dot2 per output as in version 1;
// the 1/16 of the high nibbles is applied after the slot sums.

// Column pair (A, B) of one lane against its 8 outputs 8d .. 8d + 7, groups
// along the outputs: zl = (1024 + z_A, 1024 + z_B), zh = (1024 + 16 z_A,
// 1024 + 16 z_B), xq = the scaled activations of A and B.
template <int MT>
__device__ __forceinline__ void fs_pair8_ng(uint32_t Ad, uint32_t Bd, uint32_t zl, uint32_t zh, const uint32_t (&xq)[MT],
                                            uint32_t vmagic, float (&acc)[MT][8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t sel = (0x0Cu << 24) | ((uint32_t)i << 16) | (0x0Cu << 8) | (4u + i);
        const uint32_t R = __builtin_amdgcn_perm(Ad, Bd, sel);
        const half2_t lo = as_h2(and_or(R, 0x000F000Fu, vmagic)) - as_h2(zl);   // q - z
        const half2_t hi = as_h2(and_or(R, 0x00F000F0u, vmagic)) - as_h2(zh);   // 16 (q - z)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc[m][2 * i] = __builtin_amdgcn_fdot2(lo, as_h2(xq[m]), acc[m][2 * i], false);
            acc[m][2 * i + 1] = __builtin_amdgcn_fdot2(hi, as_h2(xq[m]), acc[m][2 * i + 1], false);
        }
    }
}

// The weights' arithmetic of NP column pairs per lane (pair pr at list
// position 2 NP slot + 2 pr), groups along the outputs; mdl holds the
// metadata of positions lane and lane + 64.
template <int MT, int NP, int W>
__device__ __forceinline__ void fs_compute_ng(FsShared<MT, W>& fs, int wave, int lane, int slot, int blk,
                                              const u32x4 (&w)[2 * NP], const uint32_t (&xp)[NP][MT],
                                              const uint2 (&mdl)[2], float (&v4)[MT][4]) {
    uint2* md3s = reinterpret_cast<uint2*>(&fs.sc[wave][0]);   // 128 positions
    md3s[lane] = mdl[0];
    md3s[lane + 64] = mdl[1];
    __builtin_amdgcn_wave_barrier();
    const bool second = blk >= 4;   // the lane's 32 outputs lie in the half tile's second group
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const half2_t k16 = {(_Float16)16.0f, (_Float16)16.0f};
    uint32_t zl[NP], zh[NP], xq[NP][MT];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
        const int p = 2 * NP * slot + 2 * pr;
        const uint2 ma = md3s[p], mb = md3s[p + 1];
        const uint32_t wa = second ? ma.y : ma.x, wb = second ? mb.y : mb.x;   // s bits | z bits << 16
        const half2_t s2 = as_h2((wa & 0xFFFFu) | (wb << 16));
        const half2_t z2 = as_h2((wa >> 16) | (wb & 0xFFFF0000u));
        zl[pr] = __builtin_bit_cast(uint32_t, z2 + k1024);
        zh[pr] = __builtin_bit_cast(uint32_t, z2 * k16 + k1024);
#pragma unroll
        for (int m = 0; m < MT; ++m) xq[pr][m] = __builtin_bit_cast(uint32_t, as_h2(xp[pr][m]) * s2);
    }
    const uint32_t vmagic = 0x64006400u | __builtin_amdgcn_mbcnt_lo(0u, 0u);  // per-lane (VGPR) copy
    // the lane's final outputs sp_out(lane, d) are odd (high nibbles) when lane bit 3 is set
    const float f = ((lane >> 3) & 1) ? 0.0625f : 1.0f;
    if constexpr (MT == 1) {
        float acc[4][MT][8];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[d][0][r] = 0.f;
#pragma unroll
        for (int pr = 0; pr < NP; ++pr) {
            const u32x4 A = w[2 * pr], B = w[2 * pr + 1];
            const uint32_t Ad[4] = {A.x, A.y, A.z, A.w}, Bd[4] = {B.x, B.y, B.z, B.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) fs_pair8_ng<MT>(Ad[d], Bd[d], zl[pr], zh[pr], xq[pr], vmagic, acc[d]);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) v4[0][d] = f * sp_reduce8(acc[d][0], lane);
    } else {  // two rows: 8 outputs at a time (register budget)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            float acc[MT][8];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[m][r] = 0.f;
#pragma unroll
            for (int pr = 0; pr < NP; ++pr) {
                const u32x4 A = w[2 * pr], B = w[2 * pr + 1];
                const uint32_t Ad = d == 0 ? A.x : d == 1 ? A.y : d == 2 ? A.z : A.w;
                const uint32_t Bd = d == 0 ? B.x : d == 1 ? B.y : d == 2 ? B.z : B.w;
                fs_pair8_ng<MT>(Ad, Bd, zl[pr], zh[pr], xq[pr], vmagic, acc);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) v4[m][d] = f * sp_reduce8(acc[m], lane);
        }
    }
}

// fs_block for groups along the outputs: the metadata of the listed
// positions, then the weights, then the arithmetic.
template <int MT, int NP, int W>
__device__ __forceinline__ void fs_block_ng(FsShared<MT, W>& fs, int wave, int lane, int slot, int blk, int nact,
                                            int K, const uint8_t* __restrict__ wcol, const uint2* __restrict__ md3,
                                            float (&v4)[MT][4]) {
    const int kfirst = fs.k[wave][0];
    int kk[2 * NP];
    uint32_t xp[NP][MT];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
        const int p = 2 * NP * slot + 2 * pr;          // even, below kFsCols: 8-byte aligned pairs
        const int2 k2 = *reinterpret_cast<const int2*>(&fs.k[wave][p]);
        const bool ok0 = p < nact, ok1 = p + 1 < nact;
        const int k0 = ok0 ? k2.x : kfirst, k1 = ok1 ? k2.y : kfirst;
        kk[2 * pr] = (unsigned)k0 < (unsigned)K ? k0 : K - 1;
        kk[2 * pr + 1] = (unsigned)k1 < (unsigned)K ? k1 : K - 1;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t x2 = *reinterpret_cast<const uint32_t*>(&fs.xs[wave][m][p]);
            xp[pr][m] = (ok0 ? (x2 & 0xFFFFu) : 0u) | (ok1 ? (x2 & 0xFFFF0000u) : 0u);
        }
    }
    uint2 mdl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int pos = lane + 64 * h;
        int k = pos < nact ? fs.k[wave][pos] : kfirst;
        k = (unsigned)k < (unsigned)K ? k : K - 1;
        mdl[h] = md3[k];
    }
    u32x4 w[2 * NP];
#pragma unroll
    for (int j = 0; j < 2 * NP; ++j)
        w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wcol + (size_t)kk[j] * (2 * kHalfRun)) + blk);
    fs_compute_ng<MT, NP, W>(fs, wave, lane, slot, blk, w, xp, mdl, v4);
}

// The dense path for groups along the outputs (every column of the group).
template <int MT, int W>
__device__ __forceinline__ void fs_dense_ng(const RunArgs& a, FsShared<MT, W>& fs, int wave, int lane, int slot,
                                            int blk, int kw, const uint8_t* __restrict__ wcol,
                                            const uint2* __restrict__ md3, float (&v4)[MT][4]) {
    constexpr int NP = kFsCols / 16;        // 8 column pairs per lane
    const int k0 = kw + 2 * NP * slot;      // the lane's 16 consecutive columns
    uint32_t xp[NP][MT];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mr = m < a.M ? m : a.M - 1;
            xp[pr][m] = *reinterpret_cast<const uint32_t*>(a.x + (size_t)mr * a.ldx + k0 + 2 * pr);
        }
    const uint2 mdl[2] = {md3[kw + lane], md3[kw + lane + 64]};
    u32x4 w[2 * NP];
#pragma unroll
    for (int j = 0; j < 2 * NP; ++j)
        w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wcol + (size_t)(k0 + j) * (2 * kHalfRun)) + blk);
    if (!a.unmasked) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t code = code_of(a.tc, m < a.M ? m : a.M - 1);
#pragma unroll
            for (int pr = 0; pr < NP; ++pr) {
                const uint32_t v = xp[pr][m];
                xp[pr][m] = (is_active(v & 0xFFFFu, code) ? (v & 0xFFFFu) : 0u) |
                            (is_active(v >> 16, code) ? (v & 0xFFFF0000u) : 0u);
            }
        }
    }
    fs_compute_ng<MT, NP, W>(fs, wave, lane, slot, blk, w, xp, mdl, v4);
}

template <int MT, int V, int W, bool LIST>
__device__ __forceinline__ void fs_body(const RunArgs& a, FsLds<MT, W>& lds) {
    int bid = blockIdx.x;
    if (a.idx_out) {  // block 0 writes the list
        if (bid == 0) {
            constexpr int WL = W >= 16 ? 16 : W >= 8 ? 8 : 4;
            gather_body<WL>(a.x, a.M, a.K, a.ldx, a.tc, a.idx_out, a.count_out, lds.gl);
            return;
        }
        --bid;
    }
    FsShared<MT, W>& fs = lds.g.f;

    const int T = a.tiles;
    const int vt = bid % T;
    const int seg = bid / T;
    const int S = a.segs;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 3, blk = lane & 7;
    const int K = a.K;
    const int kw = seg * (W * kFsCols) + wave * kFsCols;  // this wavefront's first column
    const bool has = kw < K;                       // K is a multiple of 128: all of the group or none
    const int g = (has ? kw : 0) / kGroup;

    const int tt = vt >> 1, hh = vt & 1;
    const uint8_t* __restrict__ wcol = a.w + (size_t)tt * K * (2 * kHalfRun) + hh * kHalfRun;
    const MdHalf mdh = md_half<V == SGEMV_LAYOUT_Z4>(a, tt, hh);
    const uint2* __restrict__ md3 = reinterpret_cast<const uint2*>(a.md) + (size_t)vt * K;   // version 3

    if (a.all_cols) {  // every column listed: the dense path
        float v4[MT][4] = {};
        if constexpr (V == SGEMV_LAYOUT_NG) {
            if (has) fs_dense_ng<MT, W>(a, fs, wave, lane, slot, blk, kw, wcol, md3, v4);
        } else if (has) {
            fs_dense<MT, W>(a, fs, wave, lane, slot, blk, kw, wcol, mdh, g, v4);
        }
        sp_finish<MT, W>(a, vt, seg, S, wave, lane, v4, lds.g.sh);
        return;
    }

    // 1. activations (two per lane and row; a wavefront past K reads its
    //    first columns and ignores them, so the loads are unconditional)
    constexpr int H = kFsCols / 64;
    uint32_t xr[H][MT];
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mr = m < a.M ? m : a.M - 1;
            xr[h][m] = a.x[(size_t)mr * a.ldx + (has ? kw : 0) + 64 * h + lane];
        }

    // 2. over a given list (a separate build), the group's listed columns
    //    (bit h of lb: column lane + 64 h); without one, every column may be
    //    active
    uint32_t lb = 3u;
    if constexpr (LIST) {
        const int lc = *a.lcount;   // issued after the activations, waited for with them
        if (lane < 4) fs.lm[wave][lane] = 0u;
        __builtin_amdgcn_wave_barrier();
        int c = __builtin_amdgcn_readfirstlane(lc);
        c = c < 0 ? 0 : (c > K ? K : c);
        if (has && c > 0) list_group_bits(a.lidx, c, kw, lane, fs.lm[wave]);
        __builtin_amdgcn_wave_barrier();
        lb = ((fs.lm[wave][lane >> 5] >> (lane & 31)) & 1u) | (((fs.lm[wave][2 + (lane >> 5)] >> (lane & 31)) & 1u) << 1);
    }

    // 3. threshold, rank, compact into this wavefront's LDS rows (no branch
    //    before the ballots: x is waited for on every path)
    bool act[H];
    uint32_t xm[H][MT];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        act[h] = false;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mr = m < a.M ? m : a.M - 1;
            const bool am = (a.unmasked || is_active(xr[h][m], code_of(a.tc, mr))) & has & ((lb >> h) & 1u);
            act[h] = act[h] | am;
            xm[h][m] = am ? xr[h][m] : 0u;
        }
    }
    int nact = 0;
    uint32_t rank[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const unsigned long long bal = __ballot(act[h]);
        rank[h] = nact + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        nact += __popcll(bal);
    }
    const int np = (nact + 15) / 16;
#pragma unroll
    for (int h = 0; h < H; ++h) {
        if (act[h]) {
            fs.k[wave][rank[h]] = kw + 64 * h + lane;
#pragma unroll
            for (int m = 0; m < MT; ++m) fs.xs[wave][m][rank[h]] = (uint16_t)xm[h][m];
        }
    }
    __builtin_amdgcn_wave_barrier();  // LDS operations of a wavefront complete in order

    // 4. np column pairs per lane (straight-line code per np, so that every
    //      pair waits only for its own loads)
    float v4[MT][4] = {};
    if constexpr (V == SGEMV_LAYOUT_NG) {
#define SG_NG(n) fs_block_ng<MT, n, W>(fs, wave, lane, slot, blk, nact, K, wcol, md3, v4)
        switch (np) {
            case 1: SG_NG(1); break;
            case 2: SG_NG(2); break;
            case 3: SG_NG(3); break;
            case 4: SG_NG(4); break;
            case 5: SG_NG(5); break;
            case 6: SG_NG(6); break;
            case 7: SG_NG(7); break;
            case 8: SG_NG(8); break;
            default: break;
        }
#undef SG_NG
        sp_finish<MT, W>(a, vt, seg, S, wave, lane, v4, lds.g.sh);
        return;
    }
    switch (np) {
        case 1: fs_block<MT, 1, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 2: fs_block<MT, 2, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 3: fs_block<MT, 3, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 4: fs_block<MT, 4, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 5: fs_block<MT, 5, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 6: fs_block<MT, 6, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 7: fs_block<MT, 7, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        case 8: fs_block<MT, 8, W>(fs, wave, lane, slot, blk, nact, K, wcol, mdh, g, v4); break;
        default: break;
    }
    sp_finish<MT, W>(a, vt, seg, S, wave, lane, v4, lds.g.sh);
}

// Two builds of the same kernel: two wavefronts per SIMD (the whole register
// budget, for grids of at most one workgroup per CU), and four (two
// workgroups per CU, so that one's loads overlap the other's latency in
// grids that take several rounds).
template <int MT, int V, int W, bool LIST>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_fs(RunArgs a) {
    __shared__ FsLds<MT, W> lds;
    fs_body<MT, V, W, LIST>(a, lds);
}

template <int MT, int V, bool LIST>
__global__ __launch_bounds__(kFsW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_fs4(RunArgs a) {
    __shared__ FsLds<MT, kFsW> lds;
    fs_body<MT, V, kFsW, LIST>(a, lds);
}

// ---------------------------------------------------------------------------
// fused threshold + union + sparse GEMV for 3 to 16 rows, on the matrix cores
// ---------------------------------------------------------------------------
//
// With many rows the work per weight is one multiply-add per row, a dense
// contraction over the listed columns, so it goes to v_mfma_f32_16x16x32_f16:
// the MFMA's rows are 16 outputs, its columns the (up to) 16 batch rows, its
// depth 32 listed columns.  Workgroup (half tile vt, segment seg) owns
// columns seg * 1024 .., its wavefront w the group seg * 8 + w, so every
// wavefront needs one scale per output.  A wavefront
//   1. loads its 128 activations of every row (lane: row lane / 4, 32
//      columns), thresholds them per row, ORs the masks over the rows (the
//      union), and compacts the union's columns; the rows' masked
//      activations are kept by column;
//   2. issues the 16-byte weight loads of all its chunks of 32 listed columns
//      (8 columns per load instruction, as in the one-row kernels);
//   3. per chunk: stores the raw weight bytes in LDS (32 columns x 128
//      bytes), and reads them back with the transposing ds_read_b64_tr_b8:
//      lane (depth quarter g = lane / 16, i = lane % 16) receives byte i of the
//      block of 16 bytes b of 8 consecutive listed columns, that is the low
//      nibbles of output 32 b + 2 i and the high nibbles of output 32 b + 2 i
//      + 1 for those columns - an A operand row for each.  It dequantizes
//      them exactly to fp16 in registers (q - z; 16 (q - z) for the high
//      nibbles) and runs two MFMAs per block;
//   4. scales each output once (1/16 folded in for high nibbles).
// The workgroup adds its wavefronts in a fixed order in LDS (every thread a
// slice of the sums); the segments of a half tile are added by the last
// workgroup to arrive, in segment order, with only the M rows in use stored.
//
// Storage order of the sums: index s = 32 b + 16 p + r holds output
// 32 b + 2 r + p (p = 0 for low nibbles, 1 for high).

namespace fm {
constexpr int kWaves = 8;
constexpr int kCols = kGroup;            // one group per wavefront
constexpr int kSeg = kWaves * kCols;     // columns per workgroup
constexpr int kRows = 16;                // batch rows (the MFMA's N), padded with zeros
constexpr int kCh = 32;                  // listed columns per MFMA step (its K)
constexpr int kMaxCh = kCols / kCh;
constexpr int kOutFloats = kRows * kVTile;   // one workgroup's sums
// LDS row strides, padded so that the 16-byte tile writes, the transposing
// reads and the row-wise accesses spread over the banks
constexpr int kRStride = kHalfRun + 16;   // bytes per staged weight column
constexpr int kXStride = kCols + 8;       // halves per activation row
}  // namespace fm

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef int i2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int fm_out_of(int s) {  // output of storage index s
    return (s & ~31) + 2 * (s & 15) + ((s >> 4) & 1);
}
__device__ __forceinline__ int fm_store_of(int n) {  // storage index of output n
    return (n & ~31) + 16 * (n & 1) + ((n & 31) >> 1);
}

struct FmWave {
    __align__(16) uint8_t r[fm::kCh][fm::kRStride];      // one chunk's raw weight bytes
    __align__(16) uint16_t xc[fm::kRows][fm::kXStride];  // masked activations by column
    __align__(16) int k[fm::kCols];                      // the wavefront's union columns
    __align__(16) uint32_t zc[kVTile / 2];               // per weight byte: (1024 + z, 1024 + 16 z)
    __align__(16) float sc[kVTile];                      // s (s / 16 for odd outputs), storage order
    uint32_t lm[4];                                      // a given list's columns of the group, as a mask
};

union FmLds {
    FmWave w[fm::kWaves];
    float red[fm::kWaves][fm::kOutFloats];               // every wavefront's sums
    GatherShared gl;
};


template <int V>
__global__ __launch_bounds__(fm::kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_fm(RunArgs a) {
    __shared__ FmLds lds;
    __shared__ uint32_t last_flag;
    int bid = blockIdx.x;
    if (a.idx_out) {  // blocks 0 .. gblocks - 1 write the list
        const int G = a.gblocks;
        if (bid < G) {
            if (G == 1) {
                gather_body<fm::kWaves>(a.x, a.M, a.K, a.ldx, a.tc, a.idx_out, a.count_out, lds.gl);
                return;
            }
            // list of columns k0 .. k0 + kr - 1 into the scratch at k0, and its length
            const int k0 = bid * a.grange;
            const int kr = a.K - k0 < a.grange ? a.K - k0 : a.grange;
            gather_body<fm::kWaves, true>(a.x + k0, a.M, kr, a.ldx, a.tc, a.gscratch + k0,
                                          reinterpret_cast<int32_t*>(a.gsync) + 16 + bid, lds.gl, k0);
            __builtin_amdgcn_s_waitcnt(0);  // this thread's stores acknowledged
            __syncthreads();                // ... and every thread's, before the count
            if (threadIdx.x == 0) {
                const uint32_t old = __hip_atomic_fetch_add(a.gsync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last_flag = (old == (uint32_t)(G - 1)) ? 1u : 0u;
            }
            __syncthreads();
            if (last_flag == 0u) return;
            // the last to arrive joins the lists in range order
            int len[8], pre[8], tot = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                len[j] = j < G ? __hip_atomic_load(reinterpret_cast<int32_t*>(a.gsync) + 16 + j, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0;
                pre[j] = tot;
                tot += len[j];
            }
            // thread t moves list positions t, t + 512, ..., 16 loads in flight
            constexpr int kT = fm::kWaves * 64;
            for (int p0 = threadIdx.x; p0 < tot; p0 += 16 * kT) {
                int v[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int p = p0 + i * kT;
                    int j = 0;
#pragma unroll
                    for (int r = 1; r < 8; ++r) j += (r < G && p >= pre[r]) ? 1 : 0;
                    const int src = j * a.grange + (p - pre[j]);
                    v[i] = p < tot ? __hip_atomic_load(a.gscratch + src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (p0 + i * kT < tot) a.idx_out[p0 + i * kT] = v[i];
            }
            if (threadIdx.x == 0) {
                *a.count_out = tot;
                __hip_atomic_store(a.gsync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            return;
        }
        bid -= G;
    }
    const int T = a.tiles;
    const int vt = bid % T;
    const int seg = bid / T;
    const int S = a.segs;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int K = a.K;
    const int kw = seg * fm::kSeg + wave * fm::kCols;
    const bool has = kw < K;                       // K is a multiple of 128: the whole group or none
    const int g = (has ? kw : 0) / kGroup;
    FmWave& fw = lds.w[wave];

    const int tt = vt >> 1, hh = vt & 1;
    const uint8_t* __restrict__ wcol = a.w + (size_t)tt * K * (2 * kHalfRun) + hh * kHalfRun;
    const MdHalf mdh = md_half<V == SGEMV_LAYOUT_Z4>(a, tt, hh);
    constexpr bool NG = V == SGEMV_LAYOUT_NG;   // groups along N: (s, z) per column and 128 outputs

    // 1. over a given list, its length (without a list the same load reads
    //    the activations and is unused, so that no path waits for it early);
    //    the activations: lane (row xm = lane / 4, quarter xq = lane % 4)
    //    loads 32 columns, rows past M read row M - 1 and are masked out; then
    //    the group's scale/zero row, which is converted after the weight loads
    //    are issued (loads complete in order: the activations are waited for
    //    without it, and it arrives before the weights)
    const int lc = *(a.lidx ? a.lcount : reinterpret_cast<const int32_t*>(a.x));
    const int xm = lane >> 2, xq = lane & 3;
    const int xmr = xm < a.M ? xm : a.M - 1;
    uint4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xv[i] = *reinterpret_cast<const uint4*>(a.x + (size_t)xmr * a.ldx + (has ? kw : 0) + 32 * xq + 8 * i);
    __builtin_amdgcn_sched_barrier(0);   // keeps the scale/zero load behind the activations'
    u32x4 mdv = {0u, 0u, 0u, 0u};
    if constexpr (!NG) mdv = md_raw4(mdh, g, 4 * lane);

    const uint32_t code = code_of(a.tc, xmr);
    const bool row_ok = has && xm < a.M;
    uint32_t am = 0;
    uint32_t xw[16];   // the lane's 32 activations, two per word
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xw[4 * i + e] = w4[e];
            am |= (uint32_t)is_active(w4[e] & 0xFFFFu, code) << (8 * i + 2 * e);
            am |= (uint32_t)is_active(w4[e] >> 16, code) << (8 * i + 2 * e + 1);
        }
    }
    if (a.unmasked) am = ~0u;
    am = row_ok ? am : 0u;
    // union over the 16 rows: lanes with the same quarter differ in lane bits
    // 2..5; rotations by 4 and 8 inside rows of 16 lanes, then the row swaps
    uint32_t un = am;
    un |= __builtin_amdgcn_update_dpp(0u, un, 0x124 /* row_ror:4 */, 0xF, 0xF, false);
    un |= __builtin_amdgcn_update_dpp(0u, un, 0x128 /* row_ror:8 */, 0xF, 0xF, false);
    {
        const auto r16 = __builtin_amdgcn_permlane16_swap(un, un, false, false);
        un = r16[0] | r16[1];
        const auto r32 = __builtin_amdgcn_permlane32_swap(un, un, false, false);
        un = r32[0] | r32[1];
    }
    if (a.all_cols) un = has ? ~0u : 0u;
    if (a.lidx) {  // a given list: the group's entries are the union (the rows stay masked by t)
        if (lane < 4) fw.lm[lane] = 0u;
        __builtin_amdgcn_wave_barrier();
        int c = __builtin_amdgcn_readfirstlane(lc);
        c = c < 0 ? 0 : (c > K ? K : c);
        if (has && c > 0) list_group_bits(a.lidx, c, kw, lane, fw.lm);
        __builtin_amdgcn_wave_barrier();
        un = fw.lm[lane & 3];  // word q at lane q, as the union above
    }
    uint32_t U[4], base[4];
    int nact = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        U[qq] = (uint32_t)__builtin_amdgcn_readlane((int)un, qq);
        base[qq] = (uint32_t)nact;
        nact += __popc(U[qq]);
    }
    const int nch = (nact + fm::kCh - 1) / fm::kCh;

    // 2a. the union's columns, two per lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 2 * lane + h;
        const uint32_t Uq = U[c >> 5];
        const uint32_t bit = 1u << (c & 31);
        if (Uq & bit) fw.k[base[c >> 5] + __popc(Uq & (bit - 1u))] = kw + c;
    }
    // 2b. the lane's row's activations by column, zero where inactive for the row
    {
        uint32_t mw[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t lo = ((am >> (2 * j)) & 1u) ? (xw[j] & 0xFFFFu) : 0u;
            const uint32_t hi = ((am >> (2 * j + 1)) & 1u) ? (xw[j] & 0xFFFF0000u) : 0u;
            mw[j] = lo | hi;
        }
        u32x4* dst = reinterpret_cast<u32x4*>(&fw.xc[xm][32 * xq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = (u32x4){mw[4 * i], mw[4 * i + 1], mw[4 * i + 2], mw[4 * i + 3]};
    }
    __builtin_amdgcn_wave_barrier();  // LDS operations of a wavefront complete in order

    // 3. chunks of 32 listed columns
    f4_t D[16];   // [2 b + p]: output block b (32 outputs), nibble p
#pragma unroll
    for (int b = 0; b < 16; ++b) D[b] = (f4_t){0.f, 0.f, 0.f, 0.f};
    if (nch > 0) {
        // loads: instruction i of chunk c, lane (lc = lane / 8, lo = lane % 8)
        // reads bytes 16 lo .. 16 lo + 15 of listed column c * 32 + 8 i + lc;
        // every chunk's loads are issued (positions past the list re-read the
        // first column), so that chunk c waits only for its own four
        const int lc = lane >> 3, lo = lane & 7;
        u32x4 wl[fm::kMaxCh][4];
        const int kfirst = fw.k[0];
        // groups along N: the 8-byte metadata of union positions lane and
        // lane + 64 (past the union: the first column), before the weights
        uint2 md3l[2] = {make_uint2(0u, 0u), make_uint2(0u, 0u)};
        if constexpr (NG) {
            const uint2* __restrict__ md3 = reinterpret_cast<const uint2*>(a.md) + (size_t)vt * K;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int pos = lane + 64 * h;
                int k = pos < nact ? fw.k[pos] : kfirst;
                k = (unsigned)k < (unsigned)K ? k : K - 1;
                md3l[h] = md3[k];
            }
        }
#pragma unroll
        for (int c = 0; c < fm::kMaxCh; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = c * fm::kCh + 8 * i + lc;
                int k = pos < nact ? fw.k[pos] : kfirst;
                k = (unsigned)k < (unsigned)K ? k : K - 1;
                wl[c][i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(wcol + (size_t)k * (2 * kHalfRun)) + lo);
            }
        // 3a. zero codes of the weight bytes 2 lane, 2 lane + 1 (outputs 4 lane ..
        //     4 lane + 3) and their scales in storage order (groups along N:
        //     the union's metadata by position, in the scales' rows)
        if constexpr (NG) {
            uint2* md3s = reinterpret_cast<uint2*>(&fw.sc[0]);
            md3s[lane] = md3l[0];
            md3s[lane + 64] = md3l[1];
        } else {
            const u32x4 mc = md_cook4(mdv, mdh.z4);
            const uint32_t mw[4] = {mc.x, mc.y, mc.z, mc.w};
            uint32_t zpair[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const half2_t se = as_h2(mw[2 * h]), so = as_h2(mw[2 * h + 1]);
                const half2_t zp = (half2_t){(_Float16)(se.y + (_Float16)1024.0f),
                                             (_Float16)(so.y * (_Float16)16.0f + (_Float16)1024.0f)};
                zpair[h] = __builtin_bit_cast(uint32_t, zp);
            }
            *reinterpret_cast<uint2*>(&fw.zc[2 * lane]) = make_uint2(zpair[0], zpair[1]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const half2_t sz = as_h2(mw[r]);
                fw.sc[fm_store_of(4 * lane + r)] = (r & 1) ? (float)sz.x * 0.0625f : (float)sz.x;
            }
        }
        __builtin_amdgcn_wave_barrier();
        const int g = lane >> 4, li = lane & 15;   // A/B operand: depth quarter, row
        // zero codes of the lane's A rows: weight byte 16 b + li, b = 0..7
        uint32_t zq[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) zq[b] = NG ? 0u : fw.zc[16 * b + li];
        // B operands of every chunk: activations of batch row li at positions
        // c * 32 + 8 g .. + 7 (all LDS reads issued together)
        uint32_t Bx[fm::kMaxCh][4];
        {
            int kc[fm::kMaxCh][8];
#pragma unroll
            for (int c = 0; c < fm::kMaxCh; ++c) {
                const int4 k0 = *reinterpret_cast<const int4*>(&fw.k[c * fm::kCh + 8 * g]);
                const int4 k1 = *reinterpret_cast<const int4*>(&fw.k[c * fm::kCh + 8 * g + 4]);
                const int kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) kc[c][j] = kv[j] - kw;
            }
#pragma unroll
            for (int c = 0; c < fm::kMaxCh; ++c) {
                uint32_t xv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int p = c * fm::kCh + 8 * g + j;
                    const int cc = (unsigned)kc[c][j] < (unsigned)fm::kCols ? kc[c][j] : 0;
                    const uint32_t v = fw.xc[li][cc];
                    xv[j] = p < nact ? v : 0u;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) Bx[c][j] = xv[2 * j] | (xv[2 * j + 1] << 16);
            }
        }
        const uint32_t vmagic = 0x64006400u | __builtin_amdgcn_mbcnt_lo(0u, 0u);  // per-lane (VGPR) copy
#pragma unroll
        for (int c = 0; c < fm::kMaxCh; ++c) {
            if (c < nch) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4*>(&fw.r[8 * i + lc][16 * lo]) = wl[c][i];
                __builtin_amdgcn_wave_barrier();
                // byte li of block b of columns 8 g .. 8 g + 7, transposed out of LDS
                i2_t rb[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    rb[b] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i2_t*)&fw.r[8 * g + (li >> 1)][16 * b + 8 * (li & 1)]);
                __builtin_amdgcn_sched_barrier(0);  // keep the 8 reads ahead of the products
                h8_t B = __builtin_bit_cast(h8_t, (u32x4){Bx[c][0], Bx[c][1], Bx[c][2], Bx[c][3]});
                // groups along N: per group e of the half tile (output blocks
                // 4 e .. 4 e + 3), the activations scaled by their columns'
                // s (B operand) and the columns' zero codes by pair
                h8_t Bg[2] = {B, B};
                uint32_t zlg[2][4] = {}, zhg[2][4] = {};
                if constexpr (NG) {
                    const u32x4* mp = reinterpret_cast<const u32x4*>(&fw.sc[0]) + (c * fm::kCh + 8 * g) / 2;
                    uint32_t mwv[8][2];   // position 8 g + j: (s | z << 16) of groups 0 and 1
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u32x4 m4 = mp[i];
                        mwv[2 * i][0] = m4.x; mwv[2 * i][1] = m4.y;
                        mwv[2 * i + 1][0] = m4.z; mwv[2 * i + 1][1] = m4.w;
                    }
                    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
                    const half2_t k16 = {(_Float16)16.0f, (_Float16)16.0f};
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        uint32_t bw[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t wa = mwv[2 * j][e], wb = mwv[2 * j + 1][e];
                            const half2_t s2 = as_h2((wa & 0xFFFFu) | (wb << 16));
                            const half2_t z2 = as_h2((wa >> 16) | (wb & 0xFFFF0000u));
                            zlg[e][j] = __builtin_bit_cast(uint32_t, z2 + k1024);
                            zhg[e][j] = __builtin_bit_cast(uint32_t, z2 * k16 + k1024);
                            bw[j] = __builtin_bit_cast(uint32_t, as_h2(Bx[c][j]) * s2);
                        }
                        Bg[e] = __builtin_bit_cast(h8_t, (u32x4){bw[0], bw[1], bw[2], bw[3]});
                    }
                }
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const half2_t z2 = as_h2(zq[b]);
                    if constexpr (NG) B = Bg[b >> 2];
                    const uint32_t dw2[2] = {(uint32_t)rb[b].x, (uint32_t)rb[b].y};
                    uint32_t ae[4], ao[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // bytes 2 (j % 2), 2 (j % 2) + 1 of the dword into the low bytes of the halves
                        const uint32_t Dd = dw2[j >> 1];
                        const uint32_t b0 = 2 * (j & 1);
                        const uint32_t P = __builtin_amdgcn_perm(Dd, Dd, (0x0Cu << 24) | ((b0 + 1) << 16) | (0x0Cu << 8) | b0);
                        const half2_t zl = NG ? as_h2(zlg[b >> 2][j]) : (half2_t){z2.x, z2.x};
                        const half2_t zh = NG ? as_h2(zhg[b >> 2][j]) : (half2_t){z2.y, z2.y};
                        const half2_t e = as_h2(and_or(P, 0x000F000Fu, vmagic)) - zl;  // q - z
                        const half2_t o = as_h2(and_or(P, 0x00F000F0u, vmagic)) - zh;  // 16 (q - z)
                        ae[j] = __builtin_bit_cast(uint32_t, e);
                        ao[j] = __builtin_bit_cast(uint32_t, o);
                    }
                    D[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(h8_t, (u32x4){ae[0], ae[1], ae[2], ae[3]}), B, D[2 * b], 0, 0, 0);
                    D[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(h8_t, (u32x4){ao[0], ao[1], ao[2], ao[3]}), B, D[2 * b + 1], 0, 0, 0);
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
        // 4. one scale per output: D[2 b + p] row 4 g + e is storage index
        //    32 b + 16 p + 4 g + e (groups along N: the scales are in B; the
        //    high nibbles' 1/16 is left)
        if constexpr (NG) {
#pragma unroll
            for (int b = 0; b < 8; ++b) D[2 * b + 1] *= 0.0625f;
        } else {
#pragma unroll
            for (int bp = 0; bp < 16; ++bp) {
                const float4 s4 = *reinterpret_cast<const float4*>(&fw.sc[16 * bp + 4 * g]);
                D[bp].x *= s4.x; D[bp].y *= s4.y; D[bp].z *= s4.z; D[bp].w *= s4.w;
            }
        }
    }

    // 5. every wavefront's sums to LDS (lane-major: 16 bytes per lane and
    //    D block); thread t adds entries 8 t .. 8 t + 7 over the wavefronts in
    //    order: batch rows m0 = 2 t % 16 and m0 + 1, storage indices s0 .. s0 + 3
    __syncthreads();   // every wavefront is done with its own LDS rows
#pragma unroll
    for (int b = 0; b < 16; ++b)
        *reinterpret_cast<f4_t*>(&lds.red[wave][(64 * b + lane) * 4]) = D[b];
    __syncthreads();
    const int t = threadIdx.x;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < fm::kWaves; ++w) {
        const float4 u0 = *reinterpret_cast<const float4*>(&lds.red[w][8 * t]);
        const float4 u1 = *reinterpret_cast<const float4*>(&lds.red[w][8 * t + 4]);
        v[0] += u0.x; v[1] += u0.y; v[2] += u0.z; v[3] += u0.w;
        v[4] += u1.x; v[5] += u1.y; v[6] += u1.z; v[7] += u1.w;
    }
    const int l2 = (2 * t) & 63;
    const int m0 = l2 & 15;
    const int s0 = 16 * (t >> 5) + 4 * (l2 >> 4);
    auto put_y = [&](int m, int s, float val) {
        const size_t n = (size_t)vt * kVTile + fm_out_of(s);
        if (a.out_f32) static_cast<float*>(a.y)[(size_t)m * a.ldy + n] = val;
        else static_cast<_Float16*>(a.y)[(size_t)m * a.ldy + n] = (_Float16)val;
    };
    if (S == 1) {  // one segment: these are the outputs
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (m0 < a.M) put_y(m0, s0 + j, v[j]);
            if (m0 + 1 < a.M) put_y(m0 + 1, s0 + j, v[4 + j]);
        }
        return;
    }

    // 6. several segments: the workgroup's sums of the M rows go to slot seg
    //    of the half tile ([row][storage index], device-coherent stores); the
    //    last workgroup to count adds the slots in segment order
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(a.partials, (short)0, (int)a.partial_bytes, 0x00020000);
    const uint32_t slot_bytes = (uint32_t)a.M * kVTile * 4u;
    const uint32_t tile_base = (uint32_t)vt * a.slices * slot_bytes;
    const uint32_t mine = tile_base + (uint32_t)seg * slot_bytes;
    if (m0 < a.M)
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])}, prs,
                                               mine + ((uint32_t)m0 * kVTile + s0) * 4u, 0, kCacheSC1);
    if (m0 + 1 < a.M)
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7])}, prs,
                                               mine + ((uint32_t)(m0 + 1) * kVTile + s0) * 4u, 0, kCacheSC1);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores acknowledged
    __syncthreads();                // ... and every thread's, before the count
    if (t == 0) {
        last_flag = count_arrival(a.counters, vt, S);
    }
    __syncthreads();
    if (last_flag == 0u) return;
    if (last_flag == 1u) acquire_slices();

    // last to arrive: a slot's M x 256 sums are M KiB; thread t adds its
    // 16-byte pieces t and t + 512 (row c / 64, storage 4 (c % 64) .. + 3 for
    // piece c) of every slot, in segment order, 16 slots in flight (past the
    // CU's L1).  Each load instruction reads 1 KiB of a slot contiguously,
    // so no line is fetched from L2 twice.
    const int np = a.M * (kVTile / 4);   // pieces per slot
    const int c1 = t, c2 = t + fm::kWaves * 64;
    const bool h1 = c1 < np, h2 = c2 < np;
    float tot1[4] = {0.f, 0.f, 0.f, 0.f}, tot2[4] = {0.f, 0.f, 0.f, 0.f};
    if (h1) {
        for (int sb = 0; sb < S; sb += 16) {
            u32x4 u[16][2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int sl = sb + i < S ? sb + i : sb;
                const uint32_t off = tile_base + (uint32_t)sl * slot_bytes;
                u[i][0] = __builtin_amdgcn_raw_buffer_load_b128(prs, off + (uint32_t)c1 * 16u, 0, kCacheSC0);
                u[i][1] = h2 ? __builtin_amdgcn_raw_buffer_load_b128(prs, off + (uint32_t)c2 * 16u, 0, kCacheSC0)
                             : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (sb + i < S) {
                    tot1[0] += u2f(u[i][0].x); tot1[1] += u2f(u[i][0].y); tot1[2] += u2f(u[i][0].z); tot1[3] += u2f(u[i][0].w);
                    tot2[0] += u2f(u[i][1].x); tot2[1] += u2f(u[i][1].y); tot2[2] += u2f(u[i][1].z); tot2[3] += u2f(u[i][1].w);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) put_y(c1 / 64, 4 * (c1 % 64) + j, tot1[j]);
        if (h2) {
#pragma unroll
            for (int j = 0; j < 4; ++j) put_y(c2 / 64, 4 * (c2 % 64) + j, tot2[j]);
        }
    }
    if (t == 0) reset_arrivals(a.counters, vt);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

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
    if (d->version != SGEMV_LAYOUT_PAIRS && d->version != SGEMV_LAYOUT_Z4 && d->version != SGEMV_LAYOUT_NG)
        return SGEMV_EINVAL;
    sgemv_layout_fill_desc(d->N, d->K, d->tile_n, d->version, &ref);
    if (d->w_off != ref.w_off || d->w_bytes != ref.w_bytes || d->m_off != ref.m_off ||
        d->m_bytes != ref.m_bytes || d->total_bytes != ref.total_bytes)
        return SGEMV_EINVAL;
    if (d->tile_n != kTileN) return SGEMV_EUNSUPPORTED;
    return SGEMV_OK;
}

// Each arrival counter sits on its own 256-byte line, so the atomics of
// different half tiles go to different cache lines (and L2 channels).
size_t ws_counters_bytes(int tiles) { return (size_t)tiles * kCounterStride * 4; }

// The many-row fused call's list workgroups: a 256-byte line (their arrival
// counter and list lengths), then a K-entry scratch list.
size_t ws_gather_bytes(const sgemv_desc* d) { return 256 + ((size_t)d->K * 4 + 255) / 256 * 256; }

// Workspace: counters, the list workgroups' region, then the partial sums
// (whose size depends on the largest batch).
size_t ws_head_bytes(const sgemv_desc* d) { return ws_counters_bytes(d->N / kVTile) + ws_gather_bytes(d); }

// Partial sums of a call with M rows: M x 256 fp32 sums per half tile and
// segment (one or two rows: at most one segment per 512 columns, the
// smallest workgroup's; 3 to 16 rows: one per 1024 columns).
size_t ws_fused_bytes(const sgemv_desc* d, int M) {
    const int tiles = d->N / kVTile;
    const int seg_cols = M <= 2 ? kFsWSmall * kFsCols : fm::kSeg;
    const int segs = (d->K + seg_cols - 1) / seg_cols;
    return segs > 1 ? (size_t)tiles * segs * M * kVTile * sizeof(float) : 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Fused one/two-row kernel: grids of at most this many workgroups run in one
// round (one per CU) with the two-wavefronts-per-SIMD build.
constexpr int kFsOneRound = 256;
// One row: below this many 8-wavefront workgroups, 4-wavefront workgroups
// (twice as many, at most two per CU: still one round).  At decode sizes a
// workgroup's stream is bound by how many loads one CU keeps in flight, so a
// small matrix is read faster by more CUs; near one full round the extra
// partial sums cost more than that gains.
constexpr int kFsSmallGrid = 160;
// One row, grids of several rounds: 4-wavefront workgroups (up to four per
// CU) also when a half tile has at most this many of their segments; the
// smaller workgroups overlap each other's chains better (70B gate, 16
// segments: 7 % faster at 50 %), until the last workgroup's read of the
// partial sums grows too long (70B down, 56 segments: slower).
constexpr int kFsSmallMaxSegs = 32;

// Argument checks of the fused call (no HIP call); `no_thr_ok` when the
// call may go without thresholds (every column, or a given list).
int check_fused_args(const sgemv_desc* d, const void* packed, const void* x, int M, int ldx, const float* thr,
                     const int32_t* idx, const int32_t* count, const void* y, int ldy, uint32_t flags,
                     bool no_thr_ok) {
    int st = check_desc(d);
    if (st) return st;
    if (!packed || !x || !y || (!thr && !no_thr_ok)) return SGEMV_EINVAL;
    if ((idx == nullptr) != (count == nullptr)) return SGEMV_EINVAL;
    if (flags & ~SGEMV_OUT_F32) return SGEMV_EINVAL;
    if (M < 1 || M > SGEMV_MAX_BATCH) return SGEMV_ESIZE;
    if (ldx < d->K || ldy < d->N) return SGEMV_ESIZE;
    if (ldx % 8 || ldy % 8) return SGEMV_EALIGN;
    if (!aligned(packed, 256) || !aligned(x, 16) || !aligned(y, 16)) return SGEMV_EALIGN;
    if (idx && (!aligned(idx, 4) || !aligned(count, 4))) return SGEMV_EALIGN;
    if (thr) {
        Codes c;
        st = fill_codes(thr, M, c);
        if (st) return st;
    }
    return SGEMV_OK;
}

// Where a call's scratch regions are: the arrival counters (zero between
// calls), the many-row list workgroups' line and list (its first word zero
// between calls), and the partial sums (any contents), with room for
// partial_cap bytes.
struct WsRegions {
    uint32_t* counters;
    uint32_t* gsync;
    int32_t* gscratch;
    float* partials;
    size_t partial_cap;
};

// The regions inside a caller's workspace for matrix d and M rows (the
// layout sgemv_workspace_bytes sizes).
WsRegions ws_regions(void* ws, const sgemv_desc* d, int M) {
    if (!ws) return WsRegions{nullptr, nullptr, nullptr, nullptr, 0};
    uint8_t* b = static_cast<uint8_t*>(ws);
    const size_t c = ws_counters_bytes(d->N / kVTile);
    return WsRegions{reinterpret_cast<uint32_t*>(b), reinterpret_cast<uint32_t*>(b + c),
                     reinterpret_cast<int32_t*>(b + c + 256), reinterpret_cast<float*>(b + ws_head_bytes(d)),
                     ws_fused_bytes(d, M)};
}

int run_fused(const sgemv_desc* d, const void* packed, const void* x, int M, int ldx, const float* thr,
              int32_t* idx, int32_t* count, void* y, int ldy, uint32_t flags, const WsRegions* ws, void* stream,
              bool all_cols = false, const int32_t* lidx = nullptr, const int32_t* lcount = nullptr);

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
    if (ws && !aligned(ws, 256)) return SGEMV_EALIGN;
    const WsRegions r = ws_regions(ws, d, M);
    if (!idx)   // every column: the fused kernels with the whole list, which stream faster
        return run_fused(d, packed, x, M, ldx, thr, nullptr, nullptr, y, ldy, flags, ws ? &r : nullptr, stream, true);
    // over a given list the fused kernels read the list themselves
    return run_fused(d, packed, x, M, ldx, thr, nullptr, nullptr, y, ldy, flags, ws ? &r : nullptr, stream, false,
                     idx, count);

}

// The fused kernels; with all_cols every column is listed (the dense GEMV,
// rows masked by their thresholds unless thr is NULL).
template <int V, bool LIST>
void launch_fs(int M, int W, bool one_round, dim3 grid, const RunArgs& a, hipStream_t s) {
    if (M == 1 && W == kFsWSmall) hipLaunchKernelGGL((k_fs<1, V, kFsWSmall, LIST>), grid, dim3(kFsWSmall * 64), 0, s, a);
    else if (M == 1 && one_round) hipLaunchKernelGGL((k_fs<1, V, kFsW, LIST>), grid, dim3(kFsW * 64), 0, s, a);
    else if (M == 1) hipLaunchKernelGGL((k_fs4<1, V, LIST>), grid, dim3(kFsW * 64), 0, s, a);
    else if (one_round) hipLaunchKernelGGL((k_fs<2, V, kFsW, LIST>), grid, dim3(kFsW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_fs4<2, V, LIST>), grid, dim3(kFsW * 64), 0, s, a);
}

template <int V>
void launch_fused(int M, int W, bool one_round, dim3 grid, const RunArgs& a, hipStream_t s) {
    if (M > 2) {
        hipLaunchKernelGGL(k_fm<V>, grid, dim3(fm::kWaves * 64), 0, s, a);
        return;
    }
    if (a.lidx) launch_fs<V, true>(M, W, one_round, grid, a, s);
    else launch_fs<V, false>(M, W, one_round, grid, a, s);
}

int run_fused(const sgemv_desc* d, const void* packed, const void* x, int M, int ldx, const float* thr,
              int32_t* idx, int32_t* count, void* y, int ldy, uint32_t flags, const WsRegions* ws, void* stream,
              bool all_cols, const int32_t* lidx, const int32_t* lcount) {
    int st = check_fused_args(d, packed, x, M, ldx, thr, idx, count, y, ldy, flags, all_cols || lidx);
    if (st) return st;

    RunArgs a;
    std::memset(&a, 0, sizeof a);
    if (thr) {
        st = fill_codes(thr, M, a.tc);
        if (st) return st;
    }
    a.all_cols = all_cols ? 1u : 0u;
    if (lidx) {   // list mode (many rows)
        a.lidx = lidx;
        a.lcount = lcount;
    }
    a.unmasked = thr ? 0u : 1u;
    a.tiles = d->N / kVTile;
    int W = kFsW;
    if (M <= 2) {
        const int segs8 = (d->K + kFsW * kFsCols - 1) / (kFsW * kFsCols);
        const int segs4 = (d->K + kFsWSmall * kFsCols - 1) / (kFsWSmall * kFsCols);
        if (M == 1 && (a.tiles * segs8 < kFsSmallGrid ||
                       (a.tiles * segs8 > kFsOneRound && segs4 <= kFsSmallMaxSegs)))
            W = kFsWSmall;
        a.segs = (d->K + W * kFsCols - 1) / (W * kFsCols);
    } else {
        a.segs = (d->K + fm::kSeg - 1) / fm::kSeg;
    }
    a.slices = a.segs;   // stride of the partial sums
    if (a.segs > 1) {
        if (!ws) return SGEMV_EINVAL;
        // the kernels address the partial sums with 32-bit buffer offsets
        if (ws_fused_bytes(d, M) > 0xFFFFFFFFull || ws_fused_bytes(d, M) > ws->partial_cap) return SGEMV_ESIZE;
    }
    const uint8_t* blob = static_cast<const uint8_t*>(packed);
    a.w = blob + d->w_off;
    a.md = blob + d->m_off;
    a.md_z4 = d->version == SGEMV_LAYOUT_Z4 ? 1u : 0u;
    a.x = static_cast<const uint16_t*>(x);
    a.y = y;
    a.idx_out = idx;
    a.count_out = count;
    if (ws) {
        a.counters = ws->counters;
        a.partials = ws->partials;
        a.gsync = ws->gsync;
        a.gscratch = ws->gscratch;
    }
    // list workgroups of the many-row kernel: about 64 KiB of activations each, at most 8
    a.gblocks = idx ? 1 : 0;
    if (idx && M > 2 && ws) {
        long g = ((long)M * d->K * 2 + 65535) / 65536;
        g = g < 1 ? 1 : (g > 8 ? 8 : g);
        a.grange = (int)((d->K / kGroup + g - 1) / g) * kGroup;
        a.gblocks = (d->K + a.grange - 1) / a.grange;
    }
    a.partial_bytes = (uint32_t)ws_fused_bytes(d, M);
    a.K = d->K;
    a.ldx = ldx;
    a.ldy = ldy;
    a.M = M;
    a.out_f32 = (flags & SGEMV_OUT_F32) ? 1u : 0u;
    const dim3 grid((unsigned)(a.tiles * a.segs + a.gblocks));  // + the list's workgroups
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool one_round = a.tiles * a.segs <= kFsOneRound;
    if (d->version == SGEMV_LAYOUT_NG) launch_fused<SGEMV_LAYOUT_NG>(M, W, one_round, grid, a, s);
    else if (a.md_z4) launch_fused<SGEMV_LAYOUT_Z4>(M, W, one_round, grid, a, s);
    else launch_fused<SGEMV_LAYOUT_PAIRS>(M, W, one_round, grid, a, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SGEMV_EHIP;
    }
    return SGEMV_OK;
}

}  // namespace

extern "C" int sgemv_run_fused(const sgemv_desc* d, const void* packed, const void* x_f16, int32_t M,
                               int32_t ldx, const float* thresholds, int32_t* idx, int32_t* count,
                               void* y, int32_t ldy, uint32_t flags, void* workspace, void* stream) {
    if (check_desc(d)) return check_desc(d);
    if (workspace && !aligned(workspace, 256)) return SGEMV_EALIGN;
    if (M < 1 || M > SGEMV_MAX_BATCH) return SGEMV_ESIZE;
    const WsRegions r = ws_regions(workspace, d, M);
    return run_fused(d, packed, x_f16, M, ldx, thresholds, idx, count, y, ldy, flags, workspace ? &r : nullptr,
                     stream);
}

// Rows x columns up to which the gathering uses 512-thread workgroups.
constexpr long kGatherSmall = 2L * 16384;

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
    // 4096 columns per workgroup of 512 threads; with many rows (every
    // workgroup rereads all earlier rows and columns) 8192 per workgroup of
    // 1024, which halves the rereading
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xp = static_cast<const uint16_t*>(x_f16);
    if ((long)M * K <= kGatherSmall)
        hipLaunchKernelGGL(k_gather<8>, dim3((K + 4095) / 4096), dim3(512), 0, s, xp, (int)M, (int)K, (int)ldx, c,
                           idx, count);
    else
        hipLaunchKernelGGL(k_gather<16>, dim3((K + 8191) / 8192), dim3(1024), 0, s, xp, (int)M, (int)K, (int)ldx,
                           c, idx, count);
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
    size_t part = 0;  // enough for every call with up to M rows
    for (int m = 1; m <= M; ++m) {
        const size_t b = ws_fused_bytes(d, m);
        part = b > part ? b : part;
    }
    return ws_head_bytes(d) + part;
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

// ---------------------------------------------------------------------------
// the fused call without a workspace argument
// ---------------------------------------------------------------------------
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it): the scratch regions live in
// one fixed-size device array per GPU, here called `scratch`, with a fixed
// layout, so that calls on matrices of any shape that fits can follow each
// other: the arrival counters of up to kScratchTiles half tiles, the many-row
// list workgroups' line and list for up to SGEMV_MAX_K columns, then the
// partial sums.  Its device address is taken once per GPU with
// hipGetSymbolAddress (host code never passes the array's name itself to a
// kernel); the first call on a GPU also clears the counters and the line on
// the caller's stream.  Every call leaves them at zero again, as with a
// workspace.  Calls that overlap on one GPU share the array and race.
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kScratchTiles = 1024;   // half tiles: N up to 262144
constexpr size_t kScratchCounters = (size_t)kScratchTiles * kCounterStride * 4;
constexpr size_t kScratchGather = 256 + (size_t)SGEMV_MAX_K * 4;
constexpr size_t kScratchHead = kScratchCounters + kScratchGather;
static_assert(kScratchHead % 256 == 0, "the partial sums start on a 256-byte boundary");

__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ p, uint32_t n) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_addr[kMaxDevices];

// The address of this GPU's `scratch` (device of the stream), taken with the
// device current; `fresh` when it has not been kept yet (the caller keeps it
// with keep_scratch once the array is cleared).
int scratch_of(hipStream_t s, uint8_t** out, bool* fresh, int* device) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SGEMV_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return SGEMV_EUNSUPPORTED;
    *device = dev;
    uint8_t* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    *fresh = false;
    if (!p) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* q = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !q) {
            g_last_hip_error = (int)e;
            return SGEMV_EHIP;
        }
        p = static_cast<uint8_t*>(q);
        *fresh = true;
    }
    *out = p;
    return SGEMV_OK;
}

}  // namespace

extern "C" int sgemv_run_fused_static(const sgemv_desc* d, const void* packed, const void* x_f16, int32_t M,
                                      int32_t ldx, const float* thresholds, int32_t* idx, int32_t* count,
                                      void* y, int32_t ldy, uint32_t flags, void* stream) {
    int st = check_fused_args(d, packed, x_f16, M, ldx, thresholds, idx, count, y, ldy, flags, false);
    if (st) return st;
    if (d->N / kVTile > kScratchTiles || ws_fused_bytes(d, M) > kScratchBytes - kScratchHead) return SGEMV_ESIZE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* p = nullptr;
    bool fresh = false;
    int dev = 0;
    st = scratch_of(s, &p, &fresh, &dev);
    if (st) return st;
    if (fresh) {   // counters and the list workgroups' line start at zero
        const uint32_t n = (uint32_t)((kScratchCounters + 256) / 4);
        hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, s, reinterpret_cast<uint32_t*>(p), n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return SGEMV_EHIP;
        }
        g_scratch_addr[dev].store(p, std::memory_order_release);   // cleared: kept for later calls
    }
    const WsRegions r{reinterpret_cast<uint32_t*>(p), reinterpret_cast<uint32_t*>(p + kScratchCounters),
                      reinterpret_cast<int32_t*>(p + kScratchCounters + 256), reinterpret_cast<float*>(p + kScratchHead),
                      kScratchBytes - kScratchHead};
    return run_fused(d, packed, x_f16, M, ldx, thresholds, idx, count, y, ldy, flags, &r, s);
}
