/*
 * sgemv.h - C ABI of the dynamically sparse int4 GEMV for MI355X (gfx950).
 *
 * The operation ("Enabling Dynamic Sparsity in Quantized LLM Inference",
 * Abstract): during decode the activation vector x is dynamically sparse;
 * entries with small magnitude are dropped, and only the weight columns that
 * match the surviving indices are read, from a group-wise low-bit quantized
 * weight matrix stored in a layout that keeps those reads local.  The page
 * names three parts - a sparsity-consistent quantized weight layout, a GEMV
 * kernel for it, and a run-time step that gathers the active indices - and
 * this library provides one call for each, plus the batched variant:
 *
 *   sgemv_pack_layout     host: int4 codes + fp16 scale/zero -> packed blob
 *                         (sgemv_pack_layout_z4: the same with 4-bit zeros;
 *                         sgemv_pack_layout_ng: groups along the outputs)
 *   sgemv_gather_indices  device: threshold x, emit the ascending list of
 *                         active indices and its length
 *   sgemv_run             device: y = W . x over the listed columns (M = 1)
 *   sgemv_run_batched     device: M <= 16 rows over the union list, each row
 *                         masked by its own threshold
 *   sgemv_run_fused       device: threshold, union, compact and GEMV in one
 *                         launch (M <= 16), the list optional
 *
 * Weights.  W is [N][K] (output x input, like a Linear weight), quantized
 * asymmetrically to 4 bits with one fp16 scale s and one fp16 zero-point z
 * per output row n and group g of 128 consecutive inputs (k / 128):
 *   w^[n][k] = s[n][k/128] * (q[n][k] - z[n][k/128]),  q in 0..15,
 * z an integer 0..15 stored as fp16 (the GPTQ-style format that the page
 * cites; the page itself fixes no format, so this is our reading).
 *
 * Selection.  Entry k of row m is active iff float32(|x[m][k]|) >= t[m]:
 * ties are kept, NaN is never active, -0 and +0 are active when t == 0.  The
 * page does not state the rule; magnitude thresholding with a calibrated
 * per-call scalar follows "Training-Free Activation Sparsity in Large
 * Language Models", which the page builds on.
 *
 * Conventions for every call.
 *   - Every pointer marked "device" is device memory; "host" is host memory.
 *     The caller owns all buffers; the library allocates nothing and keeps
 *     no state between calls except a thread-local last HIP error.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it asynchronously; the host never waits.
 *   - Arguments are validated before any HIP call.  On a bad argument the
 *     call returns a negative status and enqueues nothing.  A failed launch
 *     returns SGEMV_EHIP (details: sgemv_last_hip_error).  Faults while a
 *     kernel runs surface at the caller's next synchronisation.
 *   - Nothing is printed, nothing throws across the ABI.
 *   - Calls are re-entrant; calls that share a workspace must not run
 *     concurrently on different streams.
 */
#ifndef SGEMV_H
#define SGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Description of one packed matrix; produced by sgemv_pack_layout or
 * sgemv_desc_from_header, read by the device calls (host memory). */
typedef struct sgemv_desc {
    int32_t  N;            /* outputs (rows of W)                          */
    int32_t  K;            /* inputs (columns of W), multiple of 128       */
    int32_t  group;        /* quantization group along K, always 128       */
    int32_t  tile_n;       /* outputs per tile of the layout               */
    uint64_t w_off;        /* byte offset of the weight region (= 256)     */
    uint64_t w_bytes;      /* N*K/2                                        */
    uint64_t m_off;        /* byte offset of the scale/zero region         */
    uint64_t m_bytes;      /* (K/128)*N*4, or (K/128)*N*5/2 for version 2  */
    uint64_t total_bytes;  /* size of the whole blob                       */
    uint32_t version;      /* SGEMV_LAYOUT_PAIRS, _Z4 or _NG               */
    uint32_t reserved;     /* 0                                            */
} sgemv_desc;

enum sgemv_status {
    SGEMV_OK           = 0,
    SGEMV_EINVAL       = -1,  /* NULL pointer, bad value, bad flag          */
    SGEMV_ESIZE        = -2,  /* a size out of range or capacity too small  */
    SGEMV_EALIGN       = -3,  /* pointer or leading dimension misaligned    */
    SGEMV_EUNSUPPORTED = -4,  /* valid layout the kernels do not implement  */
    SGEMV_EHIP         = -5   /* a HIP call failed                          */
};

#define SGEMV_GROUP       128
#define SGEMV_MAX_BATCH   16
#define SGEMV_MAX_K       65536
#define SGEMV_MAX_N       (1 << 20)
#define SGEMV_TILE_N      512   /* the tile width the device kernels run   */
#define SGEMV_OUT_F32     1u    /* flag: y is fp32 instead of fp16         */
#define SGEMV_LAYOUT_PAIRS 1u   /* layout version 1: (s, z) fp16 pairs     */
#define SGEMV_LAYOUT_Z4    2u   /* layout version 2: fp16 s, 4-bit z       */
#define SGEMV_LAYOUT_NG    3u   /* layout version 3: groups along N        */

/*
 * sgemv_pack_layout - re-lay int4 weights so that each active input index
 * maps to contiguous bytes (host only, no HIP call).
 *
 * Realises the sparsity-aware weight layout asked for by the page's
 * Abstract (weights arranged to match activation sparsity, for memory
 * locality on the GPU); the page does not give its pattern, so the pattern
 * is ours:
 *
 *   blob = header (256 B) | weights | scale/zero metadata, little-endian
 *   header 0: "SGV1", 4: u32 version 1, 8: i32 N, 12: i32 K, 16: i32 group,
 *          20: i32 tile_n, 24: u64 w_off, 32: u64 w_bytes, 40: u64 m_off,
 *          48: u64 m_bytes, 56: u64 total_bytes, 64..255 zero
 *   w_off = 256; m_off = w_off + roundup(w_bytes, 256);
 *   total = m_off + roundup(m_bytes, 256)
 *   weight byte  w_off + (t*K + k)*(tile_n/2) + j
 *                = q[t*tile_n + 2j][k] | q[t*tile_n + 2j + 1][k] << 4
 *   metadata     m_off + ((t*(K/128) + g)*tile_n + i)*4 = s bits, z bits of
 *                row t*tile_n + i, group g (two little-endian u16)
 *
 * So for every tile of tile_n outputs, one input index k is one contiguous
 * run of tile_n/2 bytes (256 B for tile_n = 512), and one group's scales
 * and zeros are one contiguous run of tile_n*4 bytes.
 *
 *   q          host uint8 [N][K], row-major, values 0..15
 *   scales_f16 host uint16 [N][K/128], fp16 bit patterns of finite values
 *   zeros_f16  host uint16 [N][K/128], fp16 bit patterns of integers 0..15
 *   group      must be 128
 *   tile_n     power of two in [64, 1024] dividing N (the device calls run
 *              tile_n = SGEMV_TILE_N only)
 *   out        host buffer of out_capacity bytes, or NULL for a size query
 *   desc_out   receives the description (may be NULL when out == NULL)
 * Returns SGEMV_OK; EINVAL for NULL inputs, a code > 15, a bad scale or
 * zero-point, group != 128; ESIZE for bad N/K/tile_n or out_capacity <
 * total_bytes.  The blob is self-describing and may be saved and reloaded.
 */
int sgemv_pack_layout(const uint8_t* q, const uint16_t* scales_f16,
                      const uint16_t* zeros_f16, int32_t N, int32_t K,
                      int32_t group, int32_t tile_n, void* out,
                      size_t out_capacity, sgemv_desc* desc_out);

/*
 * sgemv_pack_layout_z4 - the same layout with compact metadata (version 2).
 *
 * The weight region is byte for byte that of sgemv_pack_layout.  The
 * zero-points are integers 0..15, so they take 4 bits: the run of one
 * (tile, group) pair holds the tile_n fp16 scales, then tile_n/2 bytes of
 * zero-points, two per byte.  Same numbers, 2.5 instead of 4 bytes per row
 * and group: this carries the page's sparsity-consistent layout (Abstract)
 * to the metadata, which every touched group still reads in full.
 *
 *   header as above with version 2 and m_bytes = (K/128)*N*5/2
 *   scale       m_off + (t*(K/128) + g)*(5*tile_n/2) + 2i : fp16 bits of
 *               s[t*tile_n + i][g] (little-endian u16)
 *   zero-points m_off + (t*(K/128) + g)*(5*tile_n/2) + 2*tile_n + j
 *               = z[t*tile_n + 2j][g] | z[t*tile_n + 2j + 1][g] << 4
 *
 * Arguments, ownership and errors as for sgemv_pack_layout.  Every device
 * call takes either version (desc->version) and computes bit for bit the
 * same y from both.
 */
int sgemv_pack_layout_z4(const uint8_t* q, const uint16_t* scales_f16,
                         const uint16_t* zeros_f16, int32_t N, int32_t K,
                         int32_t group, int32_t tile_n, void* out,
                         size_t out_capacity, sgemv_desc* desc_out);

/*
 * sgemv_pack_layout_ng - layout version 3, for weights quantized with their
 * groups along the outputs: one fp16 scale s and one integer zero-point z
 * per input column k and group b of 128 consecutive outputs,
 *   w^[n][k] = s[n/128][k] * (q[n][k] - z[n/128][k]).
 * The page asks for a quantization layout consistent with activation
 * sparsity (Abstract); with groups along the outputs a column's scale and
 * zero-point belong to that column alone, so they are read only when the
 * column is active and the metadata bytes fall with the sparsity, as the
 * weight bytes do.
 *
 *   header as above with version 3; m_bytes = (N/128)*K*4
 *   weight bytes exactly those of sgemv_pack_layout
 *   metadata     m_off + ((h*K + k)*2 + e)*4 : fp16 bits of s[2h + e][k],
 *                then fp16 bits of z[2h + e][k]  (h < N/256, e in {0, 1}):
 *                per 256 outputs and column, 8 contiguous bytes
 *
 *   q          host uint8 [N][K], row-major, values 0..15
 *   scales_f16 host uint16 [N/128][K], fp16 bit patterns of finite values
 *   zeros_f16  host uint16 [N/128][K], fp16 bit patterns of integers 0..15
 *   tile_n     power of two in [256, 1024] dividing N
 * Other arguments, ownership and errors as for sgemv_pack_layout (ESIZE
 * also for tile_n < 256).  Every device call takes this version.  The
 * kernels fold each column's scale into its activation (s * x rounded once
 * to fp16) and subtract the zero-point exactly, so y differs from the exact
 * product by at most 2^-11 * sum_k |w^[n][k]| |x[k]| plus fp32 accumulation
 * before the final rounding of y (versions 1 and 2: fp32 accumulation
 * error only).
 */
int sgemv_pack_layout_ng(const uint8_t* q, const uint16_t* scales_f16,
                         const uint16_t* zeros_f16, int32_t N, int32_t K,
                         int32_t group, int32_t tile_n, void* out,
                         size_t out_capacity, sgemv_desc* desc_out);

/*
 * sgemv_pack_layout_parts - one blob for several projections that read the
 * same activations (the query, key and value projections of an attention
 * block; the gate and up projections of a gated feed-forward block), their
 * rows stacked along N in the order given, so that one device call
 * thresholds x once and computes all of them.  The blob is exactly the one
 * sgemv_pack_layout (version SGEMV_LAYOUT_PAIRS), sgemv_pack_layout_z4
 * (SGEMV_LAYOUT_Z4) or sgemv_pack_layout_ng (SGEMV_LAYOUT_NG) writes for the
 * row-concatenated matrix; projection p's
 * outputs are y[off_p .. off_p + n_part[p]) with off_p the sum of the
 * earlier n_part.  Host only, no HIP call.
 *
 *   parts      number of projections, >= 1
 *   q          host array of `parts` pointers, part p: uint8 [n_part[p]][K]
 *   scales_f16 host array of `parts` pointers, part p: uint16 [n_part[p]][K/128]
 *              ([n_part[p]/128][K] for SGEMV_LAYOUT_NG)
 *   zeros_f16  likewise for the zero-points
 *   n_part     host int32 [parts]: rows of each part, each a multiple of
 *              tile_n (no tile mixes two projections)
 *   K, group, tile_n, out, out_capacity, desc_out as for sgemv_pack_layout
 *   version    SGEMV_LAYOUT_PAIRS, SGEMV_LAYOUT_Z4 or SGEMV_LAYOUT_NG
 * Returns SGEMV_OK; EINVAL for parts < 1, NULL arrays or parts, a bad code,
 * scale or zero-point, a bad version; ESIZE for a part that is not whole
 * tiles, a total N out of range, or too small a capacity.  With out == NULL
 * it is a size query (q, scales and zeros may then be NULL).
 */
int sgemv_pack_layout_parts(int32_t parts, const uint8_t* const* q,
                            const uint16_t* const* scales_f16,
                            const uint16_t* const* zeros_f16, const int32_t* n_part,
                            int32_t K, int32_t group, int32_t tile_n, uint32_t version,
                            void* out, size_t out_capacity, sgemv_desc* desc_out);

/* Parse and check the 64-byte header of a blob held in host memory (for a
 * blob that was saved and reloaded; version 1, 2 or 3).  EINVAL on a bad magic,
 * version or inconsistent offsets. */
int sgemv_desc_from_header(const void* header, size_t bytes, sgemv_desc* desc_out);

/*
 * sgemv_gather_indices - the run-time step of the page's Abstract that
 * collects the indices of the surviving activations at low cost: threshold
 * every row, OR the rows' masks, and compact the union into an ascending
 * list.  A few workgroups (one per 4096 columns, or per 8192 with more
 * rows), each over its own column range; every workgroup counts the active
 * columns below its range straight from x, so they need no scratch memory
 * and no communication; wavefront ballots and bit counts give each lane its
 * rank, an LDS scan orders the wavefronts.
 *
 *   x_f16      device fp16 [M][ldx]; 16-byte aligned
 *   M          rows, 1..SGEMV_MAX_BATCH
 *   K          columns, multiple of 128, <= SGEMV_MAX_K
 *   ldx        row stride in elements, >= K, multiple of 8
 *   thresholds host float [M], each finite and >= 0
 *   idx        device int32 [K]: receives the active indices ascending in
 *              idx[0 .. count); entries beyond count are left untouched
 *   count      device int32 [1]: receives the number of active indices
 * Deterministic: the list is unique for given inputs.
 */
int sgemv_gather_indices(const void* x_f16, int32_t M, int32_t K, int32_t ldx,
                         const float* thresholds, int32_t* idx, int32_t* count,
                         void* stream);

/*
 * sgemv_run - y = W . x over the listed columns (the page's specialised
 * GEMV for the sparse layout, Abstract):
 *   y[n] = sum over j < *count of w^[n][idx[j]] * x[idx[j]]
 * accumulated in fp32 (products exact, per-lane partial sums, fixed-order
 * tree across lanes, wavefronts and workgroups), rounded once to fp16 with
 * round-to-nearest-even (or stored as fp32 with SGEMV_OUT_F32).  x is used
 * unmasked at the listed indices.  With idx == NULL every column is used
 * (the dense int4 GEMV) and count is ignored.  count == 0 gives y = +0.
 * The result is bitwise reproducible for given inputs.
 *
 *   d          host description of the packed matrix (tile_n = 512)
 *   packed     device blob from sgemv_pack_layout, 256-byte aligned
 *   x_f16      device fp16 [K], 16-byte aligned
 *   idx        device int32 buffer of K entries, 4-byte aligned, whose
 *              first *count entries are ascending, unique and < K (as
 *              produced by sgemv_gather_indices); or NULL for all columns.
 *              Entries beyond *count may hold anything.
 *   count      device int32 [1], 0 <= *count <= K (clamped to that range)
 *   y          device fp16 [N] (fp32 with SGEMV_OUT_F32), 16-byte aligned
 *   flags      0 or SGEMV_OUT_F32
 *   workspace  device, sgemv_workspace_bytes(d, 1) bytes, 256-byte
 *              aligned, zero-filled once by the caller.  It holds one
 *              arrival counter per 256 outputs, which every call returns to
 *              zero, then scratch (lists, sums) that needs no clearing, at
 *              offsets that depend on N: so it can be reused by any later
 *              call on the same stream for a matrix with the same N (sized
 *              for the largest K and row count among them).  A workspace
 *              that has served one N must be zero-filled again before it
 *              serves another.  May be NULL when the call has a single
 *              column segment (K up to 512 for one or two rows, 1024 for
 *              more); the call returns SGEMV_EINVAL when it needs one.
 */
int sgemv_run(const sgemv_desc* d, const void* packed, const void* x_f16,
              const int32_t* idx, const int32_t* count, void* y,
              uint32_t flags, void* workspace, void* stream);

/*
 * sgemv_run_batched - M rows against one matrix over the union list
 * (batched contextual sparsity as in "Polar Sparsity: High Throughput
 * Batched LLM Inferencing with Scalable Contextual Sparsity", which the
 * page builds on: the batch reads the union of its rows' active columns
 * once):
 *   y[m][n] = sum over j < *count of w^[n][idx[j]] * xe[m][idx[j]],
 *   xe[m][k] = x[m][k] if float32(|x[m][k]|) >= thresholds[m], else 0
 * With thresholds == NULL every row uses x unmasked at every listed index.
 * With idx == NULL every column is listed.
 *
 *   x_f16 device fp16 [M][ldx], 16-byte aligned, ldx >= K, ldx % 8 == 0
 *   y     device fp16/fp32 [M][ldy], 16-byte aligned, ldy >= N, ldy % 8 == 0
 *   workspace: sgemv_workspace_bytes(d, M) bytes, same contract as above.
 * Other arguments as in sgemv_run.  SGEMV_ESIZE when the call's partial
 * sums would exceed 4 GiB - 1 (half tiles x segments x M x 1 KiB; only
 * near the largest N, K and M), which the kernels address with 32-bit
 * offsets.
 */
int sgemv_run_batched(const sgemv_desc* d, const void* packed,
                      const void* x_f16, int32_t M, int32_t ldx,
                      const float* thresholds, const int32_t* idx,
                      const int32_t* count, void* y, int32_t ldy,
                      uint32_t flags, void* workspace, void* stream);

/*
 * sgemv_run_fused - the gathering step and the GEMV in one launch, so that
 * no kernel boundary and no round trip through a global list separate the
 * thresholding from the weight reads (the page's Abstract asks for index
 * gathering with minimal overhead).  Each wavefront thresholds one
 * 128-column group of every row, compacts the columns active in any row in
 * LDS and reads only their weight bytes; the workgroups of the column
 * segments (512 or 1024 columns) are summed as in sgemv_run.
 *   y[m][n] = sum over active k of w^[n][k] * xe[m][k]
 * with xe and the union of active columns as in sgemv_run_batched (with
 * thresholds), which it equals within the same error bound (the order of
 * the fp32 additions differs, so the bits may differ).
 *
 *   M          1..SGEMV_MAX_BATCH.  One or two rows run on the vector
 *              units; 3 to 16 rows run on the matrix cores
 *              (v_mfma_f32_16x16x32_f16 over exactly dequantized fp16
 *              q - z, fp32 accumulation), each row masked by its own
 *              threshold over the union of the rows' active columns
 *   thresholds host float [M], each finite and >= 0 (required)
 *   idx, count both NULL, or both device int32 ([K] and [1], 4-byte
 *              aligned): then they receive exactly what
 *              sgemv_gather_indices writes for the same x and thresholds
 *   workspace  sgemv_workspace_bytes(d, M) bytes, same contract as above
 * Other arguments as in sgemv_run_batched.  Bitwise reproducible.
 */
int sgemv_run_fused(const sgemv_desc* d, const void* packed, const void* x_f16,
                    int32_t M, int32_t ldx, const float* thresholds,
                    int32_t* idx, int32_t* count, void* y, int32_t ldy,
                    uint32_t flags, void* workspace, void* stream);

/*
 * sgemv_run_fused_static - sgemv_run_fused without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation).  The scratch
 * (arrival counters, the list workgroups' line and list, partial sums) is a
 * fixed 16 MiB device array inside the library, one per GPU, held until the
 * process ends; its address is taken once per GPU (on the first call there,
 * which also clears its counters on `stream`); nothing is allocated.
 *   - Sizes beyond the array: N above 262144 (1024 half tiles), or partial
 *     sums above its 15.5 MiB (half tiles x segments x M x 1 KiB; segments
 *     of 512 columns for one or two rows, 1024 for more) return
 *     SGEMV_ESIZE before any HIP call.  Every configuration of 8192- to
 *     28672-wide Llama-3 projections with up to 16 rows fits.
 *   - Every call on a GPU shares that GPU's array and leaves its counters
 *     at zero again; calls that overlap on one GPU (other streams, other host
 *     threads) race and must not be made.
 * Other arguments, results and errors as for sgemv_run_fused, which it
 * equals bit for bit.
 */
int sgemv_run_fused_static(const sgemv_desc* d, const void* packed, const void* x_f16,
                           int32_t M, int32_t ldx, const float* thresholds,
                           int32_t* idx, int32_t* count, void* y, int32_t ldy,
                           uint32_t flags, void* stream);

/* Bytes of workspace needed by sgemv_run (M = 1), sgemv_run_batched or
 * sgemv_run_fused with up to M rows on matrix d; 0 for an invalid
 * description. */
size_t sgemv_workspace_bytes(const sgemv_desc* d, int32_t M);

/* Static string for a status code. */
const char* sgemv_strerror(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int sgemv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMV_H */
