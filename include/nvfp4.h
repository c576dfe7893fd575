/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled GEMM library.
 *
 * The operation is C = alpha * (A . B^T):
 *   - A is M x K and B is N x K, both held as FP4 E2M1 codes packed two per
 *     byte, with one FP8 E4M3 scale per 16-element block along K ("Peeling
 *     the Kernel Onion", section "The Benchmark Design": packed uint8 data,
 *     an FP8 scale for every 16 elements; "The SM120 FP4 Kernel
 *     Disaster", section "Input Knowledge Required", item 3);
 *   - alpha is an FP32 scalar and C is a caller-provided M x N bfloat16
 *     output ("Peeling the Kernel Onion", section "The Chain of Reasoning":
 *     the GEMM takes alpha and an output tensor);
 *   - K must be a positive multiple of the 16-element block size (and so of
 *     the packing factor 2): "The SM120 FP4 Kernel Disaster", section "The
 *     Bash Command".
 *
 * Element formats (OCP Microscaling Formats v1.0): E2M1 codes are
 * sign(bit 3) | exponent(bits 2:1, bias 1) | mantissa(bit 0), values
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; E4M3 scales are the "FN" variant (bias 7,
 * subnormals, 0x7F/0xFF NaN, no infinity, max 448).
 *
 * Canonical layout (what callers produce; row-major, K contiguous):
 *   codes  [rows][K/2]  byte j of a row holds element 2j in bits 3:0 and
 *                       element 2j+1 in bits 7:4;
 *   scales [rows][K/16] byte b scales elements 16b .. 16b+15.
 * Packed layout (what nvfp4_gemm consumes; produced by nvfp4_pack): rows are
 * padded to Rp = roundup(rows, 16) and K to Kp = roundup(K, 128) with zero
 * codes and zero scales; the data is split into Kp/64 panels of 64 elements:
 *   packed codes  [Kp/64][Rp][32]  (32 bytes = 64 codes of one row, same
 *                                   byte/nibble order as canonical)
 *   packed scales [Kp/64][Rp][4]   (the row's four scale bytes of the panel)
 * Padding contributes exact zeros, so results are unaffected.
 *
 * Status codes: every entry point returns an nvfp4_status (0 = success) and
 * never aborts, throws or prints.  Argument errors are detected on the host
 * before any device work is enqueued.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_VALUE = 1, /* bad size, null pointer, K % 16 != 0, ... */
    NVFP4_ERR_MISALIGNED = 2,    /* a device pointer is not 16-byte aligned */
    NVFP4_ERR_UNSUPPORTED = 3,   /* no gfx950 device / forced path cannot run */
    NVFP4_ERR_HIP = 4,           /* a HIP runtime call failed */
    NVFP4_ERR_ALLOC = 5,         /* workspace allocation failed */
    NVFP4_ERR_CAPTURE = 6,       /* a split-K workspace would have to be created or
                                    grown while the stream is being captured */
    NVFP4_ERR_STATE = 7,         /* call not allowed in the object's current state */
    NVFP4_ERR_DEVICE_FLAGS = 8,  /* nvfp4_device_flags: a kernel raised an error flag */
    NVFP4_ERR_SCRATCH = 9        /* nvfp4_gemm_noalloc: the shape's plan needs more
                                    split-K scratch than the static maximum */
} nvfp4_status;

/* Device error flags (nvfp4_device_flags). */
enum {
    /* a two-way split-K hand-off ran out of polls waiting for its partner's
     * partial tile: that output tile was left unwritten */
    NVFP4_FLAG_HANDOFF = 1
};

/* Kernel paths for nvfp4_gemm_with_plan and nvfp4_plan. */
enum {
    NVFP4_PATH_AUTO = 0,   /* library's choice from M, N, K */
    NVFP4_PATH_TILE = 1,   /* large shapes: MFMA tiles fed through an LDS ring */
    NVFP4_PATH_SKINNY = 2, /* M <= 64: decode shapes, waves share a column group's K range */
    NVFP4_PATH_WSPLIT = 3, /* mid-size shapes: the waves of a workgroup split K */
    NVFP4_PATH_GEMV = 4    /* M <= 4: one wave per column of C, dot products */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int nvfp4_version(void);

/* Byte sizes of the packed code and scale buffers for an operand of `rows`
 * rows and K elements per row (see "Packed layout" above).
 * rows >= 1, K >= 16, K % 16 == 0, else NVFP4_ERR_INVALID_VALUE.  Output
 * pointers must be non-null. */
int nvfp4_packed_size(int64_t rows, int64_t K, size_t* code_bytes, size_t* scale_bytes);

/* Host-side layout transform, canonical -> packed (a pure byte permutation
 * plus zero padding; no arithmetic).  All pointers are HOST memory owned by
 * the caller; packed buffers must hold nvfp4_packed_size() bytes.  Used for
 * both A (rows = M) and B (rows = N).  Same size rules as nvfp4_packed_size. */
int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
               uint8_t* packed_codes, uint8_t* packed_scales);

/* Inverse of nvfp4_pack (drops the padding). HOST memory, caller-owned. */
int nvfp4_unpack(const uint8_t* packed_codes, const uint8_t* packed_scales, int64_t rows,
                 int64_t K, uint8_t* codes, uint8_t* scales);

/* Optional set-up for `device`: checks that it is a gfx950 GPU and creates
 * the split-K workspace of the calling stream lazily afterwards.  nvfp4_gemm
 * calls it implicitly for the current device.  Returns NVFP4_ERR_UNSUPPORTED
 * for a non-gfx950 device, NVFP4_ERR_HIP if the device cannot be queried. */
int nvfp4_init(int device);

/* Frees every workspace the library allocated, including buffers retired
 * when a workspace grew.  The caller must make sure no nvfp4 kernel is still
 * running and that no graph captured from nvfp4 calls will be replayed
 * again; later calls re-create what they need. */
void nvfp4_shutdown(void);

/* Sticky error flags raised by the library's kernels on the current device
 * (NVFP4_FLAG_* bits).  Synchronises the device, stores the flags in *flags,
 * clears them, and returns NVFP4_ERR_DEVICE_FLAGS if any was set (the
 * results of the calls since the last check may then be incomplete), else
 * NVFP4_OK.  The only flag is NVFP4_FLAG_HANDOFF; a kernel that raises it
 * still finishes normally and leaves the split-K counters ready for the next
 * call.  "The SM120 FP4 Kernel Disaster", section "Finding 2": a GEMM that
 * silently returns a wrong result is the failure to guard against. */
int nvfp4_device_flags(uint32_t* flags);

/* Test hook: the number of polls (each about 128 clock cycles) a two-way
 * split-K hand-off waits for its partner before it gives up; applies to the
 * calls planned afterwards (a recorded sequence keeps the value of its
 * add).  0 makes every such wait give up at once; 0xFFFFFFFF restores the
 * default (2^22).  Always NVFP4_OK. */
int nvfp4_debug_set_handoff_polls(uint32_t polls);

/* C = alpha * (A . B^T), bfloat16 output, round-to-nearest-even.
 *   a_packed, a_scales : DEVICE pointers, A packed by nvfp4_pack (rows = M)
 *   b_packed, b_scales : DEVICE pointers, B packed by nvfp4_pack (rows = N)
 *   alpha              : FP32 scale applied once to the FP32 accumulator
 *   out                : DEVICE pointer, M x N bfloat16, row-major (ld = N);
 *                        overwritten (no beta); must not alias the inputs
 *   M, N, K            : logical sizes (M, N >= 1; K >= 16, K % 16 == 0)
 *   stream             : hipStream_t to enqueue on (NULL = default stream)
 * All device buffers are caller-owned and must be 16-byte aligned (else
 * NVFP4_ERR_MISALIGNED).  The call is asynchronous: it returns after the
 * kernels are enqueued; device-side faults surface at the caller's next
 * synchronisation.  The tile and wsplit paths need each packed code buffer
 * to stay below 2 GiB (else NVFP4_ERR_UNSUPPORTED).  Split-K paths use a
 * library-owned workspace per
 * (device, stream) pair, allocated (and zero-filled on that stream, ahead of
 * the call's kernels) on the first call that needs it and again, larger, on
 * the first call of a shape that needs more; these are the only allocations
 * the library makes.  Calls on one stream are ordered, calls on different
 * streams use different workspaces.  Buffers replaced by larger ones stay
 * allocated until nvfp4_shutdown, so a graph captured earlier keeps working.
 * Under stream capture the workspace must already be large enough (make one
 * call of the same shape on that stream first), else NVFP4_ERR_CAPTURE.  A
 * captured call keeps the workspace of the stream it was captured on,
 * wherever the graph is replayed: do not let a replay overlap other calls
 * on that stream or other replays of graphs captured on it (order them, for
 * instance by replaying on the capture stream).  Launch failures return
 * NVFP4_ERR_HIP. */
int nvfp4_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
               const void* b_scales, float alpha, void* out, int64_t M, int64_t N, int64_t K,
               void* stream);

/* nvfp4_gemm with a forced launch plan, for tuning and tests:
 *   path    : NVFP4_PATH_* (NVFP4_PATH_AUTO = library's choice, then tile
 *             must be 0)
 *   tile    : 0 = library's choice; else the workgroup's output tile:
 *             its edge for NVFP4_PATH_TILE (256, 128 or 64: square tiles);
 *             rows x columns / 64 for NVFP4_PATH_WSPLIT (16 = 32 x 32,
 *             32 = 64 x 32, 64 = 64 x 64, 128 = 128 x 64; rows of C x
 *             columns of C); must be 0 for the skinny and gemv paths (fixed
 *             tiles)
 *   split_k : 0 = library's choice, else the number of K slices, clamped to
 *             the number of 128-element K steps
 * Same contract as nvfp4_gemm.  A bad path or tile is NVFP4_ERR_INVALID_VALUE;
 * NVFP4_ERR_UNSUPPORTED if the forced path cannot run the shape (skinny needs
 * M <= 64, gemv M <= 4).  Every plan gives the same result up to the order of
 * the FP32 additions (see nvfp4_gemm); a given plan is deterministic. */
int nvfp4_gemm_with_plan(const void* a_packed, const void* a_scales, const void* b_packed,
                         const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                         int64_t K, int path, int tile, int split_k, void* stream);

/* NVFP4 quantisation of fp32 rows straight into the packed layout (the step
 * before the GEMM for activations; "Peeling the Kernel Onion", section "The
 * Benchmark Design", for the format).  Per 16-element block of a row:
 *   scale = E4M3 value nearest to fp32(amax / 6), ties to the even byte,
 *           saturating at 448;
 *   code  = E2M1 magnitude nearest to fp32(x / scale), ties to the even code,
 *           saturating at 6, with the sign bit of x (a block whose scale is 0
 *           keeps only the sign bits).
 *   x             : DEVICE fp32, rows x K values, row stride ld elements
 *                   (ld >= K, ld % 4 == 0); the buffer holds at least
 *                   (rows - 1) * ld + K values
 *   packed_codes,
 *   packed_scales : DEVICE, nvfp4_packed_size(rows, K) bytes each; every byte
 *                   is written (padding rows and panels as zeros), ready for
 *                   nvfp4_gemm as A (rows = M) or B (rows = N)
 * Same size rules as nvfp4_pack; 16-byte aligned pointers (else
 * NVFP4_ERR_MISALIGNED); non-finite inputs are outside the contract
 * (infinities saturate).  Asynchronous on `stream`; no allocation. */
int nvfp4_quantize(const float* x, int64_t rows, int64_t K, int64_t ld, void* packed_codes,
                   void* packed_scales, void* stream);

/* The same quantisation of bfloat16 rows.  The GEMM's output, and so the
 * activations the next layer quantises, is bfloat16 ("Peeling the Kernel
 * Onion", section "The Benchmark Design", the BF16 output term of the byte
 * count); every bfloat16 value is exactly an fp32 value, and the result is
 * that of nvfp4_quantize on the rows widened to fp32, byte for byte.
 *   x : DEVICE bfloat16, rows x K values, row stride ld elements (ld >= K,
 *       ld % 8 == 0); the buffer holds at least (rows - 1) * ld + K values
 * Everything else as nvfp4_quantize. */
int nvfp4_quantize_bf16(const void* x, int64_t rows, int64_t K, int64_t ld, void* packed_codes,
                        void* packed_scales, void* stream);

/* Element types of activation rows given to nvfp4_gemm_quantized. */
enum { NVFP4_INPUT_F32 = 0, NVFP4_INPUT_BF16 = 1 };

/* Decode-step GEMM from unquantised activations, in one launch:
 *   C = nvfp4_gemm(quantize(X), B)
 * bit for bit, where quantize is the rule of nvfp4_quantize (fp32 rows) or
 * nvfp4_quantize_bf16 (bfloat16 rows).  At one to four rows the
 * quantisation launch costs as much as the GEMM's own work, and the pages'
 * decode regime is exactly such batches ("Peeling the Kernel Onion",
 * sections "The Critical Connection to Real Inference" and "Knowledge
 * Created and Its Impact": per-call overhead dominates small GEMMs).  Each
 * workgroup of the dot-product kernel quantises X into LDS itself while
 * its rows of B arrive.
 *   x        : DEVICE, M x K values of type x_type (NVFP4_INPUT_F32 or
 *              NVFP4_INPUT_BF16), row stride ldx elements (ldx >= K; ldx % 4
 *              == 0 for fp32, % 8 for bfloat16)
 *   b_packed, b_scales : DEVICE, B (N x K) packed by nvfp4_pack
 *   out      : DEVICE, M x N bfloat16, row-major, overwritten
 *   M        : 1..4 (NVFP4_ERR_UNSUPPORTED above); the rows rounded up to 1,
 *              2 or 4 times K rounded up to 128 must be at most 65536
 *              (NVFP4_ERR_UNSUPPORTED otherwise: the quantised rows live in
 *              LDS)
 * Same alignment, status and stream rules as nvfp4_gemm; no workspace, no
 * allocation; the quantised A is not written out. */
int nvfp4_gemm_quantized(const void* x, int x_type, int64_t ldx, const void* b_packed,
                         const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                         int64_t K, void* stream);

/* Grouped GEMM for mixture-of-experts layers: `groups` weight operands B_g
 * (each N x K) share one launch; group g owns rows
 * row_offsets[g] .. row_offsets[g+1]-1 of A and of C:
 *   C[r][n] = bf16_rne(alpha * sum_k a'[r][k] * b'_g[n][k])  for r in group g
 * ("Peeling the Kernel Onion", sections "The Critical Connection to Real
 * Inference" -- tokens routed to experts, about 16 rows per expert -- and
 * "Knowledge Created and Its Impact" -- grouped GEMMs amortise the per-call
 * overhead).
 *   a_packed, a_scales : DEVICE, A (M x K, rows in group order) packed by
 *                        nvfp4_pack as one operand (rows = M)
 *   b_packed, b_scales : DEVICE, the `groups` weight operands, each N x K
 *                        packed by nvfp4_pack, concatenated: group g starts at
 *                        g * code_bytes and g * scale_bytes of
 *                        nvfp4_packed_size(N, K)
 *   row_offsets        : DEVICE int32[groups + 1], non-decreasing, from 0 to
 *                        M (a router's output; read by the kernel; entries are
 *                        clamped to [0, M], so a malformed table gives wrong
 *                        rows but no access outside the buffers)
 *   out                : DEVICE, M x N bfloat16, row-major; rows of every
 *                        group are overwritten, rows outside every group are
 *                        left untouched
 *   M                  : total rows (0 is allowed: nothing is launched)
 * The kernel follows the average group size M / groups: up to 32 rows (the
 * decode regime, about 16 rows per expert) a skinny kernel built for the
 * memory-bound case; from 33 to 463 rows a mid-size kernel with 64 x 64
 * output tiles of every group taken in turn by a persistent grid (at most
 * 4096 groups, else the skinny kernel); from 464 rows the MFMA tile kernel
 * with 256 x 256 tiles, one workgroup per row block of a group and column
 * block.  Either
 * way the result is the same GEMM, up to the order of the FP32 additions.
 * Same alignment (row_offsets: 4 bytes), status and stream rules as
 * nvfp4_gemm; no workspace, no allocation. */
int nvfp4_grouped_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
                       const void* b_scales, const int32_t* row_offsets, int64_t groups,
                       float alpha, void* out, int64_t M, int64_t N, int64_t K, void* stream);

/* nvfp4_grouped_gemm with a forced kernel, for tuning and tests:
 *   path : NVFP4_PATH_AUTO (the choice above), NVFP4_PATH_SKINNY (the decode
 *          kernel), NVFP4_PATH_WSPLIT (the mid-size kernel) or
 *          NVFP4_PATH_TILE (256 x 256 tiles); anything else is
 *          NVFP4_ERR_INVALID_VALUE
 * NVFP4_ERR_UNSUPPORTED if the forced kernel cannot run the call: the
 * mid-size kernel needs at most 4096 groups, and it and the tile kernel need
 * the packed codes of A and of one group's B each below 2 GiB.  Otherwise
 * the same contract as nvfp4_grouped_gemm; every path gives the same result
 * up to the order of the FP32 additions. */
int nvfp4_grouped_gemm_with_plan(const void* a_packed, const void* a_scales,
                                 const void* b_packed, const void* b_scales,
                                 const int32_t* row_offsets, int64_t groups, float alpha,
                                 void* out, int64_t M, int64_t N, int64_t K, int path,
                                 void* stream);

/* Where a plan came from. */
enum {
    NVFP4_PLAN_HEURISTIC = 0, /* the library's rules from M, N, K */
    NVFP4_PLAN_TABLE = 1      /* an entry of the loaded plan table */
};

/* A launch plan: the kernel path, the output tile of one workgroup, the
 * split-K factor, and its source. */
typedef struct nvfp4_plan_t {
    int32_t path;    /* NVFP4_PATH_TILE / _SKINNY / _WSPLIT / _GEMV */
    int32_t tile_m;  /* output rows of one workgroup's tile */
    int32_t tile_n;  /* output columns of one workgroup's tile (the `tile`
                        argument of nvfp4_gemm_with_plan is tile_m for the
                        tile path, tile_m x tile_n / 64 for wsplit) */
    int32_t split_k; /* number of K slices (>= 1) */
    int32_t tail_tiles; /* tile path, split_k 1: the last tail_tiles tiles run in a */
    int32_t tail_split; /* second launch with K split tail_split ways (0 if none)  */
    int32_t source;  /* NVFP4_PLAN_HEURISTIC or NVFP4_PLAN_TABLE */
} nvfp4_plan_t;

/* The plan nvfp4_gemm would use for a shape.  Host-only, no device work.
 * NVFP4_ERR_INVALID_VALUE for sizes nvfp4_gemm rejects or a NULL `plan`. */
int nvfp4_plan(int64_t M, int64_t N, int64_t K, nvfp4_plan_t* plan);

/* Tuned plan table.  The GEMM library on the pages picks a tile
 * configuration per shape by autotuning; that search lost its best tactics
 * ("The SM120 FP4 Kernel Disaster", Finding 3) and its results were never
 * saved ("The Multi-Pronged Investigation", Task 2).  Here the choices are
 * measured once, offline, and persisted as a JSON file:
 *   { "format": "nvfp4-plan-table", "version": 1, "arch": "gfx950",
 *     "build": "<nvfp4_build_id() of the library that was timed>",
 *     "entries": [ { "M": 4096, "N": 2048, "K": 6144, "path": "tile",
 *                    "tile": 128, "split_k": 1 }, ... ] }
 * "path" is "tile", "skinny", "wsplit" or "gemv"; "tile" and "split_k" follow
 * nvfp4_gemm_with_plan (tile 0 = the library's choice for the path, e.g.
 * "wsplit" tile 16 = 32 x 32, 32 = 64 x 32; split_k >= 1); other
 * keys are ignored.  Every entry is checked: sizes as for nvfp4_gemm, the
 * tile allowed for the path, skinny only for M <= 64 and gemv for M <= 4.
 * A later entry for the same (M, N, K) replaces an earlier one.
 * nvfp4_gemm (NVFP4_PATH_AUTO, nothing forced) then uses, for (M, N, K): the
 * entry for exactly that shape, else the entry with the same N and K and the
 * smallest M' >= M, if M' <= 2 M; else its own rules.  Which plan runs
 * changes only the order of FP32 additions, never the contract.
 * nvfp4_plan_table_load replaces the loaded table with the file's, or keeps
 * the old one if the file cannot be read or parsed or an entry is invalid
 * (NVFP4_ERR_INVALID_VALUE), or the arch is not gfx950
 * (NVFP4_ERR_UNSUPPORTED).  `entries` (may be NULL) receives the number of
 * entries loaded; `same_build` (may be NULL) is set to 1 if the table's
 * "build" equals nvfp4_build_id(), else 0 (the table was timed on other
 * kernels: still valid, perhaps no longer the fastest choice).
 * Thread-safe; calls that plan concurrently see the old or the new table. */
int nvfp4_plan_table_load(const char* json_path, int64_t* entries, int* same_build);

/* Drops the loaded table: plans come from the library's rules again. */
void nvfp4_plan_table_clear(void);

/* Identifier of the kernels this library was built from (a hash of their
 * sources; static string, never NULL). */
const char* nvfp4_build_id(void);

/* Recorded sequences: launch amortisation for decode steps.
 * A decode step of a served model runs the same short list of small GEMMs
 * for every token, and at batch 1-16 each GEMM's own work takes a few
 * microseconds, so launching them one by one from the host costs about as
 * much as the work; the pages' serving stack captures such steps into
 * graphs for that reason ("Peeling the Kernel Onion", section "Knowledge
 * Created and Its Impact").  A sequence records GEMMs, grouped GEMMs and
 * quantisations with fixed buffers once, and replays all of them with one
 * graph launch per step.
 *   nvfp4_sequence_create   : an empty sequence (host object, caller-owned)
 *   nvfp4_sequence_add_*    : append one call; arguments and checks as for
 *                             nvfp4_gemm / nvfp4_grouped_gemm / nvfp4_quantize
 *                             / nvfp4_quantize_bf16 / nvfp4_gemm_quantized
 *                             (minus the stream); the plan is fixed here.
 *                             Buffers are used by address at every launch:
 *                             they must stay allocated for the sequence's
 *                             lifetime, and their contents are read when the
 *                             sequence runs, not when it is recorded
 *   nvfp4_sequence_finalize : on the current device (gfx950), allocates the
 *                             sequence's own split-K workspace, captures the
 *                             calls in order into a HIP graph and
 *                             instantiates it; no further adds
 *   nvfp4_sequence_launch   : enqueues the whole sequence on `stream` (one
 *                             graph launch; asynchronous like nvfp4_gemm);
 *                             the current device must be the finalising one
 *   nvfp4_sequence_destroy  : frees the graph and the workspace; launches
 *                             must have completed (NULL is a no-op)
 * The calls of one launch run in recorded order.  Launches of one sequence
 * share its workspace: they must not run concurrently (launch on one stream,
 * or order the streams).  A sequence is not thread-safe; different
 * sequences are independent.  Results equal those of the same eager calls
 * in the same order, bit for bit.  Adding after finalize, finalizing twice,
 * or launching before finalize is NVFP4_ERR_STATE; finalizing an empty
 * sequence is NVFP4_ERR_INVALID_VALUE. */
typedef struct nvfp4_sequence* nvfp4_sequence_t;

int nvfp4_sequence_create(nvfp4_sequence_t* seq);
int nvfp4_sequence_add_gemm(nvfp4_sequence_t seq, const void* a_packed, const void* a_scales,
                            const void* b_packed, const void* b_scales, float alpha, void* out,
                            int64_t M, int64_t N, int64_t K);
int nvfp4_sequence_add_grouped_gemm(nvfp4_sequence_t seq, const void* a_packed,
                                    const void* a_scales, const void* b_packed,
                                    const void* b_scales, const int32_t* row_offsets,
                                    int64_t groups, float alpha, void* out, int64_t M, int64_t N,
                                    int64_t K);
int nvfp4_sequence_add_quantize(nvfp4_sequence_t seq, const float* x, int64_t rows, int64_t K,
                                int64_t ld, void* packed_codes, void* packed_scales);
int nvfp4_sequence_add_quantize_bf16(nvfp4_sequence_t seq, const void* x, int64_t rows,
                                     int64_t K, int64_t ld, void* packed_codes,
                                     void* packed_scales);
int nvfp4_sequence_add_gemm_quantized(nvfp4_sequence_t seq, const void* x, int x_type,
                                      int64_t ldx, const void* b_packed, const void* b_scales,
                                      float alpha, void* out, int64_t M, int64_t N, int64_t K);
int nvfp4_sequence_finalize(nvfp4_sequence_t seq);
int nvfp4_sequence_launch(nvfp4_sequence_t seq, void* stream);
int nvfp4_sequence_destroy(nvfp4_sequence_t seq);

/* ---- allocation-free GEMM ------------------------------------------------
 * For callers that cannot allocate device memory: code being captured into
 * a graph, tight serving loops, harnesses that forbid allocation.
 * nvfp4_gemm_noalloc is nvfp4_gemm (same arguments, plan, kernels and
 * results, bit for bit) except that its split-K workspace is a static device
 * array of NVFP4_NOALLOC_SCRATCH_BYTES per GPU (arrival counters first,
 * NVFP4_NOALLOC_MAX_COUNTERS of them, then FP32 partial tiles), which each
 * GPU the library runs on holds until the process ends.  It calls no
 * allocation routine of HIP or any other library.  Its device address is
 * looked up once per device, by nvfp4_init(device) or by the first call on
 * the device; make that first call outside a graph capture if the runtime
 * might refuse the lookup there.
 * Every call on one GPU shares that GPU's array: calls that can overlap on
 * one GPU (other streams, concurrent graph replays) race and give wrong
 * results; order them.  A shape whose plan needs more scratch than the
 * maximum is rejected with NVFP4_ERR_SCRATCH before anything is enqueued
 * (nvfp4_noalloc_scratch_bytes tells in advance). */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
#define NVFP4_NOALLOC_MAX_COUNTERS 16384
int nvfp4_gemm_noalloc(const void* a_packed, const void* a_scales, const void* b_packed,
                       const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                       int64_t K, void* stream);

/* Scratch nvfp4_gemm_noalloc needs for a shape: *bytes = 4 x the plan's
 * counters + 4 x its FP32 partials (0 when the plan does not split K).
 * Returns NVFP4_OK when that fits the static array, NVFP4_ERR_SCRATCH when
 * nvfp4_gemm_noalloc would reject the shape, and nvfp4_gemm's size errors.
 * Host-only, no device call. */
int nvfp4_noalloc_scratch_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);

/* ---- measurement aids (not part of the GEMM path) ------------------------
 * The floors that bound decode-sized calls: what a kernel that does nothing
 * costs per call, and the latency of a dependent load.
 *
 * nvfp4_probe_empty: enqueues an empty kernel of `blocks` workgroups of
 *   `threads` work-items (1..1024) on `stream`.
 * nvfp4_probe_chase: one work-item follows next[] from index 0 for `steps`
 *   dependent loads and writes the last index to *out.  next (device,
 *   caller-owned) holds n uint32 indices; n must be a power of two (up to
 *   2^32): each index is masked by n - 1, so no content of next[] can make a
 *   load leave the array.  A random single cycle through next[] of a chosen
 *   size measures the load latency of the cache level it fits in.
 * Both: NVFP4_ERR_INVALID_VALUE for arguments out of range or null pointers
 * (checked on the host, nothing enqueued), NVFP4_ERR_HIP if the launch
 * fails; asynchronous on `stream`. */
int nvfp4_probe_empty(int64_t blocks, int64_t threads, void* stream);
int nvfp4_probe_chase(const uint32_t* next, int64_t n, int64_t steps, uint32_t* out,
                      void* stream);

/* The two measured peaks beside the datasheet ones (the pages stress that a
 * quoted peak is an estimate: "Peeling the Kernel Onion", section
 * "Assumptions Embedded in the Benchmark"; "The SM120 FP4 Kernel Disaster",
 * section "Finding 4").
 * nvfp4_probe_mfma: `blocks` workgroups of 4 waves; every wave issues
 *   iters x 8 fp16 MFMAs of 32 x 32 x 16 (2 x 32 x 32 x 16 FLOP each) and
 *   writes one float per work-item to out (device, caller-owned, at least
 *   blocks x 256 floats).  blocks in 1 .. 2^20, iters >= 1.
 * nvfp4_probe_read: `blocks` workgroups of 256 work-items read the first
 *   `bytes` of src (device, 16-byte aligned; bytes a positive multiple of
 *   16) once, with 16-byte loads, and write nothing to out (device, one
 *   uint32, caller-owned) unless the bytes fold to a fixed improbable value.
 * Same error rules as the probes above. */
int nvfp4_probe_mfma(int64_t blocks, int64_t iters, float* out, void* stream);
int nvfp4_probe_read(const void* src, int64_t bytes, int64_t blocks, uint32_t* out,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
