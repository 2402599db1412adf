/*
 * libpgemm -- software-pipelined tiled fp16 GEMM and streaming elementwise
 * kernels for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * Plain C ABI: raw pointers, 64-bit sizes, an opaque stream handle.  Device
 * pointers are HIP device addresses (for example torch tensor data_ptr()).
 * The stream argument is a hipStream_t passed as void*; NULL selects the
 * default (null) stream.
 *
 * Common contract for every compute entry point:
 *  - Arguments are validated on the host before any HIP call.  A rejected
 *    call returns a negative status and touches no memory.
 *  - Work is enqueued asynchronously on `stream`; the call never
 *    synchronises, never allocates device memory and keeps no pointer after
 *    it returns.  The caller keeps the buffers alive until the stream has
 *    executed the work.
 *  - Outputs are write-only: their previous contents never influence the
 *    result (the buffer-revisiting rule of the Pallas software-pipelining
 *    guide, section 7.1: output buffers are written, not read).
 *  - PGEMM_EHIP means the kernel launch itself failed; pgemm_last_hip_error()
 *    then returns the hipError_t value (as int) for the calling thread.
 *    Errors of kernels that already ran asynchronously are reported by the
 *    stream, not by this library.
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* pgemm_stream_t; /* a hipStream_t */

enum pgemm_status {
    PGEMM_OK = 0,
    PGEMM_EINVAL = -1,       /* null pointer with a non-zero size, negative size, overlap */
    PGEMM_EUNSUPPORTED = -2, /* valid request outside what the kernels handle */
    PGEMM_EHIP = -3,         /* the HIP launch failed */
    PGEMM_ESCRATCH = -4      /* needs more than the static scratch buffer holds */
};

/*
 * C[M,N] = A[M,K] . B[K,N]
 *
 * The matmul of the Pallas "Quickstart: GPU" page, section "Pipelining: a
 * matmul kernel" (and section "Hopper 上的矩阵乘法内核" of its Chinese
 * rewrite): a parallel grid of output tiles, one workgroup per tile, and a
 * sequential loop over K whose global->LDS copies for later steps are in
 * flight while the matrix cores work on the current step.
 *
 * A, B, C: IEEE binary16, dense row-major, no leading-dimension arguments
 * (A is M x K with K contiguous, B is K x N with N contiguous, C is M x N).
 * Products are accumulated in fp32; each output is rounded once to binary16,
 * round-to-nearest-even (infinities on overflow, subnormals kept).  The
 * summation order inside fp32 is unspecified but fixed: identical inputs give
 * bit-identical outputs, call after call.
 *
 * Requirements: M, N, K >= 0; K % 8 == 0 and N % 8 == 0 (rows are moved in
 * 16-byte pieces); A, B, C 16-byte aligned; K < 2^22, N < 2^23 and
 * M*N <= 2^37 (the launch grid stays under 2^32 work-items); the C
 * range must not overlap A or B.
 *   M == 0 or N == 0: PGEMM_OK, nothing is enqueued.
 *   K == 0: C is filled with +0.0 (the empty sum).
 * Rows and columns that do not fill a whole tile are handled (no
 * truncation).
 * Returns PGEMM_EINVAL (null pointer with non-zero extent, negative size,
 * overlap of C with A or B), PGEMM_EUNSUPPORTED (alignment or divisibility
 * not met, sizes beyond the limits), PGEMM_EHIP, or PGEMM_OK.
 */
int pgemm_f16(const void* A, const void* B, void* C,
              int64_t M, int64_t N, int64_t K, pgemm_stream_t stream);

/*
 * Same as pgemm_f16 with the tile configuration forced (tests and
 * benchmarks).  `variant`:
 *   0  automatic choice (what pgemm_f16 does)
 *   1  256x256 output tile per workgroup, 4 waves; LDS ring of 5 stages of
 *      K 32 filled by global->LDS copies issued 2 to 4 steps ahead
 *   2  128x128 output tile, otherwise as 1
 *   3  256x256 output tile, 4 waves; 2 LDS stages of K 64 plus a register
 *      stage (global loads 2 steps ahead)
 *   4  128x128 output tile, otherwise as 3 (the 128x128x64 tiling of the
 *      quickstart's matmul)
 *   5  256x256 output tile, 8 waves (two per SIMD, 128x64 each), otherwise
 *      as 1
 *   6  128x128 output tile, wave-specialised: 4 waves only read LDS and
 *      multiply, a fifth wave issues every global->LDS copy and waits for
 *      them (the pages' warp-specialised pipeline); ring and copy order as 2
 *   7  as 2, on the 16x16x32 matrix instruction (one instruction per 16x16
 *      output block and K step of 32 instead of two 32x32x16 ones)
 *   8  as 5, on the 16x16x32 instruction
 *   9  as 8, persistent: at most one workgroup per compute unit, each
 *      walking several output tiles; the copies of a tile's first steps
 *      are issued before the previous tile's output is stored
 *   10 as 7 with a ring of 7 stages (copies up to 6 steps ahead; the
 *      quickstart's max_concurrent_steps), one workgroup per compute unit
 *   11 as 7 with a ring of 9 stages (copies up to 8 steps ahead)
 * Variants 1-6 give bit-identical results for the same inputs, and so do
 * variants 7-11: inside a family the grouping of the K sum of each output
 * element depends neither on the tiling nor on the pipeline.  The two
 * families group the products differently (16 vs 32 per instruction), so
 * they may differ in the last bits; both are within the accuracy bound.
 * Unknown variants return PGEMM_EUNSUPPORTED.
 */
int pgemm_f16_variant(const void* A, const void* B, void* C,
                      int64_t M, int64_t N, int64_t K, int variant,
                      pgemm_stream_t stream);

/* Number of GEMM variants accepted by pgemm_f16_variant (largest id). */
int pgemm_f16_num_variants(void);

/*
 * Split-K GEMM for shapes with few output tiles and a long K (the pages'
 * parallel grid has only the output tiles to spread over the CUs, so a long
 * K leaves most CUs idle or forces small tiles).  K is cut into chunks of
 * ceil(K/splits) rounded up to a multiple of 64, P of them non-empty
 * (P <= splits); chunk p runs as its own workgroups, multiplying A[:, chunk] by
 * B[chunk, :] with fp32 accumulation into the fp32 partial
 * workspace[p*M*N .. (p+1)*M*N) (row-major, pitch N); a second kernel then
 * writes C = fp16_rne(W_0 + W_1 + ... + W_{P-1}), the partials added in
 * ascending p in fp32.  Deterministic, within the same error bound as
 * pgemm_f16 but not bit-identical to it (another summation order), except
 * when P == 1: then it is exactly pgemm_f16 and needs no workspace.
 *   splits     requested number of chunks, 1 .. 64
 *   workspace  device memory of at least
 *              pgemm_f16_splitk_workspace_bytes(M, N, K, splits) bytes,
 *              16-byte aligned, disjoint from A, B and C; owned by the
 *              caller, contents overwritten, free to reuse once the stream
 *              has passed this call
 * Other arguments and requirements as pgemm_f16.  Returns PGEMM_EINVAL for a
 * missing, too small or overlapping workspace, PGEMM_EUNSUPPORTED for splits
 * out of range, a misaligned workspace or M*N > 2^36, else as pgemm_f16.
 */
int pgemm_f16_splitk(const void* A, const void* B, void* C,
                     int64_t M, int64_t N, int64_t K, int splits,
                     void* workspace, int64_t workspace_bytes,
                     pgemm_stream_t stream);

/*
 * pgemm_f16_splitk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The fp32 partials go to a static
 * device buffer of PGEMM_STATIC_SCRATCH_BYTES that the library's code object
 * holds on every device it is loaded on, until the process ends; the call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 * Results are bit-identical to pgemm_f16_splitk with the same arguments.
 * The buffer is one per device and shared by every call on it: calls that
 * overlap in time on one device (concurrent streams, or several host
 * threads) race on it and must be serialised by the caller.  No part of it
 * needs to start at zero: each call writes every partial it reads.
 * Returns PGEMM_ESCRATCH when pgemm_f16_splitk_workspace_bytes(M, N, K,
 * splits) exceeds PGEMM_STATIC_SCRATCH_BYTES (nothing is enqueued), else as
 * pgemm_f16_splitk.
 */
#define PGEMM_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)
int pgemm_f16_splitk_noalloc(const void* A, const void* B, void* C,
                             int64_t M, int64_t N, int64_t K, int splits,
                             pgemm_stream_t stream);

/* Workspace bytes pgemm_f16_splitk needs (0 when K forms a single chunk);
 * PGEMM_EINVAL / PGEMM_EUNSUPPORTED (negative) on invalid arguments. */
int64_t pgemm_f16_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splits);

/* A split count for pgemm_f16_splitk measured to pay off on MI355X: enough
 * (256x256 output tile, K chunk) pairs to give each of the 256 CUs one, with
 * chunks of at least 4096 and at most 8 splits; 1 (no split) when the output
 * alone has 256 tiles or K is short.  Pure host function.  PGEMM_EINVAL for a
 * negative size. */
int pgemm_f16_splitk_default_splits(int64_t M, int64_t N, int64_t K);

/*
 * The variant (1 .. pgemm_f16_num_variants()) that pgemm_f16 uses for an
 * M x N x K problem on the current device.  The tuned table built into the
 * library holds every variant's measured TFLOP/s on a set of shapes; it is
 * written by the autotuner (software_pipelined_tiled_pgemm_amd/autotune.py),
 * which times every variant -- tile shape, pipeline depth and wave count;
 * the pages name block size as the main tuning knob (software pipelining
 * guide, section 6.1) and advise autotuning the number of concurrent copies
 * (Chinese quickstart, section on emit_pipeline's key parameters).  The
 * choice is the fastest variant of the tuned shape T nearest to the problem
 * (smallest sum of |log2| ratios over M, N and K), unless the tile count of
 * the problem fills the CUs far worse than T's: each variant's rate on T is
 * scaled by fill(M, N) / fill(T.M, T.N), fill being M*N / (waves * slots *
 * tile area) with slots = (workgroups per CU) * CUs and waves =
 * ceil(tiles / slots) for the variant's 256x256 or 128x128 tile, and the
 * best estimate (the lowest id within 1% of it) replaces T's variant if it
 * beats that variant's estimate by more than 30%.  Host function: its only
 * HIP calls read the current device's CU count, once per device (256 when
 * there is no device).  Returns PGEMM_EINVAL for a negative size.
 */
int pgemm_f16_choose_variant(int64_t M, int64_t N, int64_t K);

/*
 * The launches pgemm_f16 makes for an M x N x K problem on a device with
 * `cus` compute units (cus <= 0: the current device's count, 256 if it
 * cannot be read).  Usually one: the variant pgemm_f16_choose_variant picks
 * on such a device, over all M rows (*head_rows = M, *tail_variant = 0).
 * When that variant uses 256x256 tiles and their last wave over the CUs
 * would be mostly idle, the
 * first *head_rows rows (a multiple of 256) run with it and the remaining
 * M - *head_rows rows with *tail_variant, the 128x128 variant of the same
 * matrix instruction, which gives bit-identical results.  The split minimises
 * waves(head tiles) + 0.35 * waves(tail tiles) (a wave of 128x128 tiles
 * takes about 0.35 of a wave of 256x256 ones at the same K) and is taken
 * only if it models at least 5% faster, for M*N*K of 1e10 or more.  Host
 * function: with cus > 0 it makes no HIP call; with cus <= 0 its only HIP
 * calls read the current device's attribute.  head_rows, head_variant,
 * tail_variant: host pointers, written on success.  Returns PGEMM_EINVAL for
 * a negative size or a null pointer, else PGEMM_OK.
 */
int pgemm_f16_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t* head_rows,
                   int* head_variant, int* tail_variant);

/*
 * z[i] = x[i] + y[i], i in [0, n): one IEEE binary32 addition per element,
 * round-to-nearest-even, no flush to zero -- bit-identical to any IEEE
 * implementation.  The pipelined elementwise add of the Pallas
 * software-pipelining guide, section 6 (copy_in / compute / copy_out per
 * block, neighbouring blocks overlapped); the data goes global -> registers
 * -> global without LDS (quickstart, section "GPU memory spaces": ALU work
 * bypasses shared memory).
 * x, y, z: device float arrays of n elements.  z may be exactly x or exactly
 * y (in place); any other overlap returns PGEMM_EINVAL.  n == 0 enqueues
 * nothing.  Any alignment is accepted (16-byte aligned arrays take the
 * vector path).
 */
int pstream_add(const float* x, const float* y, float* z, int64_t n,
                pgemm_stream_t stream);

/*
 * pstream_add with the per-workgroup block size forced: each workgroup
 * copies in, adds and copies out one contiguous block of `block_elems`
 * elements (the block-size parameter of the guide's section 6.1, whose
 * example uses 512*512; pstream_add uses 4096, the fastest measured on
 * MI355X).  block_elems must be a positive multiple of 1024 and at most
 * 2^24, else PGEMM_EUNSUPPORTED; so is an n of more than 2^24 - 1
 * blocks (one launch of 256-lane workgroups stays under 2^32 work-items).
 * Results do not depend on the block size.
 */
int pstream_add_blocked(const float* x, const float* y, float* z, int64_t n,
                        int64_t block_elems, pgemm_stream_t stream);

/*
 * z[i] = x[i] + c: the "+1" loop of the software-pipelining guide,
 * section 4, which writes its result back over its input (z == x is
 * allowed; any other overlap returns PGEMM_EINVAL).  One binary32 addition
 * per element.  Reads one array, so it moves 8 bytes per element.
 * n above (2^24 - 1) * 8192 is PGEMM_EUNSUPPORTED.
 */
int pstream_add_scalar(const float* x, float c, float* z, int64_t n,
                       pgemm_stream_t stream);

/*
 * o[j] = x[0][j] + x[1][j] + ... + x[R-1][j] for j in [0, n): the reduction
 * of the Pallas software-pipelining guide, section 7.2, which sums an
 * (R, M, N) array over its first axis by making that axis the last,
 * sequential grid axis and zeroing the resident output block at its first
 * step.  x is [R][n] row-major f32 (n = M*N), o is [n] f32.  The adds are
 * binary32, in ascending i, starting from +0.0f, so the result equals the
 * plain sequential loop bit for bit.  R == 0 writes +0.0 everywhere;
 * n == 0 enqueues nothing.  o must not overlap x (PGEMM_EINVAL); null
 * pointers with non-zero sizes and negative sizes are PGEMM_EINVAL;
 * n >= 2^36 or R*n > 2^40 is PGEMM_EUNSUPPORTED.  16-byte aligned x and o
 * with n % 4 == 0 take the vector path.
 */
int preduce_sum_f32(const float* x, float* o, int64_t R, int64_t n, pgemm_stream_t stream);

/*
 * Worked examples of the quickstart, exported for tests:
 *  pgemm_test_fill_f32: o[i] = v for i in [0, n) ("Your first kernel":
 *    128 elements of 42.0).
 *  pgemm_test_iota_f32: o[i] = (float)i, rounded to nearest-even ("Parallel
 *    work with a grid": 8 blocks of 128, block b writes its own slice).
 * n == 0 enqueues nothing; o == NULL with n > 0 returns PGEMM_EINVAL.
 */
int pgemm_test_fill_f32(float* o, float v, int64_t n, pgemm_stream_t stream);
int pgemm_test_iota_f32(float* o, int64_t n, pgemm_stream_t stream);

/* Static English text for a status code (never NULL). */
const char* pgemm_status_string(int status);

/* hipError_t of the last PGEMM_EHIP on the calling thread (0 if none). */
int pgemm_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int pgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
