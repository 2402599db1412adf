// C ABI of libpgemm: argument validation, status codes, dispatch.
// Every check runs on the host before any HIP call; a rejected call touches
// no memory and enqueues nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pgemm.h"
#include "internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return PGEMM_OK;
    g_last_hip_error = (int)e;
    return PGEMM_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) (bytes) share at least one byte.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Elementwise operands: either the same array or disjoint.
bool bad_alias(const void* out, const void* in, int64_t bytes) {
    return out != in && overlap(out, bytes, in, bytes);
}

constexpr int64_t kMaxK = (int64_t)1 << 22;
constexpr int64_t kMaxN = (int64_t)1 << 23;
constexpr int64_t kMaxM = ((int64_t)1 << 31) - 256;
// M*N limit (256 GiB of C): keeps the tile count of a launch below 2^23, so
// that tiles times workgroup size stays under 2^32 work-items.
constexpr int64_t kMaxMN = (int64_t)1 << 37;

int check_gemm(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return PGEMM_EINVAL;
    if (M == 0 || N == 0) return PGEMM_OK;
    if (!C) return PGEMM_EINVAL;
    if (K > 0 && (!A || !B)) return PGEMM_EINVAL;
    if (K % 8 != 0 || N % 8 != 0) return PGEMM_EUNSUPPORTED;
    if (K >= kMaxK || N >= kMaxN || M >= kMaxM || M * N > kMaxMN) return PGEMM_EUNSUPPORTED;
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B)))) return PGEMM_EUNSUPPORTED;
    const int64_t cb = M * N * 2;
    if (K > 0 && (overlap(C, cb, A, M * K * 2) || overlap(C, cb, B, K * N * 2)))
        return PGEMM_EINVAL;
    return PGEMM_OK;
}

constexpr int kMaxSplits = 64;
constexpr int64_t kMaxSplitElems = (int64_t)1 << 36;  // M*N limit of the split-K path

// K chunk of each split: ceil(K / splits) rounded up to a multiple of 64 (a
// two-step period of the pipeline); the number of non-empty chunks.
int64_t splitk_chunk(int64_t K, int splits) {
    const int64_t c = (K + splits - 1) / splits;
    return (c + 63) / 64 * 64;
}
int64_t splitk_parts(int64_t K, int splits) {
    if (K <= 0) return 0;
    const int64_t c = splitk_chunk(K, splits);
    return (K + c - 1) / c;
}

}  // namespace

extern "C" {

int pgemm_f16_variant(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int variant, pgemm_stream_t stream) {
    if (variant < 0 || variant > pgemm::kGemmNumVariants) return PGEMM_EUNSUPPORTED;
    const int rc = check_gemm(A, B, C, M, N, K);
    if (rc != PGEMM_OK) return rc;
    if (M == 0 || N == 0) return PGEMM_OK;
    return hip_status(pgemm::launch_gemm_f16(A, B, C, M, N, K, variant,
                                             static_cast<hipStream_t>(stream)));
}

int pgemm_f16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
              pgemm_stream_t stream) {
    return pgemm_f16_variant(A, B, C, M, N, K, pgemm::kGemmAuto, stream);
}

int pgemm_f16_num_variants(void) { return pgemm::kGemmNumVariants; }

int pgemm_f16_splitk_default_splits(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return PGEMM_EINVAL;
    // Enough (256x256 tile, chunk) pairs for the 256 CUs, chunks of at least
    // 4096 (shorter chunks lose more to the partial traffic than they gain).
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (tiles == 0 || tiles >= 256) return 1;
    int64_t s = (256 + tiles - 1) / tiles;
    const int64_t by_k = K / 4096;
    if (s > by_k) s = by_k;
    if (s > 8) s = 8;
    return s < 1 ? 1 : (int)s;
}

int64_t pgemm_f16_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splits) {
    if (M < 0 || N < 0 || K < 0) return PGEMM_EINVAL;
    if (splits < 1 || splits > kMaxSplits) return PGEMM_EUNSUPPORTED;
    const int64_t parts = splitk_parts(K, splits);
    if (parts <= 1 || M == 0 || N == 0) return 0;
    if (N >= kMaxN || M >= kMaxM || M * N > kMaxSplitElems) return PGEMM_EUNSUPPORTED;
    return parts * M * N * 4;
}

int pgemm_f16_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                     int splits, void* workspace, int64_t workspace_bytes,
                     pgemm_stream_t stream) {
    if (splits < 1 || splits > kMaxSplits) return PGEMM_EUNSUPPORTED;
    const int rc = check_gemm(A, B, C, M, N, K);
    if (rc != PGEMM_OK) return rc;
    if (M == 0 || N == 0) return PGEMM_OK;
    const int64_t parts = splitk_parts(K, splits);
    if (parts <= 1)  // one chunk: exactly pgemm_f16
        return hip_status(pgemm::launch_gemm_f16(A, B, C, M, N, K, pgemm::kGemmAuto,
                                                 static_cast<hipStream_t>(stream)));
    if (M * N > kMaxSplitElems) return PGEMM_EUNSUPPORTED;
    const int64_t need = parts * M * N * 4;
    if (!workspace || workspace_bytes < need) return PGEMM_EINVAL;
    if (!aligned16(workspace)) return PGEMM_EUNSUPPORTED;
    if (overlap(workspace, need, A, M * K * 2) || overlap(workspace, need, B, K * N * 2) ||
        overlap(workspace, need, C, M * N * 2))
        return PGEMM_EINVAL;
    return hip_status(pgemm::launch_gemm_f16_splitk(
        A, B, C, M, N, K, splitk_chunk(K, splits), (int)parts, static_cast<float*>(workspace),
        static_cast<hipStream_t>(stream)));
}

int pgemm_f16_splitk_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N,
                             int64_t K, int splits, pgemm_stream_t stream) {
    if (splits < 1 || splits > kMaxSplits) return PGEMM_EUNSUPPORTED;
    const int rc = check_gemm(A, B, C, M, N, K);
    if (rc != PGEMM_OK) return rc;
    if (M == 0 || N == 0) return PGEMM_OK;
    const int64_t parts = splitk_parts(K, splits);
    if (parts <= 1)  // one chunk: exactly pgemm_f16, no partials
        return hip_status(pgemm::launch_gemm_f16(A, B, C, M, N, K, pgemm::kGemmAuto,
                                                 static_cast<hipStream_t>(stream)));
    if (M * N > kMaxSplitElems) return PGEMM_EUNSUPPORTED;
    if (parts * M * N * 4 > PGEMM_STATIC_SCRATCH_BYTES) return PGEMM_ESCRATCH;
    float* W = nullptr;
    const hipError_t e = pgemm::static_scratch(&W);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(pgemm::launch_gemm_f16_splitk(A, B, C, M, N, K, splitk_chunk(K, splits),
                                                    (int)parts, W,
                                                    static_cast<hipStream_t>(stream)));
}

int pgemm_f16_choose_variant(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return PGEMM_EINVAL;
    return pgemm::gemm_choose_variant(M, N, K, pgemm::compute_units());
}

int pgemm_f16_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t* head_rows,
                   int* head_variant, int* tail_variant) {
    if (M < 0 || N < 0 || K < 0 || !head_rows || !head_variant || !tail_variant)
        return PGEMM_EINVAL;
    const int c = cus > 0 ? cus : pgemm::compute_units();
    const int v = pgemm::gemm_choose_variant(M, N, K, c);
    const int64_t head = pgemm::gemm_head_rows(M, N, K, v, c);
    *head_rows = head;
    *head_variant = v;
    *tail_variant = head < M ? pgemm::gemm_small_partner(v) : 0;
    return PGEMM_OK;
}

int pstream_add_blocked(const float* x, const float* y, float* z, int64_t n, int64_t block_elems,
                        pgemm_stream_t stream) {
    if (n < 0) return PGEMM_EINVAL;
    if (block_elems <= 0 || block_elems % 1024 != 0 || block_elems > ((int64_t)1 << 24))
        return PGEMM_EUNSUPPORTED;
    if (n == 0) return PGEMM_OK;
    if (!x || !y || !z) return PGEMM_EINVAL;
    const int64_t bytes = n * (int64_t)sizeof(float);
    if (bad_alias(z, x, bytes) || bad_alias(z, y, bytes)) return PGEMM_EINVAL;
    if ((n + block_elems - 1) / block_elems > pgemm::kMaxGridBlocks) return PGEMM_EUNSUPPORTED;
    return hip_status(
        pgemm::launch_stream_add(x, y, z, n, block_elems, static_cast<hipStream_t>(stream)));
}

int pstream_add(const float* x, const float* y, float* z, int64_t n, pgemm_stream_t stream) {
    return pstream_add_blocked(x, y, z, n, pgemm::kStreamDefaultBlock, stream);
}

int pstream_add_scalar(const float* x, float c, float* z, int64_t n, pgemm_stream_t stream) {
    if (n < 0) return PGEMM_EINVAL;
    if (n == 0) return PGEMM_OK;
    if (!x || !z) return PGEMM_EINVAL;
    if (bad_alias(z, x, n * (int64_t)sizeof(float))) return PGEMM_EINVAL;
    if ((n + pgemm::kStreamScalarBlock - 1) / pgemm::kStreamScalarBlock > pgemm::kMaxGridBlocks)
        return PGEMM_EUNSUPPORTED;
    return hip_status(pgemm::launch_stream_add_scalar(x, c, z, n, static_cast<hipStream_t>(stream)));
}

int preduce_sum_f32(const float* x, float* o, int64_t R, int64_t n, pgemm_stream_t stream) {
    if (R < 0 || n < 0) return PGEMM_EINVAL;
    if (n == 0) return PGEMM_OK;
    if (!o || (R > 0 && !x)) return PGEMM_EINVAL;
    // n < 2^36: at most 2^24 - 1 workgroups of 4096 outputs.
    if (n >= ((int64_t)1 << 36) || R > ((int64_t)1 << 40) / n) return PGEMM_EUNSUPPORTED;
    if (R > 0 && overlap(o, n * 4, x, R * n * 4)) return PGEMM_EINVAL;
    return hip_status(pgemm::launch_sum_axis0(R > 0 ? x : o, o, R, n,
                                              static_cast<hipStream_t>(stream)));
}

int pgemm_test_fill_f32(float* o, float v, int64_t n, pgemm_stream_t stream) {
    if (n < 0) return PGEMM_EINVAL;
    if (n == 0) return PGEMM_OK;
    if (!o) return PGEMM_EINVAL;
    return hip_status(pgemm::launch_fill(o, v, n, static_cast<hipStream_t>(stream)));
}

int pgemm_test_iota_f32(float* o, int64_t n, pgemm_stream_t stream) {
    if (n < 0) return PGEMM_EINVAL;
    if (n == 0) return PGEMM_OK;
    if (!o) return PGEMM_EINVAL;
    return hip_status(pgemm::launch_iota(o, n, static_cast<hipStream_t>(stream)));
}

const char* pgemm_status_string(int status) {
    switch (status) {
        case PGEMM_OK: return "ok";
        case PGEMM_EINVAL: return "invalid argument (null pointer, negative size or overlapping buffers)";
        case PGEMM_EUNSUPPORTED: return "unsupported request (alignment, divisibility, size limit or variant)";
        case PGEMM_EHIP: return "HIP kernel launch failed";
        case PGEMM_ESCRATCH:
            return "split-K partials exceed the static scratch buffer (PGEMM_STATIC_SCRATCH_BYTES); "
                   "pgemm_f16_splitk takes a caller workspace of any size";
        default: return "unknown status";
    }
}

int pgemm_last_hip_error(void) { return g_last_hip_error; }

int pgemm_version(void) { return 200; }

}  // extern "C"
