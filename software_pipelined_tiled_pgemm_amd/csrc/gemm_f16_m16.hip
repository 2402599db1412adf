// fp16 GEMM entry points of the 16x16x32 family (variants 7-11) and the
// split-K path, which runs on the same kernels.
//
// This file is compiled with MFMA results kept in ordinary VGPRs (no
// accumulation registers): with them the compiler left these kernels'
// 16x16 accumulator blocks in VGPRs without the register-to-register copies
// it otherwise inserted into the K loop (measured 8-10% faster on MI355X).
// The 32x32x16 family needs the accumulation registers for its 256x256
// tile, so it is built separately.

#include "gemm_kernels.h"

namespace pgemm {

hipError_t launch_gemm_f16_m16(const void* A, const void* B, void* C, int64_t M, int64_t N,
                               int64_t K, int variant, hipStream_t stream) {
    float* const nows = nullptr;  // no split-K workspace
    switch (variant) {
        case kGemm128x128m16: {
            using TL = dm::Tile<128, 128, 2, 2, 16>;
            return launch<TL>(dm::kernel<TL, 2>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        case kGemm256x256w8m16: {
            using TL = dm::Tile<256, 256, 2, 4, 16>;
            return launch<TL>(dm::kernel<TL, 2>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        case kGemm256x256w8m16p: {
            using TL = dm::Tile<256, 256, 2, 4, 16>;
            return launch_persistent<TL>(dm::kernel_persistent<TL, 2>, TL::T, A, B, C, M, N, K,
                                         compute_units(), stream);
        }
        case kGemm128x128m16s7: {
            using TL = dm::Tile<128, 128, 2, 2, 16, 7>;
            return launch<TL>(dm::kernel<TL, 1>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        case kGemm128x128m16s9: {
            using TL = dm::Tile<128, 128, 2, 2, 16, 9>;
            return launch<TL>(dm::kernel<TL, 1>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_f16_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                  int64_t K, int64_t chunk, int splits, float* W,
                                  hipStream_t stream) {
    // 256x256 tiles (8 waves) when the (tile, chunk) pairs fill the chip's
    // 256 CUs, 128x128 otherwise.
    const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    hipError_t rc;
    if (big * splits >= 256) {
        using TL = dm::Tile<256, 256, 2, 4, 16>;
        rc = launch<TL>(dm::kernel<TL, 2, true>, TL::T, splits, A, B, C, M, N, K, stream, W,
                        (int)chunk);
    } else {
        using TL = dm::Tile<128, 128, 2, 2, 16>;
        rc = launch<TL>(dm::kernel<TL, 2, true>, TL::T, splits, A, B, C, M, N, K, stream, W,
                        (int)chunk);
    }
    if (rc != hipSuccess) return rc;
    return launch_splitk_sum(W, static_cast<_Float16*>(C), splits, M * N, stream);
}

}  // namespace pgemm
