// fp16 GEMM entry points of the 32x32x16 family (variants 1-6) and the
// shape -> variant chooser; the 16x16x32 family and split-K are in
// gemm_f16_m16.hip.  The kernels are in gemm_kernels.h.

#include "gemm_kernels.h"

namespace pgemm {

namespace {
// Shape -> fastest variant, measured by the autotuner (software_pipelined_
// tiled_pgemm_amd/autotune.py), which generates this file.
const TunedShape kTuned[] = {
#include "gemm_tuned.inc"
};

double log2_ratio(int64_t a, int64_t b) {
    const double x = log2((double)(a > 0 ? a : 1)) - log2((double)(b > 0 ? b : 1));
    return x < 0 ? -x : x;
}
}  // namespace

int gemm_choose_variant(int64_t M, int64_t N, int64_t K) {
    int best = kGemm128x128;
    double best_d = 1e300;
    for (const TunedShape& t : kTuned) {
        const double d = log2_ratio(M, t.M) + log2_ratio(N, t.N) + log2_ratio(K, t.K);
        if (d < best_d) {
            best_d = d;
            best = t.variant;
        }
    }
    return best;
}

hipError_t launch_gemm_f16(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int variant, hipStream_t stream) {
    if (variant == kGemmAuto) variant = gemm_choose_variant(M, N, K);
    float* const nows = nullptr;  // no split-K workspace
    switch (variant) {
        case kGemm256x256: {
            using TL = dm::Tile<256, 256>;
            return launch<TL>(dm::kernel<TL, 1>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        case kGemm128x128: {
            using TL = dm::Tile<128, 128>;
            return launch<TL>(dm::kernel<TL, 2>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        case kGemm256x256w8: {
            using TL = dm::Tile<256, 256, 2, 4>;
            return launch<TL>(dm::kernel<TL, 2>, TL::T, 1, A, B, C, M, N, K, stream, nows, 0);
        }
        case kGemm128x128m16:
        case kGemm256x256w8m16:
            return launch_gemm_f16_m16(A, B, C, M, N, K, variant, stream);
        case kGemmWs128x128: {
            using TL = dm::Tile<128, 128>;
            return launch<TL>(ws::kernel<TL>, TL::T + 64, 1, A, B, C, M, N, K, stream);
        }
        case kGemmRs256x256: {
            using TL = rs::Tile<256, 256>;
            return launch<TL>(rs::kernel<TL, 1>, TL::T, 1, A, B, C, M, N, K, stream);
        }
        case kGemmRs128x128: {
            using TL = rs::Tile<128, 128>;
            return launch<TL>(rs::kernel<TL, 2>, TL::T, 1, A, B, C, M, N, K, stream);
        }
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace pgemm
