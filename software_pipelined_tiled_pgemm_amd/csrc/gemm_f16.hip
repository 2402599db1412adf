// fp16 GEMM entry points of the 32x32x16 family (variants 1-6) and the
// shape -> variant chooser; the 16x16x32 family and split-K are in
// gemm_f16_m16.hip.  The kernels are in gemm_kernels.h.

#include <algorithm>
#include <atomic>

#include "gemm_kernels.h"

namespace pgemm {

namespace {
// Shape -> fastest variant, measured by the autotuner (software_pipelined_
// tiled_pgemm_amd/autotune.py), which generates this file.
const TunedShape kTuned[] = {
#include "gemm_tuned.inc"
};

constexpr int kNumTuned = sizeof(kTuned) / sizeof(kTuned[0]);

double log2_size(int64_t a) { return log2((double)(a > 0 ? a : 1)); }

// log2 of every tuned M, N, K, computed once.
struct TunedLogs {
    double m[kNumTuned], n[kNumTuned], k[kNumTuned];
    TunedLogs() {
        for (int i = 0; i < kNumTuned; ++i) {
            m[i] = log2_size(kTuned[i].M);
            n[i] = log2_size(kTuned[i].N);
            k[i] = log2_size(kTuned[i].K);
        }
    }
};
}  // namespace

// Output tile edge of a variant (256 or 128).
int variant_tile(int v) {
    switch (v) {
        case kGemm256x256:
        case kGemmRs256x256:
        case kGemm256x256w8:
        case kGemm256x256w8m16:
        case kGemm256x256w8m16p:
            return 256;
        default:
            return 128;
    }
}

// Workgroups of a variant that fit on one CU at once (LDS-bound).
int variant_wgs_per_cu(int v) {
    switch (v) {
        case kGemm128x128:
        case kGemmRs128x128:
        case kGemmWs128x128:
        case kGemm128x128m16:
            return 2;
        default:
            return 1;
    }
}

// Useful share of the slots an M x N launch of tile edge b occupies, with
// `slots` workgroups resident at once: M*N / (waves * slots * b*b),
// waves = ceil(tiles / slots).
double slot_fill(int64_t M, int64_t N, int b, int64_t slots) {
    const int64_t tiles = ((M + b - 1) / b) * ((N + b - 1) / b);
    const int64_t waves = (tiles + slots - 1) / slots;
    return (double)M * (double)N / ((double)waves * slots * b * b);
}

int gemm_choose_variant(int64_t M, int64_t N, int64_t K, int cus) {
    static const TunedLogs logs;
    if (kNumTuned == 0) return kGemm128x128;
    if (cus <= 0) cus = 256;
    if (M <= 0 || N <= 0) return kGemm128x128;
    const double lm = log2_size(M), ln = log2_size(N), lk = log2_size(K);
    int near = 0;
    double near_d = 1e300;
    for (int i = 0; i < kNumTuned; ++i) {
        const double d = fabs(lm - logs.m[i]) + fabs(ln - logs.n[i]) + fabs(lk - logs.k[i]);
        if (d < near_d) {
            near_d = d;
            near = i;
        }
    }
    const TunedShape& t = kTuned[near];
    const int v0 = t.variant;
    double est[kGemmNumVariants];
    double top = 0.0;
    for (int v = 1; v <= kGemmNumVariants; ++v) {
        const int b = variant_tile(v);
        const int64_t slots = (int64_t)variant_wgs_per_cu(v) * cus;
        est[v - 1] = t.tflops[v - 1] * slot_fill(M, N, b, slots) / slot_fill(t.M, t.N, b, slots);
        top = std::max(top, est[v - 1]);
    }
    if (v0 < 1 || v0 > kGemmNumVariants || top <= 0.0) return kGemm128x128;
    int alt = v0;
    for (int v = kGemmNumVariants; v >= 1; --v)
        if (est[v - 1] >= (1.0 - 0.01) * top) alt = v;
    return est[alt - 1] > kRefillGain * est[v0 - 1] ? alt : v0;
}

namespace {

hipError_t launch_variant(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                          int variant, hipStream_t stream) {
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
        case kGemm256x256w8m16p:
        case kGemm128x128m16s7:
        case kGemm128x128m16s9:
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

}  // namespace

int compute_units() {
    // Read once per device (the attribute query costs more host time than
    // the rest of a small GEMM call's dispatch logic).
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int gemm_small_partner(int variant) {
    switch (variant) {
        case kGemm256x256:
        case kGemm256x256w8:
            return kGemm128x128;
        case kGemm256x256w8m16:
        case kGemm256x256w8m16p:
            return kGemm128x128m16;
        default:
            return 0;
    }
}

int64_t gemm_head_rows(int64_t M, int64_t N, int64_t K, int variant, int cus) {
    if (gemm_small_partner(variant) == 0 || cus <= 0 || (double)M * N * K < kSplitRowsMinMNK)
        return M;
    const int64_t tmb = (M + 255) / 256, tnb = (N + 255) / 256, tns = (N + 127) / 128;
    auto waves = [cus](int64_t tiles) { return (double)((tiles + cus - 1) / cus); };
    double best = waves(tmb * tnb) * kSplitRowsMargin;
    int64_t head = M;
    // The cost only changes where the head's wave count does: try the
    // largest head of each wave count.
    for (int64_t w = 1; (w - 1) * cus < (tmb - 1) * tnb; ++w) {
        const int64_t r = std::min(tmb - 1, w * cus / tnb);
        if (r < 1) continue;
        const int64_t tail_tiles = ((M - 256 * r + 127) / 128) * tns;
        const double cost = waves(r * tnb) + kSmallTileWave * waves(tail_tiles);
        if (cost < best) {
            best = cost;
            head = 256 * r;
        }
    }
    return head;
}

hipError_t launch_gemm_f16(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int variant, hipStream_t stream) {
    if (variant != kGemmAuto) return launch_variant(A, B, C, M, N, K, variant, stream);
    const int cus = compute_units();
    variant = gemm_choose_variant(M, N, K, cus);
    const int64_t head = gemm_head_rows(M, N, K, variant, cus);
    if (head >= M) return launch_variant(A, B, C, M, N, K, variant, stream);
    // Head rows on the 256x256 tile, the rest on the 128x128 tile of the
    // same matrix-instruction family: every output's K sum is grouped the
    // same way, so the results are bit-identical to one launch.
    const hipError_t rc = launch_variant(A, B, C, head, N, K, variant, stream);
    if (rc != hipSuccess) return rc;
    return launch_variant(static_cast<const _Float16*>(A) + head * K, B,
                          static_cast<_Float16*>(C) + head * N, M - head, N, K,
                          gemm_small_partner(variant), stream);
}

}  // namespace pgemm
