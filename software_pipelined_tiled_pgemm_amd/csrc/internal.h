// Internal launch interface between the C ABI (pgemm_api.hip) and the
// kernels.  Arguments reaching these functions have been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgemm {

// GEMM tile configurations (ids match pgemm_f16_variant).
enum GemmVariant : int {
    kGemmAuto = 0,
    kGemm256x256 = 1,    // LDS-DMA pipeline, 5 stages of K 32
    kGemm128x128 = 2,    // LDS-DMA pipeline, 5 stages of K 32
    kGemmRs256x256 = 3,  // register-staged pipeline, 2 LDS stages of K 64
    kGemmRs128x128 = 4,  // register-staged pipeline, 2 LDS stages of K 64
    kGemm256x256w8 = 5,  // LDS-DMA pipeline, 8 waves (2 per SIMD), 128x64 per wave
    kGemmWs128x128 = 6,  // wave-specialised LDS-DMA pipeline: 4 MFMA waves + 1 copy wave
    // The same LDS-DMA pipeline on v_mfma_f32_16x16x32_f16 (one MFMA per
    // 16x16 block and K step of 32).  A different accumulation grouping, so
    // results are bit-identical within this family, not with variants 1-6.
    kGemm128x128m16 = 7,    // 4 waves, 64x64 per wave, 2 workgroups per CU
    kGemm256x256w8m16 = 8,  // 8 waves (2 per SIMD), 128x64 per wave
    // Variant 8 as a persistent kernel: one workgroup per CU walks several
    // tiles, the next tile's first copies overlapping this tile's drain.
    // Bit-identical to variants 7 and 8 (the same K order).
    kGemm256x256w8m16p = 9,
    // Variant 7 with a deeper ring (the pages' max_concurrent_steps knob): 7
    // or 9 LDS stages (112 or 144 KiB, so one workgroup per CU), copies up
    // to 6 or 8 steps ahead.  Bit-identical to variants 7-9.
    kGemm128x128m16s7 = 10,
    kGemm128x128m16s9 = 11,
    kGemmNumVariants = 11,
};

// Picks a concrete variant for a problem shape on a device with `cus` CUs.
// The tuned table (gemm_tuned.inc, written by the autotuner) holds, for each
// tuned shape, the fastest variant and every variant's measured TFLOP/s.
// Take the tuned shape T nearest to (M, N, K) (distance = sum over M, N, K
// of |log2(shape / T)|) and its fastest variant v0.  Estimate each
// variant's rate on (M, N, K) as its rate on T times fill(M, N) / fill(T),
// fill being the useful share of the workgroup slots the launch occupies:
// M*N / (waves * slots * tile area), slots = workgroups per CU * cus,
// waves = ceil(tiles / slots).  Let alt be the fastest estimate (the lowest
// id within 1% of it): the choice is alt if its estimate beats v0's by more
// than kRefillGain, else v0.  So the nearest tuned shape decides unless the
// problem's tile count lands far worse on the CUs than T's for v0 (a shape
// just past a multiple of the tile, or with far fewer tiles).
int gemm_choose_variant(int64_t M, int64_t N, int64_t K, int cus);
// Measured on 240 random shapes against the nearest-shape rule alone: a
// smaller margin changes more choices for the worse than for the better.
constexpr double kRefillGain = 1.3;

struct TunedShape {
    int64_t M, N, K;
    int variant;                      // fastest on this shape (informative)
    double tflops[kGemmNumVariants];  // measured rate of variant v at [v - 1]
};

// Variant kGemmAuto runs gemm_choose_variant's pick, except that when its
// 256x256 tiles would leave most of the last wave of CUs idle it runs the
// first gemm_head_rows(...) rows with it and the remaining rows with the
// 128x128 variant of the same matrix instruction (gemm_small_partner): the
// same results bit for bit, in two launches on the stream.
hipError_t launch_gemm_f16(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int variant, hipStream_t stream);

// CU count of the current device (256 if it cannot be read).
int compute_units();
// The 128x128 variant computing bit-identical results to a 256x256 one, or 0.
int gemm_small_partner(int variant);
// Row split for a poorly filled last wave: the head rows (a multiple of 256,
// or M for no split) minimising the modelled time
//   waves(head 256x256 tiles) + kSmallTileWave * waves(tail 128x128 tiles),
// taken only if it beats one launch by the margin; waves = ceil(tiles / cus).
int64_t gemm_head_rows(int64_t M, int64_t N, int64_t K, int variant, int cus);
// A wave of 128x128 tiles takes about this fraction of a wave of 256x256
// tiles at the same K (measured: 42 us against 122 us at K = 6144).
constexpr double kSmallTileWave = 0.35;
constexpr double kSplitRowsMargin = 0.95;  // split only for a modelled gain of 5% or more
constexpr double kSplitRowsMinMNK = 1.0e10;  // below this, launch latency dominates
// Variants of the 16x16x32 family (gemm_f16_m16.hip).
hipError_t launch_gemm_f16_m16(const void* A, const void* B, void* C, int64_t M, int64_t N,
                               int64_t K, int variant, hipStream_t stream);

// Split-K: `splits` workgroups per output tile, split s multiplying the K
// range [s*chunk, min(K, (s+1)*chunk)) into the fp32 partial W + s*M*N, then
// C = fp16(W_0 + W_1 + ... ) summed in ascending s (launch_splitk_sum).
hipError_t launch_gemm_f16_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                  int64_t K, int64_t chunk, int splits, float* W,
                                  hipStream_t stream);
hipError_t launch_splitk_sum(const float* W, _Float16* C, int64_t S, int64_t n,
                             hipStream_t stream);
// Device address of the current device's copy of the static split-K scratch
// buffer (PGEMM_STATIC_SCRATCH_BYTES), looked up once per device
// (splitk_static.hip).
hipError_t static_scratch(float** out);

// Elements per workgroup block of the streaming kernels (the block-size knob
// of the pipelined elementwise add), chosen by measurement on MI355X: small
// one-shot blocks keep many workgroups, and so many 16-byte loads, in flight.
constexpr int64_t kStreamDefaultBlock = 4096;
constexpr int64_t kStreamScalarBlock = 8192;
// Most workgroups of 256 lanes in one launch: HIP rejects a grid whose
// dimension times the workgroup size reaches 2^32 work-items.
constexpr int64_t kMaxGridBlocks = (((int64_t)1 << 32) - 1) / 256;

hipError_t launch_stream_add(const float* x, const float* y, float* z, int64_t n,
                             int64_t block_elems, hipStream_t stream);
hipError_t launch_stream_add_scalar(const float* x, float c, float* z, int64_t n,
                                    hipStream_t stream);
hipError_t launch_fill(float* o, float v, int64_t n, hipStream_t stream);
hipError_t launch_sum_axis0(const float* x, float* o, int64_t R, int64_t n, hipStream_t stream);
hipError_t launch_iota(float* o, int64_t n, hipStream_t stream);

}  // namespace pgemm
