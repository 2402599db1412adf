// Reduction along the last (sequential) grid axis, for gfx950.
//
// The Pallas software-pipelining guide, section 7.2 "reductions and
// accumulation", sums x of shape (R, M, N) over its first axis: the
// reduction axis becomes the LAST grid axis, the output block stays resident
// while consecutive steps add into it, it is set to zero at the first step,
// and it is written out once after the last step.  Here the output block of
// a lane is U float4s held in registers (lane-interleaved, so one wave reads
// U KiB contiguous of every slice); the R slices it reads are the pipeline's
// steps.  The register ring of pipeline.h (the guide's section 4
// multi-buffering, kRing slots) keeps the loads of the next slices in flight
// while the current one is added: copy_start early, copy_wait (the
// compiler's vmcnt wait) just before the add.  The adds happen in ascending slice order, one IEEE
// binary32 addition per slice, starting from +0.0f, so the result is
// bit-identical to the plain sequential loop.
//
// HBM-bound: reads R*n*4 bytes and writes n*4 bytes.  Runs of 4 KiB per
// slice and wave matter: with one float4 per lane (1 KiB runs from R slices
// 64 MiB apart at (8, 4096, 4096)) the kernel reached 2.8 TB/s, with four
// 6.2 TB/s (measured on MI355X).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "pipeline.h"

namespace pgemm {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // float4 outputs per lane
constexpr int kRing = 4;    // slices in flight per lane

// Lane t of block b owns float4 outputs b*kThreads*kUnroll + u*kThreads + t,
// u < kUnroll (x, o 16-byte aligned, n % 4 == 0).
__global__ __launch_bounds__(kThreads) void sum_axis0_vec_kernel(const float* x, float* o,
                                                                 int64_t R, int64_t n) {
    const int64_t lanes = n / 4;  // float4 per slice
    const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
    const floatx4* src = reinterpret_cast<const floatx4*>(x);
    bool in[kUnroll];
    floatx4 acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        in[u] = base + u * kThreads < lanes;
        acc[u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};  // zero-init at the first step
    }
    struct Slice {
        floatx4 v[kUnroll];
    };
    ring_pipeline<kRing, Slice>(
        R,
        [&](int64_t s, Slice& sl) {  // copy_start of slice s
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                sl.v[u] = in[u] ? __builtin_nontemporal_load(src + s * lanes + base + u * kThreads)
                                : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        },
        [&](int64_t, const Slice& sl) {  // slices arrive in ascending order
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc[u] += sl.v[u];
        });
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        if (in[u])
            __builtin_nontemporal_store(acc[u], reinterpret_cast<floatx4*>(o) + base + u * kThreads);
}

// Any alignment or length: one output element per lane and iteration of a
// grid-stride loop (the grid is capped, n is not).
__global__ __launch_bounds__(kThreads) void sum_axis0_scalar_kernel(const float* x, float* o,
                                                                    int64_t R, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < n; j += stride) {
        float acc = 0.0f;
        for (int64_t i = 0; i < R; ++i) acc = acc + x[i * n + j];
        o[j] = acc;
    }
}

// Split-K finish: C[i] = fp16_rne(W[0][i] + W[1][i] + ... + W[S-1][i]), the
// partials added in ascending order from +0.0f in fp32.  Lane t owns 8
// consecutive outputs (two float4 per partial, one 16-byte fp16 store); n is
// a multiple of 8 and both arrays are 16-byte aligned.
// Group j of the split-K finish (outputs 8j .. 8j+7).
__device__ __forceinline__ void splitk_sum_group(const float* W, _Float16* C, int64_t S, int64_t n,
                                                 int64_t j) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const floatx4* src = reinterpret_cast<const floatx4*>(W) + 2 * j;
    const int64_t stride = n / 4;  // one partial, in float4
    floatx4 lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = lo;
    struct Part {
        floatx4 a, b;
    };
    ring_pipeline<kRing, Part>(
        S,
        [&](int64_t s, Part& p) {
            p.a = __builtin_nontemporal_load(src + s * stride);
            p.b = __builtin_nontemporal_load(src + s * stride + 1);
        },
        [&](int64_t, const Part& p) {
            lo += p.a;
            hi += p.b;
        });
    u32x4 out;
    out[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{lo[0], lo[1]}), half2_t));
    out[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{lo[2], lo[3]}), half2_t));
    out[2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{hi[0], hi[1]}), half2_t));
    out[3] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{hi[2], hi[3]}), half2_t));
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(C) + j);
}

// The grid is capped (kMaxGridBlocks), so a lane walks groups j, j + lanes of
// the grid, ...
__global__ __launch_bounds__(kThreads) void splitk_sum_kernel(const float* W, _Float16* C,
                                                              int64_t S, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; 8 * j < n; j += stride)
        splitk_sum_group(W, C, S, n, j);
}

}  // namespace

hipError_t launch_splitk_sum(const float* W, _Float16* C, int64_t S, int64_t n,
                             hipStream_t stream) {
    const int64_t groups = n / 8;
    int64_t blocks = (groups + kThreads - 1) / kThreads;
    if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, W, C,
                       S, n);
    return hipGetLastError();
}

hipError_t launch_sum_axis0(const float* x, float* o, int64_t R, int64_t n, hipStream_t stream) {
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(o)) & 15u) == 0 &&
                     (n % 4) == 0;
    if (vec) {
        const int64_t lanes = n / 4;
        const int64_t per_block = (int64_t)kThreads * kUnroll;
        hipLaunchKernelGGL(sum_axis0_vec_kernel, dim3((unsigned)((lanes + per_block - 1) / per_block)),
                           dim3(kThreads), 0, stream, x, o, R, n);
    } else {
        int64_t blocks = (n + kThreads - 1) / kThreads;
        if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
        hipLaunchKernelGGL(sum_axis0_scalar_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, x, o, R, n);
    }
    return hipGetLastError();
}

}  // namespace pgemm
