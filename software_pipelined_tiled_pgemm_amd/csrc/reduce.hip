// Reduction along the last (sequential) grid axis, for gfx950.
//
// The Pallas software-pipelining guide, section 7.2 "reductions and
// accumulation", sums x of shape (R, M, N) over its first axis: the
// reduction axis becomes the LAST grid axis, the output block stays resident
// while consecutive steps add into it, it is set to zero at the first step,
// and it is written out once after the last step.  Here the output block of
// a lane is one float4 held in registers; the R slices it reads are the
// pipeline's steps.  A register ring (the guide's section 4 multi-buffering,
// with U slots) keeps the loads of the next U slices in flight while the
// current one is added: copy_start early, copy_wait (the compiler's vmcnt
// wait) just before the add.  The adds happen in ascending slice order, one
// IEEE binary32 addition per slice, starting from +0.0f, so the result is
// bit-identical to the plain sequential loop.
//
// HBM-bound: reads R*n*4 bytes and writes n*4 bytes.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pgemm {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRing = 8;  // slices in flight per lane

// Lane j owns output elements 4j .. 4j+3 (x, o 16-byte aligned, n % 4 == 0).
__global__ __launch_bounds__(kThreads) void sum_axis0_vec_kernel(const float* x, float* o,
                                                                 int64_t R, int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (4 * j >= n) return;
    const floatx4* src = reinterpret_cast<const floatx4*>(x) + j;
    const int64_t stride = n / 4;  // one slice, in float4
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};  // zero-init at the first step
    floatx4 ring[kRing];
    const int64_t pro = R < kRing ? R : kRing;
#pragma unroll
    for (int s = 0; s < kRing; ++s)  // prologue: copy_start for slices 0 .. kRing-1
        if (s < pro) ring[s] = __builtin_nontemporal_load(src + s * stride);
    int64_t i = 0;
    for (; i + kRing <= R; i += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            acc += ring[s];  // slice i+s: copy_wait, then the add
            if (i + s + kRing < R) ring[s] = __builtin_nontemporal_load(src + (i + s + kRing) * stride);
        }
    }
#pragma unroll
    for (int s = 0; s < kRing; ++s)
        if (i + s < R) acc += ring[s];
    reinterpret_cast<floatx4*>(o)[j] = acc;
}

// Any alignment or length: one output element per lane.
__global__ __launch_bounds__(kThreads) void sum_axis0_scalar_kernel(const float* x, float* o,
                                                                    int64_t R, int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= n) return;
    float acc = 0.0f;
    for (int64_t i = 0; i < R; ++i) acc = acc + x[i * n + j];
    o[j] = acc;
}

}  // namespace

hipError_t launch_sum_axis0(const float* x, float* o, int64_t R, int64_t n, hipStream_t stream) {
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(o)) & 15u) == 0 &&
                     (n % 4) == 0;
    if (vec) {
        const int64_t lanes = n / 4;
        hipLaunchKernelGGL(sum_axis0_vec_kernel, dim3((unsigned)((lanes + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, x, o, R, n);
    } else {
        hipLaunchKernelGGL(sum_axis0_scalar_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, x, o, R, n);
    }
    return hipGetLastError();
}

}  // namespace pgemm
