// Streaming elementwise kernels for gfx950.
//
// The pipelined elementwise add of the Pallas software-pipelining guide
// (sections 3, 4 and 6): the array is cut into blocks; for each block the
// copy_in, the add and the copy_out run as three stages, and the stages of
// neighbouring blocks overlap.  On a GPU the overlap comes from many blocks
// (one per workgroup) and many loads in flight per lane, and the data path is
// global -> registers -> global with no LDS (quickstart, section "GPU memory
// spaces": ALU-only work bypasses shared memory).  The kernel is bound by HBM
// bandwidth: 12 bytes move per element for x + y, 8 for x + c.
//
// Inside a workgroup's block each lane walks groups of kUnroll 16-byte
// pieces per operand through a register ring (pipeline.h, the guide's
// section 4 pipeline with kStages buffers): the loads of the next groups are
// in flight while the current group is added and stored.  With the default
// block (4096 elements for x + y, 8192 for x + c) every lane has exactly one
// group and the overlap comes from the many workgroups; with the pages'
// 512 x 512 blocks (one workgroup per CU) the ring is what keeps enough
// bytes in flight.  Loads and stores are non-temporal: the data is touched
// once, so it should not displace anything in the caches.  Arithmetic is one
// IEEE binary32 add per element (v_add_f32, RNE, denormals kept), so results
// are bit-identical to any IEEE implementation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "pipeline.h"

namespace pgemm {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte loads per operand per lane and group
#ifndef PGEMM_STREAM_STAGES
#define PGEMM_STREAM_STAGES 2
#endif
// Groups in flight per lane: 2 is the guide's double buffer.  Depths 1 to 4
// measured the same on MI355X (5.7-5.9 TB/s at the pages' 512x512 blocks,
// 6.6 TB/s at the default block), so the smallest register footprint wins.
constexpr int kStages = PGEMM_STREAM_STAGES;

struct AddSlot {
    floatx4 a[kUnroll], b[kUnroll];
};

// One workgroup per block of `block` elements (block is a multiple of 1024,
// so a block starts 16-byte aligned whenever the arrays do).  Group g of a
// block is float4s g*kUnroll*kThreads .. +kUnroll*kThreads-1, lane t taking
// every kThreads-th.  The last block may be ragged: its whole float4s past
// the last full group and its scalar tail are handled by the same workgroup.
__global__ __launch_bounds__(kThreads) void add_vec_kernel(const float* x, const float* y,
                                                           float* z, int64_t n, int64_t block) {
    const int64_t start = (int64_t)blockIdx.x * block;
    const int64_t len = min(block, n - start);
    const int64_t nv = len >> 2;  // whole float4s in this block
    const floatx4* xv = reinterpret_cast<const floatx4*>(x + start);
    const floatx4* yv = reinterpret_cast<const floatx4*>(y + start);
    floatx4* zv = reinterpret_cast<floatx4*>(z + start);
    constexpr int64_t G = (int64_t)kUnroll * kThreads;
    const int64_t groups = nv / G;
    const int t = threadIdx.x;
    ring_pipeline<kStages, AddSlot>(
        groups,
        [&](int64_t g, AddSlot& sl) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                sl.a[u] = __builtin_nontemporal_load(xv + g * G + u * kThreads + t);
                sl.b[u] = __builtin_nontemporal_load(yv + g * G + u * kThreads + t);
            }
        },
        [&](int64_t g, const AddSlot& sl) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                __builtin_nontemporal_store(sl.a[u] + sl.b[u], zv + g * G + u * kThreads + t);
        });
    for (int64_t i = groups * G + t; i < nv; i += kThreads) zv[i] = xv[i] + yv[i];
    for (int64_t e = (nv << 2) + t; e < len; e += kThreads) z[start + e] = x[start + e] + y[start + e];
}

// Any alignment: one element per lane per iteration.
__global__ __launch_bounds__(kThreads) void add_scalar_path_kernel(const float* x, const float* y,
                                                                   float* z, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        z[i] = x[i] + y[i];
}

struct AddcSlot {
    floatx4 a[2 * kUnroll];
};

// x + c: one input, so twice the float4s per group for the same bytes in
// flight.
__global__ __launch_bounds__(kThreads) void addc_vec_kernel(const float* x, float c, float* z,
                                                            int64_t n, int64_t block) {
    const int64_t start = (int64_t)blockIdx.x * block;
    const int64_t len = min(block, n - start);
    const int64_t nv = len >> 2;
    const floatx4* xv = reinterpret_cast<const floatx4*>(x + start);
    floatx4* zv = reinterpret_cast<floatx4*>(z + start);
    constexpr int64_t G = (int64_t)2 * kUnroll * kThreads;
    const int64_t groups = nv / G;
    const int t = threadIdx.x;
    ring_pipeline<kStages, AddcSlot>(
        groups,
        [&](int64_t g, AddcSlot& sl) {
#pragma unroll
            for (int u = 0; u < 2 * kUnroll; ++u)
                sl.a[u] = __builtin_nontemporal_load(xv + g * G + u * kThreads + t);
        },
        [&](int64_t g, const AddcSlot& sl) {
#pragma unroll
            for (int u = 0; u < 2 * kUnroll; ++u)
                __builtin_nontemporal_store(sl.a[u] + c, zv + g * G + u * kThreads + t);
        });
    for (int64_t i = groups * G + t; i < nv; i += kThreads) zv[i] = xv[i] + c;
    for (int64_t e = (nv << 2) + t; e < len; e += kThreads) z[start + e] = x[start + e] + c;
}

__global__ __launch_bounds__(kThreads) void addc_scalar_path_kernel(const float* x, float c,
                                                                    float* z, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        z[i] = x[i] + c;
}

// Quickstart "Your first kernel": fill with a constant.
__global__ __launch_bounds__(kThreads) void fill_kernel(float* o, float v, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) o[i] = v;
}

// Quickstart "Parallel work with a grid": each workgroup finds its own slice
// from its block index (blocks are unordered) and writes arange values.
__global__ __launch_bounds__(kThreads) void iota_kernel(float* o, int64_t n, int64_t per_block) {
    const int64_t start = (int64_t)blockIdx.x * per_block;
    const int64_t end = min(start + per_block, n);
    for (int64_t i = start + threadIdx.x; i < end; i += kThreads) o[i] = (float)i;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int grid_for(int64_t n) {
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 65536) g = 65536;
    return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_stream_add(const float* x, const float* y, float* z, int64_t n,
                             int64_t block_elems, hipStream_t stream) {
    if (aligned16(x) && aligned16(y) && aligned16(z)) {
        const int64_t blocks = (n + block_elems - 1) / block_elems;
        hipLaunchKernelGGL(add_vec_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, y,
                           z, n, block_elems);
    } else {
        hipLaunchKernelGGL(add_scalar_path_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, x,
                           y, z, n);
    }
    return hipGetLastError();
}

hipError_t launch_stream_add_scalar(const float* x, float c, float* z, int64_t n,
                                    hipStream_t stream) {
    if (aligned16(x) && aligned16(z)) {
        const int64_t block = kStreamScalarBlock;
        const int64_t blocks = (n + block - 1) / block;
        hipLaunchKernelGGL(addc_vec_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, c,
                           z, n, block);
    } else {
        hipLaunchKernelGGL(addc_scalar_path_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, x,
                           c, z, n);
    }
    return hipGetLastError();
}

hipError_t launch_fill(float* o, float v, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, o, v, n);
    return hipGetLastError();
}

hipError_t launch_iota(float* o, int64_t n, hipStream_t stream) {
    // 128 elements per workgroup as in the quickstart's grid=(8,) example,
    // widened for large n so that the launch stays within kMaxGridBlocks
    // workgroups (grid size times workgroup size below 2^32).
    int64_t per_block = 128;
    while ((n + per_block - 1) / per_block > kMaxGridBlocks) per_block *= 2;
    const int64_t blocks = (n + per_block - 1) / per_block;
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, o, n,
                       per_block);
    return hipGetLastError();
}

}  // namespace pgemm
