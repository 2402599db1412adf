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
// Each lane issues all of its 16-byte loads for an unrolled group before any
// add (copy_start early), adds once the data is back (copy_wait late) and
// stores; the loads of other workgroups overlap those stores.  With the
// default block (4096 elements for x + y, 8192 for x + c) every lane does
// exactly one such group.  Loads and stores are non-temporal: the data is
// touched once, so it should not displace anything in the caches.
// Arithmetic is one IEEE binary32 add per element (v_add_f32, RNE, denormals
// kept), so results are bit-identical to any IEEE implementation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pgemm {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte loads in flight per operand per lane

// One workgroup per block of `block` elements (block is a multiple of 1024,
// so a block starts 16-byte aligned whenever the arrays do).  The last block
// may be ragged; its scalar tail is handled by the same workgroup.
__global__ __launch_bounds__(kThreads) void add_vec_kernel(const float* x, const float* y,
                                                           float* z, int64_t n, int64_t block) {
    const int64_t start = (int64_t)blockIdx.x * block;
    const int64_t len = min(block, n - start);
    const int64_t nv = len >> 2;  // whole float4s in this block
    const floatx4* xv = reinterpret_cast<const floatx4*>(x + start);
    const floatx4* yv = reinterpret_cast<const floatx4*>(y + start);
    floatx4* zv = reinterpret_cast<floatx4*>(z + start);

    int64_t i = threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < nv; i += kUnroll * kThreads) {
        floatx4 a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            a[u] = __builtin_nontemporal_load(xv + i + u * kThreads);
            b[u] = __builtin_nontemporal_load(yv + i + u * kThreads);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(a[u] + b[u], zv + i + u * kThreads);
    }
    for (; i < nv; i += kThreads) zv[i] = xv[i] + yv[i];
    for (int64_t e = (nv << 2) + threadIdx.x; e < len; e += kThreads)
        z[start + e] = x[start + e] + y[start + e];
}

// Any alignment: one element per lane per iteration.
__global__ __launch_bounds__(kThreads) void add_scalar_path_kernel(const float* x, const float* y,
                                                                   float* z, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        z[i] = x[i] + y[i];
}

__global__ __launch_bounds__(kThreads) void addc_vec_kernel(const float* x, float c, float* z,
                                                            int64_t n, int64_t block) {
    const int64_t start = (int64_t)blockIdx.x * block;
    const int64_t len = min(block, n - start);
    const int64_t nv = len >> 2;
    const floatx4* xv = reinterpret_cast<const floatx4*>(x + start);
    floatx4* zv = reinterpret_cast<floatx4*>(z + start);

    int64_t i = threadIdx.x;
    for (; i + (2 * kUnroll - 1) * kThreads < nv; i += 2 * kUnroll * kThreads) {
        floatx4 a[2 * kUnroll];
#pragma unroll
        for (int u = 0; u < 2 * kUnroll; ++u) a[u] = __builtin_nontemporal_load(xv + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < 2 * kUnroll; ++u) __builtin_nontemporal_store(a[u] + c, zv + i + u * kThreads);
    }
    for (; i < nv; i += kThreads) zv[i] = xv[i] + c;
    for (int64_t e = (nv << 2) + threadIdx.x; e < len; e += kThreads)
        z[start + e] = x[start + e] + c;
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
    // widened for large n so the grid stays below 2^31 workgroups.
    int64_t per_block = 128;
    while ((n + per_block - 1) / per_block > (int64_t)1 << 30) per_block *= 2;
    const int64_t blocks = (n + per_block - 1) / per_block;
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, o, n,
                       per_block);
    return hipGetLastError();
}

}  // namespace pgemm
