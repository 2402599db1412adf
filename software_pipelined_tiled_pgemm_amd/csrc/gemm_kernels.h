// Software-pipelined tiled fp16 GEMM for gfx950 (CDNA4): the kernels.
// Included by gemm_f16.hip (32x32x16 variants, shape chooser) and
// gemm_f16_m16.hip (16x16x32 variants, split-K), which are compiled with
// different code-generation options.
//
// What it computes: C[M,N] = A[M,K] . B[K,N], fp16 in, fp32 accumulation, fp16
// out (round to nearest even) -- the matmul of the Pallas "Quickstart: GPU"
// page, section "Pipelining: a matmul kernel".  How, in the pages' terms:
//
//  * Parallel grid (quickstart, same section; Chinese quickstart, section
//    "Hopper 上的矩阵乘法内核"): one workgroup per BM x BN output tile; tiles
//    are independent and unordered.  The block id is remapped so that the
//    tiles one XCD runs share rows of A and columns of B in that XCD's L2.
//  * Sequential K pipeline (the emit_pipeline grid over K): each step
//    consumes an A slice [BM, BK] and a B slice [BK, BN] from LDS.
//  * copy_start early / copy_wait late with several buffers (Pallas
//    software-pipelining guide, section 4; max_concurrent_steps of the
//    quickstart's emit_pipeline).  Two pipelines are implemented:
//      - LDS-DMA pipeline (variants 1, 2, 5, 7, 8, 9 -- the persistent
//        form of 8 -- and 10, 11): a ring of 5 LDS stages of BK = 32 (7 or
//        9 in variants 10 and 11).  copy_start is a buffer_load ... lds
//        (global memory straight into LDS, no registers), issued up to S-1
//        steps ahead for a ring of S stages and spread over the MFMA
//        slots; copy_wait is an s_waitcnt on this wave's own copies followed
//        by the workgroup barrier.
//      - register-staged pipeline (variants 3, 4): 2 LDS stages of BK = 64
//        plus one register stage; global loads for step k+2 are in flight
//        while step k computes.
//  * Buffer release (the quickstart's delay_release discussion): an LDS
//    stage is refilled only after every wave has passed the barrier that
//    follows its last ds_read of it.  MFMA operands are VGPRs, so no matrix
//    instruction can still be reading LDS at that point.
//  * fp32 accumulator in registers (the quickstart's ACC): 32x32 or 16x16
//    MFMA blocks held in VGPR/AGPR for the whole K loop, zeroed before step 0
//    (the initialise-before-accumulate rule of the guide, section 7.2).
//  * Drain (quickstart's epilogue: cast, stage through shared memory, copy
//    out): fp32 -> fp16, written to LDS (the whole tile, or bands of rows
//    on the 16x16x32 path), then 16-byte coalesced non-temporal row stores.
//
// Matrix instructions: v_mfma_f32_32x32x16_f16 (variants 1-6: 32x32 output
// block, 16-deep K, 8 fp16 per lane per operand; lanes 0-31 carry K 0..7,
// lanes 32-63 K 8..15) and v_mfma_f32_16x16x32_f16 (variants 7-11: 16x16
// block, the whole K 32 of a stage; see Compute<TL, 16>).  Each MFMA computes
// the transposed block C^T = B^T A^T (B^T as the row operand), so that each
// lane ends up holding four consecutive columns of one row of C -- 8
// contiguous bytes for the epilogue.  Within one instruction family every
// variant feeds the MFMAs the same K blocks in the same order, so its
// variants produce bit-identical results.
//
// Edge tiles: buffer loads return zero outside the matrix (rows >= M,
// K >= K, columns >= N); stores are masked.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "internal.h"

namespace pgemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(8)));
#define LDS_AS __attribute__((address_space(3)))

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset that reads as zero
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Raw buffer descriptor as four dwords (base, stride 0, size in bytes, gfx9
// format word), for use as an SGPR quad operand.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = (uint32_t)a;
    r[1] = (uint32_t)(a >> 32) & 0xFFFFu;
    r[2] = bytes <= 0 ? 0u : (uint32_t)bytes;
    r[3] = (uint32_t)kRsrcWord3;
    return r;
}

// One 16-byte-per-lane copy from global memory straight into LDS: lane l's
// 16 bytes at buffer offset `off` land at LDS byte address lds + 16*l; an
// offset past the buffer size writes zeros.  Written as inline assembly so
// the compiler does not treat later LDS reads as possibly aliasing it and
// wait for every copy in flight: the pipeline orders copies and reads itself,
// with explicit vmcnt waits and workgroup barriers.  M0 is clobbered and
// reloaded by every copy; the compiler warns that it will not preserve M0
// across the statement, which is harmless here because no other code in
// these kernels uses M0 (every M0 access in the generated assembly is one of
// these copies' own s_mov).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t off, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(off), "s"(rsrc), "s"(lds)
        : "memory", "m0");
}
// The same copy with an SGPR offset added to the address.  Used only where
// every lane's address lies inside the matrix, so it does not matter whether
// the descriptor's range check includes that offset.
__device__ __forceinline__ void dma16s(u32x4 rsrc, uint32_t off, uint32_t soff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(off), "s"(rsrc), "s"(soff), "s"(lds)
        : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const LDS_AS char*)p;
}

// Race-detection build (PGEMM_POISON_LDS=1, never the product): right after
// the barrier that releases a ring stage, the workgroup fills it with fp16
// NaN and passes one more barrier before any copy may refill it.  A read of
// the stage after its release -- the overwrite the quickstart's
// delay_release guards against -- then yields NaN in C instead of a silently
// wrong value.  `threads` lanes (all of the workgroup's) share the writes.
#ifndef PGEMM_POISON_LDS
#define PGEMM_POISON_LDS 0
#endif

template <int BYTES, int THREADS>
__device__ __forceinline__ void poison_stage(char* stage, int tid) {
    const u32x4 nan4 = {0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u};
    for (int o = tid * 16; o < BYTES; o += THREADS * 16)
        *reinterpret_cast<u32x4*>(stage + o) = nan4;
}

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left at their "no wait" maxima),
// gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ floatx16 mfma(half8 row_op, half8 col_op, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(row_op, col_op, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_f16: 16x16 output block, the whole K 32 of a stage in
// one instruction.  Row operand: lane l holds row l%16, K 8(l/16)..+7; column
// operand: lane l holds column l%16, the same K values; result: lane l holds
// rows 4(l/16)..+3 of column l%16 (layout checked on gfx950 with an exact
// small-integer product).  On random fp16 data it runs at the same rate per
// cycle as the 32x32x16 form but at a markedly higher clock under the power
// limit (measured: 1.94 vs 1.65 GHz with all 256 CUs busy): it moves half the
// fp32 accumulator bytes per multiply-add.
__device__ __forceinline__ floatx4 mfma16(half8 row_op, half8 col_op, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(row_op, col_op, c, 0, 0, 0);
}

// Block id -> output tile (nwg = tiles_m * tiles_n, the grid's x extent,
// passed from the explicit arguments so that no kernel reads a hidden
// argument).  Workgroups are dealt to the 8 XCDs round-robin,
// so id b runs on XCD b % 8; the first remap gives each XCD a contiguous
// range of logical tiles.  The second walks tiles in column-major order
// inside bands of `group_m` tile rows, so a contiguous range covers a compact
// block of tiles (shared A rows and B columns).
__device__ __forceinline__ void tile_of_block(int b, int nwg, int tiles_m, int tiles_n,
                                              int group_m, int& tm, int& tn) {
    const int per = nwg >> 3;
    const int full = per << 3;
    const int t = (b < full) ? ((b & 7) * per + (b >> 3)) : b;
    const int band = group_m * tiles_n;
    const int g = t / band;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = t - g * band;
    tm = first_m + r % gm;
    tn = r / gm;
}

template <int BM, int BN, int T>
__device__ __forceinline__ void store_tile(const char* smem, _Float16* C, int M, int N, int m0,
                                           int n0, int tid);

// Drain: fp32 -> fp16 (RNE) into an LDS copy of the BM x BN tile, then
// 16-byte row stores.  Lane (lr, lk) of block (j, i) holds row wm*TM+i*32+lr
// and columns wn*TN+j*32+8g+4lk+q for accumulator element 4g+q.  The 16-byte
// chunk c of LDS row r sits at chunk position c ^ (r mod chunks-per-row), so
// the 32 lanes writing one column chunk of 32 rows spread over the banks.
// Pairs of values are converted with one packed RNE conversion
// (v_cvt_pk_f16_f32).  Tiles fully inside C store without per-store masks.
template <int BM, int BN, int TM, int TN, int FM, int FN, int T>
__device__ __forceinline__ void drain(char* smem, floatx16 (&acc)[FN][FM], _Float16* C, int M,
                                      int N, int m0, int n0, int tid, int wm, int wn) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    constexpr int CH = BN / 8;  // 16-byte chunks per C row
    const int lane = tid & 63;
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * TM + i * 32 + lr;
            char* rowp = smem + row * (BN * 2) + lk * 8;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int chunk = (wn * TN + j * 32) / 8 + g;
                const int pchunk = chunk ^ (row & (CH - 1));
                const half2_t h01 = __builtin_convertvector(
                    (float2_t{acc[j][i][4 * g + 0], acc[j][i][4 * g + 1]}), half2_t);
                const half2_t h23 = __builtin_convertvector(
                    (float2_t{acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]}), half2_t);
                u32x2 v;
                v[0] = __builtin_bit_cast(uint32_t, h01);
                v[1] = __builtin_bit_cast(uint32_t, h23);
                *reinterpret_cast<u32x2*>(rowp + pchunk * 16) = v;
            }
        }
    __syncthreads();
    store_tile<BM, BN, T>(smem, C, M, N, m0, n0, tid);
}

// Second half of a drain: the fp16 tile in LDS (16-byte chunk c of row r at
// c ^ (r mod chunks-per-row)) to C with 16-byte row stores.
// Thread t stores chunk t % CH of rows t / CH + (T / CH) * r.  The stores are
// non-temporal: this kernel never reads C, and streaming it out keeps the
// caches for the operand tiles that other workgroups still fetch.
template <int BM, int BN, int T>
__device__ __forceinline__ void store_tile(const char* smem, _Float16* C, int M, int N, int m0,
                                           int n0, int tid) {
    constexpr int CH = BN / 8;  // 16-byte chunks per C row
    constexpr int RSTEP = T / CH;
    const int chunk = tid % CH, row0 = tid / CH;
    const char* src = smem + row0 * (BN * 2);
    _Float16* dst = C + (int64_t)(m0 + row0) * N + n0 + chunk * 8;
    const int64_t dstep = (int64_t)RSTEP * N;
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    if (interior) {
#pragma unroll
        for (int r = 0; r < BM / RSTEP; ++r) {
            const int row = row0 + RSTEP * r;
            const int pchunk = chunk ^ (row & (CH - 1));
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(src + r * RSTEP * (BN * 2) + pchunk * 16);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + r * dstep));
        }
    } else {
        const bool col_ok = n0 + chunk * 8 < N;
#pragma unroll
        for (int r = 0; r < BM / RSTEP; ++r) {
            const int row = row0 + RSTEP * r;
            const int pchunk = chunk ^ (row & (CH - 1));
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(src + r * RSTEP * (BN * 2) + pchunk * 16);
            if (col_ok && m0 + row < M)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + r * dstep));
        }
    }
}

// Split-K drain: the fp32 partial tile to row-major fp32 (pitch N) at W,
// through LDS one band of wave rows (TM rows) at a time: the waves of band r
// write their blocks (lane (lr, lk) of block (j, i) holds 4 consecutive
// columns of one row), then every thread stores 16-byte row chunks.  The
// 16-byte chunk c of LDS row r sits at c ^ (r mod chunks-per-row).
template <int BN, int TM, int TN, int FM, int FN, int T, int WM>
__device__ __forceinline__ void drain_f32(char* smem, floatx16 (&acc)[FN][FM], float* W, int M,
                                          int N, int m0, int n0, int tid, int wm, int wn) {
    constexpr int CH = BN / 4;     // 16-byte chunks per fp32 row
    constexpr int ROWB = BN * 4;   // bytes per LDS row
    constexpr int RSTEP = T / CH;  // rows per store pass
    static_assert(TM % RSTEP == 0, "store passes cover the band");
    const int lane = tid & 63;
    const int lr = lane & 31, lk = lane >> 5;
    const int chunk = tid % CH, row0 = tid / CH;
    const bool col_ok = n0 + chunk * 4 < N;
#pragma unroll
    for (int r = 0; r < WM; ++r) {
        if (wm == r) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = i * 32 + lr;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c = (wn * TN + j * 32) / 4 + 2 * g + lk;
                        const floatx4 v = {acc[j][i][4 * g + 0], acc[j][i][4 * g + 1],
                                           acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]};
                        *reinterpret_cast<floatx4*>(smem + row * ROWB + (c ^ (row & (CH - 1))) * 16) = v;
                    }
                }
        }
        __syncthreads();
        const int grow0 = m0 + r * TM;
#pragma unroll
        for (int q = 0; q < TM / RSTEP; ++q) {
            const int row = row0 + RSTEP * q;
            const floatx4 v =
                *reinterpret_cast<const floatx4*>(smem + row * ROWB + (chunk ^ (row & (CH - 1))) * 16);
            if (col_ok && grow0 + row < M)
                *reinterpret_cast<floatx4*>(W + (int64_t)(grow0 + row) * N + n0 + chunk * 4) = v;
        }
        __syncthreads();
    }
}

// Drain of 16x16 accumulator blocks, lane (r, g) = (l % 16, l / 16) of block
// (j, i) holding row wm*TM + 16i + r, columns wn*TN + 16j + 4g .. +3, through
// STAGE_BYTES of LDS at `stage`: bands of RB = STAGE_BYTES / (2 BN) rows, each
// written by the waves that hold it (fp16, RNE, in the LDS tile layout of
// drain() with band-local rows) and then stored by every thread as in
// store_tile.  The stores of one band are in flight while the next band is
// converted, and a persistent kernel keeps the other ring stages free for
// the copies of its next tile.
template <int BM, int BN, int TM, int TN, int FM, int FN, int T, int STAGE_BYTES>
__device__ __forceinline__ void drain16_bands(char* stage, floatx4 (&acc)[FN][FM], _Float16* C,
                                              int M, int N, int m0, int n0, int tid, int wm,
                                              int wn) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    constexpr int CH = BN / 8;
    constexpr int RB = STAGE_BYTES / (BN * 2);  // rows per band
    static_assert(RB % 32 == 0 && TM % RB == 0, "bands of whole blocks inside one wave row");
    constexpr int BPW = TM / RB;  // bands per wave row
    const int lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int p = 0; p < BM / RB; ++p) {
        if (wm == p / BPW) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int ii = 0; ii < RB / 16; ++ii) {
                    const int i = (p % BPW) * (RB / 16) + ii;
                    const int row = ii * 16 + r;
                    const int chunk = (wn * TN + j * 16) / 8 + (g >> 1);
                    const int pchunk = chunk ^ (row & (CH - 1));
                    const half2_t h01 =
                        __builtin_convertvector((float2_t{acc[j][i][0], acc[j][i][1]}), half2_t);
                    const half2_t h23 =
                        __builtin_convertvector((float2_t{acc[j][i][2], acc[j][i][3]}), half2_t);
                    u32x2 v;
                    v[0] = __builtin_bit_cast(uint32_t, h01);
                    v[1] = __builtin_bit_cast(uint32_t, h23);
                    *reinterpret_cast<u32x2*>(stage + row * (BN * 2) + pchunk * 16 + (g & 1) * 8) =
                        v;
                }
        }
        __syncthreads();
        store_tile<RB, BN, T>(stage, C, M, N, m0 + p * RB, n0, tid);
        if (p + 1 < BM / RB) __syncthreads();
    }
}

// Split-K drain of 16x16 blocks (see drain_f32): a lane's four consecutive
// fp32 columns are exactly one 16-byte chunk of the LDS row.
template <int BN, int TM, int TN, int FM, int FN, int T, int WM>
__device__ __forceinline__ void drain16_f32(char* smem, floatx4 (&acc)[FN][FM], float* W, int M,
                                            int N, int m0, int n0, int tid, int wm, int wn) {
    constexpr int CH = BN / 4;
    constexpr int ROWB = BN * 4;
    constexpr int RSTEP = T / CH;
    static_assert(TM % RSTEP == 0, "store passes cover the band");
    const int lane = tid & 63;
    const int lr = lane & 15, g = lane >> 4;
    const int chunk = tid % CH, row0 = tid / CH;
    const bool col_ok = n0 + chunk * 4 < N;
#pragma unroll
    for (int b = 0; b < WM; ++b) {
        if (wm == b) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = i * 16 + lr;
                    const int c = (wn * TN + j * 16) / 4 + g;
                    *reinterpret_cast<floatx4*>(smem + row * ROWB + (c ^ (row & (CH - 1))) * 16) =
                        acc[j][i];
                }
        }
        __syncthreads();
        const int grow0 = m0 + b * TM;
#pragma unroll
        for (int q = 0; q < TM / RSTEP; ++q) {
            const int row = row0 + RSTEP * q;
            const floatx4 v = *reinterpret_cast<const floatx4*>(
                smem + row * ROWB + (chunk ^ (row & (CH - 1))) * 16);
            if (col_ok && grow0 + row < M)
                *reinterpret_cast<floatx4*>(W + (int64_t)(grow0 + row) * N + n0 + chunk * 4) = v;
        }
        __syncthreads();
    }
}

// ===========================================================================
// LDS-DMA pipeline: 5-stage LDS ring, BK = 32, copies straight into LDS.
// ===========================================================================
namespace dm {

constexpr int BK = 32;
constexpr int STAGES = 5;
constexpr int A_ROW = BK * 2;  // bytes per A row in a stage

// The copy engine fetches whole 128-byte lines, four lanes (64 bytes) at a
// time.  A copy runs at full rate (about 58 bytes per clock per CU, measured)
// only when every four consecutive lanes read one 64-byte segment and both
// halves of each line are read within a few instructions; with 64-byte row
// pieces or quads that straddle two rows it runs at about half that.  Both
// layouts below are chosen for this:
//  * A rows are 64 bytes per stage, so the A copies of steps 2j and 2j+1 are
//    issued in pairs, back to back: the two halves of the same lines.
//  * B rows are copied whole, lanes running along the row.

// A stage: row-major [BM][32] fp16, 64-byte rows of four 16-byte chunks;
// logical chunk c of row r is stored at chunk position c ^ aswz(r).  A
// fragment read touches one logical chunk of 32 consecutive rows.  Without a
// swizzle, rows r, r+4, r+8 and r+12 collide on the same LDS banks (four-way
// conflicts); XORing the chunk index with bits 2-3 of the row puts those
// rows on different chunk positions.  This choice was measured conflict-free
// on gfx950 (bank-conflict counter), while e.g. ((r>>1)^(r>>3))&3 is still
// two-way.  The copies keep 4 consecutive lanes on one 64-byte row segment,
// so the global reads stay coalesced.
__device__ __forceinline__ int aswz(int row) { return (row >> 2) & 3; }

// B stage: row-major [32][BN] fp16 (K rows of BN*2 bytes); the 64-byte group
// g of row r is stored at group position g ^ (r & 3), i.e. 16-byte chunk c at
// c ^ bswz(r).  One ds_read_b64_tr_b16 of 16 lanes reads 4 K rows x 16
// columns: lane i reads the 8 bytes of row i/4, columns 4(i%4)..+3, and the
// transposing read hands lane j column j with its 4 consecutive K values --
// the MFMA operand layout.  A wave reads 64 contiguous logical bytes of each
// of rows 4q..4q+3 (and of 4q+8..4q+11); the swizzle spreads those rows over
// the four 64-byte bank groups, so the read is conflict-free.  The XOR moves
// whole 64-byte groups, so each lane quad of a copy still reads one 64-byte
// global segment.
__device__ __forceinline__ int bswz(int row) { return (row & 3) << 2; }

// B stage swizzle of the 16x16x32 path.  Its transposing read takes, per
// 16-lane group, K rows 8g..8g+3 (g = lane / 16) x 16 columns (32 bytes a
// row), so the rows of two neighbouring groups (r and r + 8) share the
// 64-byte group positions that bswz gives; XORing chunk bit 1 with row bit 3
// moves the second group to the other 32-byte half of each 64-byte group,
// and 32 lanes cover all banks once.  Whole 64-byte groups still move as a
// unit, so each lane quad of a copy still reads one 64-byte global segment.
__device__ __forceinline__ int bswz16(int row) { return ((row & 3) << 2) | (((row >> 3) & 1) << 1); }

// A stage swizzle of the 16x16x32 path.  Its fragment read has 16 lanes take
// one logical chunk of 16 consecutive rows (four such groups per wave).
// Measured with the LDS bank-conflict counter on gfx950: XORing the chunk
// index with row bits 2-3 (aswz) or 0-1, or not at all, costs about 4
// conflict cycles per read; XORing it with row bits 1-2 costs none.
__device__ __forceinline__ int aswz16(int row) { return (row >> 1) & 3; }

// MF: MFMA shape, 32 (v_mfma_f32_32x32x16_f16) or 16 (v_mfma_f32_16x16x32_f16).
// S: stages in the LDS ring (odd, at least 5); copies run S-1 steps ahead.
template <int BM_, int BN_, int WM_ = 2, int WN_ = 2, int MF_ = 32, int S_ = STAGES>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WM = WM_, WN = WN_;  // waves along M and N
    static constexpr int MF = MF_;
    static constexpr int S = S_;
    static constexpr int T = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int FM16 = TM / 16, FN16 = TN / 16;  // 16x16 blocks per wave
    __device__ static __forceinline__ int bsw(int row) { return MF == 16 ? bswz16(row) : bswz(row); }
    __device__ static __forceinline__ int asw(int row) { return MF == 16 ? aswz16(row) : aswz(row); }
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int B_ROW = BN * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = S * STAGE;
    static constexpr int A_CP = A_BYTES / 1024 / (WM * WN);  // 1 KiB copies per wave per step
    static constexpr int B_CP = B_BYTES / 1024 / (WM * WN);
    static constexpr int CP = A_CP + B_CP;
    static constexpr int H = CP / 2;  // copies per half-step
    static_assert(BM * BN * 2 <= LDS, "epilogue tile must fit in the stage ring");
    static_assert(A_CP == H && B_CP == H && A_CP % 2 == 0,
                  "the copy schedule issues one operand per half-step, A in pairs");
    static_assert(LDS <= 160 * 1024, "LDS of one CU");
    static_assert(S % 2 == 1 && S >= 5, "the copy schedule pairs aligned steps: odd S >= 5");
    // vmcnt thresholds of the two waits of a period (see the copy schedule).
    static constexpr int W0 = H * (2 * S - 5);
    static constexpr int W1 = 2 * H * (S - 3);
    static_assert(2 * H * (S - 1) < 64, "copies in flight within the vmcnt range");
    static_assert(FM * FN >= 2 * H, "every copy gets its own MFMA slot");
    static_assert(MF == 32 || (FN16 % 2 == 0 && (FN16 / 2) * FM16 >= H), "16x16x32 halves");
};

template <class TL>
struct Copier {
    // Per-lane byte offsets of this wave's copies, relative to the tile
    // origin at K = 0, plus the K coordinate (A) that decides whether the
    // piece lies inside the matrix; B pieces past column N read as zeros.
    uint32_t a_off[TL::A_CP];
    int a_k[TL::A_CP];
    uint32_t b_off[TL::B_CP];
    int lda;  // row pitch of A in elements (K, or the full K of a K-chunk view)

    __device__ __forceinline__ void init(int lane, int wave, int lda_, int N, int n0) {
        lda = lda_;
#pragma unroll
        for (int t = 0; t < TL::A_CP; ++t) {
            const int p = (wave * TL::A_CP + t) * 64 + lane;  // 16-byte chunk in the A stage
            const int row = p >> 2;
            const int c = (p & 3) ^ TL::asw(row);
            a_off[t] = (uint32_t)((row * lda + c * 8) * 2);
            a_k[t] = c * 8;
        }
#pragma unroll
        for (int t = 0; t < TL::B_CP; ++t) {
            const int p = (wave * TL::B_CP + t) * 64 + lane;  // 16-byte chunk in the B stage
            const int row = p / (TL::B_ROW / 16);
            const int c = (p % (TL::B_ROW / 16)) ^ TL::bsw(row);
            const int n = c * 8;
            b_off[t] = (n0 + n < N) ? (uint32_t)((row * N + n) * 2) : kOOB;
        }
    }
    // A copy t of step k0 into the stage at LDS byte address `stage`; K is
    // the extent (pieces at K and beyond read as zeros), lda the row pitch.
    __device__ __forceinline__ void issue_a(int t, const _Float16* A, int M, int K, int m0, int k0,
                                            uint32_t stage, int wave) const {
        const int rows_valid = min(TL::BM, M - m0);
        const u32x4 ra =
            rsrc_words(A + (int64_t)m0 * lda + k0, ((int64_t)rows_valid * lda - k0) * 2);
        const uint32_t off = (a_k[t] < K - k0) ? a_off[t] : kOOB;
        dma16(ra, off, stage + (wave * TL::A_CP + t) * 1024);
    }
    // B copy t of step k0 into the stage at LDS byte address `stage`.
    __device__ __forceinline__ void issue_b(int t, const _Float16* B, int N, int K, int n0, int k0,
                                            uint32_t stage, int wave) const {
        const int kv = min(BK, K - k0);
        const u32x4 rb = rsrc_words(B + (int64_t)k0 * N + n0, ((int64_t)kv * N - n0) * 2);
        dma16(rb, b_off[t], stage + TL::A_BYTES + (wave * TL::B_CP + t) * 1024);
    }

    // Steady-state copies, for steps whose K range [k0, k0 + BK) lies inside
    // K.  They need no per-lane K test and almost no scalar work: A goes
    // through one descriptor over the tile's rows from K = 0 with the step's
    // byte offset 2*k0 in an SGPR; B through a descriptor at the step's first
    // row whose size is constant (BK rows).  Rows past M and columns past N
    // still fall outside the descriptors and read as zeros.
    u32x4 ra_fix;
    uint32_t b_size;
    __device__ __forceinline__ void init_fast(const _Float16* A, int M, int m0, int N, int n0) {
        const int rows_valid = min(TL::BM, M - m0);
        ra_fix = rsrc_words(A + (int64_t)m0 * lda, (int64_t)rows_valid * lda * 2);
        b_size = (uint32_t)(((int64_t)BK * N - n0) * 2);
    }
    // A copy t of the step at byte offset a_byte (2*k0) into `stage`.
    __device__ __forceinline__ void fast_a(int t, uint32_t a_byte, uint32_t stage, int wave) const {
        dma16s(ra_fix, a_off[t], a_byte, stage + (wave * TL::A_CP + t) * 1024);
    }
    // B copy t of the step whose rows start at bk (B + k0*N + n0) into `stage`.
    __device__ __forceinline__ void fast_b(int t, const _Float16* bk, uint32_t stage, int wave) const {
        const uint64_t a = reinterpret_cast<uint64_t>(bk);
        u32x4 rb;
        rb[0] = (uint32_t)a;
        rb[1] = (uint32_t)(a >> 32) & 0xFFFFu;
        rb[2] = b_size;
        rb[3] = (uint32_t)kRsrcWord3;
        dma16(rb, b_off[t], stage + TL::A_BYTES + (wave * TL::B_CP + t) * 1024);
    }
};

// Operand fragments of sub-step s (K values 16s .. 16s+15 of the stage).
// A: lane (lr, lk) reads row lr of 32-row block i, K values 16s+8lk .. +7.
template <class TL>
__device__ __forceinline__ half8 read_a(const char* stage, int s, int i, int wm, int lane) {
    const int lr = lane & 31, lk = lane >> 5;
    const char* pa = stage + (wm * TL::TM + lr) * A_ROW + (((2 * s + lk) ^ aswz(lr)) * 16);
    return *reinterpret_cast<const half8*>(pa + i * 32 * A_ROW);
}

// B: lane l takes column 16*((l>>4)&1) + (l&15) of 32-column block j and K
// values 16s+8lk .. +7 (two transposing reads of 4 K rows each).
template <class TL>
__device__ __forceinline__ half8 read_b(const char* stage, int s, int j, int wn, int lane) {
    const int lk = lane >> 5, i = lane & 15;
    const int nb = (wn * TL::TN) / 16 + 2 * j + ((lane >> 4) & 1);  // 16-column block
    const int row = 16 * s + 8 * lk + (i >> 2);
    const int c = (2 * nb + ((i >> 1) & 1)) ^ bswz(row);
    const char* q = stage + TL::A_BYTES + row * TL::B_ROW + c * 16 + (i & 1) * 8;
    const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS fp16x4_t*)q);
    const fp16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS fp16x4_t*)(q + 4 * TL::B_ROW));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(half8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// The operand reads of one sub-step, in the order the next half-step's MFMAs
// consume them (B block 0 and every A block first, then the other B blocks):
// unit u < FM+FN of the read sequence.
template <class TL>
__device__ __forceinline__ void read_unit(int u, const char* stage, int s, int wm, int wn, int lane,
                                          half8 (&fa)[TL::FM], half8 (&fb)[TL::FN]) {
    if (u == 0)
        fb[0] = read_b<TL>(stage, s, 0, wn, lane);
    else if (u <= TL::FM)
        fa[u - 1] = read_a<TL>(stage, s, u - 1, wm, lane);
    else
        fb[u - TL::FM] = read_b<TL>(stage, s, u - TL::FM, wn, lane);
}

// One half-step: the FN x FM MFMAs on (fa, fb), j-major, with the operand
// reads of the next half-step (into na, nb) placed one per MFMA slot from the
// first slot on, and NC copies (copy(0) .. copy(NC-1), global->LDS; NC = H
// in the dm kernel, 0 for the MFMA waves of the wave-specialised one) spread
// evenly over the slots (copy c after MFMA (2c+1)*NS/(2NC)).  sched_barrier pins the order, so every read has most of
// a half-step to land before its first use and the copies issue in the
// matrix unit's shadow.
template <class TL, int NC = TL::H, class CopyFn>
__device__ __forceinline__ void half_step(floatx16 (&acc)[TL::FN][TL::FM], const half8 (&fa)[TL::FM],
                                          const half8 (&fb)[TL::FN], const char* rstage, int rs,
                                          half8 (&na)[TL::FM], half8 (&nb)[TL::FN], int wm, int wn,
                                          int lane, CopyFn copy) {
    constexpr int NR = TL::FM + TL::FN;  // read units
    constexpr int NS = TL::FM * TL::FN;  // MFMA slots
    constexpr int ND = NC > 0 ? NC : 1;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int j = q / TL::FM, i = q % TL::FM;
        acc[j][i] = mfma(fb[j], fa[i], acc[j][i]);
        if (q < NR) read_unit<TL>(q, rstage, rs, wm, wn, lane, na, nb);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (q == (2 * c + 1) * NS / (2 * ND)) copy(c);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---- 16x16x32 path ------------------------------------------------------
// A fragment (column operand) of 16-row block i: lane (r, g) = (l % 16,
// l / 16) reads row 16i + r of the wave's rows, K values 8g .. 8g+7 of the
// stage (one 16-byte chunk), stored at chunk position g ^ aswz16(row).  Row
// bases are multiples of 16, so the swizzle depends on r only.
template <class TL>
__device__ __forceinline__ half8 read_a16(const char* stage, int i, int wm, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const char* pa = stage + (wm * TL::TM + r) * A_ROW + ((g ^ aswz16(r)) * 16);
    return *reinterpret_cast<const half8*>(pa + i * 16 * A_ROW);
}

// B fragment (row operand) of 16-column block j: lane (c, g) takes column c
// of the block and K values 8g .. 8g+7, from two transposing reads of 4 K
// rows each (lane c of a 16-lane group points at row 8g + c/4, columns
// 4(c%4) .. +3, and receives column c).
template <class TL>
__device__ __forceinline__ half8 read_b16(const char* stage, int j, int wn, int lane) {
    const int c = lane & 15, g = lane >> 4;
    const int nb = (wn * TL::TN) / 16 + j;  // 16-column block
    const int row = 8 * g + (c >> 2);
    const int ch = (2 * nb + ((c >> 1) & 1)) ^ bswz16(row);
    const char* q = stage + TL::A_BYTES + row * TL::B_ROW + ch * 16 + (c & 1) * 8;
    const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS fp16x4_t*)q);
    const fp16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS fp16x4_t*)(q + 4 * TL::B_ROW));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(half8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// MFMA slot (of NS) after which copy c (of NC) of a 16x16x32 half-step is
// issued.  256x256 tile: spread evenly, copy c after slot (2c+1)NS/(2NC).
// 128x128 tile (one MFMA wave per SIMD, 8 slots per half): the copies go
// into the second-to-last slots (5 and 6), after the half's operand reads.
// Measured on MI355X against the even spread: 2048^2 x 32768 +2.3%,
// 1024 x 8192 x 4096 +1.2%, 512 x 4096 x 4096 +1.1%, 2048^3 -0.4%.  For the
// 256x256 tile the spread (slots 4 and 12) is best: offsets 3 and 5 tie,
// 6 loses 0.6%, and 0, 2 or 7 (copies among the half's first reads or right
// before the barrier) lose 8-12%.
template <class TL>
__device__ __forceinline__ constexpr int copy_slot(int c, int nc, int ns) {
    return TL::BM == 128 ? ns - 1 - nc + c : (2 * c + 1) * ns / (2 * (nc > 0 ? nc : 1));
}

// One half of a K step on the 16x16x32 path.  A step's FM16 x FN16 MFMAs
// (all of the stage's K 32) are split by B block: half 0 takes blocks
// j < FN16/2, half 1 the others; inside a half, j-major with i snaking, so
// consecutive MFMAs share an operand.  A fragments are double-buffered (fa:
// this step, na: the next), B fragments single-buffered (fb), read right
// after their last use:
//   half 0 of step kt reads B blocks FN16/2 .. of stage kt (`rstage`), used
//          by half 1 of the same step;
//   half 1 of step kt reads every A block (into na) and B blocks < FN16/2 of
//          stage kt+1 (`rstage`), used by half 0 of step kt+1.
// So every read of a stage is issued between the barrier that publishes it
// (the one in the middle of the previous step) and the one in the middle of
// its own step, which releases the slot -- the same rule as the 32x32x16
// path.  Reads take the first slots in consumption order; the NC copies go
// after the slots copy_slot gives.
template <class TL, int HALF, int NC, class CopyFn>
__device__ __forceinline__ void half16(floatx4 (&acc)[TL::FN16][TL::FM16],
                                       const half8 (&fa)[TL::FM16], half8 (&fb)[TL::FN16],
                                       const char* rstage, half8 (&na)[TL::FM16], int wm, int wn,
                                       int lane, CopyFn copy) {
    constexpr int FM = TL::FM16, JH = TL::FN16 / 2;
    constexpr int NS = JH * FM;                      // MFMA slots
    constexpr int NR = HALF == 0 ? JH : FM + JH;     // read units
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int jj = q / FM, ii = q % FM;
        const int j = HALF * JH + jj;
        const int i = (jj & 1) ? FM - 1 - ii : ii;
        acc[j][i] = mfma16(fb[j], fa[i], acc[j][i]);
        if (q < NR) {
            if (HALF == 0)
                fb[JH + q] = read_b16<TL>(rstage, JH + q, wn, lane);
            else if (q == 0)
                fb[0] = read_b16<TL>(rstage, 0, wn, lane);
            else if (q <= FM)
                na[q - 1] = read_a16<TL>(rstage, q - 1, wm, lane);
            else
                fb[q - FM] = read_b16<TL>(rstage, q - FM, wn, lane);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (q == copy_slot<TL>(c, NC, NS)) copy(c);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int S>
__device__ __forceinline__ int wrap_slot(int s) { return s >= S ? s - S : s; }
__device__ __forceinline__ int wrap5(int s) { return wrap_slot<STAGES>(s); }

// f(j, slot) for the S periods j = 0 .. S-1 of one pass around a ring of S
// (odd) slots, with the slot of period j's first step, 2j mod S, as a
// compile-time constant.
template <int S, class F, int... J>
__device__ __forceinline__ void ring_pass(F&& f, std::integer_sequence<int, J...>) {
    (f(std::integral_constant<int, J>{}, std::integral_constant<int, (2 * J) % S>{}), ...);
}

// The compute side of the pipeline: accumulators, operand fragments, the four
// half-steps of a period and the drain, for either MFMA shape.  Call c of a
// period (c = 0..3: first and second half of step kt, then of kt+1) reads
// from `rstage`: the stage of step kt for c = 0, of kt+1 for c = 1, 2, of
// kt+2 for c = 3.
template <class TL, int MF = TL::MF>
struct Compute;

template <class TL>
struct Compute<TL, 32> {
    floatx16 acc[TL::FN][TL::FM];
    half8 fa[2][TL::FM], fb[2][TL::FN];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < TL::FN; ++j)
#pragma unroll
            for (int i = 0; i < TL::FM; ++i) acc[j][i] = floatx16{};
    }
    // Fragments of step 0, sub-step 0.
    __device__ __forceinline__ void first_reads(const char* stage, int wm, int wn, int lane) {
#pragma unroll
        for (int u = 0; u < TL::FM + TL::FN; ++u)
            read_unit<TL>(u, stage, 0, wm, wn, lane, fa[0], fb[0]);
    }
    // Call c: sub-step c&1 of its step from buffer c&1, reading the other
    // sub-step (1 - (c&1)) of `rstage` into the other buffer.
    template <int CALL, int NC, class CopyFn>
    __device__ __forceinline__ void half(const char* rstage, int wm, int wn, int lane, CopyFn copy) {
        constexpr int b = CALL & 1;
        half_step<TL, NC>(acc, fa[b], fb[b], rstage, 1 - b, fa[b ^ 1], fb[b ^ 1], wm, wn, lane,
                          copy);
    }
    __device__ __forceinline__ void drain_c(char* smem, _Float16* C, int M, int N, int m0, int n0,
                                            int tid, int wm, int wn) {
        drain<TL::BM, TL::BN, TL::TM, TL::TN, TL::FM, TL::FN, TL::T>(smem, acc, C, M, N, m0, n0,
                                                                     tid, wm, wn);
    }
    __device__ __forceinline__ void drain_w(char* smem, float* W, int M, int N, int m0, int n0,
                                            int tid, int wm, int wn) {
        drain_f32<TL::BN, TL::TM, TL::TN, TL::FM, TL::FN, TL::T, TL::WM>(smem, acc, W, M, N, m0,
                                                                         n0, tid, wm, wn);
    }
};

template <class TL>
struct Compute<TL, 16> {
    floatx4 acc[TL::FN16][TL::FM16];
    half8 fa[2][TL::FM16], fb[TL::FN16];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < TL::FN16; ++j)
#pragma unroll
            for (int i = 0; i < TL::FM16; ++i) acc[j][i] = floatx4{};
    }
    // What half 1 of the step before step 0 would have read: every A block
    // and B blocks < FN16/2 of stage 0.
    __device__ __forceinline__ void first_reads(const char* stage, int wm, int wn, int lane) {
#pragma unroll
        for (int j = 0; j < TL::FN16 / 2; ++j) fb[j] = read_b16<TL>(stage, j, wn, lane);
#pragma unroll
        for (int i = 0; i < TL::FM16; ++i) fa[0][i] = read_a16<TL>(stage, i, wm, lane);
    }
    // Call c: half c&1 of its step with A buffer c>>1.
    template <int CALL, int NC, class CopyFn>
    __device__ __forceinline__ void half(const char* rstage, int wm, int wn, int lane, CopyFn copy) {
        constexpr int b = CALL >> 1;
        half16<TL, CALL & 1, NC>(acc, fa[b], fb, rstage, fa[b ^ 1], wm, wn, lane, copy);
    }
    __device__ __forceinline__ void drain_bands(char* stage, _Float16* C, int M, int N, int m0,
                                                int n0, int tid, int wm, int wn) {
        drain16_bands<TL::BM, TL::BN, TL::TM, TL::TN, TL::FM16, TL::FN16, TL::T, TL::STAGE>(
            stage, acc, C, M, N, m0, n0, tid, wm, wn);
    }
    __device__ __forceinline__ void drain_w(char* smem, float* W, int M, int N, int m0, int n0,
                                            int tid, int wm, int wn) {
        drain16_f32<TL::BN, TL::TM, TL::TN, TL::FM16, TL::FN16, TL::T, TL::WM>(smem, acc, W, M, N,
                                                                               m0, n0, tid, wm, wn);
    }
};

// Copy schedule.  Step s lives in ring slot s mod S (S odd; 5 unless the
// tile says otherwise).  The K loop runs in periods of two steps (kt even,
// kt+1); a period issues the copies of steps kt+S-1 and kt+S (an even and
// an odd step, so an A pair reads the two halves of the same 128-byte
// lines), one operand per half-step, H copies each:
//   step kt,   first half:  B of kt+S-1
//   step kt,   second half: A pairs 0 .. A_CP/2-1 of (kt+S-1, kt+S)
//   step kt+1, first half:  A pairs A_CP/2 .. A_CP-1 of (kt+S-1, kt+S)
//   step kt+1, second half: B of kt+S
// Slot of kt+S-1 (= slot of kt-1) is free after the barrier in the middle of
// step kt-1, slot of kt+S (= slot of kt) after the one in the middle of step
// kt, so every copy lands in a released slot.  The prologue issues steps
// 0 .. S-2 in the same order.  The wait in the middle of step kt covers step
// kt+1, issued as the second step of period kt+1-S: its last copy (B) is
// followed by the (S-3)/2 periods between (4H copies each) and the first
// half of period kt (H), so vmcnt <= W0 = H(2S-5).  The wait in the middle of
// step kt+1 covers step kt+2, the first step of period kt+3-S: its last copy
// (an A pair's first half) is followed by 1 + H + 4H(S-5)/2 + 3H copies, and
// the kernel waits for vmcnt <= W1 = 2H(S-3), one more than needed.  After
// the prologue, step 0's last copy is followed by 2H(S-1) - 3H + 1 copies:
// the first wait is also W0.
//
// Copies of steps 0 .. S-2 of a tile into slots 0 .. S-2, in the order a
// period issues them; with the steady-state copies when all of them lie
// inside K.  `c` is the tile's copier (init and init_fast done); a_pairs as
// for k_loop.
template <class TL, class APairs>
__device__ __forceinline__ void prologue(const Copier<TL>& c, const _Float16* B, int N, int K,
                                         int n0, int64_t bstep, uint32_t ring, int wave,
                                         APairs&& a_pairs) {
    constexpr int H = TL::H;
    if (K >= (TL::S - 1) * BK) {
#pragma unroll
        for (int e = 0; e < TL::S - 1; e += 2) {
            const uint32_t ste = ring + e * TL::STAGE;
#pragma unroll
            for (int t = 0; t < H; ++t) c.fast_b(t, B + n0 + e * bstep, ste, wave);
#pragma unroll
            for (int q = 0; q < 2 * H; ++q) {
                const int h = q & 1;
                c.fast_a(q >> 1, (uint32_t)((e + h) * BK * 2), ste + h * TL::STAGE, wave);
            }
#pragma unroll
            for (int t = 0; t < H; ++t)
                c.fast_b(t, B + n0 + (e + 1) * bstep, ste + TL::STAGE, wave);
        }
    } else {
#pragma unroll
        for (int e = 0; e < TL::S - 1; e += 2) {
#pragma unroll
            for (int t = 0; t < H; ++t)
                c.issue_b(t, B, N, K, n0, e * BK, ring + e * TL::STAGE, wave);
#pragma unroll
            for (int q = 0; q < 2 * H; ++q) a_pairs(q, 0, e, e, e + 1);
#pragma unroll
            for (int t = 0; t < H; ++t)
                c.issue_b(t, B, N, K, n0, (e + 1) * BK, ring + (e + 1) * TL::STAGE, wave);
        }
    }
}

// Wave priority around the half-steps of an 8-wave workgroup.  The CU places
// a workgroup's waves on its four SIMDs in turn, so waves w and w+4 share a
// SIMD and its matrix core.  Half-step c runs at raised priority in the
// first group (waves 0-3) when c is even and in the second group when c is
// odd: on each SIMD one wave issues its MFMAs first and the other fills the
// cycles in which the first waits for its LDS reads, instead of both
// reaching those waits together.  Measured on MI355X: 0.5-0.9% faster at
// 4096^3 and 8192^3, 2% at 2048^2 x 32768; the same switch at a fixed
// priority per group, or with groups that put both waves of a SIMD on one
// side, gains nothing.  PH: the wave's group (0, 1), or -1 for no switching.
template <int PH, int CALL>
__device__ __forceinline__ void half_priority() {
    if constexpr (PH >= 0) __builtin_amdgcn_s_setprio((CALL & 1) == PH ? 2 : 0);
}

// The K loop of one tile: from the wait for step 0 (the prologue has issued
// the copies of steps 0 .. S-2 into slots 0 .. S-2) to the end of the copies
// past K.  a_pairs(q, t0, s, sa, sb): the general A copies of pair unit q,
// starting at copy t0, of steps (s, s+1) into slots (sa, sb); relane(): the
// lane index, recomputed; ptid(): the thread index (race-detection build);
// PH: the wave's priority group (half_priority).
template <class TL, int PH, class APairs, class Relane, class PTid>
__device__ __forceinline__ void k_loop(Compute<TL>& cm, Copier<TL>& cp, char* smem, uint32_t ring,
                                       const _Float16* B, int N, int K, int lda, int n0, int nk,
                                       int64_t bstep, int wm, int wn, int lane, int wave,
                                       APairs&& a_pairs, Relane&& relane, PTid&& ptid) {
    constexpr int H = TL::H;
    wait_vmcnt<TL::W0>();  // this wave's copies of step 0 landed ...
    __syncthreads();       // ... and every other wave's
    cm.first_reads(smem, wm, wn, lane);

    // Whole periods only: with an odd number of steps the last period's
    // second step multiplies the zeros its copies read past the end of
    // K, which leaves every accumulator unchanged (they start at +0 and
    // never become -0, so adding +0 is exact).
    // Periods whose copies (steps kt+S-1, kt+S) lie inside K take the
    // steady-state copies; the last ones, and all of a short K, the
    // general ones.  Same data either way.
    const _Float16* b4 = B + n0 + (TL::S - 1) * bstep;  // rows of step kt+S-1
    uint32_t a4 = (TL::S - 1) * BK * 2;                 // A byte offset of step kt+S-1
    // One period; `slot` is the ring slot of step kt, either the run-time
    // `se` or a compile-time constant (the unrolled loop below).
    auto period = [&](int kt, auto fast, auto slot) __attribute__((always_inline)) {
        constexpr bool F = decltype(fast)::value;
        const int se = slot;
        const int s1 = wrap_slot<TL::S>(se + 1), s2 = wrap_slot<TL::S>(se + 2);
        const int s4 = wrap_slot<TL::S>(se + TL::S - 1);  // slot of step kt+S-1
        const char* cur = smem + se * TL::STAGE;
        const char* nxt = smem + s1 * TL::STAGE;
        const uint32_t st4 = ring + s4 * TL::STAGE, st5 = ring + se * TL::STAGE;
        auto pairs = [&](int q, int t0) __attribute__((always_inline)) {
            if constexpr (F) {
                const int h = q & 1;
                cp.fast_a(t0 + (q >> 1), a4 + h * (BK * 2), h ? st5 : st4, wave);
            } else {
                a_pairs(q, t0, kt + TL::S - 1, s4, se);
            }
        };
        // first half of step kt; B of step kt+S-1
        half_priority<PH, 0>();
        cm.template half<0, H>(cur, wm, wn, lane, [&](int q) __attribute__((always_inline)) {
            if constexpr (F)
                cp.fast_b(q, b4, st4, wave);
            else
                cp.issue_b(q, B, N, K, n0, (kt + TL::S - 1) * BK, st4, wave);
        });
        // copy_wait for step kt+1; the barrier also releases slot se
        wait_vmcnt<TL::W0>();
        __syncthreads();
        if constexpr (PGEMM_POISON_LDS) {
            poison_stage<TL::STAGE, TL::T>(smem + se * TL::STAGE, ptid());
            __syncthreads();
        }
        // second half of step kt (reads of step kt+1 begin); first A pairs
        half_priority<PH, 1>();
        cm.template half<1, H>(nxt, wm, wn, lane,
                               [&](int q) __attribute__((always_inline)) { pairs(q, 0); });
        // first half of step kt+1; other A pairs
        half_priority<PH, 2>();
        cm.template half<2, H>(nxt, wm, wn, lane, [&](int q) __attribute__((always_inline)) {
            pairs(q, TL::A_CP / 2);
        });
        // copy_wait for step kt+2; the barrier also releases slot s1
        wait_vmcnt<TL::W1>();
        __syncthreads();
        if constexpr (PGEMM_POISON_LDS) {
            poison_stage<TL::STAGE, TL::T>(smem + s1 * TL::STAGE, ptid());
            __syncthreads();
        }
        // second half of step kt+1 (reads of step kt+2 begin); B of step kt+S
        half_priority<PH, 3>();
        cm.template half<3, H>(smem + s2 * TL::STAGE, wm, wn, lane,
                               [&](int q) __attribute__((always_inline)) {
                                   if constexpr (F)
                                       cp.fast_b(q, b4 + bstep, st5, wave);
                                   else
                                       cp.issue_b(q, B, N, K, n0, (kt + TL::S) * BK, st5,
                                                  wave);
                               });
        b4 += 2 * bstep;
        a4 += 2 * BK * 2;
        return s2;
    };
    constexpr int S = TL::S;
    const int fast_end = K / BK - S;  // kt < fast_end <=> step kt+S is a full step
    int kt = 0;
    // S periods (2S steps) bring the ring back to slot 0, so the
    // unrolled loop knows every slot at compile time: no slot arithmetic
    // between the MFMAs.
    for (; kt + 2 * (S - 1) < fast_end && kt + 2 * (S - 1) < nk; kt += 2 * S)
        ring_pass<S>(
            [&](auto j, auto slot) __attribute__((always_inline)) {
                period(kt + 2 * decltype(j)::value, std::true_type{}, slot);
            },
            std::make_integer_sequence<int, S>{});
    // The tail periods recompute the per-lane copy offsets (relane: the same
    // lane index, hidden from the compiler) instead of keeping them live
    // across the unrolled loop.
    cp.init(relane(), wave, lda, N, n0);
    int se = 0;  // slot of step kt
    for (; kt < fast_end && kt < nk; kt += 2) se = period(kt, std::true_type{}, se);
    for (; kt < nk; kt += 2) se = period(kt, std::false_type{}, se);
    if constexpr (PH >= 0) __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();  // drain the copies of the steps past the end
}

// k_loop<TL, PH> with PH the wave's priority group: 8-wave tiles switch
// priorities (half_priority), others do not.  `run` is called once, with
// std::integral_constant<int, PH>.
template <class TL, class Run>
__device__ __forceinline__ void with_priority_group(int wave, Run&& run) {
    if constexpr (TL::T == 512) {
        if (wave < 4)
            run(std::integral_constant<int, 0>{});
        else
            run(std::integral_constant<int, 1>{});
    } else {
        run(std::integral_constant<int, -1>{});
    }
}

// SPLIT (split-K): blockIdx.y = s takes the K chunk [s*chunk, s*chunk +
// chunk) as a sub-matrix view (A shifted by s*chunk columns with its full row
// pitch, B by s*chunk rows) and writes its fp32 partial product to
// W + s*M*N instead of rounding to C.
template <class TL, int WPE, bool SPLIT = false>
__global__ __launch_bounds__(TL::T, 1) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void kernel(const _Float16* __restrict__ A0, const _Float16* __restrict__ B0,
            _Float16* __restrict__ C, int M, int N, int Kfull, int tiles_m, int tiles_n,
            int group_m, float* __restrict__ W, int chunk) {
    __shared__ __attribute__((aligned(1024))) char smem[TL::LDS];
    const _Float16* A = A0;
    const _Float16* B = B0;
    int K = Kfull;  // extent of this workgroup's K range
    if constexpr (SPLIT) {
        const int kb = blockIdx.y * chunk;
        K = min(chunk, Kfull - kb);
        A = A0 + kb;
        B = B0 + (int64_t)kb * N;
    }

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * TL::BM, n0 = tn * TL::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / TL::WN, wn = wave % TL::WN;

    Compute<TL> cm;
    cm.zero();

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        Copier<TL> cp;
        cp.init(lane, wave, Kfull, N, n0);
        const uint32_t ring = lds_addr(smem);
        // A pairs t0 .. t0+A_CP/2-1 of steps (s, s+1) into slots (sa, sb).
        auto a_pairs = [&](int q, int t0, int s, int sa, int sb) __attribute__((always_inline)) {
            const int t = t0 + (q >> 1), h = q & 1;
            cp.issue_a(t, A, M, K, m0, (s + h) * BK, ring + (h ? sb : sa) * TL::STAGE, wave);
        };
        cp.init_fast(A, M, m0, N, n0);
        const int64_t bstep = (int64_t)BK * N;  // elements per B step
        prologue<TL>(cp, B, N, K, n0, bstep, ring, wave, a_pairs);
        with_priority_group<TL>(wave, [&](auto ph) __attribute__((always_inline)) {
            k_loop<TL, decltype(ph)::value>(
                cm, cp, smem, ring, B, N, K, Kfull, n0, nk, bstep, wm, wn, lane, wave, a_pairs,
                [&]() __attribute__((always_inline)) {
                    int l = lane;
                    asm volatile("" : "+v"(l));
                    return l;
                },
                [&]() __attribute__((always_inline)) { return tid; });
        });
    }
    __syncthreads();  // every wave is done with the stage ring
    // The drain derives its lane addresses from the thread index afresh (the
    // empty statement hides that it is the same value), so that no values
    // derived before the K loop stay live across it: the loop runs at the
    // register limit.
    int tid_d = tid;
    asm volatile("" : "+v"(tid_d));
    // The 16x16x32 path drains in bands of rows: stores of one band start
    // while the next is converted (measured on MI355X: 4096^2 x 512 5%
    // faster, long K unchanged).
    if constexpr (SPLIT)
        cm.drain_w(smem, W + (int64_t)blockIdx.y * M * N, M, N, m0, n0, tid_d, wm, wn);
    else if constexpr (TL::MF == 16)
        cm.drain_bands(smem, C, M, N, m0, n0, tid_d, wm, wn);
    else
        cm.drain_c(smem, C, M, N, m0, n0, tid_d, wm, wn);
}

// Arguments of the persistent kernel, passed as its only (by-value)
// argument, so that they are also the first bytes of its argument segment.
struct PersistentArgs {
    const _Float16* A;
    const _Float16* B;
    _Float16* C;
    int M, N, K, tiles_m, tiles_n, group_m;
    int stride;  // the grid size
};
typedef const __attribute__((address_space(4))) PersistentArgs ConstPersistentArgs;

// Persistent form of `kernel` (no split-K): a grid of at most one workgroup
// per CU walks the logical tiles blockIdx.x, blockIdx.x + stride, ...
// (stride = the grid size, a multiple of 8, which keeps the XCD-aware map
// of tile_of_block).  Right after a tile's K loop the copies of the next
// tile's steps 0..S-2 go into ring slots 0..S-2, and the finished tile is drained
// through slot S-1 in bands of rows (drain_bands), so the next tile's
// operands are in flight while this tile is converted and stored.  The next
// tile's first wait (vmcnt <= W0) then also covers the drain's stores, which
// were issued after those copies: on gfx9 one counter (vmcnt) covers loads,
// LDS-DMA loads and stores, which complete in issue order (the compiler's own
// waits rely on the same), so all but the W0 youngest are done, step 0 among
// them.
// Per-lane values are derived afresh in every tile (from an opaque copy of
// the thread index), so none is kept live across the K loop beyond what
// `kernel` keeps.  The K loop itself is `kernel`'s (k_loop).
// persistent_tiles is the tile loop of the wave group PH (half_priority).
template <class TL, int PH>
__device__ __forceinline__ void persistent_tiles(char* smem, const int wave) {
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    const uint32_t ring = lds_addr(smem);
    auto opaque_tid = []() __attribute__((always_inline)) {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t;
    };
    // The tile loop reads its arguments from the argument segment where it
    // needs them, through an opaque copy of the segment address, so that
    // none of them (nor anything derived from them) occupies a register
    // across the K loop, which runs at the register limit.
    ConstPersistentArgs* const args =
        (ConstPersistentArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    auto load_args = [&]() __attribute__((always_inline)) {
        ConstPersistentArgs* p = args;
        asm volatile("" : "+s"(p));
        return p;
    };

    int blk = blockIdx.x;
    int m0, n0;
    {
        ConstPersistentArgs* g = load_args();
        int tm, tn;
        tile_of_block(blk, g->tiles_m * g->tiles_n, g->tiles_m, g->tiles_n, g->group_m, tm, tn);
        m0 = tm * TL::BM;
        n0 = tn * TL::BN;
    }

    Compute<TL> cm;
    for (bool first = true;; first = false) {
        ConstPersistentArgs* g = load_args();
        const int M = g->M, N = g->N, K = g->K;
        const _Float16* const A = g->A;
        const _Float16* const B = g->B;
        const int nk = (K + BK - 1) / BK;
        const int64_t bstep = (int64_t)BK * N;  // elements per B step
        const int lane = opaque_tid() & 63;

        // A pairs t0 .. t0+A_CP/2-1 of steps (s, s+1) of the tile at row pm0
        // into slots (sa, sb).
        auto a_pairs = [&](const Copier<TL>& c, int pm0, int q, int t0, int s, int sa, int sb)
                           __attribute__((always_inline)) {
            const int t = t0 + (q >> 1), h = q & 1;
            c.issue_a(t, A, M, K, pm0, (s + h) * BK, ring + (h ? sb : sa) * TL::STAGE, wave);
        };
        // Steps 0..S-2 of the tile at (pm0, pn0) into slots 0..S-2.
        auto prologue_at = [&](int pl, int pm0, int pn0) __attribute__((always_inline)) {
            Copier<TL> c;
            c.init(pl, wave, K, N, pn0);
            c.init_fast(A, M, pm0, N, pn0);
            prologue<TL>(c, B, N, K, pn0, bstep, ring, wave,
                         [&](int q, int t0, int st, int sa, int sb) __attribute__((always_inline)) {
                             a_pairs(c, pm0, q, t0, st, sa, sb);
                         });
        };

        if (first && nk > 0) prologue_at(lane, m0, n0);
        cm.zero();
        if (nk > 0) {
            Copier<TL> cp;
            cp.init(lane, wave, K, N, n0);
            cp.init_fast(A, M, m0, N, n0);
            k_loop<TL, PH>(
                cm, cp, smem, ring, B, N, K, K, n0, nk, bstep, wm, wn, lane, wave,
                [&](int q, int t0, int st, int sa, int sb) __attribute__((always_inline)) {
                    a_pairs(cp, m0, q, t0, st, sa, sb);
                },
                [&]() __attribute__((always_inline)) { return opaque_tid() & 63; },
                [&]() __attribute__((always_inline)) { return opaque_tid(); });
        }
        __syncthreads();  // every wave is done with the stage ring
        const int tid_d = opaque_tid();
        const int dm0 = m0, dn0 = n0;
        ConstPersistentArgs* h = load_args();
        const int ntiles = h->tiles_m * h->tiles_n;
        blk += h->stride;
        const bool more = blk < ntiles;
        if (more) {
            int tm, tn;
            tile_of_block(blk, ntiles, h->tiles_m, h->tiles_n, h->group_m, tm, tn);
            m0 = tm * TL::BM;
            n0 = tn * TL::BN;
            if (nk > 0) prologue_at(tid_d & 63, m0, n0);
        }
        cm.drain_bands(smem + (TL::S - 1) * TL::STAGE, h->C, M, N, dm0, dn0, tid_d, wm, wn);
        if (!more) break;
    }
}

// The branch on the wave's priority group encloses the whole tile loop, not
// only its K loop as in `kernel`: inside the tile loop it left too few
// registers (VGPRs spilled).
template <class TL, int WPE>
__global__ __launch_bounds__(TL::T, 1) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void kernel_persistent(const PersistentArgs) {
    __shared__ __attribute__((aligned(1024))) char smem[TL::LDS];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    with_priority_group<TL>(wave, [&](auto ph) __attribute__((always_inline)) {
        persistent_tiles<TL, decltype(ph)::value>(smem, wave);
    });
}

}  // namespace dm

// ===========================================================================
// Wave-specialised LDS-DMA pipeline: MFMA waves that only read LDS and
// multiply, plus one copy wave that issues every global->LDS copy.
// ===========================================================================
//
// The pages' warp-specialised pipeline (Pallas Mosaic GPU pipelining, the
// emit_pipeline_warp_specialized variant in the guide's platform notes, and
// the Chinese quickstart) gives memory transfers a warpgroup of their own so
// the compute warpgroups never stall on issuing them.  On gfx950 every wave
// of a kernel gets the same register allocation, so a copy wave costs as
// many registers as an MFMA wave: it fits next to the 128x128 tile's four
// MFMA waves (about 170 registers each; the copy wave shares SIMD 0 with
// MFMA wave 0) but not next to the 256x256 ones.  Layout, ring, swizzles and
// the order of the K steps are those of the dm kernel, so the results are
// bit-identical to it.
namespace ws {

using dm::BK;
using dm::STAGES;
using dm::aswz;
using dm::bswz;
using dm::wrap5;

// Copies of the whole workgroup: piece t of the A (B) stage is the dm
// kernel's copy t % A_CP of wave t / A_CP (B likewise), same LDS place.
template <class TL>
struct Producer {
    static constexpr int NW = TL::WM * TL::WN;  // MFMA waves
    static constexpr int NA = NW * TL::A_CP;    // A copies per step
    static constexpr int NB = NW * TL::B_CP;    // B copies per step
    uint32_t a_off[NA];
    int a_k[NA];
    uint32_t b_off[NB];

    __device__ __forceinline__ void init(int lane, int K, int N, int n0) {
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            const int p = t * 64 + lane;
            const int row = p >> 2;
            const int c = (p & 3) ^ aswz(row);
            a_off[t] = (uint32_t)((row * K + c * 8) * 2);
            a_k[t] = c * 8;
        }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int p = t * 64 + lane;
            const int row = p / (TL::B_ROW / 16);
            const int c = (p % (TL::B_ROW / 16)) ^ bswz(row);
            const int n = c * 8;
            b_off[t] = (n0 + n < N) ? (uint32_t)((row * N + n) * 2) : kOOB;
        }
    }
    // B of step s into ring slot `slot`.
    __device__ __forceinline__ void b_step(const _Float16* B, int N, int K, int n0, int s,
                                           uint32_t stage) const {
        const int k0 = s * BK;
        const int kv = min(BK, K - k0);
        const u32x4 rb = rsrc_words(B + (int64_t)k0 * N + n0, ((int64_t)kv * N - n0) * 2);
#pragma unroll
        for (int t = 0; t < NB; ++t) dma16(rb, b_off[t], stage + TL::A_BYTES + t * 1024);
    }
    // A of steps s and s+1 into stages sa and sb, the two halves of each
    // 128-byte line back to back.
    __device__ __forceinline__ void a_pairs(const _Float16* A, int M, int K, int m0, int s,
                                            uint32_t sa, uint32_t sb) const {
        const int rows_valid = min(TL::BM, M - m0);
        const int k0 = s * BK, k1 = k0 + BK;
        const u32x4 r0 = rsrc_words(A + (int64_t)m0 * K + k0, ((int64_t)rows_valid * K - k0) * 2);
        const u32x4 r1 = rsrc_words(A + (int64_t)m0 * K + k1, ((int64_t)rows_valid * K - k1) * 2);
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            dma16(r0, (a_k[t] < K - k0) ? a_off[t] : kOOB, sa + t * 1024);
            dma16(r1, (a_k[t] < K - k1) ? a_off[t] : kOOB, sb + t * 1024);
        }
    }
};

// Copy-wave schedule, per period of two K steps (kt even):
//   S1: B of kt+3 and kt+4; wait for step kt+1; barrier 1 (MFMA waves are
//       in the middle of step kt; slot of kt is released)
//   S2: A pairs of (kt+4, kt+5); wait for step kt+2; barrier 2 (middle of
//       step kt+1; slot of kt+1 released)
// B of kt+3 goes to the slot of kt-2 (released a period earlier), B and A of
// kt+4 to the slot of kt-1 (released at the previous barrier 2), A of kt+5 to
// the slot of kt (released at barrier 1 just before).  The prologue issues B0,
// A(0,1), B1, B2, A(2,3) (B3 comes with S1 of the first period).  Wait
// counts: step kt+1's last copy (its B) is followed by 3NB+2NA copies at
// barrier 1; step kt+2's last copy (an A pair's first half) by 2NB+2NA+1 at
// barrier 2, waited to 2NB+2NA.
template <class TL>
__global__ __launch_bounds__(TL::T + 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kernel(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
            _Float16* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
            int group_m) {
    __shared__ __attribute__((aligned(1024))) char smem[TL::LDS];
    using P = Producer<TL>;
    constexpr int NA = P::NA, NB = P::NB;
    static_assert(3 * NB + 2 * NA < 64, "vmcnt range");

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * TL::BM, n0 = tn * TL::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nk = (K + BK - 1) / BK;
    const uint32_t ring = lds_addr(smem);

    if (wave == P::NW) {
        // ---- copy wave ----
        if (nk > 0) {
            P pr;
            pr.init(lane, K, N, n0);
            pr.b_step(B, N, K, n0, 0, ring);
            pr.a_pairs(A, M, K, m0, 0, ring, ring + TL::STAGE);
            pr.b_step(B, N, K, n0, 1, ring + TL::STAGE);
            pr.b_step(B, N, K, n0, 2, ring + 2 * TL::STAGE);
            pr.a_pairs(A, M, K, m0, 2, ring + 2 * TL::STAGE, ring + 3 * TL::STAGE);
            wait_vmcnt<2 * NB + 2 * NA>();  // step 0 landed
            __syncthreads();
            int se = 0;
            for (int kt = 0; kt < nk; kt += 2) {
                const int s2 = wrap5(se + 2), s3 = wrap5(se + 3), s4 = wrap5(se + 4);
                pr.b_step(B, N, K, n0, kt + 3, ring + s3 * TL::STAGE);
                pr.b_step(B, N, K, n0, kt + 4, ring + s4 * TL::STAGE);
                wait_vmcnt<3 * NB + 2 * NA>();  // step kt+1 landed
                __syncthreads();
                if constexpr (PGEMM_POISON_LDS) __syncthreads();  // MFMA waves poison slot se
                pr.a_pairs(A, M, K, m0, kt + 4, ring + s4 * TL::STAGE, ring + se * TL::STAGE);
                wait_vmcnt<2 * NB + 2 * NA>();  // step kt+2 landed
                __syncthreads();
                if constexpr (PGEMM_POISON_LDS) __syncthreads();  // MFMA waves poison slot s1
                se = s2;
            }
            wait_vmcnt<0>();  // the copies past the end of K
        }
        __syncthreads();  // matches the MFMA waves' barrier before the drain
        __syncthreads();  // and the one inside the drain
        return;
    }

    // ---- MFMA waves ----
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    floatx16 acc[TL::FN][TL::FM];
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int i = 0; i < TL::FM; ++i) acc[j][i] = floatx16{};
    if (nk > 0) {
        __syncthreads();  // step 0 landed
        half8 fa[2][TL::FM], fb[2][TL::FN];
#pragma unroll
        for (int u = 0; u < TL::FM + TL::FN; ++u)
            dm::read_unit<TL>(u, smem, 0, wm, wn, lane, fa[0], fb[0]);
        auto none = [](int) {};
        int se = 0;
        for (int kt = 0; kt < nk; kt += 2) {
            const int s1 = wrap5(se + 1), s2 = wrap5(se + 2);
            const char* cur = smem + se * TL::STAGE;
            const char* nxt = smem + s1 * TL::STAGE;
            dm::half_step<TL, 0>(acc, fa[0], fb[0], cur, 1, fa[1], fb[1], wm, wn, lane, none);
            __syncthreads();  // step kt+1 landed; slot se released
            if constexpr (PGEMM_POISON_LDS) {
                poison_stage<TL::STAGE, TL::T>(smem + se * TL::STAGE, tid);
                __syncthreads();
            }
            dm::half_step<TL, 0>(acc, fa[1], fb[1], nxt, 0, fa[0], fb[0], wm, wn, lane, none);
            dm::half_step<TL, 0>(acc, fa[0], fb[0], nxt, 1, fa[1], fb[1], wm, wn, lane, none);
            __syncthreads();  // step kt+2 landed; slot s1 released
            if constexpr (PGEMM_POISON_LDS) {
                poison_stage<TL::STAGE, TL::T>(smem + s1 * TL::STAGE, tid);
                __syncthreads();
            }
            dm::half_step<TL, 0>(acc, fa[1], fb[1], smem + s2 * TL::STAGE, 0, fa[0], fb[0], wm, wn,
                                 lane, none);
            se = s2;
        }
    }
    __syncthreads();  // every wave is done with the stage ring
    drain<TL::BM, TL::BN, TL::TM, TL::TN, TL::FM, TL::FN, TL::T>(smem, acc, C, M, N, m0, n0, tid,
                                                                 wm, wn);
}

}  // namespace ws

// ===========================================================================
// Register-staged pipeline: 2 LDS stages of BK = 64 plus a register stage.
// ===========================================================================
namespace rs {

constexpr int BK = 64;
constexpr int ROW = BK * 2;  // bytes per LDS operand row

// Both operands stored K-contiguous: A as [BM][64] and B transposed as
// Bt[BN][64], 128-byte rows of 16-byte chunks; chunk c of row r sits at
// chunk position c ^ (r & 7).  Eight lanes reading one logical chunk of
// eight consecutive rows (fragment reads) and eight lanes writing eight
// chunks of one row (copies, transposed B writes) hit eight chunk positions.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int BM_, int BN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WM = 2, WN = 2;
    static constexpr int T = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int A_LD = BM * (BK / 8) / T;  // 16-byte A chunks per thread
    static constexpr int KR = BK * BN / (8 * T);    // B rows per thread (4 or 8)
    static constexpr int A_BYTES = BM * ROW;
    static constexpr int STAGE = (BM + BN) * ROW;
    static constexpr int LDS = 2 * STAGE;
    static_assert(KR == 4 || KR == 8, "B staging handles 4 or 8 rows per thread");
    static_assert(BM * BN * 2 <= LDS, "epilogue tile must fit in the stage buffers");
};

template <class TL>
struct Stager {
    u32x4 a[TL::A_LD];
    u32x4 b[TL::KR];

    // copy_start of K step k0 into registers.  Thread t copies A chunks t,
    // t+T, ... (8 consecutive threads cover one 128-byte row segment) and a
    // KR x 8 block of B: KR rows from kb*KR, columns nb*8 .. nb*8+7, with
    // kb = t % (64/KR), nb = t / (64/KR).  Pieces outside the matrix get an
    // offset with bit 31 set, past the end of the buffer: they read as zero.
    __device__ __forceinline__ void load(const _Float16* A, const _Float16* B, int M, int N, int K,
                                         int m0, int n0, int k0, int tid) {
        const int rows_valid = min(TL::BM, M - m0);
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(A + (int64_t)m0 * K + k0, ((int64_t)rows_valid * K - k0) * 2);
        const int kc = tid & 7;
        const uint32_t a_mask = (k0 + kc * 8 < K) ? 0u : kOOB;
        const uint32_t a_off0 = (uint32_t)(((tid >> 3) * K + kc * 8) * 2) | a_mask;
        const uint32_t a_step = (uint32_t)((TL::T / 8) * K * 2);
#pragma unroll
        for (int r = 0; r < TL::A_LD; ++r) a[r] = buf_load16(ra, a_off0 + r * a_step);

        const int kv = min(BK, K - k0);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(B + (int64_t)k0 * N + n0, ((int64_t)kv * N - n0) * 2);
        constexpr int KG = BK / TL::KR;
        const int kb = tid % KG, nb = tid / KG;
        const uint32_t b_mask = (n0 + nb * 8 < N) ? 0u : kOOB;
        const uint32_t b_off0 = (uint32_t)((kb * TL::KR * N + nb * 8) * 2) | b_mask;
#pragma unroll
        for (int r = 0; r < TL::KR; ++r) b[r] = buf_load16(rb, b_off0 + (uint32_t)(r * N * 2));
    }

    // Write the staged registers into one LDS stage (the compiler's vmcnt
    // wait before the first write is the copy_wait); B is transposed on the
    // way: column j of the thread's block becomes KR consecutive K values of
    // Bt row nb*8 + j.
    __device__ __forceinline__ void store(char* stage, int tid) const {
        const int kc = tid & 7;
#pragma unroll
        for (int r = 0; r < TL::A_LD; ++r) {
            const int row = (tid >> 3) + (TL::T / 8) * r;
            *reinterpret_cast<u32x4*>(stage + row * ROW + swz(row, kc) * 16) = a[r];
        }
        char* bt = stage + TL::A_BYTES;
        constexpr int KG = BK / TL::KR;
        const int kb = tid % KG, nb = tid / KG;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = nb * 8 + j;
            const int sh = (j & 1) * 16;
            uint32_t h[TL::KR];
#pragma unroll
            for (int r = 0; r < TL::KR; ++r) h[r] = (b[r][j >> 1] >> sh) & 0xFFFFu;
            if constexpr (TL::KR == 8) {
                u32x4 v;
                v[0] = h[0] | (h[1] << 16);
                v[1] = h[2] | (h[3] << 16);
                v[2] = h[4] | (h[5] << 16);
                v[3] = h[6] | (h[7] << 16);
                *reinterpret_cast<u32x4*>(bt + n * ROW + swz(n, kb) * 16) = v;
            } else {
                u32x2 v;
                v[0] = h[0] | (h[1] << 16);
                v[1] = h[2] | (h[3] << 16);
                *reinterpret_cast<u32x2*>(bt + n * ROW + swz(n, kb >> 1) * 16 + (kb & 1) * 8) = v;
            }
        }
    }
};

// Operand fragments of sub-step s (16 K values): lane (lr, lk) takes row lr
// of each 32-row block, K values 16s + 8lk .. +7 (one 16-byte chunk).
template <class TL>
__device__ __forceinline__ void read_frags(const char* stage, int s, int wm, int wn, int lane,
                                           half8 (&fa)[TL::FM], half8 (&fb)[TL::FN]) {
    const int lr = lane & 31;
    const int col = swz(lr, s * 2 + (lane >> 5)) * 16;  // same for every 32-row block
    const char* pa = stage + (wm * TL::TM + lr) * ROW + col;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) fa[i] = *reinterpret_cast<const half8*>(pa + i * 32 * ROW);
    const char* pb = stage + TL::A_BYTES + (wn * TL::TN + lr) * ROW + col;
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) fb[j] = *reinterpret_cast<const half8*>(pb + j * 32 * ROW);
}

template <class TL>
__device__ __forceinline__ void mfma_block(floatx16 (&acc)[TL::FN][TL::FM],
                                           const half8 (&fa)[TL::FM], const half8 (&fb)[TL::FN]) {
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int i = 0; i < TL::FM; ++i) acc[j][i] = mfma(fb[j], fa[i], acc[j][i]);
}

template <class TL, int WPE>
__global__ __launch_bounds__(TL::T) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void kernel(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
            _Float16* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
            int group_m) {
    __shared__ __attribute__((aligned(16))) char smem[TL::LDS];

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * TL::BM, n0 = tn * TL::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    floatx16 acc[TL::FN][TL::FM];
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int i = 0; i < TL::FM; ++i) acc[j][i] = floatx16{};

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        Stager<TL> st;
        // Prologue: step 0 into LDS stage 0, step 1 in flight in registers.
        st.load(A, B, M, N, K, m0, n0, 0, tid);
        st.store(smem, tid);
        if (nk > 1) st.load(A, B, M, N, K, m0, n0, BK, tid);
        __syncthreads();

        half8 fa[2][TL::FM], fb[2][TL::FN];
        read_frags<TL>(smem, 0, wm, wn, lane, fa[0], fb[0]);

        for (int kt = 0; kt < nk; ++kt) {
            char* cur = smem + (kt & 1) * TL::STAGE;
            char* nxt = smem + ((kt & 1) ^ 1) * TL::STAGE;
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
                if (s == 1 && kt + 1 < nk) {
                    // The free stage was last read before the previous barrier.
                    st.store(nxt, tid);
                    if (kt + 2 < nk) st.load(A, B, M, N, K, m0, n0, (kt + 2) * BK, tid);
                }
                if (s < BK / 16 - 1) {
                    read_frags<TL>(cur, s + 1, wm, wn, lane, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                } else {
                    __syncthreads();  // publishes `nxt`, releases `cur`
                    if constexpr (PGEMM_POISON_LDS) {
                        poison_stage<TL::STAGE, TL::T>(cur, tid);
                        __syncthreads();
                    }
                    if (kt + 1 < nk) read_frags<TL>(nxt, 0, wm, wn, lane, fa[0], fb[0]);
                }
                mfma_block<TL>(acc, fa[s & 1], fb[s & 1]);
            }
        }
    }
    __syncthreads();  // every wave is done with the stage buffers
    drain<TL::BM, TL::BN, TL::TM, TL::TN, TL::FM, TL::FN, TL::T>(smem, acc, C, M, N, m0, n0, tid,
                                                                 wm, wn);
}

}  // namespace rs

template <class TL, class KernelFn, class... Extra>
hipError_t launch(KernelFn kern, int threads, int splits, const void* A, const void* B, void* C,
                  int64_t M, int64_t N, int64_t K, hipStream_t stream, Extra... extra) {
    const int tiles_m = (int)((M + TL::BM - 1) / TL::BM);
    const int tiles_n = (int)((N + TL::BN - 1) / TL::BN);
    const int nwg = tiles_m * tiles_n;
    // Bands of 4 tile rows: a run of consecutive logical tiles then covers
    // 4 rows x (run/4) columns of tiles.
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    hipLaunchKernelGGL(kern, dim3(nwg, splits), dim3(threads), 0, stream,
                       static_cast<const _Float16*>(A), static_cast<const _Float16*>(B),
                       static_cast<_Float16*>(C), (int)M, (int)N, (int)K, tiles_m, tiles_n, group_m,
                       extra...);
    return hipGetLastError();
}
// Launch of a persistent kernel: one workgroup per CU (its LDS ring fills the
// CU), at most one per tile, the count a multiple of 8 (the XCD count) so
// that tile_of_block's map holds for every tile a workgroup visits.
template <class TL, class KernelFn>
hipError_t launch_persistent(KernelFn kern, int threads, const void* A, const void* B, void* C,
                             int64_t M, int64_t N, int64_t K, int cus, hipStream_t stream) {
    static_assert(2 * TL::LDS > 160 * 1024, "one workgroup per CU");
    const int tiles_m = (int)((M + TL::BM - 1) / TL::BM);
    const int tiles_n = (int)((N + TL::BN - 1) / TL::BN);
    const int nwg = tiles_m * tiles_n;
    int grid = cus >= 8 ? cus & ~7 : cus;
    if (grid > nwg) grid = nwg;
    if (grid < 1) grid = 1;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const dm::PersistentArgs args = {static_cast<const _Float16*>(A),
                                     static_cast<const _Float16*>(B),
                                     static_cast<_Float16*>(C),
                                     (int)M,
                                     (int)N,
                                     (int)K,
                                     tiles_m,
                                     tiles_n,
                                     group_m,
                                     grid};
    hipLaunchKernelGGL(kern, dim3(grid, 1), dim3(threads), 0, stream, args);
    return hipGetLastError();
}
}  // namespace

}  // namespace pgemm
