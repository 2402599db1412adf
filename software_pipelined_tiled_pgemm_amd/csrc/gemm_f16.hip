// Software-pipelined tiled fp16 GEMM for gfx950 (CDNA4).
//
// What it computes: C[M,N] = A[M,K] . B[K,N], fp16 in, fp32 accumulation, fp16
// out (round to nearest even) -- the matmul of the Pallas "Quickstart: GPU"
// page, section "Pipelining: a matmul kernel".  How, in the pages' terms:
//
//  * Parallel grid (quickstart, same section; Chinese quickstart, section
//    "Hopper 上的矩阵乘法内核"): one workgroup per BM x BN output tile; tiles
//    are independent and unordered.  The block id is remapped so that the
//    tiles one XCD runs share rows of A and columns of B in that XCD's L2.
//  * Sequential K pipeline (the emit_pipeline grid over K): each step consumes
//    an A slice [BM, 64] and a B slice [64, BN] from LDS.
//  * copy_start early / copy_wait late with multiple buffers (Pallas
//    software-pipelining guide, section 4): the global loads for step k+2 are
//    issued into registers while step k computes, are written into the free
//    LDS buffer during step k+1, and one barrier per step publishes them.
//    With two LDS buffers plus the register stage, three steps are in flight.
//  * Buffer release (the quickstart's delay_release discussion): an LDS
//    buffer is overwritten only after every wave has passed the barrier that
//    follows its last ds_read of it.  MFMA operands are VGPRs, so no matrix
//    instruction can still be reading LDS at that point.
//  * fp32 accumulator in registers (the quickstart's ACC): 32x32 MFMA blocks
//    held in VGPR/AGPR for the whole K loop, zeroed before step 0 (the
//    initialise-before-accumulate rule of the guide, section 7.2).
//  * Drain (quickstart's epilogue: cast, stage through shared memory, copy
//    out): fp32 -> fp16, written to LDS, then 16-byte coalesced row stores.
//
// Matrix instruction: v_mfma_f32_32x32x16_f16 (32x32 output block, 16-deep
// K, 8 fp16 per lane per operand).  The kernel computes the transposed block
// C^T = B^T A^T per MFMA (B^T as the row operand), so that each lane ends up
// holding four consecutive columns of one row of C -- 8 contiguous bytes for
// the epilogue.
//
// LDS layout: both operands are stored K-contiguous: A as [BM][64] and B
// transposed as Bt[BN][64], 128 bytes per row, in 16-byte chunks.  Chunk c of
// row r lives at chunk position c ^ (r & 7).  Eight lanes that read the same
// logical chunk of eight consecutive rows (MFMA fragment reads), and eight
// lanes that write eight different chunks of one row (A copies, transposed B
// writes), both touch eight different chunk positions: 16-byte accesses do
// not collide on banks.
//
// B arrives row-major (N contiguous).  Each thread loads a KR x 8 block of B
// (KR rows of K, 8 columns), transposes it in registers and writes 8 rows of
// Bt.  A is copied as is.  Edge tiles: buffer loads return zero outside the
// matrix (rows >= M, K >= K, columns >= N), stores are masked.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pgemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;                 // K depth of one pipeline step
constexpr int kRowBytes = kBK * 2;      // bytes per LDS operand row
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset that reads as zero
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int BM_, int BN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WM = 2, WN = 2;                 // waves along M and N
    static constexpr int T = 64 * WM * WN;               // threads per workgroup
    static constexpr int TM = BM / WM, TN = BN / WN;     // per-wave tile
    static constexpr int FM = TM / 32, FN = TN / 32;     // 32x32 blocks per wave
    static constexpr int A_LD = BM * (kBK / 8) / T;      // 16-byte A chunks per thread
    static constexpr int KR = kBK * BN / (8 * T);        // B rows per thread (4 or 8)
    static constexpr int A_BYTES = BM * kRowBytes;
    static constexpr int STAGE = (BM + BN) * kRowBytes;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int C_CHUNKS = BN / 8;              // 16-byte chunks per C row
    static_assert(KR == 4 || KR == 8, "B staging handles 4 or 8 rows per thread");
    static_assert(BM * BN * 2 <= LDS, "epilogue tile must fit in the stage buffers");
    static_assert((BM * BN / 8) % T == 0, "epilogue chunks must divide evenly");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

template <class TL>
struct Stager {
    u32x4 a[TL::A_LD];
    u32x4 b[TL::KR];

    // Issue the global loads of K step `k0` (copy_start).  Thread t copies A
    // chunks t, t+T, ... (8 consecutive threads cover one 128-byte row
    // segment) and a KR x 8 block of B: KR rows starting at kb*KR, columns
    // nb*8 .. nb*8+7, with kb = t % (64/KR) and nb = t / (64/KR).
    // Out-of-matrix pieces get an offset with bit 31 set: past the end of
    // the buffer, so the load returns zeros.
    __device__ __forceinline__ void load(const _Float16* A, const _Float16* B, int M, int N, int K,
                                         int m0, int n0, int k0, int tid) {
        const int rows_valid = min(TL::BM, M - m0);
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(A + (int64_t)m0 * K + k0, (uint32_t)((rows_valid * (int64_t)K - k0) * 2));
        const int kc = tid & 7;
        const uint32_t a_mask = (k0 + kc * 8 < K) ? 0u : kOOB;
        const uint32_t a_off0 = (uint32_t)(((tid >> 3) * K + kc * 8) * 2) | a_mask;
        const uint32_t a_step = (uint32_t)((TL::T / 8) * K * 2);
#pragma unroll
        for (int r = 0; r < TL::A_LD; ++r) a[r] = buf_load16(ra, a_off0 + r * a_step);

        const int kv = min(kBK, K - k0);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(B + (int64_t)k0 * N + n0, (uint32_t)(((int64_t)kv * N - n0) * 2));
        constexpr int KG = kBK / TL::KR;  // row groups
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
            *reinterpret_cast<u32x4*>(stage + row * kRowBytes + swz(row, kc) * 16) = a[r];
        }
        char* bt = stage + TL::A_BYTES;
        constexpr int KG = kBK / TL::KR;
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
                *reinterpret_cast<u32x4*>(bt + n * kRowBytes + swz(n, kb) * 16) = v;
            } else {
                u32x2 v;
                v[0] = h[0] | (h[1] << 16);
                v[1] = h[2] | (h[3] << 16);
                *reinterpret_cast<u32x2*>(bt + n * kRowBytes + swz(n, kb >> 1) * 16 +
                                          (kb & 1) * 8) = v;
            }
        }
    }
};

// MFMA operand fragments of sub-step s (16 K values): lane (lr, lk) takes
// row lr of each 32-row block, K values 16s + 8lk .. +7 (one 16-byte chunk).
template <class TL>
__device__ __forceinline__ void read_frags(const char* stage, int s, int wm, int wn, int lane,
                                           half8 (&fa)[TL::FM], half8 (&fb)[TL::FN]) {
    const int lr = lane & 31;
    const int col = swz(lr, s * 2 + (lane >> 5)) * 16;  // same for every 32-row block
    const char* pa = stage + (wm * TL::TM + lr) * kRowBytes + col;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
        fa[i] = *reinterpret_cast<const half8*>(pa + i * 32 * kRowBytes);
    const char* pb = stage + TL::A_BYTES + (wn * TL::TN + lr) * kRowBytes + col;
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
        fb[j] = *reinterpret_cast<const half8*>(pb + j * 32 * kRowBytes);
}

template <class TL>
__device__ __forceinline__ void mfma_block(floatx16 (&acc)[TL::FN][TL::FM],
                                           const half8 (&fa)[TL::FM], const half8 (&fb)[TL::FN]) {
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int i = 0; i < TL::FM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[j][i], 0, 0, 0);
}

// Block id -> output tile.  Workgroups are dealt to the 8 XCDs round-robin,
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

template <class TL, int WAVES_PER_EU>
__global__ __launch_bounds__(TL::T) __attribute__((amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void gemm_f16_kernel(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
                     _Float16* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
                     int group_m) {
    __shared__ __attribute__((aligned(16))) char smem[TL::LDS];

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * TL::BM, n0 = tn * TL::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    floatx16 acc[TL::FN][TL::FM];
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int i = 0; i < TL::FM; ++i) acc[j][i] = floatx16{};

    const int nk = (K + kBK - 1) / kBK;
    if (nk > 0) {
        Stager<TL> st;
        // Prologue: step 0 into LDS stage 0, step 1 in flight in registers.
        st.load(A, B, M, N, K, m0, n0, 0, tid);
        st.store(smem, tid);
        if (nk > 1) st.load(A, B, M, N, K, m0, n0, kBK, tid);
        __syncthreads();

        half8 fa[2][TL::FM], fb[2][TL::FN];
        read_frags<TL>(smem, 0, wm, wn, lane, fa[0], fb[0]);

        for (int kt = 0; kt < nk; ++kt) {
            char* cur = smem + (kt & 1) * TL::STAGE;
            char* nxt = smem + ((kt & 1) ^ 1) * TL::STAGE;
#pragma unroll
            for (int s = 0; s < kBK / 16; ++s) {
                if (s == 1 && kt + 1 < nk) {
                    // The free stage was last read before the previous barrier.
                    st.store(nxt, tid);
                    if (kt + 2 < nk) st.load(A, B, M, N, K, m0, n0, (kt + 2) * kBK, tid);
                }
                if (s < kBK / 16 - 1) {
                    read_frags<TL>(cur, s + 1, wm, wn, lane, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                } else {
                    __syncthreads();  // publishes `nxt`, releases `cur`
                    if (kt + 1 < nk) read_frags<TL>(nxt, 0, wm, wn, lane, fa[0], fb[0]);
                }
                mfma_block<TL>(acc, fa[s & 1], fb[s & 1]);
            }
        }
    }
    __syncthreads();  // every wave is done with the stage buffers

    // Drain: fp32 -> fp16 (RNE) into an LDS copy of the C tile, then 16-byte
    // row stores.  Lane (lr, lk) of block (j, i) holds row wm*TM+i*32+lr and
    // columns wn*TN+j*32+8g+4lk+q for accumulator element 4g+q.
    {
        const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
        for (int j = 0; j < TL::FN; ++j)
#pragma unroll
            for (int i = 0; i < TL::FM; ++i) {
                const int row = wm * TL::TM + i * 32 + lr;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int chunk = (wn * TL::TN + j * 32) / 8 + g;
                    const int pchunk = chunk ^ (row & (TL::C_CHUNKS - 1));
                    u32x2 v;
                    const _Float16 h0 = (_Float16)acc[j][i][4 * g + 0];
                    const _Float16 h1 = (_Float16)acc[j][i][4 * g + 1];
                    const _Float16 h2 = (_Float16)acc[j][i][4 * g + 2];
                    const _Float16 h3 = (_Float16)acc[j][i][4 * g + 3];
                    v[0] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                    v[1] = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
                    *reinterpret_cast<u32x2*>(smem + row * (TL::BN * 2) + pchunk * 16 + lk * 8) = v;
                }
            }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < TL::BM * TL::C_CHUNKS / TL::T; ++r) {
        const int id = tid + TL::T * r;
        const int row = id / TL::C_CHUNKS, chunk = id % TL::C_CHUNKS;
        const int pchunk = chunk ^ (row & (TL::C_CHUNKS - 1));
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + row * (TL::BN * 2) + pchunk * 16);
        const int m = m0 + row, n = n0 + chunk * 8;
        if (m < M && n < N)
            *reinterpret_cast<u32x4*>(C + (int64_t)m * N + n) = v;
    }
}

template <class TL, int WPE>
hipError_t launch(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                  hipStream_t stream) {
    const int tiles_m = (int)((M + TL::BM - 1) / TL::BM);
    const int tiles_n = (int)((N + TL::BN - 1) / TL::BN);
    const int nwg = tiles_m * tiles_n;
    // Bands of 4 tile rows: a run of consecutive logical tiles then covers
    // 4 rows x (run/4) columns of tiles.
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    hipLaunchKernelGGL((gemm_f16_kernel<TL, WPE>), dim3(nwg), dim3(TL::T), 0, stream,
                       static_cast<const _Float16*>(A), static_cast<const _Float16*>(B),
                       static_cast<_Float16*>(C), (int)M, (int)N, (int)K, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

}  // namespace

int gemm_choose_variant(int64_t M, int64_t N, int64_t K) {
    (void)K;
    // Large tiles halve LDS traffic per MFMA; use them when they still give
    // every CU (256 on MI355X) at least one tile.
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    return big_tiles >= 256 ? kGemm256x256 : kGemm128x128;
}

hipError_t launch_gemm_f16(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int variant, hipStream_t stream) {
    if (variant == kGemmAuto) variant = gemm_choose_variant(M, N, K);
    switch (variant) {
        case kGemm256x256:
            return launch<Tile<256, 256>, 1>(A, B, C, M, N, K, stream);
        case kGemm128x128:
            return launch<Tile<128, 128>, 2>(A, B, C, M, N, K, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace pgemm
