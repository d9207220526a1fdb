// gemm_dma.hip -- bf16 MFMA contraction with both operands k-major, tiles
// streamed into LDS by the direct global-to-LDS loads of gfx950.
//
// C[M][N] (float32) = A[M][K] . B[N][K]^T (+ bias[N]) (+ C if accumulate),
// A(m,k) = A[m*lda + k], B(n,k) = B[n*ldb + k], K a multiple of 32.  Used
// for the forward's input projection (FlashRNN abstract: the input part of
// every gate is one dense contraction over all time steps; W is staged
// transposed so that both operands are k-major) and the backward's dx and
// recompute contractions.
//
// Block tile 256x256, K in tiles of 32, 512 threads = 8 waves in a 2 (m) x 4
// (n) grid, each wave 128x64 = 4x2 tiles of v_mfma_f32_32x32x16_bf16.  LDS
// holds a ring of four K tiles (32 KiB each, 128 KiB).  K tiles are loaded
// in pairs: a tile's rows are 64 bytes, half of a 128-byte cache line, and
// the loads of the pair's two tiles go out interleaved from the same waves,
// so each line crosses from L2 once (a line's halves requested a tile apart
// are fetched twice, which halves what L2 delivers per CU when every CU
// streams).  No register is spent on staging.  A load instruction moves 16
// bytes per lane and writes the wave's 64 lanes as one contiguous KiB of LDS,
// so a tile is stored without padding: 64-byte rows (32 k), and in row r
// the 16-byte chunk c of the k range sits in slot c ^ swz(r) (gemm_dma.h):
// the 16 lanes of one access phase of a fragment read (16 rows, one chunk)
// touch 16 different bank groups.
//
// The fragment reads are inline assembly on purpose: the compiler tracks
// loads into LDS only coarsely and would otherwise wait for every load in
// flight (the whole ring) before each LDS read.  The asm carries its own
// wait for the reads, and the ring's own waits are explicit vmcnt counts.
//
// Tile order, split K, bias, accumulate and the row-panel counters are as in
// the register-staged kernel (gemm.hip).
#include <mutex>

#include "gemm_dma.h"

namespace rnn355 {

using namespace dma;

namespace {

__global__ __launch_bounds__(NTHR) void gemm_dma_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    gemm_dma_tiles_pre<0>(g, blockIdx.x, gridDim.x, (lds_char *)smem, [](int) {});
}

// The same with a second K segment per column block (GemmArgs::A2, B2).
__global__ __launch_bounds__(NTHR) void gemm_dma_seg2_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    gemm_dma_tiles_pre<0, true>(g, blockIdx.x, gridDim.x, (lds_char *)smem,
                                           [](int) {});
}

// dst[b][c][r] = src[b][r][c] for bf16 matrices [R][C] (row pitch C), in
// 64x64 tiles through LDS with 16-byte loads and stores where a row of the
// tile is whole and aligned (C % 8 == 0 for loads, R % 8 == 0 for stores).
// One launch serves up to two such jobs: a flat grid whose first blocks
// cover job 0 (ceil(C/64) x ceil(R/64) x batch tiles) and the rest job 1.
// Block 0 also zeroes the `nclear` words at `clear` and the `nclear2` at
// `clear2` (the status words and panel counters of the forward that
// follows), saving a launch.
struct TJob {
    const uint16_t *src;
    uint16_t *dst;
    int R, C, batch, tx, ty;  // tx, ty: tiles along C and R
};
__global__ __launch_bounds__(256) void transpose_bf16_kernel(TJob j0, TJob j1, unsigned *clear,
                                                             long nclear, unsigned *clear2,
                                                             long nclear2) {
    __shared__ __attribute__((aligned(16))) uint16_t t[64][72];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        if (clear)
            for (long i = tid; i < nclear; i += 256) clear[i] = 0u;
        if (clear2)
            for (long i = tid; i < nclear2; i += 256) clear2[i] = 0u;
    }
    const int n0 = j0.tx * j0.ty * j0.batch;
    const bool second = (int)blockIdx.x >= n0;
    const TJob &j = second ? j1 : j0;
    const int f = second ? (int)blockIdx.x - n0 : (int)blockIdx.x;
    const int bx = f % j.tx, by = (f / j.tx) % j.ty, bz = f / (j.tx * j.ty);
    const int R = j.R, C = j.C;
    const long bstride = (long)R * C;
    const uint16_t *S = j.src + bz * bstride;
    uint16_t *D = j.dst + bz * bstride;
    const int c0 = bx * 64, r0 = by * 64;
    // load: 64 rows x 8 chunks of 8 columns, two chunks per thread
    for (int q = tid; q < 512; q += 256) {
        const int i = q >> 3, cc = (q & 7) * 8;
        const int r = r0 + i, c = c0 + cc;
        uint16_t v[8];
        if (r < R && c + 8 <= C && (C & 7) == 0) {
            const uint4 w = *reinterpret_cast<const uint4 *>(S + (long)r * C + c);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = (uint16_t)ws[e];
                v[2 * e + 1] = (uint16_t)(ws[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (r < R && c + e < C) ? S[(long)r * C + c + e] : (uint16_t)0;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) t[i][cc + e] = v[e];
    }
    __syncthreads();
    // store: 64 output rows (c) x 8 chunks of 8 source rows (r)
    for (int q = tid; q < 512; q += 256) {
        const int i = q >> 3, rr = (q & 7) * 8;
        const int c = c0 + i, r = r0 + rr;
        if (c >= C) continue;
        if (r + 8 <= R && (R & 7) == 0) {
            uint32_t ws[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ws[e] = (uint32_t)t[rr + 2 * e][i] | ((uint32_t)t[rr + 2 * e + 1][i] << 16);
            *reinterpret_cast<uint4 *>(D + (long)c * R + r) = make_uint4(ws[0], ws[1], ws[2], ws[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (r + e < R) D[(long)c * R + r + e] = t[rr + e][i];
        }
    }
}

// The same transposition where every job has R % 8 == 0 and C % 8 == 0 and
// 16-byte aligned rows: a thread moves one 8x8 block in registers (eight
// 16-byte loads, 32 halfword recombinations, eight 16-byte stores), no LDS.
// A workgroup covers 64 rows x 256 columns of the source, wave w columns
// [64 w, 64 w + 64); lane 8 bi + bj takes block (bi, bj) of the wave's 64x64,
// so each load instruction reads eight whole 128-byte row pieces and each
// store writes eight.  Flat grid over both jobs as above, block 0 clears.
__global__ __launch_bounds__(256) void transpose8_bf16_kernel(TJob j0, TJob j1, unsigned *clear,
                                                              long nclear, unsigned *clear2,
                                                              long nclear2) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        if (clear)
            for (long i = tid; i < nclear; i += 256) clear[i] = 0u;
        if (clear2)
            for (long i = tid; i < nclear2; i += 256) clear2[i] = 0u;
    }
    const int n0 = j0.tx * j0.ty * j0.batch;
    const bool second = (int)blockIdx.x >= n0;
    const TJob &j = second ? j1 : j0;
    const int f = second ? (int)blockIdx.x - n0 : (int)blockIdx.x;
    const int bx = f % j.tx, by = (f / j.tx) % j.ty, bz = f / (j.tx * j.ty);
    const int R = j.R, C = j.C;
    const long bstride = (long)R * C;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = by * 64 + 8 * (lane >> 3);             // the block's first source row
    const int c = bx * 256 + 64 * wave + 8 * (lane & 7);  // and first source column
    if (r >= R || c >= C) return;
    const uint16_t *S = j.src + bz * bstride + (long)r * C + c;
    uint16_t *D = j.dst + bz * bstride + (long)c * R + r;
    uint32_t w[8][4];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint4 v = *reinterpret_cast<const uint4 *>(S + (long)k * C);
        w[k][0] = v.x;
        w[k][1] = v.y;
        w[k][2] = v.z;
        w[k][3] = v.w;
    }
    // output row e (source column c + e) holds source rows r..r+7 of column e:
    // word m pairs rows 2m (low half) and 2m + 1 (high half)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = w[2 * m][e >> 1], hi = w[2 * m + 1][e >> 1];
            o[m] = (e & 1) ? (hi & 0xFFFF0000u) | (lo >> 16) : (hi << 16) | (lo & 0xFFFFu);
        }
        *reinterpret_cast<uint4 *>(D + (long)e * R) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

TJob tjob(const uint16_t *src, uint16_t *dst, int R, int C, int batch) {
    TJob j{src, dst, R, C, batch, (C + 63) / 64, (R + 63) / 64};
    if (!src || batch <= 0) j.batch = 0;
    return j;
}

}  // namespace

bool gemm_dma_ok(int K) { return K % BK == 0 && K > 0; }

hipError_t launch_gemm_dma(const GemmArgs &g0, int batch, hipStream_t s, int max_wg) {
    GemmArgs g = g0;
    if (g.ksplit < 1) g.ksplit = 1;
    if (!gemm_dma_ok(g.K)) return hipErrorInvalidValue;
    if (g.ksplit > 1 && !g.partial) return hipErrorInvalidValue;
    if (g.ready && (g.ksplit > 1 || batch != 1)) return hipErrorInvalidValue;
    const bool seg2 = g.A2 != nullptr;
    if (seg2 && (!g.B2 || batch != 1 || g.ksplit != 1 || g.accumulate || !gemm_dma_ok(g.K2) ||
                 g.seg_n <= 0 || g.seg_n % BN != 0 || g.N % g.seg_n != 0))
        return hipErrorInvalidValue;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_dma_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
        if (attr == hipSuccess)
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_dma_seg2_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)LDS_BYTES);
    });
    if (attr != hipSuccess) return attr;
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    const int wgs = max_wg > 0 && max_wg < tiles ? max_wg : tiles;
    if (seg2)
        hipLaunchKernelGGL(gemm_dma_seg2_kernel, dim3(wgs, 1, 1), dim3(NTHR), LDS_BYTES, s, g);
    else
        hipLaunchKernelGGL(gemm_dma_kernel, dim3(wgs, 1, batch * g.ksplit), dim3(NTHR),
                           LDS_BYTES, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.ksplit == 1) return e;
    return launch_splitk_reduce(g, batch, s);
}

hipError_t launch_transpose_bf16(const uint16_t *src, uint16_t *dst, int R, int C, int batch,
                                 hipStream_t s, unsigned *clear, long nclear, unsigned *clear2,
                                 long nclear2, const uint16_t *src1, uint16_t *dst1, int R1,
                                 int C1, int batch1) {
    // whole 8x8 blocks and 16-byte aligned rows in every job: the register kernel
    auto fits8 = [](const uint16_t *a, const uint16_t *b, int r, int c) {
        return r % 8 == 0 && c % 8 == 0 && ((uintptr_t)a & 15) == 0 && ((uintptr_t)b & 15) == 0;
    };
    if (fits8(src, dst, R, C) && (!src1 || batch1 <= 0 || fits8(src1, dst1, R1, C1))) {
        auto tj8 = [](const uint16_t *a, uint16_t *b, int r, int c, int n) {
            TJob j{a, b, r, c, n, (c + 255) / 256, (r + 63) / 64};
            if (!a || n <= 0) j.batch = 0;
            return j;
        };
        const TJob k0 = tj8(src, dst, R, C, batch), k1 = tj8(src1, dst1, R1, C1, batch1);
        const long blocks8 = (long)k0.tx * k0.ty * k0.batch + (long)k1.tx * k1.ty * k1.batch;
        if (blocks8 <= 0 || blocks8 > 0x7fffffffL) return hipErrorInvalidValue;
        hipLaunchKernelGGL(transpose8_bf16_kernel, dim3((unsigned)blocks8), dim3(256), 0, s, k0, k1,
                           clear, nclear, clear2, nclear2);
        return hipGetLastError();
    }
    const TJob j0 = tjob(src, dst, R, C, batch), j1 = tjob(src1, dst1, R1, C1, batch1);
    const long blocks = (long)j0.tx * j0.ty * j0.batch + (long)j1.tx * j1.ty * j1.batch;
    if (blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, j0, j1,
                       clear, nclear, clear2, nclear2);
    return hipGetLastError();
}

}  // namespace rnn355
