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
// holds a ring of four K tiles (4 x 32 KiB); the loads of tile kt+3 are
// issued while tile kt is multiplied, so three tiles are in flight and no
// register is spent on staging.  A load instruction moves 16 bytes per lane
// and writes the wave's 64 lanes as one contiguous KiB of LDS, so a tile is
// stored without padding: 64-byte rows (32 k), and in row r the 16-byte
// chunk c of the k range sits in slot c ^ ((r >> 1) & 3).  The fragment
// reads of an MFMA (32 rows, one chunk) then touch every bank group equally.
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
    gemm_dma_tiles(g, blockIdx.x, gridDim.x, (lds_char *)smem);
}

// dst[b][c][r] = src[b][r][c] for bf16 matrices [R][C] (row pitch C), in
// 64x64 tiles through LDS; grid (ceil(C/64), ceil(R/64), batch).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ src,
                                                             uint16_t *__restrict__ dst, int R,
                                                             int C, long bstride) {
    __shared__ uint16_t t[64][66];
    const uint16_t *S = src + blockIdx.z * bstride;
    uint16_t *D = dst + blockIdx.z * bstride;
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int r = r0 + i, c = c0 + tx;
        t[i][tx] = (r < R && c < C) ? S[(long)r * C + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int c = c0 + i, r = r0 + tx;
        if (c < C && r < R) D[(long)c * R + r] = t[tx][i];
    }
}

}  // namespace

bool gemm_dma_ok(int K) { return K % BK == 0 && K > 0; }

hipError_t launch_gemm_dma(const GemmArgs &g0, int batch, hipStream_t s) {
    GemmArgs g = g0;
    if (g.ksplit < 1) g.ksplit = 1;
    if (!gemm_dma_ok(g.K)) return hipErrorInvalidValue;
    if (g.ksplit > 1 && !g.partial) return hipErrorInvalidValue;
    if (g.ready && (g.ksplit > 1 || batch != 1)) return hipErrorInvalidValue;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_dma_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    });
    if (attr != hipSuccess) return attr;
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_dma_kernel, dim3(tiles, 1, batch * g.ksplit), dim3(NTHR), LDS_BYTES, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.ksplit == 1) return e;
    return launch_splitk_reduce(g, batch, s);
}

hipError_t launch_transpose_bf16(const uint16_t *src, uint16_t *dst, int R, int C, int batch,
                                 hipStream_t s) {
    dim3 grid((C + 63) / 64, (R + 63) / 64, batch);
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, src, dst, R, C, (long)R * C);
    return hipGetLastError();
}

}  // namespace rnn355
