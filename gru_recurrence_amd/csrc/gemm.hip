// gemm.hip -- dense contractions of librnn355 on MFMA (gfx950).
//
// C[M][N] (float32) = op(A)[M][K] . op(B)[K][N] (+ bias[N]) (+ C if accumulate)
// with bf16 operands and float32 accumulation in v_mfma_f32_16x16x32_bf16.
//
// The input projection of the forward pass (FlashRNN abstract: the input
// part of every gate is one dense contraction over all time steps) is the
// call A = x [T*B][Din] (k contiguous), B = W [Din][N] (n contiguous).  The
// backward pass reuses the same kernel with the other operand layouts.
//
// Each operand is either "k-major" (element (r,k) at P[r*ld + k]) or
// "r-major" (element (r,k) at P[k*ld + r]).  Tiles always land in LDS as
// [rows][k] with k contiguous so every MFMA fragment is one 16-byte LDS read;
// r-major tiles are transposed in registers (8x8 blocks of bf16, v_perm) on
// their way from HBM to LDS.
//
// Block tile 128x128x64, 256 threads = 4 waves in a 2x2 grid, each wave a
// 64x64 sub-tile = 4x4 MFMA tiles of 16x16.  The next K tile is fetched into
// registers while the current one is multiplied from LDS.
#include "common.h"
#include "kernels.h"

namespace rnn355 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row: 144 bytes (bank-spread, 16B aligned)
constexpr int NTHR = 256;

struct TileRegs {
    uint4 v[8];
};

// k-major operand: rows [r0, r0+128) x k [k0, k0+64) as 1024 16-byte chunks,
// 4 per thread.  Out-of-range chunks read as zero (R, K multiples of 8).
__device__ __forceinline__ void fetch_kmajor(const uint16_t *__restrict__ P, long ld, int r0,
                                             int k0, int R, int K, TileRegs &t) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NTHR * i;
        const int r = q >> 3, kc = (q & 7) * 8;
        const int gr = r0 + r, gk = k0 + kc;
        uint4 z = make_uint4(0, 0, 0, 0);
        if (gr < R && gk < K) z = *reinterpret_cast<const uint4 *>(P + (long)gr * ld + gk);
        t.v[i] = z;
    }
}

__device__ __forceinline__ void stash_kmajor(uint16_t *lds, const TileRegs &t) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NTHR * i;
        const int r = q >> 3, kc = (q & 7) * 8;
        *reinterpret_cast<uint4 *>(lds + r * LDS_LD + kc) = t.v[i];
    }
}

// r-major operand: element (r,k) at P[k*ld + r].  128 blocks of 8(k) x 8(r),
// one per thread of the first 128 threads (lane -> kb = tid%8, rb = tid/8, so
// each group of 16 lanes writes 16 distinct 16-byte bank groups).
__device__ __forceinline__ void fetch_rmajor(const uint16_t *__restrict__ P, long ld, int r0,
                                             int k0, int R, int K, TileRegs &t) {
    const int tid = threadIdx.x;
    if (tid < 128) {
        const int kb = tid & 7, rb = tid >> 3;
        const int gr = r0 + rb * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int gk = k0 + kb * 8 + i;
            uint4 z = make_uint4(0, 0, 0, 0);
            if (gr < R && gk < K) z = *reinterpret_cast<const uint4 *>(P + (long)gk * ld + gr);
            t.v[i] = z;
        }
    }
}

__device__ __forceinline__ void stash_rmajor(uint16_t *lds, const TileRegs &t) {
    const int tid = threadIdx.x;
    if (tid < 128) {
        const int kb = tid & 7, rb = tid >> 3;
        const uint32_t *w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = reinterpret_cast<const uint32_t *>(&t.v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // row (r) j of the block: the j-th bf16 of each of the 8 k-rows
            uint4 o;
            const int d = j >> 1;
            const bool up = j & 1;
            o.x = pack_halves(w[0][d], w[1][d], up);
            o.y = pack_halves(w[2][d], w[3][d], up);
            o.z = pack_halves(w[4][d], w[5][d], up);
            o.w = pack_halves(w[6][d], w[7][d], up);
            *reinterpret_cast<uint4 *>(lds + (rb * 8 + j) * LDS_LD + kb * 8) = o;
        }
    }
}

template <bool AK, bool BKM>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDS_LD];
    __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LDS_LD];

    const int bz = blockIdx.z;
    const uint16_t *A = g.A + (long)bz * g.strideA;
    const uint16_t *B = g.B + (long)bz * g.strideB;
    float *C = g.C + (long)bz * g.strideC;

    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;

    if (g.clear_words && blockIdx.x == 0 && blockIdx.y == 0 && bz == 0 && tid < 64)
        g.clear_words[tid] = 0u;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    TileRegs ta, tb;
    auto fetch = [&](int k0) {
        if (AK) fetch_kmajor(A, g.lda, m0, k0, g.M, g.K, ta);
        else fetch_rmajor(A, g.lda, m0, k0, g.M, g.K, ta);
        if (BKM) fetch_kmajor(B, g.ldb, n0, k0, g.N, g.K, tb);
        else fetch_rmajor(B, g.ldb, n0, k0, g.N, g.K, tb);
    };
    auto stash = [&]() {
        if (AK) stash_kmajor(sA, ta);
        else stash_rmajor(sA, ta);
        if (BKM) stash_kmajor(sB, tb);
        else stash_rmajor(sB, tb);
    };

    fetch(0);
    for (int k0 = 0; k0 < g.K; k0 += BK) {
        __syncthreads();  // previous tile's reads are done
        stash();
        __syncthreads();
        if (k0 + BK < g.K) fetch(k0 + BK);
#pragma unroll
        for (int kc = 0; kc < BK / 32; ++kc) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(
                    sA + (wm * 64 + i * 16 + lr) * LDS_LD + kc * 32 + lg * 8);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(
                    sB + (wn * 64 + j * 16 + lr) * LDS_LD + kc * 32 + lg * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32_bf16(af[i], bfr[j], acc[i][j]);
        }
    }

    // epilogue: lane holds D[4*lg + r][lr] of each 16x16 tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + lr;
        if (n >= g.N) continue;
        const float bv = g.bias ? g.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + lg * 4 + r;
                if (m < g.M) {
                    float v = acc[i][j][r] + bv;
                    float *dst = C + (long)m * g.ldc + n;
                    if (g.accumulate) v += *dst;
                    *dst = v;
                }
            }
        }
    }
}

// float32 contraction for f32 calls (small shapes): 16x16 output tile per
// 256-thread block, K in steps of 16 through LDS.  Same operand conventions
// with explicit strides: A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn].
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args g) {
    __shared__ float sA[16][17];
    __shared__ float sB[16][17];
    const int bz = blockIdx.z;
    const float *A = g.A + (long)bz * g.strideA;
    const float *B = g.B + (long)bz * g.strideB;
    float *C = g.C + (long)bz * g.strideC;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
    if (g.clear_words && blockIdx.x == 0 && blockIdx.y == 0 && bz == 0 && threadIdx.x < 64)
        g.clear_words[threadIdx.x] = 0u;
    float acc = 0.f;
    for (int k0 = 0; k0 < g.K; k0 += 16) {
        const int ka = k0 + tx, kb = k0 + ty;
        sA[ty][tx] = (m < g.M && ka < g.K) ? A[(long)m * g.sam + (long)ka * g.sak] : 0.f;
        sB[ty][tx] = (n < g.N && kb < g.K) ? B[(long)kb * g.sbk + (long)n * g.sbn] : 0.f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) acc = fmaf(sA[ty][k], sB[k][tx], acc);
        __syncthreads();
    }
    if (m < g.M && n < g.N) {
        float v = acc + (g.bias ? g.bias[n] : 0.f);
        float *dst = C + (long)m * g.ldc + n;
        if (g.accumulate) v += *dst;
        *dst = v;
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs &g, bool a_kmajor, bool b_kmajor, int batch,
                            hipStream_t s) {
    dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, batch);
    if (a_kmajor && !b_kmajor)
        hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), grid, dim3(NTHR), 0, s, g);
    else if (a_kmajor && b_kmajor)
        hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, dim3(NTHR), 0, s, g);
    else if (!a_kmajor && !b_kmajor)
        hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), grid, dim3(NTHR), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), grid, dim3(NTHR), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmF32Args &g, int batch, hipStream_t s) {
    dim3 grid((g.N + 15) / 16, (g.M + 15) / 16, batch);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace rnn355
