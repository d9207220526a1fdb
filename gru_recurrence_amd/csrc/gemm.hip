// gemm.hip -- dense contractions of librnn355 on MFMA (gfx950).
//
// C[M][N] (float32) = op(A)[M][K] . op(B)[K][N] (+ bias[N]) (+ C if accumulate)
// with bf16 operands and float32 accumulation in v_mfma_f32_32x32x16_bf16.
//
// The input projection of the forward pass (FlashRNN abstract: the input
// part of every gate is one dense contraction over all time steps) is the
// call A = x [T*B][Din] (k contiguous), B = W [Din][N] (n contiguous).  The
// backward pass reuses the kernel with the other operand layouts.
//
// Each operand is either "k-major" (element (r,k) at P[r*ld + k]) or
// "r-major" (element (r,k) at P[k*ld + r]).  Tiles always land in LDS as
// [rows][k] with k contiguous, so every MFMA fragment is one 16-byte LDS
// read; r-major tiles are transposed in registers (8x8 blocks of bf16, v_perm)
// on their way from HBM to LDS.
//
// Block tile 256x256x64, 512 threads = 8 waves in a 2 (m) x 4 (n) grid, each
// wave 128x64 = 4x2 MFMA tiles of 32x32 (128 accumulator VGPRs).  LDS holds
// two K tiles (2 x 72 KiB); the K tile after next is fetched into registers
// while the current one is multiplied.  Output tiles are dealt to XCDs in
// contiguous runs (workgroup i runs on XCD i % 8) so co-resident tiles share
// A panels in their XCD's L2.  A store instruction writes 32 consecutive
// floats of two rows (full 128-byte lines; the 32x32 accumulator layout is
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 for register r of lane l).
//
// Split K: for outputs with few tiles and a long K (the backward's dW, dR)
// the K range is cut into `ksplit` slices; each slice writes its partial
// product to a workspace buffer and a second kernel sums the slices in order
// (deterministic), adding bias and the old C where asked.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnn355 {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 256, BN = 256, BK = 64;
static_assert(BM == kGemmRowTile && BN == kGemmColTile, "row-panel counters assume the output tile");
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row: 144 bytes (bank spread, 16-byte aligned)
constexpr int NTHR = 512;
constexpr int STAGE = (BM + BN) * LDS_LD;  // bf16 per LDS stage
constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(uint16_t);

struct KRegs { uint4 v[4]; };  // k-major staging: 4 chunks of 16 bytes
struct RRegs { uint4 v[8]; };  // r-major staging: one 8x8 block

// k-major operand, rows [r0, r0+256) x k [k0, k0+64): 2048 16-byte chunks,
// 4 per thread.  Out-of-range chunks read as zero (R and K multiples of 8).
__device__ __forceinline__ void fetch_k(const uint16_t *__restrict__ P, long ld, int r0, int k0,
                                        int R, int K, KRegs &t) {
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

__device__ __forceinline__ void stash_k(uint16_t *lds, const KRegs &t) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NTHR * i;
        const int r = q >> 3, kc = (q & 7) * 8;
        *reinterpret_cast<uint4 *>(lds + r * LDS_LD + kc) = t.v[i];
    }
}

// r-major operand: element (r,k) at P[k*ld + r].  256 blocks of 8(k) x 8(r),
// one per thread of the first 256 threads (lane -> kb = tid%8, rb = tid/8,
// so each group of 16 lanes writes 16 distinct 16-byte bank groups).
__device__ __forceinline__ void fetch_r(const uint16_t *__restrict__ P, long ld, int r0, int k0,
                                        int R, int K, RRegs &t) {
    const int tid = threadIdx.x;
    if (tid < 256) {
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

__device__ __forceinline__ void stash_r(uint16_t *lds, const RRegs &t) {
    const int tid = threadIdx.x;
    if (tid < 256) {
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

template <bool AK>
struct AStage { using T = typename std::conditional<AK, KRegs, RRegs>::type; };

template <bool AK, bool BKM>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

    // z = batch * ksplit + slice
    const int slice = blockIdx.z % g.ksplit, bz = blockIdx.z / g.ksplit;
    const uint16_t *A = g.A + (long)bz * g.strideA;
    const uint16_t *B = g.B + (long)bz * g.strideB;

    // Tile order: runs of 8 row tiles, row tile 8q + x of a run on XCD x
    // (workgroup i runs on XCD i % 8) with all its column tiles, so an XCD's
    // L2 shares that row panel of A, and row tiles finish roughly in order
    // (a consumer of the rows, e.g. the time steps of a recurrence, can
    // start on the first ones).  Rows past the last whole run go in order.
    const int tiles_n = (g.N + BN - 1) / BN;
    const int tiles_m = (g.M + BM - 1) / BM;
    const int bid = blockIdx.x;
    const int run = 8 * tiles_n, full = (tiles_m >> 3) * run;
    int mt, nt;
    if (bid < full) {
        const int q = bid / run, i = bid - q * run;
        mt = 8 * q + (i & 7);
        nt = i >> 3;
    } else {
        const int i = bid - full;
        mt = (tiles_m & ~7) + i / tiles_n;
        nt = i % tiles_n;
    }
    const int m0 = mt * BM, n0 = nt * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, lh = lane >> 5;

    if (g.clear_words && bid == 0 && blockIdx.z == 0 && tid < 64) g.clear_words[tid] = 0u;

    // this slice's K range, in whole K tiles
    const int ktiles = (g.K + BK - 1) / BK;
    const int per = (ktiles + g.ksplit - 1) / g.ksplit;
    const int kt0 = slice * per, kt1 = min(ktiles, kt0 + per);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    typename AStage<AK>::T ta;
    typename AStage<BKM>::T tb;
    auto fetch = [&](int kt) {
        const int k0 = kt * BK;
        if constexpr (AK) fetch_k(A, g.lda, m0, k0, g.M, g.K, ta);
        else fetch_r(A, g.lda, m0, k0, g.M, g.K, ta);
        if constexpr (BKM) fetch_k(B, g.ldb, n0, k0, g.N, g.K, tb);
        else fetch_r(B, g.ldb, n0, k0, g.N, g.K, tb);
    };
    auto stash = [&](int stage) {
        uint16_t *sa = lds + stage * STAGE, *sb = sa + BM * LDS_LD;
        if constexpr (AK) stash_k(sa, ta);
        else stash_r(sa, ta);
        if constexpr (BKM) stash_k(sb, tb);
        else stash_r(sb, tb);
    };

    if (kt0 < kt1) {
        fetch(kt0);
        stash(0);
        if (kt0 + 1 < kt1) fetch(kt0 + 1);
        __syncthreads();
    }
    for (int kt = kt0; kt < kt1; ++kt) {
        const int stage = (kt - kt0) & 1;
        const uint16_t *sa = lds + stage * STAGE, *sb = sa + BM * LDS_LD;
#pragma unroll
        for (int kc = 0; kc < BK / 16; ++kc) {
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(
                    sa + (wm * 128 + i * 32 + l32) * LDS_LD + kc * 16 + lh * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(
                    sb + (wn * 64 + j * 32 + l32) * LDS_LD + kc * 16 + lh * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < kt1) stash(stage ^ 1);  // the other stage was released by the last barrier
        __syncthreads();
        if (kt + 2 < kt1) fetch(kt + 2);
    }

    // epilogue: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
    float *C;
    long ldc;
    bool direct;
    if (g.ksplit == 1) {
        C = g.C + (long)bz * g.strideC;
        ldc = g.ldc;
        direct = true;
    } else {
        // partial of this slice: [batch][ksplit][M][N] in the workspace
        C = g.partial + ((long)bz * g.ksplit + slice) * (long)g.M * g.N;
        ldc = g.N;
        direct = false;
    }
    const bool acc_old = direct && g.accumulate;
    // the bias of this lane's two columns, loaded before any store
    float bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + l32;
        bv[j] = (direct && g.bias && n < g.N) ? g.bias[n] : 0.f;
    }
    if (m0 + BM <= g.M && n0 + BN <= g.N && !acc_old) {
        // a whole tile and nothing to read back: stores only, without bounds
        // checks or loads between them (with either, the compiler waits for
        // every earlier store before the next -- a round trip per store)
        float *base = C + (long)(m0 + wm * 128 + 4 * lh) * ldc + n0 + wn * 64 + l32;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float *row = base + (long)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc;
#pragma unroll
                for (int j = 0; j < 2; ++j) row[j * 32] = acc[i][j][r] + bv[j];
            }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + l32;
            if (n >= g.N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    if (m < g.M) {
                        float v = acc[i][j][r] + bv[j];
                        float *dst = C + (long)m * ldc + n;
                        if (acc_old) v += *dst;
                        *dst = v;
                    }
                }
            }
        }
    }
    if (g.ready) {
        // publish the finished tile: every wave waits until its stores have
        // reached the XCD's L2 (vmcnt 0), then, after the barrier, one
        // thread writes the L2 back to memory (device-scope release) and
        // counts the tile of its row panel.  One write-back per tile rather
        // than one per wave: each write-back stalls every wave of the XCD.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(g.ready + mt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// C = sum over slices of the partials (+ bias) (+ old C), slices in order.
__global__ void splitk_reduce_kernel(GemmArgs g) {
    const long MN = (long)g.M * g.N;
    const int bz = blockIdx.y;
    const float *P = g.partial + (long)bz * g.ksplit * MN;
    float *C = g.C + (long)bz * g.strideC;
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < MN; e += (long)gridDim.x * blockDim.x) {
        const int m = (int)(e / g.N), n = (int)(e - (long)m * g.N);
        float v = 0.f;
        for (int s = 0; s < g.ksplit; ++s) v += P[s * MN + e];
        if (g.bias) v += g.bias[n];
        float *dst = C + (long)m * g.ldc + n;
        if (g.accumulate) v += *dst;
        *dst = v;
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

template <bool AK, bool BKM>
hipError_t launch_t(const GemmArgs &g, int batch, hipStream_t s) {
    // more than 64 KiB of dynamic LDS must be allowed once per kernel
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_bf16_kernel<AK, BKM>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    });
    if (attr != hipSuccess) return attr;
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM>), dim3(tiles, 1, batch * g.ksplit), dim3(NTHR),
                       LDS_BYTES, s, g);
    return hipGetLastError();
}

}  // namespace

int gemm_splitk_for(int M, int N, int K, int batch, int num_cu) {
    const long tiles = (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN) * batch;
    const int ktiles = (K + BK - 1) / BK;
    int ks = 1;
    // split while the grid fills less than the chip and each slice keeps >= 8 K tiles
    while (tiles * ks * 2 <= num_cu && ktiles / (ks * 2) >= 8) ks *= 2;
    return ks;
}

size_t gemm_partial_bytes(int M, int N, int batch, int ksplit) {
    return ksplit > 1 ? sizeof(float) * (size_t)batch * ksplit * M * N : 0;
}

hipError_t launch_gemm_bf16(const GemmArgs &g0, bool a_kmajor, bool b_kmajor, int batch,
                            hipStream_t s) {
    GemmArgs g = g0;
    if (g.ksplit < 1) g.ksplit = 1;
    if (g.ksplit > 1 && !g.partial) return hipErrorInvalidValue;
    if (g.ready && (g.ksplit > 1 || batch != 1)) return hipErrorInvalidValue;
    hipError_t e;
    if (a_kmajor && !b_kmajor) e = launch_t<true, false>(g, batch, s);
    else if (a_kmajor && b_kmajor) e = launch_t<true, true>(g, batch, s);
    else if (!a_kmajor && !b_kmajor) e = launch_t<false, false>(g, batch, s);
    else e = launch_t<false, true>(g, batch, s);
    if (e != hipSuccess || g.ksplit == 1) return e;
    return launch_splitk_reduce(g, batch, s);
}

hipError_t launch_splitk_reduce(const GemmArgs &g, int batch, hipStream_t s) {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(1024, batch), dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmF32Args &g, int batch, hipStream_t s) {
    dim3 grid((g.N + 15) / 16, (g.M + 15) / 16, batch);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace rnn355
