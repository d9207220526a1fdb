// gemm_dma.h -- device body of the bf16 MFMA contraction with both operands
// k-major and tiles streamed into LDS by the direct global-to-LDS loads of
// gfx950 (see gemm_dma.hip for the kernel and the design notes).  A header
// so that the fused forward kernel can run the same body in some of its
// workgroups.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnn355 {
namespace dma {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BM = 256, BN = 256, BK = 32, NST = 4, NTHR = 512;
constexpr int ROWB = BK * 2;                 // bytes per LDS row
constexpr int OPB = BM * ROWB;               // bytes per operand per stage (16 KiB)
constexpr int STB = 2 * OPB;                 // bytes per stage (32 KiB)
constexpr size_t LDS_BYTES = (size_t)NST * STB;
static_assert(BM == kGemmRowTile && BN == kGemmColTile, "row-panel counters assume the output tile");

// Row r of a tile keeps its k chunk c (16 bytes) in slot c ^ swz(r): any 16
// consecutive rows (or 8) read at one chunk then hit 16 (or 8) different
// 16-byte bank groups of a 256-byte (128-byte) LDS access phase.
__device__ __forceinline__ int swz(int r) { return ((r >> 2) & 3) ^ (r & 2); }

// The loads of one operand tile (256 rows x 32 k): 1024 chunks of 16 bytes,
// two per thread; chunk q goes to LDS byte 16q, i.e. row q/4, slot q%4,
// holding k chunk (q%4) ^ swz(row).  Rows past R read row R-1 (their
// products only reach outputs that are not stored).  `off` holds this
// thread's two byte offsets from the tile's (row 0, k 0) element, set once
// per output tile; a K tile only moves the wave-uniform base, so each load
// is an SGPR base plus a 32-bit VGPR offset and the LDS destination (M0) is
// wave-uniform too: no per-load vector arithmetic.
// AUX is the loads' cache policy (16: device scope, for operands that other
// workgroups of the same launch write).
__device__ __forceinline__ void tile_offsets(long ld, int r0, int R, int tid, uint32_t (&off)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + NTHR * i;
        const int r = q >> 2, slot = q & 3;
        const int chunk = slot ^ swz(r);
        const int gr = min(r0 + r, R - 1);
        off[i] = (uint32_t)(((long)gr * ld + chunk * 8) * 2);
    }
}
// The loads of a pair of K tiles: per operand and load slot, tile t0's
// load (16 bytes at k0 of each of its rows) and at once tile t1's (the next
// 64 bytes: with k0 a multiple of 64 elements, the other half of the same
// 128-byte lines), so each line crosses from L2 once -- a tile's 64-byte
// rows loaded a tile apart halve what the chip's L2 delivers per CU.  Order:
// A t0, A t1, A t0, A t1, B t0, B t1, B t0, B t1 (t1's loads only if
// `second`): one load follows the last of t0's.  A's source may differ
// between the two tiles (a second K segment begins at t1).
template <int AUX>
__device__ __forceinline__ void dma_pair(const uint16_t *A0, const uint32_t (&oA0)[2],
                                         const uint16_t *A1, const uint32_t (&oA1)[2],
                                         const uint16_t *B0, const uint32_t (&oB0)[2],
                                         const uint16_t *B1, const uint32_t (&oB1)[2],
                                         lds_char *s0, lds_char *s1, bool second, int wave_s) {
    const char *a0 = reinterpret_cast<const char *>(A0), *a1 = reinterpret_cast<const char *>(A1);
    const char *b0 = reinterpret_cast<const char *>(B0), *b1 = reinterpret_cast<const char *>(B1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int d = (64 * wave_s + NTHR * i) * 16;
        __builtin_amdgcn_global_load_lds(a0 + oA0[i], s0 + d, 16, 0, AUX);
        if (second) __builtin_amdgcn_global_load_lds(a1 + oA1[i], s1 + d, 16, 0, AUX);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int d = OPB + (64 * wave_s + NTHR * i) * 16;
        __builtin_amdgcn_global_load_lds(b0 + oB0[i], s0 + d, 16, 0, 0);
        if (second) __builtin_amdgcn_global_load_lds(b1 + oB1[i], s1 + d, 16, 0, 0);
    }
}

// vmcnt(n) for the counts the pair schedule needs (n in {0, 1, 4, 5, 8, 9});
// any other n waits for everything.
__device__ __forceinline__ void wait_vm(int n) {
    if (n == 9) __builtin_amdgcn_s_waitcnt(0x0F79);
    else if (n == 8) __builtin_amdgcn_s_waitcnt(0x0F78);
    else if (n == 5) __builtin_amdgcn_s_waitcnt(0x0F75);
    else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F71);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// The contraction's work for workgroup `wg` of `nwg`: output tiles wg,
// wg + nwg, ... of batch / split slice blockIdx.z (a persistent loop when
// nwg is smaller than the tile count).  `lds` is LDS_BYTES of dynamic LDS:
// a ring of four K tiles, loaded in pairs.  Before each tile every
// thread calls pre(row tile), ahead of the barrier that starts the tile (a
// wait for A's rows goes there); A_AUX is the cache policy of A's loads.
// SEG2: the K tiles of the second segment (A2, B2) follow those of A, B.
template <int A_AUX, bool SEG2 = false, class PreTile>
__device__ __forceinline__ void gemm_dma_tiles_pre(const GemmArgs &g, int wg, int nwg,
                                                   lds_char *lds, PreTile &&pre) {
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;

    const int slice = blockIdx.z % g.ksplit, bz = blockIdx.z / g.ksplit;
    const uint16_t *A = g.A + (long)bz * g.strideA;
    const uint16_t *B = g.B + (long)bz * g.strideB;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // in an SGPR: M0 from scalar code
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, lh = lane >> 5;

    if (g.clear_words && wg == 0 && blockIdx.z == 0 && tid < 64) g.clear_words[tid] = 0u;

    const int ktiles1 = g.K / BK;
    const int ktiles = SEG2 ? ktiles1 + g.K2 / BK : ktiles1;
    const int per = (ktiles + g.ksplit - 1) / g.ksplit;
    const int kt0 = slice * per, kt1 = min(ktiles, kt0 + per);

    // this lane's fragment byte offsets inside a stage, for the two 16-deep
    // k steps of a tile: row l32 of the wave's first A / B tile, chunk
    // 2*kc + lh in its swizzled slot (rows of the other tiles: +32 rows)
    const int sw = swz(l32);  // the tiles' row bases are multiples of 32
    uint32_t offA[2], offB[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int slot = (2 * kc + lh) ^ sw;
        offA[kc] = (uint32_t)((wm * 128 + l32) * ROWB + slot * 16);
        offB[kc] = (uint32_t)(OPB + (wn * 64 + l32) * ROWB + slot * 16);
    }

    // Workgroup i runs on XCD i % 8 (nwg is a multiple of 8 or the tile
    // count), so tile t goes to XCD t % 8.  Where the tile counts divide,
    // XCD x = 2 xr + xc takes the row tiles xr, xr + 4, ... in order and the
    // column tiles of half xc: its share of W^T (half the columns) stays in
    // its L2 while the row panels stream.  Otherwise runs of 8 row tiles,
    // row tile 8q + x of a run on XCD x with all its column tiles, rows past
    // the last whole run in order.  Either way each XCD finishes its row
    // panels in time order.
    const int tiles_n = (g.N + BN - 1) / BN;
    const int tiles_m = (g.M + BM - 1) / BM;
    const int tiles = tiles_m * tiles_n;
    const int run = 8 * tiles_n, full = (tiles_m >> 3) * run;
    const bool split = (tiles_m & 3) == 0 && (tiles_n & 1) == 0 && (nwg & 7) == 0;
    const int half_n = tiles_n >> 1;
    for (int t = wg; t < tiles; t += nwg) {
    int mt, nt;
    if (split) {
        const int x = t & 7, k = t >> 3;
        const int p = k / half_n, c = k - p * half_n;
        mt = (x >> 1) + 4 * p;
        nt = (x & 1) * half_n + c;
    } else if (t < full) {
        const int q = t / run, i = t - q * run;
        mt = 8 * q + (i & 7);
        nt = i >> 3;
    } else {
        const int i = t - full;
        mt = (tiles_m & ~7) + i / tiles_n;
        nt = i % tiles_n;
    }
    const int m0 = mt * BM, n0 = nt * BN;
    pre(mt);
    // a new tile refills the ring: every wave is past the last tile's reads
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // register r of lane l of block (i, j): row 32 i + 8 (r/4) + 4 (l/32) +
    // r%4 of the wave's rows, column 32 j + l%32 of its columns
    f32x16 acc[4][2];

    // the second segment's A columns of this tile's column block
    const uint16_t *A2 = SEG2 ? g.A2 + (long)(n0 / g.seg_n) * g.K2 : nullptr;
    uint32_t goA[2], goB[2], goA2[2], goB2[2];
    tile_offsets(g.lda, m0, g.M, tid, goA);
    tile_offsets(g.ldb, n0, g.N, tid, goB);
    if (SEG2) {
        tile_offsets(g.lda2, m0, g.M, tid, goA2);
        tile_offsets(g.ldb2, n0, g.N, tid, goB2);
    }
    // K tiles go out in pairs (tiles kt0 + j, kt0 + j + 1, j even) into a
    // ring of four stages: tile kt0 + j in stage j % 4.  Pairs 0 and 1 go out
    // before the loop, pair j/2 + 1 at the barrier of tile kt0 + j (j >= 2
    // even), into the stages of tiles kt0 + j - 2 and kt0 + j - 1, which every
    // wave has finished reading by then.
    auto issue_pair = [&](int j) {
        const int t0 = kt0 + j, t1 = t0 + 1;
        const bool second = t1 < kt1;
        lds_char *s0 = lds + (j & 3) * STB, *s1 = lds + ((j + 1) & 3) * STB;
        // a tile's source: segment 1 (A, B at k = 32 kt) or segment 2
        const bool g20 = SEG2 && t0 >= ktiles1, g21 = SEG2 && t1 >= ktiles1;
        const int k0 = (g20 ? t0 - ktiles1 : t0) * BK, k1 = (g21 ? t1 - ktiles1 : t1) * BK;
        const uint16_t *a0 = (g20 ? A2 : A) + k0, *a1 = (g21 ? A2 : A) + k1;
        const uint16_t *b0 = (g20 ? g.B2 : B) + k0, *b1 = (g21 ? g.B2 : B) + k1;
        dma_pair<A_AUX>(a0, g20 ? goA2 : goA, a1, g21 ? goA2 : goA, b0, g20 ? goB2 : goB, b1,
                        g21 ? goB2 : goB, s0, s1, second, wave_s);
    };
    // loads a pair puts out (4 per tile and thread)
    auto pair_loads = [&](int j) { return kt0 + j >= kt1 ? 0 : kt0 + j + 1 < kt1 ? 8 : 4; };
    if (kt0 < kt1) issue_pair(0);
    if (kt0 + 2 < kt1) issue_pair(2);

    // Pipelined at k-step granularity (two 16-deep k-steps per tile): the
    // reads of the next k-step are in flight while the current one's MFMAs
    // run, and the barrier that makes tile kt+1 visible sits between tile
    // kt's two k-steps, so its wait overlaps MFMAs already issued.
#define RNN355_READ_HALF(stage, kc, a0, a1, a2, a3, b0, b1)                                  \
    do {                                                                                     \
        const uint32_t sb_ = lbase + (uint32_t)((stage) * STB);                              \
        asm volatile("ds_read_b128 %0, %6\n\t"                                              \
                     "ds_read_b128 %1, %6 offset:2048\n\t"                                  \
                     "ds_read_b128 %2, %6 offset:4096\n\t"                                  \
                     "ds_read_b128 %3, %6 offset:6144\n\t"                                  \
                     "ds_read_b128 %4, %7\n\t"                                              \
                     "ds_read_b128 %5, %7 offset:2048"                                       \
                     : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1)      \
                     : "v"(sb_ + offA[kc]), "v"(sb_ + offB[kc])                              \
                     : "memory");                                                            \
    } while (0)
// the 8 MFMAs of one k-step once its reads are in (WAIT: the lgkmcnt that
// leaves the six reads issued after them in flight, or 0); the wait is tied
// to the fragment registers so that no use moves above it.  ZERO: the
// tile's first k-step, whose MFMAs start from 0 (no accumulator clearing).
#define RNN355_MFMA_HALF(WAIT, ZERO, a0, a1, a2, a3, b0, b1)                                 \
    do {                                                                                     \
        asm volatile("s_waitcnt lgkmcnt(" #WAIT ")"                                          \
                     : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b0), "+v"(b1));          \
        const bf16x8 *a_[4] = {&a0, &a1, &a2, &a3};                                          \
        const bf16x8 *b_[2] = {&b0, &b1};                                                    \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                     \
        _Pragma("unroll") for (int j_ = 0; j_ < 2; ++j_)                                     \
            acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                           \
                *a_[i_], *b_[j_], (ZERO) ? f32x16{} : acc[i_][j_], 0, 0, 0);                 \
    } while (0)

    // tile kt0 landed for everyone: after its last load, one of its pair's
    // second tile and pair 1's may fly
    wait_vm(pair_loads(0) == 8 ? 1 + pair_loads(2) : 0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8 x0, x1, x2, x3, x4, x5, y0, y1, y2, y3, y4, y5;
    RNN355_READ_HALF(0, 0, x0, x1, x2, x3, x4, x5);
    auto ktile = [&](int kt, auto first) {
        constexpr bool F = decltype(first)::value;
        const int j = kt - kt0, cur = j & 3, nxt = (j + 1) & 3;
        RNN355_READ_HALF(cur, 1, y0, y1, y2, y3, y4, y5);
        RNN355_MFMA_HALF(6, F, x0, x1, x2, x3, x4, x5);
        const bool more = kt + 1 < kt1;
        if (more) {
            // this thread's loads of tile kt+1 landed; after the barrier
            // everyone's have.  Still in flight after them: at j = 0 pair 1;
            // j odd (kt+1 opens pair (j+1)/2): that pair's last load; j even:
            // nothing (the next pair goes out after the barrier)
            wait_vm(j == 0 ? pair_loads(2) : (j & 1) ? (pair_loads(j + 1) == 8 ? 1 : 0) : 0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (j >= 2 && !(j & 1) && kt + 2 < kt1) issue_pair(j + 2);
        }
        // the next tile's first k-step (the last tile re-reads its own, unused,
        // so that the count of reads behind y stays six on every path)
        RNN355_READ_HALF(more ? nxt : cur, 0, x0, x1, x2, x3, x4, x5);
        RNN355_MFMA_HALF(6, false, y0, y1, y2, y3, y4, y5);
    };
    if (kt0 < kt1) {
        ktile(kt0, std::integral_constant<bool, true>{});
        for (int kt = kt0 + 1; kt < kt1; ++kt) ktile(kt, std::integral_constant<bool, false>{});
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the unused reads
#undef RNN355_READ_HALF
#undef RNN355_MFMA_HALF

    // epilogue (an empty K range, a split-K slice past the end, stores zeros)
    auto store_tile = [&](const f32x16 (&acc)[4][2]) {
        float *C;
        long ldc;
        bool direct;
        if (g.ksplit == 1) {
            C = g.C + (long)bz * g.strideC;
            ldc = g.ldc;
            direct = true;
        } else {
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
            // a whole tile and nothing to read back: stores only, without
            // bounds checks or loads between them (with either, the compiler
            // waits for every earlier store before the next -- a round trip
            // per store); each store writes two 128-byte row segments
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
    };
    if (kt0 < kt1) {
        store_tile(acc);
    } else {
        f32x16 zero[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) zero[i][j] = f32x16{};
        store_tile(zero);
    }
    if (g.ready) {
        // publish the finished tile (see gemm.hip): stores reach L2, one
        // device-scope release per tile, then the panel count
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(g.ready + mt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    }  // tiles
}

// The ring of NST stages (LDS_BYTES): the kernels that share a CU's LDS
// with a recurrence.
__device__ __forceinline__ void gemm_dma_tiles(const GemmArgs &g, int wg, int nwg, lds_char *lds) {
    gemm_dma_tiles_pre<0>(g, wg, nwg, lds, [](int) {});
}

}  // namespace dma
}  // namespace rnn355
