// rec_fwd.hip -- the strictly sequential forward recurrence of the multi-head
// LSTM / GRU, one persistent workgroup per (head, batch tile).
//
// Method (FlashRNN, arXiv 2412.07752, abstract; blog.hotdry.top 2025-09-21,
// the paragraphs on the step dependency, on the persistent kernel that keeps
// R out of HBM across steps, and on head-wise splitting): each head has its
// own Dh x G*Dh block of R and never talks to another head, so one workgroup
// owns one head for a tile of batch rows, loads that head's R block once,
// and then walks all T steps:
//     A_t = Gx_t + h_{t-1} R_n,   then the cell's gate update.
//
// MFMA kernel (bf16 R, Dh in {32, 64, 128}):
//   * Dh/16 waves; wave w owns hidden units [16w, 16w+16) and holds, for all
//     T steps, the B-operand fragments of v_mfma_f32_16x16x32_bf16 for those
//     units' G gate columns over all Dh/32 k-chunks (Dh=128 LSTM: 4 gates x
//     4 chunks x 4 VGPRs = 64 VGPRs of R per wave, R never re-read).
//   * h_{t-1} sits in LDS as bf16 (A operand; 16 rows = batch rows of the
//     tile, rows beyond the tile stay zero), double-buffered by step parity.
//   * per step: Dh/32 16-byte LDS reads, G*Dh/32 MFMAs, then every lane
//     already holds all G gate sums of its units (lane-local gate update in
//     float32), writes h_t as bf16 to the other LDS buffer, one barrier.
//   * HBM traffic is grouped by PD steps: Gx for the next group goes into a
//     register double buffer and the last group's h/c outputs are stored,
//     both issued at the first step of a group, so the only wait on HBM sits
//     at a group start and covers requests issued a full group earlier.
// Simple kernel (f32, or shapes the MFMA kernel does not cover): R in LDS as
// float32, one thread per (row, gate column) dot product per step.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "gates.h"
#include "gemm_dma.h"
#include "kernels.h"

namespace rnn355 {

namespace {

template <int CELL>
__device__ __forceinline__ void lstm_or_gru_unit(const float *gpre, int DH, const float *gxv,
                                                 float &cst, float &hst, float &h_out,
                                                 float &c_out) {
    if (CELL == kLSTM) {
        const float ai = gpre[0] + gxv[0];
        const float af = gpre[DH] + gxv[1];
        const float az = gpre[2 * DH] + gxv[2];
        const float ao = gpre[3 * DH] + gxv[3];
        const float ig = sigmoid_f(ai), fg = sigmoid_f(af);
        const float zg = tanh_f(az), og = sigmoid_f(ao);
        const float c = fmaf(fg, cst, ig * zg);
        const float h = og * tanh_f(c);
        cst = c;
        hst = h;
        h_out = h;
        c_out = c;
    } else {
        const float sr = gpre[0], sz = gpre[DH], sn = gpre[2 * DH];
        const float r = sigmoid_f(gxv[0] + sr);
        const float u = sigmoid_f(gxv[1] + sz);
        const float nn = tanh_f(fmaf(r, sn, gxv[2]));
        const float h = fmaf(u, hst - nn, nn);  // (1-u)*nn + u*h_{t-1}
        hst = h;
        h_out = h;
        c_out = 0.f;
    }
}

// s_waitcnt immediate for vmcnt(n), n < 64, other counters not waited on.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// 16 bytes per lane from src into the wave's contiguous KiB at dst (LDS).
__device__ __forceinline__ void load_lds16(const char *src, dma::lds_char *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The head start's results + b into gx; register r of lane l in block (i,
// mb) is row mb*32 + 8 (r/4) + 4 (l/32) + r%4, column l%32 of the block
// (wave w of the DH/16: column blocks w and w + DH/16, or w twice).  Returns
// once every wave's stores are complete in L2.
template <int G, int MB, int DH>
__device__ __forceinline__ void head_start_store(const RecArgs &a, int n, int b0, int rows,
                                                 const dma::f32x16 (&acc)[2][MB]) {
    constexpr int GD = G * DH, NB = GD / 32;
    const int B = a.B, N = a.NH * GD, M = a.hs_steps * rows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int nb1 = wave + DH / 16;
    const bool two = nb1 < NB;
    auto grow = [&](int m) -> long {
        return rows == 1 ? (long)m * B + b0 : (long)(m / rows) * B + b0 + m % rows;
    };
    float *gx = const_cast<float *>(a.gx);
    const int col0 = n * GD + wave * 32 + l32;
    const int col1 = two ? n * GD + nb1 * 32 + l32 : col0;  // GRU's last waves: block w again
    const float bv0 = a.hs_bias ? a.hs_bias[col0] : 0.f;
    const float bv1 = a.hs_bias ? a.hs_bias[col1] : 0.f;
    if (M == 32 * MB && rows == 1) {
        // whole blocks, one batch row: stores only, no bounds checks or
        // branches between them (either makes the compiler wait for every
        // earlier store first); the GRU's repeated block writes the same bits
        float *base = gx + (long)b0 * N;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float *row = base + (long)(mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)) * B * N;
                row[col0] = acc[0][mb][r] + bv0;
                row[col1] = acc[1][mb][r] + bv1;
            }
    } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m < M) {
                    float *row = gx + grow(m) * N;
                    row[col0] = acc[0][mb][r] + bv0;
                    if (two) row[col1] = acc[1][mb][r] + bv1;
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores are in L2
    __syncthreads();
}

// Head start of the pipelined forward (RecArgs::hs_*; FlashRNN card,
// abstract: the input part of every gate is one dense contraction over all
// steps, so any part of it may be computed ahead).  The workgroup of head n
// and batch rows [b0, b0 + rows), G gates of 128 units, computes gx for its
// own rows (t, b0 + i), t < hs_steps, i < rows, over its head's G*128
// columns before its first step: an M x G*128 tile, M = hs_steps * rows <=
// 32 MB, MB row blocks of 32.  Each value is made as the projection's tile
// would make it -- v_mfma_f32_32x32x16_bf16 over k-steps of 16 in increasing
// k order starting from zero, then + b[n] (or + 0) -- so gx is bitwise what
// the projection would have written.  As in the projection, K tiles of 32
// (64 rows of x, G*128 rows of W^T, 64 bytes each, 16-byte chunks swizzled)
// stream into a ring of LDS stages (four for LSTM, five for GRU) by the
// direct global-to-LDS loads, all but one stage in flight; wave w owns the 32-column blocks w and w + 8 (GRU, 12
// blocks: waves 4-7 compute block w twice and store it once).  Rows of x past
// M repeat row M - 1 (their sums are never stored).  Returns once every
// wave's stores are complete in L2, where the step loop's device-scope loads
// read.
template <int G, int MB, int DH>
__device__ __forceinline__ void head_start(const RecArgs &a, int n, int b0, int rows,
                                           char *smem) {
    constexpr int GD = G * DH, NB = GD / 32, NWV = DH / 16;  // NWV waves
    static_assert(NWV >= 4, "four waves load x's rows");
    constexpr int AB = 64 * 64, SB = AB + GD * 64;  // stage: x rows, then W^T rows
    constexpr int NS = kFusedLdsBytes / SB;          // LSTM 4 stages, GRU 5
    static_assert(NS >= 3, "the head start's ring needs three stages");
    using dma::f32x16;
    const int K = a.hs_K, B = a.B, KT = K >> 5;
    const int M = a.hs_steps * rows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, lh = lane >> 5;
    dma::lds_char *lds = (dma::lds_char *)smem;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;
    // gx / x row of head-start row m: step m / rows, batch row b0 + m % rows
    auto grow = [&](int m) -> long {
        return rows == 1 ? (long)m * B + b0 : (long)(m / rows) * B + b0 + m % rows;
    };
    // Load sources: a wave's load instruction fills 64 consecutive 16-byte
    // chunks of a stage; chunk q holds row q/4, k chunk (q%4) ^ swz(row).
    // x: chunks [0, 256) by waves 0-3; W^T: G instructions per wave.
    const char *pa;
    {
        const int q = 64 * (wave & 3) + lane, r = q >> 2;
        pa = reinterpret_cast<const char *>(a.hs_x + grow(min(r, M - 1)) * K +
                                            8 * ((q & 3) ^ dma::swz(r)));
    }
    const char *pb[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int q = 64 * (wave * G + i) + lane, r = q >> 2;
        pb[i] = reinterpret_cast<const char *>(a.hs_wt + (long)(n * GD + r) * K +
                                               8 * ((q & 3) ^ dma::swz(r)));
    }
    auto issue = [&](int kt, int stage) {
        dma::lds_char *st = lds + stage * SB;
        const int kb = 64 * kt;
        if (wave < 4) load_lds16(pa + kb, st + 1024 * wave_s);
#pragma unroll
        for (int i = 0; i < G; ++i) load_lds16(pb[i] + kb, st + AB + 1024 * (wave_s * G + i));
    };
    // fragment byte offsets in a stage: row l32 of block 0, k chunk 2 kc + lh
    const int nb1 = wave + NWV;
    const bool two = nb1 < NB;
    const int sw = dma::swz(l32);
    uint32_t oa[2], ob[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int slot = (2 * kc + lh) ^ sw;
        oa[kc] = (uint32_t)(l32 * 64 + slot * 16);
        ob[kc] = (uint32_t)(AB + (wave * 32 + l32) * 64 + slot * 16);
    }
    const uint32_t ob1 = (two ? NWV * 32 * 64 : 0);  // the second block's rows

    f32x16 acc[2][MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[0][mb] = acc[1][mb] = f32x16{};
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < KT) issue(p, p);
    for (int kt = 0; kt < KT; ++kt) {
        // this wave's loads of tile kt landed, those of up to NS - 2 later
        // tiles may fly (waves 0-3 issue G + 1 per tile, the others G:
        // counting G per tile waits for at least as much)
        const int later = min(NS - 2, KT - 1 - kt);
        if (later >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * G));
        else if (later == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * G));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(G));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // everyone's tile kt landed; stage kt-1 free
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < KT) issue(kt + NS - 1, (kt + NS - 1) % NS);
        const uint32_t sb = lbase + (uint32_t)((kt % NS) * SB);
        // the fragments of both k-steps, read and waited for in one block
        bf16x8 fa[2][2], fb[2][2];
        if constexpr (MB == 2)
            asm volatile("ds_read_b128 %0, %8\n\t"
                         "ds_read_b128 %1, %8 offset:2048\n\t"
                         "ds_read_b128 %2, %9\n\t"
                         "ds_read_b128 %3, %10\n\t"
                         "ds_read_b128 %4, %11\n\t"
                         "ds_read_b128 %5, %11 offset:2048\n\t"
                         "ds_read_b128 %6, %12\n\t"
                         "ds_read_b128 %7, %13\n\t"
                         "s_waitcnt lgkmcnt(0)"
                         : "=&v"(fa[0][0]), "=&v"(fa[0][1]), "=&v"(fb[0][0]), "=&v"(fb[0][1]),
                           "=&v"(fa[1][0]), "=&v"(fa[1][1]), "=&v"(fb[1][0]), "=&v"(fb[1][1])
                         : "v"(sb + oa[0]), "v"(sb + ob[0]), "v"(sb + ob[0] + ob1),
                           "v"(sb + oa[1]), "v"(sb + ob[1]), "v"(sb + ob[1] + ob1)
                         : "memory");
        else
            asm volatile("ds_read_b128 %0, %6\n\t"
                         "ds_read_b128 %1, %7\n\t"
                         "ds_read_b128 %2, %8\n\t"
                         "ds_read_b128 %3, %9\n\t"
                         "ds_read_b128 %4, %10\n\t"
                         "ds_read_b128 %5, %11\n\t"
                         "s_waitcnt lgkmcnt(0)"
                         : "=&v"(fa[0][0]), "=&v"(fb[0][0]), "=&v"(fb[0][1]),
                           "=&v"(fa[1][0]), "=&v"(fb[1][0]), "=&v"(fb[1][1])
                         : "v"(sb + oa[0]), "v"(sb + ob[0]), "v"(sb + ob[0] + ob1),
                           "v"(sb + oa[1]), "v"(sb + ob[1]), "v"(sb + ob[1] + ob1)
                         : "memory");
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                acc[0][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kc][mb], fb[kc][0],
                                                                     acc[0][mb], 0, 0, 0);
                acc[1][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kc][mb], fb[kc][1],
                                                                     acc[1][mb], 0, 0, 0);
            }
    }

    head_start_store<G, MB, DH>(a, n, b0, rows, acc);
}

// One workgroup = one head x one tile of up to 16 batch rows; DH/16 waves,
// wave w owns hidden units [16w, 16w+16) with all G gate tiles, so after the
// MFMA chain lane l holds every gate sum of unit 16w + l%16 for batch rows
// 4*(l/16) + r, r < R4 (R4 = register row slots in use).
//
// R4 == 1 (one batch row per workgroup) only rows 0 of the accumulators are
// live, in lanes 0..15.  Three cross-row swaps then lay the G gate sums of a
// unit out as the 4 rows of one register (gate g in lanes 16g..16g+15), so a
// single exp + rcp pass activates every gate at once (tanh(x) = 2*sigmoid(2x)
// - 1 on the z/n row), and three more swaps hand each lane back all gates.
//
// Memory traffic is grouped by PD steps: at the first step of each group the
// Gx values of the NEXT group are loaded into a register double buffer and
// the h/c outputs of the PREVIOUS group (kept in registers) are stored.  The
// only wait on HBM then sits at the first step of a group and covers
// operations issued a whole group earlier.
//
// WAIT (pipelined forward): Gx is written by the input projection while this
// kernel runs.  Before Gx of a step is requested, the wave checks that every
// row panel holding rows up to that step is complete (one counter word per
// panel, read 64 panels per poll).  The projection writes a panel's tiles
// back to memory before it counts them, and the Gx loads here are
// device-scope loads issued after the count was seen, which miss in this
// CU's L1 and the XCD's L2; so no cache invalidation is needed (an acquire
// fence would drop every cached line of the XCD, the projection's operand
// panels included).  Panels found complete are remembered; once the
// projection is ahead, a check costs a compare.
//
// HB (a stacked layer feeding the next one): h_t is also stored as bf16 at
// h_bf ([T][B][H]), with device-scope stores (written through the XCD's
// L2), and with `done` the workgroup counts a step on done[t] once every
// wave's stores of that step are complete.  No cache write-back is needed
// (one per group from every workgroup slowed the contraction running
// beside it by more than half).  Written-through stores take long to
// complete, so at a group start the Gx loads go out before the previous
// group's stores, and the next group start waits for all but those stores
// and the count that follows them: each wave's stores issued a group
// earlier are then complete.  After the barrier of that step every wave
// has passed its wait, and at the group's second step wave 0 counts the
// steps those stores hold (the group three back).

// The head start for one row block (M <= 32) where x's 32 rows of all K
// fit in LDS beside a ring of at least three W^T stages: x's rows are each
// read once, all loaded at the start (cold in the caches, they would
// otherwise cost a memory latency in every K tile), and only W^T streams
// through the ring.  Same MFMAs in the same order as head_start.
inline constexpr int hs_ares_bytes(int K) { return 64 * K; }  // 32 rows x 2K bytes
template <int G, int DH>
__device__ __forceinline__ void head_start_ares(const RecArgs &a, int n, int b0, int rows,
                                                char *smem) {
    constexpr int GD = G * DH, NB = GD / 32, BS = GD * 64;  // W^T stage: GD rows x 32 k
    constexpr int NWV = DH / 16;  // waves, >= 4
    static_assert(NWV >= 4, "four waves load x's rows");
    using dma::f32x16;
    const int K = a.hs_K, B = a.B, KT = K >> 5;
    const int M = a.hs_steps * rows;
    const int AR = hs_ares_bytes(K);              // x: K tile kt at 2048 kt
    const int NS = (kFusedLdsBytes - AR) / BS;    // >= 3: the condition for this variant
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, lh = lane >> 5;
    dma::lds_char *lds = (dma::lds_char *)smem;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;
    auto grow = [&](int m) -> long {
        return rows == 1 ? (long)m * B + b0 : (long)(m / rows) * B + b0 + m % rows;
    };
    // x: 2 KT load instructions (K tile i/2, rows 16 (i%2) .. +16), wave w
    // issues i = w, w + NWV, ...; chunk q = 64 (i%2) + lane of the tile holds
    // row q/4, k chunk (q%4) ^ swz(row).  Rows past M repeat row M - 1.
    const char *pa[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = 64 * h + lane, r = q >> 2;
        pa[h] = reinterpret_cast<const char *>(a.hs_x + grow(min(r, M - 1)) * K +
                                               8 * ((q & 3) ^ dma::swz(r)));
    }
    for (int i = wave_s; i < 2 * KT; i += NWV)
        load_lds16(pa[i & 1] + 64 * (i >> 1), lds + 2048 * (i >> 1) + 1024 * (i & 1));
    const char *pb[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int q = 64 * (wave * G + i) + lane, r = q >> 2;
        pb[i] = reinterpret_cast<const char *>(a.hs_wt + (long)(n * GD + r) * K +
                                               8 * ((q & 3) ^ dma::swz(r)));
    }
    auto issue = [&](int kt, int stage) {
        dma::lds_char *st = lds + AR + stage * BS;
#pragma unroll
        for (int i = 0; i < G; ++i) load_lds16(pb[i] + 64 * kt, st + 1024 * (wave_s * G + i));
    };
    const int nb1 = wave + NWV;
    const bool two = nb1 < NB;
    const int sw = dma::swz(l32);
    uint32_t oa[2], ob[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int slot = (2 * kc + lh) ^ sw;
        oa[kc] = (uint32_t)(l32 * 64 + slot * 16);
        ob[kc] = (uint32_t)((wave * 32 + l32) * 64 + slot * 16);
    }
    const uint32_t ob1 = (two ? NWV * 32 * 64 : 0);

    f32x16 acc[2][1];
    acc[0][0] = acc[1][0] = f32x16{};
    for (int p = 0; p < NS - 1 && p < KT; ++p) issue(p, p);
    for (int kt = 0; kt < KT; ++kt) {
        // this wave's loads of W^T tile kt landed (and, older, all of x's):
        // those of up to NS - 2 later tiles may fly, G per tile
        const int later = min(NS - 2, KT - 1 - kt);
        if (later >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * G));
        else if (later == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * G));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(G));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // everyone's tile kt landed; stage kt-1 free
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < KT) issue(kt + NS - 1, (kt + NS - 1) % NS);
        const uint32_t sa = lbase + (uint32_t)(2048 * kt);
        const uint32_t sb = lbase + (uint32_t)(AR + (kt % NS) * BS);
        bf16x8 fa[2], fb[2][2];
        asm volatile("ds_read_b128 %0, %6\n\t"
                     "ds_read_b128 %1, %7\n\t"
                     "ds_read_b128 %2, %8\n\t"
                     "ds_read_b128 %3, %9\n\t"
                     "ds_read_b128 %4, %10\n\t"
                     "ds_read_b128 %5, %11\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(fa[0]), "=&v"(fb[0][0]), "=&v"(fb[0][1]), "=&v"(fa[1]),
                       "=&v"(fb[1][0]), "=&v"(fb[1][1])
                     : "v"(sa + oa[0]), "v"(sb + ob[0]), "v"(sb + ob[0] + ob1), "v"(sa + oa[1]),
                       "v"(sb + ob[1]), "v"(sb + ob[1] + ob1)
                     : "memory");
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kc], fb[kc][0], acc[0][0], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kc], fb[kc][1], acc[1][0], 0, 0, 0);
        }
    }
    head_start_store<G, 1, DH>(a, n, b0, rows, acc);
}

template <int CELL, int DH, int R4, int PD, bool WAIT, bool HB = false, bool LANES = false>
__device__ __forceinline__ void rec_fwd_mfma_body(const RecArgs &a, const int blk,
                                                  uint16_t *h_bf = nullptr,
                                                  unsigned *done = nullptr,
                                                  char *dyn_lds = nullptr) {
    constexpr int G = CellTraits<CELL>::G;
    constexpr int GD = G * DH;
    constexpr int NW = DH / 16;   // waves = 16-unit blocks
    constexpr int KC = DH / 32;   // k chunks of one MFMA
    constexpr int HLD = DH + 8;   // bf16 per h row in LDS (bank spread)
    constexpr bool ROWS1 = R4 == 1 && !LANES;  // one batch row (gate-row layout)
    constexpr int GL = ROWS1 ? 1 : G;          // Gx values per row slot per lane
    constexpr int OUT_ROW = CELL == kLSTM ? 0 : 3;  // R4 == 1: lanes that own the result
    static_assert(DH % 32 == 0, "Dh must be a multiple of 32");
    static_assert(PD % 2 == 0, "groups must keep the h double-buffer parity");
    static_assert(3 * PD < 64, "a group's stores must fit the vmcnt field");
    constexpr bool GXK = ROWS1 && CELL == kLSTM;  // exponent as one fma (gate_rows_update)

    __shared__ __attribute__((aligned(16))) uint16_t hbuf[2][16 * HLD];

    if (a.clear_word && blk == 0 && threadIdx.x == 0) *a.clear_word = 0u;
    // Head start: workgroup i runs on XCD i % 8; numbering the (head, batch
    // tile) pairs head-major within each XCD's share keeps one or two heads'
    // W^T per XCD, which its L2 then holds for all their batch tiles.
    int wi = blk;
    if constexpr (WAIT) {
        const int grid = a.NH * ((a.B + a.BT - 1) / a.BT);
        if (a.hs_steps > 0 && (grid & 7) == 0) {
            const int nbt = grid / a.NH, lg8 = (blk & 7) * (grid >> 3) + (blk >> 3);
            wi = (lg8 % nbt) * a.NH + lg8 / nbt;  // head lg8 / nbt, batch tile lg8 % nbt
        }
    }
    const int n = wi % a.NH;
    const int b0 = (wi / a.NH) * a.BT;
    const int rows = min(a.BT, a.B - b0);
    const int H = a.NH * DH, N = a.NH * GD;
    const int T = a.T, B = a.B;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int j = 16 * wave + lr;  // this lane's hidden unit
    // head start (pipelined forward, Dh = 128): gx of the first steps here
    bool hs = false;
    if constexpr (WAIT && DH >= 64) {
        hs = a.hs_steps > 0 && dyn_lds != nullptr;
        if (hs) {
            if (a.hs_steps * rows > 32) head_start<G, 2, DH>(a, n, b0, rows, dyn_lds);
            else if (kFusedLdsBytes - hs_ares_bytes(a.hs_K) >= 3 * G * DH * 64)
                head_start_ares<G, DH>(a, n, b0, rows, dyn_lds);
            else head_start<G, 1, DH>(a, n, b0, rows, dyn_lds);
        }
    }

    // ---- R_n fragments of this wave's G tiles, resident for all T steps
    bf16x8 rf[G][KC];
    if (a.Rt != nullptr) {
        // R^T: a fragment's eight k of one column are 16 contiguous bytes
        const uint16_t *Rn = a.Rt + (long)n * GD * DH;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < KC; ++c)
                rf[g][c] = *reinterpret_cast<const bf16x8 *>(Rn + (long)(g * DH + j) * DH + 32 * c +
                                                             8 * lg);
    } else {
        const uint16_t *Rn = a.Rb + (long)n * DH * GD;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = g * DH + j;
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = 32 * c + 8 * lg + 2 * e;
                    const uint32_t lo = Rn[(long)k * GD + col];
                    const uint32_t hi = Rn[(long)(k + 1) * GD + col];
                    w[e] = lo | (hi << 16);
                }
                rf[g][c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            }
            // drain this gate's loads before the next gate's are issued: all
            // of them in flight at once would need a register each
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
    }
    for (int i = tid; i < 2 * 16 * HLD; i += NW * 64) (&hbuf[0][0])[i] = 0;
    __syncthreads();

    // Wave-uniform base pointers plus per-lane 32-bit element offsets (B*N <
    // 2^31 is checked on the host): every global access is SGPR-based.
    const float *gx_tile = a.gx + (long)b0 * N + n * GD;
    const long gx_step = (long)B * N, o_step = (long)B * H;
    const long o_tile = (long)b0 * H + n * DH;
    const bool has_h = a.h_seq != nullptr, has_c = CELL == kLSTM && a.c_seq != nullptr;
    // lane roles.  LANES: pass r holds batch row 4*r + lg (gate_update_lanes).
    // Otherwise R4 > 1: row slot r is batch row 4*lg + r.  R4 == 1: batch row
    // 0 only; lane row lg is gate lg for the Gx loads, and the lanes of row
    // OUT_ROW write results.
    bool rv[R4], ld[R4], wr[R4];
    unsigned go[R4], oo[R4];
    int brow[R4];
    float st[R4], hl[R4];
#pragma unroll
    for (int r = 0; r < R4; ++r) {
        const int b = ROWS1 ? 0 : LANES ? 4 * r + lg : 4 * lg + r;
        brow[r] = b;
        rv[r] = b < rows;
        ld[r] = ROWS1 ? lg < G : rv[r];
        wr[r] = ROWS1 ? lg == OUT_ROW : rv[r];
        go[r] = (unsigned)(b * N + (ROWS1 ? lg * DH : 0) + j);
        oo[r] = (unsigned)(b * H + j);
        const float h0 = (rv[r] && a.h0) ? a.h0[o_tile + oo[r]] : 0.f;
        const float c0 = (rv[r] && a.c0) ? a.c0[o_tile + oo[r]] : 0.f;
        st[r] = CELL == kLSTM ? c0 : h0;
        hl[r] = h0;
        if (wr[r]) hbuf[0][b * HLD + j] = f32_to_bf16_rne(h0);
    }

    float bx0[PD][R4][GL], bx1[PD][R4][GL];  // Gx of the current / next group
    float oh[PD][R4], oc[PD][R4];            // outputs of the current group
#pragma unroll
    for (int s = 0; s < PD; ++s)
#pragma unroll
        for (int r = 0; r < R4; ++r) {
            oh[s][r] = oc[s][r] = 0.f;
#pragma unroll
            for (int g = 0; g < GL; ++g) bx0[s][r][g] = bx1[s][r][g] = 0.f;
        }
    // Gx of steps [0, avail) is known complete and acquired (WAIT only).
    int avail = WAIT ? (hs ? min(a.hs_steps, T) : 0) : T, panels_ok = hs ? a.hs_panels : 0;
    auto wait_ready = [&](int tend) {
        if constexpr (WAIT) {
            tend = min(tend, T);
            if (tend <= avail) return;
            const int need = (int)(((long)tend * B + kGemmRowTile - 1) / kGemmRowTile);
            unsigned spins = 0;
            for (;;) {
                const int p = panels_ok + lane;
                const unsigned v = p < a.panels ? __hip_atomic_load(a.ready + p, __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_AGENT)
                                                : a.ready_target;
                const unsigned long long done = __ballot(v >= a.ready_target);
                const int run = ~done == 0ull ? 64 : __builtin_ctzll(~done);
                panels_ok = min(panels_ok + run, a.panels);
                if (panels_ok >= need) break;
                if (++spins >= a.spin_limit) {
                    if (lane == 0)
                        __hip_atomic_store(a.flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    panels_ok = a.panels;  // give up waiting; the results are void
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            avail = panels_ok >= a.panels ? T
                                          : (int)min((long)T, (long)panels_ok * kGemmRowTile / B);
        }
    };
    // Gx of steps [tg, tg+PD) into dst (steps at or past T are skipped).
    auto load_group = [&](int tg, float (&dst)[PD][R4][GL]) {
        const float *src = gx_tile + (long)tg * gx_step;
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (tg + s < T) {
#pragma unroll
                for (int r = 0; r < R4; ++r) {
                    if (ld[r]) {
#pragma unroll
                        for (int g = 0; g < GL; ++g) {
                            if constexpr (WAIT)
                                dst[s][r][g] = __hip_atomic_load(src + go[r] + g * DH, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT);
                            else
                                dst[s][r][g] = src[go[r] + g * DH];
                        }
                    }
                }
            }
            src += gx_step;
        }
    };
    // h/c outputs of steps [tg, tg+PD) held in oh/oc.
    auto store_group = [&](int tg) {
        float *hs = has_h ? a.h_seq + o_tile + (long)tg * o_step : nullptr;
        float *cs = has_c ? a.c_seq + o_tile + (long)tg * o_step : nullptr;
        uint16_t *hb = HB ? h_bf + o_tile + (long)tg * o_step : nullptr;
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (tg + s < T) {
#pragma unroll
                for (int r = 0; r < R4; ++r) {
                    if (wr[r]) {
                        if (has_h) hs[oo[r]] = oh[s][r];
                        if (has_c) cs[oo[r]] = oc[s][r];
                        if constexpr (HB)
                            __hip_atomic_store(hb + oo[r], f32_to_bf16_rne(oh[s][r]),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            hs += o_step;
            cs += o_step;
            if constexpr (HB) hb += o_step;
        }
    };
    // HB: a full group's stores (PD steps of h, c and the bf16 h) and the
    // count after them are the last vector-memory instructions of a group;
    // wait for all older ones.
    const int nst = (has_h ? 1 : 0) + (has_c ? 1 : 0) + 1;
    auto wait_but_stores = [&]() {
        if (nst == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PD + 1));
        else if (nst == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PD + 1));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PD + 1));
    };
    // HB with `done`, wave 0 at the second step of group tg: every wave's
    // stores of steps [tg - 3PD, tg - 2PD) are complete; count them.
    int counted = 0;  // steps [0, counted) counted (wave 0)
    auto publish = [&](int tg) {
        if constexpr (HB) {
            if (done == nullptr || wave != 0) return;
            const int t0 = tg - 3 * PD;
            if (t0 >= 0) {
                if (lane < PD)
                    __hip_atomic_fetch_add(done + t0 + lane, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                counted = t0 + PD;
            }
        }
    };
    // A operand: lanes of live batch rows load it from LDS every step; the
    // other lanes keep the zeros they start with (rewriting them every step
    // would cost a dozen moves on the step's critical path).
    bf16x8 af[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) af[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    auto read_chunks = [&](const uint16_t *hb, int c0, int c1) {
        if (lr < rows) {
#pragma unroll
            for (int c = c0; c < c1; ++c)
                af[c] = *reinterpret_cast<const bf16x8 *>(hb + lr * HLD + 32 * c + 8 * lg);
        }
    };
    // acc += h chunks [c0, c1) times this wave's R fragments, k-chunk after
    // k-chunk (the first MFMAs need only the first LDS read)
    f32x4 acc[G];
    auto mfma_chunks = [&](int c0, int c1) {
#pragma unroll
        for (int c = c0; c < c1; ++c)
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = mfma_16x16x32_bf16(af[c], rf[g][c], acc[g]);
    };
    // Group traffic at the first step of a group: the previous group's
    // outputs stored, the next group's Gx requested.
    auto group_traffic = [&](int tg, float (&nxt)[PD][R4][GL]) {
        if constexpr (HB) {
            wait_ready(tg + 2 * PD);
            load_group(tg + PD, nxt);
            if (tg > 0) store_group(tg - PD);
        } else {
            if (tg > 0) store_group(tg - PD);
            wait_ready(tg + 2 * PD);
            load_group(tg + PD, nxt);
        }
    };
    // Cell update of step s of the group and h_t into the LDS buffer hn.
    auto cell = [&](int s, float (&use)[PD][R4][GL], uint16_t *hn) {
        float h[R4], c[R4];
        if constexpr (LANES)
            gate_update_lanes<CELL, R4>(acc, use[s], st, hl, h, c);
        else
            gate_update<CELL, R4, GL, GXK>(acc, use[s], st, hl, h, c);
#pragma unroll
        for (int r = 0; r < R4; ++r) {
            oh[s][r] = h[r];
            oc[s][r] = c[r];
            if (wr[r]) hn[brow[r] * HLD + j] = f32_to_bf16_rne(h[r]);
        }
    };
    // PD steps starting at tg, reading Gx from `use`; at the first step the
    // previous group's outputs are stored and the next group's Gx requested.
    // FULL: every step of the group is < T (no per-step bound checks).
    auto run_group = [&](auto full, int tg, float (&use)[PD][R4][GL],
                         float (&nxt)[PD][R4][GL]) {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (!decltype(full)::value && tg + s >= T) break;
            // first step of a group: everything still in flight was issued a
            // whole group ago; drain it here, before the new group's requests
            // go out, so no later use of `use` has to wait on those.
            if constexpr (HB) {
                if (s == 0) wait_but_stores();
                if (s == 1) publish(tg);
            } else {
                if (s == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            }
            const uint16_t *hc = hbuf[s & 1];
            uint16_t *hn = hbuf[(s + 1) & 1];
            read_chunks(hc, 0, KC);
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            mfma_chunks(0, KC);
            // steps are unrolled: only a group's first step branches right
            // after the chain (the HBM traffic of the group), so only it needs
            // the pinned wait states
            if (s == 0) {
                mfma_chain_end();
                group_traffic(tg, nxt);
            }
            cell(s, use, hn);
            lds_barrier();
        }
    };
    wait_ready(PD);
    load_group(0, bx0);
    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;
    const int tfull = T / (2 * PD) * (2 * PD);
    for (int tg = 0; tg < tfull; tg += 2 * PD) {
        run_group(Full{}, tg, bx0, bx1);
        run_group(Full{}, tg + PD, bx1, bx0);
    }
    int tlast = tfull - PD;
    if (tfull < T) {
        run_group(Part{}, tfull, bx0, bx1);
        tlast = tfull;
        if (tfull + PD < T) {
            run_group(Part{}, tfull + PD, bx1, bx0);
            tlast = tfull + PD;
        }
    }
    store_group(tlast);
#pragma unroll
    for (int r = 0; r < R4; ++r) {
        if (wr[r]) {
            a.hT[o_tile + oo[r]] = CELL == kLSTM ? hl[r] : st[r];
            if (CELL == kLSTM) a.cT[o_tile + oo[r]] = st[r];
        }
    }
    if constexpr (HB) {
        if (done != nullptr) {
            // the steps not counted yet, once every wave's stores are done
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
            if (wave == 0)
                for (int t = counted + lane; t < T; t += 64)
                    __hip_atomic_fetch_add(done + t, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int CELL, int DH, int R4, int PD, bool WAIT, bool LANES>
__global__ __launch_bounds__(DH / 16 * 64) void rec_fwd_mfma_kernel(RecArgs a) {
    rec_fwd_mfma_body<CELL, DH, R4, PD, WAIT, false, LANES>(a, blockIdx.x);
}

// The pipelined forward as one launch (512-thread workgroups; at Dh = 64 the
// recurrence uses four of the eight waves): workgroups [0, n_gemm) compute the input projection, output
// tiles in time order and each finished tile counted on its row panel;
// the rest run the recurrence, waiting for the panels of their next steps.
// Workgroups are dispatched in index order, so every projection workgroup
// is resident before any recurrence workgroup starts to wait, and the
// projection waits on nothing: the launch cannot stall on itself, whatever
// else shares the chip.
static_assert(dma::LDS_BYTES <= (size_t)kFusedLdsBytes, "the projection's ring fits");
static_assert(kHeadStartRows <= 64, "the head start holds at most two row blocks");
template <int CELL, int DH, int R4, int PD, bool LANES>
__global__ __launch_bounds__(512) void fwd_fused_kernel(RecArgs a, GemmArgs g, int n_gemm,
                                                        int rows1, int n_gemm2) {
    static_assert(DH == 128 || DH == 64, "the recurrence takes all eight waves or the first four");
    extern __shared__ __attribute__((aligned(16))) char fused_lds[];
    if ((int)blockIdx.x < n_gemm) {
        const int wg = blockIdx.x;
        if (rows1 > 0 && rows1 < g.M && n_gemm2 > 0) {
            // the first rows1 rows (whole panels) on all n_gemm workgroups,
            // the rest on the first n_gemm2 of them
            GemmArgs g1 = g;
            g1.M = rows1;
            dma::gemm_dma_tiles(g1, wg, n_gemm, (dma::lds_char *)fused_lds);
            if (wg < n_gemm2) {
                GemmArgs g2 = g;
                g2.M = g.M - rows1;
                g2.A = g.A + (long)rows1 * g.lda;
                g2.C = g.C + (long)rows1 * g.ldc;
                g2.ready = g.ready + rows1 / kGemmRowTile;
                dma::gemm_dma_tiles(g2, wg, n_gemm2, (dma::lds_char *)fused_lds);
            }
        } else {
            dma::gemm_dma_tiles(g, wg, n_gemm, (dma::lds_char *)fused_lds);
        }
        return;
    }
    // Dh = 64: the recurrence runs on four waves; the other four end here, on
    // a scalar branch (a workgroup barrier waits only for the waves still
    // running; a wave left running with no lanes active would take part)
    if (DH < 128 && __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) >= DH / 16) return;
    rec_fwd_mfma_body<CELL, DH, R4, PD, true, false, LANES>(a, blockIdx.x - n_gemm, nullptr,
                                                            nullptr, fused_lds);
}

// Two stacked layers in one launch (see StackSync): [0, R) layer l's
// recurrence, [R, R + n_gemm) layer l+1's input projection, then layer
// l+1's recurrence.  Every role waits only on workgroups of lower index,
// which are dispatched first, so the launch cannot stall on itself; each
// wait is bounded by a.spin_limit and then sets the abort word.
//
// A tile of the projection covers rows [256 mt, 256 mt + 256) of the
// [T*B] rows of h_bf0, i.e. the steps up to (256 mt + 255) / B; wave 0
// polls the step counters (64 per poll) until those steps are counted by
// every workgroup of layer l (y.done_target), then the tile's barrier releases
// the other waves.  A's loads are device-scope (they miss in the XCD's L2,
// like the stores that wrote them); the weights load as usual.
template <int CELL, int PD0, int PD, bool HB1>
__global__ __launch_bounds__(512) void fwd_stack2_kernel(RecArgs a0, RecArgs a1, GemmArgs g,
                                                         StackSync y) {
    extern __shared__ __attribute__((aligned(16))) char stack_lds[];
    const int blk = blockIdx.x;
    if (blk < y.rec_grid) {
        rec_fwd_mfma_body<CELL, 128, 1, PD0, false, true>(a0, blk, y.h_bf0, y.done);
        return;
    }
    const int gb = blk - y.rec_grid;
    if (gb < y.n_gemm) {
        const int T = a0.T, B = a0.B, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const unsigned target = y.done_target;
        const long rows = (long)T * B;
        int steps_ok = 0;
        auto wait_rows = [&](int mt) {
            if (wave != 0) return;
            const long last = min((long)(mt + 1) * kGemmRowTile, rows) - 1;
            const int need = (int)(last / B) + 1;
            unsigned spins = 0;
            while (steps_ok < need) {
                const int t = steps_ok + lane;
                const unsigned v = t < T ? __hip_atomic_load(y.done + t, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)
                                         : target;
                const unsigned long long ok = __ballot(v >= target);
                const int run = ~ok == 0ull ? 64 : __builtin_ctzll(~ok);
                steps_ok = min(steps_ok + run, T);
                if (steps_ok >= need) break;
                if (++spins >= a0.spin_limit) {
                    if (lane == 0)
                        __hip_atomic_store(a0.flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    steps_ok = T;  // give up waiting; the results are void
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        };
        dma::gemm_dma_tiles_pre<16>(g, gb, y.n_gemm, (dma::lds_char *)stack_lds, wait_rows);
        return;
    }
    rec_fwd_mfma_body<CELL, 128, 1, PD, true, HB1>(a1, gb - y.n_gemm, y.h_bf1, nullptr);
}

// Simple kernel: dynamic LDS = R [Dh][G*Dh] f32 | h operand [BT][Dh] |
// c state [BT][Dh] | h state [BT][Dh] | gate pre-activations [BT][G*Dh].
template <int CELL, bool BF16>
__global__ __launch_bounds__(256) void rec_fwd_simple_kernel(RecArgs a) {
    constexpr int G = CellTraits<CELL>::G;
    extern __shared__ float smem[];
    const int DH = a.Dh, GD = G * DH, BT = a.BT;
    float *Rs = smem;
    float *hop = Rs + DH * GD;
    float *cs = hop + BT * DH;
    float *hs = cs + BT * DH;
    float *gs = hs + BT * DH;

    if (a.clear_word && blockIdx.x == 0 && threadIdx.x == 0) *a.clear_word = 0u;
    const int n = blockIdx.x % a.NH;
    const int b0 = (blockIdx.x / a.NH) * BT;
    const int rows = min(BT, a.B - b0);
    const int H = a.NH * DH, N = a.NH * GD;
    const int tid = threadIdx.x;

    for (int i = tid; i < DH * GD; i += 256)
        Rs[i] = BF16 ? bf16_to_f32(a.Rb[(long)n * DH * GD + i]) : a.Rf[(long)n * DH * GD + i];
    for (int i = tid; i < rows * DH; i += 256) {
        const int b = i / DH, j = i - b * DH;
        const long o = (long)(b0 + b) * H + n * DH + j;
        const float h = a.h0 ? a.h0[o] : 0.f;
        hs[i] = h;
        cs[i] = a.c0 ? a.c0[o] : 0.f;
        hop[i] = BF16 ? bf16_to_f32(f32_to_bf16_rne(h)) : h;
    }
    __syncthreads();
    for (int t = 0; t < a.T; ++t) {
        for (int p = tid; p < rows * GD; p += 256) {
            const int b = p / GD, col = p - b * GD;
            float s = 0.f;
            for (int m = 0; m < DH; ++m) s = fmaf(hop[b * DH + m], Rs[m * GD + col], s);
            gs[p] = s;
        }
        __syncthreads();
        for (int i = tid; i < rows * DH; i += 256) {
            const int b = i / DH, j = i - b * DH;
            const float *src = a.gx + ((long)t * a.B + b0 + b) * N + n * GD + j;
            float gxv[G];
#pragma unroll
            for (int g = 0; g < G; ++g) gxv[g] = src[g * DH];
            float h, c;
            lstm_or_gru_unit<CELL>(gs + b * GD + j, DH, gxv, cs[i], hs[i], h, c);
            hop[i] = BF16 ? bf16_to_f32(f32_to_bf16_rne(h)) : h;
            const long o = ((long)t * a.B + b0 + b) * H + n * DH + j;
            if (a.h_seq) a.h_seq[o] = h;
            if (CELL == kLSTM && a.c_seq) a.c_seq[o] = c;
        }
        __syncthreads();
    }
    for (int i = tid; i < rows * DH; i += 256) {
        const int b = i / DH, j = i - b * DH;
        const long o = (long)(b0 + b) * H + n * DH + j;
        a.hT[o] = hs[i];
        if (CELL == kLSTM) a.cT[o] = cs[i];
    }
}

// One batch row: the gate-row layout.  Two to eight rows: rows in lane
// groups, one cell update pass per four rows (upt passes).  More: the
// register-slot layout, four passes (the same count, with fewer live
// registers).  Each with its prefetch group length (steps).  One row with
// nothing to wait on, LSTM with Dh=128: groups of two steps (groups of eight
// cost about 4% more time per step, four or six about 2-3%); GRU with Dh=64:
// groups of sixteen (eight and twelve 0.7% slower, twenty 1.4%, two 7%).
// Other shapes keep eight (longer groups hold more registers; not measured).
// Launched beside the projection and waiting on its ready words, the LSTM
// with Dh=128 takes groups of six (per call: eight 0.539 ms, four 0.533, six
// 0.525, two 0.562) and the GRU with Dh=64 sixteen (eight 0.549, twelve
// 0.542, sixteen 0.538, twenty 0.537, four and six 2-5% slower than eight);
// in the stacked launch, layer 0 (no waits, but a count published per group)
// takes twelve and layer 1 eight (per call 0.747 ms; layer 0 at eight 0.753,
// sixteen 0.756, six 0.775, two 1.03).
template <int CELL, int DH, bool WAIT>
void launch_mfma_rows_w(const RecPlan &p, const RecArgs &a, hipStream_t s) {
    const dim3 grid(p.grid), blk(DH / 16 * 64);
    if (p.BT == 1) {
        constexpr int PD1 = WAIT                           ? 8
                            : (CELL == kLSTM && DH == 128) ? 2
                            : (CELL == kGRU && DH == 64)   ? 16
                                                           : 8;
        hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, 1, PD1, WAIT, false>), grid, blk, 0, s, a);
        return;
    }
    switch (p.upt) {
        case 1:
            hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, 1, 4, WAIT, true>), grid, blk, 0, s, a);
            break;
        case 2:
            hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, 2, 2, WAIT, true>), grid, blk, 0, s, a);
            break;
        default:
            hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, 4, 2, WAIT, false>), grid, blk, 0, s, a);
            break;
    }
}

template <int CELL, int DH>
hipError_t launch_mfma_rows(const RecPlan &p, const RecArgs &a, hipStream_t s) {
    launch_mfma_rows_w<CELL, DH, false>(p, a, s);
    return hipGetLastError();
}


template <int CELL>
hipError_t launch_mfma(const RecPlan &p, const RecArgs &a, hipStream_t s) {
    switch (a.Dh) {
        case 32: return launch_mfma_rows<CELL, 32>(p, a, s);
        case 64: return launch_mfma_rows<CELL, 64>(p, a, s);
        case 128: return launch_mfma_rows<CELL, 128>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

RecPlan plan_rec(int cell, int T, int B, int NH, int Dh, bool bf16, int num_cu,
                 int bt_override) {
    (void)T;
    RecPlan p{};
    const int G = cell == kLSTM ? 4 : 3;
    const bool mfma_ok = bf16 && (Dh == 32 || Dh == 64 || Dh == 128);
    if (mfma_ok) {
        p.kind = kRecMfma;
        int bt = 16;
        // spread the independent (head, row) chains over as many CUs as the
        // chip has: rows per workgroup shrink until the grid would overflow
        while (bt > 1 && (long)NH * ((B + bt / 2 - 1) / (bt / 2)) <= num_cu) bt /= 2;
        if (bt_override > 0) bt = bt_override < 16 ? bt_override : 16;
        if (bt > B) bt = B;
        p.BT = bt;
        p.nbt = (B + bt - 1) / bt;
        p.grid = NH * p.nbt;
        p.waves = Dh / 16;
        p.threads = p.waves * 64;
        p.upt = bt <= 4 ? 1 : bt <= 8 ? 2 : 4;  // cell update passes per step
        // (rows in lane groups up to 8 rows, register slots beyond)
        p.lds = 0;
        return p;
    }
    // simple kernel: R [Dh][G*Dh] f32 + 3 x [BT][Dh] + [BT][G*Dh] in <= 64 KiB
    int bt = B < 16 ? B : 16;
    if (bt_override > 0 && bt_override < bt) bt = bt_override;
    for (;;) {
        const size_t lds = sizeof(float) * ((size_t)Dh * G * Dh + 3u * bt * Dh + (size_t)bt * G * Dh);
        if (lds <= 65536) {
            p.kind = kRecSimple;
            p.BT = bt;
            p.nbt = (B + bt - 1) / bt;
            p.grid = NH * p.nbt;
            p.threads = 256;
            p.waves = 4;
            p.upt = 0;
            p.lds = lds;
            return p;
        }
        if (bt == 1) break;
        bt = (bt + 1) / 2;
    }
    p.kind = kRecNone;
    return p;
}

template <int CELL, int DH, int R4, int PD, bool LANES>
hipError_t launch_fused_t(const RecPlan &p, const RecArgs &a, const GemmArgs &g, int n_gemm,
                          int rows1, int n_gemm2, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&fwd_fused_kernel<CELL, DH, R4, PD, LANES>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLdsBytes);
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((fwd_fused_kernel<CELL, DH, R4, PD, LANES>), dim3(n_gemm + p.grid),
                       dim3(512), (size_t)kFusedLdsBytes, s, a, g, n_gemm, rows1, n_gemm2);
    return hipGetLastError();
}

template <int DH>
hipError_t launch_fused_dh(int cell, const RecPlan &p, const RecArgs &a, const GemmArgs &g,
                           int n_gemm, int rows1, int n_gemm2, hipStream_t s) {
    if (p.BT == 1)
        return cell == kLSTM ? launch_fused_t<kLSTM, DH, 1, (DH == 128 ? 6 : 8), false>(p, a, g, n_gemm, rows1, n_gemm2, s)
                             : launch_fused_t<kGRU, DH, 1, (DH == 64 ? 16 : 8), false>(p, a, g, n_gemm, rows1, n_gemm2, s);
    switch (p.upt) {
        case 1: return cell == kLSTM ? launch_fused_t<kLSTM, DH, 1, 4, true>(p, a, g, n_gemm, rows1, n_gemm2, s)
                                     : launch_fused_t<kGRU, DH, 1, 4, true>(p, a, g, n_gemm, rows1, n_gemm2, s);
        case 2: return cell == kLSTM ? launch_fused_t<kLSTM, DH, 2, 2, true>(p, a, g, n_gemm, rows1, n_gemm2, s)
                                     : launch_fused_t<kGRU, DH, 2, 2, true>(p, a, g, n_gemm, rows1, n_gemm2, s);
        default: return cell == kLSTM ? launch_fused_t<kLSTM, DH, 4, 2, false>(p, a, g, n_gemm, rows1, n_gemm2, s)
                                      : launch_fused_t<kGRU, DH, 4, 2, false>(p, a, g, n_gemm, rows1, n_gemm2, s);
    }
}


hipError_t launch_fwd_fused(int cell, const RecPlan &p, const RecArgs &a, const GemmArgs &g,
                            int n_gemm, hipStream_t s, int rows1, int n_gemm2) {
    if (p.kind != kRecMfma || (a.Dh != 128 && a.Dh != 64) || !a.ready || !g.ready ||
        n_gemm <= 0 || !gemm_dma_ok(g.K) || rows1 % kGemmRowTile != 0 || n_gemm2 > n_gemm ||
        (n_gemm2 > 0 && n_gemm2 % 8 != 0))
        return hipErrorInvalidValue;
    return a.Dh == 128 ? launch_fused_dh<128>(cell, p, a, g, n_gemm, rows1, n_gemm2, s)
                       : launch_fused_dh<64>(cell, p, a, g, n_gemm, rows1, n_gemm2, s);
}

template <int CELL, bool HB1>
hipError_t launch_stack2_t(const RecArgs &a0, const RecArgs &a1, const GemmArgs &g,
                           const StackSync &y, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_stack2_kernel<CELL, 12, 8, HB1>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)dma::LDS_BYTES);
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((fwd_stack2_kernel<CELL, 12, 8, HB1>), dim3(2 * y.rec_grid + y.n_gemm),
                       dim3(512), dma::LDS_BYTES, s, a0, a1, g, y);
    return hipGetLastError();
}

hipError_t launch_fwd_stack2(int cell, const RecPlan &p, const RecArgs &a0, const RecArgs &a1,
                             const GemmArgs &g, const StackSync &y, hipStream_t s) {
    if (p.kind != kRecMfma || p.upt != 1 || p.BT != 1 || a0.Dh != 128 || a1.Dh != 128 ||
        a0.ready || !a1.ready || a1.ready != g.ready || !y.done || !y.h_bf0 || y.n_gemm <= 0 ||
        y.rec_grid != p.grid || y.done_target != (unsigned)p.grid ||
        g.A != y.h_bf0 || !gemm_dma_ok(g.K) || g.ksplit != 1)
        return hipErrorInvalidValue;
    const bool hb1 = y.h_bf1 != nullptr;
    if (cell == kLSTM)
        return hb1 ? launch_stack2_t<kLSTM, true>(a0, a1, g, y, s)
                   : launch_stack2_t<kLSTM, false>(a0, a1, g, y, s);
    return hb1 ? launch_stack2_t<kGRU, true>(a0, a1, g, y, s)
               : launch_stack2_t<kGRU, false>(a0, a1, g, y, s);
}

hipError_t launch_rec_fwd(int cell, const RecPlan &p, const RecArgs &a, bool bf16,
                          hipStream_t s) {
    if (a.ready) return hipErrorInvalidValue;  // waiting recurrences run fused
    if (p.kind == kRecMfma) {
        return cell == kLSTM ? launch_mfma<kLSTM>(p, a, s) : launch_mfma<kGRU>(p, a, s);
    }
    if (p.kind == kRecSimple) {
        dim3 g(p.grid), blk(256);
        if (cell == kLSTM) {
            if (bf16) hipLaunchKernelGGL((rec_fwd_simple_kernel<kLSTM, true>), g, blk, p.lds, s, a);
            else hipLaunchKernelGGL((rec_fwd_simple_kernel<kLSTM, false>), g, blk, p.lds, s, a);
        } else {
            if (bf16) hipLaunchKernelGGL((rec_fwd_simple_kernel<kGRU, true>), g, blk, p.lds, s, a);
            else hipLaunchKernelGGL((rec_fwd_simple_kernel<kGRU, false>), g, blk, p.lds, s, a);
        }
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace rnn355
