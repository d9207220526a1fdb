// rec_mc.hip -- forward recurrence for heads whose R block does not fit one
// compute unit: the hidden units of one head are split over K workgroups
// (one per CU, all resident at once, checked on the host) that swap h_t through
// global memory at every step.
//
// FlashRNN (arXiv 2412.07752, abstract) stresses that its CUDA kernels reach
// much larger hidden sizes than its Triton ones; the blog post
// (blog.hotdry.top 2025-09-21, the paragraphs on the step dependency and on
// keeping R in registers) explains the price: R stays on chip, so a large R
// must be spread over several processors that then meet once per step.
//
// Per workgroup: U = Dh/K units, NB = U/16 unit blocks, and KS waves per unit
// block, each holding KCW = Dh/(32*KS) k-chunks of the MFMA B fragments of
// its block's G gate tiles (G * KCW * 4 VGPRs, R never re-read).  Per step:
//   1. A fragments of h_{t-1} (bf16, LDS, full Dh, double-buffered by step
//      parity) for the wave's k-range;
//   2. MFMAs -> partial gate sums; waves with ks > 0 hand theirs to the
//      ks = 0 wave of the block through LDS;
//   3. the ks = 0 waves apply the cell update (same code as the one-CU
//      kernel) and publish h_t into the group's exchange slot: 8-byte words of
//      two bf16 values plus the step number, written as relaxed agent-scope
//      atomics (single-copy atomic and coherent across XCDs), so a reader that
//      sees the step number sees the values with it -- no counter, no fence,
//      no cache write-back or invalidation (those act on a whole XCD's L2 and
//      would stall every other group on it);
//   4. every thread polls its share of the words of the slot until all carry
//      step t and copies them into LDS.  Polls are bounded: on time-out the
//      workgroup raises the abort word, which every poller checks, so all
//      members stop and the kernel ends;
//   5. the h/c outputs of step t are stored and Gx of step t+1 requested,
//      so they drain during the next step.
// XCD-local exchange (xcd.h): with the xcd_map numbering the members of a
// group run on one XCD, which each launch checks.  Then the group's words are
// stored into the shared L2 without the write-through to memory (sc0
// stores), which the members' device-scope polls (sc1 loads, served by that
// L2) see at once: measured between two CUs, a 421 ns round trip against
// 673 ns (same XCD) and 773 ns (two XCDs) with write-through stores.  Such a
// store is not seen from another XCD, so only a group found on one XCD takes
// that path; the others keep the write-through stores.
#include <hip/hip_runtime.h>

#include "common.h"
#include "gates.h"
#include "kernels.h"
#include "xcd.h"

namespace rnn355 {

namespace {

// RL: batch rows in lane groups (gate_update_lanes): each cell update pass
// serves four rows at once, R4 passes cover 4 R4 rows (the slot layout runs
// one pass per register, four passes for any tile of more than two rows).
template <int CELL, int KCW, int R4, bool RL = false>
__global__ __launch_bounds__(512) void rec_fwd_mc_kernel(McArgs m) {
    constexpr int G = CellTraits<CELL>::G;
    constexpr bool ROWS1 = R4 == 1 && !RL;
    constexpr int GL = ROWS1 ? 1 : G;
    constexpr int OUT_ROW = CELL == kLSTM ? 0 : 3;
    const RecArgs &a = m.r;
    const int Dh = a.Dh, K = m.K, KS = m.KS, NB = m.NB;
    const int U = NB * 16, GD = G * Dh, H = a.NH * Dh, N = a.NH * GD, HLD = Dh + 8;
    const int T = a.T, B = a.B;

    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    // h_{t-1} as bf16, double-buffered by step parity: step t reads buffer
    // t&1 and fills buffer (t+1)&1, which nobody reads any more (its last
    // readers finished before the closing barrier of step t-1)
    uint16_t *hbuf2 = smem;                                       // [2][16][HLD] bf16
    float *red = reinterpret_cast<float *>(smem + 2 * 16 * HLD);  // [KS-1][NB][G][16][16]
    __shared__ int s_abort, s_local;

    int group, member;
    group_member(m.xcd_map != 0, K, group, member);
    const int n = group % a.NH;
    const int b0 = (group / a.NH) * a.BT;
    const int rows = min(a.BT, B - b0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int blk = wave / KS, ks = wave - blk * KS;
    const bool gate_wave = ks == 0;
    const int j = member * U + blk * 16 + lr;  // this lane's hidden unit
    const int kc0 = ks * KCW;                  // first k-chunk of this wave

    bf16x8 rf[G][KCW];
    {
        const uint16_t *Rn = a.Rb + (long)n * Dh * GD;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = g * Dh + j;
#pragma unroll
            for (int c = 0; c < KCW; ++c) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = 32 * (kc0 + c) + 8 * lg + 2 * e;
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
    const int nthr = blockDim.x;
    for (int i = tid; i < 2 * 16 * HLD; i += nthr) {
        const int b = (i / HLD) & 15, k = i % HLD;
        float v = 0.f;
        if (i < 16 * HLD && b < rows && k < Dh && a.h0) v = a.h0[(long)(b0 + b) * H + n * Dh + k];
        hbuf2[i] = f32_to_bf16_rne(v);
    }
    if (tid == 0) {
        s_abort = 0;
        s_local = 0;
    }
    if (m.xcd_map) xcd_publish(m.xcc);

    // lanes of the ks = 0 waves own units (same roles as the one-CU kernel)
    const float *gx_tile = a.gx + (long)b0 * N + n * GD;
    const long gx_step = (long)B * N, o_step = (long)B * H;
    const long o_tile = (long)b0 * H + n * Dh;
    const bool has_h = a.h_seq != nullptr, has_c = CELL == kLSTM && a.c_seq != nullptr;
    bool rv[R4], ld[R4], wr[R4];
    unsigned go[R4], oo[R4];
    float st[R4], hl[R4], gxr[R4][GL], ph[R4], pc[R4];
#pragma unroll
    for (int r = 0; r < R4; ++r) {
        const int b = RL ? 4 * r + lg : ROWS1 ? 0 : 4 * lg + r;
        rv[r] = b < rows;
        ld[r] = gate_wave && (ROWS1 ? lg < G : rv[r]);
        wr[r] = gate_wave && (ROWS1 ? lg == OUT_ROW : rv[r]);
        go[r] = (unsigned)(b * N + (ROWS1 ? lg * Dh : 0) + j);
        oo[r] = (unsigned)(b * H + j);
        const float h0 = (rv[r] && a.h0) ? a.h0[o_tile + oo[r]] : 0.f;
        const float c0 = (rv[r] && a.c0) ? a.c0[o_tile + oo[r]] : 0.f;
        st[r] = CELL == kLSTM ? c0 : h0;
        hl[r] = h0;
        ph[r] = pc[r] = 0.f;
#pragma unroll
        for (int g = 0; g < GL; ++g) gxr[r][g] = 0.f;
    }
    auto load_gx = [&](int t) {
        const float *src = gx_tile + (long)t * gx_step;
#pragma unroll
        for (int r = 0; r < R4; ++r)
            if (ld[r])
#pragma unroll
                for (int g = 0; g < GL; ++g) gxr[r][g] = src[go[r] + g * Dh];
    };
    load_gx(0);
    __syncthreads();
    if (m.xcd_map && wave == 0) {
        const int v = xcd_members_agree(m.xcc, m.flag, m.spin_limit, group, K);
        if (lane == 0) {
            s_local = v > 0;
            if (v < 0) s_abort = 1;
        }
    }
    __syncthreads();
    const bool local = s_local != 0;

    // exchange slots of the group: [2 parities][BT rows][Dh/2] words
    unsigned long long *xs_group = m.xg + (long)group * 2 * a.BT * (Dh / 2);
    const int wpr = Dh / 2;  // words per row
    // A operand: lanes of live batch rows load it every step.  With one row
    // slot the other lanes keep the zeros they start with (rewriting them
    // every step costs a dozen moves on the step's critical path); with more
    // they are rewritten (keeping them would spill).
    bf16x8 af[KCW];
#pragma unroll
    for (int c = 0; c < KCW; ++c) af[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    int t = s_abort ? T + 1 : 0;
    for (; t < T; ++t) {
        const uint16_t *hbuf = hbuf2 + (t & 1) * 16 * HLD;
        if (lr < rows) {
#pragma unroll
            for (int c = 0; c < KCW; ++c)
                af[c] = *reinterpret_cast<const bf16x8 *>(hbuf + lr * HLD + 32 * (kc0 + c) + 8 * lg);
        } else if (R4 > 1) {
#pragma unroll
            for (int c = 0; c < KCW; ++c) af[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
        f32x4 acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KCW; ++c)
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = mfma_16x16x32_bf16(af[c], rf[g][c], acc[g]);
        mfma_chain_end();

        if (KS > 1) {
            // partial sums of the other k-ranges -> the ks = 0 wave of the block
            if (!gate_wave) {
                float *dst = red + ((long)(ks - 1) * NB + blk) * G * 256;
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(g * 16 + 4 * lg + r) * 16 + lr] = acc[g][r];
            }
            __syncthreads();
            if (gate_wave) {
                for (int k2 = 1; k2 < KS; ++k2) {
                    const float *src = red + ((long)(k2 - 1) * NB + blk) * G * 256;
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[g][r] += src[(g * 16 + 4 * lg + r) * 16 + lr];
                }
            }
        }
        unsigned long long *slot = xs_group + (long)(t & 1) * a.BT * wpr;
        const unsigned long long tag = (unsigned long long)(unsigned)(t + 1) << 32;
        if (gate_wave) {
            float h[R4], c[R4];
            if constexpr (RL) {
                gate_update_lanes<CELL, R4>(acc, gxr, st, hl, h, c);
            } else {
                gate_update<CELL, R4>(acc, gxr, st, hl, h, c);
            }
#pragma unroll
            for (int r = 0; r < R4; ++r) {
                ph[r] = h[r];
                pc[r] = c[r];
                // units j, j+1 live in neighbouring lanes: the even lane
                // writes both with the step number
                const unsigned hb = f32_to_bf16_rne(h[r]);
                const unsigned nb = (unsigned)__shfl_xor((int)hb, 1);
                if (wr[r] && (lr & 1) == 0) {
                    unsigned long long *dst =
                        slot + (RL ? 4 * r + lg : ROWS1 ? 0 : 4 * lg + r) * wpr + (j >> 1);
                    const unsigned long long w = tag | (nb << 16) | hb;
                    if (local)
                        __hip_atomic_store(dst, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    else
                        __hip_atomic_store(dst, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        // ---- collect h_t of every member: poll each word until it carries
        // step t, PW words of a thread per poll with all their loads in flight
        // together (a word already seen is read again: its slot is not
        // rewritten before every member has finished this step)
        {
            constexpr int PW = 4;
            const int words = rows * wpr;
            unsigned *hw = reinterpret_cast<unsigned *>(hbuf2 + ((t + 1) & 1) * 16 * HLD);
            for (int i0 = tid; i0 < words; i0 += PW * nthr) {
                unsigned spins = 0;
                unsigned long long w[PW];
                for (;;) {
                    bool all = true;
#pragma unroll
                    for (int q = 0; q < PW; ++q) {
                        const int i = i0 + q * nthr;
                        w[q] = i < words ? __hip_atomic_load(slot + i, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)
                                         : tag;
                    }
#pragma unroll
                    for (int q = 0; q < PW; ++q) all = all && (w[q] & 0xFFFFFFFF00000000ull) == tag;
                    if (all) break;
                    ++spins;
                    if ((spins & 255u) == 0 &&
                        __hip_atomic_load(m.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                        s_abort = 1;
                        break;
                    }
                    if (spins >= m.spin_limit) {
                        __hip_atomic_store(m.flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        s_abort = 1;
                        break;
                    }
                }
                if (s_abort) break;
#pragma unroll
                for (int q = 0; q < PW; ++q) {
                    const int i = i0 + q * nthr;
                    if (i < words) {
                        const int b = i / wpr, k2 = i - b * wpr;
                        hw[(b * HLD) / 2 + k2] = (unsigned)w[q];
                    }
                }
            }
        }
        __syncthreads();
        if (s_abort) break;
        // ---- outputs of step t, Gx of step t+1
        if (gate_wave) {
            const long base = o_tile + (long)t * o_step;
#pragma unroll
            for (int r = 0; r < R4; ++r) {
                if (wr[r]) {
                    if (has_h) a.h_seq[base + oo[r]] = ph[r];
                    if (has_c) a.c_seq[base + oo[r]] = pc[r];
                }
            }
            if (t + 1 < T) load_gx(t + 1);
        }
    }
    if (t == T) {
#pragma unroll
        for (int r = 0; r < R4; ++r) {
            if (wr[r]) {
                a.hT[o_tile + oo[r]] = CELL == kLSTM ? hl[r] : st[r];
                if (CELL == kLSTM) a.cT[o_tile + oo[r]] = st[r];
            }
        }
    }
}

// Zeroes up to three word ranges (null pointers skipped) in one launch.
__global__ void clear_words_kernel(unsigned *p, int n, unsigned *p2, int n2, unsigned *p3, int n3) {
    const int i0 = blockIdx.x * blockDim.x + threadIdx.x, step = gridDim.x * blockDim.x;
    if (p)
        for (int i = i0; i < n; i += step) p[i] = 0u;
    if (p2)
        for (int i = i0; i < n2; i += step) p2[i] = 0u;
    if (p3)
        for (int i = i0; i < n3; i += step) p3[i] = 0u;
}

template <int CELL, int KCW, int R4, bool RL = false>
hipError_t launch_mc_t(const McPlan &p, McArgs m, hipStream_t s) {
    void *args[] = {&m};
    return launch_all_resident(reinterpret_cast<const void *>(&rec_fwd_mc_kernel<CELL, KCW, R4, RL>),
                               p.grid, p.threads, args, p.lds, s);
}


template <int CELL, int KCW>
hipError_t launch_mc_rows(const McPlan &p, const McArgs &m, hipStream_t s) {
    if (mc_row_lanes(p.BT)) {
        if (p.BT <= 4) return launch_mc_t<CELL, KCW, 1, true>(p, m, s);
        if (p.BT <= 8) return launch_mc_t<CELL, KCW, 2, true>(p, m, s);
        return launch_mc_t<CELL, KCW, 4, true>(p, m, s);
    }
    switch (p.r4) {
        case 1: return launch_mc_t<CELL, KCW, 1>(p, m, s);
        case 2: return launch_mc_t<CELL, KCW, 2>(p, m, s);
        default: return launch_mc_t<CELL, KCW, 4>(p, m, s);
    }
}

}  // namespace

McPlan plan_mc(int cell, int B, int NH, int Dh, int num_cu, int bt_override, int k_override,
               int kcw) {
    McPlan p{};
    const int G = cell == kLSTM ? 4 : 3;
    if (Dh < 256 || Dh % 128 != 0) return p;
    const int KC = Dh / 32;
    p.kcw = (kcw == 4 && KC % 4 == 0) || (kcw == 8 && KC % 8 == 0) ? kcw : KC % 8 == 0 ? 8 : 4;
    p.ks = KC / p.kcw;
    const int nb_max = 8 / p.ks;  // at most 8 waves (512 threads) per workgroup
    if (nb_max < 1) return p;
    int K = 0;
    for (int k = 2; k <= Dh / 16; ++k) {
        if (Dh % (16 * k) == 0 && Dh / (16 * k) <= nb_max) {
            K = k;
            break;
        }
    }
    if (k_override > 0 && Dh % (16 * k_override) == 0 && Dh / (16 * k_override) <= nb_max)
        K = k_override;
    if (K == 0) return p;
    p.K = K;
    p.nb = Dh / (16 * K);
    p.threads = p.nb * p.ks * 64;
    int bt = 16;
    while (bt > 1 && (long)NH * ((B + bt / 2 - 1) / (bt / 2)) * K <= num_cu) bt /= 2;
    if (bt_override > 0) bt = bt_override < 16 ? bt_override : 16;
    if (bt > B) bt = B;
    const int nbt = (B + bt - 1) / bt;
    if ((long)NH * nbt * K > num_cu) return p;  // every member must be resident at once
    p.BT = bt;
    p.r4 = bt >= 3 ? 4 : bt;
    p.groups = NH * nbt;
    p.grid = p.groups * K;
    p.lds = sizeof(uint16_t) * 2 * 16 * (Dh + 8) +
            sizeof(float) * (size_t)(p.ks - 1) * p.nb * G * 256;
    p.ok = 1;
    return p;
}

hipError_t launch_rec_mc(int cell, const McPlan &p, const McArgs &m, hipStream_t s,
                         bool clear_flag) {
    hipError_t e;
    if (m.xcd_map && (!m.xcc || p.groups % 8 != 0)) return hipErrorInvalidValue;
    // one launch: the status word (clear_flag), the exchange slots (step
    // numbers start at 1: cleared slots never match a step) and the XCD table
    // (ids are published as id + 1)
    const long words = 2L * p.groups * 2 * p.BT * (m.r.Dh / 2);
    hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, s,
                       reinterpret_cast<unsigned *>(m.xg), (int)words,
                       m.xcd_map ? m.xcc : (unsigned *)nullptr, m.xcd_map ? p.grid : 0,
                       clear_flag ? m.flag : (unsigned *)nullptr, 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (cell == kLSTM)
        return p.kcw == 8 ? launch_mc_rows<kLSTM, 8>(p, m, s) : launch_mc_rows<kLSTM, 4>(p, m, s);
    return p.kcw == 8 ? launch_mc_rows<kGRU, 8>(p, m, s) : launch_mc_rows<kGRU, 4>(p, m, s);
}

}  // namespace rnn355
