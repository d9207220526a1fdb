// rec_wide.hip -- forward recurrence for heads of Dh = 256 on one compute
// unit, with the head's R block split over the accumulation registers, the
// vector registers and LDS.
//
// Method (FlashRNN, arXiv 2412.07752, abstract; blog.hotdry.top 2025-09-21,
// the paragraphs on the step dependency and on keeping R on chip): a head's
// R block stays on chip for all T steps and each step is
//     A_t = Gx_t + h_{t-1} R_n,   then the cell's gate update.
// At Dh = 256 the block is 256 x G*256 bf16 (512 KiB for the LSTM, 384 KiB
// for the GRU): as large as the whole register file of a compute unit
// (4 SIMDs x 128 KiB).  Splitting the head over several compute units costs
// a cross-unit exchange of h_t at every step (about a microsecond through
// the device-coherent memory side); here it stays on one unit instead.
//
// One workgroup per (head, batch row), 4 waves, one per SIMD (so each wave
// may hold 512 registers).  The reduction dimension is split over the waves:
// wave w multiplies h_{t-1}[64w, 64w+64) (two k-chunks of 32) with the
// matching 64 rows of R for ALL G*256 gate columns, i.e. NT = G*16 output
// tiles of v_mfma_f32_16x16x32_bf16, 2*NT MFMAs per step.  Its 2*NT B
// fragments sit 64 in the AGPRs, 32 in VGPRs and (LSTM) 32 in LDS, read
// again at every step; in the LSTM every group of 8 MFMAs takes 4 B operands
// from AGPRs, 2 from VGPRs and 2 from LDS, so the LDS reads (each issued two
// groups before its use) are spread evenly over the step.  Per step:
//   1. tile groups of 4: MFMAs, and interleaved with the next group's MFMAs
//      row 0 of the 4 tiles (the only live batch row) packed into one
//      register with cross-row swaps and written to LDS as this wave's
//      partial gate sums;
//   2. barrier; thread u sums the 4 waves' partials of unit u's G gates and
//      runs the whole cell update of unit u lane-locally;
//   3. barrier (the partial sums may be rewritten); the A operand of the
//      next step: wave w's k range is exactly the units its own threads
//      updated, so h_t goes through a per-wave LDS slot with no barrier.
// The MFMAs are inline assembly so that their B operand can be an AGPR:
// compiled from the builtin, every AGPR fragment was first copied to vector
// registers (four moves per MFMA, which a single wave per SIMD cannot hide).
// The compiler does not see these as MFMAs, so it inserts no wait states
// for them: every read of an accumulator goes through `chain_end` (16 wait
// states, twice what the compiler keeps for this instruction), and each
// MFMA starts with the two wait states a VALU write of one of its sources
// would need.  They are volatile, so they keep the order written here.
//
// HBM traffic per step: Gx_t (G*256 floats) read, h_t and c_t written, by
// thread u for unit u (coalesced).  At the start of step t the Gx of step
// t+1 is requested into registers and then the outputs of step t-1 (kept in
// registers) are stored; the only wait on memory, at the start of the next
// step, leaves those stores in flight.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "gates.h"
#include "kernels.h"
#include "xcd.h"

namespace rnn355 {

namespace {

constexpr int kWideDh = 256;

// f(integral_constant<int, i>) for i in [B, E): loop indices usable as
// template arguments (immediate LDS offsets)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
// global-memory float (address space 1): a pointer that went through an
// empty asm is otherwise treated as generic (flat)
typedef __attribute__((address_space(1))) float gfloat;
constexpr int kWideWaves = 4;

template <int CELL>
struct WideCfg {
    static constexpr int G = CellTraits<CELL>::G;
    static constexpr int NT = G * kWideDh / 16;   // output tiles (16 gate columns each)
    static constexpr int NF = 2 * NT;             // B fragments per wave (2 k-chunks per tile)
    static constexpr int FA = 64;                 // fragments in AGPRs (256 registers)
    static constexpr int FV = 32;                 // fragments in VGPRs (128 registers)
    static constexpr int FL = NF - FA - FV;       // fragments in LDS (LSTM 32, GRU 0)
    static constexpr int TG = 4;                  // tiles per group
    static constexpr int NG = NT / TG;            // groups per step
    static constexpr size_t kLdsR = (size_t)FL * kWideWaves * 64 * 16;
    static_assert(FL >= 0 && NT % TG == 0, "fragment split");
};

// acc = A . B (+ acc): v_mfma_f32_16x16x32_bf16 with B in an AGPR ("a") or a
// VGPR ("v"); the *_first forms take 0 as the addend.
__device__ __forceinline__ void mfma_b_agpr_first(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_b_agpr(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_b_vgpr_first(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_b_vgpr(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// LDS fragment reads issued where they are written (the compiler would
// move its own loads next to their uses and wait there), completed by
// lds_wait, through which the values pass so nothing reads them earlier.
// The compiler does not count these loads; its own waits on LDS only get
// stricter (LDS operations complete in order).
// (base register + immediate byte offset, so the fragments of a wave share
// one address register)
template <int OFF>
__device__ __forceinline__ bf16x8 lds_frag(unsigned base) {
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF));
    return v;
}
// Completes a fragment read with at most three LDS operations issued after
// it still in flight (LDS operations complete in order; loads the compiler
// adds in between only make the wait stricter).
__device__ __forceinline__ void lds_wait3(bf16x8 &v) {
    asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(v) :: "memory");
}

// 16 wait states between the last MFMA writing the accumulators and any
// instruction that reads them; the accumulators pass through the asm, so
// every reader depends on it.
__device__ __forceinline__ void chain_end(f32x4 (&acc)[4]) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
}

// The same packing as inline assembly, for interleaving with the MFMAs
// (swap16(x, y): x <- [x0, y0, x2, y2], y <- [x1, y1, x3, y3] by 16-lane
// rows; swap32(x, y): x <- [x0, x1, y0, y1]), and an LDS store the compiler
// does not reorder against them.  The barrier that follows waits for it.
__device__ __forceinline__ void swap16_asm(float &x, float &y) {
    asm volatile("v_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap32_asm(float &x, float &y) {
    asm volatile("v_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
template <int OFF>
__device__ __forceinline__ void lds_store_asm(unsigned base, float v) {
    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(base), "v"(v), "n"(OFF) : "memory");
}
template <int N>
__device__ __forceinline__ void tie(f32x4 &x, f32x4 &y) {
    asm volatile("" : "+v"(x), "+v"(y));
}

// Row 0 of four tiles in one register: tile i in lanes 16i .. 16i+15.
__device__ __forceinline__ float pack_row0(const f32x4 (&acc)[4]) {
    const RowPair p = swap16(acc[0][0], acc[1][0]);  // [t0, t1, ., .]
    const RowPair q = swap16(acc[2][0], acc[3][0]);  // [t2, t3, ., .]
    return swap32(p.a, q.a).a;                       // [t0, t1, t2, t3]
}

template <int CELL>
__global__ __launch_bounds__(kWideWaves * 64, 1) void rec_fwd_wide_kernel(RecArgs a,
                                                                          const uint16_t *Rt) {
    using C = WideCfg<CELL>;
    constexpr int DH = kWideDh, G = C::G, GD = G * DH, NT = C::NT;
    constexpr int FA = C::FA, FV = C::FV, FL = C::FL, TG = C::TG, NG = C::NG;
    constexpr int PD = 1;  // steps per Gx group
    constexpr bool LSTM = CELL == kLSTM;

    extern __shared__ __attribute__((aligned(16))) uint4 rl[];        // [waves][FL][64 lanes]
    __shared__ __attribute__((aligned(16))) float part[kWideWaves][NT * 16];  // partial sums
    __shared__ __attribute__((aligned(16))) uint16_t hst[kWideWaves][64];     // A operand slot

    const int n = blockIdx.x % a.NH, b = blockIdx.x / a.NH;
    const int H = a.NH * DH, N = a.NH * GD, T = a.T, B = a.B;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- R^T fragments.  Fragment f = 2*tile + kc: gate columns
    // [16 tile, +16), k-chunk 2w + kc; lane (lr, lg) holds
    // R[64w + 32kc + 8lg .. +8][16 tile + lr], 16 contiguous bytes of R^T.
    const uint4 *Rn = reinterpret_cast<const uint4 *>(Rt + (long)n * GD * DH);
    auto frag_src = [&](int f) {
        const int col = 16 * (f >> 1) + lr, k = 64 * w + 32 * (f & 1) + 8 * lg;
        return Rn[(col * DH + k) / 8];
    };
    bf16x8 ra[FA], rv[FV];

    // ---- thread tid owns unit u = tid: state, Gx, outputs
    const int u = tid;
    const long o_row = (long)b * H + n * DH;
    const float *gx_row = a.gx + (long)b * N + n * GD;
    const long gx_step = (long)B * N, o_step = (long)B * H;
    const float h0 = a.h0 ? a.h0[o_row + u] : 0.f;
    float st = LSTM ? (a.c0 ? a.c0[o_row + u] : 0.f) : h0;  // c (LSTM) or h (GRU)
    float hl = h0;
    // (scalar flags: kept in SGPRs rather than as per-lane values)
    const bool has_h = __builtin_amdgcn_readfirstlane(a.h_seq != nullptr ? 1 : 0) != 0;
    const bool has_c = LSTM && __builtin_amdgcn_readfirstlane(a.c_seq != nullptr ? 1 : 0) != 0;

    // store instructions per group (issued after the group's loads)
    const int nst = PD * ((has_h ? 1 : 0) + (has_c ? 1 : 0));
    static_assert(PD == 1, "the waits below count one step of stores");
    float bx0[PD][G], bx1[PD][G], oh[PD], oc[PD];
#pragma unroll
    for (int s = 0; s < PD; ++s) {
        oh[s] = oc[s] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) bx0[s][g] = bx1[s][g] = 0.f;
    }
    auto load_group = [&](int tg, float (&dst)[PD][G]) {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (tg + s < T) {
                // wave-uniform row base kept in SGPRs (through an empty asm,
                // so no per-lane 64-bit pointer is hoisted out of the loop)
                const float *src = gx_row + (long)(tg + s) * gx_step;
                asm volatile("" : "+s"(src));
                const gfloat *gsrc = (const gfloat *)src;
#pragma unroll
                for (int g = 0; g < G; ++g) dst[s][g] = gsrc[(unsigned)(g * DH + u)];
            }
        }
    };
    auto store_group = [&](int tg) {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (tg + s >= T) break;
            const long o = (long)(tg + s) * o_step + o_row;
            float *hp = a.h_seq + o, *cp = has_c ? a.c_seq + o : hp;
            asm volatile("" : "+s"(hp), "+s"(cp));
            if (has_h) ((gfloat *)hp)[(unsigned)u] = oh[s];
            if (has_c) ((gfloat *)cp)[(unsigned)u] = oc[s];
        }
    };
    // A operand: this wave's two k-chunks of h (rows all equal: every lane
    // of a row group reads the same 16 bytes), through the wave's own slot
    bf16x8 af[2];
    auto stage_a = [&](float hv) {
        hst[w][lane] = f32_to_bf16_rne(hv);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) af[kc] = *reinterpret_cast<const bf16x8 *>(&hst[w][32 * kc + 8 * lg]);
    };
    stage_a(h0);
    __syncthreads();

    // Where the B fragment of MFMA j of group g lives (j = kc*TG + i: tile
    // TG*g + i, k-chunk kc).  LSTM: j%4 in {0,1} AGPR, 2 VGPR, 3 LDS; GRU:
    // the first 8 groups AGPR, the rest VGPR.
    enum { kA = 0, kV = 1, kL = 2 };
    constexpr auto cls = [](int g, int j) { return LSTM ? ((j & 3) < 2 ? kA : (j & 3) == 2 ? kV : kL) : (g < 8 ? kA : kV); };
    constexpr auto idx = [](int g, int j) {
        return LSTM ? ((j & 3) < 2 ? 4 * g + 2 * (j >> 2) + (j & 3) : 2 * g + (j >> 2))
                    : (g < 8 ? 8 * g + j : 8 * (g - 8) + j);
    };
    static_assert(FL == 0 || FL == 2 * NG, "two LDS fragments per group");
    // R^T fragments, placed by class
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < 2 * TG; ++j) {
            const int tile = TG * g + (j % TG), kc = j / TG;
            const uint4 v = frag_src(2 * tile + kc);
            if (cls(g, j) == kA) ra[idx(g, j)] = __builtin_bit_cast(bf16x8, v);
            else if (cls(g, j) == kV) rv[idx(g, j)] = __builtin_bit_cast(bf16x8, v);
            else rl[(w * FL + idx(g, j)) * 64 + lane] = v;
        }
    // LDS fragments in flight: slot (g & 1)*2 + j/4, read two groups ahead
    bf16x8 lb[4];
    const unsigned rl_base = (unsigned)(uintptr_t)&rl[(w * FL) * 64 + lane];
    auto fetch = [&](auto gc, auto jc) {
        constexpr int g = decltype(gc)::value, j = decltype(jc)::value;
        lb[(g & 1) * 2 + (j >> 2)] = lds_frag<idx(g, j) * 1024>(rl_base);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I3 = std::integral_constant<int, 3>;
    using I7 = std::integral_constant<int, 7>;
    if constexpr (FL > 0) {
        fetch(I0{}, I3{}); fetch(I0{}, I7{}); fetch(I1{}, I3{}); fetch(I1{}, I7{});
    }
    // fill(j) runs after the j-th MFMA of the group (work interleaved with
    // the matrix pipe's latency)
    auto chain = [&](auto gc, f32x4 (&acc)[TG], auto &&fill) {
        constexpr int g = decltype(gc)::value;
        static_for<0, 2 * TG>([&](auto jc) {
            constexpr int j = decltype(jc)::value, i = j % TG, kc = j / TG;
            constexpr int c = cls(g, j);
            if constexpr (c == kA) {
                if constexpr (kc == 0) mfma_b_agpr_first(acc[i], af[kc], ra[idx(g, j)]);
                else mfma_b_agpr(acc[i], af[kc], ra[idx(g, j)]);
            } else {
                bf16x8 &bf = c == kV ? rv[c == kV ? idx(g, j) : 0] : lb[(g & 1) * 2 + (j >> 2)];
                if constexpr (c == kL) lds_wait3(bf);
                if constexpr (kc == 0) mfma_b_vgpr_first(acc[i], af[kc], bf);
                else mfma_b_vgpr(acc[i], af[kc], bf);
                // the same slot, two groups on
                if constexpr (c == kL) fetch(std::integral_constant<int, (g + 2) % NG>{}, jc);
            }
            fill(jc);
        });
    };
    // row 0 of the last group of a step -> this wave's partial sums
    auto publish_last = [&](int g, f32x4 (&acc)[TG]) {
        chain_end(acc);
        part[w][(TG * g) * 16 + lane] = pack_row0(acc);
    };
    // The previous group's publication, interleaved with the next group's
    // MFMAs: a tile's last MFMA is at index 4..7 of its group, and its row 0
    // is read after at least six more MFMAs (each with two wait states of its
    // own, so at least eighteen: more than the sixteen the result hazard
    // needs).  The ties keep the reads behind those MFMAs.
    const unsigned part_base = (unsigned)(uintptr_t)&part[w][lane];
    auto publish_piece = [&](auto jc, auto gpc, f32x4 (&acc)[TG], float (&x)[4]) {
        constexpr int j = decltype(jc)::value, gp = decltype(gpc)::value;
        if constexpr (j == 3) {
            tie<0>(acc[0], acc[1]);
            x[0] = acc[0][0];
            x[1] = acc[1][0];
            swap16_asm(x[0], x[1]);
        } else if constexpr (j == 5) {
            tie<1>(acc[2], acc[3]);
            x[2] = acc[2][0];
            x[3] = acc[3][0];
            swap16_asm(x[2], x[3]);
        } else if constexpr (j == 6) {
            swap32_asm(x[0], x[2]);
        } else if constexpr (j == 7) {
            lds_store_asm<(TG * gp) * 16 * 4>(part_base, x[0]);
        }
    };

    auto run_group = [&](auto full, int tg, float (&use)[PD][G], float (&nxt)[PD][G]) {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (!decltype(full)::value && tg + s >= T) break;
            if (s == 0) {
                // this group's Gx, requested a group ago; the stores issued
                // after it (nst of them) may still be in flight
                if (tg <= PD || nst == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                else if (nst == 1) __builtin_amdgcn_s_waitcnt(0x0F71);       // vmcnt(1)
                else __builtin_amdgcn_s_waitcnt(0x0F72);                     // vmcnt(2)
                load_group(tg + PD, nxt);
                if (tg > 0) store_group(tg - PD);
            }
            // 1. partial gate sums of this wave's k range, all tiles; the
            // next group's MFMAs go out before this group's results are read
            f32x4 acc0[TG], acc1[TG];
            float px[4];
            static_for<0, NG>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                f32x4 (&cur)[TG] = (g & 1) ? acc1 : acc0;
                f32x4 (&old)[TG] = (g & 1) ? acc0 : acc1;
                chain(gc, cur, [&](auto jc) {
                    if constexpr (g > 0) publish_piece(jc, std::integral_constant<int, g - 1>{}, old, px);
                });
            });
            publish_last(NG - 1, (NG & 1) ? acc0 : acc1);
            lds_barrier();
            // 2. unit u: sum over the waves, cell update
            float pre[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float v = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWideWaves; ++ww) v += part[ww][g * DH + u];
                pre[g] = (CELL == kGRU && g == 2) ? v : v + use[s][g];
            }
            float c;
            const float h = unit_update<CELL>(pre, CELL == kGRU ? use[s][2] : 0.f, st, c);
            hl = h;
            oh[s] = h;
            oc[s] = c;
            lds_barrier();
            // 3. next A operand
            stage_a(h);
        }
    };

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
    a.hT[o_row + u] = LSTM ? hl : st;
    if (LSTM) a.cT[o_row + u] = st;
}

// ---------------------------------------------------------------------------
// Reverse-time sweep of backpropagation through time for Dh = 256 on one
// compute unit per (head, batch row), the same split of R.  Per step t
// (T-1 .. 0), thread u owns unit u:
//   1. the cell backward of unit u (from the recomputed gate inputs, the
//      streamed c_t, c_{t-1} / h_{t-1} and dL/dh_t, and the carries), which
//      writes dGx_t (and the GRU's dS_t) as bf16 and accumulates db;
//   2. the carry dh = e_t R^T with e = dGx (LSTM) or dS (GRU): wave w holds
//      the gate columns of units [64w, 64w+64) of every gate -- exactly the
//      e values its own threads produced, so the A operand needs no barrier
//      -- and multiplies them with the matching columns of R for all 256
//      output units (16 tiles), publishing row 0 of its partial sums;
//   3. barrier, each thread sums the four partials of its unit (plus the
//      GRU's direct term dh u), barrier.
// B fragment (tile of units [16i, 16i+16), chunk (g, half) of the wave's
// columns): lane (lr, lg) holds R[16i + lr][g*256 + 64w + 32 half + 8lg ..
// +8], 16 contiguous bytes of R's own rows.
template <int CELL>
struct WideBwdCfg {
    static constexpr int G = CellTraits<CELL>::G;
    static constexpr int NCH = 2 * G;            // k-chunks per wave
    static constexpr int NT = kWideDh / 16;      // output tiles
    static constexpr int TG = 4;                 // tiles per group
    static constexpr int NG = NT / TG;           // groups per step
    static constexpr int MPG = TG * NCH;         // MFMAs per group
    static constexpr int NF = NT * NCH;          // B fragments per wave
    static constexpr int FA = 64, FV = 32, FL = NF - FA - FV;
    static constexpr size_t kLdsR = (size_t)FL * kWideWaves * 64 * 16;
    static_assert(FL == 0 || FL == NG * NCH, "one LDS fragment per chunk and group");
};

template <int CELL>
__global__ __launch_bounds__(kWideWaves * 64, 1) void rec_bwd_wide_kernel(BwdArgs m) {
    using C = WideBwdCfg<CELL>;
    constexpr int DH = kWideDh, G = C::G, GD = G * DH, NCH = C::NCH, TG = C::TG, NG = C::NG;
    constexpr int MPG = C::MPG, FA = C::FA, FV = C::FV, FL = C::FL;
    constexpr bool LSTM = CELL == kLSTM;
    constexpr int NIN = LSTM ? G + 3 : 2 * G + 2;  // streamed floats per step and unit
    constexpr int NST = LSTM ? G : 2 * G;          // bf16 stores per step

    extern __shared__ __attribute__((aligned(16))) uint4 rl[];        // [waves][FL][64 lanes]
    __shared__ __attribute__((aligned(16))) float part[kWideWaves][DH];       // partial carries
    __shared__ __attribute__((aligned(16))) uint16_t hs[kWideWaves][G][64];   // A operand slot

    const int n = blockIdx.x % m.NH, b = blockIdx.x / m.NH;
    const int H = m.NH * DH, N = m.NH * GD, T = m.T, B = m.B;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int u = tid;

    // ---- R fragments by class (LSTM: tiles i%4 in {0,1} AGPR, 2 VGPR, 3
    // LDS; GRU: the first 64 in MFMA order AGPR, the rest VGPR)
    enum { kA = 0, kV = 1, kL = 2 };
    constexpr auto cls = [](int gi, int j) {
        return LSTM ? ((j % TG) < 2 ? kA : (j % TG) == 2 ? kV : kL) : (gi * MPG + j < FA ? kA : kV);
    };
    constexpr auto idx = [](int gi, int j) {
        const int c = j / TG, i = j % TG;
        return LSTM ? (i < 2 ? (gi * NCH + c) * 2 + i : gi * NCH + c)
                    : (gi * MPG + j < FA ? gi * MPG + j : gi * MPG + j - FA);
    };
    const uint16_t *Rn = m.Rb + (long)n * DH * GD;
    bf16x8 ra[FA], rv[FV];
    static_for<0, NG>([&](auto gc) {
        constexpr int gi = decltype(gc)::value;
        static_for<0, MPG>([&](auto jc) {
            constexpr int j = decltype(jc)::value, c = j / TG, i = j % TG;
            const int row = 16 * (TG * gi + i) + lr;
            const int col = (c >> 1) * DH + 64 * w + 32 * (c & 1) + 8 * lg;
            const uint4 v = *reinterpret_cast<const uint4 *>(Rn + (long)row * GD + col);
            if constexpr (cls(gi, j) == kA) ra[idx(gi, j)] = __builtin_bit_cast(bf16x8, v);
            else if constexpr (cls(gi, j) == kV) rv[idx(gi, j)] = __builtin_bit_cast(bf16x8, v);
            else rl[(w * FL + idx(gi, j)) * 64 + lane] = v;
        });
    });
    // LDS fragments in flight: use q (= gi*NCH + c) in slot q % 4, read four
    // uses ahead (continuing into the next step)
    bf16x8 lb[4];
    const unsigned rl_base = (unsigned)(uintptr_t)&rl[(w * FL) * 64 + lane];
    auto fetch = [&](auto qc) {
        constexpr int q = decltype(qc)::value % (FL > 0 ? FL : 1);
        lb[q & 3] = lds_frag<q * 1024>(rl_base);
    };
    if constexpr (FL > 0)
        static_for<0, 4>([&](auto qc) { fetch(qc); });

    // ---- per-unit state and streamed inputs
    const long o_row = (long)b * H + n * DH, a_row = (long)b * N + n * GD;
    const long a_step = (long)B * N, o_step = (long)B * H;
    float dhc = m.dhT ? m.dhT[o_row + u] : 0.f;
    float dcc = (LSTM && m.dcT) ? m.dcT[o_row + u] : 0.f;
    float dir = 0.f, dbs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dbs[g] = 0.f;
    // in[]: LSTM pa[0..3], c_t, c_{t-1}, dL/dh_t; GRU pa[0..2], sv[0..2],
    // h_{t-1}, dL/dh_t
    float in0[NIN], in1[NIN];
#pragma unroll
    for (int i = 0; i < NIN; ++i) in0[i] = in1[i] = 0.f;
    auto gptr = [](const float *p) {
        asm volatile("" : "+s"(p));
        return (const gfloat *)p;
    };
    auto load_in = [&](int t, float (&d)[NIN]) {
        const gfloat *pa = gptr(m.A + a_row + (long)t * a_step);
#pragma unroll
        for (int g = 0; g < G; ++g) d[g] = pa[(unsigned)(g * DH + u)];
        const gfloat *up = gptr(m.dh_seq + o_row + (long)t * o_step);
        d[NIN - 1] = up[(unsigned)u];
        if constexpr (LSTM) {
            const gfloat *ct = gptr(m.c_seq + o_row + (long)t * o_step);
            d[G] = ct[(unsigned)u];
            if (t > 0) d[G + 1] = gptr(m.c_seq + o_row + (long)(t - 1) * o_step)[(unsigned)u];
            else d[G + 1] = m.c0 ? m.c0[o_row + u] : 0.f;
        } else {
            const gfloat *sv = gptr(m.S + a_row + (long)t * a_step);
#pragma unroll
            for (int g = 0; g < G; ++g) d[G + g] = sv[(unsigned)(g * DH + u)];
            if (t > 0) d[2 * G] = gptr(m.h_seq + o_row + (long)(t - 1) * o_step)[(unsigned)u];
            else d[2 * G] = m.h0 ? m.h0[o_row + u] : 0.f;
        }
    };
    auto store_d = [&](int t, const uint16_t (&dd)[G], const uint16_t (&de)[G]) {
        uint16_t *pa = m.dA + a_row + (long)t * a_step;
        asm volatile("" : "+s"(pa));
#pragma unroll
        for (int g = 0; g < G; ++g)
            ((__attribute__((address_space(1))) uint16_t *)pa)[(unsigned)(g * DH + u)] = dd[g];
        if constexpr (!LSTM) {
            uint16_t *ps = m.dS + a_row + (long)t * a_step;
            asm volatile("" : "+s"(ps));
#pragma unroll
            for (int g = 0; g < G; ++g)
                ((__attribute__((address_space(1))) uint16_t *)ps)[(unsigned)(g * DH + u)] = de[g];
        }
    };

    // ---- the MFMA part of a step (A operand: this wave's e values)
    bf16x8 af[NCH];
    auto chain = [&](auto gc, f32x4 (&acc)[TG], auto &&fill) {
        constexpr int gi = decltype(gc)::value;
        static_for<0, MPG>([&](auto jc) {
            constexpr int j = decltype(jc)::value, c = j / TG, i = j % TG;
            constexpr int k = cls(gi, j);
            if constexpr (k == kA) {
                if constexpr (c == 0) mfma_b_agpr_first(acc[i], af[c], ra[idx(gi, j)]);
                else mfma_b_agpr(acc[i], af[c], ra[idx(gi, j)]);
            } else {
                constexpr int q = gi * NCH + c;  // LDS use index (LSTM)
                bf16x8 &bf = k == kV ? rv[k == kV ? idx(gi, j) : 0] : lb[q & 3];
                if constexpr (k == kL) lds_wait3(bf);
                if constexpr (c == 0) mfma_b_vgpr_first(acc[i], af[c], bf);
                else mfma_b_vgpr(acc[i], af[c], bf);
                if constexpr (k == kL) fetch(std::integral_constant<int, q + 4>{});
            }
            fill(jc);
        });
    };
    const unsigned part_base = (unsigned)(uintptr_t)&part[w][lane];
    // the previous group's publication within the next group's MFMAs: a
    // tile's last MFMA is among the last four of its group, and its row 0 is
    // read after at least eight more (with their own wait states, well over
    // the sixteen the result hazard needs)
    auto publish_piece = [&](auto jc, auto gpc, f32x4 (&acc)[TG], float (&x)[4]) {
        constexpr int j = decltype(jc)::value, gp = decltype(gpc)::value;
        if constexpr (j == 5) {
            tie<0>(acc[0], acc[1]);
            x[0] = acc[0][0];
            x[1] = acc[1][0];
            swap16_asm(x[0], x[1]);
        } else if constexpr (j == 7) {
            tie<1>(acc[2], acc[3]);
            x[2] = acc[2][0];
            x[3] = acc[3][0];
            swap16_asm(x[2], x[3]);
        } else if constexpr (j == 8) {
            swap32_asm(x[0], x[2]);
        } else if constexpr (j == 9) {
            lds_store_asm<(TG * gp) * 16 * 4>(part_base, x[0]);
        }
    };
    static_assert(MPG >= 10, "publication pieces fit in a group");

    load_in(T - 1, in0);
    __syncthreads();

    auto step = [&](int s, float (&cur)[NIN], float (&nxt)[NIN]) {
        const int t = T - 1 - s;
        // this step's inputs (requested a step ago); the previous step's
        // stores may still be in flight
        if (s == 0) __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
        else if (NST == 4) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
        else __builtin_amdgcn_s_waitcnt(0x0F76);                // vmcnt(6)
        if (t > 0) load_in(t - 1, nxt);
        // 1. cell backward of unit u
        float d[G], e[G];
        const float dh = cur[NIN - 1] + dhc;
        if constexpr (LSTM) {
            const float ig = sigmoid_f(cur[0]), fg = sigmoid_f(cur[1]);
            const float zg = tanh_f(cur[2]), og = sigmoid_f(cur[3]);
            const float tc = tanh_f(cur[G]);
            const float dc = fmaf(dh * og, 1.0f - tc * tc, dcc);
            d[0] = dc * zg * ig * (1.0f - ig);
            d[1] = dc * cur[G + 1] * fg * (1.0f - fg);
            d[2] = dc * ig * (1.0f - zg * zg);
            d[3] = dh * tc * og * (1.0f - og);
            dcc = dc * fg;
#pragma unroll
            for (int g = 0; g < G; ++g) e[g] = d[g];
        } else {
            const float rg = sigmoid_f(cur[0] + cur[G]);
            const float ug = sigmoid_f(cur[1] + cur[G + 1]);
            const float ng = tanh_f(fmaf(rg, cur[G + 2], cur[2]));
            d[2] = dh * (1.0f - ug) * (1.0f - ng * ng);
            d[1] = dh * (cur[2 * G] - ng) * ug * (1.0f - ug);
            d[0] = d[2] * cur[G + 2] * rg * (1.0f - rg);
            e[0] = d[0];
            e[1] = d[1];
            e[2] = d[2] * rg;
            dir = dh * ug;
        }
        uint16_t dd[G], de[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            dbs[g] += d[g];
            dd[g] = f32_to_bf16_rne(d[g]);
            de[g] = LSTM ? dd[g] : f32_to_bf16_rne(e[g]);
            hs[w][g][lane] = de[g];
        }
        store_d(t, dd, de);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            af[c] = *reinterpret_cast<const bf16x8 *>(&hs[w][c >> 1][32 * (c & 1) + 8 * lg]);
        // 2. partial carries of this wave's columns
        f32x4 acc0[TG], acc1[TG];
        float px[4];
        static_for<0, NG>([&](auto gc) {
            constexpr int gi = decltype(gc)::value;
            f32x4 (&cu)[TG] = (gi & 1) ? acc1 : acc0;
            f32x4 (&old)[TG] = (gi & 1) ? acc0 : acc1;
            chain(gc, cu, [&](auto jc) {
                if constexpr (gi > 0) publish_piece(jc, std::integral_constant<int, gi - 1>{}, old, px);
            });
        });
        {
            f32x4 (&last)[TG] = ((NG - 1) & 1) ? acc1 : acc0;
            chain_end(last);
            part[w][(TG * (NG - 1)) * 16 + lane] = pack_row0(last);
        }
        lds_barrier();
        // 3. carry of unit u
        float v = LSTM ? 0.f : dir;
#pragma unroll
        for (int ww = 0; ww < kWideWaves; ++ww) v += part[ww][u];
        dhc = v;
        lds_barrier();
    };
    int s = 0;
    for (; s + 1 < T; s += 2) {
        step(s, in0, in1);
        step(s + 1, in1, in0);
    }
    if (s < T) step(s, in0, in1);
    if constexpr (FL > 0) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): prefetches done
    m.dh0[o_row + u] = dhc;
    if (LSTM) m.dc0[o_row + u] = dcc;
    float *dbt = m.db_part + (long)b * N + n * GD;
#pragma unroll
    for (int g = 0; g < G; ++g) dbt[g * DH + u] = dbs[g];
}

// ---------------------------------------------------------------------------
// The reverse sweep on two compute units per (head, batch row).  CU c owns
// units [128c, 128c + 128): it runs their cell backward and multiplies their
// G*128 gradient values (this step's dA, or dS for the GRU) with the matching
// R columns for all 256 output units; the two CUs' partial carries are then
// swapped (each sends the 128 partials of the other's units) and summed in a
// fixed order (CU 0's first), so each CU has the carry of its own units.
// Half of R per CU (256 KiB for the LSTM) fits the AGPRs: wave w multiplies
// its G k-chunks of 32 gradient columns with 16 output tiles, every B
// fragment in an AGPR (64 for the LSTM), no LDS fragments.  The two CUs of a
// row are numbered onto one XCD and swap the partials through its L2 when
// the launch finds them there (xcd.h), else through memory.  Per step the
// other CU's 8 output tiles come first: their partials are summed over the
// waves and sent while the waves multiply this CU's own 8 tiles, so the swap
// travels during those MFMAs.  The swap is done by the two waves that run no
// cell update: a poll waits for every earlier load and store of its thread,
// and the cell threads' next inputs and gradient stores are in flight.
template <int CELL>
__global__ __launch_bounds__(kWideWaves * 64, 1) void rec_bwd_wide2_kernel(BwdArgs m) {
    constexpr int DH = kWideDh, G = CellTraits<CELL>::G, GD = G * DH;
    constexpr int U = DH / 2;       // units per CU
    constexpr int NT = DH / 16;     // output tiles
    constexpr int NCHW = G;         // k-chunks of 32 per wave (4G per CU)
    constexpr int TG = 4, NG = NT / TG;
    constexpr bool LSTM = CELL == kLSTM;
    constexpr int NIN = LSTM ? G + 3 : 2 * G + 2;

    __shared__ __attribute__((aligned(16))) float part[kWideWaves][DH];  // partial carries
    __shared__ __attribute__((aligned(16))) uint16_t hs[G][U];           // this step's gradients
    __shared__ float dhs[U];                                             // own units' carries
    __shared__ int s_abort, s_local;

    int group, c;
    group_member(m.xcd_map != 0, 2, group, c);
    const int n = group % m.NH, b = group / m.NH;
    const int H = m.NH * DH, N = m.NH * GD, T = m.T, B = m.B;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const bool cell_thread = tid < U;
    const int u = 128 * c + (tid & (U - 1));  // the unit of a cell thread

    // ---- R fragments: wave w, k-chunk i is gradient chunk q = G w + i of
    // this CU (gate q / 4, units 128c + 32 (q % 4) ..); register slot jj holds
    // output tile tile_of(jj) (units 16 tile ..): slots 0-7 the other CU's
    // units, 8-15 this CU's
    const int tile_off = 8 * (1 - c);
    auto tile_of = [&](int jj) { return (jj + tile_off) & (NT - 1); };
    const uint16_t *Rn = m.Rb + (long)n * DH * GD;
    bf16x8 ra[NT * NCHW];
    static_for<0, NT>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        static_for<0, NCHW>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int q = G * w + i;
            const int col = (q >> 2) * DH + 128 * c + 32 * (q & 3) + 8 * lg;
            const uint4 v =
                *reinterpret_cast<const uint4 *>(Rn + (long)(16 * tile_of(jj) + lr) * GD + col);
            ra[jj * NCHW + i] = __builtin_bit_cast(bf16x8, v);
        });
    });

    if (tid == 0) {
        s_abort = 0;
        s_local = 0;
    }
    if (m.xcd_map) xcd_publish(m.xcc);

    const long o_row = (long)b * H + n * DH, a_row = (long)b * N + n * GD;
    const long a_step = (long)B * N, o_step = (long)B * H;
    float dhc = (cell_thread && m.dhT) ? m.dhT[o_row + u] : 0.f;
    float dcc = (LSTM && cell_thread && m.dcT) ? m.dcT[o_row + u] : 0.f;
    float dir = 0.f, dbs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dbs[g] = 0.f;
    float in0[NIN], in1[NIN];
#pragma unroll
    for (int i = 0; i < NIN; ++i) in0[i] = in1[i] = 0.f;
    auto load_in = [&](int t, float (&d)[NIN]) {
        const float *pa = m.A + a_row + (long)t * a_step;
#pragma unroll
        for (int g = 0; g < G; ++g) d[g] = pa[g * DH + u];
        d[NIN - 1] = m.dh_seq[o_row + (long)t * o_step + u];
        if constexpr (LSTM) {
            d[G] = m.c_seq[o_row + (long)t * o_step + u];
            d[G + 1] = t > 0 ? m.c_seq[o_row + (long)(t - 1) * o_step + u]
                             : (m.c0 ? m.c0[o_row + u] : 0.f);
        } else {
            const float *sv = m.S + a_row + (long)t * a_step;
#pragma unroll
            for (int g = 0; g < G; ++g) d[G + g] = sv[g * DH + u];
            d[2 * G] = t > 0 ? m.h_seq[o_row + (long)(t - 1) * o_step + u]
                             : (m.h0 ? m.h0[o_row + u] : 0.f);
        }
    };
    if (cell_thread) load_in(T - 1, in0);
    __syncthreads();
    if (m.xcd_map && w == 0) {
        const int v = xcd_members_agree(m.xcc, m.flag, m.spin_limit, group, 2);
        if (lane == 0) {
            s_local = v > 0;
            if (v < 0) s_abort = 1;
        }
    }
    __syncthreads();
    const bool local = s_local != 0;
    // exchange words [2 parities][2 senders][U]: sender c's partials of the
    // other CU's units, tagged with the step
    unsigned long long *xs = m.xg + (long)group * 2 * 2 * U;

    auto step = [&](int s, float (&cur)[NIN], float (&nxt)[NIN]) -> bool {
        const int t = T - 1 - s;
        // 1. cell backward of this CU's units
        if (cell_thread) {
            if (s > 0) dhc = LSTM ? dhs[tid] : dir + dhs[tid];  // the previous step's carry
            float d[G], e[G];
            const float dh = cur[NIN - 1] + dhc;
            if constexpr (LSTM) {
                const float ig = sigmoid_f(cur[0]), fg = sigmoid_f(cur[1]);
                const float zg = tanh_f(cur[2]), og = sigmoid_f(cur[3]);
                const float tc = tanh_f(cur[G]);
                const float dc = fmaf(dh * og, 1.0f - tc * tc, dcc);
                d[0] = dc * zg * ig * (1.0f - ig);
                d[1] = dc * cur[G + 1] * fg * (1.0f - fg);
                d[2] = dc * ig * (1.0f - zg * zg);
                d[3] = dh * tc * og * (1.0f - og);
                dcc = dc * fg;
#pragma unroll
                for (int g = 0; g < G; ++g) e[g] = d[g];
            } else {
                const float rg = sigmoid_f(cur[0] + cur[G]);
                const float ug = sigmoid_f(cur[1] + cur[G + 1]);
                const float ng = tanh_f(fmaf(rg, cur[G + 2], cur[2]));
                d[2] = dh * (1.0f - ug) * (1.0f - ng * ng);
                d[1] = dh * (cur[2 * G] - ng) * ug * (1.0f - ug);
                d[0] = d[2] * cur[G + 2] * rg * (1.0f - rg);
                e[0] = d[0];
                e[1] = d[1];
                e[2] = d[2] * rg;
                dir = dh * ug;
            }
            uint16_t *pa = m.dA + a_row + (long)t * a_step;
            uint16_t *ps = LSTM ? nullptr : m.dS + a_row + (long)t * a_step;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                dbs[g] += d[g];
                const uint16_t dd = f32_to_bf16_rne(d[g]);
                const uint16_t de = LSTM ? dd : f32_to_bf16_rne(e[g]);
                pa[g * DH + u] = dd;
                if constexpr (!LSTM) ps[g * DH + u] = de;
                hs[g][tid] = de;
            }
            // the next step's inputs, once this step's are used (requested
            // earlier, a wait for this step's would also wait for them)
            if (t > 0) load_in(t - 1, nxt);
        }
        __syncthreads();
        if (s_abort) return false;
        // 2. partial carries of this CU's gradient columns, all 256 units
        bf16x8 af[NCHW];
#pragma unroll
        for (int i = 0; i < NCHW; ++i) {
            const int q = G * w + i;
            af[i] = *reinterpret_cast<const bf16x8 *>(&hs[q >> 2][32 * (q & 3) + 8 * lg]);
        }
        auto tiles = [&](auto gc) {
            constexpr int gi = decltype(gc)::value;
            f32x4 acc[TG];
            static_for<0, NCHW>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                static_for<0, TG>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    if constexpr (i == 0) mfma_b_agpr_first(acc[k], af[i], ra[(TG * gi + k) * NCHW + i]);
                    else mfma_b_agpr(acc[k], af[i], ra[(TG * gi + k) * NCHW + i]);
                });
            });
            chain_end(acc);
            if (lg == 0) {
#pragma unroll
                for (int k = 0; k < TG; ++k) part[w][16 * tile_of(TG * gi + k) + lr] = acc[k][0];
            }
        };
        // the other CU's tiles, summed over the waves and sent (by the
        // threads that run no cell update) while the own tiles are multiplied
        static_for<0, NG / 2>(tiles);
        __syncthreads();
        const int j = (tid + 128 * c) & (DH - 1);  // own units on the cell threads
        unsigned long long *slot = xs + (long)(s & 1) * 2 * U;
        const unsigned long long tag = (unsigned long long)(unsigned)(s + 1) << 32;
        if (!cell_thread) {
            float p = part[0][j];
#pragma unroll
            for (int ww = 1; ww < kWideWaves; ++ww) p += part[ww][j];
            unsigned long long *dst = slot + c * U + (j & (U - 1));
            const unsigned long long wv = tag | __float_as_uint(p);
            if (local)
                __hip_atomic_store(dst, wv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            else
                __hip_atomic_store(dst, wv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // the first poll of the other CU's partials goes out between the own
        // tile groups, so that by the barrier it has usually returned with them
        const unsigned long long *src = slot + (1 - c) * U + (tid & (U - 1));
        unsigned long long wv = 0;
        static_for<NG / 2, NG / 2 + 1>(tiles);
        // (as volatile asm, kept in place among the MFMAs' asm: a device-scope
        // load the compiler does not track, completed by the wait below)
        if (!cell_thread)
            asm volatile("global_load_dwordx2 %0, %1, off sc1" : "=v"(wv) : "v"(src) : "memory");
        static_for<NG / 2 + 1, NG>(tiles);
        __syncthreads();
        if (!cell_thread) asm volatile("s_waitcnt vmcnt(0)" : "+v"(wv)::"memory");
        // 3. own units (unit 128c + k on non-cell thread 128 + k): this CU's
        // partial, completed with the other CU's, handed to the cell thread
        if (!cell_thread) {
            const int k = tid - U;
            const int jo = 128 * c + k;
            float p = part[0][jo];
#pragma unroll
            for (int ww = 1; ww < kWideWaves; ++ww) p += part[ww][jo];
            unsigned spins = 0;
            for (;;) {
                if ((wv & 0xFFFFFFFF00000000ull) == tag) break;
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
                wv = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const float q = __uint_as_float((unsigned)wv);
            dhs[k] = c == 0 ? p + q : q + p;  // CU 0's partial first in both
        }
        __syncthreads();
        return true;
    };
    int s = s_abort ? T + 1 : 0;
    bool ok = s <= T;
    for (; ok && s + 1 < T; s += 2) {
        ok = step(s, in0, in1);
        if (ok) ok = step(s + 1, in1, in0);
    }
    if (ok && s < T) ok = step(s, in0, in1), ++s;
    if (!ok || s < T || !cell_thread) return;
    if (T > 0) dhc = LSTM ? dhs[tid] : dir + dhs[tid];  // the last step's carry
    m.dh0[o_row + u] = dhc;
    if (LSTM) m.dc0[o_row + u] = dcc;
    float *dbt = m.db_part + (long)b * N + n * GD;
#pragma unroll
    for (int g = 0; g < G; ++g) dbt[g * DH + u] = dbs[g];
}

__global__ void clear_words_wide_kernel(unsigned *p, long n, unsigned *p2, long n2, unsigned *p3,
                                        long n3) {
    const long i0 = blockIdx.x * (long)blockDim.x + threadIdx.x, step = (long)gridDim.x * blockDim.x;
    if (p)
        for (long i = i0; i < n; i += step) p[i] = 0u;
    if (p2)
        for (long i = i0; i < n2; i += step) p2[i] = 0u;
    if (p3)
        for (long i = i0; i < n3; i += step) p3[i] = 0u;
}

template <int CELL>
hipError_t launch_bwd_wide2_t(const BwdArgs &m0, hipStream_t s) {
    BwdArgs m = m0;
    const int grid = 2 * m.NH * m.B;
    const long words = (long)m.NH * m.B * 2 * 2 * (kWideDh / 2) * 2;  // as 32-bit words
    hipLaunchKernelGGL(clear_words_wide_kernel, dim3(64), dim3(256), 0, s,
                       m.keep_flag ? (unsigned *)nullptr : m.flag, 1L,
                       m.xcd_map ? m.xcc : (unsigned *)nullptr, m.xcd_map ? (long)grid : 0L,
                       reinterpret_cast<unsigned *>(m.xg), words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    void *args[] = {&m};
    return launch_all_resident(reinterpret_cast<const void *>(&rec_bwd_wide2_kernel<CELL>), grid,
                               kWideWaves * 64, args, 0, s);
}

template <int CELL>
hipError_t launch_bwd_wide_t(const WidePlan &p, const BwdArgs &m, hipStream_t s) {
    if (WideBwdCfg<CELL>::kLdsR > 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&rec_bwd_wide_kernel<CELL>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)WideBwdCfg<CELL>::kLdsR);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(rec_bwd_wide_kernel<CELL>, dim3(p.grid), dim3(p.threads),
                       WideBwdCfg<CELL>::kLdsR, s, m);
    return hipGetLastError();
}

template <int CELL>
hipError_t launch_wide_t(const WidePlan &p, const RecArgs &a, const uint16_t *Rt, hipStream_t s) {
    if (WideCfg<CELL>::kLdsR > 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&rec_fwd_wide_kernel<CELL>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)WideCfg<CELL>::kLdsR);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(rec_fwd_wide_kernel<CELL>, dim3(p.grid), dim3(p.threads),
                       WideCfg<CELL>::kLdsR, s, a, Rt);
    return hipGetLastError();
}

}  // namespace

WidePlan plan_wide(int cell, int B, int NH, int Dh, bool bf16) {
    WidePlan p{};
    if (!bf16 || Dh != kWideDh || (cell != kLSTM && cell != kGRU)) return p;
    p.ok = 1;
    p.grid = NH * B;
    p.threads = kWideWaves * 64;
    p.lds = cell == kLSTM ? WideCfg<kLSTM>::kLdsR : WideCfg<kGRU>::kLdsR;
    return p;
}

hipError_t launch_rec_bwd_wide2(int cell, const BwdArgs &m, hipStream_t s) {
    if (m.Dh != kWideDh || m.T < 1 || (m.xcd_map && (!m.xcc || (m.NH * m.B) % 8 != 0)))
        return hipErrorInvalidValue;
    return cell == kLSTM ? launch_bwd_wide2_t<kLSTM>(m, s) : launch_bwd_wide2_t<kGRU>(m, s);
}

hipError_t launch_rec_bwd_wide(int cell, const WidePlan &p, const BwdArgs &m, hipStream_t s) {
    if (!p.ok || m.Dh != kWideDh) return hipErrorInvalidValue;
    return cell == kLSTM ? launch_bwd_wide_t<kLSTM>(p, m, s) : launch_bwd_wide_t<kGRU>(p, m, s);
}

hipError_t launch_rec_wide(int cell, const WidePlan &p, const RecArgs &a, const uint16_t *Rt,
                           hipStream_t s) {
    if (!p.ok || a.Dh != kWideDh || a.BT != 1 || a.ready) return hipErrorInvalidValue;
    return cell == kLSTM ? launch_wide_t<kLSTM>(p, a, Rt, s) : launch_wide_t<kGRU>(p, a, Rt, s);
}

}  // namespace rnn355
