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
// the device-coherent memory side); here it stays on one unit instead:
//   * 4 waves, one per SIMD (so each wave may hold 512 registers); wave w
//     owns hidden units [64w, 64w+64) = 4 blocks of 16 units, with all G
//     gate columns of each;
//   * the B fragments of v_mfma_f32_16x16x32_bf16 (k-chunks of 32) sit in
//     the accumulation registers (AGPRs: chunks 0..3 of the LSTM, 0..4 of
//     the GRU), in vector registers (LSTM 4..5, GRU 5..7), and the LSTM's
//     chunks 6..7 in LDS (128 KiB), read again at every step;
//   * one batch row per workgroup: the MFMA A operand holds h_{t-1} in row
//     0 only, the gate sums of a 16-unit block come out in row 0 of G
//     accumulator tiles, and the cell update runs as in the one-CU kernel
//     (cross-row swaps put the G gates of a unit in the 4 rows of one
//     register, one exp + rcp pass activates them all).  The other rows of
//     the A operand stay zero (MFMA rows are independent; the rows they
//     produce are never read).
// The MFMAs are inline assembly so that their B operand can be an AGPR:
// compiled from the builtin, every AGPR fragment was first copied to vector
// registers (four moves per MFMA, which a single wave per SIMD cannot hide).
// The compiler does not see these as MFMAs, so it inserts no wait states
// for their results; every read of an accumulator goes through
// `chain_end`, which carries the wait states of the MFMA-result hazard
// (16, twice what the compiler keeps for this instruction).  Their source
// operands come from memory loads (R fragments, h from LDS); each asm also
// carries the wait states that a VALU write of a source would need.
//
// HBM traffic per step: Gx_t (G*256 floats) read, h_t and c_t written, all
// in coalesced 16- or 4-byte lane accesses.  Steps go in groups of PD: at
// the start of group g the single wait on memory completes the Gx of group
// g+1 (requested at the start of g-1), which goes into an LDS ring slot; the
// Gx of group g+2 is requested into the same 8 registers; and the outputs
// of group g-1, staged in LDS, are written back.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "gates.h"
#include "kernels.h"

namespace rnn355 {

namespace {

constexpr int kWideDh = 256;
constexpr int kWideWaves = 4;

template <int CELL>
struct WideCfg {
    static constexpr int G = CellTraits<CELL>::G;
    static constexpr int KC = kWideDh / 32;            // k-chunks
    static constexpr int KA = CELL == kLSTM ? 4 : 5;   // chunks in AGPRs (256 / 240)
    static constexpr int KV = CELL == kLSTM ? 2 : 3;   // chunks in VGPRs (128 / 144)
    static constexpr int KL = KC - KA - KV;            // chunks in LDS
    static constexpr int NQ = kWideDh / 16 / kWideWaves;  // 16-unit blocks per wave
    static constexpr size_t kLdsR = (size_t)KL * (kWideDh / 16) * G * 64 * 16;
};

// acc = A . B (+ acc): v_mfma_f32_16x16x32_bf16 with B in an AGPR ("a") or a
// VGPR ("v").  The first MFMA of a chain takes 0 as its addend.  Each one
// starts with the two wait states an MFMA needs after a VALU write of one
// of its sources (the compiler may place a register copy right before the
// asm, not knowing it is an MFMA); inside a chain the nop overlaps the wait
// for the matrix pipe.
__device__ __forceinline__ void mfma_b_agpr_first(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_b_agpr(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_b_vgpr(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// 16 wait states between the last MFMA writing the accumulators and any
// instruction that reads them; the accumulators pass through the asm, so
// every reader depends on it.
template <int G>
__device__ __forceinline__ void chain_end(f32x4 (&acc)[G]) {
    if constexpr (G == 4)
        asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]));
}

template <int CELL>
__global__ __launch_bounds__(kWideWaves * 64, 1) void rec_fwd_wide_kernel(RecArgs a,
                                                                          const uint16_t *Rt) {
    using C = WideCfg<CELL>;
    constexpr int DH = kWideDh, G = C::G, GD = G * DH, KC = C::KC, KA = C::KA, KV = C::KV;
    constexpr int KL = C::KL, KR = KA + KV, NQ = C::NQ;
    constexpr int PD = 2;                                   // steps per Gx group
    constexpr int OUT_ROW = CELL == kLSTM ? 0 : 3;          // lanes that hold the result
    constexpr int NOUT = CELL == kLSTM ? 2 : 1;             // h (and c) outputs

    extern __shared__ __attribute__((aligned(16))) uint4 rl[];  // [KL][16 blocks][G][64 lanes]
    __shared__ __attribute__((aligned(16))) uint16_t hbuf[2][DH];     // h_{t-1}, step parity
    __shared__ __attribute__((aligned(16))) float obuf[2][PD][NOUT][DH];  // outputs, group parity
    // Gx ring, group parity; gate rows padded by 16 floats so the four lane
    // rows of a wave (one gate each) read distinct banks
    constexpr int GXP = DH + 16;
    __shared__ __attribute__((aligned(16))) float gxs[2][PD][G][GXP];

    const int n = blockIdx.x % a.NH, b = blockIdx.x / a.NH;
    const int H = a.NH * DH, N = a.NH * GD, T = a.T, B = a.B;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- R^T fragments: lane (lr, lg) of fragment (gate column col, chunk
    // c) holds R[k][col] for k = 32c + 8lg .. +8, 16 contiguous bytes of R^T
    const uint4 *Rn = reinterpret_cast<const uint4 *>(Rt + (long)n * GD * DH);
    bf16x8 ra[NQ][G][KA], rv[NQ][G][KV];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int col = g * DH + 64 * w + 16 * q + lr;
#pragma unroll
            for (int c = 0; c < KA; ++c)
                ra[q][g][c] = __builtin_bit_cast(bf16x8, Rn[(col * DH + 32 * c + 8 * lg) / 8]);
#pragma unroll
            for (int c = 0; c < KV; ++c)
                rv[q][g][c] = __builtin_bit_cast(bf16x8, Rn[(col * DH + 32 * (KA + c) + 8 * lg) / 8]);
        }
    for (int i = tid; i < KL * 16 * G * 64; i += kWideWaves * 64) {
        const int l = i & 63, f = i >> 6;
        const int g = f % G, ub = (f / G) % 16, c = KR + f / (16 * G);
        const int col = g * DH + 16 * ub + (l & 15);
        rl[i] = Rn[(col * DH + 32 * c + 8 * (l >> 4)) / 8];
    }
    const long o_row = (long)b * H + n * DH;  // this row's h/c in an output step
    for (int i = tid; i < 2 * DH; i += kWideWaves * 64) {
        const float v = (i < DH && a.h0) ? a.h0[o_row + i] : 0.f;
        (&hbuf[0][0])[i] = f32_to_bf16_rne(v);
    }

    // ---- lane roles: lane row lg takes Gx of gate lg (the GRU's fourth row
    // reads gate 2, unused); lanes of row OUT_ROW hold the results
    const bool wr = lg == OUT_ROW;
    const int lgx = lg < G ? lg : G - 1;
    const float *gx_row = a.gx + (long)b * N + n * GD;
    const long gx_step = (long)B * N, o_step = (long)B * H;
    float st[NQ], hl[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int j = 64 * w + 16 * q + lr;
        const float h0 = a.h0 ? a.h0[o_row + j] : 0.f;
        const float c0 = (CELL == kLSTM && a.c0) ? a.c0[o_row + j] : 0.f;
        st[q] = CELL == kLSTM ? c0 : h0;
        hl[q] = h0;
    }
    const bool has_h = a.h_seq != nullptr, has_c = CELL == kLSTM && a.c_seq != nullptr;

    // Gx of a group in flight: PD rows of GD floats, 16 bytes per lane
    constexpr int GX4 = PD * GD / 4;                       // float4 per group
    constexpr int GXI = (GX4 + kWideWaves * 64 - 1) / (kWideWaves * 64);
    float4 gxr[GXI];
#pragma unroll
    for (int i = 0; i < GXI; ++i) gxr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    auto load_group = [&](int tg) {
#pragma unroll
        for (int i = 0; i < GXI; ++i) {
            const int v = tid + i * kWideWaves * 64, s = v / (GD / 4), c4 = v % (GD / 4);
            if (v < GX4 && tg + s < T) {
                const float4 *src = reinterpret_cast<const float4 *>(gx_row + (long)(tg + s) * gx_step);
                gxr[i] = src[(unsigned)c4];
            }
        }
    };
    auto stage_group = [&](int tg) {
        const int par = (tg / PD) & 1;
#pragma unroll
        for (int i = 0; i < GXI; ++i) {
            const int v = tid + i * kWideWaves * 64, s = v / (GD / 4), c4 = v % (GD / 4);
            if (v < GX4) {
                const int col = 4 * c4, g = col / DH, j = col % DH;
                *reinterpret_cast<float4 *>(&gxs[par][s][g][j]) = gxr[i];
            }
        }
    };
    // outputs of steps [tg, tg+PD) from the LDS stage of that group: thread
    // i writes unit i, so each step's row is one coalesced 1 KiB store
    auto store_group = [&](int tg) {
        const int par = (tg / PD) & 1;
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (tg + s >= T) break;
            // wave-uniform row base (kept in SGPRs through an empty asm, so
            // the compiler does not hoist a per-lane 64-bit pointer out of
            // the loop) plus a 32-bit lane offset
            const long o = (long)(tg + s) * o_step + o_row;
            float *hp = a.h_seq + o, *cp = has_c ? a.c_seq + o : hp;
            asm volatile("" : "+s"(hp), "+s"(cp));
            if (has_h) hp[(unsigned)tid] = obuf[par][s][0][tid];
            if (has_c) cp[(unsigned)tid] = obuf[par][s][NOUT - 1][tid];
        }
    };

    // Gx of group 0 staged, group 1 in flight
    load_group(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    stage_group(0);
    load_group(PD);
    __syncthreads();

    bf16x8 af[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) af[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    auto run_group = [&](auto full, int tg) {
        const int par = (tg / PD) & 1;
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            const int t = tg + s;
            if (!decltype(full)::value && t >= T) break;
            if (s == 0) {
                // the next group's Gx (requested a group ago) and the stores
                // issued then are complete after this single wait.  Its ring
                // slot was last read in the previous group, before the
                // barrier that closed it.
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                stage_group(tg + PD);
                if (tg > 0) store_group(tg - PD);
                load_group(tg + 2 * PD);
            }
            const uint16_t *hc = hbuf[t & 1];
            uint16_t *hn = hbuf[(t + 1) & 1];
            // h_{t-1} as the A operand of all four blocks: row 0 only (4
            // lanes); the LDS is the LSTM's busiest unit (its R chunks are
            // read from it at every step), so the other rows are not filled
            if (lr == 0) {
#pragma unroll
                for (int c = 0; c < KC; ++c)
                    af[c] = *reinterpret_cast<const bf16x8 *>(hc + 32 * c + 8 * lg);
            }
            // Chain of block q: the LDS fragments are requested first and
            // used after the AGPR chunks, so their reads land meanwhile.
            auto chain = [&](int q, f32x4 (&acc)[G]) {
                bf16x8 lb[KL > 0 ? KL : 1][G];
#pragma unroll
                for (int c = 0; c < KL; ++c)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        lb[c][g] = __builtin_bit_cast(bf16x8, rl[((c * 16 + 4 * w + q) * G + g) * 64 + lane]);
#pragma unroll
                for (int c = 0; c < KA; ++c)
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        if (c == 0)
                            mfma_b_agpr_first(acc[g], af[c], ra[q][g][c]);
                        else
                            mfma_b_agpr(acc[g], af[c], ra[q][g][c]);
                    }
#pragma unroll
                for (int c = 0; c < KL; ++c)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        mfma_b_vgpr(acc[g], af[KR + c], lb[c][g]);
#pragma unroll
                for (int c = 0; c < KV; ++c)
#pragma unroll
                    for (int g = 0; g < G; ++g) mfma_b_vgpr(acc[g], af[KA + c], rv[q][g][c]);
                chain_end<G>(acc);
            };
            // Gate update of block q.  (Written after the chain of block q+1,
            // the two did not overlap: the compiler ran out of registers.)
            auto gates = [&](int q, f32x4 (&acc)[G]) {
                float h, cc;
                const int j = 64 * w + 16 * q + lr;
                gate_rows_update<CELL>(gate_rows_of<CELL>(acc), gxs[par][s][lgx][j], st[q], hl[q], h,
                                       cc);
                if (wr) {
                    hn[j] = f32_to_bf16_rne(h);
                    obuf[par][s][0][j] = h;
                    if (CELL == kLSTM) obuf[par][s][NOUT - 1][j] = cc;
                }
            };
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                f32x4 acc[G];
                chain(q, acc);
                gates(q, acc);
            }
            lds_barrier();
        }
    };

    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;
    const int tfull = T / PD * PD;
    for (int tg = 0; tg < tfull; tg += PD) run_group(Full{}, tg);
    int tlast = tfull - PD;
    if (tfull < T) {
        run_group(Part{}, tfull);
        tlast = tfull;
    }
    store_group(tlast);
    if (wr) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const long o = o_row + 64 * w + 16 * q + lr;
            a.hT[o] = CELL == kLSTM ? hl[q] : st[q];
            if (CELL == kLSTM) a.cT[o] = st[q];
        }
    }
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

hipError_t launch_rec_wide(int cell, const WidePlan &p, const RecArgs &a, const uint16_t *Rt,
                           hipStream_t s) {
    if (!p.ok || a.Dh != kWideDh || a.BT != 1 || a.ready) return hipErrorInvalidValue;
    return cell == kLSTM ? launch_wide_t<kLSTM>(p, a, Rt, s) : launch_wide_t<kGRU>(p, a, Rt, s);
}

}  // namespace rnn355
