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
// MFMA kernel (bf16 R, Dh a multiple of 32):
//   * R_n lives in VGPRs for the whole call as B-operand fragments of
//     v_mfma_f32_16x16x32_bf16: the G*Dh gate columns are cut into 16-wide
//     tiles, dealt round-robin to the waves; each wave holds its tiles for all
//     Dh/32 k-chunks (Dh=128, LSTM: 4 tiles x 4 chunks x 4 VGPRs = 64 VGPRs).
//   * h_{t-1} is kept in LDS as bf16 (the A operand: 16 rows = batch rows of
//     the tile, rows beyond the tile are zero).
//   * per step: one 16-byte LDS read per k-chunk, the MFMA chain, the 16x16
//     results go to LDS, barrier, then every thread updates its own units
//     (b, j) in float32 -- gate nonlinearities, c/h update, h_t back to LDS
//     as bf16 and h_t, c_t streamed to HBM -- barrier.
//   * Gx_t for a thread's units is prefetched PD steps ahead into registers.
// Simple kernel (f32, or shapes the MFMA kernel does not cover): R in LDS as
// float32, one thread per (row, gate column) dot product per step.
#include "common.h"
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

template <int CELL, int DH, int NW, int UPT, int PD>
__global__ __launch_bounds__(NW * 64) void rec_fwd_mfma_kernel(RecArgs a) {
    constexpr int G = CellTraits<CELL>::G;
    constexpr int GD = G * DH;
    constexpr int NT = GD / 16;   // 16-wide gate-column tiles
    constexpr int KC = DH / 32;   // k chunks of one MFMA
    constexpr int TPW = NT / NW;  // tiles per wave
    constexpr int NTH = NW * 64;
    constexpr int HLD = DH + 8;   // bf16 per h row in LDS (bank spread)
    constexpr int GLD = GD + 4;   // floats per gate row in LDS
    static_assert(NT % NW == 0, "tiles must split evenly over waves");
    static_assert(DH % 32 == 0, "Dh must be a multiple of 32");

    __shared__ __attribute__((aligned(16))) uint16_t hbuf[16 * HLD];
    __shared__ __attribute__((aligned(16))) float gbuf[16 * GLD];

    const int n = blockIdx.x % a.NH;
    const int b0 = (blockIdx.x / a.NH) * a.BT;
    const int rows = min(a.BT, a.B - b0);
    const int H = a.NH * DH, N = a.NH * GD;
    const int T = a.T, B = a.B;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- prologue: this wave's R fragments, resident for all T steps
    bf16x8 rf[TPW][KC];
    {
        const uint16_t *Rn = a.Rb + (long)n * DH * GD;
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
            const int col = 16 * (wave + NW * p) + lr;
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
                uint4 u4 = make_uint4(w[0], w[1], w[2], w[3]);
                rf[p][c] = __builtin_bit_cast(bf16x8, u4);
            }
        }
    }
    for (int i = tid; i < 16 * DH; i += NTH) {
        const int b = i / DH, j = i - b * DH;
        float v = 0.f;
        if (b < rows && a.h0) v = a.h0[(long)(b0 + b) * H + n * DH + j];
        hbuf[b * HLD + j] = f32_to_bf16_rne(v);
    }
    // ---- per-thread units (b, j): state stays in registers across steps
    float cst[UPT], hst[UPT];
    int ub[UPT], uj[UPT];
    bool uv[UPT];
#pragma unroll
    for (int q = 0; q < UPT; ++q) {
        const int u = tid + NTH * q;
        ub[q] = u / DH;
        uj[q] = u - ub[q] * DH;
        uv[q] = u < rows * DH;
        const long o = (long)(b0 + ub[q]) * H + n * DH + uj[q];
        cst[q] = (uv[q] && a.c0) ? a.c0[o] : 0.f;
        hst[q] = (uv[q] && a.h0) ? a.h0[o] : 0.f;
    }
    float ring[PD][UPT][G];
    auto load_gx = [&](int t, float (&dst)[UPT][G]) {
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            if (uv[q] && t < T) {
                const float *src = a.gx + ((long)t * B + b0 + ub[q]) * N + n * GD + uj[q];
#pragma unroll
                for (int g = 0; g < G; ++g) dst[q][g] = src[g * DH];
            }
        }
    };
#pragma unroll
    for (int s = 0; s < PD; ++s) load_gx(s, ring[s]);
    __syncthreads();

    for (int t0 = 0; t0 < T; t0 += PD) {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            const int t = t0 + s;
            if (t >= T) break;
            // ---- h_{t-1} R_n for this wave's tiles
            bf16x8 af[KC];
#pragma unroll
            for (int c = 0; c < KC; ++c)
                af[c] = *reinterpret_cast<const bf16x8 *>(hbuf + lr * HLD + 32 * c + 8 * lg);
            f32x4 acc[TPW];
#pragma unroll
            for (int p = 0; p < TPW; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KC; ++c)
#pragma unroll
                for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x32_bf16(af[c], rf[p][c], acc[p]);
#pragma unroll
            for (int p = 0; p < TPW; ++p) {
                const int col = 16 * (wave + NW * p) + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) gbuf[(4 * lg + r) * GLD + col] = acc[p][r];
            }
            float cur[UPT][G];
#pragma unroll
            for (int q = 0; q < UPT; ++q)
#pragma unroll
                for (int g = 0; g < G; ++g) cur[q][g] = ring[s][q][g];
            load_gx(t + PD, ring[s]);
            __syncthreads();
            // ---- gate update of this thread's units
#pragma unroll
            for (int q = 0; q < UPT; ++q) {
                if (uv[q]) {
                    float h, c;
                    lstm_or_gru_unit<CELL>(gbuf + ub[q] * GLD + uj[q], DH, cur[q], cst[q],
                                           hst[q], h, c);
                    hbuf[ub[q] * HLD + uj[q]] = f32_to_bf16_rne(h);
                    const long o = ((long)t * B + b0 + ub[q]) * H + n * DH + uj[q];
                    if (a.h_seq) a.h_seq[o] = h;
                    if (CELL == kLSTM && a.c_seq) a.c_seq[o] = c;
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int q = 0; q < UPT; ++q) {
        if (uv[q]) {
            const long o = (long)(b0 + ub[q]) * H + n * DH + uj[q];
            a.hT[o] = hst[q];
            if (CELL == kLSTM) a.cT[o] = cst[q];
        }
    }
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

// Gx prefetch distance in steps: 4, or 2 when each thread owns 4 units (the
// ring would otherwise push the Dh=128 LSTM past 256 VGPRs and spill).
template <int UPT>
constexpr int prefetch_steps() { return UPT >= 4 ? 2 : 4; }

int mfma_waves(int cell, int Dh) {
    if (cell == kLSTM) return 8;                 // NT = Dh/4 tiles: 8, 16, 32
    if (Dh == 32) return 6;                      // GRU NT = 6
    if (Dh == 64) return 12;                     // GRU NT = 12
    return 8;                                    // GRU Dh=128: NT = 24
}

template <int CELL, int DH, int NW>
hipError_t launch_mfma_upt(const RecPlan &p, const RecArgs &a, hipStream_t s) {
    switch (p.upt) {
        case 1:
            hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, NW, 1, prefetch_steps<1>()>), dim3(p.grid),
                               dim3(NW * 64), 0, s, a);
            break;
        case 2:
            hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, NW, 2, prefetch_steps<2>()>), dim3(p.grid),
                               dim3(NW * 64), 0, s, a);
            break;
        default:
            hipLaunchKernelGGL((rec_fwd_mfma_kernel<CELL, DH, NW, 4, prefetch_steps<4>()>), dim3(p.grid),
                               dim3(NW * 64), 0, s, a);
            break;
    }
    return hipGetLastError();
}

template <int CELL>
hipError_t launch_mfma(const RecPlan &p, const RecArgs &a, hipStream_t s) {
    constexpr bool L = CELL == kLSTM;
    switch (a.Dh) {
        case 32: return launch_mfma_upt<CELL, 32, L ? 8 : 6>(p, a, s);
        case 64: return launch_mfma_upt<CELL, 64, L ? 8 : 12>(p, a, s);
        case 128: return launch_mfma_upt<CELL, 128, 8>(p, a, s);
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
        p.waves = mfma_waves(cell, Dh);
        p.threads = p.waves * 64;
        const int units = bt * Dh;
        p.upt = (units + p.threads - 1) / p.threads;
        if (p.upt == 3) p.upt = 4;
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

hipError_t launch_rec_fwd(int cell, const RecPlan &p, const RecArgs &a, bool bf16,
                          hipStream_t s) {
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
