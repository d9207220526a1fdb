// rec_bwd_f32.hip -- backpropagation through time for float32 calls.
//
// The float32 path keeps every intermediate in float32 (pre-activations,
// gate gradients, carries), so that the gradients meet a float32 bar; it
// serves the small shapes float32 calls are made for.  Reverse-time chain
// rule of the textbook cells (FlashRNN card, paperdance.org/p/2412.07752,
// abstract: LSTM and GRU trained through the strictly sequential
// recurrence; blog.hotdry.top 2025-09-21, the paragraph on head-wise
// splitting: each head has its own block of R, so a head's carries never
// mix with another head's):
//   LSTM, per step t = T-1 .. 0 (dh, dc: carries from step t+1)
//     dh += dL/dh_t;  tc = tanh(c_t)
//     dA_o = dh tc o(1-o);  dc += dh o (1 - tc^2)
//     dA_i = dc z i(1-i);  dA_z = dc i (1-z^2);  dA_f = dc c_{t-1} f(1-f)
//     dc <- dc f;  dh <- dA R^T (the head's block)
//   GRU (reset-after), with S = h_{t-1} R and n = tanh(Gx_n + r S_n)
//     dh += dL/dh_t;  dn = dh (1-u);  du = dh (h_{t-1} - n)
//     dGx_n = dn (1-n^2);  dGx_r = dGx_n S_n r(1-r);  dGx_z = du u(1-u)
//     dS = (dGx_r, dGx_z, dGx_n r);  dh <- dh u + dS R^T
// One workgroup per (head, tile of batch rows) walks all T steps with the
// head's R block in LDS (float32), one thread per (row, unit) for the cell
// derivative and one per (row, unit) for the carry product.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace rnn355 {

namespace {

constexpr int kF32Threads = 256;

// LDS: R [Dh][G Dh] | dS [BT][G Dh] | dh carry [BT][Dh] | dc carry [BT][Dh]
// | direct term (GRU: dh u) [BT][Dh].
template <int CELL>
__global__ __launch_bounds__(kF32Threads) void rec_bwd_f32_kernel(BwdF32Args a) {
    constexpr int G = CellTraits<CELL>::G;
    constexpr bool LSTM = CELL == kLSTM;
    extern __shared__ float fsm[];
    const int Dh = a.Dh, GD = G * Dh, BT = a.BT;
    const int H = a.NH * Dh, N = a.NH * GD, B = a.B;
    float *Rs = fsm;
    float *dSs = Rs + (size_t)Dh * GD;
    float *dhc = dSs + (size_t)BT * GD;
    float *dcc = dhc + (size_t)BT * Dh;
    float *dir = dcc + (size_t)BT * Dh;

    const int n = blockIdx.x % a.NH;
    const int b0 = (blockIdx.x / a.NH) * BT;
    const int rows = min(BT, B - b0);
    const int tid = threadIdx.x;
    for (int i = tid; i < Dh * GD; i += kF32Threads) Rs[i] = a.R[(long)n * Dh * GD + i];
    for (int i = tid; i < rows * Dh; i += kF32Threads) {
        const int r = i / Dh, j = i - r * Dh;
        const long o = (long)(b0 + r) * H + n * Dh + j;
        dhc[i] = a.dhT ? a.dhT[o] : 0.f;
        dcc[i] = (LSTM && a.dcT) ? a.dcT[o] : 0.f;
    }
    __syncthreads();
    for (int t = a.T - 1; t >= 0; --t) {
        // cell derivative of every (row, unit) of the tile
        for (int i = tid; i < rows * Dh; i += kF32Threads) {
            const int r = i / Dh, j = i - r * Dh;
            const long row = (long)t * B + b0 + r;
            const long ou = row * H + n * Dh + j;        // unit in [T][B][H]
            const long og = row * N + (long)n * GD + j;  // gate 0 of the unit in [T][B][N]
            const float dh = a.dh_seq[ou] + dhc[i];
            if constexpr (LSTM) {
                const float ig = sigmoid_f(a.A[og]), fg = sigmoid_f(a.A[og + Dh]);
                const float zg = tanh_f(a.A[og + 2 * Dh]), og_ = sigmoid_f(a.A[og + 3 * Dh]);
                const float ct = a.c_seq[ou];
                const float cp = t > 0 ? a.c_seq[ou - (long)B * H]
                                       : (a.c0 ? a.c0[(long)(b0 + r) * H + n * Dh + j] : 0.f);
                const float tc = tanh_f(ct);
                const float dc = dcc[i] + dh * og_ * (1.f - tc * tc);
                const float d_i = dc * zg * ig * (1.f - ig);
                const float d_f = dc * cp * fg * (1.f - fg);
                const float d_z = dc * ig * (1.f - zg * zg);
                const float d_o = dh * tc * og_ * (1.f - og_);
                dcc[i] = dc * fg;
                a.dA[og] = d_i;
                a.dA[og + Dh] = d_f;
                a.dA[og + 2 * Dh] = d_z;
                a.dA[og + 3 * Dh] = d_o;
                float *ds = dSs + (size_t)r * GD + j;
                ds[0] = d_i;
                ds[Dh] = d_f;
                ds[2 * Dh] = d_z;
                ds[3 * Dh] = d_o;
            } else {
                const float sr = a.S[og], sz = a.S[og + Dh], sn = a.S[og + 2 * Dh];
                const float rg = sigmoid_f(a.A[og] + sr);
                const float ug = sigmoid_f(a.A[og + Dh] + sz);
                const float ng = tanh_f(fmaf(rg, sn, a.A[og + 2 * Dh]));
                const float hp = a.hprev[ou];
                const float dn = dh * (1.f - ug);
                const float du = dh * (hp - ng);
                const float dan = dn * (1.f - ng * ng);
                const float dar = dan * sn * rg * (1.f - rg);
                const float dau = du * ug * (1.f - ug);
                a.dA[og] = dar;
                a.dA[og + Dh] = dau;
                a.dA[og + 2 * Dh] = dan;
                a.dS[og] = dar;
                a.dS[og + Dh] = dau;
                a.dS[og + 2 * Dh] = dan * rg;
                float *ds = dSs + (size_t)r * GD + j;
                ds[0] = dar;
                ds[Dh] = dau;
                ds[2 * Dh] = dan * rg;
                dir[i] = dh * ug;
            }
        }
        __syncthreads();
        // carry into step t-1: dh[m] = (GRU: dh u +) sum_c dS[c] R[m][c]
        for (int i = tid; i < rows * Dh; i += kF32Threads) {
            const int r = i / Dh, m = i - r * Dh;
            const float *ds = dSs + (size_t)r * GD;
            const float *rr = Rs + (size_t)m * GD;
            float s = LSTM ? 0.f : dir[i];
            for (int c = 0; c < GD; ++c) s = fmaf(ds[c], rr[c], s);
            dhc[i] = s;
        }
        __syncthreads();
    }
    for (int i = tid; i < rows * Dh; i += kF32Threads) {
        const int r = i / Dh, j = i - r * Dh;
        const long o = (long)(b0 + r) * H + n * Dh + j;
        a.dh0[o] = dhc[i];
        if (LSTM) a.dc0[o] = dcc[i];
    }
}

// hprev[i] = h_{t-1} of flat entry i of [T][B][H]: h0 (or 0) for t = 0, h_seq
// of the step before otherwise.
__global__ void hprev_f32_kernel(const float *__restrict__ h0, const float *__restrict__ h_seq,
                                 float *__restrict__ hprev, long BH, long MH) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < MH;
         i += (long)gridDim.x * blockDim.x)
        hprev[i] = i < BH ? (h0 ? h0[i] : 0.f) : h_seq[i - BH];
}

// out[c] (+)= sum_m X[m][c], one column per thread, rows in order.
__global__ void colsum_f32_kernel(const float *__restrict__ X, long M, int N,
                                  float *__restrict__ out, int accumulate) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= N) return;
    float s = 0.f;
    for (long m = 0; m < M; ++m) s += X[m * N + c];
    out[c] = accumulate ? out[c] + s : s;
}

}  // namespace

BwdF32Plan plan_bwd_f32(int cell, int B, int Dh) {
    BwdF32Plan p{};
    const int G = cell == kLSTM ? 4 : 3;
    int bt = std::min(B, 8);
    for (;;) {
        const size_t lds = sizeof(float) * ((size_t)Dh * G * Dh + (size_t)bt * G * Dh + 3u * bt * Dh);
        if (lds <= kBwdF32MaxLds) {
            p.ok = 1;
            p.BT = bt;
            p.lds = lds;
            p.nbt = (B + bt - 1) / bt;
            return p;
        }
        if (bt == 1) return p;
        bt = (bt + 1) / 2;
    }
}

hipError_t launch_rec_bwd_f32(int cell, const BwdF32Plan &p, const BwdF32Args &a, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&rec_bwd_f32_kernel<kLSTM>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBwdF32MaxLds);
        if (attr == hipSuccess)
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&rec_bwd_f32_kernel<kGRU>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kBwdF32MaxLds);
    });
    if (attr != hipSuccess) return attr;
    if (!p.ok || a.BT != p.BT) return hipErrorInvalidValue;
    const dim3 grid(a.NH * p.nbt), blk(kF32Threads);
    if (cell == kLSTM)
        hipLaunchKernelGGL(rec_bwd_f32_kernel<kLSTM>, grid, blk, p.lds, s, a);
    else
        hipLaunchKernelGGL(rec_bwd_f32_kernel<kGRU>, grid, blk, p.lds, s, a);
    return hipGetLastError();
}

hipError_t launch_hprev_f32(const float *h0, const float *h_seq, float *hprev, long BH, long MH,
                            hipStream_t s) {
    const long blocks = std::min<long>(4096, (MH + 255) / 256);
    hipLaunchKernelGGL(hprev_f32_kernel, dim3((unsigned)std::max<long>(blocks, 1)), dim3(256), 0,
                       s, h0, h_seq, hprev, BH, MH);
    return hipGetLastError();
}

hipError_t launch_colsum_f32(const float *X, long M, int N, float *out, bool accumulate,
                             hipStream_t s) {
    hipLaunchKernelGGL(colsum_f32_kernel, dim3((N + 255) / 256), dim3(256), 0, s, X, M, N, out,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace rnn355
