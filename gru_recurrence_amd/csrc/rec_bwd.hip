// rec_bwd.hip -- reverse-time recurrence of LSTM and GRU backpropagation
// through time (the sequential part of the backward), plus the small helper
// kernels of the backward pass.
//
// Backward of the recurrence A_t = Gx_t + h_{t-1} R (FlashRNN, arXiv
// 2412.07752, abstract: traditional RNNs trained through their sequential
// recurrence; blog.hotdry.top 2025-09-21, the paragraphs on the step
// dependency and on keeping R resident, which apply to the reverse sweep in
// the same way).  With the pre-activations A_t recomputed beforehand (fully
// parallel over t) the reverse sweep is, per step t = T-1 .. 0:
//     dh   = dL/dh_t (upstream) + dh_carry          tc = tanh(c_t)
//     dA_o = dh tc o(1-o)                           dc = dc_carry + dh o (1-tc^2)
//     dA_i = dc z i(1-i)    dA_z = dc i (1-z^2)     dA_f = dc c_{t-1} f(1-f)
//     dc_carry = dc f       dh_carry = dA_t R^T   (per head, block-diagonal)
// and after t = 0 the carries are dL/dh_0 and dL/dc_0.
//
// GRU (reset-after: A_r = Gx_r + S_r, A_z = Gx_z + S_z, A_n = Gx_n + r S_n
// with S = h_{t-1} R, h_t = (1-u) n + u h_{t-1}), from Gx and S kept apart:
//     dh   = dL/dh_t + dh_carry
//     dA_n = dh (1-u)(1-n^2)    dA_z = dh (h_{t-1} - n) u(1-u)
//     dA_r = dA_n S_n r(1-r)
//     dGx  = (dA_r, dA_z, dA_n)          (-> dW, dx, db)
//     dS   = (dA_r, dA_z, dA_n r)        (-> dR and the carry)
//     dh_carry = dh u + dS R^T.
//
// Mapping (mirrors the forward kernels): a (head, batch tile) group of K
// workgroups; workgroup `member` owns output units [member*U, (member+1)*U),
// wave (blk, ks) the 16-unit block blk and the ks-th range of the G*Dh gate
// columns (the reduction dimension here), holding the matching fragments of
// R^T -- lane l of chunk c reads R[n][unit][32c + 8(l/16) .. +8], one 16-byte
// load, so R's own row layout serves R^T.  The A operand is the row of dA_t
// (bf16, all G*Dh gate columns) in LDS.  After the MFMAs the lane that holds
// dh_carry of unit j and row b also computes the cell backward of (b, j), so
// all per-unit state stays in registers.  dA_t reaches the other members as
// step-tagged 8-byte words (as in the multi-CU forward) or, with K = 1,
// directly through LDS.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"
#include "xcd.h"

namespace rnn355 {

namespace {

template <int CELL, int KCW, int R4>
__global__ __launch_bounds__(512) void rec_bwd_kernel(BwdArgs m) {
    constexpr int G = CellTraits<CELL>::G;
    constexpr bool LSTM = CELL == kLSTM;
    const int Dh = m.Dh, K = m.K, KS = m.KS, NB = m.NB;
    const int U = NB * 16, GD = G * Dh, H = m.NH * Dh, N = m.NH * GD, ALD = GD + 8;
    const int T = m.T, B = m.B;

    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t *dab2 = smem;                                          // [2][BT][ALD] bf16
    float *red = reinterpret_cast<float *>(smem + 2 * m.BT * ALD);  // [KS-1][NB][16][16]
    __shared__ int s_abort, s_local;

    int group, member;
    group_member(m.xcd_map != 0, K, group, member);
    const int n = group % m.NH;
    const int bt = group / m.NH;
    const int b0 = bt * m.BT;
    const int rows = min(m.BT, B - b0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int blk = wave / KS, ks = wave - blk * KS;
    const bool gate_wave = ks == 0;
    const int j = member * U + blk * 16 + lr;  // this lane's hidden unit
    const int kc0 = ks * KCW;
    const int nthr = blockDim.x;

    // R^T fragments: B[k][col] = R[n][unit][k] for k in this wave's chunks
    bf16x8 rf[KCW];
    {
        const uint16_t *Rrow = m.Rb + ((long)n * Dh + j) * GD;
#pragma unroll
        for (int c = 0; c < KCW; ++c)
            rf[c] = *reinterpret_cast<const bf16x8 *>(Rrow + 32 * (kc0 + c) + 8 * lg);
    }
    for (int i = tid; i < 2 * m.BT * ALD; i += nthr) dab2[i] = 0;
    if (tid == 0) {
        s_abort = 0;
        s_local = 0;
    }
    if (m.xcd_map) xcd_publish(m.xcc);

    // per-lane state of the gate waves: row slots r -> batch row 4*lg + r
    bool rv[R4];
    unsigned oo[R4];
    float dhc[R4], dcc[R4], dir[R4], dbs[R4][G];
    const long o_tile = (long)b0 * H + n * Dh;
    const long a_tile = (long)b0 * N + n * GD;
#pragma unroll
    for (int r = 0; r < R4; ++r) {
        const int b = 4 * lg + r;
        rv[r] = gate_wave && b < rows;
        oo[r] = (unsigned)(b * H + j);
        dhc[r] = (rv[r] && m.dhT) ? m.dhT[o_tile + oo[r]] : 0.f;
        dcc[r] = (LSTM && rv[r] && m.dcT) ? m.dcT[o_tile + oo[r]] : 0.f;
        dir[r] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) dbs[r][g] = 0.f;
    }
    // streamed per step and row slot.  LSTM: pre-activations, c_t, c_{t-1},
    // dL/dh_t.  GRU: Gx (pa), S (sv), h_{t-1} (cp), dL/dh_t.
    float pa[R4][G], sv[R4][G], ct[R4], cp[R4], up[R4];
    auto load_step = [&](int t) {
#pragma unroll
        for (int r = 0; r < R4; ++r) {
            if (rv[r]) {
                const long ao = a_tile + (long)t * B * N + (long)(4 * lg + r) * N + j;
#pragma unroll
                for (int g = 0; g < G; ++g) pa[r][g] = m.A[ao + g * Dh];
                const long oo_t = o_tile + (long)t * B * H + oo[r];
                if constexpr (LSTM) {
                    ct[r] = m.c_seq[oo_t];
                    cp[r] = t > 0 ? m.c_seq[oo_t - (long)B * H]
                                  : (m.c0 ? m.c0[o_tile + oo[r]] : 0.f);
                } else {
#pragma unroll
                    for (int g = 0; g < G; ++g) sv[r][g] = m.S[ao + g * Dh];
                    cp[r] = t > 0 ? m.h_seq[oo_t - (long)B * H]
                                  : (m.h0 ? m.h0[o_tile + oo[r]] : 0.f);
                }
                up[r] = m.dh_seq[oo_t];
            }
        }
    };
    load_step(T - 1);
    __syncthreads();
    if (m.xcd_map && wave == 0) {
        const int v = xcd_members_agree(m.xcc, m.flag, m.spin_limit, group, K);
        if (lane == 0) {
            s_local = v > 0;
            if (v < 0) s_abort = 1;
        }
    }
    __syncthreads();
    // the group's members on one XCD: dA words stay in its L2 (see the
    // forward's multi-CU kernel), polled at device scope either way
    const bool local = s_local != 0;

    const int wpr = GD / 2;  // exchange words per row
    unsigned long long *xs_group = m.xg + (long)group * 2 * m.BT * wpr;
    // A operand: lanes of live batch rows load it every step.  With one row
    // slot the other lanes keep the zeros they start with (rewriting them
    // every step costs a dozen moves on the step's critical path); with more
    // they are rewritten (keeping them would spill).
    bf16x8 af[KCW];
#pragma unroll
    for (int c = 0; c < KCW; ++c) af[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    int s = s_abort ? T + 1 : 0;  // steps done
    for (; s < T; ++s) {
        const int t = T - 1 - s;
        uint16_t *dab_next = dab2 + (s & 1) * m.BT * ALD;  // filled with dA_t this step
        unsigned long long *slot = xs_group + (long)(s & 1) * m.BT * wpr;
        const unsigned long long tag = (unsigned long long)(unsigned)(s + 1) << 32;
        // ---- cell backward of this lane's units at step t
        if (gate_wave) {
#pragma unroll
            for (int r = 0; r < R4; ++r) {
                // d: gradients of the gate inputs Gx; e: of the recurrent
                // sums S (the same for the LSTM), exchanged for the carry
                float d[G], e[G];
                if constexpr (LSTM) {
                    const float ig = sigmoid_f(pa[r][0]), fg = sigmoid_f(pa[r][1]);
                    const float zg = tanh_f(pa[r][2]), og = sigmoid_f(pa[r][3]);
                    const float tc = tanh_f(ct[r]);
                    const float dh = up[r] + dhc[r];
                    const float dc = fmaf(dh * og, 1.0f - tc * tc, dcc[r]);
                    d[0] = dc * zg * ig * (1.0f - ig);
                    d[1] = dc * cp[r] * fg * (1.0f - fg);
                    d[2] = dc * ig * (1.0f - zg * zg);
                    d[3] = dh * tc * og * (1.0f - og);
                    dcc[r] = dc * fg;
#pragma unroll
                    for (int g = 0; g < G; ++g) e[g] = d[g];
                } else {
                    const float rg = sigmoid_f(pa[r][0] + sv[r][0]);
                    const float ug = sigmoid_f(pa[r][1] + sv[r][1]);
                    const float ng = tanh_f(fmaf(rg, sv[r][2], pa[r][2]));
                    const float dh = up[r] + dhc[r];
                    d[2] = dh * (1.0f - ug) * (1.0f - ng * ng);
                    d[1] = dh * (cp[r] - ng) * ug * (1.0f - ug);
                    d[0] = d[2] * sv[r][2] * rg * (1.0f - rg);
                    e[0] = d[0];
                    e[1] = d[1];
                    e[2] = d[2] * rg;
                    dir[r] = dh * ug;
                }
                uint16_t db16[G], de16[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    dbs[r][g] += rv[r] ? d[g] : 0.f;
                    db16[g] = f32_to_bf16_rne(d[g]);
                    de16[g] = LSTM ? db16[g] : f32_to_bf16_rne(e[g]);
                }
                if (rv[r]) {
                    const long o = a_tile + (long)t * B * N + (long)(4 * lg + r) * N + j;
#pragma unroll
                    for (int g = 0; g < G; ++g) m.dA[o + g * Dh] = db16[g];
                    if constexpr (!LSTM) {
#pragma unroll
                        for (int g = 0; g < G; ++g) m.dS[o + g * Dh] = de16[g];
                    }
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const unsigned v = de16[g];
                    const unsigned nb = (unsigned)__shfl_xor((int)v, 1);
                    if (rv[r]) {
                        const int row = 4 * lg + r, col = g * Dh + j;
                        if (K == 1) {
                            dab_next[row * ALD + col] = (uint16_t)v;
                        } else if ((lr & 1) == 0) {
                            unsigned long long *dst = slot + row * wpr + (col >> 1);
                            const unsigned long long w = tag | (nb << 16) | v;
                            if (local)
                                __hip_atomic_store(dst, w, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                            else
                                __hip_atomic_store(dst, w, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
            }
        }
        // next step's streamed inputs, issued as soon as this step's cell
        // update has used them: they land during the exchange and the MFMAs
        if (gate_wave && t > 0) load_step(t - 1);
        // ---- dA_t of the whole head row into LDS
        if (K > 1) {
            // PW words of a thread per poll, their loads in flight together
            constexpr int PW = 4;
            const int words = rows * wpr;
            unsigned *hw = reinterpret_cast<unsigned *>(dab_next);
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
                        hw[(b * ALD) / 2 + k2] = (unsigned)w[q];
                    }
                }
            }
        }
        __syncthreads();
        if (s_abort) break;
        // ---- dh_carry = dA_t R^T for this wave's gate-column range
        if (lr < rows) {
#pragma unroll
            for (int c = 0; c < KCW; ++c)
                af[c] = *reinterpret_cast<const bf16x8 *>(dab_next + lr * ALD + 32 * (kc0 + c) + 8 * lg);
        } else if (R4 > 1) {
#pragma unroll
            for (int c = 0; c < KCW; ++c) af[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
        // the GRU's direct term dh u enters as the chain's initial value, so no
        // vector instruction reads the MFMA result right after the chain (a
        // read across the branch below came without the wait states an MFMA
        // result needs and saw stale values)
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!LSTM) {
#pragma unroll
            for (int r = 0; r < R4; ++r) acc[r] = dir[r];
        }
#pragma unroll
        for (int c = 0; c < KCW; ++c) acc = mfma_16x16x32_bf16(af[c], rf[c], acc);
        mfma_chain_end();
        if (KS > 1) {
            if (!gate_wave) {
                float *dst = red + ((long)(ks - 1) * NB + blk) * 256;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(4 * lg + r) * 16 + lr] = acc[r];
            }
            __syncthreads();
            if (gate_wave) {
                for (int k2 = 1; k2 < KS; ++k2) {
                    const float *src = red + ((long)(k2 - 1) * NB + blk) * 256;
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += src[(4 * lg + r) * 16 + lr];
                }
            }
            // the next step rewrites `red` only after its own barrier
        }
#pragma unroll
        for (int r = 0; r < R4; ++r) dhc[r] = acc[r];
    }
    if (s == T) {
#pragma unroll
        for (int r = 0; r < R4; ++r) {
            if (rv[r]) {
                m.dh0[o_tile + oo[r]] = dhc[r];
                if (LSTM) m.dc0[o_tile + oo[r]] = dcc[r];
            }
        }
        // db partial of this batch tile: the lane's 4 gate sums over its rows
        // (row slots are combined by the lanes of one column: lanes lr with
        // the same unit in the four 16-lane rows, reduced through LDS)
        float *dbt = m.db_part + (long)bt * N + n * GD;
        if (gate_wave) {
            float sg[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < R4; ++r) v += dbs[r][g];
                sg[g] = v;
            }
            // sum over the 4 lane rows (batch rows 4lg..4lg+3) with cross-row
            // shuffles: lanes l, l^16, l^32, l^48 share the unit
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float v = sg[g];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (lg == 0) dbt[g * Dh + j] = v;
            }
        }
    }
}

template <int CELL, int KCW, int R4>
hipError_t launch_bwd_t(const BwdPlan &p, BwdArgs m, hipStream_t s) {
    void *args[] = {&m};
    return launch_all_resident(reinterpret_cast<const void *>(&rec_bwd_kernel<CELL, KCW, R4>),
                               p.grid, p.threads, args, p.lds, s);
}

template <int CELL, int KCW>
hipError_t launch_bwd_rows(const BwdPlan &p, const BwdArgs &m, hipStream_t s) {
    switch (p.r4) {
        case 1: return launch_bwd_t<CELL, KCW, 1>(p, m, s);
        case 2: return launch_bwd_t<CELL, KCW, 2>(p, m, s);
        default: return launch_bwd_t<CELL, KCW, 4>(p, m, s);
    }
}

template <int CELL>
hipError_t launch_bwd_cell(const BwdPlan &p, const BwdArgs &m, hipStream_t s) {
    switch (p.kcw) {
        case 16: return launch_bwd_rows<CELL, 16>(p, m, s);
        case 12: return launch_bwd_rows<CELL, 12>(p, m, s);
        case 8: return launch_bwd_rows<CELL, 8>(p, m, s);
        case 6: return launch_bwd_rows<CELL, 6>(p, m, s);
        case 4: return launch_bwd_rows<CELL, 4>(p, m, s);
        case 3: return launch_bwd_rows<CELL, 3>(p, m, s);
        case 2: return launch_bwd_rows<CELL, 2>(p, m, s);
        default: return hipErrorInvalidValue;
    }
}

// Zeroes up to three word ranges (null pointers skipped) in one launch.
__global__ void clear_words_bwd_kernel(unsigned *p, long n, unsigned *p2, long n2, unsigned *p3,
                                       long n3) {
    const long i0 = blockIdx.x * (long)blockDim.x + threadIdx.x, step = (long)gridDim.x * blockDim.x;
    if (p)
        for (long i = i0; i < n; i += step) p[i] = 0u;
    if (p2)
        for (long i = i0; i < n2; i += step) p2[i] = 0u;
    if (p3)
        for (long i = i0; i < n3; i += step) p3[i] = 0u;
}

// hprev[t][b][k] = bf16(h_{t-1}[b][k]) with h_{-1} = h0 (the MFMA operand the
// forward used), as the A operand of the dR and recompute contractions.
__global__ void hprev_bf16_kernel(const float *h0, const float *h_seq, uint16_t *hprev, long BH,
                                  long total) {
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
         i += (long)gridDim.x * blockDim.x) {
        const float v = i < BH ? (h0 ? h0[i] : 0.f) : h_seq[i - BH];
        hprev[i] = f32_to_bf16_rne(v);
    }
}

// The same, four elements per thread (16-byte loads, 8-byte stores): BH and
// total multiples of 4, h0, h_seq 16-byte and hprev 8-byte aligned.
__global__ void hprev_bf16_x4_kernel(const float *h0, const float *h_seq, uint16_t *hprev, long BH,
                                     long total) {
    for (long q = blockIdx.x * (long)blockDim.x + threadIdx.x; 4 * q < total;
         q += (long)gridDim.x * blockDim.x) {
        const long i = 4 * q;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i >= BH) v = *reinterpret_cast<const float4 *>(h_seq + (i - BH));
        else if (h0) v = *reinterpret_cast<const float4 *>(h0 + i);
        const uint2 w = make_uint2((unsigned)f32_to_bf16_rne(v.x) | ((unsigned)f32_to_bf16_rne(v.y) << 16),
                                   (unsigned)f32_to_bf16_rne(v.z) | ((unsigned)f32_to_bf16_rne(v.w) << 16));
        *reinterpret_cast<uint2 *>(hprev + i) = w;
    }
}

// db[c] = sum over batch tiles of db_part[bt][c], in tile order (added to
// the old db[c] if accumulate).
__global__ void db_reduce_kernel(const float *db_part, int nbt, int N, float *db, int accumulate) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= N) return;
    float v = 0.f;
    for (int b = 0; b < nbt; ++b) v += db_part[(long)b * N + c];
    db[c] = accumulate ? db[c] + v : v;
}

}  // namespace

BwdPlan plan_bwd(int cell, int B, int NH, int Dh, int num_cu, int bt_override, int k_override) {
    BwdPlan p{};
    const int G = cell == kLSTM ? 4 : 3;
    if (Dh % 16 != 0 || (G * Dh) % 32 != 0) return p;
    const int KC = G * Dh / 32;  // reduction chunks of 32 gate columns
    // at most 16 chunks per wave (its R^T fragments and the A fragments of
    // one step then take 64 VGPRs each): the largest of 16, 12, 8, 6, 4, 3, 2
    // that divides the chunk count (GRU counts are multiples of 3, LSTM
    // counts even, so one always does)
    p.kcw = 0;
    for (const int c : {16, 12, 8, 6, 4, 3, 2}) {
        if (KC % c == 0) {
            p.kcw = c;
            break;
        }
    }
    if (p.kcw == 0) return p;
    p.ks = KC / p.kcw;
    const int nb_max = 8 / p.ks;
    if (nb_max < 1) return p;
    int K = 0;
    for (int k = 1; k <= Dh / 16; ++k) {
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
    p.nbt = (B + bt - 1) / bt;
    if ((long)NH * p.nbt * K > num_cu) return p;
    p.BT = bt;
    p.r4 = bt >= 3 ? 4 : bt;
    p.groups = NH * p.nbt;
    p.grid = p.groups * K;
    p.lds = sizeof(uint16_t) * 2 * (size_t)bt * (G * Dh + 8) + sizeof(float) * (size_t)(p.ks - 1) * p.nb * 256;
    p.ok = 1;
    return p;
}

hipError_t launch_rec_bwd(int cell, const BwdPlan &p, const BwdArgs &m, hipStream_t s) {
    const int G = cell == kLSTM ? 4 : 3;
    if (m.xcd_map && (!m.xcc || p.groups % 8 != 0)) return hipErrorInvalidValue;
    // one launch: the status word, the XCD table, the exchange slots
    const long words = p.K > 1 ? 2L * p.groups * 2 * p.BT * (G * m.Dh / 2) : 0;
    hipLaunchKernelGGL(clear_words_bwd_kernel, dim3(64), dim3(256), 0, s,
                       m.keep_flag ? (unsigned *)nullptr : m.flag, 1L,
                       m.xcd_map ? m.xcc : (unsigned *)nullptr, m.xcd_map ? (long)p.grid : 0L,
                       p.K > 1 ? reinterpret_cast<unsigned *>(m.xg) : (unsigned *)nullptr, words);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return cell == kLSTM ? launch_bwd_cell<kLSTM>(p, m, s) : launch_bwd_cell<kGRU>(p, m, s);
}

hipError_t launch_hprev_bf16(const float *h0, const float *h_seq, uint16_t *hprev, long BH,
                             long total, hipStream_t s) {
    const bool x4 = BH % 4 == 0 && total % 4 == 0 && ((uintptr_t)h0 & 15) == 0 &&
                    ((uintptr_t)h_seq & 15) == 0 && ((uintptr_t)hprev & 7) == 0;
    if (x4)
        hipLaunchKernelGGL(hprev_bf16_x4_kernel, dim3(2048), dim3(256), 0, s, h0, h_seq, hprev, BH,
                           total);
    else
        hipLaunchKernelGGL(hprev_bf16_kernel, dim3(1024), dim3(256), 0, s, h0, h_seq, hprev, BH,
                           total);
    return hipGetLastError();
}

hipError_t launch_db_reduce(const float *db_part, int nbt, int N, float *db, hipStream_t s,
                            bool accumulate) {
    hipLaunchKernelGGL(db_reduce_kernel, dim3((N + 255) / 256), dim3(256), 0, s, db_part, nbt, N, db,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace rnn355
