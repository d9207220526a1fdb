// host_bwd.hip -- host side of backpropagation through time (bf16 and float32).
#include "host.h"

namespace rnn355 {
namespace host {

// Backpropagation through time (pointers validated by the entry points).
// 1. h_{t-1} as bf16, the gate inputs recomputed for all t at once: LSTM A =
//    x W + b + h_{t-1} R; GRU Gx = x W + b and S = h_{t-1} R apart.
// 2. The reverse sweep (rec_bwd.hip) -> dA (and the GRU's dS), db partials,
//    dh0 (dc0).
// 3. db, dW = x^T dA, dx = dA W^T, dR = h_{t-1}^T dS (dS = dA for the LSTM).
// accumulate: add dW, dR and db to what they hold (a later segment of a
// checkpointed backward); clear_status: zero the status word first.
// Float32 BPTT: every step in float32 (rec_bwd_f32.hip for the sweep, the
// float32 contraction for the recompute and the parameter gradients).
rnn_status backward_f32(int cell, const rnn_dims *d, const float *x, const float *W,
                        const float *R, const float *b, const float *h0, const float *c0,
                        const float *h_seq, const float *c_seq, const float *dh_seq,
                        const float *dhT, const float *dcT, float *dx, float *dW, float *dR,
                        float *db, float *dh0, float *dc0, void *ws, size_t ws_bytes,
                        hipStream_t s, bool accumulate, bool clear_status) {
    const bool lstm = cell == kLSTM;
    const int G = lstm ? 4 : 3, Dh = d->Dh, NH = d->NH, T = d->T, B = d->B, Din = d->Din;
    const int GD = G * Dh, N = NH * GD, H = NH * Dh;
    const long M = (long)T * B;
    const BwdF32Plan p = plan_bwd_f32(cell, B, Dh);
    if (!p.ok) return RNN_ERR_UNSUPPORTED;
    const rnn_op op = lstm ? RNN_OP_BWD_LSTM : RNN_OP_BWD_GRU;
    if (!ws || ws_bytes < rnn_workspace_size(op, d, RNN_F32)) return RNN_ERR_WORKSPACE;
    char *base = (char *)ws + kHeader;
    const BwdF32Layout L = bwd_f32_layout(d, G);
    float *A = (float *)(base + L.A);
    float *S = lstm ? A : (float *)(base + L.S);
    float *dA = (float *)(base + L.dA);
    float *dS = lstm ? dA : (float *)(base + L.dS);
    float *hprev = (float *)(base + L.hprev);
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    if (clear_status) {
        hipLaunchKernelGGL(status_word_kernel, dim3(1), dim3(64), 0, s, (unsigned *)ws,
                           (unsigned *)nullptr);
        if (!ok(hipGetLastError())) return RNN_ERR_HIP;
    }
    // 1. h_{t-1}; A = x W + b, then + h_{t-1} R per head (LSTM) or S = h_{t-1} R (GRU)
    if (!ok(launch_hprev_f32(h0, h_seq, hprev, (long)B * H, M * H, s))) return RNN_ERR_HIP;
    {
        GemmF32Args g{};
        g.M = (int)M; g.N = N; g.K = Din;
        g.A = x; g.sam = Din; g.sak = 1;
        g.B = W; g.sbk = N; g.sbn = 1;
        g.bias = b; g.C = A; g.ldc = N;
        if (!ok(launch_gemm_f32(g, 1, s))) return RNN_ERR_HIP;
    }
    {
        GemmF32Args g{};
        g.M = (int)M; g.N = GD; g.K = Dh;
        g.A = hprev; g.sam = H; g.sak = 1; g.strideA = Dh;
        g.B = R; g.sbk = GD; g.sbn = 1; g.strideB = (long)Dh * GD;
        g.C = S; g.ldc = N; g.strideC = GD;
        g.accumulate = lstm ? 1 : 0;
        if (!ok(launch_gemm_f32(g, NH, s))) return RNN_ERR_HIP;
    }
    // 2. the reverse-time sweep
    {
        BwdF32Args a{};
        a.T = T; a.B = B; a.NH = NH; a.Dh = Dh; a.BT = p.BT;
        a.A = A; a.S = lstm ? nullptr : S;
        a.c_seq = c_seq; a.c0 = c0; a.hprev = hprev;
        a.dh_seq = dh_seq; a.dhT = dhT; a.dcT = dcT;
        a.R = R; a.dA = dA; a.dS = lstm ? nullptr : dS;
        a.dh0 = dh0; a.dc0 = dc0;
        if (!ok(launch_rec_bwd_f32(cell, p, a, s))) return RNN_ERR_HIP;
    }
    // 3. db = sum dA; dW = x^T dA; dx = dA W^T; dR_n = h_{t-1,n}^T dS_n
    if (!ok(launch_colsum_f32(dA, M, N, db, accumulate, s))) return RNN_ERR_HIP;
    {
        GemmF32Args g{};
        g.M = Din; g.N = N; g.K = (int)M;
        g.A = x; g.sam = 1; g.sak = Din;
        g.B = dA; g.sbk = N; g.sbn = 1;
        g.C = dW; g.ldc = N;
        g.accumulate = accumulate ? 1 : 0;
        if (!ok(launch_gemm_f32(g, 1, s))) return RNN_ERR_HIP;
    }
    {
        GemmF32Args g{};
        g.M = (int)M; g.N = Din; g.K = N;
        g.A = dA; g.sam = N; g.sak = 1;
        g.B = W; g.sbk = 1; g.sbn = N;
        g.C = dx; g.ldc = Din;
        if (!ok(launch_gemm_f32(g, 1, s))) return RNN_ERR_HIP;
    }
    {
        GemmF32Args g{};
        g.M = Dh; g.N = GD; g.K = (int)M;
        g.A = hprev; g.sam = 1; g.sak = H; g.strideA = Dh;
        g.B = dS; g.sbk = N; g.sbn = 1; g.strideB = GD;
        g.C = dR; g.ldc = GD; g.strideC = (long)Dh * GD;
        g.accumulate = accumulate ? 1 : 0;
        if (!ok(launch_gemm_f32(g, NH, s))) return RNN_ERR_HIP;
    }
    return RNN_OK;
}



// Chunk starts for a backward over T steps: starts[0] = 0 < ... <
// starts[n] = T, n chunks of ceil(T / n) steps (the last one shorter when n
// does not divide T), n = min(kBwdChunks or RNN355_BWD_CHUNKS, T /
// kBwdMinChunk), at least 1; returns n.
int bwd_chunk_starts(int T, int *starts) {
    int n = std::min(kBwdChunks, env_int_or("RNN355_BWD_CHUNKS", kBwdChunks));
    n = std::max(1, std::min(n, T / kBwdMinChunk));
    const int ch = (T + n - 1) / n;
    for (int c = 0; c < n; ++c) starts[c] = c * ch;
    starts[n] = T;
    return n;
}

BwdChoice choose_bwd(int cell, const rnn_dims *d, int cus) {
    BwdChoice c{};
    const int B = d->B, NH = d->NH, Dh = d->Dh;
    c.pw = wide_enabled() ? plan_wide(cell, B, NH, Dh, true) : WidePlan{};
    c.p = c.pw.ok ? BwdPlan{} : plan_bwd(cell, B, NH, Dh, cus, bt_override(), k_override());
    c.ok = c.pw.ok || c.p.ok;
    if (!c.ok) return c;
    c.two = c.pw.ok && env_int_or("RNN355_BWD_WIDE2", 1) != 0 && mc_xcd_enabled() &&
            mc_xcd_grouping(NH * B, 2 * NH * B) && 2 * NH * B <= cus;
    c.sweep_grid = c.two ? 2 * NH * B : c.pw.ok ? c.pw.grid : c.p.grid;
    c.free_cus = (cus - c.sweep_grid) / 8 * 8;
    int starts[kBwdChunks + 1];
    c.chunks = c.free_cus >= 64 && env_int_or("RNN355_BWD_OVERLAP", 1) != 0
                   ? bwd_chunk_starts(d->T, starts)
                   : 1;
    return c;
}

rnn_status backward(int cell, const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                    const void *R, const float *b, const float *h0, const float *c0,
                    const float *h_seq, const float *c_seq, const float *dh_seq,
                    const float *dhT, const float *dcT, float *dx, float *dW, float *dR,
                    float *db, float *dh0, float *dc0, void *ws, size_t ws_bytes,
                    hipStream_t stream, bool accumulate, bool clear_status) {
    if (dt == RNN_F32)
        return backward_f32(cell, d, (const float *)x, (const float *)W, (const float *)R, b, h0,
                            c0, h_seq, c_seq, dh_seq, dhT, dcT, dx, dW, dR, db, dh0, dc0, ws,
                            ws_bytes, stream, accumulate, clear_status);
    if (dt != RNN_BF16) return RNN_ERR_UNSUPPORTED;
    const bool lstm = cell == kLSTM;
    const int G = lstm ? 4 : 3, Dh = d->Dh, NH = d->NH, T = d->T, B = d->B, Din = d->Din;
    const int GD = G * Dh, N = NH * GD, H = NH * Dh, M = T * B;
    if (!gemm_shape_ok(Din, N, dt) || Dh % 16 != 0) return RNN_ERR_UNSUPPORTED;
    // Dh = 256: one workgroup per (head, batch row) with R split over
    // registers and LDS (or two CUs per (head, row)); otherwise the
    // exchange-based sweep
    const int cus = device_cus();
    const BwdChoice bc = choose_bwd(cell, d, cus);
    if (!bc.ok) return RNN_ERR_UNSUPPORTED;
    const WidePlan &pw = bc.pw;
    const BwdPlan &p = bc.p;
    const int nbt = pw.ok ? B : p.nbt;  // rows of db partials
    const rnn_op op = lstm ? RNN_OP_BWD_LSTM : RNN_OP_BWD_GRU;
    if (!ws || ws_bytes < rnn_workspace_size(op, d, dt)) return RNN_ERR_WORKSPACE;

    char *base = (char *)ws + kHeader;
    const BwdLayout L = bwd_layout(d, G);
    float *A = (float *)(base + L.A);
    float *S = lstm ? A : (float *)(base + L.S);
    uint16_t *dA = (uint16_t *)(base + L.dA);
    uint16_t *dS = lstm ? dA : (uint16_t *)(base + L.dS);
    uint16_t *hprev = (uint16_t *)(base + L.hprev);
    float *dbp = (float *)(base + L.dbp);
    uint16_t *wt = (uint16_t *)(base + L.wt);
    uint16_t *rt = (uint16_t *)(base + L.rt);
    const uint16_t *xb = (const uint16_t *)x, *Wb = (const uint16_t *)W, *Rb = (const uint16_t *)R;
    auto ok = [](hipError_t e) { return e == hipSuccess; };

    // 1. h_{t-1} as bf16; gate inputs for all t at once
    if (!ok(launch_hprev_bf16(h0, h_seq, hprev, (long)B * H, (long)M * H, stream))) return RNN_ERR_HIP;
    uint32_t *clear = clear_status ? (uint32_t *)ws : nullptr;
    if (lstm && GD % kGemmColTile == 0 && gemm_dma_ok(Din) && gemm_dma_ok(Dh)) {
        // one contraction: the K tiles of x W^T, then for the column tiles of
        // head n those of h_{t-1}[:, n Dh:(n+1) Dh] R_n (R^T per head)
        if (!ok(launch_transpose_bf16(Wb, wt, Din, N, 1, stream, nullptr, 0, nullptr, 0, Rb, rt,
                                      Dh, GD, NH)))
            return RNN_ERR_HIP;
        GemmArgs g{};
        g.M = M; g.N = N; g.K = Din;
        g.A = xb; g.lda = Din;
        g.B = wt; g.ldb = Din;
        g.bias = b; g.C = A; g.ldc = N;
        g.clear_words = clear;
        g.A2 = hprev; g.lda2 = H; g.K2 = Dh; g.seg_n = GD;
        g.B2 = rt; g.ldb2 = Dh;  // row n = head n/GD's gate column n%GD
        if (!ok(launch_gemm_dma(g, 1, stream))) return RNN_ERR_HIP;
    } else {
        if (input_proj(M, Din, N, dt, x, W, b, A, clear, stream, nullptr, wt) != RNN_OK)
            return RNN_ERR_HIP;
        GemmArgs g{};  // h_{t-1} R per head: added to A (LSTM) or into S (GRU)
        g.M = M; g.N = GD; g.K = Dh;
        g.A = hprev; g.lda = H; g.strideA = Dh;       // row m, k = unit of head n
        g.C = S; g.ldc = N; g.strideC = GD;
        g.accumulate = lstm ? 1 : 0;
        if (gemm_dma_ok(Dh)) {
            // R^T per head: B(c, k) = R[n][k][c] at rt[n][c][k]
            if (!ok(launch_transpose_bf16(Rb, rt, Dh, GD, NH, stream))) return RNN_ERR_HIP;
            g.B = rt; g.ldb = Dh; g.strideB = (long)GD * Dh;
            if (!ok(launch_gemm_dma(g, NH, stream))) return RNN_ERR_HIP;
        } else {
            g.B = Rb; g.ldb = GD; g.strideB = (long)Dh * GD;  // R[n][k][c]: r-major
            if (!ok(launch_gemm_bf16(g, true, false, NH, stream))) return RNN_ERR_HIP;
        }
    }
    // 2. the reverse-time sweep and 3. the parameter and input gradients.
    // Where the sweep leaves at least 64 compute units free and T allows,
    // the sweep runs in up to kBwdChunks time chunks, the last one first,
    // each from the carries (dL/dh, dL/dc at its end) the later chunk left in
    // the workspace -- the carries pass through memory as float32, so the
    // sweep's values are the same bits as in one piece.  Once a chunk is
    // swept, its dx rows (one stream) and its shares of dW, dR and db (sums
    // over its time steps; another stream) run on half the free units each,
    // beside the next chunk's sweep.  The first chunk's gradients, swept
    // last, run over the whole chip: its dx on the dx stream beside its dW,
    // dR and db on the caller's stream.  dW, dR and db
    // add the chunks' shares in sweep order (deterministic, not the one-piece
    // summation order).  RNN355_BWD_OVERLAP=0 keeps the sweep in one piece.
    const bool two = bc.two;
    const int free_cus = bc.free_cus;
    int starts[kBwdChunks + 1];
    const int nch = bc.chunks > 1 ? bwd_chunk_starts(T, starts) : 1;
    // dx on one stream, dW, dR and db on the other, each on half the free units
    hipStream_t side = nch > 1 ? side_stream(0) : nullptr, side2 = nch > 1 ? side_stream(1) : nullptr;
    CallEvents ev(nch > 1);
    const bool split = nch > 1 && side && side2 && ev.ok;
    const int half = free_cus / 16 * 8;
    if (!split) {
        starts[0] = 0;
        starts[1] = T;
    }
    const int nc = split ? nch : 1;
    const long BHl = (long)B * H;
    float *part = (float *)(base + L.part);
    const size_t bh = align_up(sizeof(float) * (size_t)BHl);
    float *car_h[2] = {(float *)(base + L.car), (float *)(base + L.car + bh)};
    float *car_c[2] = {(float *)(base + L.car + 2 * bh), (float *)(base + L.car + 3 * bh)};

    // the sweep over steps [t0, t0 + Tc)
    auto sweep = [&](int c, int t0, int Tc) -> bool {
        BwdArgs m{};
        const bool last = c == nc - 1, first = c == 0;
        m.T = Tc; m.B = B; m.NH = NH; m.Dh = Dh; m.BT = p.BT;
        m.K = p.K; m.KS = p.ks; m.NB = p.nb;
        m.A = A + (long)t0 * B * N; m.S = lstm ? nullptr : S + (long)t0 * B * N;
        m.c_seq = c_seq ? c_seq + t0 * BHl : nullptr;
        m.c0 = t0 == 0 ? c0 : c_seq ? c_seq + (t0 - 1) * BHl : nullptr;
        m.h_seq = h_seq + t0 * BHl;
        m.h0 = t0 == 0 ? h0 : h_seq + (t0 - 1) * BHl;
        m.dh_seq = dh_seq + t0 * BHl;
        m.dhT = last ? dhT : car_h[(c + 1) & 1];
        m.dcT = !lstm ? nullptr : last ? dcT : car_c[(c + 1) & 1];
        m.Rb = Rb; m.dA = dA + (long)t0 * B * N; m.dS = lstm ? nullptr : dS + (long)t0 * B * N;
        m.db_part = dbp + (long)c * nbt * N;
        m.dh0 = first ? dh0 : car_h[c & 1];
        m.dc0 = !lstm ? nullptr : first ? dc0 : car_c[c & 1];
        m.xg = (unsigned long long *)(base + L.xchg);
        m.flag = (unsigned *)ws;
        // the status word is cleared by the first sweep of a call that clears
        // it; later pieces keep what the earlier ones reported
        m.keep_flag = !clear_status || !last;
        if (!pw.ok && p.K > 1 && mc_xcd_enabled() && mc_xcd_grouping(p.groups, p.grid)) {
            m.xcd_map = 1;
            m.xcc = (unsigned *)((char *)ws + kXccOffset);
        }
        m.spin_limit = spin_limit();
        hipError_t e;
        if (two) {
            m.xcd_map = 1;
            m.xcc = (unsigned *)((char *)ws + kXccOffset);
            e = launch_rec_bwd_wide2(cell, m, stream);
        } else {
            e = pw.ok ? launch_rec_bwd_wide(cell, pw, m, stream) : launch_rec_bwd(cell, p, m, stream);
        }
        return ok(e);
    };
    // dx rows of steps [t0, t0 + Tc) on stream st; units > 0: at most that
    // many workgroups (the dx rows of a chunk are written once: no order)
    auto grad_x = [&](int t0, int Tc, hipStream_t st, int units) -> bool {
        const long r0 = (long)t0 * B;
        GemmArgs g{};  // dx[m][k] = sum_c dA[m][c] W[k][c]
        g.M = Tc * B; g.N = Din; g.K = N;
        g.A = dA + r0 * N; g.lda = N; g.B = Wb; g.ldb = N; g.C = dx + r0 * Din; g.ldc = Din;
        return ok(gemm_dma_ok(N) ? launch_gemm_dma(g, 1, st, units)
                                 : launch_gemm_bf16(g, true, true, 1, st));
    };
    // the dW, dR and db shares of chunk c, steps [t0, t0 + Tc), on stream
    // st, split for `units` compute units (units < cus: every launch at
    // most that many workgroups); acc: add to dW, dR and db
    auto grad_w = [&](int c, int t0, int Tc, hipStream_t st, int units, bool acc) -> bool {
        const long r0 = (long)t0 * B;
        const int Mc = Tc * B;
        {
            GemmArgs g{};  // dW[k][c] (+)= sum_m x[m][k] dA[m][c]
            g.M = Din; g.N = N; g.K = Mc;
            g.A = xb + r0 * Din; g.lda = Din; g.B = dA + r0 * N; g.ldb = N; g.C = dW; g.ldc = N;
            g.accumulate = acc ? 1 : 0;
            g.ksplit = std::min(gemm_splitk_for(Din, N, Mc, 1, units), kMaxSplitK);
            g.partial = part;
            if (!ok(launch_gemm_bf16(g, false, false, 1, st))) return false;
        }
        {
            GemmArgs g{};  // dR[n][i][c] (+)= sum_m h_{t-1}[m][n*Dh+i] dS[m][n*GD+c]
            g.M = Dh; g.N = GD; g.K = Mc;
            g.A = hprev + r0 * H; g.lda = H; g.strideA = Dh;
            g.B = dS + r0 * N; g.ldb = N; g.strideB = GD;
            g.C = dR; g.ldc = GD; g.strideC = (long)Dh * GD;
            g.accumulate = acc ? 1 : 0;
            g.ksplit = std::min(gemm_splitk_for(Dh, GD, Mc, NH, units), kMaxSplitKdR);
            g.partial = part;
            if (!ok(launch_gemm_bf16(g, false, false, NH, st))) return false;
        }
        return ok(launch_db_reduce(dbp + (long)c * nbt * N, nbt, N, db, st, acc));
    };
    for (int c = nc - 1; c >= 0; --c) {
        const int t0 = starts[c], Tc = starts[c + 1] - t0;
        if (!sweep(c, t0, Tc)) return RNN_ERR_HIP;
        if (c > 0) {
            // this chunk's gradients beside the next chunk's sweep
            if (!ok(hipEventRecord(ev.e[c], stream)) || !ok(hipStreamWaitEvent(side, ev.e[c], 0)) ||
                !ok(hipStreamWaitEvent(side2, ev.e[c], 0)) || !grad_x(t0, Tc, side, half) ||
                !grad_w(c, t0, Tc, side2, half, accumulate || c != nc - 1))
                return RNN_ERR_HIP;
        } else if (nc == 1) {
            if (!grad_x(t0, Tc, stream, 0) || !grad_w(0, t0, Tc, stream, cus, accumulate))
                return RNN_ERR_HIP;
        } else {
            // the first chunk: its dx on the dx stream (behind the other
            // chunks' dx) beside its dW, dR and db on the caller's stream,
            // which wait for the other chunks' shares; the call ends when
            // every dx is done
            const int xt = ((Tc * B + kGemmRowTile - 1) / kGemmRowTile) *
                           ((Din + kGemmColTile - 1) / kGemmColTile);
            const int wu = std::max(64, (cus - xt) / 8 * 8);  // CUs the dx tiles leave
            hipEvent_t swept = ev.e[0], w_done = ev.e[kBwdChunks], x_done = ev.e[kBwdChunks + 1];
            if (!ok(hipEventRecord(swept, stream)) || !ok(hipStreamWaitEvent(side, swept, 0)) ||
                !grad_x(t0, Tc, side, 0) || !ok(hipEventRecord(w_done, side2)) ||
                !ok(hipStreamWaitEvent(stream, w_done, 0)) ||
                !grad_w(0, t0, Tc, stream, wu, true) || !ok(hipEventRecord(x_done, side)) ||
                !ok(hipStreamWaitEvent(stream, x_done, 0)))
                return RNN_ERR_HIP;
        }
    }
    return RNN_OK;
}

}  // namespace host
}  // namespace rnn355
