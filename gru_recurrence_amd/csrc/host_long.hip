// host_long.hip -- long sequences: the forward in chunks of steps and the
// checkpointed backward.
#include "host.h"

namespace rnn355 {
namespace host {

// Long sequences in chunks of `chunk` steps (blog.hotdry.top 2025-09-21,
// the list of framework-level optimisations, third item: memory for long
// sequences).  The recurrence runs chunk after chunk on the caller's
// stream, each from the previous chunk's final state (the same kernels as
// an unchunked call, hence the same bits); the input projection of chunk
// k+2 runs on a second stream into the gx slot chunk k read, once chunk k's
// recurrence is done, so each chunk's projection is ready before its
// recurrence starts and runs beside the previous one, on the compute units
// that recurrence leaves.  Workspace: two gx slots of `chunk` steps in
// place of T, W^T, R^T, the exchange slots and the state between chunks.
ChunkLayout chunk_layout(const rnn_dims *d, int chunk, int G, rnn_dtype dt) {
    ChunkLayout L{};
    rnn_dims dc = *d;
    dc.T = std::min(chunk, d->T);
    const size_t bh = align_up(sizeof(float) * (size_t)d->B * d->NH * d->Dh);
    L.gx0 = kHeader + xchg_bytes(&dc);
    L.gx1 = L.gx0 + gx_bytes(&dc, G);
    L.wt = L.gx1 + gx_bytes(&dc, G);
    L.rt = L.wt + wt_bytes(d, G);
    L.st = L.rt + rt_fwd_bytes(d, dt, G);
    L.total = L.st + 4 * bh;
    return L;
}

// Fewest free compute units for which a chunk's projection runs beside the
// previous chunk's recurrence.
constexpr int kChunkMinFreeCus = 64;

rnn_status forward_chunked(int cell, const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                           const void *W, const void *R, const float *b, const float *h0,
                           const float *c0, float *h_seq, float *c_seq, float *hT, float *cT,
                           float *h_ck, float *c_ck, void *ws, hipStream_t s) {
    const bool lstm = cell == kLSTM;
    const int G = gates_of_cell(cell), T = d->T, B = d->B, Din = d->Din;
    const int H = d->NH * d->Dh, N = d->NH * G * d->Dh;
    const long BH = (long)B * H;
    chunk = std::min(chunk, T);
    const int nck = (T + chunk - 1) / chunk;
    const ChunkLayout CL = chunk_layout(d, chunk, G, dt);
    char *base = (char *)ws;
    float *gx[2] = {(float *)(base + CL.gx0), (float *)(base + CL.gx1)};
    uint16_t *wt = (uint16_t *)(base + CL.wt), *rt = (uint16_t *)(base + CL.rt);
    const size_t bh = align_up(sizeof(float) * (size_t)BH);
    float *sth[2] = {(float *)(base + CL.st), (float *)(base + CL.st + bh)};
    float *stc[2] = {(float *)(base + CL.st + 2 * bh), (float *)(base + CL.st + 3 * bh)};
    const size_t esz = dt == RNN_BF16 ? 2 : 4;

    const int cus = device_cus();
    rnn_dims dc = *d;
    dc.T = chunk;
    const Choice ch = choose(cell, &dc, dt, cus);
    if (!ch.ok) return RNN_ERR_UNSUPPORTED;
    const int rec_grid = ch.use_wide ? ch.wide.grid : ch.use_mc ? ch.mc.grid : ch.rec.grid;
    const bool dma = dt == RNN_BF16 && gemm_dma_ok(Din);
    // the projection runs beside the recurrence on the CUs it leaves; where
    // it leaves few (the multi-CU plans take them all), a capped projection
    // would take longer than the chunk it feeds, so every chunk's projection
    // runs on the whole chip, in order on the caller's stream
    const bool beside = cus - rec_grid >= kChunkMinFreeCus;
    // (all the free CUs: measured on the T = 8192 headline shape in chunks of
    // 1024, 160 workgroups 4.29 ms, 112 4.33, 64 4.44 -- unlike the fused
    // launch, a chunk's projection is done long before the chunk it feeds)
    const int gemm_wg = beside ? (cus - rec_grid) / 8 * 8 : 0;
    hipStream_t s2 = beside ? side_stream() : s;  // s may be the null stream
    CallEvents ev;
    if ((beside && !s2) || !ev.ok) return RNN_ERR_HIP;
    hipEvent_t fork = ev.e[0], eg[2] = {ev.e[1], ev.e[2]}, er[2] = {ev.e[3], ev.e[4]};
    auto ok = [](hipError_t e) { return e == hipSuccess; };

    auto proj = [&](int k) -> rnn_status {
        const int t0 = k * chunk, tk = std::min(chunk, T - t0);
        const void *xk = (const char *)x + (size_t)t0 * B * Din * esz;
        if (dma) {
            GemmArgs g{};
            g.M = tk * B; g.N = N; g.K = Din;
            g.A = (const uint16_t *)xk; g.lda = Din;
            g.B = wt; g.ldb = Din;
            g.bias = b; g.C = gx[k & 1]; g.ldc = N;
            g.ksplit = 1;
            return ok(launch_gemm_dma(g, 1, s2, gemm_wg)) ? RNN_OK : RNN_ERR_HIP;
        }
        return input_proj(tk * B, Din, N, dt, xk, W, b, gx[k & 1],
                          k == 0 ? (uint32_t *)ws : nullptr, s2);
    };
    // fork: the second stream starts after what the caller queued
    if (!ok(hipEventRecord(fork, s)) || !ok(hipStreamWaitEvent(s2, fork, 0))) return RNN_ERR_HIP;
    // W^T once; the same launch zeroes the status words
    if (dma && !ok(launch_transpose_bf16((const uint16_t *)W, wt, Din, N, 1, s2, (unsigned *)ws, 64)))
        return RNN_ERR_HIP;
    for (int k = 0; k < std::min(2, nck); ++k) {
        const rnn_status st = proj(k);
        if (st != RNN_OK) return st;
        if (!ok(hipEventRecord(eg[k & 1], s2))) return RNN_ERR_HIP;
    }
    for (int k = 0; k < nck; ++k) {
        const int t0 = k * chunk;
        rnn_dims dk = *d;
        dk.T = std::min(chunk, T - t0);
        const bool last = k == nck - 1;
        const float *hin = k == 0 ? h0 : (h_ck ? h_ck + (k - 1) * BH : sth[(k - 1) & 1]);
        const float *cin = !lstm ? nullptr
                                 : k == 0 ? c0 : (c_ck ? c_ck + (k - 1) * BH : stc[(k - 1) & 1]);
        float *hout = last ? hT : (h_ck ? h_ck + k * BH : sth[k & 1]);
        float *cout = !lstm ? nullptr : last ? cT : (c_ck ? c_ck + k * BH : stc[k & 1]);
        if (!ok(hipStreamWaitEvent(s, eg[k & 1], 0))) return RNN_ERR_HIP;
        const rnn_status st = rec_fwd(cell, &dk, dt, gx[k & 1], R, hin, cin,
                                      h_seq ? h_seq + t0 * BH : nullptr,
                                      c_seq ? c_seq + t0 * BH : nullptr, hout, cout, ws, rt, s,
                                      false);
        if (st != RNN_OK) return st;
        if (!ok(hipEventRecord(er[k & 1], s))) return RNN_ERR_HIP;
        if (k + 2 < nck) {
            if (!ok(hipStreamWaitEvent(s2, er[k & 1], 0))) return RNN_ERR_HIP;
            const rnn_status sp = proj(k + 2);
            if (sp != RNN_OK) return sp;
            if (!ok(hipEventRecord(eg[k & 1], s2))) return RNN_ERR_HIP;
        }
    }
    if (h_ck) {
        const size_t bytes = sizeof(float) * (size_t)BH;
        if (!ok(hipMemcpyAsync(h_ck + (nck - 1) * BH, hT, bytes, hipMemcpyDeviceToDevice, s)))
            return RNN_ERR_HIP;
        if (lstm && !ok(hipMemcpyAsync(c_ck + (nck - 1) * BH, cT, bytes, hipMemcpyDeviceToDevice, s)))
            return RNN_ERR_HIP;
    }
    return RNN_OK;
}

// Checkpointed backpropagation through time (blog.hotdry.top 2025-09-21,
// the list of framework-level optimisations, third item: checkpointing
// trades compute for memory).  Segments of `chunk` steps from the last to
// the first: the segment's h and c are recomputed by the forward from the
// state before it (h0/c0, else the checkpoint of the previous segment),
// then BPTT runs over the segment with the carries dh, dc that the later
// segment left, adding to dW, dR and db.  Workspace: one forward or
// backward workspace of `chunk` steps, the segment's h and c, the carries.
CkptLayout ckpt_layout(const rnn_dims *d, int chunk, int G, rnn_dtype dt) {
    CkptLayout L{};
    rnn_dims dc = *d;
    dc.T = std::min(chunk, d->T);
    const bool lstm = G == 4;
    const size_t work = std::max(rnn_workspace_size(lstm ? RNN_OP_FWD_LSTM : RNN_OP_FWD_GRU, &dc, dt),
                                 rnn_workspace_size(lstm ? RNN_OP_BWD_LSTM : RNN_OP_BWD_GRU, &dc, dt));
    const size_t seg = align_up(sizeof(float) * (size_t)dc.T * d->B * d->NH * d->Dh);
    const size_t bh = align_up(sizeof(float) * (size_t)d->B * d->NH * d->Dh);
    L.hseg = align_up(work);
    L.cseg = L.hseg + seg;
    L.car = L.cseg + (lstm ? seg : 0);
    L.scr = L.car + 4 * bh;
    L.total = L.scr + 2 * bh;
    return L;
}

rnn_status backward_ckpt(int cell, const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                         const void *W, const void *R, const float *b, const float *h0,
                         const float *c0, const float *h_ck, const float *c_ck,
                         const float *dh_seq, const float *dhT, const float *dcT, float *dx,
                         float *dW, float *dR, float *db, float *dh0, float *dc0, void *ws,
                         hipStream_t s) {
    const bool lstm = cell == kLSTM;
    const int G = gates_of_cell(cell), T = d->T, B = d->B, Din = d->Din;
    const long BH = (long)B * d->NH * d->Dh;
    chunk = std::min(chunk, T);
    const int nseg = (T + chunk - 1) / chunk;
    const CkptLayout CL = ckpt_layout(d, chunk, G, dt);
    char *base = (char *)ws;
    float *hseg = (float *)(base + CL.hseg), *cseg = lstm ? (float *)(base + CL.cseg) : nullptr;
    const size_t bh = align_up(sizeof(float) * (size_t)BH);
    float *car_h[2] = {(float *)(base + CL.car), (float *)(base + CL.car + bh)};
    float *car_c[2] = {(float *)(base + CL.car + 2 * bh), (float *)(base + CL.car + 3 * bh)};
    float *scr_h = (float *)(base + CL.scr), *scr_c = (float *)(base + CL.scr + bh);
    for (int j = nseg - 1; j >= 0; --j) {
        const int t0 = j * chunk;
        rnn_dims dj = *d;
        dj.T = std::min(chunk, T - t0);
        const bool later = j == nseg - 1;  // the last segment, run first
        const float *hin = j == 0 ? h0 : h_ck + (j - 1) * BH;
        const float *cin = !lstm ? nullptr : j == 0 ? c0 : c_ck + (j - 1) * BH;
        const size_t esz = dt == RNN_BF16 ? sizeof(uint16_t) : sizeof(float);
        const void *xj = (const char *)x + (size_t)t0 * B * Din * esz;
        rnn_status st = forward(cell, &dj, dt, xj, W, R, b, hin, cin, hseg, cseg, scr_h,
                                lstm ? scr_c : nullptr, ws, s, later);
        if (st != RNN_OK) return st;
        const float *dhTj = later ? dhT : car_h[(j + 1) & 1];
        const float *dcTj = !lstm ? nullptr : later ? dcT : car_c[(j + 1) & 1];
        float *dh0j = j == 0 ? dh0 : car_h[j & 1];
        float *dc0j = !lstm ? nullptr : j == 0 ? dc0 : car_c[j & 1];
        st = backward(cell, &dj, dt, xj, W, R, b, hin, cin, hseg, cseg, dh_seq + t0 * BH, dhTj,
                      dcTj, dx + (size_t)t0 * B * Din, dW, dR, db, dh0j, dc0j, ws, CL.hseg, s,
                      !later, false);
        if (st != RNN_OK) return st;
    }
    return RNN_OK;
}

}  // namespace host
}  // namespace rnn355
