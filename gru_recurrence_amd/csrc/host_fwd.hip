// host_fwd.hip -- host side of the forward: the input projection, the recurrence
// (serial or pipelined with the projection in one launch) and stacked layers.
#include "host.h"

namespace rnn355 {
namespace host {

bool gemm_shape_ok(int K, int N, rnn_dtype dt) {
    if (dt == RNN_BF16) return K % 8 == 0 && N % 8 == 0;
    return true;
}

// gx = x W + b.  With `wt` (bf16, K % 32 == 0) W is first transposed into
// wt and both operands stream k-major through the direct-to-LDS kernel;
// otherwise the register-staged kernel reads W as it is.
rnn_status input_proj(int M, int K, int N, rnn_dtype dt, const void *x, const void *W,
                      const float *b, float *gx, uint32_t *clear, hipStream_t s,
                      unsigned *ready, uint16_t *wt) {
    hipError_t e;
    if (dt == RNN_BF16 && wt && gemm_dma_ok(K)) {
        e = launch_transpose_bf16((const uint16_t *)W, wt, K, N, 1, s);
        if (e != hipSuccess) return RNN_ERR_HIP;
        GemmArgs g{};
        g.M = M; g.N = N; g.K = K;
        g.A = (const uint16_t *)x; g.lda = K;
        g.B = wt; g.ldb = K;
        g.bias = b; g.C = gx; g.ldc = N;
        g.clear_words = clear;
        g.ready = ready;
        e = launch_gemm_dma(g, 1, s);
    } else if (dt == RNN_BF16) {
        GemmArgs g{};
        g.M = M; g.N = N; g.K = K;
        g.A = (const uint16_t *)x; g.lda = K; g.strideA = 0;
        g.B = (const uint16_t *)W; g.ldb = N; g.strideB = 0;
        g.bias = b; g.C = gx; g.ldc = N; g.strideC = 0;
        g.accumulate = 0; g.clear_words = clear;
        g.ready = ready;
        e = launch_gemm_bf16(g, true, false, 1, s);
    } else {
        GemmF32Args g{};
        g.M = M; g.N = N; g.K = K;
        g.A = (const float *)x; g.sam = K; g.sak = 1; g.strideA = 0;
        g.B = (const float *)W; g.sbk = N; g.sbn = 1; g.strideB = 0;
        g.bias = b; g.C = gx; g.ldc = N; g.strideC = 0;
        g.accumulate = 0; g.clear_words = clear;
        e = launch_gemm_f32(g, 1, s);
    }
    return e == hipSuccess ? RNN_OK : RNN_ERR_HIP;
}

// rt: workspace region for R^T (rt_fwd_bytes), used by the Dh = 256 kernel (and, at
// Dh = 64 and 128, by the pipelined forward's recurrence).
// clear_status: zero the status word first (a stacked layer after the
// first keeps what earlier layers reported).
rnn_status rec_fwd(int cell, const rnn_dims *d, rnn_dtype dt, const float *gx, const void *R,
                   const float *h0, const float *c0, float *h_seq, float *c_seq, float *hT,
                   float *cT, void *ws, uint16_t *rt, hipStream_t s, bool clear_status) {
    const Choice ch = choose(cell, d, dt, device_cus());
    if (!ch.ok) return RNN_ERR_UNSUPPORTED;
    RecArgs a{};
    a.T = d->T; a.B = d->B; a.NH = d->NH; a.Dh = d->Dh;
    a.gx = gx;
    a.Rb = dt == RNN_BF16 ? (const uint16_t *)R : nullptr;
    a.Rf = dt == RNN_F32 ? (const float *)R : nullptr;
    a.h0 = h0; a.c0 = c0; a.h_seq = h_seq; a.c_seq = c_seq; a.hT = hT; a.cT = cT;
    hipError_t e;
    if (ch.use_wide) {
        // R^T per head; the same launch clears the status words
        const int G = gates_of_cell(cell);
        e = launch_transpose_bf16((const uint16_t *)R, rt, d->Dh, G * d->Dh, d->NH, s,
                                  clear_status ? (unsigned *)ws : nullptr, 64);
        if (e != hipSuccess) return RNN_ERR_HIP;
        a.BT = 1;
        e = launch_rec_wide(cell, ch.wide, a, rt, s);
    } else if (ch.use_mc) {
        a.BT = ch.mc.BT;
        McArgs m{};
        m.r = a;
        m.K = ch.mc.K; m.KS = ch.mc.ks; m.NB = ch.mc.nb;
        m.flag = (unsigned *)ws;
        m.xg = (unsigned long long *)((char *)ws + kHeader);
        m.spin_limit = spin_limit();
        if (mc_xcd_enabled() && mc_xcd_grouping(ch.mc.groups, ch.mc.grid)) {
            m.xcd_map = 1;
            m.xcc = (unsigned *)((char *)ws + kXccOffset);
        }
        e = launch_rec_mc(cell, ch.mc, m, s, clear_status);
    } else {
        // these kernels never wait, so nothing else writes the status word:
        // their workgroup 0 clears it, or a fresh workspace would report
        // what it held
        a.clear_word = clear_status ? (unsigned *)ws : nullptr;
        a.BT = ch.rec.BT;
        e = launch_rec_fwd(cell, ch.rec, a, dt == RNN_BF16, s);
    }
    return e == hipSuccess ? RNN_OK : RNN_ERR_HIP;
}

bool rec_supported(int cell, const rnn_dims *d, rnn_dtype dt) {
    return choose(cell, d, dt, device_cus()).ok;
}


// Whether the forward overlaps its two phases (see forward()): the one-CU
// recurrence at Dh = 128 or 64 must leave at least half the CUs free, and
// the projection (bf16, Din % 32 = 0) must take more than two waves of
// output tiles on those CUs, or more than one where the recurrence can start
// on a head start (head_start_panels) -- otherwise the first row panel is
// ready about when the whole projection would be, and the overlap only adds
// the cost of running the two side by side.
bool pipelined(const Choice &ch, const rnn_dims *d, rnn_dtype dt, int cus) {
    const int force = pipeline_override();
    if (dt != RNN_BF16 || ch.use_mc || ch.use_wide || ch.rec.kind != kRecMfma ||
        (d->Dh != 128 && d->Dh != 64) || !gemm_dma_ok(d->Din) || 2 * ch.rec.grid > cus ||
        force == 0 || gx_panels(d) < 2)
        return false;
    if (force == 1) return true;
    const int G = gates_of_cell(ch.cell);
    const long tiles = gx_panels(d) * (((long)d->NH * G * d->Dh + kGemmColTile - 1) / kGemmColTile);
    const long free = cus - ch.rec.grid;
    return tiles > 2L * free || (tiles > free && head_start_panels(ch, d, nullptr) > 0);
}

// Workgroups for an input projection that runs beside the recurrence: enough
// to produce row panels 2.5 times as fast as the recurrence consumes them (a
// 256x256 tile takes about 40 ns per unit of K on a busy chip; the recurrence
// spends kGemmRowTile / B steps of the plan's predicted step time on a panel),
// at most the `free` CUs, a multiple of 8 (whole XCD rounds).  More than
// needed only slows the recurrence beside them (measured on the headline
// shape: 112 workgroups 0.578 ms per fused call, 160 0.587).
// RNN355_FUSED_GEMM_WGS overrides (sweeps).
int proj_workgroups(const rnn_dims *d, const Choice &ch, int tiles_per_panel, int free) {
    const int cap = std::max(8, free / 8 * 8);
    const int want = env_int("RNN355_FUSED_GEMM_WGS");
    if (want >= 8) return std::min(want / 8 * 8, cap);
    const double panel_ns = (double)kGemmRowTile / d->B * std::max(ch.cand.ns_step, 1.0);
    const double need = 2.5 * 40.0 * d->Din * tiles_per_panel / panel_ns;
    return std::max(8, std::min(cap, (int)((need + 4) / 8) * 8));
}

// Projection workgroups after its first rounds (the pipelined forward's
// taper): the first rows1 rows -- two rounds of n_gemm workgroups' tiles
// and a panel more, whole panels -- run on all n_gemm, the rest on n2 of
// them, 1.25x the rate that keeps a panel ahead of the recurrence (as in
// proj_workgroups).  Fewer workgroups once the projection is ahead draw
// less power beside the latency-bound recurrence: headline forward 0.547-
// 0.552 against 0.557 ms per call.  RNN355_FUSED_TAPER=0: no taper.
void proj_taper(const rnn_dims *d, const Choice &ch, int tiles_per_panel, int n_gemm,
                long proj_panels, int *rows1, int *n2) {
    *rows1 = 0;
    *n2 = 0;
    if (env_int_or("RNN355_FUSED_TAPER", 1) == 0 || tiles_per_panel <= 0) return;
    const long p1 = (2L * n_gemm + tiles_per_panel - 1) / tiles_per_panel + 1;
    const double panel_ns = (double)kGemmRowTile / d->B * std::max(ch.cand.ns_step, 1.0);
    const double need = 40.0 * d->Din * tiles_per_panel / panel_ns;
    const int w = (int)(1.25 * need + 4) / 8 * 8;
    if (p1 >= proj_panels || w >= n_gemm || w < 8) return;
    *rows1 = (int)(p1 * kGemmRowTile);
    *n2 = w;
}

// Row panels of gx that the recurrence's workgroups of the pipelined
// forward compute themselves before their first step (RecArgs::hs_*), so
// that they start without waiting for the projection's first round of
// tiles (about 40 ns per unit of K per tile, as in proj_workgroups): the
// fewest panels whose head start and steps last that long at the plan's
// step time, or as many as fit -- whole steps per panel run (kGemmRowTile *
// P % B == 0), at
// most kHeadStartRows rows per workgroup, x 16-byte aligned, and a panel
// left to the projection.
// RNN355_HEAD_START=P asks for P panels instead (0: none), within the same
// limits.
int head_start_panels(const Choice &ch, const rnn_dims *d, const void *x) {
    const long panels = gx_panels(d);
    if ((x && ((uintptr_t)x & 15) != 0) || (d->Dh != 128 && d->Dh != 64)) return 0;
    auto fits = [&](int p) {
        if (p >= panels || ((long)kGemmRowTile * p) % d->B != 0) return false;
        const long rows = (long)kGemmRowTile * p / d->B * std::min(ch.rec.BT, d->B);
        return rows <= kHeadStartRows;
    };
    const char *e = getenv("RNN355_HEAD_START");
    if (e && e[0]) {
        const int want = atoi(e);
        int best = 0;
        for (int p = 1; p <= want && p < panels; ++p)
            if (fits(p)) best = p;
        return best;
    }
    // the head start itself takes ~22 ns per unit of K for one 32-row block,
    // ~28 for two (measured at Din = 768 beside the projection)
    const double first_round = 40.0 * d->Din, step = std::max(ch.cand.ns_step, 1.0);
    int best = 0;
    for (int p = 1; p < panels; ++p) {
        if (!fits(p)) continue;
        best = p;
        const long steps = (long)kGemmRowTile * p / d->B;
        const long rows = steps * std::min(ch.rec.BT, d->B);
        const double hs_ns = (rows > 32 ? 28.0 : 22.0) * d->Din;
        if (hs_ns + steps * step >= first_round) break;
    }
    return best;
}

// Forward = input projection + recurrence.  Pipelined (see pipelined()): one
// launch whose first workgroups compute the projection in time order and
// count finished 256-row panels of gx, while the recurrence's workgroups
// wait for the panels of their next steps (launch_fwd_fused).  Otherwise the
// projection, then the recurrence.  Results are bitwise the same.
rnn_status forward(int cell, const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                   const void *R, const float *b, const float *h0, const float *c0,
                   float *h_seq, float *c_seq, float *hT, float *cT, void *ws, hipStream_t s,
                   bool clear_status) {
    const int G = cell == kLSTM ? 4 : 3;
    const int N = d->NH * G * d->Dh, M = d->T * d->B;
    float *gx = (float *)((char *)ws + kHeader + xchg_bytes(d));
    unsigned *ready = (unsigned *)((char *)gx + gx_bytes(d, G));
    uint16_t *wt = (uint16_t *)((char *)ready + ready_bytes(d));
    const int cus = device_cus();
    const Choice ch = choose(cell, d, dt, cus);
    if (!ch.ok) return RNN_ERR_UNSUPPORTED;
    const long panels = gx_panels(d);
    if (pipelined(ch, d, dt, cus)) {
        auto ok = [](hipError_t e) { return e == hipSuccess; };
        // W^T for the k-major contraction; the same launch zeroes the status
        // words of the header and the panel counters
        // and R^T per head (16-byte fragment loads in the recurrence)
        uint16_t *rt = rt_fwd_bytes(d, dt, G) > 0 ? (uint16_t *)((char *)wt + wt_bytes(d, G))
                                                  : nullptr;
        if (!ok(launch_transpose_bf16((const uint16_t *)W, wt, d->Din, N, 1, s,
                                      clear_status ? (unsigned *)ws : nullptr, 64, ready, panels,
                                      rt ? (const uint16_t *)R : nullptr, rt, d->Dh, G * d->Dh,
                                      rt ? d->NH : 0)))
            return RNN_ERR_HIP;
        // the first hs panels come from the recurrence's workgroups
        const int hs = head_start_panels(ch, d, x);
        const long hs_rows = (long)hs * kGemmRowTile;
        GemmArgs g{};
        g.M = (int)(M - hs_rows); g.N = N; g.K = d->Din;
        g.A = (const uint16_t *)x + hs_rows * d->Din; g.lda = d->Din;
        g.B = wt; g.ldb = d->Din;
        g.bias = b; g.C = gx + hs_rows * N; g.ldc = N;
        g.ksplit = 1;
        g.ready = ready + hs;
        RecArgs a{};
        a.T = d->T; a.B = d->B; a.NH = d->NH; a.Dh = d->Dh; a.BT = ch.rec.BT;
        a.gx = gx;
        a.Rb = (const uint16_t *)R;
        a.Rt = rt;
        a.h0 = h0; a.c0 = c0; a.h_seq = h_seq; a.c_seq = c_seq; a.hT = hT; a.cT = cT;
        a.ready = ready;
        a.ready_target = (unsigned)((N + kGemmColTile - 1) / kGemmColTile);  // tiles per panel
        a.panels = (int)panels;
        a.flag = (unsigned *)ws;
        a.spin_limit = spin_limit();
        if (hs > 0) {
            a.hs_panels = hs;
            a.hs_steps = (int)(hs_rows / d->B);
            a.hs_K = d->Din;
            a.hs_x = (const uint16_t *)x;
            a.hs_wt = wt;
            a.hs_bias = b;
        }
        // projection workgroups by rate (proj_workgroups), at most one per tile
        const long tiles = (panels - hs) * a.ready_target;
        int n_gemm = proj_workgroups(d, ch, (int)a.ready_target, cus - ch.rec.grid);
        if (n_gemm > tiles) n_gemm = (int)tiles;
        if (n_gemm < 8) n_gemm = (int)std::min<long>(8, tiles);
        int rows1 = 0, n2 = 0;
        proj_taper(d, ch, (int)a.ready_target, n_gemm, panels - hs, &rows1, &n2);
        return ok(launch_fwd_fused(cell, ch.rec, a, g, n_gemm, s, rows1, n2)) ? RNN_OK
                                                                               : RNN_ERR_HIP;
    }
    rnn_status st = input_proj(M, d->Din, N, dt, x, W, b, gx,
                               clear_status ? (uint32_t *)ws : nullptr, s, nullptr, wt);
    if (st != RNN_OK) return st;
    uint16_t *rt = (uint16_t *)((char *)wt + wt_bytes(d, G));
    return rec_fwd(cell, d, dt, gx, R, h0, c0, h_seq, c_seq, hT, cT, ws, rt, s, clear_status);
}

// Stacked layers: layer l > 0 reads layer l-1's h_1..h_T (rounded to bf16
// in bf16 runs, as x is).
//
// Two layers at a time share one launch (launch_fwd_stack2) where the
// one-row MFMA recurrence at Dh = 128 leaves at least 32 CUs beside two
// copies of itself: layer l's projection runs first on the whole chip, then
// layer l's recurrence, layer l+1's projection (on the CUs left) and layer
// l+1's recurrence run side by side, each 256-row tile of the projection
// starting once layer l has produced its steps.  Otherwise the layers run
// in turn.  RNN355_STACK_OVERLAP=0 turns the overlap off.  Both ways give
// the same bits: the same kernels sum in the same order.
int stack_overlap_wgs(const Choice &ch, const rnn_dims *dh, rnn_dtype dt, int cus) {
    const char *e = getenv("RNN355_STACK_OVERLAP");
    if (e && e[0] == '0') return 0;
    if (dt != RNN_BF16 || !ch.ok || ch.use_mc || ch.use_wide || ch.rec.kind != kRecMfma ||
        ch.rec.upt != 1 || ch.rec.BT != 1 || dh->Dh != 128 || !gemm_dma_ok(dh->Din))
        return 0;
    const int free = cus - 2 * ch.rec.grid;
    if (free < 32) return 0;
    const int G = gates_of_cell(ch.cell);
    const long tiles = gx_panels(dh) * (((long)dh->NH * G * dh->Dh + kGemmColTile - 1) /
                                        kGemmColTile);
    return (int)std::min<long>(free / 8 * 8, tiles);
}

StackLayout stack_layout(const rnn_dims *d, int G, rnn_dtype dt) {
    StackLayout L{};
    rnn_dims dm = *d;
    const int H = d->NH * d->Dh;
    if (H > dm.Din) dm.Din = H;
    const size_t seq = (size_t)d->T * d->B * H;
    const bool bf = dt == RNN_BF16;
    L.fwd = align_up(kHeader + xchg_bytes(&dm) + gx_bytes(&dm, G) + ready_bytes(&dm) +
                     wt_bytes(&dm, G) + rt_fwd_bytes(&dm, dt, G));
    L.hbuf = L.fwd;
    L.hbf = L.hbuf + 2 * align_up(sizeof(float) * seq);
    L.gx2 = L.hbf + (bf ? 2 * align_up(sizeof(uint16_t) * seq) : 0);
    L.done = L.gx2 + (bf ? gx_bytes(&dm, G) : 0);
    L.total = L.done + (bf ? align_up(sizeof(unsigned) * (size_t)d->T) : 0);
    return L;
}

rnn_status forward_stack(int cell, const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                         const void *const *W, const void *const *R, const float *const *b,
                         const float *h0, const float *c0, float *h_seq, float *c_seq,
                         float *hT, float *cT, void *ws, hipStream_t s) {
    const int G = gates_of_cell(cell), H = d->NH * d->Dh, N = d->NH * G * d->Dh;
    const long BH = (long)d->B * H, seq = (long)d->T * BH;
    const StackLayout SL = stack_layout(d, G, dt);
    char *base = (char *)ws;
    float *hb[2] = {(float *)(base + SL.hbuf),
                    (float *)(base + SL.hbuf + align_up(sizeof(float) * seq))};
    uint16_t *hbf[2] = {nullptr, nullptr};
    if (dt == RNN_BF16) {
        hbf[0] = (uint16_t *)(base + SL.hbf);
        hbf[1] = (uint16_t *)(base + SL.hbf + align_up(sizeof(uint16_t) * seq));
    }
    // the forward workspace's regions (as forward() lays them out)
    float *gx = (float *)(base + kHeader + xchg_bytes(d));
    unsigned *ready = (unsigned *)((char *)gx + gx_bytes(d, G));
    uint16_t *wt = (uint16_t *)((char *)ready + ready_bytes(d));
    float *gx2 = (float *)(base + SL.gx2);
    unsigned *done = (unsigned *)(base + SL.done);

    rnn_dims dh = *d;
    dh.Din = H;
    const int cus = device_cus();
    const Choice chh = choose(cell, &dh, dt, cus);
    const int n_gemm = stack_overlap_wgs(chh, &dh, dt, cus);
    const long panels = gx_panels(d);
    const int M = d->T * d->B;
    auto hip_ok = [](hipError_t e) { return e == hipSuccess; };

    const void *xin = x;
    for (int l = 0; l < L;) {
        rnn_dims dl = *d;
        if (l > 0) dl.Din = H;
        const bool first = l == 0;
        const float *h0l = h0 ? h0 + l * BH : nullptr, *c0l = c0 ? c0 + l * BH : nullptr;
        if (n_gemm > 0 && l + 1 < L) {
            const bool last = l + 2 == L;
            // layer l's projection on the whole chip
            rnn_status st = input_proj(M, dl.Din, N, dt, xin, W[l], b ? b[l] : nullptr, gx,
                                       first ? (uint32_t *)ws : nullptr, s, nullptr, wt);
            if (st != RNN_OK) return st;
            // W[l+1]^T; the same launch zeroes the step and panel counters
            if (!hip_ok(launch_transpose_bf16((const uint16_t *)W[l + 1], wt, H, N, 1, s, done,
                                              d->T, ready, panels)))
                return RNN_ERR_HIP;
            RecArgs a0{}, a1{};
            a0.T = a1.T = d->T; a0.B = a1.B = d->B; a0.NH = a1.NH = d->NH;
            a0.Dh = a1.Dh = d->Dh; a0.BT = a1.BT = 1;
            a0.flag = a1.flag = (unsigned *)ws;
            a0.spin_limit = a1.spin_limit = spin_limit();
            a0.gx = gx;
            a0.Rb = (const uint16_t *)R[l];
            a0.h0 = h0l; a0.c0 = c0l;
            a0.hT = hT + l * BH; a0.cT = cT ? cT + l * BH : nullptr;
            a1.gx = gx2;
            a1.Rb = (const uint16_t *)R[l + 1];
            a1.h0 = h0 ? h0 + (l + 1) * BH : nullptr;
            a1.c0 = c0 ? c0 + (l + 1) * BH : nullptr;
            a1.h_seq = last ? h_seq : nullptr;
            a1.c_seq = last ? c_seq : nullptr;
            a1.hT = hT + (l + 1) * BH; a1.cT = cT ? cT + (l + 1) * BH : nullptr;
            a1.ready = ready;
            a1.ready_target = (unsigned)((N + kGemmColTile - 1) / kGemmColTile);
            a1.panels = (int)panels;
            GemmArgs g{};
            g.M = M; g.N = N; g.K = H;
            g.A = hbf[0]; g.lda = H;
            g.B = wt; g.ldb = H;
            g.bias = b ? b[l + 1] : nullptr;
            g.C = gx2; g.ldc = N;
            g.ksplit = 1;
            g.ready = ready;
            StackSync y{};
            y.h_bf0 = hbf[0];
            y.h_bf1 = last ? nullptr : hbf[1];
            y.done = done;
            y.rec_grid = chh.rec.grid;
            y.done_target = (unsigned)chh.rec.grid;
            y.n_gemm = n_gemm;
            if (!hip_ok(launch_fwd_stack2(cell, chh.rec, a0, a1, g, y, s))) return RNN_ERR_HIP;
            xin = hbf[1];
            l += 2;
            continue;
        }
        const bool last = l == L - 1;
        float *hs = last ? h_seq : hb[l & 1];
        float *cs = last ? c_seq : nullptr;
        rnn_status st = forward(cell, &dl, dt, xin, W[l], R[l], b ? b[l] : nullptr, h0l, c0l, hs,
                                cs, hT + l * BH, cT ? cT + l * BH : nullptr, ws, s, first);
        if (st != RNN_OK) return st;
        if (!last) {
            if (hbf[0]) {
                if (!hip_ok(launch_hprev_bf16(nullptr, hs, hbf[0], 0, seq, s))) return RNN_ERR_HIP;
                xin = hbf[0];
            } else {
                xin = hs;
            }
        }
        ++l;
    }
    return RNN_OK;
}

}  // namespace host
}  // namespace rnn355
