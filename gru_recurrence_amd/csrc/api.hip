// api.hip -- host side of the librnn355 C ABI (include/rnn355.h): argument
// validation, workspace layout, kernel plans and stream-ordered launches.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <algorithm>
#include <mutex>

#include "../../include/rnn355.h"
#include "common.h"
#include "kernels.h"

using namespace rnn355;

namespace {

// Workspace: [0, kHeader) status word (word 0) and the multi-CU kernel's
// XCD table (from byte kXccOffset), then the h exchange slots
// of the multi-CU kernel, then the operation's own regions, each 256-byte
// aligned.
constexpr size_t kHeader = 4096;
// dR = h_{t-1}^T dS per head has few output tiles (Dh x G Dh each) and a tall
// K (T B): up to 16 K slices so that it fills the chip (B16 NH4 Dh256: 256
// workgroups instead of 128)
constexpr int kMaxSplitKdR = 16;
// header words [256, 1024): the multi-CU kernel's table of workgroup XCDs
constexpr size_t kXccOffset = 1024;
constexpr int kXccWords = (int)((kHeader - kXccOffset) / sizeof(unsigned));
static_assert(kXccWords >= kMcXcdMaxGrid, "the XCD table holds one word per workgroup");
constexpr int kMaxLayers = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

bool dims_ok(const rnn_dims *d) {
    return d && d->T > 0 && d->B > 0 && d->Din > 0 && d->NH > 0 && d->Dh > 0 &&
           (long)d->NH * d->Dh <= (1L << 24) && (long)d->T * d->B <= (1L << 30);
}

bool dtype_ok(rnn_dtype dt) { return dt == RNN_F32 || dt == RNN_BF16; }

int gates_of_op(rnn_op op) {
    return (op == RNN_OP_FWD_GRU || op == RNN_OP_BWD_GRU || op == RNN_OP_REC_GRU) ? 3 : 4;
}

int cell_of_op(rnn_op op) { return gates_of_op(op) == 4 ? kLSTM : kGRU; }

int gates_of_cell(int cell) { return cell == kLSTM ? 4 : 3; }

// Exchange slots: [groups][2][BT][Dh/2] 8-byte words with groups =
// NH * ceil(B/BT) and BT <= 16, so groups * BT <= NH * (B + 15).
size_t xchg_bytes(const rnn_dims *d) {
    return align_up(2u * 8u * (size_t)d->NH * (d->B + 15) * ((d->Dh + 1) / 2));
}

size_t gx_bytes(const rnn_dims *d, int G) {
    return align_up(sizeof(float) * (size_t)d->T * d->B * d->NH * G * d->Dh);
}

// Row-panel counters of the pipelined forward (one word per kGemmRowTile
// rows of gx), after gx in the forward workspace.
long gx_panels(const rnn_dims *d) {
    return ((long)d->T * d->B + kGemmRowTile - 1) / kGemmRowTile;
}
size_t ready_bytes(const rnn_dims *d) { return align_up(sizeof(unsigned) * (size_t)gx_panels(d)); }

// W staged transposed ([N][Din] bf16) for the k-major contraction.
size_t wt_bytes(const rnn_dims *d, int G) {
    return align_up(sizeof(uint16_t) * (size_t)d->Din * d->NH * G * d->Dh);
}

// R staged transposed per head ([NH][G*Dh][Dh] bf16) for the Dh = 256
// one-CU recurrence; sized for every bf16 shape with Dh = 256.
size_t rt_fwd_bytes(const rnn_dims *d, rnn_dtype dt, int G) {
    if (dt != RNN_BF16 || (d->Dh != 256 && d->Dh != 128 && d->Dh != 64)) return 0;
    return align_up(sizeof(uint16_t) * (size_t)d->NH * G * d->Dh * d->Dh);
}

// Backward workspace after the header: the exchange slots of the sweep, the
// recomputed pre-activations A (LSTM: Gx + h_{t-1} R; GRU: Gx alone) and the
// GRU's recurrent sums S (f32), the gate-input gradients dA and the GRU's
// recurrent-sum gradients dS (bf16), h_{t-1} (bf16), the per-batch-tile bias
// partials (per chunk of the sweep), split-K partials, W^T, R^T per head and
// the carries between chunks of the sweep.
// The reverse sweep runs in up to kBwdChunks time chunks (see backward()):
// bias partials for each, and the carries between chunks.
constexpr int kBwdChunks = 4;
constexpr int kBwdMinChunk = 128;  // shortest chunk (steps)
struct BwdLayout {
    size_t xchg, A, S, dA, dS, hprev, dbp, part, wt, rt, car, total;
};
BwdLayout bwd_layout(const rnn_dims *d, int G) {
    BwdLayout L{};
    const bool gru = G == 3;
    const size_t TB = (size_t)d->T * d->B, N = (size_t)d->NH * G * d->Dh;
    const size_t H = (size_t)d->NH * d->Dh;
    size_t off = 0;
    L.xchg = off; off += align_up(8u * (size_t)d->NH * (d->B + 15) * 2 * ((size_t)G * d->Dh / 2));
    L.A = off;    off += align_up(sizeof(float) * TB * N);
    L.S = off;    off += gru ? align_up(sizeof(float) * TB * N) : 0;
    L.dA = off;   off += align_up(sizeof(uint16_t) * TB * N);
    L.dS = off;   off += gru ? align_up(sizeof(uint16_t) * TB * N) : 0;
    L.hprev = off; off += align_up(sizeof(uint16_t) * TB * H);
    L.dbp = off;  off += align_up(sizeof(float) * (size_t)kBwdChunks * d->B * N);
    // split-K partials of the dW and dR contractions (used one after the other)
    const size_t pw = gemm_partial_bytes(d->Din, (int)N, 1, kMaxSplitK);
    const size_t pr = gemm_partial_bytes(d->Dh, G * d->Dh, d->NH, kMaxSplitKdR);
    L.part = off; off += align_up(pw > pr ? pw : pr);
    L.wt = off;   off += wt_bytes(d, G);                                     // W^T [N][Din]
    L.rt = off;   off += align_up(sizeof(uint16_t) * (size_t)d->NH * G * d->Dh * d->Dh);  // R^T per head
    L.car = off;  off += 4 * align_up(sizeof(float) * H * d->B);  // dh, dc carries, two of each
    L.total = off;
    return L;
}

// Float32 backward workspace after the header: pre-activations A (LSTM:
// with the recurrent part; GRU: x W + b) and the GRU's recurrent sums S,
// the gate-input gradients dA and the GRU's recurrent-sum gradients dS, and
// h_{t-1}, all float32.
struct BwdF32Layout {
    size_t A, S, dA, dS, hprev, total;
};
BwdF32Layout bwd_f32_layout(const rnn_dims *d, int G) {
    BwdF32Layout L{};
    const bool gru = G == 3;
    const size_t TB = (size_t)d->T * d->B, N = (size_t)d->NH * G * d->Dh;
    const size_t H = (size_t)d->NH * d->Dh;
    size_t off = 0;
    L.A = off;     off += align_up(sizeof(float) * TB * N);
    L.S = off;     off += gru ? align_up(sizeof(float) * TB * N) : 0;
    L.dA = off;    off += align_up(sizeof(float) * TB * N);
    L.dS = off;    off += gru ? align_up(sizeof(float) * TB * N) : 0;
    L.hprev = off; off += align_up(sizeof(float) * TB * H);
    L.total = off;
    return L;
}

// out == nullptr: clear the status word; otherwise copy it to out.
__global__ void status_word_kernel(unsigned *word, unsigned *out) {
    if (threadIdx.x == 0) {
        if (out) out[0] = word[0];
        else word[0] = 0u;
    }
}

// Compute-unit count of the current device, cached per device.
int device_cus() {
    static std::mutex mu;
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

// Plan overrides for tile sweeps (rows per workgroup, workgroups per head).
int env_int(const char *name) {
    const char *e = getenv(name);
    return e ? atoi(e) : 0;
}
int bt_override() { return env_int("RNN355_REC_BT"); }
int env_int_or(const char *name, int dflt) {
    const char *e = getenv(name);
    return e ? atoi(e) : dflt;
}
// RNN355_MC_XCD=0: the multi-CU kernel numbers its workgroups group by
// group and exchanges through memory even where a group could share an L2.
bool mc_xcd_enabled() {
    const char *e = getenv("RNN355_MC_XCD");
    return !e || atoi(e) != 0;
}
// RNN355_PIPELINE=0 runs the forward's two phases one after the other;
// =1 overlaps them wherever that is safe, also where the plan would not.
int pipeline_override() {
    const char *e = getenv("RNN355_PIPELINE");
    return !e || !e[0] ? -1 : e[0] == '0' ? 0 : 1;
}
int k_override() { return env_int("RNN355_REC_K"); }
// RNN355_REC_KCW=4|8: k-chunks per wave of the multi-CU kernel.
int kcw_override() { return env_int("RNN355_REC_KCW"); }
// RNN355_REC_WIDE=0 serves Dh = 256 with the multi-CU kernel instead of the
// one-CU kernel with split R.
bool wide_enabled() {
    const char *e = getenv("RNN355_REC_WIDE");
    return !(e && e[0] == '0');
}
// Polls of a multi-CU step wait before it is declared lost (~4 s by default;
// tests lower it to force the time-out path).
unsigned spin_limit() {
    const int v = env_int("RNN355_SPIN_LIMIT");
    return v > 0 ? (unsigned)v : (1u << 22);
}

// Which recurrent kernel serves a shape, and with which tiling: the fastest
// feasible plan of the constraint search (plan_search.hip) over the
// one-CU MFMA kernel (bf16, Dh in {32, 64, 128}), the one-CU kernel with R
// split over registers and LDS (bf16, Dh = 256), the multi-CU kernel (bf16,
// Dh >= 256, Dh % 128 == 0) and the LDS kernel (R of at most 64 KiB in
// f32).  The environment overrides (RNN355_REC_BT, _K, _KCW, _WIDE=0) fix
// or exclude variables of the search.
struct Choice {
    int cell;
    RecPlan rec;
    WidePlan wide;
    McPlan mc;
    PlanCand cand;
    bool use_wide;
    bool use_mc;
    bool ok;
};

Choice choose(int cell, const rnn_dims *d, rnn_dtype dt, int num_cu) {
    Choice c{};
    c.cell = cell;
    const bool bf16 = dt == RNN_BF16;
    const PlanFix fix{bt_override(), k_override(), kcw_override(), !wide_enabled(),
                      !mc_xcd_enabled()};
    static thread_local PlanCand buf[kPlanMaxCands];
    int best = -1;
    plan_search(cell, d->T, d->B, d->NH, d->Dh, bf16, num_cu, fix, buf, kPlanMaxCands, &best);
    if (best < 0) return c;
    const PlanCand &p = buf[best];
    c.cand = p;
    switch (p.family) {
        case kFamResident:
            c.rec = plan_rec(cell, d->T, d->B, d->NH, d->Dh, true, num_cu, p.BT);
            c.ok = c.rec.kind == kRecMfma && c.rec.BT == p.BT;
            break;
        case kFamLds:
            // the LDS kernel's geometry (the launcher picks its bf16 or f32 variant)
            c.rec = plan_rec(cell, d->T, d->B, d->NH, d->Dh, false, num_cu, p.BT);
            c.ok = c.rec.kind == kRecSimple && c.rec.BT == p.BT;
            break;
        case kFamWide:
            c.wide = plan_wide(cell, d->B, d->NH, d->Dh, bf16);
            c.use_wide = c.ok = c.wide.ok != 0;
            break;
        case kFamMultiCu:
            c.mc = plan_mc(cell, d->B, d->NH, d->Dh, num_cu, p.BT, p.K, p.kcw);
            c.use_mc = c.ok = c.mc.ok && c.mc.K == p.K && c.mc.BT == p.BT && c.mc.kcw == p.kcw;
            break;
    }
    return c;
}

bool gemm_shape_ok(int K, int N, rnn_dtype dt) {
    if (dt == RNN_BF16) return K % 8 == 0 && N % 8 == 0;
    return true;
}

// gx = x W + b.  With `wt` (bf16, K % 32 == 0) W is first transposed into
// wt and both operands stream k-major through the direct-to-LDS kernel;
// otherwise the register-staged kernel reads W as it is.
rnn_status input_proj(int M, int K, int N, rnn_dtype dt, const void *x, const void *W,
                      const float *b, float *gx, uint32_t *clear, hipStream_t s,
                      unsigned *ready = nullptr, uint16_t *wt = nullptr) {
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
                   float *cT, void *ws, uint16_t *rt, hipStream_t s, bool clear_status = true) {
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

int head_start_panels(const Choice &ch, const rnn_dims *d, const void *x);

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
                   bool clear_status = true) {
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

// Workspace: one forward workspace sized for the larger input width, two
// float32 sequence buffers (layers that run in turn), two bf16 sequence
// buffers (layer inputs), a second gx and the step counters (overlapped
// pairs).
struct StackLayout {
    size_t fwd, hbuf, hbf, gx2, done, total;
};
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

// Streams of the current device (default priority) for work that runs
// beside the caller's stream, two per device (i = 0, 1); created on first use.
hipStream_t side_stream(int i = 0) {
    static std::mutex mu;
    static hipStream_t st[64][2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || i < 0 || i > 1) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!st[dev][i] && hipStreamCreateWithFlags(&st[dev][i], hipStreamNonBlocking) != hipSuccess)
        st[dev][i] = nullptr;
    return st[dev][i];
}

// Events of one call, destroyed when the call returns (the runtime keeps
// a recorded event alive until its work is done).
struct CallEvents {
    hipEvent_t e[kBwdChunks + 3] = {};
    bool ok = true;
    CallEvents() {
        for (hipEvent_t &v : e)
            if (hipEventCreateWithFlags(&v, hipEventDisableTiming) != hipSuccess) ok = false;
    }
    ~CallEvents() {
        for (hipEvent_t v : e)
            if (v) (void)hipEventDestroy(v);
    }
};

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

rnn_status backward(int cell, const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                    const void *R, const float *b, const float *h0, const float *c0,
                    const float *h_seq, const float *c_seq, const float *dh_seq,
                    const float *dhT, const float *dcT, float *dx, float *dW, float *dR,
                    float *db, float *dh0, float *dc0, void *ws, size_t ws_bytes,
                    hipStream_t stream, bool accumulate = false, bool clear_status = true) {
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
    // registers and LDS; otherwise the exchange-based sweep
    const WidePlan pw = wide_enabled() ? plan_wide(cell, B, NH, Dh, true) : WidePlan{};
    const BwdPlan p = pw.ok ? BwdPlan{} : plan_bwd(cell, B, NH, Dh, device_cus(), bt_override(),
                                                   k_override());
    if (!pw.ok && !p.ok) return RNN_ERR_UNSUPPORTED;
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
    const bool two = pw.ok && env_int_or("RNN355_BWD_WIDE2", 1) != 0 && mc_xcd_enabled() &&
                     mc_xcd_grouping(NH * B, 2 * NH * B) && 2 * NH * B <= device_cus();
    const int cus = device_cus();
    const int sweep_grid = two ? 2 * NH * B : pw.ok ? pw.grid : p.grid;
    const int free_cus = (cus - sweep_grid) / 8 * 8;
    int starts[kBwdChunks + 1];
    const int nch = free_cus >= 64 && env_int_or("RNN355_BWD_OVERLAP", 1) != 0
                        ? bwd_chunk_starts(T, starts)
                        : 1;
    // dx on one stream, dW, dR and db on the other, each on half the free units
    hipStream_t side = nch > 1 ? side_stream(0) : nullptr, side2 = nch > 1 ? side_stream(1) : nullptr;
    CallEvents ev;
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
struct ChunkLayout {
    size_t gx0, gx1, wt, rt, st, total;
};
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
struct CkptLayout {
    size_t hseg, cseg, car, scr, total;
};
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

}  // namespace

namespace rnn355 {

// A grid whose workgroups wait on one another every step (bounded polls of
// step-tagged words, no grid-wide barrier) needs all of them on the chip at
// once.  The host checks that it fits (resident workgroups per CU from the
// kernel's registers and LDS, times the CU count) and then dispatches it as
// an ordinary launch; workgroups are dispatched in index order, and a member
// that never arrived would end its partners' polls at the spin limit with
// RNN_ERR_BARRIER_TIMEOUT, not a hang.  (A cooperative launch gives the same
// residency guarantee but goes through a second device queue of the runtime,
// whose teardown at process exit outlived a profiler's interception tables.)
hipError_t launch_all_resident(const void *fn, int grid, int threads, void **args, size_t lds,
                               hipStream_t s) {
    struct Key {
        int dev;
        const void *fn;
        int threads;
        size_t lds;
        int per_cu;
    };
    static std::mutex mu;
    static Key cache[64];
    static int ncache = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int per_cu = -1;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (int i = 0; i < ncache; ++i)
            if (cache[i].dev == dev && cache[i].fn == fn && cache[i].threads == threads &&
                cache[i].lds == lds)
                per_cu = cache[i].per_cu;
    }
    if (per_cu < 0) {
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds);
        if (e != hipSuccess) return e;
        per_cu = nb;
        std::lock_guard<std::mutex> lk(mu);
        if (ncache < 64) cache[ncache++] = Key{dev, fn, threads, lds, per_cu};
    }
    if ((long)per_cu * device_cus() < grid) return hipErrorCooperativeLaunchTooLarge;
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, s);
}

}  // namespace rnn355

// ---- the allocation-free recurrence (rnn_rec_lstm_noalloc)
//
// Its scratch (status word, XCD table, exchange slots, R^T of the split-R
// plan: what rnn_rec_lstm keeps in the caller's workspace) is this
// file-scope device array; each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` is only a stand-in for the
// symbol: its device address, per device, comes from hipGetSymbolAddress
// (scratch_ptr) and is what the kernels receive.
constexpr size_t kScratchBytes = RNN_REC_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with the device current) and kept per device.
void *scratch_ptr() {
    static std::mutex mu;
    static void *ptr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

}  // namespace

extern "C" {

const char *rnn_status_str(rnn_status s) {
    switch (s) {
        case RNN_OK: return "RNN_OK";
        case RNN_ERR_INVALID_ARG: return "RNN_ERR_INVALID_ARG: bad pointer, dimension or enum";
        case RNN_ERR_UNSUPPORTED: return "RNN_ERR_UNSUPPORTED: no kernel for this shape";
        case RNN_ERR_WORKSPACE: return "RNN_ERR_WORKSPACE: workspace missing or too small";
        case RNN_ERR_HIP: return "RNN_ERR_HIP: a HIP runtime call failed";
        case RNN_ERR_BARRIER_TIMEOUT: return "RNN_ERR_BARRIER_TIMEOUT: a step wait ran out";
    }
    return "RNN_ERR_UNKNOWN";
}

size_t rnn_workspace_size(rnn_op op, const rnn_dims *d, rnn_dtype dt) {
    if (!dims_ok(d) || !dtype_ok(dt)) return 0;
    const int G = gates_of_op(op);
    switch (op) {
        case RNN_OP_FWD_LSTM:
        case RNN_OP_FWD_GRU:
            return kHeader + xchg_bytes(d) + gx_bytes(d, G) + ready_bytes(d) + wt_bytes(d, G) +
                   rt_fwd_bytes(d, dt, G);
        case RNN_OP_REC_LSTM:
        case RNN_OP_REC_GRU:
            return kHeader + xchg_bytes(d) + rt_fwd_bytes(d, dt, G);
        case RNN_OP_BWD_LSTM:
        case RNN_OP_BWD_GRU:
            return kHeader + (dt == RNN_F32 ? bwd_f32_layout(d, G).total : bwd_layout(d, G).total);
        default:
            return 0;
    }
}

rnn_status rnn_plan_describe(rnn_op op, const rnn_dims *d, rnn_dtype dt, char *buf,
                             size_t len) {
    if (!dims_ok(d) || !dtype_ok(dt) || !buf || len == 0) return RNN_ERR_INVALID_ARG;
    if (op < RNN_OP_FWD_LSTM || op > RNN_OP_REC_GRU) return RNN_ERR_INVALID_ARG;
    const int cell = cell_of_op(op);
    const Choice ch = choose(cell, d, dt, device_cus());
    if (!ch.ok) {
        snprintf(buf, len, "rec_kernel=none");
        return RNN_ERR_UNSUPPORTED;
    }
    const bool fwd = op == RNN_OP_FWD_LSTM || op == RNN_OP_FWD_GRU;
    char proj[128];
    const bool piped = fwd && pipelined(ch, d, dt, device_cus());
    char hs[32] = "";
    if (piped) snprintf(hs, sizeof hs, " head_start_panels=%d", head_start_panels(ch, d, nullptr));
    snprintf(proj, sizeof proj, " predicted_ns_per_step=%.0f%s%s", ch.cand.ns_total / d->T,
             !fwd ? "" : piped ? " input_proj=pipelined" : " input_proj=serial", hs);
    if (ch.use_wide) {
        const WidePlan &p = ch.wide;
        snprintf(buf, len,
                 "rec_kernel=mfma_split_R rows_per_wg=1 wg=%d threads=%d wg_per_head_row_tile=1 "
                 "r_lds_bytes=%zu%s",
                 p.grid, p.threads, p.lds, proj);
    } else if (ch.use_mc) {
        const McPlan &p = ch.mc;
        snprintf(buf, len,
                 "rec_kernel=mfma_multi_cu rows_per_wg=%d wg=%d threads=%d wg_per_head_row_tile=%d "
                 "units_per_wg=%d k_splits=%d exchange=%s%s",
                 p.BT, p.grid, p.threads, p.K, p.nb * 16, p.ks,
                 ch.cand.xcd_local ? "xcd_l2" : "memory", proj);
    } else {
        const RecPlan &p = ch.rec;
        snprintf(buf, len,
                 "rec_kernel=%s rows_per_wg=%d wg=%d threads=%d wg_per_head_row_tile=1 "
                 "units_per_thread=%d%s",
                 p.kind == kRecMfma ? "mfma_resident_R" : "lds_simple", p.BT, p.grid, p.threads,
                 p.upt, proj);
    }
    return RNN_OK;
}

rnn_status rnn_plan_search(rnn_op op, const rnn_dims *d, rnn_dtype dt, int num_cu,
                           rnn_plan_candidate *out, int max_out, int *n_out, int *chosen) {
    if (!dims_ok(d) || !dtype_ok(dt) || max_out < 0 || (max_out > 0 && !out) || !n_out || !chosen)
        return RNN_ERR_INVALID_ARG;
    if (op < RNN_OP_FWD_LSTM || op > RNN_OP_REC_GRU) return RNN_ERR_INVALID_ARG;
    const int cus = num_cu > 0 ? num_cu : device_cus();
    const PlanFix fix{bt_override(), k_override(), kcw_override(), !wide_enabled(),
                      !mc_xcd_enabled()};
    static thread_local PlanCand buf[kPlanMaxCands];
    int best = -1;
    const int n = plan_search(cell_of_op(op), d->T, d->B, d->NH, d->Dh, dt == RNN_BF16, cus, fix,
                              buf, kPlanMaxCands, &best);
    const int kept = std::min(n, kPlanMaxCands);
    for (int i = 0; i < kept && i < max_out; ++i) {
        const PlanCand &c = buf[i];
        rnn_plan_candidate &o = out[i];
        o.family = c.family;
        o.rows_per_wg = c.BT;
        o.wg_per_head = c.K;
        o.blocks_per_wg = c.nb;
        o.k_splits = c.ks;
        o.kchunks_per_wave = c.kcw;
        o.row_slots = c.r4;
        o.frags_agpr = c.fa;
        o.frags_vgpr = c.fv;
        o.frags_lds = c.fl;
        o.waves = c.waves;
        o.grid = c.grid;
        o.r_vgpr = c.r_vgpr;
        o.wg_per_cu = c.wg_per_cu;
        o.xcd_local = c.xcd_local;
        o.lds_bytes = c.lds;
        o.feasible = c.feasible;
        o.violated = c.violated;
        o.ns_per_step = c.ns_step;
        o.ns_total = c.ns_total;
    }
    *n_out = kept;
    *chosen = best;
    return best >= 0 ? RNN_OK : RNN_ERR_UNSUPPORTED;
}

rnn_status rnn_input_proj(int M, int K, int N, rnn_dtype dt, const void *x, const void *W,
                          const float *b, float *gx, hipStream_t stream) {
    if (M <= 0 || K <= 0 || N <= 0 || !dtype_ok(dt)) return RNN_ERR_INVALID_ARG;
    if (!x || !W || !gx) return RNN_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(W) || !aligned16(b) || !aligned16(gx))
        return RNN_ERR_INVALID_ARG;
    if (!gemm_shape_ok(K, N, dt)) return RNN_ERR_UNSUPPORTED;
    return input_proj(M, K, N, dt, x, W, b, gx, nullptr, stream);
}

rnn_status rnn_input_proj_t(int M, int K, int N, rnn_dtype dt, const void *x, const void *Wt,
                            const float *b, float *gx, hipStream_t stream) {
    if (M <= 0 || K <= 0 || N <= 0 || !dtype_ok(dt)) return RNN_ERR_INVALID_ARG;
    if (!x || !Wt || !gx) return RNN_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wt) || !aligned16(b) || !aligned16(gx))
        return RNN_ERR_INVALID_ARG;
    if (dt != RNN_BF16 || !gemm_dma_ok(K)) return RNN_ERR_UNSUPPORTED;
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = (const uint16_t *)x; g.lda = K;
    g.B = (const uint16_t *)Wt; g.ldb = K;
    g.bias = b; g.C = gx; g.ldc = N;
    return launch_gemm_dma(g, 1, stream) == hipSuccess ? RNN_OK : RNN_ERR_HIP;
}

rnn_status rnn_rec_lstm(const rnn_dims *d, rnn_dtype dt, const float *gx, const void *R,
                        const float *h0, const float *c0, float *h_seq, float *c_seq,
                        float *hT, float *cT, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || !gx || !R || !hT || !cT) return RNN_ERR_INVALID_ARG;
    const void *ps[] = {gx, R, h0, c0, h_seq, c_seq, hT, cT, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    if (!rec_supported(kLSTM, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rnn_workspace_size(RNN_OP_REC_LSTM, d, dt)) return RNN_ERR_WORKSPACE;
    uint16_t *rt = (uint16_t *)((char *)ws + kHeader + xchg_bytes(d));
    return rec_fwd(kLSTM, d, dt, gx, R, h0, c0, h_seq, c_seq, hT, cT, ws, rt, stream);
}

rnn_status rnn_rec_lstm_noalloc(const rnn_dims *d, rnn_dtype dt, const float *gx, const void *R,
                                const float *h0, const float *c0, float *h_seq, float *c_seq,
                                float *hT, float *cT, unsigned *dev_status, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || !gx || !R || !hT || !cT) return RNN_ERR_INVALID_ARG;
    const void *ps[] = {gx, R, h0, c0, h_seq, c_seq, hT, cT, dev_status};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    if (!rec_supported(kLSTM, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (rnn_workspace_size(RNN_OP_REC_LSTM, d, dt) > kScratchBytes) return RNN_ERR_WORKSPACE;
    void *ws = scratch_ptr();
    if (!ws) return RNN_ERR_HIP;
    // the array keeps the previous call's contents: the status word starts at
    // zero for every call (the kernels clear their own exchange slots)
    hipLaunchKernelGGL(status_word_kernel, dim3(1), dim3(64), 0, stream, (unsigned *)ws,
                       (unsigned *)nullptr);
    if (hipGetLastError() != hipSuccess) return RNN_ERR_HIP;
    uint16_t *rt = (uint16_t *)((char *)ws + kHeader + xchg_bytes(d));
    const rnn_status st = rec_fwd(kLSTM, d, dt, gx, R, h0, c0, h_seq, c_seq, hT, cT, ws, rt,
                                  stream);
    if (st != RNN_OK || !dev_status) return st;
    hipLaunchKernelGGL(status_word_kernel, dim3(1), dim3(64), 0, stream, (unsigned *)ws,
                       dev_status);
    return hipGetLastError() == hipSuccess ? RNN_OK : RNN_ERR_HIP;
}

rnn_status rnn_rec_gru(const rnn_dims *d, rnn_dtype dt, const float *gx, const void *R,
                       const float *h0, float *h_seq, float *hT, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || !gx || !R || !hT) return RNN_ERR_INVALID_ARG;
    const void *ps[] = {gx, R, h0, h_seq, hT, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    if (!rec_supported(kGRU, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rnn_workspace_size(RNN_OP_REC_GRU, d, dt)) return RNN_ERR_WORKSPACE;
    uint16_t *rt = (uint16_t *)((char *)ws + kHeader + xchg_bytes(d));
    return rec_fwd(kGRU, d, dt, gx, R, h0, nullptr, h_seq, nullptr, hT, nullptr, ws, rt, stream);
}

rnn_status rnn_fwd_lstm(const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                        const void *R, const float *b, const float *h0, const float *c0,
                        float *h_seq, float *c_seq, float *hT, float *cT, void *ws,
                        size_t ws_bytes, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || !x || !W || !R || !hT || !cT) return RNN_ERR_INVALID_ARG;
    const void *ps[] = {x, W, R, b, h0, c0, h_seq, c_seq, hT, cT, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    const int N = d->NH * 4 * d->Dh;
    if (!gemm_shape_ok(d->Din, N, dt) || !rec_supported(kLSTM, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rnn_workspace_size(RNN_OP_FWD_LSTM, d, dt)) return RNN_ERR_WORKSPACE;
    return forward(kLSTM, d, dt, x, W, R, b, h0, c0, h_seq, c_seq, hT, cT, ws, stream);
}

rnn_status rnn_fwd_gru(const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                       const void *R, const float *b, const float *h0, float *h_seq,
                       float *hT, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || !x || !W || !R || !hT) return RNN_ERR_INVALID_ARG;
    const void *ps[] = {x, W, R, b, h0, h_seq, hT, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    const int N = d->NH * 3 * d->Dh;
    if (!gemm_shape_ok(d->Din, N, dt) || !rec_supported(kGRU, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rnn_workspace_size(RNN_OP_FWD_GRU, d, dt)) return RNN_ERR_WORKSPACE;
    return forward(kGRU, d, dt, x, W, R, b, h0, nullptr, h_seq, nullptr, hT, nullptr, ws, stream);
}

size_t rnn_workspace_size_stack(rnn_op op, const rnn_dims *d, int L, rnn_dtype dt) {
    if (!dims_ok(d) || !dtype_ok(dt) || L < 1 || L > kMaxLayers) return 0;
    if (op != RNN_OP_FWD_LSTM && op != RNN_OP_FWD_GRU) return 0;
    return stack_layout(d, gates_of_op(op), dt).total;
}

// Common checks of the stack entry points.  W, R, b are host arrays of L
// device pointers (b may be NULL, or hold NULLs).
static rnn_status stack_args_ok(int cell, const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                                const void *const *W, const void *const *R,
                                const float *const *b, const void *const *more, int nmore,
                                void *ws, size_t ws_bytes) {
    if (!dims_ok(d) || !dtype_ok(dt) || L < 1 || L > kMaxLayers || !x || !W || !R)
        return RNN_ERR_INVALID_ARG;
    for (int i = 0; i < nmore; ++i)
        if (!aligned16(more[i])) return RNN_ERR_INVALID_ARG;
    if (!aligned16(x)) return RNN_ERR_INVALID_ARG;
    const int G = gates_of_cell(cell), H = d->NH * d->Dh, N = d->NH * G * d->Dh;
    for (int l = 0; l < L; ++l) {
        if (!W[l] || !R[l] || !aligned16(W[l]) || !aligned16(R[l])) return RNN_ERR_INVALID_ARG;
        if (b && !aligned16(b[l])) return RNN_ERR_INVALID_ARG;
        if (!gemm_shape_ok(l == 0 ? d->Din : H, N, dt)) return RNN_ERR_UNSUPPORTED;
    }
    rnn_dims dh = *d;
    dh.Din = H;
    if (!rec_supported(cell, d, dt) || !rec_supported(cell, &dh, dt)) return RNN_ERR_UNSUPPORTED;
    const rnn_op op = cell == kLSTM ? RNN_OP_FWD_LSTM : RNN_OP_FWD_GRU;
    if (!ws || ws_bytes < rnn_workspace_size_stack(op, d, L, dt)) return RNN_ERR_WORKSPACE;
    return RNN_OK;
}

rnn_status rnn_fwd_lstm_stack(const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                              const void *const *W, const void *const *R, const float *const *b,
                              const float *h0, const float *c0, float *h_seq, float *c_seq,
                              float *hT, float *cT, void *ws, size_t ws_bytes,
                              hipStream_t stream) {
    if (!hT || !cT) return RNN_ERR_INVALID_ARG;
    const void *more[] = {h0, c0, h_seq, c_seq, hT, cT, ws};
    const rnn_status st = stack_args_ok(kLSTM, d, L, dt, x, W, R, b, more, 7, ws, ws_bytes);
    if (st != RNN_OK) return st;
    return forward_stack(kLSTM, d, L, dt, x, W, R, b, h0, c0, h_seq, c_seq, hT, cT, ws, stream);
}

rnn_status rnn_fwd_gru_stack(const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                             const void *const *W, const void *const *R, const float *const *b,
                             const float *h0, float *h_seq, float *hT, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
    if (!hT) return RNN_ERR_INVALID_ARG;
    const void *more[] = {h0, h_seq, hT, ws};
    const rnn_status st = stack_args_ok(kGRU, d, L, dt, x, W, R, b, more, 4, ws, ws_bytes);
    if (st != RNN_OK) return st;
    return forward_stack(kGRU, d, L, dt, x, W, R, b, h0, nullptr, h_seq, nullptr, hT, nullptr, ws,
                         stream);
}

size_t rnn_workspace_size_chunked(rnn_op op, const rnn_dims *d, int chunk, rnn_dtype dt) {
    if (!dims_ok(d) || !dtype_ok(dt) || chunk < 1) return 0;
    const int G = gates_of_op(op);
    if (op == RNN_OP_FWD_LSTM || op == RNN_OP_FWD_GRU) return chunk_layout(d, chunk, G, dt).total;
    if (op == RNN_OP_BWD_LSTM || op == RNN_OP_BWD_GRU) return ckpt_layout(d, chunk, G, dt).total;
    return 0;
}

rnn_status rnn_fwd_lstm_chunked(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                                const void *W, const void *R, const float *b, const float *h0,
                                const float *c0, float *h_seq, float *c_seq, float *hT,
                                float *cT, float *h_ckpt, float *c_ckpt, void *ws,
                                size_t ws_bytes, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || chunk < 1 || !x || !W || !R || !hT || !cT ||
        (h_ckpt == nullptr) != (c_ckpt == nullptr))
        return RNN_ERR_INVALID_ARG;
    const void *ps[] = {x, W, R, b, h0, c0, h_seq, c_seq, hT, cT, h_ckpt, c_ckpt, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    const int N = d->NH * 4 * d->Dh;
    if (!gemm_shape_ok(d->Din, N, dt) || !rec_supported(kLSTM, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rnn_workspace_size_chunked(RNN_OP_FWD_LSTM, d, chunk, dt))
        return RNN_ERR_WORKSPACE;
    return forward_chunked(kLSTM, d, dt, chunk, x, W, R, b, h0, c0, h_seq, c_seq, hT, cT, h_ckpt,
                           c_ckpt, ws, stream);
}

rnn_status rnn_fwd_gru_chunked(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                               const void *W, const void *R, const float *b, const float *h0,
                               float *h_seq, float *hT, float *h_ckpt, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt) || chunk < 1 || !x || !W || !R || !hT)
        return RNN_ERR_INVALID_ARG;
    const void *ps[] = {x, W, R, b, h0, h_seq, hT, h_ckpt, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    const int N = d->NH * 3 * d->Dh;
    if (!gemm_shape_ok(d->Din, N, dt) || !rec_supported(kGRU, d, dt)) return RNN_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rnn_workspace_size_chunked(RNN_OP_FWD_GRU, d, chunk, dt))
        return RNN_ERR_WORKSPACE;
    return forward_chunked(kGRU, d, dt, chunk, x, W, R, b, h0, nullptr, h_seq, nullptr, hT,
                           nullptr, h_ckpt, nullptr, ws, stream);
}

// Common checks of the checkpointed backward entry points.
static rnn_status ckpt_args_ok(int cell, const rnn_dims *d, rnn_dtype dt, int chunk,
                               const void *const *req, int nreq, const void *const *all, int nall,
                               const void *h_ckpt, const void *c_ckpt, void *ws,
                               size_t ws_bytes) {
    if (!dims_ok(d) || !dtype_ok(dt) || chunk < 1) return RNN_ERR_INVALID_ARG;
    for (int i = 0; i < nreq; ++i)
        if (!req[i]) return RNN_ERR_INVALID_ARG;
    for (int i = 0; i < nall; ++i)
        if (!aligned16(all[i])) return RNN_ERR_INVALID_ARG;
    if (chunk < d->T && (!h_ckpt || (cell == kLSTM && !c_ckpt))) return RNN_ERR_INVALID_ARG;
    const int G = gates_of_cell(cell);
    const bool bwd_ok = dt == RNN_F32 ? plan_bwd_f32(cell, d->B, d->Dh).ok != 0
                                      : d->Dh % 16 == 0;
    if (!bwd_ok || !gemm_shape_ok(d->Din, d->NH * G * d->Dh, dt) || !rec_supported(cell, d, dt))
        return RNN_ERR_UNSUPPORTED;
    const rnn_op op = cell == kLSTM ? RNN_OP_BWD_LSTM : RNN_OP_BWD_GRU;
    if (!ws || ws_bytes < rnn_workspace_size_chunked(op, d, chunk, dt)) return RNN_ERR_WORKSPACE;
    return RNN_OK;
}

rnn_status rnn_bwd_lstm_ckpt(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                             const void *W, const void *R, const float *b, const float *h0,
                             const float *c0, const float *h_ckpt, const float *c_ckpt,
                             const float *dh_seq, const float *dhT, const float *dcT, float *dx,
                             float *dW, float *dR, float *db, float *dh0, float *dc0, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
    const void *req[] = {x, W, R, dh_seq, dx, dW, dR, db, dh0, dc0};
    const void *all[] = {x, W, R, b, h0, c0, h_ckpt, c_ckpt, dh_seq, dhT, dcT,
                         dx, dW, dR, db, dh0, dc0, ws};
    const rnn_status st = ckpt_args_ok(kLSTM, d, dt, chunk, req, 10, all, 18, h_ckpt, c_ckpt, ws,
                                       ws_bytes);
    if (st != RNN_OK) return st;
    return backward_ckpt(kLSTM, d, dt, chunk, x, W, R, b, h0, c0, h_ckpt, c_ckpt, dh_seq, dhT,
                         dcT, dx, dW, dR, db, dh0, dc0, ws, stream);
}

rnn_status rnn_bwd_gru_ckpt(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                            const void *W, const void *R, const float *b, const float *h0,
                            const float *h_ckpt, const float *dh_seq, const float *dhT,
                            float *dx, float *dW, float *dR, float *db, float *dh0, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
    const void *req[] = {x, W, R, dh_seq, dx, dW, dR, db, dh0};
    const void *all[] = {x, W, R, b, h0, h_ckpt, dh_seq, dhT, dx, dW, dR, db, dh0, ws};
    const rnn_status st = ckpt_args_ok(kGRU, d, dt, chunk, req, 9, all, 14, h_ckpt, nullptr, ws,
                                       ws_bytes);
    if (st != RNN_OK) return st;
    return backward_ckpt(kGRU, d, dt, chunk, x, W, R, b, h0, nullptr, h_ckpt, nullptr, dh_seq,
                         dhT, nullptr, dx, dW, dR, db, dh0, nullptr, ws, stream);
}

rnn_status rnn_bwd_lstm(const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                        const void *R, const float *b, const float *h0, const float *c0,
                        const float *h_seq, const float *c_seq, const float *dh_seq,
                        const float *dhT, const float *dcT, float *dx, float *dW, float *dR,
                        float *db, float *dh0, float *dc0, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt)) return RNN_ERR_INVALID_ARG;
    if (!x || !W || !R || !h_seq || !c_seq || !dh_seq || !dx || !dW || !dR || !db || !dh0 || !dc0)
        return RNN_ERR_INVALID_ARG;
    const void *ps[] = {x, W, R, b, h0, c0, h_seq, c_seq, dh_seq, dhT, dcT,
                        dx, dW, dR, db, dh0, dc0, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    return backward(kLSTM, d, dt, x, W, R, b, h0, c0, h_seq, c_seq, dh_seq, dhT, dcT, dx, dW, dR,
                    db, dh0, dc0, ws, ws_bytes, stream);
}

rnn_status rnn_bwd_gru(const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                       const void *R, const float *b, const float *h0, const float *h_seq,
                       const float *dh_seq, const float *dhT, float *dx, float *dW, float *dR,
                       float *db, float *dh0, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!dims_ok(d) || !dtype_ok(dt)) return RNN_ERR_INVALID_ARG;
    if (!x || !W || !R || !h_seq || !dh_seq || !dx || !dW || !dR || !db || !dh0)
        return RNN_ERR_INVALID_ARG;
    const void *ps[] = {x, W, R, b, h0, h_seq, dh_seq, dhT, dx, dW, dR, db, dh0, ws};
    for (const void *p : ps)
        if (!aligned16(p)) return RNN_ERR_INVALID_ARG;
    return backward(kGRU, d, dt, x, W, R, b, h0, nullptr, h_seq, nullptr, dh_seq, dhT, nullptr, dx,
                    dW, dR, db, dh0, nullptr, ws, ws_bytes, stream);
}

rnn_status rnn_workspace_status(const void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!ws || ws_bytes < kHeader) return RNN_ERR_INVALID_ARG;
    if (hipStreamSynchronize(stream) != hipSuccess) return RNN_ERR_HIP;
    uint32_t flag = 0;
    if (hipMemcpy(&flag, ws, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return RNN_ERR_HIP;
    return flag ? RNN_ERR_BARRIER_TIMEOUT : RNN_OK;
}

}  // extern "C"
