// host.h -- what the host side of librnn355 shares between its files: the
// workspace layout, the plan choice, environment overrides, the library's
// side streams, and the host paths each file implements:
//   host_fwd.hip   input projection, recurrence, forward, stacked layers;
//   host_bwd.hip   backpropagation through time;
//   host_long.hip  long sequences in chunks (chunked forward, checkpointed
//                  backward);
//   api.hip        the C ABI (include/rnn355.h): argument checks, workspace
//                  sizes, and the calls into the paths above.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/rnn355.h"
#include "common.h"
#include "kernels.h"

namespace rnn355 {
namespace host {

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

inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

inline bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

inline bool dims_ok(const rnn_dims *d) {
    return d && d->T > 0 && d->B > 0 && d->Din > 0 && d->NH > 0 && d->Dh > 0 &&
           (long)d->NH * d->Dh <= (1L << 24) && (long)d->T * d->B <= (1L << 30);
}

inline bool dtype_ok(rnn_dtype dt) { return dt == RNN_F32 || dt == RNN_BF16; }

inline int gates_of_op(rnn_op op) {
    return (op == RNN_OP_FWD_GRU || op == RNN_OP_BWD_GRU || op == RNN_OP_REC_GRU) ? 3 : 4;
}

inline int cell_of_op(rnn_op op) { return gates_of_op(op) == 4 ? kLSTM : kGRU; }

inline int gates_of_cell(int cell) { return cell == kLSTM ? 4 : 3; }

// Exchange slots: [groups][2][BT][Dh/2] 8-byte words with groups =
// NH * ceil(B/BT) and BT <= 16, so groups * BT <= NH * (B + 15).
inline size_t xchg_bytes(const rnn_dims *d) {
    return align_up(2u * 8u * (size_t)d->NH * (d->B + 15) * ((d->Dh + 1) / 2));
}

inline size_t gx_bytes(const rnn_dims *d, int G) {
    return align_up(sizeof(float) * (size_t)d->T * d->B * d->NH * G * d->Dh);
}

// Row-panel counters of the pipelined forward (one word per kGemmRowTile
// rows of gx), after gx in the forward workspace.
inline long gx_panels(const rnn_dims *d) {
    return ((long)d->T * d->B + kGemmRowTile - 1) / kGemmRowTile;
}
inline size_t ready_bytes(const rnn_dims *d) {
    return align_up(sizeof(unsigned) * (size_t)gx_panels(d));
}

// W staged transposed ([N][Din] bf16) for the k-major contraction.
inline size_t wt_bytes(const rnn_dims *d, int G) {
    return align_up(sizeof(uint16_t) * (size_t)d->Din * d->NH * G * d->Dh);
}

// R staged transposed per head ([NH][G*Dh][Dh] bf16) for the Dh = 256
// one-CU recurrence; sized for every bf16 shape with Dh = 256.
inline size_t rt_fwd_bytes(const rnn_dims *d, rnn_dtype dt, int G) {
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
inline BwdLayout bwd_layout(const rnn_dims *d, int G) {
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
    // R^T per head
    L.rt = off;   off += align_up(sizeof(uint16_t) * (size_t)d->NH * G * d->Dh * d->Dh);
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
inline BwdF32Layout bwd_f32_layout(const rnn_dims *d, int G) {
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
namespace {
__global__ void status_word_kernel(unsigned *word, unsigned *out) {
    if (threadIdx.x == 0) {
        if (out) out[0] = word[0];
        else word[0] = 0u;
    }
}
}  // namespace

// Compute-unit count of the current device, cached per device.
inline int device_cus() {
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
inline int env_int(const char *name) {
    const char *e = getenv(name);
    return e ? atoi(e) : 0;
}
inline int bt_override() { return env_int("RNN355_REC_BT"); }
inline int env_int_or(const char *name, int dflt) {
    const char *e = getenv(name);
    return e ? atoi(e) : dflt;
}
// RNN355_MC_XCD=0: the multi-CU kernel numbers its workgroups group by
// group and exchanges through memory even where a group could share an L2.
inline bool mc_xcd_enabled() {
    const char *e = getenv("RNN355_MC_XCD");
    return !e || atoi(e) != 0;
}
// RNN355_PIPELINE=0 runs the forward's two phases one after the other;
// =1 overlaps them wherever that is safe, also where the plan would not.
inline int pipeline_override() {
    const char *e = getenv("RNN355_PIPELINE");
    return !e || !e[0] ? -1 : e[0] == '0' ? 0 : 1;
}
inline int k_override() { return env_int("RNN355_REC_K"); }
// RNN355_REC_KCW=4|8: k-chunks per wave of the multi-CU kernel.
inline int kcw_override() { return env_int("RNN355_REC_KCW"); }
// RNN355_REC_WIDE=0 serves Dh = 256 with the multi-CU kernel instead of the
// one-CU kernel with split R.
inline bool wide_enabled() {
    const char *e = getenv("RNN355_REC_WIDE");
    return !(e && e[0] == '0');
}
// Polls of a multi-CU step wait before it is declared lost (~4 s by default;
// tests lower it to force the time-out path).
inline unsigned spin_limit() {
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

inline Choice choose(int cell, const rnn_dims *d, rnn_dtype dt, int num_cu) {
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

// Workspace: one forward workspace sized for the larger input width, two
// float32 sequence buffers (layers that run in turn), two bf16 sequence
// buffers (layer inputs), a second gx and the step counters (overlapped
// pairs).
struct StackLayout {
    size_t fwd, hbuf, hbf, gx2, done, total;
};

// Workspace of the chunked forward (host_long.hip): two gx slots of `chunk`
// steps in place of T, W^T, R^T, the exchange slots and the state between
// chunks.
struct ChunkLayout {
    size_t gx0, gx1, wt, rt, st, total;
};

// Workspace of the checkpointed backward (host_long.hip): one forward or
// backward workspace of `chunk` steps, the segment's h and c, the carries.
struct CkptLayout {
    size_t hseg, cseg, car, scr, total;
};

// Streams of the current device (default priority) for work that runs
// beside the caller's stream, two per device (i = 0, 1); created on first use.
inline hipStream_t side_stream(int i = 0) {
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
// a recorded event alive until its work is done); make = false: none
// (a call that turns out to need no second stream), ok stays false.
struct CallEvents {
    hipEvent_t e[kBwdChunks + 3] = {};
    bool ok = false;
    explicit CallEvents(bool make = true) {
        if (!make) return;
        ok = true;
        for (hipEvent_t &v : e)
            if (hipEventCreateWithFlags(&v, hipEventDisableTiming) != hipSuccess) ok = false;
    }
    ~CallEvents() {
        for (hipEvent_t v : e)
            if (v) (void)hipEventDestroy(v);
    }
};

// ---- host paths (pointers validated by the entry points in api.hip)

// host_fwd.hip
bool gemm_shape_ok(int K, int N, rnn_dtype dt);
rnn_status input_proj(int M, int K, int N, rnn_dtype dt, const void *x, const void *W,
                      const float *b, float *gx, uint32_t *clear, hipStream_t s,
                      unsigned *ready = nullptr, uint16_t *wt = nullptr);
rnn_status rec_fwd(int cell, const rnn_dims *d, rnn_dtype dt, const float *gx, const void *R,
                   const float *h0, const float *c0, float *h_seq, float *c_seq, float *hT,
                   float *cT, void *ws, uint16_t *rt, hipStream_t s, bool clear_status = true);
bool rec_supported(int cell, const rnn_dims *d, rnn_dtype dt);
bool pipelined(const Choice &ch, const rnn_dims *d, rnn_dtype dt, int cus);
int proj_workgroups(const rnn_dims *d, const Choice &ch, int tiles_per_panel, int free);
void proj_taper(const rnn_dims *d, const Choice &ch, int tiles_per_panel, int n_gemm,
                long proj_panels, int *rows1, int *n2);
int head_start_panels(const Choice &ch, const rnn_dims *d, const void *x);
rnn_status forward(int cell, const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                   const void *R, const float *b, const float *h0, const float *c0,
                   float *h_seq, float *c_seq, float *hT, float *cT, void *ws, hipStream_t s,
                   bool clear_status = true);
int stack_overlap_wgs(const Choice &ch, const rnn_dims *dh, rnn_dtype dt, int cus);
StackLayout stack_layout(const rnn_dims *d, int G, rnn_dtype dt);
rnn_status forward_stack(int cell, const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                         const void *const *W, const void *const *R, const float *const *b,
                         const float *h0, const float *c0, float *h_seq, float *c_seq,
                         float *hT, float *cT, void *ws, hipStream_t s);

// host_bwd.hip
// The bf16 backward's sweep: the split-R plan (Dh = 256; on two CUs per
// (head, row) where the pairs fit the XCD grouping) or the exchange-based
// plan, its grid, the CUs it leaves free, and the time chunks it runs in
// (1: one piece).  ok == false where no sweep fits.  Pure host function.
struct BwdChoice {
    WidePlan pw;
    BwdPlan p;
    bool two;
    int sweep_grid, free_cus, chunks;
    bool ok;
};
BwdChoice choose_bwd(int cell, const rnn_dims *d, int cus);
rnn_status backward_f32(int cell, const rnn_dims *d, const float *x, const float *W,
                        const float *R, const float *b, const float *h0, const float *c0,
                        const float *h_seq, const float *c_seq, const float *dh_seq,
                        const float *dhT, const float *dcT, float *dx, float *dW, float *dR,
                        float *db, float *dh0, float *dc0, void *ws, size_t ws_bytes,
                        hipStream_t s, bool accumulate, bool clear_status);
int bwd_chunk_starts(int T, int *starts);
rnn_status backward(int cell, const rnn_dims *d, rnn_dtype dt, const void *x, const void *W,
                    const void *R, const float *b, const float *h0, const float *c0,
                    const float *h_seq, const float *c_seq, const float *dh_seq,
                    const float *dhT, const float *dcT, float *dx, float *dW, float *dR,
                    float *db, float *dh0, float *dc0, void *ws, size_t ws_bytes,
                    hipStream_t stream, bool accumulate = false, bool clear_status = true);

// host_long.hip
ChunkLayout chunk_layout(const rnn_dims *d, int chunk, int G, rnn_dtype dt);
rnn_status forward_chunked(int cell, const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                           const void *W, const void *R, const float *b, const float *h0,
                           const float *c0, float *h_seq, float *c_seq, float *hT, float *cT,
                           float *h_ck, float *c_ck, void *ws, hipStream_t s);
CkptLayout ckpt_layout(const rnn_dims *d, int chunk, int G, rnn_dtype dt);
rnn_status backward_ckpt(int cell, const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                         const void *W, const void *R, const float *b, const float *h0,
                         const float *c0, const float *h_ck, const float *c_ck,
                         const float *dh_seq, const float *dhT, const float *dcT, float *dx,
                         float *dW, float *dR, float *db, float *dh0, float *dc0, void *ws,
                         hipStream_t s);

}  // namespace host
}  // namespace rnn355
