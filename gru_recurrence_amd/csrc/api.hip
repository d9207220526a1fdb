// api.hip -- the librnn355 C ABI (include/rnn355.h): argument validation,
// workspace sizes and the calls into the host paths (host.h), the launch of
// grids whose workgroups wait on one another, and the allocation-free
// recurrence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "host.h"

using namespace rnn355;
using namespace rnn355::host;

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
    if (op == RNN_OP_BWD_LSTM || op == RNN_OP_BWD_GRU) {
        if (dt == RNN_F32) {
            const BwdF32Plan p = plan_bwd_f32(cell, d->B, d->Dh);
            if (!p.ok) {
                snprintf(buf, len, "bwd_sweep=none");
                return RNN_ERR_UNSUPPORTED;
            }
            snprintf(buf, len, "bwd_sweep=f32_lds rows_per_wg=%d wg=%d chunks=1", p.BT,
                     p.nbt * d->NH);
            return RNN_OK;
        }
        const BwdChoice b = choose_bwd(cell, d, device_cus());
        if (!b.ok) {
            snprintf(buf, len, "bwd_sweep=none");
            return RNN_ERR_UNSUPPORTED;
        }
        snprintf(buf, len,
                 "bwd_sweep=%s rows_per_wg=%d wg=%d wg_per_head_row_tile=%d chunks=%d "
                 "free_cus=%d",
                 b.two ? "split_R_two_cu" : b.pw.ok ? "split_R" : "exchange",
                 b.pw.ok ? 1 : b.p.BT, b.sweep_grid, b.two ? 2 : b.pw.ok ? 1 : b.p.K, b.chunks,
                 b.free_cus);
        return RNN_OK;
    }
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
