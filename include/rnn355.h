/*
 * rnn355.h -- C ABI of librnn355: multi-head LSTM / GRU recurrence with a
 * block-diagonal recurrent matrix on AMD Instinct MI355X (gfx950).
 *
 * The operation (FlashRNN, arXiv 2412.07752, abstract; and "Re-examining
 * RNNs from a GPU programming perspective", blog.hotdry.top 2025-09-21, the
 * paragraphs on the step dependency, on keeping R resident across steps and
 * on head-wise splitting):
 *   a traditional LSTM or GRU whose hidden state of size H = NH*Dh is split
 *   into NH independent heads, each with its own Dh x G*Dh recurrent block, so
 *   the recurrent matrix is block-diagonal.  Every call first forms the input
 *   part of all gates for all T steps at once (Gx = x W + b, a dense
 *   contraction) and then runs the strictly sequential recurrence
 *   A_t = Gx_t + h_{t-1} R, followed by the cell's gate update.
 *
 * Cells (textbook forms; the pages name the cells but print no equations):
 *   LSTM, gates i,f,z,o:  i,f,o = sigmoid, z = tanh
 *       c_t = f*c_{t-1} + i*z,   h_t = o*tanh(c_t)
 *   GRU (reset-after), gates r,z,n with S = h_{t-1} R:
 *       r = sigmoid(Gx_r + S_r), u = sigmoid(Gx_z + S_z),
 *       n = tanh(Gx_n + r*S_n),  h_t = (1-u)*n + u*h_{t-1}
 *
 * Layouts (row-major, C order).  H = NH*Dh, G = 4 (LSTM) or 3 (GRU),
 * N = NH*G*Dh.
 *   x        [T][B][Din]          dtype of the call (f32 or bf16)
 *   W        [Din][NH][G][Dh]     dtype of the call; column (n*G+g)*Dh + j
 *   R        [NH][Dh][G*Dh]       dtype of the call; row m of block n multiplies h_{t-1}[n*Dh+m]
 *   b        [NH][G][Dh]          float32 (may be NULL = 0)
 *   h0, c0   [B][H]               float32 (may be NULL = 0)
 *   h_seq, c_seq, dh_seq [T][B][H] float32, holding h_1..h_T (not h_0)
 *   hT, cT, dh0, dc0, dhT, dcT [B][H] float32
 *   gx       [T][B][N]            float32 (the input projection incl. bias)
 *   dx       [T][B][Din]          float32
 *   dW, dR, db  shapes of W, R, b  float32
 * Arithmetic: bf16 calls multiply bf16 operands (x, W, R, and h_{t-1} rounded
 * to bf16 with round-to-nearest-even) with float32 accumulation; gates, cell
 * and hidden state, and every gradient stay float32.  f32 calls compute in
 * float32 throughout.
 *
 * Ownership and threading: every tensor pointer is DEVICE memory owned by the
 * caller; outputs are overwritten, never accumulated.  The library allocates
 * nothing: scratch comes from the caller's workspace of at least
 * rnn_workspace_size() bytes.  Calls only enqueue work and return
 * (asynchronous, stream-ordered on `stream`).  Some (the chunked forward and
 * the bf16 backward) run part of their work on up to two streams the library
 * creates per device on first use (default priority), forked from `stream`
 * and joined back into it by events, so everything a call does is ordered
 * after the work queued on `stream` before it and before the work queued on
 * `stream` after it.  The library's only global mutable state is a lazily
 * filled, lock-protected cache of device properties and those streams, so
 * calls may come from several host threads.  Two calls in flight at once
 * must not share a workspace.
 *
 * Errors: every function returns a status; nothing aborts and no C++
 * exception crosses this boundary.  Arguments are validated before anything
 * is enqueued (then nothing was enqueued): NULL required pointers, non-positive
 * dims, pointers not 16-byte aligned, unsupported shapes, a workspace that is
 * too small.  A failing launch returns RNN_ERR_HIP.  Kernels that span several
 * compute units per head wait on each other at every step with a bounded
 * spin; if a wait ever runs out they record it in the workspace and finish,
 * and rnn_workspace_status() reports RNN_ERR_BARRIER_TIMEOUT.
 */
#ifndef RNN355_H
#define RNN355_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int T;    /* time steps (>= 1) */
    int B;    /* batch rows (>= 1) */
    int Din;  /* input features (>= 1) */
    int NH;   /* heads (>= 1) */
    int Dh;   /* hidden units per head (>= 1) */
} rnn_dims;

typedef enum { RNN_F32 = 0, RNN_BF16 = 1 } rnn_dtype;

typedef enum {
    RNN_OK = 0,
    RNN_ERR_INVALID_ARG = 1,     /* NULL / misaligned pointer, dims <= 0, bad enum */
    RNN_ERR_UNSUPPORTED = 2,     /* shape this build has no kernel for */
    RNN_ERR_WORKSPACE = 3,       /* ws NULL or ws_bytes < rnn_workspace_size() */
    RNN_ERR_HIP = 4,             /* a HIP runtime call failed */
    RNN_ERR_BARRIER_TIMEOUT = 5  /* a multi-CU step wait ran out (see above) */
} rnn_status;

typedef enum {
    RNN_OP_FWD_LSTM = 0,
    RNN_OP_FWD_GRU = 1,
    RNN_OP_BWD_LSTM = 2,
    RNN_OP_BWD_GRU = 3,
    RNN_OP_REC_LSTM = 4,   /* rnn_rec_lstm alone (no input projection) */
    RNN_OP_REC_GRU = 5     /* rnn_rec_gru alone */
} rnn_op;

/* Human-readable name of a status code (static storage, never NULL). */
const char *rnn_status_str(rnn_status s);

/* Bytes of workspace `op` needs at these dims and dtype; 0 if the arguments
 * are invalid or unsupported (the call itself then says which).  Pure host
 * function: touches no device. */
size_t rnn_workspace_size(rnn_op op, const rnn_dims *d, rnn_dtype dt);

/* Write a one-line description of the kernel plan `op` would use (kernel,
 * rows per workgroup, workgroups, workgroups per head; for the forward
 * whether the projection runs fused with the recurrence; for the backward
 * the reverse sweep's kernel, the compute units it leaves free and the time
 * chunks it runs in) into buf.  Pure host function apart from reading the
 * device's compute-unit count once. */
rnn_status rnn_plan_describe(rnn_op op, const rnn_dims *d, rnn_dtype dt,
                             char *buf, size_t len);

/*
 * Input projection for all steps at once (FlashRNN abstract: the input part
 * of every gate depends only on x_t, so it is one dense contraction over all
 * T*B rows; the recurrence then only adds h_{t-1} R):
 *   gx[m][c] = b[c] + sum_k x[m][k] * W[k][c],   m < M = T*B, c < N
 * x [M][K], W [K][N] in dtype dt; b [N] float32 or NULL; gx [M][N] float32.
 * bf16 needs K % 8 == 0 and N % 8 == 0.
 */
rnn_status rnn_input_proj(int M, int K, int N, rnn_dtype dt,
                          const void *x, const void *W, const float *b,
                          float *gx, hipStream_t stream);

/*
 * The same contraction with the weights given transposed, Wt [N][K] (k
 * contiguous, as a layer would keep them): gx[m][c] = b[c] + sum_k x[m][k]
 * Wt[c][k].  bf16 only, K % 32 == 0 (else RNN_ERR_UNSUPPORTED).  Both
 * operands are then read k-major straight into LDS; this is the kernel the
 * fused forward uses after staging W transposed in its workspace, and its
 * sums are bitwise those of rnn_input_proj (same k order).
 */
rnn_status rnn_input_proj_t(int M, int K, int N, rnn_dtype dt,
                            const void *x, const void *Wt, const float *b,
                            float *gx, hipStream_t stream);

/*
 * The sequential LSTM recurrence alone, given gx from rnn_input_proj
 * (blog.hotdry.top 2025-09-21: the per-step dependency is the bottleneck; R
 * stays resident on chip for all steps):
 *   A_t = gx_t + h_{t-1} R (block-diagonal), then the LSTM gate update.
 * gx [T][B][N] float32; R in dtype dt; outputs as in rnn_fwd_lstm.
 * h_seq, c_seq may be NULL (then only hT, cT are written); hT, cT required.
 */
rnn_status rnn_rec_lstm(const rnn_dims *d, rnn_dtype dt, const float *gx,
                        const void *R, const float *h0, const float *c0,
                        float *h_seq, float *c_seq, float *hT, float *cT,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the LSTM
 * recurrence of rnn_rec_lstm, same arguments, same kernels and the same
 * result bits, but with no workspace.  Its scratch (status word, exchange
 * slots of the multi-CU plan, R^T of the split-R plan) is a device array
 * inside the library of RNN_REC_NOALLOC_MAX_BYTES per GPU, held until the
 * process ends; shapes whose rnn_workspace_size(RNN_OP_REC_LSTM, ...) is
 * larger are rejected with RNN_ERR_WORKSPACE before anything is enqueued.
 * The call makes no hipMalloc / hipFree and no allocating library call.
 * dev_status (device memory, 4 bytes, 16-byte aligned, may be NULL)
 * receives, in stream order, 0 or 1 if a step wait of this call gave up
 * (what rnn_workspace_status reports as RNN_ERR_BARRIER_TIMEOUT).
 * All calls on one GPU share its array: calls that overlap in time on one
 * GPU (other streams, other host threads) race and their results are void.
 */
#define RNN_REC_NOALLOC_MAX_BYTES ((size_t)8 << 20)
rnn_status rnn_rec_lstm_noalloc(const rnn_dims *d, rnn_dtype dt, const float *gx,
                                const void *R, const float *h0, const float *c0,
                                float *h_seq, float *c_seq, float *hT, float *cT,
                                unsigned *dev_status, hipStream_t stream);

/* The GRU recurrence alone, given gx (bias inside gx).  h_seq may be NULL. */
rnn_status rnn_rec_gru(const rnn_dims *d, rnn_dtype dt, const float *gx,
                       const void *R, const float *h0,
                       float *h_seq, float *hT,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Multi-head LSTM forward: rnn_input_proj into the workspace, then
 * rnn_rec_lstm.  h_seq, c_seq [T][B][H] may be NULL; hT, cT required.
 *
 * When the recurrence runs one workgroup per (head, batch tile) on at most
 * half the compute units (bf16, Dh = 128, Din % 32 == 0) and the projection
 * has more than two waves of 256x256 output tiles for the remaining units,
 * the two phases run as one launch: its first workgroups compute the
 * projection in time order and mark finished 256-row panels of gx, the rest
 * run the recurrence and wait for the panels of their next steps.
 * Workgroups start in index order, so the projection never waits behind the
 * recurrence, also when kernels are serialised (profilers).  Results are
 * bitwise those of the serial order.  The environment variable
 * RNN355_PIPELINE=0 forces the serial order, =1 the single launch wherever
 * the first condition holds.  A panel wait that runs out (RNN355_SPIN_LIMIT
 * polls) sets the workspace's timeout word instead of hanging
 * (rnn_workspace_status).
 */
rnn_status rnn_fwd_lstm(const rnn_dims *d, rnn_dtype dt,
                        const void *x, const void *W, const void *R,
                        const float *b, const float *h0, const float *c0,
                        float *h_seq, float *c_seq, float *hT, float *cT,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* Multi-head GRU forward (reset-after).  h_seq may be NULL; hT required. */
rnn_status rnn_fwd_gru(const rnn_dims *d, rnn_dtype dt,
                       const void *x, const void *W, const void *R,
                       const float *b, const float *h0,
                       float *h_seq, float *hT,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The recurrence's plan as an integer constraint problem (FlashRNN card,
 * paperdance.org/p/2412.07752, abstract: tiling from polyhedral-like
 * integer constraints with divisibility, solved as an integer CSP; blog.
 * hotdry.top 2025-09-21, paragraph on hardware-aware auto-tuning: register
 * total, SRAM size and matrix-unit tile in, tiling out).  Every assignment
 * of the plan variables for the recurrence of `op` on d: its family, its
 * integers, the first constraint it breaks (0 if none) and the predicted
 * time.  The forward and recurrence calls run the candidate *chosen
 * returns.  num_cu <= 0: the current device's compute units.  The
 * RNN355_REC_BT / _K / _KCW / _WIDE=0 overrides act as fixed variables.
 * Writes min(n, max_out) candidates to out (out may be NULL with max_out
 * 0), the number enumerated to *n_out and the chosen index to *chosen (-1
 * and RNN_ERR_UNSUPPORTED if no candidate is feasible).  Host only.
 */
typedef struct rnn_plan_candidate {
    int family;           /* 1 one CU per (head, rows), R in VGPRs; 2 one CU per (head,
                             row), R split over AGPRs, VGPRs, LDS; 3 several CUs per head;
                             4 R in LDS */
    int rows_per_wg;      /* BT */
    int wg_per_head;      /* workgroups per (head, row tile) */
    int blocks_per_wg;    /* 16-unit blocks */
    int k_splits;         /* waves per block (k-range splits) */
    int kchunks_per_wave; /* 32-deep k-chunks per wave */
    int row_slots;        /* register row slots per lane */
    int frags_agpr, frags_vgpr, frags_lds;  /* family 2: R fragments per wave */
    int waves;            /* per workgroup */
    int grid;             /* workgroups */
    int r_vgpr;           /* VGPRs per wave holding R */
    int wg_per_cu;        /* workgroups that fit on one CU at once */
    int xcd_local;        /* family 3: the head tile's workgroups are numbered to run on
                             one XCD and exchange through its L2 (each launch checks
                             the placement; a spread group exchanges through memory) */
    long long lds_bytes;  /* per workgroup */
    int feasible;
    int violated;         /* 1 not compiled, 2 divisibility, 3 registers, 4 LDS,
                             5 residency, 6 batch, 7 override */
    double ns_per_step;   /* predicted */
    double ns_total;      /* predicted, T steps */
} rnn_plan_candidate;
rnn_status rnn_plan_search(rnn_op op, const rnn_dims *d, rnn_dtype dt, int num_cu,
                           rnn_plan_candidate *out, int max_out, int *n_out, int *chosen);

/*
 * Stacked layers (blog.hotdry.top 2025-09-21, the list of framework-level
 * optimisations, first item: multi-layer RNNs).  Layer l > 0 takes layer
 * l-1's output sequence h_1..h_T as its input x (width H = NH*Dh; in bf16
 * runs rounded to bf16, nearest-even, as x is); every layer has its own
 * weights and initial state:
 *   W, R, b: host arrays of L device pointers; W[0] is [Din][N], W[l>0] is
 *            [H][N]; R[l] as in rnn_fwd_lstm; b itself or any b[l] may be NULL.
 *   h0, c0:  [L][B][H] float32 or NULL (zeros).
 *   h_seq, c_seq: the last layer's [T][B][H], may be NULL.
 *   hT, cT:  every layer's final states, [L][B][H], required.
 * 1 <= L <= 64.  Where the recurrence runs one batch row per workgroup
 * (bf16, Dh = 128, 2*NH*B + 32 <= compute units), layers run two at a time
 * in one launch: layer l+1's input projection and recurrence start on each
 * block of 256 rows of (t, b) as soon as layer l has produced it, on the
 * compute units layer l leaves free.  Other layers run one after the other
 * on `stream`, each as rnn_fwd_lstm would.  The results are the same bits
 * either way (RNN355_STACK_OVERLAP=0 forces the second).  Intermediate
 * sequences live in the workspace (rnn_workspace_size_stack, independent of
 * L); a bounded wait that gave up in any layer is reported by
 * rnn_workspace_status.  Errors as rnn_fwd_lstm.
 */
size_t rnn_workspace_size_stack(rnn_op op /* RNN_OP_FWD_LSTM or RNN_OP_FWD_GRU */,
                                const rnn_dims *d, int L, rnn_dtype dt);
rnn_status rnn_fwd_lstm_stack(const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                              const void *const *W, const void *const *R,
                              const float *const *b, const float *h0, const float *c0,
                              float *h_seq, float *c_seq, float *hT, float *cT,
                              void *ws, size_t ws_bytes, hipStream_t stream);
/* Stacked GRU layers, as rnn_fwd_lstm_stack without cell states. */
rnn_status rnn_fwd_gru_stack(const rnn_dims *d, int L, rnn_dtype dt, const void *x,
                             const void *const *W, const void *const *R,
                             const float *const *b, const float *h0,
                             float *h_seq, float *hT,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Long sequences (blog.hotdry.top 2025-09-21, the list of framework-level
 * optimisations, third item: memory use for long sequences and trading
 * compute for it by checkpointing).  Both calls work on chunks of `chunk`
 * time steps (chunk >= 1; the last chunk may be shorter; chunk >= T is one
 * chunk), so their workspace (rnn_workspace_size_chunked) grows with chunk,
 * not with T.
 *
 * rnn_fwd_lstm_chunked: the forward of rnn_fwd_lstm, chunk after chunk,
 * each chunk starting from the previous one's final state; the input
 * projection of a later chunk runs beside the recurrence of the current
 * one (on a second stream of the library's that joins `stream`).  Results
 * are the same bits as rnn_fwd_lstm.  h_ckpt, c_ckpt: NULL (both), or
 * [ceil(T/chunk)][B][H] float32 receiving the state at the last step of
 * every chunk (h_{k*chunk-1} for k = 1, 2, ...; the last entry equals hT).
 * Arguments otherwise as rnn_fwd_lstm.
 *
 * rnn_bwd_lstm_ckpt: the gradients of rnn_bwd_lstm without h_seq and c_seq:
 * segments of `chunk` steps are processed from the last to the first; each
 * segment's h and c are recomputed from the state before it (h0, c0 for
 * the first segment, else the previous segment's checkpoint, as
 * rnn_fwd_lstm_chunked with the same chunk writes them), then BPTT runs
 * over the segment with the gradients the later segment passes back.  dx,
 * dh0 and dc0 are the same bits as rnn_bwd_lstm; dW, dR and db are summed
 * segment by segment (float32 rounding differs).  h_ckpt and c_ckpt are
 * required when chunk < T.  dtype support as rnn_bwd_lstm.
 */
size_t rnn_workspace_size_chunked(rnn_op op /* RNN_OP_FWD_* or RNN_OP_BWD_* */,
                                  const rnn_dims *d, int chunk, rnn_dtype dt);
rnn_status rnn_fwd_lstm_chunked(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                                const void *W, const void *R, const float *b,
                                const float *h0, const float *c0,
                                float *h_seq, float *c_seq, float *hT, float *cT,
                                float *h_ckpt, float *c_ckpt,
                                void *ws, size_t ws_bytes, hipStream_t stream);
/* GRU forward in chunks, as rnn_fwd_lstm_chunked without cell states. */
rnn_status rnn_fwd_gru_chunked(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                               const void *W, const void *R, const float *b,
                               const float *h0, float *h_seq, float *hT, float *h_ckpt,
                               void *ws, size_t ws_bytes, hipStream_t stream);
rnn_status rnn_bwd_lstm_ckpt(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                             const void *W, const void *R, const float *b,
                             const float *h0, const float *c0,
                             const float *h_ckpt, const float *c_ckpt,
                             const float *dh_seq, const float *dhT, const float *dcT,
                             float *dx, float *dW, float *dR, float *db,
                             float *dh0, float *dc0,
                             void *ws, size_t ws_bytes, hipStream_t stream);
/* GRU BPTT from checkpoints, as rnn_bwd_lstm_ckpt without cell states. */
rnn_status rnn_bwd_gru_ckpt(const rnn_dims *d, rnn_dtype dt, int chunk, const void *x,
                            const void *W, const void *R, const float *b,
                            const float *h0, const float *h_ckpt,
                            const float *dh_seq, const float *dhT,
                            float *dx, float *dW, float *dR, float *db, float *dh0,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Multi-head LSTM backpropagation through time for the loss
 *   L = sum_t dh_seq[t] . h_t + dhT . h_T + dcT . c_T
 * given the forward's h_seq and c_seq (from rnn_fwd_lstm on the same inputs).
 * dhT, dcT may be NULL (= 0).  Writes dx, dW, dR, db, dh0, dc0 (all required).
 * Gate pre-activations are recomputed from x, W, b, h_seq and R.  (FlashRNN
 * card, abstract: the LSTM trained through its sequential recurrence; the
 * backward is the reverse-time recurrence of the same cell, with the same
 * block-diagonal R, held resident as R^T.)
 * bf16 calls: Dh % 16 == 0; the gate gradients are rounded to bf16 only as
 * operands of the dx, dW, dR contractions.  f32 calls: every intermediate
 * stays float32 (pre-activations, gate gradients, carries, contractions);
 * the head's R block in float32 must fit one CU's LDS (Dh <= 96 for the
 * LSTM, else RNN_ERR_UNSUPPORTED), and the workspace is sized per dtype.
 * bf16 calls with T >= 256 whose reverse sweep leaves at least 64 CUs free
 * run the sweep in up to four time chunks (of at least 128 steps), the last
 * one first, and each chunk's dx, dW, dR and db contractions on the
 * library's two streams beside the next chunk's sweep: dx, dh0 and dc0 are
 * the same bits as with the sweep in one piece, dW, dR and db add the
 * chunks' shares in chunk order (environment RNN355_BWD_OVERLAP=0: one
 * piece).
 */
rnn_status rnn_bwd_lstm(const rnn_dims *d, rnn_dtype dt,
                        const void *x, const void *W, const void *R,
                        const float *b, const float *h0, const float *c0,
                        const float *h_seq, const float *c_seq,
                        const float *dh_seq, const float *dhT, const float *dcT,
                        float *dx, float *dW, float *dR, float *db,
                        float *dh0, float *dc0,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Multi-head GRU (reset-after) backpropagation through time (FlashRNN card,
 * abstract: GRU among the cells the kernels cover) for the loss
 *   L = sum_t dh_seq[t] . h_t + dhT . h_T
 * given the forward's h_seq (from rnn_fwd_gru on the same inputs).  dhT may
 * be NULL (= 0).  Writes dx, dW, dR, db, dh0 (all required).  The gate
 * inputs Gx = x W + b and the recurrent sums S = h_{t-1} R are recomputed
 * apart (the candidate gate scales S_n by r); per step t = T-1 .. 0, with
 * dh = dh_seq[t] + the carry:
 *   dA_n = dh (1-u)(1-n^2),  dA_z = dh (h_{t-1} - n) u(1-u),
 *   dA_r = dA_n S_n r(1-r),
 *   dGx = (dA_r, dA_z, dA_n) -> dW, dx, db;  dS = (dA_r, dA_z, dA_n r) -> dR,
 *   carry = dh u + dS R^T (block-diagonal R).
 * bf16 calls: Dh % 16 == 0 and 3*Dh % 32 == 0; f32 calls as for
 * rnn_bwd_lstm (the float32 R block must fit one CU's LDS).  Same workspace
 * and stream rules as rnn_bwd_lstm.
 */
rnn_status rnn_bwd_gru(const rnn_dims *d, rnn_dtype dt,
                       const void *x, const void *W, const void *R,
                       const float *b, const float *h0, const float *h_seq,
                       const float *dh_seq, const float *dhT,
                       float *dx, float *dW, float *dR, float *db, float *dh0,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Synchronises `stream`, then reports whether a kernel of the last call that
 * used `ws` recorded a step-wait timeout (RNN_ERR_BARRIER_TIMEOUT) or not
 * (RNN_OK).  `ws` must be the workspace that call used.
 */
rnn_status rnn_workspace_status(const void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RNN355_H */
