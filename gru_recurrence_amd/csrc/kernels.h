// kernels.h -- argument blocks and launchers of the librnn355 kernels
// (internal; the public interface is include/rnn355.h).
#pragma once

#include <cstdlib>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnn355 {

// bf16 MFMA contraction, see gemm.hip.  Operand element (r,k) sits at
// P[r*ld + k] ("k-major") or P[k*ld + r] ("r-major").  Batched over
// blockIdx.z with element strides stride*.
struct GemmArgs {
    int M, N, K;
    const uint16_t *A;
    long lda, strideA;
    const uint16_t *B;
    long ldb, strideB;
    const float *bias;  // [N] or nullptr
    float *C;
    long ldc, strideC;
    int accumulate;           // C += product
    uint32_t *clear_words;    // if set, block 0 zeroes 64 words (status header)
    int ksplit;               // K slices (0 or 1: none); > 1 needs `partial`
    float *partial;           // [batch][ksplit][M][N] slice partials (workspace)
    unsigned *ready;          // if set (ksplit 1, batch 1): per 256-row panel, +1 per
                              // finished column tile, released at device scope
    // Optional second K segment (k-major kernel, batch 1, no split): C(m, n)
    // also gets sum_{k < K2} A2[m*lda2 + (n/seg_n)*K2 + k] * B2[n*ldb2 + k],
    // i.e. column block n/seg_n of the output takes its own K2 columns of A2
    // (a block-diagonal right operand).  seg_n is a multiple of the column tile.
    const uint16_t *A2, *B2;
    long lda2, ldb2;
    int K2, seg_n;
};
constexpr int kGemmRowTile = 256;  // rows per output tile of the bf16 contraction
constexpr int kGemmColTile = 256;  // columns per output tile
// Dynamic LDS of a workgroup of the pipelined forward: the projection's ring
// of four 32 KiB K tiles, and more for the ring of a recurrence workgroup's
// head start (with the recurrence's own 8.5 KiB, within the CU's 160 KiB).
constexpr int kFusedLdsBytes = 144 * 1024;
// Rows of gx a recurrence workgroup computes at most in its head start.
constexpr int kHeadStartRows = 64;


// Largest useful K split (a power of two <= what fills num_cu CUs, keeping
// >= 8 K tiles per slice) and the partial-buffer bytes it needs.
int gemm_splitk_for(int M, int N, int K, int batch, int num_cu);
size_t gemm_partial_bytes(int M, int N, int batch, int ksplit);
constexpr int kMaxSplitK = 8;

// float32 contraction with explicit strides: A(m,k) = A[m*sam + k*sak],
// B(k,n) = B[k*sbk + n*sbn].
struct GemmF32Args {
    int M, N, K;
    const float *A;
    long sam, sak, strideA;
    const float *B;
    long sbk, sbn, strideB;
    const float *bias;
    float *C;
    long ldc, strideC;
    int accumulate;
    uint32_t *clear_words;
};

hipError_t launch_gemm_bf16(const GemmArgs &g, bool a_kmajor, bool b_kmajor, int batch,
                            hipStream_t s);
// Sums the split-K partials of g into g.C (after a launch with ksplit > 1).
hipError_t launch_splitk_reduce(const GemmArgs &g, int batch, hipStream_t s);

// Both operands k-major, K % 32 == 0: tiles streamed into LDS by direct
// global-to-LDS loads (gemm_dma.hip).  B(n,k) = B[n*ldb + k].
bool gemm_dma_ok(int K);
// max_wg > 0: at most that many workgroups, each looping over output tiles
// (leaves compute units to a kernel running beside it; a multiple of 8
// keeps a row tile's column tiles on one XCD).
hipError_t launch_gemm_dma(const GemmArgs &g, int batch, hipStream_t s, int max_wg = 0);
// dst[b][c][r] = src[b][r][c], bf16 [R][C] matrices, `batch` of them; the
// same launch zeroes nclear words at `clear` and nclear2 at `clear2` (if set)
// and, if src1 is set, transposes a second batch (src1 -> dst1, [R1][C1]).
hipError_t launch_transpose_bf16(const uint16_t *src, uint16_t *dst, int R, int C, int batch,
                                 hipStream_t s, unsigned *clear = nullptr, long nclear = 0,
                                 unsigned *clear2 = nullptr, long nclear2 = 0,
                                 const uint16_t *src1 = nullptr, uint16_t *dst1 = nullptr,
                                 int R1 = 0, int C1 = 0, int batch1 = 0);
hipError_t launch_gemm_f32(const GemmF32Args &g, int batch, hipStream_t s);

// Forward recurrence (rec_fwd.hip).
struct RecArgs {
    int T, B, NH, Dh, BT;     // BT: batch rows per workgroup
    const float *gx;          // [T][B][NH*G*Dh]
    const uint16_t *Rb;       // bf16 R (MFMA kernel / bf16 simple kernel)
    const uint16_t *Rt;       // optional, MFMA kernel: R^T per head [NH][G*Dh][Dh] bf16
    const float *Rf;          // f32 R (f32 simple kernel)
    const float *h0, *c0;
    float *h_seq, *c_seq, *hT, *cT;
    // Pipelined forward: gx is still being written by the input projection.
    // ready[p] counts the finished column tiles of row panel p (kGemmRowTile
    // rows of gx); a panel is complete at ready_target.  Null: gx complete.
    const unsigned *ready;
    unsigned ready_target;
    int panels;
    unsigned *flag;       // abort word, set when a wait runs out
    unsigned spin_limit;  // polls before a wait is declared lost
    // Head start of the pipelined forward (fused kernel only): each
    // workgroup computes gx = x W + b itself for its own rows of the first
    // hs_panels row panels (hs_steps = hs_panels * kGemmRowTile / B steps),
    // which the projection's workgroups skip.  hs_wt: W^T [N][hs_K] bf16,
    // hs_x: x [T*B][hs_K] bf16, hs_bias: b [N] or null.  0: none.
    int hs_panels, hs_steps, hs_K;
    const uint16_t *hs_x, *hs_wt;
    const float *hs_bias;
    // Kernels that never wait: if set, workgroup 0 zeroes this status word
    // at its start (no other workgroup writes it), so the call reports RNN_OK
    // on a workspace that held anything.
    unsigned *clear_word;
};

enum RecKind { kRecNone = 0, kRecMfma = 1, kRecSimple = 2 };

struct RecPlan {
    RecKind kind;
    int BT;          // rows per workgroup
    int nbt;         // batch tiles
    int grid;        // workgroups
    int threads;     // per workgroup
    int waves;       // per workgroup
    int upt;         // MFMA kernel: cell update passes per step (rows in lane groups; 1 at BT = 1)
    size_t lds;      // dynamic LDS bytes (simple kernel)
};

// Chooses the kernel and tiling for (cell, dims, dtype).  bt_override > 0
// forces the rows per workgroup.  Pure host function.
RecPlan plan_rec(int cell, int T, int B, int NH, int Dh, bool bf16, int num_cu,
                 int bt_override);


// The recurrence on a finished gx (a.ready must be null).
hipError_t launch_rec_fwd(int cell, const RecPlan &p, const RecArgs &a, bool bf16,
                          hipStream_t s);

// Pipelined forward in one launch (MFMA plan, Dh = 128 or 64, bf16, Din %
// 32 == 0): n_gemm workgroups run the k-major input projection g (with g.ready),
// p.grid more run the recurrence a waiting on a.ready.  rows1 > 0 (a
// multiple of the row tile) and n_gemm2 > 0 (a multiple of 8): the first
// rows1 rows of g on all n_gemm projection workgroups, the rest on the
// first n_gemm2 of them.  Dynamic LDS of the contraction is set up here.
hipError_t launch_fwd_fused(int cell, const RecPlan &p, const RecArgs &a, const GemmArgs &g,
                            int n_gemm, hipStream_t s, int rows1 = 0, int n_gemm2 = 0);

// Two stacked layers l, l+1 in one launch (MFMA plan with one batch row per
// workgroup, Dh = 128, bf16): rec_grid workgroups run layer l on a finished
// gx (a0), storing h_t as bf16 in h_bf0 and counting each finished step on
// done[t] (one count per workgroup, done_target = rec_grid); n_gemm workgroups
// compute layer l+1's input projection g from h_bf0 (g.A), each 256-row
// tile once the steps of its rows are counted, and count finished tiles on
// g.ready; the last rec_grid
// workgroups run layer l+1 (a1, a1.ready = g.ready) and, if h_bf1 is set,
// also store its h_t as bf16 there.  done and g.ready start at zero.
struct StackSync {
    uint16_t *h_bf0, *h_bf1;
    unsigned *done;       // [T]
    unsigned done_target;  // counts of a finished step: rec_grid
    int rec_grid, n_gemm;
};
hipError_t launch_fwd_stack2(int cell, const RecPlan &p, const RecArgs &a0, const RecArgs &a1,
                             const GemmArgs &g, const StackSync &y, hipStream_t s);

// Forward recurrence for Dh = 256 on one compute unit per (head, batch row),
// R split over AGPRs, VGPRs and LDS (rec_wide.hip).  Rt holds R transposed
// per head, [NH][G*Dh][Dh] bf16.
struct WidePlan {
    int ok;
    int grid;     // NH * B workgroups (one batch row each)
    int threads;  // 256: one wave per SIMD
    size_t lds;   // dynamic LDS bytes (R chunks read every step)
};
WidePlan plan_wide(int cell, int B, int NH, int Dh, bool bf16);
hipError_t launch_rec_wide(int cell, const WidePlan &p, const RecArgs &a, const uint16_t *Rt,
                           hipStream_t s);

// Multi-CU forward recurrence (rec_mc.hip).
struct McPlan {
    int ok;
    int K;        // workgroups per (head, batch tile)
    int nb;       // 16-unit blocks per workgroup
    int ks;       // waves per unit block (k-range splits)
    int kcw;      // k-chunks of 32 per wave (4 or 8)
    int threads;  // per workgroup
    int BT;       // batch rows per group
    int r4;       // register row slots in use
    int groups;   // (head, batch tile) groups
    int grid;     // groups * K
    size_t lds;   // dynamic LDS bytes
};

struct McArgs {
    RecArgs r;
    int K, KS, NB;
    unsigned long long *xg;  // exchange slots [groups][2][BT][Dh/2] (2 bf16 + step)
    unsigned *flag;          // time-out / abort word (cleared before every launch)
    unsigned spin_limit;  // polls of the group counter before a wait is declared lost
    // xcd_map: workgroup i serves group (i % 8) + 8 * ((i / 8) / K), member
    // (i / 8) % K (needs groups % 8 == 0), so that the members of a group are
    // the workgroups the dispatcher deals to one XCD; `xcc` ([grid] words,
    // zero before the launch) lets the members check that placement.
    unsigned *xcc;
    int xcd_map;
};
// The multi-CU kernel numbers its workgroups by XCD (McArgs::xcd_map) where
// the groups divide over the 8 XCDs and the id table fits the workspace
// header.
constexpr int kMcXcdMaxGrid = 768;
// 2..16 batch rows per multi-CU workgroup run the cell update with rows in
// lane groups (one pass per four rows) unless RNN355_MC_ROWLANES=0 keeps
// them in register slots (one pass per register slot).
inline bool mc_row_lanes(int bt) {
    if (bt < 2 || bt > 16) return false;
    const char *e = getenv("RNN355_MC_ROWLANES");
    return !e || atoi(e) != 0;
}

inline bool mc_xcd_grouping(int groups, int grid) {
    return groups > 0 && groups % 8 == 0 && grid <= kMcXcdMaxGrid;
}

// Plan for heads of Dh >= 256, Dh % 128 == 0; ok == 0 if none fits the
// chip (every workgroup must be resident at once).  kcw: k-chunks of 32
// per wave (4 or 8; 0: 8 where it divides Dh/32).  Pure host function.
McPlan plan_mc(int cell, int B, int NH, int Dh, int num_cu, int bt_override, int k_override,
               int kcw = 0);

// Ordinary launch of a grid whose workgroups wait on one another, after a
// host check that the whole grid is resident at once (api.hip); returns
// hipErrorCooperativeLaunchTooLarge if it is not.
hipError_t launch_all_resident(const void *fn, int grid, int threads, void **args, size_t lds,
                               hipStream_t s);

// Clears the exchange slots and (if clear_flag) the abort word, then
// launches the grid with every workgroup resident.
hipError_t launch_rec_mc(int cell, const McPlan &p, const McArgs &m, hipStream_t s,
                         bool clear_flag = true);

// The recurrence's plan as an integer constraint problem (plan_search.hip):
// every assignment of the plan variables, the first constraint it breaks
// (kPlanOk if none) and the predicted time.  Pure host function.
enum PlanFamily { kFamResident = 1, kFamWide = 2, kFamMultiCu = 3, kFamLds = 4 };
enum PlanViolation {
    kPlanOk = 0,
    kPlanNotInstantiated = 1,  // no compiled kernel for these values
    kPlanDivisibility = 2,
    kPlanRegisters = 3,
    kPlanLds = 4,
    kPlanResidency = 5,        // not every workgroup resident at once
    kPlanBatch = 6,            // more rows per workgroup than the batch or the MFMA holds
    kPlanFixed = 7,            // excluded by an override
};
struct PlanCand {
    int family;
    int BT, K, nb, ks, kcw, r4;  // rows, workgroups per head tile, 16-unit blocks, k splits,
                                 // k-chunks per wave, row slots per lane
    int fa, fv, fl;              // split R: fragments per wave in AGPRs, VGPRs, LDS
    int waves, grid, r_vgpr;     // waves per workgroup, workgroups, VGPRs per wave holding R
    int wg_per_cu;               // workgroups that fit on one CU at once
    int xcd_local;               // multi-CU: groups exchange through one XCD's L2
    long lds;                    // LDS bytes per workgroup
    int feasible, violated;
    double ns_step, ns_total;    // predicted per-step latency, T steps
};
// Overrides (0: free): rows per workgroup, workgroups per head tile, k-chunks
// per wave; no_wide excludes the split-R family; no_xcd prices the multi-CU
// exchange through memory everywhere.
struct PlanFix {
    int bt, k, kcw;
    bool no_wide;
    bool no_xcd;  // multi-CU groups exchange through memory even where they could share an L2
};
constexpr int kPlanMaxCands = 512;
// Writes up to cap candidates to buf, the fastest feasible one's index to
// *best (-1 if none); returns the number enumerated.
int plan_search(int cell, int T, int B, int NH, int Dh, bool bf16, int cus, const PlanFix &fix,
                PlanCand *buf, int cap, int *best);

// LSTM backward (rec_bwd.hip).
struct BwdPlan {
    int ok;
    int K, nb, ks, kcw, threads, BT, r4, nbt, groups, grid;
    size_t lds;
};

struct BwdArgs {
    int T, B, NH, Dh, BT, K, KS, NB;
    // LSTM: recomputed pre-activations A = Gx + h_{t-1} R [T][B][NH*4*Dh].
    // GRU: Gx (x W + b) alone [T][B][NH*3*Dh], the recurrent sums in S.
    const float *A;
    const float *S;          // GRU: h_{t-1} R [T][B][NH*3*Dh]
    const float *c_seq;      // LSTM: [T][B][H]
    const float *c0;         // LSTM: [B][H] or null
    const float *h_seq;      // GRU: [T][B][H] (h_{t-1} of the update gate)
    const float *h0;         // GRU: [B][H] or null
    const float *dh_seq;     // [T][B][H]
    const float *dhT, *dcT;  // [B][H] or null (dcT: LSTM)
    const uint16_t *Rb;      // bf16 R
    uint16_t *dA;            // bf16 gradients of the gate inputs Gx [T][B][N]
    uint16_t *dS;            // GRU: bf16 gradients of the recurrent sums (dR, carry)
    float *db_part;          // [nbt][N]
    float *dh0, *dc0;        // [B][H] (dc0: LSTM)
    unsigned long long *xg;  // exchange slots [groups][2][BT][G*Dh/2]
    unsigned *flag;
    unsigned spin_limit;
    unsigned *xcc;  // as McArgs: members of a group numbered by XCD, checked
    int xcd_map;    // through this table of workgroup XCDs ([grid] words)
    int keep_flag;  // nonzero: the launch leaves the status word as it stands
};

// Float32 backward (rec_bwd_f32.hip): float32 operands, pre-activations,
// gate gradients and carries throughout.
struct BwdF32Args {
    int T, B, NH, Dh, BT;
    const float *A;       // LSTM: x W + b + h_{t-1} R; GRU: x W + b   [T][B][N]
    const float *S;       // GRU: h_{t-1} R                          [T][B][N]
    const float *c_seq;   // LSTM [T][B][H]
    const float *c0;      // LSTM [B][H] or null
    const float *hprev;   // GRU: h_{t-1} [T][B][H]
    const float *dh_seq;  // [T][B][H]
    const float *dhT, *dcT;
    const float *R;       // [NH][Dh][G Dh]
    float *dA;            // gradients of the gate inputs (GRU: of Gx)  [T][B][N]
    float *dS;            // GRU: gradients of the recurrent sums        [T][B][N]
    float *dh0, *dc0;
};
struct BwdF32Plan {
    int ok, BT, nbt;
    size_t lds;
};
constexpr size_t kBwdF32MaxLds = 160u * 1024u;
// Rows per workgroup such that the head's R (float32) and the tile's
// gradients fit the LDS; ok == 0 if R alone does not.  Pure host function.
BwdF32Plan plan_bwd_f32(int cell, int B, int Dh);
hipError_t launch_rec_bwd_f32(int cell, const BwdF32Plan &p, const BwdF32Args &a, hipStream_t s);
hipError_t launch_hprev_f32(const float *h0, const float *h_seq, float *hprev, long BH, long MH,
                            hipStream_t s);
hipError_t launch_colsum_f32(const float *X, long M, int N, float *out, bool accumulate,
                             hipStream_t s);

BwdPlan plan_bwd(int cell, int B, int NH, int Dh, int num_cu, int bt_override, int k_override);
hipError_t launch_rec_bwd(int cell, const BwdPlan &p, const BwdArgs &m, hipStream_t s);
// Reverse sweep of the backward for Dh = 256 on the same layout (one
// workgroup per (head, batch row); db partials per batch row).  Uses the
// fields of BwdArgs that the cell backward reads; K, KS, NB, BT, xg, flag
// and spin_limit are ignored.  The plan is plan_wide's (its lds is the
// forward's; the launcher sets its own).
hipError_t launch_rec_bwd_wide(int cell, const WidePlan &p, const BwdArgs &m, hipStream_t s);
// The Dh = 256 reverse sweep on two CUs per (head, batch row) (2 NH B
// workgroups, all resident; m.xcd_map needs NH B % 8 == 0): each holds half
// of R in AGPRs and the two swap partial carries every step.
hipError_t launch_rec_bwd_wide2(int cell, const BwdArgs &m, hipStream_t s);
hipError_t launch_hprev_bf16(const float *h0, const float *h_seq, uint16_t *hprev, long BH,
                             long total, hipStream_t s);
// db = (db if accumulate) + sum over batch tiles of db_part.
hipError_t launch_db_reduce(const float *db_part, int nbt, int N, float *db, hipStream_t s,
                            bool accumulate = false);

}  // namespace rnn355
