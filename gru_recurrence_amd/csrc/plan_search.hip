// plan_search.hip -- the recurrence's launch plan as an integer constraint
// problem (host code only).
//
// FlashRNN card (paperdance.org/p/2412.07752), abstract: the kernels'
// tiling is chosen by modelling the hardware with polyhedral-like integer
// constraints, including divisibility, and solving the resulting integer
// CSP.  GPU-perspective blog (blog.hotdry.top, 2025-09-21), paragraph on
// hardware-aware auto-tuning: the inputs are the register total, the SRAM
// size and the smallest matrix-unit tile, the outputs the tiling.
//
// Here the same idea for gfx950 and the kernels of this library.  The
// integer variables of one plan:
//   family  one CU per (head, row tile) with R resident in VGPRs; one CU
//           per (head, row) with R split over AGPRs, VGPRs and LDS
//           (Dh = 256); several CUs per head exchanging h every step; the
//           LDS kernel (R in LDS, any precision)
//   BT      batch rows per workgroup, r4 register row slots per lane
//   K       workgroups per (head, row tile), nb 16-unit blocks each
//   ks      waves per block (k-range splits), kcw 32-wide k-chunks per wave
//   fa, fv, fl  R fragments (16x32 bf16 B tiles) per wave in AGPRs, VGPRs
//           and LDS
// and the constraints, each with its source:
//   divisibility  Dh = 16 nb K (16-unit MFMA blocks), Dh/32 = kcw ks
//                 (32-deep MFMA k-chunks), G*Dh/16 tiles in groups of 4
//   registers     a wave addresses 256 VGPRs and 256 AGPRs; two waves per
//                 SIMD share 512; R's fragments take 4 registers each and
//                 must stay resident (at most 128 VGPRs of a wave for R
//                 next to the step's working set)
//   LDS           160 KiB per CU (64 KiB for the LDS kernel's one
//                 dynamic allocation)
//   residency     the multi-CU kernel needs every workgroup resident
//                 (grid <= CUs); other families run rounds of the grid
//   instantiation only the variants the library compiles (head sizes,
//                 kcw, row slots, the split-R fragment split)
//   batch         BT <= B and BT <= 16 (the MFMA's 16 rows)
// The objective is the predicted time of T steps: a per-step latency model
// whose constants are gfx950 measurements of these kernels (issue time of
// v_mfma_f32_16x16x32_bf16, the cell update per row slot, the cross-CU
// exchange, the k-split reduction, the split-R reduction, the LDS kernel's
// dot products), scaled by occupancy: workgroups that fit on one CU
// together (registers per wave as the compiler reports them for these
// kernels, LDS) run side by side, each step 35% slower per extra
// workgroup, and the rest of the grid in further rounds.  The search
// enumerates every assignment (a few hundred at most), keeps the feasible
// ones, and takes the fastest (exact ties: fewer workgroups).
#include <algorithm>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace rnn355 {

namespace {

// Measured on one MI355X (bench.py and cycle-counter probes of these
// kernels; see the calibration in the design notes).
constexpr double kMfmaNs = 7.95;          // one 16x16x32 bf16 MFMA issued per SIMD
constexpr double kGateNs[3] = {61.5, 136.5, 261.5};  // cell update per gate, 1/2/4 row slots
constexpr double kResLanesNs = 101.5;     // ... rows in lane groups (one CU), per gate
constexpr double kResLanesPassNs = 50.0;  // ... per further pass of four rows
constexpr double kResLanesRowNs = 8.4;    // ... per gate and row (Gx and outputs of a row)
constexpr double kGateLanesNs = 100.0;    // ... rows in lane groups (multi-CU), per gate
constexpr double kGateLanesPassNs = 150.0; // ... per further pass of four rows
constexpr double kGatherRoundNs = 400.0;  // multi-CU: per further poll round of the gather
constexpr double kWideRowsNs = 250.0;     // more than 8 rows of a tile: second row half
constexpr double kExchangeNs = 1480.0;    // cross-CU step exchange (flag-in-data words)
constexpr double kExchangeLocalNs = 580.0; // ... base when a group's members share one XCD's L2
constexpr double kExchangePerWgNs = 10.0; // ... per workgroup of the head
constexpr double kExchangePerValNs = 0.05; // ... per h value gathered (Dh x BT)
constexpr double kSplitBaseNs = 350.0;    // k-split partial sums through LDS + barrier
constexpr double kSplitPerWaveNs = 50.0;
constexpr double kWideBaseNs = 547.0;     // split R: partial-sum packing, reduction, cell
constexpr double kWideLdsFragNs = 4.8;    // ... per R fragment read from LDS
constexpr double kLdsBaseNs = 415.0;      // LDS kernel: barriers and cell update
constexpr double kLdsDotNs = 37.6;        // ... per k of a dot product pass
constexpr double kShareSlowdown = 0.35;   // per extra workgroup sharing a CU
// The one variant whose spills sit in the step loop (compiler report: 223
// VGPRs spilled): LSTM, several CUs per head, kcw 8, four row slots in the
// register-slot layout (the lane-group layout keeps only a few reloads).
// Fitted to 1.5-3.0 us per step more than the lane-group layout measured at
// the same shapes.
constexpr double kSpillBoundNs = 2000.0;

constexpr int kVgprWave = 256, kAgprWave = 256, kRegsSimd = 512, kSimds = 4;
constexpr int kRVgprMax = 128;
constexpr long kLdsCu = 160 * 1024, kLdsSimple = 64 * 1024;
constexpr int kWideFragsAgprMax = kAgprWave / 4;  // 64
constexpr int kWideWorkVgpr = 128;                // the split-R step's own VGPRs

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Registers per wave (VGPRs + AGPRs) of the one-CU MFMA kernel as the
// compiler reports them, [cell][Dh 32, 64, 128][one row; rows in lane groups
// with 1, 2 passes; four register row slots].
constexpr int kResRegs[2][3][4] = {{{88, 172, 170, 262}, {112, 188, 190, 258}, {184, 205, 212, 262}},
                                   {{70, 132, 136, 230}, {86, 146, 154, 246}, {138, 168, 174, 252}}};

// Workgroups of `waves` waves, `regs` registers each, `lds` bytes, that fit
// on one CU at once (at most 8).
int fit_per_cu(int waves, int regs, long lds) {
    const int per_simd = kRegsSimd / std::max(8, (regs + 7) / 8 * 8);
    int by_regs = kSimds * std::min(per_simd, 8) / std::max(waves, 1);
    if (lds > 0) by_regs = std::min<long>(by_regs, kLdsCu / lds);
    return std::max(1, std::min(by_regs, 8));
}
int r4_of(int bt) { return bt >= 3 ? 4 : bt; }
int r4_index(int r4) { return r4 == 1 ? 0 : r4 == 2 ? 1 : 2; }

struct Sink {
    PlanCand *buf;
    int cap, n;
    void add(const PlanCand &c) {
        if (n < cap) buf[n] = c;
        ++n;
    }
};

PlanCand blank(int family) {
    PlanCand c{};
    c.family = family;
    c.K = 1;
    c.ks = 1;
    c.feasible = 1;
    return c;
}

void fail(PlanCand &c, int why) {
    if (c.feasible) {
        c.feasible = 0;
        c.violated = why;
    }
}

void finish(PlanCand &c, int T, int cus) {
    if (c.wg_per_cu < 1) c.wg_per_cu = 1;
    const int share = std::min(c.wg_per_cu, std::max(1, ceil_div(c.grid, cus)));
    const int rounds = std::max(1, ceil_div(c.grid, (long)cus * c.wg_per_cu));
    c.ns_total = c.ns_step * T * (1.0 + kShareSlowdown * (share - 1)) * rounds;
}

// One CU per (head, BT rows), R resident in VGPRs (rec_fwd_mfma_kernel).
void family_resident(int cell, int T, int B, int NH, int Dh, bool bf16, int cus,
                     const PlanFix &fix, Sink &out) {
    const int G = cell == kLSTM ? 4 : 3;
    for (int bt = 1; bt <= 16; ++bt) {
        PlanCand c = blank(kFamResident);
        // one row: the gate-row cell update; two to eight rows: rows in lane
        // groups, one pass per four rows (r4 passes); more: four register
        // row slots
        const bool lanes = bt > 1 && bt <= 8;
        c.BT = bt;
        c.r4 = bt <= 4 ? 1 : bt <= 8 ? 2 : 4;
        c.nb = Dh / 16;
        c.kcw = Dh / 32;
        c.waves = Dh / 16;
        c.grid = NH * ceil_div(B, bt);
        c.r_vgpr = 4 * G * (Dh / 32);
        c.lds = 2L * 16 * (Dh + 8) * 2;
        const int di = Dh == 32 ? 0 : Dh == 64 ? 1 : 2;
        const int vi = bt == 1 ? 0 : lanes ? c.r4 : 3;
        c.wg_per_cu = fit_per_cu(c.waves, kResRegs[cell == kLSTM ? 0 : 1][di][vi], c.lds);
        if (!bf16 || (Dh != 32 && Dh != 64 && Dh != 128)) fail(c, kPlanNotInstantiated);
        if (Dh % 32 != 0) fail(c, kPlanDivisibility);
        if (bt > B) fail(c, kPlanBatch);
        if (c.r_vgpr > kRVgprMax || ceil_div(c.waves, kSimds) * kVgprWave > kRegsSimd)
            fail(c, kPlanRegisters);
        if (fix.bt > 0 && bt != std::min({fix.bt, 16, B})) fail(c, kPlanFixed);
        const int per_simd = ceil_div(c.waves, kSimds);
        c.ns_step = kMfmaNs * G * (Dh / 32) * per_simd +
                    G * (lanes ? kResLanesNs + kResLanesPassNs * (c.r4 - 1) + kResLanesRowNs * bt
                               : kGateNs[bt == 1 ? 0 : 2]) +
                    (bt > 8 ? kWideRowsNs : 0.0);
        finish(c, T, cus);
        out.add(c);
    }
}

// One CU per (head, row), R split over AGPRs, VGPRs and LDS (rec_wide.hip):
// the split is a variable; the compiled split is the one the budgets allow
// with the fewest LDS fragments.
void family_wide(int cell, int T, int B, int NH, int Dh, bool bf16, int cus, const PlanFix &fix,
                 Sink &out) {
    const int G = cell == kLSTM ? 4 : 3;
    const int nf = 2 * G * 16;  // fragments per wave: G*16 tiles x 2 k-chunks (Dh = 256)
    const int compiled_fl = cell == kLSTM ? 32 : 0;
    for (int fa = 0; fa <= kWideFragsAgprMax; fa += 16) {
        for (int fv = 0; fv <= 64; fv += 16) {
            PlanCand c = blank(kFamWide);
            c.BT = 1;
            c.r4 = 1;
            c.fa = fa;
            c.fv = fv;
            c.fl = nf - fa - fv;
            c.nb = Dh / 16;
            c.kcw = 2;
            c.waves = kSimds;
            c.grid = NH * B;
            c.r_vgpr = 4 * fv;
            c.lds = (long)std::max(c.fl, 0) * kSimds * 64 * 16 + 4L * G * 16 * 16 * 4 + 1024;
            c.wg_per_cu = 1;  // a wave per SIMD with all 512 registers
            if (!bf16 || Dh != 256) fail(c, kPlanNotInstantiated);
            if (c.fl < 0 || (G * Dh / 16) % 4 != 0) fail(c, kPlanDivisibility);
            if (4 * fa > kAgprWave || 4 * fv + kWideWorkVgpr > kVgprWave) fail(c, kPlanRegisters);
            if (c.lds > kLdsCu) fail(c, kPlanLds);
            if (c.feasible && (fa != kWideFragsAgprMax || c.fl != compiled_fl))
                fail(c, kPlanNotInstantiated);
            if (fix.no_wide) fail(c, kPlanFixed);
            if (fix.bt > 1) fail(c, kPlanFixed);
            c.ns_step = kMfmaNs * nf + kWideBaseNs + kWideLdsFragNs * std::max(c.fl, 0);
            finish(c, T, cus);
            out.add(c);
        }
    }
}

// Several CUs per (head, row tile) exchanging h every step (rec_mc.hip), all
// resident at once; through one XCD's L2 where the groups divide over the 8
// XCDs (measured: 25-40% shorter steps than through memory).
void family_multicu(int cell, int T, int B, int NH, int Dh, bool bf16, int cus,
                    const PlanFix &fix, Sink &out) {
    const int G = cell == kLSTM ? 4 : 3;
    const int KC = Dh / 32;
    for (const int kcw : {4, 8}) {
        for (int nb = 1; nb <= 8; ++nb) {
            for (int bt = 1; bt <= 16; ++bt) {
                PlanCand c = blank(kFamMultiCu);
                c.kcw = kcw;
                c.nb = nb;
                c.ks = KC > 0 && KC % kcw == 0 ? KC / kcw : 0;
                c.K = Dh % (16 * nb) == 0 ? Dh / (16 * nb) : 0;
                c.BT = bt;
                c.r4 = r4_of(bt);
                c.waves = nb * std::max(c.ks, 1);
                c.grid = NH * ceil_div(B, bt) * std::max(c.K, 1);
                c.r_vgpr = 4 * G * kcw;
                c.lds = 2L * 16 * (Dh + 8) * 2 + 4L * (std::max(c.ks, 1) - 1) * nb * G * 256;
                c.wg_per_cu = 1;  // all resident: one per CU
                if (!bf16 || Dh < 256 || Dh % 128 != 0) fail(c, kPlanNotInstantiated);
                if (c.ks == 0 || c.K < 2) fail(c, kPlanDivisibility);
                // the kernel takes the 8-chunk variant whenever it divides
                if (kcw == 4 && KC % 8 == 0 && fix.kcw != 4) fail(c, kPlanNotInstantiated);
                if (c.waves > 8) fail(c, kPlanNotInstantiated);
                if (bt > B) fail(c, kPlanBatch);
                // R resident, and up to 256 VGPRs for every wave of a SIMD
                if (c.r_vgpr > kRVgprMax || ceil_div(c.waves, kSimds) * kVgprWave > kRegsSimd)
                    fail(c, kPlanRegisters);
                if (c.lds > kLdsCu) fail(c, kPlanLds);
                if (c.grid > cus) fail(c, kPlanResidency);
                if (fix.bt > 0 && bt != std::min({fix.bt, 16, B})) fail(c, kPlanFixed);
                if (fix.k > 0 && c.K != fix.k) fail(c, kPlanFixed);
                if (fix.kcw > 0 && kcw != fix.kcw) fail(c, kPlanFixed);
                const int per_simd = ceil_div(c.waves, kSimds);
                c.xcd_local = !fix.no_xcd && mc_xcd_grouping(NH * ceil_div(B, bt), c.grid);
                // rows in lane groups: one cell update pass per four rows (1, 2
                // or 4 passes as compiled); the gather polls 4 words a thread
                const bool lanes = mc_row_lanes(bt);
                if (lanes) c.r4 = bt <= 4 ? 1 : bt <= 8 ? 2 : 4;
                const int rounds = ceil_div(bt * (Dh / 2), 4 * 64 * c.waves);
                c.ns_step = kMfmaNs * G * kcw * per_simd +
                            G * (lanes ? kGateLanesNs + kGateLanesPassNs * (c.r4 - 1)
                                       : kGateNs[r4_index(c.r4)]) +
                            kGatherRoundNs * std::max(rounds - 1, 0) +
                            (c.xcd_local ? kExchangeLocalNs : kExchangeNs) +
                            kExchangePerWgNs * std::max(c.K, 1) +
                            kExchangePerValNs * Dh * bt +
                            (c.ks > 1 ? kSplitBaseNs + kSplitPerWaveNs * c.ks : 0.0) +
                            (cell == kLSTM && kcw == 8 && c.r4 == 4 && !lanes ? kSpillBoundNs : 0.0);
                finish(c, T, cus);
                out.add(c);
            }
        }
    }
}

// R in LDS as f32, one thread per (row, gate column) dot product per step
// (rec_fwd_simple_kernel); any precision.
void family_lds(int cell, int T, int B, int NH, int Dh, int cus, const PlanFix &fix, Sink &out) {
    const int G = cell == kLSTM ? 4 : 3;
    for (int bt = 1; bt <= 16; ++bt) {
        PlanCand c = blank(kFamLds);
        c.BT = bt;
        c.waves = 4;
        c.grid = NH * ceil_div(B, bt);
        c.lds = 4L * ((long)Dh * G * Dh + 3L * bt * Dh + (long)bt * G * Dh);
        c.wg_per_cu = fit_per_cu(c.waves, 64, c.lds);
        if (bt > B) fail(c, kPlanBatch);
        if (c.lds > kLdsSimple) fail(c, kPlanLds);
        if (fix.bt > 0 && bt != std::min({fix.bt, 16, B})) fail(c, kPlanFixed);
        c.ns_step = kLdsBaseNs + kLdsDotNs * Dh * ceil_div((long)bt * G * Dh, 256);
        finish(c, T, cus);
        out.add(c);
    }
}

}  // namespace

int plan_search(int cell, int T, int B, int NH, int Dh, bool bf16, int cus, const PlanFix &fix,
                PlanCand *buf, int cap, int *best) {
    Sink s{buf, cap, 0};
    if (cus < 1) cus = 1;
    family_resident(cell, T, B, NH, Dh, bf16, cus, fix, s);
    family_wide(cell, T, B, NH, Dh, bf16, cus, fix, s);
    family_multicu(cell, T, B, NH, Dh, bf16, cus, fix, s);
    family_lds(cell, T, B, NH, Dh, cus, fix, s);
    const int n = std::min(s.n, cap);
    int b = -1;
    for (int i = 0; i < n; ++i)
        if (buf[i].feasible && (b < 0 || buf[i].ns_total < buf[b].ns_total)) b = i;
    if (b >= 0) {
        // exact ties (same prediction): the fewest workgroups, then the first
        const double lim = buf[b].ns_total * (1.0 + 1e-9);
        int t = b;
        for (int i = 0; i < n; ++i)
            if (buf[i].feasible && buf[i].ns_total <= lim && buf[i].grid < buf[t].grid) t = i;
        b = t;
    }
    if (best) *best = b;
    return s.n;
}

}  // namespace rnn355
