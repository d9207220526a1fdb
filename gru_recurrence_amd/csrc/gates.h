// gates.h -- the cell update of the recurrent kernels (LSTM / GRU), applied
// to the MFMA accumulators of one wave.
//
// Accumulator layout (v_mfma_f32_16x16x32_bf16, one 16-unit block, G gate
// tiles): acc[g][r] of lane l is the recurrent sum h_{t-1} R of gate g for
// unit l%16 and batch row 4*(l/16) + r.
#pragma once

#include "common.h"

namespace rnn355 {

// Gate update of one unit from its pre-activations.  LSTM: a[g] = Gx + h R
// for g = i,f,z,o and st = c.  GRU: a[0..1] = Gx + S for r,z, a[2] = S_n,
// gxn = Gx_n and st = h_{t-1}.
template <int CELL>
__device__ __forceinline__ float unit_update(const float *a, float gxn, float &st, float &c_out) {
    if (CELL == kLSTM) {
        const float ig = sigmoid_f(a[0]), fg = sigmoid_f(a[1]);
        const float zg = tanh_f(a[2]), og = sigmoid_f(a[3]);
        const float c = fmaf(fg, st, ig * zg);
        st = c;
        c_out = c;
        return og * tanh_f(c);
    } else {
        const float r = sigmoid_f(a[0]), u = sigmoid_f(a[1]);
        const float nn = tanh_f(fmaf(r, a[2], gxn));
        const float h = fmaf(u, st - nn, nn);  // (1-u)*nn + u*h_{t-1}
        st = h;
        c_out = 0.f;
        return h;
    }
}

// R4 == 1 (only batch row 0 is live, in lanes 0..15): three cross-row swaps
// lay the G gate sums of a unit out as the rows of one register: gate g of
// unit l%16 in lane l = 16g + l%16 (LSTM rows i, f, z, o; GRU rows r, z,
// S_n and an unused row 3).
template <int CELL>
__device__ __forceinline__ float gate_rows_of(const f32x4 (&acc)[CellTraits<CELL>::G]) {
    if constexpr (CELL == kLSTM) {
        const RowPair p = swap16(acc[0][0], acc[1][0]);
        const RowPair q = swap16(acc[2][0], acc[3][0]);
        return swap32(p.a, q.a).a;
    } else {
        const RowPair p = swap16(acc[0][0], acc[1][0]);
        return swap32(p.a, acc[2][0]).a;
    }
}

// The exponent scale of the activation on gate row `row` of the row layout
// above: sigmoid(x) = 1/(1 + 2^(x * -log2 e)); the LSTM's z row takes
// tanh(x) = 2 sigmoid(2x) - 1, scale -2 log2 e.
template <int CELL>
__device__ __forceinline__ float gate_row_scale(int row) {
    return (CELL == kLSTM && row == 2) ? -2.0f * kLog2e : -kLog2e;
}

// Cell update from the gate-row layout above, v = this lane's recurrent
// sum and gx = the Gx of the lane's gate row (GXK: the LSTM's exponent is
// fma(v, k, gx k), whose product gx k does not wait for the MFMAs, so one
// fma follows them instead of an add and a multiply).  One
// exp + rcp pass activates every gate at once, and swaps bring a unit's
// gates together.  LSTM: h = o tanh(c) = 2 o sigmoid(2c) - o (one exp and
// one rcp after c).  The LSTM result is valid in row 0 (row 0 writes it),
// the GRU result in row 3 (row 3 writes it).
template <int CELL, bool GXK = false>
__device__ __forceinline__ void gate_rows_update(float v, float gx, float &st, float &hl,
                                                 float &h, float &c) {
    const int row = (threadIdx.x & 63) >> 4;
    const float act_k = gate_row_scale<CELL>(row);
    const float arg = (GXK && CELL == kLSTM) ? fmaf(v, act_k, gx * act_k) : (v + gx) * act_k;
    const float sg = rcp_fast(1.0f + __builtin_amdgcn_exp2f(arg));
    if constexpr (CELL == kLSTM) {
        // rows of sg: sigma(a_i), sigma(a_f), sigma(2 a_z), sigma(a_o).  Row 0
        // gathers f and z with one swap each and o (needed last) with a
        // second swap; only row 0's c and h are valid (the lanes that write
        // them).  Each swap's partner register holds a constant set off the
        // chain (its contents do not matter), so no copy of sg sits between
        // the activation and c.
        const float f = swap16(sg, 0.0f).b;   // rows [f, -, o, -]
        const float zs = swap32(sg, 0.0f).b;  // rows [sigma(2 a_z), o, -, -]
        const float o = swap16(zs, 0.0f).b;   // row 0: o
        // i z = i (2 sigma(2 a_z) - 1)
        const float cn = fmaf(f, st, fmaf(sg + sg, zs, -sg));
        st = cn;
        c = cn;
        const float s2 = rcp_fast(1.0f + __builtin_amdgcn_exp2f(cn * (-2.0f * kLog2e)));
        h = fmaf(o + o, s2, -o);
        hl = h;
    } else {
        // tanh(x) = 2 sigmoid(2x) - 1 on the candidate row
        const RowPair W = swap32(0.0f, sg);               // W.a rows -, -, r, u
        const float xn = fmaf(W.a, v, gx);                // row 2: Gx_n + r S_n
        const float nn = fmaf(2.0f, rcp_fast(1.0f + __builtin_amdgcn_exp2f(xn * (-2.0f * kLog2e))),
                              -1.0f);
        const float nn3 = swap16(0.0f, nn).a;             // row 3 <- row 2
        const float hn = fmaf(W.a, st - nn3, nn3);        // row 3: (1-u) nn + u h
        st = hn;
        h = hn;
        c = 0.f;
    }
}

// Batch rows in lane groups: the MFMA leaves row 4p + r of the tile in
// register r of lane group p.  Two 16-lane and two 32-lane swaps per gate
// transpose that 4 x 4 block, so that pass r holds row 4r + q in lane group
// q and each pass of the cell update serves four rows: R4 passes cover 4 R4
// rows (the register-slot layout runs one pass per register).
//   gx[r][g]: the G gate inputs Gx of the lane's row in pass r.
template <int CELL, int R4>
__device__ __forceinline__ void gate_update_lanes(const f32x4 (&acc)[CellTraits<CELL>::G],
                                                  const float (&gx)[R4][CellTraits<CELL>::G],
                                                  float (&st)[R4], float (&hl)[R4], float (&h)[R4],
                                                  float (&c)[R4]) {
    constexpr int G = CellTraits<CELL>::G;
    static_assert(R4 == 1 || R4 == 2 || R4 == 4, "one, two or four passes");
    float v[R4][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const RowPair p = swap16(acc[g][0], acc[g][1]);
        const RowPair q = swap16(acc[g][2], acc[g][3]);
        const RowPair x = swap32(p.a, q.a);  // passes 0, 2
        v[0][g] = x.a;
        if constexpr (R4 > 1) {
            const RowPair y = swap32(p.b, q.b);  // passes 1, 3
            v[1][g] = y.a;
            if constexpr (R4 > 2) {
                v[2][g] = x.b;
                v[3][g] = y.b;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R4; ++r) {
        float pre[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pre[g] = (CELL == kGRU && g == 2) ? v[r][g] : v[r][g] + gx[r][g];
        h[r] = unit_update<CELL>(pre, CELL == kGRU ? gx[r][2] : 0.f, st[r], c[r]);
        hl[r] = h[r];
    }
}

// The cell update of all row slots of one lane.
//   gx[r][.]: for R4 > 1 the G gate inputs Gx of row slot r; for R4 == 1 a
//             single value, the Gx of gate l/16 (the lane's row, see above).
//   st[r]:    cell state c (LSTM) or h (GRU), updated in place.
//   hl[r]:    last h (LSTM only; GRU keeps h in st).
//   h[r], c[r]: this step's outputs.
template <int CELL, int R4, int GL, bool GXK = false>
__device__ __forceinline__ void gate_update(const f32x4 (&acc)[CellTraits<CELL>::G],
                                            const float (&gx)[R4][GL], float (&st)[R4],
                                            float (&hl)[R4], float (&h)[R4], float (&c)[R4]) {
    constexpr int G = CellTraits<CELL>::G;
    if constexpr (R4 == 1) {
        gate_rows_update<CELL, GXK>(gate_rows_of<CELL>(acc), gx[0][0], st[0], hl[0], h[0],
                                    c[0]);
    } else {
#pragma unroll
        for (int r = 0; r < R4; ++r) {
            // A = Gx + h R (the GRU's candidate gate keeps its recurrent sum
            // apart: it is scaled by r before Gx_n is added)
            float pre[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                pre[g] = (CELL == kGRU && g == 2) ? acc[g][r] : acc[g][r] + gx[r][g];
            h[r] = unit_update<CELL>(pre, CELL == kGRU ? gx[r][2] : 0.f, st[r], c[r]);
            hl[r] = h[r];
        }
    }
}

}  // namespace rnn355
