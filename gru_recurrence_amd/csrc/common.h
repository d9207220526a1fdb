// common.h -- device types and small helpers shared by the librnn355 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnn355 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

enum Cell { kLSTM = 0, kGRU = 1 };

template <int CELL>
struct CellTraits;
template <>
struct CellTraits<kLSTM> { static constexpr int G = 4; };
template <>
struct CellTraits<kGRU> { static constexpr int G = 3; };

// float -> bf16 bit pattern, round to nearest even (inputs are finite):
// one v_cvt_pk_bf16_f32 on gfx950.  For every finite float it gives the bits
// of the integer rule (u + 0x7FFF + ((u >> 16) & 1)) >> 16, checked on the
// device over all 2^32 patterns.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// e^x through the hardware base-2 exponential (v_exp_f32) with the argument
// scaled by log2(e).  Over/underflow saturate to inf / 0 as e^x does.
__device__ __forceinline__ float exp_fast(float x) {
    return __builtin_amdgcn_exp2f(x * kLog2e);
}

// 1/x via v_rcp_f32 (1 ulp).
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// logistic sigmoid 1/(1+e^-a); saturates cleanly to 0 and 1.
__device__ __forceinline__ float sigmoid_f(float a) {
    return rcp_fast(1.0f + exp_fast(-a));
}

// tanh held to float32 relative accuracy at every magnitude (about 1 ulp
// below |a| = 0.5, 3 ulp above).  For |a| >= 0.5, tanh|a| = (1 - e)/(1 + e)
// with e = e^{-2|a|} in (0, e^-1]: 1 - e >= 0.63, so nothing cancels, and
// nothing overflows.  Below 0.5 that difference would cancel (relative error
// ~2^-24/(2|a|)), so there tanh|a| = x + x^3 q(x^2), an odd polynomial with
// q of degree 4 whose coefficients were fitted for these kernels by
// relative-error-weighted least squares on Chebyshev nodes of [0, 0.5]
// (iteratively reweighted toward equal ripple), then rounded to float32 and
// checked in float32 Horner arithmetic against tanh in float64.  Both forms
// are evaluated and one is selected, so a wave does not diverge.
__device__ __forceinline__ float tanh_f(float a) {
    const float x = fabsf(a);
    const float e = exp_fast(-2.0f * x);
    const float t_exp = (1.0f - e) * rcp_fast(1.0f + e);
    const float x2 = x * x;
    float q = -6.647501141e-03f;
    q = fmaf(q, x2, 2.129799873e-02f);
    q = fmaf(q, x2, -5.389919132e-02f);
    q = fmaf(q, x2, 1.333296448e-01f);
    q = fmaf(q, x2, -3.333332837e-01f);
    const float t_poly = fmaf(x * x2, q, x);
    return copysignf(x < 0.5f ? t_poly : t_exp, a);
}

// tanh with an absolute error near 1 ulp of 1 (the exponential form at
// every magnitude; its relative error grows as |a| -> 0).  Only for the
// single-row gate path of the bf16 kernels, whose h is rounded to bf16
// (8 significant bits) before any further use as an operand.
__device__ __forceinline__ float tanh_abs(float a) {
    const float e = exp_fast(-2.0f * fabsf(a));
    const float t = (1.0f - e) * rcp_fast(1.0f + e);
    return copysignf(t, a);
}

// Workgroup barrier that orders LDS only: release/acquire fences limited to
// the local address space, so the barrier never waits on outstanding global
// loads or stores (a plain __syncthreads() would also drain those).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-row moves of gfx950 (a "row" is 16 lanes).  With x the first and y
// the second operand:
//   swap16(x, y) -> { [x0, y0, x2, y2], [x1, y1, x3, y3] }
//   swap32(x, y) -> { [x0, x1, y0, y1], [x2, x3, y2, y3] }
struct RowPair {
    float a, b;
};
__device__ __forceinline__ RowPair swap16(float x, float y) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ RowPair swap32(float x, float y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Eight wait states pinned right after an MFMA chain.  A vector instruction
// that reads or overwrites an MFMA destination needs them (the compiler
// spaces such pairs inside a basic block, but across a branch it has been
// seen to place a read one instruction after the MFMA, which then saw a
// stale value); with the pad in place every path after the chain is safe.
__device__ __forceinline__ void mfma_chain_end() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(const bf16x8 &a, const bf16x8 &b,
                                                     const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Select two 16-bit halves: lo half of the result from `lo_src`, hi half
// from `hi_src`; `hi_parts` picks the upper (true) or lower (false) halves
// of both sources.  (v_perm_b32 byte select.)
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo_src, uint32_t hi_src, bool upper) {
    return __builtin_amdgcn_perm(hi_src, lo_src, upper ? 0x07060302u : 0x05040100u);
}

}  // namespace rnn355
