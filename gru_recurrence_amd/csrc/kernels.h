// kernels.h -- argument blocks and launchers of the librnn355 kernels
// (internal; the public interface is include/rnn355.h).
#pragma once

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
};

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
hipError_t launch_gemm_f32(const GemmF32Args &g, int batch, hipStream_t s);

// Forward recurrence (rec_fwd.hip).
struct RecArgs {
    int T, B, NH, Dh, BT;     // BT: batch rows per workgroup
    const float *gx;          // [T][B][NH*G*Dh]
    const uint16_t *Rb;       // bf16 R (MFMA kernel / bf16 simple kernel)
    const float *Rf;          // f32 R (f32 simple kernel)
    const float *h0, *c0;
    float *h_seq, *c_seq, *hT, *cT;
};

enum RecKind { kRecNone = 0, kRecMfma = 1, kRecSimple = 2 };

struct RecPlan {
    RecKind kind;
    int BT;          // rows per workgroup
    int nbt;         // batch tiles
    int grid;        // workgroups
    int threads;     // per workgroup
    int waves;       // per workgroup
    int upt;         // units per thread (MFMA kernel)
    size_t lds;      // dynamic LDS bytes (simple kernel)
};

// Chooses the kernel and tiling for (cell, dims, dtype).  bt_override > 0
// forces the rows per workgroup.  Pure host function.
RecPlan plan_rec(int cell, int T, int B, int NH, int Dh, bool bf16, int num_cu,
                 int bt_override);

hipError_t launch_rec_fwd(int cell, const RecPlan &p, const RecArgs &a, bool bf16,
                          hipStream_t s);

}  // namespace rnn355
