// xcd.h -- placing the workgroups of one exchange group on one XCD.
//
// The dispatcher deals the workgroups of a launch to the 8 XCDs in turn
// (workgroup i on XCD i % 8; every workgroup of a residue class on the same
// XCD, measured for grids of 32 to 512).  A kernel whose K workgroups per
// group swap data every step numbers them so that group g's members are the
// workgroups ((g / 8) K + m) 8 + g % 8, m < K: one residue class, one XCD,
// one L2.  Each launch checks the placement instead of assuming it: every
// workgroup publishes the XCD it runs on (hardware register XCC_ID) in a
// table cleared before the launch, and wave 0 of each member reads the
// group's entries.  All members read the same entries, so all reach the same
// verdict; only a group found on one XCD may exchange through that XCD's L2.
#pragma once

#include <hip/hip_runtime.h>

namespace rnn355 {

// The XCD (accelerator complex die) of the calling wave: XCC_ID bits [3:0].
__device__ __forceinline__ unsigned xcc_id() {
    return (unsigned)__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u;
}

// Group and member of this workgroup, K workgroups per group: by XCD residue
// class (xcd_map; needs groups % 8 == 0) or consecutively.
__device__ __forceinline__ void group_member(bool xcd_map, int K, int &group, int &member) {
    if (xcd_map) {
        const int slot = blockIdx.x >> 3;
        group = (blockIdx.x & 7) + 8 * (slot / K);
        member = slot % K;
    } else {
        group = blockIdx.x / K;
        member = blockIdx.x - group * K;
    }
}

// Thread 0: record this workgroup's XCD (as id + 1; the table starts at 0).
__device__ __forceinline__ void xcd_publish(unsigned *xcc) {
    if (threadIdx.x == 0)
        __hip_atomic_store(xcc + blockIdx.x, xcc_id() + 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// One whole wave: 1 if every member of `group` (xcd_map numbering) runs on
// this workgroup's XCD, 0 if not, -1 if a member's entry did not appear
// within spin_limit polls (the abort word is then raised).  Every member is
// resident (checked on the host before the launch), so the entries appear.
__device__ __forceinline__ int xcd_members_agree(const unsigned *xcc, unsigned *flag,
                                                 unsigned spin_limit, int group, int K) {
    const int lane = threadIdx.x & 63;
    const unsigned mine = xcc_id() + 1u;
    bool same = true, lost = false;
    for (int mm = lane; mm < K; mm += 64) {
        const int bid = (((group >> 3) * K + mm) << 3) | (group & 7);
        unsigned v, spins = 0;
        while ((v = __hip_atomic_load(xcc + bid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ==
               0u) {
            if (++spins >= spin_limit) {
                __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                lost = true;
                break;
            }
        }
        if (v != mine) same = false;
    }
    if (__any(lost)) return -1;
    return __all(same) ? 1 : 0;
}

}  // namespace rnn355
