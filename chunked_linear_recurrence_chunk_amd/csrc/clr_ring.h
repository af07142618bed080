// clr_ring.h -- producer/consumer streaming of per-block operands into LDS.
//
// A sequential scan is latency-bound: each 64-token block needs tens of KB of
// operands, and one wave can only keep ~63 memory operations in flight.  The
// scan work-groups therefore run consumer waves (the recurrence, state in
// registers: one, or two that each hold half of the state's key rows) and NP
// producer waves (three, or enough to fill eight waves where the stream
// bounds the scan) that stream the operands of the next blocks into a ring
// of P LDS slots with direct global->LDS loads (global_load_lds_dwordx4: each
// lane's 16 bytes land at slot + unit*1024 + lane*16, exactly where the
// consumer lane reads its fragment back).
//
// Round n (all waves, separated by s_barrier):
//   consumers compute block n from slot n % P (two consumers meet once more
//             within the round, at a barrier the producers also pass);
//   producers issue block n + P - 1 into slot (n - 1) % P (read in round n-1),
//             then wait until their loads for block n + 1 have landed.
// The waits are explicit vmcnt immediates; s_barrier is used without a fence
// so that the producers' later loads stay in flight across rounds.
#pragma once

#include "clr_device.h"

namespace clr {

#define CLR_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int RING_UNIT = 1024;  // bytes per 16-byte-per-lane unit
constexpr int RING_SMALL = 256;  // one 4-byte-per-lane unit (gates)
constexpr int NPROD = 3;         // producer waves

// s_waitcnt immediate for vmcnt(n), other counters unconstrained (gfx9 encoding).
constexpr unsigned vmcnt_imm(int n) { return (unsigned)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8)); }
// s_waitcnt immediate for lgkmcnt(0) (this wave's LDS operations done), the
// other counters unconstrained.
constexpr unsigned lgkmcnt0_imm() { return (unsigned)(15 | (3 << 14) | (7 << 4)); }

template <int NU, int NP = NPROD>
struct RingGeom {
    static constexpr int SLOT = NU * RING_UNIT + RING_SMALL;
    static constexpr int NU_MIN = NU / NP;  // loads per producer per block, lower bound
    static_assert(2 * NU_MIN <= 63, "vmcnt range");
};

// Wait until at most k blocks (of >= NU_MIN loads each) are still in flight.
template <int NU_MIN>
__device__ __forceinline__ void ring_wait(int k) {
    if (k <= 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else if (k == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NU_MIN));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NU_MIN));
}


__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Issue one block's units.  unit_src(u) gives this lane's 16-byte source of
// unit u; small_src this lane's 4-byte source of the small unit.
// Producer pid issues units pid, pid + NP, ...  pid is wave-uniform; it is
// read into a scalar register so that the unit loop is straight-line code:
// a per-unit exec-masked branch costs more issue time than the loads.
template <int NU, int NP, typename F>
__device__ __forceinline__ void ring_issue_units(char* slot, int pid, F unit_src) {
    const int p = __builtin_amdgcn_readfirstlane(pid);
#pragma unroll
    for (int j = 0; j < (NU + NP - 1) / NP; ++j) {
        const int u = p + NP * j;
        if (NP * (j + 1) <= NU || u < NU)
            __builtin_amdgcn_global_load_lds(unit_src(u), CLR_LDS(slot + u * RING_UNIT), 16, 0, 0);
    }
}

template <int NU, typename F, int NP = NPROD>
__device__ __forceinline__ void ring_issue(char* slot, int pid, F unit_src, const void* small_src) {
    ring_issue_units<NU, NP>(slot, pid, unit_src);
    if (__builtin_amdgcn_readfirstlane(pid) == NP - 1)
        __builtin_amdgcn_global_load_lds(small_src, CLR_LDS(slot + NU * RING_UNIT), 4, 0, 0);
}

// Fragment f of a slot (bf16: one unit per fragment; fp32: two).
__device__ __forceinline__ Frag<bf16> ring_frag(const char* slot, int f, int l, bf16*) {
    Frag<bf16> x;
    x.v = *(const bf16x8*)(slot + f * RING_UNIT + l * 16);
    return x;
}
__device__ __forceinline__ Frag<float> ring_frag(const char* slot, int f, int l, float*) {
    Frag<float> x;
    x.lo = *(const f32x4*)(slot + (2 * f) * RING_UNIT + l * 16);
    x.hi = *(const f32x4*)(slot + (2 * f + 1) * RING_UNIT + l * 16);
    return x;
}
template <int NU>
__device__ __forceinline__ float ring_small(const char* slot, int lane) {
    return *(const float*)(slot + NU * RING_UNIT + lane * 4);
}

}  // namespace clr
