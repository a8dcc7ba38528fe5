// LDS-ring plumbing shared by the tiled GEMM kernels: the global -> LDS DMA
// copy, vmcnt waits and barriers without memory fences.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fq {

// 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4, SGPR base +
// 32-bit VGPR offset form): lane l reads base + voff and its 16 bytes land at
// lds_dst + 16 l; lds_dst must be wave uniform (it is passed in M0).  Written
// as inline asm so that the compiler does not wait for every outstanding copy
// before each LDS read; completion is tracked explicitly with wait_vmcnt and
// the stage barrier.  The s_nop covers the M0-write -> LDS-DMA hazard.  The
// instruction has no VGPR result, only the address operands, which the
// hardware consumes at issue.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* base, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_dst) : "memory");
}

// LDS byte address of a pointer into __shared__ memory (wave uniform).
__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
    typedef __attribute__((address_space(3))) const uint8_t lds_byte;
    return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lds_byte*)p)));
}

// s_waitcnt vmcnt(n) leaving the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// vmcnt(k * NHI) for a k known only at run time (0 <= k < 8, k * NHI < 64)
template <int NHI>
__device__ __forceinline__ void wait_stages_in_flight(int k) {
    switch (k) {
        case 0: wait_vmcnt<0>(); break;
        case 1: if constexpr (1 * NHI < 64) { wait_vmcnt<1 * NHI>(); break; } [[fallthrough]];
        case 2: if constexpr (2 * NHI < 64) { wait_vmcnt<2 * NHI>(); break; } [[fallthrough]];
        case 3: if constexpr (3 * NHI < 64) { wait_vmcnt<3 * NHI>(); break; } [[fallthrough]];
        case 4: if constexpr (4 * NHI < 64) { wait_vmcnt<4 * NHI>(); break; } [[fallthrough]];
        case 5: if constexpr (5 * NHI < 64) { wait_vmcnt<5 * NHI>(); break; } [[fallthrough]];
        case 6: if constexpr (6 * NHI < 64) { wait_vmcnt<6 * NHI>(); break; } [[fallthrough]];
        default: wait_vmcnt<0>(); break;
    }
}

// Workgroup barrier without a memory fence (the LDS-DMA waits are explicit);
// the empty asm statements keep the compiler from moving LDS accesses across it.
// On gfx950 s_barrier does not wait for the wave's own LDS accesses, and the
// compiler adds no wait before it either: a wave whose LDS writes other waves
// read past the barrier uses barrier_lds.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes have landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace fq
