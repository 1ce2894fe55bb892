// vc_lds.hpp -- LDS staging helpers shared by the attention kernels: direct
// global->LDS copies with explicit waits, buffer descriptors, the block
// barrier, and a three-input max.
#pragma once

#include "vc_device.hpp"

namespace vc {

typedef VC_LDS uint8_t lds_u8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// End of a block: this wave's LDS reads are complete, then all waves meet.
// The scheduling fences keep every instruction on its side of the barrier.
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

typedef int v4si __attribute__((ext_vector_type(4)));

// Buffer descriptor of `bytes` bytes at `base` (gfx9: raw 32-bit data, no
// stride); reads past the end return zeros.  All fields are wave-uniform.
__device__ __forceinline__ v4si make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    v4si r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// Direct global->LDS copies.  Written as inline assembly so that the
// compiler neither waits on them nor counts them: every wait on these copies
// is explicit (wait_vmcnt) and every LDS hand-over goes through a barrier.
// They have no register outputs; M0 (the wave's LDS base) is set in the same
// block, one wait state before the load.  M0 is declared clobbered; clang
// warns that it is a reserved register, which it does not save around the
// asm.  The kernels that include this header leave M0 to these blocks alone
// (the compiled code has no other M0 access), so the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const v4si& r, const lds_u8* lds_wave_base, uint32_t voff,
                                          uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))), "v"(voff), "s"(r),
                    "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}

__device__ __forceinline__ void lds_dma4(const v4si& r, const lds_u8* lds_wave_base, uint32_t voff,
                                         uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))), "v"(voff), "s"(r),
                    "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}

__device__ __forceinline__ void lds_dma16_flat(const void* g, const lds_u8* lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))),
                    "v"(reinterpret_cast<uint64_t>(g))
                 : "memory", "m0");
}

__device__ __forceinline__ void lds_dma4_flat(const void* g, const lds_u8* lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))),
                    "v"(reinterpret_cast<uint64_t>(g))
                 : "memory", "m0");
}

#pragma clang diagnostic pop

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// max(a, b, c): the compiler forms v_max3_f32 from the two fmaxf (NaN inputs
// are outside the library's contract and the attention sources are built
// with -fno-honor-nans) and inserts the wait states its inputs need, which it
// would not do for inline assembly reading a transcendental or matrix-core
// result (measured: same instruction mix and timing as an asm version).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    return fmaxf(fmaxf(a, b), c);
}

}  // namespace vc
