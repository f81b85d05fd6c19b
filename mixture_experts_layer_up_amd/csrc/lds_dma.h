// lds_dma.h -- direct global->LDS loads on gfx950 and their explicit waits.
//
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory into
// LDS without passing through registers: lane l's bytes land at the
// wave-uniform LDS byte address in M0 plus 16 l.  The loads are written as
// inline assembly on purpose: the compiler then leaves their completion to
// the explicit waits below (its own tracking would otherwise wait for every
// outstanding load before each LDS read and serialise the pipeline).  Loads
// it does not know about can only make its own wait counts stricter.
#pragma once

#include <stdint.h>

namespace moe_lora {

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ object, as a wave-uniform value (M0)
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((const lds_void *)p));
}

__device__ __forceinline__ void load_lds16(const void *g, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// The same for data read once (expert weights): the nontemporal hint keeps
// the stream from evicting data that other blocks are about to reuse.
__device__ __forceinline__ void load_lds16_stream(const void *g, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// Activation rows staged as 16-row MFMA A fragments keep a row's four 16-byte
// K quarters 64 bytes apart, XOR-swizzled by bits 1..3 of the row, so that
// the fragment reads (16 rows x 16 bytes per quarter of the wave) hit
// distinct LDS banks.  Physical quarter of logical quarter q of row `row`:
// q ^ act_swizzle(row).
__device__ __forceinline__ int act_swizzle(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Wait until at most N of this wave's vector loads are outstanding and its
// LDS reads are done, then synchronise the block (N = 63: LDS reads only).
// The empty asm statements keep LDS reads from moving across the barrier.
template <int N>
__device__ __forceinline__ void dma_wait_barrier()
{
    static_assert(N < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// All of this wave's vector loads complete (no direct load may land after
// the block's LDS is released or reused).
__device__ __forceinline__ void dma_drain()
{
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    asm volatile("" ::: "memory");
}

} // namespace moe_lora
