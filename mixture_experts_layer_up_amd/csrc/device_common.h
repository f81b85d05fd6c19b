// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Round to nearest even; NaN stays NaN.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32), one instruction instead of the integer rounding
// sequence.
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Streaming load for data read once per call (expert weights, LoRA stacks):
// the nontemporal hint keeps it from displacing reused lines in the caches
// and lets the memory system stream it at a higher rate.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void store16(void *p, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Streaming store for large outputs that the next kernel reads once: the
// nontemporal hint keeps tens of MB of dirty lines out of the caches, whose
// later write-back would otherwise compete with the next weight streams.
__device__ __forceinline__ void store16_stream(void *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

// v if cond else 0, without a branch: the load that produced v stays
// unconditional, so the number of loads in flight is the same on every path
// and the compiler keeps exact wait counts.
__device__ __forceinline__ u32x4 keep_if(u32x4 v, bool cond)
{
    const unsigned m = cond ? 0xffffffffu : 0u;
    return u32x4{v.x & m, v.y & m, v.z & m, v.w & m};
}

__device__ __forceinline__ u32x4 zero16()
{
    u32x4 z = {0u, 0u, 0u, 0u};
    return z;
}

// D = A * B + C for a 16x16 tile with K = 32 (bf16 in, fp32 accumulate).
// Lane l holds A[l % 16][8(l / 16) .. +7], B[8(l / 16) .. +7][l % 16] and
// D[4(l / 16) .. +3][l % 16].
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Index of the calling wave inside its block, as a wave-uniform (scalar)
// value.  MFMA instructions do not honour the EXEC mask, so every condition
// that decides whether an MFMA runs must be a scalar branch; deriving it from
// threadIdx.x directly would let the compiler lower it to EXEC masking.
__device__ __forceinline__ int wave_id()
{
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Block barrier for LDS traffic only: completes this wave's LDS operations
// and synchronises the block, but leaves global loads in flight.  A plain
// __syncthreads() also fences global memory, which waits for every
// outstanding load and would drain the register prefetch rings.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A value every lane of the wave holds identically, made scalar so that
// branches on it are scalar branches.
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  The grid is an upper bound of the work; the n_items work items
// (a count known only on the device) are split into 8 equal contiguous
// ranges, one per XCD, so that the real work is spread evenly over the XCDs
// however many blocks are spare, and neighbouring items (for example the
// column slabs of one expert, which share activation rows) share that XCD's
// L2.  Returns -1 for a block without work.
__device__ __forceinline__ int xcd_balanced_item(int bid, int n_items)
{
    const int per = (n_items + 7) >> 3;
    const int idx = bid >> 3;
    if (idx >= per)
        return -1;
    const int item = (bid & 7) * per + idx;
    return item < n_items ? item : -1;
}

// SiLU(z) = z * sigmoid(z) from the hardware base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32; each within about one fp32 ulp): the
// epilogues round the gated product to bf16, far coarser, and a library
// exp plus an IEEE division per element cost several microseconds per
// many-row GEMM block.  z -> -inf gives -0, z -> +inf gives z.
__device__ __forceinline__ float silu_f32(float z)
{
    const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896340736f);  // exp(-z)
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}
