// finalize.hip -- routing-weighted sum of each token's expert outputs.
//
// The pages' pipeline ends in a finalize that reduces the k expert outputs
// of a token back to one row, weighted by the routing weights; the down LoRA
// delta is weighted the same way ("BF16 support for the experimental_sgl_trtllm
// MoE-LoRA path", "Files changed" table, launcher row, and Flow section 2,
// down LoRA add with routing-weight multiply).  Here the down delta is
// already inside y (it was accumulated as extra K of the down GEMM), so
// out[t] = scale * sum_j w[t, j] * y[p(t, j)], j ascending, slots with
// p = -1 (not local) skipped, fp32 sum, one bf16 rounding.  No atomics: the
// result is the same on every run.
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs a)
{
    const int t = blockIdx.x;
    const int col0 = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (col0 >= a.H)
        return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.0f;
    // slots in groups of 8: every index and row load of a group is issued
    // before any is used (the rows depend on the indices, so a plain loop
    // would wait twice per slot); the sum still runs in ascending j
    constexpr int kG = 8;
    for (int j0 = 0; j0 < a.k; j0 += kG) {
        int p[kG];
        float w[kG];
#pragma unroll
        for (int i = 0; i < kG; ++i) {
            const int j = min(j0 + i, a.k - 1);
            p[i] = j0 + i < a.k ? a.exp2perm[(size_t)t * a.k + j] : -1;
            w[i] = a.weights[(size_t)t * a.k + j];
        }
        u32x4 v[kG];
#pragma unroll
        for (int i = 0; i < kG; ++i)  // slots that are not local read row 0, unused
            v[i] = load16(a.Y + (size_t)max(p[i], 0) * a.H + col0);
#pragma unroll
        for (int i = 0; i < kG; ++i) {
            const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = acc[2 * e] + w[i] * bf16_bits_to_float(u[e] & 0xffffu);
                const float hi = acc[2 * e + 1] + w[i] * bf16_bits_to_float(u[e] >> 16);
                acc[2 * e] = p[i] >= 0 ? lo : acc[2 * e];
                acc[2 * e + 1] = p[i] >= 0 ? hi : acc[2 * e + 1];
            }
        }
    }
    u32x4 o;
    o.x = float_to_bf16_bits(a.scale * acc[0]) | (float_to_bf16_bits(a.scale * acc[1]) << 16);
    o.y = float_to_bf16_bits(a.scale * acc[2]) | (float_to_bf16_bits(a.scale * acc[3]) << 16);
    o.z = float_to_bf16_bits(a.scale * acc[4]) | (float_to_bf16_bits(a.scale * acc[5]) << 16);
    o.w = float_to_bf16_bits(a.scale * acc[6]) | (float_to_bf16_bits(a.scale * acc[7]) << 16);
    store16(a.out + (size_t)t * a.H + col0, o);
}

} // namespace

hipError_t launch_finalize(const FinalizeArgs &a, hipStream_t s)
{
    if (a.T <= 0)
        return hipSuccess;
    const int col_blocks = (a.H + 2047) / 2048;
    hipLaunchKernelGGL(finalize_kernel, dim3(a.T, col_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
