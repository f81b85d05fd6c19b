// route.hip -- top-k softmax routing, one wavefront per token.
//
// The pages' launcher starts its pipeline with a routing stage that turns
// router output into top-k expert ids and weights ("BF16 support for the
// experimental_sgl_trtllm MoE-LoRA path", "Files changed" table, launcher
// row).  Reading taken here: the k largest fp32 logits, ordered by (logit
// descending, expert id ascending); weights are the softmax over the k
// selected logits (renormalised top-k softmax).
#include <climits>
#include <cmath>

#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kMaxPerLane = 16;  // up to 1024 experts

__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T)
        return;

    const float *row = a.logits + (size_t)t * a.E;
    float v[kMaxPerLane];
    unsigned taken = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + kWave * i;
        const bool in = e < a.E;
        v[i] = in ? row[e] : 0.0f;
        taken |= in ? 0u : (1u << i);
    }

    int my_id = -1;
    float my_v = 0.0f;
    for (int j = 0; j < a.k; ++j) {
        // best untaken value of this lane (ids ascend with i, strict '>' keeps the lower id)
        float bv = 0.0f;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            if (!((taken >> i) & 1u) && (bi == INT_MAX || v[i] > bv)) {
                bv = v[i];
                bi = lane + kWave * i;
            }
        }
        // wave arg-max under (value desc, id asc); every lane ends with the winner
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            const bool better = oi != INT_MAX &&
                                (bi == INT_MAX || ov > bv || (ov == bv && oi < bi));
            if (better) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & (kWave - 1)) == lane)
            taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_id = bi;
            my_v = bv;
        }
    }

    const float m = __shfl(my_v, 0);
    const float ex = lane < a.k ? expf(my_v - m) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        sum += __shfl_xor(sum, off);  // xor butterfly: identical sum on every lane
    if (lane < a.k) {
        a.topk_ids[(size_t)t * a.k + lane] = my_id;
        a.topk_weights[(size_t)t * a.k + lane] = ex / sum;
    }
}

} // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s)
{
    if (a.T <= 0)
        return hipSuccess;
    const int blocks = (a.T + 3) / 4;
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
