// route.hip -- top-k softmax routing, one wavefront per token.
//
// The pages' launcher starts its pipeline with a routing stage that turns
// router output into top-k expert ids and weights ("BF16 support for the
// experimental_sgl_trtllm MoE-LoRA path", "Files changed" table, launcher
// row).  Reading taken here: the k largest fp32 logits, ordered by (logit
// descending, expert id ascending); weights are the softmax over the k
// selected logits (renormalised top-k softmax).
//
// Selection by counting: the rank of expert e is the number of experts that
// come before it in that order, {e' : l[e'] > l[e] or (l[e'] == l[e] and
// e' < e)}.  Ranks are distinct, and rank < k means "selected, at slot rank".
// Every lane counts independently against the token's logits broadcast from
// LDS, so there is no chain of dependent cross-lane reductions.
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kTokensPerBlock = 4;

__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a)
{
    __shared__ float logit[kTokensPerBlock][kMaxExperts];
    __shared__ float sel[kTokensPerBlock][64];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * kTokensPerBlock + wave;
    const bool active = t < a.T;
    const int E = a.E;
    const float *row = a.logits + (size_t)t * E;
    if (active)
        for (int e = lane; e < E; e += kWave)
            logit[wave][e] = row[e];
    __syncthreads();
    if (active) {
        const float *lw = logit[wave];
        for (int e = lane; e < E; e += kWave) {
            const float v = lw[e];
            int rank = 0;
            for (int j = 0; j < E; ++j) {
                const float u = lw[j];
                rank += (u > v) | ((u == v) & (j < e));
            }
            if (rank < a.k) {
                a.topk_ids[(size_t)t * a.k + rank] = e;
                sel[wave][rank] = v;
            }
        }
    }
    __syncthreads();
    if (!active)
        return;
    const float m = sel[wave][0];
    const float ex = lane < a.k ? expf(sel[wave][lane] - m) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        sum += __shfl_xor(sum, off);  // xor butterfly: identical sum on every lane
    if (lane < a.k)
        a.topk_weights[(size_t)t * a.k + lane] = ex / sum;
}

} // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s)
{
    if (a.T <= 0)
        return hipSuccess;
    const int blocks = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
