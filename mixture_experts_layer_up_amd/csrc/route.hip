// route.hip -- top-k softmax routing, one wavefront per token.
//
// The pages' launcher starts its pipeline with a routing stage that turns
// router output into top-k expert ids and weights ("BF16 support for the
// experimental_sgl_trtllm MoE-LoRA path", "Files changed" table, launcher
// row; the op also names a routing bias and a routing method, undefined).
// Readings taken here: the k largest selection scores, ordered by (score
// descending, expert id ascending), where the score is the fp32 logit plus
// the expert's fp32 bias when one is given; weights come from the logits:
// the softmax over the k selected logits (method 0, renormalised top-k
// softmax) or the softmax over all E logits at the selected experts
// (method 1).
//
// Selection as a wave-level radix select.  Each (logit, id) becomes one
// 42-bit key that orders exactly like (logit descending, id ascending): the
// order-preserving integer image of the float in the high 32 bits, and
// 1023 - id in the low 10 bits.  All keys are distinct, so the k-th largest
// key is found bit by bit from the top, counting keys >= candidate with
// ballots; the k keys >= it are the selection.  A selected key's slot is the
// number of selected keys above it.  Every step is a short chain of
// wave-uniform operations (finite logits assumed).
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kMaxPerLane = 16;  // up to 1024 experts
constexpr int kTokensPerBlock = 4;

__device__ __forceinline__ unsigned long long route_key(float v, int e)
{
    const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);  // -0 and +0 compare equal
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ord << 10) | (unsigned long long)(1023 - e);
}

template <int NV>  // logits per lane: E <= 64 * NV
__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a)
{
    __shared__ unsigned long long sel_key[kTokensPerBlock][64];
    __shared__ float sel_val[kTokensPerBlock][64];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id();
    const int t = blockIdx.x * kTokensPerBlock + wave;
    const bool active = t < a.T;  // uniform per wave
    const int k = a.k;
    const unsigned long long lt = (1ull << lane) - 1ull;

    unsigned long long key[NV];
    float val[NV];
    unsigned long long thr = 0;
    if (active) {
        const float *row = a.logits + (size_t)t * a.E;
        float bv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {  // all loads first, then the keys
            const int e = lane + kWave * i;
            val[i] = e < a.E ? row[e] : 0.0f;
            bv[i] = (a.bias && e < a.E) ? a.bias[e] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + kWave * i;
            const float score = a.bias ? val[i] + bv[i] : val[i];  // one fp32 add
            key[i] = e < a.E ? route_key(score, e) : 0ull;  // 0 ranks below every real key
        }
        // the k-th largest key: the largest threshold with >= k keys at or above it
        for (int b = 41; b >= 0; --b) {
            const unsigned long long cand = thr | (1ull << b);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                cnt += __popcll(__ballot(key[i] >= cand));
            if (cnt >= k)
                thr = cand;
        }
        // compact the k selected keys into LDS (any order)
        int base = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const bool s = key[i] >= thr;
            const unsigned long long m = __ballot(s);
            if (s)
                sel_key[wave][base + __popcll(m & lt)] = key[i];
            base += __popcll(m);
        }
    }
    __syncthreads();
    if (active) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (key[i] >= thr) {
                int slot = 0;
                for (int q = 0; q < k; ++q)
                    slot += sel_key[wave][q] > key[i];
                a.topk_ids[(size_t)t * k + slot] = lane + kWave * i;
                sel_val[wave][slot] = val[i];
            }
        }
    }
    __syncthreads();
    if (!active)
        return;
    // the softmax's shift: the largest logit it runs over (selected, or all)
    float m = lane < k ? sel_val[wave][lane] : -INFINITY;
    if (a.method == 1) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + kWave * i < a.E)
                m = fmaxf(m, val[i]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off));
    const float ex = lane < k ? expf(sel_val[wave][lane] - m) : 0.0f;
    float sum = ex;
    if (a.method == 1) {  // the denominator runs over every expert
        sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + kWave * i < a.E)
                sum += expf(val[i] - m);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        sum += __shfl_xor(sum, off);  // xor butterfly: identical sum on every lane
    if (lane < k)
        a.topk_weights[(size_t)t * k + lane] = ex / sum;
}

} // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s)
{
    if (a.T <= 0)
        return hipSuccess;
    const int blocks = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
    if (a.E <= 64)
        hipLaunchKernelGGL((route_topk_kernel<1>), dim3(blocks), dim3(256), 0, s, a);
    else if (a.E <= 128)
        hipLaunchKernelGGL((route_topk_kernel<2>), dim3(blocks), dim3(256), 0, s, a);
    else if (a.E <= 256)
        hipLaunchKernelGGL((route_topk_kernel<4>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((route_topk_kernel<kMaxPerLane>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
