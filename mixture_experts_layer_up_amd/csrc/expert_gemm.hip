// expert_gemm.hip -- grouped expert GEMMs and the LoRA shrink on MFMA.
//
// What is computed (per local slot p of local expert e, token t, adapter l):
//   gate_up:  h = x_t W13[e] + B_gu[l,e] s_gu[p],  s_gu[p] = A_gu[l,e] x_t
//             act[p] = SiLU(h[:I]) * h[I:]
//   down:     y[p] = act[p] W2[e] + B_dn[l,e] s_dn[p], s_dn[p] = A_dn[l,e] act[p]
// Sources: "BF16 support for the experimental_sgl_trtllm MoE-LoRA path",
// "Files changed" table, launcher row (gate_up GEMM with K = hidden and
// N = 2 * inter; the activation adds the gate_up LoRA delta before SwiGLU and
// writes the activation that the down LoRA consumes; down GEMM with K = inter,
// N = hidden) and Flow section 2 (LoRA shrink then expand per virtual expert;
// the gate_up delta is not scaled by the routing weight).
//
// Design for gfx950:
//  * One block = 4 waves = one (local expert, 64-column slab).  The packed
//    weight layout makes every B fragment a contiguous 1 KiB block, loaded by
//    one 16-byte load per lane directly into registers (no LDS round trip):
//    the weight stream is the HBM-bound part of the layer.
//  * The 4 waves split K; each keeps its own fp32 accumulators for all rows
//    of the expert (up to 64 per pass) and the partial sums are reduced
//    through LDS once per pass.  Rows beyond 64 take further passes.
//  * The LoRA expand is folded into the same MFMA accumulation as extra K:
//    row p contributes s[p] (rank r, zero-padded to rp) in the K block of its
//    own adapter and zeros elsewhere, against B[l, e]^T, so
//    acc = X W + sum_l S_l B_l^T with no separate delta buffer.  K chunks of
//    adapters absent from the pass are skipped.
//  * gate_up blocks own matching gate and up columns (packed tile order), so
//    SwiGLU runs in the epilogue and h never reaches memory.
//  * Blocks are renumbered so each XCD processes contiguous experts.
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kMT = 4;                 // M tiles (16 rows) per pass
constexpr int kNS = 4;                 // 16-column N tiles per block
constexpr int kRows = kMT * 16;        // rows per pass
constexpr int kCH = 4;                 // K chunks (32) loaded per batch
constexpr int kPartStride = kNS * 16 + 4;
constexpr int kPartFloats = 4 * kRows * kPartStride;

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[kMT][kNS])
{
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
        for (int n = 0; n < kNS; ++n)
            acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Write this wave's accumulators as [row][col] fp32 partials.
__device__ __forceinline__ void store_partials(float *part, const f32x4 (&acc)[kMT][kNS],
                                               int n_mt, int wave, int lane)
{
    float *pw = part + wave * kRows * kPartStride;
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
        if (m < n_mt) {
#pragma unroll
            for (int n = 0; n < kNS; ++n) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pw[(m * 16 + 4 * (lane >> 4) + i) * kPartStride + n * 16 + (lane & 15)] =
                        acc[m][n][i];
            }
        }
    }
}

__device__ __forceinline__ float sum_partials(const float *part, int row, int col)
{
    const int o = row * kPartStride + col;
    return (part[o] + part[kRows * kPartStride + o]) +
           (part[2 * kRows * kPartStride + o] + part[3 * kRows * kPartStride + o]);
}

// Accumulate this wave's share of the K chunks [kbeg, kend):
// acc[m][n] += A rows (via aptr) x B tiles (via bptr).
template <typename BLoad>
__device__ __forceinline__ void k_loop(f32x4 (&acc)[kMT][kNS], const uint16_t *const (&aptr)[kMT],
                                       const bool (&ok)[kMT], int n_mt, int kbeg, int kend,
                                       BLoad bload)
{
    for (int kc0 = kbeg; kc0 < kend; kc0 += kCH) {
        u32x4 b[kCH][kNS];
        u32x4 av[kCH][kMT];
#pragma unroll
        for (int c = 0; c < kCH; ++c) {
            const int kc = kc0 + c;
            if (kc < kend) {
#pragma unroll
                for (int n = 0; n < kNS; ++n)
                    b[c][n] = bload(n, kc);
#pragma unroll
                for (int m = 0; m < kMT; ++m)
                    av[c][m] = ok[m] ? load16(aptr[m] + kc * 32) : zero16();
            }
        }
#pragma unroll
        for (int c = 0; c < kCH; ++c) {
            if (kc0 + c < kend) {
#pragma unroll
                for (int m = 0; m < kMT; ++m) {
                    if (m < n_mt) {
#pragma unroll
                        for (int n = 0; n < kNS; ++n)
                            acc[m][n] = mfma_16x16x32(av[c][m], b[c][n], acc[m][n]);
                    }
                }
            }
        }
    }
}

template <bool kGated>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmArgs a)
{
    __shared__ float part[kPartFloats];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;

    const int logical = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const int le = logical / a.n_slabs;
    const int slab = logical - le * a.n_slabs;
    const int row0 = a.offsets[le];
    const int n_rows = a.offsets[le + 1] - row0;
    if (n_rows <= 0)
        return;

    const int KC = a.K >> 5;
    const int kc_per = (KC + 3) >> 2;
    const int kbeg = min(KC, wave * kc_per);
    const int kend = min(KC, kbeg + kc_per);
    const bool lora = a.S != nullptr && a.L > 0 && a.r > 0;
    const int n_ext = lora ? (a.L * a.rp + 31) >> 5 : 0;

    // B fragments of this block's 4 packed tiles: tile n, chunk kc at
    // wbase + (n * KC + kc) * 512 elements.
    const uint16_t *wbase =
        a.Wp + ((size_t)le * a.NT + (size_t)slab * kNS) * (size_t)KC * 512 + lane * 8;
    auto bload = [&](int n, int kc) { return load16(wbase + ((size_t)n * KC + kc) * 512); };

    for (int pass = 0; pass < n_rows; pass += kRows) {
        const int rows = min(kRows, n_rows - pass);
        const int n_mt = (rows + 15) >> 4;

        const uint16_t *aptr[kMT];
        bool ok[kMT];
        int prow[kMT];
        int adapter[kMT];
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
            const int r = pass + m * 16 + (lane & 15);
            ok[m] = r < n_rows;
            const int p = row0 + min(r, n_rows - 1);
            prow[m] = p;
            const int tok = a.perm2exp[p] / a.k;
            aptr[m] = a.X + (size_t)(a.gather_by_token ? tok : p) * a.K + (lane >> 4) * 8;
            const int l = (lora && a.mapping) ? a.mapping[tok] : -1;
            adapter[m] = (l >= 0 && l < a.L) ? l : -1;
        }

        f32x4 acc[kMT][kNS];
        zero_acc(acc);
        k_loop(acc, aptr, ok, n_mt, kbeg, kend, bload);

        if (n_ext > 0) {
            unsigned long long present = 0;
            for (int l = 0; l < a.L; ++l) {
                bool has = false;
#pragma unroll
                for (int m = 0; m < kMT; ++m)
                    has |= ok[m] && adapter[m] == l;
                if (__ballot(has))
                    present |= 1ull << l;
            }
            for (int c = wave; c < n_ext; c += 4) {
                const int lo = (c * 32) / a.rp;
                const int hi = min(a.L - 1, (c * 32 + 31) / a.rp);
                const int span = hi - lo + 1;
                const unsigned long long mask = span >= 64 ? ~0ull : ((1ull << span) - 1ull);
                if (((present >> lo) & mask) == 0)
                    continue;
                const int g = c * 32 + (lane >> 4) * 8;
                const int aid = g / a.rp;
                const int q0 = g - aid * a.rp;
                u32x4 av[kMT];
                u32x4 b[kNS];
#pragma unroll
                for (int m = 0; m < kMT; ++m)
                    av[m] = (ok[m] && adapter[m] == aid)
                                ? load16(a.S + (size_t)prow[m] * a.rp + q0)
                                : zero16();
#pragma unroll
                for (int n = 0; n < kNS; ++n) {
                    b[n] = zero16();
                    if (aid < a.L) {
                        const int col = kGated
                                            ? (n & 1) * a.I + (slab * 2 + (n >> 1)) * 16 + (lane & 15)
                                            : (slab * kNS + n) * 16 + (lane & 15);
                        const uint16_t *src =
                            a.LB + (((size_t)aid * a.E_l + le) * a.n_canon + col) * a.r + q0;
                        if ((a.r & 7) == 0) {
                            b[n] = load16(src);
                        } else {
                            uint32_t w[4] = {0u, 0u, 0u, 0u};
                            for (int i = 0; i < 8; ++i)
                                if (q0 + i < a.r)
                                    w[i >> 1] |= (uint32_t)src[i] << (16 * (i & 1));
                            b[n] = u32x4{w[0], w[1], w[2], w[3]};
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < kMT; ++m) {
                    if (m < n_mt) {
#pragma unroll
                        for (int n = 0; n < kNS; ++n)
                            acc[m][n] = mfma_16x16x32(av[m], b[n], acc[m][n]);
                    }
                }
            }
        }

        __syncthreads();  // the previous pass's epilogue is done with `part`
        store_partials(part, acc, n_mt, wave, lane);
        __syncthreads();

        if (kGated) {
            // 32 activation columns per row: 4 groups of 8 (pair jj, half c0)
            for (int item = tid; item < rows * 4; item += 256) {
                const int row = item >> 2;
                const int jj = (item >> 1) & 1;
                const int c0 = (item & 1) * 8;
                uint32_t packed[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    float v[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float gate = sum_partials(part, row, (2 * jj) * 16 + c0 + i + h);
                        const float up = sum_partials(part, row, (2 * jj + 1) * 16 + c0 + i + h);
                        v[h] = silu_f32(gate) * up;
                    }
                    packed[i >> 1] = float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16);
                }
                const int p = row0 + pass + row;
                store16(a.Y + (size_t)p * a.I + (slab * 2 + jj) * 16 + c0,
                        u32x4{packed[0], packed[1], packed[2], packed[3]});
            }
        } else {
            // 64 output columns per row: 8 groups of 8
            for (int item = tid; item < rows * 8; item += 256) {
                const int row = item >> 3;
                const int c0 = (item & 7) * 8;
                uint32_t packed[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const float v0 = sum_partials(part, row, c0 + i);
                    const float v1 = sum_partials(part, row, c0 + i + 1);
                    packed[i >> 1] = float_to_bf16_bits(v0) | (float_to_bf16_bits(v1) << 16);
                }
                const int p = row0 + pass + row;
                store16(a.Y + (size_t)p * a.n_canon + slab * 64 + c0,
                        u32x4{packed[0], packed[1], packed[2], packed[3]});
            }
        }
    }
}

// LoRA shrink: S[p, 0:rp] = A[l, e] x_p for the slots of one virtual expert
// (adapter l, local expert e) per block; q >= r is written as 0.  The LoRA A
// stack [r, K] is K-contiguous, which is exactly the per-lane B operand
// layout of the MFMA (8 consecutive K values of one column q).
__global__ __launch_bounds__(256) void lora_shrink_kernel(ShrinkArgs a)
{
    __shared__ float part[kPartFloats];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int seg = blockIdx.x;  // = l * E_l + e, the stack's own order
    const int beg = a.seg_offsets[seg];
    const int n_rows = a.seg_offsets[seg + 1] - beg;
    if (n_rows <= 0)
        return;

    const int KC = a.K >> 5;
    const int kc_per = (KC + 3) >> 2;
    const int kbeg = min(KC, wave * kc_per);
    const int kend = min(KC, kbeg + kc_per);
    const int n_nt = (a.r + 15) >> 4;
    const uint16_t *abase = a.A + (size_t)seg * a.r * a.K + (lane >> 4) * 8;

    for (int pass = 0; pass < n_rows; pass += kRows) {
        const int rows = min(kRows, n_rows - pass);
        const int n_mt = (rows + 15) >> 4;
        const uint16_t *aptr[kMT];
        bool ok[kMT];
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
            const int r = pass + m * 16 + (lane & 15);
            ok[m] = r < n_rows;
            const int x = a.seg_slots[beg + min(r, n_rows - 1)];
            const int p = a.exp2perm[x];
            aptr[m] = a.X + (size_t)(a.gather_by_token ? x / a.k : p) * a.K + (lane >> 4) * 8;
        }
        for (int nt0 = 0; nt0 < n_nt; nt0 += kNS) {
            auto bload = [&](int n, int kc) {
                const int q = (nt0 + n) * 16 + (lane & 15);
                return q < a.r ? load16(abase + (size_t)q * a.K + kc * 32) : zero16();
            };
            f32x4 acc[kMT][kNS];
            zero_acc(acc);
            k_loop(acc, aptr, ok, n_mt, kbeg, kend, bload);

            __syncthreads();
            store_partials(part, acc, n_mt, wave, lane);
            __syncthreads();

            const int groups = min(kNS, n_nt - nt0) * 2;  // 8-wide q groups in this tile range
            for (int item = tid; item < rows * groups; item += 256) {
                const int row = item / groups;
                const int g = item - row * groups;
                const int q0 = nt0 * 16 + g * 8;
                if (q0 >= a.rp)
                    continue;
                uint32_t packed[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const float v0 = (q0 + i < a.r) ? sum_partials(part, row, g * 8 + i) : 0.0f;
                    const float v1 = (q0 + i + 1 < a.r) ? sum_partials(part, row, g * 8 + i + 1) : 0.0f;
                    packed[i >> 1] = float_to_bf16_bits(v0) | (float_to_bf16_bits(v1) << 16);
                }
                const int x = a.seg_slots[beg + pass + row];
                const int p = a.exp2perm[x];
                store16(a.S + (size_t)p * a.rp + q0, u32x4{packed[0], packed[1], packed[2], packed[3]});
            }
        }
    }
}

} // namespace

hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s)
{
    const int blocks = a.E_l * a.n_slabs;
    if (blocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((expert_gemm_kernel<true>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s)
{
    const int blocks = a.E_l * a.n_slabs;
    if (blocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((expert_gemm_kernel<false>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t s)
{
    const int blocks = a.L * a.E_l;
    if (blocks <= 0 || a.r <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(lora_shrink_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
