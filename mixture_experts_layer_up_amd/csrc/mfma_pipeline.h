// mfma_pipeline.h -- register-pipelined MFMA helpers shared by the
// decode-shaped GEMM and the LoRA shrink kernels: the per-wave fp32 partial
// tiles reduced through LDS, and the two-stage load/multiply pipeline over a
// wave's K chunks.
#pragma once

#include "device_common.h"

namespace moe_lora {
namespace {

constexpr int kNS = 4;  // 16-column N tiles per block (64 columns)

template <int MT>
struct Part {
    static constexpr int kRows = MT * 16;
    static constexpr int kStride = kNS * 16 + 4;
    static constexpr int kWaveFloats = kRows * kStride;
    static constexpr int kFloats = 4 * kWaveFloats;
};

template <int MT, int NS>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MT][NS])
{
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NS; ++n)
            acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Write this wave's accumulators as [row][col] fp32 partials (col < 16 * NS).
template <int MT, int NS>
__device__ __forceinline__ void store_partials(float *part, const f32x4 (&acc)[MT][NS],
                                               int n_mt, int wave, int lane)
{
    float *pw = part + wave * Part<MT>::kWaveFloats;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < n_mt) {
#pragma unroll
            for (int n = 0; n < NS; ++n) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pw[(m * 16 + 4 * (lane >> 4) + i) * Part<MT>::kStride + n * 16 + (lane & 15)] =
                        acc[m][n][i];
            }
        }
    }
}

template <int MT>
__device__ __forceinline__ float sum_partials(const float *part, int row, int col)
{
    constexpr int W = Part<MT>::kWaveFloats;
    const int o = row * Part<MT>::kStride + col;
    return (part[o] + part[W + o]) + (part[2 * W + o] + part[3 * W + o]);
}

template <int MT, int NS, int CH>
struct Stage {
    u32x4 b[CH][NS];
    u32x4 a[CH][MT];
    bool am[CH][MT];  // applied to a[][] only when the MFMA consumes it
};

// Two-stage pipeline over virtual chunks [0, nv).  load_b(vc, b[NS]) and
// load_a(vc, a[MT], am[MT]) fill one chunk's operands (am: keep-mask of each A
// fragment, applied at the MFMA so that no load result is consumed early);
// s0.b may already hold the first stage's B operands (b0_ready).
template <int MT, int NS, int CH, typename LoadB, typename LoadA>
__device__ __forceinline__ void run_pipeline(f32x4 (&acc)[MT][NS], int nv, int n_mt,
                                             Stage<MT, NS, CH> &s0, Stage<MT, NS, CH> &s1,
                                             bool b0_ready, LoadB load_b, LoadA load_a)
{
    if (nv <= 0)
        return;
    auto load_stage = [&](Stage<MT, NS, CH> &st, int vc0, bool with_b) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int vc = min(vc0 + c, nv - 1);
            if (with_b)
                load_b(vc, st.b[c]);
            load_a(vc, st.a[c], st.am[c]);
        }
    };
    auto compute_stage = [&](const Stage<MT, NS, CH> &st, int vc0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (vc0 + c < nv) {
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < n_mt) {
                        const u32x4 av = keep_if(st.a[c][m], st.am[c][m]);
#pragma unroll
                        for (int n = 0; n < NS; ++n)
                            acc[m][n] = mfma_16x16x32(av, st.b[c][n], acc[m][n]);
                    }
                }
            }
        }
    };
    load_stage(s0, 0, !b0_ready);
    int vc0 = 0;
    while (true) {
        const int v1 = vc0 + CH;
        if (v1 < nv)
            load_stage(s1, v1, true);
        compute_stage(s0, vc0);
        if (v1 >= nv)
            break;
        const int v2 = v1 + CH;
        if (v2 < nv)
            load_stage(s0, v2, true);
        compute_stage(s1, v1);
        if (v2 >= nv)
            break;
        vc0 = v2;
    }
}

} // namespace
} // namespace moe_lora
