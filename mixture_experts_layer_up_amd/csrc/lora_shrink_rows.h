// lora_shrink_rows.h -- the LoRA shrink of one virtual expert's rows.
//
// S[x, 0:rp] = A[l, e] x_row for the slots x of one virtual expert (adapter
// l, local expert e), 16 * MT rows per pass; q >= r is written as 0.  S is
// indexed by slot, so the gate_up shrink (rows = the slots' tokens) needs no
// permutation lookup at all.  The stack A[l, e] (r x K, packed in 64-value K
// chunks, kernels.h) is K-contiguous per rank row inside a chunk, which is
// exactly the per-lane B operand layout of the MFMA (8 consecutive K values
// of one column q).  NS 16-column tiles of q per pass over N; the block's 4
// waves split K.  Sources: "BF16 support for the
// experimental_sgl_trtllm MoE-LoRA path", Flow section 2 (shrink then expand
// per virtual expert), and the "PR #28091 report", key source snippets (the
// shrink intermediate has one rank-r row per (token, top-k choice)).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "mfma_pipeline.h"

namespace moe_lora {
namespace {

// The block's rows are slot_of(0 .. n_rows - 1) (n_rows > 0); `stack` is the
// index of A[l, e] in the stack array.  part and row_slot are the block's LDS
// (Part<MT>::kFloats and 16 * MT entries).  All 256 threads call it.
template <int NS, int CH, int MT, typename SlotOf>
__device__ __forceinline__ void shrink_rows(const ShrinkArgs &a, int stack, int n_rows,
                                            SlotOf slot_of, float *part, int *row_slot)
{
    constexpr int kRows = 16 * MT;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();
    const int KC = a.K >> 5;
    const int kc_per = (KC + 3) >> 2;
    const int kbeg = min(KC, wave * kc_per);
    const int nm = min(KC, kbeg + kc_per) - kbeg;
    const int n_nt = (a.r + 15) >> 4;
    // the packed stack: 64-value K chunks, each holding the r rank rows
    const uint16_t *abase =
        a.A + (size_t)stack * lora_a_chunks(a.K) * a.r * 64 + (lane >> 4) * 8;

    Stage<MT, NS, CH> s0, s1;
    auto load_b_nt = [&](int nt0, int vc, u32x4 (&b)[NS]) {
        const int kc = kbeg + vc;  // 32-value chunk: half kc % 2 of packed chunk kc / 2
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const int q = (nt0 + n) * 16 + (lane & 15);
            // q >= r reads a clamped valid row; those output columns are not stored
            b[n] = load16_stream(abase + ((size_t)(kc >> 1) * a.r + min(q, a.r - 1)) * 64 +
                                 (kc & 1) * 32);
        }
    };
    // the stack's first stage does not depend on the rows: issue it before
    // the dependent row lookups
    const bool early = nm >= CH;
    if (early) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
            load_b_nt(0, c, s0.b[c]);
    }

    bool first = true;
    for (int pass = 0; pass < n_rows; pass += kRows) {
        const int rows = min(kRows, n_rows - pass);
        const int n_mt = (rows + 15) >> 4;
        // this lane's row in each M tile (past the segment: its last row,
        // computed but never stored)
        const uint16_t *aptr[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int x = slot_of(min(pass + m * 16 + (lane & 15), n_rows - 1));
            const int xrow = a.gather_by_token ? x / a.k : a.exp2perm[x];
            aptr[m] = a.X + (size_t)xrow * a.K + (lane >> 4) * 8;
        }
        lds_barrier();  // the previous pass's epilogue is done with row_slot
        if (tid < kRows)
            row_slot[tid] = slot_of(min(pass + tid, n_rows - 1));
        auto load_a = [&](int vc, u32x4 (&av)[MT], bool (&am)[MT]) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < n_mt) {
                    av[m] = load16(aptr[m] + (kbeg + vc) * 32);
                    am[m] = true;
                }
            }
        };
        for (int nt0 = 0; nt0 < n_nt; nt0 += NS) {
            auto load_b = [&](int vc, u32x4 (&b)[NS]) { load_b_nt(nt0, vc, b); };
            f32x4 acc[MT][NS];
            zero_acc(acc);
            run_pipeline<MT, NS, CH>(acc, nm, n_mt, s0, s1, first && early, load_b, load_a);
            first = false;

            lds_barrier();  // the previous epilogue is done with `part`
            store_partials<MT, NS>(part, acc, n_mt, wave, lane);
            lds_barrier();

            const int groups = min(NS, n_nt - nt0) * 2;  // 8-wide q groups
            for (int item = tid; item < rows * groups; item += 256) {
                const int row = item / groups;
                const int g = item - row * groups;
                const int q0 = nt0 * 16 + g * 8;
                if (q0 >= a.rp)
                    continue;
                uint32_t packed[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const float v0 = (q0 + i < a.r) ? sum_partials<MT>(part, row, g * 8 + i) : 0.0f;
                    const float v1 =
                        (q0 + i + 1 < a.r) ? sum_partials<MT>(part, row, g * 8 + i + 1) : 0.0f;
                    packed[i >> 1] = float_to_bf16_bits(v0) | (float_to_bf16_bits(v1) << 16);
                }
                store16(a.S + (size_t)row_slot[row] * a.rp + q0,
                        u32x4{packed[0], packed[1], packed[2], packed[3]});
            }
        }
    }
}

// The few-row shrink's tile shape for rank r with mt M tiles per pass (NS
// rank tiles of 16 per pass over N, CH K chunks per pipeline stage): every
// launch of shrink_rows takes it from here, so that they all compute each
// row alike, bit for bit.  f(NS, CH, MT) receives std::integral_constant
// values.
template <typename F>
__host__ __forceinline__ void with_shrink_shape(int r, int mt, F f)
{
    using std::integral_constant;
    if (r <= 16) {
        if (mt == 1)
            f(integral_constant<int, 1>{}, integral_constant<int, 8>{}, integral_constant<int, 1>{});
        else if (mt == 2)
            f(integral_constant<int, 1>{}, integral_constant<int, 4>{}, integral_constant<int, 2>{});
        else
            f(integral_constant<int, 1>{}, integral_constant<int, 4>{}, integral_constant<int, 3>{});
    } else {
        if (mt == 1)
            f(integral_constant<int, 4>{}, integral_constant<int, 2>{}, integral_constant<int, 1>{});
        else if (mt == 2)
            f(integral_constant<int, 4>{}, integral_constant<int, 2>{}, integral_constant<int, 2>{});
        else
            f(integral_constant<int, 4>{}, integral_constant<int, 2>{}, integral_constant<int, 3>{});
    }
}

} // namespace
} // namespace moe_lora
