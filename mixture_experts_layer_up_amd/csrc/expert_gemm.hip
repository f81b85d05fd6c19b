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
//  * Work list: the permute kernel cuts every expert's rows into tiles of at
//    most 16 * MT rows.  One block = 4 waves = one (tile, 64-column slab).
//    Tiles of the same expert are numbered next to each other, so blocks that
//    stream the same weight slab run at the same time on the same XCD and the
//    slab comes from HBM once.
//  * The packed weight layout makes every B fragment a contiguous 1 KiB
//    block, loaded by one 16-byte load per lane straight into registers (no
//    LDS): the weight stream is the HBM-bound part of the layer.
//  * The 4 waves split K.  Each wave runs a two-stage software pipeline over
//    its K chunks (the loads of stage s + 1 are in flight while stage s
//    multiplies); the first stage's weight loads are issued before the row
//    lookups, which are a chain of dependent loads.  Partial sums are reduced
//    through LDS at the end.
//  * The LoRA expand is folded into the same accumulation as extra K chunks
//    at the end of each wave's sequence: row p contributes s[p] (rank r,
//    zero-padded to rp) in the K block of its own adapter and zeros
//    elsewhere, against B[l, e]^T, so acc = X W + sum_l S_l B_l^T and no
//    delta buffer exists.
//  * gate_up blocks own matching gate and up columns (packed tile order), so
//    SwiGLU runs in the epilogue and h never reaches memory.
//  * Every load in the pipeline is issued unconditionally (indices clamped,
//    values masked afterwards) so all paths have the same number of
//    outstanding loads and the compiler's wait counts stay exact.
#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "gemm_index.h"
#include "kernels.h"
#include "lora_shrink_rows.h"
#include "mfma_pipeline.h"

namespace moe_lora {
namespace {

// Tuning knobs of the decode-shaped (16-row tile) GEMM: K chunks per
// pipeline stage, and the minimum waves per SIMD the register budget targets.
#ifndef MOE_LORA_DECODE_CH
#define MOE_LORA_DECODE_CH 1
#endif
#ifndef MOE_LORA_DECODE_WAVES
#define MOE_LORA_DECODE_WAVES 5
#endif

template <int MT, int CH, bool kGated, bool kRank8>
__global__ __launch_bounds__(256, MT == 1 ? (kRank8 ? MOE_LORA_DECODE_WAVES : 3) : 1) void expert_gemm_kernel(GemmArgs a)
{
    constexpr int NS = kNS;
    __shared__ float part[Part<MT>::kFloats];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();

    // Work item -> (expert, slab, row tile).  The items of one expert occupy
    // logical ids [tb * n_slabs, (tb + nt) * n_slabs); inside that range the
    // nt row tiles of one slab are adjacent, so blocks that read the same
    // weight slab are dispatched together on one XCD and share its L2.
    const int logical = xcd_balanced_item(blockIdx.x, *a.tile_count * a.n_slabs);
    if (logical < 0)
        return;
    const int4 te = a.tiles[logical / a.n_slabs];
    const int le = te.x;
    if (le < 0)
        return;
    const int nt = (te.z + a.tile_rows - 1) / a.tile_rows;
    const int in_expert = logical - te.w * a.n_slabs;
    const int slab = in_expert / nt;
    const int sub = in_expert - slab * nt;
    const int row0 = te.y + sub * a.tile_rows;
    const int n_rows = min(a.tile_rows, te.z - sub * a.tile_rows);  // 1 .. 16 * MT
    const int n_mt = (n_rows + 15) >> 4;

    // waves take K chunks round-robin (wave w: chunks w, w + 4, ...), so the
    // block's loads at any moment cover one contiguous stretch of its slab
    const int KC = a.K >> 5;
    const int nm = decode_main_chunks(KC, wave);  // this wave's main chunks
    const bool lora = a.S != nullptr && a.L > 0 && a.r > 0;
    const int n_ext = lora ? (a.L * a.rp + 31) >> 5 : 0;
    const int ne = wave < n_ext ? (n_ext - wave + 3) >> 2 : 0;  // ext chunks wave, wave+4, ..
    const int nv = nm + ne;

    // Branch-free loaders: every chunk issues the same loads, at addresses
    // that are always valid (gemm_index.h), and values are masked instead.
    const DecodeBShape bs{KC, NS, a.n_slabs, kGated ? 1 : 0, a.I, a.L, a.r, a.rp,
                          a.E_l, a.n_canon, a.lb_shared};
    const uint16_t *lb = a.LB ? a.LB : a.Wp;
    auto load_b = [&](int vc, u32x4 (&b)[NS]) {
        const bool main = vc < nm;  // uniform
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const DecodeBLoad d = decode_b_load(bs, wave, lane, vc, nm, le, slab, n);
            if (kRank8) {
                // past the last adapter (aid >= L) the last stack is read; its
                // K positions meet zero activations, so it adds nothing
                b[n] = load16_stream((main ? a.Wp : lb) + d.off16);
            } else {  // rank not a multiple of 8: the expand rows need 2-byte loads
                const u32x4 vm = load16_stream(a.Wp + d.off16);
                const uint16_t *pe = lb + d.lora_row;
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const uint32_t lo = pe[min(d.q0 + i, a.r - 1)];
                    const uint32_t hi = pe[min(d.q0 + i + 1, a.r - 1)];
                    w[i >> 1] = (d.q0 + i < a.r ? lo : 0u) | ((d.q0 + i + 1 < a.r ? hi : 0u) << 16);
                }
                const u32x4 ve = keep_if(u32x4{w[0], w[1], w[2], w[3]}, d.aid < a.L);
                b[n] = main ? vm : ve;
            }
        }
    };

    Stage<MT, NS, CH> s0, s1;
    const bool early = nm >= CH;
    if (early) {  // weight loads of stage 0 do not depend on the rows
#pragma unroll
        for (int c = 0; c < CH; ++c)
            load_b(c, s0.b[c]);
    }

    // rows of this tile; lanes past the tile's rows read a clamped valid row
    const uint16_t *aptr[MT];
    int xslot[MT];
    int adapter[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int r = m * 16 + (lane & 15);
        const int p = row0 + min(r, n_rows - 1);
        const int x = a.perm2exp[p];
        xslot[m] = x;
        const int tok = x / a.k;
        aptr[m] = a.X + (size_t)(a.gather_by_token ? tok : p) * a.K + (lane >> 4) * 8;
        const int l = (lora && a.mapping) ? a.mapping[tok] : -1;
        adapter[m] = (l >= 0 && l < a.L) ? l : -1;
    }
    // rows past the tile read a clamped valid row and are never stored: main
    // chunks need no mask; expand chunks keep only the row's own adapter block
    const uint16_t *sbase = a.S ? a.S : a.X;
    auto load_a = [&](int vc, u32x4 (&av)[MT], bool (&am)[MT]) {
        const bool main = vc < nm;  // uniform
        const int kc = wave + 4 * (main ? vc : 0);
        const int g = ((vc - nm) * 4 + wave) * 32 + (lane >> 4) * 8;
        const int aid = main ? -1 : g / a.rp;
        const int q0 = main ? 0 : g - aid * a.rp;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < n_mt) {
                const uint16_t *pa = main ? aptr[m] + kc * 32 : sbase + (size_t)xslot[m] * a.rp + q0;
                av[m] = load16(pa);
                am[m] = main || adapter[m] == aid;
            }
        }
    };

    f32x4 acc[MT][NS];
    zero_acc(acc);
    run_pipeline<MT, NS, CH>(acc, nv, n_mt, s0, s1, early, load_b, load_a);

    store_partials<MT, NS>(part, acc, n_mt, wave, lane);
    __syncthreads();

    if (kGated) {
        // 32 activation columns per row: 4 groups of 8 (gate/up pair jj, half c0)
        for (int item = tid; item < n_rows * 4; item += 256) {
            const int row = item >> 2;
            const int jj = (item >> 1) & 1;
            const int c0 = (item & 1) * 8;
            uint32_t packed[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                float v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float gate = sum_partials<MT>(part, row, (2 * jj) * 16 + c0 + i + h);
                    const float up = sum_partials<MT>(part, row, (2 * jj + 1) * 16 + c0 + i + h);
                    v[h] = silu_f32(gate) * up;
                }
                packed[i >> 1] = float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16);
            }
            store16(a.Y + (size_t)(row0 + row) * a.I + (slab * 2 + jj) * 16 + c0,
                    u32x4{packed[0], packed[1], packed[2], packed[3]});
        }
    } else {
        // 64 output columns per row: 8 groups of 8
        for (int item = tid; item < n_rows * 8; item += 256) {
            const int row = item >> 3;
            const int c0 = (item & 7) * 8;
            uint32_t packed[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const float v0 = sum_partials<MT>(part, row, c0 + i);
                const float v1 = sum_partials<MT>(part, row, c0 + i + 1);
                packed[i >> 1] = float_to_bf16_bits(v0) | (float_to_bf16_bits(v1) << 16);
            }
            store16(a.Y + (size_t)(row0 + row) * a.n_canon + slab * 64 + c0,
                    u32x4{packed[0], packed[1], packed[2], packed[3]});
        }
    }
}

// LoRA shrink over the (adapter, expert) segments the permute wrote: one
// block per virtual expert, its rows from the segment's slot list.
template <int NS, int CH, int MT>
__global__ __launch_bounds__(256, 2) void lora_shrink_kernel(ShrinkArgs a)
{
    __shared__ float part[Part<MT>::kFloats];
    __shared__ int row_slot[16 * MT];
    const int seg = blockIdx.x;  // = l * E_l + e, the stack's own order
    const int beg = a.seg_offsets[seg];
    const int n_rows = a.seg_offsets[seg + 1] - beg;
    if (n_rows <= 0)
        return;
    const int stack = a.a_shared ? seg / a.E_l : seg;  // shared: one stack per adapter
    shrink_rows<NS, CH, MT>(a, stack, n_rows, [&](int i) { return a.seg_slots[beg + i]; },
                            part, row_slot);
}

template <int MT, int CH, bool kGated>
hipError_t launch_gemm_variant(const GemmArgs &a, hipStream_t s)
{
    const int blocks = gemm_grid_blocks(a.n_tiles, a.n_slabs);
    if (blocks <= 0)
        return hipSuccess;
    if ((a.r & 7) == 0)
        hipLaunchKernelGGL((expert_gemm_kernel<MT, CH, kGated, true>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((expert_gemm_kernel<MT, CH, kGated, false>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace

int gemm_tile_rows(int n_slots, int E_l, int H, int I, int r_gu, int r_dn)
{
    // the wide kernel once experts average 32 or more rows
    if (n_slots < 32 * E_l || !gemm_wide_supported(H, I, r_gu, r_dn))
        return kDecodeTileRows;
    // Every wide work item streams whole 256-column weight slabs whatever
    // its rows, so a launch costs about ceil(items / resident blocks) item
    // times: an expert split over two tiles adds a nearly empty item per
    // slab, and a few of those start a whole extra round.  Tiles therefore
    // cover the mean rows per expert plus four standard deviations of a
    // Poisson count (rounded up to 16), up to the kernel's maximum.
    const double mean = (double)n_slots / E_l;
    const int want = (int)std::ceil(mean + 4.0 * std::sqrt(mean));
    return std::min(kWideMaxTileRows, (want + 15) / 16 * 16);
}

hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s)
{
    return a.tile_rows == kDecodeTileRows ? launch_gemm_variant<1, MOE_LORA_DECODE_CH, true>(a, s)
                                          : launch_gemm_wide(a, true, s);
}

hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s)
{
    return a.tile_rows == kDecodeTileRows ? launch_gemm_variant<1, MOE_LORA_DECODE_CH, false>(a, s)
                                          : launch_gemm_wide(a, false, s);
}

bool shrink_uses_wide(const ShrinkArgs &a)
{
    // rows per (adapter, expert) segment, on average, when every slot
    // carries an adapter; segments of tens of rows take the direct-load
    // kernel (lora_shrink_wide.hip)
    const int blocks = a.L * a.E_l;
    const int mean = blocks > 0 ? (a.n_slots + blocks - 1) / blocks : 0;
    return mean >= 16 && shrink_wide_supported(a.r);
}

int shrink_row_tiles(const ShrinkArgs &a)
{
    // rows per pass from the mean rows per segment: one pass covers most
    // segments
    const int blocks = a.L * a.E_l;
    const int mean = blocks > 0 ? (a.n_slots + blocks - 1) / blocks : 0;
    return mean <= 8 ? 1 : mean <= 24 ? 2 : 3;
}

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t s)
{
    const int blocks = a.L * a.E_l;
    if (blocks <= 0 || a.r <= 0)
        return hipSuccess;
    if (shrink_uses_wide(a))
        return launch_shrink_wide(a, (a.n_slots + blocks - 1) / blocks, s);
    with_shrink_shape(a.r, shrink_row_tiles(a), [&](auto ns, auto ch, auto mt) {
        hipLaunchKernelGGL((lora_shrink_kernel<decltype(ns)::value, decltype(ch)::value,
                                               decltype(mt)::value>),
                           dim3(blocks), dim3(256), 0, s, a);
    });
    return hipGetLastError();
}

} // namespace moe_lora
