// lora_shrink_wide.hip -- LoRA shrink for (adapter, expert) segments with
// many rows (prefill).
//
// Same computation as lora_shrink_kernel in expert_gemm.hip: for every slot x
// of virtual expert (l, e), S[x, q] = sum_k X[row(x), k] * A[l, e][q, k] for
// the rank columns q < r, rounded once to bf16, zero for r <= q < rp
// ("BF16 support for the experimental_sgl_trtllm MoE-LoRA path", Flow
// section 2: the shrink is grouped by virtual expert).
//
// Design for gfx950 when segments carry tens of rows: one block (8 waves)
// per segment.  The segment's rows (gathered X rows) and the stack's rank
// rows move to LDS with direct global->LDS loads, K chunk by K chunk, eight
// chunks resident; every wave issues at most one of the chunk's loads (a
// direct load holds its wave while it issues) and waits for it with an
// explicit vmcnt before the chunk's block barrier.  Wave w owns rank tile
// w % 4 (16 columns q) and half of the M tiles, so the whole K sum of an
// output stays in one accumulator (no cross-wave reduction).  Rank rows are
// read straight in the per-lane MFMA B layout (8 consecutive K values of one
// column q per lane); activation rows are staged as swizzled A fragments.
// Needs r <= 64.  At prefill sizes the kernel streams every 128-byte line
// once and is bound by the scattered line reads of the stacks (one line per
// rank row per two K chunks), not by latency: more stages do not help.
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe_lora {
namespace {

constexpr int kSNT = 4;      // rank tiles of 16 columns: r <= 64
#ifndef MOE_LORA_SHRINK_STAGES
#define MOE_LORA_SHRINK_STAGES 8
#endif
constexpr int kSStages = MOE_LORA_SHRINK_STAGES;  // K chunks resident in LDS
#ifndef MOE_LORA_SHRINK_WAVES
#define MOE_LORA_SHRINK_WAVES 8
#endif
constexpr int kSWaves = MOE_LORA_SHRINK_WAVES;  // 4: wave w owns rank tile w; 8: and half the M tiles

template <int MT>  // M tiles per pass: 16 MT rows
__global__ __launch_bounds__(64 * kSWaves, 2) void lora_shrink_wide_kernel(ShrinkArgs a)
{
    constexpr int kRows = 16 * MT;
    constexpr int kAStage = kRows * 64;
    constexpr int kStageBytes = kAStage + kSNT * 1024;
    __shared__ __align__(1024) unsigned char smem[kSStages * kStageBytes];
    __shared__ int row_src[kRows];
    __shared__ int row_slot[kRows];
    const uint32_t smem_lds = lds_address(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();
    const int seg = blockIdx.x;  // = l * E_l + e, the stack's own order
    const int beg = a.seg_offsets[seg];
    const int n_rows = a.seg_offsets[seg + 1] - beg;
    if (n_rows <= 0)
        return;
    const int KC = a.K >> 5;
    const int NT = (a.r + 15) >> 4;
    const int stack = a.a_shared ? seg / a.E_l : seg;  // shared: one stack per adapter
    const uint16_t *A = a.A + (size_t)stack * a.r * a.K;
    const int a_lane_off = (lane & 15) * 64 + (((lane >> 4) ^ act_swizzle(lane & 15)) * 16);

    for (int pass = 0; pass < n_rows; pass += kRows) {
        const int rows = min(kRows, n_rows - pass);
        const int n_mt = (rows + 15) >> 4;
        dma_drain();     // the previous pass's direct loads have landed
        lds_barrier();   // ... in every wave, and its epilogue is done with the rows
        if (tid < kRows) {
            const int x = a.seg_slots[beg + pass + min(tid, rows - 1)];
            row_slot[tid] = x;
            row_src[tid] = a.gather_by_token ? x / a.k : a.exp2perm[x];
        }
        lds_barrier();

        // The chunk's loads j = 0 .. n_mt + NT - 1: j < n_mt are the rows of
        // M tile j (lane -> row 16 j + lane / 4, physical quarter lane % 4,
        // which holds logical quarter (lane % 4) ^ swizzle(row)); the rest
        // are rank tiles t = j - n_mt (lane -> column q = 16 t + lane % 16,
        // K quarter lane / 16; columns past r read row r - 1, never stored).
        // Wave w issues the loads j = w, w + kSWaves.
        constexpr int kLoads = (8 + kSWaves - 1) / kSWaves;  // per wave, at most
        const int n_w = (n_mt + NT - wave + kSWaves - 1) / kSWaves;  // 0 .. kLoads (uniform)
        const uint16_t *src[kLoads];
        uint32_t dst[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int j = min(wave + kSWaves * i, n_mt + NT - 1);
            if (j < n_mt) {
                const int pr = 16 * j + (lane >> 2);
                const int q = (lane & 3) ^ act_swizzle(pr);
                src[i] = a.X + (size_t)row_src[pr] * a.K + q * 8;
                dst[i] = j * 1024;
            } else {
                const int t = j - n_mt;
                const int q = min(16 * t + (lane & 15), a.r - 1);
                src[i] = A + (size_t)q * a.K + (lane >> 4) * 8;
                dst[i] = kAStage + t * 1024;
            }
        }
        auto issue = [&](int kc, int st) __attribute__((always_inline)) {
            const uint32_t base = smem_lds + (uint32_t)(st * kStageBytes);
#pragma unroll
            for (int i = 0; i < kLoads; ++i)
                if (i < n_w)
                    load_lds16(src[i] + kc * 32, base + dst[i]);
        };
        // chunk kc lives in stage kc % S; past the last chunk the last one is
        // issued again, so a wave's loads per chunk never change and chunk kc
        // has landed once only the S - 2 chunks issued after it can be
        // outstanding
        auto wait = [&]() __attribute__((always_inline)) {
            if (kLoads > 1 && n_w == 2)
                dma_wait_barrier<(kSStages - 2) * 2>();
            else if (n_w == 1)
                dma_wait_barrier<(kSStages - 2) * 1>();
            else
                dma_wait_barrier<0>();
        };

        // this wave's rank tile and M tiles m0 .. m0 + MW - 1
        constexpr int MW = MT * 4 / kSWaves;
        const int rt = wave & (kSNT - 1);
        const int m0 = (wave / kSNT) * MW;
        f32x4 acc[MW];
#pragma unroll
        for (int m = 0; m < MW; ++m)
            acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t tiles =
            __builtin_amdgcn_readfirstlane(rt < NT ? ((1u << n_mt) - 1u) >> m0 : 0u);

        for (int d = 0; d < kSStages - 1; ++d)
            issue(min(d, KC - 1), d);
        for (int kc = 0; kc < KC; ++kc) {
            wait();
            issue(min(kc + kSStages - 1, KC - 1), (kc + kSStages - 1) % kSStages);
            const unsigned char *sa = smem + (kc % kSStages) * kStageBytes;
            const u32x4 b = *reinterpret_cast<const u32x4 *>(sa + kAStage + rt * 1024 + lane * 16);
#pragma unroll
            for (int m = 0; m < MW; ++m) {
                const u32x4 av =
                    *reinterpret_cast<const u32x4 *>(sa + (m0 + m) * 1024 + a_lane_off);
                if (tiles & (1u << m))
                    acc[m] = mfma_16x16x32(av, b, acc[m]);
            }
        }

        // lane holds rows 4 (lane / 16) + i of each M tile, column lane % 16
        const int q = 16 * rt + (lane & 15);
        if (rt < NT && q < a.rp) {
#pragma unroll
            for (int m = 0; m < MW; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = (m0 + m) * 16 + 4 * (lane >> 4) + i;
                    if (m0 + m < n_mt && r < rows)
                        a.S[(size_t)row_slot[r] * a.rp + q] =
                            q < a.r ? (uint16_t)float_to_bf16_bits(acc[m][i]) : (uint16_t)0;
                }
            }
        }
    }
    dma_drain();  // no direct load may land after the block's LDS is released
}

} // namespace

bool shrink_wide_supported(int r) { return r > 0 && r <= 16 * kSNT; }

hipError_t launch_shrink_wide(const ShrinkArgs &a, int mean_rows, hipStream_t s)
{
    const int blocks = a.L * a.E_l;
    if (blocks <= 0 || a.r <= 0)
        return hipSuccess;
    if (mean_rows > 24)
        hipLaunchKernelGGL((lora_shrink_wide_kernel<4>), dim3(blocks), dim3(64 * kSWaves), 0, s, a);
    else
        hipLaunchKernelGGL((lora_shrink_wide_kernel<2>), dim3(blocks), dim3(64 * kSWaves), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
