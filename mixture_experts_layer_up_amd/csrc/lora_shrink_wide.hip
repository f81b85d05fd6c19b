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
// rows move to LDS with direct global->LDS loads, K chunk by K chunk.  The
// stack is in the packed layout (kernels.h): a chunk's rank rows are one
// contiguous run, which reads ~15% faster than r rows 2K bytes apart.
//  * A chunk is 64 K values, so each row contributes one whole 128-byte line
//    per chunk, and one direct load moves 8 rows x 128 bytes.  (Chunks of 32
//    K values read half lines, 16 rows per load: twice the line requests per
//    byte, and the per-CU request path, not HBM, bounded the kernel.)
//  * Inside a row the eight 16-byte pieces are XOR-swizzled by bits 1..3 of
//    the row, so the MFMA fragment reads (16 rows x one piece) hit distinct
//    LDS banks; a direct load writes 1 KiB contiguously.
//  * Every wave issues at most two of the chunk's loads and waits for them
//    with an explicit vmcnt before the chunk's block barrier.  Wave w owns
//    rank tile w % 4 (16 columns q) and half of the M tiles, so the whole K
//    sum of an output stays in one accumulator (no cross-wave reduction).
//  * Blocks take the segments in XCD-contiguous ranges (xcd_balanced_item):
//    consecutive segments are one adapter's, so an XCD's L2 serves the
//    gathered rows of few adapters' tokens.
// Needs r <= 64.  When K is not a multiple of 64, the last chunk holds 32 K
// values: its upper pieces re-read the lower ones (valid addresses) and its
// second MFMA step is skipped.
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe_lora {
namespace {

constexpr int kSNT = 4;          // rank tiles of 16 columns: r <= 64
constexpr int kSWaves = 8;
constexpr int kRowBytes = 128;   // one 64-value K chunk of a row: one cache line

// physical 16-byte slot of logical piece p (0..7) of LDS row `row`: p ^ swizzle
__device__ __forceinline__ int line_swizzle(int row) { return (row >> 1) & 7; }

template <int MT, int S>  // M tiles per pass (16 MT rows), K chunks resident in LDS
__global__ __launch_bounds__(64 * kSWaves, 2) void lora_shrink_wide_kernel(ShrinkArgs a)
{
    constexpr int kRows = 16 * MT;
    constexpr int kAStage = kRows * kRowBytes;                 // activation rows
    constexpr int kStageBytes = kAStage + 16 * kSNT * kRowBytes;  // + 64 rank rows
    constexpr int kLoads = (2 * MT + 2 * kSNT + kSWaves - 1) / kSWaves;  // per wave, at most
    static_assert(kLoads <= 2, "the waits below handle one or two loads per wave");
    __shared__ __align__(1024) unsigned char smem[S * kStageBytes];
    __shared__ int row_src[kRows];
    __shared__ int row_slot[kRows];
    const uint32_t smem_lds = lds_address(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();
    const int seg = xcd_balanced_item(blockIdx.x, a.L * a.E_l);  // = l * E_l + e
    if (seg < 0)
        return;
    const int beg = a.seg_offsets[seg];
    const int n_rows = a.seg_offsets[seg + 1] - beg;
    if (n_rows <= 0)
        return;
    const int KC = (a.K + 63) >> 6;
    const bool half_tail = (a.K & 63) != 0;  // the last chunk holds 32 K values
    const int NT = (a.r + 15) >> 4;
    const int stack = a.a_shared ? seg / a.E_l : seg;  // shared: one stack per adapter
    // the packed stack: chunk kc's r rank rows are one contiguous run of r x 128 bytes
    const uint16_t *A = a.A + (size_t)stack * KC * a.r * 64;

    // this wave's rank tile and M tiles m0 .. m0 + MW - 1
    constexpr int MW = MT * 4 / kSWaves;
    const int rt = wave & (kSNT - 1);
    const int m0 = (wave / kSNT) * MW;
    // per-lane LDS offsets of the fragment reads, piece (lane / 16) of step 0;
    // step 1 reads piece 4 + lane / 16
    const int fr = lane & 15;

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

        // The chunk's loads j = 0 .. n_j - 1: j < 2 n_mt are activation rows
        // 8j .. 8j + 7, the rest rank rows 8 (j - 2 n_mt) .. + 7 (rows past r
        // read row r - 1, never stored).  Lane l fills row 8j + l / 8 of its
        // group, physical slot l % 8, which holds logical piece (l % 8) ^
        // swizzle(row).  Wave w issues the loads j = w, w + kSWaves.
        const int n_j = 2 * n_mt + 2 * NT;
        const int n_w = (n_j - wave + kSWaves - 1) / kSWaves;  // 0 .. kLoads (uniform)
        const uint16_t *src[kLoads];
        uint32_t dst[kLoads];
        int piece[kLoads];
        int step[kLoads];  // elements from one chunk to the next
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int j = min(wave + kSWaves * i, n_j - 1);
            if (j < 2 * n_mt) {
                const int row = 8 * j + (lane >> 3);
                piece[i] = (lane & 7) ^ line_swizzle(row);
                src[i] = a.X + (size_t)row_src[row] * a.K;
                step[i] = 64;
                dst[i] = j * 1024;
            } else {
                const int q = 8 * (j - 2 * n_mt) + (lane >> 3);
                piece[i] = (lane & 7) ^ line_swizzle(q);
                src[i] = A + (size_t)min(q, a.r - 1) * 64;
                step[i] = a.r * 64;
                dst[i] = kAStage + (j - 2 * n_mt) * 1024;
            }
        }
        auto issue = [&](int kc, int st) __attribute__((always_inline)) {
            const uint32_t base = smem_lds + (uint32_t)(st * kStageBytes);
            const bool tail = half_tail && kc == KC - 1;  // pieces 4..7 lie past K
#pragma unroll
            for (int i = 0; i < kLoads; ++i)
                if (i < n_w)
                    load_lds16(src[i] + (size_t)kc * step[i] +
                                   (tail ? (piece[i] & 3) : piece[i]) * 8,
                               __builtin_amdgcn_readfirstlane(base + dst[i]));
        };
        // chunk kc lives in stage kc % S; past the last chunk the last one is
        // issued again, so a wave's loads per chunk never change and chunk kc
        // has landed once only the S - 2 chunks issued after it can be
        // outstanding
        auto wait = [&]() __attribute__((always_inline)) {
            if (n_w == 2)
                dma_wait_barrier<(S - 2) * 2>();
            else if (n_w == 1)
                dma_wait_barrier<(S - 2) * 1>();
            else
                dma_wait_barrier<0>();
        };

        f32x4 acc[MW];
#pragma unroll
        for (int m = 0; m < MW; ++m)
            acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t tiles =
            __builtin_amdgcn_readfirstlane(rt < NT ? ((1u << n_mt) - 1u) >> m0 : 0u);

        for (int d = 0; d < S - 1; ++d)
            issue(min(d, KC - 1), d);
        for (int kc = 0; kc < KC; ++kc) {
            wait();
            issue(min(kc + S - 1, KC - 1), (kc + S - 1) % S);
            const unsigned char *sa = smem + (kc % S) * kStageBytes;
            const int steps = (half_tail && kc == KC - 1) ? 1 : 2;  // uniform
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s < steps) {
                    const int p = 4 * s + (lane >> 4);
                    const int q = 16 * rt + fr;
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(
                        sa + kAStage + q * kRowBytes + ((p ^ line_swizzle(q)) << 4));
#pragma unroll
                    for (int m = 0; m < MW; ++m) {
                        const int row = (m0 + m) * 16 + fr;
                        const u32x4 av = *reinterpret_cast<const u32x4 *>(
                            sa + row * kRowBytes + ((p ^ line_swizzle(row)) << 4));
                        if (tiles & (1u << m))
                            acc[m] = mfma_16x16x32(av, b, acc[m]);
                    }
                }
            }
        }

        // lane holds rows 4 (lane / 16) + i of each M tile, column lane % 16
        const int q = 16 * rt + fr;
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
    const int segs = a.L * a.E_l;
    if (segs <= 0 || a.r <= 0)
        return hipSuccess;
    // a multiple of 8 blocks: xcd_balanced_item needs every (XCD, index) pair
    const dim3 grid((segs + 7) / 8 * 8);
    if (mean_rows > 24)
        hipLaunchKernelGGL((lora_shrink_wide_kernel<4, 4>), grid, dim3(64 * kSWaves), 0, s, a);
    else
        hipLaunchKernelGGL((lora_shrink_wide_kernel<2, 6>), grid, dim3(64 * kSWaves), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
