// expert_gemm_wide.hip -- grouped expert GEMMs for experts with many rows.
//
// Same computation as expert_gemm.hip (gate_up with the LoRA expand as extra
// K and SwiGLU in the epilogue; down with the LoRA expand as extra K) for
// batches where every expert carries tens to hundreds of rows (prefill).
// Sources: "BF16 support for the experimental_sgl_trtllm MoE-LoRA path",
// "Files changed" table, launcher row, and Flow section 2.
//
// Design for gfx950 when rows per expert are many:
//  * One block = 4 waves = one (row tile of at most 160 rows of one expert,
//    128-column slab).  The waves split N: wave w owns column tiles 2w and
//    2w + 1 of the slab (for gate_up a matching gate/up pair), so all four
//    waves multiply the same activation rows and no cross-wave reduction is
//    needed.
//  * Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4):
//    no register staging and no LDS store instructions.  Four K chunks of 32
//    are resident (18 KiB each: 160 activation rows + the slab's 8 weight
//    fragments); three are in flight while the fourth is multiplied.  The
//    wait for a chunk is an explicit vmcnt on the issuing wave followed by a
//    block barrier, so weight and activation loads stream continuously.
//  * Activation rows are stored 64 bytes apart with the four 16-byte K
//    quarters of a row XOR-swizzled by bits 1..3 of the row, so the 16-row
//    MFMA fragment reads hit distinct LDS banks; a direct load writes 1 KiB
//    contiguously, which is bank-conflict free by construction.
//  * LoRA expand chunks follow the main K chunks.  A row's expand values are
//    kept only in the K block of its own adapter: other lanes load from a
//    zero block in the workspace instead (a direct load cannot mask).  An M
//    tile (16 rows) skips the MFMAs of a chunk whose adapters it does not
//    contain.  Needs rank % 8 == 0 (16-byte expand rows).
//  * MFMA guards are scalar (wave-uniform) branches: MFMA ignores EXEC.
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kWMT = 10;                       // M tiles of 16 rows per block
constexpr int kWRows = kWMT * 16;              // 160 rows
constexpr int kStages = 4;                     // K chunks resident in LDS
constexpr int kAStageBytes = kWRows * 64;      // 160 rows x 32 bf16
constexpr int kBStageBytes = 8 * 1024;         // 8 MFMA B fragments
constexpr int kStageBytes = kAStageBytes + kBStageBytes;
constexpr int kAInstr = kWRows / 16;           // 1 KiB direct loads per A stage

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte direct load into LDS: lane l's 16 bytes land at LDS byte address
// lds_addr + 16 l (lds_addr wave-uniform).  Written as inline assembly on
// purpose: the compiler then leaves the completion of these loads entirely
// to the explicit waits below (its own tracking would otherwise wait for
// every outstanding load before each LDS read and serialise the pipeline).
// Loads it does not know about can only make its own wait counts stricter.
__device__ __forceinline__ void load_lds16(const void *g, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// The same for data read once (expert weights): the nontemporal hint keeps
// the weight stream from evicting the activation rows that the other column
// slabs of the expert are about to read from L2.
__device__ __forceinline__ void load_lds16_stream(const void *g, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// Physical 16-byte quarter of logical quarter q of activation row `row`.
__device__ __forceinline__ int a_swizzle(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Wait until at most N of this wave's vector loads are outstanding and its
// LDS reads are done, then synchronise the block.  The direct loads write
// LDS behind the compiler's back, so this wait is spelled out; the empty asm
// statements keep LDS reads from moving across the barrier.
template <int N>
__device__ __forceinline__ void dma_wait_barrier()
{
    static_assert(N < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma_drain()
{
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    asm volatile("" ::: "memory");
}

template <bool kGated>
__global__ __launch_bounds__(256, 2) void expert_gemm_wide_kernel(GemmArgs a)
{
    __shared__ __align__(1024) unsigned char smem[kStages * kStageBytes];
    auto stage = [&](int st) -> unsigned char * { return smem + st * kStageBytes; };
    // LDS byte address of smem, for the direct loads (M0)
    const uint32_t smem_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_void *)smem));
    auto stage_lds = [&](int st) { return smem_lds + (uint32_t)(st * kStageBytes); };
    __shared__ int row_x[kWRows];
    __shared__ int row_src[kWRows];
    __shared__ int row_adapter[kWRows];
    __shared__ unsigned long long mt_adapters[kWMT];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();

    // work item -> (expert, 128-column slab, row tile); see expert_gemm.hip
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
    const int n_rows = min(a.tile_rows, te.z - sub * a.tile_rows);
    const int n_mt = (n_rows + 15) >> 4;

    const int KC = a.K >> 5;
    const bool lora = a.S != nullptr && a.L > 0 && a.r > 0;
    const int n_ext = lora ? (a.L * a.rp + 31) >> 5 : 0;
    const int nv = KC + n_ext;
    // chunks of this launch: main K only (phase 1), expand only (phase 2), or all
    const int vbeg = a.phase == 2 ? KC : 0;
    const int vend = a.phase == 1 ? KC : nv;

    // rows of this tile: slot, source row, adapter (rows past the tile
    // repeat the last row and carry no adapter)
    for (int r = tid; r < kWRows; r += 256) {
        const int p = row0 + min(r, n_rows - 1);
        const int x = a.perm2exp[p];
        const int tok = x / a.k;
        row_x[r] = x;
        row_src[r] = a.gather_by_token ? tok : p;
        const int l = (lora && a.mapping) ? a.mapping[tok] : -1;
        row_adapter[r] = (r < n_rows && l >= 0 && l < a.L) ? l : -1;
    }
    lds_barrier();
    if (tid < kWMT) {
        unsigned long long m = 0;
        for (int r = tid * 16; r < tid * 16 + 16; ++r)
            if (row_adapter[r] >= 0)
                m |= 1ull << row_adapter[r];
        mt_adapters[tid] = m;
    }

    // Activation loads of this wave: A instructions j = wave + 4 i (waves 0
    // and 1 issue three, waves 2 and 3 two).  Lane `lane` of instruction j
    // fills physical row 16 j + lane / 4, physical quarter lane % 4, which
    // holds logical quarter (lane % 4) ^ swizzle(row).
    constexpr int kAPerWave = (kAInstr + 3) / 4;  // 3
    const int n_ai = (kAInstr - wave + 3) / 4;    // 3, 3, 2, 2 (uniform)
    const uint16_t *a_src[kAPerWave];
    int a_x[kAPerWave], a_ad[kAPerWave], a_q[kAPerWave];
#pragma unroll
    for (int i = 0; i < kAPerWave; ++i) {
        const int j = min(wave + 4 * i, kAInstr - 1);
        const int pr = 16 * j + (lane >> 2);
        const int q = (lane & 3) ^ a_swizzle(pr);
        a_src[i] = a.X + (size_t)row_src[pr] * a.K + q * 8;
        a_x[i] = row_x[pr];
        a_ad[i] = row_adapter[pr];
        a_q[i] = q;
    }
    // Weight loads of this wave: its own two fragments t0, t0 + 1 of packed
    // 64-column slab s64 (instructions 2 wave, 2 wave + 1 of the B stage).
    const int s64 = slab * 2 + (wave >> 1);
    const int t0 = (wave & 1) * 2;
    const uint16_t *b_main =
        a.Wp + (((size_t)le * (a.n_slabs * 2) + s64) * (size_t)KC * 4 + t0) * 512 + lane * 8;
    int b_col[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int nt16 = s64 * 4 + t0 + n;
        b_col[n] = kGated ? (nt16 & 1) * a.I + (nt16 >> 1) * 16 + (lane & 15)
                          : nt16 * 16 + (lane & 15);
    }
    const uint16_t *zeros = a.zeros;

    // issue the direct loads of chunk vc into LDS stage st
    auto issue_main = [&](int vc, int st) {
        const uint32_t sa = stage_lds(st);
        const uint32_t sb = sa + kAStageBytes;
#pragma unroll
        for (int i = 0; i < kAPerWave; ++i)
            if (i < n_ai)
                load_lds16(a_src[i] + vc * 32, sa + (wave + 4 * i) * 1024);
#pragma unroll
        for (int n = 0; n < 2; ++n)
            load_lds16_stream(b_main + ((size_t)vc * 4 + n) * 512, sb + (2 * wave + n) * 1024);
    };
    auto issue = [&](int vc, int st) {
        if (vc < KC) {
            issue_main(vc, st);
            return;
        }
        const uint32_t sa = stage_lds(st);
        const uint32_t sb = sa + kAStageBytes;
        const int c = vc - KC;
#pragma unroll
        for (int i = 0; i < kAPerWave; ++i) {
            if (i < n_ai) {
                const int g = c * 32 + a_q[i] * 8;
                const int aid = g / a.rp;
                const uint16_t *p =
                    a_ad[i] == aid ? a.S + (size_t)a_x[i] * a.rp + (g - aid * a.rp) : zeros;
                load_lds16(p, sa + (wave + 4 * i) * 1024);
            }
        }
        const int g = c * 32 + (lane >> 4) * 8;
        const int aid = g / a.rp;
        const int q0 = g - aid * a.rp;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint16_t *p =
                aid < a.L ? a.LB + (((a.lb_shared ? (size_t)aid : (size_t)aid * a.E_l + le) *
                                         a.n_canon + b_col[n]) * a.r + q0)
                          : zeros;
            load_lds16(p, sb + (2 * wave + n) * 1024);
        }
    };

    f32x4 acc[kWMT][2];
#pragma unroll
    for (int m = 0; m < kWMT; ++m)
        acc[m][0] = acc[m][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    lds_barrier();  // mt_adapters
    const int a_lane_off = (lane & 15) * 64 + (((lane >> 4) ^ a_swizzle(lane & 15)) * 16);
    // M tiles that exist, as a scalar bit mask
    const uint32_t main_tiles = __builtin_amdgcn_readfirstlane((1u << n_mt) - 1u);

    // multiply the chunk in stage st for the M tiles in `tiles`
    auto compute = [&](int st, uint32_t tiles) {
        const unsigned char *sa = stage(st);
        const unsigned char *sb = sa + kAStageBytes + 2 * wave * 1024 + lane * 16;
        const u32x4 b0 = *reinterpret_cast<const u32x4 *>(sb);
        const u32x4 b1 = *reinterpret_cast<const u32x4 *>(sb + 1024);
        // two halves of five M tiles: fragment reads, then their MFMAs (the
        // scheduling barriers keep only one half's fragments live)
#pragma unroll
        for (int h = 0; h < kWMT; h += kWMT / 2) {
            u32x4 av[kWMT / 2];
#pragma unroll
            for (int m = 0; m < kWMT / 2; ++m)  // rows past the tile: read, never used
                av[m] = *reinterpret_cast<const u32x4 *>(sa + (h + m) * 1024 + a_lane_off);
#pragma unroll
            for (int m = 0; m < kWMT / 2; ++m) {
                if (tiles & (1u << (h + m))) {
                    acc[h + m][0] = mfma_16x16x32(av[m], b0, acc[h + m][0]);
                    acc[h + m][1] = mfma_16x16x32(av[m], b1, acc[h + m][1]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // M tiles holding a row of an adapter whose K block meets expand chunk vc
    auto ext_tiles = [&](int vc) {
        const int lo = ((vc - KC) * 32) / a.rp;
        const int hi = min(a.L - 1, ((vc - KC) * 32 + 31) / a.rp);
        const int span = hi - lo + 1;
        const unsigned long long need = span >= 64 ? ~0ull : ((1ull << span) - 1ull) << lo;
        uint32_t t = 0;
#pragma unroll
        for (int m = 0; m < kWMT; ++m)
            t |= (mt_adapters[m] & need) != 0 ? 1u << m : 0u;
        return __builtin_amdgcn_readfirstlane(t & main_tiles);
    };
    // Per chunk a wave issues n_ai + 2 loads; chunk vc is complete once only
    // the loads of the two chunks issued after it can be outstanding.
    auto wait_chunk = [&]() {
        if (n_ai == 3)
            dma_wait_barrier<2 * (3 + 2)>();
        else
            dma_wait_barrier<2 * (2 + 2)>();
    };

    // The stage of chunk vc is vc % kStages.  Chunk vc + 3 is issued right
    // after the barrier of chunk vc, into the stage chunk vc - 1 has left
    // (every wave's reads of it are complete).  Past the last chunk the last
    // one is issued again, so the loads per chunk never change.  Groups of
    // four chunks whose loads are all main chunks take a lean path.
    static_assert(kStages == 4, "the issue distance below is kStages - 1");
    issue(vbeg, 0);
    issue(min(vbeg + 1, vend - 1), 1);
    issue(min(vbeg + 2, vend - 1), 2);
    for (int vc0 = vbeg; vc0 < vend; vc0 += kStages) {
        if (vc0 + kStages + 2 < KC) {
#pragma unroll
            for (int d = 0; d < kStages; ++d) {
                wait_chunk();
                issue_main(vc0 + d + 3, (d + 3) % kStages);
                compute(d, main_tiles);
            }
        } else {
#pragma unroll
            for (int d = 0; d < kStages; ++d) {
                const int vc = vc0 + d;
                wait_chunk();
                issue(min(vc + 3, vend - 1), (d + 3) % kStages);
                if (vc < vend)
                    compute(d, vc < KC ? main_tiles : ext_tiles(vc));
            }
        }
    }
    dma_drain();  // no direct load may land after the block's LDS is released

    // epilogue straight from the accumulators: lane holds rows 4 (lane / 16) + i
    // of each M tile, column lane % 16 of its two tiles
    const int c = lane & 15;
#pragma unroll
    for (int m = 0; m < kWMT; ++m) {
        if (m < n_mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m * 16 + 4 * (lane >> 4) + i;
                if (r < n_rows) {
                    const size_t p = (size_t)(row0 + r);
                    if (kGated) {
                        const int j = slab * 4 + wave;  // gate/up pair of this wave
                        const size_t h_at = p * 2 * a.I + j * 16 + c;
                        float gate = acc[m][0][i], up = acc[m][1][i];
                        if (a.phase == 1) {  // fp32 pre-activation for phase 2
                            a.H[h_at] = gate;
                            a.H[h_at + a.I] = up;
                        } else {
                            if (a.phase == 2) {
                                gate += a.H[h_at];
                                up += a.H[h_at + a.I];
                            }
                            a.Y[p * a.I + j * 16 + c] =
                                (uint16_t)float_to_bf16_bits(silu_f32(gate) * up);
                        }
                    } else {
                        const int col = slab * 128 + wave * 32 + c;
                        a.Y[p * a.n_canon + col] = (uint16_t)float_to_bf16_bits(acc[m][0][i]);
                        a.Y[p * a.n_canon + col + 16] = (uint16_t)float_to_bf16_bits(acc[m][1][i]);
                    }
                }
            }
        }
    }
}

} // namespace

bool gemm_wide_supported(int H, int I, int r_gu, int r_dn)
{
    return I % 64 == 0 && H % 128 == 0 && r_gu % 8 == 0 && r_dn % 8 == 0;
}

hipError_t launch_gemm_wide(const GemmArgs &a, bool gated, hipStream_t s)
{
    const int blocks = gemm_grid_blocks(a.n_tiles, a.n_slabs);
    if (blocks <= 0)
        return hipSuccess;
    if (gated)
        hipLaunchKernelGGL((expert_gemm_wide_kernel<true>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((expert_gemm_wide_kernel<false>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
