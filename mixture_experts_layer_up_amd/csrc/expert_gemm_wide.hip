// expert_gemm_wide.hip -- grouped expert GEMMs for experts with many rows.
//
// Same computation as expert_gemm.hip (gate_up with the LoRA expand as extra
// K and SwiGLU in the epilogue; down with the LoRA expand as extra K) for
// batches where every expert carries tens to hundreds of rows (prefill).
// Sources: "BF16 support for the experimental_sgl_trtllm MoE-LoRA path",
// "Files changed" table, launcher row, and Flow section 2.
//
// Design for gfx950 when rows per expert are many:
//  * One block = 8 waves = one (row tile of at most 176 rows of one expert,
//    256-column slab at a time), one block per CU.  Waves 0-3 are consumers: consumer
//    w owns the slab's 64-column group w (for gate_up two gate/up pairs) for
//    all 176 rows, and only reads LDS and issues MFMAs.  Waves 4-7 are
//    producers: they only compute addresses and issue the direct
//    global->LDS loads (global_load_lds_dwordx4), which occupy the issuing
//    wave for a long time each; on separate waves that time no longer delays
//    any MFMA.
//  * K advances in chunks of 32.  Two LDS rings: the slab's 16 weight
//    fragments of a chunk (16 KiB; 5 stages), and the activation rows of a
//    chunk pair (176 rows x 128 bytes = 22 KiB; 3 stages), so each row
//    arrives as whole 128-byte lines, 8 rows per direct load: the per-CU
//    request path, not HBM, bounded the loads of half lines (16 rows x 64
//    bytes per load).  The producers keep 4 chunks in flight.  One block
//    barrier per chunk both publishes a landed chunk (each producer waits
//    for its own loads with an explicit vmcnt first) and frees the stages
//    the consumers finished.
//  * The eight 16-byte K pieces of an activation row are XOR-swizzled by
//    bits 1..3 of the row, so the 16-row MFMA fragment reads hit distinct
//    LDS banks; a direct load writes 1 KiB contiguously, which is
//    bank-conflict free by construction.  Rows of M tiles past the tile are
//    not loaded at all.
//  * LoRA expand chunks follow the main K chunks.  A row's expand values are
//    kept only in the K block of its own adapter: other lanes load from a
//    zero block in the workspace instead (a direct load cannot mask).  An M
//    tile (16 rows) skips the MFMAs of a chunk whose adapters it does not
//    contain.  Needs rank % 8 == 0 (16-byte expand rows).
//  * A block runs several adjacent slabs of its row tile in turn (slab
//    groups, sized by the launcher so that the items fill the CUs about
//    once).  The rows, and so the loads per chunk, are the same for every
//    slab, so the producers run on into the next slab's chunks while the
//    consumers write the previous slab's outputs.
//  * Outputs (act, y: tens of MB) leave through a small per-consumer LDS
//    tile as 16-byte streaming stores.
//  * MFMA guards are scalar (wave-uniform) branches: MFMA ignores EXEC.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe_lora {
namespace {

constexpr int kWMT = kWideMaxTileRows / 16;    // M tiles of 16 rows per block: 11
constexpr int kWRows = kWMT * 16;              // 176 rows
constexpr int kCons = 4;                       // consumer waves
constexpr int kNTW = 4;                        // 16-column tiles per consumer
constexpr int kSlabCols = kCons * kNTW * 16;   // 256 columns per block
constexpr int kThreadsW = 2 * kCons * kWave;   // consumers + producers
constexpr int kWStages = 5;                    // weight chunks (32 K each) resident in LDS
constexpr int kXStages = 3;                    // activation chunk pairs (64 K each) resident
constexpr int kXRowBytes = 128;                // a row's share of a chunk pair: one cache line
constexpr int kXStageBytes = kWRows * kXRowBytes;  // 176 rows x 64 bf16
constexpr int kWStageBytes = kCons * kNTW * 1024;  // 16 MFMA B fragments
constexpr int kAPerProd = (kWMT + kCons - 1) / kCons;  // M tiles per producer: 3
constexpr int kWideCUs = 256;                  // MI355X compute units (one block each)

// physical 16-byte slot of logical piece p (0..7) of activation row `row`
// in a chunk-pair stage: p ^ xline_swizzle(row)
__device__ __forceinline__ int xline_swizzle(int row) { return (row >> 1) & 7; }

template <bool kGated>
__global__ __launch_bounds__(kThreadsW, 1) void expert_gemm_wide_kernel(GemmArgs a)
{
    __shared__ __align__(1024) unsigned char xsm[kXStages * kXStageBytes];
    __shared__ __align__(1024) unsigned char wsm[kWStages * kWStageBytes];
    // LDS byte addresses of the two rings, for the direct loads (M0)
    const uint32_t xsm_lds = lds_address(xsm);
    const uint32_t wsm_lds = lds_address(wsm);
    __shared__ int row_x[kWRows];
    __shared__ int row_src[kWRows];
    __shared__ int row_adapter[kWRows];
    __shared__ unsigned long long mt_adapters[kWMT];
    // each consumer's output staging tile: 16 rows x up to 64 bf16 columns
    __shared__ __align__(16) uint16_t otile[kCons][16 * kNTW * 16];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();

    // work item -> (expert, group of slabs_per_block 256-column slabs, row
    // tile); items are numbered as in expert_gemm.hip with slab groups in
    // place of slabs
    const int n_groups = (a.n_slabs + a.slabs_per_block - 1) / a.slabs_per_block;
    const int logical = xcd_balanced_item(blockIdx.x, *a.tile_count * n_groups);
    if (logical < 0)
        return;
    const int4 te = a.tiles[logical / n_groups];
    const int le = te.x;
    if (le < 0)
        return;
    const int nt = (te.z + a.tile_rows - 1) / a.tile_rows;
    const int in_expert = logical - te.w * n_groups;
    const int group = in_expert / nt;
    const int sub = in_expert - group * nt;
    // this block's slabs: slab0 .. slab0 + n_sl - 1, one after another
    const int slab0 = group * a.slabs_per_block;
    const int n_sl = min(a.slabs_per_block, a.n_slabs - slab0);
    const int row0 = te.y + sub * a.tile_rows;
    const int n_rows = min(a.tile_rows, te.z - sub * a.tile_rows);
    const int n_mt = (n_rows + 15) >> 4;

    const int KC = a.K >> 5;
    const bool lora = a.S != nullptr && a.L > 0 && a.r > 0;
    const int n_ext = lora ? (a.L * a.rp + 31) >> 5 : 0;
    const int nv = KC + n_ext;  // main K chunks, then the LoRA expand chunks
    // Chunks go in pairs (the activation rows of a pair are one 128-byte line
    // per row), so a slab's sequence is padded to an even length nv2 (KC is
    // even; a padding chunk reads zeros and multiplies nothing).  The block's
    // chunk sequence q = 0 .. nq - 1 runs the slabs in turn: slab slab0 +
    // q / nv2, chunk q % nv2.  Chunks of equal parity carry the same loads
    // (the rows are the same for all slabs), so the producers' wait counts
    // do not change across slabs, and they run on into the next slab while
    // the consumers finish the previous one.
    const int nv2 = (nv + 1) & ~1;
    const int nq = n_sl * nv2;

    // rows of this tile: slot, source row, adapter (rows past the tile
    // repeat the last row and carry no adapter)
    for (int r = tid; r < kWRows; r += kThreadsW) {
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
    lds_barrier();  // mt_adapters

    // The 64-column group g (0..3) of slab `slab`: packed 64-column weight
    // slab s64(slab), present when it lies inside the N columns.
    const int NS64 = a.NT >> 2;
    const int g = wave & (kCons - 1);

    if (wave >= kCons) {
        // ------------------------------------------------------------ producer
        // Activation loads, once per chunk pair: M tiles j = g + 4 i that
        // exist, two loads each (rows 16 j .. 16 j + 7, then + 8 .. + 15).
        // Lane `lane` of a load fills row 16 j + 8 u + lane / 8, physical
        // slot lane % 8, which holds logical piece (lane % 8) ^ swizzle(row):
        // eight K values of the pair (pieces 0-3: the even chunk, 4-7: the
        // odd one).
        const int n_a = max(0, min(kAPerProd, (n_mt - g + kCons - 1) / kCons));
        const uint16_t *a_src[kAPerProd][2];
        int a_x[kAPerProd][2], a_ad[kAPerProd][2], a_p[kAPerProd][2];
#pragma unroll
        for (int i = 0; i < kAPerProd; ++i) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int j = min(g + kCons * i, kWMT - 1);
                const int pr = 16 * j + 8 * u + (lane >> 3);
                const int p = (lane & 7) ^ xline_swizzle(pr);
                a_src[i][u] = a.X + (size_t)row_src[pr] * a.K + p * 8;
                a_x[i][u] = row_x[pr];
                a_ad[i][u] = row_adapter[pr];
                a_p[i][u] = p;
            }
        }
        // B loads: the four fragments of weight slab s64 (contiguous 4 KiB
        // per chunk), or the LoRA B columns of its four 16-column tiles
        const uint16_t *zeros = a.zeros;
        const size_t slab_elems = (size_t)KC * 4 * 512;  // one packed 64-column slab

        // the activation rows of the chunk pair (vc, vc + 1), vc even, into
        // pair stage xst; main K pairs read hidden / act rows, expand pairs
        // keep each row's own adapter block (others, and padding past the
        // last adapter, read the zero block)
        auto issue_x = [&](auto na, int vc, int xst) __attribute__((always_inline)) {
            constexpr int NA = decltype(na)::value;
            const uint32_t sx = xsm_lds + (uint32_t)(xst * kXStageBytes);
#pragma unroll
            for (int i = 0; i < NA; ++i) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint32_t dst = sx + (g + kCons * i) * 2048 + u * 1024;
                    if (vc < KC) {
                        load_lds16(a_src[i][u] + vc * 32, dst);
                    } else {
                        const int gq = (vc - KC) * 32 + a_p[i][u] * 8;
                        const int aid = gq / a.rp;
                        const uint16_t *p = a_ad[i][u] == aid
                                                ? a.S + (size_t)a_x[i][u] * a.rp + (gq - aid * a.rp)
                                                : zeros;
                        load_lds16(p, dst);
                    }
                }
            }
        };
        // the weight (or LoRA B) fragments of chunk vc of slab si into weight
        // stage wst
        auto issue_w = [&](int si, int vc, int wst) __attribute__((always_inline)) {
            const int s64 = (slab0 + si) * kCons + g;
            const bool has_cols = s64 < NS64;
            const uint32_t sb = wsm_lds + (uint32_t)(wst * kWStageBytes) + g * kNTW * 1024;
            if (vc < KC) {
#pragma unroll
                for (int t = 0; t < kNTW; ++t) {
                    if (has_cols)  // weights are read once: streaming hint
                        load_lds16_stream(a.Wp + ((size_t)le * NS64 + s64) * slab_elems + lane * 8 +
                                              ((size_t)vc * 4 + t) * 512,
                                          sb + t * 1024);
                    else
                        load_lds16(zeros, sb + t * 1024);
                }
                return;
            }
            const int gq = (vc - KC) * 32 + (lane >> 4) * 8;
            const int aid = gq / a.rp;
            const int q0 = gq - aid * a.rp;
#pragma unroll
            for (int t = 0; t < kNTW; ++t) {
                const int nt16 = s64 * 4 + t;
                const int col = kGated ? (nt16 & 1) * a.I + (nt16 >> 1) * 16 + (lane & 15)
                                       : nt16 * 16 + (lane & 15);
                const uint16_t *p =
                    (has_cols && aid < a.L)
                        ? a.LB + (((a.lb_shared ? (size_t)aid : (size_t)aid * a.E_l + le) *
                                       a.n_canon + col) * a.r + q0)
                        : zeros;
                load_lds16(p, sb + t * 1024);
            }
        };
        // Chunk q's weights live in weight stage q % kWStages, its pair's
        // activation rows in pair stage (q / 2) % kXStages; an even chunk
        // also issues its pair's activation rows.  Chunks 0 .. kWStages - 2
        // go out first; after the barrier of chunk q, chunk q + kWStages - 1
        // goes out into the stages chunk q - 1 (and, for an even chunk, the
        // pair before chunk q's) has left.  Past the last chunk the last pair
        // is issued again by parity, so the loads per chunk never change and
        // chunk q has landed once only the loads of the three chunks issued
        // after it can be outstanding: 3 kNTW + 2 NA of them after an even
        // chunk, 3 kNTW + 4 NA after an odd one.  (qn: the next chunk.)
        auto run = [&](auto na) __attribute__((always_inline)) {
            constexpr int NA = decltype(na)::value;
            constexpr int kAfterEven = 3 * kNTW + 2 * NA;
            constexpr int kAfterOdd = 3 * kNTW + 4 * NA;
            int qn = 0;
            auto issue_next = [&]() __attribute__((always_inline)) {
                const bool past = qn >= nq;
                const int si = past ? n_sl - 1 : qn / nv2;
                const int vc = past ? nv2 - 2 + (qn & 1) : qn - (qn / nv2) * nv2;
                if ((qn & 1) == 0)
                    issue_x(na, vc, (qn >> 1) % kXStages);
                issue_w(si, vc, qn % kWStages);
                ++qn;
            };
            for (int d = 0; d < kWStages - 1; ++d)
                issue_next();
            for (int q = 0; q < nq; ++q) {
                if (q & 1)
                    dma_wait_barrier<kAfterOdd>();
                else
                    dma_wait_barrier<kAfterEven>();
                issue_next();
            }
            dma_drain();  // no direct load may land after the block's LDS is released
        };
        switch (n_a) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        default: run(std::integral_constant<int, 3>{}); break;
        }
        return;
    }

    // -------------------------------------------------------------- consumer
    // M tiles holding a row of an adapter whose K block meets expand chunk vc
    auto ext_tiles = [&](int vc, uint32_t main_tiles) __attribute__((always_inline)) {
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

    int q = 0;  // the block's chunk counter, as in the producers
    for (int si = 0; si < n_sl; ++si) {
        // per-lane offsets are recomputed in every slab from an opaque copy
        // of the lane index: hoisted out of the loop they would stay live
        // beside the 176 accumulator registers and spill
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // fragment row ln % 16 of an M tile, K piece ln / 16 of the even
        // chunk (4 + ln / 16 of the odd one), at its swizzled slot
        const int a_off0 = (ln & 15) * kXRowBytes + ((((ln >> 4)) ^ xline_swizzle(ln & 15)) << 4);
        const int a_off1 = (ln & 15) * kXRowBytes + (((4 + (ln >> 4)) ^ xline_swizzle(ln & 15)) << 4);
        const int s64 = (slab0 + si) * kCons + g;
        const bool has_cols = s64 < NS64;
        f32x4 acc[kWMT][kNTW];
#pragma unroll
        for (int m = 0; m < kWMT; ++m)
#pragma unroll
            for (int t = 0; t < kNTW; ++t)
                acc[m][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // M tiles that exist (none for a column group past N), as a scalar mask
        const uint32_t main_tiles =
            __builtin_amdgcn_readfirstlane(has_cols ? (1u << n_mt) - 1u : 0u);

        // multiply chunk q for the M tiles in `tiles`; A fragments are read
        // two M tiles ahead of their MFMAs (a ring of three)
        auto compute = [&](int qq, uint32_t tiles) __attribute__((always_inline)) {
            const unsigned char *sa = xsm + ((qq >> 1) % kXStages) * kXStageBytes +
                                      ((qq & 1) ? a_off1 : a_off0);
            const unsigned char *sb =
                wsm + (qq % kWStages) * kWStageBytes + g * kNTW * 1024 + ln * 16;
            u32x4 b[kNTW];
#pragma unroll
            for (int t = 0; t < kNTW; ++t)
                b[t] = *reinterpret_cast<const u32x4 *>(sb + t * 1024);
            u32x4 av[3];
            av[0] = *reinterpret_cast<const u32x4 *>(sa);
            av[1] = *reinterpret_cast<const u32x4 *>(sa + 2048);
#pragma unroll
            for (int m = 0; m < kWMT; ++m) {
                if (m + 2 < kWMT)  // rows past the tile: read, never used
                    av[(m + 2) % 3] = *reinterpret_cast<const u32x4 *>(sa + (m + 2) * 2048);
                if (tiles & (1u << m)) {
#pragma unroll
                    for (int t = 0; t < kNTW; ++t)
                        acc[m][t] = mfma_16x16x32(av[m % 3], b[t], acc[m][t]);
                }
            }
        };

        for (int vc = 0; vc < nv2; ++vc, ++q) {
            dma_wait_barrier<63>();  // the chunk has landed; this wave's reads of the previous one are done
            if (vc < nv)  // uniform: the padding chunk multiplies nothing
                compute(q, vc < KC ? main_tiles : ext_tiles(vc, main_tiles));
        }

        // Epilogue of this slab (the producers meanwhile fill the stages with
        // the next slab's first chunks).  Lane holds rows 4 (lane / 16) + i of
        // each M tile, column lane % 16 of its four tiles.  Each M tile's bf16
        // outputs (SwiGLU'd for gate_up) go through this consumer's private
        // LDS tile, 16 rows x kOut columns, and leave as 16-byte row segments.
        if (!has_cols)
            continue;
        const int c = ln & 15;
        constexpr int kOut = kGated ? kNTW / 2 * 16 : kNTW * 16;  // output columns: 32 or 64
        constexpr int kSeg = kOut / 8;                            // 16-byte segments per row
        uint16_t *ot = otile[g];
        // this consumer's output columns start at column `col0` of the output rows
        const int col0 = kGated ? 2 * s64 * 16 : s64 * 64;
        const int ld = kGated ? a.I : a.n_canon;
#pragma unroll
        for (int m = 0; m < kWMT; ++m) {
            if (m < n_mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 4 * (ln >> 4) + i;
                    if (kGated) {
#pragma unroll
                        for (int q = 0; q < kNTW / 2; ++q) {
                            const float gate = acc[m][2 * q][i], up = acc[m][2 * q + 1][i];
                            ot[rr * kOut + q * 16 + c] =
                                (uint16_t)float_to_bf16_bits(silu_f32(gate) * up);
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < kNTW; ++t)
                            ot[rr * kOut + t * 16 + c] = (uint16_t)float_to_bf16_bits(acc[m][t][i]);
                    }
                }
                // one wave: its LDS operations complete in order, so the reads
                // below see every lane's writes above
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int h = 0; h < 16 * kSeg / kWave; ++h) {
                    const int e = h * kWave + ln;  // 16-byte segment: row e / kSeg
                    const int rr = e / kSeg, sg = e % kSeg;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(ot + rr * kOut + sg * 8);
                    if (m * 16 + rr < n_rows)  // tens of MB per launch: streaming store
                        store16_stream(a.Y + (size_t)(row0 + m * 16 + rr) * ld + col0 + sg * 8, v);
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
}

} // namespace

bool gemm_wide_supported(int H, int I, int r_gu, int r_dn)
{
    return I % 64 == 0 && H % 128 == 0 && r_gu % 8 == 0 && r_dn % 8 == 0;
}

int gemm_wide_slabs(int NT) { return (NT * 16 + kSlabCols - 1) / kSlabCols; }

int gemm_wide_slabs_per_block(int n_slabs, int n_tiles, int E_l)
{
    // One block per CU.  When the work list holds about one tile per expert
    // (the usual case, see gemm_tile_rows), a block takes enough adjacent
    // slabs of its tile that the items fill the CUs about once: then no
    // block waits for a second round, and a block's producers stream its
    // next slab while its consumers still write the previous one.
    const int tiles = std::max(1, std::min(n_tiles, E_l));
    const int groups = std::max(1, std::min(n_slabs, (kWideCUs + tiles / 2) / tiles));
    return (n_slabs + groups - 1) / groups;
}

hipError_t launch_gemm_wide(const GemmArgs &a_in, bool gated, hipStream_t s)
{
    GemmArgs a = a_in;
    a.slabs_per_block = gemm_wide_slabs_per_block(a.n_slabs, a.n_tiles, a.E_l);
    const int n_groups = (a.n_slabs + a.slabs_per_block - 1) / a.slabs_per_block;
    const int blocks = gemm_grid_blocks(a.n_tiles, n_groups);
    if (blocks <= 0)
        return hipSuccess;
    if (gated)
        hipLaunchKernelGGL((expert_gemm_wide_kernel<true>), dim3(blocks), dim3(kThreadsW), 0, s, a);
    else
        hipLaunchKernelGGL((expert_gemm_wide_kernel<false>), dim3(blocks), dim3(kThreadsW), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
