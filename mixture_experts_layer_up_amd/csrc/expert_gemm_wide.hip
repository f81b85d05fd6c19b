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
//    128-column slab).  The waves split N, not K: wave w owns column tiles
//    2w and 2w+1 of the slab (for gate_up a matching gate/up pair), so every
//    wave needs the same activation rows.  Those are staged once per K chunk
//    into double-buffered LDS and read back as MFMA A fragments by all 4
//    waves; no cross-wave reduction is needed.
//  * Weight fragments are streamed per wave straight into a 4-deep register
//    ring (4 K chunks ahead), so each block keeps 32 KiB of weights in flight;
//    the activation chunks run the same 4 chunks ahead in registers and are
//    written to LDS right before their chunk is multiplied.
//  * LoRA expand chunks follow the main K chunks; an M tile (16 rows) skips
//    the MFMAs of a chunk whose adapters it does not contain (tokens of one
//    adapter are usually contiguous, so most tiles hold a single adapter).
//  * MFMA guards are scalar (wave-uniform) branches: MFMA ignores EXEC.
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kWMT = 10;              // M tiles of 16 rows per block (160 rows)
constexpr int kWRows = kWMT * 16;
constexpr int kRing = 4;              // weight chunks in flight per wave
constexpr int kARowBytes = 80;        // LDS row stride: 64 B of data + 16 B pad
constexpr int kASegs = kWRows * 4;    // 16-byte segments per staged chunk
constexpr int kASegsPerThread = (kASegs + 255) / 256;

template <bool kGated, bool kRank8>
__global__ __launch_bounds__(256, 2) void expert_gemm_wide_kernel(GemmArgs a)
{
    __shared__ __align__(16) unsigned char abuf[2][kWRows * kARowBytes];
    __shared__ int row_x[kWRows];
    __shared__ int row_src[kWRows];
    __shared__ int row_adapter[kWRows];
    __shared__ unsigned long long mt_adapters[kWMT];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();

    // work item -> (expert, 128-column slab, row tile); see expert_gemm.hip
    const int logical = xcd_contiguous_index(blockIdx.x, gridDim.x);
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

    // this wave's two column tiles: packed 64-column slab s64, tiles t0, t0 + 1
    const int s64 = slab * 2 + (wave >> 1);
    const int t0 = (wave & 1) * 2;
    const uint16_t *wbase =
        a.Wp + (((size_t)le * (a.n_slabs * 2) + s64) * (size_t)KC * 4 + t0) * 512 + lane * 8;
    // Branch-free loaders: the address is selected (always a valid one) and
    // the value masked, so every chunk issues the same loads.
    const uint16_t *lb = a.LB ? a.LB : a.Wp;
    auto load_b = [&](int vc, u32x4 (&b)[2]) {
        const bool main = vc < KC;  // uniform
        const int g = (vc - KC) * 32 + (lane >> 4) * 8;
        const int aid = main ? 0 : g / a.rp;
        const int q0 = main ? 0 : g - aid * a.rp;
        const int aid_c = max(min(aid, a.L - 1), 0);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint16_t *pm = wbase + ((size_t)min(vc, KC - 1) * 4 + n) * 512;
            const int nt16 = s64 * 4 + t0 + n;  // packed 16-column tile index
            const int col = kGated ? (nt16 & 1) * a.I + (nt16 >> 1) * 16 + (lane & 15)
                                   : nt16 * 16 + (lane & 15);
            const uint16_t *pe = lb + (((size_t)aid_c * a.E_l + le) * a.n_canon + col) * a.r;
            if (kRank8) {
                // past the last adapter (aid >= L) the clamped stack is read; its
                // K positions meet zero activations, so it adds nothing
                b[n] = load16_stream(main ? pm : pe + q0);
            } else {  // rank not a multiple of 8: the expand rows need 2-byte loads
                const u32x4 vm = load16_stream(pm);
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const uint32_t lo = pe[min(q0 + i, a.r - 1)];
                    const uint32_t hi = pe[min(q0 + i + 1, a.r - 1)];
                    w[i >> 1] = (q0 + i < a.r ? lo : 0u) | ((q0 + i + 1 < a.r ? hi : 0u) << 16);
                }
                const u32x4 ve = keep_if(u32x4{w[0], w[1], w[2], w[3]}, aid < a.L);
                b[n] = main ? vm : ve;
            }
        }
    };

    // weight ring first: it does not depend on the rows
    u32x4 ring[kRing][2];
#pragma unroll
    for (int d = 0; d < kRing; ++d)
        load_b(min(d, nv - 1), ring[d]);

    // rows of this tile: slot, source row, adapter
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

    // this thread's activation segments: (row, 16-byte quarter of the chunk)
    const uint16_t *seg_src[kASegsPerThread];
    int seg_x[kASegsPerThread], seg_ad[kASegsPerThread], seg_lds[kASegsPerThread];
#pragma unroll
    for (int i = 0; i < kASegsPerThread; ++i) {
        const int s = tid + 256 * i;
        const int r = min(s >> 2, kWRows - 1);
        const int q = s & 3;
        seg_src[i] = a.X + (size_t)row_src[r] * a.K + q * 8;
        seg_x[i] = row_x[r];
        seg_ad[i] = row_adapter[r];
        seg_lds[i] = s < kASegs ? r * kARowBytes + q * 16 : 0;
    }
    // activation chunks also run kRing chunks ahead, in registers, and are
    // written to LDS right before the chunk is multiplied
    u32x4 aring[kRing][kASegsPerThread];
    // Rows past the tile read a clamped valid row and are never stored, so
    // main chunks need no mask.  An expand chunk keeps a row's values only in
    // the K block of the row's own adapter; that mask is applied when the
    // chunk is written to LDS, not at the load (which would stall on it).
    const uint16_t *sbase = a.S ? a.S : a.X;
    bool amask[kRing][kASegsPerThread];
    auto load_a = [&](int vc, u32x4 (&areg)[kASegsPerThread], bool (&am)[kASegsPerThread]) {
        const bool main = vc < KC;  // uniform
#pragma unroll
        for (int i = 0; i < kASegsPerThread; ++i) {
            const int g = (vc - KC) * 32 + ((tid + 256 * i) & 3) * 8;
            const int aid = main ? -1 : g / a.rp;
            const int q0 = main ? 0 : g - aid * a.rp;
            const uint16_t *pa = main ? seg_src[i] + vc * 32 : sbase + (size_t)seg_x[i] * a.rp + q0;
            areg[i] = load16(pa);
            am[i] = main || seg_ad[i] == aid;
        }
    };
    auto store_a = [&](int buf, const u32x4 (&areg)[kASegsPerThread],
                       const bool (&am)[kASegsPerThread]) {
#pragma unroll
        for (int i = 0; i < kASegsPerThread; ++i)
            if (tid + 256 * i < kASegs)
                *reinterpret_cast<u32x4 *>(&abuf[buf][seg_lds[i]]) = keep_if(areg[i], am[i]);
    };

    f32x4 acc[kWMT][2];
#pragma unroll
    for (int m = 0; m < kWMT; ++m)
        acc[m][0] = acc[m][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int d = 0; d < kRing; ++d)
        load_a(min(d, nv - 1), aring[d], amask[d]);
    lds_barrier();  // mt_adapters
    unsigned long long mta[kWMT];  // per M tile, in scalar registers
#pragma unroll
    for (int m = 0; m < kWMT; ++m)
        mta[m] = uniform_u64(mt_adapters[m]);
    const int a_lane_off = (lane & 15) * kARowBytes + (lane >> 4) * 16;
    // Every ring load is unconditional (past the last chunk it re-reads the
    // last chunk), so the loads in flight are the same on every path and each
    // operand is waited for only when its own chunk comes up; only LDS work
    // and MFMAs sit behind (scalar) branches.
    for (int vc0 = 0; vc0 < nv; vc0 += kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            const int vc = vc0 + d;
            const bool live = vc < nv;  // uniform
            const int nxt = min(vc + kRing, nv - 1);
            if (live)
                store_a(vc & 1, aring[d], amask[d]);
            load_a(nxt, aring[d], amask[d]);
            lds_barrier();
            if (live) {
                // adapters covered by this chunk (ext chunks only)
                unsigned long long need = ~0ull;
                if (vc >= KC) {
                    const int lo = ((vc - KC) * 32) / a.rp;
                    const int hi = min(a.L - 1, ((vc - KC) * 32 + 31) / a.rp);
                    const int span = hi - lo + 1;
                    need = (span >= 64 ? ~0ull : ((1ull << span) - 1ull)) << lo;
                }
                const unsigned char *ab = abuf[vc & 1] + a_lane_off;
                u32x4 av[kWMT];
#pragma unroll
                for (int m = 0; m < kWMT; ++m)  // rows past the tile: read, never used
                    av[m] = *reinterpret_cast<const u32x4 *>(ab + m * 16 * kARowBytes);
#pragma unroll
                for (int m = 0; m < kWMT; ++m) {
                    if (m < n_mt && (vc < KC || (mta[m] & need) != 0)) {
                        acc[m][0] = mfma_16x16x32(av[m], ring[d][0], acc[m][0]);
                        acc[m][1] = mfma_16x16x32(av[m], ring[d][1], acc[m][1]);
                    }
                }
            }
            load_b(nxt, ring[d]);
        }
    }

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
                        const float v = silu_f32(acc[m][0][i]) * acc[m][1][i];
                        a.Y[p * a.I + j * 16 + c] = (uint16_t)float_to_bf16_bits(v);
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

bool gemm_wide_supported(int H, int I) { return I % 64 == 0 && H % 128 == 0; }

hipError_t launch_gemm_wide(const GemmArgs &a, bool gated, hipStream_t s)
{
    const int blocks = a.n_tiles * a.n_slabs;
    if (blocks <= 0)
        return hipSuccess;
    const bool r8 = (a.r & 7) == 0;
    if (gated && r8)
        hipLaunchKernelGGL((expert_gemm_wide_kernel<true, true>), dim3(blocks), dim3(256), 0, s, a);
    else if (gated)
        hipLaunchKernelGGL((expert_gemm_wide_kernel<true, false>), dim3(blocks), dim3(256), 0, s, a);
    else if (r8)
        hipLaunchKernelGGL((expert_gemm_wide_kernel<false, true>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((expert_gemm_wide_kernel<false, false>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
