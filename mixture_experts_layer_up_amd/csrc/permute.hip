// permute.hip -- expert-contiguous permutation and (adapter, expert) segments.
//
// The pages' launcher permutes (gathers) tokens per expert right after
// routing, and marks expert-parallel slots that the shard does not own with
// permuted index -1 ("BF16 support for the experimental_sgl_trtllm
// MoE-LoRA path", "Files changed" table, launcher row; "sglang PR #28953
// digest", change summary).  LoRA weights are addressed per virtual expert,
// i.e. per (adapter, expert) pair (same BF16 page, Flow section 2).
//
// Reading taken here: inside one expert (and one virtual expert) slots keep
// ascending slot order x = t * k + j, so the permutation is a stable counting
// sort.  It is built without order-dependent atomics: LDS integer atomics
// only produce counts (the same in any order), and ranks come from prefix
// offsets plus a wave-local match mask built from ballots.
//
// Two key types run side by side: blockIdx.y = 0 sorts slots by local expert,
// blockIdx.y = 1 by virtual expert (adapter * E_l + local expert).  The slots
// are cut into G = ceil(n / kPermuteSlotsPerBlock) consecutive blocks.  With G > 1 a
// count kernel first writes every block's histogram to the workspace; with
// more than 16 blocks a scan kernel then turns them into, per key, the slots
// in earlier blocks and the key's total (so the work stays linear in G);
// the rank kernel's blocks then each scan the totals into the
// offsets (every block the same, redundantly) and rank their own slots:
// position = offset of the key + slots of the key in earlier blocks + in
// earlier waves of the block + in earlier 64-slot groups of the wave + lower
// lanes of the group with the same key.  With G == 1 the rank kernel's own
// histogram is the whole one and the count kernel is skipped, and in the
// forward pass the rank pass shares its launch with the gate_up LoRA shrink
// (permute_shrink_kernel, below), which needs only the routing.
#include "device_common.h"
#include "kernels.h"
#include "lora_shrink_rows.h"
#include "moe_lora.h"

namespace moe_lora {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kIters = kPermuteSlotsPerBlock / kThreads;  // 64-slot groups per wave, at most
constexpr int kMaxKeys = 8192;                            // local experts, or adapters * local experts
constexpr int kMaxExperts = 1024;
constexpr int kFusedKeys = 1024;                          // keys of the permute fused with the shrink
constexpr int kScanMinBlocks = 17;  // slot blocks from which the histograms are scanned first

// key of a slot from its expert id and its token's adapter l (-1: none)
__device__ __forceinline__ int key_from(const PermuteArgs &a, bool by_segment, int id, int l)
{
    if (id < a.off || id >= a.off + a.E_l)
        return -1;  // not local: another expert-parallel shard owns it
    const int le = id - a.off;
    if (!by_segment)
        return le;
    if (l < 0 || l >= a.L)
        return -1;  // token without adapter
    return l * a.E_l + le;
}

// row stride of the per-block histograms in the workspace (int4 loads)
__device__ __forceinline__ int round4(int v) { return (v + 3) & ~3; }

struct BlockSlots {
    int beg, end;  // the block's slots
    int chunk;     // slots per wave: 64 * groups
    int groups;    // 64-slot groups per wave (uniform)
};

__device__ __forceinline__ BlockSlots block_slots(int n, int g)
{
    BlockSlots b;
    b.beg = g * kPermuteSlotsPerBlock;
    b.end = min(n, b.beg + kPermuteSlotsPerBlock);
    const int nb = max(0, b.end - b.beg);
    b.groups = (nb + kThreads - 1) / kThreads;
    b.chunk = b.groups * kWave;
    return b;
}

// The keys of this lane's slots: group i holds slot beg + wave * chunk +
// 64 i + lane (-1 past the block or the wave's chunk).  All loads are issued
// before any is used.
// key[i] of this lane's slots; bad: MOE_LORA_FLAG_* bits of the values read
// (expert blocks check the ids, segment blocks the adapters)
__device__ __forceinline__ void load_keys(const PermuteArgs &a, bool by_segment,
                                          const BlockSlots &b, int wave, int lane,
                                          int (&key)[kIters], int &bad)
{
    int id[kIters], l[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        id[i] = -1;
        l[i] = -1;
        if (i >= b.groups)  // uniform
            break;
        const int x = b.beg + wave * b.chunk + i * kWave + lane;
        if (x < b.end) {
            id[i] = a.topk_ids[x];
            if (by_segment && a.mapping)
                l[i] = a.mapping[x / a.k];
        }
    }
    bad = 0;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int x = b.beg + wave * b.chunk + i * kWave + lane;
        const bool slot = i < b.groups && x < b.end;
        key[i] = slot ? key_from(a, by_segment, id[i], l[i]) : -1;
        if (slot && !by_segment && (id[i] < -1 || id[i] >= a.E))
            bad |= MOE_LORA_FLAG_EXPERT_ID;
        if (slot && by_segment && (l[i] < -1 || l[i] >= a.L))
            bad |= MOE_LORA_FLAG_ADAPTER;
    }
}

// Inclusive scan of one value per thread over the block; also the block total.
// Uses wave_tot[kWaves]; all threads must call it.
__device__ __forceinline__ int block_scan(int v, int lane, int wave, int *wave_tot, int &total)
{
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off)
            incl += o;
    }
    if (lane == kWave - 1)
        wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int t = wave_tot[w];
        before += w < wave ? t : 0;
        total += t;
    }
    __syncthreads();  // wave_tot is reused by the next call
    return incl + before;
}

__global__ __launch_bounds__(kThreads) void permute_count_kernel(PermuteArgs a)
{
    __shared__ int hist[kMaxKeys];
    const bool by_segment = blockIdx.y == 1;
    const int NK = by_segment ? a.L * a.E_l : a.E_l;
    if (NK == 0)
        return;
    const int g = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int n = a.T * a.k;
    const BlockSlots b = block_slots(n, g);
    int key[kIters];
    int bad;
    load_keys(a, by_segment, b, wave, lane, key, bad);
    for (int j = threadIdx.x; j < NK; j += kThreads)
        hist[j] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kIters; ++i)
        if (key[i] >= 0)
            atomicAdd(&hist[key[i]], 1);
    __syncthreads();
    const int NKs = round4(NK);
    int32_t *dst = a.block_counts + (by_segment ? (size_t)a.G * round4(a.E_l) : 0) + (size_t)g * NKs;
    for (int j = threadIdx.x; j < NKs; j += kThreads)
        dst[j] = j < NK ? hist[j] : 0;
}

// With several slot blocks: per key, the exclusive prefix over the blocks of
// their histograms (in place: row g becomes the key's slots in blocks
// 0 .. g - 1) and the key's total (the totals row after both key types'
// rows).  One thread per key, blocks in order; every block's histogram is
// read once, so the work is linear in G * keys.
__global__ __launch_bounds__(kThreads) void permute_scan_kernel(PermuteArgs a)
{
    const bool by_segment = blockIdx.y == 1;
    const int NKs = round4(by_segment ? a.L * a.E_l : a.E_l);
    const int j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= NKs)
        return;
    int32_t *rows = a.block_counts + (by_segment ? (size_t)a.G * round4(a.E_l) : 0);
    int32_t *totals = a.block_counts + (size_t)a.G * (round4(a.E_l) + round4(a.L * a.E_l)) +
                      (by_segment ? round4(a.E_l) : 0);
    int run = 0;
    for (int g0 = 0; g0 < a.G; g0 += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)  // all loads of a batch in flight together
            c[u] = g0 + u < a.G ? rows[(size_t)(g0 + u) * NKs + j] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (g0 + u < a.G) {
                rows[(size_t)(g0 + u) * NKs + j] = run;
                run += c[u];
            }
        }
    }
    totals[j] = run;
}

// The rank pass of slot block g for one key type.  kKeys bounds the keys
// (E_l, or L * E_l) and kExperts the local experts: they size the LDS tables.
template <int kKeys, int kExperts>
__device__ __forceinline__ void permute_rank_body(const PermuteArgs &a, bool by_segment, int g)
{
    __shared__ int table[kWaves * kKeys];  // per-wave counts, then per-wave running positions
    __shared__ int exp_first[kExperts];    // expert offsets and counts, for the work list
    __shared__ int exp_rows[kExperts];
    __shared__ int wave_tot[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int G = a.G;
    const int n = a.T * a.k;
    const int NK = by_segment ? a.L * a.E_l : a.E_l;
    int32_t *out_offsets = by_segment ? a.seg_offsets : a.expert_offsets;
    int32_t *out_list = by_segment ? a.seg_slots : a.perm2exp;
    const BlockSlots b = block_slots(n, g);
    const bool lead = g == 0;  // writes the per-key arrays and the work list
    if (lead && !by_segment && a.zeros && tid < kZeroBytes / 16)
        a.zeros[tid] = u32x4_t{0u, 0u, 0u, 0u};

    if (NK == 0) {  // no adapters: empty segment list
        if (lead && tid == 0)
            out_offsets[0] = 0;
        for (int x = b.beg + tid; x < b.end; x += kThreads)
            out_list[x] = -1;
        return;
    }

    int key[kIters];
    int bad;
    load_keys(a, by_segment, b, wave, lane, key, bad);
    // report bad values: one vector atomic per wave that met any
    const unsigned long long bad_id = __ballot((bad & MOE_LORA_FLAG_EXPERT_ID) != 0);
    const unsigned long long bad_ad = __ballot((bad & MOE_LORA_FLAG_ADAPTER) != 0);
    if ((bad_id | bad_ad) && lane == 0 && a.flags)
        atomicOr(a.flags, (bad_id ? MOE_LORA_FLAG_EXPERT_ID : 0) | (bad_ad ? MOE_LORA_FLAG_ADAPTER : 0));

    // 1. per-wave histograms of the block's slots
    for (int j = tid; j < kWaves * NK; j += kThreads)
        table[j] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kIters; ++i)
        if (key[i] >= 0)
            atomicAdd(&table[wave * NK + key[i]], 1);
    __syncthreads();

    // 2. totals per key, their exclusive scan (the offsets), and each wave's
    // first position per key.  Keys in rows of 4 * kThreads, four consecutive
    // keys per thread.  With up to 16 slot blocks every block reads all the
    // blocks' histogram rows (int4 loads, all in flight together); with more,
    // the scan kernel has turned them into, per key, the slots in earlier
    // blocks (row g) and the key's total (the totals row): two int4 loads per
    // thread.
    const int NKs = round4(NK);
    const int32_t *counts = a.block_counts + (by_segment ? (size_t)G * round4(a.E_l) : 0);
    const int32_t *totals = a.block_counts + (size_t)G * (round4(a.E_l) + round4(a.L * a.E_l)) +
                            (by_segment ? round4(a.E_l) : 0);
    int carry = 0;
    for (int j0 = 0; j0 < NK; j0 += 4 * kThreads) {
        const int jb = j0 + 4 * tid;
        int before[4] = {0, 0, 0, 0}, all[4] = {0, 0, 0, 0};
        if (G > kScanMinBlocks - 1 && jb < NK) {
            const int4 b = *reinterpret_cast<const int4 *>(counts + (size_t)g * NKs + jb);
            const int4 t = *reinterpret_cast<const int4 *>(totals + jb);
            before[0] = b.x, before[1] = b.y, before[2] = b.z, before[3] = b.w;
            all[0] = t.x, all[1] = t.y, all[2] = t.z, all[3] = t.w;
        } else if (G > 1 && jb < NK) {
            // few blocks: read every block's histogram row directly, all in
            // flight together (rows past G are clamped and not counted)
            int4 c[kScanMinBlocks - 1];
#pragma unroll
            for (int u = 0; u < kScanMinBlocks - 1; ++u)
                c[u] = *reinterpret_cast<const int4 *>(counts + (size_t)min(u, G - 1) * NKs + jb);
#pragma unroll
            for (int u = 0; u < kScanMinBlocks - 1; ++u) {
                const bool lo = u < g, in = u < G;
                before[0] += lo ? c[u].x : 0;
                before[1] += lo ? c[u].y : 0;
                before[2] += lo ? c[u].z : 0;
                before[3] += lo ? c[u].w : 0;
                all[0] += in ? c[u].x : 0;
                all[1] += in ? c[u].y : 0;
                all[2] += in ? c[u].z : 0;
                all[3] += in ? c[u].w : 0;
            }
        }
        int wc[4][kWaves], total[4];
        int mine = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int j = jb + m;
            const bool valid = j < NK;
            int in_block = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                wc[m][w] = valid ? table[w * NK + j] : 0;
                in_block += wc[m][w];
            }
            total[m] = valid ? (G > 1 ? all[m] : in_block) : 0;
            mine += total[m];
        }
        int row_total;
        const int incl = block_scan(mine, lane, wave, wave_tot, row_total);
        int off = carry + incl - mine;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int j = jb + m;
            if (j < NK) {
                int run = off + before[m];
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    table[w * NK + j] = run;
                    run += wc[m][w];
                }
                if (lead) {
                    out_offsets[j] = off;
                    if (!by_segment) {
                        a.expert_counts[j] = total[m];
                        exp_first[j] = off;
                        exp_rows[j] = total[m];
                    }
                }
            }
            off += total[m];
        }
        carry += row_total;
    }
    const int grand = carry;  // slots with a key
    if (lead && tid == 0)
        out_offsets[NK] = grand;
    for (int x = max(grand, b.beg) + tid; x < b.end; x += kThreads)
        out_list[x] = -1;  // past the keyed slots

    // GEMM work list: chunks of at most tile_rows rows per expert, in expert
    // order; every chunk of expert e carries e's whole row range and the
    // index of e's first chunk
    if (lead && !by_segment && a.tiles) {
        __syncthreads();  // exp_first / exp_rows
        int tcarry = 0;
        for (int j0 = 0; j0 < NK; j0 += kThreads) {
            const int j = j0 + tid;
            const int rows = j < NK ? exp_rows[j] : 0;
            const int nt = (rows + a.tile_rows - 1) / a.tile_rows;
            int row_total;
            const int incl = block_scan(nt, lane, wave, wave_tot, row_total);
            const int t0 = tcarry + incl - nt;
            for (int r = 0; r < nt; ++r)
                a.tiles[t0 + r] = make_int4(j, exp_first[j], rows, t0);
            tcarry += row_total;
        }
        if (tid == 0 && a.tile_count)
            *a.tile_count = tcarry;
        for (int i = tcarry + tid; i < a.max_tiles; i += kThreads)
            a.tiles[i] = make_int4(-1, 0, 0, 0);
    }
    __syncthreads();  // table holds the running positions

    // 3. stable ranks, one 64-slot group at a time per wave
    volatile int *tab = table + wave * NK;
    const int nbits = NK > 1 ? 32 - __clz(NK - 1) : 0;
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        if (i >= b.groups)  // uniform
            break;
        const int x = b.beg + wave * b.chunk + i * kWave + lane;
        const int k = key[i];
        unsigned long long same = __ballot(k >= 0);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool v = (k >> bit) & 1;
            const unsigned long long bb = __ballot(v);
            same &= v ? bb : ~bb;
        }
        const int pos = k >= 0 ? tab[k] + __popcll(same & lt) : -1;
        const bool placed = k >= 0 && pos < n;  // always, for consistent inputs; guards the store
        if (x < b.end) {
            if (by_segment) {
                if (placed)
                    a.seg_slots[pos] = x;
            } else {
                a.exp2perm[x] = pos;
                if (placed)
                    a.perm2exp[pos] = x;
            }
        }
        // LDS operations of one wave complete in issue order, so every
        // lane's read above precedes this update by the group's last lane.
        if (k >= 0 && (same >> lane) == 1ull)
            tab[k] = tab[k] + __popcll(same);
    }
}

__global__ __launch_bounds__(kThreads) void permute_rank_kernel(PermuteArgs a)
{
    permute_rank_body<kMaxKeys, kMaxExperts>(a, blockIdx.y == 1, blockIdx.x);
}

// The gate_up LoRA shrink straight from the routing: it reads the expert ids
// and the adapter mapping, not the permute's output.  Block s owns virtual
// expert s = l * E_l + e (adapter l, local expert e); it finds its slots by
// scanning the ids itself (kSPT slots per thread, all loads issued before
// any is used), compacts them in ascending slot order in LDS, and runs the
// shrink body, which writes S by slot.  A slot belongs to the block when its
// id is expert e and its token's adapter is l, so out-of-range ids and
// adapters never match, as in the permute's keys.  Needs T * k <= 256 kSPT.
template <int NS, int CH, int MT, int kSPT>
__device__ __forceinline__ void shrink_by_ids_body(const PermuteArgs &pa, const ShrinkArgs &sa,
                                                   int seg)
{
    __shared__ float part[Part<MT>::kFloats];
    __shared__ int row_slot[16 * MT];
    __shared__ int list[kSPT * kThreads];
    __shared__ int wave_tot[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int l = seg / pa.E_l;
    const int want = pa.off + (seg - l * pa.E_l);  // global id of expert e
    const int n = pa.T * pa.k;
    int id[kSPT], ad[kSPT];
#pragma unroll
    for (int i = 0; i < kSPT; ++i) {
        const int x = kSPT * tid + i;
        id[i] = x < n ? pa.topk_ids[x] : -1;
        ad[i] = (x < n && pa.mapping) ? pa.mapping[x / pa.k] : -1;
    }
    int hit = 0;
#pragma unroll
    for (int i = 0; i < kSPT; ++i)
        hit |= (kSPT * tid + i < n && id[i] == want && ad[i] == l) ? 1 << i : 0;
    const int c = __popc(hit);
    int total;
    int pos = block_scan(c, lane, wave, wave_tot, total) - c;
#pragma unroll
    for (int i = 0; i < kSPT; ++i)
        if ((hit >> i) & 1)
            list[pos++] = kSPT * tid + i;  // ascending slot order
    if (total == 0)
        return;
    __syncthreads();  // list
    const int stack = sa.a_shared ? l : seg;
    shrink_rows<NS, CH, MT>(sa, stack, total, [&](int i) { return list[i]; }, part, row_slot);
}

// The permute and the gate_up shrink in one launch, for batches of one slot
// block: blocks 0 and 1 are the permute's two key types, block 2 + s runs
// the shrink of virtual expert s.  The shrink then runs beside the permute
// instead of after it, and one launch boundary goes.  Requires T * k <=
// kPermuteSlotsPerBlock and E_l, L * E_l <= kFusedKeys.
template <int NS, int CH, int MT>
__global__ __launch_bounds__(kThreads, 2) void permute_shrink_kernel(PermuteArgs pa, ShrinkArgs sa)
{
    if (blockIdx.x < 2) {
        permute_rank_body<kFusedKeys, kFusedKeys>(pa, blockIdx.x == 1, 0);
        return;
    }
    shrink_by_ids_body<NS, CH, MT, kPermuteSlotsPerBlock / kThreads>(pa, sa, blockIdx.x - 2);
}

// The same shrink on its own launch (the side stream of the two-stream
// schedule), one block per virtual expert.
template <int NS, int CH, int MT, int kSPT>
__global__ __launch_bounds__(kThreads, 2) void shrink_by_ids_kernel(PermuteArgs pa, ShrinkArgs sa)
{
    shrink_by_ids_body<NS, CH, MT, kSPT>(pa, sa, blockIdx.x);
}

} // namespace

bool permute_shrink_fusable(const PermuteArgs &pa, const ShrinkArgs &sa)
{
    return pa.G == 1 && pa.T * pa.k <= kPermuteSlotsPerBlock && pa.E_l <= kFusedKeys &&
           pa.L * pa.E_l <= kFusedKeys && sa.r > 0 && sa.L == pa.L && sa.E_l == pa.E_l &&
           !shrink_uses_wide(sa);
}

hipError_t launch_permute_shrink(const PermuteArgs &pa, const ShrinkArgs &sa, hipStream_t s)
{
    const dim3 grid(2 + pa.L * pa.E_l);
    with_shrink_shape(sa.r, shrink_row_tiles(sa), [&](auto ns, auto ch, auto mt) {
        hipLaunchKernelGGL((permute_shrink_kernel<decltype(ns)::value, decltype(ch)::value,
                                                  decltype(mt)::value>),
                           grid, dim3(kThreads), 0, s, pa, sa);
    });
    return hipGetLastError();
}

bool shrink_by_ids_supported(const PermuteArgs &pa, const ShrinkArgs &sa)
{
    return pa.T * pa.k <= kShrinkByIdsMaxSlots && sa.r > 0 && sa.L == pa.L &&
           sa.E_l == pa.E_l && !shrink_uses_wide(sa);
}

hipError_t launch_shrink_by_ids(const PermuteArgs &pa, const ShrinkArgs &sa, hipStream_t s)
{
    const int blocks = pa.L * pa.E_l;
    if (blocks <= 0)
        return hipSuccess;
    const bool small = pa.T * pa.k <= kPermuteSlotsPerBlock;
    with_shrink_shape(sa.r, shrink_row_tiles(sa), [&](auto ns, auto ch, auto mt) {
        constexpr int NS = decltype(ns)::value, CH = decltype(ch)::value, MT = decltype(mt)::value;
        if (small)
            hipLaunchKernelGGL((shrink_by_ids_kernel<NS, CH, MT, 4>), dim3(blocks),
                               dim3(kThreads), 0, s, pa, sa);
        else
            hipLaunchKernelGGL((shrink_by_ids_kernel<NS, CH, MT, kShrinkByIdsMaxSlots / kThreads>),
                               dim3(blocks), dim3(kThreads), 0, s, pa, sa);
    });
    return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s)
{
    const int G = a.G;
    if (G > 1)
        hipLaunchKernelGGL(permute_count_kernel, dim3(G, 2), dim3(kThreads), 0, s, a);
    if (G >= kScanMinBlocks) {
        const int keys = round4_host(a.E_l > a.L * a.E_l ? a.E_l : a.L * a.E_l);
        hipLaunchKernelGGL(permute_scan_kernel, dim3((keys + kThreads - 1) / kThreads, 2),
                           dim3(kThreads), 0, s, a);
    }
    hipLaunchKernelGGL(permute_rank_kernel, dim3(G, 2), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
