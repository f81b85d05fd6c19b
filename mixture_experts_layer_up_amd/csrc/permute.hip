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
// only produce counts (the same in any order), and ranks come from per-wave
// prefix offsets plus a wave-local match mask built from ballots.
//
// Launch: two blocks of 1024 threads.  Block 0 sorts slots by local expert,
// block 1 by virtual expert (adapter * E_l + local expert).
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxKeys = 8192;   // local experts, or adapters * local experts
constexpr int kTable = 8192;     // per-wave running offsets, waves * keys
constexpr int kKeyCache = 16384; // slot keys kept in LDS when n fits

__device__ __forceinline__ int slot_key(const PermuteArgs &a, bool by_segment, int x)
{
    const int id = a.topk_ids[x];
    if (id < a.off || id >= a.off + a.E_l)
        return -1;  // not local: another expert-parallel shard owns it
    const int le = id - a.off;
    if (!by_segment)
        return le;
    const int l = a.mapping ? a.mapping[x / a.k] : -1;
    if (l < 0 || l >= a.L)
        return -1;  // token without adapter
    return l * a.E_l + le;
}

__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteArgs a)
{
    __shared__ int hist[kMaxKeys + 1];
    __shared__ int table[kTable];
    __shared__ int wave_excl[kWaves];
    __shared__ int tile_excl[kWaves];
    __shared__ int tile_total;
    __shared__ int key_cache[kKeyCache];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const bool by_segment = blockIdx.x == 1;
    const int n = a.T * a.k;
    const int NK = by_segment ? a.L * a.E_l : a.E_l;
    int32_t *out_offsets = by_segment ? a.seg_offsets : a.expert_offsets;
    int32_t *out_list = by_segment ? a.seg_slots : a.perm2exp;
    if (!by_segment && a.zeros && tid < kZeroBytes / 16)
        a.zeros[tid] = u32x4_t{0u, 0u, 0u, 0u};

    if (NK == 0) {  // no adapters: empty segment list
        if (tid == 0)
            out_offsets[0] = 0;
        for (int i = tid; i < n; i += kThreads)
            out_list[i] = -1;
        return;
    }

    // 0. every slot's key, once: into LDS when the batch fits (independent
    // loads, so they are all in flight together), else recomputed per pass
    const bool cached = n <= kKeyCache;
    if (cached) {
        for (int x = tid; x < n; x += kThreads)
            key_cache[x] = slot_key(a, by_segment, x);
    }
    auto key_of = [&](int x) { return cached ? key_cache[x] : slot_key(a, by_segment, x); };

    // 1. histogram
    for (int i = tid; i <= NK; i += kThreads)
        hist[i] = 0;
    __syncthreads();
    for (int x = tid; x < n; x += kThreads) {
        const int key = key_of(x);
        if (key >= 0)
            atomicAdd(&hist[key], 1);
    }
    __syncthreads();

    // 2. exclusive scan: each thread owns a contiguous run of keys
    const int per = (NK + kThreads - 1) / kThreads;
    const int beg = min(NK, tid * per);
    const int end = min(NK, beg + per);
    int local = 0;
    for (int i = beg; i < end; ++i) {
        const int c = hist[i];
        if (!by_segment)
            a.expert_counts[i] = c;
        local += c;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off)
            incl += o;
    }
    if (lane == kWave - 1)
        wave_excl[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int ws = lane < kWaves ? wave_excl[lane] : 0;
        int wi = ws;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const int o = __shfl_up(wi, off);
            if (lane >= off)
                wi += o;
        }
        if (lane < kWaves)
            wave_excl[lane] = wi - ws;
    }
    __syncthreads();
    int run = wave_excl[wave] + incl - local;
    for (int i = beg; i < end; ++i) {
        const int c = hist[i];
        hist[i] = run;
        out_offsets[i] = run;
        run += c;
    }
    if (tid == kThreads - 1) {  // its run ends at the grand total
        hist[NK] = run;
        out_offsets[NK] = run;
    }
    __syncthreads();
    const int total = hist[NK];
    for (int i = total + tid; i < n; i += kThreads)
        out_list[i] = -1;

    // GEMM work list: chunks of at most tile_rows rows per expert, in expert
    // order.  Same run-per-thread scan as above, over ceil(count / tile_rows).
    if (!by_segment && a.tiles) {
        int tl = 0;
        for (int i = beg; i < end; ++i) {
            const int c = (i + 1 < NK ? hist[i + 1] : total) - hist[i];
            tl += (c + a.tile_rows - 1) / a.tile_rows;
        }
        int ti = tl;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(ti, off);
            if (lane >= off)
                ti += o;
        }
        if (lane == kWave - 1)
            tile_excl[wave] = ti;
        __syncthreads();
        if (wave == 0) {
            const int ws = lane < kWaves ? tile_excl[lane] : 0;
            int wi = ws;
#pragma unroll
            for (int off = 1; off < kWaves; off <<= 1) {
                const int o = __shfl_up(wi, off);
                if (lane >= off)
                    wi += o;
            }
            if (lane < kWaves)
                tile_excl[lane] = wi - ws;
        }
        __syncthreads();
        int t0 = tile_excl[wave] + ti - tl;
        for (int i = beg; i < end; ++i) {
            const int first = hist[i];
            const int c = (i + 1 < NK ? hist[i + 1] : total) - first;
            const int tb = t0;  // every tile of expert i carries the expert's whole range
            for (int r = 0; r < c; r += a.tile_rows)
                a.tiles[t0++] = make_int4(i, first, c, tb);
        }
        if (tid == kThreads - 1) {  // t0 is now the number of tiles
            tile_total = t0;
            if (a.tile_count)
                *a.tile_count = t0;
        }
        __syncthreads();
        for (int i = tile_total + tid; i < a.max_tiles; i += kThreads)
            a.tiles[i] = make_int4(-1, 0, 0, 0);
    }

    // 3. stable ranks: split the slots into W contiguous chunks, one per wave
    const int W = max(1, min(kWaves, kTable / NK));
    const int chunk = (n + W - 1) / W;
    for (int i = tid; i < W * NK; i += kThreads)
        table[i] = 0;
    __syncthreads();
    if (wave < W) {
        const int cb = wave * chunk;
        const int ce = min(n, cb + chunk);
        for (int x = cb + lane; x < ce; x += kWave) {
            const int key = key_of(x);
            if (key >= 0)
                atomicAdd(&table[wave * NK + key], 1);
        }
    }
    __syncthreads();
    for (int key = tid; key < NK; key += kThreads) {  // offsets of each wave's first slot per key
        int r = hist[key];
        for (int w = 0; w < W; ++w) {
            const int c = table[w * NK + key];
            table[w * NK + key] = r;
            r += c;
        }
    }
    __syncthreads();
    if (wave < W) {
        const int cb = wave * chunk;
        const int ce = min(n, cb + chunk);
        volatile int *tab = table + wave * NK;
        const int nbits = NK > 1 ? 32 - __clz(NK - 1) : 0;
        const unsigned long long lt = (1ull << lane) - 1ull;
        for (int base = cb; base < ce; base += kWave) {
            const int x = base + lane;
            const int key = x < ce ? key_of(x) : -1;
            unsigned long long same = __ballot(key >= 0);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = (key >> b) & 1;
                const unsigned long long bb = __ballot(bit);
                same &= bit ? bb : ~bb;
            }
            if (key >= 0) {
                const int pos = tab[key] + __popcll(same & lt);
                if (by_segment) {
                    a.seg_slots[pos] = x;
                } else {
                    a.perm2exp[pos] = x;
                    a.exp2perm[x] = pos;
                }
            } else if (!by_segment && x < ce) {
                a.exp2perm[x] = -1;
            }
            // LDS operations of one wave complete in issue order, so every
            // lane's read above precedes this update by the group's last lane.
            if (key >= 0 && (same >> lane) == 1ull)
                tab[key] = tab[key] + __popcll(same);
        }
    }
}

} // namespace

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(permute_kernel, dim3(2), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
