// kernels.h -- argument blocks and host launchers of the gfx950 kernels.
// Internal to the library; the public interface is include/moe_lora.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_lora {

struct RouteArgs {
    const float *logits;   // [T, E]
    int32_t *topk_ids;     // [T, k]
    float *topk_weights;   // [T, k]
    int T, E, k;
    const float *bias;     // [E] selection bias, or null
    int method;            // 0: softmax over the selected; 1: softmax over all E
};

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

struct PermuteArgs {
    const int32_t *topk_ids;   // [T*k]
    const int32_t *mapping;    // [T] or null
    int T, k, off, E_l, L;
    int32_t *expert_counts, *expert_offsets;
    int32_t *exp2perm, *perm2exp;
    int32_t *seg_offsets, *seg_slots;
    // GEMM work list (optional): ceil(rows / tile_rows) entries per expert
    // with rows, each {local expert, its first permuted row, its rows, index
    // of its first entry}; unused entries up to max_tiles have expert -1.
    int4 *tiles;
    int tile_rows, max_tiles;
    int32_t *tile_count;       // number of used work-list entries
    u32x4_t *zeros;            // kZeroBytes written as zero (for the GEMMs)
    int G;                     // slot blocks: permute_blocks(T * k)
    int32_t *block_counts;     // G > 1: permute_scratch_bytes of workspace
    int E;                     // global experts: valid ids are [-1, E)
    int32_t *flags;            // MOE_LORA_FLAG_* bits ORed in (or null)
};

// The permute cuts the slots into blocks of kPermuteSlotsPerBlock; with more
// than one block its count kernel writes every block's histogram of both key
// types to the workspace, rows padded to a multiple of 4 keys, followed by
// one totals row per key type: (G + 1) * (round4(E_l) + round4(L * E_l))
// int32.
constexpr int kPermuteSlotsPerBlock = 1024;

inline int permute_blocks(int n)
{
    return n <= 0 ? 1 : (n + kPermuteSlotsPerBlock - 1) / kPermuteSlotsPerBlock;
}

inline size_t round4_host(size_t v) { return (v + 3) / 4 * 4; }

inline size_t permute_scratch_bytes(int n, int E_l, int L)
{
    const int G = permute_blocks(n);
    return G > 1 ? ((size_t)G + 1) * (round4_host(E_l) + round4_host((size_t)L * E_l)) * 4 : 0;
}

// A small all-zero region of the workspace, rewritten by every permute
// launch; the wide GEMM's direct loads read it in place of masked values.
constexpr int kZeroBytes = 1024;

// Blocks of a GEMM launch over n_tiles work-list entries (an upper bound)
// and n_slabs column slabs: a multiple of 8, so that every (XCD, index) pair
// the device-side work split uses exists (xcd_balanced_item hands XCD x the
// items x * per .. x * per + per - 1, per = ceil(items / 8), to the blocks
// x, x + 8, ..., which needs 8 * per blocks).
inline int gemm_grid_blocks(int n_tiles, int n_slabs)
{
    return (n_tiles * n_slabs + 7) / 8 * 8;
}

// Upper bound on the GEMM work-list length for n slots and E_l experts.
inline int max_gemm_tiles(int n, int E_l, int tile_rows)
{
    return (n + tile_rows - 1) / tile_rows + (E_l < n ? E_l : n);
}

struct PackArgs {
    const uint16_t *src;   // [E_l, K, N]
    uint16_t *dst;
    int E_l, K, N, I;      // I > 0: gate/up interleaved tile order (w13)
};

// The packed LoRA A layout the shrink kernels read.  Per stack (one r x K
// matrix), K runs in chunks of 64 values (the last one zero-padded), and a
// chunk holds the r rank rows' 64 values one after another:
//   element (stack, q, k) at ((stack * lora_a_chunks(K) + k / 64) * r + q) * 64 + k % 64
// so that the rank rows of one chunk are one contiguous r x 128-byte run.
__host__ __device__ inline int lora_a_chunks(int K) { return (K + 63) >> 6; }

struct PackAArgs {
    const uint16_t *src;   // [stacks, r, K], row-major
    uint16_t *dst;         // [stacks, lora_a_chunks(K), r, 64]
    int stacks, r, K;      // K % 32 == 0
};

// LoRA shrink S[p] = A[l, e] * X(row), grouped by (adapter, local expert).
struct ShrinkArgs {
    const uint16_t *X;        // gather_by_token ? hidden [T, K] : act [n, K]
    int gather_by_token;
    int K;
    const uint16_t *A;        // packed [L, E_l (shared: 1), lora_a_chunks(K), r, 64]
    int r, rp, L, E_l, k;
    const int32_t *seg_offsets, *seg_slots, *exp2perm;
    uint16_t *S;              // [n, rp], row = slot x = t * k + j
    int n_slots;              // T * k (sizes the rows per pass)
    int a_shared;             // A holds one stack per adapter ([L, 1, r, K])
};

// Grouped expert GEMM over one packed weight stack, with the LoRA expand
// folded in as extra K (S [n, rp] against the LoRA B stack).
struct GemmArgs {
    const uint16_t *X;        // gather_by_token ? hidden [T, K] : act [n, K]
    int gather_by_token;
    int K;                    // H for gate_up, I for down
    const uint16_t *Wp;       // packed [E_l, NT, K/32, 64, 8]
    int NT;                   // 16-column tiles per expert
    const uint16_t *S;        // [n, rp] by slot x, or null
    const uint16_t *LB;       // [L, E_l, n_canon, r] or null
    int r, rp, L, n_canon;
    const int32_t *mapping;   // [T] or null
    const int4 *tiles;        // work list written by the permute kernel
    const int32_t *tile_count; // its used length, written by the permute kernel
    int n_tiles, tile_rows;   // list length (upper bound), rows per tile
    const int32_t *perm2exp;  // [n]
    int E_l, k, I;
    uint16_t *Y;              // gated: act [n, I]; else y [n, n_canon]
    int n_slabs;
    int slabs_per_block;      // wide kernel: adjacent slabs one block runs in turn (set by its launcher)
    const uint16_t *zeros;    // kZeroBytes of zeros
    int lb_shared;            // LB holds one stack per adapter ([L, 1, n_canon, r])
};

// Rows per GEMM work-list tile: 16 for the decode-shaped kernel (few rows
// per expert); for the wide kernel (many rows per expert, when the shape
// allows it) a multiple of 16 up to kWideMaxTileRows, chosen so that one
// tile usually holds all rows of an expert.
constexpr int kDecodeTileRows = 16;
constexpr int kWideMaxTileRows = 176;
// r_gu, r_dn: ranks of the active LoRA projections (0 when inactive)
bool gemm_wide_supported(int H, int I, int r_gu, int r_dn);
int gemm_wide_slabs(int NT);  // column slabs of the wide kernel for NT 16-column tiles
int gemm_wide_slabs_per_block(int n_slabs, int n_tiles, int E_l);
int gemm_tile_rows(int n_slots, int E_l, int H, int I, int r_gu, int r_dn);
hipError_t launch_gemm_wide(const GemmArgs &a, bool gated, hipStream_t s);

struct FinalizeArgs {
    const uint16_t *Y;        // [n, H]
    const int32_t *exp2perm;  // [T*k]
    const float *weights;     // [T, k]
    uint16_t *out;            // [T, H]
    int T, H, k;
    float scale;
};

hipError_t launch_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_permute(const PermuteArgs &a, hipStream_t s);
hipError_t launch_pack(const PackArgs &a, hipStream_t s);
hipError_t launch_pack_lora_a(const PackAArgs &a, hipStream_t s);
hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t s);
// launch_shrink's choices: the many-row kernel, else the few-row kernel with
// 16 * shrink_row_tiles(a) rows per pass
bool shrink_uses_wide(const ShrinkArgs &a);
int shrink_row_tiles(const ShrinkArgs &a);
// The permute (one slot block) and the gate_up shrink (few-row kernel) in one
// launch; permute_shrink_fusable says whether the shapes allow it.
bool permute_shrink_fusable(const PermuteArgs &pa, const ShrinkArgs &sa);
hipError_t launch_permute_shrink(const PermuteArgs &pa, const ShrinkArgs &sa, hipStream_t s);
// The same few-row gate_up shrink from the routing alone (ids, mapping), on
// a launch of its own: the side stream of the two-stream schedule.  Every
// row is computed as by the permute's fused launch and by launch_shrink's
// few-row kernel, bit for bit.  Up to kShrinkByIdsMaxSlots slots.
constexpr int kShrinkByIdsMaxSlots = 2048;
// The two-stream schedule is for decode-shaped batches: at most this many
// tokens (the pages' decode gate), and the slot and segment sizes the
// side-stream shrink takes (shrink_by_ids_supported).
constexpr int kTwoStreamMaxTokens = 256;
bool shrink_by_ids_supported(const PermuteArgs &pa, const ShrinkArgs &sa);
hipError_t launch_shrink_by_ids(const PermuteArgs &pa, const ShrinkArgs &sa, hipStream_t s);
// the shrink for segments of many rows: rank r <= 64, mean_rows per segment
bool shrink_wide_supported(int r);
hipError_t launch_shrink_wide(const ShrinkArgs &a, int mean_rows, hipStream_t s);
hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs &a, hipStream_t s);

} // namespace moe_lora
