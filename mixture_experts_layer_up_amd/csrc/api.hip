// api.hip -- the C ABI: validation, workspace layout, stage sequencing.
//
// Stage order follows the pages' launcher: routing -> permute -> gate_up
// GEMM -> LoRA-aware activation -> down GEMM -> finalize, with the gate_up
// LoRA shrink/expand before the activation and the down LoRA after the down
// GEMM ("BF16 support for the experimental_sgl_trtllm MoE-LoRA path",
// "Files changed" table, launcher and single-stream dispatch rows, and Flow
// section 1(A)).  Here the two LoRA expands run inside the GEMMs, the
// activation is the gate_up GEMM's epilogue, and the down delta is summed
// into y before the finalize applies the routing weight.
//
// Validation is pure host code and touches no HIP API, so it runs (and is
// tested) on a machine without a GPU.  Forward never allocates and never
// waits on the device.
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "moe_lora.h"

using namespace moe_lora;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int round8(int r) { return (r + 7) / 8 * 8; }

int validate_shape(const moe_lora_shape *s)
{
    if (!s)
        return MOE_LORA_ERR_INVALID_ARG;
    if (s->num_tokens < 0 || s->top_k < 1 || s->top_k > 64 || s->num_experts < 1 ||
        s->num_experts > 1024 || s->top_k > s->num_experts)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)s->num_tokens * s->top_k > (int64_t)1 << 24)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if (s->hidden < 64 || s->hidden > 65536 || s->hidden % 64 != 0)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if (s->inter < 32 || s->inter > 65536 || s->inter % 32 != 0)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if (s->local_expert_offset < 0 || s->local_num_experts < 1 ||
        (int64_t)s->local_expert_offset + s->local_num_experts > s->num_experts)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if (s->num_loras < 0 || s->num_loras > 64 ||
        (int64_t)s->num_loras * s->local_num_experts > 8192)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if (s->rank_gate_up < 0 || s->rank_gate_up > 256 || s->rank_down < 0 || s->rank_down > 256)
        return MOE_LORA_ERR_UNSUPPORTED_SHAPE;
    if (!std::isfinite(s->routed_scaling_factor))
        return MOE_LORA_ERR_INVALID_ARG;
    if (s->lora_shared_outer != 0 && s->lora_shared_outer != 1)
        return MOE_LORA_ERR_INVALID_ARG;
    if (s->routing_method != 0 && s->routing_method != 1)
        return MOE_LORA_ERR_INVALID_ARG;
    return MOE_LORA_OK;
}

bool lora_gate_up_active(const moe_lora_shape *s) { return s->num_loras > 0 && s->rank_gate_up > 0; }
bool lora_down_active(const moe_lora_shape *s) { return s->num_loras > 0 && s->rank_down > 0; }

// Workspace regions; every offset is a multiple of 256 bytes.
struct Layout {
    size_t ids, weights, counts, offsets, exp2perm, perm2exp, seg_offsets, seg_slots;
    size_t perm_scratch, tiles, tile_count, zeros, s_gu, act, s_dn, y;
    int tile_rows, max_tiles;
    size_t total;
};

Layout make_layout(const moe_lora_shape *s)
{
    const size_t n = (size_t)s->num_tokens * s->top_k;
    const size_t el = (size_t)s->local_num_experts;
    const size_t segs = (size_t)s->num_loras * el;
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, kAlign);
        return at;
    };
    L.ids = take(n * 4);
    L.weights = take(n * 4);
    L.counts = take(el * 4);
    L.offsets = take((el + 1) * 4);
    L.exp2perm = take(n * 4);
    L.perm2exp = take(n * 4);
    L.seg_offsets = take((segs + 1) * 4);
    L.seg_slots = take(n * 4);
    L.perm_scratch = take(permute_scratch_bytes((int)n, (int)el, s->num_loras));
    L.tile_rows = gemm_tile_rows((int)n, (int)el, s->hidden, s->inter,
                                 lora_gate_up_active(s) ? s->rank_gate_up : 0,
                                 lora_down_active(s) ? s->rank_down : 0);
    L.max_tiles = max_gemm_tiles((int)n, (int)el, L.tile_rows);
    L.tiles = take((size_t)L.max_tiles * sizeof(int4));
    L.tile_count = take(sizeof(int32_t));
    L.zeros = take(kZeroBytes);
    L.s_gu = take(lora_gate_up_active(s) ? n * round8(s->rank_gate_up) * 2 : 0);
    L.act = take(n * (size_t)s->inter * 2);
    L.s_dn = take(lora_down_active(s) ? n * round8(s->rank_down) * 2 : 0);
    L.y = take(n * (size_t)s->hidden * 2);
    L.total = o;
    return L;
}

int check(hipError_t e) { return e == hipSuccess ? MOE_LORA_OK : MOE_LORA_ERR_HIP; }

#define MOE_TRY(expr)                  \
    do {                               \
        const int rc_ = (expr);        \
        if (rc_ != MOE_LORA_OK)        \
            return rc_;                \
    } while (0)

struct RoutingPtrs {
    int32_t *ids;
    float *weights;
    int32_t *counts, *offsets, *exp2perm, *perm2exp, *seg_offsets, *seg_slots;
};

// block_counts: permute_scratch_bytes of workspace (unused for one slot block)
int enqueue_routing(const moe_lora_shape *s, const float *logits, const float *bias,
                    const int32_t *topk_ids, const int32_t *mapping, int32_t *flags,
                    const RoutingPtrs &r, int32_t *block_counts, hipStream_t st,
                    int4 *tiles = nullptr, int tile_rows = 0, int max_tiles = 0,
                    int32_t *tile_count = nullptr, void *zeros = nullptr,
                    const ShrinkArgs *fuse_shrink = nullptr, bool *shrink_done = nullptr,
                    bool routed = false)
{
    if (logits && !routed) {
        RouteArgs ra{logits, r.ids, r.weights, s->num_tokens, s->num_experts, s->top_k,
                     bias, s->routing_method};
        MOE_TRY(check(launch_route(ra, st)));
    }
    PermuteArgs pa{};
    pa.topk_ids = logits ? r.ids : topk_ids;
    pa.mapping = mapping;
    pa.T = s->num_tokens;
    pa.k = s->top_k;
    pa.off = s->local_expert_offset;
    pa.E_l = s->local_num_experts;
    pa.L = s->num_loras;
    pa.expert_counts = r.counts;
    pa.expert_offsets = r.offsets;
    pa.exp2perm = r.exp2perm;
    pa.perm2exp = r.perm2exp;
    pa.seg_offsets = r.seg_offsets;
    pa.seg_slots = r.seg_slots;
    pa.tiles = tiles;
    pa.tile_rows = tile_rows;
    pa.max_tiles = max_tiles;
    pa.tile_count = tile_count;
    pa.zeros = static_cast<u32x4_t *>(zeros);
    pa.G = permute_blocks(s->num_tokens * s->top_k);
    pa.block_counts = block_counts;
    pa.E = s->num_experts;
    pa.flags = flags;
    // the gate_up shrink joins the permute's launch when the shapes allow it
    if (fuse_shrink && shrink_done && permute_shrink_fusable(pa, *fuse_shrink)) {
        MOE_TRY(check(launch_permute_shrink(pa, *fuse_shrink, st)));
        *shrink_done = true;
        return MOE_LORA_OK;
    }
    return check(launch_permute(pa, st));
}

// An empty batch: only the per-expert / per-segment arrays have entries; they
// are all zero.  Per-slot pointers may be NULL (empty tensors).
int enqueue_empty_batch(const moe_lora_shape *s, const moe_lora_routing *routing, hipStream_t st)
{
    if (!routing)
        return MOE_LORA_OK;
    if (!routing->expert_counts || !routing->expert_offsets || !routing->lora_seg_offsets)
        return MOE_LORA_ERR_INVALID_ARG;
    PermuteArgs pa{};
    pa.T = 0;
    pa.k = s->top_k;
    pa.off = s->local_expert_offset;
    pa.E_l = s->local_num_experts;
    pa.L = s->num_loras;
    pa.expert_counts = routing->expert_counts;
    pa.expert_offsets = routing->expert_offsets;
    pa.seg_offsets = routing->lora_seg_offsets;
    pa.G = 1;
    return check(launch_permute(pa, st));
}

int record(void *const *events, int i, hipStream_t st)
{
    if (!events || !events[i])
        return MOE_LORA_OK;
    return check(hipEventRecord(static_cast<hipEvent_t>(events[i]), st));
}

} // namespace

extern "C" {

size_t moe_lora_workspace_size(const moe_lora_shape *shape)
{
    if (validate_shape(shape) != MOE_LORA_OK)
        return 0;
    return make_layout(shape).total;
}

size_t moe_lora_packed_w13_bytes(const moe_lora_shape *shape)
{
    if (validate_shape(shape) != MOE_LORA_OK)
        return 0;
    return (size_t)shape->local_num_experts * shape->hidden * 2 * shape->inter * 2;
}

size_t moe_lora_packed_w2_bytes(const moe_lora_shape *shape)
{
    if (validate_shape(shape) != MOE_LORA_OK)
        return 0;
    return (size_t)shape->local_num_experts * shape->inter * shape->hidden * 2;
}

int moe_lora_pack_weights(const moe_lora_shape *shape, const void *w13, const void *w2,
                          void *w13_packed, void *w2_packed, void *stream)
{
    MOE_TRY(validate_shape(shape));
    if (!w13 || !w2 || !w13_packed || !w2_packed)
        return MOE_LORA_ERR_INVALID_ARG;
    if (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(w13_packed, 16) || !aligned(w2_packed, 16))
        return MOE_LORA_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    PackArgs p13{static_cast<const uint16_t *>(w13), static_cast<uint16_t *>(w13_packed),
                 shape->local_num_experts, shape->hidden, 2 * shape->inter, shape->inter};
    MOE_TRY(check(launch_pack(p13, st)));
    PackArgs p2{static_cast<const uint16_t *>(w2), static_cast<uint16_t *>(w2_packed),
                shape->local_num_experts, shape->inter, shape->hidden, 0};
    return check(launch_pack(p2, st));
}

size_t moe_lora_packed_lora_a_bytes(const moe_lora_shape *shape, int which)
{
    if (validate_shape(shape) != MOE_LORA_OK || (which != 0 && which != 1))
        return 0;
    const int r = which == 0 ? shape->rank_gate_up : shape->rank_down;
    if (shape->num_loras <= 0 || r <= 0)
        return 0;
    const int K = which == 0 ? shape->hidden : shape->inter;
    const size_t stacks = (size_t)shape->num_loras *
                          (which == 0 && shape->lora_shared_outer ? 1 : shape->local_num_experts);
    return stacks * lora_a_chunks(K) * r * 64 * 2;
}

int moe_lora_pack_lora_a(const moe_lora_shape *shape, const void *a_gate_up, const void *a_down,
                         void *a_gate_up_packed, void *a_down_packed, void *stream)
{
    MOE_TRY(validate_shape(shape));
    const bool gu = lora_gate_up_active(shape), dn = lora_down_active(shape);
    if ((gu && (!a_gate_up || !a_gate_up_packed)) || (dn && (!a_down || !a_down_packed)))
        return MOE_LORA_ERR_INVALID_ARG;
    if ((gu && (!aligned(a_gate_up, 16) || !aligned(a_gate_up_packed, 16))) ||
        (dn && (!aligned(a_down, 16) || !aligned(a_down_packed, 16))))
        return MOE_LORA_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int L = shape->num_loras, E_l = shape->local_num_experts;
    if (gu) {
        PackAArgs p{static_cast<const uint16_t *>(a_gate_up), static_cast<uint16_t *>(a_gate_up_packed),
                    L * (shape->lora_shared_outer ? 1 : E_l), shape->rank_gate_up, shape->hidden};
        MOE_TRY(check(launch_pack_lora_a(p, st)));
    }
    if (dn) {
        PackAArgs p{static_cast<const uint16_t *>(a_down), static_cast<uint16_t *>(a_down_packed),
                    L * E_l, shape->rank_down, shape->inter};
        MOE_TRY(check(launch_pack_lora_a(p, st)));
    }
    return MOE_LORA_OK;
}

size_t moe_lora_route_workspace_size(const moe_lora_shape *shape)
{
    if (validate_shape(shape) != MOE_LORA_OK)
        return 0;
    return permute_scratch_bytes(shape->num_tokens * shape->top_k, shape->local_num_experts,
                                 shape->num_loras);
}

int moe_lora_route(const moe_lora_shape *shape, const float *router_logits,
                   const float *routing_bias, const int32_t *topk_ids, const float *topk_weights,
                   const int32_t *token_lora_mapping, const moe_lora_routing *routing,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    MOE_TRY(validate_shape(shape));
    if (!routing)
        return MOE_LORA_ERR_INVALID_ARG;
    const size_t need = moe_lora_route_workspace_size(shape);
    if (need > 0 && !workspace)
        return MOE_LORA_ERR_INVALID_ARG;
    if (workspace_bytes < need)
        return MOE_LORA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, 16))
        return MOE_LORA_ERR_MISALIGNED;
    if (shape->num_tokens == 0)
        return enqueue_empty_batch(shape, routing, static_cast<hipStream_t>(stream));
    const bool from_logits = router_logits != nullptr;
    if (from_logits == (topk_ids != nullptr || topk_weights != nullptr))
        return MOE_LORA_ERR_INVALID_ARG;
    if (!from_logits && (!topk_ids || !topk_weights))
        return MOE_LORA_ERR_INVALID_ARG;
    if (from_logits && (!routing->topk_ids || !routing->topk_weights))
        return MOE_LORA_ERR_INVALID_ARG;
    if (!routing->expert_counts || !routing->expert_offsets ||
        !routing->expanded_idx_to_permuted_idx || !routing->permuted_idx_to_expanded_idx ||
        !routing->lora_seg_offsets || !routing->lora_seg_slots)
        return MOE_LORA_ERR_INVALID_ARG;
    RoutingPtrs r{routing->topk_ids, routing->topk_weights, routing->expert_counts,
                  routing->expert_offsets, routing->expanded_idx_to_permuted_idx,
                  routing->permuted_idx_to_expanded_idx, routing->lora_seg_offsets,
                  routing->lora_seg_slots};
    return enqueue_routing(shape, router_logits, routing_bias, topk_ids, token_lora_mapping,
                           routing->input_flags, r, static_cast<int32_t *>(workspace),
                           static_cast<hipStream_t>(stream));
}

} // extern "C"

namespace {

// Every argument check of a forward with tokens, except the workspace's:
// host code only, before any HIP call.
int validate_inputs(const moe_lora_shape *shape, const moe_lora_inputs *in,
                    const moe_lora_routing *routing, const void *out, const void *stream)
{
    // expert_out: the per-slot outputs go to the caller and the finalize is
    // skipped; the caller needs the routing export to finalize them
    const void *expert_out = in->expert_out;
    if ((!expert_out && !out) || (expert_out && !routing))
        return MOE_LORA_ERR_INVALID_ARG;
    if (!in->hidden || !in->w13_packed || !in->w2_packed)
        return MOE_LORA_ERR_INVALID_ARG;
    if (in->side_stream && (!in->fork_event || !in->join_event))
        return MOE_LORA_ERR_INVALID_ARG;
    if (in->side_stream && in->side_stream == stream)
        return MOE_LORA_ERR_INVALID_ARG;
    const bool from_logits = in->router_logits != nullptr;
    if (from_logits == (in->topk_ids != nullptr || in->topk_weights != nullptr))
        return MOE_LORA_ERR_INVALID_ARG;
    if (!from_logits && (!in->topk_ids || !in->topk_weights))
        return MOE_LORA_ERR_INVALID_ARG;
    const bool gu = lora_gate_up_active(shape);
    const bool dn = lora_down_active(shape);
    if (gu && (!in->lora_a_gate_up || !in->lora_b_gate_up))
        return MOE_LORA_ERR_INVALID_ARG;
    if (dn && (!in->lora_a_down || !in->lora_b_down))
        return MOE_LORA_ERR_INVALID_ARG;
    if (!aligned(in->hidden, 16) || !aligned(in->w13_packed, 16) || !aligned(in->w2_packed, 16) ||
        !aligned(out, 16) || !aligned(expert_out, 16))
        return MOE_LORA_ERR_MISALIGNED;
    if (gu && (!aligned(in->lora_a_gate_up, 16) ||
               !aligned(in->lora_b_gate_up, shape->rank_gate_up % 8 == 0 ? 16 : 2)))
        return MOE_LORA_ERR_MISALIGNED;
    if (dn && (!aligned(in->lora_a_down, 16) ||
               !aligned(in->lora_b_down, shape->rank_down % 8 == 0 ? 16 : 2)))
        return MOE_LORA_ERR_MISALIGNED;
    if (routing && (!routing->expert_counts || !routing->expert_offsets ||
                    !routing->expanded_idx_to_permuted_idx ||
                    !routing->permuted_idx_to_expanded_idx || !routing->lora_seg_offsets ||
                    !routing->lora_seg_slots ||
                    (from_logits && (!routing->topk_ids || !routing->topk_weights))))
        return MOE_LORA_ERR_INVALID_ARG;
    return MOE_LORA_OK;
}

// The layer forward on a workspace the caller or the library provides.
int forward_impl(const moe_lora_shape *shape, const moe_lora_inputs *in,
                 const moe_lora_routing *routing, void *out, void *workspace,
                 size_t workspace_bytes, void *stream)
{
    MOE_TRY(validate_shape(shape));
    if (!in)
        return MOE_LORA_ERR_INVALID_ARG;
    if (shape->num_tokens == 0) {
        hipStream_t st = static_cast<hipStream_t>(stream);
        MOE_TRY(enqueue_empty_batch(shape, routing, st));
        for (int i = 0; i < MOE_LORA_NUM_STAGE_EVENTS; ++i)
            MOE_TRY(record(in->stage_events, i, st));
        return MOE_LORA_OK;
    }
    MOE_TRY(validate_inputs(shape, in, routing, out, stream));
    if (!workspace)
        return MOE_LORA_ERR_INVALID_ARG;
    if (!aligned(workspace, kAlign))
        return MOE_LORA_ERR_MISALIGNED;
    void *expert_out = in->expert_out;
    const bool from_logits = in->router_logits != nullptr;
    const bool gu = lora_gate_up_active(shape);
    const bool dn = lora_down_active(shape);
    const Layout lay = make_layout(shape);
    if (workspace_bytes < lay.total)
        return MOE_LORA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    RoutingPtrs r{};
    if (routing) {
        r = RoutingPtrs{routing->topk_ids, routing->topk_weights, routing->expert_counts,
                        routing->expert_offsets, routing->expanded_idx_to_permuted_idx,
                        routing->permuted_idx_to_expanded_idx, routing->lora_seg_offsets,
                        routing->lora_seg_slots};
        if (!from_logits) {
            r.ids = nullptr;
            r.weights = nullptr;
        }
    } else {
        r = RoutingPtrs{reinterpret_cast<int32_t *>(ws + lay.ids),
                        reinterpret_cast<float *>(ws + lay.weights),
                        reinterpret_cast<int32_t *>(ws + lay.counts),
                        reinterpret_cast<int32_t *>(ws + lay.offsets),
                        reinterpret_cast<int32_t *>(ws + lay.exp2perm),
                        reinterpret_cast<int32_t *>(ws + lay.perm2exp),
                        reinterpret_cast<int32_t *>(ws + lay.seg_offsets),
                        reinterpret_cast<int32_t *>(ws + lay.seg_slots)};
    }
    const float *weights = from_logits ? r.weights : in->topk_weights;
    void *const *ev = in->stage_events;

    const int T = shape->num_tokens, H = shape->hidden, I = shape->inter;
    const int k = shape->top_k, E_l = shape->local_num_experts, L = shape->num_loras;
    const int rg = shape->rank_gate_up, rd = shape->rank_down;
    uint16_t *s_gu = reinterpret_cast<uint16_t *>(ws + lay.s_gu);
    uint16_t *act = reinterpret_cast<uint16_t *>(ws + lay.act);
    uint16_t *s_dn = reinterpret_cast<uint16_t *>(ws + lay.s_dn);
    uint16_t *y = expert_out ? static_cast<uint16_t *>(expert_out)
                             : reinterpret_cast<uint16_t *>(ws + lay.y);
    const uint16_t *hidden = static_cast<const uint16_t *>(in->hidden);

    const ShrinkArgs sa_gu{hidden, 1, H, static_cast<const uint16_t *>(in->lora_a_gate_up),
                           rg, round8(rg), L, E_l, k, r.seg_offsets, r.seg_slots, r.exp2perm,
                           s_gu, T * k, shape->lora_shared_outer};

    MOE_TRY(record(ev, 0, st));
    int4 *tiles = reinterpret_cast<int4 *>(ws + lay.tiles);
    void *zeros = ws + lay.zeros;
    int32_t *tile_count = reinterpret_cast<int32_t *>(ws + lay.tile_count);
    int32_t *flags = in->input_flags ? in->input_flags : routing ? routing->input_flags : nullptr;
    int32_t *perm_scratch = reinterpret_cast<int32_t *>(ws + lay.perm_scratch);

    // Two-stream schedule (decode-shaped batches only): after routing, the
    // gate_up shrink runs on the side stream, straight from the ids and the
    // adapter mapping, while this stream runs the permute; this stream waits
    // for it before the gate_up GEMM, whose expand reads its output.  The
    // shrink computes every row as the one-stream launches do, so the result
    // is bitwise the one-stream result.
    PermuteArgs side_pa{};
    side_pa.topk_ids = from_logits ? r.ids : in->topk_ids;
    side_pa.mapping = in->token_lora_mapping;
    side_pa.T = T;
    side_pa.k = k;
    side_pa.off = shape->local_expert_offset;
    side_pa.E_l = E_l;
    side_pa.L = L;
    const bool two_stream = gu && in->side_stream != nullptr && T <= kTwoStreamMaxTokens &&
                            shrink_by_ids_supported(side_pa, sa_gu);
    bool shrink_done = false;
    if (two_stream) {
        hipStream_t side = static_cast<hipStream_t>(in->side_stream);
        hipEvent_t fork = static_cast<hipEvent_t>(in->fork_event);
        hipEvent_t join = static_cast<hipEvent_t>(in->join_event);
        if (from_logits) {
            RouteArgs ra{in->router_logits, r.ids, r.weights, T, shape->num_experts, k,
                         in->routing_bias, shape->routing_method};
            MOE_TRY(check(launch_route(ra, st)));
        }
        MOE_TRY(check(hipEventRecord(fork, st)));
        MOE_TRY(check(hipStreamWaitEvent(side, fork, 0)));
        MOE_TRY(check(launch_shrink_by_ids(side_pa, sa_gu, side)));
        MOE_TRY(check(hipEventRecord(join, side)));
        MOE_TRY(enqueue_routing(shape, in->router_logits, in->routing_bias, in->topk_ids,
                                in->token_lora_mapping, flags, r, perm_scratch, st, tiles,
                                lay.tile_rows, lay.max_tiles, tile_count, zeros, nullptr,
                                nullptr, /*routed=*/true));
        MOE_TRY(record(ev, 1, st));
        MOE_TRY(check(hipStreamWaitEvent(st, join, 0)));
        shrink_done = true;
    } else {
        // one stream: the gate_up shrink may run in the permute's launch
        MOE_TRY(enqueue_routing(shape, in->router_logits, in->routing_bias, in->topk_ids,
                                in->token_lora_mapping, flags, r, perm_scratch, st, tiles,
                                lay.tile_rows, lay.max_tiles, tile_count, zeros,
                                gu ? &sa_gu : nullptr, &shrink_done));
        MOE_TRY(record(ev, 1, st));
    }
    if (gu && !shrink_done)  // a launch of its own (many slots)
        MOE_TRY(check(launch_shrink(sa_gu, st)));
    MOE_TRY(record(ev, 2, st));

    GemmArgs g1{};
    g1.X = hidden;
    g1.gather_by_token = 1;
    g1.K = H;
    g1.Wp = static_cast<const uint16_t *>(in->w13_packed);
    g1.NT = 2 * I / 16;
    g1.S = gu ? s_gu : nullptr;
    g1.LB = gu ? static_cast<const uint16_t *>(in->lora_b_gate_up) : nullptr;
    g1.r = gu ? rg : 0;
    g1.rp = gu ? round8(rg) : 8;
    g1.L = gu ? L : 0;
    g1.n_canon = 2 * I;
    g1.mapping = in->token_lora_mapping;
    g1.tiles = tiles;
    g1.tile_count = tile_count;
    g1.n_tiles = lay.max_tiles;
    g1.tile_rows = lay.tile_rows;
    g1.perm2exp = r.perm2exp;
    g1.E_l = E_l;
    g1.k = k;
    g1.I = I;
    g1.Y = act;
    // column slabs per expert: 64 columns (decode kernel) or 256 (wide kernel)
    auto slabs = [&](int NT) {
        return lay.tile_rows == kDecodeTileRows ? NT / 4 : gemm_wide_slabs(NT);
    };
    g1.n_slabs = slabs(g1.NT);
    g1.zeros = static_cast<const uint16_t *>(zeros);
    MOE_TRY(check(launch_gemm_gate_up(g1, st)));
    MOE_TRY(record(ev, 3, st));

    if (dn) {
        ShrinkArgs sa{act, 0, I, static_cast<const uint16_t *>(in->lora_a_down),
                      rd, round8(rd), L, E_l, k, r.seg_offsets, r.seg_slots, r.exp2perm, s_dn,
                      T * k, 0};
        MOE_TRY(check(launch_shrink(sa, st)));
    }
    MOE_TRY(record(ev, 4, st));

    GemmArgs g2{};
    g2.X = act;
    g2.gather_by_token = 0;
    g2.K = I;
    g2.Wp = static_cast<const uint16_t *>(in->w2_packed);
    g2.NT = H / 16;
    g2.S = dn ? s_dn : nullptr;
    g2.LB = dn ? static_cast<const uint16_t *>(in->lora_b_down) : nullptr;
    g2.r = dn ? rd : 0;
    g2.rp = dn ? round8(rd) : 8;
    g2.L = dn ? L : 0;
    g2.n_canon = H;
    g2.mapping = in->token_lora_mapping;
    g2.tiles = tiles;
    g2.tile_count = tile_count;
    g2.n_tiles = lay.max_tiles;
    g2.tile_rows = lay.tile_rows;
    g2.perm2exp = r.perm2exp;
    g2.E_l = E_l;
    g2.k = k;
    g2.I = I;
    g2.Y = y;
    g2.n_slabs = slabs(g2.NT);
    g2.zeros = static_cast<const uint16_t *>(zeros);
    g2.lb_shared = shape->lora_shared_outer;
    MOE_TRY(check(launch_gemm_down(g2, st)));
    MOE_TRY(record(ev, 5, st));

    if (!expert_out) {
        FinalizeArgs fa{y, r.exp2perm, weights, static_cast<uint16_t *>(out), T, H, k,
                        shape->routed_scaling_factor};
        MOE_TRY(check(launch_finalize(fa, st)));
    }
    MOE_TRY(record(ev, 6, st));
    return MOE_LORA_OK;
}

// The allocation-free forward's workspace: one array per device, in the
// library's code object, MOE_LORA_STATIC_SCRATCH_BYTES long.  Host code never
// uses the array's name as an address: the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device (with that device
// current) and kept here.
__device__ __align__(256) unsigned char scratch[MOE_LORA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once known

// Device address of the current device's scratch array.
int current_device_scratch(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MOE_LORA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_LORA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_LORA_OK;
}

} // namespace

extern "C" {

int moe_lora_forward(const moe_lora_shape *shape, const moe_lora_inputs *inputs,
                     const moe_lora_routing *routing, void *out, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    return forward_impl(shape, inputs, routing, out, workspace, workspace_bytes, stream);
}

int moe_lora_forward_no_alloc(const moe_lora_shape *shape, const moe_lora_inputs *inputs,
                              const moe_lora_routing *routing, void *out, void *stream)
{
    MOE_TRY(validate_shape(shape));
    if (!inputs)
        return MOE_LORA_ERR_INVALID_ARG;
    if (shape->num_tokens > 0)
        MOE_TRY(validate_inputs(shape, inputs, routing, out, stream));
    if (make_layout(shape).total > MOE_LORA_STATIC_SCRATCH_BYTES)
        return MOE_LORA_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    MOE_TRY(current_device_scratch(&ws));
    return forward_impl(shape, inputs, routing, out, ws, MOE_LORA_STATIC_SCRATCH_BYTES, stream);
}

int moe_lora_finalize(const moe_lora_shape *shape, const void *expert_out,
                      const int32_t *expanded_idx_to_permuted_idx, const float *topk_weights,
                      void *out, void *stream)
{
    MOE_TRY(validate_shape(shape));
    if (shape->num_tokens == 0)
        return MOE_LORA_OK;
    if (!expert_out || !expanded_idx_to_permuted_idx || !topk_weights || !out)
        return MOE_LORA_ERR_INVALID_ARG;
    if (!aligned(expert_out, 16) || !aligned(out, 16))
        return MOE_LORA_ERR_MISALIGNED;
    FinalizeArgs fa{static_cast<const uint16_t *>(expert_out), expanded_idx_to_permuted_idx,
                    topk_weights, static_cast<uint16_t *>(out), shape->num_tokens,
                    shape->hidden, shape->top_k, shape->routed_scaling_factor};
    return check(launch_finalize(fa, static_cast<hipStream_t>(stream)));
}

const char *moe_lora_strerror(int status)
{
    switch (status) {
    case MOE_LORA_OK:
        return "ok";
    case MOE_LORA_ERR_INVALID_ARG:
        return "invalid argument (null pointer or inconsistent inputs)";
    case MOE_LORA_ERR_UNSUPPORTED_SHAPE:
        return "unsupported shape (see limits in moe_lora.h)";
    case MOE_LORA_ERR_WORKSPACE_TOO_SMALL:
        return "workspace too small";
    case MOE_LORA_ERR_MISALIGNED:
        return "pointer not aligned as required";
    case MOE_LORA_ERR_HIP:
        return "HIP launch or event call failed";
    case MOE_LORA_ERR_SCRATCH_LIMIT:
        return "shape needs more workspace than the static scratch of moe_lora_forward_no_alloc "
               "holds (MOE_LORA_STATIC_SCRATCH_BYTES)";
    default:
        return "unknown status";
    }
}

} // extern "C"
