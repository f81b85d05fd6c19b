/*
 * moe_lora.h -- C ABI of the MI355X (gfx950) bf16 routed MoE-LoRA layer.
 *
 * One layer forward: top-k routing -> expert permutation -> gate_up grouped
 * GEMM with the per-adapter LoRA delta added before SwiGLU -> down grouped
 * GEMM with the down LoRA delta -> routing-weighted finalize back to tokens.
 * Sources for the operation:
 *   "BF16 support for the experimental_sgl_trtllm MoE-LoRA path" (GitHub PR
 *   page), "Files changed" table (launcher row: the pipeline order, where the
 *   gate_up delta enters, what the activation writes) and Flow sections 1
 *   and 2 (which LoRA add is weighted by the routing weight, virtual-expert
 *   addressing of the LoRA weights, expert-parallel masking);
 *   "sglang PR #28953 digest", change summary (permuted index -1 for
 *   expert-parallel slots that are not local; never written through).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; the shape
 *     structs are HOST memory read during the call only.
 *   - bf16 tensors are passed as `const void*` holding IEEE bfloat16 bits,
 *     row-major, contiguous.  16-byte alignment is required where noted.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All device
 *     work is enqueued on it and the call returns without waiting; inputs
 *     must stay valid until the stream has passed the call.
 *   - The library never allocates device memory and never synchronises the
 *     host inside moe_lora_route / moe_lora_forward, so both can be captured
 *     into a HIP graph.  It keeps no state between calls; concurrent calls
 *     are safe when they use distinct outputs and workspaces.
 *   - Host-side validation needs no GPU: bad arguments return a negative
 *     status before any HIP call.  No entry point throws.
 *   - An empty batch (num_tokens == 0) is valid: per-token and per-slot
 *     pointers may then be NULL, nothing but the zero per-expert /
 *     per-segment counts and offsets of `routing` (when given) is written.
 *   - Device data that is out of range never faults: a top-k id outside
 *     [local_expert_offset, local_expert_offset + local_num_experts) is a
 *     non-local slot (contributes nothing), and a token_lora_mapping value
 *     outside [-1, num_loras) is treated as -1 (no adapter).
 */
#ifndef MOE_LORA_H_
#define MOE_LORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_LORA_OK                       0
#define MOE_LORA_ERR_INVALID_ARG         -1 /* null pointer, bad combination */
#define MOE_LORA_ERR_UNSUPPORTED_SHAPE   -2 /* dimension outside the limits below */
#define MOE_LORA_ERR_WORKSPACE_TOO_SMALL -3
#define MOE_LORA_ERR_MISALIGNED          -4 /* pointer not aligned as required */
#define MOE_LORA_ERR_HIP                 -5 /* a HIP launch or event call failed */
#define MOE_LORA_ERR_SCRATCH_LIMIT       -6 /* moe_lora_forward_no_alloc: the shape needs more
                                               than MOE_LORA_STATIC_SCRATCH_BYTES of workspace */

/* Number of events moe_lora_forward records when moe_lora_inputs.stage_events
 * is set: before routing, then after each of routing+permute, gate_up LoRA
 * shrink, gate_up GEMM (+SwiGLU), down LoRA shrink, down GEMM, finalize.
 * With at most 1024 slots (T * k) on one stream the gate_up shrink runs in
 * the permute's launch, and with a side stream it runs there, so its stage
 * is then empty (the third event follows the second directly). */
#define MOE_LORA_NUM_STAGE_EVENTS 7

/*
 * Layer shape.  Limits (else MOE_LORA_ERR_UNSUPPORTED_SHAPE):
 *   0 <= num_tokens, num_tokens * top_k <= 2^24
 *   hidden % 64 == 0, 64 <= hidden <= 65536
 *   inter % 32 == 0, 32 <= inter <= 65536
 *   1 <= num_experts <= 1024, 1 <= top_k <= min(64, num_experts)
 *   0 <= local_expert_offset, 1 <= local_num_experts,
 *   local_expert_offset + local_num_experts <= num_experts
 *   0 <= num_loras <= 64, num_loras * local_num_experts <= 8192
 *   0 <= rank_gate_up, rank_down <= 256
 *   lora_shared_outer is 0 or 1, routing_method is 0 or 1 (else
 *   MOE_LORA_ERR_INVALID_ARG)
 * A LoRA projection is active when num_loras > 0 and its rank > 0.
 *
 * lora_shared_outer = 1 selects the shared-outer LoRA layout ("BF16 support
 * for the experimental_sgl_trtllm MoE-LoRA path", Flow section 2): the outer
 * matrices hold one weight set per adapter, used for every expert and never
 * sliced by the expert-parallel window (lora_a_gate_up [L, 1, r_gu, H],
 * lora_b_down [L, 1, H, r_dn]); the inner ones (lora_b_gate_up, lora_a_down)
 * stay per (adapter, local expert).
 */
typedef struct moe_lora_shape {
    int32_t num_tokens;            /* T */
    int32_t hidden;                /* H */
    int32_t inter;                 /* I, per expert; gate_up width is 2I */
    int32_t num_experts;           /* E: routed (global) experts */
    int32_t top_k;                 /* k */
    int32_t local_expert_offset;   /* first expert this shard owns */
    int32_t local_num_experts;     /* E_l: experts this shard owns */
    int32_t num_loras;             /* L: adapters in the stacks */
    int32_t rank_gate_up;          /* r_gu */
    int32_t rank_down;             /* r_dn */
    float routed_scaling_factor;   /* multiplies the routed sum (1.0 = none) */
    int32_t lora_shared_outer;     /* 0: per-expert LoRA stacks; 1: shared-outer */
    int32_t routing_method;        /* weights from router logits: 0 = softmax over
                                      the k selected logits; 1 = softmax over all
                                      E logits at the selected experts, not
                                      renormalised */
} moe_lora_shape;

/*
 * Routing results (device arrays, caller-owned).  Slot x = t * top_k + j.
 *   topk_ids      [T, k] int32  global expert ids, ordered by (logit desc,
 *                               id asc)
 *   topk_weights  [T, k] fp32   per routing_method (method 0: softmax over
 *                               the k selected logits)
 *   expert_counts [E_l]         local slots per local expert
 *   expert_offsets[E_l + 1]     exclusive prefix sum; [E_l] = P, the number
 *                               of local slots
 *   expanded_idx_to_permuted_idx [T*k]  permuted row p of slot x, or -1 for
 *                               a non-local slot; rows are expert-contiguous
 *                               and ascending in x inside one expert
 *   permuted_idx_to_expanded_idx [T*k]  inverse; entries [P, T*k) are -1
 *   lora_seg_offsets [L * E_l + 1]      exclusive prefix sum of the local
 *                               slots whose token has an adapter, keyed by
 *                               the virtual expert (adapter, local expert)
 *   lora_seg_slots   [T*k]      those slots (x), grouped by key, ascending
 *                               x inside a key; unused tail is -1
 */
typedef struct moe_lora_routing {
    int32_t *topk_ids;
    float *topk_weights;
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *expanded_idx_to_permuted_idx;
    int32_t *permuted_idx_to_expanded_idx;
    int32_t *lora_seg_offsets;
    int32_t *lora_seg_slots;
    int32_t *input_flags;   /* optional, see MOE_LORA_FLAG_* (moe_lora_route) */
} moe_lora_routing;

/*
 * Bad device-side values never fault: an expert id of a given top-k outside
 * [-1, num_experts) is a slot of no local expert (as -1 is), a
 * token_lora_mapping value outside [-1, num_loras) is -1.  When the caller
 * passes an `input_flags` pointer (one device int32, caller-owned), the call
 * ORs these bits into it for what it met; it never clears them, so the caller
 * zeroes the word and reads it after the stream has passed the call.
 */
#define MOE_LORA_FLAG_EXPERT_ID 1  /* a top-k id outside [-1, num_experts) */
#define MOE_LORA_FLAG_ADAPTER   2  /* a token_lora_mapping value outside [-1, num_loras) */

/*
 * Forward inputs.  Exactly one of `router_logits` or the pair
 * (`topk_ids`, `topk_weights`) is given.
 *   hidden             bf16 [T, H], 16-byte aligned
 *   router_logits      fp32 [T, E]
 *   routing_bias       fp32 [E] or NULL: added to the logits (one fp32 add)
 *                      for the choice of experts only; the weights still
 *                      come from the logits.  The pages name a routing bias
 *                      without defining it ("BF16 support for the
 *                      experimental_sgl_trtllm MoE-LoRA path", "Files
 *                      changed" table, launcher row); this is the reading
 *                      taken.  Ignored when top-k is given.
 *   topk_ids           int32 [T, k] (any value; out-of-window ids are
 *                      non-local slots), topk_weights fp32 [T, k]
 *   w13_packed         expert gate_up weights [E_l, H, 2I] (columns [0, I)
 *                      gate, [I, 2I) up) in the packed layout written by
 *                      moe_lora_pack_weights; 16-byte aligned
 *   w2_packed          expert down weights [E_l, I, H], packed; 16-byte aligned
 *   lora_a_gate_up     shrink stacks bf16 [L, E_l, r_gu, H] ([L, 1, r_gu, H]
 *                      in the shared-outer layout) in the packed layout
 *                      written by moe_lora_pack_lora_a; 16-byte aligned
 *   lora_b_gate_up     bf16 [L, E_l, 2I, r_gu]  (expand, as given; 16-byte
 *                      aligned when r_gu % 8 == 0, else 2-byte)
 *   lora_a_down        shrink stacks bf16 [L, E_l, r_dn, I], packed by
 *                      moe_lora_pack_lora_a; 16-byte aligned
 *   lora_b_down        bf16 [L, E_l, H, r_dn]   ([L, 1, H, r_dn] shared-outer)
 *   token_lora_mapping int32 [T], adapter of each token, -1 = none; NULL
 *                      means every token is -1
 *   stage_events       NULL, or MOE_LORA_NUM_STAGE_EVENTS hipEvent_t handles
 *                      recorded on `stream` at the stage boundaries (for
 *                      per-kernel timing); stages that do not run still get
 *                      their event recorded; a NULL entry is skipped (each
 *                      recorded event costs a few microseconds of stream
 *                      time, so record only the boundaries you need)
 *   expert_out         NULL (finalize into `out`), or bf16 [T*k, H], 16-byte
 *                      aligned: receives each local slot's expert output
 *                      (down projection plus down-LoRA delta, before the
 *                      routing weight) at its permuted row p; rows [P, T*k)
 *                      are not written.  The finalize is then skipped (the
 *                      pages' op likewise returns this triple instead of
 *                      finalizing when asked: "BF16 support for the
 *                      experimental_sgl_trtllm MoE-LoRA path", "Files
 *                      changed" table, launcher row); moe_lora_finalize
 *                      completes it.  Needs `routing`, which holds the other
 *                      two members of the triple.
 *   side_stream        NULL (everything on `stream`), or a second hipStream_t
 *                      (default priority, not `stream`) for the gate_up LoRA
 *                      shrink, the pages' two-stream schedule ("BF16 support
 *                      for the experimental_sgl_trtllm MoE-LoRA path",
 *                      Summary (phase 2) and Flow section 1(B): the gate_up
 *                      LoRA on a side stream, only for decode-sized batches,
 *                      joined before the activation).  Used for decode-shaped
 *                      batches only: num_tokens <= 256, num_tokens * top_k <=
 *                      2048, and LoRA segments of fewer than 16 rows on
 *                      average (num_tokens * top_k <= 15 * num_loras *
 *                      local_num_experts) or a gate_up rank above 64;
 *                      otherwise, and when the gate_up LoRA
 *                      is inactive, it is ignored and everything runs on
 *                      `stream`.  When used, the shrink runs on side_stream
 *                      straight from the routing while `stream` runs the
 *                      permute, and `stream` waits for it before the gate_up
 *                      GEMM (which holds the LoRA expand and the
 *                      activation).  The shrink computes every row exactly as
 *                      the one-stream path does: the output is bitwise the
 *                      one-stream output.
 *   input_flags        NULL, or one device int32 into which the MOE_LORA_FLAG_*
 *                      bits of this call are ORed (when NULL and `routing`
 *                      is given, routing->input_flags is used)
 *   fork_event,        caller-owned hipEvent_t handles (timing may be
 *   join_event         disabled), required with side_stream: fork_event is
 *                      recorded on `stream` after routing and waited by
 *                      side_stream; join_event is recorded on side_stream
 *                      after the shrink and waited by `stream` before the
 *                      gate_up GEMM.  Nothing is allocated, so a two-stream
 *                      forward can be captured into a HIP graph.  Not
 *                      touched when side_stream is ignored (see above).
 * LoRA pointers may be NULL when the projection is inactive.
 */
typedef struct moe_lora_inputs {
    const void *hidden;
    const float *router_logits;
    const float *routing_bias;
    const int32_t *topk_ids;
    const float *topk_weights;
    const void *w13_packed;
    const void *w2_packed;
    const void *lora_a_gate_up;
    const void *lora_b_gate_up;
    const void *lora_a_down;
    const void *lora_b_down;
    const int32_t *token_lora_mapping;
    void *const *stage_events;
    void *expert_out;
    void *side_stream;
    void *fork_event;
    void *join_event;
    int32_t *input_flags;
} moe_lora_inputs;

/* Bytes of device workspace moe_lora_forward needs for `shape` (host only,
 * pure; 0 for an invalid shape), with or without a side stream.  The
 * workspace must be 256-byte aligned. */
size_t moe_lora_workspace_size(const moe_lora_shape *shape);

/* Bytes of the packed expert weights (equal to the unpacked sizes). */
size_t moe_lora_packed_w13_bytes(const moe_lora_shape *shape);
size_t moe_lora_packed_w2_bytes(const moe_lora_shape *shape);

/*
 * One-time relayout of the expert weights into the MFMA operand layout the
 * grouped GEMMs stream (the pages' path likewise prepares its expert weights
 * once at load: "BF16 support for the experimental_sgl_trtllm MoE-LoRA path",
 * Summary and "Files changed" table, base_backend row).
 *   w13 bf16 [E_l, H, 2I] -> w13_packed, w2 bf16 [E_l, I, H] -> w2_packed.
 * Packed layout: for expert e, 64-column slab s, K chunk c (32 rows), tile t
 * (0..3, 16 columns), lane l (0..63), element i (0..7), the bf16 at
 *   (((e * NS + s) * KC + c) * 4 + t) * 512 + l * 8 + i
 * is W[e][32c + 8(l / 16) + i][col(4s + t) + l % 16], with NS = N / 64 slabs
 * and KC = K / 32 chunks.  For w13 (N = 2I), col(n) = (n % 2) * I + (n / 2) * 16
 * (gate and up tiles of the same columns alternate); for w2 (N = H),
 * col(n) = 16 n.  All four pointers 16-byte aligned; outputs must not overlap
 * inputs.
 */
int moe_lora_pack_weights(const moe_lora_shape *shape, const void *w13, const void *w2,
                          void *w13_packed, void *w2_packed, void *stream);

/*
 * One-time relayout of the LoRA A stacks (the shrink operands), done when
 * adapters are loaded, like the expert weights' pack.  The pages' LoRA path
 * keeps per-(adapter, expert) stacks addressed as virtual experts ("BF16
 * support for the experimental_sgl_trtllm MoE-LoRA path", Flow section 2);
 * only the order inside each stack changes here.  An r x K stack becomes
 * ceil(K / 64) chunks of r x 64 values, the rank rows of one chunk
 * contiguous:
 *   packed[((s * C + k / 64) * r + q) * 64 + k % 64] = A[s][q][k],  C = ceil(K / 64),
 * with zeros for K <= k < 64 C.  Stacks s run over [L, E_l] (gate_up in the
 * shared-outer layout: [L]); K is H for gate_up and I for down.  The shrink
 * reads a stack chunk by chunk with every rank row at once, so each chunk is
 * one sequential run instead of r rows 2K bytes apart.
 *   a_gate_up [L, E_l or 1, r_gu, H] -> a_gate_up_packed,
 *   a_down    [L, E_l, r_dn, I]      -> a_down_packed
 * (moe_lora_packed_lora_a_bytes bytes each, which = 0 gate_up, 1 down).
 * Pointers of an inactive projection may be NULL; all others 16-byte
 * aligned; outputs must not overlap inputs.
 */
size_t moe_lora_packed_lora_a_bytes(const moe_lora_shape *shape, int which);

int moe_lora_pack_lora_a(const moe_lora_shape *shape, const void *a_gate_up, const void *a_down,
                         void *a_gate_up_packed, void *a_down_packed, void *stream);

/*
 * Routing and permutation only.  Routes from `router_logits` (with the
 * optional `routing_bias`, as in moe_lora_inputs) when given, else takes
 * `topk_ids` / `topk_weights` as they are (then routing->topk_ids
 * and routing->topk_weights are not written and may be NULL).  Every other
 * field of `routing` must be non-NULL, except `input_flags` (optional: the
 * MOE_LORA_FLAG_* bits of this call are ORed into it).  `token_lora_mapping` as in
 * moe_lora_inputs.  `workspace` is device memory of at least
 * moe_lora_route_workspace_size(shape) bytes, 16-byte aligned (the permute's
 * per-block histograms; its contents on entry do not matter); it may be NULL
 * when that size is 0, i.e. for at most 1024 slots (T * k).
 */
size_t moe_lora_route_workspace_size(const moe_lora_shape *shape);

int moe_lora_route(const moe_lora_shape *shape, const float *router_logits,
                   const float *routing_bias, const int32_t *topk_ids, const float *topk_weights,
                   const int32_t *token_lora_mapping, const moe_lora_routing *routing,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * The layer forward.  Writes `out` bf16 [T, H] (16-byte aligned; NULL when
 * inputs->expert_out is set) completely:
 * rows of tokens with no local slot are 0, so `out` needs no clearing.  With
 * several expert-parallel shards, `out` is this shard's partial sum.
 * `routing` is NULL, or receives the routing arrays as moe_lora_route
 * defines them (then all its fields are written except topk_ids /
 * topk_weights when top-k was given).  `workspace` is device memory of at
 * least moe_lora_workspace_size(shape) bytes, 256-byte aligned; its
 * contents on entry do not matter.
 */
int moe_lora_forward(const moe_lora_shape *shape, const moe_lora_inputs *inputs,
                     const moe_lora_routing *routing, void *out, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * The layer forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): moe_lora_forward with the workspace taken from a static
 * array inside the library instead of from the caller.  Arguments, outputs
 * and results are those of moe_lora_forward (same kernels, bitwise the same
 * output); the caller still passes every input and output.
 *   - The array holds MOE_LORA_STATIC_SCRATCH_BYTES bytes per GPU; a shape
 *     whose moe_lora_workspace_size exceeds that returns
 *     MOE_LORA_ERR_SCRATCH_LIMIT before any HIP call (at hidden 2048,
 *     inter 768 and rank 16 that is about 2900 slots, T * top_k).
 *   - It uses the array of the current device, which must be the device of
 *     `stream`.  The first call on a device looks up that device's copy
 *     (hipGetSymbolAddress; the library then holds it until the process
 *     ends); no call allocates or frees memory.
 *   - Every call on one GPU shares that GPU's array, whose contents the next
 *     call overwrites: calls that may overlap on one GPU (on different
 *     streams, or from several threads without ordering) race, so a caller
 *     orders them (one stream, or events).  The forward needs nothing in the
 *     array to start at zero.
 */
#define MOE_LORA_STATIC_SCRATCH_BYTES (16u << 20)

int moe_lora_forward_no_alloc(const moe_lora_shape *shape, const moe_lora_inputs *inputs,
                              const moe_lora_routing *routing, void *out, void *stream);

/*
 * The finalize on its own ("BF16 support for the experimental_sgl_trtllm
 * MoE-LoRA path", "Files changed" table, launcher row: routing-weighted sum
 * of each token's slot outputs): out[t] = routed_scaling_factor *
 * sum_j topk_weights[t, j] * expert_out[expanded_idx_to_permuted_idx[t*k+j]]
 * over the slots whose permuted index is not -1, in ascending j, fp32 sum,
 * one bf16 rounding; rows of tokens without a local slot are 0.  With the
 * arrays a moe_lora_forward call exported (expert_out set), the result is
 * bitwise the `out` that call would have written without expert_out.
 * expert_out bf16 [T*k, H] and out bf16 [T, H] 16-byte aligned, device.
 */
int moe_lora_finalize(const moe_lora_shape *shape, const void *expert_out,
                      const int32_t *expanded_idx_to_permuted_idx, const float *topk_weights,
                      void *out, void *stream);

/* Static description of a status code. */
const char *moe_lora_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H_ */
