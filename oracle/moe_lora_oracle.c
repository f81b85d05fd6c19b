/*
 * moe_lora_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU definition of the bf16 routed MoE-LoRA
 * layer, used to check the HIP kernels.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * All arithmetic is IEEE double; bf16 inputs are widened exactly.  Each
 * function follows the pages' description of the layer:
 *
 *  - "BF16 support for the experimental_sgl_trtllm MoE-LoRA path" (GitHub PR
 *    page), "Files changed" table, launcher row: the pipeline is routing ->
 *    permute (bf16 gather) -> gate_up GEMM (K = hidden, N = 2 * inter) ->
 *    activation that adds the gate_up LoRA delta before SwiGLU -> down GEMM
 *    (K = inter, N = hidden) -> finalize.
 *  - same page, Flow section 2(A): the gate_up LoRA add is not multiplied by
 *    the routing weight, the down LoRA add is; LoRA weights are addressed by
 *    the virtual expert (expert id + adapter id * number of experts) and
 *    expert-parallel slots that the shard does not own are dropped to -1.
 *  - same page, Flow section 2(A): the gate_up delta has shape
 *    tokens x top_k x 2*inter, i.e. one delta per (token, choice) slot.
 *  - "sglang PR #28953 digest", change summary: permuted index -1 marks an
 *    expert-parallel slot that is not local and must never be written.
 *
 * Readings where the pages are silent (top-k tie rule, softmax
 * renormalisation, gate/up column order, LoRA stack orientation, stable
 * within-expert order) are listed in the repository's design notes; the
 * code below states each one where it is used.
 *
 * Parallelism: the forward is an OpenMP loop over tokens.  Each token's
 * result is computed by one thread in a fixed order, so the output does not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only: results do not depend on it). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Top-k routing.  For each token: the k experts with the largest selection
 * scores, ordered by (score descending, expert id ascending), where the
 * score is the fp32 logit plus, when `bias` is given, the expert's fp32
 * routing bias (one fp32 addition, the precision the kernel decides in).
 * The bias only steers the choice; the weights come from the logits:
 *   method 0: softmax over the k selected logits (softmax over all experts
 *             followed by renormalisation over the selected ones gives the
 *             same numbers);
 *   method 1: softmax over all E logits, taken at the selected experts and
 *             not renormalised.
 * Selection is a repeated linear scan: pick the best unpicked expert k times.
 */
int oracle_route(int T, int E, int k, const float *logits, const float *bias, int method,
                 int32_t *topk_ids, double *topk_weights)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E || method < 0 || method > 1)
        return -1;
    unsigned char *picked = (unsigned char *)malloc((size_t)E);
    double *ex = (double *)malloc((size_t)k * sizeof(double));
    float *score = (float *)malloc((size_t)E * sizeof(float));
    if (!picked || !ex || !score) {
        free(picked);
        free(ex);
        free(score);
        return -2;
    }
    for (int t = 0; t < T; ++t) {
        const float *row = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e)
            score[e] = bias ? row[e] + bias[e] : row[e];
        memset(picked, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (picked[e])
                    continue;
                /* strict '>' keeps the lower id on an exact tie */
                if (best < 0 || score[e] > score[best])
                    best = e;
            }
            picked[best] = 1;
            topk_ids[(size_t)t * k + j] = best;
        }
        /* the largest logit the softmax runs over, for a safe shift */
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if ((method == 1 || picked[e]) && (double)row[e] > m)
                m = (double)row[e];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            ex[j] = exp((double)row[topk_ids[(size_t)t * k + j]] - m);
            if (method == 0)
                sum += ex[j];
        }
        if (method == 1)
            for (int e = 0; e < E; ++e)
                sum += exp((double)row[e] - m);
        for (int j = 0; j < k; ++j)
            topk_weights[(size_t)t * k + j] = ex[j] / sum;
    }
    free(picked);
    free(ex);
    free(score);
    return 0;
}

/*
 * Permute.  Slot x = t*k + j is local when local_expert_offset <= id <
 * local_expert_offset + local_num_experts.  Local slots are laid out
 * expert-contiguously; inside one expert they keep ascending slot order.
 * Non-local slots get expanded_idx_to_permuted_idx = -1.  The LoRA segments
 * are the same stable grouping of the local slots whose token has an adapter,
 * keyed by (adapter, local expert) = the virtual expert; they hold slot
 * indices x.  Unused tails of permuted_idx_to_expanded_idx and
 * lora_seg_slots are -1.  A mapping value outside [-1, L) counts as -1.
 */
int oracle_permute(int T, int k, int E, int off, int E_l, int L,
                   const int32_t *topk_ids, const int32_t *mapping,
                   int32_t *expert_counts, int32_t *expert_offsets,
                   int32_t *exp2perm, int32_t *perm2exp,
                   int32_t *seg_offsets, int32_t *seg_slots)
{
    (void)E;
    const int n = T * k;
    const int nseg = L * E_l;
    int32_t *seen = (int32_t *)calloc((size_t)(E_l > nseg ? E_l : nseg) + 1, sizeof(int32_t));
    int32_t *seg_counts = (int32_t *)calloc((size_t)nseg + 1, sizeof(int32_t));
    if (!seen || !seg_counts) {
        free(seen);
        free(seg_counts);
        return -2;
    }

    for (int e = 0; e < E_l; ++e)
        expert_counts[e] = 0;
    for (int x = 0; x < n; ++x) {
        int id = topk_ids[x];
        if (id >= off && id < off + E_l)
            expert_counts[id - off] += 1;
    }
    expert_offsets[0] = 0;
    for (int e = 0; e < E_l; ++e)
        expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];
    for (int p = 0; p < n; ++p)
        perm2exp[p] = -1;
    for (int x = 0; x < n; ++x) {
        int id = topk_ids[x];
        if (id >= off && id < off + E_l) {
            int le = id - off;
            int p = expert_offsets[le] + seen[le];
            seen[le] += 1;
            exp2perm[x] = p;
            perm2exp[p] = x;
        } else {
            exp2perm[x] = -1;
        }
    }

    /* LoRA segments keyed by (adapter, local expert) */
    for (int x = 0; x < n; ++x) {
        int id = topk_ids[x];
        int l = mapping ? mapping[x / k] : -1;
        if (l < 0 || l >= L)
            continue;
        if (id >= off && id < off + E_l)
            seg_counts[l * E_l + (id - off)] += 1;
    }
    if (!seg_offsets || !seg_slots) {
        free(seen);
        free(seg_counts);
        return 0;
    }
    seg_offsets[0] = 0;
    for (int s = 0; s < nseg; ++s)
        seg_offsets[s + 1] = seg_offsets[s] + seg_counts[s];
    memset(seen, 0, ((size_t)(E_l > nseg ? E_l : nseg) + 1) * sizeof(int32_t));
    {
        for (int i = 0; i < n; ++i)
            seg_slots[i] = -1;
        for (int x = 0; x < n; ++x) {
            int id = topk_ids[x];
            int l = mapping ? mapping[x / k] : -1;
            if (l < 0 || l >= L || !(id >= off && id < off + E_l))
                continue;
            int s = l * E_l + (id - off);
            seg_slots[seg_offsets[s] + seen[s]] = x;
            seen[s] += 1;
        }
    }
    free(seen);
    free(seg_counts);
    return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * The layer, per token t (the plain definition; no grouping by expert):
 *
 *   out[t] = s * sum_{j local} w[t,j] * y_j
 *   for the slot's local expert e and the token's adapter l (l = -1: none)
 *     h   = x_t W13[e]                         W13[e] is [H, 2I]
 *     h  += B_gu[l,e] (A_gu[l,e] x_t)          if l >= 0   (not weighted)
 *     a   = SiLU(h[0:I]) * h[I:2I]             gate first, then up
 *     y   = a W2[e]                            W2[e] is [I, H]
 *     y  += B_dn[l,e] (A_dn[l,e] a)            if l >= 0   (weighted with y)
 *
 * Slots are summed in ascending j.  A token with no local slot gets a zero
 * row.  `tokens` (length n_out) selects which rows to compute; NULL means
 * all T tokens in order.  `out` is [n_out, H].
 *
 * shared_outer != 0 selects the shared-outer LoRA layout ("BF16 support for
 * the experimental_sgl_trtllm MoE-LoRA path", Flow section 2): the outer
 * matrices hold one weight set per adapter, A_gu [L, 1, r, H] and
 * B_dn [L, 1, H, r], addressed by the adapter alone for every expert; the
 * inner ones, B_gu and A_dn, stay per (adapter, expert).
 *
 * slot_out, when not NULL, receives each slot's y (before the routing weight
 * and the scaling factor) as [T * k, H] rows in slot order x = t * k + j, for
 * the selected tokens; slots of other shards get zero rows.
 */
int oracle_forward(int T, int H, int I, int E, int k, int off, int E_l,
                   int L, int r_gu, int r_dn, double routed_scaling_factor,
                   const uint16_t *hidden, const int32_t *topk_ids,
                   const double *topk_weights, const uint16_t *w13,
                   const uint16_t *w2, const uint16_t *a_gu,
                   const uint16_t *b_gu, const uint16_t *a_dn,
                   const uint16_t *b_dn, const int32_t *mapping,
                   const int32_t *tokens, int n_out, double *out,
                   int shared_outer, double *slot_out)
{
    (void)E;
    if (T < 0 || H <= 0 || I <= 0 || k <= 0 || E_l <= 0 || L < 0 || r_gu < 0 || r_dn < 0)
        return -1;
    const int two_i = 2 * I;
    int status = 0;

#pragma omp parallel
    {
        double *x = (double *)malloc((size_t)H * sizeof(double));
        double *h = (double *)malloc((size_t)two_i * sizeof(double));
        double *a = (double *)malloc((size_t)I * sizeof(double));
        double *y = (double *)malloc((size_t)H * sizeof(double));
        double *s = (double *)malloc((size_t)(r_gu > r_dn ? r_gu : r_dn) * sizeof(double) + 8);
        const int ok = x && h && a && y && s;
        if (!ok) {
#pragma omp atomic write
            status = -2;
        }
        /* every thread reaches the worksharing loop, even one whose buffers failed */
#pragma omp for schedule(dynamic, 1)
            for (int o = 0; o < n_out; ++o) {
                const int t = tokens ? tokens[o] : o;
                double *acc = out + (size_t)o * H;
                for (int n = 0; n < H; ++n)
                    acc[n] = 0.0;
                if (!ok || t < 0 || t >= T)
                    continue;
                for (int c = 0; c < H; ++c)
                    x[c] = bf16_to_double(hidden[(size_t)t * H + c]);
                int l = mapping ? mapping[t] : -1;
                if (l < 0 || l >= L)
                    l = -1;

                for (int j = 0; j < k; ++j) {
                    const int id = topk_ids[(size_t)t * k + j];
                    double *yslot = slot_out ? slot_out + ((size_t)t * k + j) * H : NULL;
                    if (yslot)
                        for (int n = 0; n < H; ++n)
                            yslot[n] = 0.0;
                    if (!(id >= off && id < off + E_l))
                        continue; /* expert-parallel slot owned by another shard */
                    const int e = id - off;

                    /* gate_up projection */
                    const uint16_t *W = w13 + (size_t)e * H * two_i;
                    for (int n = 0; n < two_i; ++n)
                        h[n] = 0.0;
                    for (int c = 0; c < H; ++c) {
                        const double xc = x[c];
                        const uint16_t *wrow = W + (size_t)c * two_i;
                        for (int n = 0; n < two_i; ++n)
                            h[n] += xc * bf16_to_double(wrow[n]);
                    }
                    /* gate_up LoRA: shrink with A_gu [r, H], expand with B_gu [2I, r] */
                    if (l >= 0 && r_gu > 0) {
                        const size_t le = (size_t)l * E_l + e;
                        const size_t outer = shared_outer ? (size_t)l : le;
                        const uint16_t *A = a_gu + outer * r_gu * H;
                        const uint16_t *B = b_gu + le * two_i * r_gu;
                        for (int q = 0; q < r_gu; ++q) {
                            double v = 0.0;
                            for (int c = 0; c < H; ++c)
                                v += bf16_to_double(A[(size_t)q * H + c]) * x[c];
                            s[q] = v;
                        }
                        for (int n = 0; n < two_i; ++n) {
                            double v = 0.0;
                            for (int q = 0; q < r_gu; ++q)
                                v += bf16_to_double(B[(size_t)n * r_gu + q]) * s[q];
                            h[n] += v;
                        }
                    }
                    /* SwiGLU: SiLU(gate) * up */
                    for (int i = 0; i < I; ++i)
                        a[i] = silu(h[i]) * h[I + i];

                    /* down projection */
                    const uint16_t *W2 = w2 + (size_t)e * I * H;
                    for (int n = 0; n < H; ++n)
                        y[n] = 0.0;
                    for (int i = 0; i < I; ++i) {
                        const double ai = a[i];
                        const uint16_t *wrow = W2 + (size_t)i * H;
                        for (int n = 0; n < H; ++n)
                            y[n] += ai * bf16_to_double(wrow[n]);
                    }
                    /* down LoRA: shrink with A_dn [r, I], expand with B_dn [H, r] */
                    if (l >= 0 && r_dn > 0) {
                        const size_t le = (size_t)l * E_l + e;
                        const size_t outer = shared_outer ? (size_t)l : le;
                        const uint16_t *A = a_dn + le * r_dn * I;
                        const uint16_t *B = b_dn + outer * (size_t)H * r_dn;
                        for (int q = 0; q < r_dn; ++q) {
                            double v = 0.0;
                            for (int i = 0; i < I; ++i)
                                v += bf16_to_double(A[(size_t)q * I + i]) * a[i];
                            s[q] = v;
                        }
                        for (int n = 0; n < H; ++n) {
                            double v = 0.0;
                            for (int q = 0; q < r_dn; ++q)
                                v += bf16_to_double(B[(size_t)n * r_dn + q]) * s[q];
                            y[n] += v;
                        }
                    }
                    if (yslot)
                        for (int n = 0; n < H; ++n)
                            yslot[n] = y[n];
                    /* finalize: routing-weighted sum over the token's slots */
                    const double w = topk_weights[(size_t)t * k + j];
                    for (int n = 0; n < H; ++n)
                        acc[n] += w * y[n];
                }
                for (int n = 0; n < H; ++n)
                    acc[n] *= routed_scaling_factor;
            }
        free(x);
        free(h);
        free(a);
        free(y);
        free(s);
    }
    return status;
}
