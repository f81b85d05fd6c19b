"""Independent float64 brute force used to pin the oracle on tiny inputs.

It is written differently from the oracle on purpose:
  * routing uses Python's ``sorted`` with the key (-logit, id) and
    ``scipy.special.softmax`` on the selected logits;
  * each slot's LoRA is MERGED into its expert's weights first
    (W13' = W13 + (B_gu A_gu)^T, W2' = W2 + (B_dn A_dn)^T), so the LoRA never
    appears as a separate shrink/expand;
  * the activation uses ``scipy.special.expit`` for the sigmoid;
  * products are numpy matrix products on whole rows.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit, softmax

from mixture_experts_layer_up_amd.synth import bf16_bits_to_f32


def f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def route(logits: np.ndarray, k: int, bias=None, method: int = 0):
    """Selection by (logit + bias in fp32, desc; id asc); weights from the
    logits: softmax over the selected (method 0) or over all experts taken at
    the selected ones (method 1)."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        if bias is None:
            score = row
        else:
            score = [float(np.float32(logits[t, e]) + np.float32(bias[e])) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-score[e], e))[:k]
        ids[t] = order
        if method == 0:
            w[t] = softmax(np.array([row[e] for e in order], dtype=np.float64))
        else:
            w[t] = softmax(np.array(row, dtype=np.float64))[order]
    return ids, w


def _slot_ffns(cfg, inp, topk_ids):
    """Per (token, slot): the merged-weight expert FFN output, or None for a
    slot of another shard.  Shared-outer stacks are broadcast over experts
    first, so the merged weights are formed the same way in both layouts."""
    T, H, I, k = cfg.num_tokens, cfg.hidden, cfg.inter, cfg.top_k
    off, E_l, L = cfg.local_expert_offset, cfg.local_num_experts, cfg.num_loras
    x_all = f64(inp["hidden"])
    w13, w2 = f64(inp["w13"]), f64(inp["w2"])
    has_gu = L > 0 and cfg.rank_gate_up > 0
    has_dn = L > 0 and cfg.rank_down > 0
    shared = getattr(cfg, "lora_shared_outer", False)

    def per_expert(name):
        a = f64(inp[name])
        return np.broadcast_to(a, (a.shape[0], E_l) + a.shape[2:]) if shared else a

    a_gu = per_expert("a_gu") if has_gu else None
    b_gu = f64(inp["b_gu"]) if has_gu else None
    a_dn = f64(inp["a_dn"]) if has_dn else None
    b_dn = per_expert("b_dn") if has_dn else None
    mapping = inp.get("mapping")
    res = {}
    for t in range(T):
        l = -1 if mapping is None else int(mapping[t])
        if not (0 <= l < L):
            l = -1
        for j in range(k):
            e = int(topk_ids[t, j]) - off
            if not (0 <= e < E_l):
                res[(t, j)] = None
                continue
            W13 = w13[e].copy()
            W2 = w2[e].copy()
            if l >= 0 and has_gu:
                W13 += (b_gu[l, e] @ a_gu[l, e]).T
            if l >= 0 and has_dn:
                W2 += (b_dn[l, e] @ a_dn[l, e]).T
            h = x_all[t] @ W13
            g, u = h[:I], h[I:]
            res[(t, j)] = (g * expit(g) * u) @ W2
    return res


def slot_outputs(cfg, inp, topk_ids):
    """[T * k, H]: each slot's expert output before the routing weight (zero
    rows for slots of other shards)."""
    T, H, k = cfg.num_tokens, cfg.hidden, cfg.top_k
    y = np.zeros((T * k, H), dtype=np.float64)
    for (t, j), v in _slot_ffns(cfg, inp, topk_ids).items():
        if v is not None:
            y[t * k + j] = v
    return y


def forward(cfg, inp, topk_ids=None, topk_weights=None):
    T, H, k = cfg.num_tokens, cfg.hidden, cfg.top_k
    if topk_ids is None:
        topk_ids, topk_weights = route(inp["logits"], k, bias=inp.get("routing_bias"),
                                       method=getattr(cfg, "routing_method", 0))
    out = np.zeros((T, H), dtype=np.float64)
    for (t, j), v in sorted(_slot_ffns(cfg, inp, topk_ids).items()):
        if v is not None:
            out[t] += float(topk_weights[t, j]) * v
    return out * cfg.routed_scaling_factor
