"""Seeded synthetic inputs for the routed MoE-LoRA layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the HIP path (tests, bench) and the CPU oracle
consume exactly the arrays produced here.

Recipe (fixed draw order from one ``numpy.random.Generator(PCG64(seed))``):
router logits, hidden, W13, W2, A_gu, B_gu, A_dn, B_dn, token_lora_mapping,
hot-expert set.  Normals are drawn in fp32, scaled by sigma, then rounded to
bf16 (round-to-nearest-even); logits stay fp32.  Expert and LoRA tensors are
drawn for all ``num_experts`` global experts and the local window
``[local_expert_offset, local_expert_offset + local_num_experts)`` is sliced
out, so that several expert-parallel shards of one seed see the same weights.

Layouts (row-major, bf16 stored as uint16 bit patterns):
  hidden  [T, H]          logits [T, E] fp32
  w13     [E_l, H, 2I]    columns [0, I) = gate (w1), [I, 2I) = up (w3)
  w2      [E_l, I, H]
  a_gu    [L, E_l, r, H]  b_gu [L, E_l, 2I, r]
  a_dn    [L, E_l, r, I]  b_dn [L, E_l, H, r]
  mapping [T] int32, -1 = token uses no adapter
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    num_tokens: int            # T
    hidden: int                # H
    inter: int                 # I (gate_up width is 2I)
    num_experts: int           # E (global routed experts)
    top_k: int                 # k
    local_expert_offset: int   # off
    local_num_experts: int     # E_l
    num_loras: int             # L
    rank_gate_up: int          # r_gu
    rank_down: int             # r_dn
    seed: int
    mapping: str = "uniform"   # "uniform" over {-1..L-1}, "zero", "runs", "none"
    run_length: int = 512      # for mapping == "runs": token t uses adapter t // run_length
    hot_experts: int = 0       # number of logit columns given a bias
    hot_bias: float = 2.0
    sigma_w: float = 0.02
    sigma_lora_a: float = 0.02
    sigma_lora_b: float = 0.02
    sigma_hidden: float = 1.0
    routed_scaling_factor: float = 1.0
    # shared-outer LoRA layout: A_gu [L, 1, r, H] and B_dn [L, 1, H, r] hold one
    # weight set per adapter for every expert; B_gu and A_dn stay per expert
    lora_shared_outer: bool = False
    # routing variants: 0 = softmax renormalised over the selected experts,
    # 1 = softmax over all experts (not renormalised); a per-expert fp32 bias
    # N(0, routing_bias_sigma) steers the selection when sigma > 0
    routing_method: int = 0
    routing_bias_sigma: float = 0.0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five layer workloads.  Shapes follow the Qwen3-30B-A3B MoE layer that the
# pages measure (hidden 2048, 128 experts, top-8, expert intermediate 768).
CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny", 8, 128, 64, 8, 2, 0, 8, 2, 4, 4, seed=1,
                        mapping="uniform"),
    "decode16": LayerConfig("decode16", 16, 2048, 768, 128, 8, 0, 128, 1, 16, 16,
                            seed=2, mapping="zero"),
    "decode64": LayerConfig("decode64", 64, 2048, 768, 128, 8, 0, 128, 4, 16, 16,
                            seed=3, mapping="uniform", hot_experts=4),
    "ep_shard": LayerConfig("ep_shard", 64, 2048, 768, 128, 8, 32, 32, 4, 16, 16,
                            seed=4, mapping="uniform"),
    "prefill": LayerConfig("prefill", 2048, 2048, 768, 128, 8, 0, 128, 4, 64, 64,
                           seed=5, mapping="runs", run_length=512),
}


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x).reshape(shape)


def make_inputs(cfg: LayerConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one seeded batch for ``cfg``; returns host numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    T, H, I, E = cfg.num_tokens, cfg.hidden, cfg.inter, cfg.num_experts
    L, rg, rd = cfg.num_loras, cfg.rank_gate_up, cfg.rank_down
    lo, hi = cfg.local_expert_offset, cfg.local_expert_offset + cfg.local_num_experts
    assert 0 <= lo < hi <= E

    logits = rng.standard_normal((T, E), dtype=np.float32)
    hidden = _normal_bf16(rng, (T, H), cfg.sigma_hidden)
    w13 = _normal_bf16(rng, (E, H, 2 * I), cfg.sigma_w)[lo:hi]
    w2 = _normal_bf16(rng, (E, I, H), cfg.sigma_w)[lo:hi]
    if cfg.lora_shared_outer:  # outer matrices: one set per adapter, not sliced
        a_gu = _normal_bf16(rng, (L, 1, rg, H), cfg.sigma_lora_a)
    else:
        a_gu = _normal_bf16(rng, (L, E, rg, H), cfg.sigma_lora_a)[:, lo:hi]
    b_gu = _normal_bf16(rng, (L, E, 2 * I, rg), cfg.sigma_lora_b)[:, lo:hi]
    a_dn = _normal_bf16(rng, (L, E, rd, I), cfg.sigma_lora_a)[:, lo:hi]
    if cfg.lora_shared_outer:
        b_dn = _normal_bf16(rng, (L, 1, H, rd), cfg.sigma_lora_b)
    else:
        b_dn = _normal_bf16(rng, (L, E, H, rd), cfg.sigma_lora_b)[:, lo:hi]

    if cfg.mapping == "uniform":
        mapping = rng.integers(-1, L, size=T, dtype=np.int64).astype(np.int32)
    elif cfg.mapping == "zero":
        mapping = np.zeros(T, dtype=np.int32)
    elif cfg.mapping == "runs":
        mapping = (np.arange(T) // cfg.run_length).astype(np.int32)
        mapping = np.minimum(mapping, L - 1).astype(np.int32)
    elif cfg.mapping == "none":
        mapping = np.full(T, -1, dtype=np.int32)
    else:
        raise ValueError(f"unknown mapping kind {cfg.mapping!r}")

    if cfg.hot_experts > 0:
        hot = rng.choice(E, cfg.hot_experts, replace=False)
        logits[:, hot] += np.float32(cfg.hot_bias)
    else:
        hot = np.zeros(0, dtype=np.int64)

    extra = {}
    if cfg.routing_bias_sigma > 0:  # drawn last: earlier draws are unchanged
        extra["routing_bias"] = (rng.standard_normal(E, dtype=np.float32) *
                                 np.float32(cfg.routing_bias_sigma)).astype(np.float32)

    return {
        **extra,
        "logits": np.ascontiguousarray(logits),
        "hidden": np.ascontiguousarray(hidden),
        "w13": np.ascontiguousarray(w13),
        "w2": np.ascontiguousarray(w2),
        "a_gu": np.ascontiguousarray(a_gu),
        "b_gu": np.ascontiguousarray(b_gu),
        "a_dn": np.ascontiguousarray(a_dn),
        "b_dn": np.ascontiguousarray(b_dn),
        "mapping": np.ascontiguousarray(mapping),
        "hot_experts": np.asarray(hot, dtype=np.int64),
    }
