"""Seeded random layer shapes across the accepted limits, each against the
oracle on every output row, with the routing arrays bit-exact.

The shapes are drawn once from a fixed seed (listed by id in the test names),
so each case is reproducible; together they cross the paths the layer picks
between (few-row and many-row GEMMs and shrinks, shrink fused with the
permute or not, one or many permute slot blocks), ranks that are and are not
multiples of 8, expert-parallel windows, shared-outer stacks, both routing
methods, a routing bias, the routed scaling factor and the adapter mappings.
"""
import numpy as np
import pytest

from mixture_experts_layer_up_amd.synth import LayerConfig, make_inputs
from oracle import oracle
from tests._gpu import announce, run_forward, tol

pytestmark = pytest.mark.gpu


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    wide = i % 3 == 0                   # every third case: many rows per expert
    H = int(rng.choice([64, 128, 192, 256, 384, 512, 1024])) if not wide else \
        int(rng.choice([128, 256, 512]))
    I = int(rng.choice([32, 64, 96, 128, 160, 256])) if not wide else int(rng.choice([64, 128, 192]))
    E = int(rng.integers(1, 65))
    k = int(rng.integers(1, min(8, E) + 1))
    E_l = int(rng.integers(1, E + 1))
    off = int(rng.integers(0, E - E_l + 1))
    L = int(rng.integers(0, 6))
    def rank():
        return int(rng.choice([0, 4, 8, 12, 16, 20, 24, 32, 40, 64, 72]))
    rg, rd = rank(), rank()
    if i % 8 == 7:  # more than 16,384 slots: the permute's histogram scan
        H, I, k = 128, 64, 8
        E = max(E, 8)
        E_l = min(E_l, E)
        off = min(off, E - E_l)
        T = int(rng.integers(2100, 4000))
    elif wide:  # the many-row kernels: rows per local expert in the tens to hundreds
        T = int(rng.integers(40, 120)) * max(1, E_l // k)
        T = min(T, 1500)
        rg, rd = (rg // 8) * 8, (rd // 8) * 8
    else:
        T = int(rng.integers(1, 300))
    return LayerConfig(
        f"rand{i}", T, H, I, E, k, off, E_l, L, rg, rd, seed=2000 + i,
        mapping=str(rng.choice(["uniform", "runs", "none", "zero"])),
        run_length=int(rng.integers(1, 64)),
        sigma_lora_a=0.1, sigma_lora_b=0.1,
        routed_scaling_factor=float(rng.choice([1.0, 1.0, 0.5, 2.5])),
        lora_shared_outer=bool(rng.random() < 0.3),
        routing_method=int(rng.random() < 0.3),
        routing_bias_sigma=float(rng.choice([0.0, 0.0, 0.5])))


CASES = [_draw(i) for i in range(64)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_random_shape_matches_oracle(cfg):
    announce(f"forward {cfg}")
    inp = make_inputs(cfg)
    got, r = run_forward(cfg, inp, routing=True)
    ids, w = oracle.route(inp["logits"], cfg.top_k, bias=inp.get("routing_bias"),
                          method=cfg.routing_method)
    np.testing.assert_array_equal(r["topk_ids"], ids)
    np.testing.assert_allclose(r["topk_weights"], w, rtol=1e-5, atol=1e-7)
    perm = oracle.permute(ids, inp["mapping"], cfg.num_experts, cfg.local_expert_offset,
                          cfg.local_num_experts, cfg.num_loras)
    for name in perm:
        np.testing.assert_array_equal(r[name], perm[name], err_msg=name)
    ref = oracle.forward(cfg, inp)
    err = np.abs(got - ref).max(initial=0.0)
    assert err <= tol(ref), f"{cfg.name}: max err {err:.3e} > bound {tol(ref):.3e}"
