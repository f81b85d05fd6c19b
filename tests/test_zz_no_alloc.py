"""moe_lora_forward_no_alloc (the library's static scratch as workspace)
against moe_lora_forward (a caller-owned workspace), through the C ABI.

The two entry points run the same kernels on the same inputs, so their
outputs and routing exports are bitwise equal.  Two calls in a row share the
GPU's scratch array: the first a full 64-token decode batch, the second a
smaller batch (its first 24 tokens) that finds the first call's data still
in the array; both are checked, the second also against the CPU oracle.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_up_amd import binding
from mixture_experts_layer_up_amd.synth import CONFIGS, make_inputs
from oracle import oracle
from tests._gpu import announce, bf16_to_np, tol

pytestmark = pytest.mark.gpu


def _call(cfg, lay, no_alloc, tokens=None):
    shape = binding.make_shape(cfg)
    sel = slice(None) if tokens is None else slice(0, tokens)
    kw = dict(router_logits=lay["router_logits"][sel].contiguous(),
              token_lora_mapping=lay["token_lora_mapping"][sel].contiguous())
    for name in ("lora_a_gate_up", "lora_b_gate_up", "lora_a_down", "lora_b_down"):
        kw[name] = lay[name]
    out = torch.full((cfg.num_tokens, cfg.hidden), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    routing = binding.alloc_routing(shape, "cuda")
    binding.forward(shape, lay["hidden"][sel].contiguous(), lay["w13_packed"],
                    lay["w2_packed"], out=out, routing=routing, no_alloc=no_alloc, **kw)
    torch.cuda.synchronize()
    return bf16_to_np(out), {k: v.cpu().numpy() for k, v in routing.items()}


def test_no_alloc_equals_forward_two_calls():
    cfg = CONFIGS["decode64"]
    inp = make_inputs(cfg)
    _, lay = binding.layer_from_host(cfg, inp)
    small = cfg.replace(num_tokens=24)
    announce("no-alloc forward: decode64, then 24 tokens")
    a_full, ra_full = _call(cfg, lay, no_alloc=True)
    a_small, ra_small = _call(small, lay, no_alloc=True, tokens=24)
    announce("workspace forward: the same two calls")
    b_full, rb_full = _call(cfg, lay, no_alloc=False)
    b_small, rb_small = _call(small, lay, no_alloc=False, tokens=24)
    np.testing.assert_array_equal(a_full, b_full)
    np.testing.assert_array_equal(a_small, b_small)
    for name in ra_full:
        np.testing.assert_array_equal(ra_full[name], rb_full[name], err_msg=name)
        np.testing.assert_array_equal(ra_small[name], rb_small[name], err_msg=name)
    ref = oracle.forward(cfg, inp)
    assert np.abs(a_full - ref).max() <= tol(ref)
    sub = {k: (v[:24] if k in ("hidden", "logits", "mapping") else v) for k, v in inp.items()}
    ref_small = oracle.forward(small, sub)
    assert np.abs(a_small - ref_small).max() <= tol(ref_small)
    # a batch whose workspace exceeds the static scratch is rejected before
    # any device work
    big = cfg.replace(num_tokens=400)
    shape = binding.make_shape(big)
    assert binding.workspace_size(shape) > binding.STATIC_SCRATCH_BYTES
    announce("no-alloc forward: 400 tokens (rejected)")
    x = torch.zeros((400, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    kw = {n: lay[n] for n in ("lora_a_gate_up", "lora_b_gate_up", "lora_a_down", "lora_b_down")}
    with pytest.raises(binding.MoELoRAError, match="static scratch"):
        binding.forward(shape, x, lay["w13_packed"], lay["w2_packed"],
                        router_logits=torch.zeros((400, cfg.num_experts), device="cuda"),
                        token_lora_mapping=torch.zeros(400, dtype=torch.int32, device="cuda"),
                        out=torch.empty_like(x), no_alloc=True, **kw)
