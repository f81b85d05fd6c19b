"""Variants of the layer on the GPU against the fp64 CPU oracle.

* Shared-outer LoRA layout ("BF16 support for the experimental_sgl_trtllm
  MoE-LoRA path", Flow section 2): A_gu and B_dn hold one weight set per
  adapter for every expert.  Checked in full, on the LoRA delta alone, on an
  expert-parallel shard (the shared stacks are not sliced by the shard), and
  through both GEMM kernels (decode tiles and the many-row tiles).
* Two-stream schedule (the same page, Summary and Flow section 1(B)): the
  gate_up LoRA shrink on a second stream beside the permute, joined before
  the gate_up GEMM, for decode-shaped batches only; bitwise equal to the
  one-stream result, against the oracle, and replayed from a HIP graph.
* Routing variants (the same page names a routing bias and a routing method
  without defining them): a selection-only bias and the softmax over all
  experts, through the whole layer.
* External finalize (the same page, "Files changed" table, launcher row: the
  op can return the per-slot outputs with the routing instead of
  finalizing): the exported per-slot outputs against the oracle's, the
  separate finalize bitwise equal to the fused one, rows past the local slots
  left untouched.

Bound as in test_gpu_forward: max|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_up_amd import binding
from mixture_experts_layer_up_amd.synth import CONFIGS, make_inputs
from oracle import oracle
from tests._gpu import (SideStream, announce, bf16_to_np, cached_inputs, cached_oracle,
                        run_forward, tol)
from tests.test_gpu_forward import MID, MID_EP, SLAB_GROUPS, SPLIT_FEW, WIDE

pytestmark = pytest.mark.gpu

SHARED_MID = MID.replace(name="shared_mid", lora_shared_outer=True, seed=51)
SHARED_MID_EP = MID_EP.replace(name="shared_mid_ep", lora_shared_outer=True, seed=52)
SHARED_WIDE = WIDE.replace(name="shared_wide", lora_shared_outer=True, seed=53)
SHARED_DECODE64 = CONFIGS["decode64"].replace(name="shared_decode64", lora_shared_outer=True)


@pytest.mark.parametrize("cfg", [SHARED_MID, SHARED_MID_EP, SHARED_WIDE],
                         ids=lambda c: c.name)
def test_shared_outer_small_shapes_and_delta(cfg):
    announce(f"forward {cfg.name}")
    inp = make_inputs(cfg)
    assert inp["a_gu"].shape[1] == 1 and inp["b_dn"].shape[1] == 1
    got, _ = run_forward(cfg, inp)
    ref = oracle.forward(cfg, inp)
    err = np.abs(got - ref).max()
    assert err <= tol(ref), f"{cfg.name}: max err {err:.3e} > {tol(ref):.3e}"
    base_cfg = cfg.replace(num_loras=0)
    got_base, _ = run_forward(base_cfg, inp)
    d_ref = ref - oracle.forward(base_cfg, inp)
    d_got = got - got_base
    assert np.abs(d_ref).max() > 10 * tol(ref - d_ref)
    bound = 1e-2 * np.abs(d_ref).max() + 2 ** -7 * np.abs(ref).max()
    assert np.abs(d_got - d_ref).max() <= bound


def test_shared_outer_decode64():
    announce("forward shared_decode64")
    cfg = SHARED_DECODE64
    inp = make_inputs(cfg)
    got, _ = run_forward(cfg, inp)
    ref = oracle.forward(cfg, inp)
    assert np.abs(got - ref).max() <= tol(ref)


def test_shared_outer_equals_per_expert_with_repeated_stacks():
    # the GPU path in shared layout and in per-expert layout with the outer
    # stacks repeated over the experts compute the same products in the same
    # order: bitwise equal
    announce("forward: shared-outer vs repeated per-expert stacks")
    cfg = SHARED_MID
    inp = make_inputs(cfg)
    tiled = dict(inp)
    tiled["a_gu"] = np.ascontiguousarray(np.repeat(inp["a_gu"], cfg.local_num_experts, axis=1))
    tiled["b_dn"] = np.ascontiguousarray(np.repeat(inp["b_dn"], cfg.local_num_experts, axis=1))
    a, _ = run_forward(cfg, inp)
    b, _ = run_forward(cfg.replace(lora_shared_outer=False), tiled)
    np.testing.assert_array_equal(a, b)


def _external(cfg, inp, canary=7.0):
    """Forward with per-slot outputs exported, then the separate finalize."""
    shape, lay = binding.layer_from_host(cfg, inp)
    T, H, k = cfg.num_tokens, cfg.hidden, cfg.top_k
    kw = {n: v for n, v in lay.items() if n not in ("hidden", "w13_packed", "w2_packed")}
    routing = binding.alloc_routing(shape, "cuda")
    fused = binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"], **kw)
    torch.cuda.synchronize()
    expert_out = torch.full((T * k, H), canary, dtype=torch.bfloat16, device="cuda")
    none = binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"],
                           routing=routing, expert_out=expert_out, **kw)
    assert none is None
    torch.cuda.synchronize()
    y = expert_out.clone()
    out = binding.finalize(shape, expert_out, routing)
    torch.cuda.synchronize()
    return (bf16_to_np(fused), bf16_to_np(out), bf16_to_np(y),
            {n: v.cpu().numpy() for n, v in routing.items()})


@pytest.mark.parametrize("name", ["decode64", "ep_shard"])
def test_external_finalize(name):
    announce(f"forward: external finalize {name}")
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    fused, out, y, r = _external(cfg, inp)
    np.testing.assert_array_equal(out, fused)
    ids, w = r["topk_ids"], r["topk_weights"]
    ref_out, ref_y = oracle.forward(cfg, inp, topk_ids=ids, topk_weights=w.astype(np.float64),
                                    slot_outputs=True)
    assert np.abs(out - ref_out).max() <= tol(ref_out)
    e2p = r["expanded_idx_to_permuted_idx"]
    local = e2p >= 0
    P = int(r["expert_offsets"][-1])
    assert local.sum() == P
    got_y = y[e2p[local]]
    err = np.abs(got_y - ref_y[local]).max()
    assert err <= tol(ref_y[local]), f"slot outputs: max err {err:.3e}"
    assert np.all(y[P:] == 7.0)   # rows past the local slots are not written


def test_external_finalize_small_shapes():
    for cfg in (MID_EP, WIDE):
        announce(f"forward: external finalize {cfg.name}")
        inp = make_inputs(cfg)
        fused, out, y, r = _external(cfg, inp)
        np.testing.assert_array_equal(out, fused)
        e2p = r["expanded_idx_to_permuted_idx"]
        local = e2p >= 0
        _, ref_y = oracle.forward(cfg, inp, topk_ids=r["topk_ids"],
                                  topk_weights=r["topk_weights"].astype(np.float64),
                                  slot_outputs=True)
        assert np.abs(y[e2p[local]] - ref_y[local]).max() <= tol(ref_y[local])


# Two-stream cases: the side stream is used for decode-shaped batches (at
# most 256 tokens and 2048 slots, few rows per LoRA segment) and ignored
# otherwise.  MID: 148 slots (one-stream: the shrink in the permute's
# launch); SPLIT_FEW: 1600 slots (one-stream: a separate few-row shrink
# launch; the side stream scans 8 slots per thread); SHARED_MID_EP: the
# shared-outer stacks on a shard; MID_TOPK: top-k given (no routing
# kernel before the fork); WIDE (700 tokens) and SLAB_GROUPS (640): above the
# token gate, so the side stream is not used.
MID_TOPK = MID.replace(name="mid_topk")
# a routing bias and the softmax over all experts, with and without the side
# stream: ids and weights bitwise equal too
MID_BIAS_M1 = MID.replace(name="mid_bias_m1", routing_method=1, routing_bias_sigma=1.0)
DECODE64_BIAS = CONFIGS["decode64"].replace(name="decode64_bias", routing_bias_sigma=1.0)


@pytest.mark.parametrize("cfg", [MID, SPLIT_FEW, SHARED_MID_EP, MID_TOPK, MID_BIAS_M1,
                                 DECODE64_BIAS, WIDE, SLAB_GROUPS],
                         ids=lambda c: c.name)
def test_two_stream_bitwise_equals_one_stream(cfg):
    announce(f"forward two-stream {cfg.name}")
    inp = make_inputs(cfg)
    kw = {}
    if cfg.name == "mid_topk":
        ids, w = oracle.route(inp["logits"], cfg.top_k)
        kw = dict(use_logits=False, topk=(ids, w.astype(np.float32)))
    side = SideStream()
    try:
        layer = binding.layer_from_host(cfg, inp)
        got, r2 = run_forward(cfg, inp, layer=layer, side=side, routing=True, **kw)
        one, r1 = run_forward(cfg, inp, layer=layer, routing=True, **kw)
    finally:
        side.close()
    # the side-stream shrink computes every row as the one-stream launches do
    np.testing.assert_array_equal(got, one)
    for name in r1:
        if cfg.name != "mid_topk" or name not in ("topk_ids", "topk_weights"):
            np.testing.assert_array_equal(r2[name], r1[name], err_msg=name)
    ref = oracle.forward(cfg, inp)
    assert np.abs(got - ref).max() <= tol(ref)


@pytest.mark.parametrize("name", ["decode64", "ep_shard", "prefill"])
def test_two_stream_layer_configs(name):
    """decode64 and ep_shard take the side stream, prefill (2048 tokens)
    runs on one stream; all rows against the oracle, and bitwise against
    the one-stream forward."""
    announce(f"forward two-stream {name}")
    cfg = CONFIGS[name]
    inp = cached_inputs(name)
    layer = binding.layer_from_host(cfg, inp)
    side = SideStream()
    try:
        got, _ = run_forward(cfg, inp, layer=layer, side=side)
    finally:
        side.close()
    one, _ = run_forward(cfg, inp, layer=layer)
    np.testing.assert_array_equal(got, one)
    ref = cached_oracle(name) if name == "prefill" else oracle.forward(cfg, inp)
    assert np.abs(got - ref).max() <= tol(ref)


def test_two_stream_graph_replay():
    """The two-stream forward captured into a HIP graph (the side stream joins
    the capture through the fork event) replays bitwise equal to eager."""
    announce("forward: two-stream HIP graph replay")
    cfg = CONFIGS["decode64"]
    inp = cached_inputs("decode64")
    shape, lay = binding.layer_from_host(cfg, inp)
    ws = torch.empty(binding.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    kw = {k: v for k, v in lay.items() if k not in ("hidden", "w13_packed", "w2_packed")}
    side = SideStream()
    try:
        def step():
            binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"], out=out,
                            workspace=ws, **kw, **side.kwargs())

        step()
        torch.cuda.synchronize()
        eager = out.clone()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step()
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for i in range(3):
            out.fill_(float("nan"))
            ws.fill_(0x33)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {i} differs from eager"
            step()
            torch.cuda.synchronize()
            assert torch.equal(out, eager)
        del g
    finally:
        side.close()


@pytest.mark.parametrize("method,bias_sigma", [(0, 1.0), (1, 0.0), (1, 1.0)])
def test_routing_variants_through_the_layer(method, bias_sigma):
    cfg = CONFIGS["decode64"].replace(name=f"route_m{method}_b{bias_sigma}",
                                      routing_method=method, routing_bias_sigma=bias_sigma)
    announce(f"forward {cfg.name}")
    inp = make_inputs(cfg)
    got, r = run_forward(cfg, inp, routing=True)
    ids, w = oracle.route(inp["logits"], cfg.top_k, bias=inp.get("routing_bias"), method=method)
    np.testing.assert_array_equal(r["topk_ids"], ids)
    ref = oracle.forward(cfg, inp)
    assert np.abs(got - ref).max() <= tol(ref)
