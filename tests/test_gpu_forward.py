"""Layer forward on the GPU against the fp64 CPU oracle.

Bound: max|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3 (bf16 output, fp32
accumulation, bf16 intermediates for the LoRA shrink output, the activation
and the per-slot expert output).  Where the LoRA contribution is too small to
be seen under that bound, amplified-LoRA variants check the LoRA delta
(out - out without adapters) on its own.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_up_amd import binding
from mixture_experts_layer_up_amd.synth import CONFIGS, LayerConfig, make_inputs
from oracle import oracle
from tests._gpu import announce, cached_inputs, cached_oracle, run_forward, tol

pytestmark = pytest.mark.gpu

# Small shapes that still span several tiles and a ragged tail: 37 tokens,
# H = 320 (5 column slabs of 64 in the down GEMM), I = 96 (3 gate/up slabs,
# 3 K chunks in the down GEMM), ranks that are not multiples of 8 or 16.
MID = LayerConfig("mid", 37, 320, 96, 16, 4, 0, 16, 3, 12, 8, seed=31, mapping="uniform",
                  sigma_lora_a=0.2, sigma_lora_b=0.2)
MID_R64 = MID.replace(name="mid_r64", rank_gate_up=64, rank_down=64, seed=32,
                      sigma_lora_a=0.05, sigma_lora_b=0.05)
MID_EP = MID.replace(name="mid_ep", local_expert_offset=5, local_num_experts=7, seed=33)
# every expert gets > 64 rows, so the GEMMs take several row passes
BIG_ROWS = LayerConfig("big_rows", 300, 128, 64, 4, 1, 0, 4, 2, 16, 16, seed=34,
                       mapping="uniform", sigma_lora_a=0.2, sigma_lora_b=0.2)
TINY_AMP = CONFIGS["tiny"].replace(name="tiny_amp", sigma_lora_a=0.2, sigma_lora_b=0.2)
# Many rows per expert (the many-row GEMM and shrink kernels): ~350 rows per
# expert, so two 176-row tiles with a ragged last one, and ~117-row LoRA
# segments, so two shrink passes of 64 rows; 3 adapters of rank 24, so a K chunk
# of the LoRA expand spans two adapters and the last chunk is partial; tokens
# without adapter leave some 16-row tiles out of the expand.
WIDE = LayerConfig("wide", 700, 256, 192, 4, 2, 0, 4, 3, 24, 24, seed=35, mapping="uniform",
                   sigma_lora_a=0.1, sigma_lora_b=0.1)
# hidden 128: the down GEMM has one column slab over 12 row tiles, a work list
# whose length is not a multiple of the 8 XCDs (every item must still run)
WIDE_H128 = WIDE.replace(name="wide_h128", hidden=128)
# one rank-8 adapter (a single, mostly empty expand chunk), adapter in runs
WIDE_R8 = WIDE.replace(name="wide_r8", num_tokens=520, num_loras=1, rank_gate_up=8,
                       rank_down=8, mapping="runs", run_length=130, seed=36,
                       sigma_lora_a=0.2, sigma_lora_b=0.2)
# ~37 rows per LoRA segment (the many-row shrink) with ranks that are not
# multiples of 8 (zero-padded shrink rows; the 16-row GEMM tiles)
SHRINK_R20 = LayerConfig("shrink_r20", 300, 256, 96, 8, 2, 0, 8, 2, 20, 12, seed=37,
                         mapping="uniform", sigma_lora_a=0.2, sigma_lora_b=0.2)
# Every token carries an adapter (mapping "runs"), so the segments average
# exactly n / (L * E_l) rows: 20 (the many-row shrink with two M tiles per
# pass), 12 (the few-row shrink with two M tiles), and 25 with rank 80 (above
# the many-row kernel's limit: the few-row shrink with three M tiles and four
# rank tiles per pass).
SHRINK_MT2 = LayerConfig("shrink_mt2", 160, 256, 96, 8, 2, 0, 8, 2, 24, 16, seed=38,
                         mapping="runs", run_length=80, sigma_lora_a=0.2, sigma_lora_b=0.2)
SHRINK_FEW2 = LayerConfig("shrink_few2", 96, 256, 96, 8, 2, 0, 8, 2, 16, 16, seed=39,
                          mapping="runs", run_length=48, sigma_lora_a=0.2, sigma_lora_b=0.2)
SHRINK_FEW3 = LayerConfig("shrink_few3", 200, 256, 96, 8, 2, 0, 8, 2, 80, 72, seed=40,
                          mapping="runs", run_length=100, sigma_lora_a=0.1, sigma_lora_b=0.1)

# The gate_up shrink's three launch shapes on decode-like (few-row) segments:
# exactly 1024 slots with 128 (adapter, expert) pairs (the largest batch whose
# shrink runs inside the permute's launch: every scan lane holds a slot);
# 1600 slots (two permute slot blocks: a separate few-row shrink launch);
# 64 adapters x 17 local experts = 1088 pairs (above the fused permute's key
# tables: separate launches on a 64-slot batch).
FUSED_FULL = LayerConfig("fused_full", 128, 256, 96, 32, 8, 0, 32, 4, 16, 16, seed=41,
                         mapping="uniform", sigma_lora_a=0.2, sigma_lora_b=0.2)
SPLIT_FEW = LayerConfig("split_few", 200, 256, 96, 64, 8, 0, 64, 4, 16, 16, seed=42,
                        mapping="uniform", sigma_lora_a=0.2, sigma_lora_b=0.2)
MANY_PAIRS = LayerConfig("many_pairs", 16, 128, 64, 17, 4, 0, 17, 64, 8, 8, seed=43,
                         mapping="uniform", sigma_lora_a=0.3, sigma_lora_b=0.3)
# The fused launch's key tables at their limit: 8 adapters x 128 experts =
# 1024 (adapter, expert) pairs, and 1024 local experts with one adapter.
PAIRS_1024 = LayerConfig("pairs_1024", 16, 128, 64, 128, 8, 0, 128, 8, 8, 8, seed=47,
                         mapping="uniform", sigma_lora_a=0.3, sigma_lora_b=0.3)
EXPERTS_1024 = LayerConfig("experts_1024", 8, 128, 64, 1024, 8, 0, 1024, 1, 8, 8, seed=48,
                           mapping="zero", sigma_lora_a=0.3, sigma_lora_b=0.3)
# The many-row GEMM with several column slabs per block: 128 experts of ~40
# rows (80-row tiles, about one per expert), so each block takes 2 of the 3
# slabs of gate_up (2I = 640) and of down (H = 640): the second slab group
# has one slab, and the last slab is half outside N in both GEMMs; 3 rank-24
# adapters.
SLAB_GROUPS = LayerConfig("slab_groups", 640, 640, 320, 128, 8, 0, 128, 3, 24, 24, seed=44,
                          mapping="uniform", sigma_lora_a=0.1, sigma_lora_b=0.1)
# inter 64 (two K chunks in the down GEMM, so two of its four waves have no
# main chunk) with four rank-20 adapters (three expand chunks, 2-byte expand
# loads): those waves run expand chunks only
K64_R20 = LayerConfig("k64_r20", 37, 128, 64, 16, 4, 0, 16, 4, 20, 20, seed=49,
                      mapping="uniform", sigma_lora_a=0.2, sigma_lora_b=0.2)
# the largest accepted rank (256): 16 expand chunks per adapter in the GEMMs
# and 16 rank tiles in the few-row shrink; few rows per expert, then ~300
# (the many-row GEMM beside the few-row shrink, several row passes per
# segment; down rank 248: a last rank tile of 8)
RANK_256 = LayerConfig("rank_256", 40, 256, 128, 8, 2, 0, 8, 2, 256, 256, seed=50,
                       mapping="uniform", sigma_lora_a=0.05, sigma_lora_b=0.05)
WIDE_RANK_256 = LayerConfig("wide_rank_256", 600, 256, 128, 4, 2, 0, 4, 2, 256, 248, seed=51,
                            mapping="uniform", sigma_lora_a=0.05, sigma_lora_b=0.05)


def _compare(cfg, inp, got, tokens=None, **kw):
    ref = oracle.forward(cfg, inp, tokens=tokens, **kw)
    sel = got if tokens is None else got[tokens]
    err = np.abs(sel - ref).max(initial=0.0)
    bound = tol(ref)
    assert err <= bound, f"{cfg.name}: max err {err:.3e} > bound {bound:.3e}"
    return ref


@pytest.mark.parametrize("name", ["tiny", "decode16", "decode64", "ep_shard"])
def test_layer_configs_match_oracle(name):
    announce(f"forward {name}")
    cfg = CONFIGS[name]
    inp = cached_inputs(name)
    got, _ = run_forward(cfg, inp)
    _compare(cfg, inp, got)


def test_prefill_all_rows():
    """The T = 2048 prefill layer, every output row against the oracle."""
    announce("forward prefill (all 2048 rows)")
    cfg = CONFIGS["prefill"]
    inp = cached_inputs("prefill")
    got, r = run_forward(cfg, inp, routing=True)
    assert np.isfinite(got).all()
    ids, _ = oracle.route(inp["logits"], cfg.top_k)
    np.testing.assert_array_equal(r["topk_ids"], ids)
    ref = cached_oracle("prefill")
    err = np.abs(got - ref).max()
    assert err <= tol(ref), f"prefill: max err {err:.3e} > bound {tol(ref):.3e}"
    # every adapter run has rows far from zero (nothing came out blank)
    for a in range(4):
        assert np.abs(got[a * 512:(a + 1) * 512]).max() > 0.1 * np.abs(ref).max()


def test_prefill_bitwise_run_to_run():
    """The many-row path has no atomics and no order-dependent sums: two
    forwards of the prefill layer agree bit for bit."""
    announce("forward prefill run-to-run")
    cfg = CONFIGS["prefill"]
    inp = cached_inputs("prefill")
    layer = binding.layer_from_host(cfg, inp)
    a, ra = run_forward(cfg, inp, routing=True, layer=layer)
    b, rb = run_forward(cfg, inp, routing=True, layer=layer)
    np.testing.assert_array_equal(a, b)
    for name in ra:
        np.testing.assert_array_equal(ra[name], rb[name], err_msg=name)


def test_prefill_4096_tokens_all_rows():
    """A 4096-token prefill (32,768 slots): 207 .. 303 rows per expert, so two
    176-row tiles per expert in the many-row GEMMs (the second ragged), more
    than 16 permute slot blocks (the histogram scan), and (adapter, expert)
    segments around the many-row shrink's 64-row pass, some taking two
    passes.  Every row against the oracle."""
    cfg = CONFIGS["prefill"].replace(name="prefill4096", num_tokens=4096, run_length=1024,
                                     seed=57)
    announce("forward prefill4096 (all rows)")
    inp = make_inputs(cfg)
    got, r = run_forward(cfg, inp, routing=True)
    ids, _ = oracle.route(inp["logits"], cfg.top_k)
    np.testing.assert_array_equal(r["topk_ids"], ids)
    perm = oracle.permute(ids, inp["mapping"], 128, 0, 128, 4)
    for name in perm:
        np.testing.assert_array_equal(r[name], perm[name], err_msg=name)
    _compare(cfg, inp, got)


@pytest.mark.parametrize("cfg", [MID, MID_R64, MID_EP, BIG_ROWS, TINY_AMP, WIDE, WIDE_R8,
                                 WIDE_H128, SHRINK_R20, SHRINK_MT2, SHRINK_FEW2, SHRINK_FEW3,
                                 FUSED_FULL, SPLIT_FEW, MANY_PAIRS, SLAB_GROUPS, PAIRS_1024,
                                 EXPERTS_1024, K64_R20, RANK_256, WIDE_RANK_256],
                         ids=lambda c: c.name)
def test_small_shapes_and_lora_delta(cfg):
    announce(f"forward {cfg.name}")
    inp = make_inputs(cfg)
    got, _ = run_forward(cfg, inp)
    ref = _compare(cfg, inp, got)
    base_cfg = cfg.replace(num_loras=0)
    got_base, _ = run_forward(base_cfg, inp)
    ref_base = oracle.forward(base_cfg, inp)
    d_ref = ref - ref_base
    d_got = got - got_base
    err = np.abs(d_got - d_ref).max()
    # the delta is far above the base bound, so a wrong LoRA term cannot hide
    assert np.abs(d_ref).max() > 10 * tol(ref_base)
    # 1% of the delta, plus one bf16 rounding of each of the two outputs
    bound = 1e-2 * np.abs(d_ref).max() + 2 ** -7 * np.abs(ref).max()
    assert err <= bound, f"{cfg.name}: LoRA delta err {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("cfg", [MID, WIDE], ids=lambda c: c.name)
def test_no_adapter_paths_equal_base_bitwise(cfg):
    """Every way of giving no token an adapter (no adapters, all -1, no
    mapping, out-of-range ids, zero B, rank 0) yields the base layer bit for
    bit, on the few-row and the many-row kernels."""
    announce(f"forward: no-adapter paths {cfg.name}")
    inp = make_inputs(cfg)
    base, _ = run_forward(cfg.replace(num_loras=0), inp)
    none_mapped, _ = run_forward(cfg, inp, mapping=np.full(cfg.num_tokens, -1, np.int32))
    np.testing.assert_array_equal(none_mapped, base)
    no_mapping, _ = run_forward(cfg, inp, mapping=None)
    np.testing.assert_array_equal(no_mapping, base)
    out_of_range, _ = run_forward(cfg, inp, mapping=np.full(cfg.num_tokens, 7, np.int32))
    np.testing.assert_array_equal(out_of_range, base)
    z = dict(inp)
    z["b_gu"] = np.zeros_like(inp["b_gu"])
    z["b_dn"] = np.zeros_like(inp["b_dn"])
    zero_b, _ = run_forward(cfg, z)
    np.testing.assert_array_equal(zero_b, base)
    r0, _ = run_forward(cfg.replace(rank_gate_up=0, rank_down=0), inp)
    np.testing.assert_array_equal(r0, base)
    _compare(cfg.replace(num_loras=0), inp, base)


@pytest.mark.parametrize("cfg,hot", [
    (LayerConfig("skewed_many_rows", 300, 256, 128, 16, 2, 0, 16, 2, 16, 16, seed=54,
                 mapping="uniform", sigma_lora_a=0.05, sigma_lora_b=0.05), (3, 7)),
    (CONFIGS["decode64"].replace(name="skewed_decode64", seed=55),
     (5, 17, 33, 64, 90, 101, 120, 127))], ids=lambda v: getattr(v, "name", "hot"))
def test_all_tokens_on_few_experts(cfg, hot):
    """Every token routed to the same k experts (their logits raised by 10):
    those experts carry T rows each (several row tiles, long segments), all
    the others none (no work items at all)."""
    announce(f"forward {cfg.name}")
    inp = dict(make_inputs(cfg))
    logits = inp["logits"].copy()
    logits[:, list(hot)] += 10.0
    inp["logits"] = logits
    got, r = run_forward(cfg, inp, routing=True)
    counts = np.zeros(cfg.local_num_experts, np.int64)
    counts[list(hot)] = cfg.num_tokens
    np.testing.assert_array_equal(r["expert_counts"], counts)
    _compare(cfg, inp, got)


@pytest.mark.parametrize("cfg", [
    LayerConfig("hidden_65536", 8, 65536, 32, 2, 1, 0, 2, 1, 8, 8, seed=52, mapping="uniform",
                sigma_lora_a=0.05, sigma_lora_b=0.05),
    LayerConfig("inter_65536", 8, 64, 65536, 1, 1, 0, 1, 1, 8, 8, seed=53, mapping="uniform",
                sigma_lora_a=0.05, sigma_lora_b=0.05)], ids=lambda c: c.name)
def test_largest_hidden_and_inter(cfg):
    """The largest hidden and inter sizes the shape check accepts (65,536):
    2,048 K chunks in one GEMM, 1,024 or 2,048 column slabs in the other, 32
    column blocks in the finalize."""
    announce(f"forward {cfg.name}")
    inp = make_inputs(cfg)
    got, _ = run_forward(cfg, inp)
    _compare(cfg, inp, got)


@pytest.mark.parametrize("cfg", [
    MID.replace(name="gate_up_lora_only", rank_down=0, seed=61),
    MID.replace(name="down_lora_only", rank_gate_up=0, seed=62),
    WIDE.replace(name="wide_down_lora_only", rank_gate_up=0, seed=63),
    WIDE.replace(name="wide_gate_up_lora_only", rank_down=0, seed=64)], ids=lambda c: c.name)
def test_lora_on_one_projection_only(cfg):
    """Rank 0 on one projection and not the other: that projection takes the
    no-LoRA path (no shrink, no expand chunks) while the other keeps its
    delta, on the few-row and the many-row kernels."""
    announce(f"forward {cfg.name}")
    inp = make_inputs(cfg)
    got, _ = run_forward(cfg, inp)
    ref = _compare(cfg, inp, got)
    base = oracle.forward(cfg.replace(num_loras=0), inp)
    assert np.abs(ref - base).max() > 10 * tol(base)  # the remaining delta is visible


@pytest.mark.parametrize("cfg", [
    MID_EP,
    SPLIT_FEW.replace(name="split_few_ep", local_expert_offset=32, local_num_experts=32, seed=45),
    SLAB_GROUPS.replace(name="slab_groups_ep", local_expert_offset=64, local_num_experts=64,
                        seed=46)], ids=lambda c: c.name)
def test_no_local_slots(cfg):
    """Every slot belongs to another expert-parallel shard: no permuted row,
    no (adapter, expert) segment, no GEMM work item, and an all-zero output.
    The three cases take the permute fused with the gate_up shrink, the
    separate few-row launches, and the many-row kernels."""
    announce(f"forward: no local slots {cfg.name}")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(7)
    T, k = cfg.num_tokens, cfg.top_k
    ids = np.stack([rng.choice(cfg.local_expert_offset, k, replace=False)
                    for _ in range(T)]).astype(np.int32)
    w = np.full((T, k), 1.0 / k, np.float32)
    got, r = run_forward(cfg, inp, use_logits=False, topk=(ids, w), routing=True)
    assert np.all(got == 0)
    assert np.all(r["expert_counts"] == 0) and np.all(r["expert_offsets"] == 0)
    assert np.all(r["expanded_idx_to_permuted_idx"] == -1)
    assert np.all(r["permuted_idx_to_expanded_idx"] == -1)
    assert np.all(r["lora_seg_offsets"] == 0) and np.all(r["lora_seg_slots"] == -1)
    ref = oracle.forward(cfg, inp, topk_ids=ids, topk_weights=w.astype(np.float64))
    assert np.all(ref == 0)


def test_topk_passthrough_with_invalid_slots():
    announce("forward: top-k passthrough")
    cfg = MID
    inp = make_inputs(cfg)
    ids, w = oracle.route(inp["logits"], cfg.top_k)
    ids = ids.copy()
    ids[0, 1] = -1
    ids[3, 0] = 999
    ids[5, :] = -1          # a token with no slot at all -> zero row
    w32 = w.astype(np.float32)
    got, _ = run_forward(cfg, inp, use_logits=False, topk=(ids, w32))
    _compare(cfg, inp, got, topk_ids=ids, topk_weights=w32.astype(np.float64))
    assert np.all(got[5] == 0)


def test_input_flags_report_bad_ids_and_adapters():
    """Bad device-side values are treated as 'none' (never fault) and are
    reported in the caller's flag word, ORed in and never cleared."""
    announce("forward/route: input flags")
    cfg = MID
    inp = make_inputs(cfg)
    ids, w = oracle.route(inp["logits"], cfg.top_k)
    w32 = w.astype(np.float32)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    # clean inputs (logits and given top-k): no flag
    run_forward(cfg, inp, input_flags=flags)
    run_forward(cfg, inp, use_logits=False, topk=(ids, w32), input_flags=flags)
    assert int(flags.item()) == 0
    # -1 is the documented 'no expert' marker, not a bad id
    ids_m1 = ids.copy()
    ids_m1[2, 0] = -1
    run_forward(cfg, inp, use_logits=False, topk=(ids_m1, w32), input_flags=flags)
    assert int(flags.item()) == 0
    # ids outside [-1, E): flagged, and the result is that of 'no expert'
    bad_ids = ids.copy()
    bad_ids[0, 1] = cfg.num_experts
    bad_ids[4, 0] = -7
    got, _ = run_forward(cfg, inp, use_logits=False, topk=(bad_ids, w32), input_flags=flags)
    assert int(flags.item()) == binding.FLAG_EXPERT_ID
    as_none = bad_ids.copy()
    as_none[0, 1] = -1
    as_none[4, 0] = -1
    _compare(cfg, inp, got, topk_ids=as_none, topk_weights=w32.astype(np.float64))
    # adapters outside [-1, L): flagged (ORed onto the earlier bit); the
    # oracle counts them as -1
    inp_bad = dict(inp)
    mapping = np.asarray(inp["mapping"], np.int32).copy()
    mapping[1] = cfg.num_loras
    mapping[6] = -4
    inp_bad["mapping"] = mapping
    got, _ = run_forward(cfg, inp_bad, input_flags=flags)
    assert int(flags.item()) == binding.FLAG_EXPERT_ID | binding.FLAG_ADAPTER
    _compare(cfg, inp_bad, got)
    # routing alone reports through its own pointer
    flags.zero_()
    shape, lay = binding.layer_from_host(cfg, inp_bad)
    binding.route(shape, router_logits=lay["router_logits"],
                  token_lora_mapping=lay["token_lora_mapping"], input_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == binding.FLAG_ADAPTER


def test_expert_parallel_offsets_and_shard_sum():
    full_cfg = MID.replace(name="ep_full", num_experts=16, local_num_experts=16)
    inp_full = make_inputs(full_cfg)
    ref_full = oracle.forward(full_cfg, inp_full)
    total = np.zeros_like(ref_full)
    for off in (0, 4, 8, 12):
        announce(f"forward: EP shard off={off}")
        cfg = full_cfg.replace(local_expert_offset=off, local_num_experts=4)
        inp = make_inputs(cfg)
        got, r = run_forward(cfg, inp, routing=True)
        _compare(cfg, inp, got)
        total += got
        ids, _ = oracle.route(inp["logits"], cfg.top_k)
        perm = oracle.permute(ids, inp["mapping"], 16, off, 4, cfg.num_loras)
        for name in perm:
            np.testing.assert_array_equal(r[name], perm[name], err_msg=name)
    assert np.abs(total - ref_full).max() <= tol(ref_full, rel=2e-2)


def test_routing_export_and_determinism():
    announce("forward: routing export, determinism")
    cfg = CONFIGS["decode64"]
    inp = cached_inputs("decode64")
    layer = binding.layer_from_host(cfg, inp)
    a, ra = run_forward(cfg, inp, routing=True, layer=layer)
    b, rb = run_forward(cfg, inp, routing=True, layer=layer)
    np.testing.assert_array_equal(a, b)                    # bitwise run-to-run
    ids, w = oracle.route(inp["logits"], cfg.top_k)
    np.testing.assert_array_equal(ra["topk_ids"], ids)
    np.testing.assert_allclose(ra["topk_weights"], w, rtol=1e-6)
    perm = oracle.permute(ids, inp["mapping"], 128, 0, 128, 4)
    for name in perm:
        np.testing.assert_array_equal(ra[name], perm[name], err_msg=name)
        np.testing.assert_array_equal(rb[name], perm[name], err_msg=name)


def test_output_and_workspace_canaries():
    """Every output row is written; nothing outside out / workspace changes."""
    announce("forward: canaries")
    cfg = MID_EP
    inp = make_inputs(cfg)
    shape, layer = binding.layer_from_host(cfg, inp)
    T, H = cfg.num_tokens, cfg.hidden
    guard = 4096
    out_buf = torch.full((T * H + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = out_buf[guard:guard + T * H].view(T, H)
    ws_bytes = binding.workspace_size(shape)
    ws_buf = torch.full((ws_bytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = ws_buf[guard:guard + ws_bytes]
    assert ws.data_ptr() % 256 == 0
    got, _ = run_forward(cfg, inp, layer=(shape, layer), out=out, workspace=ws)
    assert np.isfinite(got).all()
    ob = out_buf.float().cpu().numpy()
    assert np.isnan(ob[:guard]).all() and np.isnan(ob[guard + T * H:]).all()
    wb = ws_buf.cpu().numpy()
    assert (wb[:guard] == 0x5A).all() and (wb[guard + ws_bytes:] == 0x5A).all()
    _compare(cfg, inp, got)


def test_scaling_factor_and_tiny_batches():
    for T in (1, 2, 0):
        announce(f"forward: T={T}")
        cfg = MID.replace(num_tokens=T, routed_scaling_factor=0.5, seed=40 + T)
        inp = make_inputs(cfg)
        got, _ = run_forward(cfg, inp)
        assert got.shape == (T, cfg.hidden)
        if T:
            _compare(cfg, inp, got)


def test_hip_graph_replay_matches_eager():
    """A captured forward replays bitwise equal to eager runs, replay after replay,
    with eager work and synchronisation between the replays."""
    announce("forward: HIP graph replay")
    cfg = CONFIGS["decode64"]
    inp = cached_inputs("decode64")
    shape, lay = binding.layer_from_host(cfg, inp)
    ws = torch.empty(binding.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    kw = {k: v for k, v in lay.items() if k not in ("hidden", "w13_packed", "w2_packed")}

    def step():
        binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"], out=out,
                        workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(0x33)              # the forward must not depend on workspace contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"
        step()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
