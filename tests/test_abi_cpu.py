"""The C ABI on a machine without a GPU: load, symbols, pure host logic.

No test here enqueues device work.  Every call below either is pure host code
(workspace sizing) or must be rejected by host-side validation before any HIP
call is made.
"""
import ctypes
import re
import os

import pytest

from mixture_experts_layer_up_amd import binding
from mixture_experts_layer_up_amd.synth import CONFIGS

ERR_INVALID_ARG, ERR_SHAPE, ERR_WS, ERR_ALIGN, ERR_SCRATCH = -1, -2, -3, -4, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mixture_experts_layer_up_amd import build
        build.build(verbose=False)
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = binding.header_functions()
    assert {"moe_lora_route", "moe_lora_forward", "moe_lora_workspace_size",
            "moe_lora_pack_weights", "moe_lora_strerror"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in moe_lora.h but not exported"


def _header_struct_fields(name):
    text = open(binding.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, re.S).group(1)
    return [re.search(r"(\w+)\s*;", d).group(1) for d in body.split(";") if d.strip()
            for d in [d + ";"]]


@pytest.mark.parametrize("cname,cls", [("moe_lora_inputs", "Inputs"),
                                        ("moe_lora_routing", "Routing")])
def test_ctypes_structs_match_header(cname, cls):
    """The binding's ctypes structs list the header's fields in the header's
    order (every field is pointer-sized)."""
    fields = _header_struct_fields(cname)
    assert fields == [n for n, _ in getattr(binding, cls)._fields_]


def test_flag_bits_match_header():
    text = open(binding.HEADER_PATH).read()
    defs = dict(re.findall(r"#define (MOE_LORA_FLAG_\w+)\s+(\d+)", text))
    assert int(defs["MOE_LORA_FLAG_EXPERT_ID"]) == binding.FLAG_EXPERT_ID
    assert int(defs["MOE_LORA_FLAG_ADAPTER"]) == binding.FLAG_ADAPTER


def test_strerror(lib):
    assert lib.moe_lora_strerror(0) == b"ok"
    for rc in (-1, -2, -3, -4, -5, -6):
        assert lib.moe_lora_strerror(rc) not in (b"ok", b"unknown status")
    assert lib.moe_lora_strerror(42) == b"unknown status"


def _ws(cfg):
    return binding.workspace_size(binding.make_shape(cfg))


def test_workspace_size_is_pure_and_monotone(lib):
    small = _ws(CONFIGS["tiny"])
    assert small > 0 and small % 256 == 0
    assert _ws(CONFIGS["tiny"]) == small
    assert _ws(CONFIGS["prefill"]) > _ws(CONFIGS["decode64"]) > _ws(CONFIGS["decode16"])
    # T * k * (H + I) bf16 rows dominate: y [T*k, H] and act [T*k, I]
    c = CONFIGS["prefill"]
    n = c.num_tokens * c.top_k
    assert _ws(c) >= n * (c.hidden + c.inter) * 2
    # no adapters -> no LoRA scratch
    assert _ws(c.replace(num_loras=0)) < _ws(c)


@pytest.mark.parametrize("field,value", [
    ("hidden", 96), ("hidden", 0), ("inter", 48), ("num_experts", 2048), ("top_k", 0),
    ("top_k", 65), ("local_num_experts", 0), ("local_expert_offset", 120),
    ("num_loras", 65), ("rank_gate_up", 300), ("num_tokens", -1)])
def test_invalid_shapes_rejected(lib, field, value):
    cfg = CONFIGS["decode64"].replace(**{field: value})
    assert _ws(cfg) == 0
    shape = binding.make_shape(cfg)
    rs = binding.Routing()
    assert lib.moe_lora_route(ctypes.byref(shape), ctypes.c_void_p(256), None, None, None,
                              None, ctypes.byref(rs), None, 0, None) == ERR_SHAPE


def _fake(addr=4096):
    return ctypes.c_void_p(addr)   # never dereferenced: validation rejects first


def _inputs(**over):
    base = dict(hidden=_fake(), router_logits=_fake(), routing_bias=None, topk_ids=None,
                topk_weights=None,
                w13_packed=_fake(), w2_packed=_fake(), lora_a_gate_up=_fake(),
                lora_b_gate_up=_fake(), lora_a_down=_fake(), lora_b_down=_fake(),
                token_lora_mapping=_fake(), stage_events=None, expert_out=None,
                side_stream=None, fork_event=None, join_event=None, input_flags=None)
    base.update(over)
    return binding.Inputs(*[base[n] for n, _ in binding.Inputs._fields_])


@pytest.mark.parametrize("over,expect", [
    (dict(hidden=None), ERR_INVALID_ARG),
    (dict(router_logits=None), ERR_INVALID_ARG),                         # no routing source
    (dict(topk_ids=_fake(), topk_weights=_fake()), ERR_INVALID_ARG),     # both sources
    (dict(router_logits=None, topk_ids=_fake()), ERR_INVALID_ARG),       # ids without weights
    (dict(lora_b_down=None), ERR_INVALID_ARG),                           # active LoRA, no stack
    (dict(w2_packed=None), ERR_INVALID_ARG),
    (dict(hidden=_fake(4096 + 8)), ERR_ALIGN),
    (dict(lora_a_gate_up=_fake(4096 + 2)), ERR_ALIGN),
    (dict(expert_out=_fake()), ERR_INVALID_ARG),                         # no routing export
    (dict(side_stream=_fake()), ERR_INVALID_ARG),                        # no fork/join events
])
def test_forward_argument_validation(lib, over, expect):
    shape = binding.make_shape(CONFIGS["decode64"])
    inp = _inputs(**over)
    ws = binding.workspace_size(shape)
    rc = lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), None, _fake(),
                              _fake(1 << 20), ws, None)
    assert rc == expect


def test_forward_workspace_checks(lib):
    shape = binding.make_shape(CONFIGS["decode64"])
    ws = binding.workspace_size(shape)
    inp = _inputs()
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), None, _fake(),
                                _fake(1 << 20), ws - 1, None) == ERR_WS
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), None, _fake(),
                                _fake((1 << 20) + 16), ws, None) == ERR_ALIGN
    assert lib.moe_lora_forward(None, ctypes.byref(inp), None, _fake(), _fake(1 << 20), ws,
                                None) == ERR_INVALID_ARG


def test_lora_pointers_optional_when_inactive(lib):
    # with no adapters the LoRA pointers may be NULL; validation must then get as far
    # as the workspace check (given a too-small workspace, so nothing is launched)
    shape = binding.make_shape(CONFIGS["decode64"].replace(num_loras=0))
    inp = _inputs(lora_a_gate_up=None, lora_b_gate_up=None, lora_a_down=None,
                  lora_b_down=None)
    ws = binding.workspace_size(shape)
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), None, _fake(),
                                _fake(1 << 20), ws - 256, None) == ERR_WS


def test_route_and_pack_validation(lib):
    shape = binding.make_shape(CONFIGS["tiny"])
    rs = binding.Routing()   # all NULL
    assert lib.moe_lora_route(ctypes.byref(shape), _fake(), None, None, None, None,
                              ctypes.byref(rs), None, 0, None) == ERR_INVALID_ARG
    assert lib.moe_lora_route(ctypes.byref(shape), None, None, None, None, None,
                              None, None, 0, None) == ERR_INVALID_ARG
    assert lib.moe_lora_pack_weights(ctypes.byref(shape), None, _fake(), _fake(), _fake(),
                                     None) == ERR_INVALID_ARG
    assert lib.moe_lora_pack_weights(ctypes.byref(shape), _fake(4097), _fake(), _fake(),
                                     _fake(), None) == ERR_ALIGN
    assert lib.moe_lora_packed_w13_bytes(ctypes.byref(shape)) == 8 * 128 * 128 * 2
    assert lib.moe_lora_packed_w2_bytes(ctypes.byref(shape)) == 8 * 64 * 128 * 2


@pytest.mark.parametrize("cfg,gu,dn", [
    # tiny: H 128, I 64, L 2, E_l 8, ranks 4: stacks of 2 and 1 chunks
    (CONFIGS["tiny"], 2 * 8 * 2 * 4 * 64 * 2, 2 * 8 * 1 * 4 * 64 * 2),
    # I 96: the down stacks' 2 chunks hold 32 values of padding
    (CONFIGS["tiny"].replace(inter=96, rank_gate_up=12, rank_down=8),
     2 * 8 * 2 * 12 * 64 * 2, 2 * 8 * 2 * 8 * 64 * 2),
    # shared-outer: one gate_up stack per adapter
    (CONFIGS["decode64"].replace(lora_shared_outer=True), 4 * 1 * 32 * 16 * 64 * 2,
     4 * 128 * 12 * 16 * 64 * 2),
    # rank 0 on down: no packed down stack
    (CONFIGS["tiny"].replace(rank_down=0), 2 * 8 * 2 * 4 * 64 * 2, 0)])
def test_packed_lora_a_bytes(lib, cfg, gu, dn):
    shape = binding.make_shape(cfg)
    assert lib.moe_lora_packed_lora_a_bytes(ctypes.byref(shape), 0) == gu
    assert lib.moe_lora_packed_lora_a_bytes(ctypes.byref(shape), 1) == dn
    assert lib.moe_lora_packed_lora_a_bytes(ctypes.byref(shape), 2) == 0
    assert lib.moe_lora_packed_lora_a_bytes(None, 0) == 0


def test_pack_lora_a_validation(lib):
    shape = binding.make_shape(CONFIGS["tiny"])
    f = _fake
    assert lib.moe_lora_pack_lora_a(ctypes.byref(shape), None, f(), f(), f(), None) == ERR_INVALID_ARG
    assert lib.moe_lora_pack_lora_a(ctypes.byref(shape), f(), f(), f(), None, None) == ERR_INVALID_ARG
    assert lib.moe_lora_pack_lora_a(ctypes.byref(shape), f(4096 + 2), f(), f(), f(),
                                    None) == ERR_ALIGN
    assert lib.moe_lora_pack_lora_a(ctypes.byref(shape), f(), f(), f(), f(4096 + 8),
                                    None) == ERR_ALIGN
    assert lib.moe_lora_pack_lora_a(None, f(), f(), f(), f(), None) == ERR_INVALID_ARG
    # no adapters: nothing to pack, every pointer may be NULL
    none = binding.make_shape(CONFIGS["tiny"].replace(num_loras=0))
    assert lib.moe_lora_pack_lora_a(ctypes.byref(none), None, None, None, None, None) == 0


def _routing_fake():
    return binding.Routing(*[_fake(8192 * (i + 1)) for i in range(len(binding.Routing._fields_))])


def test_expert_out_mode_validation(lib):
    shape = binding.make_shape(CONFIGS["decode64"])
    ws = binding.workspace_size(shape)
    rs = _routing_fake()
    # per-slot outputs instead of `out`: out may be NULL; validation then reaches
    # the workspace check (too small, so nothing is launched)
    inp = _inputs(expert_out=_fake(1 << 22))
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), ctypes.byref(rs), None,
                                _fake(1 << 20), ws - 1, None) == ERR_WS
    inp = _inputs(expert_out=_fake((1 << 22) + 8))
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), ctypes.byref(rs), None,
                                _fake(1 << 20), ws, None) == ERR_ALIGN
    # neither out nor expert_out
    inp = _inputs()
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), ctypes.byref(rs), None,
                                _fake(1 << 20), ws, None) == ERR_INVALID_ARG


def test_finalize_validation(lib):
    shape = binding.make_shape(CONFIGS["decode64"])
    assert lib.moe_lora_finalize(ctypes.byref(shape), None, _fake(), _fake(), _fake(),
                                 None) == ERR_INVALID_ARG
    assert lib.moe_lora_finalize(ctypes.byref(shape), _fake(), _fake(), _fake(), None,
                                 None) == ERR_INVALID_ARG
    assert lib.moe_lora_finalize(ctypes.byref(shape), _fake(4096 + 4), _fake(), _fake(),
                                 _fake(), None) == ERR_ALIGN
    assert lib.moe_lora_finalize(None, _fake(), _fake(), _fake(), _fake(),
                                 None) == ERR_INVALID_ARG
    empty = binding.make_shape(CONFIGS["decode64"].replace(num_tokens=0))
    assert lib.moe_lora_finalize(ctypes.byref(empty), None, None, None, None, None) == 0


def test_shared_outer_flag_validation(lib):
    cfg = CONFIGS["decode64"].replace(lora_shared_outer=True)
    shape = binding.make_shape(cfg)
    assert shape.lora_shared_outer == 1
    assert binding.workspace_size(shape) > 0
    shape.lora_shared_outer = 2
    assert binding.workspace_size(shape) == 0
    inp = _inputs()
    assert lib.moe_lora_forward(ctypes.byref(shape), ctypes.byref(inp), None, _fake(),
                                _fake(1 << 20), 1 << 30, None) == ERR_INVALID_ARG


def test_routing_method_validation(lib):
    shape = binding.make_shape(CONFIGS["decode64"].replace(routing_method=1))
    assert shape.routing_method == 1 and binding.workspace_size(shape) > 0
    shape.routing_method = 2
    assert binding.workspace_size(shape) == 0
    rs = _routing_fake()
    assert lib.moe_lora_route(ctypes.byref(shape), _fake(), None, None, None, None,
                              ctypes.byref(rs), None, 0, None) == ERR_INVALID_ARG


def test_route_workspace_size_and_validation(lib):
    """moe_lora_route needs workspace only for more than one permute block
    (1024 slots): G = ceil(T * k / 1024) histograms of E_l and L * E_l counts
    and one totals row of each, each row padded to a multiple of 4."""
    small = binding.make_shape(CONFIGS["decode64"])          # 512 slots
    assert lib.moe_lora_route_workspace_size(ctypes.byref(small)) == 0
    cfg = CONFIGS["prefill"]                                 # 16384 slots
    big = binding.make_shape(cfg)
    G = cfg.num_tokens * cfg.top_k // 1024
    E_l, L = cfg.local_num_experts, cfg.num_loras
    need = (G + 1) * (E_l + L * E_l) * 4
    assert lib.moe_lora_route_workspace_size(ctypes.byref(big)) == need
    odd = binding.make_shape(cfg.replace(local_num_experts=5, num_experts=128, num_loras=3))
    assert lib.moe_lora_route_workspace_size(ctypes.byref(odd)) == (G + 1) * (8 + 16) * 4
    # the forward workspace holds it too
    assert binding.workspace_size(big) > need
    rs = _routing_fake()
    assert lib.moe_lora_route(ctypes.byref(big), _fake(), None, None, None, None,
                              ctypes.byref(rs), None, 0, None) == ERR_INVALID_ARG
    assert lib.moe_lora_route(ctypes.byref(big), _fake(), None, None, None, None,
                              ctypes.byref(rs), _fake(1 << 20), need - 4, None) == ERR_WS
    assert lib.moe_lora_route(ctypes.byref(big), _fake(), None, None, None, None,
                              ctypes.byref(rs), _fake((1 << 20) + 4), need, None) == ERR_ALIGN
    bad = binding.make_shape(cfg.replace(top_k=0))
    assert lib.moe_lora_route_workspace_size(ctypes.byref(bad)) == 0


def test_no_alloc_forward_validation(lib):
    """moe_lora_forward_no_alloc rejects bad arguments, and shapes whose
    workspace exceeds its static scratch, before any HIP call."""
    text = open(binding.HEADER_PATH).read()
    limit = re.search(r"#define MOE_LORA_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert int(limit.group(1)) << int(limit.group(2)) == binding.STATIC_SCRATCH_BYTES
    assert int(re.search(r"#define MOE_LORA_ERR_SCRATCH_LIMIT\s+(-\d+)", text).group(1)) == ERR_SCRATCH
    inp = _inputs()
    prefill = binding.make_shape(CONFIGS["prefill"])
    assert binding.workspace_size(prefill) > binding.STATIC_SCRATCH_BYTES
    assert lib.moe_lora_forward_no_alloc(ctypes.byref(prefill), ctypes.byref(inp), None,
                                         _fake(), None) == ERR_SCRATCH
    # the largest decode batch that fits, and the first that does not
    base = CONFIGS["decode64"]
    fits = [T for T in (64, 256, 360) if
            binding.workspace_size(binding.make_shape(base.replace(num_tokens=T)))
            <= binding.STATIC_SCRATCH_BYTES]
    assert fits == [64, 256, 360]
    big = binding.make_shape(base.replace(num_tokens=400))
    assert lib.moe_lora_forward_no_alloc(ctypes.byref(big), ctypes.byref(inp), None, _fake(),
                                         None) == ERR_SCRATCH
    shape = binding.make_shape(base)
    assert lib.moe_lora_forward_no_alloc(ctypes.byref(shape), None, None, _fake(),
                                         None) == ERR_INVALID_ARG
    assert lib.moe_lora_forward_no_alloc(None, ctypes.byref(inp), None, _fake(),
                                         None) == ERR_INVALID_ARG
    for over, expect in [(dict(hidden=None), ERR_INVALID_ARG),
                         (dict(hidden=_fake(4096 + 8)), ERR_ALIGN),
                         (dict(router_logits=None), ERR_INVALID_ARG),
                         (dict(side_stream=_fake()), ERR_INVALID_ARG)]:
        bad = _inputs(**over)
        assert lib.moe_lora_forward_no_alloc(ctypes.byref(shape), ctypes.byref(bad), None,
                                             _fake(), None) == expect, over
    assert lib.moe_lora_forward_no_alloc(ctypes.byref(shape), ctypes.byref(inp), None, None,
                                         None) == ERR_INVALID_ARG     # no out
    bad_shape = binding.make_shape(base.replace(hidden=96))
    assert lib.moe_lora_forward_no_alloc(ctypes.byref(bad_shape), ctypes.byref(inp), None,
                                         _fake(), None) == ERR_SHAPE
