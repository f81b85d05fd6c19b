"""ctypes binding of ``libmoe_lora.so``: argument marshalling only.

Every step of the layer runs in the HIP library; this module checks tensor
shapes / dtypes / devices, takes raw device pointers from torch tensors and
passes the current HIP stream.  torch is used for device memory and streams
only.  If the library is not built, loading fails loudly; there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_lora.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_lora.h")

_lib = None


class Shape(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("local_expert_offset", ctypes.c_int32),
        ("local_num_experts", ctypes.c_int32),
        ("num_loras", ctypes.c_int32),
        ("rank_gate_up", ctypes.c_int32),
        ("rank_down", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("lora_shared_outer", ctypes.c_int32),
        ("routing_method", ctypes.c_int32),
    ]


class Routing(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "topk_ids", "topk_weights", "expert_counts", "expert_offsets",
        "expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx",
        "lora_seg_offsets", "lora_seg_slots", "input_flags")]


class Inputs(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "hidden", "router_logits", "routing_bias", "topk_ids", "topk_weights", "w13_packed",
        "w2_packed",
        "lora_a_gate_up", "lora_b_gate_up", "lora_a_down", "lora_b_down",
        "token_lora_mapping", "stage_events", "expert_out", "side_stream", "fork_event",
        "join_event", "input_flags")]


NUM_STAGE_EVENTS = 7
STATIC_SCRATCH_BYTES = 16 << 20  # MOE_LORA_STATIC_SCRATCH_BYTES
FLAG_EXPERT_ID = 1   # a given top-k id outside [-1, num_experts)
FLAG_ADAPTER = 2     # a token_lora_mapping value outside [-1, num_loras)
STAGE_NAMES = ("route_permute", "lora_shrink_gate_up", "gemm_gate_up_swiglu",
               "lora_shrink_down", "gemm_down", "finalize")


class MoELoRAError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load the HIP library (no GPU needed to load it)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MoELoRAError(
            f"{path} is not built; run `python -m mixture_experts_layer_up_amd.build` "
            "(or __graft_entry__.build()). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.moe_lora_workspace_size.argtypes = [P(Shape)]
    lib.moe_lora_workspace_size.restype = ctypes.c_size_t
    lib.moe_lora_packed_w13_bytes.argtypes = [P(Shape)]
    lib.moe_lora_packed_w13_bytes.restype = ctypes.c_size_t
    lib.moe_lora_packed_w2_bytes.argtypes = [P(Shape)]
    lib.moe_lora_packed_w2_bytes.restype = ctypes.c_size_t
    lib.moe_lora_pack_weights.argtypes = [P(Shape), vp, vp, vp, vp, vp]
    lib.moe_lora_pack_weights.restype = ctypes.c_int
    lib.moe_lora_packed_lora_a_bytes.argtypes = [P(Shape), ctypes.c_int]
    lib.moe_lora_packed_lora_a_bytes.restype = ctypes.c_size_t
    lib.moe_lora_pack_lora_a.argtypes = [P(Shape), vp, vp, vp, vp, vp]
    lib.moe_lora_pack_lora_a.restype = ctypes.c_int
    lib.moe_lora_route_workspace_size.argtypes = [P(Shape)]
    lib.moe_lora_route_workspace_size.restype = ctypes.c_size_t
    lib.moe_lora_route.argtypes = [P(Shape), vp, vp, vp, vp, vp, P(Routing), vp,
                                   ctypes.c_size_t, vp]
    lib.moe_lora_route.restype = ctypes.c_int
    lib.moe_lora_forward.argtypes = [P(Shape), P(Inputs), P(Routing), vp, vp, ctypes.c_size_t, vp]
    lib.moe_lora_forward.restype = ctypes.c_int
    lib.moe_lora_forward_no_alloc.argtypes = [P(Shape), P(Inputs), P(Routing), vp, vp]
    lib.moe_lora_forward_no_alloc.restype = ctypes.c_int
    lib.moe_lora_finalize.argtypes = [P(Shape), vp, vp, vp, vp, vp]
    lib.moe_lora_finalize.restype = ctypes.c_int
    lib.moe_lora_strerror.argtypes = [ctypes.c_int]
    lib.moe_lora_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions the public header declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_lora_[a-z0-9_]+)\s*\(", text)))


def make_shape(cfg) -> Shape:
    return Shape(cfg.num_tokens, cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k,
                 cfg.local_expert_offset, cfg.local_num_experts, cfg.num_loras,
                 cfg.rank_gate_up, cfg.rank_down, float(cfg.routed_scaling_factor),
                 int(bool(getattr(cfg, "lora_shared_outer", False))),
                 int(getattr(cfg, "routing_method", 0)))


def _check(rc: int):
    if rc != 0:
        msg = load_library().moe_lora_strerror(rc).decode()
        raise MoELoRAError(f"moe_lora call failed ({rc}): {msg}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype=None, shape: Optional[Sequence[int]] = None,
         name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoELoRAError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MoELoRAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise MoELoRAError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoELoRAError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def workspace_size(shape: Shape) -> int:
    return int(load_library().moe_lora_workspace_size(ctypes.byref(shape)))


def pack_weights(shape: Shape, w13: torch.Tensor, w2: torch.Tensor):
    """Packed copies of w13 [E_l, H, 2I] and w2 [E_l, I, H] (bf16, device)."""
    E_l, H, I = shape.local_num_experts, shape.hidden, shape.inter
    w13p = torch.empty_like(w13)
    w2p = torch.empty_like(w2)
    _check(load_library().moe_lora_pack_weights(
        ctypes.byref(shape), _ptr(w13, _BF16, (E_l, H, 2 * I), "w13"),
        _ptr(w2, _BF16, (E_l, I, H), "w2"), w13p.data_ptr(), w2p.data_ptr(), _stream()))
    return w13p, w2p


def lora_a_shape(shape: Shape, which: int):
    """Plain shape of a LoRA A stack (which: 0 gate_up, 1 down)."""
    L, E_l = shape.num_loras, shape.local_num_experts
    if which == 0:
        return (L, 1 if shape.lora_shared_outer else E_l, shape.rank_gate_up, shape.hidden)
    return (L, E_l, shape.rank_down, shape.inter)


def packed_lora_a_shape(shape: Shape, which: int):
    """Shape of a packed LoRA A stack: [L, E_l or 1, ceil(K / 64), r, 64]."""
    L, outer, r, K = lora_a_shape(shape, which)
    return (L, outer, (K + 63) // 64, r, 64)


def pack_lora_a(shape: Shape, a_gate_up: Optional[torch.Tensor],
                a_down: Optional[torch.Tensor]):
    """Packed copies of the LoRA A stacks (bf16, device); None for an inactive
    projection."""
    lib = load_library()
    L = shape.num_loras
    gu, dn = L > 0 and shape.rank_gate_up > 0, L > 0 and shape.rank_down > 0
    out = []
    for which, a, active in ((0, a_gate_up, gu), (1, a_down, dn)):
        if not active:
            out.append(None)
            continue
        p = torch.empty(packed_lora_a_shape(shape, which), dtype=torch.bfloat16, device=a.device)
        assert p.numel() * 2 == lib.moe_lora_packed_lora_a_bytes(ctypes.byref(shape), which)
        out.append(p)
    gu_src = _ptr(a_gate_up, _BF16, lora_a_shape(shape, 0), "lora_a_gate_up") if gu else None
    dn_src = _ptr(a_down, _BF16, lora_a_shape(shape, 1), "lora_a_down") if dn else None
    _check(lib.moe_lora_pack_lora_a(
        ctypes.byref(shape), gu_src, dn_src, out[0].data_ptr() if gu else None,
        out[1].data_ptr() if dn else None, _stream()))
    return out[0], out[1]


def alloc_routing(shape: Shape, device) -> Dict[str, torch.Tensor]:
    T, k, E_l, L = shape.num_tokens, shape.top_k, shape.local_num_experts, shape.num_loras
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "topk_ids": torch.empty((T, k), **i32),
        "topk_weights": torch.empty((T, k), dtype=torch.float32, device=device),
        "expert_counts": torch.empty(E_l, **i32),
        "expert_offsets": torch.empty(E_l + 1, **i32),
        "expanded_idx_to_permuted_idx": torch.empty(T * k, **i32),
        "permuted_idx_to_expanded_idx": torch.empty(T * k, **i32),
        "lora_seg_offsets": torch.empty(L * E_l + 1, **i32),
        "lora_seg_slots": torch.empty(T * k, **i32),
    }


def _routing_struct(r: Dict[str, torch.Tensor]) -> Routing:
    return Routing(*[r[name].data_ptr() if r.get(name) is not None else None
                     for name, _ in Routing._fields_])


def route(shape: Shape, router_logits: Optional[torch.Tensor] = None,
          topk_ids: Optional[torch.Tensor] = None, topk_weights: Optional[torch.Tensor] = None,
          token_lora_mapping: Optional[torch.Tensor] = None,
          routing: Optional[Dict[str, torch.Tensor]] = None,
          routing_bias: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None,
          input_flags: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Routing and permutation only.  ``input_flags`` (int32, one element)
    receives the MOE_LORA_FLAG_* bits of bad ids / adapters met (ORed in)."""
    T, E, k = shape.num_tokens, shape.num_experts, shape.top_k
    dev = (router_logits if router_logits is not None else topk_ids).device
    r = routing if routing is not None else alloc_routing(shape, dev)
    rs = _routing_struct(r)
    if input_flags is not None:
        rs.input_flags = _ptr(input_flags, torch.int32, (1,), "input_flags")
    need = int(load_library().moe_lora_route_workspace_size(ctypes.byref(shape)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().moe_lora_route(
        ctypes.byref(shape),
        _ptr(router_logits, torch.float32, (T, E), "router_logits"),
        _ptr(routing_bias, torch.float32, (E,), "routing_bias"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(token_lora_mapping, torch.int32, (T,), "token_lora_mapping"),
        ctypes.byref(rs), ws_ptr, ws_bytes, _stream()))
    return r


def _inputs(shape: Shape, hidden, w13_packed, w2_packed, lora_a_gate_up, lora_b_gate_up,
            lora_a_down, lora_b_down, token_lora_mapping, router_logits, topk_ids, topk_weights,
            routing_bias, stage_events, expert_out, side_stream, fork_event, join_event,
            input_flags):
    """The moe_lora_inputs struct of one forward call (keeps its event array alive)."""
    T, H, I, E, k = shape.num_tokens, shape.hidden, shape.inter, shape.num_experts, shape.top_k
    E_l, L, rg, rd = shape.local_num_experts, shape.num_loras, shape.rank_gate_up, shape.rank_down
    outer = 1 if shape.lora_shared_outer else E_l
    gu = L > 0 and rg > 0
    dn = L > 0 and rd > 0
    ev = None
    if stage_events is not None:
        if len(stage_events) != NUM_STAGE_EVENTS:
            raise MoELoRAError(f"stage_events needs {NUM_STAGE_EVENTS} hipEvent_t handles")
        ev = (ctypes.c_void_p * NUM_STAGE_EVENTS)(*stage_events)
    inputs = Inputs(
        _ptr(hidden, _BF16, (T, H), "hidden"),
        _ptr(router_logits, torch.float32, (T, E), "router_logits"),
        _ptr(routing_bias, torch.float32, (E,), "routing_bias"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(w13_packed, _BF16, (E_l, H, 2 * I), "w13_packed"),
        _ptr(w2_packed, _BF16, (E_l, I, H), "w2_packed"),
        _ptr(lora_a_gate_up, _BF16, packed_lora_a_shape(shape, 0), "lora_a_gate_up (packed)")
        if gu else None,
        _ptr(lora_b_gate_up, _BF16, (L, E_l, 2 * I, rg), "lora_b_gate_up") if gu else None,
        _ptr(lora_a_down, _BF16, packed_lora_a_shape(shape, 1), "lora_a_down (packed)")
        if dn else None,
        _ptr(lora_b_down, _BF16, (L, outer, H, rd), "lora_b_down") if dn else None,
        _ptr(token_lora_mapping, torch.int32, (T,), "token_lora_mapping"),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None,
        _ptr(expert_out, _BF16, (T * k, H), "expert_out"),
        side_stream, fork_event, join_event,
        _ptr(input_flags, torch.int32, (1,), "input_flags"),
    )
    return inputs, ev


def forward(shape: Shape, hidden: torch.Tensor, w13_packed: torch.Tensor,
            w2_packed: torch.Tensor, lora_a_gate_up=None, lora_b_gate_up=None,
            lora_a_down=None, lora_b_down=None, token_lora_mapping=None,
            router_logits=None, topk_ids=None, topk_weights=None, routing_bias=None,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            routing: Optional[Dict[str, torch.Tensor]] = None,
            stage_events: Optional[Sequence[int]] = None,
            expert_out: Optional[torch.Tensor] = None,
            side_stream: Optional[int] = None, fork_event: Optional[int] = None,
            join_event: Optional[int] = None,
            input_flags: Optional[torch.Tensor] = None,
            no_alloc: bool = False) -> Optional[torch.Tensor]:
    """One layer forward on the current stream; returns ``out`` bf16 [T, H].

    ``w13_packed`` / ``w2_packed`` come from :func:`pack_weights` and
    ``lora_a_gate_up`` / ``lora_a_down`` from :func:`pack_lora_a`; the LoRA B
    stacks are passed as they are.  With ``expert_out`` (bf16 [T*k, H]) the per-slot expert outputs are
    written there at their permuted rows and the finalize is skipped (returns
    None; needs ``routing``); :func:`finalize` completes it.  ``side_stream``,
    ``fork_event``, ``join_event`` (raw hipStream_t / hipEvent_t handles)
    select the two-stream schedule for the gate_up LoRA.  ``input_flags``
    (int32, one element) receives the MOE_LORA_FLAG_* bits (ORed in).
    ``no_alloc``: call moe_lora_forward_no_alloc, whose workspace is the
    library's static per-device scratch (``workspace`` must then be None);
    ``out`` (or ``expert_out``) must then be given, since this wrapper would
    otherwise allocate it.
    """
    T, H = shape.num_tokens, shape.hidden
    if no_alloc:
        if workspace is not None:
            raise MoELoRAError("no_alloc takes no workspace")
        if out is None and expert_out is None:
            raise MoELoRAError("no_alloc needs a caller-owned out (or expert_out)")
    elif out is None and expert_out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    inputs, _ev = _inputs(shape, hidden, w13_packed, w2_packed, lora_a_gate_up, lora_b_gate_up,
                          lora_a_down, lora_b_down, token_lora_mapping, router_logits, topk_ids,
                          topk_weights, routing_bias, stage_events, expert_out, side_stream,
                          fork_event, join_event, input_flags)
    rs = _routing_struct(routing) if routing is not None else None
    lib = load_library()
    if no_alloc:
        _check(lib.moe_lora_forward_no_alloc(
            ctypes.byref(shape), ctypes.byref(inputs),
            ctypes.byref(rs) if rs is not None else None,
            _ptr(out, _BF16, (T, H), "out"), _stream()))
        return out
    if workspace is None:
        workspace = torch.empty(max(workspace_size(shape), 1), dtype=torch.uint8,
                                device=hidden.device)
    _check(lib.moe_lora_forward(
        ctypes.byref(shape), ctypes.byref(inputs), ctypes.byref(rs) if rs is not None else None,
        _ptr(out, _BF16, (T, H), "out"), _ptr(workspace, None, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream()))
    return out


def finalize(shape: Shape, expert_out: torch.Tensor, routing: Dict[str, torch.Tensor],
             topk_weights: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The routing-weighted finalize of per-slot expert outputs (as written by
    :func:`forward` with ``expert_out``); returns ``out`` bf16 [T, H].  The
    weights are ``routing['topk_weights']`` unless ``topk_weights`` is given."""
    T, H, k = shape.num_tokens, shape.hidden, shape.top_k
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=expert_out.device)
    w = topk_weights if topk_weights is not None else routing["topk_weights"]
    _check(load_library().moe_lora_finalize(
        ctypes.byref(shape), _ptr(expert_out, _BF16, (T * k, H), "expert_out"),
        _ptr(routing["expanded_idx_to_permuted_idx"], torch.int32, (T * k,),
             "expanded_idx_to_permuted_idx"),
        _ptr(w, torch.float32, (T, k), "topk_weights"),
        _ptr(out, _BF16, (T, H), "out"), _stream()))
    return out


def layer_from_host(cfg, inputs: Dict, device="cuda"):
    """Upload host arrays from the input generator and pack the expert weights
    and the LoRA A stacks.

    Returns a dict of device tensors keyed like the ``forward`` arguments.
    """
    import numpy as np

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    shape = make_shape(cfg)
    w13 = dev_bf16(inputs["w13"])
    w2 = dev_bf16(inputs["w2"])
    w13p, w2p = pack_weights(shape, w13, w2)
    del w13, w2
    L = cfg.num_loras
    layer = {
        "hidden": dev_bf16(inputs["hidden"]),
        "router_logits": torch.from_numpy(inputs["logits"]).to(device),
        "w13_packed": w13p,
        "w2_packed": w2p,
        "token_lora_mapping": torch.from_numpy(inputs["mapping"]).to(device),
    }
    if inputs.get("routing_bias") is not None:
        layer["routing_bias"] = torch.from_numpy(inputs["routing_bias"]).to(device)
    gu, dn = L > 0 and cfg.rank_gate_up > 0, L > 0 and cfg.rank_down > 0
    a_gu = dev_bf16(inputs["a_gu"]) if gu else None
    a_dn = dev_bf16(inputs["a_dn"]) if dn else None
    a_gu_p, a_dn_p = pack_lora_a(shape, a_gu, a_dn)
    del a_gu, a_dn
    if gu:
        layer["lora_a_gate_up"] = a_gu_p
        layer["lora_b_gate_up"] = dev_bf16(inputs["b_gu"])
    if dn:
        layer["lora_a_down"] = a_dn_p
        layer["lora_b_down"] = dev_bf16(inputs["b_dn"])
    return shape, layer
