"""Helpers for the GPU parity tests: run the HIP path, fetch results as numpy."""
from __future__ import annotations

import ctypes
import functools
import sys

import numpy as np
import torch

from mixture_experts_layer_up_amd import binding
from mixture_experts_layer_up_amd.synth import CONFIGS, make_inputs


@functools.lru_cache(maxsize=None)
def cached_inputs(name: str):
    """Host inputs of a named layer config, generated once per test session."""
    return make_inputs(CONFIGS[name])


@functools.lru_cache(maxsize=None)
def cached_oracle(name: str):
    """The CPU oracle's output for a named layer config (all rows), computed
    once per test session."""
    from oracle import oracle
    return oracle.forward(CONFIGS[name], cached_inputs(name))


def announce(msg: str):
    """Name the case on stdout before its GPU work starts (flushed)."""
    sys.stdout.write(f"\n[gpu case] {msg}\n")
    sys.stdout.flush()


def tol(ref: np.ndarray, rel: float = 1e-2, abs_: float = 1e-3) -> float:
    """The parity bound max|gpu - oracle| <= rel * max|oracle| + abs."""
    return rel * float(np.abs(ref).max(initial=0.0)) + abs_


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


_HIP = None


def _hip():
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _HIP.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return _HIP


class SideStream:
    """A second stream (default priority) with a fork and a join event
    (timing disabled), as the two-stream schedule takes them."""

    def __init__(self):
        self.stream = torch.cuda.Stream()
        self.events = []
        for _ in range(2):
            ev = ctypes.c_void_p()
            assert _hip().hipEventCreateWithFlags(ctypes.byref(ev), 2) == 0
            self.events.append(ev.value)

    def kwargs(self):
        return {"side_stream": self.stream.cuda_stream, "fork_event": self.events[0],
                "join_event": self.events[1]}

    def close(self):
        torch.cuda.synchronize()
        for ev in self.events:
            _hip().hipEventDestroy(ctypes.c_void_p(ev))
        self.events = []


def run_forward(cfg, inputs, *, use_logits=True, topk=None, mapping="given",
                routing=False, layer=None, out=None, workspace=None, side=None,
                input_flags=None):
    """Forward through the C ABI; returns (out numpy float64, routing numpy dict | None)."""
    shape, lay = layer if layer is not None else binding.layer_from_host(cfg, inputs)
    kw = {}
    if use_logits:
        kw["router_logits"] = lay["router_logits"]
        if "routing_bias" in lay:
            kw["routing_bias"] = lay["routing_bias"]
    else:
        ids, w = topk
        kw["topk_ids"] = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
        kw["topk_weights"] = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    if isinstance(mapping, str) and mapping == "given":
        kw["token_lora_mapping"] = lay["token_lora_mapping"]
    elif mapping is not None:
        kw["token_lora_mapping"] = torch.from_numpy(np.asarray(mapping, np.int32)).cuda()
    r = binding.alloc_routing(shape, "cuda") if routing else None
    for name in ("lora_a_gate_up", "lora_b_gate_up", "lora_a_down", "lora_b_down"):
        if name in lay:
            kw[name] = lay[name]
    if side is not None:
        kw.update(side.kwargs())
    o = binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"], out=out,
                        workspace=workspace, routing=r, input_flags=input_flags, **kw)
    torch.cuda.synchronize()
    rout = None if r is None else {k: v.cpu().numpy() for k, v in r.items()}
    return bf16_to_np(o), rout
