"""TEST INFRASTRUCTURE ONLY: Python access to the plain-C fp64 oracle.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It takes plain numpy arrays (bf16 as uint16 bit
patterns) and never imports the HIP library or its binding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_lora_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: -O3 for x86-64-v3 (AVX2, which every
    current x86 server host has), OpenMP.  -ffp-contract=off keeps every
    multiply and add a separately rounded IEEE double operation, as the C
    source writes them, so the results do not depend on the flags."""
    if force or not os.path.exists(_LIB_PATH):
        os.makedirs(_BUILD_DIR, exist_ok=True)
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off",
                               "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32, f64 = ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_route.argtypes = [i32, i32, i32, vp, vp, i32, vp, vp]
        lib.oracle_route.restype = i32
        lib.oracle_permute.argtypes = [i32] * 6 + [vp] * 8
        lib.oracle_permute.restype = i32
        lib.oracle_forward.argtypes = [i32] * 10 + [f64] + [vp] * 11 + [i32, vp, i32, vp]
        lib.oracle_forward.restype = i32
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the following oracle calls (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def route(logits: np.ndarray, top_k: int, bias: Optional[np.ndarray] = None, method: int = 0):
    """Top-k ids [T,k] int32 and fp64 weights [T,k] of fp32 logits [T,E].

    ``bias`` (fp32 [E]) is added to the logits for the selection only;
    ``method`` 0 renormalises the softmax over the selected experts, 1 takes
    the softmax over all experts at the selected ones."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    assert b is None or b.shape == (E,)
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    rc = _load().oracle_route(T, E, top_k, _ptr(logits), _ptr(b), int(method), _ptr(ids), _ptr(w))
    if rc != 0:
        raise RuntimeError(f"oracle_route failed ({rc})")
    return ids, w


def permute(topk_ids: np.ndarray, mapping: Optional[np.ndarray], num_experts: int,
            local_expert_offset: int, local_num_experts: int, num_loras: int) -> Dict[str, np.ndarray]:
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, k = ids.shape
    n = T * k
    E_l, L = local_num_experts, num_loras
    m = None if mapping is None else np.ascontiguousarray(mapping, dtype=np.int32)
    res = {
        "expert_counts": np.empty(E_l, np.int32),
        "expert_offsets": np.empty(E_l + 1, np.int32),
        "expanded_idx_to_permuted_idx": np.empty(n, np.int32),
        "permuted_idx_to_expanded_idx": np.empty(n, np.int32),
        "lora_seg_offsets": np.empty(L * E_l + 1, np.int32),
        "lora_seg_slots": np.empty(n, np.int32),
    }
    rc = _load().oracle_permute(T, k, num_experts, local_expert_offset, E_l, L,
                                _ptr(ids), _ptr(m),
                                _ptr(res["expert_counts"]), _ptr(res["expert_offsets"]),
                                _ptr(res["expanded_idx_to_permuted_idx"]),
                                _ptr(res["permuted_idx_to_expanded_idx"]),
                                _ptr(res["lora_seg_offsets"]), _ptr(res["lora_seg_slots"]))
    if rc != 0:
        raise RuntimeError(f"oracle_permute failed ({rc})")
    return res


def forward(cfg, inputs: Dict[str, np.ndarray], topk_ids: Optional[np.ndarray] = None,
            topk_weights: Optional[np.ndarray] = None,
            tokens: Optional[np.ndarray] = None, slot_outputs: bool = False):
    """fp64 layer output [n_out, H].

    ``cfg`` supplies the shape (``num_tokens, hidden, inter, num_experts,
    top_k, local_expert_offset, local_num_experts, num_loras, rank_gate_up,
    rank_down, routed_scaling_factor``, and ``lora_shared_outer`` for the
    shared-outer LoRA layout).  Routing comes from ``topk_ids`` /
    ``topk_weights`` when given, else from ``inputs['logits']`` via
    :func:`route`.  ``tokens`` selects output rows (default: all).  With
    ``slot_outputs`` the result is ``(out, y)``, ``y`` [T * k, H] holding each
    slot's expert output before the routing weight (zero rows for slots of
    other shards and for unselected tokens).
    """
    T, H, I = cfg.num_tokens, cfg.hidden, cfg.inter
    k = cfg.top_k
    if topk_ids is None:
        ids, w = route(inputs["logits"], k, bias=inputs.get("routing_bias"),
                       method=getattr(cfg, "routing_method", 0))
        topk_ids, topk_weights = ids, w
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float64)
    assert ids.shape == (T, k) and w.shape == (T, k)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n_out = T if tok is None else int(tok.shape[0])
    out = np.empty((n_out, H), dtype=np.float64)

    def arr(name):
        a = inputs.get(name)
        return None if a is None else np.ascontiguousarray(a)

    hidden, w13, w2 = arr("hidden"), arr("w13"), arr("w2")
    a_gu, b_gu, a_dn, b_dn = arr("a_gu"), arr("b_gu"), arr("a_dn"), arr("b_dn")
    mapping = arr("mapping")
    assert hidden.dtype == np.uint16 and w13.dtype == np.uint16 and w2.dtype == np.uint16
    E_l = cfg.local_num_experts
    assert w13.shape == (E_l, H, 2 * I) and w2.shape == (E_l, I, H)
    L, rg, rd = cfg.num_loras, cfg.rank_gate_up, cfg.rank_down
    shared = bool(getattr(cfg, "lora_shared_outer", False))
    outer = 1 if shared else E_l
    if L > 0 and rg > 0:
        assert a_gu.shape == (L, outer, rg, H) and b_gu.shape == (L, E_l, 2 * I, rg)
    if L > 0 and rd > 0:
        assert a_dn.shape == (L, E_l, rd, I) and b_dn.shape == (L, outer, H, rd)
    y = np.zeros((T * k, H), dtype=np.float64) if slot_outputs else None
    rc = _load().oracle_forward(
        T, H, I, cfg.num_experts, k, cfg.local_expert_offset, E_l, L, rg, rd,
        float(cfg.routed_scaling_factor),
        _ptr(hidden), _ptr(ids), _ptr(w), _ptr(w13), _ptr(w2),
        _ptr(a_gu), _ptr(b_gu), _ptr(a_dn), _ptr(b_dn), _ptr(mapping),
        _ptr(tok), n_out, _ptr(out), int(shared), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed ({rc})")
    return (out, y) if slot_outputs else out
