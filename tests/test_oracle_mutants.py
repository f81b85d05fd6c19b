"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Every mutant is compiled from a text-edited copy of ``oracle/moe_lora_oracle.c``
into a temporary library (CPU only) and run through a battery of the pins from
``test_oracle_pins``: the float64 merged-weight brute force, the hand-worked
layer and the numpy permutation.  A mutant that passes the whole battery would
mean the pins are too weak.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

from mixture_experts_layer_up_amd.synth import make_inputs
from oracle import oracle
from tests import _bruteforce as bf
from tests.test_oracle_pins import (GOLDEN, MINI_C3, MINI_EP, MINI_EP_SHARED, MINI_R16,
                                    MINI_SHARED, _amplified, _golden_cfg, _golden_inputs,
                                    _numpy_permute)

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_lora_oracle.c")

# (name, text to replace, replacement, occurrence index)
MUTANTS = [
    ("gate_up_swapped", "a[i] = silu(h[i]) * h[I + i];", "a[i] = silu(h[I + i]) * h[i];", 0),
    ("silu_sign", "z / (1.0 + exp(-z))", "z / (1.0 + exp(z))", 0),
    ("gate_up_lora_dropped", "h[n] += v;", "h[n] += 0.0 * v;", 0),
    ("down_lora_dropped", "y[n] += v;", "y[n] += 0.0 * v;", 0),
    ("a_gu_transposed", "A[(size_t)q * H + c]", "A[(size_t)c * r_gu + q]", 0),
    ("b_gu_transposed", "B[(size_t)n * r_gu + q]", "B[(size_t)q * two_i + n]", 0),
    ("a_dn_transposed", "A[(size_t)q * I + i]", "A[(size_t)i * r_dn + q]", 0),
    ("b_dn_transposed", "B[(size_t)n * r_dn + q]", "B[(size_t)q * H + n]", 0),
    ("routing_weight_dropped", "acc[n] += w * y[n];", "acc[n] += y[n];", 0),
    ("gate_up_lora_weighted",
     "h[n] += v;", "h[n] += v * topk_weights[(size_t)t * k + j];", 0),
    ("down_lora_unweighted", "y[n] += v;",
     "y[n] += v / topk_weights[(size_t)t * k + j];", 0),
    ("tie_prefers_high_id", "score[e] > score[best]", "score[e] >= score[best]", 0),
    ("bias_ignored", "score[e] = bias ? row[e] + bias[e] : row[e];", "score[e] = row[e];", 0),
    ("bias_enters_weights", "ex[j] = exp((double)row[topk_ids[(size_t)t * k + j]] - m);",
     "ex[j] = exp((double)score[topk_ids[(size_t)t * k + j]] - m);", 0),
    ("method1_renormalised", "if (method == 0)\n                sum += ex[j];",
     "sum += ex[j];", 0),
    ("weights_not_normalised", "topk_weights[(size_t)t * k + j] = ex[j] / sum;",
     "topk_weights[(size_t)t * k + j] = ex[j];", 0),
    ("ep_window_off_by_one", "if (!(id >= off && id < off + E_l))",
     "if (!(id > off && id < off + E_l))", 0),
    ("adapter_of_wrong_expert", "const size_t le = (size_t)l * E_l + e;",
     "const size_t le = (size_t)l * E_l + (E_l - 1 - e);", 0),
    ("adapter_slot_zero", "int l = mapping ? mapping[t] : -1;",
     "int l = mapping ? (mapping[t] >= 0 ? 0 : -1) : -1;", 0),
    ("permute_unstable", "int p = expert_offsets[le] + seen[le];",
     "int p = expert_offsets[le + 1] - 1 - seen[le];", 0),
    ("seg_key_transposed", "int s = l * E_l + (id - off);",
     "int s = (id - off) * L + l;", 0),
    ("hidden_row_wrong", "x[c] = bf16_to_double(hidden[(size_t)t * H + c]);",
     "x[c] = bf16_to_double(hidden[(size_t)((t + 1) % T) * H + c]);", 0),
    ("shared_outer_a_first_adapter", "const size_t outer = shared_outer ? (size_t)l : le;",
     "const size_t outer = shared_outer ? (size_t)0 : le;", 0),
    ("shared_outer_b_first_adapter", "const size_t outer = shared_outer ? (size_t)l : le;",
     "const size_t outer = shared_outer ? (size_t)0 : le;", 1),
    ("slot_output_scaled", "yslot[n] = y[n];", "yslot[n] = 0.5 * y[n];", 0),
]


def _mutate(text, old, new, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


def _build_mutant(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} missing from the oracle source"
    path = tmp_path / f"{name}.c"
    path.write_text(_mutate(src, old, new, occ))
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    return str(so)


def _battery_passes() -> bool:
    """True when the currently loaded oracle passes every pin in the battery."""
    try:
        for cfg in (_amplified(MINI_C3), _amplified(MINI_EP), MINI_R16):
            inp = make_inputs(cfg)
            out = oracle.forward(cfg, inp)
            ref = bf.forward(cfg, inp)
            if not np.abs(out - ref).max() <= 1e-10 * np.abs(ref).max():
                return False
            ids, w = oracle.route(inp["logits"], cfg.top_k)
            ids_r, w_r = bf.route(inp["logits"], cfg.top_k)
            if not (np.array_equal(ids, ids_r) and np.allclose(w, w_r, rtol=1e-13, atol=0)):
                return False
            got = oracle.permute(ids, inp["mapping"], cfg.num_experts,
                                 cfg.local_expert_offset, cfg.local_num_experts, cfg.num_loras)
            m = np.where((inp["mapping"] >= 0) & (inp["mapping"] < cfg.num_loras),
                         inp["mapping"], -1)
            ref_p = _numpy_permute(ids, m, cfg.local_expert_offset, cfg.local_num_experts,
                                   cfg.num_loras)
            for a, b in zip([got[n] for n in ("expert_counts", "expert_offsets",
                                              "expanded_idx_to_permuted_idx",
                                              "permuted_idx_to_expanded_idx",
                                              "lora_seg_offsets", "lora_seg_slots")], ref_p):
                if not np.array_equal(a, b):
                    return False
        for E, k, method in ((16, 4, 0), (16, 4, 1), (40, 5, 1)):
            rng = np.random.default_rng(300 + E + method)
            lg = rng.standard_normal((9, E), dtype=np.float32)
            bias = rng.standard_normal(E, dtype=np.float32)
            ids, w = oracle.route(lg, k, bias=bias, method=method)
            ids_r, w_r = bf.route(lg, k, bias=bias, method=method)
            if not (np.array_equal(ids, ids_r) and np.allclose(w, w_r, rtol=1e-13, atol=0)):
                return False
        for cfg in (MINI_SHARED, MINI_EP_SHARED):
            inp = make_inputs(cfg)
            out = oracle.forward(cfg, inp)
            ref = bf.forward(cfg, inp)
            if not np.abs(out - ref).max() <= 1e-10 * np.abs(ref).max():
                return False
        cfg = _amplified(MINI_EP)
        inp = make_inputs(cfg)
        ids, w = bf.route(inp["logits"], cfg.top_k)
        _, y = oracle.forward(cfg, inp, topk_ids=ids, topk_weights=w, slot_outputs=True)
        y_ref = bf.slot_outputs(cfg, inp, ids)
        if not np.abs(y - y_ref).max() <= 1e-10 * np.abs(y_ref).max():
            return False
        with open(os.path.join(GOLDEN, "hand_worked_layer.json")) as f:
            g = json.load(f)
        if oracle.forward(_golden_cfg(g), _golden_inputs(g)).tolist() != \
                np.asarray(g["expected_out"], dtype=np.float64).tolist():
            return False
    except (AssertionError, RuntimeError):
        return False
    return True


def _swap_lib(path):
    saved = oracle._lib
    oracle._lib = None
    real_path = oracle._LIB_PATH
    oracle._LIB_PATH = path
    try:
        oracle._load()
    finally:
        oracle._LIB_PATH = real_path
    return saved


def test_unmutated_oracle_passes_battery():
    assert _battery_passes()


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    so = _build_mutant(tmp_path, name, old, new, occ)
    saved = _swap_lib(so)
    try:
        caught = not _battery_passes()
    finally:
        oracle._lib = saved
    assert caught, f"mutant {name} passed every pin"
