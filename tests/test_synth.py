"""The seeded input generator: deterministic, right shapes and distributions."""
import numpy as np

from mixture_experts_layer_up_amd.synth import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits,
                                                make_inputs)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 0.0, 1.0 + 2 ** -9], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    # bf16 ulp at 1.0 is 2^-7: 1 + 2^-8 is a tie and goes to the even neighbour 1.0
    np.testing.assert_array_equal(got, [1.0, 1.0, 1.0 + 2 ** -7, -2.5, 0.0, 1.0])


def test_deterministic_and_shapes():
    cfg = CONFIGS["tiny"]
    a, b = make_inputs(cfg), make_inputs(cfg)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    T, H, I, E_l, L, r = 8, 128, 64, 8, 2, 4
    assert a["hidden"].shape == (T, H) and a["hidden"].dtype == np.uint16
    assert a["logits"].shape == (T, 8) and a["logits"].dtype == np.float32
    assert a["w13"].shape == (E_l, H, 2 * I) and a["w2"].shape == (E_l, I, H)
    assert a["a_gu"].shape == (L, E_l, r, H) and a["b_gu"].shape == (L, E_l, 2 * I, r)
    assert a["a_dn"].shape == (L, E_l, r, I) and a["b_dn"].shape == (L, E_l, H, r)
    assert set(a["mapping"].tolist()) <= {-1, 0, 1}
    c = make_inputs(cfg, seed=99)
    assert not np.array_equal(a["hidden"], c["hidden"])


def test_ep_shard_is_slice_of_full():
    full = CONFIGS["ep_shard"].replace(num_tokens=4, hidden=64, inter=32,
                                       local_expert_offset=0, local_num_experts=128)
    shard = full.replace(local_expert_offset=32, local_num_experts=32)
    f, s = make_inputs(full), make_inputs(shard)
    np.testing.assert_array_equal(f["w13"][32:64], s["w13"])
    np.testing.assert_array_equal(f["b_dn"][:, 32:64], s["b_dn"])
    np.testing.assert_array_equal(f["logits"], s["logits"])


def test_hot_experts_and_runs():
    cfg = CONFIGS["decode64"].replace(hidden=64, inter=32)
    a = make_inputs(cfg)
    assert len(set(a["hot_experts"].tolist())) == 4
    p = CONFIGS["prefill"].replace(hidden=64, inter=32)
    m = make_inputs(p)["mapping"]
    np.testing.assert_array_equal(m, np.arange(2048) // 512)
