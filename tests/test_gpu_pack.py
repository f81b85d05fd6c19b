"""The one-time weight pack against the layout its header documents.

moe_lora_pack_weights writes, for expert e, 64-column slab s, K chunk c,
16-column tile t, lane l and element i, the bf16 at
(((e * NS + s) * KC + c) * 4 + t) * 512 + 8 l + i as
W[e][32 c + 8 (l // 16) + i][col(4 s + t) + l % 16], with col(n) = (n % 2) * I
+ (n // 2) * 16 for w13 (gate and up tiles alternate) and col(n) = 16 n for
w2.  The expected arrays below are that formula written with numpy index
arrays; the weights are random 16-bit patterns, so any value the pack moved
to the wrong place, or changed, shows.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_up_amd import binding
from mixture_experts_layer_up_amd.synth import LayerConfig
from tests._gpu import announce

pytestmark = pytest.mark.gpu


def packed_by_formula(w, inter=None):
    """The documented packed order of w [E, K, N] (inter given: w13's tile order)."""
    E, K, N = w.shape
    NS, KC = N // 64, K // 32
    e, s, c, t, l, i = np.meshgrid(np.arange(E), np.arange(NS), np.arange(KC), np.arange(4),
                                   np.arange(64), np.arange(8), indexing="ij")
    n = 4 * s + t
    col = (n % 2) * inter + (n // 2) * 16 if inter is not None else 16 * n
    return w[e, 32 * c + 8 * (l // 16) + i, col + l % 16].reshape(-1)


@pytest.mark.parametrize("E,H,I", [(3, 256, 96), (2, 128, 64), (2, 2048, 768)])
def test_pack_matches_documented_layout(E, H, I):
    announce(f"pack E={E} H={H} I={I}")
    cfg = LayerConfig("pack", 1, H, I, E, 1, 0, E, 0, 0, 0, seed=0)
    shape = binding.make_shape(cfg)
    rng = np.random.default_rng(60 + E + H)
    w13 = rng.integers(-2 ** 15, 2 ** 15, size=(E, H, 2 * I), dtype=np.int16)
    w2 = rng.integers(-2 ** 15, 2 ** 15, size=(E, I, H), dtype=np.int16)
    d13 = torch.from_numpy(w13).cuda().view(torch.bfloat16)
    d2 = torch.from_numpy(w2).cuda().view(torch.bfloat16)
    p13, p2 = binding.pack_weights(shape, d13, d2)
    torch.cuda.synchronize()
    got13 = p13.view(torch.int16).cpu().numpy().reshape(-1)
    got2 = p2.view(torch.int16).cpu().numpy().reshape(-1)
    np.testing.assert_array_equal(got13, packed_by_formula(w13, inter=I))
    np.testing.assert_array_equal(got2, packed_by_formula(w2))
    # the inputs are left as they were
    np.testing.assert_array_equal(d13.view(torch.int16).cpu().numpy(), w13)
    np.testing.assert_array_equal(d2.view(torch.int16).cpu().numpy(), w2)
