"""The one-time packs (expert weights, LoRA A stacks) against the layouts
the header documents.

moe_lora_pack_weights writes, for expert e, 64-column slab s, K chunk c,
16-column tile t, lane l and element i, the bf16 at
(((e * NS + s) * KC + c) * 4 + t) * 512 + 8 l + i as
W[e][32 c + 8 (l // 16) + i][col(4 s + t) + l % 16], with col(n) = (n % 2) * I
+ (n // 2) * 16 for w13 (gate and up tiles alternate) and col(n) = 16 n for
w2.  The expected arrays below are that formula written with numpy index
arrays; the weights are random 16-bit patterns, so any value the pack moved
to the wrong place, or changed, shows.

moe_lora_pack_lora_a writes the bf16 A[s][q][k] of stack s (r x K) at
((s * C + k // 64) * r + q) * 64 + k % 64, C = ceil(K / 64), with zeros for
the padding past K; checked the same way.
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


def lora_a_packed_by_formula(a):
    """The documented packed order of LoRA A stacks a [L, O, r, K]: per stack,
    ceil(K / 64) chunks of the r rank rows' 64 values, zeros past K."""
    L, O, r, K = a.shape
    C = (K + 63) // 64
    padded = np.zeros((L, O, r, C * 64), a.dtype)
    padded[..., :K] = a
    l, o, c, q, u = np.meshgrid(np.arange(L), np.arange(O), np.arange(C), np.arange(r),
                                np.arange(64), indexing="ij")
    return padded[l, o, q, 64 * c + u].reshape(-1)


@pytest.mark.parametrize("H,I,L,E,rg,rd,shared", [
    (256, 96, 3, 4, 24, 12, False),   # I % 64 == 32: the down stack's last chunk is half padding
    (128, 64, 2, 3, 4, 20, False),    # ranks that are not multiples of 8
    (192, 160, 2, 5, 16, 16, True),   # shared-outer gate_up stacks: one per adapter
    (2048, 768, 4, 8, 64, 64, False)])
def test_lora_a_pack_matches_documented_layout(H, I, L, E, rg, rd, shared):
    announce(f"pack lora A H={H} I={I} L={L} E={E} r={rg}/{rd} shared={shared}")
    cfg = LayerConfig("pack_a", 1, H, I, E, 1, 0, E, L, rg, rd, seed=0, lora_shared_outer=shared)
    shape = binding.make_shape(cfg)
    rng = np.random.default_rng(70 + H + L)
    a_gu = rng.integers(-2 ** 15, 2 ** 15, size=(L, 1 if shared else E, rg, H), dtype=np.int16)
    a_dn = rng.integers(-2 ** 15, 2 ** 15, size=(L, E, rd, I), dtype=np.int16)
    d_gu = torch.from_numpy(a_gu).cuda().view(torch.bfloat16)
    d_dn = torch.from_numpy(a_dn).cuda().view(torch.bfloat16)
    p_gu, p_dn = binding.pack_lora_a(shape, d_gu, d_dn)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(p_gu.view(torch.int16).cpu().numpy().reshape(-1),
                                  lora_a_packed_by_formula(a_gu))
    np.testing.assert_array_equal(p_dn.view(torch.int16).cpu().numpy().reshape(-1),
                                  lora_a_packed_by_formula(a_dn))
    np.testing.assert_array_equal(d_gu.view(torch.int16).cpu().numpy(), a_gu)
    np.testing.assert_array_equal(d_dn.view(torch.int16).cpu().numpy(), a_dn)
