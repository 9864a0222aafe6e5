"""Host-side checks of bench.py's algorithmic byte counts (no GPU): the
figures the roofline lines divide by, at the benchmarked batch-1 shape, against
the per-tensor sums written out here."""
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from box_decoding_amd import synth  # noqa: E402


def _layer(d):
    """Weight descriptors of one bf16 layer (shapes only) and its small tensors."""
    H, F = d.hidden, d.inter
    return {
        "qkv": {"fmt": "bf16", "n": d.qkv_out, "k": H},
        "o": {"fmt": "bf16", "n": H, "k": d.n_heads * d.head_dim},
        "gate_up": {"fmt": "bf16", "n": 2 * F, "k": H},
        "down": {"fmt": "bf16", "n": H, "k": F},
        "in_norm": torch.empty(H), "post_norm": torch.empty(H), "qkv_bias": torch.empty(d.qkv_out),
    }


def test_layer_launch_bytes_b1_p1280():
    d = synth.ModelDims()
    lay, P, W, T = _layer(d), torch.tensor([1280]), 6, 6
    H, F = d.hidden, d.inter
    weights = (d.qkv_out * H + H * H + 2 * F * H + H * F) * 2
    small = (2 * H + d.qkv_out) * 2
    kv = (1280 + W) * 2 * d.n_kv_heads * d.head_dim * 2 + T * 2 * d.n_kv_heads * d.head_dim * 2
    rows = T * H * 4 + T * H * 4          # h read, h1 written
    sums = 4 * T * H * 4                  # the down projection's K-slice sums
    got = bench.fused_layer_bytes(lay, d, P, W)
    assert got == weights + small + kv + rows + sums == 155_771_904


def test_front_bytes_without_the_mlp():
    d = synth.ModelDims()
    lay, P, W, T = _layer(d), torch.tensor([1280]), 6, 6
    H, F = d.hidden, d.inter
    front = bench.front_bytes(lay, d, P, W)
    # the gate/up weights and the packed SiLU output replace the post-norm
    # operand (bf16 hi + lo) and its per-tile sums of squares
    assert bench.fused_front_bytes(lay, d, P, W) == (front - T * (H // 16) * 4 - 2 * T * H * 2
                                                     + 2 * F * H * 2 + T * F * 4)
