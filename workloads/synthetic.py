"""Seeded synthetic workloads.

The pages evaluate on Qwen2.5-7B (DMuon technical summary, §4 "Experimental
results"); no weights or gradients are available, so every matrix here is
drawn from a seeded generator with the shapes of that model's linear layers:
q/o 3584×3584, k/v 512×3584, gate/up 18944×3584, down 3584×18944 (stored as
PyTorch Linear weights, out × in).

Distributions (readings; the pages are silent on values):
  * NS inputs: i.i.d. N(0, 1), cast to the stated storage dtype;
  * weights: bf16 of N(0, 0.02²);
  * gradients: fp32 N(0, 0.01²);
  * momentum: zeros at the first step.

Nothing in this module computes any part of the Muon step.
"""

from __future__ import annotations

import random
from dataclasses import dataclass

import torch

__all__ = [
    "QWEN_LAYER_SHAPES", "NS_SHAPES_SMALL_MIX", "qwen_layer_shapes",
    "qwen_model_shapes", "gaussian", "ns_uniform_batch", "ns_small_mix",
    "ns_single", "MuonInputs", "muon_inputs", "shuffled_order",
]

# (name, rows, cols) of one Qwen2.5-7B decoder layer's 2-D weights.
QWEN_LAYER_SHAPES = [
    ("q", 3584, 3584),
    ("k", 512, 3584),
    ("v", 512, 3584),
    ("o", 3584, 3584),
    ("gate", 18944, 3584),
    ("up", 18944, 3584),
    ("down", 3584, 18944),
]

# Heterogeneous small-matrix batch: (count, rows, cols).
NS_SHAPES_SMALL_MIX = [(64, 256, 1024), (64, 128, 512), (32, 512, 2048), (16, 64, 4096)]


def qwen_layer_shapes():
    return [(r, c) for _, r, c in QWEN_LAYER_SHAPES]


def qwen_model_shapes(layers: int = 28):
    return [(r, c) for _ in range(layers) for (r, c) in qwen_layer_shapes()]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(shape, seed: int, std: float = 1.0, dtype=torch.float32, device="cpu"):
    """Seeded i.i.d. N(0, std²) drawn in fp32 on ``device``, cast to ``dtype``."""
    t = torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def ns_single(rows=256, cols=1024, seed=1001, dtype=torch.float32, device="cpu"):
    """One N(0,1) matrix (the small fp32 case, 256×1024, seed 1001)."""
    return gaussian((rows, cols), seed, dtype=dtype, device=device)


def ns_uniform_batch(count=32, rows=1024, cols=4096, seed0=2001,
                     dtype=torch.bfloat16, device="cpu"):
    """``count`` N(0,1) matrices of one shape, seeds seed0 + i."""
    return [gaussian((rows, cols), seed0 + i, dtype=dtype, device=device)
            for i in range(count)]


def shuffled_order(n: int, seed: int):
    order = list(range(n))
    random.Random(seed).shuffle(order)
    return order


def ns_small_mix(seed0=3001, order_seed=3000, dtype=torch.bfloat16, device="cpu",
                 tall_every_other=False, mix=None):
    """The heterogeneous small-matrix batch in shuffled descriptor order.

    ``tall_every_other`` stores every second matrix transposed (cols × rows)
    so that the orientation path is exercised.  Returns a list of tensors.
    """
    mix = NS_SHAPES_SMALL_MIX if mix is None else mix
    shapes = [(r, c) for cnt, r, c in mix for _ in range(cnt)]
    order = shuffled_order(len(shapes), order_seed)
    out = []
    for pos, idx in enumerate(order):
        r, c = shapes[idx]
        if tall_every_other and pos % 2 == 1:
            r, c = c, r
        out.append(gaussian((r, c), seed0 + idx, dtype=dtype, device=device))
    return out


@dataclass
class MuonInputs:
    params: list  # bf16 weights
    grads: list   # fp32 gradients
    momenta: list  # fp32 momentum


def muon_inputs(shapes, seed0: int, device="cpu", w_std=0.02, g_std=1e-2,
                param_dtype=torch.bfloat16, grad_seed_offset=0):
    """Weights, gradients and zero momentum for a list of (rows, cols).

    Matrix j uses seed ``seed0 + j`` for its weight and
    ``seed0 + j + 1_000_003 + grad_seed_offset`` for its gradient, so a
    second step can draw fresh gradients by changing ``grad_seed_offset``.
    """
    params, grads, momenta = [], [], []
    for j, (r, c) in enumerate(shapes):
        params.append(gaussian((r, c), seed0 + j, std=w_std, dtype=param_dtype, device=device))
        grads.append(gaussian((r, c), seed0 + j + 1_000_003 + grad_seed_offset, std=g_std,
                              device=device))
        momenta.append(torch.zeros((r, c), dtype=torch.float32, device=device))
    return MuonInputs(params, grads, momenta)


def fresh_grads(shapes, seed0: int, offset: int, device="cpu", g_std=1e-2):
    return [gaussian((r, c), seed0 + j + 1_000_003 + offset, std=g_std, device=device)
            for j, (r, c) in enumerate(shapes)]


__all__.append("fresh_grads")


def row_scales(rows: int, cols: int, seed: int, device="cpu"):
    """Distinct per-row factors 0.5 + π(i)/m along the short side (π a seeded
    permutation of 0..m−1, m = min(rows, cols)), shaped to broadcast over a
    rows × cols matrix: the selected-row step's inputs get row norms that are
    well separated (relative gaps ≥ 1/m), as real gradients' rows differ in
    size, so the selection does not hinge on rounding."""
    m = min(rows, cols)
    perm = torch.randperm(m, generator=_gen(seed, "cpu")).to(torch.float32)
    s = (0.5 + perm / m).to(device)
    return s[None, :] if rows > cols else s[:, None]


def selected_inputs(shapes, seed0: int, device="cpu", w_std=0.02, g_std=1e-2, m_std=0.0,
                    param_dtype=torch.bfloat16):
    """Inputs of the selected-row step: ``muon_inputs`` with every gradient
    (and, for ``m_std`` > 0, an N(0, m_std²) starting buffer) scaled by
    ``row_scales`` (seed ``seed0 + j + 7_000_001``)."""
    inp = muon_inputs(shapes, seed0, device=device, w_std=w_std, g_std=g_std,
                      param_dtype=param_dtype)
    for j, (r, c) in enumerate(shapes):
        if r == 0 or c == 0:
            continue
        s = row_scales(r, c, seed0 + j + 7_000_001, device=device)
        inp.grads[j].mul_(s)
        if m_std > 0:
            inp.momenta[j] = gaussian((r, c), seed0 + j + 3_000_017, std=m_std, device=device).mul_(s)
    return inp


__all__ += ["row_scales", "selected_inputs"]
