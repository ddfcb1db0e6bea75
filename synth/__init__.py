"""Seeded synthetic workloads for the routed MoE layer.

This module only draws random inputs with the shapes and distributions of the
workloads; it holds none of the layer's arithmetic (no quantiser, no packing,
no routing).  Both the tests (oracle side and library side) and ``bench.py``
draw their inputs here.

Random numbers come from ``numpy.random.default_rng`` (PCG64).  Every
generator takes an explicit seed and documents its draw order, so each side
can redraw the same values independently.

Activations, router weights and shared-expert weights are returned in the
activation dtype: ``float32`` arrays for ``act == "f32"`` and ``uint16`` arrays
of bfloat16 bit patterns for ``act == "bf16"`` (rounded to nearest-even by
torch's conversion, a library routine).
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "LayerSpec",
    "TINY",
    "FULL",
    "DEFAULT_BIAS_BETA",
    "to_bf16_bits",
    "as_act",
    "tokens",
    "correlated_tokens",
    "router",
    "shared_expert",
    "expert_weights_f32",
    "expert_codes",
    "levels_of",
]


@dataclass(frozen=True)
class LayerSpec:
    """Shape of one MoE layer."""

    hidden: int
    inter: int
    n_experts: int
    top_k: int
    has_shared: bool
    act: str                       # "f32" or "bf16"
    n_slots: Tuple[int, int, int]  # experts per tier (4-bit, 3-bit, 2-bit)
    tier_bits: Tuple[int, int, int] = (4, 3, 2)
    has_bias: bool = True
    # code width of each tier's down matrices when it differs from tier_bits
    down_bits: Optional[Tuple[int, int, int]] = None

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)


#: Tiny layer: hidden 256, 64 experts, top-4, intermediate 128, no shared
#: expert, every expert in the 4-bit tier, fp32 activations, no router bias.
TINY = LayerSpec(hidden=256, inter=128, n_experts=64, top_k=4, has_shared=False,
                 act="f32", n_slots=(64, 0, 0), has_bias=False)

#: Full-size layer: hidden 2048, 512 experts, top-10 routed + 1 shared,
#: intermediate 512, bf16 activations, tiers of 128 / 256 / 128 experts.
FULL = LayerSpec(hidden=2048, inter=512, n_experts=512, top_k=10, has_shared=True,
                 act="bf16", n_slots=(128, 256, 128))

#: Scale of the Gaussian router bias b_e = beta * z_e.  With router weights
#: N(0, 0.02^2) and N(0, 1) tokens at the full size, beta = 0.27 sends ~52%
#: of the routes of 4096 calibration tokens to the busiest quarter of experts,
#: ~95% to the busiest 80% and ~4.5% to the coldest 19%: the skew reported
#: for the average layer.  tests/test_workload.py checks it.
DEFAULT_BIAS_BETA = 0.27


#: Format code of MXFP4 tables (the C header's MOE_MXFP4).
MXFP4 = 0x14


def levels_of(bits: int) -> int:
    return 15 if bits == MXFP4 else (1 << bits) - 1


def to_bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns via torch's RNE conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def as_act(a, act: str) -> np.ndarray:
    """float32 values -> the activation dtype's storage (see module doc)."""
    a = np.asarray(a, dtype=np.float32)
    if act == "f32":
        return a
    if act == "bf16":
        return to_bf16_bits(a)
    raise ValueError(act)


def tokens(spec: LayerSpec, n: int, seed: int) -> np.ndarray:
    """``n`` token rows, iid N(0, 1), in the activation dtype.

    Draw order: one ``standard_normal((n, hidden))`` call.
    """
    rng = np.random.default_rng(seed)
    return as_act(rng.standard_normal((n, spec.hidden), dtype=np.float32), spec.act)


def correlated_tokens(spec: LayerSpec, n: int, seed: int, cosine: float = 0.6) -> np.ndarray:
    """``n`` token rows sharing a common component: x_t = sqrt(c) z_0 + sqrt(1-c) z_t.

    Pairwise cosine similarity is about ``c`` (speculative-draft verification
    batches see similar hidden states).  Draw order: z_0 ``(1, hidden)``, then
    ``(n, hidden)``.
    """
    rng = np.random.default_rng(seed)
    z0 = rng.standard_normal((1, spec.hidden), dtype=np.float32)
    zt = rng.standard_normal((n, spec.hidden), dtype=np.float32)
    x = np.float32(np.sqrt(cosine)) * z0 + np.float32(np.sqrt(1.0 - cosine)) * zt
    return as_act(x.astype(np.float32), spec.act)


def router(spec: LayerSpec, seed: int, beta: float = DEFAULT_BIAS_BETA):
    """Router weights ``E x H`` ~ N(0, 0.02^2) (activation dtype) and bias.

    The bias is ``beta * z_e`` with z_e ~ N(0, 1) (float32), or None when the
    spec has no bias.  Draw order: weights ``(E, H)``, then bias ``(E,)``.
    """
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((spec.n_experts, spec.hidden), dtype=np.float32) * np.float32(0.02)
    z = rng.standard_normal(spec.n_experts, dtype=np.float32)
    bias = (np.float32(beta) * z).astype(np.float32) if spec.has_bias else None
    return as_act(w, spec.act), bias


def shared_expert(spec: LayerSpec, seed: int):
    """Shared expert (gate ``I x H``, up ``I x H``, down ``H x I``), N(0, 1/fan_in).

    Returned in the activation dtype.  Draw order: gate, up, down.
    """
    rng = np.random.default_rng(seed)
    H, I = spec.hidden, spec.inter
    g = rng.standard_normal((I, H), dtype=np.float32) * np.float32(1 / np.sqrt(H))
    u = rng.standard_normal((I, H), dtype=np.float32) * np.float32(1 / np.sqrt(H))
    d = rng.standard_normal((H, I), dtype=np.float32) * np.float32(1 / np.sqrt(I))
    return tuple(as_act(m.astype(np.float32), spec.act) for m in (g, u, d))


def expert_weights_f32(spec: LayerSpec, seed: int, experts: Optional[Sequence[int]] = None):
    """Float32 expert weights N(0, 1/fan_in), indexed by expert id.

    Returns ``(gate [E][I][H], up [E][I][H], down [E][H][I])``.  Expert ``e``
    draws from its own stream ``default_rng([seed, e])`` in the order gate, up,
    down, so any subset can be redrawn alone.
    """
    H, I = spec.hidden, spec.inter
    ids = range(spec.n_experts) if experts is None else experts
    n = len(ids)
    gate = np.empty((n, I, H), dtype=np.float32)
    up = np.empty((n, I, H), dtype=np.float32)
    down = np.empty((n, H, I), dtype=np.float32)
    for j, e in enumerate(ids):
        rng = np.random.default_rng([seed, int(e)])
        gate[j] = rng.standard_normal((I, H), dtype=np.float32) * np.float32(1 / np.sqrt(H))
        up[j] = rng.standard_normal((I, H), dtype=np.float32) * np.float32(1 / np.sqrt(H))
        down[j] = rng.standard_normal((H, I), dtype=np.float32) * np.float32(1 / np.sqrt(I))
    return gate, up, down


def expert_codes(spec: LayerSpec, bits: int, seed: int, expert: int,
                 down_bits: Optional[int] = None):
    """Random already-quantised blocks of one expert at ``bits`` bits
    (``down_bits`` for the down matrix, when given).

    For full-size layers, where quantising 1.6 G float32 weights on the host
    would dominate the run, the blocks are drawn directly: codes uniform on
    ``0..L`` (one byte per weight), scale ``d`` such that the dequantised
    weights have standard deviation ~1/sqrt(fan_in) (times U(0.8, 1.2)), and
    min ``m = -d*L/2 + N(0, (0.05/sqrt(fan_in))^2)``; d and m are rounded to
    fp16 by NumPy.  An MXFP4 matrix draws E2M1 codes uniform on 0..15 and the
    scale byte ``127 + round(log2(sigma / 2.93)) - {0 or 1}`` (uniform E2M1
    codes have rms 2.93), returned as ``(e, None, q)`` with ``e`` uint8.

    Returns ``{"gate": (d, m, q), "up": ..., "down": ...}`` with ``q`` uint8
    ``rows x cols`` and ``d``, ``m`` float16 ``rows x cols/32``.  Stream:
    ``default_rng([seed, expert, bits])`` (``[seed, expert, bits, down_bits]``
    when down_bits is given), matrices drawn in the order gate, up, down, each
    as q then d then m (q then the scale-byte choice for MXFP4).
    """
    H, I = spec.hidden, spec.inter
    key = [seed, int(expert), int(bits)] + ([] if down_bits is None else [int(down_bits)])
    rng = np.random.default_rng(key)
    out: Dict[str, tuple] = {}
    for name, (rows, cols) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        f = down_bits if (name == "down" and down_bits is not None) else bits
        L = levels_of(f)
        sigma = 1.0 / np.sqrt(cols)
        q = rng.integers(0, L + 1, size=(rows, cols), dtype=np.uint8)
        nb = cols // 32
        if f == MXFP4:
            x0 = int(np.round(np.log2(sigma / 2.93)))
            e = (127 + x0 - rng.integers(0, 2, size=(rows, nb))).astype(np.uint8)
            out[name] = (e, None, q)
            continue
        std_q = np.sqrt(((L + 1) ** 2 - 1) / 12.0)
        d = (sigma / std_q) * rng.uniform(0.8, 1.2, size=(rows, nb))
        m = -d * (L / 2.0) + rng.normal(0.0, 0.05 * sigma, size=(rows, nb))
        out[name] = (d.astype(np.float16), m.astype(np.float16), q)
    return out
