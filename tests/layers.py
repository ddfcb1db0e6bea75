"""Test helper: one seeded synthetic layer, seen by both sides.

``make_layer`` draws the inputs with ``synth`` and returns

* ``ol`` -- an :class:`oracle.OracleLayer` built from the drawn values and
  the oracle's own quantiser / tier build, and
* ``dl`` -- a :class:`quantized_expert_ffn_route_amd.DeviceLayer` whose
  tables the library itself built (``moe_build_tiers``) from the same values.

The oracle never sees anything the library produced.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

import oracle as O
import synth


def act_f64(a, act):
    """Exact float64 values of activation-dtype storage."""
    return O.bf16_bits_to_f64(a) if act == "bf16" else np.asarray(a, dtype=np.float64)


@dataclass
class TestLayer:
    spec: synth.LayerSpec
    ol: "O.OracleLayer"
    dl: object
    tier_map: np.ndarray
    popularity: np.ndarray


def _quantise(w, fmt):
    """The oracle's quantiser of the table format ``fmt`` (a width or MXFP4)."""
    return O.quantise_rows_mx(w) if fmt == O.MXFP4 else O.quantise_rows(w, fmt)


def popularity_from_calibration(spec, w_router, bias, seed, n=1024):
    """Route counts of ``n`` calibration tokens (oracle routing, host)."""
    xc = synth.tokens(spec, n, seed)
    keys = O.router_keys(act_f64(xc, spec.act), act_f64(w_router, spec.act), bias)
    ids = O.select_topk(keys, spec.top_k)
    return np.bincount(ids.ravel(), minlength=spec.n_experts).astype(np.uint64)


def make_layer(spec: synth.LayerSpec, seed: int = 0, source: str = "f32",
               router_override=None, device: bool = True, n_calib: int = 1024,
               host_tiers=()) -> TestLayer:
    """Build one layer for both sides.

    source="f32": fp32 weights quantised by each side's own quantiser.
    source="codes": random pre-quantised blocks (full-size layers).
    host_tiers: tiers whose library tables sit in pinned host memory.
    """
    import quantized_expert_ffn_route_amd as M

    w_router, bias = synth.router(spec, seed)
    if router_override is not None:
        w_router, bias = router_override(w_router, bias)
    pop = popularity_from_calibration(spec, w_router, bias, seed + 1, n_calib)
    shared = synth.shared_expert(spec, seed + 3) if spec.has_shared else None
    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, spec.has_shared, spec.act)
    tmap_o, _ = O.build_tiers(pop, spec.n_slots)
    bits_of = [spec.tier_bits[int(v) >> 16] for v in tmap_o]
    # the down matrices' own ladder, if any
    dbits = spec.down_bits or spec.tier_bits
    dbits_of = [dbits[int(v) >> 16] for v in tmap_o]

    if source == "f32":
        gate, up, down = synth.expert_weights_f32(spec, seed + 2)
        cache = {}

        def experts(e):
            if e not in cache:
                cache[e] = O.ExpertBlocks(bits_of[e], _quantise(gate[e], bits_of[e]),
                                          _quantise(up[e], bits_of[e]),
                                          _quantise(down[e], dbits_of[e]))
            return cache[e]
        src_arrays = (gate, up, down)
        src = M.source_f32(*src_arrays)
    else:
        per = [synth.expert_codes(spec, bits_of[e], seed + 2, e,
                                  None if spec.down_bits is None else dbits_of[e])
               for e in range(spec.n_experts)]

        def as_oracle(mat):
            d, m, q = mat
            return O.MxBlocks(d, q) if m is None else mat

        def experts(e):
            p = per[e]
            return O.ExpertBlocks(bits_of[e], *[as_oracle(p[n]) for n in ("gate", "up", "down")])

        def scale_word(mat):
            # the library's code source: fp16 bits of d, or the E8M0 byte
            d, m, q = mat
            return d.astype(np.uint16) if m is None else d.view(np.uint16)

        def min_word(mat, shape):
            d, m, q = mat
            return np.zeros(shape, np.float16) if m is None else m
        names = ("gate", "up", "down")
        q = [np.ascontiguousarray(np.stack([per[e][n][2] for e in range(spec.n_experts)])) for n in names]
        dd = [np.ascontiguousarray(np.stack([scale_word(per[e][n]) for e in range(spec.n_experts)]))
              for n in names]
        mm = [np.ascontiguousarray(np.stack([min_word(per[e][n], per[e][n][0].shape)
                                             for e in range(spec.n_experts)])) for n in names]
        src_arrays = (q, dd, mm)
        src = M.source_codes(q, dd, mm)

    ol = O.OracleLayer(act=spec.act, w_router=act_f64(w_router, spec.act), bias=bias,
                       top_k=spec.top_k, experts=experts,
                       shared=None if shared is None else tuple(act_f64(s, spec.act) for s in shared))
    dl = None
    tmap = tmap_o
    if device:
        dl = M.DeviceLayer(d, spec.n_slots, spec.tier_bits, (w_router, bias), shared,
                           down_bits=spec.down_bits, host_tiers=host_tiers)
        tmap, _ = dl.load_experts(pop, src)
        del src_arrays
    return TestLayer(spec=spec, ol=ol, dl=dl, tier_map=tmap, popularity=pop)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
