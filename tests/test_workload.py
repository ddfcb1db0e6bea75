"""The synthetic router reproduces the routing skew the pages report.

P1 ("I ran a 125B model on three RTX 3090s at 80 tokens/s"), section "step 2:
the experts are not equal": in the average layer the busiest 25% of experts
handle 52% of the tokens and the busiest 80% handle 95%; section "step 3: split
every layer into hot and cold": the coldest experts holding 19% of the bytes
serve 4.5% of routed tokens.  Counts are taken on the calibration tokens, as
the page's counts come from calibration text.
"""

import numpy as np
import pytest

import oracle as O
import synth


@pytest.mark.parametrize("seed", [0, 1])
def test_full_size_router_skew_matches_pages(seed):
    spec = synth.FULL
    w, b = synth.router(spec, seed)
    x = synth.tokens(spec, 4096, seed + 1)
    keys = O.router_keys(O.bf16_bits_to_f64(x), O.bf16_bits_to_f64(w), b)
    ids = O.select_topk(keys, spec.top_k)
    counts = np.sort(np.bincount(ids.ravel(), minlength=spec.n_experts))[::-1]
    total = counts.sum()
    top25 = counts[: spec.n_experts // 4].sum() / total
    top80 = counts[: int(round(0.8 * spec.n_experts))].sum() / total
    cold19 = counts[spec.n_experts - int(round(0.19 * spec.n_experts)):].sum() / total
    assert abs(top25 - 0.52) < 0.015
    assert abs(top80 - 0.95) < 0.01
    assert abs(cold19 - 0.045) < 0.01


def test_correlated_tokens_cosine():
    spec = synth.FULL
    x = O.bf16_bits_to_f64(synth.correlated_tokens(spec, 16, 3))
    xn = x / np.linalg.norm(x, axis=1, keepdims=True)
    c = xn @ xn.T
    off = c[~np.eye(16, dtype=bool)]
    assert abs(off.mean() - 0.6) < 0.03
