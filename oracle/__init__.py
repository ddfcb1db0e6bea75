"""CPU oracle for the routed, popularity-tiered, dequantised MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``quantized_expert_ffn_route_amd`` and its HIP
library) never imports it, and this package never imports the product path.

The oracle is plain NumPy on the host: float64 everywhere except the roundings
that the layer's definition itself mandates (fp16 scale/min, fp32 dequantised
value, bf16 weights and ``h`` for bf16 activations, and the final output cast).
It computes the plain definition of each step; no blocking, fusion or
reordering beyond what that definition states.

Pages cited (by title and section):

* [P1] "I ran a 125B model on three RTX 3090s at 80 tokens/s by teaching
  llama.cpp which experts matter" (dev.to)
* [P2] "Running Qwen3.8-Flash-Next 125B on Three RTX 3090s at 80 Tokens per
  Second" (explore.n1n.ai)
* [P5] "Qwen3.8-Flash-Next hits 39 tok/s on a 24GB GPU, provided you bring
  96GB of system RAM" (deniz.in)

Pin status of every function (the pins live in ``tests/test_oracle_pins.py``
and ``tests/golden/``):

* ``bf16_round``/``f16_round``: pinned (hand ties, torch/numpy conversions).
* ``quantise_rows``: pinned (hand-computed blocks, half-even tie block,
  reconstruction bound).
* ``encode_codes``/``decode_codes``/``pack_tiles``/``pack_tiles_mx``: pinned
  (hand-derived byte strings, brute-force placement on tiny shapes).
* ``quantise_rows_mx``/``dequantise_mx`` (MXFP4): pinned (hand blocks from the
  OCP MX definition, E2M1 values from their bit fields, brute force by exact
  rational search, reconstruction bound, equality with an affine container
  holding the same values through the whole layer).
* ``dequantise``: pinned (hand blocks, exact fp64 identity).
* ``build_tiers``: pinned (brute force, uniform popularity, bijection).
* ``expert_table_bytes``/``plan_tiers``: pinned (closed forms at the budget
  extremes, brute force over every per-expert assignment on tiny shapes, the
  pages' greedy never beating it, budget monotonicity).
* ``router_keys``/``select_topk``/``gate_weights``: pinned (math.fsum exact
  sums, brute-force tuple sort, exact ties, sum-to-one, K=1, K=E).
* ``sort_routes``: pinned (lexsort of (route, expert), tiny brute force).
* ``moe_layer``: pinned through special cases (E=K=1 dense SwiGLU via
  matmul, closed-form constant-weight layer, zero input, identical experts,
  2-bit codes re-stored at 4 bits, relabelling).  Its absolute values at
  general random inputs have no worked example on the pages: beyond those
  special cases the layer output is "parity unpinned" by the pages.
"""

from .moe_oracle import *  # noqa: F401,F403
