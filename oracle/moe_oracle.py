"""Plain CPU definition of the routed, tiered, dequantised MoE FFN layer.

Test infrastructure only (see the package docstring): nothing on the product
path may import this module.

Every function computes the plain definition of one step of the layer.  Where
the pages leave a step open, the reading taken is stated in the docstring and
collected in the design notes of the repository.  Pages are cited by title and
section; see the package docstring for the full titles.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "LEVELS",
    "bf16_round",
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "f16_round",
    "quantise_rows",
    "MXFP4",
    "E2M1",
    "MX_XMIN",
    "MX_XMAX",
    "MxBlocks",
    "quantise_rows_mx",
    "dequantise_mx",
    "dequantise_any",
    "code_bit_positions",
    "encode_codes",
    "decode_codes",
    "dequantise",
    "pack_tiles",
    "pack_tiles_mx",
    "build_tiers",
    "expert_table_bytes",
    "plan_tiers",
    "router_keys",
    "select_topk",
    "gate_weights",
    "route",
    "sort_routes",
    "silu",
    "act_round",
    "ExpertBlocks",
    "OracleLayer",
    "expert_ffn",
    "moe_layer",
    "output_cast",
]

#: Format code of an MXFP4 table (a code, not a bit count): 4-bit E2M1
#: elements sharing one E8M0 power-of-two scale per block of 32.
MXFP4 = 0x14

#: Highest code of a block: L = 2**b - 1 for the b-bit affine formats; an
#: MXFP4 code is a 4-bit sign/magnitude pattern (0..15).
LEVELS = {4: 15, 3: 7, 2: 3, MXFP4: 15}

BLOCK = 32


# ---------------------------------------------------------------------------
# Roundings the definition mandates
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    bfloat16 keeps the top 16 bits of a float32.  Written out on the bit
    pattern: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits.
    NaN maps to the canonical quiet NaN 0x7FC0.
    """
    a = np.array(a, dtype=np.float32, order="C")
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    return np.where(np.isnan(a), np.uint16(0x7FC0), r.astype(np.uint16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(a) -> np.ndarray:
    """Round to bfloat16 (RNE) and return the exact values as float32."""
    bits = f32_to_bf16_bits(a).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def f16_round(a) -> np.ndarray:
    """Round to IEEE binary16, ties to even (NumPy's conversion is RNE)."""
    return np.asarray(a).astype(np.float16)


# ---------------------------------------------------------------------------
# A0: block quantiser and block code field
# ---------------------------------------------------------------------------

def quantise_rows(w, bits: int):
    """Quantise each row of ``w`` in blocks of 32 consecutive weights.

    Storing each weight with fewer bits is the method's compression [P1,
    "a small dictionary before we start"; "step 4: three shelves, all on the
    GPU"].  The pages name only llama.cpp's formats; the reading used here is
    an affine block of 32 weights with an fp16 scale ``d`` and an fp16 min
    ``m`` (value = d*q + m), quantised in float32 with one rounding per step:

        lo, hi = min, max of the block (fp32)
        m = RN_f16(lo)
        d = RN_f16(RN_f32(RN_f32(hi - lo) / L))
        q = clamp(rint_half_even(RN_f32(RN_f32(x - m) / d)), 0, L);  d == 0 -> q = 0

    Returns ``(d, m, q)``: float16 arrays of shape ``rows x cols/32`` and a
    uint8 array of shape ``rows x cols``.  Non-finite input, or a scale/min that
    overflows fp16, raises ``ValueError``.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("rows must be a multiple of 32 wide")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    L = LEVELS[bits]
    blk = w.reshape(w.shape[0], -1, BLOCK)
    lo = blk.min(axis=-1)
    hi = blk.max(axis=-1)
    m16 = f16_round(lo)
    span = (hi - lo).astype(np.float32)                  # one fp32 rounding
    d16 = f16_round((span / np.float32(L)).astype(np.float32))
    if not (np.all(np.isfinite(m16)) and np.all(np.isfinite(d16))):
        raise ValueError("block scale or min overflows fp16")
    m32 = m16.astype(np.float32)[..., None]
    d32 = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((blk - m32).astype(np.float32) / d32).astype(np.float32)
        q = np.clip(np.rint(t), 0, L)
    q = np.where(d32 == 0, 0, q).astype(np.uint8)
    return d16, m16, q.reshape(w.shape)


def _field_words(bits: int) -> int:
    """32-bit words in the code field of one block of the format."""
    if bits == MXFP4:
        return 4
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3, 4 or MXFP4")
    return bits


def code_bit_positions(bits: int) -> Sequence[Sequence[int]]:
    """Bit positions of every code inside a block's code field.

    The code field of a b-bit block is ``b`` little-endian 32-bit words (4*b
    bytes).  Reading taken (the pages fix no bit layout): in every word the low
    half-word holds even-numbered codes and the high half-word holds the next
    odd-numbered codes at the same offsets, packed upward from bit 0:

      b = 4: code k = 8i + 2p + s   -> bits 32i + 16s + 4p + (0..3),  p < 4
      b = 2: code k = 16i + 2p + s  -> bits 32i + 16s + 2p + (0..1),  p < 8
      b = 3: code k = 10i + 2p + s  -> bits 32i + 16s + 3p + (0..2),  p < 5, i < 3
             code 30 + s: bit r at 32r + 16s + 15  (r = 0, 1, 2)

    An MXFP4 field (format code ``MXFP4``) is 4 words with code k at bits
    4k .. 4k + 3: byte j holds codes 2j (low nibble) and 2j + 1 (high nibble).

    Returns, for k = 0..31, the list of field bit positions of code k, least
    significant bit first.
    """
    pos = []
    for k in range(BLOCK):
        if bits == 4:
            i, rem = divmod(k, 8)
            p, s = divmod(rem, 2)
            pos.append([32 * i + 16 * s + 4 * p + r for r in range(4)])
        elif bits == 2:
            i, rem = divmod(k, 16)
            p, s = divmod(rem, 2)
            pos.append([32 * i + 16 * s + 2 * p + r for r in range(2)])
        elif bits == MXFP4:
            pos.append([4 * k + r for r in range(4)])
        elif bits == 3:
            if k < 30:
                i, rem = divmod(k, 10)
                p, s = divmod(rem, 2)
                pos.append([32 * i + 16 * s + 3 * p + r for r in range(3)])
            else:
                s = k - 30
                pos.append([32 * r + 16 * s + 15 for r in range(3)])
        else:
            raise ValueError("bits must be 2, 3 or 4")
    return pos


def encode_codes(q, bits: int) -> np.ndarray:
    """Pack codes ``q[..., 32]`` into code fields ``[..., 4*bits]`` (uint8)."""
    q = np.asarray(q, dtype=np.uint32)
    if q.shape[-1] != BLOCK:
        raise ValueError("last axis must hold 32 codes")
    if np.any(q > LEVELS[bits]):
        raise ValueError("code out of range")
    nw = _field_words(bits)
    words = np.zeros(q.shape[:-1] + (nw,), dtype=np.uint32)
    for k, bitpos in enumerate(code_bit_positions(bits)):
        for r, p in enumerate(bitpos):
            bit = (q[..., k] >> np.uint32(r)) & np.uint32(1)
            words[..., p // 32] |= bit << np.uint32(p % 32)
    return words.astype("<u4").view(np.uint8).reshape(q.shape[:-1] + (4 * nw,))


def decode_codes(field_bytes, bits: int) -> np.ndarray:
    """Unpack code fields ``[..., 4*bits]`` (uint8) into codes ``[..., 32]``."""
    fb = np.ascontiguousarray(np.asarray(field_bytes, dtype=np.uint8))
    nw = _field_words(bits)
    if fb.shape[-1] != 4 * nw:
        raise ValueError("code field has the wrong size")
    words = fb.reshape(fb.shape[:-1] + (nw, 4)).view("<u4")[..., 0]
    q = np.zeros(fb.shape[:-1] + (BLOCK,), dtype=np.uint32)
    for k, bitpos in enumerate(code_bit_positions(bits)):
        for r, p in enumerate(bitpos):
            q[..., k] |= ((words[..., p // 32] >> np.uint32(p % 32)) & np.uint32(1)) << np.uint32(r)
    return q.astype(np.uint8)


def dequantise(d, m, q, act: str) -> np.ndarray:
    """Dequantised weights of one matrix, as exact float64 values.

    Value of code q in a block with scale d and min m: the exact d*q + m
    rounded once to float32 (the result of one fp32 fused multiply-add).  For
    bf16 activations the weight is then rounded to bfloat16 (RNE), because the
    contraction runs on bf16 operands; for fp32 activations it stays fp32.

    ``d``, ``m``: float16 ``rows x cols/32``; ``q``: uint8 ``rows x cols``.
    d*q + m is exact in float64 for every finite fp16 d, m and q <= 15 (both
    are multiples of 2**-24 below 2**21), so the cast to float32 is the single
    rounding.
    """
    rows, cols = q.shape
    d64 = np.repeat(np.asarray(d, dtype=np.float16).astype(np.float64), BLOCK, axis=1)
    m64 = np.repeat(np.asarray(m, dtype=np.float16).astype(np.float64), BLOCK, axis=1)
    v32 = (d64 * q.astype(np.float64) + m64).astype(np.float32)
    if act == "bf16":
        v32 = bf16_round(v32)
    elif act != "f32":
        raise ValueError("act must be 'f32' or 'bf16'")
    return v32.astype(np.float64)


# ---------------------------------------------------------------------------
# A0: MXFP4 blocks (the pages' low tier for the down matrices)
# ---------------------------------------------------------------------------

#: Magnitudes of the E2M1 codes 0..7; code 8 + i is the negation of code i.
E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

#: Range of the shared exponent X (block scale 2**X, stored as the E8M0 byte
#: X + 127).  With X >= -125 every non-zero element (at least 0.5 * 2**X) is a
#: normal float32/bf16 number, and with X <= 125 the largest (6 * 2**X) is
#: finite.
MX_XMIN, MX_XMAX = -125, 125


@dataclass(frozen=True)
class MxBlocks:
    """One matrix in MXFP4: ``e`` uint8 ``rows x cols/32`` (E8M0 scale bytes,
    block scale 2**(e - 127)) and ``q`` uint8 ``rows x cols`` (E2M1 codes)."""

    e: np.ndarray
    q: np.ndarray


def _e2m1_round(t: np.ndarray) -> np.ndarray:
    """E2M1 code nearest to each (exactly scaled) value ``t``.

    Ties go to the code with an even mantissa bit (an even code index), as in
    IEEE round-to-nearest-even; magnitudes above 6 saturate to 6 (E2M1 has
    no infinity).  A value that rounds to zero gets code 0 (positive zero).
    """
    a = np.abs(t)
    grid = np.asarray(E2M1, dtype=np.float64)
    dist = np.abs(a[..., None] - grid)                   # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    # among the nearest, the even index if there is one (a tie is between
    # neighbours i, i + 1, exactly one of which is even)
    cand = dist == best
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    idx = np.where(a > 6.0, 7, idx)
    sign = (t < 0) & (idx > 0)
    return (idx + 8 * sign).astype(np.uint8)


def quantise_rows_mx(w) -> MxBlocks:
    """Quantise each row of ``w`` to MXFP4 in blocks of 32 consecutive weights.

    The pages give MXFP4 as the low-tier format of the down matrices [P1,
    "step 4: three shelves, all on the GPU"; P2, "Lever 2"] and nothing of its
    recipe.  Reading taken: the OCP Microscaling (MX) v1.0 definition of
    MXFP4 and its conversion from wider floats.  Per block:

        amax = max |x|
        X    = floor(log2(amax)) - 2       (2 = largest E2M1 exponent;
                                            amax == 0: X = MX_XMIN)
        X    = clamp(X, MX_XMIN, MX_XMAX)  (kept normal and finite, above)
        q_i  = E2M1 code nearest to x_i / 2**X (ties to even, saturating at 6)

    x / 2**X is exact in float64, so each code is a decision on exact values.
    Non-finite input raises ``ValueError``.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("rows must be a multiple of 32 wide")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    blk = w.reshape(w.shape[0], -1, BLOCK).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)                 # amax = f * 2**ex, 0.5 <= f < 1
    X = np.where(amax > 0, ex - 1 - 2, MX_XMIN)
    X = np.clip(X, MX_XMIN, MX_XMAX)
    t = np.ldexp(blk, -X[..., None])
    q = _e2m1_round(t)
    return MxBlocks((X + 127).astype(np.uint8), q.reshape(w.shape))


def dequantise_mx(e, q, act: str) -> np.ndarray:
    """Dequantised weights of one MXFP4 matrix, as exact float64 values.

    Value of code q in a block with scale byte e: (-1)**(q >> 3) *
    E2M1[q & 7] * 2**(e - 127).  For e in [MX_XMIN + 127, MX_XMAX + 127] that
    value is exactly representable in bfloat16 and float32 (two significant
    bits, normal exponent), so no rounding is involved for either activation
    dtype.
    """
    e = np.asarray(e, dtype=np.int64)
    q = np.asarray(q, dtype=np.uint8)
    if act not in ("f32", "bf16"):
        raise ValueError("act must be 'f32' or 'bf16'")
    if np.any(e < MX_XMIN + 127) or np.any(e > MX_XMAX + 127):
        raise ValueError("scale byte out of range")
    mag = np.asarray(E2M1, dtype=np.float64)[q & 7]
    val = np.where(q & 8, -mag, mag)
    X = np.repeat(e - 127, BLOCK, axis=1)
    return np.ldexp(val, X)


def dequantise_any(mat, act: str) -> np.ndarray:
    """Dequantised matrix of either format: an :class:`MxBlocks`, or an affine
    ``(d, m, q)`` triple."""
    if isinstance(mat, MxBlocks):
        return dequantise_mx(mat.e, mat.q, act)
    return dequantise(*mat, act=act)


def _tile_index(S: int, R: int, C: int) -> np.ndarray:
    """Table index of every block ``[S][R][C/32]`` (flattened), in the tile
    order described in :func:`pack_tiles`."""
    if R % 16 or C % 128:
        raise ValueError("tile tables need rows % 16 == 0 and cols % 128 == 0")
    nb = C // BLOCK
    s_idx, r_idx, j_idx = np.meshgrid(np.arange(S), np.arange(R), np.arange(nb), indexing="ij")
    tile = (s_idx * (R // 16) + r_idx // 16) * (C // 128) + j_idx // 4
    lane = 16 * (j_idx % 4) + r_idx % 16
    return (tile * 64 + lane).reshape(-1)


def pack_tiles(q, d, m, bits: int):
    """Arrange quantised blocks of one tier table in device tile order.

    ``q``: uint8 ``[S][R][C]`` (S expert slots, R rows, C columns along the
    contraction axis); ``d``, ``m``: float16 ``[S][R][C/32]``.

    Tile layout (a reading: the pages fix none).  A tile is 16 rows by 4
    blocks (128 columns).  The block in slot s, row r, block column j goes to

        tile  = (s * (R/16) + r // 16) * (C/128) + j // 4
        lane  = 16 * (j % 4) + r % 16
        index = tile * 64 + lane

    and the tables are ``codes[index]`` (the 4*bits-byte code field of the
    block) and ``dm[index]`` = fp16 bits of d | (fp16 bits of m) << 16.
    Returns ``(codes uint8 [S*R*C/32 * 4*bits], dm uint32 [S*R*C/32])``.
    MXFP4 tables are packed by :func:`pack_tiles_mx`.
    """
    q = np.asarray(q, dtype=np.uint8)
    S, R, C = q.shape
    index = _tile_index(S, R, C)
    nb = C // BLOCK
    fields = encode_codes(q.reshape(S, R, nb, BLOCK), bits)           # [S][R][nb][4b]
    dbits = np.asarray(d, dtype=np.float16).view(np.uint16).astype(np.uint32)
    mbits = np.asarray(m, dtype=np.float16).view(np.uint16).astype(np.uint32)
    dm = dbits | (mbits << np.uint32(16))                              # [S][R][nb]
    nbytes = S * R * nb
    codes_out = np.zeros((nbytes, 4 * bits), dtype=np.uint8)
    dm_out = np.zeros(nbytes, dtype=np.uint32)
    codes_out[index] = fields.reshape(-1, 4 * bits)
    dm_out[index] = dm.reshape(-1)
    return codes_out.reshape(-1), dm_out


def pack_tiles_mx(q, e):
    """MXFP4 counterpart of :func:`pack_tiles`: the same tile order, a 16-byte
    code field per block (code k at bits 4k .. 4k + 3) and a one-byte scale
    table (the E8M0 byte of each block).

    ``q``: uint8 ``[S][R][C]`` E2M1 codes; ``e``: uint8 ``[S][R][C/32]``.
    Returns ``(codes uint8 [S*R*C/32 * 16], scales uint8 [S*R*C/32])``.
    """
    q = np.asarray(q, dtype=np.uint8)
    S, R, C = q.shape
    index = _tile_index(S, R, C)
    nb = C // BLOCK
    fields = encode_codes(q.reshape(S, R, nb, BLOCK), MXFP4)          # [S][R][nb][16]
    nbytes = S * R * nb
    codes_out = np.zeros((nbytes, 16), dtype=np.uint8)
    sc_out = np.zeros(nbytes, dtype=np.uint8)
    codes_out[index] = fields.reshape(-1, 16)
    sc_out[index] = np.asarray(e, dtype=np.uint8).reshape(-1)
    return codes_out.reshape(-1), sc_out


# ---------------------------------------------------------------------------
# A0: popularity tiers
# ---------------------------------------------------------------------------

def build_tiers(popularity, n_slots: Sequence[int]):
    """Expert id -> (tier, slot) map from usage counts.

    Experts are ranked by how often they are used, busiest first [P1, "step 2:
    the experts are not equal"], and the busiest get the most bits: three
    shelves, experts stored hottest-first [P1, "step 4: three shelves, all on
    the GPU"; P2, "Lever 2"].  Rank order is (popularity descending, id
    ascending).  Ranks [0, n0) form tier 0, the next n1 tier 1, the last n2
    tier 2; slot = rank minus the start of its tier.

    Returns ``(tier_map, slot_expert)``: ``tier_map[e] = tier << 16 | slot`` and
    ``slot_expert[rank] = e`` (int32).
    """
    pop = np.asarray(popularity, dtype=np.uint64)
    E = pop.shape[0]
    if sum(n_slots) != E or min(n_slots) < 0:
        raise ValueError("n_slots must be non-negative and sum to E")
    order = sorted(range(E), key=lambda e: (-int(pop[e]), e))
    tier_map = np.zeros(E, dtype=np.int32)
    starts = [0, n_slots[0], n_slots[0] + n_slots[1]]
    for rank, e in enumerate(order):
        tier = 0 if rank < starts[1] else (1 if rank < starts[2] else 2)
        tier_map[e] = (tier << 16) | (rank - starts[tier])
    return tier_map, np.asarray(order, dtype=np.int32)


def expert_table_bytes(hidden: int, inter: int, bits: int) -> int:
    """Bytes of one expert's three matrices (gate, up: inter x hidden; down:
    hidden x inter) at `bits` bits: every block of 32 weights holds a
    4*bits-byte code field and a 4-byte (d, m) word; an MXFP4 block holds a
    16-byte field and a 1-byte scale."""
    per_block = 17 if bits == MXFP4 else 4 * _field_words(bits) + 4
    return 3 * hidden * inter // BLOCK * per_block


#: Expected-error weight of a b-bit block per weight, scaled to integers:
#: 11025 / (2^b - 1)^2 (11025 = 15^2 * 7^2), so 49, 225 and 1225 for 4, 3 and 2
#: bits.
ERR_WEIGHT = {4: 49, 3: 225, 2: 1225}


def plan_tiers(popularity, tier_bits: Sequence[int], hidden: int, inter: int,
               budget_bytes: int, down_bits: Optional[Sequence[int]] = None):
    """Tier sizes (n0, n1, n2) that fit the expert tables in a byte budget.

    The pages' re-packer fills a memory budget with a planner that gives each
    byte to the expert where it removes the most expected error, weighting
    the error by how often the expert is used [P1, "step 4: three shelves,
    all on the GPU"; the command line of "reproduce it" takes the budget].
    Readings (the pages give neither the error model nor the search):

    - expected error of an expert at b bits = popularity x (2^b - 1)^-2: the
      mean square error of a uniform b-bit quantiser over a block's range,
      whose common factor (range^2 / 12 per weight) cancels.  With no
      importance data, this width-only model is the only synthetic error
      available;
    - a plan is a set of popularity bands, the layout build_tiers stores:
      ranks [0, n0) in tier 0, the next n1 in tier 1, the rest in tier 2;
    - the plan minimises the total expected error among the band plans whose
      tables take at most budget_bytes; equal errors prefer the larger n0,
      then the larger n1.

    Under a width-only error the greedy of the pages upgrades hotter experts
    first at every width step, so its result is itself a band plan, and the
    exhaustive search over bands below never does worse.  Raises ValueError
    when no plan fits, or for an MXFP4 tier (outside the error model).

    ``down_bits`` (0: the tier's width) gives the down matrices their own
    ladder, as the pages' re-packer plans with separate gate/up and down
    format lists [P1, "step 4: three shelves, all on the GPU"].  An expert of
    tier t then costs two matrices at tier_bits[t] and one at its down width,
    and its error is the sum over its three equally sized matrices.
    """
    dn = [d if d else b for b, d in zip(tier_bits, down_bits or (0, 0, 0))]
    if any(b not in ERR_WEIGHT for b in list(tier_bits) + dn):
        raise ValueError("the error model covers the 2-, 3- and 4-bit affine widths only")
    pop = [int(v) for v in np.asarray(popularity, dtype=np.uint64)]
    E = len(pop)
    order = sorted(range(E), key=lambda e: (-pop[e], e))
    # per expert: 2/3 of a whole expert at the gate/up width plus 1/3 at the
    # down width (each term is an integer: a matrix is a third of the tables)
    cost_b = [2 * expert_table_bytes(hidden, inter, b) // 3 + expert_table_bytes(hidden, inter, d) // 3
              for b, d in zip(tier_bits, dn)]
    w = [2 * ERR_WEIGHT[b] + ERR_WEIGHT[d] for b, d in zip(tier_bits, dn)]
    best = None
    for n0 in range(E, -1, -1):
        for n1 in range(E - n0, -1, -1):
            n2 = E - n0 - n1
            nbytes = n0 * cost_b[0] + n1 * cost_b[1] + n2 * cost_b[2]
            if nbytes > budget_bytes:
                continue
            err = 0
            for rank, e in enumerate(order):
                tier = 0 if rank < n0 else (1 if rank < n0 + n1 else 2)
                err += pop[e] * w[tier]
            if best is None or err < best[0]:
                best = (err, (n0, n1, n2))
    if best is None:
        raise ValueError("no tier plan fits the byte budget")
    return best[1]


# ---------------------------------------------------------------------------
# A1-A2: router
# ---------------------------------------------------------------------------

def router_keys(x, w_router, bias=None, exact: bool = False) -> np.ndarray:
    """Router score of every expert for every token.

    A router scores all experts of a layer for each token and keeps the best
    ten [P1, "a small dictionary before we start"; P2, "The Bottleneck"].  The
    pages give no arithmetic; the reading is key = x . w_e + b_e evaluated
    exactly and rounded once to float64.  ``exact=True`` uses ``math.fsum``
    (correctly rounded, for tiny inputs); otherwise a float64 matrix product,
    whose error (~1e-16 relative) is far below any gap between keys that the
    layer resolves.

    ``x``: ``T x H``; ``w_router``: ``E x H`` (exact values of the activation
    dtype); ``bias``: ``E`` or None.  Returns float64 ``T x E``.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    if exact:
        T, E = x.shape[0], w.shape[0]
        keys = np.empty((T, E), dtype=np.float64)
        for t in range(T):
            for e in range(E):
                terms = list(x[t] * w[e])          # each product exact in fp64
                if b is not None:
                    terms.append(b[e])
                keys[t, e] = math.fsum(terms)
        return keys
    keys = x @ w.T
    if b is not None:
        keys = keys + b[None, :]
    return keys


def select_topk(keys, k: int) -> np.ndarray:
    """Ids of the ``k`` best experts per token, in rank order.

    Order is (key descending, expert id ascending): equal keys go to the lower
    id.  -0 equals +0 and NaN ranks last.  The ids of one token are distinct:
    the grouping step assumes each expert appears at most once per token [P1,
    "the four bugs, briefly"].
    """
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # a stable sort of -key keeps ascending ids among equal keys; NumPy
        # sorts NaN last
        ids[t] = np.argsort(-keys[t], kind="stable")[:k]
    return ids


def gate_weights(keys, ids) -> np.ndarray:
    """Mixing weights of the selected experts.

    The outputs of the chosen experts are summed [P1, "step 4: three shelves,
    all on the GPU"]; the reading is a softmax over the selected keys, which
    equals a softmax over all E keys renormalised over the chosen ones:
    g_k = exp(key_k - key_0) / sum_j exp(key_j - key_0).  Float64.
    """
    sel = np.take_along_axis(np.asarray(keys, dtype=np.float64), ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k: int, exact: bool = False):
    """Keys, selected ids and weights for a batch of tokens."""
    keys = router_keys(x, w_router, bias, exact=exact)
    ids = select_topk(keys, k)
    return keys, ids, gate_weights(keys, ids)


# ---------------------------------------------------------------------------
# A4: grouping routes by expert
# ---------------------------------------------------------------------------

def sort_routes(ids, n_experts: int):
    """Group routes by expert with a stable counting sort.

    Route r = t*K + k is token t's k-th choice.  The batched path groups the
    words of a batch by chosen expert [P1, "the four bugs, briefly"].  Result:
    ``offsets[E+1]`` (exclusive prefix sum of per-expert counts) and
    ``sorted_routes[T*K]`` holding the routes of expert e at
    ``offsets[e]:offsets[e+1]`` in ascending route order.  Integer, exact.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_routes = np.empty(flat.shape[0], dtype=np.int64)
    for r, e in enumerate(flat):
        sorted_routes[cursor[e]] = r
        cursor[e] += 1
    return offsets.astype(np.int32), sorted_routes.astype(np.int32)


# ---------------------------------------------------------------------------
# A5-A8: expert FFN and the layer
# ---------------------------------------------------------------------------

def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def act_round(a, act: str) -> np.ndarray:
    """Round to the activation dtype (bf16 RNE or fp32), as float64 values."""
    a = np.asarray(a, dtype=np.float64)
    if act == "bf16":
        # round once from the float64 value (going through float32 first
        # could round twice)
        return _bf16_from_f64(a)
    if act == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError("act must be 'f32' or 'bf16'")


def _bf16_from_f64(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 once (RNE), returned as float64."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    flat_in = a.reshape(-1)
    flat_out = out.reshape(-1)
    mant, expo = np.frexp(flat_in)                 # a = mant * 2**expo, 0.5 <= |mant| < 1
    # bf16 has 8 significant bits: scale so that the kept bits are integral
    scaled = mant * 256.0                          # exact
    r = np.rint(scaled)                            # ties to even, exact in fp64
    res = np.ldexp(r / 256.0, expo)
    # subnormal / overflow ranges of bf16 follow float32's: fall back to the
    # bit-pattern rounding of the exact fp32 value when |a| is outside the
    # normal range (no such values occur in the layer's data)
    small = (np.abs(flat_in) < np.float64(np.finfo(np.float32).tiny)) & (flat_in != 0)
    big = np.abs(flat_in) >= np.float64(np.finfo(np.float32).max)
    bad = small | big | ~np.isfinite(flat_in)
    flat_out[:] = res
    if np.any(bad):
        flat_out[bad] = bf16_round(flat_in[bad].astype(np.float32)).astype(np.float64)
    return out


@dataclass
class ExpertBlocks:
    """Quantised matrices of one expert: (d, m, q) per matrix (or an
    :class:`MxBlocks` for an MXFP4 matrix) and the gate/up bit width.

    gate and up are ``I x H`` (rows along the hidden size), down is ``H x I``.
    """

    bits: int
    gate: Tuple[np.ndarray, np.ndarray, np.ndarray]
    up: Tuple[np.ndarray, np.ndarray, np.ndarray]
    down: Tuple[np.ndarray, np.ndarray, np.ndarray]


@dataclass
class OracleLayer:
    """One MoE layer as the oracle sees it (all values exact, float64).

    ``experts(e)`` returns the :class:`ExpertBlocks` of expert ``e``;
    ``shared`` holds the shared expert's (gate, up, down) weights already in
    the activation dtype, or None.
    """

    act: str
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    top_k: int
    experts: Callable[[int], ExpertBlocks]
    shared: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None
    _cache: Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]] = field(default_factory=dict)

    def dense(self, e: int):
        """Dequantised (gate, up, down) of expert ``e`` (cached)."""
        if e not in self._cache:
            blk = self.experts(e)
            self._cache[e] = tuple(dequantise_any(mat, self.act)
                                   for mat in (blk.gate, blk.up, blk.down))
        return self._cache[e]


def expert_ffn(x, gate_w, up_w, down_w, act: str):
    """SwiGLU expert on token rows ``x`` (``n x H``): returns ``(h, out)``.

    The decode path fuses gate, up and the activation [P1, "step 4: three
    shelves, all on the GPU"; "the four bugs, briefly"].  Reading: gate is the
    first matrix, h = RN_act(silu(x W_g^T) * (x W_u^T)), out = h W_d^T; the
    products are exact (float64), the only rounding is that of h to the
    activation dtype, which is what the down contraction consumes.
    """
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(gate_w, dtype=np.float64).T
    u = x @ np.asarray(up_w, dtype=np.float64).T
    h = act_round(silu(g) * u, act)
    return h, h @ np.asarray(down_w, dtype=np.float64).T


def moe_layer(x, layer: OracleLayer, tokens: Optional[Sequence[int]] = None,
              routing=None, exact_keys: bool = False, drop_experts: bool = False):
    """Output of the layer for the rows ``tokens`` of ``x`` (all rows if None).

    Each token runs through its K chosen experts plus the one shared expert
    [P5, "What the model actually is": 10 routed plus 1 shared], and the
    results add up [P1, "step 4: three shelves, all on the GPU"]:

        y[t] = sum_k g[t,k] * out_{ids[t,k]}(x[t]) + out_shared(x[t])

    in float64.  ``routing`` may pass precomputed ``(keys, ids, g)`` for all
    rows of ``x``.  ``drop_experts`` forgets each expert's dequantised weights
    once its bucket is done (memory only; the arithmetic is the same).
    Returns a dict with keys, ids, g (for all rows) and ``y`` (float64, one
    row per requested token).
    """
    x = np.asarray(x, dtype=np.float64)
    if routing is None:
        routing = route(x, layer.w_router, layer.bias, layer.top_k, exact=exact_keys)
    keys, ids, g = routing
    rows = list(range(x.shape[0])) if tokens is None else list(tokens)
    H = x.shape[1]
    y = np.zeros((len(rows), H), dtype=np.float64)
    # group the requested routes by expert so each expert is dequantised once
    by_expert: Dict[int, list] = {}
    for i, t in enumerate(rows):
        for k in range(ids.shape[1]):
            by_expert.setdefault(int(ids[t, k]), []).append((i, t, k))
    for e in sorted(by_expert):
        gw, uw, dw = layer.dense(e)
        lst = by_expert[e]
        _, out = expert_ffn(x[[t for _, t, _ in lst]], gw, uw, dw, layer.act)
        for j, (i, t, k) in enumerate(lst):
            y[i] += g[t, k] * out[j]
        if drop_experts:
            layer._cache.pop(e, None)
    if layer.shared is not None:
        _, out_s = expert_ffn(x[rows], *layer.shared, act=layer.act)
        y += out_s
    return {"keys": keys, "ids": ids, "g": g, "y": y}


def output_cast(y, out_dtype: str) -> np.ndarray:
    """The layer's last step: the float64 output rounded once to the output
    dtype ("f32" or "bf16", round to nearest even), returned as float64.

    The output of a bf16 layer is itself a bf16 tensor; its comparison with
    the oracle is with this rounded value (rounding alone moves a vector of
    unit-scale values by ~1.6e-3 relative L2)."""
    return act_round(y, out_dtype)
