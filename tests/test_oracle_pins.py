"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Every test here runs on the CPU.  The pins are hand-derived values
(``tests/golden``), closed forms, brute force on tiny inputs by an independent
method (counting instead of sorting, exact rational arithmetic instead of
floating point) and invariants of the definition.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _expand(expr, n=32):
    i = np.arange(n)
    k = i
    expr = expr.replace(" mod ", " % ")
    return np.asarray(eval(expr, {"i": i, "k": k, "np": np}), dtype=np.float64) * np.ones(n)


# ----------------------------------------------------------------- roundings

def test_bf16_round_hand_ties():
    # bf16 keeps 8 significant bits: the spacing at 1.0 is 2^-7
    cases = {
        1.0 + 2.0 ** -8: 1.0,                     # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,     # tie -> even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,
        -(1.0 + 2.0 ** -8): -1.0,
        65504.0: 65536.0,
    }
    for x, want in cases.items():
        assert float(O.bf16_round(np.float32(x))) == want, x


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.bf16_round(a), want)


def _bf16_exact(fr: Fraction) -> Fraction:
    """Round a rational to 8 significant bits, ties to even (brute force)."""
    if fr == 0:
        return fr
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128
    lo = math.floor(scaled)
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * Fraction(lo, 128) * Fraction(2) ** e


def test_act_round_bf16_from_f64_single_rounding():
    rng = np.random.default_rng(2)
    vals = rng.standard_normal(400) * np.exp(rng.uniform(-10, 10, 400))
    # values just beside bf16 midpoints, where fp64 -> fp32 -> bf16 would round twice
    mid = 1.0 + 2.0 ** -8
    vals = np.concatenate([vals, [mid + 2.0 ** -40, mid - 2.0 ** -40, -(mid + 2.0 ** -40)]])
    got = O.act_round(vals, "bf16")
    for v, g in zip(vals, got):
        assert Fraction(float(g)) == _bf16_exact(Fraction(float(v))), v


# ------------------------------------------------------------- quantiser

@pytest.mark.parametrize("case", _load("quant_blocks.json")["cases"], ids=lambda c: c["name"])
def test_quantiser_hand_blocks(case):
    x = np.asarray(case["x_list"]) if "x_list" in case else _expand(case["x"])
    if "const" in case["name"]:
        x = np.full(32, 1.25)
    d, m, q = O.quantise_rows(x.astype(np.float32)[None, :], case["bits"])
    assert float(d[0, 0]) == case["d"]
    assert float(m[0, 0]) == case["m"]
    want_q = np.asarray(case["q_list"]) if "q_list" in case else _expand(case["q"]).astype(int)
    np.testing.assert_array_equal(q[0], want_q)
    # dequantised values reproduce the (exactly representable) inputs
    v = O.dequantise(d, m, q, act="f32")
    if "const" not in case["name"] and "ties" not in case["name"]:
        np.testing.assert_array_equal(v[0], x)


def _derivation():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "derive_quant_rounding", os.path.join(GOLDEN, "derive_quant_rounding.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_ROUNDING = _load("quant_rounding_blocks.json")["cases"]


def _block(case):
    return np.asarray([float.fromhex(h) for h in case["x_hex"]], dtype=np.float32)[None, :]


@pytest.mark.parametrize("case", _ROUNDING, ids=lambda c: c["name"])
def test_quantiser_rounding_blocks(case):
    # blocks where m, d or a code depends on the rounding of one step; the
    # expected values come from exact rational arithmetic (Fraction), not from
    # NumPy's float16/float32 conversions
    d, m, q = O.quantise_rows(_block(case), case["bits"])
    assert int(d.view(np.uint16)[0, 0]) == case["d_bits"]
    assert int(m.view(np.uint16)[0, 0]) == case["m_bits"]
    np.testing.assert_array_equal(q[0], case["q"])


def test_rounding_blocks_follow_from_exact_arithmetic():
    # the stored values are what the Fraction derivation gives, and each block
    # separates the stated rounding from the wrong variant it names
    der = _derivation()
    fresh = der.derive()
    assert fresh == _ROUNDING
    for case in _ROUNDING:
        xs = [Fraction(float.fromhex(h)) for h in case["x_hex"]]
        wrong = (der.quantise_trunc16 if case["catches"] == "trunc16" else der.quantise_f64_steps)(
            xs, case["bits"])
        assert (der.f16_bits(wrong[0]), der.f16_bits(wrong[1]), wrong[2]) != (
            case["d_bits"], case["m_bits"], case["q"])


def test_rounding_blocks_catch_planted_oracle_mistakes(monkeypatch):
    # plant each mistake in the oracle (CPU only) and check a block fails
    def trunc_f16(a):
        a = np.asarray(a, dtype=np.float64)
        r = a.astype(np.float16)
        # step toward zero where RNE went away from zero
        away = np.abs(r.astype(np.float64)) > np.abs(a)
        r = np.where(away, np.nextafter(r, np.float16(0)), r)
        return r.astype(np.float16)

    def run_all():
        bad = 0
        for case in _ROUNDING:
            d, m, q = O.quantise_rows(_block(case), case["bits"])
            got = (int(d.view(np.uint16)[0, 0]), int(m.view(np.uint16)[0, 0]), list(q[0]))
            bad += got != (case["d_bits"], case["m_bits"], case["q"])
        return bad

    assert run_all() == 0
    with monkeypatch.context() as mp:
        mp.setattr(O.moe_oracle, "f16_round", trunc_f16)
        assert run_all() >= 2
    # fp64 intermediates: quantise with the float32 casts removed
    src = O.moe_oracle.quantise_rows

    def quantise_f64(w, bits):
        w = np.asarray(w, dtype=np.float64)
        L = O.LEVELS[bits]
        blk = w.reshape(w.shape[0], -1, 32)
        lo, hi = blk.min(-1), blk.max(-1)
        m16 = (lo).astype(np.float16)
        d16 = ((hi - lo) / L).astype(np.float16)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.clip(np.rint((blk - m16.astype(np.float64)[..., None]) /
                                d16.astype(np.float64)[..., None]), 0, L)
        q = np.where(d16[..., None] == 0, 0, q).astype(np.uint8)
        return d16, m16, q.reshape(w.shape)

    with monkeypatch.context() as mp:
        mp.setattr(O, "quantise_rows", quantise_f64)
        assert run_all() >= 2
    assert O.moe_oracle.quantise_rows is src


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_quantiser_reconstruction_bound(bits):
    rng = np.random.default_rng(bits)
    w = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 2, (64, 1)))).astype(np.float32)
    d, m, q = O.quantise_rows(w, bits)
    L = O.LEVELS[bits]
    assert q.max() <= L
    v = O.dequantise(d, m, q, act="f32").reshape(64, -1, 32)
    blk = w.astype(np.float64).reshape(64, -1, 32)
    lo = blk.min(-1, keepdims=True)
    d64 = d.astype(np.float64)[..., None]
    m64 = m.astype(np.float64)[..., None]
    # rounding to the nearest level costs at most d/2; the fp16 min and scale
    # shift the grid by |lo - m| and by at most L * d * 2^-11
    bound = 0.5 * d64 * (1 + 1e-6) + np.abs(lo - m64) + L * d64 * 2.0 ** -10 + 1e-30
    assert np.all(np.abs(blk - v) <= bound)
    # the largest and smallest weights land on the top and bottom codes
    assert np.all(q.reshape(64, -1, 32).max(-1) >= L - 1)
    assert np.all(q.reshape(64, -1, 32).min(-1) <= 1)


def test_quantiser_rejects_nonfinite():
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        O.quantise_rows(w, 4)
    w[0, 3] = 5e5  # scale 5e5/15 = 33333 still fits fp16
    O.quantise_rows(w, 4)
    w[0, 3] = 3e9  # (hi - lo) / 15 > 65504: fp16 scale overflows
    with pytest.raises(ValueError):
        O.quantise_rows(w, 4)


def test_dequantise_is_one_fp32_rounding():
    rng = np.random.default_rng(3)
    d = rng.uniform(1e-4, 10, (8, 4)).astype(np.float16)
    m = rng.uniform(-10, 10, (8, 4)).astype(np.float16)
    q = rng.integers(0, 16, (8, 128)).astype(np.uint8)
    v = O.dequantise(d, m, q, act="f32")
    for r in range(8):
        for c in range(0, 128, 7):
            exact = Fraction(float(d[r, c // 32])) * int(q[r, c]) + Fraction(float(m[r, c // 32]))
            # float32 rounding of the exact rational: compare against the two
            # neighbouring float32 values
            f = np.float32(float(exact))
            assert abs(Fraction(float(f)) - exact) <= abs(Fraction(float(np.nextafter(f, np.float32(np.inf)))) - exact)
            assert abs(Fraction(float(f)) - exact) <= abs(Fraction(float(np.nextafter(f, np.float32(-np.inf)))) - exact)
            assert v[r, c] == float(f)
    vb = O.dequantise(d, m, q, act="bf16")
    np.testing.assert_array_equal(vb, O.bf16_round(v.astype(np.float32)).astype(np.float64))


# ------------------------------------------------------------ code fields

@pytest.mark.parametrize("case", _load("code_fields.json")["cases"], ids=lambda c: str(c["bits"]))
def test_code_field_hand_words(case):
    bits = case["bits"]
    q = _expand(case["q"]).astype(np.uint8)
    field = O.encode_codes(q, bits)
    words = field.view("<u4")
    assert [f"0x{int(w):08X}" for w in words] == [w.upper().replace("0X", "0x") for w in case["words"]]
    np.testing.assert_array_equal(O.decode_codes(field, bits), q)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_code_positions_partition_the_field(bits):
    pos = O.code_bit_positions(bits)
    flat = sorted(p for code in pos for p in code)
    assert flat == list(range(32 * bits))
    assert all(len(code) == bits for code in pos)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_code_field_single_code_brute_force(bits):
    # setting one code to all-ones must set exactly its listed bits
    pos = O.code_bit_positions(bits)
    for k in range(32):
        q = np.zeros(32, np.uint8)
        q[k] = O.LEVELS[bits]
        field = O.encode_codes(q, bits)
        as_int = int.from_bytes(field.tobytes(), "little")
        assert as_int == sum(1 << p for p in pos[k])


# ------------------------------------------------------------------ tiles

@pytest.mark.parametrize("case", _load("tile_index.json")["cases"])
def test_tile_index_hand(case):
    S, R, C = case["S"], case["R"], case["C"]
    q = np.zeros((S, R, C), np.uint8)
    d = np.zeros((S, R, C // 32), np.float16)
    m = np.zeros((S, R, C // 32), np.float16)
    d[case["s"], case["r"], case["j"]] = np.float16(1.5)
    q[case["s"], case["r"], 32 * case["j"]] = 3
    codes, dm = O.pack_tiles(q, d, m, 4)
    hit = np.nonzero(dm)[0]
    assert list(hit) == [case["index"]]
    assert dm[case["index"]] == np.float16(1.5).view(np.uint16)
    nz = np.nonzero(codes)[0]
    assert list(nz // 16) == [case["index"]]


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_tile_pack_is_a_bijection(bits):
    S, R, C = 2, 32, 256
    nb = C // 32
    ident = np.arange(S * R * nb).reshape(S, R, nb)
    # encode each block's identity in d (exact in fp16 below 2048) and m
    d = (ident % 2048).astype(np.float16)
    m = (ident // 2048).astype(np.float16)
    q = np.zeros((S, R, C), np.uint8)
    _, dm = O.pack_tiles(q, d, m, bits)
    got = (dm & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.int64) + \
        2048 * ((dm >> 16).astype(np.uint16).view(np.float16).astype(np.int64))
    assert sorted(got.tolist()) == list(range(S * R * nb))


# ------------------------------------------------------------------ MXFP4

def _mx_case_x(case):
    x = np.zeros(32, np.float64)
    x[:len(case["x_head"])] = case["x_head"]
    return x


@pytest.mark.parametrize("case", _load("mx_blocks.json")["cases"], ids=lambda c: c["name"])
def test_mx_hand_blocks(case):
    x = _mx_case_x(case).astype(np.float32)            # 0.3, -0.2: their float32 values
    blk = O.quantise_rows_mx(x[None, :])
    assert int(blk.e[0, 0]) == case["e"]
    want_q = np.zeros(32, np.uint8)
    want_q[:len(case["q_head"])] = case["q_head"]
    np.testing.assert_array_equal(blk.q[0], want_q)
    for act in ("f32", "bf16"):
        v = O.dequantise_mx(blk.e, blk.q, act)[0]
        if case.get("lossless"):
            np.testing.assert_array_equal(v, x.astype(np.float64))
        if "deq_head" in case:
            np.testing.assert_array_equal(v[:len(case["deq_head"])], case["deq_head"])


def test_e2m1_values_from_bit_fields():
    # each code read as sign | 2 exponent bits (bias 1) | 1 mantissa bit, with
    # exponent field 0 subnormal: value = 2^(1-1) * mantissa/2
    for code in range(16):
        s, ef, mf = code >> 3, (code >> 1) & 3, code & 1
        mag = Fraction(mf, 2) if ef == 0 else Fraction(2) ** (ef - 1) * (1 + Fraction(mf, 2))
        want = -mag if s else mag
        q = np.full((1, 32), code, np.uint8)
        for e in (127, 127 - 5, 127 + 9):
            got = O.dequantise_mx(np.array([[e]], np.uint8), q, "f32")[0, 0]
            assert Fraction(float(got)) == want * Fraction(2) ** (e - 127), (code, e)


def _mx_brute_block(x):
    """Scale exponent and codes of one block by search: X is the integer
    with 4 * 2^X <= max|x| < 8 * 2^X (walked by doubling); each element takes
    the grid value of smallest exact distance, ties to the even mantissa."""
    amax = max(abs(Fraction(float(v))) for v in x)
    if amax == 0:
        X = -125
    else:
        X = 0
        while Fraction(4) * Fraction(2) ** X > amax:
            X -= 1
        while Fraction(8) * Fraction(2) ** X <= amax:
            X += 1
        X = min(max(X, -125), 125)
    grid = [(c, (Fraction(-1) if c & 8 else Fraction(1)) * m)
            for c, m in enumerate([Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
                                   Fraction(2), Fraction(3), Fraction(4), Fraction(6)] * 2)]
    codes = []
    for v in x:
        t = Fraction(float(v)) / Fraction(2) ** X
        if t > 6:
            codes.append(7)
            continue
        if t < -6:
            codes.append(15)
            continue
        best = min(abs(t - g) for _, g in grid)
        cands = [c for c, g in grid if abs(t - g) == best]
        if any(((c >> 1) & 3) == 0 and (c & 1) == 0 for c in cands):
            codes.append(0)                       # zero: the positive code
            continue
        even = [c for c in cands if c & 1 == 0]
        codes.append((even or cands)[0])
    return X + 127, codes


def test_mx_quantiser_brute_force():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((12, 64)) * np.exp(rng.uniform(-8, 4, (12, 1)))).astype(np.float32)
    # plant exact grid points and ties in a few blocks
    w[0, :8] = np.array([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25], np.float32) * np.float32(2.0 ** -4)
    w[1, 32:36] = np.float32(0.0)
    blk = O.quantise_rows_mx(w)
    for r in range(12):
        for b in range(2):
            e, codes = _mx_brute_block(w[r, 32 * b:32 * b + 32])
            assert int(blk.e[r, b]) == e, (r, b)
            np.testing.assert_array_equal(blk.q[r, 32 * b:32 * b + 32], codes, err_msg=f"{r},{b}")


def test_mx_reconstruction_bound():
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 2, (64, 1)))).astype(np.float32)
    blk = O.quantise_rows_mx(w)
    v = O.dequantise_mx(blk.e, blk.q, "f32").reshape(64, -1, 32)
    x = w.astype(np.float64).reshape(64, -1, 32)
    scale = np.ldexp(1.0, blk.e.astype(np.int64) - 127)[..., None]
    t = np.abs(x) / scale
    assert np.all(t < 8) and np.all(t.max(-1) >= 4)
    # half the gap of the binade below 6; above 6 the error is t - 6 < 2
    half_gap = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    err = np.abs(x - v) / scale
    assert np.all(err <= np.maximum(half_gap, t - 6))
    # signs kept, magnitudes never grow past the input's saturation point
    assert np.all((v == 0) | (np.sign(v) == np.sign(x)))


def test_mx_field_hand_words_and_layout():
    case = _load("mx_blocks.json")["field"]
    k = np.arange(32)
    q = np.where(k < 16, k % 16, 31 - k).astype(np.uint8)
    field = O.encode_codes(q, O.MXFP4)
    assert field.size == 16
    assert [f"0x{int(w):08X}" for w in field.view("<u4")] == case["words"]
    np.testing.assert_array_equal(O.decode_codes(field, O.MXFP4), q)
    pos = O.code_bit_positions(O.MXFP4)
    assert sorted(p for c in pos for p in c) == list(range(128))
    for kk in range(32):
        one = np.zeros(32, np.uint8)
        one[kk] = 15
        as_int = int.from_bytes(O.encode_codes(one, O.MXFP4).tobytes(), "little")
        assert as_int == 15 << (4 * kk)


@pytest.mark.parametrize("case", _load("tile_index.json")["cases"])
def test_mx_tile_index_hand(case):
    S, R, C = case["S"], case["R"], case["C"]
    q = np.zeros((S, R, C), np.uint8)
    e = np.zeros((S, R, C // 32), np.uint8)
    e[case["s"], case["r"], case["j"]] = 200
    q[case["s"], case["r"], 32 * case["j"] + 1] = 9
    codes, sc = O.pack_tiles_mx(q, e)
    assert list(np.nonzero(sc)[0]) == [case["index"]]
    assert sc[case["index"]] == 200
    nz = np.nonzero(codes)[0]
    assert list(nz) == [16 * case["index"]]       # code 1: high nibble of byte 0
    assert codes[16 * case["index"]] == 9 << 4


def test_mx_tile_pack_is_a_bijection():
    S, R, C = 2, 32, 128
    nb = C // 32
    ident = np.arange(S * R * nb).reshape(S, R, nb)
    assert ident.max() < 256
    _, sc = O.pack_tiles_mx(np.zeros((S, R, C), np.uint8), ident.astype(np.uint8))
    assert sorted(sc.tolist()) == list(range(S * R * nb))


def test_mx_table_bytes_and_planner_scope():
    # 16 code bytes + 1 scale byte per 32 weights: 4.25 bits per weight
    assert O.expert_table_bytes(2048, 512, O.MXFP4) == 3 * 2048 * 512 * 17 // 32
    assert O.expert_table_bytes(2048, 512, O.MXFP4) * 20 == O.expert_table_bytes(2048, 512, 4) * 17
    with pytest.raises(ValueError):
        O.plan_tiers(np.ones(4, np.uint64), (4, 3, O.MXFP4), 128, 64, 1 << 30)


def test_layer_mx_down_equals_affine_container():
    # MXFP4 codes of magnitude <= 1.5 at scale 2^0 take the values -1.5..1.5 in
    # steps of 0.5, which the affine 4-bit block d = 0.5, m = -1.5 also holds
    # exactly: the same down matrices in either container give the same layer
    layer, blocks = _random_layer(E=4, K=2, H=128, I=64, act="bf16", seed=23, bits=4)
    rng = np.random.default_rng(24)
    x = O.act_round(rng.standard_normal((3, 128)), "bf16")
    mx = {}
    aff = {}
    for e, b in blocks.items():
        mag = rng.integers(0, 4, (128, 64))
        neg = rng.integers(0, 2, (128, 64)).astype(bool) & (mag > 0)
        qmx = (mag + 8 * neg).astype(np.uint8)
        val = np.where(neg, -0.5 * mag, 0.5 * mag)
        qa = (val / 0.5 + 3).astype(np.uint8)          # value = 0.5 * qa - 1.5
        d = np.full((128, 2), 0.5, np.float16)
        m = np.full((128, 2), -1.5, np.float16)
        mx[e] = O.ExpertBlocks(b.bits, b.gate, b.up, O.MxBlocks(np.full((128, 2), 127, np.uint8), qmx))
        aff[e] = O.ExpertBlocks(b.bits, b.gate, b.up, (d, m, qa))
    layer.experts = lambda e: mx[e]
    layer._cache.clear()
    y_mx = O.moe_layer(x, layer)["y"]
    layer.experts = lambda e: aff[e]
    layer._cache.clear()
    np.testing.assert_array_equal(O.moe_layer(x, layer)["y"], y_mx)


# ------------------------------------------------------------------ tiers

def _brute_tiers(pop, n_slots):
    E = len(pop)
    tm = []
    for e in range(E):
        rank = sum(1 for f in range(E) if pop[f] > pop[e] or (pop[f] == pop[e] and f < e))
        if rank < n_slots[0]:
            tm.append((0, rank))
        elif rank < n_slots[0] + n_slots[1]:
            tm.append((1, rank - n_slots[0]))
        else:
            tm.append((2, rank - n_slots[0] - n_slots[1]))
    return tm


def test_tiers_brute_force():
    rng = np.random.default_rng(4)
    for E, ns in ((8, (2, 4, 2)), (13, (3, 7, 3)), (64, (16, 32, 16)), (5, (5, 0, 0))):
        pop = rng.integers(0, 4, E).astype(np.uint64)      # many ties
        tm, se = O.build_tiers(pop, ns)
        want = _brute_tiers(pop.tolist(), ns)
        assert [(int(v) >> 16, int(v) & 0xFFFF) for v in tm] == want
        # slot_expert inverts the ranking
        for e in range(E):
            tier, slot = want[e]
            assert se[[0, ns[0], ns[0] + ns[1]][tier] + slot] == e


def test_tiers_uniform_popularity_identity():
    tm, se = O.build_tiers(np.zeros(64, np.uint64), (64, 0, 0))
    assert tm.tolist() == list(range(64))
    assert se.tolist() == list(range(64))


def test_tiers_reject_bad_counts():
    with pytest.raises(ValueError):
        O.build_tiers(np.zeros(8, np.uint64), (2, 2, 2))


# ----------------------------------------------------------------- tier planner

def test_expert_table_bytes_closed_form():
    # 3 matrices of 2048 x 512 weights in blocks of 32: 98304 blocks, each
    # 4*bits bytes of codes and 4 bytes of (d, m)
    assert O.expert_table_bytes(2048, 512, 4) == 98304 * 20
    assert O.expert_table_bytes(2048, 512, 3) == 98304 * 16
    assert O.expert_table_bytes(2048, 512, 2) == 98304 * 12
    # the full-size layer's tiers of 128 / 256 / 128 experts: exactly 768 MiB
    total = (128 * O.expert_table_bytes(2048, 512, 4) + 256 * O.expert_table_bytes(2048, 512, 3)
             + 128 * O.expert_table_bytes(2048, 512, 2))
    assert total == 768 * 2**20


def _werr(b):
    # the error model written out: mean square error of a uniform b-bit
    # quantiser over a unit range, up to the common factor 1/12
    return Fraction(1, (2**b - 1) ** 2)


def _plan_cost(pop, tiers_of_rank_order, bits):
    return sum(int(p) * _werr(bits[t]) for p, t in zip(pop, tiers_of_rank_order))


def test_plan_budget_extremes():
    pop = np.array([5, 0, 9, 9, 1, 3], np.uint64)
    c = [O.expert_table_bytes(256, 128, b) for b in (4, 3, 2)]
    E = len(pop)
    assert O.plan_tiers(pop, (4, 3, 2), 256, 128, E * c[0]) == (E, 0, 0)
    assert O.plan_tiers(pop, (4, 3, 2), 256, 128, 10 * E * c[0]) == (E, 0, 0)
    assert O.plan_tiers(pop, (4, 3, 2), 256, 128, E * c[2]) == (0, 0, E)
    with pytest.raises(ValueError):
        O.plan_tiers(pop, (4, 3, 2), 256, 128, E * c[2] - 1)


@pytest.mark.parametrize("bits", [(4, 3, 2), (4, 4, 2), (3, 4, 2), (2, 2, 4)])
def test_plan_brute_force_every_assignment(bits):
    # independent search over every assignment of the E experts to the three
    # tiers (3^E).  Among those whose tier index never decreases down the
    # popularity order (band plans), the planner's plan has the least error,
    # and the most experts in tier 0, then in tier 1, among equals.  When the
    # widths do not increase down the tiers, no assignment at all beats it
    # (swapping a hotter and a colder expert's widths never hurts).
    import itertools
    rng = np.random.default_rng(5)
    H, I = 128, 128
    c = [O.expert_table_bytes(H, I, b) for b in bits]
    for trial in range(12):
        E = int(rng.integers(1, 7))
        pop = rng.integers(0, 6, size=E).astype(np.uint64)       # ties and zeros
        lo, hi = E * min(c), E * max(c)
        budget = int(rng.integers(lo, hi + 1))
        n = O.plan_tiers(pop, bits, H, I, budget)
        assert sum(n) == E and n[0] * c[0] + n[1] * c[1] + n[2] * c[2] <= budget
        order = sorted(range(E), key=lambda e: (-int(pop[e]), e))
        best_any = best_band = None
        for assign in itertools.product(range(3), repeat=E):
            if sum(c[t] for t in assign) > budget:
                continue
            err = sum(int(pop[e]) * _werr(bits[t]) for e, t in enumerate(assign))
            best_any = err if best_any is None else min(best_any, err)
            ranked = [assign[e] for e in order]
            if all(ranked[i] <= ranked[i + 1] for i in range(E - 1)):
                key = (err, -ranked.count(0), -ranked.count(1))
                if best_band is None or key < best_band[0]:
                    best_band = (key, (ranked.count(0), ranked.count(1), ranked.count(2)))
        assert tuple(n) == best_band[1]
        if bits[0] >= bits[1] >= bits[2]:
            bands = [0] * n[0] + [1] * n[1] + [2] * n[2]
            assert _plan_cost([pop[e] for e in order], bands, bits) == best_any


@pytest.mark.parametrize("bits,down", [((4, 3, 2), (4, 4, 3)), ((3, 3, 2), (4, 2, 4)),
                                       ((4, 3, 2), (0, 4, 0))])
def test_plan_ladder_brute_force_every_assignment(bits, down):
    # with a down ladder an expert of tier t stores gate and up at bits[t] and
    # down at its own width: costs and errors are counted per matrix here, by
    # a search over every assignment restricted to band plans
    import itertools
    rng = np.random.default_rng(8)
    H, I = 128, 256
    dn = [d if d else b for b, d in zip(bits, down)]
    # bytes of one matrix (H*I/32 blocks) at b bits, from the block size
    mat = {b: H * I // 32 * (4 * b + 4) for b in (2, 3, 4)}
    c = [2 * mat[b] + mat[d] for b, d in zip(bits, dn)]
    for trial in range(12):
        E = int(rng.integers(1, 7))
        pop = rng.integers(0, 6, size=E).astype(np.uint64)
        budget = int(rng.integers(E * min(c), E * max(c) + 1))
        n = O.plan_tiers(pop, bits, H, I, budget, down_bits=down)
        assert sum(n) == E and n[0] * c[0] + n[1] * c[1] + n[2] * c[2] <= budget
        order = sorted(range(E), key=lambda e: (-int(pop[e]), e))
        best_band = None
        for assign in itertools.product(range(3), repeat=E):
            ranked = [assign[e] for e in order]
            if sum(c[t] for t in assign) > budget or any(ranked[i] > ranked[i + 1] for i in range(E - 1)):
                continue
            err = sum(int(pop[e]) * (2 * _werr(bits[t]) + _werr(dn[t])) for e, t in enumerate(assign))
            key = (err, -ranked.count(0), -ranked.count(1))
            if best_band is None or key < best_band[0]:
                best_band = (key, (ranked.count(0), ranked.count(1), ranked.count(2)))
        assert tuple(n) == best_band[1]
    # without a ladder the plan is the single-width plan
    pop = rng.integers(0, 9, size=9).astype(np.uint64)
    budget = 9 * O.expert_table_bytes(H, I, 3)
    assert O.plan_tiers(pop, bits, H, I, budget, down_bits=(0, 0, 0)) == O.plan_tiers(pop, bits, H, I, budget)


def _greedy(pop, bits, H, I, budget):
    # the pages' planner: start every expert at the cheapest width, then keep
    # spending bytes on the single upgrade (one expert, next wider width) that
    # removes the most expected error per byte, while it fits
    widths = sorted(set(bits))
    cost = {b: O.expert_table_bytes(H, I, b) for b in widths}
    cur = [widths[0]] * len(pop)
    spent = cost[widths[0]] * len(pop)
    if spent > budget:
        return None
    while True:
        best = None
        for e, b in enumerate(cur):
            k = widths.index(b)
            if k + 1 == len(widths):
                continue
            nb = widths[k + 1]
            extra = cost[nb] - cost[b]
            if spent + extra > budget:
                continue
            gain = int(pop[e]) * (_werr(b) - _werr(nb)) / extra
            key = (gain, int(pop[e]), -e)
            if best is None or key > best[0]:
                best = (key, e, nb, extra)
        if best is None or best[0][0] == 0:
            return cur
        _, e, nb, extra = best
        cur[e] = nb
        spent += extra


def test_plan_never_worse_than_the_greedy():
    rng = np.random.default_rng(6)
    H, I = 128, 256
    bits = (4, 3, 2)
    c = [O.expert_table_bytes(H, I, b) for b in bits]
    for trial in range(20):
        E = int(rng.integers(2, 40))
        pop = rng.zipf(1.6, size=E).astype(np.uint64)
        budget = int(rng.integers(E * c[2], E * c[0] + 1))
        n = O.plan_tiers(pop, bits, H, I, budget)
        order = sorted(range(E), key=lambda e: (-int(pop[e]), e))
        plan = _plan_cost([pop[e] for e in order], [0] * n[0] + [1] * n[1] + [2] * n[2], bits)
        g = _greedy(pop, bits, H, I, budget)
        gerr = sum(int(pop[e]) * _werr(b) for e, b in enumerate(g))
        assert plan <= gerr
        # the greedy's widths never increase down the popularity order
        gw = [g[e] for e in order]
        assert all(gw[i] >= gw[i + 1] for i in range(E - 1))


def test_plan_more_budget_never_worse():
    rng = np.random.default_rng(7)
    pop = rng.zipf(1.4, size=30).astype(np.uint64)
    bits = (4, 3, 2)
    c = [O.expert_table_bytes(128, 128, b) for b in bits]
    order = sorted(range(30), key=lambda e: (-int(pop[e]), e))
    prev = None
    for budget in range(30 * c[2], 30 * c[0] + 1, (c[0] - c[2]) // 3):
        n = O.plan_tiers(pop, bits, 128, 128, budget)
        err = _plan_cost([pop[e] for e in order], [0] * n[0] + [1] * n[1] + [2] * n[2], bits)
        assert prev is None or err <= prev
        prev = err


# ----------------------------------------------------------------- router

def test_router_keys_exact_vs_fp64():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64)).astype(np.float32).astype(np.float64)
    w = (rng.standard_normal((6, 64)) * 0.02).astype(np.float32).astype(np.float64)
    b = rng.standard_normal(6).astype(np.float32).astype(np.float64)
    exact = O.router_keys(x, w, b, exact=True)
    fast = O.router_keys(x, w, b)
    np.testing.assert_allclose(fast, exact, rtol=0, atol=1e-14)
    # hand check of one key with exact rationals
    fr = sum(Fraction(float(a)) * Fraction(float(c)) for a, c in zip(x[1], w[4])) + Fraction(float(b[4]))
    assert exact[1, 4] == float(fr)


def _brute_topk(keys_row, k):
    E = len(keys_row)

    def better(a, b):           # is expert a ranked before expert b?
        ka, kb = keys_row[a], keys_row[b]
        if math.isnan(kb) and not math.isnan(ka):
            return True
        if math.isnan(ka):
            return math.isnan(kb) and a < b
        return ka > kb or (ka == kb and a < b)

    rank = {e: sum(1 for f in range(E) if f != e and better(f, e)) for e in range(E)}
    return [e for e, _ in sorted(rank.items(), key=lambda kv: kv[1])][:k]


def test_topk_brute_force_with_ties_and_nan():
    rng = np.random.default_rng(6)
    for trial in range(200):
        E = int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        keys = rng.integers(-3, 3, E).astype(np.float64)     # many exact ties
        if trial % 5 == 0:
            keys[rng.integers(0, E)] = np.nan
        if trial % 7 == 0:
            keys[rng.integers(0, E)] = -0.0
        got = O.select_topk(keys[None, :], k)[0].tolist()
        assert got == _brute_topk(keys.tolist(), k), (keys, k)


def test_duplicated_router_rows_tie_to_lower_id():
    rng = np.random.default_rng(7)
    H, E = 64, 8
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32).astype(np.float64)
    w[5] = w[2]                      # identical rows -> identical exact keys
    w[6] = w[2]
    x = rng.standard_normal((4, H)).astype(np.float32).astype(np.float64)
    # make experts 2/5/6 the best by scaling
    w[[2, 5, 6]] *= 50
    keys = O.router_keys(x, w, None, exact=True)
    assert np.all(keys[:, 2] == keys[:, 5]) and np.all(keys[:, 2] == keys[:, 6])
    ids = O.select_topk(keys, 3)
    for t in range(4):
        if keys[t, 2] > np.max(np.delete(keys[t], [2, 5, 6])):
            assert ids[t].tolist() == [2, 5, 6]


def test_gate_weights_invariants():
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((50, 32)) * 3
    for k in (1, 2, 10, 32):
        ids = O.select_topk(keys, k)
        g = O.gate_weights(keys, ids)
        assert np.all(np.abs(g.sum(1) - 1) <= 1e-15)
        assert np.all(np.diff(g, axis=1) <= 0)        # rank order -> non-increasing weights
        if k == 1:
            assert np.all(g == 1.0)
        if k == 32:
            assert np.all(np.sort(ids, 1) == np.arange(32))
    # closed form for two experts: g0 = 1/(1+e^(k1-k0))
    kk = np.array([[0.25, 1.5, -2.0]])
    ids = O.select_topk(kk, 2)
    g = O.gate_weights(kk, ids)
    assert ids.tolist() == [[1, 0]]
    assert abs(g[0, 0] - 1 / (1 + math.exp(0.25 - 1.5))) < 1e-15


# ------------------------------------------------------------------- sort

def test_sort_routes_vs_lexsort_and_brute_force():
    rng = np.random.default_rng(9)
    for T, K, E in ((1, 1, 1), (7, 3, 5), (64, 4, 64), (300, 10, 512)):
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        off, sr = O.sort_routes(ids, E)
        flat = ids.reshape(-1)
        want = np.lexsort((np.arange(flat.size), flat))
        np.testing.assert_array_equal(sr, want)
        assert off[0] == 0 and off[-1] == T * K and np.all(np.diff(off) >= 0)
        for e in range(0, E, max(1, E // 17)):
            bucket = sr[off[e]:off[e + 1]]
            assert np.all(flat[bucket] == e) and np.all(np.diff(bucket) > 0)
            assert off[e] == int(np.sum(flat < e))


# ------------------------------------------------------------------ layer

def _const_block(rows, cols, q_val, d_val):
    return (np.full((rows, cols // 32), d_val, np.float16),
            np.zeros((rows, cols // 32), np.float16),
            np.full((rows, cols), q_val, np.uint8))


def _closed_form_layer():
    H, I = 64, 32
    w_router = np.zeros((2, H))
    w_router[0] = 2.0 ** -7
    w_router[1] = 2.0 ** -6

    def experts(e):
        return O.ExpertBlocks(
            bits=4,
            gate=_const_block(I, H, 1, 0.5),
            up=_const_block(I, H, 1, 0.25),
            down=_const_block(H, I, 1, 0.125 if e == 0 else 0.0625))

    shared = (np.full((I, H), 2.0 ** -5), np.full((I, H), 2.0 ** -6), np.full((H, I), 2.0 ** -5))
    return O.OracleLayer(act="bf16", w_router=w_router, bias=None, top_k=2,
                         experts=experts, shared=shared)


def test_layer_closed_form():
    spec = _load("layer_closed_form.json")
    layer = _closed_form_layer()
    x = np.stack([np.ones(64), 2 * np.ones(64)])
    out = O.moe_layer(x, layer, exact_keys=True)
    assert out["ids"].tolist() == [spec["ids"], spec["ids"]]
    # token 0 (x = 1): y = 1024 (1 + 1/(1 + e^0.5)) + 225/128
    y0 = 1024 * (1 + 1 / (1 + math.exp(0.5))) + 225 / 128
    # token 1 (x = 2): keys 2.0, 1.0; h = bf16(silu(64)*32) = 2048; routed outs
    # 8192 and 4096; shared h_s = bf16(2*4/(1+e^-4)) = 251/32
    y1 = 4096 * (1 + 1 / (1 + math.exp(1.0))) + 251 / 32
    np.testing.assert_allclose(out["y"][0], y0, rtol=1e-15)
    np.testing.assert_allclose(out["y"][1], y1, rtol=1e-15)


def _random_layer(E, K, H, I, act, seed, shared=True, bits=4):
    rng = np.random.default_rng(seed)
    w_router = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    w_router = O.bf16_round(w_router) if act == "bf16" else w_router
    blocks = {}
    for e in range(E):
        mats = []
        for rows, cols in ((I, H), (I, H), (H, I)):
            w = (rng.standard_normal((rows, cols)) / np.sqrt(cols)).astype(np.float32)
            mats.append(O.quantise_rows(w, bits))
        blocks[e] = O.ExpertBlocks(bits, *mats)
    sh = None
    if shared:
        sh = tuple(O.act_round(rng.standard_normal((r, c)) / np.sqrt(c), act)
                   for r, c in ((I, H), (I, H), (H, I)))
    return O.OracleLayer(act=act, w_router=w_router.astype(np.float64), bias=None, top_k=K,
                         experts=lambda e: blocks[e], shared=sh), blocks


def test_layer_single_expert_is_dense_swiglu():
    layer, blocks = _random_layer(E=1, K=1, H=128, I=64, act="bf16", seed=10, shared=False)
    rng = np.random.default_rng(11)
    x = O.act_round(rng.standard_normal((5, 128)), "bf16")
    y = O.moe_layer(x, layer)["y"]
    gw, uw, dw = (O.dequantise(*m, act="bf16") for m in (blocks[0].gate, blocks[0].up, blocks[0].down))
    g = np.matmul(x, gw.T)
    u = np.matmul(x, uw.T)
    h = O.act_round(g / (1 + np.exp(-g)) * u, "bf16")
    np.testing.assert_allclose(y, np.matmul(h, dw.T), rtol=1e-13, atol=1e-13)


def test_layer_zero_input():
    layer, _ = _random_layer(E=6, K=2, H=128, I=64, act="bf16", seed=12)
    layer.bias = np.linspace(-1, 1, 6)
    out = O.moe_layer(np.zeros((3, 128)), layer)
    np.testing.assert_array_equal(out["keys"], np.tile(layer.bias, (3, 1)))
    assert out["ids"].tolist() == [[5, 4]] * 3
    np.testing.assert_array_equal(out["y"], 0.0)


def test_layer_identical_experts_independent_of_routing():
    layer, blocks = _random_layer(E=5, K=3, H=128, I=64, act="bf16", seed=13)
    same = blocks[0]
    layer.experts = lambda e: same
    layer._cache.clear()
    rng = np.random.default_rng(14)
    x = O.act_round(rng.standard_normal((4, 128)), "bf16")
    y = O.moe_layer(x, layer)["y"]
    gw, uw, dw = (O.dequantise(*m, act="bf16") for m in (same.gate, same.up, same.down))
    _, out = O.expert_ffn(x, gw, uw, dw, "bf16")
    _, out_s = O.expert_ffn(x, *layer.shared, act="bf16")
    np.testing.assert_allclose(y, out + out_s, rtol=1e-12, atol=1e-12)


def test_layer_two_bit_codes_in_four_bit_container():
    # 2-bit codes are valid 4-bit codes: storing them in the 4-bit tier with the
    # same d and m must give the same layer output
    layer, blocks = _random_layer(E=4, K=2, H=128, I=64, act="bf16", seed=15, bits=2)
    rng = np.random.default_rng(16)
    x = O.act_round(rng.standard_normal((3, 128)), "bf16")
    y2 = O.moe_layer(x, layer)["y"]
    # round-trip the codes through the 4-bit field
    def widen(mat):
        d, m, q = mat
        f = O.encode_codes(q.reshape(q.shape[0], -1, 32), 4)
        return d, m, O.decode_codes(f, 4).reshape(q.shape)
    wide = {e: O.ExpertBlocks(4, widen(b.gate), widen(b.up), widen(b.down)) for e, b in blocks.items()}
    layer.experts = lambda e: wide[e]
    layer._cache.clear()
    np.testing.assert_array_equal(O.moe_layer(x, layer)["y"], y2)


def test_layer_relabelling_invariance():
    layer, blocks = _random_layer(E=7, K=3, H=128, I=64, act="bf16", seed=17)
    rng = np.random.default_rng(18)
    x = O.act_round(rng.standard_normal((6, 128)), "bf16")
    layer.bias = rng.standard_normal(7)
    y = O.moe_layer(x, layer)["y"]
    perm = rng.permutation(7)                 # new id j holds old expert perm[j]
    layer2 = O.OracleLayer(act="bf16", w_router=layer.w_router[perm], bias=layer.bias[perm],
                           top_k=3, experts=lambda j: blocks[int(perm[j])], shared=layer.shared)
    out2 = O.moe_layer(x, layer2)
    np.testing.assert_allclose(out2["y"], y, rtol=1e-12, atol=1e-12)
    ids1 = O.moe_layer(x, layer)["ids"]
    np.testing.assert_array_equal(perm[out2["ids"]], ids1)


def test_output_cast_is_one_rounding():
    y = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, -3.0000001, 0.0, 1e-3])
    got = O.output_cast(y, "bf16")
    for v, g in zip(y, got):
        assert Fraction(float(g)) == _bf16_exact(Fraction(float(v)))
    np.testing.assert_array_equal(O.output_cast(y, "f32"), y.astype(np.float32).astype(np.float64))
