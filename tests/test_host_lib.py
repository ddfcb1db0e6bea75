"""CPU tests of the C-ABI library: symbols, validation, workspace queries and
the host tier build, bit-exact against the oracle.  No GPU is needed: these
paths make no HIP call (moe_build_tiers with host destinations, argument
validation, ws == NULL size queries)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import synth
import quantized_expert_ffn_route_amd as M

from conftest import ROOT

pytestmark = pytest.mark.skipif(not os.path.exists(M.library_path()),
                                reason="libmoe.so not built (run __graft_entry__.build())")


def _header_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_exports_every_header_symbol():
    names = _header_functions()
    assert {"moe_route", "moe_build_tiers", "moe_forward_decode", "moe_forward_prefill"} <= set(names)
    lib = ctypes.CDLL(M.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (M.MOE_OK, M.MOE_EINVAL, M.MOE_EUNSUPPORTED, M.MOE_ENOSPC, M.MOE_EHIP):
        assert M.status_string(s).startswith("MOE_")


def test_tier_table_bytes_closed_form():
    d = M.dims(2048, 512, 512, 10, True, "bf16")
    # one expert's three matrices: 3 * 2048 * 512 weights = 98304 blocks
    per_expert = {b: sum(M.tier_table_bytes(d, b, 1, m, w) for m in range(3) for w in range(2))
                  for b in (4, 3, 2)}
    assert per_expert == {4: 1966080, 3: 1572864, 2: 1179648}
    full = sum(M.tier_table_bytes(d, b, n, m, w) for b, n in ((4, 128), (3, 256), (2, 128))
               for m in range(3) for w in range(2))
    assert full == 768 * 2 ** 20
    assert M.tier_table_bytes(d, 5, 1, 0, 0) == 0


def _fake_layer(d, n_slots=(1, 0, 0), tier_bits=(4, 3, 2)):
    """A layer struct whose pointers are non-null and aligned (never dereferenced)."""
    L = M.MoeLayer()
    fake = 1 << 20
    L.w_router = fake
    L.tier_map = fake
    L.n_slots = (ctypes.c_int32 * 3)(*n_slots)
    L.tier_bits = (ctypes.c_int32 * 3)(*tier_bits)
    for t in range(3):
        for m in range(3):
            L.codes[t][m] = fake
            L.dm[t][m] = fake
    for m in range(3):
        L.w_shared[m] = fake
    return L


def _status(fn, *args):
    return fn(*args)


def test_validation_errors_without_gpu():
    lib = M.lib()
    n = ctypes.c_size_t(0)

    def route(d, L, T=4):
        return lib.moe_route(ctypes.byref(d), ctypes.byref(L), None, T, None, None, None,
                             ctypes.byref(n), None)

    ok = M.dims(256, 128, 64, 4, False, "f32")
    assert route(ok, _fake_layer(ok, (64, 0, 0))) == M.MOE_OK and n.value > 0
    # H not a multiple of 128 / K > E / K > 64 / E > 65535 / bad act
    assert route(M.dims(96, 128, 64, 4, False, "f32"), _fake_layer(ok, (64, 0, 0))) == M.MOE_EUNSUPPORTED
    assert route(M.dims(256, 128, 4, 5, False, "f32"), _fake_layer(ok, (4, 0, 0))) == M.MOE_EINVAL
    assert route(M.dims(256, 128, 128, 65, False, "f32"), _fake_layer(ok, (128, 0, 0))) == M.MOE_EINVAL
    assert route(M.dims(256, 128, 70000, 4, False, "f32"), _fake_layer(ok, (70000, 0, 0))) == M.MOE_EINVAL
    bad_act = M.dims(256, 128, 64, 4, False, "f32")
    bad_act.act = 7
    assert route(bad_act, _fake_layer(ok, (64, 0, 0))) == M.MOE_EINVAL
    # tier counts must sum to E, widths must be 2..4
    assert route(ok, _fake_layer(ok, (32, 0, 0))) == M.MOE_EINVAL
    assert route(ok, _fake_layer(ok, (32, 32, 0), (4, 5, 2))) == M.MOE_EINVAL
    # null / misaligned table pointers
    L = _fake_layer(ok, (64, 0, 0))
    L.codes[0][1] = None
    assert route(ok, L) == M.MOE_EINVAL
    L = _fake_layer(ok, (64, 0, 0))
    L.dm[0][2] = (1 << 20) + 4
    assert route(ok, L) == M.MOE_EINVAL
    # shared expert required when has_shared
    sh = M.dims(256, 128, 64, 4, True, "f32")
    L = _fake_layer(sh, (64, 0, 0))
    L.w_shared[1] = None
    assert route(sh, L) == M.MOE_EINVAL
    # negative T; T == 0 still answers the size query
    assert route(ok, _fake_layer(ok, (64, 0, 0)), T=-1) == M.MOE_EINVAL
    assert route(ok, _fake_layer(ok, (64, 0, 0)), T=0) == M.MOE_OK


def test_forward_argument_checks_without_gpu():
    lib = M.lib()
    d = M.dims(256, 128, 64, 4, False, "f32")
    L = _fake_layer(d, (64, 0, 0))
    n = ctypes.c_size_t(0)
    # size query
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), None, 8, None, M.MOE_F32, None,
                                  None, None, ctypes.byref(n), None) == M.MOE_OK
    dec = n.value
    assert dec > 0
    # bf16 output requires bf16 activations
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), None, 8, None, M.MOE_BF16, None,
                                  None, None, ctypes.byref(n), None) == M.MOE_EINVAL
    # too small a workspace, misaligned workspace, null ws_bytes
    fake_ws = 1 << 24
    small = ctypes.c_size_t(dec - 1)
    x = y = 1 << 22
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), x, 8, y, M.MOE_F32, None, None,
                                  fake_ws, ctypes.byref(small), None) == M.MOE_ENOSPC
    big = ctypes.c_size_t(dec)
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), x, 8, y, M.MOE_F32, None, None,
                                  fake_ws + 16, ctypes.byref(big), None) == M.MOE_EINVAL
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), x, 8, y, M.MOE_F32, None, None,
                                  fake_ws, None, None) == M.MOE_EINVAL
    # misaligned x
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), x + 2, 8, y, M.MOE_F32, None,
                                  None, fake_ws, ctypes.byref(big), None) == M.MOE_EINVAL
    # prefill: size grows with T, E > 4096 unsupported
    s1, s2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.moe_forward_prefill(ctypes.byref(d), ctypes.byref(L), None, 64, None, M.MOE_F32, None,
                                   None, None, None, None, ctypes.byref(s1), None) == M.MOE_OK
    assert lib.moe_forward_prefill(ctypes.byref(d), ctypes.byref(L), None, 4096, None, M.MOE_F32,
                                   None, None, None, None, None, ctypes.byref(s2), None) == M.MOE_OK
    assert s2.value > s1.value
    dbig = M.dims(256, 128, 5000, 4, False, "f32")
    Lb = _fake_layer(dbig, (5000, 0, 0))
    assert lib.moe_forward_prefill(ctypes.byref(dbig), ctypes.byref(Lb), None, 64, None, M.MOE_F32,
                                   None, None, None, None, None, ctypes.byref(s1), None) == M.MOE_EUNSUPPORTED


def test_prefill_rejects_gathers_beyond_32_bit_offsets():
    # the routed GEMMs gather x rows (T * H elements) and h rows (T * K * I
    # elements) with 32-bit element offsets: at or above 2^31 the call is
    # refused before any launch, also for a workspace-size query
    lib = M.lib()
    n = ctypes.c_size_t(0)

    def query(d, T):
        L = _fake_layer(d, (d.n_experts, 0, 0))
        return lib.moe_forward_prefill(ctypes.byref(d), ctypes.byref(L), None, T, None, M.MOE_F32,
                                       None, None, None, None, None, ctypes.byref(n), None)
    full = M.dims(2048, 512, 512, 10, True, "bf16")
    # T * K * I: 419430 * 10 * 512 = 2147481600 < 2^31 <= 419431 * 5120
    assert query(full, 419430) == M.MOE_OK
    assert query(full, 419431) == M.MOE_EUNSUPPORTED
    # T * H: with K = 1 and a narrow I, the x gather is the binding limit
    wide = M.dims(8192, 128, 64, 1, False, "bf16")
    assert query(wide, (1 << 31) // 8192 - 1) == M.MOE_OK
    assert query(wide, (1 << 31) // 8192) == M.MOE_EUNSUPPORTED


# ------------------------------------------------------------ host tier build

def _mbits(tier_bits, down_bits, t, m):
    return down_bits[t] if down_bits is not None and m == M.MOE_DOWN and down_bits[t] else tier_bits[t]


def _host_tables(d, n_slots, tier_bits, down_bits=None):
    codes = [[None] * 3 for _ in range(3)]
    dm = [[None] * 3 for _ in range(3)]
    L = M.MoeLayer()
    L.n_slots = (ctypes.c_int32 * 3)(*n_slots)
    L.tier_bits = (ctypes.c_int32 * 3)(*tier_bits)
    if down_bits is not None:
        L.down_bits = (ctypes.c_int32 * 3)(*down_bits)
    for t in range(3):
        if n_slots[t] == 0:
            continue
        for m in range(3):
            b = _mbits(tier_bits, down_bits, t, m)
            codes[t][m] = np.zeros(M.tier_table_bytes(d, b, n_slots[t], m, M.MOE_CODES), np.uint8)
            nd = M.tier_table_bytes(d, b, n_slots[t], m, M.MOE_DM)
            # MXFP4: one scale byte per block; otherwise (d, m) words
            dm[t][m] = np.zeros(nd, np.uint8) if b == M.MOE_MXFP4 else np.zeros(nd // 4, np.uint32)
            L.codes[t][m] = codes[t][m].ctypes.data
            L.dm[t][m] = dm[t][m].ctypes.data
    return L, codes, dm


def _oracle_tables(blocks_by_expert, slot_expert, n_slots, tier_bits, down_bits=None):
    """Oracle packing of every tier table from per-expert (d, m, q)."""
    out = {}
    start = [0, n_slots[0], n_slots[0] + n_slots[1]]
    for t in range(3):
        if n_slots[t] == 0:
            continue
        for m in range(3):
            experts = [slot_expert[start[t] + s] for s in range(n_slots[t])]
            if _mbits(tier_bits, down_bits, t, m) == O.MXFP4:
                out[(t, m)] = O.pack_tiles_mx(np.stack([blocks_by_expert[e][m].q for e in experts]),
                                              np.stack([blocks_by_expert[e][m].e for e in experts]))
                continue
            q = np.stack([blocks_by_expert[e][m][2] for e in experts])
            dd = np.stack([blocks_by_expert[e][m][0] for e in experts])
            mm = np.stack([blocks_by_expert[e][m][1] for e in experts])
            out[(t, m)] = O.pack_tiles(q, dd, mm, _mbits(tier_bits, down_bits, t, m))
    return out


def test_build_tiers_map_only_matches_oracle():
    rng = np.random.default_rng(20)
    for E, ns in ((64, (64, 0, 0)), (512, (128, 256, 128)), (10, (3, 4, 3))):
        pop = rng.integers(0, 5, E).astype(np.uint64)
        d = M.dims(256, 128, E, 4, False, "f32")
        tmap, sexp = M.build_tiers(d, pop, ns, (4, 3, 2))
        want_map, want_se = O.build_tiers(pop, ns)
        np.testing.assert_array_equal(tmap, want_map)
        np.testing.assert_array_equal(sexp, want_se)


MX = 0x14     # the format code of MXFP4 tables, as the C header defines it


def _quantise(w, fmt):
    return O.quantise_rows_mx(w) if fmt == O.MXFP4 else O.quantise_rows(w, fmt)


@pytest.mark.parametrize("tier_bits,down_bits", [((4, 3, 2), None), ((2, 4, 3), None),
                                                  ((4, 3, 2), (4, 4, 3)), ((3, 3, 2), (0, 4, 0)),
                                                  ((4, 3, MX), None), ((4, 3, 2), (4, MX, MX)),
                                                  ((MX, 3, 2), (2, 0, 0))])
def test_build_tiers_f32_bit_exact_vs_oracle(tier_bits, down_bits):
    spec = synth.TINY.with_(n_experts=12, n_slots=(3, 6, 3))
    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, False, spec.act)
    gate, up, down = synth.expert_weights_f32(spec, seed=21)
    pop = np.random.default_rng(22).integers(0, 100, spec.n_experts).astype(np.uint64)
    L, codes, dm = _host_tables(d, spec.n_slots, tier_bits, down_bits)
    src = M.source_f32(gate, up, down)
    tmap, sexp = M.build_tiers(d, pop, spec.n_slots, tier_bits, src, L, dst_on_device=False)
    want_map, want_se = O.build_tiers(pop, spec.n_slots)
    np.testing.assert_array_equal(tmap, want_map)
    tier_of = {e: int(want_map[e]) >> 16 for e in range(spec.n_experts)}
    blocks = {e: [_quantise(w[e], _mbits(tier_bits, down_bits, tier_of[e], m))
                  for m, w in enumerate((gate, up, down))]
              for e in range(spec.n_experts)}
    want = _oracle_tables(blocks, want_se, spec.n_slots, tier_bits, down_bits)
    for (t, m), (wc, wd) in want.items():
        np.testing.assert_array_equal(codes[t][m], wc, err_msg=f"codes tier {t} mat {m}")
        np.testing.assert_array_equal(dm[t][m], wd, err_msg=f"dm tier {t} mat {m}")


def test_build_tiers_rounding_blocks_match_exact_derivation():
    # the library's quantiser on the golden blocks whose d, m or codes depend
    # on the rounding of one step (exact Fraction derivation): block (row 0,
    # block 0) of the gate matrix of a one-expert layer sits at table index 0
    import json
    from conftest import GOLDEN
    with open(os.path.join(GOLDEN, "quant_rounding_blocks.json")) as fh:
        cases = json.load(fh)["cases"]
    H = I = 128
    d = M.dims(H, I, 1, 1, False, "f32")
    for case in cases:
        b = case["bits"]
        rng = np.random.default_rng(40)
        mats = [rng.standard_normal((1,) + shape).astype(np.float32) for shape in ((I, H), (I, H), (H, I))]
        mats[0][0, 0, :32] = [float.fromhex(h) for h in case["x_hex"]]
        L, codes, dm = _host_tables(d, (1, 0, 0), (b, b, b))
        M.build_tiers(d, np.ones(1, np.uint64), (1, 0, 0), (b, b, b), M.source_f32(*mats), L,
                      dst_on_device=False)
        assert int(dm[0][0][0]) == case["d_bits"] | (case["m_bits"] << 16), case["name"]
        np.testing.assert_array_equal(O.decode_codes(codes[0][0][:4 * b], b), case["q"],
                                      err_msg=case["name"])


def test_build_tiers_codes_source_bit_exact_vs_oracle():
    spec = synth.TINY.with_(hidden=256, inter=128, n_experts=8, n_slots=(2, 4, 2))
    tier_bits = (4, 3, 2)
    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, False, spec.act)
    pop = np.arange(spec.n_experts, dtype=np.uint64)[::-1].copy()
    tmap, sexp = M.build_tiers(d, pop, spec.n_slots, tier_bits)
    bits_of = [tier_bits[int(v) >> 16] for v in tmap]
    per = [synth.expert_codes(spec, bits_of[e], seed=23, expert=e) for e in range(spec.n_experts)]
    q = [np.ascontiguousarray(np.stack([per[e][n][2] for e in range(spec.n_experts)]))
         for n in ("gate", "up", "down")]
    dd = [np.ascontiguousarray(np.stack([per[e][n][0] for e in range(spec.n_experts)]))
          for n in ("gate", "up", "down")]
    mm = [np.ascontiguousarray(np.stack([per[e][n][1] for e in range(spec.n_experts)]))
          for n in ("gate", "up", "down")]
    L, codes, dm = _host_tables(d, spec.n_slots, tier_bits)
    M.build_tiers(d, pop, spec.n_slots, tier_bits, M.source_codes(q, dd, mm), L)
    blocks = {e: [per[e][n] for n in ("gate", "up", "down")] for e in range(spec.n_experts)}
    want = _oracle_tables(blocks, sexp, spec.n_slots, tier_bits)
    for (t, m), (wc, wd) in want.items():
        np.testing.assert_array_equal(codes[t][m], wc)
        np.testing.assert_array_equal(dm[t][m], wd)


def test_build_tiers_mx_ties_saturation_and_range_vs_oracle():
    # one expert whose blocks hit every rounding case of the MXFP4 quantiser:
    # exact grid points, midpoints (ties to even), saturation above 6, zero
    # blocks and blocks whose shared exponent is clamped at either end
    H = I = 128
    d = M.dims(H, I, 1, 1, False, "f32")
    rng = np.random.default_rng(31)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.99])
    mats = []
    for m in range(3):
        w = rng.standard_normal((I, H)) * np.exp(rng.uniform(-10, 3, (I, 1)))
        for r in range(0, I, 3):
            k = int(rng.integers(-20, 20))
            sgn = rng.choice([-1.0, 1.0], size=10)
            w[r, 32 * (r % 4):32 * (r % 4) + 10] = sgn * mids * 2.0 ** k
        w[5, :32] = 0.0
        w[6, 32:64] = 2.0 ** -140                  # exponent clamped at -125
        w[7, 64:96] = 1.5 * 2.0 ** 127             # exponent at +125
        mats.append(np.ascontiguousarray(w.astype(np.float32)[None]))
    L, codes, dm = _host_tables(d, (1, 0, 0), (MX, 3, 2))
    M.build_tiers(d, np.ones(1, np.uint64), (1, 0, 0), (MX, 3, 2), M.source_f32(*mats), L,
                  dst_on_device=False)
    for m in range(3):
        b = O.quantise_rows_mx(mats[m][0])
        wc, we = O.pack_tiles_mx(b.q[None], b.e[None])
        np.testing.assert_array_equal(codes[0][m], wc, err_msg=f"codes mat {m}")
        np.testing.assert_array_equal(dm[0][m], we, err_msg=f"scales mat {m}")


def test_build_tiers_mx_codes_source_and_range_check():
    spec = synth.TINY.with_(hidden=256, inter=128, n_experts=4, n_slots=(1, 2, 1))
    tier_bits, down_bits = (4, 3, 2), (MX, 0, MX)
    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, False, spec.act)
    pop = np.array([9, 7, 5, 3], np.uint64)
    rng = np.random.default_rng(32)
    shapes = ((128, 256), (128, 256), (256, 128))
    tmap, sexp = M.build_tiers(d, pop, spec.n_slots, tier_bits)
    tier_of = [int(v) >> 16 for v in tmap]
    q, dd, mm = [], [], []
    blocks = {e: [None] * 3 for e in range(4)}
    for mi, (r, c) in enumerate(shapes):
        qm = np.zeros((4, r, c), np.uint8)
        dm_ = np.zeros((4, r, c // 32), np.uint16)
        mn = np.zeros((4, r, c // 32), np.float16)
        for e in range(4):
            f = _mbits(tier_bits, down_bits, tier_of[e], mi)
            if f == MX:
                qm[e] = rng.integers(0, 16, (r, c))
                dm_[e] = rng.integers(2, 253, (r, c // 32))
                blocks[e][mi] = O.MxBlocks(dm_[e].astype(np.uint8), qm[e])
            else:
                qm[e] = rng.integers(0, 2 ** f, (r, c))
                dv = rng.uniform(0.01, 1, (r, c // 32)).astype(np.float16)
                mv = rng.uniform(-1, 1, (r, c // 32)).astype(np.float16)
                dm_[e] = dv.view(np.uint16)
                mn[e] = mv
                blocks[e][mi] = (dv, mv, qm[e])
        q.append(qm)
        dd.append(dm_)
        mm.append(mn)
    L, codes, dm = _host_tables(d, spec.n_slots, tier_bits, down_bits)
    M.build_tiers(d, pop, spec.n_slots, tier_bits, M.source_codes(q, dd, mm), L,
                  dst_on_device=False)
    want = _oracle_tables(blocks, sexp, spec.n_slots, tier_bits, down_bits)
    for (t, m), (wc, wd) in want.items():
        np.testing.assert_array_equal(codes[t][m], wc, err_msg=f"codes tier {t} mat {m}")
        np.testing.assert_array_equal(dm[t][m], wd, err_msg=f"scales tier {t} mat {m}")
    # an E8M0 byte outside [2, 252] is rejected
    e_mx = [e for e in range(4) if tier_of[e] == 0][0]
    for bad in (1, 253):
        dd[2][e_mx, 0, 0] = bad
        with pytest.raises(M.MoeError) as err:
            M.build_tiers(d, pop, spec.n_slots, tier_bits, M.source_codes(q, dd, mm), L,
                          dst_on_device=False)
        assert err.value.status == M.MOE_EINVAL
    dd[2][e_mx, 0, 0] = 100


def test_mx_table_bytes_and_layer_checks():
    d = M.dims(2048, 512, 512, 10, True, "bf16")
    # 16 code bytes and one scale byte per block of 32
    assert M.tier_table_bytes(d, MX, 128, M.MOE_DOWN, M.MOE_CODES) == 128 * 2048 * 512 // 32 * 16
    assert M.tier_table_bytes(d, MX, 128, M.MOE_DOWN, M.MOE_DM) == 128 * 2048 * 512 // 32
    assert M.tier_table_bytes(d, 5, 128, M.MOE_DOWN, M.MOE_DM) == 0
    # the planner's error model has no MXFP4 weight
    with pytest.raises(M.MoeError):
        M.plan_tiers(d, np.ones(512, np.uint64), (4, 3, MX), 1 << 40)


def test_build_tiers_rejects_bad_input():
    spec = synth.TINY.with_(n_experts=4, n_slots=(4, 0, 0))
    d = M.dims(spec.hidden, spec.inter, 4, 2, False, "f32")
    gate, up, down = synth.expert_weights_f32(spec, seed=24)
    L, codes, dm = _host_tables(d, (4, 0, 0), (4, 3, 2))  # keep the buffers alive
    pop = np.zeros(4, np.uint64)
    gate[2, 5, 7] = np.inf
    with pytest.raises(M.MoeError) as e:
        M.build_tiers(d, pop, (4, 0, 0), (4, 3, 2), M.source_f32(gate, up, down), L)
    assert e.value.status == M.MOE_EINVAL
    with pytest.raises(M.MoeError):
        M.build_tiers(d, pop, (2, 1, 0), (4, 3, 2))           # counts do not sum to E
    # a code above the tier's largest code
    q = [np.zeros((4, r, c), np.uint8) for r, c in ((128, 256), (128, 256), (256, 128))]
    dd = [np.ones((4, r, c // 32), np.float16) for r, c in ((128, 256), (128, 256), (256, 128))]
    mm = [np.zeros((4, r, c // 32), np.float16) for r, c in ((128, 256), (128, 256), (256, 128))]
    q[1][3, 0, 0] = 16
    with pytest.raises(M.MoeError):
        M.build_tiers(d, pop, (4, 0, 0), (4, 3, 2), M.source_codes(q, dd, mm), L)


# ----------------------------------------------------------------- tier planner

@pytest.mark.parametrize("tier_bits", [(4, 3, 2), (4, 4, 2), (3, 4, 2), (2, 3, 4), (3, 3, 3)])
def test_plan_tiers_matches_oracle(tier_bits):
    rng = np.random.default_rng(sum(tier_bits))
    H, I = 256, 128
    c = [O.expert_table_bytes(H, I, b) for b in tier_bits]
    for trial in range(25):
        E = int(rng.integers(1, 40))
        d = M.dims(H, I, E, 1, False, "bf16")
        kind = trial % 3
        if kind == 0:
            pop = rng.zipf(1.5, size=E)
        elif kind == 1:
            pop = rng.integers(0, 4, size=E)              # many ties and zeros
        else:
            pop = np.zeros(E)
        pop = pop.astype(np.uint64)
        budget = int(rng.integers(E * min(c) - c[0], E * max(c) + c[0]))
        try:
            want = O.plan_tiers(pop, tier_bits, H, I, budget)
        except ValueError:
            with pytest.raises(M.MoeError):
                M.plan_tiers(d, pop, tier_bits, budget)
            continue
        assert M.plan_tiers(d, pop, tier_bits, budget) == want


def test_plan_tiers_full_size_layer():
    # the full-size layer: a budget of exactly the 128 / 256 / 128 tables fits
    # and is used up to the last tier; more budget never raises the error
    spec = synth.FULL
    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, True, "bf16")
    pop = np.random.default_rng(1).zipf(1.3, size=spec.n_experts).astype(np.uint64)
    c = [O.expert_table_bytes(spec.hidden, spec.inter, b) for b in (4, 3, 2)]
    order = sorted(range(spec.n_experts), key=lambda e: (-int(pop[e]), e))
    ranked = [int(pop[e]) for e in order]

    def err(n):
        w = [49] * n[0] + [225] * n[1] + [1225] * n[2]
        return sum(p * x for p, x in zip(ranked, w))

    prev = None
    for budget in (768 * 2**20, 800 * 2**20, 900 * 2**20, 960 * 2**20):
        n = M.plan_tiers(d, pop, (4, 3, 2), budget)
        assert sum(n) == spec.n_experts
        assert n[0] * c[0] + n[1] * c[1] + n[2] * c[2] <= budget
        assert prev is None or err(n) <= prev
        prev = err(n)


def test_plan_tiers_rejects_bad_input():
    d = M.dims(256, 128, 8, 2, False, "bf16")
    pop = np.ones(8, np.uint64)
    with pytest.raises(M.MoeError):
        M.plan_tiers(d, pop, (4, 5, 2), 10**9)
    with pytest.raises(M.MoeError):
        M.plan_tiers(d, pop, (4, 3, 2), 8 * O.expert_table_bytes(256, 128, 2) - 1)


@pytest.mark.parametrize("tier_bits,down_bits", [((4, 3, 2), (4, 4, 3)), ((3, 3, 2), (4, 2, 4)),
                                                  ((4, 3, 2), (0, 4, 0)), ((2, 3, 4), (3, 0, 2))])
def test_plan_tiers_ladder_matches_oracle(tier_bits, down_bits):
    rng = np.random.default_rng(sum(tier_bits) + 10 * sum(down_bits))
    H, I = 256, 128
    dn = [d if d else b for b, d in zip(tier_bits, down_bits)]
    c = [2 * O.expert_table_bytes(H, I, b) // 3 + O.expert_table_bytes(H, I, d) // 3
         for b, d in zip(tier_bits, dn)]
    for trial in range(25):
        E = int(rng.integers(1, 40))
        d = M.dims(H, I, E, 1, False, "bf16")
        pop = (rng.zipf(1.5, size=E) if trial % 2 else rng.integers(0, 4, size=E)).astype(np.uint64)
        budget = int(rng.integers(E * min(c) - c[0], E * max(c) + c[0]))
        try:
            want = O.plan_tiers(pop, tier_bits, H, I, budget, down_bits=down_bits)
        except ValueError:
            with pytest.raises(M.MoeError):
                M.plan_tiers(d, pop, tier_bits, budget, down_bits=down_bits)
            continue
        assert M.plan_tiers(d, pop, tier_bits, budget, down_bits=down_bits) == want
    d = M.dims(H, I, 4, 1, False, "bf16")
    with pytest.raises(M.MoeError):
        M.plan_tiers(d, np.ones(4, np.uint64), (4, 3, 2), 1 << 40, down_bits=(4, 0x14, 2))


def test_decode_noalloc_refuses_workspaces_beyond_its_scratch():
    # a decode workspace larger than the library's scratch is refused before
    # any HIP call (MOE_ENOSPC); the header states the scratch size
    lib = M.lib()
    with open(os.path.join(ROOT, "include", "moe.h")) as fh:
        m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", fh.read())
    limit = int(m.group(1)) << int(m.group(2))
    n = ctypes.c_size_t(0)
    d = M.dims(256, 128, 40000, 4, False, "bf16")
    L = _fake_layer(d, (40000, 0, 0))
    assert lib.moe_forward_decode(ctypes.byref(d), ctypes.byref(L), None, 1, None, M.MOE_F32, None,
                                  None, None, ctypes.byref(n), None) == M.MOE_OK
    assert n.value > limit
    fake = 1 << 22
    assert lib.moe_forward_decode_noalloc(ctypes.byref(d), ctypes.byref(L), fake, 1, fake,
                                          M.MOE_F32, None, None, None) == M.MOE_ENOSPC
    # invalid arguments are refused the same way as by moe_forward_decode
    bad = M.dims(256, 128, 64, 65, False, "f32")
    assert lib.moe_forward_decode_noalloc(ctypes.byref(bad), ctypes.byref(L), fake, 1, fake,
                                          M.MOE_F32, None, None, None) == M.MOE_EINVAL
    # the full-size layer fits
    full = M.dims(2048, 512, 512, 10, True, "bf16")
    Lf = _fake_layer(full, (128, 256, 128))
    assert lib.moe_forward_decode(ctypes.byref(full), ctypes.byref(Lf), None, 1, None, M.MOE_BF16,
                                  None, None, None, ctypes.byref(n), None) == M.MOE_OK
    assert n.value <= limit


def test_check_layer_argument_errors_without_gpu():
    # argument errors are found before the tier map is read from the device
    lib = M.lib()
    d = M.dims(256, 128, 64, 4, False, "f32")
    L = _fake_layer(d, (32, 0, 0))            # counts do not sum to E
    assert lib.moe_check_layer(ctypes.byref(d), ctypes.byref(L), None) == M.MOE_EINVAL
    L = _fake_layer(d, (64, 0, 0))
    L.tier_map = None
    assert lib.moe_check_layer(ctypes.byref(d), ctypes.byref(L), None) == M.MOE_EINVAL
    assert lib.moe_check_layer(None, ctypes.byref(L), None) == M.MOE_EINVAL


def test_c_program_uses_the_abi(tmp_path):
    # the header compiled as C11 and the library called from a C program:
    # no Python, no torch (host-only calls, no GPU)
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "c_abi_host"
    lib_dir = os.path.dirname(M.library_path())
    build = subprocess.run(
        [cc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(rocm, 'include')}",
         os.path.join(ROOT, "tests", "c_abi_host.c"), "-o", str(exe), f"-L{lib_dir}", "-lmoe",
         f"-Wl,-rpath,{lib_dir}"], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    # the HIP runtime the library links against: torch's copy if it ships one
    env = dict(os.environ)
    try:
        import torch
        env["LD_LIBRARY_PATH"] = os.pathsep.join(
            [os.path.join(os.path.dirname(torch.__file__), "lib"), env.get("LD_LIBRARY_PATH", "")])
    except ImportError:
        pass
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
