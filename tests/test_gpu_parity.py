"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: expert ids, tier maps and the counting sort bit-exact; mixing weights
within 1e-6; layer outputs within max-abs 2e-2 and relative L2 1e-3 (bf16
activations), and relative L2 1e-5 for fp32 activations, where only fp32
accumulation order separates the two sides.
"""

import numpy as np
import pytest

import oracle as O
import synth

from layers import act_f64, make_layer, rel_l2

torch = pytest.importorskip("torch")
M = pytest.importorskip("quantized_expert_ffn_route_amd")

pytestmark = pytest.mark.gpu

MID = synth.LayerSpec(hidden=512, inter=256, n_experts=32, top_k=4, has_shared=True, act="bf16",
                      n_slots=(8, 16, 8))


def dev(a, act):
    if act == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def check_y(y_gpu, y_ref, act, what=""):
    y = y_gpu.float().cpu().numpy().astype(np.float64) if hasattr(y_gpu, "cpu") else y_gpu
    err = np.max(np.abs(y - y_ref))
    rl = rel_l2(y, y_ref)
    print(f"  {what}: max-abs {err:.3e}  rel-L2 {rl:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= 2e-2, (what, err)
    assert rl <= (1e-5 if act == "f32" else 1e-3), (what, rl)


def run_route(tl, x):
    spec = tl.spec
    T = x.shape[0]
    ids = torch.empty((T, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, spec.top_k), dtype=torch.float32, device="cuda")
    M.route(tl.dl.d, tl.dl.c_struct(), dev(x, spec.act), ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def run_decode(tl, x, y_dt=None):
    spec = tl.spec
    T = x.shape[0]
    y_dt = M.MOE_F32 if y_dt is None else y_dt
    y = torch.empty((T, spec.hidden), dtype=torch.float32 if y_dt == M.MOE_F32 else torch.bfloat16,
                    device="cuda")
    ids = torch.empty((T, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, spec.top_k), dtype=torch.float32, device="cuda")
    M.forward_decode(tl.dl.d, tl.dl.c_struct(), dev(x, spec.act), y, y_dt, ids, w)
    torch.cuda.synchronize()
    return y, ids.cpu().numpy(), w.cpu().numpy()


def run_prefill(tl, x, y_dt=None):
    spec = tl.spec
    T = x.shape[0]
    y_dt = M.MOE_F32 if y_dt is None else y_dt
    y = torch.empty((T, spec.hidden), dtype=torch.float32 if y_dt == M.MOE_F32 else torch.bfloat16,
                    device="cuda")
    ids = torch.empty((T, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, spec.top_k), dtype=torch.float32, device="cuda")
    off = torch.empty(spec.n_experts + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(T * spec.top_k, dtype=torch.int32, device="cuda")
    M.forward_prefill(tl.dl.d, tl.dl.c_struct(), dev(x, spec.act), y, y_dt, ids, w, off, srt)
    torch.cuda.synchronize()
    return y, ids.cpu().numpy(), w.cpu().numpy(), off.cpu().numpy(), srt.cpu().numpy()


# ------------------------------------------------------------------ layers

@pytest.fixture(scope="module")
def tiny():
    print("\n[fixture] tiny layer", flush=True)
    return make_layer(synth.TINY, seed=0)


@pytest.fixture(scope="module")
def mid():
    print("\n[fixture] mid layer", flush=True)
    return make_layer(MID, seed=5)


@pytest.fixture(scope="module")
def full():
    print("\n[fixture] full-size layer (random blocks)", flush=True)
    return make_layer(synth.FULL, seed=0, source="codes", n_calib=4096)


# ------------------------------------------------------------------ routing

def test_route_tiny_exact(tiny):
    x = synth.tokens(tiny.spec, 8, 10)
    ids, w = run_route(tiny, x)
    keys, oids, g = O.route(act_f64(x, "f32"), tiny.ol.w_router, tiny.ol.bias, tiny.spec.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert np.max(np.abs(w - g)) <= 1e-6


def test_route_ties_take_lower_id(mid):
    # duplicate router rows: equal keys must resolve to the lower expert id
    def dup(w_r, b):
        w_r = w_r.copy()
        b = b.copy()
        for src, dst in ((3, 17), (3, 29), (8, 9)):
            w_r[dst] = w_r[src]
            b[dst] = b[src]
        b[[3, 17, 29]] += 3.0        # make the tied experts the winners
        return w_r, b
    tl = make_layer(MID, seed=6, router_override=dup)
    x = synth.tokens(MID, 40, 11)
    ids, w = run_route(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MID.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert np.all(ids[:, :3] == [3, 17, 29])
    assert np.max(np.abs(w - g)) <= 1e-6


def test_route_full_size_exact(full):
    x = synth.tokens(full.spec, 512, 12)
    ids, w = run_route(full, x)
    _, oids, g = O.route(act_f64(x, "bf16"), full.ol.w_router, full.ol.bias, full.spec.top_k)
    np.testing.assert_array_equal(ids, oids)
    assert np.max(np.abs(w - g)) <= 1e-6


def test_route_paths_agree(full):
    # up to 16 tokens take the float64 router kernel, more take MFMA keys plus
    # the exact rescoring: the same tokens must get bitwise the same result
    x = synth.tokens(full.spec, 40, 13)
    ids_a, w_a = run_route(full, x[:16])
    ids_b, w_b = run_route(full, x)
    np.testing.assert_array_equal(ids_a, ids_b[:16])
    np.testing.assert_array_equal(w_a.view(np.uint32), w_b[:16].view(np.uint32))


def test_tier_map_matches_oracle(full, mid, tiny):
    for tl in (full, mid, tiny):
        want, _ = O.build_tiers(tl.popularity, tl.spec.n_slots)
        np.testing.assert_array_equal(tl.tier_map, want)
        np.testing.assert_array_equal(tl.dl.tier_map.cpu().numpy(), want)


# ------------------------------------------------------------------ decode

def test_decode_tiny(tiny):
    x = synth.tokens(tiny.spec, 8, 13)
    y, ids, w = run_decode(tiny, x)
    ref = O.moe_layer(act_f64(x, "f32"), tiny.ol)
    np.testing.assert_array_equal(ids, ref["ids"])
    check_y(y, ref["y"], "f32", "decode tiny T=8")


def test_decode_tiny_single_token(tiny):
    # one token takes the fused top-K + gate/up path
    for seed in (30, 31, 32):
        x = synth.tokens(tiny.spec, 1, seed)
        y, ids, w = run_decode(tiny, x)
        ref = O.moe_layer(act_f64(x, "f32"), tiny.ol)
        np.testing.assert_array_equal(ids, ref["ids"])
        assert np.max(np.abs(w - ref["g"])) <= 1e-6
        check_y(y, ref["y"], "f32", f"decode tiny T=1 seed {seed}")


@pytest.mark.parametrize("T", [1, 5, 16, 17, 21, 40])
def test_decode_mid_ragged(mid, T):
    x = synth.tokens(mid.spec, T, 14 + T)
    y, ids, w = run_decode(mid, x)
    ref = O.moe_layer(act_f64(x, "bf16"), mid.ol)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["g"])) <= 1e-6
    check_y(y, ref["y"], "bf16", f"decode mid T={T}")
    # bf16 output is the RNE rounding of the same fp32 sums
    yb, _, _ = run_decode(mid, x, M.MOE_BF16)
    want = O.bf16_round(y.cpu().numpy())
    np.testing.assert_array_equal(yb.float().cpu().numpy(), want)


def test_decode_full_single_tokens(full):
    xs = synth.tokens(full.spec, 4, 15)
    ref = O.moe_layer(act_f64(xs, "bf16"), full.ol)
    for t in range(4):
        y, ids, w = run_decode(full, xs[t:t + 1])
        np.testing.assert_array_equal(ids, ref["ids"][t:t + 1])
        check_y(y, ref["y"][t:t + 1], "bf16", f"decode full T=1 token {t}")
        # the benchmark's configuration: bf16 output
        yb, idb, _ = run_decode(full, xs[t:t + 1], M.MOE_BF16)
        np.testing.assert_array_equal(idb, ref["ids"][t:t + 1])
        check_y(yb, O.output_cast(ref["y"][t:t + 1], "bf16"), "bf16", f"decode full token {t} bf16 out")


def test_decode_graph_replays_match_eager(mid, full):
    # the benchmark replays captured decode calls: every replay, with new
    # inputs copied in and other eager calls in between, must give the eager
    # results bit for bit
    for tl in (mid, full):
        spec, d, L = tl.spec, tl.dl.d, tl.dl.c_struct()
        H, K = spec.hidden, spec.top_k
        X = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
        Y = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
        IDS = torch.empty((1, K), dtype=torch.int32, device="cuda")
        W = torch.empty((1, K), dtype=torch.float32, device="cuda")
        ws = torch.empty(M.workspace_bytes("decode", d, L, 1, M.MOE_BF16), dtype=torch.uint8,
                         device="cuda")
        xs = synth.tokens(spec, 4, 130)
        eager = []
        for i in range(4):
            X.copy_(dev(xs[i:i + 1], "bf16"))
            M.forward_decode(d, L, X, Y, M.MOE_BF16, IDS, W, ws=ws)
            torch.cuda.synchronize()
            eager.append((Y.clone(), IDS.clone(), W.clone()))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            M.forward_decode(d, L, X, Y, M.MOE_BF16, IDS, W, ws=ws)
        torch.cuda.synchronize()
        other = synth.tokens(spec, 3, 131)
        for rep in range(3):
            for i in range(4):
                X.copy_(dev(xs[i:i + 1], "bf16"))
                graph.replay()
                torch.cuda.synchronize()
                assert torch.equal(Y, eager[i][0]), (spec.hidden, rep, i)
                assert torch.equal(IDS, eager[i][1]) and torch.equal(W, eager[i][2])
                # eager work on the same workspace between replays
                run_decode(tl, other[rep:rep + 1], M.MOE_BF16)
                M.forward_decode(d, L, dev(other[rep:rep + 1], "bf16"), torch.empty_like(Y),
                                 M.MOE_BF16, ws=ws)
                torch.cuda.synchronize()
        del graph


def test_prefill_graph_replays_match_eager(mid, full):
    # the benchmark times captured prefill calls: every replay, with new
    # inputs copied in and eager calls on the same workspace in between, must
    # give the eager results bit for bit (ids, weights, sort, outputs)
    for tl, T in ((mid, 333), (full, 4096)):
        spec, d, L = tl.spec, tl.dl.d, tl.dl.c_struct()
        H, K, E = spec.hidden, spec.top_k, spec.n_experts
        X = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        Y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        IDS = torch.empty((T, K), dtype=torch.int32, device="cuda")
        W = torch.empty((T, K), dtype=torch.float32, device="cuda")
        OFF = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        SRT = torch.empty(T * K, dtype=torch.int32, device="cuda")
        ws = torch.empty(M.workspace_bytes("prefill", d, L, T, M.MOE_BF16), dtype=torch.uint8,
                         device="cuda")
        xs = [synth.tokens(spec, T, 140 + i) for i in range(3)]
        outs = (Y, IDS, W, OFF, SRT)
        eager = []
        for i in range(3):
            X.copy_(dev(xs[i], "bf16"))
            M.forward_prefill(d, L, X, Y, M.MOE_BF16, IDS, W, OFF, SRT, ws=ws)
            torch.cuda.synchronize()
            eager.append([o.clone() for o in outs])
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            M.forward_prefill(d, L, X, Y, M.MOE_BF16, IDS, W, OFF, SRT, ws=ws)
        torch.cuda.synchronize()
        other = dev(synth.tokens(spec, T, 150), "bf16")
        for rep in range(3):
            for i in range(3):
                X.copy_(dev(xs[i], "bf16"))
                graph.replay()
                torch.cuda.synchronize()
                for o, e in zip(outs, eager[i]):
                    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                                       e.view(torch.int16) if e.dtype == torch.bfloat16 else e), \
                        (spec.hidden, T, rep, i)
                # eager work on the same workspace between replays
                M.forward_prefill(d, L, other, torch.empty_like(Y), M.MOE_BF16, ws=ws)
                torch.cuda.synchronize()
        del graph


@pytest.mark.parametrize("T", [4, 8, 16])
def test_verify_full_correlated(full, T):
    x = synth.correlated_tokens(full.spec, T, 16 + T)
    y, ids, w = run_decode(full, x)
    ref = O.moe_layer(act_f64(x, "bf16"), full.ol)
    np.testing.assert_array_equal(ids, ref["ids"])
    print(f"  union of experts at T={T}: {len(np.unique(ids))}", flush=True)
    check_y(y, ref["y"], "bf16", f"verify full T={T}")


def test_decode_deterministic(mid):
    x = synth.tokens(mid.spec, 16, 17)
    y1, _, _ = run_decode(mid, x)
    y2, _, _ = run_decode(mid, x)
    assert torch.equal(y1, y2)


def test_decode_zero_tokens(mid):
    y = torch.empty((0, mid.spec.hidden), dtype=torch.float32, device="cuda")
    x = torch.empty((0, mid.spec.hidden), dtype=torch.bfloat16, device="cuda")
    M.forward_decode(mid.dl.d, mid.dl.c_struct(), x, y, M.MOE_F32)
    M.forward_prefill(mid.dl.d, mid.dl.c_struct(), x, y, M.MOE_F32)
    torch.cuda.synchronize()


def test_low_bit_codes_in_wider_tables_identical():
    # codes drawn at 2 bits, stored once in 2-bit tables and once in 4-bit
    # tables with the same scales and mins: outputs must be bit-identical
    spec2 = MID.with_(tier_bits=(2, 2, 2))
    spec4 = MID.with_(tier_bits=(4, 4, 4))
    a = make_layer(spec2, seed=7, source="codes")
    import layers
    per = [synth.expert_codes(spec2, 2, 7 + 2, e) for e in range(MID.n_experts)]
    names = ("gate", "up", "down")
    q = [np.ascontiguousarray(np.stack([per[e][n][2] for e in range(MID.n_experts)])) for n in names]
    dd = [np.ascontiguousarray(np.stack([per[e][n][0] for e in range(MID.n_experts)])) for n in names]
    mm = [np.ascontiguousarray(np.stack([per[e][n][1] for e in range(MID.n_experts)])) for n in names]
    w_router, bias = synth.router(MID, 7)
    b = M.DeviceLayer(a.dl.d, spec4.n_slots, spec4.tier_bits, (w_router, bias),
                      synth.shared_expert(MID, 7 + 3))
    b.load_experts(a.popularity, M.source_codes(q, dd, mm))
    x = synth.tokens(MID, 19, 18)
    ya, _, _ = run_decode(a, x)
    tb = layers.TestLayer(spec=spec4, ol=None, dl=b, tier_map=None, popularity=None)
    yb, _, _ = run_decode(tb, x)
    assert torch.equal(ya, yb)
    pa = run_prefill(a, x)[0]
    pb = run_prefill(tb, x)[0]
    check_y(pb, pa.cpu().numpy().astype(np.float64), "bf16", "prefill 2-bit vs 4-bit tables")


# ------------------------------------------------------------------ prefill

def test_prefill_tiny(tiny):
    x = synth.tokens(tiny.spec, 300, 19)
    y, ids, w, off, srt = run_prefill(tiny, x)
    ref = O.moe_layer(act_f64(x, "f32"), tiny.ol)
    np.testing.assert_array_equal(ids, ref["ids"])
    o_off, o_srt = O.sort_routes(ids, tiny.spec.n_experts)
    np.testing.assert_array_equal(off, o_off)
    np.testing.assert_array_equal(srt, o_srt)
    check_y(y, ref["y"], "f32", "prefill tiny T=300")


# T = 1000 puts about 125 routes on each of the 32 experts: every bucket
# spans two 96-row tiles of the routed GEMMs, the second one ragged
@pytest.mark.parametrize("T", [1, 63, 333, 1000])
def test_prefill_mid(mid, T):
    x = synth.tokens(mid.spec, T, 20 + T)
    y, ids, w, off, srt = run_prefill(mid, x)
    ref = O.moe_layer(act_f64(x, "bf16"), mid.ol)
    np.testing.assert_array_equal(ids, ref["ids"])
    o_off, o_srt = O.sort_routes(ids, mid.spec.n_experts)
    np.testing.assert_array_equal(off, o_off)
    np.testing.assert_array_equal(srt, o_srt)
    check_y(y, ref["y"], "bf16", f"prefill mid T={T}")
    yb = run_prefill(mid, x, M.MOE_BF16)[0]
    check_y(yb, O.output_cast(ref["y"], "bf16"), "bf16", f"prefill mid T={T} bf16 out")


# Shapes off the fast paths: 3 chunks of 128 along H and I (not a power of
# two: the routed GEMMs take the register-staged pipeline) and 48 experts (not
# a multiple of 32: the prefill router keeps the float64 GEMV + sorted top-K).
ODD = synth.LayerSpec(hidden=384, inter=384, n_experts=48, top_k=6, has_shared=True, act="bf16",
                      n_slots=(12, 24, 12))


@pytest.fixture(scope="module")
def odd():
    print("\n[fixture] odd-shape layer", flush=True)
    return make_layer(ODD, seed=9)


@pytest.mark.parametrize("T", [1, 5, 200])
def test_odd_shapes_decode_and_prefill(odd, T):
    x = synth.tokens(ODD, T, 50 + T)
    ref = O.moe_layer(act_f64(x, "bf16"), odd.ol)
    y, ids, w = run_decode(odd, x)
    np.testing.assert_array_equal(ids, ref["ids"])
    check_y(y, ref["y"], "bf16", f"decode odd T={T}")
    yp, idp, wp, off, srt = run_prefill(odd, x)
    np.testing.assert_array_equal(idp, ref["ids"])
    o_off, o_srt = O.sort_routes(idp, ODD.n_experts)
    np.testing.assert_array_equal(off, o_off)
    np.testing.assert_array_equal(srt, o_srt)
    check_y(yp, ref["y"], "bf16", f"prefill odd T={T}")


def test_prefill_full_4096_every_row(full):
    # every one of the 4096 x 2048 outputs against the oracle, which runs
    # expert by expert (each expert's dequantised weights dropped after its
    # bucket); then a second call on the same inputs must repeat the first
    # bit for bit (no atomics anywhere in the prefill path)
    T = 4096
    x = synth.tokens(full.spec, T, 21)
    y, ids, w, off, srt = run_prefill(full, x, M.MOE_BF16)
    xs = act_f64(x, "bf16")
    keys, oids, g = O.route(xs, full.ol.w_router, full.ol.bias, full.spec.top_k)
    np.testing.assert_array_equal(ids, oids)
    assert np.max(np.abs(w - g)) <= 1e-6
    o_off, o_srt = O.sort_routes(ids, full.spec.n_experts)
    np.testing.assert_array_equal(off, o_off)
    np.testing.assert_array_equal(srt, o_srt)
    y2, ids2, w2, off2, srt2 = run_prefill(full, x, M.MOE_BF16)
    assert torch.equal(y, y2)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(w.view(np.uint32), w2.view(np.uint32))
    np.testing.assert_array_equal(srt, srt2)
    print("  oracle over all 4096 rows ...", flush=True)
    ref = O.moe_layer(xs, full.ol, routing=(keys, oids, g), drop_experts=True)
    check_y(y, O.output_cast(ref["y"], "bf16"), "bf16", "prefill full T=4096 (every row)")


def test_prefill_router_ties_take_lower_id():
    # bf16 prefill ranks from approximate MFMA keys, then rescores the
    # candidates exactly: duplicated router rows must still tie-break by id
    def dup(w_r, b):
        w_r = w_r.copy()
        b = b.copy()
        for src, dst in ((3, 17), (3, 29), (8, 9)):
            w_r[dst] = w_r[src]
            b[dst] = b[src]
        b[[3, 17, 29]] += 3.0
        return w_r, b
    tl = make_layer(MID, seed=6, router_override=dup)
    x = synth.tokens(MID, 200, 31)
    y, ids, w, _, _ = run_prefill(tl, x)
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MID.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert np.all(ids[:, :3] == [3, 17, 29])
    assert np.max(np.abs(w - g)) <= 1e-6
    check_y(y, ref["y"], "bf16", "prefill with tied router rows")


def test_prefill_router_one_ulp_apart():
    # router rows that differ in a single element by one bf16 ulp: the fp32
    # MFMA keys cannot order them reliably, the exact rescoring must
    def near(w_r, b):
        w_r = w_r.copy()
        b = b.copy()
        for src, dst in ((5, 6), (5, 20), (11, 2)):
            w_r[dst] = w_r[src]
            b[dst] = b[src]
            w_r[dst, dst] = np.uint16(int(w_r[dst, dst]) + 1)   # bf16 bit pattern
        b[[5, 6, 20]] += 3.0
        return w_r, b
    tl = make_layer(MID, seed=7, router_override=near)
    x = synth.tokens(MID, 256, 32)
    _, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MID.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert np.max(np.abs(w - g)) <= 1e-6


WIDE = synth.LayerSpec(hidden=256, inter=128, n_experts=128, top_k=8, has_shared=False,
                       act="bf16", n_slots=(32, 64, 32))


def test_prefill_router_many_candidates():
    # 100 identical router rows: more near-K candidates than one wave holds,
    # which takes the exact rescoring of every expert
    def many(w_r, b):
        w_r = w_r.copy()
        b = b.copy()
        w_r[:100] = w_r[0]
        b[:100] = b[0] + 4.0
        return w_r, b
    tl = make_layer(WIDE, seed=8, router_override=many)
    x = synth.tokens(WIDE, 96, 33)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, WIDE.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert np.all(ids == np.arange(WIDE.top_k))
    assert np.max(np.abs(w - g)) <= 1e-6
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    check_y(y, ref["y"], "bf16", "prefill, 100 tied router rows")


def test_decode_router_many_ties():
    # 100 identical router rows: the threshold top-K cannot narrow the field
    # below 64 candidates and takes the sorted-list path; ids stay exact
    def many(w_r, b):
        w_r = w_r.copy()
        b = b.copy()
        w_r[:100] = w_r[0]
        b[:100] = b[0] + 4.0
        return w_r, b
    tl = make_layer(WIDE, seed=8, router_override=many)
    for T in (1, 3):
        x = synth.tokens(WIDE, T, 40 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, WIDE.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        assert np.all(ids == np.arange(WIDE.top_k))
        assert np.max(np.abs(w - g)) <= 1e-6
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        check_y(y, ref["y"], "bf16", f"decode T={T}, 100 tied router rows")


def test_router_nan_rows_rank_last():
    # router rows of NaN give NaN keys, which rank below every number
    # (moe_route's contract): the decode top-K and the prefill recheck both
    # take their all-experts paths and must still pick the oracle's ids
    def nan_rows(w_r, b):
        w_r = w_r.copy()
        w_r[[2, 9, 30]] = np.uint16(0x7FC0)          # bf16 quiet NaN
        return w_r, b
    tl = make_layer(MID, seed=9, router_override=nan_rows)
    for T in (1, 3):
        x = synth.tokens(MID, T, 50 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MID.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        assert not np.isin(ids, [2, 9, 30]).any()
        assert np.max(np.abs(w - g)) <= 1e-6
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        check_y(y, ref["y"], "bf16", f"decode T={T}, NaN router rows")
    x = synth.tokens(MID, 200, 53)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MID.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert not np.isin(ids, [2, 9, 30]).any()
    assert np.max(np.abs(w - g)) <= 1e-6
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    check_y(y, ref["y"], "bf16", "prefill, NaN router rows")


# the largest top-K (64) over more experts than one workgroup holds keys for
BIGK = synth.LayerSpec(hidden=256, inter=128, n_experts=1024, top_k=64, has_shared=False,
                       act="bf16", n_slots=(256, 512, 256))
# the largest hidden size: 64 chunks of 128 along the contraction
MAXH = synth.LayerSpec(hidden=8192, inter=128, n_experts=8, top_k=2, has_shared=True,
                       act="bf16", n_slots=(2, 4, 2))


# intermediate size 640 (down rows of 640, five chunks of 128), the width of
# the pages' own model
I640 = synth.LayerSpec(hidden=1024, inter=640, n_experts=32, top_k=4, has_shared=True,
                       act="bf16", n_slots=(8, 16, 8))


def test_intermediate_640():
    tl = make_layer(I640, seed=12)
    for T in (1, 7):
        x = synth.tokens(I640, T, 80 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, I640.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        check_y(y, ref["y"], "bf16", f"decode T={T}, I=640")
    x = synth.tokens(I640, 150, 83)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, I640.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    check_y(y, ref["y"], "bf16", "prefill T=150, I=640")


def test_top_k_64_of_1024_experts():
    tl = make_layer(BIGK, seed=10)
    for T in (1, 3):
        x = synth.tokens(BIGK, T, 60 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, BIGK.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        assert np.max(np.abs(w - g)) <= 1e-6
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        check_y(y, ref["y"], "bf16", f"decode T={T}, K=64 of E=1024")
    x = synth.tokens(BIGK, 100, 63)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, BIGK.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    assert np.max(np.abs(w - g)) <= 1e-6
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    check_y(y, ref["y"], "bf16", "prefill T=100, K=64 of E=1024")


def test_largest_hidden_size():
    tl = make_layer(MAXH, seed=11)
    for T in (1, 5):
        x = synth.tokens(MAXH, T, 70 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MAXH.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        check_y(y, ref["y"], "bf16", f"decode T={T}, H=8192")
    x = synth.tokens(MAXH, 70, 73)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, MAXH.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    check_y(y, ref["y"], "bf16", "prefill T=70, H=8192")


def test_decode_equals_prefill(mid, full):
    for tl, T in ((mid, 16), (full, 8)):
        x = synth.tokens(tl.spec, T, 22)
        yd, idd, wd = run_decode(tl, x)
        yp, idp, wp, _, _ = run_prefill(tl, x)
        np.testing.assert_array_equal(idd, idp)
        np.testing.assert_array_equal(wd, wp)
        check_y(yp, yd.cpu().numpy().astype(np.float64), "bf16", "prefill vs decode")


# per-matrix ladders: the down matrices of a tier quantised at their own width
@pytest.mark.parametrize("down_bits", [(4, 4, 3), (3, 2, 4)])
def test_per_matrix_ladder(down_bits):
    spec = MID.with_(down_bits=down_bits)
    tl = make_layer(spec, seed=13)
    for T in (1, 5):
        x = synth.tokens(spec, T, 90 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, spec.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        check_y(y, ref["y"], "bf16", f"decode T={T}, down bits {down_bits}")
        yb, _, _ = run_decode(tl, x, M.MOE_BF16)
        check_y(yb, O.output_cast(ref["y"], "bf16"), "bf16",
                f"decode T={T} bf16 out, down bits {down_bits}")
    x = synth.tokens(spec, 300, 95)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, spec.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    check_y(y, ref["y"], "bf16", f"prefill T=300, down bits {down_bits}")


# MXFP4 tables (the pages' low down tier): as a whole tier and as the down
# ladder of the lower tiers, through decode (fp32 and bf16 activations) and
# prefill
MX = 0x14


@pytest.mark.parametrize("tier_bits,down_bits,act", [
    ((4, 3, MX), None, "bf16"),
    ((4, 3, 2), (4, MX, MX), "bf16"),
    ((MX, 3, 2), None, "f32"),
])
def test_mxfp4_tiers(tier_bits, down_bits, act):
    spec = MID.with_(tier_bits=tier_bits, down_bits=down_bits, act=act)
    tl = make_layer(spec, seed=14)
    for T in (1, 6):
        x = synth.tokens(spec, T, 100 + T)
        y, ids, w = run_decode(tl, x)
        _, oids, g = O.route(act_f64(x, act), tl.ol.w_router, tl.ol.bias, spec.top_k, exact=True)
        np.testing.assert_array_equal(ids, oids)
        ref = O.moe_layer(act_f64(x, act), tl.ol)
        check_y(y, ref["y"], act, f"decode T={T}, {tier_bits}/{down_bits} {act}")
        if act == "bf16":
            yb, _, _ = run_decode(tl, x, M.MOE_BF16)
            check_y(yb, O.output_cast(ref["y"], "bf16"), act, f"decode T={T} bf16 out")
    x = synth.tokens(spec, 300, 105)
    y, ids, w, _, _ = run_prefill(tl, x)
    _, oids, g = O.route(act_f64(x, act), tl.ol.w_router, tl.ol.bias, spec.top_k, exact=True)
    np.testing.assert_array_equal(ids, oids)
    ref = O.moe_layer(act_f64(x, act), tl.ol)
    check_y(y, ref["y"], act, f"prefill T=300, {tier_bits}/{down_bits} {act}")


# Every expert chosen by every token, with h rows too large for the down
# kernel to stage in LDS (T * (K + 1) rows of 1 KB): the token-group down
# kernel then reads each tier table up to its last block, whose code field is
# loaded from a window moved back to end inside the table.
KE_WIDE = synth.LayerSpec(hidden=256, inter=512, n_experts=8, top_k=8, has_shared=True,
                          act="bf16", n_slots=(2, 4, 2))


@pytest.mark.parametrize("down_bits", [None, (MX, 2, 3)])
def test_group_down_reads_every_table_to_its_end(down_bits):
    spec = KE_WIDE.with_(down_bits=down_bits)
    tl = make_layer(spec, seed=23)
    for T in (6, 16):
        x = synth.tokens(spec, T, 180 + T)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol, exact_keys=True)
        for y_dt, want in ((M.MOE_F32, ref["y"]), (M.MOE_BF16, O.output_cast(ref["y"], "bf16"))):
            y, ids, w = run_decode(tl, x, y_dt)
            np.testing.assert_array_equal(ids, ref["ids"])
            assert np.all(np.sort(ids, axis=1) == np.arange(spec.n_experts))
            check_y(y, want, "bf16", f"decode T={T}, every expert, down bits {down_bits}")


def test_full_size_mixed_formats():
    # full-size layer with both format families in gate/up (tier 0 MXFP4,
    # tiers 1-2 affine) and in down (tier 0 affine, tiers 1-2 MXFP4), so each
    # matrix runs both prefill kernels, in the launch configuration the
    # benchmark times
    spec = synth.FULL.with_(tier_bits=(MX, 3, 2), down_bits=(4, MX, MX))
    print("\n[layer] full-size mixed formats", flush=True)
    tl = make_layer(spec, seed=8, source="codes", n_calib=4096)
    xs1 = synth.tokens(spec, 3, 120)
    for i in range(3):
        x = xs1[i:i + 1]
        y, ids, w = run_decode(tl, x, M.MOE_BF16)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        np.testing.assert_array_equal(ids, ref["ids"])
        check_y(y, O.output_cast(ref["y"], "bf16"), "bf16", f"decode full mixed token {i}")
    T = 4096
    x = synth.tokens(spec, T, 121)
    y, ids, w, off, srt = run_prefill(tl, x, M.MOE_BF16)
    xs = act_f64(x, "bf16")
    keys, oids, g = O.route(xs, tl.ol.w_router, tl.ol.bias, spec.top_k)
    np.testing.assert_array_equal(ids, oids)
    print("  oracle over all 4096 rows ...", flush=True)
    ref = O.moe_layer(xs, tl.ol, routing=(keys, oids, g), drop_experts=True)
    check_y(y, O.output_cast(ref["y"], "bf16"), "bf16", "prefill full mixed T=4096 (every row)")


@pytest.mark.parametrize("spec_name", ["odd", "i640"])
def test_mxfp4_register_staged_paths(spec_name):
    # contraction lengths that are not a power-of-two number of 128-chunks
    # (3 chunks; down K = 640, five chunks) run the register-staged prefill
    # body; here with MXFP4 and affine tiers mixed in both matrices
    base = ODD if spec_name == "odd" else I640
    spec = base.with_(tier_bits=(4, MX, 2), down_bits=(MX, 3, MX))
    tl = make_layer(spec, seed=15)
    for T in (1, 4):
        x = synth.tokens(spec, T, 140 + T)
        y, ids, w = run_decode(tl, x)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol, exact_keys=True)
        np.testing.assert_array_equal(ids, ref["ids"])
        check_y(y, ref["y"], "bf16", f"decode T={T}, {spec_name} mixed formats")
    x = synth.tokens(spec, 200, 145)
    y, ids, w, _, _ = run_prefill(tl, x)
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol, exact_keys=True)
    np.testing.assert_array_equal(ids, ref["ids"])
    check_y(y, ref["y"], "bf16", f"prefill T=200, {spec_name} mixed formats")


def test_decode_wide_default_router_128_threads():
    # hidden 256: the one-token gate/up workgroups have 128 threads, each
    # holding one of the 128 keys; the whole 256-bin histogram must start
    # cleared.  T = 17 ends with a one-token group after a full group of 16.
    tl = make_layer(WIDE, seed=18)
    for T in (1, 17):
        for seed in (150, 151, 152):
            x = synth.tokens(WIDE, T, seed + T)
            y, ids, w = run_decode(tl, x)
            _, oids, g = O.route(act_f64(x, "bf16"), tl.ol.w_router, tl.ol.bias, WIDE.top_k,
                                 exact=True)
            np.testing.assert_array_equal(ids, oids)
            assert np.max(np.abs(w - g)) <= 1e-6
            ref = O.moe_layer(act_f64(x, "bf16"), tl.ol, exact_keys=True)
            check_y(y, ref["y"], "bf16", f"decode T={T} seed {seed}, H=256 E=128")


# top-1 (every mixing weight exactly 1) and top-E (every expert chosen)
K1 = synth.LayerSpec(hidden=256, inter=128, n_experts=16, top_k=1, has_shared=True, act="bf16",
                     n_slots=(4, 8, 4))
KE = synth.LayerSpec(hidden=256, inter=128, n_experts=8, top_k=8, has_shared=False, act="bf16",
                     n_slots=(2, 4, 2))


@pytest.mark.parametrize("spec_name", ["k1", "ke"])
def test_top_one_and_top_all(spec_name):
    spec = K1 if spec_name == "k1" else KE
    tl = make_layer(spec, seed=19)
    xs = act_f64
    for T in (1, 5):
        x = synth.tokens(spec, T, 160 + T)
        y, ids, w = run_decode(tl, x)
        ref = O.moe_layer(xs(x, "bf16"), tl.ol, exact_keys=True)
        np.testing.assert_array_equal(ids, ref["ids"])
        check_y(y, ref["y"], "bf16", f"decode T={T}, {spec_name}")
        if spec.top_k == 1:
            assert np.all(w == np.float32(1.0))
        else:
            assert np.all(np.sort(ids, axis=1) == np.arange(spec.n_experts))
            assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-6
    x = synth.tokens(spec, 100, 170)
    y, ids, w, off, srt = run_prefill(tl, x)
    ref = O.moe_layer(xs(x, "bf16"), tl.ol, exact_keys=True)
    np.testing.assert_array_equal(ids, ref["ids"])
    o_off, o_srt = O.sort_routes(ids, spec.n_experts)
    np.testing.assert_array_equal(off, o_off)
    np.testing.assert_array_equal(srt, o_srt)
    check_y(y, ref["y"], "bf16", f"prefill T=100, {spec_name}")
    if spec.top_k == 1:
        assert np.all(w == np.float32(1.0))
    else:
        assert np.all(np.diff(off) == 100)


def test_planned_tiers_through_decode_and_prefill():
    # the byte-budget planner's split drives the forward path: plan with a
    # down ladder for a budget that leaves the 2-bit tier empty and the other
    # two uneven, check the oracle's planner agrees, then build the tables at
    # that split and run decode and prefill against the oracle
    import layers
    spec = MID.with_(down_bits=(4, 4, 3))
    w_router, bias = synth.router(spec, 21)
    pop = layers.popularity_from_calibration(spec, w_router, bias, 22)
    per = {b: O.expert_table_bytes(spec.hidden, spec.inter, b) for b in (4, 3, 2)}
    # room for 28 experts at 4 bits and 4 at 3 bits (down at 4 bits): the
    # least-error plan spends it exactly so, with no 2-bit expert
    budget = 28 * per[4] + 4 * (2 * per[3] // 3 + per[4] // 3)
    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, spec.has_shared, spec.act)
    plan = M.plan_tiers(d, pop, spec.tier_bits, budget, down_bits=spec.down_bits)
    want = O.plan_tiers(pop, spec.tier_bits, spec.hidden, spec.inter, budget, spec.down_bits)
    assert tuple(plan) == tuple(want)
    print(f"  planned split {tuple(plan)} for {budget} bytes", flush=True)
    assert plan[2] == 0 and plan[0] != plan[1] and sum(plan) == spec.n_experts
    tl = make_layer(spec.with_(n_slots=tuple(int(v) for v in plan)), seed=21)
    want_map, _ = O.build_tiers(tl.popularity, tuple(int(v) for v in plan))
    np.testing.assert_array_equal(tl.tier_map, want_map)
    for T in (1, 5):
        x = synth.tokens(spec, T, 180 + T)
        y, ids, w = run_decode(tl, x)
        ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
        np.testing.assert_array_equal(ids, ref["ids"])
        check_y(y, ref["y"], "bf16", f"decode T={T}, planned split {tuple(plan)}")
    x = synth.tokens(spec, 300, 186)
    y, ids, w, _, _ = run_prefill(tl, x)
    ref = O.moe_layer(act_f64(x, "bf16"), tl.ol)
    np.testing.assert_array_equal(ids, ref["ids"])
    check_y(y, ref["y"], "bf16", f"prefill T=300, planned split {tuple(plan)}")


def test_check_layer_flags_bad_tier_maps(mid):
    # a valid map passes; an entry past its tier, an unknown tier or a slot
    # named twice is refused (the forward calls would skip such an expert)
    d, L = mid.dl.d, mid.dl.c_struct()
    assert M.check_layer(d, L) == M.MOE_OK
    good = mid.dl.tier_map.clone()
    try:
        for bad in ((0, (3 << 16) | 0), (1, (0 << 16) | mid.spec.n_slots[0]),
                    (2, int(good[3].item()))):
            e, v = bad
            mid.dl.tier_map.copy_(good)
            mid.dl.tier_map[e] = v
            torch.cuda.synchronize()
            assert M.check_layer(d, L) == M.MOE_EINVAL, bad
    finally:
        mid.dl.tier_map.copy_(good)
        torch.cuda.synchronize()
    assert M.check_layer(d, L) == M.MOE_OK


# The coldest tier kept in system RAM (P1 "step 3: split every layer into hot
# and cold"): its tables in pinned host memory mapped into the device's
# address space, read by the same kernels over the host link.  Routing, ids
# and outputs are bit-identical to the layer whose tables all sit in HBM.
def test_host_resident_cold_tier(mid):
    hl = make_layer(MID, seed=5, host_tiers=(2,))
    for m in range(3):
        assert hl.dl.codes[2][m].device.type == "cpu" and hl.dl.codes[2][m].is_pinned()
        assert hl.dl.codes[0][m].is_cuda and hl.dl.codes[1][m].is_cuda
    np.testing.assert_array_equal(hl.tier_map, mid.tier_map)
    assert M.check_layer(hl.dl.d, hl.dl.c_struct()) == M.MOE_OK
    for T in (1, 5, 40):
        x = synth.tokens(MID, T, 300 + T)
        ref = O.moe_layer(act_f64(x, "bf16"), mid.ol)
        for name, run in (("decode", run_decode), ("prefill", run_prefill)):
            yd, idd, wd = run(mid, x)[:3]
            yh, idh, wh = run(hl, x)[:3]
            np.testing.assert_array_equal(idh, ref["ids"])
            np.testing.assert_array_equal(idh, idd)
            np.testing.assert_array_equal(wh.view(np.uint32), wd.view(np.uint32))
            assert torch.equal(yh.view(torch.int32), yd.view(torch.int32)), (name, T)
            check_y(yh, ref["y"], "bf16", f"{name} T={T}, 2-bit tier in host memory")

