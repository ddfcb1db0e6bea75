#!/usr/bin/env python3
"""Throughput of the routed, tiered, dequantised MoE layer on one MI355X.

Metric: MoE-layer tokens/s for batch-1 decode of one full-size layer
(hidden 2048, 512 experts, top-10 + 1 shared, intermediate 512, bf16
activations, experts tiered 128/256/128 at 4/3/2 bits in blocks of 32).

One step = one token decoded through a stack of 48 independent full-size
layers (distinct weights, 36 GiB of packed tiers resident in HBM), so every
layer reads its experts from HBM rather than from the 256 MB last-level
cache; value = 48 * steps / elapsed seconds.  Each token/layer pair has its
own N(0,1) input row.  The 48 layer calls of one token are captured in one
HIP graph; 16 graphs (16 token rows) are replayed round-robin.

Also reported: per-kernel durations from the library's launch trace (HIP
events attached to each kernel dispatch) over an eager pass of the same
16 x 48 calls right after the timed region, the HBM roofline of the dominant
decode kernel, prefill of 4096 tokens through one layer (rotating over the
stack; timed as replays of one graph of 8 layer calls, its per-kernel figures
from a traced eager pass) with the MFMA roofline of its grouped GEMM, and the
CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 64] [--warmup 16]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
N_LAYERS = 48
N_GRAPHS = 16


MXFP4 = 0x14                   # format code of MXFP4 tables


def _formats(text):
    out = tuple(MXFP4 if v.strip().lower() == "mx" else int(v) for v in text.split(","))
    if len(out) != 3:
        raise argparse.ArgumentTypeError("three comma-separated formats")
    return out


def fmt_name(f):
    return "MXFP4" if f == MXFP4 else f"{f}-bit"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prefill-steps", type=int, default=8)
    ap.add_argument("--prefill-tokens", type=int, default=4096)
    ap.add_argument("--cpu-tokens", type=int, default=320)
    ap.add_argument("--cpu-tokens-1t", type=int, default=96,
                    help="tokens of the one-thread oracle figure (0: skip)")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the verify-batch leg (T = 4, 8, 16 correlated tokens)")
    ap.add_argument("--no-cold-tier", action="store_true",
                    help="skip the leg with the 2-bit tier in pinned host memory")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-ceiling leg (torch GEMV over 48 x 25.8 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graphs")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--tier-bits", default="4,3,2", type=_formats,
                    help="code format of each tier: 2, 3, 4 or mx (MXFP4)")
    ap.add_argument("--down-bits", default=None, type=_formats,
                    help="the down matrices' own format per tier (0: the tier's)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run an elementwise copy of 256 MiB (fp32 -> fp32) three times, the "
                         "known-size reference for HBM byte counters")
    ap.add_argument("--traffic-json", nargs="+", metavar="DIR",
                    help="write profiles/hbm_traffic.json from the FETCH_SIZE / WRITE_SIZE "
                         "counter runs under DIR(s) (taken with --calib-copy)")
    ap.add_argument("--prof-summary", nargs=3, metavar=("DIR", "COMMAND", "TITLE"),
                    help="print a markdown summary of a rocprofv3 output directory and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# synthetic full-size layers, generated on the device
# ---------------------------------------------------------------------------

def make_stack(M, torch, spec, n_layers, seed):
    """48 full-size layers with seeded random tables (torch Philox on the GPU).

    Tier tables: iid uniform code bytes (every byte pattern is a valid code
    field), scales d = sigma / std(q) * U(0.8, 1.2) and mins
    m = -d L / 2 + N(0, (0.05 sigma)^2), sigma = 1/sqrt(fan_in), so the
    dequantised weights have std ~ 1/sqrt(fan_in); MXFP4 tables take the
    scale 2^X with X = round(log2(sigma / 2.93)) - {0 or 1} per block.  Router N(0, 0.02^2) in
    bf16 with bias 0.27 * N(0, 1); shared expert N(0, 1/fan_in) in bf16.
    Popularity per layer: route counts of 4096 N(0,1) calibration tokens
    (moe_route), ranked into tiers by moe_build_tiers.
    """
    import synth

    d = M.dims(spec.hidden, spec.inter, spec.n_experts, spec.top_k, True, "bf16")
    H, I, E = spec.hidden, spec.inter, spec.n_experts
    gen = torch.Generator(device="cuda")
    layers = []
    calib_ids = torch.empty((4096, spec.top_k), dtype=torch.int32, device="cuda")
    calib_w = torch.empty((4096, spec.top_k), dtype=torch.float32, device="cuda")
    for l in range(n_layers):
        gen.manual_seed(seed * 1000 + l)
        w_r = (torch.randn((E, H), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
        bias = (torch.randn(E, generator=gen, device="cuda") * synth.DEFAULT_BIAS_BETA).float()
        shared = [(torch.randn(shape, generator=gen, device="cuda") / np.sqrt(shape[1])).to(torch.bfloat16)
                  for shape in ((I, H), (I, H), (H, I))]
        lay = M.DeviceLayer(d, spec.n_slots, spec.tier_bits, (w_r, bias), shared,
                            down_bits=spec.down_bits)
        for t in range(3):
            for m in range(3):
                bits = lay.matrix_bits(t, m)
                fan_in = H if m != M.MOE_DOWN else I
                sigma = 1.0 / np.sqrt(fan_in)
                c = lay.codes[t][m]
                c.copy_(torch.randint(0, 256, c.shape, generator=gen, device="cuda", dtype=torch.uint8))
                n = lay.dm[t][m].numel()
                if bits == MXFP4:
                    # uniform E2M1 codes have rms 2.93: scale 2^X ~ sigma / 2.93
                    x0 = int(np.round(np.log2(sigma / 2.93)))
                    e = 127 + x0 - torch.randint(0, 2, (n,), generator=gen, device="cuda")
                    lay.dm[t][m].copy_(e.to(torch.uint8))
                    continue
                L = (1 << bits) - 1
                std_q = float(np.sqrt(((L + 1) ** 2 - 1) / 12.0))
                dd = (sigma / std_q) * (0.8 + 0.4 * torch.rand(n, generator=gen, device="cuda"))
                mm = -dd * (L / 2.0) + 0.05 * sigma * torch.randn(n, generator=gen, device="cuda")
                db = dd.half().view(torch.int16).to(torch.int32) & 0xFFFF
                mb = mm.half().view(torch.int16).to(torch.int32) & 0xFFFF
                lay.dm[t][m].copy_(db | (mb << 16))
        xc = torch.randn((4096, H), generator=gen, device="cuda").to(torch.bfloat16)
        M.route(d, lay.c_struct(), xc, calib_ids, calib_w)
        pop = torch.bincount(calib_ids.flatten().long(), minlength=E).cpu().numpy().astype(np.uint64)
        tmap, _ = M.build_tiers(d, pop, spec.n_slots, spec.tier_bits)
        lay.tier_map.copy_(torch.from_numpy(tmap))
        lay.popularity = pop
        lay.tmap_host = tmap
        lay.cs = lay.c_struct()
        layers.append(lay)
        if l % 8 == 7:
            log(f"built layers 0..{l}")
    torch.cuda.synchronize()
    return d, layers


def sources_sha256():
    """Hash of the library's device sources (the .hip kernels with their
    launchers and the shared device header): a kernel's memory traffic depends
    on nothing else."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_expert_ffn_route_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter record
    (profiles/hbm_traffic.json), or None when the record is missing or was
    taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != sources_sha256():
        return None
    b = rec.get("per_launch_bytes", {}).get(kernel)
    return None if b is None else int(b["read"] + b["write"])


def table_bytes(spec, bits, mat):
    rows, cols = (spec.hidden, spec.inter) if mat == 2 else (spec.inter, spec.hidden)
    blocks = rows * cols // 32
    return blocks * (17 if bits == MXFP4 else 4 * bits + 4)


def down_format(spec, t):
    return spec.down_bits[t] if spec.down_bits and spec.down_bits[t] else spec.tier_bits[t]


def decode_kernel_bytes(spec, layer, ids_row):
    """Algorithmic HBM bytes of each decode kernel for one token (T = 1).

    router_keys: router weights + bias + x + keys written.  topk_items: keys
    read, ids/weights/items written.  decode_gateup: gate+up blocks (codes and
    scale/min) of the K chosen experts at their tier widths + the shared
    expert's bf16 gate/up + x + h written.  decode_down: down blocks of the K
    experts + shared bf16 down + h read + y written (bf16).
    """
    H, I, E, K = spec.hidden, spec.inter, spec.n_experts, spec.top_k
    tiers = [int(layer.tmap_host[e]) >> 16 for e in ids_row]
    gu = sum(table_bytes(spec, spec.tier_bits[t], 0) + table_bytes(spec, spec.tier_bits[t], 1)
             for t in tiers) + 2 * I * H * 2
    dn = sum(table_bytes(spec, down_format(spec, t), 2) for t in tiers) + H * I * 2
    return {
        "router_keys": E * H * 2 + E * 4 + H * 2 + E * 8,
        "topk_items": E * 8 + K * 8 + (K + 1) * 136,
        "decode_gateup": gu + H * 2 + (K + 1) * I * 2,
        "decode_down": dn + (K + 1) * I * 2 + H * 2,
    }


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_model():
    """Model name of the host CPU (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(n_tokens, seed, n_tokens_1t=0):
    """The oracle on batch-1 decode tokens through one full-size layer, with
    BLAS on every host thread, and (n_tokens_1t > 0) again on one thread."""
    import oracle as O
    import synth
    from threadpoolctl import threadpool_limits

    spec = synth.FULL
    cores = len(os.sched_getaffinity(0))
    w_router, bias = synth.router(spec, seed)
    shared = synth.shared_expert(spec, seed + 3)
    wr64 = O.bf16_bits_to_f64(w_router)
    xc = O.bf16_bits_to_f64(synth.tokens(spec, 4096, seed + 1))
    ids_c = O.select_topk(O.router_keys(xc, wr64, bias), spec.top_k)
    pop = np.bincount(ids_c.ravel(), minlength=spec.n_experts).astype(np.uint64)
    tmap, _ = O.build_tiers(pop, spec.n_slots)
    x = O.bf16_bits_to_f64(synth.tokens(spec, n_tokens, seed + 4))
    routing = O.route(x, wr64, bias, spec.top_k)
    touched = sorted(set(int(e) for e in routing[1].ravel()))
    blocks = {}
    for e in touched:            # input generation, outside the timed region
        b = spec.tier_bits[int(tmap[e]) >> 16]
        p = synth.expert_codes(spec, b, seed + 2, e)
        blocks[e] = O.ExpertBlocks(b, p["gate"], p["up"], p["down"])
    layer = O.OracleLayer(act="bf16", w_router=wr64, bias=bias, top_k=spec.top_k,
                          experts=lambda e: blocks[e],
                          shared=tuple(O.bf16_bits_to_f64(s) for s in shared))
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for t in range(n_tokens):       # batch-1 decode: one token per call
            O.moe_layer(x[t:t + 1], layer)
        dt = time.perf_counter() - t0
    out = {"value": n_tokens / dt, "unit": "MoE-layer tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n_tokens} batch-1 decode tokens through one full-size layer (host-generated "
                     f"seeded blocks of the same shapes and tiers); NumPy fp64, BLAS on {cores} "
                     f"threads, element-wise dequantisation single-threaded; {dt:.1f} s"}
    if n_tokens_1t > 0:
        # the same tokens again on one thread; the touched experts' dequantised
        # weights are dropped first so that the rate includes them, as above
        layer._cache.clear()
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            for t in range(n_tokens_1t):
                O.moe_layer(x[t:t + 1], layer)
            dt1 = time.perf_counter() - t0
        out["one_thread"] = {"value": n_tokens_1t / dt1, "cores": 1,
                             "sample": f"the first {n_tokens_1t} of the same tokens, BLAS on one "
                                       f"thread; {dt1:.1f} s"}
    return out


# ---------------------------------------------------------------------------

def prof_summary(out_dir, command, title):
    """Markdown summary of rocprofv3 output under out_dir: per-kernel durations
    (kernel_stats / kernel_trace csv) and, when present, per-dispatch averages
    of the collected counters (counter_collection csv)."""
    import csv
    import glob

    def rows(pattern):
        out = []
        for f in sorted(glob.glob(os.path.join(out_dir, "**", pattern), recursive=True)):
            with open(f, newline="") as fh:
                out.extend(csv.DictReader(fh))
        return out

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "")
        return name.split("(")[0]

    print(f"# {title}\n")
    print("Command (repository root in `$R`, run from /tmp with TMPDIR=/tmp):\n")
    print(f"```\n{command}\n```\n")
    trace = rows("*kernel_trace.csv")
    if trace:
        agg = {}
        for r in trace:
            n = r.get("Kernel_Name", "")
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            a = agg.setdefault(short(n), [0, 0.0, 1e30, 0.0, r.get("Grid_Size_X", ""),
                                          r.get("Workgroup_Size_X", ""), r.get("VGPR_Count", ""),
                                          r.get("LDS_Block_Size", "")])
            a[0] += 1
            a[1] += d
            a[2] = min(a[2], d)
            a[3] = max(a[3], d)
        print("Per-kernel durations (`--kernel-trace`), library kernels:\n")
        print("| kernel | launches | avg us | min us | max us | grid | wg | vgpr | lds |")
        print("|---|---|---|---|---|---|---|---|---|")
        for n, a in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            if "moe::" not in n:
                continue
            print(f"| `{n}` | {a[0]} | {a[1] / a[0]:.2f} | {a[2]:.2f} | {a[3]:.2f} | {a[4]} | {a[5]} "
                  f"| {a[6]} | {a[7]} |")
        print()
        # the streaming ceiling leg: torch's bf16 GEMV over one layer's bytes
        # (a library kernel, matched by the trace's include regex)
        ceil = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                if r.get("Kernel_Name", "").startswith("Cijk_") or "gemv" in r.get("Kernel_Name", "")]
        if ceil:
            print("Streaming ceiling leg (`torch.mv`, bf16, one layer's bytes per launch): "
                  f"{len(ceil)} launches, {np.median(ceil):.2f} us median "
                  f"[{np.percentile(ceil, 10):.2f}-{np.percentile(ceil, 90):.2f}], "
                  f"{np.mean(ceil):.2f} us mean.\n")
        # the decode kernels by phase of the bench run: eager warm-up passes
        # before capture, graph replays, and the traced eager pass (the last
        # N_GRAPHS x N_LAYERS launches) whose events give the bench line's
        # per-kernel averages
        n_pass = N_GRAPHS * N_LAYERS
        phase = {}
        for r in trace:
            n = short(r.get("Kernel_Name", ""))
            if "moe::k_decode" in n or "moe::k_router_keys_dec" in n:
                phase.setdefault(n, []).append((int(r["Start_Timestamp"]),
                                                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        if phase:
            print("Decode kernels by phase of the run (average us): warm-up passes before graph "
                  "capture, graph replays, and the last traced eager pass that the bench line's "
                  "per-kernel figures time:\n")
            print("| kernel | warm-up | replays | traced eager pass |")
            print("|---|---|---|---|")
            for n, v in sorted(phase.items()):
                d = [x for _, x in sorted(v)]
                if len(d) <= 2 * n_pass:
                    continue
                warm, rep, last = d[:n_pass], d[n_pass:len(d) - n_pass], d[len(d) - n_pass:]
                print(f"| `{n}` | {sum(warm) / len(warm):.2f} | {sum(rep) / max(1, len(rep)):.2f} "
                      f"| {sum(last) / len(last):.2f} |")
            print()
        # per-layer timeline of the replayed decode graphs: each layer is the
        # chain router keys -> gate/up -> down; durations of the three kernels
        # and the gaps between one kernel's end and the next one's start
        seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short(r.get("Kernel_Name", "")))
                     for r in trace if "moe::k_decode1" in short(r.get("Kernel_Name", ""))
                     or "moe::k_router_keys_dec" in short(r.get("Kernel_Name", "")))
        order = ("k_router_keys_dec", "k_decode1_gateup", "k_decode1_down")
        layers_t = []
        for i in range(len(seq) - 3):
            a, b, c, nxt = seq[i], seq[i + 1], seq[i + 2], seq[i + 3]
            if all(o in x[2] for o, x in zip(order, (a, b, c))) and order[0] in nxt[2] \
                    and "true" in a[2] and nxt[0] - c[1] < 20000:
                layers_t.append((a[1] - a[0], b[0] - a[1], b[1] - b[0], c[0] - b[1], c[1] - c[0],
                                 nxt[0] - c[1], nxt[0] - a[0]))
        # drop the eager passes: keep layers whose chain gaps look like graph replays
        if layers_t:
            arr = np.array(layers_t, dtype=np.float64) / 1e3
            med_gap = np.median(arr[:, 5])
            rep = arr[arr[:, 5] <= 4 * max(med_gap, 0.5)]
            print(f"Per-layer timeline of batch-1 decode ({len(rep)} consecutive layer chains "
                  "router -> gate/up -> down whose next layer starts within a few us, i.e. graph "
                  "replays; us, median [10th-90th percentile]):\n")
            print("| router | gap | gate/up | gap | down | gap to next layer | layer start to next |")
            print("|---|---|---|---|---|---|---|")
            print("| " + " | ".join(f"{np.median(rep[:, k]):.2f} [{np.percentile(rep[:, k], 10):.2f}-"
                                     f"{np.percentile(rep[:, k], 90):.2f}]" for k in range(7)) + " |")
            print()
    ctr = rows("*counter_collection.csv")
    if ctr:
        agg = {}
        r_name_of = {}
        for r in ctr:
            n = short(r.get("Kernel_Name", ""))
            r_name_of[n] = r.get("Kernel_Name", "")
            key = (n, r.get("Counter_Name", ""))
            a = agg.setdefault(key, [0, 0.0])
            a[0] += 1
            a[1] += float(r.get("Counter_Value", 0.0))
        # calibration: the largest elementwise negation (bench --calib-copy, 256 MiB each way)
        calib = {}
        for r in ctr:
            if "neg_kernel" in r.get("Kernel_Name", ""):
                g = int(r.get("Grid_Size", 0))
                c = r.get("Counter_Name", "")
                if g >= calib.get(c, (0, 0.0))[0]:
                    calib[c] = (g, float(r.get("Counter_Value", 0.0)))
        factor = {c: (256 * 1024) / v for c, (g, v) in calib.items() if v > 0}
        print("Counters, average per dispatch (`--pmc`), in KiB as reported; the scaled column "
              "multiplies by the factor that maps the 256 MiB reference copy (read once, "
              "written once) onto its true size:\n")
        for c, f in sorted(factor.items()):
            print(f"- {c}: reference copy counted {calib[c][1]:.0f} KiB -> factor {f:.4f}")
        print()
        print("| kernel | counter | dispatches | avg (KiB for byte counters) | scaled bytes per dispatch |")
        print("|---|---|---|---|---|")
        for (n, c), a in sorted(agg.items()):
            if "moe::" not in n:
                continue
            v = a[1] / a[0]
            scaled = f"{v * 1024 * factor[c]:.0f}" if c in factor else "-"
            print(f"| `{n}` | {c} | {a[0]} | {v:.4g} | {scaled} |")
        print()
        # derived figures when the instruction and busy counters are present:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's active
        # cycles are a eighth of it; 256 CUs x 4 SIMDs; a wave64 VALU
        # instruction occupies its SIMD for 4 cycles
        names = sorted({n for (n, c) in agg if "moe::" in n})
        avg = {(n, c): a[1] / a[0] for (n, c), a in agg.items()}
        if any((n, "SQ_VALU_MFMA_BUSY_CYCLES") in avg for n in names):
            print("Derived per dispatch (GUI = GRBM_GUI_ACTIVE / 8, one XCD's active cycles; "
                  "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI x 1024 SIMDs); VALU issue = 4 x "
                  "SQ_INSTS_VALU / (GUI x 1024); bf16 MFMA flops = 512 x "
                  "SQ_INSTS_VALU_MFMA_MOPS_BF16):\n")
            print("| kernel | GUI cycles | MFMA busy | VALU issue | VALU / MFMA instructions | bf16 MFMA GFLOP |")
            print("|---|---|---|---|---|---|")
            for n in names:
                g = avg.get((n, "GRBM_GUI_ACTIVE"), 0.0) / 8
                if not g:
                    continue
                mb = avg.get((n, "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0) / (g * 1024)
                vi = 4 * avg.get((n, "SQ_INSTS_VALU"), 0.0) / (g * 1024)
                nm = avg.get((n, "SQ_INSTS_MFMA"), 0.0)
                ratio = f"{avg.get((n, 'SQ_INSTS_VALU'), 0.0) / nm:.2f}" if nm else "-"
                gf = 512 * avg.get((n, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), 0.0) / 1e9
                print(f"| `{n}` | {g:.0f} | {100 * mb:.1f}% | {100 * vi:.1f}% | {ratio} | {gf:.1f} |")
            print()


# the kernel that runs gate/up in batch-1 decode (the dominant decode kernel)
DECODE_GATEUP_KERNEL = "k_decode1_gateup"


def verify_batches(M, torch, spec, d, layers, args, sizes=(4, 8, 16), n_graphs=4):
    """Small-batch verify decode: T correlated tokens (x_t = sqrt(0.6) z_0 +
    sqrt(0.4) z_t, mean pairwise cosine ~0.6, so their experts overlap)
    through the 48-layer stack, one HIP graph per batch of 48 layer calls,
    n_graphs batches replayed round-robin.  Reports MoE-layer tokens/s, the
    mean union of experts per layer call, the union's algorithmic bytes and
    their HBM fraction."""
    H = spec.hidden
    out = {}
    gen = torch.Generator(device="cuda")
    for T in sizes:
        gen.manual_seed(args.seed + 100 + T)
        z0 = torch.randn((n_graphs, N_LAYERS, 1, H), generator=gen, device="cuda")
        zt = torch.randn((n_graphs, N_LAYERS, T, H), generator=gen, device="cuda")
        X = (np.sqrt(0.6) * z0 + np.sqrt(0.4) * zt).to(torch.bfloat16)
        Y = torch.empty((N_LAYERS, T, H), dtype=torch.bfloat16, device="cuda")
        IDS = torch.empty((n_graphs, N_LAYERS, T, spec.top_k), dtype=torch.int32, device="cuda")
        WTS = torch.empty((n_graphs, N_LAYERS, T, spec.top_k), dtype=torch.float32, device="cuda")
        ws = torch.empty(M.workspace_bytes("decode", d, layers[0].cs, T, M.MOE_BF16),
                         dtype=torch.uint8, device="cuda")

        def batch_pass(g):
            for l in range(N_LAYERS):
                M.forward_decode(d, layers[l].cs, X[g, l], Y[l], M.MOE_BF16, IDS[g, l], WTS[g, l],
                                 ws=ws)

        graphs = []
        for g in range(n_graphs):
            batch_pass(g)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                batch_pass(g)
            graphs.append(graph)
        for k in range(args.warmup):
            graphs[k % n_graphs].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[k % n_graphs].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # per-kernel durations: one eager pass of each batch with the launch trace
        trace = M.Trace(n_graphs * N_LAYERS * 8)
        with trace:
            for g in range(n_graphs):
                batch_pass(g)
        torch.cuda.synchronize()
        kd = {}
        for name, ms in trace.durations_ms():
            kd.setdefault(name, []).append(1e3 * ms)
        ids = IDS.cpu().numpy()
        unions, nbytes = [], []
        for g in range(n_graphs):
            for l in range(N_LAYERS):
                u = np.unique(ids[g, l])
                unions.append(len(u))
                tiers = [int(layers[l].tmap_host[e]) >> 16 for e in u]
                routed = sum(table_bytes(spec, spec.tier_bits[t], 0) + table_bytes(spec, spec.tier_bits[t], 1)
                             + table_bytes(spec, down_format(spec, t), 2) for t in tiers)
                nbytes.append(routed + 3 * spec.inter * H * 2 + spec.n_experts * (H * 2 + 4)
                              + 2 * T * H * 2)
        us_layer = 1e6 * wall / (args.steps * N_LAYERS)
        mean_bytes = float(np.mean(nbytes))
        gbs = mean_bytes / (us_layer * 1e-6) / 1e9
        out[f"T{T}"] = {"tokens_per_s": round(T * N_LAYERS * args.steps / wall, 1),
                        "us_per_layer": round(us_layer, 3),
                        "mean_union": round(float(np.mean(unions)), 2),
                        "bytes_per_layer": int(mean_bytes),
                        "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "kernels_avg_us": {n: round(float(np.mean(v)), 2) for n, v in kd.items()}}
        log(f"verify T={T}: {out[f'T{T}']}")
        del graphs, X, zt, z0
    return {"workload": "verify decode: T correlated tokens (cosine ~0.6) per layer call through "
                        "the 48-layer stack, one graph per batch of 48 layer calls",
            "unit": "MoE-layer tokens/s", **out}


def host_cold_tier(M, torch, spec, d, layers, args, n_graphs=4, tier=2):
    """Batch-1 decode with one tier kept in system RAM (P1 "step 3: split every
    layer into hot and cold"): the same 48 layers with tier `tier`'s tables
    copied into pinned host memory mapped into the device's address space, so
    the kernels read those experts over the host link.  Reports us per layer,
    the host-resident bytes a layer-token reads (the routed experts of that
    tier) and whether the outputs equal the all-HBM layers' bit for bit."""
    import copy
    H, K = spec.hidden, spec.top_k
    host_layers = []
    for lay in layers:
        hl = copy.copy(lay)
        hl.codes = [list(r) for r in lay.codes]
        hl.dm = [list(r) for r in lay.dm]
        for m in range(3):
            hl.codes[tier][m] = lay.codes[tier][m].to("cpu").pin_memory()
            hl.dm[tier][m] = lay.dm[tier][m].to("cpu").pin_memory()
        hl.host_tiers = (tier,)
        hl.cs = hl.c_struct()
        host_layers.append(hl)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed + 31)
    X = torch.randn((n_graphs, N_LAYERS, 1, H), generator=gen, device="cuda").to(torch.bfloat16)
    Y = torch.empty((N_LAYERS, 1, H), dtype=torch.bfloat16, device="cuda")
    Yd = torch.empty_like(Y)
    IDS = torch.empty((n_graphs, N_LAYERS, 1, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(M.workspace_bytes("decode", d, layers[0].cs, 1, M.MOE_BF16),
                     dtype=torch.uint8, device="cuda")

    def token_pass(g, lays, out):
        for l in range(N_LAYERS):
            M.forward_decode(d, lays[l].cs, X[g, l], out[l], M.MOE_BF16, IDS[g, l], None, ws=ws)

    # bit-for-bit against the all-HBM layers on the same inputs
    token_pass(0, layers, Yd)
    token_pass(0, host_layers, Y)
    torch.cuda.synchronize()
    same = bool(torch.equal(Y.view(torch.int16), Yd.view(torch.int16)))
    graphs = []
    for g in range(n_graphs):
        token_pass(g, host_layers, Y)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            token_pass(g, host_layers, Y)
        graphs.append(graph)
    for k in range(args.warmup):
        graphs[k % n_graphs].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        graphs[k % n_graphs].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # a 4096-token prefill touches every expert, so it reads the whole tier
    # over the host link: three calls on layer 0, after one untimed
    pf = None
    if not args.no_prefill:
        T = args.prefill_tokens
        Xp = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
        Yp = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        wsp = torch.empty(M.workspace_bytes("prefill", d, host_layers[0].cs, T, M.MOE_BF16),
                          dtype=torch.uint8, device="cuda")
        M.forward_prefill(d, host_layers[0].cs, Xp, Yp, M.MOE_BF16, ws=wsp)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(3):
            M.forward_prefill(d, host_layers[0].cs, Xp, Yp, M.MOE_BF16, ws=wsp)
        torch.cuda.synchronize()
        pf = round(1e3 * (time.perf_counter() - t1) / 3, 3)
        del Xp, Yp, wsp
    ids = IDS.cpu().numpy()
    per_expert = sum(table_bytes(spec, spec.tier_bits[tier], m) for m in (0, 1)) + \
        table_bytes(spec, down_format(spec, tier), 2)
    n_cold = [sum(1 for e in ids[g, l, 0] if int(layers[l].tmap_host[e]) >> 16 == tier)
              for g in range(n_graphs) for l in range(N_LAYERS)]
    us_layer = 1e6 * wall / (args.steps * N_LAYERS)
    out = {"workload": f"batch-1 decode through the 48-layer stack with tier {tier} "
                       f"({spec.n_slots[tier]} experts, {fmt_name(spec.tier_bits[tier])}) in pinned "
                       "host memory read over the host link",
           "layer_tokens_per_s": round(N_LAYERS * args.steps / wall, 1),
           "us_per_layer": round(us_layer, 3),
           "cold_routes_per_token": round(float(np.mean(n_cold)), 3),
           "host_bytes_per_layer": int(np.mean(n_cold) * per_expert),
           "bit_identical_to_hbm": same,
           "tier_bytes": int(spec.n_slots[tier] * per_expert),
           "prefill_ms_per_layer": pf,
           "prefill_tokens": None if pf is None else args.prefill_tokens}
    log(f"host cold tier: {out}")
    del graphs
    return out


def streaming_ceiling(torch, layer_bytes, args):
    """Measured ceiling for one layer's bytes: torch's own bf16 GEMV (one
    launch streaming a [rows x 2048] matrix of the layer's size) over 48
    distinct matrices (1.24 GB, so reads come from HBM), captured in one HIP
    graph per step like the decode step and replayed the same number of
    times.  It reads the same number of bytes per layer as the MoE layer's
    kernels but has no data-dependent step in between."""
    H = 2048
    rows = -(-layer_bytes // (2 * H))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed + 11)
    mats = [torch.randn((rows, H), generator=gen, device="cuda").to(torch.bfloat16)
            for _ in range(N_LAYERS)]
    vec = torch.randn(H, generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((N_LAYERS, rows), dtype=torch.bfloat16, device="cuda")

    def one_pass():
        for l in range(N_LAYERS):
            torch.mv(mats[l], vec, out=out[l])

    one_pass()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    us = 1e6 * (time.perf_counter() - t0) / (N_LAYERS * args.steps)
    del mats
    nbytes = rows * H * 2
    return {"op": "torch.mv, bf16 [%d x %d] (one layer's bytes), 48 distinct matrices per graph"
                  % (rows, H),
            "us_per_layer": round(us, 3), "bytes": nbytes,
            "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


# kernel symbol fragment -> name used by the launch trace and the bench line
TRAFFIC_KERNELS = [
    ("k_router_keys", "router_keys"), ("k_decode1_gateup", "decode_gateup"),
    ("k_decode_gateup", "decode_gateup"), ("k_decode1_down", "decode_down"),
    ("k_decode_down", "decode_down"),
    ("k_prefill_bf16<0,", "prefill_gateup"), ("k_prefill_bf16<2,", "prefill_down"),
    ("k_dense<0,", "route_router_approx"), ("k_dense<3,", "router_approx"),
    ("k_dense<1,", "prefill_shared_gateup"),
    ("k_dense<2,", "prefill_shared_down"), ("k_topk_recheck", "topk_recheck"),
    ("k_combine", "combine"), ("k_dense<4,", "combine"),
]


def traffic_record(dirs):
    """HBM bytes per launch of each library kernel from FETCH_SIZE / WRITE_SIZE
    counter runs (KiB per dispatch), each scaled by the factor that maps the
    256 MiB reference copy (--calib-copy) onto its true size; stamped with the
    hash of the kernel sources they were taken on."""
    import csv
    import glob
    rows = []
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(f, newline="") as fh:
                rows.extend(csv.DictReader(fh))
    calib = {}
    for r in rows:
        if "neg_kernel" in r.get("Kernel_Name", ""):
            g, c = int(r.get("Grid_Size", 0)), r["Counter_Name"]
            if g >= calib.get(c, (0, 0.0))[0]:
                calib[c] = (g, float(r["Counter_Value"]))
    factor = {c: (256 * 1024) / v for c, (g, v) in calib.items() if v > 0}
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "").replace("(anonymous namespace)::", "").replace(" ", "")
        c = r["Counter_Name"]
        key = next((k for frag, k in TRAFFIC_KERNELS if frag.replace(" ", "") in name), None)
        if key is None or c not in factor or "moe::" not in name:
            continue
        a = acc.setdefault(key, {}).setdefault(c, [0, 0.0])
        a[0] += 1
        a[1] += float(r["Counter_Value"]) * 1024 * factor[c]
    per = {k: {"read": int(v["FETCH_SIZE"][1] / v["FETCH_SIZE"][0]),
               "write": int(v["WRITE_SIZE"][1] / v["WRITE_SIZE"][0])}
           for k, v in acc.items() if "FETCH_SIZE" in v and "WRITE_SIZE" in v}
    return {
        "what": "HBM bytes per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE, each scaled by the "
                "factor that maps a 256 MiB reference copy onto its true size",
        "summary": "profiles/moe_decode_b1_prefill4096_hbm_bytes.md",
        "sources_sha256": sources_sha256(),
        "factors": {c: round(f, 4) for c, f in sorted(factor.items())},
        "per_launch_bytes": per,
    }


def main():
    args = parse()
    if args.traffic_json:
        rec = traffic_record(args.traffic_json)
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(json.dumps(rec["per_launch_bytes"]))
        return
    if args.prof_summary:
        prof_summary(*args.prof_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU build: this benchmark runs on exactly one GPU "
                          "(--gpus 1); multi-GPU sharding is not implemented"}))
        sys.exit(2)
    import torch
    import synth
    import quantized_expert_ffn_route_amd as M

    M.lib()                       # fail loudly if the HIP library is missing
    spec = synth.FULL.with_(tier_bits=args.tier_bits,
                            down_bits=None if args.down_bits is None or not any(args.down_bits)
                            else args.down_bits)
    H, I, K = spec.hidden, spec.inter, spec.top_k
    # the committed counter record was taken on the default formats
    default_fmt = spec.tier_bits == (4, 3, 2) and not spec.down_bits
    tiers_txt = "tiers 128/256/128 at " + "/".join(fmt_name(f) for f in spec.tier_bits)
    if spec.down_bits:
        tiers_txt += ", down at " + "/".join(fmt_name(down_format(spec, t)) for t in range(3))
    log("building the 48-layer stack")
    d, layers = make_stack(M, torch, spec, N_LAYERS, args.seed)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed + 7)
    X = torch.randn((N_GRAPHS, N_LAYERS, 1, H), generator=gen, device="cuda").to(torch.bfloat16)
    Y = torch.empty((N_LAYERS, 1, H), dtype=torch.bfloat16, device="cuda")
    IDS = torch.empty((N_GRAPHS, N_LAYERS, 1, K), dtype=torch.int32, device="cuda")
    WTS = torch.empty((N_GRAPHS, N_LAYERS, 1, K), dtype=torch.float32, device="cuda")
    ws_n = M.workspace_bytes("decode", d, layers[0].cs, 1, M.MOE_BF16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")

    def token_pass(g):
        for l in range(N_LAYERS):
            M.forward_decode(d, layers[l].cs, X[g, l], Y[l], M.MOE_BF16, IDS[g, l], WTS[g, l], ws=ws)

    per_graph = 4 * N_LAYERS                     # kernels per token pass
    graphs = None
    if not args.eager:
        graphs = []
        for g in range(N_GRAPHS):
            token_pass(g)                            # warm code objects and caches
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                token_pass(g)
            graphs.append(graph)
    torch.cuda.synchronize()

    def step(k):
        if graphs is None:
            token_pass(k % N_GRAPHS)
        else:
            graphs[k % N_GRAPHS].replay()

    log(f"warmup {args.warmup} steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for k in range(args.steps):
        step(k)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    value = N_LAYERS * args.steps / wall

    # Per-kernel durations: the same 16 x 48 token/layer calls launched
    # eagerly with HIP events attached to every kernel dispatch (ROCm has no
    # event-record nodes inside graphs, so the replayed graphs cannot carry
    # them).  The events time each kernel's own execution.
    trace = M.Trace(N_GRAPHS * per_graph)
    with trace:
        for g in range(N_GRAPHS):
            token_pass(g)
    torch.cuda.synchronize()
    durs = trace.durations_ms(0)
    ids_host = IDS.cpu().numpy()
    per_kernel = {}
    l = g = -1
    for name, ms in durs:
        if name == "router_keys":           # first kernel of every layer call
            l += 1
            if l % N_LAYERS == 0:
                l, g = 0, g + 1
        nbytes = decode_kernel_bytes(spec, layers[l], ids_host[g, l, 0])[name]
        pk = per_kernel.setdefault(name, {"n": 0, "ms": 0.0, "bytes": 0})
        pk["n"] += 1
        pk["ms"] += ms
        pk["bytes"] += nbytes
    kernels = {}
    for name, pk in per_kernel.items():
        avg_us = 1e3 * pk["ms"] / pk["n"]
        avg_b = pk["bytes"] / pk["n"]
        kernels[name] = {"avg_us": round(avg_us, 3), "bytes": int(avg_b),
                         "GB/s": round(avg_b / (avg_us * 1e-6) / 1e9, 1), "launches": pk["n"]}
    dom = kernels.get("decode_gateup")
    roofline = None
    if dom:
        roofline = {"bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dom["GB/s"] / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("decode_gateup") if default_fmt else None,
                    "kernel": DECODE_GATEUP_KERNEL, "bytes_per_launch": dom["bytes"],
                    "avg_us": dom["avg_us"]}
    layer_bytes = sum(k["bytes"] for k in kernels.values()) if kernels else None
    us_layer = 1e6 * wall / (N_LAYERS * args.steps)
    # the whole layer against the HBM roofline: algorithmic bytes of its
    # kernels over the graph-timed time per layer
    layer_roofline = None
    if layer_bytes:
        gbs = layer_bytes / (us_layer * 1e-6) / 1e9
        layer_roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_layer": layer_bytes, "us_per_layer": round(us_layer, 3)}
    log(f"decode: {value:.0f} layer-tokens/s, {us_layer:.2f} us/layer")

    ceiling = None if args.no_ceiling else streaming_ceiling(torch, layer_bytes or 25_838_079, args)
    verify = None if args.no_verify else verify_batches(M, torch, spec, d, layers, args)
    cold = None if args.no_cold_tier else host_cold_tier(M, torch, spec, d, layers, args)

    prefill = None
    if not args.no_prefill:
        T = args.prefill_tokens
        Xp = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
        Yp = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        wsp = torch.empty(M.workspace_bytes("prefill", d, layers[0].cs, T, M.MOE_BF16),
                          dtype=torch.uint8, device="cuda")
        def prefill_pass():
            for k in range(args.prefill_steps):
                M.forward_prefill(d, layers[k % N_LAYERS].cs, Xp, Yp, M.MOE_BF16, ws=wsp)

        prefill_pass()                           # warm code objects
        torch.cuda.synchronize()
        # timed: replays of one graph holding prefill_steps layer calls (no
        # events between the kernels); per-kernel figures: a traced eager pass
        pgraph = None
        if not args.eager:
            pgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(pgraph):
                prefill_pass()
            pgraph.replay()
            torch.cuda.synchronize()
        n_rep = 3
        t0 = time.perf_counter()
        for _ in range(n_rep):
            if pgraph is None:
                prefill_pass()
            else:
                pgraph.replay()
        torch.cuda.synchronize()
        pwall = (time.perf_counter() - t0) / n_rep
        ptrace = M.Trace(64 * args.prefill_steps)
        t1 = time.perf_counter()
        with ptrace:
            prefill_pass()
        torch.cuda.synchronize()
        pwall_traced = time.perf_counter() - t1
        del pgraph
        pk = {}
        for name, ms in ptrace.durations_ms():
            pk.setdefault(name, []).append(ms)
        routed_gu_flops = 2.0 * T * K * 2 * I * H
        layer_flops = 2.0 * T * (K * 3 * I * H + 3 * I * H + spec.n_experts * H)
        # per layer call: a matrix whose tiers mix affine and MXFP4 tables
        # runs one launch per format family
        steps = args.prefill_steps
        gu_us = 1e3 * float(np.sum(pk["prefill_gateup"])) / steps
        prefill = {
            "workload": f"prefill {T} tokens, one full-size layer (rotating over the stack)",
            "tokens_per_s": round(T * args.prefill_steps / pwall, 1),
            "ms_per_layer": round(1e3 * pwall / args.prefill_steps, 3),
            "timing": ("graph replays" if not args.eager else "eager launches")
                      + f" of {args.prefill_steps} layer calls, mean of {n_rep}",
            "ms_per_layer_traced_eager": round(1e3 * pwall_traced / args.prefill_steps, 3),
            "layer_tflops": round(layer_flops / (pwall / args.prefill_steps) / 1e12, 1),
            "kernels_avg_us": {n: round(1e3 * float(np.sum(v)) / steps, 2) for n, v in pk.items()},
            "roofline": {"bound": "mfma", "kernel": "k_prefill<routed gate/up>",
                         "achieved": round(routed_gu_flops / (gu_us * 1e-6) / 1e12, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(routed_gu_flops / (gu_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "flops_per_launch": routed_gu_flops, "avg_us": round(gu_us, 2),
                         "traffic": measured_traffic("prefill_gateup") if default_fmt else None},
        }
        log(f"prefill: {prefill['tokens_per_s']:.0f} tokens/s")

    if args.calib_copy:
        # known-size reference for the HBM byte counters: 256 MiB read + 256 MiB written
        src = torch.randn(64 << 20, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(args.cpu_tokens, args.seed, args.cpu_tokens_1t)

    line = {
        "metric": "MoE-layer tokens/s (batch-1 decode, 4k prefill) + % HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "MoE-layer tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random quantised blocks, bf16 router/shared, N(0,1) tokens)",
        "config": {"workload": "one full-size MoE layer, batch-1 decode (hidden 2048, 512 experts, "
                               f"top-10 + 1 shared, intermediate 512, {tiers_txt})"
                               ", timed as one token through 48 distinct layers per step",
                   "layers_per_step": N_LAYERS, "tokens_per_step": 1,
                   "us_per_layer": round(1e6 * wall / (N_LAYERS * args.steps), 3),
                   "gpu_event_s": round(gpu_s, 6), "graphs": not args.eager,
                   "layer_bytes": layer_bytes},
        "roofline": roofline,
        "layer_roofline": layer_roofline,
        "streaming_ceiling": ceiling,
        "verify": verify,
        "host_cold_tier": cold,
        "kernels": kernels,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
