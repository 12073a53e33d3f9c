#!/usr/bin/env python3
"""Benchmark of the 4-bit quantized decode hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  1. 4B-class speculative verify MLP block, M = 8 rows:
       rmsnorm_gateup_swiglu  X[8,2560] -> h[8,12800]   (gate+up 25600 x 2560, affine-4 g64)
       qgemv_affine4          h[8,12800] -> Y[8,2560]   (down 2560 x 12800, affine-4 g64)
  2. Q4_K MoE decode token:
       moe_expert_qgemv       x[1,2048], 128 experts, top-8, gate/up 1536 x 2048, down 2048 x 768
  3. Untied LM head with greedy verify, M = 8:
       lmhead_argmax          X[8,1024] x W[151936,1024] affine-4 g64 -> ids[8], accepted
Weights are resident in HBM; distinct copies are rotated (and the MoE router
logits change every step) so that no step is served by the 256 MB Infinity
Cache.  The same step at M = 1 gives the verify cost ratio t(M=8)/t(M=1).

Prints ONE JSON line (see the "roofline" and "cpu_baseline" objects).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for 4-bit qGEMV at M=1 and M=8; verify cost ratio"
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["bit_quantized_decode_group_amd/csrc/common.h", "bit_quantized_decode_group_amd/csrc/affine4.hip",
                  "bit_quantized_decode_group_amd/csrc/q4k.hip", "bit_quantized_decode_group_amd/csrc/abi.hip",
                  "bit_quantized_decode_group_amd/csrc/topk.hip", "bit_quantized_decode_group_amd/csrc/rht.hip",
                  "bit_quantized_decode_group_amd/csrc/mlp.hip", "bit_quantized_decode_group_amd/csrc/affine_stage.h",
                  "bit_quantized_decode_group_amd/csrc/q6k.hip", "bit_quantized_decode_group_amd/csrc/valu.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# rocprofv3 kernel-only averages of the step's kernels (written by --kernel-times from a kernel trace)
KERNEL_TIMES_FILE_REL = "profiles/kernel_times.json"
KERNEL_TIMES_FILE = os.path.join(ROOT, KERNEL_TIMES_FILE_REL)
GRAPH_STEPS = 10  # at most this many consecutive steps (rotating weights, MoE stacks, router logits) per graph
CALIB_BYTES = 384 << 20  # bytes read and written by the kernel that calibrates the HBM byte counters
# kernels launched by each entry point (once per call) with M rows (the
# bench's default tile-order layout: k_affine<M, mode, WIDE = true, TILED =
# true, top-k = false>; the MoE token is one row at every M)
def entry_kernels(M=8):
    return {
        "rmsnorm_gateup_swiglu": [f"qg::k_affine<{M}, 1, true, true, false>", "qg::k_split_reduce<1>"],
        "qgemv_affine4": [f"qg::k_affine<{M}, 0, true, true, false>", "qg::k_split_reduce<0>"],
        "moe_expert_qgemv": ["qg::k_moe_gateup", "qg::k_moe_down"],
        "lmhead_argmax": [f"qg::k_affine<{M}, 2, true, true, false>"],
        "mlp_block": [f"qg::k_mlp_block<{M}>"],
    }


ENTRY_KERNELS = entry_kernels(8)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=5, help="weight copies rotated to defeat the Infinity Cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-m1", action="store_true", help="skip the M=1 step (verify ratio)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration context timings")
    ap.add_argument("--submission", choices=["graph", "eager"], default="graph",
                    help="timed steps replayed from a HIP graph of GRAPH_STEPS captured steps (default), or "
                         "launched eagerly from Python")
    ap.add_argument("--mlp", choices=["persistent", "separate"], default="separate",
                    help="MLP block as one persistent launch (mlp_block_affine4_tiled; tile-order layout only) or "
                         "as the two entry points rmsnorm_gateup_swiglu + qgemv_affine4")
    ap.add_argument("--layout", choices=["tiled", "canonical"], default="tiled",
                    help="storage of the affine-4 weights: tile order (packed once at set-up from the canonical "
                         "arrays; same bytes, reordered) or the canonical [N][K/8] layout")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="short run for a rocprofv3 --pmc pass: a copy of CALIB_BYTES (counter calibration), "
                         "then --steps M=8 steps, then six streaming reads of 88 MiB; prints one JSON line")
    ap.add_argument("--pmc-m", type=int, choices=[1, 8], default=8,
                    help="with --pmc-pass: the rows of the steps run (8 or 1); with --traffic: the table filled")
    ap.add_argument("--kernel-times", metavar="STATS_CSV",
                    help="turn a rocprofv3 --kernel-trace --stats kernel_stats.csv of a bench run into "
                         "profiles/kernel_times.json (no GPU needed)")
    ap.add_argument("--compare-valu", metavar="NxK",
                    help="only time the affine-4 projection W[N,K] with the products on the matrix cores and on "
                         "the vector ALU (M = 1 and 8), print one JSON line; for a rocprofv3 run of that pair")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of a FETCH_SIZE and a WRITE_SIZE --pmc pass into "
                         "profiles/traffic.json (no GPU needed)")
    return ap.parse_args()


def traffic_from_counters(fetch_csv, write_csv, M=8):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel, each
    scaled by the factor that makes the calibration copy read and write
    CALIB_BYTES, summed over the kernels of each entry point.  M = 8 fills
    "kernels", M = 1 (a pass of M = 1 steps only) "kernels_m1"; an existing
    file of the same kernel sources keeps the other table."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    key = "kernels" if M == 8 else f"kernels_m{M}"
    out = {"source_hash": kernel_source_hash(), "calib_bytes": CALIB_BYTES}
    if os.path.exists(TRAFFIC_FILE):
        try:
            old = json.load(open(TRAFFIC_FILE))
            if old.get("source_hash") == out["source_hash"]:
                out.update({k: v for k, v in old.items() if k.startswith("kernels") or k.endswith("_factor")})
        except (OSError, ValueError):
            pass
    out[key] = {}
    avgs = {}
    for which, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals = per_kernel(path, counter)
        copies = [v * 1024 for n, l in vals.items() if "bitwise_not" in n for v in l]
        if not copies:
            raise SystemExit(f"bench.py --traffic: no calibration copy found in {path}")
        factor = CALIB_BYTES / float(np.mean(copies))
        out[f"{which}_factor" + ("" if M == 8 else f"_m{M}")] = round(factor, 4)
        avgs[which] = {n: float(np.mean(l)) * 1024 * factor for n, l in vals.items()}
    for entry, kernels in entry_kernels(M).items():
        ent = {"kernels": {}}
        total = 0.0
        for pat in kernels:
            names_ = [n for n in avgs["fetch"] if pat in n]
            if not names_:
                continue
            n = names_[0]
            f, w = avgs["fetch"].get(n, 0.0), avgs["write"].get(n, 0.0)
            ent["kernels"][n] = {"fetch_bytes": round(f), "write_bytes": round(w)}
            total += f + w
        if not ent["kernels"]:
            continue  # entry point not in this run (e.g. the persistent MLP block when --mlp separate)
        ent["bytes_per_launch"] = round(total)
        out[key][entry] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def kernel_times_from_stats(stats_csv):
    """Average kernel-only duration (rocprofv3 kernel_stats.csv, AverageNs) of the
    kernels of each entry point at M = 8, summed per entry point."""
    import csv
    avg = {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            avg[r["Name"]] = float(r["AverageNs"]) / 1e3
    out = {"source_hash": kernel_source_hash(), "stats": os.path.basename(stats_csv), "entries": {}}
    for entry, kernels in ENTRY_KERNELS.items():
        ks = {}
        for pat in kernels:
            hit = [n for n in avg if pat in n]
            if hit:
                ks[hit[0]] = round(avg[hit[0]], 3)
        if ks:
            out["entries"][entry] = {"kernels_us": ks, "kernel_us_m8": round(sum(ks.values()), 3)}
    with open(KERNEL_TIMES_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic:
        traffic_from_counters(*args.traffic, M=args.pmc_m)
        return
    if args.kernel_times:
        kernel_times_from_stats(args.kernel_times)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on exactly one GPU; --gpus N with N > 1 is not supported "
              "(the projection has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_quantized_decode_group_amd import ops, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.lib()

    def to_dev(a, kind):
        a = np.ascontiguousarray(a)
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        if kind == "u32":
            return torch.from_numpy(a.view(np.int32)).to(dev)
        if kind == "u8":
            return torch.from_numpy(a).to(dev)
        if kind == "f32":
            return torch.from_numpy(a.astype(np.float32)).to(dev)
        if kind == "i32":
            return torch.from_numpy(a.astype(np.int32)).to(dev)
        raise ValueError(kind)

    if args.compare_valu:
        N, K = (int(v) for v in args.compare_valu.lower().split("x"))
        r = compare_valu(torch, ops, synth, to_dev, dev, N, K, lambda fn, n, reps: per_call_us(torch, fn, reps))
        print(json.dumps({"products_mfma_vs_valu": {f"{N}x{K}": r}}), flush=True)
        return

    t0 = time.time()
    vb = synth.verify_block()          # M=8, D=2560, I=12800, seed 1003
    lm = synth.lm_head(M=8)            # V=151936, K=1024, seed 1005
    n_logit_sets = 64
    moe = synth.moe_token(n_logit_sets=n_logit_sets)  # E=128, D=2048, I=768, top-8, seed 1004
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    C = max(1, args.copies)
    base = {
        "codes_gu": to_dev(vb["codes_gu"], "u32"), "scales_gu": to_dev(vb["scales_gu"], "bf16"),
        "biases_gu": to_dev(vb["biases_gu"], "bf16"), "codes_d": to_dev(vb["codes_d"], "u32"),
        "scales_d": to_dev(vb["scales_d"], "bf16"), "biases_d": to_dev(vb["biases_d"], "bf16"),
        "codes_lm": to_dev(lm["codes"], "u32"), "scales_lm": to_dev(lm["scales"], "bf16"),
        "biases_lm": to_dev(lm["biases"], "bf16"),
    }
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(C - 1)]
    tiled = args.layout == "tiled"
    if tiled:
        # tile-order copies of the same weights (one pack per matrix, outside the timed region)
        for c in copies:
            for key in ("gu", "d", "lm"):
                ct, sb = ops.tile_pack(c["codes_" + key], c["scales_" + key], c["biases_" + key])
                c["t_" + key] = (ct, sb)
                del c["codes_" + key], c["scales_" + key], c["biases_" + key]
    moe_base = {"w_gu": to_dev(moe["w_gu"], "u8"), "w_down": to_dev(moe["w_down"], "u8")}
    moe_stacks = [moe_base, {k: v.clone() for k, v in moe_base.items()}]
    logits = to_dev(moe["logits"], "f32")
    x8 = to_dev(vb["x"], "bf16")
    gamma = to_dev(vb["gamma"], "bf16")
    xm = to_dev(moe["x"], "bf16")
    xl8 = to_dev(lm["x"], "bf16")
    draft = to_dev(lm["draft"], "i32")
    torch.cuda.synchronize()
    log(f"[bench] {C} weight copies + 2 MoE stacks resident in HBM")

    D, I, V, K5 = vb["D"], vb["I"], lm["V"], lm["K"]
    E, Dm, Im, top_k = moe["E"], moe["D"], moe["I"], moe["top_k"]

    def bufs(M):
        return {
            "x": x8[:M].contiguous(), "xl": xl8[:M].contiguous(),
            "h": torch.empty((M, I), dtype=torch.bfloat16, device=dev),
            "y": torch.empty((M, D), dtype=torch.bfloat16, device=dev),
            "ym": torch.empty((1, Dm), dtype=torch.bfloat16, device=dev),
            "mids": torch.empty(top_k, dtype=torch.int32, device=dev),
            "mw": torch.empty(top_k, dtype=torch.float32, device=dev),
            "ids": torch.empty(M, dtype=torch.int32, device=dev),
            "acc": torch.empty(1, dtype=torch.int32, device=dev),
            # one caller-owned workspace serves every call of the step (the calls are ordered on the stream)
            "ws": ops.workspace(max(ops.workspace_bytes("rmsnorm_gateup_swiglu_tiled", M, I, D),
                                    ops.workspace_bytes("rmsnorm_gateup_swiglu", M, I, D),
                                    ops.workspace_bytes("qgemv_affine4_tiled", M, D, I),
                                    ops.workspace_bytes("qgemv_affine4", M, D, I),
                                    ops.workspace_bytes("mlp_block_affine4_tiled", M, D, I),
                                    ops.workspace_bytes("moe_expert_qgemv", top_k, E, Dm, Im),
                                    ops.workspace_bytes("lmhead_argmax_tiled", M, V, K5),
                                    ops.workspace_bytes("lmhead_argmax", M, V, K5), 256), dev),
        }

    # Algorithmic bytes per step: every weight byte once (0.5625 B/weight), the
    # activations read, the outputs written, and the two intermediates (h of
    # the MLP block, the MoE expert activations) written once and read once.
    persistent = tiled and args.mlp == "persistent"

    def step_bytes(M):
        w = {
            "rmsnorm_gateup_swiglu": 2 * I * D // 2 + 2 * (2 * I * D // 64) * 2,
            "qgemv_affine4": D * I // 2 + 2 * (D * I // 64) * 2,
            "moe_expert_qgemv": top_k * (2 * Im * Dm // 256 * 144 + Dm * Im // 256 * 144),
            "lmhead_argmax": V * K5 // 2 + 2 * (V * K5 // 64) * 2,
        }
        a = {
            "rmsnorm_gateup_swiglu": M * D * 2 + D * 2 + M * I * 2,
            "qgemv_affine4": M * I * 2 + M * D * 2,
            "moe_expert_qgemv": Dm * 2 + E * 4 + 2 * top_k * Im * 2 + Dm * 2 + top_k * 8,
            "lmhead_argmax": M * K5 * 2 + M * 4 * 2 + 4,
        }
        tot = {k: w[k] + a[k] for k in w}
        if persistent:  # the block is one launch: its bytes are those of its two projections
            for dct in (tot, w):
                dct["mlp_block"] = dct.pop("rmsnorm_gateup_swiglu") + dct.pop("qgemv_affine4")
        return tot, w

    names = (["mlp_block"] if persistent else ["rmsnorm_gateup_swiglu", "qgemv_affine4"]) + \
        ["moe_expert_qgemv", "lmhead_argmax"]

    def run_step(i, M, b):
        c = copies[i % C]
        ms = moe_stacks[i % 2]
        lg = logits[i % n_logit_sets]
        dr = draft[:M]
        for name in names:
            entry_call(name, c, ms, lg, dr, b)

    def entry_call(name, c, ms, lg, dr, b):
        if name == "mlp_block":
            ops.mlp_block_affine4_tiled(b["x"], gamma, vb["eps"], c["t_gu"], c["t_d"], D, I, h=b["h"], y=b["y"],
                                        ws=b["ws"])
        elif name == "rmsnorm_gateup_swiglu":
            if tiled:
                ops.rmsnorm_gateup_swiglu_tiled(b["x"], gamma, vb["eps"], *c["t_gu"], I, h=b["h"], ws=b["ws"])
            else:
                ops.rmsnorm_gateup_swiglu(b["x"], gamma, vb["eps"], c["codes_gu"], c["scales_gu"], c["biases_gu"],
                                          h=b["h"], ws=b["ws"])
        elif name == "qgemv_affine4":
            if tiled:
                ops.qgemv_affine4_tiled(b["h"], *c["t_d"], D, y=b["y"], ws=b["ws"])
            else:
                ops.qgemv_affine4(b["h"], c["codes_d"], c["scales_d"], c["biases_d"], y=b["y"], ws=b["ws"])
        elif name == "moe_expert_qgemv":
            ops.moe_expert_qgemv(xm, lg, top_k, ms["w_gu"], ms["w_down"], y=b["ym"], out_ids=b["mids"],
                                 out_w=b["mw"], ws=b["ws"])
        elif name == "lmhead_argmax":
            if tiled:
                ops.lmhead_argmax_tiled(b["xl"], *c["t_lm"], V, draft=dr, ids=b["ids"], accepted=b["acc"],
                                        ws=b["ws"])
            else:
                ops.lmhead_argmax(b["xl"], c["codes_lm"], c["scales_lm"], c["biases_lm"], draft=dr, ids=b["ids"],
                                  accepted=b["acc"], ws=b["ws"])

    graph_checks = {}
    spread = {}
    use_graph = args.submission == "graph"

    def timed_steps(M, steps, warmup):
        """K whole steps: HIP-graph replays of GRAPH_STEPS captured consecutive steps (or eager
        launches); events on the launch stream around all of them, and at five sub-batch
        boundaries for the spread."""
        b = bufs(M)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for i in range(warmup):
                run_step(i, M, b)
        torch.cuda.synchronize()
        glen = max(d for d in range(1, GRAPH_STEPS + 1) if steps % d == 0) if use_graph else 1
        g = None
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(glen):
                    run_step(i, M, b)
            torch.cuda.synchronize()
        units = steps // glen
        nsub = 5 if units >= 5 else 1
        cut = [round(units * j / nsub) for j in range(nsub + 1)]
        evb = [torch.cuda.Event(enable_timing=True) for _ in range(nsub + 1)]
        w0 = time.perf_counter()
        with torch.cuda.stream(s):
            evb[0].record()
            for j in range(nsub):
                for i in range(cut[j], cut[j + 1]):
                    if use_graph:
                        g.replay()
                    else:
                        run_step(warmup + i, M, b)
                evb[j + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_step = evb[0].elapsed_time(evb[nsub]) / steps
        if use_graph:
            # the replayed outputs (those of captured step glen - 1) against the same step run eagerly
            b2 = bufs(M)
            with torch.cuda.stream(s):
                run_step(glen - 1, M, b2)
            torch.cuda.synchronize()
            same = all(torch.equal(b[k], b2[k]) for k in ("h", "y", "ym", "mids", "mw", "ids", "acc"))
            if not same:
                raise SystemExit(f"bench.py: graph replay at M={M} differs from the eager step")
            graph_checks[f"M{M}"] = f"{glen}-step graph: replay == eager (bit-identical)"
            del g
        sub = [evb[j].elapsed_time(evb[j + 1]) / ((cut[j + 1] - cut[j]) * glen) for j in range(nsub)]
        spread[M] = {"median_ms": round(float(np.median(sub)), 5), "p10_ms": round(float(np.percentile(sub, 10)), 5),
                     "p90_ms": round(float(np.percentile(sub, 90)), 5), "sub_batches": nsub}
        return ms_step, wall, b

    def entry_times(M):
        """Per-call time of each entry point of the step: a HIP graph of 2*C back-to-back calls
        (rotating weight copies, MoE stacks and router logits) replayed, events on its stream."""
        b = bufs(M)
        per = {}
        for name in names:
            fn = lambda i, nm=name: entry_call(nm, copies[i % C], moe_stacks[i % 2], logits[i % n_logit_sets],
                                               draft[:M], b)
            per[name] = graph_us(torch, fn, 2 * C)
        return per

    if args.pmc_pass:
        # an elementwise kernel that reads and writes CALIB_BYTES (a plain
        # device copy may go to the DMA engine and never show up as a kernel)
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        for M in (args.pmc_m,):
            b = bufs(M)
            for i in range(args.warmup + args.steps):
                run_step(i, M, b)
        # the library's plain streaming read of 88 MiB (about the LM head's
        # bytes), six buffers in turn (more than the on-package cache holds),
        # so that the read ceiling's counters sit beside the kernels'
        reads = [torch.empty(88 << 20, dtype=torch.uint8, device=dev).fill_(3) for _ in range(6)]
        for r in reads:
            ops.stream_read(r)
        torch.cuda.synchronize()
        del reads
        print(json.dumps({"pmc_pass": True, "calib_bytes": CALIB_BYTES, "steps": args.warmup + args.steps}), flush=True)
        return

    log(f"[bench] timing M=8: warmup {args.warmup}, steps {args.steps}, "
        + ("graph replays" if use_graph else "eager launches"))
    ms8, wall8, b8 = timed_steps(8, args.steps, args.warmup)
    bytes8, wbytes = step_bytes(8)
    total8 = sum(bytes8.values())
    value = total8 / (ms8 * 1e-3) / 1e9
    accepted = int(b8["acc"].cpu()[0])
    per8 = entry_times(8)
    log(f"[bench] M=8: {ms8 * 1e3:.1f} us/step -> {value:.0f} GB/s; per call (us): "
        + ", ".join(f"{n}={per8[n]:.1f}" for n in names))

    ms1 = per1 = None
    if not args.no_m1:
        s1 = max(20, args.steps // 2)
        log(f"[bench] timing M=1: steps {s1}")
        ms1, _, _ = timed_steps(1, s1, max(5, args.warmup // 2))
        per1 = entry_times(1)
        log(f"[bench] M=1: {ms1 * 1e3:.1f} us/step; ratio {ms8 / ms1:.3f}; per call (us): "
            + ", ".join(f"{n}={per1[n]:.1f}" for n in names))

    # context: the runtime's device-to-device copy of 1 GiB (bytes read + written)
    src = torch.empty(2 ** 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    # context: a plain streaming read of 1 GiB with the library's read kernel
    # (the practical HBM read ceiling a weight stream can reach on this device)
    for _ in range(2):
        ops.stream_read(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        ops.stream_read(src)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 5 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src

    cfg = None if args.no_configs else config_timings(torch, ops, synth, to_dev, dev)
    if cfg is not None:
        cfg["mlp_stack_28x1024x3072"] = stack_timings(torch, ops, synth, to_dev, dev)

    tf_tab = {}  # counted HBM bytes per call (profiles/traffic.json, when it matches these kernel sources)
    if os.path.exists(TRAFFIC_FILE):
        try:
            tf_all = json.load(open(TRAFFIC_FILE))
            if tf_all.get("source_hash") == kernel_source_hash():
                tf_tab = {"m8": tf_all.get("kernels", {}), "m1": tf_all.get("kernels_m1", {})}
        except (OSError, ValueError):
            tf_tab = {}
    kernels = {}
    for n in names:
        k = {"us_m8": round(per8[n], 2), "bytes_m8": bytes8[n], "gb_s_m8": round(bytes8[n] / (per8[n] * 1e-6) / 1e9, 1),
             "frac_m8": round(bytes8[n] / (per8[n] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        for tag in ("m8", "m1"):
            t = tf_tab.get(tag, {}).get(n)
            if t:
                k[f"traffic_{tag}"] = t["bytes_per_launch"]
        if per1 is not None:
            b1 = step_bytes(1)[0][n]
            k.update({"us_m1": round(per1[n], 2), "gb_s_m1": round(b1 / (per1[n] * 1e-6) / 1e9, 1),
                      "frac_m1": round(b1 / (per1[n] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                      "verify_ratio": round(per8[n] / per1[n], 3)})
        kernels[n] = k

    # dominant kernel = the entry point with the largest share of the step's time
    dom = max(names, key=lambda n: per8[n])
    dom_gbs = bytes8[dom] / (per8[dom] * 1e-6) / 1e9
    traffic = None
    prof = {}
    if os.path.exists(TRAFFIC_FILE):
        try:
            tf = json.load(open(TRAFFIC_FILE))
            ent = tf.get("kernels", {}).get(dom)
            if ent and tf.get("source_hash") == kernel_source_hash():
                traffic = ent.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    if os.path.exists(KERNEL_TIMES_FILE):
        try:
            kt = json.load(open(KERNEL_TIMES_FILE))
            if kt.get("source_hash") == kernel_source_hash():
                prof = kt.get("entries", {}).get(dom, {})
        except (OSError, ValueError):
            prof = {}
    entry = {"mlp_block": "mlp_block_affine4_tiled", "moe_expert_qgemv": "moe_expert_qgemv"}.get(
        dom, dom + ("_tiled" if tiled else ""))
    roofline = {"kernel": entry, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": bytes8[dom], "avg_launch_us": round(per8[dom], 2),
                "timing": "HIP events around a graph of back-to-back calls on its stream, per call"}
    if prof.get("kernel_us_m8"):
        ku = prof["kernel_us_m8"]
        roofline.update({"kernel_only_us": ku, "frac_kernel_only": round(bytes8[dom] / (ku * 1e-6) / 1e9 /
                                                                         PEAK_HBM_GBS, 4),
                         "kernel_only_source": "rocprofv3 --kernel-trace average, " + KERNEL_TIMES_FILE_REL})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(vb, lm, moe, total8)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms8, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode verify step (M=8): 4B-class MLP block X[8,2560] RMSNorm->gate+up "
                               "2560->2x12800->SwiGLU->down 12800->2560 (affine-4 g64) + Q4_K MoE token "
                               "(128 experts, top-8, 2048<->768) + untied LM head X[8,1024] x W[151936,1024] "
                               "(affine-4 g64) greedy verify",
                   "M": 8, "weight_copies": C,
                   "mlp": ("one persistent launch (mlp_block_affine4_tiled)" if persistent
                           else "rmsnorm_gateup_swiglu + qgemv_affine4"),
                   "submission": ("HIP graph replays of captured steps" if use_graph else "eager launches"),
                   "layout": "tile-order (same bytes as canonical, packed at set-up)" if tiled else "canonical",
                   "algorithmic_bytes_per_step": total8,
                   "weight_bytes_per_step": sum(wbytes.values()), "accum": "fp32", "weights": "4-bit"},
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "ms_per_step_m1": round(ms1, 5) if ms1 else None,
        "verify_ratio": round(ms8 / ms1, 4) if ms1 else None,
        "tokens_per_s_m8": round(8 / (ms8 * 1e-3), 1),
        "tokens_per_s_m1": round(1 / (ms1 * 1e-3), 1) if ms1 else None,
        "accepted_prefix": accepted,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "d2d_copy_gb_s": round(copy_gbs, 1),
        "stream_read_gb_s": round(read_gbs, 1),
        "roofline_frac_of_stream_read": round(dom_gbs / read_gbs, 4),
        "step_spread": {f"M{m}": v for m, v in spread.items()},
        "configs_context": cfg,
        "graph_check": graph_checks or None,
        "wall_s_timed": round(wall8, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


def graph_us(torch, fn, ncalls, reps=10):
    """Microseconds per call of fn(i): ncalls back-to-back calls (i = 0..ncalls-1) captured in a
    HIP graph on a side stream, replayed reps times after a warm-up, HIP events on that stream.
    The host's launch cost is out of the timed region, as it is for a caller that replays graphs."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in range(ncalls):
            fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(ncalls):
            fn(i)
    with torch.cuda.stream(s):
        for _ in range(2):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * ncalls)
    del g
    return us


def per_call_us(torch, fn, reps):
    """Microseconds per call of fn(i), graph-replayed (see graph_us)."""
    return graph_us(torch, fn, reps)


def compare_valu(torch, ops, synth, to_dev, dev, N, K, per_call):
    """Per-call times of the affine-4 projection X[M,K] x W[N,K] at M = 1 and 8 with the
    M-row products on the matrix cores (qgemv_affine4) and on the vector ALU
    (qg_affine4_valu: same plan, staging and reduce), on identical weights rotated
    over >= 512 MB of copies."""
    dv = synth.single_projection(M=8, N=N, K=K, seed=1008 + K)
    w = {k: to_dev(dv[k], "u32" if k == "codes" else "bf16") for k in ("codes", "scales", "biases")}
    nb = int(dv["codes"].nbytes + dv["scales"].nbytes + dv["biases"].nbytes)
    n = max(2, (512 << 20) // nb + 1)
    cps = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(n - 1)]
    x8 = to_dev(dv["x"], "bf16")
    r = {}
    for M in (1, 8):
        xm = x8[:M].contiguous()
        ym = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        b = nb + M * K * 2 + M * N * 2
        for name, fn in (("mfma", ops.qgemv_affine4), ("valu", ops.affine4_valu)):
            us = per_call(lambda i: fn(xm, cps[i % n]["codes"], cps[i % n]["scales"], cps[i % n]["biases"], y=ym),
                          n, max(3 * n, 30))
            r[f"M{M}_{name}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
        r[f"M{M}_valu_over_mfma"] = round(r[f"M{M}_valu"]["us"] / r[f"M{M}_mfma"]["us"], 3)
    return r


def stack_timings(torch, ops, synth, to_dev, dev, L=28, D=1024, I=3072):
    """Context: a stack of L distinct 0.6B-shaped MLP blocks (the 28 MLPs of a
    decode step), block l + 1 taking block l's output, timed per pass at M = 1
    and 8 in five ways: the separate entry points launched from the host one by
    one (eager) and captured in one graph; one persistent launch per block,
    eager and in one graph; and one persistent launch for the whole stack.
    Enough stack copies rotate (>= 512 MB) that no pass finds its weights in
    the Infinity Cache."""
    gus, dns, gams = [], [], []
    for l in range(L):
        d = synth.mlp_block(M=8, D=D, I=I, seed=21000 + l)
        if l == 0:
            x8 = to_dev(d["x"], "bf16")
        gus.append(ops.tile_pack(to_dev(d["codes_gu"], "u32"), to_dev(d["scales_gu"], "bf16"),
                                 to_dev(d["biases_gu"], "bf16")))
        dns.append(ops.tile_pack(to_dev(d["codes_d"], "u32"), to_dev(d["scales_d"], "bf16"),
                                 to_dev(d["biases_d"], "bf16")))
        gams.append(to_dev(d["gamma"], "bf16"))
    nb_layer = 2 * I * D // 2 + 2 * I * (D // 64) * 4 + D * I // 2 + D * (I // 64) * 4
    one = {"gamma": torch.stack(gams).contiguous(), "gu_c": torch.cat([g[0] for g in gus]),
           "gu_s": torch.cat([g[1] for g in gus]), "dn_c": torch.cat([g[0] for g in dns]),
           "dn_s": torch.cat([g[1] for g in dns])}
    del gus, dns
    n = max(2, (512 << 20) // (L * nb_layer) + 1)
    stacks = [one] + [{k: v.clone() for k, v in one.items()} for _ in range(n - 1)]
    gcb, gsb = ops.tiled_bytes(2 * I, D)
    dcb, dsb = ops.tiled_bytes(D, I)

    def layer(c, l):  # views of layer l of stack c
        return ((c["gu_c"][l * gcb // 4:(l + 1) * gcb // 4], c["gu_s"][l * gsb // 2:(l + 1) * gsb // 2]),
                (c["dn_c"][l * dcb // 4:(l + 1) * dcb // 4], c["dn_s"][l * dsb // 2:(l + 1) * dsb // 2]),
                c["gamma"][l])
    views = [[layer(c, l) for l in range(L)] for c in stacks]
    out = {"layers": L, "D": D, "I": I, "stack_copies": n, "weight_bytes_per_pass": L * nb_layer}
    for M in (1, 8):
        xm = x8[:M].contiguous()
        h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
        ys = torch.empty((L, M, D), dtype=torch.bfloat16, device=dev)
        ws = ops.workspace(max(ops.workspace_bytes("mlp_stack_affine4_tiled", M, D, I),
                               ops.workspace_bytes("rmsnorm_gateup_swiglu_tiled", M, I, D),
                               ops.workspace_bytes("qgemv_affine4_tiled", M, D, I)), dev)
        b = L * (nb_layer + M * D * 2 * 2 + 2 * M * I * 2 + D * 2)

        def separate(i):
            v = views[i % n]
            xin = xm
            for l in range(L):
                gu, dn, gam = v[l]
                ops.rmsnorm_gateup_swiglu_tiled(xin, gam, 1e-6, *gu, I, h=h, ws=ws)
                ops.qgemv_affine4_tiled(h, *dn, D, y=ys[l], ws=ws)
                xin = ys[l]

        def blocks(i):
            v = views[i % n]
            xin = xm
            for l in range(L):
                gu, dn, gam = v[l]
                ops.mlp_block_affine4_tiled(xin, gam, 1e-6, gu, dn, D, I, h=h, y=ys[l], ws=ws)
                xin = ys[l]

        def stack(i):
            c = stacks[i % n]
            ops.mlp_stack_affine4_tiled(xm, c["gamma"], 1e-6, c["gu_c"], c["gu_s"], c["dn_c"], c["dn_s"], L, D, I,
                                        h=h, ys=ys, ws=ws)

        def eager_us(fn, reps):
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        res = {}
        for name, fn, graphed in (("separate_eager", separate, False), ("separate_graph", separate, True),
                                  ("block_per_layer_eager", blocks, False), ("block_per_layer_graph", blocks, True),
                                  ("stack_one_launch", stack, False), ("stack_one_launch_graph", stack, True)):
            try:
                us = graph_us(torch, fn, 2 * n, reps=5) if graphed else eager_us(fn, 4 * n)
            except Exception as e:  # a launch kind the graph capture refuses is reported, not fatal
                res[name] = {"error": str(e)[:160]}
                torch.cuda.synchronize()
                continue
            res[name] = {"us": round(us, 1), "us_per_layer": round(us / L, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
        assert ops.mlp_failures(ws) == 0, "a grid barrier wait gave up during the stack timings"
        out[f"M{M}"] = res
    del stacks, views
    log("[bench] stack: " + json.dumps(out))
    return out


def config_timings(torch, ops, synth, to_dev, dev):
    """Context (not the bench value): per-call times of the smaller workloads
    and variants, each rotating enough weight copies (>= 512 MB) that the
    Infinity Cache cannot serve a call; HIP events around R back-to-back calls."""
    def per_call(fn, n_copies, reps):
        return per_call_us(torch, fn, reps)

    out = {}
    # single projection X[M,1024] x W[3072,1024] affine-4 (M = 1 and 8)
    sp = synth.single_projection(M=8)
    w = {k: to_dev(sp[k], "u32" if k == "codes" else "bf16") for k in ("codes", "scales", "biases")}
    nb = int(sp["codes"].nbytes + sp["scales"].nbytes + sp["biases"].nbytes)
    n = max(2, (512 << 20) // nb + 1)
    cps = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(n - 1)]
    x8 = to_dev(sp["x"], "bf16")
    res = {}
    for M in (1, 8):
        xm = x8[:M].contiguous()
        ym = torch.empty((M, sp["N"]), dtype=torch.bfloat16, device=dev)
        us = per_call(lambda i: ops.qgemv_affine4(xm, cps[i % n]["codes"], cps[i % n]["scales"], cps[i % n]["biases"],
                                                  y=ym), n, 3 * n)
        b = nb + M * sp["K"] * 2 + M * sp["N"] * 2
        res[f"M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    res["ratio_m8_m1"] = round(res["M8"]["us"] / res["M1"]["us"], 3)
    out["projection_3072x1024"] = res
    # the same projection behind an input randomised Hadamard transform (blocks of 1024)
    signs = torch.from_numpy(np.random.default_rng(1006).choice(np.array([-1, 1], np.int8), size=sp["K"])).to(dev)
    res = {}
    for M in (1, 8):
        xm = x8[:M].contiguous()
        ym = torch.empty((M, sp["N"]), dtype=torch.bfloat16, device=dev)
        us = per_call(lambda i: ops.qgemv_affine4_rht(xm, signs, 1024, cps[i % n]["codes"], cps[i % n]["scales"],
                                                      cps[i % n]["biases"], y=ym), n, 3 * n)
        b = nb + M * sp["K"] * 2 + sp["K"] + M * sp["N"] * 2
        res[f"M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    out["projection_rht_3072x1024"] = res
    # the same projection on tile-order weights (one contiguous KiB per wave load)
    tcs = [ops.tile_pack(c["codes"], c["scales"], c["biases"]) for c in cps]
    del cps
    res = {}
    for M in (1, 8):
        xm = x8[:M].contiguous()
        ym = torch.empty((M, sp["N"]), dtype=torch.bfloat16, device=dev)
        us = per_call(lambda i: ops.qgemv_affine4_tiled(xm, tcs[i % n][0], tcs[i % n][1], sp["N"], y=ym), n, 3 * n)
        b = nb + M * sp["K"] * 2 + M * sp["N"] * 2
        res[f"M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    out["projection_tiled_3072x1024"] = res
    del tcs
    # 8-bit affine projections: X[M,1024] x W[3072,1024] and the 4B-class down shape W[2560,12800]
    res = {}
    for (N8, K8) in ((3072, 1024), (2560, 12800)):
        d8 = synth.single_projection8(M=8, N=N8, K=K8, seed=1006 + K8)
        w = {k: to_dev(d8[k], "u32" if k == "codes" else "bf16") for k in ("codes", "scales", "biases")}
        nb = int(d8["codes"].nbytes + d8["scales"].nbytes + d8["biases"].nbytes)
        n = max(2, (512 << 20) // nb + 1)
        cps = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(n - 1)]
        x8a = to_dev(d8["x"], "bf16")
        for M in (1, 8):
            xm = x8a[:M].contiguous()
            ym = torch.empty((M, N8), dtype=torch.bfloat16, device=dev)
            us = per_call(lambda i: ops.qgemv_affine8(xm, cps[i % n]["codes"], cps[i % n]["scales"],
                                                      cps[i % n]["biases"], y=ym), n, 3 * n)
            b = nb + M * K8 * 2 + M * N8 * 2
            res[f"{N8}x{K8}_M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
        del cps
    out["projection_affine8"] = res
    # GGUF Q6_K projections, the same two shapes (210-byte superblocks as stored)
    res = {}
    for (N6, K6) in ((3072, 1024), (2560, 12800)):
        d6 = synth.single_projection_q6k(M=8, N=N6, K=K6, seed=1007 + K6)
        wb = to_dev(d6["blocks"], "u8")
        nb = int(d6["blocks"].nbytes)
        n = max(2, (512 << 20) // nb + 1)
        cps = [wb] + [wb.clone() for _ in range(n - 1)]
        x6 = to_dev(d6["x"], "bf16")
        for M in (1, 8):
            xm = x6[:M].contiguous()
            ym = torch.empty((M, N6), dtype=torch.bfloat16, device=dev)
            us = per_call(lambda i: ops.qgemv_q6k(xm, cps[i % n], y=ym), n, 3 * n)
            b = nb + M * K6 * 2 + M * N6 * 2
            res[f"{N6}x{K6}_M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
        del cps
    out["projection_q6k"] = res
    # GGUF Q4_K projections, the same two shapes (144-byte superblocks as stored)
    res = {}
    for (N4, K4) in ((3072, 1024), (2560, 12800)):
        g4 = synth.rng(1008 + K4)
        x4 = to_dev(synth.normal_bf16(g4, (8, K4)), "bf16")
        blocks4 = synth.q4k_matrix(g4, N4, K4)
        wb = to_dev(blocks4, "u8")
        nb = int(blocks4.nbytes)
        n = max(2, (512 << 20) // nb + 1)
        cps = [wb] + [wb.clone() for _ in range(n - 1)]
        for M in (1, 8):
            xm = x4[:M].contiguous()
            ym = torch.empty((M, N4), dtype=torch.bfloat16, device=dev)
            us = per_call(lambda i: ops.qgemv_q4k(xm, cps[i % n], y=ym), n, 3 * n)
            b = nb + M * K4 * 2 + M * N4 * 2
            res[f"{N4}x{K4}_M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
        del cps
    out["projection_q4k"] = res
    # the M-row products on the matrix cores or on the vector ALU, same work
    out["products_mfma_vs_valu"] = {f"{N}x{K}": compare_valu(torch, ops, synth, to_dev, dev, N, K, per_call)
                                    for (N, K) in ((3072, 1024), (2560, 12800), (151936, 1024))}
    # MLP block D=1024, I=3072 (RMSNorm -> gate/up -> SwiGLU -> down), M = 1 and 8
    mb = synth.mlp_block(M=8)
    keys = {"codes_gu": "u32", "scales_gu": "bf16", "biases_gu": "bf16", "codes_d": "u32", "scales_d": "bf16",
            "biases_d": "bf16"}
    w = {k: to_dev(mb[k], t) for k, t in keys.items()}
    nb = int(sum(mb[k].nbytes for k in keys))
    n = max(2, (512 << 20) // nb + 1)
    cps = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(n - 1)]
    x8, gam = to_dev(mb["x"], "bf16"), to_dev(mb["gamma"], "bf16")
    res = {}
    for M in (1, 8):
        xm = x8[:M].contiguous()
        hm = torch.empty((M, mb["I"]), dtype=torch.bfloat16, device=dev)
        ym = torch.empty((M, mb["D"]), dtype=torch.bfloat16, device=dev)

        def blk(i):
            c = cps[i % n]
            ops.rmsnorm_gateup_swiglu(xm, gam, mb["eps"], c["codes_gu"], c["scales_gu"], c["biases_gu"], h=hm)
            ops.qgemv_affine4(hm, c["codes_d"], c["scales_d"], c["biases_d"], y=ym)
        us = per_call(blk, n, 3 * n)
        b = nb + M * mb["D"] * 2 * 2 + 2 * M * mb["I"] * 2 + mb["D"] * 2
        res[f"M{M}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    res["ratio_m8_m1"] = round(res["M8"]["us"] / res["M1"]["us"], 3)
    out["mlp_block_1024x3072"] = res
    del cps
    # LM head variants: M = 4, and M = 8 with the fp32 logits stored
    lm = synth.lm_head(M=8)
    w = {k: to_dev(lm[k], "u32" if k == "codes" else "bf16") for k in ("codes", "scales", "biases")}
    nb = int(lm["codes"].nbytes + lm["scales"].nbytes + lm["biases"].nbytes)
    n = max(2, (512 << 20) // nb + 1)
    cps = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(n - 1)]
    x8, draft = to_dev(lm["x"], "bf16"), to_dev(lm["draft"], "i32")
    ids = torch.empty(8, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    logits = torch.empty((8, lm["V"]), dtype=torch.float32, device=dev)
    res = {}
    for M, keep in ((4, False), (8, True)):
        xm = x8[:M].contiguous()
        us = per_call(lambda i: ops.lmhead_argmax(xm, cps[i % n]["codes"], cps[i % n]["scales"], cps[i % n]["biases"],
                                                  draft=draft[:M].contiguous(), ids=ids[:M], accepted=acc,
                                                  logits=logits[:M] if keep else None), n, 6 * n)
        b = nb + M * lm["K"] * 2 + M * 8 + (M * lm["V"] * 4 if keep else 0)
        res[f"M{M}" + ("_with_logits" if keep else "")] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    # top-k readout (candidate pools), M = 8: projection + logits + selection
    tids = torch.empty((8, 64), dtype=torch.int32, device=dev)
    tvals = torch.empty((8, 64), dtype=torch.float32, device=dev)
    for k in (8, 64):
        us = per_call(lambda i: ops.lmhead_topk(x8, cps[i % n]["codes"], cps[i % n]["scales"], cps[i % n]["biases"], k,
                                                ids=tids[:, :k].contiguous() if k < 64 else tids,
                                                vals=tvals[:, :k].contiguous() if k < 64 else tvals), n, 6 * n)
        b = nb + 8 * lm["K"] * 2 + 8 * k * 8
        res[f"M8_top{k}"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    # greedy readout on tile-order weights, M = 1 and 8
    tcs = [ops.tile_pack(c["codes"], c["scales"], c["biases"]) for c in cps]
    del cps
    for M in (1, 8):
        xm = x8[:M].contiguous()
        us = per_call(lambda i: ops.lmhead_argmax_tiled(xm, tcs[i % n][0], tcs[i % n][1], lm["V"],
                                                        draft=draft[:M].contiguous(), ids=ids[:M], accepted=acc),
                      n, 6 * n)
        b = nb + M * lm["K"] * 2 + M * 8
        res[f"M{M}_tiled"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1)}
    # top-k readout on tile-order weights (selection fused into the projection)
    for M, k in ((1, 8), (8, 8), (8, 64)):
        xm = x8[:M].contiguous()
        ti, tv = tids[:M, :k].contiguous(), tvals[:M, :k].contiguous()
        us = per_call(lambda i: ops.lmhead_topk_tiled(xm, tcs[i % n][0], tcs[i % n][1], lm["V"], k, ids=ti, vals=tv),
                      n, 6 * n)
        b = nb + M * lm["K"] * 2 + M * k * 8
        res[f"M{M}_top{k}_tiled"] = {"us": round(us, 2), "gb_s": round(b / (us * 1e-6) / 1e9, 1),
                                     "over_argmax_tiled": round(us / res[f"M{M}_tiled"]["us"], 3)}
    out["lm_head_151936x1024"] = res
    del tcs
    log("[bench] context: " + json.dumps(out))
    return out


def _host_threads():
    """Threads the oracle may use on this host: the process's affinity set, capped by
    OMP_NUM_THREADS when that is set (a host may grant a GPU's process fewer CPUs than it has)."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    n = min(aff, int(env)) if env and env.isdigit() and int(env) > 0 else aff
    return max(1, n), aff


def cpu_baseline(vb, lm, moe, step_bytes, min_seconds=10.0, max_steps=64):
    """The CPU oracle (plain C, fp64) on the same step: the full MLP block at M=8,
    the MoE token, and the LM head at M=8 with its draft ids.  Whole steps are
    repeated (the MoE router logits rotating as in the GPU run) until about
    min_seconds of work have been timed.  Run twice: on all the host threads
    the process may use (the OpenMP build: output rows split over threads, the
    same bits) -- the reported value -- and on one thread.  Same unit as the GPU
    value."""
    import oracle

    def run(threads, seconds):
        used = oracle.use_threads(threads)
        n, t = 0, time.perf_counter()
        while True:
            oracle.mlp_block(vb["x"], vb["gamma"], vb["eps"], vb["codes_gu"], vb["scales_gu"], vb["biases_gu"],
                             vb["codes_d"], vb["scales_d"], vb["biases_d"])
            oracle.moe(moe["x"], moe["logits"][n % len(moe["logits"])], moe["top_k"], moe["w_gu"], moe["w_down"],
                       moe["E"], moe["D"], moe["I"])
            oracle.lmhead(lm["x"], lm["codes"], lm["scales"], lm["biases"], draft=lm["draft"], want_logits=False)
            n += 1
            dt = time.perf_counter() - t
            if dt >= seconds or n >= max_steps:
                break
        return n, dt, used

    threads, aff = _host_threads()
    n, dt, used = run(threads, min_seconds)
    n1, dt1, _ = run(1, min_seconds)
    oracle.use_threads(1)
    log(f"[bench] cpu oracle: {n} full steps in {dt:.1f}s on {used} threads; {n1} in {dt1:.1f}s on 1 thread")
    return {"value": round(n * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{n} full steps (MLP block M=8, MoE token with rotating router logits, LM head M=8), "
                      "same seeded inputs as the GPU run; output rows split over the threads (OpenMP build of "
                      "the same C, same bits)",
            "steps": n, "seconds": round(dt, 2), "cpu_count": os.cpu_count(), "affinity_cpus": aff,
            "single_thread": {"value": round(n1 * step_bytes / dt1 / 1e9, 4), "cores": 1, "steps": n1,
                              "seconds": round(dt1, 2)}}


if __name__ == "__main__":
    main()
