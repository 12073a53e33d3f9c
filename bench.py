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
GRAPH_STEPS = 10  # at most this many consecutive steps (rotating weights, MoE stacks, router logits) per graph
CALIB_BYTES = 384 << 20  # bytes read and written by the kernel that calibrates the HBM byte counters
# kernels launched by each entry point (once per call) at M = 8
ENTRY_KERNELS = {
    "rmsnorm_gateup_swiglu": ["qg::k_affine<8, 1,", "qg::k_split_reduce<1>"],
    "qgemv_affine4": ["qg::k_affine<8, 0,", "qg::k_split_reduce<0>"],
    "moe_expert_qgemv": ["qg::k_moe_gateup", "qg::k_moe_down"],
    "lmhead_argmax": ["qg::k_affine<8, 2,", "qg::k_lmhead_finalize"],
    "mlp_block": ["qg::k_mlp_block<8>"],
}


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
    ap.add_argument("--submission", choices=["graph", "eager"], default="eager",
                    help="timed steps replayed from a HIP graph of GRAPH_STEPS captured steps, or launched eagerly")
    ap.add_argument("--mlp", choices=["persistent", "separate"], default="separate",
                    help="MLP block as one persistent launch (mlp_block_affine4_tiled; tile-order layout only) or "
                         "as the two entry points rmsnorm_gateup_swiglu + qgemv_affine4")
    ap.add_argument("--layout", choices=["tiled", "canonical"], default="tiled",
                    help="storage of the affine-4 weights: tile order (packed once at set-up from the canonical "
                         "arrays; same bytes, reordered) or the canonical [N][K/8] layout")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="short run for a rocprofv3 --pmc pass: a copy of CALIB_BYTES (counter calibration), "
                         "then --steps M=8 steps; prints one JSON line")
    ap.add_argument("--compare-valu", metavar="NxK",
                    help="only time the affine-4 projection W[N,K] with the products on the matrix cores and on "
                         "the vector ALU (M = 1 and 8), print one JSON line; for a rocprofv3 run of that pair")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of a FETCH_SIZE and a WRITE_SIZE --pmc pass into "
                         "profiles/traffic.json (no GPU needed)")
    return ap.parse_args()


def traffic_from_counters(fetch_csv, write_csv):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel, each
    scaled by the factor that makes the calibration copy read and write
    CALIB_BYTES, summed over the kernels of each entry point."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {"source_hash": kernel_source_hash(), "calib_bytes": CALIB_BYTES, "kernels": {}}
    avgs = {}
    for which, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals = per_kernel(path, counter)
        copies = [v * 1024 for n, l in vals.items() if "bitwise_not" in n for v in l]
        if not copies:
            raise SystemExit(f"bench.py --traffic: no calibration copy found in {path}")
        factor = CALIB_BYTES / float(np.mean(copies))
        out[f"{which}_factor"] = round(factor, 4)
        avgs[which] = {n: float(np.mean(l)) * 1024 * factor for n, l in vals.items()}
    for entry, kernels in ENTRY_KERNELS.items():
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
        out["kernels"][entry] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic:
        traffic_from_counters(*args.traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus N with N > 1 is not supported "
              "(the projection has no multi-GPU path here)", file=sys.stderr)
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

    def run_step(i, M, b, ev=None):
        c = copies[i % C]
        ms = moe_stacks[i % 2]
        lg = logits[i % n_logit_sets]
        e = iter(ev) if ev is not None else None
        if e is not None:
            next(e).record()
        if persistent:
            ops.mlp_block_affine4_tiled(b["x"], gamma, vb["eps"], c["t_gu"], c["t_d"], D, I, h=b["h"], y=b["y"],
                                        ws=b["ws"])
        elif tiled:
            ops.rmsnorm_gateup_swiglu_tiled(b["x"], gamma, vb["eps"], *c["t_gu"], I, h=b["h"], ws=b["ws"])
        else:
            ops.rmsnorm_gateup_swiglu(b["x"], gamma, vb["eps"], c["codes_gu"], c["scales_gu"], c["biases_gu"],
                                      h=b["h"], ws=b["ws"])
        if e is not None:
            next(e).record()
        if persistent:
            pass
        elif tiled:
            ops.qgemv_affine4_tiled(b["h"], *c["t_d"], D, y=b["y"], ws=b["ws"])
            if e is not None:
                next(e).record()
        else:
            ops.qgemv_affine4(b["h"], c["codes_d"], c["scales_d"], c["biases_d"], y=b["y"], ws=b["ws"])
            if e is not None:
                next(e).record()
        ops.moe_expert_qgemv(xm, lg, top_k, ms["w_gu"], ms["w_down"], y=b["ym"], out_ids=b["mids"], out_w=b["mw"],
                             ws=b["ws"])
        if e is not None:
            next(e).record()
        dr = draft[:M].contiguous() if M < 8 else draft
        if tiled:
            ops.lmhead_argmax_tiled(b["xl"], *c["t_lm"], V, draft=dr, ids=b["ids"], accepted=b["acc"], ws=b["ws"])
        else:
            ops.lmhead_argmax(b["xl"], c["codes_lm"], c["scales_lm"], c["biases_lm"], draft=dr, ids=b["ids"],
                              accepted=b["acc"], ws=b["ws"])
        if e is not None:
            next(e).record()

    spread = {}

    graph_checks = {}

    def timed(M, steps, warmup):
        b = bufs(M)
        use_graph = args.submission == "graph"
        s = torch.cuda.Stream() if use_graph else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            for i in range(warmup):
                run_step(i, M, b)
        torch.cuda.synchronize()
        # graph length: the largest divisor of the step count up to GRAPH_STEPS, so
        # that exactly `steps` steps are timed
        glen = max(d for d in range(1, GRAPH_STEPS + 1) if steps % d == 0) if use_graph else 1
        if use_graph:
            # the graph holds glen consecutive steps and every replay repeats them
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(glen):
                    run_step(i, M, b)
            torch.cuda.synchronize()
        # K steps timed start to end; events at five sub-batch boundaries (no
        # synchronisation between them) give the spread of the per-step time
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
        per_unit = glen
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
        sub = [evb[j].elapsed_time(evb[j + 1]) / ((cut[j + 1] - cut[j]) * per_unit) for j in range(nsub)]
        spread[M] = {"median_ms": round(float(np.median(sub)), 5), "p10_ms": round(float(np.percentile(sub, 10)), 5),
                     "p90_ms": round(float(np.percentile(sub, 90)), 5), "sub_batches": nsub}
        # per-kernel durations: the same steps again with events around each launch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
        with torch.cuda.stream(s):
            for i in range(steps):
                run_step(warmup + steps + i, M, b, evs[i])
        torch.cuda.synchronize()
        per = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)])) * 1e3
               for j, n in enumerate(names)}
        inst = float(np.mean([evs[i][0].elapsed_time(evs[i][len(names)]) for i in range(steps)]))
        return ms_step, wall, per, inst, b

    if args.pmc_pass:
        # an elementwise kernel that reads and writes CALIB_BYTES (a plain
        # device copy may go to the DMA engine and never show up as a kernel)
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        b = bufs(8)
        for i in range(args.warmup + args.steps):
            run_step(i, 8, b)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": True, "calib_bytes": CALIB_BYTES, "steps": args.warmup + args.steps}), flush=True)
        return

    log(f"[bench] timing M=8: warmup {args.warmup}, steps {args.steps}")
    ms8, wall8, per8, inst8, b8 = timed(8, args.steps, args.warmup)
    bytes8, wbytes = step_bytes(8)
    total8 = sum(bytes8.values())
    value = total8 / (ms8 * 1e-3) / 1e9
    log(f"[bench] M=8: {ms8 * 1e3:.1f} us/step -> {value:.0f} GB/s; per kernel (us): "
        + ", ".join(f"{n}={per8[n]:.1f}" for n in names))
    accepted = int(b8["acc"].cpu()[0])

    ms1 = per1 = None
    if not args.no_m1:
        s1 = max(20, args.steps // 2)
        log(f"[bench] timing M=1: steps {s1}")
        ms1, _, per1, _, _ = timed(1, s1, max(5, args.warmup // 2))
        log(f"[bench] M=1: {ms1 * 1e3:.1f} us/step; ratio {ms8 / ms1:.3f}")

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

    kernels = {}
    for n in names:
        k = {"us_m8": round(per8[n], 2), "bytes_m8": bytes8[n], "gb_s_m8": round(bytes8[n] / (per8[n] * 1e-6) / 1e9, 1),
             "frac_m8": round(bytes8[n] / (per8[n] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        if per1 is not None:
            b1 = step_bytes(1)[0][n]
            k.update({"us_m1": round(per1[n], 2), "gb_s_m1": round(b1 / (per1[n] * 1e-6) / 1e9, 1),
                      "frac_m1": round(b1 / (per1[n] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                      "verify_ratio": round(per8[n] / per1[n], 3)})
        kernels[n] = k

    # dominant kernel = largest share of the step's time
    dom = max(names, key=lambda n: per8[n])
    dom_gbs = bytes8[dom] / (per8[dom] * 1e-6) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tf = json.load(open(TRAFFIC_FILE))
            ent = tf.get("kernels", {}).get(dom)
            if ent and tf.get("source_hash") == kernel_source_hash():
                traffic = ent.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    entry = {"mlp_block": "mlp_block_affine4_tiled", "moe_expert_qgemv": "moe_expert_qgemv"}.get(
        dom, dom + ("_tiled" if tiled else ""))
    roofline = {"kernel": entry, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": bytes8[dom], "avg_launch_us": round(per8[dom], 2)}

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
                   "submission": ("HIP graph replays of captured steps" if args.submission == "graph"
                                  else "eager launches"),
                   "layout": "tile-order (same bytes as canonical, packed at set-up)" if tiled else "canonical", "algorithmic_bytes_per_step": total8,
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
        "instrumented_ms_per_step": round(inst8, 5),
        "graph_check": graph_checks or None,
        "wall_s_timed": round(wall8, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


def per_call_us(torch, fn, reps):
    """Microseconds per call of fn(i): a short warm-up, then HIP events around reps back-to-back calls."""
    for i in range(min(reps, 20)):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


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
    out["lm_head_151936x1024"] = res
    del tcs
    log("[bench] context: " + json.dumps(out))
    return out


def cpu_baseline(vb, lm, moe, step_bytes, min_seconds=10.0, max_steps=12):
    """The CPU oracle (plain single-threaded C, fp64) on the same step: the
    full MLP block at M=8, the MoE token, and the LM head at M=8 with its draft
    ids.  Whole steps are repeated (the MoE router logits rotating as in the
    GPU run) until min_seconds of CPU work have been timed (at most
    max_steps); reported in the same unit as the GPU value."""
    import oracle
    n, t = 0, time.perf_counter()
    while True:
        oracle.mlp_block(vb["x"], vb["gamma"], vb["eps"], vb["codes_gu"], vb["scales_gu"], vb["biases_gu"],
                         vb["codes_d"], vb["scales_d"], vb["biases_d"])
        oracle.moe(moe["x"], moe["logits"][n % len(moe["logits"])], moe["top_k"], moe["w_gu"], moe["w_down"],
                   moe["E"], moe["D"], moe["I"])
        oracle.lmhead(lm["x"], lm["codes"], lm["scales"], lm["biases"], draft=lm["draft"], want_logits=False)
        n += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds or n >= max_steps:
            break
    log(f"[bench] cpu oracle: {n} full steps in {dt:.1f}s")
    return {"value": round(n * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full steps (MLP block M=8, MoE token with rotating router logits, LM head M=8), "
                      "same seeded inputs as the GPU run",
            "steps": n, "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
