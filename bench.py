#!/usr/bin/env python3
"""Benchmark of block-sparse FlashAttention prefill on one MI355X.

Metric: prefill attention executed TFLOP/s (bf16 MFMA, fp32 accumulate) and
speedup of the same kernel over its dense run (threshold -inf), on the
Llama-3.1-8B-shaped 32K layer (B=1, 32 query heads over 8 KV heads, d=128,
128x128 tiles, causal) with fixed-k thresholds designed for 0% (dense), 60%,
80% and 90% skipped tiles.

One step = one bsfa_prefill launch per sweep point over the same resident
inputs.  Inputs are synthetic (seeded generator), thresholds come from the
library's own calibration pass (tile maxima + fixed-k selection on the GPU),
outside the timed region.  Launch times are taken with HIP events on the
stream the kernels run on.

Also reported, outside ``value``:
  * ``long_context``: the 128K GQA layer (32 query heads over 4 KV heads) at
    threshold -inf and at its ~95% fixed-k point, timed the same way
    (``--no-128k`` skips it);
  * ``gate_study``: on the 32K inputs, the fixed-k points next to the gap gate
    (skip a tile below the running maximum minus a gap) at several gaps -
    realised skip fraction, time and error against the dense output
    (``--no-gate-study`` skips it);
  * ``tile_study``: on the same inputs, the sweep on 128 x 64 tiles (the
    pages' A100 tile: finer skip granularity, half the work per gate) next
    to 128 x 128 - skip fraction, time and error against the dense output
    (``--no-tile-study`` skips it);
  * ``cold_cache``: each sweep point timed right after a 512 MB buffer has
    been overwritten on the same stream, so that no K/V tile is left in L2 or
    the Infinity Cache when the launch starts (``--no-cold-cache`` skips it);
  * ``device``: the GPU's name and compute-unit count as the runtime reports them.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one GPU.
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
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
GAP_SWEEP = (1.0, 2.0, 3.0, 4.5, 6.0)  # gaps of the gate study, scaled-score units


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 over the forward kernel sources (template header, parameter block and the 128 x 128 instantiation)."""
    csrc = os.path.join(ROOT, "block_sparse_flashattention_tiled_amd", "csrc")
    h = hashlib.sha256()
    for f in ("bsfa_fwd_kernels.h", "bsfa_internal.h", "bsfa_fwd_128x128.hip"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"bsfa_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(data, w, ks, budget_s):
    """Time the CPU oracle on a bounded, seeded sample of query blocks."""
    sys.path.insert(0, ROOT)
    import oracle
    from block_sparse_flashattention_tiled_amd import accounting as acc

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    rng = np.random.default_rng(1)
    M, blk, d = w.n_blocks, w.block, w.head_dim
    tile = acc.tile_matmul_flops(blk, blk, d)
    flops = 0
    spent = 0.0
    n = 0
    try:
        while spent < budget_s and n < 4096:
            b = int(rng.integers(w.batch))
            h = int(rng.integers(w.heads_q))
            i = int(rng.integers(M))
            k = ks[n % len(ks)]
            # the oracle's own threshold for this block (calibration is not timed)
            tm = oracle.tile_maxima(data["q"][b:b + 1], data["k"][b:b + 1], w.causal, blk, heads=[h], rows=[i])
            tau = -np.inf if k is None else oracle.calibrate_row(tm[0, h, i], i, k, w.causal)
            thr = np.full((w.heads_q, M), tau)
            t0 = time.perf_counter()
            r = oracle.run_blocks(data["q"][b:b + 1], data["k"][b:b + 1], data["v"][b:b + 1], thr, w.causal, blk,
                                  [(0, h, i)])[0]
            spent += time.perf_counter() - t0
            computed = (i + 1) if w.causal else M
            flops += tile * computed + tile * (computed - r["skip_count"])
            n += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n} query blocks (random b/head/block, seed 1) of {w.name} over the sweep points, "
                  f"float64 numpy with BLAS on {cores} threads, {spent:.1f} s",
    }


class Layer:
    """Resident inputs, calibration and output buffers of one workload on one tile shape."""

    def __init__(self, name, seed, torch, bb, wl, acc):
        self.torch, self.bb, self.acc = torch, bb, acc
        self.w = w = wl.get_config(name)
        log(f"generating {w.name}: B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seq_len} d={w.head_dim}")
        t0 = time.time()
        self.data = wl.generate(w, seed=seed)
        log(f"generated in {time.time() - t0:.1f} s; uploading")
        self.q, self.k, self.v = (bb.bits_to_device(self.data[n]) for n in ("q", "k", "v"))
        self.out = torch.empty((w.batch, w.heads_q, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((w.batch, w.heads_q, w.seq_len), dtype=torch.float32, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.set_tile((w.block, w.block))

    def set_tile(self, tile):
        """Switch to B_M x B_N tiles: block counts, shape, and the calibration pass (untimed)."""
        w, bb = self.w, self.bb
        self.tile = tuple(tile)
        self.M, self.Mkv = -(-w.seq_len // tile[0]), -(-w.seq_len // tile[1])
        self.shape = bb.make_shape(w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, self.M)
        self.block = bb.make_block(*tile)
        self.tmax = bb.tile_max(self.q, self.k, w.causal, self.tile)

    def fixed_k_points(self, targets):
        w, (bm, bn) = self.w, self.tile
        points = []
        for tgt in targets:
            kk = self.acc.grid_k_for_target(w.seq_len, bm, bn, tgt, w.causal)
            if kk is None:
                thr = self.torch.full((w.heads_q, self.M), float("-inf"), dtype=self.torch.float32, device="cuda")
            else:
                thr = self.bb.calibrate(self.tmax, [kk], w.causal, self.tile, w.seq_len, w.head_dim)[0].contiguous()
            points.append({"target": tgt, "k": kk, "thr": thr, "gate": "threshold", "tile": list(self.tile)})
        return points

    def launch(self, pt, counts, out=None):
        w, bb = self.w, self.bb
        out = self.out if out is None else out
        if pt["gate"] == "threshold":
            bb.bsfa_prefill(self.q, self.k, self.v, out, self.lse, counts, pt["thr"], self.shape, int(w.causal),
                            self.block, self.stream)
        else:
            bb.bsfa_prefill_gated(self.q, self.k, self.v, out, self.lse, counts, pt["thr"], self.shape,
                                  int(w.causal), self.block, bb.GATES[pt["gate"]], None, None, self.stream)

    def measure(self, points, steps, warmup):
        """Time every point ``steps`` times (HIP events around each launch on the
        launching stream); fill per-point statistics.  Returns the step time."""
        torch, acc, w = self.torch, self.acc, self.w
        counts = [torch.empty((w.batch, w.heads_q, self.M), dtype=torch.int32, device="cuda") for _ in points]
        log(f"{w.name}: warmup {warmup} steps x {len(points)} launches")
        for _ in range(warmup):
            for pi, pt in enumerate(points):
                self.launch(pt, counts[pi])
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in points]
              for _ in range(steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(self.stream)
        for s in range(steps):
            for pi, pt in enumerate(points):
                ev[s][pi][0].record(self.stream)
                self.launch(pt, counts[pi])
                ev[s][pi][1].record(self.stream)
        t_end.record(self.stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        log(f"{w.name}: timed {steps} steps in {total_ms:.1f} ms")
        (bm, bn), d, n = self.tile, w.head_dim, w.seq_len
        dense_flops = acc.grid_executed_flops(w.batch, w.heads_q, n, bm, bn, d, 0, w.causal)
        computed = acc.grid_computed_tiles(n, bm, bn, w.causal) * w.batch * w.heads_q
        for pi, pt in enumerate(points):
            durs = [ev[s][pi][0].elapsed_time(ev[s][pi][1]) for s in range(steps)]
            skipped = int(counts[pi].sum().item())
            fl = acc.grid_executed_flops(w.batch, w.heads_q, n, bm, bn, d, skipped, w.causal)
            pt.update(ms_mean=float(np.mean(durs)), ms_median=float(np.median(durs)), ms_min=float(np.min(durs)),
                      skipped_tiles=skipped, skip_fraction=skipped / computed, executed_flops=fl)
            if pt.get("k") is not None or pt["gate"] == "threshold":
                pt["designed_skip_fraction"] = (acc.grid_designed_skip_fraction(n, bm, bn, pt["k"], w.causal)
                                                if pt.get("k") is not None else 0.0)
            pt["executed_tflops"] = fl / (pt["ms_mean"] * 1e-3) / 1e12
            pt["dense_equivalent_tflops"] = dense_flops / (pt["ms_mean"] * 1e-3) / 1e12
        return total_ms / steps

    def measure_cold(self, points, reps, flush_bytes=512 << 20):
        """Mean launch time of each point when the launch follows an overwrite of
        ``flush_bytes`` of device memory (caches hold no K/V tile of the layer)."""
        torch, w = self.torch, self.w
        buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
        counts = torch.empty((w.batch, w.heads_q, self.M), dtype=torch.int32, device="cuda")
        out = []
        for pt in points:
            durs = []
            for r in range(reps + 1):  # the first launch of a point is not counted
                buf.fill_(float(r))
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
                self.launch(pt, counts)
                e1.record(self.stream)
                torch.cuda.synchronize()
                if r:
                    durs.append(e0.elapsed_time(e1))
            out.append({"target": pt["target"], "k": pt["k"], "ms_cold_mean": float(np.mean(durs)),
                        "ms_warm_mean": pt["ms_mean"], "cold_over_warm": float(np.mean(durs)) / pt["ms_mean"]})
        del buf
        return out

    def errors_vs(self, ref_out, ref_lse, pt):
        """Error of one point's output against a reference output (same inputs)."""
        torch, w = self.torch, self.w
        counts = torch.empty((w.batch, w.heads_q, self.M), dtype=torch.int32, device="cuda")
        out = torch.empty_like(self.out)
        self.launch(pt, counts, out)
        torch.cuda.synchronize()
        diff = (out - ref_out).double()
        rel = float(diff.norm() / ref_out.double().norm())
        return {"rel_l2_out": rel, "max_abs_out": float(diff.abs().max()),
                "mean_abs_lse": float((self.lse - ref_lse).abs().double().mean())}


def public(points):
    return [{kk: vv for kk, vv in pt.items() if kk != "thr"} for pt in points]


def speedups(points):
    dense_ms = points[0]["ms_mean"]
    for pt in points:
        f = pt["skip_fraction"]
        pt["speedup_vs_dense"] = dense_ms / pt["ms_mean"]
        pt["flop_ratio"] = 2.0 / (2.0 - f)
        pt["speedup_floor"] = 0.8 * pt["flop_ratio"]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle baseline budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-128k", action="store_true", help="skip the 128K long-context leg")
    ap.add_argument("--no-gate-study", action="store_true", help="skip the gap-gate comparison")
    ap.add_argument("--no-tile-study", action="store_true", help="skip the 128 x 64 tile comparison")
    ap.add_argument("--no-cold-cache", action="store_true", help="skip the cold-cache timing of the sweep")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run one plain 1 GiB device copy, whose HBM counters calibrate the kernel's")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_flashattention_tiled_amd import accounting as acc
    from block_sparse_flashattention_tiled_amd import binding as bb
    from block_sparse_flashattention_tiled_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bb.load_library()

    # ---- the headline workload -------------------------------------------------
    lay = Layer(args.workload, args.seed, torch, bb, wl, acc)
    w = lay.w
    targets = list(w.skip_targets)
    if 0.0 not in targets:
        targets = [0.0] + targets  # the dense reference for speedups
    points = lay.fixed_k_points(targets)
    torch.cuda.synchronize()
    if args.traffic_probe:
        # a copy of known size: reads 1 GiB and writes 1 GiB; profiling counters
        # taken in the same run are scaled by what this copy reports
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    step_ms = lay.measure(points, args.steps, args.warmup)
    speedups(points)
    timed = [pt for pt in points if pt["target"] in w.skip_targets]
    step_flops = sum(pt["executed_flops"] for pt in timed)
    sum_dur = sum(pt["ms_mean"] for pt in timed)
    # the step also holds the dense reference launch when the sweep lacks it
    value = step_flops / (step_ms * 1e-3) / 1e12 if len(timed) == len(points) else \
        step_flops / (sum_dur * 1e-3) / 1e12
    achieved = step_flops / (sum_dur * 1e-3) / 1e12  # algorithmic FLOPs per launch / mean launch time

    res = {
        "metric": "prefill attention executed TFLOP/s + speedup vs dense at 32K/128K, bf16",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator at the layer's shape; no dataset or model weights)",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "heads_q": w.heads_q,
            "heads_kv": w.heads_kv,
            "seq_len": w.seq_len,
            "head_dim": w.head_dim,
            "block": w.block,
            "causal": w.causal,
            "skip_targets": list(w.skip_targets),
            "thresholds": "fixed-k, self-calibrated on the GPU (bsfa_tile_max + bsfa_calibrate)",
        },
        "points": public(points),
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(w.name),
        },
    }
    props = torch.cuda.get_device_properties(0)
    res["device"] = {"name": props.name, "compute_units": props.multi_processor_count,
                     "arch": getattr(props, "gcnArchName", None)}
    if not args.no_cold_cache:
        res["cold_cache"] = {
            "flush": "512 MB device buffer overwritten on the launch stream before each timed launch",
            "points": lay.measure_cold(points, 3),
        }

    # ---- the dense output: reference of both studies --------------------------
    if not (args.no_gate_study and args.no_tile_study):
        ref_out = lay.out.clone()
        lay.launch(points[0], torch.empty((w.batch, w.heads_q, lay.M), dtype=torch.int32, device="cuda"), ref_out)
        torch.cuda.synchronize()
        ref_lse = lay.lse.clone()

    # ---- gap gate next to the fixed-k table on the same inputs -----------------
    if not args.no_gate_study:
        study = [dict(pt, gate="threshold") for pt in points[1:]]
        for gap in GAP_SWEEP:
            study.append({"target": None, "k": None, "gap": gap, "gate": "gap",
                          "thr": torch.full((w.heads_q, lay.M), gap, dtype=torch.float32, device="cuda")})
        lay.measure(study, max(3, args.steps // 4), 1)
        for pt in study:
            pt.update(lay.errors_vs(ref_out, ref_lse, pt))
            pt["speedup_vs_dense"] = points[0]["ms_mean"] / pt["ms_mean"]
        res["gate_study"] = {
            "workload": w.name,
            "reference": "the same kernel at threshold -inf",
            "gap_gate": "skip tile j iff its maximum scaled score < (largest maximum of the kept tiles) - gap",
            "points": public(study),
        }

    # ---- 128 x 64 tiles next to 128 x 128 on the same inputs --------------------
    if not args.no_tile_study and w.block == 128:
        sq = [dict(pt) for pt in points]
        for pt in sq:
            pt.update(lay.errors_vs(ref_out, ref_lse, pt))
        lay.set_tile((128, 64))
        rect = lay.fixed_k_points(targets)
        lay.measure(rect, max(3, args.steps // 4), 1)
        for pt in rect:
            pt.update(lay.errors_vs(ref_out, ref_lse, pt))
            pt["speedup_vs_dense"] = points[0]["ms_mean"] / pt["ms_mean"]
        res["tile_study"] = {
            "workload": w.name,
            "reference": "the 128 x 128 kernel at threshold -inf; speedup_vs_dense relative to it",
            "tiles": {"128x128": public(sq), "128x64": public(rect)},
        }
        lay.set_tile((w.block, w.block))
    if not (args.no_gate_study and args.no_tile_study):
        del ref_out

    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline, ~{args.cpu_seconds:.0f} s")
        ks = [pt["k"] for pt in timed]
        res["cpu_baseline"] = cpu_baseline(lay.data, w, ks, args.cpu_seconds)
    del lay
    torch.cuda.empty_cache()

    # ---- the 128K long-context layer ---------------------------------------------
    if not args.no_128k and args.workload != "gqa128k":
        big = Layer("gqa128k", args.seed, torch, bb, wl, acc)
        bpts = big.fixed_k_points([0.0] + list(big.w.skip_targets))
        big.measure(bpts, max(3, args.steps // 4), 1)
        speedups(bpts)
        res["long_context"] = {
            "workload": big.w.name,
            "batch": big.w.batch, "heads_q": big.w.heads_q, "heads_kv": big.w.heads_kv,
            "seq_len": big.w.seq_len, "head_dim": big.w.head_dim, "block": big.w.block, "causal": big.w.causal,
            "points": public(bpts),
        }
        del big
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
