#!/usr/bin/env python3
"""Benchmark of block-sparse FlashAttention prefill on one MI355X.

Metric: prefill attention executed TFLOP/s (bf16 MFMA, fp32 accumulate) and
speedup of the same kernel over its dense run (threshold -inf).  The headline
(``value``) is the Llama-3.1-8B-shaped 32K layer (B=1, 32 query heads over 8
KV heads, d=128, 128x128 tiles, causal) with fixed-k thresholds designed for
0% (dense), 60%, 80% and 90% skipped tiles: one step = one ``bsfa_prefill``
launch per sweep point over the same resident inputs, and ``value`` = the
executed FLOPs of all four launches / the step time.

Inputs are synthetic (seeded generator).  Thresholds come from the library's
own calibration pass (tile maxima + fixed-k selection on the GPU) on the
evaluation inputs, outside the timed region.  Launch times are taken with HIP
events on the stream the kernels run on.

Also reported, outside ``value``:
  * ``roofline``: the forward kernel against the bf16 MFMA peak, overall and
    per sweep point, with the V tiles each point loads and, when the counter
    summary under profiles/ was taken on the current kernel sources, the
    point's MFMA-busy share, HBM bytes and L2 read bytes;
  * ``legs``: the 8K layer (dense, ~50%), the bidirectional DiT-shaped layer
    (dense, ~75%) and the 128K GQA layer (dense, ~95%), timed the same way
    after at least 300 ms of untimed launches (their inputs are generated on
    the host first, and a 0.6 ms launch timed during the clock's ramp from idle
    reads up to 10% slow); the held-out, gate and tile studies settle the same
    way;
  * ``held_out``: the 32K sweep with thresholds calibrated on two other seeds
    (the batch axis of the calibration pass as the samples, averaged) and
    evaluated on seed 0: designed against realised skip fraction, per-row and
    per-head density error, time;
  * ``gate_study``: the fixed-k points next to the gap gate (skip a tile below
    the running maximum minus a gap) at several gaps;
  * ``tile_study``: the sweep on 128 x 64 tiles next to 128 x 128;
  * ``cold_cache``: each sweep point timed right after a 512 MB overwrite;
  * ``cpu_baseline``: the CPU oracle (float64 numpy) on the host cores - whole
    layers for the tiny and 8K configurations, a bounded sample of query
    blocks for the 32K sweep and the DiT layer with the whole-layer time
    extrapolated by FLOPs.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one
GPU.  ``--profile`` times the headline sweep only (the command the rocprofv3
summaries under profiles/ are taken with); ``--summarize-trace`` and
``--summarize-counters`` turn that profiler output into those summaries.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
GAP_SWEEP = (1.0, 2.0, 3.0, 4.5, 6.0)  # gaps of the gate study, scaled-score units
FWD_KERNEL = "bsfa_fwd_pair_kernel"
PIPE_KERNEL = "bsfa_fwd_pipe_kernel"
COUNTERS_FILE = "bsfa_fwd_llama32k_counters.json"
KERNEL_SOURCES = ("bsfa_fwd_kernels.h", "bsfa_fwd_pipe.h", "bsfa_internal.h", "bsfa_fwd_128x128.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 over the forward kernel sources (template headers, parameter block and the 128 x 128 instantiation)."""
    csrc = os.path.join(ROOT, "block_sparse_flashattention_tiled_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_counters():
    """Per-point counter summary of the headline sweep from profiles/, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, COUNTERS_FILE)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha256") != kernel_source_hash():
        return None
    return rec


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:  # noqa: BLE001
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------------------------


def _oracle_time(oracle, data, w, thr, blocks):
    t0 = time.perf_counter()
    res = oracle.run_blocks(data["q"], data["k"], data["v"], thr, w.causal, w.block, blocks)
    return time.perf_counter() - t0, sum(r["skip_count"] for r in res)


def cpu_baseline(layers, sample_budget_s):
    """The oracle as it stands on the host cores: whole layers where they take
    seconds (tiny, 8K), a bounded random sample of query blocks elsewhere (32K
    sweep, DiT) with the whole-layer time extrapolated by executed FLOPs.

    ``layers``: {name: (Layer, [points with GPU thresholds "thr"])}."""
    sys.path.insert(0, ROOT)
    import oracle
    from block_sparse_flashattention_tiled_amd import accounting as acc

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    full, extrap = [], []
    headline = None
    try:
        for name, (lay, pts) in layers.items():
            w = lay.w
            M = w.n_blocks
            tile = acc.tile_matmul_flops(w.block, w.block, w.head_dim)
            dense = acc.grid_executed_flops(w.batch, w.heads_q, w.seq_len, w.block, w.block, w.head_dim, 0,
                                            w.causal)
            if name in ("tiny", "llama8k"):
                blocks = [(b, h, i) for b in range(w.batch) for h in range(w.heads_q) for i in range(M)]
                for pt in pts:
                    thr = pt["thr"].cpu().numpy()
                    s, skipped = _oracle_time(oracle, lay.data, w, thr, blocks)
                    fl = dense - skipped * tile
                    full.append({"workload": name, "target": pt["target"], "seconds": s, "tflops": fl / s / 1e12,
                                 "skipped_tiles": int(skipped)})
                continue
            rng = np.random.default_rng(1)
            budget = sample_budget_s / (2 if name == "llama32k" else 4)
            spent, flops, n = 0.0, 0, 0
            per_point = {}
            while spent < budget and n < 4096:
                pt = pts[n % len(pts)]
                b, h, i = int(rng.integers(w.batch)), int(rng.integers(w.heads_q)), int(rng.integers(M))
                s, skipped = _oracle_time(oracle, lay.data, w, pt["thr"].cpu().numpy(), [(b, h, i)])
                computed = (i + 1) if w.causal else M
                fl = tile * (2 * computed - skipped)
                spent += s
                flops += fl
                n += 1
                acc_pt = per_point.setdefault(pt["target"], [0.0, 0])
                acc_pt[0] += s
                acc_pt[1] += fl
            rate = flops / spent
            for pt in pts:
                s_pt, fl_pt = per_point.get(pt["target"], (0.0, 0))
                r = fl_pt / s_pt if s_pt else rate
                extrap.append({"workload": name, "target": pt["target"],
                               "seconds_whole_layer_extrapolated": pt["executed_flops"] / r,
                               "sample_tflops": r / 1e12})
            if name == "llama32k":
                headline = {"value": rate / 1e12, "blocks": n, "seconds": spent}
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {
        "value": headline["value"] if headline else None,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{headline['blocks']} query blocks (random b/head/block, seed 1) of llama32k over its four "
                   f"sweep points, float64 numpy with BLAS on {cores} threads, {headline['seconds']:.1f} s"
                   if headline else None),
        "full_runs": full,
        "extrapolated": extrap,
        "note": "whole-layer oracle runs where they take seconds (tiny, 8K); elsewhere a bounded sample of "
                "query blocks at the same thresholds, whole-layer time extrapolated by executed FLOPs "
                "(labelled extrapolated)",
    }


# --------------------------------------------------------------------------------------------
# GPU layers
# --------------------------------------------------------------------------------------------


class Layer:
    """Resident inputs, calibration and output buffers of one workload on one tile shape."""

    def __init__(self, name, seed, torch, bb, wl, acc, data=None):
        self.torch, self.bb, self.acc, self.wl = torch, bb, acc, wl
        self.w = w = wl.get_config(name)
        if data is None:
            log(f"generating {w.name}: B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seq_len} d={w.head_dim}")
            t0 = time.time()
            data = wl.generate(w, seed=seed)
            log(f"generated in {time.time() - t0:.1f} s; uploading")
        self.data = data
        self.q, self.k, self.v = (bb.bits_to_device(self.data[n]) for n in ("q", "k", "v"))
        self.out = torch.empty((w.batch, w.heads_q, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((w.batch, w.heads_q, w.seq_len), dtype=torch.float32, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.set_tile((w.block, w.block))

    def set_tile(self, tile, tmax=None):
        """Switch to B_M x B_N tiles: block counts, shape, and the calibration pass (untimed).
        ``tmax``: tile maxima [S, H, M, M_KV] of other calibration samples instead of this layer's."""
        w, bb = self.w, self.bb
        self.tile = tuple(tile)
        self.M, self.Mkv = -(-w.seq_len // tile[0]), -(-w.seq_len // tile[1])
        self.shape = bb.make_shape(w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, self.M)
        self.block = bb.make_block(*tile)
        self.tmax = bb.tile_max(self.q, self.k, w.causal, self.tile) if tmax is None else tmax

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

    def measure(self, points, steps, warmup, settle_ms=0.0):
        """Time every point ``steps`` times (HIP events around each launch on the
        launching stream); fill per-point statistics.  Returns the step time.

        ``settle_ms``: after the warmup steps, keep launching the points until that
        much wall time has passed, so that a layer measured after a stretch of host
        work (input generation) is timed at the clock the GPU holds under load and
        not during its ramp from idle."""
        torch, acc, w = self.torch, self.acc, self.w
        counts = [torch.empty((w.batch, w.heads_q, self.M), dtype=torch.int32, device="cuda") for _ in points]
        log(f"{w.name}: warmup {warmup} steps x {len(points)} launches" +
            (f", then at least {settle_ms:.0f} ms of launches" if settle_ms > 0 else ""))
        for _ in range(warmup):
            for pi, pt in enumerate(points):
                self.launch(pt, counts[pi])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while settle_ms > 0 and (time.perf_counter() - t0) * 1e3 < settle_ms:
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
            pt["frac_of_peak"] = pt["executed_tflops"] / PEAK_BF16_TFLOPS
        return total_ms / steps

    def tile_loads(self, pt):
        """K and V tile loads of one launch at ``pt``, from the per-tile states of a
        diagnostics launch (untimed): a workgroup streams K_j once for its two
        query units and V_j once when either unit keeps tile j."""
        torch, bb, w = self.torch, self.bb, self.w
        res = bb.prefill(self.q, self.k, self.v, pt["thr"], w.causal, self.tile, diagnostics=True)
        st = res["tile_state"]
        computed = st != bb.TILE_PRUNED
        kept = (st == bb.TILE_KEPT) | (st == bb.TILE_DIAGONAL)
        B, H, M, Mkv = st.shape
        G = w.group
        # heads run in query-head pairs (2p, 2p + 1 of a group) when G is even;
        # with G odd, bidirectional attention runs every head in block pairs
        # (query blocks 2p, 2p + 1), causal attention only the group's last head
        hp = G - (G % 2) if (G % 2 == 0 or w.causal) else 0
        k_loads = v_loads = 0
        if hp:
            c = computed.view(B, H // G, G, M, Mkv)[:, :, :hp].reshape(B, -1, 2, M, Mkv)
            kk = kept.view(B, H // G, G, M, Mkv)[:, :, :hp].reshape(B, -1, 2, M, Mkv)
            k_loads += int(c.any(2).sum())
            v_loads += int(kk.any(2).sum())
        if hp < G:
            c = computed.view(B, H // G, G, M, Mkv)[:, :, hp:].reshape(B, -1, M, Mkv)
            kk = kept.view(B, H // G, G, M, Mkv)[:, :, hp:].reshape(B, -1, M, Mkv)
            if M % 2:
                pad = torch.zeros((B, c.shape[1], 1, Mkv), dtype=torch.bool, device=st.device)
                c, kk = torch.cat([c, pad], 2), torch.cat([kk, pad], 2)
            k_loads += int(c.view(B, c.shape[1], -1, 2, Mkv).any(3).sum())
            v_loads += int(kk.view(B, kk.shape[1], -1, 2, Mkv).any(3).sum())
        del res
        bm, bn = self.tile
        tile_bytes = bn * w.head_dim * 2
        q_bytes = w.batch * w.heads_q * w.seq_len * w.head_dim * 2
        return {"k_tile_loads": k_loads, "v_tile_loads": v_loads,
                "v_loads_per_k_load": v_loads / max(k_loads, 1),
                "stream_read_bytes": q_bytes + (k_loads + v_loads) * tile_bytes}

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

    def density_errors(self, pt):
        """Realised against designed density (kept / computed tiles) per (head, query
        block) row and per head, for a fixed-k point."""
        torch, w = self.torch, self.w
        counts = torch.empty((w.batch, w.heads_q, self.M), dtype=torch.int32, device="cuda")
        self.launch(pt, counts)
        torch.cuda.synchronize()
        rows = self.acc.grid_rows(w.seq_len, self.tile[0], self.tile[1], w.causal)
        comp = np.array([c for c, _ in rows], dtype=np.float64)
        off = np.array([o for _, o in rows], dtype=np.float64)
        designed = (np.minimum(pt["k"], off) + (comp - off)) / comp
        realised = (comp[None, None, :] - counts.cpu().numpy()) / comp[None, None, :]
        err = realised - designed[None, None, :]
        gated = off > pt["k"]  # rows whose threshold can skip anything
        head_real = (comp[None, None, :] - counts.cpu().numpy()).sum(-1) / comp.sum()
        head_design = (np.minimum(pt["k"], off) + (comp - off)).sum() / comp.sum()
        return {"row_density_error_mean": float(err[..., gated].mean()),
                "row_density_error_std": float(err[..., gated].std()),
                "head_density_error_std": float((head_real - head_design).std()),
                "head_density_error_max_abs": float(np.abs(head_real - head_design).max())}


def public(points):
    return [{kk: vv for kk, vv in pt.items() if kk != "thr"} for pt in points]


def speedups(points):
    dense_ms = points[0]["ms_mean"]
    for pt in points:
        f = pt["skip_fraction"]
        pt["speedup_vs_dense"] = dense_ms / pt["ms_mean"]
        pt["flop_ratio"] = 2.0 / (2.0 - f)
        pt["speedup_floor"] = 0.8 * pt["flop_ratio"]
        pt["speedup_over_floor"] = pt["speedup_vs_dense"] / pt["speedup_floor"]


LEG_SETTLE_MS = 300.0  # launches before a leg's timed steps (its inputs are generated on the host first)


def run_leg(name, seed, steps, torch, bb, wl, acc):
    lay = Layer(name, seed, torch, bb, wl, acc)
    pts = lay.fixed_k_points([0.0] + [t for t in lay.w.skip_targets if t > 0])
    lay.measure(pts, steps, 1, settle_ms=LEG_SETTLE_MS)
    speedups(pts)
    for pt in pts:
        pt.update(lay.tile_loads(pt))
    w = lay.w
    leg = {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
           "seq_len": w.seq_len, "head_dim": w.head_dim, "block": w.block, "causal": w.causal,
           "steps": steps, "warmup": 1, "settle_ms": LEG_SETTLE_MS, "points": public(pts)}
    return lay, pts, leg


def held_out(lay, targets, seeds, torch, bb, wl):
    """Thresholds calibrated on other seeds (their tile maxima stacked on the batch
    axis, thresholds averaged over them) and evaluated on the layer's inputs."""
    w = lay.w
    tms = []
    for s in seeds:
        log(f"held-out calibration: generating {w.name} seed {s}")
        d = wl.generate(w, seed=s)
        q, k = bb.bits_to_device(d["q"]), bb.bits_to_device(d["k"])
        tms.append(bb.tile_max(q, k, w.causal, lay.tile))
        del q, k, d
    tmax = torch.cat(tms, 0)  # [S * B, H, M, M_KV]: every batch element of every seed is a sample
    del tms
    cal = Layer.__new__(Layer)
    cal.__dict__.update(lay.__dict__)
    cal.tmax = tmax
    pts = cal.fixed_k_points(targets)
    return cal, pts


# --------------------------------------------------------------------------------------------
# rocprofv3 output -> the summaries under profiles/
# --------------------------------------------------------------------------------------------


def _csv_rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _forward_production(name: str) -> bool:
    """A production forward instance (no diagnostics, not the tile-maximum pass):
    bsfa_fwd_pipe_kernel<CAUSAL, DIAG_OUT=false, HEADPAIR, RAGGED> or
    bsfa_fwd_pair_kernel<D, BM, BN, CAUSAL, DIAG_OUT=false, MAXONLY=false, ...>."""
    for kernel, flags in ((PIPE_KERNEL, (1,)), (FWD_KERNEL, (4, 5))):
        if kernel + "<" in name:
            args = [a.strip() for a in name.split(kernel + "<", 1)[1].split(">", 1)[0].split(",")]
            return all(args[f] == "false" for f in flags)
    return False


def _points_of(dispatches, steps, n_points):
    """The last ``steps`` x ``n_points`` forward dispatches (launch order), grouped by point."""
    dispatches = sorted(dispatches)
    if len(dispatches) < steps * n_points:
        raise SystemExit(f"found {len(dispatches)} forward dispatches, expected at least {steps * n_points}")
    timed = dispatches[-steps * n_points:]
    return [timed[p::n_points] for p in range(n_points)]


def summarize_trace(directory, steps, names):
    """Steady-state (timed-step) forward dispatches of a --kernel-trace run, per point."""
    files = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {directory}")
    disp = []
    for row in _csv_rows(files[0]):
        name = _col(row, "Kernel_Name")
        if _forward_production(name):
            t0, t1 = int(_col(row, "Start_Timestamp")), int(_col(row, "End_Timestamp"))
            disp.append((t0, (t1 - t0) * 1e-6, int(_col(row, "Dispatch_Id"))))
    groups = _points_of(disp, steps, len(names))
    pts = []
    for nm, g in zip(names, groups):
        ms = [d for _, d, _ in g]
        pts.append({"point": nm, "dispatches": len(ms), "ms_mean": float(np.mean(ms)),
                    "ms_min": float(np.min(ms)), "ms_max": float(np.max(ms))})
    step_ms = sum(p["ms_mean"] for p in pts)
    return {"file": os.path.relpath(files[0], directory), "points": pts, "forward_ms_per_step": step_ms,
            "forward_ms_mean": step_ms / len(pts)}


def summarize_counters(directories, steps, names, copy_bytes=1 << 30):
    """Per-point means of every counter in the --pmc runs under ``directories``
    (timed-step dispatches of the production forward kernel), plus the scale
    factors that the plain 1 GiB copy of --traffic-probe gives FETCH_SIZE,
    WRITE_SIZE and TCC_READ_SECTORS_sum."""
    per_point = {nm: {} for nm in names}
    probe = {}
    for d in directories:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}  # dispatch -> {counter: value}
        kname = {}
        dur = {}
        for row in _csv_rows(files[0]):
            did = int(_col(row, "Dispatch_Id"))
            kname[did] = _col(row, "Kernel_Name")
            if "Start_Timestamp" in row and "End_Timestamp" in row:
                dur[did] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
            c = _col(row, "Counter_Name")
            vals.setdefault(did, {})
            vals[did][c] = vals[did].get(c, 0.0) + float(_col(row, "Counter_Value"))
        fwd = [did for did in vals if _forward_production(kname[did])]
        for nm, g in zip(names, _points_of(fwd, steps, len(names))):
            for c in vals[g[0]]:
                per_point[nm][c] = float(np.mean([vals[did][c] for did in g]))
            if "GRBM_GUI_ACTIVE" in vals[g[0]] and all(did in dur for did in g):
                # GRBM_GUI_ACTIVE is summed over the 8 XCDs; the duration is the
                # profiled dispatch's, so this is a lower bound of the clock
                per_point[nm]["clock_ghz"] = float(np.mean([vals[did]["GRBM_GUI_ACTIVE"] / 8 / dur[did] / 1e9
                                                            for did in g]))
        copies = [did for did in vals if "copyBuffer" in kname[did] or "copy" in kname[did].lower()]
        for did in copies:
            for c, v in vals[did].items():
                if v > probe.get(c, 0.0):
                    probe[c] = v
    scale = {}
    if "FETCH_SIZE" in probe:
        scale["FETCH_SIZE"] = copy_bytes / (probe["FETCH_SIZE"] * 1024)
    if "WRITE_SIZE" in probe:
        scale["WRITE_SIZE"] = copy_bytes / (probe["WRITE_SIZE"] * 1024)
    if "TCC_READ_SECTORS_sum" in probe:
        scale["TCC_READ_SECTORS_sum"] = copy_bytes / (probe["TCC_READ_SECTORS_sum"] * 32)
    out = {"kernel_sha256": kernel_source_hash(), "copy_probe": probe, "scale": scale, "points": []}
    for nm in names:
        c = per_point[nm]
        p = {"point": nm, "counters": c}
        if "FETCH_SIZE" in c and "FETCH_SIZE" in scale:
            p["hbm_read_bytes"] = c["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
        if "WRITE_SIZE" in c and "WRITE_SIZE" in scale:
            p["hbm_write_bytes"] = c["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
        if "TCC_READ_SECTORS_sum" in c:
            p["l2_read_bytes"] = c["TCC_READ_SECTORS_sum"] * 32 * scale.get("TCC_READ_SECTORS_sum", 1.0)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "SQ_BUSY_CU_CYCLES" in c:
            p["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * c["SQ_BUSY_CU_CYCLES"])
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            p["mfma_coexec"] = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"]
        if "SQ_WAIT_ANY" in c and "SQ_WAVE_CYCLES" in c:
            p["waves_waiting"] = c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]
        if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c:
            p["valu_per_mfma"] = c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]
        if "clock_ghz" in c:
            p["clock_ghz"] = c["clock_ghz"]
        out["points"].append(p)
    return out


def roofline_points(points, counters):
    """Per-point roofline of the forward kernel; counters (profiles/) when current."""
    cpts = {p["point"]: p for p in (counters or {}).get("points", [])}
    rows = []
    for pt in points:
        r = {"target": pt["target"], "achieved": pt["executed_tflops"], "frac": pt["frac_of_peak"],
             "ms_mean": pt["ms_mean"], "v_tile_loads": pt.get("v_tile_loads"), "k_tile_loads": pt.get("k_tile_loads"),
             "stream_read_bytes": pt.get("stream_read_bytes")}
        c = cpts.get(f"{pt['target']:g}")
        if c:
            for key in ("mfma_busy", "mfma_coexec", "waves_waiting", "valu_per_mfma", "l2_read_bytes", "clock_ghz"):
                if key in c:
                    r[key] = c[key]
            if "hbm_read_bytes" in c and "hbm_write_bytes" in c:
                r["hbm_bytes"] = c["hbm_read_bytes"] + c["hbm_write_bytes"]
                r["hbm_gbps"] = r["hbm_bytes"] / (pt["ms_mean"] * 1e-3) / 1e9
            if "l2_read_bytes" in c and pt.get("stream_read_bytes"):
                r["l2_read_over_stream"] = c["l2_read_bytes"] / pt["stream_read_bytes"]
        rows.append(r)
    return rows


# --------------------------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="llama32k",
                    help="the headline layer (its dense point + its skip targets); llama32k by default")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="CPU-oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the 8K, DiT and 128K legs")
    ap.add_argument("--no-held-out", action="store_true", help="skip the held-out calibration")
    ap.add_argument("--no-gate-study", action="store_true", help="skip the gap-gate comparison")
    ap.add_argument("--no-tile-study", action="store_true", help="skip the 128 x 64 tile comparison")
    ap.add_argument("--no-cold-cache", action="store_true", help="skip the cold-cache timing of the sweep")
    ap.add_argument("--profile", action="store_true",
                    help="headline sweep only (no studies, legs or CPU baseline): the profiled command")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run one plain 1 GiB device copy, whose counters scale the kernel's")
    ap.add_argument("--summarize-trace", metavar="DIR", help="summarise a rocprofv3 --kernel-trace run of --profile")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+",
                    help="summarise rocprofv3 --pmc runs of --profile into the per-point counter JSON")
    ap.add_argument("--names", nargs="+", default=["0", "0.6", "0.8", "0.9"],
                    help="sweep points of the profiled run, in launch order (summaries only)")
    args = ap.parse_args()
    names = args.names
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.steps, names), indent=1))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters, args.steps, names), indent=1))
        return

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
    if args.profile:
        args.no_cpu_baseline = args.no_legs = args.no_held_out = True
        args.no_gate_study = args.no_tile_study = args.no_cold_cache = True

    # ---- the headline workload -------------------------------------------------
    lay = Layer(args.workload, args.seed, torch, bb, wl, acc)
    w = lay.w
    targets = [0.0] + [t for t in w.skip_targets if t > 0]
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
    step_flops = sum(pt["executed_flops"] for pt in points)
    sum_dur = sum(pt["ms_mean"] for pt in points)
    value = step_flops / (step_ms * 1e-3) / 1e12
    achieved = step_flops / (sum_dur * 1e-3) / 1e12  # algorithmic FLOPs per launch / mean launch time
    if not args.profile:
        for pt in points:
            pt.update(lay.tile_loads(pt))
    counters = measured_counters() if w.name == "llama32k" else None

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
            "kernel": f"{PIPE_KERNEL if w.block == 128 and w.head_dim == 128 else FWD_KERNEL} (production instance: "
                      f"{w.block} x {w.block} tiles, d = {w.head_dim}, "
                      f"{'causal' if w.causal else 'bidirectional'}, "
                      f"{'head pairs' if w.group % 2 == 0 else 'block pairs'})",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": (float(np.mean([p["hbm_read_bytes"] + p["hbm_write_bytes"] for p in counters["points"]]))
                        if counters and all("hbm_read_bytes" in p and "hbm_write_bytes" in p
                                            for p in counters["points"]) else None),
            "per_launch": "executed FLOPs of a launch (QK^T on every computed tile + P.V on kept tiles, "
                          "2 x 128 x 128 x 128 each) / its mean duration (HIP events on the launch stream)",
            "counters": ("profiles/" + COUNTERS_FILE + " (taken on the current kernel sources)") if counters
            else "none current for this kernel source",
            "points": roofline_points(points, counters),
        },
    }
    props = torch.cuda.get_device_properties(0)
    res["device"] = {"name": props.name, "compute_units": props.multi_processor_count,
                     "arch": getattr(props, "gcnArchName", None)}
    if args.profile:
        print(json.dumps(res), flush=True)
        return
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
        lay.measure(study, max(3, args.steps // 4), 1, settle_ms=LEG_SETTLE_MS)
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
    if not args.no_tile_study:
        sq = [dict(pt) for pt in points]
        for pt in sq:
            pt.update(lay.errors_vs(ref_out, ref_lse, pt))
        tmax_sq = lay.tmax
        lay.set_tile((128, 64))
        rect = lay.fixed_k_points(targets)
        lay.measure(rect, max(3, args.steps // 4), 1, settle_ms=LEG_SETTLE_MS)
        for pt in rect:
            pt.update(lay.errors_vs(ref_out, ref_lse, pt))
            pt["speedup_vs_dense"] = points[0]["ms_mean"] / pt["ms_mean"]
        res["tile_study"] = {
            "workload": w.name,
            "reference": "the 128 x 128 kernel at threshold -inf; speedup_vs_dense relative to it",
            "tiles": {"128x128": public(sq), "128x64": public(rect)},
        }
        lay.set_tile((w.block, w.block), tmax=tmax_sq)
        del tmax_sq
    if not (args.no_gate_study and args.no_tile_study):
        del ref_out

    # ---- held-out calibration ------------------------------------------------------
    if not args.no_held_out and w.name == "llama32k":
        cal, hpts = held_out(lay, [t for t in targets if t > 0], (1, 2), torch, bb, wl)
        cal.measure(hpts, max(3, args.steps // 4), 1, settle_ms=LEG_SETTLE_MS)
        dense_ms = points[0]["ms_mean"]
        for pt in hpts:
            pt.update(cal.density_errors(pt))
            pt["speedup_vs_dense"] = dense_ms / pt["ms_mean"]
            pt["flop_ratio"] = 2.0 / (2.0 - pt["skip_fraction"])
            pt["speedup_floor"] = 0.8 * pt["flop_ratio"]
        self_cal = {pt["target"]: pt for pt in points}
        for pt in points[1:]:
            pt.update(lay.density_errors(pt))
        res["held_out"] = {
            "workload": w.name,
            "calibration": "tile maxima of seeds 1 and 2 (the batch axis of bsfa_calibrate as the samples, "
                           "thresholds averaged), evaluated on seed 0",
            "density": "kept / computed tiles per (head, query block) row, designed = (min(k, n_i) + 1) / (n_i + 1)",
            "points": public(hpts),
            "self_calibrated": [{kk: self_cal[pt["target"]][kk] for kk in
                                 ("target", "k", "skip_fraction", "designed_skip_fraction",
                                  "row_density_error_mean", "row_density_error_std", "head_density_error_std")}
                                for pt in hpts],
        }
        del cal
    cpu_layers = {w.name: (lay, points)}

    # ---- the other configurations ---------------------------------------------------
    if not args.no_legs:
        res["legs"] = {}
        for name in [n for n in ("llama8k", "dit32k", "gqa128k") if n != w.name]:
            leg_lay, leg_pts, leg = run_leg(name, args.seed, args.steps if name == "llama8k"
                                            else max(3, args.steps // 4), torch, bb, wl, acc)
            res["legs"][name] = leg
            if name in ("llama8k", "dit32k"):
                cpu_layers[name] = (leg_lay, leg_pts)
            else:
                del leg_lay
            torch.cuda.empty_cache()
        if "gqa128k" in res["legs"]:
            res["long_context"] = res["legs"]["gqa128k"]

    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline, sample budget ~{args.cpu_seconds:.0f} s")
        tiny = Layer("tiny", args.seed, torch, bb, wl, acc)
        cpu_layers["tiny"] = (tiny, tiny.fixed_k_points(list(tiny.w.skip_targets)))
        if "llama8k" not in cpu_layers:
            l8 = Layer("llama8k", args.seed, torch, bb, wl, acc)
            cpu_layers["llama8k"] = (l8, l8.fixed_k_points(list(l8.w.skip_targets)))
        for name in ("tiny", "llama8k"):
            cl, cp = cpu_layers[name]
            cpu_layers[name] = (cl, [p for p in cp if p["target"] > 0])
        order = {n: cpu_layers[n] for n in ("tiny", "llama8k", "llama32k", "dit32k") if n in cpu_layers}
        res["cpu_baseline"] = cpu_baseline(order, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
