"""Benchmark: fused Ulysses-shard attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--seq-len S]
                    [--no-cpu] [--no-split] [--no-io] [--no-long] [--no-moe] [--cpu-seconds T]
                    [--rounds R]
                    [--cpu-all] [--full-limit T] [--calibrate-copy MIB]

One step = one attn_ulysses_fused call over the whole workload (attention over
the rank's Hl heads, each output tile stored into its post-All-to-All slot).
Workloads with fewer query tiles than CUs (ua.key_split > 1) run the calls
with a workspace instead (attn_ulysses_fused_ws / attn_serial_ws: each query
tile's keys split over several workgroups); detail.unsplit then times the
plain call beside them, and --no-split times the plain calls throughout.
Inputs are seeded synthetic bf16 tensors already resident in HBM when timing
starts.  Every timing follows W counted warm-up launches and at least 200 ms
of launches in all, and is bracketed by two traced calls that read the shader
clock; a timing whose clock drifts, or whose per-launch times spread, by more
than the pages' +-2% DVFS envelope (review page, Fig. 11 caption) is flagged.
Prints ONE JSON line:
  value     attention TFLOP/s of the fused call, counting 4*S^2*d per
            (batch, local head) (QK^T + PV, non-causal);
  roofline  the fused attention kernel against the bf16 MFMA peak, from HIP
            events around every launch on the launch stream;
  detail    fused / serial (attention + separate permute) / attention-alone /
            permute-alone / store-only-epilogue times (medians over
            interleaved rounds), the residual (fused - alone) / alone, the
            permute's and the epilogue layout's HBM rates, and from one traced
            fused call the per-work-unit epilogue store spans and the shader
            clock the kernel ran at; with both exchanges (detail.io): the
            call that reads Q, K, V in place from the sequence-partitioned
            inputs vs three separate gathers + attention + permute;
  detail.long_configs  the same figures (timed region, medians, TFLOP/s and
            fraction of the bf16 peak, traced clock and DVFS flag) for each
            long-sequence workload: video_dit, dit_long and mixed;
  detail.moe  the MoE expert path of one expert-parallel rank (DeepSeek-style
            layer shape, balanced and skewed routing): the fused call in its
            persistent form (one launch, a device tile queue) under the
            Expert-Wave and the interleaved schedule, the same calls as one
            launch per wave, and the serial form (experts, then a separate
            Combine scatter) and its halves;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + % bf16 MFMA peak; fused vs serial attn+A2A-permute time"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEFAULT_WORKLOAD = "video_dit"
KERNEL_SOURCE = os.path.join(ROOT, "comm_fusion_amd", "csrc", "ua_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_video_dit_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seq-len", type=int, default=0, metavar="S",
                    help="time the workload's heads and head dim at another sequence length "
                         "(a multiple of its P); the CPU baseline and counter figures then do not apply")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-split", action="store_true",
                    help="time the calls without a workspace even where a key split would run")
    ap.add_argument("--no-io", action="store_true",
                    help="skip the timings with the pre-attention exchange (detail.io)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the other long-sequence workloads (detail.long_configs)")
    ap.add_argument("--no-moe", action="store_true",
                    help="skip the MoE expert path with the fused Combine (detail.moe)")
    ap.add_argument("--moe-wave", type=int, default=8, metavar="G",
                    help="local experts per wave in the timed MoE calls")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--rounds", type=int, default=5,
                    help="interleaved rounds of fused / serial / alone / permute timing")
    ap.add_argument("--cpu-all", action="store_true",
                    help="instead of the benchmark: time the fp64 oracle on every workload "
                         "(parity-check rows, and all rows where that takes under --full-limit s)")
    ap.add_argument("--full-limit", type=float, default=120.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device-to-device copy of MIB MiB (a known-size "
                         "kernel for scaling HBM byte counters under rocprofv3 --pmc)")
    return ap.parse_args()


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def time_launches(fn, steps, warmup):
    """Per-launch durations (ms) from events recorded between back-to-back
    launches on the current stream, plus the total (ms) over the K launches."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = _events(steps + 1)
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[steps]), wall


def interleaved(fns, rounds, reps):
    """Per-launch durations (ms) of several callables, timed in interleaved
    rounds so that clock ramps and thermal drift hit all of them alike."""
    import torch
    out = {k: [] for k in fns}
    for _ in range(rounds):
        for name, fn in fns.items():
            ev = _events(reps + 1)
            ev[0].record()
            for i in range(reps):
                fn()
                ev[i + 1].record()
            torch.cuda.synchronize()
            out[name] += [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return out


def code_text(text: str) -> str:
    """C++ source with comments, trailing spaces and blank lines removed
    (string and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def source_digest() -> str:
    """sha256[:16] of the attention kernel source's code (code_text): an edit
    of comments alone keeps the committed counter figures valid, any change to
    the code voids them."""
    with open(KERNEL_SOURCE) as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, only if it
    was taken on this workload and on the current kernel code; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("code_sha256_16") != source_digest() or t.get("workload_name") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def _oracle_sample(w, target_s, probe_dt_per_row):
    """The rows the parity check uses for this workload, extended with further
    distinct seeded rows until the sample is about target_s of oracle work."""
    from ua_inputs import sampled_rows
    rows = sampled_rows(dataclasses.replace(w, sampled=True))
    want = int(target_s / max(probe_dt_per_row, 1e-9))
    total = w.B * w.Hl * w.S
    if want > len(rows):
        rng = np.random.default_rng(w.seed + 2000)
        seen = {tuple(r) for r in rows.tolist()}
        extra = []
        for flat in rng.permutation(total)[: min(total, 4 * want)]:
            b, rem = divmod(int(flat), w.Hl * w.S)
            h, srow = divmod(rem, w.S)
            if (b, h, srow) not in seen:
                extra.append((b, h, srow))
                if len(rows) + len(extra) >= want:
                    break
        if extra:
            rows = np.concatenate([rows, np.asarray(extra, dtype=np.int64)])
    return rows[: max(want, 1)] if want < len(rows) else rows


def cpu_baseline(w, Q, K, V, target_s):
    """The fp64 oracle as it stands, on the host cores, over a bounded sample of
    this workload's query rows (rows per second scaled to TFLOP/s)."""
    import oracle
    scale = 1.0 / math.sqrt(w.d)
    threads = oracle.max_threads()
    flops_per_row = 4.0 * w.S * w.d
    # calibrate on a small batch, then time a sample sized for ~target_s
    from ua_inputs import sampled_rows
    probe = sampled_rows(dataclasses.replace(w, sampled=True))[: max(4 * threads, 16)]
    t0 = time.perf_counter()
    oracle.attn_rows(Q, K, V, scale, probe)
    dt_row = max(time.perf_counter() - t0, 1e-6) / len(probe)
    sample = _oracle_sample(w, target_s, dt_row)
    t0 = time.perf_counter()
    oracle.attn_rows(Q, K, V, scale, sample)
    dt = time.perf_counter() - t0
    return {
        "value": round(flops_per_row * len(sample) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d query rows (of %d x %d; the parity-check rows first, then further seeded "
                  "rows) of the %s workload, full %d-key softmax each, fp64, %.1f s"
                  % (len(sample), w.B * w.Hl, w.S, w.name, w.S, dt),
        "rows_per_s": round(len(sample) / dt, 1),
    }


def cpu_all(full_limit_s: float) -> dict:
    """Oracle timings on the host for every workload: the parity check's
    sampled rows, and all rows where that fits full_limit_s (else the full
    time extrapolated from the per-row time, and marked so)."""
    import oracle
    from ua_inputs import WORKLOADS, sampled_rows, workload_qkv
    threads = oracle.max_threads()
    res = []
    for name, w in WORKLOADS.items():
        Q, K, V = workload_qkv(w)
        scale = 1.0 / math.sqrt(w.d)
        rows = sampled_rows(dataclasses.replace(w, sampled=True))
        t0 = time.perf_counter()
        oracle.attn_rows(Q, K, V, scale, rows)
        dt = time.perf_counter() - t0
        per_row = dt / len(rows)
        total_rows = w.B * w.Hl * w.S
        est = per_row * total_rows
        entry = {"workload": name, "check_rows": len(rows), "check_s": round(dt, 3),
                 "rows_per_s": round(len(rows) / dt, 1),
                 "gflops": round(4.0 * w.S * w.d * len(rows) / dt / 1e9, 2),
                 "full_rows": total_rows}
        if est <= full_limit_s:
            t0 = time.perf_counter()
            oracle.attn_all(Q, K, V, scale)
            entry["full_s"] = round(time.perf_counter() - t0, 3)
        else:
            entry["full_s_extrapolated"] = round(est, 1)
        res.append(entry)
        print(json.dumps(entry), file=sys.stderr, flush=True)
    return {"kind": "oracle", "cores": threads, "timings": res}


def traced_call(ua, torch, q, k, v, w, dest, workspace=None) -> dict:
    """One call of the measurement build of the timed launch (with the
    workspace of a split launch, so its clock is read on that launch):
    per-workgroup epilogue store spans (from every wave's rows ready to every
    wave's stores complete) and the shader clock (cycles over the 100 MHz
    constant clock)."""
    n = ua.work_units(w.B, w.S, w.H, w.d, w.P, workspace=workspace is not None)
    trace = torch.zeros(4 * n, dtype=torch.int64, device=q.device)
    ua.attn_ulysses_fused_trace(q, k, v, w.rank, w.P, dest, trace, workspace=workspace)
    torch.cuda.synchronize()
    return trace_stats(trace.cpu().numpy().reshape(n, 4), w.out_bytes)


def trace_stats(records, out_bytes) -> dict:
    """Statistics of a measurement build's records, one row per workgroup:
    [start, rows ready, stores complete] on the 100 MHz constant clock, then
    shader cycles from start to stores complete.  out_bytes: the bytes the
    launch's epilogues store in all."""
    t = np.asarray(records, dtype=np.float64)
    n = len(t)
    # a split launch's parts merged elsewhere store nothing: [1] == [2]
    span_us = (t[:, 2] - t[:, 1]) / 100.0          # 100 MHz ticks -> us
    life_us = (t[:, 2] - t[:, 0]) / 100.0
    ok = span_us > 0                                # the workgroups that stored rows
    unit_bytes = out_bytes / max(int(ok.sum()), 1)  # mean bytes a storing workgroup stores
    unit_mhz = t[:, 3] / np.maximum(life_us, 1e-3)   # cycles per us = MHz
    sp = span_us[ok] if ok.any() else span_us
    return {
        "trace_work_units": n,
        "epilogue_span_us_mean": round(float(sp.mean()), 3),
        "epilogue_span_us_p90": round(float(np.percentile(sp, 90)), 3),
        "epilogue_unit_GBs_mean": round(float((unit_bytes / (span_us[ok] * 1e-6)).mean() / 1e9), 1) if ok.any() else None,
        "epilogue_share_of_unit_time": round(float(span_us.sum() / life_us.sum()), 4),
        "sclk_mhz_trace": round(float(t[:, 3].sum() / (life_us.sum() * 1e-6) / 1e6), 1),
        # spread of the per-unit clocks (DVFS within the launch)
        "sclk_mhz_trace_p10_p90": [round(float(np.percentile(unit_mhz, q)), 1) for q in (10, 90)],
    }


LONG_CONFIGS = ("video_dit", "dit_long", "mixed")   # the long-sequence workloads the target covers
WARM_MS = 1000.0         # launches run for at least this long before any timing
DVFS_BAND = 0.02         # the pages' +-2% clock envelope (Fig. 11 caption)


def warm_up(fn, count, min_ms):
    """count launches, then further batches until at least min_ms of wall
    time has passed since the first, so that timing starts at the clock the
    GPU holds under this load rather than during its ramp."""
    import torch
    t0 = time.perf_counter()
    for _ in range(count):
        fn()
    torch.cuda.synchronize()
    batch = 1
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        t1 = time.perf_counter()
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t1) * 1e3 / batch
        batch = max(1, min(1000, int(20.0 / max(per, 1e-3))))


def clock_flags(sclk_before, sclk_after, per_launch):
    """DVFS check of one timing: the traced shader clock before and after it,
    and the spread of the per-launch times (half the p10-p90 range over the
    median); flagged when either leaves the +-2% band."""
    mean = 0.5 * (sclk_before + sclk_after)
    drift = (sclk_after - sclk_before) / mean if mean > 0 else None
    med = float(np.median(per_launch))
    spread = 0.5 * (np.percentile(per_launch, 90) - np.percentile(per_launch, 10)) / med
    flag = (drift is None) or abs(drift) > DVFS_BAND or spread > DVFS_BAND
    return {"sclk_mhz_before": round(sclk_before, 1), "sclk_mhz_after": round(sclk_after, 1),
            "sclk_drift_pct": round(100 * drift, 2) if drift is not None else None,
            "launch_spread_pct": round(100 * float(spread), 2),
            "outside_dvfs_band": bool(flag)}


class Case:
    """One workload on the GPU: inputs resident in HBM, the destination
    prefilled with the sentinel, and the callables that are timed."""

    def __init__(self, ua, torch, w, dev, use_split=True, with_io=True):
        from ua_inputs import SENTINEL_BITS, workload_qkv
        self.w = w
        self.ua = ua
        self.torch = torch
        Q, K, V = workload_qkv(w)
        self.host = (Q, K, V)

        def up(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

        q, k, v = up(Q), up(K), up(V)
        self.q, self.k, self.v = q, k, v
        n_dest = w.B * w.S * w.H * w.d
        dest = torch.full((n_dest,), SENTINEL_BITS, dtype=torch.int16, device=dev).view(torch.bfloat16)
        o_local = torch.empty_like(q)
        self.scratch_dest = torch.empty_like(dest)
        self.n_split = ua.key_split(w.B, w.S, w.H, w.d, w.P) if use_split else 1
        plain = lambda: ua.attn_ulysses_fused(q, k, v, w.rank, w.P, dest)  # noqa: E731
        if self.n_split > 1:
            ws = ua.new_workspace(w.B, w.S, w.H, w.d, w.P, dev)
            self.ws = ws
            fused = lambda: ua.attn_ulysses_fused_ws(q, k, v, w.rank, w.P, dest, ws)  # noqa: E731
            alone = lambda: ua.attn_serial_ws(q, k, v, w.rank, w.P, o_local, ws)      # noqa: E731
        else:
            fused = plain
            alone = lambda: ua.attn_serial(q, k, v, w.rank, w.P, o_local)  # noqa: E731
        perm = lambda: ua.a2a_permute(o_local, w.rank, w.P, dest)           # noqa: E731
        sd = self.scratch_dest
        store_only = lambda: ua.epilogue_store_only(w.B, w.S, w.H, w.d, w.rank, w.P, sd)  # noqa: E731

        def serial():
            alone()
            perm()

        self.fused = fused
        self.fns = {"fused": fused, "serial": serial, "alone": alone, "perm": perm, "store_only": store_only}
        if self.n_split > 1:
            self.fns["unsplit"] = plain
        if with_io:
            # Sequence-partitioned inputs [B][P][S/P][H][d] holding the rank's
            # Q, K, V in its head slots (the other heads are never read).
            lo, hi = w.rank * w.Hl, (w.rank + 1) * w.Hl
            xs = []
            for t in (q, k, v):
                X = torch.zeros((w.B, w.S, w.H, w.d), dtype=torch.bfloat16, device=dev)
                X[:, :, lo:hi] = t.view(w.B, w.S, w.Hl, w.d)
                xs.append(X)
            g_loc = [torch.empty_like(q) for _ in range(3)]
            if self.n_split > 1:
                self.fns["fused_io"] = lambda: ua.attn_ulysses_fused_io_ws(xs[0], xs[1], xs[2], w.rank, w.P, dest, ws)
            else:
                self.fns["fused_io"] = lambda: ua.attn_ulysses_fused_io(xs[0], xs[1], xs[2], w.rank, w.P, dest)
            self.fns["gather"] = lambda: ua.a2a_gather(xs[0], w.rank, w.P, g_loc[0])

            def serial_io():
                for X, L in zip(xs, g_loc):
                    ua.a2a_gather(X, w.rank, w.P, L)
                if self.n_split > 1:
                    ua.attn_serial_ws(g_loc[0], g_loc[1], g_loc[2], w.rank, w.P, o_local, ws)
                else:
                    ua.attn_serial(g_loc[0], g_loc[1], g_loc[2], w.rank, w.P, o_local)
                perm()
            self.fns["serial_io"] = serial_io
        torch.cuda.synchronize()

    def traced(self):
        return traced_call(self.ua, self.torch, self.q, self.k, self.v, self.w, self.scratch_dest,
                           self.ws if self.n_split > 1 else None)

    def measure(self, steps, warmup, rounds):
        """Warm-up (counted and timed), the traced clock, K fused launches back
        to back (the timed region), interleaved rounds of every callable, and
        the traced clock again."""
        w = self.w
        warm_up(self.fused, warmup, WARM_MS)
        before = self.traced()
        per, total_ms, wall_ms = time_launches(self.fused, steps, 0)
        # about 100 ms of each callable per round (at most 500 launches)
        reps = max(2, min(500, int(100.0 / max(float(np.mean(per)), 1e-3)) + 1))
        cmp = interleaved(self.fns, rounds, reps)
        after = self.traced()
        med = lambda x: float(np.median(x))  # noqa: E731
        t_f, t_s, t_a = med(cmp["fused"]), med(cmp["serial"]), med(cmp["alone"])
        ms_step = total_ms / steps
        r = {
            "per": per, "total_ms": total_ms, "wall_ms": wall_ms, "cmp": cmp, "before": before, "after": after,
            "ms_step": ms_step,
            "value": w.flops / (ms_step * 1e-3) / 1e12,
            "launch_ms": float(np.mean(per)),
            "t_f": t_f, "t_s": t_s, "t_a": t_a, "t_p": med(cmp["perm"]),
        }
        r["clock"] = clock_flags(before["sclk_mhz_trace"], after["sclk_mhz_trace"], per)
        return r

    def summary(self, r):
        """The per-workload entry of detail.long_configs."""
        w = self.w
        tf = lambda t: round(w.flops / (t * 1e-3) / 1e12, 2)  # noqa: E731
        out = {
            "workload": w.name, "B": w.B, "S": w.S, "Hl": w.Hl, "d": w.d, "flops": w.flops,
            "key_split": self.n_split,
            "timed_region_ms_per_step": round(r["ms_step"], 4),
            "timed_region_TFLOPs": round(r["value"], 2),
            "frac": round(r["value"] / PEAK_BF16_TFLOPS, 4),
            "fused_ms_median": round(r["t_f"], 4),
            "fused_TFLOPs_median": tf(r["t_f"]),
            "frac_median": round(w.flops / (r["t_f"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "serial_ms_median": round(r["t_s"], 4),
            "attn_alone_ms_median": round(r["t_a"], 4),
            "permute_ms_median": round(r["t_p"], 4),
            "residual_fused_vs_alone": round((r["t_f"] - r["t_a"]) / r["t_a"], 4),
            "speedup_serial_over_fused": round(r["t_s"] / r["t_f"], 4),
            **r["clock"],
        }
        # the fraction of the peak at the clock the timed launch itself ran at
        # (its measurement build, traced before and after the timing)
        sclk = 0.5 * (r["clock"]["sclk_mhz_before"] + r["clock"]["sclk_mhz_after"])
        if sclk > 0:
            out["pct_bf16_peak_at_traced_clock"] = round(100 * r["value"] / (PEAK_BF16_TFLOPS * sclk / 2400.0), 2)
        if "unsplit" in r["cmp"]:
            out["unsplit_fused_ms_median"] = round(float(np.median(r["cmp"]["unsplit"])), 4)
        return out


MOE_CONFIGS = ("moe_ds", "moe_ds_skewed")


class MoeCase:
    """The MoE expert path of one rank at full size: tokens, routing and this
    rank's expert weights resident in HBM, the Combine buffer, and the timed
    callables (both schedules of the fused call in the persistent form and
    as one launch per wave, the serial form and its halves)."""

    def __init__(self, ua, torch, w, dev, G, weights=None):
        from moe_inputs import moe_rank_weights, moe_tokens
        self.w = w
        self.G = G
        x, idx, tw = moe_tokens(w)
        self.weights = weights if weights is not None else moe_rank_weights(w, w.rank)
        W1, W2 = self.weights
        off, slots = ua.moe_recv_layout(idx, w.rank, w.P, w.hidden, w.inter, w.E)
        self.N = int(off[-1])
        self.rows_per_expert = np.diff(off)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        dx, dW1, dW2 = up(x), up(W1), up(W2)
        dtw = torch.from_numpy(tw).to(dev)
        drs = torch.from_numpy(slots.astype(np.int32)).to(dev)
        act = torch.empty(self.N * w.inter, dtype=torch.bfloat16, device=dev)
        comb = torch.empty(w.P * w.T * w.k * w.hidden, dtype=torch.bfloat16, device=dev)
        y = torch.empty(self.N * w.hidden, dtype=torch.bfloat16, device=dev)
        ws = ua.new_moe_workspace(dx, dW1, dtw, w.P, w.E)
        self.ws = ws

        def fused(schedule):
            return lambda: ua.moe_experts_combine_ws(dx, drs, dtw, off, dW1, dW2, w.P, w.E, comb, act, ws,
                                                     schedule=schedule, experts_per_wave=G)

        def per_wave(schedule):
            return lambda: ua.moe_experts_combine(dx, drs, dtw, off, dW1, dW2, w.P, w.E, comb, act,
                                                  schedule=schedule, experts_per_wave=G)
        alone = lambda: ua.moe_experts_local_ws(dx, drs, dtw, off, dW1, dW2, w.P, w.E, y, act, ws,  # noqa: E731
                                                experts_per_wave=G)
        scatter = lambda: ua.moe_combine_scatter(y, drs, self.N, w.P, w.T, w.hidden, w.inter, w.E, w.k,  # noqa: E731
                                                 comb)

        def serial():
            alone()
            scatter()

        self.fns = {"interleaved": fused(ua.MOE_INTERLEAVED), "expert_wave": fused(ua.MOE_EXPERT_WAVE),
                    "per_wave_interleaved": per_wave(ua.MOE_INTERLEAVED),
                    "per_wave_expert_wave": per_wave(ua.MOE_EXPERT_WAVE),
                    "serial": serial, "experts_alone": alone, "scatter": scatter}
        torch.cuda.synchronize()

    def measure(self, warmup, rounds):
        import torch
        w = self.w
        warm_up(self.fns["interleaved"], warmup, WARM_MS)
        warm_up(self.fns["expert_wave"], 1, 50.0)
        per = interleaved({"interleaved": self.fns["interleaved"]}, 1, 5)["interleaved"]
        reps = max(2, min(500, int(100.0 / max(float(np.mean(per)), 1e-3)) + 1))
        cmp = interleaved(self.fns, rounds, reps)
        med = {k: float(np.median(v)) for k, v in cmp.items()}
        flops = 6 * self.N * w.hidden * w.inter    # Linear-1 (2*inter outputs) + Linear-2, 2 flop per MAC
        tf = lambda t: round(flops / (t * 1e-3) / 1e12, 2)  # noqa: E731
        return {
            "workload": w.name, "routing": w.routing, "P": w.P, "rank": w.rank, "T": w.T, "hidden": w.hidden,
            "inter": w.inter, "E": w.E, "k": w.k, "rows_N": self.N,
            "rows_per_expert_min_max": [int(self.rows_per_expert.min()), int(self.rows_per_expert.max())],
            "experts_per_wave": self.G, "flops": flops, "form": "persistent",
            "interleaved_ms_median": round(med["interleaved"], 4),
            "expert_wave_ms_median": round(med["expert_wave"], 4),
            "per_wave_launches_interleaved_ms_median": round(med["per_wave_interleaved"], 4),
            "per_wave_launches_expert_wave_ms_median": round(med["per_wave_expert_wave"], 4),
            "speedup_persistent_over_per_wave_launches": round(med["per_wave_interleaved"] / med["interleaved"], 4),
            "bounded_waits_given_up": int(self.ws.view(torch.int32)[32]),
            "speedup_interleaved_over_expert_wave": round(med["expert_wave"] / med["interleaved"], 4),
            "serial_ms_median": round(med["serial"], 4),
            "experts_alone_ms_median": round(med["experts_alone"], 4),
            "scatter_ms_median": round(med["scatter"], 4),
            "residual_interleaved_vs_alone": round((med["interleaved"] - med["experts_alone"]) / med["experts_alone"], 4),
            "interleaved_TFLOPs": tf(med["interleaved"]),
            "frac": round(flops / (med["interleaved"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "combine_bytes": self.N * w.hidden * 2,
            "scatter_hbm_GBs": round(2 * self.N * w.hidden * 2 / (med["scatter"] * 1e-3) / 1e9, 1),
        }


def main():
    args = parse()
    if args.cpu_all:
        print(json.dumps(cpu_all(args.full_limit)), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path runs one Ulysses rank's share on "
              "one MI355X (the P ranks are P regions of its HBM); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import comm_fusion_amd as ua
    from ua_inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.seq_len:
        if args.seq_len % w.P:
            sys.exit("--seq-len must be a multiple of P = %d" % w.P)
        w = dataclasses.replace(w, name="%s_S%d" % (w.name, args.seq_len), S=args.seq_len, sampled=True)
        args.no_cpu = True
        args.no_long = True
        args.no_moe = True
    dev = torch.device("cuda:0")

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    case = Case(ua, torch, w, dev, use_split=not args.no_split, with_io=not args.no_io)
    n_split = case.n_split
    # The timed region: K fused steps back to back, after the warm-up; then
    # fused, serial (attention + separate permute), attention alone and
    # permute alone in interleaved rounds.
    r = case.measure(args.steps, args.warmup, args.rounds)
    per, cmp, tr = r["per"], r["cmp"], r["after"]
    ms_step, value, launch_ms = r["ms_step"], r["value"], r["launch_ms"]
    achieved = w.flops / (launch_ms * 1e-3) / 1e12
    med = lambda x: float(np.median(x))  # noqa: E731
    t_f, t_s, t_a, t_p = r["t_f"], r["t_s"], r["t_a"], r["t_p"]
    traffic = measured_traffic(w.name) if n_split == 1 else None
    unsplit = None
    if n_split > 1:
        t_u = med(cmp["unsplit"])
        unsplit = {"key_split": n_split, "stream_k_iters": ua.stream_k_iters(w.B, w.S, w.H, w.d, w.P),
                   "workspace_bytes": ua.workspace_bytes(w.B, w.S, w.H, w.d, w.P),
                   "unsplit_fused_ms_median": round(t_u, 4),
                   "unsplit_TFLOPs": round(w.flops / (t_u * 1e-3) / 1e12, 2),
                   "speedup_split_over_unsplit": round(t_u / t_f, 4),
                   "note": "the traced call (sclk, epilogue spans) is the split launch's measurement build"}
    io = None
    if not args.no_io:
        t_fio, t_sio, t_g = med(cmp["fused_io"]), med(cmp["serial_io"]), med(cmp["gather"])
        io = {"fused_io_ms_median": round(t_fio, 4),
              "serial_io_ms_median": round(t_sio, 4),
              "gather_ms_median": round(t_g, 4),
              "gather_hbm_GBs": round(2 * w.out_bytes / (t_g * 1e-3) / 1e9, 1),
              "speedup_serial_io_over_fused_io": round(t_sio / t_fio, 4),
              "residual_fused_io_vs_alone": round((t_fio - t_a) / t_a, 4),
              "fused_io_TFLOPs": round(w.flops / (t_fio * 1e-3) / 1e12, 2)}

    # The other long-sequence workloads, measured the same way (one entry
    # each; the headline workload's entry repeats its own figures).
    long_configs = None
    if not args.no_long:
        long_configs = {w.name: case.summary(r)} if w.name in LONG_CONFIGS else {}
        host = case.host
        del case
        torch.cuda.empty_cache()
        for name in LONG_CONFIGS:
            if name in long_configs:
                continue
            c = Case(ua, torch, WORKLOADS[name], dev, use_split=not args.no_split, with_io=False)
            long_configs[name] = c.summary(c.measure(args.steps, args.warmup, args.rounds))
            print(json.dumps({"long_config": long_configs[name]}), file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
    else:
        host = case.host

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "P": w.P, "rank": w.rank,
                   "d": w.d, "Hl": w.Hl, "flops_per_step": w.flops, "causal": False,
                   "key_split": n_split,
                   **({"tile_override": os.environ["UA_TILE"]} if os.environ.get("UA_TILE") else {})},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "detail": {
            "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
            "warmup_ms_min": WARM_MS,
            "fused_ms_median": round(t_f, 4), "fused_ms_min": round(min(cmp["fused"]), 4),
            "timed_region_launch_ms_mean": round(launch_ms, 4),
            "serial_ms_median": round(t_s, 4),
            "attn_alone_ms_median": round(t_a, 4),
            "permute_ms_median": round(t_p, 4),
            "speedup_serial_over_fused": round(t_s / t_f, 4),
            "residual_fused_vs_alone": round((t_f - t_a) / t_a, 4),
            "hiding_ratio": round((t_s - t_f) / (t_s - t_a), 3) if t_s > t_a else None,
            "permute_hbm_GBs": round(2 * w.out_bytes / (t_p * 1e-3) / 1e9, 1),
            "epilogue_store_bytes": w.out_bytes,
            "store_only_epilogue_ms_median": round(med(cmp["store_only"]), 4),
            "store_only_epilogue_GBs": round(w.out_bytes / (med(cmp["store_only"]) * 1e-3) / 1e9, 1),
            **tr,
            "clock": r["clock"],
            # the same against the peak scaled to the clock the traced call ran at
            "pct_bf16_peak_at_traced_clock": round(100.0 * value / (PEAK_BF16_TFLOPS * tr["sclk_mhz_trace"] / 2400.0), 2)
            if tr.get("sclk_mhz_trace") else None,
            "split": unsplit,
            "io": io,
            "long_configs": long_configs,
            "wall_ms_timed_region": round(r["wall_ms"], 3),
            "kernel_code_sha256_16": source_digest(),
        },
    }
    if not args.no_moe:
        from moe_inputs import MOE_WORKLOADS
        moe = {}
        weights = None
        for name in MOE_CONFIGS:
            mw = MOE_WORKLOADS[name]
            c = MoeCase(ua, torch, mw, dev, args.moe_wave, weights)
            weights = c.weights if name == "moe_ds" else None   # moe_ds_skewed shares them
            moe[name] = c.measure(args.warmup, args.rounds)
            print(json.dumps({"moe": moe[name]}), file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
        out["detail"]["moe"] = moe
    if not args.no_cpu:
        Q, K, V = host
        out["cpu_baseline"] = cpu_baseline(w, Q, K, V, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
