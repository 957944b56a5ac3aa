#!/usr/bin/env python3
"""Throughput of batched Gram Newton-Schulz on one MI355X.

Workload (default): 8 dense-MLP momentum matrices 4096 x 16384 bf16 (aspect
ratio 4), i.i.d. normal entries normalised to unit Frobenius norm, Gram
Newton-Schulz with T = 5 Muon quintic steps and a restart after iteration 2.
One step = one gns_gram_batched call over the whole batch (norm, scale,
Gram matrix, n x n iteration, restart, final Q X), inputs resident in HBM.

Prints ONE JSON line with matrices/s, algorithmic TFLOP/s and the fraction of
the dense bf16 MFMA peak, the roofline of the dominant kernel (from HIP
events recorded around every launch on the library's stream), standard
Newton-Schulz timed on the same inputs and GPU, and the fp64 CPU oracle timed
on a one-matrix sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense MFMA peaks; bf16x3 runs on the bf16 matrix cores
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "bf16x3": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_gram(n, m, T, n_restarts):
    """Dion3 §4.1/§4.2 count with symmetric products (2 FLOPs per FMA)."""
    return T * 4.0 * n ** 3 + 3.0 * m * n * n - 3.0 * n ** 3 + n_restarts * (3.0 * m * n * n - 3.0 * n ** 3)


def flops_standard_sym(n, m, T):
    return T * (3.0 * m * n * n + n ** 3)


# --------------------------------------------------------------------------
# rocprofv3 summaries (read the csv files rocprofv3 writes; nothing here runs
# on the GPU)
# --------------------------------------------------------------------------
KERNEL_SRC = os.path.join(ROOT, "gram_newton_schulz_amd", "csrc", "gns_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def short_kernel(name):
    """rocprofv3 kernel name -> the library's short name, e.g.
    'gns::gemm_nt<gns::EBF16, 256, 0, 1, 0, 0>' -> 'gemm_nt<bf16,256,sym>'.
    The fourth template argument is the plane count (2 means split bf16,
    'bf16x3'); a fifth argument of 1 marks the K-major-B product, 'gemm_nn';
    a sixth of 1 or 2 marks the two passes of a K-split Gram matrix
    ('sym_kpart', 'sym_ksum')."""
    import re
    m = re.search(r"gemm_nt<gns::E(\w+), (\d+), (\d)(?:, (\d))?(?:, (\d))?(?:, (\d))?>", name)
    if m:
        dt = m.group(1).lower()
        if m.group(4) == "2":
            dt = "bf16x3"
        kind = "gemm_nn" if m.group(5) == "1" else "gemm_nt"
        mode = ['sym', 'gen', 'final'][int(m.group(3))]
        mode += {"1": "_kpart", "2": "_ksum"}.get(m.group(6) or "0", "")
        return f"{kind}<{dt},{m.group(2)},{mode}>"
    for k in ("norm_partial", "row_partials", "scale_transpose", "scale_rows_f32", "transpose_sumsq",
              "norm_finish", "row_l1",
              "select_topk", "check_rows", "momentum_l1", "row_sumsq", "normuon_factors",
              "dion3_update"):
        if k in name:
            return k
    return name.split("(")[0][:60]


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirname}")


def summarize_stats(dirname):
    rows = _csv(_find(dirname, "kernel_stats.csv"))
    print(f"{'kernel':34s} {'calls':>6s} {'total_ms':>10s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in rows:
        name = short_kernel(r["Name"])
        print(f"{name:34s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e6:10.3f} "
              f"{float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
              f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}")


def _pmc_per_dispatch(dirname, counter):
    out = {}
    for r in _csv(_find(dirname, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        d = out.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"], "v": 0.0})
        d["v"] += float(r["Counter_Value"])
    return out


# kernels after which the next symmetric product of a call is a Gram matrix
# (the input pass, or a restart's Q X)
_BEFORE_GRAM = ("transpose_sumsq", "norm_finish", "norm_partial", "row_partials", "scale_transpose",
                "scale_rows_f32")


def classify(dispatches):
    """{dispatch id: kernel name} -> {dispatch id: short name}, with the
    symmetric products split into ':gram' (a Gram matrix: the first symmetric
    launch after the input pass or after a general product) and ':nxn' (the
    n x n iteration).  Valid for one-stream runs, where dispatch order is call
    order."""
    out, prev = {}, ""
    for i in sorted(dispatches):
        name = short_kernel(dispatches[i])
        if name.startswith("gemm_nt<") and name.endswith(",sym>"):
            name += ":gram" if (prev in _BEFORE_GRAM or prev.endswith(",gen>")) else ":nxn"
        out[i] = name
        prev = name.split(":")[0]
    return out


def summarize_mfma(dirname, workload):
    """MFMA utilisation and clock per kernel kind from a rocprofv3 --pmc run of
    SQ_INSTS_VALU_MFMA_MOPS_<dtype>, SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE with --kernel-trace (one-stream bench run).
    - utilisation = busy cycles summed over the 1024 SIMDs / (cycles x 1024);
    - clock = GRBM_GUI_ACTIVE summed over the 8 XCDs / 8 / kernel duration (the
      GPU-active count also covers a few microseconds of dispatch, so short
      kernels read high);
    - executed TFLOP/s = MOPS x 512 FLOP / duration."""
    rows = _csv(_find(dirname, "counter_collection.csv"))
    trace = {int(r["Dispatch_Id"]): r for r in _csv(_find(dirname, "kernel_trace.csv"))}
    cnt, names = {}, {}
    for r in rows:
        i = int(r["Dispatch_Id"])
        names[i] = r["Kernel_Name"]
        c = cnt.setdefault(i, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    kinds = classify(names)
    agg = {}
    for i, c in cnt.items():
        t = trace.get(i)
        if t is None or "MOPS" not in " ".join(c):
            continue
        dur = (int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) * 1e-9
        mops = sum(v for k, v in c.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS"))
        if dur <= 0 or mops == 0:
            continue
        # a symmetric launch counts toward its kernel and its kind
        for nm in {kinds[i], kinds[i].split(":")[0]}:
            a = agg.setdefault(nm, {"n": 0, "dur": 0.0, "busy": 0.0, "cycles": 0.0, "flops": 0.0})
            a["n"] += 1
            a["dur"] += dur
            a["busy"] += c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            a["cycles"] += c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
            a["flops"] += mops * 512.0
    print(f"{'kernel':36s} {'launches':>8s} {'avg_us':>9s} {'mfma_util':>9s} {'clock_GHz':>9s} {'exec_TFLOPs':>11s}")
    for name, a in sorted(agg.items()):
        util = a["busy"] / (a["cycles"] * 1024.0)
        clock = a["cycles"] / a["dur"] / 1e9
        tf = a["flops"] / a["dur"] / 1e12
        print(f"{name:36s} {a['n']:8d} {a['dur'] / a['n'] * 1e6:9.1f} {util:9.3f} {clock:9.3f} {tf:11.1f}")
        print("MFMA " + json.dumps({"kernel": name, "launches": a["n"], "avg_launch_ms": a["dur"] / a["n"] * 1e3,
                                    "mfma_util": util, "clock_ghz": clock, "exec_tflops": tf,
                                    "exec_flops_per_launch": a["flops"] / a["n"], "workload": workload,
                                    "source_sha256_16": kernel_source_hash()}))


def summarize_counters(dirname, workload):
    """Every counter of a rocprofv3 --pmc --kernel-trace run (one stream),
    per kernel kind: the sum per launch and, for SQ cycle counts, the share
    of CU cycles (sum / (GRBM_GUI_ACTIVE / 8 x 256 CUs); SQ counters are
    summed over the CUs of each shader engine, GRBM_GUI_ACTIVE over the 8
    XCDs)."""
    rows = _csv(_find(dirname, "counter_collection.csv"))
    trace = {int(r["Dispatch_Id"]): r for r in _csv(_find(dirname, "kernel_trace.csv"))}
    cnt, names = {}, {}
    for r in rows:
        i = int(r["Dispatch_Id"])
        names[i] = r["Kernel_Name"]
        c = cnt.setdefault(i, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    kinds = classify(names)
    agg = {}
    for i, c in cnt.items():
        t = trace.get(i)
        if t is None:
            continue
        a = agg.setdefault(kinds[i], {"n": 0, "dur": 0.0, "c": {}})
        a["n"] += 1
        a["dur"] += (int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) * 1e-9
        for k, v in c.items():
            a["c"][k] = a["c"].get(k, 0.0) + v
    for name, a in sorted(agg.items()):
        cyc = a["c"].get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        rec = {"kernel": name, "launches": a["n"], "avg_launch_us": round(a["dur"] / a["n"] * 1e6, 1),
               "workload": workload, "source_sha256_16": kernel_source_hash()}
        if cyc > 0:
            rec["clock_ghz"] = round(cyc / a["dur"] / 1e9, 3)
        rec["per_launch"] = {k: v / a["n"] for k, v in sorted(a["c"].items())}
        if cyc > 0:
            rec["per_cu_cycle"] = {k: round(v / (cyc * 256.0), 4) for k, v in sorted(a["c"].items())
                                   if k.startswith("SQ_") and ("CYCLES" in k or "ACTIVE" in k or "CONFLICT" in k
                                                               or "WAIT" in k)}
        print("COUNTERS " + json.dumps(rec))


def summarize_pmc(fetch_dir, write_dir, calib_mib, workload):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) per kernel, scaled by the
    reading of the calibration copy (a device copy of calib_mib MiB, which
    reads and writes exactly that many bytes)."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    for src in (fetch, write):
        kinds = classify({i: d["kernel"] for i, d in src.items()})
        for i, d in src.items():
            d["kind"] = kinds[i]
    def first(d, pred):
        for k in sorted(d):
            if pred(d[k]["kernel"]):
                return d[k]["v"]
        return None
    fs = ws = 1.0
    if calib_mib:
        is_copy = lambda k: "copy" in k.lower()
        cf, cw = first(fetch, is_copy), first(write, is_copy)
        if cf and cw:
            fs, ws = calib_mib * 1024.0 / cf, calib_mib * 1024.0 / cw
    print(f"calibration copy {calib_mib} MiB: fetch scale {fs:.4f}, write scale {ws:.4f}")
    agg = {}
    for src, key, scale in ((fetch, "fetch", fs), (write, "write", ws)):
        for d in src.values():
            name = short_kernel(d["kernel"])
            if not (name.startswith("gemm_n") or name in HBM_KERNELS):
                continue
            # every symmetric launch counts toward its kernel and its kind
            for nm in {name, d["kind"]}:
                a = agg.setdefault(nm, {"fetch": [], "write": []})
                a[key].append(d["v"] * 1024.0 * scale)
    print(f"{'kernel':34s} {'launches':>8s} {'fetch_MiB/launch':>17s} {'write_MiB/launch':>17s}")
    for name, a in sorted(agg.items()):
        nf = max(len(a["fetch"]), 1)
        nw = max(len(a["write"]), 1)
        f_avg = sum(a["fetch"]) / nf
        w_avg = sum(a["write"]) / nw
        print(f"{name:34s} {nf:8d} {f_avg / 2 ** 20:17.1f} {w_avg / 2 ** 20:17.1f}")
        print("TRAFFIC " + json.dumps({"kernel": name, "bytes_per_launch": f_avg + w_avg,
                                        "fetch_bytes": f_avg, "write_bytes": w_avg,
                                        "workload": workload,
                                        "source_sha256_16": kernel_source_hash()}))


HBM_KERNELS = ("norm_partial", "row_partials", "scale_transpose", "scale_rows_f32", "transpose_sumsq", "norm_finish",
               "momentum_l1",
               "row_sumsq", "normuon_factors", "dion3_update", "select_topk")


def mfma_from_profile(kernel, workload):
    """The MFMA record of `kernel` on `workload` written by --summarize-mfma
    into profiles/, or None when absent or taken on a different kernel
    source."""
    try:
        names = [n for n in os.listdir(PROFILES) if n.endswith(".txt")]
    except FileNotFoundError:
        return None
    h = kernel_source_hash()
    for n in names:
        with open(os.path.join(PROFILES, n)) as f:
            for line in f:
                if line.startswith("MFMA "):
                    rec = json.loads(line[len("MFMA "):])
                    if (rec.get("kernel") == kernel and rec.get("workload") == workload
                            and rec.get("source_sha256_16") == h):
                        return rec
    return None


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` recorded in profiles/ by
    --summarize-pmc, or None when absent, taken on another workload or taken
    on a different kernel source."""
    try:
        names = [n for n in os.listdir(PROFILES) if n.endswith(".txt")]
    except FileNotFoundError:
        return None
    h = kernel_source_hash()
    for n in names:
        with open(os.path.join(PROFILES, n)) as f:
            for line in f:
                if line.startswith("TRAFFIC "):
                    rec = json.loads(line[len("TRAFFIC "):])
                    if (rec.get("kernel") == kernel and rec.get("workload") == workload
                            and rec.get("source_sha256_16") == h):
                        return round(rec["bytes_per_launch"])
    return None


class SmiSampler:
    """Socket power, gfx clocks and package-power throttling while the GPU
    runs a workload, from the driver's GPU metrics table (amdsmi).  The
    table refreshes about once a second, so the window must last a few
    seconds; a thread polls it every `period` seconds and keeps each new
    table.  Between the first and the last table of the window:
    - power: energy accumulator difference (units of 15.259 uJ, 2^-16 J)
      over the firmware timestamp difference (10 ns units);
    - ppt_residency_frac: share of the accumulation ticks spent limited by
      package power tracking;
    - gfxclk: per-XCD clocks of the tables after the first.
    Every field is None where the metrics cannot be read; the benchmark never
    depends on them."""

    ENERGY_J = 2.0 ** -16
    FW_TICK_S = 1e-8

    def __init__(self, period=0.05):
        import threading
        self.period, self.tables, self.h, self.smi = period, [], None, None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            hs = amdsmi.amdsmi_get_processor_handles()
            if len(hs) == 1:        # one GPU per box here: no index mapping to get wrong
                self.smi, self.h = amdsmi, hs[0]
        except Exception:
            self.smi = None

    @staticmethod
    def _num(v):
        return float(v) if isinstance(v, (int, float)) and not isinstance(v, bool) else None

    def _metrics(self):
        try:
            return self.smi.amdsmi_get_gpu_metrics_info(self.h)
        except Exception:
            return None

    def _keep(self, m):
        if m is None:
            return
        ts = self._num(m.get("firmware_timestamp"))
        if ts is None or (self.tables and self._num(self.tables[-1].get("firmware_timestamp")) == ts):
            return
        self.tables.append(m)

    def _run(self):
        import time as _t
        while not self._stop.is_set():
            self._keep(self._metrics())
            _t.sleep(self.period)

    def __enter__(self):
        import threading
        if self.smi is not None:
            self._keep(self._metrics())          # the table current at the start (pre-window)
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        """None without metrics or with fewer than two tables refreshed inside
        the window (the table current at the start may predate the load)."""
        if self.smi is None or len(self.tables) < 3:
            return None
        win = self.tables[1:]
        first, last = win[0], win[-1]
        out = {"tables": len(win), "socket_power_w": None, "ppt_residency_frac": None, "power_cap_w": None,
               "gfxclk_mhz_mean": None, "gfxclk_mhz_min": None, "gfxclk_mhz_max": None}
        try:
            dE = self._num(last.get("energy_accumulator")) - self._num(first.get("energy_accumulator"))
            dt = (self._num(last.get("firmware_timestamp")) - self._num(first.get("firmware_timestamp"))) * self.FW_TICK_S
            if dt > 0:
                out["socket_power_w"] = round(dE * self.ENERGY_J / dt, 1)
        except Exception:
            pass
        try:
            d_ppt = self._num(last.get("ppt_residency_acc")) - self._num(first.get("ppt_residency_acc"))
            d_acc = self._num(last.get("accumulation_counter")) - self._num(first.get("accumulation_counter"))
            if d_acc > 0:
                out["ppt_residency_frac"] = round(d_ppt / d_acc, 4)
        except Exception:
            pass
        clks = []
        for m in win[1:] or win:
            c = [self._num(v) for v in (m.get("current_gfxclks") or [])]
            clks.extend(v for v in c if v and v < 10000)
        if clks:
            out["gfxclk_mhz_mean"] = round(sum(clks) / len(clks), 1)
            out["gfxclk_mhz_min"], out["gfxclk_mhz_max"] = min(clks), max(clks)
        try:
            cap = self._num(self.smi.amdsmi_get_power_cap_info(self.h).get("power_cap"))
            if cap:
                out["power_cap_w"] = cap / 1e6 if cap > 1e5 else cap      # reported in microwatts
        except Exception:
            pass
        return out


def power_window(fn, torch, seconds=3.0):
    """Run fn (one call) back to back for `seconds` under an SmiSampler and
    return its summary; None (and no time spent) without GPU metrics."""
    smi = SmiSampler()
    if smi.smi is None:
        return None
    with smi:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
    return smi.summary()


def vendor_gemm(torch, w, steps=20):
    """The vendor library's batched GEMM (torch.bmm, hipBLASLt on ROCm) on the
    products of Gram NS at the workload's shape, for comparison: Q X
    (n x n by n x m), the full X X^T (n x m by m x n, the transpose copied to
    a contiguous operand) and a full n x n product.  bf16 in and out,
    contiguous operands; median ms of `steps` calls, TFLOP/s, and the GPU's
    power and clock over 3 s of back-to-back calls."""
    B, n, m = w.batch, w.n, w.m
    g = torch.Generator(device="cuda").manual_seed(0)
    out = []
    for name, (mm, kk, nn) in (("QX", (n, n, m)), ("XXt_full", (n, m, n)), ("nxn_full", (n, n, n))):
        A = (torch.randn(B, mm, kk, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        Bm = (torch.randn(B, kk, nn, device="cuda", generator=g) * 0.02).to(torch.bfloat16).contiguous()
        C = torch.empty(B, mm, nn, device="cuda", dtype=torch.bfloat16)

        def fn():
            torch.bmm(A, Bm, out=C)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(steps):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        out.append({"product": name, "shape": [B, mm, kk, nn], "median_ms": round(ms, 4),
                    "tflops": round(2.0 * B * mm * kk * nn / (ms * 1e-3) / 1e12, 1),
                    "power": power_window(fn, torch, 3.0)})
        del A, Bm, C
        torch.cuda.empty_cache()
    return out


def bench_dion3_step(gns, synth, torch, w, coeffs, restarts, stream, steps=10):
    """One whole Dion3 update (Algorithm 4: momentum sum, l1 selection of
    k = n/4 rows, Gram NS of those rows, NorMuon, decay, row update, error
    feedback) of the workload's batch shape with fp32 W and M and a bf16
    gradient; per-kernel times from the library's launch events."""
    log(f"timing the Dion3 update on {w.batch} x {w.n}x{w.m}, f = 1/4")
    k = gns.select_count(w.n, 0.25)
    W, G, M, v = (t.cuda() for t in synth.dion3_state(w.batch, w.n, w.m, seed=77))
    ws = torch.empty(gns.dion3_workspace_bytes(torch.bfloat16, w.batch, w.n, w.m, k), dtype=torch.uint8,
                     device="cuda")
    S = torch.empty(w.batch, k, dtype=torch.int64, device="cuda")
    kw = dict(lr=0.02, weight_decay=0.1, mu=0.95, beta2=0.95, eps=1e-8, normuon=True, row_idx=S,
              workspace=ws, stream=stream)
    for _ in range(2):
        gns.dion3_step(W, G, M, v, k, coeffs, restarts, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        gns.dion3_step(W, G, M, v, k, coeffs, restarts, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gns.timing_reset()
    gns.timing_enable(True)
    for _ in range(steps):
        gns.dion3_step(W, G, M, v, k, coeffs, restarts, split_batch=False, **kw)
    torch.cuda.synchronize()
    gns.timing_enable(False)
    per = {}
    for name, kernel, fl, by, kms in gns.timing_read():
        if name in ("momentum_l1", "select_topk", "normuon", "dion3_update"):
            d = per.setdefault(name, {"ms": 0.0, "bytes": 0.0})
            d["ms"] += kms
            d["bytes"] += by
    kernels = {n: {"ms": round(d["ms"] / steps, 4),
                   "gbs": round(d["bytes"] / (d["ms"] / 1e3) / 1e9, 1),
                   "frac_hbm": round(d["bytes"] / (d["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 3)}
               for n, d in per.items() if d["ms"] > 0}
    del W, G, M, v, ws
    return {"k": k, "ms_per_step": round(ms, 4), "updates_per_s": round(w.batch / (ms / 1e3), 2),
            "hbm_kernels": kernels}


def desc_of(cfg):
    return {
        2: "16 x 1024x4096 bf16, log-uniform spectrum [1e-4,1]",
        3: "8 x 4096x16384 bf16 dense-MLP momentum, N(0,0.02^2) normalised",
        4: "64 x 2048x7168 bf16 MoE expert stack, Student-t nu=3 normalised",
        5: "8 x 4096x16384 bf16 N(0,1), 1024 seeded rows per matrix gathered/scattered",
    }[cfg]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--compute", default="bf16", choices=["bf16", "f16", "bf16x3"],
                    help="compute type of the products (bf16x3: hi/lo bf16 pairs, 3 MFMAs per product)")
    ap.add_argument("--no-standard", action="store_true", help="skip the standard-NS comparison")
    ap.add_argument("--one-stream", action="store_true",
                    help="time every pass with the whole batch on one stream (no split over the "
                         "library's two streams); used for kernel-trace profiles")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dion3", action="store_true",
                    help="skip the timing of the whole Dion3 update (f = 1/4) on the workload's shape")
    ap.add_argument("--only-dion3", action="store_true",
                    help="time only the whole Dion3 update on the workload's shape (for profiles)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a known-size "
                         "kernel that calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="print a summary of a rocprofv3 --kernel-trace --stats csv directory and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print per-kernel HBM traffic from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="print MFMA utilisation and clock per kernel from a rocprofv3 --pmc run and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print every counter per kernel kind from a rocprofv3 --pmc --kernel-trace run and exit")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor library's bf16 GEMM (torch.bmm) on the workload's products "
                         "(Q X, full X X^T, full n x n) with power and clock, print VENDOR lines and exit")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the 3 s power and clock window (for profiled runs)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the timing of the other workloads (16 x 1024x4096 in bf16x3 and fp16, "
                         "64 x 2048x7168, 8 x 4096x16384 with 1024 selected rows)")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.workload)
        return
    if args.summarize_pmc:
        # records of the Dion3 update are tagged apart from the workload's own call
        tag = f"dion3 update on workload {args.workload}'s shape" if args.only_dion3 else args.workload
        summarize_pmc(*args.summarize_pmc, calib_mib=args.calib_copy_mib, workload=tag)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library runs on one GPU; sharding across GPUs is described, not implemented",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gram_newton_schulz_amd as gns
    from gram_newton_schulz_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")   # contents irrelevant
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS[args.workload]
    if args.vendor_gemm:
        for rec in vendor_gemm(torch, w):
            print("VENDOR " + json.dumps({"workload": args.workload, **rec}), flush=True)
        return
    coeffs = synth.NS5_MUON
    T, restarts = 5, (2,)
    cdt = {"bf16": torch.bfloat16, "f16": torch.float16, "bf16x3": "bf16x3"}[args.compute]

    if args.only_dion3:
        print(json.dumps({"dion3_step": bench_dion3_step(gns, synth, torch, w, coeffs, restarts,
                                                         torch.cuda.current_stream(), steps=args.steps)}),
              flush=True)
        return

    log(f"generating workload {args.workload}: {w.batch} x {w.n}x{w.m}")
    X = synth.workload_batch(args.workload)
    rows_t = synth.workload_rows(args.workload)
    Xd = X.cuda()
    rows_d = rows_t.cuda() if rows_t is not None else None
    rows = w.k if w.k else w.n
    out = torch.zeros_like(Xd)
    ws = torch.empty(max(gns.gram_workspace_bytes(cdt, w.batch, rows, w.m),
                         gns.standard_workspace_bytes(cdt, w.batch, rows, w.m)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    split = not args.one_stream

    def step(split_batch=split):
        gns.gram_ns_batched(Xd, coeffs, restarts, row_idx=rows_d, out=out, compute_dtype=cdt,
                            workspace=ws, stream=stream, split_batch=split_batch)

    def step_one_stream():
        step(False)

    def step_std():
        gns.standard_ns_batched(Xd, coeffs, row_idx=rows_d, out=out, compute_dtype=cdt,
                                workspace=ws, stream=stream, split_batch=split)

    def timed(fn, steps, warmup, per_launch=False, per_step=None):
        """Mean ms per step over `steps` calls between two events on the
        caller's stream (the library's streams join it after every call).
        per_step, when a list, receives each call's ms from an event recorded
        before every call."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if per_launch:
            gns.timing_reset()
            gns.timing_enable(True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)] if per_step is not None else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            if ev:
                ev[i].record(stream)
            fn()
        if ev:
            ev[steps].record(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if ev:
            per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        recs = []
        if per_launch:
            gns.timing_enable(False)
            recs = gns.timing_read()
        return e0.elapsed_time(e1) / steps, wall, recs

    log(f"warmup {args.warmup}, timing {args.steps} Gram NS steps")
    # Per-launch events are taken with the whole batch on one stream, so that
    # every launch has the GPU to itself and its duration measures the kernel.
    ms, wall, recs = timed(step_one_stream, args.steps, args.warmup, per_launch=True)
    # the headline number: no per-launch events, batch split over two streams
    # (one event per call gives the median and the interquartile range)
    step_ms = []
    ms_clean, wall_clean, _ = timed(step, args.steps, 1, per_launch=False, per_step=step_ms)
    q1, med, q3 = (float(v) for v in np.percentile(step_ms, [25, 50, 75]))
    ms_one, _, _ = timed(step_one_stream, args.steps, 1, per_launch=False) if split else (ms_clean, 0, 0)
    # the same call back to back for a few seconds: socket power, package
    # power throttling and gfx clocks from the driver's metrics, and the
    # dense bf16 peak at that clock
    power = None
    if not args.no_power:
        log("power and clock window (3 s of the same call)")
        power = power_window(step, torch)
    if power and power.get("gfxclk_mhz_mean"):
        power["peak_tflops_at_clock"] = round(256 * 4096 * power["gfxclk_mhz_mean"] * 1e6 / 1e12, 1)
        power["pct_of_peak_at_clock"] = round(100 * w.batch * flops_gram(rows, w.m, T, len(restarts)) /
                                              (ms_clean / 1e3) / 1e12 / power["peak_tflops_at_clock"], 2)

    alg_flops = w.batch * flops_gram(rows, w.m, T, len(restarts))
    value = w.batch / (ms_clean / 1e3)
    tflops = alg_flops / (ms_clean / 1e3) / 1e12
    peak = PEAK_TFLOPS[args.compute]

    # per-kernel aggregation (all launches of the timed region)
    per_kernel = {}
    per_step_name = {}
    for name, kernel, fl, by, kms in recs:
        d = per_kernel.setdefault(kernel, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
        d["launches"] += 1
        d["ms"] += kms
        d["flops"] += fl
        d["bytes"] += by
        e = per_step_name.setdefault(name, {"launches": 0, "ms": 0.0, "flops": 0.0})
        e["launches"] += 1
        e["ms"] += kms
        e["flops"] += fl
    dom_name = max(per_kernel, key=lambda k: per_kernel[k]["ms"])
    dom = per_kernel[dom_name]
    dom_avg_ms = dom["ms"] / dom["launches"]
    dom_tflops = dom["flops"] / (dom["ms"] / 1e3) / 1e12
    roofline = {
        "kernel": dom_name,
        "bound": "mfma",
        "achieved": round(dom_tflops, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(dom_tflops / peak, 4),
        "traffic": traffic_from_profile(dom_name, args.workload),
        "avg_launch_ms": round(dom_avg_ms, 4),
        "launches_per_step": dom["launches"] / args.steps,
        "share_of_step": round(dom["ms"] / args.steps / ms, 4),
    }
    # MFMA counters of the same kernel (rocprofv3 --pmc, summarised into
    # profiles/ by --summarize-mfma): busy fraction of the matrix cores and
    # the sustained clock, with the peak at that clock (256 CUs x 4096 dense
    # bf16 FLOP per clock)
    mf = mfma_from_profile(dom_name, args.workload)
    if mf:
        roofline["mfma_util"] = round(mf["mfma_util"], 4)
        roofline["clock_ghz"] = round(mf["clock_ghz"], 3)
        roofline["peak_at_clock"] = round(256 * 4096 * mf["clock_ghz"] * 1e9 / 1e12, 1)
        roofline["frac_at_clock"] = round(dom_tflops / roofline["peak_at_clock"], 4)
    else:
        roofline["mfma_util"] = roofline["clock_ghz"] = None
    kernels = {k: {"ms_per_step": round(v["ms"] / args.steps, 4),
                   "avg_launch_ms": round(v["ms"] / v["launches"], 4),
                   "tflops": round(v["flops"] / (v["ms"] / 1e3) / 1e12, 2) if v["ms"] > 0 else None,
                   "gbs": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1) if v["ms"] > 0 else None}
               for k, v in per_kernel.items()}
    steps_detail = {k: {"ms_per_step": round(v["ms"] / args.steps, 4),
                        "tflops": round(v["flops"] / (v["ms"] / 1e3) / 1e12, 2) if v["ms"] > 0 else None}
                    for k, v in per_step_name.items()}
    log(json.dumps({"kernels": kernels, "steps": steps_detail}, indent=1))

    std = None
    if not args.no_standard:
        log("timing standard NS5 on the same inputs")
        ms_std, _, _ = timed(step_std, max(3, args.steps // 2), 1)
        std_flops = w.batch * flops_standard_sym(rows, w.m, T)
        std = {"ms_per_step": round(ms_std, 3), "matrices_per_s": round(w.batch / (ms_std / 1e3), 2),
               "alg_tflops_sym_count": round(std_flops / (ms_std / 1e3) / 1e12, 2),
               "gram_speedup": round(ms_std / ms_clean, 3)}

    # Dion3 selection step (the k = n/4 rows of largest l1 norm) on the same
    # batch: HBM-bound, one read of the input
    sel = None
    if not args.one_stream:
        kk = gns.select_count(w.n, 0.25)
        sel_ws = torch.empty(gns.lib().gns_select_workspace_bytes(w.batch, w.n), dtype=torch.uint8,
                             device="cuda")
        for _ in range(2):
            gns.select_rows_l1(Xd, kk, workspace=sel_ws, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            gns.select_rows_l1(Xd, kk, workspace=sel_ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        sel_ms = e0.elapsed_time(e1) / 10
        sel_bytes = Xd.numel() * Xd.element_size()
        sel = {"k": kk, "ms": round(sel_ms, 4), "gbs": round(sel_bytes / (sel_ms / 1e3) / 1e9, 1),
               "frac_hbm": round(sel_bytes / (sel_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 3)}

    dion3 = None
    if not args.one_stream and not args.no_dion3:
        dion3 = bench_dion3_step(gns, synth, torch, w, coeffs, restarts, stream)

    # the other workloads, each timed as one call per step like the headline
    # (median and interquartile range over the steps); the row subset also
    # reports the HBM rate of its gather (the input pass over the selected
    # rows: their gathered copy with per-tile sums of squares on the direct
    # path, else the norm pass and the scaled copy; from the library's
    # per-launch events)
    others = None
    if not args.one_stream and not args.no_other_workloads and args.workload == 3:
        del Xd, out, ws
        torch.cuda.empty_cache()
        others = {}
        for cfg, computes in ((2, ("bf16x3", "f16", "bf16")), (4, ("bf16",)), (5, ("bf16",))):
            wo = synth.WORKLOADS[cfg]
            log(f"generating workload {cfg}: {wo.batch} x {wo.n}x{wo.m}")
            Xo = synth.workload_batch(cfg).cuda()
            ro = synth.workload_rows(cfg)
            ro = ro.cuda() if ro is not None else None
            rows_o = wo.k or wo.n
            oo = torch.zeros_like(Xo)
            entry = {"workload": desc_of(cfg), "batch": wo.batch, "n": rows_o, "m": wo.m}
            for comp in computes:
                cd = {"bf16": torch.bfloat16, "f16": torch.float16, "bf16x3": "bf16x3"}[comp]
                wso = torch.empty(gns.gram_workspace_bytes(cd, wo.batch, rows_o, wo.m), dtype=torch.uint8,
                                  device="cuda")

                def call(split_batch=True):
                    gns.gram_ns_batched(Xo, coeffs, restarts, row_idx=ro, out=oo, compute_dtype=cd,
                                        workspace=wso, stream=stream, split_batch=split_batch)
                per = []
                mo, _, _ = timed(call, 10, 2, per_step=per)
                fl = wo.batch * flops_gram(rows_o, wo.m, T, len(restarts))
                med_o = float(np.median(per))
                e = {"ms_per_step": round(mo, 4), "median_ms": round(med_o, 4),
                     "iqr_ms": [round(float(v), 4) for v in np.percentile(per, [25, 75])],
                     "matrices_per_s": round(wo.batch / (mo / 1e3), 1),
                     "alg_tflops": round(fl / (mo / 1e3) / 1e12, 1),
                     "pct_peak": round(100 * fl / (mo / 1e3) / 1e12 / PEAK_TFLOPS[comp], 2)}
                if cfg == 5:
                    _, _, rec5 = timed(lambda: call(False), 3, 1, per_launch=True)
                    gather_kernels = ("transpose_sumsq", "norm_partial", "scale_transpose")
                    g = [(name, by, kms) for name, kern, fl_, by, kms in rec5 if name in gather_kernels]
                    gb, gms = sum(b for _, b, _ in g), sum(t for _, _, t in g)
                    ran = [k for k in gather_kernels if any(name == k for name, _, _ in g)]
                    e["gather"] = {"kernels": " + ".join(ran) + " (selected rows)",
                                   "ms_per_step": round(gms / 3, 4),
                                   "gbs": round(gb / (gms / 1e3) / 1e9, 1) if gms > 0 else None,
                                   "frac_hbm": round(gb / (gms / 1e3) / 1e9 / HBM_PEAK_GBS, 3) if gms > 0 else None}
                entry[comp] = e
                del wso
            others[str(cfg)] = entry
            del Xo, oo
            torch.cuda.empty_cache()

    cpu = cpu_std = None
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max(i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas")
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        log(f"CPU oracle baseline on one matrix ({cores} BLAS threads)")
        if w.k:
            x64 = synth.as_f64(X[0][rows_t[0]])
        else:
            x64 = synth.as_f64(X[0])
        t0 = time.perf_counter()
        oracle.gram_ns(x64, coeffs, restarts=restarts)
        dt = time.perf_counter() - t0
        cpu = {"value": round(1.0 / dt, 5), "unit": "matrices/s", "cores": int(cores), "kind": "oracle",
               "sample": f"1 of the {w.batch} matrices ({rows}x{w.m}), fp64 numpy Gram NS, {dt:.1f} s"}
        # the standard NS oracle on the same matrix, beside it
        t0 = time.perf_counter()
        oracle.standard_ns(x64, coeffs)
        dts = time.perf_counter() - t0
        cpu_std = {"value": round(1.0 / dts, 5), "unit": "matrices/s", "cores": int(cores), "kind": "oracle",
                   "sample": f"the same matrix, fp64 numpy standard NS, {dts:.1f} s"}

    desc = desc_of(args.workload)
    line = {
        "metric": "orthogonalized matrices/s + bf16 MFMA TFLOP/s (% peak), 4096x16384 Gram-NS T=5",
        "value": round(value, 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_clean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.compute,
        "data": "synthetic",
        "config": {"workload": desc + f"; Gram NS T={T}, restart after {list(restarts)}, Muon quintic",
                   "batch": w.batch, "n": rows, "m": w.m, "parallelism": "single GPU"},
        "alg_tflops": round(tflops, 2),
        "pct_peak": round(100 * tflops / peak, 2),
        "median_ms": round(med, 4),
        "iqr_ms": [round(q1, 4), round(q3, 4)],
        "ms_per_step_with_launch_events": round(ms, 4),
        "ms_per_step_one_stream": round(ms_one, 4),
        "batch_split_over_streams": split,
        "roofline": roofline,
        # socket power, package-power throttling and gfx clocks over 3 s of
        # the headline call (driver GPU metrics; null where unavailable)
        "gpu_power_clock": power,
        "cpu_baseline": cpu,
        "cpu_baseline_standard_ns": cpu_std,
        "standard_ns5": std,
        "dion3_select_l1": sel,
        "dion3_step": dion3,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
