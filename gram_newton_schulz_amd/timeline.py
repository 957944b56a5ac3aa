"""Per-workgroup timeline of the GEMM launches of one call (measurement tool).

Needs the timeline build of the library (``python -m
gram_newton_schulz_amd.build --timeline`` writes libgns_timeline.so beside
libgns.so).  Every GEMM workgroup of that build records the constant 100 MHz
clock at entry, at the end of its prologue (its first operand stage has
landed), at the end of its main loop and when its last store has completed,
plus the shader-clock cycles in between and the CU and hardware queue it ran
on.  The work is the library's own; only the timestamps are added.

    python -m gram_newton_schulz_amd.timeline [--workload 3] [--split]

prints, per launch, the mean prologue / main loop / epilogue time of a
workgroup, the share of CU time spent inside workgroups, the CU idle time at
the launch's tail and the average shader clock; then the whole call's CU time
split into prologue, main loop, epilogue and idle.
"""
from __future__ import annotations

import argparse
import collections
import ctypes
import json
import os

import numpy as np

from . import binding, build

_MODES = {0: "sym", 1: "gen", 2: "final"}


def _fields(r: np.ndarray) -> dict:
    r = r.astype(np.int64)
    mode = (r[:, 6] >> 56) & 0xFF
    hw = r[:, 7] & 0xFFFFFFFF
    xcc = r[:, 7] >> 32
    return {
        "t0": r[:, 0], "t1": r[:, 1], "t2": r[:, 2], "t3": r[:, 3], "cycles": r[:, 4],
        "ti": r[:, 5] & 0xFFFF, "tj": (r[:, 5] >> 16) & 0xFFFF, "mat": r[:, 5] >> 32,
        "K": r[:, 6] & 0xFFFFFFFF, "grid": (r[:, 6] >> 32) & 0xFFFFFF,
        "mode": mode & 3, "bk": (mode >> 2) & 1, "ks": (mode >> 3) & 3,
        # CU: XCD, shader engine, array and CU id (HW_ID bits 8-14); queue:
        # pipe, queue and micro-engine ids (one HIP stream per queue here)
        "cu": (xcc << 8) | ((hw >> 8) & 0x7F),
        "queue": ((hw >> 24) & 7) | (((hw >> 6) & 3) << 3) | (((hw >> 30) & 3) << 5),
    }


def timeline_lib():
    """The timeline build, loaded through the binding (which then serves every
    call of this process); raises if the library build is already loaded."""
    if binding._lib is not None and binding.LIB_PATH != build.TIMELINE_LIB:
        raise RuntimeError("the library build is already loaded in this process")
    if not os.path.exists(build.TIMELINE_LIB):
        raise RuntimeError(f"{build.TIMELINE_LIB} is missing: python -m gram_newton_schulz_amd.build --timeline")
    binding.LIB_PATH = build.TIMELINE_LIB
    L = binding.lib()
    L.gns_timeline_read.restype = ctypes.c_int
    L.gns_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_uint, ctypes.POINTER(ctypes.c_uint), ctypes.c_int]
    return L


def reset_records(L) -> int:
    """Start a new recording; returns the number of records dropped."""
    n = ctypes.c_uint(0)
    if L.gns_timeline_read(None, 0, ctypes.byref(n), 1) != 0:
        raise RuntimeError("gns_timeline_read failed")
    return n.value


def read_records(L, reset: bool = True, cap: int = 1 << 18) -> np.ndarray:
    """The records since the last reset (one row per workgroup)."""
    n = ctypes.c_uint(0)
    buf = np.zeros((cap, 8), dtype=np.uint64)
    if L.gns_timeline_read(buf.ctypes.data, cap, ctypes.byref(n), int(reset)) != 0:
        raise RuntimeError("gns_timeline_read failed")
    if n.value > cap:
        raise RuntimeError(f"{n.value} workgroups recorded, room for {cap}")
    return buf[: n.value].copy()


def record(workload: int = 3, split: bool = False, calls: int = 1) -> np.ndarray:
    """Run `calls` calls of the workload through the timeline library (after
    three untimed ones) and return their records, one row per workgroup."""
    import torch
    from . import synth
    L = timeline_lib()
    w = synth.WORKLOADS[workload]
    X = synth.workload_batch(workload).cuda()
    rows = synth.workload_rows(workload)
    rows = rows.cuda() if rows is not None else None
    out = torch.zeros_like(X)
    ws = torch.empty(binding.gram_workspace_bytes(X.dtype, w.batch, w.k or w.n, w.m), dtype=torch.uint8,
                     device="cuda")
    s = torch.cuda.current_stream()

    def call():
        binding.gram_ns_batched(X, synth.NS5_MUON, (2,), row_idx=rows, out=out, workspace=ws, stream=s,
                                split_batch=split)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    reset_records(L)
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    return read_records(L)


def launches(f: dict) -> list:
    """Index arrays of the launches, per hardware queue in record order: a new
    launch starts where the kernel kind or grid changes, or where a workgroup
    starts after every earlier one of its launch has finished and the launch's
    grid is complete."""
    out = []
    for q in sorted(set(f["queue"].tolist())):
        idx = np.where(f["queue"] == q)[0]
        start, end_max = 0, f["t3"][idx[0]]
        for p in range(1, len(idx)):
            i, j = idx[p], idx[p - 1]
            key_i = (f["K"][i], f["grid"][i], f["mode"][i], f["bk"][i], f["ks"][i])
            key_j = (f["K"][j], f["grid"][j], f["mode"][j], f["bk"][j], f["ks"][j])
            if key_i != key_j or (f["t0"][i] > end_max and p - start >= f["grid"][idx[start]]):
                out.append(idx[start:p])
                start, end_max = p, f["t3"][i]
            else:
                end_max = max(end_max, f["t3"][i])
        out.append(idx[start:])
    out.sort(key=lambda a: f["t0"][a].min())
    return out


def summarize(r: np.ndarray) -> dict:
    f = _fields(r)
    us = 1e-2                                       # 100 MHz ticks -> microseconds
    cus = sorted(set(f["cu"].tolist()))
    ncu = len(cus)
    T0, T1 = int(f["t0"].min()), int(f["t3"].max())
    rows = []
    for a in launches(f):
        s0, s1 = int(f["t0"][a].min()), int(f["t3"][a].max())
        per_cu = collections.defaultdict(list)
        for i in a:
            per_cu[int(f["cu"][i])].append((int(f["t0"][i]), int(f["t3"][i])))
        tails = [s1 - max(e for _, e in v) for v in per_cu.values()]
        busy = float(np.sum(f["t3"][a] - f["t0"][a]))
        kind = _MODES[int(f["mode"][a[0]])] + ("/kmajor" if f["bk"][a[0]] else "") + \
            ({1: "/kpart", 2: "/ksum"}.get(int(f["ks"][a[0]]), ""))
        rows.append({
            "kind": kind, "K": int(f["K"][a[0]]), "workgroups": int(len(a)), "start_us": (s0 - T0) * us,
            "span_us": (s1 - s0) * us,
            "prologue_us": float(np.mean(f["t1"][a] - f["t0"][a])) * us,
            "loop_us": float(np.mean(f["t2"][a] - f["t1"][a])) * us,
            "epilogue_us": float(np.mean(f["t3"][a] - f["t2"][a])) * us,
            "busy_frac": busy / (ncu * (s1 - s0)),
            "tail_idle_us": float(np.mean(tails + [s1 - s0] * (ncu - len(per_cu)))) * us,
            "clock_ghz": float(np.sum(f["cycles"][a]) / np.sum(f["t3"][a] - f["t0"][a])) / 10.0,
        })
    span = T1 - T0
    pro = float(np.sum(f["t1"] - f["t0"]))
    loop = float(np.sum(f["t2"] - f["t1"]))
    epi = float(np.sum(f["t3"] - f["t2"]))
    idle = ncu * span - pro - loop - epi
    total = {"call_us": span * us, "cus": ncu, "workgroups": int(len(r)),
             "cu_time_frac": {"prologue": pro / (ncu * span), "loop": loop / (ncu * span),
                              "epilogue": epi / (ncu * span), "idle": idle / (ncu * span)}}
    return {"launches": rows, "call": total}


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--split", action="store_true", help="two-stream batch fan-out (the library default)")
    ap.add_argument("--save", metavar="NPY", help="also save the raw records")
    args = ap.parse_args(argv)
    r = record(args.workload, args.split)
    if args.save:
        np.save(args.save, r)
    s = summarize(r)
    print(f"{'#':>3} {'kind':<14} {'K':>6} {'wgs':>5} {'start_us':>9} {'span_us':>8} {'pro_us':>7} "
          f"{'loop_us':>8} {'epi_us':>7} {'busy':>5} {'tail_us':>8} {'GHz':>5}")
    for i, x in enumerate(s["launches"]):
        print(f"{i:3d} {x['kind']:<14} {x['K']:6d} {x['workgroups']:5d} {x['start_us']:9.0f} {x['span_us']:8.1f} "
              f"{x['prologue_us']:7.1f} {x['loop_us']:8.1f} {x['epilogue_us']:7.1f} {x['busy_frac']:5.2f} "
              f"{x['tail_idle_us']:8.1f} {x['clock_ghz']:5.2f}")
    c = s["call"]
    print(f"call: {c['call_us']:.0f} us on {c['cus']} CUs; CU time: " +
          ", ".join(f"{k} {v:.3f}" for k, v in c["cu_time_frac"].items()))
    print("TIMELINE " + json.dumps({"workload": args.workload, "split": args.split, **c}))


if __name__ == "__main__":
    main()
