"""Burst-Gap microbenchmark driver: runs the store-burst kernel of
include/fa_burst_gap.h over a sweep of producer counts K, per-producer burst
sizes and compute gaps G, and fits the three parameters of the pages' model
("X-Stage" summary page, Methodology: the Burst-Gap model):

    T_iss(G; K, V) = max(T0_iss(K, V), V / R - G)

T0_iss is the backpressure-free issue time of a burst of aggregate volume V
from K producers, R the effective drain rate, Q the outstanding capacity that
sustained injection (G = 0) fills before issue slows to the drain rate.

    python -m flashattention_output_re_amd.burst_gap [--quick] [--out FILE]

prints one JSON document: the raw medians, the fit, the model's error on
every measured point, and its prediction for the fused attention kernel's
per-tile store bursts.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import sys
import time

import numpy as np
import torch

from . import binding

MAGIC = 0x9E3779B9
WARMUP_BURSTS = 4          # bursts ignored when taking steady-state medians


def run(dst: torch.Tensor, producers: int, bytes_per_producer: int, bursts: int,
        gap_iters: int, nontemporal: bool = False, coupled: bool = False):
    """One launch; returns (issue_s, gap_s, clock_hz, complete_s), the first two
    [producers][bursts] arrays in seconds.  coupled: each burst waits for its
    stores to complete before its issue time is taken."""
    need = bursts * producers * bytes_per_producer
    if dst.numel() * dst.element_size() < need:
        raise ValueError("dst too small")
    times = torch.zeros(3 * producers * bursts + 4 * producers, dtype=torch.int64,
                        device=dst.device)
    st = binding.load_library().burst_gap_run_async(
        binding._ptr(dst), binding._ptr(times), producers, bytes_per_producer, bursts, gap_iters,
        int(bool(nontemporal)), int(bool(coupled)), binding._stream(None))
    binding._raise(st, "burst_gap_run_async")
    torch.cuda.synchronize()
    t = times.cpu().numpy().astype(np.int64)
    per = t[:3 * producers * bursts].reshape(producers, bursts, 3)
    tail = t[3 * producers * bursts:].reshape(producers, 4)
    cycles = tail[:, 2] - tail[:, 0]
    ticks = tail[:, 3] - tail[:, 1]                       # 100 MHz
    clock = float(np.median(cycles / np.maximum(ticks, 1) * 1e8))
    issue = (per[:, :, 1] - per[:, :, 0]) / clock
    gap = (per[:, :, 2] - per[:, :, 1]) / clock
    complete = float(np.median(ticks)) * 1e-8
    return issue, gap, clock, complete


def expected_chunks(producers: int, bytes_per_producer: int, bursts: int) -> np.ndarray:
    """The uint32 words the kernel stores, [bursts][producers][chunks][4]."""
    chunks = bytes_per_producer // 16
    i, k, c = np.meshgrid(np.arange(bursts), np.arange(producers), np.arange(chunks), indexing="ij")
    return np.stack([i, k, c, np.full_like(c, MAGIC)], axis=-1).astype(np.uint32)


def measure(configs, bursts: int, device="cuda:0"):
    maxbytes = max(bursts * k * vp for k, vp, _, _ in configs)
    dst = torch.empty(maxbytes // 4, dtype=torch.int32, device=device)
    rows = []
    for k, vp, g, nt in configs:
        run(dst, k, vp, 2, g, nt)                          # warm-up launch
        issue, gap, clock, complete = run(dst, k, vp, bursts, g, nt)
        ss_i = issue[:, WARMUP_BURSTS:]
        ss_g = gap[:, WARMUP_BURSTS:]
        rows.append({
            "producers": k, "bytes_per_producer": vp, "volume": k * vp, "gap_iters": g,
            "nontemporal": bool(nt), "clock_hz": clock,
            "t_iss_s": float(np.median(ss_i)), "gap_s": float(np.median(ss_g)),
            "first_burst_t_iss_s": float(np.median(issue[:, 0])),
            "issue_s_by_burst": [float(x) for x in np.median(issue, axis=0)],
            "gap_s_by_burst": [float(x) for x in np.median(gap, axis=0)],
            "complete_s": complete,
        })
        print(f"K={k:4d} Vp={vp >> 10:6d} KiB g={g:6d} nt={int(nt)}: "
              f"T_iss {rows[-1]['t_iss_s'] * 1e6:8.3f} us  G {rows[-1]['gap_s'] * 1e6:8.3f} us  "
              f"clock {clock / 1e9:.2f} GHz", file=sys.stderr, flush=True)
    return rows


def model(g, t0, v, r):
    """T_iss(G) = max(T0, V / R - G)."""
    return np.maximum(t0, v / r - g)


def fit(rows):
    """T0 per (K, V, nt) from the largest gap; R per nt from the drain-dominated
    points (steady state: V drains per period T_iss + G); Q per (K, nt) from
    the G = 0 bursts as the intercept of cumulative bytes against time."""
    out = {"T0_s": {}, "R_Bps": {}, "Q_bytes": {}}
    keys = sorted({(r["producers"], r["bytes_per_producer"], r["nontemporal"]) for r in rows})
    for k, vp, nt in keys:
        sel = [r for r in rows if (r["producers"], r["bytes_per_producer"], r["nontemporal"]) ==
               (k, vp, nt)]
        big = max(sel, key=lambda r: r["gap_s"])
        out["T0_s"][f"K={k},Vp={vp},nt={int(nt)}"] = big["t_iss_s"]
    for nt in sorted({r["nontemporal"] for r in rows}):
        rates = []
        for r in rows:
            if r["nontemporal"] != nt:
                continue
            t0 = out["T0_s"][f"K={r['producers']},Vp={r['bytes_per_producer']},nt={int(nt)}"]
            if r["t_iss_s"] > 1.5 * t0:
                rates.append(r["volume"] / (r["t_iss_s"] + r["gap_s"]))
        out["R_Bps"][f"nt={int(nt)}"] = float(np.median(rates)) if rates else None
    for r in rows:
        if r["gap_iters"] != 0:
            continue
        rate = out["R_Bps"][f"nt={int(r['nontemporal'])}"]
        if not rate:
            continue
        per = np.array(r["issue_s_by_burst"]) + np.array(r["gap_s_by_burst"])
        t_end = np.cumsum(per)
        sent = r["volume"] * np.arange(1, len(per) + 1)
        q = float(np.median(sent[WARMUP_BURSTS:] - rate * t_end[WARMUP_BURSTS:]))
        key = f"K={r['producers']},nt={int(r['nontemporal'])}"
        out["Q_bytes"].setdefault(key, []).append(max(q, 0.0))
    out["Q_bytes"] = {k: float(np.median(v)) for k, v in out["Q_bytes"].items()}
    err = []
    for r in rows:
        t0 = out["T0_s"][f"K={r['producers']},Vp={r['bytes_per_producer']},nt={int(r['nontemporal'])}"]
        rate = out["R_Bps"][f"nt={int(r['nontemporal'])}"]
        if not rate:
            continue
        pred = float(model(r["gap_s"], t0, r["volume"], rate))
        err.append({"producers": r["producers"], "bytes_per_producer": r["bytes_per_producer"],
                    "gap_iters": r["gap_iters"], "nontemporal": r["nontemporal"],
                    "measured_s": r["t_iss_s"], "model_s": pred,
                    "rel_err": (pred - r["t_iss_s"]) / r["t_iss_s"]})
    out["model_error"] = err
    out["median_abs_rel_err"] = float(np.median([abs(e["rel_err"]) for e in err])) if err else None
    return out


def predict_fused(fitres, tile_bytes=256 * 128 * 2, producers=256, tile_compute_s=0.92e-3):
    """The fused kernel's stores seen as bursts: every CU stores one finished
    256-query tile (64 KiB) per unit, then computes the next unit for about
    tile_compute_s (Video: 1.84 ms per two-unit launch)."""
    key = f"K={producers},Vp={tile_bytes},nt=0"
    t0 = fitres["T0_s"].get(key)
    rate = fitres["R_Bps"].get("nt=0")
    if t0 is None or not rate:
        return None
    v = producers * tile_bytes
    t_iss = float(model(tile_compute_s, t0, v, rate))
    return {"producers": producers, "burst_volume": v, "gap_s": tile_compute_s, "T0_s": t0,
            "drain_time_s": v / rate, "T_iss_s": t_iss,
            "regime": "backpressure-free" if t_iss <= t0 else "drain-dominated",
            "predicted_overhead_frac": t_iss / (t_iss + tile_compute_s)}


def default_configs(quick: bool):
    ks = [256] if quick else [64, 256]
    vps = [64 << 10, 256 << 10] if quick else [16 << 10, 64 << 10, 256 << 10, 1 << 20]
    gaps = [0, 300, 3000, 30000] if quick else [0, 10, 30, 60, 100, 300, 1000, 3000, 10000, 30000]
    nts = [False] if quick else [False, True]
    return [(k, vp, g, nt) for nt in nts for k in ks for vp in vps for g in gaps]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--bursts", type=int, default=24)
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    t = time.perf_counter()
    rows = measure(default_configs(a.quick), a.bursts)
    res = fit(rows)
    doc = {"what": "store-burst microbenchmark, Burst-Gap model fit (local HBM, one MI355X)",
           "bursts": a.bursts, "rows": rows, "fit": res, "fused_prediction": predict_fused(res),
           "seconds": time.perf_counter() - t}
    text = json.dumps(doc)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(json.dumps({k: doc[k] for k in ("fit", "fused_prediction")}, indent=1))


if __name__ == "__main__":
    main()
