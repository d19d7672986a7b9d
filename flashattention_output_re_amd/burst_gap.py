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
    """configs: (K, bytes per producer, gap_iters, nontemporal[, coupled]).
    One row of steady-state medians per config."""
    configs = [tuple(c) + (False,) * (5 - len(c)) for c in configs]
    maxbytes = max(bursts * k * vp for k, vp, _, _, _ in configs)
    dst = torch.empty(maxbytes // 4, dtype=torch.int32, device=device)
    rows = []
    for k, vp, g, nt, cp in configs:
        run(dst, k, vp, 2, g, nt, cp)                      # warm-up launch
        issue, gap, clock, complete = run(dst, k, vp, bursts, g, nt, cp)
        ss_i = issue[:, WARMUP_BURSTS:]
        ss_g = gap[:, WARMUP_BURSTS:]
        rows.append({
            "producers": k, "bytes_per_producer": vp, "volume": k * vp, "gap_iters": g,
            "nontemporal": bool(nt), "coupled": bool(cp), "clock_hz": clock,
            "t_iss_s": float(np.median(ss_i)), "gap_s": float(np.median(ss_g)),
            "first_burst_t_iss_s": float(np.median(issue[:, 0])),
            "issue_s_by_burst": [float(x) for x in np.median(issue, axis=0)],
            "gap_s_by_burst": [float(x) for x in np.median(gap, axis=0)],
            "complete_s": complete,
        })
        print(f"K={k:4d} Vp={vp >> 10:6d} KiB g={g:6d} nt={int(nt)} coupled={int(cp)}: "
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
    coupled = [r for r in rows if r.get("coupled")]
    rows = [r for r in rows if not r.get("coupled")]
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
    # The completion-coupled issuer: each burst waits for its own drain, so
    # its issue time is T0 + V / R whatever the gap (the line the pages'
    # validation refutes for the decoupled issuer).
    cl = []
    for r in coupled:
        t0 = out["T0_s"].get(f"K={r['producers']},Vp={r['bytes_per_producer']},nt={int(r['nontemporal'])}")
        rate = out["R_Bps"].get(f"nt={int(r['nontemporal'])}")
        cl.append({"producers": r["producers"], "bytes_per_producer": r["bytes_per_producer"],
                   "gap_iters": r["gap_iters"], "gap_s": r["gap_s"], "nontemporal": r["nontemporal"],
                   "measured_s": r["t_iss_s"],
                   "coupled_line_s": (t0 + r["volume"] / rate) if (t0 and rate) else None})
    out["coupled"] = cl
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


def source_hash() -> str:
    """sha256/16 of the microbenchmark kernel's source."""
    import hashlib
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "burst_gap.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def summarize(doc: dict, command: str) -> str:
    """Markdown summary of one sweep document (the JSON main() writes)."""
    rows, fit = doc["rows"], doc["fit"]
    dec = [r for r in rows if not r.get("coupled")]
    cpl = [r for r in rows if r.get("coupled")]
    err = np.array([abs(e["rel_err"]) for e in fit["model_error"]])
    clk = np.median([r["clock_hz"] for r in rows]) / 1e9
    L = ["# Burst-Gap model fit: 16-byte store bursts into local HBM on one MI355X\n",
         "Command (from the repository root, after `python -m flashattention_output_re_amd.build`):\n",
         "```", command, f"python -m flashattention_output_re_amd.burst_gap --summarize <that file>",
         "```\n",
         f"Kernel `burst_gap_kernel` (`flashattention_output_re_amd/csrc/burst_gap.hip`, source "
         f"sha256/16 {doc.get('source_sha256_16', '?')}): K producer workgroups, one per CU, "
         f"{doc['bursts']} bursts each; per burst: Vp bytes of 16-byte stores, a barrier without "
         "release fence (issue time), then a dependent-FMA gap of `gap_iters` iterations.  The "
         "completion-coupled issuer adds, before that barrier, a device-scope release fence (L2 "
         "write-back, wait for completion): the stores are visible beyond the issuing XCD.  "
         "Times from `s_memtime` against `s_memrealtime` (100 MHz); "
         f"median shader clock {clk:.2f} GHz.  Steady-state medians skip the first "
         f"{WARMUP_BURSTS} bursts.  Model: T_iss(G; K, V) = max(T0(K, V), V/R - G), V = K * Vp.\n",
         "## Fit (decoupled issuer)\n",
         "* Effective drain rate R (median over drain-dominated points): " +
         ", ".join(f"{'plain' if k == 'nt=0' else 'non-temporal'} {v / 1e12:.2f} TB/s"
                   for k, v in fit["R_Bps"].items() if v) + " (HBM peak 8 TB/s).",
         "* Outstanding capacity Q (intercept of cumulative bytes vs time at G = 0): " +
         ", ".join(f"{k}: {v / 2**20:.1f} MiB" for k, v in fit["Q_bytes"].items()) + ".",
         "* Backpressure-free issue time T0 (largest gap), microseconds:\n",
         "| K | Vp | plain | non-temporal |", "|---|---|---|---|"]
    ks = sorted({r["producers"] for r in dec})
    vps = sorted({r["bytes_per_producer"] for r in dec})
    for k in ks:
        for vp in vps:
            a = fit["T0_s"].get(f"K={k},Vp={vp},nt=0")
            b = fit["T0_s"].get(f"K={k},Vp={vp},nt=1")
            L.append(f"| {k} | {vp >> 10} KiB | {a * 1e6:.3f} | " + (f"{b * 1e6:.3f} |" if b else "- |"))
    L.append(f"\n* Model vs measurement over all {err.size} decoupled points: median |relative "
             f"error| {100 * np.median(err):.2f} %, 90th percentile {100 * np.percentile(err, 90):.1f} %, "
             f"worst {100 * err.max():.0f} % (points at the regime boundary).")
    L.append("* Per-volume fit (the GPU test's: T0 at the largest gap, V/R from G = 0, K = "
             f"{max(ks)}, plain stores):")
    for vp in vps:
        sel = [r for r in dec if r["producers"] == max(ks) and r["bytes_per_producer"] == vp
               and not r["nontemporal"]]
        near = next(r for r in sel if r["gap_iters"] == 0)
        far = max(sel, key=lambda r: r["gap_s"])
        R = near["volume"] / (near["t_iss_s"] + near["gap_s"])
        L.append(f"  Vp = {vp >> 10} KiB (V = {near['volume'] / 2**20:.0f} MiB): T0 = "
                 f"{far['t_iss_s'] * 1e6:.3f} us, V/R = {near['volume'] / R * 1e6:.3f} us, "
                 f"R = {R / 1e12:.2f} TB/s.")
    L.append("  Bursts smaller than the L2/MALL write-back capacity drain faster than the "
             "HBM-bound rate of the largest bursts.\n")
    k = max(ks)
    for vp in vps:
        sel = sorted((r for r in dec if r["producers"] == k and r["bytes_per_producer"] == vp),
                     key=lambda r: r["gap_iters"])
        V = k * vp
        R = fit["R_Bps"]["nt=0"]
        L.append(f"## Steady-state issue time vs gap, K = {k}, Vp = {vp >> 10} KiB "
                 f"(V = {V / 2**20:.0f} MiB, V/R = {V / R * 1e6:.2f} us)\n")
        L.append("| gap_iters | G (us) | T_iss plain (us) | model (us) | T_iss non-temporal (us) | "
                 "model (us) | completion-coupled (us) | T0 + V/R (us) |")
        L.append("|---|---|---|---|---|---|---|---|")
        for g in sorted({r["gap_iters"] for r in sel}):
            pl = next((r for r in sel if r["gap_iters"] == g and not r["nontemporal"]), None)
            nt = next((r for r in sel if r["gap_iters"] == g and r["nontemporal"]), None)
            cp = next((r for r in cpl if r["producers"] == k and r["bytes_per_producer"] == vp
                       and r["gap_iters"] == g), None)
            t0p = fit["T0_s"][f"K={k},Vp={vp},nt=0"]
            cells = [str(g), f"{pl['gap_s'] * 1e6:.2f}", f"{pl['t_iss_s'] * 1e6:.3f}",
                     f"{model(pl['gap_s'], t0p, V, R) * 1e6:.3f}"]
            if nt is not None:
                t0n = fit["T0_s"][f"K={k},Vp={vp},nt=1"]
                rn = fit["R_Bps"]["nt=1"]
                cells += [f"{nt['t_iss_s'] * 1e6:.3f}", f"{model(nt['gap_s'], t0n, V, rn) * 1e6:.3f}"]
            else:
                cells += ["-", "-"]
            cells += ([f"{cp['t_iss_s'] * 1e6:.3f}", f"{(t0p + V / R) * 1e6:.3f}"] if cp else ["-", "-"])
            L.append("| " + " | ".join(cells) + " |")
        L.append("")
    if cpl:
        L.append("The decoupled issuer's time falls with slope -1 to T0 as the gap grows, as the "
                 "equation says.  The completion-coupled issuer does not reach that floor: each burst "
                 "ends only once its stores are visible device-wide, which costs the write-back of "
                 "every L2 line still dirty -- most right after earlier bursts, less as longer gaps "
                 "let the caches drain -- so at every gap it stays above the decoupled issuer, far "
                 "above it at short gaps.  The last column is the coupled form of the equation "
                 "(T0 + V/R, the drain paid in full per burst); on one GPU the visibility cost is "
                 "the L2 write-back rather than that drain, and the column does not describe it.\n")
    fp = doc.get("fused_prediction")
    if fp:
        L.append("## Prediction for the fused attention kernel\n")
        L.append(f"Each of {fp['producers']} CUs stores one finished 256-query tile "
                 f"({fp['burst_volume'] // fp['producers'] >> 10} KiB) per unit and then computes the "
                 f"next unit for G = {fp['gap_s'] * 1e3:.2f} ms.  Burst V = "
                 f"{fp['burst_volume'] / 2**20:.0f} MiB drains in {fp['drain_time_s'] * 1e6:.2f} us << G: "
                 f"{fp['regime']}, T_iss = {fp['T_iss_s'] * 1e6:.2f} us, predicted store overhead "
                 f"{100 * fp['predicted_overhead_frac']:.3f} % of the tile time.")
    return "\n".join(L) + "\n"


def default_configs(quick: bool):
    ks = [256] if quick else [64, 256]
    vps = [64 << 10, 256 << 10] if quick else [16 << 10, 64 << 10, 256 << 10, 1 << 20]
    gaps = [0, 300, 3000, 30000] if quick else [0, 10, 30, 60, 100, 300, 1000, 3000, 10000, 30000]
    nts = [False] if quick else [False, True]
    cfg = [(k, vp, g, nt, False) for nt in nts for k in ks for vp in vps for g in gaps]
    # The completion-coupled issuer on the plain-store sweep of the largest K.
    cfg += [(max(ks), vp, g, False, True) for vp in vps for g in gaps]
    return cfg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--bursts", type=int, default=24)
    ap.add_argument("--out", default=None)
    ap.add_argument("--summarize", default=None, metavar="FILE",
                    help="print the markdown summary of a sweep document written with --out")
    a = ap.parse_args()
    if a.summarize:
        with open(a.summarize) as f:
            doc = json.load(f)
        print(summarize(doc, f"python -m flashattention_output_re_amd.burst_gap --out {a.summarize}"),
              end="")
        return
    t = time.perf_counter()
    rows = measure(default_configs(a.quick), a.bursts)
    res = fit(rows)
    doc = {"what": "store-burst microbenchmark, Burst-Gap model fit (local HBM, one MI355X)",
           "bursts": a.bursts, "source_sha256_16": source_hash(), "rows": rows, "fit": res,
           "fused_prediction": predict_fused(res),
           "seconds": time.perf_counter() - t}
    text = json.dumps(doc)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(json.dumps({k: doc[k] for k in ("fit", "fused_prediction")}, indent=1))


if __name__ == "__main__":
    main()
