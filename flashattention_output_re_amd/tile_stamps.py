"""Per-tile timestamps of the fused kernel at its tile boundary.

Runs the timestamped instances of the fused attention + slab store
(include/fa_instrument.h) on a workload, for each form of the tile boundary:

  piggyback  the product kernel's: the next unit's Q loads and first K/V
             stages are issued, then the finished tile's stores, and only the
             loads are waited for -- the owner resumes the next Q-loop while
             its stores drain ("Technical Summary: X-Stage in DiT Inference",
             Key Contributions 3);
  coupled    the owner waits for its stores to complete before it issues the
             next unit's loads (the completion-coupled issuer the pages'
             validation contrasts with piggybacking);
  ordered    the stores, then the next unit's loads, one wait for both.

For every pair of consecutive units a workgroup runs (unit u, then u + grid),
per wave, it reports distributions over tiles of

  issue_span   last stage done -> last store instruction issued (normalise,
               convert, the next prologue's issue, the 128-bit stores)
  resume_wait  last store issued -> the wait before the next Q-loop returned:
               the time the owner is held at the boundary
  start_gap    last store issued -> after the barrier that starts the next
               Q-loop
  drain        (coupled only) last store issued -> the stores complete: the
               span over which a tile's stores are accepted but not done,
               the local-HBM form of the pages' per-tile remote-store span
  q_loop       the Q-loop of the unit (barrier after its prologue -> last
               stage done)

in shader-clock cycles (s_memtime) and in microseconds (cycles over the clock
the records imply: their span against the call's event time).  Each mode's
whole-call time is taken with HIP events, alternating the modes.

    python -m flashattention_output_re_amd.tile_stamps [--workload video] [--reps 5]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np
import torch

from . import binding

MODES = {"piggyback": binding.BOUNDARY_PIGGYBACK, "coupled": binding.BOUNDARY_COUPLED,
         "ordered": binding.BOUNDARY_ORDERED}
WORDS = 8            # uint32 per record
WAVES = 8


def records(stamps: np.ndarray, units: tuple) -> list:
    """Split the stamp buffer into the call's launches: a list of
    [units][waves][8] uint32 arrays."""
    out, base = [], 0
    for n in units:
        if n:
            out.append(stamps[base * WAVES * WORDS:(base + n) * WAVES * WORDS]
                       .reshape(n, WAVES, WORDS).astype(np.uint64))
        base += n
    return out


def boundaries(rec: np.ndarray) -> dict:
    """Per (consecutive unit pair of one workgroup, wave) boundary spans, in
    cycles (uint32 differences modulo 2^32), and the Q-loop of every unit."""
    m32 = np.uint64(1 << 32)

    def d(a, b):
        return ((b + m32 - a) % m32).astype(np.int64)

    n = rec.shape[0]
    assert np.array_equal(rec[:, 0, 5], np.arange(n, dtype=np.uint64)), "unit ids"
    wg = rec[:, 0, 6].astype(np.int64)
    out = {"issue_span": [], "resume_wait": [], "start_gap": [], "drain": []}
    for g in np.unique(wg):
        us = np.sort(np.nonzero(wg == g)[0])
        for u, un in zip(us[:-1], us[1:]):
            a, b = rec[u], rec[un]
            out["issue_span"].append(d(a[:, 2], a[:, 3]))
            out["resume_wait"].append(d(a[:, 3], b[:, 0]))
            out["start_gap"].append(d(a[:, 3], b[:, 1]))
            if np.any(a[:, 4]):
                out["drain"].append(d(a[:, 3], a[:, 4]))
    res = {k: np.concatenate(v) if v else np.zeros(0, np.int64) for k, v in out.items()}
    res["q_loop"] = d(rec[:, :, 1], rec[:, :, 2]).ravel()
    return res


def span_cycles(recs: list) -> int:
    """Cycles from the earliest record start to the latest store issue."""
    lo, hi = None, None
    for r in recs:
        full = (r[:, :, 7] << np.uint64(32)) | r[:, :, 3]
        # [0] and [3] of one record are within one unit; [7] dates [3].
        first = full - ((r[:, :, 3] + np.uint64(1 << 32) - r[:, :, 0]) % np.uint64(1 << 32))
        lo = first.min() if lo is None else min(lo, first.min())
        hi = full.max() if hi is None else max(hi, full.max())
    return int(hi - lo)


def summary(x: np.ndarray, hz: float) -> dict:
    if not x.size:
        return {"n": 0}
    q = np.percentile(x, [10, 50, 90, 99])
    return {"n": int(x.size), "p10_cyc": float(q[0]), "p50_cyc": float(q[1]),
            "p90_cyc": float(q[2]), "p99_cyc": float(q[3]), "max_cyc": float(x.max()),
            "mean_cyc": float(x.mean()), "p50_us": float(q[1] / hz * 1e6),
            "p90_us": float(q[2] / hz * 1e6), "mean_us": float(x.mean() / hz * 1e6)}


def measure(workload: str, reps: int = 5, seed_inputs=None) -> dict:
    import workloads as wl
    w = wl.WORKLOADS[workload]
    if w.D != 128 or not w.scale > 0:
        raise ValueError("the timestamped instances cover D = 128 and scale > 0")
    dev = torch.device("cuda:0")
    inp = wl.make(workload) if seed_inputs is None else seed_inputs
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    mask = None
    if inp.mask is not None:
        mask = torch.from_numpy(inp.mask.view(np.int64)).to(dev)
    shape = (w.P, w.B, w.S // w.P, w.H, w.D)
    ref = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    binding.attn_fwd_relayout_async(q, k, v, ref, w.B, w.H, w.S, w.D, w.P, w.scale, mask)
    words = binding.attn_instrumented_stamp_words(w.B, w.H, w.S)
    stamps = {m: torch.zeros(words, dtype=torch.int32, device=dev) for m in MODES}
    outs = {m: torch.empty(shape, dtype=torch.bfloat16, device=dev) for m in MODES}
    stream = torch.cuda.current_stream()
    units = {}
    times = {m: [] for m in list(MODES) + ["product"]}

    def call(m):
        if m == "product":
            binding.attn_fwd_relayout_async(q, k, v, ref, w.B, w.H, w.S, w.D, w.P, w.scale, mask,
                                            stream)
        else:
            units[m] = binding.attn_fwd_relayout_instrumented_async(
                q, k, v, outs[m], w.B, w.H, w.S, w.D, w.P, w.scale, mask, MODES[m], stamps[m],
                stream)

    order = list(MODES) + ["product"]
    for m in order:              # warm-up
        call(m)
    torch.cuda.synchronize()
    for i in range(reps):
        for m in (order if i % 2 == 0 else order[::-1]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(m)
            e1.record(stream)
            torch.cuda.synchronize()
            times[m].append(e0.elapsed_time(e1))
    res = {"workload": workload, "kernel_source_sha256_16": source_hash(),
           "shape": {"B": w.B, "H": w.H, "S": w.S, "D": w.D, "P": w.P},
           "masked": mask is not None, "reps": reps,
           "call_ms_median": {m: float(np.median(t)) for m, t in times.items()},
           "modes": {}}
    ref_bits = ref.view(torch.int16)
    for m in MODES:
        res["modes"][m] = {"output_equals_product": bool(torch.equal(outs[m].view(torch.int16),
                                                                      ref_bits)),
                           "launch_units": list(units[m])}
        recs = records(stamps[m].cpu().numpy().view(np.uint32), units[m])
        cyc = span_cycles(recs)
        hz = cyc / (res["call_ms_median"][m] * 1e-3)
        res["modes"][m]["clock_hz_implied"] = hz
        for li, r in enumerate(recs):
            name = ["first_launch", "second_launch"][li]
            b = boundaries(r)
            res["modes"][m][name] = {k: summary(x, hz) for k, x in b.items()}
    return res


def source_hash() -> str:
    """sha256/16 of the fused kernel's sources (as bench.py reports it)."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for name in ("fa_fwd_kernel.hip", "fa_fwd_kernel.h"):
        with open(os.path.join(base, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summarize(docs: list, command: str) -> str:
    """Markdown summary of measure() results for one or more workloads."""
    L = ["# Tile boundary of the fused kernel: per-tile timestamps\n",
         "Command (from the repository root, after `python -m flashattention_output_re_amd.build`):\n",
         "```", command, "python -m flashattention_output_re_amd.tile_stamps --summarize <those files>",
         "```\n",
         f"Kernel source sha256/16: {docs[0].get('kernel_source_sha256_16', '?')}.  Timestamped "
         "instances of `fa_fwd_pp_kernel` (last template argument 1-3; include/fa_instrument.h) "
         "record the low 32 bits of `s_memtime` per unit and wave; spans below are differences "
         "within one workgroup, in shader cycles, over every pair of consecutive units a "
         "workgroup runs (p50 / p90 over units x 8 waves).  Boundary forms: **piggyback** (the "
         "product kernel's: next unit's Q loads -- issued before the epilogue's merge and "
         "normalisation -- and first K/V stages, then the tile's stores, wait for the loads "
         "only), **ordered** (the stores, then the next unit's loads, one wait "
         "for both: the previous form of this kernel), **coupled** (the stores made visible "
         "device-wide by a device-scope release -- L2 write-back, wait for completion -- before "
         "the next unit's loads: the completion-coupled counterfactual).\n",
         "* issue span: last stage done -> last store instruction issued;",
         "* held: last store issued -> the wait before the next Q-loop returned (the time the "
         "owner is kept from resuming);",
         "* to start: last store issued -> past the barrier that starts the next Q-loop;",
         "* drain (coupled only): last store issued -> the stores complete and visible "
         "device-wide: the span of one tile's stores from acceptance to completion;",
         "* Q-loop: a unit's stage loop.\n"]
    for d in docs:
        sh = d["shape"]
        L.append(f"## {d['workload']} (B={sh['B']}, H={sh['H']}, S={sh['S']}, D={sh['D']}, "
                 f"P={sh['P']}{', block mask' if d['masked'] else ''})\n")
        cm = d["call_ms_median"]
        L.append("Whole call, median of alternated HIP-event timings: " + ", ".join(
            f"{m} {cm[m]:.4f} ms" for m in ("product", "piggyback", "ordered", "coupled")) +
            f" (coupled {100 * (cm['coupled'] / cm['piggyback'] - 1):+.1f} % against piggyback).\n")
        L.append("| form | launch | Q-loop | issue span | held | to start | drain |")
        L.append("|---|---|---|---|---|---|---|")
        for m in ("piggyback", "ordered", "coupled"):
            md = d["modes"][m]
            assert md["output_equals_product"]
            for ln, lname in (("first_launch", "whole tiles" if not d["masked"] else "masked tiles"),
                              ("second_launch", "split half tiles")):
                if ln not in md:
                    continue
                x = md[ln]

                def c(k):
                    s = x.get(k, {"n": 0})
                    return "-" if not s["n"] else f"{s['p50_cyc']:.0f} / {s['p90_cyc']:.0f}"
                L.append(f"| {m} | {lname} | {c('q_loop')} | {c('issue_span')} | "
                         f"{c('resume_wait')} | {c('start_gap')} | {c('drain')} |")
        L.append("\nOutputs of all three forms equal the product kernel's bit for bit.\n")
    return "\n".join(L) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="video")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--out", default=None)
    ap.add_argument("--summarize", nargs="+", default=None, metavar="FILE",
                    help="print the markdown summary of result files written with --out")
    a = ap.parse_args()
    if a.summarize:
        docs = [json.load(open(f)) for f in a.summarize]
        cmd = "\n".join(f"python -m flashattention_output_re_amd.tile_stamps --workload "
                         f"{d['workload']} --reps {d['reps']} --out {f}"
                         for d, f in zip(docs, a.summarize))
        print(summarize(docs, cmd), end="")
        return
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    binding.load_library()
    res = measure(a.workload, a.reps)
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
