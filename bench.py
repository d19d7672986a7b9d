"""Throughput of the fused attention + Ulysses slab re-layout on one MI355X.

One step = one launch of the fused kernel over the whole workload (every
output tile: Q-loop over K/V tiles, online softmax, PV, slab-store epilogue),
inputs already resident in HBM.  Default workload: the long video share
(B=1, H=5, S=75600 tokens of a 21x60x60 latent, D=128, P=8 slabs), the
largest configuration and the long-sequence case the throughput target is
stated for; the Video-DiT share (S=32760) is also timed and reported under
"also".

Prints one JSON line on stdout.  Besides the headline TFLOP/s it reports:
  * roofline: the fused kernel's algorithmic FLOP per launch over its mean
    launch time (HIP events on the launch stream) against the bf16 dense MFMA
    peak; `traffic` comes from the committed rocprofv3 counter summary when it
    was taken on the current kernel source, else null;
  * fused_store_overhead_pct: median fused / median plain-output time - 1,
    from alternating launches of the same kernel writing [B][H][S][D];
  * cpu_baseline: the float64 CPU oracle timed on a bounded sample of the
    same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_SCLK_MHZ = 2400.0        # the clock that peak is quoted at
EXP_PER_CLK = 256 * 4 * 4     # v_exp_f32 results per clock, whole chip
LDS_B_PER_CLK_CU = 260.0      # measured LDS read rate per CU
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["flashattention_output_re_amd/csrc/fa_fwd_kernel.hip",
                  "flashattention_output_re_amd/csrc/fa_fwd_kernel.h"]
WORKLOAD_KEYS = {"video": "video-dit-share", "long": "long-video-share",
                 "image": "image-dit-share", "sparse": "block-sparse-video", "tiny": "tiny",
                 "video64": "video-dit-share-d64"}


# What one fused call launches on its stream (the roofline's "launch" is that
# call: HIP events bracket it).  Dense, with a workspace: the kernel over
# whole 256-query tiles, its last, partial round cut into key pieces -- at
# least one full round before a last round at least half full: the full
# rounds round-robin, the rest handed out from a counter, the last round's
# tiles in pieces of falling length (a counter reset launch goes first);
# otherwise the round spread over every CU, or run as split-key half tiles
# cut into pieces -- then the merge launch of the pieces' partial results.
# Dense without a workspace: the kernel over whole tiles plus, when the last
# round would fill at most half of the CUs, a second launch of its split-key
# form for that round.  Masked: one launch of the split-key form over
# 128-query tiles (one mask row each).
def kernel_label(D: int, dense: bool, tail_spread: bool = False) -> str:
    if dense and tail_spread:
        return (f"fa_fwd_pp_kernel<{D}, Slab> (whole 256-query tiles; the last round in key "
                "pieces: handed out from a counter after full round-robin rounds, else spread "
                "over every CU or as split-key half-tile pieces) + merge kernel (the pieces' "
                "partial results)")
    if dense:
        return (f"fa_fwd_pp_kernel<{D}, Slab> (whole 256-query tiles; split-key half tiles "
                "for a short last round)")
    return f"fa_fwd_pp_kernel<{D}, Slab, masked> (split-key 128-query tiles, kept mask tiles only)"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_prefix(workload: str) -> str:
    """File-name stem of a workload's rocprofv3 summaries under profiles/: the
    kernel, then the workload."""
    return f"fa_fwd_pp_{workload}"


def load_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{profile_prefix(workload)}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(name: str, target_s: float):
    """Time the float64 oracle on a fixed sample: consecutive 128-query row
    blocks of head 0, then head 1, ..., until about target_s seconds."""
    import numpy as np
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    w = wl.WORKLOADS[name]
    inp = wl.make(name)
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    nblk = (w.S + 127) // 128
    done_rows, blocks, heads = 0, 0, set()
    t0 = time.perf_counter()
    el = 0.0
    for h in range(w.H):
        mask = None if inp.mask is None else inp.mask[h:h + 1]
        for i in range(nblk):
            rows = np.arange(128 * i, min(w.S, 128 * i + 128))
            oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], w.scale, mask, rows=rows)
            done_rows += len(rows)
            blocks += 1
            heads.add(h)
            el = time.perf_counter() - t0
            if el >= target_s:
                break
        if el >= target_s:
            break
    flop = 4.0 * w.B * done_rows * w.S * w.D     # the oracle scores every key, masked ones too
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{name}: {blocks} blocks of 128 query rows ({done_rows} rows, heads "
                      f"{min(heads)}-{max(heads)}) against all {w.S} keys, float64 numpy, "
                      f"{el:.1f} s"}


class ClockSampler:
    """Shader clock of the GPU torch uses while it runs the fused kernel, read
    through amdsmi (per-XCD current GFX clocks, averaged).  The driver refreshes
    these metrics only every few hundred milliseconds, so `window()` keeps the
    GPU busy with back-to-back calls for about `seconds` and keeps the samples
    from its second half.  Reports nothing if amdsmi cannot see the device."""

    def __init__(self):
        self.handle, self.error, self.samples = None, None, []
        try:
            import amdsmi
            import torch
            self._amdsmi = amdsmi
            amdsmi.amdsmi_init()
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
                if int(bdf.split(":")[1], 16) == bus:
                    self.handle = h
            if self.handle is None:
                self.error = f"no amdsmi device on PCI bus {bus:#x}"
        except Exception as e:  # noqa: BLE001 - the clock is reported, not required
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        xcd = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        if xcd:
            return sum(xcd) / len(xcd)
        c = m.get("current_gfxclk")
        return float(c) if isinstance(c, (int, float)) and c > 0 else None

    def window(self, call, launch_s: float, seconds: float = 1.5, max_calls: int = 30000):
        import threading
        import torch
        if self.handle is None:
            return
        n = max(1, min(max_calls, int(seconds / max(launch_s, 1e-6))))
        stop = threading.Event()
        t_start = time.perf_counter()
        span = n * launch_s

        def run():
            while not stop.is_set():
                try:
                    c = self._read()
                except Exception as e:  # noqa: BLE001
                    self.error = f"{type(e).__name__}: {e}"
                    return
                if c is not None and time.perf_counter() - t_start > 0.5 * span:
                    self.samples.append(c)
                stop.wait(0.02)

        for _ in range(n):
            call()
        th = threading.Thread(target=run, daemon=True)
        th.start()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        try:
            self._amdsmi.amdsmi_shut_down()
        except Exception:  # noqa: BLE001
            pass

    def summary(self, achieved_tflops: float):
        import numpy as np
        if not self.samples:
            return {"sclk_mhz": None, "samples": 0, "error": self.error}
        mhz = float(np.median(self.samples))
        adj = PEAK_TFLOPS * mhz / PEAK_SCLK_MHZ
        return {"sclk_mhz": round(mhz, 1),
                "sclk_mhz_min_max": [round(min(self.samples), 1), round(max(self.samples), 1)],
                "samples": len(self.samples),
                "source": "amdsmi per-XCD current GFX clock, mean over XCDs, sampled over the "
                          "second half of a ~1.5 s run of back-to-back fused calls",
                "clock_adjusted_peak_tflops": round(adj, 1),
                "frac_of_clock_adjusted_peak": round(achieved_tflops / adj, 4)}


def secondary_bounds(flop: float, D: int, launch_s: float, sclk_mhz):
    """Rates of the two other resources the kernel leans on, per fused call.
    exp2: one per score, B*H*S^2 dense (flop / (4 D) in general), against the
    transcendental unit's rate of 4 results per clock per SIMD (a wave's
    v_exp_f32 occupies it 16 clocks): 256 CUs x 4 SIMDs x 4 = 4096 per clock.
    LDS: every 32x32x16 MFMA (32768 FLOP) reads one 1 KiB operand from LDS
    (K for QK^T, V through the transposing read for PV), flop / 32 bytes,
    against ~260 B per clock per CU, the rate an in-bounds probe sustained."""
    n_exp = flop / (4.0 * D)
    lds = flop / 32.0
    out = {"exp2_count": n_exp, "exp2_per_s": round(n_exp / launch_s, 1),
           "exp2_frac_of_peak_2400MHz": round(n_exp / launch_s / (EXP_PER_CLK * 2.4e9), 4),
           "lds_read_bytes": lds, "lds_read_TBps": round(lds / launch_s / 1e12, 2),
           "lds_frac_of_measured_2400MHz": round(lds / launch_s / (LDS_B_PER_CLK_CU * 256 * 2.4e9), 4)}
    if sclk_mhz:
        f = sclk_mhz * 1e6
        out["exp2_frac_at_sclk"] = round(n_exp / launch_s / (EXP_PER_CLK * f), 4)
        out["lds_frac_at_sclk"] = round(lds / launch_s / (LDS_B_PER_CLK_CU * 256 * f), 4)
    return out


def copy_calibration(mib: int):
    """One device copy of a known size: the HBM-traffic counters read for it
    calibrate FETCH_SIZE / WRITE_SIZE (bytes moved = mib MiB each way)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def summarize(kind: str, path: str):
    """Print a short text summary of rocprofv3 CSV output under `path`."""
    import csv
    import glob
    import statistics
    if kind == "trace":
        files = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
        for f in files:
            rows = list(csv.DictReader(open(f)))
            print(f"# {os.path.relpath(f, path)}")
            print("| kernel | calls | total ns | average ns | min ns | max ns | % |")
            print("|---|---|---|---|---|---|---|")
            for r in rows:
                print(f"| {r['Name']} | {r['Calls']} | {r['TotalDurationNs']} | "
                      f"{float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                      f"{float(r['Percentage']):.2f} |")
    else:
        files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
        per = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                key = (r["Kernel_Name"], r["Counter_Name"])
                per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
                per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        print("| kernel | counter | dispatches | mean per dispatch |")
        print("|---|---|---|---|")
        for (kname, cname), d in sorted(per.items()):
            print(f"| {kname} | {cname} | {len(d)} | {statistics.mean(d.values()):.6g} |")


def _counter_means(path: str) -> dict:
    """{(kernel, counter): mean over dispatches} from rocprofv3 --pmc CSV output."""
    import csv
    import glob
    import statistics
    per = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: statistics.mean(v.values()) for k, v in per.items()}


def write_profile_report(workload: str, d: str):
    """Write profiles/<kernel>_<workload>_{kernel_trace.md,counters.md,counters.json}
    from the rocprofv3 output directories that the commands printed in them
    leave under `d` (trace_<w>, pmc_{FETCH_SIZE,WRITE_SIZE,sq1,sq2}_<w>) and the
    bench.py JSON line in d/bench_<w>.json."""
    import contextlib
    import csv
    import glob
    import io
    import numpy as np
    import workloads as wl
    w = wl.WORKLOADS[workload]
    keep = wl.tile_mask_bool(w.H, w.S, w.keep_prob, w.seed) if w.keep_prob is not None else None
    flop = wl.flop_count(w.B, w.H, w.S, w.D, keep)
    stem = os.path.join(ROOT, "profiles", profile_prefix(workload))
    short = (f"python bench.py --workload {workload} --steps 30 --warmup 10 --overhead-pairs 4 "
             "--no-cpu-baseline --no-clock --also none")
    sq1 = ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
           "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_MISC")
    sq2 = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS "
           "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE")

    def summary(kind, sub):
        buf = io.StringIO()
        with contextlib.redirect_stdout(buf):
            summarize(kind, os.path.join(d, sub))
        return buf.getvalue()

    def fused_only(text):
        return "\n".join(l for l in text.splitlines()
                         if "(fa::StoreMode)1" not in l and "relayout_kernel" not in l
                         and "elementwise" not in l and "copyBuffer" not in l
                         and "fillBuffer" not in l)

    stats_f = glob.glob(os.path.join(d, f"trace_{workload}", "**", "*kernel_stats.csv"), recursive=True)[0]
    stats = {r["Name"]: r for r in csv.DictReader(open(stats_f))}
    def flags(n):   # template arguments after StoreMode: NEG, SPLIT, MASKED, SLAB_IN, INSTR
        return [x.strip() for x in n.split("(fa::StoreMode)")[1].split(">")[0].split(",")[1:]]

    def product(n):                # not a timestamped instance
        f = flags(n)
        return len(f) < 5 or f[4] == "0"

    fwd = [n for n in stats if "fa_fwd" in n]
    fused = sorted([n for n in fwd if "(fa::StoreMode)0" in n and product(n)
                    and flags(n)[3] == "false"] +
                   [n for n in stats if "fa_merge" in n and "(fa::StoreMode)0" in n] +
                   [n for n in stats if "fa_queue_reset" in n])
    slab_in = sorted(n for n in fwd if product(n) and flags(n)[3] == "true")
    avg_s = {n: float(stats[n]["AverageNs"]) * 1e-9 for n in fused}
    call_s = sum(avg_s.values())
    bj = json.loads(open(os.path.join(d, f"bench_{workload}.json")).read().strip().splitlines()[-1])
    fe, wr = _counter_means(os.path.join(d, f"pmc_FETCH_SIZE_{workload}")), \
        _counter_means(os.path.join(d, f"pmc_WRITE_SIZE_{workload}"))
    c1, c2 = _counter_means(os.path.join(d, f"pmc_sq1_{workload}")), \
        _counter_means(os.path.join(d, f"pmc_sq2_{workload}"))
    copy = next(k for (k, c) in fe if "copyBuffer" in k)
    fscale = 1024.0 * 1024 / fe[(copy, "FETCH_SIZE")]        # the 1 GiB copy reads 1 GiB
    wscale = 1024.0 * 1024 / wr[(copy, "WRITE_SIZE")]
    fetch_b = {n: fe[(n, "FETCH_SIZE")] * 1024 * fscale for n in fused}
    write_b = {n: wr[(n, "WRITE_SIZE")] * 1024 * wscale for n in fused}
    bytes_call = sum(fetch_b.values()) + sum(write_b.values())
    min_bytes = 4.0 * w.B * w.H * w.S * w.D * 2
    hsh = kernel_source_hash()
    title = {"video": "Video-DiT share", "long": "long video share", "image": "Image-DiT share",
             "sparse": "block-sparse video", "tiny": "tiny case",
             "video64": "Video-DiT share at D = 64"}[workload]
    shape = f"B={w.B}, H={w.H}, S={w.S}, D={w.D}, P={w.P}" + (
        f", {100 * float(keep.mean()):.1f}% of 128x128 tiles kept" if keep is not None else "")

    tr = [f"# Fused kernel on the {title} ({shape}): kernel trace\n",
          "Command (from the repository root, after `python -m flashattention_output_re_amd.build`):\n",
          "```",
          f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_{workload} -o run -- {short}",
          f"python bench.py --summarize trace {d}/trace_{workload}",
          "```\n",
          f"Kernel source sha256/16: {hsh}. StoreMode 0 = slab (fused re-layout), 1 = plain "
          "[B][H][S][D] (the overhead twin and the serial baseline's attention). Template "
          "arguments of fa_fwd_pp_kernel after StoreMode: negative scale, split-key units, masked "
          "units, slab-layout inputs, timestamped instance (false, false for the middle two: whole "
          "256-query tiles; true, false: split-key half tiles of a short last round, a second launch "
          "on the same stream; true, true: masked 128-query tiles). `fa_merge_kernel`: the merge "
          "of a dense call's last-round key pieces (the workspace entry points: pieces handed out "
          "from a counter, or stage slices spread over every CU); `fa_merge_split_kernel`: the "
          "merge of split half tiles cut into key pieces; `fa_queue_reset_kernel`: the one-thread "
          "launch that zeroes the dynamic schedule's counter. `relayout_kernel<16>`: the serial "
          "baseline's standalone copy.\n",
          summary("trace", f"trace_{workload}"),
          f"One fused call = {' + '.join(f'{avg_s[n] * 1e3:.4f}' for n in fused)} = {call_s * 1e3:.4f} ms "
          f"under the tracer; {flop:.4g} algorithmic FLOP per call -> {flop / call_s / 1e12:.1f} TFLOP/s "
          f"(bench.py, HIP events around the call: {bj['roofline']['mean_launch_ms']:.4f} ms, "
          f"{bj['roofline']['achieved']:.1f} TFLOP/s)."]
    if slab_in and "slab_to_slab" in bj:
        ms_in = [float(stats[n]["AverageNs"]) * 1e-6 for n in slab_in]
        t_s = sum(ms_in) * 1e-3
        tr.append(f"\nSlab-layout inputs (attn_fwd_slab_to_slab, last template flag true): "
                  f"{' + '.join(f'{x:.4f}' for x in ms_in)} "
                  f"= {t_s * 1e3:.4f} ms per call under the tracer, {flop / t_s / 1e12:.1f} TFLOP/s "
                  f"(bench.py: {bj['slab_to_slab']['median_ms']:.4f} ms, "
                  f"{bj['slab_to_slab']['overhead_vs_fused_pct']:+.2f}% against the fused call).")
    with open(f"{stem}_kernel_trace.md", "w") as f:
        f.write("\n".join(tr) + "\n")

    cm = [f"# Fused kernel on the {title} ({shape}): hardware counters\n",
          "Commands (one rocprofv3 pass each; the FETCH/WRITE passes also run one 1 GiB device copy "
          "for calibration):\n", "```"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cm.append(f"rocprofv3 --pmc {c} --output-format csv -d {d}/pmc_{c}_{workload} -o run -- "
                  f"{short} --copy-calibration-mib 1024")
    cm.append(f"rocprofv3 --pmc {sq1} --kernel-include-regex fa_ --output-format csv "
              f"-d {d}/pmc_sq1_{workload} -o run -- {short}")
    cm.append(f"rocprofv3 --pmc {sq2} --kernel-include-regex fa_ --output-format csv "
              f"-d {d}/pmc_sq2_{workload} -o run -- {short}")
    cm.append(f"python bench.py --summarize counters <dir>   # for each directory above")
    cm.append(f"python bench.py --summarize report:{workload} {d}   # this file")
    cm.append("```\n")
    cm.append(f"Kernel source sha256/16: {hsh}. Rows of the plain-layout twin (StoreMode 1) and of "
              "other kernels omitted.\n")
    cm.append("## HBM traffic (KiB per dispatch)\n")
    cm.append(fused_only(summary("counters", f"pmc_FETCH_SIZE_{workload}")) + "\n")
    cm.append(fused_only(summary("counters", f"pmc_WRITE_SIZE_{workload}")) + "\n")
    cm.append("## SQ counters (per dispatch, summed over the chip)\n")
    cm.append(fused_only(summary("counters", f"pmc_sq1_{workload}")) + "\n")
    cm.append(fused_only(summary("counters", f"pmc_sq2_{workload}")) + "\n")
    cm.append("## Derived figures\n")
    cm.append(f"* Calibration: the 1 GiB device copy reads FETCH_SIZE = {fe[(copy, 'FETCH_SIZE')]:.0f} KiB "
              f"and WRITE_SIZE = {wr[(copy, 'WRITE_SIZE')]:.0f} KiB, so bytes fetched = {fscale:.3f} x "
              f"FETCH_SIZE KiB x 1024 and bytes written = {wscale:.3f} x WRITE_SIZE KiB x 1024.")
    cm.append(f"* HBM bytes per fused call: {bytes_call / 1e6:.1f} MB (fetched "
              f"{sum(fetch_b.values()) / 1e6:.1f}, written {sum(write_b.values()) / 1e6:.1f}) against "
              f"{min_bytes / 1e6:.1f} MB algorithmic (q, k, v read once, output written once); "
              f"{bytes_call / call_s / 1e12:.3f} TB/s over the call, "
              f"{100 * bytes_call / call_s / (HBM_PEAK_GBS * 1e9):.1f}% of 8 TB/s.")
    n_mfma = sum(c2.get((n, "SQ_INSTS_MFMA"), 0.0) for n in fused)
    if n_mfma:
        cm.append(f"* SQ_INSTS_MFMA over the call x 32768 FLOP per 32x32x16 MFMA = {n_mfma * 32768:.4g} "
                  f"FLOP issued against {flop:.4g} algorithmic ({100 * (n_mfma * 32768 / flop - 1):+.1f}%: "
                  "keys padded to 64-key stages, the unused QK^T of the stage past the end, and for "
                  "masked calls the 128-key tiles kept but partly outside the sequence).")
    for n in fused:
        short_n = n.split("(fa::FwdParams)")[0].replace("void fa::", "")
        grbm = c2.get((n, "GRBM_GUI_ACTIVE"))
        busy = c2.get((n, "SQ_VALU_MFMA_BUSY_CYCLES"))
        if grbm is None or busy is None:
            continue
        cyc = grbm / 8.0
        clk = cyc / avg_s[n]
        mf = busy / 1024.0
        co = c2[(n, "SQ_VALU_MFMA_COEXEC_CYCLES")] / busy if busy else 0.0
        cm.append(f"* `{short_n}`: {avg_s[n] * 1e3:.4f} ms per dispatch; GRBM_GUI_ACTIVE / 8 XCDs = "
                  f"{cyc:.4g} cycles -> {clk / 1e9:.2f} GHz held; matrix cores busy "
                  f"{100 * mf / cyc:.1f}% of those cycles per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024 "
                  f"SIMDs); VALU co-issued in {100 * co:.0f}% of MFMA cycles; "
                  f"SQ_LDS_BANK_CONFLICT = {c2[(n, 'SQ_LDS_BANK_CONFLICT')]:.0f}; fetched "
                  f"{fetch_b[n] / 1e6:.1f} MB, written {write_b[n] / 1e6:.1f} MB.")
    with open(f"{stem}_counters.md", "w") as f:
        f.write("\n".join(cm) + "\n")
    rec = {"workload": workload, "kernel_source_sha256_16": hsh,
           "kernels": {n: {"avg_ms": avg_s[n] * 1e3, "fetch_size_kib": fe[(n, "FETCH_SIZE")],
                           "write_size_kib": wr[(n, "WRITE_SIZE")]} for n in fused},
           "fetch_scale": fscale, "write_scale": wscale, "hbm_bytes_per_launch": round(bytes_call),
           "launch": "one fused call: every StoreMode-0 kernel it launches",
           "source": os.path.relpath(f"{stem}_counters.md", ROOT)}
    with open(f"{stem}_counters.json", "w") as f:
        json.dump(rec, f, indent=1)
    print(f"{stem}: {bytes_call:.0f} bytes per call, {call_s * 1e3:.4f} ms")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long", choices=sorted(WORKLOAD_KEYS))
    ap.add_argument("--no-workspace", action="store_true",
                    help="time the entry points without a workspace (last round as split "
                         "half tiles) instead of the _ws_ ones")
    ap.add_argument("--also", default="video",
                    help="comma-separated workloads also timed (fused call only), or none")
    ap.add_argument("--overhead-pairs", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the ~1.5 s shader-clock sampling window (profiler runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB")
    ap.add_argument("--summarize", nargs=2, metavar=("KIND", "DIR"),
                    help="print a summary of rocprofv3 CSV output (KIND: trace|counters), or "
                         "write a workload's profiles/ summaries (KIND: report:<workload>)")
    a = ap.parse_args()
    if a.summarize:
        kind, path = a.summarize
        if kind.startswith("report:"):
            write_profile_report(kind.split(":", 1)[1], path)
        else:
            summarize(kind, path)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU leg "
              "(the head-to-sequence exchange is stored into local slabs); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import flashattention_output_re_amd as fa
    import workloads as wl

    fa.load_library()
    w = wl.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    inp = wl.make(a.workload)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    mask = None
    keep = None
    if inp.mask is not None:
        mask = torch.from_numpy(inp.mask.view(np.int64)).to(dev)
        keep = wl.tile_mask_bool(w.H, w.S, w.keep_prob, w.seed)
    flop = wl.flop_count(w.B, w.H, w.S, w.D, keep)
    slabs = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device=dev)
    plain = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    # The workspace entry points (the dense tail round spread over every CU,
    # its partial results merged by a second launch), workspace allocated
    # here, outside the timed region.
    ws_bytes = 0 if a.no_workspace else fa.attn_fwd_workspace_bytes(w.B, w.H, w.S, w.D)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def fused():
        if a.no_workspace:
            fa.attn_fwd_relayout_async(q, k, v, slabs, w.B, w.H, w.S, w.D, w.P, w.scale, mask,
                                       stream)
        else:
            fa.attn_fwd_relayout_ws_async(q, k, v, slabs, w.B, w.H, w.S, w.D, w.P, w.scale, mask,
                                          ws, stream)

    def plain_out():
        if a.no_workspace:
            fa.attn_fwd_plain_async(q, k, v, plain, w.B, w.H, w.S, w.D, w.scale, mask, stream)
        else:
            fa.attn_fwd_plain_ws_async(q, k, v, plain, w.B, w.H, w.S, w.D, w.scale, mask, ws,
                                       stream)

    for _ in range(a.warmup):
        fused()
        plain_out()
    torch.cuda.synchronize()

    # ---- timed region: exactly K fused steps, per-launch HIP events.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(a.steps):
        fused()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)]
    ms_step = wall * 1e3 / a.steps
    mean_launch_ms = float(np.mean(launch_ms))
    tflops = flop / (ms_step * 1e-3) / 1e12

    # ---- fused-store overhead: alternating fused / plain launches.
    fus, pla = [], []
    for i in range(a.overhead_pairs):
        order = (fused, plain_out) if i % 2 == 0 else (plain_out, fused)
        for fn in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            (fus if fn is fused else pla).append(e0.elapsed_time(e1))
    med_f, med_p = float(np.median(fus)), float(np.median(pla))
    overhead = (med_f / med_p - 1.0) * 100.0
    rng = np.random.default_rng(0)
    boot = []
    fa_, pa_ = np.array(fus), np.array(pla)
    for _ in range(2000):
        boot.append(np.median(rng.choice(fa_, fa_.size)) / np.median(rng.choice(pa_, pa_.size)))
    ci = [float((np.percentile(boot, 2.5) - 1) * 100), float((np.percentile(boot, 97.5) - 1) * 100)]

    # ---- serial baseline: plain-layout attention, then the standalone
    # re-layout copy (the one-GPU form of attention followed by a separate
    # exchange), same stream, K steps; and the copy alone.
    slabs2 = torch.empty_like(slabs)

    def copy():
        fa.relayout_to_slabs_async(plain, slabs2, w.B, w.H, w.S, w.D, w.P, stream)

    def timed(fn, n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(n):
            fn()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(n)]))

    for _ in range(2):
        plain_out()
        copy()
    serial_ms = timed(lambda: (plain_out(), copy()), a.steps)
    copy_ms = timed(copy, a.steps)
    copy_bytes = 2.0 * w.B * w.H * w.S * w.D * 2

    # ---- both exchanges fused: Q, K, V arrive in the sequence-sharded slab
    # layout (before the pre-attention exchange) and are read from there by
    # the same kernel; alternated with the standard fused call.
    Sp = w.S // w.P
    qs, ks, vs = (t.view(w.B, w.H, w.P, Sp, w.D).permute(2, 0, 3, 1, 4).contiguous()
                  for t in (q, k, v))
    slabs3 = torch.empty_like(slabs)

    def slab_in():
        if a.no_workspace:
            fa.attn_fwd_slab_to_slab_async(qs, ks, vs, slabs3, w.B, w.H, w.S, w.D, w.P, w.scale,
                                           mask, stream)
        else:
            fa.attn_fwd_slab_to_slab_ws_async(qs, ks, vs, slabs3, w.B, w.H, w.S, w.D, w.P,
                                              w.scale, mask, ws, stream)

    for _ in range(2):
        slab_in()
    s2s, ref = [], []
    for i in range(a.overhead_pairs):
        order = (fused, slab_in) if i % 2 == 0 else (slab_in, fused)
        for fn in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            (s2s if fn is slab_in else ref).append(e0.elapsed_time(e1))
    med_s2s, med_ref = float(np.median(s2s)), float(np.median(ref))
    sa, ra = np.array(s2s), np.array(ref)
    boot2 = [np.median(rng.choice(sa, sa.size)) / np.median(rng.choice(ra, ra.size))
             for _ in range(2000)]
    del qs, ks, vs, slabs3

    # ---- other workloads, fused call only (inputs resident, same timing).
    also = {}
    for name in [x for x in a.also.split(",") if x and x not in ("none", a.workload)]:
        ow = wl.WORKLOADS[name]
        oi = wl.make(name)
        oq, ok_, ov = (t.to(dev) for t in (oi.q, oi.k, oi.v))
        om, okeep = None, None
        if oi.mask is not None:
            om = torch.from_numpy(oi.mask.view(np.int64)).to(dev)
            okeep = wl.tile_mask_bool(ow.H, ow.S, ow.keep_prob, ow.seed)
        oflop = wl.flop_count(ow.B, ow.H, ow.S, ow.D, okeep)
        oslabs = torch.empty((ow.P, ow.B, ow.S // ow.P, ow.H, ow.D), dtype=torch.bfloat16,
                             device=dev)
        ows_bytes = 0 if a.no_workspace else fa.attn_fwd_workspace_bytes(ow.B, ow.H, ow.S, ow.D)
        ows = torch.empty(max(ows_bytes, 16), dtype=torch.uint8, device=dev)

        def ofused():
            fa.attn_fwd_relayout_ws_async(oq, ok_, ov, oslabs, ow.B, ow.H, ow.S, ow.D, ow.P,
                                          ow.scale, om, ows, stream)

        for _ in range(3):
            ofused()
        oms = timed(ofused, max(10, a.steps // 2))
        also[name] = {"workload": WORKLOAD_KEYS[name], "mean_launch_ms": round(oms, 4),
                      "TFLOPs": round(oflop / (oms * 1e-3) / 1e12, 2),
                      "frac_of_peak": round(oflop / (oms * 1e-3) / 1e12 / PEAK_TFLOPS, 4)}
        del oq, ok_, ov, oslabs, om

    achieved = flop / (mean_launch_ms * 1e-3) / 1e12
    traffic = load_traffic(a.workload)
    clk = {"sclk_mhz": None, "samples": 0, "error": "not sampled (--no-clock)"}
    if not a.no_clock:
        clock = ClockSampler()
        clock.window(fused, mean_launch_ms * 1e-3)
        clk = clock.summary(achieved)
    out = {
        "metric": "fused attn+relayout TFLOP/s at 1 GPU; % bf16 MFMA peak; fused-store overhead %",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_KEYS[a.workload], "B": w.B, "H": w.H, "S": w.S,
                   "D": w.D, "P": w.P, "scale": w.scale, "seed": w.seed,
                   "mask_density": None if keep is None else float(keep.mean()),
                   "algorithmic_flop": flop},
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS, 2),
        "fused_store_overhead_pct": round(overhead, 2),
        "fused_store_overhead_ci95": [round(c, 2) for c in ci],
        "median_ms": {"fused": round(med_f, 4), "plain": round(med_p, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": kernel_label(w.D, mask is None, ws_bytes > 0),
                     "mean_launch_ms": round(mean_launch_ms, 4),
                     "launch_ms_p10_p50_p90": [round(float(np.percentile(launch_ms, x)), 4)
                                               for x in (10, 50, 90)]},
        "clock": clk,
        "secondary_bounds": secondary_bounds(flop, w.D, mean_launch_ms * 1e-3, clk.get("sclk_mhz")),
        "kernel_source_sha256_16": kernel_source_hash(),
        "serial_baseline": {
            "what": "plain-layout attention, then the standalone re-layout copy (relayout_to_slabs)",
            "ms_per_step": round(serial_ms, 4),
            "relayout_copy_ms": round(copy_ms, 4),
            "relayout_copy_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
            "relayout_copy_frac_of_8TBps": round(copy_bytes / (copy_ms * 1e-3) / 8e12, 4),
            "speedup_fused_over_serial": round(serial_ms / mean_launch_ms, 4),
        },
        "also": also,
        "workspace_bytes": ws_bytes,
        "slab_to_slab": {
            "what": "attn_fwd_slab_to_slab (its _ws_ form unless --no-workspace): q, k, v read "
                    "from [P][B][S/P][H][D] slabs (the pre-attention exchange fused into the "
                    "loads) and the output stored into slabs",
            "median_ms": round(med_s2s, 4),
            "TFLOPs": round(flop / (med_s2s * 1e-3) / 1e12, 2),
            "overhead_vs_fused_pct": round((med_s2s / med_ref - 1.0) * 100.0, 2),
            "overhead_ci95": [round(float((np.percentile(boot2, x) - 1) * 100), 2) for x in (2.5, 97.5)],
        },
    }
    if a.copy_calibration_mib:
        copy_calibration(a.copy_calibration_mib)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a.workload, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
