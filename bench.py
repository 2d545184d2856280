#!/usr/bin/env python3
"""Benchmark of the exact-attention backward on one MI355X.

Workload: causal bf16 attention backward at B=8, H=16, N=4096, d=128 (the shape
and FLOP convention of "Writing Speed-of-Light Attention Backward Kernel for
5090 in CUDA", sections "Setup" and Appendix C), seeded synthetic N(0,1)
inputs.  One timed step is the whole backward of the method: the preprocess
D = rowsum(dO o O) plus attn_bwd (every kernel it launches).  O and L come
from this library's forward, run once before the timed region; the forward is
also timed on its own and reported beside it.

Prints ONE JSON line.  Effective TFLOPS = 10*B*H*N^2*d*(1/2 if causal) / time.
`value` is the mean over the K timed steps (total time / K); the per-step
times (one HIP event between consecutive steps) give the median and p10/p90.

    python bench.py [--steps K] [--warmup W] [--config headline|noncausal|...]
    python bench.py --profile OUT [--config ...]   # rocprofv3 trace + counters
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E (published)
PAGES_BWD_TFLOPS = 160.06        # the pages' v3 backward at the headline workload (RTX 5090; context)
PAGES_SPARSE_MS = 1.533          # the pages' sparse top-k backward (B200; context)
CSRC = os.path.join(ROOT, "exact_attention_bwd_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# ----------------------------------------------------------------------------
# FLOP / byte conventions (attention-backward page "Setup" and Appendix C;
# the forward count is the 4*B*H*N^2*d of the flash_attention_cuda README table;
# the sparse count 2*H*N*topk*(3*d_qk + 2*d_v) reproduces every row of the
# cudnn-frontend PR #684 benchmark matrix)
# ----------------------------------------------------------------------------
def bwd_flops(B, H, N, d, causal):
    f = 10.0 * B * H * N * N * d
    return f * 0.5 if causal else f


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f * 0.5 if causal else f


def sparse_bwd_flops(H, N, topk, dqk, dv):
    return 2.0 * H * N * topk * (3 * dqk + 2 * dv)


def bwd_min_bytes(B, H, N, d):
    """Read Q, K, V, O, dO (bf16) and L (fp32) once, write dQ, dK, dV (bf16) once."""
    bhnd = B * H * N * d
    return {"read": 5 * bhnd * 2 + B * H * N * 4, "write": 3 * bhnd * 2}


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def dense_metric(cfg, hkv=None):
    """Metric label of a dense workload: the headline's words, with its own shape."""
    causal = "½ causal" if cfg.causal else "non-causal"
    gq = f" Hkv{hkv}" if hkv is not None and hkv != cfg.H else ""
    return (f"attn bwd effective TFLOPS (10·BHN²d{'·½ causal' if cfg.causal else ''}) & % bf16 MFMA peak, "
            f"B{cfg.B} H{cfg.H}{gq} N{cfg.N} d{cfg.d}" + ("" if cfg.causal else f" ({causal})"))


# The kernel that dominates a dense step, and the share of the conventional
# FLOP count it performs.  Causal d = 128 (grouped-query or not): the fused
# kernel forms all five products (S, dP, dV, dK, dQ); its timing events also
# cover the one-workgroup sweep launched after it.  Otherwise the dK/dV
# kernel forms S, dP, dV and dK (4 of the 5) and the dQ kernel the fifth.
def dominant_kernel(d, causal, gqa):
    if d == 128 and causal:
        return "bwd_fused_kernel", 1.0
    if d == 128:
        return "bwd_dkdv_w64_kernel", 0.8
    return "bwd_dkdv_kernel", 0.8


# ----------------------------------------------------------------------------
# HIP events through the runtime PyTorch loaded (same process, same runtime)
# ----------------------------------------------------------------------------
class HipEvents:
    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        st = self.rt.hipEventCreate(ctypes.byref(e))
        if st != 0:
            raise RuntimeError(f"hipEventCreate failed: {st}")
        return e.value

    def record(self, e, stream):
        st = self.rt.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_ms(self, a, b):
        self.rt.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        st = self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value

    def destroy(self, e):
        self.rt.hipEventDestroy(ctypes.c_void_p(e))


def _percentile(xs, p):
    s = sorted(xs)
    if not s:
        return None
    k = (len(s) - 1) * p / 100.0
    lo = int(k)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def timed_steps(ev, stream, step, K, main_events=True):
    """Run K steps with an event between consecutive steps (and, if
    `main_events`, a pair around the dominant kernel of each).  Returns
    (total ms, per-step ms list, dominant-kernel ms list)."""
    import torch
    marks = [ev.create() for _ in range(K + 1)]
    pairs = [(ev.create(), ev.create()) for _ in range(K)] if main_events else [None] * K
    torch.cuda.synchronize()
    ev.record(marks[0], stream)
    for i in range(K):
        step(pairs[i])
        ev.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    per = [ev.elapsed_ms(marks[i], marks[i + 1]) for i in range(K)]
    total = ev.elapsed_ms(marks[0], marks[K])
    main = [ev.elapsed_ms(a, b) for a, b in pairs] if main_events else []
    for e in marks:
        ev.destroy(e)
    for p in pairs:
        if p:
            ev.destroy(p[0])
            ev.destroy(p[1])
    return total, per, main


def step_stats(per):
    return {"median": round(_percentile(per, 50), 5), "p10": round(_percentile(per, 10), 5),
            "p90": round(_percentile(per, 90), 5), "min": round(min(per), 5), "max": round(max(per), 5)}


# ----------------------------------------------------------------------------
# Host and clock facts
# ----------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class SclkSampler:
    """Samples the current engine clock level of every GPU visible in sysfs
    (pp_dpm_sclk, the line marked '*') every few milliseconds while running."""

    def __init__(self, period_s=0.002):
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = {f: [] for f in self.files}
        self._stop = threading.Event()
        self._t = None

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            return int(m.group(1))
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for f in self.files:
                v = self._read(f)
                if v is not None:
                    self.samples[f].append(v)
            time.sleep(self.period)

    def __enter__(self):
        if self.files:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self._t:
            self._t.join()

    def summary(self):
        per = {}
        for f, v in self.samples.items():
            if v:
                card = f.split("/")[4]
                per[card] = {"median_mhz": _percentile(v, 50), "max_mhz": max(v), "samples": len(v)}
        if not per:
            return None
        busiest = max(per.values(), key=lambda x: x["median_mhz"])
        return {"source": "sysfs pp_dpm_sclk during the timed steps", "median_mhz": busiest["median_mhz"],
                "max_mhz": busiest["max_mhz"], "samples": busiest["samples"],
                "cards": len(per)}


# ----------------------------------------------------------------------------
# Profiles: rocprofv3 kernel trace and counter passes, summarised per kernel
# ----------------------------------------------------------------------------
COPY_BYTES = 1 << 30             # the calibration copy moves 1 GiB each way
SQ_PASS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_ANY",
           "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"]


HOST_ONLY_SOURCES = ("attn_api.hip", "attn_noalloc.hip", "api_error.hpp", "launch.hpp")


def sources_sha():
    """sha256 over the device-code sources: a profile taken on other kernels
    is stale (the host-side entry points do not count)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if p.endswith((".hip", ".hpp")) and os.path.basename(p) not in HOST_ONLY_SOURCES:
            with open(p, "rb") as f:
                h.update(os.path.basename(p).encode())
                h.update(f.read())
    return h.hexdigest()


def profile_path(config, ext):
    return os.path.join(PROFILES, f"{config}_profile.{ext}")


def profile_name(config, hkv):
    """Name of a workload's profile: the config, plus the K/V head count for
    grouped-query runs (a different kernel path than the config alone)."""
    return config if hkv is None else f"{config}_hkv{hkv}"


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, three times: the copy kernel
    reads and writes exactly COPY_BYTES, which scales the TCC byte counters."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES}), flush=True)


def short_kernel_name(name):
    """Readable kernel name from an Itanium-mangled or demangled symbol."""
    if name.startswith("_ZN"):
        s, i, parts = name, 3, []
        while i < len(s) and s[i].isdigit():
            j = i
            while s[j].isdigit():
                j += 1
            n = int(s[i:j])
            parts.append(s[j:j + n])
            i = j + n
        base = parts[-1] if parts else name
        args = []
        if i < len(s) and s[i] == "I":              # literal template arguments: L<type><value>E
            i += 1
            while i < len(s) and s[i] == "L":
                m = re.match(r"L([a-z])(n?\d+)E", s[i:])
                if not m:
                    break
                t, v = m.groups()
                args.append(("true" if v == "1" else "false") if t == "b" else v.replace("n", "-"))
                i += m.end()
        return base + ("<" + ", ".join(args) + ">" if args else "")
    m = re.search(r"([A-Za-z_]\w*(?:<[^()]*>)?)\s*\(", name)
    return m.group(1) if m else name[:60]


def _csv_rows(d, suffix):
    out = []
    for p in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(p) as f:
            out.extend(csv.DictReader(f))
    return out


def _per_kernel_counters(d):
    """{kernel: {counter: [value per dispatch]}} from a --pmc pass directory."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        k = short_kernel_name(r["Kernel_Name"])
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})[r.get("Dispatch_Id", len(acc))] = \
            float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in acc.items()}


def _mean(xs):
    return sum(xs) / len(xs) if xs else None


def _trace_durations(d, last):
    per = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        per.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = {}
    for k, v in per.items():
        v.sort()
        ds = [(e - s) / 1e3 for s, e in v]
        out[k] = {"calls": len(ds), "avg_us": _mean(ds), "avg_us_last": _mean(ds[-last:]),
                  "min_us": min(ds), "max_us": max(ds)}
    return out


def run_profile(out_dir, config, extra, name):
    """Kernel trace + counter passes of one workload, each under rocprofv3 in a
    child process of its own, then the per-kernel summary in profiles/."""
    out_dir = os.path.abspath(out_dir)
    os.makedirs(out_dir, exist_ok=True)
    me = [sys.executable, os.path.join(ROOT, "bench.py")]
    bench_args = ["--config", config, "--no-cpu-baseline", *extra]
    passes = [
        ("trace", 300, ["--kernel-trace", "--stats"], bench_args + ["--steps", "20", "--warmup", "20"]),
        ("sq", 120, ["--pmc", *SQ_PASS], bench_args + ["--steps", "3", "--warmup", "2"]),
        ("fetch", 120, ["--pmc", "FETCH_SIZE", "GRBM_COUNT"], bench_args + ["--steps", "3", "--warmup", "2"]),
        ("write", 120, ["--pmc", "WRITE_SIZE"], bench_args + ["--steps", "3", "--warmup", "2"]),
        ("cfetch", 120, ["--pmc", "FETCH_SIZE"], ["--copy-calibration"]),
        ("cwrite", 120, ["--pmc", "WRITE_SIZE"], ["--copy-calibration"]),
    ]
    commands = []
    env = dict(os.environ, TMPDIR="/tmp")
    meta = {"config": config, "source_sha256": sources_sha(), "commands": commands}
    for name, limit, prof, args in passes:
        cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", *prof, "--output-format", "csv",
               "-d", os.path.join(out_dir, name), "-o", name, "--", *me, *args]
        shown = " ".join(cmd).replace(out_dir, "OUT").replace(ROOT, "$REPO").replace(sys.executable, "python3")
        commands.append(shown)
        print(f"[profile] {name}: start", flush=True)
        with open(os.path.join(out_dir, f"{name}.log"), "w") as log:
            rc = subprocess.run(cmd, stdout=log, stderr=subprocess.STDOUT, cwd="/tmp", env=env).returncode
        print(f"[profile] {name}: rc={rc}", flush=True)
        if rc != 0:
            # rocprofv3 may end with a segmentation fault after the program and
            # its result files are complete; anything else stops the profile
            if not (rc in (139, -11) and _csv_rows(os.path.join(out_dir, name), ".csv")):
                return rc
    with open(os.path.join(out_dir, "meta.json"), "w") as f:
        json.dump(meta, f, indent=1)
    summarise_profile(out_dir, name)
    return 0


def summarise_profile(out_dir, config):
    """Per-kernel summary of a profile directory, keyed to the kernel sources
    it was taken on (OUT/meta.json), into profiles/ and OUT/."""
    with open(os.path.join(out_dir, "meta.json")) as f:
        meta = json.load(f)
    commands = meta["commands"]
    trace = _trace_durations(os.path.join(out_dir, "trace"), 20)
    sq = _per_kernel_counters(os.path.join(out_dir, "sq"))
    fe = _per_kernel_counters(os.path.join(out_dir, "fetch"))
    wr = _per_kernel_counters(os.path.join(out_dir, "write"))
    cf = _per_kernel_counters(os.path.join(out_dir, "cfetch"))
    cw = _per_kernel_counters(os.path.join(out_dir, "cwrite"))

    def copy_max(tab, counter):
        vals = [max(cs[counter]) for k, cs in tab.items() if "copyBuffer" in k and counter in cs]
        return max(vals) if vals else None

    cfetch, cwrite = copy_max(cf, "FETCH_SIZE"), copy_max(cw, "WRITE_SIZE")
    fscale = COPY_BYTES / (cfetch * 1024.0) if cfetch else None
    wscale = COPY_BYTES / (cwrite * 1024.0) if cwrite else None
    kernels = {}
    for k, t in trace.items():
        if "copyBuffer" in k or "fillBuffer" in k:
            continue
        row = {"calls_in_trace": t["calls"], "avg_us": round(t["avg_us_last"], 2),
               "min_us": round(t["min_us"], 2), "max_us": round(t["max_us"], 2)}
        c = {n: _mean(v) for n, v in sq.get(k, {}).items()}
        g = c.get("GRBM_GUI_ACTIVE")
        if g:
            cyc = g / 8.0
            row["cycles_sq_pass"] = round(cyc)
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
                row["mfma_busy_pct"] = round(100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024), 2)
            if c.get("SQ_LDS_IDX_ACTIVE"):
                row["lds_active_pct"] = round(100.0 * c["SQ_LDS_IDX_ACTIVE"] / (cyc * 256), 2)
                row["lds_bank_conflict_pct"] = round(
                    100.0 * c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"], 3)
            if c.get("SQ_WAVE_CYCLES"):
                row["wait_inst_any_pct"] = round(100.0 * c.get("SQ_WAIT_INST_ANY", 0.0) / c["SQ_WAVE_CYCLES"], 2)
            for n in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA"):
                if c.get(n) is not None:
                    row[n.lower()] = round(c[n])
        f = fe.get(k, {})
        if f.get("GRBM_COUNT"):
            cyc = _mean(f["GRBM_COUNT"]) / 8.0
            row["cycles"] = round(cyc)
            if t["avg_us_last"] >= 100:
                # under ~100 us the counter window outlasts the kernel
                row["clock_ghz_vs_trace_avg"] = round(cyc / (t["avg_us_last"] * 1e3), 3)
        if f.get("FETCH_SIZE") and fscale:
            row["hbm_read_bytes"] = round(_mean(f["FETCH_SIZE"]) * 1024.0 * fscale)
        w = wr.get(k, {})
        if w.get("WRITE_SIZE") and wscale:
            row["hbm_write_bytes"] = round(_mean(w["WRITE_SIZE"]) * 1024.0 * wscale)
        if "hbm_read_bytes" in row and "hbm_write_bytes" in row:
            row["hbm_bytes"] = row["hbm_read_bytes"] + row["hbm_write_bytes"]
            row["hbm_gbs"] = round(row["hbm_bytes"] / (t["avg_us_last"] * 1e3), 1)
        kernels[k] = row
    out = {"config": config, "source_sha256": meta["source_sha256"], "copy_bytes": COPY_BYTES,
           "copy_fetch_size_kib": cfetch, "copy_write_size_kib": cwrite,
           "fetch_scale": fscale, "write_scale": wscale, "kernels": kernels, "commands": commands}
    os.makedirs(PROFILES, exist_ok=True)
    for d in (PROFILES, out_dir):
        with open(os.path.join(d, f"{config}_profile.json"), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
    L = [f"# Profile: {config} workload", "",
         f"Source sha256 of the kernels: `{out['source_sha256']}`.", "",
         "Commands (repository root `$REPO`, output directory `OUT`), each a run of its own:", ""]
    L += ["    " + c for c in commands]
    L += ["", "Counter notes: cycles are GRBM_COUNT / 8 (summed over the 8 XCDs); MFMA busy is "
          "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs); LDS bank conflict is "
          "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; wait is SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; "
          f"HBM bytes are FETCH_SIZE x {fscale and round(fscale, 4)} and WRITE_SIZE x "
          f"{wscale and round(wscale, 4)} KiB, the factors that make a 1 GiB device copy read "
          "and write 1 GiB.  Durations are the average of the last 20 dispatches of the trace run.", "",
          "| kernel | µs | cycles (M) | GHz | MFMA busy % | LDS active % | LDS conflict % | wait % | "
          "HBM read MB | HBM write MB | HBM GB/s |",
          "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]

    def g(r, k, scale=1.0, nd=1):
        v = r.get(k)
        return "" if v is None else f"{v / scale:.{nd}f}"

    for k, r in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_us"]):
        L.append(f"| `{k}` | {r['avg_us']:.1f} | {g(r, 'cycles', 1e6, 3)} | {g(r, 'clock_ghz_vs_trace_avg', 1, 2)} | "
                 f"{g(r, 'mfma_busy_pct')} | {g(r, 'lds_active_pct')} | {g(r, 'lds_bank_conflict_pct', 1, 2)} | "
                 f"{g(r, 'wait_inst_any_pct')} | {g(r, 'hbm_read_bytes', 1e6)} | {g(r, 'hbm_write_bytes', 1e6)} | "
                 f"{g(r, 'hbm_gbs')} |")
    for d in (PROFILES, out_dir):
        with open(os.path.join(d, f"{config}_profile.md"), "w") as f:
            f.write("\n".join(L) + "\n")
    print("\n".join(L), flush=True)


def committed_traffic(config, kernel):
    """HBM bytes per launch of `kernel` from the committed profile of `config`,
    or None when absent or taken on other kernel sources."""
    try:
        with open(profile_path(config, "json")) as f:
            p = json.load(f)
    except (OSError, ValueError):
        return None
    if p.get("source_sha256") != sources_sha():
        return None
    for k, r in p.get("kernels", {}).items():
        if k.split("<")[0] == kernel and "hbm_bytes" in r:
            return float(r["hbm_bytes"])
    return None


# ----------------------------------------------------------------------------
def cpu_baseline(inp, cfg, budget_s):
    """The fp64 oracle, timed on whole heads of the same workload."""
    import oracle
    from attn_inputs import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    BH = cfg.B * cfg.H
    per_head = bwd_flops(1, 1, cfg.N, cfg.d, cfg.causal)
    done, t_total = 0, 0.0
    while done < BH and (done == 0 or t_total < budget_s):
        sl = lambda n: bf16_bits_to_f64(inp[n].reshape(BH, cfg.N, cfg.d)[done])  # noqa: E731
        q, k, v, do = sl("q"), sl("k"), sl("v"), sl("do")
        t0 = time.perf_counter()
        oracle.attention_backward(q, k, v, do, cfg.scale, causal=cfg.causal)
        t_total += time.perf_counter() - t0
        done += 1
    return {
        "value": round(tflops(per_head * done, t_total * 1e3), 6),
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"fp64 numpy forward+backward of {done} of {BH} heads "
                  f"(N={cfg.N}, d={cfg.d}, causal={cfg.causal}), {t_total:.1f} s",
        "cpu_model": cpu_model(),
        "os_cpu_count": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
    }


SPARSE_MAIN_SHARE = (2 * 576 + 2 * 512) * 2 / (2 * (3 * 576 + 2 * 512))   # S, dP, dV, dK of 5 products


def sparse_valid_pairs(topk_len) -> int:
    return int(sum(int(x) for x in topk_len))


def bench_sparse(args, cfg):
    """Top-k sparse backward (attn_bwd_preprocess + attn_sparse_bwd), same
    timing protocol as the dense benchmark."""
    import numpy as np
    import torch
    import exact_attention_bwd_amd as ea
    from attn_inputs import make_sparse_inputs

    dev = torch.device("cuda:0")
    print(f"[bench] {cfg.name}: Hq{cfg.Hq} Nq{cfg.Nq} Nkv{cfg.Nkv} dqk{cfg.dqk} dv{cfg.dv} topk{cfg.topk}: inputs",
          file=sys.stderr, flush=True)
    inp = make_sparse_inputs(cfg)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (up(inp[n]) for n in ("q", "k", "v", "do"))
    idx = torch.from_numpy(inp["idx"]).to(dev)
    tl = torch.from_numpy(inp["topk_len"]).to(dev)
    o, lse = ea.attn_sparse_fwd(q, k, v, idx, tl, cfg.scale)
    D = torch.empty((cfg.Hq, cfg.Nq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((ea.attn_sparse_bwd_workspace_bytes(cfg.Hq, cfg.Nq, cfg.Nkv, cfg.topk, cfg.dqk, cfg.dv),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = HipEvents()

    def step(events=None):
        ea.attn_bwd_preprocess(o[None], do[None], D=D[None])
        ea.attn_sparse_bwd(q, k, v, do, lse, D, idx, tl, cfg.scale, dq=dq, dk=dk, dv=dv, workspace=ws,
                           main_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    with SclkSampler() as clk:
        total, per, main_ms = timed_steps(ev, stream, step, K)
    ms_step = total / K
    main_avg = sum(main_ms) / K
    # forward on its own
    t0, t1 = ev.create(), ev.create()
    ev.record(t0, stream)
    for _ in range(K):
        ea.attn_sparse_fwd(q, k, v, idx, tl, cfg.scale, o=o, lse=lse)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    fwd_ms = ev.elapsed_ms(t0, t1) / K
    nominal = sparse_bwd_flops(cfg.Hq, cfg.Nq, cfg.topk, cfg.dqk, cfg.dv)
    valid = 2.0 * cfg.Hq * sparse_valid_pairs(inp["topk_len"]) * (3 * cfg.dqk + 2 * cfg.dv)
    main_fl = SPARSE_MAIN_SHARE * valid
    value = tflops(nominal, ms_step)
    main_tf = tflops(main_fl, main_avg)
    line = {
        "metric": "sparse top-k attn bwd effective TFLOPS (2·H·N·topk·(3·d_qk+2·d_v)) & % bf16 MFMA peak, "
                  f"Hq{cfg.Hq} N{cfg.Nq} d_qk{cfg.dqk} d_v{cfg.dv} topk{cfg.topk}",
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": step_stats(per),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"top-k sparse attention backward (preprocess + backward) Hq{cfg.Hq} "
                               f"Nq{cfg.Nq} Nkv{cfg.Nkv} d_qk{cfg.dqk} d_v{cfg.dv} topk{cfg.topk} bf16, "
                               f"seed {cfg.seed}"},
        "valid_pair_tflops": round(tflops(valid, ms_step), 3),
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "peak_tflops": PEAK_BF16_TFLOPS,
        "main_kernel": {"name": "sbwd_main_kernel", "ms": round(main_avg, 5), "tflops": round(main_tf, 3)},
        "rest_ms": round(ms_step - main_avg, 5),
        "forward": {"ms": round(fwd_ms, 5),
                    "tflops": round(tflops(2.0 * cfg.Hq * sparse_valid_pairs(inp["topk_len"])
                                           * (cfg.dqk + cfg.dv), fwd_ms), 3)},
        "roofline": {"bound": "mfma", "kernel": "sbwd_main_kernel", "achieved": round(main_tf, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(main_tf / PEAK_BF16_TFLOPS, 5),
                     "traffic": committed_traffic(cfg.name, "sbwd_main_kernel")},
        "sclk": clk.summary(),
        "context": {"pages_b200_ms": PAGES_SPARSE_MS,
                    "note": "the pages' own figure for this cell, on another machine"},
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--hkv", type=int, default=None,
                    help="grouped-query attention: K/V heads (dividing H); default H")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the 1 GiB calibration copy (for the TCC byte counters)")
    ap.add_argument("--profile", metavar="OUT",
                    help="run the kernel trace and counter passes of --config under rocprofv3 "
                         "(child processes) and write profiles/<config>_profile.{json,md}")
    ap.add_argument("--summarise", metavar="OUT",
                    help="only rebuild profiles/<config>_profile.* from an existing OUT (no GPU)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        return 2

    if args.profile:
        extra = [] if args.hkv is None else ["--hkv", str(args.hkv)]
        return run_profile(args.profile, args.config, extra, profile_name(args.config, args.hkv))
    if args.summarise:
        summarise_profile(os.path.abspath(args.summarise), profile_name(args.config, args.hkv))
        return 0

    if args.copy_calibration:
        copy_calibration()
        return 0

    import torch
    import exact_attention_bwd_amd as ea
    from attn_inputs import DENSE_CONFIGS, make_dense_inputs

    from attn_inputs import SPARSE_CONFIGS
    if args.config in SPARSE_CONFIGS:
        return bench_sparse(args, SPARSE_CONFIGS[args.config])
    cfg = DENSE_CONFIGS[args.config]
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    hkv = H if args.hkv is None else args.hkv
    gqa = hkv != H
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] {cfg.name}: B{B} H{H} N{N} d{d} causal={cfg.causal}", file=sys.stderr, flush=True)

    if gqa:
        from attn_inputs import make_gqa_inputs
        inp = make_gqa_inputs(cfg, hkv)
    else:
        inp = make_dense_inputs(cfg)
    import numpy as np

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (up(inp[n]) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    D = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((ea.attn_bwd_workspace_bytes(B, H, N, d, cfg.causal, hkv),), dtype=torch.uint8, device=dev)
    fwd = ea.attn_fwd_gqa if gqa else ea.attn_fwd
    bwd = ea.attn_bwd_gqa if gqa else ea.attn_bwd
    stream = torch.cuda.current_stream()
    ev = HipEvents()

    fwd(q, k, v, cfg.causal, cfg.scale, o=o, lse=lse)
    torch.cuda.synchronize()

    def step(events=None):
        ea.attn_bwd_preprocess(o, do, D=D)
        bwd(q, k, v, do, lse, D, cfg.causal, cfg.scale, dq=dq, dk=dk, dv=dv,
            workspace=ws, main_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    K = args.steps
    with SclkSampler() as clk:
        total_ms, per, main_ms = timed_steps(ev, stream, step, K)
    ms_step = total_ms / K
    main_avg = sum(main_ms) / K
    print(f"[bench] timed {K} steps: {ms_step:.4f} ms/step (median {_percentile(per, 50):.4f}), "
          f"dominant kernel {main_avg:.4f} ms", file=sys.stderr, flush=True)

    # forward, timed on its own (not part of the metric)
    for _ in range(max(2, args.warmup // 2)):
        fwd(q, k, v, cfg.causal, cfg.scale, o=o, lse=lse)
    t0, t1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for _ in range(K):
        fwd(q, k, v, cfg.causal, cfg.scale, o=o, lse=lse)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    fwd_ms = ev.elapsed_ms(t0, t1) / K
    ev.destroy(t0)
    ev.destroy(t1)

    fl = bwd_flops(B, H, N, d, cfg.causal)
    value = tflops(fl, ms_step)
    kname, share = dominant_kernel(d, cfg.causal, gqa)
    main_tf = tflops(share * fl, main_avg)
    line = {
        "metric": dense_metric(cfg, hkv),
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": step_stats(per),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{'causal' if cfg.causal else 'non-causal'} attention backward "
                        f"(preprocess + {'fused backward' if kname == 'bwd_fused_kernel' else 'dK/dV and dQ kernels'}) "
                        f"B{B} H{H}"
                        + (f" Hkv{hkv} (grouped-query)" if gqa else "")
                        + f" N{N} d{d} bf16, seed {cfg.seed}",
            "B": B, "H": H, "N": N, "d": d, "causal": cfg.causal, "scale": cfg.scale,
            **({"Hkv": hkv} if gqa else {}),
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "peak_tflops": PEAK_BF16_TFLOPS,
        "flops_per_step": fl,
        "dominant_kernel": {"name": kname, "ms": round(main_avg, 5), "tflops": round(main_tf, 3),
                            "flops": share * fl, "ms_min": round(min(main_ms), 5),
                            "ms_max": round(max(main_ms), 5),
                            "ms_median": round(_percentile(main_ms, 50), 5)},
        "rest_ms": round(ms_step - main_avg, 5),
        "forward": {"ms": round(fwd_ms, 5),
                    "tflops": round(tflops(fwd_flops(B, H, N, d, cfg.causal), fwd_ms), 3)},
        "roofline": {
            "bound": "mfma",
            "kernel": kname,
            "achieved": round(main_tf, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(main_tf / PEAK_BF16_TFLOPS, 5),
            "traffic": committed_traffic(profile_name(cfg.name, hkv if gqa else None), kname),
        },
        "sclk": clk.summary(),
        "context": ({"pages_rtx5090_v3_tflops": PAGES_BWD_TFLOPS,
                     "note": "the pages' own backward at this workload, on another machine"}
                    if cfg.name == "headline" and not gqa else None),
    }
    if not args.no_cpu_baseline and not gqa:       # the oracle leg times the dense workload
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb = cpu_baseline(inp, cfg, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["vs_cpu_baseline"] = round(value / cb["value"], 1) if cb["value"] > 0 else None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
