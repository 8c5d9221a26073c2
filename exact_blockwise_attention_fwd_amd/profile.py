"""rocprofv3 harness: kernel time, HBM traffic and matrix-core counters of the attention kernels.

    python -m exact_blockwise_attention_fwd_amd.profile [--what trace,traffic,counters] [--workloads a,b]
                                                        [--out DIR] [--raw DIR]

Runs on the GPU host.  Every measurement is a child process ``rocprofv3 ... -- python3 bench.py ...`` (this
process never touches the GPU, so the profiler's preloaded library starts the program itself), each under
its own time limit, and the summaries it writes (Markdown and text, a few KB) name the exact command that
produced them and the build fingerprint of the forward kernel (its source and compile flags):

  trace     rocprofv3 --kernel-trace --stats over the bench step of each workload: calls and average duration
            of every kernel; TFLOP/s of each forward launch (algorithmic FLOPs: 4 d per visible query/key pair)
            against the dense bf16 peak, merge GB/s against the HBM peak.
  traffic   FETCH_SIZE and WRITE_SIZE (one counter per pass) per forward launch of the ring-share step and per
            merge launch, each scaled by what the same counter reads for a plain 1 GiB device-to-device copy.
  streamed  --kernel-trace --memory-copy-trace over the host-streamed step: chunk copies (count, bytes, GB/s)
            and kernel durations.
  counters  GRBM_GUI_ACTIVE and SQ counters per forward launch: MFMA busy fraction, effective engine clock,
            MFMA FLOP per algorithmic FLOP, VALU co-issue beside MFMA, VALU and LDS instructions per MFMA, LDS
            bank conflicts, and the scratch (spill) bytes per lane the dispatch ran with.
  ffn       the blockwise feed-forward leg of the ring-share bench (its two GEMM kernels): a kernel trace, one
            pass of the SQ counters above, and FETCH_SIZE / WRITE_SIZE against the GEMMs' algorithmic bytes.

The ``key: value`` lines at the end of the traffic and counter summaries are read back by bench.py, which
reports them only when the fingerprint matches the library it runs.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
BENCH = os.path.join(ROOT, "bench.py")
FWD_SOURCE = "attn_fwd_bf16.hip"
BF16_PEAK_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30
# Timed and warmup steps of the trace run per workload: short workloads take more steps, so that the engine
# clock has settled and the timed region lasts tens of milliseconds (with 3 steps a 1 ms launch reads up to
# 25 % slow).  The counter passes use COUNTER_WARMUP warmup steps before the one step they summarise.
TRACE_STEPS = {"ring_share_128k": (5, 2), "ulysses_share_256k": (3, 1), "causal_prefill_4k": (300, 100),
               "peaky_16k": (100, 30), "tiny_fp32": (400, 100)}
COUNTER_WARMUP = {"ring_share_128k": 1, "ulysses_share_256k": 1, "causal_prefill_4k": 100, "peaky_16k": 30,
                  "tiny_fp32": 100}
SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_INSTS_VALU",
               "SQ_INSTS_MFMA", "SQ_BUSY_CU_CYCLES"]


def log(msg):
    print(f"[profile] {msg}", flush=True)


def fingerprint() -> str:
    sys.path.insert(0, ROOT)
    from exact_blockwise_attention_fwd_amd.build import fingerprint as fp
    return fp(FWD_SOURCE)


def rocprof() -> str:
    for c in (shutil.which("rocprofv3"), "/opt/rocm/bin/rocprofv3"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("rocprofv3 not found")


def run_profiled(tag: str, prof_args: list[str], bench_args: list[str], raw: str, limit: int) -> tuple[str, str]:
    """One profiled child run; returns (its output directory, the command line as run)."""
    out = os.path.join(raw, tag)
    shutil.rmtree(out, ignore_errors=True)
    os.makedirs(out, exist_ok=True)
    if "--calibrate-copy" not in bench_args:
        # no clock/power run after the profiled steps, and no nested harness run
        bench_args = [*bench_args, "--clock-seconds", "0", "--no-live-counters"]
    cmd = ["timeout", "-s", "KILL", str(limit), rocprof(), *prof_args, "--output-format", "csv", "-d", out, "-o", "run",
           "--", sys.executable, BENCH, *bench_args]
    shown = " ".join(["timeout", "-s", "KILL", str(limit), "rocprofv3", *prof_args, "--output-format", "csv", "-d",
                      f"<raw>/{tag}", "-o", "run", "--", "python3", "bench.py", *bench_args])
    log(f"{tag}: {shown}")
    t0 = time.time()
    with open(os.path.join(out, "stdout.txt"), "w") as fo, open(os.path.join(out, "stderr.txt"), "w") as fe:
        r = subprocess.run(cmd, cwd="/tmp", stdout=fo, stderr=fe, env=dict(os.environ, TMPDIR="/tmp"))
    log(f"{tag}: exit {r.returncode} after {time.time() - t0:.0f} s")
    if r.returncode not in (0, 139) or not glob.glob(os.path.join(out, "**", "*.csv"), recursive=True):
        # 139: rocprofv3 itself may end with a segmentation fault after the program and its results are complete
        raise RuntimeError(f"{tag}: profiled run failed (exit {r.returncode}); see {out}/stderr.txt")
    return out, shown


def read_csv(out: str, suffix: str) -> list[dict]:
    files = sorted(glob.glob(os.path.join(out, "**", f"*{suffix}"), recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def col(row: dict, *names):
    for n in names:
        for k in row:
            if k.replace("-", "_").lower() == n.lower():
                return row[k]
    raise KeyError(names)


def bench_json(out: str) -> dict | None:
    try:
        for line in open(os.path.join(out, "stdout.txt")):
            if line.startswith("{"):
                return json.loads(line)
    except OSError:
        pass
    return None


def short(name: str) -> str:
    """Readable kernel name: template arguments kept; return type, namespaces and argument list dropped."""
    name = name.replace("(anonymous namespace)::", "").replace("attn::", "")
    if name.startswith("void "):
        name = name[5:]
    if name.startswith("at::") and "<" in name:   # torch's own kernels: the template arguments run to pages
        return name[:name.index("<")] + "<…>"
    depth = 0
    for i, ch in enumerate(name):   # cut at the argument list: the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def workload(name: str):
    sys.path.insert(0, ROOT)
    import workloads as W
    return W.WORKLOADS[name]


def forward_dispatches(rows: list[dict]) -> list[dict]:
    return [r for r in rows if "fwd_" in col(r, "Kernel_Name") and "kernel" in col(r, "Kernel_Name")]


# --------------------------------------------------------------------------------------------- kernel trace
def launch_flops(w) -> list[float]:
    """Algorithmic FLOPs of each forward launch of one bench step, in launch order (the chunked step's
    chunks, or the single pass)."""
    if w.chunks <= 1:
        return [w.flops()]
    out = []
    off = w.N_kv - w.N_q
    for p in range(w.chunks):
        lo, hi = p * w.N_kv // w.chunks, (p + 1) * w.N_kv // w.chunks
        if hi == lo or (w.causal and w.N_q - 1 + off - lo < 0):
            continue
        n = hi - lo
        vis = 0
        for i in range(w.N_q):   # visible keys of row i in [lo, hi)
            last = min(hi - 1, i + off) if w.causal else hi - 1
            vis += max(0, last - lo + 1)
        out.append(4.0 * w.B * w.H * w.d * vis)
    # the metric counts a square causal block as N^2/2 pairs, not N(N+1)/2: scale to its total
    tot = sum(out)
    return [f * w.flops() / tot for f in out] if tot else out


def trace(names: list[str], raw: str, steps_override: int | None, warmup_override: int | None) -> str:
    fpr = fingerprint()
    lines = ["# Kernel trace of the attention kernels, every configured workload", "",
             f"Forward kernel build fingerprint (source and compile flags): `{fpr}`", "",
             "Each workload: one child run of the bench step under `rocprofv3 --kernel-trace --stats` (from the",
             "repository root on the GPU host, `cd /tmp && export TMPDIR=/tmp` first).  TFLOP/s of a forward launch",
             "= its algorithmic FLOPs (4 d per visible query/key pair) / its average duration under the profiler;",
             f"peak {BF16_PEAK_TFLOPS} TFLOP/s (dense bf16) or the fp64 ALU peak for the fp32 kernel.", ""]
    machine = []
    for n in names:
        w = workload(n)
        steps, warmup = TRACE_STEPS.get(n, (3, 2))
        steps = steps_override or steps
        warmup = warmup if warmup_override is None else warmup_override
        out, shown = run_profiled(f"trace_{n}", ["--kernel-trace", "--stats"],
                                  ["--workload", n, "--steps", str(steps), "--warmup", str(warmup), "--no-cpu-baseline",
                                   "--no-streamed", "--no-graph", "--no-ffn", "--no-ulysses"], raw, 300)
        stats = read_csv(out, "kernel_stats.csv")
        tr = read_csv(out, "kernel_trace.csv")
        lines += [f"## {n}", "", f"    {shown}", ""]
        b = bench_json(out)
        if b:
            lines += [f"bench line under the profiler: {b['value']} TFLOP/s per step ({b['ms_per_step']} ms/step)", ""]
        lines += ["| kernel | calls | average us | total ms |", "|---|---|---|---|"]
        for s in sorted(stats, key=lambda r: -float(col(r, "TotalDurationNs"))):
            lines.append(f"| `{short(col(s, 'Name', 'Kernel_Name'))}` | {col(s, 'Calls')} | "
                         f"{float(col(s, 'AverageNs')) / 1e3:.1f} | {float(col(s, 'TotalDurationNs')) / 1e6:.2f} |")
        fwd = forward_dispatches(tr)
        flops = launch_flops(w)
        per = len(flops)
        if fwd and per:
            fwd = sorted(fwd, key=lambda r: int(col(r, "Start_Timestamp")))[-per * steps:]
            durs = [(int(col(r, "End_Timestamp")) - int(col(r, "Start_Timestamp"))) * 1e-9 for r in fwd]
            ach = [flops[i % per] / durs[i] / 1e12 for i in range(len(durs))]
            tot = sum(flops) * steps / sum(durs) / 1e12
            peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else 78.6
            lines += ["", f"Forward launches of the last {steps} step(s): {len(durs)}, "
                          f"{sum(durs) / steps * 1e3:.3f} ms of forward per step, {tot:.1f} TFLOP/s, frac {tot / peak:.4f}",
                      "", "| launch in step | FLOP | us | TFLOP/s |", "|---|---|---|---|"]
            for i in range(per):
                us = sum(durs[i::per]) / len(durs[i::per]) * 1e6
                lines.append(f"| {i} | {flops[i]:.4e} | {us:.1f} | {flops[i] / (us * 1e-6) / 1e12:.1f} |")
            machine.append(f"{n}_fwd_tflops: {tot:.2f}")
            machine.append(f"{n}_fwd_frac: {tot / peak:.4f}")
        lines.append("")
    lines += ["Machine-readable:", "", f"kernel_build_sha256: {fpr}", *machine, ""]
    return "\n".join(lines)


# ----------------------------------------------------------------------------------------------- traffic
def counter_rows(out: str, name: str) -> list[dict]:
    rows = [r for r in read_csv(out, "counter_collection.csv") if col(r, "Counter_Name") == name]
    return sorted(rows, key=lambda r: int(col(r, "Correlation_Id", "Dispatch_Id")))


def traffic(name: str, raw: str) -> str:
    fpr = fingerprint()
    w = workload(name)
    bench_args = ["--workload", name, "--steps", "1", "--warmup", "0", "--no-cpu-baseline", "--no-streamed",
                  "--no-graph", "--no-ffn", "--no-ulysses"]
    copy_args = ["--calibrate-copy", "--steps", "2", "--warmup", "1"]
    runs = {}
    for tag, ctr, args in (("fetch", "FETCH_SIZE", bench_args), ("write", "WRITE_SIZE", bench_args),
                           ("fetch_copy", "FETCH_SIZE", copy_args), ("write_copy", "WRITE_SIZE", copy_args)):
        runs[tag] = run_profiled(f"traffic_{tag}_{name}", ["--pmc", ctr], args, raw, 120)
    def per_kernel(tag, ctr, pred):
        return [float(col(r, "Counter_Value")) for r in counter_rows(runs[tag][0], ctr) if pred(col(r, "Kernel_Name"))]
    is_fwd = lambda k: "fwd_" in k and "kernel" in k
    is_merge = lambda k: "merge" in k or "rows_kernel" in k
    is_copy = lambda k: "copy" in k.lower()
    fcopy = per_kernel("fetch_copy", "FETCH_SIZE", is_copy)
    wcopy = per_kernel("write_copy", "WRITE_SIZE", is_copy)
    f_fac = COPY_BYTES / (sum(fcopy) / len(fcopy) * 1024) if fcopy else float("nan")
    w_fac = COPY_BYTES / (sum(wcopy) / len(wcopy) * 1024) if wcopy else float("nan")
    ff = per_kernel("fetch", "FETCH_SIZE", is_fwd)
    wf = per_kernel("write", "WRITE_SIZE", is_fwd)
    mf = per_kernel("fetch", "FETCH_SIZE", is_merge)
    mw = per_kernel("write", "WRITE_SIZE", is_merge)
    per = len(launch_flops(w))
    rows_ = w.B * w.H * w.N_q
    es = 2 if w.dtype == "bf16" else 4
    lines = [f"# HBM traffic of the forward launches, {name}", "",
             f"Forward kernel build fingerprint: `{fpr}`", "",
             "Commands (one counter per pass; the copy runs calibrate each counter on a plain 1 GiB device-to-device copy):", ""]
    lines += [f"    {runs[t][1]}" for t in ("fetch", "write", "fetch_copy", "write_copy")]
    lines += ["", "| launch in step | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | written bytes (scaled) |",
              "|---|---|---|---|---|"]
    tot = []
    for i in range(min(per, len(ff), len(wf))):
        rb, wb = ff[i] * 1024 * f_fac, wf[i] * 1024 * w_fac
        tot.append(rb + wb)
        lines.append(f"| {i} | {ff[i]:.0f} | {wf[i]:.0f} | {rb:.4e} | {wb:.4e} |")
    mean = sum(tot) / len(tot) if tot else float("nan")
    q_b = w.B * w.H * w.N_q * w.d * es
    kv_b = 2 * w.B * w.H * w.N_kv * w.d * es / max(per, 1)
    lines += ["", "| quantity | value |", "|---|---|",
              f"| FETCH_SIZE of a 1 GiB copy | {sum(fcopy) / max(len(fcopy), 1):.1f} KiB -> factor {f_fac:.4f} |",
              f"| WRITE_SIZE of a 1 GiB copy | {sum(wcopy) / max(len(wcopy), 1):.1f} KiB -> factor {w_fac:.4f} |",
              f"| HBM bytes per forward launch, mean over the step (read + written, scaled) | {mean:.4e} |",
              f"| compulsory reads per launch: Q + one chunk's K and V | {q_b + kv_b:.4e} |",
              f"| output per launch: fp32 partial rows + lse ({rows_} rows) | {rows_ * (w.d + 1) * 4:.4e} |"]
    if mf and mw:
        lines.append(f"| merge launch (fp32 -> fp32), FETCH / WRITE scaled | {mf[0] * 1024 * f_fac:.4e} / "
                     f"{mw[0] * 1024 * w_fac:.4e} (algorithmic {rows_ * (w.d * 8 + 8):.3e} / {rows_ * (w.d * 4 + 4):.3e}) |")
    lines += ["", "Machine-readable (read by bench.py; valid only for the kernel build with this hash):", "",
              f"kernel_build_sha256: {fpr}", f"workload: {name}", f"hbm_bytes_per_launch: {mean:.6e}", ""]
    return "\n".join(lines)


# ---------------------------------------------------------------------------------------------- counters
def counters(name: str, raw: str) -> str:
    fpr = fingerprint()
    w = workload(name)
    args = ["--workload", name, "--steps", "1", "--warmup", str(COUNTER_WARMUP.get(name, 1)), "--no-cpu-baseline",
            "--no-streamed", "--no-graph", "--no-ffn", "--no-ulysses"]
    out, shown = run_profiled(f"counters_{name}", ["--pmc", *SQ_COUNTERS], args, raw, 150)
    rows = read_csv(out, "counter_collection.csv")
    disp = {}
    for r in rows:
        k = col(r, "Kernel_Name")
        if not ("fwd_" in k and "kernel" in k):
            continue
        d = disp.setdefault(int(col(r, "Correlation_Id", "Dispatch_Id")), {"kernel": k})
        d[col(r, "Counter_Name")] = float(col(r, "Counter_Value"))
        for key, names in (("start", ("Start_Timestamp",)), ("end", ("End_Timestamp",)), ("scratch", ("Scratch_Size",))):
            try:
                d[key] = float(col(r, *names))
            except (KeyError, ValueError):
                pass
    per = len(launch_flops(w))
    ds = [disp[k] for k in sorted(disp)][-per:]   # the timed step (the warmup step's launches come first)
    flops = launch_flops(w)
    lines = [f"# Matrix-core counters of the forward launches, {name}", "", f"Forward kernel build fingerprint: `{fpr}`", "",
             "Command (one pass):", "", f"    {shown}", "",
             "Derived per launch (counters summed over the 8 XCDs; GUI-active cycles per XCD = GRBM_GUI_ACTIVE / 8; 1024",
             "SIMDs, 256 CUs; durations are the dispatch's own under the profiler): sclk = GUI cycles per XCD / duration;",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x 1024); MFMA FLOP / algorithmic = SQ_INSTS_VALU_MFMA_MOPS_BF16",
             "x 512 / (4 d per visible pair); co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; VALU / MFMA",
             "and LDS / MFMA = SQ_INSTS_VALU (MFMAs included) and SQ_INSTS_LDS per SQ_INSTS_MFMA; LDS conflict =",
             "SQ_LDS_BANK_CONFLICT / (GUI cycles x 256); scratch = the dispatch record's private bytes per lane.",
             "Registers are in kernel_resource_usage.txt (the compiler's counts; the dispatch record's VGPR field",
             "reads 128 for the 256-VGPR kernels and is not used).", "",
             "| launch | us | sclk GHz | TFLOP/s | MFMA busy | MFMA FLOP / alg. | co-issue | VALU / MFMA | LDS / MFMA | "
             "LDS conflict | scratch B/lane |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    acc = {"busy": 0.0, "ratio": 0.0, "coexec": 0.0, "conf": 0.0, "sclk": 0.0, "w": 0.0}
    for i, d in enumerate(ds):
        try:
            us = (d["end"] - d["start"]) * 1e-3
            gui = d["GRBM_GUI_ACTIVE"] / 8
            sclk = gui / (us * 1e3)
            busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024)
            ratio = d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / flops[i]
            co = d["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(d["SQ_VALU_MFMA_BUSY_CYCLES"], 1)
            vm = d["SQ_INSTS_VALU"] / max(d["SQ_INSTS_MFMA"], 1)
            lm = d["SQ_INSTS_LDS"] / max(d["SQ_INSTS_MFMA"], 1)
            conf = d["SQ_LDS_BANK_CONFLICT"] / (gui * 256)
        except (KeyError, ZeroDivisionError):
            continue
        tf = flops[i] / (us * 1e-6) / 1e12
        lines.append(f"| {i} | {us:.0f} | {sclk:.2f} | {tf:.0f} | {busy:.3f} | {ratio:.3f} | {co:.3f} | {vm:.2f} | {lm:.2f} | "
                     f"{conf:.4f} | {d.get('scratch', float('nan')):.0f} |")
        wgt = flops[i]
        acc["busy"] += busy * wgt
        acc["ratio"] += ratio * wgt
        acc["coexec"] += co * wgt
        acc["conf"] += conf * wgt
        acc["sclk"] += sclk * wgt
        acc["w"] += wgt
    wsum = acc["w"] or float("nan")
    lines += ["", "Machine-readable (read by bench.py; FLOP-weighted means over the step's launches; valid only for the",
              "kernel build with this hash):", "", f"kernel_build_sha256: {fpr}", f"workload: {name}",
              f"mfma_busy_frac: {acc['busy'] / wsum:.4f}", f"mfma_flop_per_algorithmic_flop: {acc['ratio'] / wsum:.4f}",
              f"valu_coexec_frac_of_mfma_busy: {acc['coexec'] / wsum:.4f}",
              f"lds_bank_conflict_frac: {acc['conf'] / wsum:.6f}", f"effective_sclk_ghz: {acc['sclk'] / wsum:.3f}", ""]
    return "\n".join(lines)


# ------------------------------------------------------------------------------------------- host streaming
def streamed(raw: str) -> str:
    """Kernel and memory-copy trace of the bench's host-streamed step (K and V in page-locked host memory, each
    chunk copied on a second stream while the previous chunk computes): the chunk copies' count, duration and
    bytes, and the kernels' durations, next to the bench's own streamed figures."""
    fpr = fingerprint()
    args = ["--workload", "ring_share_128k", "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-graph",
            "--no-ffn", "--no-ulysses"]
    out, shown = run_profiled("streamed_ring_share_128k", ["--kernel-trace", "--memory-copy-trace", "--stats"], args,
                              raw, 300)
    lines = ["# Host-streamed chunked step, ring_share_128k: kernel and memory-copy trace", "",
             f"Forward kernel build fingerprint: `{fpr}`", "",
             "K and V (1 GiB each) sit in page-locked host memory; each chunk's K rows and V rows (128 MiB each, one",
             "2-D copy per tensor) go to one of two staging slots on a copy stream while the previous chunk computes.",
             "The profiled bench runs the device-resident step (1 warmup + 3 timed), the stand-alone merge (12",
             "launches), then the streamed step (1 warmup + 3 timed): 64 chunk copies of 128 MiB, which the",
             "runtime files as device-to-device copies (the GPU addresses page-locked host memory directly).", "",
             "Command:", "", f"    {shown}", ""]
    b = bench_json(out)
    if b and b.get("streamed"):
        st = b["streamed"]
        lines += [f"bench line under the profiler: streamed {st.get('ms_per_step')} ms per step, copies "
                  f"{st.get('copy_ms_per_step')} ms at {st.get('h2d_gbs')} GB/s, device-resident "
                  f"{st.get('device_resident_ms_per_step')} ms, overlap efficiency {st.get('overlap_efficiency')}", ""]
    tr = read_csv(out, "memory_copy_trace.csv")
    if tr:
        size_key = next((k for k in tr[0] if k.lower() in ("bytes", "size", "copy_bytes")), None)
        dir_key = next((k for name in ("direction", "operation", "kind") for k in tr[0] if k.lower() == name), None)
        groups = {}
        for r in tr:
            nbytes = int(float(r[size_key])) if size_key else -1
            kind = r[dir_key] if dir_key else "copy"
            us = (int(col(r, "End_Timestamp")) - int(col(r, "Start_Timestamp"))) * 1e-3
            g = groups.setdefault((kind, nbytes), [])
            g.append(us)
        lines += ["Memory copies (`memory_copy_trace.csv`), grouped by direction (and size, where the trace records it):",
                  "", "| direction | bytes per copy | copies | average us | total ms | GB/s |", "|---|---|---|---|---|---|"]
        for (kind, nbytes), us in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            avg = sum(us) / len(us)
            gbs = f"{nbytes / (avg * 1e3):.1f}" if nbytes > 0 and avg > 0 else "-"
            lines.append(f"| {kind} | {nbytes if nbytes >= 0 else '-'} | {len(us)} | {avg:.1f} | {sum(us) / 1e3:.2f} | {gbs} |")
        if not size_key:
            lines += ["", "The copy trace records no byte counts (its columns: " + ", ".join(tr[0].keys()) + "). The runtime",
                      "splits each 2-D chunk copy out of page-locked memory into many pieces, some of them blit kernels",
                      "(`__amd_rocclr_copyBuffer` below); the bench's own events around each chunk copy give the rate."]
        lines.append("")
    stats = read_csv(out, "kernel_stats.csv")
    lines += ["Kernels (`kernel_stats.csv`):", "", "| kernel | calls | average us | total ms |", "|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(col(r, "TotalDurationNs"))):
        lines.append(f"| `{short(col(r, 'Name', 'Kernel_Name'))}` | {col(r, 'Calls')} | "
                     f"{float(col(r, 'AverageNs')) / 1e3:.1f} | {float(col(r, 'TotalDurationNs')) / 1e6:.2f} |")
    lines.append("")
    return "\n".join(lines)


# --------------------------------------------------------------------------------------------- feed-forward
def ffn(raw: str) -> str:
    """The two GEMM kernels of the bench's feed-forward leg (ring-share model shape): durations, counters and
    HBM bytes against the algorithmic ones (each operand read once, the output written once)."""
    sys.path.insert(0, ROOT)
    import workloads as W
    from exact_blockwise_attention_fwd_amd.build import fingerprint as fp

    fw = W.FFN_WORKLOADS["ffn_ring_share"]
    fpr = fp("ffn_bf16.hip")
    args = ["--workload", "ring_share_128k", "--steps", "1", "--warmup", "0", "--no-cpu-baseline", "--no-streamed",
            "--no-graph", "--no-ulysses"]
    copy_args = ["--calibrate-copy", "--steps", "2", "--warmup", "1"]
    tr, tr_cmd = run_profiled("ffn_trace", ["--kernel-trace", "--stats"], args, raw, 300)
    sq, sq_cmd = run_profiled("ffn_counters", ["--pmc", *SQ_COUNTERS], args, raw, 150)
    runs = {t: run_profiled(f"ffn_{t}", ["--pmc", c], a, raw, 120)
            for t, c, a in (("fetch", "FETCH_SIZE", args), ("write", "WRITE_SIZE", args),
                            ("fetch_copy", "FETCH_SIZE", copy_args), ("write_copy", "WRITE_SIZE", copy_args))}

    def per_kernel(tag, ctr, pred):
        return [float(col(r, "Counter_Value")) for r in counter_rows(runs[tag][0], ctr) if pred(col(r, "Kernel_Name"))]

    is_copy = lambda k: "copy" in k.lower()
    fcopy, wcopy = per_kernel("fetch_copy", "FETCH_SIZE", is_copy), per_kernel("write_copy", "WRITE_SIZE", is_copy)
    f_fac = COPY_BYTES / (sum(fcopy) / len(fcopy) * 1024) if fcopy else float("nan")
    w_fac = COPY_BYTES / (sum(wcopy) / len(wcopy) * 1024) if wcopy else float("nan")
    flop = 2.0 * fw.block * fw.d_ff * fw.d_model   # per GEMM launch, either product
    kernels = [("gemm_nt_kernel<2>", "x W1^T + b1, GELU", fw.block * fw.d_model * 2 + fw.d_ff * fw.d_model * 2,
                fw.block * fw.d_ff * 2),
               ("gemm_nt_kernel<0>", "h W2^T + b2", fw.block * fw.d_ff * 2 + fw.d_model * fw.d_ff * 2,
                fw.block * fw.d_model * 2)]
    disp = {}
    for r in read_csv(sq, "counter_collection.csv"):
        k = col(r, "Kernel_Name")
        if "gemm_nt_kernel" not in k:
            continue
        d = disp.setdefault(int(col(r, "Correlation_Id", "Dispatch_Id")), {"kernel": k})
        d[col(r, "Counter_Name")] = float(col(r, "Counter_Value"))
        for key, names in (("start", ("Start_Timestamp",)), ("end", ("End_Timestamp",))):
            try:
                d[key] = float(col(r, *names))
            except (KeyError, ValueError):
                pass
    stats = {short(col(r, "Name", "Kernel_Name")): r for r in read_csv(tr, "kernel_stats.csv")}
    lines = ["# Blockwise feed-forward (attn_ffn_blockwise), ring-share model shape: kernel trace, counters, traffic", "",
             f"GEMM kernel build fingerprint (source and compile flags): `{fpr}`", "",
             f"Shape: M = {fw.M} rows, d_model = {fw.d_model}, d_ff = {fw.d_ff}, {fw.act}, blocks of {fw.block} rows:",
             f"per block one GEMM of {fw.block} x {fw.d_ff} x {fw.d_model} with the bias + activation epilogue and one of",
             f"{fw.block} x {fw.d_model} x {fw.d_ff} with the bias epilogue; {flop:.4e} FLOP each.  The bench's ffn leg",
             "runs 2 warmup calls and 10 timed ones.  Commands (the copy runs calibrate FETCH_SIZE and WRITE_SIZE on a",
             "plain 1 GiB device-to-device copy):", "", f"    {tr_cmd}", f"    {sq_cmd}"]
    lines += [f"    {runs[t][1]}" for t in ("fetch", "write", "fetch_copy", "write_copy")]
    b = bench_json(tr)
    if b and b.get("ffn"):
        f = b["ffn"]
        lines += ["", f"bench line under the profiler: {f.get('ms')} ms per call = {f.get('tflops')} TFLOP/s "
                      f"({f.get('gemm_launches')} GEMM launches per call averaging {f.get('gemm_ms_avg')} ms)"]
    lines += ["", "| kernel | calls | avg us | min us | TFLOP/s (avg) | sclk GHz | MFMA busy | LDS / MFMA | "
                  "HBM read / algorithmic | HBM written / algorithmic |", "|---|---|---|---|---|---|---|---|---|---|"]
    for name, what, alg_r, alg_w in kernels:
        st = stats.get(name)
        if st is None:
            continue
        avg = float(col(st, "AverageNs")) / 1e3
        mn = float(col(st, "MinNs")) / 1e3 if "MinNs" in st else float("nan")
        ds = [d for d in disp.values() if short(d["kernel"]) == name]
        busy = sclk = lm = float("nan")
        try:
            us = [(d["end"] - d["start"]) * 1e-3 for d in ds]
            gui = [d["GRBM_GUI_ACTIVE"] / 8 for d in ds]
            sclk = sum(g / (u * 1e3) for g, u in zip(gui, us)) / len(ds)
            busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * 1024) for d, g in zip(ds, gui)) / len(ds)
            lm = sum(d["SQ_INSTS_LDS"] / max(d["SQ_INSTS_MFMA"], 1) for d in ds) / len(ds)
        except (KeyError, ZeroDivisionError):
            pass
        pred = lambda k, name=name: short(k) == name
        fr, wr = per_kernel("fetch", "FETCH_SIZE", pred), per_kernel("write", "WRITE_SIZE", pred)
        rd = sum(fr) / len(fr) * 1024 * f_fac if fr else float("nan")
        wt = sum(wr) / len(wr) * 1024 * w_fac if wr else float("nan")
        lines.append(f"| `{name}` ({what}) | {col(st, 'Calls')} | {avg:.1f} | {mn:.1f} | {flop / (avg * 1e-6) / 1e12:.0f} | "
                     f"{sclk:.2f} | {busy:.3f} | {lm:.2f} | {rd:.3e} / {alg_r:.3e} | {wt:.3e} / {alg_w:.3e} |")
    lines += ["", f"Counter pass: {len(disp)} GEMM dispatches; copy calibration: FETCH_SIZE factor {f_fac:.4f}, "
                  f"WRITE_SIZE factor {w_fac:.4f}.  Definitions as in attn_fwd_bf16_counters.txt.", ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--what", default="trace,traffic,counters,streamed,ffn")
    ap.add_argument("--workloads", default="ring_share_128k,ulysses_share_256k,causal_prefill_4k,peaky_16k,tiny_fp32")
    ap.add_argument("--steps", type=int, default=None, help="timed steps of every trace run (default: per workload)")
    ap.add_argument("--warmup", type=int, default=None, help="warmup steps of every trace run (default: per workload)")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "profiles"))
    ap.add_argument("--raw", default=os.path.join(ROOT, "gpurun_out", "prof_raw"))
    a = ap.parse_args()
    # the profiled children run from /tmp, so relative paths are taken against this directory here
    a.out, a.raw = os.path.abspath(a.out), os.path.abspath(a.raw)
    os.makedirs(a.out, exist_ok=True)
    what = a.what.split(",")
    names = a.workloads.split(",")
    if "trace" in what:
        text = trace(names, a.raw, a.steps, a.warmup)
        open(os.path.join(a.out, "attn_kernels_all_workloads.md"), "w").write(text)
        log("wrote attn_kernels_all_workloads.md")
    if "traffic" in what:
        open(os.path.join(a.out, "attn_fwd_bf16_traffic.txt"), "w").write(traffic("ring_share_128k", a.raw))
        log("wrote attn_fwd_bf16_traffic.txt")
    if "streamed" in what:
        open(os.path.join(a.out, "attn_fwd_streamed_ring_share_128k.md"), "w").write(streamed(a.raw))
        log("wrote attn_fwd_streamed_ring_share_128k.md")
    if "ffn" in what:
        open(os.path.join(a.out, "ffn_bf16_ring_share.md"), "w").write(ffn(a.raw))
        log("wrote ffn_bf16_ring_share.md")
    if "counters" in what:
        for n in names:
            if workload(n).dtype != "bf16":
                continue
            fname = "attn_fwd_bf16_counters.txt" if n == "ring_share_128k" else f"attn_fwd_bf16_counters_{n}.txt"
            open(os.path.join(a.out, fname), "w").write(counters(n, a.raw))
            log(f"wrote {fname}")


if __name__ == "__main__":
    main()
