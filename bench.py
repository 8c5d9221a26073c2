#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic input: for the ring-share workload
(B1 H32, 16384 local query rows against 131072 keys streamed as 8 chunks of 16384, bf16, d128, the last
chunk causal) that is 8 forward launches, the first writing an fp32 partial and each later one folding its
chunk into that partial in its epilogue (the last one writing bf16 O and the fp32 LSE).  Inputs are
resident in HBM before the timed region.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

`value` is attention TFLOP/s of the whole step (algorithmic FLOPs: 4*d per visible query/key pair, a square
causal block counted as N^2/2) over the step time.  The `roofline` object covers the dominant kernel (the
forward launches), timed with HIP events that the library records on the stream the kernels run on.
`merge` times attn_merge on its own, in place on fp32 partials of the workload's shape (the operation the
chunked step fuses into its forward launches), against the HBM peak.  `streamed` runs the same chunked step
with K and V in page-locked host memory (attn_fwd_streamed): host-to-device GB/s of the chunk copies and how
much of the shorter of copies and computation the overlap hides.  `ulysses` times the other causal
long-sequence workload (B1 H8, 262144 queries and keys, d128, one pass) the same way.  `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload on this host's cores (and, inside `ulysses`, on that
workload's seeded rows).  `counters` and `roofline.traffic` are read from the rocprofv3 harness's summaries
under profiles/ when they were taken on this same build; `counters_source` and `traffic_source` say so.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP64_PEAK_TFLOPS = 78.6        # MI355X fp64 vector: 256 CUs x 2.4 GHz x 128 FLOP/clk/CU
METRIC = "attn fwd TFLOP/s and % of MI355X bf16 MFMA peak; merge GB/s vs HBM peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def merge_bytes(w) -> float:
    """Algorithmic HBM bytes of one fp32 -> fp32 merge of two partials of the workload's shape: per row, read
    two partial rows and two lse values, write one row and one lse."""
    rows = w.B * w.H * w.N_q
    return float(rows * (w.d * (4 + 4 + 4) + 12))


def time_graph(step, steps: int) -> float:
    """ms per step of the same step captured once into a HIP graph and replayed `steps` times.  The entry
    points allocate nothing and never synchronise, so a step is capturable as it stands; the replays drop
    the host's launch cost, which matters only when a step's kernels are short."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


NOMINAL_SCLK_MHZ = 2400.0       # the engine clock the dense bf16 peak is quoted at


class ClockPowerSampler:
    """Engine clock and socket power of the measured GPU, read through amdsmi (read-only queries) every `period`
    seconds on a host thread while a timed region runs.  Under the attention step the board sits near its
    power cap and the clock falls below the nominal 2.4 GHz by an amount that differs from board to board;
    these samples show what the timed region ran at.  Anything amdsmi cannot give is reported as an error
    string, never raised."""

    def __init__(self, period: float = 0.02):
        self.period = period
        self.samples = []
        self.error = None
        self.limit_w = None
        self._h = None
        self._thread = None
        self._stop = None

    def _handle(self):
        import amdsmi
        import torch

        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
        if len(hs) == 1:
            return hs[0]
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        bus = getattr(props, "pci_bus_id", None)
        for h in hs:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
            if bus is not None and int(bdf.split(":")[1], 16) == bus:
                return h
        raise RuntimeError(f"no amdsmi handle matches the device's PCI bus ({len(hs)} handles)")

    def __enter__(self):
        import threading

        try:
            import amdsmi

            self._h = self._handle()
            lim = amdsmi.amdsmi_get_power_info(self._h).get("power_limit")
            self.limit_w = lim / 1e6 if isinstance(lim, (int, float)) and lim > 1e5 else lim
        except Exception as e:   # no amdsmi, no permission, no device: report, do not fail the bench
            self.error = f"{type(e).__name__}: {e}"
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(self._h)
                    clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float)) and c > 0]
                    pw = m.get("current_socket_power")
                    if clks and isinstance(pw, (int, float)):
                        self.samples.append((time.time(), sum(clks) / len(clks), min(clks), max(clks), float(pw)))
                except Exception as e:
                    self.error = f"{type(e).__name__}: {e}"
                    return
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self, what: str, achieved_tflops=None, skip_s: float = 0.0) -> dict:
        out = {"source": f"amdsmi gpu metrics sampled every {int(self.period * 1000)} ms over {what}, the first "
                         f"{skip_s:g} s dropped (the board's figures lag the load by a few hundred ms)"}
        t0 = self.samples[0][0] if self.samples else 0.0
        sm = [x for x in self.samples if x[0] - t0 >= skip_s]
        out["samples"] = len(sm)
        if not sm:
            out["error"] = self.error or "no samples"
            return out
        clk = sum(x[1] for x in sm) / len(sm)
        out.update({"gfxclk_mhz_mean": round(clk, 1), "gfxclk_mhz_xcd_min": min(x[2] for x in sm),
                    "gfxclk_mhz_xcd_max": max(x[3] for x in sm),
                    "socket_power_w_mean": round(sum(x[4] for x in sm) / len(sm), 1),
                    "socket_power_w_max": max(x[4] for x in sm), "power_limit_w": self.limit_w})
        if achieved_tflops:
            peak = BF16_PEAK_TFLOPS * clk / NOMINAL_SCLK_MHZ
            out.update({"bf16_peak_at_sampled_clock_tflops": round(peak, 1),
                        "frac_at_sampled_clock": round(achieved_tflops / peak, 4)})
        return out


CLOCK_SECONDS = 3.0   # length of the sampled run after a timed region
CLOCK_SKIP_S = 0.8    # its first part, dropped


def sample_clock_power(step, achieved_tflops, seconds: float = CLOCK_SECONDS) -> dict:
    """Runs `step` back to back for about `seconds` after the timed region (the queue kept a few steps deep)
    and samples the engine clock and socket power meanwhile."""
    import torch

    n = 0
    with ClockPowerSampler() as power:
        t_end = time.time() + seconds
        while time.time() < t_end:
            step()
            n += 1
            if n % 2 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    return power.summary(f"{n} further steps of the same workload after the timed ones", achieved_tflops,
                         CLOCK_SKIP_S)


def time_workload(w, steps: int, warmup: int, clock_seconds: float = CLOCK_SECONDS) -> dict:
    """A second workload's step (single pass or chunked, as configured) on seeded inputs resident in HBM: ms
    per step with events on the current stream, and the forward launches' TFLOP/s from the library's events
    against the dense bf16 peak."""
    import numpy as np
    import torch

    import exact_blockwise_attention_fwd_amd as A
    import workloads as W

    def dev(t):
        s_ = W.tensor_storage(w, t)
        return torch.from_numpy(s_.view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(W.Q_T), dev(W.K_T), dev(W.V_T)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, A.workspace_bytes(w.B, w.H, w.N_q, w.d, w.chunks)), dtype=torch.uint8, device="cuda")

    def step():
        if w.chunks > 1:
            A.fwd_chunked(q, k, v, w.chunks, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)
        else:
            A.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    A.timing_enable(True)
    A.timing_read()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    A.timing_enable(False)
    n_fwd, fwd_ms = A.timing_read()["fwd"]
    ms = e0.elapsed_time(e1) / steps
    tf = w.flops() / (ms * 1e-3) / 1e12
    ktf = w.flops() * steps / (fwd_ms * 1e-3) / 1e12
    clock_power = sample_clock_power(step, ktf, clock_seconds) if clock_seconds > 0 else None
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return {"config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.N_q, "N_kv": w.N_kv, "d": w.d,
                       "causal": w.causal, "chunks": w.chunks},
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4), "tflops": round(tf, 2),
            "pct_bf16_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2),
            "fwd_kernel": {"launches_per_step": n_fwd / steps, "tflops": round(ktf, 2),
                           "frac": round(ktf / BF16_PEAK_TFLOPS, 4)},
            "clock_power": clock_power}


def time_merge(w, reps: int):
    """attn_merge in place on fp32 partials [B,H,N_q,d] (seeded values, the empty rows of a causal chunk
    included), timed with the library's own launch events."""
    import torch

    import exact_blockwise_attention_fwd_amd as A

    g = torch.Generator(device="cuda").manual_seed(w.seed)
    shape = (w.B, w.H, w.N_q, w.d)
    oa = torch.randn(shape, device="cuda", generator=g)
    ob = torch.randn(shape, device="cuda", generator=g)
    la = torch.randn(shape[:3], device="cuda", generator=g)
    lb = torch.randn(shape[:3], device="cuda", generator=g)
    lb[..., : w.N_q // 8] = -math.inf
    for _ in range(2):
        A.merge(oa, la, ob, lb, out=oa, lse=la)
    torch.cuda.synchronize()
    A.timing_enable(True)
    A.timing_read()
    for _ in range(reps):
        A.merge(oa, la, ob, lb, out=oa, lse=la)
    torch.cuda.synchronize()
    A.timing_enable(False)
    n, ms = A.timing_read()["merge"]
    del oa, ob, la, lb
    return ms / max(n, 1)


def time_copy(nbytes: int, reps: int) -> float:
    """GB/s of a plain device-to-device copy of nbytes (read + written bytes per second): the practical HBM
    ceiling the merge's GB/s is read against, measured in the same job."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def time_streamed(w, q, k, v, steps: int, compute_ms: float):
    """The same chunked step with K and V in page-locked host memory (attn_fwd_streamed): chunk p+1 is copied
    to the device on a second stream while chunk p computes.  Times the step with events on the compute
    stream, and the chunk copies with the library's events on the copy stream; the overlap efficiency is
    max(device-resident step, copies alone) over the streamed step (1.0 = the shorter one fully hidden)."""
    import torch

    import exact_blockwise_attention_fwd_amd as A

    kh, vh = k.cpu().pin_memory(), v.cpu().pin_memory()
    ws = torch.empty(A.streamed_workspace_bytes(w.B, w.H, w.N_q, w.N_kv, w.d, w.chunks, q.dtype), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device="cuda")
    cs = torch.cuda.Stream()

    def step():
        A.fwd_streamed(q, kh, vh, w.chunks, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws,
                       copy_stream=cs)

    step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    A.timing_enable(True)
    A.timing_read()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    A.timing_enable(False)
    t = A.timing_read()
    ms = e0.elapsed_time(e1) / steps
    ncopy, copy_ms = t["copy"]
    copy_ms /= steps
    nbytes = 2 * k.numel() * k.element_size()      # every key and value row crosses once per step
    del kh, vh, ws, o, lse
    return {"what": "K and V in pinned host memory, chunk p+1 copied on a second stream while chunk p computes",
            "ms_per_step": round(ms, 4), "copies_per_step": ncopy / steps, "copy_ms_per_step": round(copy_ms, 4),
            "h2d_gbs": round(nbytes / (copy_ms * 1e-3) / 1e9, 2) if copy_ms > 0 else None,
            "device_resident_ms_per_step": round(compute_ms, 4),
            "overlap_efficiency": round(max(compute_ms, copy_ms) / ms, 4)}


def time_ffn(reps: int, cpu_rows: int, vendor_context: bool):
    """The blockwise feed-forward (next to attention in a blockwise transformer block) at the ring-share
    model's shape: attn_ffn_blockwise timed with the library's events (two GEMM launches per row block) and
    the fp64 oracle on `cpu_rows` seeded rows (all BLAS threads).  With `vendor_context`, also the same two
    products through torch's bf16 matmul with torch's GELU and bias adds: context only, not a target."""
    import time

    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import exact_blockwise_attention_fwd_amd as A
    import workloads as W

    fw = W.FFN_WORKLOADS["ffn_ring_share"]
    st = [W.ffn_tensor(fw, t) for t in (W.X_T, W.W1_T, W.B1_T, W.W2_T, W.B2_T)]

    def dev(s):
        if s.dtype == np.uint16:
            return torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(s).cuda()

    x, w1, b1, w2, b2 = (dev(s) for s in st)
    ws = torch.empty(A.ffn_workspace_bytes(fw.M, fw.d_ff, fw.block), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)

    def run():
        A.ffn_blockwise(x, w1, b1, w2, b2, block=fw.block, act=fw.act, out=y, workspace=ws)

    def timed(f, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(2):   # warmup, outside the library's timing
        run()
    torch.cuda.synchronize()
    A.timing_enable(True)
    A.timing_read()
    ms = timed(run, reps)
    A.timing_enable(False)
    n_gemm, gemm_ms = A.timing_read()["ffn"]
    vms = None
    if vendor_context:
        w1t, w2t = w1.t().contiguous(), w2.t().contiguous()   # contiguous right operands for torch's products
        y2 = torch.empty_like(x)

        def vendor():
            for r0 in range(0, fw.M, fw.block):
                h = torch.nn.functional.gelu((x[r0:r0 + fw.block] @ w1t).float() + b1).to(torch.bfloat16)
                y2[r0:r0 + fw.block] = ((h @ w2t).float() + b2).to(torch.bfloat16)

        for _ in range(2):
            vendor()
        vms = timed(vendor, reps)
    cpu = None
    if cpu_rows > 0:   # the CPU-baseline leg: the oracle, timed as it stands
        import oracle.ffn64 as F

        rows = W.ffn_sample_rows(W.FfnWorkload(fw.name, fw.M, fw.d_model, fw.d_ff, fw.block, fw.act, fw.seed,
                                               sample_rows=cpu_rows))
        xr, w1r, w2r = (W.bf16_bits_to_f64(s) for s in (st[0][rows], st[1], st[3]))
        t0 = time.perf_counter()
        F.ffn_rows(xr, w1r, st[2], w2r, st[4], fw.act)
        cpu_s = time.perf_counter() - t0
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        cpu = {"value": round(4.0 * len(rows) * fw.d_model * fw.d_ff / cpu_s / 1e12, 4), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"fp64 oracle (oracle.ffn64.ffn_rows) on {len(rows)} seeded rows of the {fw.M}: {cpu_s:.1f} s"}
    tflops = fw.flops() / (ms * 1e-3) / 1e12
    return {"what": "attn_ffn_blockwise: act(x W1^T + b1) W2^T + b2 in blocks of rows",
            "config": {"workload": fw.name, "M": fw.M, "d_model": fw.d_model, "d_ff": fw.d_ff, "block": fw.block,
                       "act": fw.act},
            "ms": round(ms, 4), "tflops": round(tflops, 2),
            "gemm_launches": n_gemm / reps, "gemm_ms_avg": round(gemm_ms / max(n_gemm, 1), 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
            "context_only_torch_matmul": None if vms is None else {
                "what": "context only, not a target: torch bf16 matmul for both products per block, torch GELU and "
                        "bias adds", "ms": round(vms, 4), "tflops": round(fw.flops() / (vms * 1e-3) / 1e12, 2)},
            "cpu_baseline": cpu}


def cpu_workers() -> int:
    """Oracle worker threads: the host's CPUs this process may run on, at most 16 (the host share that goes
    with one GPU on the measurement machines)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def host_facts() -> dict:
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"affinity_cpus": len(os.sched_getaffinity(0)), "worker_threads": cpu_workers(), "cpu_model": model}


def cpu_baseline_sampled_rows(w):
    """The oracle (plain form, one pass over all keys) on the seeded query rows per head that the GPU tests
    check for a workload with a row sample (the Ulysses head share: 64 per head), timed on this host; each
    head's rows in one call, the heads on a thread pool with one BLAS thread per worker."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads as W

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows = {bh: W.sample_rows(w, *bh) for bh in heads}
    data = {}

    def run(bh):
        q, k, v = data[bh]
        r = rows[bh]
        oracle.naive_head(q[r], k, v, w.scale, w.causal, w.offset, r)

    dt = 0.0
    with threadpool_limits(limits=1, user_api="blas"):
        # inputs of two heads at a time (K and V of one head are 256 MiB each in fp64); generation is untimed
        for i in range(0, len(heads), 2):
            part = heads[i:i + 2]
            for bh in part:
                data[bh] = tuple(W.head_f64(w, t, *bh) for t in (W.Q_T, W.K_T, W.V_T))
            t0 = time.perf_counter()
            with ThreadPoolExecutor(len(part)) as ex:
                list(ex.map(run, part))
            dt += time.perf_counter() - t0
            for bh in part:
                del data[bh]
    n_rows = sum(len(r) for r in rows.values())
    vis = sum(float((np.minimum(w.N_kv, r + w.offset + 1) if w.causal else np.full(len(r), w.N_kv)).sum())
              for r in rows.values())
    flops = 4.0 * w.d * vis
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "kind": "oracle", "threads": min(2, len(heads)),
            "sample": f"fp64 oracle (plain form) on the {n_rows} seeded query rows ({w.sample_rows} per head) of "
                      f"{w.name}, each against all of its visible keys of the {w.N_kv}: {flops:.3e} FLOP in {dt:.1f} s",
            "full_workload_estimate_s": round(w.flops() / (flops / dt), 1),
            "estimate_note": "row-scaled estimate of the whole workload at this rate (an estimate, not measured)"}


def cpu_baseline(w, seconds: float):
    """Time the fp64 oracle (blockwise form, key blocks of 1024, row blocks of 256) on a bounded sample of
    the workload: about `seconds` of wall time of (head, row block) pairs spread over the heads and over
    each head's query range, every block against all of its keys, on a thread pool with one BLAS thread
    per worker.  Input generation is outside the timed region."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads as W

    workers = cpu_workers()
    rb = 256
    starts = list(range(0, w.N_q, rb))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    cache = {}

    def head(i):
        if i not in cache:
            b, h = heads[i]
            cache[i] = tuple(W.head_f64(w, t, b, h) for t in (W.Q_T, W.K_T, W.V_T))
        return cache[i]

    def run(job):
        i, s = job
        q, k, v = head(i)
        rows = np.arange(s, min(s + rb, w.N_q))
        oracle.blockwise_head(q[rows], k, v, w.scale, w.causal, w.offset, rows, 1024)
        return rows

    with threadpool_limits(limits=1, user_api="blas"):
        # probe one block (a late one: causal rows there see the most keys) to size the sample
        probe_start = starts[-1]
        t0 = time.perf_counter()
        run((0, probe_start))
        one = time.perf_counter() - t0
        nblk = int(max(1, min(len(starts) * len(heads), round(seconds / one * workers))))
        nheads = min(len(heads), -(-nblk // len(starts)))
        per_head = -(-nblk // nheads)
        hsel = [int(j * len(heads) / nheads) for j in range(nheads)]
        jobs = [(i, starts[int(j * len(starts) / per_head)]) for i in hsel for j in range(per_head)]
        for i in hsel:
            head(i)
        t0 = time.perf_counter()
        with ThreadPoolExecutor(workers) as ex:
            done = list(ex.map(run, jobs))
        dt = time.perf_counter() - t0
    rows = np.concatenate(done)
    vis = np.minimum(w.N_kv, rows + w.offset + 1) if w.causal else np.full(len(rows), w.N_kv)
    flops = 4.0 * w.d * float(vis.sum())
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle", **host_facts(),
        "sample": f"fp64 blockwise oracle (single pass, key blocks of 1024) on {len(jobs)} blocks of {rb} query "
                  f"rows: {per_head} blocks spread over the {w.N_q} rows of each of {nheads} of the {len(heads)} "
                  f"heads, each row against all of its visible keys of the {w.N_kv}; {flops:.3e} FLOP in {dt:.1f} s",
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_traffic.txt")
FWD_SOURCE = os.path.join(ROOT, "exact_blockwise_attention_fwd_amd", "csrc", "attn_fwd_bf16.hip")


COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_counters.txt")


def recorded_fields(path, w):
    """The machine-readable `key: value` lines of a counter summary under profiles/, or None when it is
    missing, covers another workload, or was taken on a different build of the forward kernel (its source
    or its compile flags)."""
    from exact_blockwise_attention_fwd_amd.build import fingerprint

    try:
        fields = {}
        for line in open(path):
            if ":" in line and not line.startswith((" ", "#", "|")):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
        if fields.get("kernel_build_sha256") != fingerprint(os.path.basename(FWD_SOURCE)) or \
                fields.get("workload") != w.name:
            return None
        return fields
    except OSError:
        return None


def recorded_source(path, w):
    """Where a recorded field comes from, for the bench line: the summary file and the build it was taken on."""
    f = recorded_fields(path, w)
    if f is None:
        return None
    return {"source": "recorded", "file": os.path.relpath(path, ROOT),
            "kernel_build_sha256": f.get("kernel_build_sha256"),
            "note": "measured by the rocprofv3 harness (python -m exact_blockwise_attention_fwd_amd.profile) on an "
                    "earlier run of this same build, not in this run"}


def recorded_traffic(w):
    """HBM bytes per forward launch (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    plain copy of known size), or None."""
    f = recorded_fields(TRAFFIC_FILE, w)
    try:
        return None if f is None else float(f["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_counters(w):
    """Matrix-core figures of the forward launches from SQ/GRBM counters (mean over the step's launches), or
    None: the fraction of SIMD cycles the MFMA unit was busy, MFMA FLOP issued per algorithmic FLOP, the
    fraction of MFMA-busy cycles with a VALU instruction issued beside it, LDS bank-conflict cycles per
    GUI-active cycle and CU, and the engine clock the GUI-active count implies."""
    f = recorded_fields(COUNTERS_FILE, w)
    keys = ("mfma_busy_frac", "mfma_flop_per_algorithmic_flop", "valu_coexec_frac_of_mfma_busy",
            "lds_bank_conflict_frac", "effective_sclk_ghz")
    try:
        return None if f is None else {k: float(f[k]) for k in keys}
    except (KeyError, ValueError):
        return None


def live_counters(w, limit_s: int = 240):
    """Traffic and matrix-core counters of this workload's forward launches measured in this run: the committed
    rocprofv3 harness (python -m exact_blockwise_attention_fwd_amd.profile) runs as a child process once this
    process has finished its own GPU work, each profiled bench step a grandchild under its own time limit.
    Returns (traffic bytes per launch or None, counters dict or None, source dict); the source carries the
    error text when the child failed."""
    import shutil
    import subprocess
    import tempfile

    from exact_blockwise_attention_fwd_amd.build import fingerprint

    what = ["counters"] if w.dtype == "bf16" else []
    if w.name == "ring_share_128k":
        what.insert(0, "traffic")
    if not what:
        return None, None, {"source": "this run", "error": "no counter passes for this workload"}
    tmp = tempfile.mkdtemp(prefix="attn_live_prof_", dir="/tmp")
    cmd = [sys.executable, "-m", "exact_blockwise_attention_fwd_amd.profile", "--what", ",".join(what),
           "--workloads", w.name, "--out", os.path.join(tmp, "out"), "--raw", os.path.join(tmp, "raw")]
    shown = " ".join(["python3", *cmd[1:7]])
    src = {"source": "this run", "command": shown + " (summaries in a temporary directory)",
           "kernel_build_sha256": fingerprint(os.path.basename(FWD_SOURCE))}
    try:
        # its own session, so that a time limit ends the harness and every profiled grandchild together
        p = subprocess.Popen(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                             start_new_session=True)
        try:
            stdout, _ = p.communicate(timeout=limit_s)
        except subprocess.TimeoutExpired:
            import signal

            os.killpg(p.pid, signal.SIGKILL)
            p.communicate()
            src["error"] = f"harness did not finish within {limit_s} s"
            return None, None, src
        if p.returncode != 0:
            src["error"] = f"harness exit {p.returncode}: {stdout[-400:]}"
            return None, None, src
        traffic = counters = None
        tf = recorded_fields(os.path.join(tmp, "out", os.path.basename(TRAFFIC_FILE)), w)
        if tf is not None:
            traffic = float(tf["hbm_bytes_per_launch"])
        cf = recorded_fields(os.path.join(tmp, "out", os.path.basename(COUNTERS_FILE) if w.name == "ring_share_128k"
                                          else f"attn_fwd_bf16_counters_{w.name}.txt"), w)
        if cf is not None:
            counters = {k: float(cf[k]) for k in ("mfma_busy_frac", "mfma_flop_per_algorithmic_flop",
                                                 "valu_coexec_frac_of_mfma_busy", "lds_bank_conflict_frac",
                                                 "effective_sclk_ghz")}
        return traffic, counters, src
    except Exception as e:   # no profiler, a time limit, unreadable output: fall back to the recorded figures
        src["error"] = f"{type(e).__name__}: {e}"
        return None, None, src
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ring_share_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streamed", action="store_true", help="skip the host-streamed variant of the chunked step")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing of the step")
    ap.add_argument("--no-ffn", action="store_true",
                    help="skip the blockwise feed-forward leg (run with the ring-share workload only)")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-live-counters", action="store_true",
                    help="report the recorded traffic and counters instead of measuring them with the harness")
    ap.add_argument("--clock-seconds", type=float, default=CLOCK_SECONDS,
                    help="length of the run after each timed region over which clock and power are sampled (0: none)")
    ap.add_argument("--no-ulysses", action="store_true",
                    help="skip the Ulysses head-share object (run with the ring-share workload only)")
    ap.add_argument("--ffn-vendor-context", action="store_true",
                    help="also time torch's matmul for the feed-forward's products (context only)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (practical HBM ceiling; also the "
                         "reference size for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is one device's share); --gpus {args.gpus} is not "
              "supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_blockwise_attention_fwd_amd as A
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / args.steps
        print(json.dumps({"copy_bytes": n, "ms_per_copy": ms, "gbs_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}))
        return
    A.lib()
    w = W.WORKLOADS[args.workload]
    log(f"workload {w}")
    t0 = time.time()

    def dev(t):
        import numpy as np
        s = W.tensor_storage(w, t)
        if s.dtype == np.uint16:
            return torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(s).cuda()

    q, k, v = dev(W.Q_T), dev(W.K_T), dev(W.V_T)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device="cuda")
    ws_n = A.workspace_bytes(w.B, w.H, w.N_q, w.d, w.chunks)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs resident in {time.time() - t0:.1f} s")

    def step():
        if w.chunks > 1:
            A.fwd_chunked(q, k, v, w.chunks, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)
        else:
            A.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    A.timing_enable(True)
    A.timing_read()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]   # per-step spread
    e0.record(stream)
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    A.timing_enable(False)
    kt = A.timing_read()
    total_ms = e0.elapsed_time(e1)
    ms = total_ms / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    log(f"timed {args.steps} steps: {ms:.3f} ms/step; kernels {kt}")

    flops = w.flops()
    value = flops / (ms * 1e-3) / 1e12
    n_fwd, fwd_ms = kt["fwd"]
    fwd_tflops = flops * args.steps / (fwd_ms * 1e-3) / 1e12 if fwd_ms > 0 else None
    clock_power = None
    if args.clock_seconds > 0:
        clock_power = sample_clock_power(step, fwd_tflops if w.dtype == "bf16" else None, args.clock_seconds)
        log(f"clock and power: {clock_power}")
    merge_ms = time_merge(w, 10)
    mb = merge_bytes(w)
    merge_gbs = mb / (merge_ms * 1e-3) / 1e9 if merge_ms > 0 else None
    copy_gbs = time_copy(1 << 30, 10)
    log(f"attn_merge alone: {merge_ms:.4f} ms, {merge_gbs:.1f} GB/s; 1 GiB device copy {copy_gbs:.1f} GB/s")
    # one exponential per visible (query, key) pair; not counted in the FLOPs
    pairs = w.B * w.H * w.visible_pairs()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.N_q, "N_kv": w.N_kv, "d": w.d,
                   "causal": w.causal, "chunks": w.chunks, "scale": w.scale, "parallelism": "single-gpu"},
        "pct_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "step_ms": {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
                    "max": round(per_step[-1], 4)},
        "fwd_kernel": {"launches_per_step": n_fwd / args.steps, "ms_per_step": fwd_ms / args.steps,
                       "tflops": None if fwd_tflops is None else round(fwd_tflops, 2),
                       "exp_per_s": None if fwd_ms <= 0 else float(f"{pairs * args.steps / (fwd_ms * 1e-3):.4e}")},
        "merge": None if merge_gbs is None else {
            "what": "attn_merge alone, fp32 partials in place, rows = B*H*N_q", "rows": w.B * w.H * w.N_q,
            "ms": round(merge_ms, 4), "bytes": mb, "gbs": round(merge_gbs, 1),
            "pct_hbm_peak": round(100 * merge_gbs / HBM_PEAK_GBS, 2),
            "device_copy_gbs": round(copy_gbs, 1), "frac_of_device_copy": round(merge_gbs / copy_gbs, 4)},
        "roofline": {"bound": "mfma", "achieved": None if fwd_tflops is None else round(fwd_tflops, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": None if fwd_tflops is None else round(fwd_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(w)},
        "clock_power": clock_power,
        "counters": recorded_counters(w),
        "counters_source": recorded_source(COUNTERS_FILE, w),
        "traffic_source": recorded_source(TRAFFIC_FILE, w),
        "ulysses": None,
        "graph": None,
        "streamed": None,
        "ffn": None,
        "cpu_baseline": None,
    }
    if w.dtype != "bf16":
        # the fp32 kernel forms QK^T in fp64 FMAs (PV in fp32); at half the fp32 rate they set its ALU ceiling
        out["roofline"].update({"bound": "alu", "peak": FP64_PEAK_TFLOPS,
                                "frac": None if fwd_tflops is None else round(fwd_tflops / FP64_PEAK_TFLOPS, 4)})
    if not args.no_graph:
        gms = time_graph(step, args.steps)
        out["graph"] = {"what": "the same step captured once into a HIP graph and replayed", "steps": args.steps,
                        "ms_per_step": round(gms, 4), "tflops": round(flops / (gms * 1e-3) / 1e12, 2)}
        log(f"graph replay: {out['graph']}")
    if w.chunks > 1 and not args.no_streamed:
        log("timing the host-streamed chunked step")
        out["streamed"] = time_streamed(w, q, k, v, max(2, min(args.steps, 5)), ms)
        log(f"streamed: {out['streamed']}")
    if w.name == "ring_share_128k" and not args.no_ffn:
        log("timing the blockwise feed-forward of the same model")
        out["ffn"] = time_ffn(10, 0 if args.no_cpu_baseline else 4096, args.ffn_vendor_context)
        log(f"ffn: {out['ffn']}")
    if w.name == "ring_share_128k" and not args.no_ulysses:
        log("timing the Ulysses head share (the other causal long-sequence workload)")
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()
        out["ulysses"] = time_workload(W.WORKLOADS["ulysses_share_256k"], 5, 1, args.clock_seconds)
        log(f"ulysses: {out['ulysses']}")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        if out["ulysses"] is not None:
            log("timing the CPU oracle on the Ulysses share's seeded rows")
            out["ulysses"]["cpu_baseline"] = cpu_baseline_sampled_rows(W.WORKLOADS["ulysses_share_256k"])
    if not args.no_live_counters:
        log("measuring traffic and matrix-core counters with the rocprofv3 harness (child processes)")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        traffic, ctrs, src = live_counters(w)
        log(f"live counters: traffic {traffic}, counters {ctrs}, source {src}")
        if traffic is not None:
            out["roofline"]["traffic"] = traffic
            out["traffic_source"] = src
        elif out["traffic_source"] is not None and "error" in src:
            out["traffic_source"]["live_error"] = src["error"]
        if ctrs is not None:
            out["counters"] = ctrs
            out["counters_source"] = src
        elif out["counters_source"] is not None and "error" in src:
            out["counters_source"]["live_error"] = src["error"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
