#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled NT GEMM hot path on one MI355X.

A step is one pass of the hot path over one batch: quantise the fp32
activations to e4m3 with 1x128 scales, then the FP8 NT GEMM with the
128x128-scaled weights (quantised once beforehand, as weights are).  The
headline workload is the dense decode shape M=64 N=2112 K=7168 (activations
N(0,1), weights N(0,0.02), seed 0), reported as HBM GB/s of algorithmic bytes.

Measurements
  * value / ms_per_step: K steps captured in one HIP graph, replayed once,
    bracketed by torch.cuda.synchronize() and the host clock.  Each step uses
    a different copy of the operands (rotation over > 512 MiB) so no step is
    served from the 256 MiB Infinity Cache.
  * roofline: the GEMM kernel alone, its own duration from events recorded at
    kernel start and end (hipExtLaunchKernel through dg_profile_next_launch),
    averaged over the timed launches.
  * cpu_baseline: the CPU oracle (numpy, fp64) running the same step on the
    host for a bounded sample.
  * extra: every other workload's GEMM kernel timed the same way.

Prints one JSON line on stdout.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4 MFMA
ROTATE_BYTES = 600 << 20       # > 2x the 256 MiB Infinity Cache
MAIN_WORKLOAD = "dense_decode_64x2112x7168"
CALIB_BYTES = 1 << 30          # plain-kernel traffic for the counter calibration
METRIC = "FP8 block-scaled GEMM TFLOPS (large) & HBM GB/s (decode) on 1 GPU; % of roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--kernel-launches", type=int, default=200,
                    help="timed GEMM launches per workload for the kernel figures")
    ap.add_argument("--workloads", default="all",
                    help="'all', 'main', or a comma list of workload names for the extra figures")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--mode", choices=["bench", "counters", "oracle", "tiles"], default="bench",
                    help="counters: run plain kernels of known traffic (1 GiB fill, 1 GiB read; "
                         "calibration for rocprofv3 FETCH_SIZE/WRITE_SIZE), then eager GEMM launches "
                         "of the headline workload and of the --workloads list ('main' = none), "
                         "print nothing; oracle: time the CPU oracle's GEMM on the five configurations "
                         "and print one JSON line; tiles: the large dense GEMM's 256 x 256 tile, "
                         "unsplit, at 256, 448 and 512 tiles (N 4096, 7168, 8192), --kernel-launches "
                         "back-to-back launches each, one JSON line")
    return ap.parse_args()


def source_hash():
    """Hash of the kernel sources with comments and blank space removed, so
    that an edit of comments alone keeps the recorded counters valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_block_scaled_nt_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(f.encode() + text.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("bytes_per_launch")


class Rotation:
    """R copies of one workload's device operands, R chosen so the copies span
    more than the Infinity Cache."""

    def __init__(self, make_set, set_bytes):
        self.r = max(2, -(-ROTATE_BYTES // max(set_bytes, 1)))
        self.sets = [make_set(i) for i in range(self.r)]

    def __getitem__(self, i):
        return self.sets[i % self.r]


class ClockSampler:
    """Samples the GPU's current shader (GFX) clock through amdsmi from a host
    thread while kernels run; the samples taken during a timed region are its
    SCLK record.  Empty when amdsmi is not available."""

    def __init__(self):
        self.handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                self.amdsmi = amdsmi
                self.handle = handles[0]
        except Exception:  # pragma: no cover - informational only
            self.handle = None
        self.samples = []
        self._stop = None

    def read_mhz(self):
        if self.handle is None:
            return None
        try:
            info = self.amdsmi.amdsmi_get_clock_info(self.handle, self.amdsmi.AmdSmiClkType.GFX)
            v = info.get("clk", info.get("cur_clk"))
            return float(v) if v is not None else None
        except Exception:  # pragma: no cover
            return None

    def __enter__(self):
        import threading
        self.samples = []
        if self.handle is None:
            return self
        self._stop = threading.Event()
        first = threading.Event()

        def run():
            while not self._stop.is_set():
                v = self.read_mhz()
                if v is not None:
                    self.samples.append(v)
                first.set()
                time.sleep(0.0005)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        # the thread's start-up and first (slowest) query stay out of the
        # timed region that follows
        first.wait(1.0)
        return self

    def __exit__(self, *exc):
        if self._stop is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        s = sorted(self.samples)
        return {"samples": len(s), "median_mhz": s[len(s) // 2], "min_mhz": s[0], "max_mhz": s[-1]}


CLOCK = None


def kernel_time_us(torch, dg, launch, rot, n_launch, warm=20):
    """Duration of the GEMM kernel itself over n_launch launches (events at
    kernel start and end): average, median, p10, p90, and the shader clock
    sampled meanwhile."""
    for i in range(warm):
        launch(rot[i])
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
    for e in starts + stops:
        e.record()  # materialise the underlying HIP events
    torch.cuda.synchronize()
    with CLOCK:
        t0 = time.perf_counter()
        for i in range(n_launch):
            dg.profile_next_launch(starts[i], stops[i])
            launch(rot[warm + i])
        torch.cuda.synchronize()
        window_ms = (time.perf_counter() - t0) * 1e3
    times = sorted(starts[i].elapsed_time(stops[i]) * 1e3 for i in range(n_launch))
    pct = lambda q: times[min(len(times) - 1, int(q * len(times)))]
    sclk = CLOCK.summary()
    if sclk is not None:
        # amdsmi reports the clock level the power manager has set; between
        # short launches that is an idle level, so the window and the share
        # of it the kernels kept the GPU busy go with the samples
        sclk["window_ms"] = round(window_ms, 2)
        sclk["busy_share"] = round(sum(times) / 1e3 / window_ms, 3)
    return {"avg": sum(times) / len(times), "median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9),
            "sclk": sclk}


def kernel_b2b_us(torch, dg, launch, rot, n_launch, start, ws_bytes=0):
    """Average duration of the GEMM kernel in back-to-back launches, the way
    the timed steps run it: n_launch launches on rotated operands captured in
    one graph, hip events around a replay of the graph, divided by n_launch
    (so the launch gaps inside the graph count against the kernel).  Single
    launches with the GPU idle in between (kernel_time_us) also pay the GPU's
    wake-up: the XCDs then begin the grid up to 4 us apart."""
    stream = torch.cuda.Stream()
    if ws_bytes:
        dg.reserve_workspace(ws_bytes, stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n_launch):
                launch(rot[start + i])
    torch.cuda.synchronize()
    g.replay()  # warm-up replay
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n_launch
    del g
    return us


def workspace_bytes(dg, kind, params):
    """Split-K workspace a dense launch of this workload takes (0 otherwise)."""
    if kind not in ("dense", "bf16", "fp4"):
        return 0
    dtype = {"dense": "fp8"}.get(kind, kind)
    return dg.dense_workspace_size(params["m"], params["n"], params["k"], dtype)


def setup_workload(torch, np, dg, W, name, dev):
    """Device operands for one workload, quantised by the library's own
    quantisers; returns (kind, params, rotation, launch, inputs)."""
    w = W.WORKLOADS[name]
    s = w.shape
    inp = W.draw(name)
    if w.kind == "dense":
        m, n, k = s["m"], s["n"], s["k"]
        xa = torch.from_numpy(inp["a"]).to(dev)
        xb = torch.from_numpy(inp["b"]).to(dev)
        qb, sfb = dg.quantize_b_128x128(xb)
        del xb

        def make(i):
            qa, sfa = dg.quantize_a_1x128(xa)
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            return {"xa": xa.clone() if i else xa, "qa": qa, "sfa": sfa,
                    "qb": qb.clone() if i else qb, "sfb": sfb.clone(), "d": d}

        set_bytes = m * k * 5 + n * k + 2 * m * n
        rot = Rotation(make, set_bytes)

        def launch(st):
            dg.fp8_gemm_nt((st["qa"], st["sfa"]), (st["qb"], st["sfb"]), st["d"])

        def quant(st):
            dg.quantize_a_1x128(st["xa"], st["qa"], st["sfa"])

        return w.kind, dict(m=m, n=n, k=k), rot, launch, quant, inp
    if w.kind == "contiguous":
        n, k = s["n"], s["k"]
        idx = torch.from_numpy(inp["m_indices"]).to(dev)
        m = idx.numel()
        xa = torch.from_numpy(inp["a"]).to(dev)
        qb, sfb = dg.quantize_b_128x128(torch.from_numpy(inp["b"]).to(dev))
        qa, sfa = dg.quantize_a_1x128(xa)
        del xa

        def make(i):
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            if i == 0:
                return {"qa": qa, "sfa": sfa, "qb": qb, "sfb": sfb, "d": d, "idx": idx}
            return {"qa": qa.clone(), "sfa": sfa.clone(), "qb": qb.clone(), "sfb": sfb.clone(),
                    "d": d, "idx": idx.clone()}

        rot = Rotation(make, m * k + qb.numel() + 2 * m * n)

        def launch(st):
            dg.m_grouped_fp8_gemm_nt_contiguous((st["qa"], st["sfa"]), (st["qb"], st["sfb"]), st["d"], st["idx"])

        return w.kind, dict(m_indices=inp["m_indices"], g=len(s["group_rows"]), n=n, k=k), rot, launch, None, inp
    if w.kind == "bf16":
        m, n, k = s["m"], s["n"], s["k"]
        a16 = torch.from_numpy(inp["a"]).to(dev).to(torch.bfloat16)
        b16 = torch.from_numpy(inp["b"]).to(dev).to(torch.bfloat16)

        def make(i):
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            if i == 0:
                return {"a": a16, "b": b16, "d": d}
            return {"a": a16.clone(), "b": b16.clone(), "d": d}

        rot = Rotation(make, 2 * (m * k + n * k + m * n))

        def launch(st):
            dg.bf16_gemm_nt(st["a"], st["b"], st["d"])

        return w.kind, dict(m=m, n=n, k=k), rot, launch, None, inp
    if w.kind == "fp4":
        m, n, k = s["m"], s["n"], s["k"]
        qa, sfa = dg.quantize_a_1x128_fp4(torch.from_numpy(inp["a"]).to(dev))
        qb, sfb = dg.quantize_b_128x128_fp4(torch.from_numpy(inp["b"]).to(dev))

        def make(i):
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            if i == 0:
                return {"qa": qa, "sfa": sfa, "qb": qb, "sfb": sfb, "d": d}
            return {"qa": qa.clone(), "sfa": sfa.clone(), "qb": qb.clone(), "sfb": sfb.clone(), "d": d}

        rot = Rotation(make, qa.numel() + qb.numel() + 2 * m * n)

        def launch(st):
            dg.fp4_gemm_nt((st["qa"], st["sfa"]), (st["qb"], st["sfb"]), st["d"])

        return w.kind, dict(m=m, n=n, k=k), rot, launch, None, inp
    if w.kind == "kgrouped":
        m, n = s["m"], s["n"]
        ks = torch.from_numpy(inp["k_sizes"]).to(dev)
        k = inp["a"].shape[1]
        qa, sfa = dg.quantize_a_1x128(torch.from_numpy(inp["a"]).to(dev))
        qb, sfb = dg.quantize_b_128x128(torch.from_numpy(inp["b"]).to(dev))
        g = ks.numel()

        def make(i):
            d = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
            if i == 0:
                return {"qa": qa, "sfa": sfa, "qb": qb, "sfb": sfb, "d": d, "ks": ks}
            return {"qa": qa.clone(), "sfa": sfa.clone(), "qb": qb.clone(), "sfb": sfb.clone(), "d": d,
                    "ks": ks.clone()}

        rot = Rotation(make, qa.numel() + qb.numel() + 2 * g * m * n)

        def launch(st):
            dg.k_grouped_fp8_gemm_nt((st["qa"], st["sfa"]), (st["qb"], st["sfb"]), st["d"], st["ks"])

        return w.kind, dict(k_sizes=inp["k_sizes"], m=m, n=n, k=k), rot, launch, None, inp
    if w.kind == "swiglu_contig":
        inter, k = s["inter"], s["k"]
        idx = torch.from_numpy(inp["m_indices"]).to(dev)
        m = idx.numel()
        qa, sfa = dg.quantize_a_1x128(torch.from_numpy(inp["a"]).to(dev))
        qb, sfb = dg.quantize_b_128x128(torch.from_numpy(inp["b"]).to(dev))
        ld = dg.get_sfa_ld(m)

        def make(i):
            hq = torch.empty((m, inter), dtype=torch.float8_e4m3fn, device=dev)
            hs = torch.empty((inter // 128, ld), dtype=torch.float32, device=dev)
            if i == 0:
                return {"qa": qa, "sfa": sfa, "qb": qb, "sfb": sfb, "hq": hq, "hs": hs, "idx": idx}
            return {"qa": qa.clone(), "sfa": sfa.clone(), "qb": qb.clone(), "sfb": sfb.clone(), "hq": hq,
                    "hs": hs, "idx": idx.clone()}

        rot = Rotation(make, qa.numel() + qb.numel() + m * inter)

        def launch(st):
            dg.m_grouped_fp8_gemm_nt_contiguous_swiglu((st["qa"], st["sfa"]), (st["qb"], st["sfb"]),
                                                       (st["hq"], st["hs"]), st["idx"])

        return (w.kind, dict(m_indices=inp["m_indices"], g=len(s["group_rows"]), n=2 * inter, k=k), rot, launch,
                None, inp)
    if w.kind == "swiglu":
        g, max_m, inter, k = s["g"], s["max_m"], s["inter"], s["k"]
        mm = torch.from_numpy(inp["masked_m"]).to(dev)
        qa, sfa = dg.quantize_a_1x128(torch.from_numpy(inp["a"]).to(dev))
        qb, sfb = dg.quantize_b_128x128(torch.from_numpy(inp["b"]).to(dev))
        ld = dg.get_sfa_ld(max_m)

        def make(i):
            hq = torch.empty((g, max_m, inter), dtype=torch.float8_e4m3fn, device=dev)
            hs = torch.empty((g, inter // 128, ld), dtype=torch.float32, device=dev)
            if i == 0:
                return {"qa": qa, "sfa": sfa, "qb": qb, "sfb": sfb, "hq": hq, "hs": hs, "mm": mm}
            return {"qa": qa.clone(), "sfa": sfa.clone(), "qb": qb.clone(), "sfb": sfb.clone(), "hq": hq,
                    "hs": hs, "mm": mm.clone()}

        rot = Rotation(make, qa.numel() + qb.numel() + g * max_m * inter)
        expected = int(np.clip(inp["masked_m"], 0, max_m).mean())

        def launch(st):
            dg.m_grouped_fp8_gemm_nt_masked_swiglu((st["qa"], st["sfa"]), (st["qb"], st["sfb"]),
                                                   (st["hq"], st["hs"]), st["mm"], expected)

        return w.kind, dict(masked_m=inp["masked_m"], max_m=max_m, n=2 * inter, k=k), rot, launch, None, inp
    g, max_m, n, k = s["g"], s["max_m"], s["n"], s["k"]
    mm = torch.from_numpy(inp["masked_m"]).to(dev)
    qa, sfa = dg.quantize_a_1x128(torch.from_numpy(inp["a"]).to(dev))
    qb, sfb = dg.quantize_b_128x128(torch.from_numpy(inp["b"]).to(dev))

    def make(i):
        d = torch.empty((g, max_m, n), dtype=torch.bfloat16, device=dev)
        if i == 0:
            return {"qa": qa, "sfa": sfa, "qb": qb, "sfb": sfb, "d": d, "mm": mm}
        return {"qa": qa.clone(), "sfa": sfa.clone(), "qb": qb.clone(), "sfb": sfb.clone(), "d": d,
                "mm": mm.clone()}

    rot = Rotation(make, qa.numel() + qb.numel() + 2 * g * max_m * n)
    expected = int(np.clip(inp["masked_m"], 0, max_m).mean())

    def launch(st):
        dg.m_grouped_fp8_gemm_nt_masked((st["qa"], st["sfa"]), (st["qb"], st["sfb"]), st["d"], st["mm"], expected)

    return w.kind, dict(masked_m=inp["masked_m"], max_m=max_m, n=n, k=k), rot, launch, None, inp


def host_info():
    """CPU model, the cores this process may run on, and NumPy's BLAS."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
    except Exception:  # pragma: no cover - informational only
        pass
    return model, cores, blas


def blas_threads(cores):
    """Context that runs NumPy's BLAS on `cores` threads (no-op without threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def cpu_oracle_baseline(np, W, inp, m, n, k, seconds):
    """Time the oracle doing the main step (quantise A, GEMM) on the host, on
    every core of this process's affinity set."""
    import oracle
    model, cores, blas = host_info()
    qb, sb = oracle.quantize_b_128x128(inp["b"])  # weights: outside the timed loop
    flops, gemm_bytes = W.algorithmic_work("dense", m=m, n=n, k=k)
    step_bytes = gemm_bytes + m * k * 4 + m * k + 4 * m * (k // 128)
    with blas_threads(cores):
        t0 = time.perf_counter()
        iters = 0
        while True:
            qa, sa = oracle.quantize_a_1x128(inp["a"])
            oracle.gemm_nt_ref(qa, sa, qb, sb)
            iters += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": step_bytes * iters / el / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu": model, "blas": blas,
            "sample": f"the whole decode step (quantise A 64x7168, fp64 GEMM 64x2112x7168) "
                      f"x{iters} in {el:.1f} s; {flops * iters / el / 1e9:.2f} GFLOP/s"}


ORACLE_CONFIGS = ["dense_128x512x1024", "dense_decode_64x2112x7168", "dense_large_4096x7168x16384",
                  "moe_contiguous_4x8192_n4096_k7168", "moe_masked_16x256_n4096_k7168"]


def tile_count_timing(np, W, launches):
    """The large dense GEMM (M 4096, K 16384) with its 256 x 256 tile and no
    split at N = 4096, 7168 and 8192: 256 tiles (one per CU), 448 and 512.
    Back-to-back launches timed by wall clock between two synchronisations,
    so the cost of the last, partial wave of tiles shows against the work."""
    import torch

    import fp8_block_scaled_nt_amd as dg
    dev = torch.device("cuda:0")
    os.environ["DG_FORCE_CONFIG"] = "dense_256x256_w8_s2"
    os.environ["DG_SPLIT_K"] = "1"
    m, k = 4096, 16384
    rows = []
    try:
        for n in (4096, 7168, 8192):
            x = W.draw_dense(m, n, k, seed=0)
            qa, sfa = dg.quantize_a_1x128(torch.from_numpy(x["a"]).to(dev))
            qb, sfb = dg.quantize_b_128x128(torch.from_numpy(x["b"]).to(dev))
            del x
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(launches):
                dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d)
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) / launches * 1e6
            tiles = (m // 256) * (n // 256)
            rows.append({"n": n, "tiles": tiles, "us": round(us, 1),
                         "tflops": round(2.0 * m * n * k / us / 1e6, 1)})
            print(f"[tiles] N {n}: {tiles} tiles, {us:.1f} us", file=sys.stderr, flush=True)
            del qa, sfa, qb, sfb, d
            torch.cuda.empty_cache()
    finally:
        os.environ.pop("DG_FORCE_CONFIG", None)
        os.environ.pop("DG_SPLIT_K", None)
    return rows


def oracle_timing(np, W):
    """The oracle's GEMM on each of the five configurations, on the host's
    cores: the two large ones once, the others best of three.  Inputs are the
    workloads' seeded draws, quantised by the oracle outside the timing."""
    import oracle
    model, cores, blas = host_info()
    rows = []
    for name in ORACLE_CONFIGS:
        w = W.WORKLOADS[name]
        inp = W.draw(name)
        if w.kind == "dense":
            qa, sa = oracle.quantize_a_1x128(inp["a"])
            qb, sb = oracle.quantize_b_128x128(inp["b"])
            run = lambda: oracle.gemm_nt_ref(qa, sa, qb, sb)
        elif w.kind == "contiguous":
            qa, sa = oracle.quantize_a_1x128(inp["a"])
            qbs = [oracle.quantize_b_128x128(inp["b"][g]) for g in range(inp["b"].shape[0])]
            qb = np.stack([q for q, _ in qbs])
            sb = np.stack([s for _, s in qbs])
            run = lambda: oracle.grouped_contiguous_ref(qa, sa, qb, sb, inp["m_indices"])
        else:
            g = inp["a"].shape[0]
            qas = [oracle.quantize_a_1x128(inp["a"][i]) for i in range(g)]
            qbs = [oracle.quantize_b_128x128(inp["b"][i]) for i in range(g)]
            qa = np.stack([q for q, _ in qas])
            sa = np.stack([s for _, s in qas])
            qb = np.stack([q for q, _ in qbs])
            sb = np.stack([s for _, s in qbs])
            run = lambda: oracle.grouped_masked_ref(qa, sa, qb, sb, inp["masked_m"])
        reps = 1 if name in ("dense_large_4096x7168x16384", "moe_contiguous_4x8192_n4096_k7168") else 3
        best = None
        with blas_threads(cores):
            for _ in range(reps):
                t0 = time.perf_counter()
                run()
                el = time.perf_counter() - t0
                best = el if best is None else min(best, el)
        fl, by = W.workload_work(name, inp)
        rows.append({"workload": name, "seconds": round(best, 3), "reps": reps,
                     "gflops": round(fl / best / 1e9, 2), "gbs": round(by / best / 1e9, 3)})
        print(f"[oracle] {name}: {best:.3f} s (best of {reps}), {fl / best / 1e9:.2f} GFLOP/s",
              file=sys.stderr, flush=True)
        del inp
    return {"cpu": model, "cores": cores, "blas": blas, "configs": rows}


def main():
    global CLOCK
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
    import numpy as np

    import workloads as W
    if args.mode == "oracle":
        print(json.dumps({"oracle_cpu_timing": oracle_timing(np, W)}))
        return 0
    if args.mode == "tiles":
        print(json.dumps({"tile_count_timing": tile_count_timing(np, W, args.kernel_launches)}))
        return 0

    import torch

    import fp8_block_scaled_nt_amd as dg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    CLOCK = ClockSampler()

    # ---- headline step: quantise A + GEMM on the decode shape
    kind, params, rot, launch, quant, inp = setup_workload(torch, np, dg, W, MAIN_WORKLOAD, dev)
    if args.mode == "counters":
        # plain kernels of known traffic: fill (writes CALIB_BYTES), a second fill
        # that evicts the first from the Infinity Cache, then a sum that reads
        # CALIB_BYTES from HBM
        x = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        float(x.sum())
        del x, y
        torch.cuda.synchronize()
        for i in range(args.kernel_launches):
            launch(rot[i])
        torch.cuda.synchronize()
        del rot
        torch.cuda.empty_cache()
        names = [] if args.workloads == "main" else (
            [x for x in W.WORKLOADS if x != MAIN_WORKLOAD] if args.workloads == "all"
            else args.workloads.split(","))
        for name in names:
            _, _, rot_x, launch_x, _, inp_x = setup_workload(torch, np, dg, W, name, dev)
            for i in range(args.kernel_launches):
                launch_x(rot_x[i])
            torch.cuda.synchronize()
            print(f"[counters] {name}: {args.kernel_launches} launches", file=sys.stderr, flush=True)
            del rot_x, inp_x
            torch.cuda.empty_cache()
        return 0
    m, n, k = params["m"], params["n"], params["k"]
    flops, gemm_bytes = W.algorithmic_work("dense", m=m, n=n, k=k)
    quant_bytes = m * k * 4 + m * k + 4 * m * (k // 128)
    step_bytes = gemm_bytes + quant_bytes

    def step(i):
        st = rot[i]
        quant(st)
        launch(st)

    for i in range(min(args.warmup, 8)):  # eager warm-up before capture
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    # the split-K workspace of the capture stream, sized before capture
    dg.reserve_workspace(dg.dense_workspace_size(m, n, k), stream)
    g_warm = torch.cuda.CUDAGraph()
    g_main = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g_warm, stream=stream):
            for i in range(args.warmup):
                step(i)
        # the timed steps continue the rotation after the warm-up's sets, so
        # no timed step finds its operands where a warm-up step left them
        with torch.cuda.graph(g_main, stream=stream):
            for i in range(args.steps):
                step(args.warmup + i)
    torch.cuda.synchronize()
    g_warm.replay()
    torch.cuda.synchronize()
    with CLOCK:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_main.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    step_clock = CLOCK.summary()
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes * args.steps / wall / 1e9

    # ---- the GEMM kernel alone: back-to-back launches (as in the timed
    # steps) for the roofline, single launches for the spread
    kt = kernel_time_us(torch, dg, launch, rot, args.kernel_launches)
    avg_us = kernel_b2b_us(torch, dg, launch, rot, args.kernel_launches, 20 + args.kernel_launches,
                           dg.dense_workspace_size(m, n, k))
    achieved = gemm_bytes / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(MAIN_WORKLOAD),
                "kernel": "gemm_fp8_nt_kernel<64, 32, 2, 2, 6, dense, three slabs per step> (dense fp8, 64 x 32 tiles, split-K 7)",
                "kernel_avg_us": round(avg_us, 3),
                "kernel_timing": "back-to-back launches in one graph, events around it / launches",
                "launches": args.kernel_launches,
                "single_launch_us": {"avg": round(kt["avg"], 3), "median": round(kt["median"], 3),
                                     "p10": round(kt["p10"], 3), "p90": round(kt["p90"], 3),
                                     "sclk": kt["sclk"]},
                "algorithmic_bytes": gemm_bytes}

    # ---- other workloads: GEMM kernel figures
    extra = {}
    names = [] if args.workloads == "main" else (
        [x for x in W.WORKLOADS if x != MAIN_WORKLOAD] if args.workloads == "all" else args.workloads.split(","))
    del rot
    torch.cuda.empty_cache()
    for name in names:
        kind_x, p_x, rot_x, launch_x, _, inp_x = setup_workload(torch, np, dg, W, name, dev)
        fl, by = W.algorithmic_work(kind_x, **p_x)
        n_x = max(10, args.kernel_launches // 4)
        kx = kernel_time_us(torch, dg, launch_x, rot_x, n_x)
        # back-to-back graph of at most ~20 ms
        n_b2b = int(min(args.kernel_launches, max(10, 20000 // max(kx["median"], 1.0))))
        a_us = kernel_b2b_us(torch, dg, launch_x, rot_x, n_b2b, 20 + n_x, workspace_bytes(dg, kind_x, p_x))
        tf = fl / (a_us * 1e-6) / 1e12
        gbs = by / (a_us * 1e-6) / 1e9
        peak_tf = {"bf16": BF16_PEAK_TFLOPS, "fp4": FP4_PEAK_TFLOPS}.get(kind_x, FP8_PEAK_TFLOPS)
        bound = "mfma" if fl / by > peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
        extra[name] = {"kernel_avg_us": round(a_us, 2), "launches": n_b2b,
                       "single_launch_us": {"avg": round(kx["avg"], 2), "median": round(kx["median"], 2),
                                            "p10": round(kx["p10"], 2), "p90": round(kx["p90"], 2)},
                       "tflops": round(tf, 1), "gbs": round(gbs, 1), "bound": bound,
                       "peak": peak_tf if bound == "mfma" else HBM_PEAK_GBS,
                       "frac": round(tf / peak_tf if bound == "mfma" else gbs / HBM_PEAK_GBS, 4),
                       "sclk": kx["sclk"],
                       "algorithmic_flops": fl, "algorithmic_bytes": by, "traffic": measured_traffic(name)}
        print(f"[bench] {name}: {a_us:.1f} us, {tf:.1f} TFLOP/s, {gbs:.0f} GB/s, sclk {kx['sclk']}",
              file=sys.stderr, flush=True)
        del rot_x, inp_x
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_oracle_baseline(np, W, inp, m, n, k, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 promotion, bf16 out)",
        "data": "synthetic (numpy default_rng(0): activations N(0,1), weights N(0,0.02))",
        "config": {"workload": MAIN_WORKLOAD, "m": m, "n": n, "k": k,
                   "step": "quantise A 1x128 + FP8 NT GEMM (B quantised 128x128 once)",
                   "step_algorithmic_bytes": step_bytes, "gemm_algorithmic_flops": flops,
                   "rotation_sets": "operand copies > 512 MiB, one per step; timed steps continue after the "
                                    "warm-up's sets", "graph": True, "step_sclk": step_clock,
                   "gpu": props.name, "cus": props.multi_processor_count},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
