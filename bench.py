"""Benchmark of the fused exact attention (forward + backward) on one MI355X.

One step = attn_fwd followed by the backward stages attn_bwd runs (the dq stage,
which also forms delta~ = rowsum(dO O), then dkdv) on
one batch of the headline workload, B=2, H=32, N=8192, d=128, bf16, causal,
with inputs already resident in device memory.  Prints one JSON line.
Workloads without a backward pass (fp32_small, bf16_n256_d64_short) time the
forward alone.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                    [--batch B] [--heads H] [--no-cpu-baseline]
                    [--block-density P] [--dropout P] [--fp8] [--decode NQ [--decode-nk NK]]

--flush-l2 writes a 512 MiB scratch buffer before every step (outside the timed
kernels), so the inputs start from HBM; value then uses the kernels' event times.
--block-density P times the block-sparse entry points instead, on a seeded
random mask over 128 x 128 blocks (each block on with probability P, diagonal
blocks always on), counting only the allowed (query, key) pairs.
--dropout P times attn_fwd_dropout + attn_bwd_dropout at rate P (every pair is
still computed, so the FLOP counts are the dense ones).
--fp8 times attn_fwd_fp8 on the workload's shape (e4m3 Q, K, V; bf16 O), with
the bf16 forward on the same shape beside it, priced against the fp8 peak.
--decode NQ times attn_decode: NQ new queries per head against a KV cache of
--decode-nk keys (B=4, H=32, d=128 unless --batch/--heads say otherwise),
priced against HBM bandwidth (it reads each cached key and value once);
--graph captures the K timed calls in one HIP graph and times its replay.

--warmup W untimed steps come first.  For the first tens of milliseconds after
the GPU leaves idle its clock is still ramping and the kernels run 10-20%
slower, so a workload whose step takes under a millisecond wants W large enough
for ~0.15 s of steps (e.g. 500 at N=2048, 2000 for bf16_n256_d64_short); at
N >= 8192 the default 3 measures the same as 60.

Reported:
  value         whole-step attention TFLOP/s, (F_fwd + F_bwd) / t_step, with the
                algorithmic FLOP counts 4*B*H*N^2*d (halved when causal) and
                2.5x that for the backward
  fwd_tflops    forward alone, from HIP events around attn_fwd
  roofline      the kernel with the largest share of the step, against the
                bf16 dense MFMA peak; its average launch time comes from HIP
                events recorded around it inside the timed steps.  A forward
                whose FLOP/byte ratio is below the machine balance (MFMA peak /
                HBM peak) is priced against HBM bandwidth instead, and the fp32
                forward against the fp32 vector peak
  cpu_baseline  the fp64 CPU oracle, timed on a bounded sample of heads
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak (published)
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (published)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3,
                    help="untimed steps first; sub-millisecond steps want ~0.15 s of them (the GPU clock ramps up)")
    ap.add_argument("--workload", default="bf16_n8192_d128_causal")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's B")
    ap.add_argument("--heads", type=int, default=None, help="override the workload's H (e.g. one GPU's share of heads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["fwdbwd", "fwd", "copy"], default="fwdbwd",
                    help="fwd: time the forward kernel alone (for profiling); copy: a plain 1 GiB device copy "
                         "(calibrates the HBM byte counters)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the oracle sample")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="after the timed steps, repeat the step this long while sampling the GPU clock (0: skip)")
    ap.add_argument("--dropout", type=float, default=None, help="time the dropout entry points at this rate")
    ap.add_argument("--fp8", action="store_true", help="time attn_fwd_fp8 (e4m3 inputs) on the workload's shape")
    ap.add_argument("--probe", action="store_true",
                    help="run the hardware probes of include/attn_probe.h (LDS, issue rates, wave placement, "
                         "atomics, exp2 accuracy) and print their rates")
    ap.add_argument("--decode", type=int, default=None, help="time attn_decode with this many queries per head")
    ap.add_argument("--decode-nk", type=int, default=16384, help="cached keys per head for --decode")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: capture the K timed calls in one HIP graph and time its replay")
    ap.add_argument("--flush-l2", action="store_true",
                    help="write a 512 MiB scratch buffer before every step, so no input is left in L2 or the MALL")
    ap.add_argument("--block-density", type=float, default=None,
                    help="time attn_fwd_block_sparse + attn_bwd_block_sparse on a random block mask of this density")
    return ap.parse_args()


def kernel_flops(w: W.Workload):
    """Algorithmic FLOPs each launch performs, by kernel.

    A forward contraction over the allowed (query, key) pairs costs
    2*B*H*N^2*d (halved when causal); the forward has two, the backward five
    (the recomputed Q K^T, dO V^T, P^T dO, dS^T Q and dS K).  dkdv executes four
    of the five; dq executes dS K (its recomputed Q K^T and dO V^T are not
    counted); the preprocess stage (folded into dq by attn_bwd) is memory
    traffic only.
    """
    one = w.fwd_flops() / 2
    return {"fwd": 2 * one, "dkdv": 4 * one, "dq": 1 * one, "preprocess": 0.0}


def timed_oracle(run_head, per_head: float, unit: str, budget_s: float, what: str):
    """Call run_head() (one head of the oracle) until about budget_s has passed.

    per_head is the head's share of the metric's numerator (FLOPs or bytes),
    so the rate is in the same unit as the GPU line.  cores = the BLAS
    threads numpy uses.
    """
    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    heads = 0
    t0 = time.perf_counter()
    while True:
        run_head()
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    div = 1e12 if unit == "TFLOP/s" else 1e9
    return {"value": per_head * heads / dt / div, "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} head(s): {what}, {dt:.1f} s; the rate counts the same algorithmic work as value",
            "cores_note": "BLAS threads the oracle's numpy matrix products used", **host_facts()}


def cpu_baseline(w: W.Workload, budget_s: float, fwd_only: bool = False):
    """Time the fp64 oracle head by head for about budget_s: forward + backward,
    or the forward alone when the GPU line times the forward alone."""
    import numpy as np
    from oracle import attention as orc

    inp = W.draw(1, 1, w.N, w.d, w.dtype, seed=w.seed + 77)
    q, k, v, do = (inp[x][0, 0].float().numpy().astype(np.float64) for x in ("q", "k", "v", "do"))

    def head():
        orc.forward_head(q, k, v, w.scale, w.causal)
        if not fwd_only:
            orc.backward_head(q, k, v, do, w.scale, w.causal)

    flops = w.fwd_flops() + (0.0 if fwd_only else w.bwd_flops())
    what = "forward" if fwd_only else "forward + backward"
    return timed_oracle(head, flops / (w.B * w.H), "TFLOP/s", budget_s,
                        f"the workload (N={w.N}, d={w.d}, causal={w.causal}), {what} in fp64 with S "
                        "and P materialised")


def host_facts():
    """The host the oracle ran on: CPU model, logical CPUs and the affinity set."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


class ClockSampler:
    """Samples the GPU's graphics clock (amdsmi GPU metrics: the per-XCD current
    gfx clocks, else the current or average gfx clock, in MHz) from a thread
    every `period` seconds while active.  The GPU is matched to torch's device
    0 by PCI bus.  mean() is None, with `error` set, when the metrics cannot be
    read on this host."""

    def __init__(self, period: float = 0.002):
        import threading

        self.period, self.samples, self.error = period, [], None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi

            self._smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                if bus is None or int(bdf.split(":")[1], 16) == int(bus):
                    self._handle = h
                    break
            if self._handle is None:
                self.error = f"no amdsmi device on PCI bus {bus}"
        except Exception as e:  # pragma: no cover - depends on the host
            self.error = f"amdsmi unavailable: {type(e).__name__}: {e}"

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        vals = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 65535]
        if vals:
            return sum(vals) / len(vals)
        for key in ("current_gfxclk", "average_gfxclk_frequency"):
            x = m.get(key)
            if isinstance(x, (int, float)) and 0 < x < 65535:
                return float(x)
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                x = self._read()
                if x is not None:
                    self.samples.append(x)
            except Exception as e:  # pragma: no cover
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading

        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def settled(self):
        """The samples of the second half of the window: the metrics table the
        samples come from refreshes only every few hundred ms, so the first
        samples of a window can still show the idle clock."""
        return self.samples[len(self.samples) // 2:]

    def mean(self):
        s = self.settled()
        return sum(s) / len(s) if s else None

    def median(self):
        """Median of the settled samples: one stray idle reading (the metrics
        table can report one between steps) moves it far less than the mean."""
        s = sorted(self.settled())
        return s[len(s) // 2] if s else None

    def report(self, window_s: float):
        m, s = self.mean(), self.settled()
        md = self.median()
        return {"gpu_clock_mhz_avg": round(m, 1) if m is not None else None,
                "gpu_clock_mhz_median": round(md, 1) if md is not None else None,
                "gpu_clock_mhz_min_max": [round(min(s), 1), round(max(s), 1)] if s else None,
                "gpu_clock_samples": len(s),
                "gpu_clock_source": "amdsmi gpu metrics, mean over XCDs of the current gfx clock, sampled every "
                                    f"{self.period * 1e3:.0f} ms while the same step repeats for {window_s:.1f} s "
                                    "after the timed steps (second half of the window)"
                                    + (f"; {self.error}" if self.error else "")}


def measure_clock(step, seconds: float):
    """Repeat step() for `seconds` (outside any timed region) while sampling the clock."""
    clock = ClockSampler(period=0.02)
    torch.cuda.synchronize()
    with clock:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            step()
            torch.cuda.synchronize()
    return clock


COPY_BYTES = 1 << 30
FLUSH_BYTES = 512 << 20


def copy_calibration(args):
    """A plain device-to-device copy of exactly 1 GiB (read 1 GiB, write 1 GiB).

    Profiled with the FETCH_SIZE / WRITE_SIZE counters, it gives the factor
    between what those counters report and the bytes actually moved.
    """
    dev = torch.device("cuda", 0)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(args.warmup, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"metric": "device copy GB/s (counter calibration)", "value": round(2 * COPY_BYTES / dt / 1e9, 1),
                      "unit": "GB/s", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "steps": args.steps}),
          flush=True)
    return 0


def bench_probe(args):
    """The hardware probes of include/attn_probe.h; prints one JSON line with
    the rates the design quotes (each probe's kernel is described in that
    header)."""
    import numpy as np

    from exact_io_aware_23_amd import binding

    lib = binding.load_library()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    P = lambda t: t.data_ptr()

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {"metric": "hardware probes (include/attn_probe.h)", "cus": cus}
    # LDS read throughput: per CU (from each workgroup's own cycle count, the
    # workgroups of a CU running together) and over the whole chip (events)
    lds = {}
    for mode, name, nbytes in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16", 8)):
        for per_cu in (1, 2, 4):
            wgs = cus * per_cu
            sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
            cyc = torch.empty(wgs, dtype=torch.int64, device=dev)

            def run():
                assert lib.attn_probe_lds_rate(mode, wgs, P(sink), P(cyc), st) == 0

            ms = timed(run)
            per_wg = 256 * 2048 * 8 * nbytes
            mean_cyc = float(cyc.double().mean())
            lds[f"{name} x{per_cu}/CU"] = {"bytes_per_clk_per_cu": round(per_wg * per_cu / mean_cyc, 1),
                                           "tb_per_s": round(per_wg * wgs / (ms * 1e-3) / 1e12, 1)}
    out["lds_read"] = lds
    # issue rates: cycles per instruction of each wave; waves w and w+4 share a SIMD
    cases = [("exp, one wave per SIMD", [1] * 4), ("fma, one wave per SIMD", [2] * 4), ("mfma, one wave per SIMD", [3] * 4),
             ("exp + exp", [1] * 8), ("mfma + exp", [3] * 4 + [1] * 4), ("mfma + fma", [3] * 4 + [2] * 4),
             ("exp + fma", [1] * 4 + [2] * 4)]
    issue = {}
    for name, kinds in cases:
        k = torch.tensor(kinds, dtype=torch.int32, device=dev)
        nw = len(kinds)
        sink = torch.empty(cus * 64 * nw, dtype=torch.float32, device=dev)
        cyc = torch.zeros(cus * 8, dtype=torch.int64, device=dev)
        assert lib.attn_probe_issue(P(k), nw, cus, P(sink), P(cyc), st) == 0
        torch.cuda.synchronize()
        assert lib.attn_probe_issue(P(k), nw, cus, P(sink), P(cyc), st) == 0
        torch.cuda.synchronize()
        c = cyc.view(cus, 8)[:, :nw].double().mean(0).tolist()
        names = {1: "exp", 2: "fma", 3: "mfma"}
        per = {}
        for grp, lo in (("waves 0-3", 0), ("waves 4-7", 4)):
            if lo >= nw:
                continue
            kind = kinds[lo]
            n_inst = 4096 if kind == 3 else 8 * 4096
            per[f"{grp} ({names[kind]})"] = round(sum(c[lo:lo + 4]) / 4 / n_inst, 2)
        issue[name] = per
    out["issue_cycles_per_instruction"] = issue
    # wave placement of 8-wave workgroups
    hw = torch.empty(512 * 8, dtype=torch.int32, device=dev)
    assert lib.attn_probe_wave_simd(512, P(hw), st) == 0
    torch.cuda.synchronize()
    h = hw.view(512, 8).cpu().to(torch.int64)
    simd, cu = (h >> 4) & 3, (h >> 8) & 0xF
    same = ((simd[:, :4] == simd[:, 4:]) & (cu[:, :4] == cu[:, 4:])).double().mean().item()
    out["waves_w_and_w+4_share_a_simd"] = round(same, 4)
    # global fp32 updates: atomics against a plain load-add-store, 4 bytes per element
    atom = {}
    for mib in (4, 64, 256):
        n = mib * (1 << 20) // 4
        t = torch.zeros(n, dtype=torch.float32, device=dev)
        for mode, name in ((1, "atomic_add_f32"), (0, "load_add_store")):
            ms = timed(lambda: lib.attn_probe_atomic(P(t), n, mode, st))
            atom[f"{name} {mib} MiB"] = round(n * 4 / (ms * 1e-3) / 1e9, 1)
    out["global_update_gb_per_s"] = atom
    # v_exp_f32 against exact exp2 (fp64), in float32 ulps of the exact value
    x = torch.linspace(-39.5, 0.5, 1 << 22, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    assert lib.attn_probe_exp2(P(x), P(y), x.numel(), st) == 0
    torch.cuda.synchronize()
    xs, ys = x.cpu().double().numpy(), y.cpu().double().numpy()
    ref = np.exp2(xs)
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    out["v_exp_f32_max_ulp_on_-39.5_0.5"] = round(float(np.max(np.abs(ys - ref) / ulp)), 3)
    # HBM read rate: a 4 GiB buffer (twice the L2s and the last-level cache many
    # times over) read once per launch, over grid sizes and loads in flight
    src = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    src.view(torch.int32).fill_(0x01020304)
    rd = {}
    for per_cu in (4, 8, 16, 32):
        wgs = cus * per_cu
        sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        for unroll in (1, 2, 4, 8):
            ms = timed(lambda: lib.attn_probe_read_rate(P(src), src.numel(), unroll, wgs, P(sink), st), reps=5)
            rd[f"{per_cu} workgroups/CU, {unroll} loads in flight"] = round(src.numel() / (ms * 1e-3) / 1e9, 1)
    out["hbm_read_gb_per_s"] = rd
    out["hbm_read_best_gb_per_s"] = max(rd.values())
    del src
    out["host"] = host_facts()
    print(json.dumps(out), flush=True)
    return 0


def kernel_source_hash(kernel: str) -> str:
    """sha256 of the HIP source file that holds `kernel` (its code plus the shared header)."""
    import hashlib

    src = {"fwd": "attn_fwd.hip", "preprocess": "attn_bwd.hip", "dq": "attn_bwd.hip", "dkdv": "attn_bwd.hip",
           "fwd_fp8": "attn_fwd_fp8.hip", "decode_partial": "attn_decode.hip", "decode_merge": "attn_decode.hip"}[kernel]
    h = hashlib.sha256()
    for f in (src, "attn_common.h"):
        with open(os.path.join(ROOT, "exact_io_aware_23_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None.

    profiles/traffic_<workload>.json holds FETCH_SIZE and WRITE_SIZE per launch
    (already scaled by the copy calibration) with the source hash they were
    taken at; a changed kernel source makes the figure stale, so None.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    return k["hbm_bytes_per_launch"]


def allowed_pairs_per_head(mask: torch.Tensor, N: int, causal: bool) -> torch.Tensor:
    """Allowed (query, key) pairs of each head under a [heads, nb, nb] block mask (and the causal mask)."""
    nb = mask.shape[-1]
    start = torch.arange(nb, dtype=torch.int64) * 128
    size = torch.clamp(N - start, max=128)  # rows (or keys) in each block
    pairs = size[:, None] * size[None, :]
    if causal:
        # keys j <= i: blocks left of the diagonal count fully, the diagonal one triangularly
        r, c = torch.meshgrid(torch.arange(nb), torch.arange(nb), indexing="ij")
        tri = size * (size + 1) // 2
        pairs = torch.where(c < r, pairs, torch.where(c == r, torch.diag(tri), torch.zeros_like(pairs)))
    return (mask.to(torch.int64).cpu() * pairs).sum(dim=(1, 2))


def bench_decode(args):
    """Decode against a KV cache; prints one JSON line with the HBM roofline."""
    import exact_io_aware_23_amd as A

    B, H, Nq, Nk, d = args.batch or 4, args.heads or 32, args.decode, args.decode_nk, 128
    dev = torch.device("cuda", 0)
    cache = W.draw(B, H, Nk, d, "bf16", seed=6000, backward=False)
    q = W.draw(B, H, Nq, d, "bf16", seed=6001, backward=False)["q"].to(dev)
    k, v = cache["k"].to(dev), cache["v"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(A.decode_workspace_bytes(B, H, Nq, Nk, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    scale = 1 / (d ** 0.5)

    def step():
        A.decode(q, k, v, scale=scale, causal=True, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    graph = None
    if args.graph:
        # the K calls are captured back to back in one graph (attn_decode only enqueues kernels), so the
        # timed replay shows the GPU's time per call without the host's launch cost of each call
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        graph.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    t_gpu = ev[0].elapsed_time(ev[1]) / args.steps
    # algorithmic bytes: K and V once, q in, O and L out
    bytes_ = 2.0 * B * H * Nk * d * 2 + 2.0 * B * H * Nq * d * 2 + 4.0 * B * H * Nq
    gbs = bytes_ / (t_gpu * 1e-3) / 1e9
    # HBM bytes of one call (partial + merge kernel), from the committed counter summary of this shape
    wl = f"decode_b{B}_h{H}_nq{Nq}_nk{Nk}_d{d}"
    parts = [measured_traffic(kern, wl) for kern in ("decode_partial", "decode_merge")]
    traffic = None if None in parts else sum(parts)
    out = {
        "metric": "decode attention GB/s against a KV cache (HBM roofline)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode", "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "causal": True,
                   "graph": bool(args.graph)},
        "gpu_ms_per_call": round(t_gpu, 4),
        "tflops": round(4.0 * d * Nq * Nk * B * H / (t_gpu * 1e-3) / 1e12, 3),
        "roofline": {"kernel": "decode (partial + merge)", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": int(bytes_), "avg_launch_ms": round(t_gpu, 4)},
    }
    if not args.no_cpu_baseline:
        from oracle import decode as dec

        qh, kh, vh = (t[0, 0].double().numpy() for t in (W.draw(B, H, Nq, d, "bf16", seed=6001, backward=False)["q"],
                                                         cache["k"], cache["v"]))
        out["cpu_baseline"] = timed_oracle(lambda: dec.decode_head(qh, kh, vh, scale, True), bytes_ / (B * H), "GB/s",
                                           args.cpu_seconds, f"decode of head (0, 0), Nq={Nq} Nk={Nk} d={d}, fp64")
    print(json.dumps(out), flush=True)
    return 0


def bench_dropout(args, w):
    """Forward + backward with dropout on P; prints one JSON line."""
    import exact_io_aware_23_amd as A

    dev = torch.device("cuda", 0)
    inp = W.draw_workload(w, B=w.B, H=w.H)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    seed = 0x5EED1234ABCD
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(A.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        A.fwd_dropout(q, k, v, args.dropout, seed, scale=w.scale, causal=w.causal, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        A.bwd_dropout(q, k, v, o, lse, do, args.dropout, seed, scale=w.scale, causal=w.causal, workspace=ws, dq=dq,
                      dk=dk, dv=dv)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    t_fwd = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    t_bwd = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    F_fwd, F_bwd = w.fwd_flops(), w.bwd_flops()
    achieved = F_fwd / (t_fwd * 1e-3) / 1e12
    out = {
        "metric": "attention with dropout TFLOP/s fwd and fwd+bwd",
        "value": round((F_fwd + F_bwd) / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal, "pass": "fwd+bwd",
                   "dropout": args.dropout, "seed": seed},
        "fwd_tflops": round(achieved, 2),
        "bwd_tflops": round(F_bwd / (t_bwd * 1e-3) / 1e12, 2),
        "kernel_ms": {"fwd": round(t_fwd, 4), "bwd (dq+dkdv)": round(t_bwd, 4)},
        "roofline": {"kernel": "fwd", "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": round(t_fwd, 4)},
    }
    if not args.no_cpu_baseline:
        from oracle import dropout as drp

        qh, kh, vh, doh = (inp[x][0, 0].double().numpy() for x in ("q", "k", "v", "do"))
        t = drp.threshold(args.dropout)

        def head():
            drp.forward_head_dropout(qh, kh, vh, w.scale, w.causal, seed, t, 0)
            drp.backward_head_dropout(qh, kh, vh, doh, w.scale, w.causal, seed, t, 0)

        out["cpu_baseline"] = timed_oracle(head, (F_fwd + F_bwd) / (B * H), "TFLOP/s", args.cpu_seconds,
                                           f"head (0, 0), N={N} d={d}, forward + backward with dropout {args.dropout} "
                                           "in fp64 (Philox decisions regenerated in numpy)")
    print(json.dumps(out), flush=True)
    return 0


def bench_block_sparse(args, w):
    """Forward + backward of block-sparse attention; prints one JSON line."""
    import exact_io_aware_23_amd as A

    dev = torch.device("cuda", 0)
    inp = W.draw_workload(w, B=w.B, H=w.H)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    nb = (N + 127) // 128
    g = torch.Generator().manual_seed(1234)
    mask = (torch.rand((B * H, nb, nb), generator=g) < args.block_density).to(torch.uint8)
    mask[:, torch.arange(nb), torch.arange(nb)] = 1
    pairs = int(allowed_pairs_per_head(mask, N, w.causal).sum())
    F_fwd = 4.0 * d * pairs
    F_bwd = 2.5 * F_fwd
    m = mask.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(A.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        A.fwd_block_sparse(q, k, v, m, scale=w.scale, causal=w.causal, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        A.bwd_block_sparse(q, k, v, o, lse, do, m, scale=w.scale, causal=w.causal, workspace=ws, dq=dq, dk=dk,
                           dv=dv)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    t_fwd = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    t_bwd = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    achieved = F_fwd / (t_fwd * 1e-3) / 1e12
    density = pairs / (B * H * (N * (N + 1) / 2 if w.causal else N * N))
    out = {
        "metric": "block-sparse attention TFLOP/s fwd and fwd+bwd (allowed pairs only)",
        "value": round((F_fwd + F_bwd) / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal, "pass": "fwd+bwd",
                   "block_density": args.block_density, "allowed_fraction": round(density, 4),
                   "mask": "random 128x128 blocks, torch seed 1234, diagonal blocks on"},
        "fwd_tflops": round(achieved, 2),
        "bwd_tflops": round(F_bwd / (t_bwd * 1e-3) / 1e12, 2),
        "kernel_ms": {"fwd": round(t_fwd, 4), "bwd (dq+dkdv)": round(t_bwd, 4)},
        "roofline": {"kernel": "fwd", "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": round(t_fwd, 4)},
    }
    if not args.no_cpu_baseline:
        from oracle import attention as orc

        qh, kh, vh, doh = (inp[x][0, 0].double().numpy() for x in ("q", "k", "v", "do"))
        mh = mask[0].numpy()
        pairs0 = int(allowed_pairs_per_head(mask[:1], N, w.causal).sum())

        def head():
            orc.forward_head(qh, kh, vh, w.scale, w.causal, block_mask=mh)
            orc.backward_head(qh, kh, vh, doh, w.scale, w.causal, block_mask=mh)

        out["cpu_baseline"] = timed_oracle(head, 3.5 * 4.0 * d * pairs0, "TFLOP/s", args.cpu_seconds,
                                           f"head (0, 0) with its block mask, N={N} d={d}, forward + backward in fp64 "
                                           "(dense S and P, masked entries -inf)")
    print(json.dumps(out), flush=True)
    return 0


def bench_fp8(args, w):
    """The FP8 forward (e4m3 Q, K, V with per-tensor scales, bf16 O) on the
    workload's shape, with the bf16 forward on the same shape timed beside it;
    prints one JSON line."""
    import exact_io_aware_23_amd as A

    dev = torch.device("cuda", 0)
    B, H, N, d = w.B, w.H, w.N, w.d
    inp = W.draw_fp8(B, H, N, d, seed=w.seed)
    q8, k8, v8 = (inp[x].to(dev) for x in ("q8", "k8", "v8"))
    ref = W.draw(B, H, N, d, "bf16", seed=w.seed, backward=False)
    qb, kb, vb = (ref[x].to(dev) for x in ("q", "k", "v"))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    warm = max(args.warmup, 50)  # one launch is under a millisecond: give the clocks ~40 ms to settle

    def timed(fn):
        for _ in range(warm):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        return wall_ms, sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps

    ms_step, t_fp8 = timed(lambda: A.fwd_fp8(q8, k8, v8, inp["dq"], inp["dk"], inp["dv"], scale=w.scale,
                                               causal=w.causal, out=o, lse=lse))
    _, t_bf16 = timed(lambda: A.fwd(qb, kb, vb, scale=w.scale, causal=w.causal, out=o, lse=lse))
    F = w.fwd_flops()
    achieved = F / (t_fp8 * 1e-3) / 1e12
    out = {
        "metric": "attention forward TFLOP/s, fp8 e4m3 inputs",
        "value": round(F / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name + "_fp8", "B": B, "H": H, "N": N, "d": d, "causal": w.causal, "pass": "fwd",
                   "warmup_launches": warm},
        "fwd_tflops": round(achieved, 2),
        "bf16_fwd_tflops_same_shape": round(F / (t_bf16 * 1e-3) / 1e12, 2),
        "kernel_ms": {"fwd_fp8": round(t_fp8, 4), "fwd_bf16": round(t_bf16, 4)},
        "roofline": {"kernel": "fwd_fp8", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("fwd_fp8", w.name + "_fp8") if (B, H) == (2, 32) else None,
                     "avg_launch_ms": round(t_fp8, 4)},
    }
    if not args.no_cpu_baseline:
        from oracle import fp8 as orc8

        qh, kh, vh = (inp[x][0, 0].numpy() for x in ("q8", "k8", "v8"))
        out["cpu_baseline"] = timed_oracle(
            lambda: orc8.forward_head_fp8(qh, kh, vh, inp["dq"], inp["dk"], inp["dv"], w.scale, w.causal),
            F / (B * H), "TFLOP/s", args.cpu_seconds,
            f"head (0, 0), N={N} d={d}, e4m3 codes dequantized to fp64, forward with S and P materialised")
    print(json.dumps(out), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(every (batch, head) pair is independent, so N GPUs would each run B*H/N heads).", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.which == "copy":
        return copy_calibration(args)
    if args.probe:
        return bench_probe(args)
    import exact_io_aware_23_amd as A

    A.load_library()
    import dataclasses

    w = W.BY_NAME[args.workload]
    w = dataclasses.replace(w, B=args.batch or w.B, H=args.heads or w.H)
    if args.block_density is not None:
        return bench_block_sparse(args, w)
    if args.dropout is not None:
        return bench_dropout(args, w)
    if args.decode is not None:
        return bench_decode(args)
    if args.fp8:
        return bench_fp8(args, w)
    fwd_only = args.which == "fwd" or not w.backward
    dev = torch.device("cuda", 0)
    inp = W.draw_workload(w, B=w.B, H=w.H)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta_exact = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = ["fwd", "dq", "dkdv"]  # the launches attn_bwd makes: the dq stage forms delta~ itself
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if args.flush_l2 else None

    def step(ev=None):
        if scratch is not None:
            scratch.fill_(1.0)  # outside the timed kernels: evicts the inputs from L2 and the MALL
        if ev is not None:
            ev[0].record(stream)
        A.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        if fwd_only:
            if ev is not None:
                for e in ev[2:]:
                    e.record(stream)
            return
        A.bwd_dq_fused(q, k, v, o, lse, do, scale=w.scale, causal=w.causal, dq=dq, delta_out=delta_exact)
        if ev is not None:
            ev[2].record(stream)
        A.bwd_dkdv(q, k, v, lse, do, delta_exact, scale=w.scale, causal=w.causal, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = measure_clock(step, args.clock_seconds) if args.clock_seconds > 0 else None

    samples = {n: [ev[j].elapsed_time(ev[j + 1]) for ev in events] for j, n in enumerate(names)}
    per_kernel = {n: sum(t) / args.steps for n, t in samples.items()}  # ms per launch
    gpu_ms = events[0][0].elapsed_time(events[-1][len(names)]) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    if scratch is not None:  # the flush writes sit between the steps: time the kernels only
        ms_per_step = sum(per_kernel.values())

    F_fwd, F_bwd = w.fwd_flops(), w.bwd_flops()
    if fwd_only:
        F_bwd = 0.0
    value = (F_fwd + F_bwd) / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = F_fwd / (per_kernel["fwd"] * 1e-3) / 1e12
    bwd_ms = per_kernel["dq"] + per_kernel["dkdv"]
    bwd_tflops = F_bwd / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 and F_bwd > 0 else None

    kf = kernel_flops(w)
    dominant = "fwd" if fwd_only else max(names, key=lambda n: per_kernel[n])
    t_dom = per_kernel[dominant] * 1e-3
    balance = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # FLOP per byte
    if w.dtype == "f32":
        bound, achieved, peak, unit = "alu", kf["fwd"] / t_dom / 1e12, FP32_VECTOR_PEAK_TFLOPS, "TFLOP/s"
    elif dominant == "fwd" and w.fwd_flops() / w.fwd_bytes() < balance:
        bound, achieved, peak, unit = "hbm", w.fwd_bytes() / t_dom / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", kf[dominant] / t_dom / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = measured_traffic(dominant, w.name) if (w.B, w.H) == (W.BY_NAME[w.name].B, W.BY_NAME[w.name].H) else None
    roof = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
            "avg_launch_ms": round(per_kernel[dominant], 4)}

    out = {
        "metric": "attention TFLOP/s fwd and fwd+bwd (bf16, N=8192 d=128 causal) + % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "pass": "fwd" if fwd_only else "fwd+bwd", **({"flush_l2_bytes": FLUSH_BYTES} if args.flush_l2 else {})},
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_frac_mfma_peak": round(fwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "bwd_tflops": round(bwd_tflops, 2) if bwd_tflops else None,
        "fwdbwd_frac_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "kernel_ms": {n: round(t, 4) for n, t in per_kernel.items()},
        "kernel_ms_median": {n: round(sorted(t)[len(t) // 2], 4) for n, t in samples.items()},
        "kernel_ms_min": {n: round(min(t), 4) for n, t in samples.items()},
        "roofline": roof,
        "host": {**host_facts(), **(clock.report(args.clock_seconds) if clock else {})},
    }
    if clock is not None and clock.mean() is not None:
        # the MFMA peak at the clock the kernels actually ran at, for context
        out["mfma_peak_at_measured_clock_tflops"] = round(MFMA_BF16_PEAK_TFLOPS * clock.median() / 2400.0, 1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, fwd_only)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
