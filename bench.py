"""Benchmark of the performer step on one MI355X.

One step = one performer_unit at the v0.2 unit shapes: kv_append of a
3712-token K/V slice (40 heads x 128, bf16) after 32 units of history
(118,784 tokens, 256-token pages, shuffled physical pages), then 4 x
(block_causal_attn over all 122,496 keys + fm_euler_step with the 5120x16
projection).  The cache is rolled back to the history length before every
step (host field only), so every step does the same work.

Prints one JSON line.  value = attention FLOPs of the unit (4 calls x
4*H*D*Lq*Nk) / wall time of the whole unit (append and Euler included).
roofline = the attention kernel alone, timed with HIP events recorded on the
launch stream around every attention call of the timed steps.
cpu_baseline = the float64 CPU oracle on a bounded sample of the same
attention (rank 0 only).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-causal attn TFLOP/s (% MFMA peak) + ms/160ms-unit at v0.2 shapes"
METRIC_WORKLOAD = "v02_unit"  # the workload METRIC names; other workloads get their own label
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
UNIT_BUDGET_MS = 160.0
# sources of the bf16 attention kernel the bench times (direct-load kernel)
ATTN_KERNEL_SRCS = [os.path.join(ROOT, "block_causal_attention_performer_amd", "csrc", f)
                    for f in ("attn_dma.hip", "attn_common.h")]
ATTN_KERNEL_NAME = "attn_dma_kernel<128, false>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_v02_unit_traffic.txt")   # v02_unit launches


class Hip:
    """hipEvent_* through the HIP runtime (events on the launch stream)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.L.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.L.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value


def _kernel_hash() -> str:
    h = hashlib.sha256()
    for f in ATTN_KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per attention launch from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != _kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model():
    """Host CPU as lscpu names it (model, sockets, cores per socket)."""
    info = {}
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            info[k.strip()] = v.strip()
    except Exception:  # pragma: no cover
        pass
    return {"model": info.get("Model name"), "sockets": info.get("Socket(s)"),
            "cores_per_socket": info.get("Core(s) per socket"),
            "threads_per_core": info.get("Thread(s) per core"), "logical_cpus": info.get("CPU(s)")}


def _oracle_attention_sample(inp, w, rows_n, heads_n):
    """Seconds and FLOPs of the float64 oracle on rows_n query rows x heads_n
    heads of the workload's unit over its whole key range (every key is
    visible to the unit's queries)."""
    import numpy as np
    import oracle
    H = w.n_heads
    rows = np.linspace(0, w.unit_tokens - 1, rows_n).astype(np.int64)
    heads = np.arange(0, H, max(1, H // heads_n))[:heads_n]
    hsel = torch.as_tensor(heads, device=inp["q"].device)
    q = inp["q"][:, hsel].float().cpu().numpy().astype(np.float64)
    k = torch.cat([inp["k_hist"][:, hsel], inp["k_new"][:, hsel]]).float().cpu().numpy().astype(np.float64)
    v = torch.cat([inp["v_hist"][:, hsel], inp["v_new"][:, hsel]]).float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oracle.attention_dense(q, k, v, rows=rows)
    dt = time.perf_counter() - t0
    return dt, 4.0 * w.head_dim * len(rows) * len(heads) * w.n_kv, len(rows), len(heads)


def cpu_baseline(inp, w, rows_n, heads_n, workloads):
    """The float64 oracle (numpy, as it stands) timed on the host: the
    workload's attention on rows_n query rows x heads_n heads with every
    BLAS thread (the reported value), the same on a 32-row sample with one
    thread, and an all-thread sample of the v0.1 unit's attention; each as
    TFLOP/s of the same FLOP count as the GPU figure, plus the unit's four
    attention calls (and those of the long fp8 history's unit) extrapolated
    at the all-thread rate."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    dt, fl, nr, nh = _oracle_attention_sample(inp, w, rows_n, heads_n)
    with threadpool_limits(limits=1):
        dt1, fl1, nr1, nh1 = _oracle_attention_sample(inp, w, 32, heads_n)
    w1 = workloads.WORKLOADS["v01_unit"]
    inp1 = workloads.make_unit_inputs(w1, device=inp["q"].device)
    dtc, flc, nrc, nhc = _oracle_attention_sample(inp1, w1, 256, w1.n_heads)
    del inp1
    rate = fl / dt
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"attention_dense (float64 numpy) of {nr} query rows x {nh} heads over all "
                      f"{w.n_kv} keys of the {w.name} workload's unit; {dt:.2f} s",
            "seconds": dt,
            "cpu": _cpu_model(),
            "one_thread": {"value": fl1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": dt1,
                           "sample": f"{nr1} query rows x {nh1} heads, same keys"},
            "v01_unit": {"value": flc / dtc / 1e12, "unit": "TFLOP/s", "cores": int(cores),
                         "seconds": dtc,
                         "sample": f"{nrc} query rows x {nhc} heads over all {w1.n_kv} keys of the "
                                   f"v01_unit workload's unit"},
            "unit_attention_s_extrapolated": w.n_steps * w.attn_flops() / rate,
            "long_fp8_unit_attention_s_extrapolated": {
                "value": w.n_steps * workloads.WORKLOADS["v02_long_fp8"].attn_flops() / rate,
                "basis": "the four attention calls of the long fp8 unit (2,787,712 keys) at the "
                         "all-thread rate above: the oracle's dense attention does the same work "
                         "per key whatever the cache dtype; decoding the E4M3 pages is not included"}}


class ClockSampler:
    """Samples the GPU's GFX clock every 10 ms from a background thread while
    the timed steps run, from two amdsmi sources: the GPU metrics table
    (current_gfxclk per XCC, averaged over the XCCs) and the clock query
    (amdsmi_get_clock_info, GFX domain).  Both are the firmware's
    instantaneous readings, so the report gives medians and the 10th/90th
    percentiles rather than means.  Fields are None when amdsmi is
    unavailable."""

    def __init__(self):
        import threading
        self.metrics, self.clk = [], []
        self._stop = threading.Event()
        self._t = None
        self.device_bdf = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            # amdsmi lists every GPU of the host; take the one this process
            # runs on (device 0), matched by its PCI domain and bus
            p = torch.cuda.get_device_properties(0)
            self._h = None
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
                dom, bus = bdf.split(":")[0], bdf.split(":")[1]
                if int(dom, 16) == p.pci_domain_id and int(bus, 16) == p.pci_bus_id:
                    self._h, self.device_bdf = h, bdf
                    break
            self._smi = amdsmi if self._h is not None else None
        except Exception:
            self._smi = None

    @staticmethod
    def _ok(x):
        return isinstance(x, (int, float)) and 0 < x < 10000

    def _run(self):
        smi = self._smi
        while not self._stop.is_set():
            try:
                m = smi.amdsmi_get_gpu_metrics_info(self._h)
                cur = m.get("current_gfxclks")
                vals = [c for c in cur if self._ok(c)] if isinstance(cur, list) else []
                if not vals and self._ok(m.get("current_gfxclk")):
                    vals = [m["current_gfxclk"]]
                if vals:
                    self.metrics.append(sum(vals) / len(vals))
            except Exception:
                pass
            try:
                c = smi.amdsmi_get_clock_info(self._h, smi.AmdSmiClkType.GFX).get("clk")
                if self._ok(c):
                    self.clk.append(c)
            except Exception:
                pass
            self._stop.wait(0.01)

    def __enter__(self):
        if self._smi is not None:
            import threading
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t is not None:
            self._t.join()

    @staticmethod
    def _stats(v):
        # the first reading is taken as the thread starts, before the timed
        # kernels have raised the clock: it is dropped; a handful of readings
        # (a timed region of under 0.1 s) is flagged as not representative
        v = sorted(v[1:])
        if not v:
            return {"samples": 0, "median_mhz": None, "p10_mhz": None, "p90_mhz": None,
                    "representative": False}
        q = lambda f: v[min(len(v) - 1, int(f * len(v)))]
        return {"samples": len(v), "median_mhz": round(q(0.5), 1), "p10_mhz": round(q(0.1), 1),
                "p90_mhz": round(q(0.9), 1), "representative": len(v) >= 10}

    def report(self, achieved_tflops=None):
        """achieved_tflops: the main kernel's rate.  One wave per SIMD issues
        a 32x32x16 bf16 MFMA at most every 32 shader cycles, so that rate
        needs a clock of at least achieved / 2500 * 2400 MHz; a median below
        it cannot be the clock the kernel ran at (some hosts' firmware
        tables report a stale or idle value), and `plausible` says so."""
        out = {"source": "amdsmi during the timed steps, every 10 ms (firmware instantaneous readings)",
               "device_bdf": self.device_bdf,
               "gpu_metrics_current_gfxclk": self._stats(self.metrics),
               "clock_info_gfx": self._stats(self.clk)}
        if achieved_tflops is not None:
            need = achieved_tflops / PEAK_BF16_TFLOPS * 2400.0
            out["min_clock_mhz_for_rate"] = round(need, 1)
            for key in ("gpu_metrics_current_gfxclk", "clock_info_gfx"):
                med = out[key]["median_mhz"]
                out[key]["plausible"] = med is not None and med >= 0.97 * need
        return out


def catchup(args, w, inp, cache, hip, stream, bca, workloads):
    """Multi-block catch-up call: queries = the last N units of the cache
    (history + the unit), block size = one unit, so future key tiles of every
    query tile are skipped and only the diagonal block's tiles are masked.
    Times the whole call (main kernel, split combine, exact rerun check)."""
    bca.kv_append(cache, inp["k_new"], inp["v_new"])
    q_pos0, n_q, flops = workloads.catchup_span(w, args.catchup_units)
    H, D = w.n_heads, w.head_dim
    q = workloads.qkv(workloads.seed_for(w.index, "q_catchup"), n_q, H, D, w.qkv_scale, "bf16", "cuda")
    ws = bca.alloc_workspace(bca.workspace_bytes(cache, n_q, w.n_kv, w.n_ch))
    out = torch.empty((n_q, H, D), dtype=torch.bfloat16, device="cuda")

    def call():
        bca.block_causal_attn(q, cache, n_kv=w.n_kv, q_pos0=q_pos0, block_size=w.unit_tokens,
                              out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(args.steps):
        call()
    hip.record(e1, stream)
    ms = hip.elapsed_ms(e0, e1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "multi-block catch-up attention TFLOP/s (% MFMA peak) at v0.2 shapes",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded device draws, 0.5*N(0,1) Q/K/V rounded to bf16)",
        "config": {"workload": f"{w.name}_catchup{args.catchup_units}", "heads": H, "head_dim": D,
                   "n_q": n_q, "q_pos0": q_pos0, "block_size": w.unit_tokens, "n_kv": w.n_kv,
                   "page_size": w.page_size, "parallelism": "none"},
        "flops_per_call": flops,
        "call_pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2)}), flush=True)


def attn_call(args, w, inp, cache, hip, stream, bca):
    """One streaming block_causal_attn call of the workload's unit (its K/V
    slice appended first), timed as a whole call: main kernel, split combine
    and the exact rerun check.  With the v02_share8 workload this is one
    GPU's share of the v0.2 call under head-sharded context parallelism over
    8 GPUs (5 of the 40 heads); with v02_long_fp8, the call over 750 units
    of fp8 history (the MFMAs stay bf16)."""
    bca.kv_append(cache, inp["k_new"], inp["v_new"])
    H, D = w.n_heads, w.head_dim
    ws = bca.alloc_workspace(bca.workspace_bytes(cache, w.unit_tokens, w.n_kv, w.n_ch))
    out = torch.empty((w.unit_tokens, H, D), dtype=torch.bfloat16, device="cuda")

    def call():
        bca.block_causal_attn(inp["q"], cache, out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(args.steps):
        call()
    hip.record(e1, stream)
    ms = hip.elapsed_ms(e0, e1) / args.steps
    flops = w.attn_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "block-causal attention call TFLOP/s (% MFMA peak)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 S (Q as two e4m3 terms), bf16 PV" if w.dtype == "fp8" else "bf16",
        "data": "synthetic (seeded device draws, 0.5*N(0,1) Q/K/V rounded to bf16)",
        "config": {"workload": f"{w.name}_attn", "heads": H, "head_dim": D, "n_q": w.unit_tokens,
                   "q_pos0": w.n_hist, "block_size": w.unit_tokens, "n_kv": w.n_kv,
                   "page_size": w.page_size, "kv_cache": w.dtype, "parallelism": "none"},
        "flops_per_call": flops,
        "call_pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2)}), flush=True)


def stream_units(args, w, inp, bca, workloads):
    """N consecutive performer units through a streaming session starting
    from the workload's history: each unit's pages come from the free list
    (every other v0.2 unit starts mid-page), eager and as replayed HIP graphs
    (one warm-up unit each, then N timed units, wall clock)."""
    H, D, ps, lq, S = w.n_heads, w.head_dim, w.page_size, w.unit_tokens, w.n_steps
    N = args.stream_units
    n_hist_pages = w.n_hist // ps
    n_log = -(-(w.n_hist + (N + 1) * lq) // ps)
    n_phys = n_log + 8
    gen = torch.Generator().manual_seed(5)
    units = []
    for u in range(N + 1):
        units.append([workloads.qkv(workloads.seed_for(w.index, slot) * 1000 + u + 1, lq, H, D,
                                    w.qkv_scale, "bf16", "cuda") for slot in ("k_new", "v_new", "q")])
    osc = torch.empty((lq, H, D), dtype=torch.bfloat16, device="cuda")
    res = {}
    for mode in ("eager", "graph"):
        perm = torch.randperm(n_phys, generator=gen).to(torch.int32)
        pt = torch.full((n_log,), -1, dtype=torch.int32)
        pt[:n_hist_pages] = perm[:n_hist_pages]
        cache = bca.KVCache(H, D, ps, pt, n_phys, "bf16")
        bca.kv_append(cache, inp["k_hist"], inp["v_hist"])
        ss = bca.Session(cache, perm[n_hist_pages:].tolist())
        ws = bca.alloc_workspace(bca.workspace_bytes(cache, lq, w.n_hist + (N + 1) * lq, w.n_ch))
        z = inp["eps"].clone()
        k, v, q = units[0]
        ss.unit(k, v, q, inp["w"], z, S, osc, workspace=ws, use_graph=mode == "graph")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for u in range(1, N + 1):
            k, v, q = units[u]
            z.copy_(inp["eps"])
            ss.unit(k, v, q, inp["w"], z, S, osc, workspace=ws, use_graph=mode == "graph")
        torch.cuda.synchronize()
        res[mode] = (time.perf_counter() - t0) * 1e3 / N
        assert cache.n_tokens == w.n_hist + (N + 1) * lq
        ss.close()
        del cache, ws
    print(json.dumps({
        "metric": "streaming performer units through a session, ms per unit at v0.2 shapes",
        "value": round(res["graph"], 4), "unit": "ms/unit", "n_gpus": 1, "steps": N,
        "warmup": 1, "ms_per_step": round(res["graph"], 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded device draws, 0.5*N(0,1) Q/K/V rounded to bf16)",
        "config": {"workload": f"{w.name}_stream{N}", "heads": H, "head_dim": D, "unit_tokens": lq,
                   "hist_tokens": w.n_hist, "page_size": ps, "solver_steps": S,
                   "parallelism": "none"},
        "eager_ms_per_unit": round(res["eager"], 4), "graph_ms_per_unit": round(res["graph"], 4),
        "unit_budget_frac": round(res["graph"] / UNIT_BUDGET_MS, 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v02_unit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--cpu-heads", type=int, default=40)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (PMC calibration)")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--catchup-units", type=int, default=0,
                    help="instead of the performer step, time one multi-block catch-up "
                         "block_causal_attn call whose queries are the last N units of the cache")
    ap.add_argument("--attn-only", action="store_true",
                    help="instead of the performer step, time one block_causal_attn call of the "
                         "workload's unit (e.g. --workload v02_share8: one GPU's 5-head share)")
    ap.add_argument("--stream-units", type=int, default=0,
                    help="instead of the performer step, stream N consecutive units through a "
                         "session (page allocation, mid-page appends), eager and as HIP graphs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    global torch
    import torch
    import block_causal_attention_performer_amd as bca
    import workloads

    w = workloads.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    print(f"[bench] workload {w.name}: generating inputs on device", file=sys.stderr, flush=True)
    inp = workloads.make_unit_inputs(w, device=dev)
    H, D, ps, lq = w.n_heads, w.head_dim, w.page_size, w.unit_tokens
    n_log = -(-w.n_kv // ps)
    pt = workloads.page_table(n_log, n_log + 1, 1234)
    cache = bca.KVCache(H, D, ps, pt, n_log + 1, w.dtype if w.dtype != "fp8" else "fp8", device=dev)
    bca.kv_append(cache, inp["k_hist"], inp["v_hist"])
    if args.catchup_units > 0:
        catchup(args, w, inp, cache, hip, stream, bca, workloads)
        return
    if args.attn_only:
        attn_call(args, w, inp, cache, hip, stream, bca)
        return
    if args.stream_units > 0:
        del cache
        stream_units(args, w, inp, bca, workloads)
        return
    ws = bca.alloc_workspace(bca.workspace_bytes(cache, lq, w.n_kv, w.n_ch))
    osc = torch.empty((lq, H, D), dtype=torch.bfloat16, device=dev)
    z = inp["eps"].clone()
    S = w.n_steps
    torch.cuda.synchronize()

    def step(events=None):
        cache.c.n_tokens = w.n_hist
        z.copy_(inp["eps"])
        bca.performer_unit(cache, inp["k_new"], inp["v_new"], inp["q"], inp["w"], z, S,
                           o_scratch=osc, workspace=ws, attn_events=events)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[hip.event() for _ in range(3 * S)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    clocks = ClockSampler()
    torch.cuda.synchronize()
    with clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_unit = wall * 1e3 / args.steps
    # main attention kernel (the roofline's kernel) and the whole call
    # (with the split combine and the exact rerun of flagged tiles)
    attn_ms = [hip.elapsed_ms(e[3 * s], e[3 * s + 1]) for e in evs for s in range(S)]
    call_ms = [hip.elapsed_ms(e[3 * s], e[3 * s + 2]) for e in evs for s in range(S)]
    attn_avg = sum(attn_ms) / len(attn_ms)
    call_avg = sum(call_ms) / len(call_ms)
    flops_call = w.attn_flops()
    attn_tflops = flops_call / (attn_avg * 1e-3) / 1e12
    value = S * flops_call / (ms_unit * 1e-3) / 1e12

    # ---- append and Euler alone (events around each call).  Between reps
    # the caches are flushed by READING a 1 GiB buffer: a write flush would
    # leave dirty lines in the 256 MB last-level cache whose write-back then
    # lands inside the timed kernel.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # float sum: no widening copy
    e0, e1 = hip.event(), hip.event()
    app_ms, eul_ms = [], []
    for _ in range(args.kernel_reps):
        flush.sum()
        cache.c.n_tokens = w.n_hist
        hip.record(e0, stream)
        bca.kv_append(cache, inp["k_new"], inp["v_new"])
        hip.record(e1, stream)
        app_ms.append(hip.elapsed_ms(e0, e1))
        flush.sum()
        hip.record(e0, stream)
        bca.fm_euler_step(z, osc, inp["w"], 1.0 / S, workspace=ws)
        hip.record(e1, stream)
        eul_ms.append(hip.elapsed_ms(e0, e1))
    # K and V read as bf16, written as bf16 (or fp8 codes; the per-page
    # scales are negligible)
    app_bytes = 2 * lq * H * D * (2 + (1 if w.dtype == "fp8" else 2))
    eul_bytes = lq * H * D * 2 + H * D * 16 * 4 + 2 * lq * 16 * 4
    app_med = sorted(app_ms)[len(app_ms) // 2]
    eul_med = sorted(eul_ms)[len(eul_ms) // 2]

    # the ceiling at these sizes: a plain device copy (torch) moving the
    # same number of bytes (half read, half written), timed the same way
    def copy_gbps(moved):
        src = torch.empty(moved // 2, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ms = []
        for _ in range(args.kernel_reps):
            flush.sum()
            hip.record(e0, stream)
            dst.copy_(src)
            hip.record(e1, stream)
            ms.append(hip.elapsed_ms(e0, e1))
        return moved / (sorted(ms)[len(ms) // 2] * 1e-3) / 1e9

    app_copy = copy_gbps(app_bytes)
    eul_copy = copy_gbps(eul_bytes)
    del flush
    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    metric = METRIC if w.name == METRIC_WORKLOAD else METRIC.replace("v0.2 shapes", f"{w.name} shapes")
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_unit, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 S (Q as two e4m3 terms), bf16 PV" if w.dtype == "fp8" else "bf16",
        "data": "synthetic (seeded device draws, 0.5*N(0,1) Q/K/V rounded to bf16)",
        "config": {"workload": w.name, "heads": H, "head_dim": D, "unit_tokens": lq,
                   "hist_tokens": w.n_hist, "n_kv": w.n_kv, "page_size": ps,
                   "solver_steps": S, "latent_channels": w.n_ch, "parallelism": "none"},
        "ms_per_unit": round(ms_unit, 4),
        "units_per_s": round(1e3 / ms_unit, 2),
        "unit_budget_frac": round(ms_unit / UNIT_BUDGET_MS, 4),
        "attn_pct_mfma_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "attn_call_ms": round(call_avg, 4),
        "attn_call_tflops": round(flops_call / (call_avg * 1e-3) / 1e12, 2),
        "gfx_clock": clocks.report(attn_tflops),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic() if w.name == METRIC_WORKLOAD else None,
                     "kernel": "attn_dma_kernel<128, true>" if w.dtype == "fp8" else ATTN_KERNEL_NAME,
                     "avg_launch_ms": round(attn_avg, 4), "flops_per_launch": flops_call},
        "kernels": {
            "kv_append": {"median_ms": round(app_med, 5), "bytes": app_bytes,
                          "GBps": round(app_bytes / (app_med * 1e-3) / 1e9, 1),
                          "hbm_frac": round(app_bytes / (app_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "same_size_copy_GBps": round(app_copy, 1),
                          "frac_of_same_size_copy": round(app_bytes / (app_med * 1e-3) / 1e9 / app_copy, 3)},
            "fm_euler_step": {"median_ms": round(eul_med, 5), "bytes": eul_bytes,
                              "GBps": round(eul_bytes / (eul_med * 1e-3) / 1e9, 1),
                              "hbm_frac": round(eul_bytes / (eul_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "same_size_copy_GBps": round(eul_copy, 1),
                              "frac_of_same_size_copy": round(eul_bytes / (eul_med * 1e-3) / 1e9 / eul_copy, 3)},
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_rows, args.cpu_heads, workloads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
