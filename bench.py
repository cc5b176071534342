"""Benchmark: sparse-FFN tokens/s of the TwELL path on one MI355X.

One step = the whole hot path over one batch, all on one HIP stream, in two
calls (together the same as one twell_ffn_forward):
  twell_pack_gate          gate GEMM (bf16 MFMA) + ReLU + TwELL epilogue
  twell_ffn_from_gate      overflow flags, ascending overflow list and work
                           order; the fused up/down gather over the TwELL
                           entries; one GEMM for the dense backup and the
                           overflow rows' up projection; their down projection
Inputs (seeded, synthetic, grid mode) are resident in HBM before timing.
Untimed steps run for --settle-seconds (clocks out of idle), then --warmup
steps, then the --steps timed ones back to back; timing events are HIP events
with a device-scope release.

Prints ONE JSON line (rank 0).  Default workload: the 2B-like layer
(T=8192, d_model=2048, d_ff=8192, bf16, tile 256, capacity 16).  Besides the
headline fields the line carries, each measured after the timed region:
stages_ms (the two calls, and the layer through the separate calls
twell_partition_overflow / twell_ffn_fused / twell_ffn_overflow), fused (gather bytes and rate), memory
(TwELL / dense backup / compact / dense h bytes), gate_stats (the gate with
activation statistics), conversions (hybrid <-> dense, compact storage),
backward (twell_ffn_backward vs the dense bf16 backward), cold_cache_stages_ms,
dense_bf16_ffn (torch on the same GPU), energy (board energy counter) and
cpu_baseline (the oracle on the host cores).  --workload decode_<T> (T <= 64)
times twell_ffn_decode instead; --workload stress_stack the 24-layer stack.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEC_WINDOWS = 64  # decode workloads: windows of the 2B layer the steps cycle through
METRIC = "sparse-FFN tokens/sec at 2B shape; HBM GB/s and MFMA util as % of peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="untimed steps before the warmup steps, so the GPU clocks leave their idle state")
    ap.add_argument("--workload", default="layer_2b")
    ap.add_argument("--max-ovf", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="target CPU-oracle time per measurement (dense / sparse x 1 thread / all threads)")
    ap.add_argument("--no-energy", action="store_true", help="skip the energy-per-token measurement")
    ap.add_argument("--no-stats", action="store_true", help="skip the gate-statistics variant timing")
    ap.add_argument("--no-conversions", action="store_true", help="skip the hybrid <-> dense conversion timing")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--batch-path", action="store_true",
                    help="decode-shaped workloads (T <= 64): time the batch path instead of twell_ffn_decode")
    ap.add_argument("--energy-seconds", type=float, default=2.0, help="run time per energy measurement")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a plain 256 MiB streaming kernel 3x first (counter calibration under rocprofv3)")
    return ap.parse_args()


COUNTERS = os.path.join(ROOT, "profiles", "counters_layer_2b.json")
GATE_SOURCES = ["unstructured_sparse_transformer_amd/csrc/gate_twell.hip",
                "unstructured_sparse_transformer_amd/csrc/twell_device.h"]


class DevEvent:
    """A timing event on the current HIP stream, recorded with a device-scope
    release (hipEventReleaseToDevice).  torch.cuda.Event uses the default
    system-scope release, whose cache write-back adds about 10-20 us to a
    bracketed kernel on MI355X; with a device-scope release the bracket reads
    within a few microseconds of the kernel's own duration in a kernel trace.
    Same interface as torch.cuda.Event: record(), elapsed_time(end) in ms."""
    _hip = None
    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self):
        import ctypes
        import torch
        if DevEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")  # the HIP runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            DevEvent._hip = hip
        self._ct = ctypes
        self._torch = torch
        self.ev = ctypes.c_void_p()
        st = DevEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.RELEASE_TO_DEVICE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        st = DevEvent._hip.hipEventRecord(self.ev, self._torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        f = self._ct.c_float()
        st = DevEvent._hip.hipEventElapsedTime(self._ct.byref(f), self.ev, end.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return float(f.value)

    def __del__(self):
        hip = type(self)._hip
        if hip is not None and self.ev:
            hip.hipEventDestroy(self.ev)


def settle(step, seconds, torch):
    """Run untimed steps for about `seconds` (in batches of 20, synchronised):
    an idle MI355X starts a burst at low clocks, and a handful of warmup steps
    (a few milliseconds) ends before the clocks have ramped up."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """Fabric-side (L2-miss) bytes per launch of `kernel` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the
    calibration kernel's known/measured ratio), or None when no summary exists
    for this workload or the kernel's sources changed since the counters were
    taken.  These bytes go to or come from the MALL or HBM: an upper bound on
    the kernel's HBM traffic, not HBM traffic itself."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    k = c.get("per_dispatch", {}).get(kernel)
    if not k or c.get("workload") != workload or c.get("sources_sha256", {}).get(kernel) != source_digest(
            c.get("sources", {}).get(kernel, [])):
        return None
    return k["fetch_bytes"] * c["calibration"]["read_factor"] + k["write_bytes"] * c["calibration"]["write_factor"]


FUSED_KERNELS = ("row_flags_kernel", "ffn_entries_kernel", "ffn_pass_kernel_up", "ffn_pass_kernel_down")


def pct(ms):
    """median, p10, p90 (ms) of a list of per-launch times."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.quantile(a, 0.1)), 4),
            "p90": round(float(np.quantile(a, 0.9)), 4), "n": int(a.size)}


def gpu_state():
    """GPU clock (current and maximum) and power cap from amdsmi, when available."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as ex:
        return {"error": f"amdsmi unavailable: {ex!r}"}
    try:
        h = amdsmi.amdsmi_get_processor_handles()[0]
        st = {}
        try:
            c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            st["sclk_mhz"] = c.get("clk")
            st["sclk_max_mhz"] = c.get("max_clk")
        except Exception as ex:
            st["sclk_error"] = repr(ex)
        try:
            pc = amdsmi.amdsmi_get_power_cap_info(h)
            cap = pc.get("power_cap")
            st["power_cap_w"] = round(cap / 1e6, 1) if cap and cap > 1e5 else cap
        except Exception as ex:
            st["power_cap_error"] = repr(ex)
        return st
    finally:
        amdsmi.amdsmi_shut_down()


def cpu_baseline(wl, seconds):
    """The oracle timed on this host: the scalar C library built here with
    -O3 -march=native (no BLAS anywhere), (a) the dense FFN -- z and u as
    scalar dot products, y = (ReLU(z) * u) . W_d -- and (b) what the path
    computes -- the gate as scalar dot products, the TwELL packer, the
    partition, the dense backup and the sum over the active neurons -- each
    with one thread and with all threads, on the first rows of the workload
    (a bounded sample sized to about `seconds` per measurement)."""
    import tempfile

    import numpy as np

    import oracle
    from oracle import build as obuild
    lib = obuild.build(native=True, out=os.path.join(tempfile.gettempdir(), f"twell_oracle_native_{os.getpid()}.so"))
    oracle.load(lib)
    all_threads = oracle.max_threads()

    def dense(sub):
        r = np.arange(sub.T)
        z = oracle.matmul_rows(sub.x, r, sub.wg_t)
        u = oracle.matmul_rows(sub.x, r, sub.wu_t)
        oracle.ffn_dense(z, u, sub.wd)

    def sparse(sub):
        z = oracle.matmul_rows(sub.x, np.arange(sub.T), sub.wg_t)
        t = oracle.pack_twell(z, sub.tile_w, sub.cap, sub.dtype)
        _, ovf_rows, _ = oracle.partition_overflow(t.cnt, sub.cap)
        oracle.dense_backup(z, ovf_rows, sub.dtype)
        oracle.ffn_active(z, sub.x, sub.wu_t, sub.wd, sub.dtype)

    res = {}
    for threads in (1, all_threads):
        oracle.set_threads(threads)
        for name, fn in (("dense", dense), ("sparse", sparse)):
            n = min(8, wl.T)
            t0 = time.perf_counter()
            fn(wl.rows(0, n))
            dt0 = time.perf_counter() - t0
            n2 = int(min(wl.T, max(n, n * seconds / max(dt0, 1e-4))))
            t0 = time.perf_counter()
            fn(wl.rows(0, n2))
            dt = time.perf_counter() - t0
            res[(name, threads)] = (n2, dt)
    oracle.load()
    try:
        os.remove(lib)
    except OSError:
        pass
    tps = {k: round(n / dt, 1) for k, (n, dt) in res.items()}
    return {"value": tps[("sparse", all_threads)], "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "sample": (f"first {res[('sparse', all_threads)][0]} of {wl.T} tokens of {wl.name}: scalar C oracle "
                       f"(fp64, no BLAS) -- gate, TwELL packer, partition, dense backup, sum over active neurons "
                       f"({res[('sparse', all_threads)][1]:.1f} s)"),
            "dense_tokens_per_s": tps[("dense", all_threads)],
            "one_thread": {"sparse_tokens_per_s": tps[("sparse", 1)], "dense_tokens_per_s": tps[("dense", 1)]},
            "samples": {f"{k[0]}_{k[1]}t": {"rows": n, "s": round(dt, 2)} for k, (n, dt) in res.items()},
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "os_cpu_count": os.cpu_count(),
            "build": obuild.build_command(native=True)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU sharding is a design note, "
                                   "not implemented", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import unstructured_sparse_transformer_amd as tw
    from workloads import make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tw.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload == "stress_stack":
        run_stack(args, tw, torch, np)
        return

    t0 = time.time()
    wl = make_workload(args.workload)
    if wl.T <= 64 and wl.dtype == "bf16" and not args.batch_path:
        run_decode(args, wl, tw, torch, np)
        return
    log(f"workload {wl.name}: T={wl.T} d={wl.d} F={wl.F} {wl.dtype} w={wl.tile_w} cap={wl.cap} "
        f"(generated in {time.time() - t0:.1f}s)")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)  # noqa: E731
    x, wg, wu, wd = to(wl.x), to(wl.wg_t), to(wl.wu_t), to(wl.wd)
    max_ovf = min(args.max_ovf, wl.T)
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    ws = tw.hybrid_workspace(hy, wl.d)
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    if args.calib_copy:
        # a plain streaming kernel of known traffic (fp32 elementwise multiply:
        # 256 MiB read + 256 MiB written per launch) for counter calibration
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("calibration: 3 x fp32 multiply, 268435456 B read + 268435456 B written each")
        del src, dst

    # One step = the layer: the gate (TwELL packing) and the rest of the layer
    # in a second call (twell_ffn_forward in two parts, so that the gate kernel
    # can be bracketed by events)
    def step():
        tw.twell_pack_gate(x, wg, hy.ell)
        tw.twell_ffn_from_gate(x, wg, wu, wd, hy, y, ws)

    def step_gate_events(ev):
        ev[0].record()
        tw.twell_pack_gate(x, wg, hy.ell)
        ev[1].record()
        tw.twell_ffn_from_gate(x, wg, wu, wd, hy, y, ws)

    # The same layer through the separate calls, events between them (the
    # per-call breakdown; there the dense backup and the overflow rows' up
    # projection are two GEMMs, one in each of the last two calls)
    def split_step(ev):
        ev[0].record()
        tw.twell_pack_gate(x, wg, hy.ell)
        ev[1].record()
        tw.twell_partition_overflow(x, wg, hy)
        ev[2].record()
        tw.twell_ffn_fused(hy.ell, x, wu, wd, y, ws, order=hy.order)
        ev[3].record()
        tw.twell_ffn_overflow(hy, x, wu, wd, y, ws)
        ev[4].record()

    # one step for the workload's statistics (host reads), then the settle and
    # warmup steps right before the timed region, with no idle gap between
    step()
    torch.cuda.synchronize()
    n_ovf = int(hy.n_ovf.item())
    if n_ovf > max_ovf:
        raise SystemExit(f"n_ovf={n_ovf} exceeds max_ovf={max_ovf}; rerun with --max-ovf {n_ovf}")
    cnt = hy.ell.cnt
    kept = torch.clamp(cnt, max=wl.cap).sum(1)
    ovf_mask = hy.row_ovf.bool()
    entries = int(kept[~ovf_mask].sum().item())
    nnz = int(cnt.sum().item())

    # ---- timed region: K whole steps back to back.  Only the dominant kernel is
    # bracketed by events (every event record costs a few microseconds of idle
    # GPU between kernels); the per-stage breakdown comes from a separate pass.
    evs = [[DevEvent() for _ in range(2)] for _ in range(args.steps)]
    settle(step, args.settle_seconds, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step_gate_events(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gate_all = [evs[k][0].elapsed_time(evs[k][1]) for k in range(args.steps)]
    gate_ms = float(np.mean(gate_all))
    ms_per_step = wall * 1e3 / args.steps
    value = wl.T * args.steps / wall

    # ---- per-step distribution: 50 steps, each between device-scope events
    dist_ev = [[DevEvent() for _ in range(2)] for _ in range(50)]
    for e in dist_ev:
        e[0].record()
        step()
        e[1].record()
    torch.cuda.synchronize()
    step_all = [e[0].elapsed_time(e[1]) for e in dist_ev]

    # ---- per-stage breakdown (after the timed region; events between all stages)
    sev = [[DevEvent() for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        sev[k][0].record()
        tw.twell_pack_gate(x, wg, hy.ell)
        sev[k][1].record()
        tw.twell_ffn_from_gate(x, wg, wu, wd, hy, y, ws)
        sev[k][2].record()
    torch.cuda.synchronize()
    main_ms = np.array([[sev[k][i].elapsed_time(sev[k][i + 1]) for i in range(2)] for k in range(args.steps)]).mean(0)
    sev = [[DevEvent() for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        split_step(sev[k])
    torch.cuda.synchronize()
    stage = np.array([[sev[k][i].elapsed_time(sev[k][i + 1]) for i in range(4)] for k in range(args.steps)])
    stage_ms = stage.mean(0)

    gate_flop = 2.0 * wl.T * wl.d * wl.F
    roofline = {"bound": "mfma", "kernel": "gate_twell_kernel (gate GEMM + TwELL epilogue)",
                "achieved": round(gate_flop / (gate_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gate_flop / (gate_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("gate_twell_kernel", wl.name)}

    # fused step: algorithmic bytes (per-token gather model and compulsory bytes)
    esz = 2 if wl.dtype == "bf16" else 4
    rows_twell = int((~ovf_mask).sum().item())
    n_b = wl.F // wl.tile_w
    gather_bytes = entries * 2 * wl.d * esz
    per_token = rows_twell * (wl.d * esz + n_b * 4 + 4 * wl.d) + entries * (esz + 1)
    kept_rows = hy.ell.idx  # noqa: F841  (union of active neurons computed on host below)
    with torch.no_grad():
        act = torch.zeros(wl.F, dtype=torch.bool, device=dev)
        b = torch.arange(n_b, device=dev).view(1, n_b, 1) * wl.tile_w
        slot = torch.arange(wl.cap, device=dev).view(1, 1, wl.cap)
        valid = (slot < torch.clamp(cnt, max=wl.cap).unsqueeze(-1)) & (~ovf_mask).view(-1, 1, 1)
        cols = (b + hy.ell.idx.long())[valid]
        act[cols] = True
        union = int(act.sum().item())
    compulsory = union * 2 * wl.d * esz + per_token
    fused_ms = float(stage_ms[2])
    fab = [measured_traffic(k, wl.name) for k in FUSED_KERNELS]
    fused = {"kernels": "twell_ffn_fused: row_flags_kernel + ffn_entries_kernel + ffn_pass_kernel (up pass) + "
                        "ffn_pass_kernel (down pass)",
             "ms": round(fused_ms, 4), "entries": entries,
             "gather_bytes": gather_bytes, "compulsory_bytes": compulsory,
             "gather_GBps": round((gather_bytes + per_token) / (fused_ms * 1e-3) / 1e9, 1),
             "compulsory_GBps": round(compulsory / (fused_ms * 1e-3) / 1e9, 1),
             "compulsory_frac_hbm": round(compulsory / (fused_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "fabric_bytes": None if None in fab else round(sum(fab)),
             "note": "compulsory_frac_hbm = compulsory bytes / time / 8 TB/s (the roofline fraction); "
                     "gather_GBps counts every gathered weight row (served mostly from L2); fabric_bytes = "
                     "calibrated FETCH_SIZE + WRITE_SIZE of the step's kernels (L2-miss traffic to MALL/HBM)"}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_s": args.settle_seconds, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded grid-mode inputs of the workload's shape and sparsity; no trained weights)",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "d_ff": wl.F, "tile_w": wl.tile_w,
                   "cap": wl.cap, "max_ovf": max_ovf, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "step_ms_dist": pct(step_all),
        "gate_ms_dist": pct(gate_all),
        "gpu": gpu_state(),
        "stages_ms": {"pack_gate": round(float(main_ms[0]), 4), "ffn_from_gate": round(float(main_ms[1]), 4),
                      "split_calls": {"pack_gate": round(float(stage_ms[0]), 4),
                                      "partition_overflow": round(float(stage_ms[1]), 4),
                                      "ffn_fused": round(float(stage_ms[2]), 4),
                                      "ffn_overflow": round(float(stage_ms[3]), 4)},
                      "note": "separate passes after the timed region, events between the calls"},
        "fused": fused,
        "workload_stats": {"nnz": nnz, "n_ovf": n_ovf, "twell_entries": entries, "union_active_twell": union,
                           "mean_active_per_token": round(nnz / wl.T, 2)},
        "memory": {"twell_bytes": int(wl.T * n_b * (4 + wl.cap * (esz + 1))),
                   "dense_backup_bytes": int(n_ovf * wl.F * esz), "dense_h_bytes": int(wl.T * wl.F * esz)},
    }

    # ---- gate with the activation statistics (per-neuron active counts, per-tile
    # L1 sums) against the plain gate, alternating, after the timed region
    if not args.no_stats:
        ncnt = torch.zeros(wl.F, dtype=torch.int32, device=dev)
        l1 = torch.empty((wl.T, n_b), dtype=torch.float32, device=dev)
        plain, with_stats = [], []
        for k in range(args.steps):
            for fn, acc in ((lambda: tw.twell_pack_gate(x, wg, hy.ell), plain),
                            (lambda: tw.twell_pack_gate_stats(x, wg, hy.ell, ncnt, l1), with_stats)):
                ev = [DevEvent() for _ in range(2)]
                ev[0].record()
                fn()
                ev[1].record()
                acc.append(ev)
        torch.cuda.synchronize()
        p_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in plain]))
        s_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in with_stats]))
        out["gate_stats"] = {"kernel": "gate_twell_kernel with statistics", "pack_gate_ms": round(p_ms, 4),
                             "pack_gate_stats_ms": round(s_ms, 4), "overhead_frac": round(s_ms / p_ms - 1, 4),
                             "dead_neurons": int((ncnt == 0).sum().item()),
                             "mean_l1_per_token": round(float(l1.sum(1).mean().item()), 4)}

    # ---- the same gate GEMM with a plain dense store of ReLU(z) (twell_gate_dense)
    # against twell_pack_gate, alternating: the price of the TwELL epilogue
    if wl.T * wl.F * esz <= (4 << 30):
        hd = torch.empty((wl.T, wl.F), dtype=dt, device=dev)
        plain_ev, twell_ev = [], []
        for k in range(args.steps):
            for fn, acc in ((lambda: tw.twell_gate_dense(x, wg, hd), plain_ev),
                            (lambda: tw.twell_pack_gate(x, wg, hy.ell), twell_ev)):
                ev = [DevEvent() for _ in range(2)]
                ev[0].record()
                fn()
                ev[1].record()
                acc.append(ev)
        torch.cuda.synchronize()
        pd = [e[0].elapsed_time(e[1]) for e in plain_ev]
        pt = [e[0].elapsed_time(e[1]) for e in twell_ev]
        out["gate_plain_store"] = {
            "kernel": "gate_dense_kernel (same GEMM core and tiles, epilogue: ReLU(z) stored densely in the "
                      "storage type)",
            "dense_ms": pct(pd), "twell_ms": pct(pt),
            "twell_epilogue_ms": round(float(np.median(pt) - np.median(pd)), 4),
            "dense_store_bytes": int(wl.T * wl.F * esz),
            "twell_store_bytes": int(out["memory"]["twell_bytes"])}
        del hd

    # ---- hybrid <-> dense conversions of this layer's activations (the training
    # kernels), HBM-bound: algorithmic bytes = the dense side (T x F elements)
    # plus the TwELL and dense-backup side
    if not args.no_conversions:
        dense_h = torch.empty((wl.T, wl.F), dtype=dt, device=dev)
        hc = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
        tw.twell_hybrid_to_dense(hy, dense_h)
        tw.twell_dense_to_hybrid(dense_h, hc)
        torch.cuda.synchronize()
        conv = {}
        side = int(wl.T * n_b * (4 + wl.cap * (esz + 1)) + n_ovf * wl.F * esz)
        for name, fn, nbytes in (("hybrid_to_dense", lambda: tw.twell_hybrid_to_dense(hy, dense_h),
                                  wl.T * wl.F * esz + side),
                                 ("dense_to_hybrid", lambda: tw.twell_dense_to_hybrid(dense_h, hc),
                                  wl.T * wl.F * esz + side)):
            evc = [(DevEvent(), DevEvent()) for _ in range(args.steps)]
            for e in evc:
                e[0].record()
                fn()
                e[1].record()
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in evc]))
            conv[name] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes,
                          "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        # compacted storage of the layer's hybrid (the activations training would save)
        cbuf = torch.empty(int(out["memory"]["twell_bytes"] + out["memory"]["dense_backup_bytes"] + (1 << 20)),
                           dtype=torch.uint8, device=dev)
        tw.twell_compact_hybrid(hy, cbuf)
        hdr = tw.compact_header(cbuf)
        if hdr["fits"]:
            for name, fn, nbytes in (("compact", lambda: tw.twell_compact_hybrid(hy, cbuf), side + hdr["bytes"]),
                                     ("compact_to_dense",
                                      lambda: tw.twell_compact_to_dense(cbuf, wl.T, wl.F, dt, dense_h),
                                      wl.T * wl.F * esz + hdr["bytes"])):
                evc = [(DevEvent(), DevEvent()) for _ in range(args.steps)]
                for e in evc:
                    e[0].record()
                    fn()
                    e[1].record()
                torch.cuda.synchronize()
                ms = float(np.mean([a.elapsed_time(b) for a, b in evc]))
                conv[name] = {"ms": round(ms, 4), "algorithmic_bytes": int(nbytes),
                              "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        out["memory"]["compact_bytes"] = int(hdr["bytes"])
        out["memory"]["compact_vs_dense_h"] = round(hdr["bytes"] / out["memory"]["dense_h_bytes"], 4)
        out["conversions"] = conv
        del dense_h, hc, cbuf

    # ---- backward pass on this layer's hybrid, next to the dense bf16 backward
    # (the same gradients as 2-D torch matmuls on the dense matrices)
    if not args.no_backward and dt == torch.bfloat16 and wl.d <= 2048:
        max_e = 1 << 19
        bws = tw.backward_workspace(wl.T, wl.F, wl.d, max_e)
        dy = torch.randn((wl.T, wl.d), dtype=torch.float32, device=dev)
        dxg = torch.empty((wl.T, wl.d), dtype=torch.float32, device=dev)
        gw = [torch.empty((wl.F, wl.d), dtype=torch.float32, device=dev) for _ in range(3)]

        def sparse_bw():
            tw.twell_ffn_backward(hy, x, wg, wu, wd, dy, dxg, gw[0], gw[1], gw[2], max_e, bws)

        dyb = dy.to(torch.bfloat16)

        def dense_bw():
            z = torch.matmul(x, wg.t())
            u = torch.matmul(x, wu.t())
            hh = torch.relu(z)
            g = torch.matmul(dyb, wd.t())
            du = g * hh
            dz = g * u * (z > 0)
            dx_ = torch.matmul(du, wu) + torch.matmul(dz, wg)
            return dx_, torch.matmul((hh * u).t(), dyb), torch.matmul(du.t(), x), torch.matmul(dz.t(), x)

        bwd = {}
        for name, fn in (("sparse", sparse_bw), ("dense_bf16", dense_bw)):
            for _ in range(3):
                fn()
            evc = [(DevEvent(), DevEvent()) for _ in range(args.steps)]
            for e in evc:
                e[0].record()
                fn()
                e[1].record()
            torch.cuda.synchronize()
            bwd[name + "_ms"] = round(float(np.mean([a.elapsed_time(b) for a, b in evc])), 4)
        ent, too_many = tw.backward_status(bws)
        bwd["entries"] = ent
        bwd["complete"] = not too_many and n_ovf <= max_ovf
        bwd["sparse_speedup"] = round(bwd["dense_bf16_ms"] / bwd["sparse_ms"], 3)
        out["backward"] = bwd
        del bws, dy, dxg, gw, dyb

    # ---- cold-cache variant: flush MALL/L2 with a 1 GiB write between steps (outside the events)
    if not args.no_cold:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = []
        for k in range(min(args.steps, 10)):
            flush.fill_(float(k))
            ev = [DevEvent() for _ in range(3)]
            step_gate_events(ev)
            ev[2].record()
            torch.cuda.synchronize()
            cold.append([ev[i].elapsed_time(ev[i + 1]) for i in range(2)])
        cold = np.array(cold).mean(0)
        out["cold_cache_stages_ms"] = {"pack_gate": round(float(cold[0]), 4),
                                       "ffn_from_gate": round(float(cold[1]), 4),
                                       "tokens_per_s": round(wl.T / (cold.sum() * 1e-3), 1)}
        del flush

    # ---- dense bf16 FFN on the same GPU (torch / hipBLASLt), comparator only
    if not args.no_dense:
        def dense_step():
            z = torch.matmul(x, wg.t())
            h = torch.relu(z) * torch.matmul(x, wu.t())
            return torch.matmul(h, wd)
        for _ in range(3):
            dense_step()
        torch.cuda.synchronize()
        e0, e1 = DevEvent(), DevEvent()
        e0.record()
        for _ in range(args.steps):
            dense_step()
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.steps
        out["dense_bf16_ffn"] = {"ms_per_step": round(dms, 4), "tokens_per_s": round(wl.T / (dms * 1e-3), 1),
                                 "tflops": round(3 * gate_flop / (dms * 1e-3) / 1e12, 1),
                                 "sparse_speedup": round(dms / ms_per_step, 3)}

    # ---- energy per token, sparse path vs the dense FFN (board energy counter)
    if not args.no_energy:
        fns = {"sparse": step}
        if not args.no_dense:
            fns["dense"] = dense_step
        out["energy"] = energy_per_token(fns, wl.T, args.energy_seconds, torch)

    # ---- CPU oracle on a bounded sample of the same workload (rank 0, N=1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def energy_per_token(fns, tokens_per_call, seconds, torch):
    """Joules per token of each callable, from the GPU's cumulative energy
    counter read before and after about `seconds` of back-to-back calls."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as ex:  # no energy counter on this machine
        return {"error": f"energy counter unavailable: {ex!r}"}

    def joules():
        e = amdsmi.amdsmi_get_energy_count(handle)
        return e["energy_accumulator"] * e["counter_resolution"] * 1e-6

    res = {}
    try:
        for name, fn in fns.items():
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            calls = 0
            while time.perf_counter() - t0 < 0.2:  # size the loop
                fn()
                calls += 1
            torch.cuda.synchronize()
            n = max(1, int(calls * seconds / max(time.perf_counter() - t0, 1e-3)))
            j0, t0 = joules(), time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            j1, t1 = joules(), time.perf_counter()
            res[name] = {"J_per_token": (j1 - j0) / (n * tokens_per_call), "avg_power_W": round((j1 - j0) / (t1 - t0), 1),
                         "seconds": round(t1 - t0, 2), "calls": n}
    finally:
        amdsmi.amdsmi_shut_down()
    if "sparse" in res and "dense" in res:
        res["sparse_vs_dense"] = round(res["sparse"]["J_per_token"] / res["dense"]["J_per_token"], 4)
    return res


def run_decode(args, wl, tw, torch, np):
    """Decode-shaped calls (T <= 64, bf16): one twell_ffn_decode call per step
    (gate, packing and partition, chunked gather, reduction: 4 kernels), next
    to the same call replayed from a HIP graph, the batch path
    (twell_ffn_forward) and the dense bf16 FFN on the same rows.  Step i
    takes window i mod 64 of the 2B layer's tokens (64 disjoint windows of T
    consecutive tokens, resident in HBM), so the timed steps see the layer's
    spread of active counts rather than one window's.
    Roofline: the step is bound by HBM; its algorithmic bytes are W_g read
    once, the W_u / W_d rows of every active (row, neuron), x, y and the TwELL
    written (averaged over the windows the timed steps take)."""
    from workloads import make_decode_windows
    dev = "cuda"
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)  # noqa: E731
    wins = make_decode_windows(wl.T, max_windows=DEC_WINDOWS)
    nw = len(wins)
    xs = to(np.concatenate([w.x for w in wins])).reshape(nw, wl.T, wl.d)
    xv = [xs[i] for i in range(nw)]
    wg, wu, wd = to(wl.wg_t), to(wl.wu_t), to(wl.wd)
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, torch.bfloat16, wl.T)
    ws = tw.decode_workspace(wl.T, wl.F, wl.d, wl.tile_w)
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device=dev)
    cur = [0]  # the next step's window

    def step():
        tw.twell_ffn_decode(xv[cur[0] % nw], wg, wu, wd, hy, y, ws)
        cur[0] += 1

    def timed(fn, k):
        evs = [(DevEvent(), DevEvent()) for _ in range(k)]
        settle(fn, args.settle_seconds, torch)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        cur[0] = 0  # the timed steps take windows 0, 1, ...
        t0 = time.perf_counter()
        for e in evs:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / k, float(np.mean([a.elapsed_time(b) for a, b in evs]))

    ms_wall, ms_ev = timed(step, args.steps)
    # per-window entries and overflow rows of the windows the timed steps took
    nnz_w, ovf_w = [], []
    for i in range(nw):
        tw.twell_ffn_decode(xv[i], wg, wu, wd, hy, y, ws)
        torch.cuda.synchronize()
        nnz_w.append(int(hy.ell.cnt.sum().item()))
        ovf_w.append(int(hy.n_ovf.item()))
    used = [i % nw for i in range(args.steps)]
    nnz = float(np.mean([nnz_w[i] for i in used]))
    esz = 2
    n_b = wl.F // wl.tile_w
    alg = int(wl.F * wl.d * esz + wl.T * wl.d * esz + nnz * 2 * wl.d * esz + wl.T * wl.d * 4 +
              wl.T * n_b * (4 + wl.cap * (esz + 1)))
    # the batch path on the same rows
    hb = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, torch.bfloat16, wl.T)
    wsb = tw.hybrid_workspace(hb, wl.d)

    def batch():
        tw.twell_ffn_forward(xv[cur[0] % nw], wg, wu, wd, hb, y, wsb)
        cur[0] += 1

    _, ms_batch = timed(batch, args.steps)
    # the same calls captured into HIP graphs (one per window) and replayed:
    # the host's launch cost of the four kernels leaves the step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []  # one graph per window (a graph keeps the x pointer it captured)
    for i in range(nw):
        graphs.append(torch.cuda.CUDAGraph())
        with torch.cuda.graph(graphs[-1]):
            tw.twell_ffn_decode(xv[i], wg, wu, wd, hy, y, ws)
    torch.cuda.synchronize()

    def replay():
        graphs[cur[0] % nw].replay()
        cur[0] += 1

    gms_wall, gms_ev = timed(replay, args.steps)
    out = {
        "metric": METRIC, "value": round(wl.T / (ms_wall * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_s": args.settle_seconds,
        "ms_per_step": round(ms_wall, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded grid-mode inputs of the workload's shape and sparsity; no trained weights)",
        "config": {"workload": f"decode_2b_T{wl.T} (windows 0..{nw - 1} of T tokens in turn)", "T": wl.T, "d_model": wl.d, "d_ff": wl.F, "tile_w": wl.tile_w,
                   "cap": wl.cap, "path": "twell_ffn_decode", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "decode step (gate, packing, gather, reduction)",
                     "achieved": round(alg / (ms_ev * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(alg / (ms_ev * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes": alg},
        "step_ms_events": round(ms_ev, 4),
        "batch_path_ms": round(ms_batch, 4),
        "graph_replay": {"ms_per_step": round(gms_wall, 4), "ms_events": round(gms_ev, 4),
                         "tokens_per_s": round(wl.T / (gms_wall * 1e-3), 1)},
        "workload_stats": {"windows": nw, "mean_nnz_timed": round(nnz, 2),
                           "nnz_per_window_min_max": [min(nnz_w), max(nnz_w)],
                           "windows_with_overflow": int(sum(1 for v in ovf_w if v > 0))},
    }
    if not args.no_dense:
        def dense_step():
            xx = xv[cur[0] % nw]
            cur[0] += 1
            h = torch.relu(torch.matmul(xx, wg.t())) * torch.matmul(xx, wu.t())
            return torch.matmul(h, wd)
        _, dms = timed(dense_step, args.steps)
        out["dense_bf16_ffn"] = {"ms_per_step": round(dms, 4), "sparse_speedup": round(dms / ms_ev, 3)}
    print(json.dumps(out), flush=True)


def run_stack(args, tw, torch, np):
    """The 24-layer overflow stress stack (T=16384, d=2048, F=8192, bf16): each
    layer's inputs are generated and uploaded in turn, then the whole path is
    timed on it; tokens/s = T / (sum over the layers of the step time)."""
    from workloads import make_stress_layer
    from workloads.gen import STRESS_LAYERS
    dev = "cuda"
    per_layer, gate_ms, n_ovf, dense_ms = [], [], [], None
    for layer in range(STRESS_LAYERS):
        wl = make_stress_layer(layer)
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)  # noqa: E731
        x, wg, wu, wd = to(wl.x), to(wl.wg_t), to(wl.wu_t), to(wl.wd)
        max_ovf = min(args.max_ovf * 4, wl.T)
        hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, torch.bfloat16, max_ovf)
        ws = tw.hybrid_workspace(hy, wl.d)
        y = torch.empty((wl.T, wl.d), dtype=torch.float32, device=dev)

        def step(ev=None):
            if ev:
                ev[0].record()
            tw.twell_pack_gate(x, wg, hy.ell)
            if ev:
                ev[1].record()
            tw.twell_ffn_from_gate(x, wg, wu, wd, hy, y, ws)

        if layer == 0:  # later layers follow without idle gaps
            settle(step, args.settle_seconds, torch)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        n = int(hy.n_ovf.item())
        if n > max_ovf:
            raise SystemExit(f"layer {layer}: n_ovf={n} exceeds max_ovf={max_ovf}")
        evs = [[DevEvent() for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(evs[k])
        torch.cuda.synchronize()
        per_layer.append((time.perf_counter() - t0) * 1e3 / args.steps)
        gate_ms.append(float(np.mean([e[0].elapsed_time(e[1]) for e in evs])))
        n_ovf.append(n)
        if dense_ms is None and not args.no_dense:  # the dense FFN's time does not depend on the layer
            def dense_step():
                h = torch.relu(torch.matmul(x, wg.t())) * torch.matmul(x, wu.t())
                return torch.matmul(h, wd)
            for _ in range(3):
                dense_step()
            torch.cuda.synchronize()
            e0, e1 = DevEvent(), DevEvent()
            e0.record()
            for _ in range(args.steps):
                dense_step()
            e1.record()
            torch.cuda.synchronize()
            dense_ms = e0.elapsed_time(e1) / args.steps
        log(f"stress layer {layer}: step {per_layer[-1]:.3f} ms, gate {gate_ms[-1]:.3f} ms, n_ovf {n}")
        del x, wg, wu, wd, hy, ws, y
    total = sum(per_layer)
    T, d, F = 16384, 2048, 8192
    gflop = 2.0 * T * d * F
    g = float(np.mean(gate_ms))
    out = {"metric": METRIC, "value": round(T / (total * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded grid-mode inputs of the workload's shape and sparsity; no trained weights)",
           "config": {"workload": "stress_stack (24 layers)", "T": T, "d_model": d, "d_ff": F, "tile_w": 256,
                      "cap": 16, "parallelism": "none (1 GPU)"},
           "roofline": {"bound": "mfma", "kernel": "gate_twell_kernel (mean over the layers)",
                        "achieved": round(gflop / (g * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(gflop / (g * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "traffic": None},
           "per_layer_ms": [round(v, 4) for v in per_layer], "n_ovf_per_layer": n_ovf}
    if dense_ms is not None:
        out["dense_bf16_ffn"] = {"ms_per_layer": round(dense_ms, 4), "ms_stack": round(24 * dense_ms, 4),
                                 "tokens_per_s": round(T / (24 * dense_ms * 1e-3), 1),
                                 "sparse_speedup": round(24 * dense_ms / total, 3)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
