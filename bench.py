"""Benchmark of the fused AllGather+GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]

One step = one persistent fused AllGather+GEMM launch of one rank's share of
a tensor-parallel MLP up-projection with 8 emulated ranks: local shard
[1024, 8192] bf16 plus 7 peer shards landing from a separate HBM region,
B [8192, 3584] bf16, C [8192, 3584] bf16 (481.04 GFLOP).  W untimed warm-up
steps, then K timed steps between device synchronisations; every step is
also bracketed by HIP events on the stream the kernel runs on, which gives
the kernel's duration per step (mean for the roofline; median, p10, p90).
The measured ceilings and GEMM alone are timed before the headline, so its
steps do not start from idle clocks.

Also measured and reported in the same JSON line (context, not the value):
  * overlap efficiency = max(GEMM alone, transfer alone) / fused, where GEMM
    alone is the same launch with A already gathered and transfer alone the
    same launch with no compute workgroups, the three timed interleaved call
    by call after the timed steps (same clock and power state for all three),
    and also each back to back in its own steady state as the timed steps run;
    the unfused baselines (the
    library's landing launch then its GEMM launch, and torch.cat + hipBLASLt
    matmul) on the same stream;
  * the same three with the 256 MB Infinity Cache flushed before each call;
  * the peers in pinned host memory (landing over PCIe): fused, transfer
    alone, landing GB/s, overlap efficiency;
  * the small AllGather+GEMM workload's latency (4 ranks, 512x256x256);
  * engine and memory clocks read before and after the timed steps;
  * GEMM+ReduceScatter and GEMM+AllReduce (fused, compute alone, transfer
    alone, with reduce workgroups, overlap efficiency), MoE dispatch +
    grouped GEMM (with and without the combine) and ring attention at their
    workload sizes (--quick skips these);
  * measured ceilings: an MFMA-only loop (TFLOP/s) and a plain device copy;
  * the CPU oracle timed on the same workload (median of 3 runs, the CPU
    model and the BLAS thread count).
Exactly one JSON line goes to stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
WORKLOAD = "ag_gemm_w8_8192x3584x8192"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources the AllGather+GEMM kernel and its launch are built from
AG_KERNEL_SOURCES = ("mk_device.h", "mk_host.hip", "mk_kernels.hip", "mk_params.h")


def kernel_source_hash() -> str:
    """Hash of the AllGather+GEMM kernel's sources: the stored counters apply
    only while it is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "communication_gemm_persistent_amd", "csrc")
    for f in AG_KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(src_hash: str):
    """HBM bytes per launch measured by rocprofv3 counters for this exact kernel
    source (profiles/ag_gemm_w8_counters.json), else None."""
    p = os.path.join(ROOT, "profiles", "ag_gemm_w8_8192x3584x8192_counters.json")
    try:
        with open(p) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed run of the headline call before the warm-up steps (0: none)")
    ap.add_argument("--profile-run", choices=["fused", "gemm_alone", "transfer_alone", "copy", "rs", "ar",
                                              "moe", "moe_combine", "ring"],
                    help="only launch the named kernel a few times (for rocprofv3 counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share; peers are emulated by buffers. "
              "Runs on more than one GPU are not supported.", file=sys.stderr)
        return 2

    import torch
    from communication_gemm_persistent_amd import inputs as I
    from communication_gemm_persistent_amd import mk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    h = mk.Handle(0, spin_timeout_ms=5000)

    def to_dev(bits_np, where="hbm"):
        t = torch.from_numpy(np.ascontiguousarray(bits_np).view(np.int16)).view(torch.bfloat16)
        return t.pin_memory() if where == "host" else t.to(dev)

    def to_dev_f32(x, where="hbm"):
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.pin_memory() if where == "host" else t.to(dev)

    if args.profile_run:
        return profile_run(args.profile_run, h, I, mk, to_dev, dev)

    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        flush_buf.fill_(1)

    def time_calls(fn, reps, warm, flushed=False):
        """Per-call kernel durations (ms) from events on the launch stream."""
        for _ in range(warm):
            fn()
        h.sync()
        durs = []
        for _ in range(reps):
            if flushed:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            durs.append((e0, e1))
        h.sync()
        return [a.elapsed_time(b) for a, b in durs]

    # ------------------------------------------------------------ headline workload
    wl = I.CONFIGS[WORKLOAD]
    p = wl.params
    W, m_s, n, k = p["world"], p["m_s"], p["n"], p["k"]
    flops = wl.flops()
    log(f"[bench] generating {WORKLOAD} inputs")
    d = I.gen_workload(WORKLOAD)
    shards = [to_dev(s) for s in d["shards"]]
    bt = to_dev(I.transpose_bits(d["b"]))
    c = torch.empty((W * m_s, n), dtype=torch.bfloat16, device=dev)
    ag = torch.empty((W * m_s, k), dtype=torch.bfloat16, device=dev)

    def fused():
        h.ag_gemm(shards, bt, c, ag, rank=0)

    # measured ceilings beside the nominal ones: an MFMA-only loop and a plain
    # device copy
    log("[bench] measured ceilings")
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    mfma_flop = [0.0]

    def mfma_loop():
        mfma_flop[0] = h.mfma_ceiling(2000, sink)

    t_mfma = float(np.median(time_calls(mfma_loop, 5, 2)))
    cp_src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    t_copy = float(np.median(time_calls(lambda: cp_dst.copy_(cp_src), 10, 2)))
    del cp_src, cp_dst
    ceilings = {"mfma_loop_tflops": round(mfma_flop[0] / (t_mfma * 1e-3) / 1e12, 1),
                "copy_read_plus_write_GBps": round(2 * COPY_BYTES / (t_copy * 1e-3) / 1e9, 1)}

    # GEMM alone (A already gathered) is timed before the headline as well:
    # these legs run first so that the headline's steps find the clocks out of
    # their idle state (the headline itself has exactly W warm-up steps)
    reps = max(10, args.steps // 2)
    log("[bench] GEMM alone")
    ag.copy_(torch.cat(shards, dim=0))
    gemm_alone = lambda: h.ag_gemm(shards, bt, c, ag, rank=0, flags=mk.F_PRELANDED)
    t_gemm_l = time_calls(gemm_alone, reps, 3)

    # untimed settle phase (see settle), then exactly W warm-up steps
    n_settle = settle(fused, torch.cuda.synchronize, args.settle_ms * 1e-3) if args.settle_ms > 0 else 0
    log("[bench] warm-up")
    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    clocks_before = read_clocks()
    log(f"[bench] timing {args.steps} fused steps")
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fused()
        e1.record(stream)
        events.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h.sync()
    kern_ms = [a.elapsed_time(b) for a, b in events]
    ms_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    value = flops * args.steps / wall / 1e12
    roles_fused, grid_fused = h.last_launch(mk.OP_AG_GEMM)

    # overlap efficiency: GEMM alone (pre-landed) and transfer alone (no compute)
    log("[bench] transfer alone / unfused")
    # the same landing with no compute: the fused launch's land workgroups, or
    # its whole grid when every workgroup lands between tiles (land = 0)
    n_land_alone = roles_fused[0] if roles_fused[0] > 0 else grid_fused

    def transfer_alone():
        h.set_roles(mk.OP_AG_GEMM, n_land=n_land_alone, n_compute=0)
        try:
            fused()
        finally:
            h.set_roles(mk.OP_AG_GEMM)

    # The three overlap legs interleaved call by call (fused, GEMM alone,
    # transfer alone, repeated), so that all three see the same clock and
    # power state; separate runs of each drift with the power management.
    def interleaved(fns, rounds):
        for fn in fns:
            fn()
        h.sync()
        ev = [[] for _ in fns]
        for _ in range(rounds):
            for i, fn in enumerate(fns):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev[i].append((e0, e1))
        h.sync()
        return [[a.elapsed_time(b) for a, b in e] for e in ev]

    t_fused_il, t_gemm_il, t_xfer_il = interleaved([fused, gemm_alone, transfer_alone], reps)
    # and each leg back to back in its own steady state, as the headline's
    # steps run (each settles first)
    settle(gemm_alone, h.sync, 0.05)
    t_gemm_bb = float(np.median(time_calls(gemm_alone, reps, 3)))
    settle(transfer_alone, h.sync, 0.02)
    t_xfer_bb = float(np.median(time_calls(transfer_alone, reps, 3)))
    # unfused: the landing launch, then the GEMM launch, on the same stream;
    # and torch's own: concatenate the shards, then hipBLASLt's matmul
    t_unfused_l = time_calls(lambda: (transfer_alone(), gemm_alone()), reps, 3)
    b_kn = bt.t()  # [k, n] view of B for torch.matmul (a column-major operand)
    a_full = torch.empty((W * m_s, k), dtype=torch.bfloat16, device=dev)
    c_torch = torch.empty((W * m_s, n), dtype=torch.bfloat16, device=dev)

    def torch_unfused():
        torch.cat(shards, dim=0, out=a_full)
        torch.matmul(a_full, b_kn, out=c_torch)

    t_torch_l = time_calls(torch_unfused, reps, 3)
    t_torch_gemm_l = time_calls(lambda: torch.matmul(a_full, b_kn, out=c_torch), reps, 3)
    t_fused_med = float(np.median(kern_ms))
    t_fused_ov = float(np.median(t_fused_il))
    t_gemm, t_xfer = float(np.median(t_gemm_il)), float(np.median(t_xfer_il))
    landed_bytes = (W - 1) * m_s * k * 2

    log("[bench] Infinity-Cache-flushed calls")
    t_fused_fl = float(np.median(time_calls(fused, reps, 2, flushed=True)))
    t_gemm_fl = float(np.median(time_calls(gemm_alone, reps, 2, flushed=True)))
    t_xfer_fl = float(np.median(time_calls(transfer_alone, reps, 2, flushed=True)))
    mall_flushed = {"t_fused_ms": round(t_fused_fl, 4), "t_gemm_alone_ms": round(t_gemm_fl, 4),
                    "t_transfer_alone_ms": round(t_xfer_fl, 4),
                    "fused_tflops": round(flops / (t_fused_fl * 1e-3) / 1e12, 2),
                    "efficiency": round(max(t_gemm_fl, t_xfer_fl) / t_fused_fl, 4)}

    # peers in pinned host memory: landing reads cross PCIe
    log("[bench] PCIe (pinned host) peers")
    shards_host = [shards[0]] + [to_dev(s, "host") for s in d["shards"][1:]]

    def fused_host():
        h.ag_gemm(shards_host, bt, c, ag, rank=0)

    t_fused_host = float(np.median(time_calls(fused_host, max(5, reps // 2), 2)))
    (nl_h, _, _), grid_h = h.last_launch(mk.OP_AG_GEMM)

    def xfer_host():
        h.set_roles(mk.OP_AG_GEMM, n_land=nl_h if nl_h > 0 else grid_h, n_compute=0)
        try:
            fused_host()
        finally:
            h.set_roles(mk.OP_AG_GEMM)

    t_xfer_host = float(np.median(time_calls(xfer_host, max(5, reps // 2), 2)))
    del shards_host
    pcie = {"t_fused_ms": round(t_fused_host, 4), "t_transfer_alone_ms": round(t_xfer_host, 4),
            "pcie_read_GBps": round(landed_bytes / (t_xfer_host * 1e-3) / 1e9, 2),
            "fused_pcie_read_GBps": round(landed_bytes / (t_fused_host * 1e-3) / 1e9, 2),
            "fused_tflops": round(flops / (t_fused_host * 1e-3) / 1e12, 2),
            "efficiency": round(max(t_gemm, t_xfer_host) / t_fused_host, 4)}

    # the small workload: latency of one call
    log("[bench] ag_gemm_w4_512x256x256 latency")
    d1 = I.gen_workload("ag_gemm_w4_512x256x256")
    sh1 = [to_dev(s) for s in d1["shards"]]
    bt1 = to_dev(I.transpose_bits(d1["b"]))
    c1 = torch.empty((4 * 128, 256), dtype=torch.bfloat16, device=dev)
    ag1 = torch.empty((4 * 128, 256), dtype=torch.bfloat16, device=dev)
    t_c1 = time_calls(lambda: h.ag_gemm(sh1, bt1, c1, ag1, rank=0), 50, 5)
    c1_latency = {"workload": "ag_gemm_w4_512x256x256", **pctl(t_c1, scale=1e3, unit="us")}
    del sh1, bt1, c1, ag1, d1

    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(src_hash)
    achieved = flops / (kern_avg * 1e-3) / 1e12
    result = {
        "metric": "fused AG+GEMM TFLOP/s & % bf16 MFMA peak; overlap eff. vs GEMM-alone",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "emulated_world": W, "rank": 0, "m_shard": m_s,
                   "m": W * m_s, "n": n, "k": k, "peers": "separate HBM region",
                   "roles": {"land": roles_fused[0], "compute": roles_fused[1]},
                   "grid": grid_fused},
        "timing": {"fused_kernel_ms": pctl(kern_ms), "settle_calls_before_warmup": n_settle,
                   "clocks_before": clocks_before,
                   "clocks_after": read_clocks()},
        "ceilings": dict(ceilings, fused_frac_of_mfma_loop=round(achieved / ceilings["mfma_loop_tflops"], 4)),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_avg_ms": round(kern_avg, 4),
                     "kernel_source_hash": src_hash},
        "overlap": {
            "measured": "fused, GEMM alone and transfer alone interleaved call by call",
            "t_fused_ms": round(t_fused_ov, 4), "t_gemm_alone_ms": round(t_gemm, 4),
            "t_transfer_alone_ms": round(t_xfer, 4), "transfer_alone_land_wgs": n_land_alone,
            "efficiency": round(max(t_gemm, t_xfer) / t_fused_ov, 4),
            "gemm_alone_over_fused": round(t_gemm / t_fused_ov, 4),
            "transfer_hidden_frac": round((t_gemm + t_xfer - t_fused_ov) / t_xfer, 4),
            "gemm_alone_tflops": round(flops / (t_gemm * 1e-3) / 1e12, 2),
            "landing_GBps": round(2 * landed_bytes / (t_xfer * 1e-3) / 1e9, 1),
            "fused_ms_pctl": pctl(t_fused_il), "gemm_alone_ms_pctl": pctl(t_gemm_il),
            "transfer_alone_ms_pctl": pctl(t_xfer_il),
            "gemm_alone_before_settle_ms": round(float(np.median(t_gemm_l)), 4),
            "back_to_back": {"t_fused_ms": round(t_fused_med, 4), "t_gemm_alone_ms": round(t_gemm_bb, 4),
                             "t_transfer_alone_ms": round(t_xfer_bb, 4),
                             "efficiency": round(max(t_gemm_bb, t_xfer_bb) / t_fused_med, 4),
                             "transfer_hidden_frac": round((t_gemm_bb + t_xfer_bb - t_fused_med) / t_xfer_bb, 4)},
        },
        "unfused": {"library_land_then_gemm_ms": round(float(np.median(t_unfused_l)), 4),
                    "torch_cat_then_matmul_ms": round(float(np.median(t_torch_l)), 4),
                    "torch_matmul_alone_ms": round(float(np.median(t_torch_gemm_l)), 4),
                    "fused_speedup_vs_library_unfused": round(float(np.median(t_unfused_l)) / t_fused_med, 4),
                    "fused_speedup_vs_torch_unfused": round(float(np.median(t_torch_l)) / t_fused_med, 4)},
        "mall_flushed": mall_flushed,
        "pcie_host_peers": pcie,
        "c1_latency": c1_latency,
    }
    del shards, bt, c, ag, d, a_full, c_torch
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ other fused ops
    if not args.quick:
        result["other_ops"] = other_ops(h, I, mk, to_dev, to_dev_f32, time_calls, dev)

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(I, flops)
    h.close()
    print(json.dumps(result), flush=True)
    return 0


def pctl(xs, scale=1.0, unit="ms"):
    """Median, p10 and p90 of per-call times (ms, times scale)."""
    a = np.asarray(xs, dtype=np.float64) * scale
    return {"unit": unit, "median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4), "p90": round(float(np.percentile(a, 90)), 4),
            "n": int(a.size)}


def read_clocks():
    """Current engine / memory clocks as amd-smi (or rocm-smi) reports them,
    best effort: a dict, or the reason none could be read."""
    import subprocess
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.TimeoutExpired) as e:
            last = f"{cmd[0]}: {e}"
            continue
        if r.returncode == 0 and r.stdout.strip():
            try:
                return {"tool": cmd[0], "data": _trim_clocks(json.loads(r.stdout))}
            except ValueError:
                return {"tool": cmd[0], "text": r.stdout.strip()[:400]}
        last = f"{cmd[0]}: rc {r.returncode} {r.stderr.strip()[:200]}"
    return {"error": last}


def _trim_clocks(j):
    """The current clock of each clock domain in an smi JSON dump, in MHz
    (keys ending in clk/value, or cur_clk-like entries)."""
    out = {}

    def walk(x, path):
        if isinstance(x, dict):
            for k, v in x.items():
                walk(v, path + [str(k)])
        elif isinstance(x, list):
            for i, v in enumerate(x):
                walk(v, path + [str(i)])
        else:
            if len(path) >= 3 and path[-1] == "value" and path[-2] == "clk":
                out[path[-3]] = x
            elif "sclk" in "/".join(path).lower() or "mclk" in "/".join(path).lower():
                out["/".join(path[-2:])] = x
    walk(j, [])
    return out


COPY_BYTES = 256 << 20


def profile_run(which, h, I, mk, to_dev, dev):
    """Launch one kernel kind 5 times (after 2 warm-ups) and exit: the program
    that rocprofv3 wraps for counter passes.  "copy" is a plain device copy of
    COPY_BYTES that calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch
    if which in ("rs", "ar", "moe", "moe_combine", "ring"):
        return profile_other(which, h, I, mk, to_dev, dev)
    if which == "copy":
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(7):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": which, "bytes": COPY_BYTES}))
        return 0
    wl = I.CONFIGS[WORKLOAD]
    p = wl.params
    W, m_s, n, k = p["world"], p["m_s"], p["n"], p["k"]
    d = I.gen_workload(WORKLOAD)
    shards = [to_dev(s) for s in d["shards"]]
    bt = to_dev(I.transpose_bits(d["b"]))
    c = torch.empty((W * m_s, n), dtype=torch.bfloat16, device=dev)
    ag = torch.empty((W * m_s, k), dtype=torch.bfloat16, device=dev)
    flags = 0
    if which == "gemm_alone":
        h.ag_gemm(shards, bt, c, ag, rank=0)      # gathers A once
        flags = mk.F_PRELANDED
    if which == "transfer_alone":                 # as the timed transfer-alone leg
        h.ag_gemm(shards, bt, c, ag, rank=0)
        (n_land, _, _), grid = h.last_launch(mk.OP_AG_GEMM)
        h.set_roles(mk.OP_AG_GEMM, n_land=n_land if n_land > 0 else grid, n_compute=0)
    for _ in range(7):
        h.ag_gemm(shards, bt, c, ag, rank=0, flags=flags)
    h.sync()
    print(json.dumps({"profile_run": which, "workload": WORKLOAD,
                      "roles": h.last_launch(mk.OP_AG_GEMM)}))
    return 0


def profile_other(which, h, I, mk, to_dev, dev):
    """--profile-run for the other fused ops at their workload sizes: 7
    launches of the default configuration."""
    import torch

    def f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    if which in ("rs", "ar"):
        name = "gemm_rs_w8_8192x8192x3584" if which == "rs" else "gemm_ar_w8_2048x8192x1024"
        p = I.CONFIGS[name].params
        d = I.gen_workload(name)
        W, m, n = p["world"], p["m"], p["n"]
        a, bt = to_dev(d["a"]), to_dev(I.transpose_bits(d["b"]))
        peers = [None] + [f32(x) for x in d["peers"][1:]]
        if which == "rs":
            ms = m // W
            c = torch.empty((ms, n), dtype=torch.bfloat16, device=dev)
            ob = [None] + [torch.empty((ms, n), dtype=torch.bfloat16, device=dev) for _ in range(W - 1)]
            call = lambda: h.gemm_rs(a, bt, peers, c, ob, rank=0)
        else:
            c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            bc = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for _ in range(p["n_bcast"])]
            call = lambda: h.gemm_ar(a, bt, peers, c, bc, rank=0)
    elif which in ("moe", "moe_combine"):
        name = "moe_s8_t4096_h4096_n1536_e64"
        p = I.CONFIGS[name].params
        d = I.gen_workload(name)
        S, T, H, N, E, E_loc, top_k = (p[x] for x in ("S", "T", "H", "N", "E", "E_loc", "top_k"))
        cap = S * T * min(top_k, E_loc)
        x = [to_dev(v) for v in d["x"]]
        lg = [f32(v) for v in d["logits"]]
        wt = to_dev(I.transpose_bits(d["w"]))
        y = torch.empty((cap, N), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((S * T, top_k), dtype=torch.int32, device=dev)
        gate = torch.empty((S * T, top_k), dtype=torch.float32, device=dev)
        st = torch.empty((cap,), dtype=torch.int32, device=dev)
        eo = torch.empty((E_loc + 1,), dtype=torch.int32, device=dev)
        co = torch.empty((E_loc, S + 1), dtype=torch.int32, device=dev)
        xs = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        if which == "moe":
            call = lambda: h.moe_dispatch_gemm(x, lg, wt, E, top_k, y, idx, gate, st, eo, co, xs, rank=0)
        else:
            yp = to_dev(np.ascontiguousarray(d["y_peer"]).reshape(T * top_k, N))
            ret = [None] + [torch.empty((T * top_k, N), dtype=torch.bfloat16, device=dev) for _ in range(S - 1)]
            o = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            call = lambda: h.moe_dispatch_gemm_combine(x, lg, wt, E, top_k, y, idx, gate, st, eo, co, xs,
                                                       yp, ret, o, rank=0)
    else:
        name = "ring_attn_w8_h32_s4096_d128"
        p = I.CONFIGS[name].params
        d = I.gen_workload(name)
        W, BH, S_q, S_kv, D = p["world"], p["B"] * p["H"], p["S_q"], p["S_kv"], p["D"]
        q = to_dev(d["q"].reshape(BH, S_q, D))
        ks = [to_dev(k.reshape(BH, S_kv, D)) for k in d["k"]]
        vs = [to_dev(v.reshape(BH, S_kv, D)) for v in d["v"]]
        o = torch.empty((BH, S_q, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((BH, S_q), dtype=torch.float32, device=dev)
        kr = torch.empty((W, BH, S_kv, D), dtype=torch.bfloat16, device=dev)
        vr = torch.empty((W, BH, D, S_kv), dtype=torch.bfloat16, device=dev)
        call = lambda: h.ring_attention(q, ks, vs, o, lse, kr, vr, rank=p["rank"])
    for _ in range(7):
        call()
    h.sync()
    print(json.dumps({"profile_run": which, "workload": name}))
    return 0


def other_ops(h, I, mk, to_dev, to_dev_f32, time_calls, dev):
    import torch
    out = {}
    # GEMM + ReduceScatter: fused (in-epilogue reduction, the default),
    # compute alone (no peer partials), transfer alone (no compute: the
    # reduce and scatter bytes), with 32 reduce workgroups
    name = "gemm_rs_w8_8192x8192x3584"
    log(f"[bench] {name}")
    wl = I.CONFIGS[name]
    p = wl.params
    d = I.gen_workload(name)
    W, m, n, k = p["world"], p["m"], p["n"], p["k"]
    ms = m // W
    a, bt = to_dev(d["a"]), to_dev(I.transpose_bits(d["b"]))
    peers = [None] + [to_dev_f32(x) for x in d["peers"][1:]]
    c_own = torch.empty((ms, n), dtype=torch.bfloat16, device=dev)
    outbox = [None] + [torch.empty((ms, n), dtype=torch.bfloat16, device=dev) for _ in range(W - 1)]
    rs = lambda fl=0: h.gemm_rs(a, bt, peers, c_own, outbox, rank=0, flags=fl)
    out[name] = reduce_op_legs(h, mk, mk.OP_GEMM_RS, rs, time_calls, wl.flops(),
                               (W - 1) * ms * n * 4 + ms * n * 2 + (W - 1) * ms * n * 2)
    del a, bt, peers, c_own, outbox, d
    torch.cuda.empty_cache()

    # GEMM + AllReduce
    name = "gemm_ar_w8_2048x8192x1024"
    log(f"[bench] {name}")
    wl = I.CONFIGS[name]
    p = wl.params
    d = I.gen_workload(name)
    W, m, n, k, nb = p["world"], p["m"], p["n"], p["k"], p["n_bcast"]
    a, bt = to_dev(d["a"]), to_dev(I.transpose_bits(d["b"]))
    peers = [None] + [to_dev_f32(x) for x in d["peers"][1:]]
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    bc = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    ar = lambda fl=0: h.gemm_ar(a, bt, peers, c, bc, rank=0, flags=fl)
    byts = (W - 1) * m * n * 4 + (1 + nb) * m * n * 2 + (m * k + n * k) * 2
    out[name] = reduce_op_legs(h, mk, mk.OP_GEMM_AR, ar, time_calls, wl.flops(), byts)
    out[name]["hbm_GBps"] = round(byts / (out[name]["ms"] * 1e-3) / 1e9, 1)
    out[name]["hbm_frac"] = round(out[name]["hbm_GBps"] / PEAK_HBM_GBS, 4)
    del a, bt, peers, c, bc, d
    torch.cuda.empty_cache()

    # MoE dispatch + grouped GEMM
    name = "moe_s8_t4096_h4096_n1536_e64"
    log(f"[bench] {name}")
    wl = I.CONFIGS[name]
    p = wl.params
    d = I.gen_workload(name)
    S, T, H, N, E, E_loc, top_k = (p[x] for x in ("S", "T", "H", "N", "E", "E_loc", "top_k"))
    cap = S * T * min(top_k, E_loc)
    x = [to_dev(v) for v in d["x"]]
    lg = [to_dev_f32(v) for v in d["logits"]]
    wt = to_dev(I.transpose_bits(d["w"]))
    y = torch.empty((cap, N), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((S * T, top_k), dtype=torch.int32, device=dev)
    gate = torch.empty((S * T, top_k), dtype=torch.float32, device=dev)
    st = torch.empty((cap,), dtype=torch.int32, device=dev)
    eo = torch.empty((E_loc + 1,), dtype=torch.int32, device=dev)
    co = torch.empty((E_loc, S + 1), dtype=torch.int32, device=dev)
    xs = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)

    def moe():
        h.moe_dispatch_gemm(x, lg, wt, E, top_k, y, idx, gate, st, eo, co, xs, rank=0)

    settle(moe, h.sync, 0.03)
    t = float(np.median(time_calls(moe, 20, 3)))
    n_slots = int(eo[-1].item())
    fl = wl.flops(n_slots)
    byts = S * T * E * 4 + 2 * n_slots * H * 2 + n_slots * H * 2 + E_loc * H * N * 2 + n_slots * N * 2
    out[name] = {"ms": round(t, 4), "n_slots": n_slots, "tflops": round(fl / (t * 1e-3) / 1e12, 2),
                 "mfma_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "hbm_frac": round(byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "GBps": round(byts / (t * 1e-3) / 1e9, 1), "roles": h.last_launch(mk.OP_MOE)[0]}

    # the same layer with the return of every remote token's rows and the combine
    log(f"[bench] {name} + combine")
    yp = to_dev(np.ascontiguousarray(d["y_peer"]).reshape(T * top_k, N))
    ret = [None] + [torch.empty((T * top_k, N), dtype=torch.bfloat16, device=dev)
                    for _ in range(S - 1)]
    o = torch.empty((T, N), dtype=torch.bfloat16, device=dev)

    def moe_combine():
        h.moe_dispatch_gemm_combine(x, lg, wt, E, top_k, y, idx, gate, st, eo, co, xs, yp, ret, o,
                                    rank=0)

    settle(moe_combine, h.sync, 0.03)
    tc = float(np.median(time_calls(moe_combine, 20, 3)))
    own = int((st[:n_slots] < T).sum().item())  # slots of this rank's own tokens stay local
    # extra over the dispatch: returned rows written, then the combine reads
    # top_k rows per own token (from y or y_peer) and writes out
    byts_c = byts + (n_slots - own) * N * 2 + T * top_k * N * 2 + T * N * 2
    out[name + "+combine"] = {
        "ms": round(tc, 4), "tflops": round(fl / (tc * 1e-3) / 1e12, 2),
        "GBps": round(byts_c / (tc * 1e-3) / 1e9, 1), "combine_extra_ms": round(tc - t, 4),
        "roles": h.last_launch(mk.OP_MOE)[0]}
    del x, lg, wt, y, idx, gate, st, eo, co, xs, d, yp, ret, o
    torch.cuda.empty_cache()

    # Ring attention
    name = "ring_attn_w8_h32_s4096_d128"
    log(f"[bench] {name}")
    wl = I.CONFIGS[name]
    p = wl.params
    d = I.gen_workload(name)
    W, BH, S_q, S_kv, D = p["world"], p["B"] * p["H"], p["S_q"], p["S_kv"], p["D"]
    q = to_dev(d["q"].reshape(BH, S_q, D))
    ks = [to_dev(k.reshape(BH, S_kv, D)) for k in d["k"]]
    vs = [to_dev(v.reshape(BH, S_kv, D)) for v in d["v"]]
    o = torch.empty((BH, S_q, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((BH, S_q), dtype=torch.float32, device=dev)
    kr = torch.empty((W, BH, S_kv, D), dtype=torch.bfloat16, device=dev)
    vr = torch.empty((W, BH, D, S_kv), dtype=torch.bfloat16, device=dev)

    def ring():
        h.ring_attention(q, ks, vs, o, lse, kr, vr, rank=p["rank"])

    t = float(np.median(time_calls(ring, 10, 2)))
    roles = h.last_launch(mk.OP_RING_ATTN)[0]
    t_alone = float(np.median(time_calls(
        lambda: h.ring_attention(q, [None] * W, [None] * W, o, lse, kr, vr, rank=p["rank"],
                                 flags=mk.F_PRELANDED), 10, 2)))
    h.set_roles(mk.OP_RING_ATTN, n_land=roles[0], n_compute=0)
    t_land = float(np.median(time_calls(ring, 10, 2)))
    h.set_roles(mk.OP_RING_ATTN)
    fl = wl.flops()
    landed = 2 * W * BH * S_kv * D * 2
    out[name] = {"ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 2),
                 "mfma_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "attn_alone_ms": round(t_alone, 4),
                 "attn_alone_tflops": round(fl / (t_alone * 1e-3) / 1e12, 2),
                 "land_alone_ms": round(t_land, 4),
                 "landing_GBps": round(2 * landed / (t_land * 1e-3) / 1e9, 1),
                 "overlap_efficiency": round(max(t_alone, t_land) / t, 4), "roles": roles}
    del q, ks, vs, o, lse, kr, vr, d
    torch.cuda.empty_cache()
    return out


def settle(fn, sync, seconds):
    """Run fn untimed for about `seconds` of wall time: after an idle period
    the first few dozen calls of a heavy launch go through a power-management
    transient (in kernel traces of the headline, calls 16-40 ran up to 20%
    slower than those before and after), which a measurement of the steady
    state must not include."""
    import time as _t
    t0 = _t.perf_counter()
    n = 0
    while n < 10 or _t.perf_counter() - t0 < seconds:
        for _ in range(5):
            fn()
        sync()
        n += 5
    return n


def reduce_op_legs(h, mk, op, call, time_calls, flops, comm_bytes):
    """GEMM+RS / GEMM+AR: fused (default roles), compute alone (MK_F_NO_PEERS),
    transfer alone (n_compute = 0: reduce workgroups move the reduce and
    scatter bytes), and fused with 32 reduce workgroups; overlap efficiency
    = max(compute alone, transfer alone) / fused.  The fused call settles
    for 50 ms first (see settle)."""
    settle(call, h.sync, 0.05)
    t = float(np.median(time_calls(call, 20, 5)))
    roles = h.last_launch(op)[0]
    t_gemm = float(np.median(time_calls(lambda: call(mk.F_NO_PEERS), 20, 3)))

    def with_roles(**r):
        def f():
            h.set_roles(op, **r)
            try:
                call()
            finally:
                h.set_roles(op)
        return f

    t_xfer = float(np.median(time_calls(with_roles(n_compute=0), 20, 3)))
    t_red = float(np.median(time_calls(with_roles(n_reduce=32), 20, 3)))
    return {"ms": round(t, 4), "tflops": round(flops / (t * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "comm_GBps": round(comm_bytes / (t * 1e-3) / 1e9, 1), "roles": roles,
            "t_compute_alone_ms": round(t_gemm, 4), "t_transfer_alone_ms": round(t_xfer, 4),
            "transfer_alone_GBps": round(comm_bytes / (t_xfer * 1e-3) / 1e9, 1),
            "efficiency": round(max(t_gemm, t_xfer) / t, 4),
            "t_fused_32_reduce_wgs_ms": round(t_red, 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(I, flops_full):
    """The float64 CPU oracle on the headline workload: the first R output
    rows (all 3584 columns, K = 8192, the gather included), R chosen from a
    short calibration so one run takes about 10 s (at most the whole
    workload); median of 3 runs."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    log("[bench] CPU oracle baseline")
    d = I.gen_workload(WORKLOAD)
    m_total = 8192
    rows = np.arange(128)
    t0 = time.perf_counter()
    O.ag_gemm_rows(d["shards"], d["b"], rows)
    t_cal = time.perf_counter() - t0
    R = int(min(m_total, max(128, 128 * 10.0 / max(t_cal, 1e-3))))
    rows = np.arange(R)
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        O.ag_gemm_rows(d["shards"], d["b"], rows)
        runs.append(time.perf_counter() - t0)
    t = float(np.median(runs))
    fl = flops_full * R / m_total
    return {"value": round(fl / t / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "runs_s": [round(x, 3) for x in runs],
            "sample": f"{R} of {m_total} output rows of {WORKLOAD} (all columns, K=8192), "
                      f"float64 numpy matmul with the gather; median of 3 runs, {t:.2f} s"}


if __name__ == "__main__":
    sys.exit(main())
