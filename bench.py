#!/usr/bin/env python3
"""MoE-FFN throughput on one MI355X, with the dominant kernel's roofline and
the fp64 CPU oracle timed beside it.

Default workload: 40 independent MoE FFN layers (seeds 0..39) at decode T=1,
the whole ~18 GB of 4-bit expert weights resident in HBM; one step = one
token through all 40 layers (40 library calls on one stream).  Other
workloads (single layers, flushed between repetitions) are available with
--workload for measurement.

With --block every call is the FFN sub-block with its boundary steps
(moe_ffn_block_forward: RMSNorm of the input on the way in, residual add on
the way out), with seeded per-layer norm weights; the workload name carries a
"+block" suffix.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
EXPERT_BYTES = 3 * (512 * 2048 // 2 + 2 * 512 * 32 * 2)  # gate+up+down packed + scales + biases = 1,769,472
GU_BYTES = 2 * (512 * 2048 // 2 + 2 * 512 * 32 * 2)      # gate+up of one expert = 1,179,648
DOWN_BYTES = 512 * 2048 // 2 + 2 * 2048 * 8 * 2           # down of one expert = 589,824
SHARED_BYTES = 3 * 512 * 2048 * 2
SHARED_DOWN_BYTES = 2048 * 512 * 2
ROUTER_BYTES = 256 * 2048 * 4
GATE_INP_BYTES = 2048 * 2

WORKLOADS = {
    "decode_T1_40layers": dict(T=1, layers=40, zipf=None, flush=False),
    "decode_T4": dict(T=4, layers=1, zipf=None, flush=True),
    "decode_T64": dict(T=64, layers=1, zipf=None, flush=True),
    "prefill_T4096_zipf1.0": dict(T=4096, layers=1, zipf=1.0, flush=True),
    "prefill_T32768_zipf1.5": dict(T=32768, layers=1, zipf=1.5, flush=True),
}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed PMC
    measurement (FETCH_SIZE + WRITE_SIZE, each scaled by the factor a plain
    copy of known size gives the same counter), or None when there is none
    or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        recs = json.load(fh)
    for r in recs:
        if r["workload"] == workload and r["kernel"] == kernel:
            if kernel_source_digest(r["sources"]) != r["sources_sha256"]:
                return None
            return int(round(1024 * (r["fetch_kib_per_dispatch"] * r["copy_factor_fetch"]
                                     + r["write_kib_per_dispatch"] * r["copy_factor_write"])))
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpus():
    """CPUs this process may run on (the affinity mask), and nproc's view."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return avail, os.cpu_count() or 1


def cpu_threads():
    """Threads of the CPU baseline: every CPU the process may use, at most 16
    (the host share of one GPU on the measurement machines)."""
    return max(1, min(16, host_cpus()[0]))


class Hip:
    """hipEvent_t handles through the HIP runtime's C API."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream)) == 0

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        """Elapsed ms between two events, NaN if they were never recorded
        (the runtime's error state is cleared again, or the next HIP call
        would report it)."""
        ms = ctypes.c_float()
        if self.L.hipEventSynchronize(b) != 0 or self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            self.L.hipGetLastError()
            return float("nan")
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="one workload (default: decode_T1_40layers, plus the sweep of the others)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 decode, 2 prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every traced kernel (stderr)")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of a HIP graph")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="how single-layer workloads evict the caches between calls: read 1 GiB (leaves clean "
                         "lines) or write 1 GiB (leaves the infinity cache full of dirty lines to write back)")
    ap.add_argument("--block", action="store_true",
                    help="time the FFN sub-block (RMSNorm in, residual out) instead of the bare FFN")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (calibrates PMC byte counters)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="with no --workload the run also times the other four workloads (one child process "
                         "each, before its own measurement) and lists them under other_workloads; this turns "
                         "that off")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    # the other workloads first, each in a child process, while this one has
    # not touched the GPU yet
    # (only when no workload was named: the profiling runs name theirs, and
    # a run under a profiler must not start other programs)
    others = None
    if args.workload is None:
        args.workload = "decode_T1_40layers"
        if not args.no_sweep and not args.block:
            others = sweep()

    import torch

    import synth
    import sparse_moe_ffn_fp32_amd as moe

    wl = WORKLOADS[args.workload]
    T, nlayers = wl["T"], wl["layers"]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    moe.lib()
    hip = Hip()
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read, {n} bytes written")
        del src, dst

    # ---------------------------------------------------------------- inputs
    # the CPU baseline runs one sampled layer per host thread
    n_cpu_layers = min(nlayers, cpu_threads())
    host_layers, dev_layers, xs, nws = [], [], [], []
    EPS = float(np.float32(1e-6))
    t0 = time.time()
    for l in range(nlayers):
        layer = synth.make_layer(l, zipf_s=wl["zipf"])
        x = synth.x_rows(l, T, 2048)
        dev_layers.append(moe.DeviceLayer.from_host(layer, dev))
        xs.append(torch.from_numpy(x.view(np.int16)).to(dev))
        nw = (1.0 + 0.2 * np.random.default_rng(1000 + l).standard_normal(2048)).astype(np.float32)
        nw = synth.bf16_to_f32(synth.f32_to_bf16(nw))
        nws.append(torch.from_numpy(nw).to(dev))
        if l < n_cpu_layers:
            host_layers.append((layer, x, nw))
        del layer
        if nlayers > 1 and (l % 8 == 7 or l == nlayers - 1):
            log(f"generated and uploaded layer {l + 1}/{nlayers} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    ys = [torch.empty((T, 2048), dtype=torch.int16, device=dev) for _ in range(nlayers)]
    idxs = [torch.empty((T, 8), dtype=torch.int32, device=dev) for _ in range(nlayers)]
    ws_ = [torch.empty((T, 8), dtype=torch.float32, device=dev) for _ in range(nlayers)]
    wspace = moe.alloc_workspace(T, dev, block=args.block)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if wl["flush"] else None
    if flush_buf is not None:
        flush_buf.fill_(1)
        flush_words = flush_buf.view(torch.int64)
        flush_sink = torch.empty((), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def call(l, trace=None, strm=None):
        strm = strm or stream
        if args.block:
            moe.moe_ffn_block_forward_traced(xs[l], nws[l], EPS, dev_layers[l], ys[l], wspace, idxs[l], ws_[l],
                                             stream=strm, path=args.path, trace=trace)
        else:
            moe.moe_ffn_forward_traced(xs[l], dev_layers[l], ys[l], wspace, idxs[l], ws_[l], stream=strm,
                                       path=args.path, trace=trace)

    dom_kernel = moe.KERNEL_EXPERT_GU

    last_step_ms = []  # per-call ms of the last single-layer run

    def run_steps_eager(nsteps, kernel=None):
        """nsteps steps launched directly; returns (wall seconds, per-launch ms of `kernel`)."""
        ev = [(hip.event(), hip.event()) for _ in range(nsteps * nlayers)] if kernel is not None else []
        if flush_buf is None:
            torch.cuda.synchronize()
            t = time.perf_counter()
            for s in range(nsteps):
                for l in range(nlayers):
                    call(l, moe.Trace(kernel, *ev[s * nlayers + l]) if kernel is not None else None)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t
        else:
            # single layer: read (or write) 1 GiB between repetitions, outside
            # the timed call, so no weights stay in the caches; time each call
            # with events.  A bounded device-side sleep queued before the start
            # event keeps the GPU busy while the host enqueues the event and
            # the call (argument checks, ctypes), so the interval holds the
            # call's GPU execution only.
            step_ms = []
            se, ee = hip.event(), hip.event()
            for s in range(nsteps):
                if args.flush == "write":
                    flush_buf.fill_(s & 0xFF)
                else:
                    flush_sink.copy_(flush_words.amax(), non_blocking=True)
                torch.cuda.synchronize()
                torch.cuda._sleep(int(2.4e9 * 300e-6))  # ~300 us of GPU time
                hip.record(se, stream)
                call(0, moe.Trace(kernel, *ev[s]) if kernel is not None else None)
                hip.record(ee, stream)
                step_ms.append(hip.elapsed_ms(se, ee))
            hip.destroy(se)
            hip.destroy(ee)
            last_step_ms[:] = step_ms
            wall = float(np.median(step_ms)) * 1e-3 * nsteps
        kms = [hip.elapsed_ms(a, b) for a, b in ev]
        for a, b in ev:
            hip.destroy(a)
            hip.destroy(b)
        return wall, kms

    def run_steps_graph(nsteps):
        """Multi-layer steps: the nsteps steps are captured into one HIP graph
        (launching 40 x several kernels per step from Python would otherwise
        leave the GPU idle between kernels), replayed once in the timed region."""
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=cap):
            for s in range(nsteps):
                for l in range(nlayers):
                    call(l, strm=cap)
        torch.cuda.synchronize()
        t = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t
        del g
        return wall

    def step_times_graph(nsteps):
        """Per-step ms of nsteps replays of a one-step graph, each between two
        events on the replay stream (for the spread of the step time)."""
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=cap):
            for l in range(nlayers):
                call(l, strm=cap)
        torch.cuda.synchronize()
        out = []
        a, b = hip.event(), hip.event()
        for _ in range(nsteps):
            hip.record(a, stream)
            g.replay()
            hip.record(b, stream)
            out.append(hip.elapsed_ms(a, b))
        hip.destroy(a)
        hip.destroy(b)
        del g
        return out

    def kernel_times(nsteps, kernel):
        """Per-launch ms of `kernel` over nsteps steps, from HIP events that the
        library records around it on the call's stream.  A bounded device-side
        sleep queued first keeps the GPU busy while Python enqueues the steps,
        so the intervals hold GPU execution only (events recorded inside a
        captured graph cannot be timed)."""
        if flush_buf is not None:
            return run_steps_eager(nsteps, kernel)[1]
        ev = [(hip.event(), hip.event()) for _ in range(nsteps * nlayers)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.004 * nsteps))  # ~4 ms of GPU time per step at 2.4 GHz
        for s in range(nsteps):
            for l in range(nlayers):
                call(l, moe.Trace(kernel, *ev[s * nlayers + l]))
        torch.cuda.synchronize()
        kms = [hip.elapsed_ms(a, b) for a, b in ev]
        for a, b in ev:
            hip.destroy(a)
            hip.destroy(b)
        return kms

    def run_steps(nsteps):
        if flush_buf is None and not args.eager:
            return run_steps_graph(nsteps)
        return run_steps_eager(nsteps)[0]

    log(f"warmup {args.warmup} steps")
    run_steps(max(1, args.warmup))
    torch.cuda.synchronize()
    distinct = [np.unique(i.cpu().numpy()).size for i in idxs]

    log(f"timing {args.steps} steps")
    wall = run_steps(args.steps)
    if flush_buf is None and not args.eager:
        step_ms = step_times_graph(args.steps)
    elif flush_buf is not None:
        step_ms = list(last_step_ms)
    else:
        step_ms = []
    kms = kernel_times(args.steps, dom_kernel)
    ms_per_step = 1000.0 * wall / args.steps
    tokens_per_step = T  # one step pushes T tokens through all `nlayers` layers
    value = tokens_per_step / (wall / args.steps)

    # dominant kernel: algorithmic bytes / flops per launch
    kernel_ms = float(np.nanmean(kms))
    if T <= 64:
        # the gate/up launch also runs the shared expert's down projection:
        # routed gate/up weights of the distinct experts, the shared down
        # weights, x and the shared h in; routed h and the shared output out.
        # For T <= 4 it also streams the selected experts' down rows from HBM
        # (the down launch then reads them from cache), so they count here.
        down_here = DOWN_BYTES if T <= 4 else 0
        gu_bytes = [d * (GU_BYTES + down_here) + SHARED_DOWN_BYTES + T * 2048 * 2 + T * 512 * 4 + T * 8 * 512 * 2
                    + T * 2048 * 4 for d in distinct]
        per_launch = float(np.mean(gu_bytes))
        achieved = per_launch / (kernel_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic(args.workload, "expert_gate_up"),
                    kernel="expert_gate_up", alg_bytes_per_launch=int(per_launch),
                    avg_launch_us=round(kernel_ms * 1e3, 2))
    else:
        flops = 2.0 * T * 8 * 1024 * 2048
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_F16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_F16_TFLOPS, 4), traffic=measured_traffic(args.workload, "expert_gate_up"),
                    kernel="expert_gate_up", alg_flops_per_launch=flops,
                    avg_launch_us=round(kernel_ms * 1e3, 2))
    step_bytes = sum(d * EXPERT_BYTES + SHARED_BYTES + ROUTER_BYTES + GATE_INP_BYTES + T * 2048 * 4
                     + (2048 * 4 + T * 2048 * 2 if args.block else 0) for d in distinct)
    log(f"step {ms_per_step * 1e3:.1f} us, {value:.1f} tok/s, step bytes {step_bytes / 1e6:.1f} MB "
        f"-> {step_bytes / (wall / args.steps) / 1e9:.0f} GB/s; dominant kernel {kernel_ms * 1e3:.2f} us/launch")

    if args.breakdown:
        for kid, name in ((moe.KERNEL_ROUTER, "router"), (moe.KERNEL_EXPERT_GU, "expert_gu"),
                          (moe.KERNEL_EXPERT_DOWN, "expert_down"), (moe.KERNEL_COMBINE, "combine")):
            km = np.array(kernel_times(max(2, args.steps // 4), kid))
            if np.isfinite(km).any():
                log(f"  kernel {name}: {np.nanmean(km) * 1e3:.2f} us/launch")
            else:
                log(f"  kernel {name}: not launched on this path")

    # ---------------------------------------------------------------- oracle
    cpu = None
    if not args.no_cpu_baseline:
        import concurrent.futures as cf

        import oracle
        O = oracle.get()
        cores = cpu_threads()
        avail, nproc = host_cpus()
        if nlayers > 1:
            threads = min(cores, len(host_layers))
            done, t = 0, time.perf_counter()
            with cf.ThreadPoolExecutor(threads) as ex:
                while time.perf_counter() - t < 10.0:
                    list(ex.map(lambda hx: (O.block_forward(hx[0], hx[1], hx[2], EPS, nthreads=1) if args.block
                                            else O.forward(hx[0], hx[1], nthreads=1)), host_layers))
                    done += len(host_layers)
            el = time.perf_counter() - t
            cpu = dict(value=round((done / nlayers) * T / el, 3), unit="tokens/s", cores=threads, kind="oracle",
                       nproc=nproc, cpus_available=avail,
                       sample=f"{len(host_layers)} of the {nlayers} layers at T={T}, {done} layer calls in "
                              f"{el:.1f}s, one layer per thread; tokens/s scaled to the {nlayers}-layer step")
        else:
            # strided slices of the layer's tokens (every stride-th token, next
            # offset each pass, wrapping around) until about 10 s have passed
            layer, x, nw0 = host_layers[0]
            stride = max(1, T // 256)
            done, passes, t = 0, 0, time.perf_counter()
            while time.perf_counter() - t < 10.0:
                tok = np.arange(passes % stride, T, stride)
                if args.block:
                    O.block_forward(layer, x, nw0, EPS, tokens=tok, nthreads=cores)
                else:
                    O.forward(layer, x, tokens=tok, nthreads=cores)
                done += tok.size
                passes += 1
            el = time.perf_counter() - t
            cpu = dict(value=round(done / el, 2), unit="tokens/s", cores=min(cores, (T + stride - 1) // stride),
                       kind="oracle", nproc=nproc, cpus_available=avail,
                       sample=f"{passes} passes over strided slices of {T} tokens (every {stride}th token, "
                              f"offset advancing per pass), {done} tokens in {el:.1f}s")
        log(f"oracle: {cpu}")

    out = {
        "metric": "MoE-FFN tokens/s (decode T=1..64; prefill T=4K) + % HBM / MFMA roofline",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # operand type of the expert contractions (fp32 accumulation): the
        # decode kernels take bf16 activations and exact bf16 codes 128 + q,
        # the prefill GEMMs row-scaled fp16 on MFMA
        "dtype": "bf16" if (T <= 64 and args.path != 2) else "f16",
        "data": "synthetic",
        "config": {"workload": args.workload + ("+block" if args.block else ""), "T": T, "layers": nlayers,
                   "router_bias_zipf_s": wl["zipf"], "distinct_experts_per_layer": float(np.mean(distinct)),
                   "alg_bytes_per_step": int(step_bytes)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if step_ms:
        q = np.nanpercentile(np.array(step_ms) * 1e3, [10, 50, 90])
        out["step_us"] = {"p10": round(float(q[0]), 2), "p50": round(float(q[1]), 2), "p90": round(float(q[2]), 2),
                          "n": len(step_ms),
                          "how": "one-step graph replays between events" if nlayers > 1 else
                                 "per call between events, caches evicted before each"}
    if others is not None:
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


def sweep(steps=10, warmup=3):
    """The other workloads, each timed by a child run of this script (its
    own process, started before this one uses the GPU), reduced to their
    headline fields; a child that fails is recorded as such."""
    import subprocess

    res = {}
    for name in WORKLOADS:
        if name == "decode_T1_40layers":
            continue
        log(f"sweep: {name}")
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--steps", str(steps),
               "--warmup", str(warmup), "--no-cpu-baseline", "--no-sweep"]
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
            line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1] if r.returncode == 0 else None
        except (subprocess.TimeoutExpired, IndexError):
            r, line = None, None
        if line is None:
            res[name] = {"error": f"child exit {None if r is None else r.returncode}"}
            continue
        d = json.loads(line)
        roof = d["roofline"]
        res[name] = {"value": d["value"], "unit": d["unit"], "ms_per_step": d["ms_per_step"], "steps": d["steps"],
                     "dtype": d["dtype"], "step_us_p50": d.get("step_us", {}).get("p50"),
                     "roofline": {k: roof.get(k) for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                                           "kernel", "avg_launch_us")}}
    return res


if __name__ == "__main__":
    main()
