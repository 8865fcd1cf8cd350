"""Benchmark of one ring member's attention share on one MI355X.

A step is one ra_share_forward call: rank `rank`'s resident query block against all
N K/V blocks of the sequence in ring order, online softmax, final rescale.  Inputs
are seeded synthetic tensors already resident in GPU memory.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA: 256 CU x 8192 FLOP/clk x 2.4 GHz
CSRC = os.path.join(ROOT, "long_context_exact_ra_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "fwd_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_share_L128K_N8.json")


def kernel_sha(src: str = KERNEL_SRC) -> str:
    """sha256[:16] of the source file that holds the timed kernel."""
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_per_launch(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


class ClockSampler:
    """Graphics clock (MHz, mean over the XCDs) during the timed steps, from the GPU
    metrics table that amdsmi (ROCm's Python module) reads.  The table is refreshed by
    the firmware only every so often, so a reading counts only when the table's
    accumulated-activity field has moved since the previous one (a fresh table); one
    more reading is taken right after the steps finish.  mean() is None where the
    module, the device or the fields are unavailable."""

    def __init__(self, period_s: float = 0.02):
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None
        self._handle = None
        self._acc = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
            self._acc, _ = self._read()
        except Exception:  # no library, no permission, no device: no clock figure
            self._handle = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = m.get("current_gfxclks")
        vals = []
        if isinstance(clks, (list, tuple)):
            vals = [float(x) for x in clks if isinstance(x, (int, float)) and 0 < x < 10000]
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
            vals = [float(m["current_gfxclk"])]
        return m.get("gfx_activity_acc"), (sum(vals) / len(vals) if vals else None)

    def _take(self):
        acc, clk = self._read()
        if clk is not None and acc is not None and acc != self._acc:
            self.samples.append(clk)
        self._acc = acc

    def _loop(self):
        while not self._stop.is_set():
            try:
                self._take()
            except Exception:
                return
            self._stop.wait(self.period)

    def start(self):
        if self._handle is None:
            return
        import threading
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()

    def stop(self):
        """Call right after the steps have finished (after synchronising)."""
        if self._thread is None:
            return
        self._stop.set()
        self._thread.join()
        try:
            self._take()
        except Exception:
            pass

    def running(self):
        return self._thread is not None and self._thread.is_alive()

    def mean(self):
        return sum(self.samples) / len(self.samples) if self.samples else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-secondary", dest="secondary", action="store_false",
                   help="skip the 32K share, FP8 and backward timings after the headline "
                        "in the default run")
    p.add_argument("--no-step-path", dest="step_path", action="store_false",
                   help="skip the secondary timing of the per-step path "
                        "(N x ra_step + ra_finalize), which runs by default")
    p.add_argument("--causal", choices=["contiguous", "striped", "zigzag"], default=None,
                   help="time the causal share under this token layout instead")
    p.add_argument("--rank", type=int, default=None, help="ring member to time")
    p.add_argument("--backward", action="store_true",
                   help="time the share's backward pass (ra_share_backward) instead")
    p.add_argument("--causal-sweep", action="store_true",
                   help="time every member's causal share under each layout (balance data)")
    p.add_argument("--fp8", action="store_true",
                   help="time the share from FP8 (e4m3) inputs (ra_share_forward_fp8) instead")
    p.add_argument("--incoherent", action="store_true",
                   help="with --fp8: quantize Q and K after a random-sign Hadamard rotation "
                        "(ra_quantize_fp8_hadamard)")
    p.add_argument("--copy-calib", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def copy_calibration():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 4 * n, "launches": 3}))


def _time_launches(step, steps: int, warmup: int):
    """Warm-ups, then `steps` launches bracketed by HIP events on the launch stream:
    (mean ms per step, sorted per-step ms)."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / steps
    return ms, sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))


def _secondary_record(name, kind, src, steps, ms, per_step, flops, peak, **more):
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[bench] {kind} {name}: {steps} steps, {ms:.4f} ms/step", file=sys.stderr, flush=True)
    return {"workload": name, "pass": kind, "steps": steps, "ms_per_step": round(ms, 4),
            "step_ms": {"median": round(per_step[len(per_step) // 2], 4),
                        "min": round(per_step[0], 4), "max": round(per_step[-1], 4)},
            "value": round(tflops, 2), "unit": "TFLOP/s", "flops_per_step": flops, **more,
            "kernel_source": os.path.basename(src), "kernel_sha": kernel_sha(src),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tflops / peak, 4)}}


def time_secondary(name, args):
    """One more bf16 share timed with the headline's protocol; its own figures only."""
    import torch

    from long_context_exact_ra_amd import ra, synth

    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"[bench] drawing {name}", file=sys.stderr, flush=True)
    q, k, v = (x.to(dev) for x in synth.draw_workload(w))
    scale = 1.0 / math.sqrt(w.d)
    O = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.float32, device=dev)

    def step():
        ra.share_forward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, q, k, v, scale, O)

    steps = max(args.steps, 100)  # a 32K share is 16x less work than the headline's
    ms, per_step = _time_launches(step, steps, max(args.warmup, 10))
    return _secondary_record(name, "forward", KERNEL_SRC, steps, ms, per_step, w.flops(),
                             PEAK_BF16_TFLOPS)


def time_secondary_fp8(name, args):
    """The same share from E4M3 inputs (quantized once, before the timed launches)."""
    import torch

    from long_context_exact_ra_amd import ra, synth

    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"[bench] drawing {name} (fp8)", file=sys.stderr, flush=True)
    q, k, v = (x.to(dev) for x in synth.draw_workload(w))
    scale = 1.0 / math.sqrt(w.d)
    T = ra.fp8_tiles(w.l)
    Q8 = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.uint8, device=dev)
    qs = torch.empty((w.B, w.H, 1, T), dtype=torch.float32, device=dev)
    K8 = torch.empty((w.B, w.H_kv, w.L, w.d), dtype=torch.uint8, device=dev)
    ks = torch.empty((w.B, w.H_kv, w.N, T), dtype=torch.float32, device=dev)
    V8 = torch.empty((w.B, w.H_kv, w.N, T, w.d, 64), dtype=torch.uint8, device=dev)
    vs = torch.empty((w.B, w.H_kv, w.d), dtype=torch.float32, device=dev)
    ra.quantize_fp8("rows", q, 1, Q8, qs)
    ra.quantize_fp8("rows", k, w.N, K8, ks)
    ra.quantize_fp8("vt", v, w.N, V8, vs)
    del q, k, v
    O = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.float32, device=dev)

    def step():
        ra.share_forward_fp8(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, Q8, qs, K8, ks, V8, vs,
                             scale, O)

    steps = max(args.steps, 20)
    ms, per_step = _time_launches(step, steps, max(args.warmup, 3))
    return _secondary_record(name, "forward, fp8 e4m3 products", os.path.join(CSRC, "fwd_fp8.hip"),
                             steps, ms, per_step, w.flops(), PEAK_FP8_TFLOPS, dtype="fp8_e4m3")


def time_secondary_backward(name, args):
    """The share's backward (ra_share_backward) after one forward; algorithmic FLOP = 2.5x
    the forward's (products S, dP, dV, dK, dQ)."""
    import torch

    from long_context_exact_ra_amd import ra, synth

    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"[bench] drawing {name} (backward)", file=sys.stderr, flush=True)
    q, k, v = (x.to(dev) for x in synth.draw_workload(w))
    scale = 1.0 / math.sqrt(w.d)
    g = torch.Generator().manual_seed(w.seed + 99)
    dO = torch.randn((w.B, w.H, w.l, w.d), generator=g).to(torch.bfloat16).to(dev)
    O = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.float32, device=dev)
    m = torch.empty((w.B, w.H, w.l), dtype=torch.float32, device=dev)
    lo = torch.empty_like(m)
    ra.share_forward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, q, k, v, scale, O, m, lo)
    dQ = torch.empty_like(O)
    dK = torch.zeros((w.B, w.H_kv, w.L, w.d), dtype=torch.float32, device=dev)
    dV = torch.zeros_like(dK)
    ws = torch.empty((max(16, int(ra.load().ra_share_backward_workspace(w.B, w.H, w.l))),),
                     dtype=torch.uint8, device=dev)

    def step():
        ra.share_backward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, q, k, v, O, dO, m, lo,
                          scale, dQ, dK, dV, ws)

    steps = max(min(args.steps, 10), 5)
    ms, per_step = _time_launches(step, steps, max(min(args.warmup, 3), 2))
    return _secondary_record(name, "backward", os.path.join(CSRC, "bwd_bf16.hip"), steps, ms,
                             per_step, 2.5 * w.flops(), PEAK_BF16_TFLOPS)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not "
              "supported (the ring transport across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from long_context_exact_ra_amd import ra, synth

    if args.copy_calib:
        copy_calibration()
        return

    name = args.workload or synth.HEADLINE
    w = synth.WORKLOADS[name]
    if w.dtype != "bf16" or w.full_q:
        raise SystemExit("bench workloads are the bf16 single-share configurations")
    if args.rank is not None:
        if not 0 <= args.rank < w.N:
            raise SystemExit(f"--rank must be in [0, {w.N})")
        w = dataclasses.replace(w, rank=args.rank)
    if args.causal_sweep:
        causal_sweep(w, args)
        return
    dev = torch.device("cuda:0")
    ra.load()
    print(f"[bench] drawing {name}", file=sys.stderr, flush=True)
    q, k, v = synth.draw_workload(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    scale = 1.0 / math.sqrt(w.d)
    O = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.float32, device=dev)

    if args.fp8 and args.backward:
        raise SystemExit("--fp8 times the forward share (optionally --causal) only")
    if args.incoherent and not args.fp8:
        raise SystemExit("--incoherent applies to --fp8 only")
    timed_src = os.path.join(
        CSRC, "fwd_fp8.hip" if args.fp8 else "bwd_bf16.hip" if args.backward else "fwd_bf16.hip")
    extra = {}
    if args.fp8:
        T = ra.fp8_tiles(w.l)
        u8, f32 = torch.uint8, torch.float32
        Q8 = torch.empty((w.B, w.H, w.l, w.d), dtype=u8, device=dev)
        qs = torch.empty((w.B, w.H, 1, T), dtype=f32, device=dev)
        K8 = torch.empty((w.B, w.H_kv, w.L, w.d), dtype=u8, device=dev)
        ks = torch.empty((w.B, w.H_kv, w.N, T), dtype=f32, device=dev)
        V8 = torch.empty((w.B, w.H_kv, w.N, T, w.d, 64), dtype=u8, device=dev)
        vs = torch.empty((w.B, w.H_kv, w.d), dtype=f32, device=dev)

        if args.incoherent:
            gs = torch.Generator().manual_seed(w.seed + 21)
            args.signs = torch.where(torch.rand(w.d, generator=gs) < 0.5, -1.0, 1.0).float()
            signs_d = args.signs.to(dev)

        def quantize():
            if args.incoherent:
                ra.quantize_fp8_hadamard(qd, signs_d, 1, Q8, qs, query_side=True)
                ra.quantize_fp8_hadamard(kd, signs_d, w.N, K8, ks, query_side=False)
            else:
                ra.quantize_fp8("rows", qd, 1, Q8, qs)
                ra.quantize_fp8("rows", kd, w.N, K8, ks)
            ra.quantize_fp8("vt", vd, w.N, V8, vs)

        quantize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        quantize()
        e1.record()
        torch.cuda.synchronize()
        qbytes = 2 * (qd.numel() + kd.numel() + vd.numel())  # bf16 read once (V: twice)
        extra["quantize"] = {"ms": round(e0.elapsed_time(e1), 4),
                             "input_GB": round(qbytes / 1e9, 3)}

    if args.backward:
        g = torch.Generator().manual_seed(w.seed + 99)
        dOd = torch.randn((w.B, w.H, w.l, w.d), generator=g).to(torch.bfloat16).to(dev)
        m_f = torch.empty((w.B, w.H, w.l), dtype=torch.float32, device=dev)
        l_f = torch.empty_like(m_f)
        if args.causal:
            ra.causal_share_forward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, args.causal, qd,
                                    kd, vd, scale, O, m_f, l_f)
        else:
            ra.share_forward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, qd, kd, vd, scale, O,
                             m_f, l_f)
        dQ = torch.empty_like(O)
        dK = torch.zeros((w.B, w.H_kv, w.L, w.d), dtype=torch.float32, device=dev)
        dV = torch.zeros_like(dK)
        ws = torch.empty((max(16, int(ra.load().ra_share_backward_workspace(w.B, w.H, w.l))),),
                         dtype=torch.uint8, device=dev)

    def step():
        if args.fp8:
            ra.share_forward_fp8(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, Q8, qs, K8, ks, V8,
                                 vs, scale, O, layout=args.causal)
        elif args.backward and args.causal:
            ra.causal_share_backward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, args.causal, qd,
                                     kd, vd, O, dOd, m_f, l_f, scale, dQ, dK, dV, ws)
        elif args.backward:
            ra.share_backward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, qd, kd, vd, O, dOd,
                              m_f, l_f, scale, dQ, dK, dV, ws)
        elif args.causal:
            ra.causal_share_forward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, args.causal, qd,
                                    kd, vd, scale, O)
        else:
            ra.share_forward(w.rank, w.N, w.L, w.H, w.H_kv, w.d, w.B, qd, kd, vd, scale, O)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # One event per step boundary as well: the per-step spread beside the mean.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    clock = ClockSampler()
    torch.cuda.synchronize()
    clock.start()
    t0.record(stream)
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    # The metrics table behind the clock figure is refreshed about once a second: if no
    # fresh table arrived during the timed steps, the same work keeps running, untimed,
    # until one does (at most 2.5 s).
    clock_steps = 0
    t_wait = time.time()
    while clock.running() and not clock.samples and time.time() - t_wait < 2.5:
        step()
        torch.cuda.synchronize()
        clock_steps += 1
    clock.stop()
    ms = t0.elapsed_time(t1) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    extra["step_ms"] = {"median": round(per_step[len(per_step) // 2], 4),
                        "min": round(per_step[0], 4), "max": round(per_step[-1], 4)}
    print(f"[bench] {args.steps} steps, {ms:.3f} ms/step", file=sys.stderr, flush=True)
    flops = w.flops()
    if args.backward:  # S, dP, dV, dK, dQ products: 2.5x the forward's two
        flops = 2.5 * w.flops()
    if args.causal:  # useful work only: the admissible (query, key) pairs
        flops = 4.0 * w.d * w.B * w.H * ra.causal_pairs(w.rank, w.N, w.L, args.causal)
        if args.backward:
            flops *= 2.5
    tflops = flops / (ms * 1e-3) / 1e12

    if args.step_path and not (args.causal or args.backward or args.fp8):
        O_acc = torch.empty_like(O)
        m = torch.empty((w.B, w.H, w.l), dtype=torch.float32, device=dev)
        s = torch.empty_like(m)
        sched = ra.ring_schedule(w.rank, w.N)

        def step_path():
            ra.state_init(O_acc, m, s)
            for j in sched:
                ra.step(qd, kd[:, :, j * w.l:(j + 1) * w.l], vd[:, :, j * w.l:(j + 1) * w.l],
                        O_acc, m, s, scale)
            ra.finalize(O_acc, s)

        step_path()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(max(1, args.steps // 2)):
            step_path()
        t1.record(stream)
        torch.cuda.synchronize()
        sp_ms = t0.elapsed_time(t1) / max(1, args.steps // 2)
        extra["step_path"] = {"ms": round(sp_ms, 4),
                              "tflops": round(flops / (sp_ms * 1e-3) / 1e12, 2)}

    traffic = None if (args.causal or args.backward or args.fp8) else traffic_per_launch(name)
    peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic}
    sclk = clock.mean()
    # The nominal peak assumes 2.4 GHz; under full matrix load the clock runs lower.
    extra["sclk"] = {"mean_mhz": round(sclk, 1) if sclk else None,
                     "samples": len(clock.samples),
                     "untimed_steps_for_a_reading": clock_steps,
                     "pct_of_peak_at_mean_sclk":
                         round(100 * tflops / (peak * sclk / 2400.0), 2) if sclk else None}

    cpu_baseline = None
    parity = None
    if args.fp8 and not args.no_cpu_baseline:
        cpu_baseline, parity = fp8_cpu_baseline(w, q, k, v, O, scale, args)
    elif args.backward and not args.no_cpu_baseline:
        cpu_baseline, parity = backward_cpu_baseline(w, q, k, v, dOd, dQ, scale, args)
    elif not args.no_cpu_baseline:
        import oracle
        Q, K, V = (synth.to_oracle_array(x) for x in (q, k, v))
        threads = oracle.max_threads()
        if args.causal:
            qpos = oracle.token_positions(args.causal, w.rank, w.N, w.l)
            row_flops = lambda rows: float(np.sum(4.0 * w.d * (qpos[np.asarray(rows) % w.l] + 1)))

            def run_oracle(rows):
                return oracle.causal_share(Q, K, V, scale, w.rank, w.N, args.causal, rows=rows)
        else:
            row_flops = lambda rows: 4.0 * w.L * w.d * len(rows)

            def run_oracle(rows):
                return oracle.share(Q, K, V, scale, w.rank, w.N, rows=rows)
        per_row = 4.0 * w.L * w.d
        probe_rows = synth.sample_rows(w.B, w.H, w.l, 1, w.seed)[: max(8, threads)]
        t = time.perf_counter()
        run_oracle(probe_rows)
        probe_s = time.perf_counter() - t
        n_rows = int(max(len(probe_rows), len(probe_rows) * args.cpu_seconds / max(probe_s, 1e-3)))
        n_rows = min(n_rows, w.B * w.H * w.l)
        g = torch.Generator().manual_seed(w.seed + 11)
        rows = sorted(set(torch.randint(0, w.B * w.H * w.l, (n_rows,), generator=g).tolist()))
        print(f"[bench] oracle baseline on {len(rows)} rows, {threads} threads",
              file=sys.stderr, flush=True)
        t = time.perf_counter()
        ref, _, _ = run_oracle(rows)
        cpu_s = time.perf_counter() - t
        cpu_tflops = row_flops(rows) / cpu_s / 1e12
        cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": threads,
                        "kind": "oracle",
                        "sample": f"{len(rows)} random query rows of the same share "
                                  f"({row_flops(rows):.3e} FLOP, {cpu_s:.1f} s, fp64)"}
        got = O.reshape(-1, w.d)[torch.tensor(rows, device=dev)].double().cpu().numpy()
        err = np.abs(got - ref)
        parity = {"rows": len(rows), "max_abs_err": float(err.max()),
                  "ok": bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ref)))}

    # The other configuration the 50 % target names (the 32K share), and the 128K share's FP8
    # forward and bf16 backward, timed the same way in the default run: warm-ups, HIP events
    # on the launch stream, mean and median.
    if (not args.workload or args.workload == synth.HEADLINE) and args.secondary and not (
            args.causal or args.backward or args.fp8):
        del qd, kd, vd, O
        extra["also"] = {"share_L32K_N8": time_secondary("share_L32K_N8", args)}
        torch.cuda.empty_cache()
        extra["also"]["fp8_share_L128K_N8"] = time_secondary_fp8("share_L128K_N8", args)
        torch.cuda.empty_cache()
        extra["also"]["backward_share_L128K_N8"] = time_secondary_backward("share_L128K_N8",
                                                                           args)

    metric = "ring-share attention TFLOP/s (bf16) + % of MFMA peak at L=128K, N=8"
    if args.causal:
        metric = f"causal ring-share attention TFLOP/s, useful pairs only ({args.causal} layout)"
    if args.fp8:
        metric = "ring-share attention TFLOP/s (fp8 e4m3 products) + % of fp8 MFMA peak"
        if args.causal:
            metric = ("causal ring-share attention TFLOP/s, useful pairs only (fp8 e4m3 "
                      f"products, {args.causal} layout)")
    if args.backward:
        metric = "ring-share attention backward TFLOP/s (bf16; 2.5x forward FLOPs)"
        if args.causal:
            metric = ("causal ring-share attention backward TFLOP/s, useful pairs only "
                      f"({args.causal} layout; 2.5x forward FLOPs)")
    line = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.fp8 else "bf16",
        "data": "synthetic (seeded normal Q/K/V, resident in HBM)",
        "config": {"workload": name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "d": w.d, "L": w.L,
                   "N": w.N, "rank": w.rank, "l": w.l, "flops_per_step": flops,
                   **({"causal": args.causal} if args.causal else {}),
                   **({"pass": "backward"} if args.backward else {}),
                   **({"inputs": "fp8_e4m3, block-quantized" + (
                       " after a random-sign Hadamard rotation of Q and K"
                       if args.incoherent else "")} if args.fp8 else {})},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity": parity,
        "kernel_source": os.path.basename(timed_src),
        "kernel_sha": kernel_sha(timed_src),
        "env": {"torch": torch.__version__, "hip": torch.version.hip,
                "device": torch.cuda.get_device_name(0)},
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


def backward_cpu_baseline(w, q, k, v, dOd, dQ, scale, args):
    """The oracle's dQ rows of the same backward on a bounded sample of query rows of one
    head (each needs that head's full softmax statistics, computed in query chunks)."""
    import numpy as np
    import torch

    import oracle
    from long_context_exact_ra_amd import synth
    Q, K, V, dO = (synth.to_oracle_array(x) for x in (q, k, v, dOd.cpu()))
    h = w.H // 2
    t = time.perf_counter()
    n = 8
    res = oracle.share_backward_rows(Q, K, V, dO, scale, [(0, h)], list(range(n)), [],
                                     rank=w.rank, N=w.N, layout=args.causal)
    probe = time.perf_counter() - t
    # one head's statistics dominate: 4 d FLOP per (query, key) pair (the admissible
    # pairs only, for a causal share), plus the sampled rows
    pairs = (w.l * w.L if not args.causal else
             oracle.causal_pairs(w.rank, w.N, w.L, args.causal))
    stat_flops = 4.0 * pairs * w.d
    cpu_tflops = stat_flops / probe / 1e12
    got = dQ[0, h, :n].double().cpu().numpy()
    ref = res[0][0]
    err = float(np.abs(got - ref).max())
    return ({"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
             "kind": "oracle",
             "sample": f"one head's backward statistics and {n} dQ rows "
                       f"({stat_flops:.3e} FLOP, {probe:.1f} s, fp64 numpy)"},
            {"rows": n, "max_abs_err": err, "ok": bool(err <= 2e-2 * np.abs(ref).max() + 1e-5)})


def fp8_cpu_baseline(w, q, k, v, O, scale, args):
    """The oracle's FP8 share (its own quantization of two heads' bf16 inputs, then
    dequantization and the plain definition) on a bounded sample of those heads' rows;
    the GPU's rows are checked against it with the derived FP8 bound."""
    import numpy as np

    import oracle
    from oracle import fp8 as ofp8
    from long_context_exact_ra_amd import synth
    heads = [0, w.H // 2]
    group = w.H // w.H_kv
    codes = {}
    for h in heads:
        g = h // group
        qh, kh, vh = (synth.to_oracle_array(x) for x in
                      (q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1]))
        if args.incoherent:
            sg = args.signs.numpy()
            codes[h] = (*ofp8.quantize_rows_hadamard(qh, sg, 1, w.l, True),
                        *ofp8.quantize_rows_hadamard(kh, sg, w.N, w.l, False),
                        *ofp8.quantize_vt(vh, w.N, w.l))
        else:
            codes[h] = (*ofp8.quantize_rows(qh, 1, w.l), *ofp8.quantize_rows(kh, w.N, w.l),
                        *ofp8.quantize_vt(vh, w.N, w.l))
    threads = oracle.max_threads()
    def run_oracle(c, rows):
        if args.causal:
            return ofp8.causal_share_fp8(*c, scale, w.rank, w.N, args.causal, rows=rows)
        return ofp8.share_fp8(*c, scale, w.rank, w.N, rows=rows)

    # cost model from two probes: fixed (dequantization) + per row (attention); probe rows
    # from the end of the block, which for a causal share see the most keys
    t = time.perf_counter()
    run_oracle(codes[heads[0]], list(range(w.l - threads, w.l)))
    t1 = time.perf_counter() - t
    t = time.perf_counter()
    run_oracle(codes[heads[0]], list(range(w.l - 4 * threads, w.l)))
    t2 = time.perf_counter() - t
    per_row = max((t2 - t1) / (3 * threads), 1e-6)
    fixed = max(t1 - threads * per_row, 0.0)
    per_head = int((args.cpu_seconds / len(heads) - fixed) / per_row)
    per_head = min(max(per_head, threads), w.l)
    g = np.random.default_rng(w.seed + 13)
    t = time.perf_counter()
    refs, picks = [], []
    for h in heads:
        rows = np.sort(g.choice(w.l, size=per_head, replace=False))
        refs.append(run_oracle(codes[h], rows)[0])
        picks.append(rows)
    cpu_s = time.perf_counter() - t
    n = sum(len(p) for p in picks)
    if args.causal:  # useful pairs only, as the GPU figure
        qpos = oracle.token_positions(args.causal, w.rank, w.N, w.l)
        flops = float(sum(np.sum(4.0 * w.d * (qpos[p] + 1)) for p in picks))
    else:
        flops = 4.0 * w.L * w.d * n
    import torch
    worst, max_err, max_ref, n_bound = 0.0, 0.0, 0.0, 0
    for h, rows, ref in zip(heads, picks, refs):
        got = O[0, h][torch.tensor(rows, device=O.device)].double().cpu().numpy()
        Q8, qs, K8, ks, V8, vs = codes[h]
        chk = rows[:: max(1, len(rows) // 32)]  # the bound needs every score of a row
        sel = np.searchsorted(rows, chk)
        n_bound += len(chk)
        bO, _, _ = ofp8.error_bounds(ofp8.dequantize_rows(Q8, qs, w.l),
                                     ofp8.dequantize_rows(K8, ks, w.l),
                                     ofp8.dequantize_vt(V8, vs, w.l), scale, w.rank, w.N,
                                     ref[sel], chk, layout=args.causal)
        err = np.abs(got - ref)
        worst = max(worst, float((err[sel] / bO).max()))
        max_err, max_ref = max(max_err, float(err.max())), max(max_ref, float(np.abs(ref).max()))
    return ({"value": round(flops / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
             "kind": "oracle",
             "sample": f"{n} random query rows of heads {heads} of the same share: oracle "
                       f"quantization of those heads (untimed), then dequantization and fp64 "
                       f"attention ({flops:.3e} FLOP, {cpu_s:.1f} s)"},
            {"rows": n, "max_abs_err": max_err, "max_rel_to_max_ref": max_err / max_ref,
             "worst_err_over_fp8_bound": worst, "bound_rows": n_bound,
             "ok": bool(worst <= 1.0)})


def causal_sweep(w, args):
    """Every member's causal share under each layout: time per member and the spread
    (the load-balance question of the slowleelab page, 4.5 limitation 2 and 4.8)."""
    import torch

    from long_context_exact_ra_amd import ra, synth
    dev = torch.device("cuda:0")
    q, k, v = synth.draw_workload(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    scale = 1.0 / math.sqrt(w.d)
    O = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    steps = max(1, args.steps // 4)
    out = {"workload": w.name, "steps_per_rank": steps, "layouts": {}}
    for layout in ("contiguous", "striped", "zigzag"):
        ms = []
        for r in range(w.N):
            def step():
                ra.causal_share_forward(r, w.N, w.L, w.H, w.H_kv, w.d, w.B, layout, qd, kd, vd,
                                        scale, O)
            step()
            torch.cuda.synchronize()
            t0.record(stream)
            for _ in range(steps):
                step()
            t1.record(stream)
            torch.cuda.synchronize()
            ms.append(t0.elapsed_time(t1) / steps)
            print(f"[sweep] {layout} rank {r}: {ms[-1]:.3f} ms", file=sys.stderr, flush=True)
        pairs = [ra.causal_pairs(r, w.N, w.L, layout) for r in range(w.N)]
        useful = [4.0 * w.d * w.B * w.H * p / (t * 1e-3) / 1e12 for p, t in zip(pairs, ms)]
        out["layouts"][layout] = {
            "ms_per_rank": [round(x, 3) for x in ms],
            "max_over_min": round(max(ms) / min(ms), 3),
            "ring_step_ms": round(max(ms), 3),  # a ring waits for its slowest member
            "useful_tflops_per_rank": [round(x, 1) for x in useful]}
    print(json.dumps({"causal_sweep": out}), flush=True)


if __name__ == "__main__":
    main()
