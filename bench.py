"""Benchmark of the HSA hot path on one MI355X.

One step = one chunk of one layer through the whole path: the CAG schedule and block
budget on the host, then pooling (query block means, key block and frame means),
selection (frame top-k and block top-k: one launch) and block-sparse attention on the
GPU, each a C-ABI call on torch's current stream.
Default workload: the 480p layer at chunk 7 of 7, the headline configuration (12 heads x
128, 4680 query tokens against 21 frames = 32760 key tokens, 64-token blocks, memory set
frames 1..17, 4 retrieved frames + sink + the chunk's 3 frames, 8 blocks per frame);
--workload selects the chunk-2 layer, the 69-frame long-memory layer, the tiny case or
the full 30-layer x 7-chunk CAG sweep.

Steps cycle over R independent layers' inputs (R chosen so that together they exceed
twice the 256 MB Infinity Cache), so every step streams its K/V from HBM as in a real
layer-by-layer rollout. Inputs are resident in HBM before timing starts.

Printed: one JSON line with the headline (dense-equivalent HSA TFLOP/s), per-kernel
times from HIP events recorded on the launch stream, the attention kernel's roofline
(algorithmic FLOPs per launch / mean duration vs the 2.5 PFLOP/s bf16 dense peak), the
selection overhead and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import sparse_attention_autoregressive_amd as lf  # noqa: E402
from sparse_attention_autoregressive_amd.profsum import read_traffic  # noqa: E402
from sparse_attention_autoregressive_amd.pipeline import (ChunkPlan, PooledKeyCache, SweepWorkspace,  # noqa: E402
                                                          Workspace, attend, hsa_chunk, new_frames, plan_sweep,
                                                          pool, pool_cached, select, select_1d, select_cached,
                                                          sweep_layer)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "HSA effective TFLOP/s (dense-equiv) + % MFMA peak + select overhead %, 480p"
KERNELS = ["pool", "select", "attn"]


def chunk_flops(w):
    fpc = len(w.current)
    return [float(fpc * w.tpf * fpc * i * w.tpf) for i in range(1, w.n_chunks + 1)]


def block_lens(w):
    nb = -(-w.tpf // w.bs)
    return np.array([min(w.bs, w.tpf - j * w.bs) for j in range(nb)], dtype=np.int64)


def flops_of(w, blocks: np.ndarray):
    """(dense-equivalent, active) attention FLOPs of one chunk, 4*d per query-key pair
    (Q K^T and P V, 2 FLOPs per multiply-add each), with true ragged block lengths."""
    lens = block_lens(w)
    nb = len(lens)
    n_qb = blocks.shape[2]
    qlen = lens[np.arange(n_qb) % nb]
    dense = 4.0 * w.d * w.B * w.H * float(qlen.sum()) * w.lk
    active = 4.0 * w.d * float((qlen[None, None, :] * lens[blocks % nb].sum(axis=-1)).sum())
    return dense, active


def pool_bytes(w, n_frames, with_frames):
    """Algorithmic HBM bytes of one lf_pool call: read every token once, write the means."""
    esz = 2 if w.dtype == "bf16" else 4
    nb = -(-w.tpf // w.bs)
    rd = w.B * w.H * n_frames * w.tpf * w.d * esz
    wr = w.B * w.H * n_frames * nb * w.d * 4 + (w.B * w.H * n_frames * w.d * 4 if with_frames else 0)
    return rd + wr


def lag_bytes(w, n_lag):
    """Algorithmic HBM bytes of the lagged frame means of a steady-state pooling launch:
    read the frames' cached block means, write one mean per frame."""
    nb = -(-w.tpf // w.bs)
    return w.B * w.H * n_lag * (nb + 1) * w.d * 4


def run_cpu_baseline(w, k_b: int, heads: int, min_s: float):
    """The CPU oracle (numpy fp64) on the first `heads` heads of one layer: pool, select
    and attend, repeated until at least `min_s` seconds have passed. Returns
    (dense-equiv TFLOP/s, seconds, repeats, dense flops of one repeat)."""
    import dataclasses

    import oracle
    ws = dataclasses.replace(w, H=heads)
    x = synth.make(ws)
    q64, k64, v64 = x.np64()
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_s:
        t0 = time.perf_counter()
        out = oracle.hsa(q64, k64, v64, tpf=ws.tpf, bs=ws.bs, n_kframes=ws.n_kframes, mem=ws.mem,
                         forced=ws.forced, k_f=ws.k_f, k_b=k_b, scale=ws.scale)
        dt += time.perf_counter() - t0
        reps += 1
    dense, _ = flops_of(ws, out["blocks"])
    return dense * reps / dt / 1e12, dt, reps, dense


def traffic_of(workload: str):
    """HBM bytes per attention launch from the committed counter summary of this workload
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size), or None when there is
    none or it was taken on a different version of the kernel source."""
    got = read_traffic(os.path.join(ROOT, "profiles", f"attn_bf16_{workload}_hbm_traffic.md"))
    return None if got is None else got[0]


_HIP = None
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


def hip_runtime():
    """The HIP runtime this process already runs on (the one torch and the library share),
    for the event flag torch does not expose."""
    global _HIP
    if _HIP is None:
        with open("/proc/self/maps") as f:
            paths = sorted({line.split()[-1] for line in f if "libamdhip64.so" in line})
        if len(paths) != 1:
            raise RuntimeError(f"expected one loaded HIP runtime, found {paths}")
        hip = ctypes.CDLL(paths[0])
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = hip
    return _HIP


class TimingEvent:
    """A timing event recorded without the system-scope fence, so recording it writes back
    and invalidates no cache between the kernels it separates (torch's events do, which
    makes the kernel after each one start with cold caches). Read only after a device
    synchronisation."""

    def __init__(self):
        self.h = ctypes.c_void_p()
        self._ok(hip_runtime().hipEventCreateWithFlags(ctypes.byref(self.h), HIP_EVENT_DISABLE_SYSTEM_FENCE))

    @staticmethod
    def _ok(err):
        if err != 0:
            raise RuntimeError(f"HIP event call failed with error {err}")

    def record(self, stream):
        self._ok(hip_runtime().hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream)))

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end`."""
        ms = ctypes.c_float()
        self._ok(hip_runtime().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h))
        return ms.value

    def __del__(self):
        if self.h and _HIP is not None:
            _HIP.hipEventDestroy(self.h)


def hold_stream(ms: float = 50.0):
    """Enqueues a spin kernel of about `ms` milliseconds on the current stream, so that the
    host can queue the next calls before the GPU reaches them."""
    torch.cuda._sleep(int(ms * 1e-3 * 2.0e9))


def mfma_ceiling(n_wg: int = 512, iters: int = 20000, reps: int = 3):
    """Measured dense bf16 matrix-core rate (register-only MFMA chains, 2 waves per SIMD on
    every CU) and the shader clock under that load; best of `reps` launches."""
    dev = torch.device("cuda")
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    flops = n_wg * 16.0 * iters * 32768.0
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lf.lf_probe_mfma_bf16(n_wg, iters, sink, clocks)
        e1.record()
        torch.cuda.synchronize()
        tf = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
        cyc, ticks = clocks.tolist()
        ghz = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else float("nan")
        if best is None or tf > best[0]:
            best = (tf, ghz)
    return {"tflops": round(best[0], 1), "clock_ghz": round(best[1], 3),
            "what": f"register-only v_mfma_f32_32x32x16_bf16 chains, {n_wg} x 4 waves, {iters} x 4 MFMAs per wave"}


def hbm_ceiling(gib: int = 2, reps: int = 3):
    """Measured HBM read rate: a plain streaming read of a `gib` GiB buffer (8x the 256 MB
    Infinity Cache, so it streams from HBM) at several launch sizes, best launch of each,
    best size reported."""
    dev = torch.device("cuda")
    x = torch.ones((gib << 30) // 4, dtype=torch.float32, device=dev)
    sizes = (2048, 4096, 8192, 16384)
    sink = torch.empty(max(sizes) * 256, dtype=torch.float32, device=dev)
    by_size = {}
    for n_wg in sizes:
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lf.lf_probe_hbm_read(x, n_wg, sink)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        by_size[n_wg] = round(best, 1)
    # read + write: a plain device copy of half the buffer (torch's copy kernel), both
    # directions' bytes counted -- the ceiling for kernels that write as much as they read
    half = x.numel() // 2
    src_, dst_ = x[:half], x[half:2 * half]
    copy_best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst_.copy_(src_)
        e1.record()
        torch.cuda.synchronize()
        copy_best = max(copy_best, 2 * half * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x, src_, dst_
    torch.cuda.empty_cache()
    n_best = max(by_size, key=by_size.get)
    return {"gbs": by_size[n_best], "by_workgroups": by_size, "copy_gbs": round(copy_best, 1),
            "what": f"plain streaming read of {gib} GiB, 256-thread workgroups, 16-byte loads, best of {reps} "
                    f"per launch size; copy_gbs: a device copy of {gib / 2:g} GiB, read and written bytes counted"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def one_core_baseline(w, k_b: int, min_s: float):
    """The CPU oracle on one head with BLAS limited to one thread (a single-core figure)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        tflops, sec, reps, dense = run_cpu_baseline(w, k_b, 1, min_s / 2)
    return {"value": tflops, "unit": "TFLOP/s", "cores": 1,
            "sample": f"{w.name}, head 0: pool + select + attention, {reps} repeats in {sec:.1f} s"}


def gpu_state_under_load(step, seconds: float = 1.5):
    """Shader and memory clocks (and socket power where the driver reports it) from
    rocm-smi, read while steps keep the GPU busy; None if the tool is unavailable."""
    import re
    import subprocess
    import threading
    res = {}

    def query():
        for exe in ("/opt/rocm/bin/rocm-smi", "rocm-smi"):
            try:
                r = subprocess.run([exe, "-P", "-c", "--json"], capture_output=True, text=True, timeout=20)
                card = next(iter(json.loads(r.stdout).values()))
            except Exception:
                continue
            for key, val in card.items():
                num = re.findall(r"[\d.]+", str(val))
                if not num:
                    continue
                kl = key.lower()
                if "power" in kl and "(w)" in kl:
                    res["power_w"] = float(num[0])
                elif "sclk clock speed" in kl:
                    res["sclk_mhz"] = float(num[0])
                elif "mclk clock speed" in kl:
                    res["mclk_mhz"] = float(num[0])
            return

    t = threading.Thread(target=query)
    t0 = time.perf_counter()
    t.start()
    i = 0
    while t.is_alive() or time.perf_counter() - t0 < seconds:
        step(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    t.join()
    torch.cuda.synchronize()
    return res or None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 500; 20 sweeps for the sweep workload)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 200, enough for the clocks to settle; 3 sweeps)")
    ap.add_argument("--workload", default="480p_chunk7of7", choices=sorted(synth.WORKLOADS) + [synth.SWEEP.name])
    ap.add_argument("--layers", type=int, default=0,
                    help="independent input sets cycled per step (0: enough to exceed 512 MB)")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads in the CPU-oracle sample (0: skip)")
    ap.add_argument("--cpu-min-s", type=float, default=10.0, help="repeat the CPU sample for at least this long")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparison legs (single-level selection, prologue, schedules, MFMA ceiling), "
                         "e.g. so a profiler trace holds only the hot path's dispatches")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the HSA path runs on one GPU and has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sweep = args.workload == synth.SWEEP.name
    if args.steps is None:
        args.steps = 20 if sweep else 500
    if args.warmup is None:
        args.warmup = 3 if sweep else 200
    if args.workload == synth.SWEEP.name:
        return bench_sweep(args)
    dev = torch.device("cuda")
    w = synth.WORKLOADS[args.workload]
    g = lf.Geom(w.B, w.H, w.d, w.tpf, w.bs)
    nb = lf.n_bpf(g)
    dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    # a0 on the host: CAG schedule and block budget
    s_sched, beta = lf.lf_cag_schedule(w.n_chunks, w.T, w.s_base, w.s_target, chunk_flops(w))
    W_f = len(w.forced) + min(w.k_f, len(w.mem))
    k_b = w.k_b if w.k_b is not None else lf.lf_block_budget(s_sched[w.chunk_index - 1],
                                                             w.n_kframes * nb, W_f, nb)
    plan = ChunkPlan(g, w.n_qframes, w.n_kframes, list(w.mem), list(w.forced), w.k_f, k_b, w.scale)

    # inputs: layer 0 from the seeded host generator, the others drawn on the device
    esz = 2 if w.dtype == "bf16" else 4
    set_bytes = w.B * w.H * (2 * w.lq + 2 * w.lk) * w.d * esz          # q, o, k, v
    if args.layers <= 0:
        args.layers = max(2, -(-(512 << 20) // set_bytes))
    print(f"[bench] generating {args.layers} input sets for {w.name}", file=sys.stderr, flush=True)
    x = synth.make(w)
    sets = [(x.q.to(dev), x.k.to(dev), x.v.to(dev))]
    pools = [w.q_pool if w.q_pool is not None else x.planted]
    for li in range(1, args.layers):
        sets.append(synth.make_on_device(w.B, w.H, w.n_qframes, w.n_kframes, w.tpf, w.bs, w.d, w.dtype,
                                         w.seed + 100 * li, dev, pools))
    wss = [Workspace(plan, dtype, dev) for _ in sets]
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    # steady state: the history frames' pooled keys sit in a per-layer cache (filled here,
    # before timing); a step pools the queries and the chunk's own key frames only
    f0 = new_frames(plan)
    n_lag = min(w.n_qframes, f0)
    caches = [PooledKeyCache(g, w.n_kframes, dev) for _ in sets]
    for c, (_, k, _) in zip(caches, sets):
        lf.lf_pool(k[:, :, :f0 * w.tpf], g, f0, blk_out=c.blk(0, f0), frm_out=c.frm(0, f0))

    def step(i, ev=None, cached=False, upto=3):
        lf.lf_cag_schedule(w.n_chunks, w.T, w.s_base, w.s_target, chunk_flops(w))
        ws = wss[i % len(sets)]
        q, k, v = sets[i % len(sets)]
        if cached:
            c = caches[i % len(sets)]
            calls = [lambda: pool_cached(ws, c, q, k), lambda: select_cached(ws, c), lambda: attend(ws, q, k, v)]
        else:
            calls = [lambda: pool(ws, q, k), lambda: select(ws), lambda: attend(ws, q, k, v)]
        calls = calls[:upto]
        for j, c_ in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            c_()
        if ev is not None:
            ev[len(calls)].record(stream)

    def timed(cached):
        """(ms per step by wall clock, per-call mean us, per-call median us)."""
        print(f"[bench] warmup {args.warmup}" + (" (steady state)" if cached else ""), file=sys.stderr, flush=True)
        for i in range(args.warmup):
            step(i, cached=cached)
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} steps" + (" (steady state)" if cached else ""), file=sys.stderr,
              flush=True)
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, cached=cached)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # per-call times: the same steps again with events between calls, all enqueued while
        # a spin kernel holds the stream, so host launch gaps do not show up as kernel time
        n_ev = min(args.steps, 100)
        evs = [[TimingEvent() for _ in range(len(KERNELS) + 1)] for _ in range(n_ev)]
        hold_stream()
        for i in range(n_ev):
            step(i, evs[i], cached=cached)
        torch.cuda.synchronize()
        per = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(len(KERNELS))]
                        for i in range(n_ev)]) * 1e3                      # us
        return wall * 1e3 / args.steps, per.mean(axis=0), np.median(per, axis=0), np.percentile(per, [10, 90], axis=0)

    def stage_times_in_loop(n, cached=False):
        """Each stage's mean time inside the step loop: n steps timed by HIP events around
        the whole loop on the launch stream (queued behind a spin kernel, so host launch
        gaps do not count) with the first 1, 2 and 3 stages, differenced. Consecutive
        kernels of a step run back to back, so each difference is that stage's launches'
        own time; event pairs around single launches add each marker's dispatch gap (about
        5 us) to every interval. Returns (per-stage us, full-step us)."""
        per = []
        for upto in (1, 2, 3):
            torch.cuda.synchronize()
            hold_stream(max(50.0, 0.25 * n))
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record(stream)
            for i in range(n):
                step(i, cached=cached, upto=upto)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / n)
        return np.array([per[0], per[1] - per[0], per[2] - per[1]]), per[2]

    ms_per_step, mean_us, med_us, pct_us = timed(False)
    ss_ms, ss_mean, ss_med, _ = timed(True)
    loop_us, loop_step_us = stage_times_in_loop(args.steps)
    ss_loop_us, ss_loop_step_us = stage_times_in_loop(args.steps, cached=True)
    attn_loop_us = float(loop_us[2])
    state = gpu_state_under_load(lambda i: step(i)) if not args.no_extras else None

    extras = not args.no_extras
    one_level = compare_one_level(args, w, g, plan, wss[0], sets[0]) if extras else None
    scaling = select_scaling(args, w, g) if extras and w.d in (64, 128) else None
    prologue = compare_prologue(args, w, g, plan, sets[0]) if extras else None
    ceiling = mfma_ceiling() if extras else None
    hbm = hbm_ceiling() if extras else None
    blocks = wss[0].blocks.cpu().numpy()
    f_dense, f_active = flops_of(w, blocks)
    # active FLOPs per attention launch of the loop (the input sets' lists differ slightly)
    f_sets = [flops_of(w, ws.blocks.cpu().numpy())[1] for ws in wss]
    f_active_loop = float(np.mean([f_sets[i % len(sets)] for i in range(args.steps)]))
    # algorithmic HBM bytes of one attention launch: Q read, O written, each K/V token of the
    # prefix read once (an upper bound of the unique bytes: a key block no row lists is not
    # read)
    esz = 2 if w.dtype == "bf16" else 4
    attn_bytes = w.B * w.H * (2 * w.lq + 2 * w.lk) * w.d * esz
    t_attn = attn_loop_us * 1e-6
    t_path = loop_step_us * 1e-6
    attn_tflops = f_active_loop / t_attn / 1e12
    value = f_dense / (ms_per_step * 1e-3) / 1e12
    sel_pct = 100.0 * loop_us[1] / loop_us[2]
    pool_gbs = {"pool": (pool_bytes(w, w.n_qframes, False) + pool_bytes(w, w.n_kframes, True))
                        / (loop_us[0] * 1e-6) / 1e9}
    n_rows = w.B * w.H * plan.n_qb
    # algorithmic HBM bytes of the selection launch: q~ rows, each head's frame means and
    # block means once (they stay in L2 across the head's rows), T_r and list writes
    sel_bytes = (n_rows * (w.d * 4 + plan.W_f * 4 + plan.W_b * 4)
                 + w.B * w.H * w.n_kframes * (nb + 1) * w.d * 4)
    sel_gbs = {"select": sel_bytes / (loop_us[1] * 1e-6) / 1e9}
    steady = {
        "what": (f"history pooled keys ({f0} frames) from a per-layer cache filled before timing; a step pools "
                 f"the queries and the chunk's own {w.n_kframes - f0} key frames (block means) with the "
                 f"previous chunk's {n_lag} frame means in one launch, selects over the cache and attends"),
        "value": f_dense / (ss_ms * 1e-3) / 1e12,
        "ms_per_step": ss_ms,
        "kernel_us_in_loop": dict(zip(KERNELS, [round(float(x), 2) for x in ss_loop_us])),
        "kernel_us_event_pairs_mean": dict(zip(KERNELS, [round(float(x), 2) for x in ss_mean])),
        "pool_select_pct_of_attn": 100.0 * ss_loop_us[:2].sum() / ss_loop_us[2],
        "dense_equiv_tflops_kernel_sum": f_dense / (ss_loop_step_us * 1e-6) / 1e12,
        "pool_gbs": round((pool_bytes(w, w.n_qframes, False) + pool_bytes(w, w.n_kframes - f0, False)
                           + lag_bytes(w, n_lag)) / (ss_loop_us[0] * 1e-6) / 1e9, 1),
    }

    cpu = None
    if args.cpu_heads > 0:
        print(f"[bench] CPU oracle on {args.cpu_heads} heads", file=sys.stderr, flush=True)
        cpu_tflops, cpu_s, reps, cpu_dense = run_cpu_baseline(w, k_b, args.cpu_heads, args.cpu_min_s)
        cpu = {"value": cpu_tflops, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"{w.name}, heads 0..{args.cpu_heads - 1} of {w.H}: pool + select + attention "
                         f"in numpy fp64, {reps} repeats ({cpu_dense:.3e} dense-equiv FLOP each) "
                         f"in {cpu_s:.1f} s",
               "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
               "one_core": one_core_baseline(w, k_b, args.cpu_min_s)}

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded planted-relevance Q/K/V; no model weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "tokens_per_frame": w.tpf,
                   "block_size": w.bs, "query_tokens": w.lq, "key_tokens": w.lk, "W_f": plan.W_f,
                   "W_b": plan.W_b, "k_f": w.k_f, "k_b": k_b, "cag_s_i": s_sched[w.chunk_index - 1],
                   "cag_beta": beta, "input_sets": len(sets)},
        "mfma_pct_peak_active": 100.0 * attn_tflops / PEAK_BF16_TFLOPS,
        "select_overhead_pct": sel_pct,
        "pool_select_pct_of_attn": 100.0 * (loop_us[:2].sum()) / loop_us[2],
        "dense_equiv_tflops_attn_only": f_dense / t_attn / 1e12,
        "dense_equiv_tflops_kernel_sum": f_dense / t_path / 1e12,
        "flops": {"dense_equiv": f_dense, "active": f_active, "block_density": f_active / f_dense},
        "kernel_us_in_loop": dict(zip(KERNELS, [round(float(x), 2) for x in loop_us])),
        "kernel_us_in_loop_what": (f"{args.steps} steps with the first 1, 2, 3 stages, HIP events around each "
                                   f"loop on the launch stream, differenced"),
        "kernel_us_event_pairs_mean": dict(zip(KERNELS, [round(float(x), 2) for x in mean_us])),
        "kernel_us_event_pairs_p10_p90": {k: [round(float(pct_us[0][i]), 2), round(float(pct_us[1][i]), 2)]
                                          for i, k in enumerate(KERNELS)},
        "hbm_gbs": {**{k: round(v, 1) for k, v in pool_gbs.items()}, **{k: round(v, 1) for k, v in sel_gbs.items()}},
        "hbm_ceiling": ({**hbm, "pool_frac": round(pool_gbs["pool"] / hbm["gbs"], 3),
                         "steady_pool_frac": round(steady["pool_gbs"] / hbm["gbs"], 3),
                         "prologue_frac": (round(prologue["hbm_gbs"] / hbm["gbs"], 3) if prologue else None),
                         "prologue_frac_of_copy": (round(prologue["hbm_gbs"] / hbm["copy_gbs"], 3)
                                                   if prologue else None)}
                        if hbm else None),
        "steady_state": steady,
        "one_level": one_level,
        "select_scaling": scaling,
        "prologue": prologue,
        "roofline": {"kernel": "attn_bf16_kernel<128>" if w.d == 128 else "attn_bf16_kernel<64>",
                     "bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic_of(w.name),
                     "algorithmic_bytes_upper": attn_bytes,
                     "traffic_over_algorithmic": (round(traffic_of(w.name) / attn_bytes, 3)
                                                  if traffic_of(w.name) else None),
                     "launch_us": round(attn_loop_us, 2), "active_flops_per_launch": f_active_loop,
                     "timing": (f"{args.steps} steps timed by HIP events around the loop on the launch "
                                f"stream, with and without the attention launch (difference)")},
        "mfma_ceiling": ({**ceiling, "attn_frac_of_ceiling": attn_tflops / ceiling["tflops"]} if ceiling else None),
        "gpu_state": state,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


STAGES = ["pool", "select", "attn"]


def bench_sweep(args):
    """The full Chunk-Aware Growth schedule of one denoising step of a 5-s 480p clip:
    30 layers x 7 chunks (chunk 1 dense). One step = the whole schedule; inputs of all 30
    layers (independent, drawn on the device) are resident before timing."""
    s = synth.SWEEP
    dev = torch.device("cuda")
    g = lf.Geom(s.B, s.H, s.d, s.tpf, s.bs)
    sp = plan_sweep(g, s.n_chunks, s.frames_per_chunk, s.k_f, s.T, s.s_base, s.s_target, s.d ** -0.5)
    sw = SweepWorkspace(sp, torch.bfloat16, dev)
    pools = [s.chunk(i).q_pool for i in range(1, s.n_chunks + 1)]
    n_layers = s.n_layers
    print(f"[bench] generating {n_layers} layers for {s.name}", file=sys.stderr, flush=True)
    layers = [synth.make_on_device(s.B, s.H, s.n_frames, s.n_frames, s.tpf, s.bs, s.d, s.dtype, s.seed(li),
                                   dev, pools) for li in range(n_layers)]
    o = torch.empty_like(layers[0][0])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # untimed pass: every (layer, chunk) block list, for the active FLOP count
    f_dense, f_active = 0.0, 0.0
    for li, (q, k, v) in enumerate(layers):
        sweep_layer(sw, q, k, v, o)
        torch.cuda.synchronize()
        for i in range(1, s.n_chunks + 1):
            w = s.chunk(i, li)
            blocks = (sw.full[i] if sp.dense(i) else sw.chunks[i - 1].blocks).cpu().numpy()
            fd, fa = flops_of(w, blocks)
            f_dense += fd
            f_active += fa

    # steady state: one pooled-key cache per layer; each chunk pools only its own key frames
    caches = [PooledKeyCache(g, sp.n_frames, dev) for _ in layers]

    def run(events=None, cached=False, stages=3):
        for li, (q, k, v) in enumerate(layers):
            mark = None
            if events is not None:
                def mark(i, stage):
                    ev = TimingEvent()
                    ev.record(stream)
                    events.append((i, stage, ev))
            # the last chunk's frame means are read by no chunk of the sweep: not formed
            sweep_layer(sw, q, k, v, o, mark, cache=caches[li] if cached else None, complete=False, stages=stages)

    def stages_in_loop(n, cached=False):
        """Per-sweep stage times inside the sweep loop: n sweeps timed by HIP events around
        the loop (queued behind a spin kernel) with the first 1, 2 and 3 stages of every
        chunk, differenced (as for one chunk)."""
        per = []
        for upto in (1, 2, 3):
            torch.cuda.synchronize()
            hold_stream(60.0 * n)
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record(stream)
            for _ in range(n):
                run(cached=cached, stages=upto)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / n)
        return {"pool": per[0], "select": per[1] - per[0], "attn": per[2] - per[1]}, per[2]

    def timed(cached):
        """(ms per sweep by wall clock, per-stage us, per-chunk us of one evented sweep)."""
        tag = " (steady state)" if cached else ""
        print(f"[bench] warmup {args.warmup}{tag}", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            run(cached=cached)
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} sweeps{tag}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run(cached=cached)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # per-stage breakdown from one extra evented sweep, enqueued behind a spin kernel so
        # that host launch gaps do not count as stage time
        events = []
        hold_stream(400.0)
        run(events, cached=cached)
        torch.cuda.synchronize()
        stage_us = {st: 0.0 for st in STAGES}
        chunk_us = [0.0] * s.n_chunks
        for (i, st, ev), (_, _, nxt) in zip(events, events[1:]):
            if st == "end":
                continue
            dt = ev.elapsed_time(nxt) * 1e3
            stage_us[st] += dt
            chunk_us[i - 1] += dt
        return wall * 1e3 / args.steps, stage_us, chunk_us

    ms_per_step, stage_us, chunk_us = timed(False)
    ss_ms, ss_stage, ss_chunk = timed(True)
    n_loop = min(args.steps, 5)
    loop_us, loop_sweep_us = stages_in_loop(n_loop)
    ss_loop_us, _ = stages_in_loop(n_loop, cached=True)
    compare = compare_schedules(args, s, g, sp, sw, layers, o) if not args.no_extras else None
    ceiling = mfma_ceiling() if not args.no_extras else None
    t_attn = loop_us["attn"] * 1e-6
    attn_tflops = f_active / t_attn / 1e12
    cpu = None
    if args.cpu_heads > 0:
        w7 = s.chunk(s.n_chunks, 0)
        k_b7 = sp.chunks[-1].k_b
        print(f"[bench] CPU oracle on {args.cpu_heads} heads of {w7.name}", file=sys.stderr, flush=True)
        cpu_tflops, cpu_s, reps, cpu_dense = run_cpu_baseline(w7, k_b7, args.cpu_heads, args.cpu_min_s)
        cpu = {"value": cpu_tflops, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"{w7.name} (chunk 7, layer 0), heads 0..{args.cpu_heads - 1}: pool + select + "
                         f"attention in numpy fp64, {reps} repeats ({cpu_dense:.3e} dense-equiv FLOP each) "
                         f"in {cpu_s:.1f} s",
               "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    line = {
        "metric": METRIC,
        "value": f_dense / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded planted-relevance Q/K/V drawn on the device; no model weights)",
        "config": {"workload": s.name, "layers": n_layers, "chunks": s.n_chunks, "H": s.H, "d": s.d,
                   "tokens_per_frame": s.tpf, "block_size": s.bs, "k_f": s.k_f,
                   "cag_s": [round(x, 6) for x in sp.s], "cag_beta": sp.beta,
                   "k_b": [c.k_b for c in sp.chunks], "W_b": [c.W_b for c in sp.chunks]},
        "mfma_pct_peak_active": 100.0 * attn_tflops / PEAK_BF16_TFLOPS,
        "select_overhead_pct": 100.0 * loop_us["select"] / loop_us["attn"],
        "pool_select_pct_of_attn": 100.0 * (loop_us["pool"] + loop_us["select"]) / loop_us["attn"],
        "flops": {"dense_equiv": f_dense, "active": f_active, "block_density": f_active / f_dense},
        "stage_us_per_sweep_in_loop": {k: round(v, 1) for k, v in loop_us.items()},
        "stage_us_per_sweep_in_loop_what": (f"{n_loop} sweeps with the first 1, 2, 3 stages of every chunk, HIP "
                                            f"events around each loop on the launch stream, differenced"),
        "stage_us_per_sweep_event_pairs": {k: round(v, 1) for k, v in stage_us.items()},
        "chunk_us_per_sweep_event_pairs": [round(x, 1) for x in chunk_us],
        "steady_state": {
            "what": "per-layer pooled-key caches: each chunk pools its queries and only its own 3 key frames "
                    "(chunk 1 its keys only) and selects over the cached prefix",
            "value": f_dense / (ss_ms * 1e-3) / 1e12,
            "ms_per_step": ss_ms,
            "stage_us_per_sweep_in_loop": {k: round(v, 1) for k, v in ss_loop_us.items()},
            "stage_us_per_sweep_event_pairs": {k: round(v, 1) for k, v in ss_stage.items()},
            "chunk_us_per_sweep_event_pairs": [round(x, 1) for x in ss_chunk],
            "pool_select_pct_of_attn": 100.0 * (ss_loop_us["pool"] + ss_loop_us["select"]) / ss_loop_us["attn"],
        },
        "roofline": {"kernel": "attn_bf16_kernel<128>", "bound": "mfma", "achieved": attn_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic_of(s.name), "launch_us": round(loop_us["attn"] / (n_layers * s.n_chunks), 2),
                     "timing": "mean per attention launch of the sweep (dense chunk 1 and sparse chunks 2-7), "
                               "from the in-loop attention time per sweep"},
        "mfma_ceiling": ({**ceiling, "attn_frac_of_ceiling": attn_tflops / ceiling["tflops"]} if ceiling else None),
        "schedules": compare,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def per_call(fn, n):
    """Mean device time of one of n back-to-back calls of fn (queued behind a spin kernel)."""
    hold_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def compare_prologue(args, w, g, plan, qkv):
    """The query/key prologue (RMSNorm + rotary embedding) fused with pooling, on the
    chunk's queries and its own key frames (the tensors a step produces before attention
    in steady state): one launch (lf_qk_prologue_step: queries, keys into a KV cache view,
    block means, the previous chunk's frame means), its HBM rate, the two-call form it
    replaces (one lf_qk_prologue per tensor) and the separate pooling pass over their
    outputs that the fusion removes."""
    q, k, _ = qkv
    dev = q.device
    nb = lf.n_bpf(g)
    f0, tpf, nq = new_frames(plan), w.tpf, w.n_qframes
    n_lag = min(nq, f0)
    lat_w = 52 if tpf == 1560 else int(round(tpf ** 0.5))
    kc = k[:, :, f0 * tpf:].contiguous()                  # the chunk's new keys, packed as projected
    gamma = torch.from_numpy((1.0 + 0.1 * np.random.default_rng(77).standard_normal(w.d)).astype(np.float32)).to(dev)
    qo, ko = torch.empty_like(q), torch.empty((w.B, w.H, nq * tpf, w.d), dtype=q.dtype, device=dev)
    qb = torch.empty((w.B, w.H, nq * nb, w.d), dtype=torch.float32, device=dev)
    kb = torch.empty_like(qb)
    kf = torch.empty((w.B, w.H, nq, w.d), dtype=torch.float32, device=dev)
    cache = PooledKeyCache(g, w.n_kframes, dev)
    lf.lf_pool(k[:, :, :f0 * tpf], g, f0, blk_out=cache.blk(0, f0), frm_out=cache.frm(0, f0))

    def one_launch():
        lf.lf_qk_prologue_step(q, kc, gamma, gamma, g, nq, f0, lat_w, f0, f0 - n_lag, n_lag, ko, cache.k_blk,
                               cache.k_frm, q_out=qo, q_blk=qb)

    def two_calls():
        lf.lf_qk_prologue(q, gamma, g, nq, f0, lat_w, x_out=qo, blk_out=qb, with_frames=False)
        lf.lf_qk_prologue(kc, gamma, g, nq, f0, lat_w, x_out=ko, blk_out=kb, frm_out=kf)

    n = max(5, min(args.steps, 50))
    t_step = per_call(one_launch, n)
    t_two = per_call(two_calls, n)
    t_pool = per_call(lambda: lf.lf_pool_qk(qo, ko, g, nq, nq, qb, kb, kf), n)
    esz = 2 if w.dtype == "bf16" else 4
    tokens = 2 * w.B * w.H * nq * tpf
    moved = tokens * w.d * esz * 2 + 2 * w.B * w.H * nq * nb * w.d * 4 + lag_bytes(w, n_lag)
    moved_two = tokens * w.d * esz * 2 + 2 * w.B * w.H * nq * nb * w.d * 4 + w.B * w.H * nq * w.d * 4
    return {"what": (f"queries and the chunk's own {nq} key frames: RMSNorm + rotary + block means, with the "
                     f"previous chunk's {n_lag} frame means, in one launch"),
            "lat_w": lat_w, "fused_us": round(t_step, 2), "hbm_gbs": round(moved / (t_step * 1e-6) / 1e9, 1),
            "algorithmic_bytes": moved,
            "two_calls_us": round(t_two, 2), "two_calls_hbm_gbs": round(moved_two / (t_two * 1e-6) / 1e9, 1),
            "separate_pool_pass_us": round(t_pool, 2)}


def select_scaling(args, w, g):
    """The fused selection call over growing histories at this layer's geometry (the
    chunk's query blocks; k_f and k_b as configured; 3 current frames and a sink frame
    always kept, every other frame in M): per-call time for several key-frame counts.
    Attention over the resulting lists has a fixed width (W_b), so it stays constant while
    the frame stage grows with |M|. Pooled tensors are random fp32 drawn on the device
    (timing only)."""
    dev = torch.device("cuda")
    nb = lf.n_bpf(g)
    n_qb = w.n_qframes * nb
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    q_blk = torch.randn((w.B, w.H, n_qb, w.d), generator=gen, device=dev)
    res = {}
    for n in (21, 69, 300, 1200, 4096):
        k_frm = torch.randn((w.B, w.H, n, w.d), generator=gen, device=dev)
        k_blk = torch.randn((w.B, w.H, n * nb, w.d), generator=gen, device=dev)
        forced = [0, n - 3, n - 2, n - 1]
        mem = list(range(1, n - 3))
        k_f, k_b = w.k_f, min(w.k_b or 8, nb)
        fo, bo = lf.lf_select(q_blk, k_frm, k_blk, g, n_qb, n, mem, forced, k_f, k_b)
        reps = max(5, min(args.steps, 30))
        t = per_call(lambda: lf.lf_select(q_blk, k_frm, k_blk, g, n_qb, n, mem, forced, k_f, k_b, fo, bo), reps)
        res[str(n)] = round(t, 2)
        del k_frm, k_blk
    torch.cuda.empty_cache()
    return {"what": (f"lf_select at {w.name}'s geometry ({w.B * w.H * n_qb} rows), |M| = n - 4, k_f = {w.k_f}: "
                     f"us per call by key frames n"), "us_by_key_frames": res}


def compare_one_level(args, w, g, plan, ws, qkv):
    """HSA against single-level block top-K at the same budget (K = W_b) on one input set:
    selection time per call, attention time over each list and over the full lists
    (dense attention, the context ratio against sparse), and the relative L2 distance of
    each output from dense attention (a fidelity measure on synthetic inputs). The calls
    repeat on one input set, so these are warm (cache-resident) times."""
    q, k, v = qkv
    dev = q.device
    nb = lf.n_bpf(g)
    K = plan.W_b
    lists_1d = torch.empty((w.B, w.H, plan.n_qb, K), dtype=torch.int32, device=dev)
    n_kb = w.n_kframes * nb
    full = torch.arange(n_kb, dtype=torch.int32, device=dev).expand(w.B, w.H, plan.n_qb, n_kb).contiguous()
    hsa_chunk(ws, q, k, v)
    select_1d(ws, lists_1d)
    torch.cuda.synchronize()

    n = max(5, min(args.steps, 50))
    o_h, o_1, o_d = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    t_sel_hsa = per_call(lambda: select(ws), n)
    t_sel_1d = per_call(lambda: select_1d(ws, lists_1d), n)
    t_att_hsa = per_call(lambda: lf.lf_sparse_attn(q, k, v, g, w.n_qframes, w.n_kframes, ws.blocks, w.scale,
                                                   out=o_h), n)
    t_att_1d = per_call(lambda: lf.lf_sparse_attn(q, k, v, g, w.n_qframes, w.n_kframes, lists_1d, w.scale,
                                                  out=o_1), n)
    t_att_dense = per_call(lambda: lf.lf_sparse_attn(q, k, v, g, w.n_qframes, w.n_kframes, full, w.scale,
                                                     out=o_d), max(3, n // 5))
    torch.cuda.synchronize()
    ref = o_d.float()
    rel = lambda o: float((o.float() - ref).norm() / ref.norm())
    hb, ob = ws.blocks.cpu().numpy(), lists_1d.cpu().numpy()
    shared = np.mean([len(np.intersect1d(a, b)) / K for a, b in zip(hb.reshape(-1, K), ob.reshape(-1, K))])
    return {"K": K, "select_us": {"hsa": round(t_sel_hsa, 2), "one_level": round(t_sel_1d, 2)},
            "attn_us": {"hsa": round(t_att_hsa, 2), "one_level": round(t_att_1d, 2), "dense": round(t_att_dense, 2)},
            "dense_over_hsa_attn": round(t_att_dense / t_att_hsa, 3),
            "rel_l2_vs_dense": {"hsa": round(rel(o_h), 5), "one_level": round(rel(o_1), 5)},
            "shared_block_fraction": round(float(shared), 4)}


def compare_schedules(args, s, g, sp_cag, sw_cag, layers, o):
    """CAG against the uniform allocation under the same FLOP budget, and both against
    dense attention: wall time per sweep (all layers) and, on two layers, each chunk's
    relative L2 distance of the attention output from the dense output (a per-chunk
    fidelity measure on synthetic inputs; the pages compare the schedules by the quality
    of generated video, which needs a trained model)."""
    dev = o.device
    sp_uni = plan_sweep(g, s.n_chunks, s.frames_per_chunk, s.k_f, s.T, s.s_base, s.s_target, s.d ** -0.5,
                        schedule="uniform")
    sw_uni = SweepWorkspace(sp_uni, torch.bfloat16, dev)
    tpf, fpc = s.tpf, s.frames_per_chunk
    full = []
    for p in sp_cag.chunks:
        n_kb = p.n_kframes * p.n_bpf
        full.append(torch.arange(n_kb, dtype=torch.int32, device=dev).expand(s.B, s.H, p.n_qb, n_kb).contiguous())

    def dense_layer(q, k, v, out):
        for i, p in enumerate(sp_cag.chunks, 1):
            a, b = (i - 1) * fpc * tpf, i * fpc * tpf
            lf.lf_sparse_attn(q[:, :, a:b], k[:, :, :b], v[:, :, :b], p.geom, p.n_qframes, p.n_kframes, full[i - 1],
                              p.scale, out=out[:, :, a:b])

    def wall(fn, reps):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    reps = max(1, min(args.steps, 3))
    print("[bench] schedule comparison (uniform, dense)", file=sys.stderr, flush=True)
    t_uni = wall(lambda: [sweep_layer(sw_uni, q, k, v, o) for q, k, v in layers], reps)
    t_cag = wall(lambda: [sweep_layer(sw_cag, q, k, v, o) for q, k, v in layers], reps)
    t_dense = wall(lambda: [dense_layer(q, k, v, o) for q, k, v in layers], reps)
    fid = {"cag": [], "uniform": []}
    for li in (0, len(layers) - 1):
        q, k, v = layers[li]
        od, oc, ou = torch.empty_like(o), torch.empty_like(o), torch.empty_like(o)
        dense_layer(q, k, v, od)
        sweep_layer(sw_cag, q, k, v, oc)
        sweep_layer(sw_uni, q, k, v, ou)
        torch.cuda.synchronize()
        for name, os_ in (("cag", oc), ("uniform", ou)):
            row = []
            for i in range(1, s.n_chunks + 1):
                a, b = (i - 1) * fpc * tpf, i * fpc * tpf
                ref = od[:, :, a:b].float()
                row.append(round(float((os_[:, :, a:b].float() - ref).norm() / ref.norm()), 5))
            fid[name].append({"layer": li, "rel_l2_vs_dense_by_chunk": row})
    return {
        "budget_s_target": s.s_target,
        "cag": {"s": [round(x, 6) for x in sp_cag.s], "k_b": [c.k_b for c in sp_cag.chunks],
                "ms_per_sweep": t_cag, "fidelity": fid["cag"]},
        "uniform": {"s": [round(x, 6) for x in sp_uni.s], "k_b": [c.k_b for c in sp_uni.chunks],
                    "ms_per_sweep": t_uni, "fidelity": fid["uniform"]},
        "dense": {"ms_per_sweep": t_dense, "speedup_cag": t_dense / t_cag, "speedup_uniform": t_dense / t_uni},
    }


if __name__ == "__main__":
    main()
