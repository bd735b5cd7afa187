"""Benchmark: streaming-chunk attention at 1344x768 on one MI355X.

A step is one chunk through the whole hot path: rotary tables of the chunk's
position template, in-place pack of the dynamic K/V region (history and the
current chunk; the static prompt/reference prefix is packed once, before
timing), and the forward pass. Inputs are resident in HBM before timing.

Prints ONE JSON line. ``value`` is attention TFLOP/s over the whole step
(4*Nq*Nk*d*H flops per chunk / step time); ``ms_per_step`` is ms per chunk.
``roofline`` prices the forward (the dominant kernel: one launch at 1344x768,
whose 1280 units fill five rounds; where a stream-K tail applies, also its
tail launch and merge) from HIP events around each forward in the timed
region; ``cpu_baseline``
times the fp64 oracle on a bounded sample of the same workload on the host
cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + ms/chunk at 1344x768 (12096 q x 28480 kv, 40 heads)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector peak (published)
HBM_PEAK_BPS = 8.0e12       # MI355X HBM3E bandwidth (published)
FWD_SOURCE = os.path.join(ROOT, "streaming_video_diffusion_amd", "csrc", "fwd_bf16.hip")
# HBM traffic of one forward at 1344x768, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (KiB per forward; profiles/fwd_bf16_1344x768_hbm_traffic.txt),
# each scaled by what the same counter reads for a plain device copy of known
# size (FETCH_SIZE counts 0.5x the bytes read, WRITE_SIZE 1.0x the bytes
# written). Valid only for the forward source these counters were taken on
# (None: not taken on the current source).
TRAFFIC = {
    "source_sha256": "ff3bef451d868e6afd1faa1a076543104ce4c16cbbd3659416af7220bff10d4d",
    "fetch_kib": 466617.6,
    "write_kib": 120963.7,
    "fetch_scale": 2.0,
    "write_scale": 1.0,
}


def bf16_rows_per_workgroup():
    """Query rows per (head, query tile) unit of the bf16 forward, read off the
    workspace the library asks for: n_cu / 2 heads of SA_FEW_QUERY_ROWS + 1
    query rows (one more than the few-query path takes) over 16 key tiles make
    one part-empty round of n_cu / 2 units, which the stream-K tail spreads over
    every CU, with 2 * n_cu slots of rows * (head_dim + 1) floats."""
    import torch
    from streaming_video_diffusion_amd import binding as B
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = B.PackedContext(n_cu // 2, 128, torch.bfloat16, 1024, device="cuda")
    ctx.rows = 1024
    return B.sa_forward_workspace_bytes(ctx, B.SA_FEW_QUERY_ROWS + 1) // (2 * n_cu * 129 * 4)


def fwd_kernel_name(ca):
    bm = bf16_rows_per_workgroup()
    units = -(-ca.w.nq // bm) * ca.w.heads
    if ca.workspace is not None:
        return (f"fwd_bf16_kernel<128, false, false, *> ({units} units of {bm} queries, the last round's spread "
                f"over every CU) + tail_combine_kernel<128, false>")
    return f"fwd_bf16_kernel<128, false, false, false> ({units} workgroups of {bm} queries)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="full_1344x768")
    p.add_argument("--cpu-rows", type=int, default=2560, help="query rows in the oracle's timed sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--qk-norm", action="store_true",
                   help="fuse per-head RMS QK-norm (shared weights) into the pack and the query load")
    p.add_argument("--no-others", action="store_true",
                   help="skip the forward times of the other workloads and query variants")
    p.add_argument("--no-shard", action="store_true",
                   help="skip the extra measurement of one GPU's head shard (40/8 = 5 heads)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (3 times) and exit; "
                        "its FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic figures")
    p.add_argument("--few-query-only", action="store_true",
                   help="only time the 40 audio-only queries of the video+audio chunk (few-query path, "
                        "split-KV, plain forward) and print them as one JSON line")
    return p.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size (read mib MiB, write mib MiB), for
    scaling the profiler's FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "dispatches": 3}), flush=True)


def cpu_baseline(w, rows_n):
    """Time the fp64 oracle on a bounded sample: rotation of every key of the
    call plus ``rows_n`` query rows (all heads); extrapolate linearly in rows
    (rows are independent)."""
    import numpy as np
    from oracle import attn64
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = int(blas[0]["num_threads"]) if blas else 1
    except Exception:  # pragma: no cover
        threads = 1
    q = w.q(0)
    segs = [(*w.kv(i, 0), s.pos) for i, s in enumerate(w.segments)]
    rows = np.random.default_rng(7).choice(w.nq, size=min(rows_n, w.nq), replace=False)
    t0 = time.perf_counter()
    kr, vr = attn64.rotated_keys(segs, w.axis_dims, w.theta)
    t1 = time.perf_counter()
    from oracle import rope64
    qs = rope64.rotate(q[rows], rope64.angles(w.q_pos[rows], w.axis_dims, w.theta))
    attn64.attention(qs, kr, vr, w.scale)
    t2 = time.perf_counter()
    per_call = (t1 - t0) + (t2 - t1) * w.nq / len(rows)
    ms_chunk = per_call * w.calls * 1e3
    return {
        "value": w.flops_per_call() * w.calls / (ms_chunk * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(rows)} of {w.nq} query rows x {w.heads} heads plus rotation of all {w.nk} keys, "
                   f"one call, fp64 numpy; extrapolated linearly to {w.nq} rows x {w.calls} call(s)"),
        "ms_per_chunk": ms_chunk,
        "measured_s": t2 - t0,
        "host_cpus": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)),
    }


def measured_traffic():
    """HBM bytes per forward launch from the stored counters, or None when
    the forward kernel's source has changed since they were taken."""
    import hashlib
    if TRAFFIC["source_sha256"] is None:
        return None
    with open(FWD_SOURCE, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != TRAFFIC["source_sha256"]:
            return None
    return (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"] + TRAFFIC["write_kib"] * TRAFFIC["write_scale"]) * 1024.0


def shard_measure(steps):
    """Forward pass on one GPU's share of an 8-way head split (5 of 40 heads)
    at the full 1344x768 shape: an extra line, not the metric."""
    import torch
    from streaming_video_diffusion_amd import inputs as I
    from streaming_video_diffusion_amd.stream import ChunkAttention
    import dataclasses
    w = dataclasses.replace(I.full_1344x768(), name="full_1344x768_h5", heads=5)
    ca = ChunkAttention(w, device="cuda:0")
    stream = torch.cuda.current_stream()
    ca.pack_static(stream)
    ca.step(stream)
    ms = _time(lambda: ca.forward(stream), stream, steps)
    return {"heads": 5, "nq": w.nq, "nk": w.nk, "forward_ms": ms,
            "tflops": w.flops_per_call() / (ms * 1e-3) / 1e12,
            "workgroups": -(-w.nq // bf16_rows_per_workgroup()) * w.heads}


def _time(fn, stream, steps, warm_s=0.2):
    """Mean ms per call of ``fn`` over ``steps`` calls, after warming for at
    least ``warm_s`` seconds: the shader clock drops while the GPU idles (as
    it does while inputs are built on the host) and takes tens of ms under
    load to come back."""
    import time
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def other_workloads(steps, skip):
    """Forward and per-chunk pack time of the other 1344x768 workloads
    (hierarchical history, with its pooled tiers given or produced by the pack
    from full-resolution frames; joint video+audio; the query-side variants:
    history + current as queries, the 7-frame first window, the prefix
    self-attention pass), and
    the 40 audio-only queries of the video+audio chunk run over 32 key splits
    + merge, through the few-query path (sa_forward_ws: key runs per wave +
    merge, with its HBM rate over the K/V, Q and output bytes), and as one
    plain forward. Extra lines, not the metric."""
    import torch
    from streaming_video_diffusion_amd import binding as B
    from streaming_video_diffusion_amd import inputs as I
    from streaming_video_diffusion_amd.stream import ChunkAttention
    stream = torch.cuda.current_stream()
    res = {}
    makers = [f for n, f in list(I.CONFIGS.items()) + list(I.VARIANTS.items())
              if n != skip and f().nq >= 4096] + [I.hier_pooled_1344x768]
    for make in makers:
        w = make()
        ca = ChunkAttention(w, device="cuda:0")
        ca.pack_static(stream)
        ca.step(stream)
        ms = _time(lambda: ca.forward(stream), stream, steps)
        pack = _time(lambda: (ca._tables(True, stream), ca._pack(True, stream)), stream, steps)
        res[w.name] = {"nq": w.nq, "nk": w.nk, "forward_ms": ms, "pack_tables_ms": pack,
                       "tflops": w.flops_per_call() / (ms * 1e-3) / 1e12}
        if w.name == "video_audio_1344x768":
            res["audio_40q_over_52752kv"] = audio_measure(ca, w, stream, steps)
        del ca
        torch.cuda.empty_cache()
    res["tier_stream_1344x768"] = tier_stream_measure(steps)
    return res


def audio_measure(ca, w, stream, steps):
    """The 40 audio-only queries of the video+audio chunk (packed in ``ca``)
    over its 52752 keys: one plain forward, 32 key splits + merge, and the
    few-query path (sa_forward_ws: one key run per wave + merge) with its
    rate over the K/V, Q and output bytes."""
    import torch
    from streaming_video_diffusion_amd import binding as B
    q, qt = ca.q[w.nq - 40:], ca.q_table[w.nq - 40:]
    out = torch.empty((40, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda:0")
    part = torch.empty((32, 40, w.heads, w.head_dim), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((32, 40, w.heads), dtype=torch.float32, device="cuda:0")

    def split():
        B.sa_forward_split(ca.ctx, q, 32, qt, w.scale, partial=part, lse=lse, stream=stream)
        B.sa_combine_splits(part, lse, out=out, stream=stream)

    plain = _time(lambda: B.sa_forward(ca.ctx, q, qt, w.scale, out=out, stream=stream), stream, steps)
    need = B.sa_forward_workspace_bytes(ca.ctx, 40)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0") if need else None
    fewq = _time(lambda: B.sa_forward_ws(ca.ctx, q, qt, w.scale, out=out, stream=stream, workspace=ws), stream, steps)
    nbytes = w.nk * w.heads * w.head_dim * 2 * 2 + 2 * 40 * w.heads * w.head_dim * 2
    return {"plain_forward_ms": plain, "split32_plus_merge_ms": _time(split, stream, steps),
            "few_query_ms": fewq, "few_query_bytes": nbytes,
            "few_query_tb_per_s": nbytes / (fewq * 1e-3) / 1e12,
            "few_query_hbm_frac": nbytes / (fewq * 1e-3) / HBM_PEAK_BPS}


def tier_stream_measure(steps):
    """Per-chunk cost of the ageing history at 1344x768 in steady state (all
    three tiers present: 32260 keys): the in-place repack of the dynamic
    region from the raw K/V of the last four chunks (pooling the two older
    tiers again), then the forward."""
    import torch
    from streaming_video_diffusion_amd import inputs as I
    from streaming_video_diffusion_amd.stream import TierStreamAttention
    st = I.tier_stream_1344x768()
    stream = torch.cuda.current_stream()
    dt = torch.bfloat16
    chunks = []
    for c in range(5):
        k, v = st.chunk_kv(c)
        chunks.append(tuple(torch.from_numpy(x).to("cuda:0").to(dt) for x in (st.chunk_q(c), k, v)))
    ts = TierStreamAttention(st, device="cuda:0")
    ts.pack_static(stream)
    for c in range(4):
        ts.step(*chunks[c], stream=stream)
    i = [4]

    def age():
        q, k, v = chunks[i[0] % 5]
        ts.age(k, v, stream)
        i[0] += 1

    age_ms = _time(age, stream, steps)
    q = chunks[(i[0] - 1) % 5][0]
    fwd_ms = _time(lambda: ts.forward(q, stream), stream, steps)
    step_ms = _time(lambda: (age(), ts.forward(chunks[(i[0] - 1) % 5][0], stream)), stream, steps)
    w_flops = 4.0 * st.chunk_rows * ts.ctx.rows * st.head_dim * st.heads
    return {"nq": st.chunk_rows, "nk": int(ts.ctx.rows), "age_repack_ms": age_ms, "forward_ms": fwd_ms,
            "step_ms": step_ms, "tflops_step": w_flops / (step_ms * 1e-3) / 1e12}


class SclkSampler:
    """Samples the shader clock the driver reports (the line marked '*' in
    the DRM device's pp_dpm_sclk) and, where the device's hwmon exposes it,
    the board power it reports (power1_average, else power1_input, in uW, and
    its cap power1_cap) every ``period`` seconds on a host thread, while the
    GPU runs the timed steps. Reports nothing where the files are absent or
    unreadable."""

    def __init__(self, period=0.01):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.power_paths = []
        for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
            for name in ("power1_average", "power1_input"):
                if os.path.exists(os.path.join(d, name)):
                    self.power_paths.append((os.path.join(d, name), os.path.join(d, "power1_cap")))
                    break
        self.period, self.samples, self.power = period, [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for path in self.paths:
            try:
                with open(path) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            mhz = line.split(":", 1)[1].strip().split()[0].lower().replace("mhz", "")
                            return float(mhz)
            except (OSError, ValueError, IndexError):
                continue
        return None

    @staticmethod
    def _read_uw(path):
        try:
            with open(path) as f:
                return float(f.read().strip())
        except (OSError, ValueError):
            return None

    def _run(self):
        while not self._stop.wait(self.period):
            v = self._read()
            if v is not None:
                self.samples.append(v)
            for path, _ in self.power_paths[:1]:
                uw = self._read_uw(path)
                if uw is not None:
                    self.power.append(uw * 1e-6)

    def __enter__(self):
        if self.paths or self.power_paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths or self.power_paths:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        out = {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
               "source": "pp_dpm_sclk (driver-reported current shader clock), sampled during the timed steps"}
        if self.power:
            pw = sorted(self.power)
            cap = self._read_uw(self.power_paths[0][1])
            out["board_power_w"] = {"median": pw[len(pw) // 2], "max": pw[-1], "samples": len(pw),
                                    "cap": cap * 1e-6 if cap else None,
                                    "source": os.path.basename(self.power_paths[0][0]) + " (hwmon, driver-reported)"}
        return out


def few_query_only(steps):
    """The audio-query measurement alone (for profiling the few-query kernel)."""
    import torch
    from streaming_video_diffusion_amd import inputs as I
    from streaming_video_diffusion_amd.stream import ChunkAttention
    stream = torch.cuda.current_stream()
    w = I.video_audio_1344x768()
    ca = ChunkAttention(w, device="cuda:0")
    ca.pack_static(stream)
    ca.step(stream)
    res = audio_measure(ca, w, stream, steps)
    print(json.dumps({"workload": "audio_40q_over_52752kv", "steps": steps, **res}), flush=True)


def main():
    args = parse()
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.few_query_only:
        few_query_only(args.steps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the attention shards by head; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from streaming_video_diffusion_amd import inputs as I
    from streaming_video_diffusion_amd.stream import ChunkAttention

    w = I.CONFIGS[args.workload]()
    if args.qk_norm:
        import dataclasses
        w = dataclasses.replace(w, name=w.name + "_qknorm", qk_norm="shared")
    calls = [ChunkAttention(w, call=c, device="cuda:0") for c in range(w.calls)]
    stream = torch.cuda.current_stream()
    for ca in calls:
        ca.pack_static(stream)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for ca in calls:
            ca.step(stream)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    fwd_ev, pack_ev = [], []
    start, end = ev(), ev()
    torch.cuda.synchronize()
    with SclkSampler() as sclk:
        start.record(stream)
        for _ in range(args.steps):
            for ca in calls:
                p0, p1, f1 = ev(), ev(), ev()
                p0.record(stream)
                ca._tables(True, stream)
                ca._pack(True, stream)
                p1.record(stream)
                ca.forward(stream)
                f1.record(stream)
                pack_ev.append((p0, p1))
                fwd_ev.append((p1, f1))
        end.record(stream)
        torch.cuda.synchronize()

    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    fwd_ms = [a.elapsed_time(b) for a, b in fwd_ev]
    pack_ms = [a.elapsed_time(b) for a, b in pack_ev]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    flops_chunk = w.flops_per_call() * w.calls
    flops_launch = w.flops_per_call()
    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    achieved = flops_launch / (fwd_avg * 1e-3) / 1e12
    fwd_sorted = sorted(fwd_ms)

    out = {
        "metric": METRIC,
        "value": flops_chunk / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1), bf16-rounded; no real latents or weights)",
        "config": {
            "workload": w.name,
            "description": w.description,
            "nq": w.nq, "nk": w.nk, "heads": w.heads, "head_dim": w.head_dim, "calls": w.calls,
            "segments": [[s.name, s.rows, "dynamic" if s.dynamic else "static"] for s in w.segments],
            "step": "rope tables (dynamic template) + in-place pack of dynamic K/V + forward",
            "flops_per_chunk": flops_chunk,
            "entropy": I.ENTROPY,
        },
        "forward_ms_avg": fwd_avg,
        "forward_ms_median": fwd_sorted[len(fwd_sorted) // 2],
        "forward_tflops": achieved,
        "pack_tables_ms_avg": sum(pack_ms) / len(pack_ms),
        "sclk": sclk.summary(),
        "roofline": {
            "bound": "mfma" if bf16 else "alu",
            "kernel": fwd_kernel_name(calls[0]) if bf16 else "fwd_f32_kernel",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": measured_traffic() if (bf16 and w.name == "full_1344x768") else None,
        },
    }
    if not args.no_shard:
        out["one_gpu_head_shard"] = shard_measure(20)
    if not args.no_others:
        out["other_workloads"] = other_workloads(10, w.name)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
