"""Benchmark of the LongFlow fused decode + score + evict step on one MI355X.

Default workload: the DeepSeek-R1-Distill-Llama-8B-shaped attention layer
(batch 64, 32 query heads over 8 KV heads, head_dim 128, bfloat16, budget
3277 = 20% of 16384) in its steady state: every pair holds 3277 tokens and
every step scores all of them, evicts one per pair and writes the new token
in place. One step = one lf_decode_step over the whole batch.

Prints ONE JSON line with the throughput, the roofline of the fused kernel
(algorithmic HBM bytes per launch / average launch time, against the 8 TB/s
HBM3E peak), the full-KV baseline on the same GPU (same kernel family with
no eviction over a growing cache) and the CPU oracle on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused decode+evict steps/sec (tokens/s) and achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, AMD public specification
KERNEL_SOURCES = [os.path.join(ROOT, "decode_kv_cache_02_amd", "csrc", f)
                  for f in ("lf_decode.h", "lf_decode_w4.hip", "lf_decode_w8.hip", "lf_decode_w4i.hip",
                            "lf_decode_w8i.hip", "lf_kernels.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_llama8b_layer.json")
RING = 64


def algorithmic_bytes_per_pair(n: int, G: int, d: int, e: int, evict: bool) -> int:
    """HBM bytes the method itself must move for one pair and one step.

    Read K and V of the n valid slots, read the query group, write the output
    group, read k_new and v_new, write the new token's K, V and ||v||_1, write
    the evicted slot. The ||v||_1 sidecar reads (4 bytes per slot) are
    excluded: the method could derive them from the V rows it already reads.
    """
    return (n * 2 * d * e          # K, V of the valid slots
            + 2 * G * d * e         # q in, out
            + 2 * d * e             # k_new, v_new in
            + 2 * d * e + 4         # slot write: K, V, ||v||_1
            + (4 if evict else 0))  # evicted slot


def kernel_sha() -> str:
    """sha256[:16] over the kernel sources (decode kernel, its instances, fill)
    with comments and whitespace removed, so only code changes alter it."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(bytes_alg_per_launch: float):
    """HBM traffic from committed rocprofv3 --pmc counters, if the kernel is unchanged."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return float(t["hbm_bytes_per_launch"])


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama8b_layer")
    ap.add_argument("--budget", type=int, default=0, help="override the budget")
    ap.add_argument("--batch", type=int, default=0, help="override the batch")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="override the KV heads, keeping the group width (1 gives one GPU's share "
                         "under tensor parallelism over 8 KV heads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-kv", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--suite-part", default="", help=argparse.SUPPRESS)
    ap.add_argument("--suite", action="store_true",
                    help="measure every workload shape (one JSON line each) instead of the bench line")
    ap.add_argument("--wg-timing", action="store_true",
                    help="per-workgroup timing records: how each launch spreads over the XCDs")
    ap.add_argument("--phases", action="store_true",
                    help="per-workgroup phase records: where one launch's time goes")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="the Llama-8B layer at batches 1-256 with the automatic launch")
    ap.add_argument("--stack-trajectory", type=int, default=0, metavar="B",
                    help="time the 36-layer Qwen3-8B stack at budget B over its whole run "
                         "(512-token prompt, 16,384 model steps)")
    return ap.parse_args()


def prepared_ring(cache, ring, out, ev, layers=1):
    """lf_decode_step arguments for every (ring entry, layer), checked once, so
    the timed loops spend no host time on tensor checks (short kernels would
    otherwise be timed on the host)."""
    return [[cache.step_args(layer, q, kn, vn, out, ev) for layer in range(layers)]
            for q, kn, vn in ring]


REPEATS = 5


def timed_windows(run, steps, repeats=REPEATS):
    """Time `steps` calls of run(t) as `repeats` consecutive windows, each
    bracketed by HIP events on the current stream (the one the library's
    kernels are queued on). Returns ms per step of every window."""
    import torch
    stream = torch.cuda.current_stream()
    bounds = [round(steps * r / repeats) for r in range(repeats + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.synchronize()
    events[0].record(stream)
    for r in range(repeats):
        for t in range(bounds[r], bounds[r + 1]):
            run(t)
        events[r + 1].record(stream)
    torch.cuda.synchronize()
    return [events[r].elapsed_time(events[r + 1]) / max(1, bounds[r + 1] - bounds[r])
            for r in range(repeats)]


def time_steps(cache, ring, out, ev, steps, warmup):
    """Warmup, then `steps` timed steps in 5 windows; returns (median ms per
    step, the windows' ms per step)."""
    args = prepared_ring(cache, ring, out, ev)
    step = cache.step_prepared
    for t in range(warmup):
        step(args[t % RING][0])
    windows = timed_windows(lambda t: step(args[t % RING][0]), steps)
    return float(np.median(windows)), windows


def make_ring(wl, dtype):
    import torch
    from decode_kv_cache_02_amd.synth import step_ring
    q, k, v = step_ring(wl, RING)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(x).cuda().to(dt)
    return [(dev(q[i]), dev(k[i]), dev(v[i])) for i in range(RING)]


def _cpu_worker(wl, pairs, fills, seconds, start, results):
    """One host core: step its share of the pairs through the oracle for
    about `seconds` after the common start, each pair from its fill level
    (`fills[b]` tokens of sequence b; full pairs evict at every step, the
    others append until they reach the budget). Inputs are drawn before the
    start (they are resident, as on the GPU)."""
    from threadpoolctl import threadpool_limits
    from decode_kv_cache_02_amd.synth import PairTokenStream
    from oracle.longflow_oracle import PairCache
    with threadpool_limits(limits=1):
        caches, inputs = [], []
        for b, h in pairs:
            ps = PairTokenStream(wl, b, h, seed_offset=99)
            c = PairCache(wl.budget, wl.head_dim)
            c.prefill(*ps.prefill(int(fills[b])))
            caches.append(c)
            inputs.append(ps.steps(RING))
        start.wait()
        steps = 0
        t0 = time.perf_counter()
        while True:
            for c, (q, kn, vn) in zip(caches, inputs):
                i = steps % RING
                c.step(q[i], kn[i], vn[i])
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    results.put((len(pairs), steps, el))


def cpu_baseline(wl, seconds: float, sample: int = 0, fills=None):
    """The float64 oracle on every host core, on a bounded sample of the same
    workload: one process per core (one BLAS thread each), the pairs dealt out
    round robin, each pair from its fill level (every pair full unless
    `fills`, one level per sequence, is given). Each process steps all of its
    pairs once per round, for about `seconds`. `sample` > 0 times that many
    pairs spread evenly over the layer instead of all of them; the rates are
    per pair-step, so they scale to the layer. Must run before the process
    touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    all_pairs = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    timed = all_pairs
    if 0 < sample < len(all_pairs):
        timed = [all_pairs[i * len(all_pairs) // sample] for i in range(sample)]
    if fills is None:
        fills = np.full(wl.batch, wl.budget, dtype=np.int64)
    workers = max(1, min(cores, len(timed)))
    ctx = mp.get_context("fork")
    start = ctx.Barrier(workers + 1)
    results = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker,
                         args=(wl, timed[w::workers], fills, seconds, start, results))
             for w in range(workers)]
    for p in procs:
        p.start()
    # Every wait is bounded: a worker that dies (and so never reaches the
    # barrier or never reports) ends the baseline with an error, not a hang.
    limit = 4 * seconds + 300
    try:
        start.wait(timeout=limit)
        got = [results.get(timeout=limit) for _ in procs]
    except Exception as exc:
        for p in procs:
            if p.is_alive():
                p.terminate()
        raise RuntimeError(f"CPU baseline worker failed: {exc!r}") from exc
    finally:
        for p in procs:
            p.join(timeout=60)
    pair_steps_per_s = sum(n * st / el for n, st, el in got)
    steps_per_s = pair_steps_per_s / len(all_pairs)     # layer steps
    pair_steps = sum(n * st for n, st, _ in got)
    full = bool(np.all(np.asarray(fills) >= wl.budget))
    return {"value": steps_per_s * wl.batch, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "steps_per_s": steps_per_s, "pair_steps_per_s": pair_steps_per_s,
            "host_cores_available": cores,
            "sample": f"{wl.name} with {'every pair full' if full else 'its ragged fill levels'} "
                      f"({len(all_pairs)} pairs x {wl.budget} slots; "
                      f"{'all' if len(timed) == len(all_pairs) else len(timed)} of the pairs "
                      f"timed): {workers} processes, one per host core, each stepping its "
                      f"share of the pairs through the float64 NumPy oracle (one BLAS thread) "
                      f"for {seconds:.0f} s; {pair_steps} pair-steps in all. tokens/s = "
                      f"pair-steps/s / {len(all_pairs)} pairs per layer step x batch {wl.batch}"}


def cpu_suite(seconds: float):
    """The oracle on every host core for each workload configuration, one JSON
    line each (before any GPU work: the workers are forked). Stacks are timed
    on one layer with the stack's per-layer shape and fill levels; their
    model-step rate is that layer rate divided by the layer count
    (extrapolated)."""
    from decode_kv_cache_02_amd.native import lf_cache_bytes, make_config
    from decode_kv_cache_02_amd.synth import WORKLOADS, TokenStream

    def line(name, wl, layers, cpu):
        cpu = dict(cpu)
        per_layer = cpu["steps_per_s"]
        cpu["model_steps_per_s"] = per_layer / layers
        cpu["value"] = per_layer / layers * wl.batch
        if layers > 1:
            cpu["extrapolated"] = f"one layer timed; model steps/s = layer steps/s / {layers}"
        print(json.dumps({"workload": name, "batch": wl.batch, "budget": wl.budget, "layers": layers,
                          "cpu_oracle": cpu}), flush=True)

    sample = 64
    line("tiny_f32", WORKLOADS["tiny_f32"], 1, cpu_baseline(WORKLOADS["tiny_f32"], seconds))
    for name in ("qwen3_0p6b_layer", "llama8b_layer"):
        wl = WORKLOADS[name]
        line(name, wl, 1, cpu_baseline(wl, seconds, sample=sample))
    wl4 = WORKLOADS["llama8b_stack32_ragged"]
    per_seq = (lf_cache_bytes(make_config(32, 1, 32, 8, 128, wl4.budget))
               + lf_cache_bytes(make_config(32, 1, 32, 8, 128, 16384 + 512 + 64, mode="full")))
    wl4 = wl4.with_(batch=int(0.95 * 288e9 // per_seq))
    fills = np.minimum(TokenStream(wl4).start_offsets(), wl4.budget)
    line("llama8b_stack32_ragged LongFlow", wl4, 32, cpu_baseline(wl4, seconds, sample=sample, fills=fills))
    wl5 = WORKLOADS["qwen3_8b_stack36_ties"]
    for budget in (512, 1024, 2048, 4096):
        w = wl5.with_(budget=budget)
        line(f"qwen3_8b_stack36 B={budget}", w, 36, cpu_baseline(w, seconds, sample=sample))


def full_kv_baseline(wl, steps, warmup, fills=(8704, 16384)):
    """LF_MODE_FULL at the same batch: no eviction, the cache keeps growing."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    cap = max(fills) + steps + warmup + 64
    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, cap,
                          dtype=wl.dtype, mode="full")
    ring = make_ring(wl, wl.dtype)
    dt = ring[0][0].dtype
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=dt, device="cuda")
    ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
    res = {}
    try:
        for n in fills:
            k, v = device_prefill(wl, n, seed=7 + n)
            cache.prefill(0, k, v, np.full(wl.batch, n, dtype=np.int32))
            del k, v
            torch.cuda.synchronize()
            ms, win = time_steps(cache, ring, out, ev, steps, warmup)
            nb = wl.batch * wl.num_kv_heads * algorithmic_bytes_per_pair(
                n + warmup + steps // 2, wl.group, wl.head_dim, 2 if wl.dtype == "bf16" else 4,
                False)
            res[str(n)] = {"ms_per_step": ms, "ms_windows": win, "tokens_per_s": wl.batch / ms * 1e3,
                           "achieved_GBs": nb / ms / 1e6}
    finally:
        cache.close()
    return {"mode": "full-KV decode attention (no eviction, growing cache), same GPU, same batch",
            "capacity": cap, "at_fill": res}


def steady_state(wl, steps, warmup, fill=None, mode="evict", layers=1, capacity=None,
                 ragged=None, seed=0, order="same_step", scope="kv_head", norm="l1"):
    """Time `steps` model steps (one lf_decode_step per layer) at the given
    fill levels, in 5 windows; returns (median ms per model step, algorithmic
    bytes per model step, the windows' ms per model step)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    e = 2 if wl.dtype == "bf16" else 4
    cap = wl.budget if capacity is None else capacity
    torch.cuda.empty_cache()
    cache = LongFlowCache(layers, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, cap,
                          dtype=wl.dtype, mode=mode, order=order, scope=scope, norm=norm)
    try:
        n = np.full(wl.batch, wl.budget if fill is None else fill, dtype=np.int64)
        if ragged is not None:
            n = np.asarray(ragged, dtype=np.int64)
        n_max = int(n.max(initial=0))
        for layer in range(layers):
            if n_max > 0:
                k, v = device_prefill(wl.with_(), n_max, seed=seed * 1000 + layer)
                cache.prefill(layer, k, v, n.astype(np.int32))
                del k, v
            else:
                cache.prefill(layer, None, None, n.astype(np.int32))
        ring = make_ring(wl, wl.dtype)
        dt = ring[0][0].dtype
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=dt, device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        args = prepared_ring(cache, ring, out, ev, layers)
        step = cache.step_prepared
        for t in range(warmup):
            for a in args[t % RING]:
                step(a)

        def model_step(t):
            for a in args[(warmup + t) % RING]:
                step(a)

        windows = timed_windows(model_step, steps)
        ms = float(np.median(windows))
        # fill levels during the timed window (EVICT caps at the budget)
        n_mid = n + warmup + steps // 2
        if mode == "evict":
            n_mid = np.minimum(n_mid, wl.budget)
        evict_flags = (n + warmup >= wl.budget) if mode == "evict" else np.zeros_like(n, bool)
        per_layer = sum(algorithmic_bytes_per_pair(int(nb), wl.group, wl.head_dim, e, bool(ev_))
                        for nb, ev_ in zip(n_mid, evict_flags)) * wl.num_kv_heads
        return ms, per_layer * layers, windows
    finally:
        cache.close()


COLD_STEPS = 60


def warm_vs_cold(wl, steps: int = COLD_STEPS, read_bytes: int = 1 << 30):
    """Every pair full; each decode step timed alone by an event pair, (a) back
    to back and (b) after a read of `read_bytes` queued just before it (a max
    reduction over an unrelated buffer: its reads replace what the last-level
    cache held, and it writes nothing back). Returns (median us back to back,
    median us after the read, algorithmic bytes per step). The per-step events
    cost a little, so both figures sit slightly above the windowed
    steady-state line."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    e = 2 if wl.dtype == "bf16" else 4
    src = torch.ones(read_bytes // 2, dtype=torch.float16, device="cuda")
    sink = torch.empty((), dtype=torch.float16, device="cuda")
    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        k, v = device_prefill(wl, wl.budget, seed=5)
        cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
        del k, v
        ring = make_ring(wl, wl.dtype)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                          device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        args = prepared_ring(cache, ring, out, ev)
        med = {}
        for cold in (False, True, False, True):
            for t in range(10):
                cache.step_prepared(args[t % RING][0])
            marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(steps)]
            torch.cuda.synchronize()
            for t, (a, b) in enumerate(marks):
                if cold:
                    torch.amax(src, dim=0, out=sink)
                a.record()
                cache.step_prepared(args[t % RING][0])
                b.record()
            torch.cuda.synchronize()
            med.setdefault(cold, []).append(float(np.median([a.elapsed_time(b) * 1e3 for a, b in marks])))
        nb = wl.batch * wl.num_kv_heads * algorithmic_bytes_per_pair(wl.budget, wl.group, wl.head_dim,
                                                                       e, True)
        return float(np.mean(med[False])), float(np.mean(med[True])), nb
    finally:
        cache.close()
        del src, sink


def churn(wl, steps, warmup, every=16, per_event=4, prompt=512):
    """Serving churn over the static buffer: start with every pair full; every
    `every` steps, `per_event` sequences (round robin) finish and their slots
    are recycled for a new request (lf_seq_reset, then lf_prefill_fill of a
    `prompt`-token prompt with -1 for every other sequence). The reset and
    prefill calls are inside the timed window. Returns (ms per step, algorithmic
    bytes per step: decode at the actual fill levels plus the prompts' K and V
    read and written)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    e = 2 if wl.dtype == "bf16" else 4
    torch.cuda.empty_cache()
    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        k, v = device_prefill(wl, wl.budget, seed=11)
        cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
        del k, v
        pk, pv = device_prefill(wl, prompt, seed=12)     # prompts, [batch][prompt][hkv][d]
        ring = make_ring(wl, wl.dtype)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                          device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        fill = np.full(wl.batch, wl.budget, dtype=np.int64)
        nbytes = 0
        nxt = 0

        def one(t, count):
            nonlocal nxt, nbytes
            if t % every == every - 1:
                seqs = [(nxt + i) % wl.batch for i in range(per_event)]
                nxt = (nxt + per_event) % wl.batch
                cache.seq_reset(seqs)
                n = np.full(wl.batch, -1, dtype=np.int32)
                n[seqs] = prompt
                cache.prefill(0, pk, pv, n)
                fill[seqs] = prompt
                if count:
                    nbytes += len(seqs) * wl.num_kv_heads * prompt * (4 * wl.head_dim * e + 4)
            q, kn, vn = ring[t % RING]
            cache.decode_step(0, q, kn, vn, out, ev)
            if count:
                nbytes += wl.num_kv_heads * sum(
                    algorithmic_bytes_per_pair(int(nb), wl.group, wl.head_dim, e, nb >= wl.budget)
                    for nb in fill)
            np.minimum(fill + 1, wl.budget, out=fill)

        for t in range(warmup):
            one(t, False)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for t in range(warmup, warmup + steps):
            one(t, True)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps, nbytes / steps
    finally:
        cache.close()


def stream_read_ceiling(total_bytes: int = 860_160_000, workgroups: int = 512, reps: int = 50):
    """Attainable streaming-read bandwidth: lf_probe_stream_read (the decode
    kernel's K/V loads) over `total_bytes`, split like the Llama-8B layer
    launch (512 workgroups, ~1.68 MB each). Returns GB/s (best of 3)."""
    import torch
    from decode_kv_cache_02_amd.native import lf_probe_stream_read
    unit = 16 * workgroups
    total_bytes -= total_bytes % unit
    buf = torch.ones(total_bytes // 2, dtype=torch.int16, device="cuda")
    sink = torch.empty(workgroups * 256 * 4, dtype=torch.int32, device="cuda")
    for _ in range(5):
        lf_probe_stream_read(buf, workgroups, sink)
    best = 0.0
    for _ in range(3):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            lf_probe_stream_read(buf, workgroups, sink)
        end.record()
        torch.cuda.synchronize()
        best = max(best, total_bytes / (start.elapsed_time(end) / reps) / 1e6)
    del buf, sink
    return best


def trajectory(wl, steps: int, prompt: int, mode: str):
    """A whole generation: every sequence starts from a `prompt`-token prompt
    and decodes `steps` tokens (LongFlow: fill, then evict at the budget;
    full-KV: the cache grows to prompt + steps). One event pair around the
    whole run. Returns (ms per step, algorithmic bytes per step)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    e = 2 if wl.dtype == "bf16" else 4
    cap = wl.budget if mode == "evict" else prompt + steps + 64
    torch.cuda.empty_cache()
    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, cap,
                          dtype=wl.dtype, mode=mode)
    try:
        k, v = device_prefill(wl, prompt, seed=13)
        cache.prefill(0, k, v, np.full(wl.batch, prompt, dtype=np.int32))
        del k, v
        ring = make_ring(wl, wl.dtype)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                          device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        args = prepared_ring(cache, ring, out, ev)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for t in range(steps):
            cache.step_prepared(args[t % RING][0])
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        nbytes = 0
        for t in range(steps):
            n = prompt + t
            evict = mode == "evict" and n >= wl.budget
            if mode == "evict":
                n = min(n, wl.budget)
            nbytes += algorithmic_bytes_per_pair(n, wl.group, wl.head_dim, e, evict)
        return ms, nbytes * wl.batch * wl.num_kv_heads / steps
    finally:
        cache.close()


def stack_trajectory(wl, layers: int, steps: int, prompt: int, segment: int = 1024):
    """A whole generation through a `layers`-layer stack: every sequence of
    every layer starts from a `prompt`-token prompt, then `steps` model steps
    (one lf_decode_step per layer each) fill the cache to the budget and evict
    from then on. One event pair per `segment` model steps, each printed to
    stderr as it ends. Returns a dict: ms per model step over the whole run,
    algorithmic bytes per model step, and the fill and evict phases apart."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    e = 2 if wl.dtype == "bf16" else 4
    torch.cuda.empty_cache()
    cache = LongFlowCache(layers, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        for layer in range(layers):
            k, v = device_prefill(wl, prompt, seed=17 * 1000 + layer)
            cache.prefill(layer, k, v, np.full(wl.batch, prompt, dtype=np.int32))
            del k, v
        ring = make_ring(wl, wl.dtype)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                          device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        args = prepared_ring(cache, ring, out, ev, layers)
        step = cache.step_prepared
        torch.cuda.synchronize()
        seg_ms = []
        for s0 in range(0, steps, segment):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record()
            for t in range(s0, min(steps, s0 + segment)):
                for a in args[t % RING]:
                    step(a)
            end.record()
            torch.cuda.synchronize()
            seg_ms.append(start.elapsed_time(end))
            print(f"[stack] B={wl.budget}: model steps {s0}-{min(steps, s0 + segment) - 1}: "
                  f"{seg_ms[-1] / (min(steps, s0 + segment) - s0):.3f} ms each", file=sys.stderr, flush=True)
        per_pair = [algorithmic_bytes_per_pair(min(prompt + t, wl.budget), wl.group, wl.head_dim, e,
                                               prompt + t >= wl.budget) for t in range(steps)]
        pairs = wl.batch * wl.num_kv_heads
        fill_steps = max(0, min(steps, wl.budget - prompt))
        total_ms = float(sum(seg_ms))
        res = {"ms_per_model_step": total_ms / steps,
               "bytes_per_model_step": float(np.mean(per_pair)) * pairs * layers,
               "fill_steps": fill_steps, "segment_ms_per_model_step":
               [round(m / min(segment, steps - i * segment), 4) for i, m in enumerate(seg_ms)]}
        # phases apart, from the segments wholly inside each phase
        fill_segs = [m / segment for i, m in enumerate(seg_ms) if (i + 1) * segment <= fill_steps]
        evict_segs = [m / min(segment, steps - i * segment) for i, m in enumerate(seg_ms)
                      if i * segment >= fill_steps]
        if evict_segs:
            res["evict_ms_per_model_step"] = float(np.mean(evict_segs))
            res["evict_bytes_per_model_step"] = per_pair[-1] * pairs * layers
        if fill_segs:
            res["fill_ms_per_model_step"] = float(np.mean(fill_segs))
        return res
    finally:
        cache.close()


SWEEP_BATCHES = (1, 2, 4, 8, 12, 16, 24, 31, 32, 33, 36, 40, 48, 56, 64, 65, 68, 72, 80, 88, 96,
                 102, 112, 120, 127, 128, 129, 136, 144, 160, 192, 193, 200, 224, 256)


def launch_workgroups(wl):
    """Workgroups of the automatic launch of one step of `wl` with every pair
    full (one lf_probe_decode_timing call on a fresh cache)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache, lf_probe_decode_timing
    from decode_kv_cache_02_amd.synth import device_prefill, device_steps
    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        k, v = device_prefill(wl, wl.budget, seed=3)
        cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
        del k, v
        Q, KN, VN = device_steps(wl, 1, seed=3)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=Q.dtype, device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        rec = torch.zeros((max(4096, wl.batch * wl.num_kv_heads), 4), dtype=torch.int64, device="cuda")
        n = lf_probe_decode_timing(cache.handle, 0, Q[0], KN[0], VN[0], out, ev, rec)
        torch.cuda.synchronize()
        return n
    finally:
        cache.close()


def batch_sweep(args):
    """The Llama-8B layer (B = 3277, every pair full) at every batch of
    SWEEP_BATCHES with the automatic launch: one JSON line per batch (median
    of 5 windows x 200 steps, and the launch's workgroup count)."""
    from decode_kv_cache_02_amd.synth import WORKLOADS
    w3 = WORKLOADS["llama8b_layer"]
    for b in SWEEP_BATCHES:
        w = w3.with_(batch=b)
        ms, nb, win = steady_state(w, 200, 20)
        print(json.dumps({"batch": b, "pairs": b * w.num_kv_heads, "workgroups": launch_workgroups(w),
                          "us_per_step": ms * 1e3, "us_per_pair": ms * 1e3 / (b * w.num_kv_heads),
                          "tokens_per_s": b / ms * 1e3, "achieved_GBs": nb / ms / 1e6,
                          "frac_of_peak": nb / ms / 1e6 / HBM_PEAK_GBS, "ms_windows": win}), flush=True)


def tiny_latency(wl, steps: int = 2000, per_graph: int = 64):
    """The launch-latency-bound tiny workload (one pair, B = 64, fp32): steps/s
    with one lf_decode_step call per step, and with 64 steps captured in one
    HIP graph and replayed. Returns (eager ms per step, graph ms per step)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        k, v = device_prefill(wl, wl.budget, seed=1)
        cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
        ring = make_ring(wl, wl.dtype)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                          device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        eager, _ = time_steps(cache, ring, out, ev, steps, 50)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            args = prepared_ring(cache, ring, out, ev)
            for t in range(per_graph):
                cache.step_prepared(args[t % RING][0])
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            args = prepared_ring(cache, ring, out, ev)
            for t in range(per_graph):
                cache.step_prepared(args[t % RING][0])
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        return eager, start.elapsed_time(end) / (reps * per_graph)
    finally:
        cache.close()


def stack_graph(wl, layers, model_steps, seed=0):
    """A stack with every pair full, one model step (an lf_decode_step per
    layer) captured in one HIP graph and replayed `model_steps` times with the
    same inputs (the step's cost depends on fill levels, not values). Returns
    (median ms per model step over 5 windows, algorithmic bytes per model
    step, the windows)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill
    e = 2 if wl.dtype == "bf16" else 4
    torch.cuda.empty_cache()
    cache = LongFlowCache(layers, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        n = np.full(wl.batch, wl.budget, dtype=np.int32)
        for layer in range(layers):
            k, v = device_prefill(wl.with_(), wl.budget, seed=seed * 1000 + layer)
            cache.prefill(layer, k, v, n)
            del k, v
        q, kn, vn = make_ring(wl, wl.dtype)[0]
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=q.dtype, device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                for layer in range(layers):
                    cache.step_prepared(cache.step_args(layer, q, kn, vn, out, ev))
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for layer in range(layers):
                cache.step_prepared(cache.step_args(layer, q, kn, vn, out, ev))
        for _ in range(3):
            graph.replay()
        windows = timed_windows(lambda t: graph.replay(), model_steps)
        ms = float(np.median(windows))
        per_layer = wl.batch * wl.num_kv_heads * algorithmic_bytes_per_pair(wl.budget, wl.group,
                                                                            wl.head_dim, e, True)
        return ms, per_layer * layers, windows
    finally:
        cache.close()


def batch_gain(wl, model_steps):
    """Each method on the 32-layer ragged stack at the largest batch its own
    cache allows in 0.95 x 288 GB, with the same start-offset distribution:
    the comparison of tokens/s at each method's own batch. Yields (workload,
    ms per model step, algorithmic bytes per model step, windows, extra
    fields)."""
    from decode_kv_cache_02_amd.native import lf_cache_bytes, make_config
    from decode_kv_cache_02_amd.synth import TokenStream
    rate = {}
    for method, mode, cap in (("LongFlow", "evict", wl.budget), ("full-KV", "full", 16384 + 512 + 64)):
        b = int(0.95 * 288e9 // lf_cache_bytes(make_config(32, 1, 32, 8, 128, cap, mode=mode)))
        w = wl.with_(batch=b)
        offs = TokenStream(w).start_offsets()
        ms, nb, win = steady_state(w, model_steps, 2, layers=32, mode=mode, capacity=cap,
                                   ragged=np.minimum(offs, cap) if mode == "evict" else offs, seed=6)
        rate[method] = b / ms
        extra = {"method": method,
                 "batch_rule": "largest batch with this method's cache alone in 0.95 x 288 GB"}
        if method == "full-KV":
            extra["longflow_tokens_per_s_over_full_kv"] = rate["LongFlow"] / rate["full-KV"]
        yield w, ms, nb, win, extra


SUITE_PARTS = ("tiny", "qwen06", "llama", "generation", "variants", "churn", "small", "ragged",
               "gain", "qwen_b512", "qwen_b1024", "qwen_b2048", "qwen_b4096", "qwen_graph", "cold")


def suite(args):
    """One JSON line per workload shape (steady state unless stated). Lines
    timed in windows report the median of 5 windows and every window. Each
    group of lines runs in a child process of its own, so no measurement
    inherits another's allocations; this process never touches the GPU."""
    import subprocess
    for part in SUITE_PARTS:
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--suite-part", part,
               "--steps", str(args.steps)]
        proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, text=True)
        for line in proc.stdout:
            print(line, end="", flush=True)
        if proc.wait() != 0:
            raise RuntimeError(f"suite part {part} failed with status {proc.returncode}")


def suite_part(part, args):
    """One group of suite lines (see suite)."""
    from decode_kv_cache_02_amd.native import lf_cache_bytes, make_config
    from decode_kv_cache_02_amd.synth import WORKLOADS, TokenStream

    def emit(name, wl, ms, nbytes, layers=1, extra=None, windows=None, steps=None):
        line = {"workload": name, "batch": wl.batch, "heads": f"{wl.num_q_heads}/{wl.num_kv_heads}",
                "head_dim": wl.head_dim, "budget": wl.budget, "layers": layers,
                "ms_per_model_step": ms, "tokens_per_s": wl.batch / ms * 1e3,
                "achieved_GBs": nbytes / ms / 1e6,
                "frac_of_peak": nbytes / ms / 1e6 / HBM_PEAK_GBS}
        if steps is not None:
            line["timed_model_steps"] = steps
        if windows is not None:
            line["ms_windows"] = windows
        line.update(extra or {})
        print(json.dumps(line), flush=True)

    steps, warmup = min(args.steps, 300), 20
    wl3 = WORKLOADS["llama8b_layer"]
    wl5 = WORKLOADS["qwen3_8b_stack36_ties"]

    def ragged_stack():
        # 32-layer ragged stack at the batch where both caches fit 0.95 x 288 GB
        wl4 = WORKLOADS["llama8b_stack32_ragged"]
        cfg_c = make_config(32, 1, 32, 8, 128, wl4.budget)
        cfg_f = make_config(32, 1, 32, 8, 128, 16384 + 512 + 64, mode="full")
        per_seq = lf_cache_bytes(cfg_c) + lf_cache_bytes(cfg_f)
        return wl4.with_(batch=int(0.95 * 288e9 // per_seq))

    if part == "tiny":
        wl1 = WORKLOADS["tiny_f32"]
        e_ms, g_ms = tiny_latency(wl1)
        nb1 = wl1.num_kv_heads * algorithmic_bytes_per_pair(wl1.budget, wl1.group, wl1.head_dim, 4, True)
        emit("tiny_f32 (launch-latency bound), one call per step", wl1, e_ms, nb1)
        emit("tiny_f32 (launch-latency bound), 64 steps per HIP graph replay", wl1, g_ms, nb1)
    elif part == "qwen06":
        wl2 = WORKLOADS["qwen3_0p6b_layer"]
        ms, nb, win = steady_state(wl2, steps, warmup)
        emit("qwen3_0p6b_layer", wl2, ms, nb, windows=win, steps=steps)
        # the workload's whole run: a full 1024-token prompt, 4096 evicting
        # steps (5 consecutive windows; the mean of the windows is the run)
        ms, nb, win = steady_state(wl2, wl2.steps, 0)
        emit(f"qwen3_0p6b_layer whole run: {wl2.steps} evicting steps", wl2, float(np.mean(win)), nb,
             windows=win, steps=wl2.steps)
    elif part == "llama":
        for fill in (512, 1638, 3000):
            ms, nb, win = steady_state(wl3, steps, warmup, fill=fill)
            emit(f"llama8b_layer fill {fill} (appending)", wl3, ms, nb, windows=win, steps=steps)
        ms, nb, win = steady_state(wl3, steps, warmup)
        emit("llama8b_layer steady state", wl3, ms, nb, windows=win, steps=steps)
    elif part == "generation":
        # a whole 16k-token generation from a 512-token prompt, LongFlow vs full-KV
        ms_lf, nb_lf = trajectory(wl3, 16384, 512, "evict")
        ms_fk, nb_fk = trajectory(wl3, 16384, 512, "full")
        emit("llama8b_layer whole generation: prompt 512 + 16384 tokens, LongFlow", wl3, ms_lf, nb_lf,
             extra={"fill_steps": wl3.budget - 512}, steps=16384)
        emit("llama8b_layer whole generation: prompt 512 + 16384 tokens, full-KV", wl3, ms_fk, nb_fk,
             extra={"speedup_of_longflow": ms_fk / ms_lf}, steps=16384)
    elif part == "variants":
        for label, kw in (("deferred order (the blog engine's)", dict(order="deferred")),
                          ("one victim per sequence", dict(scope="sequence")),
                          ("one victim per sequence, deferred order", dict(scope="sequence", order="deferred")),
                          ("l2 score", dict(norm="l2"))):
            ms, nb, win = steady_state(wl3, steps, warmup, **kw)
            emit(f"llama8b_layer steady state, {label}", wl3, ms, nb, extra={"variant": kw},
                 windows=win, steps=steps)
    elif part == "churn":
        ms, nb = churn(wl3, min(steps, 256), warmup)
        emit("llama8b_layer churn: 4 sequences recycled every 16 steps (512-token prompts)", wl3, ms, nb,
             extra={"note": "reset + prefill inside the timed window; bytes include the prompts"},
             steps=min(steps, 256))
    elif part == "small":
        shard = wl3.with_(num_q_heads=4, num_kv_heads=1)
        ms, nb, win = steady_state(shard, steps, warmup)
        emit("llama8b_layer tp8 shard (1 KV head per GPU)", shard, ms, nb, windows=win, steps=steps)
        # small batches: fewer pairs than CUs, so every launch is split-K
        for b in (1, 4, 16):
            small = wl3.with_(batch=b)
            ms, nb, win = steady_state(small, steps, warmup)
            emit(f"llama8b_layer batch {b} (split-K)", small, ms, nb, windows=win, steps=steps)
        # just past a round of resident workgroups: stream launches
        for b, how in ((33, "256 workgroups of 8 waves, 8 pairs cut"),
                       (65, "512 workgroups of 4 waves, 8 pairs cut")):
            w = wl3.with_(batch=b)
            ms, nb, win = steady_state(w, steps, warmup)
            emit(f"llama8b_layer batch {b} (stream launch: {how})", w, ms, nb, windows=win, steps=steps)
    elif part == "ragged":
        # over the workload's 512-step window (fill levels advance through it)
        wl4 = ragged_stack()
        offsets = TokenStream(wl4).start_offsets()
        ms, nb, win = steady_state(wl4, wl4.steps, 5, layers=32,
                                   ragged=np.minimum(offsets, wl4.budget), seed=4)
        emit("llama8b_stack32_ragged LongFlow", wl4, ms, nb, 32,
             {"batch_rule": "largest batch with both caches in 0.95 x 288 GB",
              "evicting_seqs": int(np.sum(offsets >= wl4.budget))}, windows=win, steps=wl4.steps)
        ms, nb, win = steady_state(wl4, wl4.steps, 2, layers=32, mode="full",
                                   capacity=16384 + 512 + 64, ragged=offsets, seed=4)
        emit("llama8b_stack32_ragged full-KV", wl4, ms, nb, 32, windows=win, steps=wl4.steps)
    elif part == "gain":
        for w, ms, nb, win, extra in batch_gain(ragged_stack(), 50):
            emit(f"llama8b_stack32_ragged {extra.pop('method')} at its own largest batch", w, ms, nb, 32,
                 extra, windows=win, steps=50)
    elif part.startswith("qwen_b"):
        # Qwen3-8B stack at one budget of the sweep, every pair full: 512 model
        # steps (of the workload's 16,384; the GPU time of a suite run bounds
        # the window)
        budget = int(part[len("qwen_b"):])
        w = wl5.with_(budget=budget)
        ms, nb, win = steady_state(w, 512, 3, layers=36, seed=5)
        emit(f"qwen3_8b_stack36 B={budget}", w, ms, nb, 36, windows=win, steps=512)
    elif part == "cold":
        # one layer stepped back to back can keep part of its bytes in the
        # 256 MB last-level cache; in a model the other layers' reads replace
        # them between two steps of one layer
        for label, w in (("llama8b_layer", wl3), ("llama8b_layer tp8 shard", wl3.with_(num_q_heads=4, num_kv_heads=1)),
                         ("llama8b_layer batch 1", wl3.with_(batch=1)),
                         ("llama8b_layer batch 4", wl3.with_(batch=4)),
                         ("llama8b_layer batch 16", wl3.with_(batch=16)),
                         ("qwen3_0p6b_layer", WORKLOADS["qwen3_0p6b_layer"]),
                         ("qwen3_8b layer B=512", wl5.with_(budget=512))):
            warm_us, cold_us, nb = warm_vs_cold(w)
            emit(f"{label}, each step timed alone after a 1 GiB read (last-level cache cold)", w,
                 cold_us * 1e-3, nb, extra={"back_to_back_us_each_step_timed_alone": warm_us,
                                            "cold_over_back_to_back": cold_us / warm_us},
                 steps=COLD_STEPS)
    elif part == "qwen_graph":
        w = wl5.with_(budget=512)
        ms, nb, win = stack_graph(w, 36, 512, seed=5)
        emit("qwen3_8b_stack36 B=512, one HIP graph per model step", w, ms, nb, 36, windows=win,
             steps=512)
    else:
        raise ValueError(f"unknown suite part {part}")


TICK_US = 0.01          # the device's constant clock (s_memrealtime): 100 MHz


PHASES = ("first tile processed (interleaved) / K stream done (phased)", "stream done",
          "split part published and drained", "split part's ticket back",
          "last part: every part's max and sum in", "last part: score done", "in-place write reached")


def summarize_phase_records(rec, ph):
    """One launch's records ([wgs][4] and [wgs][8] int64,
    lf_probe_decode_phases): per phase the median over the workgroups that
    reached it, in us from the launch's first workgroup start; the last parts
    of split pairs apart."""
    rec = np.asarray(rec, dtype=np.int64)
    ph = np.asarray(ph, dtype=np.int64)
    t0 = rec[:, 0].min()
    us = lambda x: float(np.median((x - t0) * TICK_US)) if len(x) else None
    last = ph[:, 4] > 0                      # phase 5 reached: the last part of a pair
    out = {"workgroups": int(len(rec)), "span_us": float((rec[:, 1].max() - t0) * TICK_US),
           "last_start_us": float((rec[:, 0].max() - t0) * TICK_US), "phases": {}}
    for k, name in enumerate(PHASES, start=1):
        col = ph[:, k - 1]
        if (col > 0).any():                  # phases 5-7 of a split launch: its last parts only
            out["phases"][f"{k} {name}"] = us(col[col > 0])
    out["end_us"] = us(rec[last, 1] if last.any() else rec[:, 1])
    if last.any():
        out["other_parts_end_us"] = us(rec[~last, 1])
        out["last_parts"] = int(last.sum())
    return out


def phase_timing(args):
    """Phase records (lf_probe_decode_phases, in the measurement build
    liblongflow_phases.so) of the split-K shapes and two one-workgroup-per-pair
    layers: where one launch's time goes. One JSON line per case, from the
    launch with the median span of 7 (after warmup)."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache, lf_probe_decode_phases
    from decode_kv_cache_02_amd.synth import WORKLOADS, device_prefill
    w3 = WORKLOADS["llama8b_layer"]
    cases = [("llama8b_layer tp8 shard (64 pairs, 4 splits x 8 waves)", w3.with_(num_q_heads=4, num_kv_heads=1)),
             ("llama8b_layer batch 4 (32 pairs, 8 splits x 8 waves)", w3.with_(batch=4)),
             ("llama8b_layer batch 1 (8 pairs, 12 splits x 8 waves)", w3.with_(batch=1)),
             ("qwen3_0p6b_layer (256 pairs, one 8-wave workgroup each, interleaved)", WORKLOADS["qwen3_0p6b_layer"]),
             ("llama8b_layer steady state (512 pairs, one 4-wave workgroup each, phased)", w3)]
    for name, wl in cases:
        cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                              dtype=wl.dtype)
        try:
            k, v = device_prefill(wl, wl.budget, seed=wl.cfg_id)
            cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
            del k, v
            ring = make_ring(wl, wl.dtype)
            out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                              device="cuda")
            ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
            recs = torch.zeros((4096, 4), dtype=torch.int64, device="cuda")
            phs = torch.zeros((4096, 8), dtype=torch.int64, device="cuda")
            args_ = prepared_ring(cache, ring, out, ev)
            for t in range(30):
                cache.step_prepared(args_[t % RING][0])
            runs = []
            for t in range(7):
                recs.zero_()
                phs.zero_()
                q, kn, vn = ring[t % RING]
                n = lf_probe_decode_phases(cache.handle, 0, q, kn, vn, out, ev, recs, phs)
                torch.cuda.synchronize()
                runs.append(summarize_phase_records(recs[:n].cpu().numpy(), phs[:n].cpu().numpy()))
            runs.sort(key=lambda r: r["span_us"])
            r = runs[3]
            r["case"] = name
            print(json.dumps(r), flush=True)
        finally:
            cache.close()


def summarize_wg_records(rec):
    """Per-XCD and per-CU view of one launch's timing records ([wgs][4]
    int64: start, end, XCC id | hardware id << 32, workgroup; 100 MHz)."""
    rec = np.asarray(rec, dtype=np.int64)
    start, end = rec[:, 0], rec[:, 1]
    xcc = rec[:, 2] & 0xFFFF
    hw = (rec[:, 2] >> 32) & 0xFFFFFFFF
    cu_key = xcc * 256 + ((hw >> 8) & 0xFF)     # XCC, then the CU, SH and SE fields of HW_ID
    t0 = int(start.min())
    dur = (end - start) * TICK_US
    xcds = []
    for x in sorted(set(int(v) for v in xcc)):
        m = xcc == x
        xcds.append({"xcd": x, "workgroups": int(m.sum()), "mean_wg_us": float(dur[m].mean()),
                     "mean_end_us": float(((end[m] - t0) * TICK_US).mean()),
                     "last_end_us": float(((end[m] - t0) * TICK_US).max())})
    busy = []
    for k in set(int(v) for v in cu_key):
        iv = sorted(zip(start[cu_key == k], end[cu_key == k]))
        covered, cur_s, cur_e = 0, iv[0][0], iv[0][1]
        for a, b in iv[1:]:
            if a > cur_e:
                covered += cur_e - cur_s
                cur_s, cur_e = a, b
            else:
                cur_e = max(cur_e, b)
        covered += cur_e - cur_s
        busy.append(covered)
    span = (int(end.max()) - t0) * TICK_US
    ends = [x["last_end_us"] for x in xcds]
    return {"workgroups": int(len(rec)), "span_us": span, "mean_wg_us": float(dur.mean()),
            "cus": len(busy), "workgroups_per_cu_max": int(np.bincount(
                np.unique(cu_key, return_inverse=True)[1]).max()),
            "cu_busy_frac_mean": float(np.mean(busy) * TICK_US / span),
            "xcd_last_end_spread_us": float(max(ends) - min(ends)), "xcd": xcds}


def wg_timing(args):
    """Per-workgroup timing records (lf_probe_decode_timing,
    lf_probe_stream_read_timing) of the decode kernel on the benchmark shapes
    and of the bare streaming read over the same bytes: how each launch
    spreads over the XCDs. One JSON line per case: the launch with the median
    span of 5 recorded launches (after warmup)."""
    import torch
    from decode_kv_cache_02_amd.native import (LongFlowCache, lf_probe_decode_timing,
                                               lf_probe_stream_read_timing)
    from decode_kv_cache_02_amd.synth import WORKLOADS, device_prefill
    w3 = WORKLOADS["llama8b_layer"]
    cases = [("llama8b_layer steady state", w3),
             ("llama8b_layer tp8 shard", w3.with_(num_q_heads=4, num_kv_heads=1)),
             ("qwen3_8b layer B=512 (batch 256)", WORKLOADS["qwen3_8b_stack36_ties"].with_(budget=512))]
    for name, wl in cases:
        e = 2 if wl.dtype == "bf16" else 4
        cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                              dtype=wl.dtype)
        try:
            k, v = device_prefill(wl, wl.budget, seed=wl.cfg_id)
            cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
            del k, v
            ring = make_ring(wl, wl.dtype)
            out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=ring[0][0].dtype,
                              device="cuda")
            ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
            recs = torch.zeros((wl.batch * wl.num_kv_heads * 16, 4), dtype=torch.int64, device="cuda")
            args_ = prepared_ring(cache, ring, out, ev)
            for t in range(20):
                cache.step_prepared(args_[t % RING][0])
            runs = []
            for t in range(5):
                q, kn, vn = ring[t % RING]
                n = lf_probe_decode_timing(cache.handle, 0, q, kn, vn, out, ev, recs)
                torch.cuda.synchronize()
                runs.append(summarize_wg_records(recs[:n].cpu().numpy()))
            runs.sort(key=lambda r: r["span_us"])
            r = runs[2]
            nb = wl.batch * wl.num_kv_heads * algorithmic_bytes_per_pair(
                wl.budget, wl.group, wl.head_dim, e, True)
            r.update({"case": f"decode_kernel, {name}", "algorithmic_bytes": nb,
                      "GBs_over_span": nb / r["span_us"] / 1e3})
            print(json.dumps(r), flush=True)
        finally:
            cache.close()
    for name, total, wgs in (("read probe, the Llama-8B layer's bytes", 860_160_000, 512),
                             ("read probe, the Qwen3-8B B=512 layer's bytes", 537_001_984, 2048)):
        total -= total % (16 * wgs)
        buf = torch.ones(total // 2, dtype=torch.int16, device="cuda")
        sink = torch.empty(wgs * 256 * 4, dtype=torch.int32, device="cuda")
        recs = torch.zeros((wgs, 4), dtype=torch.int64, device="cuda")
        runs = []
        for t in range(8):
            lf_probe_stream_read_timing(buf, wgs, sink, recs)
            torch.cuda.synchronize()
            if t >= 3:
                runs.append(summarize_wg_records(recs.cpu().numpy()))
        runs.sort(key=lambda r: r["span_us"])
        r = runs[2]
        r.update({"case": f"{name} ({wgs} workgroups)", "algorithmic_bytes": total,
                  "GBs_over_span": total / r["span_us"] / 1e3})
        print(json.dumps(r), flush=True)
        del buf, sink, recs


def main():
    args = parse_args()
    if args.wg_timing:
        import torch
        torch.cuda.set_device(0)
        wg_timing(args)
        return
    if args.batch_sweep:
        import torch
        torch.cuda.set_device(0)
        batch_sweep(args)
        return
    if args.stack_trajectory:
        import torch
        torch.cuda.set_device(0)
        from decode_kv_cache_02_amd.synth import WORKLOADS
        w = WORKLOADS["qwen3_8b_stack36_ties"].with_(budget=args.stack_trajectory)
        r = stack_trajectory(w, 36, w.steps, w.prefill)
        ms = r["ms_per_model_step"]
        line = {"workload": f"qwen3_8b_stack36 B={w.budget}, whole generation: prompt {w.prefill} + "
                            f"{w.steps} model steps", "batch": w.batch, "layers": 36, "budget": w.budget,
                "ms_per_model_step": ms, "tokens_per_s": w.batch / ms * 1e3,
                "achieved_GBs": r["bytes_per_model_step"] / ms / 1e6,
                "frac_of_peak": r["bytes_per_model_step"] / ms / 1e6 / HBM_PEAK_GBS}
        line.update({k: v for k, v in r.items() if k != "ms_per_model_step"})
        if "evict_ms_per_model_step" in r:
            line["evict_achieved_GBs"] = r["evict_bytes_per_model_step"] / r["evict_ms_per_model_step"] / 1e6
        print(json.dumps(line), flush=True)
        return
    if args.phases:
        # the measurement build: the library with phase stamps compiled in
        from decode_kv_cache_02_amd import native
        native.load_library(native.PHASES_LIB_PATH)
        import torch
        torch.cuda.set_device(0)
        phase_timing(args)
        return
    if args.suite_part:
        import torch
        torch.cuda.set_device(0)
        suite_part(args.suite_part, args)
        return
    if args.suite:
        # the oracle lines first (their workers are forked); this process
        # never touches the GPU, each group of GPU lines runs in a child
        if not args.no_cpu_baseline:
            cpu_suite(min(args.cpu_seconds, 6.0))
        suite(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(each (sequence, KV head) pair is independent: a multi-GPU run would shard "
              f"the batch with no exchange).", file=sys.stderr)
        sys.exit(2)
    from decode_kv_cache_02_amd.synth import WORKLOADS, device_prefill

    wl = WORKLOADS[args.workload]
    if args.budget:
        wl = wl.with_(budget=args.budget)
    if args.batch:
        wl = wl.with_(batch=args.batch)
    if args.kv_heads:
        wl = wl.with_(num_kv_heads=args.kv_heads, num_q_heads=args.kv_heads * wl.group)
    e = 2 if wl.dtype == "bf16" else 4
    # The CPU baseline forks one worker per host core, so it runs before this
    # process touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)
        print(f"[bench] cpu oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)

    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache, lf_probe_hbm_attributes
    torch.cuda.set_device(0)
    print(f"[bench] {wl.name}: batch {wl.batch}, {wl.num_q_heads}/{wl.num_kv_heads} heads, "
          f"d {wl.head_dim}, B {wl.budget}, {wl.dtype}", file=sys.stderr, flush=True)

    cache = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype, mode="evict")
    k, v = device_prefill(wl, wl.budget, seed=wl.cfg_id)
    cache.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
    del k, v
    ring = make_ring(wl, wl.dtype)
    dt = ring[0][0].dtype
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=dt, device="cuda")
    ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    ms, windows = time_steps(cache, ring, out, ev, args.steps, args.warmup)
    ev_host = ev.cpu().numpy()
    assert np.all(ev_host >= 0), "steady state must evict on every pair"
    pairs = wl.batch * wl.num_kv_heads
    bytes_launch = pairs * algorithmic_bytes_per_pair(wl.budget, wl.group, wl.head_dim, e, True)
    achieved = bytes_launch / ms / 1e6            # GB/s
    steps_per_s = 1e3 / ms
    traffic = load_traffic(bytes_launch)
    print(f"[bench] {ms * 1e3:.1f} us/step, {achieved:.0f} GB/s algorithmic", file=sys.stderr,
          flush=True)

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cache.close()
    ceiling = stream_read_ceiling(int(bytes_launch))
    print(f"[bench] streaming-read ceiling: {ceiling:.0f} GB/s", file=sys.stderr, flush=True)
    full = None
    llc = None
    if not args.no_full_kv:
        full = full_kv_baseline(wl, min(args.steps, 200), 10)
        print(f"[bench] full-KV: {json.dumps(full['at_fill'])}", file=sys.stderr, flush=True)
        # does the measured layer owe anything to the last-level cache? (in a
        # model, other layers' reads pass between two steps of one layer)
        warm_us, cold_us, _ = warm_vs_cold(wl)
        llc = {"back_to_back_us": warm_us, "after_1GiB_read_us": cold_us,
               "ratio": cold_us / warm_us,
               "note": "each step timed alone by an event pair, back to back and right after a "
                       "1 GiB read of an unrelated buffer (256 MB last-level cache cold); "
                       "not part of value"}
        print(f"[bench] last-level cache: {warm_us:.1f} us back to back, {cold_us:.1f} us cold",
              file=sys.stderr, flush=True)
    mem_clock_khz, bus_bits = lf_probe_hbm_attributes()
    per_transfer = mem_clock_khz * 1e3 * bus_bits / 8 / 1e9     # GB/s at one transfer per clock
    line = {
        "metric": METRIC,
        "value": steps_per_s * wl.batch,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "budget": wl.budget, "fill": wl.budget,
                   "phase": "steady state: every pair full, one eviction per pair per step"},
        "steps_per_s": steps_per_s,
        "timing": {"ms_per_step": "median of 5 consecutive windows of steps/5 steps each, "
                                  "HIP events on the stream the kernels run on",
                   "ms_windows": windows, "ms_mean": float(np.mean(windows))},
        "hbm_peak_device": {
            "memory_clock_khz": mem_clock_khz, "bus_width_bits": bus_bits,
            "GBs_at_2_transfers_per_clock": 2 * per_transfer,
            "GBs_at_4_transfers_per_clock": 4 * per_transfer,
            "consistent_with_measured": [k for k, m in (("2 per clock", 2), ("4 per clock", 4))
                                         if m * per_transfer >= achieved],
            "note": "clock x bus width / 8 per transfer, from the device attributes; a rate "
                    "below the measured algorithmic GB/s is ruled out. roofline.peak stays "
                    "the 8 TB/s vendor figure"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_launch,
                     "kernel": "decode_kernel (lf_decode_step)", "kernel_sha": kernel_sha()},
        "cpu_baseline": cpu,
        "stream_read_ceiling": {
            "GBs": ceiling, "frac_of_peak": ceiling / HBM_PEAK_GBS,
            "decode_frac_of_ceiling": achieved / ceiling,
            "kernel": "lf_probe_stream_read: the decode kernel's 16-byte non-temporal buffer loads, "
                      "512 workgroups over the same bytes as one launch"},
        "full_kv": full,
        "last_level_cache_check": llc,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
