"""GPU parity when workgroups take several pairs in turn, and of stream
launches (pairs cut into runs of tiles shared evenly by the workgroups).

The evicting main path (4 waves per workgroup, same-step order, one victim
per KV head, no split) has a second kernel whose workgroups take pairs w,
w + grid, w + 2 grid, ... The runtime uses it where one workgroup per pair
would take two rounds of resident workgroups with the second 40-85% full
(the 32-layer ragged stack's 816-pair layers; the Llama-8B layer at batch
96);
lf_cache_set_grid caps the grid so that small shapes run it too. Every
dtype, head size, group width and both loops run here on a handful of
workgroups, through fill and eviction, against the oracle (the lockstep
protocol and tolerances of test_gpu_parity). Launches the kernel does not
serve (8 waves, split-K, the variants, FULL mode) ignore the cap, and a
full-shape layer gives the same bits with the automatic grid as with one
workgroup per pair.
"""
import numpy as np
import pytest

from decode_kv_cache_02_amd.synth import WORKLOADS, TokenStream
from lockstep import run_lockstep

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd import native
    native.load_library()
    yield


SMALL = WORKLOADS["tiny_f32"].with_(batch=3, num_kv_heads=2)


@pytest.mark.parametrize("dtype,G,d,budget,prefill,steps", [
    ("bf16", 4, 128, 100, 90, 30),       # fill -> evict
    ("f32", 2, 64, 300, 300, 20),
    ("bf16", 1, 128, 1100, 1100, 12),    # past the interleaved loop's 1024 slots
    ("f32", 4, 128, 70, 70, 12),
    ("bf16", 2, 64, 64, 40, 30),
])
@pytest.mark.parametrize("grid", [1, 2, 5])
@pytest.mark.parametrize("loop", ["phased", "interleaved"])
def test_small_shapes_capped_grid(dtype, G, d, budget, prefill, steps, grid, loop):
    """6 pairs on 1, 2 or 5 workgroups of 4 waves."""
    wl = SMALL.with_(dtype=dtype, num_q_heads=2 * G, head_dim=d, budget=budget, prefill=prefill,
                     steps=steps)
    _say(f"{dtype} G={G} d={d} B={budget} prefill={prefill} steps={steps} grid={grid} {loop}")
    rep = run_lockstep(wl, steps, check_cache_every=10, waves=4, loop=loop, grid=grid)
    assert rep.steps == steps


def test_ragged_fills_on_few_workgroups():
    """Pairs of different lengths (empty, one tile, ragged, full) taken in
    turn by 2 workgroups: each unit bounds its own stream."""
    wl = WORKLOADS["tiny_f32"].with_(dtype="bf16", batch=6, num_q_heads=8, num_kv_heads=2,
                                     head_dim=128, budget=300)
    n = np.array([0, 1, 16, 150, 299, 300], dtype=np.int32)
    _say("bf16 G=4 B=300, fills 0..300, 2 workgroups, 24 steps")
    rep = run_lockstep(wl, 24, prefill_n=n, check_cache_every=8, waves=4, grid=2)
    assert rep.steps == 24


@pytest.mark.parametrize("kw", [dict(waves=8), dict(splits=3), dict(order="deferred"),
                                dict(scope="sequence"), dict(mode="full", capacity=400)],
                         ids=["8 waves", "split-K", "deferred", "sequence", "full"])
def test_other_launches_ignore_the_cap(kw):
    """Launches the units kernel does not serve keep one workgroup per unit
    under a cap of 1 and stay exact."""
    wl = SMALL.with_(dtype="bf16", num_q_heads=8, head_dim=128, budget=300, prefill=280, steps=20)
    _say(f"bf16 G=4 B=300 prefill 280, {kw}, grid 1")
    rep = run_lockstep(wl, 20, check_cache_every=10, grid=1, **kw)
    assert rep.steps == 20


@pytest.mark.parametrize("batch", [96, 102])
def test_llama8b_layer_partial_round_is_bit_identical(batch):
    """The Llama-8B layer at batch 96 and 102 (768 and 816 pairs; 512
    workgroups of 4 waves fit at once): the automatic launch cuts the grid
    to 384 and 408 workgroups of two pairs each. Outputs, slots and the whole
    cache match one workgroup per pair bit for bit over 6 steps."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache, lf_probe_decode_timing
    from decode_kv_cache_02_amd.synth import device_prefill, device_steps
    wl = WORKLOADS["llama8b_layer"].with_(batch=batch)
    _say(f"llama8b layer batch {batch}: automatic grid vs one workgroup per pair, 6 steps")
    caches = [LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                            dtype=wl.dtype) for _ in range(2)]
    try:
        caches[1].set_grid(-1)
        k, v = device_prefill(wl, wl.budget, seed=3)
        fills = np.full(wl.batch, wl.budget, dtype=np.int32)
        fills[::7] = wl.budget - 40       # a few pairs append, the rest evict
        for c in caches:
            c.prefill(0, k, v, fills)
        del k, v
        Q, KN, VN = device_steps(wl, 6, seed=4)
        outs = [[], []]
        for q, kn, vn in zip(Q, KN, VN):
            for i, c in enumerate(caches):
                out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                                  device="cuda")
                ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
                c.decode_step(0, q, kn, vn, out, ev)
                outs[i].append((out, ev))
        torch.cuda.synchronize()
        for (o0, e0), (o1, e1) in zip(*outs):
            assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
            assert torch.equal(e0, e1)
        s0, s1 = caches[0].snapshot(0), caches[1].snapshot(0)
        for a, b in zip(s0, s1):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
        # the automatic launch did cut the grid
        rec = torch.zeros((wl.batch * wl.num_kv_heads, 4), dtype=torch.int64, device="cuda")
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
        wgs = lf_probe_decode_timing(caches[0].handle, 0, Q[0], KN[0], VN[0], out, ev, rec)
        torch.cuda.synchronize()
        assert wgs == wl.batch * wl.num_kv_heads // 2
    finally:
        for c in caches:
            c.close()


# ---------------- Stream launches ----------------
# Every pair of a small layer cut into runs of `tiles` 16-slot tiles: a pair
# may be held whole by one workgroup or cut into up to 16 parts, and a
# workgroup's run may end one pair and start the next. Split count 1 and 4
# waves (the stream launch serves one-workgroup-per-pair launches of 4 waves).

@pytest.mark.parametrize("dtype,G,d,budget,prefill,steps", [
    ("bf16", 4, 128, 100, 90, 24),       # 7 tiles per pair, fill -> evict
    ("f32", 2, 64, 300, 300, 16),        # 19 tiles
    ("bf16", 1, 128, 1100, 1100, 10),    # 69 tiles: parts of at least 5 tiles
    ("bf16", 2, 64, 64, 40, 30),         # 3 -> 4 tiles
])
@pytest.mark.parametrize("tiles", [1, 3, 8])
@pytest.mark.parametrize("loop", ["phased", "interleaved"])
def test_stream_small_shapes(dtype, G, d, budget, prefill, steps, tiles, loop):
    wl = SMALL.with_(dtype=dtype, num_q_heads=2 * G, head_dim=d, budget=budget, prefill=prefill,
                     steps=steps)
    _say(f"stream: {dtype} G={G} d={d} B={budget} prefill={prefill} steps={steps} "
         f"{tiles} tiles per workgroup, {loop}")
    rep = run_lockstep(wl, steps, check_cache_every=8, splits=1, waves=4, loop=loop, stream=tiles)
    assert rep.steps == steps


@pytest.mark.parametrize("tiles", [2, 5])
def test_stream_small_shapes_eight_waves(tiles):
    wl = SMALL.with_(dtype="bf16", num_q_heads=8, head_dim=128, budget=300, prefill=290, steps=20)
    _say(f"stream: bf16 G=4 B=300, 8 waves, {tiles} tiles per workgroup, 20 steps")
    rep = run_lockstep(wl, 20, check_cache_every=10, splits=1, waves=8, stream=tiles)
    assert rep.steps == 20


def test_stream_ragged_fills():
    """Pairs of different lengths (empty, one slot, one tile, ragged, full):
    runs planned on the longest pair leave some parts without slots."""
    wl = WORKLOADS["tiny_f32"].with_(dtype="bf16", batch=6, num_q_heads=8, num_kv_heads=2,
                                     head_dim=128, budget=300)
    n = np.array([0, 1, 16, 150, 299, 300], dtype=np.int32)
    _say("stream: bf16 G=4 B=300, fills 0..300, 5 tiles per workgroup, 24 steps")
    rep = run_lockstep(wl, 24, prefill_n=n, check_cache_every=8, splits=1, waves=4, stream=5)
    assert rep.steps == 24


def _grid_of(wl, cache):
    """Workgroups of one decode launch of `cache` (timing probe), on
    throw-away inputs of a copy of its state."""
    import torch
    from decode_kv_cache_02_amd.native import lf_probe_decode_timing
    from decode_kv_cache_02_amd.synth import device_steps
    Q, KN, VN = device_steps(wl, 1, seed=9)
    # room for a stream launch, which may run more workgroups than pairs
    rec = torch.zeros((max(wl.batch * wl.num_kv_heads, 4096), 4), dtype=torch.int64, device="cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
    wgs = lf_probe_decode_timing(cache.handle, 0, Q[0], KN[0], VN[0], out, ev, rec)
    torch.cuda.synchronize()
    return wgs


@pytest.mark.parametrize("batch,grid", [(33, 256), (65, 512), (72, 512)])
def test_llama8b_layer_stream_launch(batch, grid):
    """The Llama-8B layer at batch 33, 65 and 72 (264, 520 and 576 pairs):
    whole pairs would leave a round of resident workgroups mostly idle, so
    the automatic launch streams. At batch 33, 256 workgroups of 8 waves
    each take a whole pair and share the last 8 pairs' tiles; at 65 and 72,
    512 workgroups of 4 waves each take a whole pair and then a run of the
    last 8 or 64 pairs' tiles. Sampled pairs, among them cut ones (the last
    sequences), follow the oracle through the fill -> evict boundary."""
    from decode_kv_cache_02_amd.native import LongFlowCache
    wl = WORKLOADS["llama8b_layer"].with_(batch=batch)
    probe = LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                          dtype=wl.dtype)
    try:
        from decode_kv_cache_02_amd.synth import device_prefill
        k, v = device_prefill(wl, wl.budget, seed=3)
        probe.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
        del k, v
        assert _grid_of(wl, probe) == grid
    finally:
        probe.close()
    last = batch - 1
    pairs = [(0, 0), (last, 7), (last, 0), (last - 1, 3), (batch // 2, 5), (7, 6), (last, 4),
             (batch - 8, 1)]
    n = np.full(wl.batch, 3270, dtype=np.int32)
    _say(f"stream: llama8b layer batch {batch}, prefill 3270, 14 steps, pairs {pairs}")
    rep = run_lockstep(wl, 14, pairs=pairs, prefill_n=n, check_cache_every=14)
    assert rep.appends == 7 * len(pairs) and rep.evictions == 7 * len(pairs)


def test_stream_launch_noalloc_is_bit_identical():
    """lf_decode_step_noalloc takes the same stream launch with its workspace
    in the static array: outputs, slots and cache bit for bit."""
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import device_prefill, device_steps
    wl = WORKLOADS["llama8b_layer"].with_(batch=65)
    _say("stream: llama8b layer batch 65, lf_decode_step vs lf_decode_step_noalloc, 4 steps")
    caches = [LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget,
                            dtype=wl.dtype) for _ in range(2)]
    try:
        k, v = device_prefill(wl, wl.budget, seed=5)
        for c in caches:
            c.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
        del k, v
        Q, KN, VN = device_steps(wl, 4, seed=6)
        outs = [[], []]
        for q, kn, vn in zip(Q, KN, VN):
            for i, c in enumerate(caches):
                out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                                  device="cuda")
                ev = torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
                c.decode_step(0, q, kn, vn, out, ev, noalloc=(i == 1))
                outs[i].append((out, ev))
        torch.cuda.synchronize()
        for (o0, e0), (o1, e1) in zip(*outs):
            assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
            assert torch.equal(e0, e1)
        for a, b in zip(caches[0].snapshot(0), caches[1].snapshot(0)):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    finally:
        for c in caches:
            c.close()
