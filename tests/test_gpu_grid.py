"""GPU parity when a workgroup takes several units of work in turn.

A launch with more units (pairs, or pairs x splits) than fit on the device
at once gets as many workgroups as fit, each taking units w, w + grid, ...
lf_cache_set_grid caps the grid so that small shapes take the same path:
every loop, wave count, split count and variant runs here with a handful of
workgroups. A full Llama-8B layer at batch 102 (816 pairs) takes it on its
own, and with -1 (one workgroup per unit) for comparison. Same lockstep
protocol and tolerances as test_gpu_parity.
"""
import pytest

from decode_kv_cache_02_amd.synth import WORKLOADS
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
])
@pytest.mark.parametrize("grid", [1, 2, 5])
@pytest.mark.parametrize("waves,loop", [(4, "phased"), (8, "phased"), (4, "interleaved"),
                                        (8, "interleaved")])
def test_small_shapes_capped_grid(dtype, G, d, budget, prefill, steps, grid, waves, loop):
    """6 pairs on 1, 2 or 5 workgroups."""
    wl = SMALL.with_(dtype=dtype, num_q_heads=2 * G, head_dim=d, budget=budget, prefill=prefill,
                     steps=steps)
    _say(f"{dtype} G={G} d={d} B={budget} prefill={prefill} steps={steps} grid={grid} "
         f"waves={waves} {loop}")
    rep = run_lockstep(wl, steps, check_cache_every=10, waves=waves, loop=loop, grid=grid)
    assert rep.steps == steps


@pytest.mark.parametrize("splits,grid", [(3, 1), (3, 4), (5, 7)])
@pytest.mark.parametrize("loop", ["phased", "interleaved"])
def test_split_units_on_few_workgroups(splits, grid, loop):
    """6 pairs x splits units: a workgroup may hold two splits of one pair,
    the last split of one pair and a first of another, in any order."""
    wl = SMALL.with_(dtype="bf16", num_q_heads=8, head_dim=128, budget=300, prefill=280, steps=30)
    _say(f"bf16 G=4 B=300 prefill 280, {splits} splits on {grid} workgroups, {loop}")
    rep = run_lockstep(wl, 30, splits=splits, check_cache_every=10, loop=loop, grid=grid)
    assert rep.steps == 30


@pytest.mark.parametrize("order,scope", [("deferred", "kv_head"), ("same_step", "sequence"),
                                         ("deferred", "sequence")])
@pytest.mark.parametrize("grid", [1, 4])
def test_variants_on_few_workgroups(order, scope, grid):
    """One victim per sequence: the sequence's KV heads may be taken by one
    workgroup one after the other; the last to finish decides for all."""
    wl = SMALL.with_(dtype="bf16", num_q_heads=8, head_dim=128, budget=200, prefill=190, steps=30)
    _say(f"bf16 G=4 B=200, {order} order, {scope} scope, grid {grid}")
    rep = run_lockstep(wl, 30, order=order, scope=scope, check_cache_every=10, grid=grid)
    assert rep.steps == 30


def test_full_mode_capped_grid():
    wl = SMALL.with_(dtype="bf16", num_q_heads=8, head_dim=128, budget=2200, prefill=2040)
    _say("bf16 FULL mode, capacity 2200, prefill 2040, grid 2")
    rep = run_lockstep(wl, 20, mode="full", capacity=2200, check_cache_every=10, grid=2)
    assert rep.appends == 20 * 6


@pytest.mark.parametrize("grid", [0, -1])
def test_llama8b_layer_816_pairs(grid):
    """Batch 102 x 8 KV heads = 816 pairs, every sequence full: the automatic
    launch (grid 0) runs 408 workgroups of 2 pairs each instead of a full
    round of 512 and a partial one; -1 gives each pair its own workgroup."""
    wl = WORKLOADS["llama8b_layer"].with_(batch=102, prefill=3277)
    pairs = [(0, 0), (101, 7), (51, 3), (50, 4), (77, 1), (25, 6), (90, 2), (13, 5)]
    _say(f"llama8b layer, batch 102, B 3277 full, 8 steps, {len(pairs)} sampled pairs, grid {grid}")
    rep = run_lockstep(wl, 8, pairs=pairs, check_cache_every=8, grid=grid)
    assert rep.evictions == 8 * len(pairs)


@pytest.mark.parametrize("grid", [0, 512])
def test_qwen3_8b_layer_2048_pairs(grid):
    """Batch 256 x 8 KV heads = 2048 pairs: four whole rounds, one workgroup
    per pair by default; 512 forces four pairs per workgroup."""
    wl = WORKLOADS["qwen3_8b_stack36_ties"].with_(budget=512, prefill=512)
    pairs = [(0, 0), (255, 7), (64, 3), (128, 5), (191, 1), (37, 6), (200, 2), (99, 4)]
    _say(f"qwen3_8b layer, batch 256, B 512, 12 steps, {len(pairs)} sampled pairs, grid {grid}")
    rep = run_lockstep(wl, 12, pairs=pairs, check_cache_every=12, grid=grid)
    assert rep.evictions == 12 * len(pairs)
