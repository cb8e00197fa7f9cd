"""Whole trajectories at the workloads' full shapes, checked against the oracle
on 8 sampled pairs (tests/trajectory.py): every step's output rows and evicted
slot, and the pairs' cache regions every 1024 steps.

  * Llama-8B layer: batch 64, 32/8 heads, B = 3277, prompt 512, then 16,384
    steps with the automatic launch. The pairs fill for 2,765 steps and evict
    from then on (LongFlow Guide, §Static Memory Pre-Allocation and In-Place
    Eviction, items 1-3: fill, then evict every step); the launch moves from
    the interleaved loop to the phased one when the cache passes 1024 slots.
  * Qwen3-0.6B layer: batch 32, 16/8 heads, B = 1024, full prompt, all 4,096
    evicting steps.
  * Qwen3-8B layer at batch 256 with 10% duplicated tokens at every budget of
    the sweep, B = 512, 1024, 2048 and 4096 (the suite's one-workgroup-per-pair
    launches): prompt 512, then all 16,384 steps, filling up to the budget and
    evicting from then on. Duplicates make exact score ties; each must go to
    the lowest slot.
  * Split-K over the Llama-8B layer's whole trajectory: one GPU's share under
    8-way tensor parallelism (64 pairs of one KV head) and batch 1 (8 pairs,
    all checked). The planned split count grows with the cache (2 splits at
    512 slots; 4 and 12 once it is full), so the trajectory crosses launch
    shapes as well as the fill -> evict boundary.
  * Stream launches over the Llama-8B layer's whole trajectory: batch 65
    (520 pairs, 4-wave workgroups), batch 33 (264 pairs, 8-wave) and batch
    129 (1032 pairs, two whole pairs per workgroup first), 8 pairs cut
    between workgroups every step; four cut and four whole pairs checked.
  * The full-KV baseline growing past 16k tokens (14,976 -> 16,896, the
    Llama-8B layer at batch 8: split-K, each split streaming its ~4k slots
    in 2048-slot LDS chunks).
  * The variants of the cache over whole trajectories: the deferred order
    and the l2 score on the Llama-8B layer (8 pairs), and one victim per
    sequence on the Qwen3-0.6B layer (two sequences, every KV head), in
    either order.
Each test prints its near-tie and exact-tie counts.
"""
import pytest

from decode_kv_cache_02_amd.synth import WORKLOADS
import trajectory

pytestmark = pytest.mark.gpu


def _run(wl, steps, prefill, check_every=1024, pairs=8, seed=0, mode="evict",
         sampled=None, **variant):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if sampled is None:
        sampled = trajectory.sample_pairs(wl, pairs, seed=seed)
    print(f"\n[case] {wl.name} {mode} {variant or ''} B={wl.budget} batch={wl.batch} "
          f"{wl.num_q_heads}/{wl.num_kv_heads}: prompt {prefill}, {steps} steps, "
          f"pairs {sampled}", flush=True)
    rec = trajectory.record_trajectory(wl, steps, sampled, prefill, check_every=check_every,
                                       mode=mode, **variant)
    print(f"[case] recorded; checking {len(sampled)} pairs in the oracle", flush=True)
    reports = trajectory.check_trajectory(rec)
    print(trajectory.summary(rec, reports), flush=True)
    return reports


def test_llama8b_layer_whole_trajectory():
    wl = WORKLOADS["llama8b_layer"]
    reports = _run(wl, wl.steps, wl.prefill, seed=3)
    fill_steps = wl.budget - wl.prefill
    for r in reports:
        assert r.appends == fill_steps and r.evictions == wl.steps - fill_steps
        assert r.fill_to_evict_step == fill_steps
        assert r.snapshots == wl.steps // 1024


def test_qwen3_0p6b_layer_whole_trajectory():
    wl = WORKLOADS["qwen3_0p6b_layer"]
    reports = _run(wl, wl.steps, wl.budget, seed=2)
    for r in reports:
        assert r.evictions == wl.steps and r.appends == 0


@pytest.mark.parametrize("budget", [512, 1024, 2048, 4096])
def test_qwen3_8b_layer_budget_with_ties(budget):
    wl = WORKLOADS["qwen3_8b_stack36_ties"].with_(budget=budget)
    reports = _run(wl, wl.steps, wl.prefill, check_every=2048, seed=5)
    for r in reports:
        assert r.appends == budget - wl.prefill and r.evictions == wl.steps - r.appends
    exact = sum(r.exact_ties for r in reports)
    assert exact > 0
    assert sum(r.tie_lowest_index for r in reports) == exact


def _check_fill_then_evict(wl, reports):
    fill_steps = wl.budget - wl.prefill
    for r in reports:
        assert r.appends == fill_steps and r.evictions == wl.steps - fill_steps
        assert r.fill_to_evict_step == fill_steps


def test_tp8_shard_whole_trajectory():
    wl = WORKLOADS["llama8b_layer"].with_(num_q_heads=4, num_kv_heads=1)
    _check_fill_then_evict(wl, _run(wl, wl.steps, wl.prefill, seed=7))


def test_llama8b_batch1_whole_trajectory():
    wl = WORKLOADS["llama8b_layer"].with_(batch=1)
    _check_fill_then_evict(wl, _run(wl, wl.steps, wl.prefill, seed=1))


@pytest.mark.parametrize("batch", [65, 33, 129])
def test_llama8b_stream_launch_whole_trajectory(batch):
    # Batch 65: 520 pairs, 8 past the 512 resident 4-wave workgroups. Batch
    # 33: 264 pairs, 8 past one 8-wave workgroup per compute unit. Batch 129:
    # 1032 pairs, each workgroup takes two whole pairs first. Every step
    # is a stream launch whose last 8 pairs (the last sequence) are cut into
    # parts and combined like split-K, through the fill, the interleaved ->
    # phased switch at 1024 slots and eviction. Four cut pairs, four whole.
    wl = WORKLOADS["llama8b_layer"].with_(batch=batch)
    last = batch - 1
    sampled = [(0, 0), (11, 3), (last // 2, 6), (last - 1, 7), (last, 0), (last, 3), (last, 5), (last, 7)]
    _check_fill_then_evict(wl, _run(wl, wl.steps, wl.prefill, seed=9, sampled=sampled))


def test_full_kv_growing_past_16k():
    wl = WORKLOADS["llama8b_layer"].with_(batch=8)
    prompt, steps = 14976, 1920
    reports = _run(wl, steps, prompt, check_every=640, seed=4, mode="full")
    for r in reports:
        assert r.appends == steps and r.evictions == 0 and r.snapshots == 3


def test_llama8b_stack32_ragged_window():
    """The 32-layer ragged stack at the batch where its cache and the full-KV
    cache both fit 0.95 x 288 GB, over the workload's 512-step window: every
    layer steps every model step; layers 0 and 17 are checked on 8 pairs of
    sequences that are full, partial, and one that reaches the budget inside
    the window."""
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd.native import lf_cache_bytes, make_config
    from decode_kv_cache_02_amd.synth import TokenStream
    wl = WORKLOADS["llama8b_stack32_ragged"]
    per_seq = (lf_cache_bytes(make_config(32, 1, 32, 8, 128, wl.budget))
               + lf_cache_bytes(make_config(32, 1, 32, 8, 128, 16384 + 512 + 64, mode="full")))
    wl = wl.with_(batch=int(0.95 * 288e9 // per_seq))
    fills = np.minimum(TokenStream(wl).start_offsets(), wl.budget).astype(np.int32)
    full = [int(b) for b in np.flatnonzero(fills == wl.budget)[:4]]
    crossing = [int(b) for b in np.flatnonzero((fills < wl.budget) & (fills > wl.budget - 400))[:1]]
    short = [int(b) for b in np.flatnonzero(fills < wl.budget - 600)[:3]]
    seqs = full + crossing + short
    assert len(seqs) == 8 and crossing
    pairs = [(b, h) for b, h in zip(seqs, (0, 7, 3, 5, 1, 2, 6, 4))]
    print(f"\n[case] llama8b stack32 ragged, batch {wl.batch}, 512 steps, layers 0 and 17, "
          f"pairs {pairs}, fills {[int(fills[b]) for b in seqs]}", flush=True)
    rec = trajectory.record_trajectory(wl, wl.steps, pairs, fills, check_every=256,
                                       num_layers=32, layers=(0, 17))
    reports = trajectory.check_trajectory(rec)
    print(trajectory.summary(rec, reports), flush=True)
    for r in reports:
        b = r.pair[1]
        assert r.appends == max(0, min(wl.steps, wl.budget - int(fills[b])))
        assert r.appends + r.evictions == wl.steps


def test_llama8b_layer_deferred_order_whole_trajectory():
    """The Guide engine's order: the new token takes the slot chosen at the
    step before (the last slot when none was chosen), then the next victim is
    picked (LongFlow Guide, §End-to-End Implementation, the cache's step)."""
    wl = WORKLOADS["llama8b_layer"]
    reports = _run(wl, wl.steps, wl.prefill, seed=11, order="deferred")
    fill_steps = wl.budget - wl.prefill
    for r in reports:
        assert r.appends == fill_steps and r.evictions == wl.steps - fill_steps + 1
        assert r.tie_lowest_index == r.exact_ties


def test_llama8b_layer_l2_score_whole_trajectory():
    """The score with the l2 norm of the value rows (LongFlow Guide,
    §Mathematical Derivation of the LongFlow Score: the score may take the l1
    or the l2 norm of the contribution vector)."""
    wl = WORKLOADS["llama8b_layer"]
    _check_fill_then_evict(wl, _run(wl, wl.steps, wl.prefill, seed=12, norm="l2"))


@pytest.mark.parametrize("order", ["same_step", "deferred"])
def test_qwen3_0p6b_layer_one_victim_per_sequence_whole_trajectory(order):
    """One victim per sequence, the argmin of the scores summed over every
    KV head (the sum over all heads in the LongFlow Guide, §End-to-End
    Implementation), with the same-step and the deferred order: two sequences, all 8 KV heads of each, from a
    512-token prompt through 512 filling steps and 3,584 evicting ones."""
    wl = WORKLOADS["qwen3_0p6b_layer"]
    sampled = [(b, h) for b in (5, 26) for h in range(wl.num_kv_heads)]
    reports = _run(wl, wl.steps, 512, sampled=sampled, scope="sequence", order=order)
    assert len(reports) == 2
    H = wl.num_kv_heads
    for r in reports:
        assert r.appends == (wl.budget - 512) * H
        assert r.evictions == (wl.steps - (wl.budget - 512) + (order == "deferred")) * H
        assert r.tie_lowest_index == r.exact_ties
