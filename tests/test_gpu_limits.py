"""GPU parity at the size limits and at full workload shapes (sampled pairs).

* the largest budgets one workgroup's LDS holds (144 KB of logits: 9216 slots
  at G = 4, 36864 at G = 1), and the first budget past it is refused;
* the full-KV baseline at the 16k-token context the bench times;
* the 32-layer ragged Llama-8B stack at its full shape (batch 103), a middle
  layer, pairs that append and pairs that evict in the same launch.
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


@pytest.mark.parametrize("G,d,budget,dtype", [(4, 128, 9216, "bf16"), (1, 128, 36864, "bf16"),
                                              (2, 64, 18432, "f32")])
@pytest.mark.parametrize("splits,loop", [(0, "auto"), (1, "phased"), (1, "interleaved")])
def test_largest_budget(G, d, budget, dtype, splits, loop):
    """The automatic launch splits these 4 pairs 16 ways; one workgroup per
    pair holds all of a pair's logits in LDS, with either loop."""
    wl = WORKLOADS["tiny_f32"].with_(dtype=dtype, batch=2, num_kv_heads=2, num_q_heads=2 * G,
                                     head_dim=d, budget=budget, prefill=budget - 2)
    _say(f"{dtype} G={G} d={d} B={budget} (LDS cap), prefill {budget - 2}, 5 steps, every pair, "
         f"splits {splits or 'auto'}, {loop}")
    rep = run_lockstep(wl, 5, check_cache_every=5, splits=splits, loop=loop)
    assert rep.appends == 2 * 4 and rep.evictions == 3 * 4


@pytest.mark.parametrize("G,budget", [(4, 9217), (1, 36865)])
def test_budget_past_lds_cap_is_refused(G, budget):
    from decode_kv_cache_02_amd.native import LongFlowCache, LongFlowError, LF_ERR_UNSUPPORTED
    _say(f"G={G} B={budget}: refused")
    with pytest.raises(LongFlowError) as ei:
        LongFlowCache(1, 1, G, 1, 128, budget)
    assert ei.value.status == LF_ERR_UNSUPPORTED


def test_full_kv_long_context():
    """LF_MODE_FULL at the bench's 16k context: 9 LDS chunks per pair."""
    wl = WORKLOADS["llama8b_layer"].with_(batch=2, prefill=16384)
    _say("bf16 FULL mode, capacity 16960, prefill 16384, 6 steps, every pair (batch 2)")
    rep = run_lockstep(wl, 6, mode="full", capacity=16960, check_cache_every=6)
    assert rep.appends == 6 * 16


def test_llama8b_stack32_ragged_full_shape():
    wl = WORKLOADS["llama8b_stack32_ragged"].with_(batch=103)
    offs = TokenStream(wl).start_offsets()
    n = np.minimum(offs, wl.budget).astype(np.int32)
    short = [int(b) for b in np.flatnonzero(n < wl.budget)[:3]]
    full = [int(b) for b in np.flatnonzero(n == wl.budget)[:3]]
    pairs = [(b, h) for b, h in zip(short + full, (0, 3, 7, 1, 4, 6))]
    _say(f"llama8b stack32 ragged, batch 103, layer 17 of 32, 4 steps, pairs {pairs}")
    rep = run_lockstep(wl, 4, pairs=pairs, prefill_n=n, layer=17, num_layers=32,
                       check_cache_every=4)
    assert rep.appends > 0 and rep.evictions > 0


@pytest.mark.parametrize("budget", [512, 1024])
def test_qwen3_8b_stack36_full_shape(budget):
    """The 36-layer Qwen3-8B stack at batch 256 (the suite's launch), a middle
    layer, sampled pairs, duplicated tokens included."""
    wl = WORKLOADS["qwen3_8b_stack36_ties"].with_(budget=budget, prefill=budget)
    pairs = [(0, 0), (77, 3), (128, 5), (255, 7), (200, 1), (31, 6)]
    _say(f"qwen3_8b stack36, batch 256, B {budget}, layer 20 of 36, 4 steps, pairs {pairs}")
    rep = run_lockstep(wl, 4, pairs=pairs, layer=20, num_layers=36, check_cache_every=4)
    assert rep.evictions == 4 * len(pairs)
    assert rep.exact_ties > 0
    assert rep.tie_lowest_index == rep.exact_ties
