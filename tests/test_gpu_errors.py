"""Error paths of the C ABI that need a live cache (host-side validation):
every failing call returns its status and leaves the cache as it was."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture
def cache():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd.native import LongFlowCache
    c = LongFlowCache(2, 3, 8, 2, 128, 40, dtype="bf16")
    k = torch.randn((3, 20, 2, 128), device="cuda").to(torch.bfloat16)
    c.prefill(0, k, k, [20, 10, 0])
    c.prefill(1, k, k, [5, 5, 5])
    torch.cuda.synchronize()
    yield c
    c.close()


def _io(dt=None):
    import torch
    dt = dt or torch.bfloat16
    q = torch.randn((3, 8, 128), device="cuda").to(dt)
    kn = torch.randn((3, 2, 128), device="cuda").to(dt)
    out = torch.empty((3, 8, 128), dtype=dt, device="cuda")
    ev = torch.empty((3, 2), dtype=torch.int32, device="cuda")
    return q, kn, out, ev


def _state(c):
    snaps = [c.snapshot(layer, with_victim=True) for layer in range(2)]
    return [[t.clone() for t in s] for s in snaps], [c.fill_levels(layer).copy() for layer in range(2)]


def _same(a, b):
    import torch
    for sa, sb in zip(a[0], b[0]):
        for x, y in zip(sa, sb):
            assert torch.equal(x, y)
    for fa, fb in zip(a[1], b[1]):
        assert np.array_equal(fa, fb)


def test_misaligned_pointer_rejected(cache):
    import torch
    from decode_kv_cache_02_amd import native
    print("\n[case] misaligned q", flush=True)
    before = _state(cache)
    q, kn, out, ev = _io()
    big = torch.empty(q.numel() + 8, dtype=q.dtype, device="cuda")
    q_off = big[1:1 + q.numel()].view(q.shape)          # 2-byte offset: not 16-byte aligned
    with pytest.raises(native.LongFlowError) as ei:
        native.lf_decode_step(cache.handle, 0, q_off, kn, kn, out, ev)
    assert ei.value.status == native.LF_ERR_INVALID_ARG
    torch.cuda.synchronize()
    _same(before, _state(cache))


def test_layer_out_of_range(cache):
    from decode_kv_cache_02_amd import native
    print("\n[case] layer out of range", flush=True)
    before = _state(cache)
    q, kn, out, ev = _io()
    for layer in (-1, 2):
        with pytest.raises(native.LongFlowError) as ei:
            native.lf_decode_step(cache.handle, layer, q, kn, kn, out, ev)
        assert ei.value.status == native.LF_ERR_INVALID_ARG
    _same(before, _state(cache))


def test_prefill_errors_change_nothing(cache):
    import torch
    from decode_kv_cache_02_amd import native
    print("\n[case] prefill errors", flush=True)
    before = _state(cache)
    k = torch.zeros((3, 50, 2, 128), device="cuda").to(torch.bfloat16)
    with pytest.raises(native.LongFlowError) as ei:
        cache.prefill(0, k, k, [41, 0, 0])                # past the budget of 40
    assert ei.value.status == native.LF_ERR_CAPACITY
    k10 = k[:, :10].contiguous()
    with pytest.raises(native.LongFlowError) as ei:
        cache.prefill(0, k10, k10, [11, 0, 0])            # longer than n_max
    assert ei.value.status == native.LF_ERR_INVALID_ARG
    with pytest.raises(native.LongFlowError) as ei:
        cache.prefill(0, k10, k10, [-2, 0, 0])            # only -1 means "leave as is"
    assert ei.value.status == native.LF_ERR_INVALID_ARG
    with pytest.raises(ValueError):                        # the binding refuses non-contiguous views
        cache.prefill(0, k[:, :10], k[:, :10], [5, 0, 0])
    for short in ([5, 0], [5, 0, 0, 0]):                   # one length per sequence, no more, no less
        with pytest.raises(ValueError):
            cache.prefill(0, k10, k10, short)
    torch.cuda.synchronize()
    _same(before, _state(cache))


def test_reset_and_tuning_errors(cache):
    from decode_kv_cache_02_amd import native
    print("\n[case] reset / tuning errors", flush=True)
    before = _state(cache)
    for seqs in ([3], [-1], [0, 5]):
        with pytest.raises(native.LongFlowError) as ei:
            cache.seq_reset(seqs)
        assert ei.value.status == native.LF_ERR_INVALID_ARG
    for w in (1, 5, 16, -4):
        with pytest.raises(native.LongFlowError) as ei:
            cache.set_waves(w)
        assert ei.value.status == native.LF_ERR_INVALID_ARG
    with pytest.raises(native.LongFlowError) as ei:
        cache.set_splits(-1)
    assert ei.value.status == native.LF_ERR_INVALID_ARG
    for loop in (3, -1):
        with pytest.raises(native.LongFlowError) as ei:
            cache.set_loop(loop)
        assert ei.value.status == native.LF_ERR_INVALID_ARG
    _same(before, _state(cache))


def test_partial_prefill_and_reset_touch_only_their_sequences(cache):
    import torch
    print("\n[case] partial prefill / reset", flush=True)
    before = _state(cache)
    k = torch.ones((3, 7, 2, 128), device="cuda").to(torch.bfloat16)
    cache.prefill(0, k, k, [-1, 7, -1])
    cache.seq_reset([2])
    torch.cuda.synchronize()
    after = _state(cache)
    # layer 0: sequence 0 untouched, 1 refilled with 7 tokens; layer 1 untouched except seq 2
    assert list(after[1][0]) == [20, 7, 0]
    assert list(after[1][1]) == [5, 5, 0]
    kb, vb, nb, fb, xb = before[0][0]
    ka, va, na, fa, xa = after[0][0]
    assert torch.equal(ka[0], kb[0]) and torch.equal(va[0], vb[0]) and torch.equal(na[0], nb[0])
    assert torch.equal(ka[1, :, :7].float(), torch.ones_like(ka[1, :, :7]).float())
    assert int(fa[2].max()) == 0 and int(xa[2].min()) == -1
