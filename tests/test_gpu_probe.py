"""GPU check of the streaming-read probe (include/longflow_probe.h): every
16-byte chunk of the buffer is read exactly once, by the thread the XOR sink
says. The expected XORs are computed on the host from the same buffer."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("workgroups,chunks_per_thread", [(1, 8), (3, 5), (8, 1)])
def test_probe_reads_every_chunk_once(workgroups, chunks_per_thread):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd import native
    print(f"\n[case] probe {workgroups} workgroups, {chunks_per_thread} chunks per thread", flush=True)
    words = workgroups * 256 * chunks_per_thread * 4          # int32 words, 16 bytes per chunk
    host = np.random.default_rng(workgroups * 10 + chunks_per_thread).integers(
        -2**31, 2**31 - 1, size=words, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = torch.zeros(workgroups * 256 * 4, dtype=torch.int32, device="cuda")
    native.lf_probe_stream_read(buf, workgroups, sink)
    got = sink.cpu().numpy().reshape(workgroups, 256, 4)
    chunks = host.reshape(workgroups, chunks_per_thread * 256, 4)
    want = np.zeros((workgroups, 256, 4), dtype=np.int32)
    for j in range(chunks_per_thread):
        want ^= chunks[:, j * 256:(j + 1) * 256, :]
    np.testing.assert_array_equal(got, want)


def test_probe_rejects_bad_sizes():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd import native
    buf = torch.zeros(1000, dtype=torch.int32, device="cuda")     # 4000 bytes: not 16 x 256-aligned per WG
    sink = torch.zeros(256 * 4, dtype=torch.int32, device="cuda")
    with pytest.raises(native.LongFlowError) as ei:
        native.lf_probe_stream_read(buf[:999], 1, sink)
    assert ei.value.status == native.LF_ERR_INVALID_ARG


def test_hbm_attributes():
    """The device reports its memory clock and bus width (MI355X: eight
    1024-bit HBM3E stacks)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd.native import lf_probe_hbm_attributes
    clock_khz, bus_bits = lf_probe_hbm_attributes()
    print(f"\nHBM attributes: memory clock {clock_khz} kHz, bus {bus_bits} bits", flush=True)
    assert clock_khz > 0
    assert bus_bits % 1024 == 0 and bus_bits >= 4096


def test_timing_records_of_a_read_and_of_a_decode_step():
    """The timing variants: every workgroup leaves one record (start <= end,
    an XCC id, its index), and the timed decode step gives exactly what
    lf_decode_step gives on a twin cache."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd import native
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import WORKLOADS, TokenStream
    wgs = 512
    buf = torch.ones(wgs * 256 * 4 * 16, dtype=torch.int32, device="cuda")
    sink = torch.empty(wgs * 256 * 4, dtype=torch.int32, device="cuda")
    rec = torch.zeros((wgs, 4), dtype=torch.int64, device="cuda")
    native.lf_probe_stream_read_timing(buf, wgs, sink, rec)
    r = rec.cpu().numpy()
    assert (r[:, 1] >= r[:, 0]).all() and (r[:, 0] > 0).all()
    assert sorted(r[:, 3]) == list(range(wgs))
    xcc = r[:, 2] & 0xFFFF
    print(f"\nread probe: {wgs} workgroups over XCCs {sorted(set(xcc.tolist()))}", flush=True)
    assert (xcc < 64).all()

    wl = WORKLOADS["llama8b_layer"].with_(batch=4, budget=600, prefill=600)   # 32 pairs: split-K
    caches = [LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget)
              for _ in range(2)]
    try:
        pf = TokenStream(wl).prefill()
        dev = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)
        for c in caches:
            c.prefill(0, dev(pf.k), dev(pf.v), pf.n_per_seq)
        st = TokenStream(wl, seed_offset=1).step()
        q, kn, vn = dev(st.q), dev(st.k_new), dev(st.v_new)
        outs = [torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                            device="cuda") for _ in range(2)]
        evs = [torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
               for _ in range(2)]
        caches[0].decode_step(0, q, kn, vn, outs[0], evs[0])
        recs = torch.zeros((1024, 4), dtype=torch.int64, device="cuda")
        n = native.lf_probe_decode_timing(caches[1].handle, 0, q, kn, vn, outs[1], evs[1], recs)
        torch.cuda.synchronize()
        assert n % 32 == 0 and n >= 32
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
        assert torch.equal(evs[0], evs[1])
        r = recs[:n].cpu().numpy()
        assert (r[:, 1] >= r[:, 0]).all() and (r[:, 0] > 0).all()
        assert sorted(r[:, 3]) == list(range(n))
        assert not recs[n:].any()
        with pytest.raises(native.LongFlowError) as ei:
            native.lf_probe_decode_timing(caches[1].handle, 0, q, kn, vn, outs[1], evs[1], recs[:n - 1])
        assert ei.value.status == native.LF_ERR_INVALID_ARG
    finally:
        for c in caches:
            c.close()


def test_phase_probe_needs_the_measurement_build():
    """The library leaves the phase stamps out: lf_probe_decode_phases says
    LF_ERR_UNSUPPORTED and queues nothing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd import native
    from decode_kv_cache_02_amd.native import LongFlowCache
    cache = LongFlowCache(1, 2, 8, 2, 128, 64)
    try:
        q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
        kv = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
        out = torch.empty_like(q)
        ev = torch.empty((2, 2), dtype=torch.int32, device="cuda")
        recs = torch.zeros((64, 4), dtype=torch.int64, device="cuda")
        phs = torch.zeros((64, 8), dtype=torch.int64, device="cuda")
        with pytest.raises(native.LongFlowError) as ei:
            native.lf_probe_decode_phases(cache.handle, 0, q, kv, kv, out, ev, recs, phs)
        assert ei.value.status == native.LF_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert not recs.any() and not phs.any()
        assert cache.fill_levels(0).tolist() == [0, 0]
    finally:
        cache.close()


def test_phase_records_of_the_measurement_build():
    """tests/phase_check.py, run in a process of its own on
    liblongflow_phases.so: the probed step equals lf_decode_step on a twin
    cache, and every workgroup's phase stamps are in order (a split launch,
    and one workgroup per pair with either loop)."""
    import subprocess
    import sys
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_kv_cache_02_amd import native
    import os
    if not os.path.exists(native.PHASES_LIB_PATH):
        pytest.fail(f"{native.PHASES_LIB_PATH} is missing: python -m decode_kv_cache_02_amd.build --phases")
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "phase_check.py")
    res = subprocess.run([sys.executable, "-u", script], capture_output=True, text=True, timeout=240)
    print(res.stdout[-4000:], res.stderr[-4000:], flush=True)
    assert res.returncode == 0
