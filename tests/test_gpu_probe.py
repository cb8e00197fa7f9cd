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
