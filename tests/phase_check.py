"""Check of lf_probe_decode_phases in the measurement build
(liblongflow_phases.so), run in a process of its own by
tests/test_gpu_probe.py: for a split launch (32 pairs, split-K) and for one
workgroup per pair (512 pairs, interleaved and phased loop), the probed step
equals lf_decode_step on a twin cache bit for bit, and every workgroup's
phase stamps are in order:
  split: every part reaches phases 1-4 in order after its start; exactly one
         part per pair (the last) reaches 5-7, in order, before its end;
  whole: phases 1, 2 and 7 in order between start and end, no split phases.
Exits non-zero (an AssertionError) on any mismatch."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from decode_kv_cache_02_amd import native  # noqa: E402


def check(shape):
    import torch
    from decode_kv_cache_02_amd.native import LongFlowCache
    from decode_kv_cache_02_amd.synth import WORKLOADS, device_prefill, device_steps
    wl = {"split": WORKLOADS["llama8b_layer"].with_(batch=4, budget=600),
          "whole_interleaved": WORKLOADS["llama8b_layer"].with_(budget=600),
          "whole_phased": WORKLOADS["llama8b_layer"].with_(budget=1100)}[shape]
    print(f"[case] phase records, {shape}: batch {wl.batch}, B {wl.budget}", flush=True)
    pairs = wl.batch * wl.num_kv_heads
    caches = [LongFlowCache(1, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.budget)
              for _ in range(2)]
    try:
        for c in caches:
            k, v = device_prefill(wl, wl.budget, seed=5)
            c.prefill(0, k, v, np.full(wl.batch, wl.budget, dtype=np.int32))
            del k, v
        Q, KN, VN = device_steps(wl, 1, seed=6)
        q, kn, vn = Q[0], KN[0], VN[0]
        outs = [torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                            device="cuda") for _ in range(2)]
        evs = [torch.empty((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
               for _ in range(2)]
        caches[0].decode_step(0, q, kn, vn, outs[0], evs[0])
        recs = torch.zeros((2048, 4), dtype=torch.int64, device="cuda")
        phs = torch.zeros((2048, 8), dtype=torch.int64, device="cuda")
        n = native.lf_probe_decode_phases(caches[1].handle, 0, q, kn, vn, outs[1], evs[1], recs, phs)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
        assert torch.equal(evs[0], evs[1])
        r = recs[:n].cpu().numpy()
        assert not recs[n:].any() and not phs[n:].any()
        assert sorted(r[:, 3]) == list(range(n))
        start, end, ph = r[:, 0], r[:, 1], phs[:n].cpu().numpy()
        assert (start > 0).all() and (end >= start).all()
        assert not ph[:, 7].any()                                   # phase 8 unused
        if shape == "split":
            assert n > pairs and n % pairs == 0
            assert (ph[:, :4] > 0).all()
            seq = np.concatenate([start[:, None], ph[:, :4]], axis=1)
            assert (np.diff(seq, axis=1) >= 0).all()
            last = ph[:, 4] > 0
            assert last.sum() == pairs
            assert not ph[~last, 4:7].any()
            seq = np.concatenate([ph[last, 3:7], end[last, None]], axis=1)
            assert (np.diff(seq, axis=1) >= 0).all()
        else:
            assert n == pairs
            assert not ph[:, 2:6].any()
            seq = np.stack([start, ph[:, 0], ph[:, 1], ph[:, 6], end], axis=1)
            assert (seq[:, 1:4] > 0).all() and (np.diff(seq, axis=1) >= 0).all()
        print(f"[case] {shape}: {n} workgroups, phases in order", flush=True)
    finally:
        for c in caches:
            c.close()


if __name__ == "__main__":
    native.load_library(native.PHASES_LIB_PATH)
    import torch
    torch.cuda.set_device(0)
    for shape in ("split", "whole_interleaved", "whole_phased"):
        check(shape)
    print("phase records: all in order", flush=True)
