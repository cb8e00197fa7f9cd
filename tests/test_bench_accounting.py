"""The bench line's accounting, on the CPU: the algorithmic bytes behind the
roofline fraction, the kernel-source hash that ties committed counter runs to
the source they measured, and the rule that stale counters are not reported.

Expected byte counts are worked out by hand from the definition: per pair and
step, K and V of the n cached slots, the query group in and the output group
out, k_new and v_new in, the new token's K, V and float32 norm written, and
the int32 evicted slot.
"""
import json

import bench


def test_algorithmic_bytes_of_the_configured_workloads():
    # Llama-8B layer: n = 3277 slots, G = 4, head_dim 128, bfloat16
    per_pair = 3277 * 2 * 128 * 2 + 2 * 4 * 128 * 2 + 2 * 128 * 2 + (2 * 128 * 2 + 4) + 4
    assert per_pair == 1_680_904
    assert bench.algorithmic_bytes_per_pair(3277, 4, 128, 2, True) == per_pair
    assert 512 * per_pair == 860_622_848
    # Qwen3-0.6B layer: 256 pairs of 1024 slots, G = 2
    assert 256 * bench.algorithmic_bytes_per_pair(1024, 2, 128, 2, True) == 134_744_064
    # tiny float32 case: one pair of 64 slots, G = 2, head_dim 64
    assert bench.algorithmic_bytes_per_pair(64, 2, 64, 4, True) == 34_824
    # an appending step writes no evicted slot index
    assert (bench.algorithmic_bytes_per_pair(100, 4, 128, 2, True)
            - bench.algorithmic_bytes_per_pair(100, 4, 128, 2, False)) == 4


def test_kernel_hash_ignores_comments_and_layout_but_not_code(tmp_path, monkeypatch):
    a = tmp_path / "a.h"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a)])
    h0 = bench.kernel_sha()
    a.write_text("int   f(int x) { return x + 1; }\n// another comment\n")
    assert bench.kernel_sha() == h0
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_sha() != h0


def test_counter_traffic_is_reported_only_for_the_source_it_measured(tmp_path, monkeypatch):
    t = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(t))
    assert bench.load_traffic(1.0) is None          # no counter run committed
    t.write_text(json.dumps({"kernel_sha": bench.kernel_sha(), "hbm_bytes_per_launch": 123.0}))
    assert bench.load_traffic(1.0) == 123.0
    t.write_text(json.dumps({"kernel_sha": "0" * 16, "hbm_bytes_per_launch": 123.0}))
    assert bench.load_traffic(1.0) is None          # counters of another source


def test_committed_counters_match_the_current_kernel_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["kernel_sha"] == bench.kernel_sha(), \
        "profiles/traffic_decode_llama8b_layer.json was measured on another kernel source"
    # calibrated traffic of the Llama-8B layer: within 2% above the algorithmic bytes
    assert 1.0 <= t["hbm_bytes_per_launch"] / 860_622_848 < 1.02


def test_every_profile_names_the_current_kernel_source():
    import glob
    import os
    import re
    stale = []
    for path in sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "*.md"))):
        text = open(path).read()
        for sha in re.findall(r"sha256\[:16\]\s*=\s*([0-9a-f]{16})", text):
            if sha != bench.kernel_sha():
                stale.append((os.path.basename(path), sha))
    assert not stale, f"profiles taken on another kernel source: {stale}"
