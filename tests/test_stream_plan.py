"""The launch planner of the evicting main path (lf_probe_stream_plan: the
library's own plan_stream, host only), checked on the CPU.

A stream launch must cover every pair exactly once: whole pairs [0,
sk_first) taken in turn by the grid's workgroups, and the tiles of the cut
pairs [sk_first, pairs) dealt out sk_q at a time to workgroups 0 ..
sk_wgs - 1. The walk below follows the stream kernel's unit loop
(decode_kernel_stream): a run that holds a pair whole runs it as a whole
pair; otherwise the run's part of the pair gets index w - (the pair's first
workgroup) of (its last - its first + 1) parts, and its workspace row is
pair - sk_first. The checks: every tile of every cut pair is covered once,
the parts of a pair are 0 .. count - 1 with count <= the partial states per
row, rows stay below the layer's workspace rows, and the bands of the rule
are where they are documented (MI355X: 256 compute units, two resident
4-wave workgroups per compute unit).
"""
import pytest

from decode_kv_cache_02_amd import native


@pytest.fixture(scope="module")
def plan():
    native.load_library()
    return native.lf_probe_stream_plan


def walk(p, w):
    units = []
    if w < p["sk_wgs"]:
        tn, q = p["sk_tiles"], p["sk_q"]
        end = min(w * q + q, p["sk_pairs"] * tn)
        t = w * q
        while t < end:
            row = t // tn
            base = row * tn
            fw, lw = base // q, (base + tn - 1) // q
            if fw == lw:
                units.append(("whole", p["sk_first"] + row))
            else:
                units.append(("part", p["sk_first"] + row, w - fw, lw - fw + 1, row, t - base,
                              min(end - base, tn)))
            t = base + tn
    units += [("whole", u) for u in range(w, p["sk_first"], p["grid"])]
    return units


def check_cover(p, pairs, rows):
    if p["grid"] == 0:
        return
    assert p["grid"] >= p["sk_wgs"]
    whole, parts = [], {}
    for w in range(p["grid"]):
        for u in walk(p, w):
            if u[0] == "whole":
                whole.append(u[1])
                continue
            _, pair, idx, cnt, row, t0, t1 = u
            assert row == pair - p["sk_first"] and 0 <= row < rows
            assert 0 <= idx < cnt <= p["sk_stride"]
            assert 0 <= t0 < t1 <= p["sk_tiles"]
            parts.setdefault(pair, []).append((idx, cnt, t0, t1))
    for pair, ps in parts.items():
        counts = {c for _, c, _, _ in ps}
        assert len(counts) == 1
        assert sorted(i for i, *_ in ps) == list(range(counts.pop()))
        assert sorted(t for *_, t0, t1 in ps for t in range(t0, t1)) == list(range(p["sk_tiles"]))
    assert sorted(whole + list(parts)) == list(range(pairs))


def mi355x_rows(pairs):
    """Workspace rows the cache allocates for cut pairs (the stream bands on
    256 compute units)."""
    rows = 0
    if pairs > 256 and (pairs - 256) * 4 <= 256:
        rows = pairs - 256
    cut = pairs % 512
    if pairs > 512 and cut * 4 <= 512:
        rows = max(rows, cut)
    return min(rows, 512)


@pytest.mark.parametrize("n_max", [0, 1, 17, 1000, 3277, 4096])
def test_automatic_plans_cover_every_pair(plan, n_max):
    for pairs in range(200, 2700, 7):
        rows = mi355x_rows(pairs)
        for resident, fits8 in ((2, True), (1, True), (2, False)):
            p = plan(pairs, n_max, 256, resident, fits8, rows, 16)
            check_cover(p, pairs, max(rows, 1))
            if p["sk_pairs"]:
                assert p["sk_pairs"] <= rows


@pytest.mark.parametrize("tiles", [1, 2, 3, 7, 16, 100])
def test_forced_stream_plans_cover_every_pair(plan, tiles):
    """Small layers with a split-K workspace (a row per pair) streamed with
    any run length: runs too short for the row's partial states are raised."""
    for pairs in (1, 2, 5, 6, 17, 64, 255):
        stride = max(1, min(512 // pairs, 16))
        for n_max in (0, 5, 16, 100, 300, 1100, 4096):
            p = plan(pairs, n_max, 256, 2, True, pairs, stride, forced_stream=tiles)
            if stride > 1:
                assert p["grid"] > 0 and p["sk_first"] == 0 and p["sk_pairs"] == pairs
            check_cover(p, pairs, pairs)


def test_the_bands_on_mi355x(plan):
    def at(pairs, n_max=3277):
        return plan(pairs, n_max, 256, 2, True, mi355x_rows(pairs), 16)
    # whole rounds: one workgroup per pair
    for pairs in (256, 512, 1024, 2048):
        assert at(pairs)["grid"] == 0
    # just past the compute units: 256 workgroups of 8 waves
    p = at(264)
    assert (p["grid"], p["waves"], p["sk_first"], p["sk_pairs"]) == (256, 8, 256, 8)
    # just past 1, 2 and 3 rounds of two 4-wave workgroups per compute unit
    for pairs, first in ((520, 512), (576, 512), (1032, 1024), (1544, 1536)):
        p = at(pairs)
        assert (p["grid"], p["waves"], p["sk_first"], p["sk_pairs"]) == (512, 4, first, pairs - first)
    # past the 25% band: whole pairs (the 8-wave band ends at 320)
    assert at(321)["grid"] == 0 and at(641)["grid"] == 0 and at(1153)["grid"] == 0
    # a second round 40-85% full: two whole pairs per workgroup
    for pairs in (768, 816, 947):
        p = at(pairs)
        assert (p["grid"], p["sk_first"], p["sk_pairs"]) == ((pairs + 1) // 2, pairs, 0)
    assert at(960)["grid"] == 0
    # no workspace rows: no stream launch
    assert plan(520, 3277, 256, 2, True, 0, 16)["grid"] == 0
    # overrides
    assert plan(520, 3277, 256, 2, True, 8, 16, forced_grid=-1)["grid"] == 0
    p = plan(520, 3277, 256, 2, True, 8, 16, forced_grid=100)
    assert (p["grid"], p["sk_first"], p["sk_pairs"]) == (100, 520, 0)


def test_bad_arguments(plan):
    with pytest.raises(native.LongFlowError):
        plan(0, 10, 256, 2, True, 0, 16)
    with pytest.raises(native.LongFlowError):
        plan(10, -1, 256, 2, True, 0, 16)
