"""Pins of the oracle's variants: l2 score, deferred order, head-shared eviction,
sequence recycling. No GPU.

Each variant is checked against something other than its own code: hand-derived
fixtures (tests/golden), the explicit contribution tensor, and the blog
engine's step semantics re-expressed independently in oracle/page_step.py.
"""
import json
import os

import numpy as np
import pytest

from decode_kv_cache_02_amd.synth import WORKLOADS, TokenStream
from oracle import longflow_oracle as lo
from oracle.page_step import DeferredEvictionEngine

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    conv = lambda v: np.inf if v == "inf" else v
    if isinstance(x[0], list):
        return np.array([[conv(v) for v in row] for row in x], dtype=np.float64)
    return np.array([conv(v) for v in x], dtype=np.float64)


# ----------------------------------------------------------------------------
# l2 score (Guide, §Mathematical Derivation: l1 or l2 norm of c_{t,i})
# ----------------------------------------------------------------------------

def test_golden_l2_vs_l1():
    fx = _load("hand_l2_vs_l1.json")
    for case in fx["cases"]:
        c = lo.PairCache(fx["budget"], fx["head_dim"], norm=case["norm"])
        c.prefill(_f(fx["prefill_k"]), _f(fx["prefill_v"]))
        r = c.step(_f(fx["q"]), _f(fx["k_new"]), _f(fx["v_new"]))
        np.testing.assert_allclose(r.out, _f(fx["expected_out"]), rtol=0, atol=1e-15)
        np.testing.assert_allclose(r.scores, _f(case["expected_scores"]), rtol=1e-15, atol=0)
        assert r.evicted == case["expected_evicted"]
        np.testing.assert_allclose(c.vnorm, _f(case["expected_final_vnorm"]), rtol=1e-15, atol=0)


@pytest.mark.parametrize("seed", range(4))
def test_l2_score_is_l2_of_explicit_contribution(seed):
    """score_i = sum_g ||alpha_{g,i} v_i||_2, from the explicit tensor c[g][i][:]."""
    wl = WORKLOADS["tiny_f32"].with_(num_q_heads=4, num_kv_heads=1)
    ts = TokenStream(wl, seed_offset=seed)
    pf = ts.prefill()
    st = ts.step()
    c = lo.PairCache(64, 64, norm="l2")
    c.prefill(pf.k[0, :, 0], pf.v[0, :, 0])
    r = c.attend(st.q[0], st.k_new[0, 0], st.v_new[0, 0])
    V = pf.v[0, :, 0].astype(np.float64)
    contrib = r.alpha[:, :64, None] * V[None]                  # [G][B][d]
    explicit = np.linalg.norm(contrib, axis=2).sum(axis=0)
    np.testing.assert_allclose(r.scores, explicit, rtol=1e-12)
    # Cauchy-Schwarz brackets the l1 score of the same step
    c1 = lo.PairCache(64, 64, norm="l1")
    c1.prefill(pf.k[0, :, 0], pf.v[0, :, 0])
    r1 = c1.attend(st.q[0], st.k_new[0, 0], st.v_new[0, 0])
    assert np.all(r.scores <= r1.scores * (1 + 1e-12))
    assert np.all(r1.scores <= np.sqrt(64) * r.scores * (1 + 1e-12))


# ----------------------------------------------------------------------------
# Deferred order (Guide, §End-to-End Implementation)
# ----------------------------------------------------------------------------

def test_golden_deferred_order():
    fx = _load("hand_deferred_order.json")
    c = lo.PairCache(fx["budget"], fx["head_dim"], order="deferred")
    c.prefill(_f(fx["prefill_k"]), _f(fx["prefill_v"]))
    for st in fx["steps"]:
        r = c.step(_f(st["q"]), _f(st["k_new"]), _f(st["v_new"]))
        np.testing.assert_allclose(r.out, _f(st["expected_out"]), rtol=0, atol=1e-15)
        np.testing.assert_array_equal(r.scores, _f(st["expected_scores"]))
        assert r.evicted == st["expected_replaced"]
        assert r.next_victim == st["expected_next_victim"]
        assert c.victim == st["expected_next_victim"]
    fb = fx["fallback"]
    c = lo.PairCache(fx["budget"], fx["head_dim"], order="deferred")
    c.prefill(_f(fb["prefill_k"]), _f(fb["prefill_v"]))
    r = c.step(_f(fb["q"]), _f(fb["k_new"]), _f(fb["v_new"]))
    np.testing.assert_allclose(r.out, _f(fb["expected_out"]), rtol=0, atol=1e-15)
    assert r.evicted == fb["expected_replaced"]
    assert r.next_victim == fb["expected_next_victim"]


def _engine_run(wl, prompt, steps, sink, shared, budget_engine, order, seed=0):
    """Step the oracle and blog engines side by side on the same tokens.

    shared=True : one engine per sequence over all KV heads (MHA: G = 1).
    shared=False: one engine per KV head, its G query heads each holding a
                  copy of the head's K and V.
    Returns (our replaced-token list, their replaced-token list) per engine.
    """
    B = wl.budget
    G, hkv, d = wl.group, wl.num_kv_heads, wl.head_dim
    ts = TokenStream(wl, seed_offset=seed)
    pf = ts.prefill(n_max=prompt, n_per_seq=np.full(wl.batch, prompt, np.int32))
    ours = lo.LayerCache(1, wl.num_q_heads, hkv, d, B, sink_size=sink, order=order,
                         scope="sequence" if shared else "kv_head")
    ours.prefill(pf.k, pf.v, [prompt])
    k0 = pf.k[0].astype(np.float64)            # [prompt][Hkv][d]
    v0 = pf.v[0].astype(np.float64)
    groups = [list(range(hkv))] if shared else [[h] for h in range(hkv)]
    engines = []
    for hs in groups:
        heads = len(hs) * G
        e = DeferredEvictionEngine(heads, d, budget_engine, sink)
        rep = lambda x: np.repeat(x[:, hs].transpose(1, 0, 2), G, axis=0)   # [heads][m][d]
        e.load(rep(k0), rep(v0), np.arange(prompt))
        engines.append((hs, e))
    token_at = {h: list(range(prompt)) + [-1] * (B - prompt) for h in range(hkv)}
    ours_rep = {i: [] for i in range(len(groups))}
    theirs_rep = {i: [] for i in range(len(groups))}
    for t in range(steps):
        st = ts.step()
        res = ours.step(st.q[0:1], st.k_new[0:1], st.v_new[0:1])
        tid = prompt + t
        for gi, (hs, e) in enumerate(engines):
            qh = np.concatenate([st.q[0, h * G:(h + 1) * G] for h in hs]).astype(np.float64)
            kk = np.repeat(st.k_new[0, hs].astype(np.float64), G, axis=0)
            vv = np.repeat(st.v_new[0, hs].astype(np.float64), G, axis=0)
            out, replaced = e.advance(qh, kk, vv, tid)
            ref = np.concatenate([res[(0, h)].out for h in hs])
            np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
            theirs_rep[gi].append(replaced)
            r0 = res[(0, hs[0])]
            if order == "deferred":
                ours_rep[gi].append(-1 if r0.evicted < 0 else token_at[hs[0]][r0.evicted])
            else:
                ours_rep[gi].append(-1 if r0.evicted < 0 else token_at[hs[0]][r0.evicted])
            for h in hs:
                rh = res[(0, h)]
                assert not rh.near_tie
                target = rh.slot if order == "deferred" else (rh.evicted if rh.evicted >= 0 else rh.slot)
                token_at[h][target] = tid
    return ours_rep, theirs_rep


@pytest.mark.parametrize("prompt,sink", [(64, 0), (40, 0), (48, 4)])
def test_deferred_shared_mha_is_the_blog_engine(prompt, sink):
    """order=deferred, scope=sequence, G = 1 is the engine itself, same budget."""
    wl = WORKLOADS["tiny_f32"].with_(num_q_heads=3, num_kv_heads=3)
    ours, theirs = _engine_run(wl, prompt, 80, sink, True, wl.budget, "deferred")
    assert ours[0] == theirs[0]
    assert sum(x >= 0 for x in ours[0]) >= 80 - (64 - prompt)


@pytest.mark.parametrize("prompt", [64, 30])
def test_deferred_per_kv_head_is_one_engine_per_group(prompt):
    """order=deferred, scope=kv_head with G = 2: each KV head behaves as an
    engine whose G heads hold copies of that head's K and V."""
    wl = WORKLOADS["tiny_f32"].with_(num_q_heads=4, num_kv_heads=2)
    ours, theirs = _engine_run(wl, prompt, 70, 0, False, wl.budget, "deferred", seed=3)
    for gi in ours:
        assert ours[gi] == theirs[gi]


def test_shared_same_step_evicts_what_the_engine_evicts_one_slot_later():
    """order=same_step, scope=sequence at budget B evicts the tokens that the
    blog engine (deferred) at budget B+1 replaces one call later."""
    wl = WORKLOADS["tiny_f32"].with_(num_q_heads=3, num_kv_heads=3)
    ours, theirs = _engine_run(wl, 64, 60, 0, True, wl.budget + 1, "same_step", seed=7)
    assert theirs[0][0] == -1
    assert ours[0][:-1] == theirs[0][1:]


def test_sequence_scope_sums_heads_before_the_argmin():
    """The shared victim minimises the head-summed score, which need not be
    any single head's own minimum."""
    wl = WORKLOADS["tiny_f32"].with_(batch=1, num_q_heads=8, num_kv_heads=4)
    differs = 0
    for seed in range(6):
        ts = TokenStream(wl, seed_offset=seed)
        pf = ts.prefill()
        st = ts.step()
        lay = lo.LayerCache(1, 8, 4, 64, 64, scope="sequence")
        lay.prefill(pf.k, pf.v, [64])
        res = lay.attend(st.q, st.k_new, st.v_new)
        own = [lo.first_argmin(res[(0, h)].scores_own) for h in range(4)]
        total = sum(res[(0, h)].scores_own for h in range(4))
        victim = res[(0, 0)].evicted
        assert victim == int(np.argmin(total))
        assert all(res[(0, h)].evicted == victim for h in range(4))
        differs += int(any(o != victim for o in own))
    assert differs > 0


# ----------------------------------------------------------------------------
# Sequence recycling in the static buffer (Guide, §Static Memory
# Pre-Allocation and In-Place Eviction)
# ----------------------------------------------------------------------------

def test_recycled_sequence_behaves_like_a_fresh_one():
    wl = WORKLOADS["tiny_f32"].with_(batch=3, budget=32, prefill=20)
    ts = TokenStream(wl, seed_offset=11)
    pf = ts.prefill()
    lay = lo.LayerCache(3, 2, 1, 64, 32)
    lay.prefill(pf.k, pf.v, [20, 20, 20])
    for _ in range(30):
        st = ts.step()
        lay.step(st.q, st.k_new, st.v_new)
    before = {p: (c.n, c.K.copy()) for p, c in lay.cache.items()}
    lay.reset({1})
    assert lay.cache[(1, 0)].n == 0 and lay.cache[(1, 0)].victim == -1
    # a new prompt only for sequence 1; the others are left as they are
    pf2 = TokenStream(wl, seed_offset=99).prefill()
    lay.prefill(pf2.k, pf2.v, [-1, 12, -1])
    for b in (0, 2):
        assert lay.cache[(b, 0)].n == before[(b, 0)][0]
        np.testing.assert_array_equal(lay.cache[(b, 0)].K, before[(b, 0)][1])
    fresh = lo.PairCache(32, 64)
    fresh.prefill(pf2.k[1, :12, 0], pf2.v[1, :12, 0])
    for _ in range(40):
        st = ts.step()
        res = lay.step(st.q, st.k_new, st.v_new)
        r = fresh.step(st.q[1], st.k_new[1, 0], st.v_new[1, 0])
        np.testing.assert_array_equal(res[(1, 0)].out, r.out)
        assert res[(1, 0)].evicted == r.evicted


# ----------------------------------------------------------------------------
# Planted mistakes in the variants are caught by the pins above
# ----------------------------------------------------------------------------

def test_planted_deferred_keeps_replaced_token_is_caught(monkeypatch):
    """An oracle that still attends the replaced token fails the engine pin."""
    real = lo.PairCache._attend_deferred

    def wrong(self, q, k_new, v_new):
        n, B = self.n, self.budget
        if n < B:
            return real(self, q, k_new, v_new)
        slot = self.victim if self.victim >= 0 else B - 1
        keys = np.vstack([self.K[:n], k_new[None]])
        vals = np.vstack([self.V[:n], v_new[None]])
        alpha = lo.attention_weights(q, keys, self.scale)
        res = real(self, q, k_new, v_new)
        res.out = lo.attention_output(alpha, vals)
        return res

    monkeypatch.setattr(lo.PairCache, "_attend_deferred", wrong)
    with pytest.raises(AssertionError):
        test_deferred_shared_mha_is_the_blog_engine(64, 0)


def test_planted_l2_without_sqrt_is_caught(monkeypatch):
    monkeypatch.setattr(lo, "l2_norms", lambda v: (np.asarray(v, np.float64) ** 2).sum(axis=-1))
    with pytest.raises(AssertionError):
        test_golden_l2_vs_l1()


def test_planted_shared_scope_max_instead_of_sum_is_caught(monkeypatch):
    real = lo.LayerCache._share_victims

    def wrong(self, res):
        real(self, res)
        for b in {b for b, _ in res}:
            heads = [res[(b, h)] for h in range(self.hkv)]
            if heads[0].scores is None:
                continue
            worst = np.max([r.scores_own for r in heads], axis=0)
            choice = lo.first_argmin(worst)
            for r in heads:
                r.evicted = r.slot = choice

    monkeypatch.setattr(lo.LayerCache, "_share_victims", wrong)
    with pytest.raises(AssertionError):
        test_sequence_scope_sums_heads_before_the_argmin()
