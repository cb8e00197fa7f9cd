"""Seeded synthetic inputs shaped like the LongFlow decode workloads.

This module only draws random numbers, rounds them once to the storage dtype
and lays them out. It holds none of the method's arithmetic (no attention, no
score, no eviction), so that the CPU oracle and the HIP path can both consume
the exact same tensors without sharing any code that computes the method.

Workload shapes follow the LongFlow pages: a ~500-token prompt followed by a
~16k-token chain of thought (LongFlow Guide, "The Asymmetry of Modern Reasoning
Workloads" diagram), a 3.2k-token budget, i.e. 20% of 16k (LongFlow Guide,
"Downstream Reasoning Accuracy Retention" table; gist.science summary, §4), and
the head shapes of the models the pages evaluate (DeepSeek-R1-Distill-Llama-8B,
Qwen3-0.6B and Qwen3-8B; gist.science summary, §4).

Value recipe (one reading each, stated where the pages are silent):
  * K and V entries are N(0, 1); each (token, KV head) V row is multiplied by
    one scalar drawn from lognormal(0, 0.5).
  * Each query head follows its own walk q_{t+1} = nrm(0.95 q_t + 0.31 z),
    z ~ N(0, I), with nrm() rescaling to L2 norm sqrt(d) (unit RMS per entry,
    the scale of K's entries); q_0 = nrm(z). Consecutive queries then have a
    cosine of about 0.95, the "consecutive queries are similar" regime of the
    query approximation (gist.science summary, §2.2 item 2).
  * Values are drawn in float32/float64 and rounded once to the storage dtype
    (bfloat16 with round-to-nearest-even, or float32).
  * Near-tie stress: with probability `dup_frac` a token copies both the K and
    V rows of a uniformly chosen earlier token of the same (sequence, KV head),
    so the two tokens' scores collide exactly. With dup_scope="sequence" the
    draw is made once per sequence and the same earlier token is copied in
    every KV head, so scores summed over the heads collide as well.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_STREAMS = ("prefill_k", "prefill_v", "v_scale", "decode_k", "decode_v",
            "q_walk", "dup", "offsets")

QUERY_WALK_KEEP = 0.95
QUERY_WALK_NOISE = 0.31
V_LOGNORMAL_SIGMA = 0.5


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even.

    Returns float32 values that are exactly representable in bfloat16. Inputs
    must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bfloat16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bfloat16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, budget and trajectory length."""

    name: str
    cfg_id: int
    dtype: str               # "f32" or "bf16": cache, q, k_new, v_new and out
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    budget: int
    layers: int
    prefill: int             # prompt tokens per sequence (uniform workloads)
    steps: int               # decode steps in the full trajectory
    dup_frac: float = 0.0
    dup_scope: str = "pair"      # "sequence": one draw per sequence, copied in every KV head
    ragged_max_offset: int = 0   # >0: per-sequence start offset ~ U[0, this)
    sink_size: int = 0
    note: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def pairs_per_layer(self) -> int:
        return self.batch * self.num_kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", 1, "f32", batch=1, num_q_heads=2, num_kv_heads=1,
        head_dim=64, budget=64, layers=1, prefill=64, steps=256,
        note="tiny single-layer fp32 loop, every step evicts"),
    "qwen3_0p6b_layer": Workload(
        "qwen3_0p6b_layer", 2, "bf16", batch=32, num_q_heads=16,
        num_kv_heads=8, head_dim=128, budget=1024, layers=1, prefill=1024,
        steps=4096, note="Qwen3-0.6B-shaped attention layer"),
    "llama8b_layer": Workload(
        "llama8b_layer", 3, "bf16", batch=64, num_q_heads=32, num_kv_heads=8,
        head_dim=128, budget=3277, layers=1, prefill=512, steps=16384,
        note="DeepSeek-R1-Distill-Llama-8B-shaped attention layer, B = 20% of 16384"),
    "llama8b_stack32_ragged": Workload(
        "llama8b_stack32_ragged", 4, "bf16", batch=103, num_q_heads=32,
        num_kv_heads=8, head_dim=128, budget=3277, layers=32, prefill=0,
        steps=512, ragged_max_offset=16384,
        note="32-layer Llama-8B stack, ragged fill from a U[0,16384) offset"),
    "qwen3_8b_stack36_ties": Workload(
        "qwen3_8b_stack36_ties", 5, "bf16", batch=256, num_q_heads=32,
        num_kv_heads=8, head_dim=128, budget=1024, layers=36, prefill=512,
        steps=16384, dup_frac=0.10,
        note="36-layer Qwen3-8B stack, budget swept over 512..4096, 10% duplicated tokens"),
}


def _rng_children(cfg_id: int, layer: int, seed_offset: int):
    ss = np.random.SeedSequence([cfg_id, layer, seed_offset])
    kids = ss.spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(k))
            for name, k in zip(_STREAMS, kids)}


def _normalise_rows(x: np.ndarray) -> np.ndarray:
    d = x.shape[-1]
    nrm = np.linalg.norm(x, axis=-1, keepdims=True)
    return x * (np.sqrt(d) / nrm)


@dataclass
class StepInputs:
    """Inputs of one decode step for every sequence of one layer."""

    q: np.ndarray        # [batch][num_q_heads][head_dim], dtype-exact float32
    k_new: np.ndarray    # [batch][num_kv_heads][head_dim]
    v_new: np.ndarray    # [batch][num_kv_heads][head_dim]
    dup_src: Optional[np.ndarray] = None   # [batch][num_kv_heads] token index copied, -1 = fresh


@dataclass
class PrefillInputs:
    k: np.ndarray        # [batch][n_max][num_kv_heads][head_dim]
    v: np.ndarray        # same
    n_per_seq: np.ndarray  # [batch] int32
    dup_src: Optional[np.ndarray] = None   # [batch][n_max][num_kv_heads]


@dataclass
class TokenStream:
    """Deterministic stream of prefill and decode inputs for one layer.

    Every draw comes from a PCG64 generator spawned from
    SeedSequence([cfg_id, layer, seed_offset]), one child per stream, so the
    same (workload, layer, seed_offset) always yields the same tensors.
    """

    wl: Workload
    layer: int = 0
    seed_offset: int = 0
    _rngs: dict = field(init=False, repr=False)
    _q: np.ndarray = field(init=False, repr=False)
    _hist_k: list = field(init=False, repr=False)
    _hist_v: list = field(init=False, repr=False)
    tokens_emitted: int = field(init=False, default=0)

    def __post_init__(self):
        self._rngs = _rng_children(self.wl.cfg_id, self.layer, self.seed_offset)
        wl = self.wl
        z = self._rngs["q_walk"].standard_normal(
            (wl.batch, wl.num_q_heads, wl.head_dim))
        self._q = _normalise_rows(z)
        self._hist_k = []
        self._hist_v = []

    # -- token rows -------------------------------------------------------
    def _fresh_rows(self, count: int, k_stream: str, v_stream: str):
        wl = self.wl
        shape = (wl.batch, count, wl.num_kv_heads, wl.head_dim)
        k = self._rngs[k_stream].standard_normal(shape, dtype=np.float32)
        v = self._rngs[v_stream].standard_normal(shape, dtype=np.float32)
        scale = self._rngs["v_scale"].lognormal(
            0.0, V_LOGNORMAL_SIGMA, size=shape[:3]).astype(np.float32)
        v = v * scale[..., None]
        return round_to_dtype(k, wl.dtype), round_to_dtype(v, wl.dtype)

    def _apply_duplicates(self, k, v):
        """Replace a `dup_frac` share of tokens by copies of earlier tokens."""
        wl = self.wl
        count = k.shape[1]
        src = np.full((wl.batch, count, wl.num_kv_heads), -1, dtype=np.int64)
        if wl.dup_frac <= 0.0:
            return k, v, src
        rng = self._rngs["dup"]
        for j in range(count):
            t = self.tokens_emitted + j
            if t == 0:
                continue
            if wl.dup_scope == "sequence":
                pick = np.repeat((rng.random(wl.batch) < wl.dup_frac)[:, None], wl.num_kv_heads, 1)
                choice = np.repeat(rng.integers(0, t, size=wl.batch)[:, None], wl.num_kv_heads, 1)
            else:
                pick = rng.random((wl.batch, wl.num_kv_heads)) < wl.dup_frac
                choice = rng.integers(0, t, size=(wl.batch, wl.num_kv_heads))
            for b, h in zip(*np.nonzero(pick)):
                s = int(choice[b, h])
                if s >= self.tokens_emitted:
                    ks, vs = k[b, s - self.tokens_emitted, h], v[b, s - self.tokens_emitted, h]
                else:
                    ks, vs = self._hist_k[s][b, h], self._hist_v[s][b, h]
                k[b, j, h] = ks
                v[b, j, h] = vs
                src[b, j, h] = s
        return k, v, src

    def _remember(self, k, v):
        if self.wl.dup_frac > 0.0:
            for j in range(k.shape[1]):
                self._hist_k.append(k[:, j].copy())
                self._hist_v.append(v[:, j].copy())
        self.tokens_emitted += k.shape[1]

    # -- public -------------------------------------------------------------
    def start_offsets(self) -> np.ndarray:
        """Per-sequence start offsets p_b ~ U[0, ragged_max_offset) (ragged workloads)."""
        wl = self.wl
        if wl.ragged_max_offset <= 0:
            return np.full(wl.batch, wl.prefill, dtype=np.int64)
        return self._rngs["offsets"].integers(0, wl.ragged_max_offset, size=wl.batch)

    def prefill(self, n_max: Optional[int] = None,
                n_per_seq: Optional[np.ndarray] = None) -> PrefillInputs:
        wl = self.wl
        if n_max is None:
            n_max = wl.prefill if n_per_seq is None else int(np.max(n_per_seq, initial=0))
        if n_per_seq is None:
            n_per_seq = np.full(wl.batch, n_max, dtype=np.int32)
        k, v = self._fresh_rows(n_max, "prefill_k", "prefill_v")
        k, v, src = self._apply_duplicates(k, v)
        self._remember(k, v)
        return PrefillInputs(k=k, v=v, n_per_seq=np.asarray(n_per_seq, dtype=np.int32),
                             dup_src=src)

    def step(self) -> StepInputs:
        wl = self.wl
        k, v = self._fresh_rows(1, "decode_k", "decode_v")
        k, v, src = self._apply_duplicates(k, v)
        self._remember(k, v)
        q = self._q
        z = self._rngs["q_walk"].standard_normal(q.shape)
        self._q = _normalise_rows(QUERY_WALK_KEEP * q + QUERY_WALK_NOISE * z)
        return StepInputs(q=round_to_dtype(q.astype(np.float32), wl.dtype),
                          k_new=k[:, 0], v_new=v[:, 0], dup_src=src[:, 0])


def step_ring(wl: Workload, count: int, layer: int = 0, seed_offset: int = 0):
    """`count` consecutive decode-step inputs stacked along a leading axis."""
    ts = TokenStream(wl, layer=layer, seed_offset=seed_offset)
    steps = [ts.step() for _ in range(count)]
    q = np.stack([s.q for s in steps])
    k = np.stack([s.k_new for s in steps])
    v = np.stack([s.v_new for s in steps])
    return q, k, v


def device_prefill(wl: Workload, n: int, seed: int, device: str = "cuda"):
    """Prefill K, V [batch][n][num_kv_heads][head_dim] drawn on the device.

    Same value recipe as TokenStream (K, V entries N(0,1), one lognormal(0,0.5)
    scale per V row, one rounding to the storage dtype) but drawn with torch's
    device generator seeded by `seed`, so multi-gigabyte caches can be filled
    in well under a second. Used where only the cost of a step matters.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    shape = (wl.batch, n, wl.num_kv_heads, wl.head_dim)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    k = torch.empty(shape, device=device, dtype=dt)
    v = torch.empty(shape, device=device, dtype=dt)
    # Drawn a few sequences at a time, so the float32 temporaries stay near
    # 1 GB even when the caches being filled take most of the device.
    per_seq = max(1, n * wl.num_kv_heads * wl.head_dim)
    step = max(1, (1 << 27) // per_seq)
    for b0 in range(0, wl.batch, step):
        b1 = min(wl.batch, b0 + step)
        sub = (b1 - b0,) + shape[1:]
        k[b0:b1] = torch.randn(sub, generator=g, device=device, dtype=torch.float32).to(dt)
        vv = torch.randn(sub, generator=g, device=device, dtype=torch.float32)
        scale = torch.empty(sub[:3] + (1,), device=device, dtype=torch.float32)
        scale.log_normal_(0.0, V_LOGNORMAL_SIGMA, generator=g)
        v[b0:b1] = (vv * scale).to(dt)
        del vv, scale
    return k, v


@dataclass
class PairTokenStream:
    """Deterministic inputs of ONE pair (sequence b, KV head h) of one layer.

    The same value recipe as TokenStream, drawn for this pair alone from
    SeedSequence([cfg_id, layer, seed_offset, b, h, 1]), so a long trajectory
    can be checked on a few sampled pairs without drawing the whole batch:
    K and V rows N(0, 1), one lognormal(0, 0.5) scale per V row, the G query
    heads' correlated walks, and (with dup_frac > 0) duplicated tokens that
    copy both rows of a uniformly chosen earlier token of the pair. Everything
    is rounded once to the storage dtype.
    """

    wl: Workload
    b: int
    h: int
    layer: int = 0
    seed_offset: int = 0
    _rngs: dict = field(init=False, repr=False)
    _q: np.ndarray = field(init=False, repr=False)
    _hist_k: np.ndarray = field(init=False, repr=False)
    _hist_v: np.ndarray = field(init=False, repr=False)
    tokens_emitted: int = field(init=False, default=0)

    def __post_init__(self):
        ss = np.random.SeedSequence([self.wl.cfg_id, self.layer, self.seed_offset,
                                     self.b, self.h, 1])
        self._rngs = {name: np.random.Generator(np.random.PCG64(k))
                      for name, k in zip(_STREAMS, ss.spawn(len(_STREAMS)))}
        self._q = _normalise_rows(self._rngs["q_walk"].standard_normal(
            (self.wl.group, self.wl.head_dim)))
        self._hist_k = np.zeros((0, self.wl.head_dim), dtype=np.float32)
        self._hist_v = np.zeros((0, self.wl.head_dim), dtype=np.float32)

    def _rows(self, count: int, k_stream: str, v_stream: str):
        wl = self.wl
        k = self._rngs[k_stream].standard_normal((count, wl.head_dim), dtype=np.float32)
        v = self._rngs[v_stream].standard_normal((count, wl.head_dim), dtype=np.float32)
        scale = self._rngs["v_scale"].lognormal(0.0, V_LOGNORMAL_SIGMA, size=count)
        v = v * scale.astype(np.float32)[:, None]
        k, v = round_to_dtype(k, wl.dtype), round_to_dtype(v, wl.dtype)
        if wl.dup_frac > 0.0:
            # Two uniforms per token, drawn in token order, so the stream does
            # not depend on how the tokens are grouped into calls.
            t0 = self.tokens_emitted
            du = self._rngs["dup"].random((count, 2))
            pick = du[:, 0] < wl.dup_frac
            u = du[:, 1]
            hist_k = np.concatenate([self._hist_k, k])
            hist_v = np.concatenate([self._hist_v, v])
            for j in np.flatnonzero(pick):
                t = t0 + int(j)
                if t == 0:
                    continue
                s = min(int(u[j] * t), t - 1)   # uniform over the t earlier tokens
                hist_k[t] = hist_k[s]
                hist_v[t] = hist_v[s]
            k, v = hist_k[t0:].copy(), hist_v[t0:].copy()
            self._hist_k, self._hist_v = hist_k, hist_v
        self.tokens_emitted += count
        return k, v

    def prefill(self, n: int):
        """The first n tokens: K, V [n][head_dim]."""
        return self._rows(n, "prefill_k", "prefill_v")

    def steps(self, count: int):
        """The next `count` decode steps: q [count][G][d], k_new and v_new
        [count][d]."""
        k, v = self._rows(count, "decode_k", "decode_v")
        q = np.empty((count, self.wl.group, self.wl.head_dim), dtype=np.float32)
        for t in range(count):
            q[t] = round_to_dtype(self._q.astype(np.float32), self.wl.dtype)
            z = self._rngs["q_walk"].standard_normal(self._q.shape)
            self._q = _normalise_rows(QUERY_WALK_KEEP * self._q + QUERY_WALK_NOISE * z)
        return q, k, v


def device_steps(wl: Workload, count: int, seed: int, device: str = "cuda"):
    """`count` decode-step inputs for the whole batch drawn on the device:
    q [count][batch][num_q_heads][d] (unit-RMS rows), k_new and v_new
    [count][batch][num_kv_heads][d] (V rows scaled by lognormal(0, 0.5)), in
    the storage dtype. Load for the pairs a test does not check."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q = torch.randn((count, wl.batch, wl.num_q_heads, wl.head_dim), generator=g, device=device)
    q = q * (wl.head_dim ** 0.5) / q.norm(dim=-1, keepdim=True)
    kv_shape = (count, wl.batch, wl.num_kv_heads, wl.head_dim)
    k = torch.randn(kv_shape, generator=g, device=device)
    v = torch.randn(kv_shape, generator=g, device=device)
    scale = torch.empty(kv_shape[:3] + (1,), device=device)
    scale.log_normal_(0.0, V_LOGNORMAL_SIGMA, generator=g)
    return q.to(dt), k.to(dt), (v * scale).to(dt)
