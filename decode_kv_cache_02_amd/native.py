"""ctypes binding of liblongflow.so (include/longflow.h), same names as the C ABI.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device addresses and the current HIP stream are passed
to the library. Every step of the computation runs in the library's kernels.
If the library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "liblongflow.so")
# The measurement build (decode_kv_cache_02_amd/build.py --phases): the same
# library with the phase stamps of lf_probe_decode_phases compiled in.
PHASES_LIB_PATH = os.path.join(os.path.dirname(LIB_PATH), "liblongflow_phases.so")

LF_OK = 0
LF_ERR_INVALID_ARG = 1
LF_ERR_UNSUPPORTED = 2
LF_ERR_CAPACITY = 3
LF_ERR_OOM = 4
LF_ERR_HIP = 5
LF_ERR_SCRATCH = 6

LF_DTYPE_F32 = 0
LF_DTYPE_BF16 = 1
LF_MODE_EVICT = 0
LF_MODE_FULL = 1
LF_ORDER_SAME_STEP = 0
LF_ORDER_DEFERRED = 1
LF_SCOPE_KV_HEAD = 0
LF_SCOPE_SEQUENCE = 1
LF_NORM_L1 = 0
LF_NORM_L2 = 1

DTYPES = {"f32": LF_DTYPE_F32, "bf16": LF_DTYPE_BF16}
MODES = {"evict": LF_MODE_EVICT, "full": LF_MODE_FULL}
ORDERS = {"same_step": LF_ORDER_SAME_STEP, "deferred": LF_ORDER_DEFERRED}
SCOPES = {"kv_head": LF_SCOPE_KV_HEAD, "sequence": LF_SCOPE_SEQUENCE}
NORMS = {"l1": LF_NORM_L1, "l2": LF_NORM_L2}


class lf_config(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("budget", ctypes.c_int32),
        ("sink_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("order", ctypes.c_int32),
        ("scope", ctypes.c_int32),
        ("norm", ctypes.c_int32),
    ]


class lf_view(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("vnorm", ctypes.c_void_p),
        ("fill", ctypes.c_void_p),
        ("victim", ctypes.c_void_p),
        ("pair_stride", ctypes.c_int64),
        ("slots_padded", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
    ]


# (name, restype, argtypes) of every exported function of include/longflow.h
SIGNATURES = [
    ("lf_cache_bytes", ctypes.c_int, [ctypes.POINTER(lf_config), ctypes.POINTER(ctypes.c_size_t)]),
    ("lf_cache_create", ctypes.c_int, [ctypes.POINTER(lf_config), ctypes.POINTER(ctypes.c_void_p)]),
    ("lf_prefill_fill", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.c_int32, ctypes.c_void_p]),
    ("lf_decode_step", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    ("lf_decode_step_noalloc", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p]),
    ("lf_cache_view", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(lf_view)]),
    ("lf_cache_snapshot", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    ("lf_seq_reset", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                     ctypes.c_void_p]),
    ("lf_cache_set_splits", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("lf_cache_set_waves", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("lf_cache_set_loop", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("lf_cache_set_grid", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("lf_cache_set_stream", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("lf_cache_max_splits", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
    ("lf_fill_levels", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    ("lf_cache_destroy", None, [ctypes.c_void_p]),
    ("lf_status_str", ctypes.c_char_p, [ctypes.c_int]),
    # include/longflow_probe.h
    ("lf_probe_stream_read", ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p]),
    ("lf_probe_hbm_attributes", ctypes.c_int, [ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_int32)]),
    ("lf_probe_stream_plan", ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int32)]),
    ("lf_probe_stream_read_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("lf_probe_decode_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    ("lf_probe_decode_phases", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                                               ctypes.c_void_p]),
]

_lib = None


class LongFlowError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblongflow.so once; raises if it has not been built.

    torch is imported first: it ships a HIP runtime with the same SONAME as
    the system one, and the library must bind to that one copy rather than
    bring a second runtime into the process.
    """
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the process's HIP runtime)
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m decode_kv_cache_02_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().lf_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != LF_OK:
        raise LongFlowError(status, where)


def make_config(num_layers, batch, num_q_heads, num_kv_heads, head_dim, budget,
                sink_size=0, softmax_scale=0.0, dtype="bf16", mode="evict",
                order="same_step", scope="kv_head", norm="l1") -> lf_config:
    pick = lambda table, x: table[x] if isinstance(x, str) else int(x)
    return lf_config(int(num_layers), int(batch), int(num_q_heads), int(num_kv_heads),
                     int(head_dim), int(budget), int(sink_size), float(softmax_scale),
                     pick(DTYPES, dtype), pick(MODES, mode), pick(ORDERS, order),
                     pick(SCOPES, scope), pick(NORMS, norm))


# ----------------------------------------------------------------------------
# C-ABI names
# ----------------------------------------------------------------------------

def lf_cache_bytes(cfg: lf_config) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().lf_cache_bytes(ctypes.byref(cfg), ctypes.byref(out)), "lf_cache_bytes")
    return int(out.value)


def lf_cache_create(cfg: lf_config) -> int:
    h = ctypes.c_void_p(None)
    _check(load_library().lf_cache_create(ctypes.byref(cfg), ctypes.byref(h)), "lf_cache_create")
    return int(h.value)


def lf_cache_destroy(handle: Optional[int]) -> None:
    load_library().lf_cache_destroy(ctypes.c_void_p(handle))


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def lf_prefill_fill(handle: int, layer: int, k, v, n_per_seq, n_max: int, stream=None) -> None:
    """`n_per_seq` must hold the cache's batch of entries: the library reads that many."""
    n = np.ascontiguousarray(n_per_seq, dtype=np.int32)
    kp = k.data_ptr() if k is not None else 0
    vp = v.data_ptr() if v is not None else 0
    st = load_library().lf_prefill_fill(
        ctypes.c_void_p(handle), int(layer), ctypes.c_void_p(kp), ctypes.c_void_p(vp),
        n.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(n_max),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check(st, "lf_prefill_fill")


def lf_decode_step(handle: int, layer: int, q, k_new, v_new, out, evicted_slot, stream=None) -> None:
    st = load_library().lf_decode_step(
        ctypes.c_void_p(handle), int(layer), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(evicted_slot.data_ptr()),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check(st, "lf_decode_step")


def lf_decode_step_noalloc(handle: int, layer: int, q, k_new, v_new, out, evicted_slot,
                           stream=None) -> None:
    st = load_library().lf_decode_step_noalloc(
        ctypes.c_void_p(handle), int(layer), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(evicted_slot.data_ptr()),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check(st, "lf_decode_step_noalloc")


def lf_cache_view(handle: int, layer: int) -> lf_view:
    v = lf_view()
    _check(load_library().lf_cache_view(ctypes.c_void_p(handle), int(layer), ctypes.byref(v)),
           "lf_cache_view")
    return v


def lf_cache_snapshot(handle: int, layer: int, k=None, v=None, vnorm=None, fill=None,
                      victim=None, stream=None) -> None:
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    _check(load_library().lf_cache_snapshot(ctypes.c_void_p(handle), int(layer), ptr(k), ptr(v),
                                            ptr(vnorm), ptr(fill), ptr(victim),
                                            ctypes.c_void_p(_stream_ptr(stream))),
           "lf_cache_snapshot")


def lf_seq_reset(handle: int, seqs, stream=None) -> None:
    s = np.ascontiguousarray(seqs, dtype=np.int32)
    _check(load_library().lf_seq_reset(ctypes.c_void_p(handle),
                                       s.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                       int(s.size), ctypes.c_void_p(_stream_ptr(stream))),
           "lf_seq_reset")


def lf_cache_set_splits(handle: int, splits: int) -> None:
    _check(load_library().lf_cache_set_splits(ctypes.c_void_p(handle), int(splits)),
           "lf_cache_set_splits")


def lf_cache_set_waves(handle: int, waves: int) -> None:
    _check(load_library().lf_cache_set_waves(ctypes.c_void_p(handle), int(waves)),
           "lf_cache_set_waves")


LOOPS = {"auto": 0, "phased": 1, "interleaved": 2}


def lf_cache_set_loop(handle: int, loop) -> None:
    value = LOOPS[loop] if isinstance(loop, str) else int(loop)
    _check(load_library().lf_cache_set_loop(ctypes.c_void_p(handle), value), "lf_cache_set_loop")


def lf_cache_set_grid(handle: int, workgroups: int) -> None:
    _check(load_library().lf_cache_set_grid(ctypes.c_void_p(handle), int(workgroups)),
           "lf_cache_set_grid")


def lf_cache_set_stream(handle: int, tiles: int) -> None:
    _check(load_library().lf_cache_set_stream(ctypes.c_void_p(handle), int(tiles)),
           "lf_cache_set_stream")


def lf_cache_max_splits(handle: int) -> int:
    v = ctypes.c_int32(0)
    _check(load_library().lf_cache_max_splits(ctypes.c_void_p(handle), ctypes.byref(v)),
           "lf_cache_max_splits")
    return int(v.value)


def lf_fill_levels(handle: int, layer: int, batch: int) -> np.ndarray:
    """`batch` must be the cache's batch: the library writes that many entries."""
    out = np.zeros(batch, dtype=np.int32)
    _check(load_library().lf_fill_levels(ctypes.c_void_p(handle), int(layer),
                                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
           "lf_fill_levels")
    return out


def lf_status_str(status: int) -> str:
    return status_str(status)


def lf_probe_stream_read(buf, workgroups: int, sink, stream=None) -> None:
    """Read the device tensor `buf` once (include/longflow_probe.h)."""
    _check(load_library().lf_probe_stream_read(
        ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(buf.numel() * buf.element_size()),
        int(workgroups), ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(_stream_ptr(stream))),
        "lf_probe_stream_read")


def lf_probe_stream_read_timing(buf, workgroups: int, sink, records, stream=None) -> None:
    """lf_probe_stream_read with per-workgroup timing records (int64 device
    tensor [workgroups][4]; include/longflow_probe.h)."""
    _check(load_library().lf_probe_stream_read_timing(
        ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(buf.numel() * buf.element_size()),
        int(workgroups), ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(records.data_ptr()),
        ctypes.c_void_p(_stream_ptr(stream))), "lf_probe_stream_read_timing")


PLAN_FIELDS = ("grid", "sk_first", "sk_pairs", "sk_tiles", "sk_q", "sk_wgs", "sk_stride", "waves")


def lf_probe_stream_plan(pairs: int, n_max: int, cus: int, resident4: int, fits8: bool, rows: int,
                         stride: int, forced_stream: int = 0, forced_grid: int = 0) -> dict:
    """The library's launch plan for an evicting main-path layer (host only)."""
    out = (ctypes.c_int32 * 8)()
    _check(load_library().lf_probe_stream_plan(int(pairs), int(n_max), int(cus), int(resident4),
                                               int(bool(fits8)), int(rows), int(stride),
                                               int(forced_stream), int(forced_grid), out),
           "lf_probe_stream_plan")
    return dict(zip(PLAN_FIELDS, list(out)))


def _check_records(records, width: int) -> None:
    """The kernel writes `width` uint64 words per workgroup: the tensor must
    be a contiguous int64 device tensor [capacity][width]."""
    import torch
    if (records.dtype != torch.int64 or records.dim() != 2 or records.shape[1] != width
            or not records.is_contiguous() or not records.is_cuda):
        raise ValueError(f"records must be a contiguous int64 device tensor [capacity][{width}]")


def lf_probe_decode_timing(handle: int, layer: int, q, k_new, v_new, out, evicted_slot, records,
                           stream=None) -> int:
    """One lf_decode_step writing per-workgroup timing records (int64 device
    tensor [capacity][4]); returns the launch's workgroup count."""
    _check_records(records, 4)
    wgs = ctypes.c_int32(0)
    _check(load_library().lf_probe_decode_timing(
        ctypes.c_void_p(handle), int(layer), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(evicted_slot.data_ptr()),
        ctypes.c_void_p(records.data_ptr()), int(records.shape[0]), ctypes.byref(wgs),
        ctypes.c_void_p(_stream_ptr(stream))), "lf_probe_decode_timing")
    return int(wgs.value)


def lf_probe_decode_phases(handle: int, layer: int, q, k_new, v_new, out, evicted_slot, records,
                           phases, stream=None) -> int:
    """lf_probe_decode_timing that also records when each phase of every
    workgroup's step ended (int64 device tensors records [capacity][4] and
    phases [capacity][8]; include/longflow_probe.h); returns the launch's
    workgroup count."""
    _check_records(records, 4)
    _check_records(phases, 8)
    if phases.shape[0] != records.shape[0]:
        raise ValueError("records and phases must have the same capacity")
    wgs = ctypes.c_int32(0)
    _check(load_library().lf_probe_decode_phases(
        ctypes.c_void_p(handle), int(layer), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(evicted_slot.data_ptr()),
        ctypes.c_void_p(records.data_ptr()), ctypes.c_void_p(phases.data_ptr()),
        int(records.shape[0]), ctypes.byref(wgs), ctypes.c_void_p(_stream_ptr(stream))),
        "lf_probe_decode_phases")
    return int(wgs.value)


def lf_probe_hbm_attributes():
    """(memory clock kHz, bus width bits) of the current device
    (include/longflow_probe.h)."""
    clk, width = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().lf_probe_hbm_attributes(ctypes.byref(clk), ctypes.byref(width)),
           "lf_probe_hbm_attributes")
    return int(clk.value), int(width.value)


def untile_k(k_tiled, head_dim: int):
    """Row-major view of a K snapshot [..., slots_padded * head_dim] stored in
    the tiled MFMA-operand layout documented in include/longflow.h."""
    elem_bytes = k_tiled.element_size()
    per_chunk = 16 // elem_bytes                  # elements per 16-byte chunk
    blocks = head_dim * elem_bytes // 64          # 1 KB blocks per 16-slot tile
    lead = tuple(k_tiled.shape[:-1])
    tiles = k_tiled.shape[-1] // (16 * head_dim)
    t = k_tiled.reshape(lead + (tiles, blocks, 16, 4, per_chunk))   # tile, block, slot, j, elem
    nd = len(lead)
    t = t.permute(*range(nd), nd, nd + 2, nd + 1, nd + 3, nd + 4)   # tile, slot, block, j, elem
    return t.reshape(lead + (tiles * 16, head_dim))


# ----------------------------------------------------------------------------
# Convenience owner of one handle, with tensor checks
# ----------------------------------------------------------------------------

class LongFlowCache:
    """Owns one lf_cache handle. Tensors are torch device tensors in the cache dtype."""

    def __init__(self, num_layers, batch, num_q_heads, num_kv_heads, head_dim, budget,
                 sink_size=0, softmax_scale=0.0, dtype="bf16", mode="evict",
                 order="same_step", scope="kv_head", norm="l1"):
        import torch
        self.cfg = make_config(num_layers, batch, num_q_heads, num_kv_heads, head_dim, budget,
                               sink_size, softmax_scale, dtype, mode, order, scope, norm)
        self.dtype = dtype
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.num_layers, self.batch = int(num_layers), int(batch)
        self.hq, self.hkv, self.head_dim = int(num_q_heads), int(num_kv_heads), int(head_dim)
        self.budget = int(budget)
        self.handle = lf_cache_create(self.cfg)

    @property
    def nbytes(self) -> int:
        return lf_cache_bytes(self.cfg)

    def _check_tensor(self, t, shape, name, dtype=None):
        import torch
        dtype = self.torch_dtype if dtype is None else dtype
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, "
                             f"got {t.dtype} {tuple(t.shape)}")

    def prefill(self, layer, k, v, n_per_seq, stream=None):
        n_per_seq = np.asarray(n_per_seq, dtype=np.int32)
        if n_per_seq.shape != (self.batch,):
            raise ValueError(f"n_per_seq: expected shape ({self.batch},), got {n_per_seq.shape}")
        n_max = int(k.shape[1]) if k is not None else 0
        if k is not None:
            self._check_tensor(k, (self.batch, n_max, self.hkv, self.head_dim), "k")
            self._check_tensor(v, (self.batch, n_max, self.hkv, self.head_dim), "v")
        lf_prefill_fill(self.handle, layer, k, v, n_per_seq, n_max, stream)

    def decode_step(self, layer, q, k_new, v_new, out, evicted_slot, stream=None,
                    noalloc: bool = False):
        """lf_decode_step, or lf_decode_step_noalloc when `noalloc`."""
        import torch
        self._check_tensor(q, (self.batch, self.hq, self.head_dim), "q")
        self._check_tensor(k_new, (self.batch, self.hkv, self.head_dim), "k_new")
        self._check_tensor(v_new, (self.batch, self.hkv, self.head_dim), "v_new")
        self._check_tensor(out, (self.batch, self.hq, self.head_dim), "out")
        self._check_tensor(evicted_slot, (self.batch, self.hkv), "evicted_slot", torch.int32)
        fn = lf_decode_step_noalloc if noalloc else lf_decode_step
        fn(self.handle, layer, q, k_new, v_new, out, evicted_slot, stream)

    def seq_reset(self, seqs, stream=None) -> None:
        lf_seq_reset(self.handle, seqs, stream)

    def step_args(self, layer, q, k_new, v_new, out, evicted_slot, stream=None):
        """Check the tensors once and return the ctypes argument tuple of one
        lf_decode_step call, for callers that issue the same step many times
        (the tensors must stay alive and unchanged in shape)."""
        import torch
        self._check_tensor(q, (self.batch, self.hq, self.head_dim), "q")
        self._check_tensor(k_new, (self.batch, self.hkv, self.head_dim), "k_new")
        self._check_tensor(v_new, (self.batch, self.hkv, self.head_dim), "v_new")
        self._check_tensor(out, (self.batch, self.hq, self.head_dim), "out")
        self._check_tensor(evicted_slot, (self.batch, self.hkv), "evicted_slot", torch.int32)
        return (ctypes.c_void_p(self.handle), int(layer), ctypes.c_void_p(q.data_ptr()),
                ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(evicted_slot.data_ptr()),
                ctypes.c_void_p(_stream_ptr(stream)))

    @staticmethod
    def step_prepared(args) -> None:
        """One lf_decode_step with arguments from step_args."""
        _check(load_library().lf_decode_step(*args), "lf_decode_step")

    def set_splits(self, splits: int) -> None:
        lf_cache_set_splits(self.handle, splits)

    def set_waves(self, waves: int) -> None:
        lf_cache_set_waves(self.handle, waves)

    def set_loop(self, loop) -> None:
        """'auto' (or 0), 'phased' (1) or 'interleaved' (2)."""
        lf_cache_set_loop(self.handle, loop)

    def set_grid(self, workgroups: int) -> None:
        """0 automatic, -1 one workgroup per pair, n > 0 n workgroups taking
        whole pairs in turn (evicting main path with 4 waves)."""
        lf_cache_set_grid(self.handle, workgroups)

    def set_stream(self, tiles: int) -> None:
        """0 automatic, n > 0 a stream launch over every pair with n tiles
        per workgroup (evicting main path with 4 waves, no split)."""
        lf_cache_set_stream(self.handle, tiles)

    @property
    def max_splits(self) -> int:
        return lf_cache_max_splits(self.handle)

    def view(self, layer) -> lf_view:
        return lf_cache_view(self.handle, layer)

    def fill_levels(self, layer) -> np.ndarray:
        return lf_fill_levels(self.handle, layer, self.batch)

    def snapshot(self, layer, with_victim: bool = False):
        """Copies of one layer: K, V [batch][hkv][slots_pad][d] (K un-tiled to
        row-major), the ||v|| sidecar [batch][hkv][slots_pad], fill [batch][hkv]
        and, if asked, the pending victims [batch][hkv]; device tensors,
        stream-ordered."""
        import torch
        slots = self.view(layer).slots_padded
        k = torch.empty((self.batch, self.hkv, slots * self.head_dim), dtype=self.torch_dtype,
                        device="cuda")
        v = torch.empty_like(k)
        vn = torch.empty((self.batch, self.hkv, slots), dtype=torch.float32, device="cuda")
        fill = torch.empty((self.batch, self.hkv), dtype=torch.int32, device="cuda")
        victim = torch.empty_like(fill) if with_victim else None
        lf_cache_snapshot(self.handle, layer, k, v, vn, fill, victim)
        res = (untile_k(k, self.head_dim), v.view(self.batch, self.hkv, slots, self.head_dim),
               vn, fill)
        return res + (victim,) if with_victim else res

    def close(self):
        if getattr(self, "handle", None):
            lf_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

