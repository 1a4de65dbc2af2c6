"""Packed attention over a rollout DAG on AMD MI355X -- Python binding of libdag_attn.

This module only marshals arguments to the C ABI declared in
``include/dag_attn.h``; every step of the computation runs in the library
(host compactor in C++, HIP kernels on the GPU).  PyTorch provides device
memory and the stream.  If the library cannot be loaded (or built in place),
importing this package fails.

Names follow the C ABI: :class:`Plan` wraps ``dag_build`` and the plan
queries, :func:`attn_fwd` / :func:`attn_bwd` wrap ``dag_attn_fwd`` /
``dag_attn_bwd``; :func:`gdn_fwd` / :func:`gdn_bwd` and :func:`logprob_fwd` /
:func:`logprob_bwd` likewise, with :meth:`Plan.logprob_map` for the position map, and
:func:`conv_fwd` / :func:`conv_bwd` for the short causal convolution.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DAG_ATTN_DEBUG=1 selects the device debug build (plan-table checks in the kernels)
DEBUG = os.environ.get("DAG_ATTN_DEBUG", "0") == "1"
LIB_PATH = os.path.join(_HERE, "libdag_attn_debug.so" if DEBUG else "libdag_attn.so")

DAG_OK = 0
STATUS = {0: "OK", 1: "INVALID", 2: "NOT_TOPO", 3: "MOUNT_CYCLE", 4: "MOUNT_RANGE",
          5: "SELF_ANCESTOR_MOUNT", 6: "OVERFLOW", 7: "WORKSPACE", 8: "UNSUPPORTED", 9: "DEVICE"}
DTYPE_BF16, DTYPE_FP32 = 0, 1


class DagNode(ctypes.Structure):
    _fields_ = [("parent", ctypes.c_int32), ("length", ctypes.c_int32),
                ("mount_first", ctypes.c_int32), ("mount_count", ctypes.c_int32)]


class DagMount(ctypes.Structure):
    _fields_ = [("src_node", ctypes.c_int32), ("begin", ctypes.c_int32), ("end", ctypes.c_int32)]


class DagBuildOpts(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("q_block", ctypes.c_int32),
                ("transitive", ctypes.c_int32), ("page_shuffle", ctypes.c_int32),
                ("gdn_chunk", ctypes.c_int32), ("view", ctypes.c_int32), ("pack_pages", ctypes.c_int32)]


class DagPlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("rows", "tokens", "pages", "query_pages", "visible_pairs",
                                             "flat_rows", "flat_pairs", "n_trajectories", "fwd_tiles",
                                             "bwd_entries")] + \
               [("max_position", ctypes.c_int32), ("transitive", ctypes.c_int32),
                ("gdn_chunk", ctypes.c_int32), ("gdn_rounds", ctypes.c_int32)] + \
               [(n, ctypes.c_int64) for n in ("gdn_sequences", "gdn_replay", "gdn_slots", "gdn_chunks",
                                             "gdn_segments")] + [("view", ctypes.c_int32),
                                                                 ("semantic_tokens", ctypes.c_int64),
                                                                 ("pack_pages", ctypes.c_int32)]

class DagPlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("fwd_tiles", "dkdv_groups", "dkdv_group_steps", "dkdv_pairs",
                                             "dkdv_pair_steps", "fwd_staged_bytes", "dq_staged_bytes",
                                             "dkdv_staged_bytes")]


VIEWS = {"mounted": 0, "mount_free": 1, "unshifted": 2}


class DagGdnSeq(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("round", "first_node", "last_node", "start", "fork",
                                             "own_tokens", "init_seq", "init_boundary")]


class DagAttnParams(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("rope_base", ctypes.c_float)]


class DagGdnParams(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("keep_states", ctypes.c_int32)]


class DagLogprobParams(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("n_pos", ctypes.c_int64), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


class DagConvParams(ctypes.Structure):
    _fields_ = [("channels", ctypes.c_int32), ("width", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32)]


class DagMbOpts(ctypes.Structure):
    _fields_ = [("replicas", ctypes.c_int32), ("exact_max", ctypes.c_int32), ("capacity", ctypes.c_int64)]


class DagMbInfo(ctypes.Structure):
    _fields_ = [("microbatches", ctypes.c_int32), ("exact", ctypes.c_int32),
                ("natural_microbatches", ctypes.c_int32), ("candidates", ctypes.c_int32),
                ("total_work", ctypes.c_int64), ("slot_critical_work", ctypes.c_int64),
                ("max_replica_work", ctypes.c_int64), ("trie_work", ctypes.c_int64)]


class DagError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.code = STATUS.get(status, str(status))


def _load() -> ctypes.CDLL:
    # PyTorch's HIP runtime must be the one the library binds to (it provides the device
    # memory and streams); loading torch first makes the dynamic linker reuse it.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        from . import build_lib
        build_lib.build(debug=DEBUG)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "dag_build": ([ctypes.POINTER(DagNode), I32, ctypes.POINTER(DagMount), I32,
                       ctypes.POINTER(DagBuildOpts), ctypes.POINTER(P)], I32),
        "dag_plan_destroy": ([P], None),
        "dag_plan_info_get": ([P, ctypes.POINTER(DagPlanInfo)], I32),
        "dag_plan_stats_get": ([P, ctypes.POINTER(DagPlanStats)], I32),
        "dag_plan_rows": ([P, P, P], I32),
        "dag_plan_starts": ([P, P], I32),
        "dag_plan_multiplicity": ([P, P], I32),
        "dag_plan_visibility": ([P, I32, P, I32, ctypes.POINTER(I32)], I32),
        "dag_plan_readers": ([P, I32, P, I32, ctypes.POINTER(I32)], I32),
        "dag_plan_node_ranges": ([P, I32, P, I32, ctypes.POINTER(I32)], I32),
        "dag_plan_upload": ([P, P], I32),
        "dag_plan_gdn_seqs": ([P, P, I32, ctypes.POINTER(I32)], I32),
        "dag_attn_workspace": ([P, ctypes.POINTER(DagAttnParams), ctypes.POINTER(SZ),
                                ctypes.POINTER(SZ)], I32),
        "dag_attn_fwd": ([P, ctypes.POINTER(DagAttnParams), P, P, P, P, P, P, P, SZ, P], I32),
        "dag_attn_bwd": ([P, ctypes.POINTER(DagAttnParams), P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "dag_attn_fwd_noalloc": ([P, ctypes.POINTER(DagAttnParams), P, P, P, P, P, P, P], I32),
        "dag_gdn_workspace": ([P, ctypes.POINTER(DagGdnParams), ctypes.POINTER(SZ), ctypes.POINTER(SZ)], I32),
        "dag_gdn_fwd": ([P, ctypes.POINTER(DagGdnParams), P, P, P, P, P, P, P, SZ, P], I32),
        "dag_gdn_bwd": ([P, ctypes.POINTER(DagGdnParams), P, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "dag_plan_logprob_map": ([P, P, I64, P, P, P, P, ctypes.POINTER(I64)], I32),
        "dag_logprob_fwd": ([ctypes.POINTER(DagLogprobParams), P, P, P, P, P, P, P], I32),
        "dag_logprob_bwd": ([ctypes.POINTER(DagLogprobParams), P, P, P, P, P, P, P, P], I32),
        "dag_conv_workspace": ([P, ctypes.POINTER(DagConvParams), ctypes.POINTER(SZ)], I32),
        "dag_conv_fwd": ([P, ctypes.POINTER(DagConvParams), P, P, P, P], I32),
        "dag_conv_bwd": ([P, ctypes.POINTER(DagConvParams), P, P, P, P, P, P, SZ, P], I32),
        "dag_trie_build": ([P, P, I32, I32, P, P, I64, P, P, ctypes.POINTER(I32), ctypes.POINTER(I64)], I32),
        "dag_microbatch_plan": ([P, P, I32, ctypes.POINTER(DagMbOpts), P, I32, P, P, P,
                                 ctypes.POINTER(DagMbInfo)], I32),
        "dag_attn_timing_enable": ([P, I32, I32], I32),
        "dag_attn_timing_read": ([P, P, P], I32),
        "dag_last_error": ([], ctypes.c_char_p),
        "dag_debug_build": ([], I32),
        "dag_debug_limit_pages": ([I32], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != DAG_OK:
        raise DagError(status, _lib.dag_last_error().decode())


def last_error() -> str:
    return _lib.dag_last_error().decode()


# ---------------------------------------------------------------------------
# plans
# ---------------------------------------------------------------------------

class Plan:
    """An immutable compiled DAG (``dag_build``).  ``spec`` has the node and mount
    tables as attributes ``parent, length, mount_first, mount_count, mount_src,
    mount_begin, mount_end``."""

    def __init__(self, spec, transitive: Optional[bool] = None, page_shuffle: int = 0, gdn_chunk: int = 0,
                 view: str = "mounted", pack: bool = False):
        if transitive is None:
            transitive = bool(getattr(spec, "meta", {}).get("transitive", True))
        n = len(spec.parent)
        nodes = (DagNode * max(n, 1))()
        for u in range(n):
            nodes[u] = DagNode(int(spec.parent[u]), int(spec.length[u]), int(spec.mount_first[u]),
                               int(spec.mount_count[u]))
        m = len(spec.mount_src)
        mounts = (DagMount * max(m, 1))()
        for i in range(m):
            mounts[i] = DagMount(int(spec.mount_src[i]), int(spec.mount_begin[i]), int(spec.mount_end[i]))
        opts = DagBuildOpts(64, 64, 1 if transitive else 0, int(page_shuffle), int(gdn_chunk), VIEWS[view],
                            1 if pack else 0)
        self._h = ctypes.c_void_p()
        _check(_lib.dag_build(nodes, n, mounts, m, ctypes.byref(opts), ctypes.byref(self._h)))
        info = DagPlanInfo()
        _check(_lib.dag_plan_info_get(self._h, ctypes.byref(info)))
        self.info = {f: getattr(info, f) for f, _ in DagPlanInfo._fields_}
        self.n_nodes = n
        self._rows = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.dag_plan_destroy(h)
            self._h = None

    @property
    def rows(self) -> int:
        return int(self.info["rows"])

    @property
    def tokens(self) -> int:
        return int(self.info["tokens"])

    def row_maps(self) -> Tuple[np.ndarray, np.ndarray]:
        """(row_of_token [U], pos_of_row [C]) as int32 arrays."""
        if self._rows is None:
            rot = np.zeros(max(self.tokens, 1), np.int32)
            por = np.zeros(max(self.rows, 1), np.int32)
            _check(_lib.dag_plan_rows(self._h, rot.ctypes.data, por.ctypes.data))
            self._rows = (rot[: self.tokens], por[: self.rows])
        return self._rows

    def stats(self) -> dict:
        """``dag_plan_stats_get``: tiles, dK/dV groups and pairs with their reader steps, and the
        bytes each attention kernel stages per KV head before any cache reuse."""
        st = DagPlanStats()
        _check(_lib.dag_plan_stats_get(self._h, ctypes.byref(st)))
        return {f: int(getattr(st, f)) for f, _ in DagPlanStats._fields_}

    def multiplicity(self) -> np.ndarray:
        """``dag_plan_multiplicity``: trajectories holding each token (node-major order), int32 [U]."""
        out = np.zeros(max(self.tokens, 1), np.int32)
        _check(_lib.dag_plan_multiplicity(self._h, out.ctypes.data))
        return out[: self.tokens]

    def _rows_query(self, fn, row: int) -> np.ndarray:
        n = ctypes.c_int32(0)
        _check(fn(self._h, int(row), None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), np.int32)
        _check(fn(self._h, int(row), out.ctypes.data, n.value, ctypes.byref(n)))
        return out[: n.value]

    def visibility(self, row: int) -> np.ndarray:
        """``dag_plan_visibility``: rows that query row ``row`` sees, as the forward reads the plan."""
        return self._rows_query(_lib.dag_plan_visibility, row)

    def readers(self, row: int) -> np.ndarray:
        """``dag_plan_readers``: query rows the dK/dV kernel sums into key row ``row``."""
        return self._rows_query(_lib.dag_plan_readers, row)

    def starts(self) -> np.ndarray:
        out = np.zeros(self.n_nodes, np.int32)
        _check(_lib.dag_plan_starts(self._h, out.ctypes.data))
        return out

    def node_ranges(self, u: int):
        """[(src, lo, hi), ...]: non-self visibility of node u in kernel visiting order."""
        n = ctypes.c_int32(0)
        _check(_lib.dag_plan_node_ranges(self._h, int(u), None, 0, ctypes.byref(n)))
        buf = np.zeros(max(3 * n.value, 3), np.int32)
        _check(_lib.dag_plan_node_ranges(self._h, int(u), buf.ctypes.data, n.value, ctypes.byref(n)))
        return [tuple(int(x) for x in buf[3 * i: 3 * i + 3]) for i in range(n.value)]

    def gdn_seqs(self):
        """The linear-attention schedule's sequences (``dag_plan_gdn_seqs``) as dicts."""
        n = ctypes.c_int32(0)
        _check(_lib.dag_plan_gdn_seqs(self._h, None, 0, ctypes.byref(n)))
        buf = (DagGdnSeq * max(n.value, 1))()
        _check(_lib.dag_plan_gdn_seqs(self._h, buf, n.value, ctypes.byref(n)))
        return [{f: getattr(buf[i], f) for f, _ in DagGdnSeq._fields_} for i in range(n.value)]

    def logprob_map(self, labels) -> dict:
        """``dag_plan_logprob_map``: labels [C] (vocabulary id per row) -> the semantic map.

        Returns int32 arrays ``pos_row``, ``pos_target`` [n], ``row_first`` [C+1], ``row_pos`` [n]."""
        lab = np.ascontiguousarray(labels, dtype=np.int32)
        if lab.shape != (self.rows,):
            raise ValueError(f"labels: expected [{self.rows}], got {lab.shape}")
        n = ctypes.c_int64(0)
        _check(_lib.dag_plan_logprob_map(self._h, lab.ctypes.data, 0, None, None, None, None, ctypes.byref(n)))
        k = n.value
        out = {"pos_row": np.zeros(max(k, 1), np.int32), "pos_target": np.zeros(max(k, 1), np.int32),
               "row_first": np.zeros(self.rows + 1, np.int32), "row_pos": np.zeros(max(k, 1), np.int32)}
        _check(_lib.dag_plan_logprob_map(self._h, lab.ctypes.data, k, out["pos_row"].ctypes.data,
                                         out["pos_target"].ctypes.data, out["row_first"].ctypes.data,
                                         out["row_pos"].ctypes.data, ctypes.byref(n)))
        for name in ("pos_row", "pos_target", "row_pos"):
            out[name] = out[name][:k]
        return out

    def upload(self, stream=None) -> None:
        _check(_lib.dag_plan_upload(self._h, _stream_ptr(stream)))

    KERNELS = ("prologue_fwd", "fwd", "prologue_bwd", "dkdv", "dq", "gdn_fwd", "gdn_states", "gdn_bwd",
               "conv_fwd", "conv_bwd")

    def timing_enable(self, enable: bool = True, capacity: int = 256) -> None:
        """Record HIP events around each kernel the library launches for this plan."""
        _check(_lib.dag_attn_timing_enable(self._h, 1 if enable else 0, int(capacity)))

    def timing_read(self):
        """{kernel: (total ms, launches)} since the last read (waits for the events)."""
        ms = np.zeros(len(self.KERNELS), np.float64)
        cnt = np.zeros(len(self.KERNELS), np.int64)
        _check(_lib.dag_attn_timing_read(self._h, ms.ctypes.data, cnt.ctypes.data))
        return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(self.KERNELS)}


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

@dataclass
class AttnParams:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str = "bf16"          # "bf16" or "fp32"
    scale: float = 0.0           # 0 -> 1/sqrt(head_dim)
    rope_base: float = 10000.0   # 0 -> no rotation
    grad_dtype: Optional[str] = None   # dq/dk/dv element type; None -> same as dtype

    def c(self) -> DagAttnParams:
        m = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}
        return DagAttnParams(self.n_q_heads, self.n_kv_heads, self.head_dim, m[self.dtype],
                             m[self.grad_dtype or self.dtype], float(self.scale), float(self.rope_base))

    @property
    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def torch_grad_dtype(self):
        import torch
        return torch.bfloat16 if (self.grad_dtype or self.dtype) == "bf16" else torch.float32


def _stream_ptr(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_bytes(plan: Plan, p: AttnParams) -> Tuple[int, int]:
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    cp = p.c()
    _check(_lib.dag_attn_workspace(plan._h, ctypes.byref(cp), ctypes.byref(f), ctypes.byref(b)))
    return int(f.value), int(b.value)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, rows, heads, d, dtype, device):
    if t.dtype != dtype or tuple(t.shape) != (rows, heads, d) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} [{rows}, {heads}, {d}] on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def attn_fwd(plan: Plan, p: AttnParams, q, k, v, o=None, lse=None, ws=None, stream=None, o_lo=None):
    """``dag_attn_fwd``: q [C,Hq,D], k/v [C,Hkv,D] in row layout -> (o [C,Hq,D], lse [C,Hq] fp32).

    For bf16, ``o_lo=True`` (or a tensor) also returns O's rounding residual, which
    :func:`attn_bwd` takes to form rowsum(dO * O) precisely; the result is then
    (o, lse, o_lo)."""
    import torch
    C, dt, dev = plan.rows, p.torch_dtype, q.device
    _check_tensor("q", q, C, p.n_q_heads, p.head_dim, dt, dev)
    _check_tensor("k", k, C, p.n_kv_heads, p.head_dim, dt, dev)
    _check_tensor("v", v, C, p.n_kv_heads, p.head_dim, dt, dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((C, p.n_q_heads), dtype=torch.float32, device=dev)
    need, _ = workspace_bytes(plan, p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    want_lo = o_lo is not None and o_lo is not False
    if o_lo is True:
        o_lo = torch.empty_like(q)
    lo_ptr = _ptr(o_lo) if want_lo else None
    cp = p.c()
    _check(_lib.dag_attn_fwd(plan._h, ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), lo_ptr,
                             _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return (o, lse, o_lo) if want_lo else (o, lse)


def attn_fwd_noalloc(plan: Plan, p: AttnParams, q, k, v, o, lse, o_lo=None, stream=None):
    """``dag_attn_fwd_noalloc``: the forward into caller-allocated ``o`` / ``lse`` (and ``o_lo``
    for bf16, or None) with the library's static device workspace; the plan must be uploaded."""
    C, dt, dev = plan.rows, p.torch_dtype, q.device
    _check_tensor("q", q, C, p.n_q_heads, p.head_dim, dt, dev)
    _check_tensor("k", k, C, p.n_kv_heads, p.head_dim, dt, dev)
    _check_tensor("v", v, C, p.n_kv_heads, p.head_dim, dt, dev)
    _check_tensor("o", o, C, p.n_q_heads, p.head_dim, dt, dev)
    if o_lo is not None:
        _check_tensor("o_lo", o_lo, C, p.n_q_heads, p.head_dim, dt, dev)
    cp = p.c()
    _check(_lib.dag_attn_fwd_noalloc(plan._h, ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     _ptr(o_lo) if o_lo is not None else None, _stream_ptr(stream)))
    return o, lse


def attn_bwd(plan: Plan, p: AttnParams, q, k, v, o, lse, dO, dq=None, dk=None, dv=None, ws=None,
             stream=None, o_lo=None):
    """``dag_attn_bwd``: returns (dq [C,Hq,D], dk [C,Hkv,D], dv [C,Hkv,D]).  For bf16, ``o_lo``
    (the forward's rounding residual of o) is required."""
    import torch
    C, dt, dev = plan.rows, p.torch_dtype, q.device
    for name, t, h in (("q", q, p.n_q_heads), ("k", k, p.n_kv_heads), ("v", v, p.n_kv_heads),
                       ("o", o, p.n_q_heads), ("dO", dO, p.n_q_heads)):
        _check_tensor(name, t, C, h, p.head_dim, dt, dev)
    gdt = p.torch_grad_dtype
    if dq is None:
        dq = torch.empty(q.shape, dtype=gdt, device=dev)
    if dk is None:
        dk = torch.empty(k.shape, dtype=gdt, device=dev)
    if dv is None:
        dv = torch.empty(v.shape, dtype=gdt, device=dev)
    for name, t, h in (("dq", dq, p.n_q_heads), ("dk", dk, p.n_kv_heads), ("dv", dv, p.n_kv_heads)):
        _check_tensor(name, t, C, h, p.head_dim, gdt, dev)
    _, need = workspace_bytes(plan, p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    cp = p.c()
    _check(_lib.dag_attn_bwd(plan._h, ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             _ptr(o_lo) if o_lo is not None else None, _ptr(dO), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# gated delta rule
# ---------------------------------------------------------------------------

@dataclass
class GdnParams:
    n_heads: int
    head_dim: int = 128
    scale: float = 0.0               # 0 -> 1
    grad_dtype: str = "bf16"         # dq/dk/dv element type: "bf16" or "fp32"
    keep_states: bool = False        # forward saves chunk states in ws for the backward

    def c(self) -> DagGdnParams:
        m = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}
        return DagGdnParams(self.n_heads, self.head_dim, DTYPE_BF16, m[self.grad_dtype], float(self.scale),
                            int(bool(self.keep_states)))

    @property
    def torch_grad_dtype(self):
        import torch
        return torch.bfloat16 if self.grad_dtype == "bf16" else torch.float32


def gdn_workspace_bytes(plan: Plan, p: GdnParams) -> Tuple[int, int]:
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    cp = p.c()
    _check(_lib.dag_gdn_workspace(plan._h, ctypes.byref(cp), ctypes.byref(f), ctypes.byref(b)))
    return int(f.value), int(b.value)


def _check_gates(name, t, rows, heads, device):
    import torch
    if t.dtype != torch.float32 or tuple(t.shape) != (rows, heads) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous float32 [{rows}, {heads}] on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def gdn_fwd(plan: Plan, p: GdnParams, q, k, v, beta, alpha, o=None, ws=None, stream=None):
    """``dag_gdn_fwd``: q, k, v [C,H,128] bf16, beta/alpha [C,H] fp32 -> o [C,H,128] bf16.
    With ``p.keep_states`` the caller passes ``ws`` (backward size) and hands the same
    buffer, untouched, to ``gdn_bwd``."""
    import torch
    if p.keep_states and ws is None:
        raise ValueError("keep_states: pass the workspace that the backward will read")
    C, dev = plan.rows, q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, C, p.n_heads, p.head_dim, torch.bfloat16, dev)
    _check_gates("beta", beta, C, p.n_heads, dev)
    _check_gates("alpha", alpha, C, p.n_heads, dev)
    if o is None:
        o = torch.empty_like(v)
    need, _ = gdn_workspace_bytes(plan, p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    cp = p.c()
    _check(_lib.dag_gdn_fwd(plan._h, ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                            _ptr(o), _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return o


def gdn_bwd(plan: Plan, p: GdnParams, q, k, v, beta, alpha, dO, ws=None, stream=None, out=None):
    """``dag_gdn_bwd``: returns (dq, dk, dv [C,H,128] grad_dtype, dbeta, dalpha [C,H] fp32).
    With ``p.keep_states``, ``ws`` must be the buffer the forward filled."""
    import torch
    if p.keep_states and ws is None:
        raise ValueError("keep_states: pass the workspace the forward filled")
    C, dev = plan.rows, q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _check_tensor(name, t, C, p.n_heads, p.head_dim, torch.bfloat16, dev)
    _check_gates("beta", beta, C, p.n_heads, dev)
    _check_gates("alpha", alpha, C, p.n_heads, dev)
    gdt = p.torch_grad_dtype
    if out is None:
        out = (torch.empty(q.shape, dtype=gdt, device=dev), torch.empty(k.shape, dtype=gdt, device=dev),
               torch.empty(v.shape, dtype=gdt, device=dev), torch.empty_like(beta), torch.empty_like(alpha))
    dq, dk, dv, db, da = out
    _, need = gdn_workspace_bytes(plan, p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    cp = p.c()
    _check(_lib.dag_gdn_bwd(plan._h, ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                            _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(da), _ptr(ws), ws.numel(),
                            _stream_ptr(stream)))
    return dq, dk, dv, db, da


# ---------------------------------------------------------------------------
# short causal convolution
# ---------------------------------------------------------------------------

ACT_NONE, ACT_SILU = 0, 1


@dataclass
class ConvParams:
    channels: int
    width: int = 4
    activation: str = "silu"         # "none" or "silu"
    grad_dtype: str = "bf16"         # dx element type: "bf16" or "fp32"

    def c(self) -> DagConvParams:
        a = {"none": ACT_NONE, "silu": ACT_SILU}[self.activation]
        return DagConvParams(self.channels, self.width, a, {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}[self.grad_dtype])


def conv_workspace_bytes(plan: Plan, p: ConvParams) -> int:
    b = ctypes.c_size_t(0)
    cp = p.c()
    _check(_lib.dag_conv_workspace(plan._h, ctypes.byref(cp), ctypes.byref(b)))
    return int(b.value)


def _check_conv(name, t, rows, ch, dtype, device):
    if t.dtype != dtype or tuple(t.shape) != (rows, ch) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} [{rows}, {ch}] on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def conv_fwd(plan: Plan, p: ConvParams, x, weight, y=None, stream=None):
    """``dag_conv_fwd``: x [C, Ch] bf16, weight [Ch, w] fp32 -> y [C, Ch] bf16."""
    import torch
    _check_conv("x", x, plan.rows, p.channels, torch.bfloat16, x.device)
    _check_conv("weight", weight, p.channels, p.width, torch.float32, x.device)
    if y is None:
        y = torch.empty_like(x)
    cp = p.c()
    _check(_lib.dag_conv_fwd(plan._h, ctypes.byref(cp), _ptr(x), _ptr(weight), _ptr(y), _stream_ptr(stream)))
    return y


def conv_bwd(plan: Plan, p: ConvParams, x, weight, dy, dx=None, dweight=None, ws=None, stream=None):
    """``dag_conv_bwd``: returns (dx [C, Ch] grad_dtype, dweight [Ch, w] fp32)."""
    import torch
    _check_conv("x", x, plan.rows, p.channels, torch.bfloat16, x.device)
    _check_conv("dy", dy, plan.rows, p.channels, torch.bfloat16, x.device)
    _check_conv("weight", weight, p.channels, p.width, torch.float32, x.device)
    if dx is None:
        dx = torch.empty(x.shape, dtype=torch.bfloat16 if p.grad_dtype == "bf16" else torch.float32, device=x.device)
    if dweight is None:
        dweight = torch.empty_like(weight)
    if ws is None:
        ws = torch.empty(max(conv_workspace_bytes(plan, p), 16), dtype=torch.uint8, device=x.device)
    cp = p.c()
    _check(_lib.dag_conv_bwd(plan._h, ctypes.byref(cp), _ptr(x), _ptr(weight), _ptr(dy), _ptr(dx), _ptr(dweight),
                             _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return dx, dweight


# ---------------------------------------------------------------------------
# compact-to-semantic log-probabilities
# ---------------------------------------------------------------------------

_LP_DT = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}


def _lp_params(z, n_pos: int, grad_dtype: str) -> DagLogprobParams:
    import torch
    if z.dim() != 2 or not z.is_contiguous() or z.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"z: expected contiguous bf16/fp32 [C, V], got {z.dtype} {tuple(z.shape)}")
    dt = DTYPE_BF16 if z.dtype == torch.bfloat16 else DTYPE_FP32
    return DagLogprobParams(z.shape[0], int(n_pos), z.shape[1], dt, _LP_DT[grad_dtype])


def _check_map(z, row_first, row_pos, pos_target):
    import torch
    for name, t, n in (("row_first", row_first, z.shape[0] + 1), ("row_pos", row_pos, pos_target.numel()),
                       ("pos_target", pos_target, row_pos.numel())):
        if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != n or not t.is_contiguous() or t.device != z.device:
            raise ValueError(f"{name}: expected contiguous int32 [{n}] on {z.device}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def logprob_fwd(z, row_first, row_pos, pos_target, lse=None, lam=None, stream=None):
    """``dag_logprob_fwd``: z [C, V] (bf16/fp32), the row-grouped map (int32 device tensors)
    -> (lse [C] fp32, lambda [n] fp32)."""
    import torch
    _check_map(z, row_first, row_pos, pos_target)
    n = pos_target.numel()
    if lse is None:
        lse = torch.empty(z.shape[0], dtype=torch.float32, device=z.device)
    if lam is None:
        lam = torch.empty(n, dtype=torch.float32, device=z.device)
    cp = _lp_params(z, n, "fp32")
    _check(_lib.dag_logprob_fwd(ctypes.byref(cp), _ptr(z), _ptr(row_first), _ptr(row_pos), _ptr(pos_target),
                                _ptr(lse), _ptr(lam), _stream_ptr(stream)))
    return lse, lam


def logprob_bwd(z, lse, row_first, row_pos, pos_target, g, grad_dtype: str = "bf16", dz=None, stream=None):
    """``dag_logprob_bwd``: g [n] fp32 (dL/dlambda) -> dz [C, V] in ``grad_dtype``."""
    import torch
    _check_map(z, row_first, row_pos, pos_target)
    n = pos_target.numel()
    if g.dtype != torch.float32 or g.numel() != n or not g.is_contiguous():
        raise ValueError(f"g: expected contiguous float32 [{n}]")
    if lse.dtype != torch.float32 or lse.numel() != z.shape[0]:
        raise ValueError(f"lse: expected float32 [{z.shape[0]}]")
    if dz is None:
        dz = torch.empty(z.shape, dtype=torch.bfloat16 if grad_dtype == "bf16" else torch.float32, device=z.device)
    cp = _lp_params(z, n, grad_dtype)
    _check(_lib.dag_logprob_bwd(ctypes.byref(cp), _ptr(z), _ptr(lse), _ptr(row_first), _ptr(row_pos),
                                _ptr(pos_target), _ptr(g), _ptr(dz), _stream_ptr(stream)))
    return dz


# ---------------------------------------------------------------------------
# trajectory ingestion and prefix-aware microbatch planning (host only)
# ---------------------------------------------------------------------------

def _traj_arrays(trajs):
    """(tokens int32, offsets int64) from a list of sequences, or passed through when
    ``trajs`` already is such a pair."""
    if isinstance(trajs, tuple) and len(trajs) == 2 and isinstance(trajs[0], np.ndarray):
        tok, off = np.ascontiguousarray(trajs[0], np.int32), np.ascontiguousarray(trajs[1], np.int64)
        return (tok if tok.size else np.zeros(1, np.int32)), off
    off = np.zeros(len(trajs) + 1, np.int64)
    for i, t in enumerate(trajs):
        off[i + 1] = off[i] + len(t)
    tok = np.zeros(max(int(off[-1]), 1), np.int32)
    for i, t in enumerate(trajs):
        tok[off[i]:off[i + 1]] = np.asarray(t, np.int32)
    return tok, off


def _n_traj(trajs) -> int:
    if isinstance(trajs, tuple) and len(trajs) == 2 and isinstance(trajs[0], np.ndarray):
        return len(trajs[1]) - 1
    return len(trajs)


def trie_build(trajs) -> dict:
    """``dag_trie_build``: raw token sequences (a list, or a (tokens, offsets) pair of
    arrays) -> the trie as a node table.

    Returns {"parent", "length" (int32 [n_nodes]), "node_tok_off" (int64 [n_nodes+1]),
    "node_tokens" (int32), "leaf_of_traj" (int32 [N])} plus ``spec`` (a node-table object
    accepted by :class:`Plan`)."""
    tok, off = _traj_arrays(trajs)
    N = _n_traj(trajs)
    nn, nt = ctypes.c_int32(0), ctypes.c_int64(0)
    _check(_lib.dag_trie_build(tok.ctypes.data, off.ctypes.data, N, 0, None, None, 0, None, None,
                               ctypes.byref(nn), ctypes.byref(nt)))
    nodes = (DagNode * max(nn.value, 1))()
    noff = np.zeros(nn.value + 1, np.int64)
    ntok = np.zeros(max(nt.value, 1), np.int32)
    leaf = np.zeros(N, np.int32)
    _check(_lib.dag_trie_build(tok.ctypes.data, off.ctypes.data, N, nn.value, nodes, noff.ctypes.data,
                               nt.value, ntok.ctypes.data, leaf.ctypes.data, ctypes.byref(nn), ctypes.byref(nt)))
    parent = np.array([nodes[i].parent for i in range(nn.value)], np.int32)
    length = np.array([nodes[i].length for i in range(nn.value)], np.int32)

    class _Spec:
        pass
    spec = _Spec()
    spec.parent, spec.length = parent, length
    spec.mount_first = np.zeros(nn.value, np.int32)
    spec.mount_count = np.zeros(nn.value, np.int32)
    spec.mount_src = spec.mount_begin = spec.mount_end = np.zeros(0, np.int32)
    spec.n_tokens = int(nt.value)
    spec.meta = {"transitive": True}
    return {"parent": parent, "length": length, "node_tok_off": noff, "node_tokens": ntok[:nt.value],
            "leaf_of_traj": leaf, "spec": spec}


def microbatch_plan(trajs, replicas: int, capacity: int, exact_max: int = 0) -> dict:
    """``dag_microbatch_plan``: {"mb_of_traj", "replica", "slot", "work", "info"}."""
    tok, off = _traj_arrays(trajs)
    N = _n_traj(trajs)
    o = DagMbOpts(int(replicas), int(exact_max), int(capacity))
    info = DagMbInfo()
    _check(_lib.dag_microbatch_plan(tok.ctypes.data, off.ctypes.data, N, ctypes.byref(o), None, 0, None,
                                    None, None, ctypes.byref(info)))
    K = info.microbatches
    mb = np.zeros(N, np.int32)
    rep, slot = np.zeros(max(K, 1), np.int32), np.zeros(max(K, 1), np.int32)
    work = np.zeros(max(K, 1), np.int64)
    _check(_lib.dag_microbatch_plan(tok.ctypes.data, off.ctypes.data, N, ctypes.byref(o),
                                    mb.ctypes.data, K, rep.ctypes.data, slot.ctypes.data, work.ctypes.data,
                                    ctypes.byref(info)))
    return {"mb_of_traj": mb, "replica": rep[:K], "slot": slot[:K], "work": work[:K],
            "info": {f: getattr(info, f) for f, _ in DagMbInfo._fields_}}


# ---------------------------------------------------------------------------
# layout helpers (token-major <-> row layout); pure data movement
# ---------------------------------------------------------------------------

def to_rows(plan: Plan, x_tok, fill: float = 0.0):
    """Scatter token-major [U, H, D] into the plan's row layout [C, H, D] (padding = fill)."""
    import torch
    rot, _ = plan.row_maps()
    out = torch.full((plan.rows,) + tuple(x_tok.shape[1:]), fill, dtype=x_tok.dtype, device=x_tok.device)
    if plan.tokens:
        out[torch.as_tensor(rot, dtype=torch.long, device=x_tok.device)] = x_tok
    return out


def from_rows(plan: Plan, x_rows):
    """Gather the plan's row layout [C, ...] back to token-major [U, ...]."""
    import torch
    rot, _ = plan.row_maps()
    return x_rows[torch.as_tensor(rot, dtype=torch.long, device=x_rows.device)]


__all__ = ["Plan", "AttnParams", "GdnParams", "DagError", "attn_fwd", "attn_fwd_noalloc", "attn_bwd", "workspace_bytes", "gdn_fwd",
           "gdn_bwd", "gdn_workspace_bytes", "ConvParams", "conv_fwd", "conv_bwd", "conv_workspace_bytes",
           "logprob_fwd", "logprob_bwd", "trie_build", "microbatch_plan", "to_rows", "from_rows", "last_error",
           "LIB_PATH"]
