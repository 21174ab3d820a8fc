"""ctypes binding of ``libsparsepr.so`` (declared in ``include/sparsepr.h``).

Argument marshalling only: torch tensors are used for device memory and the
current HIP stream; every step of the operator runs in the library's kernels.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import build as _build
from .configs import Params

_c_i32 = ctypes.c_int32
_c_p = ctypes.c_void_p
_c_sz = ctypes.c_size_t

SPARSEPR_F32 = 0
SPARSEPR_BF16 = 1
STATUS = {0: "SPARSEPR_OK", 1: "SPARSEPR_ERR_INVALID_ARG", 2: "SPARSEPR_ERR_UNSUPPORTED",
          3: "SPARSEPR_ERR_WORKSPACE", 4: "SPARSEPR_ERR_HIP"}

# every entry point declared in include/sparsepr.h
EXPORTS = ("sparsepr_abi_version", "sparsepr_status_string", "sparsepr_last_error",
           "sparsepr_workspace_bytes", "sparsepr_partition", "sparsepr_route", "sparsepr_attend",
           "sparsepr_attend_subset", "sparsepr_probe_fit", "sparsepr_apply",
           "sparsepr_apply_noalloc", "sparsepr_dense_attention", "sparsepr_support_stats")
BLOCKS_ALL, BLOCKS_WITH_PROBE, BLOCKS_WITHOUT_PROBE = 0, 1, 2
QUEUE_BYTES = 1024        # SPARSEPR_QUEUE_BYTES: the attention's optional work-queue buffer
RESPONSE_COUPLED, RANDOM_BLOCK, SEMANTIC = 0, 1, 2   # partition modes


class CParams(ctypes.Structure):
    _fields_ = [("heads", _c_i32), ("n_tokens", _c_i32), ("head_dim", _c_i32), ("dtype", _c_i32),
                ("q_block", _c_i32), ("n_groups", _c_i32), ("n_samples", _c_i32),
                ("kmeans_iters", _c_i32), ("density", ctypes.c_double), ("n_probes", _c_i32),
                ("rank", _c_i32), ("ridge_lambda", ctypes.c_double), ("partition_mode", _c_i32),
                ("reserved", _c_i32), ("probe_pos", ctypes.c_void_p)]


class SparsePRError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_LIB = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or _build.lib_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} not found: build the HIP library with `python -m free_block_sparse_rcp_amd.build`")
    lib = ctypes.CDLL(path)
    lib.sparsepr_abi_version.restype = _c_i32
    lib.sparsepr_status_string.restype = ctypes.c_char_p
    lib.sparsepr_status_string.argtypes = [_c_i32]
    lib.sparsepr_last_error.restype = ctypes.c_char_p
    lib.sparsepr_workspace_bytes.argtypes = [ctypes.POINTER(CParams), ctypes.POINTER(_c_sz)]
    lib.sparsepr_workspace_bytes.restype = _c_i32
    pp = ctypes.POINTER(CParams)
    lib.sparsepr_partition.argtypes = [pp] + [_c_p] * 14 + [_c_p, _c_sz, _c_p]
    lib.sparsepr_route.argtypes = [pp] + [_c_p] * 13 + [_c_p, _c_sz, _c_p]
    lib.sparsepr_attend.argtypes = [pp] + [_c_p] * 11 + [_c_p, _c_sz, _c_p]
    lib.sparsepr_attend_subset.argtypes = [pp] + [_c_p] * 11 + [_c_i32, _c_p, _c_sz, _c_p]
    lib.sparsepr_probe_fit.argtypes = [pp] + [_c_p] * 10 + [_c_p, _c_sz, _c_p]
    lib.sparsepr_apply.argtypes = [pp] + [_c_p] * 7 + [_c_p, _c_sz, _c_p]
    lib.sparsepr_apply_noalloc.argtypes = [pp] + [_c_p] * 7 + [_c_p]
    lib.sparsepr_dense_attention.argtypes = [pp] + [_c_p] * 6 + [_c_p, _c_sz, _c_p]
    lib.sparsepr_support_stats.argtypes = ([pp, _c_i32] + [_c_p] * 8 + [_c_i32, ctypes.c_double] +
                                           [_c_p] * 7 + [_c_sz, _c_p])
    for name in ("sparsepr_partition", "sparsepr_route", "sparsepr_attend", "sparsepr_attend_subset",
                 "sparsepr_probe_fit", "sparsepr_apply", "sparsepr_apply_noalloc",
                 "sparsepr_dense_attention"):
        getattr(lib, name).restype = _c_i32
    if lib.sparsepr_abi_version() != 4:
        raise RuntimeError("libsparsepr ABI version mismatch")
    _LIB = lib
    return lib


def loaded_path() -> Optional[str]:
    return _build.lib_path() if _LIB is not None else None


def _check(status: int) -> None:
    if status != 0:
        msg = load().sparsepr_last_error().decode()
        raise SparsePRError(status, msg)


def c_params(p: Params, probe_pos: Optional[torch.Tensor] = None) -> CParams:
    """The C params struct; probe_pos is the call's device array of probe
    positions (from probe_positions_tensor) or None for the default rule."""
    return CParams(p.heads, p.n_tokens, p.head_dim, SPARSEPR_BF16 if p.dtype == "bf16" else SPARSEPR_F32,
                   p.q_block, p.n_groups, p.n_samples, p.kmeans_iters, float(p.density), p.n_probes,
                   p.rank, float(p.ridge_lambda), p.partition_mode, 0,
                   None if probe_pos is None else probe_pos.data_ptr())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def torch_dtype(p: Params):
    return torch.bfloat16 if p.dtype == "bf16" else torch.float32


def workspace_bytes(p: Params) -> int:
    n = _c_sz(0)
    _check(load().sparsepr_workspace_bytes(ctypes.byref(c_params(p)), ctypes.byref(n)))
    return int(n.value)


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def index_tensor(a, n: int, length: int, name: str, device, distinct: bool = False) -> torch.Tensor:
    """Validate an index array on the host and upload it as int32."""
    arr = np.asarray(a.cpu().numpy() if isinstance(a, torch.Tensor) else a).astype(np.int64).ravel()
    if arr.size != length:
        raise ValueError(f"{name} must have {length} entries (got {arr.size})")
    if arr.size and (arr.min() < 0 or arr.max() >= n):
        raise ValueError(f"{name} entries must lie in [0, {n})")
    if distinct and np.unique(arr).size != arr.size:
        raise ValueError(f"{name} entries must be distinct")
    return torch.from_numpy(arr.astype(np.int32)).to(device)


def probe_positions_tensor(positions, p: Params, device) -> torch.Tensor:
    """Check caller-chosen probe positions on the host (m entries, strictly
    increasing, in [0, N)) and upload them for Buffers.probe_pos."""
    arr = np.asarray(positions.cpu().numpy() if isinstance(positions, torch.Tensor) else positions)
    arr = arr.astype(np.int64).ravel()
    if arr.size and np.any(np.diff(arr) <= 0):
        raise ValueError("probe positions must be strictly increasing")
    return index_tensor(arr, p.n_tokens, p.n_probes, "probe positions", device)


@dataclass
class Buffers:
    """Every device buffer of one call; reused across calls of the same shape."""

    key_label: torch.Tensor
    key_perm: torch.Tensor
    group_off: torch.Tensor
    key_centroid: torch.Tensor
    Kp: torch.Tensor
    Vp: torch.Tensor
    query_perm: torch.Tensor
    block_ptr: torch.Tensor
    block_groups: torch.Tensor
    executed_pairs: torch.Tensor
    S: torch.Tensor
    S_probe: torch.Tensor
    lse: torch.Tensor
    O_probe: torch.Tensor
    U: torch.Tensor
    Theta: torch.Tensor
    rank_eff: torch.Tensor
    O: torch.Tensor
    workspace: torch.Tensor
    queue: torch.Tensor          # the attention's work-queue counters
    # semantic mode only: the query partition (its key_perm is the query order)
    query_label: Optional[torch.Tensor] = None
    query_order: Optional[torch.Tensor] = None
    query_group_off: Optional[torch.Tensor] = None
    query_centroid: Optional[torch.Tensor] = None
    # caller-chosen probe positions [m] (int32), or None for floor((i + 1/2) N / m)
    probe_pos: Optional[torch.Tensor] = None


def alloc_buffers(p: Params, device) -> Buffers:
    H, N, D, G = p.heads, p.n_tokens, p.head_dim, p.n_groups
    nb = p.n_blocks
    dt = torch_dtype(p)
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    semantic = {}
    if p.partition_mode == SEMANTIC:
        semantic = dict(query_label=torch.empty(H, N, **i32), query_order=torch.empty(H, N, **i32),
                        query_group_off=torch.empty(H, G + 1, **i32),
                        query_centroid=torch.empty(H, G, D, **f32))
    return Buffers(
        key_label=torch.empty(H, N, **i32), key_perm=torch.empty(H, N, **i32),
        group_off=torch.empty(H, G + 1, **i32), key_centroid=torch.empty(H, G, D, **f32),
        Kp=torch.empty(H, N, D, dtype=dt, device=device),
        Vp=torch.empty(H, N, D, dtype=dt, device=device),
        query_perm=torch.empty(H, N, **i32), block_ptr=torch.empty(H, nb + 1, **i32),
        block_groups=torch.empty(H, nb * G, **i32),
        executed_pairs=torch.empty(H, dtype=torch.int64, device=device),
        S=torch.empty(H, N, D, dtype=dt, device=device),
        S_probe=torch.empty(H, max(p.n_probes, 1), D, **f32), lse=torch.empty(H, N, **f32),
        O_probe=torch.empty(H, max(p.n_probes, 1), D, **f32),
        U=torch.empty(H, D, max(p.rank, 1), **f32),
        Theta=torch.empty(H, D + 1, max(p.rank, 1), **f32),
        rank_eff=torch.empty(H, **i32), O=torch.empty(H, N, D, dtype=dt, device=device),
        workspace=torch.empty(workspace_bytes(p), dtype=torch.uint8, device=device),
        queue=torch.empty(QUEUE_BYTES, dtype=torch.uint8, device=device), **semantic)


# ------------------------------------------------------------ stage calls

def partition(p: Params, Q, K, V, scale, sample_idx, init_idx, b: Buffers, rand_key_perm=None,
              dbg_assign_scores: Optional[torch.Tensor] = None) -> None:
    lib = load()
    cp = c_params(p)
    _check(lib.sparsepr_partition(
        ctypes.byref(cp), _ptr(Q), _ptr(K), _ptr(V), _ptr(scale), _ptr(sample_idx), _ptr(init_idx),
        _ptr(rand_key_perm), _ptr(b.key_label), _ptr(b.key_perm), _ptr(b.group_off),
        _ptr(b.key_centroid), _ptr(b.Kp), _ptr(b.Vp), _ptr(dbg_assign_scores),
        _ptr(b.workspace), b.workspace.numel(), _stream(K.device)))


def partition_queries(p: Params, Q, init_idx, b: Buffers,
                      dbg_assign_scores: Optional[torch.Tensor] = None) -> None:
    """Semantic mode: the partition stage run on the queries (no gather); its
    group-contiguous order b.query_order is the query order for route."""
    lib = load()
    cp = c_params(p)
    _check(lib.sparsepr_partition(
        ctypes.byref(cp), None, _ptr(Q), None, None, None, _ptr(init_idx), None,
        _ptr(b.query_label), _ptr(b.query_order), _ptr(b.query_group_off),
        _ptr(b.query_centroid), None, None, _ptr(dbg_assign_scores),
        _ptr(b.workspace), b.workspace.numel(), _stream(Q.device)))


def route(p: Params, Q, scale, b: Buffers, rand_query_perm=None, dbg_coords=None,
          dbg_dominant=None, dbg_dominant_val=None, dbg_block_score=None) -> None:
    lib = load()
    cp = c_params(p)
    _check(lib.sparsepr_route(
        ctypes.byref(cp), _ptr(Q), _ptr(scale), _ptr(b.key_centroid), _ptr(b.group_off),
        _ptr(rand_query_perm), _ptr(b.query_perm), _ptr(b.block_ptr), _ptr(b.block_groups),
        _ptr(b.executed_pairs), _ptr(dbg_coords), _ptr(dbg_dominant), _ptr(dbg_dominant_val),
        _ptr(dbg_block_score), _ptr(b.workspace), b.workspace.numel(), _stream(Q.device)))


def _queue_args(queue):
    return (None, 0) if queue is None else (_ptr(queue), queue.numel() * queue.element_size())


def attend(p: Params, Q, scale, b: Buffers, subset: int = BLOCKS_ALL,
           use_queue: bool = True) -> None:
    """Stage 3; use_queue=False deals the blocks out statically (same results)."""
    lib = load()
    cp = c_params(p, b.probe_pos)
    args = (ctypes.byref(cp), _ptr(Q), _ptr(b.Kp), _ptr(b.Vp), _ptr(scale), _ptr(b.group_off),
            _ptr(b.query_perm), _ptr(b.block_ptr), _ptr(b.block_groups), _ptr(b.S),
            _ptr(b.S_probe), _ptr(b.lse))
    q = _queue_args(b.queue if use_queue else None)
    if subset == BLOCKS_ALL:
        _check(lib.sparsepr_attend(*args, *q, _stream(Q.device)))
    else:
        _check(lib.sparsepr_attend_subset(*args, subset, *q, _stream(Q.device)))


def probe_fit(p: Params, Q, scale, b: Buffers, K=None, V=None) -> None:
    lib = load()
    cp = c_params(p, b.probe_pos)
    K = b.Kp if K is None else K
    V = b.Vp if V is None else V
    _check(lib.sparsepr_probe_fit(
        ctypes.byref(cp), _ptr(Q), _ptr(K), _ptr(V), _ptr(scale), _ptr(b.query_perm),
        _ptr(b.S_probe), _ptr(b.O_probe), _ptr(b.U), _ptr(b.Theta), _ptr(b.rank_eff), _ptr(b.workspace),
        b.workspace.numel(), _stream(Q.device)))


def apply(p: Params, b: Buffers) -> None:
    lib = load()
    cp = c_params(p, b.probe_pos)
    _check(lib.sparsepr_apply(
        ctypes.byref(cp), _ptr(b.S), _ptr(b.query_perm), _ptr(b.O_probe), _ptr(b.U),
        _ptr(b.Theta), _ptr(b.rank_eff), _ptr(b.O), _ptr(b.workspace), b.workspace.numel(),
        _stream(b.S.device)))


def apply_noalloc(p: Params, b: Buffers, O=None) -> torch.Tensor:
    """Stage 5 through the entry point that uses the library's fixed scratch
    instead of the workspace; writes O (default: b.O)."""
    lib = load()
    cp = c_params(p, b.probe_pos)
    O = b.O if O is None else O
    _check(lib.sparsepr_apply_noalloc(
        ctypes.byref(cp), _ptr(b.S), _ptr(b.query_perm), _ptr(b.O_probe), _ptr(b.U),
        _ptr(b.Theta), _ptr(b.rank_eff), _ptr(O), _stream(b.S.device)))
    return O


def dense_attention(p: Params, Q, K, V, scale, O=None, lse=None, queue=None,
                    use_queue: bool = True):
    """Exact attention. With use_queue, the work queue is ``queue`` or else a
    buffer from torch's allocator on the current stream; use_queue=False deals
    the blocks out statically (same results)."""
    lib = load()
    cp = c_params(p)
    if O is None:
        O = torch.empty_like(Q)
    if lse is None:
        lse = torch.empty(p.heads, p.n_tokens, dtype=torch.float32, device=Q.device)
    if not use_queue:
        queue = None
    elif queue is None:
        queue = torch.empty(QUEUE_BYTES, dtype=torch.uint8, device=Q.device)
    _check(lib.sparsepr_dense_attention(ctypes.byref(cp), _ptr(Q), _ptr(K), _ptr(V), _ptr(scale),
                                        _ptr(O), _ptr(lse), *_queue_args(queue),
                                        _stream(Q.device)))
    return O, lse


@dataclass
class SupportStats:
    """Per-row and per-block support and mass diagnostics (host arrays)."""

    lse: np.ndarray             # [n_blocks, B_q] full-row log-sum-exp
    routed_mass: np.ndarray     # [n_blocks, B_q] softmax mass on the block's routed keys
    support: np.ndarray         # [n_blocks, B_q] keys holding the target mass
    support_routed: np.ndarray  # [n_blocks, B_q] of those, keys routed to the block
    pooled: np.ndarray          # [n_blocks] union of the rows' supports
    pooled_routed: np.ndarray   # [n_blocks] its part on routed keys
    valid: np.ndarray           # [n_blocks, B_q] row lies inside N


def support_stats(p: Params, head: int, Q, K, scale, b: Buffers, blocks, mass: float = 0.9,
                  workspace: Optional[torch.Tensor] = None) -> SupportStats:
    """Diagnostics of sampled blocks of one head (K in token order), after route."""
    lib = load()
    cp = c_params(p)
    dev = Q.device
    blk = index_tensor(blocks, p.n_blocks, len(blocks), "blocks", dev)
    nbk, BQ = len(blocks), p.q_block
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    lse, rm = torch.empty(nbk * BQ, **f32), torch.empty(nbk * BQ, **f32)
    sup, supr = torch.empty(nbk * BQ, **i32), torch.empty(nbk * BQ, **i32)
    pool, poolr = torch.empty(nbk, **i32), torch.empty(nbk, **i32)
    need = 4 * nbk * BQ * (p.n_tokens + 1)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib.sparsepr_support_stats(
        ctypes.byref(cp), int(head), _ptr(Q), _ptr(K), _ptr(scale), _ptr(b.key_label),
        _ptr(b.query_perm), _ptr(b.block_ptr), _ptr(b.block_groups), _ptr(blk), nbk, float(mass),
        _ptr(lse), _ptr(rm), _ptr(sup), _ptr(supr), _ptr(pool), _ptr(poolr), _ptr(workspace),
        workspace.numel(), _stream(dev)))
    torch.cuda.synchronize(dev)
    pos = np.asarray(blocks, np.int64)[:, None] * BQ + np.arange(BQ)[None, :]
    return SupportStats(lse=lse.view(nbk, BQ).cpu().numpy(), routed_mass=rm.view(nbk, BQ).cpu().numpy(),
                        support=sup.view(nbk, BQ).cpu().numpy(),
                        support_routed=supr.view(nbk, BQ).cpu().numpy(),
                        pooled=pool.cpu().numpy(), pooled_routed=poolr.cpu().numpy(),
                        valid=pos < p.n_tokens)


class SparsePR:
    """One SparsePR operator of a fixed shape with preallocated buffers.

    ``run`` enqueues the five stages on the current stream; the result is
    ``buffers.O`` (token order) once the stream has been synchronised.
    """

    def __init__(self, p: Params, device="cuda", use_queue: bool = True):
        load()
        self.p = p
        self.device = torch.device(device)
        self.buffers = alloc_buffers(p, self.device)
        self.use_queue = use_queue      # the attention's work queue (False: static blocks)
        self._side = None

    def upload_indices(self, sample_idx=None, init_idx=None, rand_key_perm=None,
                       rand_query_perm=None) -> Dict[str, torch.Tensor]:
        p, dev = self.p, self.device
        out = {}
        if p.partition_mode == 0:
            out["sample_idx"] = index_tensor(sample_idx, p.n_tokens, p.n_samples, "sample_idx", dev, True)
            out["init_idx"] = index_tensor(init_idx, p.n_tokens, p.n_groups, "init_idx", dev, True)
        elif p.partition_mode == SEMANTIC:
            out["init_idx"] = index_tensor(init_idx, p.n_tokens, p.n_groups, "init_idx", dev, True)
        else:
            out["rand_key_perm"] = index_tensor(rand_key_perm, p.n_tokens, p.n_tokens, "rand_key_perm", dev, True)
            out["rand_query_perm"] = index_tensor(rand_query_perm, p.n_tokens, p.n_tokens, "rand_query_perm", dev, True)
        return out

    def check_inputs(self, Q, K, V, scale):
        p = self.p
        shp = (p.heads, p.n_tokens, p.head_dim)
        for name, t in (("Q", Q), ("K", K), ("V", V)):
            _check_tensor(name, t, shp, torch_dtype(p), self.device)
        _check_tensor("scale", scale, (p.heads,), torch.float32, self.device)

    def side_stream(self) -> torch.cuda.Stream:
        """Second stream (default priority) for the probe fit."""
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
        return self._side

    def run(self, Q, K, V, scale, idx: Dict[str, torch.Tensor], overlap: bool = False,
            events: Optional[Dict[str, torch.cuda.Event]] = None) -> torch.Tensor:
        """One call on the current stream. With ``overlap``, the blocks that hold
        probe rows are attended first, then the probe fit runs on a side stream
        while the remaining blocks are attended; apply waits for both. ``events``
        (optional) receives HIP events recorded between the stages."""
        p, b = self.p, self.buffers
        main = torch.cuda.current_stream(self.device)

        def mark(name, stream=None):
            if events is not None:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(stream or main)
                events[name] = ev

        mark("start")
        partition(p, Q, K, V, scale, idx.get("sample_idx"), idx.get("init_idx"), b,
                  rand_key_perm=idx.get("rand_key_perm"))
        qorder = idx.get("rand_query_perm")
        if p.partition_mode == SEMANTIC:
            partition_queries(p, Q, idx["init_idx"], b)
            qorder = b.query_order
        mark("partition")
        route(p, Q, scale, b, rand_query_perm=qorder)
        mark("route")
        uq = self.use_queue
        if not overlap:
            attend(p, Q, scale, b, use_queue=uq)
            mark("attend")
            probe_fit(p, Q, scale, b)
            mark("probe_fit")
            apply(p, b)
            mark("apply")
            return b.O
        attend(p, Q, scale, b, subset=BLOCKS_WITH_PROBE, use_queue=uq)
        mark("attend_probe_blocks")
        fork = torch.cuda.Event()
        fork.record(main)
        side = self.side_stream()
        side.wait_event(fork)
        with torch.cuda.stream(side):
            mark("probe_fit_start", side)
            probe_fit(p, Q, scale, b)
            mark("probe_fit", side)
        join = torch.cuda.Event()
        join.record(side)
        attend(p, Q, scale, b, subset=BLOCKS_WITHOUT_PROBE, use_queue=uq)
        mark("attend")
        main.wait_event(join)
        mark("join")
        apply(p, b)
        mark("apply")
        return b.O
