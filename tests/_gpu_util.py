"""Helpers of the GPU parity tests: run the HIP stages through the C-ABI with
every debug dump enabled and bring the results back as numpy arrays."""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

from free_block_sparse_rcp_amd import binding, configs
from free_block_sparse_rcp_amd.configs import Params, Workload


def small_bf16(name="small_bf16", grid=(7, 15, 29), heads=2, d=128, G=64, S=256, BQ=128,
               rho=0.22, m=128, k=32, seed=11, scales=None, smoothing=False, mode=0) -> Workload:
    """A G2 workload small enough for the oracle, spanning many tiles and a
    ragged last query block (N = 3045 = 23 * 128 + 101)."""
    n = grid[0] * grid[1] * grid[2]
    p = Params(heads=heads, n_tokens=n, head_dim=d, dtype="bf16", q_block=BQ, n_groups=G,
               n_samples=S, kmeans_iters=8, density=rho, n_probes=m, rank=k, ridge_lambda=1e-3,
               partition_mode=mode)
    sc = scales if scales is not None else [1.0 / math.sqrt(d)] * heads
    return Workload(name=name, grid=grid, params=p, scales=sc, generator="g2", seed=seed,
                    blur=(1.5, 3.0, 3.0), key_smoothing=smoothing)


@dataclass
class GpuRun:
    p: Params
    inp: object
    Q: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    scale: torch.Tensor
    idx: Dict[str, torch.Tensor]
    b: binding.Buffers
    dbg: Dict[str, torch.Tensor]

    def np(self, name):
        t = getattr(self.b, name) if hasattr(self.b, name) else self.dbg[name]
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.detach().cpu().numpy()


def to_device(inp, p: Params, device="cuda"):
    dt = binding.torch_dtype(p)
    Q = torch.from_numpy(inp.Q).to(device=device, dtype=dt).contiguous()
    K = torch.from_numpy(inp.K).to(device=device, dtype=dt).contiguous()
    V = torch.from_numpy(inp.V).to(device=device, dtype=dt).contiguous()
    scale = torch.from_numpy(inp.scale).to(device)
    return Q, K, V, scale


def run_pipeline(wl: Workload, heads=None, dbg: bool = True, dbg_heads_ok: bool = True,
                 inp=None, p: Optional[Params] = None, probe_pos=None) -> GpuRun:
    p = p or wl.params
    inp = inp if inp is not None else wl.make_inputs(heads)
    if heads is not None:
        p = replace(p, heads=len(heads))
    dev = torch.device("cuda")
    op = binding.SparsePR(p, dev)
    Q, K, V, scale = to_device(inp, p)
    idx = op.upload_indices(inp.sample_idx, inp.init_idx, inp.rand_key_perm, inp.rand_query_perm)
    b = op.buffers
    if probe_pos is not None:
        b.probe_pos = binding.probe_positions_tensor(probe_pos, p, dev)
    H, N, G, nb = p.heads, p.n_tokens, p.n_groups, p.n_blocks
    d: Dict[str, torch.Tensor] = {}
    if dbg:
        f32 = dict(dtype=torch.float32, device=dev)
        d["assign"] = torch.full((H, N, G), float("nan"), **f32)
        d["coords"] = torch.full((H, N, G), float("nan"), **f32)
        d["dom"] = torch.full((H, N), -1, dtype=torch.int32, device=dev)
        d["domval"] = torch.full((H, N), float("nan"), **f32)
        d["sigma"] = torch.full((H, nb, G), float("nan"), **f32)
    binding.partition(p, Q, K, V, scale, idx.get("sample_idx"), idx.get("init_idx"), b,
                      rand_key_perm=idx.get("rand_key_perm"),
                      dbg_assign_scores=d.get("assign") if p.partition_mode != 1 else None)
    qorder = idx.get("rand_query_perm")
    if p.partition_mode == binding.SEMANTIC:
        if dbg:
            d["qassign"] = torch.full((H, N, G), float("nan"), dtype=torch.float32, device=dev)
        binding.partition_queries(p, Q, idx["init_idx"], b, dbg_assign_scores=d.get("qassign"))
        qorder = b.query_order
    binding.route(p, Q, scale, b, rand_query_perm=qorder,
                  dbg_coords=d.get("coords"), dbg_dominant=d.get("dom"),
                  dbg_dominant_val=d.get("domval"), dbg_block_score=d.get("sigma"))
    binding.attend(p, Q, scale, b)
    binding.probe_fit(p, Q, scale, b)
    binding.apply(p, b)
    torch.cuda.synchronize()
    return GpuRun(p=p, inp=inp, Q=Q, K=K, V=V, scale=scale, idx=idx, b=b, dbg=d)


def map_in_subspace(U, Theta):
    """The map on [s; 1] (Theta [d+1, k]) written on the subspace coordinates
    [U^T s; 1]: rows U^T Theta[:d] and the bias row. Also returns how far the
    slopes stray from span(U) (0 for a map that reads only U^T s)."""
    U = np.asarray(U, np.float64)
    Th = np.asarray(Theta, np.float64)
    slopes = Th[:-1]
    inside = U.T @ slopes
    stray = float(np.abs(slopes - U @ inside).max()) if slopes.size else 0.0
    return np.vstack([inside, Th[-1:]]), stray


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def bf16_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def csr_lists(block_ptr, block_groups):
    return [block_groups[block_ptr[b]:block_ptr[b + 1]] for b in range(len(block_ptr) - 1)]
