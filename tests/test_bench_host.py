"""Host-side checks of bench.py's diagnostics (CPU tensors, no GPU)."""
import os
import sys
from types import SimpleNamespace

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _call(H=2, N=40, D=6, k=2, seed=0):
    """A fake call: sparse output S in query order, a query permutation, and a
    fitted map (U orthonormal [D, k], Theta [D+1, k])."""
    g = torch.Generator().manual_seed(seed)
    S = torch.randn(H, N, D, generator=g)
    qp = torch.stack([torch.randperm(N, generator=g) for _ in range(H)]).int()
    U = torch.linalg.qr(torch.randn(H, D, D, generator=g))[0][:, :, :k].contiguous()
    Theta = torch.randn(H, D + 1, k, generator=g)
    b = SimpleNamespace(S=S, query_perm=qp, U=U, Theta=Theta,
                        rank_eff=torch.full((H,), k, dtype=torch.int32))
    p = SimpleNamespace(heads=H, n_tokens=N, head_dim=D, n_probes=4)
    S_tok = torch.empty_like(S)
    S_tok.scatter_(1, qp.long()[:, :, None].expand(-1, -1, D), S)
    xa = torch.cat([S_tok, torch.ones(H, N, 1)], dim=2)
    R_fit = (xa @ Theta) @ U.transpose(1, 2)
    return p, b, S_tok, R_fit


def test_residual_r2_is_one_for_an_exactly_affine_residual():
    p, b, S_tok, R_fit = _call()
    mask = bench.unprobed_mask(p, b)
    assert int((~mask).sum()) == p.heads * p.n_probes
    assert abs(bench.residual_r2(p, b, S_tok + R_fit, mask) - 1.0) < 1e-12


def test_residual_r2_closed_form_without_a_fit():
    """rank 0: R_hat = 0, so R^2 = 1 - sum |R|^2 / sum |R - mean R|^2 (per head)."""
    p, b, S_tok, R_fit = _call(seed=3)
    b.rank_eff[:] = 0
    mask = bench.unprobed_mask(p, b)
    R = (R_fit + 0.5)                      # a residual with a nonzero mean
    num = den = 0.0
    for h in range(p.heads):
        r = R[h][mask[h]].double().numpy()
        num += (r ** 2).sum()
        den += ((r - r.mean(axis=0)) ** 2).sum()
    got = bench.residual_r2(p, b, S_tok + R, mask)
    # the reference output S + R is rounded to fp32 (relative 6e-8 per element)
    assert abs(got - (1 - num / den)) < 1e-6
    assert got < 0


def test_unprobed_mask_removes_the_probe_tokens():
    p, b, _, _ = _call(N=37)
    mask = bench.unprobed_mask(p, b)
    pos = [((2 * i + 1) * p.n_tokens) // (2 * p.n_probes) for i in range(p.n_probes)]
    for h in range(p.heads):
        probe_tokens = set(b.query_perm[h, pos].tolist())
        assert set(np.nonzero(~mask[h].numpy())[0].tolist()) == probe_tokens


def test_error_summary_over_all_unprobed_rows():
    """Mean and 99th percentile of ||o - ref|| / ||ref|| over every unprobed
    row, for the output and for the sparse output in token order."""
    p, b, S_tok, R_fit = _call(H=3, N=50, seed=5)
    g = torch.Generator().manual_seed(9)
    ref = torch.randn(3, 50, 6, generator=g)
    b.O = S_tok + R_fit
    mask = bench.unprobed_mask(p, b)
    rn = ref.norm(dim=2)
    got = bench.error_summary(p, b, ref, rn, mask)
    e, e0 = [], []
    for h in range(3):
        for t in range(50):
            if mask[h, t]:
                r = ref[h, t].double().numpy()
                e.append(np.linalg.norm(b.O[h, t].double().numpy() - r) / np.linalg.norm(r))
                e0.append(np.linalg.norm(S_tok[h, t].double().numpy() - r) / np.linalg.norm(r))
    assert got["rows"] == len(e) == 3 * (50 - p.n_probes)
    assert abs(got["rel_l2_mean_unprobed"] - np.mean(e)) < 1e-6
    assert abs(got["rel_l2_p99_unprobed"] - np.percentile(e, 99)) < 1e-6
    assert abs(got["hard_drop_rel_l2_mean"] - np.mean(e0)) < 1e-6
    assert abs(got["hard_drop_rel_l2_p99"] - np.percentile(e0, 99)) < 1e-6
