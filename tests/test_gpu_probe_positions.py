"""GPU parity with caller-chosen probe positions (sparsepr_params.probe_pos),
through the C-ABI, against the fp64 oracle run on the GPU's own groups, order
and routes with the same positions: sparse output, exact probe rows, the
fit's copy of the probe rows' sparse outputs and the final output, within
relative L2 1e-4 (fp32) or 2e-2 (bf16); the pair count does not depend on
the positions. The split of stage 3 into blocks with and without probes
follows the given positions."""
import numpy as np
import pytest
import torch

from oracle import sparsepr_oracle as orc
from free_block_sparse_rcp_amd import binding, configs

from _gpu_util import bf16_round, rel_l2, run_pipeline, small_bf16
from test_gpu_parity import head_arrays, oracle_on_gpu_indices, to_token_order

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def positions(p, kind):
    N, m = p.n_tokens, p.n_probes
    if kind == "random":
        return np.sort(np.random.default_rng(77).choice(N, m, replace=False))
    if kind == "front":                 # every probe in the first blocks
        return np.arange(m)
    return np.arange(N - m, N)          # the last positions, ragged last block included


CASES = [("tiny", configs.TINY, k) for k in ("random", "front", "tail")] + \
        [("bf16_d128", small_bf16(), k) for k in ("random", "tail")]


@pytest.mark.parametrize("name,wl,kind", CASES, ids=[f"{c[0]}-{c[2]}" for c in CASES])
def test_given_probe_positions_match_oracle(name, wl, kind):
    p = wl.params
    pos = positions(p, kind)
    print(f"[gpu] {name} probe positions {kind}", flush=True)
    r = run_pipeline(wl, probe_pos=pos)
    tol = TOL[p.dtype]
    for h in range(p.heads):
        g = head_arrays(r, h)
        Q, K, V = (x[h].astype(np.float64) for x in (r.inp.Q, r.inp.K, r.inp.V))
        o = oracle_on_gpu_indices(Q, K, V, float(r.inp.scale[h]), p, g, probe_pos=pos)
        assert np.array_equal(o["ptok"], g["query_perm"][pos])
        assert rel_l2(to_token_order(g["S"], g["query_perm"]), o["S"]) < tol, "sparse attention"
        assert int(g["executed_pairs"]) == o["E"]
        assert rel_l2(g["O_probe"], o["Op"]) < tol, "probe rows"
        Sp = g["S_probe"] if p.dtype == "f32" else bf16_round(g["S_probe"])
        assert np.array_equal(Sp, g["S"][pos])
        assert rel_l2(g["O"], o["O"]) < tol, "final output"
        # probe tokens carry their exact rows
        assert rel_l2(g["O"][o["ptok"]], o["Op"]) < tol


def test_attend_subsets_follow_given_positions():
    wl = configs.TINY
    p = wl.params
    pos = positions(p, "front")
    r = run_pipeline(wl, probe_pos=pos, dbg=False)
    b = r.b
    full = b.S.clone()
    with_probe = np.unique(pos // p.q_block)
    for subset in (binding.BLOCKS_WITH_PROBE, binding.BLOCKS_WITHOUT_PROBE):
        b.S.fill_(float("nan"))
        binding.attend(p, r.Q, r.scale, b, subset=subset)
        torch.cuda.synchronize()
        S = b.S.cpu().numpy()
        for blk in range(p.n_blocks):
            rows = slice(blk * p.q_block, min(p.n_tokens, (blk + 1) * p.q_block))
            ran = (blk in with_probe) == (subset == binding.BLOCKS_WITH_PROBE)
            if ran:
                assert np.array_equal(S[:, rows], full.cpu().numpy()[:, rows])
            else:
                assert np.isnan(S[:, rows]).all()
