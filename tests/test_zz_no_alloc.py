"""The allocation-free apply entry point (sparsepr_apply_noalloc) against
sparsepr_apply on the same inputs, through the C-ABI: bit-identical outputs on
two calls in a row, the second with a smaller input (fewer heads, fewer
tokens), on the bf16 path (which uses the fixed scratch) and the fp32 path."""
import math

import numpy as np
import pytest
import torch

from free_block_sparse_rcp_amd import binding, configs

from _gpu_util import run_pipeline, small_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _compare(run):
    """Apply through both entry points into fresh outputs and compare them."""
    p, b = run.p, run.b
    ref = torch.full_like(b.O, float("nan"))
    got = torch.full_like(b.O, float("nan"))
    binding.apply(p, b)
    torch.cuda.synchronize()
    ref.copy_(b.O)
    binding.apply_noalloc(p, b, O=got)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    assert torch.equal(got, ref)
    assert torch.equal(ref, b.O)
    return got


def test_noalloc_apply_matches_apply_twice_second_smaller():
    big = small_bf16(name="noalloc_big", heads=3, seed=31)
    small = small_bf16(name="noalloc_small", grid=(5, 11, 23), heads=1, G=48, m=64, k=16,
                       seed=32)
    assert small.params.heads * small.params.n_tokens < big.params.heads * big.params.n_tokens
    print("[gpu] noalloc: first call, 3 heads, N = 3045", flush=True)
    r1 = run_pipeline(big, dbg=False)
    o1 = _compare(r1)
    assert int(r1.b.rank_eff.min().item()) > 0        # a real correction was applied
    print("[gpu] noalloc: second call, 1 head, N = 1265", flush=True)
    r2 = run_pipeline(small, dbg=False)
    _compare(r2)
    # the first call's output is unchanged by the second
    assert torch.equal(r1.b.O, o1)


def test_noalloc_apply_fp32_path():
    print("[gpu] noalloc: fp32 tiny", flush=True)
    r = run_pipeline(configs.TINY, dbg=False)
    _compare(r)
