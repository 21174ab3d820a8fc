"""Host-only checks of the C-ABI library: it loads, exports every function
that include/sparsepr.h declares, and its validation returns the documented
status codes before anything is launched (no GPU is needed or touched)."""
import ctypes
import os
import re

import numpy as np
import torch

import pytest

from free_block_sparse_rcp_amd import binding, build, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsepr.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsepr_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.lib_path()):
        pytest.skip("libsparsepr.so not built (run python -m free_block_sparse_rcp_amd.build)")
    return binding.load()


def test_header_declares_the_five_stages_and_helpers():
    names = declared_functions()
    for n in ("sparsepr_partition", "sparsepr_route", "sparsepr_attend", "sparsepr_probe_fit",
              "sparsepr_apply", "sparsepr_dense_attention", "sparsepr_workspace_bytes"):
        assert n in names
    assert sorted(binding.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert lib.sparsepr_abi_version() == 4


def test_status_strings(lib):
    for code, name in binding.STATUS.items():
        assert lib.sparsepr_status_string(code).decode() == name
    assert lib.sparsepr_status_string(99).decode() == "SPARSEPR_UNKNOWN_STATUS"


def test_queue_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define SPARSEPR_QUEUE_BYTES (\d+)", src)
    assert m and int(m.group(1)) == binding.QUEUE_BYTES


def test_params_struct_layout_matches_header():
    assert ctypes.sizeof(binding.CParams) == 72
    assert binding.CParams.density.offset == 32
    assert binding.CParams.ridge_lambda.offset == 48
    assert binding.CParams.probe_pos.offset == 64


def _ws(lib, p):
    n = ctypes.c_size_t(0)
    st = lib.sparsepr_workspace_bytes(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("name", ["tiny", "wan", "hunyuan", "cosmos", "sweep"])
def test_workspace_bytes_for_every_workload(lib, name):
    p = binding.c_params(configs.get(name).params)
    st, n = _ws(lib, p)
    assert st == 0 and n > 0
    assert n < 64 * 2**30


BAD = [
    ("heads", 0, 1), ("heads", 65536, 2), ("n_tokens", 0, 1), ("head_dim", 96, 2), ("dtype", 7, 1),
    ("q_block", 32, 2),
    ("n_groups", 0, 1), ("n_groups", 2000, 1), ("n_samples", 0, 1), ("kmeans_iters", 0, 1),
    ("density", 0.0, 1), ("density", 1.5, 1), ("n_probes", -1, 1), ("rank", 200, 1),
    ("ridge_lambda", 0.0, 1), ("partition_mode", 3, 1), ("reserved", 1, 1),
]


@pytest.mark.parametrize("field,value,code", BAD)
def test_invalid_params_are_rejected_on_host(lib, field, value, code):
    p = binding.c_params(configs.TINY.params)
    setattr(p, field, value)
    st, _ = _ws(lib, p)
    assert st == code
    assert lib.sparsepr_last_error().decode() != ""


def test_budget_below_one_key_is_rejected(lib):
    p = binding.c_params(configs.TINY.params)
    p.density = 0.03          # 0.03 * 2048 - 64 < 1
    st, _ = _ws(lib, p)
    assert st == 1 and "key budget" in lib.sparsepr_last_error().decode()


def test_null_pointers_and_small_workspace_are_rejected(lib):
    p = binding.c_params(configs.TINY.params)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    # partition with K missing
    st = lib.sparsepr_partition(ctypes.byref(p), fake, None, fake, fake, fake, fake, None, fake,
                                fake, fake, fake, fake, fake, None, fake, 1 << 40, None)
    assert st == 1 and "K is NULL" in lib.sparsepr_last_error().decode()
    # workspace too small
    st = lib.sparsepr_partition(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake,
                                fake, fake, fake, fake, fake, None, fake, 16, None)
    assert st == 3
    # route without the random-block permutation in random-block mode
    p.partition_mode = 1
    st = lib.sparsepr_route(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, fake,
                            None, None, None, None, fake, 1 << 40, None)
    assert st == 1 and "rand_query_perm" in lib.sparsepr_last_error().decode()
    # semantic comparator mode: init_idx is required, Kp/Vp come as a pair,
    # and route needs the per-head query order
    p.partition_mode = 2
    st = lib.sparsepr_partition(ctypes.byref(p), None, fake, fake, None, None, None, None, fake,
                                fake, fake, fake, fake, fake, None, fake, 1 << 40, None)
    assert st == 1 and "init_idx" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_partition(ctypes.byref(p), None, fake, fake, None, None, fake, None, fake,
                                fake, fake, fake, fake, None, None, fake, 1 << 40, None)
    assert st == 1 and "Kp and Vp" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_route(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, fake,
                            None, None, None, None, fake, 1 << 40, None)
    assert st == 1 and "rand_query_perm" in lib.sparsepr_last_error().decode()
    # support diagnostics: head, block count, mass and workspace are validated
    p.partition_mode = 0
    args = [fake] * 8
    outs = [fake] * 6
    st = lib.sparsepr_support_stats(ctypes.byref(p), 1, *args, 1, 0.9, *outs, fake, 1 << 40, None)
    assert st == 1 and "head" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_support_stats(ctypes.byref(p), 0, *args, 0, 0.9, *outs, fake, 1 << 40, None)
    assert st == 1 and "n_blocks" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_support_stats(ctypes.byref(p), 0, *args, 1, 1.5, *outs, fake, 1 << 40, None)
    assert st == 1 and "mass" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_support_stats(ctypes.byref(p), 0, *args, 1, 0.9, *outs[:5], None, fake,
                                    1 << 40, None)
    assert st == 1 and "pooled_routed" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_support_stats(ctypes.byref(p), 0, *args, 2, 0.9, *outs, fake,
                                    4 * 2 * 64 * 2049 - 1, None)
    assert st == 3
    # attend with no lse, then with probes but no fp32 copy of their rows
    p.partition_mode = 0
    st = lib.sparsepr_attend(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                             fake, None, None, 0, None)
    assert st == 1 and "lse" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_attend(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                             None, fake, None, 0, None)
    assert st == 1 and "S_probe" in lib.sparsepr_last_error().decode()
    # the optional work queue: aligned, and at least SPARSEPR_QUEUE_BYTES
    st = lib.sparsepr_attend(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                             fake, fake, fake, binding.QUEUE_BYTES - 1, None)
    assert st == 3 and "queue" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_attend(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                             fake, fake, ctypes.c_void_p(0x1002), binding.QUEUE_BYTES, None)
    assert st == 1 and "aligned" in lib.sparsepr_last_error().decode()
    # attention on a block subset: the subset value is validated
    st = lib.sparsepr_attend_subset(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                                    fake, fake, fake, 3, None, 0, None)
    assert st == 1 and "subset" in lib.sparsepr_last_error().decode()
    # apply: output missing, then a workspace too small for the per-head matrix
    st = lib.sparsepr_apply(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake,
                            1 << 40, None)
    assert st == 1 and "O is NULL" in lib.sparsepr_last_error().decode()
    st = lib.sparsepr_apply(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, 16,
                            None)
    assert st == 3
    # apply without a workspace: NULL output, then more heads than the fixed
    # scratch holds (bf16, d = 128: 66048 bytes per head, 8 MiB in all)
    st = lib.sparsepr_apply_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None,
                                    None)
    assert st == 1 and "O is NULL" in lib.sparsepr_last_error().decode()
    big = binding.c_params(configs.HUNYUAN.params)
    big.heads = 128
    st = lib.sparsepr_apply_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, fake,
                                    None)
    assert st == 3 and "fixed scratch" in lib.sparsepr_last_error().decode()
    # dense attention validates only the shape fields
    q = binding.c_params(configs.TINY.params)
    q.head_dim = 80
    st = lib.sparsepr_dense_attention(ctypes.byref(q), fake, fake, fake, fake, fake, None, None, 0,
                                      None)
    assert st == 2
    q.head_dim = 128
    st = lib.sparsepr_dense_attention(ctypes.byref(q), fake, fake, fake, fake, fake, None, fake, 16,
                                      None)
    assert st == 3 and "queue" in lib.sparsepr_last_error().decode()


def test_index_validation_in_binding():
    import numpy as np
    with pytest.raises(ValueError):
        binding.index_tensor(np.array([0, 5]), 5, 2, "x", "cpu")
    with pytest.raises(ValueError):
        binding.index_tensor(np.array([1, 1]), 5, 2, "x", "cpu", distinct=True)
    t = binding.index_tensor(np.array([4, 0]), 5, 2, "x", "cpu", distinct=True)
    assert t.dtype.is_floating_point is False and t.tolist() == [4, 0]


def test_probe_positions_checked_on_the_host():
    p = configs.TINY.params
    t = binding.probe_positions_tensor(np.arange(p.n_probes) * 3, p, "cpu")
    assert t.dtype == torch.int32 and t.tolist() == list(range(0, 3 * p.n_probes, 3))
    good = np.arange(p.n_probes) * 3
    for bad in (good[:-1], np.r_[good[:-1], good[-2]], np.r_[-1, good[1:]],
                np.r_[good[:-1], p.n_tokens], good[::-1]):
        with pytest.raises(ValueError):
            binding.probe_positions_tensor(bad, p, "cpu")
