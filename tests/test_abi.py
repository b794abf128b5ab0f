"""The C ABI library: it loads, exports every function include/mla_decode.h
declares, and rejects bad configurations before touching a GPU."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _lib():
    from mla_latent_kv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from mla_latent_kv_amd import build
        build.build()
    return binding.load_library()


def test_every_declared_symbol_is_exported():
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|void|const char\*)\s+(mla_\w+)\s*\(", src, re.M))
    assert declared == {"mla_decode_init", "mla_decode_workspace_size", "mla_decode_run",
                        "mla_decode_run_profiled", "mla_decode_destroy",
                        "mla_decode_status_string", "mla_cache_append",
                        "mla_cache_append_workspace_size", "mla_output_project",
                        "mla_output_project_workspace_size", "mla_query_project",
                        "mla_query_project_workspace_size", "mla_pack_weight",
                        "mla_naive_workspace_size", "mla_naive_run",
                        "mla_project_new_tokens_workspace_size", "mla_project_new_tokens",
                        "mla_decode_range_flags", "mla_decode_run_noalloc",
                        "mla_decode_check_inputs"}
    lib = _lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_debug_build_exports_the_same_symbols():
    """libmla_decode_debug.so (the ABI compiled with host-side precondition
    checks) loads and exports every symbol the release library does."""
    from mla_latent_kv_amd import binding
    _lib()
    if not os.path.exists(binding.DEBUG_LIB_PATH):
        from mla_latent_kv_amd import build
        build.build()
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|void|const char\*)\s+(mla_\w+)\s*\(", src, re.M))
    dbg = binding.load_library(binding.DEBUG_LIB_PATH)
    for name in declared:
        assert hasattr(dbg, name), name
    # argument errors come back before any device call in both builds
    assert dbg.mla_decode_run(None, None, None, 0, None) == -1
    assert dbg.mla_decode_status_string(-6) == b"inputs break a documented precondition"


def test_status_strings():
    from mla_latent_kv_amd import binding
    _lib()
    assert binding.mla_decode_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6):
        s = binding.mla_decode_status_string(code)
        assert s and s != "unknown status"
    assert binding.mla_decode_status_string(-99) == "unknown status"


@pytest.mark.parametrize("dims", [(64, 128, 64, 512, 128, 64), (128, 128, 64, 512, 128, 16),
                                  (128, 192, 64, 512, 128, 64)])
def test_init_rejects_other_dims(dims):
    from mla_latent_kv_amd import binding
    _lib()
    with pytest.raises(RuntimeError, match="unsupported"):
        binding.mla_decode_init(0, dims=dims)


def test_init_rejects_bad_q_tokens_and_nulls():
    from mla_latent_kv_amd import binding
    lib = _lib()
    with pytest.raises(RuntimeError, match="unsupported"):
        binding.mla_decode_init(0, max_q_tokens=3)
    assert lib.mla_decode_init(None, 0, None) == -1
    assert lib.mla_decode_run(None, None, None, 0, None) == -1
    n = ctypes.c_size_t()
    assert lib.mla_decode_workspace_size(None, 1, 1, 1, ctypes.byref(n)) == -1
    lib.mla_decode_destroy(None)


def test_split_plan_invariants():
    """The split plan (host mirror of the prep kernel's plan) on random
    batches, both its searched and its simple form: every sequence's tokens
    covered once by 64-aligned pieces, partial slots contiguous per sequence
    and within the workspace's capacity, each position's entries dense."""
    import numpy as np
    from tests import plan_mirror as pm
    rng = np.random.default_rng(0)
    for _ in range(1500):
        B = int(rng.choice([1, 2, 3, 7, 32, 64, 128, 255, 256, 300, 1024, 1025, 2000]))
        P = int(rng.choice([1, 7, 8, 128, 256, 1000]))
        mx = int(rng.choice([1, 63, 64, 65, 512, 4096, 40000, 131072]))
        kind = rng.integers(0, 4)
        if kind == 0:
            lens = rng.integers(0, mx + 1, B)
        elif kind == 1:
            lens = np.full(B, mx)
        elif kind == 2:
            lens = np.where(rng.random(B) < 0.5, 0, rng.integers(1, mx + 1, B))
        else:
            lens = rng.integers(-5, mx + 50, B)
        pm.check(lens, mx, P)


def test_split_plan_choices_on_the_workloads():
    """The searched plan picks one round for equal lengths and several for
    ragged ones: uniform 32 x 4096 -> 256 pieces of 512; the ragged and
    two-token workloads -> more pieces than slots, each no longer than C."""
    from mla_latent_kv_amd import synth
    from tests import plan_mirror as pm
    uni = synth.make_batch(synth.CONFIGS[1], seed=1)["seq_lens"]
    r = pm.check(uni, 4096, 256)
    assert r["search"] and r["C"] == 512 and r["n_items"] == 256
    rag = synth.make_batch(synth.CONFIGS[2], seed=2)["seq_lens"]
    r = pm.check(rag, 32768, 256)
    assert r["search"] and 256 < r["n_items"] <= 4 * 256
    mtp = synth.make_batch(synth.CONFIGS[4], seed=4)["seq_lens"]
    r = pm.check(mtp, 16384, 128)
    assert r["search"] and 128 < r["n_items"] <= 4 * 128


def test_cache_append_rejects_nulls_before_any_device_call():
    import ctypes
    from mla_latent_kv_amd import binding
    lib = _lib()
    n = ctypes.c_size_t()
    assert lib.mla_cache_append_workspace_size(None, 4, 1, ctypes.byref(n)) == -1
    args = binding.MlaAppendArgs()
    assert lib.mla_cache_append(None, ctypes.byref(args), None, 0, None) == -1
    assert lib.mla_cache_append(None, None, None, 0, None) == -1


def test_output_project_rejects_nulls_before_any_device_call():
    import ctypes
    from mla_latent_kv_amd import binding
    lib = _lib()
    n = ctypes.c_size_t()
    assert lib.mla_output_project_workspace_size(None, 4, ctypes.byref(n)) == -1
    args = binding.MlaOprojArgs()
    assert lib.mla_output_project(None, ctypes.byref(args), None, 0, None) == -1
    assert lib.mla_output_project(None, None, None, 0, None) == -1


def test_pack_weight_rejects_nulls_before_any_device_call():
    lib = _lib()
    assert lib.mla_pack_weight(None, None, None, 32, 16, None) == -1


def test_query_project_rejects_nulls_before_any_device_call():
    import ctypes
    from mla_latent_kv_amd import binding
    lib = _lib()
    n = ctypes.c_size_t()
    assert lib.mla_query_project_workspace_size(None, 4, 1, ctypes.byref(n)) == -1
    args = binding.MlaQueryArgs()
    assert lib.mla_query_project(None, ctypes.byref(args), None, 0, None) == -1


def test_naive_rejects_nulls_before_any_device_call():
    import ctypes
    from mla_latent_kv_amd import binding
    lib = _lib()
    n = ctypes.c_size_t()
    assert lib.mla_naive_workspace_size(None, 1, 4096, ctypes.byref(n)) == -1
    args = binding.MlaNaiveArgs()
    assert lib.mla_naive_run(None, ctypes.byref(args), None, 0, None) == -1
    assert lib.mla_naive_run(None, None, None, 0, None) == -1


def test_prologue_rejects_nulls_before_any_device_call():
    import ctypes
    from mla_latent_kv_amd import binding
    lib = _lib()
    n = ctypes.c_size_t()
    assert lib.mla_project_new_tokens_workspace_size(None, 4, 1, ctypes.byref(n)) == -1
    args = binding.MlaPrologueArgs()
    assert lib.mla_project_new_tokens(None, ctypes.byref(args), None, 0, None) == -1
    assert lib.mla_project_new_tokens(None, None, None, 0, None) == -1
