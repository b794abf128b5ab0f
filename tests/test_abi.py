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
                        "mla_project_new_tokens_workspace_size", "mla_project_new_tokens"}
    lib = _lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    from mla_latent_kv_amd import binding
    _lib()
    assert binding.mla_decode_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
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


def test_workspace_layout_bounds():
    """The split plan can never need more partial slots than the layout holds:
    sum_b ceil(L_b / C) <= target + B when C >= total / target (host mirror of
    the plan's arithmetic, checked on random lengths)."""
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(2000):
        B = int(rng.integers(1, 300))
        target = int(rng.integers(1, 600))
        max_len = int(rng.integers(1, 200000))
        lens = rng.integers(0, max_len + 1, size=B)
        total = int(lens.sum())
        C = max(64, -(-max(1, -(-total // target)) // 64) * 64)
        chunks = int(sum(-(-int(l) // C) for l in lens))
        cap = min(target + B, B * -(-max_len // 64))
        assert chunks <= cap


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
