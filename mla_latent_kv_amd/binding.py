"""Thin ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels. PyTorch provides device memory and the current stream. The library
must be built in-tree (``python -m mla_latent_kv_amd.build``); if it is
missing, loading raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")
# the same kernels with host-side precondition checks before every launch
DEBUG_LIB_PATH = os.path.join(HERE, "libmla_decode_debug.so")

MLA_OK = 0
N_HEADS, D_NOPE, D_ROPE, D_LATENT, D_V, BLOCK = 128, 128, 64, 512, 128, 64
D_HIDDEN = 7168


class MlaDecodeConfig(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_q_tokens", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("split_target", ctypes.c_int32),
    ]


class MlaDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q_nope", ctypes.c_void_p),
        ("q_pe", ctypes.c_void_p),
        ("w_uk", ctypes.c_void_p),
        ("w_uv", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


class MlaAppendArgs(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_void_p),
        ("w_kv", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
    ]


class MlaQueryArgs(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_void_p),
        ("w_dq", ctypes.c_void_p),
        ("w_uq", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("q_nope", ctypes.c_void_p),
        ("q_pe", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
    ]


class MlaPrologueArgs(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_void_p),
        ("w_dq", ctypes.c_void_p),
        ("w_uq", ctypes.c_void_p),
        ("w_kv", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("q_nope", ctypes.c_void_p),
        ("q_pe", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
    ]


class MlaOprojArgs(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("w_o", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("rows", ctypes.c_int32),
    ]


class MlaNaiveArgs(ctypes.Structure):
    _fields_ = [
        ("q_nope", ctypes.c_void_p),
        ("q_pe", ctypes.c_void_p),
        ("w_uk", ctypes.c_void_p),
        ("w_uv", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


_libs = {}
MLA_ERR_PRECONDITION = -6


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load a built library (once per path; the release build by default).
    Raises RuntimeError when it is absent."""
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mla_latent_kv_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    lib.mla_decode_init.argtypes = [ctypes.POINTER(MlaDecodeConfig), ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_void_p)]
    lib.mla_decode_init.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    lib.mla_decode_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaDecodeArgs),
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_decode_run.restype = ctypes.c_int
    lib.mla_decode_run_profiled.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaDecodeArgs),
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_void_p)]
    lib.mla_decode_run_profiled.restype = ctypes.c_int
    lib.mla_cache_append_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_cache_append_workspace_size.restype = ctypes.c_int
    lib.mla_cache_append.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaAppendArgs),
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_cache_append.restype = ctypes.c_int
    lib.mla_query_project_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_query_project_workspace_size.restype = ctypes.c_int
    lib.mla_query_project.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaQueryArgs),
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_query_project.restype = ctypes.c_int
    lib.mla_project_new_tokens_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_project_new_tokens_workspace_size.restype = ctypes.c_int
    lib.mla_project_new_tokens.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaPrologueArgs), ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_project_new_tokens.restype = ctypes.c_int
    lib.mla_output_project_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_output_project_workspace_size.restype = ctypes.c_int
    lib.mla_output_project.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaOprojArgs),
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_output_project.restype = ctypes.c_int
    lib.mla_pack_weight.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p]
    lib.mla_pack_weight.restype = ctypes.c_int
    lib.mla_naive_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_naive_workspace_size.restype = ctypes.c_int
    lib.mla_naive_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaNaiveArgs), ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_naive_run.restype = ctypes.c_int
    lib.mla_decode_run_noalloc.argtypes = [ctypes.c_void_p, ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    lib.mla_decode_run_noalloc.restype = ctypes.c_int
    lib.mla_decode_range_flags.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]
    lib.mla_decode_range_flags.restype = ctypes.c_int
    lib.mla_decode_destroy.argtypes = [ctypes.c_void_p]
    lib.mla_decode_destroy.restype = None
    lib.mla_decode_status_string.argtypes = [ctypes.c_int]
    lib.mla_decode_status_string.restype = ctypes.c_char_p
    lib.mla_decode_check_inputs.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)]
    lib.mla_decode_check_inputs.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def mla_decode_check_inputs(seq_lens, block_table, q_tokens: int, max_seq_len: int,
                            num_blocks: int):
    """The library's host-side precondition check on host arrays (numpy or CPU
    tensors): seq_lens int32 [B], block_table int32 [B, max_blocks_per_seq].
    Returns (status, first_bad): (0, -1) when the inputs meet the decode
    preconditions, (MLA_ERR_PRECONDITION, b) naming the lowest-numbered
    sequence that breaks one."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens), dtype=np.int32)
    table = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    if lens.ndim != 1 or table.ndim != 2 or table.shape[0] != lens.shape[0]:
        raise ValueError("seq_lens must be [B] and block_table [B, max_blocks_per_seq]")
    bad = ctypes.c_int32(-2)
    st = load_library().mla_decode_check_inputs(
        lens.ctypes.data, table.ctypes.data, int(lens.shape[0]), int(q_tokens), int(table.shape[1]),
        int(max_seq_len), int(num_blocks), ctypes.byref(bad))
    return int(st), int(bad.value)


def mla_decode_status_string(status: int) -> str:
    return load_library().mla_decode_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != MLA_OK:
        raise RuntimeError(f"{what}: {mla_decode_status_string(status)} ({status})")


def mla_decode_init(device: int = 0, max_q_tokens: int = 2, softmax_scale: float = 0.0,
                    split_target: int = 0, dims=None) -> ctypes.c_void_p:
    """Create a context; ``dims`` overrides (H, d_nope, d_rope, d_latent, d_v, block)."""
    h, dn, dr, dc, dv, bs = dims or (N_HEADS, D_NOPE, D_ROPE, D_LATENT, D_V, BLOCK)
    cfg = MlaDecodeConfig(h, dn, dr, dc, dv, bs, max_q_tokens, float(softmax_scale),
                          int(split_target))
    ctx = ctypes.c_void_p()
    _check(load_library().mla_decode_init(ctypes.byref(cfg), int(device), ctypes.byref(ctx)),
           "mla_decode_init")
    return ctx


def mla_decode_workspace_size(ctx, batch: int, q_tokens: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mla_decode_workspace_size(ctx, int(batch), int(q_tokens),
                                                    int(max_seq_len), ctypes.byref(n)),
           "mla_decode_workspace_size")
    return n.value


def mla_decode_destroy(ctx) -> None:
    if ctx:
        load_library().mla_decode_destroy(ctx)


def _require(t, name, dtypes, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got {tuple(t.shape)}")


MLA_RANGE_QABS = 1


def mla_decode_range_flags(ctx, workspace, stream=None) -> int:
    """Range flags of the last decode call on ``workspace`` (synchronises the
    stream): 0, or MLA_RANGE_QABS when a q_abs value was past fp16's range."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(workspace.device)
    flags = ctypes.c_int32()
    _check(load_library().mla_decode_range_flags(ctx, workspace.data_ptr(),
                                                 workspace.numel() * workspace.element_size(),
                                                 ctypes.c_void_p(s.cuda_stream), ctypes.byref(flags)),
           "mla_decode_range_flags")
    return flags.value


def mla_decode_run(ctx, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seq_lens,
                   max_seq_len: int, out=None, workspace=None, stream=None, check_range=False):
    """Enqueue one decode step; returns ``out`` (fp32 [B, Sq, 128, 128]).

    bf16 tensors may be torch.bfloat16 or 16-bit integer views of the same bits.
    ``workspace``: a uint8 CUDA tensor of at least mla_decode_workspace_size bytes
    (allocated here when None). ``stream``: a torch.cuda.Stream or None for the
    current stream. ``check_range``: read the range flags back after the call
    (synchronises) and raise FloatingPointError when q_abs left fp16's range.
    """
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    _require(q_nope, "q_nope", b16, 4)
    _require(q_pe, "q_pe", b16, 4)
    _require(w_uk, "w_uk", b16, 3)
    _require(w_uv, "w_uv", b16, 3)
    _require(kv_cache, "kv_cache", b16, 3)
    _require(block_table, "block_table", (torch.int32,), 2)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    if tuple(q_nope.shape[2:]) != (N_HEADS, D_NOPE) or tuple(q_pe.shape) != (B, Sq, N_HEADS, D_ROPE):
        raise ValueError("q_nope / q_pe shapes must be [B, Sq, 128, 128] / [B, Sq, 128, 64]")
    if tuple(w_uk.shape) != (N_HEADS, D_NOPE, D_LATENT) or tuple(w_uv.shape) != (N_HEADS, D_V, D_LATENT):
        raise ValueError("w_uk / w_uv must be [128, 128, 512]")
    if tuple(kv_cache.shape[1:]) != (BLOCK, D_LATENT + D_ROPE):
        raise ValueError("kv_cache must be [num_blocks, 64, 576]")
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table / seq_lens batch mismatch")
    if out is None:
        out = torch.empty((B, Sq, N_HEADS, D_V), dtype=torch.float32, device=q_nope.device)
    _require(out, "out", (torch.float32,), 4)
    if tuple(out.shape) != (B, Sq, N_HEADS, D_V):
        raise ValueError("out must be [B, Sq, 128, 128] fp32")
    need = mla_decode_workspace_size(ctx, B, Sq, max_seq_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, needs {need}")
    s = stream if stream is not None else torch.cuda.current_stream(q_nope.device)
    args = MlaDecodeArgs(
        q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
        kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
        kv_cache.shape[0], B, Sq, block_table.shape[1], int(max_seq_len))
    _check(load_library().mla_decode_run(ctx, ctypes.byref(args), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         ctypes.c_void_p(s.cuda_stream)),
           "mla_decode_run")
    if check_range and mla_decode_range_flags(ctx, workspace, s) & MLA_RANGE_QABS:
        raise FloatingPointError("mla_decode_run: a q_abs value is past 1048064 (fp16 range after the "
                                 "2^-4 scaling); the output may hold inf or NaN")
    return out


def mla_decode_run_noalloc(ctx, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seq_lens,
                           max_seq_len: int, out, stream=None):
    """mla_decode_run on the library's own per-GPU scratch array (no workspace,
    nothing allocated by the library); ``out`` is required (fp32 [B, Sq, 128,
    128]). The same argument checks as mla_decode_run."""
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    _require(q_nope, "q_nope", b16, 4)
    _require(q_pe, "q_pe", b16, 4)
    _require(w_uk, "w_uk", b16, 3)
    _require(w_uv, "w_uv", b16, 3)
    _require(kv_cache, "kv_cache", b16, 3)
    _require(block_table, "block_table", (torch.int32,), 2)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    _require(out, "out", (torch.float32,), 4)
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    if (tuple(q_nope.shape[2:]) != (N_HEADS, D_NOPE) or tuple(q_pe.shape) != (B, Sq, N_HEADS, D_ROPE)
            or tuple(w_uk.shape) != (N_HEADS, D_NOPE, D_LATENT) or tuple(w_uv.shape) != (N_HEADS, D_V, D_LATENT)
            or tuple(kv_cache.shape[1:]) != (BLOCK, D_LATENT + D_ROPE) or block_table.shape[0] != B
            or tuple(seq_lens.shape) != (B,) or tuple(out.shape) != (B, Sq, N_HEADS, D_V)):
        raise ValueError("mla_decode_run_noalloc: shapes as for mla_decode_run")
    s = stream if stream is not None else torch.cuda.current_stream(q_nope.device)
    args = MlaDecodeArgs(
        q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
        kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
        kv_cache.shape[0], B, Sq, block_table.shape[1], int(max_seq_len))
    _check(load_library().mla_decode_run_noalloc(ctx, ctypes.byref(args), ctypes.c_void_p(s.cuda_stream)),
           "mla_decode_run_noalloc")
    return out


def _workspace(workspace, need, device):
    import torch
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, needs {need}")
    return workspace


def _require_packed(t, name, n, k):
    """A weight packed by mla_pack_weight: a flat bf16 tensor of n * k elements."""
    import torch
    _require(t, name, (torch.bfloat16, torch.int16, torch.uint16), 1)
    if t.numel() != n * k:
        raise ValueError(f"{name} must be the packed {n} x {k} weight ({n * k} elements), "
                         f"got {t.numel()}")


def mla_pack_weight(ctx, w, packed=None, stream=None):
    """Pack a row-major bf16 weight [n, k] (a 3-d tensor is viewed as [prod of
    leading dims, k]) into the layout the projections stream (include/mla_decode.h,
    mla_pack_weight). Returns a flat tensor of n * k elements, w's dtype."""
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    if isinstance(w, torch.Tensor) and w.dim() > 2:
        w = w.reshape(-1, w.shape[-1])
    _require(w, "w", b16, 2)
    n, k = w.shape
    if packed is None:
        packed = torch.empty(n * k, dtype=w.dtype, device=w.device)
    _require(packed, "packed", b16, 1)
    if packed.numel() != n * k:
        raise ValueError("packed must hold n * k elements")
    s = stream if stream is not None else torch.cuda.current_stream(w.device)
    _check(load_library().mla_pack_weight(ctx, w.data_ptr(), packed.data_ptr(), n, k,
                                          ctypes.c_void_p(s.cuda_stream)),
           "mla_pack_weight")
    return packed


def mla_cache_append_workspace_size(ctx, batch: int, q_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mla_cache_append_workspace_size(ctx, int(batch), int(q_tokens),
                                                          ctypes.byref(n)),
           "mla_cache_append_workspace_size")
    return n.value


def mla_cache_append(ctx, hidden, w_kv, kv_cache, block_table, seq_lens,
                     rope_base: float = 0.0, workspace=None, stream=None):
    """Enqueue the cache-append producer: writes the new tokens' rows
    [W_DKV h | RoPE(W_KR h, pos)] (bf16) into ``kv_cache`` in place and returns it.

    hidden [B, Sq, 7168]; w_kv the stacked [W_DKV; W_KR] (576 x 7168) packed by
    mla_pack_weight; kv_cache [num_blocks, 64, 576] (bf16 or 16-bit integer
    views of the bits), block_table int32 [B, max_blocks_per_seq], seq_lens
    int32 [B] counting the new tokens. ``rope_base`` <= 0 selects 10000.
    """
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    _require(hidden, "hidden", b16, 3)
    _require_packed(w_kv, "w_kv", D_LATENT + D_ROPE, D_HIDDEN)
    _require(kv_cache, "kv_cache", b16, 3)
    _require(block_table, "block_table", (torch.int32,), 2)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    B, Sq = hidden.shape[0], hidden.shape[1]
    if hidden.shape[2] != D_HIDDEN:
        raise ValueError("hidden must be [B, Sq, 7168]")
    if tuple(kv_cache.shape[1:]) != (BLOCK, D_LATENT + D_ROPE):
        raise ValueError("kv_cache must be [num_blocks, 64, 576]")
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table / seq_lens batch mismatch")
    workspace = _workspace(workspace, mla_cache_append_workspace_size(ctx, B, Sq), hidden.device)
    s = stream if stream is not None else torch.cuda.current_stream(hidden.device)
    args = MlaAppendArgs(hidden.data_ptr(), w_kv.data_ptr(), kv_cache.data_ptr(),
                         block_table.data_ptr(), seq_lens.data_ptr(), kv_cache.shape[0], B, Sq,
                         block_table.shape[1], float(rope_base))
    _check(load_library().mla_cache_append(ctx, ctypes.byref(args), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(),
                                           ctypes.c_void_p(s.cuda_stream)),
           "mla_cache_append")
    return kv_cache


def mla_query_project_workspace_size(ctx, batch: int, q_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mla_query_project_workspace_size(ctx, int(batch), int(q_tokens),
                                                           ctypes.byref(n)),
           "mla_query_project_workspace_size")
    return n.value


def mla_query_project(ctx, hidden, w_dq, w_uq, seq_lens, rope_base: float = 0.0,
                      q_nope=None, q_pe=None, workspace=None, stream=None):
    """Enqueue the query side: returns (q_nope [B, Sq, 128, 128], q_pe [B, Sq, 128, 64]),
    both bf16, from hidden [B, Sq, 7168] and the packed W_DQ (1536 x 7168) and
    W_UQ (128 x 192 rows x 1536) of mla_pack_weight."""
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    _require(hidden, "hidden", b16, 3)
    _require_packed(w_dq, "w_dq", 1536, D_HIDDEN)
    _require_packed(w_uq, "w_uq", N_HEADS * (D_NOPE + D_ROPE), 1536)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    B, Sq = hidden.shape[0], hidden.shape[1]
    if hidden.shape[2] != D_HIDDEN or tuple(seq_lens.shape) != (B,):
        raise ValueError("hidden must be [B, Sq, 7168] and seq_lens [B]")
    if q_nope is None:
        q_nope = torch.empty((B, Sq, N_HEADS, D_NOPE), dtype=torch.bfloat16, device=hidden.device)
    if q_pe is None:
        q_pe = torch.empty((B, Sq, N_HEADS, D_ROPE), dtype=torch.bfloat16, device=hidden.device)
    _require(q_nope, "q_nope", b16, 4)
    _require(q_pe, "q_pe", b16, 4)
    if tuple(q_nope.shape) != (B, Sq, N_HEADS, D_NOPE) or tuple(q_pe.shape) != (B, Sq, N_HEADS, D_ROPE):
        raise ValueError("q_nope / q_pe shapes must be [B, Sq, 128, 128] / [B, Sq, 128, 64]")
    workspace = _workspace(workspace, mla_query_project_workspace_size(ctx, B, Sq), hidden.device)
    s = stream if stream is not None else torch.cuda.current_stream(hidden.device)
    args = MlaQueryArgs(hidden.data_ptr(), w_dq.data_ptr(), w_uq.data_ptr(), seq_lens.data_ptr(),
                        q_nope.data_ptr(), q_pe.data_ptr(), B, Sq, float(rope_base))
    _check(load_library().mla_query_project(ctx, ctypes.byref(args), workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(),
                                            ctypes.c_void_p(s.cuda_stream)),
           "mla_query_project")
    return q_nope, q_pe


def mla_project_new_tokens_workspace_size(ctx, batch: int, q_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mla_project_new_tokens_workspace_size(ctx, int(batch), int(q_tokens),
                                                                ctypes.byref(n)),
           "mla_project_new_tokens_workspace_size")
    return n.value


def mla_project_new_tokens(ctx, hidden, w_dq, w_uq, w_kv, kv_cache, block_table, seq_lens,
                           rope_base: float = 0.0, q_nope=None, q_pe=None, workspace=None, stream=None):
    """Enqueue the decode-step prologue: the new tokens' cache rows (as
    mla_cache_append) and their queries (as mla_query_project) in one call.
    Weights packed by mla_pack_weight. Returns (q_nope, q_pe); kv_cache is
    written in place."""
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    _require(hidden, "hidden", b16, 3)
    _require_packed(w_dq, "w_dq", 1536, D_HIDDEN)
    _require_packed(w_uq, "w_uq", N_HEADS * (D_NOPE + D_ROPE), 1536)
    _require_packed(w_kv, "w_kv", D_LATENT + D_ROPE, D_HIDDEN)
    _require(kv_cache, "kv_cache", b16, 3)
    _require(block_table, "block_table", (torch.int32,), 2)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    B, Sq = hidden.shape[0], hidden.shape[1]
    if hidden.shape[2] != D_HIDDEN:
        raise ValueError("hidden must be [B, Sq, 7168]")
    if tuple(kv_cache.shape[1:]) != (BLOCK, D_LATENT + D_ROPE):
        raise ValueError("kv_cache must be [num_blocks, 64, 576]")
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table / seq_lens batch mismatch")
    if q_nope is None:
        q_nope = torch.empty((B, Sq, N_HEADS, D_NOPE), dtype=torch.bfloat16, device=hidden.device)
    if q_pe is None:
        q_pe = torch.empty((B, Sq, N_HEADS, D_ROPE), dtype=torch.bfloat16, device=hidden.device)
    _require(q_nope, "q_nope", b16, 4)
    _require(q_pe, "q_pe", b16, 4)
    if tuple(q_nope.shape) != (B, Sq, N_HEADS, D_NOPE) or tuple(q_pe.shape) != (B, Sq, N_HEADS, D_ROPE):
        raise ValueError("q_nope / q_pe shapes must be [B, Sq, 128, 128] / [B, Sq, 128, 64]")
    workspace = _workspace(workspace, mla_project_new_tokens_workspace_size(ctx, B, Sq), hidden.device)
    s = stream if stream is not None else torch.cuda.current_stream(hidden.device)
    args = MlaPrologueArgs(hidden.data_ptr(), w_dq.data_ptr(), w_uq.data_ptr(), w_kv.data_ptr(),
                           kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), q_nope.data_ptr(),
                           q_pe.data_ptr(), kv_cache.shape[0], B, Sq, block_table.shape[1], float(rope_base))
    _check(load_library().mla_project_new_tokens(ctx, ctypes.byref(args), workspace.data_ptr(),
                                                 workspace.numel() * workspace.element_size(),
                                                 ctypes.c_void_p(s.cuda_stream)),
           "mla_project_new_tokens")
    return q_nope, q_pe


def mla_output_project_workspace_size(ctx, rows: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mla_output_project_workspace_size(ctx, int(rows), ctypes.byref(n)),
           "mla_output_project_workspace_size")
    return n.value


def mla_output_project(ctx, x, w_o, y=None, workspace=None, stream=None):
    """Enqueue y = W_O x: x fp32 [T, 16384] (or mla_decode_run's out [B, Sq,
    128, 128], viewed flat), w_o the packed W_O (7168 x 16384) of
    mla_pack_weight; returns y fp32 [T, 7168]."""
    import torch
    if x.dim() == 4:
        x = x.reshape(-1, N_HEADS * D_V)
    _require(x, "x", (torch.float32,), 2)
    _require_packed(w_o, "w_o", D_HIDDEN, N_HEADS * D_V)
    if x.shape[1] != N_HEADS * D_V:
        raise ValueError("x must be [T, 16384]")
    if y is None:
        y = torch.empty((x.shape[0], D_HIDDEN), dtype=torch.float32, device=x.device)
    _require(y, "y", (torch.float32,), 2)
    if tuple(y.shape) != (x.shape[0], D_HIDDEN):
        raise ValueError("y must be [T, 7168] fp32")
    workspace = _workspace(workspace, mla_output_project_workspace_size(ctx, x.shape[0]), x.device)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    args = MlaOprojArgs(x.data_ptr(), w_o.data_ptr(), y.data_ptr(), x.shape[0])
    _check(load_library().mla_output_project(ctx, ctypes.byref(args), workspace.data_ptr(),
                                             workspace.numel() * workspace.element_size(),
                                             ctypes.c_void_p(s.cuda_stream)),
           "mla_output_project")
    return y


def mla_naive_workspace_size(ctx, batch: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mla_naive_workspace_size(ctx, int(batch), int(max_seq_len), ctypes.byref(n)),
           "mla_naive_workspace_size")
    return n.value


def mla_naive_run(ctx, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seq_lens,
                  max_seq_len: int, out=None, workspace=None, stream=None):
    """Enqueue the naive path (materialised K and V, then causal softmax
    attention); any Sq in [1, max_seq_len] (Sq = L: prefill). w_uk / w_uv are
    W_UK / W_UV packed by mla_pack_weight. Returns ``out`` (fp32 [B, Sq, 128, 128])."""
    import torch
    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    _require(q_nope, "q_nope", b16, 4)
    _require(q_pe, "q_pe", b16, 4)
    _require_packed(w_uk, "w_uk", N_HEADS * D_NOPE, D_LATENT)
    _require_packed(w_uv, "w_uv", N_HEADS * D_V, D_LATENT)
    _require(kv_cache, "kv_cache", b16, 3)
    _require(block_table, "block_table", (torch.int32,), 2)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    if tuple(q_nope.shape[2:]) != (N_HEADS, D_NOPE) or tuple(q_pe.shape) != (B, Sq, N_HEADS, D_ROPE):
        raise ValueError("q_nope / q_pe shapes must be [B, Sq, 128, 128] / [B, Sq, 128, 64]")
    if tuple(kv_cache.shape[1:]) != (BLOCK, D_LATENT + D_ROPE):
        raise ValueError("kv_cache must be [num_blocks, 64, 576]")
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table / seq_lens batch mismatch")
    if out is None:
        out = torch.empty((B, Sq, N_HEADS, D_V), dtype=torch.float32, device=q_nope.device)
    _require(out, "out", (torch.float32,), 4)
    if tuple(out.shape) != (B, Sq, N_HEADS, D_V):
        raise ValueError("out must be [B, Sq, 128, 128] fp32")
    workspace = _workspace(workspace, mla_naive_workspace_size(ctx, B, max_seq_len), q_nope.device)
    s = stream if stream is not None else torch.cuda.current_stream(q_nope.device)
    args = MlaNaiveArgs(q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                        kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                        kv_cache.shape[0], B, Sq, block_table.shape[1], int(max_seq_len))
    _check(load_library().mla_naive_run(ctx, ctypes.byref(args), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        ctypes.c_void_p(s.cuda_stream)),
           "mla_naive_run")
    return out


class MLADecoder:
    """Owns a context; ``decoder(...)`` forwards to mla_decode_run."""

    def __init__(self, device: int = 0, max_q_tokens: int = 2, softmax_scale: float = 0.0,
                 split_target: int = 0):
        self.device = device
        self.ctx = mla_decode_init(device, max_q_tokens, softmax_scale, split_target)

    def workspace_size(self, batch, q_tokens, max_seq_len) -> int:
        return mla_decode_workspace_size(self.ctx, batch, q_tokens, max_seq_len)

    def __call__(self, *args, **kw):
        return mla_decode_run(self.ctx, *args, **kw)

    def pack(self, w, **kw):
        """Forwards to mla_pack_weight (a weight in the projections' packed layout)."""
        return mla_pack_weight(self.ctx, w, **kw)

    def naive(self, *args, **kw):
        """Forwards to mla_naive_run (materialised K and V; prefill when Sq = L)."""
        return mla_naive_run(self.ctx, *args, **kw)

    def append(self, *args, **kw):
        """Forwards to mla_cache_append (the new tokens' cache rows)."""
        return mla_cache_append(self.ctx, *args, **kw)

    def query_project(self, *args, **kw):
        """Forwards to mla_query_project (q_nope, q_pe of the new tokens)."""
        return mla_query_project(self.ctx, *args, **kw)

    def project_new_tokens(self, *args, **kw):
        """Forwards to mla_project_new_tokens (cache rows and queries of the new tokens)."""
        return mla_project_new_tokens(self.ctx, *args, **kw)

    def output_project(self, *args, **kw):
        """Forwards to mla_output_project (y = W_O x)."""
        return mla_output_project(self.ctx, *args, **kw)

    def close(self):
        if self.ctx:
            mla_decode_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
