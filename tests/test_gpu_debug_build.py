"""The debug build (libmla_decode_debug.so: the same kernels, host-side
precondition checks before every launch) through the C ABI.

On valid inputs it gives the release build's output bit for bit. On inputs
that break a documented precondition (a block id outside the cache, a length
past max_seq_len, two sequences' new tokens in one slot) it returns
MLA_ERR_PRECONDITION before launching anything: the output and the cache keep
the sentinel bytes they held. No kernel ever runs on the broken inputs.
"""

import ctypes
import os

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, oracle, say

pytestmark = pytest.mark.gpu

PRE = -6


def _dbg():
    from mla_latent_kv_amd import binding
    if not os.path.exists(binding.DEBUG_LIB_PATH):
        pytest.fail("libmla_decode_debug.so is missing: build with python -m mla_latent_kv_amd.build")
    return binding.load_library(binding.DEBUG_LIB_PATH)


def _ctx(lib):
    from mla_latent_kv_amd import binding
    cfg = binding.MlaDecodeConfig(128, 128, 64, 512, 128, 64, 2, 0.0, 0)
    ctx = ctypes.c_void_p()
    assert lib.mla_decode_init(ctypes.byref(cfg), 0, ctypes.byref(ctx)) == 0
    return ctx


def _run(lib, ctx, d, out, max_seq_len=None, table=None, noalloc=False):
    """Status of one decode call of `lib` on uploaded batch `d`."""
    import torch
    from mla_latent_kv_amd import binding
    table = d["block_table"] if table is None else table
    msl = d["max_seq_len"] if max_seq_len is None else max_seq_len
    B, Sq = d["q_nope"].shape[:2]
    args = binding.MlaDecodeArgs(
        d["q_nope"].data_ptr(), d["q_pe"].data_ptr(), d["w_uk"].data_ptr(), d["w_uv"].data_ptr(),
        d["kv_cache"].data_ptr(), table.data_ptr(), d["seq_lens"].data_ptr(), out.data_ptr(),
        d["kv_cache"].shape[0], B, Sq, table.shape[1], msl)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = lib.mla_decode_run_noalloc(ctx, ctypes.byref(args), s)
    else:
        n = ctypes.c_size_t()
        assert lib.mla_decode_workspace_size(ctx, B, Sq, msl, ctypes.byref(n)) == 0
        ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
        st = lib.mla_decode_run(ctx, ctypes.byref(args), ws.data_ptr(), n.value, s)
    torch.cuda.synchronize()
    return st


def test_debug_build_gives_the_release_output_bitwise():
    import torch
    from mla_latent_kv_amd import binding, device
    lib = _dbg()
    batch = synth.make_batch(synth.Spec("dbg_valid", 4, 2, (300, 1100, 64, 2049)), seed=71)
    say(f"case debug build, valid: lens={batch['seq_lens'].tolist()} Sq=2")
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2)
    ref = dec(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"],
              d["seq_lens"], d["max_seq_len"])
    torch.cuda.synchronize()
    ctx = _ctx(lib)
    out = torch.full_like(ref, float("nan"))
    assert _run(lib, ctx, d, out) == 0
    got = out.cpu().numpy()
    assert np.array_equal(got, ref.cpu().numpy())
    assert_parity(got.astype(np.float64), oracle(batch), "debug build")
    out2 = torch.full_like(ref, float("nan"))
    assert _run(lib, ctx, d, out2, noalloc=True) == 0
    assert np.isfinite(out2.cpu().numpy()).all()
    lib.mla_decode_destroy(ctx)
    dec.close()


def test_debug_build_refuses_broken_inputs_before_any_launch():
    import torch
    from mla_latent_kv_amd import device
    lib = _dbg()
    # no NaN padding: the accepted case below lets sequence 1 read a block
    # whose tail slots belong to it
    batch = synth.make_batch(synth.Spec("dbg_broken", 3, 1, (130, 64, 700)), seed=72, poison=False)
    d = device.upload(batch)
    ctx = _ctx(lib)
    B = batch["seq_lens"].shape[0]
    sentinel = 7.25
    nblk = d["kv_cache"].shape[0]
    cases = []
    t = d["block_table"].clone()
    t[2, 5] = nblk                        # sequence 2 uses blocks 0..10
    cases.append(("block id = num_blocks", dict(table=t)))
    t = d["block_table"].clone()
    t[0, 1] = -1
    cases.append(("block id -1 in use", dict(table=t)))
    cases.append(("length past max_seq_len", dict(max_seq_len=699)))
    t = d["block_table"].clone()
    t[1, 0] = t[0, 2]                     # sequence 1's last token (slot 63) vs sequence 0's (slot 1): no clash
    cases.append(("shared block, distinct new-token slots", dict(table=t, ok=True)))
    for name, kw in cases:
        ok = kw.pop("ok", False)
        for noalloc in (False, True):
            say(f"case debug build: {name}, noalloc={noalloc}")
            out = torch.full((B, 1, 128, 128), sentinel, dtype=torch.float32, device="cuda")
            st = _run(lib, ctx, d, out, noalloc=noalloc, **kw)
            if ok:
                assert st == 0
                assert np.isfinite(out.cpu().numpy()).all()
            else:
                assert st == PRE, st
                assert (out.cpu().numpy() == sentinel).all(), "a kernel ran on refused inputs"
    lib.mla_decode_destroy(ctx)


def test_debug_build_refuses_a_shared_new_token_slot_in_the_append():
    import torch
    from mla_latent_kv_amd import binding
    lib = _dbg()
    ctx = _ctx(lib)
    B, Sq, nblk = 2, 1, 4
    lens = torch.tensor([5, 69], dtype=torch.int32, device="cuda")
    # sequence 1's token 68 is slot 4 of its second block, block 0: sequence
    # 0's token 4 is slot 4 of block 0 too
    table = torch.tensor([[0, 1], [2, 0]], dtype=torch.int32, device="cuda")
    cache = torch.full((nblk, 64, 576), 0x3f80, dtype=torch.int16, device="cuda")   # bf16 1.0
    hidden = torch.zeros((B, Sq, 7168), dtype=torch.int16, device="cuda")
    w_kv = torch.zeros((576 * 7168,), dtype=torch.int16, device="cuda")
    n = ctypes.c_size_t()
    assert lib.mla_cache_append_workspace_size(ctx, B, Sq, ctypes.byref(n)) == 0
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    args = binding.MlaAppendArgs(hidden.data_ptr(), w_kv.data_ptr(), cache.data_ptr(), table.data_ptr(),
                                 lens.data_ptr(), nblk, B, Sq, 2, 0.0)
    say("case debug build: append with a shared new-token slot")
    st = lib.mla_cache_append(ctx, ctypes.byref(args), ws.data_ptr(), n.value,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == PRE, st
    assert (cache.cpu().numpy() == 0x3f80).all(), "the append wrote rows after refusing its inputs"
    lib.mla_decode_destroy(ctx)


def test_debug_build_checks_the_naive_path():
    """mla_naive_run of the debug build: a prefill whose table repeats one of
    the sequence's blocks is refused before any launch; the valid table gives
    the release build's output bit for bit."""
    import torch
    from mla_latent_kv_amd import binding, device
    lib = _dbg()
    batch = synth.make_batch(synth.Spec("dbg_naive", 1, 200, (300,)), seed=73)
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2)
    w_uk, w_uv = dec.pack(d["w_uk"]), dec.pack(d["w_uv"])
    ref = dec.naive(d["q_nope"], d["q_pe"], w_uk, w_uv, d["kv_cache"], d["block_table"], d["seq_lens"],
                    d["max_seq_len"])
    torch.cuda.synchronize()
    ctx = _ctx(lib)
    B, Sq = d["q_nope"].shape[:2]
    n = ctypes.c_size_t()
    assert lib.mla_naive_workspace_size(ctx, B, d["max_seq_len"], ctypes.byref(n)) == 0
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")

    def run(table, out):
        args = binding.MlaNaiveArgs(
            d["q_nope"].data_ptr(), d["q_pe"].data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
            d["kv_cache"].data_ptr(), table.data_ptr(), d["seq_lens"].data_ptr(), out.data_ptr(),
            d["kv_cache"].shape[0], B, Sq, table.shape[1], d["max_seq_len"])
        st = lib.mla_naive_run(ctx, ctypes.byref(args), ws.data_ptr(), n.value,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        return st

    say("case debug build: naive prefill, block repeated within the sequence")
    bad = d["block_table"].clone()
    bad[0, 3] = bad[0, 1]              # blocks 1 and 3 of the 5 the sequence uses
    out = torch.full_like(ref, 7.25)
    assert run(bad, out) == PRE
    assert (out.cpu().numpy() == 7.25).all(), "a kernel ran on refused inputs"
    say("case debug build: naive prefill, valid")
    out = torch.full_like(ref, float("nan"))
    assert run(d["block_table"], out) == 0
    assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())
    lib.mla_decode_destroy(ctx)
    dec.close()
