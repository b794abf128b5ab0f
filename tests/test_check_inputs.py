"""The host-side precondition check (mla_decode_check_inputs), on the CPU:
the workloads' tables pass, each documented violation is reported with the
lowest offending sequence, and the sanitizer build (AddressSanitizer and
UndefinedBehaviorSanitizer) runs it over random malformed inputs against a
direct restatement of the conditions."""

import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

from mla_latent_kv_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PRE = binding.MLA_ERR_PRECONDITION
BAD_ARG = -1


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        from mla_latent_kv_amd import build
        build.build()
    return binding.load_library()


def check(lens, table, sq, max_len, nblk):
    _lib()
    return binding.mla_decode_check_inputs(lens, table, sq, max_len, nblk)


@pytest.mark.parametrize("cfg", range(len(synth.CONFIGS)))
def test_workload_tables_pass(cfg):
    """Every workload's lengths and block table (random block permutation,
    -1 past each sequence's blocks) meets the preconditions."""
    spec = synth.CONFIGS[cfg]
    lens, table, max_len, nblk = synth.make_tables(spec, seed=cfg)
    assert check(lens, table, spec.q_tokens, max_len, nblk) == (0, -1)


def _base():
    # three sequences of 130, 64 and 1 tokens in distinct blocks 0..4
    lens = np.array([130, 64, 1], np.int32)
    table = np.array([[3, 0, 4], [1, -1, -1], [2, -1, -1]], np.int32)
    return lens, table


def test_valid_small_case_and_unread_tail_entries():
    lens, table = _base()
    assert check(lens, table, 1, 192, 5) == (0, -1)
    assert check(lens, table, 2, 192, 5) == (0, -1)
    # entries past ceil(L_b / 64) are never read: any value passes
    t = table.copy()
    t[1, 1:] = [99, -7]
    assert check(lens, t, 1, 192, 5) == (0, -1)


def test_lengths_outside_zero_to_max_seq_len():
    lens, table = _base()
    for b, v in ((0, 193), (1, -1), (2, 1 << 30)):
        x = lens.copy()
        x[b] = v
        assert check(x, table, 1, 192, 5) == (PRE, b)
    x = lens.copy()
    x[1] = 0                     # an empty sequence is allowed
    assert check(x, table, 1, 192, 5) == (0, -1)
    assert check(lens, table, 1, 130, 5) == (0, -1)     # L_b == max_seq_len
    assert check(lens, table, 1, 129, 5) == (PRE, 0)


@pytest.mark.parametrize("val", [-1, 5, (1 << 31) - 1])
def test_block_ids_outside_the_cache(val):
    lens, table = _base()
    t = table.copy()
    t[0, 2] = val                # the third block of sequence 0 (tokens 128, 129)
    assert check(lens, t, 1, 192, 5) == (PRE, 0)
    t = table.copy()
    t[2, 0] = val
    assert check(lens, t, 1, 192, 5) == (PRE, 2)
    # one block fewer in the cache makes id 4 out of range
    assert check(lens, table, 1, 192, 4) == (PRE, 0)


def test_shared_new_token_slot_names_the_later_sequence():
    lens, table = _base()
    # sequence 2's only token (slot 0 of block 2) moved into sequence 0's
    # last block, slot 0: sequence 0's new token is at slot 1 (token 129)
    t = table.copy()
    t[2, 0] = 4
    assert check(lens, t, 1, 192, 5) == (0, -1)
    # with two new tokens, sequence 0's are tokens 128 and 129: slot 0 clashes
    assert check(lens, t, 2, 192, 5) == (PRE, 2)
    # sequences 1 and 2 both ending in slot 0 of block 2
    x = np.array([130, 65, 1], np.int32)
    t = np.array([[3, 0, 4], [1, 2, -1], [2, -1, -1]], np.int32)
    assert check(x, t, 1, 192, 5) == (PRE, 2)


def test_shared_prefix_blocks_are_allowed():
    # two sequences on the same first block (a common 64-token prefix), each
    # with its own second block for its new tokens
    lens = np.array([100, 90], np.int32)
    table = np.array([[0, 1], [0, 2]], np.int32)
    assert check(lens, table, 2, 128, 3) == (0, -1)
    # if both new-token rows land in the shared block, the later one breaks it
    assert check(np.array([40, 30], np.int32), table, 1, 128, 3) == (0, -1)
    assert check(np.array([40, 40], np.int32), table, 1, 128, 3) == (PRE, 1)


def test_a_sequence_repeating_one_of_its_blocks():
    # sequence 0 maps its first and third logical blocks to physical block 3
    lens, table = _base()
    t = table.copy()
    t[0, 2] = 3
    assert check(lens, t, 1, 192, 5) == (PRE, 0)
    # a repeat past the blocks the sequence uses is never read
    t = table.copy()
    t[1, 1] = 1
    assert check(lens, t, 1, 192, 5) == (0, -1)


def test_lowest_offender_is_reported():
    lens = np.array([10, 900, 10, -5], np.int32)
    table = np.array([[0, 9], [1, 9], [2, 9], [3, 9]], np.int32)
    assert check(lens, table, 1, 128, 4) == (PRE, 1)
    lens[1] = 10
    assert check(lens, table, 1, 128, 4) == (PRE, 3)


def test_invalid_arguments():
    lens, table = _base()
    lib = _lib()
    bad = ctypes.c_int32(7)
    assert lib.mla_decode_check_inputs(None, None, 3, 1, 3, 192, 5, ctypes.byref(bad)) == BAD_ARG
    assert bad.value == -1
    assert check(lens, table, 0, 192, 5)[0] == BAD_ARG            # q_tokens < 1
    assert check(lens, table, 1, 193, 5)[0] == BAD_ARG            # past 64 * max_blocks_per_seq
    assert check(lens, table, 1, 0, 5)[0] == BAD_ARG
    assert check(lens, table, 1, 192, 0)[0] == BAD_ARG


def test_random_cases_match_a_restatement():
    """Small random batches (valid and broken) against the conditions as the
    header states them, written out directly."""
    rng = np.random.default_rng(3)

    def want(lens, table, sq, max_len, nblk):
        in_range, ok = [], []
        for b, L in enumerate(lens):
            used = [int(table[b, k]) for k in range(-(-L // 64))] if 0 <= L <= max_len else None
            in_range.append(used is not None and all(0 <= x < nblk for x in used))
            ok.append(in_range[b] and len(set(used)) == len(used))
        seen = {}
        for b, L in enumerate(lens):
            if not in_range[b]:
                continue
            slots = {int(table[b, j // 64]) * 64 + j % 64 for j in range(max(0, L - sq), L)}
            if any(s in seen for s in slots):
                ok[b] = False
            for s in slots:
                seen.setdefault(s, b)
        bad = [b for b, v in enumerate(ok) if not v]
        return (PRE, bad[0]) if bad else (0, -1)

    for _ in range(400):
        B, sq, mbps = int(rng.integers(1, 9)), int(rng.integers(1, 3)), int(rng.integers(1, 4))
        max_len = int(rng.integers(1, 64 * mbps + 1))
        nblk = int(rng.integers(1, 3 * B * mbps + 1))
        lens = rng.integers(-2, max_len + 20, B).astype(np.int32)
        table = rng.integers(-1, nblk + 1, (B, mbps)).astype(np.int32)
        assert check(lens, table, sq, max_len, nblk) == want(lens, table, sq, max_len, nblk)


def test_checker_under_address_and_undefined_sanitizers(tmp_path):
    """check.cpp built on its own with g++ -fsanitize=address,undefined: 20,000
    random cases with exactly-sized heap arrays, statuses compared with a
    direct restatement inside the driver (tests/native/check_inputs_fuzz.cpp)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "check_inputs_fuzz")
    # the sanitizer runtimes linked statically, so they come first whatever
    # else the process loads
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-static-libasan", "-static-libubsan", "-fno-omit-frame-pointer", os.path.join(ROOT, "mla_latent_kv_amd", "csrc", "check.cpp"),
           os.path.join(ROOT, "tests", "native", "check_inputs_fuzz.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "cases ok" in run.stdout
