#!/usr/bin/env python3
"""Benchmark: MLA absorbed-path decode on one MI355X.

One step = one call of mla_decode_run over the uniform decode workload
(B = 32 sequences, one new token each, 4096 cached tokens each, 128 heads,
paged 576-wide bf16 latent cache with 64-token blocks and a permuted block
table): split plan, absorb product, fused score / softmax / latent pass, split
merge with the W_UV product. Inputs are resident in HBM before the timed
region; consecutive steps rotate over several independent copies of the
inputs (each ~188 MB, together well past the 256 MB Infinity Cache) so that
every step streams its cache from HBM, as successive layers of a model do.
The default warm-up (1000 steps, ~75 ms) outlasts the clock ramp the GPU
goes through after idle, so the timed steps run at the steady rate.

Prints one JSON line (see the keys below). Per-kernel durations come from HIP
events the library records between its launches (mla_decode_run_profiled);
the roofline entry is for the dominant kernel, the attention pass, whose
algorithmic bytes are the cached rows it must read (1152 B per cached token).
The CPU baseline times the fp64 oracle on a bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s + latent-cache HBM TB/s, MLA absorb B=32 L=4K"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, published
MALL_BYTES = 256 << 20         # Infinity Cache
APPEND_WEIGHT_BYTES = (512 + 64) * 7168 * 2   # W_DKV and W_KR, bf16
OPROJ_WEIGHT_BYTES = 7168 * 16384 * 2         # W_O, bf16
QPROJ_WEIGHT_BYTES = (1536 * 7168 + 128 * 192 * 1536) * 2   # W_DQ and W_UQ, bf16

# HBM traffic of one attention launch from two rocprofv3 --pmc runs of this
# script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what
# the same counter reads for a plain device copy of known size (--copy-probe).
# The figures belong to the workload and the attention source they were taken
# on: for another workload, or when the source hash differs, traffic is null.
ATTN_TRAFFIC = {"workload": "uniform_b32_l4096",
                "src_sha256": "4194bb4f4ec7237603627b66cdc975c9efcc654655d82559428a1054a986d0a6",
                "fetch_kib": 76340.2, "write_kib": 32896.0,
                "fetch_scale": 1048576.0 / 524302.6, "write_scale": 1.0}
TRAFFIC_SOURCES = ("mla_latent_kv_amd/csrc/attn.hip", "mla_latent_kv_amd/csrc/common.h")


def attn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def attn_traffic(workload: str):
    t = ATTN_TRAFFIC
    if not t or t["workload"] != workload or t["src_sha256"] != attn_source_hash():
        return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def copy_probe(mib: int) -> int:
    """A plain device-to-device copy of `mib` MiB, five times: the calibration
    kernel for the FETCH_SIZE / WRITE_SIZE counters (reads and writes exactly
    mib MiB per dispatch)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 5}), flush=True)
    return 0


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


# hipEventDisableSystemFence: the event's record skips the system-scope fence
# (an L2 writeback and invalidate), which would otherwise slow the kernel after
# it; these events only time, and are read after a device synchronisation
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _events(hip, n):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    return evs


def _elapsed(hip, a, b):
    ms = ctypes.c_float()
    if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


def copy_bandwidth(mib: int = 1024, reps: int = 5) -> dict:
    """A plain device-to-device copy of `mib` MiB on the same GPU (torch's
    copy kernel), timed with events: the practical HBM ceiling beside the
    published 8 TB/s."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return {"bytes_read_and_written": 2 * n, "TBps": 2 * n / s / 1e12}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(batch, budget_s: float, max_seqs: int, gpu_out=None) -> dict:
    """The fp64 oracle (naive path) on whole sequences of the batch until the
    time budget is spent; reported as query tokens per second. Beside it the
    oracle's absorb-order routine on the whole batch, whose result also checks
    every output of the timed GPU steps (`gpu_out`, the last timed step's
    output) against the parity tolerance."""
    from oracle import mla_oracle as orc
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = os.cpu_count() or 1
    done, t0 = 0, time.perf_counter()
    B = batch["seq_lens"].shape[0]
    for b in range(min(B, max_seqs)):
        sl = slice(b, b + 1)
        orc.decode_batch(batch["q_nope"][sl], batch["q_pe"][sl], batch["w_uk"], batch["w_uv"],
                         batch["cache"], batch["block_table"][sl], batch["seq_lens"][sl],
                         batch["block_size"])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    q = done * batch["q_nope"].shape[1]
    tokens = int(batch["seq_lens"][:done].sum())
    # the absorb-order routine of the oracle (the GPU path's algorithm, fp64)
    # on the whole batch
    ta = time.perf_counter()
    ref = orc.decode_batch(batch["q_nope"], batch["q_pe"], batch["w_uk"], batch["w_uv"], batch["cache"],
                           batch["block_table"], batch["seq_lens"], batch["block_size"], path="absorb")
    da = time.perf_counter() - ta
    qa = B * batch["q_nope"].shape[1]
    out = {"value": q / dt, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
           "cpu_model": cpu_model(), "blas_threads": int(threads),
           "sample": f"{done} of {B} sequences ({tokens} cached tokens x 128 heads), "
                     f"fp64 NumPy naive path, {dt:.1f} s",
           "absorb_order": {"value": qa / da, "unit": "query-tokens/s",
                            "sample": f"all {B} sequences, fp64 NumPy absorb order, {da:.2f} s"}}
    if gpu_out is not None:
        g = gpu_out.astype(np.float64)
        err = np.abs(g - ref)
        max_rel = float(err.max() / np.abs(ref).max())
        mean_rel = float(err.sum() / np.abs(ref).sum())
        out["check"] = {"outputs": int(ref.size), "max_rel": max_rel, "mean_rel": mean_rel,
                        "finite": bool(np.isfinite(g).all()),
                        "pass": bool(np.isfinite(g).all() and max_rel <= 1e-2 and mean_rel <= 2e-3),
                        "against": "oracle absorb order, every output of the last timed step"}
    return out


def time_cache_append(lib, dec, d, B, Sq, stream, args) -> dict:
    """The cache-append producer on the same batch shape (its new tokens'
    rows), HIP events around `steps` calls on the launch stream. The weights
    rotate over enough copies (8.3 MB each) to exceed the Infinity Cache, as
    successive layers' weights would."""
    import torch
    from mla_latent_kv_amd import binding, synth
    n_w = max(1, math.ceil(MALL_BYTES / (APPEND_WEIGHT_BYTES)) + 1)
    inp = synth.make_append_inputs(B, Sq, seed=1000)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    hid = bf16(inp["hidden"])
    # the stacked [W_DKV; W_KR] packed once (a load-time step, not timed)
    ws = [dec.pack(bf16(np.concatenate([inp["w_dkv"], inp["w_kr"]])))]
    ws += [ws[0].clone() for _ in range(n_w - 1)]
    cache = d["kv_cache"].clone()   # the decode inputs stay as they were
    need = binding.mla_cache_append_workspace_size(dec.ctx, B, Sq)
    wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
    cargs = [binding.MlaAppendArgs(hid.data_ptr(), w.data_ptr(), cache.data_ptr(),
                                   d["block_table"].data_ptr(), d["seq_lens"].data_ptr(),
                                   cache.shape[0], B, Sq, d["block_table"].shape[1], 0.0)
             for w in ws]
    sh = ctypes.c_void_p(stream.cuda_stream)

    def call(i):
        rc = lib.mla_cache_append(dec.ctx, ctypes.byref(cargs[i % n_w]), ctypes.c_void_p(wsp.data_ptr()),
                                  need, sh)
        if rc != 0:
            raise RuntimeError(binding.mla_decode_status_string(rc))

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    rows = B * Sq
    nbytes = APPEND_WEIGHT_BYTES + rows * 7168 * 2 + rows * 1152
    out = {"us_per_call": us, "new_tokens": rows, "rotating_weight_sets": n_w,
           "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
           "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "launches": 2}
    if not args.no_cpu:
        # the oracle's fp64 rows for the same tokens, timed on the host
        from oracle import mla_oracle as orc
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 1.0:
            orc.append_batch(inp["hidden"], inp["w_dkv"], inp["w_kr"],
                             d["seq_lens"].cpu().numpy(), Sq)
            reps += 1
        out["cpu_oracle_us_per_call"] = (time.perf_counter() - t0) / reps * 1e6
    return out


def time_output_project(lib, dec, B, Sq, stream, args) -> dict:
    """The output projection for the batch's tokens (y = W_O x, 235 MB of
    weights), HIP events around `steps` calls; two weight copies alternate so
    the Infinity Cache cannot hold the stream."""
    import torch
    from mla_latent_kv_amd import binding, synth
    rows = B * Sq
    inp = synth.make_oproj_inputs(rows, seed=2000)
    x = torch.from_numpy(inp["x"]).cuda()
    w0 = dec.pack(torch.from_numpy(np.ascontiguousarray(inp["w_o"]).view(np.int16)).cuda())
    n_w = max(2, math.ceil(MALL_BYTES / OPROJ_WEIGHT_BYTES) + 1)
    ws = [w0] + [w0.clone() for _ in range(n_w - 1)]
    y = torch.empty((rows, 7168), dtype=torch.float32, device="cuda")
    need = binding.mla_output_project_workspace_size(dec.ctx, rows)
    wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
    cargs = [binding.MlaOprojArgs(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows) for w in ws]
    sh = ctypes.c_void_p(stream.cuda_stream)

    def call(i):
        rc = lib.mla_output_project(dec.ctx, ctypes.byref(cargs[i % n_w]), ctypes.c_void_p(wsp.data_ptr()),
                                    need, sh)
        if rc != 0:
            raise RuntimeError(binding.mla_decode_status_string(rc))

    for i in range(max(2, args.warmup // 4)):
        call(i)
    torch.cuda.synchronize()
    n = max(4, args.steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    nbytes = OPROJ_WEIGHT_BYTES + rows * 16384 * 4 + rows * 7168 * 4
    out = {"us_per_call": us, "tokens": rows, "rotating_weight_sets": n_w, "calls": n,
           "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
           "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "launches": 3}
    if not args.no_cpu:
        from oracle import mla_oracle as orc
        w64 = orc.bf16_bits_to_f64(inp["w_o"])
        x64 = inp["x"].astype(np.float64)
        reps, t0 = 0, time.perf_counter()
        while reps < 2 or time.perf_counter() - t0 < 1.0:
            orc.output_project(x64, w64)
            reps += 1
        out["cpu_oracle_us_per_call"] = (time.perf_counter() - t0) / reps * 1e6
        del w64
    return out


def time_query_project(lib, dec, d, B, Sq, stream, args) -> dict:
    """The query side for the batch's new tokens (W_DQ and W_UQ, 97.5 MB of
    weights), HIP events around the calls; weight copies alternate past the
    Infinity Cache."""
    import torch
    from mla_latent_kv_amd import binding, synth
    rows = B * Sq
    inp = synth.make_query_inputs(B, Sq, seed=3000)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    hid = bf16(inp["hidden"])
    w0 = (dec.pack(bf16(inp["w_dq"])), dec.pack(bf16(inp["w_uq"])))
    n_w = max(2, math.ceil(MALL_BYTES / QPROJ_WEIGHT_BYTES) + 1)
    ws = [w0] + [(w0[0].clone(), w0[1].clone()) for _ in range(n_w - 1)]
    qn = torch.empty((B, Sq, 128, 128), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((B, Sq, 128, 64), dtype=torch.bfloat16, device="cuda")
    need = binding.mla_query_project_workspace_size(dec.ctx, B, Sq)
    wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
    cargs = [binding.MlaQueryArgs(hid.data_ptr(), a.data_ptr(), b.data_ptr(), d["seq_lens"].data_ptr(),
                                  qn.data_ptr(), qp.data_ptr(), B, Sq, 0.0) for a, b in ws]
    sh = ctypes.c_void_p(stream.cuda_stream)

    def call(i):
        rc = lib.mla_query_project(dec.ctx, ctypes.byref(cargs[i % n_w]), ctypes.c_void_p(wsp.data_ptr()),
                                   need, sh)
        if rc != 0:
            raise RuntimeError(binding.mla_decode_status_string(rc))

    for i in range(max(2, args.warmup // 2)):
        call(i)
    torch.cuda.synchronize()
    n = max(4, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    nbytes = QPROJ_WEIGHT_BYTES + rows * 7168 * 2 + rows * 128 * 192 * 2
    out = {"us_per_call": us, "tokens": rows, "rotating_weight_sets": n_w, "calls": n,
           "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
           "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "launches": 3}
    if not args.no_cpu:
        from oracle import mla_oracle as orc
        reps, t0 = 0, time.perf_counter()
        while reps < 2 or time.perf_counter() - t0 < 1.0:
            orc.query_batch(inp["hidden"], inp["w_dq"], inp["w_uq"], d["seq_lens"].cpu().numpy(), Sq)
            reps += 1
        out["cpu_oracle_us_per_call"] = (time.perf_counter() - t0) / reps * 1e6
    return out


def time_prologue(lib, dec, d, B, Sq, stream, args) -> dict:
    """The decode-step prologue (mla_project_new_tokens: the cache append and
    the query side of the new tokens in one call, W_DQ and [W_DKV; W_KR]
    streamed together), HIP events around the calls; weight copies rotate
    past the Infinity Cache."""
    import torch
    from mla_latent_kv_amd import binding, synth
    rows = B * Sq
    qin = synth.make_query_inputs(B, Sq, seed=3000)
    ain = synth.make_append_inputs(B, Sq, seed=1000)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    hid = bf16(qin["hidden"])
    w0 = (dec.pack(bf16(qin["w_dq"])), dec.pack(bf16(qin["w_uq"])),
          dec.pack(bf16(np.concatenate([ain["w_dkv"], ain["w_kr"]]))))
    wbytes = QPROJ_WEIGHT_BYTES + APPEND_WEIGHT_BYTES
    n_w = max(2, math.ceil(MALL_BYTES / wbytes) + 1)
    ws = [w0] + [tuple(w.clone() for w in w0) for _ in range(n_w - 1)]
    cache = d["kv_cache"].clone()
    qn = torch.empty((B, Sq, 128, 128), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((B, Sq, 128, 64), dtype=torch.bfloat16, device="cuda")
    need = binding.mla_project_new_tokens_workspace_size(dec.ctx, B, Sq)
    wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
    cargs = [binding.MlaPrologueArgs(hid.data_ptr(), a.data_ptr(), b.data_ptr(), c.data_ptr(), cache.data_ptr(),
                                     d["block_table"].data_ptr(), d["seq_lens"].data_ptr(), qn.data_ptr(),
                                     qp.data_ptr(), cache.shape[0], B, Sq, d["block_table"].shape[1], 0.0)
             for a, b, c in ws]
    sh = ctypes.c_void_p(stream.cuda_stream)

    def call(i):
        rc = lib.mla_project_new_tokens(dec.ctx, ctypes.byref(cargs[i % n_w]), ctypes.c_void_p(wsp.data_ptr()),
                                        need, sh)
        if rc != 0:
            raise RuntimeError(binding.mla_decode_status_string(rc))

    for i in range(max(2, args.warmup // 2)):
        call(i)
    torch.cuda.synchronize()
    n = max(4, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    nbytes = wbytes + rows * 7168 * 2 + rows * 128 * 192 * 2 + rows * 1152
    return {"us_per_call": us, "tokens": rows, "rotating_weight_sets": n_w, "calls": n,
            "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "launches": 3}


PREFILL_SPEC = ("prefill_b1_l4096", 1, 4096)   # one 4096-token prompt, every token a query


def time_naive(lib, dec, d, B, Sq, stream, args, absorb_ms) -> dict:
    """The naive path (mla_naive_run: per-head K and V materialised, then
    causal softmax attention). Prefill of one 4096-token prompt (all 128 heads,
    matrix-core bound: measured against the bf16/fp16 MFMA peak), and the same
    path on this decode workload beside the absorbed step (the absorb win).
    HIP events around the calls on the launch stream."""
    import torch
    from mla_latent_kv_amd import binding, device, synth
    name, pb, L = PREFILL_SPEC
    pbatch = synth.make_batch(synth.Spec(name, pb, L, ("fixed", L)), seed=5000)
    pd = device.upload(pbatch)
    w_uk, w_uv = dec.pack(pd["w_uk"]), dec.pack(pd["w_uv"])
    pws = torch.empty(binding.mla_naive_workspace_size(dec.ctx, pb, L), dtype=torch.uint8, device="cuda")
    pout = torch.empty((pb, L, 128, 128), dtype=torch.float32, device="cuda")

    def prefill():
        dec.naive(pd["q_nope"], pd["q_pe"], w_uk, w_uv, pd["kv_cache"], pd["block_table"], pd["seq_lens"],
                  L, out=pout, workspace=pws, stream=stream)

    def timed(fn, warm, n):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    us = timed(prefill, 2, 10)
    attn_flop = pb * sum(i + 1 for i in range(L)) * 128 * (192 + 128) * 2   # causal: row i sees i + 1 keys
    exp_flop = pb * L * 128 * (128 + 128) * 512 * 2                            # K_nope and V from c_KV
    tflops = (attn_flop + exp_flop) / (us * 1e-6) / 1e12
    out = {"prefill": {"workload": name, "prompt_tokens": pb * L, "us_per_call": us,
                       "prompt_tokens_per_s": pb * L / (us * 1e-6), "algorithmic_TFLOP": (attn_flop + exp_flop) / 1e12,
                       "TFLOPs": tflops, "mfma_frac": tflops / MFMA_PEAK_TFLOPS, "launches": 2,
                       "expanded_bytes_per_token": 128 * 256 * 2 + 128, "latent_bytes_per_token": 1152}}
    del pws, pout
    torch.cuda.empty_cache()
    # the decode workload on the naive path
    w_uk, w_uv = dec.pack(d["w_uk"]), dec.pack(d["w_uv"])
    dws = torch.empty(binding.mla_naive_workspace_size(dec.ctx, B, d["max_seq_len"]), dtype=torch.uint8,
                      device="cuda")
    dout = torch.empty((B, Sq, 128, 128), dtype=torch.float32, device="cuda")

    def naive_decode():
        dec.naive(d["q_nope"], d["q_pe"], w_uk, w_uv, d["kv_cache"], d["block_table"], d["seq_lens"],
                  d["max_seq_len"], out=dout, workspace=dws, stream=stream)

    nus = timed(naive_decode, 1, 3)
    out["decode_naive"] = {"us_per_call": nus, "absorb_us_per_step": absorb_ms * 1e3,
                           "absorb_speedup": nus / (absorb_ms * 1e3), "workspace_GB": dws.numel() / 1e9}
    del dws, dout
    torch.cuda.empty_cache()
    if not args.no_cpu:
        # the oracle's naive path on one head of the prompt, scaled to 128 heads
        from oracle import mla_oracle as orc
        t0 = time.perf_counter()
        orc.decode_batch(pbatch["q_nope"], pbatch["q_pe"], pbatch["w_uk"], pbatch["w_uv"], pbatch["cache"],
                         pbatch["block_table"], pbatch["seq_lens"], 64, sample=[(0, 0)])
        out["prefill"]["cpu_oracle_us_per_call"] = (time.perf_counter() - t0) * 1e6 * 128
        out["prefill"]["cpu_oracle_sample"] = "1 of 128 heads, scaled by 128"
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # the GPU's clock settles over the first ~300 steps after idle (122 -> 72 us
    # per step); 1000 warm-up steps (~75 ms) put the timed steps past that ramp
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", type=int, default=1, help="workload index (0-4)")
    ap.add_argument("--sets", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-append", action="store_true",
                    help="skip the timings of the cache-append producer, the query side, the "
                         "output projection and the naive path")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested). Sequences shard across GPUs with no exchange; run one process "
              "per GPU instead.", file=sys.stderr)
        return 2

    import torch
    from mla_latent_kv_amd import binding, device, synth, workloads
    if not os.path.exists(binding.LIB_PATH):
        from mla_latent_kv_amd import build
        build.build()
    lib = binding.load_library()
    hip = _hip()

    spec = synth.CONFIGS[args.config]
    batch = synth.make_batch(spec, seed=args.config)
    work = workloads.algorithmic_work(batch["seq_lens"], spec.q_tokens)
    d = device.upload(batch)
    n_sets = args.sets or max(1, math.ceil(3 * MALL_BYTES / work["total_bytes"]))
    sets = [d]
    for _ in range(n_sets - 1):
        sets.append({k: (v.clone() if isinstance(v, torch.Tensor) and k not in
                         ("block_table", "seq_lens") else v) for k, v in d.items()})
    B, Sq = spec.batch, spec.q_tokens
    dec = binding.MLADecoder(0, max_q_tokens=2)
    ws_bytes = dec.workspace_size(B, Sq, d["max_seq_len"])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, Sq, 128, 128), dtype=torch.float32, device="cuda") for _ in sets]
    cargs = []
    for s, o in zip(sets, outs):
        cargs.append(binding.MlaDecodeArgs(
            s["q_nope"].data_ptr(), s["q_pe"].data_ptr(), s["w_uk"].data_ptr(),
            s["w_uv"].data_ptr(), s["kv_cache"].data_ptr(), s["block_table"].data_ptr(),
            s["seq_lens"].data_ptr(), o.data_ptr(), s["kv_cache"].shape[0], B, Sq,
            s["block_table"].shape[1], d["max_seq_len"]))
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    wsp = ctypes.c_void_p(ws.data_ptr())

    def step(i):
        rc = lib.mla_decode_run(dec.ctx, ctypes.byref(cargs[i % n_sets]), wsp, ws_bytes, sh)
        if rc != 0:
            raise RuntimeError(binding.mla_decode_status_string(rc))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # warm figure: one input set, so the cache may sit in the Infinity Cache
    for i in range(5):
        lib.mla_decode_run(dec.ctx, ctypes.byref(cargs[0]), wsp, ws_bytes, sh)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        lib.mla_decode_run(dec.ctx, ctypes.byref(cargs[0]), wsp, ws_bytes, sh)
    e1.record(stream)
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / args.steps

    # per-kernel durations (events recorded by the library between launches)
    n_prof = min(args.steps, 100)
    evs = _events(hip, 5 * n_prof)
    ev_arr = [(ctypes.c_void_p * 5)(*[evs[5 * i + j].value for j in range(5)]) for i in range(n_prof)]
    for i in range(n_prof):
        rc = lib.mla_decode_run_profiled(dec.ctx, ctypes.byref(cargs[i % n_sets]), wsp, ws_bytes,
                                         sh, ctypes.cast(ev_arr[i], ctypes.POINTER(ctypes.c_void_p)))
        if rc != 0:
            raise RuntimeError(binding.mla_decode_status_string(rc))
    torch.cuda.synchronize()
    # stage boundaries: 1 -> 2 plan + absorb (prep), 2 -> 3 attention, 3 -> 4 merge + W_UV
    names = {1: "prep", 2: "attention", 3: "merge"}
    kern_ms = {n: 0.0 for n in names.values()}
    step_ms = []
    for i in range(n_prof):
        for j, n in names.items():
            kern_ms[n] += _elapsed(hip, evs[5 * i + j], evs[5 * i + j + 1]) / n_prof
        step_ms.append(_elapsed(hip, evs[5 * i], evs[5 * i + 4]))
    step_pct = {f"p{q}": float(np.percentile(step_ms, q)) for q in (10, 50, 90)}
    for e in evs:
        hip.hipEventDestroy(e)

    attn_s = kern_ms["attention"] * 1e-3
    achieved = work["cache_bytes"] / attn_s / 1e9
    step_s = ms * 1e-3
    result = {
        "metric": METRIC,
        "value": B * Sq / step_s,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16/bf16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "q_tokens": Sq,
                   "seq_len": int(batch["seq_lens"].max()), "cached_tokens": int(batch["seq_lens"].sum()),
                   "heads": 128, "latent": 512, "rope": 64, "block": 64, "paged": spec.paged,
                   "rotating_input_sets": n_sets},
        "latent_cache_TBps": work["cache_bytes"] / step_s / 1e12,
        "total_TBps": work["total_bytes"] / step_s / 1e12,
        "mfma_TFLOPs": work["flops"] / step_s / 1e12,
        "warm_ms_per_step": warm_ms,
        "step_ms_percentiles": dict(step_pct, steps=n_prof,
                                    note="first to last launch of one step, events between launches"),
        "kernel_ms": kern_ms,
        "roofline": {
            "bound": "hbm",
            "kernel": "attention pass (mla::attn_kernel)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": attn_traffic(spec.name),
            "algorithmic_bytes_per_launch": work["cache_bytes"],
            "mfma_TFLOPs": work["attn_flops"] / attn_s / 1e12,
            "mfma_frac": work["attn_flops"] / attn_s / 1e12 / MFMA_PEAK_TFLOPS,
        },
        "whole_step_roofline_frac": work["total_bytes"] / step_s / 1e9 / HBM_PEAK_GBS,
    }
    if not args.no_append:
        result["cache_append"] = time_cache_append(lib, dec, d, B, Sq, stream, args)
        result["query_project"] = time_query_project(lib, dec, d, B, Sq, stream, args)
        result["prologue"] = time_prologue(lib, dec, d, B, Sq, stream, args)
        result["prologue"]["separate_calls_us"] = (result["cache_append"]["us_per_call"]
                                                   + result["query_project"]["us_per_call"])
        result["output_project"] = time_output_project(lib, dec, B, Sq, stream, args)
        result["naive"] = time_naive(lib, dec, d, B, Sq, stream, args, ms)
    result["copy_bandwidth"] = copy_bandwidth()
    rc = 0
    if not args.no_cpu:
        # the output of the last timed step (its input set), read back after
        # every timed region has ended
        last = outs[(args.steps - 1) % n_sets].cpu().numpy()
        cb = cpu_baseline(batch, args.cpu_budget, batch["seq_lens"].shape[0], gpu_out=last)
        result["output_check"] = cb.pop("check")
        result["cpu_baseline"] = cb
        if not result["output_check"]["pass"]:
            rc = 3
    print(json.dumps(result), flush=True)
    dec.close()
    return rc


if __name__ == "__main__":
    sys.exit(main())
