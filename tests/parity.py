"""Helpers shared by the GPU parity tests: run the HIP library on a synthetic
batch and compare with the fp64 oracle under the stated tolerance:
max|err| <= 1e-2 * max|o_ref| and sum|err| / sum|o_ref| <= 2e-3."""

from __future__ import annotations

import sys

import numpy as np

MAX_REL = 1e-2
MEAN_REL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(batch: dict, decoder=None, split_target: int = 0, out=None):
    import torch
    from mla_latent_kv_amd import binding, device
    d = device.upload(batch)
    dec = decoder or binding.MLADecoder(0, max_q_tokens=2, split_target=split_target)
    o = dec(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"],
            d["seq_lens"], d["max_seq_len"], out=out)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def oracle(batch: dict, sample=None, path="naive"):
    from oracle import mla_oracle as orc
    return orc.decode_batch(batch["q_nope"], batch["q_pe"], batch["w_uk"], batch["w_uv"],
                            batch["cache"], batch["block_table"], batch["seq_lens"],
                            batch["block_size"], sample=sample, path=path)


def metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    m = np.isfinite(ref)
    g, r = got[m], ref[m]
    err = np.abs(g - r)
    return {
        "n": int(m.sum()),
        "max_rel": float(err.max() / np.abs(r).max()),
        "mean_rel": float(err.sum() / np.abs(r).sum()),
        "l2_rel": float(np.sqrt((err ** 2).sum() / (r ** 2).sum())),
        "finite": bool(np.isfinite(g).all()),
    }


def assert_parity(got, ref, what=""):
    mt = metrics(got, ref)
    say(f"parity {what}: {mt}")
    assert mt["finite"], f"{what}: non-finite output"
    assert mt["max_rel"] <= MAX_REL, f"{what}: max rel {mt['max_rel']:.3e}"
    assert mt["mean_rel"] <= MEAN_REL, f"{what}: mean rel {mt['mean_rel']:.3e}"
    return mt
