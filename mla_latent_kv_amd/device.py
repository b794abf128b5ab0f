"""Move a synthetic batch (uint16 bf16 bit arrays from ``synth``) to a GPU."""

from __future__ import annotations

import numpy as np


def upload(batch: dict, device="cuda"):
    """Return a dict of torch tensors on `device` holding the same bytes."""
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    return {
        "q_nope": bf16(batch["q_nope"]),
        "q_pe": bf16(batch["q_pe"]),
        "w_uk": bf16(batch["w_uk"]),
        "w_uv": bf16(batch["w_uv"]),
        "kv_cache": bf16(batch["cache"]),
        "block_table": torch.from_numpy(np.ascontiguousarray(batch["block_table"])).to(device),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(batch["seq_lens"])).to(device),
        "max_seq_len": int(batch["max_seq_len"]),
    }
