"""Copy a synthetic :class:`~synthetic.Case` into torch tensors (no arithmetic).

Stored values move bit for bit: float32 and float16 arrays keep their type,
bfloat16 patterns are reinterpreted as ``torch.bfloat16``.
"""

from __future__ import annotations

import numpy as np


def as_tensor(x: np.ndarray, dtype: str, device):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


def to_device(case, device="cuda"):
    """Dict of device tensors: q, k, v (or None), seq_lens, block_table (or None)."""
    import torch

    return {
        "q": as_tensor(case.q, case.q_dtype, device),
        "k": as_tensor(case.k, case.kv_dtype, device),
        "v": None if case.v is None else as_tensor(case.v, case.kv_dtype, device),
        "seq_lens": torch.from_numpy(case.seq_lens.astype(np.int32)).to(device),
        "block_table": None if case.block_table is None
        else torch.from_numpy(case.block_table.astype(np.int32)).to(device),
    }
