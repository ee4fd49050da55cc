"""Copy a synthetic :class:`workloads.synth.Batch` to device tensors (plumbing only)."""

from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def storage_to_torch(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def torch_to_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.uint16).numpy()
    return t.numpy()


def to_device(b, device="cuda") -> SimpleNamespace:
    d = SimpleNamespace()
    d.query = storage_to_torch(b.query, b.dtype, device)
    d.k_pool = storage_to_torch(b.k_pool, b.dtype, device)
    d.v_pool = storage_to_torch(b.v_pool, b.dtype, device)
    d.block_tables = torch.from_numpy(np.ascontiguousarray(b.block_tables, dtype=np.int32)).to(device)
    d.context_lens = torch.from_numpy(np.ascontiguousarray(b.context_lens, dtype=np.int32)).to(device)
    d.new_key = d.new_value = d.slot_mapping = d.block_mapping = None
    if b.new_key is not None:
        d.new_key = storage_to_torch(b.new_key, b.dtype, device)
        d.new_value = storage_to_torch(b.new_value, b.dtype, device)
        d.slot_mapping = torch.from_numpy(np.ascontiguousarray(b.slot_mapping, dtype=np.int64)).to(device)
    if b.block_mapping is not None:
        d.block_mapping = torch.from_numpy(np.ascontiguousarray(b.block_mapping, dtype=np.int32)).to(device)
    return d
