"""Place a host workload into device memory (torch tensors).

The device pool has ``num_blocks`` pages; the workload's compact pages are
scattered to their physical ids.  With ``poison`` every other page is NaN, so
a kernel that reads a page or slot it should not read produces NaN.
"""

from __future__ import annotations

import numpy as np
import torch


def _tensor(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device).view(
            torch.float8_e4m3fn)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "fp8":
        return torch.float8_e4m3fn
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _pool(compact: np.ndarray, page_ids: np.ndarray, num_blocks: int, dtype: str, device,
          poison: bool) -> torch.Tensor:
    shape = (num_blocks,) + tuple(compact.shape[1:])
    td = torch_dtype(dtype)
    if dtype == "fp8":                                 # bytes; NaN code 0x7F
        pool = torch.empty(shape, dtype=torch.uint8, device=device)
        if poison:
            pool.fill_(0x7F)
    else:
        pool = (torch.full(shape, float("nan"), dtype=td, device=device) if poison
                else torch.empty(shape, dtype=td, device=device))
    idx = torch.from_numpy(page_ids.astype(np.int64)).to(device)
    # upload in slices so the host-side staging copy stays bounded
    step = max(1, (1 << 28) // max(1, int(np.prod(compact.shape[1:])) * compact.itemsize))
    for lo in range(0, compact.shape[0], step):
        hi = min(compact.shape[0], lo + step)
        part = _tensor(compact[lo:hi], dtype, device)
        pool.index_copy_(0, idx[lo:hi], part.view(torch.uint8) if dtype == "fp8" else part)
    return pool.view(td) if dtype == "fp8" else pool


def to_device(inp, device="cuda", poison: bool = True) -> dict:
    """Tensors for one decode call: q, caches, block_table, context_lens."""
    t = {
        "q": _tensor(inp.q, inp.dtype, device),
        "block_table": torch.from_numpy(inp.block_table.astype(np.int32)).to(device),
        "context_lens": torch.from_numpy(inp.context_lens.astype(np.int32)).to(device),
    }
    if inp.kind == "mla":
        t["kv_cache"] = _pool(inp.c_pages, inp.page_ids, inp.num_blocks, inp.kv_dtype or inp.dtype,
                              device, poison)
    else:
        kvd = inp.kv_dtype or inp.dtype
        t["k_cache"] = _pool(inp.k_pages, inp.page_ids, inp.num_blocks, kvd, device, poison)
        t["v_cache"] = _pool(inp.v_pages, inp.page_ids, inp.num_blocks, kvd, device, poison)
    return t


def from_device(x: torch.Tensor) -> np.ndarray:
    """Device tensor to a float64 numpy array (bf16 widened exactly)."""
    return x.detach().to("cpu", torch.float64).numpy()
