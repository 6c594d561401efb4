"""Paged KV append on the GPU: the appended cache equals the cache that held
the token from the start (byte for byte), and decoding it matches the oracle.

Each case draws a workload with context n + 1, removes every sequence's last
token (its slot is NaN in the device pool, as every slot past a context is),
appends it back through the C ABI, and compares.  Positions include a page's
first slot (a new page), its last slot and position 0.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import decode_attention_paged_amd as pa
from workloads import make_paged_inputs
from workloads.device import from_device, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "mha_f32": dict(kind="mha", dtype="f32", batch=4, num_q_heads=8, num_kv_heads=8, head_dim=64,
                    block_size=16, context_lens=[17, 16, 1, 40], num_blocks=20),
    "gqa_bf16": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=2,
                     head_dim=128, block_size=16, context_lens=[33, 1, 300, 16], num_blocks=40),
    "gqa_fp8": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=2,
                    head_dim=128, block_size=16, context_lens=[33, 1, 300, 16], num_blocks=40,
                    kv_dtype="fp8", k_scale=0.05, v_scale=0.3),
    # 32-token pages with 64-dim heads (the grouped-query kernel decodes them), and 256-dim
    # heads on 32-token pages (the VALU kernel)
    "gqa_bf16_d64_bs32": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=16, num_kv_heads=4,
                              head_dim=64, block_size=32, context_lens=[31, 32, 100],
                              num_blocks=20),
    "mha_bf16_d256_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                               head_dim=256, block_size=32, context_lens=[63, 1], num_blocks=10),
    "mla_bf16": dict(kind="mla", dtype="bf16", batch=3, num_q_heads=16, num_kv_heads=1,
                     head_dim=576, head_dim_v=512, block_size=64, context_lens=[65, 64, 1],
                     num_blocks=12, scale=192 ** -0.5),
    "mla_fp8": dict(kind="mla", dtype="bf16", batch=3, num_q_heads=128, num_kv_heads=1,
                    head_dim=576, head_dim_v=512, block_size=64, context_lens=[65, 64, 1],
                    num_blocks=12, scale=192 ** -0.5, kv_dtype="fp8", k_scale=0.05,
                    v_scale=0.06),
    # token-index lists (one-token pages), 32 heads: the role-split kernel
    "mla_fp8_bs1": dict(kind="mla", dtype="bf16", batch=3, num_q_heads=32, num_kv_heads=1,
                        head_dim=576, head_dim_v=512, block_size=1, context_lens=[65, 64, 1],
                        num_blocks=200, scale=192 ** -0.5, kv_dtype="fp8", k_scale=0.05,
                        v_scale=0.06),
}


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Raw element bits (NaN-safe equality)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _poison(t: torch.Tensor, idx):
    """Set t[idx] to NaN (the FP8 NaN code for FP8 caches)."""
    if t.dtype == torch.float8_e4m3fn:
        t.view(torch.uint8)[idx] = 0x7F
    else:
        t[idx] = float("nan")


def _rows(inp, b, n):
    """The host rows of sequence b's token n, as they sit in the compact pages."""
    bt = inp.compact_block_table()
    page, slot = bt[b, n // inp.block_size], n % inp.block_size
    if inp.kind == "mla":
        return inp.c_pages[page, slot, :].copy(), None
    return inp.k_pages[page, :, slot, :].copy(), inp.v_pages[page, :, :, slot].copy()


def _dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda().view(
            torch.float8_e4m3fn)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_then_decode(name):
    spec = CASES[name]
    full = make_paged_inputs(name=name, seed=61, **spec)
    before = make_paged_inputs(name=name, seed=61, **spec)
    before.context_lens = full.context_lens - 1
    # what the device holds before the append: the token's slot is poisoned
    t_full = to_device(full, "cuda", poison=True)
    t_before = to_device(full, "cuda", poison=True)
    t_before["context_lens"] = torch.from_numpy(before.context_lens.astype(np.int32)).cuda()
    rows = [_rows(full, b, int(before.context_lens[b])) for b in range(full.batch)]
    for b in range(full.batch):
        n = int(before.context_lens[b])
        page = int(full.block_table[b, n // full.block_size])
        slot = n % full.block_size
        if full.kind == "mla":
            _poison(t_before["kv_cache"], (page, slot, slice(None)))
        else:
            _poison(t_before["k_cache"], (page, slice(None), slot, slice(None)))
            _poison(t_before["v_cache"], (page, slice(None), slice(None), slot))
    if full.kind == "mla":
        c_new = _dev(np.stack([r[0] for r in rows]), full.kv_dtype or full.dtype)
        pa.append_latent(c_new, t_before["kv_cache"], t_before["block_table"],
                         t_before["context_lens"])
        torch.cuda.synchronize()
        assert torch.equal(_bits(t_before["kv_cache"]), _bits(t_full["kv_cache"]))
    else:
        kvd = full.kv_dtype or full.dtype
        k_new = _dev(np.stack([r[0] for r in rows]), kvd)
        v_new = _dev(np.stack([r[1] for r in rows]), kvd)
        pa.append_kv(k_new, v_new, t_before["k_cache"], t_before["v_cache"],
                     t_before["block_table"], t_before["context_lens"])
        torch.cuda.synchronize()
        assert torch.equal(_bits(t_before["k_cache"]), _bits(t_full["k_cache"]))
        assert torch.equal(_bits(t_before["v_cache"]), _bits(t_full["v_cache"]))
    # the caller advances the lengths, then decodes the new token
    t_before["context_lens"] += 1
    ref_out, ref_lse = oracle.decode_inputs(full)
    fp8 = dict(k_scale=full.k_scale, v_scale=full.v_scale) if full.kv_dtype == "fp8" else {}
    if full.kind == "mla":
        out, lse = pa.decode_mla(t_before["q"], t_before["kv_cache"], t_before["block_table"],
                                 t_before["context_lens"], scale=full.scale, num_splits=2, **fp8)
    else:
        out, lse = pa.decode(t_before["q"], t_before["k_cache"], t_before["v_cache"],
                             t_before["block_table"], t_before["context_lens"],
                             scale=full.scale, num_splits=2, **fp8)
    torch.cuda.synchronize()
    tol = 1e-5 if full.dtype == "f32" else 2e-2
    assert np.abs(from_device(out) - ref_out).max() <= tol
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= (1e-5 if full.dtype == "f32" else 1e-3)


def test_append_outside_the_table_writes_nothing():
    spec = CASES["gqa_bf16"]
    inp = make_paged_inputs(name="oob", seed=62, **spec)
    t = to_device(inp, "cuda", poison=True)
    k0, v0 = t["k_cache"].clone(), t["v_cache"].clone()
    full_len = inp.block_table.shape[1] * inp.block_size
    pos = torch.tensor([full_len, -1, full_len + 100, -7], dtype=torch.int32, device="cuda")
    k_new = torch.ones((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    v_new = torch.ones((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    pa.append_kv(k_new, v_new, t["k_cache"], t["v_cache"], t["block_table"], pos)
    torch.cuda.synchronize()
    assert torch.equal(_bits(t["k_cache"]), _bits(k0))
    assert torch.equal(_bits(t["v_cache"]), _bits(v0))
