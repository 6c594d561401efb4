"""The in-kernel split merge and workspace reuse, on the GPU.

The last workgroup of each (sequence, head unit) merges that unit's split
partials, which other workgroups (on any XCD) wrote moments before: a wrong
release/acquire order shows up as a merge of stale partials.  Every call here
uses fresh query rows on one shared workspace (so the previous call's
partials are still in it) and is compared with the float64 oracle; the loop
stops at the first mismatch.

Also: one workspace reused across split counts and across row counts.
Tolerances as in the parity tests (bf16: max abs 2e-2, rel L2 1e-2, lse 1e-3).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import decode_attention_paged_amd as pa
from workloads import f32_to_bf16_bits, make_paged_inputs
from workloads.device import from_device, to_device

pytestmark = pytest.mark.gpu

# MHA: one head per unit, so S x 129 x 4 B <= 4 KiB merges in-kernel for S <= 7.
# GQA with 2 heads per KV head: 2 x S x 129 x 4 B <= 4 KiB for S <= 3.
FUSED = {
    "mha": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=16,
                head_dim=128, block_size=16, context_lens=[300, 33, 257, 160], num_blocks=64),
    "gqa_g2": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=8,
                   head_dim=128, block_size=16, context_lens=[300, 33, 257, 160], num_blocks=64),
}
CALLS = 200


def _shape(inp):
    return pa.make_shape(batch=inp.batch, num_q_heads=inp.num_q_heads,
                         num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                         head_dim_v=inp.head_dim_v, block_size=inp.block_size,
                         max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
                         max_context_len=inp.max_context_len, scale=inp.scale,
                         dtype=torch.bfloat16)


def _check(inp, out, lse, ref_out, ref_lse, what):
    o = from_device(out)
    l = lse.detach().cpu().numpy().astype(np.float64)
    err = float(np.abs(o - ref_out).max())
    rel = float(np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out))
    lerr = float(np.abs(l - ref_lse).max())
    assert err <= 2e-2 and rel <= 1e-2 and lerr <= 1e-3, \
        f"{what}: max_abs={err:.3e} rel_l2={rel:.3e} lse_err={lerr:.3e}"
    return err


@pytest.mark.parametrize("S", [2, 3])
@pytest.mark.parametrize("name", sorted(FUSED))
def test_fused_merge_back_to_back(name, S):
    inp = make_paged_inputs(name=name, seed=500 + S, **FUSED[name])
    shape = _shape(inp)
    assert pa.decode_launches(shape, S) == 1, "this shape must take the in-kernel merge"
    t = to_device(inp, "cuda")
    ws = torch.zeros(pa.workspace_size(shape, S), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(600 + S)
    worst = 0.0
    print(f"fused {name} S={S}: {CALLS} calls", flush=True)
    for call in range(CALLS):
        # fresh query rows each call: stale partials from the call before differ
        inp.q = f32_to_bf16_bits(rng.standard_normal(inp.q.shape, dtype=np.float32) *
                                 np.float32(1 + call % 5))
        t["q"].copy_(torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16))
        out, lse = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["context_lens"], max_context_len=inp.max_context_len,
                             scale=inp.scale, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_inputs(inp)
        worst = max(worst, _check(inp, out, lse, ref_out, ref_lse, f"{name} S={S} call {call}"))
    print(f"fused {name} S={S}: worst max_abs {worst:.3e}", flush=True)
    # every completed call leaves the arrival counters at zero
    rows = inp.batch * inp.num_q_heads
    assert int(ws[:4 * rows].view(torch.int32).abs().sum().item()) == 0


def test_workspace_reuse_across_split_counts():
    """The arrival counters sit at the start of the workspace whatever S is, so
    one workspace serves calls with S = 16, 4, 7, 4 (fused and two-launch
    alike) without re-initialisation."""
    inp = make_paged_inputs(name="reuse", seed=510, **FUSED["mha"])
    shape = _shape(inp)
    t = to_device(inp, "cuda")
    ref_out, ref_lse = oracle.decode_inputs(inp)
    size = max(pa.workspace_size(shape, S) for S in (16, 4, 7))
    ws = torch.full((size,), 0xAB, dtype=torch.uint8, device="cuda")
    pa.workspace_init(shape, ws, 16)
    launches = []
    for S in (16, 4, 7, 4, 16, 2):
        launches.append(pa.decode_launches(shape, S))
        out, lse = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["context_lens"], max_context_len=inp.max_context_len,
                             scale=inp.scale, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        _check(inp, out, lse, ref_out, ref_lse, f"reuse S={S}")
    assert 1 in launches and 2 in launches, launches


def test_workspace_reuse_across_row_counts():
    """A smaller batch's partials lie where a larger batch keeps counters (8
    sequences x 16 heads: 512 bytes of counters; 1 sequence: its partials
    start at byte 256): the binding re-initialises the counters when a
    workspace moves to more rows."""
    lens = [300, 33, 257, 160, 1, 77, 200, 16]
    big = dict(FUSED["mha"], batch=8, context_lens=lens, num_blocks=100)
    ws = torch.zeros(pa.workspace_size(_shape(make_paged_inputs(name="rows", seed=0, values=False,
                                                                **big)), 7),
                     dtype=torch.uint8, device="cuda")
    for it, B in enumerate((8, 1, 8, 2, 8)):
        inp = make_paged_inputs(name="rows", seed=520 + it, **dict(big, batch=B,
                                                                   context_lens=lens[:B]))
        shape = _shape(inp)
        assert pa.decode_launches(shape, 3) == 1
        t = to_device(inp, "cuda")
        out, lse = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["context_lens"], max_context_len=inp.max_context_len,
                             scale=inp.scale, num_splits=3, workspace=ws)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_inputs(inp)
        _check(inp, out, lse, ref_out, ref_lse, f"rows B={B}")
