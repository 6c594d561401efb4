"""Decode calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every kernel of a call is a plain launch on the caller's stream: no memset,
no allocation and no host synchronisation inside the call when the buffers and
max_context_len are given.  A captured call must therefore replay to the
eager call's result.  Each case captures one call, then replays it three
times with eager work between the replays: torch writes new queries on the
same stream, and the process synchronises.  Every replay is compared bit for
bit with an eager call on the same inputs, and the first one with the oracle.
The cases cover each launch pattern:
- the unit-order launch before the grouped-query kernel (ragged batch, 3 launches);
- the in-kernel merge with its arrival counters (1 launch);
- the latent kernel with its reduction, bf16 and FP8 latent caches (2 launches);
- the entry point without a workspace.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import decode_attention_paged_amd as pa
from decode_attention_paged_amd import _lib
from workloads import make_paged_inputs
from workloads.device import from_device, to_device

pytestmark = pytest.mark.gpu

MLA = dict(kind="mla", dtype="bf16", num_q_heads=128, num_kv_heads=1, head_dim=576,
           head_dim_v=512, block_size=64, scale=192 ** -0.5)
CASES = {
    # (spec, split count, launches per call)
    "ragged_gqa_unit_order": (dict(kind="mha", dtype="bf16", batch=7, num_q_heads=16,
                                   num_kv_heads=2, head_dim=128, block_size=16,
                                   context_lens=[1, 17, 300, 1600, 0, 1024, 3200],
                                   num_blocks=600), 3, 3),
    "mha_fused_merge": (dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=16,
                             head_dim=128, block_size=16, context_lens=[300, 33, 257, 160],
                             num_blocks=60), 4, 1),
    "mla_bf16": (dict(MLA, batch=2, context_lens=[200, 1000], num_blocks=24), 3, 2),
    "mla_fp8": (dict(MLA, batch=2, context_lens=[200, 1000], num_blocks=24, kv_dtype="fp8",
                     k_scale=0.037, v_scale=0.045), 3, 2),
    "static_ragged_gqa": (dict(kind="mha", dtype="bf16", batch=7, num_q_heads=16, num_kv_heads=2,
                               head_dim=128, block_size=16,
                               context_lens=[1, 17, 300, 1600, 0, 1024, 3200],
                               num_blocks=600), 3, 3),
}


def _shape(inp):
    return pa.make_shape(
        batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
        head_dim=inp.head_dim, head_dim_v=inp.head_dim_v, block_size=inp.block_size,
        max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
        max_context_len=inp.max_context_len, scale=inp.scale, dtype=torch.bfloat16,
        q_len=inp.q_len, kv_dtype=_lib.PA_FP8_E4M3 if inp.kv_dtype == "fp8" else 0,
        k_scale=inp.k_scale, v_scale=inp.v_scale)


def _caller(name, inp, t, S, out, lse, ws):
    """One decode call writing into out/lse, every buffer given (capturable)."""
    fp8 = dict(k_scale=inp.k_scale, v_scale=inp.v_scale) if inp.kv_dtype == "fp8" else {}
    if inp.kind == "mla":
        return lambda: pa.decode_mla(t["q"], t["kv_cache"], t["block_table"], t["context_lens"],
                                     max_context_len=inp.max_context_len, scale=inp.scale,
                                     head_dim_v=inp.head_dim_v, num_splits=S, out=out, lse=lse,
                                     workspace=ws, **fp8)
    if name.startswith("static"):
        shape = _shape(inp)
        P = lambda x: ctypes.c_void_p(x.data_ptr())

        def call():
            st = _lib.load().pa_decode_static(
                ctypes.byref(shape), P(t["q"]), P(t["k_cache"]), P(t["v_cache"]),
                P(t["block_table"]), P(t["context_lens"]), S, P(out), P(lse),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert st == _lib.PA_OK, _lib.status_string(st)
        return call
    return lambda: pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["context_lens"], max_context_len=inp.max_context_len,
                             scale=inp.scale, num_splits=S, out=out, lse=lse, workspace=ws, **fp8)


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    spec, S, launches = CASES[name]
    print(f"graph {name}: S={S}", flush=True)
    inp = make_paged_inputs(seed=31, **spec)
    t = to_device(inp, "cuda", poison=True)
    mla = inp.kind == "mla"
    shape = _shape(inp)
    assert pa.decode_launches(shape, S, mla) == launches
    rows = (inp.batch, inp.num_q_heads)
    dev = dict(device="cuda")
    out = torch.empty(rows + (inp.head_dim_v,), dtype=torch.bfloat16, **dev)
    lse = torch.empty(rows, dtype=torch.float32, **dev)
    ws = torch.zeros(max(pa.workspace_size(shape, S, mla), 256), dtype=torch.uint8, **dev)
    call = _caller(name, inp, t, S, out, lse, ws)
    # queries for the replays: the drawn ones first, then two more sets
    gen = torch.Generator(device="cuda").manual_seed(7)
    qs = [t["q"].clone()] + [torch.randn(t["q"].shape, generator=gen, **dev).to(torch.bfloat16)
                             for _ in range(2)]
    call()                                            # eager first: one-time set-up outside
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_inputs(inp)
    for rep, q in enumerate(qs):
        print(f"graph {name}: replay {rep}", flush=True)
        t["q"].copy_(q)                               # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        call()                                        # the eager call on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_o, out), f"replay {rep}: outputs differ from the eager call"
        assert torch.equal(got_l, lse), f"replay {rep}: lse differs from the eager call"
        if rep == 0:
            o = from_device(got_o)
            assert np.abs(o - ref_out).max() <= 2e-2
            gl = got_l.cpu().numpy().astype(np.float64)
            fin = np.isfinite(ref_lse)
            assert np.array_equal(gl[~fin], ref_lse[~fin])
            assert np.abs(gl[fin] - ref_lse[fin]).max() <= 1e-3
