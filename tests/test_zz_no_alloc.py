"""pa_decode_static (no allocation: partials in the library's static device
array) against pa_decode (caller's workspace), through the C ABI.

Both run the same kernels in the same order, so the outputs must agree bit
for bit; each call is also within the parity tolerance of the oracle (bf16:
max abs 2e-2, rel L2 1e-2, lse 1e-3).  Calls follow each other on one device,
so the static array keeps the previous call's partials and counters: a call
with fewer rows, then more rows again, must still find zeroed counters.
"""
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

MHA = dict(kind="mha", dtype="bf16", num_q_heads=16, num_kv_heads=16, head_dim=128,
           block_size=16, num_blocks=120)
GQA = dict(kind="mha", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
           block_size=16, num_blocks=300)
LENS = [300, 33, 257, 160, 1, 77, 200, 16]


def _shape(inp):
    return pa.make_shape(batch=inp.batch, num_q_heads=inp.num_q_heads,
                         num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                         head_dim_v=inp.head_dim_v, block_size=inp.block_size,
                         max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
                         max_context_len=inp.max_context_len, scale=inp.scale,
                         dtype=torch.bfloat16)


def _static(inp, t, S):
    shape = _shape(inp)
    out = torch.empty(inp.batch, inp.num_q_heads, inp.head_dim_v, dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.empty(inp.batch, inp.num_q_heads, dtype=torch.float32, device="cuda")
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    st = _lib.load().pa_decode_static(
        ctypes.byref(shape), P(t["q"]), P(t["k_cache"]), P(t["v_cache"]), P(t["block_table"]),
        P(t["context_lens"]), S, P(out), P(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.PA_OK, _lib.status_string(st)
    return out, lse


def _check(inp, t, S, what):
    o1, l1 = _static(inp, t, S)
    o2, l2 = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                       max_context_len=inp.max_context_len, scale=inp.scale, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{what}: differs from pa_decode"
    ref_out, ref_lse = oracle.decode_inputs(inp)
    o = from_device(o1)
    err = float(np.abs(o - ref_out).max())
    rel = float(np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out))
    lerr = float(np.abs(l1.cpu().numpy() - ref_lse).max())
    assert err <= 2e-2 and rel <= 1e-2 and lerr <= 1e-3, (what, err, rel, lerr)


# (spec, batch, num_splits): the in-kernel merge (counters in the array) and the
# reduction launch, larger then smaller inputs, then larger again
SEQUENCE = [(MHA, 8, 3), (MHA, 2, 3), (MHA, 8, 4), (GQA, 8, 0), (MHA, 1, 2), (GQA, 3, 0),
            (MHA, 8, 3)]


def test_static_matches_decode_call_after_call():
    for i, (spec, B, S) in enumerate(SEQUENCE):
        inp = make_paged_inputs(name="static", seed=700 + i, batch=B, context_lens=LENS[:B],
                                **spec)
        t = to_device(inp, "cuda")
        print(f"static call {i}: B={B} Hq={inp.num_q_heads} S={S} "
              f"launches={pa.decode_launches(_shape(inp), S)}", flush=True)
        _check(inp, t, S, f"call {i}")


def test_static_rejects_partials_beyond_its_array():
    # 64 sequences x 64 heads x 64 splits x 129 floats: 129 MiB of partials
    inp = make_paged_inputs(name="big", seed=710, values=False, kind="mha", dtype="bf16",
                            batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
                            block_size=16, context_lens=[4096] * 64, num_blocks=20000)
    shape = _shape(inp)
    assert pa.workspace_size(shape, 64) > 64 << 20
    F = ctypes.c_void_p(0x1000)   # never dereferenced: refused before any launch
    st = _lib.load().pa_decode_static(ctypes.byref(shape), F, F, F, F, F, 64, F, F, None)
    assert st == _lib.PA_ERR_SCRATCH
