"""HIP path against the hand-derived closed forms of ``golden/closed_forms.json``.

Every case runs through the C ABI (the ctypes binding) at the heuristic split
count and at 1, 2 and 3 splits (more splits than pages: empty splits), with
every pool element the case does not set poisoned with NaN.  Bars: float32
outputs and lse within 1e-5; bfloat16 outputs within one bfloat16 ulp of the
exact value (every expected value is a bfloat16 number), lse within 1e-3.
"""

import numpy as np
import pytest
import torch

import decode_attention_paged_amd as pa
import golden_cases

pytestmark = pytest.mark.gpu

CASES = golden_cases.cases()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "fp8":
        return torch.from_numpy(a.astype(np.uint8)).cuda().view(torch.float8_e4m3fn)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32)).cuda()


@pytest.mark.parametrize("num_splits", [0, 1, 2, 3])
@pytest.mark.parametrize("c", CASES, ids=lambda c: c.name)
def test_closed_form(c, num_splits):
    print(f"golden {c.name} S={num_splits}", flush=True)
    q = dev(c.q, c.dtype)
    bt = torch.from_numpy(c.block_table).cuda()
    ctx = torch.from_numpy(c.context_lens).cuda()
    fp8 = dict(k_scale=c.k_scale, v_scale=c.v_scale) if c.kv_dtype == "fp8" else {}
    maxc = int(c.context_lens.max())
    if c.kind == "mla":
        out, lse = pa.decode_mla(q, dev(c.pools["c"], c.kv_dtype), bt, ctx, max_context_len=maxc,
                                 scale=c.scale, head_dim_v=c.dv, num_splits=num_splits, **fp8)
    else:
        out, lse = pa.decode(q, dev(c.pools["k"], c.kv_dtype), dev(c.pools["v"], c.kv_dtype), bt,
                             ctx, max_context_len=maxc, scale=c.scale, num_splits=num_splits,
                             **fp8)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64).reshape(c.out.shape)
    l = lse.float().cpu().numpy().astype(np.float64).reshape(c.lse.shape)
    if c.dtype == "f32":
        np.testing.assert_allclose(o, c.out, rtol=0, atol=1e-5)
        lse_tol = 1e-5
    else:
        ulp = 2.0 ** -7 * np.maximum(np.abs(c.out), 2.0 ** -126)
        bad = np.abs(o - c.out) > ulp
        assert not bad.any(), f"{c.name}: {o[bad][:4]} against {c.out[bad][:4]}"
        lse_tol = 1e-3
    fin = np.isfinite(c.lse)
    assert np.array_equal(np.isfinite(l), fin)
    assert (l[~fin] == -np.inf).all()
    assert np.abs(l[fin] - c.lse[fin]).max(initial=0.0) <= lse_tol
