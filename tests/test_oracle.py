"""The float64 oracle against its pins (brute force, torch SDPA, closed forms, invariants)."""

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_empty_context_reading():
    """An empty context gives out = 0 and lse = -inf, never NaN."""
    q = np.ones((1, 2, 4))
    k = np.full((2, 1, 4, 4), np.nan)
    v = np.full((2, 1, 4, 4), np.nan)
    out, lse = oracle.paged_decode(q, k, v, np.array([[0]]), np.array([0]), 0.5, dtype="f64")
    assert (out == 0).all() and (lse == -np.inf).all()


def test_poisoned_tail_not_read():
    """Slots past the context and pages past the last one never reach the result."""
    from oracle_pins import tiny_paged
    q, k, v, bt, ctx, scale = tiny_paged(60, 1, 2, 1, 8, 8, 4, [6])
    out, lse = oracle.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    k2, v2 = k.copy(), v.copy()
    last = bt[0, 1]
    k2[last, :, 2:, :] = np.nan
    v2[last, :, :, 2:] = np.nan
    unused = [p for p in range(k.shape[0]) if p not in bt[0, :2]]
    k2[unused] = np.nan
    v2[unused] = np.nan
    out2, lse2 = oracle.paged_decode(q, k2, v2, bt, ctx, scale, dtype="f64")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_workload_inputs_roundtrip():
    """The oracle reads compact workload pages the same as a full physical pool."""
    from workloads import make_paged_inputs
    inp = make_paged_inputs(kind="mha", dtype="bf16", batch=3, num_q_heads=4, num_kv_heads=2,
                            head_dim=16, block_size=4, context_lens=[9, 1, 14], num_blocks=40,
                            seed=7)
    out_c, lse_c = oracle.decode_inputs(inp)
    # rebuild the full pool at physical ids, NaN elsewhere
    nan = np.uint16(0x7FC0)
    k_full = np.full((40,) + inp.k_pages.shape[1:], nan, dtype=np.uint16)
    v_full = np.full((40,) + inp.v_pages.shape[1:], nan, dtype=np.uint16)
    k_full[inp.page_ids] = inp.k_pages
    v_full[inp.page_ids] = inp.v_pages
    bt = np.where(inp.block_table >= 0, inp.block_table, 0)
    out_f, lse_f = oracle.paged_decode(inp.q, k_full, v_full, bt, inp.context_lens, inp.scale,
                                       dtype="bf16")
    assert np.array_equal(out_c, out_f) and np.array_equal(lse_c, lse_f)
    assert np.isfinite(out_c).all()
