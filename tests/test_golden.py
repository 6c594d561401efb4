"""The float64 oracle against hand-derived closed forms (``golden/closed_forms.json``).

Each case's expected output and log-sum-exp were worked out by hand from the
definition (the derivation is written beside it in the file), so these pin the
oracle to something other than itself: the paging, the GQA head map, the
causal rows, FP8 code widening with both scales, the latent key/value split,
index-list decode and the log-sum-exp merge.
"""

import numpy as np
import pytest

import oracle
import golden_cases

CASES = golden_cases.cases()


def oracle_of(c):
    kw = dict(dtype=c.dtype)
    if c.kv_dtype == "fp8":
        kw.update(kv_dtype="fp8", k_scale=c.k_scale, v_scale=c.v_scale)
    if c.kind == "mla":
        fn = oracle.paged_decode_mla_rows if c.q_len > 1 else oracle.paged_decode_mla
        out, lse = fn(c.q, c.pools["c"], c.block_table, c.context_lens, c.scale, dv=c.dv, **kw)
    else:
        fn = oracle.paged_decode_rows if c.q_len > 1 else oracle.paged_decode
        out, lse = fn(c.q, c.pools["k"], c.pools["v"], c.block_table, c.context_lens, c.scale,
                      **kw)
    if c.q_len == 1:
        out, lse = out[:, None], lse[:, None]
    return out, lse


@pytest.mark.parametrize("c", CASES, ids=lambda c: c.name)
def test_oracle_matches_closed_form(c):
    out, lse = oracle_of(c)
    assert out.shape == c.out.shape
    np.testing.assert_allclose(out, c.out, rtol=0, atol=1e-12)
    fin = np.isfinite(c.lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert (lse[~fin] == -np.inf).all()
    np.testing.assert_allclose(lse[fin], c.lse[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("m", golden_cases.merges(), ids=lambda m: m[0])
def test_merge_matches_closed_form(m):
    _, o_parts, lse_parts, want_out, want_lse = m
    out, lse = oracle.merge_partials(o_parts, lse_parts)
    np.testing.assert_allclose(out, want_out, rtol=0, atol=1e-12)
    if np.isfinite(want_lse):
        assert abs(lse - want_lse) <= 1e-12
    else:
        assert lse == -np.inf


def test_every_case_is_exercised():
    """The fixture covers each path the library exposes at least once."""
    kinds = {(c.kind, c.dtype, c.kv_dtype, c.q_len > 1, c.spec["block_size"]) for c in CASES}
    assert ("mha", "f32", "f32", False, 16) in kinds
    assert ("mha", "bf16", "bf16", False, 16) in kinds
    assert ("mha", "bf16", "bf16", True, 16) in kinds
    assert ("mha", "bf16", "fp8", False, 16) in kinds
    assert ("mla", "bf16", "bf16", False, 64) in kinds
    assert ("mla", "bf16", "bf16", False, 1) in kinds
