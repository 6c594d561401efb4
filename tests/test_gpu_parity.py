"""HIP path vs the float64 oracle, element by element, on seeded inputs.

Tolerances (written here, from the required bars):
  float32 inputs: max |out - ref| <= 1e-5, max |lse - ref| <= 1e-5
  bf16 inputs:    max |out - ref| <= 2e-2 and ||out - ref||_2 / ||ref||_2 <= 1e-2;
                  max |lse - ref| <= 1e-3
Unused pool pages and the slots past each context are NaN, so any read of
memory the method must not read shows up as NaN in the output.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import decode_attention_paged_amd as pa
from workloads import make_config, make_paged_inputs
from workloads.device import from_device, to_device

pytestmark = pytest.mark.gpu

TOL = {
    "f32": dict(max_abs=1e-5, rel_l2=None, lse=1e-5),
    "bf16": dict(max_abs=2e-2, rel_l2=1e-2, lse=1e-3),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(inp, t=None, num_splits=0, poison=True):
    if t is None:
        t = to_device(inp, "cuda", poison)
    fp8 = dict(k_scale=inp.k_scale, v_scale=inp.v_scale) if inp.kv_dtype == "fp8" else {}
    if inp.kind == "mla":
        out, lse = pa.decode_mla(t["q"], t["kv_cache"], t["block_table"], t["context_lens"],
                                 max_context_len=inp.max_context_len, scale=inp.scale,
                                 head_dim_v=inp.head_dim_v, num_splits=num_splits, **fp8)
    else:
        out, lse = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["context_lens"], max_context_len=inp.max_context_len,
                             scale=inp.scale, num_splits=num_splits, **fp8)
    torch.cuda.synchronize()
    return out, lse


# Where the full-size test appends one JSON line of error margins per workload
# (unset: not recorded).
MARGINS_OUT = os.environ.get("PA_PARITY_MARGINS")


def compare(inp, out, lse, ref_out, ref_lse, what=""):
    o = from_device(out)
    l = lse.detach().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(ref_lse)           # rows the reference computed (a NaN row was not asked for)
    tol = TOL[inp.dtype]
    ro, rl = ref_out[sel], ref_lse[sel]
    go, gl = o[sel], l[sel]
    assert np.isfinite(go).all(), f"{what}: non-finite outputs"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: lse finiteness differs"
    assert np.array_equal(gl[~fin], rl[~fin])
    err = np.abs(go - ro)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ro))
    rel = float(np.linalg.norm(go - ro) / denom) if denom > 0 else float(np.linalg.norm(go))
    lerr = float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} lse_err={lerr:.3e} rows={int(sel.sum())}")
    assert max_abs <= tol["max_abs"], f"{what}: max abs {max_abs}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: rel l2 {rel}"
    assert lerr <= tol["lse"], f"{what}: lse err {lerr}"
    return dict(max_abs=max_abs, rel_l2=rel, lse_err=lerr, rows=int(sel.sum()),
                ref_max_abs=float(np.abs(ro).max()) if ro.size else 0.0)


# ----------------------------------------------------------------------------------------------
# The tiny fp32 workload, both required split counts
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("num_splits", [1, 4, 0])
def test_tiny_mha_f32(num_splits):
    inp = make_config("tiny_mha_f32")
    say(f"tiny_mha_f32 S={num_splits}")
    ref_out, ref_lse = oracle.decode_inputs(inp)
    out, lse = run(inp, num_splits=num_splits)
    compare(inp, out, lse, ref_out, ref_lse, f"tiny S={num_splits}")


# ----------------------------------------------------------------------------------------------
# Small shapes, every output compared: several tiles, ragged tails, many split counts
# ----------------------------------------------------------------------------------------------

SMALL = {
    "mha_bf16_d128": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=4, num_kv_heads=4,
                          head_dim=128, block_size=16, context_lens=[1, 37, 300], num_blocks=64),
    "mha_bf16_d64": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=3, num_kv_heads=3,
                         head_dim=64, block_size=16, context_lens=[129, 16], num_blocks=40),
    "mha_bf16_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                          head_dim=128, block_size=32, context_lens=[100, 31], num_blocks=20),
    "mha_f32_d128": dict(kind="mha", dtype="f32", batch=2, num_q_heads=2, num_kv_heads=2,
                         head_dim=128, block_size=16, context_lens=[77, 160], num_blocks=30),
    "mha_f32_d64_bs32": dict(kind="mha", dtype="f32", batch=2, num_q_heads=4, num_kv_heads=4,
                             head_dim=64, block_size=32, context_lens=[65, 3], num_blocks=10),
    # every lanes-per-V-row case of the VALU kernel: bf16 D64 bs32 (4), f32 D128 bs32 (8)
    "mha_bf16_d64_bs32": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=3, num_kv_heads=3,
                              head_dim=64, block_size=32, context_lens=[200, 1, 33], num_blocks=20),
    "mha_f32_d128_bs32": dict(kind="mha", dtype="f32", batch=2, num_q_heads=2, num_kv_heads=2,
                              head_dim=128, block_size=32, context_lens=[190, 17], num_blocks=12),
    "gqa_f32_g4": dict(kind="mha", dtype="f32", batch=2, num_q_heads=8, num_kv_heads=2,
                       head_dim=64, block_size=16, context_lens=[50, 200], num_blocks=30),
    "gqa_bf16_g4": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=8, num_kv_heads=2,
                        head_dim=128, block_size=16, context_lens=[17, 333], num_blocks=40),
    "gqa_bf16_g8": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=2,
                        head_dim=128, block_size=16, context_lens=[1, 16, 1000, 47], num_blocks=90),
    "gqa_bf16_g16": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=16, num_kv_heads=1,
                         head_dim=128, block_size=16, context_lens=[15, 515], num_blocks=40),
    "gqa_bf16_g2": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=6, num_kv_heads=3,
                        head_dim=128, block_size=16, context_lens=[33, 95], num_blocks=20),
    "mla_bf16_h16": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=16, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, block_size=64, context_lens=[1, 700],
                         num_blocks=20, scale=192 ** -0.5),
    "mla_bf16_h128": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=128, num_kv_heads=1,
                          head_dim=576, head_dim_v=512, block_size=64, context_lens=[65, 300],
                          num_blocks=12, scale=192 ** -0.5),
    "mla_bf16_h64": dict(kind="mla", dtype="bf16", batch=1, num_q_heads=64, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, block_size=64, context_lens=[129],
                         num_blocks=5, scale=192 ** -0.5),
    # one-token pages: block_table rows are token-index lists
    "mla_bf16_bs1_h128": dict(kind="mla", dtype="bf16", batch=3, num_q_heads=128,
                              num_kv_heads=1, head_dim=576, head_dim_v=512, block_size=1,
                              context_lens=[1, 100, 333], num_blocks=600, scale=192 ** -0.5),
    "mla_bf16_bs1_h32": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=32, num_kv_heads=1,
                             head_dim=576, head_dim_v=512, block_size=1, context_lens=[47, 65],
                             num_blocks=200, scale=192 ** -0.5),
    # two 128-head groups (wide workgroups paired on an XCD), three 64-head groups
    "mla_bf16_h256": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=256, num_kv_heads=1,
                          head_dim=576, head_dim_v=512, block_size=64, context_lens=[100, 257],
                          num_blocks=12, scale=192 ** -0.5),
    "mla_bf16_h192": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=192, num_kv_heads=1,
                          head_dim=576, head_dim_v=512, block_size=64, context_lens=[33, 190],
                          num_blocks=10, scale=192 ** -0.5),
    # 24 x 8 (sequence, KV head) units: grids above one workgroup per CU take the 4-wave
    # grouped-query workgroups, smaller ones the 8-wave ones
    "gqa_bf16_g4_b24": dict(kind="mha", dtype="bf16", batch=24, num_q_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16,
                            context_lens=[1, 300, 17, 64, 65, 250, 3, 129, 200, 31, 32, 33,
                                          280, 90, 7, 160, 161, 15, 16, 100, 45, 222, 2, 199],
                            num_blocks=400),
    # grouped heads on 32-token pages: the matrix-core kernel takes each page as one 32-token
    # step (its two 16-token halves), ragged tails inside a page and one-page contexts included
    "gqa_bf16_g4_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=8, num_kv_heads=2,
                             head_dim=128, block_size=32, context_lens=[40, 300], num_blocks=20),
    "gqa_bf16_g8_bs32": dict(kind="mha", dtype="bf16", batch=5, num_q_heads=16, num_kv_heads=2,
                             head_dim=128, block_size=32, context_lens=[1, 16, 17, 32, 1000],
                             num_blocks=60),
    "gqa_f32_g4_bs32": dict(kind="mha", dtype="f32", batch=2, num_q_heads=8, num_kv_heads=2,
                            head_dim=128, block_size=32, context_lens=[33, 250], num_blocks=20),
    # 256-dim heads (bf16) on the VALU kernel: plain, grouped and on 32-token pages
    "mha_bf16_d256": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                          head_dim=256, block_size=16, context_lens=[1, 200], num_blocks=20),
    "gqa_bf16_g2_d256": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=4, num_kv_heads=2,
                             head_dim=256, block_size=16, context_lens=[37, 300], num_blocks=30),
    "mha_bf16_d256_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                               head_dim=256, block_size=32, context_lens=[33, 150], num_blocks=12),
    # 64-dim heads on the matrix-core kernel (two score k-steps, four value dim blocks)
    "gqa_bf16_g4_d64": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=8, num_kv_heads=2,
                            head_dim=64, block_size=16, context_lens=[1, 47, 400], num_blocks=40),
    "gqa_bf16_g8_d64_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=16,
                                 num_kv_heads=2, head_dim=64, block_size=32,
                                 context_lens=[31, 700], num_blocks=30),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes(name):
    inp = make_paged_inputs(name=name, seed=100 + sorted(SMALL).index(name), **SMALL[name])
    ref_out, ref_lse = oracle.decode_inputs(inp)
    t = to_device(inp, "cuda", poison=True)
    P = -(-inp.max_context_len // inp.block_size)
    for S in [0, 1, 2, 3, 7, P + 5]:
        say(f"{name} S={S}")
        out, lse = run(inp, t, num_splits=S)
        compare(inp, out, lse, ref_out, ref_lse, f"{name} S={S}")


# ----------------------------------------------------------------------------------------------
# Several query rows per sequence (the last q_len tokens, causal): every output compared.
# Contexts shorter than q_len leave early rows with no token (out = 0, lse = -inf).
# ----------------------------------------------------------------------------------------------

ROWS = {
    "rows_mha_q4": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=4, num_kv_heads=4,
                        head_dim=128, block_size=16, context_lens=[3, 37, 300], num_blocks=64,
                        q_len=4),
    "rows_mha_q16": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                         head_dim=128, block_size=16, context_lens=[16, 200], num_blocks=30,
                         q_len=16),
    "rows_gqa_g4_q4": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=8, num_kv_heads=2,
                           head_dim=128, block_size=16, context_lens=[2, 17, 333], num_blocks=60,
                           q_len=4),
    "rows_gqa_g8_q2": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=2,
                           head_dim=128, block_size=16, context_lens=[1, 16, 1000, 47],
                           num_blocks=90, q_len=2),
    "rows_gqa_g2_q8": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=6, num_kv_heads=3,
                           head_dim=128, block_size=16, context_lens=[33, 95], num_blocks=20,
                           q_len=8),
    "rows_gqa_g4_q4_bs32": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=8,
                                num_kv_heads=2, head_dim=128, block_size=32,
                                context_lens=[2, 33, 333], num_blocks=30, q_len=4),
    "rows_gqa_g4_q2_d64": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=8,
                               num_kv_heads=2, head_dim=64, block_size=16,
                               context_lens=[1, 250], num_blocks=30, q_len=2),
    "rows_mla_h128_q2": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=128, num_kv_heads=1,
                             head_dim=576, head_dim_v=512, block_size=64, context_lens=[65, 300],
                             num_blocks=12, scale=192 ** -0.5, q_len=2),
    "rows_mla_h64_q3": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=64, num_kv_heads=1,
                            head_dim=576, head_dim_v=512, block_size=64, context_lens=[129, 2],
                            num_blocks=8, scale=192 ** -0.5, q_len=3),
    "rows_mla_h16_q4": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=16, num_kv_heads=1,
                            head_dim=576, head_dim_v=512, block_size=64, context_lens=[1, 700],
                            num_blocks=20, scale=192 ** -0.5, q_len=4),
    "rows_mla_h32_q3": dict(kind="mla", dtype="bf16", batch=2, num_q_heads=32, num_kv_heads=1,
                            head_dim=576, head_dim_v=512, block_size=64, context_lens=[66, 3],
                            num_blocks=8, scale=192 ** -0.5, q_len=3),
    "rows_mla_bs1_h128_q2": dict(kind="mla", dtype="bf16", batch=3, num_q_heads=128,
                                 num_kv_heads=1, head_dim=576, head_dim_v=512, block_size=1,
                                 context_lens=[1, 100, 333], num_blocks=600, scale=192 ** -0.5,
                                 q_len=2),
}


@pytest.mark.parametrize("name", sorted(ROWS))
def test_several_rows(name):
    inp = make_paged_inputs(name=name, seed=300 + sorted(ROWS).index(name), **ROWS[name])
    assert inp.q_len == ROWS[name]["q_len"]
    ref_out, ref_lse = oracle.decode_inputs(inp)
    t = to_device(inp, "cuda", poison=True)
    P = -(-inp.max_context_len // inp.block_size)
    for S in [0, 1, 2, 3, 7, P + 5]:
        say(f"{name} S={S}")
        out, lse = run(inp, t, num_splits=S)
        assert tuple(out.shape) == (inp.batch, inp.q_len, inp.num_q_heads, inp.head_dim_v)
        compare(inp, out, lse, ref_out, ref_lse, f"{name} S={S}")


# ----------------------------------------------------------------------------------------------
# FP8 E4M3 caches with bf16 queries (both kernels, one and several rows; the latent kernel on
# 128-head groups): every output compared.  Unused pages and tail slots hold the FP8 NaN code.
# ----------------------------------------------------------------------------------------------

FP8_KV = dict(kv_dtype="fp8", k_scale=0.037, v_scale=1.9)
# One latent row holds keys and values: codes are N(0,1) / k_scale, so v_scale below k_scale
# keeps the values (and outputs) near unit size, where the absolute bound applies: a latent
# output is rounded to bfloat16 twice (the split partial, then the output), up to 2^-8 |o|
# each time, which stays within 2e-2 for |o| <= 2.5 (one-token contexts copy a value).
FP8_LATENT = dict(kv_dtype="fp8", k_scale=0.037, v_scale=0.02)
MLA_DIMS = dict(kind="mla", dtype="bf16", num_kv_heads=1, head_dim=576, head_dim_v=512,
                block_size=64, scale=192 ** -0.5)
FP8 = {
    "fp8_mha_bs16": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=4, num_kv_heads=4,
                         head_dim=128, block_size=16, context_lens=[1, 37, 300], num_blocks=64,
                         **FP8_KV),
    "fp8_mha_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                         head_dim=128, block_size=32, context_lens=[100, 31], num_blocks=20,
                         **FP8_KV),
    "fp8_gqa_g4": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, context_lens=[17, 333], num_blocks=40, **FP8_KV),
    "fp8_gqa_g8": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=2,
                       head_dim=128, block_size=16, context_lens=[1, 16, 1000, 47], num_blocks=90,
                       **FP8_KV),
    "fp8_gqa_g16": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=16, num_kv_heads=1,
                        head_dim=128, block_size=16, context_lens=[15, 515], num_blocks=40,
                        **FP8_KV),
    "fp8_rows_mha_q4": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=4, num_kv_heads=4,
                            head_dim=128, block_size=16, context_lens=[3, 37, 300], num_blocks=64,
                            q_len=4, **FP8_KV),
    "fp8_rows_gqa_g4_q4": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=8, num_kv_heads=2,
                               head_dim=128, block_size=16, context_lens=[2, 17, 333],
                               num_blocks=60, q_len=4, **FP8_KV),
    # 64-dim heads on the VALU kernel: a K row is 4 lanes of 16 codes
    "fp8_mha_d64": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=3, num_kv_heads=3,
                        head_dim=64, block_size=16, context_lens=[1, 16, 333], num_blocks=40,
                        **FP8_KV),
    "fp8_mha_d64_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                             head_dim=64, block_size=32, context_lens=[31, 200], num_blocks=12,
                             **FP8_KV),
    "fp8_mha_d256": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=2, num_kv_heads=2,
                         head_dim=256, block_size=16, context_lens=[15, 260], num_blocks=30,
                         **FP8_KV),
    "fp8_gqa_g2_d256_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=4,
                                 num_kv_heads=2, head_dim=256, block_size=32,
                                 context_lens=[1, 170], num_blocks=12, **FP8_KV),
    "fp8_gqa_g4_d64": dict(kind="mha", dtype="bf16", batch=3, num_q_heads=8, num_kv_heads=2,
                           head_dim=64, block_size=16, context_lens=[1, 17, 500], num_blocks=50,
                           **FP8_KV),
    "fp8_gqa_g8_bs32": dict(kind="mha", dtype="bf16", batch=4, num_q_heads=16, num_kv_heads=2,
                            head_dim=128, block_size=32, context_lens=[1, 31, 48, 900],
                            num_blocks=60, **FP8_KV),
    "fp8_rows_gqa_g4_q2_bs32": dict(kind="mha", dtype="bf16", batch=2, num_q_heads=8,
                                    num_kv_heads=2, head_dim=128, block_size=32,
                                    context_lens=[1, 333], num_blocks=30, q_len=2, **FP8_KV),
    # pages of one, two and eleven (the last ragged) with a one-token sequence
    "fp8_mla_h128": dict(MLA_DIMS, batch=3, num_q_heads=128, context_lens=[1, 100, 700],
                         num_blocks=24, **FP8_LATENT),
    # two head groups; a context of exactly one page
    "fp8_mla_h256": dict(MLA_DIMS, batch=2, num_q_heads=256, context_lens=[64, 129],
                         num_blocks=8, **FP8_LATENT),
    "fp8_rows_mla_h128_q3": dict(MLA_DIMS, batch=2, num_q_heads=128, context_lens=[3, 300],
                                 num_blocks=10, q_len=3, **FP8_LATENT),
    # the role-split latent kernel: 16, 32 and 64 heads on 64-token pages, and one-token pages
    # (token-index lists) with 128 and 32 heads
    "fp8_mla_h16": dict(MLA_DIMS, batch=2, num_q_heads=16, context_lens=[1, 700], num_blocks=20,
                        **FP8_LATENT),
    "fp8_mla_h32": dict(MLA_DIMS, batch=2, num_q_heads=32, context_lens=[64, 129], num_blocks=8,
                        **FP8_LATENT),
    "fp8_mla_h64": dict(MLA_DIMS, batch=1, num_q_heads=64, context_lens=[300], num_blocks=6,
                        **FP8_LATENT),
    "fp8_mla_bs1_h128": dict(MLA_DIMS, batch=3, num_q_heads=128, block_size=1,
                             context_lens=[1, 100, 333], num_blocks=600, **FP8_LATENT),
    "fp8_mla_bs1_h32": dict(MLA_DIMS, batch=2, num_q_heads=32, block_size=1, context_lens=[47, 65],
                            num_blocks=200, **FP8_LATENT),
    "fp8_rows_mla_bs1_h128_q2": dict(MLA_DIMS, batch=2, num_q_heads=128, block_size=1,
                                     context_lens=[2, 150], num_blocks=300, q_len=2,
                                     **FP8_LATENT),
}


@pytest.mark.parametrize("name", sorted(FP8))
def test_fp8_kv(name):
    inp = make_paged_inputs(name=name, seed=400 + sorted(FP8).index(name), **FP8[name])
    ref_out, ref_lse = oracle.decode_inputs(inp)
    t = to_device(inp, "cuda", poison=True)
    assert t["kv_cache" if inp.kind == "mla" else "k_cache"].dtype == torch.float8_e4m3fn
    P = -(-inp.max_context_len // inp.block_size)
    for S in [0, 1, 2, 3, 7, P + 5]:
        say(f"{name} S={S}")
        out, lse = run(inp, t, num_splits=S)
        compare(inp, out, lse, ref_out, ref_lse, f"{name} S={S}")


# ----------------------------------------------------------------------------------------------
# Full-size workloads in the launch configuration the benchmark times (heuristic split count):
# every output row against the oracle (the float64 oracle takes at most ~10 s per workload).
# ----------------------------------------------------------------------------------------------

FULL = ["tiny_mha_f32", "llama_mha_bf16", "long_gqa_bf16", "ragged_gqa_bf16", "mla_bf16",
        "mla_topk_bf16", "mla_allentries_bf16", "llama_mha_q4_bf16", "long_gqa_q4_bf16",
        "mla_q2_bf16", "llama_mha_fp8", "long_gqa_fp8", "ragged_gqa_fp8", "mla_fp8",
        "mla_topk_fp8", "serving_gqa_bf16", "long_gqa_d64_bf16", "ragged_gqa_bs32_bf16",
        "llama_mha_d256_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_all_rows(name):
    say(f"full {name}: drawing inputs")
    inp = make_config(name)
    say(f"full {name}: oracle")
    ref_out, ref_lse = oracle.decode_inputs(inp)
    t = to_device(inp, "cuda", poison=True)
    say(f"full {name}: running")
    out, lse = run(inp, t, num_splits=0)
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    m = compare(inp, out, lse, ref_out, ref_lse, f"{name} all rows")
    if MARGINS_OUT:
        mla = inp.kind == "mla"
        shape = pa.make_shape(
            batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
            head_dim=inp.head_dim, head_dim_v=inp.head_dim_v, block_size=inp.block_size,
            max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
            max_context_len=inp.max_context_len, scale=inp.scale,
            dtype=torch.bfloat16 if inp.dtype == "bf16" else torch.float32, q_len=inp.q_len,
            kv_dtype=pa._lib.PA_FP8_E4M3 if inp.kv_dtype == "fp8" else 0,
            k_scale=inp.k_scale, v_scale=inp.v_scale)
        m.update(workload=name, num_splits=pa.choose_num_splits(shape, 0, mla),
                 dtype=inp.dtype, kv_dtype=inp.kv_dtype or inp.dtype, tol=TOL[inp.dtype])
        with open(MARGINS_OUT, "a") as f:
            f.write(json.dumps(m) + "\n")
    del t


# ----------------------------------------------------------------------------------------------
# Properties that hold at any size
# ----------------------------------------------------------------------------------------------

PROP = dict(kind="mha", dtype="bf16", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128,
            block_size=16, context_lens=[70, 1, 260], num_blocks=60)
PROP_MHA = dict(PROP, num_kv_heads=16)
PROP_MLA = dict(kind="mla", dtype="bf16", batch=2, num_q_heads=32, num_kv_heads=1, head_dim=576,
                head_dim_v=512, block_size=64, context_lens=[200, 1], num_blocks=10,
                scale=192 ** -0.5)
# 128 heads on 64-token pages: the wide latent workgroup
PROP_MLA128 = dict(PROP_MLA, num_q_heads=128)
# the same on an FP8 latent cache
PROP_MLA128_FP8 = dict(PROP_MLA128, **FP8_LATENT)


def _permuted(t, inp, seed):
    """Same logical KV with physical pages relabelled by a permutation."""
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(inp.num_blocks)).cuda()
    u = dict(t)
    for key in ("k_cache", "v_cache", "kv_cache"):
        if key in t:
            src = t[key]
            if src.dtype == torch.float8_e4m3fn:       # move FP8 pages as bytes
                src = src.view(torch.uint8)
            pool = torch.empty_like(src)
            pool[perm] = src
            u[key] = pool.view(t[key].dtype)
    bt = t["block_table"].long()
    u["block_table"] = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32)
    return u


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA, PROP_MLA128, PROP_MLA128_FP8],
                         ids=["gqa", "mha", "mla", "mla128", "mla128_fp8"])
@pytest.mark.parametrize("S", [0, 1, 5])
def test_page_permutation_bitwise(spec, S):
    inp = make_paged_inputs(seed=11, **spec)
    t = to_device(inp, "cuda")
    o1, l1 = run(inp, t, num_splits=S)
    o2, l2 = run(inp, _permuted(t, inp, 3), num_splits=S)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA], ids=["gqa", "mha", "mla"])
def test_determinism_and_batch_independence(spec):
    inp = make_paged_inputs(seed=12, **spec)
    t = to_device(inp, "cuda")
    o1, l1 = run(inp, t, num_splits=4)
    o2, l2 = run(inp, t, num_splits=4)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run-to-run difference"
    # each sequence alone (same max_context_len so the split plan is the same)
    for b in range(inp.batch):
        u = {k: v for k, v in t.items()}
        u["q"] = t["q"][b:b + 1].contiguous()
        u["block_table"] = t["block_table"][b:b + 1].contiguous()
        u["context_lens"] = t["context_lens"][b:b + 1].contiguous()
        one = make_paged_inputs(seed=12, values=False, **spec)
        one.batch = 1
        one.context_lens = inp.context_lens[b:b + 1]
        one.block_table = inp.block_table[b:b + 1]
        ob, lb = run(_with_max(one, inp.max_context_len), u, num_splits=4)
        assert torch.equal(ob[0], o1[b]) and torch.equal(lb[0], l1[b]), f"sequence {b}"


class _with_max:
    """Workload view that keeps a given max_context_len (same split plan)."""

    def __init__(self, inp, max_ctx):
        self._inp = inp
        self.max_context_len = max_ctx

    def __getattr__(self, k):
        return getattr(self._inp, k)


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA, PROP_MLA128],
                         ids=["gqa", "mha", "mla", "mla128"])
def test_context_one_returns_v0_exactly(spec):
    s = dict(spec, context_lens=[1] * spec["batch"])
    inp = make_paged_inputs(seed=13, **s)
    out, lse = run(inp, num_splits=0)
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(inp.batch):
        row = inp.compact_block_table()[b, 0]
        for h in range(inp.num_q_heads):
            if inp.kind == "mla":
                v0 = inp.c_pages[row, 0, :inp.head_dim_v]
            else:
                g = h // (inp.num_q_heads // inp.num_kv_heads)
                v0 = inp.v_pages[row, g, :, 0]
            assert np.array_equal(o[b, h], v0), (b, h)
    ref_out, ref_lse = oracle.decode_inputs(inp)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA], ids=["gqa", "mha", "mla"])
def test_identical_keys_give_mean_of_values(spec):
    """Equal keys weight every token equally: out is the mean of the values.

    For the latent variant keys and values are the same rows, so equal keys
    mean equal rows and the output is that row's value part.
    """
    inp = make_paged_inputs(seed=14, **spec)
    b = 2 if inp.batch > 2 else 0
    bt = inp.compact_block_table()
    n = int(inp.context_lens[b])
    if inp.kind == "mla":
        inp.c_pages[:] = inp.c_pages[bt[b, 0], 0, :][None, None, :]
        want = np.broadcast_to(oracle.as_f64(inp.c_pages[0, 0, :inp.head_dim_v], "bf16"),
                               (inp.num_q_heads, inp.head_dim_v))
    else:
        inp.k_pages[:] = inp.k_pages[bt[b, 0], :, 0, :][None, :, None, :]
        pages = bt[b, :-(-n // inp.block_size)]
        vals = oracle.as_f64(inp.v_pages[pages], "bf16")            # [p][Hkv][D][bs]
        vals = vals.transpose(0, 3, 1, 2).reshape(-1, inp.num_kv_heads, inp.head_dim)[:n]
        mean = vals.mean(axis=0)
        G = inp.num_q_heads // inp.num_kv_heads
        want = np.stack([mean[h // G] for h in range(inp.num_q_heads)])
    ref_out, ref_lse = oracle.decode_inputs(inp)
    out, lse = run(inp, num_splits=3)
    compare(inp, out, lse, ref_out, ref_lse, "identical keys")
    assert np.abs(from_device(out)[b] - want).max() <= 2e-2


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA, PROP_MLA128_FP8],
                         ids=["gqa", "mha", "mla", "mla128_fp8"])
def test_empty_context(spec):
    s = dict(spec, context_lens=[0] + list(spec["context_lens"][1:]))
    inp = make_paged_inputs(seed=15, **s)
    ref_out, ref_lse = oracle.decode_inputs(inp)
    for S in (1, 4):
        out, lse = run(inp, num_splits=S)
        assert (out[0].float() == 0).all().item()
        assert torch.isinf(lse[0]).all().item() and (lse[0] < 0).all().item()
        compare(inp, out, lse, ref_out, ref_lse, f"empty ctx S={S}")


def _shape_of(inp):
    return pa.make_shape(batch=inp.batch, num_q_heads=inp.num_q_heads,
                         num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                         head_dim_v=inp.head_dim_v, block_size=inp.block_size,
                         max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
                         max_context_len=inp.max_context_len, scale=inp.scale,
                         dtype=torch.bfloat16 if inp.dtype == "bf16" else torch.float32)


def _bf16_ulps(a, b):
    """Largest distance in bf16 units in the last place between two bf16 tensors."""
    ia = a.view(torch.int16).to(torch.int32)
    ib = b.view(torch.int16).to(torch.int32)
    # map sign-magnitude to a monotone integer line
    ia = torch.where(ia < 0, -32768 - ia, ia)
    ib = torch.where(ib < 0, -32768 - ib, ib)
    return int((ia - ib).abs().max().item())


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA], ids=["gqa", "mha", "mla"])
def test_partial_then_reduce_matches_decode(spec):
    """The separate partial + reduce launches give the fused call's result.

    Both reach the same sum in a different order, so the outputs may differ
    by rounding only: at most one bf16 unit in the last place.
    """
    inp = make_paged_inputs(seed=16, **spec)
    t = to_device(inp, "cuda")
    S = 3
    o1, l1 = run(inp, t, num_splits=S)
    mla = inp.kind == "mla"
    shape = _shape_of(inp)
    ws = torch.zeros(pa.workspace_size(shape, S, mla), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    if mla:
        pa.decode_mla_partial(shape, t["q"], t["kv_cache"], t["block_table"], t["context_lens"],
                              S, o2, l2, ws)
    else:
        pa.decode_partial(shape, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                          t["context_lens"], S, o2, l2, ws)
    pa.reduce(shape, t["context_lens"], S, ws, o2, l2, mla=mla)
    torch.cuda.synchronize()
    assert _bf16_ulps(o1, o2) <= 1
    assert (l1 - l2).abs().max().item() <= 1e-5
    ref_out, ref_lse = oracle.decode_inputs(inp)
    compare(inp, o2, l2, ref_out, ref_lse, "partial+reduce")


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA], ids=["gqa", "mha", "mla"])
def test_workspace_reuse_and_init(spec):
    """One workspace across calls: the fused reduction leaves its counters at zero.

    A workspace filled with garbage and re-initialised with pa_workspace_init
    works as well.
    """
    mla = spec["kind"] == "mla"
    S = 4
    ws = None
    for it, seed in enumerate((21, 22, 23)):
        inp = make_paged_inputs(seed=seed, **spec)
        shape = _shape_of(inp)
        if ws is None:
            ws = torch.full((pa.workspace_size(shape, S, mla),), 0xAB, dtype=torch.uint8,
                            device="cuda")
            pa.workspace_init(shape, ws, S, mla)
        t = to_device(inp, "cuda")
        if mla:
            out, lse = pa.decode_mla(t["q"], t["kv_cache"], t["block_table"], t["context_lens"],
                                     max_context_len=inp.max_context_len, scale=inp.scale,
                                     num_splits=S, workspace=ws)
        else:
            out, lse = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                                 t["context_lens"], max_context_len=inp.max_context_len,
                                 scale=inp.scale, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_inputs(inp)
        compare(inp, out, lse, ref_out, ref_lse, f"reuse call {it}")


def test_bf16_output_rounding_is_nearest_even():
    """A one-token context copies v0; with S = 1 and S > 1 alike the bits survive."""
    inp = make_paged_inputs(seed=17, **dict(PROP_MHA, context_lens=[1, 1, 1]))
    for S in (1, 2):
        out, _ = run(inp, num_splits=S)
        o = out.view(torch.int16).cpu().numpy().view(np.uint16)
        bt = inp.compact_block_table()
        for b in range(3):
            assert np.array_equal(o[b, :, :], inp.v_pages[bt[b, 0], :, :, 0])


@pytest.mark.parametrize("spec", [PROP, PROP_MHA, PROP_MLA, PROP_MLA128],
                         ids=["gqa", "mha", "mla", "mla128"])
def test_rising_scores(spec):
    """Scores that climb steeply with the token index: every tile's max exceeds
    the running max by far more than the bf16 weights could hold unrescaled,
    so each kernel's handling of a rising max (rescaling, or starting a split
    over with a raised reference max) runs at every tile."""
    from workloads import f32_to_bf16_bits
    lens = [1000, 77] + list(spec["context_lens"][2:])
    s = dict(spec, context_lens=lens,
             num_blocks=sum(-(-n // spec["block_size"]) for n in lens) + 10)
    inp = make_paged_inputs(seed=18, **s)
    bt = inp.compact_block_table()
    step = 8.0 if inp.kind == "mla" else 3.0
    d = inp.head_dim - 1      # for the latent: a key-only dim, outside the value part
    for b in range(inp.batch):
        for tok in range(int(inp.context_lens[b])):
            page, slot = bt[b, tok // inp.block_size], tok % inp.block_size
            bits = f32_to_bf16_bits(np.array([step * tok], np.float32))[0]
            if inp.kind == "mla":
                inp.c_pages[page, slot, d] = bits
            else:
                inp.k_pages[page, :, slot, d] = bits
    inp.q[:, :, d] = f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    ref_out, ref_lse = oracle.decode_inputs(inp)
    t = to_device(inp, "cuda")
    for S in (1, 3, 0):
        say(f"rising scores {inp.kind} S={S}")
        out, lse = run(inp, t, num_splits=S)
        compare(inp, out, lse, ref_out, ref_lse, f"rising scores S={S}")


@pytest.mark.parametrize("heads,bs", [(128, 64), (64, 64), (128, 1)],
                         ids=["wide", "roles", "roles_bs1"])
def test_rising_scores_fp8_latent(heads, bs):
    """The rising-scores case on an FP8 latent cache: the codes of a key-only
    dim climb with the token index (a quarter of it, rounded to E4M3), and the
    query's weight on that dim makes each 32-token chunk's max exceed the
    previous one by far more than the headroom, so the latent kernels start
    their splits over with a raised reference max."""
    lens = [1000, 77]
    s = dict(PROP_MLA128_FP8, num_q_heads=heads, block_size=bs, context_lens=lens, k_scale=0.25,
             v_scale=0.3, num_blocks=sum(-(-n // bs) for n in lens) + 10)
    inp = make_paged_inputs(seed=19, **s)
    bt = inp.compact_block_table()
    d = inp.head_dim - 1
    codes = torch.from_numpy(np.arange(max(lens), dtype=np.float32) / 4).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    for b in range(inp.batch):
        for tok in range(int(inp.context_lens[b])):
            inp.c_pages[bt[b, tok // bs], tok % bs, d] = codes[tok]
    from workloads import f32_to_bf16_bits
    inp.q[:, :, d] = f32_to_bf16_bits(np.array([256.0], np.float32))[0]
    ref_out, ref_lse = oracle.decode_inputs(inp)
    t = to_device(inp, "cuda")
    for S in (1, 3, 0):
        say(f"rising scores fp8 latent S={S}")
        out, lse = run(inp, t, num_splits=S)
        compare(inp, out, lse, ref_out, ref_lse, f"rising scores fp8 latent S={S}")
