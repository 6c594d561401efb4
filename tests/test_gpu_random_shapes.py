"""Seeded random shapes across every supported kernel path, against the oracle.

Each case draws one valid shape: the kernel family (MHA/GQA on the VALU or
MFMA kernel, the latent kernels on 64-token pages or token-index lists),
dtype, FP8 caches, head counts and grouping, page size, query rows, a batch of
ragged lengths (0 and 1 included at random) and a split count (heuristic,
1, small, or more than the pages), and compares every output with the float64
oracle at the parity bar (fp32: max abs 1e-5; bf16: max abs 2e-2, rel L2
1e-2; lse 1e-5 / 1e-3).  The draws are fixed by the seed, so a failure names
a reproducible shape.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_paged_inputs

from test_gpu_parity import compare, run, say

pytestmark = pytest.mark.gpu

N_CASES = 192


def _draw(seed: int) -> tuple[dict, int]:
    r = np.random.default_rng(1000 + seed)
    kind = r.choice(["mha_valu", "gqa_mfma", "gqa_valu", "mla_pages", "mla_index"])
    B = int(r.integers(1, 6))
    fp8 = False
    if kind == "mha_valu":
        dtype = str(r.choice(["f32", "bf16"]))
        D = int(r.choice([64, 128] if dtype == "f32" else [64, 128, 256]))
        bs = int(r.choice([16, 32]))
        H = int(r.integers(1, 9))
        fp8 = dtype == "bf16" and r.random() < 0.4
        spec = dict(kind="mha", dtype=dtype, num_q_heads=H, num_kv_heads=H, head_dim=D,
                    block_size=bs)
        ql, maxlen = 1, 700
    elif kind == "gqa_mfma":
        G = int(r.choice([2, 4, 8, 16]))
        ql = int(r.choice([q for q in (1, 2, 4, 8, 16) if G * q <= 16]))
        Hkv = int(r.integers(1, 4))
        fp8 = r.random() < 0.4
        bs = int(r.choice([16, 32]))
        D = int(r.choice([64, 128]))
        spec = dict(kind="mha", dtype="bf16", num_q_heads=G * Hkv, num_kv_heads=Hkv,
                    head_dim=D, block_size=bs)
        maxlen = 900
    elif kind == "gqa_valu":                 # grouped heads in fp32: the VALU kernel
        G = int(r.choice([2, 4]))
        D, bs = [(64, 16), (128, 32), (64, 32)][int(r.integers(0, 3))]
        spec = dict(kind="mha", dtype="f32", num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                    block_size=bs)
        ql, maxlen = 1, 600
    else:
        bs = 64 if kind == "mla_pages" else 1
        Hq = int(r.choice([16, 32, 64, 128, 192, 256] if bs == 64 else [16, 32, 64, 128]))
        ql = int(r.choice([1, 1, 2, 3]))
        fp8 = r.random() < 0.5
        spec = dict(kind="mla", dtype="bf16", num_q_heads=Hq, num_kv_heads=1, head_dim=576,
                    head_dim_v=512, block_size=bs, scale=192 ** -0.5)
        maxlen = 900 if bs == 64 else 500
    lens = [int(x) for x in r.integers(0, maxlen + 1, B)]
    if r.random() < 0.3:
        lens[int(r.integers(0, B))] = int(r.choice([0, 1]))
    if max(lens) == 0:
        lens[0] = 1
    pages = sum(-(-n // spec["block_size"]) for n in lens)
    spec.update(batch=B, context_lens=lens, num_blocks=max(1, pages + int(r.integers(0, 20))),
                q_len=ql)
    if fp8:
        ks = float(r.choice([0.02, 0.05, 0.1]))
        # a latent row serves keys and values: keep the values near unit size (an output is
        # rounded to bfloat16 twice, split partial and output, within 2e-2 up to |o| = 2.5)
        vs = ks * float(r.uniform(0.4, 0.7)) if spec["kind"] == "mla" else float(r.uniform(0.2, 2))
        spec.update(kv_dtype="fp8", k_scale=ks, v_scale=vs)
    P = -(-max(lens) // spec["block_size"]) if max(lens) else 1
    choices = [0, 1, 2, 5, P + 3]
    if spec["kind"] == "mla" and spec["block_size"] == 1:
        choices = [S for S in choices if S == 0 or -(-max(max(lens), 1) // max(S, 1)) <= 2048]
    S = int(r.choice(choices))
    return spec, S


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    spec, S = _draw(seed)
    say(f"random {seed}: S={S} {spec}")
    inp = make_paged_inputs(name=f"random{seed}", seed=2000 + seed, **spec)
    ref_out, ref_lse = oracle.decode_inputs(inp)
    out, lse = run(inp, num_splits=S)
    compare(inp, out, lse, ref_out, ref_lse, f"random {seed} S={S}")
