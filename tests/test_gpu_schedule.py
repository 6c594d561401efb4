"""The unit order of a ragged batch on the grouped-query kernel.

The schedule launch writes, into the workspace after the split partials, one
u32 per (sequence, split) slot of the grid: every real unit exactly once
(sequence | split << 16), full splits first, then each sequence's last split
by decreasing size at the schedule's bucket resolution, then the "no unit"
marker for the remaining slots.  The decode over that order must match the
oracle, whatever the order.
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

NO_UNIT = 0xFFFFFFFF
BUCKETS = 1024

# 200 pages at most: splits of 100, 67 and 50 pages are units of >= 384 KiB of
# bf16 KV (400 KiB at 100 pages of FP8), which the library schedules
SPEC = dict(kind="mha", dtype="bf16", batch=7, num_q_heads=16, num_kv_heads=2, head_dim=128,
            block_size=16, context_lens=[1, 17, 300, 1600, 0, 1024, 3200], num_blocks=600)


def _up(x):
    return -(-x // 256) * 256


def _units(ctx, bs, c):
    """(full splits, size of the last split or None) per sequence."""
    out = []
    for n in ctx:
        pages = -(-int(n) // bs)
        ns = -(-pages // c) if pages > 0 else 1
        last = pages - (ns - 1) * c
        out.append((ns, None) if last == c else (ns - 1, last))
    return out


@pytest.mark.parametrize("fp8,q_len,heads", [(False, 1, 16), (True, 1, 16), (False, 2, 16),
                                              (True, 3, 8)],
                         ids=["bf16", "fp8", "bf16_q2", "fp8_q3_g4"])
def test_unit_order_and_result(fp8, q_len, heads):
    spec = dict(SPEC, num_q_heads=heads, q_len=q_len,
                **(dict(kv_dtype="fp8", k_scale=0.037, v_scale=0.045) if fp8 else {}))
    inp = make_paged_inputs(seed=21, **spec)
    t = to_device(inp, "cuda", poison=True)
    ref_out, ref_lse = oracle.decode_inputs(inp)
    shape = pa.make_shape(
        batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
        head_dim=inp.head_dim, head_dim_v=inp.head_dim_v, block_size=inp.block_size,
        max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
        max_context_len=inp.max_context_len, scale=inp.scale, dtype=torch.bfloat16,
        q_len=q_len, kv_dtype=pa._lib.PA_FP8_E4M3 if fp8 else 0, k_scale=inp.k_scale,
        v_scale=inp.v_scale)
    B, bs = inp.batch, inp.block_size
    P = -(-inp.max_context_len // bs)
    rows = B * q_len * inp.num_q_heads
    qdims = (B, q_len) if q_len > 1 else (B,)
    for S in ((2,) if fp8 else (2, 3, 4)):
        print(f"unit order fp8={fp8} q_len={q_len} heads={heads} S={S}", flush=True)
        c = -(-P // S)
        nbytes = pa.workspace_size(shape, S)
        sched_off = _up(rows * 4) + _up(rows * S * inp.head_dim_v * 4) + _up(rows * S * 4)
        assert nbytes == sched_off + _up(B * S * 4)
        ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
        out = torch.empty(qdims + (inp.num_q_heads, inp.head_dim_v), dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.empty(qdims + (inp.num_q_heads,), dtype=torch.float32, device="cuda")
        pa.decode_partial(shape, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                          t["context_lens"], S, out, lse, ws)
        torch.cuda.synchronize()
        tab = ws[sched_off:sched_off + 4 * B * S].cpu().numpy().view(np.uint32)
        units = _units(inp.context_lens, bs, c)
        n_full = sum(f for f, _ in units)
        want_part = sorted((b for b, (_, last) in enumerate(units) if last is not None))
        n_real = n_full + len(want_part)
        assert (tab[n_real:] == NO_UNIT).all()
        got = tab[:n_real]
        assert (got != NO_UNIT).all()
        seq, split = (got & 0xFFFF).astype(int), (got >> 16).astype(int)
        # every real unit once
        want = sorted((b, s) for b, (f, last) in enumerate(units)
                      for s in range(f + (last is not None)))
        assert sorted(zip(seq.tolist(), split.tolist())) == want
        # full splits first, then last splits by decreasing size (bucketed)
        full = np.array([split[i] < units[seq[i]][0] for i in range(n_real)])
        assert full[:n_full].all() and not full[n_full:].any()
        sizes = [units[b][1] for b in seq[n_full:]]
        buckets = [(c - x) * (BUCKETS - 1) // c for x in sizes]
        assert buckets == sorted(buckets)
        pa.reduce(shape, t["context_lens"], S, ws, out, lse)
        torch.cuda.synchronize()
        o = from_device(out)
        assert np.abs(o - ref_out).max() <= 2e-2
        gl = lse.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lse)
        assert np.array_equal(gl[~fin], ref_lse[~fin])      # empty sequences: -inf
        assert np.abs(gl[fin] - ref_lse[fin]).max() <= 1e-3


def test_unit_order_more_sequences_than_threads():
    """A batch of 1300 sequences (more than the schedule's 1024 threads, so
    its placement pass reads some lengths again), mostly short, with a few
    long ones whose units reach 384 KiB: the order is still a permutation of
    the real units, longest first, and the result matches the oracle."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 120, 1300)]
    for i in (3, 700, 1100, 1299):
        lens[i] = 3200
    spec = dict(kind="mha", dtype="bf16", batch=len(lens), num_q_heads=8, num_kv_heads=2,
                head_dim=128, block_size=16, context_lens=lens,
                num_blocks=sum(-(-n // 16) for n in lens) + 16)
    inp = make_paged_inputs(seed=22, **spec)
    t = to_device(inp, "cuda", poison=True)
    ref_out, ref_lse = oracle.decode_inputs(inp)
    shape = pa.make_shape(
        batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
        head_dim=inp.head_dim, head_dim_v=inp.head_dim_v, block_size=inp.block_size,
        max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
        max_context_len=inp.max_context_len, scale=inp.scale, dtype=torch.bfloat16)
    B, S = inp.batch, 2
    assert pa.decode_launches(shape, S) == 3
    P = -(-inp.max_context_len // 16)
    c = -(-P // S)
    rows = B * inp.num_q_heads
    sched_off = _up(rows * 4) + _up(rows * S * inp.head_dim_v * 4) + _up(rows * S * 4)
    ws = torch.full((pa.workspace_size(shape, S),), 0xAB, dtype=torch.uint8, device="cuda")
    out = torch.empty((B, inp.num_q_heads, inp.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, inp.num_q_heads), dtype=torch.float32, device="cuda")
    print("unit order: 1300 sequences", flush=True)
    pa.decode_partial(shape, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                      t["context_lens"], S, out, lse, ws)
    torch.cuda.synchronize()
    tab = ws[sched_off:sched_off + 4 * B * S].cpu().numpy().view(np.uint32)
    units = _units(inp.context_lens, 16, c)
    n_full = sum(f for f, _ in units)
    want = sorted((b, s) for b, (f, last) in enumerate(units) for s in range(f + (last is not None)))
    n_real = len(want)
    assert (tab[n_real:] == NO_UNIT).all()
    got = tab[:n_real]
    assert sorted(zip((got & 0xFFFF).astype(int).tolist(), (got >> 16).astype(int).tolist())) == want
    seq = (got & 0xFFFF).astype(int)
    sizes = [units[b][1] for b in seq[n_full:]]
    assert [(c - x) * (BUCKETS - 1) // c for x in sizes] == \
        sorted((c - x) * (BUCKETS - 1) // c for x in sizes)
    pa.reduce(shape, t["context_lens"], S, ws, out, lse)
    torch.cuda.synchronize()
    assert np.abs(from_device(out) - ref_out).max() <= 2e-2
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(gl[~fin], ref_lse[~fin])
    assert np.abs(gl[fin] - ref_lse[fin]).max() <= 1e-3
