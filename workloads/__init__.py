"""Seeded synthetic inputs for paged decode attention.

This module only draws and lays out inputs: context lengths, page
assignments, the query and the paged key/value (or latent) cache.  It holds
none of the attention arithmetic, so that the CPU oracle and the HIP path can
both be fed from it without sharing any of the method.

One generator, ``numpy.random.default_rng(seed)`` (PCG64), draws everything
in this order: the context lengths, the page assignment (a permutation of
the pool, whose prefix is handed out sequence by sequence in logical page
order), q, then K and V (or the latent) in logical token order (page, slot,
head, dim).  Every value is drawn as float32 N(0, 1) and, for bf16
workloads, rounded to bfloat16 with round-to-nearest-even; bf16 arrays are
carried as their uint16 bit patterns.  Large tensors are drawn in sequential
chunks of ``CHUNK`` values from the same generator, which yields the same
stream as one draw.

Pool layouts (physical page ``p``):

* MHA/GQA key pool    ``k[num_blocks][Hkv][block_size][D]``
* MHA/GQA value pool  ``v[num_blocks][Hkv][D][block_size]``
* MLA latent pool     ``c[num_blocks][block_size][Dqk]`` (V = first Dv dims)

Only the pages a workload uses are materialised on the host ("compact"
arrays, row ``i`` holding physical page ``page_ids[i]``); a device pool of
``num_blocks`` pages is filled from them by scattering rows to ``page_ids``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22
BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F          # E4M3 NaN (S.1111.111)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite draws, so the NaN/overflow corners of the rounding are
    not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


class _Draw:
    """N(0,1) values from the workload's one generator, drawn in sequence."""

    def __init__(self, rng: np.random.Generator):
        self.rng = rng

    def normal_fp8(self, n: int, scale: float) -> np.ndarray:
        """n N(0,1) values as FP8 E4M3 codes (uint8) of value / scale: rounded to
        nearest even by torch's float8_e4m3fn cast, after clipping to the
        format's largest finite magnitude, 448."""
        import torch
        f = self.normal(n, "f32")
        x = np.clip(f / np.float32(scale), -448.0, 448.0).astype(np.float32)
        return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    def normal(self, n: int, dtype: str) -> np.ndarray:
        """n values in the workload dtype (float32, or bf16 bits as uint16)."""
        out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
        for lo in range(0, n, CHUNK):
            hi = min(n, lo + CHUNK)
            vals = self.rng.standard_normal(hi - lo, dtype=np.float32)
            out[lo:hi] = vals if dtype == "f32" else f32_to_bf16_bits(vals)
        return out


@dataclass
class PagedDecodeInputs:
    """One decode step's inputs, with the KV pages held compactly on the host."""

    name: str
    kind: str                 # "mha" (MHA/GQA) or "mla"
    dtype: str                # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int         # 1 for MLA
    head_dim: int             # Dqk
    head_dim_v: int           # Dv
    block_size: int
    num_blocks: int           # physical pages in the device pool
    scale: float
    context_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray   # int32 [B][max_blocks_per_seq], physical ids
    page_ids: np.ndarray      # int32 [n_used]: physical id of compact row i
    q: np.ndarray             # [B][Hq][Dqk] (or [B][q_len][Hq][Dqk]) float32 or uint16 bf16 bits
    k_pages: np.ndarray | None = None   # [n_used][Hkv][bs][D]
    v_pages: np.ndarray | None = None   # [n_used][Hkv][D][bs]
    c_pages: np.ndarray | None = None   # [n_used][bs][Dqk] (MLA latent)
    meta: dict = field(default_factory=dict)
    kv_dtype: str | None = None         # cache dtype when not the query's: "fp8" (E4M3 codes)
    k_scale: float = 1.0                # FP8: a key is k_scale times its code's value
    v_scale: float = 1.0

    @property
    def q_len(self) -> int:
        """Query rows per sequence (the last q_len tokens, causal)."""
        return int(self.q.shape[1]) if self.q.ndim == 4 else 1

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def esize(self) -> int:
        """Bytes per cache element."""
        if self.kv_dtype == "fp8":
            return 1
        return 4 if self.dtype == "f32" else 2

    def compact_block_table(self) -> np.ndarray:
        """The block table with physical ids replaced by compact row indices.

        Entries that point at no used page become -1.
        """
        lut = np.full(self.num_blocks, -1, dtype=np.int64)
        lut[self.page_ids] = np.arange(len(self.page_ids))
        bt = self.block_table.astype(np.int64)
        out = np.where(bt >= 0, lut[np.clip(bt, 0, self.num_blocks - 1)], -1)
        return out.astype(np.int32)

    def kv_bytes_read(self) -> int:
        """Bytes of K and V the step must read: every context token's rows."""
        toks = int(self.context_lens.astype(np.int64).sum())
        if self.kind == "mla":
            return toks * self.head_dim * self.esize
        return toks * self.num_kv_heads * (self.head_dim + self.head_dim_v) * self.esize


def _assign_pages(rng: np.random.Generator, n_pages: np.ndarray, num_blocks: int,
                  max_blocks: int) -> tuple[np.ndarray, np.ndarray]:
    """Give each sequence its pages from a seeded permutation of the pool.

    Returns (block_table [B][max_blocks] with -1 padding, page_ids in logical
    order: sequence-major, then logical page).
    """
    total = int(n_pages.sum())
    if total > num_blocks:
        raise ValueError(f"pool of {num_blocks} pages cannot hold {total}")
    perm = rng.permutation(num_blocks)[:total].astype(np.int32)
    bt = np.full((len(n_pages), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages.tolist()):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, perm


def make_paged_inputs(*, name: str = "custom", kind: str = "mha", dtype: str = "bf16",
                      batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      head_dim_v: int | None = None, block_size: int,
                      context_lens, num_blocks: int | None = None,
                      max_blocks_per_seq: int | None = None, scale: float | None = None,
                      seed: int = 0, poison: bool = True, values: bool = True,
                      meta: dict | None = None, q_len: int = 1, kv_dtype: str | None = None,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> PagedDecodeInputs:
    """Draw a paged decode workload.

    ``context_lens`` is an int sequence (or a callable ``rng -> array`` drawn
    first from the workload's generator).  Pages are assigned from a seeded
    permutation of a pool of ``num_blocks`` pages.  With ``poison`` the slots
    past each context's end in its last page are NaN; the device pool's
    unassigned pages are to be NaN-filled by the caller as well.  With
    ``values=False`` only the shapes, lengths and tables are drawn.  With
    ``q_len`` > 1, q is [B][q_len][Hq][Dqk]: the sequences' last q_len tokens
    as query rows.  With ``kv_dtype="fp8"`` (bf16 queries) the caches hold
    FP8 E4M3 codes of the same N(0,1) draws divided by k_scale / v_scale.
    """
    if kind not in ("mha", "mla"):
        raise ValueError(kind)
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    fp8 = kv_dtype == "fp8"
    if kv_dtype not in (None, dtype, "fp8") or (fp8 and dtype != "bf16"):
        raise ValueError(f"cache dtype {kv_dtype} with {dtype} queries / {kind}")
    if kind == "mla":
        num_kv_heads = 1
    head_dim_v = head_dim if head_dim_v is None else head_dim_v
    rng = np.random.default_rng(seed)
    if callable(context_lens):
        ctx = np.asarray(context_lens(rng), dtype=np.int64)
    else:
        ctx = np.asarray(context_lens, dtype=np.int64)
    ctx = ctx.reshape(batch).astype(np.int32)
    n_pages = (ctx.astype(np.int64) + block_size - 1) // block_size
    need = int(n_pages.max()) if batch else 0
    max_blocks = max(1, need) if max_blocks_per_seq is None else max_blocks_per_seq
    if max_blocks < need:
        raise ValueError("max_blocks_per_seq too small for the context lengths")
    total = int(n_pages.sum())
    nb = max(1, total) if num_blocks is None else num_blocks
    bt, page_ids = _assign_pages(rng, n_pages, nb, max_blocks)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)

    dq = head_dim
    if q_len > 1:
        q = _Draw(rng).normal(batch * q_len * num_q_heads * dq, dtype).reshape(
            batch, q_len, num_q_heads, dq)
    else:
        q = _Draw(rng).normal(batch * num_q_heads * dq, dtype).reshape(batch, num_q_heads, dq)
    inp = PagedDecodeInputs(name=name, kind=kind, dtype=dtype, batch=batch,
                            num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                            head_dim=head_dim, head_dim_v=head_dim_v, block_size=block_size,
                            num_blocks=nb, scale=float(scale), context_lens=ctx,
                            block_table=bt, page_ids=page_ids, q=q, meta=dict(meta or {}),
                            kv_dtype="fp8" if fp8 else None,
                            k_scale=float(k_scale) if fp8 else 1.0,
                            v_scale=float(v_scale) if fp8 else 1.0)
    if not values:
        return inp

    nan = np.float32("nan") if dtype == "f32" else np.uint16(BF16_NAN_BITS)
    # Tail mask in logical order: [n_used][bs], True where the slot is past ctx.
    tail = np.zeros((total, block_size), dtype=bool)
    off = 0
    for b in range(batch):
        n = int(n_pages[b])
        if n:
            used = int(ctx[b]) - (n - 1) * block_size
            tail[off + n - 1, used:] = True
        off += n

    if kind == "mla":
        if fp8:        # one code row per token, codes of value / k_scale
            nan = np.uint8(FP8_NAN_CODE)
            c = _Draw(rng).normal_fp8(total * block_size * dq, k_scale)
        else:
            c = _Draw(rng).normal(total * block_size * dq, dtype)
        c = c.reshape(total, block_size, dq)
        if poison:
            c[tail] = nan
        inp.c_pages = c
        return inp

    hkv, dv = num_kv_heads, head_dim_v
    # Drawn token-major ([page][slot][head][dim], logical order), then laid out.
    if fp8:
        nan = np.uint8(FP8_NAN_CODE)
        k = _Draw(rng).normal_fp8(total * block_size * hkv * dq, k_scale)
    else:
        k = _Draw(rng).normal(total * block_size * hkv * dq, dtype)
    k = k.reshape(total, block_size, hkv, dq)
    if poison:
        k[tail] = nan
    inp.k_pages = np.ascontiguousarray(k.transpose(0, 2, 1, 3))   # [n][Hkv][bs][D]
    del k
    if fp8:
        v = _Draw(rng).normal_fp8(total * block_size * hkv * dv, v_scale)
    else:
        v = _Draw(rng).normal(total * block_size * hkv * dv, dtype)
    v = v.reshape(total, block_size, hkv, dv)
    if poison:
        v[tail] = nan
    inp.v_pages = np.ascontiguousarray(v.transpose(0, 2, 3, 1))   # [n][Hkv][Dv][bs]
    return inp


# ---------------------------------------------------------------------------
# The five benchmark workloads (shapes, dtypes, length mixes and pools).
# ---------------------------------------------------------------------------

def _uniform_ctx(lo, hi, n):
    return lambda rng: rng.integers(lo, hi, n, endpoint=True)


def _loguniform_ctx(lo, hi, n):
    return lambda rng: np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), n)))


CONFIGS = {
    "tiny_mha_f32": dict(
        kind="mha", dtype="f32", batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64,
        block_size=16, context_lens=[512], num_blocks=32, scale=1.0 / 8.0, seed=1,
        meta=dict(num_splits=[1, 4],
                  desc="tiny MHA fp32: B1, 8 heads, D64, ctx 512, bs16, 32 permuted pages")),
    "llama_mha_bf16": dict(
        kind="mha", dtype="bf16", batch=16, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, context_lens=_uniform_ctx(1024, 4096, 16), num_blocks=65536,
        max_blocks_per_seq=256, scale=1.0 / math.sqrt(128), seed=2,
        meta=dict(desc="Llama-style MHA bf16: B16, 32 heads, D128, ctx U[1024,4096], bs16, 65536-page pool")),
    "long_gqa_bf16": dict(
        kind="mha", dtype="bf16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, context_lens=[131072], num_blocks=8192, scale=1.0 / math.sqrt(128), seed=3,
        meta=dict(desc="long-context GQA bf16: B1, 32 q / 8 kv heads, D128, ctx 131072, bs16")),
    "ragged_gqa_bf16": dict(
        kind="mha", dtype="bf16", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
        block_size=16, context_lens=_loguniform_ctx(128, 32768, 64), num_blocks=65536,
        max_blocks_per_seq=2048, scale=1.0 / math.sqrt(128), seed=4,
        meta=dict(desc="ragged GQA bf16: 64 seqs, ctx log-U[128,32768], 64 q / 8 kv heads, D128, bs16")),
    "mla_bf16": dict(
        kind="mla", dtype="bf16", batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, block_size=64, context_lens=[8192] * 32, num_blocks=4096,
        scale=1.0 / math.sqrt(192), seed=5,
        meta=dict(desc="MLA latent bf16: B32, 128 heads, latent 576 (V = first 512), ctx 8192, bs64")),
    # Token-index lists over a latent cache (one-token pages): each sequence
    # attends to 1152 scattered entries (a top-1024 selection plus a 128-entry
    # window), or densely to 8192 entries, out of a pool of 32 x 8192 rows.
    "mla_topk_bf16": dict(
        kind="mla", dtype="bf16", batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, block_size=1, context_lens=[1152] * 32, num_blocks=262144,
        scale=1.0 / math.sqrt(192), seed=6,
        meta=dict(desc="MLA latent bf16 over token-index lists: B32, 128 heads, 1152 entries "
                       "per sequence (top-1024 + 128-window stand-in), bs1, 262144-row pool")),
    "mla_allentries_bf16": dict(
        kind="mla", dtype="bf16", batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, block_size=1, context_lens=[8192] * 32, num_blocks=262144,
        scale=1.0 / math.sqrt(192), seed=7,
        meta=dict(desc="MLA latent bf16 over token-index lists: B32, 128 heads, 8192 entries "
                       "per sequence (every entry), bs1, 262144-row pool")),
    # Several query rows per sequence (the last q_len tokens, causal): draft
    # verification / chunked prefill over caches shaped like the decode
    # workloads above (same seeds, so the same lengths and pages; the query
    # rows take more draws, so the K/V values that follow them differ).
    "llama_mha_q4_bf16": dict(
        kind="mha", dtype="bf16", batch=16, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, context_lens=_uniform_ctx(1024, 4096, 16), num_blocks=65536,
        max_blocks_per_seq=256, scale=1.0 / math.sqrt(128), seed=2, q_len=4,
        meta=dict(desc="Llama-style MHA bf16, 4 query rows per sequence (causal): B16, 32 heads, "
                       "D128, ctx U[1024,4096], bs16")),
    "long_gqa_q4_bf16": dict(
        kind="mha", dtype="bf16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, context_lens=[131072], num_blocks=8192, scale=1.0 / math.sqrt(128), seed=3,
        q_len=4,
        meta=dict(desc="long-context GQA bf16, 4 query rows (causal): B1, 32 q / 8 kv heads, "
                       "D128, ctx 131072, bs16")),
    "mla_q2_bf16": dict(
        kind="mla", dtype="bf16", batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, block_size=64, context_lens=[8192] * 32, num_blocks=4096,
        scale=1.0 / math.sqrt(192), seed=5, q_len=2,
        meta=dict(desc="MLA latent bf16, 2 query rows per sequence (causal): B32, 128 heads, "
                       "latent 576, ctx 8192, bs64")),
    # FP8 E4M3 caches (bf16 queries, one scale per cache tensor) over the decode
    # workloads' lengths and pages: the same N(0,1) draws, quantised.
    "llama_mha_fp8": dict(
        kind="mha", dtype="bf16", batch=16, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, context_lens=_uniform_ctx(1024, 4096, 16), num_blocks=65536,
        max_blocks_per_seq=256, scale=1.0 / math.sqrt(128), seed=2, kv_dtype="fp8",
        k_scale=0.017, v_scale=0.019,
        meta=dict(desc="Llama-style MHA, FP8 E4M3 KV (bf16 q): B16, 32 heads, D128, "
                       "ctx U[1024,4096], bs16")),
    "long_gqa_fp8": dict(
        kind="mha", dtype="bf16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, context_lens=[131072], num_blocks=8192, scale=1.0 / math.sqrt(128), seed=3,
        kv_dtype="fp8", k_scale=0.017, v_scale=0.019,
        meta=dict(desc="long-context GQA, FP8 E4M3 KV (bf16 q): B1, 32 q / 8 kv heads, D128, "
                       "ctx 131072, bs16")),
    "mla_fp8": dict(
        kind="mla", dtype="bf16", batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, block_size=64, context_lens=[8192] * 32, num_blocks=4096,
        scale=1.0 / math.sqrt(192), seed=5, kv_dtype="fp8", k_scale=0.02, v_scale=0.02,
        meta=dict(desc="MLA latent, FP8 E4M3 cache (bf16 q): B32, 128 heads, latent 576 "
                       "(V = first 512), ctx 8192, bs64")),
    "serving_gqa_bf16": dict(
        kind="mha", dtype="bf16", batch=192, num_q_heads=64, num_kv_heads=8, head_dim=128,
        block_size=16, context_lens=_loguniform_ctx(128, 16384, 192), num_blocks=65536,
        scale=1.0 / math.sqrt(128), seed=7,
        meta=dict(desc="serving-mix GQA bf16: 192 seqs, ctx log-U[128,16384], 64 q / 8 kv heads, "
                       "D128, bs16")),
    "mla_topk_fp8": dict(
        kind="mla", dtype="bf16", batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, block_size=1, context_lens=[1152] * 32, num_blocks=262144,
        scale=1.0 / math.sqrt(192), seed=6, kv_dtype="fp8", k_scale=0.02, v_scale=0.02,
        meta=dict(desc="MLA latent, FP8 E4M3 cache (bf16 q), over token-index lists: B32, "
                       "128 heads, 1152 entries per sequence, bs1, 262144-row pool")),
    "ragged_gqa_fp8": dict(
        kind="mha", dtype="bf16", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
        block_size=16, context_lens=_loguniform_ctx(128, 32768, 64), num_blocks=65536,
        max_blocks_per_seq=2048, scale=1.0 / math.sqrt(128), seed=4, kv_dtype="fp8",
        k_scale=0.017, v_scale=0.019,
        meta=dict(desc="ragged GQA, FP8 E4M3 KV (bf16 q): 64 seqs, ctx log-U[128,32768], "
                       "64 q / 8 kv heads, D128, bs16")),
    # Other head sizes and page sizes on the same kernels: grouped 64-dim heads at long
    # context (a 32 q / 8 kv-head, 64-dim model), the ragged batch on 32-token pages, and
    # 256-dim MHA heads (16 heads of 256).
    "long_gqa_d64_bf16": dict(
        kind="mha", dtype="bf16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=64,
        block_size=16, context_lens=[131072], num_blocks=8192, scale=1.0 / 8.0, seed=3,
        meta=dict(desc="long-context GQA bf16, 64-dim heads: B1, 32 q / 8 kv heads, D64, "
                       "ctx 131072, bs16")),
    "ragged_gqa_bs32_bf16": dict(
        kind="mha", dtype="bf16", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
        block_size=32, context_lens=_loguniform_ctx(128, 32768, 64), num_blocks=32768,
        max_blocks_per_seq=1024, scale=1.0 / math.sqrt(128), seed=4,
        meta=dict(desc="ragged GQA bf16 on 32-token pages: 64 seqs, ctx log-U[128,32768], "
                       "64 q / 8 kv heads, D128, bs32")),
    "llama_mha_d256_bf16": dict(
        kind="mha", dtype="bf16", batch=16, num_q_heads=16, num_kv_heads=16, head_dim=256,
        block_size=16, context_lens=_uniform_ctx(1024, 4096, 16), num_blocks=65536,
        max_blocks_per_seq=256, scale=1.0 / 16.0, seed=2,
        meta=dict(desc="MHA bf16, 256-dim heads: B16, 16 heads, D256, ctx U[1024,4096], bs16, "
                       "65536-page pool")),
}

CONFIG_ORDER = ["tiny_mha_f32", "llama_mha_bf16", "long_gqa_bf16", "ragged_gqa_bf16", "mla_bf16",
                "mla_topk_bf16", "mla_allentries_bf16", "llama_mha_q4_bf16", "long_gqa_q4_bf16",
                "mla_q2_bf16", "llama_mha_fp8", "long_gqa_fp8", "ragged_gqa_fp8", "mla_fp8",
                "mla_topk_fp8", "serving_gqa_bf16", "long_gqa_d64_bf16", "ragged_gqa_bs32_bf16",
                "llama_mha_d256_bf16"]


def make_config(name: str, *, poison: bool = True, values: bool = True, seed: int | None = None,
                **overrides) -> PagedDecodeInputs:
    """Draw one of the named workloads (optionally with fields overridden)."""
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    if seed is not None:
        spec["seed"] = seed
    return make_paged_inputs(name=name, poison=poison, values=values, **spec)
