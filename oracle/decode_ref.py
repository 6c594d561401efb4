"""CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP library and imports nothing from it.

What it computes
----------------
Decode attention is ordinary scaled dot-product softmax attention for one
query row per head (the wenku.it search page for "paged attention", its
"Transformer introduction" snippet, the attention-per-word passage: every
query is scored against every key of the sequence and the scores re-weight
the values; the wenku.it search page for "Multi-head Latent Attention (MLA)",
its Multi-Head Attention passage: h self-attentions side by side, whose
formula the page cuts off at its left-hand side).  Softmax needs a reduction
along the whole row (the "llms-attention" post, its SoftmaxAttn blurb).  The
Flash-Decoding snippets of the "flash decoding ++" entry (the three-step
description and the "main idea" paragraph) state that
splitting K/V into chunks, recording a log-sum-exp per chunk and rescaling
the chunk results gives the same, correct attention output.  So the
reference result is the plain definition, written out in float64:

    for each sequence b, query head h, logical token i < ctx_b
        p_i  = block_table[b][i // bs],  t_i = i % bs,  g = h // (Hq / Hkv)
        s_i  = scale * <q[b,h], k_i>
        out  = sum_i exp(s_i - m) v_i / sum_i exp(s_i - m),  m = max_i s_i
        lse  = m + ln sum_i exp(s_i - m)          (natural log)

``paged_decode_split`` additionally walks the three Flash-Decoding steps in
the order that entry gives (split, per-chunk attention with a running max and sum,
log-sum-exp rescale and merge) so the merge identity itself can be checked.
``paged_decode_mla`` is the latent (MLA) variant of the two search pages and
the FlashMLA-ETAP related-papers page (its MLA abstracts): every
query head attends to one shared latent vector per token; keys are the whole
latent, values its leading ``dv`` entries.

Readings where the pages are silent (each also listed in the design notes):
no mask other than the context length; lse is natural-log of the sum over the
scaled scores; GQA head h reads KV head h // (Hq/Hkv); an empty context gives
out = 0 and lse = -inf; slots past the context and table entries past the
last page are never read.  bf16 inputs are widened bit-exactly (bits << 16).

An FP8 KV cache (the "llms-attention" post names FP8 only as hardware low
precision FlashAttention-3 uses) is read as OCP E4M3 codes with one scale per
tensor: a key is k_scale times its code's value, a value v_scale times its
code's value; queries and outputs keep their own dtype.  An FP8 latent cache
holds one code row per token: the key is k_scale times the whole row, the
value v_scale times its leading dv entries.

Pool layouts (the library's documented layouts):
    k_pool [num_blocks][Hkv][bs][D]
    v_pool [num_blocks][Hkv][Dv][bs]
    c_pool [num_blocks][bs][Dqk]        (MLA latent; V = c[..., :dv])
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Inputs as float64
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns exactly: bits << 16 is the float32 value."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def fp8_e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen FP8 E4M3 codes (OCP layout) exactly: 1 sign, 4 exponent (bias 7)
    and 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is
    NaN; there is no infinity."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign, e, m = b >> 7, (b >> 3) & 15, b & 7
    # normal: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10)
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    v = np.where(sign == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, v)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "fp8":
        return fp8_e4m3_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Paging: logical token -> (physical page, slot)
# --------------------------------------------------------------------------

def token_locations(block_table_row: np.ndarray, ctx: int, bs: int):
    """Physical page and in-page slot of logical tokens 0..ctx-1."""
    i = np.arange(ctx, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[i // bs]
    slots = i % bs
    return pages, slots


def gather_kv(k_pool, v_pool, pages, slots):
    """Rows of every KV head for the given tokens: K [n][Hkv][D], V [n][Hkv][Dv]."""
    k = k_pool[pages, :, slots, :]          # [n][Hkv][D]
    v = v_pool[pages, :, :, slots]          # [n][Hkv][Dv]
    return k, v


def gather_latent(c_pool, pages, slots):
    """Latent rows [n][Dqk] for the given tokens."""
    return c_pool[pages, slots, :]


def latent_kv(c, dv: int):
    """MLA keys and values from latent rows: keys = c, values = c[:, :dv]."""
    return c, c[:, :dv]


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Query head h reads KV head h // G, G = Hq / Hkv (contiguous groups)."""
    return h // (num_q_heads // num_kv_heads)


# --------------------------------------------------------------------------
# Attention of one query row
# --------------------------------------------------------------------------

def scores(q_vec: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s_i = scale * <q, k_i>."""
    return scale * (keys @ q_vec)


def attend(q_vec, keys, values, scale):
    """Plain softmax attention of one query row: (out [Dv], lse)."""
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1], dtype=np.float64), -np.inf
    s = scores(q_vec, keys, scale)
    m = np.max(s)
    p = np.exp(s - m)
    l = np.sum(p)
    out = (p @ values) / l
    return out, m + np.log(l)


# --------------------------------------------------------------------------
# Flash-Decoding steps ("flash decoding ++" entry): split, per-chunk partials, LSE merge
# --------------------------------------------------------------------------

def split_page_ranges(num_pages: int, pages_per_split: int, num_splits: int):
    """Contiguous page ranges [s*c, min((s+1)*c, num_pages)) for s < num_splits."""
    out = []
    for s in range(num_splits):
        p0 = min(num_pages, s * pages_per_split)
        p1 = min(num_pages, (s + 1) * pages_per_split)
        out.append((p0, p1))
    return out


def chunk_partial(q_vec, keys, values, scale, bs: int, tok0: int):
    """One chunk's (o_s, lse_s), computed page by page with a running max/sum.

    keys/values hold the chunk's tokens; tok0 is its first logical token (only
    used to cut the chunk into pages).  The running state is (m, l, acc):
    for each page, m' = max(m, max s), alpha = exp(m - m'), l = alpha*l + sum
    exp(s - m'), acc = alpha*acc + sum exp(s - m') v.  The partial is
    o_s = acc / l and lse_s = m + ln l; an empty chunk gives (0, -inf).
    """
    n = keys.shape[0]
    dv = values.shape[1]
    if n == 0:
        return np.zeros(dv, dtype=np.float64), -np.inf
    m = -np.inf
    l = 0.0
    acc = np.zeros(dv, dtype=np.float64)
    start = 0
    while start < n:
        # tokens up to the next page boundary of the logical sequence
        end = min(n, start + bs - ((tok0 + start) % bs))
        s = scores(q_vec, keys[start:end], scale)
        m_new = max(m, float(np.max(s)))
        alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + np.sum(p)
        acc = alpha * acc + p @ values[start:end]
        m = m_new
        start = end
    return acc / l, m + np.log(l)


def merge_partials(o_parts, lse_parts):
    """Rescale and combine chunk partials: weights exp(lse_s - max lse)."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    big = np.max(lse_parts)
    if not np.isfinite(big):
        return np.zeros(o_parts.shape[1], dtype=np.float64), -np.inf
    w = np.exp(lse_parts - big)
    tot = np.sum(w)
    return (w @ o_parts) / tot, big + np.log(tot)


# --------------------------------------------------------------------------
# Whole-batch entry points
# --------------------------------------------------------------------------

def _check_common(q, block_table, context_lens, bs):
    if q.ndim != 3:
        raise ValueError("q must be [B][Hq][D]")
    if block_table.ndim != 2 or block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table must be [B][max_blocks]")
    ctx = np.asarray(context_lens, dtype=np.int64)
    if ctx.shape != (q.shape[0],) or np.any(ctx < 0):
        raise ValueError("context_lens must be [B], non-negative")
    if np.any((ctx + bs - 1) // bs > block_table.shape[1]):
        raise ValueError("context longer than the block table allows")
    return ctx


def paged_decode(q, k_pool, v_pool, block_table, context_lens, scale, dtype="bf16",
                 heads=None, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Reference decode attention over paged K/V (MHA and GQA).

    Returns (out [B][Hq][Dv], lse [B][Hq]) in float64.  ``heads`` optionally
    restricts the work to a list of (b, h) pairs (others stay NaN), which lets
    a test sample outputs of a large batch one by one.  ``kv_dtype`` is the
    caches' dtype when it differs from the query's ("fp8": E4M3 codes, read
    as k_scale / v_scale times their values).
    """
    kvd = dtype if kv_dtype is None else kv_dtype
    qf = as_f64(q, dtype)
    B, Hq, _ = qf.shape
    nb, Hkv, bs, _ = k_pool.shape
    Dv = v_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    ctx = _check_common(qf, block_table, context_lens, bs)
    out = np.full((B, Hq, Dv), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = None if heads is None else {}
    if heads is not None:
        for b, h in heads:
            want.setdefault(int(b), []).append(int(h))
    for b in range(B):
        if want is not None and b not in want:
            continue
        pages, slots = token_locations(block_table[b], int(ctx[b]), bs)
        k, v = gather_kv(k_pool, v_pool, pages, slots)
        k = as_f64(k, kvd) * k_scale
        v = as_f64(v, kvd) * v_scale
        for h in (range(Hq) if want is None else want[b]):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h], lse[b, h] = attend(qf[b, h], k[:, g, :], v[:, g, :], scale)
    return out, lse


def paged_decode_split(q, k_pool, v_pool, block_table, context_lens, scale, dtype="bf16",
                       pages_per_split=1, num_splits=None):
    """The same result reached through the split / partial / merge steps.

    Sequence b is cut into contiguous page ranges of ``pages_per_split`` pages
    (``num_splits`` ranges; by default just enough to cover the longest
    context, so shorter sequences end with empty ranges).  Also returns the
    partials: (out, lse, o_parts [B][Hq][S][Dv], lse_parts [B][Hq][S]).
    """
    qf = as_f64(q, dtype)
    B, Hq, _ = qf.shape
    nb, Hkv, bs, _ = k_pool.shape
    Dv = v_pool.shape[2]
    ctx = _check_common(qf, block_table, context_lens, bs)
    max_pages = int(((ctx + bs - 1) // bs).max()) if B else 0
    if num_splits is None:
        num_splits = max(1, -(-max_pages // pages_per_split))
    out = np.zeros((B, Hq, Dv))
    lse = np.zeros((B, Hq))
    o_parts = np.zeros((B, Hq, num_splits, Dv))
    l_parts = np.zeros((B, Hq, num_splits))
    for b in range(B):
        n = int(ctx[b])
        pages, slots = token_locations(block_table[b], n, bs)
        k, v = gather_kv(k_pool, v_pool, pages, slots)
        k = as_f64(k, dtype)
        v = as_f64(v, dtype)
        ranges = split_page_ranges(-(-n // bs), pages_per_split, num_splits)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for s, (p0, p1) in enumerate(ranges):
                t0, t1 = p0 * bs, min(n, p1 * bs)
                o_parts[b, h, s], l_parts[b, h, s] = chunk_partial(
                    qf[b, h], k[t0:t1, g, :], v[t0:t1, g, :], scale, bs, t0)
            out[b, h], lse[b, h] = merge_partials(o_parts[b, h], l_parts[b, h])
    return out, lse, o_parts, l_parts


def paged_decode_mla(q, c_pool, block_table, context_lens, scale, dv=512, dtype="bf16",
                     heads=None, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Reference MLA decode: all query heads attend to one latent per token.

    Keys are the full latent rows c_i [Dqk]; values are c_i[:dv] (the same
    stored vector).  ``kv_dtype`` is the latent cache's element type when it
    differs from ``dtype`` ("fp8": E4M3 codes; keys are k_scale times the
    row, values v_scale times its head).  Returns (out [B][Hq][dv],
    lse [B][Hq]) in float64.
    """
    kvd = dtype if kv_dtype is None else kv_dtype
    qf = as_f64(q, dtype)
    B, Hq, Dqk = qf.shape
    nb, bs, Dc = c_pool.shape
    if Dc != Dqk or dv > Dqk:
        raise ValueError("latent width must equal the query width and cover dv")
    ctx = _check_common(qf, block_table, context_lens, bs)
    out = np.full((B, Hq, dv), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = None if heads is None else {}
    if heads is not None:
        for b, h in heads:
            want.setdefault(int(b), []).append(int(h))
    for b in range(B):
        if want is not None and b not in want:
            continue
        pages, slots = token_locations(block_table[b], int(ctx[b]), bs)
        c = as_f64(gather_latent(c_pool, pages, slots), kvd)
        keys, values = latent_kv(c, dv)
        keys, values = keys * k_scale, values * v_scale
        for h in (range(Hq) if want is None else want[b]):
            out[b, h], lse[b, h] = attend(qf[b, h], keys, values, scale)
    return out, lse


# --------------------------------------------------------------------------
# Several query rows per sequence (chunked prefill, draft verification).  The
# pages name the prefill stage and FlashAttention's exact attention over many
# query rows (the FlashMLA-ETAP related-papers page, its FlashAttention
# abstracts; the "llms-attention" post) but give no mask.  Reading taken: the
# q_len rows are the sequence's last q_len tokens, whose K/V are already in
# the cache, and row j (position ctx - q_len + j) attends causally to the
# tokens up to and including its own position.  At q_len = 1 this is the
# decode definition above.
# --------------------------------------------------------------------------

def row_context(ctx: int, q_len: int, j: int) -> int:
    """Tokens that query row j of q_len sees: ctx - q_len + 1 + j, at least 0."""
    return max(0, int(ctx) - q_len + 1 + j)


def _rows_by_j(rows, q_len):
    if rows is None:
        return {j: None for j in range(q_len)}
    by = {}
    for b, j, h in rows:
        by.setdefault(int(j), []).append((int(b), int(h)))
    return by


def paged_decode_rows(q, k_pool, v_pool, block_table, context_lens, scale, dtype="bf16",
                      rows=None, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Reference attention of q_len query rows per sequence over paged K/V.

    q [B][q_len][Hq][D]; returns (out [B][q_len][Hq][Dv], lse [B][q_len][Hq]).
    Row j is the decode of its own query row over the first
    row_context(ctx_b, q_len, j) tokens.  ``rows`` optionally restricts the
    work to (b, j, h) triples (others stay NaN).
    """
    if q.ndim != 4:
        raise ValueError("q must be [B][q_len][Hq][D]")
    B, L, Hq, _ = q.shape
    Dv = v_pool.shape[2]
    ctx = np.asarray(context_lens, dtype=np.int64)
    out = np.full((B, L, Hq, Dv), np.nan)
    lse = np.full((B, L, Hq), np.nan)
    for j, heads in _rows_by_j(rows, L).items():
        ctx_j = np.array([row_context(c, L, j) for c in ctx], dtype=np.int64)
        out[:, j], lse[:, j] = paged_decode(np.ascontiguousarray(q[:, j]), k_pool, v_pool,
                                            block_table, ctx_j, scale, dtype=dtype, heads=heads,
                                            kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale)
    return out, lse


def paged_decode_mla_rows(q, c_pool, block_table, context_lens, scale, dv=512, dtype="bf16",
                          rows=None, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """The latent variant with q_len query rows per sequence (q [B][q_len][Hq][Dqk])."""
    if q.ndim != 4:
        raise ValueError("q must be [B][q_len][Hq][Dqk]")
    B, L, Hq, _ = q.shape
    ctx = np.asarray(context_lens, dtype=np.int64)
    out = np.full((B, L, Hq, dv), np.nan)
    lse = np.full((B, L, Hq), np.nan)
    for j, heads in _rows_by_j(rows, L).items():
        ctx_j = np.array([row_context(c, L, j) for c in ctx], dtype=np.int64)
        out[:, j], lse[:, j] = paged_decode_mla(np.ascontiguousarray(q[:, j]), c_pool, block_table,
                                                ctx_j, scale, dv=dv, dtype=dtype, heads=heads,
                                                kv_dtype=kv_dtype, k_scale=k_scale,
                                                v_scale=v_scale)
    return out, lse


def decode_inputs(inp, heads=None):
    """Run the reference on a workload object (compact pages + compact table).

    For workloads with several query rows (q [B][q_len][Hq][D]) ``heads`` are
    (b, j, h) triples."""
    bt = inp.compact_block_table()
    if inp.q.ndim == 4:
        if inp.kind == "mla":
            return paged_decode_mla_rows(inp.q, inp.c_pages, bt, inp.context_lens, inp.scale,
                                         dv=inp.head_dim_v, dtype=inp.dtype, rows=heads,
                                         **_kv_args(inp))
        return paged_decode_rows(inp.q, inp.k_pages, inp.v_pages, bt, inp.context_lens,
                                 inp.scale, dtype=inp.dtype, rows=heads, **_kv_args(inp))
    if inp.kind == "mla":
        return paged_decode_mla(inp.q, inp.c_pages, bt, inp.context_lens, inp.scale,
                                dv=inp.head_dim_v, dtype=inp.dtype, heads=heads, **_kv_args(inp))
    return paged_decode(inp.q, inp.k_pages, inp.v_pages, bt, inp.context_lens, inp.scale,
                        dtype=inp.dtype, heads=heads, **_kv_args(inp))


def _kv_args(inp):
    """Cache dtype and scales of a workload (none for caches in the query dtype)."""
    kvd = getattr(inp, "kv_dtype", None)
    if kvd is None or kvd == inp.dtype:
        return {}
    return dict(kv_dtype=kvd, k_scale=inp.k_scale, v_scale=inp.v_scale)


# ---------------------------------------------------------------------------
# Paged KV append (the step before decode: the new token's K/V rows go to the
# page and slot its position selects; the "paged attention" search page, its
# vLLM README snippets on KV memory managed in pages through a block table).
# ---------------------------------------------------------------------------

def append_slot(block_table_row: np.ndarray, n: int, bs: int):
    """(page, slot) where the token at position n lives, or None when the
    position is outside the block table or the table entry is negative."""
    if n < 0 or n >= len(block_table_row) * bs:
        return None
    page = int(block_table_row[n // bs])
    if page < 0:
        return None
    return page, n % bs


def append_kv(k_pool, v_pool, block_table, context_lens, k_new, v_new):
    """Copies of the K/V pools with row k_new[b] / v_new[b] written at position
    context_lens[b] of every sequence.  Layouts: k_pool [pages][Hkv][bs][D],
    v_pool [pages][Hkv][Dv][bs]; k_new [B][Hkv][D], v_new [B][Hkv][Dv].  The
    elements are moved as they are (bits for bf16)."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    bs = k_pool.shape[2]
    for b in range(len(context_lens)):
        loc = append_slot(block_table[b], int(context_lens[b]), bs)
        if loc is None:
            continue
        page, slot = loc
        k_out[page, :, slot, :] = k_new[b]
        v_out[page, :, :, slot] = v_new[b]
    return k_out, v_out


def append_latent(c_pool, block_table, context_lens, c_new):
    """MLA: a copy of the latent pool [pages][bs][D] with c_new[b] written at
    position context_lens[b] of every sequence."""
    out = c_pool.copy()
    bs = c_pool.shape[1]
    for b in range(len(context_lens)):
        loc = append_slot(block_table[b], int(context_lens[b]), bs)
        if loc is not None:
            out[loc[0], loc[1], :] = c_new[b]
    return out
