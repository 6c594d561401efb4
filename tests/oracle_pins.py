"""Pins that tie the float64 oracle to something other than itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with a brute-force computation, a library routine, a
closed form or an invariant of softmax attention.  They are run against the
real oracle (all must pass) and against planted mistakes (each mistake must
make at least one of them fail).
"""

from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


# --------------------------------------------------------------------------
# Tiny float64 inputs, built directly here (pins do not need the workloads)
# --------------------------------------------------------------------------

def tiny_paged(seed, B, Hq, Hkv, D, Dv, bs, ctxs, extra_pages=3, scale=None):
    rng = np.random.default_rng(seed)
    n_pages = [-(-c // bs) for c in ctxs]
    total = sum(n_pages) + extra_pages
    perm = rng.permutation(total)
    maxb = max(1, max(n_pages))
    bt = np.full((B, maxb), -1, dtype=np.int64)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    k = rng.standard_normal((total, Hkv, bs, D))
    v = rng.standard_normal((total, Hkv, Dv, bs))
    q = rng.standard_normal((B, Hq, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return q, k, v, bt, np.asarray(ctxs, dtype=np.int64), scale


def brute_force(q, k, v, bt, ctxs, scale):
    """Pure-Python softmax attention with explicit page/slot arithmetic."""
    B, Hq, D = q.shape
    _, Hkv, bs, _ = k.shape
    Dv = v.shape[2]
    G = Hq // Hkv
    ql, kl, vl, btl = q.tolist(), k.tolist(), v.tolist(), bt.tolist()
    outs, lses = [], []
    for b in range(B):
        orow, lrow = [], []
        for h in range(Hq):
            g = h // G
            s = []
            for i in range(int(ctxs[b])):
                page, slot = btl[b][i // bs], i % bs
                s.append(scale * math.fsum(ql[b][h][d] * kl[page][g][slot][d] for d in range(D)))
            if not s:
                orow.append([0.0] * Dv)
                lrow.append(-math.inf)
                continue
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            o = []
            for d in range(Dv):
                acc = math.fsum(e[i] * vl[btl[b][i // bs]][g][d][i % bs] for i in range(len(s)))
                o.append(acc / tot)
            orow.append(o)
            lrow.append(m + math.log(tot))
        outs.append(orow)
        lses.append(lrow)
    return np.array(outs), np.array(lses)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin])))
        assert err <= tol, f"{what}: error {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

BRUTE_CASES = [
    # (seed, B, Hq, Hkv, D, Dv, bs, ctxs)
    (10, 1, 1, 1, 4, 4, 4, [7]),
    (11, 2, 2, 2, 8, 8, 16, [33, 1]),
    (12, 3, 4, 2, 5, 3, 2, [9, 0, 4]),
    (13, 2, 4, 1, 6, 6, 1, [5, 12]),
    (14, 1, 4, 4, 8, 8, 4, [40]),
    (15, 2, 3, 1, 3, 7, 16, [16, 17]),
]


def pin_bruteforce(o):
    """P-1: the whole definition against pure-Python loops on tiny inputs."""
    for seed, B, Hq, Hkv, D, Dv, bs, ctxs in BRUTE_CASES:
        q, k, v, bt, ctx, scale = tiny_paged(seed, B, Hq, Hkv, D, Dv, bs, ctxs)
        ref_o, ref_l = brute_force(q, k, v, bt, ctx, scale)
        out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
        _close(out, ref_o, what=f"out case {seed}")
        _close(lse, ref_l, what=f"lse case {seed}")


def pin_mla_bruteforce(o):
    """P-1 for the latent variant: keys are whole latents, values their head."""
    _mla_brute(o, 21, 4, [6, 9])


def pin_mla_token_index_list(o):
    """The latent variant with one-token pages: block_table rows are token-id
    lists (a sparse top-k selection), checked against the brute force."""
    _mla_brute(o, 22, 1, [5, 11])


def _mla_brute(o, seed, bs, ctxs):
    rng = np.random.default_rng(seed)
    B, Hq, Dc, dv = 2, 3, 6, 4
    n_pages = [-(-c // bs) for c in ctxs]
    total = sum(n_pages) + 2
    perm = rng.permutation(total)
    bt = np.full((B, max(n_pages)), -1, dtype=np.int64)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    c = rng.standard_normal((total, bs, Dc))
    q = rng.standard_normal((B, Hq, Dc))
    scale = 0.37
    cl, ql, btl = c.tolist(), q.tolist(), bt.tolist()
    ref_o = np.zeros((B, Hq, dv))
    ref_l = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            rows = [cl[btl[b][i // bs]][i % bs] for i in range(ctxs[b])]
            s = [scale * math.fsum(ql[b][h][d] * r[d] for d in range(Dc)) for r in rows]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            ref_o[b, h] = [math.fsum(e[i] * rows[i][d] for i in range(len(rows))) / tot
                           for d in range(dv)]
            ref_l[b, h] = m + math.log(tot)
    out, lse = o.paged_decode_mla(q, c, bt, np.array(ctxs), scale, dv=dv, dtype="f64")
    _close(out, ref_o, what="mla out")
    _close(lse, ref_l, what="mla lse")


def pin_bf16_widening(o):
    """bf16 bit patterns widen to the exact values bfloat16 defines."""
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC000, 0x3FC0, 0x4049,
                     0x0001, 0x7F7F, 0x7F80, 0xFF80, 0x3E00], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 1.5, 3.140625,
            2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, math.inf, -math.inf, 0.125]
    got = o.as_f64(bits, "bf16")
    assert got.dtype == np.float64
    for g, w in zip(got.tolist(), want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w), (g, w)
    nan = o.as_f64(np.array([0x7FC0], dtype=np.uint16), "bf16")
    assert np.isnan(nan).all()


def pin_sdpa(o):
    """P-2: dense (identity-paged) inputs reduce to torch's SDPA on CPU in float64."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(31)
    for (B, Hq, Hkv, D, bs, ctx) in [(2, 4, 4, 16, 8, 40), (1, 8, 2, 32, 16, 64), (2, 6, 3, 8, 4, 13)]:
        pages = -(-ctx // bs)
        kd = rng.standard_normal((B, Hkv, pages * bs, D))
        vd = rng.standard_normal((B, Hkv, pages * bs, D))
        q = rng.standard_normal((B, Hq, D))
        # identity paging: sequence b owns pages b*pages .. b*pages+pages-1
        k_pool = kd.reshape(B, Hkv, pages, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * pages, Hkv, bs, D)
        v_pool = vd.reshape(B, Hkv, pages, bs, D).transpose(0, 2, 1, 4, 3).reshape(B * pages, Hkv, D, bs)
        bt = np.arange(B * pages).reshape(B, pages)
        ctxs = np.full(B, ctx)
        scale = 1.0 / math.sqrt(D)
        out, _ = o.paged_decode(q, k_pool, v_pool, bt, ctxs, scale, dtype="f64")
        G = Hq // Hkv
        kt = torch.from_numpy(np.ascontiguousarray(kd[:, :, :ctx])).repeat_interleave(G, dim=1)
        vt = torch.from_numpy(np.ascontiguousarray(vd[:, :, :ctx])).repeat_interleave(G, dim=1)
        qt = torch.from_numpy(q).unsqueeze(2)
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale).squeeze(2).numpy()
        _close(out, ref, what=f"sdpa B{B} Hq{Hq} Hkv{Hkv}")


def pin_ctx_one(o):
    """P-3: a one-token context returns that token's value exactly; lse = its score."""
    q, k, v, bt, _, scale = tiny_paged(41, 2, 4, 2, 8, 8, 4, [1, 1])
    ctx = np.array([1, 1])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    for b in range(2):
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[b, h], v[bt[b, 0], g, :, 0]), "ctx=1 out != v0"
            s0 = scale * math.fsum(q[b, h, d] * k[bt[b, 0], g, 0, d] for d in range(8))
            assert abs(lse[b, h] - s0) <= TOL * max(1, abs(s0)), "ctx=1 lse != s0"


def pin_identical_keys(o):
    """P-4: equal keys give the mean of the values and lse = s + ln(ctx)."""
    q, k, v, bt, _, scale = tiny_paged(42, 1, 2, 1, 8, 8, 4, [11])
    k[:] = k[bt[0, 0], 0, 0, :]
    ctx = np.array([11])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    vals = np.stack([v[bt[0, i // 4], 0, :, i % 4] for i in range(11)])
    for h in range(2):
        s = scale * math.fsum(q[0, h, d] * k[0, 0, 0, d] for d in range(8))
        _close(out[0, h], vals.mean(axis=0), what="identical keys out")
        _close(lse[0, h], s + math.log(11), what="identical keys lse")


def pin_two_token_closed_form(o):
    """Two tokens: out = sigma(s0 - s1) v0 + sigma(s1 - s0) v1, lse = ln(e^s0 + e^s1)."""
    D, bs = 4, 2
    a, scale = 2.5, 0.5
    q = np.zeros((1, 1, D)); q[0, 0, 0] = a; q[0, 0, 1] = -1.0
    k = np.zeros((1, 1, bs, D)); k[0, 0, 0, 0] = 1.0; k[0, 0, 1, 1] = 3.0
    v = np.zeros((1, 1, D, bs)); v[0, 0, :, 0] = [1.0, 2.0, 3.0, 4.0]; v[0, 0, :, 1] = [-1.0, 0.5, 0.0, 8.0]
    s0, s1 = scale * a, scale * (-3.0)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    want = [w0 * x + (1 - w0) * y for x, y in zip(v[0, 0, :, 0], v[0, 0, :, 1])]
    out, lse = o.paged_decode(q, k, v, np.array([[0]]), np.array([2]), scale, dtype="f64")
    _close(out[0, 0], want, what="two-token out")
    _close(lse[0, 0], math.log(math.exp(s0) + math.exp(s1)), what="two-token lse")


def pin_split_invariance(o):
    """P-5: the split / partial / merge route equals plain attention for any split."""
    q, k, v, bt, ctx, scale = tiny_paged(43, 3, 4, 2, 8, 6, 4, [37, 1, 16])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    for pps, ns in [(1, None), (2, None), (3, None), (4, 7), (10, None), (1, 16), (100, 3)]:
        so, sl, op, lp = o.paged_decode_split(q, k, v, bt, ctx, scale, dtype="f64",
                                              pages_per_split=pps, num_splits=ns)
        _close(so, out, what=f"split out c={pps}")
        _close(sl, lse, what=f"split lse c={pps}")
        # each partial is itself the attention over its own page range
        for b in range(3):
            pages = -(-int(ctx[b]) // 4)
            for s in range(op.shape[2]):
                p0, p1 = min(pages, s * pps), min(pages, (s + 1) * pps)
                t0, t1 = p0 * 4, min(int(ctx[b]), p1 * 4)
                if t1 <= t0:
                    assert lp[b, 0, s] == -np.inf and not op[b, 0, s].any()
                    continue
                sub_bt = bt[b:b + 1, p0:]
                ref_o, ref_l = brute_force(q[b:b + 1, :1], k[:, :1], v[:, :1], sub_bt,
                                           np.array([t1 - t0]), scale)
                _close(op[b, 0, s], ref_o[0, 0], what="partial out")
                _close(lp[b, 0, s], ref_l[0, 0], what="partial lse")


def pin_page_permutation(o):
    """P-6: relabelling physical pages (and moving their data) changes nothing."""
    q, k, v, bt, ctx, scale = tiny_paged(44, 2, 2, 2, 8, 8, 4, [13, 22], extra_pages=5)
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    perm = np.random.default_rng(45).permutation(k.shape[0])
    k2 = np.empty_like(k); k2[perm] = k
    v2 = np.empty_like(v); v2[perm] = v
    bt2 = np.where(bt >= 0, perm[np.clip(bt, 0, None)], -1)
    out2, lse2 = o.paged_decode(q, k2, v2, bt2, ctx, scale, dtype="f64")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def pin_constant_values(o):
    """P-7: when every value row is the same vector c, the output is c."""
    q, k, v, bt, ctx, scale = tiny_paged(46, 2, 3, 3, 8, 5, 4, [9, 30])
    c = np.array([0.5, -2.0, 3.25, 0.0, 1e-3])
    v[:] = c[None, None, :, None]
    out, _ = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    _close(out, np.broadcast_to(c, out.shape), what="constant values")


def pin_stability(o):
    """P-8: huge scores neither overflow nor lose the dominant token."""
    q, k, v, bt, ctx, scale = tiny_paged(47, 1, 2, 1, 8, 8, 4, [12])
    q *= 1e4
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    for h in range(2):
        s = [scale * float(np.dot(q[0, h], k[bt[0, i // 4], 0, i % 4])) for i in range(12)]
        top = int(np.argmax(s))
        _close(out[0, h], v[bt[0, top // 4], 0, :, top % 4], tol=1e-9, what="dominant token")
        _close(lse[0, h], max(s), tol=1e-9, what="dominant lse")
    # the split route too
    so, sl, _, _ = o.paged_decode_split(q, k, v, bt, ctx, scale, dtype="f64", pages_per_split=1)
    _close(so, out, what="split stability out")
    _close(sl, lse, what="split stability lse")


def pin_score_shift(o):
    """Adding u to every key shifts all scores by scale*<q,u>: out unchanged, lse shifted."""
    q, k, v, bt, ctx, scale = tiny_paged(48, 1, 1, 1, 8, 8, 4, [10])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    u = np.linspace(-1, 1, 8)
    k2 = k + u[None, None, None, :]
    out2, lse2 = o.paged_decode(q, k2, v, bt, ctx, scale, dtype="f64")
    _close(out2, out, tol=1e-11, what="shifted keys out")
    _close(lse2, lse + scale * float(np.dot(q[0, 0], u)), tol=1e-11, what="shifted keys lse")


def pin_gqa_equals_mha(o):
    """P-9a: GQA equals MHA over KV heads repeated G times (contiguous groups)."""
    q, k, v, bt, ctx, scale = tiny_paged(49, 2, 6, 2, 8, 8, 4, [10, 19])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    k_rep = np.repeat(k, 3, axis=1)
    v_rep = np.repeat(v, 3, axis=1)
    out2, lse2 = o.paged_decode(q, k_rep, v_rep, bt, ctx, scale, dtype="f64")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def pin_mla_equals_mqa(o):
    """P-9b: MLA equals single-KV-head attention with K = latent, V = latent[:dv]."""
    rng = np.random.default_rng(50)
    nb, bs, Dc, dv, B, Hq = 6, 4, 10, 6, 2, 5
    c = rng.standard_normal((nb, bs, Dc))
    q = rng.standard_normal((B, Hq, Dc))
    bt = np.array([[3, 1, 4], [0, 5, 2]])
    ctx = np.array([11, 7])
    out, lse = o.paged_decode_mla(q, c, bt, ctx, 0.3, dv=dv, dtype="f64")
    k_pool = c[:, None, :, :]                                   # [nb][1][bs][Dc]
    v_pool = np.ascontiguousarray(c[:, :, :dv].transpose(0, 2, 1))[:, None]   # [nb][1][dv][bs]
    out2, lse2 = o.paged_decode(q, k_pool, v_pool, bt, ctx, 0.3, dtype="f64")
    _close(out, out2, what="mla vs mqa out")
    _close(lse, lse2, what="mla vs mqa lse")


def pin_batch_independence(o):
    """P-10: each sequence alone equals its row of the batched result."""
    q, k, v, bt, ctx, scale = tiny_paged(51, 3, 2, 2, 8, 8, 4, [5, 17, 9])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    for b in range(3):
        o1, l1 = o.paged_decode(q[b:b + 1], k, v, bt[b:b + 1], ctx[b:b + 1], scale, dtype="f64")
        assert np.array_equal(o1[0], out[b]) and np.array_equal(l1[0], lse[b])


def pin_sampled_heads(o):
    """Computing a sample of (b, h) pairs alone gives the same numbers."""
    q, k, v, bt, ctx, scale = tiny_paged(52, 3, 4, 2, 8, 8, 4, [5, 17, 9])
    out, lse = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64")
    pairs = [(0, 3), (2, 0), (2, 1)]
    so, sl = o.paged_decode(q, k, v, bt, ctx, scale, dtype="f64", heads=pairs)
    for b, h in pairs:
        assert np.array_equal(so[b, h], out[b, h]) and sl[b, h] == lse[b, h]


def _nan_equal(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def pin_append_then_decode(o):
    """Append: removing each sequence's last token (NaN in its slot) and
    appending it back restores the pools exactly, and decoding at ctx + 1 then
    matches the pure-Python brute force.  Positions cover a new page (4 with
    bs = 4), a page's last slot (15) and the first token (0)."""
    full = [5, 16, 1]
    q, k, v, bt, ctx, scale = tiny_paged(53, 3, 4, 2, 6, 5, 4, full)
    before = ctx - 1
    k0, v0 = k.copy(), v.copy()
    k_new = np.zeros((3, 2, 6))
    v_new = np.zeros((3, 2, 5))
    for b in range(3):
        n = int(before[b])
        page, slot = bt[b, n // 4], n % 4
        k_new[b], v_new[b] = k[page, :, slot, :], v[page, :, :, slot]
        k0[page, :, slot, :] = np.nan
        v0[page, :, :, slot] = np.nan
    k1, v1 = o.append_kv(k0, v0, bt, before, k_new, v_new)
    assert _nan_equal(k1, k) and _nan_equal(v1, v)
    assert np.isnan(k0).any() and not np.isnan(k1).any()        # the inputs are not modified
    out, lse = o.paged_decode(q, k1, v1, bt, ctx, scale, dtype="f64")
    bo, bl = brute_force(q, k, v, bt, ctx, scale)
    _close(out, bo, what="append out")
    _close(lse, bl, what="append lse")


def pin_append_out_of_range(o):
    """A position past the block table, a negative one, or a -1 table entry
    writes nothing."""
    q, k, v, bt, ctx, scale = tiny_paged(54, 3, 2, 1, 4, 4, 4, [8, 3, 2])
    bt = bt.copy()
    bt[2, 0] = -1
    pos = np.array([8, -1, 1])                 # 8 = 2 pages x 4 slots: table full
    k_new = np.ones((3, 1, 4))
    v_new = np.ones((3, 1, 4))
    k1, v1 = o.append_kv(k, v, bt, pos, k_new, v_new)
    assert np.array_equal(k1, k) and np.array_equal(v1, v)


def pin_append_latent(o):
    """MLA append restores the latent pool, and the latent decode at ctx + 1
    then matches the MQA reading decoded by brute force."""
    rng = np.random.default_rng(55)
    bs, Dc, dv = 4, 6, 4
    full = [4, 7]
    n_pages = [-(-c // bs) for c in full]
    perm = rng.permutation(sum(n_pages) + 2)
    bt = np.full((2, max(n_pages)), -1, dtype=np.int64)
    bt[0, :n_pages[0]] = perm[:n_pages[0]]
    bt[1, :n_pages[1]] = perm[n_pages[0]:n_pages[0] + n_pages[1]]
    c = rng.standard_normal((len(perm), bs, Dc))
    q = rng.standard_normal((2, 3, Dc))
    ctx = np.asarray(full)
    before = ctx - 1
    c0 = c.copy()
    c_new = np.zeros((2, Dc))
    for b in range(2):
        n = int(before[b])
        page, slot = bt[b, n // bs], n % bs
        c_new[b] = c[page, slot]
        c0[page, slot] = np.nan
    c1 = o.append_latent(c0, bt, before, c_new)
    assert _nan_equal(c1, c)
    out, lse = o.paged_decode_mla(q, c1, bt, ctx, 0.4, dv=dv, dtype="f64")
    k = c[:, None, :, :]                                  # MQA: one KV head, K = whole row
    v = np.transpose(c[:, :, :dv], (0, 2, 1))[:, None]    # V = leading dv entries, [D][bs]
    bo, bl = brute_force(q, k, v, bt, ctx, 0.4)
    _close(out, bo, what="latent append out")
    _close(lse, bl, what="latent append lse")


# --------------------------------------------------------------------------
# Several query rows per sequence: the rows are the last q_len tokens and
# row j attends causally to positions 0 .. ctx - q_len + j
# --------------------------------------------------------------------------

ROW_CASES = [
    # (seed, B, q_len, Hq, Hkv, D, Dv, bs, ctxs)
    (50, 2, 3, 4, 2, 6, 6, 4, [7, 3]),          # ctx == q_len for b = 1
    (51, 1, 4, 2, 1, 5, 3, 2, [9]),
    (52, 3, 2, 3, 3, 4, 4, 16, [1, 17, 2]),     # ctx < q_len: row 0 of b = 0 sees nothing
]


def _tiny_rows(seed, B, L, Hq, Hkv, D, Dv, bs, ctxs):
    q0, k, v, bt, ctx, scale = tiny_paged(seed, B, Hq, Hkv, D, Dv, bs, ctxs)
    q = np.random.default_rng(seed + 1000).standard_normal((B, L, Hq, D))
    return q, k, v, bt, ctx, scale


def brute_force_rows(q, k, v, bt, ctxs, scale):
    """Pure-Python causal attention: row j of sequence b sees positions i with
    i <= ctx_b - q_len + j."""
    B, L, Hq, D = q.shape
    _, Hkv, bs, _ = k.shape
    Dv = v.shape[2]
    G = Hq // Hkv
    ql, kl, vl, btl = q.tolist(), k.tolist(), v.tolist(), bt.tolist()
    out = np.zeros((B, L, Hq, Dv))
    lse = np.zeros((B, L, Hq))
    for b in range(B):
        last = int(ctxs[b]) - L          # position of row 0
        for j in range(L):
            for h in range(Hq):
                g = h // G
                vis = [i for i in range(int(ctxs[b])) if i <= last + j]
                if not vis:
                    out[b, j, h] = 0.0
                    lse[b, j, h] = -math.inf
                    continue
                s = [scale * math.fsum(ql[b][j][h][d] * kl[btl[b][i // bs]][g][i % bs][d]
                                       for d in range(D)) for i in vis]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for d in range(Dv):
                    out[b, j, h, d] = math.fsum(e[n] * vl[btl[b][i // bs]][g][d][i % bs]
                                                for n, i in enumerate(vis)) / tot
                lse[b, j, h] = m + math.log(tot)
    return out, lse


def pin_rows_bruteforce(o):
    """Several query rows against pure-Python causal loops on tiny inputs."""
    for case in ROW_CASES:
        q, k, v, bt, ctx, scale = _tiny_rows(*case)
        ref_o, ref_l = brute_force_rows(q, k, v, bt, ctx, scale)
        out, lse = o.paged_decode_rows(q, k, v, bt, ctx, scale, dtype="f64")
        _close(out, ref_o, what=f"rows out case {case[0]}")
        _close(lse, ref_l, what=f"rows lse case {case[0]}")


def pin_rows_sdpa(o):
    """Dense (identity-paged) inputs against torch's SDPA on CPU in float64: a
    fresh prompt (ctx == q_len) with is_causal, and a continuation with the
    equivalent explicit mask."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(53)
    for (B, L, Hq, Hkv, D, bs, ctx) in [(2, 8, 4, 2, 16, 4, 8), (1, 5, 6, 3, 8, 16, 37)]:
        pages = -(-ctx // bs)
        kd = rng.standard_normal((B, Hkv, pages * bs, D))
        vd = rng.standard_normal((B, Hkv, pages * bs, D))
        q = rng.standard_normal((B, L, Hq, D))
        k_pool = kd.reshape(B, Hkv, pages, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * pages, Hkv, bs, D)
        v_pool = vd.reshape(B, Hkv, pages, bs, D).transpose(0, 2, 1, 4, 3).reshape(B * pages, Hkv, D, bs)
        bt = np.arange(B * pages).reshape(B, pages)
        scale = 1.0 / math.sqrt(D)
        out, _ = o.paged_decode_rows(q, k_pool, v_pool, bt, np.full(B, ctx), scale, dtype="f64")
        G = Hq // Hkv
        kt = torch.from_numpy(np.ascontiguousarray(kd[:, :, :ctx])).repeat_interleave(G, dim=1)
        vt = torch.from_numpy(np.ascontiguousarray(vd[:, :, :ctx])).repeat_interleave(G, dim=1)
        qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))     # [B][Hq][L][D]
        if ctx == L:
            ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=True)
        else:
            allowed = torch.arange(ctx)[None, :] <= (ctx - L + torch.arange(L))[:, None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=scale)
        _close(out, ref.numpy().transpose(0, 2, 1, 3), what=f"rows sdpa L{L} ctx{ctx}")


def pin_rows_single_is_decode(o):
    """One query row is the single-token decode, bit for bit; the last of
    several rows sees the whole context and equals the decode of that row."""
    q, k, v, bt, ctx, scale = _tiny_rows(54, 2, 3, 4, 2, 8, 8, 4, [10, 5])
    out1, lse1 = o.paged_decode_rows(q[:, :1], k, v, bt, ctx, scale, dtype="f64")
    ref_o, ref_l = o.paged_decode(np.ascontiguousarray(q[:, 0]), k, v, bt, ctx, scale, dtype="f64")
    assert np.array_equal(out1[:, 0], ref_o) and np.array_equal(lse1[:, 0], ref_l)
    out, lse = o.paged_decode_rows(q, k, v, bt, ctx, scale, dtype="f64")
    ref_o, ref_l = brute_force(np.ascontiguousarray(q[:, 2]), k, v, bt, ctx, scale)
    _close(out[:, 2], ref_o, what="last row out")
    _close(lse[:, 2], ref_l, what="last row lse")


def pin_rows_causality(o):
    """Changing K/V at positions a row cannot see leaves that row unchanged
    (bitwise) and changes the rows that can see them."""
    q, k, v, bt, ctx, scale = _tiny_rows(55, 1, 4, 2, 2, 4, 4, 4, [11])
    base_o, _ = o.paged_decode_rows(q, k, v, bt, ctx, scale, dtype="f64")
    pos = 11 - 4 + 2                       # rows 0, 1 see up to 7, 8; rows 2, 3 see it
    k2, v2 = k.copy(), v.copy()
    page, slot = bt[0][pos // 4], pos % 4
    k2[page, :, slot, :] += 3.0
    v2[page, :, :, slot] -= 5.0
    new_o, _ = o.paged_decode_rows(q, k2, v2, bt, ctx, scale, dtype="f64")
    assert np.array_equal(new_o[0, :2], base_o[0, :2])
    assert not np.allclose(new_o[0, 2:], base_o[0, 2:])


def pin_mla_rows_bruteforce(o):
    """The latent variant with several query rows, 64-token-like pages and
    one-token pages (token-id lists), against pure-Python causal loops."""
    for seed, bs, ctxs, L in ((56, 4, [6, 9], 3), (57, 1, [5, 2], 3)):
        rng = np.random.default_rng(seed)
        B, Hq, Dc, dv = 2, 3, 6, 4
        n_pages = [-(-c // bs) for c in ctxs]
        total = sum(n_pages) + 2
        perm = rng.permutation(total)
        bt = np.full((B, max(n_pages)), -1, dtype=np.int64)
        off = 0
        for b, n in enumerate(n_pages):
            bt[b, :n] = perm[off:off + n]
            off += n
        c = rng.standard_normal((total, bs, Dc))
        q = rng.standard_normal((B, L, Hq, Dc))
        scale = 0.41
        cl, qll, btl = c.tolist(), q.tolist(), bt.tolist()
        ref_o = np.zeros((B, L, Hq, dv))
        ref_l = np.zeros((B, L, Hq))
        for b in range(B):
            for j in range(L):
                vis = [i for i in range(ctxs[b]) if i <= ctxs[b] - L + j]
                for h in range(Hq):
                    if not vis:
                        ref_l[b, j, h] = -math.inf
                        continue
                    r = [cl[btl[b][i // bs]][i % bs] for i in vis]
                    s = [scale * math.fsum(qll[b][j][h][d] * x[d] for d in range(Dc)) for x in r]
                    m = max(s)
                    e = [math.exp(x - m) for x in s]
                    tot = math.fsum(e)
                    ref_o[b, j, h] = [math.fsum(e[i] * r[i][d] for i in range(len(r))) / tot
                                      for d in range(dv)]
                    ref_l[b, j, h] = m + math.log(tot)
        out, lse = o.paged_decode_mla_rows(q, c, bt, np.array(ctxs), scale, dv=dv, dtype="f64")
        _close(out, ref_o, what=f"mla rows out bs{bs}")
        _close(lse, ref_l, what=f"mla rows lse bs{bs}")


# --------------------------------------------------------------------------
# FP8 (E4M3) KV caches with one scale per tensor
# --------------------------------------------------------------------------

def pin_fp8_widening(o):
    """E4M3 codes widen to the values the format defines: known codes, and all
    256 codes against torch's float8_e4m3fn conversion."""
    import torch
    known = {0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x30: 0.5, 0x3C: 1.5,
             0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x0F: 1.875 * 2.0 ** -6, 0x77: 240.0}
    codes = np.array(sorted(known), dtype=np.uint8)
    got = o.as_f64(codes, "fp8")
    for c, g in zip(codes.tolist(), got.tolist()):
        w = known[c]
        assert g == w and math.copysign(1, g) == math.copysign(1, w), (hex(c), g, w)
    for c in (0x7F, 0xFF):
        assert np.isnan(o.as_f64(np.array([c], dtype=np.uint8), "fp8")).all()
    allc = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = o.as_f64(allc, "fp8")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]) and np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def _fp8_codes(rng, shape):
    """Random E4M3 codes, NaN codes excluded."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x3A), c)


def pin_fp8_decode(o):
    """Decode over FP8 caches equals the brute force on the dequantized values
    (codes widened by torch, times their tensor's scale), one and several rows."""
    import torch
    widen = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for seed, L in ((60, 1), (61, 3)):
        _, k, v, bt, ctx, scale = tiny_paged(seed, 2, 4, 2, 8, 8, 4, [9, 5])
        rng = np.random.default_rng(seed)
        kc, vc = _fp8_codes(rng, k.shape), _fp8_codes(rng, v.shape)
        ks, vs = 0.037, 1.9
        q = rng.standard_normal((2, L, 4, 8))
        out, lse = o.paged_decode_rows(q, kc, vc, bt, ctx, scale, dtype="f64", kv_dtype="fp8",
                                       k_scale=ks, v_scale=vs)
        ref_o, ref_l = brute_force_rows(q, widen(kc) * ks, widen(vc) * vs, bt, ctx, scale)
        _close(out, ref_o, what=f"fp8 rows out L{L}")
        _close(lse, ref_l, what=f"fp8 rows lse L{L}")
        if L == 1:
            o1, l1 = o.paged_decode(np.ascontiguousarray(q[:, 0]), kc, vc, bt, ctx, scale,
                                    dtype="f64", kv_dtype="fp8", k_scale=ks, v_scale=vs)
            _close(o1, ref_o[:, 0], what="fp8 out")
            _close(l1, ref_l[:, 0], what="fp8 lse")


def pin_mla_fp8_decode(o):
    """The latent variant over FP8 codes equals pure-Python loops over the
    rows dequantized by torch: keys k_scale times the row, values v_scale
    times its head (one and three query rows)."""
    import torch
    widen = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for seed, L in ((62, 1), (63, 3)):
        rng = np.random.default_rng(seed)
        B, Hq, Dc, dv, bs, ctxs = 2, 3, 6, 4, 4, [6, 9]
        n_pages = [-(-c // bs) for c in ctxs]
        total = sum(n_pages) + 2
        perm = rng.permutation(total)
        bt = np.full((B, max(n_pages)), -1, dtype=np.int64)
        off = 0
        for b, n in enumerate(n_pages):
            bt[b, :n] = perm[off:off + n]
            off += n
        codes = _fp8_codes(rng, (total, bs, Dc))
        ks, vs = 0.037, 1.9
        kd, vd = (widen(codes) * ks).tolist(), (widen(codes) * vs).tolist()
        q = rng.standard_normal((B, L, Hq, Dc))
        scale = 0.43
        qll, btl = q.tolist(), bt.tolist()
        ref_o = np.zeros((B, L, Hq, dv))
        ref_l = np.zeros((B, L, Hq))
        for b in range(B):
            for j in range(L):
                vis = [i for i in range(ctxs[b]) if i <= ctxs[b] - L + j]
                for h in range(Hq):
                    kr = [kd[btl[b][i // bs]][i % bs] for i in vis]
                    vr = [vd[btl[b][i // bs]][i % bs] for i in vis]
                    s_ = [scale * math.fsum(qll[b][j][h][d] * x[d] for d in range(Dc)) for x in kr]
                    m = max(s_)
                    e = [math.exp(x - m) for x in s_]
                    tot = math.fsum(e)
                    ref_o[b, j, h] = [math.fsum(e[i] * vr[i][d] for i in range(len(vr))) / tot
                                      for d in range(dv)]
                    ref_l[b, j, h] = m + math.log(tot)
        out, lse = o.paged_decode_mla_rows(q, codes, bt, np.array(ctxs), scale, dv=dv, dtype="f64",
                                           kv_dtype="fp8", k_scale=ks, v_scale=vs)
        _close(out, ref_o, what=f"mla fp8 rows out L{L}")
        _close(lse, ref_l, what=f"mla fp8 rows lse L{L}")
        if L == 1:
            o1, l1 = o.paged_decode_mla(np.ascontiguousarray(q[:, 0]), codes, bt, np.array(ctxs),
                                        scale, dv=dv, dtype="f64", kv_dtype="fp8", k_scale=ks,
                                        v_scale=vs)
            _close(o1, ref_o[:, 0], what="mla fp8 out")
            _close(l1, ref_l[:, 0], what="mla fp8 lse")


ALL_PINS = [
    pin_bruteforce, pin_mla_bruteforce, pin_mla_token_index_list, pin_bf16_widening, pin_sdpa,
    pin_ctx_one,
    pin_identical_keys, pin_two_token_closed_form, pin_split_invariance,
    pin_page_permutation, pin_constant_values, pin_stability, pin_score_shift,
    pin_gqa_equals_mha, pin_mla_equals_mqa, pin_batch_independence, pin_sampled_heads,
    pin_append_then_decode, pin_append_out_of_range, pin_append_latent,
    pin_rows_bruteforce, pin_rows_sdpa, pin_rows_single_is_decode, pin_rows_causality,
    pin_mla_rows_bruteforce, pin_fp8_widening, pin_fp8_decode, pin_mla_fp8_decode,
]
