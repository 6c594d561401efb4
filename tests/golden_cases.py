"""Host arrays for the hand-derived cases in ``golden/closed_forms.json``.

Builds the inputs of each case in the library's storage layouts (no attention
arithmetic here): queries, the K/V or latent pools, block tables and context
lengths, plus the expected outputs written in the file.  Every pool element
the case does not set is NaN (bf16 0x7FC0, FP8 code 0x7F): pages outside the
table, slots past the context and latent rows outside an index list, so any
read the method must not make shows up in the output.
"""

from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bits of values that bfloat16 holds exactly (refuses others)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any((u & 0xFFFF) != 0):
        raise ValueError("value not exact in bfloat16")
    return (u >> 16).astype(np.uint16)


def _sparse(vec: dict, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.float64)
    for k, v in vec.items():
        out[int(k)] = v
    return out


def _dense(vals, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.float64)
    out[:len(vals)] = vals
    return out


@dataclass
class Case:
    spec: dict
    name: str
    kind: str
    dtype: str            # query / output dtype: "f32" or "bf16"
    kv_dtype: str         # cache element type: dtype, or "fp8"
    q: np.ndarray         # storage dtype, [B][Hq][D] or [B][q_len][Hq][D]
    pools: dict           # "k", "v" (MHA) or "c" (MLA), storage dtype
    block_table: np.ndarray
    context_lens: np.ndarray
    scale: float
    k_scale: float
    v_scale: float
    q_len: int
    dv: int
    out: np.ndarray       # expected, float64 [B][q_len][Hq][Dv]
    lse: np.ndarray       # expected, float64 [B][q_len][Hq]


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "bf16":
        bits = np.full(a.shape, BF16_NAN, dtype=np.uint16)
        fin = ~np.isnan(a)
        bits[fin] = bf16_bits(a[fin])
        return bits
    raise ValueError(dtype)


def build(spec: dict) -> Case:
    kind, dtype = spec["kind"], spec["dtype"]
    kvd = spec.get("kv_dtype", dtype)
    B = len(spec["context_lens"])
    L = spec["q_len"]
    Hq, Hkv = spec["num_q_heads"], spec["num_kv_heads"]
    D, bs, nb = spec["head_dim"], spec["block_size"], spec["num_blocks"]
    Dv = spec.get("head_dim_v", D)
    ctx = np.array(spec["context_lens"], dtype=np.int32)
    maxb = max(1, max(len(r) for r in spec["block_tables"]))
    bt = np.zeros((B, maxb), dtype=np.int32)
    for b, row in enumerate(spec["block_tables"]):
        bt[b, :len(row)] = row
    q = np.zeros((B, L, Hq, D))
    for b in range(B):
        for j in range(L):
            for h in range(Hq):
                vec = spec["q_all_heads"] if "q_all_heads" in spec else spec["q"][b][j][h]
                q[b, j, h] = _sparse(vec, D)
    q_store = _store(q if L > 1 else q[:, 0], dtype)

    def place(b, i):
        """(physical page, slot) of token i of sequence b."""
        return spec["block_tables"][b][i // bs], i % bs

    pools = {}
    if kind == "mla":
        if kvd == "fp8":
            c = np.full((nb, bs, D), FP8_NAN, dtype=np.uint8)
            for b in range(B):
                for i, row in enumerate(spec["latent_codes"][b]):
                    p, t = place(b, i)
                    c[p, t] = 0
                    for d, code in row.items():
                        c[p, t, int(d)] = code
            pools["c"] = c
        else:
            c = np.full((nb, bs, D), np.nan)
            for b in range(B):
                for i, row in enumerate(spec["latent"][b]):
                    p, t = place(b, i)
                    c[p, t] = _sparse(row, D)
            pools["c"] = _store(c, dtype)
        # every sequence and head alike; several query rows: one entry per row
        rows_out = spec["out_all_heads"] if L > 1 else [spec["out_all_heads"]]
        rows_lse = spec["lse_all_heads"] if L > 1 else [spec["lse_all_heads"]]
        out = np.zeros((B, L, Hq, Dv))
        lse = np.zeros((B, L, Hq))
        for j in range(L):
            out[:, j] = _dense(rows_out[j], Dv)
            lse[:, j] = -math.inf if rows_lse[j] is None else rows_lse[j]
    else:
        if kvd == "fp8":
            k = np.full((nb, Hkv, bs, D), FP8_NAN, dtype=np.uint8)
            v = np.full((nb, Hkv, Dv, bs), FP8_NAN, dtype=np.uint8)
            for b in range(B):
                for i in range(len(spec["key_codes"][b])):
                    p, t = place(b, i)
                    for g in range(Hkv):
                        k[p, g, t] = 0
                        for d, code in spec["key_codes"][b][i][g].items():
                            k[p, g, t, int(d)] = code
                        codes = spec["value_codes"][b][i][g]
                        v[p, g, :, t] = 0
                        v[p, g, :len(codes), t] = codes
            pools["k"], pools["v"] = k, v
        else:
            k = np.full((nb, Hkv, bs, D), np.nan)
            v = np.full((nb, Hkv, Dv, bs), np.nan)
            for b in range(B):
                for i in range(len(spec["keys"][b])):
                    p, t = place(b, i)
                    for g in range(Hkv):
                        k[p, g, t] = _sparse(spec["keys"][b][i][g], D)
                        v[p, g, :, t] = _dense(spec["values"][b][i][g], Dv)
            pools["k"], pools["v"] = _store(k, dtype), _store(v, dtype)
        out = np.zeros((B, L, Hq, Dv))
        lse = np.zeros((B, L, Hq))
        for b in range(B):
            for j in range(L):
                for h in range(Hq):
                    out[b, j, h] = _dense(spec["out"][b][j][h], Dv)
                    x = spec["lse"][b][j][h]
                    lse[b, j, h] = -math.inf if x is None else x
    return Case(spec=spec, name=spec["name"], kind=kind, dtype=dtype, kv_dtype=kvd, q=q_store,
                pools=pools, block_table=bt, context_lens=ctx, scale=float(spec["scale"]),
                k_scale=float(spec.get("k_scale", 1.0)), v_scale=float(spec.get("v_scale", 1.0)),
                q_len=L, dv=Dv, out=out, lse=lse)


def cases():
    return [build(s) for s in load()["cases"]]


def merges():
    out = []
    for m in load()["merges"]:
        lse_parts = np.array([-math.inf if x is None else x for x in m["lse_parts"]])
        lse = -math.inf if m["lse"] is None else m["lse"]
        out.append((m["name"], np.array(m["o_parts"], dtype=np.float64), lse_parts,
                    np.array(m["out"], dtype=np.float64), lse))
    return out
