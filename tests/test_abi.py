"""The C ABI on the host: the library loads, exports every declared entry point,
and rejects bad arguments before touching the GPU.

No call here reaches a kernel launch: every call either fails validation or
is a host-only query with an explicit CU count / split count.
"""

import ctypes
import math
import os
import re

import pytest

from decode_attention_paged_amd import _lib
from decode_attention_paged_amd._lib import PaShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_decode.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails before any use
NULL = ctypes.c_void_p(0)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libpa_decode.so not built")
    return _lib.load()


def shape(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128, head_dim_v=128,
                block_size=16, max_blocks_per_seq=8, num_blocks=64, max_context_len=100,
                scale=128 ** -0.5, dtype=_lib.PA_BF16)
    base.update(kw)
    return PaShape(**base)


def decode(lib, s, *, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, ctx=FAKE, splits=1, out=FAKE, ws=NULL,
           ws_bytes=0):
    return lib.pa_decode(ctypes.byref(s) if s is not None else None, q, k, v, bt, ctx, splits, out,
                         NULL, ws, ws_bytes, NULL)


def test_header_and_binding_agree():
    assert header_functions() == sorted(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(6):
        assert _lib.status_string(code)
    assert _lib.status_string(99) == "unknown status"
    assert lib.pa_version() >= 100


def test_shape_struct_matches_header(tmp_path):
    """The ctypes struct has the header's size and field offsets (checked by
    compiling the header with the host C compiler)."""
    import shutil
    import subprocess
    assert ctypes.sizeof(PaShape) == 15 * 4       # 12 int32 fields + three floats, no padding
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    names = [f[0] for f in PaShape._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "pa_decode.h"\n'
                   'int main(void) {\n  printf("%zu\\n", sizeof(pa_shape));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(pa_shape, {n}));\n' for n in names)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(PaShape)
    assert got[1:] == [getattr(PaShape, n).offset for n in names]


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("num_q_heads", 0), ("num_kv_heads", 0), ("head_dim", -1), ("block_size", 0),
    ("max_blocks_per_seq", 0), ("num_blocks", 0), ("max_context_len", -5), ("dtype", 7),
    ("num_kv_heads", 3),            # 8 % 3 != 0
    ("max_context_len", 8 * 16 + 1),  # longer than the block table allows
    ("scale", math.inf), ("scale", 0.0), ("scale", -0.125), ("scale", math.nan),
    ("q_len", -1),
    ("kv_dtype", 7),                # not a cache dtype
    ("kv_dtype", -1),
])
def test_invalid_shapes(lib, field, value):
    assert decode(lib, shape(**{field: value})) == _lib.PA_ERR_INVALID


def test_null_shape_and_pointers(lib):
    assert decode(lib, None) == _lib.PA_ERR_INVALID
    s = shape()
    for kw in ("q", "k", "v", "bt", "ctx", "out"):
        assert decode(lib, s, **{kw: NULL}) == _lib.PA_ERR_INVALID, kw


@pytest.mark.parametrize("kw", [
    dict(head_dim=96, head_dim_v=96),                   # no kernel for D = 96
    dict(head_dim=128, head_dim_v=64),                  # Dv != D for MHA
    dict(block_size=8, max_context_len=50),             # no kernel for bs = 8
    dict(q_len=17),                                     # more query rows than any kernel takes
    dict(q_len=2, dtype=_lib.PA_F32),                   # several rows: bf16 MFMA kernel only
    dict(q_len=2, head_dim=256, head_dim_v=256),        # several rows: head_dim 64 or 128 only
    dict(q_len=5, num_kv_heads=2),                      # G = 4 heads x 5 rows: 20 > 16 columns
    dict(max_context_len=(1 << 29) + 16, max_blocks_per_seq=(1 << 25) + 1),  # past 2^29 tokens
    dict(num_q_heads=1 << 16, num_kv_heads=1 << 16, batch=65535),             # rows past 2^31
    dict(kv_dtype=_lib.PA_FP8_E4M3, k_scale=0.1, v_scale=0.1, dtype=_lib.PA_F32),   # FP8: bf16 q
    # FP8 with 256-dim heads: one query row only (the VALU kernel)
    dict(kv_dtype=_lib.PA_FP8_E4M3, k_scale=0.1, v_scale=0.1, head_dim=256, head_dim_v=256,
         q_len=2),
])

def test_unsupported(lib, kw):
    assert decode(lib, shape(**kw)) == _lib.PA_ERR_UNSUPPORTED


@pytest.mark.parametrize("ks,vs", [(0.0, 1.0), (1.0, -1.0), (math.nan, 1.0), (1.0, math.inf)])
def test_fp8_scales_checked(lib, ks, vs):
    s = shape(kv_dtype=_lib.PA_FP8_E4M3, k_scale=ks, v_scale=vs)
    assert decode(lib, s) == _lib.PA_ERR_INVALID


def test_fp8_shapes_pass_validation(lib):
    """FP8 caches with bf16 queries validate (the workspace check fails first,
    so nothing launches); an explicit cache dtype equal to the query's is the
    default; FP8 latent caches take the bf16 latent shapes."""
    for kw in (dict(), dict(num_kv_heads=2), dict(q_len=2), dict(block_size=32, max_context_len=200)):
        s = shape(kv_dtype=_lib.PA_FP8_E4M3, k_scale=0.02, v_scale=3.0, **kw)
        assert decode(lib, s, splits=4) == _lib.PA_ERR_WORKSPACE, kw
    assert decode(lib, shape(kv_dtype=_lib.PA_BF16), splits=4) == _lib.PA_ERR_WORKSPACE
    def mla(**kw):
        base = dict(num_q_heads=128, num_kv_heads=1, head_dim=576, head_dim_v=512, block_size=64,
                    max_context_len=300, kv_dtype=_lib.PA_FP8_E4M3, k_scale=0.1, v_scale=0.1)
        base.update(kw)
        m = shape(**base)
        return lib.pa_decode_mla(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, 4, FAKE, NULL, NULL, 0,
                                 NULL)
    for kw in (dict(), dict(num_q_heads=256), dict(q_len=2), dict(num_q_heads=64),
               dict(num_q_heads=16), dict(num_q_heads=32), dict(block_size=1, max_blocks_per_seq=300)):
        assert mla(**kw) == _lib.PA_ERR_WORKSPACE, kw
    for kw in (dict(num_q_heads=48), dict(block_size=16, max_blocks_per_seq=20),
               dict(dtype=_lib.PA_F32)):
        assert mla(**kw) == _lib.PA_ERR_UNSUPPORTED, kw


def test_several_rows_supported(lib):
    """Several query rows pass validation (explicit split count, no launch: the
    workspace check fails first) and the workspace holds a row per (b, j, h)."""
    for kw in (dict(q_len=2), dict(q_len=16), dict(q_len=4, num_kv_heads=2)):
        s = shape(**kw)
        assert decode(lib, s, splits=4) == _lib.PA_ERR_WORKSPACE, kw
        up = lambda x: -(-x // 256) * 256
        rows = 2 * kw["q_len"] * 8
        # counters, float32 partials, their lse (units of 2 pages: no unit order)
        assert lib.pa_decode_workspace_size(ctypes.byref(s), 4, 0) == \
            up(rows * 4 * 128 * 4) + up(rows * 4 * 4) + up(rows * 4), kw
        # q_len = 0 and 1 both mean one row
    assert lib.pa_decode_workspace_size(ctypes.byref(shape(q_len=0)), 4, 0) == \
        lib.pa_decode_workspace_size(ctypes.byref(shape(q_len=1)), 4, 0)
    # several rows never fuse the merge into the partial kernel
    assert lib.pa_decode_launches(ctypes.byref(shape(q_len=2)), 2, 0) == 2


def test_unit_order_region(lib):
    """Several sequences on the grouped-query kernel with units of >= 384 KiB
    of KV get a unit-order table (one u32 per (sequence, split)) after the
    partials; one sequence, smaller units, or the VALU kernel do not."""
    up = lambda x: -(-x // 256) * 256
    def size(**kw):
        base = dict(batch=4, num_q_heads=16, num_kv_heads=2, max_context_len=6400,
                    max_blocks_per_seq=400)
        base.update(kw)
        s = shape(**base)
        return lib.pa_decode_workspace_size(ctypes.byref(s), 4, 0), s
    def plain(B, Hq, S, Dv=128):
        rows = B * Hq
        return up(rows * 4) + up(rows * S * Dv * 4) + up(rows * S * 4)
    # 400 pages, S = 4: c = 100 pages x 16 tokens x 512 B = 800 KiB per unit
    n, _ = size()
    assert n == plain(4, 16, 4) + up(4 * 4 * 4)
    # FP8 halves the unit: 400 KiB, still scheduled
    n, _ = size(kv_dtype=_lib.PA_FP8_E4M3, k_scale=0.1, v_scale=0.1)
    assert n == plain(4, 16, 4) + up(4 * 4 * 4)
    # units of 25 pages (200 KiB): plain order
    n, s = size(max_context_len=1600, max_blocks_per_seq=100)
    assert n == plain(4, 16, 4)
    # one sequence: plain order
    n, s = size(batch=1)
    assert n == plain(1, 16, 4)
    # MHA on the VALU kernel: plain order
    n, s = size(num_kv_heads=16)
    assert n == plain(4, 16, 4)


def test_workspace_checks(lib):
    s = shape()
    assert decode(lib, s, splits=4) == _lib.PA_ERR_WORKSPACE
    need = lib.pa_decode_workspace_size(ctypes.byref(s), 4, 0)
    rows = 2 * 8 * 4
    up = lambda x: -(-x // 256) * 256
    # one arrival counter per (sequence, head) | o partials | lse partials
    assert need == up(2 * 8 * 4) + up(rows * 128 * 4) + up(rows * 4)
    assert decode(lib, s, splits=4, ws=FAKE, ws_bytes=need - 1) == _lib.PA_ERR_WORKSPACE
    # one split needs no workspace
    assert lib.pa_decode_workspace_size(ctypes.byref(s), 1, 0) == 0


def test_mla_workspace_layout(lib):
    """MLA partials are bfloat16: counters | o partials (2 bytes each) | float32 lse."""
    s = shape(num_q_heads=128, num_kv_heads=1, head_dim=576, head_dim_v=512, block_size=64,
              max_context_len=300)
    rows = 2 * 128
    up = lambda x: -(-x // 256) * 256
    assert lib.pa_decode_workspace_size(ctypes.byref(s), 4, 1) == \
        up(rows * 4) + up(rows * 4 * 512 * 2) + up(rows * 4 * 4)


def test_workspace_init_checks(lib):
    s = shape()
    init = lambda sh, ws, n, splits=4: lib.pa_workspace_init(ctypes.byref(sh), splits, 0, ws, n, NULL)
    need = lib.pa_decode_workspace_size(ctypes.byref(s), 4, 0)
    assert init(s, NULL, 0) == _lib.PA_ERR_WORKSPACE
    assert init(s, FAKE, need - 1) == _lib.PA_ERR_WORKSPACE
    assert init(shape(batch=0), FAKE, need) == _lib.PA_ERR_INVALID
    assert init(s, NULL, 0, splits=1) == _lib.PA_OK     # one split: nothing to initialise


def test_mla_checks(lib):
    s = shape(num_q_heads=128, num_kv_heads=1, head_dim=576, head_dim_v=512, block_size=64,
              max_context_len=300, max_blocks_per_seq=8)
    mla = lambda sh, **kw: lib.pa_decode_mla(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, 1,
                                             kw.get("out", FAKE), NULL, NULL, 0, NULL)
    assert mla(shape(num_q_heads=128, num_kv_heads=2, head_dim=576, head_dim_v=512,
                     block_size=64, max_context_len=300, max_blocks_per_seq=8)) == _lib.PA_ERR_INVALID
    assert mla(shape(num_q_heads=120, num_kv_heads=1, head_dim=576, head_dim_v=512,
                     block_size=64, max_context_len=300, max_blocks_per_seq=8)) == _lib.PA_ERR_UNSUPPORTED
    assert mla(s, out=NULL) == _lib.PA_ERR_INVALID
    assert lib.pa_decode_mla(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 3, FAKE, NULL, NULL, 0,
                             NULL) == _lib.PA_ERR_WORKSPACE


def test_reduce_checks(lib):
    s = shape()
    assert lib.pa_reduce(ctypes.byref(s), NULL, 4, 0, FAKE, 1 << 20, FAKE, NULL, NULL) == _lib.PA_ERR_INVALID
    assert lib.pa_reduce(ctypes.byref(s), FAKE, 4, 0, NULL, 0, FAKE, NULL, NULL) == _lib.PA_ERR_WORKSPACE
    # a single split has nothing to reduce
    assert lib.pa_reduce(ctypes.byref(s), FAKE, 1, 0, NULL, 0, FAKE, NULL, NULL) == _lib.PA_OK


def _splits(lib, mla=False, **kw):
    s = shape(**kw)
    return lib.pa_choose_num_splits(ctypes.byref(s), 256, int(mla))


def test_split_heuristic_fills_the_gpu(lib):
    # long context, 8 KV heads, one sequence: must split, one workgroup per CU
    # (fewer units than CUs: 8-wave workgroups with 2 MiB splits)
    S = _splits(lib, batch=1, num_q_heads=32, num_kv_heads=8, max_context_len=131072,
                max_blocks_per_seq=8192, num_blocks=8192)
    assert 32 <= S <= 8192
    assert S * 8 >= 256                        # at least one workgroup per CU
    # Llama-style MHA batch of 16 x 32 heads, contexts up to 4096
    S2 = _splits(lib, batch=16, num_q_heads=32, num_kv_heads=32, max_context_len=4096,
                 max_blocks_per_seq=256, num_blocks=65536)
    assert 2 <= S2 <= 256
    # ragged GQA batch of 64 up to 30011 tokens
    S3 = _splits(lib, batch=64, num_q_heads=64, num_kv_heads=8, max_context_len=30011,
                 max_blocks_per_seq=2048, num_blocks=65536)
    assert S3 * 64 * 8 <= 64 * 256 and S3 >= 8
    # MLA: 32 sequences of 8192 tokens, 64-token pages, 128 heads in two 64-head workgroups
    S4 = _splits(lib, mla=True, batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576,
                 head_dim_v=512, block_size=64, max_context_len=8192, max_blocks_per_seq=128,
                 num_blocks=4096)
    assert S4 * 32 * 2 >= 256 and S4 <= 128
    # a single page never splits
    assert _splits(lib, max_context_len=16) == 1
    assert _splits(lib, max_context_len=0) == 1


def test_split_heuristic_tiny_problem_is_one_launch(lib):
    """A problem far too small to fill the CUs (1 sequence, 8 heads of 64 dims,
    512 float32 tokens: 2 MiB) is not cut into CU-filling slivers: no split
    reads less than 32 KiB, and the few splits merge in-kernel (one launch)."""
    s = shape(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64, head_dim_v=64,
              max_context_len=512, max_blocks_per_seq=32, num_blocks=32, scale=0.125,
              dtype=_lib.PA_F32)
    S = lib.pa_choose_num_splits(ctypes.byref(s), 256, 0)
    unit_bytes = 512 * 64 * 2 * 4                # one head's K and V
    assert S >= 2 and unit_bytes / S >= 32 * 1024
    assert lib.pa_decode_launches(ctypes.byref(s), S, 0) == 1
    # grouped heads: no split reads less than 64 KiB
    g = shape(batch=1, num_q_heads=32, num_kv_heads=8, max_context_len=1024,
              max_blocks_per_seq=64, num_blocks=64)
    Sg = lib.pa_choose_num_splits(ctypes.byref(g), 256, 0)
    assert 1024 * 128 * 2 * 2 / Sg >= 64 * 1024


def test_split_heuristic_invalid_shape(lib):
    s = shape(batch=0)
    assert lib.pa_choose_num_splits(ctypes.byref(s), 256, 0) == 0


# ----------------------------------------------------------------------------
# Paged KV append: validation only (no launch)
# ----------------------------------------------------------------------------

def append(lib, s, *, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE):
    return lib.pa_append_kv(ctypes.byref(s) if s is not None else None, kn, vn, kc, vc, bt, ctx,
                            NULL)


def append_latent(lib, s, *, cn=FAKE, cc=FAKE, bt=FAKE, ctx=FAKE):
    return lib.pa_append_latent(ctypes.byref(s) if s is not None else None, cn, cc, bt, ctx, NULL)


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("num_kv_heads", 0), ("head_dim", 0), ("head_dim_v", -3), ("block_size", 0),
    ("max_blocks_per_seq", 0), ("num_blocks", 0), ("dtype", 5),
])
def test_append_invalid_shapes(lib, field, value):
    assert append(lib, shape(**{field: value})) == _lib.PA_ERR_INVALID


def test_append_null_pointers(lib):
    assert append(lib, None) == _lib.PA_ERR_INVALID
    s = shape()
    for kw in ("kn", "vn", "kc", "vc", "bt", "ctx"):
        assert append(lib, s, **{kw: NULL}) == _lib.PA_ERR_INVALID, kw
    ms = shape(num_q_heads=16, num_kv_heads=1, head_dim=576, head_dim_v=512, block_size=64)
    assert append_latent(lib, None) == _lib.PA_ERR_INVALID
    for kw in ("cn", "cc", "bt", "ctx"):
        assert append_latent(lib, ms, **{kw: NULL}) == _lib.PA_ERR_INVALID, kw
    # the latent pool has one KV head
    assert append_latent(lib, shape(num_kv_heads=2, num_q_heads=2)) == _lib.PA_ERR_INVALID
    # FP8 latent rows only in the layout the FP8 latent decode reads
    for kw in (dict(head_dim=512, head_dim_v=512), dict(block_size=16)):
        base = dict(num_q_heads=1, num_kv_heads=1, head_dim=576, head_dim_v=576, block_size=64,
                    kv_dtype=_lib.PA_FP8_E4M3)
        base.update(kw)
        assert append_latent(lib, shape(**base)) == _lib.PA_ERR_UNSUPPORTED, kw


def test_append_grid_limits(lib):
    assert append(lib, shape(batch=70000)) == _lib.PA_ERR_UNSUPPORTED
    assert append(lib, shape(num_kv_heads=70000, num_q_heads=70000)) == _lib.PA_ERR_UNSUPPORTED


def test_decode_launches(lib):
    """One launch when the splits merge in-kernel (small per-unit partials) or
    S == 1; two when a reduction launch follows; three with the unit-order
    launch; 0 for a bad shape."""
    def n(s, S, mla=0):
        return lib.pa_decode_launches(ctypes.byref(s), S, mla)
    mha = shape(batch=16, num_q_heads=32, num_kv_heads=32, max_context_len=4096,
                max_blocks_per_seq=256, num_blocks=65536)
    assert n(mha, 1) == 1
    assert n(mha, 4) == 1                        # 4 x 1 head x 129 x 4 B = 2 KiB per unit
    assert n(mha, 16) == 2                       # 8 KiB: separate reduction
    gqa = shape(batch=1, num_q_heads=32, num_kv_heads=8, max_context_len=131072,
                max_blocks_per_seq=8192, num_blocks=8192)
    assert n(gqa, 2) == 2                        # 2 x 4 heads x 129 x 4 B: just over 4 KiB
    assert n(gqa, 64) == 2
    mla = shape(batch=32, num_q_heads=128, num_kv_heads=1, head_dim=576, head_dim_v=512,
                block_size=64, max_context_len=8192, max_blocks_per_seq=128, num_blocks=4096)
    assert n(mla, 4, 1) == 2 and n(mla, 1, 1) == 1
    # several sequences with units of >= 384 KiB: the unit-order launch first
    ragged = shape(batch=64, num_q_heads=64, num_kv_heads=8, max_context_len=32768,
                   max_blocks_per_seq=2048, num_blocks=65536)
    assert n(ragged, 10) == 3                    # 205 pages x 8 KiB per unit
    assert n(ragged, 64) == 2                    # 32 pages: plain order
    assert n(shape(batch=1, num_q_heads=64, num_kv_heads=8, max_context_len=32768,
                   max_blocks_per_seq=2048, num_blocks=65536), 10) == 2
    assert n(shape(batch=0), 4) == 0


def test_token_index_split_limit(lib):
    """With one-token pages the latent kernel holds at most 2048 token ids per
    split: an explicit split count that needs more is unsupported, and the
    heuristic never picks one."""
    s = shape(batch=1, num_q_heads=128, num_kv_heads=1, head_dim=576, head_dim_v=512,
              block_size=1, max_context_len=5000, max_blocks_per_seq=5000, num_blocks=10000,
              scale=192 ** -0.5)
    st = lib.pa_decode_mla(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 2, FAKE, NULL, FAKE, 1 << 40,
                           NULL)
    assert st == _lib.PA_ERR_UNSUPPORTED              # ceil(5000 / 2) > 2048
    assert lib.pa_choose_num_splits(ctypes.byref(s), 256, 1) >= 3


def test_stream_read_checks(lib):
    """The streaming-read probe validates before launching."""
    sink = FAKE
    assert lib.pa_stream_read(NULL, 1024, sink, NULL) == _lib.PA_ERR_INVALID
    assert lib.pa_stream_read(FAKE, 1024, NULL, NULL) == _lib.PA_ERR_INVALID
    assert lib.pa_stream_read(FAKE, 0, sink, NULL) == _lib.PA_ERR_INVALID
    assert lib.pa_stream_read(FAKE, 1000, sink, NULL) == _lib.PA_ERR_INVALID     # not 16-byte rows
    assert lib.pa_stream_read(ctypes.c_void_p(0x1008), 1024, sink, NULL) == _lib.PA_ERR_INVALID


def test_static_entry_point_checks(lib):
    """pa_decode_static validates like pa_decode and refuses partials beyond its
    64 MiB array before touching the device."""
    def static(s, splits, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, ctx=FAKE, out=FAKE)
        a.update(kw)
        return lib.pa_decode_static(ctypes.byref(s) if s is not None else None, a["q"], a["k"],
                                    a["v"], a["bt"], a["ctx"], splits, a["out"], NULL, NULL)
    assert static(None, 4) == _lib.PA_ERR_INVALID
    assert static(shape(batch=0), 4) == _lib.PA_ERR_INVALID
    for kw in ("q", "k", "v", "bt", "ctx", "out"):
        assert static(shape(), 4, **{kw: NULL}) == _lib.PA_ERR_INVALID, kw
    big = shape(batch=64, num_q_heads=64, num_kv_heads=8, max_context_len=4096,
                max_blocks_per_seq=256, num_blocks=20000)
    assert lib.pa_decode_workspace_size(ctypes.byref(big), 64, 0) > 64 << 20
    assert static(big, 64) == _lib.PA_ERR_SCRATCH
    assert "64 MiB" in _lib.status_string(_lib.PA_ERR_SCRATCH)


def test_split_plan_for_batches_run_longest_first(lib):
    """With the units run longest first, the longest sequence gets 10 splits,
    or 3 when the batch's (sequence, KV head) units fill every workgroup slot
    (two per CU) twice over, and then no split reads less than 512 KiB (a
    short longest sequence is not split at all).  Units that fill the CUs but
    hold at most 4 MiB each are only halved."""
    def S(**kw):
        base = dict(num_q_heads=64, num_kv_heads=8, max_context_len=32768,
                    max_blocks_per_seq=2048, num_blocks=65536)
        base.update(kw)
        s = shape(**base)
        n = lib.pa_choose_num_splits(ctypes.byref(s), 256, 0)
        return n, lib.pa_decode_launches(ctypes.byref(s), n, 0)
    assert S(batch=64) == (10, 3)                       # 512 units: 10 for the longest
    assert S(batch=128) == (3, 3)                       # 1024 units: 3
    assert S(batch=256, max_context_len=8192, max_blocks_per_seq=512) == (3, 3)
    # 128 sequences of at most 1024 tokens (64 pages, 512 KiB): unsplit, one launch
    assert S(batch=128, max_context_len=1024, max_blocks_per_seq=64) == (1, 1)
    # 512 sequences of at most 2048 tokens: two splits of 512 KiB, run longest first
    assert S(batch=512, max_context_len=2048, max_blocks_per_seq=128) == (2, 3)
    # MHA on the VALU kernel (4 workgroups per CU): 64 x 32 units fill the slots twice
    # over, so the longest sequence gets 4 splits; 16 x 32 keep the byte target (16)
    mha = dict(num_q_heads=32, num_kv_heads=32, max_context_len=4096, max_blocks_per_seq=256)
    assert S(batch=64, **mha)[0] == 4
    assert S(batch=16, **mha)[0] == 16
    # units that fill the CUs but are short (the longest at most 4 MiB of KV): halved only
    assert S(batch=16, num_q_heads=32, num_kv_heads=32, q_len=4, max_context_len=4096,
             max_blocks_per_seq=256)[0] == 2               # Llama-style 4-row MHA, 2 MiB
    assert S(batch=32, max_context_len=8192, max_blocks_per_seq=512)[0] == 2    # 256 units, 4 MiB
    assert S(batch=128, num_q_heads=16, num_kv_heads=4, max_context_len=2048,
             max_blocks_per_seq=128)[0] == 2              # 512 units, 1 MiB
    # the same units past 4 MiB keep the long-unit plan (1 MiB splits: 8 here)
    assert S(batch=32, max_context_len=16384, max_blocks_per_seq=1024)[0] == 8
