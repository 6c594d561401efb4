"""Plain, slow float64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the library.  It shares no
code with the HIP path.  See ``decode_ref`` for what it computes and the
passages it follows.  Every function here is pinned by ``tests/test_oracle.py``
(brute force, a library routine, closed forms and invariants); none is
"parity unpinned".
"""

from .decode_ref import (  # noqa: F401
    append_kv,
    append_latent,
    append_slot,
    as_f64,
    attend,
    bf16_bits_to_f64,
    chunk_partial,
    decode_inputs,
    fp8_e4m3_bits_to_f64,
    gather_kv,
    gather_latent,
    kv_head_of,
    latent_kv,
    merge_partials,
    paged_decode,
    paged_decode_mla,
    paged_decode_mla_rows,
    paged_decode_rows,
    paged_decode_split,
    row_context,
    scores,
    split_page_ranges,
    token_locations,
)
