"""Plain fp64 CPU oracle for split-KV verify attention over a paged fp8 KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. The oracle shares no code with the
HIP library (no kernels, headers, helpers, tables or pre/post-processing) and
imports nothing from the ``paged_fp8_kv_split_amd`` package.

What it computes (sources: aiter PR #5190 "gfx950 assembly MTP-verify attention
for head_dim 256 fp8 paged KV", sections Motivation, Modifications, Kernel notes
and Supported; SGLang PR #37465 "gfx950 assembly attention for EAGLE verify,
draft extend and decode", Modifications): for every query token of every
sequence, masked softmax attention over that sequence's paged KV cache, with
K/V decoded from fp8 e4m3 bytes and multiplied by their per-tensor descales,
queries attending under a bottom-right causal mask to the last q_len positions,
and G query heads sharing one KV head; optionally the log-sum-exp of each row's
visible scores (aiter PR #7375 "gfx1250 fp8 varlen FMHA", Summary). Split-KV
segmentation is an exact rewrite of these quantities, so the oracle does not
depend on the segment count.

``fp8_model.py`` computes the same attention with Q and P rounded to e4m3 under
power-of-two block scales, the arithmetic class of the pages' fp8 kernel, so
that tests can separate the error that rounding carries from the error an
implementation adds.

The second workload, fp8 varlen prefill attention (aiter PR #7375, Summary:
e4m3 Q/K/V with per-tensor descales, packed THD layout, qk head dim 192 and v
head dim 128, causal aligned to the bottom right or not, optional LSE), is in
``prefill.py``.

Every function here is pinned by ``tests/test_oracle.py`` to something other
than itself (a library routine, brute force, closed forms, invariants, and the
value printed for the fp8 probability-underflow example on aiter PR #7375).
"""

from .attention import (  # noqa: F401
    E4M3FN_MAX,
    attend,
    attend_lse,
    bf16_bits_to_f64,
    e4m3fn_decode_table,
    first_visible_key,
    segment_page_ranges,
    segment_partials,
    visible_key_count,
)
from .fp8_model import attend_fp8, block_round, e4m3_round  # noqa: F401
from .prefill import causal_visible, default_scale, kv_head_of, prefill_attend, prefill_lse  # noqa: F401
