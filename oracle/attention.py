"""fp64 reference for split-KV verify attention over a paged fp8 KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Each step below is written from the definition, in the order the pages state the
problem, with no blocking, fusion or reordering beyond it:

1. fp8 decode: the cache holds OCP FP8 E4M3 ("e4m3fn") bytes. aiter PR #5190,
   section Supported, names "K/V fp8 e4m3 with per-tensor scales"; aiter PR #7375,
   section Performance, quantizes per tensor with scale amax / 448, which fixes
   the finite-only flavour whose largest value is 448.
2. Paged gather: for sequence b, KV position j lives in page
   ``block_tables[b, j // page_size]`` at slot ``j % page_size``, NHD order
   ``[page, slot, kv_head, dim]`` (aiter PR #5190, Motivation: "NHD page-16 fp8
   KV cache" read in place). Only the first ``seq_lens[b]`` positions exist.
3. Descale: K and V values are the decoded bytes times ``k_descale`` /
   ``v_descale`` (aiter PR #5190, Kernel notes and Supported: per-tensor scales
   read from device pointers).
4. Scores: ``softmax_scale * <q, k>``; query head ``hq`` reads KV head
   ``hq // G`` with ``G = Hq / Hkv`` (aiter PR #5190, Motivation: 16 or 8 query
   heads on one KV head).
5. Bottom-right causal mask: a sequence with q_len n and KV length L has its n
   query tokens at positions L-n .. L-1, and query i sees KV positions
   0 .. L-n+i (aiter PR #5190, Motivation: "a causal mask over the last 4
   positions"; SGLang PR #37465, Modifications: q_len 1 to 4 per sequence).
6. Softmax over the visible keys with exact ``exp`` in fp64, then the weighted
   sum of V rows. A query with no visible key yields zeros.
7. The optional log-sum-exp of the same scores (:func:`attend_lse`).
8. Options the pages only name (a left window, a score soft-cap, per-head sink
   logits), in their common reading (:func:`attend`).
"""

from __future__ import annotations

import math

import numpy as np

# Largest finite e4m3fn value: exponent field 15 with mantissa 6 (110b).
E4M3FN_MAX = 448.0


def e4m3fn_decode_table() -> np.ndarray:
    """All 256 e4m3fn codes decoded to float64 from the OCP 8-bit FP definition.

    Sign bit 7; exponent bits 6..3 with bias 7; mantissa bits 2..0. Exponent
    field 0 is subnormal: m * 2^-9. S.1111.111 is NaN; there is no infinity.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = math.nan
        elif exp_field == 0:
            table[code] = sign * math.ldexp(mant, -9)
        else:
            table[code] = sign * math.ldexp(8 + mant, exp_field - 7 - 3)
    return table


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns (the top half of a float32)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    widened = bits.astype(np.uint32) << 16
    return widened.view(np.float32).astype(np.float64)


def visible_key_count(seq_len: int, q_len: int, i: int) -> int:
    """Number of KV positions query i (0-based, of q_len) may attend to.

    Query i sits at position seq_len - q_len + i and sees positions up to and
    including its own, so it sees seq_len - q_len + i + 1 keys (never more than
    seq_len, never fewer than 0).
    """
    return max(0, min(seq_len, seq_len - q_len + i + 1))


def _queries_f64(q) -> np.ndarray:
    q = np.asarray(q)
    if q.dtype == np.uint16:
        return bf16_bits_to_f64(q)
    return q.astype(np.float64)


def _gather_sequence(table, cache, block_row, seq_len, descale):
    """Dequantized ``[seq_len, Hkv, D]`` float64 rows of one sequence's cache."""
    page_size = cache.shape[1]
    n_pages = -(-seq_len // page_size)
    ids = np.asarray(block_row[:n_pages], dtype=np.int64)
    codes = cache[ids].reshape(n_pages * page_size, cache.shape[2], cache.shape[3])[:seq_len]
    return table[codes] * descale


def first_visible_key(seq_len: int, q_len: int, i: int, window_left: int) -> int:
    """First KV position query i may attend to under a left window.

    The window convention of the varlen attention APIs that aiter PR #7375
    routes through (section Changes: a negative window is unlimited): query i at
    position seq_len - q_len + i sees positions from that position minus
    ``window_left`` on (never before 0).
    """
    if window_left < 0:
        return 0
    return max(0, seq_len - q_len + i - window_left)


def _softcapped(scores: np.ndarray, softcap: float) -> np.ndarray:
    """cap * tanh(score / cap) when cap > 0 (a score soft-cap), else the scores."""
    if softcap > 0.0:
        return softcap * np.tanh(scores / softcap)
    return scores


def attend(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q,
           k_descale, v_descale, softmax_scale, window_left=-1, softcap=0.0, sinks=None) -> np.ndarray:
    """Exact masked softmax attention; returns float64 ``[T, Hq, D]``.

    q: bf16 bit patterns (uint16) or real values, ``[T, Hq, D]`` packed by
    ``cu_seqlens_q``. k_cache / v_cache: uint8 e4m3fn codes
    ``[num_pages, page_size, Hkv, D]``. block_tables: int ``[N, max_pages]``.
    seq_lens: int ``[N]``. cu_seqlens_q: int ``[N + 1]``. The descales and the
    softmax scale are taken at float32 precision, as the device receives them.

    Options the pages name only as features their gates exclude (SGLang PR
    #37465, Modifications: no sliding window, soft-cap or sinks; aiter PR #7375,
    Changes: windows, sinks, soft-cap), taken in their common reading:
    ``window_left`` >= 0 keeps only the keys at most that many positions before
    the query (:func:`first_visible_key`); ``softcap`` > 0 replaces every score
    s by softcap * tanh(s / softcap); ``sinks`` (float ``[Hq]``) adds exp(sink)
    of the row's head to the softmax denominator, a probability mass that
    carries no value.
    """
    table = e4m3fn_decode_table()
    qf = _queries_f64(q)
    k_cache = np.asarray(k_cache, dtype=np.uint8)
    v_cache = np.asarray(v_cache, dtype=np.uint8)
    block_tables = np.asarray(block_tables)
    seq_lens = np.asarray(seq_lens)
    cu = np.asarray(cu_seqlens_q)
    kd = float(np.float32(k_descale))
    vd = float(np.float32(v_descale))
    scale = float(np.float32(softmax_scale))
    cap = float(np.float32(softcap))

    total_q, num_q_heads, head_dim = qf.shape
    num_kv_heads = k_cache.shape[2]
    group = num_q_heads // num_kv_heads
    sink = None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64)
    out = np.zeros((total_q, num_q_heads, head_dim), dtype=np.float64)

    for b in range(len(seq_lens)):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        q_len, seq_len = q1 - q0, int(seq_lens[b])
        if q_len <= 0 or seq_len <= 0:
            continue
        keys = _gather_sequence(table, k_cache, block_tables[b], seq_len, kd)
        vals = _gather_sequence(table, v_cache, block_tables[b], seq_len, vd)
        for h in range(num_kv_heads):
            heads = slice(h * group, (h + 1) * group)
            for i in range(q_len):
                lo = first_visible_key(seq_len, q_len, i, window_left)
                vis = visible_key_count(seq_len, q_len, i)
                if vis <= lo:
                    continue
                scores = _softcapped((qf[q0 + i, heads, :] @ keys[lo:vis, h, :].T) * scale, cap)   # [G, n]
                top = scores.max(axis=1, keepdims=True)
                weights = np.exp(scores - top)
                den = weights.sum(axis=1, keepdims=True)
                if sink is not None:
                    den = den + np.exp(sink[heads][:, None] - top)
                out[q0 + i, heads, :] = (weights @ vals[lo:vis, h, :]) / den
    return out


def attend_lse(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q,
               k_descale, v_descale, softmax_scale, window_left=-1, softcap=0.0, sinks=None) -> np.ndarray:
    """Exact log-sum-exp of each row's visible scores; returns float64 ``[T, Hq]``.

    lse[t, h] = ln sum_j exp(score_j) over the keys row (t, h) may see, with the
    scores of :func:`attend` (steps 1-5 above); a row with no visible key gets
    -inf (aiter PR #7375: the optional LSE of a varlen attention call, with
    -inf for rows that have no finite value). Evaluated as top + ln sum_j
    exp(score_j - top) so that no exp overflows. ``v_cache`` and ``v_descale``
    do not enter; they are accepted so that the call matches :func:`attend`.
    The options are those of :func:`attend`; a sink adds exp(sink) to the sum,
    so a row with a sink and no visible key gets lse = sink.
    """
    table = e4m3fn_decode_table()
    qf = _queries_f64(q)
    k_cache = np.asarray(k_cache, dtype=np.uint8)
    seq_lens = np.asarray(seq_lens)
    cu = np.asarray(cu_seqlens_q)
    kd = float(np.float32(k_descale))
    scale = float(np.float32(softmax_scale))
    cap = float(np.float32(softcap))

    total_q, num_q_heads, _ = qf.shape
    num_kv_heads = k_cache.shape[2]
    group = num_q_heads // num_kv_heads
    sink = None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64)
    lse = np.full((total_q, num_q_heads), -np.inf)

    for b in range(len(seq_lens)):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        q_len, seq_len = q1 - q0, int(seq_lens[b])
        if q_len <= 0 or seq_len <= 0:
            continue
        keys = _gather_sequence(table, k_cache, block_tables[b], seq_len, kd)
        for h in range(num_kv_heads):
            heads = slice(h * group, (h + 1) * group)
            for i in range(q_len):
                lo = first_visible_key(seq_len, q_len, i, window_left)
                vis = visible_key_count(seq_len, q_len, i)
                if vis <= lo:
                    if sink is not None:
                        lse[q0 + i, heads] = sink[heads]
                    continue
                scores = _softcapped((qf[q0 + i, heads, :] @ keys[lo:vis, h, :].T) * scale, cap)
                if sink is not None:
                    scores = np.concatenate([scores, sink[heads][:, None]], axis=1)
                top = scores.max(axis=1)
                lse[q0 + i, heads] = top + np.log(np.exp(scores - top[:, None]).sum(axis=1))
    return lse


def segment_page_ranges(n_pages: int, num_segments: int):
    """Page ranges ``[begin, end)`` of the split-KV segments of one sequence.

    The pages do not spell out the partition; this is the plainest reading that
    keeps every segment count in [1, 64] valid with empty tail segments (aiter
    PR #5190, Kernel notes): each segment takes ceil(n_pages / S) whole pages in
    order, and the segments past the last page are empty.
    """
    chunk = -(-n_pages // num_segments) if n_pages > 0 else 0
    ranges = []
    for s in range(num_segments):
        begin = min(s * chunk, n_pages)
        end = min((s + 1) * chunk, n_pages)
        ranges.append((begin, end))
    return ranges


def segment_partials(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q,
                     k_descale, v_descale, softmax_scale, num_segments: int):
    """Per-segment softmax statistics, the quantities a split-KV partial fixes.

    Returns ``(lse2, o)`` with ``lse2`` float64 ``[S, T, Hq]`` = log2 of the sum
    of exp(score) over the segment's visible keys (-inf when it has none), and
    ``o`` float64 ``[S, T, Hq, D]`` = that segment's own softmax-weighted mean of
    descaled V rows (0 when it has none). Merging segments by log-sum-exp weights
    ``2^(lse2_s)`` reproduces :func:`attend`.
    """
    table = e4m3fn_decode_table()
    qf = _queries_f64(q)
    k_cache = np.asarray(k_cache, dtype=np.uint8)
    v_cache = np.asarray(v_cache, dtype=np.uint8)
    seq_lens = np.asarray(seq_lens)
    cu = np.asarray(cu_seqlens_q)
    kd = float(np.float32(k_descale))
    vd = float(np.float32(v_descale))
    scale = float(np.float32(softmax_scale))
    page_size = k_cache.shape[1]

    total_q, num_q_heads, head_dim = qf.shape
    num_kv_heads = k_cache.shape[2]
    group = num_q_heads // num_kv_heads
    lse2 = np.full((num_segments, total_q, num_q_heads), -np.inf)
    o = np.zeros((num_segments, total_q, num_q_heads, head_dim))

    for b in range(len(seq_lens)):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        q_len, seq_len = q1 - q0, int(seq_lens[b])
        if q_len <= 0 or seq_len <= 0:
            continue
        keys = _gather_sequence(table, k_cache, block_tables[b], seq_len, kd)
        vals = _gather_sequence(table, v_cache, block_tables[b], seq_len, vd)
        n_pages = -(-seq_len // page_size)
        for s, (pb, pe) in enumerate(segment_page_ranges(n_pages, num_segments)):
            for h in range(num_kv_heads):
                heads = slice(h * group, (h + 1) * group)
                for i in range(q_len):
                    lo = pb * page_size
                    hi = min(pe * page_size, visible_key_count(seq_len, q_len, i))
                    if hi <= lo:
                        continue
                    scores = (qf[q0 + i, heads, :] @ keys[lo:hi, h, :].T) * scale
                    top = scores.max(axis=1, keepdims=True)
                    weights = np.exp(scores - top)
                    total = weights.sum(axis=1)
                    lse2[s, q0 + i, heads] = (top[:, 0] + np.log(total)) / math.log(2.0)
                    o[s, q0 + i, heads, :] = (weights @ vals[lo:hi, h, :]) / total[:, None]
    return lse2, o
