"""fp64 model of the fp8 arithmetic class of the verify attention: Q and P rounded to e4m3.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages' kernel quantises Q and the softmax probabilities P to fp8 (aiter PR
#5190, Kernel notes: fp8-quantised Q/P; Accuracy: its error against a 16-bit
reference), and the review on aiter PR #7375 ("Keep FP8 attention opt-in until
probability underflow is bounded") shows what plain e4m3 rounding of P loses:
probabilities below half the smallest subnormal become 0. This module computes
attention with exactly those roundings and nothing else, in fp64, so that a
test can tell the error the arithmetic itself carries on an input from the
error an implementation adds:

1. e4m3 rounding (:func:`e4m3_round`): round to nearest, ties to even, onto the
   OCP E4M3 ("e4m3fn") grid: 3 mantissa bits, normal binades 2^-6 .. 2^8,
   subnormal spacing 2^-9, largest finite 448.
2. Power-of-two block scales (:func:`block_round`): a block of values is
   multiplied by 2^-e, rounded, and multiplied back, with e = floor(log2 of the
   block's largest magnitude) - 7, so that the largest lands in [128, 256) and
   the others keep 3 mantissa bits down to 2^-13 of it. Reading: the pages give
   no block size or scale rule; this takes 32 elements per block and one E8M0
   (power-of-two) scale per block, the shape of the OCP microscaling formats
   the gfx950 scaled fp8 MFMA takes.
3. Q: each query row's head_dim values in consecutive blocks of 32 dims.
4. P = exp(s - max) over the row's visible keys (scores, masks and options as
   :func:`oracle.attention.attend`), in consecutive blocks of 32 key positions
   (positions 32 j .. 32 j + 31 of the sequence); with ``p_block_scale=False``
   P is rounded with no scale, the model of the review's example.
5. Output = sum_j P~_j v_j / (sum_j P~_j + sink term), the rounded P~ in both
   sums; K, V, the descales and the sink logits are exact.
6. Which way each P rounds depends on where the block's largest P falls within
   its binade, that is on the reference an implementation subtracts before
   exponentiating (a running or lazy maximum rather than the row's exact one).
   ``p_offsets`` (``[T, Hq]``, in [0, 1), log2 units) moves that reference:
   every P of the row is multiplied by 2^-offset before rounding. The offset
   cancels in the normalisation, so it changes nothing but the roundings; a
   few offsets give a few equally valid realizations of the same arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import (
    _gather_sequence,
    _queries_f64,
    _softcapped,
    e4m3fn_decode_table,
    first_visible_key,
    visible_key_count,
)

E4M3_MIN_NORMAL_EXP = -6    # smallest normal binade 2^-6
E4M3_MANTISSA_BITS = 3
E4M3_MAX = 448.0
BLOCK = 32


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to even); |x| must not exceed 448.

    A value in binade [2^E, 2^(E+1)) with E >= -6 lies on a grid of spacing
    2^(E-3); below 2^-6 the subnormal grid has spacing 2^-9. numpy's ``rint``
    rounds halves to even, which on these grids is the even mantissa.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    if np.any(mag > E4M3_MAX):
        raise ValueError("e4m3_round: |x| > 448")
    _, ex = np.frexp(mag)                        # mag = m 2^ex, m in [0.5, 1)
    binade = np.maximum(ex - 1, E4M3_MIN_NORMAL_EXP)
    spacing = np.ldexp(1.0, binade - E4M3_MANTISSA_BITS)
    return np.sign(x) * np.rint(mag / spacing) * spacing


def block_exponent(block) -> int:
    """e = floor(log2 max|block|) - 7 (0 for an all-zero block)."""
    top = float(np.max(np.abs(block))) if np.size(block) else 0.0
    if top == 0.0:
        return 0
    _, ex = np.frexp(top)
    return int(ex) - 1 - 7


def block_round(x, block: int = BLOCK) -> np.ndarray:
    """e4m3 rounding under one power-of-two scale per ``block`` consecutive
    elements of the last axis (a short last block keeps its own scale)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    n = x.shape[-1]
    for j in range(0, n, block):
        part = x[..., j:j + block]
        flat = part.reshape(-1, part.shape[-1])
        res = np.empty_like(flat)
        for r in range(flat.shape[0]):
            e = block_exponent(flat[r])
            res[r] = e4m3_round(np.ldexp(flat[r], -e)) * 2.0 ** e
        out[..., j:j + block] = res.reshape(part.shape)
    return out


def _round_p(p: np.ndarray, lo: int, block_scale: bool) -> np.ndarray:
    """P of keys lo .. lo + n - 1 ([G, n]), rounded in blocks of 32 positions
    aligned to position 0 of the sequence."""
    if not block_scale:
        return e4m3_round(p)
    g, n = p.shape
    start = lo - lo % BLOCK
    width = -(-(lo + n - start) // BLOCK) * BLOCK
    padded = np.zeros((g, width))
    padded[:, lo - start:lo - start + n] = p
    blocks = padded.reshape(g, width // BLOCK, BLOCK)
    top = blocks.max(axis=2, keepdims=True)
    _, ex = np.frexp(np.where(top > 0, top, 1.0))
    e = np.where(top > 0, ex - 1 - 7, 0)
    scaled = np.ldexp(blocks, -e)
    rounded = e4m3_round(scaled) * np.ldexp(1.0, e)
    return rounded.reshape(g, width)[:, lo - start:lo - start + n]


def attend_fp8(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, k_descale, v_descale,
               softmax_scale, quantize_q=True, p_block_scale=True, window_left=-1, softcap=0.0,
               sinks=None, p_offsets=None) -> np.ndarray:
    """Attention with e4m3 P (and, with ``quantize_q``, e4m3 Q); float64 ``[T, Hq, D]``.

    Arguments as :func:`oracle.attention.attend`, which this equals except for
    the roundings of steps 3-5 in the module docstring.
    """
    table = e4m3fn_decode_table()
    qf = _queries_f64(q)
    if quantize_q:
        qf = block_round(qf)
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
                scores = _softcapped((qf[q0 + i, heads, :] @ keys[lo:vis, h, :].T) * scale, cap)
                top = scores.max(axis=1, keepdims=True)
                shift = np.zeros((group, 1))
                if p_offsets is not None:
                    shift = np.asarray(p_offsets, dtype=np.float64)[q0 + i, heads][:, None] * math.log(2.0)
                weights = _round_p(np.exp(scores - top - shift), lo, p_block_scale)
                den = weights.sum(axis=1, keepdims=True)
                if sink is not None:
                    den = den + np.exp(sink[heads][:, None] - top - shift)
                out[q0 + i, heads, :] = (weights @ vals[lo:vis, h, :]) / den
    return out
