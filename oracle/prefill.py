"""fp64 reference for fp8 varlen prefill attention (the second workload).

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

What it computes follows aiter PR #7375 ("gfx1250 fp8 varlen FMHA"), section
Summary, written out from the definition with no blocking or reordering:

1. Q, K and V are e4m3fn bytes (the OCP FP8 E4M3 codes, decoded exactly by
   :func:`oracle.attention.e4m3fn_decode_table`), each with one per-tensor fp32
   descale: real value = decoded byte * descale.
2. Packed varlen (THD) layout: sequence b owns query rows
   ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1`` and key/value rows
   ``cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1``; q is ``[total_q, Hq, Dqk]``, k is
   ``[total_k, Hkv, Dqk]`` and v is ``[total_k, Hkv, Dv]`` (the pages' shape:
   Dqk 192, Dv 128).
3. Query head hq reads KV head hq // (Hq / Hkv).
4. Scores ``softmax_scale * <q, k>``; the default scale is 1 / sqrt(Dqk) (the
   same page's review on probability underflow runs its example at the default
   scale, which its printed value fixes to 1 / sqrt(192)).
5. With ``causal``, the mask is aligned to the bottom right (Summary): with Lq
   queries and Lk keys, query i sees keys 0 .. Lk - Lq + i. A query that sees
   no key yields zeros.
6. Softmax with exact ``exp`` in fp64, then the weighted sum of V rows; the
   optional log-sum-exp of the visible scores, laid out ``[Hq, total_q]``
   (Changes: the varlen API layout (nheads, total_q)).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import e4m3fn_decode_table


def _decode(codes, descale):
    return e4m3fn_decode_table()[np.asarray(codes, dtype=np.uint8)] * float(descale)


def default_scale(dqk: int) -> float:
    """1 / sqrt(Dqk), the scale used when none is given."""
    return 1.0 / math.sqrt(dqk)


def kv_head_of(hq: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head hq: consecutive groups of Hq / Hkv share one."""
    return hq // (num_q_heads // num_kv_heads)


def causal_visible(lq: int, lk: int) -> np.ndarray:
    """Boolean [lq, lk]: query i sees key j iff j <= lk - lq + i (bottom right)."""
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= lk - lq + i


def _rows(q, k, v, cu_seqlens_q, cu_seqlens_k, q_descale, k_descale, v_descale, softmax_scale, causal):
    """Yield (b, hq, query rows, scores [Lq, Lk] with masked entries -inf, V rows)."""
    Q = _decode(q, q_descale)
    K = _decode(k, k_descale)
    V = _decode(v, v_descale)
    num_q_heads, dqk = Q.shape[1], Q.shape[2]
    num_kv_heads = K.shape[1]
    scale = default_scale(dqk) if softmax_scale is None else float(np.float32(softmax_scale))
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        lq, lk = q1 - q0, k1 - k0
        for hq in range(num_q_heads):
            h = kv_head_of(hq, num_q_heads, num_kv_heads)
            scores = scale * (Q[q0:q1, hq, :] @ K[k0:k1, h, :].T)
            if causal:
                scores = np.where(causal_visible(lq, lk), scores, -np.inf)
            yield b, hq, np.arange(q0, q1), scores, V[k0:k1, h, :]


def prefill_attend(q, k, v, cu_seqlens_q, cu_seqlens_k, q_descale, k_descale, v_descale,
                   softmax_scale=None, causal=False) -> np.ndarray:
    """Attention output, fp64 ``[total_q, Hq, Dv]``.

    q, k, v: uint8 e4m3fn codes ``[T, H, D]``; cu_seqlens_q / cu_seqlens_k: int
    ``[B + 1]``; descales: floats; softmax_scale: None for 1 / sqrt(Dqk).
    """
    out = np.zeros((np.asarray(q).shape[0], np.asarray(q).shape[1], np.asarray(v).shape[2]))
    for _, hq, rows, scores, vals in _rows(q, k, v, cu_seqlens_q, cu_seqlens_k, q_descale, k_descale,
                                           v_descale, softmax_scale, causal):
        for r, row in enumerate(rows):
            s = scores[r]
            if not np.isfinite(s).any():
                continue
            w = np.exp(s - s[np.isfinite(s)].max())
            out[row, hq, :] = (w @ vals) / w.sum()
    return out


def prefill_lse(q, k, v, cu_seqlens_q, cu_seqlens_k, q_descale, k_descale, v_descale,
                softmax_scale=None, causal=False) -> np.ndarray:
    """Natural-log log-sum-exp of each row's visible scores, fp64 ``[Hq, total_q]``
    (-inf for a row that sees no key)."""
    lse = np.full((np.asarray(q).shape[1], np.asarray(q).shape[0]), -np.inf)
    for _, hq, rows, scores, _ in _rows(q, k, v, cu_seqlens_q, cu_seqlens_k, q_descale, k_descale,
                                        v_descale, softmax_scale, causal):
        for r, row in enumerate(rows):
            s = scores[r][np.isfinite(scores[r])]
            if s.size:
                top = s.max()
                lse[hq, row] = top + math.log(np.exp(s - top).sum())
    return lse
