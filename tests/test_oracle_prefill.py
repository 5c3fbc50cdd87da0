"""Pins of the prefill oracle (oracle/prefill.py) to things other than itself.

- The value printed for the fp8 probability-underflow example on aiter PR #7375
  (tests/golden/fp8_p_underflow_example.txt): that example is this workload's
  own shape (non-causal, 64 queries, 16384 keys, qk head dim 192).
- Brute force with pure-Python loops and math.fsum on tiny varlen batches,
  causal and not, with GQA, fewer keys than queries and empty KV.
- A library special case: torch's scaled_dot_product_attention in fp64 over
  each sequence with an explicit bottom-right mask.
- Closed forms (one key, identical keys, the dominant key) and invariants (GQA
  duplication, descale algebra, batch order, LSE merge of key chunks, the
  chunked-prefill merge the same page tests).
- Planted mistakes in the oracle's steps, each caught by a pin above.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.prefill as oracle_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TABLE = oracle.e4m3fn_decode_table()
FINITE = np.flatnonzero(np.isfinite(TABLE) & (np.abs(TABLE) <= 4))


def _code(value):
    return int(np.flatnonzero(TABLE == value)[0])


def _case(lens, hq, hkv, dqk, dv, seed, causal):
    """Random codes for a varlen batch; lens = [(Lq, Lk), ...]."""
    rng = np.random.default_rng(seed)
    tq = sum(a for a, _ in lens)
    tk = sum(b for _, b in lens)
    return dict(
        q=rng.choice(FINITE, size=(tq, hq, dqk)).astype(np.uint8),
        k=rng.choice(FINITE, size=(tk, hkv, dqk)).astype(np.uint8),
        v=rng.choice(FINITE, size=(tk, hkv, dv)).astype(np.uint8),
        cu_seqlens_q=np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32),
        cu_seqlens_k=np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32),
        q_descale=0.75, k_descale=0.375, v_descale=1.25, softmax_scale=0.3, causal=causal)


def _brute(c):
    """Pure-Python definition: returns (out [Tq][Hq][Dv] lists, lse [Hq][Tq])."""
    q, k, v = c["q"], c["k"], c["v"]
    hq_n, hkv_n = q.shape[1], k.shape[1]
    out = np.zeros((q.shape[0], hq_n, v.shape[2]))
    lse = np.full((hq_n, q.shape[0]), -np.inf)
    scale = float(np.float32(c["softmax_scale"]))
    cq, ck = c["cu_seqlens_q"], c["cu_seqlens_k"]
    for b in range(len(cq) - 1):
        lq, lk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        for h in range(hq_n):
            kvh = h * hkv_n // hq_n
            for i in range(lq):
                qi = int(cq[b]) + i
                scores = []
                for j in range(lk):
                    if c["causal"] and j > lk - lq + i:
                        continue
                    kj = int(ck[b]) + j
                    dot = math.fsum(TABLE[q[qi, h, d]] * c["q_descale"] * TABLE[k[kj, kvh, d]] * c["k_descale"]
                                    for d in range(q.shape[2]))
                    scores.append((j, scale * dot))
                if not scores:
                    continue
                top = max(s for _, s in scores)
                w = [(j, math.exp(s - top)) for j, s in scores]
                den = math.fsum(x for _, x in w)
                lse[h, qi] = top + math.log(den)
                for d in range(v.shape[2]):
                    out[qi, h, d] = math.fsum(x * TABLE[v[int(ck[b]) + j, kvh, d]] * c["v_descale"] for j, x in w) / den
    return out, lse


CASES = [
    ([(3, 5), (4, 2), (2, 0), (1, 1)], 4, 2, 6, 5, 1, True),
    ([(3, 5), (4, 2), (2, 0), (1, 1)], 4, 2, 6, 5, 2, False),
    ([(5, 5), (2, 7)], 2, 1, 8, 4, 3, True),
    ([(6, 3)], 3, 3, 5, 3, 4, True),
]


@pytest.mark.parametrize("cfg", CASES)
def test_prefill_matches_brute_force(cfg):
    c = _case(*cfg)
    ref_out, ref_lse = _brute(c)
    out = oracle.prefill_attend(**c)
    lse = oracle.prefill_lse(**c)
    assert np.allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_sdpa_fp64(causal):
    c = _case([(7, 9), (5, 3), (4, 4)], 4, 2, 12, 10, 7, causal)
    out = oracle.prefill_attend(**c)
    cq, ck = c["cu_seqlens_q"], c["cu_seqlens_k"]
    for b in range(len(cq) - 1):
        q = torch.from_numpy(TABLE[c["q"][cq[b]:cq[b + 1]]] * c["q_descale"]).permute(1, 0, 2)
        k = torch.from_numpy(TABLE[c["k"][ck[b]:ck[b + 1]]] * c["k_descale"]).permute(1, 0, 2)
        v = torch.from_numpy(TABLE[c["v"][ck[b]:ck[b + 1]]] * c["v_descale"]).permute(1, 0, 2)
        k = k.repeat_interleave(2, dim=0)
        v = v.repeat_interleave(2, dim=0)
        lq, lk = q.shape[1], k.shape[1]
        mask = torch.ones((lq, lk), dtype=torch.bool)
        if causal:
            mask = torch.arange(lk)[None, :] <= (lk - lq + torch.arange(lq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=mask, scale=float(np.float32(c["softmax_scale"]))).permute(1, 0, 2).numpy()
        seen = mask.any(dim=1).numpy()
        got = out[cq[b]:cq[b + 1]]
        assert np.allclose(got[seen], ref[seen], rtol=1e-12, atol=1e-13)
        assert np.all(got[~seen] == 0)


def _dominant(sq, sk, dqk, dv, causal=False):
    q = np.zeros((sq, 1, dqk), np.uint8)
    k = np.zeros((sk, 1, dqk), np.uint8)
    v = np.full((sk, 1, dv), _code(-1.0), np.uint8)
    q[:, 0, 0] = _code(8.0)
    k[0, 0, 0] = _code(14.0)
    v[0] = _code(1.0)
    return dict(q=q, k=k, v=v, cu_seqlens_q=np.array([0, sq], np.int32), cu_seqlens_k=np.array([0, sk], np.int32),
                q_descale=1.0, k_descale=1.0, v_descale=1.0, softmax_scale=None, causal=causal)


def test_printed_underflow_example():
    """The page's example on this very workload: exact O ~ -0.6699."""
    fields = {}
    for line in open(os.path.join(GOLDEN, "fp8_p_underflow_example.txt")):
        if line.strip() and not line.startswith("#"):
            key, val = line.split()
            fields[key] = float(val)
    sq, sk, dqk = int(fields["num_queries"]), int(fields["num_keys"]), int(fields["qk_head_dim"])
    out = oracle.prefill_attend(**_dominant(sq, sk, dqk, 128))
    half_ulp = 0.5 * 10.0 ** -int(fields["printed_decimals"])
    assert out.shape == (sq, 1, 128)
    assert np.all(np.abs(out - fields["exact_output"]) <= half_ulp)
    a = math.exp(fields["q_dim0"] * fields["k_key0_dim0"] / math.sqrt(dqk))
    assert np.allclose(out, (a - (sk - 1)) / (a + (sk - 1)), rtol=0, atol=1e-12)


def test_dominant_key_causal_closed_form():
    """Causal with Lq = Lk: row i sees i + 1 keys, key 0 dominant."""
    n = 300
    out = oracle.prefill_attend(**_dominant(n, n, 192, 16, causal=True))
    a = math.exp(8 * 14 / math.sqrt(192))
    for i in range(n):
        expect = (a - i) / (a + i)
        assert np.allclose(out[i], expect, rtol=0, atol=1e-12)


def test_single_key_and_identical_keys():
    c = _case([(1, 1)], 2, 1, 192, 128, 11, False)
    out = oracle.prefill_attend(**c)
    assert np.allclose(out[0], TABLE[c["v"][0, 0]] * c["v_descale"], rtol=0, atol=0)
    # identical keys, causal, Lq = Lk: row i is the mean of V rows 0..i
    L = 40
    c = _case([(L, L)], 1, 1, 16, 8, 12, True)
    c["k"][:] = c["k"][0]
    out = oracle.prefill_attend(**c)
    vals = TABLE[c["v"][:, 0, :]] * c["v_descale"]
    for i in range(L):
        assert np.allclose(out[i, 0], vals[: i + 1].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_invariants():
    c = _case([(6, 9), (3, 3)], 4, 1, 8, 6, 13, True)
    base = oracle.prefill_attend(**c)
    # GQA duplication: two identical KV heads serve the same result as one
    d = dict(c)
    d["k"] = np.repeat(c["k"], 2, axis=1)
    d["v"] = np.repeat(c["v"], 2, axis=1)
    assert np.allclose(oracle.prefill_attend(**d), base, rtol=1e-12, atol=1e-13)
    # v_descale x 2 doubles the output; (k_descale c, scale / c) leaves it alone
    d = dict(c, v_descale=2 * c["v_descale"])
    assert np.allclose(oracle.prefill_attend(**d), 2 * base, rtol=1e-12, atol=1e-13)
    d = dict(c, k_descale=c["k_descale"] * 4, softmax_scale=c["softmax_scale"] / 4)
    assert np.allclose(oracle.prefill_attend(**d), base, rtol=1e-12, atol=1e-13)
    # batch order: the sequences swapped give the same rows
    lq0, lk0 = 6, 9
    d = dict(c, q=np.concatenate([c["q"][lq0:], c["q"][:lq0]]), k=np.concatenate([c["k"][lk0:], c["k"][:lk0]]),
             v=np.concatenate([c["v"][lk0:], c["v"][:lk0]]), cu_seqlens_q=np.array([0, 3, 9], np.int32),
             cu_seqlens_k=np.array([0, 3, 12], np.int32))
    swapped = oracle.prefill_attend(**d)
    assert np.allclose(swapped[3:], base[:6], rtol=1e-12, atol=1e-13)
    assert np.allclose(swapped[:3], base[6:], rtol=1e-12, atol=1e-13)


def test_lse_merge_of_key_chunks():
    """Non-causal: attention over keys [0, n) equals the LSE merge of [0, m) and [m, n)
    (the chunked-prefill merge the same page tests)."""
    c = _case([(5, 20)], 2, 1, 8, 6, 17, False)
    full, full_lse = oracle.prefill_attend(**c), oracle.prefill_lse(**c)
    parts = []
    for lo, hi in ((0, 7), (7, 20)):
        d = dict(c, k=c["k"][lo:hi], v=c["v"][lo:hi], cu_seqlens_k=np.array([0, hi - lo], np.int32))
        parts.append((oracle.prefill_attend(**d), oracle.prefill_lse(**d)))
    (o1, l1), (o2, l2) = parts
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (o1 * w1.T[:, :, None] + o2 * w2.T[:, :, None]) / (w1 + w2).T[:, :, None]
    assert np.allclose(merged, full, rtol=1e-12, atol=1e-13)
    assert np.allclose(m + np.log(w1 + w2), full_lse, rtol=1e-12, atol=1e-13)


def test_rows_without_keys():
    c = _case([(4, 2), (2, 0)], 2, 1, 8, 6, 19, True)
    out, lse = oracle.prefill_attend(**c), oracle.prefill_lse(**c)
    # sequence 0: rows 0, 1 see no key (Lk - Lq + i < 0); sequence 1 has no keys at all
    assert np.all(out[[0, 1, 4, 5]] == 0) and np.all(np.isneginf(lse[:, [0, 1, 4, 5]]))
    assert np.all(np.isfinite(lse[:, [2, 3]]))


# ---------------------------------------------------------------- planted mistakes
def _mutations():
    good_decode = oracle_prefill._decode
    return {
        "top_left_mask": ("causal_visible", lambda lq, lk: np.arange(lk)[None, :] <= np.arange(lq)[:, None]),
        "mask_off_by_one": ("causal_visible", lambda lq, lk: np.arange(lk)[None, :] < (lk - lq + np.arange(lq))[:, None]),
        "gqa_interleaved": ("kv_head_of", lambda hq, nq, nkv: hq % nkv),
        "default_scale_dv": ("default_scale", lambda d: 1.0 / math.sqrt(128.0)),
        "dropped_descale": ("_decode", lambda codes, ds: good_decode(codes, 1.0)),
    }


@pytest.mark.parametrize("name", sorted(_mutations()))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, bad = _mutations()[name]
    cfg = _case(*CASES[0])
    ref_out, _ = _brute(cfg)
    n = 4096
    golden = _dominant(64, n, 192, 8)
    a = math.exp(8 * 14 / math.sqrt(192))
    closed = (a - (n - 1)) / (a + (n - 1))
    monkeypatch.setattr(oracle_prefill, attr, bad)
    caught = not np.allclose(oracle_prefill.prefill_attend(**cfg), ref_out, rtol=1e-9, atol=1e-12)
    caught |= not np.allclose(oracle_prefill.prefill_attend(**golden), closed, rtol=0, atol=1e-12)
    assert caught, name
