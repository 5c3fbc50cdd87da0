"""Pins for the CPU oracle: each check compares it with something other than itself.

- the fp8 table against torch's own e4m3fn decode (a library routine) and the
  OCP definition's named points;
- the whole computation against a brute-force token-by-token walk with
  math.fsum (tiny inputs), and against torch's fp64
  scaled_dot_product_attention on densely gathered K/V with an explicit
  bottom-right mask (a library special case);
- closed forms (one visible key, identical keys, one dominant key) and the
  value printed for the fp8 probability-underflow example on aiter PR #7375;
- invariants (page-pool permutation, duplicated KV heads, descale algebra);
- planted mistakes in the oracle's steps, each of which some pin must catch.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention
from paged_fp8_kv_split_amd.workloads import Workload, make_case, permute_pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(ctx, q_lens, hq, hkv, d=8, page=4, seed=0, descale="amax", scale=None):
    w = Workload(name="t", ctx=tuple(ctx), q_lens=tuple(q_lens), num_q_heads=hq, num_kv_heads=hkv,
                 num_segments=1, seed=seed, head_dim=d, page_size=page, descale=descale,
                 softmax_scale=scale if scale is not None else 1.0 / math.sqrt(d))
    return make_case(w, "cpu")


def _run_oracle(case):
    return oracle.attend(**case.host_arrays())


# ---------------------------------------------------------------- fp8 / bf16 decode
def test_e4m3fn_table_matches_torch():
    table = oracle.e4m3fn_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(table[ok], ref[ok])
    assert np.array_equal(np.signbit(table[ok]), np.signbit(ref[ok]))


def test_e4m3fn_named_points():
    t = oracle.e4m3fn_decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0 == -oracle.E4M3FN_MAX
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0 and t[0xB8] == -1.0 and t[0x39] == 1.125
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.sum(np.isnan(t)) == 2 and np.nanmax(t) == 448.0


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(0)
    x = (torch.randn(4096, generator=g) * 10.0 ** torch.randint(-30, 30, (4096,), generator=g)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


# ---------------------------------------------------------------- brute force
def _brute_force(case):
    a = case.host_arrays()
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    q = case.q.to(torch.float64).numpy()
    kc, vc, bt = a["k_cache"], a["v_cache"], a["block_tables"]
    page = kc.shape[1]
    hkv, d = kc.shape[2], kc.shape[3]
    hq = q.shape[1]
    kd, vd, sc = (float(np.float32(a[k])) for k in ("k_descale", "v_descale", "softmax_scale"))
    out = np.zeros(q.shape)
    cu = a["cu_seqlens_q"]
    for b, seq_len in enumerate(a["seq_lens"]):
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            t = int(cu[b]) + i
            last_visible = int(seq_len) - n + i
            for head in range(hq):
                kvh = head // (hq // hkv)
                scores, rows = [], []
                for j in range(int(seq_len)):
                    if j > last_visible:
                        continue
                    pg, slot = int(bt[b][j // page]), j % page
                    kvec = [dec[kc[pg, slot, kvh, e]] * kd for e in range(d)]
                    vvec = [dec[vc[pg, slot, kvh, e]] * vd for e in range(d)]
                    scores.append(math.fsum(q[t, head, e] * kvec[e] for e in range(d)) * sc)
                    rows.append(vvec)
                if not scores:
                    continue
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                den = math.fsum(w)
                for e in range(d):
                    out[t, head, e] = math.fsum(w[j] * rows[j][e] for j in range(len(w))) / den
    return out


def _brute_force_lse(case):
    """ln sum exp(score) per (token, head) in pure Python (math.fsum), -inf without a visible key."""
    a = case.host_arrays()
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    q = case.q.to(torch.float64).numpy()
    kc, bt = a["k_cache"], a["block_tables"]
    page, hkv, d = kc.shape[1], kc.shape[2], kc.shape[3]
    hq = q.shape[1]
    kd, sc = float(np.float32(a["k_descale"])), float(np.float32(a["softmax_scale"]))
    lse = np.full(q.shape[:2], -math.inf)
    cu = a["cu_seqlens_q"]
    for b, seq_len in enumerate(a["seq_lens"]):
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            t = int(cu[b]) + i
            for head in range(hq):
                kvh = head // (hq // hkv)
                scores = []
                for j in range(min(int(seq_len), int(seq_len) - n + i + 1)):
                    pg, slot = int(bt[b][j // page]), j % page
                    scores.append(math.fsum(q[t, head, e] * dec[kc[pg, slot, kvh, e]] * kd for e in range(d)) * sc)
                if scores:
                    top = max(scores)
                    lse[t, head] = top + math.log(math.fsum(math.exp(x - top) for x in scores))
    return lse


def _brute_force_options(case, window_left, softcap, sinks):
    """(out, lse) with a left window, a score soft-cap and sink logits, in pure Python."""
    a = case.host_arrays()
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    q = case.q.to(torch.float64).numpy()
    kc, vc, bt = a["k_cache"], a["v_cache"], a["block_tables"]
    page, hkv, d = kc.shape[1], kc.shape[2], kc.shape[3]
    hq = q.shape[1]
    kd, vd, sc = (float(np.float32(a[k])) for k in ("k_descale", "v_descale", "softmax_scale"))
    out = np.zeros(q.shape)
    lse = np.full(q.shape[:2], -math.inf)
    cu = a["cu_seqlens_q"]
    for b, seq_len in enumerate(a["seq_lens"]):
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            t = int(cu[b]) + i
            pos = int(seq_len) - n + i
            for head in range(hq):
                kvh = head // (hq // hkv)
                scores, rows = [], []
                for j in range(int(seq_len)):
                    if j > pos or (window_left >= 0 and j < pos - window_left):
                        continue
                    pg, slot = int(bt[b][j // page]), j % page
                    x = math.fsum(q[t, head, e] * dec[kc[pg, slot, kvh, e]] * kd for e in range(d)) * sc
                    scores.append(softcap * math.tanh(x / softcap) if softcap > 0 else x)
                    rows.append([dec[vc[pg, slot, kvh, e]] * vd for e in range(d)])
                terms = scores + ([float(np.float32(sinks[head]))] if sinks is not None else [])
                if not terms:
                    continue
                top = max(terms)
                w = [math.exp(x - top) for x in scores]
                den = math.fsum(math.exp(x - top) for x in terms)
                lse[t, head] = top + math.log(den)
                for e in range(d):
                    out[t, head, e] = math.fsum(w[j] * rows[j][e] for j in range(len(w))) / den
    return out, lse


OPTION_CASES = [
    dict(window_left=5, softcap=0.0, sinks=None),
    dict(window_left=0, softcap=0.0, sinks=None),
    dict(window_left=-1, softcap=2.0, sinks=None),
    dict(window_left=-1, softcap=0.0, sinks=[0.5, -1.0, 3.0, -20.0]),
    dict(window_left=17, softcap=1.5, sinks=[1.0, 2.0, -0.5, 0.0]),
]


@pytest.mark.parametrize("opts", OPTION_CASES, ids=[str(i) for i in range(len(OPTION_CASES))])
def test_oracle_options_match_brute_force(opts):
    case = _tiny([40, 9, 23], [4, 2, 3], 4, 1, d=8, page=4, seed=31, descale="fixed")
    arrs = case.host_arrays()
    got = oracle.attend(**arrs, **opts)
    got_lse = oracle.attend_lse(**arrs, **opts)
    ref, ref_lse = _brute_force_options(case, **opts)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * max(np.abs(ref).max(), 1e-300))
    assert np.array_equal(np.isinf(got_lse), np.isinf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.allclose(got_lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)


def test_oracle_option_closed_forms():
    d = 8
    k_codes = np.stack([np.full((1, d), c, np.uint8) for c in (0x30, 0x38, 0x40, 0x44, 0x48)])   # 0.5, 1, 2, 3, 4
    v_codes = np.stack([np.full((1, d), c, np.uint8) for c in (0x38, 0x40, 0x44, 0x48, 0x4c)])   # 1, 2, 3, 4, 6
    q_vals = np.full((4, 1, d), 0.25)
    prob = _single_page_problem(k_codes, v_codes, q_vals, q_len=4, scale=0.5)
    score = [0.5 * 0.25 * d * k for k in (0.5, 1.0, 2.0, 3.0, 4.0)]
    # window 0: each query sees only its own position
    out0 = oracle.attend(**prob, window_left=0)
    lse0 = oracle.attend_lse(**prob, window_left=0)
    for i in range(4):
        pos = 1 + i
        assert np.all(out0[i, 0] == (1.0, 2.0, 3.0, 4.0, 6.0)[pos])
        assert lse0[i, 0] == pytest.approx(score[pos], rel=1e-15)
    # a window at least the sequence length is no window
    assert np.array_equal(oracle.attend(**prob, window_left=5), oracle.attend(**prob))
    # soft-cap on a single visible key: lse = cap tanh(s / cap), out unchanged
    one = _single_page_problem(k_codes[:1], v_codes[:1], q_vals[:1], q_len=1, scale=0.5)
    assert oracle.attend_lse(**one, softcap=0.375)[0, 0] == pytest.approx(0.375 * math.tanh(score[0] / 0.375),
                                                                         rel=1e-14)
    assert np.all(oracle.attend(**one, softcap=0.375) == 1.0)
    # a sink on a single key: out = v sigmoid(s - sink), lse = logaddexp(s, sink)
    sink = 0.75
    out_s = oracle.attend(**one, sinks=[sink])
    assert out_s[0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(sink - score[0])), rel=1e-14)
    assert oracle.attend_lse(**one, sinks=[sink])[0, 0] == pytest.approx(np.logaddexp(score[0], sink), rel=1e-14)
    # a sink of -inf is no sink
    assert np.array_equal(oracle.attend(**prob, sinks=[-np.inf]), oracle.attend(**prob))


BRUTE_CASES = [
    dict(ctx=[13], q_lens=[4], hq=2, hkv=1),
    dict(ctx=[1, 7, 40], q_lens=[1, 3, 4], hq=4, hkv=2),
    dict(ctx=[16, 17, 5], q_lens=[2, 4, 1], hq=4, hkv=1, d=4),
    dict(ctx=[33, 2], q_lens=[4, 2], hq=2, hkv=2, page=16),
    dict(ctx=[9, 25], q_lens=[3, 4], hq=4, hkv=1, descale="fixed"),
]


@pytest.mark.parametrize("cfg", BRUTE_CASES, ids=[str(i) for i in range(len(BRUTE_CASES))])
def test_oracle_matches_brute_force(cfg):
    case = _tiny(seed=11, **cfg)
    got = _run_oracle(case)
    ref = _brute_force(case)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("cfg", BRUTE_CASES, ids=[str(i) for i in range(len(BRUTE_CASES))])
def test_oracle_lse_matches_brute_force(cfg):
    case = _tiny(seed=13, **cfg)
    got = oracle.attend_lse(**case.host_arrays())
    ref = _brute_force_lse(case)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_oracle_lse_closed_forms():
    """One visible key: lse is its score. n identical visible keys: ln n + score."""
    d = 8
    k_codes = np.full((5, 1, d), 0x38, np.uint8)            # e4m3fn 0x38 = 1.0
    v_codes = np.zeros_like(k_codes)
    q_vals = np.array([[[0.5] * d], [[1.0] * d], [[-2.0] * d], [[0.25] * d]], np.float64)   # [4, 1, d]
    prob = _single_page_problem(k_codes, v_codes, q_vals, q_len=4, kd=0.5, scale=0.25)
    lse = oracle.attend_lse(**prob)
    for i in range(4):
        n_vis = 5 - 4 + i + 1
        score = 0.25 * float(q_vals[i, 0, 0]) * 0.5 * d
        assert lse[i, 0] == pytest.approx(math.log(n_vis) + score, rel=1e-14, abs=1e-14)
    one = _single_page_problem(k_codes[:1], v_codes[:1], q_vals[:1], q_len=1, kd=0.5, scale=0.25)
    assert oracle.attend_lse(**one)[0, 0] == pytest.approx(0.25 * 0.5 * 0.5 * d, rel=1e-15)


@pytest.mark.parametrize("num_segments", [1, 3, 16])
def test_oracle_lse_is_the_merge_of_segment_statistics(num_segments):
    """ln sum_s 2^(lse2_s) over the segments' own statistics equals the whole row's lse."""
    case = _tiny([70, 33, 5], [4, 2, 1], 4, 1, d=16, page=4, seed=21)
    a = case.host_arrays()
    lse2, _ = oracle.segment_partials(**a, num_segments=num_segments)
    merged = np.logaddexp.reduce(lse2 * math.log(2.0), axis=0)
    ref = oracle.attend_lse(**a)
    assert np.array_equal(np.isinf(merged), np.isinf(ref))
    fin = np.isfinite(ref)
    assert np.allclose(merged[fin], ref[fin], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- library special case
def _sdpa_reference(case):
    a = case.host_arrays()
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    q = case.q.to(torch.float64)
    kc, vc = torch.from_numpy(a["k_cache"]).long(), torch.from_numpy(a["v_cache"]).long()
    page, hkv = kc.shape[1], kc.shape[2]
    hq = q.shape[1]
    out = torch.zeros_like(q)
    cu = a["cu_seqlens_q"]
    for b, seq_len in enumerate(a["seq_lens"].tolist()):
        n = int(cu[b + 1] - cu[b])
        pos = torch.arange(seq_len)
        ids = torch.from_numpy(a["block_tables"][b]).long()[pos // page]
        k = dec[kc[ids, pos % page]] * float(np.float32(a["k_descale"]))   # [L, Hkv, D]
        v = dec[vc[ids, pos % page]] * float(np.float32(a["v_descale"]))
        k = k.repeat_interleave(hq // hkv, dim=1).transpose(0, 1)          # [Hq, L, D]
        v = v.repeat_interleave(hq // hkv, dim=1).transpose(0, 1)
        qs = q[int(cu[b]):int(cu[b + 1])].transpose(0, 1)                  # [Hq, n, D]
        mask = torch.arange(seq_len)[None, :] <= (seq_len - n + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qs, k.contiguous(), v.contiguous(), attn_mask=mask, scale=float(np.float32(a["softmax_scale"])))
        out[int(cu[b]):int(cu[b + 1])] = o.transpose(0, 1)
    return out.numpy()


@pytest.mark.parametrize("cfg", [
    dict(ctx=[300, 77, 1, 129], q_lens=[4, 2, 1, 3], hq=16, hkv=1, d=64, page=16),
    dict(ctx=[200, 150], q_lens=[4, 4], hq=8, hkv=2, d=32, page=16, descale="fixed"),
])
def test_oracle_matches_sdpa_fp64(cfg):
    case = _tiny(seed=5, **cfg)
    got = _run_oracle(case)
    ref = _sdpa_reference(case)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- closed forms
def _single_page_problem(k_codes, v_codes, q_vals, q_len, kd=1.0, vd=1.0, scale=0.0625, page=None):
    """Hand-built one-sequence problem; k/v codes [L, Hkv, D], q [n, Hq, D] real values."""
    L, hkv, d = k_codes.shape
    page = page or max(L, 1)
    n_pages = -(-L // page)
    kc = np.zeros((n_pages, page, hkv, d), np.uint8)
    vc = np.zeros_like(kc)
    kc.reshape(-1, hkv, d)[:L] = k_codes
    vc.reshape(-1, hkv, d)[:L] = v_codes
    q_bits = torch.tensor(q_vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return dict(q=q_bits, k_cache=kc, v_cache=vc, block_tables=np.arange(n_pages, dtype=np.int32)[None],
                seq_lens=np.array([L], np.int32), cu_seqlens_q=np.array([0, q_len], np.int32),
                k_descale=kd, v_descale=vd, softmax_scale=scale)


def test_single_key_returns_v_exactly():
    rng = np.random.default_rng(0)
    d = 256
    table = oracle.e4m3fn_decode_table()
    finite = np.flatnonzero(~np.isnan(table))
    k = rng.choice(finite, size=(1, 1, d)).astype(np.uint8)
    v = rng.choice(finite, size=(1, 1, d)).astype(np.uint8)
    q = rng.standard_normal((1, 16, d))
    out = oracle.attend(**_single_page_problem(k, v, q, 1, kd=0.37, vd=1.75))
    expect = table[v[0, 0]] * float(np.float32(1.75))
    assert np.array_equal(out[0], np.broadcast_to(expect, (16, d)))


def test_identical_keys_give_prefix_means():
    rng = np.random.default_rng(1)
    L, d, n = 37, 16, 4
    table = oracle.e4m3fn_decode_table()
    finite = np.flatnonzero(np.abs(table) < 8)
    k_row = rng.choice(finite, size=(1, 1, d)).astype(np.uint8)
    k = np.repeat(k_row, L, axis=0)
    v = rng.choice(finite, size=(L, 1, d)).astype(np.uint8)
    q = rng.standard_normal((n, 2, d))
    out = oracle.attend(**_single_page_problem(k, v, q, n, page=16))
    vals = table[v[:, 0, :]]
    for i in range(n):
        vis = L - n + i + 1
        assert np.allclose(out[i], vals[:vis].mean(axis=0)[None], rtol=1e-13, atol=1e-13)


def _dominant_key_problem(num_keys, d, scale):
    # Q[...,0] = 8, K[key 0, dim 0] = 14, every other Q/K coordinate 0; V = +1 for
    # key 0 and -1 for the others; unit descales; one query that sees every key.
    code = {v: c for c, v in enumerate(oracle.e4m3fn_decode_table()) if not np.isnan(v) and c < 128}
    k = np.zeros((num_keys, 1, d), np.uint8)
    k[0, 0, 0] = code[14.0]
    v = np.full((num_keys, 1, d), 0x80 | code[1.0], np.uint8)
    v[0] = code[1.0]
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 8.0
    return _single_page_problem(k, v, q, 1, scale=scale, page=16)


def test_dominant_key_closed_form_hd256():
    n, d, scale = 4000, 256, 1.0 / 16.0
    out = oracle.attend(**_dominant_key_problem(n, d, scale))
    a = math.exp(8 * 14 * scale)
    expect = (a - (n - 1)) / (a + (n - 1))
    assert np.allclose(out, expect, rtol=0, atol=1e-12)


def test_dominant_key_matches_printed_value():
    fields = {}
    for line in open(os.path.join(GOLDEN, "fp8_p_underflow_example.txt")):
        if line.strip() and not line.startswith("#"):
            key, val = line.split()
            fields[key] = float(val)
    n, d = int(fields["num_keys"]), int(fields["qk_head_dim"])
    out = oracle.attend(**_dominant_key_problem(n, d, 1.0 / math.sqrt(d)))
    half_ulp = 0.5 * 10.0 ** -int(fields["printed_decimals"])
    assert np.all(np.abs(out - fields["exact_output"]) <= half_ulp)
    # the same value from the closed form, and the fp8-P failure mode the page describes
    a = math.exp(fields["q_dim0"] * fields["k_key0_dim0"] * float(np.float32(1.0 / math.sqrt(d))))
    assert abs(out[0, 0, 0] - (a - (n - 1)) / (a + (n - 1))) < 1e-12
    tail_p = math.exp(-fields["q_dim0"] * fields["k_key0_dim0"] / math.sqrt(d))
    assert torch.tensor(tail_p).to(torch.float8_e4m3fn).item() == 0.0  # rounds to 0 in fp8
    assert fields["fp8_p_output"] == 1.0


# ---------------------------------------------------------------- invariants
def test_page_pool_permutation_invariance():
    case = _tiny([45, 30, 3], [4, 2, 1], 4, 2, d=16, page=16, seed=3)
    shuffled = permute_pool(case, seed=9)
    assert not torch.equal(case.block_tables, shuffled.block_tables)
    assert np.array_equal(_run_oracle(case), _run_oracle(shuffled))


def test_duplicated_kv_heads_match_single_head():
    one = _tiny([50, 20], [4, 3], 4, 1, d=16, page=16, seed=4)
    two_k = one.k_cache.repeat_interleave(2, dim=2)
    two_v = one.v_cache.repeat_interleave(2, dim=2)
    a = one.host_arrays()
    a2 = dict(a, k_cache=two_k.numpy(), v_cache=two_v.numpy())
    # with 2 KV heads and G = 2, query heads {0,1} read head 0 and {2,3} read head 1
    assert np.allclose(oracle.attend(**a), oracle.attend(**a2), rtol=1e-15, atol=0)


def test_descale_algebra():
    case = _tiny([60, 9], [4, 4], 4, 1, d=16, page=16, seed=6)
    a = case.host_arrays()
    base = oracle.attend(**a)
    doubled = oracle.attend(**dict(a, v_descale=a["v_descale"] * 2))
    assert np.array_equal(doubled, 2 * base)
    c = 4.0
    moved = oracle.attend(**dict(a, k_descale=a["k_descale"] * c, softmax_scale=a["softmax_scale"] / c))
    assert np.allclose(moved, base, rtol=1e-13, atol=1e-13)


def test_empty_query_and_no_visible_key_rows():
    case = _tiny([10, 2, 8], [0, 3, 2], 2, 1, d=8, page=4, seed=7)
    out = _run_oracle(case)
    # sequence 1 has 2 keys for 3 queries: its first query sees none
    assert np.all(out[0] == 0.0)
    assert np.all(np.isfinite(out))


# ---------------------------------------------------------------- segment partials
@pytest.mark.parametrize("num_segments", [1, 2, 3, 7, 16])
def test_segment_partials_merge_to_attend(num_segments):
    case = _tiny([100, 33, 5], [4, 1, 2], 4, 2, d=16, page=16, seed=8)
    a = case.host_arrays()
    lse2, o = oracle.segment_partials(**a, num_segments=num_segments)
    top = lse2.max(axis=0)
    w = np.where(np.isneginf(lse2), 0.0, np.exp2(lse2 - top))
    merged = (w[..., None] * o).sum(axis=0) / w.sum(axis=0)[..., None]
    assert np.allclose(merged, oracle.attend(**a), rtol=1e-12, atol=1e-12)
    # a 5-token sequence has one page: every segment after the first is empty
    assert np.all(np.isneginf(lse2[1:, 5:7])) and np.all(o[1:, 5:7] == 0)


def test_segment_ranges_cover_pages_in_order():
    for pages in (0, 1, 5, 63, 137, 2188):
        for s in (1, 2, 3, 16, 64):
            r = oracle.segment_page_ranges(pages, s)
            assert len(r) == s
            flat = [p for b, e in r for p in range(b, e)]
            assert flat == list(range(pages))
    assert sum(e > b for b, e in oracle.segment_page_ranges(2188, 64)) == 63
    assert sum(e > b for b, e in oracle.segment_page_ranges(49, 64)) == 49


# ---------------------------------------------------------------- planted mistakes
def _mutations():
    good_table = oracle_attention.e4m3fn_decode_table
    good_visible = oracle_attention.visible_key_count
    good_gather = oracle_attention._gather_sequence

    def table_bad_bias():
        t = good_table().copy()
        t[(np.arange(256) & 0x78) == 0] *= 2.0      # subnormals with the wrong exponent
        return t

    def table_bad_sign():
        t = good_table().copy()
        t[0x80:] = np.abs(t[0x80:])
        return t

    return {
        "mask_off_by_one": ("visible_key_count", lambda L, n, i: good_visible(L, n, i) - 1),
        "mask_top_left": ("visible_key_count", lambda L, n, i: max(0, min(L, i + 1))),
        "subnormal_exponent": ("e4m3fn_decode_table", table_bad_bias),
        "dropped_sign": ("e4m3fn_decode_table", table_bad_sign),
        "dropped_descale": ("_gather_sequence", lambda t, c, row, L, ds: good_gather(t, c, row, L, 1.0)),
        "page_slot_swap": ("_gather_sequence",
                           lambda t, c, row, L, ds: good_gather(t, c[:, ::-1], row, L, ds)),
    }


@pytest.mark.parametrize("name", ["mask_off_by_one", "mask_top_left", "subnormal_exponent", "dropped_sign",
                                  "dropped_descale", "page_slot_swap"])
def test_planted_mistake_is_caught_in_lse(monkeypatch, name):
    attr, bad = _mutations()[name]
    case = _tiny([21, 6], [4, 3], 4, 2, d=8, page=4, seed=12, descale="fixed")
    ref = _brute_force_lse(case)
    monkeypatch.setattr(oracle_attention, attr, bad)
    got = oracle_attention.attend_lse(**case.host_arrays())
    fin = np.isfinite(ref) & np.isfinite(got)
    assert not (np.array_equal(np.isinf(got), np.isinf(ref)) and np.allclose(got[fin], ref[fin], rtol=1e-6, atol=1e-9))


def _option_mutations():
    good_first = oracle_attention.first_visible_key
    good_cap = oracle_attention._softcapped
    return {
        "window_off_by_one": ("first_visible_key", lambda L, n, i, w: good_first(L, n, i, w) + (1 if w >= 0 else 0)),
        "window_ignored": ("first_visible_key", lambda L, n, i, w: 0),
        "softcap_outer_factor_dropped": ("_softcapped", lambda x, c: np.tanh(x / c) if c > 0 else x),
        "softcap_ignored": ("_softcapped", lambda x, c: x),
    }


@pytest.mark.parametrize("name", sorted(_option_mutations()))
def test_planted_option_mistake_is_caught(monkeypatch, name):
    attr, bad = _option_mutations()[name]
    case = _tiny([40, 9, 23], [4, 2, 3], 4, 1, d=8, page=4, seed=31, descale="fixed")
    opts = dict(window_left=6, softcap=1.5, sinks=None)
    ref, _ = _brute_force_options(case, **opts)
    monkeypatch.setattr(oracle_attention, attr, bad)
    got = oracle_attention.attend(**case.host_arrays(), **opts)
    assert not np.allclose(got, ref, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("name", sorted(_mutations()))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, bad = _mutations()[name]
    case = _tiny([21, 6], [4, 3], 4, 2, d=8, page=4, seed=12, descale="fixed")
    ref = _brute_force(case)
    monkeypatch.setattr(oracle_attention, attr, bad)
    got = oracle_attention.attend(**case.host_arrays())
    assert not np.allclose(got, ref, rtol=1e-6, atol=1e-9)
