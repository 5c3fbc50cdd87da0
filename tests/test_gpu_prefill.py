"""fp8 varlen prefill (the second workload) against the CPU oracle, through the C ABI.

What is computed: aiter PR #7375, Summary (e4m3 q/k/v with per-tensor descales,
qk head dim 192 / v head dim 128, packed THD rows, causal bottom-right or not,
optional LSE). The inputs are exact e4m3 bytes on both sides, so the only
differences from the exact fp64 oracle are the kernel's e4m3 rounding of P (a
relative error of at most delta = 2^-4 per weight, with a power-of-two scale per
32 keys so that small weights keep their mantissa), fp32 accumulation and the
bf16 output. Bars, from that arithmetic:
- per element: weights off by at most delta move a softmax average by at most
  delta / (1 - delta) < 0.07 times the spread (max - min) of the V values the
  row averages; plus one bf16 rounding (2^-8 relative);
- typical: mean error <= 0.03 sigma of the output and cosine similarity >= 0.999
  (each weight's error is about 2% RMS, so the output's relative error is about
  2% and 1 - cos about 2e-4);
- lse within ln(1 + 2^-4) rounded up to 0.07.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import PrefillWorkload, make_prefill_case, prefill_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SPREAD, MEAN_SIGMA, LSE_TOL, COS_MIN = 0.07, 0.03, 0.07, 0.999
TABLE = oracle.e4m3fn_decode_table()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _run(c, **kw):
    return pfkv.prefill_attn(c.q, c.k, c.v, c.q_descale, c.k_descale, c.v_descale, c.cu_seqlens_q, c.cu_seqlens_k,
                             c.max_seqlen_q, is_causal=c.causal, **kw)


def _v_spread(arrs):
    """Per output element, max - min of the V values its row can see (over all of
    its sequence's keys for the row's KV head, an upper bound under a causal mask)."""
    q, v = arrs["q"], TABLE[arrs["v"]] * arrs["v_descale"]
    hq_n, hkv_n = q.shape[1], v.shape[1]
    spread = np.zeros((q.shape[0], hq_n, v.shape[2]))
    cq, ck = arrs["cu_seqlens_q"], arrs["cu_seqlens_k"]
    for b in range(len(cq) - 1):
        if ck[b + 1] == ck[b]:
            continue
        vb = v[ck[b]:ck[b + 1]]
        rng = vb.max(axis=0) - vb.min(axis=0)          # [Hkv, Dv]
        for h in range(hq_n):
            spread[cq[b]:cq[b + 1], h] = rng[h * hkv_n // hq_n]
    return spread


def _check(got, ref, label, arrs):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), label
    sigma = ref.std()
    err = np.abs(g - ref)
    bound = SPREAD * _v_spread(arrs) + 2.0 ** -8 * np.abs(ref)
    cos = float((g * ref).sum() / max(np.linalg.norm(g) * np.linalg.norm(ref), 1e-300))
    print(f"[prefill] {label}: max err/bound={np.max(err / np.maximum(bound, 1e-30)):.3f} "
          f"max|err|/std={err.max() / sigma:.4f} mean|err|/std={err.mean() / sigma:.5f} cos={cos:.7f}", flush=True)
    assert np.all(err <= bound), label
    assert err.mean() / sigma <= MEAN_SIGMA and cos >= COS_MIN, label


def _check_lse(got, ref, label):
    g = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), label
    fin = np.isfinite(ref)
    err = np.abs(g[fin] - ref[fin]).max() if fin.any() else 0.0
    print(f"[prefill lse] {label}: max|err|={err:.2e}", flush=True)
    assert err <= LSE_TOL, label


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_parity_varlen(causal):
    w = prefill_workload("prefill_small", causal=causal)
    c = make_prefill_case(w, "cpu").to(DEV)
    out, lse = _run(c, return_lse=True)
    torch.cuda.synchronize()
    arrs = c.to("cpu").host_arrays()
    _check(out, oracle.prefill_attend(**arrs), f"small causal={causal}", arrs)
    _check_lse(lse, oracle.prefill_lse(**arrs), f"small causal={causal}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 2), (6, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_heads_and_tiles(hq, hkv, causal):
    """Several 256-row query tiles, key counts off the 64-key tile, GQA."""
    w = PrefillWorkload("t", ((600, 600), (257, 1000), (3, 65)), hq, hkv, causal, seed=hq * 10 + hkv)
    c = make_prefill_case(w, "cpu").to(DEV)
    out = _run(c)
    torch.cuda.synchronize()
    arrs = c.to("cpu").host_arrays()
    _check(out, oracle.prefill_attend(**arrs), f"hq={hq} hkv={hkv} causal={causal}", arrs)


def test_prefill_edge_sequences():
    """No keys at all, fewer keys than queries (causal rows with nothing to see),
    one query, one key."""
    w = PrefillWorkload("e", ((5, 0), (40, 7), (1, 1), (1, 300), (70, 64)), 2, 1, True, seed=5)
    c = make_prefill_case(w, "cpu").to(DEV)
    out, lse = _run(c, return_lse=True)
    torch.cuda.synchronize()
    arrs = c.to("cpu").host_arrays()
    ref = oracle.prefill_attend(**arrs)
    ref_lse = oracle.prefill_lse(**arrs)
    _check_lse(lse, ref_lse, "edges")
    empty = np.isneginf(ref_lse).T   # [T, Hq]
    got = out.float().cpu().numpy()
    assert np.all(got[empty] == 0)
    _check(out, ref, "edges", arrs)
    # the one-key sequence (query row 45, key row 7) returns that key's V, to one bf16 rounding
    expect = torch.from_numpy(TABLE[c.v[7, 0].cpu().numpy()] * float(c.v_descale.item())).float()
    assert torch.allclose(out[45, 0].cpu().float(), expect, rtol=2.0 ** -8, atol=0)


def test_prefill_keeps_small_probabilities():
    """The same page's underflow example (tests/golden/fp8_p_underflow_example.txt):
    64 queries, 16384 keys, one head, unit descales, Q[:,0,0] = 8, K[0,0,0] = 14,
    V = +1 on key 0 and -1 elsewhere. Exact O ~ -0.6699; e4m3 P without a block
    scale gives +1. The per-32-key scale keeps the tail."""
    sq, sk = 64, 16384
    code = lambda x: int(np.flatnonzero(TABLE == x)[0])
    q = torch.zeros((sq, 1, 192), dtype=torch.uint8)
    k = torch.zeros((sk, 1, 192), dtype=torch.uint8)
    v = torch.full((sk, 1, 128), code(-1.0), dtype=torch.uint8)
    q[:, 0, 0] = code(8.0)
    k[0, 0, 0] = code(14.0)
    v[0] = code(1.0)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    cq = torch.tensor([0, sq], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, sk], dtype=torch.int32, device=DEV)
    out = pfkv.prefill_attn(q.to(DEV), k.to(DEV), v.to(DEV), one, one, one, cq, ck, sq)
    torch.cuda.synchronize()
    a = math.exp(8 * 14 / math.sqrt(192))
    exact = (a - (sk - 1)) / (a + (sk - 1))
    got = out.float().cpu().numpy()
    print(f"[prefill dominant] got {got[0, 0, 0]:.5f} exact {exact:.5f}", flush=True)
    assert np.max(np.abs(got - exact)) < 1e-2


def test_prefill_strided_views_bitwise():
    """q / k / v as head slices of wider buffers and out inside a wider buffer give
    the dense call's bits."""
    w = PrefillWorkload("s", ((200, 333), (90, 90)), 4, 2, True, seed=21)
    c = make_prefill_case(w, "cpu").to(DEV)
    dense = _run(c)
    qw = torch.zeros((c.q.shape[0], 6, 192), dtype=torch.uint8, device=DEV)
    kw = torch.zeros((c.k.shape[0], 5, 192), dtype=torch.uint8, device=DEV)
    vw = torch.zeros((c.v.shape[0], 3, 144), dtype=torch.uint8, device=DEV)
    qw[:, 1:5] = c.q
    kw[:, 2:4] = c.k
    vw[:, 1:3, :128] = c.v
    ow = torch.zeros((c.q.shape[0], 5, 136), dtype=torch.bfloat16, device=DEV)
    out = ow[:, 1:5, :128]
    pfkv.prefill_attn(qw[:, 1:5], kw[:, 2:4], vw[:, 1:3, :128], c.q_descale, c.k_descale, c.v_descale,
                      c.cu_seqlens_q, c.cu_seqlens_k, c.max_seqlen_q, is_causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous().view(torch.int16), dense.view(torch.int16))
    assert torch.all(ow[:, 0] == 0) and torch.all(ow[:, :, 128:] == 0)


def test_prefill_rerun_and_graph_replay_bitwise():
    c = make_prefill_case(prefill_workload("prefill_small"), "cpu").to(DEV)
    first = _run(c).clone()
    for _ in range(3):
        again = _run(c)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
    out = torch.empty_like(first)
    _run(c, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        _run(c, out=out)
    for k in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), k


def test_prefill_chunked_merge():
    """One call over prefix + chunk (non-causal) equals two calls over the key
    halves merged by their lse, to the fp8-P band (the page's chunked-prefill test)."""
    w = PrefillWorkload("m", ((128, 700),), 2, 1, False, seed=23)
    c = make_prefill_case(w, "cpu").to(DEV)
    full = _run(c).float()
    parts = []
    for lo, hi in ((0, 300), (300, 700)):
        ck = torch.tensor([0, hi - lo], dtype=torch.int32, device=DEV)
        parts.append(pfkv.prefill_attn(c.q, c.k[lo:hi], c.v[lo:hi], c.q_descale, c.k_descale, c.v_descale,
                                       c.cu_seqlens_q, ck, c.max_seqlen_q, return_lse=True))
    (o1, l1), (o2, l2) = parts
    m = torch.maximum(l1, l2)
    w1, w2 = torch.exp(l1 - m).T[:, :, None], torch.exp(l2 - m).T[:, :, None]
    merged = (o1.float() * w1 + o2.float() * w2) / (w1 + w2)
    torch.cuda.synchronize()
    arrs = c.to("cpu").host_arrays()
    ref = oracle.prefill_attend(**arrs)
    _check(merged, ref, "merged halves", arrs)
    _check(full, ref, "one call", arrs)


def _sub_problem(arrs, head, q_lo, q_hi, k_lo, k_hi):
    """Rows q_lo..q_hi of one head against keys k_lo..k_hi, as a one-sequence problem."""
    sub = dict(arrs)
    sub["q"] = arrs["q"][q_lo:q_hi, head:head + 1]
    sub["k"] = arrs["k"][k_lo:k_hi, head:head + 1]
    sub["v"] = arrs["v"][k_lo:k_hi, head:head + 1]
    sub["cu_seqlens_q"] = np.array([0, q_hi - q_lo], np.int32)
    sub["cu_seqlens_k"] = np.array([0, k_hi - k_lo], np.int32)
    return sub


@pytest.mark.parametrize("name", ["prefill_12k", "prefill_12k_causal"])
def test_prefill_target_shape_sampled(name):
    """The pages' target shape (12288 queries over 14336 keys, 96 heads) in the
    benchmark's launch configuration. Sampled against the oracle: the first and
    the last 384 rows of two heads. With the bottom-right causal mask the first R
    rows see keys 0 .. Lk - Lq + R - 1 and the last R rows all keys, each again a
    bottom-right problem of its own, so the samples are exact sub-problems."""
    w = prefill_workload(name)
    c = make_prefill_case(w, DEV)
    out, lse = _run(c, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    lq, lk = w.lens[0]
    arrs = dict(q=c.q.cpu().numpy(), k=c.k.cpu().numpy(), v=c.v.cpu().numpy(), q_descale=float(c.q_descale.item()),
                k_descale=float(c.k_descale.item()), v_descale=float(c.v_descale.item()), softmax_scale=None,
                causal=w.causal)
    r = 384
    for head in (0, 61):
        for q_lo, q_hi, k_hi in ((0, r, lk - lq + r if w.causal else lk), (lq - r, lq, lk)):
            sub = _sub_problem(arrs, head, q_lo, q_hi, 0, k_hi)
            label = f"{name} head {head} rows {q_lo}..{q_hi}"
            _check(out[q_lo:q_hi, head:head + 1], oracle.prefill_attend(**sub), label, sub)
            _check_lse(lse[head:head + 1, q_lo:q_hi], oracle.prefill_lse(**sub), label)


def test_prefill_rows_past_4_gib_bitwise():
    """K and V rows 1 MiB apart, so that keys from 4096 on sit past the first
    4 GiB of their buffers (byte offsets above 32 bits): the dense call's bits."""
    w = PrefillWorkload("far", ((100, 3000), (64, 2200)), 2, 1, True, seed=23)
    c = make_prefill_case(w, "cpu").to(DEV)
    dense = _run(c)
    total_k, stride = c.k.shape[0], 1 << 20
    assert (total_k - 1) * stride > 1 << 32
    kb = torch.empty(total_k * stride, dtype=torch.uint8, device=DEV)
    vb = torch.empty(total_k * stride, dtype=torch.uint8, device=DEV)
    try:
        k = kb.as_strided((total_k, 1, 192), (stride, 192, 1))
        v = vb.as_strided((total_k, 1, 128), (stride, 128, 1))
        k.copy_(c.k)
        v.copy_(c.v)
        far = pfkv.prefill_attn(c.q, k, v, c.q_descale, c.k_descale, c.v_descale, c.cu_seqlens_q, c.cu_seqlens_k,
                                c.max_seqlen_q, is_causal=True)
        torch.cuda.synchronize()
        assert torch.equal(far.view(torch.int16), dense.view(torch.int16))
    finally:
        del kb, vb
        torch.cuda.empty_cache()


def _draw_prefill_cases(n=32, seed=77):
    """Seeded combinations: 1 to 4 sequences of 1 to 700 queries over 0 to 1200
    keys (some with fewer keys than queries), 1 to 4 KV heads with 1 to 4 query
    heads each, causal or not."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        lens = tuple((int(rng.integers(1, 701)), int(rng.integers(0, 1201))) for _ in range(int(rng.integers(1, 5))))
        hkv = int(rng.integers(1, 5))
        hq = hkv * int(rng.integers(1, 5))
        cases.append(dict(id=k, lens=lens, hq=hq, hkv=hkv, causal=bool(rng.integers(0, 2)), seed=500 + k))
    return cases


PREFILL_SWEEP = _draw_prefill_cases()


@pytest.mark.parametrize("c", PREFILL_SWEEP, ids=[f"case{c['id']}" for c in PREFILL_SWEEP])
def test_prefill_sweep_case(c):
    print(f"[prefill sweep] {c}", flush=True)
    w = PrefillWorkload(f"sw{c['id']}", c["lens"], c["hq"], c["hkv"], c["causal"], seed=c["seed"])
    cs = make_prefill_case(w, "cpu").to(DEV)
    out, lse = _run(cs, return_lse=True)
    torch.cuda.synchronize()
    arrs = cs.to("cpu").host_arrays()
    _check(out, oracle.prefill_attend(**arrs), f"sweep case {c['id']}", arrs)
    _check_lse(lse, oracle.prefill_lse(**arrs), f"sweep case {c['id']}")
