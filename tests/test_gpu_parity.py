"""Parity of the HIP path with the CPU oracle, and its bit-exactness invariants.

Every call goes through the C ABI (ctypes binding) of the in-tree libpfkv.so.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Case, Workload, make_case, permute_pool, workload

from gpu_util import assert_parity, error_stats, oracle_for, rows_of, run, subset

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()
    arch, cus = pfkv.binding.device_info(0)
    print(f"[device] {arch} CUs={cus}", flush=True)


def _case(name, **over):
    w = workload(name, **over)
    return make_case(w, "cpu").to(DEV)


# ------------------------------------------------------------------ small configs, full oracle
@pytest.mark.parametrize("name", ["tiny", "tiny_fixed_descale", "tiny_override_descale"])
def test_tiny_parity(name):
    case = _case(name)
    out = run(case, num_segments=4)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), name)


@pytest.mark.parametrize("segments", [None, 1, 3, 7, 64])
def test_multigroup_parity(segments):
    case = _case("multigroup")    # 32 q heads / 2 KV heads, context 777, 2 sequences
    out = run(case, num_segments=segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"multigroup S={segments}")


def test_ragged_parity():
    case = _case("ragged")        # 8 sequences, contexts 6..105000, q_len 1..4
    print(f"[ragged] ctx={case.workload.ctx} q_lens={case.workload.q_lens}", flush=True)
    out = run(case)               # heuristic: 32 segments on 256 CUs, empty tail segments
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), "ragged")


def test_gqa8_three_seqs_parity():
    w = Workload(name="g8x3", ctx=(8000, 8000, 8000), q_lens=(4, 4, 4), num_q_heads=8, num_kv_heads=1,
                 num_segments=16, seed=31)
    case = make_case(w, "cpu").to(DEV)
    out = run(case, num_segments=16)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), "gqa8 3x8000")


@pytest.mark.parametrize("segments", [1, 2, 3, 7, 16, 17, 24, 33, 40, 64])
def test_segment_count_independence(segments):
    # 17-32 segments: the reduce merges each row with two waves, 33-64 with four
    # (uneven shares at 17, 33 and 40)
    w = Workload(name="s", ctx=(8000, 1234, 31), q_lens=(4, 2, 1), num_q_heads=16, num_kv_heads=1,
                 num_segments=segments, seed=32)
    case = make_case(w, "cpu").to(DEV)
    ref = oracle_for(case)
    out = run(case, num_segments=segments)
    base = run(case, num_segments=16)
    torch.cuda.synchronize()
    assert_parity(out, ref, f"S={segments}")
    sigma = ref.std()
    diff = (out.float() - base.float()).abs().max().item()
    assert diff <= 0.05 * sigma, diff


@pytest.mark.parametrize("segments", [1, 2, 5])
def test_long_segments_parity(segments):
    # 20000 tokens in one to five segments: hundreds of steps per work-group,
    # several 64-step windows of cached page ids per wave
    w = Workload(name="longseg", ctx=(20000, 4100, 33), q_lens=(4, 1, 2), num_q_heads=16, num_kv_heads=1,
                 num_segments=segments, seed=36)
    case = make_case(w, "cpu").to(DEV)
    out = run(case, num_segments=segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"long segments S={segments}")


# ------------------------------------------------------------------ full-size shapes, every row
@pytest.mark.parametrize("name", ["prod", "gqa8", "long", "occupancy", "decode"])
def test_full_size_all_rows(name):
    """The full-size shapes in the bench's launch configuration, every output
    row of every sequence against the oracle (which reads only the pages the
    sequences use)."""
    w = workload(name)
    case = make_case(w, DEV)
    out = run(case, num_segments=w.num_segments)
    torch.cuda.synchronize()
    seqs = list(range(w.num_seqs))
    ref = oracle_for(subset(case, seqs))
    assert_parity(out, ref, f"{name}, all {w.num_seqs} sequences")


@pytest.mark.parametrize("n,segments,balance", [(1024, None, False), (1024, 3, False), (200, 16, True)])
def test_large_decode_batch(n, segments, balance):
    """Many short sequences (contexts log-uniform in [1, 2000], 1 to 4 query
    tokens), every row against the oracle: 1024 of them with the heuristic's
    one segment (N x Hkv above the CU count: the direct path) and with 3
    segments (3072 work-groups, renumbered over the XCDs); 200 with balanced
    segments (cap 16), where the 56 slots beyond one per sequence go to the
    longest contexts."""
    rng = np.random.default_rng(36)
    q_lens = tuple(int(x) for x in rng.integers(1, 5, size=n))
    ctx = tuple(max(int(round(math.exp(rng.uniform(0.0, math.log(2000))))), q) for q in q_lens)
    w = Workload(name=f"batch{n}", ctx=ctx, q_lens=q_lens, num_q_heads=16, num_kv_heads=1,
                 num_segments=segments, seed=36)
    case = make_case(w, "cpu").to(DEV)
    out = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q,
                           case.k_descale, case.v_descale, case.softmax_scale, num_segments=segments,
                           balance_segments=balance)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"{n} sequences S={segments} balanced={balance}")


@pytest.mark.parametrize("segments", [1, None])
def test_long_single_sequence(segments):
    """One sequence of 200000 keys and 4 query tokens: at one segment a single
    work-group streams all 12500 pages (3125 steps, one page-id window refill
    per 64 steps); at the heuristic's 64 segments the partials are row-major.
    Every row against the oracle."""
    w = Workload(name="long1", ctx=(200000,), q_lens=(4,), num_q_heads=16, num_kv_heads=1,
                 num_segments=segments, seed=37)
    case = make_case(w, "cpu").to(DEV)
    out = run(case, num_segments=segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"200000 keys S={segments}")


def _tiled(case: Case, reps: int) -> Case:
    """reps copies of a problem side by side in one call: copy r has its own
    pool pages (block tables offset by r pages of the pool) and its own rows."""
    pages = case.k_cache.shape[0]
    q_lens = case.cu_seqlens_q[1:] - case.cu_seqlens_q[:-1]
    cu = torch.zeros(case.seq_lens.numel() * reps + 1, dtype=torch.int32, device=case.q.device)
    cu[1:] = torch.cumsum(q_lens.repeat(reps), 0)
    return Case(case.q.repeat(reps, 1, 1), case.k_cache.repeat(reps, 1, 1, 1), case.v_cache.repeat(reps, 1, 1, 1),
                torch.cat([case.block_tables + r * pages for r in range(reps)]), case.seq_lens.repeat(reps), cu,
                case.k_descale, case.v_descale, case.softmax_scale, -1, case.workload)


@pytest.mark.parametrize("segments", [1, 2])
def test_more_sequences_than_grid_rows(segments):
    """70000 sequences: the grid's y dimension (one row per sequence) passes
    65535. The call is 70 copies of a 1000-sequence problem (contexts 1 to 40,
    1 to 4 query tokens); every copy's output must equal the first's bit for
    bit, and the first is checked against the oracle."""
    rng = np.random.default_rng(38)
    n, reps = 1000, 70
    q_lens = tuple(int(x) for x in rng.integers(1, 5, size=n))
    ctx = tuple(int(max(q, x)) for q, x in zip(q_lens, rng.integers(1, 41, size=n)))
    w = Workload(name="n1000", ctx=ctx, q_lens=q_lens, num_q_heads=16, num_kv_heads=1, num_segments=segments,
                 seed=38)
    one = make_case(w, "cpu").to(DEV)
    many = _tiled(one, reps)
    assert many.seq_lens.numel() == n * reps > 65535
    out = run(many, num_segments=segments)
    torch.cuda.synchronize()
    T = one.q.shape[0]
    first = out[:T]
    for r in range(1, reps):
        assert torch.equal(out[r * T:(r + 1) * T].view(torch.int16), first.view(torch.int16)), r
    assert_parity(first, oracle_for(one), f"70000 sequences S={segments}, first copy")
    del many, out
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ workspace partials
@pytest.mark.parametrize("S", [8, 24])
def test_segment_partials_match_oracle(S):
    w = Workload(name="p", ctx=(3000, 300, 20), q_lens=(4, 3, 1), num_q_heads=16, num_kv_heads=1,
                 num_segments=S, seed=33)
    case = make_case(w, "cpu").to(DEV)
    T, Hq = w.total_q, w.num_q_heads
    ws = torch.zeros(pfkv.workspace_bytes(S, T, Hq), dtype=torch.uint8, device=DEV)
    run(case, num_segments=S, workspace=ws)
    torch.cuda.synchronize()
    # layout: fp16 o[S][T][Hq][256], then fp32 (m, l)[S][T][Hq]; above 16
    # segments row-major, o[T][Hq][S][256] and (m, l)[T][Hq][S]
    n_o = S * T * Hq * 256 * 2
    o16 = ws[:n_o].view(torch.float16)
    ml = ws[n_o:n_o + S * T * Hq * 8].view(torch.float32)
    if S > 16:
        o16 = o16.view(T, Hq, S, 256).permute(2, 0, 1, 3)
        ml = ml.view(T, Hq, S, 2).permute(2, 0, 1, 3)
    else:
        o16, ml = o16.view(S, T, Hq, 256), ml.view(S, T, Hq, 2)
    o16, ml = o16.double().cpu().numpy(), ml.double().cpu().numpy()
    lse2, o = oracle.segment_partials(**case.to("cpu").host_arrays(), num_segments=S)
    m, l = ml[..., 0], ml[..., 1]
    empty = np.isneginf(lse2)
    assert np.array_equal(empty, l == 0), "empty segments must carry l = 0"
    assert np.all(np.isneginf(m[empty])) and np.all(o16[empty] == 0)
    got_lse2 = m[~empty] + np.log2(l[~empty])
    assert np.max(np.abs(got_lse2 - lse2[~empty])) < 2e-3
    vd = float(case.v_descale.item())
    seg_out = o16[~empty] * vd
    sigma = o[~empty].std()
    assert np.max(np.abs(seg_out - o[~empty])) <= 0.05 * sigma


@pytest.mark.parametrize("precision", [0, 1])
def test_partials_layout_by_mode(precision):
    """Row-major partials only where documented (16-bit mode, head dim 256,
    pages of 16 or more, above 16 segments). At 24 segments the three
    sequences fill 24, 19 and 2 of them, so read in the wrong layout the
    empty-segment pattern and the segment log-sum-exps would not match the
    oracle's. The e4m3-P mode's l sums e4m3-rounded weights (relative error at
    most 2^-4 each), hence its looser bound, log2(1 + 2^-4) plus rounding."""
    w = Workload(name="p", ctx=(3000, 300, 20), q_lens=(4, 3, 1), num_q_heads=16, num_kv_heads=1,
                 num_segments=24, seed=34)
    case = make_case(w, "cpu").to(DEV)
    S, T, Hq = 24, w.total_q, w.num_q_heads
    ws = torch.zeros(pfkv.workspace_bytes(S, T, Hq), dtype=torch.uint8, device=DEV)
    run(case, num_segments=S, workspace=ws, precision=precision)
    torch.cuda.synchronize()
    ml = ws[S * T * Hq * 512:S * T * Hq * 520].view(torch.float32)
    assert pfkv.partials_row_major(precision, 256, 16, S) == (precision == 0)
    if precision == 0:
        ml = ml.view(T, Hq, S, 2).permute(2, 0, 1, 3)
    else:
        ml = ml.view(S, T, Hq, 2)
    ml = ml.double().cpu().numpy()
    lse2, _ = oracle.segment_partials(**case.to("cpu").host_arrays(), num_segments=S)
    m, l = ml[..., 0], ml[..., 1]
    empty = np.isneginf(lse2)
    assert empty.any() and (~empty).any()
    assert np.array_equal(empty, l == 0) and np.all(np.isneginf(m[empty]))
    got = m[~empty] + np.log2(l[~empty])
    tol = 2e-3 if precision == 0 else math.log2(1 + 2.0 ** -4) + 2e-3
    assert np.max(np.abs(got - lse2[~empty])) < tol


# ------------------------------------------------------------------ bit-exact invariants
def test_graph_replay_bitwise():
    case = _case("tiny")
    S = 4
    out = torch.empty_like(case.q)
    ws = torch.empty(pfkv.workspace_bytes(S, case.q.shape[0], case.q.shape[1]), dtype=torch.uint8, device=DEV)
    eager = run(case, num_segments=S).clone()
    stream = torch.cuda.Stream()
    run(case, num_segments=S, out=out, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run(case, num_segments=S, out=out, workspace=ws)
    for k in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {k} differs"
        other = run(case, num_segments=S)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))


def test_page_permutation_bitwise():
    case = _case("multigroup")
    shuffled = permute_pool(case, seed=123)
    a = run(case, num_segments=5)
    b = run(shuffled, num_segments=5)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rerun_bitwise():
    case = _case("ragged")
    a = run(case)
    outs = [run(case) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(a.view(torch.int16), o.view(torch.int16))


@pytest.mark.parametrize("group,segments", [(16, 8), (8, 8), (16, 1), (16, 40)])
def test_short_qlen_rows_match_verify_bitwise(group, segments):
    """Draft-extend (q_len 1..3) and decode rows equal the verify call's rows bit for bit
    (with one segment, through the main kernel's direct bf16 output)."""
    w = Workload(name="v", ctx=(5000, 777, 40, 16), q_lens=(4, 4, 4, 4), num_q_heads=group, num_kv_heads=1,
                 num_segments=segments, seed=34)
    case = make_case(w, "cpu").to(DEV)
    verify = run(case, num_segments=segments)
    for q_len in (1, 2, 3):
        rows = [4 * b + 4 - q_len + i for b in range(w.num_seqs) for i in range(q_len)]
        q = case.q[torch.tensor(rows, device=DEV)].contiguous()
        cu = torch.arange(0, q_len * (w.num_seqs + 1), q_len, dtype=torch.int32, device=DEV)
        short = pfkv.verify_attn(q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, cu,
                                 case.k_descale, case.v_descale, case.softmax_scale, num_segments=segments)
        torch.cuda.synchronize()
        assert torch.equal(short.view(torch.int16), verify[torch.tensor(rows, device=DEV)].view(torch.int16)), q_len


def test_single_segment_writes_out_directly():
    """With one segment the main kernel writes the bf16 output itself: the workspace stays
    untouched, the reduce entry point enqueues nothing, and the result is the full call's."""
    case = _case("multigroup")
    T, Hq = case.q.shape[0], case.q.shape[1]
    lib = pfkv.load_library()
    stream = torch.cuda.current_stream()
    handle = ctypes.c_void_p(stream.cuda_stream)
    full = run(case, num_segments=1)
    ws = torch.full((pfkv.workspace_bytes(1, T, Hq),), 0x5A, dtype=torch.uint8, device=DEV)
    out = torch.full_like(case.q, 7.0)
    args = pfkv.binding.build_args(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                                   case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale, 1, out, ws)
    assert lib.pfkv_splitkv_main(ctypes.byref(args), handle) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), full.view(torch.int16))
    assert bool((ws == 0x5A).all()), "the single-segment path must not touch the workspace"
    out.fill_(7.0)
    assert lib.pfkv_segment_reduce(ctypes.byref(args), handle) == 0
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "the reduce has nothing to do with one segment"
    assert_parity(full, oracle_for(case), "multigroup S=1 direct")


@pytest.mark.parametrize("segments,precision,balance", [(8, 0, False), (24, 0, False), (64, 0, False),
                                                         (24, 1, False), (40, 0, True)])
def test_exported_kernels_match_the_call(segments, precision, balance):
    """pfkv_splitkv_main then pfkv_segment_reduce, called by hand on the same
    arguments, give the one call's bits, on both partials layouts (segment-major
    at 8 segments and in the e4m3-P mode, row-major above 16 in the 16-bit mode,
    balanced or not)."""
    case = _case("ragged")
    T, Hq = case.q.shape[0], case.q.shape[1]
    lib = pfkv.load_library()
    handle = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    full = run(case, num_segments=segments, precision=precision) if not balance else pfkv.verify_attn(
        case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q, case.k_descale,
        case.v_descale, case.softmax_scale, num_segments=segments, balance_segments=True)
    ws = torch.zeros(pfkv.workspace_bytes(segments, T, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full_like(case.q, 7.0)
    args = pfkv.binding.build_args(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                                   case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale, segments,
                                   out, ws, precision, balance_segments=balance)
    assert lib.pfkv_splitkv_main(ctypes.byref(args), handle) == 0
    assert lib.pfkv_segment_reduce(ctypes.byref(args), handle) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), full.view(torch.int16))


# ------------------------------------------------------------------ closed forms and edge cases
def _one_sequence(k_codes, v_codes, q, q_len, kd=1.0, vd=1.0, scale=1.0 / 16, hkv=1):
    """Device Case for one sequence with hand-set fp8 codes ([L, Hkv, 256]) and Q values."""
    L = k_codes.shape[0]
    n_pages = -(-L // 16)
    kc = torch.zeros((n_pages + 1, 16, hkv, 256), dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    kc.view(-1, hkv, 256)[:L] = torch.from_numpy(k_codes)
    vc.view(-1, hkv, 256)[:L] = torch.from_numpy(v_codes)
    kc[n_pages] = 0x7F
    vc[n_pages] = 0x7F
    table = torch.arange(n_pages, dtype=torch.int32)[None]
    w = Workload(name="h", ctx=(L,), q_lens=(q_len,), num_q_heads=q.shape[1], num_kv_heads=hkv, num_segments=1,
                 seed=0)
    case = Case(torch.from_numpy(q).to(torch.bfloat16), kc, vc, table, torch.tensor([L], dtype=torch.int32),
                torch.tensor([0, q_len], dtype=torch.int32), torch.tensor([kd], dtype=torch.float32),
                torch.tensor([vd], dtype=torch.float32), scale, n_pages, w)
    return case.to(DEV)


def _code(value):
    table = oracle.e4m3fn_decode_table()
    return int(np.flatnonzero(table == value)[0])


@pytest.mark.parametrize("n", [4000, 16384])
def test_dominant_key_keeps_small_probabilities(n):
    # one key with score 7, the other n - 1 keys score 0; V = +1 on key 0, -1
    # elsewhere: exact (e^7 - (n - 1)) / (e^7 + (n - 1)), -0.5696 at 4000 keys
    # and -0.8745 at 16384 (the key count of the aiter PR #7375 review example)
    k = np.zeros((n, 1, 256), np.uint8)
    k[0, 0, 0] = _code(14.0)
    v = np.full((n, 1, 256), _code(-1.0), np.uint8)
    v[0] = _code(1.0)
    q = np.zeros((1, 16, 256), np.float32)
    q[0, :, 0] = 8.0
    case = _one_sequence(k, v, q, 1)
    exact = (math.exp(7.0) - (n - 1)) / (math.exp(7.0) + (n - 1))
    ref = oracle_for(case)
    assert abs(ref[0, 0, 0] - exact) < 1e-12
    for segments in (1, 4, 16):
        out = run(case, num_segments=segments)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        print(f"[dominant] S={segments} got {got[0, 0, 0]:.5f} exact {exact:.5f}", flush=True)
        assert np.max(np.abs(got - exact)) < 1e-2


def test_single_key_returns_v_exactly():
    rng = np.random.default_rng(7)
    finite = np.flatnonzero(~np.isnan(oracle.e4m3fn_decode_table()))
    k = rng.choice(finite, size=(1, 1, 256)).astype(np.uint8)
    v = rng.choice(finite, size=(1, 1, 256)).astype(np.uint8)
    q = rng.standard_normal((1, 16, 256)).astype(np.float32)
    case = _one_sequence(k, v, q, 1, kd=0.37, vd=0.25)
    out = run(case, num_segments=1)
    torch.cuda.synchronize()
    expect = torch.from_numpy(oracle.e4m3fn_decode_table()[v[0, 0]] * 0.25).to(torch.bfloat16)
    assert torch.equal(out[0].cpu().view(torch.int16), expect[None].expand(16, 256).view(torch.int16))


def test_identical_keys_give_prefix_means():
    rng = np.random.default_rng(8)
    table = oracle.e4m3fn_decode_table()
    small = np.flatnonzero(np.abs(table) < 4)
    L = 333
    k = np.repeat(rng.choice(small, size=(1, 1, 256)).astype(np.uint8), L, axis=0)
    v = rng.choice(small, size=(L, 1, 256)).astype(np.uint8)
    q = rng.standard_normal((4, 16, 256)).astype(np.float32)
    case = _one_sequence(k, v, q, 4)
    out = run(case, num_segments=3).float().cpu().numpy()
    vals = table[v[:, 0, :]]
    for i in range(4):
        mean = vals[: L - 4 + i + 1].mean(axis=0)
        assert np.max(np.abs(out[i] - mean[None])) < 4e-3


def test_zero_length_query_sequences():
    w = Workload(name="z", ctx=(100, 50, 80, 2000), q_lens=(4, 0, 2, 0), num_q_heads=16, num_kv_heads=1,
                 num_segments=4, seed=35)
    case = make_case(w, "cpu").to(DEV)
    out = run(case, num_segments=4)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), "zero q_len entries")


def test_strided_q_and_out():
    case = _case("multigroup")
    T, Hq, D = case.q.shape
    big_q = torch.zeros((T, Hq + 3, D + 64), dtype=torch.bfloat16, device=DEV)
    big_q[:, :Hq, :D] = case.q
    q_view = big_q[:, :Hq, :D]
    big_out = torch.zeros((T, Hq + 1, D + 32), dtype=torch.bfloat16, device=DEV)
    out_view = big_out[:, :Hq, :D]
    ref = run(case, num_segments=6)
    pfkv.verify_attn(q_view, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q,
                     case.k_descale, case.v_descale, case.softmax_scale, num_segments=6, out=out_view)
    torch.cuda.synchronize()
    assert torch.equal(out_view.contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.all(big_out[:, Hq:, :] == 0) and torch.all(big_out[:, :, D:] == 0)


def test_q_rows_spanning_just_under_4_gib():
    """A work-group addresses its Q rows (up to 4 query tokens x its query
    heads) with 32-bit byte offsets from a 64-bit base, so the call accepts
    strides whose rows span just under 4 GiB: at that largest stride the result
    is the contiguous call's, bit for bit; one stride step more is refused."""
    w = Workload(name="qspan", ctx=(2000, 700), q_lens=(4, 3), num_q_heads=16, num_kv_heads=1,
                 num_segments=4, seed=35)
    case = make_case(w, "cpu").to(DEV)
    T, Hq, D = case.q.shape
    head = D   # heads of a token contiguous
    st = (((1 << 32) - 1) // 2 - (Hq - 1) * head - D) // 3 // 8 * 8
    assert (3 * st + (Hq - 1) * head + D) * 2 < 1 << 32 <= (3 * (st + 8) + (Hq - 1) * head + D) * 2
    buf = torch.empty((T - 1) * (st + 8) + Hq * head, dtype=torch.bfloat16, device=DEV)
    try:
        q = buf.as_strided((T, Hq, D), (st, head, 1))
        q.copy_(case.q)
        ref = run(case, num_segments=4)
        got = pfkv.verify_attn(q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q,
                               case.k_descale, case.v_descale, case.softmax_scale, num_segments=4)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        too_far = buf.as_strided((T, Hq, D), (st + 8, head, 1))
        with pytest.raises(pfkv.PfkvError) as info:
            pfkv.verify_attn(too_far, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                             case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale, num_segments=4)
        assert "4 GiB" in str(info.value)
    finally:
        del buf
        torch.cuda.empty_cache()


def test_unsupported_group_is_refused():
    w = Workload(name="u", ctx=(64,), q_lens=(4,), num_q_heads=2, num_kv_heads=1, num_segments=1, seed=1)
    case = make_case(w, "cpu").to(DEV)
    with pytest.raises(pfkv.PfkvError) as info:
        run(case, num_segments=1)
    assert info.value.status == 2


def test_host_pointer_is_refused():
    case = _case("tiny")
    with pytest.raises(ValueError):
        pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables.cpu(), case.seq_lens,
                         case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale, num_segments=4)


def test_host_pointer_is_refused_by_the_library_after_a_good_call():
    """The C ABI's own pointer check (pfkv_verify_attn_fwd -> PFKV_DEVICE): a call
    that passes host memory as block_tables is refused without a launch, also
    right after a good call with the same other buffers (whose checks the
    library remembers)."""
    import ctypes
    case = _case("tiny")
    lib = pfkv.load_library()
    out = torch.zeros_like(case.q)
    ws = torch.empty(pfkv.workspace_bytes(4, case.q.shape[0], case.q.shape[1]), dtype=torch.uint8, device=DEV)
    a = pfkv.binding.build_args(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                                case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale, 4, out, ws)
    handle = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pfkv_verify_attn_fwd(ctypes.byref(a), handle) == 0
    torch.cuda.synchronize()
    good = out.clone()
    host_table = case.block_tables.cpu().numpy().copy()
    a.block_tables = host_table.ctypes.data
    out.zero_()
    assert lib.pfkv_verify_attn_fwd(ctypes.byref(a), handle) == 3
    assert "block_tables" in pfkv.binding.last_error()
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()
    a.block_tables = case.block_tables.data_ptr()
    assert lib.pfkv_verify_attn_fwd(ctypes.byref(a), handle) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), good.view(torch.int16))


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_stream_read_reads_every_byte(variant):
    """Each streaming-read variant folds every 32-bit word it reads into the sink
    by XOR; over a 64 MiB buffer of random words (a random block order for the
    ordered variants) that must equal the XOR of the whole buffer, computed on
    the host: a variant that skipped or repeated a block would not match."""
    nbytes = 64 << 20
    g = torch.Generator().manual_seed(77 + variant)
    host = torch.randint(0, 1 << 31, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    buf = host.to(DEV).view(torch.uint8)
    order = torch.randperm(nbytes // 4096, generator=g).to(torch.int32).to(DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    pfkv.stream_read(buf, variant, page_order=order if variant in (2, 3) else None, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == want
