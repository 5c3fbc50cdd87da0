"""head_dim 128, which the pages' gate rejects (aiter PR #5190, Supported: head_dim
256 only; SGLang PR #37465, Modifications: other shapes fall back). The same
kernel at D = 128: 2 KiB blocks, two 1 KiB transfers per wave per step, 32 output
dims per P.V wave. Checked against the oracle (generic over the head dim) at the
default bars, across groups, segment counts, page sizes, the options, the lse
output and the fp8 variants; plus the bit-exact invariants (graph replay, q_len-1
rows, page permutation) and sampled rows at 16 x 35000. Every call goes
through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Case, Workload, make_case, permute_pool, workload

from gpu_util import assert_fp8_parity, assert_parity, oracle_for, rows_of, run, subset

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B = pfkv.binding
SCALE = 1.0 / math.sqrt(128.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _case(group=16, seed=1, ctx=(4100, 1000, 77, 33, 5), q_lens=(4, 3, 2, 4, 1), page=16, hkv=1, segments=None):
    w = Workload(name="hd128", ctx=ctx, q_lens=q_lens, num_q_heads=group * hkv, num_kv_heads=hkv,
                 num_segments=segments, seed=seed, page_size=page, head_dim=128, softmax_scale=SCALE)
    return make_case(w, "cpu").to(DEV)


def _lse_call(case, segments, **kw):
    return pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                            case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                            num_segments=segments, return_lse=True, **kw)


def _assert_lse(got, ref, tol, label):
    g = got.cpu().numpy().astype(np.float64).T
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), label
    fin = np.isfinite(ref)
    err = np.abs(g[fin] - ref[fin]).max()
    print(f"[lse] {label}: max|err|={err:.2e}", flush=True)
    assert err <= tol, (label, err)


@pytest.mark.parametrize("group", [16, 8])
@pytest.mark.parametrize("segments", [None, 1, 5, 64])
def test_hd128_parity(group, segments):
    case = _case(group, seed=300 + group)
    out = run(case, num_segments=segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"hd128 G={group} S={segments}")


@pytest.mark.parametrize("group", [4, 32])
def test_hd128_other_groups(group):
    case = _case(group, seed=400 + group)
    out = run(case, num_segments=None)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"hd128 G={group}")


def test_hd128_several_kv_heads_and_long_segments():
    case = _case(8, seed=17, ctx=(20000, 4100, 33), q_lens=(4, 3, 1), hkv=2)
    arrs = case.to("cpu").host_arrays()
    ref, ref_lse = oracle.attend(**arrs), oracle.attend_lse(**arrs)
    for segments in (1, 7, 16):
        out, lse = _lse_call(case, segments)
        torch.cuda.synchronize()
        assert_parity(out, ref, f"hd128 Hkv=2 S={segments}")
        _assert_lse(lse, ref_lse, 1e-3, f"hd128 Hkv=2 S={segments}")


@pytest.mark.parametrize("page", [1, 32, 64])
def test_hd128_page_sizes(page):
    case = _case(16, seed=500 + page, page=page)
    out = run(case, num_segments=6)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"hd128 page {page}")


def test_hd128_options_lse():
    case = _case(16, seed=19)
    arrs = case.to("cpu").host_arrays()
    g = torch.Generator().manual_seed(19)
    sinks = (torch.randn(case.q.shape[1], generator=g) * 2.0).to(DEV)
    opts = dict(window_left=300, softcap=20.0)
    for segments in (1, 6):
        out, lse = _lse_call(case, segments, sinks=sinks, **opts)
        torch.cuda.synchronize()
        ref = oracle.attend(**arrs, sinks=sinks.cpu().numpy(), **opts)
        assert_parity(out, ref, f"hd128 options S={segments}")
        _assert_lse(lse, oracle.attend_lse(**arrs, sinks=sinks.cpu().numpy(), **opts), 1e-3,
                    f"hd128 options S={segments}")


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("segments", [None, 1])
def test_hd128_fp8_variants(mode, segments):
    case = _case(16, seed=21, ctx=(4100, 1000, 777, 300), q_lens=(4, 3, 2, 4))
    out = run(case, num_segments=segments, precision=mode)
    torch.cuda.synchronize()
    assert_fp8_parity(out, case, mode, f"hd128 precision {mode} S={segments}")


def test_hd128_eight_query_tokens():
    case = _case(16, seed=23, ctx=(3000, 517, 9), q_lens=(8, 5, 8))
    out = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                           case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                           num_segments=None, max_q_len=8)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), "hd128 q_len 8")


@pytest.mark.parametrize("segments", [8, 1])
def test_hd128_short_qlen_rows_match_verify_bitwise(segments):
    w = Workload(name="v", ctx=(5000, 777, 40, 16), q_lens=(4, 4, 4, 4), num_q_heads=16, num_kv_heads=1,
                 num_segments=segments, seed=34, head_dim=128, softmax_scale=SCALE)
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


def test_hd128_graph_replay_and_permutation_bitwise():
    case = _case(16, seed=25)
    S = 5
    eager = run(case, num_segments=S).clone()
    out = torch.empty_like(case.q)
    ws = torch.empty(pfkv.workspace_bytes(S, case.q.shape[0], case.q.shape[1]), dtype=torch.uint8, device=DEV)
    run(case, num_segments=S, out=out, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        run(case, num_segments=S, out=out, workspace=ws)
    for k in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {k} differs"
    shuffled = run(permute_pool(case, seed=9), num_segments=S)
    torch.cuda.synchronize()
    assert torch.equal(shuffled.view(torch.int16), eager.view(torch.int16))


def test_hd128_single_key_returns_v_exactly():
    rng = np.random.default_rng(27)
    table = oracle.e4m3fn_decode_table()
    finite = np.flatnonzero(~np.isnan(table))
    kc = torch.zeros((2, 16, 1, 128), dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    v = rng.choice(finite, size=128).astype(np.uint8)
    kc[0, 0, 0] = torch.from_numpy(rng.choice(finite, size=128).astype(np.uint8))
    vc[0, 0, 0] = torch.from_numpy(v)
    kc[1] = 0x7F
    vc[1] = 0x7F
    q = torch.from_numpy(rng.standard_normal((1, 16, 128)).astype(np.float32)).to(torch.bfloat16)
    w = Workload(name="h", ctx=(1,), q_lens=(1,), num_q_heads=16, num_kv_heads=1, num_segments=1, seed=0,
                 head_dim=128)
    case = Case(q, kc, vc, torch.zeros((1, 1), dtype=torch.int32), torch.tensor([1], dtype=torch.int32),
                torch.tensor([0, 1], dtype=torch.int32), torch.tensor([0.37], dtype=torch.float32),
                torch.tensor([0.25], dtype=torch.float32), SCALE, 1, w).to(DEV)
    for segments in (1, 3):
        out = run(case, num_segments=segments)
        torch.cuda.synchronize()
        expect = torch.from_numpy(table[v] * 0.25).to(torch.bfloat16)
        assert torch.equal(out[0].cpu().view(torch.int16), expect[None].expand(16, 128).view(torch.int16))


def test_hd128_production_shape_sampled():
    """16 sequences x 35000 keys, GQA 16, head_dim 128, in the benchmark's launch
    configuration; three sequences checked against the oracle."""
    w = workload("prod_hd128")
    case = make_case(w, DEV)
    out, lse = _lse_call(case, w.num_segments)
    torch.cuda.synchronize()
    seqs = [0, 7, 15]
    sub = subset(case, seqs)
    arrs = sub.host_arrays()
    rows = torch.tensor(rows_of(case, seqs), device=DEV)
    assert_parity(out[rows], oracle.attend(**arrs), "prod hd128 sampled")
    _assert_lse(lse[:, rows], oracle.attend_lse(**arrs), 1e-3, "prod hd128 sampled")
