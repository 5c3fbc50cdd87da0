"""The optional log-sum-exp output against the CPU oracle, through the C ABI.

lse[h][t] = ln sum_j exp(score_j) over the row's visible keys (aiter PR #7375,
Summary: the optional LSE in the varlen layout (heads, tokens)), computed from
the same rounded probabilities that normalise out (aiter PR #7375, Behavior and
intent). Tolerance, from the arithmetic of the 16-bit path: each probability
is rounded once to fp16 (relative error <= 2^-11), so the row sum, and hence
lse, moves by at most ln(1 + 2^-11) = 4.9e-4; fp32 scores of bf16 Q against
exactly converted K, and the hardware exp2/log2 (about 1 ulp each), add about
1e-5 at these score magnitudes. The bar is 1e-3. With e4m3 P (relative error
<= 2^-4) it is ln(1 + 2^-4) = 0.061, rounded up to 0.07.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Workload, make_case, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B = pfkv.binding
LSE_TOL = 1e-3
# e4m3 P under its block scales is within 2^-4 of the exact P wherever it is
# above 2^-13 of its block's largest (what lies below is negligible), so the
# row sum, and exp(lse), is within a factor 1 + 2^-4
LSE_TOL_FP8_P = math.log1p(2.0 ** -4) + 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _case(name, **over):
    return make_case(workload(name, **over), "cpu").to(DEV)


def _call(case, segments, precision=0):
    return pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                            case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                            num_segments=segments, precision=precision, return_lse=True)


def _oracle_lse(case):
    return oracle.attend_lse(**case.to("cpu").host_arrays())   # [T, Hq]


def _assert_lse(got, ref, tol, label):
    g = got.cpu().numpy().astype(np.float64).T                 # [Hq, T] -> [T, Hq]
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), label
    fin = np.isfinite(ref)
    err = np.abs(g[fin] - ref[fin]).max() if fin.any() else 0.0
    print(f"[lse] {label}: max|err|={err:.2e}", flush=True)
    assert err <= tol, (label, err)


@pytest.mark.parametrize("name,segments", [("tiny", 4), ("tiny", 1), ("multigroup", None), ("multigroup", 1),
                                           ("multigroup", 3), ("multigroup", 64), ("ragged", None)])
def test_lse_parity(name, segments):
    case = _case(name)
    out, lse = _call(case, segments)
    torch.cuda.synchronize()
    _assert_lse(lse, _oracle_lse(case), LSE_TOL, f"{name} S={segments}")


def test_lse_parity_fp8_p():
    case = _case("multigroup")
    _, lse = _call(case, 3, precision=B.PRECISION_FP8_P)
    torch.cuda.synchronize()
    _assert_lse(lse, _oracle_lse(case), LSE_TOL_FP8_P, "multigroup fp8 P")


def test_lse_gqa8_and_long_segments():
    w = Workload(name="lse8", ctx=(20000, 4100, 33), q_lens=(4, 3, 1), num_q_heads=8, num_kv_heads=1,
                 num_segments=None, seed=71)
    case = make_case(w, "cpu").to(DEV)
    for segments in (1, 7, 16):
        _, lse = _call(case, segments)
        torch.cuda.synchronize()
        _assert_lse(lse, _oracle_lse(case), LSE_TOL, f"gqa8 long S={segments}")


def test_out_is_unchanged_by_requesting_lse():
    case = _case("ragged")
    for segments in (None, 1):
        plain = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                                 case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                                 num_segments=segments)
        out, _ = _call(case, segments)
        torch.cuda.synchronize()
        assert torch.equal(plain.view(torch.int16), out.view(torch.int16)), segments


@pytest.mark.parametrize("group,segments", [(16, 8), (8, 8), (16, 1)])
def test_short_qlen_lse_matches_verify_bitwise(group, segments):
    """A decode or draft-extend row's lse has the same bits as in the verify call."""
    w = Workload(name="v", ctx=(5000, 777, 40, 16), q_lens=(4, 4, 4, 4), num_q_heads=group, num_kv_heads=1,
                 num_segments=segments, seed=34)
    case = make_case(w, "cpu").to(DEV)
    _, verify = _call(case, segments)
    for q_len in (1, 2, 3):
        rows = [4 * b + 4 - q_len + i for b in range(w.num_seqs) for i in range(q_len)]
        q = case.q[torch.tensor(rows, device=DEV)].contiguous()
        cu = torch.arange(0, q_len * (w.num_seqs + 1), q_len, dtype=torch.int32, device=DEV)
        _, short = pfkv.verify_attn(q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, cu,
                                    case.k_descale, case.v_descale, case.softmax_scale, num_segments=segments,
                                    return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(short.view(torch.int32), verify[:, torch.tensor(rows, device=DEV)].view(torch.int32)), q_len


def test_lse_graph_replay_bitwise():
    case = _case("tiny")
    S = 4
    out = torch.empty_like(case.q)
    lse = torch.empty((case.q.shape[1], case.q.shape[0]), dtype=torch.float32, device=DEV)
    ws = torch.empty(pfkv.workspace_bytes(S, case.q.shape[0], case.q.shape[1]), dtype=torch.uint8, device=DEV)
    args = (case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q,
            case.k_descale, case.v_descale, case.softmax_scale)
    _, eager = pfkv.verify_attn(*args, num_segments=S, return_lse=True)
    eager = eager.clone()
    stream = torch.cuda.Stream()
    pfkv.verify_attn(*args, num_segments=S, out=out, workspace=ws, lse=lse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pfkv.verify_attn(*args, num_segments=S, out=out, workspace=ws, lse=lse)
    for k in range(3):
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(lse.view(torch.int32), eager.view(torch.int32)), f"replay {k} differs"


def test_lse_production_shape_sampled_rows():
    """Full production shape in the bench's launch configuration; rows of three sequences
    checked against the oracle (the oracle computes them one sequence at a time)."""
    case = _case("prod")
    _, lse = _call(case, None)
    torch.cuda.synchronize()
    from gpu_util import rows_of, subset
    seqs = [0, 7, 15]
    sub = subset(case, seqs)
    ref = oracle.attend_lse(**sub.host_arrays())
    rows = torch.tensor(rows_of(case, seqs), device=DEV)
    _assert_lse(lse[:, rows], ref, LSE_TOL, "prod sampled")
