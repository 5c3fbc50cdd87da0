"""Up to 8 query tokens per sequence (max_q_len = 8; the pages serve 4). A
work-group stacks at most 64 query rows, so with 16 query heads per work-group
a sequence's tokens run as two blocks of 4 (two work-groups). Same oracle and
bars as the default path, and the same bit-identity: a row computed in a call
with fewer tokens per sequence has the bits it has in the 8-token call. Every
call goes through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Workload, make_case

from gpu_util import assert_fp8_parity, assert_parity, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _case(group, hkv=1, seed=1, q_lens=(8, 5, 1, 7, 3), ctx=(3000, 800, 40, 16, 9)):
    w = Workload(name="q8", ctx=ctx, q_lens=q_lens, num_q_heads=group * hkv, num_kv_heads=hkv,
                 num_segments=None, seed=seed)
    return make_case(w, "cpu").to(DEV)


def _call(case, segments, q=None, cu=None, **opts):
    return pfkv.verify_attn(case.q if q is None else q, case.k_cache, case.v_cache, case.block_tables,
                            case.seq_lens, case.cu_seqlens_q if cu is None else cu, case.k_descale,
                            case.v_descale, case.softmax_scale, num_segments=segments, max_q_len=8, **opts)


@pytest.mark.parametrize("group,hkv", [(4, 2), (8, 1), (16, 1), (32, 1)])
@pytest.mark.parametrize("segments", [None, 1, 5])
def test_qlen8_parity(group, hkv, segments):
    case = _case(group, hkv, seed=40 + group)
    out = _call(case, segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"q_len<=8 G={group} S={segments}")


@pytest.mark.parametrize("group,segments", [(16, 6), (16, 1), (8, 6), (32, 3)])
def test_qlen8_short_rows_match_bitwise(group, segments):
    """Rows of calls with 1..7 tokens per sequence equal the 8-token call's rows bit for bit."""
    w = Workload(name="v8", ctx=(5000, 777, 40, 16), q_lens=(8, 8, 8, 8), num_q_heads=group, num_kv_heads=1,
                 num_segments=segments, seed=37)
    case = make_case(w, "cpu").to(DEV)
    verify = _call(case, segments)
    for q_len in (1, 3, 4, 5, 7):
        rows = [8 * b + 8 - q_len + i for b in range(w.num_seqs) for i in range(q_len)]
        q = case.q[torch.tensor(rows, device=DEV)].contiguous()
        cu = torch.arange(0, q_len * (w.num_seqs + 1), q_len, dtype=torch.int32, device=DEV)
        short = _call(case, segments, q=q, cu=cu)
        torch.cuda.synchronize()
        assert torch.equal(short.view(torch.int16), verify[torch.tensor(rows, device=DEV)].view(torch.int16)), q_len


def test_qlen8_lse_window_and_sinks():
    case = _case(16, seed=44)
    g = torch.Generator().manual_seed(3)
    sinks = torch.randn(16, generator=g).to(DEV)
    out, lse = _call(case, 4, return_lse=True, window_left=700, sinks=sinks)
    torch.cuda.synchronize()
    arrs = case.to("cpu").host_arrays()
    opts = dict(window_left=700, sinks=sinks.cpu().numpy())
    assert_parity(out, oracle.attend(**arrs, **opts), "q_len<=8 window sinks")
    ref = oracle.attend_lse(**arrs, **opts)
    assert np.abs(lse.cpu().numpy().astype(np.float64).T - ref).max() <= 1e-3


def test_qlen8_fp8_variants():
    case = _case(8, seed=45)
    for mode in (1, 2):
        out = _call(case, 4, precision=mode)
        torch.cuda.synchronize()
        assert_fp8_parity(out, case, mode, f"q_len<=8 fp8 mode {mode}")
