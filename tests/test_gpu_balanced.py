"""Balanced segments (balance_segments = 1): segments in proportion to each
sequence's pages, scheduled on the device from seq_lens. Checked against the
oracle on ragged batches, bitwise against the uniform split where the schedule
gives every sequence the same count, and for the bit identities the call
promises (rerun, graph replay, q_len-1 rows with the same seq_lens)."""

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd import binding
from paged_fp8_kv_split_amd.workloads import Workload, make_case, workload

from gpu_util import assert_fp8_parity, assert_parity, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _run(case, cap=128, **kw):
    return pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                            case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                            num_segments=cap, balance_segments=True, **kw)


@pytest.mark.parametrize("cap", [128, 100, 65, 64, 40, 17, 4, 2])
def test_balanced_ragged_parity(cap):
    case = make_case(workload("ragged"), "cpu").to(DEV)
    print(f"[balanced] ragged cap={cap} ctx={case.workload.ctx}", flush=True)
    out = _run(case, cap)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"balanced ragged cap={cap}")


def test_balanced_gqa8_and_empty_queries():
    w = Workload(name="b8", ctx=(30000, 7, 500, 3000, 16), q_lens=(4, 0, 3, 1, 4), num_q_heads=8, num_kv_heads=1,
                 num_segments=None, seed=61)
    case = make_case(w, "cpu").to(DEV)
    out = _run(case)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), "balanced gqa8")


def test_balanced_options_and_lse():
    w = Workload(name="bo", ctx=(20000, 300, 1000), q_lens=(4, 2, 3), num_q_heads=16, num_kv_heads=1,
                 num_segments=None, seed=62)
    case = make_case(w, "cpu").to(DEV)
    sinks = (torch.randn(16, generator=torch.Generator().manual_seed(3)) * 2.0).to(DEV)
    out, lse = _run(case, sinks=sinks, window_left=900, softcap=30.0, return_lse=True)
    torch.cuda.synchronize()
    arrs = case.to("cpu").host_arrays()
    opts = dict(window_left=900, softcap=30.0, sinks=sinks.cpu().numpy())
    assert_parity(out, oracle.attend(**arrs, **opts), "balanced options")
    ref_lse = oracle.attend_lse(**arrs, **opts)
    got = lse.cpu().numpy().astype(np.float64).T
    assert np.abs(got - ref_lse).max() <= 1e-3


def test_balanced_equals_uniform_on_equal_lengths():
    """16 equal sequences on 256 CUs, cap 16: every sequence gets
    min(16, (256 - 16) / 16 + 1) = 16 segments, the uniform split of S = 16, and
    the reduce merges them with one wave per row as for S = 16, so the bits agree.
    (With a cap above 16 the reduce splits each row over several waves and adds
    in another order: same values to rounding, other bits.)"""
    _, cus = binding.device_info(0)
    if cus != 256:
        pytest.skip("the 16-segment schedule assumes 256 CUs")
    w = Workload(name="be", ctx=(3000,) * 16, q_lens=(4,) * 16, num_q_heads=16, num_kv_heads=1, num_segments=16,
                 seed=63)
    case = make_case(w, "cpu").to(DEV)
    bal = _run(case, 16)
    uni = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                           case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale, num_segments=16)
    torch.cuda.synchronize()
    assert torch.equal(bal.view(torch.int16), uni.view(torch.int16))


def test_balanced_rerun_graph_and_short_rows_bitwise():
    case = make_case(workload("ragged"), "cpu").to(DEV)
    base = _run(case)
    again = _run(case)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), again.view(torch.int16))
    # graph replay, with eager calls between replays
    out = torch.empty_like(base)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _run(case, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _run(case, out=out)
    for k in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), base.view(torch.int16)), k
        _run(case)
    # the last query token of every sequence, alone (decode rows), same seq_lens
    cu = case.cu_seqlens_q.cpu().numpy()
    rows = [int(cu[b + 1]) - 1 for b in range(len(cu) - 1) if cu[b + 1] > cu[b]]
    q = case.q[torch.tensor(rows, device=DEV)].contiguous()
    ones = torch.tensor([0] + [1 if cu[b + 1] > cu[b] else 0 for b in range(len(cu) - 1)], dtype=torch.int32)
    cu1 = torch.cumsum(ones, 0).to(torch.int32).to(DEV)
    short = pfkv.verify_attn(q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, cu1,
                             case.k_descale, case.v_descale, case.softmax_scale, num_segments=128,
                             balance_segments=True)
    torch.cuda.synchronize()
    assert torch.equal(short.view(torch.int16), base[torch.tensor(rows, device=DEV)].view(torch.int16))


@pytest.mark.parametrize("hq,hkv,max_q,page,head_dim", [(32, 2, 4, 16, 256), (16, 1, 8, 16, 256),
                                                        (16, 1, 4, 1, 256), (8, 1, 4, 32, 128)])
def test_balanced_other_shapes(hq, hkv, max_q, page, head_dim):
    """Balanced segments with two work-groups per KV head (32 query heads),
    two query-token blocks per sequence (up to 8 tokens), one-token and 32-token
    pages, and head dim 128: the schedule's slots per work-group column change."""
    q_lens = (max_q, 1, 3, max_q)
    w = Workload(name="bs", ctx=(12000, 40, 700, 9), q_lens=q_lens, num_q_heads=hq, num_kv_heads=hkv,
                 num_segments=None, seed=64 + hq + max_q + page, page_size=page, head_dim=head_dim,
                 softmax_scale=1.0 / head_dim ** 0.5)
    case = make_case(w, "cpu").to(DEV)
    print(f"[balanced] hq={hq} hkv={hkv} max_q={max_q} page={page} d={head_dim}", flush=True)
    out = _run(case, max_q_len=max_q)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"balanced hq={hq} max_q={max_q} page={page} d={head_dim}")


@pytest.mark.parametrize("balanced", [False, True])
def test_stale_workspace_does_not_leak(balanced):
    """Every partial the reduce reads is written by the main kernel of the same
    call (empty segments write neutral records): a workspace full of 0xFF bytes
    (fp16 NaN) gives the same bits as a zeroed one."""
    case = make_case(workload("ragged"), "cpu").to(DEV)
    segs = 128 if balanced else 40
    need = pfkv.workspace_bytes(segs, case.q.shape[0], case.q.shape[1])
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        outs.append(pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                                     case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                                     num_segments=segs, workspace=ws, balance_segments=balanced,
                                     return_lse=True))
    torch.cuda.synchronize()
    (o0, l0), (o1, l1) = outs
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))


@pytest.mark.parametrize("mode", [1, 2])
def test_balanced_fp8_variants(mode):
    """The fp8 arithmetic under the balanced schedule (up to 128 segments, the
    eight-wave reduce), at the fp8 bar of gpu_util.assert_fp8_parity."""
    case = make_case(workload("ragged"), "cpu").to(DEV)
    out = _run(case, 128, precision=mode)
    torch.cuda.synchronize()
    assert_fp8_parity(out, case, mode, f"balanced ragged precision={mode}")
