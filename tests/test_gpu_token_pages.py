"""One-token cache pages (page_size 1: one block-table entry per token, which
the pages' gate rejects, SGLang PR #37465 Modifications; aiter PR #5190
Supported). The kernel still works in 16-token blocks, gathering each key row
through its own table entry. Checked against the oracle, which gathers token by
token, at the default bars, and bit for bit against a 16-token-page cache viewed
as one-token pages with the table expanded per token (same blocks, same
arithmetic). Every call goes through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Workload, make_case, workload

from gpu_util import assert_fp8_parity, assert_parity, oracle_for, run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B = pfkv.binding


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _token_case(group=16, seed=1, ctx=(4100, 1000, 77, 33, 5), q_lens=(4, 3, 2, 4, 1)):
    w = Workload(name="p1", ctx=ctx, q_lens=q_lens, num_q_heads=group, num_kv_heads=1,
                 num_segments=None, seed=seed, page_size=1)
    return make_case(w, "cpu").to(DEV)


def _as_token_pages(k_cache, v_cache, block_tables):
    """A paged cache viewed as one-token pages, with the table expanded per token."""
    page = k_cache.shape[1]
    k1 = k_cache.reshape(k_cache.shape[0] * page, 1, *k_cache.shape[2:])
    v1 = v_cache.reshape(v_cache.shape[0] * page, 1, *v_cache.shape[2:])
    bt = block_tables.long()
    expanded = (bt[:, :, None] * page + torch.arange(page, device=bt.device)[None, None, :]).reshape(bt.shape[0], -1)
    return k1, v1, expanded.to(torch.int32).contiguous()


def _call(case, k, v, bt, segments, **kw):
    return pfkv.verify_attn(case.q, k, v, bt, case.seq_lens, case.cu_seqlens_q, case.k_descale, case.v_descale,
                            case.softmax_scale, num_segments=segments, return_lse=True, **kw)


@pytest.mark.parametrize("group", [16, 8])
@pytest.mark.parametrize("segments", [None, 1, 5, 64])
def test_token_pages_parity(group, segments):
    case = _token_case(group, seed=100 + group)
    out = run(case, num_segments=segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"page 1 G={group} S={segments}")


@pytest.mark.parametrize("group", [4, 32])
def test_token_pages_other_groups(group):
    case = _token_case(group, seed=200 + group)
    out = run(case, num_segments=None)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"page 1 G={group}")


def test_token_pages_long_single_segment_lse():
    """One segment over 20000 keys: the table windows are refilled every four
    steps, over a thousand times."""
    case = _token_case(16, seed=7, ctx=(20000, 3001), q_lens=(4, 2))
    out, lse = _call(case, case.k_cache, case.v_cache, case.block_tables, 1)
    torch.cuda.synchronize()
    arrs = case.to("cpu").host_arrays()
    assert_parity(out, oracle.attend(**arrs), "page 1 long S=1")
    ref = oracle.attend_lse(**arrs)
    assert np.abs(lse.cpu().numpy().astype(np.float64).T - ref).max() <= 1e-3


@pytest.mark.parametrize("segments", [None, 1, 7])
def test_token_view_equals_16_token_pages_bitwise(segments):
    w = Workload(name="v", ctx=(4100, 1000, 77, 33, 5), q_lens=(4, 3, 2, 4, 1), num_q_heads=16, num_kv_heads=1,
                 num_segments=None, seed=5)
    case = make_case(w, "cpu").to(DEV)
    a, lse_a = _call(case, case.k_cache, case.v_cache, case.block_tables, segments)
    b, lse_b = _call(case, *_as_token_pages(case.k_cache, case.v_cache, case.block_tables), segments)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))


def test_token_view_equals_16_token_pages_production_shape():
    """16 sequences x 35000 keys, GQA 16, the benchmark's segment count: the
    one-token view gives the same bits as the 16-token pages."""
    case = make_case(workload("prod"), "cuda")
    a, lse_a = _call(case, case.k_cache, case.v_cache, case.block_tables, None)
    b, lse_b = _call(case, *_as_token_pages(case.k_cache, case.v_cache, case.block_tables), None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))


def test_token_pages_options_and_fp8():
    case = _token_case(16, seed=11)
    arrs = case.to("cpu").host_arrays()
    g = torch.Generator().manual_seed(11)
    sinks = (torch.randn(case.q.shape[1], generator=g) * 2.0).to(DEV)
    out, _ = _call(case, case.k_cache, case.v_cache, case.block_tables, 6, window_left=300, softcap=20.0,
                   sinks=sinks)
    torch.cuda.synchronize()
    ref = oracle.attend(**arrs, window_left=300, softcap=20.0, sinks=sinks.cpu().numpy())
    assert_parity(out, ref, "page 1 window/softcap/sinks")
    out8 = run(case, num_segments=6, precision=B.PRECISION_FP8_P)
    torch.cuda.synchronize()
    assert_fp8_parity(out8, case, 1, "page 1 fp8 P")


def test_token_pages_eight_query_tokens():
    case = _token_case(16, seed=13, ctx=(3000, 517, 9), q_lens=(8, 5, 8))
    out = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                           case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                           num_segments=None, max_q_len=8)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), "page 1 q_len 8")
