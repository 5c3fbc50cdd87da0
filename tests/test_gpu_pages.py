"""Cache pages of 32 and 64 tokens (the pages' kernel takes 16 only). A page of
16 R tokens in NHD order is R 16-token blocks back to back, so the kernel reads
block j of a sequence from cache page block_tables[j / R], part j mod R. Checked
against the oracle (which gathers by the cache's own page size) at the default
bars, and bit for bit against the same cache viewed as 16-token pages with the
block table expanded accordingly. Every call goes through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Workload, make_case

from gpu_util import assert_fp8_parity, assert_parity, oracle_for, run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _paged_case(page, group=16, seed=1):
    w = Workload(name=f"p{page}", ctx=(4100, 1000, 77, 33, 5), q_lens=(4, 3, 2, 4, 1), num_q_heads=group,
                 num_kv_heads=1, num_segments=None, seed=seed, page_size=page)
    return make_case(w, "cpu").to(DEV)


def _as_16_token_pages(case):
    """The same cache viewed as 16-token pages, with the block table expanded."""
    page = case.k_cache.shape[1]
    r = page // 16
    k16 = case.k_cache.reshape(case.k_cache.shape[0] * r, 16, *case.k_cache.shape[2:])
    v16 = case.v_cache.reshape(case.v_cache.shape[0] * r, 16, *case.v_cache.shape[2:])
    bt = case.block_tables.long()
    expanded = (bt[:, :, None] * r + torch.arange(r, device=bt.device)[None, None, :]).reshape(bt.shape[0], -1)
    return k16, v16, expanded.to(torch.int32).contiguous()


@pytest.mark.parametrize("page", [32, 64])
@pytest.mark.parametrize("group", [16, 8])
@pytest.mark.parametrize("segments", [None, 1, 5, 64])
def test_page_size_parity(page, group, segments):
    case = _paged_case(page, group, seed=page + group)
    out = run(case, num_segments=segments)
    torch.cuda.synchronize()
    assert_parity(out, oracle_for(case), f"page {page} G={group} S={segments}")


@pytest.mark.parametrize("page", [32, 64])
@pytest.mark.parametrize("segments", [None, 1, 7])
def test_page_size_equals_16_token_view_bitwise(page, segments):
    case = _paged_case(page, seed=3)
    k16, v16, bt16 = _as_16_token_pages(case)
    a, lse_a = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                                case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                                num_segments=segments, return_lse=True)
    b, lse_b = pfkv.verify_attn(case.q, k16, v16, bt16, case.seq_lens, case.cu_seqlens_q, case.k_descale,
                                case.v_descale, case.softmax_scale, num_segments=segments, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))


def test_page_64_lse_and_fp8_variant():
    case = _paged_case(64, seed=9)
    _, lse = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                              case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                              num_segments=6, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attend_lse(**case.to("cpu").host_arrays())
    assert np.abs(lse.cpu().numpy().astype(np.float64).T - ref).max() <= 1e-3
    out = run(case, num_segments=6, precision=pfkv.binding.PRECISION_FP8_P)
    torch.cuda.synchronize()
    assert_fp8_parity(out, case, 1, "page 64 fp8 P")
