"""Debug mode: a checking kernel rejects inputs that break the device-side
contract before any attention kernel runs (the pages' kernel rejects what it
does not serve: aiter PR #5190, Supported). Each broken input below is caught by
the check and never reaches the main kernel; valid inputs give the same bits as
without the check. Every call goes through the C ABI."""

import pytest
import torch

import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import make_case, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _debug_on():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()
    prev = pfkv.set_debug(True)
    yield
    pfkv.set_debug(prev)


def _case():
    return make_case(workload("ragged"), "cpu").to(DEV)


def _call(case, **over):
    args = dict(q=case.q, k_cache=case.k_cache, v_cache=case.v_cache, block_tables=case.block_tables,
                seq_lens=case.seq_lens, cu_seqlens_q=case.cu_seqlens_q, k_descale=case.k_descale,
                v_descale=case.v_descale, softmax_scale=case.softmax_scale)
    args.update(over)
    return pfkv.verify_attn(**args, num_segments=5)


def test_valid_input_passes_with_the_same_bits():
    case = _case()
    checked = _call(case)
    pfkv.set_debug(False)
    plain = _call(case)
    torch.cuda.synchronize()
    assert torch.equal(checked.view(torch.int16), plain.view(torch.int16))


def _expect_invalid(case, text, **over):
    with pytest.raises(pfkv.PfkvError) as info:
        _call(case, **over)
    assert info.value.status == 1
    assert text in str(info.value), str(info.value)


def test_block_table_entry_out_of_range():
    case = _case()
    bt = case.block_tables.clone()
    bt[2, 0] = case.k_cache.shape[0] + 5
    _expect_invalid(case, "sequence 2", block_tables=bt)


def test_negative_block_table_entry():
    case = _case()
    bt = case.block_tables.clone()
    bt[1, 1] = -1                       # sequence 1 has 254 keys: it uses entries 0..15
    _expect_invalid(case, "block-table entry", block_tables=bt)


def test_unused_table_entries_are_not_checked():
    """Entries past a sequence's last page are never read, by the check or the kernels."""
    case = _case()
    bt = case.block_tables.clone()
    bt[0, 1] = -1                       # sequence 0 has 10 keys: only entry 0 is used
    checked = _call(case, block_tables=bt)
    pfkv.set_debug(False)
    plain = _call(case)
    torch.cuda.synchronize()
    assert torch.equal(checked.view(torch.int16), plain.view(torch.int16))


def test_seq_len_below_query_tokens():
    case = _case()
    sl = case.seq_lens.clone()
    q_len = int(case.cu_seqlens_q[4] - case.cu_seqlens_q[3])
    sl[3] = q_len - 1
    _expect_invalid(case, "sequence 3", seq_lens=sl)


def test_seq_len_beyond_the_table():
    case = _case()
    sl = case.seq_lens.clone()
    sl[1] = case.block_tables.shape[1] * 16 + 1
    _expect_invalid(case, "page_size * max_pages_per_seq", seq_lens=sl)


def test_too_many_query_tokens():
    case = _case()
    cu = case.cu_seqlens_q.clone()
    # move the boundary between sequences 0 and 1 so that sequence 1 has 6 tokens
    n1 = int(cu[2] - cu[1])
    cu[1] = cu[2] - 6 if n1 < 6 else cu[1]
    if int(cu[1]) < int(cu[0]):
        pytest.skip("ragged draw leaves no room for 6 tokens")
    _expect_invalid(case, "max_q_len", cu_seqlens_q=cu)


def test_cu_seqlens_not_ending_at_total():
    case = _case()
    cu = case.cu_seqlens_q.clone()
    cu[-1] = cu[-1] - 1
    _expect_invalid(case, "cu_seqlens_q", cu_seqlens_q=cu)
