"""Left window, score soft-cap and sink logits against the CPU oracle, through
the C ABI. The pages name these only as features their gates leave out (SGLang
PR #37465, Modifications; aiter PR #7375, Changes); the library and the oracle
take their common reading (include/pfkv.h). Bars as for the default path:
max 0.15 sigma, mean 0.02 sigma of the output, and lse within 1e-3. The
soft-cap's tanh is computed from the hardware exp2 and reciprocal (about 1e-7
absolute each), far below those bars."""

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Workload, make_case

from gpu_util import assert_fp8_parity, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _case(group=16, seed=1, page=16):
    w = Workload(name="opt", ctx=(4100, 1000, 77, 33, 5), q_lens=(4, 3, 2, 4, 1), num_q_heads=group,
                 num_kv_heads=1, num_segments=None, seed=seed, page_size=page)
    return make_case(w, "cpu").to(DEV)


def _sinks(case, seed, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(case.q.shape[1], generator=g) * scale).to(DEV)


def _call(case, segments, **opts):
    return pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                            case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                            num_segments=segments, return_lse=True, **opts)


def _check(case, segments, label, **opts):
    out, lse = _call(case, segments, **opts)
    torch.cuda.synchronize()
    ref_opts = dict(opts)
    if "sinks" in ref_opts:
        ref_opts["sinks"] = ref_opts["sinks"].cpu().numpy()
    arrs = case.to("cpu").host_arrays()
    assert_parity(out, oracle.attend(**arrs, **ref_opts), label)
    ref_lse = oracle.attend_lse(**arrs, **ref_opts)
    got_lse = lse.cpu().numpy().astype(np.float64).T
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse)), label
    fin = np.isfinite(ref_lse)
    assert np.abs(got_lse[fin] - ref_lse[fin]).max() <= 1e-3, label


@pytest.mark.parametrize("window", [0, 5, 100, 1000, 5000])
@pytest.mark.parametrize("segments", [None, 1, 5])
def test_window(window, segments):
    _check(_case(seed=11), segments, f"window {window} S={segments}", window_left=window)


@pytest.mark.parametrize("softcap", [2.0, 30.0])
@pytest.mark.parametrize("segments", [None, 1])
def test_softcap(softcap, segments):
    _check(_case(seed=12), segments, f"softcap {softcap} S={segments}", softcap=softcap)


@pytest.mark.parametrize("segments", [None, 1, 7])
@pytest.mark.parametrize("scale", [2.0, 20.0])
def test_sinks(segments, scale):
    case = _case(seed=13)
    _check(case, segments, f"sinks x{scale} S={segments}", sinks=_sinks(case, 5, scale))


@pytest.mark.parametrize("segments", [None, 1])
def test_all_options_gqa8_page32(segments):
    case = _case(group=8, seed=14, page=32)
    _check(case, segments, f"all options G8 page 32 S={segments}", window_left=300, softcap=5.0,
           sinks=_sinks(case, 6))


@pytest.mark.parametrize("segments", [8, 1])
def test_window_short_qlen_rows_match_verify_bitwise(segments):
    """With a window, a decode or draft-extend row still has the verify call's bits."""
    w = Workload(name="v", ctx=(5000, 777, 40, 16), q_lens=(4, 4, 4, 4), num_q_heads=16, num_kv_heads=1,
                 num_segments=segments, seed=36)
    case = make_case(w, "cpu").to(DEV)
    opts = dict(window_left=301, softcap=7.0)
    verify, _ = _call(case, segments, **opts)
    for q_len in (1, 2, 3):
        rows = [4 * b + 4 - q_len + i for b in range(w.num_seqs) for i in range(q_len)]
        q = case.q[torch.tensor(rows, device=DEV)].contiguous()
        cu = torch.arange(0, q_len * (w.num_seqs + 1), q_len, dtype=torch.int32, device=DEV)
        short = pfkv.verify_attn(q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, cu,
                                 case.k_descale, case.v_descale, case.softmax_scale, num_segments=segments, **opts)
        torch.cuda.synchronize()
        assert torch.equal(short.view(torch.int16), verify[torch.tensor(rows, device=DEV)].view(torch.int16)), q_len


def test_window_fp8_variants():
    case = _case(seed=15)
    for mode in (1, 2):
        out = pfkv.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                               case.cu_seqlens_q, case.k_descale, case.v_descale, case.softmax_scale,
                               num_segments=4, precision=mode, window_left=64)
        torch.cuda.synchronize()
        assert_fp8_parity(out, case, mode, f"window fp8 mode {mode}", window_left=64)
