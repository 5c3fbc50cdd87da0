"""The allocation-free entry point (pfkv_verify_attn_fwd_noalloc) against the
workspace entry point (pfkv_verify_attn_fwd), through the C ABI.

Both run the same kernels on the same inputs, so the outputs and the lse must be
equal bit for bit. Two calls in a row, the second on a smaller problem, check
that the library's partials array keeps no state a call depends on; a request
beyond the array's size must fail with PFKV_INVALID and launch nothing."""

import pytest
import torch

import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd import binding
from paged_fp8_kv_split_amd.workloads import Workload, make_case, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIMIT = 16 << 20   # PFKV_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _args(case):
    return (case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q,
            case.k_descale, case.v_descale, case.softmax_scale)


def _both(case, segments, **opts):
    print(f"[no_alloc] {case.workload} segments={segments} T={case.q.shape[0]} opts={sorted(opts)}", flush=True)
    ref_out, ref_lse = pfkv.verify_attn(*_args(case), num_segments=segments, return_lse=True, **opts)
    out = torch.full_like(case.q, float("nan"))
    lse = torch.full((case.q.shape[1], case.q.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    binding.verify_attn_noalloc(*_args(case), segments, out, lse=lse, **opts)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), case.workload
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), case.workload


def test_two_calls_second_smaller():
    # the production shape: 16 sequences of 35000 keys, 4 query tokens, GQA 16, 16 segments
    big = make_case(workload("prod"), "cpu").to(DEV)
    assert binding.workspace_bytes(16, big.q.shape[0], big.q.shape[1]) <= LIMIT
    _both(big, 16)
    small = make_case(Workload(name="small", ctx=(4100, 77, 33, 5), q_lens=(4, 2, 1, 3), num_q_heads=16,
                               num_kv_heads=1, num_segments=None, seed=3), "cpu").to(DEV)
    _both(small, 5)


def test_options_and_fp8_precision():
    case = make_case(Workload(name="opts", ctx=(2000, 600, 17), q_lens=(4, 1, 3), num_q_heads=8,
                              num_kv_heads=1, num_segments=None, seed=5), "cpu").to(DEV)
    sinks = torch.linspace(-1.0, 1.0, case.q.shape[1], dtype=torch.float32, device=DEV)
    _both(case, 7, sinks=sinks, window_left=900, softcap=30.0)
    _both(case, 4, precision=binding.PRECISION_FP8)
    _both(case, 1)   # one segment: the main kernel writes out directly


def test_ragged_balanced():
    case = make_case(workload("ragged"), "cpu").to(DEV)
    _both(case, 64, balance_segments=True)
    _both(case, 40)


def test_graph_capture_replays_bitwise():
    """The use the entry point exists for: a call captured into a HIP graph (no
    allocation inside the capture), replayed with eager work in between."""
    case = make_case(workload("tiny"), "cpu").to(DEV)
    ref = pfkv.verify_attn(*_args(case), num_segments=4)
    out = torch.zeros_like(case.q)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        binding.verify_attn_noalloc(*_args(case), 4, out, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        binding.verify_attn_noalloc(*_args(case), 4, out, stream=stream)
    for k in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), k
        other = pfkv.verify_attn(*_args(case), num_segments=4)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))


def test_beyond_limit_is_rejected():
    case = make_case(Workload(name="tiny", ctx=(64,), q_lens=(4,), num_q_heads=16, num_kv_heads=1,
                              num_segments=None, seed=9), "cpu").to(DEV)
    # segments x T x Hq x 520 bytes just above the limit
    segments = LIMIT // (case.q.shape[0] * case.q.shape[1] * 520) + 1
    out = torch.zeros_like(case.q)
    with pytest.raises(binding.PfkvError) as e:
        binding.verify_attn_noalloc(*_args(case), segments, out)
    assert e.value.status == 1 and "allocation-free" in str(e.value)
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()
