"""The in-launch merge (merge_sync) against the two launches, through the C ABI.

With merge_sync, the main kernel's work-groups merge their group's partials
themselves with the segment reduce's per-row code, so the output and the lse
must equal those of the two launches bit for bit: on every waves-per-row choice
(16, 32 and 64 segments), every head split (GQA 4 / 8 / 16 / 32, 8-token
drafts), with the options, with no waiting at all (every share handed to the
last arrival), over repeated calls and graph replays on one sync buffer, which
each call must leave ready for the next. Calls the merge does not serve run
the two launches and leave the buffer untouched."""

import numpy as np
import pytest
import torch

import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd import binding
from paged_fp8_kv_split_amd.workloads import Workload, make_case, workload

from gpu_util import assert_parity, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WORDS = 128   # sync words per merge group


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _cus():
    return binding.device_info(0)[1]


def _args(case):
    return (case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.cu_seqlens_q,
            case.k_descale, case.v_descale, case.softmax_scale)


def _case(name, ctx, q_lens, hq, hkv, seed):
    return make_case(Workload(name=name, ctx=tuple(ctx), q_lens=tuple(q_lens), num_q_heads=hq, num_kv_heads=hkv,
                              num_segments=None, seed=seed), "cpu").to(DEV)


def _split(hq, hkv, max_q_len):
    """(merge groups per sequence, query blocks per head group, tokens per block)"""
    g = hq // hkv
    kv_split = 2 if g == 32 else 1
    q_per_wg = min(64 // (16 if g == 32 else g), 8)
    q_split = -(-max_q_len // q_per_wg)
    return hkv * kv_split * q_split, q_split, q_per_wg


def _groups_per_seq(hq, hkv, max_q_len):
    return _split(hq, hkv, max_q_len)[0]


def _active(case, max_q_len):
    """Per merge group: does it hold query tokens (a query block past a
    sequence's tokens has none, and its work-groups return at once)?"""
    hq, hkv = case.q.shape[1], case.k_cache.shape[2]
    per_seq, q_split, q_per_wg = _split(hq, hkv, max_q_len or 4)
    cu = case.cu_seqlens_q.cpu().numpy()
    act = []
    for b in range(case.seq_lens.numel()):
        n = int(cu[b + 1] - cu[b])
        act += [n > (z % q_split) * q_per_wg for z in range(per_seq)]
    return np.array(act)


def _state(sync, groups):
    """Per merge group: arrivals, generation, mask of handed-over shares."""
    w = sync.view(torch.int32).cpu().numpy()[:groups * WORDS].reshape(groups, WORDS)
    return w[:, 0] & 0xff, w[:, 0] >> 8, w[:, 64:66]


def _compare(case, segments, sync, calls_before=0, max_q_len=0, **opts):
    """Two launches vs in-launch merge (default wait, then no wait); returns the merge output."""
    hq, hkv = case.q.shape[1], case.k_cache.shape[2]
    groups = case.seq_lens.numel() * _groups_per_seq(hq, hkv, max_q_len or 4)
    assert groups * segments <= _cus(), "the merge serves grids of at most one work-group per CU"
    print(f"[merge] {case.workload} S={segments} T={case.q.shape[0]} Hq={hq} Hkv={hkv} opts={sorted(opts)}",
          flush=True)
    ref, ref_lse = pfkv.verify_attn(*_args(case), num_segments=segments, return_lse=True, max_q_len=max_q_len,
                                    **opts)
    for wait in (0, -1):
        out = torch.full_like(case.q, float("nan"))
        lse = torch.full((hq, case.q.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
        pfkv.verify_attn(*_args(case), num_segments=segments, out=out, lse=lse, max_q_len=max_q_len,
                         merge_sync=sync, merge_wait_us=wait, **opts)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (case.workload, wait)
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), (case.workload, wait)
    arrivals, gen, handed = _state(sync, groups)
    assert not arrivals.any() and not handed.any(), "a call left the sync words dirty"
    active = _active(case, max_q_len)
    assert (gen == np.where(active, calls_before + 2, 0)).all(), (gen, active)
    return out


SHAPES = [
    # name, ctx, q_lens, Hq, Hkv, segments, max_q_len
    ("s16", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, 16, 0),
    ("s32", [5000, 33, 1777, 4096, 900, 64, 2500, 3001], [4, 1, 2, 4, 3, 4, 1, 2], 16, 1, 32, 0),
    ("s64", [9000, 7001, 35, 4000], [4, 2, 1, 3], 16, 1, 64, 0),
    ("decode", [2500 + 97 * i for i in range(16)], [1] * 16, 16, 1, 16, 0),
    ("gqa8", [2000, 333, 4500, 129] * 4, [4, 1, 3, 2] * 4, 16, 2, 8, 0),
    ("gqa4", [2000, 333, 4500, 129, 77, 6000, 1024, 2048], [4, 1, 3, 2, 4, 4, 1, 2], 16, 4, 8, 0),
    ("gqa32", [2000, 333, 4500, 129, 77, 6000, 1024, 2048], [4, 1, 3, 2, 4, 4, 1, 2], 32, 1, 16, 0),
    ("q8", [3000, 40, 1500, 777, 2222, 16, 4096, 999], [8, 5, 1, 4, 7, 8, 2, 6], 16, 1, 16, 8),
]


@pytest.mark.parametrize("name,ctx,q_lens,hq,hkv,segments,max_q_len", SHAPES, ids=[s[0] for s in SHAPES])
def test_matches_two_launches(name, ctx, q_lens, hq, hkv, segments, max_q_len):
    case = _case(name, ctx, q_lens, hq, hkv, seed=len(name) + 11)
    sync = pfkv.merge_sync_buffer(len(ctx), hq, DEV)
    _compare(case, segments, sync, max_q_len=max_q_len)


@pytest.mark.parametrize("segments", [2, 3, 5, 24, 40, 63])
def test_uneven_shares(segments):
    """Segment counts that do not divide the 64 rows of a group: several
    passes per share (2, 3, 5: 32, 22 and 13 rows), uneven parts (24, 40) and
    126 (row, segment) vectors gathered at once (63, the most a share holds)."""
    case = _case(f"uneven{segments}", [5000, 3100, 977, 4096], [4, 4, 4, 4], 16, 1, seed=80 + segments)
    sync = pfkv.merge_sync_buffer(4, 16, DEV)
    _compare(case, segments, sync)


def test_options():
    case = _case("opts", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, seed=21)
    sync = pfkv.merge_sync_buffer(16, 16, DEV)
    sinks = torch.linspace(-2.0, 3.0, 16, dtype=torch.float32, device=DEV)
    _compare(case, 16, sync, sinks=sinks, window_left=700, softcap=25.0)
    _compare(case, 16, sync, calls_before=2, window_left=0)


def test_production_shape_and_oracle():
    # 16 sequences of 35000 keys, 4 query tokens, GQA 16, 16 segments: the shape the merge is timed on
    case = make_case(workload("prod"), "cpu").to(DEV)
    sync = pfkv.merge_sync_buffer(16, 16, DEV)
    out = _compare(case, 16, sync)
    occ = make_case(workload("occupancy"), "cpu").to(DEV)
    sync_occ = pfkv.merge_sync_buffer(4, 16, DEV)
    out_occ = _compare(occ, 64, sync_occ)
    assert_parity(out_occ, oracle_for(occ), "occupancy, in-launch merge")
    del out


def test_repeated_calls_on_one_buffer():
    """Calls of different shapes share one buffer; each leaves it ready for the next."""
    a = _case("rep_a", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, seed=31)
    b = _case("rep_b", [9000, 7001, 35, 4000], [4, 2, 1, 3], 16, 1, seed=32)
    sync = pfkv.merge_sync_buffer(16, 16, DEV)
    ref_a = pfkv.verify_attn(*_args(a), num_segments=16)
    ref_b = pfkv.verify_attn(*_args(b), num_segments=64)
    for k in range(4):
        print(f"[merge] repeated call {k}", flush=True)
        got_a = pfkv.verify_attn(*_args(a), num_segments=16, merge_sync=sync)
        got_b = pfkv.verify_attn(*_args(b), num_segments=64, merge_sync=sync)
        torch.cuda.synchronize()
        assert torch.equal(got_a.view(torch.int16), ref_a.view(torch.int16)), k
        assert torch.equal(got_b.view(torch.int16), ref_b.view(torch.int16)), k
    arrivals, gen, handed = _state(sync, 16)
    assert not arrivals.any() and not handed.any()
    assert (gen[:4] == 8).all() and (gen[4:] == 4).all(), gen


def test_graph_replays_bitwise():
    """Calls captured into a HIP graph, replayed with eager merge calls on the
    same buffer in between; every replay equals the eager result."""
    case = _case("graph", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, seed=41)
    sync = pfkv.merge_sync_buffer(16, 16, DEV)
    ref = pfkv.verify_attn(*_args(case), num_segments=16)
    out = torch.zeros_like(case.q)
    ws = torch.empty(binding.workspace_bytes(16, case.q.shape[0], 16), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        pfkv.verify_attn(*_args(case), num_segments=16, out=out, workspace=ws, stream=stream, merge_sync=sync)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(2):
            pfkv.verify_attn(*_args(case), num_segments=16, out=out, workspace=ws, stream=stream, merge_sync=sync)
    for k in range(4):
        print(f"[merge] graph replay {k}", flush=True)
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), k
        other = pfkv.verify_attn(*_args(case), num_segments=16, merge_sync=sync)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16)), k
    arrivals, gen, handed = _state(sync, 16)
    assert not arrivals.any() and not handed.any()
    assert (gen == 1 + 4 * 3).all(), gen


def test_allocation_free_entry_point():
    case = _case("noalloc", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, seed=51)
    sync = pfkv.merge_sync_buffer(16, 16, DEV)
    ref, ref_lse = pfkv.verify_attn(*_args(case), num_segments=16, return_lse=True)
    out = torch.zeros_like(case.q)
    lse = torch.zeros((16, case.q.shape[0]), dtype=torch.float32, device=DEV)
    binding.verify_attn_noalloc(*_args(case), 16, out, lse=lse, merge_sync=sync)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    assert (_state(sync, 16)[1] == 1).all()


def test_calls_it_does_not_serve_leave_the_buffer():
    """Larger grids, the fp8 modes, balanced segments, one-token pages, head
    dim 128 and a single segment run the two launches; the buffer stays zero."""
    big = _case("big", [600 + 13 * i for i in range(32)], [4, 1, 2, 3] * 8, 16, 1, seed=61)
    small = _case("small", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, seed=62)
    sync = pfkv.merge_sync_buffer(32, 16, DEV)
    runs = [(big, dict(num_segments=16)),
            (small, dict(num_segments=16, precision=binding.PRECISION_FP8_P)),
            (small, dict(num_segments=16, precision=binding.PRECISION_FP8)),
            (small, dict(num_segments=64, balance_segments=True)),
            (small, dict(num_segments=1))]
    for case, opts in runs:
        print(f"[merge] not served: {case.workload} {opts}", flush=True)
        ref = pfkv.verify_attn(*_args(case), **opts)
        got = pfkv.verify_attn(*_args(case), merge_sync=sync, **opts)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), opts
    for name, page, hd in (("page1", 1, 256), ("hd128", 16, 128)):
        w = Workload(name=name, ctx=(3000, 1200, 517, 2049), q_lens=(4, 3, 1, 2), num_q_heads=16, num_kv_heads=1,
                     num_segments=None, seed=63, page_size=page, head_dim=hd)
        case = make_case(w, "cpu").to(DEV)
        print(f"[merge] not served: {name}", flush=True)
        ref = pfkv.verify_attn(*_args(case), num_segments=16)
        got = pfkv.verify_attn(*_args(case), num_segments=16, merge_sync=sync)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name
    assert not sync.any()


@pytest.mark.parametrize("wait_us", [0, 5])
def test_correct_while_another_stream_holds_the_cus(wait_us):
    """Merge calls on one stream while full-device calls run on another: the
    merge's work-groups may then not all be resident at once, so waits can end
    by the time limit (5 us makes that likely) and shares go to the last
    arrival. Every result must still equal the two launches' bits."""
    case = _case("contend", [3000, 1200, 517, 2049] * 4, [4, 3, 1, 2] * 4, 16, 1, seed=71)
    busy = make_case(workload("prod"), "cpu").to(DEV)
    sync = pfkv.merge_sync_buffer(16, 16, DEV)
    ref = pfkv.verify_attn(*_args(case), num_segments=16)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [torch.zeros_like(case.q) for _ in range(6)]
    ws = torch.empty(binding.workspace_bytes(16, case.q.shape[0], 16), dtype=torch.uint8, device=DEV)
    busy_out = torch.empty_like(busy.q)
    busy_ws = torch.empty(binding.workspace_bytes(16, busy.q.shape[0], 16), dtype=torch.uint8, device=DEV)
    print(f"[merge] contention, wait_us={wait_us}", flush=True)
    with torch.cuda.stream(sb):
        for _ in range(8):
            pfkv.verify_attn(*_args(busy), num_segments=16, out=busy_out, workspace=busy_ws, stream=sb)
    with torch.cuda.stream(sa):
        for o in outs:
            pfkv.verify_attn(*_args(case), num_segments=16, out=o, workspace=ws, stream=sa, merge_sync=sync,
                             merge_wait_us=wait_us)
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), k
    arrivals, gen, handed = _state(sync, 16)
    assert not arrivals.any() and not handed.any()
    assert (gen == len(outs)).all(), gen
