"""Cache pools larger than 4 GiB, with the pages a call reads beyond the first
4 GiB of the pool: the byte offset of a page then needs more than 32 bits.

Each case takes a seeded problem, copies its whole pool into a larger device
pool at page index `base` (so that page `base` starts past 4 GiB) and adds
`base` to every block-table entry. The rest of the large pool is left
unwritten: a call reads only the pages its block tables name. The result must
be bit for bit that of the original pool, and within the bars of the oracle.
Every call goes through the C ABI.
"""

import pytest
import torch

import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd.workloads import Case, Workload, make_case

from gpu_util import assert_fp8_parity, assert_parity, oracle_for, run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pfkv.load_library()


def _far(case: Case) -> Case:
    """The same problem with its pool moved past 4 GiB of a larger pool."""
    pages, page, hkv, d = case.k_cache.shape
    page_bytes = page * hkv * d
    base = FOUR_GIB // page_bytes + 3
    assert base * page_bytes > FOUR_GIB
    big_k = torch.empty((base + pages, page, hkv, d), dtype=torch.uint8, device=DEV)
    big_v = torch.empty_like(big_k)
    big_k[base:] = case.k_cache
    big_v[base:] = case.v_cache
    print(f"[far] page {page} Hkv {hkv} D {d}: pages at {base * page_bytes / FOUR_GIB:.4f} x 4 GiB, "
          f"pool {2 * big_k.numel() / 2**30:.1f} GiB", flush=True)
    return Case(case.q, big_k, big_v, case.block_tables + base, case.seq_lens, case.cu_seqlens_q,
                case.k_descale, case.v_descale, case.softmax_scale, case.poison_page + base, case.workload)


# name, page size, query heads, KV heads, head dim, segments
SHAPES = [
    ("page16", 16, 16, 1, 256, 8),
    ("page16_rowmajor", 16, 16, 1, 256, 24),
    ("page64", 64, 16, 1, 256, 8),
    ("page1", 1, 16, 1, 256, 8),
    ("hd128", 16, 16, 1, 128, 8),
    ("two_kv_heads", 16, 16, 2, 256, 5),
]


@pytest.mark.parametrize("name,page,hq,hkv,d,segments", SHAPES, ids=[s[0] for s in SHAPES])
def test_pages_past_4_gib(name, page, hq, hkv, d, segments):
    w = Workload(name=name, ctx=(3000, 517, 40), q_lens=(4, 2, 1), num_q_heads=hq, num_kv_heads=hkv,
                 num_segments=segments, seed=61, page_size=page, head_dim=d)
    near = make_case(w, "cpu").to(DEV)
    far = _far(near)
    try:
        a = run(near, num_segments=segments)
        b = run(far, num_segments=segments)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        assert_parity(b, oracle_for(near), f"far pages {name}")
    finally:
        del far
        torch.cuda.empty_cache()


@pytest.mark.parametrize("precision", [pfkv.binding.PRECISION_FP8_P, pfkv.binding.PRECISION_FP8],
                         ids=["fp8_p", "fp8_qp"])
def test_pages_past_4_gib_fp8(precision):
    w = Workload(name="far_fp8", ctx=(3000, 517, 40), q_lens=(4, 2, 1), num_q_heads=16, num_kv_heads=1,
                 num_segments=8, seed=62)
    near = make_case(w, "cpu").to(DEV)
    far = _far(near)
    try:
        a = run(near, num_segments=8, precision=precision)
        b = run(far, num_segments=8, precision=precision)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert_fp8_parity(b, near, precision, f"far pages precision {precision}")
    finally:
        del far
        torch.cuda.empty_cache()
