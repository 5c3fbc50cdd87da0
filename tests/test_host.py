"""Host-side checks of the C ABI (no GPU needed): exports, validation, heuristics."""

import ctypes
import glob
import os
import subprocess
import re

import pytest

import paged_fp8_kv_split_amd as pfkv
from paged_fp8_kv_split_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pfkv.library_path()):
        from paged_fp8_kv_split_amd.build import build
        build()
    return pfkv.load_library()


def _declared_symbols():
    names = set()
    for header in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names |= set(re.findall(r"\b(pfkv_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(lib):
    names = _declared_symbols()
    assert {"pfkv_verify_attn_fwd", "pfkv_prefill_fwd", "pfkv_prefill_check_args"} <= set(names)
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header(tmp_path):
    """Every field of the ctypes mirror sits at the offset the C compiler gives it."""
    fields = [f for f, _ in binding.PfkvArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"pfkv.h\"\nint main(void) {\n"
                   f'  printf("%zu\\n", sizeof(pfkv_args));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(pfkv_args, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(binding.PfkvArgs)
    for f, off in zip(fields, got[1:]):
        assert getattr(binding.PfkvArgs, f).offset == off, f


def _valid_args(**over):
    a = binding.PfkvArgs()
    base = 0x100000
    for k, name in enumerate(["q", "k_cache", "v_cache", "block_tables", "seq_lens", "cu_seqlens_q",
                              "k_descale", "v_descale", "workspace", "out"]):
        setattr(a, name, base + 0x10000 * k)
    a.q_stride_token, a.q_stride_head = 16 * 256, 256
    a.out_stride_token, a.out_stride_head = 16 * 256, 256
    a.block_table_stride = 2200
    a.num_seqs, a.total_q, a.num_q_heads, a.num_kv_heads = 16, 64, 16, 1
    a.head_dim, a.page_size, a.num_pages, a.max_pages_per_seq = 256, 16, 70000, 2188
    a.num_segments = 16
    a.softmax_scale = 1.0 / 16
    a.workspace_size = pfkv.workspace_bytes(16, 64, 16)
    for k, v in over.items():
        setattr(a, k, v)
    return a


OK, INVALID, UNSUPPORTED = 0, 1, 2

CASES = [
    ("valid", {}, "gfx950:sramecc+:xnack-", OK),
    ("bare arch name", {}, "gfx950", OK),
    ("gqa8", dict(num_q_heads=8, q_stride_token=8 * 256, out_stride_token=8 * 256,
                  workspace_size=pfkv.workspace_bytes(16, 64, 8)), "gfx950", OK),
    ("two kv heads", dict(num_q_heads=32, num_kv_heads=2, workspace_size=pfkv.workspace_bytes(16, 64, 32)),
     "gfx950", OK),
    ("null q", dict(q=0), "gfx950", INVALID),
    ("null out", dict(out=0), "gfx950", INVALID),
    ("null descale", dict(v_descale=0), "gfx950", INVALID),
    ("zero seqs", dict(num_seqs=0), "gfx950", INVALID),
    ("too many queries", dict(total_q=65), "gfx950", INVALID),
    ("max_q_len 8", dict(max_q_len=8, total_q=128, workspace_size=pfkv.workspace_bytes(16, 128, 16)), "gfx950", OK),
    ("balanced", dict(balance_segments=1), "gfx950", OK),
    ("balanced, cap 1", dict(balance_segments=1, num_segments=1, workspace_size=pfkv.workspace_bytes(1, 64, 16)),
     "gfx950", INVALID),
    ("balance flag 2", dict(balance_segments=2), "gfx950", INVALID),
    ("balanced, cap 128", dict(balance_segments=1, num_segments=128, workspace_size=pfkv.workspace_bytes(128, 64, 16)),
     "gfx950", OK),
    ("balanced, cap 129", dict(balance_segments=1, num_segments=129, workspace_size=pfkv.workspace_bytes(129, 64, 16)),
     "gfx950", INVALID),
    ("uniform, 65 segments", dict(num_segments=65, workspace_size=pfkv.workspace_bytes(65, 64, 16)), "gfx950", INVALID),
    ("max_q_len 8 too many queries", dict(max_q_len=8, total_q=129), "gfx950", INVALID),
    ("max_q_len 9", dict(max_q_len=9), "gfx950", INVALID),
    ("max_q_len negative", dict(max_q_len=-1), "gfx950", INVALID),
    ("heads not divisible", dict(num_q_heads=15, num_kv_heads=2), "gfx950", INVALID),
    ("zero kv heads", dict(num_kv_heads=0), "gfx950", INVALID),
    ("segments 0", dict(num_segments=0), "gfx950", INVALID),
    ("segments 65", dict(num_segments=65), "gfx950", INVALID),
    ("workspace too small", dict(workspace_size=pfkv.workspace_bytes(16, 64, 16) - 1), "gfx950", INVALID),
    ("nan scale", dict(softmax_scale=float("nan")), "gfx950", INVALID),
    ("inf scale", dict(softmax_scale=float("inf")), "gfx950", INVALID),
    ("negative scale", dict(softmax_scale=-0.0625), "gfx950", INVALID),
    ("table stride", dict(block_table_stride=100), "gfx950", INVALID),
    ("q stride odd", dict(q_stride_head=255), "gfx950", INVALID),
    ("q misaligned", dict(q=0x100008), "gfx950", INVALID),
    ("q rows span 4 GiB", dict(q_stride_token=1 << 30), "gfx950", INVALID),
    ("q rows just under 4 GiB", dict(q_stride_token=((1 << 31) // 3 - 4096) // 8 * 8), "gfx950", 0),
    ("out stride", dict(out_stride_head=2), "gfx950", INVALID),
    ("workspace misaligned", dict(workspace=0x180004), "gfx950", INVALID),
    ("head_dim 128", dict(head_dim=128), "gfx950", OK),
    ("head_dim 64", dict(head_dim=64), "gfx950", UNSUPPORTED),
    ("head_dim 192", dict(head_dim=192), "gfx950", UNSUPPORTED),
    ("page 32", dict(page_size=32), "gfx950", OK),
    ("page 64", dict(page_size=64), "gfx950", OK),
    ("page 1", dict(page_size=1), "gfx950", OK),
    ("page 2", dict(page_size=2), "gfx950", UNSUPPORTED),
    ("page 8", dict(page_size=8), "gfx950", UNSUPPORTED),
    ("page 128", dict(page_size=128), "gfx950", UNSUPPORTED),
    ("page 64 table too wide", dict(page_size=64, max_pages_per_seq=(1 << 25), block_table_stride=(1 << 25)),
     "gfx950", INVALID),
    ("gqa 4", dict(num_q_heads=4, workspace_size=pfkv.workspace_bytes(16, 64, 4)), "gfx950", OK),
    ("gqa 32", dict(num_q_heads=32, workspace_size=pfkv.workspace_bytes(16, 64, 32)), "gfx950", OK),
    ("gqa 2", dict(num_q_heads=2, workspace_size=pfkv.workspace_bytes(16, 64, 2)), "gfx950", UNSUPPORTED),
    ("gqa 64", dict(num_q_heads=64, workspace_size=pfkv.workspace_bytes(16, 64, 64)), "gfx950", UNSUPPORTED),
    ("precision fp8 P", dict(precision=1), "gfx950", OK),
    ("precision fp8 Q/P", dict(precision=2), "gfx950", OK),
    ("precision 3", dict(precision=3), "gfx950", INVALID),
    ("lse given", dict(lse=0x1c0000), "gfx950", OK),
    ("sinks given", dict(sinks=0x1d0000), "gfx950", OK),
    ("sinks misaligned", dict(sinks=0x1d0001), "gfx950", INVALID),
    ("window one key", dict(window_keys=1), "gfx950", OK),
    ("window negative", dict(window_keys=-5), "gfx950", OK),
    ("softcap", dict(softcap=30.0), "gfx950", OK),
    ("softcap negative", dict(softcap=-1.0), "gfx950", INVALID),
    ("softcap nan", dict(softcap=float("nan")), "gfx950", INVALID),
    ("lse misaligned", dict(lse=0x1c0002), "gfx950", INVALID),
    ("precision -1", dict(precision=-1), "gfx950", INVALID),
    # in-launch merge sync words: 16 sequences x 1 merge group x 512 bytes
    ("merge sync", dict(merge_sync=0x1e0000, merge_sync_size=16 * 512), "gfx950", OK),
    ("merge sync too small", dict(merge_sync=0x1e0000, merge_sync_size=16 * 512 - 1), "gfx950", INVALID),
    ("merge sync misaligned", dict(merge_sync=0x1e0080, merge_sync_size=1 << 20), "gfx950", INVALID),
    ("merge sync, gqa 32", dict(num_q_heads=32, workspace_size=pfkv.workspace_bytes(16, 64, 32),
                                merge_sync=0x1e0000, merge_sync_size=16 * 2 * 512 - 1), "gfx950", INVALID),
    ("merge sync, 8 tokens", dict(max_q_len=8, total_q=128, workspace_size=pfkv.workspace_bytes(16, 128, 16),
                                  merge_sync=0x1e0000, merge_sync_size=16 * 2 * 512), "gfx950", OK),
    ("merge wait negative", dict(merge_wait_us=-1), "gfx950", OK),
    ("merge wait too long", dict(merge_wait_us=100001), "gfx950", INVALID),
    ("mi300", {}, "gfx942:sramecc+:xnack-", UNSUPPORTED),
    ("gfx9500 lookalike", {}, "gfx9500", UNSUPPORTED),
]


@pytest.mark.parametrize("name,over,arch,expect", CASES, ids=[c[0] for c in CASES])
def test_check_args_table(lib, name, over, arch, expect):
    a = _valid_args(**over)
    status = binding.check_args(a, arch)
    assert status == expect, (name, status, binding.last_error())
    if expect != OK:
        assert binding.last_error()


def test_check_args_rejects_bad_host_inputs(lib):
    assert lib.pfkv_check_args(None, b"gfx950", 256) == INVALID
    a = _valid_args()
    assert lib.pfkv_check_args(ctypes.byref(a), None, 256) == INVALID
    assert lib.pfkv_check_args(ctypes.byref(a), b"gfx950", 0) == INVALID


@pytest.mark.parametrize("cus,n,hkv,expect", [
    (256, 16, 1, 16), (256, 4, 1, 64), (256, 8, 1, 32), (256, 2, 2, 64), (256, 1, 1, 64),
    (256, 300, 1, 1), (256, 256, 1, 1), (256, 128, 1, 2), (304, 16, 1, 19), (0, 16, 1, 0), (256, 0, 1, 0),
])
def test_num_segments_heuristic(lib, cus, n, hkv, expect):
    assert pfkv.num_segments(cus, n, hkv) == expect


def test_workspace_bytes(lib):
    # fp16 o[256] + fp32 (m, l) per (segment, token, head)
    assert pfkv.workspace_bytes(16, 64, 16) == 16 * 64 * 16 * (256 * 2 + 8)
    assert pfkv.workspace_bytes(0, 64, 16) == 0
    assert pfkv.workspace_bytes(64, 8, 32) == 64 * 8 * 32 * (256 * 2 + 8)


def test_merge_sync_bytes(lib):
    # 128 words per merge group, at most num_q_heads / 4 groups per sequence
    assert pfkv.merge_sync_bytes(16, 16) == 16 * 4 * 512
    assert pfkv.merge_sync_bytes(4, 32) == 4 * 8 * 512
    assert pfkv.merge_sync_bytes(0, 16) == 0
    # the bound covers every split that check_args accepts
    for hq, hkv, qmax in ((16, 1, 4), (16, 1, 8), (32, 1, 8), (8, 1, 8), (4, 1, 8), (32, 8, 4)):
        need = pfkv.merge_sync_bytes(3, hq)
        a = _valid_args(num_seqs=3, total_q=3, num_q_heads=hq, num_kv_heads=hkv, max_q_len=qmax,
                        workspace_size=pfkv.workspace_bytes(16, 3, hq), merge_sync=0x1e0000, merge_sync_size=need)
        assert binding.check_args(a, "gfx950") == OK, (hq, hkv, qmax, binding.last_error())


def test_stream_read_validation(lib):
    assert lib.pfkv_stream_read(None, 4096, 0, None, 0, None, None) == INVALID
    assert lib.pfkv_stream_read(ctypes.c_void_p(0x1000), 4096, 4, None, 0, ctypes.c_void_p(0x2000), None) == INVALID
    assert lib.pfkv_stream_read(ctypes.c_void_p(0x1000), 4096, -1, None, 0, ctypes.c_void_p(0x2000), None) == INVALID
    for variant in (0, 1, 2, 3):
        # whole 4 KiB blocks only
        assert lib.pfkv_stream_read(ctypes.c_void_p(0x1000), 100, variant, None, 0, ctypes.c_void_p(0x2000), None) == INVALID
    for variant in (2, 3):
        # the ordered variants need a page order
        assert lib.pfkv_stream_read(ctypes.c_void_p(0x1000), 4096, variant, None, 0, ctypes.c_void_p(0x2000), None) == INVALID


def test_python_wrapper_needs_gpu_tensors():
    import torch
    q = torch.zeros(4, 16, 256, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        pfkv.verify_attn(q, None, None, None, None, None, None, None, 0.0625)


def test_ragged_workload_is_seeded_and_in_range():
    from paged_fp8_kv_split_amd.workloads import workload
    w = workload("ragged")
    assert w.num_seqs == 8 and all(1 <= q <= 4 for q in w.q_lens)
    assert all(6 <= c <= 105000 and c >= q for c, q in zip(w.ctx, w.q_lens))
    assert w == workload("ragged")


# ---------------------------------------------------------------- prefill
def test_prefill_struct_layout_matches_header(tmp_path):
    fields = [f for f, _ in binding.PfkvPrefillArgs._fields_]
    src = tmp_path / "layout_prefill.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"pfkv_prefill.h\"\nint main(void) {\n"
                   f'  printf("%zu\\n", sizeof(pfkv_prefill_args));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(pfkv_prefill_args, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout_prefill"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(binding.PfkvPrefillArgs)
    for f, off in zip(fields, got[1:]):
        assert getattr(binding.PfkvPrefillArgs, f).offset == off, f


def _valid_prefill(**over):
    a = binding.PfkvPrefillArgs()
    for k, name in enumerate(["q", "k", "v", "out", "cu_seqlens_q", "cu_seqlens_k", "q_descale", "k_descale",
                              "v_descale"]):
        setattr(a, name, 0x100000 + 0x10000 * k)
    a.q_stride_token, a.q_stride_head = 96 * 192, 192
    a.k_stride_token, a.k_stride_head = 96 * 192, 192
    a.v_stride_token, a.v_stride_head = 96 * 128, 128
    a.out_stride_token, a.out_stride_head = 96 * 128, 128
    a.num_seqs, a.total_q, a.total_k, a.num_q_heads, a.num_kv_heads = 1, 12288, 14336, 96, 96
    a.head_dim_qk, a.head_dim_v, a.max_seqlen_q = 192, 128, 12288
    a.softmax_scale, a.causal = 192 ** -0.5, 1
    for k, v in over.items():
        setattr(a, k, v)
    return a


PREFILL_CASES = [
    ("valid", {}, "gfx950", OK),
    ("non-causal", dict(causal=0), "gfx950", OK),
    ("with lse", dict(lse=0x1f0000), "gfx950", OK),
    ("gqa 8", dict(num_kv_heads=12), "gfx950", OK),
    ("no keys", dict(total_k=0), "gfx950", OK),
    ("gfx942", {}, "gfx942:sramecc+:xnack-", UNSUPPORTED),
    ("head dims 128/128", dict(head_dim_qk=128), "gfx950", UNSUPPORTED),
    ("v head dim 192", dict(head_dim_v=192), "gfx950", UNSUPPORTED),
    ("q NULL", dict(q=None), "gfx950", INVALID),
    ("v_descale NULL", dict(v_descale=None), "gfx950", INVALID),
    ("zero seqs", dict(num_seqs=0), "gfx950", INVALID),
    ("too many seqs", dict(num_seqs=70000), "gfx950", INVALID),
    ("zero q heads", dict(num_q_heads=0), "gfx950", INVALID),
    ("zero kv heads", dict(num_kv_heads=0), "gfx950", INVALID),
    ("heads not divisible", dict(num_kv_heads=7), "gfx950", INVALID),
    ("negative total_k", dict(total_k=-1), "gfx950", INVALID),
    ("zero max_seqlen_q", dict(max_seqlen_q=0), "gfx950", INVALID),
    ("tiles x heads at 2^31 - 1", dict(max_seqlen_q=(2**31 - 1) // 65535 * 256, num_q_heads=65535,
                                       num_kv_heads=65535), "gfx950", OK),
    ("tiles x heads above 2^31 - 1", dict(max_seqlen_q=((2**31 - 1) // 65535 + 1) * 256, num_q_heads=65535,
                                          num_kv_heads=65535), "gfx950", INVALID),
    ("nan scale", dict(softmax_scale=float("nan")), "gfx950", INVALID),
    ("zero scale", dict(softmax_scale=0.0), "gfx950", INVALID),
    ("q stride not 16", dict(q_stride_head=200), "gfx950", INVALID),
    ("k stride zero", dict(k_stride_token=0), "gfx950", INVALID),
    ("out stride odd", dict(out_stride_head=130), "gfx950", INVALID),
    ("q misaligned", dict(q=0x100008), "gfx950", INVALID),
    ("out misaligned", dict(out=0x130004), "gfx950", INVALID),
    ("lse misaligned", dict(lse=0x1f0002), "gfx950", INVALID),
]


@pytest.mark.parametrize("name,over,arch,expect", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_check_args(lib, name, over, arch, expect):
    assert binding.check_prefill_args(_valid_prefill(**over), arch) == expect, (name, binding.last_error())


def test_partials_row_major_table(lib):
    """Row-major partials exactly for the 16-bit mode at head dim 256 with pages
    of 16, 32 or 64 tokens and more than 16 segments (up to the 128-segment cap)."""
    P16, P8P, P8 = binding.PRECISION_16BIT, binding.PRECISION_FP8_P, binding.PRECISION_FP8
    assert pfkv.partials_row_major(P16, 256, 16, 17)
    for page in (16, 32, 64):
        for S in (17, 24, 32, 64, 65, 128):
            assert pfkv.partials_row_major(P16, 256, page, S), (page, S)
        for S in (0, 1, 2, 15, 16):
            assert not pfkv.partials_row_major(P16, 256, page, S), (page, S)
    for S in (17, 64, 128):
        assert not pfkv.partials_row_major(P8P, 256, 16, S)
        assert not pfkv.partials_row_major(P8, 256, 16, S)
        assert not pfkv.partials_row_major(P16, 128, 16, S)
        assert not pfkv.partials_row_major(P16, 256, 1, S)
    for bad in ((P16, 256, 8, 32), (P16, 256, 16, 129), (P16, 192, 16, 32), (7, 256, 16, 32), (-1, 256, 16, 32)):
        assert not pfkv.partials_row_major(*bad), bad
