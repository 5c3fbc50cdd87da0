"""Pins for the fp64 model of the fp8 arithmetic (oracle/fp8_model.py), each
against something other than the model itself:

- e4m3 rounding against torch's own float32 -> float8_e4m3fn conversion (a
  library routine) on every grid point, every midpoint and random values;
- the power-of-two block scale against its defining properties (largest
  element in [128, 256), exactly representable blocks unchanged, 2^-4 relative
  error above the subnormal range);
- attention with rounded P against closed forms whose weights are exact powers
  of two, and the invariants that rounding cannot break (one visible key gives
  V, identical keys give the mean of V, page-pool permutation);
- the printed fp8 probability-underflow example on aiter PR #7375: unscaled
  e4m3 P gives the printed +1, block-scaled P stays at the exact value to within
  the rounding of its tail weight;
- planted mistakes (a per-row Q scale, a dropped P block scale) that some pin
  must catch.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_model
from paged_fp8_kv_split_amd.workloads import Workload, make_case, permute_pool

from test_oracle import _dominant_key_problem, _single_page_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TABLE = oracle.e4m3fn_decode_table()
CODE = {v: c for c, v in enumerate(TABLE) if not np.isnan(v) and c < 128}


def _torch_e4m3(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).double().numpy()


# ---------------------------------------------------------------- e4m3 rounding

def test_e4m3_round_matches_torch_on_grid_and_midpoints():
    grid = np.unique(np.abs(TABLE[~np.isnan(TABLE)]))          # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2                           # ties: to the even mantissa
    quarter = grid[:-1] + (grid[1:] - grid[:-1]) / 4
    x = np.concatenate([grid, mids, quarter, -grid, -mids, -quarter])
    assert np.array_equal(fp8_model.e4m3_round(x), _torch_e4m3(x))


def test_e4m3_round_matches_torch_on_random_values():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), 200000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32).astype(np.float64)
    x = np.clip(x, -448.0, 448.0)
    assert np.array_equal(fp8_model.e4m3_round(x), _torch_e4m3(x))


def test_e4m3_round_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8_model.e4m3_round(np.array([449.0]))


# ---------------------------------------------------------------- block scales

def test_block_scale_puts_the_largest_in_128_256():
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = rng.standard_normal(32) * 2.0 ** rng.uniform(-40, 40)
        e = fp8_model.block_exponent(x)
        top = np.max(np.abs(x)) * 2.0 ** -e
        assert 128.0 <= top < 256.0
    assert fp8_model.block_exponent(np.zeros(32)) == 0


def test_block_round_keeps_representable_blocks_and_bounds_the_error():
    rng = np.random.default_rng(4)
    normal = np.unique(TABLE[(TABLE >= 2.0 ** -6) & (TABLE < 256.0)])
    for k in (-30, -7, 0, 5, 20):
        vals = rng.choice(normal, size=(3, 64)) * rng.choice([-1.0, 1.0], size=(3, 64))
        vals[:, 0], vals[:, 32] = 240.0, -192.0        # each block's largest in [128, 256)
        x = vals * 2.0 ** k
        assert np.array_equal(fp8_model.block_round(x), x)
    x = rng.standard_normal((50, 96))
    got = fp8_model.block_round(x)
    for j in range(0, 96, 32):
        blk, r = x[:, j:j + 32], got[:, j:j + 32]
        top = np.max(np.abs(blk), axis=1, keepdims=True)
        normal_range = np.abs(blk) >= top * 2.0 ** -7      # scaled value >= 2^-6 (normal)
        rel = np.abs(r - blk) / np.abs(blk)
        assert np.all(rel[normal_range] <= 2.0 ** -4 + 1e-15)


# ---------------------------------------------------------------- attention with rounded P

def _power_of_two_weights_problem():
    """One query over 96 keys whose scores are -k ln 2 (so P = 2^-k): keys 0-31
    take k = j mod 13, keys 32-63 all k = 20, keys 64-95 k in {14, 15, 16, 18, 20}
    (every k an e4m3 value)."""
    n, d = 96, 16
    ks = np.concatenate([np.arange(32) % 13, np.full(32, 20), np.array([14, 15, 16, 18, 20])[np.arange(32) % 5]])
    k = np.zeros((n, 1, d), np.uint8)
    k[:, 0, 0] = [0x80 | CODE[float(x)] if x else 0 for x in ks]   # K dim 0 = -k (e4m3 exact)
    rng = np.random.default_rng(5)
    finite = np.flatnonzero(~np.isnan(TABLE))
    v = rng.choice(finite, size=(n, 1, d)).astype(np.uint8)
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    prob = _single_page_problem(k, v, q, 1, scale=float(np.float32(math.log(2.0))), page=16)
    return prob, ks, TABLE[v[:, 0, :]]


def test_block_scaled_p_is_exact_for_power_of_two_weights():
    prob, ks, vals = _power_of_two_weights_problem()
    w = 2.0 ** -ks.astype(np.float64)
    expect = (w @ vals) / w.sum()
    got = fp8_model.attend_fp8(**prob, quantize_q=False)
    assert np.allclose(got[0, 0], expect, rtol=1e-12, atol=1e-12)
    # planted mistake: no block scale. Then 2^-10 (half the smallest subnormal,
    # a tie to the even 0) and everything below it round to 0
    plain = fp8_model.attend_fp8(**prob, quantize_q=False, p_block_scale=False)
    w_plain = np.where(ks >= 10, 0.0, w)
    assert np.allclose(plain[0, 0], (w_plain @ vals) / w_plain.sum(), rtol=1e-12, atol=1e-12)
    assert not np.allclose(plain[0, 0], expect, rtol=1e-6, atol=1e-6)


def test_single_key_and_identical_keys():
    rng = np.random.default_rng(6)
    finite = np.flatnonzero(~np.isnan(TABLE))
    d = 64
    k = rng.choice(finite, size=(1, 1, d)).astype(np.uint8)
    v = rng.choice(finite, size=(1, 1, d)).astype(np.uint8)
    q = rng.standard_normal((1, 8, d))
    out = fp8_model.attend_fp8(**_single_page_problem(k, v, q, 1, kd=0.37, vd=1.75))
    assert np.array_equal(out[0], np.broadcast_to(TABLE[v[0, 0]] * float(np.float32(1.75)), (8, d)))
    L = 50
    k = np.repeat(rng.choice(finite, size=(1, 1, d)).astype(np.uint8), L, axis=0)
    v = rng.choice(finite, size=(L, 1, d)).astype(np.uint8)
    out = fp8_model.attend_fp8(**_single_page_problem(k, v, q[:, :1], 1, page=16))
    assert np.allclose(out[0, 0], TABLE[v[:, 0]].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_page_pool_permutation_invariance():
    w = Workload(name="p", ctx=(300, 77), q_lens=(4, 2), num_q_heads=4, num_kv_heads=2, num_segments=1,
                 seed=9, head_dim=64, page_size=16)
    case = make_case(w, "cpu")
    a = fp8_model.attend_fp8(**case.host_arrays())
    b = fp8_model.attend_fp8(**permute_pool(case, seed=11).host_arrays())
    assert np.array_equal(a, b)


def test_without_rounding_the_model_is_the_oracle():
    """With Q already on its block grid and every P block a single key
    (one-key rows), the model reduces to attend."""
    w = Workload(name="z", ctx=(1, 1), q_lens=(1, 1), num_q_heads=2, num_kv_heads=1, num_segments=1, seed=12,
                 head_dim=32, page_size=16)
    arrs = make_case(w, "cpu").host_arrays()
    assert np.allclose(fp8_model.attend_fp8(**arrs, quantize_q=False), oracle.attend(**arrs), rtol=0, atol=1e-15)


def test_q_blocks_are_32_dims():
    """Q whose first 32 dims are about 2^7 and the rest about 2^-8: each block is
    exactly representable under its own scale, so rounding Q changes nothing;
    one scale for the whole row (a planted mistake) would flush the small block."""
    d = 64
    rng = np.random.default_rng(13)
    normal = np.unique(TABLE[(TABLE >= 16.0) & (TABLE < 256.0)])
    q = np.empty((1, 2, d))
    q[..., :32] = rng.choice(normal, size=(1, 2, 32)) * rng.choice([-1.0, 1.0], size=(1, 2, 32))
    q[..., 32:] = rng.choice(normal, size=(1, 2, 32)) * 2.0 ** -15
    qb = torch.tensor(q, dtype=torch.float32).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(fp8_model.block_round(qb), qb)
    finite = np.flatnonzero(~np.isnan(TABLE) & (np.abs(TABLE) < 4))
    L = 40
    k = rng.choice(finite, size=(L, 1, d)).astype(np.uint8)
    v = rng.choice(finite, size=(L, 1, d)).astype(np.uint8)
    prob = _single_page_problem(k, v, qb, 1, scale=1.0, page=16)
    a = fp8_model.attend_fp8(**prob, quantize_q=True)
    b = fp8_model.attend_fp8(**prob, quantize_q=False)
    assert np.array_equal(a, b)
    s = 448.0 / np.abs(qb).max()
    row_scaled = _torch_e4m3(qb * s) / s
    assert not np.array_equal(row_scaled, qb)


# ---------------------------------------------------------------- the printed example

def _golden():
    fields = {}
    for line in open(os.path.join(GOLDEN, "fp8_p_underflow_example.txt")):
        if line.strip() and not line.startswith("#"):
            key, val = line.split()
            fields[key] = float(val)
    return fields


def test_printed_underflow_example_plain_and_block_scaled():
    f = _golden()
    n, d = int(f["num_keys"]), int(f["qk_head_dim"])
    prob = _dominant_key_problem(n, d, 1.0 / math.sqrt(d))
    plain = fp8_model.attend_fp8(**prob, p_block_scale=False)
    assert np.all(plain == f["fp8_p_output"])                     # the printed +1
    got = fp8_model.attend_fp8(**prob)
    # closed form with the tail weight t rounded under each block's scale:
    # block 0 holds the dominant key (P = 1, scale 2^-7), the other blocks only tail keys
    scale = float(np.float32(1.0 / math.sqrt(d)))
    t = math.exp(-f["q_dim0"] * f["k_key0_dim0"] * scale)
    e_tail = math.floor(math.log2(t)) - 7
    t0 = _torch_e4m3(t * 2.0 ** 7)[()] * 2.0 ** -7
    t1 = _torch_e4m3(t * 2.0 ** -e_tail)[()] * 2.0 ** e_tail
    tails = 31 * t0 + (n - 32) * t1
    expect = (1.0 - tails) / (1.0 + tails)
    assert np.allclose(got, expect, rtol=0, atol=1e-12)
    assert abs(expect - f["exact_output"]) < 0.02                  # near the exact -0.6699


def test_reference_offsets_change_only_the_roundings():
    """Without rounding (one key per row) an offset changes nothing; with it the
    results differ by no more than the rounding itself, and offset 0 is the default."""
    w = Workload(name="o", ctx=(700, 300), q_lens=(4, 2), num_q_heads=8, num_kv_heads=1, num_segments=1,
                 seed=21, head_dim=64, page_size=16)
    arrs = make_case(w, "cpu").host_arrays()
    exact = oracle.attend(**arrs)
    base = fp8_model.attend_fp8(**arrs)
    assert np.array_equal(base, fp8_model.attend_fp8(**arrs, p_offsets=np.zeros((6, 8))))
    rng = np.random.default_rng(0)
    other = fp8_model.attend_fp8(**arrs, p_offsets=rng.uniform(0, 1, (6, 8)))
    assert not np.array_equal(base, other)
    sigma = exact.std()
    for got in (base, other):
        assert np.abs(got - exact).mean() / sigma < 0.05
    one = Workload(name="o1", ctx=(1, 1), q_lens=(1, 1), num_q_heads=2, num_kv_heads=1, num_segments=1, seed=22,
                   head_dim=32, page_size=16)
    a1 = make_case(one, "cpu").host_arrays()
    assert np.array_equal(fp8_model.attend_fp8(**a1, p_offsets=np.full((2, 2), 0.7)), fp8_model.attend_fp8(**a1))
