"""Pins of the oracle's int8 quantization (CPU only).

The formula (CANN "low_latency_dispatch", Function / Formula, dynamic
quantization scenario) is pinned by hand-worked vectors, by an exact
rational evaluation in which each binary32 operation is rounded once
(tests/_exact.py), and by invariants that a wrong sign, a dropped smooth
scale, a wrong rounding mode or a reassociated product would break.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from combine_moe_get_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
from tests._exact import quant_row_exact, round_binary32

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf(vals):
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_hand_vectors():
    with open(os.path.join(GOLD, "quant_hand_vectors.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        x = _bf(case["x"])
        assert np.array_equal(bf16_bits_to_f32(x), np.asarray(case["x"], np.float32))
        q, scale = oracle.quant_token(x)
        assert q.tolist() == case["q"], case["note"]
        if case["dyn"] == 0:
            assert scale == 0.0
        else:
            # the sent scale is the binary32 rounding of 1/dyn
            assert scale == np.float32(float(round_binary32(Fraction(1) / Fraction(case["dyn"]))))


def test_sent_scale_is_reciprocal_of_dyn_not_amax_over_127():
    # find an amax where fl(1/fl(127/amax)) != fl(amax/127) and check the oracle sends the former
    found = 0
    for m in range(1, 400):
        amax = np.float32(1.0 + m / 512.0)
        x = _bf([float(amax), 0.5])
        if bf16_bits_to_f32(x)[0] != amax:
            continue
        dyn = round_binary32(Fraction(127) / Fraction(float(amax)))
        recip = float(round_binary32(Fraction(1) / dyn))
        direct = float(round_binary32(Fraction(float(amax)) / 127))
        if recip != direct:
            _, scale = oracle.quant_token(x)
            assert float(scale) == recip
            found += 1
    assert found > 0


@pytest.mark.parametrize("seed", range(25))
def test_exact_rational_evaluation(seed):
    r = np.random.default_rng(1000 + seed)
    H = int(r.integers(1, 24))
    xf = r.standard_normal(H).astype(np.float32) * np.float32(10.0 ** r.integers(-3, 3))
    if seed % 5 == 0:
        xf[r.integers(0, H)] = 0.0
    x = f32_to_bf16_bits(xf)
    s = r.uniform(0.5, 1.5, H).astype(np.float32) if seed % 2 else None
    q, scale = oracle.quant_token(x, s)
    qe, se = quant_row_exact([float(v) for v in bf16_bits_to_f32(x)],
                             None if s is None else [float(v) for v in s])
    assert q.tolist() == qe
    assert float(scale) == se


def test_tiny_amax_overflowing_dyn():
    # amax = 2^-126: 127/amax overflows binary32, so every nonzero element saturates and the
    # sent scale is 1/inf = 0 (the reading taken for this corner of the formula)
    tiny = np.float32(2.0 ** -126)
    x = _bf([tiny, -tiny, 0.0, tiny])
    q, scale = oracle.quant_token(x)
    assert q.tolist() == [127, -127, 0, 127]
    assert scale == 0.0
    qe, se = quant_row_exact([float(tiny), -float(tiny), 0.0, float(tiny)])
    assert q.tolist() == qe and se == 0.0


def _rows(seed, n, H):
    r = np.random.default_rng(seed)
    return f32_to_bf16_bits(r.standard_normal((n, H)).astype(np.float32))


def test_invariants_max_code_and_error_bound():
    X = _rows(5, 64, 1024)
    s = np.random.default_rng(6).uniform(0.5, 1.5, 1024).astype(np.float32)
    for row in X:
        q, scale = oracle.quant_token(row, s)
        xf = bf16_bits_to_f32(row).astype(np.float64) * s.astype(np.float64)
        assert np.abs(q).max() == 127
        # dequantized value is within half a step (plus binary32 rounding) of x*s
        err = np.abs(q.astype(np.float64) * float(scale) - xf)
        assert err.max() <= float(scale) * (0.5 + 1e-5)


def test_sign_symmetry():
    X = _rows(9, 32, 256)
    for row in X:
        q, scale = oracle.quant_token(row)
        qn, scale_n = oracle.quant_token(row ^ np.uint16(0x8000))
        assert np.array_equal(qn, -q) and scale_n == scale


@pytest.mark.parametrize("m", [-20, -3, 1, 7])
def test_power_of_two_scaling(m):
    # scaling x by 2^m leaves the codes unchanged and scales the sent scale by 2^m
    X = _rows(11, 16, 512)
    for row in X:
        q, scale = oracle.quant_token(row)
        xs = f32_to_bf16_bits(bf16_bits_to_f32(row) * np.float32(2.0 ** m))
        q2, scale2 = oracle.quant_token(xs)
        assert np.array_equal(q, q2)
        assert float(scale2) == float(scale) * 2.0 ** m


def test_smooth_scale_is_applied_per_channel():
    # a per-channel power-of-two scale equals pre-scaling the input exactly
    row = _rows(13, 1, 512)[0]
    r = np.random.default_rng(14)
    s = (2.0 ** r.integers(-3, 4, 512)).astype(np.float32)
    q, scale = oracle.quant_token(row, s)
    pre = f32_to_bf16_bits(bf16_bits_to_f32(row) * s)
    q2, scale2 = oracle.quant_token(pre)
    assert np.array_equal(q, q2) and scale == scale2


def test_static_quant_rounds_and_saturates():
    # quant_mode 1: CastToInt8(fp32(x) * scales), no dynamic scale
    x = _bf([0.5, 1.5, 2.5, -2.5, 300.0, -1000.0, 126.6, 0.0, 128.0, -128.0])
    q = oracle.quant_static(x)
    assert q.tolist() == [0, 2, 2, -2, 127, -127, 126, 0, 127, -127]  # 126.6 is 126.5 in bf16, a tie to 126
    s = np.full(10, 2.0, np.float32)
    q = oracle.quant_static(x, s)
    assert q.tolist() == [1, 3, 5, -5, 127, -127, 127, 0, 127, -127]


def test_dispatch_rows_equal_token_quant():
    # every routed copy of a token carries the same codes and the same scale
    sh = oracle.make_shape(8, 64, 3, 4, 2)
    r = np.random.default_rng(3)
    topk = np.argsort(r.random((8, 4)), axis=1)[:, :3].astype(np.int32)
    x = _rows(4, 8, 64)
    s = r.uniform(0.5, 1.5, 64).astype(np.float32)
    w = r.random((8, 3)).astype(np.float32)
    lay = oracle.layout(sh, topk)
    d = oracle.dispatch(sh, 2, x, lay, smooth=s, weights=w, topk_idx=topk)
    for t in range(8):
        q, scale = oracle.quant_token(x[t], s)
        for j in range(3):
            row = lay["dst_row"][t, j]
            assert np.array_equal(d["expand_x"][row], q)
            assert d["dynamic_scales"][row] == scale
            assert d["expand_weights"][row] == w[t, j]
    d0 = oracle.dispatch(sh, 0, x, lay)
    for t in range(8):
        for j in range(3):
            assert np.array_equal(d0["expand_x"][lay["dst_row"][t, j]], x[t])


def test_per_expert_smooth_scales():
    # [E, H] scales: each copy is quantized with its own expert's vector
    sh = oracle.make_shape(4, 32, 2, 4, 2)
    topk = np.array([[0, 3], [1, 2], [3, 0], [2, 1]], np.int32)
    x = _rows(21, 4, 32)
    s = np.random.default_rng(22).uniform(0.5, 1.5, (4, 32)).astype(np.float32)
    lay = oracle.layout(sh, topk)
    d = oracle.dispatch(sh, 2, x, lay, smooth=s, topk_idx=topk)
    for t in range(4):
        for j in range(2):
            q, scale = oracle.quant_token(x[t], s[topk[t, j]])
            row = lay["dst_row"][t, j]
            assert np.array_equal(d["expand_x"][row], q) and d["dynamic_scales"][row] == scale


def test_static_dispatch_hand_case_shared_and_per_expert_scales():
    # quant_mode 1 through the whole dispatch, against codes worked by hand (every product is
    # exact in binary32; rint ties to even, saturation at 127).  E = 4 experts over P = 2 ranks,
    # token 0 routed to experts 1 and 3, token 1 to experts 2 and 0, so the expert-major rows are
    # row 0 = (token 1, expert 0), row 1 = (token 0, expert 1), row 2 = (token 1, expert 2),
    # row 3 = (token 0, expert 3).
    sh = oracle.make_shape(2, 4, 2, 4, 2)
    topk = np.array([[1, 3], [2, 0]], np.int32)
    x = _bf([[0.5, 1.5, 2.5, -3.0], [10.0, -20.0, 0.25, 100.0]])
    lay = oracle.layout(sh, topk)
    np.testing.assert_array_equal(lay["dst_row"], [[1, 3], [2, 0]])
    # one [H] vector for every copy: token 0 -> 0.5, 3, 1.25, -12; token 1 -> 10, -40, 0.125, 400
    s = np.array([1.0, 2.0, 0.5, 4.0], np.float32)
    d = oracle.dispatch(sh, 1, x, lay, smooth=s, topk_idx=topk)
    np.testing.assert_array_equal(d["expand_x"], [[10, -40, 0, 127], [0, 3, 1, -12], [10, -40, 0, 127],
                                                  [0, 3, 1, -12]])
    # [E, H]: each copy takes its expert's row
    se = np.array([[1, 1, 1, 1], [2, 2, 2, 2], [0.5, 0.5, 0.5, 0.5], [-1, 1, 64, 0.25]], np.float32)
    d = oracle.dispatch(sh, 1, x, lay, smooth=se, topk_idx=topk)
    np.testing.assert_array_equal(d["expand_x"], [[10, -20, 0, 100],   # token 1 x expert 0's row
                                                  [1, 3, 5, -6],       # token 0 x expert 1's row
                                                  [5, -10, 0, 50],     # token 1 x expert 2's row
                                                  [0, 2, 127, -1]])    # token 0 x expert 3's row
    # no scales: CastToInt8 of x itself
    d = oracle.dispatch(sh, 1, x, lay, topk_idx=topk)
    np.testing.assert_array_equal(d["expand_x"], [[10, -20, 0, 100], [0, 2, 2, -3], [10, -20, 0, 100],
                                                  [0, 2, 2, -3]])
