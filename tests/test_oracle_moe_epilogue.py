"""Pins of the oracle's MoE epilogue ("Binade" package page, "How it works"
and "Limitations": the expert products of a MoE layer; gate and up meet in
an activation, and a token's chosen experts are summed with the router's
weights) and of the small-batch matvec's definition.

- silu_mul: closed forms (silu(0) = 0, silu(1) = e / (1 + e), silu(-1) =
  -1 / (1 + e), silu(g) = g for large g), the odd-part identity silu(x) -
  silu(-x) = x, a subnormal result, and the IEEE special cases the formula
  gives.
- combine: one-hot weights select a slot; small integers are exact in any
  order; a 2^24 cancellation fixes the slot order, and a product whose low
  bits only a fused multiply-add keeps fixes the fma.
- gemv_rows_replay: each row is the batch-1 replay of that row."""
import math

import numpy as np
import pytest

import oracle



def f32(v):
    return np.float32(v)


def test_silu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 2.0, 60.0, -0.0], np.float32)
    h = oracle.silu_mul(g, np.ones_like(g))
    e = math.e
    assert h[0] == 0.0
    assert h[1] == f32(e / (1.0 + e))
    assert h[2] == f32(-1.0 / (1.0 + e))
    assert h[3] == f32(2.0 * e * e / (1.0 + e * e))
    assert h[4] == f32(60.0)            # 1 + e^-60 == 1 in double
    assert h[5] == 0.0 and np.signbit(h[5])
    # the multiplier is applied after the activation, in the same rounding
    assert oracle.silu_mul(np.array([1.0], np.float32), np.array([3.0], np.float32))[0] == \
        f32(3.0 * e / (1.0 + e))


def test_silu_odd_part_and_subnormal():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4096) * 4).astype(np.float32)
    one = np.ones_like(x)
    d = oracle.silu_mul(x, one).astype(np.float64) - oracle.silu_mul(-x, one).astype(np.float64)
    # silu(x) - silu(-x) = x; each side is rounded once to fp32
    ulp = np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(d - x.astype(np.float64)) <= 2 * ulp)
    # silu(-100) = -100 e^-100 / (1 + e^-100): an fp32 subnormal
    h = oracle.silu_mul(np.array([-100.0], np.float32), np.array([1.0], np.float32))[0]
    assert h == f32(-100.0 * math.exp(-100.0)) and h != 0.0 and abs(h) < np.finfo(np.float32).tiny


def test_silu_special_values():
    g = np.array([np.inf, -np.inf, np.nan, -1000.0], np.float32)
    h = oracle.silu_mul(g, np.array([2.0, 1.0, 1.0, 5.0], np.float32))
    assert h[0] == np.inf
    assert np.isnan(h[1])               # -inf / inf, as the formula gives
    assert np.isnan(h[2])
    assert h[3] == 0.0 and np.signbit(h[3])


def test_combine_selects_and_integers():
    rng = np.random.default_rng(5)
    T, k, n = 3, 4, 37
    y = rng.standard_normal((T * k, n)).astype(np.float32)
    w = np.zeros(T * k, np.float32)
    for t in range(T):
        w[t * k + (t % k)] = 1.0
    out = oracle.moe_combine(y, w, k)
    for t in range(T):
        assert np.array_equal(out[t], y[t * k + (t % k)])
    yi = rng.integers(-1000, 1000, (T * k, n)).astype(np.float32)
    wi = rng.integers(-8, 9, T * k).astype(np.float32)
    want = (wi.reshape(T, k, 1).astype(np.int64) * yi.reshape(T, k, n).astype(np.int64)).sum(1)
    assert np.array_equal(oracle.moe_combine(yi, wi, k), want.astype(np.float32))


def test_combine_order_and_fma():
    one = np.ones(3, np.float32)
    # slot order: ((0 + 2^24) + 1) - 2^24 = 0 in fp32; the reverse order gives 1
    y = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], np.float32)
    assert oracle.moe_combine(y, one, 3)[0, 0] == 0.0
    assert oracle.moe_combine(y[::-1].copy(), one, 3)[0, 0] == 1.0
    # fused multiply-add: (1 + 2^-12)^2 - (1 + 2^-11) = 2^-24 only without
    # rounding the product first
    a = 1.0 + 2.0 ** -12
    y2 = np.array([[-(1.0 + 2.0 ** -11)], [a]], np.float32)
    w2 = np.array([1.0, a], np.float32)
    assert oracle.moe_combine(y2, w2, 2)[0, 0] == f32(2.0 ** -24)
    # the chain starts at +0.0: all -0 products give +0
    y3 = np.array([[-0.0], [-0.0]], np.float32)
    r = oracle.moe_combine(y3, np.ones(2, np.float32), 2)[0, 0]
    assert r == 0.0 and not np.signbit(r)


def test_gemv_rows_replay_is_the_rowwise_matvec():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((7, 96)) * 0.02).astype(np.float32)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y = oracle.gemv_rows_replay(wb, xb)
    assert y.shape == (3, 7)
    for b in range(3):
        assert np.array_equal(y[b], oracle.gemv_replay(wb, xb[b]))
