"""Pins of the oracle's matrix-core step and prompt-GEMM replay (CPU only).

The step's arithmetic and the GEMM order are readings (the pages describe a
chain of matrix-core steps along K with a fixed split rule, "Binade" package
page, "NVIDIA GPUs"). What pins the oracle to them, independently of its own
code:
- hand-derived cases (tests/golden/mfma_step_cases.json,
  tests/golden/gemm_order_cases.json), each built so that a plausible mistake
  gives another value;
- exact integer arithmetic: with small integers nothing rounds, so the replay
  must equal an integer matrix product for every shape of slices and tails;
- the plain definition: within 1e-2 * sum |x w| of the fp64 product.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _value(s: str) -> float:
    s = s.strip()
    if s == "-0":
        return -0.0
    if s in ("inf", "-inf", "nan"):
        return float(s)
    if s.startswith("0x") or s.startswith("-0x"):
        return float.fromhex(s)
    if "*" in s:
        a, b = s.split("*")
        return _value(a) * _value(b)
    if "^" in s:
        neg = s.startswith("-")
        base, e = s.lstrip("-").split("^")
        v = float(base) ** int(e)
        return -v if neg else v
    return float(s)


def _bf16(v: float) -> int:
    u = int(np.array([v], np.float32).view(np.uint32)[0])
    assert u & 0xFFFF == 0, f"{v} is not a bf16 value"
    return u >> 16


def _f32_bits(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


STEP = _load("mfma_step_cases.json")["cases"]
ORDER = _load("gemm_order_cases.json")["cases"]


@pytest.mark.parametrize("case", STEP, ids=[c["name"] for c in STEP])
def test_mfma_step_hand_derived(case):
    a = np.zeros(32, np.uint16)
    b = np.full(32, _bf16(1.0), np.uint16)
    for t in case["terms"]:
        a[t[0]] = _bf16(_value(t[1]))
        if len(t) > 2:
            b[t[0]] = _bf16(_value(t[2]))
    got = oracle.mfma_step(a, b, _value(case["c"]))
    want = np.float32(_value(case["expect"]))
    if np.isnan(want):
        assert np.isnan(got), case["name"]
    else:
        assert _f32_bits(got) == _f32_bits(want), (case["name"], float(got).hex(), float(want).hex())


@pytest.mark.parametrize("case", ORDER, ids=[c["name"] for c in ORDER])
def test_gemm_order_hand_derived(case):
    K = case["K"]
    x = np.zeros((1, K), np.uint16)
    for col, v in case["x"]:
        x[0, col] = _bf16(_value(v))
    w = np.full((1, K), _bf16(1.0), np.uint16)
    got = oracle.gemm_replay(w, x)[0, 0]
    want = np.float32(_value(case["expect"]))
    assert _f32_bits(got) == _f32_bits(want), (case["name"], float(got).hex(), float(want).hex())
    # the chosen-entry form gives the same bits
    e = oracle.gemm_replay_entries(w, x, [0], [0])[0]
    assert _f32_bits(e) == _f32_bits(got)


def _bf16_of_ints(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("mnk", [(3, 5, 32), (4, 7, 96), (2, 3, 160), (5, 4, 1056),
                                 (3, 6, 2080), (2, 3, 3072), (2, 2, 9216)])
def test_gemm_replay_exact_on_small_integers(mnk):
    """Integers in [-8, 8]: every product and partial sum is an integer far
    below 2^24, so no step, slice or combine rounds; the replay must equal the
    integer product whatever the order."""
    M, N, K = mnk
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    xi = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (N, K))
    y = oracle.gemm_replay(_bf16_of_ints(wi), _bf16_of_ints(xi))
    assert np.array_equal(y.astype(np.int64), xi @ wi.T)


@pytest.mark.parametrize("mnk", [(4, 6, 128), (3, 5, 1056), (2, 4, 3840)])
def test_gemm_replay_within_fp64_bound(mnk):
    M, N, K = mnk
    rng = np.random.default_rng(K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    wb = ((w.view(np.uint32) + 0x7FFF + ((w.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    y = oracle.gemm_replay(wb, xb)
    ref = oracle.gemm_f64(wb, xb)
    scale = oracle.gemm_f64(wb & 0x7FFF, xb & 0x7FFF)
    assert np.all(np.abs(y.astype(np.float64) - ref) <= 1e-2 * scale)
    # not the same bits as a plain fp32 loop in column order: the order matters
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    wf = (wb.astype(np.uint32) << 16).view(np.float32)
    plain = np.zeros((M, N), np.float32)
    for k in range(K):
        plain = (plain + np.outer(xf[:, k], wf[:, k]).astype(np.float32)).astype(np.float32)
    assert not np.array_equal(plain.view(np.uint32), y.view(np.uint32))


def test_gemm_replay_entries_match_whole_replay():
    rng = np.random.default_rng(7)
    M, N, K = 5, 6, 1056
    xb = rng.integers(0, 1 << 16, (M, K)).astype(np.uint16) & 0xBFFF  # finite: no exponent 255
    wb = rng.integers(0, 1 << 16, (N, K)).astype(np.uint16) & 0xBFFF
    y = oracle.gemm_replay(wb, xb)
    mi = np.array([0, 4, 2, 3]); ni = np.array([5, 0, 3, 3])
    e = oracle.gemm_replay_entries(wb, xb, mi, ni)
    assert np.array_equal(e.view(np.uint32), y[mi, ni].view(np.uint32))


def test_gemm_replay_rejects_non_finite_inputs():
    x = np.zeros((1, 32), np.uint16)
    w = np.zeros((1, 32), np.uint16)
    w[0, 3] = 0x7F80  # +Inf
    with pytest.raises(oracle.OracleError):
        oracle.gemm_replay(w, x)
