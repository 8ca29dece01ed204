"""The prompt GEMM against the oracle's replay of its documented order, bit for
bit, through the C ABI (binade_r4_gemm and its bf16-weight twin).

- Whole outputs on shapes that span one step, tail blocks, one to eight
  slices, ragged M and N, every kernel the M and the workspace select
  (streamed, small, tiled, register-W with 2, 4 and 8 X tiles, DMA-fed),
  both with the split workspace and without it, fp32 and bf16 outputs.
- The hand-derived step and order cases of tests/golden, run on the device.
- Special bf16 values (all 65,536 weight patterns, subnormal and signed-zero
  activations): R4 equals its twin bit for bit, NaN positions included.

The order is the one binade_r4_gemm documents ("Binade" package page,
"NVIDIA GPUs": a chain of matrix-core steps along K with a fixed split
rule); the step's arithmetic is the reading above oracle_mfma_step."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from decode_gemv_tensor_amd import binade as B

pytestmark = pytest.mark.gpu

DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(*a):
    print(*a, flush=True)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_bf16_tensor(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def same_f32(a, b) -> bool:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and
                np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


def rne_bits(f: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def inputs(M, N, K, dist, seed):
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((M, K)).astype(np.float32)
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    else:  # integers times powers of two: heavy cancellation, wide exponents
        x = (rng.integers(-128, 128, (M, K)) * 2.0 ** rng.integers(-12, 12, (M, K))).astype(np.float32)
        w = (rng.integers(-128, 128, (N, K)) * 2.0 ** rng.integers(-12, 12, (N, K))).astype(np.float32)
    return rne_bits(x), rne_bits(w)


SHAPES = [(1, 64, 32), (16, 48, 96), (17, 64, 128), (32, 80, 160), (64, 64, 1024),
          (130, 96, 1056), (128, 64, 3840), (256, 40, 4128), (16, 64, 15360),
          (300, 40, 2080), (520, 24, 9216), (48, 200, 2080), (100, 136, 3104),
          (20, 40, 24576)]


@pytest.mark.parametrize("mnk", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("dist", ["normal", "cancel"])
def test_gemm_whole_output_equals_oracle_replay(mnk, dist):
    M, N, K = mnk
    say("gemm replay", M, N, K, dist)
    xb, wb = inputs(M, N, K, dist, seed=M * 7919 + N * 31 + K + (dist == "cancel"))
    want = oracle.gemm_replay(wb, xb)
    X = to_bf16_tensor(xb).to(DEV)
    Wt = to_bf16_tensor(wb)
    Wd = Wt.to(DEV)
    r4 = B.rice_to_r4(B.pack_rice(Wt).to(DEV))
    no_ws = torch.empty(0, dtype=torch.uint8, device=DEV)
    outs = {
        "r4": B.r4_gemm(r4, X),
        "r4 unsplit": B.r4_gemm(r4, X, workspace=no_ws),
        "twin": B.bf16_gemm(Wd, X),
        "twin unsplit": B.bf16_gemm(Wd, X, workspace=no_ws),
    }
    ybf = B.r4_gemm(r4, X, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for name, y in outs.items():
        assert same_f32(y.cpu().numpy(), want), name
    assert np.array_equal(bits_np(ybf), oracle.f32_to_bf16(want))


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
    assert u & 0xFFFF == 0
    return u >> 16


# The running value c of a step case is made on the device by a first step
# (K = 64: two tail steps): columns 0..31 hold terms whose step gives c.
C_TERMS = {
    "0": [],
    "1": [(0, "1")],
    "-1": [(0, "-1")],
    "-2^-30": [(0, "-2^-15", "2^-15")],
    "0x1.fffffep-1": [(0, "1"), (1, "-2^-24")],
    "2^-148": [(0, "2^-74", "2^-74")],
    "inf": [(0, "1.9921875*2^127", "1.9921875")],
}


def test_hand_derived_cases_on_the_device():
    with open(os.path.join(GOLDEN, "mfma_step_cases.json")) as f:
        steps = json.load(f)["cases"]
    with open(os.path.join(GOLDEN, "gemm_order_cases.json")) as f:
        orders = json.load(f)["cases"]
    one = _bf16(1.0)
    rows = []  # (name, K, x row, w row, expected)
    for c in steps:
        if c["c"] not in C_TERMS:  # a -0 running value cannot come from a step
            continue
        x = np.zeros(64, np.uint16)
        w = np.full(64, one, np.uint16)
        for t in C_TERMS[c["c"]]:
            x[t[0]] = _bf16(_value(t[1]))
            if len(t) > 2:
                w[t[0]] = _bf16(_value(t[2]))
        for t in c["terms"]:
            x[32 + t[0]] = _bf16(_value(t[1]))
            if len(t) > 2:
                w[32 + t[0]] = _bf16(_value(t[2]))
        rows.append((c["name"], 64, x, w, _value(c["expect"])))
    for c in orders:
        x = np.zeros(c["K"], np.uint16)
        for col, v in c["x"]:
            x[col] = _bf16(_value(v))
        rows.append((c["name"], c["K"], x, np.full(c["K"], one, np.uint16), _value(c["expect"])))
    assert len(rows) == len(steps) - 1 + len(orders)
    for name, K, x, w, want in rows:
        say("case", name)
        X = to_bf16_tensor(x.reshape(1, K)).to(DEV)
        Wt = to_bf16_tensor(w.reshape(1, K))
        y = B.bf16_gemm(Wt.to(DEV), X).cpu().numpy()[0, 0]
        yr = B.r4_gemm(B.rice_to_r4(B.pack_rice(Wt).to(DEV)), X).cpu().numpy()[0, 0]
        if np.isnan(want):
            assert np.isnan(y) and np.isnan(yr), name
            continue
        wb = np.float32(want).view(np.uint32)
        assert np.float32(y).view(np.uint32) == wb, (name, float(y).hex(), float(want).hex())
        assert np.float32(yr).view(np.uint32) == wb, (name, float(yr).hex(), float(want).hex())


def test_gemm_special_values_r4_equals_twin():
    """Every bf16 bit pattern as a weight (256 x 256, Inf and NaN included),
    against activations with subnormals, signed zeros and normal values."""
    wb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    rng = np.random.default_rng(11)
    xb = rne_bits(rng.standard_normal((48, 256)).astype(np.float32))
    xb[0] = np.arange(256, dtype=np.uint16)            # positive subnormals and +0
    xb[1] = np.arange(256, dtype=np.uint16) | 0x8000   # negative subnormals and -0
    xb[2] = 0x8000                                     # all -0
    xb[3, ::2] = 0x0001                                # smallest subnormal
    Wt = to_bf16_tensor(wb)
    X = to_bf16_tensor(xb).to(DEV)
    r4 = B.rice_to_r4(B.pack_rice(Wt).to(DEV))
    for m in (16, 48):
        say("special values M =", m)
        y = B.r4_gemm(r4, X[:m].contiguous()).cpu().numpy()
        t = B.bf16_gemm(Wt.to(DEV), X[:m].contiguous()).cpu().numpy()
        assert same_f32(y, t), m
    # rows of W whose patterns are all finite also equal the oracle's replay
    finite = [r for r in range(256) if ((wb[r] >> 7) & 0xFF).max() < 0xFF]
    assert len(finite) == 254
    want = oracle.gemm_replay(wb[finite], xb)
    y = B.r4_gemm(r4, X).cpu().numpy()[:, finite]
    assert same_f32(y, want)
