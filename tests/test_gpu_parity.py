"""GPU parity: every device entry point through the C-ABI against the oracle
(and against its bf16 twin), on seeded inputs at sizes the oracle finishes
in seconds, spanning several tiles, chunks and ragged tails.

Bars: bit-exact for R4 / escapes / unpacked bits; matvec and expert gather
bit-identical to the oracle's replay of the fixed fp32 order and to the
bf16-weight twin, and within 1e-2 (relative to sum |w x|) of the fp64 sum.
NaN outputs compare as NaN (payload not compared)."""
import os

import numpy as np
import pytest
import torch

import oracle
from decode_gemv_tensor_amd import binade as B
from decode_gemv_tensor_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def spec(rows, cols, sigma=0.02, seed=0, frac=1e-3, scale=20.0, count=0):
    return synth.TensorSpec("t", rows, cols, sigma, seed, outlier_frac=frac,
                            outlier_scale=scale, outlier_count=count)


def to_r4(w_cpu: torch.Tensor, status=None):
    planes = B.pack_rice(w_cpu).to(DEV)
    r4 = B.rice_to_r4(planes, status=status)
    return planes, r4


def same_f32(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and
                np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


def within_f64(y, w_bits, x_bits):
    y64 = oracle.gemv_f64(w_bits, x_bits)
    wf = (w_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    scale = np.abs(wf) @ np.abs(xf)
    return bool(np.all(np.abs(np.asarray(y, np.float64) - y64) <= 1e-2 * scale + 1e-30))


GEMV_SHAPES = [(1024, 1024, 0.02, 0, 0.0, 1.0, 16, 50.0),   # single 1024 tensor
               (37, 96, 0.02, 1, 1e-2, 1e4, 0, 1.0),          # ragged rows, 3 tiles
               (5, 4160, 0.02, 2, 5e-3, 1e4, 0, 1.0),         # ragged chunk 4096+64
               (300, 3072, 0.02, 3, 1e-3, 20.0, 0, 1.0),      # Llama q/o width
               (64, 8192, 0.02, 4, 1e-3, 20.0, 0, 1.0),       # down width
               (19, 15360, 0.015, 5, 0.0, 1.0, 0, 1.0),       # 12B down width
               (4100, 256, 0.015, 6, 0.0, 1.0, 0, 1.0)]       # short rows, many


# Decode jobs: two row-chunks of a row, or 2 * (2048 / cols) short rows;
# streamed spans: 8 row-chunks (rows longer than a chunk) or 16384 / cols
# rows. Edge cases of those mappings: a one-row tensor, rows of exactly one
# chunk, a 32-column second chunk, an odd chunk count, spans that end inside
# a row, 32 short rows per job (31 inner chunk starts), one row per run, and
# rows too short for the byte-table path.
DECODE_SHAPES = [(1, 1024, 0.02, 13, 1e-3, 20.0, 0, 1.0),      # one row: a span of one round
                 (3, 1152, 0.02, 14, 5e-3, 1e3, 0, 1.0),      # rows of 1152: one chunk each
                 (2, 17408, 0.015, 15, 1e-3, 20.0, 0, 1.0),   # 9 chunks per row, spans across rows
                 (9, 2048, 0.02, 7, 1e-3, 20.0, 0, 1.0),
                 (7, 2080, 0.02, 8, 2e-3, 1e3, 0, 1.0),
                 (11, 6144, 0.02, 9, 1e-3, 20.0, 0, 1.0),
                 (130, 128, 0.02, 10, 5e-3, 1e3, 0, 1.0),
                 (33, 1344, 0.015, 11, 1e-3, 20.0, 0, 1.0),
                 (50, 64, 0.02, 12, 1e-2, 1e3, 0, 1.0)]


@pytest.mark.parametrize("shape", GEMV_SHAPES + DECODE_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_rice_to_r4_is_byte_exact_and_unpacks(shape):
    rows, cols, sigma, seed, frac, scale, count, cscale = shape
    sp = spec(rows, cols, sigma, seed, frac, scale if count == 0 else cscale, count)
    w = synth.normal_bf16(sp)
    wn = bits_np(w)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    planes, r4 = to_r4(w, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = oracle.make_r4(wn, oracle.build_table(wn))
    assert bytes(bytearray(r4.lut)) == bytes(ref["lut"])
    assert np.array_equal(r4.nib.cpu().numpy(), ref["nib"].reshape(-1))
    assert r4.n_esc == ref["n_esc"]
    if r4.n_esc:
        assert np.array_equal(r4.esc[: r4.n_esc].cpu().numpy().view(np.uint32), ref["esc"])
    assert np.array_equal(r4.esc_pre.cpu().numpy().view(np.uint32), ref["esc_pre"])
    assert np.array_equal(bits_np(B.unpack(r4)), wn)


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_r4_gemv_matches_oracle_twin_and_f64(shape):
    rows, cols, sigma, seed, frac, scale, count, cscale = shape
    sp = spec(rows, cols, sigma, seed, frac, scale if count == 0 else cscale, count)
    w = synth.normal_bf16(sp)
    wn = bits_np(w)
    x = synth.vector_bf16(cols, 100 + seed)
    xn = bits_np(x)
    _, r4 = to_r4(w)
    xd = x.to(DEV)
    y = B.r4_gemv(r4, xd).cpu().numpy()
    y_twin = B.bf16_gemv(w.to(DEV), xd).cpu().numpy()
    y_ref = oracle.gemv_replay(wn, xn)
    assert same_f32(y, y_ref)
    assert same_f32(y_twin, y_ref)
    assert within_f64(y, wn, xn)
    yb = bits_np(B.r4_gemv(r4, xd, out_dtype=torch.bfloat16))
    assert np.array_equal(yb, oracle.f32_to_bf16(y_ref))


_SHAPE_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
from decode_gemv_tensor_amd import binade as B
w = torch.from_numpy(np.load(sys.argv[2]).view(np.int16)).view(torch.bfloat16)
x = torch.from_numpy(np.load(sys.argv[3]).view(np.int16)).view(torch.bfloat16)
r4 = B.rice_to_r4(B.pack_rice(w).to("cuda"))
y = B.r4_gemv(r4, x.to("cuda")).cpu().numpy()
np.save(sys.argv[4], y)
"""


def test_gemv_bits_do_not_depend_on_launch_shape(tmp_path):
    """The launch-shape knobs are read once per process, so each variant runs
    in a child process of its own (one at a time)."""
    import subprocess
    import sys
    w = synth.normal_bf16(spec(203, 3072, seed=9))
    x = synth.vector_bf16(3072, 10)
    np.save(tmp_path / "w.npy", bits_np(w))
    np.save(tmp_path / "x.npy", bits_np(x))
    ref = oracle.gemv_replay(bits_np(w), bits_np(x))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for env in ({"BINADE_GEMV_ROWS_PER_WAVE": "2"}, {"BINADE_GEMV_ROWS_PER_WAVE": "4"},
                {"BINADE_GEMV_PREFETCH": "1"}):
        out = tmp_path / "y.npy"
        r = subprocess.run([sys.executable, "-c", _SHAPE_CHILD, root, str(tmp_path / "w.npy"),
                            str(tmp_path / "x.npy"), str(out)],
                           env={**os.environ, **env}, timeout=300, capture_output=True, text=True)
        assert r.returncode == 0, (env, r.stderr[-2000:])
        assert same_f32(np.load(out), ref), env
    _, r4 = to_r4(w)
    assert same_f32(B.r4_gemv(r4, x.to(DEV)).cpu().numpy(), ref)
    assert same_f32(B.bf16_gemv(w.to(DEV), x.to(DEV)).cpu().numpy(), ref)


def test_exhaustive_bit_patterns_through_the_device():
    """All 65,536 bf16 patterns in one tensor (241 of 256 exponents escape):
    Rice -> R4 on the device, unpack back bit for bit, matvec = oracle."""
    w = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).reshape(64, 1024)
    wn = bits_np(w)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, r4 = to_r4(w, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert r4.n_esc == 241 * 256
    ref = oracle.make_r4(wn, oracle.build_table(wn))
    assert np.array_equal(r4.nib.cpu().numpy(), ref["nib"].reshape(-1))
    assert np.array_equal(r4.esc.cpu().numpy().view(np.uint32), ref["esc"])
    assert np.array_equal(bits_np(B.unpack(r4)), wn)
    x = synth.vector_bf16(1024, 11)
    y = B.r4_gemv(r4, x.to(DEV)).cpu().numpy()
    assert same_f32(y, oracle.gemv_replay(wn, bits_np(x)))


@pytest.mark.parametrize("sigma,frac,scale", [(1.0, 0.0, 1.0), (1e-30, 0.01, 1e30),
                                              (3e4, 0.0, 1.0), (0.02, 0.2, 1e6)])
def test_other_rice_parameters(sigma, frac, scale):
    """Tables whose best k is not 1 (wide or bimodal exponent spreads)."""
    w = synth.normal_bf16(spec(48, 2080, sigma, 21, frac, scale))
    wn = bits_np(w)
    planes, r4 = to_r4(w)
    ref = oracle.make_r4(wn, oracle.build_table(wn))
    assert np.array_equal(r4.nib.cpu().numpy(), ref["nib"].reshape(-1))
    assert np.array_equal(bits_np(B.unpack(r4)), wn)


def test_corrupt_stream_sets_status():
    w = synth.normal_bf16(spec(8, 2080, seed=12))
    planes = B.pack_rice(w)
    # flip a unary bit: the affected chunk holds one weight too many or few
    bad_unary = planes.unary.clone()
    bad_unary[5] ^= 1 << 7
    bad = B.RicePlanes(planes.rows, planes.cols, planes.table, planes.sm,
                       bad_unary, planes.rem, planes.anchor, planes.esc_pre,
                       planes.unary_bits, planes.n_esc).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.rice_to_r4(bad, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & B.DEV_CORRUPT_STREAM
    # inconsistent escape prefix
    esc_pre = planes.esc_pre.clone()
    esc_pre[1] += 1
    bad2 = B.RicePlanes(planes.rows, planes.cols, planes.table, planes.sm,
                        planes.unary, planes.rem, planes.anchor, esc_pre,
                        planes.unary_bits, planes.n_esc).to(DEV)
    status.zero_()
    B.rice_to_r4(bad2, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & B.DEV_CORRUPT_ESC


def test_rank_outside_the_table_sets_status():
    """Planes whose codes agree with their anchors and prefixes, decoded with
    a table one rank short: the weights of the missing rank are flagged, not
    decoded through a stale entry. A 1 x 64 tensor over three exponents (the
    per-weight walk) and a 64 x 2080 tensor with outliers (the byte walk of
    tables of 15 ranks or more)."""
    exps = np.array([120] * 40 + [121] * 20 + [122] * 4, np.uint16)
    small = torch.from_numpy((((exps << 7) | np.arange(64, dtype=np.uint16))
                              .reshape(1, 64)).view(np.int16)).view(torch.bfloat16)
    wide = synth.normal_bf16(synth.TensorSpec("t", 64, 2080, 0.02, 21, outlier_frac=1e-3,
                                              outlier_scale=20.0))
    for name, w in (("1x64", small), ("64x2080", wide)):
        planes = B.pack_rice(w)
        print("rank outside the table", name, "n =", planes.table.n, "k =", planes.table.k, flush=True)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        B.rice_to_r4(planes.to(DEV), status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, name
        short = B.Table.from_buffer_copy(planes.table)
        short.n -= 1
        bad = B.RicePlanes(planes.rows, planes.cols, short, planes.sm, planes.unary,
                           planes.rem, planes.anchor, planes.esc_pre, planes.unary_bits,
                           planes.n_esc).to(DEV)
        B.rice_to_r4(bad, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & B.DEV_CORRUPT_STREAM, name


def _wide_exponents(rows, cols, seed, spread_frac):
    """N(0, 0.02) with a fraction of the weights given exponents spread over
    2^-100 .. 2^100 (a table of about 200 ranks, many escapes)."""
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(rows, cols, generator=g) * 0.02
    pick = torch.rand(rows, cols, generator=g) < spread_frac
    e = torch.randint(-100, 100, (rows, cols), generator=g).to(torch.float32)
    return torch.where(pick, w.sign() * torch.exp2(e), w).to(torch.bfloat16)


@pytest.mark.parametrize("rows,cols", [(64, 3072), (96, 256), (23, 15360)])
def test_streamed_decode_with_dense_escapes(rows, cols):
    """Rice k = 1 with 2% of the weights far from the bulk: codes of up to 100
    unary bits cross lane and round boundaries, and many 64-bit lane windows
    hold three or more escapes (written by a second walk)."""
    w = _wide_exponents(rows, cols, 31 + cols, 0.02)
    wn = bits_np(w)
    planes = B.pack_rice(w)
    assert planes.k == 1 and planes.table.n >= 15
    ref = oracle.make_r4(wn, oracle.build_table(wn))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    r4 = B.rice_to_r4(planes.to(DEV), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert r4.n_esc == ref["n_esc"]
    assert np.array_equal(r4.nib.cpu().numpy(), ref["nib"].reshape(-1))
    assert np.array_equal(r4.esc[: r4.n_esc].cpu().numpy().view(np.uint32), ref["esc"])
    assert np.array_equal(bits_np(B.unpack(r4)), wn)


def _replace(planes, **kw):
    f = dict(rows=planes.rows, cols=planes.cols, table=planes.table, sm=planes.sm,
             unary=planes.unary, rem=planes.rem, anchor=planes.anchor, esc_pre=planes.esc_pre,
             unary_bits=planes.unary_bits, n_esc=planes.n_esc)
    f.update(kw)
    return B.RicePlanes(f["rows"], f["cols"], f["table"], f["sm"], f["unary"], f["rem"],
                        f["anchor"], f["esc_pre"], f["unary_bits"], f["n_esc"])


@pytest.mark.parametrize("chunk", [1, 4, 9])
def test_streamed_decode_checks_every_chunk_start(chunk):
    """A 64 x 3072 tensor (two row-chunks per row, several per decode span):
    an escape prefix one too large, an anchor one bit late and a flipped
    unary bit, at a chunk inside a span (1, 9) and at a span's first chunk
    (4), each set the status word."""
    w = _wide_exponents(64, 3072, 77, 0.005)
    planes = B.pack_rice(w)
    assert planes.k == 1 and planes.table.n >= 15
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.rice_to_r4(planes.to(DEV), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    esc_pre = planes.esc_pre.clone()
    esc_pre[chunk:] += 1
    n_esc = planes.n_esc + 1
    cases = {"escape prefix": _replace(planes, esc_pre=esc_pre, n_esc=n_esc)}
    anchor = planes.anchor.clone()
    anchor[chunk] += 1
    cases["anchor"] = _replace(planes, anchor=anchor)
    unary = planes.unary.clone()
    word = int(planes.anchor[chunk].item()) // 32 + 3
    unary[word] ^= 1 << 9
    cases["unary bit"] = _replace(planes, unary=unary)
    for name, bad in cases.items():
        print("streamed decode corruption", name, "chunk", chunk, flush=True)
        status.zero_()
        r4 = B.rice_to_r4(bad.to(DEV), status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & (B.DEV_CORRUPT_STREAM | B.DEV_CORRUPT_ESC), name


# ---------------------------------------------------------- order pins on GPU
BIG = 4096.0


def _pin(K, terms):
    w = np.zeros(K, np.float32)
    x = np.zeros(K, np.float32)
    for i, wi, xi in terms:
        w[i], x[i] = wi, xi
    wt = torch.tensor(w).to(torch.bfloat16).reshape(1, K)
    xt = torch.tensor(x).to(torch.bfloat16)
    _, r4 = to_r4(wt)
    return (B.r4_gemv(r4, xt.to(DEV)).item(), B.bf16_gemv(wt.to(DEV), xt.to(DEV)).item())


def test_order_pins_hold_on_the_device():
    # same hand-derived cases as the oracle's pins
    assert _pin(32, [(0, BIG, BIG), (2, 1, 1), (4, -BIG, BIG)]) == (0.0, 0.0)
    assert _pin(32, [(1, BIG, BIG), (2, 1, 1), (4, -BIG, BIG)]) == (1.0, 1.0)
    assert _pin(4096, [(0, BIG, BIG), (2050, 1, 1), (2052, -BIG, BIG)]) == (0.0, 0.0)
    assert _pin(2048, [(0, BIG, BIG), (1024, 1, 1), (512, -BIG, BIG)]) == (0.0, 0.0)
    w = -torch.ones(3, 64, dtype=torch.bfloat16)
    x = torch.zeros(64, dtype=torch.bfloat16)
    _, r4 = to_r4(w)
    y = B.r4_gemv(r4, x.to(DEV)).cpu()
    assert y.view(torch.int32).tolist() == [0, 0, 0]
    # one rounding per chain step: 2^-149 then a 2^-150 product, fused,
    # is a tie that goes to the even 2^-148 (the oracle's pin of the fma)
    t = 2.0 ** -148
    assert _pin(32, [(0, 2.0 ** -74, 2.0 ** -75), (2, 2.0 ** -75, 2.0 ** -75)]) == (t, t)


# ---------------------------------------------------------- MoE
def _moe_case(E, N, K, n_tokens, top_k, seed, x_per_slot):
    w = synth.normal_bf16(spec(E * N, K, 0.02, seed, 1e-3, 20.0))
    idx = synth.topk_indices(n_tokens, top_k, E, seed + 1)
    nx = n_tokens * top_k if x_per_slot else n_tokens
    x = synth.vector_bf16(K, seed + 2, count=nx)
    return w, idx, x


@pytest.mark.parametrize("case", [(16, 40, 96, 3, 4, False), (128, 704, 2816, 8, 8, False),
                                  (128, 2816, 704, 8, 8, True), (6, 33, 4160, 5, 2, True),
                                  (5, 37, 2240, 6, 3, False), (7, 9, 3072, 4, 5, True)],
                         ids=["small", "gate_up", "down", "ragged", "paired_rows_odd",
                              "paired_rows_96"])
def test_moe_matches_oracle_and_twin(case):
    E, N, K, T, k, per_slot = case
    w, idx, x = _moe_case(E, N, K, T, k, 40 + E, per_slot)
    _, r4 = to_r4(w)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = B.r4_moe_gemv(r4, E, x.to(DEV), idx.to(DEV), x_per_slot=per_slot,
                      status=status).cpu().numpy()
    y2 = B.bf16_moe_gemv(w.to(DEV), E, x.to(DEV), idx.to(DEV),
                         x_per_slot=per_slot).cpu().numpy()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = oracle.moe_replay(bits_np(w).reshape(E, N, K), bits_np(x), idx.numpy(), per_slot)
    assert same_f32(y, ref)
    assert same_f32(y2, ref)


def test_moe_paired_rows_with_many_escapes_and_bf16_output():
    """Rows of 88 tiles (gate/up width 2816) run two per wave with a merged
    second pass; exponents spread over 41 values put most weights in the side
    list (hundreds of escapes per row pair, beyond what a wave keeps in
    registers). Outputs in fp32 and bf16 against the oracle and the twin."""
    E, N, K, T, k = 5, 9, 2816, 4, 3
    rng = np.random.default_rng(123)
    sign = rng.integers(0, 2, (E * N, K)).astype(np.uint16) << 15
    expo = rng.integers(100, 141, (E * N, K)).astype(np.uint16) << 7
    mant = rng.integers(0, 128, (E * N, K)).astype(np.uint16)
    wb = sign | expo | mant
    w = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16)
    idx = synth.topk_indices(T, k, E, 9)
    x = synth.vector_bf16(K, 10, count=T)
    planes, r4 = to_r4(w)
    assert planes.n_esc > 0.5 * E * N * K
    ref = oracle.moe_replay(wb.reshape(E, N, K), bits_np(x), idx.numpy(), False)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = B.r4_moe_gemv(r4, E, x.to(DEV), idx.to(DEV), status=status).cpu().numpy()
    yb = B.r4_moe_gemv(r4, E, x.to(DEV), idx.to(DEV), out_dtype=torch.bfloat16)
    tb = B.bf16_moe_gemv(w.to(DEV), E, x.to(DEV), idx.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert same_f32(y, ref)
    assert np.array_equal(bits_np(yb), oracle.f32_to_bf16(ref))
    assert np.array_equal(bits_np(tb), oracle.f32_to_bf16(ref))


def test_moe_shared_experts_and_bad_index():
    E, N, K = 8, 24, 64
    w, _, x = _moe_case(E, N, K, 6, 2, 77, False)
    idx = torch.tensor([[3, 3], [3, 1], [3, 0], [3, 3], [3, 5], [3, 3]], dtype=torch.int32)
    _, r4 = to_r4(w)
    y = B.r4_moe_gemv(r4, E, x.to(DEV), idx.to(DEV)).cpu().numpy()
    ref = oracle.moe_replay(bits_np(w).reshape(E, N, K), bits_np(x), idx.numpy(), False)
    assert same_f32(y, ref)
    idx_bad = idx.clone()
    idx_bad[2, 1] = E + 4
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = B.r4_moe_gemv(r4, E, x.to(DEV), idx_bad.to(DEV), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & B.DEV_BAD_INDEX
    assert torch.count_nonzero(y[5]).item() == 0


# ---------------------------------------------------------- GEMM
@pytest.mark.parametrize("mnk", [(16, 64, 64), (33, 200, 96), (128, 384, 3840), (5, 70, 4160),
                                 (300, 136, 4160), (260, 40, 96), (130, 70, 4160)])
def test_gemm_small_integers_exact_and_twin(mnk):
    M, N, K = mnk
    g = torch.Generator().manual_seed(M * N)
    W = torch.randint(-4, 5, (N, K), generator=g).to(torch.bfloat16)
    X = torch.randint(-4, 5, (M, K), generator=g).to(torch.bfloat16)
    _, r4 = to_r4(W)
    Y = B.r4_gemm(r4, X.to(DEV)).cpu()
    Y2 = B.bf16_gemm(W.to(DEV), X.to(DEV)).cpu()
    exact = X.to(torch.int64) @ W.to(torch.int64).T
    assert torch.equal(Y.to(torch.int64), exact)
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))


@pytest.mark.parametrize("mnk", [(16, 128, 3840), (32, 96, 15360), (130, 64, 3840),
                                 (7, 33, 512), (24, 1000, 1024), (20, 300, 4160),
                                 (260, 96, 8192), (520, 130, 4160)])
def test_gemm_random_twin_and_f64(mnk):
    M, N, K = mnk
    W = synth.normal_bf16(spec(N, K, 0.015, M, 1e-3, 20.0))
    X = synth.vector_bf16(K, M + 1, count=M)
    _, r4 = to_r4(W)
    Y = B.r4_gemm(r4, X.to(DEV)).cpu()
    Y2 = B.bf16_gemm(W.to(DEV), X.to(DEV)).cpu()
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    wb, xb = bits_np(W), bits_np(X)
    ref = oracle.gemm_f64(wb, xb)
    # sum of |products|: the same definition on the magnitudes
    scale = oracle.gemm_f64(wb & 0x7FFF, xb & 0x7FFF)
    assert np.all(np.abs(Y.numpy().astype(np.float64) - ref) <= 1e-2 * scale)
    Yb = B.r4_gemm(r4, X.to(DEV), out_dtype=torch.bfloat16).cpu()
    assert np.array_equal(bits_np(Yb), oracle.f32_to_bf16(Y.numpy()))


@pytest.mark.parametrize("m", [16, 30, 33, 300])
def test_gemm_strided_x_and_y(m):
    """X and Y wider than the product (ldx = K + 72, ldy = N + 8) through the
    C ABI, on the streamed (M <= 32), tiled (33) and DMA-fed (300) kernels:
    the same bits as the contiguous call, and Y's padding columns untouched."""
    import ctypes
    N, K = 136, 4160
    W = synth.normal_bf16(spec(N, K, 0.015, m, 2e-3, 1e3))
    X = synth.vector_bf16(K, m + 3, count=m)
    _, r4 = to_r4(W)
    Xd = X.to(DEV)
    ref = B.r4_gemm(r4, Xd).cpu()
    xw = torch.zeros(m, K + 72, dtype=torch.bfloat16, device=DEV)
    xw[:, :K] = Xd
    sentinel = -12345.0
    for r4_side in (True, False):
        yw = torch.full((m, N + 8), sentinel, dtype=torch.float32, device=DEV)
        nb = B.gemm_workspace_bytes(m, N, K)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
        st = B._stream(None)
        if r4_side:
            d = r4.desc()
            B._call("binade_r4_gemm", ctypes.byref(d), B._ptr(xw), m, xw.stride(0), B._ptr(yw),
                    yw.stride(0), B.F32, B._ptr(ws), nb, st)
        else:
            wd = W.to(DEV)
            B._call("binade_bf16_gemm", B._ptr(wd), N, K, B._ptr(xw), m, xw.stride(0),
                    B._ptr(yw), yw.stride(0), B.F32, B._ptr(ws), nb, st)
        torch.cuda.synchronize()
        y = yw.cpu()
        assert torch.equal(y[:, :N].contiguous().view(torch.int32), ref.view(torch.int32))
        assert torch.all(y[:, N:] == sentinel)


# ---------------------------------------------------------- batched launches
def test_batched_decode_and_gemv_equal_single_calls():
    shapes = [(300, 3072), (64, 8192), (37, 96), (4100, 256), (5, 4160), (1024, 1024),
              (19, 15360), (128, 2816), (33, 704), (8, 2080)] * 2   # 20: two launches each
    ws = [synth.normal_bf16(spec(n, k, 0.02, 200 + i, 1e-3, 20.0)) for i, (n, k) in enumerate(shapes)]
    planes = [B.pack_rice(w).to(DEV) for w in ws]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = B.rice_to_r4_batch(planes, status=status)
    singles = [B.rice_to_r4(p) for p in planes]
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for o, s1 in zip(outs, singles):
        assert o.lut == s1.lut
        assert torch.equal(o.nib, s1.nib)
        assert torch.equal(o.esc[: o.n_esc], s1.esc[: s1.n_esc])
    xs = [synth.vector_bf16(k, 300 + i).to(DEV) for i, (n, k) in enumerate(shapes)]
    ys = B.r4_gemv_batch(outs, xs)
    for i, (o, x, y) in enumerate(zip(outs, xs, ys)):
        y1 = B.r4_gemv(o, x)
        assert torch.equal(y.view(torch.int32), y1.view(torch.int32)), shapes[i]
    wn = bits_np(ws[0])
    assert same_f32(ys[0].cpu().numpy(), oracle.gemv_replay(wn, bits_np(xs[0].cpu())))
    yt = B.bf16_gemv_batch([w.to(DEV) for w in ws], xs, out_dtype=torch.bfloat16)
    for i, (o, x, y) in enumerate(zip(outs, xs, yt)):
        y1 = B.r4_gemv(o, x, out_dtype=torch.bfloat16)
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), shapes[i]


def test_batched_decode_splits_on_wide_tables():
    """Tensors whose tables hold many exponents (their escape exponents fill
    a launch's argument pool after a few tensors): the batched call splits
    into several launches and still equals the single calls."""
    def wide(rows, cols, seed, spread_frac):
        # N(0, 0.02), with a fraction of the weights given exponents spread
        # over 2^-100 .. 2^100
        g = torch.Generator().manual_seed(seed)
        w = torch.randn(rows, cols, generator=g) * 0.02
        pick = torch.rand(rows, cols, generator=g) < spread_frac
        e = torch.randint(-100, 100, (rows, cols), generator=g).to(torch.float32)
        return torch.where(pick, w.sign() * torch.exp2(e), w).to(torch.bfloat16)

    # Rice k = 1 (byte-table path) and k = 5 (general path) in turn
    ws = [wide(64 + 16 * i, 512 + 1536 * (i % 2), 600 + i, 0.5 if i % 2 else 0.005)
          for i in range(12)]
    planes = [B.pack_rice(w).to(DEV) for w in ws]
    assert min(p.table.n for p in planes) > 100
    assert {p.k for p in planes} == {1, 5}
    assert sum(p.table.n - 15 for p in planes) > 1024   # more than one launch's pool
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = B.rice_to_r4_batch(planes, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for w, o in zip(ws, outs):
        wn = bits_np(w)
        ref = oracle.make_r4(wn, oracle.build_table(wn))
        assert o.n_esc == ref["n_esc"] and o.n_esc > 0
        assert np.array_equal(o.nib.cpu().numpy(), ref["nib"].reshape(-1))
        assert np.array_equal(o.esc[: o.n_esc].cpu().numpy().view(np.uint32), ref["esc"])
        assert np.array_equal(bits_np(B.unpack(o)), wn)


def test_decode_plan_runs_every_tensor_in_one_launch():
    """A plan of 20 tensors (more than one batched launch holds), wide tables
    with dense escapes among them, run twice over outputs filled with junk:
    every tensor's R4 equals the oracle's both times."""
    shapes = [(300, 3072), (64, 8192), (1, 4096), (3, 1152), (2, 17408), (7, 2176),
              (33, 1344), (9, 2048), (11, 6144), (19, 15360), (24, 3072), (4, 8192),
              (5, 4352), (128, 2816), (1, 15360), (6, 5120), (40, 1024), (2, 3072)]
    ws = [synth.normal_bf16(spec(n, k, 0.02, 700 + i, 1e-3, 20.0)) for i, (n, k) in enumerate(shapes)]
    ws += [_wide_exponents(64, 3072, 731, 0.02), _wide_exponents(23, 15360, 732, 0.02)]
    planes = [B.pack_rice(w).to(DEV) for w in ws]
    assert all(p.k == 1 and p.table.n >= 15 for p in planes)
    plan = B.RicePlan(planes)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    refs = []
    for w in ws:
        wn = bits_np(w)
        refs.append(oracle.make_r4(wn, oracle.build_table(wn)))
    for rep in range(2):
        print("decode plan run", rep, flush=True)
        for o in plan.outs:
            o.nib.fill_(0xA5)
            o.esc.fill_(-1)
        outs = plan.run(status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert o.lut == bytes(ref["lut"]), i
            assert o.n_esc == ref["n_esc"], i
            assert np.array_equal(o.nib.cpu().numpy(), ref["nib"].reshape(-1)), i
            if o.n_esc:
                assert np.array_equal(o.esc[: o.n_esc].cpu().numpy().view(np.uint32), ref["esc"]), i
    assert np.array_equal(bits_np(B.unpack(plan.outs[-1])), bits_np(ws[-1]))


def test_decode_plan_flags_a_corrupt_tensor():
    """One tensor of a plan with an anchor one bit late: the run sets the
    status word; the same plan without it runs clean."""
    ws = [synth.normal_bf16(spec(n, k, 0.02, 750 + i, 1e-3, 20.0))
          for i, (n, k) in enumerate([(64, 3072), (16, 8192), (48, 3072)])]
    planes = [B.pack_rice(w) for w in ws]
    anchor = planes[1].anchor.clone()
    anchor[5] += 1
    bad = _replace(planes[1], anchor=anchor)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    good = B.RicePlan([p.to(DEV) for p in planes])
    good.run(status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    plan = B.RicePlan([planes[0].to(DEV), bad.to(DEV), planes[2].to(DEV)])
    plan.run(status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & (B.DEV_CORRUPT_STREAM | B.DEV_CORRUPT_ESC)


@pytest.mark.parametrize("nk", [(200, 15360), (136, 8192), (72, 3840), (72, 4160), (40, 96)])
def test_gemm_rows_do_not_depend_on_m(nk):
    """The GEMM order depends on K only: the same X row gives the same bits
    whether the call has 16 or 32 rows (small-M kernel) or 33 .. 300 rows
    (tiled kernel, slices in separate blocks or in one), with split-K slices
    (K = 8192, 15360), 32-column tail blocks (K = 4160, 96) and escapes."""
    N, K = nk
    W = synth.normal_bf16(spec(N, K, 0.015, N + 7, 2e-3, 1e3))
    X = synth.vector_bf16(K, N + 8, count=300)
    _, r4 = to_r4(W)
    Xd, Wd = X.to(DEV), W.to(DEV)
    full = B.r4_gemm(r4, Xd).cpu()
    assert torch.equal(full.view(torch.int32), B.bf16_gemm(Wd, Xd).cpu().view(torch.int32))
    no_ws = torch.empty(0, dtype=torch.uint8, device=DEV)   # slices in one block
    for m in (16, 32, 33, 64, 65, 128, 129):
        xm = Xd[:m].contiguous()
        part = B.r4_gemm(r4, xm).cpu()
        assert torch.equal(part.view(torch.int32), full[:m].view(torch.int32)), m
        twin = B.bf16_gemm(Wd, xm).cpu()
        assert torch.equal(twin.view(torch.int32), part.view(torch.int32)), m
        one = B.r4_gemm(r4, xm, workspace=no_ws).cpu()
        assert torch.equal(one.view(torch.int32), part.view(torch.int32)), m
    assert torch.equal(B.r4_gemm(r4, Xd, workspace=no_ws).cpu().view(torch.int32),
                       full.view(torch.int32))
    wb, xb = bits_np(W), bits_np(X[:40])
    ref = oracle.gemm_f64(wb, xb)
    scale = oracle.gemm_f64(wb & 0x7FFF, xb & 0x7FFF)
    assert np.all(np.abs(full[:40].numpy().astype(np.float64) - ref) <= 1e-2 * scale)
