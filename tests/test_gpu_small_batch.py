"""GPU parity of the small-batch decode product and the MoE epilogue through
the C ABI ("Binade" package page, "Limitations": the fused kernels cover the
small dense products and every expert product; "How it works": the MoE
layer's gather).

- binade_r4_gemv_rows / binade_bf16_gemv_rows: every row of Y bit-identical
  to the oracle's replay of the batch-1 order for that row of X, to the
  batch-1 device product of that row, and to the twin; m = 1..8, ragged K,
  short and escape-heavy rows, strided X and Y, bf16 output, and the 12B-FFN
  shapes at m = 8 on sampled rows.
- binade_moe_silu_mul: within one fp32 ulp of the oracle (fp64 inside on
  both sides; their exp may differ in the last bits of a double), equal
  bits almost everywhere; specials as the formula gives.
- binade_moe_combine: bit-identical to the oracle's fma chain, fp32 and bf16.
- A whole MoE layer (gate, up, silu*up, down per slot, combine) against the
  oracle stage by stage."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from decode_gemv_tensor_amd import binade as B
from decode_gemv_tensor_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def same_f32(a, b) -> bool:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and
                np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


def spec(rows, cols, sigma=0.02, seed=0, frac=1e-3, scale=20.0):
    return synth.TensorSpec("t", rows, cols, sigma, seed, outlier_frac=frac, outlier_scale=scale)


def to_r4(w_cpu):
    return B.rice_to_r4(B.pack_rice(w_cpu).to(DEV))


ROWS_SHAPES = [(37, 96, 1e-2, 1e4), (5, 4160, 5e-3, 1e4), (300, 3072, 1e-3, 20.0),
               (64, 8192, 1e-3, 20.0), (19, 15360, 0.0, 1.0), (700, 256, 0.0, 1.0)]


@pytest.mark.parametrize("shape", ROWS_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_gemv_rows_equal_batch1_order(shape, m):
    N, K, frac, scale = shape
    say("gemv rows", N, K, "m =", m)
    w = synth.normal_bf16(spec(N, K, 0.02, N + K, frac, scale))
    x = synth.vector_bf16(K, 7 * m + K, count=m)
    r4 = to_r4(w)
    xd = x.to(DEV)
    y = B.r4_gemv_rows(r4, xd)
    yt = B.bf16_gemv_rows(w.to(DEV), xd)
    ybf = B.r4_gemv_rows(r4, xd, out_dtype=torch.bfloat16)
    single = [B.r4_gemv(r4, xd[b].contiguous()) for b in range(m)]
    torch.cuda.synchronize()
    ref = oracle.gemv_rows_replay(bits_np(w), bits_np(x))
    assert same_f32(y.cpu().numpy(), ref)
    assert same_f32(yt.cpu().numpy(), ref)
    assert np.array_equal(bits_np(ybf), oracle.f32_to_bf16(ref))
    for b in range(m):
        assert same_f32(single[b].cpu().numpy(), ref[b])


def test_gemv_rows_all_bit_patterns():
    """Every bf16 pattern as a weight (Inf and NaN included): R4 rows equal
    the twin's rows, NaN positions included, and finite rows equal the
    oracle."""
    wb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    w = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16)
    x = synth.vector_bf16(256, 3, count=6)
    r4 = to_r4(w)
    y = B.r4_gemv_rows(r4, x.to(DEV)).cpu().numpy()
    yt = B.bf16_gemv_rows(w.to(DEV), x.to(DEV)).cpu().numpy()
    assert same_f32(y, yt)
    finite = [r for r in range(256) if ((wb[r] >> 7) & 0xFF).max() < 0xFF]
    ref = oracle.gemv_rows_replay(wb[finite], bits_np(x))
    assert same_f32(y[:, finite], ref)


def test_gemv_rows_strided_through_the_abi():
    """X and Y rows further apart than K and N, called through the C ABI."""
    N, K, m = 70, 4160, 4
    w = synth.normal_bf16(spec(N, K, 0.02, 17))
    x = synth.vector_bf16(K, 18, count=m)
    r4 = to_r4(w)
    ldx, ldy = K + 24, N + 5
    xs = torch.zeros(m, ldx, dtype=torch.bfloat16)
    xs[:, :K] = x
    xs = xs.to(DEV)
    ys = torch.full((m, ldy), -7.0, dtype=torch.float32, device=DEV)
    d = r4.desc()
    rc = B.lib().binade_r4_gemv_rows(ctypes.byref(d), ctypes.c_void_p(xs.data_ptr()), ldx, m,
                                     ctypes.c_void_p(ys.data_ptr()), ldy, B.F32,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == B.OK
    torch.cuda.synchronize()
    out = ys.cpu().numpy()
    assert same_f32(out[:, :N], oracle.gemv_rows_replay(bits_np(w), bits_np(x)))
    assert np.all(out[:, N:] == -7.0)
    # m outside 1..8 and a too-short ldx are refused
    for mm, lx in [(0, ldx), (9, ldx), (m, K - 32)]:
        assert B.lib().binade_r4_gemv_rows(ctypes.byref(d), ctypes.c_void_p(xs.data_ptr()), lx, mm,
                                           ctypes.c_void_p(ys.data_ptr()), ldy, B.F32,
                                           None) == B.EINVAL


def test_gemv_rows_full_size_sampled():
    """The 12B-FFN shapes at m = 8 (the bench's launch), 48 sampled weight
    rows of each against the oracle's replay; all rows against the twin."""
    x8 = {3840: synth.vector_bf16(3840, 51, count=8), 15360: synth.vector_bf16(15360, 52, count=8)}
    rng = np.random.default_rng(4)
    for sp in synth.gemma_12b_ffn()[1:]:
        say("gemv rows full size", sp.name, sp.rows, sp.cols)
        w = synth.normal_bf16(sp)
        x = x8[sp.cols]
        r4 = to_r4(w)
        y = B.r4_gemv_rows(r4, x.to(DEV)).cpu().numpy()
        yt = B.bf16_gemv_rows(w.to(DEV), x.to(DEV)).cpu().numpy()
        assert same_f32(y, yt)
        rows = np.sort(rng.choice(sp.rows, 48, replace=False))
        ref = oracle.gemv_rows_replay(bits_np(w)[rows], bits_np(x))
        assert same_f32(y[:, rows], ref)


def f32_ulps(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def test_silu_mul_against_oracle():
    rng = np.random.default_rng(21)
    g = (rng.standard_normal(200_003) * 4).astype(np.float32)
    u = rng.standard_normal(200_003).astype(np.float32)
    g[:12] = [0.0, -0.0, np.inf, -np.inf, np.nan, 100.0, -100.0, -1000.0, 1e-40, -1e-40,
              3.4e38, -88.0]
    u[:12] = 1.0
    ref = oracle.silu_mul(g, u)
    h = B.moe_silu_mul(torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV),
                       out_dtype=torch.float32).cpu().numpy()
    hb = B.moe_silu_mul(torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV),
                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(h))
    d = f32_ulps(h[~nan], ref[~nan])
    assert d.max() <= 1
    assert np.count_nonzero(d) <= 20        # exp in fp64 on both sides: equal almost always
    assert np.array_equal(bits_np(hb)[~nan], oracle.f32_to_bf16(h)[~nan])
    assert np.signbit(h[1]) == np.signbit(ref[1]) and h[7] == 0.0


@pytest.mark.parametrize("tkn", [(8, 8, 2816), (5, 3, 77), (1, 1, 31), (3, 16, 1000)])
def test_combine_against_oracle(tkn):
    T, k, n = tkn
    rng = np.random.default_rng(T * 100 + k)
    y = rng.standard_normal((T * k, n)).astype(np.float32)
    y[0, :3] = [2.0 ** 24, np.inf, np.nan]
    w = synth.router_weights(T, k, 33 + k).numpy()
    ref = oracle.moe_combine(y, w, k)
    out = B.moe_combine(torch.from_numpy(y).to(DEV), torch.from_numpy(w).to(DEV), k).cpu().numpy()
    outb = B.moe_combine(torch.from_numpy(y).to(DEV), torch.from_numpy(w).to(DEV), k,
                         out_dtype=torch.bfloat16)
    assert same_f32(out, ref)
    assert np.array_equal(bits_np(outb), oracle.f32_to_bf16(ref))


def test_combine_order_and_fma_on_the_device():
    y = torch.tensor([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], dtype=torch.float32, device=DEV)
    assert B.moe_combine(y, torch.ones(3, device=DEV), 3).item() == 0.0
    a = 1.0 + 2.0 ** -12
    y2 = torch.tensor([[-(1.0 + 2.0 ** -11)], [a]], dtype=torch.float32, device=DEV)
    w2 = torch.tensor([1.0, a], dtype=torch.float32, device=DEV)
    assert B.moe_combine(y2, w2, 2).item() == 2.0 ** -24


def test_moe_layer_stage_by_stage():
    """gate and up (input per token), silu*up, down (input per slot), combine:
    the MoE workload's shapes with 16 experts, each stage against the oracle
    fed the device's previous stage."""
    E, H, F, T, k = 16, 2816, 704, 8, 8
    gate = synth.normal_bf16(spec(E * F, H, 0.02, 61))
    up = synth.normal_bf16(spec(E * F, H, 0.02, 62))
    down = synth.normal_bf16(spec(E * H, F, 0.02, 63))
    idx = synth.topk_indices(T, k, E, 64)
    rw = synth.router_weights(T, k, 65)
    x = synth.vector_bf16(H, 66, count=T)
    rg, ru, rd = to_r4(gate), to_r4(up), to_r4(down)
    xd, idd = x.to(DEV), idx.to(DEV)
    yg = B.r4_moe_gemv(rg, E, xd, idd)
    yu = B.r4_moe_gemv(ru, E, xd, idd)
    h = B.moe_silu_mul(yg, yu, out_dtype=torch.bfloat16)
    yd = B.r4_moe_gemv(rd, E, h, idd, x_per_slot=True)
    out = B.moe_combine(yd, rw.to(DEV).reshape(-1), k)
    torch.cuda.synchronize()
    g_ref = oracle.moe_replay(bits_np(gate).reshape(E, F, H), bits_np(x), idx.numpy(), False)
    u_ref = oracle.moe_replay(bits_np(up).reshape(E, F, H), bits_np(x), idx.numpy(), False)
    assert same_f32(yg.cpu().numpy(), g_ref) and same_f32(yu.cpu().numpy(), u_ref)
    h_ref = oracle.f32_to_bf16(oracle.silu_mul(g_ref, u_ref))
    hb = bits_np(h)
    assert np.count_nonzero(hb != h_ref) <= 4    # one-ulp fp32 differences that cross a bf16 rounding
    d_ref = oracle.moe_replay(bits_np(down).reshape(E, H, F), hb, idx.numpy(), True)
    assert same_f32(yd.cpu().numpy(), d_ref)
    assert same_f32(out.cpu().numpy(), oracle.moe_combine(d_ref, rw.numpy(), k))
