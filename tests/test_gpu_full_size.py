"""GPU parity at the benchmark's full sizes, in the launch configurations the
benchmark times (batched decode of up to 16 tensors per launch, batched
GEMV of up to 16, the prompt GEMM with its workspace).

Whole-output checks need no oracle: R4 equals the oracle's R4 of the
weights bit for bit (the oracle's conversion is plain C and fast), the
unpacked bits equal the weights, and every product equals its bf16-weight
twin bit for bit. Against the oracle's products, sampled outputs: rows of
the matvec and entries of the GEMM replayed in their fixed fp32 orders
(bit-exact), and both within 1e-2 of the fp64 sum (relative to
sum |w x|)."""
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


def check_r4_against_oracle(name, wb: np.ndarray, r4) -> None:
    ref = oracle.make_r4(wb, oracle.build_table(wb))
    assert bytes(bytearray(r4.lut)) == bytes(ref["lut"]), name
    assert r4.n_esc == ref["n_esc"], name
    assert np.array_equal(r4.nib.cpu().numpy().reshape(-1), ref["nib"].reshape(-1)), name
    if r4.n_esc:
        assert np.array_equal(r4.esc[: r4.n_esc].cpu().numpy().view(np.uint32), ref["esc"]), name
    assert np.array_equal(r4.esc_pre.cpu().numpy().view(np.uint32), ref["esc_pre"]), name


def decode_and_gemv(specs, sample_rows=48, seed=0):
    """Decode the tensors in one batched call (16 per launch), multiply each by
    its own vector in one batched GEMV call (16 per launch), and check both
    at full size."""
    ws = [synth.normal_bf16(sp) for sp in specs]
    planes = [B.pack_rice(w).to(DEV) for w in ws]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("decode", [f"{sp.name} {sp.rows}x{sp.cols}" for sp in specs])
    outs = B.rice_to_r4_batch(planes, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for sp, w, o in zip(specs, ws, outs):
        wb = bits_np(w)
        check_r4_against_oracle(sp.name, wb, o)
        assert torch.equal(B.unpack(o).cpu().view(torch.int16), w.view(torch.int16)), sp.name
    xs = [synth.vector_bf16(sp.cols, 500 + i).to(DEV) for i, sp in enumerate(specs)]
    say("gemv batch")
    ys = B.r4_gemv_batch(outs, xs)
    yt = B.bf16_gemv_batch([w.to(DEV) for w in ws], xs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for sp, w, x, y, t in zip(specs, ws, xs, ys, yt):
        assert torch.equal(y.view(torch.int32), t.view(torch.int32)), sp.name
        rows = np.sort(rng.choice(sp.rows, size=min(sample_rows, sp.rows), replace=False))
        wb = bits_np(w)[rows]
        xb = bits_np(x.cpu())
        yr = y.cpu().numpy()[rows]
        assert same_f32(yr, oracle.gemv_replay(wb, xb)), sp.name
        ref = oracle.gemv_f64(wb, xb)
        wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.abs(yr.astype(np.float64) - ref) <= 1e-2 * (np.abs(wf) @ np.abs(xf))), sp.name


def test_single_1024_tensor_full_size():
    """One 1024 x 1024 tensor, N(0, 0.02), 16 outliers x50."""
    decode_and_gemv(synth.single_1024(), sample_rows=1024)


def test_llama_layer_full_size():
    """One layer of the Llama-3.2-3B-shaped stack: q, k, v, o, gate, up,
    down at their full shapes, in one batched decode launch and one batched
    GEMV launch."""
    decode_and_gemv(synth.llama32_3b_stack(1), seed=1)


def test_12b_ffn_full_size():
    """The 12B-class FFN shapes 15360 x 3840 (gate, up) and 3840 x 15360."""
    decode_and_gemv(synth.gemma_12b_ffn(), seed=2)


def test_64m_embedding_decode_full_size():
    """The 262144 x 256 bulk-decode tensor (jobs of 16 short rows)."""
    sp = synth.embedding_64m()
    w = synth.normal_bf16(sp)
    planes = B.pack_rice(w).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("decode", sp.name)
    r4 = B.rice_to_r4(planes, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_r4_against_oracle(sp.name, bits_np(w), r4)
    assert torch.equal(B.unpack(r4).cpu().view(torch.int16), w.view(torch.int16))


@pytest.mark.parametrize("nk", [(15360, 3840), (3840, 15360)], ids=["15360x3840", "3840x15360"])
def test_prompt_gemm_full_size(nk):
    """Y = X W^T for M = 16, 32, 128, 2048 on the full FFN shapes: bit-equal
    to the bf16 twin everywhere, rows independent of M, sampled entries
    bit-equal to the oracle's replay and within the fp64 bound."""
    N, K = nk
    w = synth.normal_bf16(synth.TensorSpec("w", N, K, 0.015, 2000 + N))
    r4 = B.rice_to_r4(B.pack_rice(w).to(DEV))
    wd = w.to(DEV)
    X = synth.vector_bf16(K, 2200 + N, count=2048)
    Xd = X.to(DEV)
    rng = np.random.default_rng(N)
    wb_all = bits_np(w)
    first = None
    for m in (2048, 128, 32, 16):
        say("gemm", N, K, "M =", m)
        xm = Xd[:m].contiguous()
        y = B.r4_gemm(r4, xm)
        t = B.bf16_gemm(wd, xm)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), t.view(torch.int32)), m
        if first is None:
            first = y.cpu()
        else:
            assert torch.equal(y.cpu().view(torch.int32), first[:m].view(torch.int32)), m
        rows = np.sort(rng.choice(m, size=min(8, m), replace=False))
        cols = np.sort(rng.choice(N, size=64, replace=False))
        wb = wb_all[cols]
        xb = bits_np(X[rows])
        ref = oracle.gemm_f64(wb, xb)
        scale = oracle.gemm_f64(wb & 0x7FFF, xb & 0x7FFF)
        got32 = y.cpu().numpy()[np.ix_(rows, cols)]
        mi, ni = np.meshgrid(rows, cols, indexing="ij")
        rep = oracle.gemm_replay_entries(wb_all, bits_np(X[:m]), mi.reshape(-1), ni.reshape(-1))
        assert same_f32(got32.reshape(-1), rep), m
        got = got32.astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1e-2 * scale), m
