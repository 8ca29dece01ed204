"""GPU parity of format 1 -> R4 ("Binade" package page, "How it works": at
load a GPU kernel turns either file format into R4) through the C ABI:
binade_f1_to_r4's nibbles, side list and table equal the oracle's R4 of the
same weights byte for byte, and unpack back to the original bits, on shapes
spanning short rows, ragged chunks, every tile width (0 to 8), every bf16
pattern, and at full size one Llama-3.2-3B layer and the 262144 x 256
tensor; corrupt planes set the device status word."""
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


def as_bf16(wn: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(wn).view(np.int16)).view(torch.bfloat16)


def check_against_oracle(name, wn, r4):
    ref = oracle.make_r4(wn, oracle.build_table(wn))
    assert bytes(bytearray(r4.lut)) == bytes(ref["lut"]), name
    assert r4.n_esc == ref["n_esc"], name
    assert np.array_equal(r4.nib.cpu().numpy().reshape(-1), ref["nib"].reshape(-1)), name
    if r4.n_esc:
        assert np.array_equal(r4.esc[: r4.n_esc].cpu().numpy().view(np.uint32), ref["esc"]), name
    assert np.array_equal(r4.esc_pre.cpu().numpy().view(np.uint32), ref["esc_pre"]), name
    assert np.array_equal(bits_np(B.unpack(r4)), wn), name


def weights(case):
    rng = np.random.default_rng(31)
    if case == "all_patterns":
        return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    if case == "one_exponent":
        return ((rng.integers(0, 2, (7, 4160)) << 15) | (125 << 7)
                | rng.integers(0, 128, (7, 4160))).astype(np.uint16)
    if case == "two_exponents":   # width-2 tiles over a 2-entry table (every code checked)
        return ((rng.integers(0, 2, (5, 2080)) << 15) | (rng.integers(120, 122, (5, 2080)) << 7)
                | rng.integers(0, 128, (5, 2080))).astype(np.uint16)
    if case == "wide":
        return ((rng.integers(0, 2, (9, 2080)) << 15) | (rng.integers(20, 220, (9, 2080)) << 7)
                | rng.integers(0, 128, (9, 2080))).astype(np.uint16)
    rows, cols, sigma, seed, frac, scale = case
    spec = synth.TensorSpec("t", rows, cols, sigma, seed, outlier_frac=frac, outlier_scale=scale)
    return bits_np(synth.normal_bf16(spec))


CASES = ["all_patterns", "one_exponent", "two_exponents", "wide",
         (1024, 1024, 0.02, 0, 0.0, 1.0), (37, 96, 0.02, 1, 1e-2, 1e4), (5, 4160, 0.02, 2, 5e-3, 1e4),
         (300, 3072, 0.02, 3, 1e-3, 20.0), (64, 8192, 0.02, 4, 1e-3, 20.0),
         (19, 15360, 0.015, 5, 0.0, 1.0), (4100, 256, 0.015, 6, 0.0, 1.0), (50, 64, 0.02, 12, 1e-2, 1e3),
         (130, 128, 0.02, 10, 5e-3, 1e3), (11, 6144, 0.02, 9, 1e-3, 20.0), (33, 1344, 0.015, 11, 1e-3, 20.0),
         (70, 32, 0.02, 13, 0.2, 1e6)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c if isinstance(c, str) else f"{c[0]}x{c[1]}")
def test_f1_to_r4_equals_oracle_r4(case):
    wn = weights(case)
    say("format1", case if isinstance(case, str) else wn.shape)
    planes = B.pack_f1(as_bf16(wn)).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    r4 = B.f1_to_r4(planes, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_against_oracle(str(case), wn, r4)


def test_f1_and_rice_give_the_same_r4():
    wn = weights((300, 3072, 0.02, 3, 1e-3, 20.0))
    w = as_bf16(wn)
    a = B.f1_to_r4(B.pack_f1(w).to(DEV))
    b = B.rice_to_r4(B.pack_rice(w).to(DEV))
    torch.cuda.synchronize()
    assert a.lut == b.lut and a.n_esc == b.n_esc
    assert torch.equal(a.nib, b.nib)
    assert torch.equal(a.esc[: a.n_esc], b.esc[: b.n_esc])


def test_f1_full_size():
    """One Llama-3.2-3B layer (q, k, v, o, gate, up, down) and the 262144 x
    256 tensor, whole outputs against the oracle's R4."""
    specs = synth.llama32_3b_stack(1) + [synth.embedding_64m()]
    for sp in specs:
        say("format1 full size", sp.name, sp.rows, sp.cols)
        w = synth.normal_bf16(sp)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        r4 = B.f1_to_r4(B.pack_f1(w).to(DEV), status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, sp.name
        check_against_oracle(sp.name, bits_np(w), r4)


def test_f1_corrupt_planes_set_status():
    wn = weights((6, 4160, 0.02, 8, 1e-2, 1e3))
    good = B.pack_f1(as_bf16(wn))

    def run(planes):
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        B.f1_to_r4(planes.to(DEV), status=status)
        torch.cuda.synchronize()
        return int(status.item())

    assert run(good) == 0
    bad = B.F1Planes(**{**good.__dict__, "width": good.width.clone()})
    bad.width[5] = 9                                   # no such width
    assert run(bad) & B.DEV_CORRUPT_STREAM
    bad = B.F1Planes(**{**good.__dict__, "anchor": good.anchor.clone()})
    bad.anchor[3] += 3                                 # a chunk's codes start elsewhere
    assert run(bad) & B.DEV_CORRUPT_STREAM
    bad = B.F1Planes(**{**good.__dict__, "esc_rank": good.esc_rank.clone()})
    bad.esc_rank[0] = 1                                # an escape below its escape code
    assert run(bad) & B.DEV_CORRUPT_STREAM
    bad = B.F1Planes(**{**good.__dict__, "esc_pre": good.esc_pre.clone()})
    bad.esc_pre[-1] += 1                               # R4's escape total disagrees
    assert run(bad) & B.DEV_CORRUPT_ESC


def test_f1_self_consistent_planes_outside_the_format_set_status():
    """Planes whose counts, anchors and prefixes all agree but which break
    the format: a width of 9 (128 codes of 9 zero bits) and an escape whose
    listed rank is below its escape code (width 1, rank 0 listed)."""
    exps = np.full(128, 120, np.uint16)
    exps[7] = 121
    wn = ((exps << 7) | np.arange(128, dtype=np.uint16)).reshape(1, 128)
    good = B.pack_f1(as_bf16(wn))
    assert good.width.tolist() == [1] and good.n_f1esc == 1

    def run(planes):
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        B.f1_to_r4(planes.to(DEV), status=status)
        torch.cuda.synchronize()
        return int(status.item())

    assert run(good) == 0
    wide = B.F1Planes(**{**good.__dict__, "width": torch.tensor([9], dtype=torch.uint8),
                         "codes": torch.zeros(38, dtype=good.codes.dtype), "code_bits": 128 * 9,
                         "n_f1esc": 0, "anchor": torch.tensor([0, 1152], dtype=good.anchor.dtype),
                         "f1_pre": torch.zeros(2, dtype=good.f1_pre.dtype)})
    assert run(wide) & B.DEV_CORRUPT_STREAM
    low = B.F1Planes(**{**good.__dict__, "esc_rank": torch.zeros_like(good.esc_rank)})
    assert run(low) & B.DEV_CORRUPT_STREAM
