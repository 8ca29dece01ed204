"""GPU parity of the device-side table build and format 2 pack through the C
ABI ("Binade" package page, intro and "How it works": one frequency-rank
table per tensor and the Rice-coded format 2; "Use": packing before load).

- binade_build_table_gpu: the table (n, k, exponent of each rank, rank of
  each exponent, counts) equals the oracle's on every distribution tried:
  one exponent, all 65,536 patterns (256 exponents), tables whose best Rice
  k is 0, 1 and above.
- binade_pack_rice_gpu: sm, unary (padding words zero), remainder, anchor
  and escape-prefix planes byte-identical to the oracle's pack, on shapes
  spanning short rows, ragged row-chunks, one row-chunk, long codes (the
  global-memory path) and full sizes (a Llama-3.2-3B layer's gate and the
  262144 x 256 tensor); the GPU-packed planes decode to the oracle's R4.
- A table that is not the tensor's sets the device status word and writes
  nothing outside the planes."""
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


def weights(case):
    rng = np.random.default_rng(77)
    if case == "all_patterns":
        return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    if case == "one_exponent":
        return ((rng.integers(0, 2, (7, 4160)) << 15) | (125 << 7)
                | rng.integers(0, 128, (7, 4160))).astype(np.uint16)
    rows, cols, sigma, seed, frac, scale = case
    sp = synth.TensorSpec("t", rows, cols, sigma, seed, outlier_frac=frac, outlier_scale=scale)
    return bits_np(synth.normal_bf16(sp))


CASES = ["all_patterns", "one_exponent",
         (1024, 1024, 0.02, 0, 0.0, 1.0), (37, 96, 0.02, 1, 1e-2, 1e4), (5, 4160, 0.02, 2, 5e-3, 1e4),
         (300, 3072, 0.02, 3, 1e-3, 20.0), (4100, 256, 0.015, 6, 0.0, 1.0), (9, 2048, 0.02, 7, 1e-3, 20.0),
         (50, 64, 0.02, 12, 1e-2, 1e3), (70, 32, 0.02, 13, 0.2, 1e6), (45, 96, 0.02, 14, 1e-2, 1e3),
         (23, 1344, 0.015, 11, 1e-3, 20.0), (48, 2080, 1.0, 21, 0.0, 1.0), (48, 2080, 1e-30, 21, 0.01, 1e30),
         (48, 2080, 3e4, 21, 0.0, 1.0), (48, 2080, 0.02, 21, 0.2, 1e6)]


def table_equal(t: B.Table, ref: dict) -> bool:
    n = int(ref["n"])
    rank_of = np.full(256, 0xFFFF, np.uint16)
    rank_of[np.asarray(ref["exp_of_rank"][:n])] = np.arange(n)
    counts = np.zeros(256, np.uint64)
    counts[:n] = np.asarray(ref["count_of_rank"][:n], np.uint64)
    eor = np.zeros(256, np.uint8)
    eor[:n] = np.asarray(ref["exp_of_rank"][:n], np.uint8)
    return (int(t.n) == n and int(t.k) == oracle.rice_k(ref["count_of_rank"], n) and
            np.array_equal(np.frombuffer(bytes(t.exp_of_rank), np.uint8), eor) and
            np.array_equal(np.frombuffer(bytes(t.rank_of_exp), np.uint16), rank_of) and
            np.array_equal(np.frombuffer(bytes(t.count_of_rank), np.uint64), counts))


def planes_equal(p: B.RicePlanes, ref: dict) -> None:
    assert p.unary_bits == ref["unary_bits"] and p.n_esc == ref["n_esc"]
    assert np.array_equal(p.sm.cpu().numpy().reshape(-1), ref["sm"].reshape(-1))
    u = p.unary.cpu().numpy().view(np.uint32)
    nu = ref["unary"].size
    assert np.array_equal(u[:nu], ref["unary"]) and not u[nu:].any()
    if ref["k"] > 0:
        r = p.rem.cpu().numpy().view(np.uint32)
        nr = ref["rem"].size
        assert np.array_equal(r[:nr], ref["rem"]) and not r[nr:].any()
    else:
        assert p.rem is None
    assert np.array_equal(p.anchor.cpu().numpy().view(np.uint64), ref["anchor"])
    assert np.array_equal(p.esc_pre.cpu().numpy().view(np.uint32), ref["esc_pre"])


@pytest.mark.parametrize("case", CASES, ids=lambda c: c if isinstance(c, str) else
                         f"{c[0]}x{c[1]}_s{c[2]:g}")
def test_table_and_pack_equal_oracle(case):
    wn = weights(case)
    say("gpu pack", case if isinstance(case, str) else wn.shape)
    ref_t = oracle.build_table(wn)
    wd = as_bf16(wn).to(DEV)
    t = B.build_table_gpu(wd)
    assert table_equal(t, ref_t)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = B.pack_rice_gpu(wd, t, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    planes_equal(p, oracle.pack_rice(wn, ref_t))
    # the device-packed planes decode to the oracle's R4
    r4 = B.rice_to_r4(p)
    ref = oracle.make_r4(wn, ref_t)
    assert np.array_equal(r4.nib.cpu().numpy().reshape(-1), ref["nib"].reshape(-1))
    assert np.array_equal(bits_np(B.unpack(r4)), wn)


def test_long_codes_at_forced_k0():
    """A table whose k is forced to 0 over exponents spread evenly: about 128
    unary bits per weight, so a row-chunk's bits exceed the LDS stage and
    take the global-memory path."""
    rng = np.random.default_rng(5)
    wn = ((rng.integers(0, 2, (6, 4160)) << 15) | (rng.integers(0, 256, (6, 4160)) << 7)
          | rng.integers(0, 128, (6, 4160))).astype(np.uint16)
    ref_t = oracle.build_table(wn)
    wd = as_bf16(wn).to(DEV)
    t = B.build_table_gpu(wd)
    assert table_equal(t, ref_t)
    t.k = 0
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = B.pack_rice_gpu(wd, t, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = oracle.pack_rice(wn, ref_t, k=0)
    assert ref["unary_bits"] > 100 * wn.size
    planes_equal(p, ref)


def test_full_size():
    for sp in [synth.llama32_3b_stack(1)[4], synth.embedding_64m()]:
        say("gpu pack full size", sp.name, sp.rows, sp.cols)
        w = synth.normal_bf16(sp)
        wn = bits_np(w)
        ref_t = oracle.build_table(wn)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        p = B.pack_rice_gpu(w.to(DEV), status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert table_equal(p.table, ref_t)
        planes_equal(p, oracle.pack_rice(wn, ref_t))


def test_wrong_table_sets_status():
    """The table of another tensor of the same shape: its counts promise
    fewer unary bits than these weights need, and one exponent is missing."""
    a = weights((64, 2080, 0.02, 40, 0.0, 1.0))
    b = weights((64, 2080, 2.0, 41, 0.0, 1.0))
    t_a = B.build_table(as_bf16(a))
    guard = 1 << 20
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    wd = as_bf16(b).to(DEV)
    sz = B.sizes_of(t_a, *b.shape)
    # planes inside one buffer with a guard band after the unary plane
    p = B.pack_rice_gpu(as_bf16(a).to(DEV), t_a)   # valid planes of a, for their layout
    big = torch.full((int(sz.unary_words) + guard,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    p.unary = big[: int(sz.unary_words)]
    d = p.desc()
    ws = torch.empty(int(B.lib().binade_pack_gpu_workspace_bytes(*b.shape)), dtype=torch.uint8,
                     device=DEV)
    import ctypes
    rc = B.lib().binade_pack_rice_gpu(ctypes.c_void_p(wd.data_ptr()), b.shape[0], b.shape[1],
                                      ctypes.byref(t_a), ctypes.byref(d),
                                      ctypes.c_void_p(ws.data_ptr()),
                                      ctypes.c_void_p(status.data_ptr()),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == B.OK
    assert int(status.item()) & B.DEV_CORRUPT_STREAM
    assert torch.all(big[int(sz.unary_words):] == 0x5A5A5A5A)
