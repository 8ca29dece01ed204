"""GPU parity of the Huffman comparison decoder through the C ABI ("Lossless
BF16 weight compression" page, "Best measured configuration": canonical
Huffman codes of the exponent field in blocks of 64 symbols, 8-bit block
lengths and a prefix sum; sign and mantissa raw).

binade_huff_decode's bf16 output equals the original weights and the
oracle's decode bit for bit on: LLM-like tensors (several groups, a ragged
last block), every bf16 pattern, one exponent (one-bit codes), codes longer
than the 11-bit table (the canonical walk), groups larger than the LDS stage
(uniform exponents, 8-bit codes), tiny tensors, and the 262144 x 256 tensor;
a corrupt block length or group offset sets the status word."""
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
    rng = np.random.default_rng(91)
    if case == "llm":
        sp = synth.TensorSpec("t", 300, 3072, 0.02, 3, outlier_frac=1e-3, outlier_scale=20.0)
        return bits_np(synth.normal_bf16(sp)).reshape(-1)
    if case == "ragged":
        sp = synth.TensorSpec("t", 7, 3001, 0.015, 4)
        return bits_np(synth.normal_bf16(sp)).reshape(-1)
    if case == "all_patterns":
        return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if case == "one_exponent":
        return ((rng.integers(0, 2, 20000) << 15) | (125 << 7) | rng.integers(0, 128, 20000)).astype(np.uint16)
    if case == "long_codes":   # geometric exponent counts: lengths well past 11 bits
        e = np.minimum(rng.geometric(0.45, 200_000) + 100, 140)
        return ((rng.integers(0, 2, e.size) << 15) | (e << 7) | rng.integers(0, 128, e.size)).astype(np.uint16)
    if case == "uniform":      # 8-bit codes: a group's bytes exceed the LDS stage
        return ((rng.integers(0, 256, 50_000) << 7) | rng.integers(0, 128, 50_000)).astype(np.uint16)
    if case == "tiny":
        return (rng.standard_normal(37).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(case)


@pytest.mark.parametrize("case", ["llm", "ragged", "all_patterns", "one_exponent", "long_codes",
                                  "uniform", "tiny"])
def test_huff_decode_is_bit_exact(case):
    wn = weights(case)
    say("huffman", case, wn.size)
    p = B.pack_huff(as_bf16(wn))
    if case == "long_codes":
        assert max(p.len) > 11
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = B.huff_decode(p.to(DEV), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = bits_np(out)
    assert np.array_equal(got, wn)
    pk = {"n": p.n, "len": np.frombuffer(p.len, np.uint8), "sm": p.sm.numpy(),
          "stream": p.stream.numpy()[: p.stream_bytes], "stream_bytes": p.stream_bytes,
          "block_len": p.block_len.numpy(), "group_off": p.group_off.numpy().view(np.uint64)}
    assert np.array_equal(got, oracle.huff_decode(pk))


def test_huff_decode_full_size():
    sp = synth.embedding_64m()
    say("huffman full size", sp.rows, sp.cols)
    w = synth.normal_bf16(sp)
    p = B.pack_huff(w)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = B.huff_decode(p.to(DEV), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out.cpu().view(torch.int16), w.reshape(-1).view(torch.int16))


def test_huff_corrupt_index_sets_status():
    wn = weights("llm")[:40_000]
    p = B.pack_huff(as_bf16(wn))

    def run(planes):
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        B.huff_decode(planes.to(DEV), status=status)
        torch.cuda.synchronize()
        return int(status.item())

    assert run(p) == 0
    bad = B.HuffPlanes(**{**p.__dict__, "block_len": p.block_len.clone()})
    bad.block_len[5] += 1
    assert run(bad) & B.DEV_CORRUPT_STREAM
    bad = B.HuffPlanes(**{**p.__dict__, "group_off": p.group_off.clone()})
    bad.group_off[2] += 3
    assert run(bad) & B.DEV_CORRUPT_STREAM
