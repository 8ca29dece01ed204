"""Pins of the oracle's Huffman comparison codec ("Lossless BF16 weight
compression" page, intro and "Best measured configuration": the exponent
field in canonical Huffman codes, blocks of 64 symbols with 8-bit byte
lengths and a prefix sum, sign and mantissa raw).

- A hand-derived 9-weight case (tests/golden/huff_tiny_9.json): lengths,
  stream bytes, block length and group offsets.
- Code lengths: Kraft's sum is exactly 1 (a full binary tree); the cost
  equals the brute-force optimum over all prefix-code length vectors for
  alphabets of up to 5 symbols; the mean length is within [H, H + 1).
- Canonical codes are prefix-free and consecutive within a length.
- Round trip on random, single-exponent, all-pattern and multi-group
  inputs; a Fibonacci histogram whose tree is deeper than 31 is refused;
  corrupt block lengths or group offsets are rejected."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def weights_from(exps, rng):
    exps = np.asarray(exps, np.uint16)
    return (exps << 7) | rng.integers(0, 128, exps.size).astype(np.uint16) | \
        (rng.integers(0, 2, exps.size).astype(np.uint16) << 15)


def test_hand_derived_case():
    with open(os.path.join(GOLDEN, "huff_tiny_9.json")) as f:
        g = json.load(f)
    e = np.array(g["exponents"], np.uint16)
    i = np.arange(e.size, dtype=np.uint16)
    w = (e << 7) | i | ((i % 2) << 15)
    ln = oracle.huff_lengths(oracle.exponent_counts(w))
    assert {str(k): int(ln[k]) for k in np.nonzero(ln)[0]} == g["lengths"]
    pk = oracle.huff_pack(w, ln)
    assert pk["stream"].tolist() == g["stream"]
    assert pk["block_len"].tolist() == g["block_len"]
    assert pk["group_off"].tolist() == g["group_off"]
    assert np.array_equal(oracle.huff_decode(pk), w)


def test_merge_ties_go_to_the_smaller_id():
    """Equal weights merge the smaller id first (an exponent is its own id,
    merged nodes take 256, 257, ...). Counts 1, 1, 2, 2 for exponents 10,
    11, 12, 13: 10 and 11 make node 256 of weight 2; the nodes of weight 2
    are then 12, 13 and 256, so 12 and 13 make 257, and 256 with 257 the
    root: every length is 2. Taking the larger id first would merge 256
    with 13 and give lengths 3, 3, 1, 2."""
    counts = np.zeros(256, np.uint64)
    counts[[10, 11, 12, 13]] = [1, 1, 2, 2]
    ln = oracle.huff_lengths(counts)
    assert {int(e): int(ln[e]) for e in np.nonzero(ln)[0]} == {10: 2, 11: 2, 12: 2, 13: 2}


def canonical(ln):
    code, c, prev = {}, 0, 0
    for l in range(1, 32):
        for e in range(256):
            if ln[e] == l:
                if prev:
                    c <<= l - prev
                code[e] = (c, l)
                c += 1
                prev = l
    return code


@pytest.mark.parametrize("seed", range(6))
def test_kraft_entropy_and_canonical(seed):
    rng = np.random.default_rng(seed)
    counts = np.zeros(256, np.uint64)
    k = int(rng.integers(2, 60))
    counts[rng.choice(256, k, replace=False)] = rng.integers(1, 10 ** int(rng.integers(1, 7)), k)
    ln = oracle.huff_lengths(counts)
    present = counts > 0
    assert np.all((ln > 0) == present)
    kraft = sum(2.0 ** -int(l) for l in ln[present])
    assert kraft == 1.0
    p = counts[present].astype(np.float64) / counts.sum()
    H = -(p * np.log2(p)).sum()
    mean = (p * ln[present]).sum()
    assert H - 1e-12 <= mean < H + 1
    code = canonical(ln)
    items = sorted(code.items(), key=lambda kv: (kv[1][1], kv[0]))
    for (e1, (c1, l1)), (e2, (c2, l2)) in itertools.combinations(items, 2):
        # prefix-free: no code is the start of another
        a, b = ((c1, l1), (c2, l2)) if l1 <= l2 else ((c2, l2), (c1, l1))
        assert (b[0] >> (b[1] - a[1])) != a[0]
    for (e1, (c1, l1)), (e2, (c2, l2)) in zip(items, items[1:]):
        if l1 == l2:
            assert c2 == c1 + 1 and e2 > e1


@pytest.mark.parametrize("seed", range(8))
def test_optimal_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    k = int(rng.integers(2, 6))
    c = rng.integers(1, 50, k).astype(np.uint64)
    counts = np.zeros(256, np.uint64)
    syms = rng.choice(256, k, replace=False)
    counts[syms] = c
    ln = oracle.huff_lengths(counts)
    best = min(sum(int(ci) * li for ci, li in zip(c, lens))
               for lens in itertools.product(range(1, k + 1), repeat=k)
               if sum(2.0 ** -l for l in lens) <= 1.0)
    assert sum(int(counts[s]) * int(ln[s]) for s in syms) == best


@pytest.mark.parametrize("case", ["normal", "one", "all", "groups"])
def test_round_trip(case):
    rng = np.random.default_rng(7)
    if case == "normal":
        x = (rng.standard_normal(5000) * 0.02).astype(np.float32)
        w = (x.view(np.uint32) >> 16).astype(np.uint16)
    elif case == "one":
        w = weights_from(np.full(200, 126), rng)
    elif case == "all":
        w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    else:   # several groups of 128 blocks and a ragged last block
        x = (rng.standard_normal(3 * 8192 + 77) * 0.02).astype(np.float32)
        w = (x.view(np.uint32) >> 16).astype(np.uint16)
    ln = oracle.huff_lengths(oracle.exponent_counts(w))
    pk = oracle.huff_pack(w, ln)
    assert np.array_equal(oracle.huff_decode(pk), w)
    nb = (w.size + 63) // 64
    assert pk["block_len"].size == nb and int(pk["block_len"].sum()) == pk["stream_bytes"]
    assert pk["group_off"].size == (nb + 127) // 128 + 1
    if case == "one":
        assert ln[126] == 1 and pk["stream_bytes"] == 25   # 200 one-bit codes: 8 + 8 + 8 + 1 bytes
    if case == "all":
        assert np.all(ln == 8)


def test_one_symbol_blocks():
    rng = np.random.default_rng(8)
    w = weights_from(np.full(200, 126), rng)
    pk = oracle.huff_pack(w, oracle.huff_lengths(oracle.exponent_counts(w)))
    # one bit per weight: blocks of 64 bits (8 bytes) and a last block of 8 bits
    assert pk["block_len"].tolist() == [8, 8, 8, 1]
    assert not pk["stream"].any()


def test_deep_tree_is_refused():
    counts = np.zeros(256, np.uint64)
    f = [1, 1]
    while len(f) < 40:
        f.append(f[-1] + f[-2])
    counts[:40] = f
    with pytest.raises(oracle.OracleError) as e:
        oracle.huff_lengths(counts)
    assert e.value.code == -3


def test_corrupt_index_rejected():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(9000) * 0.02).astype(np.float32)
    w = (x.view(np.uint32) >> 16).astype(np.uint16)
    pk = oracle.huff_pack(w, oracle.huff_lengths(oracle.exponent_counts(w)))
    bad = dict(pk, block_len=pk["block_len"].copy())
    bad["block_len"][3] += 1
    with pytest.raises(oracle.OracleError):
        oracle.huff_decode(bad)
    bad = dict(pk, group_off=pk["group_off"].copy())
    bad["group_off"][1] += 1
    with pytest.raises(oracle.OracleError):
        oracle.huff_decode(bad)
