"""Pins of the oracle's format 1 ("Binade" package page, "How it works": a
fixed code width per 128-weight tile with escapes, about 11.27 bits per
weight): a hand-derived tensor (tests/golden/f1_tiny.json), the round trip
back to the original bits over every bf16 pattern and several exponent
spreads, the code-bit count from the widths, the widths' optimality against
every other width of each tile, corrupt planes, and bits per weight near the
pages' figure on LLM-like tensors."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from decode_gemv_tensor_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_bits():
    with open(os.path.join(GOLDEN, "f1_tiny.json")) as f:
        g = json.load(f)
    exps = [120] * 100 + [121] * 20 + [119] * 6 + [122] * 2 + \
           [120] * 10 + [121] * 5 + [119] * 5 + [122] * 8 + [130] * 4
    w = np.array([(e << 7) | (c % 128) for c, e in enumerate(exps)], np.uint16).reshape(1, 160)
    return g, w


def test_hand_derived_format1():
    g, w = _golden_bits()
    tab = oracle.build_table(w)
    assert list(tab["exp_of_rank"][: tab["n"]]) == g["exp_of_rank"]
    pk = oracle.pack_f1(w, tab)
    assert pk["width"].reshape(-1).tolist() == g["width"]
    assert pk["code_bits"] == g["code_bits"]
    words = pk["codes"]
    ones = [p for p in range(pk["code_bits"]) if (int(words[p >> 5]) >> (p & 31)) & 1]
    assert ones == g["code_one_bits"]
    assert pk["esc"].tolist() == g["esc"]
    assert pk["anchor"].tolist() == g["anchor"]
    assert pk["f1_pre"].tolist() == g["f1_pre"]
    assert pk["esc_pre"].tolist() == g["esc_pre"]
    assert np.array_equal(oracle.f1_decode(pk), w)


def test_width_ties_go_to_the_smaller_width():
    """A 128-weight tile with 8 ranks of 1, 8 of 2 and 112 of 0 costs
    128 * 1 + 8 * 16 = 256 bits at width 1 (escape code 1: the 16 ranks
    escape) and 128 * 2 = 256 bits at width 2 (escape code 3: none do);
    width 3 costs 384. The tie goes to width 1: 128 code bits, all ones at
    the 16 escapes, and the escape list holds their ranks in order."""
    exps = np.full(128, 120, np.uint16)
    exps[5:13] = 121          # rank 1 (count 8, the smaller exponent of the tie)
    exps[40:48] = 125         # rank 2 (count 8)
    w = ((exps << 7) | (np.arange(128, dtype=np.uint16) % 128)).reshape(1, 128)
    tab = oracle.build_table(w)
    assert list(tab["exp_of_rank"][: tab["n"]]) == [120, 121, 125]
    pk = oracle.pack_f1(w, tab)
    assert pk["width"].reshape(-1).tolist() == [1]
    assert pk["code_bits"] == 128
    ones = [p for p in range(128) if (int(pk["codes"][p >> 5]) >> (p & 31)) & 1]
    assert ones == list(range(5, 13)) + list(range(40, 48))
    assert pk["esc"].tolist() == [1] * 8 + [2] * 8
    assert np.array_equal(oracle.f1_decode(pk), w)


def _ranks(w, tab):
    rank_of = {int(e): r for r, e in enumerate(tab["exp_of_rank"][: tab["n"]])}
    return np.vectorize(lambda b: rank_of[(int(b) >> 7) & 0xFF])(w)


def _check_widths(w, tab, pk):
    """Every tile's width has the fewest bits (ties to the smaller), counted
    from the ranks; the code plane holds exactly the widths' bits and the
    escape list exactly the ranks at or above each tile's escape code."""
    ranks = _ranks(w, tab)
    rows, cols = w.shape
    total_bits = 0
    n_esc = 0
    for r in range(rows):
        for t in range((cols + 127) // 128):
            rk = ranks[r, 128 * t: 128 * t + 128]
            wt = int(pk["width"][r, t])
            cost = {}
            for cand in range(9):
                if cand == 0:
                    if np.all(rk == 0):
                        cost[0] = 0
                    continue
                cost[cand] = len(rk) * cand + 8 * int(np.sum(rk >= (1 << cand) - 1))
            best = min(cost.values())
            assert cost[wt] == best and all(c > best for k, c in cost.items() if k < wt)
            total_bits += len(rk) * wt
            if wt:
                n_esc += int(np.sum(rk >= (1 << wt) - 1))
    assert pk["code_bits"] == total_bits
    assert pk["n_f1esc"] == n_esc


@pytest.mark.parametrize("case", ["all_patterns", "llm", "one_exponent", "wide", "short_rows"])
def test_round_trip_and_widths(case):
    rng = np.random.default_rng(5)
    if case == "all_patterns":
        w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    elif case == "llm":
        w = synth.normal_bf16(synth.TensorSpec("t", 40, 3072, 0.02, 3, outlier_frac=1e-3,
                                               outlier_scale=20.0)).view(torch.int16).numpy().view(np.uint16)
    elif case == "one_exponent":   # every rank 0: width-0 tiles, no codes at all
        w = ((rng.integers(0, 2, (7, 4160)) << 15) | (125 << 7) | rng.integers(0, 128, (7, 4160))).astype(np.uint16)
    elif case == "wide":          # exponents spread over 200 values: widths up to 8
        w = ((rng.integers(0, 2, (9, 2080)) << 15) | (rng.integers(20, 220, (9, 2080)) << 7)
             | rng.integers(0, 128, (9, 2080))).astype(np.uint16)
    else:                          # rows shorter than a tile and than a chunk
        w = synth.normal_bf16(synth.TensorSpec("t", 300, 96, 0.02, 4)).view(torch.int16).numpy().view(np.uint16)
    tab = oracle.build_table(w)
    pk = oracle.pack_f1(w, tab)
    assert np.array_equal(oracle.f1_decode(pk), w)
    _check_widths(w, tab, pk)
    if case == "one_exponent":
        assert pk["code_bits"] == 0 and pk["width"].max() == 0


def test_corrupt_planes_are_rejected():
    w = synth.normal_bf16(synth.TensorSpec("t", 6, 4160, 0.02, 8, outlier_frac=1e-2,
                                           outlier_scale=1e3)).view(torch.int16).numpy().view(np.uint16)
    tab = oracle.build_table(w)
    good = oracle.pack_f1(w, tab)
    bad = dict(good, width=good["width"].copy())
    bad["width"][2, 5] = 9 if bad["width"][2, 5] != 9 else 8
    with pytest.raises(oracle.OracleError):
        oracle.f1_decode(bad)
    bad = dict(good, esc=good["esc"][:-1].copy(), n_f1esc=good["n_f1esc"] - 1)
    with pytest.raises(oracle.OracleError):
        oracle.f1_decode(bad)
    bad = dict(good, anchor=good["anchor"].copy())
    bad["anchor"][3] += 1
    with pytest.raises(oracle.OracleError):
        oracle.f1_decode(bad)


def test_self_consistent_streams_outside_the_format_are_rejected():
    """Planes whose counts, anchors and prefixes all agree but which break
    the format: a width above 8 (128 codes of 9 zero bits) and an escape
    whose listed rank is below its escape code (width 1, escape rank 0)."""
    exps = np.full(128, 120, np.uint16)
    exps[7] = 121
    w = ((exps << 7) | np.arange(128, dtype=np.uint16)).reshape(1, 128)
    tab = oracle.build_table(w)
    good = oracle.pack_f1(w, tab)
    assert good["width"].reshape(-1).tolist() == [1] and good["n_f1esc"] == 1
    wide = dict(good, width=np.array([[9]], np.uint8), codes=np.zeros(36, np.uint32),
                code_bits=128 * 9, esc=np.zeros(0, np.uint8), n_f1esc=0,
                anchor=np.array([0, 1152], np.uint64), f1_pre=np.array([0, 0], np.uint32))
    with pytest.raises(oracle.OracleError):
        oracle.f1_decode(wide)
    low = dict(good, esc=np.array([0], np.uint8))   # code 1 at column 7 lists rank 0
    with pytest.raises(oracle.OracleError):
        oracle.f1_decode(low)


def test_bits_per_weight_near_the_pages_figure():
    """About 11.27 bits per weight on the pages' models; LLM-like synthetic
    tensors land within 0.15 of it (the index adds 0.06 bits per weight)."""
    for sp in synth.llama32_3b_stack(1)[:4]:
        w = synth.normal_bf16(sp).view(torch.int16).numpy().view(np.uint16)
        pk = oracle.pack_f1(w, oracle.build_table(w))
        n = w.size
        nch = pk["anchor"].size
        bits = 8 * n + pk["code_bits"] + 8 * pk["n_f1esc"] + 8 * pk["width"].size + 128 * nch
        assert abs(bits / n - 11.27) < 0.15, (sp.name, bits / n)
