"""CPU tests of libbinade's host half and of the ABI surface: the library
loads, exports every symbol include/binade.h declares, its table and format 2
pack are byte-identical to the oracle's, and bad arguments give the declared
status codes. No device call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from decode_gemv_tensor_amd import binade as B
from decode_gemv_tensor_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "binade.h")).read()
    pat = r"^(?:int32_t|int64_t|const char \*)\s*(binade_\w+)\("
    return sorted(set(re.findall(pat, text, flags=re.M)))


def test_library_exports_every_declared_function():
    declared = _header_functions()
    assert len(declared) >= 13
    L = B.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(B.EXPORTS) == declared


def test_gemm_workspace_bytes_policy():
    """Host-only sizing: partials are S*M*N fp32 for shapes whose slices run
    in separate blocks (S = min(8, ceil(K/1024)) slices), 0 otherwise."""
    # M <= 32 streams each slice separately when its X columns fit in LDS
    assert B.gemm_workspace_bytes(16, 3840, 15360) == 8 * 16 * 3840 * 4
    assert B.gemm_workspace_bytes(32, 64, 15360) == 8 * 32 * 64 * 4
    assert B.gemm_workspace_bytes(16, 15360, 3840) == 4 * 16 * 15360 * 4
    # ... but not with one slice, without a full super-block, or when a
    # slice's X columns would not fit in LDS
    assert B.gemm_workspace_bytes(16, 512, 1024) == 0
    assert B.gemm_workspace_bytes(16, 512, 96) == 0
    assert B.gemm_workspace_bytes(16, 64, 131072) == 0
    # few tiles, K = 15360 -> 8 slices
    assert B.gemm_workspace_bytes(128, 3840, 15360) == 8 * 128 * 3840 * 4
    # K = 3840 -> 4 slices
    assert B.gemm_workspace_bytes(128, 15360, 3840) == 4 * 128 * 15360 * 4
    # one slice: nothing to split
    assert B.gemm_workspace_bytes(200, 512, 1024) == 0
    # large M: enough tiles, and partials would cost more than they save
    assert B.gemm_workspace_bytes(2048, 15360, 3840) == 0
    for bad in ((0, 64, 64), (64, 0, 64), (64, 64, 0), (64, 64, 48), (-1, 64, 64)):
        assert B.gemm_workspace_bytes(*bad) == 0


def test_struct_layouts_match_header_sizes():
    # natural alignment on x86-64 / gfx950: the ctypes mirrors must agree
    assert ctypes.sizeof(B.Table) == 8 + 256 + 512 + 2048
    assert ctypes.sizeof(B.RiceDesc) == 352
    assert ctypes.sizeof(B.R4Desc) == 72
    assert ctypes.sizeof(B.Sizes) == 56


def _tensor(rows, cols, sigma=0.02, seed=0, frac=1e-3, scale=20.0):
    spec = synth.TensorSpec("t", rows, cols, sigma, seed, outlier_frac=frac,
                            outlier_scale=scale)
    return synth.normal_bf16(spec)


def _np(t):
    return synth.bits(t).numpy().view(np.uint16)


@pytest.mark.parametrize("shape,sigma,frac,scale", [
    ((1, 32), 0.02, 0.0, 1.0), ((64, 1024), 0.02, 1e-3, 20.0),
    ((3, 2080), 0.02, 5e-3, 1e4), ((16, 4096 + 64), 1.0, 0.0, 1.0),
    ((8, 256), 1e-30, 0.01, 1e30)])
def test_table_and_pack_match_oracle_bytes(shape, sigma, frac, scale):
    w = _tensor(*shape, sigma=sigma, seed=shape[1], frac=frac, scale=scale)
    wn = _np(w)
    t = B.build_table(w)
    to = oracle.build_table(wn)
    assert t.n == to["n"]
    assert bytes(t.exp_of_rank)[: t.n] == bytes(to["exp_of_rank"][: t.n])
    assert list(t.count_of_rank)[: t.n] == to["count_of_rank"][: t.n].tolist()
    assert t.k == oracle.rice_k(to["count_of_rank"], to["n"])
    for e in range(256):
        r = t.rank_of_exp[e]
        if r != 0xFFFF:
            assert t.exp_of_rank[r] == e
    p = B.pack_rice(w, t)
    po = oracle.pack_rice(wn, to)
    assert p.unary_bits == po["unary_bits"]
    assert p.n_esc == po["n_esc"]
    assert np.array_equal(p.sm.numpy(), po["sm"])
    nu = po["unary"].size
    assert np.array_equal(p.unary.numpy().view(np.uint32)[:nu], po["unary"])
    assert not p.unary.numpy()[nu:].any()          # padding words are zero
    if p.k:
        nr = po["rem"].size
        assert np.array_equal(p.rem.numpy().view(np.uint32)[:nr], po["rem"])
        assert not p.rem.numpy()[nr:].any()
    assert np.array_equal(p.anchor.numpy().view(np.uint64), po["anchor"])
    assert np.array_equal(p.esc_pre.numpy().view(np.uint32), po["esc_pre"])
    s = B.sizes_of(t, *shape)
    assert s.unary_bits == p.unary_bits and s.n_esc == p.n_esc


def test_exhaustive_patterns_pack_matches_oracle():
    w = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).reshape(64, 1024)
    wn = _np(w)
    p = B.pack_rice(w)
    po = oracle.pack_rice(wn, oracle.build_table(wn))
    assert p.table.n == 256 and p.k == po["k"]
    assert np.array_equal(p.unary.numpy().view(np.uint32)[: po["unary"].size], po["unary"])
    assert np.array_equal(p.anchor.numpy().view(np.uint64), po["anchor"])


def test_bits_per_weight_matches_pages_order_of_magnitude():
    """"Binade" package page, "How it works": format 2 ~10.75 bits/weight.
    Synthetic N(0, 0.02) weights land within a few hundredths of that."""
    p = B.pack_rice(_tensor(256, 3072, seed=3))
    assert 10.6 < p.bits_per_weight() < 10.85


def test_status_codes():
    L = B.lib()
    t = B.Table()
    assert L.binade_build_table(None, 10, ctypes.byref(t)) == B.EINVAL
    w = torch.zeros(4, dtype=torch.bfloat16)
    assert L.binade_build_table(ctypes.c_void_p(w.data_ptr()), 0, ctypes.byref(t)) == B.EINVAL
    assert L.binade_status_str(B.EUNSUPPORTED) == b"unsupported shape or alignment"
    # table from another tensor: sizes refuse
    t = B.build_table(_tensor(4, 64))
    s = B.Sizes()
    assert L.binade_sizes_of(ctypes.byref(t), 4, 32, ctypes.byref(s)) == B.EINVAL
    # weights with an exponent the table does not hold
    w1 = _tensor(2, 64, sigma=0.02)
    w2 = _tensor(2, 64, sigma=100.0)
    with pytest.raises(B.BinadeError) as e:
        B.pack_rice(w2, B.build_table(w1))
    assert e.value.code in (B.EINVAL,)
    # too small a unary plane
    p = B.pack_rice(w1)
    d = p.desc()
    d.unary_words = 1
    assert L.binade_pack_rice(ctypes.c_void_p(w1.data_ptr()), 2, 64,
                              ctypes.byref(p.table), ctypes.byref(d)) == B.ENOSPACE


def test_device_entry_points_validate_before_touching_the_gpu():
    """Argument checks run on the host and return before any HIP call."""
    L = B.lib()
    d = B.R4Desc()
    d.rows, d.cols = 4, 48            # cols % 32 != 0
    assert L.binade_r4_gemv(ctypes.byref(d), None, None, 0, None) == B.EUNSUPPORTED
    d.cols = -1
    assert L.binade_r4_gemv(ctypes.byref(d), None, None, 0, None) == B.EINVAL
    d.cols = 64
    assert L.binade_r4_gemv(ctypes.byref(d), None, None, 0, None) == B.EINVAL
    assert L.binade_r4_gemv(None, None, None, 0, None) == B.EINVAL
    assert L.binade_bf16_gemv(None, 4, 40, None, None, 0, None) == B.EUNSUPPORTED
    assert L.binade_unpack(None, None, None) == B.EINVAL
    r = B.RiceDesc()
    assert L.binade_rice_to_r4(ctypes.byref(r), ctypes.byref(d), None, None) == B.EINVAL
    # zero rows: a valid no-op that launches nothing
    d.rows, d.cols = 0, 64
    assert L.binade_r4_gemv(ctypes.byref(d), None, None, 0, None) == B.OK


@pytest.mark.parametrize("case", ["llm", "all_patterns", "one_exponent", "wide", "short_rows", "ragged"])
def test_format1_pack_matches_oracle_bytes(case):
    """binade_pack_f1 (host C++) against the oracle's format 1 pack, plane by
    plane, on the spreads the oracle's pins cover."""
    rng = np.random.default_rng(21)
    if case == "llm":
        wn = _np(_tensor(40, 3072, sigma=0.02, seed=3, frac=1e-3, scale=20.0))
    elif case == "all_patterns":
        wn = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    elif case == "one_exponent":
        wn = ((rng.integers(0, 2, (7, 4160)) << 15) | (125 << 7) | rng.integers(0, 128, (7, 4160))).astype(np.uint16)
    elif case == "wide":
        wn = ((rng.integers(0, 2, (9, 2080)) << 15) | (rng.integers(20, 220, (9, 2080)) << 7)
              | rng.integers(0, 128, (9, 2080))).astype(np.uint16)
    elif case == "short_rows":
        wn = _np(_tensor(300, 96, sigma=0.02, seed=4, frac=0.0, scale=1.0))
    else:   # columns not a multiple of 32 (host packing takes any width)
        wn = _np(_tensor(5, 1000, sigma=0.02, seed=5, frac=1e-2, scale=1e3))
    w = torch.from_numpy(wn.view(np.int16)).view(torch.bfloat16)
    t = B.build_table(w)
    p = B.pack_f1(w, t)
    po = oracle.pack_f1(wn, oracle.build_table(wn))
    assert p.code_bits == po["code_bits"] and p.n_f1esc == po["n_f1esc"] and p.n_esc == po["n_esc"]
    assert np.array_equal(p.sm.numpy(), po["sm"])
    assert np.array_equal(p.width.numpy(), po["width"].reshape(-1))
    nc = po["codes"].size
    assert np.array_equal(p.codes.numpy().view(np.uint32)[:nc], po["codes"])
    assert not p.codes.numpy()[nc:].any()
    assert np.array_equal(p.esc_rank.numpy()[: p.n_f1esc], po["esc"])
    assert np.array_equal(p.anchor.numpy().view(np.uint64), po["anchor"])
    assert np.array_equal(p.f1_pre.numpy().view(np.uint32), po["f1_pre"])
    assert np.array_equal(p.esc_pre.numpy().view(np.uint32), po["esc_pre"])


@pytest.mark.parametrize("case", ["llm", "all_patterns", "one_exponent", "ties", "groups"])
def test_huffman_pack_matches_oracle_bytes(case):
    """binade_huff_lengths / binade_huff_pack (host C++) against the oracle's
    Huffman codec: the same lengths (tie rule included) and the same bytes."""
    rng = np.random.default_rng(31)
    if case == "llm":
        wn = _np(_tensor(40, 3072, sigma=0.02, seed=6, frac=1e-3, scale=20.0))
    elif case == "all_patterns":
        wn = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    elif case == "one_exponent":
        wn = ((rng.integers(0, 2, (7, 100)) << 15) | (125 << 7) | rng.integers(0, 128, (7, 100))).astype(np.uint16)
    elif case == "ties":   # many equal counts: the merge order decides the lengths
        e = np.repeat(np.arange(100, 124), 37)
        rng.shuffle(e)
        wn = ((e << 7) | rng.integers(0, 128, e.size)).astype(np.uint16).reshape(1, -1)
    else:   # several groups of 128 blocks and a ragged block
        wn = _np(_tensor(3, 9000, sigma=0.015, seed=7, frac=0.0, scale=1.0))
    w = torch.from_numpy(np.ascontiguousarray(wn).view(np.int16)).view(torch.bfloat16)
    p = B.pack_huff(w)
    ln = oracle.huff_lengths(oracle.exponent_counts(wn))
    assert bytes(p.len) == ln.tobytes()
    po = oracle.huff_pack(wn, ln)
    assert p.stream_bytes == po["stream_bytes"]
    assert np.array_equal(p.sm.numpy(), po["sm"])
    s = p.stream.numpy()
    assert np.array_equal(s[: p.stream_bytes], po["stream"]) and not s[p.stream_bytes:].any()
    assert s.size >= p.stream_bytes + 8
    assert np.array_equal(p.block_len.numpy(), po["block_len"])
    assert np.array_equal(p.group_off.numpy().view(np.uint64), po["group_off"])


def test_huffman_deep_tree_refused():
    # Fibonacci counts over 34 exponents make a chain: depth 33 > 31
    f = [1, 1]
    while len(f) < 34:
        f.append(f[-1] + f[-2])
    e = np.concatenate([np.full(c, i, np.uint16) for i, c in enumerate(f)])
    wn = (e << 7).astype(np.uint16)
    ln = (ctypes.c_uint8 * 256)()
    cap = ctypes.c_uint64(0)
    rc = B.lib().binade_huff_lengths(ctypes.c_void_p(wn.ctypes.data), wn.size, ln, ctypes.byref(cap))
    assert rc == B.EUNSUPPORTED


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """The ctypes mirrors have the sizes and field offsets gcc gives the
    header's structs."""
    import subprocess
    src = tmp_path / "sizes.c"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src.write_text("""#include <stdio.h>
#include <stddef.h>
#include "binade.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(binade_table), sizeof(binade_rice),
         sizeof(binade_r4), sizeof(binade_f1), sizeof(binade_huff),
         offsetof(binade_f1, sm), offsetof(binade_huff, sm), offsetof(binade_f1, n_esc));
  return 0;
}
""")
    exe = tmp_path / "sizes"
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got == [ctypes.sizeof(B.Table), ctypes.sizeof(B.RiceDesc), ctypes.sizeof(B.R4Desc),
                   ctypes.sizeof(B.F1Desc), ctypes.sizeof(B.HuffDesc), B.F1Desc.sm.offset,
                   B.HuffDesc.sm.offset, B.F1Desc.n_esc.offset]


def test_new_device_entry_points_validate_before_touching_the_gpu():
    """The format 1, small-batch, MoE epilogue, device pack and Huffman entry
    points refuse bad arguments on the host, before any HIP call."""
    L = B.lib()
    P = ctypes.c_void_p
    # format 1
    f = B.F1Desc()
    r = B.R4Desc()
    assert L.binade_f1_to_r4(None, ctypes.byref(r), None, None) == B.EINVAL
    f.rows, f.cols, f.n = 4, 48, 5
    assert L.binade_f1_to_r4(ctypes.byref(f), ctypes.byref(r), None, None) == B.EUNSUPPORTED
    f.cols = 64
    assert L.binade_f1_to_r4(ctypes.byref(f), ctypes.byref(r), None, None) == B.EINVAL   # null planes
    # small-batch product: m outside 1..8, short strides
    d = B.R4Desc()
    d.rows, d.cols = 4, 64
    d.sm = d.nib = d.esc_pre = 16
    for m, ldx, ldy in [(0, 64, 4), (9, 64, 4), (2, 32, 4), (2, 64, 3)]:
        assert L.binade_r4_gemv_rows(ctypes.byref(d), P(16), ldx, m, P(16), ldy, B.F32, None) == B.EINVAL
    assert L.binade_r4_gemv_rows(ctypes.byref(d), P(8), 64, 2, P(16), 4, B.F32, None) == B.EUNSUPPORTED
    assert L.binade_r4_gemv_rows(ctypes.byref(d), P(16), 68, 2, P(16), 4, B.F32, None) == B.EUNSUPPORTED
    assert L.binade_bf16_gemv_rows(P(16), 4, 48, P(16), 64, 2, P(16), 4, B.F32, None) == B.EUNSUPPORTED
    # MoE epilogue
    assert L.binade_moe_silu_mul(None, None, -1, None, B.BF16, None) == B.EINVAL
    assert L.binade_moe_silu_mul(None, None, 10, None, 7, None) == B.EINVAL
    assert L.binade_moe_silu_mul(None, None, 0, None, B.BF16, None) == B.OK      # empty: no launch
    assert L.binade_moe_silu_mul(None, P(16), 10, P(16), B.BF16, None) == B.EINVAL
    for k in (0, 65):
        assert L.binade_moe_combine(P(16), P(16), 2, k, 8, P(16), B.F32, None) == B.EINVAL
    assert L.binade_moe_combine(P(16), P(16), 0, 8, 8, P(16), B.F32, None) == B.OK
    # device table and pack
    t = B.Table()
    assert L.binade_build_table_gpu(None, 10, P(16), P(16), None) == B.EINVAL
    assert L.binade_build_table_gpu(P(8), 10, P(16), P(16), None) == B.EUNSUPPORTED
    assert B.lib().binade_pack_gpu_workspace_bytes(0, 64) == 0
    assert B.lib().binade_pack_gpu_workspace_bytes(4, 64) >= 2048
    rd = B.RiceDesc()
    assert L.binade_pack_rice_gpu(P(16), 4, 48, ctypes.byref(t), ctypes.byref(rd), P(16), None,
                                  None) == B.EUNSUPPORTED
    t.n, t.k = 1, 0
    t.count_of_rank[0] = 4 * 64
    assert L.binade_pack_rice_gpu(P(16), 4, 64, ctypes.byref(t), ctypes.byref(rd), P(16), None,
                                  None) == B.EINVAL      # null planes
    rd.sm, rd.unary, rd.anchor, rd.esc_pre = 16, 16, 16, 16
    rd.unary_words = 1
    assert L.binade_pack_rice_gpu(P(16), 4, 64, ctypes.byref(t), ctypes.byref(rd), P(16), None,
                                  None) == B.ENOSPACE
    # Huffman decode
    h = B.HuffDesc()
    assert L.binade_huff_decode(None, P(16), P(16), None, None) == B.EINVAL
    h.n = 100
    h.sm, h.stream, h.block_len, h.group_off = 16, 16, 16, 16
    h.stream_bytes, h.stream_cap = 100, 104       # needs 8 bytes of look-ahead
    assert L.binade_huff_decode(ctypes.byref(h), P(16), P(16), None, None) == B.EUNSUPPORTED
    h.stream_cap = 108
    h.len[3] = 32
    assert L.binade_huff_decode(ctypes.byref(h), P(16), P(16), None, None) == B.EINVAL
    assert B.lib().binade_huff_workspace_bytes() > 4096


def _plan_header(plan):
    raw = bytes(plan.host)
    magic, count, spans, first_off, items_off, pool_off, nbytes, _ = np.frombuffer(
        raw[:32], dtype=np.uint32)
    first = np.frombuffer(raw[first_off:first_off + 4 * (int(count) + 1)], dtype=np.uint32)
    return raw, int(magic), int(count), int(spans), first, int(pool_off), int(nbytes)


def test_decode_plan_layout_and_checks():
    """binade_rice_to_r4_plan on host planes (it records addresses and never
    reads through them): one span per 32768 weights of row-chunks (16 chunks
    of 2048 for long rows, 32768 / cols short rows), the escape exponents of
    every table in order, the R4 tables the oracle gives, and the declared
    status codes for sizes, headers and tensors the streamed decoder does
    not take."""
    L = B.lib()
    assert L.binade_rice_plan_bytes(0) == 40
    assert L.binade_rice_plan_bytes(-1) == B.EINVAL
    assert L.binade_rice_plan_bytes(65537) == B.EINVAL
    shapes = [(24, 3072), (8, 8192), (3, 1152)]
    ws = [synth.normal_bf16(synth.TensorSpec("p", r, c, 0.02, 40 + i, outlier_frac=2e-3,
                                             outlier_scale=1e3))
          for i, (r, c) in enumerate(shapes)]
    planes = [B.pack_rice(w) for w in ws]
    plan = B.RicePlan(planes)
    raw, magic, count, spans, first, pool_off, nbytes = _plan_header(plan)
    assert magic == 0x31505242 and count == 3
    assert first.tolist() == [0, 3, 5, 6] and spans == 6
    pool = b"".join(bytes(bytearray(p.table.exp_of_rank))[15:p.table.n] for p in planes)
    assert raw[pool_off:nbytes] == pool and len(pool) > 0
    for w, o in zip(ws, plan.outs):
        wn = w.contiguous().view(torch.int16).numpy().view(np.uint16)
        assert o.lut == bytes(oracle.make_r4(wn, oracle.build_table(wn))["lut"])
    # a buffer one byte short
    n = len(planes)
    din = (B.RiceDesc * n)(*[p.desc() for p in planes])
    dout = (B.R4Desc * n)()
    for i, o in enumerate(plan.outs):
        dout[i].nib = o.nib.data_ptr()
        dout[i].esc = o.esc.data_ptr()
    short = (ctypes.c_uint8 * (L.binade_rice_plan_bytes(n) - 1))()
    assert L.binade_rice_to_r4_plan(din, dout, n, short, len(short)) == B.EINVAL
    # rows shorter than 1024 weights, a last row-chunk of 64 columns, and
    # Rice k != 1 take the per-job kernel only
    for w in (synth.normal_bf16(synth.TensorSpec("s", 50, 64, 0.02, 7)),
              synth.normal_bf16(synth.TensorSpec("s", 5, 4160, 0.02, 8)),
              (torch.randn(64, 2048, generator=torch.Generator().manual_seed(3)) *
               torch.exp2(torch.randint(-60, 60, (64, 2048),
                                        generator=torch.Generator().manual_seed(4)))
               ).to(torch.bfloat16)):
        p = B.pack_rice(w)
        with pytest.raises(B.BinadeError) as e:
            B.RicePlan([planes[0], p])
        assert e.value.code == B.EUNSUPPORTED, (p.rows, p.cols, p.k)
    # headers that are not a plan's; an empty plan launches nothing
    assert L.binade_rice_to_r4_run(bytes(32), None, None, None) == B.EINVAL
    bad = bytearray(raw)
    bad[12] ^= 4   # first_job's offset
    assert L.binade_rice_to_r4_run(bytes(bad), None, None, None) == B.EINVAL
    assert L.binade_rice_to_r4_run(None, None, None, None) == B.EINVAL
    empty = B.RicePlan([])
    assert L.binade_rice_to_r4_run(empty.host, None, None, None) == B.OK
