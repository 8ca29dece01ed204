"""Binade oracle: TEST INFRASTRUCTURE ONLY.

A plain, slow CPU statement of the Binade hot path (the C file beside this
one), wrapped for numpy. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``decode_gemv_tensor_amd``) never imports it and shares no code with it.

Every function cites the passage of the pages it follows; the readings taken
where the pages are silent are stated in ``binade_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "binade_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_SO = os.path.join(_OUT_DIR, "liboracle.so")

CHUNK = 2048  # weights per row-chunk (the oracle's own constant)

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no contraction)."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    srcs = [_SRC]
    if not force and os.path.exists(_SO):
        newest = max(os.path.getmtime(s) for s in srcs)
        if os.path.getmtime(_SO) >= newest:
            return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", tmp] + srcs + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # BINADE_ORACLE_LIB: a copy of the oracle built elsewhere (the
            # planted-mistake test runs the pins against deliberately broken
            # copies); otherwise the library beside this file
            path = os.environ.get("BINADE_ORACLE_LIB")
            if not path:
                build()   # compiles when the library is missing or older than its source
                path = _SO
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            U32 = ctypes.c_uint32
            I = ctypes.c_int
            lib.oracle_build_table.argtypes = [P, I64, P, P, P]
            lib.oracle_rice_code_bits.argtypes = [P, U32, I]
            lib.oracle_rice_code_bits.restype = ctypes.c_uint64
            lib.oracle_rice_k.argtypes = [P, U32]
            lib.oracle_pack_rice.argtypes = [P, I64, I64, P, U32, I, P, P, I64,
                                             P, I64, P, P, P]
            lib.oracle_rice_decode.argtypes = [I64, I64, I, P, U32, P, P,
                                               ctypes.c_uint64, P, P, P, P]
            lib.oracle_make_r4.argtypes = [P, I64, I64, P, U32, P, P, P, P,
                                           I64, P]
            lib.oracle_r4_unpack.argtypes = [I64, I64, P, P, P, P, P, I64, P]
            lib.oracle_gemv_replay.argtypes = [P, I64, I64, P, P]
            lib.oracle_gemv_f64.argtypes = [P, I64, I64, P, P]
            lib.oracle_moe_replay.argtypes = [P, I64, I64, I64, P, I, P, I64,
                                              I64, P]
            lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
            lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
            lib.oracle_f32_to_bf16_array.argtypes = [P, I64, P]
            lib.oracle_gemm_f64.argtypes = [P, I64, I64, P, I64, P]
            lib.oracle_pack_f1.argtypes = [P, I64, I64, P, U32, P, P, P, I64, P, I64,
                                           P, P, P, P, P]
            lib.oracle_f1_decode.argtypes = [I64, I64, P, U32, P, P, P, ctypes.c_uint64,
                                             P, I64, P, P, P, P]
            lib.oracle_mfma_step.argtypes = [P, P, ctypes.c_float]
            lib.oracle_mfma_step.restype = ctypes.c_float
            lib.oracle_gemm_replay.argtypes = [P, I64, I64, P, I64, P]
            lib.oracle_huff_lengths.argtypes = [P, P]
            lib.oracle_huff_pack.argtypes = [P, I64, P, P, P, I64, P, P, P]
            lib.oracle_huff_decode.argtypes = [I64, P, P, P, I64, P, P, P]
            lib.oracle_silu_mul.argtypes = [P, P, I64, P]
            lib.oracle_silu_mul.restype = None
            lib.oracle_moe_combine.argtypes = [P, P, I64, I, I64, P]
            lib.oracle_gemm_replay_entries.argtypes = [P, I64, I64, P, I64, P,
                                                       P, I64, P]
            _lib = lib
    return _lib


class OracleError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code}")
        self.code = code


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _check(fn: str, rc: int):
    if rc != 0:
        raise OracleError(fn, rc)


# ---------------------------------------------------------------- table
def build_table(w_bits) -> dict:
    """Frequency-rank table of the exponent field ("Binade" package page,
    intro and "How it works": one table per tensor)."""
    w = _u16(w_bits).reshape(-1)
    lib = _load()
    n = ctypes.c_uint32(0)
    exp_of_rank = np.zeros(256, np.uint8)
    count_of_rank = np.zeros(256, np.uint64)
    _check("oracle_build_table",
           lib.oracle_build_table(_p(w), w.size, ctypes.byref(n),
                                  _p(exp_of_rank), _p(count_of_rank)))
    return {"n": int(n.value), "exp_of_rank": exp_of_rank,
            "count_of_rank": count_of_rank}


def rice_code_bits(count_of_rank: np.ndarray, n: int, k: int) -> int:
    c = np.ascontiguousarray(count_of_rank, np.uint64)
    return int(_load().oracle_rice_code_bits(_p(c), n, k))


def rice_k(count_of_rank: np.ndarray, n: int) -> int:
    c = np.ascontiguousarray(count_of_rank, np.uint64)
    return int(_load().oracle_rice_k(_p(c), n))


# ---------------------------------------------------------------- format 2
def pack_rice(w_bits, table: dict, k: int | None = None) -> dict:
    """Format 2: sign+mantissa bytes plus Rice-coded ranks ("Binade" package
    page, "How it works")."""
    w = _u16(w_bits)
    rows, cols = w.shape
    n = table["n"]
    if k is None:
        k = rice_k(table["count_of_rank"], n)
    nsym = rows * cols
    # capacity: every symbol's longest possible code, then trimmed
    max_q = (255 >> k) + 1
    unary_words = (nsym * max_q + 31) // 32 + 1
    unary_words = min(unary_words,
                      (rice_code_bits(table["count_of_rank"], n, k) + 31) // 32 + 1)
    rem_words = (nsym * k + 31) // 32 + 1
    cpr = (cols + CHUNK - 1) // CHUNK
    nchunks = rows * cpr
    sm = np.zeros(nsym, np.uint8)
    unary = np.zeros(unary_words, np.uint32)
    rem = np.zeros(max(rem_words, 1), np.uint32)
    anchor = np.zeros(nchunks + 1, np.uint64)
    esc_pre = np.zeros(nchunks + 1, np.uint32)
    bits = ctypes.c_uint64(0)
    _check("oracle_pack_rice",
           _load().oracle_pack_rice(_p(w), rows, cols, _p(table["exp_of_rank"]),
                                    n, k, _p(sm), _p(unary), unary_words,
                                    _p(rem), rem_words, _p(anchor),
                                    _p(esc_pre), ctypes.byref(bits)))
    ub = int(bits.value)
    return {"rows": rows, "cols": cols, "k": k, "n": n,
            "exp_of_rank": table["exp_of_rank"].copy(),
            "sm": sm.reshape(rows, cols),
            "unary": unary[: (ub + 31) // 32].copy(), "unary_bits": ub,
            "rem": rem[: (nsym * k + 31) // 32].copy(),
            "anchor": anchor, "esc_pre": esc_pre,
            "n_esc": int(esc_pre[-1])}


def rice_decode(pk: dict) -> np.ndarray:
    rows, cols = pk["rows"], pk["cols"]
    out = np.zeros((rows, cols), np.uint16)
    unary = np.concatenate([pk["unary"], np.zeros(1, np.uint32)])
    rem = np.concatenate([pk["rem"], np.zeros(1, np.uint32)])
    sm = np.ascontiguousarray(pk["sm"])
    _check("oracle_rice_decode",
           _load().oracle_rice_decode(rows, cols, pk["k"],
                                      _p(np.ascontiguousarray(pk["exp_of_rank"])),
                                      pk["n"], _p(sm), _p(unary),
                                      pk["unary_bits"], _p(rem),
                                      _p(np.ascontiguousarray(pk["anchor"])),
                                      _p(np.ascontiguousarray(pk["esc_pre"])),
                                      _p(out)))
    return out


# ---------------------------------------------------------------- format 1
TILE = 128  # columns per format 1 tile (the oracle's own constant)


def pack_f1(w_bits, table: dict) -> dict:
    """Format 1: a code width per 128-column tile with escapes ("Binade"
    package page, "How it works": the second file format)."""
    w = _u16(w_bits)
    rows, cols = w.shape
    nsym = rows * cols
    tpr = (cols + TILE - 1) // TILE
    cpr = (cols + CHUNK - 1) // CHUNK
    nchunks = rows * cpr
    code_words = nsym * 8 // 32 + 2
    sm = np.zeros(nsym, np.uint8)
    width = np.zeros(rows * tpr, np.uint8)
    codes = np.zeros(code_words, np.uint32)
    esc = np.zeros(max(nsym, 1), np.uint8)
    anchor = np.zeros(nchunks + 1, np.uint64)
    f1_pre = np.zeros(nchunks + 1, np.uint32)
    esc_pre = np.zeros(nchunks + 1, np.uint32)
    bits = ctypes.c_uint64(0)
    nf1 = ctypes.c_int64(0)
    _check("oracle_pack_f1",
           _load().oracle_pack_f1(_p(w), rows, cols, _p(table["exp_of_rank"]), table["n"],
                                  _p(sm), _p(width), _p(codes), code_words, _p(esc), esc.size,
                                  _p(anchor), _p(f1_pre), _p(esc_pre), ctypes.byref(bits),
                                  ctypes.byref(nf1)))
    cb = int(bits.value)
    return {"rows": rows, "cols": cols, "n": table["n"],
            "exp_of_rank": table["exp_of_rank"].copy(), "sm": sm.reshape(rows, cols),
            "width": width.reshape(rows, tpr), "codes": codes[: (cb + 31) // 32].copy(),
            "code_bits": cb, "esc": esc[: nf1.value].copy(), "n_f1esc": int(nf1.value),
            "anchor": anchor, "f1_pre": f1_pre, "esc_pre": esc_pre,
            "n_esc": int(esc_pre[-1])}


def f1_decode(pk: dict) -> np.ndarray:
    rows, cols = pk["rows"], pk["cols"]
    out = np.zeros((rows, cols), np.uint16)
    codes = np.concatenate([pk["codes"], np.zeros(1, np.uint32)])
    esc = pk["esc"] if pk["esc"].size else np.zeros(1, np.uint8)
    _check("oracle_f1_decode",
           _load().oracle_f1_decode(rows, cols, _p(np.ascontiguousarray(pk["exp_of_rank"])),
                                    pk["n"], _p(np.ascontiguousarray(pk["sm"])),
                                    _p(np.ascontiguousarray(pk["width"])), _p(codes),
                                    pk["code_bits"], _p(np.ascontiguousarray(esc)),
                                    pk["n_f1esc"], _p(np.ascontiguousarray(pk["anchor"])),
                                    _p(np.ascontiguousarray(pk["f1_pre"])),
                                    _p(np.ascontiguousarray(pk["esc_pre"])), _p(out)))
    return out


# ---------------------------------------------------------------- R4
def make_r4(w_bits, table: dict) -> dict:
    """R4 runtime layout ("Binade" package page, "How it works": a 4-bit code
    per rank, the few large ranks escaping to a side list)."""
    w = _u16(w_bits)
    rows, cols = w.shape
    cpr = (cols + CHUNK - 1) // CHUNK
    lut = np.zeros(16, np.uint8)
    nib = np.zeros(rows * cols // 2, np.uint8)
    esc_pre = np.zeros(rows * cpr + 1, np.uint32)
    cap = rows * cols
    esc = np.zeros(max(cap, 1), np.uint32)
    nesc = ctypes.c_int64(0)
    _check("oracle_make_r4",
           _load().oracle_make_r4(_p(w), rows, cols, _p(table["exp_of_rank"]),
                                  table["n"], _p(lut), _p(nib), _p(esc_pre),
                                  _p(esc), cap, ctypes.byref(nesc)))
    sm = ((w >> 8) & 0x80 | (w & 0x7F)).astype(np.uint8)
    return {"rows": rows, "cols": cols, "lut": lut, "sm": sm,
            "nib": nib.reshape(rows, cols // 2), "esc_pre": esc_pre,
            "esc": esc[: nesc.value].copy(), "n_esc": int(nesc.value)}


def r4_unpack(r4: dict) -> np.ndarray:
    rows, cols = r4["rows"], r4["cols"]
    out = np.zeros((rows, cols), np.uint16)
    esc = r4["esc"] if r4["esc"].size else np.zeros(1, np.uint32)
    _check("oracle_r4_unpack",
           _load().oracle_r4_unpack(rows, cols, _p(np.ascontiguousarray(r4["lut"])),
                                    _p(np.ascontiguousarray(r4["sm"])),
                                    _p(np.ascontiguousarray(r4["nib"])),
                                    _p(np.ascontiguousarray(r4["esc_pre"])),
                                    _p(np.ascontiguousarray(esc)), r4["n_esc"],
                                    _p(out)))
    return out


# ---------------------------------------------------------------- products
def gemv_replay(w_bits, x_bits) -> np.ndarray:
    """y = W x in the library's fixed fp32 order (see binade_oracle.c)."""
    w = _u16(w_bits)
    x = _u16(x_bits).reshape(-1)
    rows, cols = w.shape
    assert x.size == cols
    y = np.zeros(rows, np.float32)
    _check("oracle_gemv_replay",
           _load().oracle_gemv_replay(_p(w), rows, cols, _p(x), _p(y)))
    return y


def gemv_f64(w_bits, x_bits) -> np.ndarray:
    """y = W x summed in double: the plain definition."""
    w = _u16(w_bits)
    x = _u16(x_bits).reshape(-1)
    rows, cols = w.shape
    y = np.zeros(rows, np.float64)
    _check("oracle_gemv_f64",
           _load().oracle_gemv_f64(_p(w), rows, cols, _p(x), _p(y)))
    return y


def moe_replay(experts_bits, x_bits, idx, x_per_slot: bool) -> np.ndarray:
    """Expert-gather GEMV: every (token, slot) pair in the matvec order."""
    e = _u16(experts_bits)
    n_experts, N, K = e.shape
    x = _u16(x_bits)
    idx = np.ascontiguousarray(idx, np.int32)
    n_tokens, top_k = idx.shape
    y = np.zeros((n_tokens * top_k, N), np.float32)
    _check("oracle_moe_replay",
           _load().oracle_moe_replay(_p(e), n_experts, N, K, _p(x),
                                     1 if x_per_slot else 0, _p(idx),
                                     n_tokens, top_k, _p(y)))
    return y


def gemv_rows_replay(w_bits, x_rows_bits) -> np.ndarray:
    """Y[b] = W x_b for each row of X, each row in the matvec order: the
    small-batch decode product's definition."""
    x = _u16(x_rows_bits)
    return np.stack([gemv_replay(w_bits, x[b]) for b in range(x.shape[0])])


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """MoE activation h = silu(gate) * up, in double, rounded once to fp32."""
    g = np.ascontiguousarray(gate, np.float32)
    u = np.ascontiguousarray(up, np.float32)
    assert g.shape == u.shape
    out = np.zeros(g.shape, np.float32)
    _load().oracle_silu_mul(_p(g), _p(u), g.size, _p(out))
    return out


def moe_combine(y: np.ndarray, weights: np.ndarray, top_k: int) -> np.ndarray:
    """out[t] = fp32 fma chain over the token's top_k slots, slot order."""
    y = np.ascontiguousarray(y, np.float32)
    w = np.ascontiguousarray(weights, np.float32).reshape(-1)
    pairs, n = y.shape
    assert pairs % top_k == 0 and w.size == pairs
    out = np.zeros((pairs // top_k, n), np.float32)
    _check("oracle_moe_combine",
           _load().oracle_moe_combine(_p(y), _p(w), pairs // top_k, top_k, n, _p(out)))
    return out


HUFF_BLOCK, HUFF_GROUP, HUFF_MAXLEN = 64, 128, 31


def exponent_counts(w_bits) -> np.ndarray:
    """Count of each exponent byte (the Huffman codec's symbol counts)."""
    w = _u16(w_bits).reshape(-1)
    return np.bincount((w >> 7) & 0xFF, minlength=256).astype(np.uint64)


def huff_lengths(counts) -> np.ndarray:
    """Huffman code length of each exponent ("Lossless BF16 weight
    compression" page: canonical Huffman over the exponent field)."""
    c = np.ascontiguousarray(counts, np.uint64)
    assert c.size == 256
    ln = np.zeros(256, np.uint8)
    _check("oracle_huff_lengths", _load().oracle_huff_lengths(_p(c), _p(ln)))
    return ln


def huff_pack(w_bits, lengths) -> dict:
    """Blocks of 64 exponents in canonical Huffman codes, MSB-first, each
    padded to a byte; 8-bit block lengths; a byte offset per 128 blocks."""
    w = _u16(w_bits).reshape(-1)
    ln = np.ascontiguousarray(lengths, np.uint8)
    n = w.size
    counts = exponent_counts(w)
    nb = (n + HUFF_BLOCK - 1) // HUFF_BLOCK
    cap = int((counts * ln.astype(np.uint64)).sum() + 7) // 8 + nb
    sm = np.zeros(n, np.uint8)
    stream = np.zeros(max(cap, 1), np.uint8)
    block_len = np.zeros(nb, np.uint8)
    group_off = np.zeros((nb + HUFF_GROUP - 1) // HUFF_GROUP + 1, np.uint64)
    used = ctypes.c_uint64(0)
    _check("oracle_huff_pack",
           _load().oracle_huff_pack(_p(w), n, _p(ln), _p(sm), _p(stream), stream.size,
                                    _p(block_len), _p(group_off), ctypes.byref(used)))
    return {"n": n, "len": ln.copy(), "sm": sm, "stream": stream[: used.value].copy(),
            "stream_bytes": int(used.value), "block_len": block_len, "group_off": group_off}


def huff_decode(pk: dict) -> np.ndarray:
    """The packed stream back to bf16 bits, code by code."""
    n = pk["n"]
    out = np.zeros(n, np.uint16)
    stream = pk["stream"] if pk["stream"].size else np.zeros(1, np.uint8)
    _check("oracle_huff_decode",
           _load().oracle_huff_decode(n, _p(np.ascontiguousarray(pk["len"], np.uint8)),
                                      _p(np.ascontiguousarray(pk["sm"], np.uint8)),
                                      _p(np.ascontiguousarray(stream, np.uint8)),
                                      pk["stream_bytes"],
                                      _p(np.ascontiguousarray(pk["block_len"], np.uint8)),
                                      _p(np.ascontiguousarray(pk["group_off"], np.uint64)),
                                      _p(out)))
    return out


def gemm_f64(w_bits, x_bits) -> np.ndarray:
    """Y = X W^T summed in double (the prompt GEMM's plain definition)."""
    w = _u16(w_bits)
    x = _u16(x_bits)
    N, K = w.shape
    M = x.shape[0]
    y = np.zeros((M, N), np.float64)
    _check("oracle_gemm_f64", _load().oracle_gemm_f64(_p(w), N, K, _p(x), M, _p(y)))
    return y


def mfma_step(a_bits, b_bits, c: float) -> np.float32:
    """One output of one bf16 matrix-core step, c + sum of 32 products, by the
    reading stated above oracle_mfma_step in binade_oracle.c."""
    a = _u16(a_bits).reshape(-1)
    b = _u16(b_bits).reshape(-1)
    assert a.size == 32 and b.size == 32
    return np.float32(_load().oracle_mfma_step(_p(a), _p(b), ctypes.c_float(c)))


def gemm_replay(w_bits, x_bits) -> np.ndarray:
    """Y = X W^T in the prompt GEMM's documented order of matrix-core steps
    and slices ("Binade" package page, "NVIDIA GPUs")."""
    w = _u16(w_bits)
    x = _u16(x_bits)
    N, K = w.shape
    M, K2 = x.shape
    assert K == K2
    y = np.zeros((M, N), np.float32)
    _check("oracle_gemm_replay", _load().oracle_gemm_replay(_p(w), N, K, _p(x), M, _p(y)))
    return y


def gemm_replay_entries(w_bits, x_bits, mi, ni) -> np.ndarray:
    """The replay of the entries Y[mi[i], ni[i]] only."""
    w = _u16(w_bits)
    x = _u16(x_bits)
    N, K = w.shape
    M = x.shape[0]
    mi = np.ascontiguousarray(mi, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    out = np.zeros(mi.size, np.float32)
    _check("oracle_gemm_replay_entries",
           _load().oracle_gemm_replay_entries(_p(w), N, K, _p(x), M, _p(mi),
                                              _p(ni), mi.size, _p(out)))
    return out


def f32_to_bf16(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    out = np.zeros(y.shape, np.uint16)
    _load().oracle_f32_to_bf16_array(_p(y), y.size, _p(out))
    return out
