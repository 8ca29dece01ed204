"""Python binding of libbinade (include/binade.h): argument marshalling only.

Every step of the path runs in the library: the table and the format 2 pack
in its host C++, the format 2 -> R4 conversion, the products and the unpack in
its HIP kernels. PyTorch provides device memory (tensors) and streams. If the
built library is missing this module raises on first use; there is no other
implementation behind it.
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libbinade.so")
CHUNK = 2048

OK, EINVAL, ECORRUPT, EUNSUPPORTED, EHIP, ENOSPACE = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
DEV_CORRUPT_STREAM, DEV_BAD_INDEX, DEV_CORRUPT_ESC = 0x1, 0x2, 0x4

EXPORTS = ["binade_status_str", "binade_last_hip_error", "binade_build_table",
           "binade_sizes_of", "binade_pack_rice", "binade_rice_to_r4",
           "binade_f1_sizes_of", "binade_pack_f1", "binade_f1_to_r4",
           "binade_rice_to_r4_batch", "binade_unpack", "binade_r4_gemv",
           "binade_r4_gemv_batch", "binade_bf16_gemv", "binade_bf16_gemv_batch",
           "binade_r4_gemm", "binade_bf16_gemm", "binade_gemm_workspace_bytes",
           "binade_r4_gemm_noalloc", "binade_gemm_scratch_bytes",
           "binade_r4_moe_gemv", "binade_bf16_moe_gemv", "binade_r4_gemv_rows",
           "binade_bf16_gemv_rows", "binade_moe_silu_mul", "binade_moe_combine",
           "binade_build_table_gpu", "binade_pack_gpu_workspace_bytes", "binade_pack_rice_gpu",
           "binade_huff_lengths", "binade_huff_pack", "binade_huff_workspace_bytes",
           "binade_huff_decode", "binade_rice_plan_bytes", "binade_rice_to_r4_plan",
           "binade_rice_to_r4_run"]


class Table(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("exp_of_rank", ctypes.c_uint8 * 256),
                ("rank_of_exp", ctypes.c_uint16 * 256),
                ("count_of_rank", ctypes.c_uint64 * 256)]


class HuffDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("len", ctypes.c_uint8 * 256),
                ("sm", ctypes.c_void_p), ("stream", ctypes.c_void_p),
                ("stream_bytes", ctypes.c_uint64), ("stream_cap", ctypes.c_uint64),
                ("block_len", ctypes.c_void_p), ("group_off", ctypes.c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("n_weights", "n_chunks", "unary_bits", "unary_words",
                 "rem_words", "n_esc", "nib_bytes")]


class RiceDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("k", ctypes.c_uint32), ("n", ctypes.c_uint32),
                ("exp_of_rank", ctypes.c_uint8 * 256),
                ("sm", ctypes.c_void_p), ("unary", ctypes.c_void_p),
                ("unary_bits", ctypes.c_uint64), ("unary_words", ctypes.c_uint64),
                ("rem", ctypes.c_void_p), ("rem_words", ctypes.c_uint64),
                ("anchor", ctypes.c_void_p), ("esc_pre", ctypes.c_void_p),
                ("n_esc", ctypes.c_uint64)]


class F1Desc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("n", ctypes.c_uint32), ("exp_of_rank", ctypes.c_uint8 * 256),
                ("sm", ctypes.c_void_p), ("width", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("code_bits", ctypes.c_uint64),
                ("code_words", ctypes.c_uint64), ("esc_rank", ctypes.c_void_p),
                ("n_f1esc", ctypes.c_uint64), ("esc_cap", ctypes.c_uint64),
                ("anchor", ctypes.c_void_p), ("f1_pre", ctypes.c_void_p),
                ("esc_pre", ctypes.c_void_p), ("n_esc", ctypes.c_uint64)]


class F1Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("n_weights", "n_tiles", "n_chunks", "code_words", "esc_cap")]


class R4Desc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("lut", ctypes.c_uint8 * 16),
                ("sm", ctypes.c_void_p), ("nib", ctypes.c_void_p),
                ("esc_pre", ctypes.c_void_p), ("esc", ctypes.c_void_p),
                ("n_esc", ctypes.c_uint64)]


class BinadeError(RuntimeError):
    def __init__(self, fn: str, code: int, hip: int = 0):
        lib = _lib_or_none()
        text = lib.binade_status_str(code).decode() if lib else str(code)
        super().__init__(f"{fn}: {text} ({code})" + (f", hip error {hip}" if hip else ""))
        self.code = code


_lock = threading.Lock()
_lib = None


def _lib_or_none():
    return _lib


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("BINADE_LIB") or LIB_PATH   # another build of the library
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is not built; run "
                    "`python -m decode_gemv_tensor_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(path)
            P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            L.binade_status_str.argtypes = [I32]
            L.binade_status_str.restype = ctypes.c_char_p
            L.binade_last_hip_error.restype = I32
            L.binade_gemm_workspace_bytes.argtypes = [I64, I64, I64]
            L.binade_gemm_workspace_bytes.restype = I64
            L.binade_gemm_scratch_bytes.argtypes = []
            L.binade_gemm_scratch_bytes.restype = I64
            L.binade_pack_gpu_workspace_bytes.argtypes = [I64, I64]
            L.binade_pack_gpu_workspace_bytes.restype = I64
            L.binade_huff_workspace_bytes.argtypes = []
            L.binade_huff_workspace_bytes.restype = I64
            L.binade_rice_plan_bytes.argtypes = [I32]
            L.binade_rice_plan_bytes.restype = I64
            sig = {
                "binade_build_table": [P, I64, P],
                "binade_sizes_of": [P, I64, I64, P],
                "binade_pack_rice": [P, I64, I64, P, P],
                "binade_rice_to_r4": [P, P, P, P],
                "binade_rice_to_r4_batch": [P, P, I32, P, P],
                "binade_rice_to_r4_plan": [P, P, I32, P, I64],
                "binade_rice_to_r4_run": [P, P, P, P],
                "binade_f1_sizes_of": [I64, I64, P],
                "binade_pack_f1": [P, I64, I64, P, P],
                "binade_f1_to_r4": [P, P, P, P],
                "binade_r4_gemv_batch": [P, P, P, I32, I32, P],
                "binade_bf16_gemv_batch": [P, P, P, P, P, I32, I32, P],
                "binade_unpack": [P, P, P],
                "binade_r4_gemv": [P, P, P, I32, P],
                "binade_bf16_gemv": [P, I64, I64, P, P, I32, P],
                "binade_r4_gemv_rows": [P, P, I64, I32, P, I64, I32, P],
                "binade_bf16_gemv_rows": [P, I64, I64, P, I64, I32, P, I64, I32, P],
                "binade_moe_silu_mul": [P, P, I64, P, I32, P],
                "binade_moe_combine": [P, P, I64, I32, I64, P, I32, P],
                "binade_build_table_gpu": [P, I64, P, P, P],
                "binade_huff_lengths": [P, I64, P, P],
                "binade_huff_pack": [P, P],
                "binade_huff_decode": [P, P, P, P, P],
                "binade_pack_rice_gpu": [P, I64, I64, P, P, P, P, P],
                "binade_r4_gemm": [P, P, I64, I64, P, I64, I32, P, I64, P],
                "binade_r4_gemm_noalloc": [P, P, I64, I64, P, I64, I32, P],
                "binade_bf16_gemm": [P, I64, I64, P, I64, I64, P, I64, I32, P, I64,
                                     P],
                "binade_r4_moe_gemv": [P, I32, P, I32, P, I64, I32, P, I32, P, P],
                "binade_bf16_moe_gemv": [P, I32, I64, I64, P, I32, P, I64, I32,
                                         P, I32, P, P],
            }
            for name, args in sig.items():
                if hasattr(L, name):
                    fn = getattr(L, name)
                    fn.argtypes = args
                    fn.restype = I32
            _lib = L
    return _lib


def _call(name: str, *args):
    rc = getattr(lib(), name)(*args)
    if rc != OK:
        raise BinadeError(name, rc, lib().binade_last_hip_error() if rc == EHIP else 0)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_stream(fn):
    """Run a device binding with `stream` as torch's current stream, so the
    temporaries it makes (contiguous copies, outputs, GEMM workspace) are
    allocated and filled in the same stream order as the kernel that uses
    them, and the caching allocator does not hand them to other streams while
    that kernel runs."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _bits16(t: torch.Tensor) -> torch.Tensor:
    """bf16 / int16 / uint16 tensor -> contiguous view of its 16-bit patterns"""
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16, torch.float16):
        raise TypeError(f"expected 16-bit weights, got {t.dtype}")
    return t.contiguous()


# ------------------------------------------------------------------ host
def build_table(w: torch.Tensor) -> Table:
    """binade_build_table on a host bf16 tensor."""
    w = _bits16(w)
    if w.is_cuda:
        raise ValueError("build_table runs on host memory")
    t = Table()
    _call("binade_build_table", _ptr(w), w.numel(), ctypes.byref(t))
    return t


def sizes_of(table: Table, rows: int, cols: int) -> Sizes:
    s = Sizes()
    _call("binade_sizes_of", ctypes.byref(table), rows, cols, ctypes.byref(s))
    return s


@dataclass
class RicePlanes:
    """Format 2 planes of one tensor (host or device tensors) + descriptor."""
    rows: int
    cols: int
    table: Table
    sm: torch.Tensor
    unary: torch.Tensor
    rem: torch.Tensor | None
    anchor: torch.Tensor
    esc_pre: torch.Tensor
    unary_bits: int
    n_esc: int

    @property
    def k(self) -> int:
        return int(self.table.k)

    def desc(self) -> RiceDesc:
        d = RiceDesc()
        d.rows, d.cols = self.rows, self.cols
        d.k, d.n = self.table.k, self.table.n
        ctypes.memmove(d.exp_of_rank, self.table.exp_of_rank, 256)
        d.sm = self.sm.data_ptr()
        d.unary = self.unary.data_ptr()
        d.unary_bits = self.unary_bits
        d.unary_words = self.unary.numel()
        d.rem = self.rem.data_ptr() if self.rem is not None else None
        d.rem_words = self.rem.numel() if self.rem is not None else 0
        d.anchor = self.anchor.data_ptr()
        d.esc_pre = self.esc_pre.data_ptr()
        d.n_esc = self.n_esc
        return d

    def to(self, device) -> "RicePlanes":
        mv = lambda t: None if t is None else t.to(device, non_blocking=False)
        return RicePlanes(self.rows, self.cols, self.table, mv(self.sm),
                          mv(self.unary), mv(self.rem), mv(self.anchor),
                          mv(self.esc_pre), self.unary_bits, self.n_esc)

    def nbytes(self) -> dict:
        """Bytes of each plane as stored (padding words included)."""
        return {"sm": self.sm.numel(), "unary": 4 * self.unary.numel(),
                "rem": 0 if self.rem is None else 4 * self.rem.numel(),
                "anchor": 8 * self.anchor.numel(),
                "esc_pre": 4 * self.esc_pre.numel()}

    def bits_per_weight(self) -> float:
        n = self.rows * self.cols
        bits = 8 * n + self.unary_bits + self.k * n + 96 * (self.anchor.numel() - 1)
        return bits / n


def pack_rice(w: torch.Tensor, table: Table | None = None) -> RicePlanes:
    """binade_pack_rice: host bf16 [rows, cols] -> host format 2 planes."""
    w = _bits16(w)
    if w.is_cuda or w.dim() != 2:
        raise ValueError("pack_rice takes a 2-D host tensor")
    rows, cols = w.shape
    if table is None:
        table = build_table(w)
    s = sizes_of(table, rows, cols)
    sm = torch.empty(rows, cols, dtype=torch.uint8)
    unary = torch.empty(int(s.unary_words), dtype=torch.int32)
    rem = torch.empty(int(s.rem_words), dtype=torch.int32) if table.k > 0 else None
    anchor = torch.empty(int(s.n_chunks) + 1, dtype=torch.int64)
    esc_pre = torch.empty(int(s.n_chunks) + 1, dtype=torch.int32)
    planes = RicePlanes(rows, cols, table, sm, unary, rem, anchor, esc_pre, 0, 0)
    d = planes.desc()
    _call("binade_pack_rice", _ptr(w), rows, cols, ctypes.byref(table), ctypes.byref(d))
    planes.unary_bits = int(d.unary_bits)
    planes.n_esc = int(d.n_esc)
    return planes


def build_table_gpu(w: torch.Tensor, workspace: torch.Tensor | None = None,
                    stream=None) -> Table:
    """binade_build_table_gpu on a device bf16 tensor; the table is copied
    back to the host (one synchronisation)."""
    w = _bits16(w)
    if not w.is_cuda:
        raise ValueError("build_table_gpu takes a device tensor")
    if workspace is None:
        workspace = torch.empty(2048, dtype=torch.uint8, device=w.device)
    dt = torch.empty(ctypes.sizeof(Table), dtype=torch.uint8, device=w.device)
    s = torch.cuda.current_stream(w.device) if stream is None else stream
    with torch.cuda.stream(s):
        _call("binade_build_table_gpu", _ptr(w), w.numel(), _ptr(workspace), _ptr(dt),
              _stream(s))
        host = dt.cpu()
    t = Table()
    ctypes.memmove(ctypes.addressof(t), host.numpy().ctypes.data, ctypes.sizeof(Table))
    return t


def pack_rice_gpu(w: torch.Tensor, table: Table | None = None, status: torch.Tensor | None = None,
                  stream=None) -> RicePlanes:
    """binade_pack_rice_gpu: device bf16 [rows, cols] -> device format 2
    planes, byte-identical to pack_rice; the table is built on the device
    when not given."""
    w = _bits16(w)
    if not w.is_cuda or w.dim() != 2:
        raise ValueError("pack_rice_gpu takes a 2-D device tensor")
    rows, cols = w.shape
    dev = w.device
    s = torch.cuda.current_stream(dev) if stream is None else stream
    ws_bytes = int(lib().binade_pack_gpu_workspace_bytes(rows, cols))
    with torch.cuda.stream(s):
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if table is None:
            table = build_table_gpu(w, ws, stream=s)
        sz = sizes_of(table, rows, cols)
        sm = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
        unary = torch.empty(int(sz.unary_words), dtype=torch.int32, device=dev)
        rem = (torch.empty(int(sz.rem_words), dtype=torch.int32, device=dev)
               if table.k > 0 else None)
        anchor = torch.empty(int(sz.n_chunks) + 1, dtype=torch.int64, device=dev)
        esc_pre = torch.empty(int(sz.n_chunks) + 1, dtype=torch.int32, device=dev)
        planes = RicePlanes(rows, cols, table, sm, unary, rem, anchor, esc_pre, 0, 0)
        d = planes.desc()
        _call("binade_pack_rice_gpu", _ptr(w), rows, cols, ctypes.byref(table), ctypes.byref(d),
              _ptr(ws), _ptr(status), _stream(s))
        ws.record_stream(s)
    planes.unary_bits = int(d.unary_bits)
    planes.n_esc = int(d.n_esc)
    return planes


@dataclass
class HuffPlanes:
    """Huffman comparison-codec planes (host or device tensors)."""
    n: int
    len: bytes
    sm: torch.Tensor
    stream: torch.Tensor
    stream_bytes: int
    block_len: torch.Tensor
    group_off: torch.Tensor

    def desc(self) -> HuffDesc:
        d = HuffDesc()
        d.n = self.n
        ctypes.memmove(d.len, self.len, 256)
        d.sm = self.sm.data_ptr()
        d.stream = self.stream.data_ptr()
        d.stream_bytes = self.stream_bytes
        d.stream_cap = self.stream.numel()
        d.block_len = self.block_len.data_ptr()
        d.group_off = self.group_off.data_ptr()
        return d

    def to(self, device) -> "HuffPlanes":
        return HuffPlanes(self.n, self.len, self.sm.to(device), self.stream.to(device),
                          self.stream_bytes, self.block_len.to(device), self.group_off.to(device))

    def bits_per_weight(self) -> float:
        return (8 * self.n + 8 * self.stream_bytes + 8 * self.block_len.numel()
                + 64 * self.group_off.numel()) / self.n


def pack_huff(w: torch.Tensor) -> HuffPlanes:
    """binade_huff_lengths + binade_huff_pack on a host bf16 tensor."""
    w = _bits16(w).reshape(-1)
    if w.is_cuda:
        raise ValueError("pack_huff takes a host tensor")
    n = w.numel()
    ln = (ctypes.c_uint8 * 256)()
    cap = ctypes.c_uint64(0)
    _call("binade_huff_lengths", _ptr(w), n, ln, ctypes.byref(cap))
    nb = (n + 63) // 64
    planes = HuffPlanes(n, bytes(ln), torch.empty(n, dtype=torch.uint8),
                        torch.empty(int(cap.value), dtype=torch.uint8), 0,
                        torch.empty(nb, dtype=torch.uint8),
                        torch.empty((nb + 127) // 128 + 1, dtype=torch.int64))
    d = planes.desc()
    _call("binade_huff_pack", _ptr(w), ctypes.byref(d))
    planes.stream_bytes = int(d.stream_bytes)
    return planes


@_on_stream
def huff_decode(p: HuffPlanes, out: torch.Tensor | None = None, status: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """binade_huff_decode: device planes -> bf16[n]."""
    dev = p.sm.device
    if out is None:
        out = torch.empty(p.n, dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().binade_huff_workspace_bytes()), dtype=torch.uint8,
                                device=dev)
    d = p.desc()
    _call("binade_huff_decode", ctypes.byref(d), _ptr(out), _ptr(workspace), _ptr(status),
          _stream(stream))
    return out


@dataclass
class F1Planes:
    """Format 1 planes of one tensor (host or device tensors) + descriptor."""
    rows: int
    cols: int
    table: Table
    sm: torch.Tensor
    width: torch.Tensor
    codes: torch.Tensor
    esc_rank: torch.Tensor
    anchor: torch.Tensor
    f1_pre: torch.Tensor
    esc_pre: torch.Tensor
    code_bits: int
    n_f1esc: int
    n_esc: int

    def desc(self) -> F1Desc:
        d = F1Desc()
        d.rows, d.cols, d.n = self.rows, self.cols, self.table.n
        ctypes.memmove(d.exp_of_rank, self.table.exp_of_rank, 256)
        d.sm = self.sm.data_ptr()
        d.width = self.width.data_ptr()
        d.codes = self.codes.data_ptr()
        d.code_bits = self.code_bits
        d.code_words = self.codes.numel()
        d.esc_rank = self.esc_rank.data_ptr()
        d.n_f1esc = self.n_f1esc
        d.esc_cap = self.esc_rank.numel()
        d.anchor = self.anchor.data_ptr()
        d.f1_pre = self.f1_pre.data_ptr()
        d.esc_pre = self.esc_pre.data_ptr()
        d.n_esc = self.n_esc
        return d

    def to(self, device) -> "F1Planes":
        """The planes on `device`; the code and escape planes trimmed to what
        the tensor uses (plus a padding word)."""
        cw = (self.code_bits + 31) // 32 + 2
        mv = lambda t: t.to(device, non_blocking=False)
        return F1Planes(self.rows, self.cols, self.table, mv(self.sm), mv(self.width),
                        mv(self.codes[:cw]), mv(self.esc_rank[: max(self.n_f1esc, 1)]),
                        mv(self.anchor), mv(self.f1_pre), mv(self.esc_pre),
                        self.code_bits, self.n_f1esc, self.n_esc)

    def bits_per_weight(self) -> float:
        """Format 1 as stored: sm byte, codes, escape bytes, a width byte per
        tile and 16 index bytes per row-chunk."""
        n = self.rows * self.cols
        bits = (8 * n + self.code_bits + 8 * self.n_f1esc + 8 * self.width.numel()
                + 128 * self.anchor.numel())
        return bits / n


def pack_f1(w: torch.Tensor, table: Table | None = None) -> F1Planes:
    """binade_pack_f1: host bf16 [rows, cols] -> host format 1 planes."""
    w = _bits16(w)
    if w.is_cuda or w.dim() != 2:
        raise ValueError("pack_f1 takes a 2-D host tensor")
    rows, cols = w.shape
    if table is None:
        table = build_table(w)
    s = F1Sizes()
    _call("binade_f1_sizes_of", rows, cols, ctypes.byref(s))
    planes = F1Planes(rows, cols, table, torch.empty(rows, cols, dtype=torch.uint8),
                      torch.empty(int(s.n_tiles), dtype=torch.uint8),
                      torch.empty(int(s.code_words), dtype=torch.int32),
                      torch.empty(int(s.esc_cap), dtype=torch.uint8),
                      torch.empty(int(s.n_chunks) + 1, dtype=torch.int64),
                      torch.empty(int(s.n_chunks) + 1, dtype=torch.int32),
                      torch.empty(int(s.n_chunks) + 1, dtype=torch.int32), 0, 0, 0)
    d = planes.desc()
    _call("binade_pack_f1", _ptr(w), rows, cols, ctypes.byref(table), ctypes.byref(d))
    planes.code_bits = int(d.code_bits)
    planes.n_f1esc = int(d.n_f1esc)
    planes.n_esc = int(d.n_esc)
    return planes


# ------------------------------------------------------------------ device
@dataclass
class R4Tensor:
    """R4 weights on the device. sm and esc_pre are the format 2 planes'."""
    rows: int
    cols: int
    lut: bytes
    sm: torch.Tensor
    nib: torch.Tensor
    esc_pre: torch.Tensor
    esc: torch.Tensor
    n_esc: int
    _keep: list = field(default_factory=list, repr=False)

    def desc(self) -> R4Desc:
        """The C descriptor (built once; the tensors must not be replaced)."""
        d = getattr(self, "_desc", None)
        if d is None or d.lut[:] != list(self.lut):
            d = R4Desc()
            d.rows, d.cols = self.rows, self.cols
            ctypes.memmove(d.lut, self.lut, 16)
            d.sm = self.sm.data_ptr()
            d.nib = self.nib.data_ptr()
            d.esc_pre = self.esc_pre.data_ptr()
            d.esc = self.esc.data_ptr() if self.n_esc > 0 else None
            d.n_esc = self.n_esc
            self._desc = d
        return d

    def nbytes(self) -> int:
        return (self.sm.numel() + self.nib.numel() + 4 * self.esc_pre.numel()
                + 4 * self.n_esc)

    def bits_per_weight(self) -> float:
        return 8.0 * self.nbytes() / (self.rows * self.cols)


def r4_from_planes(rows, cols, lut, sm, nib, esc_pre, esc) -> R4Tensor:
    """Wrap R4 planes that are already on the device."""
    return R4Tensor(rows, cols, bytes(bytearray(lut)), sm, nib, esc_pre, esc,
                    int(esc.numel()))


@_on_stream
def rice_to_r4(planes: RicePlanes, status: torch.Tensor | None = None,
               stream=None, out: R4Tensor | None = None) -> R4Tensor:
    """binade_rice_to_r4 on device planes; allocates nib / esc unless `out`."""
    if not planes.sm.is_cuda:
        raise ValueError("rice_to_r4 takes device planes (RicePlanes.to('cuda'))")
    dev = planes.sm.device
    if out is None:
        nib = torch.empty(planes.rows * planes.cols // 2, dtype=torch.uint8, device=dev)
        esc = torch.empty(max(planes.n_esc, 1), dtype=torch.int32, device=dev)
    else:
        nib, esc = out.nib, out.esc
    d_in = planes.desc()
    d_out = R4Desc()
    d_out.nib = nib.data_ptr()
    d_out.esc = esc.data_ptr()
    _call("binade_rice_to_r4", ctypes.byref(d_in), ctypes.byref(d_out),
          _ptr(status), _stream(stream))
    lut = bytes(d_out.lut)
    if out is not None:
        out.lut = lut
        return out
    return R4Tensor(planes.rows, planes.cols, lut, planes.sm, nib,
                    planes.esc_pre, esc, planes.n_esc)


@_on_stream
def f1_to_r4(planes: F1Planes, status: torch.Tensor | None = None,
             stream=None, out: R4Tensor | None = None) -> R4Tensor:
    """binade_f1_to_r4 on device planes; allocates nib / esc unless `out`."""
    if not planes.sm.is_cuda:
        raise ValueError("f1_to_r4 takes device planes (F1Planes.to('cuda'))")
    dev = planes.sm.device
    if out is None:
        nib = torch.empty(planes.rows * planes.cols // 2, dtype=torch.uint8, device=dev)
        esc = torch.empty(max(planes.n_esc, 1), dtype=torch.int32, device=dev)
    else:
        nib, esc = out.nib, out.esc
    d_in = planes.desc()
    d_out = R4Desc()
    d_out.nib = nib.data_ptr()
    d_out.esc = esc.data_ptr()
    _call("binade_f1_to_r4", ctypes.byref(d_in), ctypes.byref(d_out),
          _ptr(status), _stream(stream))
    lut = bytes(d_out.lut)
    if out is not None:
        out.lut = lut
        return out
    return R4Tensor(planes.rows, planes.cols, lut, planes.sm, nib,
                    planes.esc_pre, esc, planes.n_esc)


def _r4_out(p) -> "R4Tensor":
    """Device buffers for the R4 form of format 2 tensor p."""
    dev = p.sm.device
    return R4Tensor(p.rows, p.cols, bytes(16), p.sm,
                    torch.empty(p.rows * p.cols // 2, dtype=torch.uint8, device=dev),
                    p.esc_pre,
                    torch.empty(max(p.n_esc, 1), dtype=torch.int32, device=dev),
                    p.n_esc)


@_on_stream
def rice_to_r4_batch(planes: list, status: torch.Tensor | None = None,
                     stream=None, outs: list | None = None) -> list:
    """binade_rice_to_r4_batch: decode several tensors (up to 16 per launch)."""
    n = len(planes)
    if outs is None:
        outs = [_r4_out(p) for p in planes]
    din = (RiceDesc * n)(*[p.desc() for p in planes])
    dout = (R4Desc * n)()
    for i, o in enumerate(outs):
        dout[i].nib = o.nib.data_ptr()
        dout[i].esc = o.esc.data_ptr()
    _call("binade_rice_to_r4_batch", din, dout, n, _ptr(status), _stream(stream))
    for i, o in enumerate(outs):
        o.lut = bytes(dout[i].lut)
    return outs


class RicePlan:
    """A decode plan over format 2 tensors (binade_rice_to_r4_plan): their R4
    outputs, the plan's host bytes and its copy in device memory. run()
    decodes every tensor in one launch (binade_rice_to_r4_run). The plan
    keeps references to the planes and outputs whose addresses it holds."""

    def __init__(self, planes: list, outs: list | None = None):
        n = len(planes)
        self.planes = list(planes)
        self.outs = [_r4_out(p) for p in planes] if outs is None else list(outs)
        din = (RiceDesc * n)(*[p.desc() for p in planes])
        dout = (R4Desc * n)()
        for i, o in enumerate(self.outs):
            dout[i].nib = o.nib.data_ptr()
            dout[i].esc = o.esc.data_ptr()
        nbytes = lib().binade_rice_plan_bytes(n)
        if nbytes < 0:
            raise BinadeError("binade_rice_plan_bytes", int(nbytes), 0)
        self.host = (ctypes.c_uint8 * nbytes)()
        _call("binade_rice_to_r4_plan", din, dout, n, self.host, nbytes)
        for i, o in enumerate(self.outs):
            o.lut = bytes(dout[i].lut)
        device = planes[0].sm.device if n else torch.device("cpu")   # an empty plan never launches
        self.dev = torch.frombuffer(bytearray(self.host), dtype=torch.uint8).to(device)

    @_on_stream
    def run(self, status: torch.Tensor | None = None, stream=None) -> list:
        _call("binade_rice_to_r4_run", self.host, ctypes.c_void_p(self.dev.data_ptr()),
              _ptr(status), _stream(stream))
        return self.outs


@_on_stream
def r4_gemv_batch(ws: list, xs: list, out_dtype=torch.float32,
                  ys: list | None = None, stream=None) -> list:
    """binade_r4_gemv_batch: several independent R4 GEMVs in one launch."""
    code = _dtype_code(out_dtype)
    n = len(ws)
    if ys is None:
        ys = [_y((w.rows,), code, x.device, None) for w, x in zip(ws, xs)]
    dws = (R4Desc * n)(*[w.desc() for w in ws])
    dxs = (ctypes.c_void_p * n)(*[_bits16(x).data_ptr() for x in xs])
    dys = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    _call("binade_r4_gemv_batch", dws, dxs, dys, n, code, _stream(stream))
    return ys


@_on_stream
def bf16_gemv_batch(ws: list, xs: list, out_dtype=torch.float32,
                    ys: list | None = None, stream=None) -> list:
    """binade_bf16_gemv_batch: the batched twin."""
    code = _dtype_code(out_dtype)
    n = len(ws)
    ws = [_bits16(w) for w in ws]
    if ys is None:
        ys = [_y((w.shape[0],), code, x.device, None) for w, x in zip(ws, xs)]
    dws = (ctypes.c_void_p * n)(*[w.data_ptr() for w in ws])
    rows = (ctypes.c_int64 * n)(*[w.shape[0] for w in ws])
    cols = (ctypes.c_int64 * n)(*[w.shape[1] for w in ws])
    dxs = (ctypes.c_void_p * n)(*[_bits16(x).data_ptr() for x in xs])
    dys = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    _call("binade_bf16_gemv_batch", dws, rows, cols, dxs, dys, n, code, _stream(stream))
    return ys


def _y(rows_shape, y_dtype, device, y):
    if y is not None:
        return y
    dt = torch.float32 if y_dtype == F32 else torch.bfloat16
    return torch.empty(rows_shape, dtype=dt, device=device)


def _dtype_code(out_dtype) -> int:
    if out_dtype in (torch.float32, F32, "f32"):
        return F32
    if out_dtype in (torch.bfloat16, BF16, "bf16"):
        return BF16
    raise ValueError(out_dtype)


@_on_stream
def r4_gemv(w: R4Tensor, x: torch.Tensor, out_dtype=torch.float32,
            y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    code = _dtype_code(out_dtype)
    x = _bits16(x)
    y = _y((w.rows,), code, x.device, y)
    d = w.desc()
    _call("binade_r4_gemv", ctypes.byref(d), _ptr(x), _ptr(y), code, _stream(stream))
    return y


@_on_stream
def bf16_gemv(w: torch.Tensor, x: torch.Tensor, out_dtype=torch.float32,
              y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    code = _dtype_code(out_dtype)
    w = _bits16(w)
    x = _bits16(x)
    rows, cols = w.shape
    y = _y((rows,), code, x.device, y)
    _call("binade_bf16_gemv", _ptr(w), rows, cols, _ptr(x), _ptr(y), code,
          _stream(stream))
    return y


@_on_stream
def r4_gemv_rows(w: R4Tensor, x: torch.Tensor, out_dtype=torch.float32,
                 y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """binade_r4_gemv_rows: Y[b] = W x[b] for the 1..8 rows of x [m, K]; each
    row bit-identical to r4_gemv of that row."""
    code = _dtype_code(out_dtype)
    x = _bits16(x)
    m = x.shape[0]
    y = _y((m, w.rows), code, x.device, y)
    d = w.desc()
    _call("binade_r4_gemv_rows", ctypes.byref(d), _ptr(x), x.shape[1], m, _ptr(y),
          y.shape[1], code, _stream(stream))
    return y


@_on_stream
def bf16_gemv_rows(w: torch.Tensor, x: torch.Tensor, out_dtype=torch.float32,
                   y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """binade_bf16_gemv_rows: the twin of r4_gemv_rows."""
    code = _dtype_code(out_dtype)
    w = _bits16(w)
    x = _bits16(x)
    rows, cols = w.shape
    m = x.shape[0]
    y = _y((m, rows), code, x.device, y)
    _call("binade_bf16_gemv_rows", _ptr(w), rows, cols, _ptr(x), x.shape[1], m, _ptr(y),
          y.shape[1], code, _stream(stream))
    return y


@_on_stream
def moe_silu_mul(gate: torch.Tensor, up: torch.Tensor, out_dtype=torch.bfloat16,
                 h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """binade_moe_silu_mul: h = silu(gate) * up (fp64 inside, one rounding)."""
    code = _dtype_code(out_dtype)
    if gate.dtype != torch.float32 or up.dtype != torch.float32 or gate.shape != up.shape:
        raise ValueError("gate and up: fp32 tensors of one shape")
    gate = gate.contiguous()
    up = up.contiguous()
    h = _y(tuple(gate.shape), code, gate.device, h)
    _call("binade_moe_silu_mul", _ptr(gate), _ptr(up), gate.numel(), _ptr(h), code,
          _stream(stream))
    return h


@_on_stream
def moe_combine(y: torch.Tensor, weights: torch.Tensor, top_k: int, out_dtype=torch.float32,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """binade_moe_combine: out[t] = sum over the token's top_k slots of
    weight * y, an fp32 fma chain in slot order."""
    code = _dtype_code(out_dtype)
    if y.dtype != torch.float32 or weights.dtype != torch.float32:
        raise ValueError("y and weights: fp32")
    y = y.contiguous()
    weights = weights.contiguous()
    pairs, n = y.shape
    if pairs % top_k or weights.numel() != pairs:
        raise ValueError("y rows and weights must be n_tokens * top_k")
    out = _y((pairs // top_k, n), code, y.device, out)
    _call("binade_moe_combine", _ptr(y), _ptr(weights), pairs // top_k, top_k, n, _ptr(out),
          code, _stream(stream))
    return out


@_on_stream
def unpack(w: R4Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device=w.nib.device)
    d = w.desc()
    _call("binade_unpack", ctypes.byref(d), _ptr(out), _stream(stream))
    return out


def gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    """Bytes of workspace with which an M x N x K GEMM splits its slices
    over blocks (0: it never does)."""
    return int(lib().binade_gemm_workspace_bytes(m, n, k))


def _workspace(m, n, k, device, workspace):
    if workspace is None:
        nb = gemm_workspace_bytes(m, n, k)
        if nb == 0:
            return None, 0
        workspace = torch.empty(nb, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


@_on_stream
def r4_gemm(w: R4Tensor, x: torch.Tensor, out_dtype=torch.float32,
            y: torch.Tensor | None = None, stream=None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W^T. workspace: optional device buffer (a fresh one of
    gemm_workspace_bytes is taken from torch's allocator when None)."""
    code = _dtype_code(out_dtype)
    x = _bits16(x)
    m = x.shape[0]
    y = _y((m, w.rows), code, x.device, y)
    ws, nb = _workspace(m, w.rows, w.cols, x.device, workspace)
    d = w.desc()
    _call("binade_r4_gemm", ctypes.byref(d), _ptr(x), m, x.stride(0), _ptr(y),
          y.stride(0), code, _ptr(ws), nb, _stream(stream))
    return y


@_on_stream
def r4_gemm_noalloc(w: R4Tensor, x: torch.Tensor, out_dtype=torch.float32,
                    y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X W^T through binade_r4_gemm_noalloc (the library's fixed scratch,
    no workspace). With y given, nothing is allocated here either."""
    code = _dtype_code(out_dtype)
    x = _bits16(x)
    m = x.shape[0]
    y = _y((m, w.rows), code, x.device, y)
    d = w.desc()
    _call("binade_r4_gemm_noalloc", ctypes.byref(d), _ptr(x), m, x.stride(0),
          _ptr(y), y.stride(0), code, _stream(stream))
    return y


def gemm_scratch_bytes() -> int:
    return int(lib().binade_gemm_scratch_bytes())


@_on_stream
def bf16_gemm(w: torch.Tensor, x: torch.Tensor, out_dtype=torch.float32,
              y: torch.Tensor | None = None, stream=None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    code = _dtype_code(out_dtype)
    w = _bits16(w)
    x = _bits16(x)
    rows, cols = w.shape
    m = x.shape[0]
    y = _y((m, rows), code, x.device, y)
    ws, nb = _workspace(m, rows, cols, x.device, workspace)
    _call("binade_bf16_gemm", _ptr(w), rows, cols, _ptr(x), m, x.stride(0),
          _ptr(y), y.stride(0), code, _ptr(ws), nb, _stream(stream))
    return y


@_on_stream
def r4_moe_gemv(experts: R4Tensor, n_experts: int, x: torch.Tensor,
                idx: torch.Tensor, x_per_slot: bool = False,
                out_dtype=torch.float32, y: torch.Tensor | None = None,
                status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    code = _dtype_code(out_dtype)
    x = _bits16(x)
    idx = idx.contiguous()
    n_tokens, top_k = idx.shape
    N = experts.rows // n_experts
    y = _y((n_tokens * top_k, N), code, x.device, y)
    d = experts.desc()
    _call("binade_r4_moe_gemv", ctypes.byref(d), n_experts, _ptr(x),
          1 if x_per_slot else 0, _ptr(idx), n_tokens, top_k, _ptr(y), code,
          _ptr(status), _stream(stream))
    return y


@_on_stream
def bf16_moe_gemv(experts: torch.Tensor, n_experts: int, x: torch.Tensor,
                  idx: torch.Tensor, x_per_slot: bool = False,
                  out_dtype=torch.float32, y: torch.Tensor | None = None,
                  status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    code = _dtype_code(out_dtype)
    experts = _bits16(experts)
    x = _bits16(x)
    idx = idx.contiguous()
    rows, cols = experts.shape
    N = rows // n_experts
    n_tokens, top_k = idx.shape
    y = _y((n_tokens * top_k, N), code, x.device, y)
    _call("binade_bf16_moe_gemv", _ptr(experts), n_experts, N, cols, _ptr(x),
          1 if x_per_slot else 0, _ptr(idx), n_tokens, top_k, _ptr(y), code,
          _ptr(status), _stream(stream))
    return y
