"""binade_r4_gemm_noalloc (the GEMM entry point for callers that cannot
allocate) against binade_r4_gemm with a caller workspace, through the C ABI:
two calls in a row, the second smaller, both splitting their slices into the
library's fixed scratch; and a shape whose partial sums exceed the scratch,
which is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

from decode_gemv_tensor_amd import binade as B

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _r4(n, k, seed):
    g = torch.Generator().manual_seed(seed)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    return B.rice_to_r4(B.pack_rice(w).to(DEV))


def _x(m, k, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(m, k, generator=g).to(torch.bfloat16).to(DEV)


def _noalloc(r4, x, y, code):
    d = r4.desc()
    stream = torch.cuda.current_stream().cuda_stream
    return B.lib().binade_r4_gemm_noalloc(ctypes.byref(d), B._ptr(x), x.shape[0], x.stride(0),
                                          B._ptr(y), y.stride(0), code, ctypes.c_void_p(stream))


def test_noalloc_equals_workspace_gemm_on_two_calls():
    scratch = B.gemm_scratch_bytes()
    assert scratch == 32 << 20
    cases = [(64, 1024, 3840, torch.float32), (16, 512, 2048, torch.bfloat16)]  # second is smaller
    for m, n, k, dt in cases:
        need = B.gemm_workspace_bytes(m, n, k)
        assert 0 < need <= scratch, (m, n, k, need)  # the split path, through the scratch
        print("noalloc", m, n, k, dt, need, flush=True)
        r4 = _r4(n, k, seed=n + k)
        x = _x(m, k, seed=m)
        code = 1 if dt == torch.bfloat16 else 0
        y = torch.full((m, n), float("nan"), dtype=dt, device=DEV)
        assert _noalloc(r4, x, y, code) == B.OK
        ref = B.r4_gemm(r4, x, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), (m, n, k)


def test_noalloc_refuses_partials_beyond_the_scratch():
    m, n, k = 512, 8320, 1056
    need = B.gemm_workspace_bytes(m, n, k)
    assert need > B.gemm_scratch_bytes()
    r4 = _r4(n, k, seed=3)
    x = _x(m, k, seed=4)
    y = torch.full((m, n), 7.0, dtype=torch.float32, device=DEV)
    assert _noalloc(r4, x, y, 0) == B.ENOSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))  # nothing was launched
