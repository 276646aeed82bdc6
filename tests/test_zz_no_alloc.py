"""aqlm_gemv_packed_noalloc (scratch in the library's fixed device array) against
aqlm_gemv_packed (caller's workspace), through the C ABI: two calls in a row on one
GPU, the second with a smaller input, each equal bit for bit to the workspace call
(same kernels, same summation order) and within the oracle bar (max_o |y - y_ref| /
(max_o |y_ref| + 1e-6) <= 2e-3 per token; the product of page "AQLM (Additive
Quantization for LLMs)", section "Niveau intermediaire")."""
import ctypes

import numpy as np
import pytest

from additive_quantized_gemv_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3

# (out, in, K, B, batch): a larger call, then a smaller one
SEQUENCES = [
    [(11008, 4096, 1, 16, 1), (4096, 4096, 1, 16, 1)],      # split kernel (1x16)
    [(4096, 11008, 2, 8, 1), (1000, 4096, 2, 8, 1)],        # lookup tables on code tiles (2x8)
    [(2000, 4096, 1, 16, 4), (300, 1024, 1, 16, 2)],        # split kernel, several tokens
    [(1500, 4096, 1, 16, 12), (200, 2048, 1, 16, 6)],       # split on the matrix cores
]


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import additive_quantized_gemv_amd as aq
    lib = aq._load()
    lib.aqlm_gemv_packed_noalloc.argtypes = [ctypes.c_void_p] * 4 + [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.aqlm_gemv_packed_noalloc.restype = ctypes.c_int
    lib.aqlm_noalloc_scratch_bytes.argtypes = []
    lib.aqlm_noalloc_scratch_bytes.restype = ctypes.c_int64
    return aq


def _rel_err(y, yref):
    return np.max(np.abs(y - yref), axis=1) / (np.max(np.abs(yref), axis=1) + 1e-6)


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-then-".join("x".join(map(str, c)) for c in s))
def test_noalloc_matches_workspace_call(aq, orc, seq):
    import torch
    lib = aq._load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i, (out, in_, K, B, batch) in enumerate(seq):
        print(f"noalloc case {out}x{in_} {K}x{B} b{batch}", flush=True)
        p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=3500 + 7 * i + out)
        codes = p["codes"].view(np.int16) if B == 16 else p["codes"]
        ct = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
        cbt = torch.from_numpy(np.ascontiguousarray(p["codebooks"])).cuda()
        xt = torch.from_numpy(np.ascontiguousarray(p["x"])).cuda()
        W = aq.pack_weights(ct, cbt)
        need = aq.packed_workspace_bytes(W, xt)
        assert 0 < need <= lib.aqlm_noalloc_scratch_bytes()
        y_ws = aq.gemv_packed(W, xt)
        y_na = torch.full_like(y_ws, 7.0)
        st = lib.aqlm_gemv_packed_noalloc(W.codes.data_ptr(), W.codebooks.data_ptr(), xt.data_ptr(),
                                          y_na.data_ptr(), out, in_, K, B, batch, stream)
        assert st == 0, lib.aqlm_last_error()
        torch.cuda.synchronize()
        assert bool((y_na == y_ws).all()), f"{out}x{in_} b{batch}: differs from aqlm_gemv_packed"
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
        e = _rel_err(y_na.float().cpu().numpy().astype(np.float64), yref)
        assert np.all(e <= TOL), f"{out}x{in_} b{batch}: {e.max():.3e}"


def test_noalloc_rejects_beyond_scratch(aq):
    """A call whose scratch need exceeds the fixed array is refused before any device
    work (here: packed 2x8 code tiles above batch 1 are unpacked into the scratch,
    58.7 MB for 28672 x 8192)."""
    import torch
    lib = aq._load()
    out, in_, batch = 28672, 8192, 2
    codes = torch.empty(aq.packed_codes_bytes(out, in_, 2, 8), dtype=torch.uint8, device="cuda")
    cb = torch.empty((2, 8, 256), dtype=torch.float16, device="cuda")
    x = torch.empty((batch, in_), dtype=torch.float16, device="cuda")
    y = torch.full((batch, out), 3.0, dtype=torch.float16, device="cuda")
    st = lib.aqlm_gemv_packed_noalloc(codes.data_ptr(), cb.data_ptr(), x.data_ptr(), y.data_ptr(),
                                      out, in_, 2, 8, batch, None)
    assert st == 1
    assert str(lib.aqlm_noalloc_scratch_bytes()).encode() in lib.aqlm_last_error()
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
