"""libaqlm_mi355x: additive-quantized GEMV / small-batch GEMM on MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/aqlm_mi355x.h``.  It
only marshals arguments -- every step of the product runs in the HIP kernels of
``libaqlm_mi355x.so``.  PyTorch supplies device memory and the current stream.
There is no CPU fallback: if the library is missing, importing the compute
functions raises.

Format (page "AQLM (Additive Quantization for LLMs)", section "Niveau
intermediaire"): codes [out][in/8][K] (uint8 for 8-bit codes, int16/uint16 bit
patterns for 16-bit codes), codebooks [K][2^B][8] fp16, x [batch][in] fp16,
y [batch][out] fp16.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gemv", "gemm", "gemv_variant", "gemv_packed", "pack_codebooks", "unpack_codebooks",
           "pack_codes", "unpack_codes", "packed_codes_bytes", "PackedWeights", "pack_weights",
           "gemv_grouped", "gemm_grouped", "gemv_packed_grouped",
           "dequantize", "bits_per_weight", "codes_bytes",
           "codebooks_bytes", "variant_supported", "selected_variant", "VARIANTS", "library_path",
           "AqlmError", "version", "workspace_bytes", "grouped_workspace_bytes", "OPS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libaqlm_mi355x.so")

VARIANTS = {"auto": 0, "generic": 1, "lds": 2, "lut": 3, "l2": 4, "mfma": 5, "split": 6,
            "prefill": 7}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error"}
OPS = {"gemv": 0, "gemm": 1, "gemv_packed": 2}


class AqlmError(RuntimeError):
    """A non-OK status from libaqlm_mi355x."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def library_path() -> str:
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run additive_quantized_gemv_amd/build.py "
                          "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    # codes, codebooks, x, y, out, in, K, B, batch, workspace, workspace_bytes, stream
    prod = [vp, vp, vp, vp, i64, i64, ci, ci, ci, vp, i64, vp]
    for name in ("aqlm_gemv", "aqlm_gemm", "aqlm_gemv_packed"):
        getattr(lib, name).argtypes = prod
        getattr(lib, name).restype = ci
    lib.aqlm_gemv_variant.argtypes = [ci] + prod
    lib.aqlm_gemv_variant.restype = ci
    lib.aqlm_variant_supported.argtypes = [ci, vp, vp, vp, vp, i64, i64, ci, ci, ci, i64]
    lib.aqlm_variant_supported.restype = ci
    lib.aqlm_selected_variant.argtypes = [ci, vp, vp, vp, vp, i64, i64, ci, ci, ci, i64]
    lib.aqlm_selected_variant.restype = ci
    lib.aqlm_workspace_bytes.argtypes = [ci, ci, vp, vp, vp, vp, i64, i64, ci, ci, ci]
    lib.aqlm_workspace_bytes.restype = i64
    lib.aqlm_grouped_workspace_bytes.argtypes = [ci, ci, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                 vp, ctypes.POINTER(vp), ctypes.POINTER(i64), i64,
                                                 ci, ci, ci]
    lib.aqlm_grouped_workspace_bytes.restype = i64
    grouped = [ci, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, ctypes.POINTER(vp),
               ctypes.POINTER(i64), i64, ci, ci, ci, vp, i64, vp]
    for name in ("aqlm_gemv_grouped", "aqlm_gemm_grouped", "aqlm_gemv_packed_grouped"):
        getattr(lib, name).argtypes = grouped
        getattr(lib, name).restype = ci
    lib.aqlm_packed_codes_bytes.argtypes = [i64, i64, ci, ci]
    lib.aqlm_packed_codes_bytes.restype = i64
    for name in ("aqlm_pack_codes", "aqlm_unpack_codes"):
        getattr(lib, name).argtypes = [vp, vp, i64, i64, ci, ci, vp]
        getattr(lib, name).restype = ci
    for name in ("aqlm_pack_codebooks", "aqlm_unpack_codebooks"):
        getattr(lib, name).argtypes = [vp, vp, ci, ci, vp]
        getattr(lib, name).restype = ci
    lib.aqlm_dequantize.argtypes = [vp, vp, vp, ci, i64, i64, ci, ci, vp]
    lib.aqlm_dequantize.restype = ci
    lib.aqlm_bits_per_weight.argtypes = [ci, ci, ci]
    lib.aqlm_bits_per_weight.restype = ctypes.c_double
    lib.aqlm_codes_bytes.argtypes = [i64, i64, ci, ci]
    lib.aqlm_codes_bytes.restype = i64
    lib.aqlm_codebooks_bytes.argtypes = [ci, ci]
    lib.aqlm_codebooks_bytes.restype = i64
    for name in ("aqlm_version", "aqlm_last_error"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = ctypes.c_char_p
    lib.aqlm_status_string.argtypes = [ci]
    lib.aqlm_status_string.restype = ctypes.c_char_p
    lib.aqlm_variant_name.argtypes = [ci]
    lib.aqlm_variant_name.restype = ctypes.c_char_p
    lib.aqlm_cpu_gemv.argtypes = [vp, vp, vp, vp, i64, i64, ci, ci, ci, ci]
    lib.aqlm_cpu_gemv.restype = ci
    lib.aqlm_cpu_isa.argtypes = []
    lib.aqlm_cpu_isa.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        lib = _load()
        detail = lib.aqlm_last_error().decode()
        raise AqlmError(status, f"{what}: {lib.aqlm_status_string(status).decode()}"
                                f"{' (' + detail + ')' if detail else ''}")


def _torch():
    import torch
    return torch


def _bits_of(codes) -> int:
    torch = _torch()
    if codes.dtype == torch.uint8:
        return 8
    if codes.dtype in (torch.int16, getattr(torch, "uint16", torch.int16)):
        return 16
    raise TypeError("codes must be uint8 (8-bit codes) or int16/uint16 (16-bit codes)")


def _prep(codes, codebooks, x, K, B, packed=False):
    torch = _torch()
    if codes.dim() != 3:
        raise ValueError("codes must be [out][in/8][K]")
    Bc = _bits_of(codes)
    K = codes.shape[2] if K is None else int(K)
    B = Bc if B is None else int(B)
    if B != Bc or K != codes.shape[2]:
        raise ValueError("K/B do not match the codes tensor")
    want = packed_codebooks_shape(K, B) if packed else (K, 1 << B, 8)
    if codebooks.dtype != torch.float16 or tuple(codebooks.shape) != want:
        raise ValueError(f"codebooks must be float16 {list(want)}")
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if x2.dim() != 2 or x2.shape[1] != codes.shape[1] * 8:
        raise ValueError("x must be [batch][in] with in = 8 * codes.shape[1]")
    for t, n in ((codes, "codes"), (codebooks, "codebooks"), (x2, "x")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    return K, B, x2


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes: int, device, workspace=None):
    """(pointer, size, holder) of the call's workspace: the caller's uint8 tensor; 0 for
    none (the library then runs the kernels that need no workspace); else a fresh one
    from torch's caching allocator on the current stream (a graph being captured takes
    it from its own pool, so replays keep a valid workspace).  The holder keeps the
    tensor alive across the launch call; the allocator's stream ordering keeps it from
    being reused before the kernels that use it have run."""
    torch = _torch()
    if nbytes < 0:
        raise ValueError("invalid arguments (workspace query failed)")
    if isinstance(workspace, int) and not isinstance(workspace, bool) and workspace == 0:
        return None, 0, None            # explicitly none: the kernels that need no workspace
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace of {workspace.numel()} bytes is smaller than the "
                             f"{nbytes} bytes this call needs")
        return workspace.data_ptr(), workspace.numel(), workspace
    if nbytes == 0:
        return None, 0, None
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t.data_ptr(), nbytes, t


def _product(fn_name, codes, codebooks, x, K=None, B=None, out=None, variant=None,
             workspace=None):
    torch = _torch()
    lib = _load()
    K, B, x2 = _prep(codes, codebooks, x, K, B)
    out_f, in_f, batch = codes.shape[0], codes.shape[1] * 8, x2.shape[0]
    y = out if out is not None else torch.empty((batch, out_f), dtype=torch.float16,
                                                 device=codes.device)
    if y.dtype != torch.float16 or tuple(y.shape) != (batch, out_f) or not y.is_contiguous():
        raise ValueError("out must be a contiguous float16 [batch][out] tensor")
    ptrs = (codes.data_ptr(), codebooks.data_ptr(), x2.data_ptr(), y.data_ptr(), out_f, in_f,
            K, B, batch)
    op = OPS["gemm"] if fn_name == "aqlm_gemm" else OPS["gemv"]
    v = 0 if variant is None else (VARIANTS[variant] if isinstance(variant, str) else int(variant))
    need = lib.aqlm_workspace_bytes(op, v, *ptrs)
    wp, wn, _keep = _workspace(need, codes.device, workspace)
    if variant is None:
        _check(getattr(lib, fn_name)(*ptrs, wp, wn, _stream()), fn_name)
    else:
        _check(lib.aqlm_gemv_variant(v, *ptrs, wp, wn, _stream()), f"aqlm_gemv_variant({variant})")
    return y if x.dim() == 2 else y[0]


def gemv(codes, codebooks, x, K=None, B=None, out=None, workspace=None):
    """y = W x (token generation path: gather / lookup-table kernels).  ``workspace``: an
    optional uint8 device tensor of at least workspace_bytes("gemv", ...) bytes; by
    default one is taken from torch's caching allocator for the call."""
    return _product("aqlm_gemv", codes, codebooks, x, K, B, out, workspace=workspace)


def gemm(codes, codebooks, x, K=None, B=None, out=None, workspace=None):
    """Y = X W^T; from batch 2 (4 for eight codebooks) decodes to fp16 and runs on the matrix cores."""
    return _product("aqlm_gemm", codes, codebooks, x, K, B, out, workspace=workspace)


class PackedWeights:
    """Codes and codebooks of one matrix in the packed layouts (pack_codes,
    pack_codebooks), with the shape they describe."""

    __slots__ = ("codes", "codebooks", "out_features", "in_features", "K", "B")

    def __init__(self, codes, codebooks, out_features, in_features, K, B):
        self.codes, self.codebooks = codes, codebooks
        self.out_features, self.in_features, self.K, self.B = out_features, in_features, K, B


def pack_weights(codes, codebooks) -> PackedWeights:
    """Packed copies of codes [out][in/8][K] and codebooks [K][2^B][8] (one-time layout change)."""
    K, B = codes.shape[2], _bits_of(codes)
    return PackedWeights(pack_codes(codes), pack_codebooks(codebooks), codes.shape[0],
                         codes.shape[1] * 8, K, B)


def gemv_packed(weights: PackedWeights, x, out=None, workspace=None):
    """y = W x from packed weights (aqlm_gemv_packed)."""
    torch = _torch()
    lib = _load()
    w = weights
    if w.codebooks.dtype != torch.float16 or tuple(w.codebooks.shape) != packed_codebooks_shape(w.K, w.B):
        raise ValueError(f"packed codebooks must be float16 {list(packed_codebooks_shape(w.K, w.B))}")
    if w.codes.numel() * w.codes.element_size() != packed_codes_bytes(w.out_features,
                                                                       w.in_features, w.K, w.B):
        raise ValueError("packed codes have the wrong size")
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if x2.dim() != 2 or x2.shape[1] != w.in_features:
        raise ValueError("x must be [batch][in_features]")
    for t, n in ((w.codes, "codes"), (w.codebooks, "codebooks"), (x2, "x")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    batch = x2.shape[0]
    y = out if out is not None else torch.empty((batch, w.out_features), dtype=torch.float16,
                                                 device=x2.device)
    if y.dtype != torch.float16 or tuple(y.shape) != (batch, w.out_features) or \
            not y.is_contiguous():
        raise ValueError("out must be a contiguous float16 [batch][out] tensor")
    ptrs = (w.codes.data_ptr(), w.codebooks.data_ptr(), x2.data_ptr(), y.data_ptr(),
            w.out_features, w.in_features, w.K, w.B, batch)
    need = lib.aqlm_workspace_bytes(OPS["gemv_packed"], 0, *ptrs)
    wp, wn, _keep = _workspace(need, x2.device, workspace)
    _check(lib.aqlm_gemv_packed(*ptrs, wp, wn, _stream()), "aqlm_gemv_packed")
    return y if x.dim() == 2 else y[0]


def _grouped(fn_name, codes, codebooks, x, out_features, in_features, K, B, outs,
             workspace=None):
    torch = _torch()
    lib = _load()
    n = len(codes)
    if n < 1 or n > 4 or len(codebooks) != n:
        raise ValueError("1 to 4 matrices, each with codes and codebooks")
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if x2.dim() != 2 or x2.shape[1] != in_features or not x2.is_cuda or not x2.is_contiguous():
        raise ValueError("x must be a contiguous device [batch][in] tensor")
    batch = x2.shape[0]
    ys = outs if outs is not None else [
        torch.empty((batch, o), dtype=torch.float16, device=x2.device) for o in out_features]
    for y, o in zip(ys, out_features):
        if y.dtype != torch.float16 or tuple(y.shape) != (batch, o) or not y.is_contiguous():
            raise ValueError("each out must be a contiguous float16 [batch][out] tensor")
    vp = ctypes.c_void_p
    arr = lambda ts: (vp * n)(*[t.data_ptr() for t in ts])
    outs_arr = (ctypes.c_int64 * n)(*out_features)
    op = {"aqlm_gemv_grouped": 0, "aqlm_gemm_grouped": 1, "aqlm_gemv_packed_grouped": 2}[fn_name]
    args = (arr(codes), arr(codebooks), x2.data_ptr(), arr(ys), outs_arr, in_features, K, B, batch)
    need = lib.aqlm_grouped_workspace_bytes(op, n, *args)
    wp, wn, _keep = _workspace(need, x2.device, workspace)
    _check(getattr(lib, fn_name)(n, *args, wp, wn, _stream()), fn_name)
    return ys if x.dim() == 2 else [y[0] for y in ys]


def _grouped_canonical(fn_name, codes, codebooks, x, out, workspace=None):
    K, B, x2 = _prep(codes[0], codebooks[0], x, None, None)
    for c, cb in zip(codes, codebooks):
        _prep(c, cb, x, K, B)
    return _grouped(fn_name, codes, codebooks, x, [c.shape[0] for c in codes],
                    codes[0].shape[1] * 8, K, B, out, workspace)


def gemv_grouped(codes, codebooks, x, out=None, workspace=None):
    """[W_m x for each m] in one launch: lists of codes and codebooks of matrices that share x."""
    return _grouped_canonical("aqlm_gemv_grouped", codes, codebooks, x, out, workspace)


def gemm_grouped(codes, codebooks, x, out=None, workspace=None):
    """gemv_grouped with the matrix-core kernels from batch 2 (as gemm)."""
    return _grouped_canonical("aqlm_gemm_grouped", codes, codebooks, x, out, workspace)


def cpu_gemv(codes, codebooks, x, out=None, threads: int = 0):
    """y = W x on the host cores from host (CPU) tensors, same layouts as gemv.

    Token generation without a GPU: lookup tables for 8-bit codes, F16C decode for
    16-bit codes, rows split over ``threads`` OpenMP threads (0: the OpenMP default);
    the result does not depend on the thread count.
    """
    torch = _torch()
    lib = _load()
    if codes.dim() != 3:
        raise ValueError("codes must be [out][in/8][K]")
    K, B = codes.shape[2], _bits_of(codes)
    if codebooks.dtype != torch.float16 or tuple(codebooks.shape) != (K, 1 << B, 8):
        raise ValueError(f"codebooks must be float16 {[K, 1 << B, 8]}")
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if x2.dim() != 2 or x2.shape[1] != codes.shape[1] * 8:
        raise ValueError("x must be [batch][in] with in = 8 * codes.shape[1]")
    for t, n in ((codes, "codes"), (codebooks, "codebooks"), (x2, "x")):
        if t.is_cuda:
            raise ValueError(f"{n} must be a host tensor")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    out_f, in_f, batch = codes.shape[0], codes.shape[1] * 8, x2.shape[0]
    y = out if out is not None else torch.empty((batch, out_f), dtype=torch.float16)
    if (y.dtype != torch.float16 or tuple(y.shape) != (batch, out_f) or not y.is_contiguous()
            or y.is_cuda):
        raise ValueError("out must be a contiguous float16 [batch][out] host tensor")
    _check(lib.aqlm_cpu_gemv(codes.data_ptr(), codebooks.data_ptr(), x2.data_ptr(), y.data_ptr(),
                             out_f, in_f, K, B, batch, int(threads)), "aqlm_cpu_gemv")
    return y if x.dim() == 2 else y[0]


def cpu_isa() -> str:
    """Vector instruction set the host kernel uses here ("avx512", "avx2" or "none")."""
    return _load().aqlm_cpu_isa().decode()


def gemv_packed_grouped(weights, x, out=None, workspace=None):
    """[W_m x for each m] in one launch from a list of PackedWeights that share x."""
    w0 = weights[0]
    for w in weights:
        if (w.in_features, w.K, w.B) != (w0.in_features, w0.K, w0.B):
            raise ValueError("grouped matrices must share in_features, K and B")
        if w.codes.numel() * w.codes.element_size() != packed_codes_bytes(
                w.out_features, w.in_features, w.K, w.B):
            raise ValueError("packed codes have the wrong size")
    return _grouped("aqlm_gemv_packed_grouped", [w.codes for w in weights],
                    [w.codebooks for w in weights], x, [w.out_features for w in weights],
                    w0.in_features, w0.K, w0.B, out, workspace)


def packed_codes_bytes(out_features, in_features, K, B) -> int:
    return int(_load().aqlm_packed_codes_bytes(out_features, in_features, K, B))


def pack_codes(codes, out=None):
    """Packed copy of codes [out][in/8][K] as a flat uint8 device tensor (aqlm_pack_codes)."""
    torch = _torch()
    lib = _load()
    if codes.dim() != 3 or not codes.is_cuda or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous device [out][in/8][K] tensor")
    B, K = _bits_of(codes), codes.shape[2]
    o, i = codes.shape[0], codes.shape[1] * 8
    n = packed_codes_bytes(o, i, K, B)
    if n < 0:
        raise ValueError("bad code shape")
    P = out if out is not None else torch.empty(n, dtype=torch.uint8, device=codes.device)
    if P.numel() * P.element_size() != n or not P.is_contiguous():
        raise ValueError(f"out must be a contiguous buffer of {n} bytes")
    _check(lib.aqlm_pack_codes(codes.data_ptr(), P.data_ptr(), o, i, K, B, _stream()),
           "aqlm_pack_codes")
    return P


def unpack_codes(packed, out_features, in_features, K, B):
    """Inverse of pack_codes: codes [out][in/8][K] (uint8 for B = 8, int16 for B = 16)."""
    torch = _torch()
    lib = _load()
    n = packed_codes_bytes(out_features, in_features, K, B)
    if n < 0 or packed.numel() * packed.element_size() != n or not packed.is_cuda \
            or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous device buffer of aqlm_packed_codes_bytes")
    dt = torch.uint8 if B == 8 else torch.int16
    C = torch.empty((out_features, in_features // 8, K), dtype=dt, device=packed.device)
    _check(lib.aqlm_unpack_codes(packed.data_ptr(), C.data_ptr(), out_features, in_features, K, B,
                                 _stream()), "aqlm_unpack_codes")
    return C


def packed_codebooks_shape(K: int, B: int) -> tuple:
    """Shape of pack_codebooks' result: [K][8][256] planes (B = 8) or [K][4][65536][2]
    position pairs (B = 16)."""
    return (K, 8, 256) if B == 8 else (K, 4, 1 << B, 2)


def pack_codebooks(codebooks, out=None):
    """Packed copy of codebooks [K][2^B][8] (a one-time weight layout change): for B = 8
    the planes P[k][t][c] = C[k][c][t]; for B = 16 the position pairs
    P[k][q][c][s] = C[k][c][2q + s]."""
    torch = _torch()
    lib = _load()
    K, E, g = codebooks.shape
    if codebooks.dtype != torch.float16 or g != 8 or E not in (256, 65536) or not codebooks.is_cuda \
            or not codebooks.is_contiguous():
        raise ValueError("codebooks must be a contiguous device float16 [K][2^B][8] tensor")
    P = out if out is not None else torch.empty(packed_codebooks_shape(K, E.bit_length() - 1),
                                                 dtype=torch.float16, device=codebooks.device)
    if P.dtype != torch.float16 or P.numel() != K * E * 8 or not P.is_contiguous():
        raise ValueError("out must be a contiguous float16 tensor of the codebooks' size")
    _check(lib.aqlm_pack_codebooks(codebooks.data_ptr(), P.data_ptr(), K, E.bit_length() - 1,
                                   _stream()), "aqlm_pack_codebooks")
    return P


def unpack_codebooks(packed, out=None):
    """Inverse of pack_codebooks: -> [K][2^B][8]."""
    torch = _torch()
    lib = _load()
    K = packed.shape[0]
    E = 256 if tuple(packed.shape) == (K, 8, 256) else 65536
    if packed.dtype != torch.float16 or tuple(packed.shape) != packed_codebooks_shape(K, E.bit_length() - 1) \
            or not packed.is_cuda or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous device float16 [K][8][256] or [K][4][65536][2] tensor")
    C = out if out is not None else torch.empty((K, E, 8), dtype=torch.float16,
                                                 device=packed.device)
    _check(lib.aqlm_unpack_codebooks(packed.data_ptr(), C.data_ptr(), K, E.bit_length() - 1,
                                     _stream()), "aqlm_unpack_codebooks")
    return C


def gemv_variant(variant, codes, codebooks, x, K=None, B=None, out=None, workspace=None):
    """The product with a named kernel variant ('generic', 'lds', 'lut', 'l2', 'mfma', ...)."""
    return _product(None, codes, codebooks, x, K, B, out, variant=variant, workspace=workspace)


def _query_args(codes, codebooks, x, K, B):
    torch = _torch()
    K, B, x2 = _prep(codes, codebooks, x, K, B)
    y = torch.empty((x2.shape[0], codes.shape[0]), dtype=torch.float16, device=codes.device)
    return (codes.data_ptr(), codebooks.data_ptr(), x2.data_ptr(), y.data_ptr(), codes.shape[0],
            codes.shape[1] * 8, K, B, x2.shape[0]), y


def variant_supported(variant, codes, codebooks, x, K=None, B=None, workspace_bytes=None) -> bool:
    """Would gemv_variant run?  workspace_bytes None: with the workspace it needs."""
    lib = _load()
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    args, _y = _query_args(codes, codebooks, x, K, B)
    if workspace_bytes is None:
        workspace_bytes = max(0, lib.aqlm_workspace_bytes(OPS["gemv"], v, *args))
    return bool(lib.aqlm_variant_supported(v, *args, int(workspace_bytes)))


def workspace_bytes(op, codes, codebooks, x, K=None, B=None, variant="auto") -> int:
    """Workspace bytes of the call op ("gemv", "gemm", "gemv_packed"; for the packed
    call pass the PackedWeights' codes and codebooks tensors)."""
    lib = _load()
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    if op == "gemv_packed":
        raise ValueError("use packed_workspace_bytes for packed weights")
    args, _y = _query_args(codes, codebooks, x, K, B)
    return int(lib.aqlm_workspace_bytes(OPS[op], v, *args))


def packed_workspace_bytes(weights, x) -> int:
    """Workspace bytes of gemv_packed(weights, x)."""
    torch = _torch()
    lib = _load()
    w = weights
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    y = torch.empty((x2.shape[0], w.out_features), dtype=torch.float16, device=x2.device)
    return int(lib.aqlm_workspace_bytes(OPS["gemv_packed"], 0, w.codes.data_ptr(),
                                        w.codebooks.data_ptr(), x2.data_ptr(), y.data_ptr(),
                                        w.out_features, w.in_features, w.K, w.B, x2.shape[0]))


def grouped_workspace_bytes(op, codes, codebooks, x, out_features, in_features, K, B) -> int:
    """Workspace bytes of a grouped call (op "gemv", "gemm" or "gemv_packed")."""
    torch = _torch()
    lib = _load()
    n = len(codes)
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    ys = [torch.empty((x2.shape[0], o), dtype=torch.float16, device=x2.device) for o in out_features]
    vp = ctypes.c_void_p
    arr = lambda ts: (vp * n)(*[t.data_ptr() for t in ts])
    return int(lib.aqlm_grouped_workspace_bytes(OPS[op], n, arr(codes), arr(codebooks),
                                                x2.data_ptr(), arr(ys),
                                                (ctypes.c_int64 * n)(*out_features), in_features,
                                                K, B, x2.shape[0]))


def selected_variant(codes, codebooks, x, gemm: bool = False, K=None, B=None,
                     workspace_bytes=None) -> str:
    """Name of the kernel aqlm_gemv (or aqlm_gemm) would run for these tensors, with the
    workspace the call needs (workspace_bytes None, as the binding's calls pass it) or
    the given size (0: the kernels that need none)."""
    lib = _load()
    args, _y = _query_args(codes, codebooks, x, K, B)
    if workspace_bytes is None:
        workspace_bytes = max(0, lib.aqlm_workspace_bytes(OPS["gemm" if gemm else "gemv"], 0, *args))
    v = lib.aqlm_selected_variant(1 if gemm else 0, *args, int(workspace_bytes))
    return lib.aqlm_variant_name(v).decode() if v >= 0 else "error"


def dequantize(codes, codebooks, K=None, B=None, dtype=None, out=None):
    """Dense W [out][in]: float32 (the exact fp32 fold) or float16 (rounded once)."""
    torch = _torch()
    lib = _load()
    dtype = torch.float32 if dtype is None else dtype
    if dtype not in (torch.float32, torch.float16):
        raise TypeError("dtype must be float32 or float16")
    dummy_x = torch.empty((1, codes.shape[1] * 8), dtype=torch.float16, device=codes.device)
    K, B, _ = _prep(codes, codebooks, dummy_x, K, B)
    out_f, in_f = codes.shape[0], codes.shape[1] * 8
    W = out if out is not None else torch.empty((out_f, in_f), dtype=dtype, device=codes.device)
    if W.dtype != dtype or tuple(W.shape) != (out_f, in_f) or not W.is_contiguous():
        raise ValueError("out must be a contiguous [out][in] tensor of the requested dtype")
    _check(lib.aqlm_dequantize(codes.data_ptr(), codebooks.data_ptr(), W.data_ptr(),
                               1 if dtype == torch.float16 else 0, out_f, in_f, K, B, _stream()),
           "aqlm_dequantize")
    return W


def bits_per_weight(K: int, B: int, group: int = 8) -> float:
    return _load().aqlm_bits_per_weight(K, B, group)


def codes_bytes(out_features: int, in_features: int, K: int, B: int) -> int:
    return _load().aqlm_codes_bytes(out_features, in_features, K, B)


def codebooks_bytes(K: int, B: int) -> int:
    return _load().aqlm_codebooks_bytes(K, B)


def version() -> str:
    return _load().aqlm_version().decode()
