"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aqlm_mi355x.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    import additive_quantized_gemv_amd as aq
    if not os.path.exists(aq.library_path()):
        from additive_quantized_gemv_amd import build
        build.build()
    return aq._load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aqlm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"aqlm_gemv", "aqlm_gemm", "aqlm_dequantize", "aqlm_gemv_variant"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_bitrate_matches_worked_examples(lib):
    with open(os.path.join(GOLDEN, "bitrate_examples.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for K, entries, g, bits, *_ in rows:
        B = int(np.log2(int(entries)))
        assert lib.aqlm_bits_per_weight(int(K), B, int(g)) == float(bits)


def test_sizes(lib):
    assert lib.aqlm_codes_bytes(11008, 4096, 2, 8) == 11272192
    assert lib.aqlm_codes_bytes(4096, 4096, 1, 16) == 4194304
    assert lib.aqlm_codes_bytes(28672, 8192, 1, 16) == 58720256
    assert lib.aqlm_codes_bytes(10, 12, 2, 8) == -1      # in not a multiple of 8
    assert lib.aqlm_codes_bytes(10, 16, 9, 8) == -1      # K out of range
    assert lib.aqlm_codebooks_bytes(2, 8) == 8192
    assert lib.aqlm_codebooks_bytes(1, 16) == 1 << 20
    assert lib.aqlm_codebooks_bytes(1, 12) == -1


def test_strings(lib):
    for s in range(4):
        assert lib.aqlm_status_string(s)
    names = [lib.aqlm_variant_name(v).decode() for v in range(7)]
    assert names == ["auto", "generic", "lds", "lut", "l2", "mfma", "split"]
    assert lib.aqlm_variant_name(99) == b"unknown"
    assert lib.aqlm_version()


# fake, well-separated "device" addresses: validation must fail before any use
C, CB, X, Y, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.mark.parametrize("args", [
    (0, CB, X, Y, 16, 64, 2, 8, 1),          # null codes
    (C, 0, X, Y, 16, 64, 2, 8, 1),           # null codebooks
    (C, CB, 0, Y, 16, 64, 2, 8, 1),          # null x
    (C, CB, X, 0, 16, 64, 2, 8, 1),          # null y
    (C, CB, X, Y, 0, 64, 2, 8, 1),           # out < 1
    (C, CB, X, Y, 16, 0, 2, 8, 1),           # in < 1
    (C, CB, X, Y, 16, 60, 2, 8, 1),          # in % 8
    (C, CB, X, Y, 16, 64, 0, 8, 1),          # K < 1
    (C, CB, X, Y, 16, 64, 9, 8, 1),          # K > 8
    (C, CB, X, Y, 16, 64, 2, 4, 1),          # B not 8/16
    (C, CB, X, Y, 16, 64, 2, 8, 0),          # batch < 1
    (C, CB, X, Y, 1 << 62, 1 << 40, 2, 8, 1),  # byte counts overflow
    (C, CB, X, C + 8, 16, 64, 2, 8, 1),      # y overlaps codes
    (C, CB, X, X, 16, 64, 2, 8, 1),          # y overlaps x
    (C, CB + 1, X, Y, 16, 64, 2, 8, 1),      # misaligned fp16 codebooks
    (C + 1, CB, X, Y, 16, 64, 1, 16, 1),     # misaligned 16-bit codes
])
def test_invalid_arguments_rejected(lib, args):
    for fn in (lib.aqlm_gemv, lib.aqlm_gemm):
        assert fn(*args, None, 0, None) == 1
    assert lib.aqlm_gemv_variant(1, *args, None, 0, None) == 1
    assert lib.aqlm_variant_supported(1, *args, 0) == 0
    assert lib.aqlm_selected_variant(0, *args, 0) == -1
    for op in (0, 1, 2):
        assert lib.aqlm_workspace_bytes(op, 0, *args) == -1


def test_dequantize_invalid(lib):
    assert lib.aqlm_dequantize(C, CB, Y, 2, 16, 64, 2, 8, None) == 1    # bad dtype
    assert lib.aqlm_dequantize(C, CB, C, 0, 16, 64, 2, 8, None) == 1    # W overlaps codes
    assert lib.aqlm_dequantize(C, CB, Y + 2, 0, 16, 64, 2, 8, None) == 1  # fp32 W misaligned
    assert lib.aqlm_dequantize(0, CB, Y, 0, 16, 64, 2, 8, None) == 1


def test_pack_invalid(lib):
    assert lib.aqlm_pack_codebooks(0, Y, 1, 16, None) == 1
    assert lib.aqlm_pack_codebooks(CB, Y, 0, 16, None) == 1
    assert lib.aqlm_pack_codebooks(CB, Y, 1, 12, None) == 1
    assert lib.aqlm_pack_codebooks(CB, CB + 64, 1, 16, None) == 1     # overlapping
    assert lib.aqlm_unpack_codebooks(CB + 1, Y, 1, 16, None) == 1     # misaligned
    assert lib.aqlm_pack_codebooks(CB + 2, Y, 1, 16, None) == 1       # pairs need 4 bytes
    assert lib.aqlm_gemv_packed(0, CB, X, Y, 16, 64, 1, 16, 1, WS, 1 << 20, None) == 1
    assert lib.aqlm_gemv_packed(C, CB, X, Y, 16, 60, 1, 16, 1, WS, 1 << 20, None) == 1


def test_packed_codes_sizes(lib):
    # 2x8: ceil(G/64) slices x ceil(out/8) row octets x 1 KiB tiles
    assert lib.aqlm_packed_codes_bytes(11008, 4096, 2, 8) == 8 * 1376 * 1024
    assert lib.aqlm_packed_codes_bytes(4096, 11008, 2, 8) == 22 * 512 * 1024
    assert lib.aqlm_packed_codes_bytes(65, 520, 2, 8) == 2 * 9 * 1024
    assert lib.aqlm_packed_codes_bytes(1, 64, 2, 8) == 1024
    # other schemes keep the canonical layout
    assert lib.aqlm_packed_codes_bytes(4096, 4096, 1, 16) == 4096 * 512 * 2
    assert lib.aqlm_packed_codes_bytes(10, 24, 3, 8) == 10 * 3 * 3
    assert lib.aqlm_packed_codes_bytes(10, 12, 2, 8) == -1
    assert lib.aqlm_packed_codes_bytes(10, 16, 2, 12) == -1


def test_pack_codes_invalid(lib):
    assert lib.aqlm_pack_codes(0, Y, 16, 64, 2, 8, None) == 1
    assert lib.aqlm_pack_codes(C, 0, 16, 64, 2, 8, None) == 1
    assert lib.aqlm_pack_codes(C, Y, 16, 60, 2, 8, None) == 1          # in % 8
    assert lib.aqlm_pack_codes(C, C + 100, 16, 64, 2, 8, None) == 1    # overlapping
    assert lib.aqlm_pack_codes(C + 1, Y, 16, 64, 2, 8, None) == 1      # 2x8 words misaligned
    assert lib.aqlm_unpack_codes(C, Y + 1, 16, 64, 2, 8, None) == 1
    # y inside the padded packed codes (beyond the canonical size) is rejected
    n = lib.aqlm_packed_codes_bytes(9, 64, 2, 8)
    assert n == 2 * 1024 and lib.aqlm_codes_bytes(9, 64, 2, 8) == 144
    assert lib.aqlm_gemv_packed(C, CB, X, C + 512, 9, 64, 2, 8, 1, WS, 1 << 20, None) == 1


def _grouped_args(n, outs, ys, codes=None):
    vp, k = ctypes.c_void_p, max(n, 4)
    codes = codes or [C + 0x100000 * i for i in range(k)]
    return (n, (vp * k)(*codes), (vp * k)(*[CB + 0x100000 * i for i in range(k)]), X,
            (vp * k)(*(ys + [Y + 0x800000] * (k - len(ys)))),
            (ctypes.c_int64 * k)(*(outs + [16] * (k - len(outs)))))


@pytest.mark.parametrize("fn", ["aqlm_gemv_grouped", "aqlm_gemm_grouped", "aqlm_gemv_packed_grouped"])
def test_grouped_invalid(lib, fn):
    f = getattr(lib, fn)
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    ys = [Y, Y + 0x100000, Y + 0x200000, Y + 0x300000]
    def call(n, outs, ys_, in_=64, K=2, B=8, batch=1, codes=None):
        a = _grouped_args(n, outs, ys_, codes)
        return f(a[0], ctypes.cast(a[1], ctypes.c_void_p), ctypes.cast(a[2], ctypes.c_void_p), a[3],
                 ctypes.cast(a[4], ctypes.c_void_p), ctypes.cast(a[5], ctypes.c_void_p), in_, K, B,
                 batch, WS, 1 << 24, None)
    assert call(0, [16] * 4, ys) == 1                       # no matrices
    assert call(5, [16] * 4, ys) == 1                       # more than 4
    assert call(2, [16, 0, 0, 0], ys) == 1                  # empty matrix
    assert call(2, [16, 16, 0, 0], ys, in_=60) == 1         # in % 8
    assert call(2, [16, 16, 0, 0], [Y, Y + 16, 0, 0]) == 1  # y_0 overlaps y_1
    assert call(2, [16, 16, 0, 0], [Y, C + 8, 0, 0]) == 1   # y_1 overlaps codes_0
    assert call(2, [16, 16, 0, 0], [Y, X, 0, 0]) == 1       # y_1 overlaps x
    assert call(2, [1 << 29, 1 << 29 + 1, 0, 0], ys, in_=8) == 1   # more than 2^30 rows


def test_variant_choice_host_logic(lib):
    # pointers aligned to 256 B, shapes of the benchmark configurations
    def sel(gemm, out, in_, K, B, batch, ws=1 << 40):
        return lib.aqlm_variant_name(
            lib.aqlm_selected_variant(gemm, C, CB, X, Y, out, in_, K, B, batch, ws)).decode()
    assert sel(0, 11008, 4096, 2, 8, 1) == "lut"
    assert sel(0, 4096, 11008, 2, 8, 1) == "lut"
    assert sel(0, 4096, 4096, 2, 8, 4) == "lds"
    # 16-bit codes at small batches: the split kernel (codebook packed per call)
    assert sel(0, 4096, 4096, 1, 16, 1) == "split"
    assert sel(0, 8192, 28672, 1, 16, 4) == "split"
    assert sel(0, 4096, 4096, 1, 16, 8) == "l2"
    assert sel(1, 4096, 4096, 1, 16, 2) == "split"
    assert sel(1, 4096, 4096, 1, 16, 4) == "mfma"
    assert sel(1, 4096, 4096, 2, 8, 16) == "mfma"
    assert sel(1, 4096, 4096, 1, 16, 128) == "mfma"
    assert sel(1, 4096, 4096, 1, 16, 256) == "mfma"        # prefill from 512 (16-bit codes)
    assert sel(1, 4096, 4096, 1, 16, 512) == "prefill"
    assert sel(1, 4096, 4096, 2, 8, 1024) == "mfma"        # 2x8, inputs a multiple of 64:
    assert sel(1, 4096, 4096, 2, 8, 8192) == "mfma"        # the matrix cores at any batch
    assert sel(1, 4096, 4128, 2, 8, 512) == "mfma"         # other 2x8: prefill from 1024
    assert sel(1, 4096, 4128, 2, 8, 1024) == "prefill"
    assert sel(1, 4096, 4096, 4, 8, 512) == "prefill"      # K >= 4: from 512
    assert sel(1, 4096, 4096, 2, 8, 8) == "mfma"
    assert sel(1, 4096, 4096, 2, 8, 1) == "lut"
    assert sel(1, 4096, 4096, 8, 8, 2) == "lds"       # eight codebooks: matrix cores from 4
    assert sel(1, 4096, 4096, 8, 8, 4) == "mfma"
    assert sel(0, 64, 24, 3, 8, 1) == "generic"
    assert lib.aqlm_variant_supported(3, C, CB, X, Y, 4096, 4096, 1, 16, 1, 1 << 40) == 0  # lut: 2x8
    assert lib.aqlm_variant_supported(5, C, CB, X, Y, 4096, 4096, 3, 8, 16, 1 << 40) == 0  # mfma: K<=2
    # without a workspace: the kernels that need none (the matrix cores unsplit)
    assert sel(0, 11008, 4096, 2, 8, 1, 0) == "lds"
    assert sel(0, 4096, 4096, 1, 16, 1, 0) == "l2"
    assert sel(1, 4096, 4096, 2, 8, 128, 0) == "mfma"
    assert sel(1, 4096, 4096, 2, 8, 1, 0) == "lds"
    assert lib.aqlm_variant_supported(3, C, CB, X, Y, 4096, 4096, 2, 8, 1, 0) == 0   # lut: partials
    assert lib.aqlm_variant_supported(5, C, CB, X, Y, 4096, 4096, 2, 8, 128, 0) == 1  # unsplit


def test_workspace_rule_host_logic(lib):
    """The workspace a call needs is a function of its arguments; a size between 0 and
    that need is an argument error, reported before any device work; 0 selects the
    kernels that need none."""
    args = (C, CB, X, Y, 11008, 4096, 2, 8, 1)
    need = lib.aqlm_workspace_bytes(0, 0, *args)
    # lut: one fp32 partial sum per row and 64-group input slice
    assert need == 11008 * (512 // 64) * 4
    assert lib.aqlm_selected_variant(0, *args, need - 1) == -1
    assert b"too small" in lib.aqlm_last_error() or True    # message is per call, see below
    assert lib.aqlm_gemv(*args, WS, need - 1, None) == 1
    assert b"too small" in lib.aqlm_last_error()
    assert lib.aqlm_gemv(*args, WS + 8, need, None) == 1         # misaligned workspace
    assert lib.aqlm_gemv(*args, Y, need, None) == 1              # overlaps y
    assert lib.aqlm_gemv(*args, C, need, None) == 1              # overlaps codes
    assert lib.aqlm_gemv(*args, None, 64, None) == 1             # size without a pointer
    assert lib.aqlm_gemv(*args, WS, -1, None) == 1
    # 16-bit codes: the codebook packed per call (1 MiB) + 8 position-pair partial sums
    a16 = (C, CB, X, Y, 4096, 11008, 1, 16, 1)
    assert lib.aqlm_workspace_bytes(0, 0, *a16) == (1 << 20) + 8 * 4096 * 4
    assert lib.aqlm_workspace_bytes(0, 4, *a16) == 0            # l2 needs none
    # packed 2x8 and 1x16 at batch 1: slice / part partial sums only
    assert lib.aqlm_workspace_bytes(2, 0, *args) == 11008 * 8 * 4
    assert lib.aqlm_workspace_bytes(2, 0, *a16) == 8 * 4096 * 4
    assert lib.aqlm_workspace_bytes(2, 3, *args) == -1          # packed takes no variant
    assert lib.aqlm_workspace_bytes(7, 0, *args) == -1          # unknown op
    # a packed call needs its workspace in every case
    assert lib.aqlm_gemv_packed(*a16, None, 0, None) == 1
    # gemm at batch 128: the input-split partial sums; without them the kernel is unsplit
    a128 = (C, CB, X, Y, 4096, 4096, 2, 8, 128)
    assert lib.aqlm_workspace_bytes(1, 0, *a128) > 0
    assert lib.aqlm_variant_name(lib.aqlm_selected_variant(1, *a128, 0)) == b"mfma"


def test_library_imports_no_allocation_or_sync(lib):
    """No allocation, free, stream/device synchronisation or capture query is reachable
    from the library's calls: none of those HIP entry points is even imported."""
    import subprocess
    import additive_quantized_gemv_amd as aq
    out = subprocess.run(["nm", "-D", "--undefined-only", aq.library_path()], capture_output=True,
                         text=True, check=True).stdout
    imported = {ln.split()[-1].split("@")[0] for ln in out.splitlines() if ln.strip()}
    hip = {n for n in imported if n.startswith("hip")}
    assert hip, "expected HIP imports"
    banned = [n for n in hip if re.match(
        r"hip(Malloc|Free|HostMalloc|HostFree|ExtMalloc|MallocAsync|FreeAsync|MemPool|"
        r"StreamSynchronize|DeviceSynchronize|EventSynchronize|StreamIsCapturing|"
        r"StreamGetCaptureInfo|HostRegister)", n)]
    assert not banned, banned
    # and no library that allocates or keeps handles behind the calls' back (the prefill
    # GEMM is the library's own kernel)
    assert not any(n.startswith(("hipblas", "rocblas")) for n in imported)


def test_no_device_reports_hip_error(lib):
    """With no GPU present a valid call fails as AQLM_ERR_HIP, with a message."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path only")
    assert lib.aqlm_gemv_variant(1, C, CB, X, Y, 16, 64, 2, 8, 1, None, 0, None) == 3
    assert lib.aqlm_last_error()


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import additive_quantized_gemv_amd as aq
    monkeypatch.setattr(aq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(aq, "_lib", None)
    with pytest.raises(ImportError):
        aq._load()


def test_traffic_record_keyed_on_code_not_comments():
    """bench.py reports measured HBM traffic only while the kernel source hashes as it did
    when the counters were taken; the hash covers the code with comments and whitespace
    removed, so a comment edit keeps the record and a code edit voids it."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a = b"int f(int x) { return x + 1; }  // add one\n/* a block\n   comment */\n"
    b = b"int f(int x)\n{\n    return x + 1;   // a different comment\n}\n"
    c = b"int f(int x) { return x + 2; }\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert len(bench.source_sha("split")) == 16


def test_noalloc_rejects_beyond_scratch_on_host(lib):
    """aqlm_gemv_packed_noalloc refuses a call whose scratch need exceeds its fixed array
    before touching any device (fake, disjoint addresses; packed 2x8 code tiles above
    batch 1 are unpacked into the scratch: 58.7 MB for 28672 x 8192)."""
    lib.aqlm_gemv_packed_noalloc.argtypes = [ctypes.c_void_p] * 4 + [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.aqlm_noalloc_scratch_bytes.restype = ctypes.c_int64
    big = 0x1000000000
    assert lib.aqlm_noalloc_scratch_bytes() == 16 << 20
    assert lib.aqlm_gemv_packed_noalloc(big, 2 * big, 3 * big, 4 * big, 28672, 8192, 2, 8, 2,
                                        None) == 1
    assert b"16777216" in lib.aqlm_last_error()
    assert lib.aqlm_gemv_packed_noalloc(0, CB, X, Y, 16, 64, 1, 16, 1, None) == 1


def test_trace_record_read_back():
    """bench.py reads the kernel-only times of the headline products from the committed
    kernel-trace summary while the kernel sources hash as they did when it was taken."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for name, o, i, K, B in bench.WORKLOAD:
        main_us, call_us = bench.trace_times(name, "split" if B == 16 else "lut_packed")
        assert main_us is not None and 0 < main_us < call_us, name
    assert bench.trace_times("1x16 4096x11008", "lut_packed") == (None, None)
