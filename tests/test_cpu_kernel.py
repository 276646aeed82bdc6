"""Host-core kernel (aqlm_cpu_gemv) against the oracle on the same seeded bytes.

Bar as for the GPU kernels (decode rule of page "AQLM (Additive Quantization for
LLMs)", section "Niveau intermediaire"): for every token b,
max_o |y - y_ref| / (max_o |y_ref| + 1e-6) <= 2e-3, y_ref being the oracle's
unrounded double result.  The kernel sums in fp32 and rounds y once to fp16
(relative 2^-11), so the bar leaves room for fp32 sums over up to 28672 inputs.
Runs on the CPU: no GPU is involved.
"""
import numpy as np
import pytest

from additive_quantized_gemv_amd import synth

TOL = 2e-3


@pytest.fixture(scope="module")
def aq():
    import additive_quantized_gemv_amd as aq
    try:
        aq._load()
    except (ImportError, OSError) as e:
        pytest.skip(f"library not built: {e}")
    if aq.cpu_isa() == "none":
        pytest.skip("host lacks AVX2/FMA/F16C")
    return aq


def _host(p):
    import torch
    codes = p["codes"]
    if codes.dtype == np.uint16:
        codes = codes.view(np.int16)
    return (torch.from_numpy(np.ascontiguousarray(codes)),
            torch.from_numpy(np.ascontiguousarray(p["codebooks"])),
            torch.from_numpy(np.ascontiguousarray(p["x"])))


def _rel(y, yref):
    y = np.asarray(y, dtype=np.float64)
    return np.max(np.abs(y - yref), axis=1) / (np.max(np.abs(yref), axis=1) + 1e-6)


# (out, in, K, B, batch): G = in / 8 ragged against the 64-group table slices and the
# 16- and 8-lane gather steps; out ragged against the 32-row blocks.
CASES = [
    (77, 1624, 2, 8, 1), (77, 1624, 2, 8, 3), (130, 1032, 1, 8, 2), (33, 520, 4, 8, 1),
    (40, 1032, 3, 8, 2), (21, 264, 8, 8, 1), (65, 1032, 1, 16, 1), (65, 1624, 1, 16, 3),
    (31, 520, 2, 16, 2), (9, 136, 3, 16, 1), (1, 8, 2, 8, 1), (1, 8, 1, 16, 1),
    (3, 24, 4, 8, 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_cpu_gemv_matches_oracle(aq, orc, case):
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.05, config=31, copy=K * 100 + B)
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    codes, cb, x = _host(p)
    y = aq.cpu_gemv(codes, cb, x).float().numpy()
    assert y.shape == yref.shape
    assert np.all(np.isfinite(y))
    e = _rel(y, yref)
    assert np.all(e <= TOL), f"max rel err {e.max():.3e}"


@pytest.mark.parametrize("case", [c for c in CASES if c[2] <= 2 or c[2] == 4],
                         ids=lambda c: "x".join(map(str, c)))
def test_cpu_gemv_avx2_kernels(aq, orc, case, monkeypatch):
    """The AVX2 kernels (8-lane gathers, one-group F16C decode) on an AVX-512 host."""
    if aq.cpu_isa() != "avx512":
        pytest.skip("host already runs the AVX2 kernels")
    monkeypatch.setenv("AQLM_CPU_ISA", "avx2")
    assert aq.cpu_isa() == "avx2"
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.05, config=36, copy=K * 100 + B)
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    codes, cb, x = _host(p)
    e = _rel(aq.cpu_gemv(codes, cb, x).float().numpy(), yref)
    assert np.all(e <= TOL), f"max rel err {e.max():.3e}"


@pytest.mark.parametrize("KB", [(2, 8), (1, 16), (3, 8)])
def test_cpu_gemv_thread_count_invariant(aq, KB):
    K, B = KB
    p = synth.make_problem(203, 2056, K, B, batch=2, config=32, copy=K)
    codes, cb, x = _host(p)
    y1 = aq.cpu_gemv(codes, cb, x, threads=1).numpy()
    for t in (3, 8, 0):
        assert np.array_equal(aq.cpu_gemv(codes, cb, x, threads=t).numpy(), y1), t


@pytest.mark.parametrize("name,KB", [("mlp_2x8_7b", (2, 8)), ("mlp_1x16_7b", (1, 16))])
def test_cpu_gemv_full_size_sampled(aq, orc, name, KB):
    """Both 7B MLP shapes at full size; the oracle checks 96 sampled rows of each."""
    K, B = KB
    cfg = synth.CONFIGS[name]
    rng = np.random.default_rng(7)
    for i, (out, in_) in enumerate(cfg["shapes"]):
        p = synth.make_problem(out, in_, K, B, sigma_cb=cfg["sigma_cb"], config=33, copy=i)
        codes, cb, x = _host(p)
        y = aq.cpu_gemv(codes, cb, x).float().numpy()
        rows = np.sort(rng.choice(out, 96, replace=False))
        rows[0], rows[-1] = 0, out - 1
        yref = orc.gemv_rows(p["codes"], p["codebooks"], p["x"], K, B, rows)
        scale = np.max(np.abs(yref), axis=1, keepdims=True) + 1e-6
        e = np.max(np.abs(y[:, rows] - yref) / scale)
        assert e <= TOL, f"{name} {out}x{in_}: max rel err {e:.3e}"


def test_cpu_gemv_special_inputs(aq, orc):
    """x = 0 gives y = +-0; a one-hot x picks one input column of the decoded W."""
    import torch
    p = synth.make_problem(45, 520, 2, 8, batch=1, config=34)
    codes, cb, x = _host(p)
    y = aq.cpu_gemv(codes, cb, torch.zeros_like(x)).float().numpy()
    assert np.all(y == 0)
    W = orc.decode(p["codes"], p["codebooks"], 2, 8)       # fp32 [out][in]
    xo = torch.zeros_like(x)
    xo[0, 77] = 1.0
    y = aq.cpu_gemv(codes, cb, xo).numpy()
    want = W[:, 77].astype(np.float16)
    assert np.array_equal(y[0], want)


def test_cpu_gemv_rejects_bad_arguments(aq):
    import torch
    p = synth.make_problem(8, 64, 2, 8, config=35)
    codes, cb, x = _host(p)
    with pytest.raises(ValueError):
        aq.cpu_gemv(codes, cb, x[:, :32])
    with pytest.raises(ValueError):
        aq.cpu_gemv(codes, cb[:1], x)
    with pytest.raises(TypeError):
        aq.cpu_gemv(codes, cb, x.float())
    lib = aq._load()
    # null pointers, in not a multiple of 8, K out of range, B not 8/16, batch 0
    assert lib.aqlm_cpu_gemv(None, cb.data_ptr(), x.data_ptr(), x.data_ptr(), 8, 64, 2, 8, 1, 1) == 1
    for out, in_, K, B, batch in ((8, 60, 2, 8, 1), (8, 64, 0, 8, 1), (8, 64, 9, 8, 1),
                                  (8, 64, 2, 12, 1), (8, 64, 2, 8, 0), (0, 64, 2, 8, 1)):
        y = torch.empty(8, dtype=torch.float16)
        assert lib.aqlm_cpu_gemv(codes.data_ptr(), cb.data_ptr(), x.data_ptr(), y.data_ptr(),
                                 out, in_, K, B, batch, 1) == 1


@pytest.mark.parametrize("KB", [(2, 8), (1, 8), (1, 16), (2, 16)])
def test_cpu_gemv_token_blocks_match_single_tokens(aq, KB):
    """The decode paths take up to 4 tokens per pass over the codes; each token's sums are
    formed as with one token, so batch 5 (a block of 4 and one more) equals the tokens
    computed one at a time, bit for bit."""
    import torch
    K, B = KB
    p = synth.make_problem(97, 1032, K, B, batch=5, sigma_cb=0.05, config=37, copy=K * 10 + B)
    codes, cb, x = _host(p)
    y = aq.cpu_gemv(codes, cb, x).numpy()
    for b in range(5):
        yb = aq.cpu_gemv(codes, cb, x[b:b + 1].contiguous()).numpy()
        assert np.array_equal(y[b], yb[0]), (KB, b)
