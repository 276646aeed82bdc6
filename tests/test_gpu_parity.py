"""GPU parity: every kernel variant against the CPU oracle on the same seeded bytes.

Bars (decode rule of page "AQLM (Additive Quantization for LLMs)", section
"Niveau intermediaire"):
  * dequantized W: fp32 output equal to the oracle's fp32 fold element by
    element (+0 == -0); fp16 output bit-equal to the round-to-nearest-even fp16
    of the oracle's W;
  * y: for every token b, max_o |y - y_ref| / (max_o |y_ref| + 1e-6) <= 2e-3,
    y_ref being the oracle's unrounded double result.
"""
import numpy as np
import pytest

from additive_quantized_gemv_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import additive_quantized_gemv_amd as aq
    aq._load()
    return aq


def _dev(p):
    import torch
    codes = p["codes"]
    if codes.dtype == np.uint16:
        codes = codes.view(np.int16)
    return (torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
            torch.from_numpy(np.ascontiguousarray(p["codebooks"])).cuda(),
            torch.from_numpy(np.ascontiguousarray(p["x"])).cuda())


def rel_err(y, yref):
    y = np.asarray(y, dtype=np.float64)
    return np.max(np.abs(y - yref), axis=1) / (np.max(np.abs(yref), axis=1) + 1e-6)


def check_y(y_t, yref, what):
    import torch
    torch.cuda.synchronize()
    y = y_t.float().cpu().numpy()
    if y.ndim == 1:
        y = y[None]
    assert np.all(np.isfinite(y)), what
    e = rel_err(y, yref)
    assert np.all(e <= TOL), f"{what}: max rel err {e.max():.3e}"
    return e.max()


def _variants_for(K, B, batch):
    v = ["generic", "mfma"]
    if B == 8:
        v.append("lds")
    if B == 16:
        v += ["l2", "split"]
    if K == 2 and B == 8 and batch == 1:
        v.append("lut")
    return v


SMALL = [
    # out, in, K, B, batch, sigma
    (256, 512, 2, 8, 1, 0.05),      # the tiny 2x8 workload
    (300, 1024, 2, 8, 1, 0.02),
    (65, 520, 2, 8, 1, 0.02),       # ragged rows and a partial 64-group slice
    (17, 4160, 2, 8, 1, 0.02),
    (1, 64, 2, 8, 1, 0.02),
    (200, 768, 1, 16, 1, 0.02),
    (129, 2048, 1, 16, 4, 0.02),
    (96, 512, 2, 8, 4, 0.02),
    (96, 512, 2, 8, 3, 0.02),
    (64, 512, 1, 8, 2, 0.05),
    (64, 512, 4, 8, 1, 0.02),
    (64, 512, 8, 8, 8, 0.01),
    (80, 256, 2, 16, 2, 0.02),
    (70, 24, 3, 8, 2, 0.02),        # generic only (K = 3, in = 24)
    (33, 8, 1, 16, 1, 0.02),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])))
def test_small_all_variants(aq, orc, case):
    out, in_, K, B, batch, sigma = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=sigma, config=101 + out + in_)
    codes, cb, x = _dev(p)
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    ran = []
    for v in _variants_for(K, B, batch):
        if not aq.variant_supported(v, codes, cb, x):
            continue
        check_y(aq.gemv_variant(v, codes, cb, x), yref, f"{v} {case}")
        ran.append(v)
    check_y(aq.gemv(codes, cb, x), yref, f"auto gemv {case}")
    check_y(aq.gemm(codes, cb, x), yref, f"auto gemm {case}")
    assert "generic" in ran


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8, 15, 16, 17, 33, 64, 128])
@pytest.mark.parametrize("KB", [(2, 8), (1, 16)])
def test_batches(aq, orc, batch, KB):
    K, B = KB
    out, in_ = 160, 1024
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=500 + batch)
    codes, cb, x = _dev(p)
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    check_y(aq.gemm(codes, cb, x), yref, f"gemm b={batch}")
    check_y(aq.gemv(codes, cb, x), yref, f"gemv b={batch}")
    check_y(aq.gemv_variant("mfma", codes, cb, x), yref, f"mfma b={batch}")
    # aqlm_gemm takes the matrix cores from batch 2 (16-bit codes: from 3, the split kernel
    # before); aqlm_gemv never does
    want = batch >= (3 if B == 16 else 2)
    assert (aq.selected_variant(codes, cb, x, gemm=True) == "mfma") == want
    assert aq.selected_variant(codes, cb, x, gemm=False) != "mfma"


@pytest.mark.parametrize("KB", [(1, 8), (2, 8), (3, 8), (4, 8), (8, 8), (1, 16), (2, 16)])
def test_dequantize_bit_exact(aq, orc, KB):
    import torch
    K, B = KB
    p = synth.make_problem(96, 256, K, B, batch=1, sigma_cb=0.02, config=700 + K * B)
    codes, cb, _ = _dev(p)
    Wref = orc.decode(p["codes"], p["codebooks"], K, B)
    W32 = aq.dequantize(codes, cb, dtype=torch.float32).cpu().numpy()
    assert np.array_equal(W32, Wref)
    W16 = aq.dequantize(codes, cb, dtype=torch.float16).cpu().numpy()
    assert np.array_equal(W16.view(np.uint16), Wref.astype(np.float16).view(np.uint16))


def test_dequantize_special_values(aq, orc):
    """fp16 subnormals, signed zeros and +-65504 in the codebooks (2x8 and 1x16)."""
    import torch
    for K, B in [(2, 8), (1, 16), (3, 8)]:
        p = synth.make_problem(64, 128, K, B, batch=1, sigma_cb=0.02, config=800 + K)
        cb = p["codebooks"].copy()
        sub = np.arange(1, 1024, 37, dtype=np.uint16).view(np.float16)   # subnormals
        cb.reshape(-1)[: sub.size] = sub
        cb.reshape(-1)[-sub.size:] = -sub
        cb[0, 5] = np.float16(-0.0)
        cb[-1, 6] = np.float16(0.0)
        cb[0, 7] = np.float16(65504)
        cb[-1, 8] = np.float16(-65504)
        codes = p["codes"].copy()
        codes[:, :, 0] = np.arange(codes.shape[0] * codes.shape[1]).reshape(codes.shape[:2]) % 16
        p["codebooks"] = cb
        p["codes"] = codes
        ct, cbt, _ = _dev(p)
        Wref = orc.decode(codes, cb, K, B)
        W32 = aq.dequantize(ct, cbt, dtype=torch.float32).cpu().numpy()
        assert np.array_equal(W32, Wref)
        with np.errstate(over="ignore"):
            ref16 = Wref.astype(np.float16)
        W16 = aq.dequantize(ct, cbt, dtype=torch.float16).cpu().numpy()
        same = (W16.view(np.uint16) == ref16.view(np.uint16)) | ((W16 == 0) & (ref16 == 0))
        assert np.all(same)


def test_special_inputs(aq, orc):
    """x = 0 gives 0; x = e_i gives column i; subnormal codebooks; identical codes everywhere."""
    import torch
    for K, B in [(2, 8), (1, 16)]:
        p = synth.make_problem(130, 1024, K, B, batch=1, sigma_cb=0.02, config=900 + K)
        codes, cb, x = _dev(p)
        variants = [v for v in _variants_for(K, B, 1) if aq.variant_supported(v, codes, cb, x)]
        zero = torch.zeros_like(x)
        for v in variants:
            assert torch.all(aq.gemv_variant(v, codes, cb, zero).float() == 0), v
        W = orc.decode(p["codes"], p["codebooks"], K, B)
        for i in (0, 7, 513, 1023):
            e = torch.zeros_like(x)
            e[0, i] = 1
            for v in variants:
                y = aq.gemv_variant(v, codes, cb, e).float().cpu().numpy()[0]
                assert np.array_equal(y, W[:, i].astype(np.float16).astype(np.float32)), (v, i)
        # all group-rows use the same code (every lane gathers the same entry)
        same = p["codes"].copy()
        same[...] = 7
        ct, _, _ = _dev(dict(p, codes=same))
        yref = orc.gemv(same, p["codebooks"], p["x"], K, B)
        for v in variants:
            check_y(aq.gemv_variant(v, ct, cb, x), yref, f"same-code {v}")
        # codebooks made of subnormals only
        cbs = (np.abs(p["codebooks"].astype(np.float64)) * 2.0 ** -12).astype(np.float16)
        cbs = np.where(p["codebooks"] < 0, -cbs, cbs).astype(np.float16)
        assert np.mean(np.abs(cbs) < 2.0 ** -14) > 0.9
        _, cbt, _ = _dev(dict(p, codebooks=cbs))
        yref = orc.gemv(p["codes"], cbs, p["x"], K, B)
        for v in variants:
            check_y(aq.gemv_variant(v, codes, cbt, x), yref, f"subnormal {v}")


def test_lut_repeat_deterministic(aq, orc):
    """Repeated lookup-table calls on shapes of changing size give bit-identical y (the
    slice partial sums are added in a fixed order)."""
    shapes = [(100, 1024), (3000, 8192), (100, 1024), (5000, 520), (3000, 8192)]
    for i, (out, in_) in enumerate(shapes):
        p = synth.make_problem(out, in_, 2, 8, batch=1, sigma_cb=0.02, config=1000 + i)
        codes, cb, x = _dev(p)
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], 2, 8)
        ys = [aq.gemv_variant("lut", codes, cb, x) for _ in range(3)]
        check_y(ys[0], yref, f"lut {out}x{in_}")
        for y in ys[1:]:
            assert bool((y == ys[0]).all())     # deterministic slice order


def test_binding_rejects_host_tensors(aq):
    import torch
    p = synth.make_problem(16, 64, 2, 8)
    with pytest.raises(ValueError):
        aq.gemv(torch.from_numpy(p["codes"]), torch.from_numpy(p["codebooks"]),
                torch.from_numpy(p["x"]))


# ----------------------------------------------------------------- full sizes
# The benchmark workloads at full size, in the launch configuration the
# benchmark uses (auto variant choice).

def _sampled_rows(out, n=192, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, out - 1], rng.integers(0, out, n)]))
    return rows


FULL = []
for _name, _cfg in synth.CONFIGS.items():
    for _si, _shape in enumerate(dict.fromkeys(_cfg["shapes"])):
        for _b in _cfg["batches"]:
            FULL.append((_name, _shape[0], _shape[1], _cfg["K"], _cfg["B"], _b, _cfg["sigma_cb"]))


# Every row is compared up to batch 4 (the oracle's decode and matvec of a 70B-shaped
# product take a few seconds on the host cores); larger batches on sampled rows.
FULL_ROWS_MAX_BATCH = 4


def _check_rows(y, p, K, B, out, seed, what, orc, batch):
    import torch
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy()
    yg = yg[None] if yg.ndim == 1 else yg
    assert np.all(np.isfinite(yg)), what
    if batch <= FULL_ROWS_MAX_BATCH:
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
        e = rel_err(yg, yref)
    else:
        rows = _sampled_rows(out, seed=seed)
        yref = orc.gemv_rows(p["codes"], p["codebooks"], p["x"], K, B, rows)
        e = rel_err(yg[:, rows], yref)
    assert np.all(e <= TOL), f"{what}: {e.max():.3e}"


@pytest.mark.parametrize("case", FULL, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-b{c[5]}")
def test_full_size(aq, orc, case):
    name, out, in_, K, B, batch, sigma = case
    cid = list(synth.CONFIGS).index(name)
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=sigma, config=cid)
    codes, cb, x = _dev(p)
    fn = aq.gemm if batch >= 16 else aq.gemv
    _check_rows(fn(codes, cb, x), p, K, B, out, cid, str(case), orc, batch)


def test_graph_capture_replay(aq, orc):
    """Products captured in a HIP graph and replayed several times, with eager work and
    synchronisations between replays, match the eager results every time."""
    import torch
    # batch 128 and 200 with 8-bit codes: the DMA-staged matrix-core kernel, at 128 with
    # input-axis splits and the partial-sum kernel
    cases = [(1000, 4096, 2, 8, 1), (1000, 4096, 1, 16, 1), (512, 1024, 2, 8, 4),
             (512, 1024, 2, 8, 32), (512, 1024, 1, 16, 16), (512, 1024, 2, 8, 128),
             (300, 2048, 1, 8, 200)]
    stream = torch.cuda.Stream()
    probs, eager, outs = [], [], []
    with torch.cuda.stream(stream):
        for i, (out, in_, K, B, batch) in enumerate(cases):
            p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=1200 + i)
            t = _dev(p)
            probs.append((p, t))
            eager.append(aq.gemm(*t).clone())
            outs.append(torch.empty_like(eager[-1]))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for (p, t), o in zip(probs, outs):
                aq.gemm(*t, out=o)
        for rep in range(4):
            for o in outs:
                o.fill_(7.0)                         # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for e, o in zip(eager, outs):
                assert bool((e == o).all()), f"replay {rep}"
    for (p, _), e in zip(probs, eager):
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], p["K"], p["B"])
        check_y(e, yref, "eager before capture")


HEADLINE = [("mlp_2x8_7b", 11008, 4096), ("mlp_2x8_7b", 4096, 11008),
            ("mlp_1x16_7b", 11008, 4096), ("mlp_1x16_7b", 4096, 11008)]


@pytest.mark.parametrize("case", HEADLINE, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_capture_fresh_stream_same_kernel(aq, orc, case):
    """A headline product captured with no eager call before it, on torch's own capture
    stream (torch.cuda.graph without a stream), runs the kernel the eager call runs:
    its replays equal the eager y bit for bit (canonical and packed weights), and the
    eager y meets the bar on every row.  The kernel choice depends on the arguments only."""
    import torch
    name, out, in_ = case
    cfg = synth.CONFIGS[name]
    K, B = cfg["K"], cfg["B"]
    p = synth.make_problem(out, in_, K, B, batch=1, sigma_cb=cfg["sigma_cb"], config=3100 + out)
    codes, cb, x = _dev(p)
    W = aq.pack_weights(codes, cb)
    torch.cuda.synchronize()
    y_c = torch.empty((1, out), dtype=torch.float16, device="cuda")
    y_p = torch.empty_like(y_c)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        aq.gemv(codes, cb, x, out=y_c)
        aq.gemv_packed(W, x, out=y_p)
    want = "split" if B == 16 else "lut"
    assert aq.selected_variant(codes, cb, x) == want
    eager_c = aq.gemv(codes, cb, x)
    eager_p = aq.gemv_packed(W, x)
    for _ in range(3):
        y_c.fill_(5.0)
        y_p.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bool((y_c == eager_c).all()) and bool((y_p == eager_p).all())
    _check_rows(eager_c, p, K, B, out, 0, f"{case} canonical", orc, 1)
    _check_rows(eager_p, p, K, B, out, 0, f"{case} packed", orc, 1)


def test_graph_replay_after_large_eager_call(aq, orc):
    """Decode-size products captured into a graph, then a prefill-size product run
    eagerly on the same stream (a much larger workspace), then the graph replayed: the
    replays still equal the eager results bit for bit (a graph keeps the workspace its
    capture was given; nothing the library holds is resized or freed)."""
    import torch
    stream = torch.cuda.Stream()
    dec = [synth.make_problem(1000, 4096, 2, 8, batch=1, sigma_cb=0.02, config=3200),
           synth.make_problem(1000, 4096, 1, 16, batch=1, sigma_cb=0.02, config=3201)]
    big = synth.make_problem(512, 2048, 1, 16, batch=1024, sigma_cb=0.02, config=3202)
    with torch.cuda.stream(stream):
        td = [_dev(p) for p in dec]
        eager = [aq.gemv(*t).clone() for t in td]
        outs = [torch.empty_like(e) for e in eager]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t, o in zip(td, outs):
                aq.gemv(*t, out=o)
        tb = _dev(big)
        yb = aq.gemm(*tb)
        for _ in range(3):
            for o in outs:
                o.fill_(7.0)
            g.replay()
            yb2 = aq.gemm(*tb)          # eager work between replays, on the same stream
            torch.cuda.synchronize()
            for e, o in zip(eager, outs):
                assert bool((e == o).all())
            assert bool((yb2 == yb).all())
    check_y(yb, orc.gemv(big["codes"], big["codebooks"], big["x"], 1, 16), "prefill-size eager")
    for p, e in zip(dec, eager):
        check_y(e, orc.gemv(p["codes"], p["codebooks"], p["x"], p["K"], p["B"]), "decode eager")


DQ = [
    # out, in, K, B, batch: the matrix-core kernel with DMA-staged operands (8-bit codes,
    # K <= 2, batch > 64, in a multiple of 64; 64-token tiles up to batch 128)
    (300, 4096, 2, 8, 128),      # ragged row tile, input axis split
    (4096, 4096, 2, 8, 128),     # 16 row tiles x 2 token tiles x 4 splits of 16 k-tiles
    (257, 1024, 1, 8, 70),       # one codebook; the second token tile holds 6 tokens
    (512, 640, 2, 8, 65),        # 10 k-tiles; a second token tile of one token
    (1000, 2048, 2, 8, 200),     # 128-token tiles, the second ragged
    (64, 64, 2, 8, 100),         # a single k-tile: every prologue load clamped
    (520, 1536, 1, 8, 129),
    (96, 192, 2, 8, 1000),       # 8 token tiles of a 3-k-tile product
]


@pytest.mark.parametrize("case", DQ, ids=lambda c: "x".join(map(str, c)))
def test_mfma_dma_staged(aq, orc, case):
    """Batched matrix cores on 8-bit codes: with the workspace (input axis split, partial
    sums added in split order) and without it (one split), both against the oracle on
    sampled rows, and the two outputs within the bar of each other."""
    import torch
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=4100 + out + batch)
    codes, cb, x = _dev(p)
    assert aq.selected_variant(codes, cb, x, gemm=True) in ("mfma", "prefill")
    rows = _sampled_rows(out, seed=out + batch)
    yref = orc.gemv_rows(p["codes"], p["codebooks"], p["x"], K, B, rows)
    y1 = aq.gemv_variant("mfma", codes, cb, x)
    y0 = aq.gemv_variant("mfma", codes, cb, x, workspace=0)
    torch.cuda.synchronize()
    for y, what in ((y1, "split"), (y0, "unsplit")):
        yg = y.float().cpu().numpy()
        assert np.all(np.isfinite(yg)), what
        e = rel_err(yg[:, rows], yref)
        assert np.all(e <= TOL), f"{what} {case}: {e.max():.3e}"


@pytest.mark.parametrize("case", [
    # out, in, K, B, batch, variant expected without a workspace
    (700, 2048, 2, 8, 1, "lds"), (700, 2048, 1, 16, 1, "l2"), (300, 8192, 2, 8, 128, "mfma"),
    (257, 4096, 1, 16, 64, "mfma"),
], ids=lambda c: "x".join(map(str, c[:5])))
def test_no_workspace_kernels(aq, orc, case):
    """workspace=0: the kernels that need no workspace (the matrix cores unsplit), same
    bar; a workspace between 0 and the need is an argument error, nothing launched."""
    import torch
    out, in_, K, B, batch, want = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=3300 + out + batch)
    codes, cb, x = _dev(p)
    gemm = batch > 1
    assert aq.selected_variant(codes, cb, x, gemm=gemm, workspace_bytes=0) == want
    fn = aq.gemm if gemm else aq.gemv
    y = fn(codes, cb, x, workspace=0)
    check_y(y, orc.gemv(p["codes"], p["codebooks"], p["x"], K, B), f"no workspace {case}")
    need = aq.workspace_bytes("gemm" if gemm else "gemv", codes, cb, x)
    assert need > 0
    small = torch.empty(need - 4, dtype=torch.uint8, device="cuda")
    lib = aq._load()
    st = getattr(lib, "aqlm_gemm" if gemm else "aqlm_gemv")(
        codes.data_ptr(), cb.data_ptr(), x.data_ptr(), y.data_ptr(), out, in_, K, B, batch,
        small.data_ptr(), need - 4, None)
    assert st == 1 and b"too small" in lib.aqlm_last_error()


def test_grouped_no_workspace(aq, orc):
    """A grouped batch-128 product without a workspace: the unsplit matrix-core kernel."""
    ps = _group((500, 300, 64), 2048, 2, 8, 128, 2300)
    dev = [_dev(p) for p in ps]
    ys = aq.gemm_grouped([d[0] for d in dev], [d[1] for d in dev], dev[0][2], workspace=0)
    for m, p in enumerate(ps):
        check_y(ys[m], orc.gemv(p["codes"], p["codebooks"], p["x"], 2, 8), f"no workspace {m}")


# ------------------------------------------------------------ packed codebooks

@pytest.mark.parametrize("KB", [(1, 16), (2, 16), (2, 8)])
def test_pack_unpack_exact(aq, KB):
    import torch
    K, B = KB
    p = synth.make_problem(8, 64, K, B, sigma_cb=0.02, config=1400 + K)
    cb = torch.from_numpy(p["codebooks"]).cuda()
    P = aq.pack_codebooks(cb)
    torch.cuda.synchronize()
    c = p["codebooks"].view(np.uint16)
    # B = 8: planes P[k][t][c] = C[k][c][t]; B = 16: pairs P[k][q][c][s] = C[k][c][2q + s]
    want = c.transpose(0, 2, 1) if B == 8 else c.reshape(K, 1 << B, 4, 2).transpose(0, 2, 1, 3)
    assert P.shape == want.shape
    assert np.array_equal(P.cpu().numpy().view(np.uint16), np.ascontiguousarray(want))
    assert np.array_equal(aq.unpack_codebooks(P).cpu().numpy().view(np.uint16),
                          p["codebooks"].view(np.uint16))


def _tiles_2x8(codes):
    """Packed 2x8 code tiles as the header defines them, built with numpy."""
    out, G, _ = codes.shape
    w = np.ascontiguousarray(codes).view(np.uint16).reshape(out, G)   # byte 0 = c0, byte 1 = c1
    S, NQ = -(-G // 64), -(-out // 8)
    pad = np.zeros((NQ * 8, S * 64), np.uint16)
    pad[:out, :G] = w
    return np.ascontiguousarray(pad.reshape(NQ, 8, S, 64).transpose(2, 0, 3, 1)).view(np.uint8).ravel()


@pytest.mark.parametrize("case", [(16, 512, 2, 8), (65, 520, 2, 8), (1, 64, 2, 8), (300, 11008, 2, 8),
                                  (40, 512, 1, 16), (9, 64, 3, 8)],
                         ids=lambda c: "x".join(map(str, c)))
def test_pack_codes_exact(aq, case):
    import torch
    out, in_, K, B = case
    p = synth.make_problem(out, in_, K, B, sigma_cb=0.02, config=1450 + out)
    codes = _dev(p)[0]
    P = aq.pack_codes(codes)
    torch.cuda.synchronize()
    got = P.cpu().numpy()
    if (K, B) == (2, 8):
        assert np.array_equal(got, _tiles_2x8(p["codes"]))
    else:
        assert np.array_equal(got, np.ascontiguousarray(p["codes"]).view(np.uint8).ravel())
    back = aq.unpack_codes(P, out, in_, K, B)
    assert np.array_equal(back.cpu().numpy().view(np.uint8),
                          np.ascontiguousarray(p["codes"]).view(np.uint8))


PACKED = [
    # out, in, K, B, batch
    (300, 4096, 1, 16, 1), (65, 520, 1, 16, 1), (1, 64, 1, 16, 1), (257, 11008, 1, 16, 1),
    (130, 2048, 1, 16, 2), (77, 1024, 1, 16, 3), (160, 8192, 1, 16, 4), (96, 512, 2, 16, 1),
    (50, 1024, 2, 16, 4), (64, 512, 1, 16, 8), (1000, 28672, 1, 16, 1),
    # the split kernel's two forms: pairs at batch 1 (activations in registers up to 7 chunk
    # positions per lane, in 28672) and at batch b with b x positions <= 8 (batch 2 up to
    # in 16384, 3..4 up to 8192); one position per workgroup past that
    (64, 16384, 1, 16, 1), (40, 20480, 1, 16, 1), (100, 11008, 1, 16, 2), (33, 2048, 2, 16, 2),
    (70, 32768, 1, 16, 1), (100, 16384, 1, 16, 2), (129, 8192, 1, 16, 3), (200, 8192, 1, 16, 4),
    (64, 4104, 1, 16, 4), (48, 24576, 1, 16, 2), (1, 64, 1, 16, 4),
    # 2x8: the tiled lookup-table kernel at batch 1 (ragged rows, partial slices), else unpacked
    (40, 512, 2, 8, 1), (65, 520, 2, 8, 1), (1, 64, 2, 8, 1), (300, 4096, 2, 8, 1),
    (257, 11008, 2, 8, 1), (1023, 4160, 2, 8, 1), (5000, 512, 2, 8, 1), (96, 512, 2, 8, 4),
    (64, 512, 1, 8, 2),
    # 16-bit codes above batch 4: the position split on the matrix cores (one-step rows,
    # a partial last k-step, several tiles per wave, token blocks of 32 past batch 32)
    (300, 4096, 1, 16, 5), (100, 4096, 1, 16, 16), (257, 11008, 1, 16, 17),
    (130, 2048, 1, 16, 33), (77, 1024, 1, 16, 64), (64, 512, 1, 16, 100), (40, 4096, 1, 16, 128),
    (1000, 4096, 1, 16, 16), (17, 256, 1, 16, 7), (33, 64, 1, 16, 16), (50, 1024, 2, 16, 16),
    (96, 520, 2, 16, 40),
    (65, 520, 1, 16, 16),      # in/8 not a multiple of 8: unpacked, generic kernel
    # 2x8 from batch 16: unpacked, then the matrix cores (persistent / tiled with partial sums)
    (300, 4096, 2, 8, 16), (257, 4096, 2, 8, 33), (96, 512, 2, 8, 128),
]


@pytest.mark.parametrize("KB", [(1, 16), (2, 8)])
def test_gemv_packed_unaligned_x(aq, orc, KB):
    """x 2 bytes off a 4-byte boundary: the split and lookup-table kernels stage x with
    wider loads, so the product takes the unpacked path, with the same result."""
    import torch
    K, B = KB
    p = synth.make_problem(256, 4096, K, B, batch=1, sigma_cb=0.02, config=1490 + K)
    codes, cb, x = _dev(p)
    buf = torch.empty(4096 + 1, dtype=torch.float16, device=x.device)
    buf[1:] = x[0]
    xu = buf[1:]
    assert xu.data_ptr() % 4 == 2
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    check_y(aq.gemv_packed(aq.pack_weights(codes, cb), xu), yref, f"packed unaligned x {KB}")


@pytest.mark.parametrize("case", PACKED, ids=lambda c: "x".join(map(str, c)))
def test_gemv_packed(aq, orc, case):
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=1500 + out + in_)
    codes, cb, x = _dev(p)
    W = aq.pack_weights(codes, cb)
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    ys = [aq.gemv_packed(W, x) for _ in range(2)]
    check_y(ys[0], yref, f"packed {case}")
    assert bool((ys[0] == ys[1]).all())      # partial sums are added in a fixed order


@pytest.mark.parametrize("case", [("mlp_1x16_7b", 11008, 4096, 1), ("mlp_1x16_7b", 4096, 11008, 1),
                                  ("mlp_1x16_70b", 28672, 8192, 4), ("mlp_1x16_70b", 8192, 28672, 1),
                                  ("proj_1x16_4096", 4096, 4096, 1), ("mlp_2x8_7b", 11008, 4096, 1),
                                  ("mlp_2x8_7b", 4096, 11008, 1), ("mlp_1x16_7b", 11008, 4096, 16),
                                  ("mlp_1x16_7b", 4096, 11008, 128), ("mlp_2x8_7b", 4096, 11008, 16)],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-b{c[3]}")
def test_full_size_packed(aq, orc, case):
    name, out, in_, batch = case
    cfg = synth.CONFIGS[name]
    cid = list(synth.CONFIGS).index(name)
    p = synth.make_problem(out, in_, cfg["K"], cfg["B"], batch=batch, sigma_cb=cfg["sigma_cb"],
                           config=cid)
    codes, cb, x = _dev(p)
    y = aq.gemv_packed(aq.pack_weights(codes, cb), x)
    _check_rows(y, p, cfg["K"], cfg["B"], out, cid, str(case), orc, batch)


def _pass_rows(out, rows_per_block, seed):
    """Sampled rows plus every row next to a 512-row pass boundary inside a row block."""
    rows = set(_sampled_rows(out, seed=seed).tolist())
    for b0 in range(0, out, rows_per_block):
        for p0 in range(b0, min(out, b0 + rows_per_block), 512):
            rows.update(r for r in (p0 - 1, p0, p0 + 1, p0 + 511) if 0 <= r < out)
    return np.array(sorted(rows), dtype=np.int64)


# 2x8 row blocks of more than 512 rows (the lookup-table kernel's multi-pass form):
# out > 512 * (256 / slices), slices = in / 512
MULTIPASS = [(4500, 16384), (4103, 16384), (28672, 8192), (2000, 65536)]


@pytest.mark.parametrize("case", MULTIPASS, ids=lambda c: f"{c[0]}x{c[1]}")
def test_packed_multipass(aq, orc, case):
    import torch
    out, in_ = case
    p = synth.make_problem(out, in_, 2, 8, batch=1, sigma_cb=0.02, config=1800 + out)
    codes, cb, x = _dev(p)
    y = aq.gemv_packed(aq.pack_weights(codes, cb), x)
    torch.cuda.synchronize()
    slices = (in_ // 8 + 63) // 64
    nrb = max(1, 256 // slices)
    rows = _pass_rows(out, (-(-out // nrb) + 7) // 8 * 8, seed=out)   # blocks start on octets
    yref = orc.gemv_rows(p["codes"], p["codebooks"], p["x"], 2, 8, rows)
    e = rel_err(y.float().cpu().numpy()[:, rows], yref)
    assert np.all(e <= TOL), f"{case}: {e.max():.3e}"


def test_packed_grouped_multipass(aq, orc):
    """Two matrices sharing x, one past the one-pass block size, in one grouped call."""
    import torch
    outs, in_ = (4099, 700), 16384
    ps = [synth.make_problem(o, in_, 2, 8, batch=1, sigma_cb=0.02, config=1900 + i)
          for i, o in enumerate(outs)]
    x = torch.from_numpy(np.ascontiguousarray(ps[0]["x"])).cuda()
    ws = []
    for p in ps:
        codes, cb, _ = _dev(p)
        ws.append(aq.pack_weights(codes, cb))
    ys = aq.gemv_packed_grouped(ws, x)
    torch.cuda.synchronize()
    for p, y, o in zip(ps, ys, outs):
        rows = np.arange(o, dtype=np.int64)          # every row (the grouped blocks grow)
        yref = orc.gemv_rows(p["codes"], p["codebooks"], ps[0]["x"], 2, 8, rows)
        e = rel_err(y.float().cpu().numpy()[:, rows], yref)
        assert np.all(e <= TOL), f"grouped {o}x{in_}: {e.max():.3e}"


@pytest.mark.parametrize("batch", [1, 16, 40])
@pytest.mark.parametrize("KB", [(1, 16), (2, 8)])
def test_packed_graph_replay(aq, orc, KB, batch):
    import torch
    K, B = KB
    p = synth.make_problem(2000, 4096, K, B, batch=batch, sigma_cb=0.02, config=1600 + K + batch)
    codes, cb, x = _dev(p)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        W = aq.pack_weights(codes, cb)
        eager = aq.gemv_packed(W, x).clone()
        y = torch.empty_like(eager)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            aq.gemv_packed(W, x, out=y)
        for _ in range(3):
            y.fill_(3.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert bool((y == eager).all())
    check_y(eager, orc.gemv(p["codes"], p["codebooks"], p["x"], K, B), "packed eager")


# ------------------------------------------------------------ grouped calls (shared x)

def _group(outs, in_, K, B, batch, cfg):
    """Matrices that share one x: problems with their own codes/codebooks, x from the first."""
    ps = [synth.make_problem(o, in_, K, B, batch=batch, sigma_cb=0.02, config=cfg + i)
          for i, o in enumerate(outs)]
    for p in ps[1:]:
        p["x"] = ps[0]["x"]
    return ps


GROUPED = [
    # outs, in, K, B, batch
    ((100, 257, 64), 512, 2, 8, 1),          # lookup tables, ragged matrices
    ((65, 33), 520, 2, 8, 1),                # partial 64-group slice
    ((300, 17, 1), 1024, 1, 16, 1),          # L2 gathers
    ((96, 64), 512, 2, 8, 4),                # per-matrix kernels
    ((130, 200, 50), 2048, 1, 16, 3),
    ((100, 257, 64), 512, 2, 8, 16),         # matrix cores, input split over waves
    ((300, 17), 1024, 1, 16, 16),
    ((120, 40, 64, 8), 4096, 2, 8, 32),      # four matrices, two token tiles
    ((200, 33, 100), 11008, 2, 8, 16),       # three units per wave
    ((130, 70), 512, 2, 8, 128),             # DMA-staged matrix cores, split partial sums
    ((300, 257, 40), 1024, 1, 8, 70),        # the same, one codebook, three matrices
    ((130, 70), 520, 2, 8, 128),             # tiled (in not a multiple of 64)
    ((129, 300), 2048, 1, 16, 64),
]


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: "-".join(map(str, c[0])) + "x" + "x".join(map(str, c[1:])))
def test_grouped(aq, orc, case):
    outs, in_, K, B, batch = case
    ps = _group(outs, in_, K, B, batch, 1700 + sum(outs) + in_ + batch)
    dev = [_dev(p) for p in ps]
    x = dev[0][2]
    refs = [orc.gemv(p["codes"], p["codebooks"], p["x"], K, B) for p in ps]
    for fn in (aq.gemv_grouped, aq.gemm_grouped):
        ys = fn([d[0] for d in dev], [d[1] for d in dev], x)
        for m, (y, r) in enumerate(zip(ys, refs)):
            check_y(y, r, f"{fn.__name__} {case} matrix {m}")


PACKED_GROUPED = [
    ((100, 257, 64), 4096, 2, 8, 1),         # tiled lookup-table kernel
    ((65, 33, 8), 520, 2, 8, 1),
    ((300, 17, 1), 4096, 1, 16, 1),          # position-split kernel
    ((130, 50), 2048, 1, 16, 3),
    ((96, 64), 512, 2, 8, 2),                # unpacked matrix by matrix
    ((40, 24), 512, 2, 16, 1),
    ((300, 17, 64), 4096, 1, 16, 16),        # position split on the matrix cores
    ((130, 50), 2048, 1, 16, 40),
    ((96, 64), 512, 2, 8, 16),               # unpacked, matrix cores
]


@pytest.mark.parametrize("case", PACKED_GROUPED, ids=lambda c: "-".join(map(str, c[0])) + "x" + "x".join(map(str, c[1:])))
def test_packed_grouped(aq, orc, case):
    outs, in_, K, B, batch = case
    ps = _group(outs, in_, K, B, batch, 1800 + sum(outs) + in_ + batch)
    dev = [_dev(p) for p in ps]
    W = [aq.pack_weights(d[0], d[1]) for d in dev]
    ys = aq.gemv_packed_grouped(W, dev[0][2])
    for m, (y, p) in enumerate(zip(ys, ps)):
        check_y(y, orc.gemv(p["codes"], p["codebooks"], p["x"], K, B), f"packed grouped {case} {m}")
    again = aq.gemv_packed_grouped(W, dev[0][2])
    assert all(bool((a == b).all()) for a, b in zip(ys, again))


@pytest.mark.parametrize("case", [
    ("qkv 2x8", (4096, 4096, 4096), 4096, 2, 8, 1), ("qkv 2x8", (4096, 4096, 4096), 4096, 2, 8, 16),
    ("qkv 2x8", (4096, 4096, 4096), 4096, 2, 8, 128), ("gate|up 2x8", (11008, 11008), 4096, 2, 8, 1),
    ("gate|up 2x8", (11008, 11008), 4096, 2, 8, 16), ("qkv 1x16", (4096, 4096, 4096), 4096, 1, 16, 1),
    ("qkv 1x16", (4096, 4096, 4096), 4096, 1, 16, 16), ("gate|up 1x16", (11008, 11008), 4096, 1, 16, 1)],
    ids=lambda c: f"{c[0].replace(' ', '-')}-b{c[5]}")
def test_grouped_full_size(aq, orc, case):
    """The 7B layer's shared-x groups at full size, through aqlm_gemm_grouped and (batch 1)
    aqlm_gemv_packed_grouped, checked on every row at batch 1 (sampled rows above)."""
    import torch
    name, outs, in_, K, B, batch = case
    ps = _group(outs, in_, K, B, batch, 1900 + len(outs) * 10 + K * 100 + batch)
    dev = [_dev(p) for p in ps]
    x = dev[0][2]
    runs = [aq.gemm_grouped([d[0] for d in dev], [d[1] for d in dev], x)]
    if batch == 1:
        runs.append(aq.gemv_packed_grouped([aq.pack_weights(d[0], d[1]) for d in dev], x))
    torch.cuda.synchronize()
    for ys in runs:
        for m, (y, p) in enumerate(zip(ys, ps)):
            _check_rows(y, p, K, B, outs[m], m + batch, f"{case} matrix {m}", orc, batch)


@pytest.mark.parametrize("mode", ["gemm b16", "packed b1"])
def test_grouped_graph_replay(aq, orc, mode):
    import torch
    batch = 16 if mode == "gemm b16" else 1
    ps = _group((500, 300, 64), 2048, 2, 8, batch, 2000 + batch)
    dev = [_dev(p) for p in ps]
    x = dev[0][2]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        if batch == 1:
            W = [aq.pack_weights(d[0], d[1]) for d in dev]
            fn = lambda out=None: aq.gemv_packed_grouped(W, x, out=out)
        else:
            fn = lambda out=None: aq.gemm_grouped([d[0] for d in dev], [d[1] for d in dev], x, out=out)
        eager = [y.clone() for y in fn()]
        ys = [torch.empty_like(y) for y in eager]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn(out=ys)
        for _ in range(3):
            for y in ys:
                y.fill_(3.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert all(bool((a == b).all()) for a, b in zip(ys, eager))
    for m, p in enumerate(ps):
        check_y(eager[m], orc.gemv(p["codes"], p["codebooks"], p["x"], 2, 8), f"graph {mode} {m}")


@pytest.mark.parametrize("case", [
    # out, in, K, B, batch: persistent kernel (in <= 4096, batch <= 16), tiled kernel otherwise
    (160, 1024, 4, 8, 16), (160, 1024, 8, 8, 16), (160, 1024, 4, 8, 17), (160, 1024, 8, 8, 33),
    (300, 4160, 4, 8, 16), (257, 2048, 8, 8, 128), (96, 512, 4, 8, 64), (33, 64, 8, 8, 20),
], ids=lambda c: "x".join(map(str, c)))
def test_mfma_four_and_eight_codebooks(aq, orc, case):
    """K = 4 and 8 codebooks of 8-bit codes on the matrix cores: each group's fp32 fold
    rounded once to fp16 (the dequantized fp16 W) times x."""
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.01, config=2400 + out + K + batch)
    codes, cb, x = _dev(p)
    assert aq.variant_supported("mfma", codes, cb, x)
    assert aq.selected_variant(codes, cb, x, gemm=True) == "mfma"
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    check_y(aq.gemm(codes, cb, x), yref, f"gemm {case}")


@pytest.mark.parametrize("case", [((100, 257), 1024, 4, 8, 16), ((64, 33), 512, 8, 8, 16),
                                  ((64, 33, 17), 1024, 4, 8, 40)],
                         ids=lambda c: "-".join(map(str, c[0])) + "x" + "x".join(map(str, c[1:])))
def test_grouped_four_and_eight_codebooks(aq, orc, case):
    outs, in_, K, B, batch = case
    ps = _group(outs, in_, K, B, batch, 2500 + sum(outs) + K)
    dev = [_dev(p) for p in ps]
    ys = aq.gemm_grouped([d[0] for d in dev], [d[1] for d in dev], dev[0][2])
    for m, (y, p) in enumerate(zip(ys, ps)):
        check_y(y, orc.gemv(p["codes"], p["codebooks"], p["x"], K, B), f"grouped {case} {m}")


@pytest.mark.parametrize("case", [
    # out, in, K, B, batch (aqlm_gemm from batch 512 (16-bit codes, K >= 4) or 1024 (2x8 with
    # in not a multiple of 64): W decoded once, then the dense GEMM kernel; in % 64 == 0 stages
    # k-tiles straight into LDS, other input sizes through registers with the last k-tile's
    # chunks past the input zeroed)
    (300, 4128, 2, 8, 1024), (257, 1024, 1, 16, 600), (96, 512, 4, 8, 513), (1000, 2080, 2, 8, 1100),
    (64, 256, 8, 8, 520), (130, 512, 2, 16, 512), (200, 520, 2, 8, 1030), (129, 4104, 1, 16, 530),
    (513, 8, 1, 16, 515), (1100, 1024, 1, 16, 2050),
], ids=lambda c: "x".join(map(str, c)))
def test_prefill(aq, orc, case):
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=2600 + out + batch)
    codes, cb, x = _dev(p)
    assert aq.selected_variant(codes, cb, x, gemm=True) == "prefill"
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    y = aq.gemm(codes, cb, x)
    check_y(y, yref, f"prefill {case}")
    assert bool((aq.gemm(codes, cb, x) == y).all())


def test_prefill_forced_small_batch(aq, orc):
    """The prefill variant at any batch (named), and its grouped form (matrix by matrix)."""
    for batch in (1, 3, 16):
        p = synth.make_problem(200, 1024, 2, 8, batch=batch, sigma_cb=0.02, config=2700 + batch)
        codes, cb, x = _dev(p)
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], 2, 8)
        check_y(aq.gemv_variant("prefill", codes, cb, x), yref, f"prefill forced b{batch}")
    ps = _group((300, 17, 64), 1024, 1, 16, 520, 2800)
    dev = [_dev(p) for p in ps]
    ys = aq.gemm_grouped([d[0] for d in dev], [d[1] for d in dev], dev[0][2])
    for m, (y, p) in enumerate(zip(ys, ps)):
        check_y(y, orc.gemv(p["codes"], p["codebooks"], p["x"], 1, 16), f"prefill grouped {m}")


def test_prefill_graph_replay(aq, orc):
    """The prefill path captured into a graph (its workspace from the graph's pool) and
    replayed with eager work between replays equals the eager result every time."""
    import torch
    p = synth.make_problem(512, 2048, 1, 16, batch=1024, sigma_cb=0.02, config=2900)
    codes, cb, x = _dev(p)
    assert aq.selected_variant(codes, cb, x, gemm=True) == "prefill"
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = aq.gemm(codes, cb, x).clone()
        y = torch.empty((1024, 512), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            aq.gemm(codes, cb, x, out=y)
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], 1, 16)
        for _ in range(3):
            y.fill_(3.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            check_y(y, yref, "prefill graph")
            assert bool((y == eager).all())


# ------------------------------------------------------------ the C ABI from plain C

C_CHECK = [(300, 4096, 2, 8, 1), (1001, 4096, 1, 16, 1), (257, 2048, 1, 16, 2), (130, 2048, 2, 16, 1),
           (256, 1024, 2, 8, 16)]


@pytest.mark.parametrize("case", C_CHECK, ids=lambda c: "x".join(map(str, c)))
def test_c_abi_program(aq, orc, case, tmp_path):
    """tests/c_abi_check.c (built by build()) runs aqlm_gemv, aqlm_gemm and the packed
    product from C with its own device buffers; its three y match the oracle."""
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(__file__), "c_abi_check")
    if not os.path.exists(exe):
        pytest.skip("tests/c_abi_check not built (build() compiles it)")
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=1700 + out)
    src = tmp_path / "problem.bin"
    with open(src, "wb") as f:
        f.write(np.array([out, in_, K, B, batch], dtype=np.int64).tobytes())
        f.write(np.ascontiguousarray(p["codes"]).tobytes())
        f.write(np.ascontiguousarray(p["codebooks"]).tobytes())
        f.write(np.ascontiguousarray(p["x"]).tobytes())
    dst = tmp_path / "y.bin"
    r = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    ys = np.fromfile(dst, dtype=np.float16).reshape(3, batch, out)
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    for name, y in zip(("aqlm_gemv", "aqlm_gemm", "aqlm_gemv_packed"), ys):
        assert np.all(np.isfinite(y)), name
        e = rel_err(y, yref)
        assert np.all(e <= TOL), f"{name} from C: max rel err {e.max():.3e}"


# The split kernel at its limits: 8 chunk positions per lane (the largest rows it
# takes), the plane form's activation staging full (batch x in/8 = 14336 halves),
# two codebooks, and the two-token pair form; row counts leave waves of a workgroup
# without a first chunk (fewer chunks than waves) or with many.
SPLIT_LIMITS = [
    (300, 32768, 1, 16, 1),    # pair form, activation pairs read from LDS
    (300, 32768, 1, 16, 3),    # plane form, 3 tokens
    (77, 28672, 1, 16, 4),     # plane form, 4 x 3584 activations
    (130, 16384, 2, 16, 1),    # two codebooks, 16 parts
    (2000, 4096, 1, 16, 2),    # two tokens, activation pairs in registers
]


@pytest.mark.parametrize("case", SPLIT_LIMITS, ids=lambda c: "x".join(map(str, c)))
def test_split_limits(aq, orc, case):
    out, in_, K, B, batch = case
    p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=0.02, config=2100 + out + K)
    codes, cb, x = _dev(p)
    assert aq.variant_supported("split", codes, cb, x), case
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
    ys = [aq.gemv_variant("split", codes, cb, x) for _ in range(2)]
    check_y(ys[0], yref, f"split {case}")
    assert bool((ys[0] == ys[1]).all())
    check_y(aq.gemv_packed(aq.pack_weights(codes, cb), x), yref, f"packed {case}")


# Row ranges that end inside a row chunk: 4099 rows = 31 ranges of 129 (chunks of 2
# rows, the last of 1) and one of 100; 1001 rows = 31 ranges of 32 (chunks of 8) and
# one of 9 (a chunk of 8 and one of 1).
SPLIT_RAGGED = [(4099, 11008, 1), (1001, 4096, 1), (1001, 4096, 2), (1001, 11008, 3)]


@pytest.mark.parametrize("case", SPLIT_RAGGED, ids=lambda c: "x".join(map(str, c)))
def test_split_ragged_chunks(aq, orc, case):
    out, in_, batch = case
    p = synth.make_problem(out, in_, 1, 16, batch=batch, sigma_cb=0.02, config=2200 + out + batch)
    codes, cb, x = _dev(p)
    assert aq.variant_supported("split", codes, cb, x), case
    yref = orc.gemv(p["codes"], p["codebooks"], p["x"], 1, 16)
    check_y(aq.gemv_variant("split", codes, cb, x), yref, f"split {case}")
    check_y(aq.gemv_packed(aq.pack_weights(codes, cb), x), yref, f"packed {case}")
