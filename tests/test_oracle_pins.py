"""Pins of the CPU oracle to what the pages and mathematics fix (no GPU needed).

Each ``pin_*`` function raises AssertionError when the oracle it is given is
wrong.  The ``test_*`` wrappers run them on the real oracle; ``test_mutants``
compiles deliberately broken copies of the oracle (a dropped codebook term, a
shifted group index, reversed vector entries, a flipped sign, a shifted
activation index) and checks that each one fails at least one pin.

Sources: page "AQLM (Additive Quantization for LLMs)" (brain.gartu.xyz),
section "Niveau intermediaire" (decode rule, codebook shape, bitrate formula and
its worked examples); page "AQLM -- ..." (devtrends.ru), sections
"Kak eto rabotaet tekhnicheski?" (groups of 8) and "Skhemy kvantovaniya"
(1x16, 2x8); page "AQLM Additive Quantization (Egiazarian 2024)" (jisaku.com),
feature list (8x memory reduction from fp16 to 2 bits).
"""
import json
import os

import numpy as np
import pytest

from additive_quantized_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cb_from_entries(K, B, entries):
    cb = np.zeros((K, 1 << B, 8), dtype=np.float16)
    for key, vec in entries.items():
        k, c = (int(v) for v in key.split(","))
        cb[k, c] = np.array(vec, dtype=np.float16)
    return cb


def _small(K, B, out=24, in_=64, sigma=0.05, seed=7, batch=2):
    return synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=sigma, config=seed)


# ---------------------------------------------------------------- pins

def pin_bitrate(orc):
    """Worked examples of the bitrate formula; 8x reduction from fp16."""
    with open(os.path.join(GOLDEN, "bitrate_examples.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for K, entries, g, bits, *_ in rows:
        B = int(np.log2(int(entries)))
        assert orc.bits_per_weight(int(K), B, int(g)) == float(bits)
    assert 16.0 / orc.bits_per_weight(1, 16, 8) == 8.0
    assert 16.0 / orc.bits_per_weight(2, 8, 8) == 8.0
    for out_f, in_f in [(256, 512), (4096, 4096), (11008, 4096), (4096, 11008),
                        (28672, 8192)]:
        for K, B in [(1, 16), (2, 8), (2, 16), (8, 8), (3, 8)]:
            bits = orc.bits_per_weight(K, B, 8)
            assert orc.codes_bytes(out_f, in_f, K, B) * 8 == bits * out_f * in_f


def pin_half_conversion(orc):
    """All 65,536 binary16 patterns decode like numpy's independent conversion."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = orc.half_to_float(pats)
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def pin_float_to_half(orc):
    """RNE float -> binary16 agrees with numpy on random values and on every tie kind."""
    rng = np.random.default_rng(5)
    vals = [rng.standard_normal(3000).astype(np.float32) * s for s in (1e-7, 1e-5, 0.02, 1, 300)]
    # exact midpoints between neighbouring halves (ties), normal and subnormal
    h = np.arange(0, 0x7BFF, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    specials = np.array([0.0, -0.0, 65504, 65519.99, 65520, -65520, 1e30, 2.0 ** -25,
                         2.0 ** -25 * 1.0000001, 2.0 ** -24 * 1.5, 6.1035156e-05],
                        dtype=np.float32)
    x = np.concatenate(vals + [mids, -mids, specials])
    mine = orc.float_to_half(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def pin_int_cases(orc):
    """Hand-computed integer cases: decoded W and y exactly."""
    with open(os.path.join(GOLDEN, "int_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        K, B = c["K"], c["B"]
        dt = np.uint8 if B == 8 else np.uint16
        codes = np.array(c["codes"], dtype=dt)
        cb = _cb_from_entries(K, B, c["codebook_entries"])
        x = np.array(c["x"], dtype=np.float16)
        W = orc.decode(codes, cb, K, B)
        assert np.array_equal(W, np.array(c["W"], dtype=np.float32)), c["name"]
        y = orc.matvec(W, x)
        assert np.array_equal(y, np.array(c["y"], dtype=np.float64)), c["name"]
        yr = orc.gemv_rows(codes, cb, x, K, B, np.arange(c["out"]))
        assert np.array_equal(yr, y), c["name"]


def pin_onehot_bruteforce(orc):
    """Decode equals the explicit sum of one-hot selections (dense matmul in double)."""
    for K, B in [(2, 8), (1, 16), (3, 8), (1, 8)]:
        p = _small(K, B, out=6, in_=32, sigma=0.05, seed=11 + K)
        codes, cb = p["codes"], p["codebooks"]
        W = orc.decode(codes, cb, K, B)
        out_f, G, _ = codes.shape
        E = 1 << B
        ref = np.zeros((out_f, G, 8), dtype=np.float64)
        for k in range(K):
            onehot = np.zeros((out_f * G, E), dtype=np.float64)
            onehot[np.arange(out_f * G), codes[:, :, k].ravel().astype(np.int64)] = 1.0
            ref += (onehot @ cb[k].astype(np.float64)).reshape(out_f, G, 8)
        # at these magnitudes (|c| < 1) sums of <= 3 fp16 values are exact in fp32
        assert np.array_equal(W.astype(np.float64), ref.reshape(out_f, G * 8))


def pin_exhaustive_group(orc):
    """One group over every code value: all 256x256 pairs (2x8) and all 65,536 codes (1x16)."""
    p = _small(2, 8, out=1, in_=8, sigma=0.05, seed=21)
    cb = p["codebooks"]
    c0, c1 = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    codes = np.stack([c0.ravel(), c1.ravel()], axis=1).astype(np.uint8).reshape(-1, 1, 2)
    W = orc.decode(codes, cb, 2, 8)
    ref = cb[0][c0.ravel()].astype(np.float64) + cb[1][c1.ravel()].astype(np.float64)
    assert np.array_equal(W.astype(np.float64), ref)
    p = _small(1, 16, out=1, in_=8, sigma=0.02, seed=22)
    cb = p["codebooks"]
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(-1, 1, 1)
    W = orc.decode(codes, cb, 1, 16)
    assert np.array_equal(W, cb[0].astype(np.float32))  # K = 1 is a pure table lookup


def pin_k1_lookup(orc):
    """K = 1: each row is its codebook rows concatenated, in group order."""
    p = _small(1, 16, out=9, in_=48, seed=31)
    W = orc.decode(p["codes"], p["codebooks"], 1, 16)
    ref = p["codebooks"][0][p["codes"][:, :, 0].astype(np.int64)].reshape(9, 48)
    assert np.array_equal(W, ref.astype(np.float32))


def pin_additivity(orc):
    """decode(C0, C1) == decode(C0, 0) + decode(0, C1) bit-exactly; y adds up in double."""
    p = _small(2, 8, out=16, in_=64, seed=41)
    codes, cb, x = p["codes"], p["codebooks"], p["x"]
    z = np.zeros_like(cb[0])
    W = orc.decode(codes, cb, 2, 8)
    Wa = orc.decode(codes, np.stack([cb[0], z]), 2, 8)
    Wb = orc.decode(codes, np.stack([z, cb[1]]), 2, 8)
    assert np.array_equal(W, Wa + Wb)
    y, ya, yb = orc.matvec(W, x), orc.matvec(Wa, x), orc.matvec(Wb, x)
    assert np.max(np.abs(y - (ya + yb))) <= 1e-12 * np.max(np.abs(y))


def pin_linearity(orc):
    """Linear in x (integer-valued activations keep every sum exact) and in the codebooks."""
    p = _small(2, 8, out=20, in_=96, seed=51)
    codes, cb = p["codes"], p["codebooks"]
    W = orc.decode(codes, cb, 2, 8)
    rng = np.random.default_rng(3)
    x1 = rng.integers(-8, 9, size=(1, 96)).astype(np.float16)
    x2 = rng.integers(-8, 9, size=(1, 96)).astype(np.float16)
    a, b = 2.0, -3.0
    x3 = (a * x1.astype(np.float64) + b * x2.astype(np.float64)).astype(np.float16)
    y1, y2, y3 = orc.matvec(W, x1), orc.matvec(W, x2), orc.matvec(W, x3)
    assert np.max(np.abs(y3 - (a * y1 + b * y2))) <= 1e-12 * max(1.0, np.max(np.abs(y3)))
    # scaling the codebooks up by a power of two (no fp16 overflow, and subnormals
    # only gain bits) scales W and y exactly
    for m in (2, 5):
        cbs = (cb.astype(np.float64) * 2.0 ** m).astype(np.float16)
        Ws = orc.decode(codes, cbs, 2, 8)
        assert np.array_equal(Ws, W * np.float32(2.0 ** m))
        assert np.array_equal(orc.matvec(Ws, p["x"]), orc.matvec(W, p["x"]) * 2.0 ** m)


def pin_permutation(orc):
    """Relabel codebook entries (and remap codes), or swap the two codebooks: W unchanged."""
    p = _small(2, 8, out=12, in_=64, seed=61)
    codes, cb = p["codes"], p["codebooks"]
    W = orc.decode(codes, cb, 2, 8)
    rng = np.random.default_rng(8)
    perm = rng.permutation(256)            # new entry n holds old entry perm[n]
    inv = np.argsort(perm)                 # old entry e now sits at inv[e]
    cbp = np.stack([cb[0][perm], cb[1][perm]])
    codesp = inv[codes.astype(np.int64)].astype(np.uint8)
    assert np.array_equal(orc.decode(codesp, cbp, 2, 8), W)
    swapped = np.ascontiguousarray(codes[:, :, ::-1])
    assert np.array_equal(orc.decode(swapped, cb[::-1].copy(), 2, 8), W)


def pin_unit_vectors(orc):
    """x = e_i gives column i; x = 1 gives row sums; x = 0 gives +0; column-major loop agrees."""
    p = _small(2, 8, out=10, in_=40, seed=71)
    W = orc.decode(p["codes"], p["codebooks"], 2, 8)
    for i in (0, 7, 8, 39):
        e = np.zeros((1, 40), dtype=np.float16)
        e[0, i] = 1
        assert np.array_equal(orc.matvec(W, e)[0], W[:, i].astype(np.float64))
    ones = np.ones((1, 40), dtype=np.float16)
    rs = W.astype(np.float64).sum(axis=1)
    assert np.max(np.abs(orc.matvec(W, ones)[0] - rs)) <= 1e-12 * np.max(np.abs(rs))
    y0 = orc.matvec(W, np.zeros((1, 40), dtype=np.float16))
    assert np.all(y0 == 0) and not np.any(np.signbit(y0))
    x = p["x"]
    colmajor = np.zeros((x.shape[0], 10))
    for i in range(40):                    # independent loop order: column by column
        colmajor += np.outer(x[:, i].astype(np.float64), W[:, i].astype(np.float64))
    y = orc.matvec(W, x)
    assert np.max(np.abs(y - colmajor)) <= 1e-12 * np.max(np.abs(y))


def pin_signed_zero_fold(orc):
    """The fold starts from C_0's value: -0 + -0 stays -0 (a +0 start would give +0)."""
    cb = np.zeros((2, 256, 8), dtype=np.float16)
    cb[:, 3] = np.float16(-0.0)
    codes = np.full((1, 1, 2), 3, dtype=np.uint8)
    W = orc.decode(codes, cb, 2, 8)
    assert np.all(np.signbit(W))


def pin_model_sizes(orc):
    """Soft closed-form check of the format against sizes quoted on the pages."""
    with open(os.path.join(GOLDEN, "model_sizes.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for name, L, h, inter, kv, vocab, quoted, tol in rows:
        L, h, inter, kv, vocab = int(L), int(h), int(inter), int(kv), int(vocab)
        shapes = [(h, h), (kv, h), (kv, h), (h, h), (inter, h), (inter, h), (h, inter)]
        code_b = sum(orc.codes_bytes(o, i, 1, 16) for o, i in shapes) * L
        cb_b = 7 * L * (1 << 16) * 8 * 2
        emb_b = 2 * vocab * h * 2
        gb = (code_b + cb_b + emb_b) / 1e9
        assert abs(gb - float(quoted)) <= float(tol), (name, gb)


ALL_PINS = [pin_bitrate, pin_half_conversion, pin_float_to_half, pin_int_cases,
            pin_onehot_bruteforce, pin_exhaustive_group, pin_k1_lookup, pin_additivity,
            pin_linearity, pin_permutation, pin_unit_vectors, pin_signed_zero_fold,
            pin_model_sizes]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_invariance(orc):
    """Rows are split across threads but each row is summed in a fixed order."""
    from oracle import Oracle
    p = _small(2, 8, out=64, in_=256, seed=81, batch=3)
    y1 = Oracle(nthreads=1).gemv(p["codes"], p["codebooks"], p["x"], 2, 8)
    y8 = Oracle(nthreads=8).gemv(p["codes"], p["codebooks"], p["x"], 2, 8)
    assert np.array_equal(y1, y8)
    rows = np.array([0, 5, 63, 17])
    assert np.array_equal(orc.gemv_rows(p["codes"], p["codebooks"], p["x"], 2, 8, rows),
                          y1[:, rows])


def test_rejects_bad_args(orc):
    p = _small(2, 8, out=4, in_=16, seed=91)
    with pytest.raises(ValueError):
        orc.decode(p["codes"], p["codebooks"], 3, 8)
    with pytest.raises(ValueError):
        orc.gemv_rows(p["codes"], p["codebooks"], p["x"], 2, 8, [4])


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5])
def test_mutants_fail_a_pin(tmp_path, mutant):
    """A planted mistake in a copy of the oracle is caught by at least one pin."""
    import oracle
    path = str(tmp_path / f"liboracle_mutant{mutant}.so")
    oracle.build(path, extra_flags=[f"-DORACLE_MUTANT={mutant}"])
    bad = oracle.Oracle(lib=oracle.load(path))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(bad)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant} passed every pin"
