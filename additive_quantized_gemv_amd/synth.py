"""Seeded synthetic inputs for the additive-quantized matrix-vector product.

This module only draws random numbers.  It holds none of the method's arithmetic
(no decode, no dot products): it produces the three raw buffers that define one
problem -- codes, codebooks and activations -- and both the GPU path and the CPU
checker read the very same bytes.

Generator (stated so that anyone can re-derive the bytes):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014), used in counter form: word n of stream ``seed`` is
  ``mix64(seed + (n + 1) * 0x9E3779B97F4A7C15)`` with the published finaliser
  (shifts 30, 27, 31; multipliers 0xBF58476D1CE4E5B9, 0x94D049BB133111EB).
* Codes: the top ``B`` bits of one 64-bit word per code.  Uniform over all
  ``2**B`` patterns; 16-bit codes are the unsigned pattern 0..65535.
* Normals: Box-Muller in double precision on pairs of words
  (u1 = ((w >> 11) + 1) * 2**-53 in (0, 1], u2 = (w >> 11) * 2**-53 in [0, 1)),
  scaled by sigma and rounded to fp16 in ONE round-to-nearest-even step from
  double (numpy converts double to half directly, without going through float).
* Seed of (config c, rotation copy r, tensor t) is ``1000003*c + 1009*r + t``
  with t = 0 codes, 1 codebooks, 2 activations.

Shapes follow the format of the AQLM pages (page "AQLM (Additive Quantization
for LLMs)", section "Niveau intermediaire"): codebooks are [K][2**B][8] fp16,
codes are [out][in/8][K] (uint8 for B = 8, uint16 for B = 16), activations are
[batch][in] fp16.
"""
from __future__ import annotations

import hashlib

import numpy as np

GROUP = 8
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def stream_seed(config: int, copy: int, tensor: int) -> int:
    """Seed for (config id, rotation copy, tensor id); tensor 0/1/2 = codes/codebooks/x."""
    return 1000003 * int(config) + 1009 * int(copy) + int(tensor)


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Words start..start+n-1 of the counter-form SplitMix64 stream ``seed``."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + ctr * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform_codes(seed: int, shape, bits: int) -> np.ndarray:
    """Codes drawn uniformly over 2**bits patterns: top ``bits`` bits of each word."""
    if bits not in (8, 16):
        raise ValueError("bits must be 8 or 16")
    n = int(np.prod(shape))
    dt = np.uint8 if bits == 8 else np.uint16
    out = np.empty(n, dtype=dt)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = (splitmix64(seed, m, s) >> np.uint64(64 - bits)).astype(dt)
    return out.reshape(shape)


def normal_f64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """n standard normals (double) by Box-Muller over word pairs of stream ``seed``."""
    npairs = (n + 1) // 2
    w = splitmix64(seed, 2 * npairs, 2 * (start // 2))
    u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    r = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * np.pi * u2
    z = np.empty(2 * npairs, dtype=np.float64)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    return z[:n]


def normal_f16(seed: int, shape, sigma: float) -> np.ndarray:
    """fp16 values ~ N(0, sigma^2), rounded once from double (RNE)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    step = _CHUNK & ~1
    for s in range(0, n, step):
        m = min(step, n - s)
        out[s:s + m] = (normal_f64(seed, m, s) * float(sigma)).astype(np.float16)
    return out.reshape(shape)


def make_problem(out_features: int, in_features: int, K: int, B: int, batch: int = 1,
                 sigma_cb: float = 0.02, sigma_x: float = 1.0, config: int = 0,
                 copy: int = 0) -> dict:
    """One seeded problem: codes [out][in/8][K], codebooks [K][2^B][8] fp16, x [batch][in] fp16."""
    if in_features % GROUP:
        raise ValueError("in_features must be a multiple of 8")
    G = in_features // GROUP
    codes = uniform_codes(stream_seed(config, copy, 0), (out_features, G, K), B)
    codebooks = normal_f16(stream_seed(config, copy, 1), (K, 1 << B, GROUP), sigma_cb)
    x = normal_f16(stream_seed(config, copy, 2), (batch, in_features), sigma_x)
    return {"codes": codes, "codebooks": codebooks, "x": x, "out": out_features,
            "in": in_features, "K": K, "B": B, "batch": batch}


def buffer_hash(a: np.ndarray) -> str:
    """Short content hash of a buffer, for logs."""
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]


# The five workloads the pages' format is exercised on.  Sizes are
# Llama-2-7B / 70B projection shapes; every one is a synthetic stand-in.
CONFIGS = {
    "tiny_2x8": dict(shapes=[(256, 512)], K=2, B=8, sigma_cb=0.05, batches=[1]),
    "proj_1x16_4096": dict(shapes=[(4096, 4096)], K=1, B=16, sigma_cb=0.02, batches=[1]),
    "mlp_2x8_7b": dict(shapes=[(11008, 4096), (4096, 11008)], K=2, B=8, sigma_cb=0.02,
                       batches=[1]),
    "mlp_1x16_7b": dict(shapes=[(11008, 4096), (4096, 11008)], K=1, B=16, sigma_cb=0.02,
                        batches=[1]),
    "mlp_1x16_70b": dict(shapes=[(28672, 8192), (8192, 28672)], K=1, B=16, sigma_cb=0.02,
                         batches=[1, 4]),
    "layer_2x8_7b": dict(shapes=[(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)],
                         K=2, B=8, sigma_cb=0.02, batches=[1, 16, 128]),
    "layer_1x16_7b": dict(shapes=[(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)],
                          K=1, B=16, sigma_cb=0.02, batches=[1, 16, 128]),
}
