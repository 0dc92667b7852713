"""Pins for the oracle's expert activation (SiLU-and-multiply) and its
per-128 FP8 re-quantization.

silu_mul is pinned by torch's float64 silu (a library special case) within
1 fp32 ulp, by silu(0) = 0 and by the identity silu(v) - silu(-v) = v (up = 1),
which fails for a wrong sign or a dropped term.  The re-quantization of fp32
activations is pinned, as the dispatch quantizer is, by numpy float32
division and torch's E4M3 cast, the amax -> +-448 property and the
half-ulp error bound; and the whole silu_mul_quant is checked to be
silu_mul followed by that quantizer.
"""
import numpy as np
import torch

import oracle
from workloads import bf16_from_f32


def rows(n, I, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    return bf16_from_f32((rng.standard_normal((n, 2 * I)) * scale).astype(np.float32))


def test_silu_mul_matches_torch_float64():
    r = rows(64, 512, 1)
    a = oracle.silu_mul(r)
    f = oracle.bf16_to_f32(r).astype(np.float64)
    g, u = f[:, :512], f[:, 512:]
    ref = (torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u).astype(np.float32)
    assert np.all(np.abs(a - ref) <= np.abs(np.spacing(ref)))


def test_silu_identities():
    I = 256
    v = bf16_from_f32(np.linspace(-20, 20, I).astype(np.float32))
    one = bf16_from_f32(np.ones(I, np.float32))
    neg = (v ^ np.uint16(0x8000)).astype(np.uint16)
    ap = oracle.silu_mul(np.concatenate([v, one])[None, :])[0].astype(np.float64)
    an = oracle.silu_mul(np.concatenate([neg, one])[None, :])[0].astype(np.float64)
    x = oracle.bf16_to_f32(v).astype(np.float64)
    # silu(v) - silu(-v) = v, each side rounded once to fp32
    assert np.all(np.abs((ap - an) - x) <= 2 * np.abs(np.spacing(np.float32(np.abs(ap) + np.abs(an)))))
    zero = oracle.silu_mul(np.zeros((1, 2 * I), np.uint16))
    assert np.all(zero == 0)


def test_quantize_f32_matches_numpy_and_torch():
    a = oracle.silu_mul(rows(48, 1024, 2))
    q, s = oracle.quantize_f32_rows(a)
    blocks = a.reshape(48, 8, 128)
    amax = np.abs(blocks).max(axis=2)
    s2 = (amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    ratio = (blocks / s2[:, :, None]).astype(np.float32)
    q2 = torch.from_numpy(np.ascontiguousarray(ratio)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, q2.reshape(48, 1024))
    at = np.abs(blocks).argmax(axis=2)
    top = np.take_along_axis(q.reshape(48, 8, 128), at[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    dec = oracle.e4m3_decode(q).reshape(48, 8, 128).astype(np.float64) * s.astype(np.float64)[:, :, None]
    bound = np.maximum(2.0 ** -4 * np.abs(blocks), 2.0 ** -10 * s[:, :, None]) * (1 + 2.0 ** -20)
    assert np.all(np.abs(dec - blocks) <= bound)


def test_silu_mul_quant_is_composition():
    r = rows(16, 2048, 3)
    q, s = oracle.silu_mul_quant(r)
    q2, s2 = oracle.quantize_f32_rows(oracle.silu_mul(r))
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
