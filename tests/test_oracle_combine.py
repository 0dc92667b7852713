"""Pins for the oracle's top-k weighted combine (fp32 fused multiply-add in
ascending j from +0, one bf16 rounding at the end).

Pinned against:
  * exact rational arithmetic (Python fractions) of sum_j w_j * y_j, rounded
    once to bf16 by a rounding written here from the definition: agreement to
    <= 1 bf16 ulp (the fp32 accumulation may move a sum across a bf16 rounding
    boundary only by its own rounding error);
  * identity experts with weights that sum to 1: combine(dispatch(x)) == x
    bitwise (BF16), == the dequantized row (FP8);
  * k = 1, unit weights: combine == un-permute;
  * a float64 numpy sum within the 1e-2 relative tolerance on a full-size
    workload, and x * sum(w) for the workload whose weights are not
    renormalized.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from workloads import make_workload, make_expert_rows, bf16_from_f32


def bf16_rne_exact(S: Fraction) -> int:
    """Nearest bf16 (8 significant bits, min exponent -126, subnormal spacing
    2^-133), ties to even, of an exact rational; returns the bit pattern."""
    if S == 0:
        return 0
    neg = S < 0
    a = -S if neg else S
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    n = a / q
    fl = math.floor(n)
    d = n - fl
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * q
    if val >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        bits = int(np.array([float(val)], np.float32).view(np.uint32)[0] >> 16)
    return bits | (0x8000 if neg else 0)


def ordered(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_combine_matches_exact_rational(seed):
    rng = np.random.default_rng(seed)
    T, H, k, E, R = 6, 16, 5, 8, 2
    idx = rng.integers(0, E, (T, k), dtype=np.int32)
    L = oracle.layout(idx, E, R)
    ys = [bf16_from_f32((rng.standard_normal((int(c), H)) * 2.0 ** rng.integers(-3, 4, (int(c), 1)))
                        .astype(np.float32)) for c in L.rank_counts]
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.combine(ys, idx, L, w)
    rank = idx.ravel() // (E // R)
    exact = np.empty((T, H), np.uint16)
    for t in range(T):
        for h in range(H):
            S = Fraction(0)
            for j in range(k):
                p = t * k + j
                yv = float(oracle.bf16_to_f32(ys[rank[p]][L.row_of[p], h:h + 1])[0])
                S += Fraction(float(w[t, j])) * Fraction(yv)
            exact[t, h] = bf16_rne_exact(S)
    assert np.max(np.abs(ordered(out) - ordered(exact))) <= 1


def test_combine_identity_bf16_is_exact():
    w = make_workload("tiny")
    L = oracle.layout(w.topk_idx, w.E, w.R)
    recv = oracle.dispatch_bf16(w.x, w.topk_idx, L)
    out = oracle.combine(recv, w.topk_idx, L, w.topk_w)
    assert np.array_equal(out, w.x)


def test_combine_identity_fp8_returns_dequantized_row():
    w = make_workload("decode")
    L = oracle.layout(w.topk_idx, w.E, w.R)
    rq, rs = oracle.dispatch_fp8(w.x, w.topk_idx, L)
    yhat = oracle.dequant_identity_expert(rq, rs)
    out = oracle.combine(yhat, w.topk_idx, L, w.topk_w)
    q, s = oracle.quantize_rows(w.x)
    ref = oracle.dequant_identity_expert([q], [s])[0]
    # the accumulator starts at +0 and (+0) + (-0) = +0, so a -0 row element
    # (a small negative value that quantized to the -0 code) comes back as +0
    ref = np.where(ref == 0x8000, np.uint16(0), ref)
    assert np.array_equal(out, ref)


def test_combine_k1_unit_weights_is_unpermute():
    rng = np.random.default_rng(7)
    T, H, E, R = 50, 64, 6, 3
    idx = rng.integers(0, E, (T, 1), dtype=np.int32)
    L = oracle.layout(idx, E, R)
    ys = [bf16_from_f32(rng.standard_normal((int(c), H)).astype(np.float32)) for c in L.rank_counts]
    assert np.array_equal(oracle.combine(ys, idx, L, None), oracle.unpermute(ys, idx, L))
    ones = np.ones((T, 1), np.float32)
    assert np.array_equal(oracle.combine(ys, idx, L, ones), oracle.unpermute(ys, idx, L))


def rel_err(g: np.ndarray, r: np.ndarray) -> float:
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), 1e-3)))


def test_combine_identity_not_renormalized():
    w = make_workload("ds16b", T=512)
    L = oracle.layout(w.topk_idx, w.E, w.R)
    recv = oracle.dispatch_bf16(w.x, w.topk_idx, L)
    out = oracle.bf16_to_f32(oracle.combine(recv, w.topk_idx, L, w.topk_w)).astype(np.float64)
    ref = oracle.bf16_to_f32(w.x).astype(np.float64) * w.topk_w.astype(np.float64).sum(1, keepdims=True)
    assert rel_err(out, ref) <= 1e-2


def test_combine_random_experts_vs_float64():
    w = make_workload("ds16b")
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    out = oracle.bf16_to_f32(oracle.combine(ys, w.topk_idx, L, w.topk_w)).astype(np.float64)
    yrow = oracle.bf16_to_f32(y[L.slot_of]).astype(np.float64).reshape(w.T, w.k, w.H)
    ref = np.einsum("tk,tkh->th", w.topk_w.astype(np.float64), yrow)
    assert rel_err(out, ref) <= 1e-2
