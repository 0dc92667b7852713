"""Pins for the oracle's combine-with-shared-expert and combine backward.

combine_shared is pinned by: shared = 0 reduces it to combine bit for bit;
exact rational arithmetic (sum_j w_j y_j + shared, rounded once to bf16)
within 1 bf16 ulp wherever the sum is not cancelling; a float64 numpy sum
within the 1e-2 tolerance everywhere.

combine_backward is pinned by: grad_recv against numpy float32 multiplies and
torch's bf16 cast, placed with the layout's rows; unit weights make grad_recv
an exact copy of grad_out; grad_w against float64 numpy dot products (within
1 fp32 ulp) and exact fractions on tiny inputs; the adjoint identity
sum_t <combine(y)_t, g_t> = sum_p w_p grad_w[p] up to combine's bf16 rounding.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, make_expert_rows, bf16_from_f32


def f32(b):
    return oracle.bf16_to_f32(b)


def setup(name="ds16b", T=256, seed=0):
    w = make_workload(name, T=T)
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H, seed=seed + 1)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    return w, L, ys


def test_combine_shared_zero_is_combine():
    w, L, ys = setup()
    zero = np.zeros((w.T, w.H), np.uint16)
    assert np.array_equal(oracle.combine_shared(ys, w.topk_idx, L, w.topk_w, zero),
                          oracle.combine(ys, w.topk_idx, L, w.topk_w))


def test_combine_shared_against_float64_and_exact():
    w, L, ys = setup(T=64)
    rng = np.random.default_rng(4)
    shared = bf16_from_f32(rng.standard_normal((w.T, w.H)).astype(np.float32))
    out = oracle.combine_shared(ys, w.topk_idx, L, w.topk_w, shared)
    yrow = f32(np.concatenate(ys)[L.slot_of]).astype(np.float64).reshape(w.T, w.k, w.H)
    wt = w.topk_w.astype(np.float64)
    terms = np.einsum("tk,tkh->th", wt, yrow)
    ref = terms + f32(shared).astype(np.float64)
    got = f32(out).astype(np.float64)
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3)) <= 1e-2
    # exact rational check on well-conditioned entries of a few tokens
    mag = np.einsum("tk,tkh->th", np.abs(wt), np.abs(yrow)) + np.abs(f32(shared))
    for t in range(4):
        for h in range(0, w.H, 97):
            S = sum(Fraction(float(w.topk_w[t, j])) * Fraction(float(yrow[t, j, h])) for j in range(w.k))
            S += Fraction(float(f32(shared[t, h:h + 1])[0]))
            if abs(float(S)) < 2.0 ** -6 * mag[t, h]:
                continue
            exact = bf16_from_f32(np.array([float(S)], np.float32))[0]
            # float(S) -> float32 -> bf16 is a double rounding; allow the 1 ulp it can cost
            assert abs(int(out[t, h]) - int(exact)) <= 1


def test_combine_backward_grad_recv_matches_numpy_and_torch():
    w, L, ys = setup()
    rng = np.random.default_rng(5)
    g = bf16_from_f32(rng.standard_normal((w.T, w.H)).astype(np.float32))
    gr, gw = oracle.combine_backward(g, w.topk_idx, L, w.topk_w, None)
    assert gw is None
    allrows = np.concatenate(gr)
    prod = (w.topk_w.reshape(-1, 1).astype(np.float32)
            * np.repeat(f32(g), w.k, axis=0)).astype(np.float32)       # one binary32 multiply
    ref = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(allrows[L.slot_of], ref)


def test_combine_backward_unit_weights_copy():
    w, L, ys = setup()
    g = bf16_from_f32(np.random.default_rng(6).standard_normal((w.T, w.H)).astype(np.float32))
    gr, _ = oracle.combine_backward(g, w.topk_idx, L, None, None)
    assert np.array_equal(np.concatenate(gr)[L.slot_of], np.repeat(g, w.k, axis=0))


def test_combine_backward_grad_w_dot_products():
    w, L, ys = setup()
    g = bf16_from_f32(np.random.default_rng(7).standard_normal((w.T, w.H)).astype(np.float32))
    _, gw = oracle.combine_backward(g, w.topk_idx, L, w.topk_w, ys)
    yrow = f32(np.concatenate(ys)[L.slot_of]).astype(np.float64).reshape(w.T, w.k, w.H)
    ref = np.einsum("th,tkh->tk", f32(g).astype(np.float64), yrow).astype(np.float32)
    ulp = np.abs(np.spacing(ref))
    assert np.all(np.abs(gw - ref) <= ulp)


def test_combine_backward_grad_w_exact_tiny():
    rng = np.random.default_rng(8)
    T, H, k, E, R = 3, 16, 3, 6, 2
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    L = oracle.layout(idx, E, R)
    ys = [bf16_from_f32(rng.standard_normal((int(c), H)).astype(np.float32)) for c in L.rank_counts]
    g = bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    _, gw = oracle.combine_backward(g, idx, L, None, ys)
    rank = idx.ravel() // (E // R)
    for t in range(T):
        for j in range(k):
            p = t * k + j
            yr = f32(ys[rank[p]][L.row_of[p]])
            S = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(f32(g[t]), yr))
            assert gw[t, j] == np.float32(float(S))


def test_combine_backward_adjoint_identity():
    w, L, ys = setup(T=128)
    g = bf16_from_f32(np.random.default_rng(9).standard_normal((w.T, w.H)).astype(np.float32))
    out = f32(oracle.combine(ys, w.topk_idx, L, w.topk_w)).astype(np.float64)
    _, gw = oracle.combine_backward(g, w.topk_idx, L, w.topk_w, ys)
    gd = f32(g).astype(np.float64)
    lhs = float(np.sum(out * gd))
    rhs = float(np.sum(w.topk_w.astype(np.float64) * gw.astype(np.float64)))
    bound = 2.0 ** -8 * float(np.sum(np.abs(out * gd)))   # combine's bf16 rounding
    assert abs(lhs - rhs) <= bound
