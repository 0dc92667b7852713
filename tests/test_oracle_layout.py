"""Pins for the oracle's routing layout (per-expert counts, prefix sums, rank
ranges, stable slot assignment).

Pinned against:
  * numpy library special cases: counts == bincount, src == stable argsort;
  * brute force: every index array of a few tiny (T, k, E) shapes, against a
    sort of the (expert, pair) tuples written here in plain Python;
  * the invariants the method fixes: the counts sum to T*k, slot and src are
    inverse bijections onto [0, T*k), each slot lies in its expert's segment,
    segments keep ascending pair order, rank r's range starts at expert r*E/R;
  * the pages' worked arithmetic (tests/golden/pages_arithmetic.json).
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import CONFIGS, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_arithmetic.json")


def check_invariants(idx: np.ndarray, E: int, R: int, L) -> None:
    T, k = idx.shape
    P = T * k
    flat = idx.ravel()
    El = E // R
    assert L.expert_counts.sum() == P and L.rank_counts.sum() == P
    assert L.expert_offsets[0] == 0 and L.expert_offsets[-1] == P
    assert np.all(np.diff(L.expert_offsets) == L.expert_counts)
    assert np.array_equal(np.sort(L.slot_of), np.arange(P))
    assert np.array_equal(L.src_of[L.slot_of], np.arange(P))
    assert np.array_equal(L.slot_of[L.src_of], np.arange(P))
    lo = L.expert_offsets[flat]
    hi = L.expert_offsets[flat + 1]
    assert np.all((L.slot_of >= lo) & (L.slot_of < hi))
    # stability: within each expert segment the source pairs ascend
    seg_expert = flat[L.src_of]
    same = seg_expert[1:] == seg_expert[:-1]
    assert np.all(L.src_of[1:][same] > L.src_of[:-1][same])
    for r in range(R):
        assert L.rank_offsets[r] == L.expert_offsets[r * El]
        assert L.rank_counts[r] == L.expert_offsets[(r + 1) * El] - L.expert_offsets[r * El]
    assert L.rank_offsets[R] == P
    rank = flat // El
    assert np.array_equal(L.row_of, L.slot_of - L.rank_offsets[rank])
    assert np.all((L.row_of >= 0) & (L.row_of < L.rank_counts[rank]))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_layout_library_special_cases(name):
    w = make_workload(name)
    L = oracle.layout(w.topk_idx, w.E, w.R)
    flat = w.topk_idx.ravel()
    assert np.array_equal(L.expert_counts, np.bincount(flat, minlength=w.E))
    assert np.array_equal(L.src_of, np.argsort(flat, kind="stable"))
    check_invariants(w.topk_idx, w.E, w.R, L)


def brute_layout(idx, E, R):
    """Pure-Python definition: sort pairs by (expert, pair index)."""
    flat = [int(v) for v in np.asarray(idx).ravel()]
    P = len(flat)
    order = sorted(range(P), key=lambda p: (flat[p], p))
    slot = [0] * P
    for s, p in enumerate(order):
        slot[p] = s
    counts = [flat.count(e) for e in range(E)]
    return counts, order, slot


@pytest.mark.parametrize("T,k,E,R", [(1, 1, 1, 1), (1, 1, 2, 1), (1, 1, 3, 3), (1, 1, 4, 2),
                                     (2, 2, 3, 1), (3, 2, 3, 3), (2, 3, 4, 2), (1, 4, 4, 4),
                                     (6, 1, 4, 2)])
def test_layout_exhaustive_tiny(T, k, E, R):
    n = 0
    for combo in itertools.product(range(E), repeat=T * k):
        idx = np.array(combo, np.int32).reshape(T, k)
        L = oracle.layout(idx, E, R)
        counts, order, slot = brute_layout(idx, E, R)
        assert list(L.expert_counts) == counts
        assert list(L.src_of) == order
        assert list(L.slot_of) == slot
        check_invariants(idx, E, R, L)
        n += 1
    assert n == E ** (T * k)


@settings(max_examples=150, deadline=None)
@given(T=st.integers(1, 300), k=st.integers(1, 9), R=st.integers(1, 12), El=st.integers(1, 24),
       skew=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_layout_random_properties(T, k, R, El, skew, seed):
    E = R * El
    rng = np.random.default_rng(seed)
    if skew:
        p = 1.0 / (1.0 + np.arange(E)) ** 1.5
        idx = rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k), dtype=np.int32)
    L = oracle.layout(idx, E, R)
    flat = idx.ravel()
    assert np.array_equal(L.expert_counts, np.bincount(flat, minlength=E))
    assert np.array_equal(L.src_of, np.argsort(flat, kind="stable"))
    check_invariants(idx, E, R, L)


def test_layout_pages_arithmetic():
    g = json.load(open(GOLDEN))
    c = g["tokens_per_expert_ep128"]
    T = c["batch_per_gpu"] * c["query_len"] * c["dp_groups"]
    k, E = c["top_k"], c["num_experts"]
    rng = np.random.default_rng(0)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    L = oracle.layout(idx, E, 1)
    assert L.expert_counts.mean() == c["mean_rows_per_expert"]
    c = g["activated_experts_per_gpu_batch1"]
    idx = np.stack([rng.permutation(256)[:c["top_k"]] for _ in range(c["tokens"])]).astype(np.int32)
    L = oracle.layout(idx, 256, c["num_ranks"])
    assert L.rank_counts.mean() == c["mean_rows_per_rank"]
    for E, R, El in g["experts_per_rank"]["cases"]:
        idx = np.arange(E, dtype=np.int32).reshape(1, E)
        L = oracle.layout(idx, E, R)
        assert np.all(L.rank_counts == El)


def test_layout_rejects_bad_input():
    idx = np.array([[0, 5]], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.layout(idx, 4, 2)          # index outside [0, E)
    with pytest.raises(oracle.OracleError):
        oracle.layout(np.array([[-1]], np.int32), 4, 2)
    with pytest.raises(oracle.OracleError):
        oracle.layout(np.array([[0]], np.int32), 6, 4)  # E % R != 0
    assert oracle.validate(1, 130, 1, 4, 2, True, np.zeros((1, 1), np.int32)) == 1  # H % 128 under FP8
    assert oracle.validate(1, 12, 1, 4, 2, False, np.zeros((1, 1), np.int32)) == 1  # H % 8
    assert oracle.validate(1, 256, 1, 4, 2, True, np.zeros((1, 1), np.int32)) == 0


def test_layout_single_hot_expert():
    T, k, E, R = 1000, 4, 32, 4
    idx = np.full((T, k), 7, np.int32)
    L = oracle.layout(idx, E, R)
    assert L.expert_counts[7] == T * k and L.rank_counts[0] == T * k
    assert np.array_equal(L.slot_of, np.arange(T * k))
    check_invariants(idx, E, R, L)
