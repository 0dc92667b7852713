"""Pins of the oracle's router (oracle.route) to things other than itself.

Pages: [Perplexity blog] "Lower latency and higher throughput with multi-node
DeepSeek deployment", "MoE-beirari" (one router for every MoE model: DeepSeek
group-limited top-k, with Mixtral routing the case where the top-k group is
all experts; indices and scores come out per token); [EPLB page] "DeepSeek
V3/R1 ... DualPipe, EPLB, Profile-Data" (group-limited expert routing,
redundant experts); [torchtitan PR] "Integrate DeepEP to experimental
torchtitan" (node-limited routing).

The pins: the workload generator's independent numpy routing (stable argsort
on float32 scores) on all five workloads; scipy's softmax / expit for the
gate scores; numpy stable argsort for plain top-k, including exact ties; the
closed form of Mixtral's weights (a softmax over the k chosen logits); the
group-limited invariants checked with numpy sorts; the reductions G = 1,
TG = G and one expert per group; and the replica rule.
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from workloads import CONFIGS, make_workload


def f32_ulps(a, b):
    """|a - b| in units of the float32 spacing at b (both float32 arrays)."""
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32)
    sp = np.spacing(np.abs(b)).astype(np.float64)
    return np.abs(a - b.astype(np.float64)) / np.maximum(sp, np.finfo(np.float32).smallest_subnormal)


def gate_scores(z, gate):
    """Gate scores from scipy in binary64, rounded once to float32."""
    z64 = z.astype(np.float64)
    return (softmax(z64, axis=1) if gate == "softmax" else expit(z64)).astype(np.float32)


def topk_by_order(s, k, eligible=None):
    """k best by (score desc, id asc): numpy's stable argsort of -score."""
    key = s.astype(np.float64)
    if eligible is not None:
        key = np.where(eligible, key, -np.inf)
    return np.argsort(-key, axis=1, kind="stable")[:, :k]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_matches_generator_routing(name):
    # the generator routes with its own float32 numpy code; same draws in
    w = make_workload(name)
    x = w.extra
    idx, wt = oracle.route(x["logits"], w.k, bias=x.get("bias"), rep_offsets=x.get("rep_offsets"),
                           rep_slots=x.get("rep_slots"), **x["router"])
    assert np.array_equal(idx, w.topk_idx)
    rel = np.abs(wt.astype(np.float64) - w.topk_w) / np.abs(w.topk_w.astype(np.float64))
    assert rel.max() <= 1e-6


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_plain_topk_is_argsort_and_scores_are_scipy(gate):
    rng = np.random.default_rng(3)
    z = rng.standard_normal((300, 48)).astype(np.float32) * 2
    idx, wt = oracle.route(z, 5, gate=gate, renorm=False)
    s = gate_scores(z, gate)
    assert np.array_equal(idx, topk_by_order(s, 5))
    assert np.array_equal(idx, topk_by_order(z, 5))   # a monotone gate keeps the logit order
    ref = np.take_along_axis(s, idx, axis=1)
    assert f32_ulps(wt, ref).max() <= 1.0


def test_ties_go_to_the_lower_id():
    rng = np.random.default_rng(4)
    z = (np.round(rng.standard_normal((400, 32)) * 2) / 2).astype(np.float32)  # many equal logits
    for gate in ("softmax", "sigmoid"):
        idx, _ = oracle.route(z, 7, gate=gate, renorm=False)
        assert np.array_equal(idx, topk_by_order(gate_scores(z, gate), 7))


def test_mixtral_weights_closed_form():
    # softmax over all experts, renormalized over the chosen k, equals a
    # softmax over the k chosen logits alone
    rng = np.random.default_rng(5)
    z = rng.standard_normal((256, 8)).astype(np.float32) * 3
    idx, wt = oracle.route(z, 2, gate="softmax", renorm=True)
    zs = np.take_along_axis(z, idx, axis=1).astype(np.float64)
    ref = softmax(zs, axis=1)
    assert np.max(np.abs(wt - ref) / ref) <= 4e-7
    assert np.max(np.abs(wt.sum(axis=1, dtype=np.float64) - 1)) <= 1e-6


def test_renorm_of_sigmoid_scores():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((200, 64)).astype(np.float32)
    i0, w0 = oracle.route(z, 6, gate="sigmoid", renorm=False)
    i1, w1 = oracle.route(z, 6, gate="sigmoid", renorm=True)
    assert np.array_equal(i0, i1)
    ref = w0.astype(np.float64) / w0.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.max(np.abs(w1 - ref) / ref) <= 1e-6


def group_limited_reference(s, k, G, TG, topn):
    """Group-limited selection from numpy sorts: group score = best, or the
    float32 sum of the two best, per group; TG best groups by stable argsort;
    then stable top-k over their experts."""
    T, El = s.shape
    gs = El // G
    srt = np.sort(s.reshape(T, G, gs), axis=2)
    n = min(topn, gs)
    g = srt[:, :, -1] if n == 1 else (srt[:, :, -1] + srt[:, :, -2]).astype(np.float32)
    keep = np.argsort(-g.astype(np.float64), axis=1, kind="stable")[:, :TG]
    mask = np.zeros((T, G), bool)
    np.put_along_axis(mask, keep, True, axis=1)
    return topk_by_order(s, k, eligible=np.repeat(mask, gs, axis=1)), mask


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
@pytest.mark.parametrize("G,TG,topn,k", [(8, 3, 2, 6), (8, 4, 1, 8), (4, 1, 2, 5), (16, 2, 2, 4)])
def test_group_limited(gate, G, TG, topn, k):
    rng = np.random.default_rng(7 + G + TG)
    El = 64
    z = rng.standard_normal((500, El)).astype(np.float32)
    idx, _ = oracle.route(z, k, gate=gate, n_groups=G, topk_groups=TG, group_topn=topn,
                          renorm=False)
    s = gate_scores(z, gate)
    ref, mask = group_limited_reference(s, k, G, TG, topn)
    assert np.array_equal(idx, ref)
    # invariant: every chosen expert lies in a kept group, so at most TG
    # groups (nodes, for node-limited routing) are touched per token
    gs = El // G
    assert np.all(np.take_along_axis(mask, idx // gs, axis=1))
    assert np.all([len(set(r)) <= TG for r in (idx // gs)])


def test_group_reductions():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((300, 32)).astype(np.float32)
    plain, wp = oracle.route(z, 4, gate="sigmoid")
    all_groups, wa = oracle.route(z, 4, gate="sigmoid", n_groups=8, topk_groups=8)
    singles, ws = oracle.route(z, 4, gate="sigmoid", n_groups=32, topk_groups=6, group_topn=1)
    assert np.array_equal(plain, all_groups) and np.array_equal(wp, wa)
    assert np.array_equal(plain, singles) and np.array_equal(wp, ws)


def test_bias_is_added_to_the_logits():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((200, 64)).astype(np.float32)
    b = (-1.1 * np.log1p(rng.permutation(64))).astype(np.float32)
    a = oracle.route(z, 8, gate="sigmoid", n_groups=8, topk_groups=4, bias=b)
    r = oracle.route((z + b).astype(np.float32), 8, gate="sigmoid", n_groups=8, topk_groups=4)
    assert np.array_equal(a[0], r[0]) and np.array_equal(a[1], r[1])


def test_replicas_round_robin_by_token():
    rng = np.random.default_rng(10)
    El, T, k = 16, 64, 4
    n = rng.integers(0, 4, El)
    n[:12] = np.maximum(n[:12], 1)     # experts 12..15 may have no replica
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    slots = rng.permutation(int(off[-1])).astype(np.int32)
    z = rng.standard_normal((T, El)).astype(np.float32)
    logical, w0 = oracle.route(z, k, gate="softmax")
    phys, w1 = oracle.route(z, k, gate="softmax", rep_offsets=off, rep_slots=slots)
    assert np.array_equal(w0, w1)
    for t in range(T):
        for j in range(k):
            l = logical[t, j]
            want = slots[off[l] + t % n[l]] if n[l] > 0 else -1
            assert phys[t, j] == want


def test_zero_score_sum_keeps_zero_weights():
    z = np.full((4, 16), -200.0, np.float32)   # sigmoid underflows to +0 in float32
    idx, w = oracle.route(z, 3, gate="sigmoid", renorm=True)
    assert np.array_equal(idx, np.tile(np.arange(3), (4, 1)))
    assert np.all(w == 0) and not np.any(np.signbit(w))


@pytest.mark.parametrize("kw", [dict(k=0), dict(k=17), dict(n_groups=3), dict(n_groups=4, topk_groups=0),
                                dict(n_groups=4, topk_groups=5), dict(k=9, n_groups=4, topk_groups=2),
                                dict(group_topn=3)])
def test_router_rejects_bad_parameters(kw):
    args = dict(k=2, gate="softmax", n_groups=1, topk_groups=1)
    args.update(kw)
    with pytest.raises(oracle.OracleError):
        oracle.route(np.zeros((2, 16), np.float32), **args)


@pytest.mark.parametrize("seed", range(6))
def test_router_properties_on_random_shapes(seed):
    """Invariants on random shapes, including non-finite logits (for which the
    choice is unspecified): k distinct ids in [0, El) per token, all inside
    the TG kept groups; finite logits with renormalization give weights that
    sum to 1."""
    rng = np.random.default_rng(100 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    gs = int(rng.integers(1, 9))
    El = G * gs
    TG = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(TG * gs, 16) + 1))
    T = int(rng.integers(1, 200))
    gate = ["softmax", "sigmoid"][seed % 2]
    z = (rng.standard_normal((T, El)) * 4).astype(np.float32)
    idx, w = oracle.route(z, k, gate=gate, n_groups=G, topk_groups=TG, renorm=True)
    assert np.all((idx >= 0) & (idx < El))
    assert all(len(set(r)) == k for r in idx)
    assert all(len(set(r // gs)) <= TG for r in idx)
    assert np.allclose(w.sum(axis=1, dtype=np.float64), 1.0, atol=1e-5)
    zb = z.copy()
    zb[rng.random(z.shape) < 0.2] = np.nan
    zb[rng.random(z.shape) < 0.1] = np.inf
    zb[rng.random(z.shape) < 0.1] = -np.inf
    idx, _ = oracle.route(zb, k, gate=gate, n_groups=G, topk_groups=TG, renorm=True)
    assert np.all((idx >= 0) & (idx < El))
    assert all(len(set(r)) == k for r in idx)
