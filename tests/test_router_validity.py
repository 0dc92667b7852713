"""CPU checks of the router validity rule (tests/router_validity.py) that the
GPU router tests apply where a result is not bit-identical to the oracle's.
Near-tie logits are built on purpose: two experts whose binary32 scores are
one ulp apart may come out in either order on a device whose binary64 exp
differs from the host's in the last bit, and the rule must accept that, yet
reject any choice that no such one-ulp difference explains."""
import numpy as np
import pytest

import oracle
from router_validity import expected_weights, invalid_tokens


def near_tie_logit(z_ref, gate_score_bits_target, gate="sigmoid"):
    """A logit below z_ref whose sigmoid score has exactly the target bits."""
    z = np.float32(z_ref)
    for _ in range(200):
        z = np.nextafter(z, np.float32(-np.inf), dtype=np.float32)
        b = int(oracle.route_scores(np.array([[z]], np.float32), gate)[0, 0].view(np.int32))
        if b == gate_score_bits_target:
            return z
        if b < gate_score_bits_target:
            return None
    return None


def build_near_ties(T=64, El=32, k=4, seed=3):
    """Sigmoid logits where, in every token, the best expert outside the top-k
    scores exactly one ulp below the k-th pick."""
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((T, El)) * 0.5 + 1.0).astype(np.float32)
    made = []
    for t in range(T):
        s = oracle.route_scores(z[t:t + 1], "sigmoid")[0]
        order = np.argsort(-s, kind="stable")
        kth, nxt = int(order[k - 1]), int(order[k])
        target = int(s[kth].view(np.int32)) - 1
        zz = near_tie_logit(z[t, kth], target)
        if zz is not None:
            z[t, nxt] = zz
            made.append((t, kth, nxt))
    return z, made


@pytest.mark.parametrize("renorm", [False, True])
def test_identical_results_pass(renorm):
    z, _ = build_near_ties()
    idx, w = oracle.route(z, 4, "sigmoid", renorm=renorm)
    s = oracle.route_scores(z, "sigmoid")
    assert invalid_tokens(idx, w, idx, w, s, k=4, renorm=renorm) == []


@pytest.mark.parametrize("renorm", [False, True])
def test_one_ulp_tie_may_go_either_way(renorm):
    z, made = build_near_ties()
    assert len(made) >= 40
    idx, w = oracle.route(z, 4, "sigmoid", renorm=renorm)
    s = oracle.route_scores(z, "sigmoid")
    got_i, got_w = idx.copy(), w.copy()
    for t, kth, nxt in made:
        assert s[t, kth].view(np.int32) - s[t, nxt].view(np.int32) == 1   # the planted near tie
        picks = [e if e != kth else nxt for e in idx[t]]
        got_i[t] = picks
        got_w[t] = expected_weights(s[t], picks, renorm)
    assert invalid_tokens(got_i, got_w, idx, w, s, k=4, renorm=renorm) == []


def test_a_clear_loser_is_rejected():
    z, made = build_near_ties()
    idx, w = oracle.route(z, 4, "sigmoid", renorm=False)
    s = oracle.route_scores(z, "sigmoid")
    t, kth, _ = made[0]
    order = np.argsort(-s[t], kind="stable")
    far = int(order[-1])                                   # the worst expert of the token
    assert s[t, kth].view(np.int32) - s[t, far].view(np.int32) > 2
    got_i, got_w = idx.copy(), w.copy()
    picks = [e if e != kth else far for e in idx[t]]
    got_i[t] = picks
    got_w[t] = expected_weights(s[t], picks, False)
    bad = invalid_tokens(got_i, got_w, idx, w, s, k=4, renorm=False)
    assert [b[0] for b in bad] == [t] and "beats a pick" in bad[0][1]


def test_order_and_duplicates_and_range():
    z, _ = build_near_ties()
    idx, w = oracle.route(z, 4, "sigmoid", renorm=False)
    s = oracle.route_scores(z, "sigmoid")
    t = next(t for t in range(len(z)) if s[t, idx[t, 0]].view(np.int32) - s[t, idx[t, 1]].view(np.int32) > 2)
    for mutate, why in ((lambda r: r[[1, 0, 2, 3]], "out of order"),
                        (lambda r: np.array([r[0], r[0], r[2], r[3]]), "repeated"),
                        (lambda r: np.array([r[0], r[1], r[2], 99]), "names no expert")):
        got_i = idx.copy()
        got_i[t] = mutate(idx[t])
        got_w = w.copy()
        if why != "names no expert":
            got_w[t] = expected_weights(s[t], list(got_i[t]), False)
        bad = invalid_tokens(got_i, got_w, idx, w, s, k=4, renorm=False)
        assert [b[0] for b in bad] == [t] and why in bad[0][1], (why, bad)


@pytest.mark.parametrize("renorm,ok,too_far", [(False, 1, 2), (True, 3, 4)])
def test_weight_tolerance(renorm, ok, too_far):
    z, _ = build_near_ties()
    idx, w = oracle.route(z, 4, "sigmoid", renorm=renorm)
    s = oracle.route_scores(z, "sigmoid")
    for d, valid in ((ok, True), (too_far, False)):
        got_w = w.copy()
        got_w[5, 2] = (w[5, 2:3].view(np.int32) + d).view(np.float32)[0]
        bad = invalid_tokens(idx, got_w, idx, w, s, k=4, renorm=renorm)
        assert (bad == []) == valid, (d, bad)


def test_groups_and_replicas():
    rng = np.random.default_rng(9)
    T, El, G, TG, k = 48, 64, 8, 3, 6
    z = rng.standard_normal((T, El)).astype(np.float32)
    n = np.ones(El, np.int64)
    n[rng.choice(El, 8, replace=False)] += 1
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    slots = rng.permutation(int(off[-1])).astype(np.int32)
    kw = dict(n_groups=G, topk_groups=TG, group_topn=2, renorm=True, rep_offsets=off, rep_slots=slots)
    idx, w = oracle.route(z, k, "sigmoid", **kw)
    s = oracle.route_scores(z, "sigmoid")
    assert invalid_tokens(idx, w, idx, w, s, k=k, **kw) == []
    # a pick from a group far below the TG-th best group
    gsc = np.array([[np.sort(s[t, c * 8:(c + 1) * 8])[-2:].sum() for c in range(G)] for t in range(T)])
    t = next(t for t in range(T) if np.sort(gsc[t])[-TG] - np.sort(gsc[t])[0] > 0.2)
    worst_g = int(np.argmin(gsc[t]))
    e = worst_g * 8 + int(np.argmax(s[t, worst_g * 8:(worst_g + 1) * 8]))
    phys2log = {int(slots[q]): l for l in range(El) for q in range(off[l], off[l + 1])}
    logical = [phys2log[int(p)] for p in idx[t]]
    logical[-1] = e
    got_i, got_w = idx.copy(), w.copy()
    got_i[t] = [slots[off[l] + t % (off[l + 1] - off[l])] for l in logical]
    got_w[t] = expected_weights(s[t], logical, True)
    bad = invalid_tokens(got_i, got_w, idx, w, s, k=k, **kw)
    assert [b[0] for b in bad] == [t] and "cannot be kept" in bad[0][1], bad
    # the right expert through the wrong replica
    t2 = next(t for t in range(T) if any(off[phys2log[int(p)] + 1] - off[phys2log[int(p)]] == 2
                                         for p in idx[t]))
    j = next(j for j, p in enumerate(idx[t2]) if off[phys2log[int(p)] + 1] - off[phys2log[int(p)]] == 2)
    l = phys2log[int(idx[t2, j])]
    got_i = idx.copy()
    got_i[t2, j] = slots[off[l] + (t2 + 1) % 2]
    bad = invalid_tokens(got_i, w, idx, w, s, k=k, **kw)
    assert [b[0] for b in bad] == [t2] and "replica" in bad[0][1], bad
