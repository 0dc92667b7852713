"""Validity rule for a router result that is not bit-identical to the oracle's.

The router's gate is evaluated in binary64 and rounded once to binary32 on
both sides, with the softmax denominator summed in the same ascending expert
order; what still differs between host and device is the binary64 exp, whose
last bit may disagree.  That moves a binary32 score by at most one ulp (and
only when the binary64 value sits within that bit of a rounding boundary).  So
a device result is correct iff it is the exact result for SOME scores s' with
every s'_e within `tol` ulps of the oracle's s_e ([Perplexity blog] "Lower
latency and higher throughput with multi-node DeepSeek deployment",
"MoE-beirari": k best experts of the kept groups, best first; ties to the
lower id).  The rule below checks the consequences of that:

  * picks: k distinct logical experts, mapped to physical slots by the replica
    rule (token t takes replica t mod n_l);
  * groups: each pick's group could be among the TG best groups (its group
    score within the group tolerance of the TG-th best), and the picks touch
    at most TG groups;
  * order: each pick's score is at least the next pick's minus 2*tol ulps;
  * completeness: every expert of a group that is kept under any such
    perturbation and not picked scores at most the last pick + 2*tol ulps;
  * weights: within `wtol` ulps of the oracle's weight formula applied to the
    device's picks (raw scores: tol; renormalized: s_j / sum over j, where
    s_j and the sum each move by <= tol ulps, so 2*tol + 1 with the division's
    own rounding).

Scores are non-negative binary32, so their bit patterns order like the values
and a bit-pattern difference counts ulps inside a binade.  Tokens whose result
is bit-identical to the oracle's pass without further checks.
"""
from __future__ import annotations

import numpy as np


def _bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)


def expected_weights(scores_row: np.ndarray, picks, renorm: bool) -> np.ndarray:
    """The weight formula on given picks: the chosen scores, divided by their
    binary32 sum in pick order when renormalizing and that sum is > 0."""
    ws = np.array([scores_row[e] for e in picks], np.float32)
    if renorm:
        tot = np.float32(0.0)
        for v in ws:
            tot = np.float32(tot + v)
        if tot > 0:
            ws = (ws / tot).astype(np.float32)
    return ws


def invalid_tokens(got_idx, got_w, ref_idx, ref_w, scores, *, k, n_groups=1, topk_groups=1,
                   group_topn=2, renorm=True, rep_offsets=None, rep_slots=None, tol=1,
                   **_ignored) -> list[tuple[int, str]]:
    """(token, reason) for every token whose result is not valid under the rule."""
    got_idx, ref_idx = np.asarray(got_idx), np.asarray(ref_idx)
    got_w, ref_w = np.asarray(got_w, np.float32), np.asarray(ref_w, np.float32)
    T, El = scores.shape
    G, TG = n_groups, topk_groups
    gs = El // G
    wtol = 2 * tol + 1 if renorm else tol
    gtol = 2 * tol + 1 if (group_topn == 2 and gs > 1) else tol
    phys2log = None
    if rep_offsets is not None:
        phys2log = {}
        for l in range(El):
            for q in range(int(rep_offsets[l]), int(rep_offsets[l + 1])):
                phys2log[int(rep_slots[q])] = l
    same = (np.all(got_idx == ref_idx, axis=1)
            & np.all(got_w.view(np.uint32) == ref_w.view(np.uint32), axis=1))
    bad = []
    for t in np.nonzero(~same)[0]:
        t = int(t)
        s = scores[t]
        sb = _bits(s)
        # picks back to logical ids, through the replica rule
        picks = []
        why = None
        for j in range(k):
            p = int(got_idx[t, j])
            if phys2log is None:
                l = p
            else:
                l = phys2log.get(p, -1)
                if l >= 0:
                    n = int(rep_offsets[l + 1] - rep_offsets[l])
                    if p != int(rep_slots[int(rep_offsets[l]) + t % n]):
                        why = f"pick {j}: slot {p} is not token {t}'s replica of expert {l}"
            if not (0 <= l < El):
                why = why or f"pick {j}: index {p} names no expert"
            picks.append(l)
        if why is None and len(set(picks)) != k:
            why = f"repeated expert in {picks}"
        if why is None:
            # groups that may be / must be among the TG best under the tolerance
            if G > 1:
                g = np.empty(G, np.float32)
                for c in range(G):
                    v = np.sort(s[c * gs:(c + 1) * gs])[::-1]
                    g[c] = v[0] if (group_topn == 1 or gs == 1) else np.float32(v[0] + v[1])
                gb = _bits(g)
                order = np.sort(gb)[::-1]
                may = gb + 2 * gtol >= order[TG - 1]
                must = gb - 2 * gtol > (order[TG] if TG < G else -1)
                used = {e // gs for e in picks}
                if not all(may[c] for c in used):
                    why = f"a pick's group {sorted(c for c in used if not may[c])} cannot be kept"
                elif len(used) > TG:
                    why = f"picks touch {len(used)} groups > {TG}"
                eligible = np.zeros(El, bool)
                for c in range(G):
                    if must[c]:
                        eligible[c * gs:(c + 1) * gs] = True
            else:
                eligible = np.ones(El, bool)
        if why is None:
            pb = sb[picks]
            for j in range(k - 1):
                if pb[j + 1] > pb[j] + 2 * tol:
                    why = f"picks {j},{j + 1} out of order ({s[picks[j]]!r} < {s[picks[j + 1]]!r})"
                    break
        if why is None:
            rest = eligible.copy()
            rest[picks] = False
            if rest.any() and sb[rest].max() > pb.min() + 2 * tol:
                e = int(np.nonzero(rest)[0][np.argmax(sb[rest])])
                why = f"expert {e} ({s[e]!r}) beats a pick ({s[picks[int(np.argmin(pb))]]!r})"
        if why is None:
            want = expected_weights(s, picks, renorm)
            d = np.abs(_bits(got_w[t]) - _bits(want))
            if d.max() > wtol:
                why = f"weights {got_w[t]} vs {want} ({int(d.max())} ulps > {wtol})"
        if why is not None:
            bad.append((t, why))
    return bad
