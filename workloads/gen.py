"""Seeded generators for the five workloads of the MoE dispatch / combine path.

Pages cited (title, section):
  [DeepEP overview]  "DeepSeek merilis library open source DeepEP untuk
                     pelatihan dan inferensi MoE", "Hasil pengukuran performa"
                     (the "V3 config": 8K tokens per batch, hidden 7168, top-8
                     experts, FP8 dispatch, BF16 combine)
  [Perplexity blog]  "Lower latency and higher throughput with multi-node
                     DeepSeek deployment", "Sérfræðinga-samsíðun" (256 routed
                     experts, 8 per token, weighted sum) and "MoE-beirari"
                     (top-k routing; Mixtral-style softmax routing is a special
                     case of DeepSeek's)
  [EPLB page]        "DeepSeek V3/R1 ... DualPipe, EPLB, Profile-Data"
                     (GeekNews, Turkish): redundant experts (replicate heavily
                     loaded experts) and group-limited expert routing
  [torchtitan PR]    "Integrate DeepEP to experimental torchtitan" (DeepSeek
                     16B model, node-limited routing)

Recipe (every array comes from numpy.random.default_rng(seed), drawn in this
order: token activations, router logits, then the workload's extras; the expert
outputs used by combine come from default_rng(seed + 1)):
  * x ~ N(0,1) in float32, rounded to bf16 (nearest, ties to even);
  * logits ~ N(0,1) float32, one per (token, logical expert);
  * gate: softmax (max-subtracted) or sigmoid, in float32;
  * top-k by a stable descending sort, so ties go to the lower expert id;
  * weights: the chosen gate scores, renormalized to sum 1 where the workload
    says so.
For the dispatch / combine rows the gates and routing are inputs: both the
HIP path and the oracle consume the same arrays.  The router's own inputs
(unbiased logits, the Zipf bias, the group parameters and the replica table
as CSR offsets / slot lists) are kept in Workload.extra for the on-device
router, which recomputes the routing from them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED = 0

# name -> workload parameters.  E is the number of physical experts (what the
# routing indices address); E_logical is what the router scores.
CONFIGS = {
    # Tiny: T=128, H=256, 16 experts, top-2 softmax renormalized, 4 ranks, BF16.
    "tiny": dict(T=128, H=256, k=2, E=16, E_logical=16, R=4, fp8=False,
                 gate="softmax", renorm=True),
    # DeepSeek-16B-like (the torchtitan PR's model size): 64 experts, top-6
    # softmax, not renormalized, 8 ranks, BF16 dispatch and combine.
    "ds16b": dict(T=4096, H=2048, k=6, E=64, E_logical=64, R=8, fp8=False,
                  gate="softmax", renorm=False),
    # V3-shaped headline (the DeepEP overview's V3 config): 256 experts, top-8
    # sigmoid renormalized, 8 ranks x 32 experts, FP8 dispatch, BF16 combine.
    "v3": dict(T=8192, H=7168, k=8, E=256, E_logical=256, R=8, fp8=True,
               gate="sigmoid", renorm=True),
    # Group-limited and skewed: 8 groups of 32, top-4 groups by the sum of each
    # group's two best scores, top-8 inside them, Zipf(1.1) logit bias.
    "v3_skew": dict(T=8192, H=7168, k=8, E=256, E_logical=256, R=8, fp8=True,
                    gate="sigmoid", renorm=True, n_groups=8, topk_groups=4,
                    zipf_s=1.1),
    # Decode with redundant experts: 256 logical experts plus 32 replicas =
    # 288 physical slots over 36 ranks (8 each), replica chosen by token id.
    "decode": dict(T=128, H=7168, k=8, E=288, E_logical=256, R=36, fp8=True,
                   gate="sigmoid", renorm=True, n_extra=32),
}


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), nearest with ties to even
    (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass
class Workload:
    name: str
    T: int
    H: int
    k: int
    E: int
    R: int
    fp8: bool
    x: np.ndarray            # [T, H] uint16 (bf16 bits)
    topk_idx: np.ndarray     # [T, k] int32, physical expert ids
    topk_w: np.ndarray       # [T, k] float32
    seed: int = SEED
    extra: dict = field(default_factory=dict)

    @property
    def P(self) -> int:
        return self.T * self.k


def _topk_stable(score: np.ndarray, k: int) -> np.ndarray:
    # descending by score, ties to the lower index
    return np.argsort(-score, axis=1, kind="stable")[:, :k].astype(np.int32)


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-z, dtype=np.float32))).astype(np.float32)


def make_workload(name: str, seed: int = SEED, T: int | None = None) -> Workload:
    """Build one of CONFIGS (optionally with a different token count T, used
    for small parity cases of the same shape family)."""
    c = dict(CONFIGS[name])
    if T is not None:
        c["T"] = T
    T_, H, k, E, El, R = c["T"], c["H"], c["k"], c["E"], c["E_logical"], c["R"]
    rng = np.random.default_rng(seed)
    x = bf16_from_f32(rng.standard_normal((T_, H), dtype=np.float32))
    logits = rng.standard_normal((T_, El), dtype=np.float32)
    # the router's inputs, kept for the on-device router (which recomputes the
    # routing from them); the arrays below are derived from the same draws
    extra = {"logits": logits, "router": dict(
        gate=c["gate"], n_groups=c.get("n_groups", 1), topk_groups=c.get("topk_groups", 1),
        group_topn=2, renorm=bool(c["renorm"]))}

    if "zipf_s" in c:
        # popularity rank pi(e) from a seeded permutation; bias -s*ln(1+pi(e))
        pi = rng.permutation(El)
        bias = (-c["zipf_s"] * np.log1p(pi.astype(np.float64))).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
        extra.update(zipf_rank=pi, bias=bias)

    score = _softmax(logits) if c["gate"] == "softmax" else _sigmoid(logits)

    if "n_groups" in c:
        G = c["n_groups"]
        gs = El // G
        grouped = score.reshape(T_, G, gs)
        top2 = np.sort(grouped, axis=2)[:, :, -2:].sum(axis=2, dtype=np.float32)
        keep = np.argsort(-top2, axis=1, kind="stable")[:, :c["topk_groups"]]
        mask = np.zeros((T_, G), bool)
        np.put_along_axis(mask, keep, True, axis=1)
        sel_score = np.where(np.repeat(mask, gs, axis=1), score, -np.inf).astype(np.float32)
        logical = _topk_stable(sel_score, k)
        extra["groups"] = keep
    else:
        logical = _topk_stable(score, k)

    w = np.take_along_axis(score, logical, axis=1).astype(np.float32)
    if c["renorm"]:
        w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)

    if "n_extra" in c:
        # redundant experts: 32 distinct logical experts get one more replica;
        # the 288 physical slots are shuffled; slot s lives on rank s // 8.
        extra_ids = np.sort(rng.choice(El, size=c["n_extra"], replace=False))
        phys2log = np.concatenate([np.arange(El), extra_ids])
        perm = rng.permutation(E)
        slot_log = phys2log[perm]            # logical expert held by slot s
        replicas = [np.sort(np.nonzero(slot_log == e)[0]) for e in range(El)]
        n_rep = np.array([len(r) for r in replicas])
        tok = np.arange(T_)[:, None]
        choice = tok % n_rep[logical]
        phys = np.empty_like(logical)
        for t in range(T_):
            for j in range(k):
                phys[t, j] = replicas[logical[t, j]][choice[t, j]]
        topk_idx = phys.astype(np.int32)
        rep_offsets = np.concatenate([[0], np.cumsum(n_rep)]).astype(np.int32)
        rep_slots = np.concatenate(replicas).astype(np.int32)
        extra.update(slot_logical=slot_log, n_replicas=n_rep, rep_offsets=rep_offsets,
                     rep_slots=rep_slots)
    else:
        topk_idx = logical

    return Workload(name, T_, H, k, E, R, bool(c["fp8"]), x, np.ascontiguousarray(topk_idx),
                    np.ascontiguousarray(w), seed, extra)


def make_expert_rows(P: int, H: int, seed: int = SEED + 1, chunk_rows: int = 4096) -> np.ndarray:
    """Expert outputs y ~ N(0,1) rounded to bf16, one row per received slot
    ([P, H] uint16 in global slot order), drawn in fixed chunks of rows."""
    rng = np.random.default_rng(seed)
    y = np.empty((P, H), np.uint16)
    for s in range(0, P, chunk_rows):
        n = min(chunk_rows, P - s)
        y[s:s + n] = bf16_from_f32(rng.standard_normal((n, H), dtype=np.float32))
    return y


def edge_case_x(T: int, H: int, seed: int = SEED) -> np.ndarray:
    """bf16 activations that hit the quantizer's corner cases, one pattern per
    128-channel block, cycling: all-zero blocks (+0 and -0 mixed), blocks with
    bf16 subnormals only, +-max finite bf16, a single nonzero value, values
    that land on E4M3 rounding midpoints, huge dynamic range, and plain
    N(0,1) blocks."""
    rng = np.random.default_rng(seed)
    x = bf16_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    nb = H // 128
    for t in range(T):
        for b in range(nb):
            kind = (t * nb + b) % 8
            blk = x[t, b * 128:(b + 1) * 128]
            if kind == 0:      # all zero, signs mixed
                blk[:] = np.where(rng.random(128) < 0.5, 0x0000, 0x8000)
            elif kind == 1:    # bf16 subnormals only (exponent field 0)
                mant = rng.integers(0, 128, 128).astype(np.uint16)
                sign = np.where(rng.random(128) < 0.5, 0, 0x8000).astype(np.uint16)
                blk[:] = sign | mant
            elif kind == 2:    # +-max finite bf16 mixed with ordinary values
                blk[::7] = 0x7F7F
                blk[3::11] = 0xFF7F
            elif kind == 3:    # one nonzero value, the rest +-0
                blk[:] = 0x8000
                blk[rng.integers(0, 128)] = x[t, b * 128]
            elif kind == 4:    # amax 448 exactly; others at E4M3 midpoints
                mids = np.array([0.5 + 1 / 32, 1.0 + 1 / 16, 3.0 + 1 / 8, 17.0, 2.0 ** -7 * 3,
                                 416.0 + 16.0, 2.0 ** -10, 2.0 ** -10 * 3], np.float32)
                vals = mids[rng.integers(0, len(mids), 128)] * np.where(rng.random(128) < 0.5, 1, -1)
                vals[0] = 448.0
                blk[:] = bf16_from_f32(vals.astype(np.float32))
            elif kind == 5:    # dynamic range: 2^-100 .. 2^100
                e = rng.integers(-100, 100, 128)
                blk[:] = bf16_from_f32((rng.standard_normal(128) * 2.0 ** e).astype(np.float32))
            # kinds 6, 7: plain N(0,1)
    return x
