"""GPU parity of ep_route / ep_route_layout (the on-device router feeding the
layout) against the oracle's router, through the C ABI.

Both sides round the binary64 gate once to binary32, sum the softmax
denominator in ascending expert order and take every decision (groups, top-k,
ties) on those binary32 values, so indices and weights are expected to match
bit for bit.  A device exp and a host exp may still differ in the last
binary64 bit, which moves a binary32 score by at most one ulp; a token whose
result is not bit-identical is therefore checked with the validity rule of
tests/router_validity.py (the exact result for scores within one ulp of the
oracle's), and the number of such tokens is printed.
"""
import numpy as np
import pytest
import torch

import combine_ep_layout_03_amd as ep
import oracle
from workloads import CONFIGS, make_workload

from gpu_util import POISON, GpuRun, say, to_dev
from router_validity import invalid_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load()


def run_route(T, k, E, logits, gate="sigmoid", n_groups=1, topk_groups=1, group_topn=2,
              renorm=True, bias=None, rep_offsets=None, rep_slots=None, num_workgroups=0):
    El = logits.shape[1]
    cfg = ep.Config(T, 128, k, E, 1, num_workgroups=num_workgroups)
    rt = ep.Router(El, gate, n_groups, topk_groups, group_topn, renorm)
    d = dict(logits=to_dev(logits), bias=None if bias is None else to_dev(bias),
             ro=None if rep_offsets is None else to_dev(rep_offsets),
             rs=None if rep_slots is None else to_dev(rep_slots))
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    ep.ep_route(cfg, rt, d["logits"], d["bias"], d["ro"], d["rs"], idx, w)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


def check_routing(gi, gw, logits, k, **kw):
    """The device's routing against the oracle's: bit-identical tokens pass,
    any other token must satisfy the validity rule."""
    okw = {a: b for a, b in kw.items() if a != "num_workgroups"}
    ri, rw = oracle.route(logits, k, **okw)
    differ = np.any(gi != ri, axis=1) | np.any(gw.view(np.uint32) != rw.view(np.uint32), axis=1)
    if differ.any():
        scores = oracle.route_scores(logits, okw.get("gate", "sigmoid"), okw.get("bias"))
        rule = {a: b for a, b in okw.items() if a not in ("gate", "bias")}
        bad = invalid_tokens(gi, gw, ri, rw, scores, k=k, **rule)
        say(f"  {int(differ.sum())} of {len(gi)} tokens not bit-identical; {len(bad)} invalid")
        assert not bad, f"{len(bad)} invalid tokens, first: {bad[:3]}"


def check(T, k, E, logits, **kw):
    say(f"route T={T} El={logits.shape[1]} k={k} E={E} "
        + " ".join(f"{a}={b}" for a, b in kw.items() if not isinstance(b, np.ndarray)))
    gi, gw = run_route(T, k, E, logits, **kw)
    check_routing(gi, gw, logits, k, **kw)
    return gi, gw


@pytest.mark.parametrize("name", list(CONFIGS))
def test_route_full_workloads(name):
    w = make_workload(name)
    x = w.extra
    gi, gw = check(w.T, w.k, w.E, x["logits"], bias=x.get("bias"), rep_offsets=x.get("rep_offsets"),
                   rep_slots=x.get("rep_slots"), **x["router"])
    assert np.array_equal(gi, w.topk_idx)   # the generator's own routing, too


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_plain_topk(gate, renorm):
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((333, 160)) * 1.5).astype(np.float32)   # El not a multiple of 64
    check(333, 6, 160, z, gate=gate, renorm=renorm)


@pytest.mark.parametrize("G,TG,topn,k", [(8, 4, 2, 8), (8, 3, 1, 6), (64, 5, 2, 8), (64, 8, 1, 8),
                                         (4, 1, 2, 7), (32, 32, 2, 8), (16, 2, 1, 3)])
def test_route_group_limited(G, TG, topn, k):
    rng = np.random.default_rng(12 + G)
    z = rng.standard_normal((517, 256)).astype(np.float32)
    for gate in ("sigmoid", "softmax"):
        check(517, k, 256, z, gate=gate, n_groups=G, topk_groups=TG, group_topn=topn)


def test_route_max_sizes():
    # El = E = 2048 (the build's maximum), k = 32 (its maximum), 64 groups
    rng = np.random.default_rng(13)
    z = rng.standard_normal((96, 2048)).astype(np.float32)
    check(96, 32, 2048, z, gate="softmax", renorm=True)
    check(96, 32, 2048, z, gate="sigmoid", n_groups=64, topk_groups=8, renorm=False)


def test_route_single_token_and_single_expert():
    rng = np.random.default_rng(14)
    check(1, 4, 64, rng.standard_normal((1, 64)).astype(np.float32), gate="softmax")
    check(5, 1, 1, rng.standard_normal((5, 1)).astype(np.float32), gate="sigmoid")
    check(7, 3, 3, rng.standard_normal((7, 3)).astype(np.float32), gate="softmax", renorm=False)


def test_route_ties_and_extremes():
    rng = np.random.default_rng(15)
    zt = (np.round(rng.standard_normal((400, 64)) * 2) / 2).astype(np.float32)   # exact ties
    check(400, 8, 64, zt, gate="sigmoid", n_groups=8, topk_groups=4)
    check(400, 8, 64, zt, gate="softmax", renorm=False)
    ze = (rng.standard_normal((300, 64)) * 60).astype(np.float32)    # saturated gates, many equal scores
    check(300, 8, 64, ze, gate="sigmoid", n_groups=4, topk_groups=2)
    check(300, 8, 64, ze, gate="softmax")
    zu = np.full((20, 32), -200.0, np.float32)                        # every score underflows to 0
    gi, gw = check(20, 4, 32, zu, gate="sigmoid", renorm=True)
    assert np.all(gw == 0)


def test_route_bias_and_replicas():
    rng = np.random.default_rng(16)
    El, E, T, k = 64, 80, 250, 6
    n = np.ones(El, np.int64)
    n[rng.choice(El, 16, replace=False)] += 1
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    slots = rng.permutation(E).astype(np.int32)
    z = rng.standard_normal((T, El)).astype(np.float32)
    b = (-1.1 * np.log1p(rng.permutation(El))).astype(np.float32)
    check(T, k, E, z, gate="sigmoid", n_groups=8, topk_groups=4, bias=b, rep_offsets=off,
          rep_slots=slots)


# Batches of at least 2048 tokens take the four-tokens-per-wave kernel when
# El <= 512, k <= 16 and the groups cover power-of-two runs of <= 16 lanes
# (16-lane rows, each lane holding the next power of two >= El/16 experts);
# other shapes fall back to the one-token kernel.  T = 2101 leaves a ragged
# last wave.
@pytest.mark.parametrize("El,k,gate,G,TG,topn,renorm", [
    (256, 8, "sigmoid", 1, 1, 2, True), (256, 8, "softmax", 1, 1, 2, False),
    (256, 8, "sigmoid", 8, 3, 1, True), (512, 16, "softmax", 4, 2, 2, True),
    (64, 6, "sigmoid", 16, 4, 2, True), (48, 5, "softmax", 3, 2, 2, True),
    (16, 3, "sigmoid", 1, 1, 2, False), (160, 8, "sigmoid", 8, 4, 2, True),  # 160: falls back
])
def test_route_large_batches(El, k, gate, G, TG, topn, renorm):
    rng = np.random.default_rng(El + k + G)
    T = 2101
    z = rng.standard_normal((T, El)).astype(np.float32)
    check(T, k, El, z, gate=gate, n_groups=G, topk_groups=TG, group_topn=topn, renorm=renorm)
    zt = (np.round(z * 2) / 2).astype(np.float32)     # exact ties
    check(T, k, El, zt, gate=gate, n_groups=G, topk_groups=TG, group_topn=topn, renorm=renorm)


def test_route_large_batch_bias_replicas_and_grid():
    rng = np.random.default_rng(21)
    El, E, T, k = 256, 288, 2500, 8
    n = np.ones(El, np.int64)
    n[rng.choice(El, 32, replace=False)] += 1
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    slots = rng.permutation(E).astype(np.int32)
    z = rng.standard_normal((T, El)).astype(np.float32)
    b = (-1.1 * np.log1p(rng.permutation(El))).astype(np.float32)
    for nwg in (0, 1, 7, 300):
        check(T, k, E, z, gate="sigmoid", n_groups=8, topk_groups=4, bias=b, rep_offsets=off,
              rep_slots=slots, num_workgroups=nwg)


@pytest.mark.parametrize("T,El,k,G,TG", [(300, 256, 8, 1, 1), (2200, 256, 8, 8, 4), (70, 64, 6, 4, 2)])
@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_route_non_finite_logits_give_valid_picks(T, El, k, G, TG, gate):
    """NaN / +-inf logits leave the choice unspecified, but every token still
    gets k distinct experts inside its kept groups, on both router kernels."""
    rng = np.random.default_rng(T + El)
    z = rng.standard_normal((T, El)).astype(np.float32)
    z[rng.random(z.shape) < 0.2] = np.nan
    z[rng.random(z.shape) < 0.1] = np.inf
    z[rng.random(z.shape) < 0.1] = -np.inf
    say(f"route non-finite T={T} El={El} G={G} {gate}")
    gi, _ = run_route(T, k, El, z, gate=gate, n_groups=G, topk_groups=TG)
    gs = El // G
    assert np.all((gi >= 0) & (gi < El))
    assert all(len(set(r)) == k for r in gi)
    assert all(len(set(r // gs)) <= TG for r in gi)


def test_route_grid_size_invariance():
    w = make_workload("v3_skew", T=1000)
    x = w.extra
    for nwg in (1, 7, 300):
        check(w.T, w.k, w.E, x["logits"], bias=x["bias"], num_workgroups=nwg, **x["router"])


@pytest.mark.parametrize("name", ["v3_skew", "decode", "ds16b"])
def test_route_layout_builds_the_handle(name):
    w = make_workload(name)
    x = w.extra
    r = x["router"]
    run = GpuRun(w)
    logits = to_dev(x["logits"])
    bias = None if "bias" not in x else to_dev(x["bias"])
    ro = None if "rep_offsets" not in x else to_dev(x["rep_offsets"])
    rs = None if "rep_slots" not in x else to_dev(x["rep_slots"])
    idx = torch.full((w.T, w.k), -7, dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    rt = ep.Router(x["logits"].shape[1], r["gate"], r["n_groups"], r["topk_groups"], r["group_topn"],
                   r["renorm"])
    say(f"route_layout {name}")
    ep.ep_route_layout(run.cfg, rt, logits, bias, ro, rs, idx, wts, run.h, run.ws)
    hnp = run.handle_np()
    gi = idx.cpu().numpy()
    check_routing(gi, wts.cpu().numpy(), x["logits"], w.k, bias=x.get("bias"),
                  rep_offsets=x.get("rep_offsets"), rep_slots=x.get("rep_slots"), **r)
    L = oracle.layout(gi, w.E, w.R)   # the layout of the device's own routing, bit for bit
    assert hnp["error_flag"][0] == 0
    assert np.array_equal(hnp["expert_counts"], L.expert_counts)
    assert np.array_equal(hnp["expert_offsets"], L.expert_offsets)
    assert np.array_equal(hnp["rank_counts"], L.rank_counts)
    assert np.array_equal(hnp["rank_offsets"], L.rank_offsets)
    assert np.array_equal(hnp["slot_of"].reshape(-1), L.slot_of.reshape(-1))
    assert np.array_equal(hnp["src_of"], L.src_of)


def test_route_layout_flags_a_missing_replica():
    # logical expert 0 has no replica: its picks become -1 and the layout
    # raises EP_DEVERR_INDEX
    El, E, T, k = 16, 16, 64, 4
    off = np.array([0, 0] + list(range(1, El)), np.int32)   # n_0 = 0, the others 1
    assert off.shape == (El + 1,)
    slots = np.arange(E, dtype=np.int32)
    z = np.zeros((T, El), np.float32)
    z[:, 0] = 5.0   # everyone picks expert 0 first
    gi, _ = check(T, k, E, z, gate="softmax", rep_offsets=off, rep_slots=slots)
    assert np.all(gi[:, 0] == -1)
    cfg = ep.Config(T, 128, k, E, 4)
    from combine_ep_layout_03_amd.buffers import Handle, alloc_workspace
    h = Handle.alloc(cfg, "cuda")
    for t in vars(h).values():
        t.view(torch.uint8).fill_(POISON)
    ws = alloc_workspace(cfg, "cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ep.ep_route_layout(cfg, ep.Router(El, "softmax"), to_dev(z), None, to_dev(off), to_dev(slots),
                       idx, wts, h, ws)
    torch.cuda.synchronize()
    assert int(h.error_flag.cpu()[0]) & ep.EP_DEVERR_INDEX


def route_layout(T, k, E, R, z, num_workgroups=0, **kw):
    """ep_route_layout on fresh poisoned buffers: (idx, weights, handle arrays)."""
    from combine_ep_layout_03_amd.buffers import Handle, alloc_workspace
    cfg = ep.Config(T, 128, k, E, R, num_workgroups=num_workgroups)
    rt = ep.Router(z.shape[1], kw.get("gate", "sigmoid"), kw.get("n_groups", 1), kw.get("topk_groups", 1),
                   kw.get("group_topn", 2), kw.get("renorm", True))
    h = Handle.alloc(cfg, "cuda")
    for t in vars(h).values():
        t.view(torch.uint8).fill_(POISON)
    ws = alloc_workspace(cfg, "cuda")
    ws.fill_(0x5A)   # contents on entry must not matter
    opt = lambda a: None if kw.get(a) is None else to_dev(kw[a])
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    ep.ep_route_layout(cfg, rt, to_dev(z), opt("bias"), opt("rep_offsets"), opt("rep_slots"), idx, wts, h, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wts.cpu().numpy(), {n: t.cpu().numpy() for n, t in vars(h).items()}


# Shapes of the router-counted layout (the router writes the chunk table, the
# scatter kernel follows): one router step per chunk (2048 and 8192 tokens),
# a one-token tail chunk with odd k, two steps per chunk (8193 tokens), three
# steps with E = 512 and odd k, groups + bias, replicas; and the same call
# with num_workgroups set, which takes router + two-launch layout instead.
@pytest.mark.parametrize("T,El,k,G,TG,extra", [
    (2048, 256, 8, 1, 1, ""), (2049, 64, 5, 1, 1, ""), (8192, 256, 8, 8, 4, "bias"),
    (8193, 256, 8, 8, 4, ""), (20000, 512, 3, 1, 1, ""), (3000, 128, 16, 4, 2, "bias"),
    (4100, 256, 8, 8, 4, "replicas"),
])
def test_route_layout_router_counted(T, El, k, G, TG, extra):
    rng = np.random.default_rng(T + El + k)
    z = (rng.standard_normal((T, El)) * 2).astype(np.float32)
    kw = dict(gate="sigmoid" if T % 2 == 0 else "softmax", n_groups=G, topk_groups=TG)
    E = El
    if extra == "bias":
        kw["bias"] = (rng.standard_normal(El) * 0.5).astype(np.float32)
    if extra == "replicas":
        n = 1 + (rng.random(El) < 0.125).astype(np.int64)
        kw["rep_offsets"] = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        E = int(kw["rep_offsets"][-1])
        kw["rep_slots"] = rng.permutation(E).astype(np.int32)
    R = 8 if E % 8 == 0 else 1
    say(f"route_layout counted T={T} El={El} k={k} E={E} R={R} G={G} TG={TG} {extra}")
    for nwg in (0, 7):
        gi, gw, h = route_layout(T, k, E, R, z, num_workgroups=nwg, **kw)
        check_routing(gi, gw, z, k, **kw)
        L = oracle.layout(gi, E, R)   # the layout of the device's own routing, bit for bit
        assert h["error_flag"][0] == 0, nwg
        for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "src_of"):
            assert np.array_equal(h[key].reshape(-1), getattr(L, key).reshape(-1)), (nwg, key)
        assert np.array_equal(h["slot_of"].reshape(-1), L.slot_of.reshape(-1)), nwg


def test_route_layout_router_counted_flags_a_missing_replica():
    # at a size where the router counts the table: the -1 picks land in the
    # table's bad-index entry and the scatter raises EP_DEVERR_INDEX
    El, T, k = 64, 2048, 5     # 10240 pairs: the two-launch layout's size
    off = np.array([0, 0] + list(range(1, El)), np.int32)   # n_0 = 0, the others 1
    slots = np.arange(El - 1, dtype=np.int32)
    z = np.zeros((T, El), np.float32)
    z[:, 0] = 5.0
    gi, _, h = route_layout(T, k, El - 1, 1, z, gate="softmax", rep_offsets=off, rep_slots=slots)
    assert np.all(gi[:, 0] == -1)
    assert int(h["error_flag"][0]) & ep.EP_DEVERR_INDEX
