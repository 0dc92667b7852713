"""Randomized parity sweep: seeded random shapes through layout, dispatch,
combine and the one-launch layout + dispatch, each against the oracle.

Every case draws T, k, E, R, H, the dispatch dtype and an index distribution
(uniform, Zipf-skewed, few experts with repeats inside a token's row), so the
sweep crosses the layout's three launch shapes (<= 2048 pairs, <= 8192 pairs
with E <= 384, two launches) and ragged tails in combinations the hand-picked
cases do not.  Sizes stay small enough for the oracle to finish in a second.
The bar is the usual one: layout and dispatch bytes exact, combine within
1e-2 relative (bit mismatches reported).

Two more sweeps draw random router configurations (gate, groups, kept
groups, group score form, bias, replicas; both router kernels by batch size)
checked bit for bit, and random shapes through the shared-expert combine,
both combine-backward paths and the SiLU re-quantization.  A last sweep draws
ep_route_layout shapes on which the router counts the layout's chunk table.
"""
import numpy as np
import pytest
import torch

import combine_ep_layout_03_amd as ep
import oracle
from workloads import make_expert_rows

from gpu_util import GpuRun, POISON, rel_err, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load()


def random_case(seed):
    from test_gpu_parity import custom
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16, 36, 64]))
    E = R * int(rng.choice([1, 2, 3, 8, 16, 32]))
    E = min(E, 2048)
    k = int(rng.integers(1, min(32, 2 * E) + 1))
    T = int(rng.choice([1, 7, 63, 200, 511, 1100, 2600])) + int(rng.integers(0, 5))
    fp8 = bool(rng.integers(0, 2))
    H = 128 * int(rng.integers(1, 9)) if fp8 else 8 * int(rng.integers(1, 80))
    kind = ["uniform", "zipf", "few"][seed % 3]
    if kind == "uniform":
        idx = rng.integers(0, E, (T, k))
    elif kind == "zipf":
        p = 1.0 / (1.0 + np.arange(E)) ** 1.2
        idx = rng.choice(E, (T, k), p=p / p.sum())
    else:
        idx = rng.integers(0, min(E, 3), (T, k))   # repeats inside a row
    return custom(f"rand{seed}", T, H, k, E, R, fp8, idx, seed=seed), kind


def check_path(w, run, label):
    L = oracle.layout(w.topk_idx, w.E, w.R)
    g = run.handle_np()
    assert g["error_flag"][0] == 0, label
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "src_of"):
        assert np.array_equal(g[key].reshape(-1), getattr(L, key).reshape(-1)), (label, key)
    assert np.array_equal(g["slot_of"].reshape(-1), L.slot_of.reshape(-1)), label
    xs, ss = run.recv_np(L.rank_counts)
    if w.fp8:
        rq, rs = oracle.dispatch_fp8(w.x, w.topk_idx, L)
        for r in range(w.R):
            assert np.array_equal(xs[r], rq[r]), (label, r)
            assert np.array_equal(ss[r].view(np.uint32), rs[r].view(np.uint32)), (label, r)
    else:
        rx = oracle.dispatch_bf16(w.x, w.topk_idx, L)
        for r in range(w.R):
            assert np.array_equal(xs[r], rx[r]), (label, r)
    full, _ = run.recv_np(L.rank_counts, full=True)
    for r in range(w.R):
        assert np.all(full[r][int(L.rank_counts[r]):].view(np.uint8) == POISON), (label, r)
    return L


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(seed):
    w, kind = random_case(seed)
    say(f"random {seed}: T={w.T} H={w.H} k={w.k} E={w.E} R={w.R} fp8={w.fp8} {kind} P={w.P}")
    run = GpuRun(w).layout().dispatch()
    L = check_path(w, run, "layout + dispatch")
    y = make_expert_rows(w.P, w.H, seed=seed + 7)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    run.put_expert_rows(ys).combine()
    torch.cuda.synchronize()
    ref = oracle.combine(ys, w.topk_idx, L, w.topk_w)
    got = u16(run.out)
    assert rel_err(got, ref) <= 1e-2
    say(f"  combine bit mismatches {int(np.count_nonzero(got != ref))} / {got.size}")
    # the one-launch layout + dispatch gives the same handle and bytes
    from combine_ep_layout_03_amd.buffers import RecvBuffers
    run2 = GpuRun(w)
    run2.recv = RecvBuffers.alloc(run2.cfg, run2.cap, device="cuda", fill=POISON)
    ep.ep_layout_dispatch(run2.cfg, run2.idx, run2.h, run2.ws, run2.x, run2.recv.x, run2.recv.scales,
                          run2.cap)
    check_path(w, run2, "layout_dispatch")


@pytest.mark.parametrize("seed", range(16))
def test_random_router(seed):
    """Random router configurations (both kernels, every group form, bias,
    replicas) bit for bit against the oracle."""
    from test_gpu_router import check
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([1, 1, 2, 4, 8, 16]))
    gs = int(rng.choice([1, 2, 4, 8, 16, 32]))
    El = min(G * gs, 512)
    gs = El // G
    TG = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(TG * gs, 16) + 1))
    T = int(rng.choice([1, 37, 300, 2048, 2300]))
    gate = ["softmax", "sigmoid"][int(rng.integers(0, 2))]
    z = (rng.standard_normal((T, El)) * float(rng.choice([0.5, 2, 8]))).astype(np.float32)
    kw = dict(gate=gate, n_groups=G, topk_groups=TG, group_topn=int(rng.integers(1, 3)),
              renorm=bool(rng.integers(0, 2)))
    E = El
    if rng.integers(0, 2):
        kw["bias"] = (rng.standard_normal(El) * 0.5).astype(np.float32)
    if rng.integers(0, 2):
        n = 1 + rng.integers(0, 3, El)
        kw["rep_offsets"] = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        E = int(kw["rep_offsets"][-1])
        kw["rep_slots"] = rng.permutation(E).astype(np.int32)
    check(T, k, E, z, **kw)


@pytest.mark.parametrize("seed", range(8))
def test_random_shared_backward_and_silu(seed):
    """Random shapes through the shared-expert combine, the combine backward
    (both paths) and the SiLU re-quantization against the oracle."""
    from test_gpu_parity import custom
    from test_gpu_backward import check_backward
    from gpu_util import rows_to_dev, to_dev
    from workloads import bf16_from_f32
    rng = np.random.default_rng(3000 + seed)
    R = int(rng.choice([1, 2, 8, 36]))
    E = R * int(rng.choice([1, 4, 8]))
    k = int(rng.integers(1, min(16, 2 * E) + 1))
    T = int(rng.choice([5, 130, 1500, 2500])) + int(rng.integers(0, 3))
    H = 8 * int(rng.integers(1, 200))
    w = custom(f"rsb{seed}", T, H, k, E, R, False, rng.integers(0, E, (T, k)), seed=seed)
    say(f"random shared/backward {seed}: T={T} H={H} k={k} E={E} R={R}")
    run = GpuRun(w).layout()
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H, seed=seed + 9)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    shared = bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine_shared(run.cfg, run.h, run.idx, rows_to_dev(run.cap, H, ys), run.wts, to_dev(shared),
                         out, run.cap)
    torch.cuda.synchronize()
    ref = oracle.combine_shared(ys, w.topk_idx, L, w.topk_w, shared)
    assert rel_err(u16(out), ref) <= 1e-2
    check_backward(w, run, L, ys)
    # SiLU re-quantization on the same layout: I a multiple of 128
    I = 128 * int(rng.integers(1, 5))
    act = bf16_from_f32((rng.standard_normal((w.P, 2 * I)) * 2).astype(np.float32))
    act_r = [act[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    qs = [torch.full((run.cap, I), POISON, dtype=torch.uint8, device="cuda") for _ in range(w.R)]
    ss = [torch.full((run.cap, I // 128), float("nan"), dtype=torch.float32, device="cuda")
          for _ in range(w.R)]
    ep.ep_silu_mul_quant(run.cfg, run.h, I, rows_to_dev(run.cap, 2 * I, act_r), qs, ss, run.cap)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.silu_mul_quant(act)
    a_ref = oracle.silu_mul(act).astype(np.float64)
    for r in range(w.R):
        n, lo = int(L.rank_counts[r]), int(L.rank_offsets[r])
        q, s = qs[r].cpu().numpy(), ss[r].cpu().numpy()
        assert np.all(q[n:] == POISON) and np.all(np.isnan(s[n:]))
        q, s = q[:n], s[:n].astype(np.float64)
        sr, ar = s_ref[lo:lo + n].astype(np.float64), a_ref[lo:lo + n]
        assert np.all(np.abs(s - sr) <= 1e-6 * np.abs(sr))
        sg = np.repeat(s, 128, axis=1)
        dec = oracle.e4m3_decode(q).astype(np.float64) * sg
        bound = np.maximum(2.0 ** -4 * np.abs(ar), 2.0 ** -10 * sg) * (1 + 1e-5) + 1e-6 * (np.abs(ar) + sg)
        assert np.all(np.abs(dec - ar) <= bound), r


@pytest.mark.parametrize("seed", range(8))
def test_random_route_layout(seed):
    """Random shapes for ep_route_layout where the router counts the layout's
    chunk table (T >= 2048, two-launch layout sizes, E <= 512): indices and
    weights against the oracle's router (bit for bit, else the validity rule),
    the handle against the oracle's layout of the device's routing, and the same bytes with num_workgroups set (router, then
    the two-launch layout)."""
    from test_gpu_router import check_routing, route_layout
    rng = np.random.default_rng(4000 + seed)
    G = int(rng.choice([1, 1, 2, 4, 8]))
    El = int(rng.choice([64, 128, 256, 512]))
    gs = El // G
    TG = int(rng.integers(1, G + 1))
    k = int(rng.integers(2, min(TG * gs, 16) + 1))
    T = int(rng.integers(2048, 12001))
    z = (rng.standard_normal((T, El)) * float(rng.choice([0.5, 2, 8]))).astype(np.float32)
    kw = dict(gate=["softmax", "sigmoid"][seed % 2], n_groups=G, topk_groups=TG,
              group_topn=int(rng.integers(1, 3)), renorm=bool(rng.integers(0, 2)))
    if rng.integers(0, 2):
        kw["bias"] = (rng.standard_normal(El) * 0.5).astype(np.float32)
    E = El
    if El <= 256 and rng.integers(0, 2):
        n = 1 + (rng.random(El) < 0.25).astype(np.int64)
        kw["rep_offsets"] = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        E = int(kw["rep_offsets"][-1])
        kw["rep_slots"] = rng.permutation(E).astype(np.int32)
    R = int(rng.choice([r for r in (1, 2, 4, 8, 16) if E % r == 0]))
    say(f"random route_layout {seed}: T={T} El={El} k={k} E={E} R={R} G={G} TG={TG} "
        f"topn={kw['group_topn']} bias={'bias' in kw}")
    for nwg in (0, 5):
        gi, gw, h = route_layout(T, k, E, R, z, num_workgroups=nwg, **kw)
        check_routing(gi, gw, z, k, **kw)
        L = oracle.layout(gi, E, R)   # the layout of the device's own routing, bit for bit
        assert h["error_flag"][0] == 0, nwg
        for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "src_of"):
            assert np.array_equal(h[key].reshape(-1), getattr(L, key).reshape(-1)), (nwg, key)
        assert np.array_equal(h["slot_of"].reshape(-1), L.slot_of.reshape(-1)), nwg
