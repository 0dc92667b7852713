"""GPU parity of the combine-with-shared-expert and combine-backward entry
points against the oracle, through the C ABI.

Bar: combine_shared within the 1e-2 combine tolerance (bit mismatches
reported); grad_recv rows bit-exact (one fp32 multiply, then bf16 nearest
even, on both sides); grad_weights within 1e-5 * sum_h |g_h y_h| of the
oracle's float64 dot product (the fp32 accumulation of a thread's channels,
a 64-lane butterfly and a sum over 8 waves is bounded by well under
120 * 2^-24 of that sum at H <= 7168).
"""
import numpy as np
import pytest
import torch

import combine_ep_layout_03_amd as ep
import oracle
from workloads import CONFIGS, make_workload, make_expert_rows, bf16_from_f32

from gpu_util import GpuRun, POISON, rel_err, rows_to_dev, say, u16, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load()


def prep(name, T=None):
    w = make_workload(name, T=T)
    run = GpuRun(w).layout()
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    return w, run, L, ys


@pytest.mark.parametrize("name", list(CONFIGS))
def test_combine_shared_full_configs(name):
    w, run, L, ys = prep(name)
    say(f"combine_shared {name}")
    shared = bf16_from_f32(np.random.default_rng(3).standard_normal((w.T, w.H)).astype(np.float32))
    run.put_expert_rows(ys)
    out = torch.empty((w.T, w.H), dtype=torch.int16, device="cuda")
    ep.ep_combine_shared(run.cfg, run.h, run.idx, run.ybufs, run.wts, to_dev(shared), out, run.cap)
    torch.cuda.synchronize()
    ref = oracle.combine_shared(ys, w.topk_idx, L, w.topk_w, shared)
    got = u16(out)
    say(f"  max rel err {rel_err(got, ref):.3g}, bit mismatches {int(np.count_nonzero(got != ref))}")
    assert rel_err(got, ref) <= 1e-2
    assert np.array_equal(got, ref)


def check_backward(w, run, L, ys, weights=True, with_w=True):
    rng = np.random.default_rng(11)
    g = bf16_from_f32(rng.standard_normal((w.T, w.H)).astype(np.float32))
    grad_rows = rows_to_dev(run.cap, w.H, [np.zeros((0, w.H), np.uint16)] * w.R)
    ybufs = rows_to_dev(run.cap, w.H, ys) if with_w else None
    gw = torch.full((w.T, w.k), float("nan"), dtype=torch.float32, device="cuda") if with_w else None
    ep.ep_combine_backward(run.cfg, run.h, run.idx, to_dev(g), run.wts if weights else None, ybufs,
                           grad_rows, gw, run.cap)
    torch.cuda.synchronize()
    ref_rows, ref_gw = oracle.combine_backward(g, w.topk_idx, L, w.topk_w if weights else None,
                                               ys if with_w else None)
    for r in range(w.R):
        n = int(L.rank_counts[r])
        got = grad_rows[r].cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:n], ref_rows[r]), f"rank {r}"
        assert np.all(got[n:].view(np.uint8) == POISON)
    if with_w:
        got_w = gw.cpu().numpy()
        yrow = oracle.bf16_to_f32(np.concatenate(ys)[L.slot_of]).astype(np.float64).reshape(w.T, w.k, w.H)
        mag = np.einsum("th,tkh->tk", np.abs(oracle.bf16_to_f32(g).astype(np.float64)), np.abs(yrow))
        err = np.abs(got_w.astype(np.float64) - ref_gw.astype(np.float64))
        say(f"  grad_w max err / sum|gy| = {float(np.max(err / np.maximum(mag, 1e-30))):.3g}")
        assert np.all(err <= 1e-5 * mag + 1e-30)


@pytest.mark.parametrize("name", ["tiny", "ds16b", "decode", "v3"])
def test_combine_backward_full_configs(name):
    w, run, L, ys = prep(name)
    say(f"combine_backward {name}")
    check_backward(w, run, L, ys)


def test_combine_backward_unit_weights_no_grad_w():
    w, run, L, ys = prep("ds16b", T=777)
    say("combine_backward unit weights, no grad_w")
    check_backward(w, run, L, ys, weights=False, with_w=False)


@pytest.mark.parametrize("T,H,k,E,R", [(1, 8, 1, 1, 1), (33, 264, 9, 18, 6), (70, 512, 32, 64, 8)])
def test_combine_backward_small_ragged(T, H, k, E, R):
    from test_gpu_parity import custom
    rng = np.random.default_rng(T + k)
    w = custom("bw", T, H, k, E, R, False, rng.integers(0, E, (T, k)), seed=T)
    run = GpuRun(w).layout()
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    say(f"combine_backward small T={T} H={H} k={k}")
    check_backward(w, run, L, ys)


def test_combine_backward_grid_size_invariance():
    """Gradient rows and grad_w are bit-identical for any grid size (the
    reduction order is fixed by the thread, not the grid); H = 12296 takes
    several ragged chunk rounds per thread."""
    from test_gpu_parity import custom
    rng = np.random.default_rng(5)
    w = custom("bwg", 150, 12296, 8, 64, 8, False, rng.integers(0, 64, (150, 8)), seed=5)
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    g = to_dev(bf16_from_f32(rng.standard_normal((w.T, w.H)).astype(np.float32)))
    outs = []
    for nwg in (0, 1, 7, 300):
        run = GpuRun(w, num_workgroups=nwg).layout()
        say(f"combine_backward num_workgroups={nwg}")
        rows = rows_to_dev(run.cap, w.H, [np.zeros((0, w.H), np.uint16)] * w.R)
        gw = torch.full((w.T, w.k), float("nan"), dtype=torch.float32, device="cuda")
        ep.ep_combine_backward(run.cfg, run.h, run.idx, g, run.wts, rows_to_dev(run.cap, w.H, ys),
                               rows, gw, run.cap)
        torch.cuda.synchronize()
        outs.append(([r[:int(L.rank_counts[i])].cpu().numpy() for i, r in enumerate(rows)],
                     gw.cpu().numpy()))
        del rows
    check_backward(w, GpuRun(w).layout(), L, ys)   # and the result is right
    for rows, gwn in outs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(rows, outs[0][0]))
        assert np.array_equal(gwn.view(np.uint32), outs[0][1].view(np.uint32))


@pytest.mark.parametrize("nwg", [0, 7, 300])
def test_combine_backward_two_launch_form(nwg):
    """T >= 2048 takes two launches (the gradient rows as a weighted BF16
    dispatch, then grad_w alone).  k = 12 > 8 runs the grad_w kernel's second
    block of pairs, H = 1544 (193 chunks) leaves the last 128-chunk unit
    ragged, and the results are bit-identical for any grid size."""
    from test_gpu_parity import custom
    T, H, k, E, R = 2100, 1544, 12, 24, 4
    rng = np.random.default_rng(21)
    w = custom("bw2", T, H, k, E, R, False, rng.integers(0, E, (T, k)), seed=21)
    run = GpuRun(w, num_workgroups=nwg).layout()
    L = oracle.layout(w.topk_idx, w.E, w.R)
    y = make_expert_rows(w.P, w.H)
    ys = [y[L.rank_offsets[r]:L.rank_offsets[r + 1]] for r in range(w.R)]
    say(f"combine_backward two launches T={T} H={H} k={k} num_workgroups={nwg}")
    check_backward(w, run, L, ys)
    check_backward(w, run, L, ys, weights=False, with_w=False)


def test_combine_backward_two_launch_form_after_a_bad_index():
    """An index outside [0,E) stops both launches of the large-batch backward:
    no gradient row and no grad_w is written."""
    from test_gpu_parity import custom
    T, H, k, E, R = 2048, 256, 4, 16, 4
    idx = np.random.default_rng(4).integers(0, E, (T, k))
    idx[1500, 2] = -3
    w = custom("bad2", T, H, k, E, R, False, idx)
    run = GpuRun(w).layout()
    assert int(run.handle_np()["error_flag"][0]) & ep.EP_DEVERR_INDEX
    say("combine_backward two launches after a bad index")
    ones = lambda *shape: to_dev(bf16_from_f32(np.ones(shape, np.float32)))
    ys = [ones(run.cap, H) for _ in range(R)]
    grows = [torch.full((run.cap, H), 0x5A5A, dtype=torch.int16, device="cuda") for _ in range(R)]
    gw = torch.full((T, k), 7.0, dtype=torch.float32, device="cuda")
    ep.ep_combine_backward(run.cfg, run.h, run.idx, ones(T, H), run.wts, ys, grows, gw, run.cap)
    torch.cuda.synchronize()
    assert all(torch.all(g == 0x5A5A) for g in grows) and torch.all(gw == 7.0)


def test_dispatch_backward_is_unit_weight_combine():
    """The backward of dispatch: sum each token's k gradient rows (ep_combine
    with unit weights) equals the oracle's unit-weight combine."""
    w, run, L, ys = prep("ds16b", T=1000)
    say("dispatch backward")
    run.put_expert_rows(ys).combine(weights=False)
    torch.cuda.synchronize()
    ref = oracle.combine(ys, w.topk_idx, L, None)
    assert np.array_equal(u16(run.out), ref)


def test_backward_rejects_half_given_grad_w():
    w, run, L, ys = prep("tiny")
    g = torch.zeros((w.T, w.H), dtype=torch.int16, device="cuda")
    rows = rows_to_dev(run.cap, w.H, [np.zeros((0, w.H), np.uint16)] * w.R)
    with pytest.raises(ep.EpError) as ei:
        ep.ep_combine_backward(run.cfg, run.h, run.idx, g, run.wts, rows, rows, None, run.cap)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG


def test_entry_points_write_nothing_after_a_bad_index():
    """An index outside [0,E) sets EP_DEVERR_INDEX in the handle; the shared-
    expert combine, the combine backward and the SiLU re-quantization read the
    error word first and leave every output byte untouched."""
    from test_gpu_parity import custom
    T, H, k, E, R, I = 64, 256, 4, 16, 4, 256
    idx = np.random.default_rng(3).integers(0, E, (T, k))
    idx[17, 1] = E + 5
    w = custom("bad", T, H, k, E, R, False, idx)
    run = GpuRun(w).layout()
    assert int(run.handle_np()["error_flag"][0]) & ep.EP_DEVERR_INDEX
    say("entry points after a bad index")
    rnd = lambda *shape: to_dev(bf16_from_f32(np.ones(shape, np.float32)))
    ys = [rnd(run.cap, H) for _ in range(R)]
    out = torch.full((T, H), 0x5A5A, dtype=torch.int16, device="cuda")
    ep.ep_combine_shared(run.cfg, run.h, run.idx, ys, run.wts, rnd(T, H), out, run.cap)
    grows = [torch.full((run.cap, H), 0x5A5A, dtype=torch.int16, device="cuda") for _ in range(R)]
    gw = torch.full((T, k), 7.0, dtype=torch.float32, device="cuda")
    ep.ep_combine_backward(run.cfg, run.h, run.idx, rnd(T, H), run.wts, ys, grows, gw, run.cap)
    q = [torch.full((run.cap, I), POISON, dtype=torch.uint8, device="cuda") for _ in range(R)]
    s = [torch.full((run.cap, I // 128), 7.0, dtype=torch.float32, device="cuda") for _ in range(R)]
    ep.ep_silu_mul_quant(run.cfg, run.h, I, [rnd(run.cap, 2 * I) for _ in range(R)], q, s, run.cap)
    torch.cuda.synchronize()
    assert torch.all(out == 0x5A5A)
    assert all(torch.all(g == 0x5A5A) for g in grows) and torch.all(gw == 7.0)
    assert all(torch.all(t == POISON) for t in q) and all(torch.all(t == 7.0) for t in s)
