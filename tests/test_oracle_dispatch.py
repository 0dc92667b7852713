"""Pins for the oracle's dispatch (BF16 copy and FP8 per-128-channel
quantization) and un-permute.

Pinned against:
  * the closed form unpermute(dispatch_bf16(x))[t*k + j] == x[t];
  * an independent FP8 computation built from library primitives: numpy
    float32 max / division for amax and the scale, torch's float8_e4m3fn cast
    for the code (exact for |x/s| <= 464, which always holds here);
  * properties the method fixes: every nonzero block has a code of magnitude
    448 at its amax, the half-ulp error bound of E4M3, byte-identical copies.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, edge_case_x


def independent_fp8(x_bits: np.ndarray):
    """amax / 448 scale and E4M3 codes from numpy float32 arithmetic and
    torch's cast."""
    T, H = x_bits.shape
    xf = oracle.bf16_to_f32(x_bits).reshape(T, H // 128, 128)
    a = np.abs(xf).max(axis=2)                                   # exact
    s = (a / np.float32(448.0)).astype(np.float32)               # binary32 division
    zero = a == 0
    s_safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
    ratio = (xf / s_safe[:, :, None]).astype(np.float32)         # binary32 division
    assert np.all(np.abs(ratio[~zero]) <= 464.0)
    q = torch.from_numpy(np.ascontiguousarray(ratio)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy().copy()
    q[zero] = 0
    s = np.where(zero, np.float32(0.0), s).astype(np.float32)
    return q.reshape(T, H), s


@pytest.mark.parametrize("src", ["normal", "edge"])
def test_quantize_matches_independent_computation(src):
    if src == "normal":
        x = make_workload("v3", T=64).x
    else:
        x = edge_case_x(64, 1024, seed=3)
    q, s = oracle.quantize_rows(x)
    q2, s2 = independent_fp8(x)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(q, q2)


@pytest.mark.parametrize("src", ["normal", "edge"])
def test_quantize_properties(src):
    x = make_workload("v3", T=32).x if src == "normal" else edge_case_x(96, 1024, seed=4)
    T, H = x.shape
    q, s = oracle.quantize_rows(x)
    xf = oracle.bf16_to_f32(x).reshape(T, H // 128, 128).astype(np.float64)
    qb = q.reshape(T, H // 128, 128)
    a = np.abs(xf).max(axis=2)
    nz = a > 0
    # P-Q4: the amax element of each nonzero block maps to +-448 (0x7E / 0xFE)
    arg = np.abs(xf).argmax(axis=2)
    at_max = np.take_along_axis(qb, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((at_max[nz] & 0x7F) == 0x7E)
    # zero blocks: s == 0 and all codes 0x00
    assert np.all(s[~nz] == 0) and np.all(qb[~nz] == 0)
    # P-Q5: |dec(q)*s - x| <= max(2^-4 |x|, 2^-10 s) * (1 + 2^-20)
    dec = oracle.e4m3_decode(qb).astype(np.float64)
    sd = s.astype(np.float64)[:, :, None]
    err = np.abs(dec * sd - xf)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sd) * (1 + 2.0 ** -20)
    assert np.all(err[nz] <= bound[nz])
    # signed zeros keep their sign inside nonzero blocks
    negzero = (x.reshape(T, H // 128, 128) == 0x8000) & nz[:, :, None]
    assert np.all(qb[negzero] == 0x80)


@pytest.mark.parametrize("name", ["tiny", "ds16b", "decode"])
def test_bf16_dispatch_unpermute_closed_form(name):
    w = make_workload(name)
    L = oracle.layout(w.topk_idx, w.E, w.R)
    recv = oracle.dispatch_bf16(w.x, w.topk_idx, L)
    assert [r.shape[0] for r in recv] == list(L.rank_counts)
    u = oracle.unpermute(recv, w.topk_idx, L)
    assert np.array_equal(u, np.repeat(w.x, w.k, axis=0))
    # each rank's rows in slot order are x of the source tokens
    src_tok = L.src_of // w.k
    allrows = np.concatenate(recv)
    assert np.array_equal(allrows, w.x[src_tok])


@pytest.mark.parametrize("name", ["v3", "decode"])
def test_fp8_dispatch_copies_and_placement(name):
    w = make_workload(name, T=48)
    L = oracle.layout(w.topk_idx, w.E, w.R)
    rq, rs = oracle.dispatch_fp8(w.x, w.topk_idx, L)
    q, s = oracle.quantize_rows(w.x)
    allq = np.concatenate(rq)
    alls = np.concatenate(rs)
    src_tok = L.src_of // w.k
    # P-Q6: every received copy of token t is q[t] / s[t], byte for byte
    assert np.array_equal(allq, q[src_tok])
    assert np.array_equal(alls.view(np.uint32), s[src_tok].view(np.uint32))


def test_fp8_dispatch_full_headline_shape():
    """The headline shape end to end through the C oracle (a few seconds)."""
    w = make_workload("v3")
    L = oracle.layout(w.topk_idx, w.E, w.R)
    rq, rs = oracle.dispatch_fp8(w.x, w.topk_idx, L)
    assert sum(r.shape[0] for r in rq) == w.T * w.k
    # sample 64 tokens and recheck them against the independent computation
    rng = np.random.default_rng(5)
    toks = rng.choice(w.T, 64, replace=False)
    q2, s2 = independent_fp8(w.x[toks])
    rank = w.topk_idx.ravel() // (w.E // w.R)
    for i, t in enumerate(toks):
        for j in range(w.k):
            p = t * w.k + j
            r, row = rank[p], L.row_of[p]
            assert np.array_equal(rq[r][row], q2[i])
            assert np.array_equal(rs[r][row].view(np.uint32), s2[i].view(np.uint32))


def nonfinite_rows(seed=0):
    """Rows whose 128-channel blocks hold, in turn: a finite control, +inf,
    -inf, a NaN, a NaN and an inf, every value inf, signed zeros with an inf."""
    rng = np.random.default_rng(seed)
    H = 128 * 7
    xf = rng.standard_normal((3, H)).astype(np.float32)
    for t in range(3):
        xf[t, 128 + 5 + t] = np.inf
        xf[t, 256 + 17] = -np.inf
        xf[t, 384 + 100 - t] = np.nan
        xf[t, 512 + 3] = np.nan
        xf[t, 512 + 90] = -np.inf
        xf[t, 640:768] = np.inf * np.where(rng.random(128) < 0.5, 1, -1)
        xf[t, 768:896] = np.where(rng.random(128) < 0.5, 0.0, -0.0)
        xf[t, 768 + 64] = np.inf
    from workloads import bf16_from_f32
    return bf16_from_f32(xf)


def test_nonfinite_blocks_follow_ieee_arithmetic():
    """The quantizer with non-finite inputs (R29): a = max|x| taken so that a
    NaN makes it NaN (numpy's max), s = a/448 and the codes of x/s in IEEE
    binary32 (x/inf = 0 with x's sign, inf/inf = NaN), NaN codes and NaN
    scales compared as NaN, whatever their sign or payload."""
    x = nonfinite_rows()
    T, H = x.shape
    q, s = oracle.quantize_rows(x)
    xf = oracle.bf16_to_f32(x).reshape(T, H // 128, 128)
    with np.errstate(invalid="ignore"):
        a = np.abs(xf).max(axis=2)                               # NaN propagates
        s2 = (a / np.float32(448.0)).astype(np.float32)
        ratio = (xf / s2[:, :, None]).astype(np.float32)
    q2 = torch.from_numpy(np.ascontiguousarray(ratio)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q2 = q2.reshape(T, H)
    nan_q, nan_q2 = (q & 0x7F) == 0x7F, (q2 & 0x7F) == 0x7F
    assert np.array_equal(nan_q, nan_q2)
    assert np.array_equal(q[~nan_q], q2[~nan_q2])
    assert np.array_equal(np.isnan(s), np.isnan(s2))
    fin = ~np.isnan(s)
    assert np.array_equal(s[fin].view(np.uint32), s2[fin].view(np.uint32))
    qb = q.reshape(T, H // 128, 128)
    # the cases spelled out: control block finite; an inf block scales by inf
    # and its finite values encode as signed zeros; a NaN poisons its block
    assert np.all(np.isfinite(s[:, 0])) and not np.any((qb[:, 0] & 0x7F) == 0x7F)
    assert np.all(np.isinf(s[:, 1])) and np.all(np.isinf(s[:, 2]))
    for t in range(T):
        fin1 = np.isfinite(xf[t, 1])
        assert np.all(qb[t, 1][fin1] & 0x7F == 0) and np.all((qb[t, 1][~fin1] & 0x7F) == 0x7F)
        assert np.array_equal(qb[t, 1][fin1] >> 7, np.signbit(xf[t, 1][fin1]).astype(np.uint8))
    assert np.all(np.isnan(s[:, 3])) and np.all((qb[:, 3] & 0x7F) == 0x7F)
    assert np.all(np.isnan(s[:, 4])) and np.all((qb[:, 4] & 0x7F) == 0x7F)
    assert np.all(np.isinf(s[:, 5])) and np.all((qb[:, 5] & 0x7F) == 0x7F)
    # the pure-Python twin agrees
    from oracle import twin
    for t in range(T):
        ct, st = twin.quantize_row(x[t].tolist())
        ct = np.array(ct, np.uint8)
        nt = (ct & 0x7F) == 0x7F
        assert np.array_equal(nt, nan_q[t]) and np.array_equal(ct[~nt], q[t][~nan_q[t]])
        st = np.array(st, np.float32)
        assert np.array_equal(np.isnan(st), np.isnan(s[t]))
        assert np.array_equal(st[~np.isnan(st)].view(np.uint32), s[t][~np.isnan(s[t])].view(np.uint32))


def test_silu_requant_of_nonfinite_activations():
    """The SiLU re-quantization's quantizer follows the same R29 arithmetic on
    the oracle's activation: gates +inf (activation +-inf), -inf and NaN
    (activation NaN) among finite ones."""
    rng = np.random.default_rng(4)
    I = 128 * 4
    from workloads import bf16_from_f32
    g = rng.standard_normal((2, I)).astype(np.float32)
    u = rng.standard_normal((2, I)).astype(np.float32)
    g[:, 128 + 7] = np.inf
    g[:, 256 + 9] = -np.inf
    g[:, 384 + 1] = np.nan
    rows = bf16_from_f32(np.concatenate([g, u], axis=1))
    q, s = oracle.silu_mul_quant(rows)
    act = oracle.silu_mul(rows).reshape(2, I // 128, 128)
    with np.errstate(invalid="ignore"):
        a = np.abs(act).max(axis=2)
        s2 = (a / np.float32(448.0)).astype(np.float32)
        ratio = (act / s2[:, :, None]).astype(np.float32)
    q2 = torch.from_numpy(np.ascontiguousarray(ratio)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(2, I)
    nan_q, nan_q2 = (q & 0x7F) == 0x7F, (q2 & 0x7F) == 0x7F
    assert np.array_equal(nan_q, nan_q2) and np.array_equal(q[~nan_q], q2[~nan_q2])
    assert np.array_equal(np.isnan(s), np.isnan(s2))
    assert np.array_equal(s[~np.isnan(s)].view(np.uint32), s2[~np.isnan(s2)].view(np.uint32))
    assert np.all(np.isinf(s[:, 1])) and np.all(np.isnan(s[:, 2])) and np.all(np.isnan(s[:, 3]))
