"""The C oracle against its pure-Python twin (oracle/twin.py) on tiny inputs.

The twin is a second, independently written implementation of the same
definitions (integers, lists, struct and exact fractions; nothing shared with
ep_oracle.c), so agreement bit for bit is a consistency check of both -- a
slip in either one's indexing, rounding or tie rule shows up here.  It is not
counted as a pin: the pins are the independent facts in the other oracle
tests.
"""
import numpy as np
import pytest

import oracle
from oracle import twin
from workloads import bf16_from_f32, edge_case_x


def case(seed, T, H, k, E, R, edge=False):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)      # repeats allowed
    x = edge_case_x(T, H, seed) if edge else bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    return idx, x, w


CASES = [(1, 3, 128, 2, 4, 2), (2, 5, 256, 3, 6, 3), (3, 7, 128, 1, 4, 4), (4, 4, 128, 4, 8, 1),
         (5, 2, 384, 3, 3, 3), (6, 6, 128, 2, 2, 1)]


@pytest.mark.parametrize("seed,T,H,k,E,R", CASES)
def test_layout_and_dispatch_match_the_twin(seed, T, H, k, E, R):
    idx, x, _ = case(seed, T, H, k, E, R)
    L = oracle.layout(idx, E, R)
    Lt = twin.layout(idx.tolist(), E, R)
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "slot_of", "src_of"):
        assert getattr(L, key).tolist() == Lt[key], key
    rb = oracle.dispatch_bf16(x, idx, L)
    rbt = twin.dispatch_bf16(x.tolist(), idx.tolist(), E, R, Lt)
    for r in range(R):
        assert rb[r].tolist() == rbt[r]
    u = oracle.unpermute(rb, idx, L)
    assert u.tolist() == twin.unpermute(rbt, idx.tolist(), E, R, Lt)


@pytest.mark.parametrize("seed,T,H,k,E,R", CASES[:4])
@pytest.mark.parametrize("edge", [False, True])
def test_fp8_dispatch_matches_the_twin(seed, T, H, k, E, R, edge):
    idx, x, _ = case(seed, T, H, k, E, R, edge)
    L = oracle.layout(idx, E, R)
    Lt = twin.layout(idx.tolist(), E, R)
    rq, rs = oracle.dispatch_fp8(x, idx, L)
    rqt, rst = twin.dispatch_fp8(x.tolist(), idx.tolist(), E, R, Lt)
    for r in range(R):
        assert rq[r].tolist() == rqt[r]
        assert rs[r].view(np.uint32).tolist() == [[twin.f32_bits(v) for v in row] for row in rst[r]]


@pytest.mark.parametrize("seed,T,H,k,E,R", CASES)
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_matches_the_twin(seed, T, H, k, E, R, weighted):
    idx, _, w = case(seed, T, H, k, E, R)
    L = oracle.layout(idx, E, R)
    Lt = twin.layout(idx.tolist(), E, R)
    rng = np.random.default_rng(seed + 100)
    ys = [bf16_from_f32((rng.standard_normal((int(n), H)) * 3).astype(np.float32)) for n in L.rank_counts]
    out = oracle.combine(ys, idx, L, w if weighted else None)
    outt = twin.combine([y.tolist() for y in ys], idx.tolist(), E, R, Lt,
                        w.tolist() if weighted else None)
    assert out.tolist() == outt


def test_twin_codecs_on_special_values():
    # spot values with known codes: 448 -> 0x7E, 2^-9 -> 0x01, a tie between
    # 1.0 and 1.125 goes to the even mantissa (1.0), -0 keeps its sign
    assert twin.e4m3_encode(448.0) == 0x7E and twin.e4m3_encode(1000.0) == 0x7E
    assert twin.e4m3_encode(2.0 ** -9) == 0x01 and twin.e4m3_encode(1.0625) == 0x38
    assert twin.e4m3_encode(-0.0) == 0x80 and twin.e4m3_encode(2.0 ** -11) == 0x00
    for c in range(256):
        v = twin.e4m3_value(c)
        if v == v:
            assert twin.e4m3_encode(v) == c or (v == 0 and c in (0x00, 0x80))
    assert twin.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80       # tie to even
    assert twin.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert twin.round_f32_exact(twin.Fraction(1, 3)) == twin.f32(1 / 3)
