"""ep_layout_noalloc (the layout with its chunk table in the library's
file-scope device array, for callers that cannot allocate) against ep_layout
(caller workspace) and the oracle, through the C ABI: two calls in a row, the
second with a smaller input, then the largest table any valid config needs
and a bad index.  The handle is integer work, so every array must match bit
for bit."""
import numpy as np
import pytest
import torch

import combine_ep_layout_03_amd as ep
import oracle
from combine_ep_layout_03_amd.buffers import Handle, alloc_workspace

from gpu_util import POISON, say, to_dev

pytestmark = pytest.mark.gpu

FIELDS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "slot_of", "src_of",
          "error_flag")


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load()


def fresh_handle(cfg):
    h = Handle.alloc(cfg, "cuda")
    for t in vars(h).values():
        t.view(torch.uint8).fill_(POISON)
    return h


def both_layouts(T, k, E, R, idx):
    cfg = ep.Config(T, 128, k, E, R)
    d = to_dev(idx)
    h_ws, h_na = fresh_handle(cfg), fresh_handle(cfg)
    ws = alloc_workspace(cfg, "cuda")
    ws.fill_(POISON)
    ep.ep_layout(cfg, d, h_ws, ws)
    ep.ep_layout_noalloc(cfg, d, h_na)
    torch.cuda.synchronize()
    a = {n: getattr(h_ws, n).cpu().numpy() for n in FIELDS}
    b = {n: getattr(h_na, n).cpu().numpy() for n in FIELDS}
    return a, b


def check(T, k, E, R, idx):
    say(f"layout_noalloc T={T} k={k} E={E} R={R}")
    a, b = both_layouts(T, k, E, R, idx)
    for n in FIELDS:
        assert np.array_equal(a[n], b[n]), n
    assert b["error_flag"][0] == 0
    L = oracle.layout(idx, E, R)
    for n in FIELDS[:-1]:
        assert np.array_equal(b[n].reshape(-1), getattr(L, n).reshape(-1)), n


def test_two_calls_in_a_row_second_smaller():
    rng = np.random.default_rng(71)
    # 65536 pairs, 256 experts: two launches, a 128-chunk table
    check(8192, 8, 256, 8, rng.integers(0, 256, (8192, 8)).astype(np.int32))
    # 18000 pairs, 64 experts: two launches, a smaller table over the first
    # call's leftovers
    check(3000, 6, 64, 8, rng.integers(0, 64, (3000, 6)).astype(np.int32))
    # and a one-launch size (no table at all)
    check(100, 8, 288, 36, rng.integers(0, 288, (100, 8)).astype(np.int32))


def test_largest_table_and_skew():
    rng = np.random.default_rng(72)
    # E = 1984 at 2^20 pairs: the largest chunk table of any valid config
    T, k, E = 131072, 8, 1984
    z = rng.zipf(1.3, (T, k)) % E
    check(T, k, E, 8, z.astype(np.int32))


def test_bad_index_sets_the_error_word():
    rng = np.random.default_rng(73)
    T, k, E, R = 4096, 4, 128, 8
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[1234, 2] = E + 5
    a, b = both_layouts(T, k, E, R, idx)
    assert a["error_flag"][0] == ep.EP_DEVERR_INDEX
    assert b["error_flag"][0] == ep.EP_DEVERR_INDEX
    # the same handle reused with good indices: the word is cleared again
    idx[1234, 2] = 3
    check(T, k, E, R, idx)
