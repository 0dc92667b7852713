"""The README's Python example, run as written, then checked against the
oracle: the routing (indices and weight bits), the handle, the FP8 dispatch
(codes and scales) and the combine (1e-2 relative, bit mismatches reported)."""
import os
import re

import numpy as np
import pytest
import torch

import oracle

from gpu_util import rel_err, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def readme_example() -> str:
    text = open(os.path.join(ROOT, "README.md")).read()
    sec = text[text.index("## Example (Python)"):]
    m = re.search(r"```python\n(.*?)```", sec, re.S)
    assert m, "no python block under the example heading"
    return m.group(1)


def test_readme_example_runs_and_matches_the_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ns = {}
    exec(compile(readme_example(), "README.md example", "exec"), ns)
    T, k, E, R, H = ns["T"], ns["k"], ns["E"], ns["R"], ns["H"]
    say(f"README example T={T} H={H} k={k} E={E} R={R}")
    # routing
    z = ns["logits"].cpu().numpy()
    ri, rw = oracle.route(z, k, gate="sigmoid", n_groups=8, topk_groups=4)
    assert np.array_equal(ns["idx"].cpu().numpy(), ri)
    assert np.array_equal(ns["w"].cpu().numpy().view(np.uint32), rw.view(np.uint32))
    # handle
    L = oracle.layout(ri, E, R)
    h = ns["h"]
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "slot_of", "src_of"):
        assert np.array_equal(getattr(h, key).cpu().numpy().reshape(-1), getattr(L, key).reshape(-1)), key
    # FP8 dispatch
    xb = ns["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    rq, rs = oracle.dispatch_fp8(xb, ri, L)
    recv = ns["recv"]
    for r in range(R):
        n = int(L.rank_counts[r])
        assert np.array_equal(recv.x[r][:n].cpu().numpy(), rq[r]), r
        assert np.array_equal(recv.scales[r][:n].cpu().numpy().view(np.uint32), rs[r].view(np.uint32)), r
    # combine
    ys = [ns["y"][r][:int(L.rank_counts[r])].view(torch.int16).cpu().numpy().view(np.uint16) for r in range(R)]
    ref = oracle.combine(ys, ri, L, rw)
    got = ns["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    say(f"  combine max rel err {rel_err(got, ref):.3g}, bit mismatches {int(np.count_nonzero(got != ref))}")
    assert rel_err(got, ref) <= 1e-2
