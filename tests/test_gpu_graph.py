"""Every entry point captured in a HIP graph: one MoE-layer step from the
router logits -- ep_route_layout, ep_dispatch, ep_silu_mul_quant,
ep_combine_shared, ep_combine_backward -- and the decode form -- ep_route,
ep_layout_dispatch, ep_combine -- each captured once and replayed several
times with eager work (output poisoning, synchronization) between replays;
every replay must reproduce the eager run's bytes exactly.  The workloads
take the one-launch layout (decode), the two-launch layout with FP8 (a
2048-token V3-shaped batch) and BF16 (DeepSeek-16B-like), and both
combine-backward paths.  The same steps of three workloads also run at the
same time on three streams and must give the bytes of a sequential run.
"""
import numpy as np
import pytest
import torch

import combine_ep_layout_03_amd as ep
from combine_ep_layout_03_amd.buffers import Handle, RecvBuffers, alloc_workspace
from workloads import make_workload

from gpu_util import POISON, say, to_dev

pytestmark = pytest.mark.gpu

INTER = 512  # expert intermediate size of the SiLU stage in these tests


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load()


class Step:
    """Device buffers of one MoE-layer step on a workload."""

    def __init__(self, w):
        self.w = w
        self.cfg = ep.Config(w.T, w.H, w.k, w.E, w.R, fp8=w.fp8)
        self.cap = ep.ep_recv_capacity_rows(self.cfg)
        rin = w.extra
        self.router = ep.Router(rin["logits"].shape[1], **rin["router"])
        opt = lambda key: to_dev(rin[key]) if key in rin else None
        self.logits, self.bias = to_dev(rin["logits"]), opt("bias")
        self.ro, self.rs = opt("rep_offsets"), opt("rep_slots")
        self.x = to_dev(w.x)
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        rnd = lambda *shape: torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
        self.idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
        self.wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
        self.h = Handle.alloc(self.cfg, "cuda")
        self.ws = alloc_workspace(self.cfg, "cuda")
        self.recv = RecvBuffers.alloc(self.cfg, self.cap, device="cuda", fill=POISON)
        self.act = [rnd(self.cap, 2 * INTER) for _ in range(w.R)]
        self.q = [torch.empty((self.cap, INTER), dtype=torch.uint8, device="cuda") for _ in range(w.R)]
        self.qs = [torch.empty((self.cap, INTER // 128), dtype=torch.float32, device="cuda")
                   for _ in range(w.R)]
        self.y = [rnd(self.cap, w.H) for _ in range(w.R)]
        self.shared = rnd(w.T, w.H)
        self.gout = rnd(w.T, w.H)
        self.out = torch.empty((w.T, w.H), dtype=torch.int16, device="cuda")
        self.grows = [torch.empty((self.cap, w.H), dtype=torch.int16, device="cuda") for _ in range(w.R)]
        self.gw = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")

    def fixed_outputs(self):
        return [self.idx, self.wts, self.out, self.gw] + list(vars(self.h).values())

    def rank_outputs(self):
        return self.recv.x + (self.recv.scales or []) + self.q + self.qs + self.grows

    def poison(self):
        for t in self.fixed_outputs() + self.rank_outputs():
            t.view(torch.uint8).fill_(POISON)

    def snapshot(self):
        """Every byte of the fixed-size outputs and the valid rows of the
        per-rank buffers (rows past rank_counts are never written)."""
        torch.cuda.synchronize()
        counts = self.h.rank_counts.cpu().numpy()
        snap = [t.cpu().numpy().view(np.uint8) for t in self.fixed_outputs()]
        R = self.w.R
        for i, t in enumerate(self.rank_outputs()):
            snap.append(t[:int(counts[i % R])].cpu().numpy().view(np.uint8))
        return snap, counts

    def layer(self, stream):
        c = self
        ep.ep_route_layout(c.cfg, c.router, c.logits, c.bias, c.ro, c.rs, c.idx, c.wts, c.h, c.ws, stream=stream)
        ep.ep_dispatch(c.cfg, c.h, c.idx, c.x, c.recv.x, c.recv.scales, c.cap, stream=stream)
        ep.ep_silu_mul_quant(c.cfg, c.h, INTER, c.act, c.q, c.qs, c.cap, stream=stream)
        ep.ep_combine_shared(c.cfg, c.h, c.idx, c.y, c.wts, c.shared, c.out, c.cap, stream=stream)
        ep.ep_combine_backward(c.cfg, c.h, c.idx, c.gout, c.wts, c.y, c.grows, c.gw, c.cap, stream=stream)

    def decode(self, stream):
        c = self
        ep.ep_route(c.cfg, c.router, c.logits, c.bias, c.ro, c.rs, c.idx, c.wts, stream=stream)
        ep.ep_layout_dispatch(c.cfg, c.idx, c.h, c.ws, c.x, c.recv.x, c.recv.scales, c.cap, stream=stream)
        ep.ep_combine(c.cfg, c.h, c.idx, c.y, c.wts, c.out, c.cap, stream=stream)


def run_graph(step, body, replays=4):
    cur = torch.cuda.current_stream()
    step.poison()
    body(step, cur)
    eager, counts = step.snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            body(step, s)
    cur.wait_stream(s)
    torch.cuda.synchronize()
    assert int(step.h.error_flag.item()) == 0
    for rep in range(replays):
        step.poison()                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got, n2 = step.snapshot()
        assert np.array_equal(n2, counts), rep
        for i, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a, b), (rep, i)


@pytest.mark.parametrize("name,T", [("decode", None), ("v3", 2048), ("ds16b", 1024), ("v3_skew", 3000)])
def test_layer_step_in_a_graph(name, T):
    w = make_workload(name, T=T)
    say(f"graph: layer step {name} T={w.T} P={w.P}")
    run_graph(Step(w), Step.layer)


@pytest.mark.parametrize("name,T", [("decode", None), ("decode", 200), ("tiny", None)])
def test_decode_step_in_a_graph(name, T):
    w = make_workload(name, T=T)
    say(f"graph: decode step {name} T={w.T} P={w.P}")
    run_graph(Step(w), Step.decode)


@pytest.mark.parametrize("body", ["layer", "decode"])
def test_independent_calls_on_concurrent_streams(body):
    """The library keeps no state between calls: three workloads' steps run
    at the same time on three streams (default priority) give the bytes of
    the same steps run one after another."""
    steps = [Step(make_workload("decode")), Step(make_workload("v3", T=2048)),
             Step(make_workload("ds16b", T=1024))]
    fn = getattr(Step, body)
    cur = torch.cuda.current_stream()
    ref = []
    for st in steps:
        st.poison()
        fn(st, cur)
        ref.append(st.snapshot())
    say(f"concurrent streams: {body} x {len(steps)}")
    for rep in range(3):
        for st in steps:
            st.poison()
        streams = [torch.cuda.Stream() for _ in steps]
        for st, s in zip(steps, streams):
            s.wait_stream(cur)
            with torch.cuda.stream(s):
                fn(st, s)
        for s in streams:
            cur.wait_stream(s)
        torch.cuda.synchronize()
        for i, st in enumerate(steps):
            got, counts = st.snapshot()
            assert np.array_equal(counts, ref[i][1]), (rep, i)
            for j, (a, b) in enumerate(zip(got, ref[i][0])):
                assert np.array_equal(a, b), (rep, i, j)
