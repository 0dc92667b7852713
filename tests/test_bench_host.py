"""Host-side checks of bench.py: its algorithmic byte model (the bytes the
method must move per call, which every GB/s figure divides by), its
one-GPU guard and its handling of a failing secondary figure.  No GPU is
used.

The byte model counts, per token, the reads of x and the indices and the
writes of the k rows (and, for FP8, their per-128-channel scales) for
dispatch, and the reads of the k expert rows, the weights and indices and
the write of the output row for combine ([DeepEP overview] "DeepSeek merilis
library open source DeepEP ...", "Hasil pengukuran performa": the V3 config,
FP8 dispatch and BF16 combine; [Perplexity blog] "Lower latency and higher
throughput with multi-node DeepSeek deployment", "Magntölun": one fp32 scale
per 128 channels)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


# per call: (T, H, k, E, R, fp8) -> dispatch bytes, combine bytes, as tabulated
# for the five workloads
TABLE = {
    "tiny": ((128, 256, 2, 16, 4, False), 198_656, 199_680),
    "ds16b": ((4096, 2048, 6, 64, 8, False), 117_637_120, 117_735_424),
    "v3": ((8192, 7168, 8, 256, 8, True), 602_406_912, 1_057_751_040),
    "v3_skew": ((8192, 7168, 8, 256, 8, True), 602_406_912, 1_057_751_040),
    "decode": ((128, 7168, 8, 288, 36, True), 9_412_608, 16_527_360),
}


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_bytes_match_the_table(name):
    cfg, dispatch, combine = TABLE[name]
    b = bench.algorithmic_bytes(*cfg)
    assert b["dispatch"] == dispatch and b["combine"] == combine


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_bytes_per_token(name):
    """The same bytes built token by token: dispatch reads a 2H-byte row and
    writes k rows of H codes + H/128 fp32 scales (FP8) or of 2H bytes (BF16),
    plus the k index and k slot words; combine reads k 2H-byte rows and the
    k weights, indices and slots, and writes one 2H-byte row."""
    (T, H, k, E, R, fp8), _, _ = TABLE[name]
    row_out = (H + 4 * (H // 128)) if fp8 else 2 * H
    per_tok_d = 2 * H + k * row_out + 4 * k + 4 * k
    per_tok_c = k * 2 * H + 4 * k * 3 + 2 * H
    b = bench.algorithmic_bytes(T, H, k, E, R, fp8)
    assert b["dispatch"] == T * per_tok_d
    assert b["combine"] == T * per_tok_c
    # the headline's 60 % bar: dispatch + combine within 345.9 us at 8 TB/s
    if name == "v3":
        assert (b["dispatch"] + b["combine"]) / (0.6 * 8e12) * 1e6 == pytest.approx(345.87, abs=0.01)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_a_failing_secondary_figure_does_not_cost_the_line(capsys):
    assert bench.guarded("ok", lambda: {"us": 1.0}) == {"us": 1.0}

    def boom():
        raise RuntimeError("no such kernel")

    got = bench.guarded("configs.tiny", boom)
    assert set(got) == {"error"} and "no such kernel" in got["error"]
    assert "configs.tiny failed" in capsys.readouterr().err


def test_kernel_keys_name_every_kernel():
    """The profile summaries find kernels by the KERNEL_KEYS patterns, applied
    to the names the kernel trace prints (namespace::name<template args>(...)).
    Every __global__ kernel of the HIP sources but the debug un-permute must
    match one pattern, in each template form it is launched with, so a
    renamed or new kernel cannot drop out of profiles/ unnoticed; and every
    pattern must match some kernel."""
    import glob
    import re
    csrc = os.path.join(ROOT, "combine_ep_layout_03_amd", "csrc")
    src = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(csrc, "*.hip"))))
    kernels = {}
    decl = r"(template\s*<([^>]*)>\s*)?__global__\s+__launch_bounds__\([^)]*\)\s+void\s+(\w+)\s*\("
    for m in re.finditer(decl, src):
        params = m.group(2)
        if params is None:
            forms = [""]
        else:
            # one instance per template form the launchers use
            n = params.count(",") + 1
            if n == 1 and "bool" in params:
                forms = ["<true>", "<false>"]
            elif n == 1:
                forms = ["<4>", "<16>"]
            else:
                forms = ["<16, true>", "<16, false>"]
        kernels[m.group(3)] = forms
    assert len(kernels) >= 15, sorted(kernels)
    keys = list(bench.KERNEL_KEYS.values())
    for name, forms in kernels.items():
        if name == "unpermute_kernel":
            continue
        for f in forms:
            printed = f"ep::(anonymous namespace)::{name}{f}(int const*, int)"
            assert any(re.search(k, printed) for k in keys), printed
    for k in keys:
        assert any(re.search(k, f"ep::(anonymous namespace)::{n}{f}(int const*)")
                   for n, forms in kernels.items() for f in forms), k
