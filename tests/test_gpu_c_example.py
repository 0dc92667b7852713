"""The plain-C example (examples/ep_c_example.c, built by
combine_ep_layout_03_amd/build.py beside libep.so) run as a child process:
the C ABI used with no Python and no torch.  It checks layout counts against
a host histogram and that a BF16 dispatch followed by an identity-expert
combine returns every input row bit for bit; exit status 0 means all held."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "examples", "ep_c_example")

pytestmark = pytest.mark.gpu


def test_c_example_runs_through_the_c_abi():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "examples/ep_c_example is not built (combine_ep_layout_03_amd/build.py)"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith(": ok"), r.stdout
