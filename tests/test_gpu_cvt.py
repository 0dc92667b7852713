"""The hardware FP8 conversion the quantizers use (ep::dev::e4m3_pack4,
gfx950's packed binary32 -> OCP E4M3 convert) against the oracle's E4M3
encoder, code for code ([Perplexity blog] "Lower latency and higher throughput
with multi-node DeepSeek deployment", "Magntölun": 128-element blocks scaled
by amax and stored as FP8).

Both quantizers (dispatch's x/s and the SiLU re-quantization's a*(1/s)) feed
binary32 quotients with |q| <= 448 * (1 + 2^-23) to that conversion, so the
encoder must equal the oracle's nearest-even, saturating E4M3 on every
binary32 value of that range.  Swept here, both signs:
  * every binary32 value within 2^12 ulps of each E4M3 value and of each
    midpoint between neighbouring E4M3 values (the rounding boundaries),
    including zero, the subnormal / normal boundary 2^-6 and the saturation
    boundary between 448 and 464, clipped to |v| <= 450;
  * every 257th binary32 bit pattern from +0 to 450.
The kernel is tests/hip/cvt_e4m3.hip, built with the library (build()).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_03_amd import build as epbuild

from gpu_util import say

pytestmark = pytest.mark.gpu

NEAR = 1 << 12
LIMIT = np.float32(450.0)


def sweep_values() -> np.ndarray:
    lim_bits = int(LIMIT.view(np.int32))
    codes = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)  # +0 .. 448
    mids = (codes[:-1] + codes[1:]) / 2.0            # exact in binary32 (<= 4 significant bits)
    centres = np.concatenate([codes, mids, [464.0]]).astype(np.float32).view(np.int32).astype(np.int64)
    near = (centres[:, None] + np.arange(-NEAR, NEAR + 1)[None, :]).ravel()
    strided = np.arange(0, lim_bits + 1, 257, dtype=np.int64)
    bits = np.unique(np.concatenate([near, strided, [lim_bits]]))
    bits = bits[(bits >= 0) & (bits <= lim_bits)]
    pos = bits.astype(np.int32).view(np.float32)
    v = np.concatenate([pos, -pos])
    pad = (-len(v)) % 4
    return np.concatenate([v, np.zeros(pad, np.float32)])


@pytest.fixture(scope="module")
def cvt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    path = epbuild.test_kernel_path("cvt_e4m3")
    assert os.path.exists(path), "tests/hip/libcvt_e4m3.so is not built: run __graft_entry__.build()"
    L = ctypes.CDLL(path)
    L.cvt_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    L.cvt_e4m3.restype = ctypes.c_int
    return L


def test_hardware_e4m3_equals_the_oracle_encoder(cvt):
    v = sweep_values()
    assert np.all(np.abs(v) <= LIMIT)
    say(f"cvt sweep: {v.size} binary32 values")
    dv = torch.from_numpy(v).cuda()
    out = torch.full((v.size,), 0xAA, dtype=torch.uint8, device="cuda")
    st = cvt.cvt_e4m3(dv.data_ptr(), out.data_ptr(), v.size, torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.e4m3_encode(v)
    bad = np.nonzero(got != ref)[0]
    say(f"  {bad.size} mismatches")
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]
    # the sweep reaches every code: each finite E4M3 code is produced, saturation included
    assert set(np.unique(got).tolist()) == set(range(256)) - {0x7F, 0xFF}
    assert np.all(got[np.abs(v) > 448] & 0x7F == 0x7E)
