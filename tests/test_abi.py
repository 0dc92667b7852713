"""CPU-side checks of the C ABI: libep.so loads, exports every function that
include/ep.h declares, and its host-only calls (size helpers, status text,
argument validation) behave as documented.  No kernel is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_ep_layout_03_amd as ep
from combine_ep_layout_03_amd import _lib, build as epbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


@pytest.fixture(scope="module")
def lib():
    if epbuild.is_stale():
        epbuild.build()
    return ep.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][A-Za-z0-9_ \*]*?\b(ep_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ep_[a-z_]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (EP_[A-Z0-9_]+) (\d+)u?\b", text))
    for name in ("EP_OK", "EP_ERR_INVALID_ARG", "EP_ERR_UNSUPPORTED", "EP_ERR_CAPACITY",
                 "EP_ERR_HIP", "EP_DEVERR_INDEX", "EP_DEVERR_ROW", "EP_DEVERR_INTERNAL", "EP_DTYPE_BF16",
                 "EP_DTYPE_FP8_E4M3", "EP_MAX_RANKS", "EP_MAX_TOPK", "EP_MAX_EXPERTS",
                 "EP_MAX_HIDDEN", "EP_MAX_GROUPS", "EP_GATE_SOFTMAX", "EP_GATE_SIGMOID"):
        assert int(consts[name]) == getattr(_lib, name), name
    assert int(consts["EP_ABI_VERSION"]) == ep.ep_abi_version()
    # struct layouts: 7 int32 fields, 7 pointers
    assert ctypes.sizeof(_lib.ep_config) == 28
    assert ctypes.sizeof(_lib.ep_layout_t) == 56
    assert ctypes.sizeof(_lib.ep_router_t) == 24


def test_status_strings(lib):
    for s in range(5):
        assert ep.ep_status_string(s)
    assert ep.ep_status_string(99) == "unknown status"


def test_capacity_and_workspace(lib):
    c = ep.Config(8192, 7168, 8, 256, 8, fp8=True)
    assert ep.ep_recv_capacity_rows(c) == 8192 * 8
    # ep_layout: 128 chunks of 512 pairs; ep_route_layout's router-counted
    # table: one chunk per router workgroup of 32 tokens, 256 chunks -- the
    # larger one is returned
    assert ep.ep_layout_workspace_bytes(c) == 256 * 257 * 4
    # 20000 tokens, k=3, E=512: the router-counted table has 3 router steps
    # (96 tokens) per chunk, 209 chunks, padded to 212 columns
    c = ep.Config(20000, 256, 3, 512, 8)
    assert ep.ep_layout_workspace_bytes(c) == 212 * 513 * 4
    # up to 8192 pairs and 512 experts the layout is one launch: no table
    c = ep.Config(128, 7168, 8, 288, 36, fp8=True)
    assert ep.ep_layout_workspace_bytes(c) == 256
    c = ep.Config(30000, 7168, 8, 256, 8)  # 240000 pairs: chunks grow to 960 pairs so C <= 255
    assert ep.ep_layout_workspace_bytes(c) == 252 * 257 * 4  # 250 chunks in groups of 4
    # (the router-counted table: 128-token chunks, 235 of them -> 236 columns, smaller)
    # many pairs, many experts: the chunk count is capped so the table stays small
    c = ep.Config(1 << 20, 256, 8, 2048, 8)
    ws = ep.ep_layout_workspace_bytes(c)
    assert ws <= 65536 * 4 + 2049 * 4 * 4 and ws % (2049 * 4) == 0


@pytest.mark.parametrize("bad", [
    dict(num_tokens=0), dict(hidden=7), dict(hidden=100, fp8=True), dict(num_topk=0),
    dict(num_topk=33), dict(num_experts=255), dict(num_ranks=65, num_experts=65 * 4),
    dict(num_experts=4096, num_ranks=8), dict(num_workgroups=-1), dict(hidden=65544),
])
def test_invalid_configs_rejected(lib, bad):
    base = dict(num_tokens=16, hidden=256, num_topk=2, num_experts=16, num_ranks=4, fp8=False)
    base.update(bad)
    c = ep.Config(**base)
    assert ep.ep_recv_capacity_rows(c) == -1
    assert ep.ep_layout_workspace_bytes(c) == 0
    with pytest.raises(ep.EpError) as ei:
        ep.ep_layout(c, 1, _lib.ep_layout_t(*([8] * 7)), 8, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG


def test_null_pointers_and_capacity_rejected_before_any_launch(lib):
    c = ep.Config(16, 256, 2, 16, 4)
    h = _lib.ep_layout_t(*([8] * 7))
    hnull = _lib.ep_layout_t(*([8] * 6 + [None]))
    with pytest.raises(ep.EpError) as ei:
        ep.ep_layout(c, None, h, 8, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:
        ep.ep_layout(c, 8, hnull, 8, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:
        ep.ep_layout(c, 8, h, None, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    for call in (lambda: ep.ep_layout(c, 8, h, 4100, 0),     # workspace not 16-byte aligned
                 lambda: ep.ep_layout_dispatch(c, 8, h, 4100, 8, [8] * 4, None, 32, 0),
                 lambda: ep.ep_route_layout(c, ep.Router(16), 8, None, None, None, 8, 8, h, 4100, 0)):
        with pytest.raises(ep.EpError) as ei:
            call()
        assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:
        ep.ep_dispatch(c, h, 8, 8, [8] * 4, None, 31, 0)
    assert ei.value.status == ep.EP_ERR_CAPACITY
    with pytest.raises(ep.EpError) as ei:
        ep.ep_dispatch(c, h, 8, 8, [8, 8, None, 8], None, 32, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    cf = ep.Config(16, 256, 2, 16, 4, fp8=True)
    with pytest.raises(ep.EpError) as ei:
        ep.ep_dispatch(cf, h, 8, 8, [8] * 4, None, 32, 0)   # FP8 needs scale buffers
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:
        ep.ep_combine(c, h, 8, [8] * 4, None, None, 32, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:
        ep.ep_combine(c, h, 8, [8] * 4, None, 8, 10, 0)
    assert ei.value.status == ep.EP_ERR_CAPACITY
    with pytest.raises(ep.EpError) as ei:
        ep.ep_unpermute(c, h, 8, [8, None, 8, 8], 8, 32, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG


@pytest.mark.parametrize("bad_router,bad_cfg,replicas", [
    (dict(num_logical=0), {}, False), (dict(num_logical=4096), {}, False),
    (dict(gate=2), {}, False), (dict(num_groups=3), {}, False),
    (dict(num_groups=128, num_logical=256), dict(num_experts=256), False),
    (dict(num_groups=4, topk_groups=0), {}, False), (dict(num_groups=4, topk_groups=5), {}, False),
    (dict(group_topn=0), {}, False), (dict(group_topn=3), {}, False),
    (dict(num_groups=8, topk_groups=1), dict(num_topk=3), False),  # k > TG * El/G = 2
    (dict(num_logical=8), {}, False),                              # E != El without replicas
    (dict(), dict(num_topk=17, num_experts=32), True),             # k > El
])
def test_router_parameters_rejected(lib, bad_router, bad_cfg, replicas):
    base = dict(num_tokens=16, hidden=256, num_topk=2, num_experts=16, num_ranks=4)
    base.update(bad_cfg)
    c = ep.Config(**base)
    r = dict(num_logical=16, gate=1, num_groups=1, topk_groups=1, group_topn=2, renormalize=1)
    r.update(bad_router)
    rt = _lib.ep_router_t(*r.values())
    rep = (8, 8) if replicas else (None, None)
    with pytest.raises(ep.EpError) as ei:
        ep.ep_route(c, rt, 8, None, rep[0], rep[1], 8, 8, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:
        ep.ep_route_layout(c, rt, 8, None, rep[0], rep[1], 8, 8, _lib.ep_layout_t(*([8] * 7)), 8, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG


def test_router_null_pointers_rejected(lib):
    c = ep.Config(16, 256, 2, 16, 4)
    rt = ep.Router(16).c()
    for args in [(None, None, None, None, 8, 8), (8, None, None, None, None, 8),
                 (8, None, None, None, 8, None), (8, None, 8, None, 8, 8),
                 (8, None, None, 8, 8, 8)]:
        with pytest.raises(ep.EpError) as ei:
            ep.ep_route(c, rt, *args, 0)
        assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:   # handle with a NULL array
        ep.ep_route_layout(c, rt, 8, None, None, None, 8, 8, _lib.ep_layout_t(*([8] * 6 + [None])), 8, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError) as ei:   # no workspace
        ep.ep_route_layout(c, rt, 8, None, None, None, 8, 8, _lib.ep_layout_t(*([8] * 7)), None, 0)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(tmp_path):
    missing = str(tmp_path / "libep.so")
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            _lib.load(missing)
    finally:
        _lib._lib = saved


def test_header_is_plain_c():
    """include/ep.h is a C header: the C example compiles as C11 with every
    warning an error (syntax only: no library or GPU needed)."""
    import shutil
    gcc = shutil.which("gcc")
    rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    if not gcc or not os.path.isdir(rocm_inc):
        pytest.skip("gcc or the HIP headers are not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([gcc, "-std=c11", "-fsyntax-only", "-Wall", "-Wextra", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"), "-I", rocm_inc,
                        os.path.join(root, "examples", "ep_c_example.c")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


A, M = 4096, 4104   # fake device addresses: 16-byte aligned, and 8- but not 16-byte aligned


def _misaligned_cases():
    c = ep.Config(16, 256, 2, 16, 4)
    cf = ep.Config(16, 256, 2, 16, 4, fp8=True)
    h = _lib.ep_layout_t(*([A] * 7))
    R, cap = 4, 32

    def rows(bad=None):
        return [M if r == bad else A for r in range(R)]

    return {
        "dispatch x": lambda: ep.ep_dispatch(c, h, A, M, rows(), None, cap, 0),
        "dispatch recv_x": lambda: ep.ep_dispatch(c, h, A, A, rows(2), None, cap, 0),
        "dispatch recv_scales": lambda: ep.ep_dispatch(cf, h, A, A, rows(), rows(1), cap, 0),
        "layout_dispatch x": lambda: ep.ep_layout_dispatch(cf, A, h, A, M, rows(), rows(), cap, 0),
        "layout_dispatch recv_x": lambda: ep.ep_layout_dispatch(cf, A, h, A, A, rows(0), rows(), cap, 0),
        "combine out": lambda: ep.ep_combine(c, h, A, rows(), A, M, cap, 0),
        "combine recv_y": lambda: ep.ep_combine(c, h, A, rows(3), A, A, cap, 0),
        "combine_shared shared": lambda: ep.ep_combine_shared(c, h, A, rows(), A, M, A, cap, 0),
        "combine_shared out": lambda: ep.ep_combine_shared(c, h, A, rows(), A, A, M, cap, 0),
        "combine_backward grad_out": lambda: ep.ep_combine_backward(c, h, A, M, A, rows(), rows(), A,
                                                                   cap, 0),
        "combine_backward grad_recv": lambda: ep.ep_combine_backward(c, h, A, A, A, rows(), rows(0), A,
                                                                    cap, 0),
        "combine_backward recv_y": lambda: ep.ep_combine_backward(c, h, A, A, A, rows(1), rows(), A,
                                                                 cap, 0),
        "silu act_in": lambda: ep.ep_silu_mul_quant(c, h, 128, rows(2), rows(), rows(), cap, 0),
        "silu q_out": lambda: ep.ep_silu_mul_quant(c, h, 128, rows(), rows(0), rows(), cap, 0),
        "silu scales_out": lambda: ep.ep_silu_mul_quant(c, h, 128, rows(), rows(), rows(3), cap, 0),
        "unpermute out": lambda: ep.ep_unpermute(c, h, A, rows(), M, cap, 0),
        "unpermute recv_y": lambda: ep.ep_unpermute(c, h, A, rows(0), A, cap, 0),
    }


@pytest.mark.parametrize("case", sorted(_misaligned_cases()))
def test_row_buffers_must_be_16_byte_aligned(lib, case):
    """Every row buffer is moved with 16-byte vector loads and stores, so a
    pointer that is not 16-byte aligned is rejected on the host (nothing is
    launched: exactly one argument of each call is bad)."""
    with pytest.raises(ep.EpError) as ei:
        _misaligned_cases()[case]()
    assert ei.value.status == ep.EP_ERR_INVALID_ARG


def test_binding_checks_tensor_sizes():
    """The binding rejects a tensor smaller than the rows the call addresses
    (CPU tensors suffice: the check runs before any pointer is taken)."""
    import torch
    c = ep.Config(16, 256, 2, 16, 4, fp8=True)
    h = _lib.ep_layout_t(*([A] * 7))
    small = torch.empty(10, dtype=torch.uint8)
    with pytest.raises(ValueError, match="x holds"):
        ep.ep_dispatch(c, h, A, small, [A] * 4, [A] * 4, 32, 0)
    with pytest.raises(ValueError, match=r"recv_x\[1\]"):
        ep.ep_dispatch(c, h, A, A, [A, small, A, A], [A] * 4, 32, 0)
    with pytest.raises(ValueError, match=r"recv_scales\[0\]"):
        ep.ep_dispatch(c, h, A, A, [A] * 4, [small, A, A, A], 32, 0)
    with pytest.raises(ValueError, match="out holds"):
        ep.ep_combine(c, h, A, [A] * 4, None, small, 32, 0)
    with pytest.raises(ValueError, match=r"grad_recv\[3\]"):
        ep.ep_combine_backward(c, h, A, A, None, None, [A, A, A, small], None, 32, 0)
    with pytest.raises(ValueError, match=r"q_out\[2\]"):
        ep.ep_silu_mul_quant(c, h, 128, [A] * 4, [A, A, small, A], [A] * 4, 32, 0)


def test_layout_noalloc_rejects_before_any_launch(lib):
    c = ep.Config(16, 256, 2, 16, 4)
    h = _lib.ep_layout_t(*([A] * 7))
    for call in (lambda: ep.ep_layout_noalloc(c, None, h, 0),
                 lambda: ep.ep_layout_noalloc(c, A, _lib.ep_layout_t(*([A] * 6 + [None])), 0),
                 lambda: ep.ep_layout_noalloc(ep.Config(16, 256, 2, 15, 4), A, h, 0)):
        with pytest.raises(ep.EpError) as ei:
            call()
        assert ei.value.status == ep.EP_ERR_INVALID_ARG
