"""CPU oracle for MoE token dispatch / combine -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does, and the two share no code.

The arithmetic lives in ``ep_oracle.c`` (plain C, single thread, built with
``gcc -O2 -ffp-contract=off``); this module only builds it, marshals numpy
arrays and slices the per-rank receive buffers.

Pages cited (title, section):
  [DeepEP overview]  "DeepSeek merilis library open source DeepEP untuk
                     pelatihan dan inferensi MoE", "Pola penggunaan ..."
  [Perplexity blog]  "Lower latency and higher throughput with multi-node
                     DeepSeek deployment", "Sérfræðinga-samsíðun",
                     "Magntölun", "MoE-beirari"
  [torchtitan PR]    "Integrate DeepEP to experimental torchtitan"

Parity pins: every function here is pinned by tests in ``tests/test_oracle_*``
against library special cases (numpy bincount / stable argsort, torch's
float8_e4m3fn and bfloat16 casts), brute force on tiny inputs, exact rational
arithmetic and the closed-form invariants of the method.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile ep_oracle.c into libep_oracle.so (gcc).  Returns the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC),
                                                os.path.getmtime(os.path.join(_HERE, "ep_oracle.h")))):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i32, vp = ctypes.c_int, ctypes.c_void_p
        L.oracle_validate.argtypes = [i32, i32, i32, i32, i32, i32, vp]
        L.oracle_validate.restype = i32
        L.oracle_layout.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_layout.restype = i32
        L.oracle_dispatch_bf16.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_dispatch_fp8.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_quantize_row.argtypes = [i32, vp, vp, vp]
        L.oracle_unpermute.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_combine.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_combine_shared.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_combine_backward.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_silu_mul_row.argtypes = [i32, vp, vp]
        L.oracle_silu_mul_quant_row.argtypes = [i32, vp, vp, vp]
        L.oracle_quantize_f32_row.argtypes = [i32, vp, vp, vp]
        L.oracle_route.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_route.restype = i32
        L.oracle_route_scores.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_route_scores.restype = i32
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        for name in ("oracle_e4m3_encode_n", "oracle_e4m3_decode_n", "oracle_bf16_rne_n"):
            getattr(L, name).argtypes = [vp, vp, ctypes.c_int64]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _ptr_array(arrs) -> ctypes.Array:
    return (ctypes.c_void_p * len(arrs))(*[_p(a) for a in arrs])


# ----------------------------------------------------------------- codecs
def e4m3_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_p(v), _p(out), v.size)
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().oracle_e4m3_decode_n(_p(c), _p(out), c.size)
    return out


def bf16_rne(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_rne_n(_p(v), _p(out), v.size)
    return out


def bf16_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- layout
@dataclass
class Layout:
    """The routing handle: per-expert / per-rank counts and offsets and the
    stable permutation ([DeepEP overview], "Pola penggunaan ...": the handle
    carries the routing metadata and the per-expert token counts)."""
    T: int
    k: int
    E: int
    R: int
    expert_counts: np.ndarray   # [E]
    expert_offsets: np.ndarray  # [E+1]
    rank_counts: np.ndarray     # [R]
    rank_offsets: np.ndarray    # [R+1]
    slot_of: np.ndarray         # [T*k]  pair -> global slot
    src_of: np.ndarray          # [T*k]  global slot -> pair
    row_of: np.ndarray          # [T*k]  pair -> row inside its rank buffer

    @property
    def rank_of(self) -> np.ndarray:
        """rank of each pair (only valid with the topk_idx that built it)."""
        return np.searchsorted(self.rank_offsets, self.slot_of, side="right") - 1


class OracleError(ValueError):
    pass


def validate(T, H, k, E, R, fp8, topk_idx) -> int:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    return lib().oracle_validate(T, H, k, E, R, int(bool(fp8)), _p(idx))


def layout(topk_idx: np.ndarray, E: int, R: int) -> Layout:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    P = T * k
    cnt = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    rcnt = np.empty(R, np.int32)
    roff = np.empty(R + 1, np.int32)
    slot = np.empty(P, np.int32)
    src = np.empty(P, np.int32)
    row = np.empty(P, np.int32)
    rc = lib().oracle_layout(T, k, E, R, _p(idx), _p(cnt), _p(off), _p(rcnt), _p(roff),
                             _p(slot), _p(src), _p(row))
    if rc:
        raise OracleError("oracle_layout rejected the input (code %d)" % rc)
    return Layout(T, k, E, R, cnt, off, rcnt, roff, slot, src, row)


# --------------------------------------------------------------- dispatch
def dispatch_bf16(x: np.ndarray, topk_idx: np.ndarray, L: Layout):
    """Returns R arrays [rank_counts[r], H] uint16 (bf16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, H = x.shape
    recv = [np.empty((int(L.rank_counts[r]), H), np.uint16) for r in range(L.R)]
    lib().oracle_dispatch_bf16(T, H, L.k, L.E, L.R, _p(idx), _p(L.slot_of), _p(L.rank_offsets),
                               _p(x), _ptr_array(recv))
    return recv


def quantize_rows(x: np.ndarray):
    """Per-token FP8 quantization (q [T,H] uint8, s [T,H/128] fp32)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // 128), np.float32)
    for t in range(T):
        lib().oracle_quantize_row(H, _p(x[t]), _p(q[t]), _p(s[t]))
    return q, s


def dispatch_fp8(x: np.ndarray, topk_idx: np.ndarray, L: Layout):
    """Returns (recv_q, recv_s): R arrays [rank_counts[r], H] uint8 and R
    arrays [rank_counts[r], H/128] float32."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, H = x.shape
    rq = [np.empty((int(L.rank_counts[r]), H), np.uint8) for r in range(L.R)]
    rs = [np.empty((int(L.rank_counts[r]), H // 128), np.float32) for r in range(L.R)]
    lib().oracle_dispatch_fp8(T, H, L.k, L.E, L.R, _p(idx), _p(L.slot_of), _p(L.rank_offsets),
                              _p(x), _ptr_array(rq), _ptr_array(rs))
    return rq, rs


# ------------------------------------------------------- unpermute/combine
def _rows_or_empty(recv_y, H):
    # ctypes needs a valid pointer even for zero-row buffers
    return [r if r.size else np.zeros((1, H), np.uint16) for r in recv_y]


def unpermute(recv_y, topk_idx: np.ndarray, L: Layout) -> np.ndarray:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    H = recv_y[0].shape[1]
    ys = [np.ascontiguousarray(r, dtype=np.uint16) for r in _rows_or_empty(recv_y, H)]
    u = np.empty((L.T * L.k, H), np.uint16)
    lib().oracle_unpermute(L.T, H, L.k, L.E, L.R, _p(idx), _p(L.slot_of), _p(L.rank_offsets),
                           _ptr_array(ys), _p(u))
    return u


def combine(recv_y, topk_idx: np.ndarray, L: Layout, weights=None) -> np.ndarray:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    H = recv_y[0].shape[1]
    ys = [np.ascontiguousarray(r, dtype=np.uint16) for r in _rows_or_empty(recv_y, H)]
    out = np.empty((L.T, H), np.uint16)
    if weights is None:
        wp = None
    else:
        w = np.ascontiguousarray(weights, dtype=np.float32)
        assert w.shape == (L.T, L.k)
        wp = _p(w)
    lib().oracle_combine(L.T, H, L.k, L.E, L.R, _p(idx), _p(L.slot_of), _p(L.rank_offsets),
                         _ptr_array(ys), wp, _p(out))
    return out


def _weights_or_none(weights):
    return None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)


def combine_shared(recv_y, topk_idx: np.ndarray, L: Layout, weights, shared: np.ndarray) -> np.ndarray:
    """Weighted combine with the shared expert's output added last (see
    ep_oracle.h)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    H = recv_y[0].shape[1]
    ys = [np.ascontiguousarray(r, dtype=np.uint16) for r in _rows_or_empty(recv_y, H)]
    sh = np.ascontiguousarray(shared, dtype=np.uint16)
    assert sh.shape == (L.T, H)
    w = _weights_or_none(weights)
    out = np.empty((L.T, H), np.uint16)
    lib().oracle_combine_shared(L.T, H, L.k, L.E, L.R, _p(idx), _p(L.slot_of), _p(L.rank_offsets),
                                _ptr_array(ys), None if w is None else _p(w), _p(sh), _p(out))
    return out


def combine_backward(grad_out: np.ndarray, topk_idx: np.ndarray, L: Layout, weights=None,
                     recv_y=None):
    """Backward of combine: (grad_recv, grad_w).  grad_recv is R arrays
    [rank_counts[r], H] uint16; grad_w is [T, k] float32, or None when
    recv_y is None."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    g = np.ascontiguousarray(grad_out, dtype=np.uint16)
    T, H = g.shape
    gr = [np.empty((int(L.rank_counts[r]), H), np.uint16) for r in range(L.R)]
    w = _weights_or_none(weights)
    ys = None if recv_y is None else [np.ascontiguousarray(r, dtype=np.uint16)
                                      for r in _rows_or_empty(recv_y, H)]
    gw = None if recv_y is None else np.empty((T, L.k), np.float32)
    lib().oracle_combine_backward(T, H, L.k, L.E, L.R, _p(idx), _p(L.slot_of), _p(L.rank_offsets),
                                  _p(g), None if w is None else _p(w),
                                  None if ys is None else _ptr_array(ys),
                                  _ptr_array(_rows_or_empty(gr, H)),
                                  None if gw is None else _p(gw))
    return gr, gw


def silu_mul(rows: np.ndarray) -> np.ndarray:
    """a = RN32(silu(gate) * up) per row of 2I bf16 values -> [n, I] float32."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    n, I2 = rows.shape
    a = np.empty((n, I2 // 2), np.float32)
    for i in range(n):
        lib().oracle_silu_mul_row(I2 // 2, _p(rows[i]), _p(a[i]))
    return a


def silu_mul_quant(rows: np.ndarray):
    """SiLU-and-multiply then per-128 FP8 quantization, per row of 2I bf16
    values -> (q [n, I] uint8, s [n, I/128] float32)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    n, I2 = rows.shape
    I = I2 // 2
    q = np.empty((n, I), np.uint8)
    s = np.empty((n, I // 128), np.float32)
    for i in range(n):
        lib().oracle_silu_mul_quant_row(I, _p(rows[i]), _p(q[i]), _p(s[i]))
    return q, s


def quantize_f32_rows(a: np.ndarray):
    a = np.ascontiguousarray(a, dtype=np.float32)
    n, I = a.shape
    q = np.empty((n, I), np.uint8)
    s = np.empty((n, I // 128), np.float32)
    for i in range(n):
        lib().oracle_quantize_f32_row(I, _p(a[i]), _p(q[i]), _p(s[i]))
    return q, s


def dequant_identity_expert(recv_q, recv_s):
    """The identity expert on FP8 rows: y = BF16_RNE(RN32(decode(q) * s)) per
    element -- the dequantized activation rounded once to binary32 (numpy
    float32 multiply) and once to bf16.  Returns R arrays [rank_counts[r], H]
    uint16.  This is a test stand-in for the experts, not part of the path."""
    out = []
    for q, s in zip(recv_q, recv_s):
        if q.shape[0] == 0:
            out.append(np.zeros((0, q.shape[1]), np.uint16))
            continue
        d = e4m3_decode(q)
        sc = np.repeat(s, 128, axis=1)
        prod = (d * sc).astype(np.float32)
        out.append(bf16_rne(prod))
    return out


# ----------------------------------------------------------------- router
GATES = {"softmax": 0, "sigmoid": 1}


def route_scores(logits: np.ndarray, gate: str = "sigmoid", bias=None) -> np.ndarray:
    """The router's gate scores (oracle_route_scores): [T, El] float32, the
    binary64 gate of logit + bias rounded once to binary32."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, El = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, El), np.float32)
    rc = lib().oracle_route_scores(T, El, GATES[gate], _p(logits), None if b is None else _p(b),
                                   _p(out))
    if rc:
        raise OracleError("router parameters rejected (code %d)" % rc)
    return out


def route(logits: np.ndarray, k: int, gate: str = "sigmoid", n_groups: int = 1,
          topk_groups: int = 1, group_topn: int = 2, renorm: bool = True, bias=None,
          rep_offsets=None, rep_slots=None):
    """Group-limited top-k router (oracle_route) -> (topk_idx [T,k] int32,
    topk_weights [T,k] float32).  logits [T, El] float32; bias [El] float32 or
    None; rep_offsets [El+1] / rep_slots int32 (redundant experts) or None."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, El = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ro = None if rep_offsets is None else np.ascontiguousarray(rep_offsets, dtype=np.int32)
    rs = None if rep_slots is None else np.ascontiguousarray(rep_slots, dtype=np.int32)
    if b is not None:
        assert b.shape == (El,)
    if ro is not None:
        assert ro.shape == (El + 1,) and rs is not None and rs.size >= int(ro[-1])
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib().oracle_route(T, El, k, GATES[gate], n_groups, topk_groups, group_topn, int(renorm),
                            _p(logits), None if b is None else _p(b),
                            None if ro is None else _p(ro), None if rs is None else _p(rs),
                            _p(idx), _p(w))
    if rc:
        raise OracleError("router parameters rejected (code %d)" % rc)
    return idx, w
