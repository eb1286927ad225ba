"""CPU oracle for the H-BitLinear forward pass -- TEST INFRASTRUCTURE ONLY.

A ctypes view of ``bitnet_oracle.c`` (plain C, built with gcc -O2 -ffp-contract=off).
Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product library (``ternary_weight_bit_bitlinear_amd``) never
imports it, and it imports nothing of the product.

Each wrapper takes and returns numpy arrays; the passage of the source pages that each
function follows is cited in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitnet_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_bitnet.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_bitnet.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        F = ctypes.c_float
        L.bitnet_ref_encode5.argtypes = [P]; L.bitnet_ref_encode5.restype = I
        L.bitnet_ref_decode5.argtypes = [I, P]; L.bitnet_ref_decode5.restype = I
        L.bitnet_ref_absmean.argtypes = [P, I64]; L.bitnet_ref_absmean.restype = F
        L.bitnet_ref_ternarize.argtypes = [P, I, I, P, P]; L.bitnet_ref_ternarize.restype = None
        L.bitnet_ref_row_bytes.argtypes = [I]; L.bitnet_ref_row_bytes.restype = I64
        L.bitnet_ref_packed_bytes.argtypes = [I, I]; L.bitnet_ref_packed_bytes.restype = I64
        L.bitnet_ref_pack.argtypes = [P, I, I, P]; L.bitnet_ref_pack.restype = None
        L.bitnet_ref_unpack.argtypes = [P, I, I, P]; L.bitnet_ref_unpack.restype = I
        L.bitnet_ref_fwht.argtypes = [P, I]; L.bitnet_ref_fwht.restype = None
        L.bitnet_ref_fwht_f64.argtypes = [P, I]; L.bitnet_ref_fwht_f64.restype = None
        L.bitnet_ref_hadamard_scale.argtypes = [I]; L.bitnet_ref_hadamard_scale.restype = F
        L.bitnet_ref_hadamard.argtypes = [P, I]; L.bitnet_ref_hadamard.restype = None
        L.bitnet_ref_quantize_row.argtypes = [P, I, I, P, P]
        L.bitnet_ref_quantize_row.restype = None
        L.bitnet_ref_pack_int4.argtypes = [P, I64, P]; L.bitnet_ref_pack_int4.restype = None
        L.bitnet_ref_unpack_int4.argtypes = [P, I64, P]; L.bitnet_ref_unpack_int4.restype = None
        L.bitnet_ref_quantize.argtypes = [P, I, I, I, I, P, P, P]
        L.bitnet_ref_quantize.restype = None
        L.bitnet_ref_gemm.argtypes = [P, P, I, I, I, P]; L.bitnet_ref_gemm.restype = None
        L.bitnet_ref_epilogue.argtypes = [P, P, F, I, I, P]; L.bitnet_ref_epilogue.restype = None
        L.bitnet_ref_forward.argtypes = [P, I, I, I, I, I, P, F, P]
        L.bitnet_ref_forward.restype = I
        L.bitnet_ref_rotate_weights.argtypes = [P, I, I, P]; L.bitnet_ref_rotate_weights.restype = None
        L.bitnet_ref_pack_weights_hadamard.argtypes = [P, I, I, P, P]
        L.bitnet_ref_pack_weights_hadamard.restype = None
        L.bitnet_ref_rms_scale.argtypes = [P, I, F]; L.bitnet_ref_rms_scale.restype = F
        L.bitnet_ref_rmsnorm.argtypes = [P, I, I, P, F, P]; L.bitnet_ref_rmsnorm.restype = None
        L.bitnet_ref_forward_rmsnorm.argtypes = [P, I, I, I, P, F, I, I, P, F, P]
        L.bitnet_ref_forward_rmsnorm.restype = I
        L.bitnet_ref_forward_segments.argtypes = [P, I, I, I, P, I, I, P, P, P]
        L.bitnet_ref_forward_segments.restype = I
        L.bitnet_ref_silu.argtypes = [F]; L.bitnet_ref_silu.restype = F
        L.bitnet_ref_swiglu.argtypes = [P, P, I64, P]; L.bitnet_ref_swiglu.restype = None
        L.bitnet_ref_forward_swiglu.argtypes = [P, I, I, I, I, I, P, F, P, F, P]
        L.bitnet_ref_forward_swiglu.restype = I
        L.bitnet_ref_quantize_states.argtypes = [P, I, I, I, P, P, I, P, P]
        L.bitnet_ref_quantize_states.restype = None
        L.bitnet_ref_forward_qkv_states.argtypes = [P, I, I, I, P, I, I, P, P, P, I, P, P]
        L.bitnet_ref_forward_qkv_states.restype = I
        L.bitnet_ref_num_threads.argtypes = []; L.bitnet_ref_num_threads.restype = I
        L.bitnet_ref_set_num_threads.argtypes = [I]; L.bitnet_ref_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- base-3 byte code -------------------------------------------------------------------

def encode5(digits) -> int:
    d = _c(digits, np.int32)
    assert d.shape == (5,)
    return lib().bitnet_ref_encode5(_p(d))


def decode5(byte: int):
    d = np.zeros(5, np.int32)
    rc = lib().bitnet_ref_decode5(int(byte), _p(d))
    return None if rc != 0 else d


# ---- weights ----------------------------------------------------------------------------

def absmean(W) -> np.float32:
    W = _c(W, np.float32)
    return np.float32(lib().bitnet_ref_absmean(_p(W), W.size))


def ternarize(W):
    """absmean ternarisation of an N x K fp32 matrix -> (t int8 N x K, gamma float32)."""
    W = _c(W, np.float32)
    N, K = W.shape
    t = np.empty((N, K), np.int8)
    g = np.zeros(1, np.float32)
    lib().bitnet_ref_ternarize(_p(W), N, K, _p(t), _p(g))
    return t, np.float32(g[0])


def row_bytes(K: int) -> int:
    return int(lib().bitnet_ref_row_bytes(K))


def packed_bytes(N: int, K: int) -> int:
    return int(lib().bitnet_ref_packed_bytes(N, K))


def pack(t):
    t = _c(t, np.int8)
    N, K = t.shape
    out = np.empty(packed_bytes(N, K), np.uint8)
    lib().bitnet_ref_pack(_p(t), N, K, _p(out))
    return out


def unpack(packed, N: int, K: int):
    packed = _c(packed, np.uint8)
    t = np.empty((N, K), np.int8)
    rc = lib().bitnet_ref_unpack(_p(packed), N, K, _p(t))
    if rc != 0:
        raise ValueError("packed buffer does not decode")
    return t


def pack_weights(W):
    """Offline step: ternarise then pack -> (packed uint8, gamma float32, t int8)."""
    t, g = ternarize(W)
    return pack(t), g, t


# ---- activations ------------------------------------------------------------------------

def fwht(x):
    """Unnormalised fast Walsh-Hadamard transform of the last axis, fp32, in a copy."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    n = x.shape[-1]
    for row in x.reshape(-1, n):
        lib().bitnet_ref_fwht(_p(row), n)
    return x


def fwht_f64(x):
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    n = x.shape[-1]
    for row in x.reshape(-1, n):
        lib().bitnet_ref_fwht_f64(_p(row), n)
    return x


def hadamard_scale(n: int) -> np.float32:
    return np.float32(lib().bitnet_ref_hadamard_scale(n))


def hadamard(x):
    """Normalised transform x H_n / sqrt(n) of the last axis, fp32, in a copy."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    n = x.shape[-1]
    for row in x.reshape(-1, n):
        lib().bitnet_ref_hadamard(_p(row), n)
    return x


def quantize_row(x, bits: int):
    x = _c(x, np.float32)
    q = np.empty(x.shape[0], np.int8)
    s = np.zeros(1, np.float32)
    lib().bitnet_ref_quantize_row(_p(x), x.shape[0], bits, _p(q), _p(s))
    return q, np.float32(s[0])


def pack_int4(q):
    q = _c(q, np.int8)
    out = np.empty(q.size // 2, np.uint8)
    lib().bitnet_ref_pack_int4(_p(q), q.size, _p(out))
    return out.reshape(q.shape[:-1] + (q.shape[-1] // 2,))


def unpack_int4(b, K: int):
    b = _c(b, np.uint8)
    rows = b.size * 2 // K
    q = np.empty((rows, K), np.int8)
    lib().bitnet_ref_unpack_int4(_p(b), q.size, _p(q))
    return q


def quantize(x, bits: int, use_hadamard: bool, want_xh: bool = False):
    """Activation stage for M x K rows -> (q int8 M x K, scales float32 M[, xh])."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    xh = np.empty((M, K), np.float32) if want_xh else None
    lib().bitnet_ref_quantize(_p(x), M, K, bits, int(bool(use_hadamard)), _p(q), _p(s),
                              _p(xh) if xh is not None else None)
    return (q, s, xh) if want_xh else (q, s)


def gemm(q, t):
    """acc = q t^T as add/subtract/skip, int32 (q: M x K int8, t: N x K int8)."""
    q = _c(q, np.int8)
    t = _c(t, np.int8)
    M, K = q.shape
    N, K2 = t.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    lib().bitnet_ref_gemm(_p(q), _p(t), M, N, K, _p(acc))
    return acc


def epilogue(acc, scales, gamma_w):
    acc = _c(acc, np.int32)
    scales = _c(scales, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    lib().bitnet_ref_epilogue(_p(acc), _p(scales), float(gamma_w), M, N, _p(y))
    return y


def forward(x, packed, gamma_w, N: int, bits: int, use_hadamard: bool):
    x = _c(x, np.float32)
    packed = _c(packed, np.uint8)
    M, K = x.shape
    y = np.empty((M, N), np.float32)
    rc = lib().bitnet_ref_forward(_p(x), M, K, N, bits, int(bool(use_hadamard)), _p(packed),
                                  float(gamma_w), _p(y))
    if rc != 0:
        raise ValueError("packed buffer does not decode")
    return y


def rotate_weights(W):
    """W_h = W H / sqrt(K) row by row (double, one rounding to fp32)."""
    W = _c(W, np.float32)
    N, K = W.shape
    Wh = np.empty((N, K), np.float32)
    lib().bitnet_ref_rotate_weights(_p(W), N, K, _p(Wh))
    return Wh


def pack_weights_hadamard(W):
    """Offline step of the weight + activation variant -> (packed uint8, gamma float32)."""
    W = _c(W, np.float32)
    N, K = W.shape
    out = np.empty(packed_bytes(N, K), np.uint8)
    g = np.zeros(1, np.float32)
    lib().bitnet_ref_pack_weights_hadamard(_p(W), N, K, _p(out), _p(g))
    return out, np.float32(g[0])


def rms_scale(row, eps: float) -> np.float32:
    row = _c(row, np.float32)
    return np.float32(lib().bitnet_ref_rms_scale(_p(row), row.size, float(eps)))


def rmsnorm(x, gain, eps: float):
    """y = (x * r) * gain per row, r = 1 / sqrt(mean(x^2) + eps) (double sum, fp32 r)."""
    x = _c(x, np.float32)
    gain = _c(gain, np.float32)
    M, K = x.shape
    assert gain.shape == (K,)
    y = np.empty((M, K), np.float32)
    lib().bitnet_ref_rmsnorm(_p(x), M, K, _p(gain), float(eps), _p(y))
    return y


def forward_rmsnorm(x, gain, eps: float, packed, gamma_w, N: int, bits: int, use_hadamard: bool):
    x = _c(x, np.float32)
    gain = _c(gain, np.float32)
    packed = _c(packed, np.uint8)
    M, K = x.shape
    y = np.empty((M, N), np.float32)
    rc = lib().bitnet_ref_forward_rmsnorm(_p(x), M, K, N, _p(gain), float(eps), bits,
                                          int(bool(use_hadamard)), _p(packed), float(gamma_w), _p(y))
    if rc != 0:
        raise ValueError("packed buffer does not decode")
    return y


def forward_segments(x, packs, gammas, seg_n, bits: int, use_hadamard: bool):
    """Several linears of one input: y = [forward(x, packs[s], gammas[s]) for s] side by side
    (M x sum(seg_n)); packs are separately packed matrices."""
    x = _c(x, np.float32)
    M, K = x.shape
    S = len(seg_n)
    bufs = [_c(p, np.uint8) for p in packs]
    ptrs = (ctypes.c_void_p * S)(*[b.ctypes.data for b in bufs])
    n = np.asarray(seg_n, np.int32)
    g = np.asarray(gammas, np.float32)
    y = np.empty((M, int(n.sum())), np.float32)
    rc = lib().bitnet_ref_forward_segments(_p(x), M, K, S, _p(n), bits, int(bool(use_hadamard)),
                                           ctypes.cast(ptrs, ctypes.c_void_p), _p(g), _p(y))
    if rc != 0:
        raise ValueError("packed buffer does not decode")
    return y


def silu(z) -> np.float32:
    return np.float32(lib().bitnet_ref_silu(float(z)))


def swiglu(g, u):
    """h = SiLU(g) * u elementwise (double arithmetic, one rounding to fp32)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.float32)
    lib().bitnet_ref_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def forward_swiglu(x, packed_gate, gamma_gate, packed_up, gamma_up, F: int, bits: int,
                   use_hadamard: bool):
    """h (M x F) = SwishGLU of the gate and up forwards of x."""
    x = _c(x, np.float32)
    M, K = x.shape
    pg = _c(packed_gate, np.uint8)
    pu = _c(packed_up, np.uint8)
    h = np.empty((M, F), np.float32)
    rc = lib().bitnet_ref_forward_swiglu(_p(x), M, K, F, bits, int(bool(use_hadamard)), _p(pg),
                                         float(gamma_gate), _p(pu), float(gamma_up), _p(h))
    if rc != 0:
        raise ValueError("packed buffer does not decode")
    return h


def quantize_states(y, seg_n, bits, group: int):
    """Low-bit Q/K/V states: y (M x sum(seg_n) fp32) -> (codes int8 M x Ntot, scales fp32
    M x Ntot/group), absmax per token and per group of `group` columns, bits[s] per segment."""
    y = _c(y, np.float32)
    M, ntot = y.shape
    n = np.asarray(seg_n, np.int32)
    b = np.asarray(bits, np.int32)
    assert n.size == b.size and int(n.sum()) == ntot and np.all(n % group == 0)
    codes = np.empty((M, ntot), np.int8)
    scales = np.empty((M, ntot // group), np.float32)
    lib().bitnet_ref_quantize_states(_p(y), M, ntot, n.size, _p(n), _p(b), group, _p(codes),
                                     _p(scales))
    return codes, scales


def forward_qkv_states(x, packs, gammas, seg_n, act_bits: int, use_hadamard: bool, bits, group: int):
    """forward_segments, then quantize_states of its output -> (codes, scales)."""
    x = _c(x, np.float32)
    M, K = x.shape
    S = len(seg_n)
    bufs = [_c(p, np.uint8) for p in packs]
    ptrs = (ctypes.c_void_p * S)(*[q.ctypes.data for q in bufs])
    n = np.asarray(seg_n, np.int32)
    g = np.asarray(gammas, np.float32)
    b = np.asarray(bits, np.int32)
    ntot = int(n.sum())
    codes = np.empty((M, ntot), np.int8)
    scales = np.empty((M, ntot // group), np.float32)
    rc = lib().bitnet_ref_forward_qkv_states(_p(x), M, K, S, _p(n), act_bits, int(bool(use_hadamard)),
                                             ctypes.cast(ptrs, ctypes.c_void_p), _p(g), _p(b), group,
                                             _p(codes), _p(scales))
    if rc != 0:
        raise ValueError("packed buffer does not decode")
    return codes, scales


def num_threads() -> int:
    return int(lib().bitnet_ref_num_threads())


def set_num_threads(n: int) -> None:
    lib().bitnet_ref_set_num_threads(int(n))
