"""Python binding of libbitnet_hip.so: argument marshalling only.

Every function has the name of the C entry point it calls (include/bitnet.h).  Device buffers
are torch CUDA (HIP) tensors; PyTorch supplies the memory and the stream, and every step of
the forward runs in the library's HIP kernels.  There is no fallback: if the library is not
built, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitnet_hip.so")

BITNET_OK = 0
BITNET_ERR_NULL = -1
BITNET_ERR_SHAPE = -2
BITNET_ERR_UNSUPPORTED = -3
BITNET_ERR_WORKSPACE = -4
BITNET_ERR_HIP = -5
BITNET_ERR_FORMAT = -6

_lib = None


class BitnetError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bitnet_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m ternary_weight_bit_bitlinear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        PSZ = ctypes.POINTER(ctypes.c_size_t)
        sigs = {
            "bitnet_status_string": ([I], ctypes.c_char_p),
            "bitnet_abi_version": ([], I),
            "bitnet_packed_bytes": ([I, I, PSZ], I),
            "bitnet_pack_weights": ([P, I, I, P, P], I),
            "bitnet_unpack_weights": ([P, I, I, P], I),
            "hbitlinear_workspace_bytes": ([I, I, I, PSZ], I),
            "hbitlinear_codes_bytes": ([I, I, I, PSZ], I),
            "hbitlinear_forward": ([P, I, I, I, I, I, P, P, F, P, SZ, P], I),
            "hbitlinear_forward_noalloc": ([P, I, I, I, I, I, P, P, F, P], I),
            "hbitlinear_quantize": ([P, I, I, I, I, P, P, P, P], I),
            "bitnet_ternary_gemm_i32": ([P, I, I, I, I, P, P, P], I),
            "hbitlinear_gemm_dequant": ([P, P, I, I, I, I, P, F, P, P], I),
            "hbitlinear_grouped_workspace_bytes": ([I, I, I, I, PSZ], I),
            "hbitlinear_forward_grouped": ([I, P, I, I, I, I, I, P, P, P, P, SZ, P], I),
            "hbitlinear_gemm_dequant_grouped": ([P, P, I, I, I, I, I, P, P, P, P], I),
            "hbitlinear_quantize_rmsnorm": ([P, I, I, P, F, I, I, P, P, P, P], I),
            "hbitlinear_forward_rmsnorm": ([P, I, I, I, P, F, I, I, P, P, F, P, SZ, P], I),
            "bitnet_pack_weights_hadamard": ([P, I, I, P, P], I),
            "bitnet_pack_weights_segments": ([P, I, P, I, P, P], I),
            "bitnet_pack_gate_up": ([P, P, I, I, P, P, P], I),
            "hbitlinear_forward_segments": ([P, I, I, I, P, I, I, P, P, P, P, SZ, P], I),
            "hbitlinear_gemm_dequant_segments": ([P, P, I, I, I, P, I, P, P, P, P], I),
            "hbitlinear_forward_swiglu": ([P, I, I, I, I, I, P, P, F, F, P, SZ, P], I),
            "hbitlinear_gemm_swiglu": ([P, P, I, I, I, I, P, F, F, P, P], I),
            "hbitlinear_forward_qkv_states": ([P, I, I, I, P, I, I, P, P, P, I, P, P, P, SZ, P], I),
            "hbitlinear_gemm_qkv_states": ([P, P, I, I, I, P, I, P, P, P, I, P, P, P], I),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != BITNET_OK:
        raise BitnetError(status, where)


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(None)
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return ctypes.c_void_p(t.ctypes.data)
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _rows_k(x, name="x"):
    if len(x.shape) != 2:
        raise ValueError(f"{name} must be 2-D (M x K)")
    return int(x.shape[0]), int(x.shape[1])


def _packed_check(packed, rows: int, K: int, name: str) -> None:
    # the kernels size their reads from N and K, not from the allocation: a short buffer would
    # be read past its end on the device, so it is refused here, before anything else
    if packed.numel() < bitnet_packed_bytes(rows, K):
        raise ValueError(f"{name} holds {packed.numel()} bytes, the packed {rows} x {K} weight "
                         f"needs {bitnet_packed_bytes(rows, K)}")


def _dev_check(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---- status / sizes -------------------------------------------------------------------------

def bitnet_status_string(status: int) -> str:
    return lib().bitnet_status_string(int(status)).decode()


def bitnet_abi_version() -> int:
    return int(lib().bitnet_abi_version())


def bitnet_packed_bytes(N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().bitnet_packed_bytes(N, K, ctypes.byref(out)), "bitnet_packed_bytes")
    return int(out.value)


def hbitlinear_workspace_bytes(M: int, K: int, act_bits: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().hbitlinear_workspace_bytes(M, K, act_bits, ctypes.byref(out)),
           "hbitlinear_workspace_bytes")
    return int(out.value)


def hbitlinear_codes_bytes(M: int, K: int, act_bits: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().hbitlinear_codes_bytes(M, K, act_bits, ctypes.byref(out)), "hbitlinear_codes_bytes")
    return int(out.value)


# ---- offline weights (host) -----------------------------------------------------------------

def bitnet_pack_weights(W):
    """absmean-ternarise and pack an N x K fp32 host matrix -> (packed uint8, w_scale float)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    packed = np.empty(bitnet_packed_bytes(N, K), np.uint8)
    g = ctypes.c_float(0.0)
    _check(lib().bitnet_pack_weights(_ptr(W), N, K, _ptr(packed), ctypes.byref(g)),
           "bitnet_pack_weights")
    return packed, float(g.value)


def bitnet_pack_weights_hadamard(W):
    """Rotate an N x K fp32 host matrix by H_K / sqrt(K) (row by row), then ternarise and pack
    -> (packed uint8, w_scale float).  Pair with use_hadamard=True in the forward."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    packed = np.empty(bitnet_packed_bytes(N, K), np.uint8)
    g = ctypes.c_float(0.0)
    _check(lib().bitnet_pack_weights_hadamard(_ptr(W), N, K, _ptr(packed), ctypes.byref(g)),
           "bitnet_pack_weights_hadamard")
    return packed, float(g.value)


def bitnet_pack_weights_segments(W, seg_n):
    """Pack S matrices stacked by rows in W (sum(seg_n) x K fp32, host), each with its own
    absmean scale -> (packed uint8, w_scales float32 array of S)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    n = np.ascontiguousarray(seg_n, dtype=np.int32)
    S = n.size
    rows, K = W.shape
    if int(n.sum()) != rows:
        raise ValueError("W must have sum(seg_n) rows")
    packed = np.empty(bitnet_packed_bytes(rows, K), np.uint8)
    g = np.zeros(S, np.float32)
    _check(lib().bitnet_pack_weights_segments(_ptr(W), S, _ptr(n), K, _ptr(packed), _ptr(g)),
           "bitnet_pack_weights_segments")
    return packed, g


def bitnet_pack_gate_up(W_gate, W_up):
    """Pack the gate and up matrices (F x K fp32 each, host), interleaved by 16-row groups ->
    (packed uint8, gate_scale, up_scale)."""
    Wg = np.ascontiguousarray(W_gate, dtype=np.float32)
    Wu = np.ascontiguousarray(W_up, dtype=np.float32)
    if Wg.shape != Wu.shape:
        raise ValueError("gate and up must have the same shape")
    F, K = Wg.shape
    packed = np.empty(bitnet_packed_bytes(2 * F, K), np.uint8)
    gg, gu = ctypes.c_float(0.0), ctypes.c_float(0.0)
    _check(lib().bitnet_pack_gate_up(_ptr(Wg), _ptr(Wu), F, K, _ptr(packed), ctypes.byref(gg),
                                     ctypes.byref(gu)), "bitnet_pack_gate_up")
    return packed, float(gg.value), float(gu.value)


def bitnet_unpack_weights(packed, N: int, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    t = np.empty((N, K), np.int8)
    _check(lib().bitnet_unpack_weights(_ptr(packed), N, K, _ptr(t)), "bitnet_unpack_weights")
    return t


# ---- forward (device) -----------------------------------------------------------------------

def hbitlinear_forward(x, N: int, act_bits: int, use_hadamard: bool, packed_w, w_scale: float,
                       out=None, workspace=None, stream=None):
    """out = H-BitLinear(x) for x (M x K fp32, device); returns out (M x N fp32, device)."""
    import torch
    M, K = _rows_k(x)
    _packed_check(packed_w, N, K, "packed_w")
    _dev_check(x, torch.float32, "x")
    _dev_check(packed_w, torch.uint8, "packed_w")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < M * N:
        raise ValueError("out is too small")
    if workspace is None:
        workspace = torch.empty(hbitlinear_workspace_bytes(M, K, act_bits), dtype=torch.uint8,
                                device=x.device)
    _dev_check(workspace, torch.uint8, "workspace")
    _check(lib().hbitlinear_forward(_ptr(x), M, K, N, act_bits, int(bool(use_hadamard)),
                                    _ptr(out), _ptr(packed_w), float(w_scale), _ptr(workspace),
                                    workspace.numel(), _stream(stream)), "hbitlinear_forward")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20   # BITNET_NOALLOC_SCRATCH_BYTES


def hbitlinear_forward_noalloc(x, N: int, act_bits: int, use_hadamard: bool, packed_w,
                               w_scale: float, out, stream=None):
    """hbitlinear_forward with the library's static device workspace: x (M x K fp32, device),
    out (M x N fp32, device, the caller's: nothing is allocated here or in the library).
    Calls that overlap on one GPU race on the shared workspace."""
    import torch
    M, K = _rows_k(x)
    _packed_check(packed_w, N, K, "packed_w")
    if out.numel() < M * N:
        raise ValueError("out is too small")
    _dev_check(x, torch.float32, "x")
    _dev_check(packed_w, torch.uint8, "packed_w")
    _dev_check(out, torch.float32, "out")
    _check(lib().hbitlinear_forward_noalloc(_ptr(x), M, K, N, act_bits, int(bool(use_hadamard)),
                                            _ptr(out), _ptr(packed_w), float(w_scale),
                                            _stream(stream)), "hbitlinear_forward_noalloc")
    return out


def _seg_arrays(seg_n, w_scales):
    n = np.ascontiguousarray(seg_n, dtype=np.int32)
    g = np.ascontiguousarray(w_scales, dtype=np.float32)
    if g.size != n.size:
        raise ValueError("seg_n and w_scales need the same number of entries")
    return n, g


def hbitlinear_forward_segments(x, seg_n, act_bits: int, use_hadamard: bool, packed_w, w_scales,
                                out=None, workspace=None, stream=None):
    """Several linears of one input: x (M x K fp32, device), packed_w from
    bitnet_pack_weights_segments (device), seg_n / w_scales (host sequences of S) ->
    out (M x sum(seg_n) fp32, device)."""
    import torch
    n, g = _seg_arrays(seg_n, w_scales)
    M, K = _rows_k(x)
    N = int(n.sum())
    _packed_check(packed_w, N, K, "packed_w")
    _dev_check(x, torch.float32, "x")
    _dev_check(packed_w, torch.uint8, "packed_w")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < M * N:
        raise ValueError("out is too small")
    if workspace is None:
        workspace = torch.empty(hbitlinear_workspace_bytes(M, K, act_bits), dtype=torch.uint8,
                                device=x.device)
    _dev_check(workspace, torch.uint8, "workspace")
    _check(lib().hbitlinear_forward_segments(_ptr(x), M, K, n.size, _ptr(n), act_bits,
                                             int(bool(use_hadamard)), _ptr(out), _ptr(packed_w),
                                             _ptr(g), _ptr(workspace), workspace.numel(),
                                             _stream(stream)), "hbitlinear_forward_segments")
    return out


def _state_outputs(M, N, group, state_codes, state_scales, device):
    import torch
    if state_codes is None:
        state_codes = torch.empty((M, N), dtype=torch.int8, device=device)
    if state_scales is None:
        state_scales = torch.empty((M, N // group), dtype=torch.float32, device=device)
    if state_codes.numel() < M * N or state_scales.numel() < M * (N // group):
        raise ValueError("state_codes or state_scales is too small")
    _dev_check(state_codes, torch.int8, "state_codes")
    _dev_check(state_scales, torch.float32, "state_scales")
    return state_codes, state_scales


def hbitlinear_forward_qkv_states(x, seg_n, act_bits: int, use_hadamard: bool, packed_w, w_scales,
                                  state_bits, group: int, state_codes=None, state_scales=None,
                                  workspace=None, stream=None):
    """Low-bit Q/K/V states: the projections of x (M x K fp32, device) by the stacked matrices
    of bitnet_pack_weights_segments, quantised per row and per `group` columns to
    state_bits[s] bits -> (state_codes int8 M x N, state_scales fp32 M x N/group), device."""
    import torch
    n, g = _seg_arrays(seg_n, w_scales)
    b = np.ascontiguousarray(state_bits, dtype=np.int32)
    if b.size != n.size:
        raise ValueError("state_bits needs one entry per segment")
    M, K = _rows_k(x)
    N = int(n.sum())
    _packed_check(packed_w, N, K, "packed_w")
    _dev_check(x, torch.float32, "x")
    _dev_check(packed_w, torch.uint8, "packed_w")
    state_codes, state_scales = _state_outputs(M, N, group, state_codes, state_scales, x.device)
    if workspace is None:
        workspace = torch.empty(hbitlinear_workspace_bytes(M, K, act_bits), dtype=torch.uint8,
                                device=x.device)
    _dev_check(workspace, torch.uint8, "workspace")
    _check(lib().hbitlinear_forward_qkv_states(_ptr(x), M, K, n.size, _ptr(n), act_bits,
                                               int(bool(use_hadamard)), _ptr(packed_w), _ptr(g),
                                               _ptr(b), group, _ptr(state_codes), _ptr(state_scales),
                                               _ptr(workspace), workspace.numel(), _stream(stream)),
           "hbitlinear_forward_qkv_states")
    return state_codes, state_scales


def hbitlinear_gemm_qkv_states(codes, scales, M: int, K: int, seg_n, act_bits: int, packed_w,
                               w_scales, state_bits, group: int, state_codes=None,
                               state_scales=None, stream=None):
    """Product stage of hbitlinear_forward_qkv_states from device codes and scales."""
    import torch
    n, g = _seg_arrays(seg_n, w_scales)
    b = np.ascontiguousarray(state_bits, dtype=np.int32)
    if b.size != n.size:
        raise ValueError("state_bits needs one entry per segment")
    N = int(n.sum())
    _packed_check(packed_w, N, K, "packed_w")
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits) or scales.numel() < M:
        raise ValueError("codes or scales buffer is too small")
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    _dev_check(packed_w, torch.uint8, "packed_w")
    state_codes, state_scales = _state_outputs(M, N, group, state_codes, state_scales, codes.device)
    _check(lib().hbitlinear_gemm_qkv_states(_ptr(codes), _ptr(scales), M, K, n.size, _ptr(n),
                                            act_bits, _ptr(packed_w), _ptr(g), _ptr(b), group,
                                            _ptr(state_codes), _ptr(state_scales), _stream(stream)),
           "hbitlinear_gemm_qkv_states")
    return state_codes, state_scales


def hbitlinear_forward_swiglu(x, F: int, act_bits: int, use_hadamard: bool, packed_gate_up,
                              gate_scale: float, up_scale: float, out=None, workspace=None,
                              stream=None):
    """h = SiLU(gate(x)) * up(x): x (M x K fp32, device), packed_gate_up from
    bitnet_pack_gate_up (device) -> h (M x F fp32, device)."""
    import torch
    M, K = _rows_k(x)
    _packed_check(packed_gate_up, 2 * F, K, "packed_gate_up")
    _dev_check(x, torch.float32, "x")
    _dev_check(packed_gate_up, torch.uint8, "packed_gate_up")
    if out is None:
        out = torch.empty((M, F), dtype=torch.float32, device=x.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < M * F:
        raise ValueError("out is too small")
    if workspace is None:
        workspace = torch.empty(hbitlinear_workspace_bytes(M, K, act_bits), dtype=torch.uint8,
                                device=x.device)
    _dev_check(workspace, torch.uint8, "workspace")
    _check(lib().hbitlinear_forward_swiglu(_ptr(x), M, K, F, act_bits, int(bool(use_hadamard)),
                                           _ptr(out), _ptr(packed_gate_up), float(gate_scale),
                                           float(up_scale), _ptr(workspace), workspace.numel(),
                                           _stream(stream)), "hbitlinear_forward_swiglu")
    return out


def hbitlinear_grouped_workspace_bytes(L: int, M: int, K: int, act_bits: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().hbitlinear_grouped_workspace_bytes(L, M, K, act_bits, ctypes.byref(out)),
           "hbitlinear_grouped_workspace_bytes")
    return int(out.value)


def hbitlinear_forward_grouped(x, N: int, act_bits: int, use_hadamard: bool, packed_ptrs,
                               w_scales, out=None, workspace=None, stream=None):
    """L independent forwards: x (L x M x K fp32), packed_ptrs (int64 device tensor of L
    device addresses of packed weights), w_scales (L fp32 device tensor) -> out (L x M x N).
    The buffers behind packed_ptrs are not visible here: each must hold
    bitnet_packed_bytes(N, K) bytes."""
    import torch
    _dev_check(x, torch.float32, "x")
    _dev_check(packed_ptrs, torch.int64, "packed_ptrs")
    _dev_check(w_scales, torch.float32, "w_scales")
    L, M, K = x.shape
    if packed_ptrs.numel() < L or w_scales.numel() < L:
        raise ValueError("packed_ptrs / w_scales need L entries")
    if out is None:
        out = torch.empty((L, M, N), dtype=torch.float32, device=x.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < L * M * N:
        raise ValueError("out is too small")
    if workspace is None:
        workspace = torch.empty(hbitlinear_grouped_workspace_bytes(L, M, K, act_bits),
                                dtype=torch.uint8, device=x.device)
    _dev_check(workspace, torch.uint8, "workspace")
    _check(lib().hbitlinear_forward_grouped(L, _ptr(x), M, K, N, act_bits, int(bool(use_hadamard)),
                                            _ptr(out), _ptr(packed_ptrs), _ptr(w_scales),
                                            _ptr(workspace), workspace.numel(), _stream(stream)),
           "hbitlinear_forward_grouped")
    return out


def hbitlinear_quantize(x, act_bits: int, use_hadamard: bool, codes=None, scales=None,
                        want_xh: bool = False, stream=None):
    """Activation stage -> (codes uint8, scales fp32[, xh fp32]) on the device."""
    import torch
    _dev_check(x, torch.float32, "x")
    M, K = x.shape
    if codes is None:
        codes = torch.empty(hbitlinear_codes_bytes(M, K, act_bits), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits) or scales.numel() < M:
        raise ValueError("codes or scales buffer is too small")
    xh = torch.empty((M, K), dtype=torch.float32, device=x.device) if want_xh else None
    _check(lib().hbitlinear_quantize(_ptr(x), M, K, act_bits, int(bool(use_hadamard)), _ptr(codes),
                                     _ptr(scales), _ptr(xh), _stream(stream)), "hbitlinear_quantize")
    return (codes, scales, xh) if want_xh else (codes, scales)


def bitnet_ternary_gemm_i32(codes, M: int, K: int, N: int, act_bits: int, packed_w, acc=None,
                            stream=None):
    """acc = sum_k q t (exact int32, M x N, device) from device codes and packed weights."""
    import torch
    _packed_check(packed_w, N, K, "packed_w")
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits):
        raise ValueError("codes buffer is too small")
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(packed_w, torch.uint8, "packed_w")
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=codes.device)
    _dev_check(acc, torch.int32, "acc")
    _check(lib().bitnet_ternary_gemm_i32(_ptr(codes), M, K, N, act_bits, _ptr(packed_w), _ptr(acc),
                                         _stream(stream)), "bitnet_ternary_gemm_i32")
    return acc


def hbitlinear_gemm_dequant(codes, scales, M: int, K: int, N: int, act_bits: int, packed_w,
                            w_scale: float, out=None, stream=None):
    import torch
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    _dev_check(packed_w, torch.uint8, "packed_w")
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits) or scales.numel() < M:
        raise ValueError("codes or scales buffer is too small")
    if packed_w.numel() < bitnet_packed_bytes(N, K):
        raise ValueError("packed_w buffer is too small")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _dev_check(out, torch.float32, "out")
    _check(lib().hbitlinear_gemm_dequant(_ptr(codes), _ptr(scales), M, K, N, act_bits,
                                         _ptr(packed_w), float(w_scale), _ptr(out),
                                         _stream(stream)), "hbitlinear_gemm_dequant")
    return out


def hbitlinear_gemm_dequant_grouped(codes, scales, L: int, M: int, K: int, N: int, act_bits: int,
                                    packed_ptrs, w_scales, out=None, stream=None):
    """Product stage of the grouped forward: codes/scales of L*M rows -> out (L x M x N)."""
    import torch
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    _dev_check(packed_ptrs, torch.int64, "packed_ptrs")
    _dev_check(w_scales, torch.float32, "w_scales")
    if codes.numel() < hbitlinear_codes_bytes(L * M, K, act_bits) or scales.numel() < L * M:
        raise ValueError("codes or scales buffer is too small")
    if packed_ptrs.numel() < L or w_scales.numel() < L:
        raise ValueError("packed_ptrs / w_scales need L entries")
    if out is None:
        out = torch.empty((L, M, N), dtype=torch.float32, device=codes.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < L * M * N:
        raise ValueError("out is too small")
    _check(lib().hbitlinear_gemm_dequant_grouped(_ptr(codes), _ptr(scales), L, M, K, N, act_bits,
                                                 _ptr(packed_ptrs), _ptr(w_scales), _ptr(out),
                                                 _stream(stream)), "hbitlinear_gemm_dequant_grouped")
    return out


def hbitlinear_gemm_dequant_segments(codes, scales, M: int, K: int, seg_n, act_bits: int,
                                     packed_w, w_scales, out=None, stream=None):
    """Product stage of hbitlinear_forward_segments from device codes and scales."""
    import torch
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    _dev_check(packed_w, torch.uint8, "packed_w")
    n, g = _seg_arrays(seg_n, w_scales)
    N = int(n.sum())
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits) or scales.numel() < M:
        raise ValueError("codes or scales buffer is too small")
    if packed_w.numel() < bitnet_packed_bytes(N, K):
        raise ValueError("packed_w buffer is too small")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < M * N:
        raise ValueError("out is too small")
    _check(lib().hbitlinear_gemm_dequant_segments(_ptr(codes), _ptr(scales), M, K, n.size, _ptr(n),
                                                  act_bits, _ptr(packed_w), _ptr(g), _ptr(out),
                                                  _stream(stream)), "hbitlinear_gemm_dequant_segments")
    return out


def hbitlinear_gemm_swiglu(codes, scales, M: int, K: int, F: int, act_bits: int, packed_gate_up,
                           gate_scale: float, up_scale: float, out=None, stream=None):
    """Product stage of hbitlinear_forward_swiglu from device codes and scales -> h (M x F)."""
    import torch
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    _dev_check(packed_gate_up, torch.uint8, "packed_gate_up")
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits) or scales.numel() < M:
        raise ValueError("codes or scales buffer is too small")
    if packed_gate_up.numel() < bitnet_packed_bytes(2 * F, K):
        raise ValueError("packed_gate_up buffer is too small")
    if out is None:
        out = torch.empty((M, F), dtype=torch.float32, device=codes.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < M * F:
        raise ValueError("out is too small")
    _check(lib().hbitlinear_gemm_swiglu(_ptr(codes), _ptr(scales), M, K, F, act_bits,
                                        _ptr(packed_gate_up), float(gate_scale), float(up_scale),
                                        _ptr(out), _stream(stream)), "hbitlinear_gemm_swiglu")
    return out


def hbitlinear_quantize_rmsnorm(x, gain, eps: float, act_bits: int, use_hadamard: bool, codes=None,
                                scales=None, want_xh: bool = False, stream=None):
    """Activation stage with the RMS norm in front -> (codes, scales[, x' after the transform])."""
    import torch
    _dev_check(x, torch.float32, "x")
    _dev_check(gain, torch.float32, "gain")
    M, K = x.shape
    if gain.numel() < K:
        raise ValueError("gain needs K entries")
    if codes is None:
        codes = torch.empty(hbitlinear_codes_bytes(M, K, act_bits), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    _dev_check(codes, torch.uint8, "codes")
    _dev_check(scales, torch.float32, "scales")
    if codes.numel() < hbitlinear_codes_bytes(M, K, act_bits) or scales.numel() < M:
        raise ValueError("codes or scales buffer is too small")
    xh = torch.empty((M, K), dtype=torch.float32, device=x.device) if want_xh else None
    _check(lib().hbitlinear_quantize_rmsnorm(_ptr(x), M, K, _ptr(gain), float(eps), act_bits,
                                             int(bool(use_hadamard)), _ptr(codes), _ptr(scales),
                                             _ptr(xh), _stream(stream)), "hbitlinear_quantize_rmsnorm")
    return (codes, scales, xh) if want_xh else (codes, scales)


def hbitlinear_forward_rmsnorm(x, gain, eps: float, N: int, act_bits: int, use_hadamard: bool,
                               packed_w, w_scale: float, out=None, workspace=None, stream=None):
    """out = forward(RMSNorm(x) * gain) for x (M x K fp32, device)."""
    import torch
    M, K = _rows_k(x)
    _packed_check(packed_w, N, K, "packed_w")
    _dev_check(x, torch.float32, "x")
    _dev_check(gain, torch.float32, "gain")
    _dev_check(packed_w, torch.uint8, "packed_w")
    if gain.numel() < K:
        raise ValueError("gain needs K entries")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _dev_check(out, torch.float32, "out")
    if out.numel() < M * N:
        raise ValueError("out is too small")
    if workspace is None:
        workspace = torch.empty(hbitlinear_workspace_bytes(M, K, act_bits), dtype=torch.uint8,
                                device=x.device)
    _dev_check(workspace, torch.uint8, "workspace")
    _check(lib().hbitlinear_forward_rmsnorm(_ptr(x), M, K, N, _ptr(gain), float(eps), act_bits,
                                            int(bool(use_hadamard)), _ptr(out), _ptr(packed_w),
                                            float(w_scale), _ptr(workspace), workspace.numel(),
                                            _stream(stream)), "hbitlinear_forward_rmsnorm")
    return out
