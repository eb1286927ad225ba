"""Host-side checks of libbitnet_hip.so: exported symbols, the offline packer against the oracle,
and argument validation (every failing check returns before anything reaches the GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import ternary_weight_bit_bitlinear_amd as tb
from conftest import ROOT
from packed_layout import device_groups, from_device, to_device

HEADER = os.path.join(ROOT, "include", "bitnet.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", src)) - {"if", "sizeof"})


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "hbitlinear_forward" in names and "bitnet_pack_weights" in names
    L = ctypes.CDLL(tb.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", tb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_library_is_independent_of_the_oracle():
    out = subprocess.run(["nm", "-D", tb.LIB_PATH], capture_output=True, text=True).stdout
    assert "bitnet_ref_" not in out
    ldd = subprocess.run(["ldd", tb.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in ldd
    csrc = os.path.join(ROOT, "ternary_weight_bit_bitlinear_amd", "csrc")
    for f in os.listdir(csrc):
        assert "oracle" not in open(os.path.join(csrc, f)).read().lower(), f


def test_abi_version_and_status_strings():
    assert tb.bitnet_abi_version() == 1
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert tb.bitnet_status_string(s) != "unknown status"
    assert tb.bitnet_status_string(-99) == "unknown status"


# The product packer against the oracle's canonical row-major bytes, three ways: the trits the
# product's unpacker reads back are the oracle's; the product's bytes are the canonical bytes
# placed by the documented tile permutation (pad rows all 121); and, read back through the
# inverse permutation, they decode with the oracle's unpacker to the same trits.
@pytest.mark.parametrize("N,K", [(1, 1), (3, 5), (4, 64), (7, 319), (5, 320), (9, 321),
                                 (16, 1000), (256, 256), (64, 4096), (33, 16384)])
def test_packer_matches_oracle_bytes(N, K):
    W = si.gaussian_weights(9, N, K)
    packed, g = tb.bitnet_pack_weights(W)
    opacked, og, ot = oracle.pack_weights(W)
    assert np.float32(g) == og
    assert opacked.size == oracle.packed_bytes(N, K) == N * 64 * ((K + 319) // 320)
    assert packed.size == tb.bitnet_packed_bytes(N, K) == (N + 15) // 16 * 16 * 64 * ((K + 319) // 320)
    assert np.array_equal(tb.bitnet_unpack_weights(packed, N, K), ot)
    assert np.array_equal(packed, to_device(opacked, N, K))
    assert np.array_equal(oracle.unpack(from_device(packed, N, K), N, K), ot)


def test_packer_matches_oracle_at_full_size():
    W = si.gaussian_weights(3, 4096, 4096)
    packed, g = tb.bitnet_pack_weights(W)
    opacked, og, ot = oracle.pack_weights(W)
    assert np.float32(g) == og and np.array_equal(packed, to_device(opacked, 4096, 4096))
    assert np.array_equal(tb.bitnet_unpack_weights(packed, 4096, 4096), ot)


def test_device_permutation_helper_is_a_bijection():
    # the helper's permutation: every canonical byte lands on its own device byte, pad rows
    # hold 121, and from_device inverts it
    N, K = 35, 700
    nb = (K + 319) // 320
    canon = np.arange(N * 64 * nb, dtype=np.int64)
    dev = to_device((canon % 241).astype(np.uint8), N, K)
    assert dev.size == 48 * 64 * nb
    assert np.array_equal(from_device(dev, N, K), (canon % 241).astype(np.uint8))
    # positions: row 1 of a tile follows row 0 by 16 bytes; the tile of block 1 starts at 1 KB
    idx = to_device(np.zeros(N * 64 * nb, np.uint8), N, K)
    assert np.count_nonzero(idx == 121) == (48 - N) * 64 * nb
    one = np.zeros((N, 64 * nb), np.uint8); one[1, 0] = 7; one[0, 64] = 9; one[20, 64 + 10] = 5
    d = to_device(one.reshape(-1), N, K)
    assert d[16] == 7 and d[1024] == 9
    assert d[(1 * nb + 1) * 1024 + (0 * 16 + 4) * 16 + 10] == 5


def test_packer_zero_and_worked_example():
    packed, g = tb.bitnet_pack_weights(np.zeros((2, 10), np.float32))
    assert g == 0.0 and np.all(packed == 121)
    # a row whose weights at k = 0, 64, 128, 192, 256 ternarise to (1, -1, 0, 1, 0)
    W = np.zeros((1, 320), np.float32)
    W[0, :] = 0.0
    W[0, [0, 64, 128, 192, 256]] = [1.0, -1.0, 0.0, 1.0, 0.0]
    W[0, 1] = 1.0          # keeps gamma small enough that +-1 stay +-1
    packed, g = tb.bitnet_pack_weights(W)
    assert packed[0] == 178


def test_unpack_rejects_bad_bytes():
    packed, _ = tb.bitnet_pack_weights(np.ones((1, 10), np.float32))
    bad = packed.copy(); bad[0] = 243
    with pytest.raises(tb.BitnetError) as e:
        tb.bitnet_unpack_weights(bad, 1, 10)
    assert e.value.status == tb.BITNET_ERR_FORMAT
    bad = packed.copy(); bad[40] = 0       # a padding trit of -1
    with pytest.raises(tb.BitnetError):
        tb.bitnet_unpack_weights(bad, 1, 10)


def _size(fn, *args):
    out = ctypes.c_size_t(0)
    return fn(*args, ctypes.byref(out)), out.value


def test_size_queries():
    L = tb.lib()
    assert _size(L.hbitlinear_codes_bytes, 16, 4096, 8) == (0, 16 * 4096)
    assert _size(L.hbitlinear_codes_bytes, 16, 4096, 4) == (0, 8 * 4096)
    rc, ws = _size(L.hbitlinear_workspace_bytes, 16, 4096, 8)
    assert rc == 0 and ws == 65536 + 256
    assert _size(L.bitnet_packed_bytes, 4096, 4096) == (0, 4096 * 832)
    assert L.hbitlinear_workspace_bytes(16, 4096, 8, None) == tb.BITNET_ERR_NULL
    assert _size(L.hbitlinear_workspace_bytes, 0, 4096, 8)[0] == tb.BITNET_ERR_SHAPE
    assert _size(L.hbitlinear_workspace_bytes, 4, 4096, 5)[0] == tb.BITNET_ERR_UNSUPPORTED
    assert _size(L.bitnet_packed_bytes, -1, 5)[0] == tb.BITNET_ERR_SHAPE


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first
NUL = ctypes.c_void_p(None)


@pytest.mark.parametrize("args,expect", [
    # (x, M, K, N, bits, had, out, packed, ws, ws_bytes)
    ((NUL, 4, 4096, 64, 8, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_NULL),
    ((FAKE, 4, 4096, 64, 8, 0, NUL, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_NULL),
    ((FAKE, 4, 4096, 64, 8, 0, FAKE, NUL, FAKE, 1 << 20), tb.BITNET_ERR_NULL),
    ((FAKE, 0, 4096, 64, 8, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_SHAPE),
    ((FAKE, 4, 0, 64, 8, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_SHAPE),
    ((FAKE, 4, 4096, -1, 8, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_SHAPE),
    ((FAKE, 4, 4096, 64, 2, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 4, 4096, 64, 8, 2, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 4, 4000, 64, 8, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 4, 4032, 64, 8, 1, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 4, 128, 64, 8, 1, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 4, 32768, 64, 8, 1, FAKE, FAKE, FAKE, 1 << 30), tb.BITNET_ERR_UNSUPPORTED),
    # an output of 4 M N >= 2 GiB, a layer's codes >= 2 GiB, packed weights >= 2 GiB
    ((FAKE, 16384, 4096, 32768, 8, 0, FAKE, FAKE, FAKE, 1 << 30), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 1 << 16, 32768, 64, 8, 0, FAKE, FAKE, FAKE, 1 << 40), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 1, 65536, 200000, 8, 0, FAKE, FAKE, FAKE, 1 << 20), tb.BITNET_ERR_UNSUPPORTED),
    ((FAKE, 4, 4096, 64, 8, 0, FAKE, FAKE, NUL, 1 << 20), tb.BITNET_ERR_WORKSPACE),
    ((FAKE, 4, 4096, 64, 8, 0, FAKE, FAKE, FAKE, 4 * 4096), tb.BITNET_ERR_WORKSPACE),
])
def test_forward_validation(args, expect):
    x, M, K, N, bits, had, out, packed, ws, wsb = args
    rc = tb.lib().hbitlinear_forward(x, M, K, N, bits, had, out, packed, ctypes.c_float(1.0), ws,
                                     wsb, NUL)
    assert rc == expect


def test_stage_validation():
    L = tb.lib()
    assert L.hbitlinear_quantize(NUL, 4, 256, 8, 1, FAKE, FAKE, NUL, NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_quantize(FAKE, 4, 200, 8, 1, FAKE, FAKE, NUL, NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.bitnet_ternary_gemm_i32(FAKE, 4, 256, 8, 8, NUL, FAKE, NUL) == tb.BITNET_ERR_NULL
    assert L.bitnet_ternary_gemm_i32(FAKE, 4, 256, 0, 8, FAKE, FAKE, NUL) == tb.BITNET_ERR_SHAPE
    assert L.hbitlinear_gemm_dequant(FAKE, NUL, 4, 256, 8, 4, FAKE, ctypes.c_float(1.0), FAKE,
                                     NUL) == tb.BITNET_ERR_NULL
    assert L.bitnet_pack_weights(NUL, 1, 1, FAKE, FAKE) == tb.BITNET_ERR_NULL
    # the product stages refuse outputs of 2 GiB or more before launching anything
    assert L.bitnet_ternary_gemm_i32(FAKE, 16384, 256, 32768, 8, FAKE, FAKE, NUL) == \
        tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_gemm_dequant(FAKE, FAKE, 16384, 256, 32768, 4, FAKE, ctypes.c_float(1.0),
                                     FAKE, NUL) == tb.BITNET_ERR_UNSUPPORTED


# --------------------------------------------- stacked and gate / up weight layouts ----

@pytest.mark.parametrize("seg_n,K", [([16, 32, 48], 640), ([4096 // 8, 1024 // 8, 1024 // 8], 1024),
                                     ([16], 320)])
def test_pack_segments_is_the_concatenation_of_separate_packs(seg_n, K):
    Ws = [si.gaussian_weights(10, n, K, layer=s, std=0.01 * (s + 1)) for s, n in enumerate(seg_n)]
    packed, gs = tb.bitnet_pack_weights_segments(np.concatenate(Ws), seg_n)
    parts = [oracle.pack_weights(W) for W in Ws]
    assert packed.size == tb.bitnet_packed_bytes(sum(seg_n), K)
    assert np.array_equal(packed, np.concatenate([to_device(p, n, K) for (p, _, _), n in zip(parts, seg_n)]))
    assert np.array_equal(gs, np.array([g for _, g, _ in parts], np.float32))
    # and the stacked buffer decodes to the stacked trits
    assert np.array_equal(tb.bitnet_unpack_weights(packed, sum(seg_n), K),
                          np.concatenate([t for _, _, t in parts]))


@pytest.mark.parametrize("F,K", [(16, 320), (48, 1000), (256, 4096)])
def test_pack_gate_up_interleaves_16_row_groups(F, K):
    Wg = si.gaussian_weights(11, F, K, layer=0)
    Wu = si.gaussian_weights(11, F, K, layer=1, std=0.05)
    packed, gg, gu = tb.bitnet_pack_gate_up(Wg, Wu)
    pg, og, tg = oracle.pack_weights(Wg)
    pu, ou, tu = oracle.pack_weights(Wu)
    assert (np.float32(gg), np.float32(gu)) == (og, ou)
    G = device_groups(packed, K)
    assert G.shape[0] == 2 * F // 16
    assert np.array_equal(G[0::2], device_groups(to_device(pg, F, K), K))
    assert np.array_equal(G[1::2], device_groups(to_device(pu, F, K), K))
    t = tb.bitnet_unpack_weights(packed, 2 * F, K).reshape(F // 16, 2, 16, K)
    assert np.array_equal(t[:, 0].reshape(F, K), tg)
    assert np.array_equal(t[:, 1].reshape(F, K), tu)


def test_segment_and_gate_up_validation():
    L = tb.lib()
    n3 = (ctypes.c_int * 3)(16, 32, 16)
    bad = (ctypes.c_int * 2)(16, 24)
    w3 = (ctypes.c_float * 3)(1.0, 1.0, 1.0)
    nine = (ctypes.c_int * 9)(*([16] * 9))
    w9 = (ctypes.c_float * 9)(*([1.0] * 9))
    f = ctypes.c_float(1.0)
    assert L.bitnet_pack_weights_segments(NUL, 3, n3, 64, FAKE, FAKE) == tb.BITNET_ERR_NULL
    assert L.bitnet_pack_weights_segments(FAKE, 2, bad, 64, FAKE, FAKE) == tb.BITNET_ERR_UNSUPPORTED
    assert L.bitnet_pack_weights_segments(FAKE, 9, nine, 64, FAKE, FAKE) == tb.BITNET_ERR_UNSUPPORTED
    assert L.bitnet_pack_weights_segments(FAKE, 0, n3, 64, FAKE, FAKE) == tb.BITNET_ERR_UNSUPPORTED
    assert L.bitnet_pack_gate_up(FAKE, NUL, 16, 64, FAKE, FAKE, FAKE) == tb.BITNET_ERR_NULL
    assert L.bitnet_pack_gate_up(FAKE, FAKE, 24, 64, FAKE, FAKE, FAKE) == tb.BITNET_ERR_UNSUPPORTED
    # forward entries: pointers, segment lists, shapes and workspace before any launch
    assert L.hbitlinear_forward_segments(NUL, 4, 256, 3, n3, 8, 0, FAKE, FAKE, w3, FAKE, 1 << 20,
                                         NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_forward_segments(FAKE, 4, 256, 3, NUL, 8, 0, FAKE, FAKE, w3, FAKE, 1 << 20,
                                         NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_forward_segments(FAKE, 4, 256, 2, bad, 8, 0, FAKE, FAKE, w3, FAKE, 1 << 20,
                                         NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_forward_segments(FAKE, 4, 256, 9, nine, 8, 0, FAKE, FAKE, w9, FAKE, 1 << 20,
                                         NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_forward_segments(FAKE, 4, 200, 3, n3, 8, 0, FAKE, FAKE, w3, FAKE, 1 << 20,
                                         NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_forward_segments(FAKE, 4, 256, 3, n3, 8, 0, FAKE, FAKE, w3, FAKE, 16,
                                         NUL) == tb.BITNET_ERR_WORKSPACE
    assert L.hbitlinear_gemm_dequant_segments(FAKE, FAKE, 4, 256, 3, n3, 8, FAKE, NUL, FAKE,
                                              NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_forward_swiglu(FAKE, 4, 256, 24, 8, 0, FAKE, FAKE, f, f, FAKE, 1 << 20,
                                       NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_forward_swiglu(FAKE, 4, 256, 0, 8, 0, FAKE, FAKE, f, f, FAKE, 1 << 20,
                                       NUL) == tb.BITNET_ERR_SHAPE
    assert L.hbitlinear_forward_swiglu(FAKE, 4, 256, 32, 8, 1, NUL, FAKE, f, f, FAKE, 1 << 20,
                                       NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_forward_swiglu(FAKE, 4, 256, 32, 8, 0, FAKE, FAKE, f, f, FAKE, 16,
                                       NUL) == tb.BITNET_ERR_WORKSPACE
    assert L.hbitlinear_gemm_swiglu(FAKE, FAKE, 4, 256, 32, 5, FAKE, f, f, FAKE,
                                    NUL) == tb.BITNET_ERR_UNSUPPORTED


def test_rmsnorm_validation():
    L = tb.lib()
    f = ctypes.c_float
    assert L.hbitlinear_quantize_rmsnorm(FAKE, 4, 1024, NUL, f(1e-6), 8, 0, FAKE, FAKE, NUL,
                                         NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_quantize_rmsnorm(FAKE, 4, 1024, FAKE, f(-1.0), 8, 0, FAKE, FAKE, NUL,
                                         NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_quantize_rmsnorm(FAKE, 4, 1024, FAKE, f(float("nan")), 8, 0, FAKE, FAKE,
                                         NUL, NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_quantize_rmsnorm(FAKE, 4, 1024, FAKE, f(float("inf")), 8, 0, FAKE, FAKE,
                                         NUL, NUL) == tb.BITNET_ERR_UNSUPPORTED
    # the norm needs the one-pass row kernel: power-of-two K in [256, 16384], with or without
    # the transform
    assert L.hbitlinear_quantize_rmsnorm(FAKE, 4, 960, FAKE, f(0.0), 8, 0, FAKE, FAKE, NUL,
                                         NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_quantize_rmsnorm(FAKE, 4, 32768, FAKE, f(0.0), 8, 0, FAKE, FAKE, NUL,
                                         NUL) == tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_forward_rmsnorm(FAKE, 4, 1024, 64, FAKE, f(0.0), 8, 1, NUL, FAKE, f(1.0),
                                        FAKE, 1 << 20, NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_forward_rmsnorm(FAKE, 4, 1024, 64, FAKE, f(0.0), 8, 1, FAKE, FAKE, f(1.0),
                                        FAKE, 16, NUL) == tb.BITNET_ERR_WORKSPACE


@pytest.mark.parametrize("N,K", [(16, 256), (33, 1024), (8, 4096)])
def test_pack_weights_hadamard_matches_oracle_bytes(N, K):
    W = si.gaussian_weights(17, N, K)
    packed, g = tb.bitnet_pack_weights_hadamard(W)
    opacked, og = oracle.pack_weights_hadamard(W)
    assert np.float32(g) == og
    assert np.array_equal(packed, to_device(opacked, N, K))


def test_pack_weights_hadamard_validation():
    L = tb.lib()
    assert L.bitnet_pack_weights_hadamard(NUL, 4, 256, FAKE, FAKE) == tb.BITNET_ERR_NULL
    assert L.bitnet_pack_weights_hadamard(FAKE, 4, 320, FAKE, FAKE) == tb.BITNET_ERR_UNSUPPORTED
    assert L.bitnet_pack_weights_hadamard(FAKE, 4, 128, FAKE, FAKE) == tb.BITNET_ERR_UNSUPPORTED
    assert L.bitnet_pack_weights_hadamard(FAKE, 0, 256, FAKE, FAKE) == tb.BITNET_ERR_SHAPE


# The binding refuses a packed weight buffer shorter than bitnet_packed_bytes for the rows the
# call reads (N, sum(seg_n), 2 F) before it looks at devices or calls the library: the kernels
# size their reads from the shape, so a short buffer would be read past its end on the GPU.
def test_binding_refuses_short_packed_weights():
    torch = pytest.importorskip("torch")
    M, K, N, F = 4, 640, 48, 32
    x = torch.zeros((M, K), dtype=torch.float32)
    g = torch.ones(K, dtype=torch.float32)
    seg = [16, 16, 32]
    cases = [
        (lambda p: tb.hbitlinear_forward(x, N, 8, False, p, 1.0), N),
        (lambda p: tb.hbitlinear_forward_rmsnorm(x, g, 1e-6, N, 8, False, p, 1.0), N),
        (lambda p: tb.hbitlinear_forward_segments(x, seg, 8, False, p, [1.0, 1.0, 1.0]), sum(seg)),
        (lambda p: tb.hbitlinear_forward_swiglu(x, F, 8, False, p, 1.0, 1.0), 2 * F),
        (lambda p: tb.bitnet_ternary_gemm_i32(torch.zeros(M * K, dtype=torch.uint8), M, K, N, 8, p), N),
    ]
    for call, rows in cases:
        need = tb.bitnet_packed_bytes(rows, K)
        with pytest.raises(ValueError, match="packed"):
            call(torch.zeros(need - 1, dtype=torch.uint8))
        # a buffer of the right size passes this check and stops at the device check instead
        with pytest.raises(TypeError):
            call(torch.zeros(need, dtype=torch.uint8))


def test_noalloc_validation_without_launch():
    # checks that fail return before the entry point touches the GPU (no device here)
    L = tb.lib()
    f = ctypes.c_float(1.0)
    assert L.hbitlinear_forward_noalloc(NUL, 4, 256, 64, 8, 1, FAKE, FAKE, f, NUL) == tb.BITNET_ERR_NULL
    assert L.hbitlinear_forward_noalloc(FAKE, 4, 200, 64, 8, 1, FAKE, FAKE, f, NUL) == \
        tb.BITNET_ERR_UNSUPPORTED
    assert L.hbitlinear_forward_noalloc(FAKE, 0, 256, 64, 8, 1, FAKE, FAKE, f, NUL) == tb.BITNET_ERR_SHAPE
    # the workspace limit: 16 MiB of codes and scales
    assert tb.hbitlinear_workspace_bytes(8192, 4096, 4) > tb.NOALLOC_SCRATCH_BYTES
    assert L.hbitlinear_forward_noalloc(FAKE, 8192, 4096, 64, 4, 1, FAKE, FAKE, f, NUL) == \
        tb.BITNET_ERR_WORKSPACE
    assert L.hbitlinear_forward_noalloc(FAKE, 4096, 4096, 64, 8, 0, FAKE, FAKE, f, NUL) == \
        tb.BITNET_ERR_WORKSPACE
    assert tb.hbitlinear_workspace_bytes(4096, 4096, 4) <= tb.NOALLOC_SCRATCH_BYTES


def test_qkv_states_validation():
    L = tb.lib()
    n3 = (ctypes.c_int * 3)(128, 128, 128)
    w3 = (ctypes.c_float * 3)(1.0, 1.0, 1.0)
    b3 = (ctypes.c_int * 3)(4, 3, 3)
    bad_b = (ctypes.c_int * 3)(4, 1, 3)
    odd = (ctypes.c_int * 3)(128, 64, 128)
    args = lambda M=4096, K=4096, S=3, n=n3, act=4, bits=b3, grp=128, sc=FAKE, ws=1 << 30: (
        FAKE, M, K, S, n, act, 0, FAKE, w3, bits, grp, FAKE, sc, FAKE, ws, NUL)
    f = L.hbitlinear_forward_qkv_states
    assert f(*args(sc=NUL)) == tb.BITNET_ERR_NULL
    assert f(*args(grp=32)) == tb.BITNET_ERR_UNSUPPORTED             # group 64 or 128
    assert f(*args(n=odd)) == tb.BITNET_ERR_UNSUPPORTED              # 64 rows: not whole groups
    assert f(*args(bits=bad_b)) == tb.BITNET_ERR_UNSUPPORTED         # 1-bit states
    assert f(*args(act=6)) == tb.BITNET_ERR_UNSUPPORTED              # INT8 or INT4 activations
    # every shape class has the form (batched and decode, INT8 and INT4): these pass the
    # checks and stop at the workspace, before any launch
    for M, act in ((4096, 8), (17, 8), (16, 8), (1, 4)):
        assert f(*args(M=M, act=act, ws=16)) == tb.BITNET_ERR_WORKSPACE
    g = L.hbitlinear_gemm_qkv_states
    assert g(FAKE, FAKE, 4096, 4096, 3, n3, 4, FAKE, w3, b3, 128, NUL, FAKE, NUL) == tb.BITNET_ERR_NULL
    assert g(FAKE, FAKE, 16, 4096, 3, n3, 8, FAKE, w3, b3, 32, FAKE, FAKE, NUL) == \
        tb.BITNET_ERR_UNSUPPORTED
