"""Pins of the CPU oracle to facts the source pages and mathematics fix.

None of these tests re-types the oracle's formulas: each checks the oracle against a printed
example, a closed form, an invariant, a brute-force count or an independent library routine.
"""
import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from conftest import read_golden


# ---------------------------------------------------------------- base-3 byte code ----

def test_worked_example_178():
    g = read_golden("base3_worked_example.txt")
    digits = [int(v) for v in g["digits"]]
    byte = int(g["byte"][0])
    assert oracle.encode5(digits) == byte
    assert format(byte, "08b") == g["binary"][0]
    assert list(oracle.decode5(byte)) == digits
    # least-significant-first order would give a different byte: the example fixes the order
    assert oracle.encode5(digits[::-1]) != byte


def test_storage_efficiency_closed_form():
    g = read_golden("base3_worked_example.txt")
    eff = 5 * math.log2(3) / 8
    assert round(100 * eff, 2) == float(g["efficiency_percent"][0])
    assert 3 ** 5 <= 256                       # five trits fit in a byte
    assert 3 ** 6 > 256                        # six do not
    # 64 bytes per 320 weights: 1.6 bits per weight, 10x less than fp16
    for K in (320, 640, 3200):
        assert oracle.row_bytes(K) * 8 / K == pytest.approx(1.6)
        assert 16 / (oracle.row_bytes(K) * 8 / K) == pytest.approx(10.0)


def test_byte_code_is_bijection_onto_0_242():
    seen = {}
    for a in range(3):
        for b in range(3):
            for c in range(3):
                for d in range(3):
                    for e in range(3):
                        v = oracle.encode5([a, b, c, d, e])
                        assert 0 <= v <= 242
                        assert v not in seen
                        seen[v] = (a, b, c, d, e)
                        assert tuple(oracle.decode5(v)) == (a, b, c, d, e)
    assert len(seen) == 243
    for v in range(243, 256):
        assert oracle.decode5(v) is None
    assert oracle.encode5([3, 0, 0, 0, 0]) == -1


def test_pack_groups_five_weights_per_byte():
    # weights at k = 0, 64, 128, 192, 256 of row 0 share byte 0 (layout reading); with
    # trits (1, -1, 0, 1, 0) = digits (2, 0, 1, 2, 1) that byte is the page's 178.
    K = 320
    t = np.zeros((2, K), np.int8)
    t[0, [0, 64, 128, 192, 256]] = [1, -1, 0, 1, 0]
    p = oracle.pack(t)
    assert p.shape == (128,)                    # two rows of one 64-byte block, row-major
    assert p[0] == 178
    assert np.all(p[1:] == 121)                 # all-zero trits: digits 1,1,1,1,1 = 121
    assert oracle.encode5([1, 1, 1, 1, 1]) == 121


@pytest.mark.parametrize("N,K", [(1, 1), (3, 5), (2, 64), (4, 319), (5, 320), (3, 321),
                                 (7, 1000), (16, 4096), (17, 640), (40, 100)])
def test_pack_roundtrip_and_size(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    p = oracle.pack(t)
    assert p.size == N * 64 * ((K + 319) // 320)
    assert p.max() <= 242
    assert np.array_equal(oracle.unpack(p, N, K), t)


def test_pack_byte_positions_brute_force():
    # every byte decoded by hand (base-3 digits by repeated division) against the trits it
    # should hold: byte b of block B of row n is byte n * row_bytes + 64 B + b and holds
    # k = 320 B + b + 64 i as digit i, most significant first; pad weights are t = 0
    N, K = 3, 700
    rng = np.random.default_rng(5)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    p = oracle.pack(t)
    rb = 64 * 3
    for n in range(N):
        for B in range(3):
            for b in range(64):
                v = int(p[n * rb + 64 * B + b])
                digs = []
                for _ in range(5):
                    digs.append(v % 3)
                    v //= 3
                digs = digs[::-1]
                for i in range(5):
                    k = 320 * B + b + 64 * i
                    assert digs[i] - 1 == (t[n, k] if k < K else 0)
    # the page's byte at a block other than the first
    t = np.zeros((N, K), np.int8)
    t[2, [330, 394, 458, 522, 586]] = [1, -1, 0, 1, 0]       # block 1, byte 10, row 2
    p = oracle.pack(t)
    assert p[2 * rb + 64 + 10] == 178
    assert np.count_nonzero(p != 121) == 1


def test_unpack_rejects_bad_bytes():
    t = np.zeros((1, 10), np.int8)
    p = oracle.pack(t)
    p2 = p.copy(); p2[3] = 243
    with pytest.raises(ValueError):
        oracle.unpack(p2, 1, 10)
    p3 = p.copy(); p3[20] = 0                    # a padding position holding t = -1
    with pytest.raises(ValueError):
        oracle.unpack(p3, 1, 10)


# ------------------------------------------------------------- absmean ternarisation ----

def test_ternary_values_and_exact_mean():
    W = si.gaussian_weights(1, 64, 333)
    t, g = oracle.ternarize(W)
    assert set(np.unique(t)).issubset({-1, 0, 1})
    exact = math.fsum(abs(float(v)) for v in W.ravel()) / W.size
    assert g == np.float32(exact)


def test_ternarize_scale_invariance():
    W = si.gaussian_weights(2, 32, 128)
    t, g = oracle.ternarize(W)
    for e in (-3, 1, 7):
        t2, g2 = oracle.ternarize(W * np.float32(2.0 ** e))
        assert np.array_equal(t, t2)
        assert g2 == np.float32(g * 2.0 ** e)


def test_ternarize_zero_matrix():
    t, g = oracle.ternarize(np.zeros((3, 7), np.float32))
    assert g == 0 and not t.any()


def test_ternarize_brute_force_thresholds():
    # t = +1 above gamma/2, -1 below -gamma/2, 0 inside; checked in exact arithmetic away from
    # the two boundaries (rounding of the fp32 quotient can only matter within an ulp of them)
    W = si.gaussian_weights(3, 40, 50)
    t, g = oracle.ternarize(W)
    r = W.astype(np.float64) / float(g)
    far = np.abs(np.abs(r) - 0.5) > 1e-6
    expect = np.where(r > 0.5, 1, np.where(r < -0.5, -1, 0))
    assert np.array_equal(t[far], expect[far])
    # large ratios clip to +-1
    W2 = W.copy(); W2[0, 0] = 100 * g; W2[0, 1] = -100 * g
    t2, _ = oracle.ternarize(W2)
    assert t2[0, 0] == 1 and t2[0, 1] == -1


def test_gaussian_zero_fraction_closed_form():
    # For W ~ N(0, s^2): gamma = s sqrt(2/pi); P(t = 0) = P(|Z| < sqrt(2/pi)/2) = 2 Phi(.) - 1
    W = si.gaussian_weights(2, 4096, 4096)
    t, _ = oracle.ternarize(W)
    frac = float(np.mean(t == 0))
    c = 0.5 * math.sqrt(2.0 / math.pi)
    expect = math.erf(c / math.sqrt(2.0))
    assert abs(expect - 0.3101) < 1e-4
    assert abs(frac - expect) < 2e-3
    # and the signs are balanced
    assert abs(float(np.mean(t == 1)) - float(np.mean(t == -1))) < 2e-3


# -------------------------------------------------------------- Hadamard transform ----

def _sylvester(n):
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_hadamard_entries_and_orthogonality_dense():
    g = read_golden("hadamard_definition.txt")
    for n in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        rows = oracle.fwht(np.eye(n, dtype=np.float32)).astype(np.int64)
        assert set(np.unique(rows)).issubset({int(v) for v in g["entries"]})
        gram = rows @ rows.T
        assert np.array_equal(gram, n * np.eye(n, dtype=np.int64))
        # Sylvester closed form H[i][j] = (-1)^popcount(i & j)
        i = np.arange(n)[:, None]; j = np.arange(n)[None, :]
        pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
        assert np.array_equal(rows, np.where(pc % 2 == 0, 1, -1))


def test_fwht_equals_dense_matmul_small():
    rng = np.random.default_rng(5)
    for n in (2, 4, 8, 16, 32, 64):
        x = rng.integers(-50, 51, size=(9, n)).astype(np.float32)
        dense = x.astype(np.int64) @ _sylvester(n)
        assert np.array_equal(oracle.fwht(x), dense.astype(np.float32))
        # normalised: one fp32 multiply by the rounded 1/sqrt(n)
        c = np.float32(1.0 / math.sqrt(n))
        assert oracle.hadamard_scale(n) == c
        assert np.array_equal(oracle.hadamard(x), dense.astype(np.float32) * c)


@pytest.mark.parametrize("n", [2 ** p for p in range(1, 15)])
def test_h_ht_equals_n_identity(n):
    # H H^T = n I, checked column by column as FWHT(FWHT(e_j)) = n e_j (exact integers)
    for j in sorted({0, 1, n // 3, n // 2, n - 1}):
        e = np.zeros(n, np.float32); e[j] = 1
        r = oracle.fwht(oracle.fwht(e))
        expect = np.zeros(n, np.float32); expect[j] = n
        assert np.array_equal(r, expect)


def test_normalised_transform_is_involution():
    rng = np.random.default_rng(7)
    for n in (4, 16, 64, 256, 1024, 4096, 16384):     # n = 4^k: 1/sqrt(n) is a power of two
        x = rng.integers(-100, 101, size=(2, n)).astype(np.float32)
        assert np.array_equal(oracle.hadamard(oracle.hadamard(x)), x)
    for n in (2, 8, 32, 512, 8192):                    # otherwise within a few ulp
        x = rng.standard_normal((2, n)).astype(np.float32)
        back = oracle.hadamard(oracle.hadamard(x))
        assert np.max(np.abs(back - x)) <= 8 * np.finfo(np.float32).eps * np.max(np.abs(x)) * math.log2(n)


def test_parseval_and_fp64_error_bound():
    rng = np.random.default_rng(9)
    for n in (256, 4096, 16384):
        x = rng.standard_normal((3, n)).astype(np.float32)
        y = oracle.hadamard(x)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
        exact = oracle.fwht_f64(x.astype(np.float64)) / math.sqrt(n)
        # each output is a sum of n terms formed by log2(n) rounded additions
        bound = (math.log2(n) + 2) * np.finfo(np.float32).eps * np.sum(np.abs(x), axis=1, keepdims=True) / math.sqrt(n)
        assert np.all(np.abs(y - exact) <= bound)


def test_spike_is_spread_flat():
    # a single outlier channel c e_j maps to a vector whose entries all have magnitude c/sqrt(n)
    for n in (256, 4096, 16384):
        for j in (0, 3, n - 1):
            x = np.zeros(n, np.float32); x[j] = 40.0
            y = oracle.hadamard(x)
            assert np.all(np.abs(y) == np.float32(40.0 / math.sqrt(n)))


# --------------------------------------------------------------- absmax quantisation ----

@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_closed_forms(bits):
    qp = 2 ** (bits - 1) - 1
    x = si.wo_activations(8, 4096)
    for row in x:
        q, s = oracle.quantize_row(row, bits)
        g = np.max(np.abs(row))
        assert s == np.float32(g / np.float32(qp))
        imax = int(np.argmax(np.abs(row)))
        assert q[imax] == (qp if row[imax] > 0 else -qp)
        assert q.min() >= -qp - 1 and q.max() <= qp
        err = np.abs(row.astype(np.float64) - float(s) * q.astype(np.float64))
        assert np.all(err <= 0.5 * float(s) * (1 + 1e-5))


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_integer_grid_is_lossless(bits):
    qp = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(bits)
    x = rng.integers(-qp, qp + 1, size=(6, 512)).astype(np.float32)
    x[:, 17] = qp                                        # row max is exactly Qp
    q, s = oracle.quantize(x, bits, False)
    assert np.all(s == 1.0)
    assert np.array_equal(q.astype(np.float32), x)


def test_quantize_zero_row_and_sign_symmetry():
    x = np.zeros((2, 64), np.float32)
    x[1] = np.linspace(-3, 3, 64)
    q, s = oracle.quantize(x, 8, False)
    assert s[0] == 0 and not q[0].any()
    qn, sn = oracle.quantize(-x, 8, False)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def test_int4_nibble_layout():
    q = np.array([[1, -1, 7, -8, 0, 3, -2, 5]], np.int8)
    b = oracle.pack_int4(q)
    # byte p holds code p (low nibble) and code p + 4 (high nibble)
    assert list(b[0]) == [0x01, 0x3F, 0xE7, 0x58]
    assert np.array_equal(oracle.unpack_int4(b, 8), q)
    rng = np.random.default_rng(3)
    q2 = rng.integers(-8, 8, size=(3, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q2), 64), q2)


# ------------------------------------------------------------------- ternary product ----

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (16, 33, 320), (5, 8, 1000)])
def test_add_sub_skip_equals_integer_matmul(M, N, K):
    rng = np.random.default_rng(M + N + K)
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    acc = oracle.gemm(q, t)
    assert np.array_equal(acc, q.astype(np.int64) @ t.astype(np.int64).T)


def test_gemm_extremes():
    K = 16384
    q = np.full((1, K), -128, np.int8)
    t = np.full((2, K), 1, np.int8); t[1] = -1
    acc = oracle.gemm(q, t)
    assert acc[0, 0] == -128 * K and acc[0, 1] == 128 * K


# ----------------------------------------------------------------------- end to end ----

def test_forward_integer_grid_without_hadamard():
    # x on the integer grid with row max Qp: s = 1 exactly, so y = gamma_w * (x t^T) exactly
    rng = np.random.default_rng(11)
    M, K, N = 4, 640, 24
    x = rng.integers(-127, 128, size=(M, K)).astype(np.float32); x[:, 0] = 127
    W = si.gaussian_weights(1, N, K)
    packed, gw, t = oracle.pack_weights(W)
    y = oracle.forward(x, packed, gw, N, 8, False)
    exact = (x.astype(np.int64) @ t.astype(np.int64).T).astype(np.float32) * gw
    assert np.array_equal(y, exact)


@pytest.mark.parametrize("bits", [8, 4])
def test_forward_hadamard_row_closed_form(bits):
    # x = a * H[j, :]: the normalised transform gives a sqrt(K) e_j, the code is +-Qp at j,
    # the scale a sqrt(K) / Qp, so y[n] = a sqrt(K) t[n, j] gamma_w
    K, N = 1024, 40
    H = oracle.fwht(np.eye(K, dtype=np.float32))
    W = si.gaussian_weights(4, N, K)
    packed, gw, t = oracle.pack_weights(W)
    for j, a in ((0, 0.75), (5, -1.5), (K - 1, 3.0)):
        x = (np.float32(a) * H[j])[None, :]
        y = oracle.forward(x, packed, gw, N, bits, True)
        expect = a * math.sqrt(K) * t[:, j].astype(np.float64) * float(gw)
        assert np.allclose(y[0], expect, rtol=1e-6, atol=0)


def test_forward_is_composition_of_stages():
    lin = si.workload(1).linears[0]
    x = si.activations(1, lin)
    W = si.weights(1, lin)
    packed, gw, t = oracle.pack_weights(W)
    y = oracle.forward(x, packed, gw, lin.N, lin.act_bits, lin.use_hadamard)
    q, s = oracle.quantize(x, lin.act_bits, lin.use_hadamard)
    y2 = oracle.epilogue(oracle.gemm(q, t), s, gw)
    assert np.array_equal(y, y2)
    # the Hadamard spreads the 4 outlier channels: the transformed row is flatter
    xh = oracle.hadamard(x)
    kurt = lambda v: np.mean(v ** 4, axis=1) / np.mean(v ** 2, axis=1) ** 2
    assert np.all(kurt(xh) < kurt(x))


# ------------------------------------------------------- several linears, one input ----

def test_forward_segments_hadamard_row_closed_form():
    # Three linears with their own weights and scales on x = a * H[j, :]: each segment's
    # columns follow the single-linear closed form a sqrt(K) t_s[n, j] gamma_s.
    K = 1024
    seg_n = [48, 16, 32]
    H = oracle.fwht(np.eye(K, dtype=np.float32))
    packs, gammas, ts = [], [], []
    for s, n in enumerate(seg_n):
        packed, g, t = oracle.pack_weights(si.gaussian_weights(6, n, K, layer=s, std=0.02 * (s + 1)))
        packs.append(packed); gammas.append(g); ts.append(t)
    assert len(set(float(g) for g in gammas)) == 3
    for j, a in ((3, 1.25), (K - 2, -0.5)):
        x = (np.float32(a) * H[j])[None, :]
        y = oracle.forward_segments(x, packs, gammas, seg_n, 4, True)
        assert y.shape == (1, sum(seg_n))
        expect = np.concatenate([a * math.sqrt(K) * t[:, j].astype(np.float64) * float(g)
                                 for t, g in zip(ts, gammas)])
        assert np.allclose(y[0], expect, rtol=1e-6, atol=0)


def test_forward_segments_integer_grid_exact():
    # integer-grid input (s = 1): every segment is gamma_s * (x t_s^T) exactly, in its columns
    rng = np.random.default_rng(12)
    M, K = 3, 640
    x = rng.integers(-127, 128, size=(M, K)).astype(np.float32); x[:, 7] = -127
    seg_n = [16, 40]
    packs, gammas, ts = [], [], []
    for s, n in enumerate(seg_n):
        packed, g, t = oracle.pack_weights(si.gaussian_weights(7, n, K, layer=s))
        packs.append(packed); gammas.append(g); ts.append(t)
    y = oracle.forward_segments(x, packs, gammas, seg_n, 8, False)
    exact = np.concatenate([(x.astype(np.int64) @ t.astype(np.int64).T).astype(np.float32) * g
                            for t, g in zip(ts, gammas)], axis=1)
    assert np.array_equal(y, exact)


# ------------------------------------------------------------------ SwishGLU glue ----

def test_silu_textbook_values_and_identities():
    # SiLU(z) = z sigmoid(z): SiLU(0) = 0, SiLU(1) = sigmoid(1) = 1 / (1 + 1/e)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == np.float32(1.0 / (1.0 + math.exp(-1.0)))
    assert abs(float(oracle.silu(1.0)) - 0.7310585786300049) < 1e-7
    # SiLU(z) - SiLU(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    for z in np.linspace(-12, 12, 97):
        d = float(oracle.silu(z)) - float(oracle.silu(-z))
        assert abs(d - float(np.float32(z))) <= 4e-7 * max(1.0, abs(z))
    # tails: -> z for large z, -> 0 from below for very negative z
    assert oracle.silu(40.0) == np.float32(40.0)
    assert -1e-15 < float(oracle.silu(-40.0)) < 0.0


def test_silu_minimum_is_lambert_w():
    # d/dz z sigmoid(z) = 0 at z* = -(1 + W(1/e)); the minimum value is z* + 1 = -W(1/e)
    from scipy.special import lambertw
    w = float(lambertw(1.0 / math.e).real)
    zs = np.linspace(-1.35, -1.2, 30001).astype(np.float32)
    vals = np.array([float(oracle.silu(z)) for z in zs])
    i = int(np.argmin(vals))
    # near z* the curve is flat to within fp32 resolution of the values (f'' ~ 0.2, an ulp of
    # 0.28 is 3e-8), so the location is pinned to about 1e-3 and the value to 1e-7
    assert abs(float(zs[i]) + 1.0 + w) < 1e-3
    assert abs(vals[i] + w) < 1e-7


def test_swiglu_elementwise_matches_definition_and_zeros():
    rng = np.random.default_rng(13)
    g = rng.normal(0, 3, size=(5, 64)).astype(np.float32)
    u = rng.normal(0, 2, size=(5, 64)).astype(np.float32)
    h = oracle.swiglu(g, u)
    gd = g.astype(np.float64)
    ref = (gd / (1.0 + np.exp(-gd)) * u.astype(np.float64)).astype(np.float32)
    assert np.array_equal(h, ref)
    assert np.all(oracle.swiglu(np.zeros_like(g), u) == 0)
    assert np.all(oracle.swiglu(g, np.zeros_like(u)) == 0)


@pytest.mark.parametrize("bits", [8, 4])
def test_forward_swiglu_hadamard_row_closed_form(bits):
    # x = a * H[j, :]: gate and up each follow the single-linear closed form, so
    # h[n] = SiLU(a sqrt(K) t_g[n, j] gamma_g) * a sqrt(K) t_u[n, j] gamma_u
    K, F = 1024, 48
    H = oracle.fwht(np.eye(K, dtype=np.float32))
    pg, gg, tg = oracle.pack_weights(si.gaussian_weights(8, F, K, layer=0))
    pu, gu, tu = oracle.pack_weights(si.gaussian_weights(8, F, K, layer=1, std=0.05))
    for j, a in ((1, 0.5), (K - 3, -2.0)):
        x = (np.float32(a) * H[j])[None, :]
        h = oracle.forward_swiglu(x, pg, gg, pu, gu, F, bits, True)
        gv = a * math.sqrt(K) * tg[:, j].astype(np.float64) * float(gg)
        uv = a * math.sqrt(K) * tu[:, j].astype(np.float64) * float(gu)
        expect = gv / (1.0 + np.exp(-gv)) * uv
        assert np.allclose(h[0], expect, rtol=1e-6, atol=1e-12)


def test_forward_swiglu_zero_gate_or_up_gives_zero():
    rng = np.random.default_rng(14)
    M, K, F = 4, 512, 32
    x = rng.normal(size=(M, K)).astype(np.float32)
    pz, gz, _ = oracle.pack_weights(np.zeros((F, K), np.float32))
    pw, gw, _ = oracle.pack_weights(si.gaussian_weights(9, F, K))
    assert gz == 0
    assert np.all(oracle.forward_swiglu(x, pz, gz, pw, gw, F, 8, True) == 0)
    assert np.all(oracle.forward_swiglu(x, pw, gw, pz, gz, F, 8, True) == 0)


# ------------------------------------------------------------------- RMS normalisation ----

def test_rmsnorm_constant_rows_power_of_two():
    # x = c (c a power of two), eps = 0: r = 1/|c| exactly, so y = sign(c) exactly
    K = 512
    ones = np.ones(K, np.float32)
    for c in (4.0, -0.125, 1024.0):
        y = oracle.rmsnorm(np.full((1, K), c, np.float32), ones, 0.0)
        assert np.all(y == np.float32(math.copysign(1.0, c)))


def test_rmsnorm_unit_rms_and_exact_power_of_two_invariance():
    x = si.wo_activations(6, 1024)
    ones = np.ones(1024, np.float32)
    y = oracle.rmsnorm(x, ones, 0.0)
    assert np.allclose(np.mean(y.astype(np.float64) ** 2, axis=1), 1.0, rtol=1e-6, atol=0)
    for p in (-7, 5):
        assert np.array_equal(oracle.rmsnorm(x * np.float32(2.0 ** p), ones, 0.0), y)


def test_rmsnorm_spike_closed_form_and_eps():
    K, j, a = 2048, 77, np.float32(-3.5)
    x = np.zeros((1, K), np.float32); x[0, j] = a
    g = si.normal(si.seed_for(1, 9), K, 1.0, 0.1)
    for eps in (0.0, 1e-6, 0.25):
        y = oracle.rmsnorm(x, g, eps)
        r = 1.0 / math.sqrt(float(a) ** 2 / K + eps)
        assert abs(float(y[0, j]) - float(a) * r * float(g[j])) <= 2e-7 * abs(float(a) * r * float(g[j]))
        assert np.count_nonzero(y) == 1
        # the fp32 scale is the double formula rounded once
        assert oracle.rms_scale(x[0], eps) == np.float32(r)


def test_rmsnorm_zero_rows_and_gain_factor():
    K = 256
    g = si.normal(si.seed_for(1, 10), K, 1.0, 0.2)
    z = np.zeros((2, K), np.float32)
    assert np.all(oracle.rmsnorm(z, g, 0.0) == 0) and np.all(oracle.rmsnorm(z, g, 1e-5) == 0)
    x = si.gaussian_activations(1, 3, K)
    # y(x, g) = y(x, 1) * g elementwise, exactly: (x r) g vs ((x r) 1) g
    assert np.array_equal(oracle.rmsnorm(x, g, 1e-6),
                          oracle.rmsnorm(x, np.ones(K, np.float32), 1e-6) * g)


def test_forward_rmsnorm_is_norm_then_forward():
    rng = np.random.default_rng(21)
    M, K, N = 5, 1024, 48
    x = rng.normal(0, 3, size=(M, K)).astype(np.float32)
    g = si.normal(si.seed_for(1, 11), K, 1.0, 0.1)
    packed, gw, t = oracle.pack_weights(si.gaussian_weights(12, N, K))
    y = oracle.forward_rmsnorm(x, g, 1e-6, packed, gw, N, 4, True)
    assert np.array_equal(y, oracle.forward(oracle.rmsnorm(x, g, 1e-6), packed, gw, N, 4, True))


# ------------------------------------------------- weight + activation Hadamard variant ----

def test_rotate_weights_equals_dense_sylvester_product():
    # W H / sqrt(K) against the dense Sylvester matrix in float64 (an independent product)
    for K in (8, 64, 256):
        W = si.gaussian_weights(13, 5, K)
        H = _sylvester(K).astype(np.float64)
        ref = (W.astype(np.float64) @ H) / math.sqrt(K)
        Wh = oracle.rotate_weights(W)
        assert np.allclose(Wh, ref, rtol=0, atol=1e-7 * np.max(np.abs(ref)))
        # fp32 rounding of the double result: within half an ulp of it, up to the double's error
        assert np.all(np.abs(Wh.astype(np.float64) - ref) <= np.spacing(np.abs(ref).astype(np.float32)) * 0.5 + 1e-15)


def test_rotate_weights_is_orthogonal_and_an_involution():
    W = si.gaussian_weights(14, 7, 1024)
    Wh = oracle.rotate_weights(W)
    assert np.allclose(np.linalg.norm(Wh.astype(np.float64), axis=1),
                       np.linalg.norm(W.astype(np.float64), axis=1), rtol=1e-6)
    back = oracle.rotate_weights(Wh)
    assert np.max(np.abs(back - W)) <= 4 * np.max(np.spacing(np.abs(W)))


def test_rotated_product_preserves_x_w_before_quantisation():
    # x_h W_h^T = x W^T: the rotation of both operands cancels (orthogonal H / sqrt(K))
    K = 512
    x = si.gaussian_activations(1, 4, K)
    W = si.gaussian_weights(15, 9, K)
    xh = oracle.hadamard(x).astype(np.float64)
    Wh = oracle.rotate_weights(W).astype(np.float64)
    assert np.allclose(xh @ Wh.T, x.astype(np.float64) @ W.astype(np.float64).T, rtol=1e-5, atol=1e-5)


def test_pack_weights_hadamard_is_rotate_then_pack():
    W = si.gaussian_weights(16, 32, 1024)
    packed, g = oracle.pack_weights_hadamard(W)
    p2, g2, _ = oracle.pack_weights(oracle.rotate_weights(W))
    assert g == g2 and np.array_equal(packed, p2)
    # a row that is a scaled Hadamard row rotates to a spike: one +-1 trit, the rest 0
    K = 256
    H = oracle.fwht(np.eye(K, dtype=np.float32))
    Wr = np.zeros((16, K), np.float32)
    for n in range(16):
        Wr[n] = H[3 * n + 1] * np.float32(0.5)
    t = oracle.unpack(oracle.pack_weights_hadamard(Wr)[0], 16, K)
    for n in range(16):
        assert np.count_nonzero(t[n]) == 1 and t[n, 3 * n + 1] == 1


# ------------------------------------------------------------ low-bit Q/K/V states ----

def _nearest_in_range(v, qp):
    """Brute force: the integer in [-qp-1, qp] nearest to v, ties to the even one."""
    cands = np.arange(-qp - 1, qp + 1)
    d = np.abs(cands - float(v))
    best = cands[d == d.min()]
    return int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])


@pytest.mark.parametrize("b", [3, 4, 8])
def test_states_integer_grid_is_lossless(b):
    # a group on the integer grid whose largest magnitude is Qp: inv = 1, scale = 1, q = y
    qp = 2 ** (b - 1) - 1
    rng = np.random.default_rng(b)
    group = 32
    y = rng.integers(-qp, qp + 1, size=(5, 3 * group)).astype(np.float32)
    y[:, ::group] = qp
    codes, scales = oracle.quantize_states(y, [group, 2 * group], [b, b], group)
    assert np.array_equal(codes, y.astype(np.int8))
    assert np.all(scales == 1.0)


@pytest.mark.parametrize("bits", [(3, 3, 3), (4, 3, 3), (8, 3, 3)])
def test_states_group_max_bound_and_brute_force(bits):
    seg_n, group = [128, 128, 256], 64
    rng = np.random.default_rng(sum(bits))
    y = (rng.standard_normal((6, 512)) * rng.uniform(0.1, 30, size=(6, 1))).astype(np.float32)
    y[2, 128:192] = 0.0                       # one all-zero group: codes 0, scale 0
    codes, scales = oracle.quantize_states(y, seg_n, bits, group)
    seg_of_col = np.repeat(np.arange(3), seg_n)
    for m in range(6):
        for j in range(512 // group):
            cols = slice(j * group, (j + 1) * group)
            qp = 2 ** (bits[seg_of_col[j * group]] - 1) - 1
            g = np.float32(np.max(np.abs(y[m, cols])))
            q, s = codes[m, cols].astype(np.int64), scales[m, j]
            if g == 0:
                assert not np.any(q) and s == 0.0
                continue
            # the group's largest magnitude lands on +-Qp; -Qp-1 is never used; the scale is
            # gamma / Qp
            k = int(np.argmax(np.abs(y[m, cols])))
            assert abs(q[k]) == qp and q.min() >= -qp
            assert s == np.float32(g / np.float32(qp))
            # each code is the in-range integer nearest to y * (Qp / gamma), found by search
            inv = np.float32(qp) / g
            for i in range(0, group, 7):
                assert q[i] == _nearest_in_range(np.float32(y[m, j * group + i] * inv), qp)
            # and dequantises within half a step
            assert np.all(np.abs(y[m, cols].astype(np.float64) - s * q) <= 0.5 * s * (1 + 1e-6))


def test_states_groups_are_independent_and_scale_exactly():
    group = 16
    rng = np.random.default_rng(3)
    y = rng.standard_normal((3, 96)).astype(np.float32)
    c0, s0 = oracle.quantize_states(y, [32, 64], [3, 4], group)
    y2 = y.copy()
    y2[:, 16:32] *= np.float32(8.0)           # a power of two: codes kept, scale x8 exactly
    y2[:, 64:80] = rng.standard_normal((3, 16)).astype(np.float32)   # another group replaced
    c2, s2 = oracle.quantize_states(y2, [32, 64], [3, 4], group)
    assert np.array_equal(c2[:, 16:32], c0[:, 16:32]) and np.array_equal(s2[:, 1], 8 * s0[:, 1])
    keep = np.r_[0:16, 32:64, 80:96]
    assert np.array_equal(c2[:, keep], c0[:, keep])
    assert np.array_equal(s2[:, [0, 2, 3, 5]], s0[:, [0, 2, 3, 5]])


@pytest.mark.parametrize("act", [4, 8])
def test_forward_qkv_states_hadamard_row_closed_form(act):
    # x = a * H[j, :]: each projection's output is a sqrt(K) t_s[n, j] gamma_s (values 0 and
    # +-gamma) with INT4 or INT8 activations alike (the transformed row is a spike, coded +-Qp),
    # so every group that holds a non-zero trit quantises to q = sign(a) Qp t_s[n, j] with
    # scale |a| sqrt(K) gamma_s / Qp; a group of zero trits gives codes 0, scale 0
    K, group = 512, 32
    seg_n, bits = [64, 32, 96], [4, 3, 3]
    H = oracle.fwht(np.eye(K, dtype=np.float32))
    packs, gammas, ts = [], [], []
    for s, n in enumerate(seg_n):
        p, g, t = oracle.pack_weights(si.gaussian_weights(13, n, K, layer=s, std=0.01 * (s + 1)))
        packs.append(p); gammas.append(g); ts.append(t)
    for j, a in ((3, 1.25), (K - 2, -0.5)):
        x = (np.float32(a) * H[j])[None, :]
        codes, scales = oracle.forward_qkv_states(x, packs, gammas, seg_n, act, True, bits, group)
        col = 0
        for s, n in enumerate(seg_n):
            qp = 2 ** (bits[s] - 1) - 1
            tj = ts[s][:, j].astype(np.int64)
            assert np.array_equal(codes[0, col:col + n], (np.sign(a) * qp * tj).astype(np.int8))
            for gi in range(n // group):
                sc = scales[0, (col + gi * group) // group]
                if np.any(tj[gi * group:(gi + 1) * group]):
                    assert sc == pytest.approx(abs(a) * math.sqrt(K) * float(gammas[s]) / qp, rel=1e-6)
                else:
                    assert sc == 0.0
            col += n
