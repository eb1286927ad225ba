"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded synthetic inputs.

Tolerances:
  - post-Hadamard fp32 values: bit-identical (the kernel runs the oracle's butterfly order and
    its single multiply by fp32(1/sqrt(K))); with the RMS norm in front, rows whose fp32 r
    matches are bit-identical and any other row within 1e-5 of its absmax;
  - codes: at most 1e-4 of them differ, each by exactly 1;
  - int32 products: bit-exact when both sides get the same codes;
  - outputs: rows whose codes match are bit-exact, all rows within 1e-3 relative (elementwise,
    against max(|y_ref|, 1e-3 * row max)); rows with a code difference are checked exactly
    against the oracle's product and epilogue run on the GPU's own codes.
"""
import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from packed_layout import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tb():
    import ternary_weight_bit_bitlinear_amd as m
    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(*a):
    print(*a, flush=True)


def codes_to_int8(codes_u8, M, K, bits):
    c = codes_u8.cpu().numpy()
    if bits == 8:
        return c.view(np.int8).reshape(M, K)
    return oracle.unpack_int4(c.reshape(M, K // 2), K)


def check_quant(tb, x, bits, had, rows=None, label=""):
    """Run the GPU activation stage on x (all rows); compare the sampled rows with the oracle.
    Returns the GPU codes (int8, sampled rows) and whether they equal the oracle's."""
    M, K = x.shape
    xd = dev(x)
    codes, scales, xh = tb.hbitlinear_quantize(xd, bits, had, want_xh=True)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else np.asarray(rows)
    oq, os_, oxh = oracle.quantize(x[rows], bits, had, want_xh=True)
    gxh = xh.cpu().numpy()[rows]
    gs = scales.cpu().numpy()[rows]
    gq = codes_to_int8(codes, M, K, bits)[rows]
    amax = np.maximum(np.max(np.abs(oxh), axis=1, keepdims=True), 1e-30)
    rel = float(np.max(np.abs(gxh - oxh) / amax))
    np.testing.assert_array_equal(gxh, oxh, err_msg=f"{label}: post-Hadamard values differ")
    diff = gq.astype(np.int32) - oq.astype(np.int32)
    nd = int(np.count_nonzero(diff))
    assert nd <= 1e-4 * diff.size, f"{label} {nd} codes differ"
    assert np.all(np.abs(diff) <= 1)
    same_codes = nd == 0
    if same_codes:
        np.testing.assert_array_equal(gs, os_)
    else:
        assert np.allclose(gs, os_, rtol=1e-5, atol=0)
    say(f"  {label}: xh rel {rel:.2e}, codes differing {nd}/{diff.size}")
    return gq, gs, same_codes


# ---------------------------------------------------------------- activation stage ----

@pytest.mark.parametrize("K", [256, 512, 1024, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("had", [True, False])
def test_quantize_all_widths(tb, K, bits, had):
    M = 7
    x = si.normal(si.seed_for(1, 7) + K, M * K).reshape(M, K)
    x[2] = 0.0                       # zero row: codes 0, scale 0
    x[3] = 0.0; x[3, K // 3] = 5.0   # single spike
    x[4, 5] *= 40.0                  # outlier channel
    check_quant(tb, x, bits, had, label=f"K={K} bits={bits} had={had}")


# Many rows: more workgroups than the chip holds at once at every width (at most 160 KB / 4K
# bytes of LDS per workgroup with the transform, 256 CUs), row counts that are not multiples of
# anything the launch uses; sampled rows, including the first and last, against the oracle.
@pytest.mark.parametrize("M,K,bits,had", [(7757, 4096, 4, True), (7757, 4096, 8, False),
                                          (3001, 8192, 8, True), (1500, 16384, 4, True)])
def test_quantize_many_rows(tb, M, K, bits, had):
    x = si.wo_activations(M, K)
    x[M - 1] = 0.0                    # last row zero: codes 0, scale 0
    rng = np.random.default_rng(M + K)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), rng.choice(M, 48, replace=False)]))
    check_quant(tb, x, bits, had, rows=rows, label=f"many rows M={M} K={K} bits={bits} had={had}")


@pytest.mark.parametrize("K", [64, 320, 960, 4032])
@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_generic_widths(tb, K, bits):
    x = si.normal(si.seed_for(1, 8) + K, 9 * K).reshape(9, K)
    x[1] = 0.0
    check_quant(tb, x, bits, False, label=f"generic K={K} bits={bits}")


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_rounding_ties(tb, bits):
    # integer-grid rows with max Qp: inv = 1, so x + 0.5 values sit exactly on ties
    qp = 2 ** (bits - 1) - 1
    K = 512
    rng = np.random.default_rng(bits)
    x = rng.integers(-qp, qp, size=(6, K)).astype(np.float32) + np.float32(0.5)
    x[:, 0] = qp
    gq, gs, same = check_quant(tb, x, bits, False, label="ties")
    assert same
    assert np.all(gs == 1.0)


# ------------------------------------------------------------------ ternary product ----

GEMM_SHAPES = [(16, 256, 256), (1, 64, 64), (300, 200, 1024), (257, 513, 4096), (64, 64, 320),
               (33, 17, 960), (512, 256, 16384), (5, 1000, 4032),
               # large-M INT4 control flow: two blocks (one loop iteration, no remainder block)
               # over two ragged M-tiles and N-tiles; one padded block at M just above 16
               (520, 130, 640), (17, 16, 64),
               # 17 x 17 = 289 tiles of 512 x 128, more than one round of the CUs: the INT4
               # kernel's tile order by XCD runs, over a tile count that is not a multiple of 8
               (8193, 2176, 640)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_i32_bit_exact(tb, M, N, K, bits):
    say(f"  gemm M={M} N={N} K={K} bits={bits}")
    qp = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(M * 7 + N * 3 + K + bits)
    q = rng.integers(-qp - 1, qp + 1, size=(M, K)).astype(np.int8)
    W = si.gaussian_weights(2, N, K, layer=M % 5)
    packed, g = tb.bitnet_pack_weights(W)
    t, _ = oracle.ternarize(W)
    cb = q.view(np.uint8) if bits == 8 else oracle.pack_int4(q)
    acc = tb.bitnet_ternary_gemm_i32(dev(cb.reshape(-1)), M, K, N, bits, dev(packed))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), oracle.gemm(q, t))


def test_gemm_extreme_sums(tb):
    # |acc| reaches 128 * 16384 = 2^21: every code -128, every weight +1 or -1
    M, N, K = 3, 64, 16384
    q = np.full((M, K), -128, np.int8)
    W = np.ones((N, K), np.float32)
    W[1::2] = -1.0
    packed, _ = tb.bitnet_pack_weights(W)
    acc = tb.bitnet_ternary_gemm_i32(dev(q.view(np.uint8).reshape(-1)), M, K, N, 8, dev(packed))
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    assert np.all(a[:, 0::2] == -128 * K) and np.all(a[:, 1::2] == 128 * K)


# ------------------------------------------------------------------------ forward ----

_cache = {}


def linear_inputs(config, idx=0, M=None):
    key = (config, idx, M)
    if key not in _cache:
        wl = si.workload(config, M)
        lin = wl.linears[idx]
        x = si.activations(config, lin)
        W = si.weights(config, lin)
        _cache.clear()
        _cache[key] = (lin, x, W)
    return _cache[key]


def check_forward(tb, lin, x, W, rows, label):
    M, K, N = lin.M, lin.K, lin.N
    packed, g = tb.bitnet_pack_weights(W)
    opacked, og, t = oracle.pack_weights(W)
    assert np.array_equal(packed, to_device(opacked, N, K)) and np.float32(g) == og
    xd = dev(x)
    pd = dev(packed)
    y = tb.hbitlinear_forward(xd, N, lin.act_bits, lin.use_hadamard, pd, g)
    # the stage exports on the same input, for the codes the forward used
    codes, scales = tb.hbitlinear_quantize(xd, lin.act_bits, lin.use_hadamard)
    torch.cuda.synchronize()
    rows = np.asarray(rows)
    gy = y.cpu().numpy()[rows]
    gq = codes_to_int8(codes, M, K, lin.act_bits)[rows]
    gs = scales.cpu().numpy()[rows]
    del y, codes, scales, xd
    xs = x[rows]
    oy = oracle.forward(xs, opacked, og, N, lin.act_bits, lin.use_hadamard)
    oq, os_ = oracle.quantize(xs, lin.act_bits, lin.use_hadamard)
    match = np.all(gq == oq, axis=1)
    # rows with identical codes: bit-exact
    np.testing.assert_array_equal(gy[match], oy[match])
    # every row: 1e-3 relative
    scale = np.maximum(np.abs(oy), 1e-3 * np.max(np.abs(oy), axis=1, keepdims=True))
    assert np.all(np.abs(gy - oy) <= 1e-3 * scale + 0.0), f"{label}: relative error above 1e-3"
    # rows with a code difference: exact against the oracle fed the GPU's codes
    if not np.all(match):
        y2 = oracle.epilogue(oracle.gemm(gq[~match], t), gs[~match], og)
        np.testing.assert_array_equal(gy[~match], y2)
    say(f"  {label}: {int(np.sum(match))}/{len(rows)} sampled rows with identical codes")


def sample_rows(M, n, seed):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    r = np.sort(rng.choice(M, size=n - 2, replace=False))
    return np.unique(np.concatenate([[0], r, [M - 1]]))


def tile_rows(M, seed, tile=512):
    """One random row in every `tile`-row M-tile of the large-M INT4 kernel, and every row of
    the last tile (the grid's tail)."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, tile)
    picks = [s + int(rng.integers(0, min(tile, M - s))) for s in starts]
    return np.unique(np.concatenate([picks, np.arange(starts[-1], M)]))


def test_forward_config1_tiny(tb):
    lin, x, W = linear_inputs(1)
    check_forward(tb, lin, x, W, np.arange(lin.M), "cfg1 tiny")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_forward_config2_decode(tb, M):
    lin, x, W = linear_inputs(2, 0, M)
    check_forward(tb, lin, x, W, np.arange(M), f"cfg2 decode M={M}")


def test_forward_config3_wo(tb):
    lin, x, W = linear_inputs(3)
    check_quant(tb, x, 4, True, rows=sample_rows(lin.M, 512, 3), label="cfg3 quant")
    check_forward(tb, lin, x, W, tile_rows(lin.M, 3), "cfg3 Wo")


def test_forward_config4_wdown(tb):
    lin, x, W = linear_inputs(4)
    check_quant(tb, x, 4, True, rows=sample_rows(lin.M, 256, 4), label="cfg4 quant")
    check_forward(tb, lin, x, W, tile_rows(lin.M, 4), "cfg4 Wdown")


@pytest.mark.parametrize("idx", range(7))
def test_forward_config5_block(tb, idx):
    lin, x, W = linear_inputs(5, idx)
    check_forward(tb, lin, x, W, tile_rows(lin.M, 50 + idx), f"cfg5 {lin.name}")


@pytest.mark.parametrize("M,N,K,bits,had", [(300, 200, 4096, 4, True), (1, 17, 256, 8, True),
                                            (257, 1000, 8192, 8, True), (5, 64, 64, 8, False),
                                            (70, 300, 960, 4, False), (2, 4096, 16384, 4, True)])
def test_forward_ragged_shapes(tb, M, N, K, bits, had):
    x = si.laplace(si.seed_for(6, 0) + M + K, M * K, 0.05).reshape(M, K)
    x[M // 2] = 0.0
    W = si.gaussian_weights(6, N, K)
    lin = si.Linear("ragged", M, K, N, bits, had, "x")
    check_forward(tb, lin, x, W, np.arange(M), f"ragged M={M} N={N} K={K} b={bits} h={had}")


# The widest rows the library takes (K = 65536, and 65472, the widest that is not a power of
# two): the activation stage's two-pass kernel, 205 packed blocks per row, int32 sums up to
# 2^23; decode shapes (split K and streaming) and both large-M kernels.
@pytest.mark.parametrize("M,N,K,bits", [(5, 200, 65536, 8), (16, 40, 65536, 4), (40, 200, 65536, 4),
                                        (33, 130, 65472, 8), (7, 48, 65472, 4)])
def test_forward_widest_rows(tb, M, N, K, bits):
    x = si.normal(si.seed_for(6, 1) + M + K, M * K).reshape(M, K)
    x[M - 1, ::3] *= 40.0                       # one row with a few large channels
    W = si.gaussian_weights(6, N, K, layer=1)
    lin = si.Linear("widest", M, K, N, bits, False, "x")
    check_forward(tb, lin, x, W, np.arange(M), f"widest M={M} N={N} K={K} b={bits}")


def test_forward_zero_input_gives_zero(tb):
    M, N, K = 4, 64, 4096
    W = si.gaussian_weights(7, N, K)
    packed, g = tb.bitnet_pack_weights(W)
    y = tb.hbitlinear_forward(dev(np.zeros((M, K), np.float32)), N, 4, True, dev(packed), g)
    torch.cuda.synchronize()
    assert not np.any(y.cpu().numpy())


# Degenerate weights: an all-zero matrix (gamma_w = 0, every trit 0: every byte the code of
# digits 1,1,1,1,1 = 121, every output 0) and constant matrices (every trit +1 or -1: each
# output is +-the row's code sum times s_x gamma_w), on the decode and large-M paths.
@pytest.mark.parametrize("M", [1, 16, 300])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("wval", [0.0, 0.37, -2.5])
def test_forward_degenerate_weights(tb, M, bits, wval):
    N, K = 96, 1024
    W = np.full((N, K), wval, np.float32)
    packed, g = tb.bitnet_pack_weights(W)
    if wval == 0.0:
        assert g == 0.0
        assert np.all(packed == 121)
        assert not np.any(oracle.ternarize(W)[0])
    else:
        assert np.float32(g) == np.float32(abs(wval))
    x = si.normal(si.seed_for(7, 3) + M + bits, M * K).reshape(M, K)
    lin = si.Linear("degenerate", M, K, N, bits, True, "x")
    check_forward(tb, lin, x, W, np.arange(M), f"degenerate W={wval} M={M} b={bits}")
    if wval == 0.0:
        y = tb.hbitlinear_forward(dev(x), N, bits, True, dev(packed), g)
        torch.cuda.synchronize()
        assert not np.any(y.cpu().numpy())


def test_forward_is_deterministic_and_stream_safe(tb):
    lin, x, W = linear_inputs(3, 0, 512)
    packed, g = tb.bitnet_pack_weights(W)
    xd, pd = dev(x), dev(packed)
    y1 = tb.hbitlinear_forward(xd, lin.N, 4, True, pd, g)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = tb.hbitlinear_forward(xd, lin.N, 4, True, pd, g, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_forward_rejects_small_workspace(tb):
    M, N, K = 4, 64, 256
    packed, g = tb.bitnet_pack_weights(si.gaussian_weights(7, N, K))
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tb.BitnetError) as e:
        tb.hbitlinear_forward(dev(np.ones((M, K), np.float32)), N, 8, True, dev(packed), g,
                              workspace=ws)
    assert e.value.status == tb.BITNET_ERR_WORKSPACE


# ------------------------------------------------------------------- grouped calls ----

@pytest.mark.parametrize("L,M,K,N,bits,had", [(5, 16, 4096, 512, 8, False), (3, 1, 1024, 300, 8, True),
                                              (4, 40, 4096, 256, 4, True), (2, 7, 960, 100, 4, False),
                                              # tiles whose rows and columns all lie inside the output
                                              (3, 600, 1024, 384, 4, True), (2, 300, 640, 272, 8, False),
                                              # 2 x 9 x 17 = 306 INT4 tiles, more than one round of the
                                              # CUs: the tile order by XCD runs across two layers
                                              (2, 4196, 640, 2112, 4, False)])
def test_forward_grouped_matches_oracle(tb, L, M, K, N, bits, had):
    say(f"  grouped L={L} M={M} K={K} N={N} bits={bits} had={had}")
    x = si.normal(si.seed_for(8, 0) + K + M, L * M * K).reshape(L, M, K)
    x[0, 0] = 0.0
    packs, gs, ts = [], [], []
    for l in range(L):
        W = si.gaussian_weights(8, N, K, layer=l)
        packed, g = tb.bitnet_pack_weights(W)
        packs.append(dev(packed)); gs.append(g); ts.append(oracle.ternarize(W)[0])
    ptrs = torch.tensor([p.data_ptr() for p in packs], dtype=torch.int64, device="cuda")
    wsc = torch.tensor(gs, dtype=torch.float32, device="cuda")
    xd = dev(x)
    y = tb.hbitlinear_forward_grouped(xd, N, bits, had, ptrs, wsc)
    # the product stage on its own, from the activation stage's codes
    codes, scales = tb.hbitlinear_quantize(xd.view(L * M, K), bits, had)
    y2 = tb.hbitlinear_gemm_dequant_grouped(codes, scales, L, M, K, N, bits, ptrs, wsc)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    for l in range(L):
        yl = tb.hbitlinear_forward(xd[l].contiguous(), N, bits, had, packs[l], gs[l])
        torch.cuda.synchronize()
        assert torch.equal(y[l], yl), f"layer {l} differs from its single call"
        oq, os_ = oracle.quantize(x[l], bits, had)
        oy = oracle.epilogue(oracle.gemm(oq, ts[l]), os_, np.float32(gs[l]))
        gq = codes_to_int8(codes, L * M, K, bits)[l * M:(l + 1) * M]
        match = np.all(gq == oq, axis=1)
        np.testing.assert_array_equal(y[l].cpu().numpy()[match], oy[match])


@pytest.mark.parametrize("M", [1, 3, 8, 16])
@pytest.mark.parametrize("bits", [8, 4])
def test_decode_kernel_gemm_i32(tb, M, bits):
    # M <= 16 runs the decode-shape kernel: check it bit-exactly on shared codes, with a ragged N
    K, N = 4096, 4096 + 80
    qp = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(M + bits)
    q = rng.integers(-qp - 1, qp + 1, size=(M, K)).astype(np.int8)
    W = si.gaussian_weights(9, N, K)
    packed, _ = tb.bitnet_pack_weights(W)
    cb = q.view(np.uint8) if bits == 8 else oracle.pack_int4(q)
    acc = tb.bitnet_ternary_gemm_i32(dev(cb.reshape(-1)), M, K, N, bits, dev(packed))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), oracle.gemm(q, oracle.ternarize(W)[0]))


# Decode shapes (M <= 16) run one of three kernels, chosen by the work items a call makes on a
# 256-CU device: 256-row streaming items when there are at least 256 of them; else one
# workgroup per 16-row group, K split over its four waves, when there are at most 512 groups;
# else 64-row streaming items.  Each case lands on one of them; the K values give waves with no
# block, uneven block counts and more than four blocks per wave.
@pytest.mark.parametrize("L,M,K,N,bits", [
    (1, 16, 16384, 1000, 4),    # split K: 52 blocks, 13 per wave
    (1, 7, 8192, 4100, 8),      # split K: 26 blocks (7, 7, 6, 6 per wave), ragged N
    (2, 2, 256, 200, 8),        # split K: one block, three idle waves
    (3, 9, 960, 300, 4),        # split K: three blocks, one idle wave
    (1, 16, 2048, 12000, 8),    # 64-row items: 750 groups
    (2, 5, 4096, 8200, 4),      # 64-row items over two layers
    (20, 3, 1024, 4096, 8),     # 256-row items: 320 of them
])
def test_decode_paths_match_oracle(tb, L, M, K, N, bits):
    say(f"  decode path L={L} M={M} K={K} N={N} bits={bits}")
    qp = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(L * 100003 + M * 101 + K + N + bits)
    q = rng.integers(-qp - 1, qp + 1, size=(L, M, K)).astype(np.int8)
    sx = rng.uniform(1e-3, 1e-1, size=(L, M)).astype(np.float32)
    packs, gs, ts = [], [], []
    for l in range(L):
        W = si.gaussian_weights(9, N, K, layer=l)
        packed, g = tb.bitnet_pack_weights(W)
        packs.append(dev(packed)); gs.append(g); ts.append(oracle.ternarize(W)[0])
    ptrs = torch.tensor([p.data_ptr() for p in packs], dtype=torch.int64, device="cuda")
    wsc = torch.tensor(gs, dtype=torch.float32, device="cuda")
    cb = [q[l].view(np.uint8) if bits == 8 else oracle.pack_int4(q[l]) for l in range(L)]
    codes = dev(np.concatenate([c.reshape(-1) for c in cb]))
    y = tb.hbitlinear_gemm_dequant_grouped(codes, dev(sx.reshape(-1)), L, M, K, N, bits, ptrs, wsc)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for l in range(L):
        oy = oracle.epilogue(oracle.gemm(q[l], ts[l]), sx[l], np.float32(gs[l]))
        np.testing.assert_array_equal(yh[l], oy, err_msg=f"layer {l}")


# The decode workload at full size, built and launched as the benchmark does: 128 distinct
# packed 4096 x 4096 weight buffers (copies of four seeded matrices), one activation-stage
# launch over all 128 M rows, one grouped product launch.  Every code and scale against the
# oracle; the outputs of sampled layers (all rows, all columns) against the oracle's product
# and epilogue; the one-layer product launch (the layer-by-layer decode) on the same codes
# equal to the grouped result.
@pytest.mark.parametrize("M", [16, 4, 1])
def test_decode_workload_full_size(tb, M):
    L, K, N, unique = 128, 4096, 4096, 4
    say(f"  decode workload L={L} M={M} K=N={K}")
    packs, gs, ts = [], [], []
    for u in range(unique):
        W = si.gaussian_weights(2, N, K, layer=u)
        packed, g = tb.bitnet_pack_weights(W)
        packs.append(dev(packed)); gs.append(g); ts.append(oracle.ternarize(W)[0])
    ws = [packs[l % unique].clone() for l in range(L)]
    ptrs = torch.tensor([w.data_ptr() for w in ws], dtype=torch.int64, device="cuda")
    wsc = torch.tensor([gs[l % unique] for l in range(L)], dtype=torch.float32, device="cuda")
    x = si.normal(si.seed_for(2, 0), L * M * K).reshape(L * M, K)
    codes, scales = tb.hbitlinear_quantize(dev(x), 8, False)
    y = tb.hbitlinear_gemm_dequant_grouped(codes, scales, L, M, K, N, 8, ptrs, wsc)
    torch.cuda.synchronize()
    gq = codes_to_int8(codes, L * M, K, 8)
    gsx = scales.cpu().numpy()
    oq, osx = oracle.quantize(x, 8, False)
    np.testing.assert_array_equal(gq, oq)
    np.testing.assert_array_equal(gsx, osx)
    yh = y.cpu().numpy()
    for l in (0, 1, 2, 3, 66, L - 1):
        r = slice(l * M, (l + 1) * M)
        oy = oracle.epilogue(oracle.gemm(oq[r], ts[l % unique]), osx[r], np.float32(gs[l % unique]))
        np.testing.assert_array_equal(yh[l], oy, err_msg=f"layer {l}")
        y1 = tb.hbitlinear_gemm_dequant(codes[l * M * K:(l + 1) * M * K], scales[r], M, K, N, 8,
                                        ws[l], gs[l % unique])
        torch.cuda.synchronize()
        assert torch.equal(y1, y[l]), f"layer {l}: one-layer launch differs from the grouped one"


# -------------------------------------------------------------------- graph capture ----

@pytest.mark.parametrize("L,M,K,N,bits,had", [(4, 16, 4096, 512, 8, False), (1, 600, 4096, 384, 4, True)])
def test_forward_graph_replays_match_eager(tb, L, M, K, N, bits, had):
    """The grouped forward captured once as a HIP graph (torch.cuda.CUDAGraph) and replayed
    three times, with eager work and a synchronisation between the replays: every replay
    gives the eager output bit for bit (the library issues kernel launches only, so the
    captured graph holds no memset or copy nodes)."""
    say(f"  graph L={L} M={M} K={K} N={N} bits={bits} had={had}")
    x = si.normal(si.seed_for(9, 0) + M, L * M * K).reshape(L, M, K)
    packs, gs = [], []
    for l in range(L):
        packed, g = tb.bitnet_pack_weights(si.gaussian_weights(9, N, K, layer=l))
        packs.append(dev(packed))
        gs.append(g)
    ptrs = torch.tensor([p.data_ptr() for p in packs], dtype=torch.int64, device="cuda")
    wsc = torch.tensor(gs, dtype=torch.float32, device="cuda")
    xd = dev(x)
    ws = torch.empty(tb.hbitlinear_grouped_workspace_bytes(L, M, K, bits), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((L, M, N), dtype=torch.float32, device="cuda")

    def fwd():
        tb.hbitlinear_forward_grouped(xd, N, bits, had, ptrs, wsc, out=out, workspace=ws)

    fwd()
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        fwd()
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager output"


# -------------------------------------------- several linears of one input; SwishGLU ----

def _gpu_codes(tb, x, bits, had):
    M, K = x.shape
    codes, scales = tb.hbitlinear_quantize(dev(x), bits, had)
    torch.cuda.synchronize()
    return codes, scales, codes_to_int8(codes, M, K, bits), scales.cpu().numpy()


# Paths (256 CUs): M <= 16 with 768 groups -> 64-row streaming items; 6 groups -> split K;
# 65536 rows -> 256-row streaming items; M > 16 -> the INT4 / INT8 large-M kernels, with
# segment boundaries inside a 128-row tile.
@pytest.mark.parametrize("M,K,seg_n,bits,had", [
    (16, 4096, [4096, 1024, 1024], 4, False),
    (5, 1024, [16, 48, 32], 8, True),
    (1, 256, [16384, 16384, 16384, 16384], 8, False),
    (300, 2048, [144, 96, 64], 4, True),
    (100, 1024, [48, 80, 16], 8, False),
    (17, 512, [16, 32, 16, 48, 16, 64, 16, 32], 4, True),   # eight segments, M just above 16
    (16, 256, [16] * 8, 8, False),                            # eight one-group segments, split K
])
def test_forward_segments_matches_oracle(tb, M, K, seg_n, bits, had):
    say(f"  segments M={M} K={K} seg_n={seg_n} bits={bits} had={had}")
    x = si.normal(si.seed_for(9, 1) + K + M, M * K).reshape(M, K)
    Ws = [si.gaussian_weights(9, n, K, layer=s, std=0.01 * (s + 1)) for s, n in enumerate(seg_n)]
    packed, gs = tb.bitnet_pack_weights_segments(np.concatenate(Ws), seg_n)
    ots = [oracle.ternarize(W) for W in Ws]
    ts = [t for t, _ in ots]
    assert np.array_equal(np.asarray(gs, np.float32), np.array([g for _, g in ots], np.float32))
    pw = dev(packed)
    codes, scales, q, s = _gpu_codes(tb, x, bits, had)
    y = tb.hbitlinear_gemm_dequant_segments(codes, scales, M, K, seg_n, bits, pw, gs)
    y_full = tb.hbitlinear_forward_segments(dev(x), seg_n, bits, had, pw, gs)
    torch.cuda.synchronize()
    assert torch.equal(y, y_full)
    expect = np.concatenate([oracle.epilogue(oracle.gemm(q, t), s, g) for t, g in zip(ts, gs)], axis=1)
    np.testing.assert_array_equal(y.cpu().numpy(), expect)


# Paths: M <= 16 with few groups -> two tiles per wave; 65536 weight rows -> four tiles per
# wave; M > 16 -> INT4 / INT8 large-M kernels, with F not a multiple of the tile.
@pytest.mark.parametrize("M,K,F,bits,had", [
    (16, 4096, 1024, 8, False),
    (7, 1024, 208, 4, True),
    (3, 256, 32768, 8, False),
    (300, 2048, 208, 4, True),
    (100, 1024, 80, 8, False),
    (17, 256, 16, 4, True),      # one gate / up pair, M just above 16 (large-M kernel)
    (1, 256, 16, 8, False),      # one pair at decode shape
])
def test_forward_swiglu_matches_oracle(tb, M, K, F, bits, had):
    say(f"  swiglu M={M} K={K} F={F} bits={bits} had={had}")
    x = si.normal(si.seed_for(9, 2) + K + M, M * K).reshape(M, K)
    Wg = si.gaussian_weights(9, F, K, layer=10)
    Wu = si.gaussian_weights(9, F, K, layer=11, std=0.05)
    packed, gg, gu = tb.bitnet_pack_gate_up(Wg, Wu)
    (tg, ogg), (tu, ogu) = oracle.ternarize(Wg), oracle.ternarize(Wu)
    assert (np.float32(gg), np.float32(gu)) == (ogg, ogu)
    pw = dev(packed)
    codes, scales, q, s = _gpu_codes(tb, x, bits, had)
    h = tb.hbitlinear_gemm_swiglu(codes, scales, M, K, F, bits, pw, gg, gu)
    h_full = tb.hbitlinear_forward_swiglu(dev(x), F, bits, had, pw, gg, gu)
    torch.cuda.synchronize()
    assert torch.equal(h, h_full)
    g_ref = oracle.epilogue(oracle.gemm(q, tg), s, np.float32(gg))
    u_ref = oracle.epilogue(oracle.gemm(q, tu), s, np.float32(gu))
    expect = oracle.swiglu(g_ref, u_ref)
    got = h.cpu().numpy()
    # fp32 SiLU with the hardware exp2 and reciprocal, then a product: e^-g carries the rounding
    # of g * log2(e) (relative error ~|g| * 6e-8) plus about one ulp per operation; |g| stays
    # far below 80 here, so 1e-5 relative bounds the difference from the double-rounded oracle
    assert np.max(np.abs(g_ref)) < 80
    np.testing.assert_allclose(got, expect, rtol=1e-5, atol=1e-30)
    assert np.count_nonzero(expect) > 0.9 * expect.size
    # end to end against the oracle's own activation stage, rows whose codes agree
    oh = oracle.forward_swiglu(x, oracle.pack(tg), np.float32(gg), oracle.pack(tu), np.float32(gu),
                               F, bits, had)
    oq, _ = oracle.quantize(x, bits, had)
    match = np.all(oq == q, axis=1)
    assert match.mean() > 0.9
    np.testing.assert_allclose(got[match], oh[match], rtol=1e-5, atol=1e-30)


# The fused launches of the 7B block at full size (M = 16384), on the block workload's inputs
# and weights and launched as the benchmark does: Q, K and V as one three-segment product
# launch; gate and up as one launch with the SwishGLU glue.  Sampled rows against the oracle:
# codes and scales identical, each segment bit-exact, the glue within 1e-5 relative.
def test_fused_block_full_size(tb):
    wl = si.workload(5)
    L = {l.name: l for l in wl.linears}
    M, K = L["q"].M, L["q"].K
    rows = sample_rows(M, 12, 55)
    say(f"  fused block M={M} K={K}, rows {rows.tolist()}")

    def stage(x):
        codes, scales = tb.hbitlinear_quantize(dev(x), 4, False)
        oq, osx = oracle.quantize(x[rows], 4, False)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes_to_int8(codes, M, K, 4)[rows], oq)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], osx)
        return codes, scales, oq, osx

    # Q, K, V: one launch over the stacked matrices, a gamma_w per segment
    x = si.activations(5, L["q"])
    seg_n = [L[n].N for n in ("q", "k", "v")]
    Ws = [si.weights(5, L[n]) for n in ("q", "k", "v")]
    packed, gs = tb.bitnet_pack_weights_segments(np.concatenate(Ws), seg_n)
    codes, scales, oq, osx = stage(x)
    y = tb.hbitlinear_gemm_dequant_segments(codes, scales, M, K, seg_n, 4, dev(packed), gs)
    torch.cuda.synchronize()
    gy = y.cpu().numpy()[rows]
    del y, codes, scales, x
    c0 = 0
    for s, W in enumerate(Ws):
        _, og, t = oracle.pack_weights(W)
        assert np.float32(gs[s]) == og
        oy = oracle.epilogue(oracle.gemm(oq, t), osx, og)
        np.testing.assert_array_equal(gy[:, c0:c0 + seg_n[s]], oy, err_msg=f"segment {s}")
        c0 += seg_n[s]
    del Ws

    # gate and up with SwishGLU in the epilogue
    x = si.activations(5, L["gate"])
    F = L["gate"].N
    Wg, Wu = si.weights(5, L["gate"]), si.weights(5, L["up"])
    packed, gg, gu = tb.bitnet_pack_gate_up(Wg, Wu)
    codes, scales, oq, osx = stage(x)
    h = tb.hbitlinear_gemm_swiglu(codes, scales, M, K, F, 4, dev(packed), gg, gu)
    torch.cuda.synchronize()
    gh = h.cpu().numpy()[rows]
    del h, codes, scales, x
    _, ogg, tg = oracle.pack_weights(Wg)
    _, ogu, tu = oracle.pack_weights(Wu)
    assert np.float32(gg) == ogg and np.float32(gu) == ogu
    g_ref = oracle.epilogue(oracle.gemm(oq, tg), osx, ogg)
    u_ref = oracle.epilogue(oracle.gemm(oq, tu), osx, ogu)
    assert np.max(np.abs(g_ref)) < 80
    np.testing.assert_allclose(gh, oracle.swiglu(g_ref, u_ref), rtol=1e-5, atol=1e-30)


# ------------------------------------------------------------ RMS norm in the activation stage ----

@pytest.mark.parametrize("M,K,bits,had,eps", [(7, 4096, 4, True, 1e-6), (33, 1024, 8, False, 0.0),
                                              (5, 16384, 4, True, 1e-5), (3, 256, 8, True, 0.5),
                                              (600, 4096, 4, True, 1e-6)])
def test_rmsnorm_stage_and_forward_match_oracle(tb, M, K, bits, had, eps):
    say(f"  rmsnorm M={M} K={K} bits={bits} had={had} eps={eps}")
    x = si.wo_activations(M, K) * np.float32(7.0)
    x[1] = 0.0                         # zero row: r = 0 with eps = 0, codes 0 either way
    gain = si.normal(si.seed_for(9, 3) + K, K, 1.0, 0.1)
    codes, scales, xh = tb.hbitlinear_quantize_rmsnorm(dev(x), dev(gain), eps, bits, had, want_xh=True)
    torch.cuda.synchronize()
    xn = oracle.rmsnorm(x, gain, eps)
    oq, os_, oxh = oracle.quantize(xn, bits, had, want_xh=True)
    gxh = xh.cpu().numpy()
    amax = np.maximum(np.max(np.abs(oxh), axis=1, keepdims=True), 1e-30)
    rel = float(np.max(np.abs(gxh - oxh) / amax))
    assert rel <= 1e-5, rel
    # r is a double sum rounded to fp32 once: only a row whose sum lands within a double
    # rounding of an fp32 boundary can differ; every other row is bit-identical
    same_rows = np.all(gxh == oxh, axis=1)
    assert np.count_nonzero(~same_rows) <= max(1, M // 1000), f"{np.count_nonzero(~same_rows)} rows differ"
    gq = codes_to_int8(codes, M, K, bits)
    diff = gq.astype(np.int32) - oq.astype(np.int32)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size and np.all(np.abs(diff) <= 1)
    assert np.allclose(scales.cpu().numpy(), os_, rtol=1e-5, atol=0)
    assert np.all(gq[1] == 0)
    # the forward: rows whose codes agree are bit-exact against the oracle's forward
    N = 96
    W = si.gaussian_weights(9, N, K, layer=20)
    packed, gw = tb.bitnet_pack_weights(W)
    y = tb.hbitlinear_forward_rmsnorm(dev(x), dev(gain), eps, N, bits, had, dev(packed), gw)
    torch.cuda.synchronize()
    opacked, ogw, _ = oracle.pack_weights(W)
    assert ogw == np.float32(gw)
    oy = oracle.forward_rmsnorm(x, gain, eps, opacked, ogw, N, bits, had)
    match = np.all(gq == oq, axis=1)
    assert match.mean() > 0.9
    np.testing.assert_array_equal(y.cpu().numpy()[match], oy[match])


# The activation stage with the norm at the three full sizes the benchmark times (its inputs:
# Wo-like activations, gains N(1, 0.1), eps 1e-6, INT4), sampled rows against the oracle.
@pytest.mark.parametrize("M,K,had", [(4096, 4096, True), (8192, 16384, True), (16384, 4096, False)])
def test_rmsnorm_stage_full_size(tb, M, K, had):
    x = si.wo_activations(M, K)
    gain = si.normal(si.seed_for(5, 12), K, 1.0, 0.1)
    rows = sample_rows(M, 64, M + K)
    say(f"  rmsnorm full size M={M} K={K} had={had}")
    codes, scales = tb.hbitlinear_quantize_rmsnorm(dev(x), dev(gain), 1e-6, 4, had)
    torch.cuda.synchronize()
    gq = codes_to_int8(codes, M, K, 4)[rows]
    gs = scales.cpu().numpy()[rows]
    del codes, scales
    oq, os_ = oracle.quantize(oracle.rmsnorm(x[rows], gain, 1e-6), 4, had)
    diff = gq.astype(np.int32) - oq.astype(np.int32)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size and np.all(np.abs(diff) <= 1)
    assert np.allclose(gs, os_, rtol=1e-5, atol=0)


# ------------------------------------------------- weight + activation Hadamard variant ----

def test_weight_activation_hadamard_variant(tb):
    M, K, N = 64, 4096, 256
    x = si.wo_activations(M, K)                   # Laplace with 1 % outlier channels x50
    W = si.gaussian_weights(18, N, K)
    p1, g1 = tb.bitnet_pack_weights_hadamard(W)
    y1 = tb.hbitlinear_forward(dev(x), N, 4, True, dev(p1), g1)
    p0, g0 = tb.bitnet_pack_weights(W)
    y0 = tb.hbitlinear_forward(dev(x), N, 4, False, dev(p0), g0)
    torch.cuda.synchronize()
    # parity: the oracle's forward on the oracle's rotated pack, rows whose codes agree
    op, og = oracle.pack_weights_hadamard(W)
    assert np.array_equal(to_device(op, N, K), p1) and og == np.float32(g1)
    oy = oracle.forward(x, op, og, N, 4, True)
    codes, _ = tb.hbitlinear_quantize(dev(x), 4, True)
    torch.cuda.synchronize()
    oq, _ = oracle.quantize(x, 4, True)
    match = np.all(codes_to_int8(codes, M, K, 4) == oq, axis=1)
    assert match.mean() > 0.9
    np.testing.assert_array_equal(y1.cpu().numpy()[match], oy[match])
    # the error the INT4 activation quantisation adds, each variant against its own ternary
    # weights in full precision (the ternarisation error is common to both).  Without the
    # rotation the outlier channels set each token's scale and the Laplace bulk rounds to zero:
    # the error is about the bulk's share of the product (~0.2); with it the row is near
    # Gaussian and the error is INT4 absmax rounding (~0.15).  Measured: 0.230 and 0.140.
    t0 = oracle.ternarize(W)[0].astype(np.float64) * g0
    t1 = oracle.unpack(op, N, K).astype(np.float64) * g1
    xh = oracle.fwht_f64(x.astype(np.float64)) / math.sqrt(K)
    r0, r1 = x.astype(np.float64) @ t0.T, xh @ t1.T
    e_plain = np.linalg.norm(y0.cpu().numpy() - r0) / np.linalg.norm(r0)
    e_rot = np.linalg.norm(y1.cpu().numpy() - r1) / np.linalg.norm(r1)
    say(f"  INT4 activation-quantisation error: rotated {e_rot:.4f}, plain {e_plain:.4f}")
    assert e_rot < 0.75 * e_plain


# ------------------------------------------------------------- low-bit Q/K/V states ----

def _states_reference(q_rows, s_rows, ts, gs, seg_n, bits, group):
    """The oracle's product and epilogue on the given codes, then its state quantiser."""
    y = np.concatenate([oracle.epilogue(oracle.gemm(q_rows, t), s_rows, np.float32(g))
                        for t, g in zip(ts, gs)], axis=1)
    return oracle.quantize_states(y, seg_n, bits, group)


# The states form of the large-M kernels (INT4: groups inside a wave's 128 columns; INT8: a
# group of 128 over two waves' 64 columns, combined through LDS): segment boundaries inside a
# tile (groups of 64), ragged M and N, Q at 4 or 8 bits with K and V at 3; every row and column
# against the oracle run on the GPU's own activation codes (bit-identical codes and scales),
# and the whole call against the oracle's forward on rows whose activation codes agree.
@pytest.mark.parametrize("M,K,seg_n,bits,group,had,act", [
    (300, 2048, [256, 128, 128], [4, 3, 3], 128, False, 4),
    (17, 512, [128, 64, 192], [8, 3, 3], 64, True, 4),
    (600, 4096, [512, 512, 512], [4, 3, 3], 128, True, 4),
    (300, 2048, [256, 128, 128], [4, 3, 3], 128, False, 8),
    (40, 1024, [128, 64, 192], [8, 3, 3], 64, True, 8),
    (600, 4096, [512, 512, 640], [4, 3, 3], 128, True, 8),
])
def test_qkv_states_match_oracle(tb, M, K, seg_n, bits, group, had, act):
    say(f"  qkv states M={M} K={K} seg_n={seg_n} bits={bits} group={group} had={had} act={act}")
    x = si.wo_activations(M, K) if had else si.normal(si.seed_for(9, 5) + M, M * K).reshape(M, K)
    x[M // 3] = 0.0                                   # a zero row: every group zero
    Ws = [si.gaussian_weights(9, n, K, layer=30 + s, std=0.01 * (s + 1)) for s, n in enumerate(seg_n)]
    packed, gs = tb.bitnet_pack_weights_segments(np.concatenate(Ws), seg_n)
    ots = [oracle.ternarize(W) for W in Ws]
    assert np.array_equal(np.asarray(gs, np.float32), np.array([g for _, g in ots], np.float32))
    pw = dev(packed)
    codes, scales, q, s = _gpu_codes(tb, x, act, had)
    sc, ss = tb.hbitlinear_gemm_qkv_states(codes, scales, M, K, seg_n, act, pw, gs, bits, group)
    fc, fs = tb.hbitlinear_forward_qkv_states(dev(x), seg_n, act, had, pw, gs, bits, group)
    torch.cuda.synchronize()
    assert torch.equal(sc, fc) and torch.equal(ss, fs)
    ec, es = _states_reference(q, s, [t for t, _ in ots], gs, seg_n, bits, group)
    np.testing.assert_array_equal(sc.cpu().numpy(), ec)
    np.testing.assert_array_equal(ss.cpu().numpy(), es)
    assert np.all(sc.cpu().numpy()[M // 3] == 0) and np.all(ss.cpu().numpy()[M // 3] == 0)
    # 3-bit states use the codes -3..3 only
    col = np.cumsum([0] + seg_n)
    for sgi, b in enumerate(bits):
        part = sc.cpu().numpy()[:, col[sgi]:col[sgi + 1]]
        assert part.min() >= -(2 ** (b - 1) - 1) and part.max() <= 2 ** (b - 1) - 1
    # end to end against the oracle's own activation stage
    oc, os_ = oracle.forward_qkv_states(x, [oracle.pack(t) for t, _ in ots], gs, seg_n, act, had, bits, group)
    oq, _ = oracle.quantize(x, act, had)
    match = np.all(oq == q, axis=1)
    assert match.mean() > 0.9
    np.testing.assert_array_equal(sc.cpu().numpy()[match], oc[match])
    np.testing.assert_array_equal(ss.cpu().numpy()[match], os_[match])


# The states form of the decode kernel (M <= 16, INT8 or INT4 activations, always the
# streaming kernel with four column tiles per wave): heads of 64 columns (one wave's tiles) and
# of 128 (two waves, their maxima combined through LDS), segment boundaries inside a
# workgroup's 256 columns, a workgroup past the last column, a zero row, and the width of the
# block's Q/K/V projections; every row and column against the oracle run on the GPU's own
# activation codes (bit-identical codes and scales).
@pytest.mark.parametrize("M,K,seg_n,act_bits,bits,group,had", [
    (1, 4096, [4096, 4096, 4096], 8, [4, 3, 3], 128, False),
    (16, 1024, [256, 128, 128], 4, [8, 3, 3], 64, True),
    (5, 2048, [128, 384, 128], 8, [4, 3, 3], 128, True),
    (16, 4096, [4096, 1024, 1024], 4, [4, 3, 3], 128, False),
])
def test_qkv_states_decode_match_oracle(tb, M, K, seg_n, act_bits, bits, group, had):
    say(f"  qkv states decode M={M} K={K} seg_n={seg_n} act_bits={act_bits} bits={bits} group={group} had={had}")
    x = si.wo_activations(M, K) if had else si.normal(si.seed_for(9, 6) + M, M * K).reshape(M, K)
    if M > 2:
        x[M // 2] = 0.0                               # a zero row: every group zero
    Ws = [si.gaussian_weights(9, n, K, layer=40 + s, std=0.01 * (s + 1)) for s, n in enumerate(seg_n)]
    packed, gs = tb.bitnet_pack_weights_segments(np.concatenate(Ws), seg_n)
    ots = [oracle.ternarize(W) for W in Ws]
    pw = dev(packed)
    codes, scales, q, s = _gpu_codes(tb, x, act_bits, had)
    sc, ss = tb.hbitlinear_gemm_qkv_states(codes, scales, M, K, seg_n, act_bits, pw, gs, bits, group)
    fc, fs = tb.hbitlinear_forward_qkv_states(dev(x), seg_n, act_bits, had, pw, gs, bits, group)
    torch.cuda.synchronize()
    assert torch.equal(sc, fc) and torch.equal(ss, fs)
    ec, es = _states_reference(q, s, [t for t, _ in ots], gs, seg_n, bits, group)
    np.testing.assert_array_equal(sc.cpu().numpy(), ec)
    np.testing.assert_array_equal(ss.cpu().numpy(), es)
    if M > 2:
        assert np.all(sc.cpu().numpy()[M // 2] == 0) and np.all(ss.cpu().numpy()[M // 2] == 0)


# The block's Q, K and V at full size (M = 16384, K = 4096, three 4096-row segments), launched
# with the states fused as the benchmark does: Q at 4 bits, K and V at 3, heads of 128; one
# sampled row in every 512-row tile of the kernel plus the whole last tile's first and last
# rows, against the oracle on the GPU's codes.
def test_qkv_states_full_size(tb):
    wl = si.workload(5)
    L = {l.name: l for l in wl.linears}
    M, K = L["q"].M, L["q"].K
    seg_n = [L[n].N for n in ("q", "k", "v")]
    bits, group = [4, 3, 3], 128
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([np.arange(0, M, 512) + rng.integers(0, 512, M // 512),
                                     [0, M - 512, M - 1]]))
    say(f"  qkv states full size M={M}: {rows.size} rows, one in each 512-row tile")
    x = si.activations(5, L["q"])
    Ws = [si.weights(5, L[n]) for n in ("q", "k", "v")]
    packed, gs = tb.bitnet_pack_weights_segments(np.concatenate(Ws), seg_n)
    ts = [oracle.ternarize(W)[0] for W in Ws]
    del Ws
    codes, scales = tb.hbitlinear_quantize(dev(x), 4, False)
    sc, ss = tb.hbitlinear_gemm_qkv_states(codes, scales, M, K, seg_n, 4, dev(packed), gs, bits, group)
    torch.cuda.synchronize()
    q = codes_to_int8(codes, M, K, 4)[rows]
    sx = scales.cpu().numpy()[rows]
    oq, osx = oracle.quantize(x[rows], 4, False)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sx, osx)
    ec, es = _states_reference(q, sx, ts, gs, seg_n, bits, group)
    np.testing.assert_array_equal(sc.cpu().numpy()[rows], ec)
    np.testing.assert_array_equal(ss.cpu().numpy()[rows], es)
