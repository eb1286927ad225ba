"""hbitlinear_forward_noalloc (workspace in the library's static device array) against
hbitlinear_forward (caller's workspace), through the C ABI: bit for bit on consecutive calls,
a large one first and then smaller ones, which reuse the same array with stale contents from
the call before."""
import numpy as np
import pytest

import seeded_inputs as si

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


def test_noalloc_matches_forward_on_consecutive_calls():
    import ternary_weight_bit_bitlinear_amd as tb
    # (M, K, N, bits, hadamard): the attention-output shape (workspace 8 MiB + 16 KiB, the
    # large-M kernel), then a decode shape and a ragged one, each smaller than the first
    cases = [(4096, 4096, 4096, 4, True), (16, 4096, 4096, 8, False), (300, 1024, 200, 8, True)]
    for i, (M, K, N, bits, had) in enumerate(cases):
        say(f"  noalloc call {i}: M={M} K={K} N={N} bits={bits} had={had}")
        assert tb.hbitlinear_workspace_bytes(M, K, bits) <= tb.NOALLOC_SCRATCH_BYTES
        x = si.wo_activations(M, K) if had else si.normal(si.seed_for(10, i), M * K).reshape(M, K)
        W = si.gaussian_weights(10, N, K, layer=i)
        packed, g = tb.bitnet_pack_weights(W)
        xd = torch.from_numpy(x).cuda()
        pd = torch.from_numpy(packed).cuda()
        ref = tb.hbitlinear_forward(xd, N, bits, had, pd, g)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        tb.hbitlinear_forward_noalloc(xd, N, bits, had, pd, g, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i} differs from hbitlinear_forward"
        assert bool(torch.isfinite(out).all())


def test_noalloc_rejects_oversize_before_any_launch():
    import ternary_weight_bit_bitlinear_amd as tb
    M, K, N = 8192, 4096, 64      # INT4 workspace 16 MiB + 32 KiB: one row group too many
    assert tb.hbitlinear_workspace_bytes(M, K, 4) > tb.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    packed, g = tb.bitnet_pack_weights(np.zeros((N, K), np.float32))
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(tb.BitnetError) as e:
        tb.hbitlinear_forward_noalloc(x, N, 4, True, torch.from_numpy(packed).cuda(), g, out)
    assert e.value.status == tb.BITNET_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was launched
