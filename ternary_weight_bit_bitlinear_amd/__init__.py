"""H-BitLinear (BitNet b1.58 / BitNet v2) forward pass for AMD MI355X (gfx950).

The compute lives in ``libbitnet_hip.so`` (hand-written HIP kernels behind the C ABI of
``include/bitnet.h``); :mod:`.bitnet` is its Python binding.  Build the library with
``python -m ternary_weight_bit_bitlinear_amd.build``.
"""
from .bitnet import (  # noqa: F401
    BITNET_ERR_FORMAT, BITNET_ERR_HIP, BITNET_ERR_NULL, BITNET_ERR_SHAPE,
    BITNET_ERR_UNSUPPORTED, BITNET_ERR_WORKSPACE, BITNET_OK, BitnetError, LIB_PATH,
    bitnet_abi_version, bitnet_pack_weights, bitnet_packed_bytes, bitnet_status_string,
    bitnet_ternary_gemm_i32, bitnet_unpack_weights, hbitlinear_codes_bytes, hbitlinear_forward,
    hbitlinear_forward_grouped, hbitlinear_gemm_dequant, hbitlinear_gemm_dequant_grouped,
    hbitlinear_grouped_workspace_bytes, hbitlinear_quantize, hbitlinear_workspace_bytes, lib,
    bitnet_pack_gate_up, bitnet_pack_weights_segments, hbitlinear_forward_segments,
    hbitlinear_forward_swiglu, hbitlinear_gemm_dequant_segments, hbitlinear_gemm_swiglu,
    hbitlinear_forward_rmsnorm, hbitlinear_quantize_rmsnorm, bitnet_pack_weights_hadamard,
    hbitlinear_forward_noalloc, NOALLOC_SCRATCH_BYTES, hbitlinear_forward_qkv_states,
    hbitlinear_gemm_qkv_states,
)
