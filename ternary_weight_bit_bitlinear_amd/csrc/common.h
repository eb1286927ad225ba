// common.h -- internal helpers shared by the kernels and the C ABI of libbitnet_hip.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bitnet.h"

namespace bitnet {

// Packed weight geometry: a row is cut into blocks of 320 weights stored in 64 bytes; byte b
// of block B holds the weights k = 320 B + b + 64 i, i = 0..4, as base-3 digit i (MSB first).
constexpr int kBlockWeights = 320;
constexpr int kBlockBytes = 64;
constexpr int kSlab = 64;  // weights per digit slab of a block (one MFMA k-extent)

inline int64_t row_bytes(int K) { return (int64_t)kBlockBytes * ((K + kBlockWeights - 1) / kBlockWeights); }

inline int64_t codes_row_bytes(int K, int bits) { return bits == 8 ? (int64_t)K : (int64_t)K / 2; }

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Compute units of the current device, queried once per device (256 if the query fails).
int device_cus();

// Output form of a one-layer product launch beyond the plain epilogue (one weight scale):
//  - segments: nseg weight matrices stacked by rows, segment s covering the 16-row groups
//    [seg_end[s-1], seg_end[s]) (seg_end[-1] = 0) with weight scale seg_scale[s]; the output
//    keeps one column per weight row;
//  - glu: a gate matrix and an up matrix of F rows each, interleaved by 16-row groups (group
//    2i = gate rows 16i..16i+15, group 2i+1 = the same up rows); the output is M x F,
//    h = SiLU(gate) * up, each of gate and up dequantised with its own weight scale.
//  - states (with segments): every dequantised output is quantised again, per row and per
//    group of 16 * state_tiles consecutive columns (an attention head), to its segment's
//    seg_qp[s] = 2^(b-1) - 1; the output is the int8 codes (M x N), and state_scales (M x
//    N / (16 * state_tiles) fp32) receives gamma / Qp per group.
// The default (nseg = 0, glu = 0, states = 0) is the plain epilogue.
constexpr int kMaxSegments = 8;
struct OutForm {
    int nseg = 0;
    int seg_end[kMaxSegments] = {};
    float seg_scale[kMaxSegments] = {};
    int glu = 0;
    float gate_scale = 0.0f, up_scale = 0.0f;
    int states = 0;
    int state_tiles = 0;
    int seg_qp[kMaxSegments] = {};
    float* state_scales = nullptr;
};

// Weight scale of 16-row group grp: its segment's scale, or dflt without segments.
__host__ __device__ inline float group_scale(const OutForm& of, int grp, float dflt)
{
    if (of.nseg == 0) return dflt;
    float s = of.seg_scale[0];
    for (int i = 1; i < kMaxSegments; i++)
        if (i < of.nseg && grp >= of.seg_end[i - 1]) s = of.seg_scale[i];
    return s;
}

// Qp of the states of 16-row group grp: its segment's seg_qp.
__host__ __device__ inline int group_qp(const OutForm& of, int grp)
{
    int q = of.seg_qp[0];
    for (int i = 1; i < kMaxSegments; i++)
        if (i < of.nseg && grp >= of.seg_end[i - 1]) q = of.seg_qp[i];
    return q;
}

// SiLU(g) * u in fp32, SiLU(z) = z / (1 + e^-z), with the hardware exp2 and reciprocal:
// e^-z = 2^(-z log2 e) costs one rounding of the product, a relative error of about
// |z| * 6e-8 in e^-z (and less in the sigmoid), plus about one ulp each for exp2, the
// reciprocal and the products -- within 1e-5 relative for |z| < 80.  e^-z overflowing to
// infinity gives a zero reciprocal and h = -0 * u.
__device__ inline float silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Maximum over the 16 lanes 16 i .. 16 i + 15 that share an MFMA 16x16 output row group, by
// DPP moves inside the row of 16 lanes: swap neighbours, swap pairs, mirror the halves of
// eight, mirror the row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}
__device__ __forceinline__ float max16(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror
    return v;
}

// Internal launchers (quant.hip, gemm.hip).  Arguments are validated by the caller.
// gain != nullptr: RMS-normalise each row first (gain: K fp32, device; eps >= 0); K must then
// be a power of two in [256, 16384].
hipError_t launch_quantize(const float* x, int M, int K, int bits, int use_hadamard,
                           uint8_t* codes, float* scales, float* xh, hipStream_t stream,
                           const float* gain = nullptr, float eps = 0.0f);

// Ternary product over L layers of one shape (L = 1 for a single layer).  Layer l reads codes
// rows [l*M, (l+1)*M), scales[l*M ...], weights wptrs[l] (or w0 when wptrs is null) and
// wscales[l] (or wscale0), and writes rows [l*M, (l+1)*M) of the output.
// out_f32 != nullptr: out = (float(acc) * scale[m]) * w_scale;  else acc_i32 receives acc.
// of: output form (segments / gate-up pairs), only with L = 1 and out_f32.
hipError_t launch_gemm(const uint8_t* codes, int L, int M, int K, int N, int bits,
                       const uint8_t* const* wptrs, const uint8_t* w0, const float* scales,
                       const float* wscales, float wscale0, float* out_f32, int32_t* acc_i32,
                       hipStream_t stream, const OutForm& of = OutForm());

// Kernel variants behind launch_gemm: M <= 16 (gemm_decode.hip) and any M (gemm.hip).
hipError_t launch_gemm_decode(const uint8_t* codes, int L, int M, int K, int N, int bits,
                              const uint8_t* const* wptrs, const uint8_t* w0,
                              const float* scales, const float* wscales, float wscale0,
                              float* out_f32, int32_t* acc_i32, hipStream_t stream,
                              const OutForm& of);
hipError_t launch_gemm_large(const uint8_t* codes, int L, int M, int K, int N, int bits,
                             const uint8_t* const* wptrs, const uint8_t* w0,
                             const float* scales, const float* wscales, float wscale0,
                             float* out_f32, int32_t* acc_i32, hipStream_t stream,
                             const OutForm& of);

}  // namespace bitnet
