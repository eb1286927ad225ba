// abi.hip -- the extern "C" entry points of libbitnet_hip.so (declared in include/bitnet.h).
// Every entry point checks its arguments on the host first and launches nothing when a check
// fails; work is queued on the caller's stream.
#include <atomic>
#include <mutex>

#include "common.h"

using namespace bitnet;

namespace {

// Workspace of hbitlinear_forward_noalloc: the activation codes and scales of one call live in
// this array, which the HIP runtime places in each device's memory when the library's code is
// loaded there and keeps until the process ends.  Host code never uses the name itself as an
// address (on the host it is only a handle): the device address is looked up once per device
// with hipGetSymbolAddress and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[BITNET_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mutex;

// The current device's copy of `scratch`, resolved on the first call on that device.
int scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return BITNET_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return BITNET_ERR_UNSUPPORTED;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return BITNET_ERR_HIP;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BITNET_OK;
}

int check_shape(int M, int K, int N, int bits, int use_hadamard)
{
    if (M <= 0 || K <= 0 || N <= 0) return BITNET_ERR_SHAPE;
    if (bits != 4 && bits != 8) return BITNET_ERR_UNSUPPORTED;
    if (use_hadamard != 0 && use_hadamard != 1) return BITNET_ERR_UNSUPPORTED;
    if (K % 64 != 0 || K > 65536) return BITNET_ERR_UNSUPPORTED;
    if (use_hadamard) {
        if ((K & (K - 1)) != 0 || K < 256 || K > 16384) return BITNET_ERR_UNSUPPORTED;
    }
    if ((int64_t)M > (int64_t)65535 * 256) return BITNET_ERR_UNSUPPORTED;  // grid limit
    return BITNET_OK;
}

// The product kernels address one layer's packed weights, codes and output with 32-bit
// buffer offsets: each must stay below 2 GiB.
int check_gemm_limits(int M, int K, int N, int bits)
{
    const int64_t packed = (int64_t)1024 * ((N + 15) / 16) * ((K + 319) / 320);
    const int64_t codes = (int64_t)M * codes_row_bytes(K, bits);
    const int64_t out = (int64_t)4 * M * N;
    const int64_t lim = (int64_t)1 << 31;
    return packed < lim && codes < lim && out < lim ? BITNET_OK : BITNET_ERR_UNSUPPORTED;
}

int status_of(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_ERR_HIP; }

size_t codes_bytes(int M, int K, int bits) { return (size_t)M * (size_t)codes_row_bytes(K, bits); }

size_t workspace_bytes(int M, int K, int bits)
{
    return align256(codes_bytes(M, K, bits)) + align256((size_t)M * sizeof(float));
}

// The RMS-norm front of the activation stage: a gain vector, a finite eps >= 0, and a
// power-of-two K in [256, 16384] (the one-pass row kernel).
int check_norm(int K, const float* gain, float eps)
{
    if (gain == nullptr) return BITNET_ERR_NULL;
    if (!(eps >= 0.0f) || eps > 3.4e38f) return BITNET_ERR_UNSUPPORTED;
    if ((K & (K - 1)) != 0 || K < 256 || K > 16384) return BITNET_ERR_UNSUPPORTED;
    return BITNET_OK;
}

// Segments of a stacked weight (host arrays): checks them and fills the output form.
int segment_form(int S, const int* seg_n, const float* w_scales, int* n_total, OutForm* of)
{
    if (seg_n == nullptr || w_scales == nullptr) return BITNET_ERR_NULL;
    if (S <= 0 || S > BITNET_MAX_SEGMENTS || S > kMaxSegments) return BITNET_ERR_UNSUPPORTED;
    int64_t rows = 0;
    for (int s = 0; s < S; s++) {
        if (seg_n[s] <= 0) return BITNET_ERR_SHAPE;
        if (seg_n[s] % 16 != 0) return BITNET_ERR_UNSUPPORTED;
        rows += seg_n[s];
        of->seg_end[s] = (int)(rows / 16);
        of->seg_scale[s] = w_scales[s];
    }
    if (rows > (int64_t)1 << 30) return BITNET_ERR_UNSUPPORTED;
    of->nseg = S;
    *n_total = (int)rows;
    return BITNET_OK;
}

// Low-bit states of stacked linears: the segments' form plus, per segment, the states' Qp,
// and the group (head) size (64 or 128).  Every product kernel has the form: the INT4
// large-M kernel (a wave's 128 columns hold whole groups), the INT8 one (a group of 128 spans
// two waves' 64 columns, combined through LDS) and the decode streaming kernel (one group per
// workgroup).
int states_form(int S, const int* seg_n, const float* w_scales, const int* state_bits, int group,
                int M, int act_bits, float* state_scales, int* n_total, OutForm* of)
{
    int rc = segment_form(S, seg_n, w_scales, n_total, of);
    if (rc != BITNET_OK) return rc;
    if (state_bits == nullptr || state_scales == nullptr) return BITNET_ERR_NULL;
    if (group != 64 && group != 128) return BITNET_ERR_UNSUPPORTED;
    for (int s = 0; s < S; s++) {
        if (seg_n[s] % group != 0) return BITNET_ERR_UNSUPPORTED;
        if (state_bits[s] < 2 || state_bits[s] > 8) return BITNET_ERR_UNSUPPORTED;
        of->seg_qp[s] = (1 << (state_bits[s] - 1)) - 1;
    }
    of->states = 1;
    of->state_tiles = group / 16;
    of->state_scales = state_scales;
    return BITNET_OK;
}

// Gate / up pairs of F rows each (F % 16 == 0): 2F weight rows, M x F output.
int glu_form(int F, float gate_scale, float up_scale, OutForm* of)
{
    if (F <= 0) return BITNET_ERR_SHAPE;
    if (F % 16 != 0 || F > (1 << 29)) return BITNET_ERR_UNSUPPORTED;
    of->glu = 1;
    of->gate_scale = gate_scale;
    of->up_scale = up_scale;
    return BITNET_OK;
}

}  // namespace

extern "C" {

const char* bitnet_status_string(int status)
{
    switch (status) {
    case BITNET_OK: return "ok";
    case BITNET_ERR_NULL: return "a required pointer is NULL";
    case BITNET_ERR_SHAPE: return "invalid size (M, N or K <= 0, or buffer too small)";
    case BITNET_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case BITNET_ERR_WORKSPACE: return "workspace missing or too small";
    case BITNET_ERR_HIP: return "HIP runtime or launch error";
    case BITNET_ERR_FORMAT: return "packed weight byte is not a base-3 code";
    default: return "unknown status";
    }
}

int bitnet_abi_version(void) { return 1; }

int hbitlinear_codes_bytes(int M, int K, int act_bits, size_t* bytes_out)
{
    if (bytes_out == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, 1, act_bits, 0);
    if (rc != BITNET_OK) return rc;
    *bytes_out = codes_bytes(M, K, act_bits);
    return BITNET_OK;
}

int hbitlinear_workspace_bytes(int M, int K, int act_bits, size_t* bytes_out)
{
    if (bytes_out == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, 1, act_bits, 0);
    if (rc != BITNET_OK) return rc;
    *bytes_out = workspace_bytes(M, K, act_bits);
    return BITNET_OK;
}

int hbitlinear_quantize(const float* x, int M, int K, int act_bits, int use_hadamard,
                        uint8_t* codes, float* scales, float* xh_or_null, void* stream)
{
    if (x == nullptr || codes == nullptr || scales == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, 1, act_bits, use_hadamard);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, xh_or_null,
                                     (hipStream_t)stream));
}

int hbitlinear_quantize_rmsnorm(const float* x, int M, int K, const float* gain, float eps,
                                int act_bits, int use_hadamard, uint8_t* codes, float* scales,
                                float* xh_or_null, void* stream)
{
    if (x == nullptr || codes == nullptr || scales == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, 1, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_norm(K, gain, eps);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, xh_or_null,
                                     (hipStream_t)stream, gain, eps));
}

int hbitlinear_forward_rmsnorm(const float* x, int M, int K, int N, const float* gain, float eps,
                               int act_bits, int use_hadamard, float* out, const uint8_t* packed_w,
                               float w_scale, void* workspace, size_t workspace_size, void* stream)
{
    if (x == nullptr || out == nullptr || packed_w == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, N, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_norm(K, gain, eps);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    if (workspace == nullptr || workspace_size < workspace_bytes(M, K, act_bits))
        return BITNET_ERR_WORKSPACE;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(M, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, nullptr, s, gain, eps);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 w_scale, out, nullptr, s));
}

int bitnet_ternary_gemm_i32(const uint8_t* codes, int M, int K, int N, int act_bits,
                            const uint8_t* packed_w, int32_t* acc, void* stream)
{
    if (codes == nullptr || packed_w == nullptr || acc == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, N, act_bits, 0);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, nullptr, nullptr,
                                 0.0f, nullptr, acc, (hipStream_t)stream));
}

int hbitlinear_gemm_dequant(const uint8_t* codes, const float* scales, int M, int K, int N,
                            int act_bits, const uint8_t* packed_w, float w_scale, float* out,
                            void* stream)
{
    if (codes == nullptr || scales == nullptr || packed_w == nullptr || out == nullptr)
        return BITNET_ERR_NULL;
    int rc = check_shape(M, K, N, act_bits, 0);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 w_scale, out, nullptr, (hipStream_t)stream));
}

int hbitlinear_forward(const float* x, int M, int K, int N, int act_bits, int use_hadamard,
                       float* out, const uint8_t* packed_w, float w_scale, void* workspace,
                       size_t workspace_size, void* stream)
{
    if (x == nullptr || out == nullptr || packed_w == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, N, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    if (workspace == nullptr || workspace_size < workspace_bytes(M, K, act_bits))
        return BITNET_ERR_WORKSPACE;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(M, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, nullptr, s);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 w_scale, out, nullptr, s));
}

int hbitlinear_forward_noalloc(const float* x, int M, int K, int N, int act_bits, int use_hadamard,
                               float* out, const uint8_t* packed_w, float w_scale, void* stream)
{
    if (x == nullptr || out == nullptr || packed_w == nullptr) return BITNET_ERR_NULL;
    int rc = check_shape(M, K, N, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    // the same workspace layout as hbitlinear_forward, inside the static array
    if (workspace_bytes(M, K, act_bits) > (size_t)BITNET_NOALLOC_SCRATCH_BYTES)
        return BITNET_ERR_WORKSPACE;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != BITNET_OK) return rc;
    uint8_t* codes = static_cast<uint8_t*>(ws);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(M, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, nullptr, s);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 w_scale, out, nullptr, s));
}

int hbitlinear_gemm_dequant_segments(const uint8_t* codes, const float* scales, int M, int K,
                                     int S, const int* seg_n, int act_bits,
                                     const uint8_t* packed_w, const float* w_scales, float* out,
                                     void* stream)
{
    if (codes == nullptr || scales == nullptr || packed_w == nullptr || out == nullptr)
        return BITNET_ERR_NULL;
    OutForm of;
    int N = 0;
    int rc = segment_form(S, seg_n, w_scales, &N, &of);
    if (rc == BITNET_OK) rc = check_shape(M, K, N, act_bits, 0);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 0.0f, out, nullptr, (hipStream_t)stream, of));
}

int hbitlinear_forward_segments(const float* x, int M, int K, int S, const int* seg_n,
                                int act_bits, int use_hadamard, float* out,
                                const uint8_t* packed_w, const float* w_scales, void* workspace,
                                size_t workspace_size, void* stream)
{
    if (x == nullptr || out == nullptr || packed_w == nullptr) return BITNET_ERR_NULL;
    OutForm of;
    int N = 0;
    int rc = segment_form(S, seg_n, w_scales, &N, &of);
    if (rc == BITNET_OK) rc = check_shape(M, K, N, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    if (workspace == nullptr || workspace_size < workspace_bytes(M, K, act_bits))
        return BITNET_ERR_WORKSPACE;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(M, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, nullptr, s);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 0.0f, out, nullptr, s, of));
}

int hbitlinear_gemm_qkv_states(const uint8_t* codes, const float* scales, int M, int K, int S,
                               const int* seg_n, int act_bits, const uint8_t* packed_w,
                               const float* w_scales, const int* state_bits, int group,
                               int8_t* state_codes, float* state_scales, void* stream)
{
    if (codes == nullptr || scales == nullptr || packed_w == nullptr || state_codes == nullptr)
        return BITNET_ERR_NULL;
    OutForm of;
    int N = 0;
    int rc = states_form(S, seg_n, w_scales, state_bits, group, M, act_bits, state_scales, &N, &of);
    if (rc == BITNET_OK) rc = check_shape(M, K, N, act_bits, 0);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 0.0f, reinterpret_cast<float*>(state_codes), nullptr,
                                 (hipStream_t)stream, of));
}

int hbitlinear_forward_qkv_states(const float* x, int M, int K, int S, const int* seg_n,
                                  int act_bits, int use_hadamard, const uint8_t* packed_w,
                                  const float* w_scales, const int* state_bits, int group,
                                  int8_t* state_codes, float* state_scales, void* workspace,
                                  size_t workspace_size, void* stream)
{
    if (x == nullptr || packed_w == nullptr || state_codes == nullptr) return BITNET_ERR_NULL;
    OutForm of;
    int N = 0;
    int rc = states_form(S, seg_n, w_scales, state_bits, group, M, act_bits, state_scales, &N, &of);
    if (rc == BITNET_OK) rc = check_shape(M, K, N, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    if (workspace == nullptr || workspace_size < workspace_bytes(M, K, act_bits))
        return BITNET_ERR_WORKSPACE;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(M, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, nullptr, s);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, 1, M, K, N, act_bits, nullptr, packed_w, scales, nullptr,
                                 0.0f, reinterpret_cast<float*>(state_codes), nullptr, s, of));
}

int hbitlinear_gemm_swiglu(const uint8_t* codes, const float* scales, int M, int K, int F,
                           int act_bits, const uint8_t* packed_gate_up, float gate_scale,
                           float up_scale, float* h, void* stream)
{
    if (codes == nullptr || scales == nullptr || packed_gate_up == nullptr || h == nullptr)
        return BITNET_ERR_NULL;
    OutForm of;
    int rc = glu_form(F, gate_scale, up_scale, &of);
    if (rc == BITNET_OK) rc = check_shape(M, K, 2 * F, act_bits, 0);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, 2 * F, act_bits);
    if (rc != BITNET_OK) return rc;
    return status_of(launch_gemm(codes, 1, M, K, 2 * F, act_bits, nullptr, packed_gate_up, scales,
                                 nullptr, 0.0f, h, nullptr, (hipStream_t)stream, of));
}

int hbitlinear_forward_swiglu(const float* x, int M, int K, int F, int act_bits,
                              int use_hadamard, float* h, const uint8_t* packed_gate_up,
                              float gate_scale, float up_scale, void* workspace,
                              size_t workspace_size, void* stream)
{
    if (x == nullptr || h == nullptr || packed_gate_up == nullptr) return BITNET_ERR_NULL;
    OutForm of;
    int rc = glu_form(F, gate_scale, up_scale, &of);
    if (rc == BITNET_OK) rc = check_shape(M, K, 2 * F, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, 2 * F, act_bits);
    if (rc != BITNET_OK) return rc;
    if (workspace == nullptr || workspace_size < workspace_bytes(M, K, act_bits))
        return BITNET_ERR_WORKSPACE;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(M, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, M, K, act_bits, use_hadamard, codes, scales, nullptr, s);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, 1, M, K, 2 * F, act_bits, nullptr, packed_gate_up, scales,
                                 nullptr, 0.0f, h, nullptr, s, of));
}

int hbitlinear_gemm_dequant_grouped(const uint8_t* codes, const float* scales, int L, int M,
                                    int K, int N, int act_bits, const uint8_t* const* packed_ws,
                                    const float* w_scales, float* out, void* stream)
{
    if (codes == nullptr || scales == nullptr || packed_ws == nullptr || w_scales == nullptr ||
        out == nullptr)
        return BITNET_ERR_NULL;
    if (L <= 0) return BITNET_ERR_SHAPE;
    int rc = check_shape(M, K, N, act_bits, 0);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    if ((int64_t)L * M > (int64_t)1 << 30 || L > 65535) return BITNET_ERR_UNSUPPORTED;
    return status_of(launch_gemm(codes, L, M, K, N, act_bits, packed_ws, nullptr, scales, w_scales,
                                 0.0f, out, nullptr, (hipStream_t)stream));
}

int hbitlinear_grouped_workspace_bytes(int L, int M, int K, int act_bits, size_t* bytes_out)
{
    if (bytes_out == nullptr) return BITNET_ERR_NULL;
    if (L <= 0) return BITNET_ERR_SHAPE;
    int rc = check_shape(M, K, 1, act_bits, 0);
    if (rc != BITNET_OK) return rc;
    if ((int64_t)L * M > (int64_t)1 << 30) return BITNET_ERR_UNSUPPORTED;
    *bytes_out = workspace_bytes(L * M, K, act_bits);
    return BITNET_OK;
}

int hbitlinear_forward_grouped(int L, const float* x, int M, int K, int N, int act_bits,
                               int use_hadamard, float* out, const uint8_t* const* packed_ws,
                               const float* w_scales, void* workspace, size_t workspace_size,
                               void* stream)
{
    if (x == nullptr || out == nullptr || packed_ws == nullptr || w_scales == nullptr)
        return BITNET_ERR_NULL;
    if (L <= 0) return BITNET_ERR_SHAPE;
    int rc = check_shape(M, K, N, act_bits, use_hadamard);
    if (rc == BITNET_OK) rc = check_gemm_limits(M, K, N, act_bits);
    if (rc != BITNET_OK) return rc;
    if ((int64_t)L * M > (int64_t)1 << 30 || L > 65535) return BITNET_ERR_UNSUPPORTED;
    const int rows = L * M;
    if (workspace == nullptr || workspace_size < workspace_bytes(rows, K, act_bits))
        return BITNET_ERR_WORKSPACE;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + align256(codes_bytes(rows, K, act_bits)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize(x, rows, K, act_bits, use_hadamard, codes, scales, nullptr, s);
    if (e != hipSuccess) return BITNET_ERR_HIP;
    return status_of(launch_gemm(codes, L, M, K, N, act_bits, packed_ws, nullptr, scales, w_scales,
                                 0.0f, out, nullptr, s));
}

}  // extern "C"
