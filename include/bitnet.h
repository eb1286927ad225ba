/*
 * bitnet.h -- C ABI of libbitnet_hip.so: the H-BitLinear forward pass on AMD MI355X (gfx950).
 *
 * The layer (BitNet b1.58 / BitNet v2):
 *   - weights are ternarised offline by absmean and stored five trits per byte, base 3
 *     [BitNet b1.58 summary of arXiv 2402.17764 (gptget.net), method; BitNet b1.58 2B4T
 *      write-up (itdecent.cn), section 1.1, worked example (2,0,1,2,1) -> 178];
 *   - each token's activations optionally go through an online normalised Hadamard transform
 *     [BitNet v2 news write-up (Xinzhiyuan, kaiyunao.com), H-BitLinear passage; BitNet v2
 *      abstract (chatpaper.ai)], then are quantised by per-token absmax to INT8 or INT4
 *     [2B4T write-up section 1.2 (W1.58A8, absmax activations); v2 write-up (4-bit
 *      activations for all linears)];
 *   - the product with the ternary weights is integer (add / subtract / skip, int32 sums)
 *     and is rescaled to fp32 with no bias [2B4T write-up section 1.2; v2 write-up: bias
 *     removed].
 *
 * Conventions (all functions):
 *   - extern "C", return an int status: BITNET_OK (0) or a negative BITNET_ERR_* code.
 *   - Shapes: x is M x K fp32 row-major (one token per row); the weight is N x K
 *     (nn.Linear convention, y = x W^T); out is M x N fp32 row-major.
 *   - The caller owns every buffer.  The library never allocates or frees device memory and
 *     keeps no state between calls, so calls are thread-safe -- except
 *     hbitlinear_forward_noalloc, whose workspace is one static array per device (see there).
 *   - "Device" pointers are HIP device memory on the current device; "host" pointers are
 *     ordinary CPU memory.  `stream` is a hipStream_t passed as void* (NULL = null stream).
 *   - Argument checks run on the host before anything is launched; a failing check launches
 *     nothing and writes nothing.  A HIP launch error maps to BITNET_ERR_HIP.  Device-side
 *     faults surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Supported shapes: 1 <= M, 1 <= N, 64 <= K <= 65536 with K % 64 == 0; with
 *     use_hadamard = 1, K must be a power of two, 256 <= K <= 16384.  act_bits is 4 or 8.
 *     Per layer, the packed weights, the activation codes and the output (4 M N bytes) must
 *     each stay below 2 GiB.  Anything else returns BITNET_ERR_UNSUPPORTED (or
 *     BITNET_ERR_SHAPE for sizes <= 0).
 */
#ifndef BITNET_H
#define BITNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BITNET_OK = 0,
    BITNET_ERR_NULL = -1,        /* a required pointer is NULL */
    BITNET_ERR_SHAPE = -2,       /* M, N or K <= 0, or an output buffer is too small */
    BITNET_ERR_UNSUPPORTED = -3, /* valid but unsupported shape or mode (see above) */
    BITNET_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the query returned */
    BITNET_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
    BITNET_ERR_FORMAT = -6       /* a packed weight byte is not a base-3 code (> 242) */
};

/* Static text for a status code (never NULL). */
const char *bitnet_status_string(int status);

/* ABI version, currently 1. */
int bitnet_abi_version(void);

/* ------------------------------------------------------------------------------------ */
/* Offline weight preparation (host memory, synchronous).                                */
/* ------------------------------------------------------------------------------------ */

/* Size in bytes of a packed N x K weight: 16 * ceil(N / 16) * 64 * ceil(K / 320).
 * Byte code: five trits per byte, base 3, digit = t + 1, the first digit most significant,
 * byte = 81 d0 + 27 d1 + 9 d2 + 3 d3 + d4 (so the digits 2,0,1,2,1 give 178, the 2B4T
 * write-up's section 1.1 example).
 * Layout (this library's choice; the pages fix only the byte code):
 *   - which weights share a byte: row n is cut into blocks of 320 weights, 64 bytes each;
 *     byte b of block B holds the weights k = 320 B + b + 64 i as digit i (i = 0..4);
 *   - canonical order of the bytes: row-major, byte b of block B of row n at
 *     n * 64 * ceil(K/320) + 64 B + b (N * 64 * ceil(K/320) bytes);
 *   - where a byte sits in this library's buffers (a permutation of the canonical order plus
 *     pad rows): rows go in groups of 16 (the last group padded with zero rows); group G and
 *     block B form one 1024-byte tile at offset (G * ceil(K/320) + B) * 1024, and byte b of
 *     row n sits in it at ((b / 16) * 16 + n % 16) * 16 + b % 16.
 * Weights at k >= K and pad rows n >= N are t = 0.  Grouping weights 64 apart lets one
 * 16-byte load decode into five 64-wide MFMA slices, and the tile order lets one wave load
 * the 16 x 64 bytes of a tile as one contiguous kilobyte. */
int bitnet_packed_bytes(int N, int K, size_t *bytes_out);

/* absmean ternarisation and packing [gptget.net 2402.17764 summary, method; 2B4T write-up
 * section 1.1].  W_host: N x K fp32 (host).  gamma = mean |W| (double accumulation, rounded
 * to fp32 once); t = clamp(round_half_even(W / gamma), -1, 1) with an fp32 division; an
 * all-zero W gives gamma = 0 and t = 0.  packed_host: bitnet_packed_bytes(N, K) bytes
 * (host); *w_scale_out receives gamma, the value hbitlinear_forward takes as w_scale. */
int bitnet_pack_weights(const float *W_host, int N, int K, uint8_t *packed_host,
                        float *w_scale_out);

/* The weight + activation Hadamard variant [v2 write-up, model-size table: rotating weights
 * and activations, or activations only, both stabilise low-bit training]: W_host (N x K fp32,
 * host, K a power of two in [256, 16384]) is rotated the way the activations are,
 * W_h = W H_K / sqrt(K) row by row (radix-2 butterflies with span 1, 2, ..., K/2 in double,
 * times 1/sqrt(K) in double, rounded to fp32 once; a host copy of W_h is made), then
 * ternarised and packed exactly as bitnet_pack_weights.  Use with use_hadamard = 1: then
 * x_h W_h^T = x W^T before quantisation. */
int bitnet_pack_weights_hadamard(const float *W_host, int N, int K, uint8_t *packed_host,
                                 float *w_scale_out);

/* Most weight matrices one packed buffer can stack (bitnet_pack_weights_segments). */
#define BITNET_MAX_SEGMENTS 8

/* Several linears that read the same input -- e.g. the Q, K and V projections of a block --
 * prepared for one product launch: W_host stacks S matrices by rows (seg_n[s] x K each,
 * host, seg_n[s] a multiple of 16, 1 <= S <= BITNET_MAX_SEGMENTS); each is ternarised with
 * its own absmean scale (w_scales_out[s], host) exactly as bitnet_pack_weights, and the packed
 * matrices follow one another in packed_host (bitnet_packed_bytes(sum seg_n, K) bytes: whole
 * 16-row groups, so the result is the packed layout of the stacked matrix). */
int bitnet_pack_weights_segments(const float *W_host, int S, const int *seg_n, int K,
                                 uint8_t *packed_host, float *w_scales_out);

/* Gate and up projections of a gated feed-forward [v2 write-up: LLaMA-like components,
 * among them the SwishGLU activation], prepared for one product launch with the glue fused:
 * W_gate_host and W_up_host are F x K (host, F a multiple of 16), each ternarised with its own
 * absmean scale exactly as bitnet_pack_weights; packed_host (bitnet_packed_bytes(2 F, K)
 * bytes) interleaves them by 16-row groups: group 2i holds gate rows 16i..16i+15, group 2i+1
 * the same up rows.  Uses a host copy of one packed matrix while interleaving. */
int bitnet_pack_gate_up(const float *W_gate_host, const float *W_up_host, int F, int K,
                        uint8_t *packed_host, float *gate_scale_out, float *up_scale_out);

/* Inverse of the packing [2B4T write-up section 1.1: a byte holds five base-3 digits, the
 * first most significant; digit d is the trit d - 1]: packed_host (bitnet_packed_bytes(N, K)
 * bytes, host, in this library's tiled placement) is decoded into trits_host (N x K int8,
 * host, row-major), t in {-1, 0, +1}; this defines the canonical order of the packed weights.
 * Two passes: every byte is checked before anything is written, so on error trits_host is
 * untouched.  Returns BITNET_ERR_FORMAT if a byte is > 242 or a padding position (k >= K or a
 * pad row) is not t = 0. */
int bitnet_unpack_weights(const uint8_t *packed_host, int N, int K, int8_t *trits_host);

/* ------------------------------------------------------------------------------------ */
/* Forward pass (device memory, asynchronous on `stream`).                               */
/* ------------------------------------------------------------------------------------ */

/* Bytes of device workspace hbitlinear_forward needs for M tokens of width K:
 * the activation codes (hbitlinear_codes_bytes) and M fp32 scales, each 256-byte aligned. */
int hbitlinear_workspace_bytes(int M, int K, int act_bits, size_t *bytes_out);

/* H-BitLinear (use_hadamard = 1) or BitLinear (use_hadamard = 0) forward [v2 write-up,
 * H-BitLinear passage: an online Hadamard transform of the activations before their
 * quantisation, +1/-1 entries with orthogonal rows; BitNet v2 abstract (chatpaper.ai); 2B4T
 * write-up section 1.2: absmax activations, absmean ternary weights, multiplications become
 * add / subtract / skip; v2 write-up: no bias]:
 *   x_h = use_hadamard ? x H_K / sqrt(K) : x                (per token, Sylvester H_K)
 *   q, s = per-token absmax quantisation of x_h to act_bits  (Qp = 2^(b-1) - 1)
 *   out[m][n] = (float(sum_k q[m][k] t[n][k]) * s[m]) * w_scale
 * x (M x K fp32), out (M x N fp32), packed_w (bitnet_packed_bytes(N, K) bytes) and workspace
 * are device pointers; w_scale is the gamma returned by bitnet_pack_weights.  Equal to
 * hbitlinear_quantize into the workspace followed by hbitlinear_gemm_dequant. */
int hbitlinear_forward(const float *x, int M, int K, int N, int act_bits, int use_hadamard,
                       float *out, const uint8_t *packed_w, float w_scale, void *workspace,
                       size_t workspace_bytes, void *stream);

/* For callers that cannot allocate memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): hbitlinear_forward with its workspace taken from
 * a static device array of BITNET_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * GPU it runs on until the process ends, instead of a caller buffer.  Same arguments (minus
 * the workspace), same arithmetic, same result bit for bit.  It calls no allocating routine;
 * the first call on a device looks up that device's copy of the array (call it once outside
 * graph capture if the first real call is captured).  Every call on one GPU shares that GPU's
 * array, and nothing in it needs to start at any value (the activation stage writes the codes
 * and scales before the product reads them), so calls that overlap in time on one GPU -- on
 * different streams, or from different threads -- race and must be serialised by the caller.
 * Returns BITNET_ERR_WORKSPACE when hbitlinear_workspace_bytes(M, K, act_bits) exceeds
 * BITNET_NOALLOC_SCRATCH_BYTES (for example INT4 with M * K / 2 + 4 M above 16 MiB), before
 * touching the GPU; other rules as hbitlinear_forward. */
#define BITNET_NOALLOC_SCRATCH_BYTES (16u << 20)
int hbitlinear_forward_noalloc(const float *x, int M, int K, int N, int act_bits,
                               int use_hadamard, float *out, const uint8_t *packed_w,
                               float w_scale, void *stream);

/* L independent forwards of one shape in a single call -- e.g. a stack of layers whose
 * inputs are already held separately, or projections of one block -- each exactly as
 * hbitlinear_forward (same passages, same arithmetic):
 *   out[l] = forward(x[l], packed_ws[l], w_scales[l]),  l = 0 .. L-1.
 * x: L x M x K fp32 (device, contiguous); out: L x M x N fp32 (device, contiguous);
 * packed_ws: device array of L device pointers to packed N x K weights; w_scales: device
 * array of L fp32 gammas; workspace: hbitlinear_grouped_workspace_bytes(L, M, K, act_bits)
 * bytes of device memory.  The call reads packed_ws and w_scales on the device, in stream
 * order.  Shape rules as hbitlinear_forward, plus 1 <= L <= 65535. */
int hbitlinear_grouped_workspace_bytes(int L, int M, int K, int act_bits, size_t *bytes_out);
int hbitlinear_forward_grouped(int L, const float *x, int M, int K, int N, int act_bits,
                               int use_hadamard, float *out, const uint8_t *const *packed_ws,
                               const float *w_scales, void *workspace, size_t workspace_bytes,
                               void *stream);

/* The forward with the RMS normalisation in front folded into the activation stage's single
 * read of x [v2 write-up: LLaMA-like components with RMS normalisation; 2B4T write-up section
 * 1.3: subln normalisation; reading taken: per token
 *   r = fp32(1 / sqrt(sum_k x[k]^2 / K + eps))   (the sum and r in double)
 *   x'[k] = (x[k] * r) * gain[k]                  (fp32; a row with mean square + eps == 0
 *                                                  gives r = 0)
 * then exactly hbitlinear_forward on x'].  gain: K fp32 (device); eps: finite, >= 0 (the pages
 * give none; the caller's).  K must be a power of two in [256, 16384]; other rules and the
 * workspace as hbitlinear_forward. */
int hbitlinear_forward_rmsnorm(const float *x, int M, int K, int N, const float *gain, float eps,
                               int act_bits, int use_hadamard, float *out,
                               const uint8_t *packed_w, float w_scale, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Several linears of one input in one call: x's activation stage runs once, then one product
 * launch covers the S stacked matrices of bitnet_pack_weights_segments:
 *   out[m][c] = forward(x, matrix s, w_scales[s])[m][c - c_s] for the columns
 *   c_s <= c < c_s + seg_n[s] of segment s (c_s = seg_n[0] + ... + seg_n[s-1]),
 * each exactly as hbitlinear_forward.  seg_n and w_scales are host arrays of S entries;
 * x (M x K), out (M x sum seg_n), packed_w and workspace (hbitlinear_workspace_bytes(M, K,
 * act_bits)) are device pointers.  Shape rules as hbitlinear_forward with N = sum seg_n,
 * plus seg_n[s] % 16 == 0 and 1 <= S <= BITNET_MAX_SEGMENTS. */
int hbitlinear_forward_segments(const float *x, int M, int K, int S, const int *seg_n,
                                int act_bits, int use_hadamard, float *out,
                                const uint8_t *packed_w, const float *w_scales, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Low-bit Q/K/V states [v2 write-up: the attention's QKV states kept at reduced bit widths
 * (zero-shot tables 2 and 3, with 8-bit and 4-bit activations), and a 3-bit KV cache matching
 * a full-precision one; the page gives no quantiser, reading taken: the layer's absmax rule
 * per token and per head]: the projections of hbitlinear_forward_segments, y (never written
 * to memory), quantised in the product's epilogue per row and per group of `group` consecutive
 * output columns (one head) with the segment's bit width b = state_bits[s]:
 *   gamma = max |y| over the group;  Qp = 2^(b-1) - 1;
 *   q = clamp(round_half_even(y * (Qp / gamma)), -Qp-1, Qp);  scale = gamma / Qp
 *   (a group of zeros gives q = 0, scale = 0).
 * state_codes (device): M x sum(seg_n) int8, one code per byte, row-major; state_scales
 * (device): M x (sum(seg_n) / group) fp32, group j of row m at m * (sum seg_n / group) + j.
 * seg_n, w_scales, state_bits are host arrays of S entries; state_bits[s] in [2, 8]; group is
 * 64 or 128 and divides every seg_n[s].  INT8 or INT4 activations, batched shapes and decode
 * shapes (M <= 16: the new tokens' states a low-bit KV cache appends each step).  Other rules,
 * the packed weights and the workspace as hbitlinear_forward_segments. */
int hbitlinear_forward_qkv_states(const float *x, int M, int K, int S, const int *seg_n,
                                  int act_bits, int use_hadamard, const uint8_t *packed_w,
                                  const float *w_scales, const int *state_bits, int group,
                                  int8_t *state_codes, float *state_scales, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Gated feed-forward input projections with the SwishGLU glue in the product's epilogue
 * [v2 write-up: SwishGLU; reading taken: Swish with beta = 1, SiLU(z) = z / (1 + e^-z)]:
 *   g = forward(x, gate), u = forward(x, up)   (each exactly as hbitlinear_forward)
 *   h[m][f] = SiLU(g[m][f]) * u[m][f]          (fp32 with the hardware exp2 and reciprocal:
 *                                               within 1e-5 relative of the exact value for
 *                                               |g| < 80)
 * packed_gate_up as bitnet_pack_gate_up; h is M x F fp32; x, h, packed_gate_up and workspace
 * (hbitlinear_workspace_bytes(M, K, act_bits)) are device pointers.  Neither g nor u is
 * written to memory.  Shape rules as hbitlinear_forward with N = 2 F, plus F % 16 == 0. */
int hbitlinear_forward_swiglu(const float *x, int M, int K, int F, int act_bits,
                              int use_hadamard, float *h, const uint8_t *packed_gate_up,
                              float gate_scale, float up_scale, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------ */
/* The two stages of the forward, exported so each can be checked and timed on its own.  */
/* ------------------------------------------------------------------------------------ */

/* Size of the activation codes of M x K: M*K bytes (INT8) or M*K/2 bytes (INT4). */
int hbitlinear_codes_bytes(int M, int K, int act_bits, size_t *bytes_out);

/* Activation stage [v2 write-up H-BitLinear passage; 2B4T write-up section 1.2]: optional
 * normalised Hadamard (radix-2 stages with span 1, 2, 4, ..., K/2, then one fp32 multiply by
 * (float)(1/sqrt(K))), then per-token absmax quantisation:
 *   gamma = max_k |x_h[k]|;  q = clamp(round_half_even(x_h * (Qp / gamma)), -Qp-1, Qp);
 *   s = gamma / Qp;  a zero row gives q = 0, s = 0.
 * codes (device): INT8 -> M x K int8; INT4 -> M x K/2 bytes: the codes k = 8w .. 8w+7 of a row
 * live in its 4-byte word w, byte p (0..3) holding code 8w+p in the low nibble and code
 * 8w+p+4 in the high nibble (two's complement), so a word unpacks to two int8 words in k
 * order with one mask and one shift.  scales (device): M fp32.  xh_or_null (device, M x K
 * fp32, may be NULL) receives x_h. */
int hbitlinear_quantize(const float *x, int M, int K, int act_bits, int use_hadamard,
                        uint8_t *codes, float *scales, float *xh_or_null, void *stream);

/* The activation stage of hbitlinear_forward_rmsnorm: hbitlinear_quantize applied to the
 * RMS-normalised rows x' (xh_or_null receives x' after the optional transform). */
int hbitlinear_quantize_rmsnorm(const float *x, int M, int K, const float *gain, float eps,
                                int act_bits, int use_hadamard, uint8_t *codes, float *scales,
                                float *xh_or_null, void *stream);

/* Ternary product [2B4T write-up section 1.2]: acc[m][n] = sum_k q[m][k] t[n][k], exact
 * int32.  codes as written by hbitlinear_quantize; packed_w as bitnet_pack_weights; acc is
 * M x N int32 (device). */
int bitnet_ternary_gemm_i32(const uint8_t *codes, int M, int K, int N, int act_bits,
                            const uint8_t *packed_w, int32_t *acc, void *stream);

/* Ternary product fused with the dequantisation epilogue (no bias [v2 write-up]):
 * out[m][n] = (float(acc[m][n]) * scales[m]) * w_scale, fp32, left to right.  All pointers
 * device. */
int hbitlinear_gemm_dequant(const uint8_t *codes, const float *scales, int M, int K, int N,
                            int act_bits, const uint8_t *packed_w, float w_scale, float *out,
                            void *stream);

/* The product stage of hbitlinear_forward_grouped: codes / scales of L*M rows as written by
 * hbitlinear_quantize on the L x M x K input viewed as (L*M) x K; packed_ws / w_scales device
 * arrays of L entries; out L x M x N fp32.  All pointers device. */
int hbitlinear_gemm_dequant_grouped(const uint8_t *codes, const float *scales, int L, int M,
                                    int K, int N, int act_bits, const uint8_t *const *packed_ws,
                                    const float *w_scales, float *out, void *stream);

/* The product stages of hbitlinear_forward_segments, hbitlinear_forward_qkv_states and
 * hbitlinear_forward_swiglu, from codes and scales as written by hbitlinear_quantize
 * (device); seg_n, w_scales, state_bits host arrays. */
int hbitlinear_gemm_dequant_segments(const uint8_t *codes, const float *scales, int M, int K,
                                     int S, const int *seg_n, int act_bits,
                                     const uint8_t *packed_w, const float *w_scales, float *out,
                                     void *stream);
int hbitlinear_gemm_qkv_states(const uint8_t *codes, const float *scales, int M, int K, int S,
                               const int *seg_n, int act_bits, const uint8_t *packed_w,
                               const float *w_scales, const int *state_bits, int group,
                               int8_t *state_codes, float *state_scales, void *stream);
int hbitlinear_gemm_swiglu(const uint8_t *codes, const float *scales, int M, int K, int F,
                           int act_bits, const uint8_t *packed_gate_up, float gate_scale,
                           float up_scale, float *h, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H */
