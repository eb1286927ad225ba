/*
 * bitnet_oracle.c -- plain CPU statement of the H-BitLinear forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls this
 * file, and this file includes nothing of the product.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark load it (as liboracle_bitnet.so through ctypes).
 *
 * Every function follows one passage of the source pages, cited by page and section:
 *   [v2-news]   BitNet v2 news write-up (Xinzhiyuan, kaiyunao.com mirror): the H-BitLinear
 *               passage (online Hadamard before activation quantisation; +1/-1 entries with
 *               mutually orthogonal rows; INT4 activations for every linear but embeddings).
 *   [v2-abs]    "BitNet v2: Native 4-bit Activations with Hadamard Transformation for 1-bit
 *               LLMs" (chatpaper.ai abstract): H-BitLinear applies an online Hadamard
 *               transformation prior to activation quantization.
 *   [2B4T-1.1]  BitNet b1.58 2B4T write-up (itdecent.cn), section 1.1 "ternary weights and
 *               1.58-bit storage": five ternary weights packed into one byte, worked example
 *               (2,0,1,2,1) -> 178 = 0b10110010.
 *   [2B4T-1.2]  same page, section 1.2 "BitLinear": weights by absmean to 1.58 bit,
 *               activations by absmax to 8 bit (W1.58A8); x1 is an add, x-1 a subtract,
 *               x0 is skipped.
 *   [b158]      BitNet b1.58 summary of arXiv 2402.17764 (gptget.net), "method" and
 *               "method details": absmean quantisation constrains weights to {-1,0,+1};
 *               BitLinear replaces nn.Linear.
 *
 * Where the pages are silent the plainest reading is taken; each such reading is noted at
 * the function that makes it.  Every function is pinned by the tests to values the pages or
 * the mathematics fix, except one choice: the rounding mode of the quantisers (round half to
 * even) is a reading no page fixes -- parity unpinned for that choice; the kernels make the
 * same one, so parity holds by construction.  Floating point follows the precision the layer computes in
 * (fp32 activations and scales; the weight mean is accumulated in double).  Build with
 * -O2 -ffp-contract=off and no fast-math so that every fp32 operation is one IEEE rounding.
 *
 * Loops over independent rows carry an OpenMP pragma; that changes no result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------- */
/* Base-3 byte code [2B4T-1.1].                                                           */
/* A byte holds five ternary digits d_0..d_4 (d = t + 1 in {0,1,2}), d_0 most significant: */
/* byte = 81 d_0 + 27 d_1 + 9 d_2 + 3 d_3 + d_4.  The worked example (2,0,1,2,1) -> 178    */
/* fixes the digit order (least-significant-first would give 146).                          */
/* ------------------------------------------------------------------------------------- */

int bitnet_ref_encode5(const int *digits)
{
    int v = 0;
    for (int i = 0; i < 5; i++) {
        if (digits[i] < 0 || digits[i] > 2) return -1;
        v = v * 3 + digits[i];
    }
    return v;
}

/* Returns 0 on success, -1 for a byte that is not a base-3 code (> 242). */
int bitnet_ref_decode5(int byte, int *digits)
{
    if (byte < 0 || byte > 242) return -1;
    int v = byte;
    for (int i = 4; i >= 0; i--) {
        digits[i] = v % 3;
        v /= 3;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------- */
/* absmean ternarisation [b158 method; 2B4T-1.2].                                          */
/* gamma = mean |W| over the whole matrix (one scale per tensor: the pages give no finer     */
/* granularity), summed in double in row-major order; t = RoundClip(W / gamma, -1, 1) with    */
/* an fp32 division and round-half-to-even.  The pages give no epsilon: a zero matrix (gamma */
/* == 0) ternarises to all zeros.                                                           */
/* ------------------------------------------------------------------------------------- */

float bitnet_ref_absmean(const float *W, int64_t count)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; i++) s += fabs((double)W[i]);
    return (float)(s / (double)count);
}

void bitnet_ref_ternarize(const float *W, int N, int K, int8_t *t, float *gamma_out)
{
    int64_t count = (int64_t)N * K;
    float g = bitnet_ref_absmean(W, count);
    *gamma_out = g;
    for (int64_t i = 0; i < count; i++) {
        if (g == 0.0f) { t[i] = 0; continue; }
        float r = nearbyintf(W[i] / g);
        t[i] = (int8_t)(r > 1.0f ? 1 : (r < -1.0f ? -1 : (int)r));
    }
}

/* ------------------------------------------------------------------------------------- */
/* Packed weight matrix.  The pages fix the byte code (five trits, base 3, MSB first) but    */
/* not which five weights share a byte.  Reading taken: a row is cut into blocks of 320      */
/* weights (64 bytes); byte b of block B holds the weights k = 320 B + b + 64 i as digit i    */
/* (i = 0..4).  Bytes are stored row-major: byte b of block B of row n is byte               */
/* n * row_bytes + 64 B + b, row_bytes = 64 * ceil(K / 320).  Weights past the end of a row   */
/* (k >= K) are t = 0 (digit 1).  Where a device keeps these bytes is its own affair: any     */
/* other placement is a permutation of this array.                                          */
/* ------------------------------------------------------------------------------------- */

int64_t bitnet_ref_row_bytes(int K) { return 64 * (int64_t)((K + 319) / 320); }

int64_t bitnet_ref_packed_bytes(int N, int K) { return (int64_t)N * bitnet_ref_row_bytes(K); }

void bitnet_ref_pack(const int8_t *t, int N, int K, uint8_t *packed)
{
    int nblk = (K + 319) / 320;
    int64_t rb = bitnet_ref_row_bytes(K);
    for (int n = 0; n < N; n++) {
        for (int B = 0; B < nblk; B++) {
            for (int b = 0; b < 64; b++) {
                int digits[5];
                for (int i = 0; i < 5; i++) {
                    int64_t k = 320 * (int64_t)B + b + 64 * i;
                    int tv = k < K ? t[(int64_t)n * K + k] : 0;
                    digits[i] = tv + 1;
                }
                packed[(int64_t)n * rb + 64 * B + b] = (uint8_t)bitnet_ref_encode5(digits);
            }
        }
    }
}

/* Inverse of bitnet_ref_pack.  Returns 0, or -1 if a byte is not a base-3 code or a padding */
/* position (k >= K) holds a non-zero weight.                                                */
int bitnet_ref_unpack(const uint8_t *packed, int N, int K, int8_t *t)
{
    int nblk = (K + 319) / 320;
    int64_t rb = bitnet_ref_row_bytes(K);
    for (int n = 0; n < N; n++) {
        for (int B = 0; B < nblk; B++) {
            for (int b = 0; b < 64; b++) {
                int digits[5];
                if (bitnet_ref_decode5(packed[(int64_t)n * rb + 64 * B + b], digits) != 0)
                    return -1;
                for (int i = 0; i < 5; i++) {
                    int64_t k = 320 * (int64_t)B + b + 64 * i;
                    if (k < K) t[(int64_t)n * K + k] = (int8_t)(digits[i] - 1);
                    else if (digits[i] != 1) return -1;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------- */
/* Online Hadamard transform [v2-news H-BitLinear passage; v2-abs].                         */
/* H_n has +1/-1 entries and orthogonal rows; reading taken: the Sylvester matrix            */
/* H[i][j] = (-1)^popcount(i & j), normalised by 1/sqrt(n), applied to each token row.       */
/* The fast transform runs its radix-2 stages with the butterfly span h = 1, 2, 4, ..., n/2  */
/* (low index bit first); the pages give no order, and this one is what the in-place         */
/* butterfly computes.  Unnormalised here; bitnet_ref_hadamard applies the 1/sqrt(n) once,   */
/* after the last stage, as the fp32 constant (float)(1/sqrt((double)n)).                    */
/* ------------------------------------------------------------------------------------- */

void bitnet_ref_fwht(float *x, int n)
{
    for (int h = 1; h < n; h *= 2) {
        for (int base = 0; base < n; base += 2 * h) {
            for (int j = base; j < base + h; j++) {
                float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
        }
    }
}

void bitnet_ref_fwht_f64(double *x, int n)
{
    for (int h = 1; h < n; h *= 2) {
        for (int base = 0; base < n; base += 2 * h) {
            for (int j = base; j < base + h; j++) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
        }
    }
}

float bitnet_ref_hadamard_scale(int n) { return (float)(1.0 / sqrt((double)n)); }

void bitnet_ref_hadamard(float *x, int n)
{
    bitnet_ref_fwht(x, n);
    float c = bitnet_ref_hadamard_scale(n);
    for (int k = 0; k < n; k++) x[k] = x[k] * c;
}

/* ------------------------------------------------------------------------------------- */
/* Per-token absmax quantisation [2B4T-1.2 (8 bit, absmax); v2-news (4 bit for all          */
/* linears)].  The 4-bit formula is missing from the page; reading taken: the same absmax    */
/* rule with Qp = 2^(b-1) - 1 (127 or 7) and codes clipped to [-Qp-1, Qp].                   */
/*   gamma = max_k |x_k|;  inv = Qp / gamma (fp32 division);                                */
/*   q_k = clamp(rne(x_k * inv), -Qp-1, Qp);  scale = gamma / Qp (fp32 division).           */
/* No epsilon: an all-zero row has gamma = 0, codes 0 and scale 0.                          */
/* ------------------------------------------------------------------------------------- */

void bitnet_ref_quantize_row(const float *x, int K, int bits, int8_t *q, float *scale_out)
{
    int qp = (1 << (bits - 1)) - 1;
    float g = 0.0f;
    for (int k = 0; k < K; k++) {
        float a = fabsf(x[k]);
        if (a > g) g = a;
    }
    if (g == 0.0f) {
        for (int k = 0; k < K; k++) q[k] = 0;
        *scale_out = 0.0f;
        return;
    }
    float inv = (float)qp / g;
    for (int k = 0; k < K; k++) {
        float r = nearbyintf(x[k] * inv);
        int v = (int)r;
        if (v > qp) v = qp;
        if (v < -qp - 1) v = -qp - 1;
        q[k] = (int8_t)v;
    }
    *scale_out = g / (float)qp;
}

/* INT4 codes two to a byte.  The pages say only that activations are 4-bit; the nibble order  */
/* taken here: codes are grouped in eights, k = 8w .. 8w+7, stored in the 4-byte word w of the */
/* row; byte p (p = 0..3) of that word holds code 8w+p in its low nibble and code 8w+p+4 in   */
/* its high nibble (two's complement nibbles).  count must be a multiple of 8.               */
void bitnet_ref_pack_int4(const int8_t *q, int64_t count, uint8_t *out)
{
    for (int64_t w = 0; w < count / 8; w++)
        for (int p = 0; p < 4; p++)
            out[4 * w + p] = (uint8_t)((q[8 * w + p] & 0xF) | ((q[8 * w + p + 4] & 0xF) << 4));
}

void bitnet_ref_unpack_int4(const uint8_t *in, int64_t count, int8_t *q)
{
    for (int64_t w = 0; w < count / 8; w++)
        for (int p = 0; p < 4; p++) {
            int lo = in[4 * w + p] & 0xF, hi = in[4 * w + p] >> 4;
            q[8 * w + p] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            q[8 * w + p + 4] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
}

/* Activation stage of H-BitLinear for M token rows: optional normalised Hadamard, then      */
/* absmax quantisation.  q is M x K int8 (one code per byte, unpacked); xh (M x K fp32, may   */
/* be NULL) receives the post-Hadamard values (the input itself when use_hadamard == 0).    */
void bitnet_ref_quantize(const float *x, int M, int K, int bits, int use_hadamard,
                         int8_t *q, float *scales, float *xh)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; m++) {
        float *row = (float *)malloc(sizeof(float) * (size_t)K);
        memcpy(row, x + (int64_t)m * K, sizeof(float) * (size_t)K);
        if (use_hadamard) bitnet_ref_hadamard(row, K);
        if (xh) memcpy(xh + (int64_t)m * K, row, sizeof(float) * (size_t)K);
        bitnet_ref_quantize_row(row, K, bits, q + (int64_t)m * K, &scales[m]);
        free(row);
    }
}

/* ------------------------------------------------------------------------------------- */
/* Ternary matrix product [2B4T-1.2]: with weights in {-1,0,+1} a product term is an add     */
/* (t = +1), a subtract (t = -1) or nothing (t = 0).  acc[m][n] = sum_k q[m][k] t[n][k] in   */
/* int32; t is N x K (nn.Linear convention, [b158 method details]).                          */
/* ------------------------------------------------------------------------------------- */

void bitnet_ref_gemm(const int8_t *q, const int8_t *t, int M, int N, int K, int32_t *acc)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; m++) {
        const int8_t *qr = q + (int64_t)m * K;
        for (int n = 0; n < N; n++) {
            const int8_t *tr = t + (int64_t)n * K;
            int32_t s = 0;
            for (int k = 0; k < K; k++) {
                if (tr[k] == 1) s += qr[k];
                else if (tr[k] == -1) s -= qr[k];
            }
            acc[(int64_t)m * N + n] = s;
        }
    }
}

/* Dequantisation: y = (float(acc) * scale_x[m]) * gamma_w, left to right in fp32.  The      */
/* block has no bias term [v2-news: LLaMA-like components with the bias removed].            */
void bitnet_ref_epilogue(const int32_t *acc, const float *scales, float gamma_w, int M, int N,
                         float *y)
{
    for (int m = 0; m < M; m++)
        for (int n = 0; n < N; n++) {
            int64_t i = (int64_t)m * N + n;
            y[i] = ((float)acc[i] * scales[m]) * gamma_w;
        }
}

/* The whole forward for a packed weight matrix: unpack, activation stage, ternary product,  */
/* dequantisation.  Returns 0, or -1 if the packed buffer does not decode.                  */
int bitnet_ref_forward(const float *x, int M, int K, int N, int bits, int use_hadamard,
                       const uint8_t *packed, float gamma_w, float *y)
{
    int8_t *t = (int8_t *)malloc((size_t)N * (size_t)K);
    int8_t *q = (int8_t *)malloc((size_t)M * (size_t)K);
    float *s = (float *)malloc(sizeof(float) * (size_t)M);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)M * (size_t)N);
    int rc = bitnet_ref_unpack(packed, N, K, t);
    if (rc == 0) {
        bitnet_ref_quantize(x, M, K, bits, use_hadamard, q, s, NULL);
        bitnet_ref_gemm(q, t, M, N, K, acc);
        bitnet_ref_epilogue(acc, s, gamma_w, M, N, y);
    }
    free(t); free(q); free(s); free(acc);
    return rc;
}

/* ------------------------------------------------------------------------------------- */
/* Weight + activation Hadamard variant [v2-news: Hadamard rotation of weights and           */
/* activations, or of activations only, both stabilise low-bit training (model-size table)]. */
/* With the activations rotated, x_h = x H / sqrt(K), the weights are rotated the same way,   */
/* W_h = W H / sqrt(K) row by row, so that x_h W_h^T = x W^T before quantisation.  Reading    */
/* taken: the rotation is offline, in double with the same radix-2 order as the activation    */
/* transform, multiplied by 1/sqrt(K) in double and rounded to fp32 once; then W_h is         */
/* ternarised and packed exactly as any weight.  K must be a power of two.                    */
/* ------------------------------------------------------------------------------------- */
void bitnet_ref_rotate_weights(const float *W, int N, int K, float *Wh)
{
    double *row = (double *)malloc(sizeof(double) * (size_t)K);
    const double c = 1.0 / sqrt((double)K);
    for (int n = 0; n < N; n++) {
        for (int k = 0; k < K; k++) row[k] = (double)W[(int64_t)n * K + k];
        bitnet_ref_fwht_f64(row, K);
        for (int k = 0; k < K; k++) Wh[(int64_t)n * K + k] = (float)(row[k] * c);
    }
    free(row);
}

/* rotate, ternarise, pack: the offline step of the variant */
void bitnet_ref_pack_weights_hadamard(const float *W, int N, int K, uint8_t *packed, float *gamma_out)
{
    float *Wh = (float *)malloc(sizeof(float) * (size_t)N * (size_t)K);
    int8_t *t = (int8_t *)malloc((size_t)N * (size_t)K);
    bitnet_ref_rotate_weights(W, N, K, Wh);
    bitnet_ref_ternarize(Wh, N, K, t, gamma_out);
    bitnet_ref_pack(t, N, K, packed);
    free(Wh); free(t);
}

/* ------------------------------------------------------------------------------------- */
/* RMS normalisation of a token row before its activation stage [v2-news: LLaMA-like        */
/* components, among them RMS normalisation; 2B4T write-up section 1.3: subln               */
/* normalisation].  Reading taken: y[k] = (x[k] * r) * gain[k] with                          */
/* r = 1 / sqrt(mean_k x[k]^2 + eps); eps is the caller's (the pages give none).  The sum of  */
/* squares is taken in double (each fp32 square is exact there), r is computed in double and */
/* rounded to fp32 once; a row whose mean square plus eps is 0 gives r = 0 (a zero row).      */
/* ------------------------------------------------------------------------------------- */
float bitnet_ref_rms_scale(const float *x, int K, float eps)
{
    double ss = 0.0;
    for (int k = 0; k < K; k++) ss += (double)x[k] * (double)x[k];
    const double ms = ss / (double)K + (double)eps;
    return ms > 0.0 ? (float)(1.0 / sqrt(ms)) : 0.0f;
}

void bitnet_ref_rmsnorm(const float *x, int M, int K, const float *gain, float eps, float *y)
{
    for (int m = 0; m < M; m++) {
        const float *xr = x + (int64_t)m * K;
        const float r = bitnet_ref_rms_scale(xr, K, eps);
        for (int k = 0; k < K; k++) y[(int64_t)m * K + k] = (xr[k] * r) * gain[k];
    }
}

/* The forward with the norm in front: rmsnorm, then bitnet_ref_forward. */
int bitnet_ref_forward_rmsnorm(const float *x, int M, int K, int N, const float *gain, float eps,
                               int bits, int use_hadamard, const uint8_t *packed, float gamma_w,
                               float *y)
{
    float *xn = (float *)malloc(sizeof(float) * (size_t)M * (size_t)K);
    bitnet_ref_rmsnorm(x, M, K, gain, eps, xn);
    int rc = bitnet_ref_forward(xn, M, K, N, bits, use_hadamard, packed, gamma_w, y);
    free(xn);
    return rc;
}

/* ------------------------------------------------------------------------------------- */
/* Several linears that read the same input (for instance Q, K and V of a block), each with  */
/* its own packed weights and weight scale: y is M x (N_0 + ... + N_{S-1}), segment s in the */
/* columns that follow segments 0 .. s-1, each exactly bitnet_ref_forward of that matrix.     */
/* packed: S pointers to separately packed matrices (N_s x K each).                          */
/* ------------------------------------------------------------------------------------- */
int bitnet_ref_forward_segments(const float *x, int M, int K, int S, const int *seg_n, int bits,
                                int use_hadamard, const uint8_t *const *packed,
                                const float *gammas, float *y)
{
    int ntot = 0;
    for (int s = 0; s < S; s++) ntot += seg_n[s];
    int rc = 0, col = 0;
    for (int s = 0; s < S && rc == 0; s++) {
        const int N = seg_n[s];
        float *ys = (float *)malloc(sizeof(float) * (size_t)M * (size_t)N);
        rc = bitnet_ref_forward(x, M, K, N, bits, use_hadamard, packed[s], gammas[s], ys);
        for (int m = 0; m < M && rc == 0; m++)
            memcpy(y + (int64_t)m * ntot + col, ys + (int64_t)m * N, sizeof(float) * (size_t)N);
        free(ys);
        col += N;
    }
    return rc;
}

/* ------------------------------------------------------------------------------------- */
/* Gated feed-forward glue [v2-news: LLaMA-like components, among them the SwishGLU          */
/* activation].  Reading taken: Swish with beta = 1, i.e. SiLU(z) = z * sigmoid(z) =          */
/* z / (1 + e^-z), and SwishGLU(x) = SiLU(x W_gate^T) (elementwise product) (x W_up^T), the    */
/* two products being two BitLinear forwards of the same input.  The pages fix no precision  */
/* for the glue; it is evaluated in double and rounded to fp32 once.                          */
/* ------------------------------------------------------------------------------------- */
float bitnet_ref_silu(float z)
{
    const double d = (double)z;
    return (float)(d / (1.0 + exp(-d)));
}

void bitnet_ref_swiglu(const float *g, const float *u, int64_t count, float *h)
{
    for (int64_t i = 0; i < count; i++) {
        const double d = (double)g[i];
        h[i] = (float)((d / (1.0 + exp(-d))) * (double)u[i]);
    }
}

/* h (M x F) = SwishGLU of the gate and up forwards of x (each a bitnet_ref_forward with its  */
/* own packed F x K matrix and weight scale).                                                */
int bitnet_ref_forward_swiglu(const float *x, int M, int K, int F, int bits, int use_hadamard,
                              const uint8_t *packed_gate, float gamma_gate,
                              const uint8_t *packed_up, float gamma_up, float *h)
{
    float *g = (float *)malloc(sizeof(float) * (size_t)M * (size_t)F);
    float *u = (float *)malloc(sizeof(float) * (size_t)M * (size_t)F);
    int rc = bitnet_ref_forward(x, M, K, F, bits, use_hadamard, packed_gate, gamma_gate, g);
    if (rc == 0) rc = bitnet_ref_forward(x, M, K, F, bits, use_hadamard, packed_up, gamma_up, u);
    if (rc == 0) bitnet_ref_swiglu(g, u, (int64_t)M * F, h);
    free(g); free(u);
    return rc;
}

/* ------------------------------------------------------------------------------------- */
/* Low-bit Q/K/V states [v2-news: the QKV states of the attention are kept at a reduced bit  */
/* width (zero-shot tables 2 and 3, a8 and a4, QKV-state widths varied), and a 3-bit KV      */
/* cache matches a full-precision one].  The page gives no quantiser.  Reading taken: the     */
/* layer's own absmax rule, applied to the fp32 outputs y of the Q, K and V projections per  */
/* token and per group of `group` consecutive output columns (one attention head):           */
/*   gamma = max |y| over the group;  Qp = 2^(b-1) - 1 with b the segment's bit width;        */
/*   q = clamp(rne(y * (Qp / gamma)), -Qp-1, Qp) (fp32 division, then a multiply);           */
/*   scale = gamma / Qp;  a group of zeros gives codes 0 and scale 0.                          */
/* y is M x Ntot with the segments side by side (Ntot = sum seg_n); `group` divides every    */
/* seg_n.  codes: M x Ntot int8 (one code per byte); scales: M x (Ntot / group) fp32, group j  */
/* of row m at m * (Ntot / group) + j.                                                         */
/* ------------------------------------------------------------------------------------- */
void bitnet_ref_quantize_states(const float *y, int M, int Ntot, int S, const int *seg_n,
                                const int *bits, int group, int8_t *codes, float *scales)
{
    const int ngroups = Ntot / group;
    for (int m = 0; m < M; m++) {
        int col = 0;
        for (int s = 0; s < S; s++) {
            for (int c = col; c < col + seg_n[s]; c += group) {
                const int64_t off = (int64_t)m * Ntot + c;
                bitnet_ref_quantize_row(y + off, group, bits[s], codes + off,
                                        &scales[(int64_t)m * ngroups + c / group]);
            }
            col += seg_n[s];
        }
    }
}

/* The projections and their states in one: bitnet_ref_forward_segments, then               */
/* bitnet_ref_quantize_states of its output.                                                 */
int bitnet_ref_forward_qkv_states(const float *x, int M, int K, int S, const int *seg_n,
                                  int act_bits, int use_hadamard, const uint8_t *const *packed,
                                  const float *gammas, const int *bits, int group, int8_t *codes,
                                  float *scales)
{
    int ntot = 0;
    for (int s = 0; s < S; s++) ntot += seg_n[s];
    float *y = (float *)malloc(sizeof(float) * (size_t)M * (size_t)ntot);
    int rc = bitnet_ref_forward_segments(x, M, K, S, seg_n, act_bits, use_hadamard, packed, gammas, y);
    if (rc == 0) bitnet_ref_quantize_states(y, M, ntot, S, seg_n, bits, group, codes, scales);
    free(y);
    return rc;
}

/* Number of OpenMP threads a parallel region here uses (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int bitnet_ref_num_threads(void) { return omp_get_max_threads(); }
void bitnet_ref_set_num_threads(int n) { omp_set_num_threads(n); }
#else
int bitnet_ref_num_threads(void) { return 1; }
void bitnet_ref_set_num_threads(int n) { (void)n; }
#endif
