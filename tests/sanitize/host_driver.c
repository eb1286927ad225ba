/* host_driver.c -- exercises the CPU oracle and the library's host-side packer under
 * AddressSanitizer and UndefinedBehaviorSanitizer (built with gcc by tests/test_sanitizers.py).
 * Test infrastructure only: every call below is checked, and the process exits non-zero on the
 * first disagreement; a memory or UB error aborts it through the sanitizers. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bitnet.h"

/* the oracle's entry points (oracle/bitnet_oracle.c) */
int bitnet_ref_encode5(const int *digits);
int bitnet_ref_decode5(int byte, int *digits);
void bitnet_ref_ternarize(const float *W, int N, int K, int8_t *t, float *gamma_out);
int64_t bitnet_ref_packed_bytes(int N, int K);
int64_t bitnet_ref_row_bytes(int K);
void bitnet_ref_pack(const int8_t *t, int N, int K, uint8_t *packed);
int bitnet_ref_unpack(const uint8_t *packed, int N, int K, int8_t *t);
void bitnet_ref_hadamard(float *x, int n);
void bitnet_ref_quantize(const float *x, int M, int K, int bits, int use_hadamard, int8_t *q,
                         float *scales, float *xh);
void bitnet_ref_pack_int4(const int8_t *q, int64_t count, uint8_t *out);
void bitnet_ref_unpack_int4(const uint8_t *in, int64_t count, int8_t *q);
void bitnet_ref_gemm(const int8_t *q, const int8_t *t, int M, int N, int K, int32_t *acc);
int bitnet_ref_forward(const float *x, int M, int K, int N, int bits, int use_hadamard,
                       const uint8_t *packed, float gamma_w, float *y);
int bitnet_ref_forward_segments(const float *x, int M, int K, int S, const int *seg_n, int bits,
                                int use_hadamard, const uint8_t *const *packed,
                                const float *gammas, float *y);
int bitnet_ref_forward_swiglu(const float *x, int M, int K, int F, int bits, int use_hadamard,
                              const uint8_t *packed_gate, float gamma_gate,
                              const uint8_t *packed_up, float gamma_up, float *h);
int bitnet_ref_forward_rmsnorm(const float *x, int M, int K, int N, const float *gain, float eps,
                               int bits, int use_hadamard, const uint8_t *packed, float gamma_w,
                               float *y);
void bitnet_ref_pack_weights_hadamard(const float *W, int N, int K, uint8_t *packed,
                                      float *gamma_out);
int bitnet_ref_forward_qkv_states(const float *x, int M, int K, int S, const int *seg_n,
                                  int act_bits, int use_hadamard, const uint8_t *const *packed,
                                  const float *gammas, const int *bits, int group, int8_t *codes,
                                  float *scales);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float frand(void) /* xorshift64*, uniform in [-1, 1) */
{
    rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
    return (float)((double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0) * 2.0f - 1.0f;
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); exit(1); } } while (0)

static float *random_matrix(int rows, int cols, float scale)
{
    float *a = malloc(sizeof(float) * (size_t)rows * (size_t)cols);
    for (int64_t i = 0; i < (int64_t)rows * cols; i++) a[i] = scale * frand();
    return a;
}

/* the library's packer against the oracle: same scale, same trits read back */
static void check_packer(int N, int K)
{
    float *W = random_matrix(N, K, 0.05f);
    size_t bytes = 0;
    CHECK(bitnet_packed_bytes(N, K, &bytes) == BITNET_OK);
    uint8_t *packed = malloc(bytes);
    float g = 0.0f, og = 0.0f;
    CHECK(bitnet_pack_weights(W, N, K, packed, &g) == BITNET_OK);
    int8_t *t = malloc((size_t)N * K), *ot = malloc((size_t)N * K);
    CHECK(bitnet_unpack_weights(packed, N, K, t) == BITNET_OK);
    bitnet_ref_ternarize(W, N, K, ot, &og);
    CHECK(g == og);
    CHECK(memcmp(t, ot, (size_t)N * K) == 0);
    /* the oracle's canonical bytes round-trip too */
    uint8_t *op = malloc((size_t)bitnet_ref_packed_bytes(N, K));
    bitnet_ref_pack(ot, N, K, op);
    int8_t *t2 = malloc((size_t)N * K);
    CHECK(bitnet_ref_unpack(op, N, K, t2) == 0);
    CHECK(memcmp(t2, ot, (size_t)N * K) == 0);
    free(W); free(packed); free(t); free(ot); free(op); free(t2);
}

int main(void)
{
    /* byte code */
    for (int v = 0; v < 256; v++) {
        int d[5];
        int rc = bitnet_ref_decode5(v, d);
        CHECK((v <= 242) == (rc == 0));
        if (rc == 0) CHECK(bitnet_ref_encode5(d) == v);
    }
    /* packers: ragged widths and row counts (pad rows, pad blocks) */
    const int shapes[][2] = {{1, 1}, {3, 5}, {17, 319}, {5, 320}, {33, 321}, {16, 1000}, {40, 4096}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); i++) check_packer(shapes[i][0], shapes[i][1]);

    /* stacked segments and gate / up interleave (in-place moves inside the output) */
    {
        const int K = 640, S = 3, seg[3] = {16, 48, 32};
        float *W = random_matrix(96, K, 0.02f);
        size_t bytes = 0;
        CHECK(bitnet_packed_bytes(96, K, &bytes) == BITNET_OK);
        uint8_t *p = malloc(bytes);
        float gs[3];
        CHECK(bitnet_pack_weights_segments(W, S, seg, K, p, gs) == BITNET_OK);
        int8_t *t = malloc((size_t)96 * K);
        CHECK(bitnet_unpack_weights(p, 96, K, t) == BITNET_OK);
        free(W); free(p); free(t);
    }
    for (int F = 16; F <= 64; F += 48) {
        const int K = 1000;
        float *Wg = random_matrix(F, K, 0.02f), *Wu = random_matrix(F, K, 0.03f);
        size_t bytes = 0;
        CHECK(bitnet_packed_bytes(2 * F, K, &bytes) == BITNET_OK);
        uint8_t *p = malloc(bytes);
        float gg = 0, gu = 0, og = 0, ou = 0;
        CHECK(bitnet_pack_gate_up(Wg, Wu, F, K, p, &gg, &gu) == BITNET_OK);
        int8_t *t = malloc((size_t)2 * F * K), *tg = malloc((size_t)F * K), *tu = malloc((size_t)F * K);
        CHECK(bitnet_unpack_weights(p, 2 * F, K, t) == BITNET_OK);
        bitnet_ref_ternarize(Wg, F, K, tg, &og);
        bitnet_ref_ternarize(Wu, F, K, tu, &ou);
        CHECK(gg == og && gu == ou);
        for (int i = 0; i < F / 16; i++) {
            CHECK(memcmp(t + (int64_t)(32 * i) * K, tg + (int64_t)(16 * i) * K, (size_t)16 * K) == 0);
            CHECK(memcmp(t + (int64_t)(32 * i + 16) * K, tu + (int64_t)(16 * i) * K, (size_t)16 * K) == 0);
        }
        free(Wg); free(Wu); free(p); free(t); free(tg); free(tu);
    }
    /* rotated packing: the library and the oracle agree on the trits */
    {
        const int N = 16, K = 256;
        float *W = random_matrix(N, K, 0.02f);
        size_t bytes = 0;
        CHECK(bitnet_packed_bytes(N, K, &bytes) == BITNET_OK);
        uint8_t *p = malloc(bytes), *op = malloc((size_t)bitnet_ref_packed_bytes(N, K));
        float g = 0, og = 0;
        CHECK(bitnet_pack_weights_hadamard(W, N, K, p, &g) == BITNET_OK);
        bitnet_ref_pack_weights_hadamard(W, N, K, op, &og);
        int8_t *t = malloc((size_t)N * K), *ot = malloc((size_t)N * K);
        CHECK(bitnet_unpack_weights(p, N, K, t) == BITNET_OK);
        CHECK(bitnet_ref_unpack(op, N, K, ot) == 0);
        CHECK(g == og && memcmp(t, ot, (size_t)N * K) == 0);
        free(W); free(p); free(op); free(t); free(ot);
    }
    /* oracle forward paths on small shapes */
    {
        const int M = 5, K = 512, N = 64;
        float *x = random_matrix(M, K, 3.0f);
        memset(x + K, 0, sizeof(float) * K);            /* a zero row */
        float *W = random_matrix(N, K, 0.02f), *gain = random_matrix(1, K, 1.0f);
        int8_t *t = malloc((size_t)N * K);
        float g = 0;
        bitnet_ref_ternarize(W, N, K, t, &g);
        uint8_t *op = malloc((size_t)bitnet_ref_packed_bytes(N, K));
        bitnet_ref_pack(t, N, K, op);
        float *y = malloc(sizeof(float) * M * N), *xh = malloc(sizeof(float) * M * K), s[5];
        int8_t *q = malloc((size_t)M * K);
        for (int bits = 4; bits <= 8; bits += 4)
            for (int had = 0; had <= 1; had++) {
                bitnet_ref_quantize(x, M, K, bits, had, q, s, xh);
                CHECK(bitnet_ref_forward(x, M, K, N, bits, had, op, g, y) == 0);
                CHECK(bitnet_ref_forward_rmsnorm(x, M, K, N, gain, 1e-6f, bits, had, op, g, y) == 0);
            }
        uint8_t *b4 = malloc((size_t)M * K / 2);
        int8_t *q2 = malloc((size_t)M * K);
        bitnet_ref_quantize(x, M, K, 4, 1, q, s, NULL);
        bitnet_ref_pack_int4(q, (int64_t)M * K, b4);
        bitnet_ref_unpack_int4(b4, (int64_t)M * K, q2);
        CHECK(memcmp(q, q2, (size_t)M * K) == 0);
        int32_t *acc = malloc(sizeof(int32_t) * M * N);
        bitnet_ref_gemm(q, t, M, N, K, acc);
        const uint8_t *packs[3] = {op, op, op};
        const float gs[3] = {g, g, g};
        const int seg[3] = {64, 64, 64}, sbits[3] = {4, 3, 3};
        float *y3 = malloc(sizeof(float) * M * 192), *h = malloc(sizeof(float) * M * N);
        CHECK(bitnet_ref_forward_segments(x, M, K, 3, seg, 4, 1, packs, gs, y3) == 0);
        CHECK(bitnet_ref_forward_swiglu(x, M, K, N, 4, 1, op, g, op, g, h) == 0);
        int8_t *sc = malloc((size_t)M * 192);
        float *ss = malloc(sizeof(float) * M * 3);
        CHECK(bitnet_ref_forward_qkv_states(x, M, K, 3, seg, 4, 1, packs, gs, sbits, 64, sc, ss) == 0);
        free(x); free(W); free(gain); free(t); free(op); free(y); free(xh); free(q); free(b4);
        free(q2); free(acc); free(y3); free(h); free(sc); free(ss);
    }
    /* argument checks of the host entry points */
    size_t bytes = 0;
    CHECK(bitnet_packed_bytes(0, 5, &bytes) == BITNET_ERR_SHAPE);
    CHECK(bitnet_pack_weights(NULL, 1, 1, NULL, NULL) == BITNET_ERR_NULL);
    puts("host driver ok");
    return 0;
}
