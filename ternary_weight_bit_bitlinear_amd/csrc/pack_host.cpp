// pack_host.cpp -- offline weight preparation of libbitnet_hip.so (host code).
//
// absmean ternarisation [BitNet b1.58 summary of arXiv 2402.17764 (gptget.net), method: weights
// constrained to {-1, 0, +1} by the absmean function] and base-3 packing, five trits per byte
// [BitNet b1.58 2B4T write-up (itdecent.cn), section 1.1: a byte holds five ternary digits,
// most significant first -- the digits 2,0,1,2,1 give 178].
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <new>

#include "../../include/bitnet.h"

namespace {

constexpr int kBlock = 320;  // weights per 64-byte block of a packed row

int64_t packed_row_bytes(int K) { return 64 * (int64_t)((K + kBlock - 1) / kBlock); }

// Rows go in groups of 16; group G and block B form one 1024-byte tile, in which byte b of
// row n sits at ((b / 16) * 16 + n % 16) * 16 + b % 16.  One wave can then load the 16 rows x
// 64 bytes of a tile as one contiguous kilobyte.
inline int64_t tile_offset(int n, int B, int b, int nblk)
{
    return ((int64_t)(n / 16) * nblk + B) * 1024 + (int64_t)((b / 16) * 16 + n % 16) * 16 + b % 16;
}

int64_t padded_rows(int N) { return (int64_t)(N + 15) / 16 * 16; }

int check_nk(int N, int K)
{
    if (N <= 0 || K <= 0) return BITNET_ERR_SHAPE;
    if ((int64_t)N * (int64_t)K > ((int64_t)1 << 40)) return BITNET_ERR_UNSUPPORTED;
    return BITNET_OK;
}

// One trit in {-1, 0, +1}: round-half-to-even of an fp32 quotient, clipped.
inline int ternary(float w, float gamma)
{
    float r = std::nearbyint(w / gamma);
    return r >= 1.0f ? 1 : (r <= -1.0f ? -1 : 0);
}

}  // namespace

extern "C" {

int bitnet_packed_bytes(int N, int K, size_t* bytes_out)
{
    if (bytes_out == nullptr) return BITNET_ERR_NULL;
    int rc = check_nk(N, K);
    if (rc != BITNET_OK) return rc;
    *bytes_out = (size_t)padded_rows(N) * (size_t)packed_row_bytes(K);
    return BITNET_OK;
}

int bitnet_pack_weights(const float* W, int N, int K, uint8_t* packed, float* w_scale_out)
{
    if (W == nullptr || packed == nullptr || w_scale_out == nullptr) return BITNET_ERR_NULL;
    int rc = check_nk(N, K);
    if (rc != BITNET_OK) return rc;
    const int64_t count = (int64_t)N * K;
    // gamma = mean |W|: one double sum over the matrix in row-major order, rounded once.
    double sum = 0.0;
    for (int64_t i = 0; i < count; i++) sum += std::fabs((double)W[i]);
    const float gamma = (float)(sum / (double)count);
    *w_scale_out = gamma;

    const int nblk = (K + kBlock - 1) / kBlock;
    for (int n = 0; n < padded_rows(N); n++) {
        const float* wr = n < N ? W + (int64_t)n * K : W;
        for (int blk = 0; blk < nblk; blk++) {
            for (int b = 0; b < 64; b++) {
                // byte b of the block: weights k = 320 blk + b + 64 i as digit i, MSB first;
                // pad rows (n >= N) and pad columns (k >= K) are zero weights
                int v = 0;
                for (int i = 0; i < 5; i++) {
                    const int k = kBlock * blk + b + 64 * i;
                    const int t = (n < N && k < K && gamma != 0.0f) ? ternary(wr[k], gamma) : 0;
                    v = 3 * v + (t + 1);
                }
                packed[tile_offset(n, blk, b, nblk)] = (uint8_t)v;
            }
        }
    }
    return BITNET_OK;
}

int bitnet_pack_weights_hadamard(const float* W, int N, int K, uint8_t* packed, float* w_scale_out)
{
    if (W == nullptr || packed == nullptr || w_scale_out == nullptr) return BITNET_ERR_NULL;
    int rc = check_nk(N, K);
    if (rc != BITNET_OK) return rc;
    if ((K & (K - 1)) != 0 || K < 256 || K > 16384) return BITNET_ERR_UNSUPPORTED;
    // W_h = W H / sqrt(K) row by row: radix-2 butterflies with span 1, 2, ..., K/2 in double,
    // one multiply by 1/sqrt(K) in double, one rounding to fp32.
    float* Wh = new (std::nothrow) float[(size_t)N * (size_t)K];
    double* row = new (std::nothrow) double[(size_t)K];
    if (Wh == nullptr || row == nullptr) {
        delete[] Wh;
        delete[] row;
        return BITNET_ERR_UNSUPPORTED;
    }
    const double c = 1.0 / std::sqrt((double)K);
    for (int n = 0; n < N; n++) {
        for (int k = 0; k < K; k++) row[k] = (double)W[(int64_t)n * K + k];
        for (int h = 1; h < K; h *= 2)
            for (int base = 0; base < K; base += 2 * h)
                for (int j = base; j < base + h; j++) {
                    const double a = row[j], b = row[j + h];
                    row[j] = a + b;
                    row[j + h] = a - b;
                }
        for (int k = 0; k < K; k++) Wh[(int64_t)n * K + k] = (float)(row[k] * c);
    }
    rc = bitnet_pack_weights(Wh, N, K, packed, w_scale_out);
    delete[] Wh;
    delete[] row;
    return rc;
}

int bitnet_pack_weights_segments(const float* W, int S, const int* seg_n, int K, uint8_t* packed,
                                 float* w_scales_out)
{
    if (W == nullptr || seg_n == nullptr || packed == nullptr || w_scales_out == nullptr)
        return BITNET_ERR_NULL;
    if (S <= 0 || S > BITNET_MAX_SEGMENTS) return BITNET_ERR_UNSUPPORTED;
    int64_t rows = 0;
    for (int s = 0; s < S; s++) {
        if (seg_n[s] <= 0) return BITNET_ERR_SHAPE;
        if (seg_n[s] % 16 != 0) return BITNET_ERR_UNSUPPORTED;
        rows += seg_n[s];
    }
    if (rows > (int64_t)1 << 30) return BITNET_ERR_UNSUPPORTED;
    int rc = check_nk((int)rows, K);
    if (rc != BITNET_OK) return rc;
    // Whole 16-row groups: segment s's packed matrix is the next run of tiles.
    int64_t row = 0, off = 0;
    for (int s = 0; s < S; s++) {
        rc = bitnet_pack_weights(W + row * K, seg_n[s], K, packed + off, &w_scales_out[s]);
        if (rc != BITNET_OK) return rc;
        row += seg_n[s];
        off += (int64_t)seg_n[s] / 16 * 1024 * ((K + kBlock - 1) / kBlock);
    }
    return BITNET_OK;
}

int bitnet_pack_gate_up(const float* W_gate, const float* W_up, int F, int K, uint8_t* packed,
                        float* gate_scale_out, float* up_scale_out)
{
    if (W_gate == nullptr || W_up == nullptr || packed == nullptr || gate_scale_out == nullptr ||
        up_scale_out == nullptr)
        return BITNET_ERR_NULL;
    int rc = check_nk(F, K);
    if (rc != BITNET_OK) return rc;
    if (F % 16 != 0 || F > (1 << 29)) return BITNET_ERR_UNSUPPORTED;
    const int nblk = (K + kBlock - 1) / kBlock;
    const int64_t group = (int64_t)1024 * nblk;   // bytes of one 16-row group
    const int64_t one = (int64_t)F / 16 * group;  // bytes of one packed F x K matrix
    // Each matrix packed on its own (its own scale), then their groups interleaved: group 2i
    // of the result is gate group i, group 2i + 1 up group i.  The gate matrix is packed into
    // the second half of the output (gate group i at group slot F/16 + i), the up matrix into
    // the first half and copied aside.  Step i writes slots 2i and 2i + 1; every gate group
    // j > i still to be moved sits at slot F/16 + j > 2i + 1, so nothing unread is overwritten.
    uint8_t* gate = packed + one;
    rc = bitnet_pack_weights(W_gate, F, K, gate, gate_scale_out);
    if (rc != BITNET_OK) return rc;
    rc = bitnet_pack_weights(W_up, F, K, packed, up_scale_out);
    if (rc != BITNET_OK) return rc;
    uint8_t* up = new (std::nothrow) uint8_t[one];
    if (up == nullptr) return BITNET_ERR_UNSUPPORTED;
    std::memcpy(up, packed, (size_t)one);
    for (int64_t i = 0; i < F / 16; i++) {
        std::memmove(packed + (2 * i) * group, gate + i * group, (size_t)group);
        std::memcpy(packed + (2 * i + 1) * group, up + i * group, (size_t)group);
    }
    delete[] up;
    return BITNET_OK;
}

int bitnet_unpack_weights(const uint8_t* packed, int N, int K, int8_t* trits)
{
    if (packed == nullptr || trits == nullptr) return BITNET_ERR_NULL;
    int rc = check_nk(N, K);
    if (rc != BITNET_OK) return rc;
    const int nblk = (K + kBlock - 1) / kBlock;
    // Two passes: check every byte first, so a malformed buffer leaves trits untouched.
    for (int pass = 0; pass < 2; pass++) {
        for (int n = 0; n < padded_rows(N); n++) {
            int8_t* tr = trits + (int64_t)n * K;
            for (int blk = 0; blk < nblk; blk++) {
                for (int b = 0; b < 64; b++) {
                    int v = packed[tile_offset(n, blk, b, nblk)];
                    if (v > 242) return BITNET_ERR_FORMAT;
                    for (int i = 4; i >= 0; i--) {  // least significant digit is i = 4
                        const int d = v % 3;
                        v /= 3;
                        const int k = kBlock * blk + b + 64 * i;
                        if (n >= N || k >= K) {
                            if (d != 1) return BITNET_ERR_FORMAT;
                        } else if (pass == 1) {
                            tr[k] = (int8_t)(d - 1);
                        }
                    }
                }
            }
        }
    }
    return BITNET_OK;
}

}  // extern "C"
