// gemm.hip -- ternary x INT8/INT4 product of H-BitLinear on gfx950 for any number of tokens,
// with the dequantisation epilogue fused.  (Decode shapes, M <= 16, use gemm_decode.hip.)
//
// Method: BitNet b1.58 2B4T write-up (itdecent.cn), section 1.2 -- with weights in {-1, 0, +1}
// the matrix product needs only additions and subtractions, accumulated exactly in int32;
// section 3.3 -- GPUs run it as "pack, store, load, unpack, compute".  Here the packed weights
// (five trits per byte, section 1.1) stream from HBM, are unpacked to int8 trits in LDS and
// feed the int8 matrix cores (v_mfma_i32_16x16x64_i8): a product with a trit is exact, so the
// int32 sums equal the add/subtract/skip sums.  Epilogue: y = (float(acc) * s_x[m]) * gamma_w,
// no bias (BitNet v2 write-up: bias removed).
//
// Workgroup tile: 256 tokens x 256 outputs, eight waves (two per SIMD) of 128 x 64 (8 x 4 MFMA
// tiles).  K is walked in 64-wide slabs.  A packed weight block (320 weights, 64 bytes per row)
// holds five slabs, one per base-3 digit; digits come out least significant first, so a
// block's slabs run 4, 3, 2, 1, 0.  Per slab: the MFMAs read one pair of LDS buffers while the
// next slab's trits (unpacked from registers) and activation codes (INT4 sign-extended to
// int8) are written to the other pair.  Global loads run ahead in registers: the packed
// weights one block (five slabs) ahead, the activation codes two slabs ahead.
#include "common.h"

namespace bitnet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, NT = 512;
constexpr int LROW = 80;  // LDS bytes per tile row: 64 codes + 16 bytes of padding (bank spread)

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 3 q in one v_lshl_add_u32 (left to itself the compiler folds w - 3 q into a 64-bit
// multiply-add, a slow instruction here)
__device__ __forceinline__ uint32_t times3(uint32_t q)
{
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, 1, %1" : "=v"(r) : "v"(q));
    return r;
}

// Four packed bytes being decoded digit by digit, least significant digit first.  The state is
// one word: floor(byte / 3^j) for each of the four bytes.  One step: q = floor(pb / 3) per
// byte, computed in 16-bit lanes (bytes 0,2 and bytes 1,3) with floor(x / 3) = (85 x + 85) >> 8,
// exact for 0 <= x < 256; the digit is pb - 3 q, which never borrows across bytes.  A digit
// {0,1,2} becomes the trit {-1,0,+1} by a byte-permute that uses the digits as selectors.
__device__ __forceinline__ uint32_t tern_step(uint32_t& pb)
{
    const uint32_t e = pb & 0x00FF00FFu;            // [b0, 0, b2, 0]
    const uint32_t o = perm(0u, pb, 0x0C030C01u);   // [b1, 0, b3, 0]
    const uint32_t te = __umul24(e, 85u) + 0x00550055u;
    const uint32_t to = __umul24(o, 85u) + 0x00550055u;
    const uint32_t q = perm(to, te, 0x07030501u);   // [te.b1, to.b1, te.b3, to.b3]
    const uint32_t d = pb - times3(q);
    pb = q;
    return perm(0u, 0x000100FFu, d);
}

__device__ __forceinline__ uint32_t tern_last(uint32_t pb) { return perm(0u, 0x000100FFu, pb); }

// Nibbles (two's complement) in the low half of each byte -> int8 in each byte:
// ((n ^ 8) + 0x78) ^ 0x80 stays within the byte, so four lanes go at once.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t n)
{
    return ((n ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

struct LargeArgs {
    const uint8_t* codes;          // L x M rows of activation codes
    const float* scales;           // L x M
    const uint8_t* const* wptrs;   // device array of L packed weights, or null (then w0)
    const uint8_t* w0;
    const float* wscales;          // device array of L weight scales, or null (then wscale0)
    float wscale0;
    float* out;                    // L x M x N fp32, or null
    int32_t* acc;                  // L x M x N int32, or null
    int M, K, N;
};

template <int BITS, bool DEQ>
__global__ __launch_bounds__(NT) void gemm_tern_kernel(LargeArgs args)
{
    __shared__ __align__(16) uint8_t As[2][BM * LROW];
    __shared__ __align__(16) uint8_t Bs[2][BN * LROW];

    // Layer blockIdx.z of a grouped call.
    const int layer = blockIdx.z;
    const int M = args.M, N = args.N, K = args.K;
    const int crow = BITS == 8 ? K : K / 2;             // code bytes per activation row
    const uint8_t* codes = args.codes + (int64_t)layer * M * crow;
    const uint8_t* packed = args.wptrs ? args.wptrs[layer] : args.w0;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;            // 128-row half, 64-column quarter
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int nblk = (K + 319) / 320;
    const int groups = (N + 15) / 16;

    // ---- packed weights: a block of 16 rows x 64 bytes is one contiguous 1 KB tile whose
    // 16-byte piece p = 16 c + r holds bytes 16c..16c+15 of row r.  Thread tid takes piece
    // (tid & 63) of tiles (tid >> 6) + 8 s, s = 0, 1.  Buffer loads: tiles past the last row
    // group read as zero (their outputs are never stored).
    const int g0 = n0 / 16;
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(packed + (int64_t)g0 * nblk * 1024), 0, (groups - g0) * nblk * 1024, 0x00020000);
    uint32_t w_off[2];
#pragma unroll
    for (int s = 0; s < 2; s++) w_off[s] = (uint32_t)((tid >> 6) + 8 * s) * (uint32_t)nblk * 1024u + 16u * (tid & 63);
    auto load_w = [&](u4 (&dst)[2], int blk) {
#pragma unroll
        for (int s = 0; s < 2; s++) dst[s] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)w_off[s], 1024 * blk, 0);
    };
    const int brow = (tid >> 6) * 16 + (tid & 15), bcol = 16 * ((tid >> 4) & 3);

    // ---- activation codes: per slab, 256 rows x 64 codes.  INT8: thread tid copies 16-byte
    // chunk (tid & 3) of rows (tid >> 2) and (tid >> 2) + 128; INT4: chunk (tid & 1) (32 codes)
    // of row tid >> 1.  Rows past M read as zero (buffer range).
    const auto ars = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + (int64_t)m0 * crow), 0, (M - m0) * crow, 0x00020000);
    constexpr int ACH = BITS == 8 ? 2 : 1;
    uint32_t a_off[ACH];
    if constexpr (BITS == 8) {
        a_off[0] = (uint32_t)(tid >> 2) * (uint32_t)crow + 16u * (tid & 3);
        a_off[1] = (uint32_t)((tid >> 2) + 128) * (uint32_t)crow + 16u * (tid & 3);
    } else {
        a_off[0] = (uint32_t)(tid >> 1) * (uint32_t)crow + 16u * (tid & 1);
    }
    struct ASlot {
        u4 v[ACH];
    };
    auto load_a = [&](ASlot& dst, int s) {
        // slab s of the flat sequence: block s / 5, digit 4 - s % 5; pad slabs load a valid
        // slab instead (their weights are zero trits and their MFMAs are skipped anyway)
        int k = 320 * (s / 5) + 64 * (4 - s % 5);
        k = k < K ? k : K - 64;
#pragma unroll
        for (int c = 0; c < ACH; c++)
            dst.v[c] = __builtin_amdgcn_raw_buffer_load_b128(ars, (int)a_off[c], BITS == 8 ? k : k / 2, 0);
    };

    v4i acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v4i{0, 0, 0, 0};

    auto write_slab = [&](int p, const uint32_t (&t)[2][4], const ASlot& x) {
        uint8_t* bs = Bs[p];
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<u4*>(bs + (brow + 128 * s) * LROW + bcol) = u4{t[s][0], t[s][1], t[s][2], t[s][3]};
        uint8_t* as = As[p];
        if constexpr (BITS == 8) {
            *reinterpret_cast<u4*>(as + (tid >> 2) * LROW + 16 * (tid & 3)) = x.v[0];
            *reinterpret_cast<u4*>(as + ((tid >> 2) + 128) * LROW + 16 * (tid & 3)) = x.v[1];
        } else {
            const u4 w = x.v[0];
            uint8_t* dst = as + (tid >> 1) * LROW + 32 * (tid & 1);
            *reinterpret_cast<u4*>(dst) = u4{sext_nibbles(w[0] & 0x0F0F0F0Fu), sext_nibbles((w[0] >> 4) & 0x0F0F0F0Fu),
                                             sext_nibbles(w[1] & 0x0F0F0F0Fu), sext_nibbles((w[1] >> 4) & 0x0F0F0F0Fu)};
            *reinterpret_cast<u4*>(dst + 16) = u4{sext_nibbles(w[2] & 0x0F0F0F0Fu), sext_nibbles((w[2] >> 4) & 0x0F0F0F0Fu),
                                                  sext_nibbles(w[3] & 0x0F0F0F0Fu), sext_nibbles((w[3] >> 4) & 0x0F0F0F0Fu)};
        }
    };
    auto mfma_slab = [&](int p) {
        const uint8_t* as = As[p] + (wm * 128 + (lane & 15)) * LROW + 16 * (lane >> 4);
        const uint8_t* bs = Bs[p] + (wn * 64 + (lane & 15)) * LROW + 16 * (lane >> 4);
        v4i a[8], b[4];
#pragma unroll
        for (int f = 0; f < 4; f++) b[f] = *reinterpret_cast<const v4i*>(bs + f * 16 * LROW);
#pragma unroll
        for (int f = 0; f < 8; f++) a[f] = *reinterpret_cast<const v4i*>(as + f * 16 * LROW);
#pragma unroll
        for (int fn = 0; fn < 4; fn++)
#pragma unroll
            for (int fm = 0; fm < 8; fm++)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    };

    // Highest slab (digit) of block blk that lies inside K; slabs above it are padding.
    auto top_slab = [&](int blk) {
        const int rem = K - 320 * blk;
        return rem >= 320 ? 4 : rem / 64 - 1;
    };
    const int S = 5 * nblk;   // flat slab sequence, padding included

    // Prologue: packed weights of block 0, activations of slabs 0 and 1.
    u4 wnext[2];
    load_w(wnext, 0);
    // keep the weight loads ahead of the activation loads (waits count loads in issue order)
    __builtin_amdgcn_sched_barrier(0);
    ASlot x0, x1, x2;
    load_a(x0, 0);
    load_a(x1, 1 < S ? 1 : 0);

    // Decoder state: the packed words of the current block, divided by 3 once per slab.
    uint32_t pb[2][4];
    uint32_t t[2][4];
    int buf = 0;
    bool have = false;   // a slab is waiting in LDS buffer `buf`
    for (int blk = 0; blk < nblk; blk++) {
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int j = 0; j < 4; j++) pb[s][j] = wnext[s][j];
        // weights of block blk + 1 (clamped) load while this block is decoded
        load_w(wnext, blk + 1 < nblk ? blk + 1 : nblk - 1);
        const int top = top_slab(blk);
        // the five slabs of the block, digit 4 first
#pragma unroll
        for (int i = 4; i >= 0; i--) {
            const int sidx = 5 * blk + (4 - i);
#pragma unroll
            for (int s = 0; s < 2; s++)
#pragma unroll
                for (int j = 0; j < 4; j++) t[s][j] = i > 0 ? tern_step(pb[s][j]) : tern_last(pb[s][j]);
            // activations two slabs ahead (ring of three, rotated by value)
            load_a(x2, sidx + 2 < S ? sidx + 2 : S - 1);
            if (i <= top) {
                if (have) mfma_slab(buf);
                write_slab(buf ^ 1, t, x0);
                __syncthreads();
                buf ^= 1;
                have = true;
            }
            x0 = x1;
            x1 = x2;
        }
    }
    if (have) mfma_slab(buf);

    // Epilogue.  MFMA 16x16 output: lane l, register r -> row 4 (l >> 4) + r, column l & 15.
    const float w_scale = args.wscales ? args.wscales[layer] : args.wscale0;
    const float* scales = args.scales ? args.scales + (int64_t)layer * M : nullptr;
    float* out = args.out ? args.out + (int64_t)layer * M * N : nullptr;
    int32_t* acc_out = args.acc ? args.acc + (int64_t)layer * M * N : nullptr;
#pragma unroll
    for (int fm = 0; fm < 8; fm++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = m0 + wm * 128 + fm * 16 + 4 * (lane >> 4) + r;
            if (row >= M) continue;
            float sx = 0.0f;
            if constexpr (DEQ) sx = scales[row];
#pragma unroll
            for (int fn = 0; fn < 4; fn++) {
                const int col = n0 + wn * 64 + fn * 16 + (lane & 15);
                if (col >= N) continue;
                const int32_t a = acc[fm][fn][r];
                if constexpr (DEQ)
                    out[(int64_t)row * N + col] = ((float)a * sx) * w_scale;
                else
                    acc_out[(int64_t)row * N + col] = a;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_large(const uint8_t* codes, int L, int M, int K, int N, int bits,
                             const uint8_t* const* wptrs, const uint8_t* w0,
                             const float* scales, const float* wscales, float wscale0,
                             float* out_f32, int32_t* acc_i32, hipStream_t stream)
{
    // Buffer ranges are 32-bit: one weight matrix and one layer's codes stay below 2 GiB.
    const int64_t packed = (int64_t)((N + 15) / 16) * 1024 * ((K + 319) / 320);
    const int64_t crow = bits == 8 ? K : K / 2;
    if (packed >= ((int64_t)1 << 31) || (int64_t)M * crow >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    LargeArgs a{codes, scales, wptrs, w0, wscales, wscale0, out_f32, acc_i32, M, K, N};
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, L);
    if (out_f32 != nullptr) {
        if (bits == 8) hipLaunchKernelGGL((gemm_tern_kernel<8, true>), grid, dim3(NT), 0, stream, a);
        else hipLaunchKernelGGL((gemm_tern_kernel<4, true>), grid, dim3(NT), 0, stream, a);
    } else {
        if (bits == 8) hipLaunchKernelGGL((gemm_tern_kernel<8, false>), grid, dim3(NT), 0, stream, a);
        else hipLaunchKernelGGL((gemm_tern_kernel<4, false>), grid, dim3(NT), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* codes, int L, int M, int K, int N, int bits,
                       const uint8_t* const* wptrs, const uint8_t* w0, const float* scales,
                       const float* wscales, float wscale0, float* out_f32, int32_t* acc_i32,
                       hipStream_t stream)
{
    if (M <= 16)
        return launch_gemm_decode(codes, L, M, K, N, bits, wptrs, w0, scales, wscales, wscale0,
                                  out_f32, acc_i32, stream);
    return launch_gemm_large(codes, L, M, K, N, bits, wptrs, w0, scales, wscales, wscale0,
                             out_f32, acc_i32, stream);
}

}  // namespace bitnet
