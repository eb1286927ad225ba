// gemm.hip -- ternary x INT8/INT4 product of H-BitLinear on gfx950, with the dequantisation
// epilogue fused.
//
// Method: BitNet b1.58 2B4T write-up (itdecent.cn), section 1.2 -- with weights in {-1, 0, +1}
// the matrix product needs only additions and subtractions, accumulated exactly in int32;
// section 3.3 -- GPUs run it as "pack, store, load, unpack, compute".  Here the packed weights
// (five trits per byte, section 1.1) stream from HBM, are unpacked to int8 trits in LDS and
// feed the int8 matrix cores (v_mfma_i32_16x16x64_i8): a product with a trit is exact, so the
// int32 sums equal the add/subtract/skip sums.  Epilogue: y = (float(acc) * s_x[m]) * gamma_w,
// no bias (BitNet v2 write-up: bias removed).
//
// Workgroup tile: 256 tokens x 256 outputs, four waves of 128 x 128 (8 x 8 MFMA tiles).
// K is walked in 64-wide slabs.  A packed weight block (320 weights, 64 bytes per row) holds
// five slabs, one per base-3 digit; digits come out least significant first, so a block's
// slabs run 4, 3, 2, 1, 0.  Each slab: the weight trits and the activation codes (INT4
// sign-extended to int8) are written to one of two LDS buffers while the MFMAs read the other.
#include "common.h"

namespace bitnet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, NT = 256;
constexpr int LROW = 80;  // LDS bytes per tile row: 64 codes + 16 bytes of padding (bank spread)

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four packed bytes being decoded digit by digit, least significant digit first.  The state is
// one word: floor(byte / 3^j) for each of the four bytes.  One step: q = floor(pb / 3) per
// byte, computed in 16-bit lanes (bytes 0,2 and bytes 1,3) with floor(x / 3) = (85 x + 85) >> 8,
// exact for 0 <= x < 256; the digit is pb - 3 q, which never borrows across bytes.
__device__ __forceinline__ uint32_t digits_to_trits(uint32_t d)
{
    // digit {0,1,2} per byte -> trit {-1,0,+1} as int8: a byte-permute with the digits as selectors
    return perm(0u, 0x000100FFu, d);
}

__device__ __forceinline__ uint32_t tern_step(uint32_t& pb)
{
    const uint32_t e = pb & 0x00FF00FFu;          // [b0, 0, b2, 0]
    const uint32_t o = perm(0u, pb, 0x0C030C01u);   // [b1, 0, b3, 0]
    const uint32_t te = __umul24(e, 85u) + 0x00550055u;
    const uint32_t to = __umul24(o, 85u) + 0x00550055u;
    const uint32_t q = perm(to, te, 0x07030501u);   // [te.b1, to.b1, te.b3, to.b3]
    const uint32_t d = pb - (q + (q << 1));
    pb = q;
    return digits_to_trits(d);
}

__device__ __forceinline__ uint32_t tern_last(uint32_t pb) { return digits_to_trits(pb); }

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
    // Layer blockIdx.z of a grouped call.
    const int layer = blockIdx.z;
    const int M = args.M, N = args.N, K = args.K;
    const int64_t crow_ = BITS == 8 ? (int64_t)K : (int64_t)K / 2;
    const uint8_t* __restrict__ codes = args.codes + (int64_t)layer * M * crow_;
    const uint8_t* __restrict__ packed = args.wptrs ? args.wptrs[layer] : args.w0;
    const float* __restrict__ scales = args.scales ? args.scales + (int64_t)layer * M : nullptr;
    const float w_scale = args.wscales ? args.wscales[layer] : args.wscale0;
    float* __restrict__ out = args.out ? args.out + (int64_t)layer * M * N : nullptr;
    int32_t* __restrict__ acc_out = args.acc ? args.acc + (int64_t)layer * M * N : nullptr;

    __shared__ __align__(16) uint8_t As[2][BM * LROW];
    __shared__ __align__(16) uint8_t Bs[2][BN * LROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int nblk = (K + 319) / 320;
    const int64_t crow = BITS == 8 ? (int64_t)K : (int64_t)K / 2;

    // Weight tiles this thread streams: a block of 16 rows x 64 bytes is one contiguous 1 KB
    // tile whose 16-byte piece p = 16 c + r holds bytes 16c..16c+15 of row r.  Thread tid takes
    // piece (tid & 63) of tiles (tid >> 6) + 4 s, s = 0..3; tiles past the last row group are
    // clamped (their outputs are never stored).
    const int groups = (N + 15) / 16;
    const uint8_t* bsrc[4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
        int grp = n0 / 16 + (tid >> 6) + 4 * s;
        grp = grp < groups ? grp : groups - 1;
        bsrc[s] = packed + (int64_t)grp * nblk * 1024 + 16 * (tid & 63);
    }
    // Activation rows this thread stages.
    constexpr int ACH = BITS == 8 ? 4 : 2;
    const uint8_t* asrc[ACH];
#pragma unroll
    for (int s = 0; s < ACH; s++) {
        int m = BITS == 8 ? m0 + (tid >> 2) + 64 * s : m0 + (tid >> 1) + 128 * s;
        m = m < M ? m : M - 1;
        asrc[s] = codes + (int64_t)m * crow + (BITS == 8 ? 16 * (tid & 3) : 16 * (tid & 1));
    }

    v4i acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = v4i{0, 0, 0, 0};

    uint4 bnext[4];
    auto load_b = [&](int blk) {
#pragma unroll
        for (int s = 0; s < 4; s++)
            bnext[s] = *reinterpret_cast<const uint4*>(bsrc[s] + 1024 * (int64_t)blk);
    };
    uint4 areg[ACH];
    auto load_a = [&](int blk, int i) {
        const int64_t k0 = 320 * (int64_t)blk + 64 * i;
#pragma unroll
        for (int s = 0; s < ACH; s++)
            areg[s] = *reinterpret_cast<const uint4*>(asrc[s] + (BITS == 8 ? k0 : k0 / 2));
    };

    uint32_t dec[4][4];
    int cur = 4;  // next digit the decoder produces
    auto init_block = [&]() {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            dec[s][0] = bnext[s].x;
            dec[s][1] = bnext[s].y;
            dec[s][2] = bnext[s].z;
            dec[s][3] = bnext[s].w;
        }
        cur = 4;
    };
    uint32_t tdw[4][4];
    auto decode_to = [&](int i) {
        while (cur > i) {
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int w = 0; w < 4; w++) (void)tern_step(dec[s][w]);
            cur--;
        }
        if (i > 0) {
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int w = 0; w < 4; w++) tdw[s][w] = tern_step(dec[s][w]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int w = 0; w < 4; w++) tdw[s][w] = tern_last(dec[s][w]);
        }
        cur = i - 1;
    };
    auto write_lds = [&](int p) {
        uint8_t* bs = Bs[p];
        const int prow = (tid >> 6) * 16 + (tid & 15), pcol = 16 * ((tid >> 4) & 3);
#pragma unroll
        for (int s = 0; s < 4; s++)
            *reinterpret_cast<uint4*>(bs + (prow + 64 * s) * LROW + pcol) =
                make_uint4(tdw[s][0], tdw[s][1], tdw[s][2], tdw[s][3]);
        uint8_t* as = As[p];
        if constexpr (BITS == 8) {
#pragma unroll
            for (int s = 0; s < 4; s++)
                *reinterpret_cast<uint4*>(as + ((tid >> 2) + 64 * s) * LROW + 16 * (tid & 3)) = areg[s];
        } else {
#pragma unroll
            for (int s = 0; s < 2; s++) {
                const uint32_t w[4] = {areg[s].x, areg[s].y, areg[s].z, areg[s].w};
                uint32_t o[8];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    o[2 * j] = sext_nibbles(w[j] & 0x0F0F0F0Fu);
                    o[2 * j + 1] = sext_nibbles((w[j] >> 4) & 0x0F0F0F0Fu);
                }
                uint8_t* dst = as + ((tid >> 1) + 128 * s) * LROW + 32 * (tid & 1);
                *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
            }
        }
    };
    auto mfma_slab = [&](int p) {
        const uint8_t* as = As[p] + (wm * 128 + (lane & 15)) * LROW + 16 * (lane >> 4);
        const uint8_t* bs = Bs[p] + (wn * 128 + (lane & 15)) * LROW + 16 * (lane >> 4);
        v4i a[8];
#pragma unroll
        for (int fm = 0; fm < 8; fm++) a[fm] = *reinterpret_cast<const v4i*>(as + fm * 16 * LROW);
#pragma unroll
        for (int fn = 0; fn < 8; fn++) {
            const v4i b = *reinterpret_cast<const v4i*>(bs + fn * 16 * LROW);
#pragma unroll
            for (int fm = 0; fm < 8; fm++)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[fm], b, acc[fm][fn], 0, 0, 0);
        }
    };
    // Highest slab of block blk that lies inside K.
    auto top_slab = [&](int blk) {
        const int rem = K - 320 * blk;
        return rem >= 320 ? 4 : rem / 64 - 1;
    };

    // Prologue: slab (0, top) into buffer 0.
    load_b(0);
    init_block();
    if (nblk > 1) load_b(1);
    int blk = 0, i = top_slab(0);
    const int nslabs = 5 * (nblk - 1) + top_slab(nblk - 1) + 1;
    load_a(blk, i);
    decode_to(i);
    write_lds(0);
    __syncthreads();
    int p = 0;
    // Steady state: MFMAs on buffer p while the next slab is staged into buffer p ^ 1.
    for (int it = 0; it + 1 < nslabs; it++) {
        int nb = blk, ni = i - 1;
        if (ni < 0) {
            nb = blk + 1;
            ni = top_slab(nb);
        }
        load_a(nb, ni);
        mfma_slab(p);
        if (nb != blk) {
            init_block();
            if (nb + 1 < nblk) load_b(nb + 1);
        }
        decode_to(ni);
        write_lds(p ^ 1);
        __syncthreads();
        p ^= 1;
        blk = nb;
        i = ni;
    }
    mfma_slab(p);

    // Epilogue.  MFMA 16x16 output: lane l, register r -> row 4 (l >> 4) + r, column l & 15.
#pragma unroll
    for (int fm = 0; fm < 8; fm++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = m0 + wm * 128 + fm * 16 + 4 * (lane >> 4) + r;
            if (row >= M) continue;
            float sx = 0.0f;
            if constexpr (DEQ) sx = scales[row];
#pragma unroll
            for (int fn = 0; fn < 8; fn++) {
                const int col = n0 + wn * 128 + fn * 16 + (lane & 15);
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
