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
// K is walked in 64-wide slabs.  A packed weight block (320 weights, 64 bytes per row) holds
// five slabs, one per base-3 digit, decoded least significant digit first.
//
// Two kernels:
//   gemm_tern4_kernel (INT4 activations, the BitNet v2 case).  Workgroup tile 512 tokens x
//     128 outputs, four waves (one per SIMD), each 128 x 128 outputs (8 x 8 MFMA tiles, int32
//     accumulators in the accumulation registers).  The tile is tall because the unpacked
//     trits of a weight row serve every token row of the tile.  Per slab the codes go from
//     global memory straight into LDS (buffer loads with the LDS as destination), four slabs
//     ahead and still packed; every thread turns the next digit of the packed words it holds
//     into trits for two slabs ahead; each wave issues the 64 MFMAs of the slab from
//     registers and, in their shadow, reads its operands of the next slab -- weight trits and
//     its own 128 rows of codes, widened in registers.  A short last block keeps its pad
//     digits (trits 0), so every block has five slabs and slot d of the five LDS slots holds
//     digit 4 - d.  Widening needs no sign arithmetic: a nibble moved to the high half of a
//     byte is the int8 value 16 x code, so the MFMA sums are 16 x the code sums and one
//     arithmetic shift restores them.
//   gemm_tern_kernel (INT8 activations).  Workgroup tile 256 x 256, eight waves (two per SIMD)
//     of 128 x 64; per slab the MFMAs read one pair of LDS buffers while the next slab's trits
//     and codes are written to the other pair; global loads run ahead in registers.
#include "common.h"

namespace bitnet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BM = 256, BN = 256, NT = 512;       // INT8 kernel
constexpr int BM4 = 512, BN4 = 128, NT4 = 256;    // INT4 kernel
constexpr int LROW = 80;  // INT8 kernel: LDS bytes per tile row, 64 codes + 16 bytes of padding

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

// Four packed bytes being decoded digit by digit, least significant digit first: the state
// is floor(byte / 3^j) per byte.  q = floor(pb / 3) per byte, in 16-bit lanes (bytes 0,2 and
// bytes 1,3) with floor(x / 3) = (85 x + 85) >> 8, exact for 0 <= x < 256; the digit is
// pb - 3 q (no borrow across bytes); a digit {0,1,2} becomes the trit {-1,0,+1} by a
// byte-permute that uses the digits as selectors.  At the last digit pb < 3, so q = 0.
__device__ __forceinline__ uint32_t tern_step(uint32_t& pb)
{
    const uint32_t e = pb & 0x00FF00FFu;
    const uint32_t o = perm(0u, pb, 0x0C030C01u);
    const uint32_t te = __umul24(e, 85u) + 0x00550055u;
    const uint32_t to = __umul24(o, 85u) + 0x00550055u;
    const uint32_t q = perm(to, te, 0x07030501u);
    const uint32_t d = pb - times3(q);
    pb = q;
    return perm(0u, 0x000100FFu, d);
}

__device__ __forceinline__ uint32_t tern_last(uint32_t pb) { return perm(0u, 0x000100FFu, pb); }

// The per-layer pointer and scale arrays are never written while a kernel runs; reading them
// through the constant address space makes them scalar loads.
typedef const __attribute__((address_space(4))) uint64_t* const_u64_ptr;
typedef const __attribute__((address_space(4))) float* const_f32_ptr;

struct LargeArgs {
    const uint8_t* codes;          // L x M rows of activation codes
    const float* scales;           // L x M
    const uint8_t* const* wptrs;   // device array of L packed weights, or null (then w0)
    const uint8_t* w0;
    const float* wscales;          // device array of L weight scales, or null (then wscale0)
    float wscale0;
    float* out;                    // L x M x N fp32 (M x N/2 with of.glu), or null
    int32_t* acc;                  // L x M x N int32, or null
    int M, K, N;
    OutForm of;                    // segments / gate-up pairs (L = 1, out only)
};

// Workgroup barrier after this wave's LDS operations have completed.  Written out (rather
// than __syncthreads) so that it does not also wait for the loads still streaming codes into
// other LDS slots; those are waited for by count (wait_vmcnt) where they are needed.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// v_mfma_i32_16x16x64_i8 with the accumulator tied to one set of accumulation registers
// (acc += a . b).  Written out because the compiler otherwise moves accumulators between
// register sets around every MFMA.  The accumulators are read only by later MFMAs of the
// same kind (many MFMAs later) and, after mfma_drain, by the epilogue.
__device__ __forceinline__ void mfma_acc(v4i& acc, const v4i& a, const v4i& b)
{
    asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last MFMA and the first read of its result by other instructions
// (more than the longest MFMA latency).
__device__ __forceinline__ void mfma_drain()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// s_waitcnt for vector-memory operations only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef float f4 __attribute__((ext_vector_type(4)));

// Writes one wave's FM x FN grid of 16x16 MFMA output tiles: tile (fm, fn), lane l, register r
// is row row0 + 16 fm + 4 (l >> 4) + r, column col0 + 16 fn + (l & 15).  With DEQ the value is
// y = (float(acc >> SHIFT) * s_x[row]) * gamma_w, else the int32 sum acc >> SHIFT; sxf(fm)
// gives s_x of the lane's four rows of tile fm, wsf(fn) gamma_w of tile column fn.  Every
// store is issued without waiting on the ones before it: an output outside M x N gets a byte
// offset past the buffer's range, and the hardware drops it.  The caller guarantees
// 4 M N < 2^31.
template <int FM, int FN, int SHIFT, bool DEQ, typename ScaleFn, typename WScaleFn>
__device__ __forceinline__ void store_tiles(const v4i (&acc)[FM][FN], int row0, int col0, int lane,
                                            int M, int N, ScaleFn sxf, WScaleFn wsf, void* obase)
{
    const int g = lane >> 4;
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(obase, 0, 0x7FFFFFFF, 0x00020000);
    // the weight scale of each tile column, formed once (the store loop below has FM * 4 * FN
    // stores); it is the same for the whole wave, so it is held in scalar registers
    float wsv[FN];
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
        wsv[fn] = DEQ ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wsf(fn))))
                      : 0.0f;
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        f4 sx = f4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (DEQ) sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = row0 + 16 * fm + 4 * g + r;
#pragma unroll
            for (int fn = 0; fn < FN; fn++) {
                const int col = col0 + 16 * fn + (lane & 15);
                const int32_t a = acc[fm][fn][r] >> SHIFT;
                uint32_t v;
                if constexpr (DEQ)
                    v = __builtin_bit_cast(uint32_t, ((float)a * sx[r]) * wsv[fn]);
                else
                    v = (uint32_t)a;
                const uint32_t off = (row < M && col < N) ? 4u * (uint32_t)(row * N + col) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(v, ors, (int)off, 0, 0);
            }
        }
    }
}

// Gate / up pairs: tile columns 2j (gate rows) and 2j + 1 (the same up rows) of the grid above
// give h = SiLU(gate) * up, each dequantised as in store_tiles with its own weight scale, in
// column col0 / 2 + 16 j + (l & 15) of the M x F output (col0 a multiple of 32).
template <int FM, int FN, int SHIFT, typename ScaleFn>
__device__ __forceinline__ void store_tiles_glu(const v4i (&acc)[FM][FN], int row0, int col0, int lane,
                                                int M, int F, ScaleFn sxf, float gate_scale,
                                                float up_scale, void* obase)
{
    static_assert(FN % 2 == 0, "gate / up tiles come in pairs");
    const int g = lane >> 4;
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(obase, 0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const f4 sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = row0 + 16 * fm + 4 * g + r;
#pragma unroll
            for (int j = 0; j < FN / 2; j++) {
                const int col = col0 / 2 + 16 * j + (lane & 15);
                const float gv = ((float)(acc[fm][2 * j][r] >> SHIFT) * sx[r]) * gate_scale;
                const float uv = ((float)(acc[fm][2 * j + 1][r] >> SHIFT) * sx[r]) * up_scale;
                const uint32_t v = __builtin_bit_cast(uint32_t, silu_mul(gv, uv));
                const uint32_t off = (row < M && col < F) ? 4u * (uint32_t)(row * F + col) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(v, ors, (int)off, 0, 0);
            }
        }
    }
}

// Nibbles (two's complement) in the low half of each byte -> int8 in each byte:
// ((n ^ 8) + 0x78) ^ 0x80 stays within the byte, so four lanes go at once.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t n)
{
    return ((n ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

// Epilogue forms, one instantiation each (the plain one carries none of the others' code):
// one weight scale per layer; a scale per row segment; gate / up pairs.
enum Epi { kPlain = 0, kSegments = 1, kGlu = 2 };

template <int BITS, bool DEQ, int EPI>
__global__ __launch_bounds__(NT) void gemm_tern_kernel(LargeArgs args)
{
    __shared__ __align__(16) uint8_t As[2][BM * LROW];
    __shared__ __align__(16) uint8_t Bs[2][BN * LROW];

    // Layer blockIdx.z of a grouped call.
    const int layer = blockIdx.z;
    const int M = args.M, N = args.N, K = args.K;
    const int crow = BITS == 8 ? K : K / 2;             // code bytes per activation row
    const uint8_t* codes = args.codes + (int64_t)layer * M * crow;
    const uint8_t* packed = args.wptrs ? (const uint8_t*)((const_u64_ptr)(const void*)args.wptrs)[layer] : args.w0;

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

    const float w_scale = args.wscales ? ((const_f32_ptr)(const void*)args.wscales)[layer] : args.wscale0;
    void* obase = DEQ ? (void*)(args.out + (int64_t)layer * M * N) : (void*)(args.acc + (int64_t)layer * M * N);
    // The lane's 32 row scales are loaded before the first store, so no wait for them has to
    // wait for stores as well.
    f4 sxr[8];
    if constexpr (DEQ) {
        const auto srs = __builtin_amdgcn_make_buffer_rsrc((void*)(args.scales + (int64_t)layer * M), 0, 4 * M, 0x00020000);
#pragma unroll
        for (int fm = 0; fm < 8; fm++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                sxr[fm][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    srs, 4 * (m0 + wm * 128 + 16 * fm + 4 * (lane >> 4) + r), 0, 0));
    }
    const int col0 = n0 + wn * 64;
    auto sxf = [&](int fm) __attribute__((always_inline)) { return sxr[fm]; };
    if constexpr (EPI == kGlu)
        store_tiles_glu<8, 4, 0>(acc, m0 + wm * 128, col0, lane, M, N / 2, sxf, args.of.gate_scale,
                                 args.of.up_scale, obase);
    else if constexpr (EPI == kSegments)
        store_tiles<8, 4, 0, DEQ>(acc, m0 + wm * 128, col0, lane, M, N, sxf,
                                  [&](int fn) __attribute__((always_inline)) {
                                      return group_scale(args.of, col0 / 16 + fn, w_scale);
                                  }, obase);
    else
        store_tiles<8, 4, 0, DEQ>(acc, m0 + wm * 128, col0, lane, M, N, sxf,
                                  [&](int) __attribute__((always_inline)) { return w_scale; }, obase);
}


template <bool DEQ, int EPI>
__global__ __launch_bounds__(NT4) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tern4_kernel(LargeArgs args)
{
    constexpr int BITS = 4, BM = BM4, BN = BN4, NT = NT4;
    constexpr int AROW = 32;                        // code bytes of one token row per slab
    constexpr int AJ = BM * AROW / 16 / NT;         // 16-byte code loads per thread per slab
    // Five slots of codes and of trits, one per digit of a block, each slot its own array so
    // that the compiler sees the loads into one slot do not touch the others.
    __shared__ __align__(16) uint8_t A0[BM * AROW], A1[BM * AROW], A2[BM * AROW], A3[BM * AROW], A4[BM * AROW];
    __shared__ __align__(16) uint8_t Bt[5][BN * 64];
    __shared__ __align__(16) float sxs[BM];         // s_x of the tile's rows, for the epilogue
    auto araw = [&](int s) __attribute__((always_inline)) -> uint8_t* {
        return s == 0 ? A0 : s == 1 ? A1 : s == 2 ? A2 : s == 3 ? A3 : A4;
    };

    // Layer blockIdx.z of a grouped call.
    const int layer = blockIdx.z;
    const int M = args.M, N = args.N, K = args.K;
    const int crow = BITS == 8 ? K : K / 2;             // code bytes per activation row
    const uint8_t* codes = args.codes + (int64_t)layer * M * crow;
    const uint8_t* packed = args.wptrs ? (const uint8_t*)((const_u64_ptr)(const void*)args.wptrs)[layer] : args.w0;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int nblk = (K + 319) / 320;
    const int groups = (N + 15) / 16;

    // ---- packed weights: a block of 16 rows x 64 bytes is one contiguous 1 KB tile whose
    // 16-byte piece q = 16 c + r holds bytes 16c..16c+15 of row r.  Thread tid holds pieces
    // p = tid + 256 s (s = 0, 1): piece p & 63 of tile p >> 6.  Buffer loads: tiles past the
    // last row group read as zero (their outputs are never stored).
    const int g0 = n0 / 16;
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(packed + (int64_t)g0 * nblk * 1024), 0, (groups - g0) * nblk * 1024, 0x00020000);
    // piece tid: tile tid >> 6, q = tid & 63; piece tid + 256: four tiles (64 rows) further
    const int wq = tid & 63, wr = 16 * (tid >> 6) + (wq & 15);
    const uint32_t w_off = (uint32_t)(tid >> 6) * (uint32_t)nblk * 1024u + 16u * wq;
    const int w_step = 4 * nblk * 1024;
    const uint32_t b_lds = (uint32_t)(wr * 64 + 16 * ((wq >> 4) ^ ((wr >> 2) & 3)));   // chunk swizzled by row
    auto load_w = [&](u4 (&dst)[2], int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; s++) dst[s] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)w_off, 1024 * blk + s * w_step, 0);
    };

    // ---- activation codes: per slab the 512 token rows' AROW bytes go to Araw in AJ
    // instructions per wave-thread; instruction (s, wave) fills 1 KB of LDS, lane l the 16
    // bytes at chunk Q = 64 (4 s + wave) + l: row Q / (AROW / 16), chunk Q % (AROW / 16),
    // with the chunk index swizzled by row (INT4: by bit 3 of the row; INT8: by bits 2..3).
    // Rows past M read as zero.  A pad digit's slab (k >= K) loads the last slab instead.
    const auto ars = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + (int64_t)m0 * crow), 0, (M - m0) * crow, 0x00020000);
    constexpr int CPR = AROW / 16;                      // 16-byte chunks per row and slab
    // Instruction s covers rows 256 s / CPR further than instruction 0 with the same swizzle.
    uint32_t a_off;
    {
        const int Q = 64 * wave + lane, row = Q / CPR, phys = Q % CPR;
        const int c = BITS == 8 ? phys ^ ((row >> 2) & 3) : phys ^ ((row >> 3) & 1);
        a_off = (uint32_t)row * (uint32_t)crow + 16u * c;
    }
    const int a_step = 256 / CPR * crow;
    auto load_a = [&](int v, int slot) __attribute__((always_inline)) {
        int k = 320 * (v / 5) + 64 * (4 - v % 5);
        k = k < K ? k : K - 64;
        const int kb = BITS == 8 ? k : k / 2;
#pragma unroll
        for (int s = 0; s < AJ; s++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_ptr)(araw(slot) + 1024 * (4 * s + wave)), 16,
                                                     a_off, kb + s * a_step, 0, 0);
    };

    v4i acc[8][8];   // this wave's 128 x 128 outputs
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = v4i{0, 0, 0, 0};

    // ---- operands.  MFMA lane l: A row (l & 15) of the 16-row tile, B row (l & 15), k-slots
    // 16 g .. 16 g + 15 with g = l >> 4.
    const int am = 128 * wave + (lane & 15), g = lane >> 4;
    // Fragment i of a 16-row tile sits 16 rows below fragment 0, with the same swizzle.
    uint32_t a_rd, b_rd;
    {
        const int row = am;
        if constexpr (BITS == 8)
            a_rd = (uint32_t)(row * 64 + 16 * (g ^ ((row >> 2) & 3)));
        else
            a_rd = (uint32_t)(row * 32 + 16 * ((g >> 1) ^ ((row >> 3) & 1)) + 8 * (g & 1));
        const int brow = lane & 15;
        b_rd = (uint32_t)(brow * 64 + 16 * (g ^ ((brow >> 2) & 3)));
    }
    typedef u2 ARaw;
    auto read_a = [&](int slot, int i) __attribute__((always_inline)) {
        return *reinterpret_cast<const ARaw*>(araw(slot) + a_rd + 16 * AROW * i);
    };
    // INT4: 16 codes (two words, code 8w + p in the low nibble of byte p, 8w + p + 4 in the
    // high nibble) -> 16 bytes of 16 x code
    auto widen = [&](const ARaw& x) __attribute__((always_inline)) {
        return v4i{(int)((x[0] << 4) & 0xF0F0F0F0u), (int)(x[0] & 0xF0F0F0F0u),
                   (int)((x[1] << 4) & 0xF0F0F0F0u), (int)(x[1] & 0xF0F0F0F0u)};
    };

    // ---- weight decoding of one slab into Bt slot p: the next digit of the held words.
    u4 wnext[2];
    uint32_t pb[2][4];
    auto produce = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; s++) {
            u4 t;
#pragma unroll
            for (int w = 0; w < 4; w++) t[w] = tern_step(pb[s][w]);   // at digit 0, pb < 3: q = 0
            *reinterpret_cast<u4*>(Bt[p] + b_lds + 4096 * s) = t;
        }
    };
    auto take_block = [&](int next_blk) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int w = 0; w < 4; w++) pb[s][w] = wnext[s][w];
        load_w(wnext, next_blk < nblk ? next_blk : nblk - 1);
    };

    // Prologue: weights of block 0 (then 1 in flight); codes of slabs 0..3 in LDS; trits of
    // slabs 0 and 1; operands of slab 0 in registers (A tiles 4..7 still packed).  The codes
    // and scales are requested together with the first weights, so the prologue waits for
    // one round trip to memory, not two.
    load_w(wnext, 0);
    load_a(0, 0);
    load_a(1, 1);
    load_a(2, 2);
    load_a(3, 3);
    constexpr int NSX = DEQ ? BM / NT : 0;            // scale loads
    if constexpr (DEQ) {
        // s_x of the tile's rows straight into LDS, 64 rows per wave-wide load; rows past M
        // read as zero.
        const auto srs = __builtin_amdgcn_make_buffer_rsrc((void*)(args.scales + (int64_t)layer * M), 0, 4 * M, 0x00020000);
#pragma unroll
        for (int s = 0; s < NSX; s++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_ptr)(sxs + NT * s + 64 * wave), 4,
                                                     4u * (uint32_t)(m0 + NT * s + 64 * wave + lane), 0, 0, 0);
    }
    wait_vmcnt<4 * AJ + NSX>();                         // the two weight loads of block 0
    take_block(1);
    produce(0);
    produce(1);
    wait_vmcnt<2>();                                    // all but block 1's two weight loads
    block_sync();
    v4i af[8], bf[8];
    ARaw rhi[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        af[i] = widen(read_a(0, i));
        rhi[i] = read_a(0, 4 + i);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) bf[i] = *reinterpret_cast<const v4i*>(Bt[0] + b_rd + 1024 * i);

    // Slab v = 5 blk + d (digit 4 - d of block blk), slots indexed by d: MFMAs of v; operand
    // reads of v + 1 (slots d + 1); trits of v + 2 into Bt slot d + 2; codes of v + 4 into
    // code slot d + 4 (all mod 5).  With one wave per SIMD, the vector work only overlaps the
    // matrix core if it sits between the MFMAs, so the slab is written as a fixed sequence of
    // short chunks -- a few MFMAs and a little vector or LDS work each -- separated by
    // scheduling barriers that keep the compiler from regrouping them.
    //   first half (A tiles 0..3 x B tiles 0..7): packed A tiles 0..3 of v + 1 requested, the
    //     next digit of the held weight words decoded and written, A tiles 4..7 of v widened;
    //   second half (A tiles 4..7 x B tiles 0..7): B tile n - 1 of v + 1 read behind B tile
    //     n's MFMAs, A tiles 0..3 of v + 1 widened, packed A tiles 4..7 of v + 1 requested.
    auto mf = [&](int m, int n) __attribute__((always_inline)) { mfma_acc(acc[m][n], af[m], bf[n]); };
    auto slab = [&](int v, int d) __attribute__((always_inline)) {
        const int s1 = (d + 1) % 5, s2 = (d + 2) % 5, s4 = (d + 4) % 5;
        ARaw rlo[4];
        u4 t[2];
        mf(0, 0);
        mf(1, 0);
        if (d == 3) take_block(v / 5 + 2);        // slab v + 2 opens block v / 5 + 1
        load_a(v + 4, s4);
#pragma unroll
        for (int i = 0; i < 4; i++) rlo[i] = read_a(s1, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const int c = k + 1;
            mf(2 * (c & 1), c >> 1);
            mf(2 * (c & 1) + 1, c >> 1);
            t[k >> 2][k & 3] = tern_step(pb[k >> 2][k & 3]);   // at digit 0, pb < 3: q = 0
            if ((k & 3) == 3) *reinterpret_cast<u4*>(Bt[s2] + b_lds + 4096 * (k >> 2)) = t[k >> 2];
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c = 9; c < 16; c++) {
            mf(2 * (c & 1), c >> 1);
            mf(2 * (c & 1) + 1, c >> 1);
            if (c < 13) af[4 + c - 9] = widen(rhi[c - 9]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int n = 0; n < 8; n++) {
            mf(4, n);
            mf(5, n);
            mf(6, n);
            mf(7, n);
            if (n >= 1) bf[n - 1] = *reinterpret_cast<const v4i*>(Bt[s1] + b_rd + 1024 * (n - 1));
            if (n >= 2 && n < 6) af[n - 2] = widen(rlo[n - 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf[7] = *reinterpret_cast<const v4i*>(Bt[s1] + b_rd + 1024 * 7);
#pragma unroll
        for (int i = 0; i < 4; i++) rhi[i] = read_a(s1, 4 + i);
        // the codes of slab v + 2 (issued two slabs earlier) must be in LDS before the
        // barrier; issued since: AJ code loads in each of the last two slabs, and two weight
        // loads when one of them opened a block
        if (d >= 3) wait_vmcnt<2 * AJ + 2>();
        else wait_vmcnt<2 * AJ>();
        block_sync();
    };
    for (int blk = 0; blk < nblk; blk++) {
        const int v = 5 * blk;
        slab(v, 0);
        slab(v + 1, 1);
        slab(v + 2, 2);
        slab(v + 3, 3);
        slab(v + 4, 4);
    }

    wait_vmcnt<0>();   // the loads issued past the last slab
    mfma_drain();

    // The codes entered the MFMAs as 16 x code, so the sums are 16 x the integer dot products.
    const float w_scale = args.wscales ? ((const_f32_ptr)(const void*)args.wscales)[layer] : args.wscale0;
    void* obase = DEQ ? (void*)(args.out + (int64_t)layer * M * N) : (void*)(args.acc + (int64_t)layer * M * N);
    auto sxf = [&](int fm) __attribute__((always_inline)) {
        return *(const f4*)&sxs[128 * wave + 16 * fm + 4 * g];
    };
    if constexpr (EPI == kGlu)
        store_tiles_glu<8, 8, 4>(acc, m0 + 128 * wave, n0, lane, M, N / 2, sxf, args.of.gate_scale,
                                 args.of.up_scale, obase);
    else if constexpr (EPI == kSegments)
        store_tiles<8, 8, 4, DEQ>(acc, m0 + 128 * wave, n0, lane, M, N, sxf,
                                  [&](int fn) __attribute__((always_inline)) {
                                      return group_scale(args.of, n0 / 16 + fn, w_scale);
                                  }, obase);
    else
        store_tiles<8, 8, 4, DEQ>(acc, m0 + 128 * wave, n0, lane, M, N, sxf,
                                  [&](int) __attribute__((always_inline)) { return w_scale; }, obase);
}

}  // namespace

hipError_t launch_gemm_large(const uint8_t* codes, int L, int M, int K, int N, int bits,
                             const uint8_t* const* wptrs, const uint8_t* w0,
                             const float* scales, const float* wscales, float wscale0,
                             float* out_f32, int32_t* acc_i32, hipStream_t stream,
                             const OutForm& of)
{
    // Buffer ranges are 32-bit: one weight matrix, one layer's codes and one layer's output
    // stay below 2 GiB.
    const int64_t packed = (int64_t)((N + 15) / 16) * 1024 * ((K + 319) / 320);
    const int64_t crow = bits == 8 ? K : K / 2;
    if (packed >= ((int64_t)1 << 31) || (int64_t)M * crow >= ((int64_t)1 << 31) ||
        4 * (int64_t)M * N >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    LargeArgs a{codes, scales, wptrs, w0, wscales, wscale0, out_f32, acc_i32, M, K, N, of};
    if (bits == 4) {
        dim3 grid((N + BN4 - 1) / BN4, (M + BM4 - 1) / BM4, L);
        if (out_f32 != nullptr && of.glu) hipLaunchKernelGGL((gemm_tern4_kernel<true, kGlu>), grid, dim3(NT4), 0, stream, a);
        else if (out_f32 != nullptr && of.nseg > 0) hipLaunchKernelGGL((gemm_tern4_kernel<true, kSegments>), grid, dim3(NT4), 0, stream, a);
        else if (out_f32 != nullptr) hipLaunchKernelGGL((gemm_tern4_kernel<true, kPlain>), grid, dim3(NT4), 0, stream, a);
        else hipLaunchKernelGGL((gemm_tern4_kernel<false, kPlain>), grid, dim3(NT4), 0, stream, a);
    } else {
        dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, L);
        if (out_f32 != nullptr && of.glu) hipLaunchKernelGGL((gemm_tern_kernel<8, true, kGlu>), grid, dim3(NT), 0, stream, a);
        else if (out_f32 != nullptr && of.nseg > 0) hipLaunchKernelGGL((gemm_tern_kernel<8, true, kSegments>), grid, dim3(NT), 0, stream, a);
        else if (out_f32 != nullptr) hipLaunchKernelGGL((gemm_tern_kernel<8, true, kPlain>), grid, dim3(NT), 0, stream, a);
        else hipLaunchKernelGGL((gemm_tern_kernel<8, false, kPlain>), grid, dim3(NT), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* codes, int L, int M, int K, int N, int bits,
                       const uint8_t* const* wptrs, const uint8_t* w0, const float* scales,
                       const float* wscales, float wscale0, float* out_f32, int32_t* acc_i32,
                       hipStream_t stream, const OutForm& of)
{
    if (M <= 16)
        return launch_gemm_decode(codes, L, M, K, N, bits, wptrs, w0, scales, wscales, wscale0,
                                  out_f32, acc_i32, stream, of);
    return launch_gemm_large(codes, L, M, K, N, bits, wptrs, w0, scales, wscales, wscale0,
                             out_f32, acc_i32, stream, of);
}

}  // namespace bitnet
