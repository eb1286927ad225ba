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
//     128 outputs, eight waves (two per SIMD), each 64 x 128 outputs (4 x 8 MFMA tiles, int32
//     accumulators in the accumulation registers).  The tile is tall because the unpacked
//     trits of a weight row serve every token row of the tile.  Per slab the codes go from
//     global memory straight into LDS (buffer loads with the LDS as destination), four slabs
//     ahead and still packed; every thread turns the next digit of the packed words it holds
//     into trits for three slabs ahead; each wave issues the 32 MFMAs of the slab from
//     registers and, in their shadow, reads its operands of the next slab -- weight trits and
//     its own 64 rows of codes, widened in registers.  A short last block keeps its pad
//     digits (trits 0), so every block has five slabs and slot d of the five LDS slots holds
//     digit 4 - d.  Widening needs no sign arithmetic: a nibble moved to the high half of a
//     byte is the int8 value 16 x code, so the MFMA sums are 16 x the code sums and one
//     arithmetic shift restores them.
//   gemm_tern_kernel (INT8 activations).  Workgroup tile 256 x 256, eight waves (two per SIMD)
//     of 128 x 64; per slab the MFMAs read one pair of LDS buffers while the next slab's trits
//     and codes are written to the other pair; global loads run ahead in registers.
#include <type_traits>

#include "common.h"

namespace bitnet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BM = 256, BN = 256, NT = 512;       // INT8 kernel
constexpr int BM4 = 512, BN4 = 128, NT4 = 512;    // INT4 kernel
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
    int xcd_runs;                  // INT4 kernel: tile order by XCD runs (else launch order)
};

// Workgroup barrier after this wave's LDS operations have completed.  Written out (rather
// than __syncthreads) so that it does not also wait for the loads still streaming codes into
// other LDS slots; those are waited for by count (wait_vmcnt) where they are needed.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The same barrier, but this wave's last N LDS operations may still be in flight.  LDS
// operations complete in issue order, so every earlier one -- in particular every LDS write
// the barrier publishes -- has completed.  For a caller whose last LDS write is followed by at
// least N LDS reads it does not need before the barrier (the next slab's operands).
template <int N = 10>
__device__ __forceinline__ void block_sync_reads_in_flight()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}

// v_mfma_i32_16x16x64_i8 with the accumulator tied to one set of accumulation registers
// (acc += a . b).  Written out because the compiler otherwise moves accumulators between
// register sets around every MFMA.  The accumulators are read only by later MFMAs of the
// same kind (many MFMAs later) and, after mfma_drain, by the epilogue.
__device__ __forceinline__ void mfma_acc(v4i& acc, const v4i& a, const v4i& b)
{
    asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between a vector instruction that writes an MFMA operand and the MFMA that reads
// it (the MFMAs are inline asm, so the compiler inserts none).  The operand is an input of the
// asm, so the instructions that write it cannot be moved below the wait.
__device__ __forceinline__ void mfma_operand_wait(const v4i& x)
{
    asm volatile("s_nop 4" :: "v"(x) : "memory");
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

// store_tiles for a wave tile that lies wholly inside M x N, so no output needs a bounds test:
// the lane's offset is one VGPR, the row of (fm, r) a scalar offset and the tile column an
// immediate offset, and each output costs its dequantisation and one store.
template <int FM, int FN, int SHIFT, typename ScaleFn, typename WScaleFn>
__device__ __forceinline__ void store_tiles_inside(const v4i (&acc)[FM][FN], int row0, int col0, int lane,
                                                   int N, ScaleFn sxf, WScaleFn wsf, float* out)
{
    const int g = lane >> 4;
    const auto ors = __builtin_amdgcn_make_buffer_rsrc((void*)(out + (int64_t)row0 * N + col0), 0,
                                                       0x7FFFFFFF, 0x00020000);
    float wsv[FN];
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
        wsv[fn] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wsf(fn))));
    const int voff = 4 * (4 * g * N + (lane & 15));
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const f4 sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int soff = __builtin_amdgcn_readfirstlane(4 * (16 * fm + r) * N);
#pragma unroll
            for (int fn = 0; fn < FN; fn++) {
                const float v = ((float)(acc[fm][fn][r] >> SHIFT) * sx[r]) * wsv[fn];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ors, voff + 64 * fn, soff, 0);
            }
        }
    }
}

// store_tiles_glu for a wave tile wholly inside the M x F output (addressing as
// store_tiles_inside, on the output columns col0 / 2 + 16 j + (l & 15)).
template <int FM, int FN, int SHIFT, typename ScaleFn>
__device__ __forceinline__ void store_tiles_glu_inside(const v4i (&acc)[FM][FN], int row0, int col0, int lane,
                                                       int F, ScaleFn sxf, float gate_scale, float up_scale,
                                                       float* out)
{
    static_assert(FN % 2 == 0, "gate / up tiles come in pairs");
    const int g = lane >> 4;
    const auto ors = __builtin_amdgcn_make_buffer_rsrc((void*)(out + (int64_t)row0 * F + col0 / 2), 0,
                                                       0x7FFFFFFF, 0x00020000);
    const int voff = 4 * (4 * g * F + (lane & 15));
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const f4 sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int soff = __builtin_amdgcn_readfirstlane(4 * (16 * fm + r) * F);
#pragma unroll
            for (int j = 0; j < FN / 2; j++) {
                const float gv = ((float)(acc[fm][2 * j][r] >> SHIFT) * sx[r]) * gate_scale;
                const float uv = ((float)(acc[fm][2 * j + 1][r] >> SHIFT) * sx[r]) * up_scale;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, silu_mul(gv, uv)), ors,
                                                      voff + 64 * j, soff, 0);
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

// Low-bit Q/K/V states (BitNet v2 write-up: QKV states at reduced bit widths, zero-shot
// tables 2 and 3; a 3-bit KV cache): each output y, dequantised as in store_tiles, is
// quantised per row and per group of 16 TG consecutive columns (one attention head) with its
// segment's Qp: gamma = max |y| over the group, q = clamp(rne(y * (Qp / gamma)), -Qp-1, Qp)
// (IEEE division), scale = gamma / Qp, a zero group giving codes 0 and scale 0.  The group's
// columns are this wave's tiles TG j .. TG j + TG - 1 of one row, held by the 16 lanes of the
// row's lane group, so the maximum runs over TG registers and then max16.  Codes go out as
// bytes (M x N int8 at cbase), scales as M x N / (16 TG) fp32.  Offsets outside the outputs
// are dropped by the buffer range, as in store_tiles.
template <int FM, int FN, int SHIFT, int TG, typename ScaleFn, typename WScaleFn>
__device__ __forceinline__ void store_tiles_states(const v4i (&acc)[FM][FN], int row0, int col0, int lane,
                                                   int M, int N, ScaleFn sxf, WScaleFn wsf,
                                                   const OutForm& of, void* cbase)
{
    static_assert(FN % TG == 0, "a group is whole tiles of the wave");
    constexpr int NG = FN / TG;
    const int g = lane >> 4;
    const auto crs = __builtin_amdgcn_make_buffer_rsrc(cbase, 0, 0x7FFFFFFF, 0x00020000);
    const auto srs = __builtin_amdgcn_make_buffer_rsrc((void*)of.state_scales, 0, 0x7FFFFFFF, 0x00020000);
    const int ngroups = N / (16 * TG);
    float wsv[FN];
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
        wsv[fn] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wsf(fn))));
    int qpv[NG];
#pragma unroll
    for (int j = 0; j < NG; j++) qpv[j] = __builtin_amdgcn_readfirstlane(group_qp(of, col0 / 16 + TG * j));
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const f4 sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = row0 + 16 * fm + 4 * g + r;
            float y[FN];
#pragma unroll
            for (int fn = 0; fn < FN; fn++) y[fn] = ((float)(acc[fm][fn][r] >> SHIFT) * sx[r]) * wsv[fn];
#pragma unroll
            for (int j = 0; j < NG; j++) {
                float a = 0.0f;
#pragma unroll
                for (int t = 0; t < TG; t++) a = fmaxf(a, fabsf(y[TG * j + t]));
                a = max16(a);
                const int qp = qpv[j];
                const float inv = a > 0.0f ? (float)qp / a : 0.0f;   // IEEE division
#pragma unroll
                for (int t = 0; t < TG; t++) {
                    const int fn = TG * j + t;
                    const int col = col0 + 16 * fn + (lane & 15);
                    int q = (int)__builtin_rintf(y[fn] * inv);        // round half to even
                    q = q > qp ? qp : (q < -qp - 1 ? -qp - 1 : q);
                    const uint32_t off = (row < M && col < N) ? (uint32_t)(row * N + col) : 0x80000000u;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q, crs, (int)off, 0, 0);
                }
                const int grp = (col0 + 16 * TG * j) / (16 * TG);
                const float sc = a > 0.0f ? a / (float)qp : 0.0f;
                const uint32_t soff = (row < M && grp < ngroups && (lane & 15) == 0)
                                          ? 4u * (uint32_t)(row * ngroups + grp) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), srs, (int)soff, 0, 0);
            }
        }
    }
}

// store_tiles_states for a group (head) of 2 FN tiles split over this wave and a partner wave
// holding the same rows and the next FN tiles (or the previous): the maxima of every row over
// this wave's tiles and lanes are formed first and exchanged through xch (FM * 16 floats per
// wave, at slot 16 FM wave; the caller's LDS, free of other use, every wave of the workgroup
// taking part); then each output is quantised with the group's maximum and stored, and the
// wave holding the group's first columns (first) stores the scales.
template <int FM, int FN, int SHIFT, typename ScaleFn, typename WScaleFn>
__device__ __forceinline__ void store_tiles_states_pair(const v4i (&acc)[FM][FN], int row0, int col0, int lane,
                                                        int M, int N, ScaleFn sxf, WScaleFn wsf,
                                                        const OutForm& of, void* cbase, float* xch,
                                                        int wave, int partner, bool first)
{
    const int g = lane >> 4;
    const auto crs = __builtin_amdgcn_make_buffer_rsrc(cbase, 0, 0x7FFFFFFF, 0x00020000);
    const auto srs = __builtin_amdgcn_make_buffer_rsrc((void*)of.state_scales, 0, 0x7FFFFFFF, 0x00020000);
    const int ngroups = N / (32 * FN);
    const int grp = (first ? col0 : col0 - 16 * FN) / (32 * FN);
    float wsv[FN];
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
        wsv[fn] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wsf(fn))));
    const int qp = __builtin_amdgcn_readfirstlane(group_qp(of, col0 / 16));
    auto yv = [&](int fm, int fn, int r, float sx) __attribute__((always_inline)) {
        return ((float)(acc[fm][fn][r] >> SHIFT) * sx) * wsv[fn];
    };
    float amax[FM][4];
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const f4 sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float a = 0.0f;
#pragma unroll
            for (int fn = 0; fn < FN; fn++) a = fmaxf(a, fabsf(yv(fm, fn, r, sx[r])));
            amax[fm][r] = max16(a);
        }
    }
    __syncthreads();                  // every wave is past its last operand read of xch's LDS
    if ((lane & 15) == 0) {
#pragma unroll
        for (int fm = 0; fm < FM; fm++)
#pragma unroll
            for (int r = 0; r < 4; r++) xch[16 * FM * wave + 16 * fm + 4 * g + r] = amax[fm][r];
    }
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < FM; fm++) {
        const f4 sx = sxf(fm);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = row0 + 16 * fm + 4 * g + r;
            const float a = fmaxf(amax[fm][r], xch[16 * FM * partner + 16 * fm + 4 * g + r]);
            const float inv = a > 0.0f ? (float)qp / a : 0.0f;        // IEEE division
#pragma unroll
            for (int fn = 0; fn < FN; fn++) {
                const int col = col0 + 16 * fn + (lane & 15);
                int q = (int)__builtin_rintf(yv(fm, fn, r, sx[r]) * inv);   // round half to even
                q = q > qp ? qp : (q < -qp - 1 ? -qp - 1 : q);
                const uint32_t off = (row < M && col < N) ? (uint32_t)(row * N + col) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q, crs, (int)off, 0, 0);
            }
            const float sc = a > 0.0f ? a / (float)qp : 0.0f;
            const uint32_t soff = (first && row < M && grp < ngroups && (lane & 15) == 0)
                                      ? 4u * (uint32_t)(row * ngroups + grp) : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), srs, (int)soff, 0, 0);
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
enum Epi { kPlain = 0, kSegments = 1, kGlu = 2, kStates = 3 };

template <int BITS, bool DEQ, int EPI, int SG = 0>
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
    if constexpr (EPI == kStates) {
        // Low-bit states: a wave holds 64 columns, a head of 64 (SG = 4) or half of one of
        // 128 (SG = 8) whose other half is the wave of the neighbouring column quarter and
        // the same rows (wave ^ 2); the operand buffers, no longer read, carry the exchange.
        static_assert(DEQ && (SG == 4 || SG == 8), "states: fp32 epilogue, heads of 64 or 128");
        auto wsf = [&](int fn) __attribute__((always_inline)) { return group_scale(args.of, col0 / 16 + fn, w_scale); };
        if constexpr (SG == 4)
            store_tiles_states<8, 4, 0, 4>(acc, m0 + wm * 128, col0, lane, M, N, sxf, wsf, args.of,
                                           (void*)args.out);
        else
            store_tiles_states_pair<8, 4, 0>(acc, m0 + wm * 128, col0, lane, M, N, sxf, wsf, args.of,
                                             (void*)args.out, reinterpret_cast<float*>(&As[0][0]), wave,
                                             wave ^ 2, (wn & 1) == 0);
    } else if constexpr (EPI == kGlu)
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


// gemm_tern4_kernel: see the head of the file.  Each wave holds 4 x 8 MFMA tiles (128
// accumulation registers) and fits in half of its SIMD's registers, so the two waves of a SIMD
// fill each other's gaps between MFMAs.  Per slab a wave issues 32 MFMAs; every thread decodes
// one 16-byte piece of packed weights (four tern_steps) and widens its own four A tiles.
template <bool DEQ, int EPI, int SG = 0>
__global__ __launch_bounds__(NT4) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tern4_kernel(LargeArgs args)
{
    constexpr int BM = BM4, BN = BN4, NT = NT4;
    constexpr int AROW = 32;                        // code bytes of one token row per slab
    constexpr int AJ = BM * AROW / 16 / NT;         // 16-byte code loads per thread per slab
    static_assert(AJ == 2, "two code loads per thread and slab");
    __shared__ __align__(16) uint8_t A0[BM * AROW], A1[BM * AROW], A2[BM * AROW], A3[BM * AROW], A4[BM * AROW];
    __shared__ __align__(16) uint8_t Bt[5][BN * 64];
    __shared__ __align__(16) float sxs[BM];
    auto araw = [&](int s) __attribute__((always_inline)) -> uint8_t* {
        return s == 0 ? A0 : s == 1 ? A1 : s == 2 ? A2 : s == 3 ? A3 : A4;
    };

    // Tile order: workgroups are dispatched to the 8 XCDs in turn (linear index mod 8).  With
    // xcd_runs, XCD j takes a contiguous run of the tiles in (layer, row block, column block)
    // order, so that the workgroups resident on one XCD at a time share their activation rows
    // in that XCD's L2; the launcher asks for it when the tiles take more than one round of the
    // CUs (a single round measured faster in launch order).
    int layer = blockIdx.z, tile_y = blockIdx.y, tile_x = blockIdx.x;
    if (args.xcd_runs) {
        const int gx = gridDim.x, gy = gridDim.y, total = gx * gy * gridDim.z;
        const int id = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
        const int xcd = id & 7, q = total >> 3, r = total & 7;
        const int p = xcd * q + (xcd < r ? xcd : r) + (id >> 3);
        tile_x = p % gx;
        tile_y = (p / gx) % gy;
        layer = p / (gx * gy);
    }
    const int M = args.M, N = args.N, K = args.K;
    const int crow = K / 2;
    const uint8_t* codes = args.codes + (int64_t)layer * M * crow;
    const uint8_t* packed = args.wptrs ? (const uint8_t*)((const_u64_ptr)(const void*)args.wptrs)[layer] : args.w0;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = tile_y * BM, n0 = tile_x * BN;
    const int nblk = (K + 319) / 320;
    const int groups = (N + 15) / 16;

    // ---- packed weights: thread tid holds piece tid & 63 of the tile (16 rows) tid >> 6.
    const int g0 = n0 / 16;
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(packed + (int64_t)g0 * nblk * 1024), 0, (groups - g0) * nblk * 1024, 0x00020000);
    const int wq = tid & 63, wr = 16 * (tid >> 6) + (wq & 15);
    const uint32_t w_off = (uint32_t)(tid >> 6) * (uint32_t)nblk * 1024u + 16u * wq;
    // chunk swizzled by bits 1..2 of the row: each eight consecutive lanes of a 16-byte LDS
    // access (rows r..r+7 of one chunk column) then cover all 32 banks once
    const uint32_t b_lds = (uint32_t)(wr * 64 + 16 * ((wq >> 4) ^ ((wr >> 1) & 3)));
    auto load_w = [&](u4& dst, int blk) __attribute__((always_inline)) {
        dst = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)w_off, blk < nblk ? 1024 * blk : (int)0x80000000u, 0);
    };

    // ---- activation codes: per slab the 512 rows' 32 bytes go to the code slot in two
    // instructions per thread; instruction (s, wave) fills 1 KB, lane l the 16 bytes of chunk
    // Q = 64 (8 s + wave) + l: row Q / 2, chunk Q % 2 swizzled by bit 3 of the row.
    const auto ars = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + (int64_t)m0 * crow), 0, (M - m0) * crow, 0x00020000);
    uint32_t a_off;
    {
        const int Q = 64 * wave + lane, row = Q / 2, phys = Q % 2;
        a_off = (uint32_t)row * (uint32_t)crow + 16u * (phys ^ ((row >> 3) & 1));
    }
    const int a_step = 256 * crow;                      // instruction s: 256 rows further
    // instruction s of the code request of slab v (rows 256 s .. 256 s + 255 of the tile)
    auto load_a_part = [&](int v, int slot, int s) __attribute__((always_inline)) {
        int k = 320 * (v / 5) + 64 * (4 - v % 5);
        k = k < K ? k : K - 64;
        const int kb = v < 5 * nblk ? k / 2 : (int)0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_ptr)(araw(slot) + 1024 * (8 * s + wave)), 16,
                                                 a_off, kb + s * a_step, 0, 0);
    };
    auto load_a = [&](int v, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < AJ; s++) load_a_part(v, slot, s);
    };

    v4i acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = v4i{0, 0, 0, 0};

    const int am = 64 * wave + (lane & 15), g = lane >> 4;
    const uint32_t a_rd = (uint32_t)(am * 32 + 16 * ((g >> 1) ^ ((am >> 3) & 1)) + 8 * (g & 1));
    const int brow = lane & 15;
    const uint32_t b_rd = (uint32_t)(brow * 64 + 16 * (g ^ ((brow >> 1) & 3)));
    typedef u2 ARaw;
    auto read_a = [&](int slot, int i) __attribute__((always_inline)) {
        return *reinterpret_cast<const ARaw*>(araw(slot) + a_rd + 16 * AROW * i);
    };
    auto read_b = [&](int slot, int n) __attribute__((always_inline)) {
        return *reinterpret_cast<const v4i*>(Bt[slot] + b_rd + 1024 * n);
    };
    auto widen = [&](const ARaw& x) __attribute__((always_inline)) {
        return v4i{(int)((x[0] << 4) & 0xF0F0F0F0u), (int)(x[0] & 0xF0F0F0F0u),
                   (int)((x[1] << 4) & 0xF0F0F0F0u), (int)(x[1] & 0xF0F0F0F0u)};
    };

    u4 wnext;
    uint32_t pb[4];
    auto produce = [&](int p) __attribute__((always_inline)) {
        u4 t;
#pragma unroll
        for (int w = 0; w < 4; w++) t[w] = tern_step(pb[w]);
        *reinterpret_cast<u4*>(Bt[p] + b_lds) = t;
    };
    auto take_block = [&](int next_blk) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < 4; w++) pb[w] = wnext[w];
        load_w(wnext, next_blk);
    };

    // Prologue: weights of block 0 (then 1 in flight); codes of slabs 0..3 in LDS; trits of
    // slabs 0, 1 and 2; operands of slab 0 in registers.  The codes and scales are requested
    // together with the first weights, so the prologue waits for one round trip to memory.
    load_w(wnext, 0);
    load_a(0, 0);
    load_a(1, 1);
    load_a(2, 2);
    load_a(3, 3);
    constexpr int NSX = DEQ ? BM / NT : 0;
    if constexpr (DEQ) {
        const auto srs = __builtin_amdgcn_make_buffer_rsrc((void*)(args.scales + (int64_t)layer * M), 0, 4 * M, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_ptr)(sxs + 64 * wave), 4,
                                                 4u * (uint32_t)(m0 + 64 * wave + lane), 0, 0, 0);
    }
    wait_vmcnt<4 * AJ + NSX>();                         // the weight load of block 0
    take_block(1);
    produce(0);
    produce(1);
    produce(2);
    // the codes of slabs 0..2 (slab 1 reads those of slab 2); slab 3's, the scales and block
    // 1's weights may stay in flight: the barrier after slab 1 waits for slab 3's codes
    wait_vmcnt<AJ + NSX + 1>();
    block_sync();
    v4i af[2][4], bf[8];                                // A operands of slabs of even / odd index
    ARaw rn[4];                                         // packed A tiles of the next slab
#pragma unroll
    for (int i = 0; i < 4; i++) af[0][i] = widen(read_a(0, i));
#pragma unroll
    for (int n = 0; n < 8; n++) bf[n] = read_b(0, n);

    // Slab v = 5 blk + d (digit 4 - d of block blk), slots indexed by d: operands of v in
    // registers, the trits of v + 1 read from slot d + 1, those of v + 3 written to slot
    // d + 3, the codes of v + 4 requested into slot d + 4 (all mod 5).  Writing trits three
    // slabs ahead lets one workgroup barrier, after every odd slab, serve two slabs: every
    // write is published by a barrier before its slot is read, and every slot is read before
    // the barrier that precedes its next write.  The 32 MFMAs go B tile by B tile
    // (MFMA slot 4 n + m is A tile m x B tile n), so B tile n is free once slot 4 n + 3 is
    // issued: its operand of v + 1 is read behind slot 4 n + 5 and has the rest of the slab to
    // arrive.  The A operands of v + 1 go to the other register set (v odd / even), widened
    // from packed tiles read at slot 1.  Slot 0 requests the codes of v + 4; slots 2, 6, 10 and
    // 14 decode the next digit of the held weight words, written as the trits of v + 3 after
    // slot 14; slots 18, 22, 26 and 30 widen the A tiles of v + 1.
    auto slab = [&](int v, int d, auto parity, bool last = false) __attribute__((always_inline)) {
        constexpr int P = decltype(parity)::value, Q = 1 - P;
        const int s1 = (d + 1) % 5, s3 = (d + 3) % 5, s4 = (d + 4) % 5;
        u4 t;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const int n = j >> 2, m = j & 3;
            mfma_acc(acc[m][n], af[P][m], bf[n]);
            // the code request of v + 4, its two instructions half a slab apart
            if (j == 0) {
                if (d == 2) take_block(v / 5 + 2);    // slab v + 3 opens block v / 5 + 1
                load_a_part(v + 4, s4, 0);
            }
            if (j == 16) load_a_part(v + 4, s4, 1);
            if (j == 1) {
#pragma unroll
                for (int i = 0; i < 4; i++) rn[i] = read_a(s1, i);
            }
            if (j == 2 || j == 6 || j == 10 || j == 14) t[j >> 2] = tern_step(pb[j >> 2]);   // at digit 0, pb < 3: q = 0
            if (j == 14) *reinterpret_cast<u4*>(Bt[s3] + b_lds) = t;
            if ((j & 3) == 1 && j >= 5) bf[(j >> 2) - 1] = read_b(s1, (j >> 2) - 1);
            if (j == 18 || j == 22 || j == 26 || j == 30) af[Q][(j - 18) >> 2] = widen(rn[(j - 18) >> 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf[7] = read_b(s1, 7);
        // one barrier per two slabs, after each odd slab: the codes of v + 2 and v + 3 in LDS
        // before it (issued since: the AJ code loads of this slab and its weight load, if any);
        // after the trit write come, behind scheduling barriers, the B reads of tiles 3..7
        // (ds_read_b128, which cannot be merged), which may stay in flight.  The tile's last
        // slab (even) ends with a full barrier: its reads of a next slab are dropped as unused.
        if (P == 1) {
            if (d == 2) wait_vmcnt<AJ + 1>();
            else wait_vmcnt<AJ>();
            block_sync_reads_in_flight<5>();
        } else if (last) {
            block_sync();
        }
    };
    // Two blocks per iteration, so that the register set of each slab is known at compile
    // time (slab v uses set v & 1); an odd last block starts on an even slab.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The other forms run the tile's last block separately (below) and store each A tile row's
    // outputs while the next row computes; the states form, whose epilogue per row is large,
    // runs every block here and stores after the last one.
    constexpr bool FB = EPI != kStates;
    const int nbb = FB ? nblk - 1 : nblk;
    int blk = 0;
    for (; blk + 1 < nbb; blk += 2) {
        const int v = 5 * blk;
        slab(v, 0, P0{});
        slab(v + 1, 1, P1{});
        slab(v + 2, 2, P0{});
        slab(v + 3, 3, P1{});
        slab(v + 4, 4, P0{});
        slab(v + 5, 0, P1{});
        slab(v + 6, 1, P0{});
        slab(v + 7, 2, P1{});
        slab(v + 8, 3, P0{});
        slab(v + 9, 4, P1{});
    }
    if (blk < nbb) {
        const int v = 5 * blk;
        slab(v, 0, P0{});
        slab(v + 1, 1, P1{});
        slab(v + 2, 2, P0{});
        slab(v + 3, 3, P1{});
        slab(v + 4, 4, P0{}, !FB);
    }

    const float w_scale = args.wscales ? ((const_f32_ptr)(const void*)args.wscales)[layer] : args.wscale0;
    // this layer's outputs (the SwishGLU and segment forms run one layer)
    void* obase = DEQ ? (void*)(args.out + (int64_t)layer * M * N) : (void*)(args.acc + (int64_t)layer * M * N);
    const int row0 = m0 + 64 * wave;
    // The outputs of A tile row fm (16 token rows x 128 outputs), in the tile's output form.
    auto epilogue_row = [&](int fm) __attribute__((always_inline)) {
        v4i ar[1][8];
#pragma unroll
        for (int n = 0; n < 8; n++) ar[0][n] = acc[fm][n];
        const int r0 = row0 + 16 * fm;
        const bool inside = r0 + 16 <= M && n0 + 128 <= N;
        auto sxf = [&](int) __attribute__((always_inline)) {
            return *(const f4*)&sxs[64 * wave + 16 * fm + 4 * g];
        };
        if constexpr (EPI == kGlu) {
            if (inside)
                store_tiles_glu_inside<1, 8, 4>(ar, r0, n0, lane, N / 2, sxf, args.of.gate_scale,
                                                args.of.up_scale, (float*)obase);
            else
                store_tiles_glu<1, 8, 4>(ar, r0, n0, lane, M, N / 2, sxf, args.of.gate_scale,
                                         args.of.up_scale, obase);
        } else if constexpr (EPI == kSegments) {
            auto wsf = [&](int fn) __attribute__((always_inline)) { return group_scale(args.of, n0 / 16 + fn, w_scale); };
            if (DEQ && inside)
                store_tiles_inside<1, 8, 4>(ar, r0, n0, lane, N, sxf, wsf, (float*)obase);
            else
                store_tiles<1, 8, 4, DEQ>(ar, r0, n0, lane, M, N, sxf, wsf, obase);
        } else if (DEQ && inside)
            store_tiles_inside<1, 8, 4>(ar, r0, n0, lane, N, sxf,
                                        [&](int) __attribute__((always_inline)) { return w_scale; }, (float*)obase);
        else
            store_tiles<1, 8, 4, DEQ>(ar, r0, n0, lane, M, N, sxf,
                                      [&](int) __attribute__((always_inline)) { return w_scale; }, obase);
    };

    // The last block (slabs v0 .. v0 + 4 in slots 0 .. 4): its codes and trits all in LDS at
    // once, the MFMAs A tile row by A tile row (step 5 m + d: row m x slab d), so that the
    // outputs of row m leave while row m + 1 runs: they are stored after the first four MFMAs
    // of row m + 1, well past the latency of row m's last MFMA.  Operands are read one step
    // ahead into the other register set.  Slot 4's codes, requested here, are waited for at
    // step 4; slot 4 and trit slots 3 and 4 are free once every wave's reads have completed.
    if constexpr (FB) {
        const int v0 = 5 * nbb;
        // every wave's reads of the slots written below have landed (the last barrier may have
        // been a relaxed one, with a wave's last B reads -- of trit slot 4 -- still in flight)
        block_sync();
        load_a(v0 + 4, 4);
        produce(3);                                     // at digit 0, pb < 3: q = 0
        produce(4);
        wait_vmcnt<AJ>();                               // every code load but those of slot 4
        block_sync();
        v4i fa[2], fbv[2][8];
        ARaw fr;
        fa[0] = widen(read_a(0, 0));
#pragma unroll
        for (int n = 0; n < 8; n++) fbv[0][n] = read_b(0, n);
        mfma_operand_wait(fa[0]);
#pragma unroll
        for (int st = 0; st < 20; st++) {
            const int m = st / 5, d = st % 5, cur = st & 1, nxt = cur ^ 1;
            const int sn = st + 1, mn = sn / 5, dn = sn % 5;
            if (st == 4) {
                wait_vmcnt<0>();                        // the codes of slot 4
                block_sync();
                fa[cur] = widen(read_a(4, 0));
                mfma_operand_wait(fa[cur]);
            }
            const bool pre = sn < 20 && !(dn == 4 && mn == 0);   // slot 4's codes of row 0: after step 4's barrier
            if (pre) fr = read_a(dn, mn);
#pragma unroll
            for (int n = 0; n < 8; n++) {
                mfma_acc(acc[m][n], fa[cur], fbv[cur][n]);
                if (sn < 20) fbv[nxt][n] = read_b(dn, n);
                if (n == 3 && d == 0 && m >= 1) epilogue_row(m - 1);
                if (n == 4 && pre) fa[nxt] = widen(fr);   // three MFMAs before its first reader
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    wait_vmcnt<0>();
    mfma_drain();
    if constexpr (FB) {
        epilogue_row(3);
    } else {
        auto sxf = [&](int fm) __attribute__((always_inline)) {
            return *(const f4*)&sxs[64 * wave + 16 * fm + 4 * g];
        };
        store_tiles_states<4, 8, 4, SG>(acc, row0, n0, lane, M, N, sxf,
                                        [&](int fn) __attribute__((always_inline)) {
                                            return group_scale(args.of, n0 / 16 + fn, w_scale);
                                        }, args.of, (void*)args.out);
    }
}

}  // namespace

// Compute units of the current device, queried once per device (256 on MI355X).
static int device_cu_count()
{
    static int count[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (count[dev] <= 0) {
        int n = 0;
        count[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    }
    return count[dev];
}

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
    LargeArgs a{codes, scales, wptrs, w0, wscales, wscale0, out_f32, acc_i32, M, K, N, of, 0};
    if (of.states && (L != 1 || out_f32 == nullptr || of.nseg == 0 ||
                      (of.state_tiles != 4 && of.state_tiles != 8) || N % (16 * of.state_tiles) != 0))
        return hipErrorInvalidValue;
    if (bits == 4) {
        dim3 grid((N + BN4 - 1) / BN4, (M + BM4 - 1) / BM4, L);
        a.xcd_runs = (int64_t)grid.x * grid.y * grid.z > device_cu_count();
        if (of.states && of.state_tiles == 8) hipLaunchKernelGGL((gemm_tern4_kernel<true, kStates, 8>), grid, dim3(NT4), 0, stream, a);
        else if (of.states) hipLaunchKernelGGL((gemm_tern4_kernel<true, kStates, 4>), grid, dim3(NT4), 0, stream, a);
        else if (out_f32 != nullptr && of.glu) hipLaunchKernelGGL((gemm_tern4_kernel<true, kGlu>), grid, dim3(NT4), 0, stream, a);
        else if (out_f32 != nullptr && of.nseg > 0) hipLaunchKernelGGL((gemm_tern4_kernel<true, kSegments>), grid, dim3(NT4), 0, stream, a);
        else if (out_f32 != nullptr) hipLaunchKernelGGL((gemm_tern4_kernel<true, kPlain>), grid, dim3(NT4), 0, stream, a);
        else hipLaunchKernelGGL((gemm_tern4_kernel<false, kPlain>), grid, dim3(NT4), 0, stream, a);
    } else {
        dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, L);
        if (of.states && of.state_tiles == 8) hipLaunchKernelGGL((gemm_tern_kernel<8, true, kStates, 8>), grid, dim3(NT), 0, stream, a);
        else if (of.states) hipLaunchKernelGGL((gemm_tern_kernel<8, true, kStates, 4>), grid, dim3(NT), 0, stream, a);
        else if (out_f32 != nullptr && of.glu) hipLaunchKernelGGL((gemm_tern_kernel<8, true, kGlu>), grid, dim3(NT), 0, stream, a);
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
