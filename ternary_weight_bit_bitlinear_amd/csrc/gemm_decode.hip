// gemm_decode.hip -- ternary product for decode shapes (M <= 16 tokens) on gfx950, with the
// dequantisation epilogue fused; one launch can cover L independent layers.
//
// Method: BitNet b1.58 2B4T write-up (itdecent.cn), section 1.2 -- the product with {-1,0,+1}
// weights is exact integer arithmetic; section 1.1 -- five trits per byte, base 3, the first
// trit most significant.
//
// At decode shapes the kernel is bound by the packed weight stream, so each weight byte must
// be unpacked with as few vector instructions as possible:
//   - a lane loads the 16 packed bytes (one 16-byte load) that form its part of the MFMA B
//     operands for one 320-weight block: row n, bytes 16g..16g+15 of the row's 64-byte block
//     (g = lane/16);
//   - all five trits of a byte come from one 8-byte LDS lookup: a table of the 256 byte
//     values, entry = [t0 t1 t2 t3 | t4 0 0 0] as int8, replicated 32 times (lanes l and l+32
//     share a copy; an 8-byte read is served 32 lanes at a time, so lookups never conflict);
//     the lookup address 256*byte + 8*(lane%32) is built by one v_perm_b32.
// Two table entries are one 16-slot B operand, so an MFMA covers two packed bytes (ten trits
// and six zero slots): eight MFMAs per 16-row tile and block.  The MFMA only needs A and B to
// agree on what each of the 64 k-slots holds; the activation operand is assembled to match
// (a 4 x 4 byte transpose of four 16-code runs plus the fifth digit's codes, shifted into
// place), once per wave and block, shared by the wave's four column tiles.  The zero slots
// meet arbitrary activation codes and add 0; so do pad slabs (k >= K), whose trits are 0.
// MFMAs go operand by operand, each preceded by the two lookups of the operand six places
// ahead, so a wave keeps twelve lookups in flight without exceeding what its LDS counter
// tracks exactly.
//
// Two kernels share that inner step: a persistent streaming kernel that walks (layer, row
// chunk) items block by block with the activations staged in LDS, for calls that give every
// CU work; and a split-K kernel for calls of a few thousand rows, in which the four waves of a
// workgroup divide one 16-row group's blocks and add their partial tiles at the end.
#include "common.h"

#include <atomic>
#include <type_traits>

namespace bitnet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int DT = 256;             // threads per workgroup: four waves
// Weight rows of a workgroup's item: four waves of TPW 16-row MFMA column tiles each.  TPW = 4
// when there are enough items to fill the chip; a single layer of 4096 rows would then be only
// 16 workgroups, so few-item calls use TPW = 1 (64-row items).
__host__ __device__ constexpr int wg_rows(int tpw) { return DT / 64 * 16 * tpw; }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4 x 4 byte transpose: out[i] = [r0.b_i, r1.b_i, r2.b_i, r3.b_i]
__device__ __forceinline__ v4i transpose4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3)
{
    const uint32_t p01l = perm(r1, r0, 0x05010400u), p01h = perm(r1, r0, 0x07030602u);
    const uint32_t p23l = perm(r3, r2, 0x05010400u), p23h = perm(r3, r2, 0x07030602u);
    return v4i{(int)perm(p23l, p01l, 0x05040100u), (int)perm(p23l, p01l, 0x07060302u),
               (int)perm(p23h, p01h, 0x05040100u), (int)perm(p23h, p01h, 0x07060302u)};
}

// The per-layer pointer and scale arrays are never written while a kernel runs; reading them
// through the constant address space makes them scalar loads (a plain load next to the
// output stores would be a vector load, and a vector-held buffer address needs a loop).
typedef const __attribute__((address_space(4))) uint64_t* const_u64_ptr;
typedef const __attribute__((address_space(4))) float* const_f32_ptr;

__device__ __forceinline__ const uint8_t* layer_ptr(const uint8_t* const* ptrs, const uint8_t* p0, int l)
{
    return ptrs ? (const uint8_t*)((const_u64_ptr)(const void*)ptrs)[l] : p0;
}

__device__ __forceinline__ float layer_scale(const float* scales, float s0, int l)
{
    return scales ? ((const_f32_ptr)(const void*)scales)[l] : s0;
}

__device__ __forceinline__ uint32_t sext_nibbles(uint32_t n)
{
    return ((n ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

struct DecodeArgs {
    const uint8_t* codes;          // L x M rows of activation codes
    const float* scales;           // L x M
    const uint8_t* const* wptrs;   // device array of L packed weights, or null (then w0)
    const uint8_t* w0;
    const float* wscales;          // device array of L weight scales, or null (then wscale0)
    float wscale0;
    float* out;                    // L x M x N fp32 (M x N/2 with of.glu), or null
    int32_t* acc;                  // L x M x N int32, or null
    int L, M, K, N;
    OutForm of;                    // segments / gate-up pairs (L = 1, out only)
};

// Cache policy of the weight loads and output stores: non-temporal.  Each weight byte and each
// output is touched once, so keeping them in the caches only evicts the activation codes,
// which every row chunk of a layer reads again.
constexpr int kNonTemporal = 2;

constexpr int ASTRIDE = 336;     // LDS bytes per staged activation row: 320 codes + 16 (banks)

typedef unsigned int u2 __attribute__((ext_vector_type(2)));

// Table entry of byte value v (< 256): the five base-3 digits, most significant first, each
// minus one, as int8 -- lo = digits 0..3, hi = digit 4 -- or zeros for v >= 243, a value no
// packed byte takes.  floor(x / 3) = (171 x) >> 9 for x < 256 (171 / 512 exceeds 1/3 by
// less than 1/(3 * 256)); a byte b in 0..2 becomes b - 1 as ((b | 0x80) - 1) ^ 0x80, four
// bytes at a time without borrows.
__device__ __forceinline__ void table_entry(uint32_t v, uint32_t& lo, uint32_t& hi)
{
    const uint32_t q1 = (171u * v) >> 9, q2 = (171u * q1) >> 9, q3 = (171u * q2) >> 9, q4 = (171u * q3) >> 9;
    const uint32_t d4 = v - 3u * q1, d3 = q1 - 3u * q2, d2 = q2 - 3u * q3, d1 = q3 - 3u * q4, d0 = q4;
    const uint32_t packed = d0 | d1 << 8 | d2 << 16 | d3 << 24;
    lo = v < 243u ? ((packed | 0x80808080u) - 0x01010101u) ^ 0x80808080u : 0u;
    hi = v < 243u ? (d4 - 1u) & 0xFFu : 0u;
}

// The lookup table, 256 values x 32 replicas x 8 bytes, filled with 16-byte stores (chunk q:
// value q / 16, replicas 2 (q % 16) and + 1), consecutive threads on consecutive chunks.
// Every entry is computed where it is stored, so the stores do not wait on anything.
__device__ __forceinline__ void build_table(uint32_t* lut, int tid)
{
    static_assert(256 * 16 % DT == 0, "chunks per thread");
#pragma unroll
    for (int j = 0; j < 256 * 16 / DT; j++) {
        const int q = tid + DT * j;
        uint32_t lo, hi;
        table_entry((uint32_t)(q >> 4), lo, hi);
        *reinterpret_cast<u4*>(reinterpret_cast<uint8_t*>(lut) + 16 * q) = u4{lo, hi, lo, hi};
    }
    __syncthreads();
}

// B operand q of a block (q = TPW j + f: operand j of column tile f) = the table entries of the
// lane's bytes 2j and 2j + 1 of tile f; the lookup address 256 * byte + 8 * (lane % 32)
// (laneoff = 8 * (lane % 32)) is one byte permute.
template <int TPW>
__device__ __forceinline__ v4i lookup_operand(const uint32_t* lut, uint32_t laneoff, const u4 (&w)[TPW], int q)
{
    const int f = q % TPW, j = q / TPW;
    const uint32_t word = w[f][j >> 1];
    const uint32_t sh = (uint32_t)(2 * (j & 1)) << 8;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(lut);
    const u2 e0 = *reinterpret_cast<const u2*>(base + perm(word, laneoff, 0x0C0C0400u | sh));
    const u2 e1 = *reinterpret_cast<const u2*>(base + perm(word, laneoff, 0x0C0C0500u | sh));
    return v4i{(int)e0[0], (int)e0[1], (int)e1[0], (int)e1[1]};
}

// The 8 TPW MFMAs of one 320-weight block for TPW column tiles.  d[i]: the lane's 16 codes of
// digit slab i, k = 320 B + 64 i + 16 g + (0..15) of row lane & 15.  The A operand j matching B operand j:
// for the lane's bytes p = 2j + h (h = 0, 1), slots 8h..8h+3 hold the codes of digits 0..3
// (k = b + 64 i, b = 16 g + p) and slot 8h + 4 the code of digit 4; slots 8h+5..8h+7 meet
// zero trits.  The lookups run LA operands ahead of the MFMAs, two per MFMA, so that 2 LA of
// them are in flight at each MFMA -- fewer than the 15 LDS operations a wave can count, so
// each MFMA waits exactly for its own operand.  bn: the block's first LA operands.
template <int TPW, int LA>
__device__ __forceinline__ void block_mfmas(const uint32_t* lut, uint32_t laneoff, const u4 (&d)[5],
                                            const u4 (&w)[TPW], const v4i (&bn)[LA], v4i (&acc)[TPW])
{
    constexpr int NQ = 8 * TPW;
    v4i ring[LA + 1];
#pragma unroll
    for (int i = 0; i < LA; i++) ring[i] = bn[i];
    v4i A0, A1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NQ; q++) {
        const int j = q / TPW, f = q % TPW;
        if (f == 0 && (j & 1) == 0) {
            // A operands 2u and 2u + 1 (u = j / 2), used by the next 2 TPW MFMAs
            const int u = j >> 1;
            const v4i t = transpose4(d[0][u], d[1][u], d[2][u], d[3][u]);   // t[v]: byte 4u + v
            const uint32_t e = d[4][u];
            A0 = v4i{t[0], (int)e, t[1], (int)(e >> 8)};
            A1 = v4i{t[2], (int)(e >> 16), t[3], (int)(e >> 24)};
        }
        if (q + LA < NQ) ring[(q + LA) % (LA + 1)] = lookup_operand<TPW>(lut, laneoff, w, q + LA);
        acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8((j & 1) ? A1 : A0, ring[q % (LA + 1)], acc[f], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

constexpr int kLookahead = 6;

// Position in a workgroup's stream of (item, block) steps.  An item is (layer l, chunk c of
// wg_rows(TPW) weight rows); the workgroup's items are blockIdx.x, blockIdx.x + gridDim.x, ...  The
// layer's weight pointer and weight scale are fetched once per item, when the position
// enters it: a scalar load inside every step would make every step wait for it, and that
// wait also drains all outstanding LDS reads.
struct StreamPos {
    int item, B, l, c;
    __amdgpu_buffer_rsrc_t wrs;   // the item's weight tiles
    __amdgpu_buffer_rsrc_t crs;   // the layer's activation codes
    __amdgpu_buffer_rsrc_t srs;   // the layer's activation scales
    float ws;
};

// Epilogue forms of the streaming kernel, one instantiation each, so that the plain one carries
// none of the others' code inside its loop: one weight scale per layer; a scale per row
// segment; gate / up pairs; segments whose outputs leave as low-bit states (SG tiles of 16
// columns per head).
enum Epi { kPlain = 0, kSegments = 1, kGlu = 2, kStates = 3 };

template <int BITS, bool DEQ, int TPW, int EPI = kPlain, int SG = 0>
__global__ __launch_bounds__(DT, 2) void gemm_decode_kernel(DecodeArgs a)
{
    constexpr int WAVE_ROWS = 16 * TPW, WG_ROWS = wg_rows(TPW);
    __shared__ __align__(16) uint32_t lut[256 * 64];   // 256 values x 32 copies x 8 bytes
    __shared__ __align__(16) uint8_t abuf[2][16 * ASTRIDE];
    __shared__ float sbuf[2][17];     // activation scales of the 16 rows, then the weight scale
    __shared__ float sred[EPI == kStates ? 4 * 16 : 1];   // states: a wave's head maxima per row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    build_table(lut, tid);

    const int K = a.K, N = a.N, M = a.M;
    const int nblk = (K + 319) / 320;
    const int crow = BITS == 8 ? K : K / 2;            // code bytes per activation row
    const int groups = (N + 15) / 16;                   // 16-row weight groups (tiles per block)
    const int nchunk = (N + WG_ROWS - 1) / WG_ROWS;
    const int items = a.L * nchunk;
    const int my_items = (int)blockIdx.x < items ? (items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int total = my_items * nblk;
    if (total == 0) return;
    const uint32_t laneoff = 8u * (uint32_t)(lane & 31);
    const int g = lane >> 4;

    // Workgroups are dispatched to the eight XCDs round-robin (workgroup b on XCD b % 8), and
    // each XCD has its own L2.  When the grid and the item count are multiples of eight, the
    // workgroup's k-th item slot s = b + k * grid is mapped to item (s % 8) * (items / 8) +
    // s / 8: each XCD then works through a contiguous range of items (whole layers), and a
    // layer's activation codes are fetched into one L2 instead of eight.  The mapping is a
    // bijection on the slots either way.
    const bool xcd_map = items % 8 == 0 && gridDim.x % 8 == 0;
    const int per_xcd = items / 8;
    const uint32_t tile_bytes = 1024u * (uint32_t)nblk;         // one 16-row group of weights
    auto start = [&](StreamPos& p, int item) {
        p.item = item;
        p.B = 0;
        const int it = xcd_map && item < items ? (item & 7) * per_xcd + (item >> 3) : item;
        p.l = it / nchunk;
        p.c = it - p.l * nchunk;
        // Past the last item the position is never used for data that is kept; clamp the
        // layer so the pointer and scale reads stay inside their arrays.
        const int lc = p.l < a.L ? p.l : a.L - 1;
        const int g0 = p.c * (WG_ROWS / 16);
        p.wrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(layer_ptr(a.wptrs, a.w0, lc) + (int64_t)g0 * tile_bytes), 0,
            (int)((uint32_t)(groups - g0) * tile_bytes), 0x00020000);
        p.crs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.codes + (int64_t)lc * M * crow), 0, (int)((uint32_t)M * (uint32_t)crow), 0x00020000);
        p.srs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(DEQ ? a.scales + (int64_t)lc * M : nullptr), 0, DEQ ? 4 * M : 0, 0x00020000);
        p.ws = DEQ ? layer_scale(a.wscales, a.wscale0, lc) : 0.0f;
    };
    auto advance = [&](StreamPos& p) {
        if (++p.B == nblk) start(p, p.item + (int)gridDim.x);
    };

    // ---- weights: one 1 KB tile (16 rows x 64 bytes) per MFMA column tile and block; the
    // tile's 16-byte pieces are in lane order, so lane l reads piece l.  Buffer loads: rows
    // past the last 16-row group read as zero (their outputs are not stored).
    uint32_t w_off[TPW];
#pragma unroll
    for (int f = 0; f < TPW; f++) w_off[f] = (uint32_t)(wave * TPW + f) * tile_bytes + 16u * lane;
    auto load_w = [&](u4 (&dst)[TPW], const StreamPos& p) {
#pragma unroll
        for (int f = 0; f < TPW; f++)
            dst[f] = __builtin_amdgcn_raw_buffer_load_b128(p.wrs, (int)w_off[f], 1024 * p.B, kNonTemporal);
    };

    // ---- activations: the workgroup stages the 16 rows x 320 codes of a block in LDS with
    // coalesced loads (rows past M read as zero; slabs past K meet zero trits), plus the 16
    // activation scales of the item.
    constexpr int ACH = BITS == 8 ? 20 : 10;            // 16-byte chunks per row and block
    const int q0 = tid, q1 = tid + DT;                  // this thread's chunks (q1 only if < 16*ACH)
    constexpr bool TWO = DT < 16 * ACH;                 // some threads stage two chunks
    const bool has_q0 = q0 < 16 * ACH, has_q1 = TWO && q1 < 16 * ACH;
    const uint32_t c0 = 16u * (q0 % ACH), c1 = 16u * (q1 % ACH);   // chunk offsets in a block
    struct ASlot {
        u4 v0, v1;       // this thread's one or two 16-byte chunks of codes
        float s;         // threads 0..15: activation scale of row tid
        float ws;        // weight scale of the layer (uniform)
    };
    // Branch-free loads: a thread without a chunk reads at an offset past the buffer range,
    // which returns zeros.  A chunk past the end of the row (a pad slab, whose trits are 0)
    // reads the row's last 16 bytes instead, so no load leaves the row.
    const uint32_t kOut = 0x7FFFFFF0u;
    const uint32_t rb0 = has_q0 ? (uint32_t)(q0 / ACH) * (uint32_t)crow : kOut;
    const uint32_t rb1 = has_q1 ? (uint32_t)(q1 / ACH) * (uint32_t)crow : kOut;
    const uint32_t clast = (uint32_t)crow - 16u;
    auto load_a = [&](ASlot& dst, const StreamPos& p) {
        const auto rs = p.crs;
        const uint32_t kb = (BITS == 8 ? 320u : 160u) * (uint32_t)p.B;
        const uint32_t o0 = rb0 + min(kb + c0, clast), o1 = rb1 + min(kb + c1, clast);
        dst.v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o0, 0, 0);
        if constexpr (TWO) dst.v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o1, 0, 0);
        if constexpr (DEQ) {
            dst.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(p.srs, 4 * (tid & 15), 0, 0));
            dst.ws = p.ws;
        }
    };
    auto stage_a = [&](int buf, const ASlot& x) {
        auto put = [&](u4 v, int q) {
            uint8_t* row = abuf[buf] + (q / ACH) * ASTRIDE;
            if constexpr (BITS == 8) {
                *reinterpret_cast<u4*>(row + 16 * (q % ACH)) = v;
            } else {
                u4 lo = u4{sext_nibbles(v[0] & 0x0F0F0F0Fu), sext_nibbles((v[0] >> 4) & 0x0F0F0F0Fu),
                           sext_nibbles(v[1] & 0x0F0F0F0Fu), sext_nibbles((v[1] >> 4) & 0x0F0F0F0Fu)};
                u4 hi = u4{sext_nibbles(v[2] & 0x0F0F0F0Fu), sext_nibbles((v[2] >> 4) & 0x0F0F0F0Fu),
                           sext_nibbles(v[3] & 0x0F0F0F0Fu), sext_nibbles((v[3] >> 4) & 0x0F0F0F0Fu)};
                *reinterpret_cast<u4*>(row + 32 * (q % ACH)) = lo;
                *reinterpret_cast<u4*>(row + 32 * (q % ACH) + 16) = hi;
            }
        };
        if (has_q0) put(x.v0, q0);
        if (TWO && has_q1) put(x.v1, q1);
        if (DEQ && tid < 16) sbuf[buf][tid] = x.s;
        if (DEQ && tid == 16) sbuf[buf][16] = x.ws;
    };

    auto lookup_op = [&](const u4 (&w)[TPW], int q) -> v4i { return lookup_operand<TPW>(lut, laneoff, w, q); };

    v4i acc[TPW];
#pragma unroll
    for (int f = 0; f < TPW; f++) acc[f] = v4i{0, 0, 0, 0};

    // One block of one item: 8 TPW MFMAs; the first kLookahead operands of a step are looked
    // up at the end of the previous step (bn).
    constexpr int LA = kLookahead;
    auto compute = [&](const u4 (&w)[TPW], int buf, v4i (&bn)[LA]) {
        const uint8_t* ar = abuf[buf] + (lane & 15) * ASTRIDE + 16 * g;
        u4 d[5];
#pragma unroll
        for (int i = 0; i < 5; i++) d[i] = *reinterpret_cast<const u4*>(ar + 64 * i);
        block_mfmas<TPW, LA>(lut, laneoff, d, w, bn, acc);
    };

    // Epilogue of an item.  MFMA 16x16 output: lane l, register r -> row 4 (l >> 4) + r,
    // column l & 15.  Gate / up pairs (tiles 2j, 2j + 1) leave as SiLU(gate) * up in column
    // (first row of the wave) / 2 + 16 j + (l & 15) of the M x N/2 output.
    auto finish = [&](const StreamPos& p, int buf) {
        const float wsc = DEQ ? sbuf[buf][16] : 0.0f;
        const int row0 = p.c * WG_ROWS + wave * WAVE_ROWS;
        if constexpr (EPI == kStates) {
            // Low-bit states, as the large-M kernel's store_tiles_states: each output y,
            // dequantised as below, is quantised per row and per head of 16 SG columns with its
            // segment's Qp.  A head is WPH = SG / TPW consecutive waves of the workgroup (the
            // launcher takes TPW = SG / 4: one head per workgroup): the head's maximum for a row
            // is the lane's maximum over its tiles, then over the 16 lanes of the row group
            // (max16), then over the head's waves through LDS.  Every wave reaches this point at
            // the same step, so the barrier is met by all.
            constexpr int WPH = SG / TPW;
            static_assert(DEQ && (SG == 4 || SG == 8) && SG % TPW == 0 && (WPH == 1 || WPH == 2 || WPH == 4),
                          "states: fp32 epilogue, a head within one workgroup");
            const int nheads = N / (16 * SG), head = row0 / (16 * SG);
            const int qp = group_qp(a.of, row0 / 16);
            float wsv[TPW];
#pragma unroll
            for (int f = 0; f < TPW; f++) wsv[f] = group_scale(a.of, row0 / 16 + f, wsc);
            float y[TPW][4], amax[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float sx = sbuf[buf][4 * g + r];
                float m = 0.0f;
#pragma unroll
                for (int f = 0; f < TPW; f++) {
                    y[f][r] = ((float)acc[f][r] * sx) * wsv[f];
                    m = fmaxf(m, fabsf(y[f][r]));
                }
                amax[r] = max16(m);
            }
            if constexpr (WPH > 1) {
                if ((lane & 15) == 0) {
#pragma unroll
                    for (int r = 0; r < 4; r++) sred[16 * wave + 4 * g + r] = amax[r];
                }
                __syncthreads();
                const int w0 = wave & ~(WPH - 1);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    float m = sred[16 * w0 + 4 * g + r];
#pragma unroll
                    for (int w = 1; w < WPH; w++) m = fmaxf(m, sred[16 * (w0 + w) + 4 * g + r]);
                    amax[r] = m;
                }
            }
            const auto cs = __builtin_amdgcn_make_buffer_rsrc((void*)a.out, 0, M * N, 0x00020000);
            const auto ss = __builtin_amdgcn_make_buffer_rsrc((void*)a.of.state_scales, 0, 4 * M * nheads,
                                                              0x00020000);
            const bool owner = (lane & 15) == 0 && wave % WPH == 0;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int mo = 4 * g + r;
                const float inv = amax[r] > 0.0f ? (float)qp / amax[r] : 0.0f;   // IEEE division
#pragma unroll
                for (int f = 0; f < TPW; f++) {
                    const int n = row0 + 16 * f + (lane & 15);
                    int q = (int)__builtin_rintf(y[f][r] * inv);              // round half to even
                    q = q > qp ? qp : (q < -qp - 1 ? -qp - 1 : q);
                    const uint32_t o = mo < M && n < N ? (uint32_t)(mo * N + n) : 0x80000000u;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q, cs, (int)o, 0, kNonTemporal);
                }
                const float sc = amax[r] > 0.0f ? amax[r] / (float)qp : 0.0f;
                const uint32_t so = owner && mo < M && head < nheads ? 4u * (uint32_t)(mo * nheads + head)
                                                                     : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), ss, (int)so, 0,
                                                      kNonTemporal);
            }
#pragma unroll
            for (int f = 0; f < TPW; f++) acc[f] = v4i{0, 0, 0, 0};
            return;
        }
        if constexpr (EPI == kGlu) {
            static_assert(DEQ && TPW % 2 == 0, "gate / up pairs need the fp32 epilogue and tile pairs");
            {
                const int F = N / 2;
                const auto hs = __builtin_amdgcn_make_buffer_rsrc((void*)a.out, 0, 4 * M * F, 0x00020000);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int mo = 4 * g + r;
                    const float sx = sbuf[buf][mo];
#pragma unroll
                    for (int j = 0; j < TPW / 2; j++) {
                        const int col = row0 / 2 + 16 * j + (lane & 15);
                        uint32_t o = 4u * ((uint32_t)mo * (uint32_t)F + (uint32_t)col);
                        o = mo < M && col < F ? o : 0x80000000u;
                        const float gv = ((float)acc[2 * j][r] * sx) * a.of.gate_scale;
                        const float uv = ((float)acc[2 * j + 1][r] * sx) * a.of.up_scale;
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, silu_mul(gv, uv)), hs,
                                                              (int)o, 0, kNonTemporal);
                    }
                }
#pragma unroll
                for (int f = 0; f < TPW; f++) acc[f] = v4i{0, 0, 0, 0};
                return;
            }
        }
        const int nbase = row0 + (lane & 15);
        void* obase = DEQ ? (void*)(a.out + (int64_t)p.l * M * N) : (void*)(a.acc + (int64_t)p.l * M * N);
        const auto os = __builtin_amdgcn_make_buffer_rsrc(obase, 0, 4 * M * N, 0x00020000);
        // Buffer stores: an element outside the M x N output gets an offset past the buffer
        // range and is dropped, so the stores need no branches.
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int mo = 4 * g + r;
            const float sx = DEQ ? sbuf[buf][mo] : 0.0f;
#pragma unroll
            for (int f = 0; f < TPW; f++) {
                const int n = nbase + 16 * f;
                uint32_t o = 4u * ((uint32_t)mo * (uint32_t)N + (uint32_t)n);
                o = mo < M ? o : 0x80000000u;
                o = n < N ? o : 0x80000000u;
                uint32_t v;
                if constexpr (DEQ)
                    v = __builtin_bit_cast(uint32_t, ((float)acc[f][r] * sx) *
                                                     (EPI == kSegments ? group_scale(a.of, row0 / 16 + f, wsc) : wsc));
                else
                    v = (uint32_t)acc[f][r];
                __builtin_amdgcn_raw_buffer_store_b32(v, os, (int)o, 0, kNonTemporal);
            }
        }
#pragma unroll
        for (int f = 0; f < TPW; f++) acc[f] = v4i{0, 0, 0, 0};
    };

    // Pipeline: weights run three steps ahead (a four-slot register ring); activations are
    // loaded three steps ahead into registers and staged into LDS one step ahead.  Waiting for
    // a load also waits for every load issued before it, so the activations of step t + 1
    // (staged during step t) must have been issued no later than the weights of step t + 1.
    // Loads are unconditional -- past the last step the positions stay put -- so that no
    // branch separates a load from its use.
    StreamPos pc, pa, pw;
    start(pc, blockIdx.x);
    pa = pc;
    pw = pc;
    u4 w0[TPW], w1[TPW], w2[TPW], w3[TPW];          // weight ring
    ASlot x0, x1, x2, x3;                           // activation ring
    load_a(x0, pa);                                 // step 0
    load_w(w0, pw);
    stage_a(0, x0);
    if (1 < total) { advance(pa); advance(pw); }
    load_a(x1, pa);                                 // step 1
    load_w(w1, pw);
    if (2 < total) { advance(pa); advance(pw); }
    load_a(x2, pa);                                 // step 2
    load_w(w2, pw);
    __syncthreads();                                // table and step 0 activations in LDS
    v4i bn[LA];                                     // the next step's first operands
#pragma unroll
    for (int i = 0; i < LA; i++) bn[i] = lookup_op(w0, i);

    // Step t: loads for step t + 3, MFMAs of step t, tile-0 lookups of step t + 1, staging of
    // step t + 1.
    auto step = [&](const u4 (&w)[TPW], const u4 (&wn)[TPW], u4 (&wpre)[TPW], const ASlot& xnext,
                    ASlot& xpre, int t) {
        if (t + 3 < total) { advance(pa); advance(pw); }
        load_a(xpre, pa);
        load_w(wpre, pw);
        compute(w, t & 1, bn);
        stage_a((t + 1) & 1, xnext);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < LA; i++) bn[i] = lookup_op(wn, i);
        if (pc.B == nblk - 1) finish(pc, t & 1);
        advance(pc);
        __syncthreads();
    };
    int t = 0;
    for (; t + 4 <= total; t += 4) {
        step(w0, w1, w3, x1, x3, t);
        step(w1, w2, w0, x2, x0, t + 1);
        step(w2, w3, w1, x3, x1, t + 2);
        step(w3, w0, w2, x0, x2, t + 3);
    }
    if (t < total) step(w0, w1, w3, x1, x3, t);
    if (t + 1 < total) step(w1, w2, w0, x2, x0, t + 1);
    if (t + 2 < total) step(w2, w3, w1, x3, x1, t + 2);
}

// Few-item calls (one layer of a few thousand rows): a workgroup per 16-row weight group, the
// group's K blocks split over the four waves (wave w takes blocks w, w + 4, ...), so that a
// 4096-row layer is 256 workgroups with a few blocks per wave instead of 64 workgroups that
// each walk all the blocks.  A wave reads its activation operands straight from memory (the
// layer's codes stay in the L2): the lane's 16 codes of each digit slab are one load.  Each
// wave prefetches four blocks; the four partial int32 tiles are added in LDS (integer sums,
// exact in any order) and the sum goes through the same epilogue as the streaming kernel.
template <int BITS, bool DEQ>
__global__ __launch_bounds__(DT, 2) void gemm_decode_splitk_kernel(DecodeArgs a)
{
    static_assert(DT == 256, "four waves: one per register of the summed tile");
    __shared__ __align__(16) uint32_t lut[256 * 64];
    __shared__ __align__(16) int32_t part[4 * 64 * 4];   // partial tiles: wave, lane, register

    // The wave index is made visibly uniform: the wave's block count then steers scalar
    // branches and selects instead of per-lane control flow.
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, N = a.N, M = a.M;
    const int nblk = (K + 319) / 320;
    const int crow = BITS == 8 ? K : K / 2;
    const int groups = (N + 15) / 16;
    const int l = (int)blockIdx.x / groups, gi = (int)blockIdx.x - l * groups;
    const uint32_t tile_bytes = 1024u * (uint32_t)nblk;
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(layer_ptr(a.wptrs, a.w0, l) + (int64_t)gi * tile_bytes), 0, (int)tile_bytes, 0x00020000);
    // Rows past M fall outside the range and read as zero (their outputs are not stored).
    const auto crs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.codes + (int64_t)l * M * crow), 0, (int)((uint32_t)M * (uint32_t)crow), 0x00020000);
    const int nb = wave < nblk ? (nblk - 1 - wave) / 4 + 1 : 0;   // this wave's blocks

    // Loads of the wave's i-th block (block wave + 4 i): the lane's weight piece and its codes of
    // the five digit slabs.  Past the wave's last block the offsets leave the buffer ranges and
    // the loads return zeros, so every load is unconditional.  A slab past K (whose trits are
    // 0) reads the row's last codes instead, so no load leaves its row.
    typedef typename std::conditional<BITS == 8, u4, u2>::type CodeVec;
    struct Slot {
        u4 w[1];
        CodeVec x[5];
    };
    constexpr uint32_t CB = BITS == 8 ? 16u : 8u;        // code bytes per lane and slab
    const uint32_t rowoff = (uint32_t)(lane & 15) * (uint32_t)crow;
    const uint32_t clast = (uint32_t)crow - CB;
    const uint32_t kOut = 0x80000000u;
    auto load = [&](Slot& s, int i) {
        // past = 2^31 when i >= nb, else 0 (the sign of nb - 1 - i; arithmetic rather than a
        // select, which the compiler would turn into branches around the loads)
        const uint32_t past = (uint32_t)(nb - 1 - i) & kOut;
        const uint32_t B = (uint32_t)(wave + 4 * i);
        s.w[0] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)(1024u * B + 16u * lane + past), 0, kNonTemporal);
#pragma unroll
        for (int d = 0; d < 5; d++) {
            const uint32_t k0 = 320u * B + 64u * d + 16u * g;
            const uint32_t o = rowoff + min(BITS == 8 ? k0 : k0 / 2, clast) + past;
            if constexpr (BITS == 8) s.x[d] = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)o, 0, 0);
            else s.x[d] = __builtin_amdgcn_raw_buffer_load_b64(crs, (int)o, 0, 0);
        }
    };
    auto codes = [&](const Slot& s, u4 (&d)[5]) {
#pragma unroll
        for (int i = 0; i < 5; i++) {
            if constexpr (BITS == 8) {
                d[i] = s.x[i];
            } else {
                const u2 v = s.x[i];
                d[i] = u4{sext_nibbles(v[0] & 0x0F0F0F0Fu), sext_nibbles((v[0] >> 4) & 0x0F0F0F0Fu),
                          sext_nibbles(v[1] & 0x0F0F0F0Fu), sext_nibbles((v[1] >> 4) & 0x0F0F0F0Fu)};
            }
        }
    };

    Slot s0, s1, s2, s3;
    load(s0, 0);
    load(s1, 1);
    load(s2, 2);
    load(s3, 3);
    build_table(lut, tid);

    const uint32_t laneoff = 8u * (uint32_t)(lane & 31);
    constexpr int LA = kLookahead;
    v4i acc[1] = {v4i{0, 0, 0, 0}};
    v4i bn[LA];
#pragma unroll
    for (int i = 0; i < LA; i++) bn[i] = lookup_operand<1>(lut, laneoff, s0.w, i);
    // Step i: the MFMAs of block i, the loads of block i + 4 into the freed slot, the first
    // lookups of block i + 1.
    auto step = [&](Slot& s, const Slot& sn, int i) {
        u4 d[5];
        codes(s, d);
        block_mfmas<1, LA>(lut, laneoff, d, s.w, bn, acc);
        load(s, i + 4);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < LA; q++) bn[q] = lookup_operand<1>(lut, laneoff, sn.w, q);
    };
    int i = 0;
    for (; i + 4 <= nb; i += 4) {
        step(s0, s1, i);
        step(s1, s2, i + 1);
        step(s2, s3, i + 2);
        step(s3, s0, i + 3);
    }
    if (i < nb) step(s0, s1, i);
    if (i + 1 < nb) step(s1, s2, i + 1);
    if (i + 2 < nb) step(s2, s3, i + 2);

    // Sum of the four partial tiles: thread (wave r, lane l) forms register r of lane l, i.e.
    // output row 4 (l >> 4) + r, column l & 15 of the group.
    *reinterpret_cast<v4i*>(&part[4 * (64 * wave + lane)]) = acc[0];
    __syncthreads();
    int32_t sum = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) sum += part[4 * (64 * w + lane) + wave];
    const int m = 4 * g + wave, n = 16 * gi + (lane & 15);
    void* obase = DEQ ? (void*)(a.out + (int64_t)l * M * N) : (void*)(a.acc + (int64_t)l * M * N);
    const auto os = __builtin_amdgcn_make_buffer_rsrc(obase, 0, 4 * M * N, 0x00020000);
    uint32_t o = 4u * ((uint32_t)m * (uint32_t)N + (uint32_t)n);
    o = m < M && n < N ? o : kOut;
    uint32_t v;
    if constexpr (DEQ) {
        const auto srs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales + (int64_t)l * M), 0, 4 * M, 0x00020000);
        const float sx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, 4 * m, 0, 0));
        const float ws = group_scale(a.of, gi, layer_scale(a.wscales, a.wscale0, l));
        v = __builtin_bit_cast(uint32_t, ((float)sum * sx) * ws);
    } else {
        v = (uint32_t)sum;
    }
    __builtin_amdgcn_raw_buffer_store_b32(v, os, (int)o, 0, kNonTemporal);
}

enum class DecodeKind { Wide, Pairs, Narrow, SplitK };

template <int BITS, bool DEQ, int EPI>
void launch_streaming(DecodeKind kind, int grid, const DecodeArgs& a, hipStream_t stream)
{
    if constexpr (EPI == kGlu) {
        if (kind == DecodeKind::Wide)
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, DEQ, 4, EPI>), dim3(grid), dim3(DT), 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, DEQ, 2, EPI>), dim3(grid), dim3(DT), 0, stream, a);
    } else {
        if (kind == DecodeKind::Wide)
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, DEQ, 4, EPI>), dim3(grid), dim3(DT), 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, DEQ, 1, EPI>), dim3(grid), dim3(DT), 0, stream, a);
    }
}

template <int BITS, bool DEQ>
void launch_decode(DecodeKind kind, int grid, const DecodeArgs& a, hipStream_t stream)
{
    if (kind == DecodeKind::SplitK)
        hipLaunchKernelGGL((gemm_decode_splitk_kernel<BITS, DEQ>), dim3(grid), dim3(DT), 0, stream, a);
    else if constexpr (DEQ) {
        if (a.of.states && a.of.state_tiles == 8)   // one head of 128 per workgroup
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, DEQ, 2, kStates, 8>), dim3(grid), dim3(DT), 0, stream, a);
        else if (a.of.states)                       // one head of 64 per workgroup
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, DEQ, 1, kStates, 4>), dim3(grid), dim3(DT), 0, stream, a);
        else if (a.of.glu) launch_streaming<BITS, DEQ, kGlu>(kind, grid, a, stream);
        else if (a.of.nseg > 0) launch_streaming<BITS, DEQ, kSegments>(kind, grid, a, stream);
        else launch_streaming<BITS, DEQ, kPlain>(kind, grid, a, stream);
    } else {
        launch_streaming<BITS, DEQ, kPlain>(kind, grid, a, stream);
    }
}

}  // namespace

int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_gemm_decode(const uint8_t* codes, int L, int M, int K, int N, int bits,
                              const uint8_t* const* wptrs, const uint8_t* w0,
                              const float* scales, const float* wscales, float wscale0,
                              float* out_f32, int32_t* acc_i32, hipStream_t stream,
                              const OutForm& of)
{
    // Buffer ranges and lane offsets are 32-bit: one weight matrix and one layer's codes must
    // stay below 2 GiB.
    const int64_t packed = (int64_t)((N + 15) / 16) * 16 * 64 * ((K + 319) / 320);
    if (packed >= ((int64_t)1 << 31) || (int64_t)M * K >= ((int64_t)1 << 31) ||
        4 * (int64_t)M * N >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    DecodeArgs a{codes, scales, wptrs, w0, wscales, wscale0, out_f32, acc_i32, L, M, K, N, of};
    // Low-bit states: the streaming kernel with one head per workgroup (items of the head's 64
    // or 128 rows, one or two tiles per wave).  Else, enough 256-row items to give every CU
    // one: the streaming kernel with four tiles per wave.  Else, for gate / up pairs, the
    // streaming kernel with two tiles per wave (128-row items).
    // Else, when the 16-row groups fit two workgroups per CU: one workgroup per group, K split
    // over its waves.  Else the streaming kernel with one tile per wave (64-row items).
    const int cus = device_cus();
    const int items4 = L * ((N + wg_rows(4) - 1) / wg_rows(4));
    const int groups = L * ((N + 15) / 16);
    DecodeKind kind;
    int grid;
    if (of.states && (out_f32 == nullptr || L != 1 || (of.state_tiles != 4 && of.state_tiles != 8) ||
                      N % (16 * of.state_tiles) != 0))
        return hipErrorInvalidValue;
    if (of.states) {
        kind = DecodeKind::Wide;                 // the kind is not used for states
        const int itemsh = L * ((N + 16 * of.state_tiles - 1) / (16 * of.state_tiles));
        grid = itemsh < 2 * cus ? itemsh : 2 * cus;
    } else if (items4 >= cus) {
        kind = DecodeKind::Wide;
        grid = items4 < 2 * cus ? items4 : 2 * cus;
    } else if (of.glu) {
        // gate / up tiles must meet in one wave: two tiles per wave (128-row items)
        kind = DecodeKind::Pairs;
        const int items2 = L * ((N + wg_rows(2) - 1) / wg_rows(2));
        grid = items2 < 2 * cus ? items2 : 2 * cus;
    } else if (groups <= 2 * cus) {
        kind = DecodeKind::SplitK;
        grid = groups;
    } else {
        kind = DecodeKind::Narrow;
        const int items1 = L * ((N + wg_rows(1) - 1) / wg_rows(1));
        grid = items1 < 2 * cus ? items1 : 2 * cus;
    }
    if (out_f32 != nullptr) {
        if (bits == 8) launch_decode<8, true>(kind, grid, a, stream);
        else launch_decode<4, true>(kind, grid, a, stream);
    } else {
        if (bits == 8) launch_decode<8, false>(kind, grid, a, stream);
        else launch_decode<4, false>(kind, grid, a, stream);
    }
    return hipGetLastError();
}

}  // namespace bitnet
