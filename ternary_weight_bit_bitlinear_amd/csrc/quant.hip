// quant.hip -- activation stage of H-BitLinear on gfx950: online normalised Hadamard transform,
// per-token absmax, quantisation to INT8 / INT4 codes.  One workgroup per token row.
//
// Method: BitNet v2 news write-up (Xinzhiyuan), H-BitLinear passage -- an online Hadamard
// transform (entries +1/-1, orthogonal rows) applied before activation quantisation; BitNet
// b1.58 2B4T write-up (itdecent.cn), section 1.2 -- absmax activation quantisation.
//
// The transform is the Sylvester H_K / sqrt(K).  Its radix-2 stages run with butterfly span
// 1, 2, 4, ..., K/2 (index bit 0 first), each butterfly (a, b) -> (a + b, a - b), and the
// 1/sqrt(K) is one fp32 multiply after the last stage.  Every thread keeps E = K/T values of
// the row in registers.  The stages are grouped: a group handles the index bits that are
// register bits in the current data layout; between groups the row is exchanged through LDS
// into the next layout.  Whatever the grouping, every element is formed from the same
// operands in the same stage order as the plain in-place butterfly, so the fp32 results do
// not depend on the grouping.
//
// Layouts (K = 2^L, T threads, E = K/T = 2^LE):
//   load layout A: thread t, register e = 4 r + j holds k = r*4T + 4t + j (float4 loads,
//                  fully coalesced); its register bits are {0, 1} and the top LE-2 bits.
//   group p >= 1:  register bits are the next LE not-yet-transformed index bits, padded with
//                  the lowest bits when fewer remain; the other bits index the thread.
// LDS addresses are XOR-swizzled (swz below): 16-byte chunks stay whole and the strided
// accesses of the middle groups spread over the banks.
#include "common.h"

namespace bitnet {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// Threads per row: 64 up to K = 2048, then K / 32 (32 elements per thread).  Fewer elements
// per thread (more waves per row) hide more of the load latency; 16 per thread measured slower
// (one more LDS exchange), 64 per thread slower at K >= 4096.
__host__ __device__ constexpr int threads_for(int L) { return L >= 12 ? (1 << (L - 5)) : 64; }

// Without the transform there are no exchanges, so the thread count only sets how many waves
// share a row: kPlainE elements per thread, 64 to 1024 threads.  16 measured 3-4 % faster than
// 32 at 16384 rows of 4096 and 8192, and the same at 2048 rows (8 and 64 no better).
constexpr int kPlainE = 16;
__host__ __device__ constexpr int threads_plain(int L)
{
    return (1 << L) / kPlainE < 64 ? 64 : ((1 << L) / kPlainE > 1024 ? 1024 : (1 << L) / kPlainE);
}
__host__ __device__ constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v >> 1); }

// Deposit the low bits of v into the set bits of mask, lowest first.
__host__ __device__ constexpr uint32_t pdep(uint32_t v, uint32_t mask)
{
    uint32_t r = 0;
    for (int b = 0; b < 32; b++) {
        if (mask & (1u << b)) {
            if (v & 1u) r |= 1u << b;
            v >>= 1;
        }
    }
    return r;
}

// Register-bit mask of group p (p = 0 is the load layout).
__host__ __device__ constexpr uint32_t group_mask(int L, int LE, int p)
{
    if (p == 0) {
        int LT = L - LE;
        uint32_t hi = ((1u << (LE - 2)) - 1u) << (2 + LT);
        return 3u | hi;
    }
    int lo = 2 + (p - 1) * LE;
    int hi = lo + LE < L ? lo + LE : L;
    uint32_t m = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
    int pad = LE - (hi - lo);
    return m | ((1u << pad) - 1u);
}

__host__ __device__ constexpr int num_groups(int L, int LE) { return 1 + (L - 2 + LE - 1) / LE; }

// LDS index of element k: index bits 2.. XOR-ed with higher bits, so that 16-byte chunks stay
// whole and the strided accesses of the exchanges spread over the banks (32 consecutive lanes
// are served together).  For K >= 4096 bits 7..10 go into bits 2..5: with bits 8..10 only,
// two lanes that differ in bit 7 of k meet in one bank (1-6 % slower at K = 4096..16384;
// K = 1024 measured faster with the narrower form).  Either form is its own inverse on [0, K).
template <int L>
__host__ __device__ constexpr uint32_t swz(uint32_t k)
{
    if constexpr (L >= 12) return k ^ (((k >> 7) & 15u) << 2);
    else return k ^ (((k >> 8) & 7u) << 2);
}

// Index bits that swz can change (bits 2..5, or 2..4 below K = 4096).
template <int L>
__host__ __device__ constexpr uint32_t swz_bits() { return L >= 12 ? 15u << 2 : 7u << 2; }

// Position of index bit b among the register bits of MASK.
__host__ __device__ constexpr int regpos(uint32_t mask, int b)
{
    int pos = 0;
    for (int c = 0; c < b; c++)
        if (mask & (1u << c)) pos++;
    return pos;
}

// Stage of index bit B: butterflies between registers whose indices differ in regpos(MASK, B).
template <int E, uint32_t MASK, int B>
__device__ __forceinline__ void stage(float (&v)[E])
{
    constexpr int h = 1 << regpos(MASK, B);
#pragma unroll
    for (int e = 0; e < E; e++) {
        if ((e & h) == 0) {
            float a = v[e], b = v[e + h];
            v[e] = a + b;
            v[e + h] = a - b;
        }
    }
}

// Stages for index bits LO, LO+1, ..., HI-1, in that order.
template <int E, uint32_t MASK, int LO, int HI>
__device__ __forceinline__ void butterflies(float (&v)[E])
{
    if constexpr (LO < HI) {
        stage<E, MASK, LO>(v);
        butterflies<E, MASK, LO + 1, HI>(v);
    }
}

template <int L, bool HAD = true>
struct Geometry {
    static constexpr int K = 1 << L;
    static constexpr int T = HAD ? threads_for(L) : threads_plain(L);
    static constexpr int LT = ilog2c(T);
    static constexpr int LE = L - LT;
    static constexpr int E = 1 << LE;
    static constexpr int G = num_groups(L, LE);
};

// Thread part of k in a layout with register mask MASK.
template <int L, uint32_t MASK>
__device__ __forceinline__ uint32_t thread_bits(uint32_t t)
{
    return pdep(t, ((1u << L) - 1u) & ~MASK);
}

// LDS byte address of register e of layout MASK.  swz is linear over XOR and the thread part
// tb and register part of k have no bit in common, so swz(k) = swz(tb) ^ swz(ke); the two
// parts can share only bits that swz changes, so swz(k) = (swz(tb) ^ lo) + hi with lo the
// register part's share of those bits and hi the rest.  tb4 = 4 swz(tb) is formed once per
// thread; each distinct lo costs one XOR and hi becomes the instruction's immediate offset.
template <int L, uint32_t MASK>
__device__ __forceinline__ uint32_t layout_addr(uint32_t tb4, int e)
{
    const uint32_t c = swz<L>(pdep((uint32_t)e, MASK));
    const uint32_t lo = c & swz_bits<L>(), hi = c & ~swz_bits<L>();
    return (tb4 ^ (lo << 2)) + (hi << 2);
}

template <int L, uint32_t MASK, int E>
__device__ __forceinline__ void store_layout(float* lds, uint32_t t, const float (&v)[E])
{
    const uint32_t tb4 = swz<L>(thread_bits<L, MASK>(t)) << 2;
    char* base = reinterpret_cast<char*>(lds);
    if constexpr ((MASK & 3u) == 3u) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
            *reinterpret_cast<float4*>(base + layout_addr<L, MASK>(tb4, e)) =
                make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    } else {
#pragma unroll
        for (int e = 0; e < E; e++) *reinterpret_cast<float*>(base + layout_addr<L, MASK>(tb4, e)) = v[e];
    }
}

template <int L, uint32_t MASK, int E>
__device__ __forceinline__ void load_layout(const float* lds, uint32_t t, float (&v)[E])
{
    const uint32_t tb4 = swz<L>(thread_bits<L, MASK>(t)) << 2;
    const char* base = reinterpret_cast<const char*>(lds);
    if constexpr ((MASK & 3u) == 3u) {
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            float4 f = *reinterpret_cast<const float4*>(base + layout_addr<L, MASK>(tb4, e));
            v[e] = f.x; v[e + 1] = f.y; v[e + 2] = f.z; v[e + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; e++) v[e] = *reinterpret_cast<const float*>(base + layout_addr<L, MASK>(tb4, e));
    }
}

// Groups 1.. of the transform, recursively (each step: LDS exchange, then its stages).
template <int L, int P>
__device__ __forceinline__ void transform_groups(float* lds, uint32_t t,
                                                 float (&v)[Geometry<L>::E])
{
    using G = Geometry<L>;
    if constexpr (P < G::G) {
        constexpr uint32_t PREV = group_mask(L, G::LE, P - 1);
        constexpr uint32_t CUR = group_mask(L, G::LE, P);
        constexpr int LO = 2 + (P - 1) * G::LE;
        constexpr int HI = LO + G::LE < L ? LO + G::LE : L;
        store_layout<L, PREV, G::E>(lds, t, v);
        __syncthreads();
        load_layout<L, CUR, G::E>(lds, t, v);
        __syncthreads();
        butterflies<G::E, CUR, LO, HI>(v);
        transform_groups<L, P + 1>(lds, t, v);
    }
}

template <int L, bool HAD>
__device__ __forceinline__ constexpr uint32_t final_mask()
{
    using G = Geometry<L, HAD>;
    return HAD ? group_mask(L, G::LE, G::G - 1) : group_mask(L, G::LE, 0);
}

template <int BITS>
__device__ __forceinline__ int quant_code(float x, float inv)
{
    constexpr int QP = (1 << (BITS - 1)) - 1;
    float r = __builtin_rintf(x * inv);        // round half to even (v_rndne_f32)
    int q = (int)r;
    q = q > QP ? QP : q;
    q = q < -QP - 1 ? -QP - 1 : q;
    return q;
}

// The code of x as the low bits of a float: fl(fl(x * inv) + 1.5 * 2^23) rounds fl(x * inv) to
// the nearest integer, ties to even (the sum's unit in the last place is 1), and for
// |fl(x * inv)| < 2^22 its low mantissa bits hold that integer in two's complement, so the low
// byte (nibble) is the INT8 (INT4) code.  No clamp is needed: x is at most gamma in magnitude
// and inv = fl(Qp / gamma), so |x * inv| <= Qp (1 + 2^-24), which rounds to at most Qp.
__device__ __forceinline__ uint32_t code_bits(float x, float inv)
{
    return __builtin_bit_cast(uint32_t, x * inv + 12582912.0f);
}

// NORM: the row is first RMS-normalised, y[k] = (x[k] * r) * gain[k] with
// r = fp32(1 / sqrt(sum_k x[k]^2 / K + eps)), the sum and r taken in double.
template <int L, int BITS, bool HAD, bool NORM>
__global__ __launch_bounds__((Geometry<L, HAD>::T)) void quantize_rows_kernel(
    const float* __restrict__ x, uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ xh, float hadamard_c, const float* __restrict__ gain, float eps)
{
    using G = Geometry<L, HAD>;
    constexpr int K = G::K, T = G::T, E = G::E;
    constexpr int QP = (1 << (BITS - 1)) - 1;
    // With the transform: the row for the exchanges, then the code bytes; the reduction slots
    // sit past the K code bytes.  Without: only the reduction slots.
    __shared__ __align__(16) float lds[HAD ? K : 64];
    float* red = HAD ? lds + K / 2 : lds;

    const uint32_t t = threadIdx.x;
    const int64_t m = blockIdx.x;
    const float* xr = x + m * K;

    // Load layout A: coalesced float4 loads.
    float v[E];
#pragma unroll
    for (int r = 0; r < E / 4; r++) {
        f4 f = __builtin_nontemporal_load(reinterpret_cast<const f4*>(xr) + r * T + t);
        v[4 * r] = f[0]; v[4 * r + 1] = f[1]; v[4 * r + 2] = f[2]; v[4 * r + 3] = f[3];
    }

    if constexpr (NORM) {
        // The gains in load layout A (the same float4 positions as the row), requested with
        // the row: loaded after the barrier below (a memory fence), they would cost each row
        // one more round trip.
        f4 gv[E / 4];
#pragma unroll
        for (int r = 0; r < E / 4; r++) gv[r] = reinterpret_cast<const f4*>(gain)[r * T + t];
        // Each fp32 square is exact in double, so the row sum is the same to ~K 2^-53 relative
        // in any order: far below the fp32 rounding of r.  Waves reduce with shuffles, then in
        // a fixed order through LDS.
        __shared__ double rss[T / 64];
        double ss = 0.0;
#pragma unroll
        for (int e = 0; e < E; e++) ss += (double)v[e] * (double)v[e];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if ((t & 63) == 0) rss[t >> 6] = ss;
        __syncthreads();
        ss = rss[0];
#pragma unroll
        for (int w = 1; w < T / 64; w++) ss += rss[w];
        const double ms = ss / (double)K + (double)eps;
        const float rs = ms > 0.0 ? (float)(1.0 / __builtin_sqrt(ms)) : 0.0f;
#pragma unroll
        for (int r = 0; r < E / 4; r++)
#pragma unroll
            for (int j = 0; j < 4; j++) v[4 * r + j] = (v[4 * r + j] * rs) * gv[r][j];
    }

    // For even L, c = 1/sqrt(K) = 2^(-L/2) exactly, and c * y is exact unless it falls below
    // the normal range: then max |c y| = c max |y|, and fl(fl(c y) * inv) = fl(y * (c inv))
    // with c inv exact, so the multiply by c folds into inv.  A row whose largest |y| is below
    // 2^-100 (where c y might round) takes the multiply, as does a call that wants x_h.
    constexpr bool FOLD = HAD && (L % 2 == 0);
    if constexpr (HAD) {
        butterflies<E, group_mask(L, G::LE, 0), 0, 2>(v);
        transform_groups<L, 1>(lds, t, v);
        if constexpr (!FOLD) {
#pragma unroll
            for (int e = 0; e < E; e++) v[e] = v[e] * hadamard_c;
        }
    }
    constexpr uint32_t FM = final_mask<L, HAD>();
    const uint32_t tb = thread_bits<L, FM>(t);

    // absmax over the row: exact, so the reduction order does not matter.
    float g = 0.0f;
#pragma unroll
    for (int e = 0; e < E; e++) g = fmaxf(g, fabsf(v[e]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) g = fmaxf(g, __shfl_xor(g, off, 64));
    if ((t & 63) == 0) red[t >> 6] = g;
    __syncthreads();
    g = red[0];
#pragma unroll
    for (int w = 1; w < T / 64; w++) g = fmaxf(g, red[w]);

    float vscale = 1.0f;   // the factor still to apply to v: c when it could not be folded
    if constexpr (FOLD) {
        if (xh != nullptr || g < 0x1p-100f) {
#pragma unroll
            for (int e = 0; e < E; e++) v[e] = v[e] * hadamard_c;
            g = g * hadamard_c;
        } else {
            g = g * hadamard_c;   // exact: a power of two times a normal number
            vscale = hadamard_c;
        }
    }

    if (xh != nullptr) {
        float* xo = xh + m * K;
#pragma unroll
        for (int e = 0; e < E; e++) xo[tb | pdep((uint32_t)e, FM)] = v[e];
    }

    const float inv0 = g > 0.0f ? (float)QP / g : 0.0f;   // IEEE division
    const float inv = inv0 * vscale;                       // exact (power-of-two scaling)
    if (t == 0) scales[m] = g > 0.0f ? g / (float)QP : 0.0f;

    if constexpr (!HAD) {
        // Load layout A: register 4 r + j holds k = 4 T r + 4 t + j, so the four codes of a
        // float4 are consecutive: INT8, one 4-byte store; INT4, the four nibbles of this
        // thread (low nibbles of word k / 8 when t is even, high when odd) joined with the
        // neighbour's, and stored by the even thread.
#pragma unroll
        for (int r = 0; r < E / 4; r++) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t q = code_bits(v[4 * r + j], inv);
                if constexpr (BITS == 8) w |= (q & 255u) << (8 * j);
                else w |= (q & 15u) << (8 * j + 4 * (t & 1));
            }
            if constexpr (BITS == 8) {
                *reinterpret_cast<uint32_t*>(codes + m * K + 4 * T * r + 4 * t) = w;
            } else {
                w |= (uint32_t)__shfl_xor((int)w, 1, 64);
                if ((t & 1) == 0) *reinterpret_cast<uint32_t*>(codes + m * (K / 2) + 2 * T * r + 2 * t) = w;
            }
        }
        return;
    }

    // Codes into LDS as bytes at position k, then out with 16-byte stores.
    int8_t* qb = reinterpret_cast<int8_t*>(lds);
#pragma unroll
    for (int e = 0; e < E; e++) qb[tb | pdep((uint32_t)e, FM)] = (int8_t)code_bits(v[e], inv);
    __syncthreads();
    if constexpr (BITS == 8) {
        uint4* dst = reinterpret_cast<uint4*>(codes + m * K);
        const uint4* src = reinterpret_cast<const uint4*>(qb);
        for (int c = t; c < K / 16; c += T) dst[c] = src[c];
    } else {
        // 32 codes -> 16 bytes: word w holds codes 8w+p (low nibble) and 8w+p+4 (high nibble).
        uint4* dst = reinterpret_cast<uint4*>(codes + m * (K / 2));
        const uint32_t* src = reinterpret_cast<const uint32_t*>(qb);
        for (int c = t; c < K / 32; c += T) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t lo = src[8 * c + 2 * i], hi = src[8 * c + 2 * i + 1];
                w[i] = (lo & 0x0F0F0F0Fu) | ((hi & 0x0F0F0F0Fu) << 4);
            }
            dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// Rows whose width is not a power of two in [256, 16384] (no Hadamard): two passes over the row.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_rows_generic_kernel(
    const float* __restrict__ x, int K, uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ xh)
{
    constexpr int QP = (1 << (BITS - 1)) - 1;
    __shared__ float red[4];
    const int t = threadIdx.x;
    const int64_t m = blockIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + m * K);
    const int nc = K / 4;
    float g = 0.0f;
    for (int c = t; c < nc; c += 256) {
        float4 f = xr[c];
        g = fmaxf(g, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) g = fmaxf(g, __shfl_xor(g, off, 64));
    if ((t & 63) == 0) red[t >> 6] = g;
    __syncthreads();
    g = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = g > 0.0f ? (float)QP / g : 0.0f;
    if (t == 0) scales[m] = g > 0.0f ? g / (float)QP : 0.0f;
    if (xh != nullptr) {
        float4* xo = reinterpret_cast<float4*>(xh + m * K);
        for (int c = t; c < nc; c += 256) xo[c] = xr[c];
    }
    // 8 codes per step (two float4): keeps INT4 words whole.
    for (int c2 = t; c2 < nc / 2; c2 += 256) {
        float4 a = xr[2 * c2], b = xr[2 * c2 + 1];
        float vals[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; i++) q[i] = g > 0.0f ? quant_code<BITS>(vals[i], inv) : 0;
        if constexpr (BITS == 8) {
            uint32_t lo = (q[0] & 255) | (q[1] & 255) << 8 | (q[2] & 255) << 16 | (uint32_t)(q[3] & 255) << 24;
            uint32_t hi = (q[4] & 255) | (q[5] & 255) << 8 | (q[6] & 255) << 16 | (uint32_t)(q[7] & 255) << 24;
            reinterpret_cast<uint2*>(codes + m * K)[c2] = make_uint2(lo, hi);
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int p = 0; p < 4; p++) w |= (uint32_t)((q[p] & 15) | ((q[p + 4] & 15) << 4)) << (8 * p);
            reinterpret_cast<uint32_t*>(codes + m * (K / 2))[c2] = w;
        }
    }
}

template <int L, int BITS, bool HAD>
hipError_t launch_rows(const float* x, int M, uint8_t* codes, float* scales, float* xh, float c,
                       const float* gain, float eps, hipStream_t s)
{
    if (gain != nullptr)
        hipLaunchKernelGGL((quantize_rows_kernel<L, BITS, HAD, true>), dim3(M), dim3(Geometry<L, HAD>::T), 0,
                           s, x, codes, scales, xh, c, gain, eps);
    else
        hipLaunchKernelGGL((quantize_rows_kernel<L, BITS, HAD, false>), dim3(M), dim3(Geometry<L, HAD>::T), 0,
                           s, x, codes, scales, xh, c, gain, eps);
    return hipGetLastError();
}

template <int BITS, bool HAD>
hipError_t dispatch_L(int L, const float* x, int M, uint8_t* codes, float* scales, float* xh,
                      float c, const float* gain, float eps, hipStream_t s)
{
    switch (L) {
    case 8: return launch_rows<8, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    case 9: return launch_rows<9, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    case 10: return launch_rows<10, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    case 11: return launch_rows<11, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    case 12: return launch_rows<12, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    case 13: return launch_rows<13, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    case 14: return launch_rows<14, BITS, HAD>(x, M, codes, scales, xh, c, gain, eps, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize(const float* x, int M, int K, int bits, int use_hadamard,
                           uint8_t* codes, float* scales, float* xh, hipStream_t stream,
                           const float* gain, float eps)
{
    int L = 0;
    while ((1 << L) < K) L++;
    const bool pow2 = (1 << L) == K && L >= 8 && L <= 14;
    // 1/sqrt(K) rounded once to fp32 from a correctly rounded double square root.
    const float c = (float)(1.0 / __builtin_sqrt((double)K));
    if (use_hadamard) {
        if (!pow2) return hipErrorInvalidValue;
        return bits == 8 ? dispatch_L<8, true>(L, x, M, codes, scales, xh, c, gain, eps, stream)
                         : dispatch_L<4, true>(L, x, M, codes, scales, xh, c, gain, eps, stream);
    }
    if (pow2)
        return bits == 8 ? dispatch_L<8, false>(L, x, M, codes, scales, xh, c, gain, eps, stream)
                         : dispatch_L<4, false>(L, x, M, codes, scales, xh, c, gain, eps, stream);
    if (gain != nullptr) return hipErrorInvalidValue;   // the norm needs the one-pass row kernel
    if (bits == 8)
        hipLaunchKernelGGL(quantize_rows_generic_kernel<8>, dim3(M), dim3(256), 0, stream, x, K, codes,
                           scales, xh);
    else
        hipLaunchKernelGGL(quantize_rows_generic_kernel<4>, dim3(M), dim3(256), 0, stream, x, K, codes,
                           scales, xh);
    return hipGetLastError();
}

}  // namespace bitnet
