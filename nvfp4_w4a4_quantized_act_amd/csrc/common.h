// Shared device helpers and host-side argument checks for the QUADS kernels.
//
// NVFP4 arithmetic follows arXiv 2607.15810, section 2.2 ("FP4" and "FP8"
// paragraphs): E2M1 element codes with magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
// one OCP E4M3FN scale byte per 16 elements; one fp32 tensor scale.  Every
// rounding is round-to-nearest-even of the exact real value; the helpers
// below reach that with exact fp64 products and directed fp32 thresholds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/quads.h"

namespace quads {

constexpr int kBlock = 16;              // NVFP4 block length
constexpr int kScoreFanin = 64;         // fixed order of the channel-score sum
constexpr int kE4m3MaxCode = 0x7E;      // 448
constexpr int kAmaxGroups = 1024;       // partial maxima per tensor (max)

// ---------------------------------------------------------------- device --

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 value of an E4M3FN code 0..0x7E (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    return c < 8 ? (float)c * 0x1p-9f
                 : ldexpf((float)(8u + (c & 7u)), (int)(c >> 3) - 10);
}

// Magnitude of an E2M1 code 0..7.
__device__ __forceinline__ float e2m1_value(uint32_t m) {
    // 0, .5, 1, 1.5 -> m/2 ; 2, 3, 4, 6 -> (2 + (m&1)) * 2^((m>>1)-1)
    return m < 4 ? 0.5f * (float)m : ldexpf((float)(2u + (m & 1u)), (int)(m >> 1) - 2);
}

// E4M3FN code nearest to q >= 0 (ties to even mantissa), saturating at 448.
// q must lie on the same side of every E4M3 midpoint as the exact quotient it
// stands for; a correctly rounded fp64 quotient of the operands used here does.
__device__ __forceinline__ uint32_t e4m3_rne_code(double q) {
    if (!(q < 448.0)) return kE4m3MaxCode;
    if (q < 0x1p-6) return (uint32_t)rint(q * 512.0);       // subnormal codes 0..8
    uint64_t b = (uint64_t)__double_as_longlong(q);
    uint64_t r = (b + 0xFFFFFFFFFFFFull + ((b >> 49) & 1ull)) >> 49;   // exp | 3-bit mantissa
    uint32_t c = (uint32_t)r - (1016u << 3);                 // rebias 1023 -> 7
    return c > (uint32_t)kE4m3MaxCode ? (uint32_t)kE4m3MaxCode : c;
}

// Block-scale codes without the fp64 division.  thr2[c] (c = 0 .. 126) packs
// thr(c) | thr(c + 1) << 16, where thr(c) is the smallest bf16 magnitude
// (bits) whose code RNE_E4M3(a / (6 s_t)) is c or more (thr(0) = 0; thr(127)
// = 0xFFFF, above every finite magnitude).  The E4M3 midpoint between codes
// c - 1 and c, times 6 s_t, is exact in fp64 (at most 7 + 24 significant
// bits); at a tie the even code wins.  Built by threads 0 .. 126 of a block.
__device__ __forceinline__ uint32_t scale_threshold(uint32_t c, double six_st) {
    if (c == 0) return 0u;
    if (c > (uint32_t)kE4m3MaxCode) return 0xFFFFu;
    const double t = 0.5 * ((double)e4m3_value(c - 1) + (double)e4m3_value(c)) * six_st;
    const float f = (float)t;
    uint32_t fb = __float_as_uint(f);
    if ((double)f < t) fb += 1u;                          // smallest fp32 >= t
    uint32_t b = (fb + 0xFFFFu) >> 16;                    // smallest bf16 >= that
    if ((c & 1u) && (double)__uint_as_float(b << 16) == t) b += 1u;   // tie: even code
    return b > 0x7F80u ? 0xFFFFu : b;
}

__device__ __forceinline__ void build_scale_thresholds(float s_t, uint32_t* thr2) {
    const uint32_t c = threadIdx.x;
    if (c <= (uint32_t)kE4m3MaxCode) {
        const double six_st = 6.0 * (double)s_t;
        thr2[c] = scale_threshold(c, six_st) | (scale_threshold(c + 1u, six_st) << 16);
    }
}

// Block-scale code of a block with bf16 maximum magnitude `am` (bits), for a
// tensor scale s_t >= 2^-100 (inv6st = RN32(1 / (6 s_t))): the code of the
// fp32 quotient estimate (relative error under 2^-22, against a 1/16 relative
// spacing of the E4M3 midpoints, so at most one code off), then one compare
// with each threshold around it.
__device__ __forceinline__ uint32_t scale_code_thr(uint32_t am, float inv6st,
                                                   const uint32_t* thr2) {
    const float q = __uint_as_float(am << 16) * inv6st;
    uint32_t c;
    if (!(q < 448.0f)) {
        c = kE4m3MaxCode;
    } else if (q < 0x1p-6f) {
        c = (uint32_t)__builtin_rintf(q * 512.0f);              // subnormal codes 0 .. 8
    } else {
        const uint32_t b = __float_as_uint(q);
        c = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);   // rebias 127 -> 7
        c = c > (uint32_t)kE4m3MaxCode ? (uint32_t)kE4m3MaxCode : c;
    }
    const uint32_t pr = thr2[c];
    c += am >= (pr >> 16) ? 1u : 0u;
    c -= am < (pr & 0xFFFFu) ? 1u : 0u;
    return c;
}

// Value of the neighbouring lane (lane ^ 1), by a DPP quad permutation.
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

// Tensor scale s_t = RN32(A / 2688) for A = max|x| >= 0.  fp64 division then
// one fp32 rounding equals the exact RN32 for every bf16 and fp32 A here.
__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
    return (float)((double)amax / 2688.0);
}

// Largest fp32 <= t and smallest fp32 >= t, for t >= 0 (exact, via compares).
__device__ __forceinline__ uint32_t f32_bits_rd(double t) {
    float f = (float)t;
    uint32_t b = __float_as_uint(f);
    if ((double)f > t) b -= 1;
    return b;
}
__device__ __forceinline__ uint32_t f32_bits_ru(double t) {
    float f = (float)t;
    uint32_t b = __float_as_uint(f);
    if ((double)f < t) b += 1;
    return b;
}

// Element-code thresholds for one block scale.  E2M1 decision boundaries in
// units of s_b*s_t are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (midpoints of the
// grid).  thr[i] is an fp32 bit pattern such that, for |x| in fp32,
// magnitude code = #{ i : bits(|x|) > thr[i] } exactly: at boundary i the
// tie goes to the even code, so for even i the code rises when |x| > T_i
// (thr = RD32(T_i)) and for odd i when |x| >= T_i (thr = RU32(T_i) - 1 ulp).
// T_i = b_i * s_b * s_t is exact in fp64 (at most 31 significant bits).
// Non-negative fp32 bit patterns order like their values, so the compares are
// integer compares and independent of the denormal mode.
__device__ __forceinline__ void e2m1_thresholds(float s_b, float s_t, uint32_t thr[7]) {
    const float bnd[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    if (!(s_b > 0.0f) || !(s_t > 0.0f)) {
#pragma unroll
        for (int i = 0; i < 7; ++i) thr[i] = 0x7F800000u;   // never exceeded
        return;
    }
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        double t = (double)(bnd[i] * s_b) * (double)s_t;     // b_i*s_b exact in fp32
        thr[i] = (i & 1) ? f32_bits_ru(t) - 1u : f32_bits_rd(t);
    }
}

__device__ __forceinline__ uint32_t e2m1_mag_code(uint32_t abs_bits, const uint32_t thr[7]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) m += abs_bits > thr[i] ? 1u : 0u;
    return m;
}

// bf16 bit pattern nearest to d (ties to even), subnormals kept; |d| finite
// and below the bf16 overflow threshold.
__device__ __forceinline__ uint32_t bf16_rne_from_f64(double d) {
    uint64_t b = (uint64_t)__double_as_longlong(d);
    uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    uint64_t ab = b & 0x7FFFFFFFFFFFFFFFull;
    double a = __longlong_as_double((long long)ab);
    uint32_t out;
    if (a < 0x1p-126) {
        out = (uint32_t)rint(a * 0x1p133);
    } else {
        uint64_t r = (ab + 0xFFFFFFFFFFFull + ((ab >> 45) & 1ull)) >> 45;
        out = (uint32_t)(r - ((uint64_t)(1023 - 127) << 7));
    }
    return sign | out;
}

// bf16 nearest to an fp32 value (ties to even); finite inputs.
__device__ __forceinline__ uint32_t bf16_rne_from_f32(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Wave64 reductions.
// Maximum over the 64 lanes of a wave (every lane active), returned to all:
// DPP moves within each row of 16 lanes (quad permutations, then rotations
// by 4 and 8), then the four row maxima read as scalars -- no LDS round
// trips, unlike lane shuffles.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad 1,0,3,2
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad 2,3,0,1
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
    v = o > v ? o : v;
    const uint32_t a = __builtin_amdgcn_readlane(v, 15), b = __builtin_amdgcn_readlane(v, 31);
    const uint32_t c = __builtin_amdgcn_readlane(v, 47), d = __builtin_amdgcn_readlane(v, 63);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active), by
// DPP: shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the last
// lane of row 0 and 2 broadcast into rows 1 and 3, and of rows 0-1 into rows
// 2 and 3.
__device__ __forceinline__ int wave_incl_add(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    us2 r = __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b));
    return __builtin_bit_cast(uint32_t, r);
}

// Tensor scale of segment `seg` from its partial maxima (or the caller's fixed
// scale), computed by the whole work-group (sixteen partials per thread
// loaded together, as many rounds as `groups` needs) into *s_out (LDS; s_red
// holds one value per wave).
__device__ __forceinline__ void tensor_scale_prologue(const uint32_t* partial, int64_t groups,
                                                      const float* ts_in, int seg, float* s_out,
                                                      uint32_t* s_red) {
    const int nw = (blockDim.x + 63) >> 6;
    if (ts_in != nullptr) {
        if (threadIdx.x == 0) *s_out = ts_in[0];
        return;
    }
    const uint32_t* p = partial + (int64_t)seg * groups;
    uint32_t m = 0;
    for (int64_t b = 0; b < groups; b += 16 * (int64_t)blockDim.x) {
        uint32_t v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int64_t i = b + threadIdx.x + q * (int64_t)blockDim.x;
            v[q] = i < groups ? p[i] : 0u;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) m = v[q] > m ? v[q] : m;
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < nw; ++i) r = s_red[i] > r ? s_red[i] : r;
        *s_out = tensor_scale_from_amax(bf16_to_f32(r));
    }
}

// Per-tensor code table, one 32-byte row per block-scale code c = 0..126
// (row 127 unused): words 0..6 are the exact element-code thresholds of
// e2m1_thresholds, word 7 is the fast-path multiplier (fp32 bits) or
// kSlowPath.
//
// Fast path: for bf16 |x| in a block with scale code c, the hardware E2M1
// conversion of RN32(x * mul) (round to nearest even, saturating, sign kept)
// gives exactly the code the thresholds give, for every bf16 input.  Both
// RN32(a * mul) and the conversion are monotone in a, so it suffices that for
// each boundary i the largest bf16 value at or below threshold i converts to
// a code <= i and the smallest bf16 value above it to a code >= i + 1.  The
// table builder tries mul = RN32(1 / (s_b s_t)) and its neighbours up to two
// ulps away and checks exactly that, with the same instruction the kernels
// use, and that the largest finite bf16 gives code 7 (so that |x| * mul may
// overflow); codes where no candidate passes keep the exact compare path.
constexpr uint32_t kSlowPath = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t fast_code(float a, float mul) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a * mul, 0.0f, 1.0f, 0) & 0xFu;
}

__device__ __forceinline__ void build_table_row(int c, float s_t, bool allow_fast,
                                                uint32_t* row) {
    uint32_t thr[7];
    const float s_b = e4m3_value((uint32_t)c);
    e2m1_thresholds(s_b, s_t, thr);
    uint32_t mul = kSlowPath;
    if (!(s_b > 0.0f) || !(s_t > 0.0f)) {
        mul = 0u;                                   // every code is 0 (sign kept)
    } else if (allow_fast) {
        const float r0 = (float)(1.0 / ((double)s_b * (double)s_t));
        if (r0 > 0.0f && r0 < 3.0e38f) {
            const int offs[5] = {0, -1, 1, -2, 2};
            for (int q = 0; q < 5 && mul == kSlowPath; ++q) {
                const float r = __uint_as_float(__float_as_uint(r0) + offs[q]);
                // the largest finite bf16 must give code 7 too (x * mul may
                // overflow to inf under a caller-given tensor scale)
                bool ok = fast_code(__uint_as_float(0x7F7F0000u), r) == 7u;
                for (int i = 0; i < 7; ++i) {
                    const uint32_t lo = thr[i] & 0xFFFF0000u;   // largest bf16 <= threshold
                    const uint32_t hi = lo + 0x10000u;           // smallest bf16 above it
                    ok = ok && fast_code(__uint_as_float(lo), r) <= (uint32_t)i;
                    if (hi < 0x7F800000u)
                        ok = ok && fast_code(__uint_as_float(hi), r) >= (uint32_t)(i + 1);
                }
                if (ok) mul = __float_as_uint(r);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 7; ++i) row[i] = thr[i];
    row[7] = mul;
}

// Threshold table in LDS or global memory: s_thr[c][0..7] for c = 0..126.
__device__ __forceinline__ void build_threshold_table(float s_t, uint32_t (*s_thr)[8],
                                                      bool allow_fast = false) {
    for (int c = threadIdx.x; c <= kE4m3MaxCode; c += blockDim.x)
        build_table_row(c, s_t, allow_fast, s_thr[c]);
}

// 16 codes of one block (bf16 bits in w[8], two per word) with the table row
// of its scale: 8 packed bytes (even channel in the low nibble).
__device__ __forceinline__ uint2 encode_block_bf16(const uint32_t w[8], const uint4 t0,
                                                   const uint4 t1) {
    uint32_t packed[2] = {0u, 0u};
    if (t1.w != kSlowPath) {
        const float mul = __uint_as_float(t1.w);
#define QUADS_ENC_PAIR(e, sel)                                                           \
    packed[(e) >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(                          \
        packed[(e) >> 2], __uint_as_float(w[e] << 16) * mul,                              \
        __uint_as_float(w[e] & 0xFFFF0000u) * mul, 1.0f, sel)
        QUADS_ENC_PAIR(0, 0); QUADS_ENC_PAIR(1, 1); QUADS_ENC_PAIR(2, 2); QUADS_ENC_PAIR(3, 3);
        QUADS_ENC_PAIR(4, 0); QUADS_ENC_PAIR(5, 1); QUADS_ENC_PAIR(6, 2); QUADS_ENC_PAIR(7, 3);
#undef QUADS_ENC_PAIR
    } else {
        const uint32_t thr[7] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const uint32_t code = e2m1_mag_code((h & 0x7FFFu) << 16, thr) | ((h >> 12) & 8u);
            packed[e >> 3] |= code << (4 * (e & 7));
        }
    }
    return make_uint2(packed[0], packed[1]);
}

// Exact signed value v (E2M1, unscaled) of the 8 codes in one packed word.
__device__ __forceinline__ void decode8(uint32_t w, float v[8]) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
}

// ------------------------------------------------------------------ host --

#define QUADS_CHECK_LAUNCH()                                                  \
    do {                                                                      \
        hipError_t e__ = hipGetLastError();                                   \
        if (e__ != hipSuccess) return ::quads::set_hip_error(e__);            \
    } while (0)

int set_hip_error(hipError_t e);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
inline bool ok_opt_ptr(const void* p) { return p == nullptr || aligned16(p); }
// Arrays read and written one 32-bit word at a time.
inline bool ok_ptr4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launchers shared between translation units (defined in quantize.hip).
// Partial maxima of |x| over nseg contiguous segments of seg_elems elements
// each, `groups` values per segment into partial[seg * groups + g].
// The first segment's work-groups also zero clear[0 .. nclear).
void launch_amax_partial(const uint16_t* x, int64_t seg_elems, int nseg, uint32_t* partial,
                         int groups, hipStream_t s, uint32_t* clear = nullptr, int nclear = 0);
void launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// Tensor scale and code table per segment (1024 words of `table` each).
void launch_scale_finalize(const uint32_t* partial, int groups, const float* ts_in, int nseg,
                           float* ts_out, uint32_t* table, hipStream_t s);

// Number of work-groups of the partial-max pass for n elements.
inline int amax_groups(int64_t n) {
    int64_t g = (n + 8 * 256 * 8 - 1) / (8 * 256 * 8);   // >= 8 vectors of 8 per thread
    if (g < 1) g = 1;
    if (g > kAmaxGroups) g = kAmaxGroups;
    return (int)g;
}

// Direct HBM -> LDS loads (lane i's bytes land at LDS address m0 + i * size).
// Written as inline assembly so that the compiler does not see an LDS write:
// its conservative wait (every LDS read after such a load waits for it) would
// make each stage wait for the next stage's prefetch.  A kernel that uses them
// waits for its own loads explicitly (s_waitcnt vmcnt) before reading the
// bytes they bring.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(void* l) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)l);
}
// `l` is an LDS byte address (wave-uniform)
__device__ __forceinline__ void g2l16(const void* g, uint32_t l) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(g)
                 : "memory", "m0");
}
__device__ __forceinline__ void g2l4(const void* g, uint32_t l) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(l), "v"(g)
                 : "memory", "m0");
}

}  // namespace quads
