// MX block-scaled comparator: quantizer and grouped GEMM.
//
// The paper's rollout speed claim (arXiv 2607.15810, section 4.4.2 and
// Fig. 9(a)) is relative to FP8 W8A8 with fine-grained block scaling, where
// each tile of values carries its own scale (section 2.2, "FP8" paragraph).
// gfx950's block-scaled MFMA takes one power-of-two (E8M0) scale per 32
// consecutive elements of each operand row and applies it inside the
// instruction, so the comparator uses that layout (OCP MX): FP8 E4M3 or FP4
// E2M1 elements, E = floor(log2 max|x|) - emax per 32-element block (emax 8
// for E4M3, 2 for E2M1), elements x / 2^E rounded to nearest even and
// saturated.  Unlike the NVFP4 path, nothing is converted before the MFMA:
// the codes go from HBM to LDS with direct loads and from LDS to the matrix
// cores.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured on the
// device; lane l = 32 h + i holds row i, and its scale byte applies to the
// 32-element block h of the 64-deep step):
//   FP8: bytes 0-15 are k = 16 h .. 16 h + 15, bytes 16-31 are
//        k = 32 + 16 h .. 32 + 16 h + 15;
//   FP4: 32 codes (16 bytes) are k = 32 h .. 32 h + 31.
// Element j of lane (i, h) of one operand meets element j of lane (i', h) of
// the other.
#include "common.h"
#include "gemm_tiles.h"

namespace quads {
namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kMxBlock = 32;
constexpr int kFp8 = QUADS_MX_FP8;

// --------------------------------------------------------------- quantize --
// One lane per 16-element half block (two 16-byte bf16 loads); the block
// maximum is shared with the partner lane.  x * 2^-E is exact in fp32 (E is
// an integer power of two and values far below the element grid only need
// to round to zero); it is clamped to the largest finite element and
// converted by the hardware's round-to-nearest-even conversion, which keeps
// the sign of zero.
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits, int emax) {
    // floor(log2) of a non-negative bf16 bit pattern (0 for zero is unused)
    const int ef = (int)(amax_bits >> 7) & 0xFF;
    int fl;
    if (ef > 0) {
        fl = ef - 127;
    } else {                                   // subnormal: -133 + top mantissa bit
        const uint32_t m = amax_bits & 0x7F;
        fl = -133 + (31 - __builtin_clz(m | 1u));
    }
    int e = fl - emax;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    return amax_bits == 0 ? -127 : e;
}

template <int FMT>
__global__ __launch_bounds__(256) void k_mx_quantize(const uint16_t* __restrict__ x,
                                                     int64_t nhalf, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
    constexpr int emax = FMT == kFp8 ? 8 : 2;
    constexpr float vmax = FMT == kFp8 ? 448.0f : 6.0f;
    const int64_t stride = (int64_t)gridDim.x * 256;
    // nhalf is even (K % 32 == 0), so partner lanes are both in or both out
    for (int64_t h0 = (int64_t)blockIdx.x * 256; h0 < nhalf; h0 += stride) {
        const int64_t h = h0 + threadIdx.x;
        const bool live = h < nhalf;
        uint4 q0 = make_uint4(0, 0, 0, 0), q1 = q0;
        if (live) {
            const uint4* p = reinterpret_cast<const uint4*>(x + h * 16);
            q0 = ld_stream16(p);
            q1 = ld_stream16(p + 1);
        }
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = pk_max_u16(am, w[i] & 0x7FFF7FFFu);
        uint32_t a = (am & 0xFFFFu) > (am >> 16) ? (am & 0xFFFFu) : (am >> 16);
        const uint32_t o = __shfl_xor(a, 1, 64);
        a = o > a ? o : a;
        const int e = mx_exponent(a, emax);
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float xv = __uint_as_float(i & 1 ? w[i >> 1] & 0xFFFF0000u : w[i >> 1] << 16);
            const float s = __builtin_ldexpf(xv, -e);
            v[i] = __builtin_fminf(__builtin_fmaxf(s, -vmax), vmax);
        }
        if (FMT == kFp8) {
            uint32_t out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i], v[4 * i + 1], 0, false);
                r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2], v[4 * i + 3], r, true);
                out[i] = (uint32_t)r;
            }
            if (live)
                *reinterpret_cast<uint4*>(codes + h * 16) = make_uint4(out[0], out[1], out[2], out[3]);
        } else {
            uint32_t out[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float* u = v + 8 * i;
                uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, u[0], u[1], 1.0f, 0);
                r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, u[2], u[3], 1.0f, 1);
                r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, u[4], u[5], 1.0f, 2);
                out[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, u[6], u[7], 1.0f, 3);
            }
            if (live) *reinterpret_cast<uint2*>(codes + h * 8) = make_uint2(out[0], out[1]);
        }
        if (live && (h & 1) == 0) scales[h >> 1] = (uint8_t)(e + 127);
    }
}

// -------------------------------------------------------------------- gemm --
// 256 x 256 output tile, 8 waves (2 x 4) of 128 x 64, K staged 128 at a time
// through two LDS buffers: per stage the A and W code tiles (256 rows x 128
// bytes for FP8, x 64 for FP4) and their scale bytes (4 per row).  Every
// byte reaches LDS with global_load_lds (16 bytes per lane for codes, 4 for
// scales): no registers, no conversion.  The code rows are swizzled by
// 16-byte chunk (FP8: chunk c of row r at c ^ ((r >> 1) & 7); FP4: at
// c ^ ((r >> 2) & 3)), so each 16-lane group of a fragment read hits 64
// distinct banks; the loader lanes fetch the global chunk that belongs at
// their LDS slot.  Weights are the first MFMA operand, as in the NVFP4 GEMM,
// so the accumulators and the epilogue are the same.
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 512;

template <int FMT>
struct Cfg {
    static constexpr int kRowBytes = FMT == kFp8 ? 128 : 64;    // per row per stage
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kTile = 256 * kRowBytes;                // one operand, one stage
    static constexpr int kStage = 2 * kTile + 2 * 256 * 4;       // + A and W scales
    static constexpr int kLoads = 256 * kChunks / kThreads;      // 16-byte loads per operand
};

template <int FMT>
__device__ __forceinline__ int lds_pos(int r, int c) {
    return FMT == kFp8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
}

struct MxArgs {
    const uint8_t* a; const uint8_t* as; const int32_t* row_token; int64_t rows; int K;
    const uint8_t* w; const uint8_t* ws; const int32_t* offsets; int E; int N;
    int epilogue; int out_bf16; void* out;
    // compensation (RAC on the MX FP4 mode): the second pass of the residual
    // on the selected channels (MX FP4 [Ta, k/2] codes, [Ta, k/32] scales),
    // and W[:, S] of every weight row as exact bf16 values [E * N, k]
    const uint8_t* r_codes; const uint8_t* r_scales; int k; const __bf16* w_sel;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Loads of stage s into LDS buffer `buf`: code tiles (kLoads 16-byte loads per
// operand per thread) and scale rows (one 4-byte load per thread: waves 0-3
// take A rows 64 w .., waves 4-7 W rows).
template <int FMT>
__device__ __forceinline__ void load_stage(const MxArgs& g, uint32_t buf, int s,
                                           const int32_t a_row[], const int64_t w_row[],
                                           int64_t sc_row, bool sc_is_a) {
    using C = Cfg<FMT>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t a_len = FMT == kFp8 ? g.K : g.K / 2;           // bytes per code row
#pragma unroll
    for (int q = 0; q < C::kLoads; ++q) {
        const int slot = (q * 8 + wave) * 64 + lane;
        const int r = slot / C::kChunks, pos = slot % C::kChunks;
        const int c = lds_pos<FMT>(r, pos);                       // involution
        const int64_t off = (int64_t)s * C::kRowBytes + 16 * c;
        const uint32_t dst_a = buf + (q * 8 + wave) * 64 * 16;
        g2l16(g.a + (int64_t)a_row[q] * a_len + off, dst_a);
        g2l16(g.w + w_row[q] * a_len + off, dst_a + C::kTile);
    }
    const uint8_t* sc = (sc_is_a ? g.as : g.ws) + sc_row * (g.K / kMxBlock) + 4 * s;
    g2l4(sc, buf + 2 * C::kTile + (wave >> 2) * 1024 + (wave & 3) * 256);
}

// One 64-deep step t (0 or 1) of a stage for the wave's first MACT row blocks.
template <int FMT, int MACT>
__device__ __forceinline__ void mma_step(const uint8_t* buf, int t, int wm, int wn,
                                         const uint32_t sa_w[4], const uint32_t sw_w[2],
                                         f32x16 acc[4][2]) {
    using C = Cfg<FMT>;
    if (MACT == 0) return;
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    v8i a[4], b[2];
    auto frag = [&](int row) {
        const uint8_t* base = buf + row * C::kRowBytes;
        v8i f;
        if (FMT == kFp8) {
            const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * lds_pos<FMT>(row, 4 * t + h));
            const uint4 hi =
                *reinterpret_cast<const uint4*>(base + 16 * lds_pos<FMT>(row, 4 * t + 2 + h));
            f = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
            const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * lds_pos<FMT>(row, 2 * t + h));
            f = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        }
        return f;
    };
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) b[nj] = frag(BM + wn * 64 + nj * 32 + r);
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi) a[mi] = frag(wm * 128 + mi * 32 + r);
    const int sh = 8 * (2 * t + h);
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            acc[mi][nj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                b[nj], a[mi], acc[mi][nj], FMT, FMT, 0, (int)((sw_w[nj] >> sh) & 0xFFu), 0,
                (int)((sa_w[mi] >> sh) & 0xFFu));
}

template <int FMT, int MACT>
__device__ __forceinline__ void main_loop(const MxArgs& g, uint8_t* smem, const int32_t a_row[],
                                          const int64_t w_row[], int64_t sc_row, bool sc_is_a,
                                          int wm, int wn, f32x16 acc[4][2]) {
    using C = Cfg<FMT>;
    const int ns = g.K / BK;
    const int r = threadIdx.x & 31;
    const uint32_t smem_lds = lds_addr(smem);
    load_stage<FMT>(g, smem_lds, 0, a_row, w_row, sc_row, sc_is_a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = 0; s < ns; ++s) {
        uint8_t* cur = smem + (s & 1) * C::kStage;
        if (s + 1 < ns)
            load_stage<FMT>(g, smem_lds + ((s + 1) & 1) * C::kStage, s + 1, a_row, w_row, sc_row,
                            sc_is_a);
        const uint32_t* sca = reinterpret_cast<const uint32_t*>(cur + 2 * C::kTile);
        uint32_t sa_w[4], sw_w[2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) sa_w[mi] = mi < MACT ? sca[wm * 128 + mi * 32 + r] : 0u;
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) sw_w[nj] = sca[256 + wn * 64 + nj * 32 + r];
        mma_step<FMT, MACT>(cur, 0, wm, wn, sa_w, sw_w, acc);
        mma_step<FMT, MACT>(cur, 1, wm, wn, sa_w, sw_w, acc);
        __builtin_amdgcn_s_waitcnt(0);        // this thread's loads of stage s + 1 landed
        __syncthreads();
    }
}

// 8 MX FP4 codes (one dword) of a block with scale byte sb as exact bf16
// values: the unscaled E2M1 values times 2^(sb - 127), exact in fp32 (at
// least 2^-128) and in bf16.
__device__ __forceinline__ bf16x8 mx_fp4_bf16x8(uint32_t w, uint32_t sb) {
    const float sc = ldexpf(1.0f, (int)sb - 127);
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    return (bf16x8){(__bf16)(f0[0] * sc), (__bf16)(f0[1] * sc), (__bf16)(f1[0] * sc),
                    (__bf16)(f1[1] * sc), (__bf16)(f2[0] * sc), (__bf16)(f2[1] * sc),
                    (__bf16)(f3[0] * sc), (__bf16)(f3[1] * sc)};
}

// W[:, S] of every weight row as exact bf16 values [E * N, k]: a thread
// writes 8 consecutive selected channels of one row.
__global__ __launch_bounds__(256) void k_mx_gather_wsel(const uint8_t* __restrict__ w,
                                                        const uint8_t* __restrict__ ws,
                                                        const int32_t* __restrict__ sel, int K,
                                                        int k, int64_t nrows,
                                                        __bf16* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_row = k / 8;
    if (t >= nrows * per_row) return;
    const int64_t row = t / per_row;
    const int j0 = (int)(t - row * per_row) * 8;
    const uint8_t* crow = w + row * (K / 2);
    const uint8_t* srow = ws + row * (K / kMxBlock);
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int c = sel[j0 + i];
        c = c < 0 ? 0 : (c >= K ? K - 1 : c);                 // bounds only: sel < K
        const uint32_t code = (crow[c >> 1] >> (4 * (c & 1))) & 15u;
        v[i] = mx_fp4_bf16x8(code, srow[c / kMxBlock])[0];
    }
    *reinterpret_cast<bf16x8*>(out + row * k + j0) = v;
}

// The compensation R x W[:, S] of the wave's output blocks, in bf16 MFMAs
// (32x32x16, the same accumulator layout as the block-scaled MFMA): lane
// (i, h) holds channels 16 t + 8 h .. + 7 of row i of both operands.
template <int kEpi>
__device__ __forceinline__ void mx_compensation(const MxArgs& g, int e, int m0, int mend, int f0,
                                                int wm, int wn, int mact, f32x16 acc[4][2]) {
    constexpr bool swiglu = kEpi == QUADS_EPI_SWIGLU;
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    int64_t wrow[2];
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) {
        bool ok;
        const int wr = v2::w_row_v2(wn * 64 + nj * 32 + r, f0, g.N, swiglu, &ok);
        wrow[nj] = (int64_t)e * g.N + (ok ? wr : 0);
    }
    int64_t arow[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int p = m0 + wm * 128 + mi * 32 + r;
        arow[mi] = p < mend ? (g.row_token ? (int64_t)g.row_token[p] : (int64_t)p) : 0;
    }
    for (int t = 0; t < g.k / 16; ++t) {
        const int ch = 16 * t + 8 * h;
        bf16x8 b[2];
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            b[nj] = *reinterpret_cast<const bf16x8*>(g.w_sel + wrow[nj] * g.k + ch);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= mact) break;
            const uint32_t code =
                *reinterpret_cast<const uint32_t*>(g.r_codes + arow[mi] * (g.k / 2) + ch / 2);
            const bf16x8 a = mx_fp4_bf16x8(code, g.r_scales[arow[mi] * (g.k / kMxBlock) +
                                                            ch / kMxBlock]);
#pragma unroll
            for (int nj = 0; nj < 2; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nj], a, acc[mi][nj], 0, 0, 0);
        }
    }
}

template <int FMT, int kEpi, bool kComp = false>
__global__ __launch_bounds__(kThreads) void k_mx_gemm(MxArgs g, int nt_n, int grp) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Cfg<FMT>::kStage];
    const int hid = blockIdx.x;
    const int slot = hid / v2::kXcds;
    const int tile = (slot / grp) * (v2::kXcds * grp) + (hid % v2::kXcds) * grp + slot % grp;
    const int tile_m = tile / nt_n, tile_n = tile - tile_m * nt_n;
    int e, m0, mend;
    if (!v2::find_tile_wave<BM>(g.offsets, g.E, g.rows, tile_m, &e, &m0, &mend)) return;
    constexpr bool swiglu = kEpi == QUADS_EPI_SWIGLU;
    const int f0 = tile_n * (swiglu ? BN / 2 : BN);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    int mact = (mend - (m0 + wm * 128) + 31) / 32;
    mact = __builtin_amdgcn_readfirstlane(mact < 0 ? 0 : (mact > 4 ? 4 : mact));

    // rows this thread loads: A rows (through row_token), W rows of the tile
    using C = Cfg<FMT>;
    auto a_src = [&](int r) {
        const int p = m0 + r;
        return p < mend ? (g.row_token ? g.row_token[p] : p) : 0;
    };
    auto w_src = [&](int r) {
        bool ok;
        const int wr = v2::w_row_v2(r, f0, g.N, swiglu, &ok);
        return (int64_t)e * g.N + (ok ? wr : 0);
    };
    int32_t a_row[C::kLoads];
    int64_t w_row[C::kLoads];
#pragma unroll
    for (int q = 0; q < C::kLoads; ++q) {
        const int r = ((q * 8 + wave) * 64 + lane) / C::kChunks;
        a_row[q] = a_src(r);
        w_row[q] = w_src(r);
    }
    const int sr = (wave & 3) * 64 + lane;                      // scale row in its tile
    const bool sc_is_a = wave < 4;
    const int64_t sc_row = sc_is_a ? (int64_t)a_src(sr) : w_src(sr);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    switch (mact) {
        case 4: main_loop<FMT, 4>(g, smem, a_row, w_row, sc_row, sc_is_a, wm, wn, acc); break;
        case 3: main_loop<FMT, 3>(g, smem, a_row, w_row, sc_row, sc_is_a, wm, wn, acc); break;
        case 2: main_loop<FMT, 2>(g, smem, a_row, w_row, sc_row, sc_is_a, wm, wn, acc); break;
        case 1: main_loop<FMT, 1>(g, smem, a_row, w_row, sc_row, sc_is_a, wm, wn, acc); break;
        default: main_loop<FMT, 0>(g, smem, a_row, w_row, sc_row, sc_is_a, wm, wn, acc); break;
    }
    if (kComp && g.k > 0 && mact > 0) mx_compensation<kEpi>(g, e, m0, mend, f0, wm, wn, mact, acc);
    GemmArgs ga{};
    ga.N = g.N;
    ga.out = g.out;
    ga.out_bf16 = g.out_bf16;
    v2::epilogue<kEpi>(ga, acc, 1.0f, m0, mend, f0, wm, wn, mact, lane);
}

}  // namespace mx
}  // namespace quads

using namespace quads;

extern "C" int quads_mx_quantize(const uint16_t* x, int64_t M, int64_t K, int fmt,
                                 uint8_t* codes, uint8_t* scales, void* stream) {
    if (fmt != QUADS_MX_FP8 && fmt != QUADS_MX_FP4) return QUADS_EINVAL;
    if (M < 0 || K <= 0 || K % mx::kMxBlock || M >= ((int64_t)1 << 40)) return QUADS_ESHAPE;
    if (M == 0) return QUADS_OK;
    if (!ok_ptr(x) || !ok_ptr(codes) || !ok_ptr(scales)) return QUADS_EINVAL;
    const int64_t nhalf = M * K / 16;
    int64_t grid = (nhalf + 255) / 256;
    if (grid > 8192) grid = 8192;
    hipStream_t s = (hipStream_t)stream;
    if (fmt == QUADS_MX_FP8)
        hipLaunchKernelGGL(mx::k_mx_quantize<QUADS_MX_FP8>, dim3((unsigned)grid), dim3(256), 0, s,
                           x, nhalf, codes, scales);
    else
        hipLaunchKernelGGL(mx::k_mx_quantize<QUADS_MX_FP4>, dim3((unsigned)grid), dim3(256), 0, s,
                           x, nhalf, codes, scales);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}

template <int FMT, bool kComp = false>
static void launch_mx_gemm(const mx::MxArgs& g, int epilogue, dim3 grid, int nt_n, int grp,
                           hipStream_t s) {
    if (epilogue == QUADS_EPI_SWIGLU)
        hipLaunchKernelGGL((mx::k_mx_gemm<FMT, QUADS_EPI_SWIGLU, kComp>), grid, dim3(mx::kThreads),
                           0, s, g, nt_n, grp);
    else
        hipLaunchKernelGGL((mx::k_mx_gemm<FMT, QUADS_EPI_NONE, kComp>), grid, dim3(mx::kThreads), 0,
                           s, g, nt_n, grp);
}

extern "C" int quads_moe_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scale,
                                 const int32_t* row_token, int64_t rows, int64_t K,
                                 const uint8_t* w_codes, const uint8_t* w_scale,
                                 const int32_t* offsets, int32_t E, int64_t N, int fmt,
                                 int epilogue, int out_dtype, void* out, void* stream) {
    if (fmt != QUADS_MX_FP8 && fmt != QUADS_MX_FP4) return QUADS_EINVAL;
    if (epilogue != QUADS_EPI_NONE && epilogue != QUADS_EPI_SWIGLU) return QUADS_EINVAL;
    if (out_dtype != QUADS_OUT_F32 && out_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (epilogue == QUADS_EPI_SWIGLU && out_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (rows < 0 || rows >= ((int64_t)1 << 31) || K <= 0 || K % mx::BK || K >= ((int64_t)1 << 30))
        return QUADS_ESHAPE;
    if (E < 1 || E > 4096 || N < 1 || N >= ((int64_t)1 << 30)) return QUADS_ESHAPE;
    if (epilogue == QUADS_EPI_SWIGLU && N % 2) return QUADS_ESHAPE;
    if (offsets == nullptr && E != 1) return QUADS_EINVAL;
    if (rows == 0) return QUADS_OK;                   // size 0: a no-op, whatever the pointers
    if (!ok_opt_ptr(offsets) || !ok_opt_ptr(row_token)) return QUADS_EINVAL;
    if (!ok_ptr(a_codes) || !ok_ptr(a_scale) || !ok_ptr(w_codes) || !ok_ptr(w_scale) ||
        !ok_ptr(out))
        return QUADS_EINVAL;
    mx::MxArgs g{a_codes, a_scale, row_token, rows, (int)K, w_codes, w_scale, offsets, (int)E,
                 (int)N, epilogue, out_dtype == QUADS_OUT_BF16, out};
    const int64_t nt_n = epilogue == QUADS_EPI_SWIGLU ? (N / 2 + mx::BN / 2 - 1) / (mx::BN / 2)
                                                      : (N + mx::BN - 1) / mx::BN;
    const int64_t nt_m = (rows + mx::BM - 1) / mx::BM + (offsets ? E : 0);
    const int64_t grp = 2 * nt_n;
    const int64_t span = grp * v2::kXcds;
    const dim3 grid((unsigned)((nt_m * nt_n + span - 1) / span * span));
    hipStream_t s = (hipStream_t)stream;
    if (fmt == QUADS_MX_FP8)
        launch_mx_gemm<QUADS_MX_FP8>(g, epilogue, grid, (int)nt_n, (int)grp, s);
    else
        launch_mx_gemm<QUADS_MX_FP4>(g, epilogue, grid, (int)nt_n, (int)grp, s);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}

// RAC on the MX FP4 mode: the MX FP4 grouped GEMM plus the compensation term
// over the selected channels.  Workspace: W[:, S] as bf16, E * N * k * 2
// bytes.
extern "C" size_t quads_moe_mx_rac_gemm_ws(int32_t E, int64_t N, int32_t k) {
    if (E < 1 || N < 1 || k < 0) return 0;
    return align_up((size_t)E * (size_t)N * (size_t)k * 2, 256);
}

extern "C" int quads_moe_mx_rac_gemm(const uint8_t* a_codes, const uint8_t* a_scale,
                                     const int32_t* row_token, int64_t rows, int64_t K,
                                     const uint8_t* r_codes, const uint8_t* r_scale,
                                     const int32_t* sel, int32_t k, const uint8_t* w_codes,
                                     const uint8_t* w_scale, const int32_t* offsets, int32_t E,
                                     int64_t N, int epilogue, int out_dtype, void* out, void* ws,
                                     size_t ws_bytes, void* stream) {
    if (k < 0 || k % 32 || k > K) return QUADS_ESHAPE;
    if (rows > 0 && k > 0 && (!ok_ptr(r_codes) || !ok_ptr(r_scale) || !ok_ptr(sel)))
        return QUADS_EINVAL;
    if (k == 0)
        return quads_moe_mx_gemm(a_codes, a_scale, row_token, rows, K, w_codes, w_scale, offsets,
                                 E, N, QUADS_MX_FP4, epilogue, out_dtype, out, stream);
    if (epilogue != QUADS_EPI_NONE && epilogue != QUADS_EPI_SWIGLU) return QUADS_EINVAL;
    if (out_dtype != QUADS_OUT_F32 && out_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (epilogue == QUADS_EPI_SWIGLU && out_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (rows < 0 || rows >= ((int64_t)1 << 31) || K <= 0 || K % mx::BK || K >= ((int64_t)1 << 30))
        return QUADS_ESHAPE;
    if (E < 1 || E > 4096 || N < 1 || N >= ((int64_t)1 << 30)) return QUADS_ESHAPE;
    if (epilogue == QUADS_EPI_SWIGLU && N % 2) return QUADS_ESHAPE;
    if (offsets == nullptr && E != 1) return QUADS_EINVAL;
    if (rows == 0) return QUADS_OK;                   // size 0: a no-op, whatever the pointers
    if (!ok_opt_ptr(offsets) || !ok_opt_ptr(row_token)) return QUADS_EINVAL;
    if (!ok_ptr(a_codes) || !ok_ptr(a_scale) || !ok_ptr(w_codes) || !ok_ptr(w_scale) ||
        !ok_ptr(out))
        return QUADS_EINVAL;
    if (ws_bytes < quads_moe_mx_rac_gemm_ws(E, N, k) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int64_t nrows = (int64_t)E * N, threads = nrows * (k / 8);
    hipLaunchKernelGGL(mx::k_mx_gather_wsel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       w_codes, w_scale, sel, (int)K, (int)k, nrows, static_cast<__bf16*>(ws));
    QUADS_CHECK_LAUNCH();
    mx::MxArgs g{a_codes, a_scale, row_token, rows, (int)K, w_codes, w_scale, offsets, (int)E,
                 (int)N, epilogue, out_dtype == QUADS_OUT_BF16, out, r_codes, r_scale, (int)k,
                 static_cast<const __bf16*>(ws)};
    const int64_t nt_n = epilogue == QUADS_EPI_SWIGLU ? (N / 2 + mx::BN / 2 - 1) / (mx::BN / 2)
                                                      : (N + mx::BN - 1) / mx::BN;
    const int64_t nt_m = (rows + mx::BM - 1) / mx::BM + (offsets ? E : 0);
    const int64_t grp = 2 * nt_n;
    const int64_t span = grp * v2::kXcds;
    const dim3 grid((unsigned)((nt_m * nt_n + span - 1) / span * span));
    launch_mx_gemm<QUADS_MX_FP4, true>(g, epilogue, grid, (int)nt_n, (int)grp, s);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}
