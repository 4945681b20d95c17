// Grouped W4A4 GEMM with the RAC compensation term (arXiv 2607.15810, Eq. (6)
// applied to the compensated activation of Eq. (21)), for MoE experts.
//
// MFMA operand type.  An NVFP4 value v * s_b (E2M1 times an E4M3 block scale)
// has at most 6 significant bits and magnitude in [2^-10, 2688], so it is
// exact in fp16; products of two are exact in fp32.  The kernel therefore
// dequantizes both operands exactly to fp16 and issues 32x32x16 fp16 MFMA
// with fp32 accumulation; the fp32 tensor scales are applied in the epilogue.
// gfx950's block-scaled fp4 MFMA takes one power-of-two scale per 32
// elements, which cannot express E4M3 scales over 16 elements exactly.
//
// Two kernels.  When K and k are multiples of 64 (every workload here), the
// 256 x 256-tile kernel in namespace v2 below runs; its comment describes it.
// Otherwise a plain 128 x 128-tile kernel does: 256 threads, K staged 64 at a
// time; each thread dequantizes 32 codes of one A row and one W row to fp16
// (hardware fp4 -> fp16 convert, then a packed fp16 multiply by the block
// scale) into LDS, and four waves (2 x 2) each own a 64 x 64 sub-tile.
//
// Compensation in the 128 x 128 kernel: after the main K loop the same tile
// runs a second, short loop over the k selected channels: A = the
// second-pass residual codes, B = the weight columns sel[i] gathered per row.
// It accumulates into its own fp32 registers because its tensor scale
// differs; the epilogue forms
//   Y = acc_main * (s_tA s_tW[e]) + acc_comp * (s_tR s_tW[e]).
#include "common.h"
#include "gemm_tiles.h"

namespace quads {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLd = kBK + 8;           // halfs per LDS row (16-byte pad)
constexpr int kGemmMaxE = 4096;


// (expert, first row, end row) of M-tile `tile`: experts' rows are cut into
// tiles of kBM; tiles are numbered expert by expert.  Returns false (for the
// whole work-group) when `tile` is past the last tile.
__device__ bool find_tile_bm(const int32_t* offsets, int E, int64_t rows, int tile, int bm,
                             int* s_scan, int* s_res, int* e_out, int* m0_out, int* mend_out,
                             int skip) {
    if (offsets == nullptr) {                      // one expert, all rows
        const int64_t m0 = (int64_t)tile * bm;
        *e_out = 0;
        *m0_out = (int)m0;
        *mend_out = (int)rows;
        return m0 < rows;
    }
    const int nthr = blockDim.x;
    const int per = (E + nthr - 1) / nthr;
    const int e0 = threadIdx.x * per;
    const int e1 = e0 + per < E ? e0 + per : E;
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (v2::rows_of(offsets, e, skip, 0) + bm - 1) / bm;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = local;
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_scan[wid] = x;
    if (threadIdx.x == 0) s_res[3] = 0;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wid; ++i) base += s_scan[i];
    int run = x - local + base;
    for (int e = e0; e < e1; ++e) {
        const int t = (v2::rows_of(offsets, e, skip, 0) + bm - 1) / bm;
        if (tile >= run && tile < run + t) {     // exactly one thread matches
            s_res[0] = e;
            s_res[1] = offsets[e] + (tile - run) * bm;
            s_res[2] = offsets[e + 1];
            s_res[3] = 1;
        }
        run += t;
    }
    __syncthreads();
    *e_out = s_res[0];
    *m0_out = s_res[1];
    *mend_out = s_res[2];
    return s_res[3] != 0;
}

// 16 fp4 codes (8 bytes) times an E4M3 block scale -> 16 exact fp16 values.
__device__ __forceinline__ void dequant16(uint2 q, uint32_t sbyte, f16x8* lo, f16x8* hi) {
    const _Float16 sb = (_Float16)e4m3_value(sbyte);
    const f16x2 s2 = {sb, sb};
    const uint32_t w[2] = {q.x, q.y};
    f16x2 v[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        v[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0) * s2;
        v[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1) * s2;
        v[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2) * s2;
        v[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3) * s2;
    }
    *lo = (f16x8){v[0][0], v[0][1], v[1][0], v[1][1], v[2][0], v[2][1], v[3][0], v[3][1]};
    *hi = (f16x8){v[4][0], v[4][1], v[5][0], v[5][1], v[6][0], v[6][1], v[7][0], v[7][1]};
}

// Load and dequantize 32 consecutive codes (two blocks) of one row starting at
// channel kc (a multiple of 16); channels >= kend read as zero.
__device__ __forceinline__ void load_row32(const uint8_t* nib_row, const uint8_t* sc_row, int kc,
                                           int kend, bool valid, f16x8 out[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = kc + 16 * j;
        if (valid && c < kend) {
            const uint2 q = *reinterpret_cast<const uint2*>(nib_row + c / 2);
            dequant16(q, sc_row[c / 16], &out[2 * j], &out[2 * j + 1]);
        } else {
            out[2 * j] = (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
            out[2 * j + 1] = out[2 * j];
        }
    }
}

__device__ __forceinline__ void store_lds32(_Float16* dst, const f16x8 v[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f16x8*>(dst + 8 * i) = v[i];
}

__device__ __forceinline__ void mma_stage(const _Float16* sA, const _Float16* sB, int wm, int wn,
                                          int lane, f32x16 acc[2][2]) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
        const int kof = kk * 16 + 8 * (lane >> 5);
        f16x8 a[2], b[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            a[mi] = *reinterpret_cast<const f16x8*>(sA + (wm * 64 + mi * 32 + (lane & 31)) * kLd + kof);
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            b[nj] = *reinterpret_cast<const f16x8*>(sB + (wn * 64 + nj * 32 + (lane & 31)) * kLd + kof);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nj = 0; nj < 2; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mi], b[nj], acc[mi][nj], 0, 0, 0);
    }
}

// Weight row of B-tile row r.  Plain: f0 + r.  SwiGLU: the tile holds 64
// output features; rows 0-31 / 32-63 of each 64-row half are gate / up.
__device__ __forceinline__ int w_row_of(int r, int f0, int N, bool swiglu, bool* valid) {
    if (!swiglu) {
        const int n = f0 + r;
        *valid = n < N;
        return n;
    }
    const int feat = f0 + (r >> 6) * 32 + (r & 31);
    *valid = feat < N / 2;
    return ((r >> 5) & 1) * (N / 2) + feat;
}

template <int kEpi>
__global__ __launch_bounds__(256) void k_gemm_w4a4(GemmArgs g) {
    __shared__ _Float16 sA[kBM * kLd];
    __shared__ _Float16 sB[kBN * kLd];
    __shared__ int s_scan[8];
    __shared__ int s_res[4];
    int e, m0, mend;
    if (!find_tile_bm(g.offsets, g.E, g.rows, blockIdx.y, kBM, s_scan, s_res, &e, &m0, &mend,
                      g.dec_rows)) {
        if (g.amax) amax_group_none(g);
        return;
    }
    bind_expert(g, e);
    constexpr bool swiglu = kEpi == QUADS_EPI_SWIGLU;
    const int f0 = blockIdx.x * (swiglu ? kBN / 2 : kBN);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = tid >> 1, lh = tid & 1;           // loader: tile row, 32-channel half

    // A row of this thread's loader slot
    const int p = m0 + lr;
    const bool a_valid = p < mend;
    const int64_t src = a_valid ? (g.row_token ? (int64_t)g.row_token[p] : (int64_t)p) : 0;
    const uint8_t* a_nib_row = g.a_nib + src * (g.K / 2);
    const uint8_t* a_sc_row = g.a_scale + src * (g.K / kBlock);
    bool b_valid;
    const int wrow = w_row_of(lr, f0, g.N, swiglu, &b_valid);
    const int64_t wbase = ((int64_t)e * g.N + (b_valid ? wrow : 0));
    const uint8_t* w_nib_row = g.w_nib + wbase * (g.K / 2);
    const uint8_t* w_sc_row = g.w_scale + wbase * (g.K / kBlock);

    // acc / accc: the MFMA chains of the main product and the compensation,
    // restarted every kAccChain channels into the fp32 totals tot / totc
    f32x16 acc[2][2], accc[2][2], tot[2][2], totc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc[i][j][v] = 0.f; accc[i][j][v] = 0.f; tot[i][j][v] = 0.f; totc[i][j][v] = 0.f;
            }
    auto flush = [](f32x16 (&a)[2][2], f32x16 (&t)[2][2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) { t[i][j][v] += a[i][j][v]; a[i][j][v] = 0.f; }
    };

    for (int k0 = 0; k0 < g.K; k0 += kBK) {
        f16x8 va[4], vb[4];
        load_row32(a_nib_row, a_sc_row, k0 + 32 * lh, g.K, a_valid, va);
        load_row32(w_nib_row, w_sc_row, k0 + 32 * lh, g.K, b_valid, vb);
        __syncthreads();
        store_lds32(sA + lr * kLd + 32 * lh, va);
        store_lds32(sB + lr * kLd + 32 * lh, vb);
        __syncthreads();
        mma_stage(sA, sB, wm, wn, lane, acc);
        if ((k0 + kBK) % kAccChain == 0 || k0 + kBK >= g.K) flush(acc, tot);
    }

    if (g.k > 0) {
        const uint8_t* r_nib_row = g.r_nib + src * (g.k / 2);
        const uint8_t* r_sc_row = g.r_scale + src * (g.k / kBlock);
        for (int i0 = 0; i0 < g.k; i0 += kBK) {
            f16x8 va[4], vb[4];
            load_row32(r_nib_row, r_sc_row, i0 + 32 * lh, g.k, a_valid, va);
            // gathered weight columns sel[i] of row wrow
            _Float16 h[32];
#pragma unroll 4
            for (int u = 0; u < 32; ++u) {
                const int i = i0 + 32 * lh + u;
                float v = 0.0f;
                if (b_valid && i < g.k) {
                    int j = g.sel[i];
                    j = j < 0 ? 0 : (j >= g.K ? g.K - 1 : j);   // bounds only
                    const uint32_t code = (w_nib_row[j >> 1] >> (4 * (j & 1))) & 0xFu;
                    v = e2m1_value(code & 7u) * e4m3_value(w_sc_row[j >> 4]);
                    if (code & 8u) v = -v;
                }
                h[u] = (_Float16)v;                  // exact
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                vb[q] = (f16x8){h[8 * q], h[8 * q + 1], h[8 * q + 2], h[8 * q + 3], h[8 * q + 4],
                                h[8 * q + 5], h[8 * q + 6], h[8 * q + 7]};
            __syncthreads();
            store_lds32(sA + lr * kLd + 32 * lh, va);
            store_lds32(sB + lr * kLd + 32 * lh, vb);
            __syncthreads();
            mma_stage(sA, sB, wm, wn, lane, accc);
            if ((i0 + kBK) % kAccChain == 0 || i0 + kBK >= g.k) flush(accc, totc);
        }
    }

    // epilogue
    const float s_ta = tensor_scale_a(g), s_tw = g.w_ts[e];
    const float ca = s_ta * s_tw;
    const float cr = g.k > 0 ? g.r_ts[0] * s_tw : 0.0f;
    uint32_t hmax = 0;                               // largest |h| stored (SwiGLU)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row_t = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int prow = m0 + row_t;
            if (prow >= mend) continue;
            const float ca_row = row_scale(g, prow, ca);
            float y[2];
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) {
                y[nj] = tot[mi][nj][v] * ca_row;
                if (g.k > 0) y[nj] = fmaf(totc[mi][nj][v], cr, y[nj]);
            }
            if (swiglu) {
                const int feat = f0 + wn * 32 + (lane & 31);
                if (feat < g.N / 2) {
                    const float gt = y[0], up = y[1];
                    const float hval = silu_mul(gt, up);
                    const uint32_t hb = bf16_rne_from_f32(hval);
                    ((uint16_t*)g.out)[(int64_t)prow * (g.N / 2) + feat] = (uint16_t)hb;
                    hmax = umax32(hmax, hb & 0x7FFFu);
                }
            } else {
#pragma unroll
                for (int nj = 0; nj < 2; ++nj) {
                    const int n = f0 + wn * 64 + nj * 32 + (lane & 31);
                    if (n >= g.N) continue;
                    const int64_t o = (int64_t)prow * g.N + n;
                    if (g.out_bf16)
                        ((uint16_t*)g.out)[o] = (uint16_t)bf16_rne_from_f32(y[nj]);
                    else
                        ((float*)g.out)[o] = y[nj];
                }
            }
        }
    }
    if (swiglu && g.amax) amax_group_store(g, hmax, reinterpret_cast<uint32_t*>(sA));
}


// ------------------------------------------------------------ big tiles --
// 256 x 256 output tile, 512 threads = 8 waves in a 2 x 4 grid, two waves per
// SIMD so that one wave's dequantization overlaps the other's MFMAs; each
// wave owns a 128 x 64 sub-tile = 4 x 2 MFMA tiles.  K advances 64 channels
// per stage through two fp16 LDS buffers (2 x 64 KB, A and W slices).
//
// Thread t loads half-row t%2 of A row t/2 and of W row t/2 (32 codes = 16
// bytes + 2 scale bytes each).  Loads run two stages ahead (two register
// sets): while the waves run the MFMAs of stage i, the thread dequantizes
// the data of stage i+1, which arrived during stage i-1, exactly to fp16 and
// stores it into the other LDS buffer, and the loads of stage i+2 are in
// flight.  In a 128-byte LDS row, 16-byte chunk c sits at chunk
// c ^ ((row >> 1) & 7), so the 16 rows served together by the 64-bank LDS
// hit distinct banks.
//
// Work-group numbering: the hardware deals work-group ids round-robin over
// the 8 XCDs, each with its own L2.  Tiles are numbered M-tile-major and cut
// into groups of `grp` consecutive tiles (two M tiles' worth of N tiles:
// shared activation rows, usually one expert's weights); group g of XCD x is
// tile group 8 g + x, so every XCD walks the tile list at the same pace and
// the (upper-bound) tail of empty tiles is shared evenly.
//
// Compensation (k > 0): its stages run first into the same accumulators,
// which are then multiplied by s_tR / s_tA before the main stages; the
// epilogue multiplies by s_tA s_tW[e].  32-row MFMA blocks past the end of
// an expert's rows are skipped.  Requires K % 64 == 0 and k % 64 == 0.
namespace v2 {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
constexpr int kStage = (BM + BN) * BK;          // halfs per LDS stage

__device__ __forceinline__ int swz(int r, int c) { return r * BK + 8 * (c ^ ((r >> 1) & 7)); }

struct Raw {
    uint4 n;            // 32 fp4 codes
    uint32_t sc;        // 2 E4M3 block scales (low 16 bits)
};

__device__ __forceinline__ Raw load_raw(const uint8_t* nib_row, const uint8_t* sc_row, int kc,
                                        bool valid) {
    Raw r;
    if (valid) {
        r.n = *reinterpret_cast<const uint4*>(nib_row + kc / 2);
        r.sc = *reinterpret_cast<const uint16_t*>(sc_row + kc / kBlock);
    } else {
        r.n = make_uint4(0, 0, 0, 0);
        r.sc = 0;
    }
    return r;
}


__device__ __forceinline__ f16x8 cvt8(uint32_t w, _Float16 s) {
    const f16x2 s2 = {s, s};
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Dequantize the 32-code half-row exactly to fp16 and store it as chunks
// 4 half .. 4 half + 3 of LDS row `row` (st = start of the A or W region).
__device__ __forceinline__ void store_slice(const Raw& r, _Float16* st, int row, int half) {
    const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sc, 1.0f, false);   // exact
    const int c = 4 * half;
    *reinterpret_cast<f16x8*>(st + swz(row, c + 0)) = cvt8(r.n.x, s01[0]);
    *reinterpret_cast<f16x8*>(st + swz(row, c + 1)) = cvt8(r.n.y, s01[0]);
    *reinterpret_cast<f16x8*>(st + swz(row, c + 2)) = cvt8(r.n.z, s01[1]);
    *reinterpret_cast<f16x8*>(st + swz(row, c + 3)) = cvt8(r.n.w, s01[1]);
}

// Compensation W half-row: codes w[n, sel[i0 + 32 half + u]], u = 0..31, each
// with its own block scale, stored like store_slice.
__device__ __forceinline__ void gather_store(const uint8_t* w_nib_row, const uint8_t* w_sc_row,
                                             const int32_t* sel, int i0, int kdim, bool valid,
                                             _Float16* st, int row, int half) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t nb[8], sb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            int j = sel[i0 + 32 * half + 8 * q + u];
            j = j < 0 ? 0 : (j >= kdim ? kdim - 1 : j);      // bounds only; sel must be in [0, K)
            nb[u] = w_nib_row[j >> 1] >> (4 * (j & 1));
            sb[u] = w_sc_row[j >> 4];
        }
        _Float16 hv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const _Float16 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb[u], 1.0f, false)[0];
            const _Float16 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nb[u] & 0xFu, 1.0f, 0)[0] * s;
            hv[u] = valid ? v : (_Float16)0;
        }
        *reinterpret_cast<f16x8*>(st + swz(row, 4 * half + q)) =
            (f16x8){hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
    }
}

// Per-lane LDS offset (halfs, relative to a 32-row block) of the fragment of
// sub-step kk: row lane%32, logical chunk 2 kk + lane/32.  Block bases are
// multiples of 32 rows, so the swizzle depends on the lane only.
__device__ __forceinline__ int frag_off(int lane, int kk) {
    const int r = lane & 31;
    return r * BK + 8 * ((2 * kk + (lane >> 5)) ^ ((r >> 1) & 7));
}

// MFMAs of one 16-deep sub-step of a stage (foff = frag_off(lane, kk)) for
// the wave's first MACT 32-row blocks.  MACT is a template argument so that
// the loop bodies have no branches around the MFMAs, which lets the compiler
// interleave them with the loads, conversions and LDS stores of the stage.
template <int MACT>
__device__ __forceinline__ void mma_kk(const _Float16* sa_base, const _Float16* sb_base, int foff,
                                       int wm, int wn, f32x16 acc[4][2]) {
    if (MACT == 0) return;
    const _Float16* sa = sa_base + wm * 128 * BK + foff;
    const _Float16* sb = sb_base + wn * 64 * BK + foff;
    f16x8 a[4], b[2];
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) b[nj] = *reinterpret_cast<const f16x8*>(sb + nj * 32 * BK);
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi) a[mi] = *reinterpret_cast<const f16x8*>(sa + mi * 32 * BK);
    // weights as the first operand: acc[mi][nj] holds the transposed 32 x 32
    // block, lane l owning activation row l % 32 and output features
    // 8 (v / 4) + 4 (l / 32) + v % 4 of register v (four consecutive ones)
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[nj], a[mi], acc[mi][nj], 0, 0, 0);
}

// Capture of the weight columns of the selected channels that fall in a
// stage (k0 .. k0 + 63) from the stage's W tile into ws_s (column = index
// into sel): thread rows crow, indices of parity cpar.  Lane i of every wave
// holds my_sel = sel[i] (kc <= 64 channels), so the stage's channels are one
// ballot and their indices come from readlane: no memory loads.  The first
// kCapBatch values are read before the stage's MFMAs and written after them
// (their LDS latency hides behind the MFMAs instead of standing before the
// stage's barrier); further ones, if any, are copied one by one at the end.
constexpr int kCapBatch = 4;
struct CapBatch {
    unsigned long long rest;      // channels not in the batch (sel indices)
    int ic[kCapBatch];            // sel index of each batch entry, -1: none
    _Float16 v[kCapBatch];
};

__device__ __forceinline__ void capture_read(const _Float16* cur_w, int my_sel, int k0, int crow,
                                             int cpar, CapBatch& b) {
    unsigned long long m = __ballot(my_sel >= k0 && my_sel < k0 + BK) &
                           (cpar ? 0xAAAAAAAAAAAAAAAAull : 0x5555555555555555ull);
#pragma unroll
    for (int u = 0; u < kCapBatch; ++u) {
        b.ic[u] = -1;
        if (m) {
            const int ic = __ffsll(m) - 1;
            m &= m - 1;
            const int c = __builtin_amdgcn_readlane(my_sel, ic) - k0;
            b.ic[u] = ic;
            b.v[u] = cur_w[swz(crow, c >> 3) + (c & 7)];
        }
    }
    b.rest = m;
}

__device__ __forceinline__ void capture_write(const _Float16* cur_w, _Float16* ws_s, int my_sel,
                                              int k0, int crow, CapBatch& b) {
#pragma unroll
    for (int u = 0; u < kCapBatch; ++u)
        if (b.ic[u] >= 0) ws_s[swz(crow, b.ic[u] >> 3) + (b.ic[u] & 7)] = b.v[u];
    unsigned long long m = b.rest;
    while (m) {
        const int ic = __ffsll(m) - 1;
        m &= m - 1;
        const int c = __builtin_amdgcn_readlane(my_sel, ic) - k0;
        ws_s[swz(crow, ic >> 3) + (ic & 7)] = cur_w[swz(crow, c >> 3) + (c & 7)];
    }
}

// One stage: MFMAs on `cur` with the dequantization of (ra, rb) into `nxt`
// spread between the sub-steps.
// ALIVE: this wave's A slice (tile rows 32 wave .. 32 wave + 31) holds rows
// of the tile; otherwise the wave neither loads nor stores A (those LDS rows
// feed only MFMA blocks that are skipped).  LATE: the two waves that share a
// SIMD (waves w and w + 4) run the stage in opposite phase -- one starts with
// MFMAs, the other with its conversions and LDS stores -- so that one wave's
// vector work overlaps the other's MFMAs.
template <int MACT, bool ALIVE, bool LATE>
__device__ __forceinline__ void stage(const _Float16* cur, _Float16* nxt, const Raw& ra,
                                      const Raw& rb, int lr, int lh, int wm, int wn,
                                      const int fo[4], f32x16 acc[4][2]) {
    if (LATE) {
        if (ALIVE) store_slice(ra, nxt, lr, lh);
        mma_kk<MACT>(cur, cur + BM * BK, fo[0], wm, wn, acc);
        mma_kk<MACT>(cur, cur + BM * BK, fo[1], wm, wn, acc);
        store_slice(rb, nxt + BM * BK, lr, lh);
        mma_kk<MACT>(cur, cur + BM * BK, fo[2], wm, wn, acc);
        mma_kk<MACT>(cur, cur + BM * BK, fo[3], wm, wn, acc);
    } else {
        mma_kk<MACT>(cur, cur + BM * BK, fo[0], wm, wn, acc);
        mma_kk<MACT>(cur, cur + BM * BK, fo[1], wm, wn, acc);
        if (ALIVE) store_slice(ra, nxt, lr, lh);
        mma_kk<MACT>(cur, cur + BM * BK, fo[2], wm, wn, acc);
        mma_kk<MACT>(cur, cur + BM * BK, fo[3], wm, wn, acc);
        store_slice(rb, nxt + BM * BK, lr, lh);
    }
}


// Compensation stages with gathered weight columns (first, before the main
// stages), then acc *= s_tR / s_tA.  Used when the captured order below
// cannot be taken (k > 64, or s_tR < 2^-80 s_tA).
template <int MACT>
__device__ __forceinline__ void comp_first(const GemmArgs& g, _Float16* smem, int64_t src,
                                           bool a_valid, bool b_valid, const uint8_t* w_nib_row,
                                           const uint8_t* w_sc_row, int lr, int lh, int wm,
                                           int wn, const int fo[4], f32x16 acc[4][2]) {
    const uint8_t* r_nib_row = g.r_nib + src * (g.k / 2);
    const uint8_t* r_sc_row = g.r_scale + src * (g.k / kBlock);
    for (int i0 = 0; i0 < g.k; i0 += BK) {
        const Raw ra = load_raw(r_nib_row, r_sc_row, i0 + 32 * lh, a_valid);
        store_slice(ra, smem, lr, lh);
        gather_store(w_nib_row, w_sc_row, g.sel, i0, g.K, b_valid, smem + BM * BK, lr, lh);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) mma_kk<MACT>(smem, smem + BM * BK, fo[kk], wm, wn, acc);
        __syncthreads();
    }
    const float rho = g.r_ts[0] / g.a_ts[0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = acc[i][j][v] * rho;
}

// Main stages through two LDS buffers, the loads of stage s + 1 in flight
// during stage s.  Stage offsets past the end are clamped to the last stage
// (a redundant, in-bounds load whose data goes to the idle buffer and is
// never read), so the loop body has no conditional loads or stores; rows
// past the tile's end load a valid row and their results are never written.
//
// With kc = 64 the weight columns of the selected channels are captured from
// the staged W tiles into ws_s on the way, and one compensation stage follows:
// acc *= up (= s_tA / s_tR <= 2^80, so |acc| stays below 2^120), then acc +=
// R x W[:, S]; the epilogue scale is then s_tR s_tW.
template <int MACT, bool ALIVE, bool LATE>
__device__ __forceinline__ void main_stages(const GemmArgs& g, _Float16* smem, _Float16* ws_s,
                                            int kc, float up, int64_t src, bool a_valid,
                                            const uint8_t* a_nib_row, const uint8_t* a_sc_row,
                                            const uint8_t* w_nib_row, const uint8_t* w_sc_row,
                                            int lr, int lh, int wm, int wn, const int fo[4],
                                            f32x16 acc[4][2]) {
    const int crow = threadIdx.x & 255, cpar = threadIdx.x >> 8;
    const int lane = threadIdx.x & 63;
    const int my_sel = lane < kc ? g.sel[lane] : -1;
    const int nk = g.K / BK;
    const int klast = g.K - BK;
    // With kc > 0, the load that would fetch the (clamped) stage past the end
    // fetches this row's R codes instead; the last stage stores them into the
    // idle buffer's A slice for the compensation stage.  Rows past the tile's
    // end read R row 0 (src = 0); their results are never written.
    const uint8_t* r_nib_row = kc > 0 ? g.r_nib + src * (g.k / 2) : a_nib_row;
    const uint8_t* r_sc_row = kc > 0 ? g.r_scale + src * (g.k / kBlock) : a_sc_row;
    // stages 0 and 1 are loaded together, then stage 0 is converted and stored
    Raw ra, a0;
    if (!ALIVE) {
        ra.n = a0.n = make_uint4(0, 0, 0, 0);
        ra.sc = a0.sc = 0;
    } else {
        ra = load_raw(a_nib_row, a_sc_row, 32 * lh, true);
        a0 = nk > 1 ? load_raw(a_nib_row, a_sc_row, BK + 32 * lh, true)
                    : load_raw(r_nib_row, r_sc_row, 32 * lh, true);
    }
    const Raw rb = load_raw(w_nib_row, w_sc_row, 32 * lh, true);
    Raw b0 = load_raw(w_nib_row, w_sc_row, min(BK, klast) + 32 * lh, true);
    store_slice(rb, smem + BM * BK, lr, lh);
    if (ALIVE) store_slice(ra, smem, lr, lh);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        _Float16* cur = smem + (it & 1) * kStage;
        _Float16* nxt = smem + ((it & 1) ^ 1) * kStage;
        CapBatch cb;
        if (kc > 0) capture_read(cur + BM * BK, my_sel, it * BK, crow, cpar, cb);
        stage<MACT, ALIVE, LATE>(cur, nxt, a0, b0, lr, lh, wm, wn, fo, acc);
        if (ALIVE) {
            const bool past = it + 2 >= nk;
            const uint8_t* an = past ? r_nib_row : a_nib_row + (it + 2) * (BK / 2);
            const uint8_t* as = past ? r_sc_row : a_sc_row + (it + 2) * (BK / kBlock);
            a0 = load_raw(an, as, 32 * lh, true);
        }
        b0 = load_raw(w_nib_row, w_sc_row, min((it + 2) * BK, klast) + 32 * lh, true);
        if (kc > 0) capture_write(cur + BM * BK, ws_s, my_sel, it * BK, crow, cb);
        __syncthreads();
    }
    if (kc == 0) return;
    // compensation stage: A = R in the buffer the last stage stored into, B = ws_s
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = acc[i][j][v] * up;
    const _Float16* rbuf = smem + (nk & 1) * kStage;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mma_kk<MACT>(rbuf, ws_s, fo[kk], wm, wn, acc);
}

template <int kEpi>
__global__ __launch_bounds__(kThreads) void k_gemm_w4a4_v2(GemmArgs g, int nt_n, int grp) {
    __shared__ _Float16 smem[2 * kStage];
    __shared__ _Float16 ws_s[BN * BK];           // captured weight columns W[:, S]
    // XCD-aware numbering: hardware id h runs on XCD h % 8
    const int h = blockIdx.x;
    const int slot = h / kXcds;
    const int tile = (slot / grp) * (kXcds * grp) + (h % kXcds) * grp + slot % grp;
    const int tile_m = tile / nt_n, tile_n = tile - tile_m * nt_n;
    int e, m0, mend;
    if (!find_tile_wave<BM>(g.offsets, g.E, g.rows, tile_m, &e, &m0, &mend, g.dec_rows,
                            g.tail_rows)) {
        if (g.amax) amax_group_none(g);
        return;
    }
    bind_expert(g, e);
    constexpr bool swiglu = kEpi == QUADS_EPI_SWIGLU;
    const int f0 = tile_n * (swiglu ? BN / 2 : BN);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    int mact = (mend - (m0 + wm * 128) + 31) / 32;
    mact = __builtin_amdgcn_readfirstlane(mact < 0 ? 0 : (mact > 4 ? 4 : mact));
    const int lr = tid >> 1, lh = tid & 1;

    const int p = m0 + lr;
    const bool a_valid = p < mend;
    const int64_t src = a_valid ? (g.row_token ? (int64_t)g.row_token[p] : (int64_t)p) : 0;
    bool b_valid;
    const int wrow = w_row_v2(lr, f0, g.N, swiglu, &b_valid);
    const int64_t wr = (int64_t)e * g.N + (b_valid ? wrow : 0);
    const uint8_t* a_nib_row = g.a_nib + src * (g.K / 2);
    const uint8_t* a_sc_row = g.a_scale + src * (g.K / kBlock);
    const uint8_t* w_nib_row = g.w_nib + wr * (g.K / 2);
    const uint8_t* w_sc_row = g.w_scale + wr * (g.K / kBlock);
    int fo[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fo[kk] = frag_off(lane, kk);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // Compensation order.  With kc = 64 selected channels (one stage) and
    // s_tR >= 2^-80 s_tA, the weight columns are captured during the main
    // stages and the compensation runs last, after acc *= s_tA / s_tR
    // (<= 2^80, so |acc| stays below 2^120).  Otherwise it runs first with
    // gathered weight columns and acc *= s_tR / s_tA.  s_tR = 0 means every
    // residual code is 0 and the compensation is skipped.
    const float s_ta = tensor_scale_a(g);
    const float s_tr = g.k > 0 ? g.r_ts[0] : 0.0f;
    const bool comp = g.k > 0 && s_tr > 0.0f;
    const bool capture_path = !comp || (g.k == BK && s_tr >= s_ta * 0x1p-80f);
    const float cscale = comp && capture_path ? s_tr : s_ta;
    const int kc = comp && capture_path ? g.k : 0;
    const float up = kc > 0 ? s_ta / s_tr : 1.0f;
    if (kc > 0) {                                       // no stale values in unused columns
        for (int i = tid; i < BN * BK / 8; i += kThreads)
            reinterpret_cast<f16x8*>(ws_s)[i] = (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
    // wave-uniform: does this wave's A slice (tile rows 32 wave ..) hold rows?
    const bool alive = m0 + 32 * wave < mend;
    switch (__builtin_amdgcn_readfirstlane(mact + (alive ? 8 : 0))) {
#define QUADS_TILE(M, L)                                                                       \
    case M + (L ? 8 : 0):                                                                      \
        if (comp && !capture_path)                                                             \
            comp_first<M>(g, smem, src, a_valid, b_valid, w_nib_row, w_sc_row, lr, lh, wm, wn, \
                          fo, acc);                                                            \
        if (wm)                                                                                \
            main_stages<M, L, true>(g, smem, ws_s, kc, up, src, a_valid, a_nib_row, a_sc_row,  \
                                    w_nib_row, w_sc_row, lr, lh, wm, wn, fo, acc);             \
        else                                                                                   \
            main_stages<M, L, false>(g, smem, ws_s, kc, up, src, a_valid, a_nib_row, a_sc_row, \
                                     w_nib_row, w_sc_row, lr, lh, wm, wn, fo, acc);            \
        break;
        QUADS_TILE(4, true) QUADS_TILE(3, true) QUADS_TILE(2, true) QUADS_TILE(1, true)
        QUADS_TILE(0, true) QUADS_TILE(4, false) QUADS_TILE(3, false) QUADS_TILE(2, false)
        QUADS_TILE(1, false)
        default: QUADS_TILE(0, false)
#undef QUADS_TILE
    }

    // epilogue
    const uint32_t hmax = epilogue<kEpi>(g, acc, cscale * g.w_ts[e], m0, mend, f0, wm, wn, mact,
                                         lane);
    if (swiglu && g.amax) amax_group_store(g, hmax, reinterpret_cast<uint32_t*>(ws_s));
}

}  // namespace v2


}  // namespace quads

using namespace quads;

// Workspace: only the tiled kernel's gathered compensation uses one (W[:, S]
// as fp16, E * N * k * 2 bytes, for long contractions with k above 256).
extern "C" size_t quads_moe_w4a4_gemm_ws(int64_t rows, int64_t K, int32_t k, int32_t E,
                                         int64_t N) {
    (void)rows;
    return gemm_v3_gather_ws(K, k, E, N);
}

// The kernels of one call, in launch order (see LaunchPlan).
static int gemm_dispatch(GemmArgs g, void* ws, size_t ws_bytes, hipStream_t st, LaunchPlan* lp) {
    const int64_t rows = g.rows;
    const int64_t K = g.K, k = g.k, E = g.E, N = g.N;
    const int epilogue = g.epilogue;
    const int32_t* offsets = g.offsets;
    if (gemm_decode_fits(g)) {
        // few rows per expert: the decode kernel takes every expert with at
        // most kDecodeMaxRows rows, or all of them at most kDecodeAllRows
        // rows in all; when some expert may have more than it takes, the
        // tiled kernel below takes those
        g.dec_rows = rows <= kDecodeAllRows ? (int)rows : kDecodeMaxRows;
        const int rc = launch_gemm_decode(g, st, lp);
        if (rc != QUADS_OK || rows <= g.dec_rows) return rc;
    }
    // one accumulator chain is short enough for the error bound: the
    // 256 x 256-tile kernel; longer chains: the kernels that restart their
    // accumulators every kAccChain channels
    const bool one_chain = K + k <= kSingleChainMax;
    const bool tiles_v3 = !one_chain && gemm_v3_fits(g);
    const bool tiles_v2 = one_chain && K % v2::BK == 0 && k % v2::BK == 0;
    // near 256 rows per expert on average, the experts of 257 .. 320 rows
    // leave their rows past 256 to the decode kernel (which streams the
    // expert's weights once for them), so the long-chain kernel's 256-row
    // tiles stay full.  Measured on the 128-expert layer (32768 packed rows,
    // half of the experts at 257 .. 301 rows): gate/up (K = 2048 + 64) 365 ->
    // 295 + 57 us; for the single-chain kernel (down, K = 768 + 64) the
    // decode share costs more than the tiles save (200 -> 175 + 33 us), so
    // it keeps its split tiles.
    if (tiles_v3 && g.dec_rows == 0 && offsets != nullptr && rows <= (int64_t)512 * E &&
        gemm_decode_tail_fits(g)) {
        g.tail_rows = kTailRows;
        const int rc = launch_gemm_decode(g, st, lp);
        if (rc != QUADS_OK) return rc;
    }
    if (tiles_v3) return launch_gemm_v3(g, st, lp);
    if (!one_chain && gemm_v3_gather_fits(g) && ws_bytes >= gemm_v3_gather_ws(K, k, E, N) &&
        ws != nullptr)
        return launch_gemm_v3_gather(g, ws, st, lp);
    if (tiles_v2) {
        const int64_t nt_n = epilogue == QUADS_EPI_SWIGLU ? (N / 2 + v2::BN / 2 - 1) / (v2::BN / 2)
                                                          : (N + v2::BN - 1) / v2::BN;
        // M-tiles: at most rows / BM + one partial tile per expert that has
        // tiles (with a decode share, only experts above g.dec_rows rows)
        const int64_t big = g.dec_rows > 0 ? rows / (g.dec_rows + 1) : E;
        const int64_t nt_m = (rows + v2::BM - 1) / v2::BM + (offsets ? (big < E ? big : E) : 0);
        const int64_t grp = 2 * nt_n;
        const int64_t span = grp * v2::kXcds;
        const int64_t blocks = (nt_m * nt_n + span - 1) / span * span;
        g.amax_base = lp->blocks;
        lp->blocks += blocks;
        if (lp->dry) return QUADS_OK;
        const dim3 grid2((unsigned)blocks);
        if (epilogue == QUADS_EPI_SWIGLU)
            hipLaunchKernelGGL(v2::k_gemm_w4a4_v2<QUADS_EPI_SWIGLU>, grid2, dim3(v2::kThreads), 0,
                               st, g, (int)nt_n, (int)grp);
        else
            hipLaunchKernelGGL(v2::k_gemm_w4a4_v2<QUADS_EPI_NONE>, grid2, dim3(v2::kThreads), 0,
                               st, g, (int)nt_n, (int)grp);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    const int64_t ntiles_n = epilogue == QUADS_EPI_SWIGLU ? (N / 2 + kBN / 2 - 1) / (kBN / 2)
                                                          : (N + kBN - 1) / kBN;
    const int64_t big = g.dec_rows > 0 ? rows / (g.dec_rows + 1) : E;
    int64_t ntiles_m = (rows + kBM - 1) / kBM + (offsets ? (big < E ? big : E) : 0);
    g.amax_base = lp->blocks;
    lp->blocks += ntiles_n * ntiles_m;
    if (lp->dry) return QUADS_OK;
    const dim3 grid((unsigned)ntiles_n, (unsigned)ntiles_m);
    if (epilogue == QUADS_EPI_SWIGLU)
        hipLaunchKernelGGL(k_gemm_w4a4<QUADS_EPI_SWIGLU>, grid, dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL(k_gemm_w4a4<QUADS_EPI_NONE>, grid, dim3(256), 0, st, g);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}


// Both entry points: a_ts_rows is null (one tensor scale a_ts[0]) or the
// per-row scales [Ta] (then a_ts == a_ts_rows and k == 0).
static int gemm_w4a4(const uint8_t* a_nib, const uint8_t* a_scale, const float* a_ts,
                     const float* a_ts_rows, int sel_per_expert, const int32_t* row_token,
                     int64_t rows, int64_t K,
                     const uint8_t* r_nib, const uint8_t* r_scale, const float* r_ts,
                     const int32_t* sel, int32_t k, const uint8_t* w_nib,
                     const uint8_t* w_scale, const float* w_ts, const int32_t* offsets,
                     int32_t E, int64_t N, int epilogue, int out_dtype, void* out,
                     uint32_t* amax, int64_t amax_groups, void* ws, size_t ws_bytes,
                     void* stream) {
    if (epilogue != QUADS_EPI_NONE && epilogue != QUADS_EPI_SWIGLU) return QUADS_EINVAL;
    if (out_dtype != QUADS_OUT_F32 && out_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (epilogue == QUADS_EPI_SWIGLU && out_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (rows < 0 || rows >= ((int64_t)1 << 31) || K <= 0 || K % kBlock || K >= ((int64_t)1 << 30))
        return QUADS_ESHAPE;
    if (k < 0 || k % kBlock || k > K) return QUADS_ESHAPE;
    if (E < 1 || E > kGemmMaxE || N < 1 || N >= ((int64_t)1 << 30)) return QUADS_ESHAPE;
    if (epilogue == QUADS_EPI_SWIGLU && N % 2) return QUADS_ESHAPE;
    if (offsets == nullptr && E != 1) return QUADS_EINVAL;
    if (rows == 0) return QUADS_OK;                   // size 0: a no-op, whatever the pointers
    if (!ok_opt_ptr(offsets) || !ok_opt_ptr(row_token)) return QUADS_EINVAL;
    if (!ok_ptr(a_nib) || !ok_ptr(a_scale) || !ok_ptr(a_ts) || !ok_ptr(w_nib) ||
        !ok_ptr(w_scale) || !ok_ptr(w_ts) || !ok_ptr(out))
        return QUADS_EINVAL;
    if (k > 0 && (!ok_ptr(r_nib) || !ok_ptr(r_scale) || !ok_ptr(r_ts) || !ok_ptr(sel)))
        return QUADS_EINVAL;
    const size_t need = quads_moe_w4a4_gemm_ws(rows, K, k, E, N);
    if (ws_bytes < need || (need > 0 && !ok_ptr(ws))) return QUADS_EWORKSPACE;
    if (amax != nullptr && (epilogue != QUADS_EPI_SWIGLU || !ok_ptr4(amax) || amax_groups < 1))
        return QUADS_EINVAL;
    GemmArgs g{a_nib, a_scale, a_ts, row_token, rows, (int)K, r_nib, r_scale, r_ts, sel, (int)k,
               w_nib, w_scale, w_ts, offsets, (int)E, (int)N, epilogue,
               out_dtype == QUADS_OUT_BF16, out, 0, a_ts_rows, sel_per_expert};
    hipStream_t st = (hipStream_t)stream;
    if (amax != nullptr) {
        // the work-groups of every launch of the call, one slot each
        LaunchPlan dry{true, 0};
        const int rc = gemm_dispatch(g, ws, ws_bytes, st, &dry);
        if (rc != QUADS_OK) return rc;
        if (dry.blocks > amax_groups) return QUADS_EWORKSPACE;
        g.amax = amax;
        g.amax_end = amax_groups;
    }
    LaunchPlan lp{false, 0};
    return gemm_dispatch(g, ws, ws_bytes, st, &lp);
}

extern "C" int quads_moe_w4a4_gemm(const uint8_t* a_nib, const uint8_t* a_scale,
                                   const float* a_ts, const int32_t* row_token, int64_t rows,
                                   int64_t K, const uint8_t* r_nib, const uint8_t* r_scale,
                                   const float* r_ts, const int32_t* sel, int32_t k,
                                   const uint8_t* w_nib, const uint8_t* w_scale,
                                   const float* w_ts, const int32_t* offsets, int32_t E,
                                   int64_t N, int epilogue, int out_dtype, void* out, void* ws,
                                   size_t ws_bytes, void* stream) {
    return gemm_w4a4(a_nib, a_scale, a_ts, nullptr, 0, row_token, rows, K, r_nib, r_scale, r_ts,
                     sel, k, w_nib, w_scale, w_ts, offsets, E, N, epilogue, out_dtype, out,
                     nullptr, 0, ws, ws_bytes, stream);
}

// Partial-maximum slots of a SwiGLU call of these sizes: the work-groups of
// its launches, the largest over a call with or without offsets (E == 1)
// and with or without a workspace.
extern "C" int64_t quads_moe_w4a4_gemm_amax_groups(int64_t rows, int64_t K, int32_t k, int32_t E,
                                                   int64_t N) {
    if (rows < 1 || rows >= ((int64_t)1 << 31) || K <= 0 || K % kBlock ||
        K >= ((int64_t)1 << 30) || k < 0 || k % kBlock || k > K || E < 1 || E > kGemmMaxE ||
        N < 2 || N % 2 || N >= ((int64_t)1 << 30))
        return 0;
    static const int32_t dummy_offsets[1] = {0};
    char dummy_ws[1];
    int64_t most = 0;
    for (int with_offsets = 0; with_offsets < 2; ++with_offsets) {
        if (!with_offsets && E != 1) continue;
        for (int with_ws = 0; with_ws < 2; ++with_ws) {
            GemmArgs g{};
            g.rows = rows; g.K = (int)K; g.k = (int)k; g.E = (int)E; g.N = (int)N;
            g.epilogue = QUADS_EPI_SWIGLU; g.out_bf16 = 1;
            g.offsets = with_offsets ? dummy_offsets : nullptr;
            LaunchPlan dry{true, 0};
            const size_t wsb = with_ws ? quads_moe_w4a4_gemm_ws(rows, K, k, E, N) : 0;
            if (gemm_dispatch(g, with_ws ? dummy_ws : nullptr, wsb, nullptr, &dry) != QUADS_OK)
                continue;
            most = dry.blocks > most ? dry.blocks : most;
        }
    }
    return most;
}

extern "C" int quads_moe_w4a4_gemm_amax(const uint8_t* a_nib, const uint8_t* a_scale,
                                        const float* a_ts, const int32_t* row_token, int64_t rows,
                                        int64_t K, const uint8_t* r_nib, const uint8_t* r_scale,
                                        const float* r_ts, const int32_t* sel, int32_t k,
                                        const uint8_t* w_nib, const uint8_t* w_scale,
                                        const float* w_ts, const int32_t* offsets, int32_t E,
                                        int64_t N, void* out, uint32_t* amax_part,
                                        int64_t amax_groups, void* ws, size_t ws_bytes,
                                        void* stream) {
    if (rows > 0 && !ok_ptr4(amax_part)) return QUADS_EINVAL;
    return gemm_w4a4(a_nib, a_scale, a_ts, nullptr, 0, row_token, rows, K, r_nib, r_scale, r_ts,
                     sel, k, w_nib, w_scale, w_ts, offsets, E, N, QUADS_EPI_SWIGLU,
                     QUADS_OUT_BF16, out, amax_part, amax_groups, ws, ws_bytes, stream);
}

extern "C" int quads_moe_w4a4_gemm_rowscale(const uint8_t* a_nib, const uint8_t* a_scale,
                                            const float* a_ts_rows, const int32_t* row_token,
                                            int64_t rows, int64_t K, const uint8_t* w_nib,
                                            const uint8_t* w_scale, const float* w_ts,
                                            const int32_t* offsets, int32_t E, int64_t N,
                                            int epilogue, int out_dtype, void* out, void* ws,
                                            size_t ws_bytes, void* stream) {
    if (rows > 0 && !ok_ptr(a_ts_rows)) return QUADS_EINVAL;
    return gemm_w4a4(a_nib, a_scale, a_ts_rows, a_ts_rows, 0, row_token, rows, K, nullptr, nullptr,
                     nullptr, nullptr, 0, w_nib, w_scale, w_ts, offsets, E, N, epilogue,
                     out_dtype, out, nullptr, 0, ws, ws_bytes, stream);
}

extern "C" int quads_moe_w4a4_gemm_sel_experts(const uint8_t* a_nib, const uint8_t* a_scale,
                                               const float* a_ts, int64_t rows, int64_t K,
                                               const uint8_t* r_nib, const uint8_t* r_scale,
                                               const float* r_ts, const int32_t* sel, int32_t k,
                                               const uint8_t* w_nib, const uint8_t* w_scale,
                                               const float* w_ts, const int32_t* offsets,
                                               int32_t E, int64_t N, int epilogue,
                                               int out_dtype, void* out, void* ws,
                                               size_t ws_bytes, void* stream) {
    if (!ok_ptr(offsets)) return QUADS_EINVAL;
    if (k > 0 && !ok_ptr(r_ts)) return QUADS_EINVAL;
    return gemm_w4a4(a_nib, a_scale, a_ts, nullptr, 1, nullptr, rows, K, r_nib, r_scale, r_ts,
                     sel, k, w_nib, w_scale, w_ts, offsets, E, N, epilogue, out_dtype, out,
                     nullptr, 0, ws, ws_bytes, stream);
}
