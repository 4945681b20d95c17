// Pieces shared by the 256 x 256-tile grouped GEMM kernels (the NVFP4
// W4A4 GEMM and the MX block-scaled comparator): the argument block, the
// MoE tile lookup and the epilogue of a 256 x 256 output tile whose waves
// each own 128 x 64 outputs as 4 x 2 transposed 32 x 32 MFMA blocks.
#pragma once

#include "common.h"

namespace quads {

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
    const uint8_t* a_nib; const uint8_t* a_scale; const float* a_ts;
    const int32_t* row_token; int64_t rows; int K;
    const uint8_t* r_nib; const uint8_t* r_scale; const float* r_ts; const int32_t* sel; int k;
    const uint8_t* w_nib; const uint8_t* w_scale; const float* w_ts;
    const int32_t* offsets; int E; int N;
    int epilogue; int out_bf16; void* out;
    // Experts with at most this many rows belong to the decode kernel
    // (gemm_decode.hip); the tiled kernels skip them.  0: the tiled kernel
    // takes every expert.
    int dec_rows;
    // Per-row activation scales [Ta] (one per activation row, indexed through
    // row_token), or null for the single tensor scale a_ts[0].  Only with
    // k == 0.
    const float* a_ts_rows;
    // 1: sel is [E, k] and r_ts [E], one selection and residual scale per
    // expert (activations in packed order); 0: one shared sel [k], r_ts [1].
    int sel_per_expert;
    // The tiled kernel's gathered compensation (k above kCapMaxV3): W[:, S]
    // as exact fp16 values [E, N, k] in the caller's workspace, else null.
    const _Float16* w_sel;
    // > 0: an expert of 257 .. 256 + tail_rows rows leaves its rows past the
    // first 256 (its tail) to the decode kernel, so that the 256-row tiled
    // kernels run one full tile for it instead of two part-filled ones.
    int tail_rows;
    // Non-null (SwiGLU only): each work-group of the launch writes the
    // largest |h| it stores (bf16 magnitude bits, 0 if none) to
    // amax[amax_base + its linear id]; work-group 0 also zeroes amax
    // [amax_base + grid size, amax_end), the slots past the call's last
    // launch, so that every one of the caller's amax_end slots is written.
    uint32_t* amax;
    int64_t amax_base, amax_end;
};

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// The magnitudes of two packed bf16 values, the larger one.
__device__ __forceinline__ uint32_t bf16x2_mag_max(uint32_t p) {
    const uint32_t lo = p & 0x7FFFu, hi = (p >> 16) & 0x7FFFu;
    return lo > hi ? lo : hi;
}

// One partial maximum per work-group (see GemmArgs::amax): the threads'
// values m folded through s_amax, one word per wave of LDS that the
// work-group no longer reads (a barrier comes first).  Every thread of the
// work-group calls it.
__device__ __forceinline__ void amax_group_store(const GemmArgs& g, uint32_t m,
                                                 uint32_t* s_amax) {
    const int64_t id = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y;
    for (int64_t i = g.amax_base + nblk + threadIdx.x; id == 0 && i < g.amax_end; i += blockDim.x)
        g.amax[i] = 0u;
    m = wave_max_u32(m);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s_amax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < (int)((blockDim.x + 63) >> 6); ++i) r = s_amax[i] > r ? s_amax[i] : r;
        g.amax[g.amax_base + id] = r;
    }
}

// The same for a work-group that stores nothing and leaves early (called by
// every thread; no barrier).
__device__ __forceinline__ void amax_group_none(const GemmArgs& g) {
    const int64_t id = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y;
    for (int64_t i = g.amax_base + nblk + threadIdx.x; id == 0 && i < g.amax_end; i += blockDim.x)
        g.amax[i] = 0u;
    if (threadIdx.x == 0) g.amax[g.amax_base + id] = 0u;
}

// Rows at the end of an n-row expert that belong to the decode kernel.
__host__ __device__ inline int expert_tail(int n, int tail_rows) {
    return tail_rows > 0 && n > 256 && n <= 256 + tail_rows ? n - 256 : 0;
}

// Once a work-group knows its expert e: point sel and r_ts at that expert's
// selection and residual scale, so that the kernels read g.sel[i] and
// g.r_ts[0] either way.
__device__ __forceinline__ void bind_expert(GemmArgs& g, int e) {
    if (g.sel_per_expert) {
        g.sel += (int64_t)e * g.k;
        g.r_ts += e;
        g.sel_per_expert = 0;
    }
}

// The activation tensor scale that multiplies a packed row's output: the
// tensor's, or (per-row scales) 1, the row's own scale being applied in the
// epilogue by row_scale().
__device__ __forceinline__ float tensor_scale_a(const GemmArgs& g) {
    return g.a_ts_rows ? 1.0f : g.a_ts[0];
}

// ca for packed row p: the epilogue's ca (s_tA s_tW, or s_tW with per-row
// scales) times the row's own scale.
__device__ __forceinline__ float row_scale(const GemmArgs& g, int p, float ca) {
    if (!g.a_ts_rows) return ca;
    const int64_t src = g.row_token ? (int64_t)g.row_token[p] : (int64_t)p;
    return g.a_ts_rows[src] * ca;
}

// SwiGLU's product silu(g) u = g u / (1 + e^-g), within a few 1e-6 relative
// (half a bf16 ulp is 2^-9) wherever the result and g u are finite in fp32.
// Short form (a = -g log2(e) <= 64, i.e. g >= -44.36): the hardware exp2 and
// reciprocal.  Full form: with the integer c = ceil(max(a - 64, 0)),
// g u / (1 + 2^a) = (g u / (1 + 2^(a-c))) 2^-c, since 1 + 2^a rounds to 2^a
// in fp32 once a > 64; exp2 and the reciprocal then never overflow, and a
// gate far below -88 still gives the small product instead of 0.  With c = 0
// the full form gives the short form's value exactly.
constexpr float kSiluShortMaxA = 64.0f;
__device__ __forceinline__ float silu_a(float g) { return g * -1.4426950408889634f; }
__device__ __forceinline__ float silu_mul_short(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(silu_a(g))) * u;
}
__device__ __forceinline__ float silu_mul_full(float g, float u) {
    const float a = silu_a(g);
    const float c = fminf(ceilf(fmaxf(a - kSiluShortMaxA, 0.0f)), 400.0f);   // beyond: 0
    const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a - c));
    return __builtin_amdgcn_ldexpf(g * r * u, -(int)c);
}
// Per element: a wave takes the full form only when one of its active lanes
// needs it (the result does not depend on the neighbours).
__device__ __forceinline__ float silu_mul(float g, float u) {
    if (__builtin_expect(__ballot(silu_a(g) > kSiluShortMaxA) == 0ull, 1))
        return silu_mul_short(g, u);
    return silu_mul_full(g, u);
}

namespace v2 {

constexpr int kXcds = 8;                // XCDs of an MI355X (work-group ids dealt round-robin)

// Two fp32 values to packed bf16 (round to nearest even, hardware convert).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Tile `tile` of the M-tile list, found by each wave on its own (no LDS, no
// barrier).  An expert with n rows gets t = ceil(n / bm) tiles, its rows split
// evenly over them in 32-row multiples (a 280-row expert gets 160 + 120 rows
// rather than 256 + 24, so neither tile is a near-empty one).  The list is
// ordered by tile height, tallest first (experts in index order within a
// height): the hardware hands each next work-group to the first free CU, so
// the short tiles, dispatched last, fill in the tail (longest-first list
// scheduling).  Lane l looks after experts l*per .. l*per + per - 1; for each
// height a wave scan gives the first tile of each lane's share, and the
// owning lane broadcasts the result.
__device__ __forceinline__ int tile_height(int n, int bm, int* t_out) {
    const int t = (n + bm - 1) / bm;
    *t_out = t;
    return t > 0 ? ((n + t - 1) / t + 31) / 32 : 0;          // in 32-row blocks
}

// Inclusive prefix sum over the wave (every lane active).
__device__ __forceinline__ int wave_scan(int x, int lane) {
    (void)lane;
    return wave_incl_add(x);
}

// Rows of expert e the tiled kernel takes: none for an expert of at most
// `skip` rows, and not its tail (expert_tail) -- the decode kernel takes those.
__device__ __forceinline__ int rows_of(const int32_t* offsets, int e, int skip, int tail_rows) {
    const int n = offsets[e + 1] - offsets[e];
    return n > skip ? n - expert_tail(n, tail_rows) : 0;
}

constexpr int kTileCache = 4;    // experts per lane whose offsets the tile lookup keeps

template <int BMT>
__device__ __forceinline__ bool find_tile_wave(const int32_t* offsets, int E, int64_t rows, int tile, int* e_out,
                               int* m0_out, int* mend_out, int skip = 0, int tail_rows = 0) {
    constexpr int kH = BMT / 32;                  // tile heights 1 .. kH blocks
    if (offsets == nullptr) {
        const int64_t m0 = (int64_t)tile * BMT;
        *e_out = 0;
        *m0_out = (int)m0;
        *mend_out = (int)rows;
        return m0 < rows;
    }
    const int lane = threadIdx.x & 63;
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    const int e1 = e0 + per < E ? e0 + per : E;
    int cnt[kH];                                  // this lane's tiles of each height
#pragma unroll
    for (int q = 0; q < kH; ++q) cnt[q] = 0;
    if (per <= kTileCache) {
        // up to 256 experts: the lane's offsets loaded together once, and the
        // tile found from registers
        int o[kTileCache + 1], n[kTileCache];
#pragma unroll
        for (int u = 0; u <= kTileCache; ++u) o[u] = e0 + u <= e1 ? offsets[e0 + u] : 0;
#pragma unroll
        for (int u = 0; u < kTileCache; ++u) {
            const int r = e0 + u < e1 ? o[u + 1] - o[u] : 0;
            n[u] = r > skip ? r - expert_tail(r, tail_rows) : 0;
            int t;
            const int hgt = tile_height(n[u], BMT, &t);
#pragma unroll
            for (int q = 0; q < kH; ++q) cnt[q] += hgt == q + 1 ? t : 0;
        }
        int all = 0;
#pragma unroll
        for (int q = 0; q < kH; ++q) all += cnt[q];
        if (tile >= __builtin_amdgcn_readlane(wave_incl_add(all), 63)) return false;
        int base = 0;
#pragma unroll
        for (int q = kH - 1; q >= 0; --q) {
            const int hgt = q + 1;
            const int x = wave_incl_add(cnt[q]);
            const int total = __builtin_amdgcn_readlane(x, 63);   // uniform: scalar branches
            if (tile < base + total) {
                int run = base + x - cnt[q], fe = -1, fm0 = 0, fme = 0;
                if (tile >= run && tile < run + cnt[q]) {
#pragma unroll
                    for (int u = 0; u < kTileCache; ++u) {
                        int t;
                        if (fe >= 0 || tile_height(n[u], BMT, &t) != hgt) continue;
                        if (tile < run + t) {
                            fe = e0 + u;
                            fm0 = o[u] + (tile - run) * hgt * 32;
                            fme = fm0 + hgt * 32 < o[u] + n[u] ? fm0 + hgt * 32 : o[u] + n[u];
                        }
                        run += t;
                    }
                }
                const int src = __ffsll(__ballot(fe >= 0)) - 1;
                *e_out = __builtin_amdgcn_readlane(fe, src);
                *m0_out = __builtin_amdgcn_readlane(fm0, src);
                *mend_out = __builtin_amdgcn_readlane(fme, src);
                return true;
            }
            base += total;
        }
        return false;
    }
    for (int e = e0; e < e1; ++e) {
        int t;
        const int hgt = tile_height(rows_of(offsets, e, skip, tail_rows), BMT, &t);
#pragma unroll
        for (int q = 0; q < kH; ++q) cnt[q] += hgt == q + 1 ? t : 0;
    }
    int all = 0;
#pragma unroll
    for (int q = 0; q < kH; ++q) all += cnt[q];
    // work-groups past the last tile leave after one scan
    if (tile >= __builtin_amdgcn_readlane(wave_scan(all, lane), 63)) return false;
    int base = 0;                                 // tiles of the taller heights
#pragma unroll
    for (int q = kH - 1; q >= 0; --q) {
        const int hgt = q + 1;
        const int x = wave_scan(cnt[q], lane);
        const int total = __builtin_amdgcn_readlane(x, 63);       // uniform: scalar branches
        if (tile < base + total) {
            int run = base + x - cnt[q], fe = -1, fm0 = 0, fme = 0;
            if (tile >= run && tile < run + cnt[q]) {
                for (int e = e0; e < e1; ++e) {
                    const int n = rows_of(offsets, e, skip, tail_rows);
                    int t;
                    if (tile_height(n, BMT, &t) != hgt) continue;
                    if (tile < run + t) {
                        fe = e;
                        fm0 = offsets[e] + (tile - run) * hgt * 32;
                        fme = fm0 + hgt * 32 < offsets[e] + n ? fm0 + hgt * 32 : offsets[e] + n;
                        break;
                    }
                    run += t;
                }
            }
            const int src = __ffsll(__ballot(fe >= 0)) - 1;
            *e_out = __builtin_amdgcn_readlane(fe, src);
            *m0_out = __builtin_amdgcn_readlane(fm0, src);
            *mend_out = __builtin_amdgcn_readlane(fme, src);
            return true;
        }
        base += total;
    }
    return false;
}

// SwiGLU outputs of the tile: the short form everywhere (kFull false; *need
// set when a gate needs the full form), or the full form everywhere.
template <bool kFull>
__device__ __forceinline__ void swiglu_store(const GemmArgs& g, const f32x16 acc[4][2], float ca,
                                             int m0, int mend, int f0, int wm, int wn, int mact,
                                             int lane, bool* need, uint32_t* mx) {
    uint32_t m = 0;
    const int prow_l = m0 + wm * 128 + (lane & 31);
    const int nq = 4 * (lane >> 5);
    bool nd = false;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi >= mact) continue;
        const int prow = prow_l + mi * 32;
        if (prow >= mend) continue;
        const float ca_row = row_scale(g, prow, ca);
#pragma unroll
        for (int q = 0; q < 4; ++q) {                 // registers 4q .. 4q + 3
            const int feat = f0 + wn * 32 + 8 * q + nq;          // features feat .. feat + 3
            float hv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float gt = acc[mi][0][4 * q + u] * ca_row;
                const float up = acc[mi][1][4 * q + u] * ca_row;
                if (kFull) {
                    hv[u] = silu_mul_full(gt, up);
                } else {
                    hv[u] = silu_mul_short(gt, up);
                    nd = nd || silu_a(gt) > kSiluShortMaxA;
                }
            }
            const uint32_t p01 = pk_bf16(hv[0], hv[1]), p23 = pk_bf16(hv[2], hv[3]);
            const uint32_t hb[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu, p23 >> 16};
            const int nh = g.N / 2;
            uint16_t* o = (uint16_t*)g.out + (int64_t)prow * nh + feat;
            if (feat + 3 < nh && (nh & 3) == 0) {
                *reinterpret_cast<uint2*>(o) = make_uint2(p01, p23);
                m = umax32(m, umax32(bf16x2_mag_max(p01), bf16x2_mag_max(p23)));
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (feat + u < nh) {
                        o[u] = (uint16_t)hb[u];
                        m = umax32(m, hb[u] & 0x7FFFu);
                    }
            }
        }
    }
    *need = nd;
    *mx = m;
}

// Epilogue of a 256 x 256 tile: acc scaled by ca; SwiGLU to bf16 or plain
// fp32 / bf16 stores, four consecutive features per lane.
// Returns the largest |h| the thread stored (SwiGLU; else 0).
template <int kEpi>
__device__ __forceinline__ uint32_t epilogue(const GemmArgs& g, const f32x16 acc[4][2], float ca,
                                             int m0, int mend, int f0, int wm, int wn, int mact,
                                             int lane) {
    constexpr bool swiglu = kEpi == QUADS_EPI_SWIGLU;
    if (swiglu) {
        // rare: a gate below -44.36 somewhere in the wave's tile -- the same
        // outputs again with the full form (equal values elsewhere)
        bool need;
        uint32_t m;
        swiglu_store<false>(g, acc, ca, m0, mend, f0, wm, wn, mact, lane, &need, &m);
        if (__ballot(need) != 0ull)
            swiglu_store<true>(g, acc, ca, m0, mend, f0, wm, wn, mact, lane, &need, &m);
        return m;
    }
    const int prow_l = m0 + wm * 128 + (lane & 31);
    const int nq = 4 * (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi >= mact) continue;
        const int prow = prow_l + mi * 32;
        if (prow >= mend) continue;
        const float ca_row = row_scale(g, prow, ca);
#pragma unroll
        for (int q = 0; q < 4; ++q) {                 // registers 4q .. 4q + 3
            {
#pragma unroll
                for (int nj = 0; nj < 2; ++nj) {
                    const int n = f0 + wn * 64 + nj * 32 + 8 * q + nq;  // features n .. n + 3
                    float y[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) y[u] = acc[mi][nj][4 * q + u] * ca_row;
                    const int64_t o = (int64_t)prow * g.N + n;
                    const bool vec = n + 3 < g.N && (g.N & 3) == 0;
                    if (g.out_bf16) {
                        uint16_t* ob = (uint16_t*)g.out + o;
                        const uint32_t p01 = pk_bf16(y[0], y[1]), p23 = pk_bf16(y[2], y[3]);
                        if (vec) {
                            *reinterpret_cast<uint2*>(ob) = make_uint2(p01, p23);
                        } else {
                            const uint32_t b4[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu,
                                                    p23 >> 16};
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                if (n + u < g.N) ob[u] = (uint16_t)b4[u];
                        }
                    } else {
                        float* of = (float*)g.out + o;
                        if (vec) {
                            *reinterpret_cast<float4*>(of) = make_float4(y[0], y[1], y[2], y[3]);
                        } else {
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                if (n + u < g.N) of[u] = y[u];
                        }
                    }
                }
            }
        }
    }
    return 0u;
}


// Weight row of B-tile row r.  Plain: f0 + r.  SwiGLU: the tile holds 128
// output features; in each wave's 64 rows, rows 0-31 are gate and 32-63 up
// for the same 32 features.
__device__ __forceinline__ int w_row_v2(int r, int f0, int N, bool swiglu, bool* valid) {
    if (!swiglu) {
        const int n = f0 + r;
        *valid = n < N;
        return n;
    }
    const int feat = f0 + (r >> 6) * 32 + (r & 31);
    *valid = feat < N / 2;
    return ((r >> 5) & 1) * (N / 2) + feat;
}

}  // namespace v2

// Grouped GEMM for experts with few rows (gemm_decode.hip): used when K is a
// multiple of 128, k <= 64 and there are at most kDecodeRowsPerExpert packed
// rows per expert on average; it takes the experts with at most
// kDecodeMaxRows rows, the tiled kernel the others.  With at most
// kDecodeAllRows packed rows in all (a decode step of up to 64 tokens at
// top-8, where distinct routes give an expert at most 64 rows) it takes every
// expert, so that the tiled kernel is not launched only to find no expert
// above kDecodeMaxRows rows; an expert that still holds more (routes that
// repeat an expert within a token, or top-1 routing) is then split into
// work-groups of at most kDecodeMaxRows rows.
constexpr int kDecodeRowsPerExpert = 32;
// Channels after which every GEMM kernel restarts its MFMA accumulators and
// adds them into separate fp32 totals: gfx950's f16 MFMA rounds once per group
// of 8 products, so a chain of at most 1024 channels is 128 roundings.
constexpr int kAccChain = 1024;
// A single accumulator chain of at most this many channels (main product and
// compensation together) stays within 1e-5 sum|a w|: at most 144 group
// roundings plus the in-group truncation and the scaling roundings, (144 + 14
// + 4) 2^-24 < 9.7e-6.  The 256 x 256-tile kernel (one chain) serves those
// shapes; longer ones go to the kernels with split accumulation.
constexpr int kSingleChainMax = 1152;
// Tiled kernel for many rows per expert (gemm_v3.hip): K a multiple of 128,
// at most kCapMaxV3 compensation channels.
constexpr int kCapMaxV3 = 256;
// The launches of one GEMM call.  `dry`: count their work-groups without
// launching; otherwise each launch takes the next `blocks` as its
// GemmArgs::amax_base (the partial-maximum slots of the call, in launch
// order) and adds its work-group count.
struct LaunchPlan {
    bool dry;
    int64_t blocks;
};
bool gemm_v3_fits(const GemmArgs& g);
int launch_gemm_v3(GemmArgs g, hipStream_t st, LaunchPlan* lp);
// Long chains with k above kCapMaxV3 (k % 128 == 0, one shared selection):
// the tiled kernel with W[:, S] gathered into `ws` (gemm_v3_gather_ws bytes).
size_t gemm_v3_gather_ws(int64_t K, int64_t k, int64_t E, int64_t N);
bool gemm_v3_gather_fits(const GemmArgs& g);
int launch_gemm_v3_gather(GemmArgs g, void* ws, hipStream_t st, LaunchPlan* lp);
constexpr int kDecodeMaxRows = 128;
constexpr int kDecodeAllRows = 512;
bool gemm_decode_fits(const GemmArgs& g);
bool gemm_decode_tail_fits(const GemmArgs& g);
int launch_gemm_decode(GemmArgs g, hipStream_t st, LaunchPlan* lp);
// Tail rows the decode kernel takes from experts just above 256 rows.
constexpr int kTailRows = 64;

}  // namespace quads
