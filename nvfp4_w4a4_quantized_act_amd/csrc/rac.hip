// Residual Activation Compensation (arXiv 2607.15810, section 3.3).
//
//  pass 1  (one 64-token x 64-channel tile per work-group): NVFP4 of x as in
//          the quantizer, the fp32 residual r = x - DQ(Q(x)) (Eq. (20), sign
//          flipped) with one fused multiply-add, then per channel the
//          in-order fp64 sum of r^2 over the tile's 64 tokens and max |r|.
//  levels  the 64-ary fixed-order tree over those per-tile partials, one
//          launch per level, until one score per channel is left (Eq. (23)).
//  select  one work-group: radix select of the k largest scores (Eq. (24)),
//          ties to the lower index, written ascending; the tensor scale of
//          the gathered residual from the per-channel maxima.
//  pass 2  gathers r[:, S] (recomputed from x, the codes and the block
//          scales of pass 1) and NVFP4-quantizes it in 16-blocks along the
//          compacted index (the second term of Eq. (21)).
#include "common.h"

namespace quads {

constexpr int kTileRows = 64;          // == kScoreFanin: one level-0 group
constexpr int kTileCols = 64;
constexpr int kRacMaxK = 8192;         // channels handled by the select kernel

// ------------------------------------------------------------------ pass 1 --
__global__ __launch_bounds__(256) void k_rac_pass1(
    const uint16_t* __restrict__ x, int64_t M, int K, const uint32_t* __restrict__ partial,
    int groups, uint8_t* __restrict__ nib, uint8_t* __restrict__ scale, float* __restrict__ ts,
    double* __restrict__ p0, uint32_t* __restrict__ cm0) {
    __shared__ uint32_t s_thr[kE4m3MaxCode + 1][8];
    __shared__ double s_r2[kTileRows][kTileCols + 1];
    __shared__ uint32_t s_ra[kTileRows][kTileCols + 1];
    __shared__ float s_st;
    tensor_scale_prologue(partial, groups, nullptr, 0, &s_st);
    __syncthreads();
    const float s_t = s_st;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts[0] = s_t;
    build_threshold_table(s_t, s_thr);
    __syncthreads();

    const int rl = threadIdx.x >> 2;                 // tile row 0..63
    const int cb = threadIdx.x & 3;                  // 16-channel block in the tile
    const int64_t row = (int64_t)blockIdx.x * kTileRows + rl;
    const int c0 = blockIdx.y * kTileCols + cb * kBlock;
    float r[16];
    if (row < M && c0 < K) {
        const int64_t b = (row * K + c0) / kBlock;   // block index in the tensor
        const uint4* p = reinterpret_cast<const uint4*>(x + row * K + c0);
        uint4 q0 = ld_stream16(p);
        uint4 q1 = ld_stream16(p + 1);
        uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = pk_max_u16(am, w[i] & 0x7FFF7FFFu);
        uint32_t lo = am & 0xFFFFu, hi = am >> 16;
        const float amax_b = bf16_to_f32(lo > hi ? lo : hi);
        const uint32_t sb =
            s_t > 0.0f ? e4m3_rne_code((double)amax_b / (6.0 * (double)s_t)) : 0u;
        uint32_t thr[7];
        {
            uint4 t0 = *reinterpret_cast<const uint4*>(&s_thr[sb][0]);
            uint4 t1 = *reinterpret_cast<const uint4*>(&s_thr[sb][4]);
            thr[0] = t0.x; thr[1] = t0.y; thr[2] = t0.z; thr[3] = t0.w;
            thr[4] = t1.x; thr[5] = t1.y; thr[6] = t1.z;
        }
        const float s_b = e4m3_value(sb);
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const uint32_t mag = e2m1_mag_code((h & 0x7FFFu) << 16, thr);
            const uint32_t code = mag | ((h >> 12) & 8u);
            packed[e >> 3] |= code << (4 * (e & 7));
            float sv = e2m1_value(mag) * s_b;                      // exact
            if (code & 8u) sv = -sv;
            r[e] = fmaf(-sv, s_t, bf16_to_f32(h));                  // RN32(x - v s_b s_t)
        }
        *reinterpret_cast<uint2*>(nib + b * 8) = make_uint2(packed[0], packed[1]);
        scale[b] = (uint8_t)sb;
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) r[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const double rd = (double)r[e];
        s_r2[rl][cb * kBlock + e] = rd * rd;                         // exact
        s_ra[rl][cb * kBlock + e] = __float_as_uint(r[e]) & 0x7FFFFFFFu;
    }
    __syncthreads();
    const int col = threadIdx.x & 63;
    const int gc = blockIdx.y * kTileCols + col;
    if (threadIdx.x < 64) {
        double acc = 0.0;
        for (int i = 0; i < kTileRows; ++i) acc = acc + s_r2[i][col];   // token order
        if (gc < K) p0[(int64_t)blockIdx.x * K + gc] = acc;
    } else if (threadIdx.x < 128) {
        uint32_t m = 0;
        for (int i = 0; i < kTileRows; ++i) m = s_ra[i][col] > m ? s_ra[i][col] : m;
        if (gc < K) cm0[(int64_t)blockIdx.x * K + gc] = m;
    }
}

// ------------------------------------------------------------- tree level --
// out[g][c] = ((+0 + in[64g][c]) + in[64g+1][c]) + ...  (rows < n), and the
// max of the per-channel maxima alongside.
__global__ __launch_bounds__(256) void k_tree_level(const double* __restrict__ in,
                                                    const uint32_t* __restrict__ cin, int64_t n,
                                                    int K, double* __restrict__ out,
                                                    uint32_t* __restrict__ cout) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= K) return;
    const int64_t g = blockIdx.y;
    const int64_t r0 = g * kScoreFanin;
    const int64_t r1 = r0 + kScoreFanin < n ? r0 + kScoreFanin : n;
    double acc = 0.0;
    uint32_t m = 0;
    for (int64_t r = r0; r < r1; ++r) {
        acc = acc + in[r * K + c];
        const uint32_t v = cin[r * K + c];
        m = v > m ? v : m;
    }
    out[g * K + c] = acc;
    cout[g * K + c] = m;
}

// ----------------------------------------------------------------- select --
// Exclusive scan of one value per thread over a 1024-thread work-group.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* s_tmp, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tmp[wid] = x;
    __syncthreads();
    if (threadIdx.x < 16) {
        int w = s_tmp[threadIdx.x];
        int sum = w;
        for (int off = 1; off < 16; off <<= 1) {
            int y = __shfl_up(sum, off, 16);
            if ((int)threadIdx.x >= off) sum += y;
        }
        s_tmp[16 + threadIdx.x] = sum - w;       // exclusive wave offsets
        if (threadIdx.x == 15) s_tmp[32] = sum;
    }
    __syncthreads();
    const int res = x - v + s_tmp[16 + wid];
    *total = s_tmp[32];
    __syncthreads();
    return res;
}

__global__ __launch_bounds__(1024) void k_rac_select(const double* __restrict__ score,
                                                     const uint32_t* __restrict__ colmax, int K,
                                                     int k, int32_t* __restrict__ sel,
                                                     float* __restrict__ r_ts,
                                                     double* __restrict__ score_out) {
    __shared__ unsigned long long s_key[kRacMaxK];
    __shared__ int s_hist[256];
    __shared__ int s_tmp[40];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_need;
    __shared__ uint32_t s_amax[16];
    const int tid = threadIdx.x;
    for (int j = tid; j < K; j += 1024) {
        const double v = score[j];
        s_key[j] = (unsigned long long)__double_as_longlong(v);   // v >= +0: bits order
        if (score_out) score_out[j] = v;
    }
    if (tid == 0) { s_prefix = 0ull; s_need = k; }
    __syncthreads();
    // MSB-first radix select of the k-th largest key, 8 bits per pass.
    unsigned long long mask = 0ull;
    for (int shift = 56; shift >= 0; shift -= 8) {
        if (tid < 256) s_hist[tid] = 0;
        __syncthreads();
        const unsigned long long prefix = s_prefix;
        for (int j = tid; j < K; j += 1024) {
            const unsigned long long key = s_key[j];
            if ((key & mask) == prefix) atomicAdd(&s_hist[(int)((key >> shift) & 0xFF)], 1);
        }
        __syncthreads();
        if (tid == 0) {
            int need = s_need, d = 255;
            for (; d > 0; --d) {
                if (s_hist[d] >= need) break;
                need -= s_hist[d];
            }
            s_need = need;
            s_prefix = prefix | ((unsigned long long)d << shift);
        }
        mask |= 0xFFull << shift;
        __syncthreads();
    }
    const unsigned long long thr = s_prefix;    // the k-th largest key
    const int need_ties = s_need;               // how many keys equal to thr to take
    // ties at thr in index order: rank among equal keys via a chunked scan
    const int per = (K + 1023) / 1024;
    const int j0 = tid * per;
    const int j1 = j0 + per < K ? j0 + per : K;
    int n_eq = 0;
    for (int j = j0; j < j1; ++j) n_eq += s_key[j] == thr;
    int total;
    int eq_before = block_excl_scan_1024(n_eq, s_tmp, &total);
    int n_sel = 0;
    {
        int e = eq_before;
        for (int j = j0; j < j1; ++j) {
            const unsigned long long key = s_key[j];
            if (key > thr || (key == thr && e++ < need_ties)) ++n_sel;
        }
    }
    int sel_before = block_excl_scan_1024(n_sel, s_tmp, &total);
    uint32_t am = 0;
    {
        int e = eq_before, o = sel_before;
        for (int j = j0; j < j1; ++j) {
            const unsigned long long key = s_key[j];
            if (key > thr || (key == thr && e++ < need_ties)) {
                sel[o++] = j;
                const uint32_t c = colmax[j];
                am = c > am ? c : am;
            }
        }
    }
    am = wave_max_u32(am);
    if ((tid & 63) == 0) s_amax[tid >> 6] = am;
    __syncthreads();
    if (tid == 0) {
        uint32_t m = 0;
        for (int i = 0; i < 16; ++i) m = s_amax[i] > m ? s_amax[i] : m;
        r_ts[0] = tensor_scale_from_amax(__uint_as_float(m));
    }
}

// ----------------------------------------------------------------- pass 2 --
// One thread per (row, 16-block of the compacted index).
__global__ __launch_bounds__(256) void k_rac_pass2(
    const uint16_t* __restrict__ x, int64_t M, int K, const int32_t* __restrict__ sel, int k,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ scale,
    const float* __restrict__ ts, const float* __restrict__ r_ts, uint8_t* __restrict__ r_nib,
    uint8_t* __restrict__ r_scale) {
    __shared__ uint32_t s_thr[kE4m3MaxCode + 1][8];
    __shared__ int s_sel[kRacMaxK];
    const float s_t = ts[0];
    const float s_tr = r_ts[0];
    build_threshold_table(s_tr, s_thr);
    for (int i = threadIdx.x; i < k; i += blockDim.x) s_sel[i] = sel[i];
    __syncthreads();
    const int kb = k / kBlock;
    const int64_t nblk = M * kb;
    const double six_str = 6.0 * (double)s_tr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nblk;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = t / kb;
        const int bi = (int)(t - row * kb);
        const uint16_t* xr = x + row * K;
        const uint8_t* nr = nib + row * (K / 2);
        const uint8_t* sr = scale + row * (K / kBlock);
        float r[16];
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = s_sel[bi * kBlock + e];
            const uint32_t h = xr[j];
            const uint32_t code = (nr[j >> 1] >> (4 * (j & 1))) & 0xFu;
            float sv = e2m1_value(code & 7u) * e4m3_value(sr[j >> 4]);
            if (code & 8u) sv = -sv;
            r[e] = fmaf(-sv, s_t, bf16_to_f32(h));
            const uint32_t ab = __float_as_uint(r[e]) & 0x7FFFFFFFu;
            am = ab > am ? ab : am;
        }
        const uint32_t sb =
            s_tr > 0.0f ? e4m3_rne_code((double)__uint_as_float(am) / six_str) : 0u;
        uint32_t thr[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) thr[i] = s_thr[sb][i];
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t rb = __float_as_uint(r[e]);
            const uint32_t code = e2m1_mag_code(rb & 0x7FFFFFFFu, thr) | ((rb >> 28) & 8u);
            packed[e >> 3] |= code << (4 * (e & 7));
        }
        *reinterpret_cast<uint2*>(r_nib + t * 8) = make_uint2(packed[0], packed[1]);
        r_scale[t] = (uint8_t)sb;
    }
}

__global__ void k_iota_i32(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = i;
}
__global__ void k_fill_f64(double* p, int n, double v) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

struct RacWs {
    uint32_t* partial;
    double* pa;
    uint32_t* ca;
    double* pb;
    uint32_t* cb;
    size_t bytes;
};

RacWs rac_ws_layout(char* base, int64_t M, int64_t K) {
    const int64_t c0 = (M + kTileRows - 1) / kTileRows;
    const int64_t c1 = (c0 + kScoreFanin - 1) / kScoreFanin;
    RacWs w;
    size_t off = 0;
    w.partial = (uint32_t*)(base + off); off += align_up(kAmaxGroups * 4, 256);
    w.pa = (double*)(base + off); off += align_up((size_t)(c0 > 1 ? c0 : 1) * K * 8, 256);
    w.ca = (uint32_t*)(base + off); off += align_up((size_t)(c0 > 1 ? c0 : 1) * K * 4, 256);
    w.pb = (double*)(base + off); off += align_up((size_t)c1 * K * 8, 256);
    w.cb = (uint32_t*)(base + off); off += align_up((size_t)c1 * K * 4, 256);
    w.bytes = off;
    return w;
}

}  // namespace quads

using namespace quads;

extern "C" size_t quads_rac_quantize_ws(int64_t M, int64_t K, int32_t k) {
    (void)k;
    if (M < 0 || K <= 0) return 0;
    return rac_ws_layout(nullptr, M, K).bytes;
}

extern "C" int quads_rac_quantize(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                  uint8_t* nib, uint8_t* scale, float* ts, int32_t* sel,
                                  uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                                  double* score_out, void* ws, size_t ws_bytes, void* stream) {
    if (M < 0 || K <= 0 || K % kBlock || K > kRacMaxK) return QUADS_ESHAPE;
    if (k < 0 || k % kBlock || k > K) return QUADS_ESHAPE;
    if (!ok_ptr(ts) || !ok_ptr(r_ts) || !ok_opt_ptr(score_out)) return QUADS_EINVAL;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(nib) || !ok_ptr(scale))) return QUADS_EINVAL;
    if (k > 0 && !ok_ptr(sel)) return QUADS_EINVAL;
    if (k > 0 && M > 0 && (!ok_ptr(r_nib) || !ok_ptr(r_scale))) return QUADS_EINVAL;
    if (ws_bytes < quads_rac_quantize_ws(M, K, k) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {
        launch_fill_f32(ts, 1, 0.0f, s);
        launch_fill_f32(r_ts, 1, 0.0f, s);
        if (k > 0) hipLaunchKernelGGL(k_iota_i32, dim3((k + 255) / 256), dim3(256), 0, s, sel, k);
        if (score_out)
            hipLaunchKernelGGL(k_fill_f64, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s,
                               score_out, (int)K, 0.0);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    RacWs w = rac_ws_layout((char*)ws, M, K);
    const int groups = amax_groups(M * K);
    launch_amax_partial(x, M * K, 1, w.partial, groups, s);
    QUADS_CHECK_LAUNCH();
    const int64_t c0 = (M + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL(k_rac_pass1, dim3((unsigned)c0, (unsigned)((K + kTileCols - 1) / kTileCols)),
                       dim3(256), 0, s, x, M, (int)K, w.partial, groups, nib, scale, ts, w.pa,
                       w.ca);
    QUADS_CHECK_LAUNCH();
    // fixed-order tree over the level-0 partials
    double* pin = w.pa; uint32_t* cin = w.ca;
    double* pout = w.pb; uint32_t* cout = w.cb;
    int64_t n = c0;
    while (n > 1) {
        const int64_t g = (n + kScoreFanin - 1) / kScoreFanin;
        hipLaunchKernelGGL(k_tree_level, dim3((unsigned)((K + 255) / 256), (unsigned)g), dim3(256),
                           0, s, pin, cin, n, (int)K, pout, cout);
        QUADS_CHECK_LAUNCH();
        n = g;
        double* tp = pin; pin = pout; pout = tp;
        uint32_t* tc = cin; cin = cout; cout = tc;
    }
    if (k == 0 && score_out == nullptr) {
        launch_fill_f32(r_ts, 1, 0.0f, s);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    hipLaunchKernelGGL(k_rac_select, dim3(1), dim3(1024), 0, s, pin, cin, (int)K, (int)k, sel,
                       r_ts, score_out);
    QUADS_CHECK_LAUNCH();
    if (k > 0) {
        const int64_t nblk = M * (k / kBlock);
        int64_t grid = (nblk + 255) / 256;
        if (grid > 4096) grid = 4096;
        hipLaunchKernelGGL(k_rac_pass2, dim3((unsigned)grid), dim3(256), 0, s, x, M, (int)K, sel,
                           (int)k, nib, scale, ts, r_ts, r_nib, r_scale);
        QUADS_CHECK_LAUNCH();
    } else {
        launch_fill_f32(r_ts, 1, 0.0f, s);
        QUADS_CHECK_LAUNCH();
    }
    return QUADS_OK;
}
