// NVFP4 quantization of bf16 tensors: activation quantizer Q_A (Eq. (9)) and
// the shared weight QDQ Q_W (Eq. (7), (12)) of arXiv 2607.15810, with the
// format of its section 2.2.
//
// Two passes over the tensor: a partial-max pass (one value per work-group)
// and the quantize pass.  The partial maxima give the tensor scale, and the
// scale the per-tensor table of element-code thresholds for all 127
// block-scale codes: for one activation tensor every quantize work-group
// does this itself; for the per-expert weight tensors one work-group per
// expert does it in a launch of its own.  The quantize pass
// streams half-blocks: one 16-byte load per lane (a wave reads 1 KB
// contiguous), the block maximum shared with the neighbouring lane, one
// 4-byte nibble store, one scale byte per block.
#include "common.h"

namespace quads {

// Max of |x| (as bf16 bit patterns) over segment blockIdx.y of seg_elems
// elements; one result per work-group into partial[blockIdx.y * gridDim.x + x].
// `clear` (optional): nclear words zeroed by the first segment's work-groups
// (counters of a kernel that runs after this one on the same stream).
__global__ __launch_bounds__(256) void k_amax_partial(const uint16_t* __restrict__ x,
                                                      int64_t seg_elems,
                                                      uint32_t* __restrict__ partial,
                                                      uint32_t* __restrict__ clear, int nclear) {
    if (blockIdx.y == 0)
        for (int i = blockIdx.x * 256 + threadIdx.x; i < nclear; i += gridDim.x * 256) clear[i] = 0u;
    const int64_t nvec = seg_elems / 8;
    const uint4* v = reinterpret_cast<const uint4*>(x + (int64_t)blockIdx.y * seg_elems);
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    // two vectors requested before either is used: a thread's loads are in
    // flight together rather than one memory latency each (dynamic-scale
    // quantizer, us at 16384 x 4096 / 131072 x 1536: two 55.9 / 150.2, four
    // 57.5 / 158.5, eight 60.0 / 172.3)
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + stride < nvec; i += 2 * stride) {
        uint4 q[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) q[u] = ld_stream16(v + i + u * stride);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            m = pk_max_u16(m, q[u].x & 0x7FFF7FFFu);
            m = pk_max_u16(m, q[u].y & 0x7FFF7FFFu);
            m = pk_max_u16(m, q[u].z & 0x7FFF7FFFu);
            m = pk_max_u16(m, q[u].w & 0x7FFF7FFFu);
        }
    }
    for (; i < nvec; i += stride) {
        uint4 q = ld_stream16(v + i);
        m = pk_max_u16(m, q.x & 0x7FFF7FFFu);
        m = pk_max_u16(m, q.y & 0x7FFF7FFFu);
        m = pk_max_u16(m, q.z & 0x7FFF7FFFu);
        m = pk_max_u16(m, q.w & 0x7FFF7FFFu);
    }
    uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    m = wave_max_u32(lo > hi ? lo : hi);
    __shared__ uint32_t s_w[4];
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = s_w[0];
        for (int i = 1; i < 4; ++i) r = s_w[i] > r ? s_w[i] : r;
        partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = r;
    }
}

// Tensor scale and code table of segment blockIdx.x, once per tensor:
// s_t = RN32(max|x| / 2688) from the partial maxima (or the caller's fixed
// scale), then the 127-row code table (see build_table_row).
__global__ __launch_bounds__(128) void k_scale_finalize(const uint32_t* __restrict__ partial,
                                                        int groups, const float* __restrict__ ts_in,
                                                        float* __restrict__ ts_out,
                                                        uint32_t* __restrict__ table) {
    __shared__ float s_st;
    __shared__ uint32_t s_red[2];
    const int seg = blockIdx.x;
    tensor_scale_prologue(partial, groups, ts_in, seg, &s_st, s_red);
    __syncthreads();
    const float s_t = s_st;
    if (threadIdx.x == 0) ts_out[seg] = s_t;
    build_threshold_table(s_t, reinterpret_cast<uint32_t(*)[8]>(table + (int64_t)seg * 1024),
                          true);
}

// half-blocks per batch per lane (two batches in flight).  Given-scale pass,
// us at 16384 x 4096 / 131072 x 1536, grid at the resident count: 1: 33.6 /
// 90.2, 2: 33.0 / 88.1, 3: 34.7 / 91.4, 4: 35.7 / 94.3, 8: 35.4 / 91.6; at 2,
// half or a quarter of that grid is slower
constexpr int kQuantUnroll = 2;

// Half-block h (8 elements) of a segment, the other half on the neighbouring
// lane (h ^ 1): block maximum by one shuffle, then codes (4 bytes), the
// block's scale byte (even lane) and the optional bf16 QDQ (16 bytes).
template <bool kDq>
__device__ __forceinline__ void quantize_half(const uint4 q, int64_t h, float s_t, double six_st,
                                              float inv6st, bool fast_sc, const uint32_t* thr2,
                                              const uint4* s_tab, uint8_t* ns, uint8_t* ss,
                                              uint16_t* ds) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t am = pk_max_u16(pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                             pk_max_u16(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
    am = (am & 0xFFFFu) > (am >> 16) ? (am & 0xFFFFu) : (am >> 16);
    const uint32_t o = lane_xor1(am);
    am = o > am ? o : am;
    const uint32_t sb = !(s_t > 0.0f) ? 0u
                        : fast_sc     ? scale_code_thr(am, inv6st, thr2)
                                      : e4m3_rne_code((double)bf16_to_f32(am) / six_st);
    const uint4 t1 = s_tab[2 * sb + 1];                       // word 7: fast-path multiplier
    uint32_t codes = 0u;
    if (t1.w != kSlowPath) {
        const float mul = __uint_as_float(t1.w);
#define QUADS_ENC_HALF(e, sel)                                                          \
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, __uint_as_float(w[e] << 16) * mul, \
                                                     __uint_as_float(w[e] & 0xFFFF0000u) * mul, \
                                                     1.0f, sel)
        QUADS_ENC_HALF(0, 0); QUADS_ENC_HALF(1, 1); QUADS_ENC_HALF(2, 2); QUADS_ENC_HALF(3, 3);
#undef QUADS_ENC_HALF
    } else {
        const uint4 t0 = s_tab[2 * sb];
        const uint32_t thr[7] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t hb = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            codes |= (e2m1_mag_code((hb & 0x7FFFu) << 16, thr) | ((hb >> 12) & 8u)) << (4 * e);
        }
    }
    *reinterpret_cast<uint32_t*>(ns + h * 4) = codes;
    if ((h & 1) == 0) ss[h >> 1] = (uint8_t)sb;
    if (kDq) {
        const float s_b = e4m3_value(sb);
        float v[8];
        decode8(codes, v);
        uint32_t ob[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const uint32_t r0 = bf16_rne_from_f64((double)(v[e] * s_b) * (double)s_t);
            const uint32_t r1 = bf16_rne_from_f64((double)(v[e + 1] * s_b) * (double)s_t);
            ob[e >> 1] = r0 | (r1 << 16);                    // v*s_b exact; product exact
        }
        *reinterpret_cast<uint4*>(ds + h * 8) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
    }
}

// kFold: one segment; every work-group takes the tensor scale (the caller's
// `ts_in`, or the fold of the partial maxima in `table`) and builds the code
// table itself, so no finalize launch runs before it; work-group 0 writes the
// scale to `ts`.  Otherwise the table and the scale come from
// k_scale_finalize (the per-expert weight tensors).
//
// Lane i of a wave reads 16 contiguous bytes (a wave: 1 KB); the two lanes of
// a block are neighbours.  A thread takes kQuantUnroll half-blocks per batch
// (`stride` apart) and keeps two batches in registers: the first is
// requested before the table set-up, and each next one before the current
// one is encoded, so a work-group's loads never wait on its own set-up or
// encoding.  A lane and its neighbour are both in range or both out (the
// half-block count is even).
template <bool kDq>
__device__ __forceinline__ void quant_load_batch(uint4 (&q)[kQuantUnroll], const uint16_t* xs,
                                                 int64_t h0, int64_t stride, int64_t nhalf) {
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
        const int64_t h = h0 + u * stride;
        q[u] = ld_stream16(xs + (h < nhalf ? h : 0) * 8);
    }
}

template <bool kDq, bool kFold = false>
__global__ __launch_bounds__(256) void k_quantize_bf16(
    const uint16_t* __restrict__ x, int64_t seg_elems, float* __restrict__ ts,
    const uint32_t* __restrict__ table, uint8_t* __restrict__ nib, uint8_t* __restrict__ scale,
    uint16_t* __restrict__ dq, int groups = 0, const float* __restrict__ ts_in = nullptr) {
    __shared__ uint4 s_tab[2 * (kE4m3MaxCode + 1)];
    __shared__ uint32_t s_thr2[kE4m3MaxCode + 1];
    const int seg = blockIdx.y;
    const int64_t nhalf = seg_elems / 8;                      // even: whole blocks
    const uint16_t* xs = x + (int64_t)seg * seg_elems;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t step = kQuantUnroll * stride;
    int64_t h0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint4 qa[kQuantUnroll], qb[kQuantUnroll];
    quant_load_batch<kDq>(qa, xs, h0, stride, nhalf);

    float s_t;
    if (kFold) {
        __shared__ float s_st;
        __shared__ uint32_t s_red[4];
        tensor_scale_prologue(table, groups, ts_in, 0, &s_st, s_red);
        __syncthreads();
        s_t = s_st;
        build_threshold_table(s_t, reinterpret_cast<uint32_t(*)[8]>(s_tab), true);
        if (blockIdx.x == 0 && threadIdx.x == 0) ts[0] = s_t;
    } else {
        const uint4* tg = reinterpret_cast<const uint4*>(table + (int64_t)seg * 1024);
        for (int i = threadIdx.x; i < 2 * (kE4m3MaxCode + 1); i += blockDim.x) s_tab[i] = tg[i];
        s_t = ts[seg];
    }
    // block-scale thresholds (exact codes from an fp32 quotient estimate) for
    // s_t >= 2^-100; below that the fp64 division
    const bool fast_sc = s_t >= 0x1p-100f;
    const float inv6st = fast_sc ? (float)(1.0 / (6.0 * (double)s_t)) : 0.0f;
    if (fast_sc) build_scale_thresholds(s_t, s_thr2);
    __syncthreads();

    uint8_t* ns = nib + (int64_t)seg * (seg_elems / 2);
    uint8_t* ss = scale + (int64_t)seg * (seg_elems / kBlock);
    uint16_t* ds = kDq ? dq + (int64_t)seg * seg_elems : nullptr;
    const double six_st = 6.0 * (double)s_t;                  // exact
    auto encode = [&](const uint4 (&q)[kQuantUnroll], int64_t hb) {
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t h = hb + u * stride;
            if (h < nhalf)
                quantize_half<kDq>(q[u], h, s_t, six_st, inv6st, fast_sc, s_thr2, s_tab, ns, ss,
                                   ds);
        }
    };
    while (h0 < nhalf) {
        int64_t hn = h0 + step;
        if (hn < nhalf) quant_load_batch<kDq>(qb, xs, hn, stride, nhalf);
        encode(qa, h0);
        h0 = hn;
        if (h0 >= nhalf) break;
        hn = h0 + step;
        if (hn < nhalf) quant_load_batch<kDq>(qa, xs, hn, stride, nhalf);
        encode(qb, h0);
        h0 = hn;
    }
}

// Per-row variant: one wave per row, the row's own tensor scale.  Lane l
// takes half-blocks l, l + 64, ... of the row (8 elements each; the other half
// of its block is on lane l ^ 1): a max pass over the row, then the block
// scale from the pair's maximum and the exact threshold compares.
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t* __restrict__ x,
                                                       int64_t M, int K,
                                                       uint8_t* __restrict__ nib,
                                                       uint8_t* __restrict__ scale,
                                                       float* __restrict__ ts) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;                            // whole wave
    const int nh = K / 8;                            // half-blocks in the row
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
    uint32_t m = 0;
    for (int hb = lane; hb < nh; hb += 64) {
        const uint4 q = xr[hb];
        m = pk_max_u16(m, q.x & 0x7FFF7FFFu);
        m = pk_max_u16(m, q.y & 0x7FFF7FFFu);
        m = pk_max_u16(m, q.z & 0x7FFF7FFFu);
        m = pk_max_u16(m, q.w & 0x7FFF7FFFu);
    }
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    const uint32_t am_row = wave_max_u32(lo > hi ? lo : hi);
    const float s_t = tensor_scale_from_amax(bf16_to_f32(am_row));
    if (lane == 0) ts[row] = s_t;
    const double six_st = 6.0 * (double)s_t;                     // exact
    // nh is even, so a lane and its pair partner are both in range or both out
    for (int hb0 = 0; hb0 < nh; hb0 += 64) {
        const int hb = hb0 + lane;
        const bool live = hb < nh;
        const uint4 q = xr[live ? hb : 0];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        uint32_t am = pk_max_u16(pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                                 pk_max_u16(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
        am = (am & 0xFFFFu) > (am >> 16) ? (am & 0xFFFFu) : (am >> 16);
        const uint32_t o = __shfl_xor(am, 1, 64);
        am = o > am ? o : am;
        const uint32_t sb = s_t > 0.0f ? e4m3_rne_code((double)bf16_to_f32(am) / six_st) : 0u;
        uint32_t thr[7];
        e2m1_thresholds(e4m3_value(sb), s_t, thr);
        uint32_t codes = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t hbits = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            codes |= (e2m1_mag_code((hbits & 0x7FFFu) << 16, thr) | ((hbits >> 12) & 8u)) << (4 * e);
        }
        if (live) {
            *reinterpret_cast<uint32_t*>(nib + row * (K / 2) + (int64_t)hb * 4) = codes;
            if ((hb & 1) == 0) scale[row * (K / kBlock) + hb / 2] = (uint8_t)sb;
        }
    }
}

__global__ void k_fill_f32(float* p, int n, float v) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

void launch_amax_partial(const uint16_t* x, int64_t seg_elems, int nseg, uint32_t* partial,
                         int groups, hipStream_t s, uint32_t* clear, int nclear) {
    hipLaunchKernelGGL(k_amax_partial, dim3(groups, nseg), dim3(256), 0, s, x, seg_elems, partial,
                       clear, nclear);
}

void launch_scale_finalize(const uint32_t* partial, int groups, const float* ts_in, int nseg,
                           float* ts_out, uint32_t* table, hipStream_t s) {
    hipLaunchKernelGGL(k_scale_finalize, dim3(nseg), dim3(128), 0, s, partial, groups, ts_in,
                       ts_out, table);
}

void launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
    if (n > 0)
        hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p,
                           (int)n, v);
}

// Work-groups of 256 threads of `kernel` the current device holds at once
// (the occupancy query, once per kernel and device; 2048 if it fails).
template <typename F>
int resident_groups(F kernel) {
    static int cached[16] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 2048;
    if (cached[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            per_cu < 1 || cus < 1)
            return 2048;
        cached[dev] = per_cu * cus;
    }
    return cached[dev];
}

int quant_grid(int64_t nblk) {
    int64_t g = (2 * nblk + 256 * kQuantUnroll - 1) / (256 * kQuantUnroll);  // half-blocks
    if (g > 8192) g = 8192;
    return (int)(g < 1 ? 1 : g);
}

}  // namespace quads

using namespace quads;

// Workspace: partial maxima (kAmaxGroups words) then the code table (1024
// words) per segment.
static size_t quant_ws_bytes(int64_t nseg) {
    return align_up((size_t)nseg * kAmaxGroups * 4, 256) + align_up((size_t)nseg * 1024 * 4, 256);
}

extern "C" size_t quads_nvfp4_quantize_ws(int64_t M, int64_t K) {
    (void)M; (void)K;
    return quant_ws_bytes(1);
}

extern "C" int quads_nvfp4_quantize(const uint16_t* x, int64_t M, int64_t K, const float* ts_in,
                                    uint8_t* nib, uint8_t* scale, float* ts_out, void* ws,
                                    size_t ws_bytes, void* stream) {
    if (M < 0 || K <= 0 || K % kBlock) return QUADS_ESHAPE;
    if (!ok_ptr(ts_out) || !ok_opt_ptr(ts_in)) return QUADS_EINVAL;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(nib) || !ok_ptr(scale))) return QUADS_EINVAL;
    if (ws_bytes < quads_nvfp4_quantize_ws(M, K) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {
        hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(64), 0, s, ts_out, 1, 0.0f);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    const int64_t n = M * K;
    uint32_t* partial = static_cast<uint32_t*>(ws);
    if (!ts_in) {
        // dynamic scale: the partial maxima, then the quantize pass folds
        // them itself, with at most one work-group per resident slot (2048 =
        // 8 per CU) so that the per-work-group table build is paid once
        const int groups = amax_groups(n);
        hipLaunchKernelGGL(k_amax_partial, dim3(groups, 1), dim3(256), 0, s, x, n, partial,
                           (uint32_t*)nullptr, 0);
        QUADS_CHECK_LAUNCH();
        const int qg = quant_grid(n / kBlock), qr = resident_groups(k_quantize_bf16<false, true>);
        hipLaunchKernelGGL((k_quantize_bf16<false, true>), dim3(qg < qr ? qg : qr, 1),
                           dim3(256), 0, s, x, n, ts_out, partial, nib, scale, (uint16_t*)nullptr,
                           groups);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    // the caller's scale: one launch, every work-group building the table
    const int qg = quant_grid(n / kBlock), qr = resident_groups(k_quantize_bf16<false, true>);
    hipLaunchKernelGGL((k_quantize_bf16<false, true>), dim3(qg < qr ? qg : qr, 1), dim3(256), 0, s,
                       x, n, ts_out, partial, nib, scale, (uint16_t*)nullptr, 0, ts_in);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}

// The dynamic-scale quantizer with max|x| from a producer's partial maxima
// (bf16 magnitude bits, e.g. quads_moe_w4a4_gemm_amax): one launch, every
// work-group folding them into the tensor scale itself.
extern "C" int quads_nvfp4_quantize_partials(const uint16_t* x, int64_t M, int64_t K,
                                             const uint32_t* amax_part, int64_t groups,
                                             uint8_t* nib, uint8_t* scale, float* ts_out,
                                             void* stream) {
    if (M < 0 || K <= 0 || K % kBlock) return QUADS_ESHAPE;
    if (groups < 1 || groups >= ((int64_t)1 << 31)) return QUADS_ESHAPE;
    if (!ok_ptr(ts_out) || !ok_ptr4(amax_part)) return QUADS_EINVAL;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(nib) || !ok_ptr(scale))) return QUADS_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {
        hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(64), 0, s, ts_out, 1, 0.0f);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    const int64_t n = M * K;
    const int qg = quant_grid(n / kBlock), qr = resident_groups(k_quantize_bf16<false, true>);
    hipLaunchKernelGGL((k_quantize_bf16<false, true>), dim3(qg < qr ? qg : qr, 1), dim3(256), 0, s,
                       x, n, ts_out, amax_part, nib, scale, (uint16_t*)nullptr, (int)groups);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}

extern "C" int quads_nvfp4_quantize_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* nib,
                                         uint8_t* scale, float* ts, void* stream) {
    if (M < 0 || K <= 0 || K % kBlock || K >= ((int64_t)1 << 30)) return QUADS_ESHAPE;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(nib) || !ok_ptr(scale) || !ok_ptr(ts)))
        return QUADS_EINVAL;
    if (M == 0) return QUADS_OK;
    if ((M + 3) / 4 > 0x7FFFFFFF) return QUADS_ESHAPE;           // grid of M / 4 work-groups
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)((M + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, x, M, (int)K, nib, scale, ts);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}

extern "C" size_t quads_nvfp4_weight_qdq_ws(int64_t E, int64_t N, int64_t K) {
    (void)N; (void)K;
    if (E < 1) return 0;
    return quant_ws_bytes(E);
}

extern "C" int quads_nvfp4_weight_qdq(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                                      uint8_t* w_nib, uint8_t* w_scale, float* w_ts,
                                      uint16_t* w_dq, void* ws, size_t ws_bytes, void* stream) {
    if (E < 1 || E > 65535 || N < 0 || K <= 0 || K % kBlock) return QUADS_ESHAPE;
    if (!ok_ptr(w_ts) || !ok_opt_ptr(w_dq)) return QUADS_EINVAL;
    if (N > 0 && (!ok_ptr(w) || !ok_ptr(w_nib) || !ok_ptr(w_scale))) return QUADS_EINVAL;
    if (ws_bytes < quads_nvfp4_weight_qdq_ws(E, N, K) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (N == 0) {
        hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, w_ts,
                           (int)E, 0.0f);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    const int64_t n = N * K;
    int groups = amax_groups(n);
    uint32_t* partial = static_cast<uint32_t*>(ws);
    uint32_t* table = partial + align_up((size_t)E * kAmaxGroups * 4, 256) / 4;
    hipLaunchKernelGGL(k_amax_partial, dim3(groups, (unsigned)E), dim3(256), 0, s, w, n, partial,
                       (uint32_t*)nullptr, 0);
    QUADS_CHECK_LAUNCH();
    launch_scale_finalize(partial, groups, nullptr, (int)E, w_ts, table, s);
    QUADS_CHECK_LAUNCH();
    int64_t qg = quant_grid(n / kBlock);
    int64_t cap = (4096 + E - 1) / E;
    if (qg > cap) qg = cap < 1 ? 1 : cap;
    if (w_dq)
        hipLaunchKernelGGL(k_quantize_bf16<true>, dim3((unsigned)qg, (unsigned)E), dim3(256), 0, s,
                           w, n, w_ts, table, w_nib, w_scale, w_dq);
    else
        hipLaunchKernelGGL(k_quantize_bf16<false>, dim3((unsigned)qg, (unsigned)E), dim3(256), 0,
                           s, w, n, w_ts, table, w_nib, w_scale, w_dq);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}
