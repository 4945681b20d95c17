// Residual Activation Compensation (arXiv 2607.15810, section 3.3).
//
//  max     partial maxima of |x| (the quantizer's pass).
//  pass 1  every work-group folds the partial maxima into the tensor scale
//          and builds the code table in LDS (as the quantizer's finalize step
//          does once), then (64-token x 256-channel tiles; a work-group walks
//          several token chunks of one channel slice) NVFP4 of x as in the
//          quantizer, the fp32 residual r = x - DQ(Q(x)) (Eq. (20), sign
//          flipped) with one fused multiply-add, staged in LDS, then per
//          channel the in-order fp64 sum of r^2 over the chunk's 64 tokens and
//          max |r|.
//  levels  the 64-ary fixed-order tree over those per-tile partials, one
//          launch per level, until at most 16 partial rows per channel are
//          left (Eq. (23)); none when neither S nor the scores are wanted.
//  select  one work-group: the tree's last level (at most 16 rows, summed in
//          order), then radix select of the k largest scores (Eq. (24)),
//          ties to the lower index, written ascending; the tensor scale of
//          the gathered residual from the per-channel maxima, and its code
//          table (exact compare path: the residual is fp32, not bf16).
//  pass 2  one thread per element of r[:, S] (recomputed from x, the codes
//          and the block scales of pass 1), NVFP4-quantized in 16-blocks along
//          the compacted index (the second term of Eq. (21)).
#include <mutex>

#include "common.h"

namespace quads {

constexpr int kTileRows = 64;          // == kScoreFanin: one level-0 group
constexpr int kRacMaxK = 8192;         // channels handled by the select kernel
constexpr int kSelectFold = 16;        // partial rows the select kernel sums itself

// ------------------------------------------------------------------ pass 1 --
// Tile: 64 tokens x 256 channels.  Thread t quantizes 4 blocks (tile rows
// t/16 + 16 q, channel block t%16; the eight 16-byte loads issued together),
// keeps the fp32 residuals in LDS, then owns channel t of the tile for the
// in-order sum over the 64 tokens.
constexpr int kP1Cols = 256;

__global__ __launch_bounds__(256) void k_rac_pass1(
    const uint16_t* __restrict__ x, int64_t M, int K, const uint32_t* __restrict__ partial,
    int groups, float* __restrict__ ts, uint8_t* __restrict__ nib, uint8_t* __restrict__ scale,
    double* __restrict__ p0, uint32_t* __restrict__ cm0) {
    __shared__ __align__(16) uint32_t s_tab[kE4m3MaxCode + 2][8];
    __shared__ float s_r[kTileRows / 2][kP1Cols + 4];  // one half of the chunk at a time
    __shared__ float s_st;
    __shared__ uint32_t s_red[4];
    tensor_scale_prologue(partial, groups, nullptr, 0, &s_st, s_red);
    __syncthreads();
    const float s_t = s_st;
    build_threshold_table(s_t, s_tab, true);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts[0] = s_t;
    const double six_st = 6.0 * (double)s_t;
    __syncthreads();

    const int tid = threadIdx.x;
    const int cb = tid & 15;                          // 16-channel block in the tile
    const int c0 = blockIdx.y * kP1Cols + cb * kBlock;
    const int gc = blockIdx.y * kP1Cols + tid;
    const int64_t nchunk = (M + kTileRows - 1) / kTileRows;
    for (int64_t ch = blockIdx.x; ch < nchunk; ch += gridDim.x) {
        uint4 q0[4], q1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {                 // loads first, addresses clamped
            const int64_t row = ch * kTileRows + (tid >> 4) + 16 * q;
            const bool ok = row < M && c0 < K;
            const uint4* p = reinterpret_cast<const uint4*>(x + (ok ? row * K + c0 : 0));
            q0[q] = ld_stream16(p);
            q1[q] = ld_stream16(p + 1);
        }
        // the chunk's residuals in two halves of 32 rows (LDS of one half): the
        // per-channel sum continues over rows 0 .. 63 in order
        double acc = 0.0;
        uint32_t m = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int q = 2 * half + qq;
                const int rl = (tid >> 4) + 16 * q;   // row in the chunk
                const int64_t row = ch * kTileRows + rl;
                float r[16];
                if (row < M && c0 < K) {
                    const int64_t b = (row * K + c0) / kBlock;
                    const uint32_t w[8] = {q0[q].x, q0[q].y, q0[q].z, q0[q].w,
                                           q1[q].x, q1[q].y, q1[q].z, q1[q].w};
                    uint32_t am = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) am = pk_max_u16(am, w[i] & 0x7FFF7FFFu);
                    const uint32_t lo = am & 0xFFFFu, hi = am >> 16;
                    const float amax_b = bf16_to_f32(lo > hi ? lo : hi);
                    const uint32_t sb =
                        s_t > 0.0f ? e4m3_rne_code((double)amax_b / six_st) : 0u;
                    const uint4 t0 = *reinterpret_cast<const uint4*>(&s_tab[sb][0]);
                    const uint4 t1 = *reinterpret_cast<const uint4*>(&s_tab[sb][4]);
                    const uint2 packed = encode_block_bf16(w, t0, t1);
                    *reinterpret_cast<uint2*>(nib + b * 8) = packed;
                    scale[b] = (uint8_t)sb;
                    const float s_b = e4m3_value(sb);
                    float v[16];
                    decode8(packed.x, v);
                    decode8(packed.y, v + 8);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float xv =
                            __uint_as_float(e & 1 ? w[e >> 1] & 0xFFFF0000u : w[e >> 1] << 16);
                        r[e] = fmaf(-(v[e] * s_b), s_t, xv);  // RN32(x - v s_b s_t), v s_b exact
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) r[e] = 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 16; e += 4)
                    *reinterpret_cast<float4*>(&s_r[rl - 32 * half][cb * kBlock + e]) =
                        make_float4(r[e], r[e + 1], r[e + 2], r[e + 3]);
            }
            __syncthreads();
            if (p0 != nullptr) {                       // scores wanted
#pragma unroll 16
                for (int i = 0; i < kTileRows / 2; ++i) {     // token order
                    const float rv = s_r[i][tid];
                    const double rd = (double)rv;
                    acc = acc + rd * rd;                      // r^2 exact in fp64
                    const uint32_t ab = __float_as_uint(rv) & 0x7FFFFFFFu;
                    m = ab > m ? ab : m;
                }
            }
            __syncthreads();
        }
        if (p0 != nullptr && gc < K) {
            p0[ch * K + gc] = acc;
            cm0[ch * K + gc] = m;
        }
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
    if (r1 - r0 == kScoreFanin) {
        double v[kScoreFanin];
#pragma unroll
        for (int i = 0; i < kScoreFanin; ++i) v[i] = in[(r0 + i) * K + c];   // loads first
#pragma unroll
        for (int i = 0; i < kScoreFanin; ++i) acc = acc + v[i];              // then the chain
#pragma unroll 16
        for (int i = 0; i < kScoreFanin; ++i) {
            const uint32_t u = cin[(r0 + i) * K + c];
            m = u > m ? u : m;
        }
    } else {
        for (int64_t r = r0; r < r1; ++r) {
            acc = acc + in[r * K + c];
            const uint32_t u = cin[r * K + c];
            m = u > m ? u : m;
        }
    }
    out[g * K + c] = acc;
    cout[g * K + c] = m;
}

// ----------------------------------------------------------------- select --
// Exclusive scan of one value per thread over a work-group of kT threads
// with one barrier: DPP wave scans, the wave totals through s_tmp[0 .. kT/64)
// (its own buffer), and every wave adds up the totals before it itself.
template <int kT>
__device__ __forceinline__ int block_excl_scan_dpp(int v, int* s_tmp, int* total) {
    constexpr int kW = kT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int x = wave_incl_add(v);
    if (lane == 63) s_tmp[wid] = x;
    __syncthreads();
    const int w = lane < kW ? s_tmp[lane] : 0;
    const int incl = wave_incl_add(w);                  // over the wave totals
    *total = __builtin_amdgcn_readlane(incl, kW - 1);
    const int before = wid > 0 ? __builtin_amdgcn_readlane(incl, wid - 1) : 0;
    return x - v + before;
}

// Radix select of the k largest of K keys (K <= 8192; fp64 scores as bit
// patterns in LDS; ties to the lower index), by a work-group of kT threads: S
// into sel (ascending), and the tensor scale of the gathered residual, from
// the selected channels' maxima s_cmax, into *s_rts (LDS).
//
// Thread t holds keys t * per .. t * per + per - 1 in registers.  MSB-first
// passes of 8-bit digits: the histogram of the digit among the keys under
// the prefix chosen so far, then every wave reads the histogram and finds
// the digit where the count from the top reaches the number still needed,
// so the selection state stays in registers and a pass costs one barrier
// (three histogram buffers in turn: a pass clears the next pass's buffer,
// which every wave last read two passes ago, before the barrier it has
// passed since).  It stops once every key under the chosen prefix is
// needed (the selected set is then the keys whose prefix is greater plus
// all keys with that prefix), or once all 64 bits are chosen.  Of the keys
// equal to the prefix the first ones in index order are taken; when all of
// them are needed (the usual case) one scan of the per-thread selection
// counts places S, otherwise a scan of the equal keys comes first.  Scans
// and wave reductions run on DPP moves and scalar lane reads: the
// work-group's time is its chain of dependent steps.
template <int kT>
__device__ void select_keys(const unsigned long long* s_key, const uint32_t* s_cmax, int K, int k,
                            int32_t* __restrict__ sel, float* s_rts) {
    constexpr int kSelPer = kRacMaxK / kT;
    constexpr int kW = kT / 64;
    __shared__ int s_hist[3][256];
    __shared__ int s_tmp[2][16];
    __shared__ uint32_t s_amax[16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int per = (K + kT - 1) / kT;
    const int j0 = tid * per;
    for (int i = tid; i < 256; i += kT) {
        s_hist[0][i] = 0;
        s_hist[1][i] = 0;
    }
    __syncthreads();                            // s_key (the caller's) and the histograms
    unsigned long long key[kSelPer];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) key[u] = u < per && j0 + u < K ? s_key[j0 + u] : 0ull;
    unsigned long long prefix = 0ull, mask = 0ull;
    int need = k, eq = K, shift = 56, buf = 0;
    bool done = k == 0;
    while (!done) {                                            // uniform
        // histogram of the digit under the prefix.  The keys are scores of
        // one tensor, so in the first passes whole waves share one digit,
        // and LDS atomics on one bin would queue: such a wave adds its count
        // once; other waves add per lane.
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            if (u >= per) break;                               // uniform
            const bool in = j0 + u < K && (key[u] & mask) == prefix;
            const int bin = (int)((key[u] >> shift) & 0xFF);
            const unsigned long long inb = __ballot(in);
            if (inb != 0ull) {
                const int leader = __ffsll((long long)inb) - 1;
                const int lb = __builtin_amdgcn_readlane(bin, leader);
                if (__ballot(in && bin == lb) == inb) {
                    if (lane == leader) atomicAdd(&s_hist[buf][lb], __popcll(inb));
                } else if (in) {
                    atomicAdd(&s_hist[buf][bin], 1);
                }
            }
        }
        for (int i = tid; i < 256; i += kT) s_hist[buf == 2 ? 0 : buf + 1][i] = 0;   // next
        __syncthreads();
        // lane l owns bins 255-4l .. 252-4l (descending); the lane where the
        // count from the top first reaches `need` finds the digit
        int h[4], own = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h[q] = s_hist[buf][255 - 4 * lane - q];
            own += h[q];
        }
        const int incl = wave_incl_add(own);
        const int above = incl - own;                         // count in higher bins
        int rem = need - above, d = 255 - 4 * lane, hd = h[0];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if (h[q] >= rem) break;
            rem -= h[q];
            --d;
            hd = h[q + 1];
        }
        const int src = __ffsll((long long)__ballot(above < need && incl >= need)) - 1;
        rem = __builtin_amdgcn_readlane(rem, src);
        d = __builtin_amdgcn_readlane(d, src);
        hd = __builtin_amdgcn_readlane(hd, src);
        need = rem;
        eq = hd;
        prefix |= (unsigned long long)d << shift;
        mask |= 0xFFull << shift;
        done = hd == rem || shift == 0;
        shift -= 8;
        buf = buf == 2 ? 0 : buf + 1;
    }
    // keys compare on the bits resolved so far (all 64 unless stopped early)
    const unsigned long long thr = prefix;      // the k-th largest key (under mask)
    const int need_ties = need;                 // how many keys equal to thr to take
    const bool all_ties = need_ties == eq;      // uniform
    int eq_before = 0, total;
    if (!all_ties) {                            // rank the equal keys by index
        int n_eq = 0;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u)
            n_eq += u < per && j0 + u < K && (key[u] & mask) == thr;
        eq_before = block_excl_scan_dpp<kT>(n_eq, s_tmp[0], &total);
    }
    bool take[kSelPer];
    int n_sel = 0;
    {
        int e = eq_before;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const unsigned long long kv = key[u] & mask;
            take[u] = k > 0 && u < per && j0 + u < K &&
                      (kv > thr || (kv == thr && (all_ties || e < need_ties)));
            if (u < per && j0 + u < K && kv == thr) ++e;
            n_sel += take[u];
        }
    }
    const int sel_before = block_excl_scan_dpp<kT>(n_sel, s_tmp[1], &total);
    uint32_t am = 0;
    {
        int o = sel_before;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            if (take[u]) {
                sel[o++] = j0 + u;
                am = s_cmax[j0 + u] > am ? s_cmax[j0 + u] : am;
            }
        }
    }
    am = wave_max_u32(am);
    if (lane == 0) s_amax[tid >> 6] = am;
    __syncthreads();
    if (tid == 0) {
        uint32_t m = 0;
        for (int i = 0; i < kW; ++i) m = s_amax[i] > m ? s_amax[i] : m;
        *s_rts = tensor_scale_from_amax(__uint_as_float(m));
    }
    __syncthreads();
}

// Threads of the select kernel (measured at 2048 keys: four waves take
// twice as long as sixteen, the per-thread share of the keys being the
// longer chain).
constexpr int kSelThreads = 1024;
constexpr int kSelRowBatch = 4;            // partial rows loaded together

__global__ __launch_bounds__(kSelThreads) void k_rac_select(const double* __restrict__ score,
                                                            const uint32_t* __restrict__ colmax,
                                                            int nrows, int K,
                                                            int k, int32_t* __restrict__ sel,
                                                            float* __restrict__ r_ts,
                                                            double* __restrict__ score_out,
                                                            uint32_t* __restrict__ r_table) {
    __shared__ unsigned long long s_key[kRacMaxK];
    __shared__ uint32_t s_cmax[kRacMaxK];          // per-channel max |r| over the rows
    __shared__ float s_rts;
    const int tid = threadIdx.x;
    {   // work-group b selects for expert b (one work-group: the shared selection)
        const int64_t b = blockIdx.x;
        score += b * nrows * (int64_t)K;
        colmax += b * nrows * (int64_t)K;
        sel += b * k;
        r_ts += b;
        if (score_out) score_out += b * (int64_t)K;
        r_table += b * 1024;
    }
    // the last level of the fixed-order tree: nrows (<= kSelectFold) partial
    // rows summed in order from +0, kSelRowBatch rows of a channel requested
    // together
    for (int j = tid; j < K; j += kSelThreads) {
        double v = 0.0;
        uint32_t cm = 0;
        for (int r0 = 0; r0 < nrows; r0 += kSelRowBatch) {
            double sv[kSelRowBatch];
            uint32_t cv[kSelRowBatch];
#pragma unroll
            for (int q = 0; q < kSelRowBatch; ++q) {
                const int r = r0 + q < nrows ? r0 + q : nrows - 1;
                sv[q] = score[(int64_t)r * K + j];
                cv[q] = colmax[(int64_t)r * K + j];
            }
#pragma unroll
            for (int q = 0; q < kSelRowBatch; ++q) {
                if (r0 + q < nrows) {
                    v = v + sv[q];
                    cm = cv[q] > cm ? cv[q] : cm;
                }
            }
        }
        s_key[j] = (unsigned long long)__double_as_longlong(v);   // v >= +0: bits order
        s_cmax[j] = cm;
        if (score_out) score_out[j] = v;
    }
    select_keys<kSelThreads>(s_key, s_cmax, K, k, sel, &s_rts);
    if (tid == 0) r_ts[0] = s_rts;
    build_threshold_table(s_rts, reinterpret_cast<uint32_t(*)[8]>(r_table), false);
}

// ------------------------------------------------------------------ small --
// Tiny activations (at most 64 rows, one level-0 group, and at most 16384
// elements, e.g. a decode step of a few tokens): the whole RAC in one
// 1024-thread work-group and one launch, with the same arithmetic as the
// launches above.  Measured against the five launches: 11.2 / 13.5 us
// against 17.0 / 18.2 us at 16 x 128 and 32 x 256 (k = 64), but 23.9 against
// 20.5 us at 64 x 512 and 55.7 against 23.7 us at 64 x 2048, where one CU's
// share of the work outweighs the launches it saves.
//  1. max |x| -> s_t, and the code table of x in LDS;
//  2. rows in groups of RG = 1024 / (K/16) (thread = one 16-block of one row
//     of the group, loads of four groups in flight): NVFP4 codes and scale
//     bytes, r = RN32(x - v s_b s_t) into LDS, then thread = channel adds the
//     group's r^2 to its in-order fp64 sum (and max |r|), so every channel's
//     score is the sum over rows 0 .. M-1 in order from +0;
//  3. the radix selection (select_keys), the residual's tensor scale and its
//     code table in LDS;
//  4. the second pass as in k_rac_pass2.
constexpr int kSmallMaxK = 2048;
constexpr int64_t kSmallMaxElems = 16384;
constexpr int kSmallPre = 4;                      // row groups loaded together

__global__ __launch_bounds__(1024) void k_rac_small(
    const uint16_t* __restrict__ x, int M, int K, int k, bool want_scores,
    uint8_t* __restrict__ nib, uint8_t* __restrict__ scale, float* __restrict__ ts,
    int32_t* __restrict__ sel, uint8_t* __restrict__ r_nib, uint8_t* __restrict__ r_scale,
    float* __restrict__ r_ts, double* __restrict__ score_out) {
    __shared__ __align__(16) uint32_t s_tab[kE4m3MaxCode + 2][8];
    __shared__ __align__(16) float s_r[16 * 1024];    // one group's residuals, [RG][K]
    __shared__ unsigned long long s_key[kSmallMaxK];
    __shared__ uint32_t s_cmax[kSmallMaxK];
    __shared__ uint32_t s_w[16];
    __shared__ float s_st, s_rts;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

    // 1. tensor scale: 8 bf16 per load, 8 loads in flight per thread
    const int64_t n8 = (int64_t)M * K / 8;
    const uint4* x8 = reinterpret_cast<const uint4*>(x);
    uint32_t mx = 0;
    for (int64_t b = 0; b < n8; b += 8 * 1024) {
        uint4 q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = b + u * 1024 + tid;
            q[u] = i < n8 ? x8[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            mx = pk_max_u16(mx, q[u].x & 0x7FFF7FFFu);
            mx = pk_max_u16(mx, q[u].y & 0x7FFF7FFFu);
            mx = pk_max_u16(mx, q[u].z & 0x7FFF7FFFu);
            mx = pk_max_u16(mx, q[u].w & 0x7FFF7FFFu);
        }
    }
    {
        const uint32_t lo = mx & 0xFFFFu, hi = mx >> 16;
        const uint32_t m = wave_max_u32(lo > hi ? lo : hi);
        if (lane == 0) s_w[wid] = m;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t m = 0;
        for (int w = 0; w < 16; ++w) m = s_w[w] > m ? s_w[w] : m;
        s_st = tensor_scale_from_amax(bf16_to_f32(m));
        ts[0] = s_st;
    }
    __syncthreads();
    const float s_t = s_st;
    const double six_st = 6.0 * (double)s_t;
    build_threshold_table(s_t, s_tab, true);
    __syncthreads();

    // 2. codes, residuals and the in-order channel sums
    const int kb = K / kBlock;                        // blocks per row
    const int rg = 1024 / kb;                         // rows per group (>= 8)
    const int ngroups = (M + rg - 1) / rg;
    const int bcol = tid % kb, rr = tid / kb;         // this thread's block in a group
    double acc[2] = {0.0, 0.0};
    uint32_t cm[2] = {0u, 0u};
    for (int g0 = 0; g0 < ngroups; g0 += kSmallPre) {
        uint4 q0[kSmallPre], q1[kSmallPre];
#pragma unroll
        for (int u = 0; u < kSmallPre; ++u) {          // loads of four groups first
            const int row = (g0 + u) * rg + rr;
            const bool ok = rr < rg && row < M;
            const uint4* p = reinterpret_cast<const uint4*>(x + (ok ? (int64_t)row * K + bcol * kBlock : 0));
            q0[u] = p[0];
            q1[u] = p[1];
        }
#pragma unroll
        for (int u = 0; u < kSmallPre; ++u) {
            const int g = g0 + u;
            if (g >= ngroups) break;                  // uniform
            const int row = g * rg + rr;
            if (rr < rg && row < M) {
                const int64_t b = (int64_t)row * kb + bcol;
                const uint32_t w[8] = {q0[u].x, q0[u].y, q0[u].z, q0[u].w,
                                       q1[u].x, q1[u].y, q1[u].z, q1[u].w};
                uint32_t am = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) am = pk_max_u16(am, w[i] & 0x7FFF7FFFu);
                const uint32_t lo = am & 0xFFFFu, hi = am >> 16;
                const float amax_b = bf16_to_f32(lo > hi ? lo : hi);
                const uint32_t sb = s_t > 0.0f ? e4m3_rne_code((double)amax_b / six_st) : 0u;
                const uint4 t0 = *reinterpret_cast<const uint4*>(&s_tab[sb][0]);
                const uint4 t1 = *reinterpret_cast<const uint4*>(&s_tab[sb][4]);
                const uint2 packed = encode_block_bf16(w, t0, t1);
                *reinterpret_cast<uint2*>(nib + b * 8) = packed;
                scale[b] = (uint8_t)sb;
                const float s_b = e4m3_value(sb);
                float v[16];
                decode8(packed.x, v);
                decode8(packed.y, v + 8);
#pragma unroll
                for (int e = 0; e < 16; e += 4) {
                    float r4[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int ee = e + t;
                        const float xv =
                            __uint_as_float(ee & 1 ? w[ee >> 1] & 0xFFFF0000u : w[ee >> 1] << 16);
                        r4[t] = fmaf(-(v[ee] * s_b), s_t, xv);   // RN32(x - v s_b s_t)
                    }
                    *reinterpret_cast<float4*>(&s_r[rr * K + bcol * kBlock + e]) =
                        make_float4(r4[0], r4[1], r4[2], r4[3]);
                }
            }
            __syncthreads();
            if (want_scores) {
#pragma unroll
                for (int ci = 0; ci < 2; ++ci) {
                    const int c = tid + 1024 * ci;
                    if (c < K) {
                        const int nr = M - g * rg < rg ? M - g * rg : rg;
                        for (int i = 0; i < nr; ++i) {        // row order
                            const float rv = s_r[i * K + c];
                            const double rd = (double)rv;
                            acc[ci] = acc[ci] + rd * rd;      // r^2 exact in fp64
                            const uint32_t ab = __float_as_uint(rv) & 0x7FFFFFFFu;
                            cm[ci] = ab > cm[ci] ? ab : cm[ci];
                        }
                    }
                }
            }
            __syncthreads();
        }
    }
    if (!want_scores) {                               // neither S nor the scores
        if (tid == 0) r_ts[0] = 0.0f;
        return;
    }
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
        const int c = tid + 1024 * ci;
        if (c < K) {
            s_key[c] = (unsigned long long)__double_as_longlong(acc[ci]);   // >= +0: bits order
            s_cmax[c] = cm[ci];
            if (score_out) score_out[c] = acc[ci];
        }
    }
    __syncthreads();

    // 3. selection, the residual's tensor scale and code table
    select_keys<1024>(s_key, s_cmax, K, k, sel, &s_rts);
    const float s_tr = s_rts;
    if (tid == 0) r_ts[0] = s_tr;
    build_threshold_table(s_tr, s_tab, false);
    __syncthreads();                                  // sel, codes and scales written above

    // 4. second pass: one thread per element of r[:, S], 16-lane blocks
    const int64_t n = (int64_t)M * k;                 // k % 16 == 0: blocks never straddle
    const double six_str = 6.0 * (double)s_tr;
    for (int64_t t = tid; t - tid < n; t += 1024) {
        const bool live = t < n;                      // uniform over each 16-lane block
        float r = 0.0f;
        if (live) {
            const int64_t row = t / k;
            const int i = (int)(t - row * k);
            const int j = sel[i];
            const uint32_t h = x[row * K + j];
            const uint32_t code = (nib[row * (K / 2) + (j >> 1)] >> (4 * (j & 1))) & 0xFu;
            float sv = e2m1_value(code & 7u) * e4m3_value(scale[row * kb + (j >> 4)]);
            if (code & 8u) sv = -sv;
            r = fmaf(-sv, s_t, bf16_to_f32(h));
        }
        const uint32_t rb = __float_as_uint(r);
        uint32_t am = rb & 0x7FFFFFFFu;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            const uint32_t o = __shfl_xor(am, off, 16);
            am = o > am ? o : am;
        }
        const uint32_t sb =
            s_tr > 0.0f ? e4m3_rne_code((double)__uint_as_float(am) / six_str) : 0u;
        const uint4 t0 = *reinterpret_cast<const uint4*>(&s_tab[sb][0]);
        const uint4 t1 = *reinterpret_cast<const uint4*>(&s_tab[sb][4]);
        const uint32_t thr[7] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z};
        const uint32_t c = e2m1_mag_code(rb & 0x7FFFFFFFu, thr) | ((rb >> 28) & 8u);
        const uint32_t other = __shfl_xor(c, 1, 16);
        if (live) {
            if ((t & 1) == 0) r_nib[t >> 1] = (uint8_t)(c | (other << 4));
            if ((t & 15) == 0) r_scale[t >> 4] = (uint8_t)sb;
        }
    }
}

// ----------------------------------------------------------------- pass 2 --
// One thread per residual element (row, i); the 16 lanes of a block reduce
// its maximum with shuffles, neighbouring lanes pair their nibbles.
__global__ __launch_bounds__(256) void k_rac_pass2(
    const uint16_t* __restrict__ x, int64_t M, int K, const int32_t* __restrict__ sel, int k,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ scale,
    const float* __restrict__ ts, const float* __restrict__ r_ts,
    const uint32_t* __restrict__ r_table, uint8_t* __restrict__ r_nib,
    uint8_t* __restrict__ r_scale) {
    __shared__ uint4 s_tab[2 * (kE4m3MaxCode + 1)];
    for (int i = threadIdx.x; i < 2 * (kE4m3MaxCode + 1); i += blockDim.x)
        s_tab[i] = reinterpret_cast<const uint4*>(r_table)[i];
    const float s_t = ts[0];
    const float s_tr = r_ts[0];
    const double six_str = 6.0 * (double)s_tr;
    __syncthreads();
    const int64_t n = M * k;                       // k % 16 == 0: blocks never straddle
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < n;
         base += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = base + threadIdx.x;
        const bool live = t < n;                       // uniform over each 16-lane block
        float r = 0.0f;
        if (live) {
            const int64_t row = t / k;
            const int i = (int)(t - row * k);
            const int j = sel[i];
            const uint32_t h = x[row * K + j];
            const uint32_t code = (nib[row * (K / 2) + (j >> 1)] >> (4 * (j & 1))) & 0xFu;
            float sv = e2m1_value(code & 7u) * e4m3_value(scale[row * (K / kBlock) + (j >> 4)]);
            if (code & 8u) sv = -sv;
            r = fmaf(-sv, s_t, bf16_to_f32(h));
        }
        const uint32_t rb = __float_as_uint(r);
        uint32_t am = rb & 0x7FFFFFFFu;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            const uint32_t o = __shfl_xor(am, off, 16);
            am = o > am ? o : am;
        }
        const uint32_t sb =
            s_tr > 0.0f ? e4m3_rne_code((double)__uint_as_float(am) / six_str) : 0u;
        const uint4 t0 = s_tab[2 * sb], t1 = s_tab[2 * sb + 1];
        const uint32_t thr[7] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z};
        const uint32_t c = e2m1_mag_code(rb & 0x7FFFFFFFu, thr) | ((rb >> 28) & 8u);
        const uint32_t other = __shfl_xor(c, 1, 16);
        if (live) {
            if ((t & 1) == 0) r_nib[t >> 1] = (uint8_t)(c | (other << 4));
            if ((t & 15) == 0) r_scale[t >> 4] = (uint8_t)sb;
        }
    }
}

// ------------------------------------------------------ per-expert S --
// Expert e's rows split into chunks of 64 from its first row (the tree's
// level-0 groups); chunk_start[e] = sum over e' < e of ceil(rows_e' / 64).
constexpr int64_t kExpertMaxRows = (int64_t)kScoreFanin * kScoreFanin * kScoreFanin;
constexpr int kExpertMaxE = 4096;          // chunk starts kept in LDS

// Level-0 partials of every chunk: work-group (x, slice) takes chunks x,
// x + gridDim.x, ...; thread = two neighbouring channels (one 4-byte load of
// x, one nibble byte and one scale byte per row); r recomputed from x and the
// main NVFP4 exactly as pass 1 forms it, 32 rows loaded at a time, summed in
// row order from +0.  Work-group (0, 0) also writes chunk_start.
constexpr int kPartThreads = 128;          // 256 channels per slice

__global__ __launch_bounds__(kPartThreads) void k_rac_expert_partials(
    const uint16_t* __restrict__ x, int K, const uint8_t* __restrict__ nib,
    const uint8_t* __restrict__ scale, const float* __restrict__ ts,
    const int32_t* __restrict__ offsets, int E, double* __restrict__ part,
    uint32_t* __restrict__ pmax, int32_t* __restrict__ chunk_start) {
    __shared__ int s_cs[kExpertMaxE + 1];
    __shared__ int s_w[kPartThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // chunk starts: each thread a run of experts, then a scan over the block
    const int per = (E + kPartThreads - 1) / kPartThreads;
    const int e0 = tid * per, e1 = e0 + per < E ? e0 + per : E;
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (offsets[e + 1] - offsets[e] + kTileRows - 1) / kTileRows;
    int xs = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(xs, off, 64);
        if (lane >= off) xs += y;
    }
    if (lane == 63) s_w[wid] = xs;
    __syncthreads();
    int run = xs - local;
    for (int w = 0; w < wid; ++w) run += s_w[w];
    for (int e = e0; e < e1; ++e) {
        s_cs[e] = run;
        run += (offsets[e + 1] - offsets[e] + kTileRows - 1) / kTileRows;
    }
    if (tid == kPartThreads - 1) s_cs[E] = run;        // the last thread ends at the total
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int e = tid; e <= E; e += kPartThreads) chunk_start[e] = s_cs[e];
    const int nchunks = s_cs[E];
    const int c = blockIdx.y * 2 * kPartThreads + 2 * tid;   // channels c, c + 1 (K even)
    const float s_t = ts[0];
    for (int ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
        int lo = 0, hi = E;                           // s_cs[lo] <= ch < s_cs[lo + 1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_cs[mid] <= ch) lo = mid; else hi = mid;
        }
        const int64_t row0 = offsets[lo] + (int64_t)(ch - s_cs[lo]) * kTileRows;
        const int64_t rend = offsets[lo + 1];
        const int nr = (int)(rend - row0 < kTileRows ? rend - row0 : kTileRows);
        if (c >= K) continue;
        double acc[2] = {0.0, 0.0};
        uint32_t m[2] = {0u, 0u};
        for (int b = 0; b < nr; b += 32) {             // 32 rows in flight, loads first
            uint32_t xv[32], cv[32], sv[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int64_t p = row0 + (b + u < nr ? b + u : nr - 1);
                xv[u] = *reinterpret_cast<const uint32_t*>(x + p * K + c);
                cv[u] = nib[p * (K / 2) + (c >> 1)];
                sv[u] = scale[p * (K / kBlock) + (c >> 4)];
            }
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                if (b + u < nr) {
                    const float s_b = e4m3_value(sv[u]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {      // channel c + h: nibble h, bf16 h
                        const uint32_t code = (cv[u] >> (4 * h)) & 0xFu;
                        float v = e2m1_value(code & 7u);
                        if (code & 8u) v = -v;
                        const float xf = __uint_as_float(h ? xv[u] & 0xFFFF0000u : xv[u] << 16);
                        const float r = fmaf(-(v * s_b), s_t, xf);
                        const double rd = (double)r;
                        acc[h] = acc[h] + rd * rd;        // r^2 exact in fp64, row order
                        const uint32_t ab = __float_as_uint(r) & 0x7FFFFFFFu;
                        m[h] = ab > m[h] ? ab : m[h];
                    }
                }
            }
        }
        part[(int64_t)ch * K + c] = acc[0];
        part[(int64_t)ch * K + c + 1] = acc[1];
        pmax[(int64_t)ch * K + c] = m[0];
        pmax[(int64_t)ch * K + c + 1] = m[1];
    }
}

// Scores of expert e from its chunk partials, work-group (slice, e), thread
// = channel: the tree's upper levels streamed -- acc1 sums the chunk partials
// of the current level-1 node in order from +0, acc2 the finished level-1
// nodes (at most 64^2 chunks per expert).
__global__ __launch_bounds__(256) void k_rac_expert_scores(
    const double* __restrict__ part, const uint32_t* __restrict__ pmax,
    const int32_t* __restrict__ chunk_start, int K, double* __restrict__ score,
    uint32_t* __restrict__ colmax) {
    const int e = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= K) return;                               // no barriers below
    const int q0 = chunk_start[e], q1 = chunk_start[e + 1];
    double acc1 = 0.0, acc2 = 0.0;
    int n1 = 0, n2 = 0;
    uint32_t m = 0;
    for (int q = q0; q < q1; q += 16) {
        double v[16];
        uint32_t u[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {                   // loads first, then the chain
            const int qq = q + i < q1 ? q + i : q1 - 1;
            v[i] = part[(int64_t)qq * K + c];
            u[i] = pmax[(int64_t)qq * K + c];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (q + i < q1) {
                acc1 = acc1 + v[i];
                m = u[i] > m ? u[i] : m;
                if (++n1 == kScoreFanin) {                // a level-1 node is done
                    acc2 = acc2 + acc1;
                    acc1 = 0.0;
                    n1 = 0;
                    ++n2;
                }
            }
        }
    }
    // at most 64 chunks: their in-order sum (acc1, or acc2 when exactly 64
    // were pushed up); more: the in-order sum of the level-1 nodes
    const double sc = n2 == 0 ? acc1 : (n1 > 0 ? acc2 + acc1 : acc2);
    score[(int64_t)e * K + c] = sc;
    colmax[(int64_t)e * K + c] = m;
}

// Second pass with per-expert S: one thread per residual element (row, i);
// the row's expert by binary search in offsets; as k_rac_pass2 otherwise,
// with the expert's selection, residual scale and code table.
__global__ __launch_bounds__(256) void k_rac_pass2_experts(
    const uint16_t* __restrict__ x, int64_t M, int K, const int32_t* __restrict__ sel, int k,
    const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ nib,
    const uint8_t* __restrict__ scale, const float* __restrict__ ts,
    const float* __restrict__ r_ts, const uint32_t* __restrict__ r_table,
    uint8_t* __restrict__ r_nib, uint8_t* __restrict__ r_scale) {
    const float s_t = ts[0];
    const int64_t n = M * k;                       // k % 16 == 0: blocks never straddle
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < n;
         base += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = base + threadIdx.x;
        const bool live = t < n;                       // uniform over each 16-lane block
        const int64_t row = live ? t / k : 0;
        const int i = (int)(t - row * k);
        int lo = 0, hi = E;                            // expert: offsets[e] <= row < offsets[e+1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (offsets[mid] <= row) lo = mid; else hi = mid;
        }
        const int e = lo;
        float r = 0.0f;
        if (live) {
            const int j = sel[(int64_t)e * k + i];
            const uint32_t h = x[row * K + j];
            const uint32_t code = (nib[row * (K / 2) + (j >> 1)] >> (4 * (j & 1))) & 0xFu;
            float sv = e2m1_value(code & 7u) * e4m3_value(scale[row * (K / kBlock) + (j >> 4)]);
            if (code & 8u) sv = -sv;
            r = fmaf(-sv, s_t, bf16_to_f32(h));
        }
        const float s_tr = r_ts[e];
        const uint32_t rb = __float_as_uint(r);
        uint32_t am = rb & 0x7FFFFFFFu;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            const uint32_t o = __shfl_xor(am, off, 16);
            am = o > am ? o : am;
        }
        const uint32_t sb = s_tr > 0.0f ? e4m3_rne_code((double)__uint_as_float(am) /
                                                        (6.0 * (double)s_tr))
                                        : 0u;
        const uint32_t* tr = r_table + (int64_t)e * 1024 + 8 * sb;
        const uint32_t thr[7] = {tr[0], tr[1], tr[2], tr[3], tr[4], tr[5], tr[6]};
        const uint32_t c = e2m1_mag_code(rb & 0x7FFFFFFFu, thr) | ((rb >> 28) & 8u);
        const uint32_t other = __shfl_xor(c, 1, 16);
        if (live) {
            if ((t & 1) == 0) r_nib[t >> 1] = (uint8_t)(c | (other << 4));
            if ((t & 15) == 0) r_scale[t >> 4] = (uint8_t)sb;
        }
    }
}

__global__ void k_iota_experts(int32_t* p, int n, int k) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = i % k;
}

__global__ void k_iota_i32(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = i;
}
__global__ void k_fill_f64(double* p, int n, double v) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ------------------------------------------------------- MX FP4 mode --
// RAC with the MX FP4 quantizer (section 3.3 on the MX FP4 format the "FP4"
// paragraph of section 2.2 sets beside NVFP4): E2M1 elements with one
// power-of-two scale per 32 consecutive channels, no tensor scale.  The main
// codes come from the MX quantizer; the residual, scores and selection are
// those of the NVFP4 path (the same fixed-order fp64 sums, the same select
// kernel); the second pass MX-quantizes r[:, S] in 32-element blocks along
// the compacted index.

// Value of main MX FP4 element (code c, scale byte sb): v * 2^(sb - 127),
// exact in fp32 (at least 2^-128, at most two significant bits).
__device__ __forceinline__ float mx_fp4_value(uint32_t c, uint32_t sb) {
    const float v = ldexpf(e2m1_value(c & 7u), (int)sb - 127);
    return c & 8u ? -v : v;
}

// r = x - DQ(Q(x)) of element (row, col): exact in fp32 (x has 8
// significant bits, the value at most two, and |r| <= |x|).
__device__ __forceinline__ float mx_residual(const uint16_t* x, const uint8_t* codes,
                                             const uint8_t* scales, int64_t row, int K, int col) {
    const uint32_t byte = codes[row * (K / 2) + col / 2];
    const uint32_t sb = scales[row * (K / 32) + col / 32];
    const float xv = __uint_as_float((uint32_t)x[row * K + col] << 16);
    return xv - mx_fp4_value((byte >> (4 * (col & 1))) & 15u, sb);
}

// Shared exponent of an MX FP4 block from its largest |r| (fp32 bits):
// floor(log2) - 2, clamped to [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx_fp4_exponent(uint32_t bits) {
    if (bits == 0u) return -127;
    const int ef = (int)(bits >> 23) & 0xFF;
    const int fl = ef > 0 ? ef - 127 : -149 + (31 - __builtin_clz(bits & 0x7FFFFFu));
    const int e = fl - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Level-0 score partials: thread = channel, rows of one 64-row chunk in
// order from +0 (the layout of k_rac_pass1's partials, and their max |r|).
__global__ __launch_bounds__(256) void k_mx_rac_pass1(const uint16_t* __restrict__ x, int64_t M,
                                                      int K, const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      double* __restrict__ pa,
                                                      uint32_t* __restrict__ ca) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= K) return;
    const int64_t r0 = (int64_t)blockIdx.y * kTileRows;
    const int64_t r1 = r0 + kTileRows < M ? r0 + kTileRows : M;
    double acc = 0.0;
    uint32_t m = 0;
#pragma unroll 8
    for (int64_t r = r0; r < r1; ++r) {
        const float rv = mx_residual(x, codes, scales, r, K, c);
        acc = acc + (double)rv * (double)rv;                  // the square is exact in fp64
        const uint32_t u = __float_as_uint(rv) & 0x7FFFFFFFu;
        m = u > m ? u : m;
    }
    pa[(int64_t)blockIdx.y * K + c] = acc;
    ca[(int64_t)blockIdx.y * K + c] = m;
}

// Second pass: thread = 8 consecutive selected channels of one row; the four
// threads of a 32-block (neighbouring lanes: k % 32 == 0) share its maximum.
// Elements are r * 2^-E (exact), clamped to +-6 and rounded to the nearest
// E2M1 value, ties to even, by the hardware conversion.
__global__ __launch_bounds__(256) void k_mx_rac_pass2(const uint16_t* __restrict__ x, int64_t M,
                                                      int K, const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const int32_t* __restrict__ sel, int k,
                                                      uint8_t* __restrict__ r_codes,
                                                      uint8_t* __restrict__ r_scales) {
    const int per_row = k / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = t < M * per_row;                        // whole 4-lane groups
    const int64_t row = live ? t / per_row : 0;
    const int j0 = live ? (int)(t - row * per_row) * 8 : 0;
    float rv[8];
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int c = sel[j0 + i];
        c = c < 0 ? 0 : (c >= K ? K - 1 : c);                 // bounds only: sel < K
        rv[i] = live ? mx_residual(x, codes, scales, row, K, c) : 0.0f;
        const uint32_t u = __float_as_uint(rv[i]) & 0x7FFFFFFFu;
        am = u > am ? u : am;
    }
    uint32_t o = __shfl_xor(am, 1, 64);
    am = o > am ? o : am;
    o = __shfl_xor(am, 2, 64);
    am = o > am ? o : am;
    const int e = mx_fp4_exponent(am);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(ldexpf(rv[i], -e), -6.0f), 6.0f);
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
    if (live) {
        *reinterpret_cast<uint32_t*>(r_codes + row * (k / 2) + j0 / 2) = w;
        if (j0 % 32 == 0) r_scales[row * (k / 32) + j0 / 32] = (uint8_t)(e + 127);
    }
}

struct RacWs {
    uint32_t* partial;
    uint32_t* r_table;     // code table of the gathered residual
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
    w.r_table = (uint32_t*)(base + off); off += 1024 * 4;
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

// Argument checks of quads_rac_quantize other than the workspace.
static int rac_check_args(const uint16_t* x, int64_t M, int64_t K, int32_t k, uint8_t* nib,
                          uint8_t* scale, float* ts, int32_t* sel, uint8_t* r_nib,
                          uint8_t* r_scale, float* r_ts, double* score_out) {
    if (M < 0 || K <= 0 || K % kBlock || K > kRacMaxK) return QUADS_ESHAPE;
    if (k < 0 || k % kBlock || k > K) return QUADS_ESHAPE;
    if (!ok_ptr(ts) || !ok_ptr(r_ts) || !ok_opt_ptr(score_out)) return QUADS_EINVAL;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(nib) || !ok_ptr(scale))) return QUADS_EINVAL;
    if (k > 0 && !ok_ptr(sel)) return QUADS_EINVAL;
    if (k > 0 && M > 0 && (!ok_ptr(r_nib) || !ok_ptr(r_scale))) return QUADS_EINVAL;
    return QUADS_OK;
}

// The launches of quads_rac_quantize once the arguments are checked; `ws`
// holds at least quads_rac_quantize_ws(M, K, k) bytes of device memory.
// With amax_part, max|x| comes from those `part_groups` partial maxima
// instead of a max pass over x.
static int rac_run(const uint16_t* x, int64_t M, int64_t K, int32_t k, uint8_t* nib,
                   uint8_t* scale, float* ts, int32_t* sel, uint8_t* r_nib, uint8_t* r_scale,
                   float* r_ts, double* score_out, void* ws, hipStream_t s,
                   const uint32_t* amax_part = nullptr, int64_t part_groups = 0) {
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
    if (M <= kTileRows && K <= kSmallMaxK && M * K <= kSmallMaxElems) {   // one launch
        hipLaunchKernelGGL(k_rac_small, dim3(1), dim3(1024), 0, s, x, (int)M, (int)K, (int)k,
                           k > 0 || score_out != nullptr, nib, scale, ts, sel, r_nib, r_scale,
                           r_ts, score_out);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    RacWs w = rac_ws_layout((char*)ws, M, K);
    const uint32_t* partial = amax_part;
    int groups = (int)part_groups;
    if (partial == nullptr) {
        groups = amax_groups(M * K);
        launch_amax_partial(x, M * K, 1, w.partial, groups, s);
        QUADS_CHECK_LAUNCH();
        partial = w.partial;
    }
    const bool want_scores = k > 0 || score_out != nullptr;
    const int64_t c0 = (M + kTileRows - 1) / kTileRows;
    const int64_t ctiles = (K + kP1Cols - 1) / kP1Cols;
    // about the work-groups the device holds at once (four per CU), each
    // walking its chunks, so the per-work-group fold of the maxima and code
    // table are paid fewer times (32768 x 768, maxima from 4608 producer
    // slots: 57.5 -> 55.7 us for the whole RAC call; a quarter of that grid
    // or less is slower)
    int64_t gx = 1024 / ctiles;
    gx = gx < 1 ? 1 : (gx > c0 ? c0 : gx);
    hipLaunchKernelGGL(k_rac_pass1, dim3((unsigned)gx, (unsigned)ctiles), dim3(256), 0, s, x, M,
                       (int)K, partial, groups, ts, nib, scale,
                       want_scores ? w.pa : nullptr, want_scores ? w.ca : nullptr);
    QUADS_CHECK_LAUNCH();
    if (!want_scores) {                            // neither S nor the scores are wanted
        launch_fill_f32(r_ts, 1, 0.0f, s);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    // fixed-order tree over the level-0 partials (its last level runs in select)
    double* pin = w.pa; uint32_t* cin = w.ca;
    double* pout = w.pb; uint32_t* cout = w.cb;
    int64_t n = c0;
    while (n > kSelectFold) {
        const int64_t g = (n + kScoreFanin - 1) / kScoreFanin;
        hipLaunchKernelGGL(k_tree_level, dim3((unsigned)((K + 255) / 256), (unsigned)g), dim3(256),
                           0, s, pin, cin, n, (int)K, pout, cout);
        QUADS_CHECK_LAUNCH();
        n = g;
        double* tp = pin; pin = pout; pout = tp;
        uint32_t* tc = cin; cin = cout; cout = tc;
    }
    hipLaunchKernelGGL(k_rac_select, dim3(1), dim3(kSelThreads), 0, s, pin, cin, (int)n, (int)K,
                       (int)k, sel, r_ts, score_out, w.r_table);
    QUADS_CHECK_LAUNCH();
    if (k > 0) {
        const int64_t nel = M * (int64_t)k;
        int64_t grid = (nel + 255) / 256;
        if (grid > 2048) grid = 2048;
        hipLaunchKernelGGL(k_rac_pass2, dim3((unsigned)grid), dim3(256), 0, s, x, M, (int)K, sel,
                           (int)k, nib, scale, ts, r_ts, w.r_table, r_nib, r_scale);
        QUADS_CHECK_LAUNCH();
    } else {
        launch_fill_f32(r_ts, 1, 0.0f, s);
        QUADS_CHECK_LAUNCH();
    }
    return QUADS_OK;
}

extern "C" int quads_rac_quantize(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                  uint8_t* nib, uint8_t* scale, float* ts, int32_t* sel,
                                  uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                                  double* score_out, void* ws, size_t ws_bytes, void* stream) {
    const int st = rac_check_args(x, M, K, k, nib, scale, ts, sel, r_nib, r_scale, r_ts,
                                  score_out);
    if (st != QUADS_OK) return st;
    if (ws_bytes < quads_rac_quantize_ws(M, K, k) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    return rac_run(x, M, K, k, nib, scale, ts, sel, r_nib, r_scale, r_ts, score_out, ws,
                   (hipStream_t)stream);
}

extern "C" int quads_rac_quantize_partials(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                           const uint32_t* amax_part, int64_t groups,
                                           uint8_t* nib, uint8_t* scale, float* ts,
                                           int32_t* sel, uint8_t* r_nib, uint8_t* r_scale,
                                           float* r_ts, double* score_out, void* ws,
                                           size_t ws_bytes, void* stream) {
    const int st = rac_check_args(x, M, K, k, nib, scale, ts, sel, r_nib, r_scale, r_ts,
                                  score_out);
    if (st != QUADS_OK) return st;
    if (groups < 1 || groups >= ((int64_t)1 << 31)) return QUADS_ESHAPE;
    if (!ok_ptr4(amax_part)) return QUADS_EINVAL;
    if (ws_bytes < quads_rac_quantize_ws(M, K, k) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    return rac_run(x, M, K, k, nib, scale, ts, sel, r_nib, r_scale, r_ts, score_out, ws,
                   (hipStream_t)stream, amax_part, groups);
}

// Workspace of quads_rac_quantize_noalloc.  In host code `scratch` names a
// host-side shadow, not device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) char scratch[QUADS_RAC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_hip_error(e);
    if (dev < 0 || dev >= kMaxDevices) return QUADS_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return set_hip_error(e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QUADS_OK;
}
}  // namespace

extern "C" int quads_rac_quantize_noalloc(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                          uint8_t* nib, uint8_t* scale, float* ts,
                                          int32_t* sel, uint8_t* r_nib, uint8_t* r_scale,
                                          float* r_ts, double* score_out, void* stream) {
    int st = rac_check_args(x, M, K, k, nib, scale, ts, sel, r_nib, r_scale, r_ts, score_out);
    if (st != QUADS_OK) return st;
    if (quads_rac_quantize_ws(M, K, k) > QUADS_RAC_NOALLOC_SCRATCH_BYTES) return QUADS_ESCRATCH;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != QUADS_OK) return st;
    return rac_run(x, M, K, k, nib, scale, ts, sel, r_nib, r_scale, r_ts, score_out, ws,
                   (hipStream_t)stream);
}

// Per-expert selection: workspace = partial maxima, scores [E, K] (fp64),
// per-channel maxima [E, K], code tables [E, 1024], chunk starts [E + 1],
// chunk partials [chunks, K] (fp64) and their maxima [chunks, K], with at
// most M / 64 + E chunks.
struct RacExpertWs {
    uint32_t* partial;
    double* score;
    uint32_t* cmax;
    uint32_t* tables;
    int32_t* chunk_start;
    double* part;
    uint32_t* pmax;
    size_t bytes;
};

static RacExpertWs rac_experts_ws_layout(char* base, int64_t M, int64_t K, int64_t E) {
    const int64_t nch = M / kTileRows + E;
    RacExpertWs w;
    size_t off = 0;
    w.partial = (uint32_t*)(base + off); off += align_up(kAmaxGroups * 4, 256);
    w.score = (double*)(base + off); off += align_up((size_t)E * K * 8, 256);
    w.cmax = (uint32_t*)(base + off); off += align_up((size_t)E * K * 4, 256);
    w.tables = (uint32_t*)(base + off); off += align_up((size_t)E * 1024 * 4, 256);
    w.chunk_start = (int32_t*)(base + off); off += align_up((size_t)(E + 1) * 4, 256);
    w.part = (double*)(base + off); off += align_up((size_t)nch * K * 8, 256);
    w.pmax = (uint32_t*)(base + off); off += align_up((size_t)nch * K * 4, 256);
    w.bytes = off;
    return w;
}

extern "C" size_t quads_rac_quantize_experts_ws(int64_t M, int64_t K, int32_t k, int32_t E) {
    (void)k;
    if (M < 0 || K <= 0 || E < 1) return 0;
    return rac_experts_ws_layout(nullptr, M, K, E).bytes;
}

extern "C" int quads_rac_quantize_experts(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                          const int32_t* offsets, int32_t E, uint8_t* nib,
                                          uint8_t* scale, float* ts, int32_t* sel,
                                          uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                                          double* score_out, void* ws, size_t ws_bytes,
                                          void* stream) {
    if (M < 0 || M > kExpertMaxRows || K <= 0 || K % kBlock || K > kRacMaxK) return QUADS_ESHAPE;
    if (k < 0 || k % kBlock || k > K || E < 1 || E > kExpertMaxE) return QUADS_ESHAPE;
    if (!ok_ptr(ts) || !ok_ptr(r_ts) || !ok_ptr(offsets) || !ok_opt_ptr(score_out))
        return QUADS_EINVAL;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(nib) || !ok_ptr(scale))) return QUADS_EINVAL;
    if (k > 0 && !ok_ptr(sel)) return QUADS_EINVAL;
    if (k > 0 && M > 0 && (!ok_ptr(r_nib) || !ok_ptr(r_scale))) return QUADS_EINVAL;
    if (ws_bytes < quads_rac_quantize_experts_ws(M, K, k, E) || !ok_ptr(ws))
        return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {
        launch_fill_f32(ts, 1, 0.0f, s);
        launch_fill_f32(r_ts, E, 0.0f, s);
        if (k > 0)
            hipLaunchKernelGGL(k_iota_experts, dim3((unsigned)(((int64_t)E * k + 255) / 256)),
                               dim3(256), 0, s, sel, (int)(E * k), (int)k);
        if (score_out)
            hipLaunchKernelGGL(k_fill_f64, dim3((unsigned)((E * K + 255) / 256)), dim3(256), 0, s,
                               score_out, (int)(E * K), 0.0);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    const RacExpertWs w = rac_experts_ws_layout(static_cast<char*>(ws), M, K, E);
    uint32_t* partial = w.partial;
    const int groups = amax_groups(M * K);
    launch_amax_partial(x, M * K, 1, partial, groups, s);
    QUADS_CHECK_LAUNCH();
    const int64_t c0 = (M + kTileRows - 1) / kTileRows;
    const int64_t ctiles = (K + kP1Cols - 1) / kP1Cols;
    int64_t gx = 2048 / ctiles;
    gx = gx < 1 ? 1 : (gx > c0 ? c0 : gx);
    hipLaunchKernelGGL(k_rac_pass1, dim3((unsigned)gx, (unsigned)ctiles), dim3(256), 0, s, x, M,
                       (int)K, partial, groups, ts, nib, scale, (double*)nullptr,
                       (uint32_t*)nullptr);
    QUADS_CHECK_LAUNCH();
    int64_t gp = 2048 / ctiles;                     // chunk partials: at most M / 64 + E chunks
    const int64_t nch = M / kTileRows + E;
    gp = gp < 1 ? 1 : (gp > nch ? nch : gp);
    hipLaunchKernelGGL(k_rac_expert_partials, dim3((unsigned)gp, (unsigned)ctiles),
                       dim3(kPartThreads), 0, s, x, (int)K, nib, scale, ts, offsets, (int)E,
                       w.part, w.pmax, w.chunk_start);
    QUADS_CHECK_LAUNCH();
    hipLaunchKernelGGL(k_rac_expert_scores, dim3((unsigned)ctiles, (unsigned)E), dim3(256), 0, s,
                       w.part, w.pmax, w.chunk_start, (int)K, w.score, w.cmax);
    QUADS_CHECK_LAUNCH();
    hipLaunchKernelGGL(k_rac_select, dim3((unsigned)E), dim3(kSelThreads), 0, s, w.score, w.cmax, 1,
                       (int)K, (int)k, sel, r_ts, score_out, w.tables);
    QUADS_CHECK_LAUNCH();
    if (k > 0) {
        const int64_t nel = M * (int64_t)k;
        int64_t grid = (nel + 255) / 256;
        if (grid > 2048) grid = 2048;
        hipLaunchKernelGGL(k_rac_pass2_experts, dim3((unsigned)grid), dim3(256), 0, s, x, M,
                           (int)K, sel, (int)k, offsets, (int)E, nib, scale, ts, r_ts, w.tables,
                           r_nib, r_scale);
        QUADS_CHECK_LAUNCH();
    }
    return QUADS_OK;
}


// RAC on the MX FP4 mode.  Workspace: that of quads_rac_quantize (the score
// partials and their tree).
extern "C" size_t quads_mx_rac_quantize_ws(int64_t M, int64_t K, int32_t k) {
    return quads_rac_quantize_ws(M, K, k);
}

extern "C" int quads_mx_rac_quantize(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                     uint8_t* codes, uint8_t* scales, int32_t* sel,
                                     uint8_t* r_codes, uint8_t* r_scales, double* score_out,
                                     void* ws, size_t ws_bytes, void* stream) {
    if (M < 0 || K <= 0 || K % 32 || K > kRacMaxK) return QUADS_ESHAPE;
    if (k < 0 || k % 32 || k > K) return QUADS_ESHAPE;
    if (!ok_opt_ptr(score_out)) return QUADS_EINVAL;
    if (M > 0 && (!ok_ptr(x) || !ok_ptr(codes) || !ok_ptr(scales))) return QUADS_EINVAL;
    if (k > 0 && !ok_ptr(sel)) return QUADS_EINVAL;
    if (k > 0 && M > 0 && (!ok_ptr(r_codes) || !ok_ptr(r_scales))) return QUADS_EINVAL;
    if (ws_bytes < quads_mx_rac_quantize_ws(M, K, k) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {
        if (k > 0) hipLaunchKernelGGL(k_iota_i32, dim3((k + 255) / 256), dim3(256), 0, s, sel, k);
        if (score_out)
            hipLaunchKernelGGL(k_fill_f64, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s,
                               score_out, (int)K, 0.0);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    int st = quads_mx_quantize(x, M, K, QUADS_MX_FP4, codes, scales, stream);
    if (st != QUADS_OK) return st;
    if (k == 0 && score_out == nullptr) return QUADS_OK;
    RacWs w = rac_ws_layout((char*)ws, M, K);
    const int64_t c0 = (M + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL(k_mx_rac_pass1, dim3((unsigned)((K + 255) / 256), (unsigned)c0), dim3(256), 0,
                       s, x, M, (int)K, codes, scales, w.pa, w.ca);
    QUADS_CHECK_LAUNCH();
    // the fixed-order tree and the selection of the NVFP4 path (the residual
    // tensor scale and code table it also writes go to workspace, unused)
    double* pin = w.pa; uint32_t* cin = w.ca;
    double* pout = w.pb; uint32_t* cout = w.cb;
    int64_t n = c0;
    while (n > kSelectFold) {
        const int64_t g = (n + kScoreFanin - 1) / kScoreFanin;
        hipLaunchKernelGGL(k_tree_level, dim3((unsigned)((K + 255) / 256), (unsigned)g), dim3(256),
                           0, s, pin, cin, n, (int)K, pout, cout);
        QUADS_CHECK_LAUNCH();
        n = g;
        double* tp = pin; pin = pout; pout = tp;
        uint32_t* tc = cin; cin = cout; cout = tc;
    }
    hipLaunchKernelGGL(k_rac_select, dim3(1), dim3(kSelThreads), 0, s, pin, cin, (int)n, (int)K,
                       (int)k, sel, reinterpret_cast<float*>(w.partial), score_out, w.r_table);
    QUADS_CHECK_LAUNCH();
    if (k > 0) {
        const int64_t threads = M * (int64_t)(k / 8);
        hipLaunchKernelGGL(k_mx_rac_pass2, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           x, M, (int)K, codes, scales, sel, (int)k, r_codes, r_scales);
        QUADS_CHECK_LAUNCH();
    }
    return QUADS_OK;
}
