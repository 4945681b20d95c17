// Token-to-expert packing and the MoE combine.
//
// Packing is a stable counting sort of the T*topk (token, slot) pairs by
// expert id.  Up to 4096 pairs and 512 experts: one work-group, one launch
// (k_pack_small).  Up to 16384 per-chunk counts (e.g. 32768 pairs over 128
// experts): per-chunk histograms, then a scatter whose work-groups each sum
// the histograms into their own chunk's bases (k_pack_scatter_prefix).
// Otherwise three launches: per-chunk histograms, one work-group that turns
// them into expert offsets and per-chunk bases, and a scatter in which one
// wave walks its chunk 64 entries at a time, ranking equal ids with ballots
// so that equal ids keep their flattened order.
//
// Combine: out[t] = sum over slots (in order) of w[t, slot] * y[pos[t, slot]],
// eight output features per thread, fp32 fused multiply-adds.
#include "common.h"

namespace quads {

constexpr int kPackChunk = 256;        // entries per chunk
constexpr int kPackMaxE = 4096;
constexpr int kPackScanLds = 24576;    // chunk counts the scan keeps in LDS

__global__ __launch_bounds__(256) void k_pack_count(const int32_t* __restrict__ ids, int64_t n,
                                                    int E, int32_t* __restrict__ cnt) {
    __shared__ int s_h[kPackMaxE];
    for (int e = threadIdx.x; e < E; e += 256) s_h[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kPackChunk;
    for (int i = threadIdx.x; i < kPackChunk; i += 256) {
        const int64_t idx = base + i;
        if (idx < n) {
            const int e = ids[idx];
            if (e >= 0 && e < E) atomicAdd(&s_h[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) cnt[(int64_t)blockIdx.x * E + e] = s_h[e];
}

// One work-group: offsets[e] = exclusive scan of expert totals; cnt[c][e] is
// replaced by the number of expert e's entries in chunks before c (the
// scatter adds offsets[e]).
__global__ __launch_bounds__(1024) void k_pack_scan(int32_t* __restrict__ cnt, int nchunks, int E,
                                                    int64_t n, int32_t* __restrict__ offsets) {
    __shared__ int s_tot[kPackMaxE];
    __shared__ int s_wave[16];
    __shared__ int s_cnt[kPackScanLds];
    // Per-expert exclusive scans over chunks, kPackScanLds counts at a time
    // through LDS (coalesced in and out).  Thread groups of P lanes share an
    // expert: each lane sums a run of chunks, a shuffle scan over the group
    // gives the lane's base, then the lane writes its run.  s_tot carries the
    // running total of each expert across LDS tiles.
    for (int e = threadIdx.x; e < E; e += 1024) s_tot[e] = 0;
    int P = 1;
    while (P < 64 && 2 * P * E <= 1024) P *= 2;
    const int tile = kPackScanLds / E;                    // chunks per LDS tile (>= 6)
    const int lane = threadIdx.x & 63;
    for (int c0 = 0; c0 < nchunks; c0 += tile) {
        const int nc = nchunks - c0 < tile ? nchunks - c0 : tile;
        const int64_t g0 = (int64_t)c0 * E;
        __syncthreads();
        for (int b = 0; b < nc * E; b += 8 * 1024) {       // 8 loads in flight per thread
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = b + u * 1024 + (int)threadIdx.x;
                v[u] = i < nc * E ? cnt[g0 + i] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = b + u * 1024 + (int)threadIdx.x;
                if (i < nc * E) s_cnt[i] = v[u];
            }
        }
        __syncthreads();
        const int L = (nc + P - 1) / P;
        for (int t = threadIdx.x; t < ((E * P + 63) / 64) * 64; t += 1024) {
            const int e = t / P, part = t % P;              // groups never straddle a wave
            const bool act = e < E;
            const int ca = part * L, cb = ca + L < nc ? ca + L : nc;
            int local = 0;
            if (act)
                for (int c = ca; c < cb; ++c) local += s_cnt[c * E + e];
            int incl = local;
            for (int off = 1; off < P; off <<= 1) {
                const int y = __shfl_up(incl, off, P);
                if ((lane % P) >= off) incl += y;
            }
            const int total = __shfl(incl, P - 1, P);
            if (act) {
                int run = s_tot[e] + incl - local;
                for (int c = ca; c < cb; ++c) {
                    const int v = s_cnt[c * E + e];
                    s_cnt[c * E + e] = run;
                    run += v;
                }
            }
            // every lane of the group has read s_tot[e] before part 0 updates it
            __builtin_amdgcn_wave_barrier();
            if (act && part == 0) s_tot[e] += total;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nc * E; i += 1024) cnt[g0 + i] = s_cnt[i];
    }
    __syncthreads();
    // exclusive scan of s_tot over E entries: each thread owns a contiguous run
    const int per = (E + 1023) / 1024;
    const int e0 = threadIdx.x * per;
    const int e1 = e0 + per < E ? e0 + per : E;
    int local = 0;
    for (int e = e0; e < e1; ++e) local += s_tot[e];
    const int wid = threadIdx.x >> 6;
    int x = local;
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wid] = x;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < wid; ++i) wbase += s_wave[i];
    int run = x - local + wbase;
    __syncthreads();
    for (int e = e0; e < e1; ++e) {
        const int t = s_tot[e];
        s_tot[e] = run;
        run += t;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 1024) offsets[e] = s_tot[e];
    if (threadIdx.x == 0) offsets[E] = (int32_t)n;
}

// One wave per chunk.
__global__ __launch_bounds__(64) void k_pack_scatter(const int32_t* __restrict__ ids, int64_t n,
                                                     int topk, int E,
                                                     const int32_t* __restrict__ base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ row_token,
                                                     int32_t* __restrict__ pos) {
    __shared__ int s_next[kPackMaxE];
    for (int e = threadIdx.x; e < E; e += 64)
        s_next[e] = offsets[e] + base[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int lane = threadIdx.x;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int64_t c0 = (int64_t)blockIdx.x * kPackChunk;
    int ev[kPackChunk / 64];                               // all ids of the chunk in flight
#pragma unroll
    for (int it = 0; it < kPackChunk / 64; ++it) {
        const int64_t idx = c0 + it * 64 + lane;
        ev[it] = idx < n ? ids[idx] : -1;
    }
#pragma unroll
    for (int it = 0; it < kPackChunk / 64; ++it) {
        const int64_t idx = c0 + it * 64 + lane;
        int e = ev[it];
        if (e < 0 || e >= E) e = -1;
        uint64_t peers = __ballot(e >= 0);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t m = __ballot(e >= 0 && ((e >> b) & 1));
            peers &= (e >= 0 && ((e >> b) & 1)) ? m : ~m;
        }
        int rank = 0, p = 0;
        if (e >= 0) {
            rank = __popcll(peers & lt);
            p = s_next[e] + rank;
        }
        __syncthreads();
        if (e >= 0) {
            row_token[p] = (int32_t)(idx / topk);
            pos[idx] = p;
            if (rank == 0) s_next[e] += __popcll(peers);
        }
        __syncthreads();
    }
}

// Mid-size inputs (nchunks * E <= kPackPrefixMax counts, E % 4 == 0): the
// scatter work-group of chunk c finds its experts' first packed rows itself
// -- the column totals of the per-chunk counts, scanned over experts, plus
// the counts of chunks before c -- so no scan launch runs between the count
// and the scatter.  The counts come in with 16-byte loads, all of a
// thread's in flight together, and are summed with LDS atomics; work-group 0
// writes offsets.  Then wave 0 walks the chunk as k_pack_scatter does.
constexpr int kPackPrefixMax = 16384;
constexpr int kPackPrefixLoads = kPackPrefixMax / 4 / 256;     // 16 per thread

__global__ __launch_bounds__(256) void k_pack_scatter_prefix(
    const int32_t* __restrict__ ids, int64_t n, int topk, int E, int nchunks,
    const int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ pos) {
    __shared__ int s_tot[kPackPrefixMax / 4];     // E <= nchunks * E / 4 here
    __shared__ int s_next[kPackPrefixMax / 4];
    __shared__ int s_wave[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = blockIdx.x;
    for (int e = tid; e < E; e += 256) {
        s_tot[e] = 0;
        s_next[e] = 0;
    }
    const int nq = nchunks * E / 4;
    uint4 v[kPackPrefixLoads];
#pragma unroll
    for (int u = 0; u < kPackPrefixLoads; ++u) {
        const int q = tid + 256 * u;
        v[u] = q < nq ? reinterpret_cast<const uint4*>(cnt)[q] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    if (1024 % E == 0) {
        // E divides the 1024 counts of a load round: the thread's four
        // experts are the same in every round, so it sums in registers, the
        // lanes holding the same experts add up by shuffles, and one lane per
        // expert quad and wave adds into LDS
        int tot[4] = {0, 0, 0, 0}, below[4] = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kPackPrefixLoads; ++u) {
            const int q = tid + 256 * u;
            const int a[4] = {(int)v[u].x, (int)v[u].y, (int)v[u].z, (int)v[u].w};
            const bool before = q < nq && 4 * q / E < c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tot[i] += a[i];                            // zero past the counts
                below[i] += before ? a[i] : 0;
            }
        }
        for (int off = 32; off >= E / 4 && off > 0; off >>= 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tot[i] += __shfl_xor(tot[i], off, 64);
                below[i] += __shfl_xor(below[i], off, 64);
            }
        }
        if (lane < E / 4 || E >= 256) {
            const int e = (4 * tid) % E;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (tot[i]) atomicAdd(&s_tot[e + i], tot[i]);
                if (below[i]) atomicAdd(&s_next[e + i], below[i]);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < kPackPrefixLoads; ++u) {
            const int q = tid + 256 * u;
            if (q < nq) {
                const int cc = 4 * q / E, e = 4 * q - cc * E;
                const int a[4] = {(int)v[u].x, (int)v[u].y, (int)v[u].z, (int)v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (a[i] == 0) continue;
                    atomicAdd(&s_tot[e + i], a[i]);
                    if (cc < c) atomicAdd(&s_next[e + i], a[i]);
                }
            }
        }
    }
    __syncthreads();
    // exclusive scan of the totals over experts: each thread a contiguous run
    const int per = (E + 255) / 256;
    const int e0 = tid * per, e1 = e0 + per < E ? e0 + per : E;
    int local = 0;
    for (int e = e0; e < e1; ++e) local += s_tot[e];
    int x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[w] = x;
    __syncthreads();
    int run = x - local;
    for (int q = 0; q < w; ++q) run += s_wave[q];
    for (int e = e0; e < e1; ++e) {
        const int t = s_tot[e];
        if (c == 0) offsets[e] = run;
        s_next[e] += run;
        run += t;
    }
    if (c == 0 && tid == 0) offsets[E] = (int32_t)n;
    __syncthreads();
    if (w != 0) return;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int64_t c0 = (int64_t)c * kPackChunk;
    int ev[kPackChunk / 64];                               // all ids of the chunk in flight
#pragma unroll
    for (int it = 0; it < kPackChunk / 64; ++it) {
        const int64_t idx = c0 + it * 64 + lane;
        ev[it] = idx < n ? ids[idx] : -1;
    }
#pragma unroll
    for (int it = 0; it < kPackChunk / 64; ++it) {
        const int64_t idx = c0 + it * 64 + lane;
        int e = ev[it];
        if (e < 0 || e >= E) e = -1;
        uint64_t peers = __ballot(e >= 0);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t m = __ballot(e >= 0 && ((e >> b) & 1));
            peers &= (e >= 0 && ((e >> b) & 1)) ? m : ~m;
        }
        int rank = 0, p = 0;
        if (e >= 0) {
            rank = __popcll(peers & lt);
            p = s_next[e] + rank;
        }
        // every lane has read its expert's next row before the first peer moves it
        __builtin_amdgcn_wave_barrier();
        if (e >= 0) {
            row_token[p] = (int32_t)(idx / topk);
            pos[idx] = p;
            if (rank == 0) s_next[e] += __popcll(peers);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Small inputs (n <= kPackOneMaxN entries, E <= kPackOneMaxE) in one
// work-group of 16 waves and one launch.  Wave w owns the contiguous entries
// [w S, w S + S) (S a multiple of 64, at most 4 steps of 64, all ids held in
// registers): per-wave expert counts; per expert the exclusive scan over the
// waves plus the expert's offset (the scan over experts); then each wave
// walks its entries 64 at a time, ranking equal ids with ballots.  Entries of
// one expert thus keep their flattened order, as in the three-launch path.
constexpr int kPackOneMaxN = 4096;        // above it the three launches are faster
constexpr int kPackOneMaxE = 512;
constexpr int kPackOneSteps = kPackOneMaxN / 16 / 64;     // 4

__global__ __launch_bounds__(1024) void k_pack_small(const int32_t* __restrict__ ids, int n,
                                                     int topk, int E,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ row_token,
                                                     int32_t* __restrict__ pos) {
    __shared__ int s_h[16][kPackOneMaxE];    // per-wave counts, then next packed row
    __shared__ int s_tot[kPackOneMaxE];
    __shared__ int s_wave[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < 16 * kPackOneMaxE; i += 1024) (&s_h[0][0])[i] = 0;
    const int S = ((n + 15) / 16 + 63) / 64 * 64;
    const int steps = S / 64;                             // <= kPackOneSteps
    const int b0 = w * S;
    int ev[kPackOneSteps];                                // this lane's ids, -1 = none
#pragma unroll
    for (int it = 0; it < kPackOneSteps; ++it) {          // every load in flight at once
        const int idx = b0 + it * 64 + lane;
        const bool ok = it < steps && idx < n;
        const int e = ids[ok ? idx : 0];
        ev[it] = ok && e >= 0 && e < E ? e : -1;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kPackOneSteps; ++it)
        if (ev[it] >= 0) atomicAdd(&s_h[w][ev[it]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {                 // exclusive over waves, totals
        int run = 0;
        for (int q = 0; q < 16; ++q) {
            const int c = s_h[q][e];
            s_h[q][e] = run;
            run += c;
        }
        s_tot[e] = run;
    }
    __syncthreads();
    const int v = tid < E ? s_tot[tid] : 0;               // exclusive scan over experts
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[w] = x;
    __syncthreads();
    int wb = 0;
    for (int q = 0; q < w; ++q) wb += s_wave[q];
    const int off_e = x - v + wb;
    if (tid < E) {
        offsets[tid] = off_e;
        s_tot[tid] = off_e;
    }
    if (tid == 0) offsets[E] = n;
    __syncthreads();
    for (int e = tid; e < E; e += 1024)
        for (int q = 0; q < 16; ++q) s_h[q][e] += s_tot[e];
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
    for (int it = 0; it < kPackOneSteps; ++it) {
        if (it >= steps) break;                           // uniform
        const int e = ev[it];
        uint64_t peers = __ballot(e >= 0);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t m = __ballot(e >= 0 && ((e >> b) & 1));
            peers &= (e >= 0 && ((e >> b) & 1)) ? m : ~m;
        }
        if (e >= 0) {
            const int idx = b0 + it * 64 + lane;
            const int p = s_h[w][e] + __popcll(peers & lt);
            row_token[p] = idx / topk;
            pos[idx] = p;
        }
        // every lane has read its expert's next row before the first peer moves it
        __builtin_amdgcn_wave_barrier();
        if (e >= 0 && __popcll(peers & lt) == 0) s_h[w][e] += __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
}

// ---------------------------------------------------------------- combine --
template <bool kBf16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y,
                                                 const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int64_t T, int topk,
                                                 int64_t N, float* __restrict__ out) {
    const int64_t groups = N / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= T * groups) return;
    const int64_t t = gid / groups;
    const int64_t c = (gid - t * groups) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < topk; ++s) {
        const float ws = w[t * topk + s];
        const int64_t p = pos[t * topk + s];
        float v[8];
        if (kBf16) {
            const uint4 q = *reinterpret_cast<const uint4*>((const uint16_t*)y + p * N + c);
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(u[i] << 16);
                v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            }
        } else {
            const float4* q = reinterpret_cast<const float4*>((const float*)y + p * N + c);
            const float4 a = q[0], b = q[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws, v[i], acc[i]);
    }
    float4* o = reinterpret_cast<float4*>(out + t * N + c);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

}  // namespace quads

using namespace quads;

extern "C" size_t quads_moe_pack_ws(int64_t T, int32_t topk, int32_t E) {
    if (T < 0 || topk < 1 || E < 1) return 0;
    const int64_t nchunks = (T * topk + kPackChunk - 1) / kPackChunk;
    return align_up((size_t)(nchunks > 0 ? nchunks : 1) * E * 4, 256);
}

extern "C" int quads_moe_pack(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                              int32_t* offsets, int32_t* row_token, int32_t* pos, void* ws,
                              size_t ws_bytes, void* stream) {
    if (T < 0 || topk < 1 || topk > 64 || E < 1 || E > kPackMaxE) return QUADS_ESHAPE;
    if ((int64_t)T * topk >= ((int64_t)1 << 31)) return QUADS_ESHAPE;
    if (!ok_ptr(offsets)) return QUADS_EINVAL;
    if (T > 0 && (!ok_ptr(topk_ids) || !ok_ptr(row_token) || !ok_ptr(pos))) return QUADS_EINVAL;
    if (ws_bytes < quads_moe_pack_ws(T, topk, E) || !ok_ptr(ws)) return QUADS_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int64_t n = T * topk;
    const int nchunks = (int)((n + kPackChunk - 1) / kPackChunk);
    int32_t* cnt = static_cast<int32_t*>(ws);
    if (n > 0 && n <= kPackOneMaxN && E <= kPackOneMaxE) {
        hipLaunchKernelGGL(k_pack_small, dim3(1), dim3(1024), 0, s, topk_ids, (int)n, (int)topk,
                           (int)E, offsets, row_token, pos);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    if (nchunks > 0) {
        hipLaunchKernelGGL(k_pack_count, dim3(nchunks), dim3(256), 0, s, topk_ids, n, (int)E, cnt);
        QUADS_CHECK_LAUNCH();
    }
    if (nchunks > 0 && (int64_t)nchunks * E <= kPackPrefixMax && E % 4 == 0) {
        hipLaunchKernelGGL(k_pack_scatter_prefix, dim3(nchunks), dim3(256), 0, s, topk_ids, n,
                           (int)topk, (int)E, nchunks, cnt, offsets, row_token, pos);
        QUADS_CHECK_LAUNCH();
        return QUADS_OK;
    }
    hipLaunchKernelGGL(k_pack_scan, dim3(1), dim3(1024), 0, s, cnt, nchunks, (int)E, n, offsets);
    QUADS_CHECK_LAUNCH();
    if (nchunks > 0) {
        hipLaunchKernelGGL(k_pack_scatter, dim3(nchunks), dim3(64), 0, s, topk_ids, n, (int)topk,
                           (int)E, cnt, offsets, row_token, pos);
        QUADS_CHECK_LAUNCH();
    }
    return QUADS_OK;
}

extern "C" int quads_moe_combine(const void* y, int y_dtype, const int32_t* pos,
                                 const float* topk_w, int64_t T, int32_t topk, int64_t N,
                                 float* out, void* stream) {
    if (y_dtype != QUADS_OUT_F32 && y_dtype != QUADS_OUT_BF16) return QUADS_EINVAL;
    if (T < 0 || topk < 1 || N <= 0 || N % 8) return QUADS_ESHAPE;
    if (T > 0 && (!ok_ptr(y) || !ok_ptr(pos) || !ok_ptr(topk_w) || !ok_ptr(out)))
        return QUADS_EINVAL;
    if (T == 0) return QUADS_OK;
    hipStream_t s = (hipStream_t)stream;
    const int64_t threads = T * (N / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (y_dtype == QUADS_OUT_BF16)
        hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, y, pos, topk_w, T, (int)topk, N,
                           out);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, y, pos, topk_w, T, (int)topk,
                           N, out);
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}
