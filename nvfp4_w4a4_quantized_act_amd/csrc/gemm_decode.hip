// Grouped W4A4 GEMM for experts with few rows (the decode step): the same
// product as the tiled kernels in gemm.hip -- arXiv 2607.15810, Eq. (6) on
// the compensated activation of Eq. (21) -- laid out for the regime where an
// expert holds a handful of token rows and the weight stream is the cost.
//
// A 256-row tile with four rows in it spends its MFMA work on empty rows and
// converts and stages a full weight tile through LDS per K step.  Here a
// work-group of two waves owns one expert and a 128-row slab of its weight
// matrix (SwiGLU: per wave 32 gate rows and the 32 matching up rows, so the
// epilogue pairs them in registers) and streams it from HBM once per 32 token
// rows of the expert (later passes find it in L2); a work-group of an expert
// without rows leaves at once, so only active experts' weights are read.  An
// expert with more than g.dec_rows rows (kDecodeMaxRows, or all rows when
// there are at most kDecodeAllRows) is left to the tiled kernel, which the
// caller launches after this one (gemm.hip); an expert above kDecodeMaxRows
// rows that this kernel takes is split over work-groups of at most
// kDecodeMaxRows rows each.
//
// Streaming.  A lane (row r = lane % 32, half h = lane / 32) of a wave holds,
// per 128-deep chunk of K, codes 64h .. 64h + 63 of one weight row in each of
// the wave's two 32-row blocks and of one token row, with the block scales
// that cover them.  The loads go straight to registers in that layout, three
// or four chunks ahead of the MFMAs (a ring of named register slots, unrolled
// so the slot of each chunk is fixed and the compiler's waits are plain
// counts).  A chunk is
// converted exactly to fp16 (hardware fp4 -> fp16 convert, then a packed
// multiply by the E4M3 block scale; every v * s_b is an fp16 number) and fed
// to 32x32x16 fp16 MFMAs, weights as the first operand.  MFMA step j of a
// chunk contracts codes 8j .. 8j + 7 of each half, channels k0 + 8j + u and
// k0 + 64 + 8j + u: both operands take the same channels in the same slots,
// so the MFMAs sum exactly the products of Eq. (6).
//
// Scale windows (K of at least two chunks).  The block scales are not
// loaded with the codes: per 4-chunk window each wave brings the 32 scale
// bytes of every row it reads (its two weight blocks and its token rows)
// with one 16-byte direct-to-LDS load per lane -- lane (r, h) the scales of
// chunks w0 + 2 h, w0 + 2 h + 1 of row r -- into one of two LDS buffers, four
// chunks ahead, and each step reads its scale dwords from there.  A 4-byte
// load per lane per piece costs the vector memory pipeline as much as a
// 16-byte one, so this takes a third of the load instructions away.
//
// Accumulation.  The MFMA accumulators restart from zero every kAccChain
// channels and are added into fp32 totals (gfx950's f16 MFMA rounds once per
// group of 8 products, so a chain of 1024 channels is 128 roundings).
//
// Compensation.  The weight columns W[n, sel[i]] are taken from the chunks as
// they stream by (sel ascending: chunk c holds the selected channels in
// [128c, 128c + 128), a uniform range), converted to fp16 and parked in LDS,
// row by row; after the main loop they are the first MFMA operand against the
// residual codes R (second pass of Eq. (21)), accumulated apart from the main
// product since the tensor scale differs:
//   Y = acc_main * s_tA s_tW[e] + acc_comp * s_tR s_tW[e].
#include "common.h"
#include "gemm_tiles.h"

namespace quads {
namespace dec {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 128;          // channels per chunk: 64 codes per lane
constexpr int kRows = 32;            // token rows per pass (one MFMA operand)
constexpr int kCapMax = 64;          // compensation channels kept in LDS
constexpr int kCapLd = kCapMax + 8;  // halfs per LDS row (conflict-free 16-byte reads)

// One lane's share of a chunk of one row: codes 64h .. 64h + 63 and the E4M3
// scales of blocks 4h .. 4h + 3.
struct Piece {
    uint4 lo, hi;
    uint32_t sc;
};

// Rows are addressed as a uniform base plus a 32-bit byte offset per lane.
// The loads are unconditional: a lane without a row reads a valid row and its
// values are zeroed at conversion time through a zero block scale (v * 0 = 0
// for every code), so no branch makes the compiler drain the loads in flight.
template <bool kWin>
__device__ __forceinline__ Piece load_piece(const uint8_t* nib, const uint8_t* sc,
                                            uint32_t nib_off, uint32_t sc_off) {
    const uint4* q = reinterpret_cast<const uint4*>(nib + nib_off);
    Piece p;
    p.lo = q[0];
    p.hi = q[1];
    p.sc = kWin ? 0u : *reinterpret_cast<const uint32_t*>(sc + sc_off);
    return p;
}

// Scale windows: piece h of the window starting at chunk w0 covers chunks
// ps, ps + 1 with ps = min(w0 + 2 h, nch - 2) (no read past a row's scales).
constexpr int kWinChunks = 4;
__device__ __forceinline__ int win_start(int w0, int h, int nch) {
    const int p = w0 + 2 * h;
    return p < nch - 2 ? p : nch - 2;
}
// The scale dword of chunk c for lane (r, h) of a window block (1 KB) whose
// window starts at chunk w0.
__device__ __forceinline__ uint32_t win_scales(const char* blk, int w0, int c, int r, int h,
                                               int nch) {
    const int pi = (c - w0) >> 1;
    const int half = c - win_start(w0, pi, nch);
    return *reinterpret_cast<const uint32_t*>(blk + (32 * pi + r) * 16 + 8 * half + 4 * h);
}

__device__ __forceinline__ uint32_t word(const Piece& p, int j) {
    const uint4 v = j < 4 ? p.lo : p.hi;
    const int i = j & 3;
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// 8 codes (one dword) times an fp16 block scale -> 8 exact fp16 values.
__device__ __forceinline__ f16x8 cvt8(uint32_t w, _Float16 s) {
    const f16x2 s2 = {s, s};
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The four block scales of a piece as fp16 (E4M3 -> fp16 is exact).
__device__ __forceinline__ void scales4(uint32_t sc, _Float16 s[4]) {
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true);
    s[0] = lo[0]; s[1] = lo[1]; s[2] = hi[0]; s[3] = hi[1];
}

// The 8 MFMA steps of one chunk: both weight row blocks against the rows (a
// piece whose row does not exist converts with zero scales).
__device__ __forceinline__ void chunk_mma(const Piece& w0, const Piece& w1, const Piece& a,
                                          const bool wv[2], bool av, f32x16 acc[2]) {
    _Float16 sw0[4], sw1[4], sa[4];
    scales4(wv[0] ? w0.sc : 0u, sw0);
    scales4(wv[1] ? w1.sc : 0u, sw1);
    scales4(av ? a.sc : 0u, sa);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // convert one step at a time: the empty asm pins the step's codes
        // here, so the conversions of all eight steps are not hoisted ahead
        // (about 70 registers); the MFMAs still overlap the next conversions
        uint32_t xa = word(a, j), x0 = word(w0, j), x1 = word(w1, j);
        asm volatile("" : "+v"(xa), "+v"(x0), "+v"(x1));
        const f16x8 af = cvt8(xa, sa[j >> 1]);
        const f16x8 f0 = cvt8(x0, sw0[j >> 1]);
        const f16x8 f1 = cvt8(x1, sw1[j >> 1]);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f0, af, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f1, af, acc[1], 0, 0, 0);
    }
}

// Work units: each expert this kernel takes (0 < rows <= dec_rows) splits
// into units of at most kDecodeMaxRows rows (one unit, unless dec_rows is
// raised above kDecodeMaxRows), so that an expert of many rows is spread over
// work-groups rather than run in many passes by one.  At most
// E + rows / kDecodeMaxRows units.
static __host__ __device__ inline int decode_units_max(const GemmArgs& g) {
    return g.E + (g.dec_rows > kDecodeMaxRows ? (int)(g.rows / kDecodeMaxRows) : 0);
}

// Rows of an n-row expert this kernel takes: its tail (expert_tail) when the
// tiled kernel takes the full 256-row blocks, else all of it when it has
// 1 .. dec_rows rows.  They are the expert's last rows.
__device__ __forceinline__ int decode_rows(const GemmArgs& g, int n) {
    if (g.tail_rows > 0) return expert_tail(n, g.tail_rows);
    return n > 0 && n <= g.dec_rows ? n : 0;
}

// Grid: 8 ceil(units / 8) x slabs work-groups over the units, ranked in
// expert and row order: block b runs on XCD b % 8 and takes slab
// (b / 8) % slabs of the unit of rank 8 ((b / 8) / slabs) + b % 8, so all
// slabs of a unit share one XCD's L2 (where its activation rows stay) and
// the blocks past the last unit, which only look up their unit and leave,
// come last in dispatch order.
// (Ordering by expert index instead interleaved those idle blocks with the
// working ones: at the decode step, 16 active experts of 128 took 45 us
// against 17 us for the same 16 experts alone.)
// kSplit: accumulators restarted every two ring turns into fp32 totals
// (chains longer than kSingleChainMax channels).
// kRing (2, 3 or 4): chunks in flight per wave, chosen so that the chunk count
// is a multiple of it where it can be (the loads past the last chunk are
// wasted work).
template <int kEpi, int kRing, bool kSplit, bool kWin>
__global__ __launch_bounds__(kThreads) void k_gemm_w4a4_decode(GemmArgs g) {
    constexpr bool swiglu = kEpi == QUADS_EPI_SWIGLU;
    // scale windows: [wave][buffer][weight block 0, weight block 1, token rows]
    __shared__ __align__(16) char swin[kWaves][2][3][1024];
    // compensation weight columns, per wave and row block: [row][channel]
    __shared__ __align__(16) _Float16 capt[kWaves][2][32][kCapLd];
    // a chunk's weight pieces, word-major, while its compensation columns are taken
    __shared__ uint32_t stage[kWaves][2][9][64];
    // the selected channels, per wave (read by lane-dependent index in code
    // where some lanes are inactive: no cross-lane reads there)
    __shared__ int s_sel[kWaves][kCapMax];

    const int lane = threadIdx.x & 63;
    const int nslab = (int)(gridDim.x / (8u * (((unsigned)decode_units_max(g) + 7u) / 8u)));
    const int local = (int)(blockIdx.x >> 3);
    const int rank = 8 * (local / nslab) + (int)(blockIdx.x & 7u);
    const int slab = local % nslab;
    int e = 0, p0 = 0, cnt = (int)g.rows;
    if (g.offsets) {
        // the unit of this rank: lane l counts the units of experts l*per ..
        // l*per + per - 1, a wave scan finds the lane, the lane finds the
        // expert and the unit's place in it
        const int per = (g.E + 63) / 64;
        const int e0 = lane * per, e1 = e0 + per < g.E ? e0 + per : g.E;
        int na = 0;
        for (int x = e0; x < e1; ++x) {
            const int n = decode_rows(g, g.offsets[x + 1] - g.offsets[x]);
            na += (n + kDecodeMaxRows - 1) / kDecodeMaxRows;
        }
        const int inc = wave_incl_add(na);
        if (rank >= __builtin_amdgcn_readlane(inc, 63)) {         // uniform: past the last
            if (g.amax) amax_group_none(g);
            return;
        }
        int found = -1, part = 0;
        if (rank >= inc - na && rank < inc) {                       // exactly one lane
            int rr = rank - (inc - na);
            for (int x = e0; x < e1; ++x) {
                const int n = decode_rows(g, g.offsets[x + 1] - g.offsets[x]);
                const int u = (n + kDecodeMaxRows - 1) / kDecodeMaxRows;
                if (rr < u) { found = x; part = rr; break; }
                rr -= u;
            }
        }
        const int src = __ffsll(__ballot(found >= 0)) - 1;
        e = __builtin_amdgcn_readlane(found, src);
        const int taken = decode_rows(g, g.offsets[e + 1] - g.offsets[e]);
        p0 = g.offsets[e + 1] - taken + kDecodeMaxRows * __builtin_amdgcn_readlane(part, src);
        cnt = min(g.offsets[e + 1] - p0, kDecodeMaxRows);
    } else if (rank > 0 || cnt <= 0 || cnt > g.dec_rows) {
        if (g.amax) amax_group_none(g);
        return;                                       // one expert, all rows
    }
    bind_expert(g, e);

    // the wave index as a scalar, so that every branch on it is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 31, h = lane >> 5;
    const uint32_t kn = (uint32_t)g.K / 2, ks = (uint32_t)g.K / kBlock;

    // the expert's weights (uniform base) and the lane's rows in the wave's
    // two 32-row blocks
    const uint8_t* wnib = g.w_nib + (int64_t)e * g.N * kn;
    const uint8_t* wsc = g.w_scale + (int64_t)e * g.N * ks;
    uint32_t wrow_n[2], wrow_s[2];
    const uint8_t* wsrow[2];
    bool wv[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        int row;
        if (swiglu) {
            const int feat = slab * 64 + wave * 32 + r;
            wv[q] = feat < g.N / 2;
            row = q * (g.N / 2) + feat;
        } else {
            row = slab * 128 + wave * 64 + 32 * q + r;
            wv[q] = row < g.N;
        }
        row = wv[q] ? row : 0;
        wrow_n[q] = (uint32_t)row * kn + 32 * h;
        wrow_s[q] = (uint32_t)row * ks + 4 * h;
        wsrow[q] = wsc + (uint64_t)row * ks;
    }

    const int nch = g.K / kChunk;
    const int ncs = g.k / kBlock;                     // compensation steps of 16
    const float s_tw = g.w_ts[e];
    const float ca = tensor_scale_a(g) * s_tw;
    const float cr = g.k > 0 ? g.r_ts[0] * s_tw : 0.0f;

    // the selected channels, one per lane, read back one at a time as scalars
    int sel_lo = 0;
    if (g.k > 0) {                                    // a column never captured reads as 0
        for (int i = lane; i < 2 * 32 * kCapLd / 8; i += 64)
            reinterpret_cast<uint4*>(&capt[wave][0][0][0])[i] = make_uint4(0, 0, 0, 0);
        sel_lo = lane < g.k ? g.sel[lane] : 0;
        s_sel[wave][lane] = sel_lo;
    }

    uint32_t hmax = 0;                                // largest |h| stored (SwiGLU)
    for (int c0 = 0; c0 < cnt; c0 += kRows) {
        const bool rv = c0 + r < cnt;
        const int p = p0 + c0 + r;
        // acc: the MFMA chain, restarted every kAccChain channels into the
        // fp32 totals tot (the error bound of split accumulation)
        f32x16 acc[2], tot[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) { acc[q][v] = 0.0f; tot[q][v] = 0.0f; }

        // The ring: chunk c lives in slot c % kRing (named slots, no array,
        // so everything stays in registers); loads past the last chunk repeat
        // it (no branch) and are never used.  The prologue issues its loads in
        // the steady state's order (the weights of chunk c, then its token
        // rows), after the token-row index: the load counter waits are shared
        // by every turn of the loop, and any other order would make them the
        // prologue's (one chunk in flight instead of kRing - 1).
        const int64_t src = rv ? (g.row_token ? (int64_t)g.row_token[p] : (int64_t)p) : 0;
        auto ldw = [&](Piece& w0, Piece& w1, int c) {
            const uint32_t cl = (uint32_t)(c < nch ? c : nch - 1);
            w0 = load_piece<kWin>(wnib, wsc, wrow_n[0] + 64 * cl, wrow_s[0] + 8 * cl);
            w1 = load_piece<kWin>(wnib, wsc, wrow_n[1] + 64 * cl, wrow_s[1] + 8 * cl);
        };
        // the token row: a per-lane base (the activation tensor may exceed 4 GB)
        const uint8_t* an = g.a_nib + src * kn + 32 * h;
        const uint8_t* as = g.a_scale + src * ks + 4 * h;
        const uint8_t* asrow = g.a_scale + src * ks;
        auto lda = [&](Piece& a, int c) {
            const uint32_t cl = (uint32_t)(c < nch ? c : nch - 1);
            a = load_piece<kWin>(an, as, 64 * cl, 8 * cl);
        };
        // the scale window of chunks w0 .. w0 + 3 into buffer `b`
        const uint32_t swin_lds = lds_addr(&swin[wave][0][0][0]);
        auto stage_win = [&](int w0, int b) {
            if (!kWin) return;
            const int ps = win_start(w0, h, nch);
            const uint32_t l = swin_lds + 3072 * b;
            g2l16(wsrow[0] + 8 * ps, l);
            g2l16(wsrow[1] + 8 * ps, l + 1024);
            g2l16(asrow + 8 * ps, l + 2048);
        };
        // the previous pass's last window reads are done before the buffers
        // are written again
        if (kWin && c0 > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_win(0, 0);
        Piece w0a, w1a, aa, w0b, w1b, ab, w0c, w1c, ac, w0d, w1d, ad;
        ldw(w0a, w1a, 0);
        lda(aa, 0);
        ldw(w0b, w1b, 1);
        lda(ab, 1);
        if (kRing >= 3) {
            ldw(w0c, w1c, 2);
            lda(ac, 2);
        }
        if (kRing == 4) {
            ldw(w0d, w1d, 3);
            lda(ad, 3);
        }
        // the residual codes of this pass's rows (k <= 64: at most 4 steps of
        // 16 channels, a dword of codes and a scale byte each), requested now
        // so the compensation after the main loop waits for nothing
        uint32_t rw[kCapMax / kBlock], rs[kCapMax / kBlock];
#pragma unroll
        for (int t = 0; t < kCapMax / kBlock; ++t) {
            const int tt = t < ncs ? t : 0;
            rw[t] = ncs > 0 ? *reinterpret_cast<const uint32_t*>(g.r_nib + src * (g.k / 2) +
                                                                 8 * tt + 4 * h)
                            : 0u;
            rs[t] = ncs > 0 ? g.r_scale[src * ncs + tt] : 0u;
        }
        int ci = 0;                                   // next compensation channel to capture
        auto step = [&](Piece& w0, Piece& w1, Piece& a, int c) {
            if (c < nch) {
                if (kWin) {
                    const int wb = (c / kWinChunks) & 1;
                    const int w0c = c - c % kWinChunks;
                    // this chunk's codes have arrived (the compiler waits for
                    // them here), and with them its window, requested before
                    // them; then its scale dwords
                    asm volatile("" ::"v"(w0.lo.x), "v"(w1.lo.x), "v"(a.lo.x) : "memory");
                    const char* blk = &swin[wave][wb][0][0];
                    w0.sc = win_scales(blk, w0c, c, r, h, nch);
                    w1.sc = win_scales(blk + 1024, w0c, c, r, h, nch);
                    a.sc = win_scales(blk + 2048, w0c, c, r, h, nch);
                    // the next window, into the buffer the previous one used
                    // (last read one chunk ago)
                    if (c % kWinChunks == 0 && c + kWinChunks < nch) {
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        stage_win(c + kWinChunks, wb ^ 1);
                    }
                }
                if (c0 == 0 && ci < g.k &&
                    __builtin_amdgcn_readlane(sel_lo, ci) < kChunk * (c + 1)) {
                    // capture W[:, sel[i]] for the selected channels in this
                    // chunk: channel j of the chunk is code j % 64 of half
                    // j / 64, in dword (j % 64) / 8.  The pieces go to LDS
                    // word-major, so a uniform word index is one LDS read.
#pragma unroll
                    for (int d = 0; d < 8; ++d) {
                        stage[wave][0][d][lane] = word(w0, d);
                        stage[wave][1][d][lane] = word(w1, d);
                    }
                    stage[wave][0][8][lane] = wv[0] ? w0.sc : 0u;
                    stage[wave][1][8][lane] = wv[1] ? w1.sc : 0u;
                    // channels ci .. cend - 1 lie in this chunk (sel ascending);
                    // the (row, channel) pairs are spread over the 64 lanes,
                    // each reading the staged word of the lane that holds it
                    const int cend = __popcll(__ballot(lane < g.k && sel_lo < kChunk * (c + 1)));
                    for (int idx = lane; idx < 32 * (cend - ci); idx += 64) {
                        const int rr = idx & 31, ch = ci + (idx >> 5);
                        const int j = s_sel[wave][ch] - kChunk * c;
                        if (j < 0 || j >= kChunk) continue;   // not ascending: skipped (reads 0)
                        const int src = rr + 32 * (j >> 6), jj = j & 63;
                        const int sh = 4 * (jj & 7), sb = 8 * (jj >> 4);
                        const uint32_t y0 = stage[wave][0][jj >> 3][src];
                        const uint32_t y1 = stage[wave][1][jj >> 3][src];
                        const uint32_t b0 = (stage[wave][0][8][src] >> sb) & 0xFFu;
                        const uint32_t b1 = (stage[wave][1][8][src] >> sb) & 0xFFu;
                        capt[wave][0][rr][ch] =
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((y0 >> sh) & 0xFu, 1.0f, 0)[0] *
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, 1.0f, false)[0];
                        capt[wave][1][rr][ch] =
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((y1 >> sh) & 0xFu, 1.0f, 0)[0] *
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, 1.0f, false)[0];
                    }
                    ci = cend;
                }
                chunk_mma(w0, w1, a, wv, rv, acc);
            }
            // the slot's next chunk is requested after this chunk's work, so
            // it reuses the slot's registers (hoisting it would need a second
            // set)
            __builtin_amdgcn_sched_barrier(0);
            ldw(w0, w1, c + kRing);
            lda(a, c + kRing);
        };
        auto flush = [&]() {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) { tot[q][v] += acc[q][v]; acc[q][v] = 0.0f; }
        };
        for (int cb = 0; cb < nch; cb += kRing) {
            step(w0a, w1a, aa, cb);
            step(w0b, w1b, ab, cb + 1);
            if (kRing >= 3) step(w0c, w1c, ac, cb + 2);
            if (kRing == 4) step(w0d, w1d, ad, cb + 3);
            // with split accumulation a chain is two ring turns (4 chunks,
            // 512 channels); otherwise one chain covers every chunk
            if (kSplit && ((cb / kRing) & 1)) flush();
        }
        if (kSplit) flush();

        // compensation: captured columns against this pass's residual rows,
        // in the same accumulators once the main product, scaled, has moved
        // to registers the ring no longer needs
        const float ca_row = g.a_ts_rows ? g.a_ts_rows[src] * ca : ca;   // per-row scales
        float ym[2][16];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                ym[q][v] = (kSplit ? tot[q][v] : acc[q][v]) * ca_row;
                acc[q][v] = 0.0f;
            }
#pragma unroll
        for (int t = 0; t < kCapMax / kBlock; ++t) {
            if (t < ncs) {
                const f16x8 rf = cvt8(rv ? rw[t] : 0u, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                                                           rv ? rs[t] : 0u, 1.0f, false)[0]);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const f16x8 wf =
                        *reinterpret_cast<const f16x8*>(&capt[wave][q][r][16 * t + 8 * h]);
                    acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf, rf, acc[q], 0, 0, 0);
                }
            }
        }

        // epilogue: lane holds output row c0 + r; registers 4g .. 4g + 3 are
        // features 8g + 4h .. 8g + 4h + 3 of each 32-row block
        if (rv) {
            const int nq = 4 * h;
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                float y[2][4];
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        y[q][u] = ym[q][4 * grp + u] + acc[q][4 * grp + u] * cr;
                if (swiglu) {
                    const int nh = g.N / 2;
                    const int feat = slab * 64 + wave * 32 + 8 * grp + nq;
                    const uint32_t p01 = v2::pk_bf16(silu_mul(y[0][0], y[1][0]),
                                                     silu_mul(y[0][1], y[1][1]));
                    const uint32_t p23 = v2::pk_bf16(silu_mul(y[0][2], y[1][2]),
                                                     silu_mul(y[0][3], y[1][3]));
                    uint16_t* o = (uint16_t*)g.out + (int64_t)p * nh + feat;
                    if (feat + 3 < nh && (nh & 3) == 0) {
                        *reinterpret_cast<uint2*>(o) = make_uint2(p01, p23);
                        hmax = umax32(hmax, umax32(bf16x2_mag_max(p01), bf16x2_mag_max(p23)));
                    } else {
                        const uint32_t hb[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu,
                                                p23 >> 16};
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (feat + u < nh) {
                                o[u] = (uint16_t)hb[u];
                                hmax = umax32(hmax, hb[u] & 0x7FFFu);
                            }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int n = slab * 128 + wave * 64 + 32 * q + 8 * grp + nq;
                        const int64_t o = (int64_t)p * g.N + n;
                        const bool vec = n + 3 < g.N && (g.N & 3) == 0;
                        if (g.out_bf16) {
                            uint16_t* ob = (uint16_t*)g.out + o;
                            const uint32_t p01 = v2::pk_bf16(y[q][0], y[q][1]);
                            const uint32_t p23 = v2::pk_bf16(y[q][2], y[q][3]);
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
                                *reinterpret_cast<float4*>(of) =
                                    make_float4(y[q][0], y[q][1], y[q][2], y[q][3]);
                            } else {
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    if (n + u < g.N) of[u] = y[q][u];
                            }
                        }
                    }
                }
            }
        }
    }
    if (swiglu && g.amax) amax_group_store(g, hmax, reinterpret_cast<uint32_t*>(&swin[0][0][0][0]));
}

}  // namespace dec

// The decode kernel for the tails of experts just above a multiple of 256
// rows (tail_rows set by the caller): its shape rules without the
// rows-per-expert limit.
bool gemm_decode_tail_fits(const GemmArgs& g) {
    const int64_t slabs = g.epilogue == QUADS_EPI_SWIGLU ? (g.N / 2 + 63) / 64 : (g.N + 127) / 128;
    return g.offsets != nullptr && g.K % dec::kChunk == 0 && g.k <= dec::kCapMax &&
           slabs * 8 * ((g.E + 7) / 8) < ((int64_t)1 << 31) &&
           (int64_t)g.N * g.K / 2 < ((int64_t)1 << 31);
}

bool gemm_decode_fits(const GemmArgs& g) {
    const int64_t slabs = g.epilogue == QUADS_EPI_SWIGLU ? (g.N / 2 + 63) / 64 : (g.N + 127) / 128;
    return g.K % dec::kChunk == 0 && g.k <= dec::kCapMax &&
           g.rows <= (int64_t)kDecodeRowsPerExpert * g.E &&
           slabs * 8 * ((g.E + kDecodeAllRows / kDecodeMaxRows + 7) / 8) < ((int64_t)1 << 31) &&
           (int64_t)g.N * g.K / 2 < ((int64_t)1 << 31);
}

int launch_gemm_decode(GemmArgs g, hipStream_t st, LaunchPlan* lp) {
    const int64_t slabs = g.epilogue == QUADS_EPI_SWIGLU ? (g.N / 2 + 63) / 64 : (g.N + 127) / 128;
    const int64_t blocks = slabs * 8 * ((dec::decode_units_max(g) + 7) / 8);
    g.amax_base = lp->blocks;
    lp->blocks += blocks;
    if (lp->dry) return QUADS_OK;
    const dim3 grid((unsigned)blocks), block(dec::kThreads);
    const int nch = g.K / dec::kChunk;
    const bool ring3 = nch % 4 != 0 && nch % 3 == 0;
    const bool sw = g.epilogue == QUADS_EPI_SWIGLU;
    // a chain longer than kSingleChainMax channels needs split accumulation;
    // its totals take registers, so that variant keeps two chunks in flight
    // per wave (two waves per SIMD instead of one: the same loads in flight)
    const bool split = g.K + g.k > kSingleChainMax;
    // scale windows need two chunks per row (a window piece covers two)
    const bool win = nch >= 2;
#define QUADS_DEC(EPI, RING, SPLIT)                                                             \
    do {                                                                                        \
        if (win)                                                                                \
            hipLaunchKernelGGL((dec::k_gemm_w4a4_decode<EPI, RING, SPLIT, true>), grid, block,  \
                               0, st, g);                                                       \
        else                                                                                    \
            hipLaunchKernelGGL((dec::k_gemm_w4a4_decode<EPI, RING, SPLIT, false>), grid, block, \
                               0, st, g);                                                       \
    } while (0)
    if (split) {
        if (sw) QUADS_DEC(QUADS_EPI_SWIGLU, 2, true);
        else QUADS_DEC(QUADS_EPI_NONE, 2, true);
    } else if (sw && ring3) {
        QUADS_DEC(QUADS_EPI_SWIGLU, 3, false);
    } else if (sw) {
        QUADS_DEC(QUADS_EPI_SWIGLU, 4, false);
    } else if (ring3) {
        QUADS_DEC(QUADS_EPI_NONE, 3, false);
    } else {
        QUADS_DEC(QUADS_EPI_NONE, 4, false);
    }
#undef QUADS_DEC
    QUADS_CHECK_LAUNCH();
    return QUADS_OK;
}

}  // namespace quads
