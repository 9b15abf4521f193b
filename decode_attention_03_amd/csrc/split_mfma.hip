// split_mfma.hip -- split stage for grouped-query attention on the gfx950
// matrix cores.
//
// Sources (pages; sections as printed on them):
//   [P1] "FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15)
//   [P3] "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
//        (my-webpage-adu.pages.dev, 2026-07-16)
//   [P4] "从第一性原理推导 Flash Attention：IO 复杂度、Tiling 策略与在线 Softmax 的数学工程"
//        (www.ybb.press), §8 item 1 (grouped-query attention: fewer KV heads)
//
// When G = heads_q / heads_kv query heads share one KV head, every K and V
// row a split reads serves G query rows, and the split step is a small dense
// contraction: S = Q_g K_tile^T (G x tokens) and O += P V_tile.  For G <= 16
// one wave (one work-group) owns one (sequence b, KV head, split i) and the
// tokens [i*L, min((i+1)*L, N_b)) ([P1] §2.5 stage 1), in tiles of 16
// tokens (larger groups, and a prefix shared by the whole batch, use the
// tiled kernel further down: 16-query tiles, several per work-group, on up to
// eight waves that share each K/V step staged in LDS):
//
//   S^T (16 tokens x 16 heads) = K_tile (16 x d) . Q_g^T (d x 16):
//     v_mfma_f32_16x16x32 over d.  A 128-bit load of 8 contiguous d-elements
//     of one token is already an A-operand fragment; Q_g^T (zero beyond G
//     heads) stays in registers.  The result leaves each lane with 4 tokens
//     of one head.
//   online softmax per head ([P1] §2.4.1; [P4] §3.1): the reference max m
//     of a head only moves (and O, l are rescaled) when a score exceeds it
//     by more than 2^8 ([P4] §3.2: any common reference gives the same
//     result); the four lanes holding a head then agree on the new max
//     through two shuffles.  In steady state a step costs one ballot.
//     p = exp2(s - m) is rounded to the input type for the matrix core; o is
//     normalised by the sum of the rounded weights (so the weights applied
//     to V sum to 1) and the LSE uses the sum of the fp32 weights.
//   O (16 heads x d) += P (16 x 16 tokens) . V_tile (16 x d):
//     v_mfma_f32_16x16x16, one per 16-wide d slice.  P is the A operand
//     exactly as the S step left it.  V, stored row-major (tokens x d) in
//     LDS, is read back with ds_read_b64_tr_b16, which hands each lane four
//     tokens of one d column: the B-operand fragment.
//
// Data movement: each step's K and V tiles are loaded with the same
// pattern as the vector kernel (16-byte non-temporal loads, 16 lanes per
// 256-byte head row, so one instruction reads whole rows), into one of two
// register sets; up to d = 128 a set is refilled with the loads two steps
// ahead as soon as its rows are staged in LDS, so two steps of loads stay in
// flight while a step is read back and computed.  The staging writes each row
// to LDS with its 16-byte chunks XOR-swizzled by the row index, which keeps
// the 128-bit fragment reads of K and the transpose reads of V free of bank
// conflicts.
// (Direct-to-LDS loads were measured slower here: their LDS destination is
// opaque to the compiler's wait counting, which then allows only one batch in
// flight per wave.)  Steps are 8 KB of K+V per wave (one 16-token tile of
// each at d = 128) and at most kMfmaWgPerCU = 2 work-groups are resident per CU
// (LDS reservation), as in the vector kernel: fewer concurrent request streams
// keep HBM nearer its efficient depth.  (Measured against 3 or 4 per CU, 16 KB
// steps, a third register set of loads in flight, and K fragments loaded
// straight from HBM without the LDS round trip, each slower.)
//
// The split writes o = O / l and S = m + log l per query head ([P3]
// §2.3.2-§2.3.3), or, in the m/l/o format, o with the split's max score m and
// l = sum exp(s - m) ([P1] §2.4.1 direct form).  Scores are in the log2 domain (scale * log2(e) applied to
// the fp32 MFMA result).
#include <atomic>

#include "dev_common.h"
#include "partition.h"

namespace fd {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

[[maybe_unused]] constexpr float kRescaleGap = 8.f;  // log2 units the running max may lag

template <int DT>
struct Mma;

template <>
struct Mma<kBF16> {
    static __device__ __forceinline__ f32x4_t s_tile(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
    }
    static __device__ __forceinline__ f32x4_t pv_tile(u32x2 a, s16x4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), b, c, 0,
                                                         0, 0);
    }
    // P . V over two token tiles in one product: a holds the weights of
    // tiles u and u + 1, b0 / b1 their V fragments (see the step body).
    static __device__ __forceinline__ f32x4_t pv_tile2(u32x4 a, s16x4_t b0, s16x4_t b1,
                                                       f32x4_t c) {
        const s16x8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
    }
    // Round four weights to bf16 (nearest even), two per conversion; returns
    // the packed pair and adds the rounded values to *sum.
    static __device__ __forceinline__ u32x2 pack(const float *p, float *sum) {
        const bf16x2_t lo = __builtin_convertvector((f32x2_t){p[0], p[1]}, bf16x2_t);
        const bf16x2_t hi = __builtin_convertvector((f32x2_t){p[2], p[3]}, bf16x2_t);
        *sum += ((float)lo[0] + (float)lo[1]) + ((float)hi[0] + (float)hi[1]);
        return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    }
};

template <>
struct Mma<kF16> {
    static __device__ __forceinline__ f32x4_t s_tile(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv_tile(u32x2 a, s16x4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv_tile2(u32x4 a, s16x4_t b0, s16x4_t b1,
                                                       f32x4_t c) {
        const s16x8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x2 pack(const float *p, float *sum) {
        const f16x2_t lo = __builtin_convertvector((f32x2_t){p[0], p[1]}, f16x2_t);
        const f16x2_t hi = __builtin_convertvector((f32x2_t){p[2], p[3]}, f16x2_t);
        *sum += ((float)lo[0] + (float)lo[1]) + ((float)hi[0] + (float)hi[1]);
        return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    }
};

#ifndef FD_MFMA_STEP_KB
#define FD_MFMA_STEP_KB 8
#endif
// Weights computed after the rescale check (0) or speculatively before it,
// against the reference max as it stands, and redone in the rare rescale
// branch (1): the check's ballot then no longer sits between the scores and
// the exponentials.
#ifndef FD_SPEC_WEIGHTS
#define FD_SPEC_WEIGHTS 1
#endif
// P . V of a step with an even number of token tiles: one 16x16x32 product
// per pair of tiles and d tile (1) or one 16x16x16 product per tile (0).
#ifndef FD_PV32
#define FD_PV32 1
#endif

template <int D, int STEP_KB = FD_MFMA_STEP_KB>
struct Tiles {
    static constexpr int ROW = D * 2;         // bytes of one head row (16-bit types)
    static constexpr int CPR = ROW / 16;      // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;      // rows per 1 KB direct-to-LDS instruction
    static constexpr int NC = D / 32;         // K-dim chunks of the S product (32 elements)
    static constexpr int NT = D / 16;         // 16-wide d slices of O
    static constexpr int TILE = 16 * ROW;     // bytes of one 16-token tile of K or V
    static constexpr int IPT = TILE / 1024;   // direct-to-LDS instructions per tile
    // 16-token tiles per step: FD_MFMA_STEP_KB of K+V per wave and step
    static constexpr int U = STEP_KB * 1024 / (2 * TILE) > 0 ? STEP_KB * 1024 / (2 * TILE) : 1;
    static constexpr int BUF = 2 * U * TILE;  // LDS: U tiles of K, then U tiles of V
    // Chunk swizzles: physical chunk p of row r holds logical chunk
    // p ^ swz_k(r) in a K tile and p ^ swz_v(r) in a V tile.  gfx950 LDS has
    // 64 four-byte banks.  Chosen from the LDS bank-conflict counter on
    // micro-benchmarks of exactly these two access patterns (16 x 256-byte
    // tiles): the K fragment reads (128-bit, one logical chunk in each of 16
    // rows) run conflict-free with swz_k(r) = r, while the V transpose reads
    // (served 32 lanes per pass: two adjacent chunks, one 16-wide d slice, in
    // each of 8 rows) need swz_v >> 1 distinct on 8 consecutive rows, which
    // 2*(r mod 8) + r/8 gives.  128-byte rows (d = 64) alternate between the
    // two bank halves, so there the V condition applies to rows of one
    // parity: 2*((r/2) mod 4) + r/8.
    static __device__ __forceinline__ int swz_k(int r) { return r & ((CPR < 16 ? CPR : 16) - 1); }
    static __device__ __forceinline__ int swz_v(int r) {
        if (CPR >= 16)
            return ((r & 7) << 1) | (r >> 3);
        return (((r >> 1) & 3) << 1) | (r >> 3);
    }
};

typedef __attribute__((address_space(3))) char lds_char;

// K/V bytes per step of the tiled kernel (both halves).
#ifndef FD_PREFIX_STEP_KB
#define FD_PREFIX_STEP_KB 16
#endif
constexpr int kPrefixStepKB = FD_PREFIX_STEP_KB;  // K/V bytes per step of the tiled kernel
// Work-groups of several waves (tiled and token-balanced kernels): K/V bytes
// per step, shared by the waves (0: 8 KB per wave); non-temporal loads (1),
// ordinary loads (0), or (-1) non-temporal when each wave holds one query
// tile and ordinary when it holds more (measured: with one tile per wave the
// non-temporal hint is 3-9 % faster, with two it is 4 % slower).
#ifndef FD_WIDE_STEP_KB
#define FD_WIDE_STEP_KB 0
#endif
#ifndef FD_WIDE_NT
#define FD_WIDE_NT -1
#endif
// Work-groups of several waves: register sets of K/V loads in flight per wave
// (2: the next two steps; more keeps deeper pipelines of loads going while
// the waves wait for each other at every step's barrier).  Contiguous K/V at
// d <= 128 only; paged K/V and d = 256 keep two.
#ifndef FD_WIDE_SETS
#define FD_WIDE_SETS 2
#endif
template <int D, bool PAGED, int W>
constexpr int wide_sets() {
    return (W > 1 && !PAGED && D <= 128) ? FD_WIDE_SETS : 2;
}
#ifndef FD_MFMA_NT
#define FD_MFMA_NT 1  // one-wave grouped kernels: non-temporal K/V loads
#endif
// 0: 8 KB per wave (16 KB for two waves, 32 KB for four)
template <int W>
constexpr int wide_step_kb() {
    // eight waves (two per SIMD, 256 registers each): 16 KB, so that a step's
    // fragments fit
    return FD_WIDE_STEP_KB > 0 ? FD_WIDE_STEP_KB : (W > 4 ? 16 : 8 * W);
}
// Token-balanced work-groups of four one-tile waves at d <= 128: 16 KB steps
// and two waves per SIMD (two work-groups per CU), which measured 1.5-5 %
// faster there than 32 KB steps at one wave per SIMD (on the tiled kernel's
// fixed splits the same change was slower).
template <int D, int QT, int W>
constexpr bool bal_two_per_simd() {
    return fd::bal_two_per_simd(D, QT, W);
}
template <int QT>
constexpr int wide_nt() {
    return FD_WIDE_NT < 0 ? (QT == 1 ? 1 : 0) : FD_WIDE_NT;
}

// Whether a step of a piece is full (every token before the piece's end), as
// a type, so that both kinds of step are compiled without a per-score branch.
template <bool FULL>
struct StepKind {
    static constexpr bool value = FULL;
};

// Where a piece's results go.  Partial i of query row `row` (slot h of a
// tile when `local`) is at index (row or h) * stride + off: o at o + index * D
// (fp32, normalised), its LSE at lse[index] (m/l/o format: m there and l at
// l[index]).  With o null the piece covers whole rows and writes the final
// output (a.o, a.lse) itself.
struct PieceOut {
    float *o;
    float *lse;
    float *l;
    int stride, off;
    bool local;
};

// The query rows one work-group serves, in tiles of 16 (the matrix-core
// width).  nq == 0: the G query heads of (sequence b, KV head kvh), in
// ceil(G / 16) tiles (one for G <= 16).
// Tiled: the queries of KV head kvh numbered qi = 0 .. nq - 1 (the G heads of
// sequence b, or for a shared prefix all batch * G queries, sequence
// qi / G), tiles tile0, tile0 + 1, ...  row() is the query's row in
// q [batch * heads_q, d], -1 for an unused slot.
struct QMap {
    int base;   // a group's own tiles: b * heads_q + kvh * G; tiled: b * heads_q (0 for a
                // shared prefix)
    int G;
    int nq;     // tiled: queries of the KV head (G, or batch * G for a shared prefix); 0: the
                // G heads of (b, kvh) from base
    int tile0;
    int heads_q, kvh;
    __device__ __forceinline__ int row(int qt, int i) const {
        const int qi = (tile0 + qt) * 16 + i;
        if (nq == 0)
            return qi < G ? base + qi : -1;
        return qi < nq ? base + (qi / G) * heads_q + kvh * G + qi % G : -1;
    }
};

#if defined(__HIP_DEVICE_COMPILE__)
// One piece: tokens [t0, t1) of KV head kvh of sequence b (of the shared
// cache when a.shared_kv) for QT tiles of 16 query rows (qm).  Every K/V tile
// staged in LDS serves all QT tiles.  K/V loads carry the non-temporal hint
// (NTLOAD) unless other work-groups will read the same rows.  Called by the whole wave; t0 >= t1
// writes (0, -inf).  (Device pass only: the body uses LDS address-space
// pointers and gfx950-only builtins that the host pass cannot type.)
template <int DT, int D, bool PAGED, int QT, int NTLOAD = 1, int STEP_KB = FD_MFMA_STEP_KB,
          int W = 1, int NS = 2>
__device__ __forceinline__ void mfma_piece(const SplitArgs &a, lds_char *const tb, int b, int kvh,
                                           long t0, long t1, const QMap &qm,
                                           const PieceOut &out) {
    using T = Tiles<D, STEP_KB>;
    constexpr int NC = T::NC, NT = T::NT, U = T::U;
    using M = Mma<DT>;
    // W waves share each step, and all of them compute on all of its rows
    // (two LDS buffers, one barrier per step; W == 1: one wave, one buffer,
    // no barrier).  The loads are shared out by 1 KB row group: with no more
    // waves than a tile has row groups (IPT), wave wv loads row groups wv,
    // wv + W, ... of every tile; with more, the R = W / IPT waves with the
    // same wv % IPT take every R-th tile, starting at tile wv / IPT.
    constexpr int R = W > T::IPT ? W / T::IPT : 1;
    static_assert(W <= T::IPT ? T::IPT % W == 0 : (W % T::IPT == 0 && U % R == 0),
                  "a step's row groups must divide evenly among the waves");
    constexpr int TU = U / R;                        // tiles a wave loads rows of
    constexpr int JW = W > T::IPT ? 1 : T::IPT / W;  // row groups per tile a wave loads

    const int lane = W > 1 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int wv = W > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    const int col = lane & 15;  // tile token (K reads) / query slot (S) / d column (O)
    const int grp = lane >> 4;  // 0..3

    f32x4_t oacc[QT][NT];  // O[slot 4*grp + r][16*t + col] of each tile
    float m_used[QT];      // reference max of slot `col` (log2 domain)
    // This lane's share of l for slot `col`, twice: over the weights as
    // rounded for the matrix core (o is normalised by it, so the weights
    // applied to V sum to exactly 1) and over the fp32 weights (the LSE uses
    // it, free of the rounding).  (Summing the rounded weights on the matrix
    // cores instead, as P . ones, measured 4 us slower per step on the ragged
    // grouped-query batch: one more dependent product per token tile.)
    float lsum[QT], lexact[QT];
    float mtrue[QT];  // max of this lane's scores (the m/l/o format's m)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            oacc[qt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_used[qt] = -INFINITY;
        lsum[qt] = 0.f;
        lexact[qt] = 0.f;
        mtrue[qt] = -INFINITY;
    }

    if (t0 < t1) {
        // Q^T fragments: query slot `col` of each tile, d = 32c + 8*grp + [0, 8);
        // unused slots stay zero (their rows are never written).
        u32x4 qf[QT][NC];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int qr = qm.row(qt, col);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                qf[qt][c] = u32x4{0u, 0u, 0u, 0u};
            if (qr >= 0) {
                const char *qrow = static_cast<const char *>(a.q) + (size_t)qr * T::ROW;
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    qf[qt][c] = ld128<0>(qrow + c * 64 + grp * 16);
            }
        }
        const size_t tok_stride = (size_t)a.heads_kv * T::ROW;
        const int ntok = (int)(t1 - t0);
        constexpr int kStepTok = 16 * U;
        const int nsteps = (ntok + kStepTok - 1) / kStepTok;

        // One step's loads: for tile u and row group j, lane L reads the
        // 16-byte chunk q = L % CPR of row r = j*RPI + L/CPR (token
        // first + 16u + r, clamped to the last valid token; a step past the
        // last one re-reads the last step, so prefetches need no condition).
        struct Stage {
            u32x4 k[TU][JW];
            u32x4 v[TU][JW];
        };
        // the tile and row group of this wave's uu-th tile and jj-th row group
        const int u_first = W > T::IPT ? wv / T::IPT : 0;
        auto tile_of = [&](int uu) { return uu * R + u_first; };
        auto group_of = [&](int jj) { return W > T::IPT ? wv % T::IPT : jj * W + wv; };
        const int lrow = lane / T::CPR;  // row within a row group
        const int lq = lane % T::CPR;    // logical chunk this lane carries
        const size_t lane_off = (size_t)kvh * T::ROW + lq * 16;
        // Paged K/V: the page of each of a step's U tiles, read before the
        // step's loads (see the loop below for when).  A tile is 16-aligned
        // (so are t0 and the step start), so it lies in one page, also after
        // its rows are clamped to the last valid token.
        struct Pages {
            int pg[TU];  // of the tiles this wave loads
        };
        auto lookup = [&](int st, Pages &P) {
            if constexpr (PAGED) {
                const int sa = st < nsteps ? st : nsteps - 1;
                const int first = sa * kStepTok;
                const int last_rel = ntok - 1 - first;
                // read through the constant address space: the table is never
                // written by the kernel, and scalar loads keep it out of the
                // in-order vector-load counter the K/V pipeline waits on
                const __attribute__((address_space(4))) int32_t *bt =
                    (const __attribute__((address_space(4))) int32_t *)a.block_table +
                    (size_t)b * a.max_pages;
#pragma unroll
                for (int uu = 0; uu < TU; ++uu) {
                    const int u = tile_of(uu);
                    const int rel = 16 * u < last_rel ? 16 * u : last_rel;
                    P.pg[uu] = bt[((int)t0 + first + rel) >> a.page_shift];  // clamped at use
                }
            }
        };
        // Addressing: a base per tile (sequence and step start, or the tile's
        // page) plus a 32-bit per-lane row offset.  Paged, the base is uniform
        // and the lane's column offset joins the 32-bit part, so the loads
        // take the scalar-base form (measured 5 % faster there; contiguous,
        // a per-lane 64-bit base measured slightly faster).  One token's row
        // over all heads is at most 16 MiB and a page at most 2 GiB (both
        // checked on the host), so the offsets fit in 32 bits.
        const uint32_t stride32 = (uint32_t)tok_stride;
        const uint32_t lane_off32 = PAGED ? (uint32_t)lane_off : 0u;
        const size_t lane_off64 = PAGED ? 0 : lane_off;
        auto load_step = [&](int st, const Pages &P, Stage &g) {
            const int sa = st < nsteps ? st : nsteps - 1;
            const int first = sa * kStepTok;
            const int last_rel = ntok - 1 - first;
#pragma unroll
            for (int uu = 0; uu < TU; ++uu) {
                const int u = tile_of(uu);
                // base of tile u: contiguous K/V, or the tile's page
                size_t base;
                uint32_t pmask = 0xffffffffu;
                if constexpr (!PAGED) {
                    const size_t seq = a.shared_kv ? 0 : (size_t)b * a.max_kv_len;
                    base = (seq + (size_t)t0 + first) * tok_stride;
                } else {
                    int pg = P.pg[uu];
                    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
                    base = ((size_t)pg << a.page_shift) * tok_stride;
                    pmask = (1u << a.page_shift) - 1u;
                }
                const char *kb = static_cast<const char *>(a.k) + base + lane_off64;
                const char *vb = static_cast<const char *>(a.v) + base + lane_off64;
#pragma unroll
                for (int jj = 0; jj < JW; ++jj) {
                    int rel = 16 * u + group_of(jj) * T::RPI + lrow;
                    rel = rel < last_rel ? rel : last_rel;
                    // row within the base: the step-relative token, or the
                    // token's row within its page
                    const uint32_t row =
                        PAGED ? ((uint32_t)((int)t0 + first + rel) & pmask) : (uint32_t)rel;
                    const uint32_t off = row * stride32 + lane_off32;
                    g.k[uu][jj] = ld128<NTLOAD>(kb + off);
                    g.v[uu][jj] = ld128<NTLOAD>(vb + off);
                }
            }
        };

        // Write a step's rows into LDS tiles at buf, chunks swizzled per row.
        auto stage = [&](const Stage &g, lds_char *buf) {
#pragma unroll
            for (int uu = 0; uu < TU; ++uu)
#pragma unroll
                for (int jj = 0; jj < JW; ++jj) {
                    const int u = tile_of(uu);
                    const int r = group_of(jj) * T::RPI + lrow;
                    *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(
                        buf + u * T::TILE + r * T::ROW + (lq ^ T::swz_k(r)) * 16) = g.k[uu][jj];
                    *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(
                        buf + (U + u) * T::TILE + r * T::ROW + (lq ^ T::swz_v(r)) * 16) =
                        g.v[uu][jj];
                }
        };
        // Several waves: even steps in buffer 0, odd steps in buffer 1.  A
        // wave stages step s + 1 only after the barrier that follows every
        // wave's staging of step s, which each wave reaches after computing
        // step s - 1: the buffer it overwrites has been read by all.
        lds_char *const b0 = tb;
        lds_char *const b1 = W > 1 ? tb + T::BUF : tb;
        auto wg_sync = [] {
            if constexpr (W > 1)
                __syncthreads();
        };

        // All LDS fragments of one step: K for the S product, V (read
        // transposed) for the PV product.
        struct Frags {
            u32x4 k[U][NC];
            s16x4_t v[U][NT];
        };
        const int vr = 4 * grp + (col >> 2);  // V row this lane addresses for the transpose read
        const int vq = (col & 3) >> 1;        // chunk within the 32-byte slice of a d tile
        const int vh = (col & 1) * 8;         // half of that chunk
        auto fetch = [&](const lds_char *buf, Frags &f) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const lds_char *krow = buf + u * T::TILE + col * T::ROW;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int p = (4 * c + grp) ^ T::swz_k(col);
                    f.k[u][c] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                        krow + p * 16);
                }
                const lds_char *vrow = buf + (U + u) * T::TILE + vr * T::ROW + vh;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int pc = (2 * t + vq) ^ T::swz_v(vr);
                    f.v[u][t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4_t *)(vrow + pc * 16));
                }
            }
        };

        // One step's arithmetic.  Every weight is p = 2^(x - m) with x the
        // score scaled into the log2 domain (one product, rounded), and the
        // lane's max is the max of the x, so both kinds of step give
        // bit-identical weights for the same tokens (and paged K/V, which
        // takes only the masked kind, bit-identical results).  FULL (every
        // token of the step lies before the piece's end, and the scale is
        // positive, as it is for 1/sqrt(d)): no per-score end mask, and the
        // max is taken over the unscaled scores and scaled once (a positive
        // scale keeps the order, and rounding keeps it too, so it is the
        // same float).  Otherwise (the last step of a piece, or a scale
        // <= 0) scores past the end are masked to -inf.
        auto compute_step_impl = [&](int st, const Frags &f, auto full_tag) {
            // each product and difference rounded on its own: on a full step
            // the compiler would otherwise fuse x = s * scale and x - m into
            // one operation, which the masked step cannot, and the two kinds
            // of step would round differently
#pragma clang fp contract(off)
            constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                // S^T tiles on the matrix cores, scaled into the log2 domain
                float x[U][4];
                float mx = -INFINITY;  // max of this lane's tokens
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        s = M::s_tile(f.k[u][c], qf[qt][c], s);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (FULL) {
                            x[u][r] = s[r] * a.scale_log2;
                            mx = fmaxf(mx, s[r]);
                        } else {
                            const int rel = st * kStepTok + 16 * u + 4 * grp + r;
                            x[u][r] = rel < ntok ? s[r] * a.scale_log2 : -INFINITY;
                            mx = fmaxf(mx, x[u][r]);
                        }
                    }
                }
                if constexpr (FULL)
                    mx *= a.scale_log2;
                mtrue[qt] = fmaxf(mtrue[qt], mx);
                // The reference max of a slot only has to bound its scores
                // within 2^kRescaleGap, so the four lanes of a slot synchronise
                // (and O, l are rescaled) only when some lane's tokens outgrow
                // it; in steady state this is a single ballot.
                float p[U][4];
                if constexpr (FD_SPEC_WEIGHTS) {
                    // the weights against the reference max as it stands,
                    // computed while the check below resolves; redone in the
                    // (rare) rescale branch
                    const float mref0 = m_used[qt] == -INFINITY ? 0.f : m_used[qt];
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            p[u][r] = fast_exp2(x[u][r] - mref0);
                }
                if (__ballot(mx > m_used[qt] + kRescaleGap)) {
                    float hm = fmaxf(mx, __shfl_xor(mx, 16, 64));
                    hm = fmaxf(hm, __shfl_xor(hm, 32, 64));
                    const float m_new = fmaxf(m_used[qt], hm);
                    const bool grow = m_new > m_used[qt] + kRescaleGap;  // same on a slot's 4 lanes
                    const float alpha = grow ? fast_exp2(m_used[qt] - m_new) : 1.f;
                    if (grow)
                        m_used[qt] = m_new;
                    lsum[qt] *= alpha;
                    lexact[qt] *= alpha;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float ar = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            oacc[qt][t][r] *= ar;
                    }
                    if constexpr (FD_SPEC_WEIGHTS) {
                        const float mref1 = m_used[qt] == -INFINITY ? 0.f : m_used[qt];
#pragma unroll
                        for (int u = 0; u < U; ++u)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                p[u][r] = fast_exp2(x[u][r] - mref1);
                    }
                }
                if constexpr (!FD_SPEC_WEIGHTS) {
                    const float mref = m_used[qt] == -INFINITY ? 0.f : m_used[qt];
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            p[u][r] = fast_exp2(x[u][r] - mref);
                }
                if constexpr (FD_PV32 && U % 2 == 0) {
                    // Two token tiles per product.  The contraction runs over
                    // 32 tokens in the order k = 8 * grp + 4 * j + r for token
                    // 16 * (u + j) + 4 * grp + r: the lane holding slot `col`
                    // in group grp has exactly those eight weights (S^T
                    // element r of tiles u and u + 1), and the transposed V
                    // reads of the two tiles give the same eight tokens of
                    // its d column.
#pragma unroll
                    for (int u = 0; u < U; u += 2) {
                        lexact[qt] += (p[u][0] + p[u][1]) + (p[u][2] + p[u][3]);
                        const u32x2 pa0 = M::pack(p[u], &lsum[qt]);
                        lexact[qt] += (p[u + 1][0] + p[u + 1][1]) + (p[u + 1][2] + p[u + 1][3]);
                        const u32x2 pa1 = M::pack(p[u + 1], &lsum[qt]);
                        const u32x4 pa = {pa0[0], pa0[1], pa1[0], pa1[1]};
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            oacc[qt][t] = M::pv_tile2(pa, f.v[u][t], f.v[u + 1][t], oacc[qt][t]);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        lexact[qt] += (p[u][0] + p[u][1]) + (p[u][2] + p[u][3]);
                        const u32x2 pa = M::pack(p[u], &lsum[qt]);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            oacc[qt][t] = M::pv_tile(pa, f.v[u][t], oacc[qt][t]);
                    }
                }
            }
        };
        // The full-step body pays where the arithmetic bounds the step:
        // work-groups of several waves or several query tiles per wave
        // (cascade -1.5 us, large groups 2-10 %).  One-wave one-tile kernels
        // are bound by their load stream, and a branch between two step
        // bodies slowed them (ragged grouped-query workload 162.3 -> 164.2
        // us per split stage; through 16-token pages 175 -> 181 us per step:
        // the block-table reads are scalar loads waited on with the LDS
        // counter, and the compiler then waited for them too early), so they,
        // and every paged kernel, keep the one masked body.
        auto compute_step = [&](int st, const Frags &f) {
            if constexpr (PAGED || (W == 1 && QT == 1)) {
                compute_step_impl(st, f, StepKind<false>{});
            } else {
                if ((st + 1) * kStepTok <= ntok && a.scale_log2 > 0.f)
                    compute_step_impl(st, f, StepKind<true>{});
                else
                    compute_step_impl(st, f, StepKind<false>{});
            }
        };

        // Pipeline over two register sets.  A step's rows leave their
        // registers as soon as they are staged in LDS, so the loads two steps
        // ahead go into those registers right then, before the step's
        // fragments are read back and computed: two steps of loads stay in
        // flight throughout.  (Issuing them after the arithmetic instead
        // measured 1-3 % slower at d = 128.)  At d = 256 that keeps 128 more
        // registers live across the arithmetic than the register file holds
        // without spilling, so there the next step's loads are issued when
        // the current step starts (one to two steps in flight).  Paged K/V:
        // a step's table entries are scalar loads, and a wave's LDS reads are
        // waited on with the same counter (which then cannot tell them apart),
        // so each lookup is issued after a step's arithmetic, once that
        // step's fragment reads have been waited on: it has the next staging
        // (which waits for that step's rows) to arrive.  The LDS tile is
        // rewritten each step;
        // one wave's LDS operations execute in order, so a step's writes
        // follow the previous step's reads.
        Frags f;
        if constexpr (NS > 2) {
            // NS register sets (contiguous K/V, d <= 128): steps 0 .. NS - 1
            // go out first; step st is staged from set st % NS, which is then
            // refilled with step st + NS, so NS - 1 to NS steps of loads stay
            // in flight while a step is computed.  Every refill is issued,
            // past the last step too (load_step re-reads the last step then):
            // with no conditional loads the compiler's wait for a set counts
            // exactly the 2 (NS - 1) younger loads.  LDS still alternates
            // two buffers by step parity, with the same barrier rule as below.
            static_assert(!PAGED && D <= 128, "deeper load pipelines: contiguous K/V, d <= 128");
            Stage g[NS];
            Pages none;
#pragma unroll
            for (int i = 0; i < NS; ++i)
                load_step(i, none, g[i]);
            const int ngroups = nsteps / NS;
            for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int st = gi * NS + j;
                    lds_char *const buf = (st & 1) ? b1 : b0;
                    stage(g[j], buf);
                    __builtin_amdgcn_sched_barrier(0);
                    load_step(st + NS, none, g[j]);
                    __builtin_amdgcn_sched_barrier(0);
                    wg_sync();
                    fetch(buf, f);
                    compute_step(st, f);
                }
            }
            // the last nsteps % NS steps: already in flight, no more loads
            const int rem = nsteps - ngroups * NS;
#pragma unroll
            for (int j = 0; j < NS - 1; ++j) {
                if (j < rem) {
                    const int st = ngroups * NS + j;
                    lds_char *const buf = (st & 1) ? b1 : b0;
                    stage(g[j], buf);
                    wg_sync();
                    fetch(buf, f);
                    compute_step(st, f);
                }
            }
        } else {
        Stage ga, gb;
        Pages pa, pb;
        const int npairs = nsteps >> 1;
        lookup(0, pa);
        lookup(1, pb);
        load_step(0, pa, ga);
        if constexpr (D <= 128) {
            load_step(1, pb, gb);
            lookup(2, pa);
            for (int pr = 0; pr < npairs; ++pr) {
                const int st = 2 * pr;
                stage(ga, b0);
                __builtin_amdgcn_sched_barrier(0);
                load_step(st + 2, pa, ga);
                __builtin_amdgcn_sched_barrier(0);
                wg_sync();
                fetch(b0, f);
                compute_step(st, f);
                if constexpr (PAGED)
                    __builtin_amdgcn_sched_barrier(0);
                lookup(st + 3, pb);
                stage(gb, b1);
                __builtin_amdgcn_sched_barrier(0);
                load_step(st + 3, pb, gb);
                __builtin_amdgcn_sched_barrier(0);
                wg_sync();
                fetch(b1, f);
                compute_step(st + 1, f);
                if constexpr (PAGED)
                    __builtin_amdgcn_sched_barrier(0);
                lookup(st + 4, pa);
            }
        } else {
            for (int pr = 0; pr < npairs; ++pr) {
                const int st = 2 * pr;
                load_step(st + 1, pb, gb);
                lookup(st + 2, pa);
                __builtin_amdgcn_sched_barrier(0);
                stage(ga, b0);
                wg_sync();
                fetch(b0, f);
                compute_step(st, f);
                load_step(st + 2, pa, ga);
                lookup(st + 3, pb);
                __builtin_amdgcn_sched_barrier(0);
                stage(gb, b1);
                wg_sync();
                fetch(b1, f);
                compute_step(st + 1, f);
            }
        }
        if (nsteps & 1) {
            stage(ga, b0);
            wg_sync();
            fetch(b0, f);
            compute_step(nsteps - 1, f);
        }
        }  // NS == 2
    }

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        // l of slot `col`: the four lanes holding it each summed their tokens.
        float ltot = lsum[qt] + __shfl_xor(lsum[qt], 16, 64);
        ltot += __shfl_xor(ltot, 32, 64);
        float lex = lexact[qt] + __shfl_xor(lexact[qt], 16, 64);
        lex += __shfl_xor(lex, 32, 64);
        float mtop = fmaxf(mtrue[qt], __shfl_xor(mtrue[qt], 16, 64));
        mtop = fmaxf(mtop, __shfl_xor(mtop, 32, 64));
        // Output rows: this lane holds slots 4*grp + r of O.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * grp + r;
            const float lr = __shfl(ltot, h, 64);
            const float le = __shfl(lex, h, 64);
            const float mr = __shfl(m_used[qt], h, 64);
            const float mt = __shfl(mtop, h, 64);
            const int row = qm.row(qt, h);
            if (row < 0)
                continue;
            // a non-empty piece has a weight >= 1 (its max score is at or
            // above the reference), which rounds to >= 1: lr > 0 exactly when
            // le > 0
            const bool any = lr > 0.f;
            const float inv = any ? 1.f / lr : 0.f;
            const float lse = any ? (mr + fast_log2(le)) * kLn2 : -INFINITY;
            if (out.o) {
                const size_t idx =
                    (size_t)(out.local ? (qm.tile0 + qt) * 16 + h : row) * out.stride + out.off;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    out.o[idx * D + 16 * t + col] = oacc[qt][t][r] * inv;
                if (col == 0) {
                    if (out.l) {  // m/l/o triple: the piece's max score and l relative to it
                        // (the reference max trails the max by at most 2^8: no overflow)
                        out.lse[idx] = any ? mt * kLn2 : -INFINITY;
                        out.l[idx] = any ? le * fast_exp2(mr - mt) : 0.f;
                    } else {
                        out.lse[idx] = lse;
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    store_out(a.o, (size_t)row * D + 16 * t + col, oacc[qt][t][r] * inv,
                              a.out_dtype);
                if (col == 0 && a.lse)
                    a.lse[row] = lse;
            }
        }
    }
}

#endif  // __HIP_DEVICE_COMPILE__

// Fixed splits: work-group -> (b, KV head, split), KV head fastest; split i
// covers [i*L, min((i+1)*L, N_b)).
template <int DT, int D, bool PAGED>
__global__ __launch_bounds__(64) void split_mfma_kernel(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ __attribute__((aligned(1024))) char tile_buf[Tiles<D>::BUF];
    const int kvh = blockIdx.x % a.heads_kv;
    const int rest = blockIdx.x / a.heads_kv;
    const int split = rest % a.num_splits;
    const int b = rest / a.num_splits;
    const int n = clamp_len(a.kv_lens, b, a.max_kv_len);
    const long t0 = (long)split * a.split_len;
    const long t1 = t0 + a.split_len < n ? t0 + a.split_len : n;
    const int G = a.heads_q / a.heads_kv;
    const QMap qm{b * a.heads_q + kvh * G, G, 0, 0, a.heads_q, kvh};
    PieceOut out{nullptr, nullptr, nullptr, 0, 0, false};
    if (a.o_part) {
        out.o = a.o_part;
        out.stride = a.part_stride ? a.part_stride : a.num_splits;
        out.off = a.part_offset + split;
        out.lse = a.m_part ? a.m_part : a.lse_part;
        out.l = a.m_part ? a.l_part : nullptr;
    }
    mfma_piece<DT, D, PAGED, 1, FD_MFMA_NT>(a, (lds_char *)tile_buf, b, kvh, t0, t1, qm, out);
#endif  // __HIP_DEVICE_COMPILE__
}

// Query tiles: all queries of a KV head that read the same K/V, in tiles of
// 16, QT tiles per wave and W waves per work-group (the waves share every K/V
// step staged in LDS, each loading a 1/W share of its rows); a (KV head,
// split) unit with more tiles gets several work-groups.  Two uses: a shared prefix (cascade), whose batch * G
// queries all read the prefix, and groups of more than 16 query heads per KV
// head (up to multi-query attention), whose G queries read their sequence's
// K/V.  Each work-group serves its QT tiles from every K/V tile it stages,
// and the work-groups sharing one unit are given block indices congruent mod
// 8: blocks are dispatched round-robin over the eight XCDs, so they run on
// one XCD and meet the unit's K/V in its L2.  blockIdx -> (xcd = idx % 8,
// slot = idx / 8); slot -> (unit / 8 within the XCD, tile group j fastest);
// unit = (sequence, split, KV head), KV head fastest (one sequence for a
// shared prefix).  The K/V loads are ordinary (temporal) loads, as other
// work-groups may read the same rows.
template <int DT, int D, int QT, bool PAGED, int W, bool PAIR = false>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W > 4 || PAIR ? 2 : 1)))
void split_mfma_tiled_kernel(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int SKB = PAIR ? 16 : W > 1 ? wide_step_kb<W>() : kPrefixStepKB;
    __shared__ __attribute__((aligned(1024))) char tile_buf[(W > 1 ? 2 : 1) * Tiles<D, SKB>::BUF];
    const int G = a.heads_q / a.heads_kv;
    const int nq = a.shared_kv ? a.batch * G : G;
    const int groups = ((nq + 15) / 16 + QT * W - 1) / (QT * W);  // tile groups per unit
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    const int unit = (slot / groups) * 8 + xcd;
    const int j = slot % groups;
    const int seqs = a.shared_kv ? 1 : a.batch;
    if (unit >= seqs * a.heads_kv * a.num_splits)
        return;
    const int kvh = unit % a.heads_kv;
    const int rest = unit / a.heads_kv;
    const int split = rest % a.num_splits;
    const int b = rest / a.num_splits;
    const int n = a.shared_kv ? a.max_kv_len : clamp_len(a.kv_lens, b, a.max_kv_len);
    const long t0 = (long)split * a.split_len;
    const long t1 = t0 + a.split_len < n ? t0 + a.split_len : n;
    // wave wv of the work-group takes tiles (j * W + wv) * QT ...
    const int wv = W > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    const QMap qm{a.shared_kv ? 0 : b * a.heads_q, G, nq, (j * W + wv) * QT, a.heads_q, kvh};
    PieceOut out{nullptr, nullptr, nullptr, 0, 0, false};
    if (a.o_part) {
        out.o = a.o_part;
        out.stride = a.part_stride ? a.part_stride : a.num_splits;
        out.off = a.part_offset + split;
        out.lse = a.m_part ? a.m_part : a.lse_part;
        out.l = a.m_part ? a.l_part : nullptr;
    }
    // (paired work-groups read the unit's rows through L2: ordinary loads)
    constexpr int NTL = PAIR ? 0 : W > 1 ? wide_nt<QT>() : 0;
    mfma_piece<DT, D, PAGED, QT, NTL, SKB, W, wide_sets<D, PAGED, W>()>(
        a, (lds_char *)tile_buf, b, kvh, t0, t1, qm, out);
#endif  // __HIP_DEVICE_COMPILE__
}

// Token-balanced partition (partition.h): work-group w walks its share of the
// flattened (KV head, sequence, token) space piece by piece; the piece of unit
// u goes to slot w + rank(u) of the slot arrays (o [slot][G][d], LSE [slot][G]).
// The G query heads of a unit take ceil(G / 16) tiles: QT per wave, W waves
// per work-group (W > 1: the waves share each K/V step staged in LDS, as in
// the tiled kernel).
template <int DT, int D, bool PAGED, int QT, int W = 1>
__global__ __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(W > 4 || bal_two_per_simd<D, QT, W>() ? 2 : 1)))
void split_mfma_balanced_kernel(SplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
#if FD_WG_CLOCKS
    const unsigned long long clk0 = (unsigned long long)wall_clock64();
    unsigned long long clk_work = 0;  // (pieces << 32) | tokens
#endif
    constexpr int SKB = bal_two_per_simd<D, QT, W>() ? 16
                        : W > 1                     ? wide_step_kb<W>()
                                                    : FD_MFMA_STEP_KB;
    __shared__ __attribute__((aligned(1024))) char tile_buf[(W > 1 ? 2 : 1) * Tiles<D, SKB>::BUF];
    const int wv = W > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    // share index (partition_plan.h: neighbouring work-groups take consecutive
    // heads of one token range when the KV heads come in multiples of 8)
    const int w = share_index((int)blockIdx.x, a.heads_kv, a.num_wgs);
    const int G = a.heads_q / a.heads_kv;
    PieceCursor c;
#if FD_WG_CLOCKS
    // stamps of share w: start and end clocks, work, block index (thread 0,
    // ordinary vector stores; w < num_wgs and the host sized the buffer)
    auto stamp = [&] {
        if (a.wg_clock && threadIdx.x == 0) {
            const unsigned long long clk1 = (unsigned long long)wall_clock64();
            a.wg_clock[4 * (size_t)w + 0] = clk0;
            a.wg_clock[4 * (size_t)w + 1] = clk1;
            a.wg_clock[4 * (size_t)w + 2] = clk_work;
            // where it ran: the HW_ID register (CU, SIMD, shader engine) in the
            // high word, the XCD (XCC_ID register) above the block index
            const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
            const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 0xff;
            a.wg_clock[4 * (size_t)w + 3] =
                ((unsigned long long)hw << 32) | ((unsigned long long)xcc << 24) | blockIdx.x;
        }
    };
    if (!balanced_start(a.kv_lens, a.batch, a.max_kv_len, a.heads_kv, w, a.num_wgs, c)) {
        stamp();
        return;
    }
#else
    if (!balanced_start(a.kv_lens, a.batch, a.max_kv_len, a.heads_kv, w, a.num_wgs, c))
        return;
#endif
    walk_share(a.kv_lens, a.batch, a.max_kv_len, a.heads_kv, w, c, [&](const Piece &p) {
        const QMap qm{p.b * a.heads_q + p.x * G, G, 0, wv * QT, a.heads_q, p.x};
        const PieceOut out{a.o_part + (size_t)p.slot * G * D, a.lse_part + (size_t)p.slot * G,
                           nullptr, 1, 0, true};
        mfma_piece<DT, D, PAGED, QT, (W > 1 ? wide_nt<QT>() : FD_MFMA_NT), SKB, W,
                   wide_sets<D, PAGED, W>()>(a, (lds_char *)tile_buf, p.b, p.x, p.t0, p.t1, qm,
                                             out);
        if (p.first && threadIdx.x == 0) {  // the unit's descriptor {first slot, count}
            const size_t u = (size_t)p.b * a.heads_kv + p.x;
            a.unit_desc[2 * u] = p.slot;
            a.unit_desc[2 * u + 1] = p.desc_count;
        }
#if FD_WG_CLOCKS
        clk_work += (1ull << 32) + (unsigned long long)(p.t1 - p.t0);
#endif
    });
#if FD_WG_CLOCKS
    stamp();
#endif
#endif  // __HIP_DEVICE_COMPILE__
}

int lds_per_cu_mfma() {
    // per device; several host threads may fill an entry at once (same value)
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess || v <= 0)
            v = -1;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

// The tiled kernel for QT query tiles per wave and W waves, paged or
// contiguous.
template <int DT, int D, int QT, int W = 1, bool PAIR = false>
void launch_tiled(const SplitArgs &a, dim3 g, size_t pad, hipStream_t stream) {
    const dim3 blk(64 * W);
    if (a.block_table)
        hipLaunchKernelGGL((split_mfma_tiled_kernel<DT, D, QT, true, W, PAIR>), g, blk, pad,
                           stream, a);
    else
        hipLaunchKernelGGL((split_mfma_tiled_kernel<DT, D, QT, false, W, PAIR>), g, blk, pad,
                           stream, a);
}

// The token-balanced kernel for QT query tiles per wave and W waves, paged or
// contiguous.
template <int DT, int D, int QT, int W = 1>
void launch_balanced(const SplitArgs &a, dim3 g, size_t pad, hipStream_t stream) {
    const dim3 blk(64 * W);
    if (a.block_table)
        hipLaunchKernelGGL((split_mfma_balanced_kernel<DT, D, true, QT, W>), g, blk, pad, stream,
                           a);
    else
        hipLaunchKernelGGL((split_mfma_balanced_kernel<DT, D, false, QT, W>), g, blk, pad, stream,
                           a);
}

template <int DT, int D>
hipError_t launch(const SplitArgs &a, hipStream_t stream) {
    using T = Tiles<D>;
    const int tw = a.tile_waves > 1 ? a.tile_waves : 1;
    // several smaller tiled work-groups per unit (mfma_policy.h tiled_pair)
    long tile_groups = 1;
    if (a.tile_qt > 0) {
        const long nq = (long)(a.shared_kv ? a.batch : 1) * (a.heads_q / a.heads_kv);
        const long tiles = (nq + 15) / 16;
        tile_groups = (tiles + (long)a.tile_qt * tw - 1) / ((long)a.tile_qt * tw);
    }
    const bool pair = a.tile_qt > 0 && !a.balanced && tiled_pair(D, a.tile_qt, tw, tile_groups);
    // balanced four-wave work-groups with one tile per wave (bal_two_per_simd)
    const bool bal_two = a.balanced && tw == 4 && D <= 128 &&
                         (a.heads_q / a.heads_kv + 15) / 16 <= tw;
    const size_t kStatic =
        bal_two                        ? (size_t)2 * Tiles<D, 16>::BUF
        : pair                         ? (size_t)2 * Tiles<D, 16>::BUF
        : tw == 8                      ? (size_t)2 * Tiles<D, wide_step_kb<8>()>::BUF
        : tw == 4                      ? (size_t)2 * Tiles<D, wide_step_kb<4>()>::BUF
        : tw == 2                      ? (size_t)2 * Tiles<D, wide_step_kb<2>()>::BUF
        : a.tile_qt > 0 && !a.balanced ? (size_t)Tiles<D, kPrefixStepKB>::BUF
                                       : (size_t)T::BUF;
    long grid = a.balanced ? (long)a.num_wgs : (long)a.batch * a.heads_kv * a.num_splits;
    if (a.tile_qt > 0) {  // query tiles: (8-aligned units) x tile groups
        const long nq = (long)(a.shared_kv ? a.batch : 1) * (a.heads_q / a.heads_kv);
        const long tiles = (nq + 15) / 16;
        const long groups = (tiles + (long)a.tile_qt * tw - 1) / ((long)a.tile_qt * tw);
        const long units = (long)(a.shared_kv ? 1 : a.batch) * a.heads_kv * a.num_splits;
        grid = (units + 7) / 8 * 8 * groups;
        if (grid > 0x7fffffffL)
            return hipErrorInvalidValue;
    }
    size_t pad = 0;
    const int lds = lds_per_cu_mfma();
    const int per_cu = a.balanced ? split_mfma_balanced_wg_per_cu(D, a.heads_q / a.heads_kv)
                       : a.tile_qt == 0 ? kMfmaWgPerCU
                                        : split_mfma_tiled_wg_per_cu(tw, pair);
    if (per_cu > 0 && lds > 0) {
        const size_t want = (size_t)lds / (per_cu + 1) + 256;
        pad = want > kStatic ? want - kStatic : 0;
    }
    const dim3 g((unsigned)grid), blk(64);
    if (a.tile_qt > 0 && tw > 1) {
        // several waves per work-group, each with one tile or wide_qt
        constexpr int Q = wide_qt<D>();
        if ((a.tile_qt != Q && a.tile_qt != 1) || tw > tile_max_waves<D>())
            return hipErrorInvalidValue;
        const bool one = a.tile_qt == 1;
        if (tw == 2) {
            if (pair) {
                if constexpr (D <= 128)
                    launch_tiled<DT, D, 1, 2, true>(a, g, pad, stream);
            } else if (one) {
                launch_tiled<DT, D, 1, 2>(a, g, pad, stream);
            } else {
                launch_tiled<DT, D, Q, 2>(a, g, pad, stream);
            }
        } else if (tw == 4) {
            if constexpr (tile_max_waves<D>() >= 4) {
                if (pair) {
                    if constexpr (D <= 128)
                        launch_tiled<DT, D, 1, 4, true>(a, g, pad, stream);
                } else if (one) {
                    launch_tiled<DT, D, 1, 4>(a, g, pad, stream);
                } else {
                    launch_tiled<DT, D, Q, 4>(a, g, pad, stream);
                }
            }
        } else if (tw == 8) {
            if constexpr (tile_max_waves<D>() >= 8) {
                if (!one)
                    return hipErrorInvalidValue;
                launch_tiled<DT, D, 1, 8>(a, g, pad, stream);
            }
        } else
            return hipErrorInvalidValue;
    } else if (a.tile_qt > 0) {
        if (a.tile_qt == 1) {
            launch_tiled<DT, D, 1>(a, g, pad, stream);
        } else if (a.tile_qt == 2 && tile_max_qt<D>() >= 2) {
            if constexpr (tile_max_qt<D>() >= 2)
                launch_tiled<DT, D, 2>(a, g, pad, stream);
        } else if (a.tile_qt == 4 && tile_max_qt<D>() >= 4) {
            if constexpr (tile_max_qt<D>() >= 4)
                launch_tiled<DT, D, 4>(a, g, pad, stream);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (a.balanced) {
        // QT = ceil(G / 16) tiles on one wave (up to two), or two (one at
        // d = 256) per wave on tw waves
        const int tiles = (a.heads_q / a.heads_kv + 15) / 16;
        constexpr int QB = wide_qt<D>();
        if (tw > 1) {
            // one tile per wave when the waves cover the group, else QB
            if (tiles > QB * tw || tw > tile_max_waves<D>())
                return hipErrorInvalidValue;
            const bool one = tiles <= tw;
            if (tw == 2) {
                if (one)
                    launch_balanced<DT, D, 1, 2>(a, g, pad, stream);
                else
                    launch_balanced<DT, D, QB, 2>(a, g, pad, stream);
            } else if (tw == 4) {
                if constexpr (tile_max_waves<D>() >= 4) {
                    if (one)
                        launch_balanced<DT, D, 1, 4>(a, g, pad, stream);
                    else
                        launch_balanced<DT, D, QB, 4>(a, g, pad, stream);
                }
            } else if (tw == 8) {
                if constexpr (tile_max_waves<D>() >= 8) {
                    if (!one)
                        return hipErrorInvalidValue;
                    launch_balanced<DT, D, 1, 8>(a, g, pad, stream);
                }
            } else
                return hipErrorInvalidValue;
        } else if (tiles == 1) {
            launch_balanced<DT, D, 1>(a, g, pad, stream);
        } else if (tiles == 2 && QB >= 2) {
            if constexpr (QB >= 2)
                launch_balanced<DT, D, 2>(a, g, pad, stream);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        if (a.block_table)
            hipLaunchKernelGGL((split_mfma_kernel<DT, D, true>), g, blk, pad, stream, a);
        else
            hipLaunchKernelGGL((split_mfma_kernel<DT, D, false>), g, blk, pad, stream, a);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const SplitArgs &a, hipStream_t stream) {
    switch (a.head_dim) {
    case 64: return launch<DT, 64>(a, stream);
    case 128: return launch<DT, 128>(a, stream);
    case 256: return launch<DT, 256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_mfma(const SplitArgs &a, int in_dtype, hipStream_t stream) {
    switch (in_dtype) {
    case kBF16: return launch_dt<kBF16>(a, stream);
    case kF16: return launch_dt<kF16>(a, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace fd
