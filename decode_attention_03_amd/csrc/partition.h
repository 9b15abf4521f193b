// partition.h -- the token-balanced partition of a ragged batch, shared by
// the split kernels (which walk it) and the combine kernel (which reads the
// per-unit descriptors it leaves behind).
//
// The pages cut each sequence's KV range into splits of one fixed length
// ("FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15), §2.5
// stage 1; "adv04: Flash-Decoding" (mini-vllm-tutorial), §4).  With ragged
// lengths, fixed splits leave the GPU's work-groups unevenly loaded, so for
// ragged batches the library also offers a partition that gives every
// work-group the same cost: its 16-token granules of K/V rows plus a fixed
// charge for every piece it starts.  It is still a split-K partition
// in the pages' sense: every (sequence, head) row's tokens are cut into
// contiguous pieces, each piece yields an (o, LSE) pair, and the combine merges
// a row's pieces ("FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法", §2.3.4;
// the merge does not depend on where the cuts fall, §2.3.5).
//
// Definitions (all positions 64-bit; a position is one granule of
// kGranule = 16 tokens, so every piece starts on a 16-token tile boundary):
//   unit (b, x): one (sequence b, KV head x) pair; hx = heads_kv;
//   N_b    = kv_lens[b] clamped to [0, max_kv_len], g_b = ceil(N_b / 16);
//   a unit of a non-empty sequence costs g_b + kPieceCost positions: the
//            first kPieceCost stand for the fixed cost of starting a piece
//            (loading q, filling the load pipeline, writing the partial),
//            so that shares balance time rather than bytes; its granule j
//            (tokens [16 j, min(16 j + 16, N_b))) is position kPieceCost + j
//            of the unit; empty sequences cost nothing;
//   the flattened space lists units head-major, (0, 0), (1, 0), ...,
//            (batch - 1, 0), (0, 1), ..., each unit covering its cost in
//            positions; head x therefore holds [x P, (x + 1) P), P being the
//            summed cost of the sequences, and when hx divides num_wgs the
//            work-groups of different heads get the same token ranges and
//            stream the same K/V rows (one row of every head) side by side,
//            as fixed splits do;
//   T      = hx P, W_eff = min(num_wgs, T);
//   work-group w < W_eff covers [floor(w T / W_eff), floor((w+1) T / W_eff)),
//            never empty; work-groups w >= W_eff do nothing; a work-group's
//            piece of unit u is the unit's granules inside its range (none
//            when the range only touches the unit's leading cost positions);
//   the piece of unit u handled by work-group w writes slot w + rank(u),
//            rank(u) = number of non-empty units before u in that order; a unit's pieces
//            therefore fill consecutive slots, and slots < num_wgs + units;
//   the work-group that handles a unit's granule 0 writes the unit's
//            descriptor {first slot, slot count}; units of empty sequences
//            get none (the combine checks N_b itself).
#pragma once

#include "dev_common.h"

namespace fd {

constexpr int kGranule = 16;   // tokens per position of the balanced partition
#ifndef FD_PIECE_COST
#define FD_PIECE_COST 5
#endif
constexpr int kPieceCost = FD_PIECE_COST;  // positions charged per unit for starting a piece

__device__ __forceinline__ int clamp_len(const int32_t *kv_lens, int b, int max_kv_len) {
    int n = kv_lens ? kv_lens[b] : max_kv_len;
    return n < 0 ? 0 : (n > max_kv_len ? max_kv_len : n);
}

// Granules of sequence b.
__device__ __forceinline__ int granules(const int32_t *kv_lens, int b, int max_kv_len) {
    return (clamp_len(kv_lens, b, max_kv_len) + kGranule - 1) / kGranule;
}

// Positions one unit of sequence b costs (0 for an empty sequence).
__device__ __forceinline__ int unit_cost(const int32_t *kv_lens, int b, int max_kv_len) {
    const int g = granules(kv_lens, b, max_kv_len);
    return g > 0 ? g + kPieceCost : 0;
}

__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ long long wave_scan_ll(long long v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const long long y = __shfl_up(v, d, 64);
        if (lane >= d)
            v += y;
    }
    return v;
}

// A wave-uniform value the compiler cannot prove uniform (it came through a
// shuffle), moved to a scalar register so that addresses built from it stay
// scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform(long long v) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// Where one work-group's share of the flattened space starts.  Called by all
// 64 lanes of the wave together; every result is the same on every lane.
struct PieceCursor {
    long long pos, end;  // [pos, end): this work-group's positions
    long long total;     // T
    int w_eff;           // W_eff
    int b, x, t;         // unit (b, x) and position t within it (0 .. cost - 1) at `pos`
    int rank;            // rank of unit (b, x) among non-empty units
};

__device__ __forceinline__ bool balanced_start(const int32_t *kv_lens, int batch, int max_kv_len,
                                               int hx, int w, int num_wgs, PieceCursor &c) {
    const int lane = threadIdx.x & 63;
    long long gsum = 0;  // positions of one head: the sum of the unit costs
    int ne_all = 0;      // non-empty sequences
    for (int base = 0; base < batch; base += 64) {
        const int i = base + lane;
        const int n = i < batch ? unit_cost(kv_lens, i, max_kv_len) : 0;
        gsum += n;
        ne_all += __popcll(__ballot(n > 0));
    }
    const long long per_head = uniform(wave_sum_ll(gsum));
    c.total = per_head * hx;
    c.w_eff = c.total < num_wgs ? (int)c.total : num_wgs;
    if (w >= c.w_eff)
        return false;
    c.pos = c.total * w / c.w_eff;
    c.end = c.total * (w + 1) / c.w_eff;
    // head-major order: head x holds positions [x * per_head, (x + 1) * per_head)
    c.x = uniform((int)(c.pos / per_head));
    const long long off = c.pos - (long long)c.x * per_head;
    // the sequence whose unit of head x contains `pos`
    long long before = 0;  // positions of the sequences before this chunk
    int nonempty = 0;      // non-empty sequences before this chunk
    for (int base = 0; base < batch; base += 64) {
        const int i = base + lane;
        const long long n = i < batch ? unit_cost(kv_lens, i, max_kv_len) : 0;
        const long long incl = wave_scan_ll(n, lane);
        const unsigned long long hit = __ballot(i < batch && before + incl > off);
        const unsigned long long ne = __ballot(n > 0);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            const long long nb = __shfl(n, l, 64);
            c.b = uniform(base + l);
            c.t = uniform((int)(off - (before + __shfl(incl, l, 64) - nb)));
            const int ne_before = nonempty + __popcll(ne & ((1ull << l) - 1ull));
            c.rank = uniform(c.x * ne_all + ne_before);
            return true;
        }
        before += __shfl(incl, 63, 64);
        nonempty += __popcll(ne);
    }
    return false;  // not reached: pos < T lies in some non-empty sequence
}

// The work-group whose range holds position p.
__device__ __forceinline__ int balanced_owner(long long p, long long total, int w_eff) {
    return (int)(((p + 1) * w_eff - 1) / total);
}

}  // namespace fd
