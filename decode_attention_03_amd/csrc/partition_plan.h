// partition_plan.h -- the token-balanced partition of a ragged batch: its
// definitions and the walk of one work-group's share, shared by the split
// kernel (which walks it), the combine kernel (which reads the per-unit
// descriptors it leaves behind) and host checks (plain C++, no device code).
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

#include <cstdint>

#if defined(__HIPCC__)
#define FD_HD __host__ __device__ __forceinline__
#else
#define FD_HD inline
#endif

namespace fd {

constexpr int kGranule = 16;   // tokens per position of the balanced partition
#ifndef FD_PIECE_COST
#define FD_PIECE_COST 5
#endif
constexpr int kPieceCost = FD_PIECE_COST;  // positions charged per unit for starting a piece

FD_HD int clamp_len(const int32_t *kv_lens, int b, int max_kv_len) {
    int n = kv_lens ? kv_lens[b] : max_kv_len;
    return n < 0 ? 0 : (n > max_kv_len ? max_kv_len : n);
}

// Granules of sequence b.
FD_HD int granules(const int32_t *kv_lens, int b, int max_kv_len) {
    return (clamp_len(kv_lens, b, max_kv_len) + kGranule - 1) / kGranule;
}

// Positions one unit of sequence b costs (0 for an empty sequence).
FD_HD int unit_cost(const int32_t *kv_lens, int b, int max_kv_len) {
    const int g = granules(kv_lens, b, max_kv_len);
    return g > 0 ? g + kPieceCost : 0;
}

// The work-group whose range holds position p.
FD_HD int balanced_owner(long long p, long long total, int w_eff) {
    return (int)(((p + 1) * w_eff - 1) / total);
}

// The share a work-group takes, by block index.  When the KV heads come in
// multiples of the 8 XCDs (which take work-groups round-robin) and divide
// the work-group count, neighbouring work-groups take the same token range of
// consecutive heads, so each XCD streams whole heads, as it does under fixed
// splits (measured 1.2 us faster per step on 8 KV heads and 0.7 us slower on
// 2, where the plain order stays).  A bijection of [0, num_wgs) either way.
#ifndef FD_SHARE_ROTATE
#define FD_SHARE_ROTATE 0
#endif
FD_HD int share_index(int block, int hx, int num_wgs) {
    if (hx % 8 != 0 || num_wgs % hx != 0)
        return block;
    const int s = block / hx;  // token range (share within a head)
    // FD_SHARE_ROTATE: head of position j within range s rotated by s, so that
    // each XCD streams every head in turn rather than the same ones throughout
    const int x = FD_SHARE_ROTATE ? (block % hx + s) % hx : block % hx;
    return x * (num_wgs / hx) + s;
}

// Where one work-group's share of the flattened space starts.
struct PieceCursor {
    long long pos, end;  // [pos, end): this work-group's positions
    long long total;     // T
    int w_eff;           // W_eff
    int b, x, t;         // unit (b, x) and position t within it (0 .. cost - 1) at `pos`
    int rank;            // rank of unit (b, x) among non-empty units
};

// The definition of a share's start, in plain loops (the kernel finds the
// same cursor with a wave-wide scan, partition.h).  Returns false when work
// group w has no positions (w >= W_eff).
inline bool balanced_start_ref(const int32_t *kv_lens, int batch, int max_kv_len, int hx, int w,
                               int num_wgs, PieceCursor &c) {
    long long per_head = 0;
    int ne_all = 0;
    for (int i = 0; i < batch; ++i) {
        const int n = unit_cost(kv_lens, i, max_kv_len);
        per_head += n;
        ne_all += n > 0;
    }
    c.total = per_head * hx;
    c.w_eff = c.total < num_wgs ? (int)c.total : num_wgs;
    if (w >= c.w_eff)
        return false;
    c.pos = c.total * w / c.w_eff;
    c.end = c.total * (w + 1) / c.w_eff;
    c.x = (int)(c.pos / per_head);
    long long off = c.pos - (long long)c.x * per_head;
    int nonempty = 0;
    for (int i = 0; i < batch; ++i) {
        const int n = unit_cost(kv_lens, i, max_kv_len);
        if (off < n) {
            c.b = i;
            c.t = (int)off;
            c.rank = c.x * ne_all + nonempty;
            return true;
        }
        off -= n;
        nonempty += n > 0;
    }
    return false;  // not reached: pos < T lies in some non-empty sequence
}

// One piece of a share: the granules [lo, hi) of unit (b, x) inside it, that
// is tokens [t0, t1) of the unit's n tokens, written to slot w + rank(unit).
// The piece that holds the unit's granule 0 also carries the unit's
// descriptor count: the work-groups between the owners of its first and last
// granule.
struct Piece {
    int b, x;
    int lo, hi;     // granules, hi > lo
    long t0, t1;    // tokens
    int n;          // tokens of the sequence
    int slot;
    bool first;     // lo == 0: this piece writes the unit's descriptor
    int desc_count; // when first: the unit's slot count
};

// Walk work-group w's share from the cursor of balanced_start (the kernel's
// or balanced_start_ref), calling visit(piece) for each piece in order; the
// flattened space lists units head-major, and a unit of an empty sequence is
// skipped (it costs nothing).
template <class Visit>
FD_HD void walk_share(const int32_t *kv_lens, int batch, int max_kv_len, int hx, int w,
                      PieceCursor c, Visit &&visit) {
    int n = clamp_len(kv_lens, c.b, max_kv_len);  // tokens of the current sequence
    int ng = (n + kGranule - 1) / kGranule;        // and its granules
    while (true) {
        // this work-group covers positions [c.t, c.t + avail) of unit (c.b, c.x),
        // whose granule j is position kPieceCost + j
        const long long left = c.end - c.pos;
        const int ucost = ng + kPieceCost;
        const int avail = left < (long long)(ucost - c.t) ? (int)left : ucost - c.t;
        const int lo = c.t > kPieceCost ? c.t - kPieceCost : 0;
        const int hi = c.t + avail - kPieceCost < ng ? c.t + avail - kPieceCost : ng;
        if (hi > lo) {
            Piece p;
            p.b = c.b;
            p.x = c.x;
            p.lo = lo;
            p.hi = hi;
            p.n = n;
            p.t0 = (long)lo * kGranule;
            p.t1 = (long)hi * kGranule < n ? (long)hi * kGranule : n;
            p.slot = w + c.rank;
            p.first = lo == 0;
            p.desc_count = 0;
            if (p.first) {  // this work-group owns granule 0: the unit's first slot is p.slot
                const long long ustart = c.pos - c.t;  // the unit's first position
                const int first = balanced_owner(ustart + kPieceCost, c.total, c.w_eff);
                const int last = balanced_owner(ustart + kPieceCost + ng - 1, c.total, c.w_eff);
                p.desc_count = last - first + 1;
            }
            visit(p);
        }
        c.pos += avail;
        if (c.pos >= c.end)
            break;
        // next unit: the next non-empty sequence of this KV head, else the
        // first one of the next KV head
        c.t = 0;
        ++c.rank;
        do {
            if (++c.b == batch) {
                c.b = 0;
                if (++c.x == hx)
                    break;
            }
            n = clamp_len(kv_lens, c.b, max_kv_len);
        } while (n == 0);
        if (c.x == hx)
            break;  // not reached: positions remain, so a non-empty unit follows
        ng = (n + kGranule - 1) / kGranule;
    }
}

}  // namespace fd
