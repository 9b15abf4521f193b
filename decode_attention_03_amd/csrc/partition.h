// partition.h -- the device side of the token-balanced partition (definitions,
// layout and the walk of a share are in partition_plan.h): the wave-wide scan
// that finds where a work-group's share starts.
#pragma once

#include "dev_common.h"
#include "partition_plan.h"

namespace fd {

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

// Where one work-group's share of the flattened space starts: the cursor
// balanced_start_ref defines, found with a wave-wide scan over the sequences.
// Called by all 64 lanes of the wave together; every result is the same on
// every lane.
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

}  // namespace fd
