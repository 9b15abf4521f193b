// split_valu.hip -- split stage of split-KV decode attention on the gfx950
// vector ALUs.
//
// Sources (pages; sections as printed on them):
//   [P1] "FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15)
//   [P3] "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
//        (my-webpage-adu.pages.dev, 2026-07-16)
//   [P4] "从第一性原理推导 Flash Attention：IO 复杂度、Tiling 策略与在线 Softmax 的数学工程"
//        (www.ybb.press)
//
// A work-group owns one split i of one sequence b for HPW consecutive query
// heads: tokens [i*L, min((i+1)*L, N_b)) of the KV heads those query heads
// read ([P1] §2.5 stage 1, step 2a).  The lanes form 16-lane DPP rows; a row
// holds one (head, token) pair at a time, every lane of the row owning d/16
// contiguous elements of that token's K and V rows, so one 128-bit load per
// lane fetches a whole 256-byte head row (d = 128, 16-bit types).  With
// HPW > 1 (fp32 grouped heads) the work-group serves HPW query heads of one
// KV head: every row holds all HPW q rows in registers and computes HPW dot
// products, HPW running states, from each K/V row it loads once.  A row reduces its q.K partial sums with four
// DPP adds and keeps a running (m, l, o) with the online update ([P1] §2.4.1
// incremental form, o left unnormalised as in the block update of [P4]
// §3.1); the rows of one head are merged in LDS with the same rule ([P4]
// §3.2 merge lemma), and the split writes o = o_acc / l and S = m + log l
// ([P3] §2.3.2-§2.3.3), or, in the m/l/o format, o with the split's max
// score m and l = sum exp(s - m) ([P1] §2.4.1 direct form).
//
// Scores are kept in the log2 domain: q is pre-multiplied by scale*log2(e)
// so every exponential is one v_exp_f32; the LSE is converted back to the
// natural log on output.  K/V go straight from HBM to VGPRs with
// non-temporal 128-bit loads (each byte is used once, by the lane that loads
// it, so staging through LDS would add traffic without reuse).  The next
// step's loads are issued before the current step's arithmetic.
//
// HBM efficiency on MI355X peaks when each CU has about two waves with
// ~16 KB of loads in flight each; more concurrent requests lower the
// achieved bandwidth.  So the launcher caps resident waves per CU at two by
// reserving LDS (the reservation is never touched), whatever the grid size:
// two one-wave work-groups, or one two-wave work-group whose waves take
// alternate token slots of the same split (used when there are fewer
// work-groups than wave slots, e.g. with one split per row, where it also
// makes the combine stage unnecessary).  When even the splits of all rows
// leave wave slots empty, one work-group per row runs one wave per split and
// merges the splits in LDS (FUSED), so a small decode is a single launch.
// Ragged batches instead take the token-balanced partition (BAL,
// partition_plan.h): 2 * CUs one-wave work-groups, each walking an equal
// share of the (query head, sequence, token) space piece by piece, every
// piece an ordinary split of one row written to its slot.
#include <atomic>

#include "dev_common.h"
#include "partition.h"

namespace fd {
namespace {

#ifndef FD_VALU_STEP_BYTES
#define FD_VALU_STEP_BYTES 64
#endif

template <int DT, int D, int LPR>
struct Layout {
    static constexpr int E = ElemInfo<DT>::bytes;
    static constexpr int ROW_BYTES = D * E;             // one token, one head
    static constexpr int LANE_BYTES = ROW_BYTES / LPR;  // 8, 16, 32 or 64
    static constexpr bool HALF = LANE_BYTES == 8;       // one 64-bit load per lane
    static constexpr int NV = HALF ? 1 : LANE_BYTES / 16;
    static constexpr int WORDS = LANE_BYTES / 4;
    static constexpr int EPL = D / LPR;                 // elements per lane
    static constexpr int PW = ElemInfo<DT>::per_word;
    static constexpr int SPAN = LPR * 16;               // bytes one 128-bit load covers per row
    static_assert(LANE_BYTES >= 8, "row too short for this lane count");
    // Element index held by lane `sub` in word j, sub-element e.  Full 16-byte
    // vectors are spread so that each load instruction covers whole
    // contiguous spans of a row.
    __device__ static constexpr int elem(int sub, int j, int e) {
        if (HALF)
            return sub * (8 / E) + j * PW + e;
        return (j / 4) * (SPAN / E) + sub * (16 / E) + (j % 4) * PW + e;
    }
    // Tokens per row per step: FD_VALU_STEP_BYTES of K (and as many of V)
    // per lane.
    static constexpr int U =
        FD_VALU_STEP_BYTES / LANE_BYTES > 0 ? FD_VALU_STEP_BYTES / LANE_BYTES : 1;
};

// Load this lane's words of one row; `p` already includes the lane's byte
// offset inside the row (sub * 8 or sub * 16).
template <int DT, int D, int LPR>
__device__ __forceinline__ void load_row(const char *p, uint32_t *w) {
    using L = Layout<DT, D, LPR>;
    if constexpr (L::HALF) {
        const u32x2 x = ld64<1>(p);
        w[0] = x[0];
        w[1] = x[1];
    } else {
#pragma unroll
        for (int c = 0; c < L::NV; ++c) {
            const u32x4 x = ld128<1>(p + c * L::SPAN);
            w[4 * c + 0] = x[0];
            w[4 * c + 1] = x[1];
            w[4 * c + 2] = x[2];
            w[4 * c + 3] = x[3];
        }
    }
}

template <int DT, int D, int LPR>
__device__ __forceinline__ void unpack_row(const uint32_t *w, float *f) {
    using L = Layout<DT, D, LPR>;
#pragma unroll
    for (int j = 0; j < L::WORDS; ++j)
        unpack_word<DT>(w[j], f + j * L::PW);
}

// FUSED: one work-group per (sequence, head group) whose wave w computes split
// w (num_splits <= THREADS / 64); the LDS merge then combines the splits and
// the work-group writes the final output (a combine stage in LDS).
// BAL: token-balanced partition (partition_plan.h) over units of HPW query
// heads: a one-wave work-group walks its share piece by piece, each piece of
// unit (b, head group) writing its HPW (o, LSE) pairs to slot w + rank(unit)
// and the unit's first piece its descriptor {first slot, count}, as the
// matrix-core balanced kernel does for a group.
template <int DT, int D, int THREADS, int HPW, int LPR, bool PAGED, bool FUSED = false,
          bool BAL = false>
__global__ __launch_bounds__(THREADS) void split_valu_kernel(SplitArgs a) {
    using L = Layout<DT, D, LPR>;
    constexpr int EPL = L::EPL;
    constexpr int WORDS = L::WORDS;
    constexpr int U = L::U;
    constexpr int kRows = THREADS / LPR;  // rows of LPR lanes
    constexpr int RPW = 64 / LPR;         // rows per wave
    // token slots per step position: the work-group's rows share one split,
    // or (FUSED) each wave's rows share that wave's split
    constexpr int TPS = FUSED ? RPW : kRows;
    static_assert(HPW >= 1 && HPW <= 8, "one to eight query heads per work-group");
    static_assert(!BAL || (THREADS == 64 && !FUSED),
                  "balanced pieces run on one-wave work-groups");

    __shared__ float sm_acc[HPW][kRows][D];
    __shared__ float sm_m[HPW][kRows];
    __shared__ float sm_l[HPW][kRows];

    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    const int row = tid / LPR;
    const int tslot = FUSED ? row % RPW : row;  // token slot of this row

    // One piece: tokens [t0, t1) of sequence b for head group hg (query heads
    // hg * HPW .. hg * HPW + HPW - 1, one KV head), written as split `split`
    // of its rows (fixed splits) or to slot `bslot` (BAL).
    auto run = [&](int b, int hg, int split, long t0, long t1, long bslot) {
    const int kvh = hg * HPW / (a.heads_q / a.heads_kv);

    // per head of the group: running max of log2-domain scores in this row,
    // running sum of exp2(s - m), and of exp2(s - m) * V (unnormalised)
    float m[HPW], l[HPW], acc[HPW][EPL];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            acc[h][i] = 0.f;
    }

    if (t0 < t1) {
        const uint32_t lane_byte = L::HALF ? sub * 8u : sub * 16u;
        // q rows of the group's heads.  fp32: pre-scaled into the log2 domain.
        // 16-bit types: kept packed for the two-wide dot products (the
        // products of two bf16 or two fp16 values are exact in fp32), and the
        // scale is applied to the reduced score instead.
        uint32_t qw[HPW][WORDS];
        float qf[HPW][EPL];
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            const char *qrow = static_cast<const char *>(a.q) +
                               ((size_t)b * a.heads_q + hg * HPW + h) * (size_t)L::ROW_BYTES;
            load_row<DT, D, LPR>(qrow + lane_byte, qw[h]);
            if constexpr (DT == kF32) {
                unpack_row<DT, D, LPR>(qw[h], qf[h]);
#pragma unroll
                for (int i = 0; i < EPL; ++i)
                    qf[h][i] *= a.scale_log2;
            }
        }
        // K/V addressing: a uniform (scalar) base per step plus a 32-bit
        // per-lane byte offset (token slot, head, lane), so the loads use the
        // SGPR-base form.  One token's row over all heads is at most 16 MiB,
        // and a page at most 2 GiB (both checked on the host), so every offset
        // below fits in 32 bits.
        const size_t tok_stride = (size_t)a.heads_kv * L::ROW_BYTES;
        const uint32_t stride32 = (uint32_t)tok_stride;
        const uint32_t lane_off = (uint32_t)kvh * (uint32_t)L::ROW_BYTES + lane_byte;
        const int ntok = (int)(t1 - t0);
        constexpr int kStepTok = TPS * U;  // tokens per step
        const int nsteps = (ntok + kStepTok - 1) / kStepTok;

        uint32_t kw[U][WORDS], vw[U][WORDS];
        // Paged K/V: the pages of a step's 16-token tiles, looked up one step
        // ahead of the loads that use them (the loop below), so the table
        // read's latency hides behind a step of arithmetic.  t0 and the step
        // start are multiples of min(16, kStepTok), so each slot group of TPS
        // tokens lies in one tile, hence in one page, also after clamping to
        // the last valid token.
        constexpr int NTILE = kStepTok >= 16 ? kStepTok / 16 : 1;
        struct Pages {
            int pg[NTILE];
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
                for (int j = 0; j < NTILE; ++j) {
                    const int rel = 16 * j < last_rel ? 16 * j : last_rel;
                    P.pg[j] = bt[((int)t0 + first + rel) >> a.page_shift];  // clamped at use
                }
            }
        };
        // Step `st` covers tokens t0 + st*TPS*U + u*TPS + tslot.  Slots past
        // the end re-read the last valid token (always in bounds) and are
        // masked, and a step past the last one re-reads the last step.
        auto load_step = [&](int st, const Pages &P, uint32_t (*kd)[WORDS],
                             uint32_t (*vd)[WORDS]) {
            const int sa = st < nsteps ? st : nsteps - 1;
            const int first = sa * kStepTok;
            const int last_rel = ntok - 1 - first;
            if constexpr (!PAGED) {
                const size_t seq = a.shared_kv ? 0 : (size_t)b * a.max_kv_len;
                const size_t base = (seq + (size_t)t0 + first) * tok_stride;
                const char *kb = static_cast<const char *>(a.k) + base;
                const char *vb = static_cast<const char *>(a.v) + base;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int rel = u * TPS + tslot;
                    rel = rel < last_rel ? rel : last_rel;
                    const uint32_t off = (uint32_t)rel * stride32 + lane_off;
                    load_row<DT, D, LPR>(kb + off, kd[u]);
                    load_row<DT, D, LPR>(vb + off, vd[u]);
                }
            } else {
                const size_t page_stride = tok_stride << a.page_shift;
                const uint32_t pmask = (1u << a.page_shift) - 1u;
                const int t_first = (int)t0 + first;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int j = kStepTok >= 16 ? (u * TPS) / 16 : 0;
                    int rel = u * TPS + tslot;
                    rel = rel < last_rel ? rel : last_rel;
                    const uint32_t off =
                        ((uint32_t)(t_first + rel) & pmask) * stride32 + lane_off;
                    int pg = P.pg[j];
                    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
                    const size_t pbase = (size_t)pg * page_stride;
                    load_row<DT, D, LPR>(static_cast<const char *>(a.k) + pbase + off, kd[u]);
                    load_row<DT, D, LPR>(static_cast<const char *>(a.v) + pbase + off, vd[u]);
                }
            }
        };
        // One step of arithmetic on the K/V words of step `st`.
        auto compute_step = [&](int st, const uint32_t (*kc)[WORDS],
                                const uint32_t (*vc)[WORDS]) {
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
                // scores s_u = (q * scale * log2e) . K_u, summed over the row's lanes
                float s[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float part = 0.f;
                    if constexpr (DT == kF32) {
                        float kf[EPL];
                        unpack_row<DT, D, LPR>(kc[u], kf);
#pragma unroll
                        for (int i = 0; i < EPL; ++i)
                            part = __builtin_fmaf(qf[h][i], kf[i], part);
                        s[u] = row_sum<LPR>(part);
                    } else {
#pragma unroll
                        for (int j = 0; j < WORDS; ++j)
                            part = dot2<DT>(qw[h][j], kc[u][j], part);
                        s[u] = row_sum<LPR>(part) * a.scale_log2;
                    }
                    const int rel = st * kStepTok + u * TPS + tslot;
                    s[u] = rel < ntok ? s[u] : -INFINITY;
                }
                // online update of (m, l, acc) of head h by U tokens
                float mx = m[h];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    mx = fmaxf(mx, s[u]);
                const float mref = mx == -INFINITY ? 0.f : mx;  // no token seen yet
                const float alpha = fast_exp2(m[h] - mref);
                float p[U];
                float psum = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    p[u] = fast_exp2(s[u] - mref);
                    psum += p[u];
                }
                l[h] = __builtin_fmaf(l[h], alpha, psum);
#pragma unroll
                for (int i = 0; i < EPL; ++i)
                    acc[h][i] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float vf[EPL];
                    unpack_row<DT, D, LPR>(vc[u], vf);
#pragma unroll
                    for (int i = 0; i < EPL; ++i)
                        acc[h][i] = __builtin_fmaf(p[u], vf[i], acc[h][i]);
                }
                m[h] = mx;
            }
        };

        // Software pipeline over two register buffers: while step st is
        // computed from one buffer, the loads of step st+1 fill the other.
        // The loop runs whole pairs of steps with unconditional prefetches (a
        // step past the end re-reads the last one, see load_step), so no path
        // into the loop header has the newer loads pending; the scheduling
        // barriers keep the compiler from sinking a prefetch below the waits
        // for the step being computed.
        uint32_t kx[U][WORDS], vx[U][WORDS];
        const int npairs = nsteps >> 1;
        Pages pa, pb;
        lookup(0, pa);
        load_step(0, pa, kw, vw);
        lookup(1, pb);
        for (int pr = 0; pr < npairs; ++pr) {
            const int st = 2 * pr;
            load_step(st + 1, pb, kx, vx);
            lookup(st + 2, pa);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(st, kw, vw);
            load_step(st + 2, pa, kw, vw);
            lookup(st + 3, pb);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(st + 1, kx, vx);
        }
        if (nsteps & 1)
            compute_step(nsteps - 1, kw, vw);
    }

    // Merge the row states of each head (BAL: after the previous piece's
    // merge has read the LDS rows this one overwrites).
    if constexpr (BAL)
        __syncthreads();
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        if (sub == 0) {
            sm_m[h][row] = m[h];
            sm_l[h][row] = l[h];
        }
#pragma unroll
        for (int j = 0; j < WORDS; ++j)
#pragma unroll
            for (int e = 0; e < L::PW; ++e)
                sm_acc[h][row][L::elem(sub, j, e)] = acc[h][j * L::PW + e];
    }
    __syncthreads();

    for (int idx = tid; idx < HPW * D; idx += THREADS) {
        const int hh = idx / D;
        const int dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int r = 0; r < kRows; ++r)
            M = fmaxf(M, sm_m[hh][r]);
        float out = 0.f, lse = -INFINITY, Ls = 0.f;
        if (M != -INFINITY) {
            float Os = 0.f;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const float w = fast_exp2(sm_m[hh][r] - M);
                Ls = __builtin_fmaf(w, sm_l[hh][r], Ls);
                Os = __builtin_fmaf(w, sm_acc[hh][r][dd], Os);
            }
            out = Os / Ls;
            lse = (M + fast_log2(Ls)) * kLn2;
        }
        const size_t rowid = (size_t)b * a.heads_q + hg * HPW + hh;
        if constexpr (BAL) {  // slot bslot holds the HPW heads' rows
            a.o_part[((size_t)bslot * HPW + hh) * D + dd] = out;
            if (dd == 0)
                a.lse_part[(size_t)bslot * HPW + hh] = lse;
        } else if (a.o_part) {
            const size_t slot =
                rowid * (a.part_stride ? a.part_stride : a.num_splits) + a.part_offset + split;
            a.o_part[slot * D + dd] = out;
            if (dd == 0) {
                if (a.m_part) {  // m/l/o triple: the split's max score and l relative to it
                    a.m_part[slot] = M == -INFINITY ? -INFINITY : M * kLn2;
                    a.l_part[slot] = M == -INFINITY ? 0.f : Ls;
                } else {
                    a.lse_part[slot] = lse;
                }
            }
        } else {
            store_out(a.o, rowid * D + dd, out, a.out_dtype);
            if (dd == 0 && a.lse)
                a.lse[rowid] = lse;
        }
    }
    };

    if constexpr (BAL) {
        // share index (partition_plan.h: neighbouring work-groups take
        // consecutive heads of one token range when the heads come in
        // multiples of 8)
        // units: (sequence, group of HPW query heads)
        const int hx = a.heads_q / HPW;
        const int w = share_index((int)blockIdx.x, hx, a.num_wgs);
        PieceCursor c;
        if (!balanced_start(a.kv_lens, a.batch, a.max_kv_len, hx, w, a.num_wgs, c))
            return;
        walk_share(a.kv_lens, a.batch, a.max_kv_len, hx, w, c, [&](const Piece &p) {
            run(p.b, p.x, 0, p.t0, p.t1, p.slot);
            if (p.first && threadIdx.x == 0) {  // the unit's descriptor {first slot, count}
                const size_t u = (size_t)p.b * hx + p.x;
                a.unit_desc[2 * u] = p.slot;
                a.unit_desc[2 * u + 1] = p.desc_count;
            }
        });
    } else {
        // Work-group -> (b, head group, split); the head group varies fastest so
        // that neighbouring work-groups read neighbouring head rows of the same
        // tokens.  FUSED: work-group -> (b, head group), split = wave.
        const int ngroups = a.heads_q / HPW;
        const int hg = blockIdx.x % ngroups;
        const int rest = blockIdx.x / ngroups;
        const int split = FUSED ? tid / 64 : rest % a.num_splits;
        const int b = FUSED ? rest : rest / a.num_splits;
        int n = a.kv_lens ? a.kv_lens[b] : a.max_kv_len;
        n = n < 0 ? 0 : (n > a.max_kv_len ? a.max_kv_len : n);
        // (FUSED waves past num_splits get an empty range)
        const long t0 = split < a.num_splits ? (long)split * a.split_len : (long)n;
        const long t1 = t0 + a.split_len < n ? t0 + a.split_len : n;
        run(b, hg, split, t0, t1, 0);
    }
}

// Resident work-groups per CU are capped by reserving LDS: a work-group
// asks for just over 1/(cap+1) of the CU's LDS, so cap of them fit.
int lds_per_cu() {
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

template <int DT, int D, int THREADS, int HPW, int LPR, bool PAGED, bool FUSED = false,
          bool BAL = false>
hipError_t launch_cfg(const SplitArgs &a, int wg_per_cu, hipStream_t stream) {
    constexpr int kRows = THREADS / LPR;
    constexpr size_t kStatic = sizeof(float) * (size_t)HPW * (kRows * D + 2 * kRows);
    const long grid =
        BAL ? (long)a.num_wgs : (long)a.batch * (a.heads_q / HPW) * (FUSED ? 1 : a.num_splits);
    auto kern = split_valu_kernel<DT, D, THREADS, HPW, LPR, PAGED, FUSED, BAL>;
    size_t pad = 0;
    const int lds = lds_per_cu();
    if (wg_per_cu > 0 && lds > 0) {
        const size_t want = (size_t)lds / (size_t)(wg_per_cu + 1) + 256;
        pad = want > kStatic ? want - kStatic : 0;
        if (pad > 65536) {
            // once per kernel and device (the pad depends only on the device)
            static std::atomic<bool> raised[64];
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 ||
                !raised[dev].load(std::memory_order_relaxed)) {
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)pad);
                if (e != hipSuccess)
                    return e;
                if (dev >= 0 && dev < 64)
                    raised[dev].store(true, std::memory_order_relaxed);
            }
        }
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(THREADS), pad, stream, a);
    return hipGetLastError();
}

#ifndef FD_VALU_ROW_BYTES
#define FD_VALU_ROW_BYTES 16  // bytes of a head row per lane (sets lanes per row)
#endif

// Lanes per token row: ROW_BYTES / FD_VALU_ROW_BYTES, clamped to [4, 16].
template <int DT, int D>
constexpr int lanes_per_row() {
    constexpr int r = D * ElemInfo<DT>::bytes / FD_VALU_ROW_BYTES;
    return r > 16 ? 16 : (r < 4 ? 4 : r);
}

// Every route but the fused one, HPW query heads per work-group.
template <int DT, int D, int HPW>
hipError_t launch_rows(const SplitArgs &a, hipStream_t stream) {
    constexpr int LPR = lanes_per_row<DT, D>();
    const int per_cu = valu_wg_per_cu(HPW);  // one-wave work-groups per CU
    if (a.balanced) {  // token-balanced shares, one-wave work-groups
        return a.block_table
                   ? launch_cfg<DT, D, 64, HPW, LPR, true, false, true>(a, per_cu, stream)
                   : launch_cfg<DT, D, 64, HPW, LPR, false, false, true>(a, per_cu, stream);
    }
    if (a.block_table) {
        if (a.valu_waves > 1)
            return launch_cfg<DT, D, 64 * kWavesPerCU, HPW, LPR, true>(a, 1, stream);
        return launch_cfg<DT, D, 64, HPW, LPR, true>(a, per_cu, stream);
    }
    if (a.valu_waves > 1)
        return launch_cfg<DT, D, 64 * kWavesPerCU, HPW, LPR, false>(a, 1, stream);
    return launch_cfg<DT, D, 64, HPW, LPR, false>(a, per_cu, stream);
}

template <int DT, int D>
hipError_t launch(const SplitArgs &a, hipStream_t stream) {
    constexpr int LPR = lanes_per_row<DT, D>();
    if (a.fused_waves > 0) {  // small grid: all splits of a row in one work-group
        const bool pg = a.block_table != nullptr;
        switch (a.fused_waves) {
        case 2:
            return pg ? launch_cfg<DT, D, 128, 1, LPR, true, true>(a, 0, stream)
                      : launch_cfg<DT, D, 128, 1, LPR, false, true>(a, 0, stream);
        case 4:
            return pg ? launch_cfg<DT, D, 256, 1, LPR, true, true>(a, 0, stream)
                      : launch_cfg<DT, D, 256, 1, LPR, false, true>(a, 0, stream);
        case 8:
            return pg ? launch_cfg<DT, D, 512, 1, LPR, true, true>(a, 0, stream)
                      : launch_cfg<DT, D, 512, 1, LPR, false, true>(a, 0, stream);
        default:
            return hipErrorInvalidValue;
        }
    }
    if constexpr (DT == kF32) {  // grouped heads: HPW heads of one KV head per work-group
        switch (valu_heads_per_wg(DT, D, a.heads_q / a.heads_kv)) {
        case 8:
            if constexpr (D <= 128)
                return launch_rows<DT, D, 8>(a, stream);
            return hipErrorInvalidValue;
        case 4: return launch_rows<DT, D, 4>(a, stream);
        case 2: return launch_rows<DT, D, 2>(a, stream);
        default: break;
        }
    }
    return launch_rows<DT, D, 1>(a, stream);
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

hipError_t launch_split_valu(const SplitArgs &a, int in_dtype, hipStream_t stream) {
    switch (in_dtype) {
    case kF32: return launch_dt<kF32>(a, stream);
    case kF16: return launch_dt<kF16>(a, stream);
    case kBF16: return launch_dt<kBF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fd
