// split_valu.hip -- split stage of split-KV decode attention on the gfx950
// vector ALUs (one query row per work-group).
//
// Sources (pages; sections as printed on them):
//   [P1] "FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15)
//   [P3] "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
//        (my-webpage-adu.pages.dev, 2026-07-16)
//   [P4] "从第一性原理推导 Flash Attention：IO 复杂度、Tiling 策略与在线 Softmax 的数学工程"
//        (www.ybb.press)
//
// One work-group (256 threads = 4 waves) owns one (sequence b, query head h,
// split i) and the tokens [i*L, min((i+1)*L, N_b)) of KV head h / group
// ([P1] §2.5 stage 1, step 2a).  The 64 lanes of a wave form four 16-lane
// DPP rows; each row holds one token at a time, every lane of the row owning
// d/16 contiguous elements of that token's K and V rows.  So one wave-wide
// 128-bit load instruction fetches four whole 256-byte rows (d = 128, 16-bit
// types), and the 16 rows of the work-group walk 16 consecutive tokens per
// step.  A row reduces its q.K partial sums with four DPP adds, keeps a
// running (m, l, o) with the online update ([P1] §2.4.1 incremental form,
// with o left unnormalised as in the block update of [P4] §3.1), and the 16
// row states are merged in LDS with the same rule ([P4] §3.2 merge lemma).
// The split writes o = o_acc / l and S = m + log l ([P3] §2.3.2-§2.3.3).
//
// Scores are kept in the log2 domain: q is pre-multiplied by scale*log2(e)
// so every exponential is one v_exp_f32; the LSE is converted back to the
// natural log on output.  K/V go straight from HBM to VGPRs: each lane uses
// exactly the bytes it loads, so staging through LDS would add traffic
// without reuse.  The next step's loads are issued before the current step's
// arithmetic so that every wave keeps two steps of K/V in flight.
#include "dev_common.h"

namespace fd {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = kThreads / 16;  // token slots per work-group step

template <int DT, int D>
struct Layout {
    static constexpr int E = ElemInfo<DT>::bytes;
    static constexpr int ROW_BYTES = D * E;            // one token, one head
    static constexpr int LANE_BYTES = ROW_BYTES / 16;  // 8, 16, 32 or 64
    static constexpr bool HALF = LANE_BYTES == 8;      // d = 64 with 16-bit types
    static constexpr int NV = HALF ? 1 : LANE_BYTES / 16;
    static constexpr int WORDS = LANE_BYTES / 4;
    static constexpr int EPL = D / 16;                 // elements per lane
    static constexpr int PW = ElemInfo<DT>::per_word;
    // Element index held by lane `sub` in word j, sub-element e.  Full 16-byte
    // vectors are spread so that each load instruction covers whole
    // contiguous 256-byte spans of a row.
    __device__ static constexpr int elem(int sub, int j, int e) {
        if (HALF)
            return sub * 4 + j * PW + e;
        return (j / 4) * (256 / E) + sub * (16 / E) + (j % 4) * PW + e;
    }
    // Default tokens per row per step: 64 bytes of K (and of V) per lane.
    static constexpr int U = 64 / LANE_BYTES;
};

// Load this lane's words of one row; `p` already includes the lane's byte
// offset inside the row (sub * 8 or sub * 16).
template <int DT, int D>
__device__ __forceinline__ void load_row(const char *p, uint32_t *w) {
    using L = Layout<DT, D>;
    if constexpr (L::HALF) {
        uint2 x = ld64(p);
        w[0] = x.x;
        w[1] = x.y;
    } else {
#pragma unroll
        for (int c = 0; c < L::NV; ++c) {
            uint4 x = ld128(p + c * 256);
            w[4 * c + 0] = x.x;
            w[4 * c + 1] = x.y;
            w[4 * c + 2] = x.z;
            w[4 * c + 3] = x.w;
        }
    }
}

template <int DT, int D>
__device__ __forceinline__ void unpack_row(const uint32_t *w, float *f) {
    using L = Layout<DT, D>;
#pragma unroll
    for (int j = 0; j < L::WORDS; ++j)
        unpack_word<DT>(w[j], f + j * L::PW);
}

template <int DT, int D, int U>
__global__ __launch_bounds__(kThreads) void split_valu_kernel(SplitArgs a) {
    using L = Layout<DT, D>;
    constexpr int EPL = L::EPL;
    constexpr int WORDS = L::WORDS;

    __shared__ float sm_acc[kRows][D];
    __shared__ float sm_m[kRows];
    __shared__ float sm_l[kRows];

    const int tid = threadIdx.x;
    const int sub = tid & 15;
    const int row = tid >> 4;

    // Work-group -> (b, hq, split); the query head varies fastest so that
    // neighbouring work-groups read neighbouring head rows of the same tokens.
    const int hq = blockIdx.x % a.heads_q;
    const int rest = blockIdx.x / a.heads_q;
    const int split = rest % a.num_splits;
    const int b = rest / a.num_splits;
    const int kvh = hq / (a.heads_q / a.heads_kv);

    int n = a.kv_lens ? a.kv_lens[b] : a.max_kv_len;
    n = n < 0 ? 0 : (n > a.max_kv_len ? a.max_kv_len : n);
    const long t0 = (long)split * a.split_len;
    const long t1 = t0 + a.split_len < n ? t0 + a.split_len : n;

    float m = -INFINITY;  // running max of log2-domain scores in this row
    float l = 0.f;        // running sum of exp2(s - m)
    float acc[EPL];       // running sum of exp2(s - m) * V (unnormalised)
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        acc[i] = 0.f;

    if (t0 < t1) {
        // q row of this head, pre-scaled into the log2 domain.
        float qf[EPL];
        {
            uint32_t qw[WORDS];
            const char *qrow = static_cast<const char *>(a.q) +
                               ((size_t)b * a.heads_q + hq) * (size_t)L::ROW_BYTES;
            load_row<DT, D>(qrow + (L::HALF ? sub * 8 : sub * 16), qw);
            unpack_row<DT, D>(qw, qf);
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                qf[i] *= a.scale_log2;
        }
        // K/V addressing: a uniform (scalar) base per step plus a 32-bit
        // per-lane byte offset, so the loads use the SGPR-base form and cost
        // two VALU ops of address arithmetic each.  tok_stride < 2^24 is
        // checked on the host, so every offset below fits in 32 bits.
        const size_t tok_stride = (size_t)a.heads_kv * L::ROW_BYTES;
        const size_t split_base =
            (((size_t)b * a.max_kv_len + (size_t)t0) * a.heads_kv + kvh) * L::ROW_BYTES;
        const char *kbase = static_cast<const char *>(a.k) + split_base;
        const char *vbase = static_cast<const char *>(a.v) + split_base;
        const uint32_t stride32 = (uint32_t)tok_stride;
        const uint32_t lane_byte = L::HALF ? sub * 8u : sub * 16u;
        const int ntok = (int)(t1 - t0);
        const int nsteps = (ntok + kRows * U - 1) / (kRows * U);

        uint32_t kw[U][WORDS], vw[U][WORDS];
        // Step `st` covers tokens t0 + st*16U + u*16 + row.  Slots past the end
        // re-read the last valid token (always in bounds) and are masked, and
        // a step past the last one re-reads the last step.
        auto load_step = [&](int st, uint32_t (*kd)[WORDS], uint32_t (*vd)[WORDS]) {
            const int sa = st < nsteps ? st : nsteps - 1;
            const int first = sa * (kRows * U);
            const int last_rel = ntok - 1 - first;
            const char *kb = kbase + (size_t)first * tok_stride;
            const char *vb = vbase + (size_t)first * tok_stride;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int rel = u * kRows + row;
                rel = rel < last_rel ? rel : last_rel;
                const uint32_t off = (uint32_t)rel * stride32 + lane_byte;
                load_row<DT, D>(kb + off, kd[u]);
                load_row<DT, D>(vb + off, vd[u]);
            }
        };
        // One step of arithmetic on the K/V words of step `st`.
        auto compute_step = [&](int st, const uint32_t (*kc)[WORDS],
                                const uint32_t (*vc)[WORDS]) {
            // scores s_u = (q * scale * log2e) . K_u, summed over the 16 lanes
            float s[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[EPL];
                unpack_row<DT, D>(kc[u], kf);
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; ++i)
                    part = __builtin_fmaf(qf[i], kf[i], part);
                s[u] = row16_sum(part);
                const int rel = st * (kRows * U) + u * kRows + row;
                s[u] = rel < ntok ? s[u] : -INFINITY;
            }
            // online update of (m, l, acc) by U tokens
            float mx = m;
#pragma unroll
            for (int u = 0; u < U; ++u)
                mx = fmaxf(mx, s[u]);
            const float mref = mx == -INFINITY ? 0.f : mx;  // no token seen yet
            const float alpha = fast_exp2(m - mref);
            float p[U];
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = fast_exp2(s[u] - mref);
                psum += p[u];
            }
            l = __builtin_fmaf(l, alpha, psum);
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                acc[i] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[EPL];
                unpack_row<DT, D>(vc[u], vf);
#pragma unroll
                for (int i = 0; i < EPL; ++i)
                    acc[i] = __builtin_fmaf(p[u], vf[i], acc[i]);
            }
            m = mx;
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
        load_step(0, kw, vw);
        for (int pr = 0; pr < npairs; ++pr) {
            const int st = 2 * pr;
            load_step(st + 1, kx, vx);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(st, kw, vw);
            load_step(st + 2, kw, vw);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(st + 1, kx, vx);
        }
        if (nsteps & 1)
            compute_step(nsteps - 1, kw, vw);
    }

    // Merge the 16 row states of the work-group.
    if (sub == 0) {
        sm_m[row] = m;
        sm_l[row] = l;
    }
#pragma unroll
    for (int j = 0; j < WORDS; ++j)
#pragma unroll
        for (int e = 0; e < L::PW; ++e)
            sm_acc[row][L::elem(sub, j, e)] = acc[j * L::PW + e];
    __syncthreads();

    if (tid < D) {
        float M = -INFINITY;
#pragma unroll
        for (int r = 0; r < kRows; ++r)
            M = fmaxf(M, sm_m[r]);
        float out = 0.f, lse = -INFINITY;
        if (M != -INFINITY) {
            float Ls = 0.f, Os = 0.f;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const float w = fast_exp2(sm_m[r] - M);
                Ls = __builtin_fmaf(w, sm_l[r], Ls);
                Os = __builtin_fmaf(w, sm_acc[r][tid], Os);
            }
            out = Os / Ls;
            lse = (M + fast_log2(Ls)) * kLn2;
        }
        const size_t rowid = (size_t)b * a.heads_q + hq;
        if (a.o_part) {
            const size_t slot = rowid * a.num_splits + split;
            a.o_part[slot * D + tid] = out;
            if (tid == 0)
                a.lse_part[slot] = lse;
        } else {
            store_out(a.o, rowid * D + tid, out, a.out_dtype);
            if (tid == 0 && a.lse)
                a.lse[rowid] = lse;
        }
    }
}

template <int DT, int D>
hipError_t launch(const SplitArgs &a, hipStream_t stream) {
    const long grid = (long)a.batch * a.heads_q * a.num_splits;
    hipLaunchKernelGGL((split_valu_kernel<DT, D, Layout<DT, D>::U>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, a);
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

hipError_t launch_split_valu(const SplitArgs &a, int in_dtype, hipStream_t stream) {
    switch (in_dtype) {
    case kF32: return launch_dt<kF32>(a, stream);
    case kF16: return launch_dt<kF16>(a, stream);
    case kBF16: return launch_dt<kBF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fd
