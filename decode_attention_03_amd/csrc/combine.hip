// combine.hip -- combine stage: LSE merge of the per-split partials.
//
// Source: "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
// (my-webpage-adu.pages.dev, 2026-07-16), §2.3.4 (global LSE, then
// exp(S_b - S_global)-weighted sum of the split outputs); the pages describe
// this stage as a light second reduction kernel ("FlashDecoding 数学推导",
// §2.5 stage 2).
//
// One work-group of 256 threads per (sequence, query head) row.  The row's
// num_splits LSE values are reduced by the whole work-group (max, then the
// shifted exp-sum) and the merge weights kept in LDS.  Each thread then owns
// four consecutive output elements (one float4 column slice) for every
// SP-th split, with four independent loads in flight, and the SP partial
// sums of each element are added in LDS in a fixed order, so the result is
// reproducible.  -inf partials (empty splits) get weight 0 and contribute
// exactly nothing; a row whose partials are all -inf yields o = 0, S = -inf.
//
// The m/l/o variant merges (m, l, o) triples instead ("FlashDecoding 数学推导"
// (my-webpage-adu.pages.dev, 2026-07-15) §2.4.2 and §2.5 stage 2).
//
// Two sources of partials: fixed splits ([batch, heads_q, B, d], B per row),
// or the slots of the token-balanced partition (partition.h), where a row's
// unit descriptor names its first slot and slot count and the row's partials
// sit gsz rows apart.
#include "dev_common.h"
#include "partition.h"

namespace fd {
namespace {

constexpr int kCombineThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// A row's partials: LSE i at S[i * s_stride], o_i at O + i * o_stride.  In the
// m/l/o format S holds m_i and L holds l_i (same stride).
struct RowSource {
    const float *S;
    const float *O;
    int count, s_stride, o_stride;
    const float *L;
    // optional second segment (LSE format only): partials count .. count +
    // count2 - 1 at S2[j * s_stride2] and O2 + j * o_stride2
    const float *S2 = nullptr;
    const float *O2 = nullptr;
    int count2 = 0, s_stride2 = 0, o_stride2 = 0;
};

// LSE (or m) of partial i over both segments of a row.
__device__ __forceinline__ float row_s(const RowSource &src, int i) {
    return i < src.count ? src.S[(size_t)i * src.s_stride]
                         : src.S2[(size_t)(i - src.count) * src.s_stride2];
}

// Column slice c (float4) of partial i over both segments of a row.
__device__ __forceinline__ float4 row_o(const RowSource &src, int i, int c) {
    const float *base = i < src.count ? src.O + (size_t)i * src.o_stride
                                      : src.O2 + (size_t)(i - src.count) * src.o_stride2;
    return reinterpret_cast<const float4 *>(base)[c];
}

template <int D, bool MLO = false>
__device__ __forceinline__ void combine_row(const RowSource src, size_t rowid, void *o,
                                            int out_dtype, float *lse, float *weights) {
    constexpr int V4 = D / 4;                     // float4 slices per row
    constexpr int SP = kCombineThreads / V4;      // splits processed side by side
    constexpr int NW = kCombineThreads / 64;
    __shared__ float red[NW];
    __shared__ float part[SP][D];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const float *S = src.S;
    const int num_splits = src.count + src.count2;
    const int ss = src.s_stride;

    // S_max over the row
    float mx = -INFINITY;
    for (int i = tid; i < num_splits; i += kCombineThreads)
        mx = fmaxf(mx, row_s(src, i));
    mx = wave_max(mx);
    if (lane == 0)
        red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        mx = fmaxf(mx, red[w]);
    __syncthreads();
    float sg;
    if constexpr (!MLO) {
        // S_global = S_max + log sum_i exp(S_i - S_max)
        float sum = 0.f;
        if (mx != -INFINITY)
            for (int i = tid; i < num_splits; i += kCombineThreads)
                sum += fast_exp2((row_s(src, i) - mx) * kLog2e);
        sum = wave_sum(sum);
        if (lane == 0)
            red[wave] = sum;
        __syncthreads();
        sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            sum += red[w];
        sg = mx == -INFINITY ? -INFINITY : mx + fast_log2(sum) * kLn2;
        for (int i = tid; i < num_splits; i += kCombineThreads)
            weights[i] = mx == -INFINITY ? 0.f : fast_exp2((row_s(src, i) - sg) * kLog2e);
    } else {
        // m/l/o ("FlashDecoding 数学推导" §2.4.2): m_g = max m_i (mx above),
        // l_g = sum_i exp(m_i - m_g) l_i, weights exp(m_i - m_g) l_i / l_g
        const float *Lp = src.L;
        float lg = 0.f;
        if (mx != -INFINITY)
            for (int i = tid; i < num_splits; i += kCombineThreads) {
                const float m = S[(size_t)i * ss];
                lg += m == -INFINITY ? 0.f : fast_exp2((m - mx) * kLog2e) * Lp[(size_t)i * ss];
            }
        lg = wave_sum(lg);
        if (lane == 0)
            red[wave] = lg;
        __syncthreads();
        lg = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            lg += red[w];
        sg = mx == -INFINITY ? -INFINITY : mx + fast_log2(lg) * kLn2;
        const float inv = mx == -INFINITY ? 0.f : 1.f / lg;
        for (int i = tid; i < num_splits; i += kCombineThreads) {
            const float m = S[(size_t)i * ss];
            weights[i] = m == -INFINITY
                             ? 0.f
                             : fast_exp2((m - mx) * kLog2e) * Lp[(size_t)i * ss] * inv;
        }
    }
    __syncthreads();

    // o = sum_i w_i o_i: thread (sp, c) takes splits sp, sp + SP, ... of slice c
    const int c = tid % V4;
    const int sp = tid / V4;

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](float w, float4 x) {
        // weight 0 (an empty split) contributes nothing, whatever the slot holds
        acc.x += w == 0.f ? 0.f : w * x.x;
        acc.y += w == 0.f ? 0.f : w * x.y;
        acc.z += w == 0.f ? 0.f : w * x.z;
        acc.w += w == 0.f ? 0.f : w * x.w;
    };
    int i = sp;
    for (; i + 3 * SP < num_splits; i += 4 * SP) {
        const float4 x0 = row_o(src, i, c);
        const float4 x1 = row_o(src, i + SP, c);
        const float4 x2 = row_o(src, i + 2 * SP, c);
        const float4 x3 = row_o(src, i + 3 * SP, c);
        add(weights[i], x0);
        add(weights[i + SP], x1);
        add(weights[i + 2 * SP], x2);
        add(weights[i + 3 * SP], x3);
    }
    for (; i < num_splits; i += SP)
        add(weights[i], row_o(src, i, c));
    part[sp][4 * c + 0] = acc.x;
    part[sp][4 * c + 1] = acc.y;
    part[sp][4 * c + 2] = acc.z;
    part[sp][4 * c + 3] = acc.w;
    __syncthreads();
    if (tid < D) {
        float out = 0.f;
#pragma unroll
        for (int r = 0; r < SP; ++r)
            out += part[r][tid];
        store_out(o, rowid * D + tid, out, out_dtype);
        if (tid == 0 && lse)
            lse[rowid] = sg;
    }
}

// One pass over a row's partials, the merge folded in as it goes ("FlashDecoding
// 数学推导：传统 m/l/o 方法与 LSE 方法" §2.3.5: merging (o, S) pairs one at a time
// in any order gives the global pair).  The running pair is kept as (m, l, acc):
// the largest S so far, l = sum_i exp(S_i - m) and acc = sum_i exp(S_i - m) o_i;
// a partial with a larger S rescales both by exp(m_old - m_new).  At the end
// o = acc / l and S = m + log l.  The V4 threads of a row each own one float4
// column slice and read every partial's S (the same address for the row's
// threads) and their slice of its o; sixteen partials are loaded before any
// is merged, so a thread has up to 32 loads in flight, and nothing crosses
// threads: no LDS, no barrier.  -inf partials (empty splits) are skipped, so
// whatever their o slot holds contributes nothing.  The order is fixed, so the
// result is reproducible.
template <int D>
__device__ __forceinline__ void combine_row_online(const RowSource &src, int c, size_t rowid,
                                                   void *o, int out_dtype, float *lse) {
    const int n = src.count + src.count2;
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto merge = [&](float s, float4 x) {
        if (s == -INFINITY)
            return;
        if (s > m) {  // the new term sets the reference: rescale what is held
            const float alpha = m == -INFINITY ? 0.f : fast_exp2((m - s) * kLog2e);
            l = l * alpha + 1.f;
            acc.x = acc.x * alpha + x.x;
            acc.y = acc.y * alpha + x.y;
            acc.z = acc.z * alpha + x.z;
            acc.w = acc.w * alpha + x.w;
            m = s;
        } else {
            const float e = fast_exp2((s - m) * kLog2e);
            l += e;
            acc.x += e * x.x;
            acc.y += e * x.y;
            acc.z += e * x.z;
            acc.w += e * x.w;
        }
    };
    // up to kChunk partials' loads in flight before they are merged (all of a
    // row's partials at once for rows of up to kChunk, e.g. 16 splits)
    constexpr int kChunk = 16;
    for (int i = 0; i < n; i += kChunk) {
        float s[kChunk];
        float4 x[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            s[k] = -INFINITY;
            x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (i + k < n) {
                s[k] = row_s(src, i + k);
                x[k] = row_o(src, i + k, c);
            }
        }
#pragma unroll
        for (int k = 0; k < kChunk; ++k)
            merge(s[k], x[k]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t base = rowid * D + 4 * c;
    store_out(o, base + 0, acc.x * inv, out_dtype);
    store_out(o, base + 1, acc.y * inv, out_dtype);
    store_out(o, base + 2, acc.z * inv, out_dtype);
    store_out(o, base + 3, acc.w * inv, out_dtype);
    if (c == 0 && lse)
        lse[rowid] = l > 0.f ? m + fast_log2(l) * kLn2 : -INFINITY;
}

// Rows per one-pass combine work-group: 256 threads, D / 4 per row.
template <int D>
constexpr int online_rows() {
    return kCombineThreads / (D / 4);
}

// Fixed splits, one pass: rows_per_block rows of B contiguous partials each.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_online_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part, int num_splits,
    int rows, void *o, int out_dtype, float *lse) {
    constexpr int V4 = D / 4;
    const size_t rowid = (size_t)blockIdx.x * online_rows<D>() + threadIdx.x / V4;
    if (rowid >= (size_t)rows)
        return;
    const RowSource src{lse_part + rowid * num_splits, o_part + rowid * num_splits * D,
                        num_splits, 1, D, nullptr};
    combine_row_online<D>(src, (int)(threadIdx.x % V4), rowid, o, out_dtype, lse);
}

// Fixed splits: row r's partials are contiguous, B of them.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part, int num_splits, void *o,
    int out_dtype, float *lse) {
    extern __shared__ float weights[];  // num_splits entries
    const size_t rowid = blockIdx.x;
    const RowSource src{lse_part + rowid * num_splits, o_part + rowid * num_splits * D, num_splits,
                        1, D, nullptr};
    combine_row<D>(src, rowid, o, out_dtype, lse, weights);
}

// m/l/o triples of fixed splits.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_mlo_kernel(
    const float *__restrict__ o_part, const float *__restrict__ m_part,
    const float *__restrict__ l_part, int num_splits, void *o, int out_dtype, float *lse) {
    extern __shared__ float weights[];  // num_splits entries
    const size_t rowid = blockIdx.x;
    const RowSource src{m_part + rowid * num_splits, o_part + rowid * num_splits * D, num_splits,
                        1, D, l_part + rowid * num_splits};
    combine_row<D, true>(src, rowid, o, out_dtype, lse, weights);
}

// Token-balanced slots: row (b, h) of unit u = b * (heads_q / gsz) + h / gsz
// reads slots first .. first + count - 1 of its unit's descriptor; a sequence
// with no tokens has no descriptor and contributes nothing (alone: (0, -inf)).
// A cascade adds the row's pre_count prefix partials in front.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_slots_kernel(SlotCombineArgs a) {
    extern __shared__ float weights[];  // max_count entries
    const size_t rowid = blockIdx.x;
    const int b = (int)(rowid / a.heads_q);
    const int h = (int)(rowid % a.heads_q);
    const int g = h % a.gsz;
    const size_t u = (size_t)b * (a.heads_q / a.gsz) + h / a.gsz;
    // first segment: the row's fixed partials (a cascade's prefix splits), if any
    RowSource src{a.pre_lse + rowid * a.pre_count, a.pre_o + rowid * a.pre_count * D,
                  a.pre_count, 1, D, nullptr};
    src.S2 = a.lse_slots;
    src.O2 = a.o_slots;
    src.s_stride2 = a.gsz;
    src.o_stride2 = a.gsz * D;
    if (clamp_len(a.kv_lens, b, a.max_kv_len) > 0) {
        const int first = a.unit_desc[2 * u];
        src.count2 = a.unit_desc[2 * u + 1];
        src.S2 = a.lse_slots + (size_t)first * a.gsz + g;
        src.O2 = a.o_slots + ((size_t)first * a.gsz + g) * D;
    }
    combine_row<D>(src, rowid, a.o, a.out_dtype, a.lse, weights);
}

// Token-balanced slots (and a cascade's prefix partials), one pass:
// rows_per_block rows per work-group, each row as in combine_slots_kernel.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_slots_online_kernel(SlotCombineArgs a) {
    constexpr int V4 = D / 4;
    const size_t rowid = (size_t)blockIdx.x * online_rows<D>() + threadIdx.x / V4;
    if (rowid >= (size_t)a.batch * a.heads_q)
        return;
    const int b = (int)(rowid / a.heads_q);
    const int h = (int)(rowid % a.heads_q);
    const int g = h % a.gsz;
    const size_t u = (size_t)b * (a.heads_q / a.gsz) + h / a.gsz;
    // the descriptor is read whether or not the sequence has tokens (units of
    // empty sequences have none written; their entries are read, then ignored),
    // so its load and the length's go out together
    const int first = a.unit_desc[2 * u];
    const int count = a.unit_desc[2 * u + 1];
    const bool any = clamp_len(a.kv_lens, b, a.max_kv_len) > 0;
    RowSource src{a.pre_lse + rowid * a.pre_count, a.pre_o + rowid * a.pre_count * D,
                  a.pre_count, 1, D, nullptr};
    src.s_stride2 = a.gsz;
    src.o_stride2 = a.gsz * D;
    src.count2 = any ? count : 0;
    src.S2 = a.lse_slots + (any ? (size_t)first * a.gsz + g : 0);
    src.O2 = a.o_slots + (any ? ((size_t)first * a.gsz + g) * D : 0);
    combine_row_online<D>(src, (int)(threadIdx.x % V4), rowid, a.o, a.out_dtype, a.lse);
}

}  // namespace

// One-pass combine kernels (1) or the work-group-per-row kernels with LDS
// reductions (0).  Measured by kernel trace: 4.6 us either way on rows of up
// to 16 partials; on the cascade's rows of 36 partials the one-pass kernel
// took 9.6 us against 6.5 (its chain of merges is as long as the row), so the
// work-group-per-row kernels are the default.
#ifndef FD_COMBINE_ONLINE
#define FD_COMBINE_ONLINE 0
#endif

template <int D>
void launch_online(const float *o_part, const float *lse_part, int rows, int num_splits, void *o,
                   int out_dtype, float *lse, hipStream_t stream) {
    const unsigned blocks = (unsigned)((rows + online_rows<D>() - 1) / online_rows<D>());
    hipLaunchKernelGGL(combine_online_kernel<D>, dim3(blocks), dim3(kCombineThreads), 0, stream,
                       o_part, lse_part, num_splits, rows, o, out_dtype, lse);
}

template <int D>
void launch_slots_online(const SlotCombineArgs &c, hipStream_t stream) {
    const size_t rows = (size_t)c.batch * c.heads_q;
    const unsigned blocks = (unsigned)((rows + online_rows<D>() - 1) / online_rows<D>());
    hipLaunchKernelGGL(combine_slots_online_kernel<D>, dim3(blocks), dim3(kCombineThreads), 0,
                       stream, c);
}

hipError_t launch_combine(const float *o_part, const float *lse_part, int rows, int num_splits,
                          int head_dim, void *o, int out_dtype, float *lse, hipStream_t stream) {
    if (FD_COMBINE_ONLINE) {
        switch (head_dim) {
        case 64: launch_online<64>(o_part, lse_part, rows, num_splits, o, out_dtype, lse, stream);
            break;
        case 128: launch_online<128>(o_part, lse_part, rows, num_splits, o, out_dtype, lse, stream);
            break;
        case 256: launch_online<256>(o_part, lse_part, rows, num_splits, o, out_dtype, lse, stream);
            break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const size_t shmem = sizeof(float) * (size_t)num_splits;
    switch (head_dim) {
    case 64:
        hipLaunchKernelGGL(combine_kernel<64>, dim3(rows), dim3(kCombineThreads), shmem, stream,
                           o_part, lse_part, num_splits, o, out_dtype, lse);
        break;
    case 128:
        hipLaunchKernelGGL(combine_kernel<128>, dim3(rows), dim3(kCombineThreads), shmem, stream,
                           o_part, lse_part, num_splits, o, out_dtype, lse);
        break;
    case 256:
        hipLaunchKernelGGL(combine_kernel<256>, dim3(rows), dim3(kCombineThreads), shmem, stream,
                           o_part, lse_part, num_splits, o, out_dtype, lse);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine_mlo(const float *o_part, const float *m_part, const float *l_part,
                              int rows, int num_splits, int head_dim, void *o, int out_dtype,
                              float *lse, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (size_t)num_splits;
    switch (head_dim) {
    case 64:
        hipLaunchKernelGGL(combine_mlo_kernel<64>, dim3(rows), dim3(kCombineThreads), shmem, stream,
                           o_part, m_part, l_part, num_splits, o, out_dtype, lse);
        break;
    case 128:
        hipLaunchKernelGGL(combine_mlo_kernel<128>, dim3(rows), dim3(kCombineThreads), shmem,
                           stream, o_part, m_part, l_part, num_splits, o, out_dtype, lse);
        break;
    case 256:
        hipLaunchKernelGGL(combine_mlo_kernel<256>, dim3(rows), dim3(kCombineThreads), shmem,
                           stream, o_part, m_part, l_part, num_splits, o, out_dtype, lse);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine_slots(const SlotCombineArgs &c, hipStream_t stream) {
    if (FD_COMBINE_ONLINE) {
        switch (c.head_dim) {
        case 64: launch_slots_online<64>(c, stream); break;
        case 128: launch_slots_online<128>(c, stream); break;
        case 256: launch_slots_online<256>(c, stream); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const size_t shmem = sizeof(float) * (size_t)(c.max_count + c.pre_count);
    const dim3 grid((unsigned)((size_t)c.batch * c.heads_q));
    switch (c.head_dim) {
    case 64:
        hipLaunchKernelGGL(combine_slots_kernel<64>, grid, dim3(kCombineThreads), shmem, stream, c);
        break;
    case 128:
        hipLaunchKernelGGL(combine_slots_kernel<128>, grid, dim3(kCombineThreads), shmem, stream, c);
        break;
    case 256:
        hipLaunchKernelGGL(combine_slots_kernel<256>, grid, dim3(kCombineThreads), shmem, stream, c);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fd
