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
#include "dev_common.h"

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

template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part, int num_splits, void *o,
    int out_dtype, float *lse) {
    constexpr int V4 = D / 4;                     // float4 slices per row
    constexpr int SP = kCombineThreads / V4;      // splits processed side by side
    constexpr int NW = kCombineThreads / 64;
    extern __shared__ float weights[];            // num_splits entries
    __shared__ float red[NW];
    __shared__ float part[SP][D];
    const int rowid = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const float *S = lse_part + (size_t)rowid * num_splits;

    // S_max over the row
    float mx = -INFINITY;
    for (int i = tid; i < num_splits; i += kCombineThreads)
        mx = fmaxf(mx, S[i]);
    mx = wave_max(mx);
    if (lane == 0)
        red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        mx = fmaxf(mx, red[w]);
    __syncthreads();
    // S_global = S_max + log sum_i exp(S_i - S_max)
    float sum = 0.f;
    if (mx != -INFINITY)
        for (int i = tid; i < num_splits; i += kCombineThreads)
            sum += fast_exp2((S[i] - mx) * kLog2e);
    sum = wave_sum(sum);
    if (lane == 0)
        red[wave] = sum;
    __syncthreads();
    sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        sum += red[w];
    const float sg = mx == -INFINITY ? -INFINITY : mx + fast_log2(sum) * kLn2;
    for (int i = tid; i < num_splits; i += kCombineThreads)
        weights[i] = mx == -INFINITY ? 0.f : fast_exp2((S[i] - sg) * kLog2e);
    __syncthreads();

    // o = sum_i w_i o_i: thread (sp, c) takes splits sp, sp + SP, ... of slice c
    const int c = tid % V4;
    const int sp = tid / V4;
    const float4 *col = reinterpret_cast<const float4 *>(o_part + (size_t)rowid * num_splits * D) + c;
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
        const float4 x0 = col[(size_t)i * V4];
        const float4 x1 = col[(size_t)(i + SP) * V4];
        const float4 x2 = col[(size_t)(i + 2 * SP) * V4];
        const float4 x3 = col[(size_t)(i + 3 * SP) * V4];
        add(weights[i], x0);
        add(weights[i + SP], x1);
        add(weights[i + 2 * SP], x2);
        add(weights[i + 3 * SP], x3);
    }
    for (; i < num_splits; i += SP)
        add(weights[i], col[(size_t)i * V4]);
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
        store_out(o, (size_t)rowid * D + tid, out, out_dtype);
        if (tid == 0 && lse)
            lse[rowid] = sg;
    }
}

}  // namespace

hipError_t launch_combine(const float *o_part, const float *lse_part, int rows, int num_splits,
                          int head_dim, void *o, int out_dtype, float *lse, hipStream_t stream) {
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

}  // namespace fd
