// combine.hip -- combine stage: LSE merge of the per-split partials.
//
// Source: "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
// (my-webpage-adu.pages.dev, 2026-07-16), §2.3.4 (global LSE, then
// exp(S_b - S_global)-weighted sum of the split outputs); the pages describe
// this stage as a light second reduction kernel ("FlashDecoding 数学推导",
// §2.5 stage 2).
//
// One work-group per (sequence, query head) row, head_dim threads.  Wave 0
// reduces the row's num_splits LSE values (max, then the shifted exp-sum),
// writes the merge weights to LDS, and every thread then forms one output
// element as the weighted sum down its column of o_part (consecutive threads
// read consecutive addresses).  -inf partials (empty splits) get weight 0;
// a row whose partials are all -inf yields o = 0 and S = -inf.
#include "dev_common.h"

namespace fd {
namespace {

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
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o_part,
                                                      const float *__restrict__ lse_part,
                                                      int num_splits, void *o, int out_dtype,
                                                      float *lse) {
    extern __shared__ float weights[];  // num_splits entries
    __shared__ float s_global;
    const int rowid = blockIdx.x;
    const int tid = threadIdx.x;
    const float *S = lse_part + (size_t)rowid * num_splits;

    if (tid < 64) {
        float mx = -INFINITY;
        for (int i = tid; i < num_splits; i += 64)
            mx = fmaxf(mx, S[i]);
        mx = wave_max(mx);
        float sum = 0.f;
        if (mx != -INFINITY)
            for (int i = tid; i < num_splits; i += 64)
                sum += fast_exp2((S[i] - mx) * kLog2e);
        sum = wave_sum(sum);
        const float sg = mx == -INFINITY ? -INFINITY : mx + fast_log2(sum) * kLn2;
        for (int i = tid; i < num_splits; i += 64)
            weights[i] = mx == -INFINITY ? 0.f : fast_exp2((S[i] - sg) * kLog2e);
        if (tid == 0)
            s_global = sg;
    }
    __syncthreads();

    if (tid < D) {
        const float *col = o_part + (size_t)rowid * num_splits * D + tid;
        float acc = 0.f;
        for (int i = 0; i < num_splits; ++i) {
            const float w = weights[i];
            // an empty split's o_part is 0, but skip it so nothing non-finite
            // left in an unwritten slot can leak in
            if (w != 0.f)
                acc = __builtin_fmaf(w, col[(size_t)i * D], acc);
        }
        store_out(o, (size_t)rowid * D + tid, acc, out_dtype);
        if (tid == 0 && lse)
            lse[rowid] = s_global;
    }
}

}  // namespace

hipError_t launch_combine(const float *o_part, const float *lse_part, int rows, int num_splits,
                          int head_dim, void *o, int out_dtype, float *lse, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (size_t)num_splits;
    const int threads = head_dim < 64 ? 64 : head_dim;
    switch (head_dim) {
    case 64:
        hipLaunchKernelGGL(combine_kernel<64>, dim3(rows), dim3(threads), shmem, stream, o_part,
                           lse_part, num_splits, o, out_dtype, lse);
        break;
    case 128:
        hipLaunchKernelGGL(combine_kernel<128>, dim3(rows), dim3(threads), shmem, stream, o_part,
                           lse_part, num_splits, o, out_dtype, lse);
        break;
    case 256:
        hipLaunchKernelGGL(combine_kernel<256>, dim3(rows), dim3(threads), shmem, stream, o_part,
                           lse_part, num_splits, o, out_dtype, lse);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fd
