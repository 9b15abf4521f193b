/*
 * fd.h -- C ABI of libfd, split-KV ("FlashDecoding") decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (pages; sections as printed on them):
 *   [P1] "FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15)
 *   [P2] "adv04: Flash-Decoding（长序列 Decode 切分 + FlashInfer 简介）"
 *        (mini-vllm-tutorial.vercel.app)
 *   [P3] "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
 *        (my-webpage-adu.pages.dev, 2026-07-16)
 *
 * The operation.  For every sequence b and query head h there is one query
 * row q[b,h,:] of length d.  Against the first N_b cached tokens of the key /
 * value head kvh = h / (heads_q / heads_kv) it computes
 *     o[b,h,:] = softmax(s) V,   s_j = scale * q[b,h,:] . K[b,j,kvh,:]
 *     lse[b,h] = log sum_j exp(s_j)            (natural log)
 * ([P1] §2.1.1; [P3] §2.1.1 and §2.3.1).  The KV range is cut into
 * num_splits splits of split_len tokens ([P1] §2.1.3 and §2.5; [P2] §3);
 * fd_decode_split emits one (o, LSE) pair per split ([P3] §2.3.3) and
 * fd_combine merges them with exp(S_b - S_global) weights ([P3] §2.3.4).
 *
 * Layouts (row-major, innermost dimension contiguous, no padding):
 *   q        [batch, heads_q, head_dim]              in_dtype
 *   k, v     [batch, max_kv_len, heads_kv, head_dim] in_dtype
 *   kv_lens  [batch] int32 (device memory), or NULL: every N_b = max_kv_len.
 *            Values are clamped to [0, max_kv_len].
 *   o        [batch, heads_q, head_dim]              out_dtype
 *   lse      [batch, heads_q] float32, natural log of the scaled scores'
 *            exp-sum; -inf for a sequence with no tokens (o is then 0).
 *   o_part   [batch, heads_q, num_splits, head_dim]  float32
 *   lse_part [batch, heads_q, num_splits]            float32
 *   m_part, l_part [batch, heads_q, num_splits]      float32 (m/l/o format)
 *
 * Conventions shared by every entry point:
 *   - All pointers except the fd_choose_splits and workspace-size outputs
 *     are device pointers on the current HIP device.  q, k, v, o_part and
 *     workspace are 16-byte aligned; o, lse, lse_part, m_part, l_part,
 *     kv_lens and block_table 4-byte aligned (FD_ERR_UNSUPPORTED
 *     otherwise).  The caller owns every
 *     buffer; the library allocates no device memory and keeps no state
 *     besides a cached per-device compute-unit count.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is queued on it; no call synchronizes; a call returns after the
 *     launches are queued.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and fd_last_error() describes the problem.
 *   - Results are bitwise reproducible for fixed inputs, num_splits and
 *     split_len (no atomics, fixed reduction orders).
 *   - Accumulation is fp32 for every input dtype; outputs are rounded to
 *     nearest-even into out_dtype.
 *   - Supported: head_dim in {64, 128, 256}; in_dtype any FD_* code;
 *     out_dtype equal to in_dtype or FD_F32; heads_q % heads_kv == 0.
 */
#ifndef FD_H_
#define FD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define FD_F32 0
#define FD_F16 1
#define FD_BF16 2

/* Return codes. */
#define FD_OK 0
#define FD_ERR_INVALID (-1)     /* null pointer, bad size, heads_q % heads_kv, B*L < N */
#define FD_ERR_UNSUPPORTED (-2) /* head_dim, dtype or pointer alignment */
#define FD_ERR_WORKSPACE (-3)   /* workspace missing or too small */
#define FD_ERR_HIP (-4)         /* a HIP runtime call or a launch failed */

/* Library version as 10000*major + 100*minor + patch. */
int fd_version(void);

/* Message for the last non-FD_OK return on the calling thread ("" if none).
 * The pointer stays valid until the thread's next fd_* call. */
const char *fd_last_error(void);

/* Pick the split count B and split length L for a decode launch ([P2] §3 Q2
 * gives the rule of thumb this starts from: more splits for longer caches, up
 * to a cap; here the count is set so the launch fills the GPU's compute
 * units).  Host-only and deterministic.
 *   ragged:  nonzero when sequences may have different lengths (kv_lens is
 *            given); the split length is then shortened so that short and
 *            partial splits balance out.
 *   num_cus <= 0: query the current HIP device (cached); > 0: use as given.
 *   Outputs: *num_splits >= 1, *split_len >= 1, and
 *            (*num_splits) * (*split_len) >= max_kv_len.
 * Returns FD_OK, FD_ERR_INVALID (bad sizes or null outputs),
 * FD_ERR_UNSUPPORTED (head_dim or dtype) or FD_ERR_HIP. */
int fd_choose_splits(int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                     int in_dtype, int ragged, int num_cus, int *num_splits, int *split_len);

/* Bytes of workspace fd_decode needs for num_splits splits: o_part and
 * lse_part as laid out above, each starting on a 256-byte boundary.  Returns
 * 0 when num_splits <= 1 (fd_decode then writes o and lse directly) or on
 * non-positive sizes. */
size_t fd_workspace_bytes(int batch, int heads_q, int num_splits, int head_dim);

/* Bytes of workspace fd_decode needs when called with exactly these
 * arguments (has_kv_lens: nonzero when kv_lens will be non-NULL), including
 * the automatic plan of num_splits == 0 described at fd_decode.  Writes 0 when
 * no workspace is needed; equals fd_decode_plan's workspace_bytes for the
 * same arguments.  May query the current HIP device (compute units).
 * Returns FD_OK, FD_ERR_INVALID (bad sizes, null bytes), FD_ERR_UNSUPPORTED
 * (head_dim or dtype) or FD_ERR_HIP. */
int fd_decode_workspace_bytes(int batch, int heads_q, int heads_kv, int max_kv_len,
                              int head_dim, int in_dtype, int has_kv_lens, int num_splits,
                              int split_len, size_t *bytes);

/* Routes of a decode step (fd_plan.route). */
#define FD_ROUTE_DIRECT 0   /* one split per row: the split kernel writes o and lse */
#define FD_ROUTE_FUSED 1    /* 2..8 splits of a row in one work-group, merged in LDS */
#define FD_ROUTE_SPLITS 2   /* fixed splits into the workspace, then the combine */
#define FD_ROUTE_BALANCED 3 /* token-balanced pieces into the workspace, then the combine */

/* Split kernels (fd_plan.kernel). */
#define FD_KERNEL_VECTOR 0   /* vector ALUs (MHA, fp32; fp32 groups: up to eight query
                                heads of one KV head per work-group); on
                                FD_ROUTE_BALANCED it walks the token-balanced shares */
#define FD_KERNEL_GROUPED 1  /* matrix cores, one 16-query tile of a KV head's group */
#define FD_KERNEL_TILED 2    /* matrix cores, several 16-query tiles per K/V read */
#define FD_KERNEL_BALANCED 3 /* matrix cores over the token-balanced partition */

/* What fd_decode / fd_decode_paged launch for a set of arguments. */
typedef struct fd_plan {
    int route;           /* FD_ROUTE_* */
    int kernel;          /* FD_KERNEL_* */
    int num_splits;      /* B (0 on FD_ROUTE_BALANCED) */
    int split_len;       /* L (0 on FD_ROUTE_BALANCED) */
    int waves_per_group; /* wave64s per work-group of the split kernel */
    int query_tiles;     /* 16-query tiles per matrix-core work-group (0: vector kernel) */
    int launches;        /* kernel launches of the step: 1 or 2 */
    int64_t work_groups; /* grid size of the split kernel */
    size_t workspace_bytes; /* what fd_decode_workspace_bytes reports */
} fd_plan;

/* The plan fd_decode (paged == 0) or fd_decode_paged (paged != 0, max_kv_len
 * = max_pages_per_seq * page_size) follows for these arguments: the route,
 * the split kernel, B and L, and the workspace (the rules are at fd_decode).
 * has_kv_lens: nonzero when kv_lens will be non-NULL.  num_cus <= 0 queries
 * the current HIP device (cached); > 0 plans for that many compute units
 * without touching a device.  Host-only and deterministic.  Returns FD_OK,
 * FD_ERR_INVALID (bad sizes, B * L < max_kv_len, a paged split_len that is
 * not a multiple of 16, null plan), FD_ERR_UNSUPPORTED (head_dim or dtype)
 * or FD_ERR_HIP; the same arguments make fd_decode fail the same way. */
int fd_decode_plan(int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                   int in_dtype, int has_kv_lens, int paged, int num_splits, int split_len,
                   int num_cus, fd_plan *plan);

/* Split stage ([P1] §2.5 stage 1; [P3] §3.2.1 stage 1): for every
 * (b, h, split i) with token range [i*L, min((i+1)*L, N_b)) write
 *   o_part[b,h,i,:] = sum_j exp(s_j - m) V_j / l,
 *   lse_part[b,h,i] = m + log l      (m = max s_j, l = sum_j exp(s_j - m)),
 * and (0, -inf) for an empty range ([P3] §3.2.1 merge identity).
 * num_splits >= 1; split_len == 0 means L = ceil(max_kv_len / num_splits)
 * ([P2] §4 chunking), else split_len >= 1 with
 * num_splits * split_len >= max_kv_len. */
int fd_decode_split(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                    int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                    int in_dtype, float scale, int num_splits, int split_len, float *o_part,
                    float *lse_part, void *stream);

/* Split stage in the m/l/o format ([P1] §2.4.1 direct form; [P3] §2.2.1):
 * for every (b, h, split i) over the same token range as fd_decode_split,
 *   m_part[b,h,i] = m = max_j s_j             (natural-log domain, like lse)
 *   l_part[b,h,i] = l = sum_j exp(s_j - m)
 *   o_part[b,h,i,:] = sum_j exp(s_j - m) V_j / l,
 * and (o, m, l) = (0, -inf, 0) for an empty range.  m + log l equals what
 * fd_decode_split writes to lse_part.  Same arguments, conditions and errors
 * as fd_decode_split, with m_part and l_part in place of lse_part. */
int fd_decode_split_mlo(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                        int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                        int in_dtype, float scale, int num_splits, int split_len, float *o_part,
                        float *m_part, float *l_part, void *stream);

/* Combine stage ([P3] §2.3.4; [P1] §2.5 stage 2, a light reduction):
 *   S = log sum_i exp(lse_part[b,h,i]),  o[b,h,:] = sum_i exp(lse_part[b,h,i] - S) o_part[b,h,i,:]
 * Terms at -inf contribute nothing; if every term is -inf, o = 0 and S = -inf.
 * lse may be NULL.  num_splits >= 1. */
int fd_combine(const float *o_part, const float *lse_part, int batch, int heads_q,
               int num_splits, int head_dim, void *o, int out_dtype, float *lse, void *stream);

/* Combine stage for the m/l/o format ([P1] §2.4.2 and §2.5 stage 2; [P3]
 * §2.2.2):
 *   m_g = max_i m_part[b,h,i],  l_g = sum_i exp(m_part[b,h,i] - m_g) l_part[b,h,i],
 *   o[b,h,:] = sum_i exp(m_part[b,h,i] - m_g) l_part[b,h,i] o_part[b,h,i,:] / l_g,
 *   lse[b,h] = m_g + log l_g (may be NULL).
 * Splits with m = -inf contribute nothing; if every split is empty, o = 0
 * and lse = -inf.  Same conditions and errors as fd_combine. */
int fd_combine_mlo(const float *o_part, const float *m_part, const float *l_part, int batch,
                   int heads_q, int num_splits, int head_dim, void *o, int out_dtype, float *lse,
                   void *stream);

/* Whole decode step: split + combine.
 *   num_splits == 0 (automatic plan, split_len ignored):
 *     - kv_lens given and grouped heads on the matrix cores (bf16/f16,
 *       2 <= heads_q/heads_kv <= 128, 128, 64 at head_dim 64, 128, 256): a
 *       token-balanced partition.  The
 *       (KV head, sequence, token) space of the actual lengths is cut into
 *       equal shares, one per work-group (CUs x 2, or CUs x 1 for the
 *       larger groups whose work-groups have four or eight waves), so every
 *       work-group
 *       streams the same number of K/V rows whatever the length mix; a share
 *       may end inside one (sequence, head) row and continue in the next, and
 *       each such piece yields one (o, LSE) pair that the combine merges with
 *       the row's other pieces ([P3] §2.3.4; any cut gives the same result,
 *       [P3] §2.3.5).  The split points depend on the lengths, so results
 *       agree with a fixed-split run up to rounding, and are reproducible
 *       for fixed inputs.
 *     - kv_lens given and heads the vector kernel serves (one query head per
 *       KV head in bf16/f16, or fp32 with any group): the same partition
 *       with one unit per (sequence, query head) instead of (sequence, KV
 *       head), on one-wave work-groups (CUs x 2).
 *     - otherwise: B and L from fd_choose_splits (ragged = kv_lens != NULL).
 *   num_splits > 0, split_len == 0: L = ceil(max_kv_len / num_splits)
 *     ([P2] §4 chunking).  num_splits > 0, split_len > 0: used as given.
 * Grouped heads in bf16/f16 run on the matrix cores: up to 16 query heads per
 * KV head in one tile, larger groups (up to multi-query attention) in tiles
 * of 16 that read each K/V row once for all of them.
 * With B == 1 the split stage writes o and lse itself.  On the vector path
 * (fp32 inputs, or no grouped heads) a small grid with 2 <= B <= 8 splits
 * (batch * heads_q * B below two waves per CU) runs every split of a row in
 * one work-group, one wave per split, and merges the splits in LDS: again a
 * single launch that writes o and lse.  Otherwise workspace must hold the
 * bytes fd_decode_workspace_bytes reports for the same arguments (0 in the
 * cases above, where workspace may be NULL; for other explicit B it is
 * fd_workspace_bytes(batch, heads_q, B, head_dim)).  lse may be NULL. */
int fd_decode(const void *q, const void *k, const void *v, const int32_t *kv_lens, int batch,
              int heads_q, int heads_kv, int max_kv_len, int head_dim, int in_dtype,
              int out_dtype, float scale, int num_splits, int split_len, void *o, float *lse,
              void *workspace, size_t workspace_bytes, void *stream);

/* The two launches of fd_decode, one call each ([P1] §2.5: stage 1 writes
 * the splits' partial results to a temporary buffer, stage 2 reduces them;
 * [P2] §5 names the same split -> temporary buffer -> reduce structure).
 * stages = FD_STAGE_SPLIT queues only the split launch, FD_STAGE_COMBINE only
 * the combine launch, both bits the whole step (= fd_decode).  A combine
 * call must follow a split call with the same arguments and workspace on the
 * same stream (or after it has completed); in between the workspace holds
 * the partial results in the plan's internal layout.  On the single-launch
 * routes (FD_ROUTE_DIRECT, FD_ROUTE_FUSED) the split call writes o and lse
 * and the combine call queues nothing.  Arguments and errors as fd_decode,
 * plus FD_ERR_INVALID for stages outside {1, 2, 3}.  Lets a caller time or
 * schedule the two kernels separately. */
#define FD_STAGE_SPLIT 1
#define FD_STAGE_COMBINE 2
int fd_decode_stages(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                     int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                     int in_dtype, int out_dtype, float scale, int num_splits, int split_len,
                     void *o, float *lse, void *workspace, size_t workspace_bytes, int stages,
                     void *stream);

/* fd_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, plan, kernels and results as fd_decode, without the
 * workspace arguments.  The partial results go to a scratch buffer the
 * library owns: 32 MiB of device memory per GPU, a file-scope device array
 * each GPU holds from the first such call until the process ends.  Steps
 * whose plan needs more (fd_decode_workspace_bytes > 32 MiB) are refused
 * with FD_ERR_WORKSPACE before anything is launched.  No call allocates or
 * frees memory.  Every call on one GPU shares that GPU's buffer: calls that
 * overlap on one GPU (other host threads, other streams) race, so callers
 * serialise them (one stream, or their own ordering).  Nothing in the buffer
 * needs clearing between calls. */
int fd_decode_noalloc(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                      int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                      int in_dtype, int out_dtype, float scale, int num_splits, int split_len,
                      void *o, float *lse, void *stream);

/* Paged K/V cache ([P2] §5: the kernel follows a block table over
 * non-contiguous pages instead of gathering them first; [P4] §7.1: the page
 * offsets cost an index lookup).  Same operation as fd_decode_split /
 * fd_decode, with K and V in pages:
 *   k_pages, v_pages [num_pages, page_size, heads_kv, head_dim]  in_dtype
 *   block_table      [batch, max_pages_per_seq] int32 (device): token t of
 *                    sequence b is row t % page_size of page
 *                    block_table[b][t / page_size].
 *   kv_lens          as above, clamped to [0, max_pages_per_seq * page_size];
 *                    NULL: every sequence has max_pages_per_seq * page_size.
 * page_size is a power of two in [16, 2^20] (a 16-token tile never straddles
 * two pages); one page is at most 2 GiB.  Only the first ceil(N_b /
 * page_size) entries of a table row are read; an entry outside
 * [0, num_pages) is clamped into it (memory stays in bounds, that sequence's
 * result is then meaningless).  split_len must be a multiple of 16 (the
 * automatic plan's is; given num_splits > 0 and split_len == 0, both paged
 * calls round ceil(N / num_splits) up to one).  Workspace: fd_decode_workspace_bytes with max_kv_len
 * = max_pages_per_seq * page_size.  Extra errors: FD_ERR_INVALID for a null
 * block_table, max_pages_per_seq or num_pages < 1, or split_len % 16 != 0;
 * FD_ERR_UNSUPPORTED for page_size or page bytes out of range. */
int fd_decode_split_paged(const void *q, const void *k_pages, const void *v_pages,
                          const int32_t *block_table, const int32_t *kv_lens, int batch,
                          int heads_q, int heads_kv, int page_size, int max_pages_per_seq,
                          int num_pages, int head_dim, int in_dtype, float scale, int num_splits,
                          int split_len, float *o_part, float *lse_part, void *stream);

int fd_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                    const int32_t *block_table, const int32_t *kv_lens, int batch, int heads_q,
                    int heads_kv, int page_size, int max_pages_per_seq, int num_pages,
                    int head_dim, int in_dtype, int out_dtype, float scale, int num_splits,
                    int split_len, void *o, float *lse, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Cascade (shared-prefix) decode ([P2] §5: the KV cache is handled in two
 * layers, a stable prefix shared across requests and a per-request dynamic
 * suffix).  Every sequence b attends over its prefix-then-suffix cache
 *   [k_prefix[0 .. prefix_len), k_suffix[b][0 .. N_b)]
 * and the result equals fd_decode over that concatenation: the prefix and
 * the suffix are cut into fixed splits (one shared prefix copy, read by every
 * sequence; B_p and B_s from fd_choose_splits, the suffix as ragged when
 * suffix_lens is given), both stages write (o, LSE) pairs into one partial
 * buffer of B_p + B_s splits per row, and fd_combine's kernel merges them
 * ([P3] §2.3.4; the merge is order- and cut-independent, [P3] §2.3.5).
 *   k_prefix, v_prefix [prefix_len, heads_kv, head_dim]            in_dtype
 *   k_suffix, v_suffix [batch, max_suffix_len, heads_kv, head_dim] in_dtype
 *   suffix_lens        [batch] int32 (device) or NULL (all max_suffix_len),
 *                      clamped to [0, max_suffix_len].
 * prefix_len and max_suffix_len may be 0 (then the pointers may be NULL).
 * The workspace must hold fd_cascade_workspace_bytes(...) bytes.  Errors as
 * fd_decode. */
int fd_cascade_workspace_bytes(int batch, int heads_q, int heads_kv, int prefix_len,
                               int max_suffix_len, int head_dim, int in_dtype,
                               int has_suffix_lens, size_t *bytes);

int fd_decode_cascade(const void *q, const void *k_prefix, const void *v_prefix, int prefix_len,
                      const void *k_suffix, const void *v_suffix, const int32_t *suffix_lens,
                      int batch, int heads_q, int heads_kv, int max_suffix_len, int head_dim,
                      int in_dtype, int out_dtype, float scale, void *o, float *lse,
                      void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FD_H_ */
