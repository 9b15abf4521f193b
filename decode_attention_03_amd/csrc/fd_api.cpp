// fd_api.cpp -- the C ABI of libfd: argument validation, the split-count
// heuristic, workspace carving and kernel dispatch.  Host code only; every
// step of the computation runs in the HIP kernels of this library.
//
// Sources (pages; sections as printed on them):
//   [P1] "FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15)
//   [P2] "adv04: Flash-Decoding（长序列 Decode 切分 + FlashInfer 简介）"
//        (mini-vllm-tutorial.vercel.app)
//   [P3] "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
//        (my-webpage-adu.pages.dev, 2026-07-16)
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "fd.h"
#include "fd_internal.h"

namespace {

constexpr int kVersion = 200;          // 0.2.0
constexpr int kMaxSplits = 8192;       // combine keeps one weight per split in LDS
constexpr int kRaggedRounds = 4;       // work-group rounds aimed at for ragged batches
constexpr int kMinSplitLenMha = 256;   // tokens; partial traffic ~0.8% of K/V at d = 128
constexpr int kMinSplitLenPerHead = 64;  // grouped: tokens per query head of the group
// Groups past one tile: at least this many tokens per query head, so that a
// split's partials (written and read back: G (d + 1) 4-byte values twice) stay
// within about a quarter of its K/V bytes; a long floor would leave these
// small-K/V, many-query shapes with too few work-groups.
constexpr int kMinSplitLenPerHeadTiled = 8;
constexpr int kMaxAutoSplits = 512;
constexpr int kBalancedRounds = 1;     // token-balanced work-groups: CUs * per-CU * rounds
// When those floors would leave the GPU's work-group slots partly empty
// (small batches), splits may shrink to this many tokens per query head of
// the group (at least kMinSplitLenFill), up to one round of work-groups: more
// partial traffic (a few percent of the K/V bytes) against idle CUs, which
// cost far more (FD_SPLIT_FILL 0 keeps the floors).
#ifndef FD_SPLIT_FILL
#define FD_SPLIT_FILL 1
#endif
constexpr int kMinSplitLenPerHeadFill = 16;
constexpr int kMinSplitLenFill = 64;
// Split counts for equal lengths are chosen by rounds of work-groups
// (FD_SPLIT_ROUNDS 0: the first count that fills the slots); a work-group's
// fixed cost (first loads, partial write, the spread of a round's finish
// times), as the K/V bytes it could have streamed meanwhile.
#ifndef FD_SPLIT_ROUNDS
#define FD_SPLIT_ROUNDS 1
#endif
constexpr long long kWgFixedBytes = 64 << 10;

thread_local std::string g_error;

#if FD_WG_CLOCKS
// Instrumented builds: the stamp buffer the token-balanced kernel writes
// (fd_debug_wg_clocks); used while it holds four words per work-group.
unsigned long long *g_wg_clock = nullptr;
size_t g_wg_clock_bytes = 0;
#endif

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dtype_ok(int dt) { return dt == FD_F32 || dt == FD_F16 || dt == FD_BF16; }
bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
size_t elem_bytes(int dt) { return dt == FD_F32 ? 4 : 2; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

std::mutex g_cu_mutex;
int g_cu_cache[64];  // 0 = not queried yet

int device_cus(int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (dev >= 0 && dev < 64 && g_cu_cache[dev] > 0) {
        *out = g_cu_cache[dev];
        return FD_OK;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0)
        return fail(FD_ERR_HIP, "hipDeviceGetAttribute(compute units): %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64)
        g_cu_cache[dev] = n;
    *out = n;
    return FD_OK;
}

// Checks shared by the split stage and the whole decode.
int check_split_inputs(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                       int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                       int in_dtype, float scale) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || max_kv_len < 0)
        return fail(FD_ERR_INVALID, "sizes must be positive (batch=%d heads_q=%d heads_kv=%d "
                    "max_kv_len=%d)", batch, heads_q, heads_kv, max_kv_len);
    if (heads_q % heads_kv != 0)
        return fail(FD_ERR_INVALID, "heads_q (%d) is not a multiple of heads_kv (%d)", heads_q,
                    heads_kv);
    if (!q)
        return fail(FD_ERR_INVALID, "q is null");
    if (max_kv_len > 0 && (!k || !v))
        return fail(FD_ERR_INVALID, "k or v is null");
    if (!head_dim_ok(head_dim))
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128, 256)", head_dim);
    if (!dtype_ok(in_dtype))
        return fail(FD_ERR_UNSUPPORTED, "in_dtype %d not supported", in_dtype);
    if (!aligned16(q) || (max_kv_len > 0 && (!aligned16(k) || !aligned16(v))))
        return fail(FD_ERR_UNSUPPORTED, "q, k and v must be 16-byte aligned");
    if (kv_lens && !aligned4(kv_lens))
        return fail(FD_ERR_UNSUPPORTED, "kv_lens must be 4-byte aligned");
    if (!std::isfinite(scale))
        return fail(FD_ERR_INVALID, "scale is not finite");
    // the kernels address K/V with 32-bit offsets from a per-split base
    if ((size_t)heads_kv * head_dim * elem_bytes(in_dtype) > ((size_t)1 << 24))
        return fail(FD_ERR_UNSUPPORTED, "one token's K row over all heads exceeds 16 MiB");
    return FD_OK;
}

// split_len 0 with num_splits > 0: ceil(max_kv_len / num_splits) tokens per
// split ("adv04: Flash-Decoding" §4 chunking), in whole 16-token tiles for a
// paged cache (a tile must not straddle two pages).
int resolve_split_len(int max_kv_len, int num_splits, int split_len, bool paged) {
    if (num_splits < 1 || split_len != 0)
        return split_len;
    long long len = max_kv_len > 0 ? ((long long)max_kv_len + num_splits - 1) / num_splits : 1;
    if (paged)
        len = (len + 15) / 16 * 16;
    return (int)(len < 0x7fffffffLL ? len : 0x7ffffff0LL);
}

int check_partition(int batch, int heads_q, int max_kv_len, int num_splits, int split_len) {
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FD_ERR_INVALID, "num_splits %d outside [1, %d]", num_splits, kMaxSplits);
    if (split_len < 1)
        return fail(FD_ERR_INVALID, "split_len %d < 1", split_len);
    if ((long long)num_splits * split_len < max_kv_len)
        return fail(FD_ERR_INVALID, "num_splits * split_len (%lld) < max_kv_len (%d)",
                    (long long)num_splits * split_len, max_kv_len);
    if ((long long)batch * heads_q * num_splits > 0x7fffffffLL)
        return fail(FD_ERR_INVALID, "batch * heads_q * num_splits exceeds the launch limit");
    return FD_OK;
}

// Paged K/V description, validated by check_paging.
struct Paging {
    const int32_t *block_table = nullptr;
    int page_shift = 0, max_pages = 0, num_pages = 0;
};

int check_paging(const int32_t *block_table, int page_size, int max_pages, int num_pages,
                 int heads_kv, int head_dim, int in_dtype, Paging *pg) {
    if (!block_table)
        return fail(FD_ERR_INVALID, "block_table is null");
    if (!aligned4(block_table))
        return fail(FD_ERR_UNSUPPORTED, "block_table must be 4-byte aligned");
    if (max_pages < 1 || num_pages < 1)
        return fail(FD_ERR_INVALID, "max_pages_per_seq (%d) and num_pages (%d) must be >= 1",
                    max_pages, num_pages);
    if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)))
        return fail(FD_ERR_UNSUPPORTED, "page_size %d must be a power of two in [16, 2^20]",
                    page_size);
    if ((long long)max_pages * page_size > 0x7fffffffLL)
        return fail(FD_ERR_INVALID, "max_pages_per_seq * page_size exceeds the int range");
    if (heads_kv >= 1 && head_dim_ok(head_dim) && dtype_ok(in_dtype) &&
        (long long)page_size * heads_kv * head_dim * (long long)elem_bytes(in_dtype) >
            (1LL << 31))
        return fail(FD_ERR_UNSUPPORTED, "one page exceeds 2 GiB");
    pg->block_table = block_table;
    pg->page_shift = __builtin_ctz((unsigned)page_size);
    pg->max_pages = max_pages;
    pg->num_pages = num_pages;
    return FD_OK;
}

void set_paging(fd::SplitArgs &a, const Paging *pg) {
    if (!pg)
        return;
    a.block_table = pg->block_table;
    a.page_shift = pg->page_shift;
    a.max_pages = pg->max_pages;
    a.num_pages = pg->num_pages;
}

// Groups of more than one matrix-core tile of query heads (bf16/f16): the
// tiled kernel, which reads each K/V row once for all of them.
bool large_group(int in_dtype, int head_dim, int group) {
    return group >= 2 && !fd::split_mfma_supported(in_dtype, head_dim, group) &&
           fd::split_mfma_tiled_supported(in_dtype, head_dim);
}

// Ragged batches whose heads the vector kernel serves (one query head per KV
// head, or fp32) take the token-balanced partition on it, one unit per
// (sequence, query head).
#ifndef FD_VALU_BALANCED
#define FD_VALU_BALANCED 1
#endif
bool balanced_vector(int in_dtype, int head_dim, int group) {
    return FD_VALU_BALANCED && !fd::split_mfma_supported(in_dtype, head_dim, group) &&
           !large_group(in_dtype, head_dim, group);
}

// Shape of the tiled kernel's work-groups for nq queries per KV head: qt
// query tiles per wave (the most a wave holds, but no more than there are
// tiles) and, past what one wave holds, several waves per work-group sharing
// each staged K/V step (up to the most the head size allows), so that the
// work-groups of a unit read its rows as few times as possible; groups is
// the number of work-groups per unit.
struct TiledShape {
    int qt = 1, waves = 1;
    long long groups = 1;
    bool pair = false;  // 5..8 tiles on several smaller work-groups of one tile per wave
    int per_cu() const { return fd::split_mfma_tiled_wg_per_cu(waves, pair); }
};

TiledShape tiled_shape(int head_dim, long long nq) {
    TiledShape t;
    const long long tiles = (nq + 15) / 16;
    const int wmax = fd::split_mfma_tile_max_waves(head_dim);
    if (fd::split_mfma_tile_spread() && tiles > 1 && tiles <= wmax) {
        t.qt = 1;  // one tile on each of the waves
        while (t.waves < tiles)
            t.waves *= 2;
        constexpr int pw = fd::tiled_pair_waves();
        if (t.waves == 8 && pw > 0 && fd::tiled_pair(head_dim, 1, pw, 2)) {
            t.waves = pw;  // several smaller work-groups per unit
            t.groups = (tiles + pw - 1) / pw;
            t.pair = true;
        }
        return t;
    }
    t.qt = fd::split_mfma_tile_max_qt(head_dim);
    while (t.qt > 1 && t.qt / 2 >= tiles)
        t.qt /= 2;
    if (tiles > t.qt) {  // several waves, each with at most wide_qt tiles
        const int wq = fd::split_mfma_wide_qt(head_dim);
        t.qt = t.qt < wq ? t.qt : wq;
    }
    const int wcap = wmax < 4 ? wmax : 4;  // more than four waves hold one tile each
    while (t.waves < wcap && (long long)t.qt * t.waves < tiles)
        t.waves *= 2;
    t.groups = (tiles + (long long)t.qt * t.waves - 1) / ((long long)t.qt * t.waves);
    return t;
}

// Waves per work-group when the vector kernel runs every split of a row in one
// work-group and merges them in LDS (no combine launch, no workspace): fixed
// splits, 2..8 of them, on a grid whose split work-groups would not even fill
// the GPU's wave slots once.  0 when not applicable.
int fused_waves(int batch, int heads_q, int heads_kv, int head_dim, int in_dtype,
                int num_splits, int cus) {
    if (num_splits < 2 || num_splits > 8 ||
        fd::split_mfma_supported(in_dtype, head_dim, heads_q / heads_kv) ||
        large_group(in_dtype, head_dim, heads_q / heads_kv))
        return 0;
    if ((long long)batch * heads_q * num_splits >= (long long)cus * fd::kWavesPerCU)
        return 0;
    return num_splits <= 2 ? 2 : (num_splits <= 4 ? 4 : 8);
}

// Which split kernel a launch described by a runs (FD_KERNEL_*).
int split_kernel(const fd::SplitArgs &a, int in_dtype) {
    const int group = a.heads_q / a.heads_kv;
    if (a.balanced)
        return balanced_vector(in_dtype, a.head_dim, group) ? FD_KERNEL_VECTOR
                                                            : FD_KERNEL_BALANCED;
    if (a.tile_qt > 0 || large_group(in_dtype, a.head_dim, group))
        return FD_KERNEL_TILED;
    if (fd::split_mfma_supported(in_dtype, a.head_dim, group))
        return FD_KERNEL_GROUPED;
    return FD_KERNEL_VECTOR;
}

// Waves per vector-kernel work-group: the fused small-grid count, else two
// when one-wave work-groups would leave wave slots of the GPU empty, else one.
int vector_waves(const fd::SplitArgs &a, int in_dtype, int cus) {
    if (a.fused_waves > 0)
        return a.fused_waves;
    // two-wave work-groups only where they all fit in the wave slots at once
    // (a work-group takes valu_heads_per_wg query heads)
    const long long wgs = (long long)a.batch * a.heads_q * a.num_splits /
                          fd::valu_heads_per_wg(in_dtype, a.head_dim, a.heads_q / a.heads_kv);
    return wgs <= cus ? fd::kWavesPerCU : 1;  // kWavesPerCU waves each on at most one per CU
}

int launch_split(fd::SplitArgs a, int in_dtype, hipStream_t stream) {
    hipError_t e;
    switch (split_kernel(a, in_dtype)) {
    case FD_KERNEL_TILED:
        if (a.tile_qt == 0) {
            const TiledShape t = tiled_shape(a.head_dim, a.heads_q / a.heads_kv);
            a.tile_qt = t.qt;
            a.tile_waves = t.waves;
        }
        e = fd::launch_split_mfma(a, in_dtype, stream);
        break;
    case FD_KERNEL_GROUPED:
    case FD_KERNEL_BALANCED:
        e = fd::launch_split_mfma(a, in_dtype, stream);
        break;
    default: {
        int cus = 0;
        int rc = device_cus(&cus);
        if (rc != FD_OK)
            return rc;
        a.valu_waves = a.fused_waves > 0 || a.balanced ? 0 : vector_waves(a, in_dtype, cus);
        e = fd::launch_split_valu(a, in_dtype, stream);
    }
    }
    if (e != hipSuccess)
        return fail(FD_ERR_HIP, "split kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

// Token-balanced partition of a ragged batch (partition.h): used by
// fd_decode's automatic plan when kv_lens is given and the grouped kernel
// applies, or (FD_VALU_BALANCED) the vector kernel would run.  Workspace: o
// slots, LSE slots, unit descriptors, each 256-aligned.
struct BalancedPlan {
    int num_wgs = 0, units = 0, gsz = 0;
    int waves = 1;  // per work-group (fd::split_mfma_balanced_waves)
    bool vector = false;  // vector kernel: units (b, query-head group), gsz heads each
    size_t o_bytes = 0, lse_bytes = 0, desc_bytes = 0;
    size_t total() const { return o_bytes + lse_bytes + desc_bytes; }
};

bool balanced_applies(int heads_q, int heads_kv, int max_kv_len, int head_dim, int in_dtype,
                      bool has_lens, int num_splits) {
    const int group = heads_q / heads_kv;
    return num_splits == 0 && has_lens && max_kv_len > 0 &&
           (fd::split_mfma_supported(in_dtype, head_dim, group) ||
            (large_group(in_dtype, head_dim, group) &&
             group <= fd::split_mfma_balanced_max_group(head_dim)) ||
            balanced_vector(in_dtype, head_dim, group));
}

int balanced_plan(int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                  int in_dtype, int cus, BalancedPlan *p) {
    // slot indices (work-group + unit rank) and the combine's row grid
    // (batch * heads_q) are 32-bit in the kernels
    p->vector = balanced_vector(in_dtype, head_dim, heads_q / heads_kv);
    // vector kernel: one unit per (sequence, group of valu_heads_per_wg query
    // heads), one-wave work-groups at valu_wg_per_cu per CU; matrix cores:
    // one per (sequence, KV head)
    const int hpw = fd::valu_heads_per_wg(in_dtype, head_dim, heads_q / heads_kv);
    const long long units = (long long)batch * (p->vector ? heads_q / hpw : heads_kv);
    p->gsz = p->vector ? hpw : heads_q / heads_kv;
    p->waves = p->vector ? 1 : fd::split_mfma_balanced_waves(head_dim, p->gsz);
    if (p->waves < 1)
        return fail(FD_ERR_INVALID, "group of %d too large for the balanced plan", p->gsz);
    const long long wgs =
        (long long)cus *
        (p->vector ? fd::valu_wg_per_cu(hpw) : fd::split_mfma_balanced_wg_per_cu(head_dim, p->gsz)) *
        kBalancedRounds;
    if (units + wgs > 0x7fffffffLL || (long long)batch * heads_q > 0x7fffffffLL)
        return fail(FD_ERR_INVALID, "batch * heads exceeds the launch limit of the balanced plan");
    p->units = (int)units;
    p->num_wgs = (int)wgs;
    // positions (units * max_kv_len) times work-groups must stay within int64
    if ((double)p->units * max_kv_len * p->num_wgs > 4.0e18)
        return fail(FD_ERR_INVALID, "batch * heads_kv * max_kv_len too large for the balanced plan");
    const size_t slots = (size_t)p->num_wgs + p->units;
    p->o_bytes = round256(slots * p->gsz * head_dim * sizeof(float));
    p->lse_bytes = round256(slots * p->gsz * sizeof(float));
    p->desc_bytes = round256((size_t)p->units * 2 * sizeof(int));
    return FD_OK;
}

// The plan of one decode step (fd_decode / fd_decode_paged): the single place
// where the route, the split kernel, B and L and the workspace are decided.
// fd_decode_plan reports it, fd_decode_workspace_bytes its workspace, and
// decode_impl carries it out.
struct Plan {
    fd_plan pub{};
    int fused = 0;  // vector-kernel waves per row on FD_ROUTE_FUSED
    BalancedPlan bal;
};

int make_plan(int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim, int in_dtype,
              bool has_lens, bool paged, int num_splits, int split_len, int cus, Plan *p) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || max_kv_len < 0 || heads_q % heads_kv)
        return fail(FD_ERR_INVALID, "bad sizes (batch=%d heads_q=%d heads_kv=%d max_kv_len=%d)",
                    batch, heads_q, heads_kv, max_kv_len);
    if (!head_dim_ok(head_dim) || !dtype_ok(in_dtype))
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d / dtype %d not supported", head_dim,
                    in_dtype);
    if (num_splits < 0 || split_len < 0)
        return fail(FD_ERR_INVALID, "num_splits (%d) and split_len (%d) must be >= 0",
                    num_splits, split_len);
    // explicit splits: checked before the device is asked for anything
    if (num_splits > 0) {
        split_len = resolve_split_len(max_kv_len, num_splits, split_len, paged);
        int rc = check_partition(batch, heads_q, max_kv_len, num_splits, split_len);
        if (rc != FD_OK)
            return rc;
        if (paged && split_len % 16 != 0)
            return fail(FD_ERR_INVALID, "paged K/V needs split_len (%d) to be a multiple of 16",
                        split_len);
    }
    // the device's compute units, asked for only where a decision needs them
    auto need_cus = [&cus]() { return cus > 0 ? FD_OK : device_cus(&cus); };
    *p = Plan{};
    fd_plan &r = p->pub;
    fd::SplitArgs a{};
    a.batch = batch;
    a.heads_q = heads_q;
    a.heads_kv = heads_kv;
    a.max_kv_len = max_kv_len;
    a.head_dim = head_dim;
    const int group = heads_q / heads_kv;
    int rc;
    if (balanced_applies(heads_q, heads_kv, max_kv_len, head_dim, in_dtype, has_lens,
                         num_splits)) {
        if ((rc = need_cus()) != FD_OK ||
            (rc = balanced_plan(batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype, cus,
                               &p->bal)) !=
                FD_OK)
            return rc;
        r.route = FD_ROUTE_BALANCED;
        r.kernel = p->bal.vector ? FD_KERNEL_VECTOR : FD_KERNEL_BALANCED;
        r.work_groups = p->bal.num_wgs;
        r.waves_per_group = p->bal.waves;
        r.query_tiles = p->bal.vector ? 0 : (group + 15) / 16;
        r.launches = 2;
        r.workspace_bytes = p->bal.total();
        return FD_OK;
    }
    if (num_splits == 0) {  // the automatic plan: whole 16-token tiles, B * L >= max_kv_len
        if ((rc = need_cus()) != FD_OK ||
            (rc = fd_choose_splits(batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                                   has_lens, cus, &num_splits, &split_len)) != FD_OK ||
            (rc = check_partition(batch, heads_q, max_kv_len, num_splits, split_len)) != FD_OK)
            return rc;
    }
    a.num_splits = num_splits;
    a.split_len = split_len;
    r.num_splits = num_splits;
    r.split_len = split_len;
    r.kernel = split_kernel(a, in_dtype);
    switch (r.kernel) {
    case FD_KERNEL_VECTOR:
        if ((rc = need_cus()) != FD_OK)
            return rc;
        p->fused = num_splits > 1 ? fused_waves(batch, heads_q, heads_kv, head_dim, in_dtype,
                                                num_splits, cus)
                                  : 0;
        a.fused_waves = p->fused;
        r.waves_per_group = vector_waves(a, in_dtype, cus);
        r.query_tiles = 0;
        r.work_groups = p->fused > 0 ? (int64_t)batch * heads_q
                                     : (int64_t)batch * heads_q * num_splits /
                                           fd::valu_heads_per_wg(in_dtype, head_dim, group);
        break;
    case FD_KERNEL_GROUPED:
        r.waves_per_group = 1;
        r.query_tiles = 1;
        r.work_groups = (int64_t)batch * heads_kv * num_splits;
        break;
    default: {  // FD_KERNEL_TILED: units padded to multiples of 8, times tile groups
        const TiledShape t = tiled_shape(head_dim, group);
        const long long units = (long long)batch * heads_kv * num_splits;
        r.waves_per_group = t.waves;
        r.query_tiles = t.qt * t.waves;
        r.work_groups = (units + 7) / 8 * 8 * t.groups;
    }
    }
    r.route = num_splits == 1 ? FD_ROUTE_DIRECT : (p->fused > 0 ? FD_ROUTE_FUSED : FD_ROUTE_SPLITS);
    r.launches = r.route == FD_ROUTE_SPLITS ? 2 : 1;
    r.workspace_bytes =
        r.route == FD_ROUTE_SPLITS ? fd_workspace_bytes(batch, heads_q, num_splits, head_dim) : 0;
    return FD_OK;
}

}  // namespace

extern "C" {

int fd_version(void) { return kVersion; }

const char *fd_last_error(void) { return g_error.c_str(); }

// Split count: [P2] §3 Q2 suggests roughly one split per 1K tokens, capped,
// and notes that the best count depends on the GPU.  Here it is derived from
// the GPU: the split kernels run one-wave work-groups (two-wave ones where the
// grid is small), with a fixed number resident per CU (the request depth at
// which MI355X HBM streams best: fd::kWavesPerCU for the vector kernel,
// fd::kMfmaWgPerCU for the grouped one), and a work-group costs a start-up
// latency, so
//   - equal lengths: one full round, batch * units * B ~ CUs * per-CU count;
//     a vector-kernel plan of two splits becomes one split per row run by
//     two-wave work-groups (same wave slots, no combine stage);
//   - ragged lengths (unknown to the host): about kRaggedRounds rounds judged
//     by the longest sequence, so that the short and partial splits even out;
// never with splits shorter than a floor that keeps the partial (o, LSE)
// traffic small next to the K/V bytes.
int fd_choose_splits(int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                     int in_dtype, int ragged, int num_cus, int *num_splits, int *split_len) {
    if (!num_splits || !split_len)
        return fail(FD_ERR_INVALID, "null output pointer");
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || max_kv_len < 0 || heads_q % heads_kv)
        return fail(FD_ERR_INVALID, "bad sizes (batch=%d heads_q=%d heads_kv=%d max_kv_len=%d)",
                    batch, heads_q, heads_kv, max_kv_len);
    if (!head_dim_ok(head_dim) || !dtype_ok(in_dtype))
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d / dtype %d not supported", head_dim,
                    in_dtype);
    if (num_cus <= 0) {
        int rc = device_cus(&num_cus);
        if (rc != FD_OK)
            return rc;
    }
    if (max_kv_len == 0) {
        *num_splits = 1;
        *split_len = 1;
        return FD_OK;
    }
    const int group = heads_q / heads_kv;
    const bool grouped = fd::split_mfma_supported(in_dtype, head_dim, group);
    const bool tiled = large_group(in_dtype, head_dim, group);
    // work-groups per split index: one per (sequence, KV head) when a group is
    // computed together, one per (sequence, KV head, tile group) when it takes
    // several tiles, else one per (sequence, query head)
    long long units = (long long)batch * (grouped ? heads_kv : heads_q);
    if (!grouped)  // vector kernel: valu_heads_per_wg query heads per work-group
        units /= fd::valu_heads_per_wg(in_dtype, head_dim, group);
    int per_cu = grouped ? fd::kMfmaWgPerCU
                         : fd::valu_wg_per_cu(fd::valu_heads_per_wg(in_dtype, head_dim, group));
    if (tiled) {
        const TiledShape t = tiled_shape(head_dim, group);
        units = (long long)batch * heads_kv * t.groups;
        per_cu = t.per_cu();
    }
    const long long target = (long long)num_cus * per_cu * (ragged ? kRaggedRounds : 1);
    long long b = (target + units - 1) / units;
    long long min_len = grouped ? kMinSplitLenPerHead * group : kMinSplitLenMha;
    if (tiled && (long long)kMinSplitLenPerHeadTiled * group > min_len)
        min_len = (long long)kMinSplitLenPerHeadTiled * group;
    long long bmax = (max_kv_len + min_len - 1) / min_len;
    if (bmax < 1)
        bmax = 1;
    if (FD_SPLIT_FILL && b > bmax && !tiled) {
        // the floor would leave work-group slots empty: let the splits shrink
        // towards the fill floor, up to what fills the slots once
        long long fill_len = (long long)kMinSplitLenPerHeadFill * (grouped ? group : 1);
        fill_len = fill_len > kMinSplitLenFill ? fill_len : kMinSplitLenFill;
        fill_len = fill_len < min_len ? fill_len : min_len;
        const long long once = ((long long)num_cus * per_cu + units - 1) / units;
        long long bfill = (max_kv_len + fill_len - 1) / fill_len;
        bfill = bfill < once ? bfill : once;
        bmax = bfill > bmax ? bfill : bmax;
    }
    if (b > bmax)
        b = bmax;
    if (b > kMaxAutoSplits)
        b = kMaxAutoSplits;
    if (b < 1)
        b = 1;
    if (FD_SPLIT_ROUNDS && !ragged) {
        // Equal lengths: every work-group streams the same rows, so the launch
        // takes rounds(B) = ceil(units * B / slots) times one split's time.  A
        // count just past a multiple of the slots leaves a mostly idle last
        // round (16 sequences x 6 KV heads x 6 splits = 576 work-groups on 512
        // slots ran twice as long as 480).  Take the count that minimises
        // rounds x (split length + a work-group's fixed cost), and among counts
        // within 1 % of that the fewest splits (fewer partials to merge).
        const long long slots = (long long)num_cus * per_cu;
        const long long hi = bmax < kMaxAutoSplits ? bmax : kMaxAutoSplits;
        const long long row = 2LL * head_dim * (in_dtype == FD_F32 ? 4 : 2);  // K + V per token
        const long long fixed = (kWgFixedBytes + row - 1) / row;
        auto cost = [&](long long c) {
            const long long len = ((max_kv_len + c - 1) / c + 15) / 16 * 16;
            return (double)((units * c + slots - 1) / slots) * (double)(len + fixed);
        };
        // Counts with the same number of rounds form bands [lo_r, top_r], top_r
        // the largest count that takes r rounds; within a band the cost only
        // falls as the count grows (shorter splits), so the least cost is at
        // some band's top, and the fewest splits within 1 % of it is the first
        // count of the first band whose top qualifies (binary search).  Only
        // the 64 bands from one split's rounds up are searched: past them a
        // partial last round costs little, and the fixed costs of more
        // work-groups only add up.
        const long long rounds_lo = (units + slots - 1) / slots;  // rounds of one split
        long long rounds_hi = (units * hi + slots - 1) / slots;
        rounds_hi = rounds_hi < rounds_lo + 63 ? rounds_hi : rounds_lo + 63;
        if (hi >= 1) {
            auto top = [&](long long r) {
                const long long t = r * slots / units;
                return t < hi ? t : hi;
            };
            double best = cost(b);
            for (long long r = rounds_lo; r <= rounds_hi; ++r)
                if (top(r) >= 1)
                    best = cost(top(r)) < best ? cost(top(r)) : best;
            const double thr = best * 1.01;
            long long lo = 1;
            for (long long r = rounds_lo; r <= rounds_hi && lo <= hi; ++r) {
                const long long t = top(r);
                if (t < lo)
                    continue;
                if (cost(t) <= thr) {
                    long long a0 = lo, a1 = t;  // smallest count in [lo, t] within thr
                    while (a0 < a1) {
                        const long long mid = (a0 + a1) / 2;
                        if (cost(mid) <= thr)
                            a1 = mid;
                        else
                            a0 = mid + 1;
                    }
                    b = a0;
                    break;
                }
                lo = t + 1;
            }
        }
    }
    // the vector kernel runs a lone split per row with one multi-wave
    // work-group per CU, which fills the same wave slots as up to kWavesPerCU
    // splits and needs no combine stage
    if (!grouped && !tiled && !ragged && b >= 2 && b <= fd::kWavesPerCU && units <= num_cus)
        b = 1;
    long long len = (max_kv_len + b - 1) / b;
    len = (len + 15) / 16 * 16;  // whole 16-token tiles
    b = (max_kv_len + len - 1) / len;
    *num_splits = (int)b;
    *split_len = (int)len;
    return FD_OK;
}

size_t fd_workspace_bytes(int batch, int heads_q, int num_splits, int head_dim) {
    if (batch < 1 || heads_q < 1 || num_splits <= 1 || head_dim < 1)
        return 0;
    const size_t rows = (size_t)batch * heads_q * num_splits;
    return round256(rows * head_dim * sizeof(float)) + round256(rows * sizeof(float));
}

int fd_decode_workspace_bytes(int batch, int heads_q, int heads_kv, int max_kv_len,
                              int head_dim, int in_dtype, int has_kv_lens, int num_splits,
                              int split_len, size_t *bytes) {
    if (!bytes)
        return fail(FD_ERR_INVALID, "null output pointer");
    *bytes = 0;
    Plan p;
    int rc = make_plan(batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                       has_kv_lens != 0, false, num_splits, split_len, 0, &p);
    if (rc != FD_OK)
        return rc;
    *bytes = p.pub.workspace_bytes;
    return FD_OK;
}

int fd_decode_plan(int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                   int in_dtype, int has_kv_lens, int paged, int num_splits, int split_len,
                   int num_cus, fd_plan *plan) {
    if (!plan)
        return fail(FD_ERR_INVALID, "null output pointer");
    Plan p;
    int rc = make_plan(batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                       has_kv_lens != 0, paged != 0, num_splits, split_len, num_cus, &p);
    if (rc != FD_OK)
        return rc;
    *plan = p.pub;
    return FD_OK;
}

}  // extern "C"

namespace {

// Split stage with either partial format: lse_part (LSE pair) or m_part and
// l_part (m/l/o triple).
int split_stage(const void *q, const void *k, const void *v, const int32_t *kv_lens, int batch,
                int heads_q, int heads_kv, int max_kv_len, int head_dim, int in_dtype, float scale,
                int num_splits, int split_len, float *o_part, float *lse_part, float *m_part,
                float *l_part, void *stream, const Paging *pg = nullptr) {
    int rc = check_split_inputs(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim,
                                in_dtype, scale);
    if (rc != FD_OK)
        return rc;
    split_len = resolve_split_len(max_kv_len, num_splits, split_len, pg != nullptr);
    rc = check_partition(batch, heads_q, max_kv_len, num_splits, split_len);
    if (rc != FD_OK)
        return rc;
    const bool mlo = m_part || l_part;
    if (!o_part || (mlo ? !(m_part && l_part) : !lse_part))
        return fail(FD_ERR_INVALID, mlo ? "o_part, m_part or l_part is null"
                                        : "o_part or lse_part is null");
    if (!aligned16(o_part) || (mlo ? !(aligned4(m_part) && aligned4(l_part)) : !aligned4(lse_part)))
        return fail(FD_ERR_UNSUPPORTED,
                    "o_part must be 16-byte and the per-split scalars 4-byte aligned");
    fd::SplitArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kv_lens = kv_lens;
    a.batch = batch;
    a.heads_q = heads_q;
    a.heads_kv = heads_kv;
    a.max_kv_len = max_kv_len;
    a.head_dim = head_dim;
    a.num_splits = num_splits;
    a.split_len = split_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o_part = o_part;
    a.lse_part = mlo ? nullptr : lse_part;
    a.m_part = m_part;
    a.l_part = l_part;
    set_paging(a, pg);
    return launch_split(a, in_dtype, static_cast<hipStream_t>(stream));
}

// Checks shared by both combine entry points.
int check_combine(const float *o_part, int batch, int heads_q, int num_splits, int head_dim,
                  const void *o, int out_dtype, const float *lse) {
    if (batch < 1 || heads_q < 1)
        return fail(FD_ERR_INVALID, "sizes must be positive (batch=%d heads_q=%d)", batch,
                    heads_q);
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FD_ERR_INVALID, "num_splits %d outside [1, %d]", num_splits, kMaxSplits);
    if (!o_part || !o)
        return fail(FD_ERR_INVALID, "o_part or o is null");
    if (!head_dim_ok(head_dim))
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128, 256)", head_dim);
    if (!dtype_ok(out_dtype))
        return fail(FD_ERR_UNSUPPORTED, "out_dtype %d not supported", out_dtype);
    if (!aligned16(o_part) || !aligned4(o) || (lse && !aligned4(lse)))
        return fail(FD_ERR_UNSUPPORTED, "misaligned pointer");
    if ((long long)batch * heads_q > 0x7fffffffLL)
        return fail(FD_ERR_INVALID, "batch * heads_q exceeds the launch limit");
    return FD_OK;
}

// Cascade plan: fixed splits for the shared prefix (B_p, uniform length);
// the suffixes on the token-balanced partition when they are ragged and
// grouped, else fixed splits (B_s) in the same partial buffer as the prefix
// (B_p + B_s slots per row, prefix first).
struct CascadePlan {
    int bp = 0, lp = 0, bs = 1, ls = 1;
    int tile_qt = 0;  // > 0: the prefix runs on the tiled matrix-core kernel
    int tile_waves = 1;
    // ragged grouped suffixes: token-balanced partition (bal), its slots merged
    // with the prefix partials by the slot combine; bs/ls unused then
    bool balanced = false;
    BalancedPlan bal;
    size_t o_bytes = 0;    // partial o of the fixed splits (prefix, and suffix if not balanced)
    size_t lse_bytes = 0;
    size_t bytes = 0;      // whole workspace
};

constexpr int kMinPrefixSplitLen = 256;  // tokens

// Prefix splits for the tiled kernel over the shared prefix: its work-groups
// per split are heads_kv x (query tile groups), and the split count fills
// the GPU's wave slots once.
int prefix_plan(int batch, int heads_q, int heads_kv, int prefix_len, int head_dim,
                CascadePlan *p) {
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != FD_OK)
        return rc;
    const long long nq = (long long)batch * (heads_q / heads_kv);
    const TiledShape t = tiled_shape(head_dim, nq);
    const long long per_split = (long long)heads_kv * t.groups;
    long long b = ((long long)cus * t.per_cu() + per_split - 1) / per_split;
    const long long bmax = (prefix_len + kMinPrefixSplitLen - 1) / kMinPrefixSplitLen;
    b = b > bmax ? bmax : b;
    b = b > kMaxAutoSplits ? kMaxAutoSplits : (b < 1 ? 1 : b);
    long long len = (prefix_len + b - 1) / b;
    len = (len + 15) / 16 * 16;
    p->bp = (int)((prefix_len + len - 1) / len);
    p->lp = (int)len;
    p->tile_qt = t.qt;
    p->tile_waves = t.waves;
    return FD_OK;
}

int cascade_plan(int batch, int heads_q, int heads_kv, int prefix_len, int max_suffix_len,
                 int head_dim, int in_dtype, bool has_lens, CascadePlan *p) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || prefix_len < 0 || max_suffix_len < 0 ||
        heads_q % heads_kv)
        return fail(FD_ERR_INVALID,
                    "bad sizes (batch=%d heads_q=%d heads_kv=%d prefix_len=%d max_suffix_len=%d)",
                    batch, heads_q, heads_kv, prefix_len, max_suffix_len);
    if (!head_dim_ok(head_dim) || !dtype_ok(in_dtype))
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d / dtype %d not supported", head_dim,
                    in_dtype);
    int rc;
    if (prefix_len > 0 && fd::split_mfma_tiled_supported(in_dtype, head_dim)) {
        rc = prefix_plan(batch, heads_q, heads_kv, prefix_len, head_dim, p);
        if (rc != FD_OK)
            return rc;
    } else if (prefix_len > 0) {
        rc = fd_choose_splits(batch, heads_q, heads_kv, prefix_len, head_dim, in_dtype, 0, 0,
                              &p->bp, &p->lp);
        if (rc != FD_OK)
            return rc;
    }
    p->balanced = balanced_applies(heads_q, heads_kv, max_suffix_len, head_dim, in_dtype, has_lens,
                                   0);
    if (p->balanced) {
        int cus = 0;
        rc = device_cus(&cus);
        if (rc != FD_OK)
            return rc;
        rc = balanced_plan(batch, heads_q, heads_kv, max_suffix_len, head_dim, in_dtype, cus,
                           &p->bal);
        if (rc != FD_OK)
            return rc;
        p->bs = 0;
        p->ls = 0;
    } else if (max_suffix_len > 0) {
        rc = fd_choose_splits(batch, heads_q, heads_kv, max_suffix_len, head_dim, in_dtype,
                              has_lens, 0, &p->bs, &p->ls);
        if (rc != FD_OK)
            return rc;
    }
    if ((long long)p->bp + p->bs > kMaxSplits)
        return fail(FD_ERR_INVALID, "cascade needs more than %d splits per row", kMaxSplits);
    const size_t rows = (size_t)batch * heads_q * (size_t)(p->bp + p->bs);
    p->o_bytes = round256(rows * head_dim * sizeof(float));
    p->lse_bytes = round256(rows * sizeof(float));
    p->bytes = p->o_bytes + p->lse_bytes + (p->balanced ? p->bal.total() : 0);
    return FD_OK;
}

}  // namespace

extern "C" {

int fd_cascade_workspace_bytes(int batch, int heads_q, int heads_kv, int prefix_len,
                               int max_suffix_len, int head_dim, int in_dtype,
                               int has_suffix_lens, size_t *bytes) {
    if (!bytes)
        return fail(FD_ERR_INVALID, "null output pointer");
    *bytes = 0;
    CascadePlan p;
    int rc = cascade_plan(batch, heads_q, heads_kv, prefix_len, max_suffix_len, head_dim,
                          in_dtype, has_suffix_lens != 0, &p);
    if (rc != FD_OK)
        return rc;
    *bytes = p.bytes;
    return FD_OK;
}

int fd_decode_cascade(const void *q, const void *k_prefix, const void *v_prefix, int prefix_len,
                      const void *k_suffix, const void *v_suffix, const int32_t *suffix_lens,
                      int batch, int heads_q, int heads_kv, int max_suffix_len, int head_dim,
                      int in_dtype, int out_dtype, float scale, void *o, float *lse,
                      void *workspace, size_t workspace_bytes, void *stream) {
    CascadePlan p;
    int rc = cascade_plan(batch, heads_q, heads_kv, prefix_len, max_suffix_len, head_dim,
                          in_dtype, suffix_lens != nullptr, &p);
    if (rc != FD_OK)
        return rc;
    rc = check_split_inputs(q, k_prefix, v_prefix, nullptr, batch, heads_q, heads_kv, prefix_len,
                            head_dim, in_dtype, scale);
    if (rc != FD_OK)
        return rc;
    rc = check_split_inputs(q, k_suffix, v_suffix, suffix_lens, batch, heads_q, heads_kv,
                            max_suffix_len, head_dim, in_dtype, scale);
    if (rc != FD_OK)
        return rc;
    if (!workspace || workspace_bytes < p.bytes)
        return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.bytes,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
        return fail(FD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    rc = check_combine(static_cast<const float *>(workspace), batch, heads_q,
                       p.bp + p.bs > 0 ? p.bp + p.bs : 1, head_dim, o, out_dtype, lse);
    if (rc != FD_OK)
        return rc;
    if (out_dtype != in_dtype && out_dtype != FD_F32)
        return fail(FD_ERR_UNSUPPORTED, "out_dtype %d must equal in_dtype (%d) or be FD_F32",
                    out_dtype, in_dtype);
    char *ws = static_cast<char *>(workspace);
    float *o_part = reinterpret_cast<float *>(ws);
    float *lse_part = reinterpret_cast<float *>(ws + p.o_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    fd::SplitArgs a{};
    a.q = q;
    a.batch = batch;
    a.heads_q = heads_q;
    a.heads_kv = heads_kv;
    a.head_dim = head_dim;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.part_stride = p.bp + p.bs;
    if (p.bp > 0) {  // the shared prefix, read by every sequence
        fd::SplitArgs pa = a;
        pa.k = k_prefix;
        pa.v = v_prefix;
        pa.max_kv_len = prefix_len;
        pa.shared_kv = 1;
        pa.num_splits = p.bp;
        pa.split_len = p.lp;
        pa.tile_qt = p.tile_qt;
        pa.tile_waves = p.tile_waves;
        rc = launch_split(pa, in_dtype, st);
        if (rc != FD_OK)
            return rc;
    }
    if (p.balanced) {  // ragged suffixes: token-balanced pieces, then one slot combine
        char *bws = ws + p.o_bytes + p.lse_bytes;
        fd::SplitArgs sa = a;
        sa.k = k_suffix;
        sa.v = v_suffix;
        sa.kv_lens = suffix_lens;
        sa.max_kv_len = max_suffix_len;
        sa.part_stride = 0;
        sa.o_part = reinterpret_cast<float *>(bws);
        sa.lse_part = reinterpret_cast<float *>(bws + p.bal.o_bytes);
        sa.balanced = 1;
        sa.num_wgs = p.bal.num_wgs;
        sa.tile_waves = p.bal.waves;
        sa.unit_desc = reinterpret_cast<int *>(bws + p.bal.o_bytes + p.bal.lse_bytes);
        rc = launch_split(sa, in_dtype, st);
        if (rc != FD_OK)
            return rc;
        fd::SlotCombineArgs c{};
        c.o_slots = sa.o_part;
        c.lse_slots = sa.lse_part;
        c.unit_desc = sa.unit_desc;
        c.kv_lens = suffix_lens;
        c.batch = batch;
        c.heads_q = heads_q;
        c.gsz = p.bal.gsz;
        c.max_kv_len = max_suffix_len;
        c.head_dim = head_dim;
        c.max_count = p.bal.num_wgs;
        c.o = o;
        c.out_dtype = out_dtype;
        c.lse = lse;
        c.pre_o = o_part;
        c.pre_lse = lse_part;
        c.pre_count = p.bp;
        hipError_t e = fd::launch_combine_slots(c, st);
        if (e != hipSuccess)
            return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
        return FD_OK;
    }
    fd::SplitArgs sa = a;  // each sequence's own suffix
    sa.k = k_suffix;
    sa.v = v_suffix;
    sa.kv_lens = suffix_lens;
    sa.max_kv_len = max_suffix_len;
    sa.num_splits = p.bs;
    sa.split_len = p.ls;
    sa.part_offset = p.bp;
    rc = launch_split(sa, in_dtype, st);
    if (rc != FD_OK)
        return rc;
    hipError_t e = fd::launch_combine(o_part, lse_part, batch * heads_q, p.bp + p.bs, head_dim, o,
                                      out_dtype, lse, st);
    if (e != hipSuccess)
        return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

int fd_decode_split(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                    int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                    int in_dtype, float scale, int num_splits, int split_len, float *o_part,
                    float *lse_part, void *stream) {
    return split_stage(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim,
                       in_dtype, scale, num_splits, split_len, o_part, lse_part, nullptr, nullptr,
                       stream);
}

int fd_decode_split_mlo(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                        int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                        int in_dtype, float scale, int num_splits, int split_len, float *o_part,
                        float *m_part, float *l_part, void *stream) {
    if (!m_part || !l_part)
        return fail(FD_ERR_INVALID, "m_part or l_part is null");
    return split_stage(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim,
                       in_dtype, scale, num_splits, split_len, o_part, nullptr, m_part, l_part,
                       stream);
}

int fd_combine(const float *o_part, const float *lse_part, int batch, int heads_q,
               int num_splits, int head_dim, void *o, int out_dtype, float *lse, void *stream) {
    int rc = check_combine(o_part, batch, heads_q, num_splits, head_dim, o, out_dtype, lse);
    if (rc != FD_OK)
        return rc;
    if (!lse_part)
        return fail(FD_ERR_INVALID, "lse_part is null");
    if (!aligned4(lse_part))
        return fail(FD_ERR_UNSUPPORTED, "misaligned pointer");
    hipError_t e = fd::launch_combine(o_part, lse_part, batch * heads_q, num_splits, head_dim, o,
                                      out_dtype, lse, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

int fd_combine_mlo(const float *o_part, const float *m_part, const float *l_part, int batch,
                   int heads_q, int num_splits, int head_dim, void *o, int out_dtype, float *lse,
                   void *stream) {
    int rc = check_combine(o_part, batch, heads_q, num_splits, head_dim, o, out_dtype, lse);
    if (rc != FD_OK)
        return rc;
    if (!m_part || !l_part)
        return fail(FD_ERR_INVALID, "m_part or l_part is null");
    if (!aligned4(m_part) || !aligned4(l_part))
        return fail(FD_ERR_UNSUPPORTED, "misaligned pointer");
    hipError_t e = fd::launch_combine_mlo(o_part, m_part, l_part, batch * heads_q, num_splits,
                                          head_dim, o, out_dtype, lse,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

}  // extern "C"

namespace {

// The whole decode step, contiguous (pg null) or paged K/V, as make_plan
// decides it; stages (FD_STAGE_*) selects the split launch, the combine
// launch or both.
int decode_impl(const void *q, const void *k, const void *v, const int32_t *kv_lens, int batch,
                int heads_q, int heads_kv, int max_kv_len, int head_dim, int in_dtype,
                int out_dtype, float scale, int num_splits, int split_len, void *o, float *lse,
                void *workspace, size_t workspace_bytes, void *stream, const Paging *pg,
                int stages = FD_STAGE_SPLIT | FD_STAGE_COMBINE) {
    if (stages < 1 || stages > (FD_STAGE_SPLIT | FD_STAGE_COMBINE))
        return fail(FD_ERR_INVALID, "stages %d is not FD_STAGE_SPLIT, FD_STAGE_COMBINE or both",
                    stages);
    const bool run_split = (stages & FD_STAGE_SPLIT) != 0;
    const bool run_combine = (stages & FD_STAGE_COMBINE) != 0;
    int rc = check_split_inputs(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim,
                                in_dtype, scale);
    if (rc != FD_OK)
        return rc;
    if (!o)
        return fail(FD_ERR_INVALID, "o is null");
    if (!dtype_ok(out_dtype) || (out_dtype != in_dtype && out_dtype != FD_F32))
        return fail(FD_ERR_UNSUPPORTED, "out_dtype %d must equal in_dtype (%d) or be FD_F32",
                    out_dtype, in_dtype);
    if (!aligned4(o) || (lse && !aligned4(lse)))
        return fail(FD_ERR_UNSUPPORTED, "o and lse must be 4-byte aligned");
    Plan p;
    rc = make_plan(batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype, kv_lens != nullptr,
                   pg != nullptr, num_splits, split_len, 0, &p);
    if (rc != FD_OK)
        return rc;
    const fd_plan &r = p.pub;
    if (r.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < r.workspace_bytes)
            return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                        r.workspace_bytes, workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace))
            return fail(FD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    fd::SplitArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kv_lens = kv_lens;
    a.batch = batch;
    a.heads_q = heads_q;
    a.heads_kv = heads_kv;
    a.max_kv_len = max_kv_len;
    a.head_dim = head_dim;
    a.num_splits = r.num_splits;
    a.split_len = r.split_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out_dtype = out_dtype;
    set_paging(a, pg);
    hipError_t e = hipSuccess;
    switch (r.route) {
    case FD_ROUTE_BALANCED: {
        a.o_part = reinterpret_cast<float *>(ws);
        a.lse_part = reinterpret_cast<float *>(ws + p.bal.o_bytes);
        a.balanced = 1;
        a.num_wgs = p.bal.num_wgs;
        a.tile_waves = p.bal.waves;
        a.unit_desc = reinterpret_cast<int *>(ws + p.bal.o_bytes + p.bal.lse_bytes);
#if FD_WG_CLOCKS
        a.wg_clock = g_wg_clock_bytes >= (size_t)p.bal.num_wgs * 4 * sizeof(unsigned long long)
                         ? g_wg_clock
                         : nullptr;
#endif
        if (run_split && (rc = launch_split(a, in_dtype, st)) != FD_OK)
            return rc;
        if (!run_combine)
            return FD_OK;
        fd::SlotCombineArgs c{};
        c.o_slots = a.o_part;
        c.lse_slots = a.lse_part;
        c.unit_desc = a.unit_desc;
        c.kv_lens = kv_lens;
        c.batch = batch;
        c.heads_q = heads_q;
        c.gsz = p.bal.gsz;
        c.max_kv_len = max_kv_len;
        c.head_dim = head_dim;
        c.max_count = p.bal.num_wgs;
        c.o = o;
        c.out_dtype = out_dtype;
        c.lse = lse;
        e = fd::launch_combine_slots(c, st);
        break;
    }
    case FD_ROUTE_DIRECT:  // one split per row: the split stage writes o and lse itself
    case FD_ROUTE_FUSED:   // small grid: splits merged in LDS, final output directly
        a.o = o;
        a.lse = lse;
        a.fused_waves = p.fused;
        return run_split ? launch_split(a, in_dtype, st) : FD_OK;
    default: {  // FD_ROUTE_SPLITS
        const size_t rows = (size_t)batch * heads_q * r.num_splits;
        a.o_part = reinterpret_cast<float *>(ws);
        a.lse_part = reinterpret_cast<float *>(ws + round256(rows * head_dim * sizeof(float)));
        if (run_split && (rc = launch_split(a, in_dtype, st)) != FD_OK)
            return rc;
        if (!run_combine)
            return FD_OK;
        e = fd::launch_combine(a.o_part, a.lse_part, batch * heads_q, r.num_splits, head_dim, o,
                               out_dtype, lse, st);
    }
    }
    if (e != hipSuccess)
        return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

}  // namespace

extern "C" {

int fd_decode(const void *q, const void *k, const void *v, const int32_t *kv_lens, int batch,
              int heads_q, int heads_kv, int max_kv_len, int head_dim, int in_dtype,
              int out_dtype, float scale, int num_splits, int split_len, void *o, float *lse,
              void *workspace, size_t workspace_bytes, void *stream) {
    return decode_impl(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                       out_dtype, scale, num_splits, split_len, o, lse, workspace,
                       workspace_bytes, stream, nullptr);
}

#if FD_WG_CLOCKS
// Instrumented builds only (not part of fd.h): from now on the token-balanced
// split kernel of fd_decode writes per-work-group stamps into buf (device
// memory, 4 x 8 bytes per work-group, see SplitArgs::wg_clock) when it holds
// that many bytes; buf NULL turns the stamps off.
int fd_debug_wg_clocks(void *buf, size_t bytes) {
    g_wg_clock = static_cast<unsigned long long *>(buf);
    g_wg_clock_bytes = buf ? bytes : 0;
    return FD_OK;
}
#endif

int fd_decode_stages(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                     int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                     int in_dtype, int out_dtype, float scale, int num_splits, int split_len,
                     void *o, float *lse, void *workspace, size_t workspace_bytes, int stages,
                     void *stream) {
    return decode_impl(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                       out_dtype, scale, num_splits, split_len, o, lse, workspace,
                       workspace_bytes, stream, nullptr, stages);
}

int fd_decode_noalloc(const void *q, const void *k, const void *v, const int32_t *kv_lens,
                      int batch, int heads_q, int heads_kv, int max_kv_len, int head_dim,
                      int in_dtype, int out_dtype, float scale, int num_splits, int split_len,
                      void *o, float *lse, void *stream) {
    size_t need = 0;
    int rc = fd_decode_workspace_bytes(batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                                       kv_lens != nullptr, num_splits, split_len, &need);
    if (rc != FD_OK)
        return rc;
    if (need > fd::kScratchBytes)
        return fail(FD_ERR_WORKSPACE,
                    "fd_decode_noalloc: this step needs %zu bytes of scratch, more than the "
                    "library's %zu; call fd_decode with a workspace of that size instead",
                    need, fd::kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        hipError_t e = fd::scratch_buffer(&ws);
        if (e != hipSuccess)
            return fail(FD_ERR_HIP, "scratch buffer address: %s", hipGetErrorString(e));
    }
    return decode_impl(q, k, v, kv_lens, batch, heads_q, heads_kv, max_kv_len, head_dim, in_dtype,
                       out_dtype, scale, num_splits, split_len, o, lse, ws, need, stream, nullptr);
}

int fd_decode_split_paged(const void *q, const void *k_pages, const void *v_pages,
                          const int32_t *block_table, const int32_t *kv_lens, int batch,
                          int heads_q, int heads_kv, int page_size, int max_pages_per_seq,
                          int num_pages, int head_dim, int in_dtype, float scale, int num_splits,
                          int split_len, float *o_part, float *lse_part, void *stream) {
    Paging pg;
    int rc = check_paging(block_table, page_size, max_pages_per_seq, num_pages, heads_kv,
                          head_dim, in_dtype, &pg);
    if (rc != FD_OK)
        return rc;
    if (split_len % 16 != 0)
        return fail(FD_ERR_INVALID, "paged K/V needs split_len (%d) to be a multiple of 16",
                    split_len);
    return split_stage(q, k_pages, v_pages, kv_lens, batch, heads_q, heads_kv,
                       max_pages_per_seq * page_size, head_dim, in_dtype, scale, num_splits,
                       split_len, o_part, lse_part, nullptr, nullptr, stream, &pg);
}

int fd_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                    const int32_t *block_table, const int32_t *kv_lens, int batch, int heads_q,
                    int heads_kv, int page_size, int max_pages_per_seq, int num_pages,
                    int head_dim, int in_dtype, int out_dtype, float scale, int num_splits,
                    int split_len, void *o, float *lse, void *workspace, size_t workspace_bytes,
                    void *stream) {
    Paging pg;
    int rc = check_paging(block_table, page_size, max_pages_per_seq, num_pages, heads_kv,
                          head_dim, in_dtype, &pg);
    if (rc != FD_OK)
        return rc;
    return decode_impl(q, k_pages, v_pages, kv_lens, batch, heads_q, heads_kv,
                       max_pages_per_seq * page_size, head_dim, in_dtype, out_dtype, scale,
                       num_splits, split_len, o, lse, workspace, workspace_bytes, stream, &pg);
}

}  // extern "C"
