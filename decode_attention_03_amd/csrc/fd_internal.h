// fd_internal.h -- declarations shared by the host API and the kernel files
// of libfd (not installed, not part of the C ABI).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#ifndef FD_WG_CLOCKS
#define FD_WG_CLOCKS 0
#endif

namespace fd {

// Element type codes (same values as the FD_* codes of the public header).
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Resident waves per CU the split kernels aim at: MI355X HBM streams best
// with about two waves per CU, each with ~16 KB of loads in flight.
#ifndef FD_WAVES_PER_CU
#define FD_WAVES_PER_CU 2
#endif
constexpr int kWavesPerCU = FD_WAVES_PER_CU;

// Query heads per vector-kernel work-group (the kernel's HPW).  fp32 grouped
// heads run on the vector kernel; taking up to eight heads of one KV head
// together (eight at d <= 128, where their q rows and states fit the
// registers, else four), every row of lanes holds their q rows and running
// states, so each K/V row it loads serves all of them instead of being
// loaded once per query head.  One head otherwise (bf16/fp16 groups run on
// the matrix cores).
#ifndef FD_VALU_HEAD_GROUP
#define FD_VALU_HEAD_GROUP 1
#endif
inline int valu_heads_per_wg(int in_dtype, int head_dim, int group) {
    if (!FD_VALU_HEAD_GROUP || in_dtype != kF32 || group < 2)
        return 1;
    if (group % 8 == 0 && head_dim <= 128)
        return 8;
    return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

// Resident one-wave vector-kernel work-groups per CU: kWavesPerCU, or four
// (one per SIMD) with eight heads per work-group, whose steps are bound by
// their arithmetic rather than by the load stream.
inline int valu_wg_per_cu(int heads_per_wg) { return heads_per_wg >= 8 ? 4 : kWavesPerCU; }

// Resident one-wave work-groups per CU of the grouped (matrix-core) split
// kernels; the token-balanced partition makes this many shares per CU.
#ifndef FD_MFMA_WG_PER_CU
#define FD_MFMA_WG_PER_CU 2
#endif
constexpr int kMfmaWgPerCU = FD_MFMA_WG_PER_CU;

// Resident work-groups per CU of the tiled kernel (shared prefix, groups of
// more than 16 query heads): its K/V rows are read by several work-groups
// each, so more of them in flight per CU pays.
#ifndef FD_PREFIX_WG_PER_CU
#define FD_PREFIX_WG_PER_CU 4
#endif
constexpr int kPrefixWgPerCU = FD_PREFIX_WG_PER_CU;
// With several waves per work-group (tile_waves) the same number of waves
// per CU: kPrefixWgPerCU / tile_waves work-groups (each wave needs over half
// of a SIMD's registers, so one wave per SIMD is what fits anyway).

// Everything one split-stage launch needs.  Shapes follow the public layouts:
// q [batch, heads_q, d], K/V [batch, max_kv_len, heads_kv, d].
struct SplitArgs {
    const void *q;
    const void *k;
    const void *v;
    const int32_t *kv_lens;  // device [batch] or nullptr
    int batch, heads_q, heads_kv, max_kv_len, head_dim;
    int num_splits, split_len;
    float scale_log2;        // scale * log2(e): scores are kept in the log2 domain
    float *o_part;           // fixed splits: [batch, heads_q, num_splits, d] (num_splits > 1)
                             // balanced: slot array [slots][gsz][d]
    float *lse_part;         // fixed: [batch, heads_q, num_splits]; balanced: [slots][gsz]
    // m/l/o partial format (fixed splits only): with m_part set, each split
    // writes its max score m (natural log domain) and l = sum exp(s - m) to
    // m_part / l_part ([batch, heads_q, num_splits]) instead of lse_part.
    float *m_part;
    float *l_part;
    void *o;                 // final output                       (num_splits == 1)
    float *lse;              // final LSE, may be null             (num_splits == 1)
    int out_dtype;
    // Token-balanced partition (partition.h), used when `balanced` is set:
    // num_wgs work-groups, per-unit descriptors {first slot, count} in unit_desc.
    int balanced;
    int num_wgs;
    int *unit_desc;
    // Paged K/V: k and v point at pages [num_pages, page_size, heads_kv, d];
    // token t of sequence b sits in page block_table[b * max_pages + t /
    // page_size], row t % page_size.  page_size = 1 << page_shift >= 16, so a
    // 16-token tile never straddles two pages; max_kv_len = max_pages *
    // page_size.  Table entries outside [0, num_pages) are clamped into it.
    const int32_t *block_table;  // null: contiguous K/V
    int page_shift;
    int max_pages;
    int num_pages;
    // Shared cache: with shared_kv set every sequence reads the same K/V
    // ([max_kv_len, heads_kv, d], batch stride 0), as the cascade's prefix.
    int shared_kv;
    // Query tiles on the matrix cores (bf16/f16): the queries of a KV head in
    // tiles of 16 rows, tile_qt tiles per work-group (1, 2 or 4), several
    // work-groups per (KV head, split) when there are more tiles.  With
    // shared_kv set (the cascade's prefix) the queries are all batch * G of
    // the KV head; otherwise the G queries of one sequence (groups larger
    // than one tile).  0 selects the one-tile kernels.
    int tile_qt;
    // Tiled and token-balanced kernels: waves per work-group (1, 2, 4 or 8;
    // 0 means 1).  The waves take their own query tiles and share every K/V
    // step staged in LDS, so a work-group serves all of its tiles from one
    // read of the rows.
    int tile_waves;
    // Fixed-split partial slots: split i of row r is slot r * part_stride +
    // part_offset + i (part_stride 0 means num_splits), so two launches can
    // fill one partial buffer.
    int part_stride, part_offset;
    // Vector kernel only: with fused_waves (2, 4 or 8 >= num_splits) one
    // work-group per row runs wave w on split w and merges the splits in LDS,
    // writing the final o / lse (a.o, a.lse); small grids only.
    int fused_waves;
    // Vector kernel only: waves per work-group (1, or kWavesPerCU for one
    // work-group per CU).  Two waves share a
    // split (and merge in LDS) when the grid has fewer work-groups than the
    // GPU has wave slots, e.g. one split per row.
    int valu_waves;
#if FD_WG_CLOCKS
    // Instrumented builds only (-DFD_WG_CLOCKS=1): the token-balanced kernel
    // writes four 64-bit words per share w at wg_clock[4 w ..]: the constant
    // 100 MHz clock at its start and at its end, (pieces << 32) | tokens
    // (the K/V rows its pieces read, per KV head), and where it ran: the
    // HW_ID register << 32 | the XCD << 24 | its block index.  Null: no
    // stamps.
    unsigned long long *wg_clock;
#endif
};

// VALU split kernel: one work-group (a.valu_waves waves) per (sequence, query
// head, split).  Handles every head_dim/dtype; used for one query head per
// KV head and for fp32 (with heads_q > heads_kv each query head reads its
// shared KV head on its own).
hipError_t launch_split_valu(const SplitArgs &a, int in_dtype, hipStream_t stream);

// MFMA split kernels for grouped heads (bf16/f16): one work-group per
// (sequence, KV head, split) computing all G <= 16 query rows of the group in
// one tile; with tile_qt set, the tiled kernel (16-query tiles, several
// work-groups per unit); with balanced set, the token-balanced kernel.  Which
// one serves a group, and in what shape, is decided by the functions of
// mfma_policy.h (included below).
hipError_t launch_split_mfma(const SplitArgs &a, int in_dtype, hipStream_t stream);

// LSE merge of num_splits partials for `rows` = batch * heads_q rows.
hipError_t launch_combine(const float *o_part, const float *lse_part, int rows, int num_splits,
                          int head_dim, void *o, int out_dtype, float *lse, hipStream_t stream);

// m/l/o merge of num_splits triples per row: m_g = max m, weights
// exp(m - m_g) l / l_g with l_g = sum exp(m - m_g) l; lse = m_g + log l_g.
hipError_t launch_combine_mlo(const float *o_part, const float *m_part, const float *l_part,
                              int rows, int num_splits, int head_dim, void *o, int out_dtype,
                              float *lse, hipStream_t stream);

// LSE merge of the slots a token-balanced split stage wrote: row (b, h) reads
// the descriptor of unit b * (heads_q / gsz) + h / gsz (gsz query heads per
// unit); max_count bounds any unit's slot count.
struct SlotCombineArgs {
    const float *o_slots;     // [slots][gsz][d]
    const float *lse_slots;   // [slots][gsz]
    const int *unit_desc;     // [units][2]
    const int32_t *kv_lens;   // device [batch] or nullptr
    int batch, heads_q, gsz, max_kv_len, head_dim, max_count;
    void *o;
    int out_dtype;
    float *lse;
    // optional fixed partials merged in front of every row's slots (a
    // cascade's prefix): [batch * heads_q, pre_count, d] and [.., pre_count]
    const float *pre_o;
    const float *pre_lse;
    int pre_count;
};
hipError_t launch_combine_slots(const SlotCombineArgs &c, hipStream_t stream);

// The library-owned scratch of fd_decode_noalloc (noalloc.hip): kScratchBytes
// of device memory per device, 256-byte aligned, held until the process ends.
// scratch_buffer returns its device address on the current device (looked up
// once per device with hipGetSymbolAddress).
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_buffer(void **ptr);

}  // namespace fd

#include "mfma_policy.h"
