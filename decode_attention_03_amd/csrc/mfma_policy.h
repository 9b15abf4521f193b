// mfma_policy.h -- which grouped-query (matrix-core) kernel shape serves a
// group of query heads, shared by the host planner and the kernels: the
// constexpr limits the kernels are instantiated with, and the host functions
// that the plan (fd_api.cpp) asks.  No device code; compiles as plain C++.
//
// G = heads_q / heads_kv query heads share one KV head.  They are served in
// tiles of 16 queries (the matrix-core width): one tile for G <= 16 on the
// one-tile kernel; larger groups on the tiled kernel (several tiles per wave,
// several waves per work-group sharing each K/V step staged in LDS), or on
// the token-balanced kernel for ragged batches.
#pragma once

namespace fd {

constexpr int kMaxGroup = 16;  // query heads per KV head one wave can hold in one tile

// Query tiles per wave of a one-wave tiled work-group that fit in the
// register file without spilling next to 16 KB steps (every tile keeps its
// own Q fragments, O accumulators and softmax state).  Four tiles fit at
// d = 128 with 8 KB steps, but measured slower: the smaller steps and the
// shorter splits that the fewer work-groups need cost more than the halved
// re-reads save.
#ifndef FD_PREFIX_QT128
#define FD_PREFIX_QT128 2
#endif
template <int D>
constexpr int tile_max_qt() {
    return D == 64 ? 4 : (D == 128 ? FD_PREFIX_QT128 : 1);
}

// Query tiles per wave in multi-wave work-groups and in the token-balanced
// kernel: at most two (four tiles on one wave, at d = 64, measured slower in
// the balanced kernel than the tiled kernel's fixed splits, and with four
// waves they spill).
template <int D>
constexpr int wide_qt() {
    return tile_max_qt<D>() < 2 ? tile_max_qt<D>() : 2;
}

// Waves of a multi-wave work-group: up to 4 at every head size (each loads
// an equal share of every staged step's row groups), 8 at d <= 128 (one tile
// per wave, two waves per SIMD), capped by FD_TILE_MAX_WAVES.
#ifndef FD_TILE_MAX_WAVES
#define FD_TILE_MAX_WAVES 8
#endif
template <int D>
constexpr int tile_max_waves() {
    constexpr int w = D <= 128 ? 8 : 4;
    return w < FD_TILE_MAX_WAVES ? w : FD_TILE_MAX_WAVES;
}

// One query tile per wave while the waves cover the group (else each wave
// takes as many tiles as it holds): the token-balanced plan, the tiled kernel.
#ifndef FD_BAL_SPREAD
#define FD_BAL_SPREAD 1
#endif
#ifndef FD_TILE_SPREAD
#define FD_TILE_SPREAD 1
#endif

// Most tiles a multi-wave work-group holds: qt per wave on up to four waves,
// or one per wave on more.
constexpr int max_tiles_per_wg(int qt, int wmax) {
    return qt * (wmax < 4 ? wmax : 4) > wmax ? qt * (wmax < 4 ? wmax : 4) : wmax;
}

// The host-side questions of the plan, by run-time head size.
inline int split_mfma_tile_max_qt(int head_dim) {
    switch (head_dim) {
    case 64: return tile_max_qt<64>();
    case 128: return tile_max_qt<128>();
    case 256: return tile_max_qt<256>();
    default: return 0;
    }
}

inline int split_mfma_wide_qt(int head_dim) {
    switch (head_dim) {
    case 64: return wide_qt<64>();
    case 128: return wide_qt<128>();
    case 256: return wide_qt<256>();
    default: return 1;
    }
}

inline int split_mfma_tile_max_waves(int head_dim) {
    switch (head_dim) {
    case 64: return tile_max_waves<64>();
    case 128: return tile_max_waves<128>();
    case 256: return tile_max_waves<256>();
    default: return 1;
    }
}

inline bool split_mfma_tile_spread() { return FD_TILE_SPREAD != 0; }

// Five to eight query tiles at d <= 128 on the tiled kernel: one eight-wave
// work-group per unit (FD_TILE_PAIR 0), or several work-groups of
// FD_TILE_PAIR waves (4 or 2) with one tile per wave, 16 KB steps and eight
// waves per CU in all (two per SIMD, from different work-groups), the unit's
// K/V shared through L2; their barriers are independent of each other.
#ifndef FD_TILE_PAIR
#define FD_TILE_PAIR 4
#endif
constexpr int tiled_pair_waves() { return FD_TILE_PAIR; }
constexpr bool tiled_pair(int head_dim, int qt, int waves, long long groups) {
    return FD_TILE_PAIR != 0 && head_dim <= 128 && qt == 1 && waves == FD_TILE_PAIR &&
           groups > 1;
}
// Resident tiled work-groups per CU with this many waves each (pair: the
// four-wave work-groups above, two per CU).
inline int split_mfma_tiled_wg_per_cu(int waves, bool pair = false) {
    if (pair)
        return 8 / waves;
    if (waves <= 1)
        return kPrefixWgPerCU;
    const int n = kPrefixWgPerCU / waves;  // one wave per SIMD
    return n > 1 ? n : 1;
}

// Largest group the token-balanced kernel takes (all of a unit's query tiles
// in one work-group): up to two tiles per wave (with four, 64 heads at
// d = 64, one wave's pieces were bound by their arithmetic: the tiled
// kernel's fixed splits measured 5 % faster on a ragged batch), on up to the
// most waves the head size allows.
inline int split_mfma_balanced_max_group(int head_dim) {
    switch (head_dim) {
    case 64: return 16 * max_tiles_per_wg(wide_qt<64>(), tile_max_waves<64>());
    case 128: return 16 * max_tiles_per_wg(wide_qt<128>(), tile_max_waves<128>());
    case 256: return 16 * max_tiles_per_wg(wide_qt<256>(), tile_max_waves<256>());
    default: return 0;
    }
}

// Waves of the token-balanced kernel's work-groups for a group size (0: too
// large for it).
inline int split_mfma_balanced_waves(int head_dim, int group) {
    const int tiles = (group + 15) / 16;
    int qt = 0, wmax = 1;
    switch (head_dim) {
    case 64: qt = wide_qt<64>(); wmax = tile_max_waves<64>(); break;
    case 128: qt = wide_qt<128>(); wmax = tile_max_waves<128>(); break;
    case 256: qt = wide_qt<256>(); wmax = tile_max_waves<256>(); break;
    default: return 0;
    }
    if (tiles <= 1)
        return 1;
    int w = 2;
    if (FD_BAL_SPREAD && tiles <= wmax) {  // one tile on each of w waves
        while (w < tiles)
            w *= 2;
        return w;
    }
    if (tiles <= qt)
        return 1;
    const int wq = wmax < 4 ? wmax : 4;  // more than four waves hold one tile each
    while (w < wq && qt * w < tiles)
        w *= 2;
    return qt * w >= tiles ? w : 0;
}

// Token-balanced work-groups of four one-tile waves at d <= 128 run two per
// SIMD (16 KB steps), measured 1.5-5 % faster than 32 KB steps at one wave
// per SIMD.
constexpr bool bal_two_per_simd(int head_dim, int qt, int waves) {
    return waves == 4 && qt == 1 && head_dim <= 128;
}

// Resident token-balanced work-groups per CU for a group size.
inline int split_mfma_balanced_wg_per_cu(int head_dim, int group) {
    const int waves = split_mfma_balanced_waves(head_dim, group);
    if (waves <= 1)
        return kMfmaWgPerCU;
    if (bal_two_per_simd(head_dim, (group + 15) / 16 <= waves ? 1 : 2, waves))
        return 2;
    const int n = kPrefixWgPerCU / waves;  // one wave per SIMD
    return n > 1 ? n : 1;
}

inline bool split_mfma_tiled_supported(int in_dtype, int head_dim) {
    return (in_dtype == kBF16 || in_dtype == kF16) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

inline bool split_mfma_supported(int in_dtype, int head_dim, int group) {
    return (in_dtype == kBF16 || in_dtype == kF16) && group >= 2 && group <= kMaxGroup &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

}  // namespace fd
