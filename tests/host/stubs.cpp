// stubs.cpp -- host-only stand-ins for the HIP runtime calls and the kernel
// launchers of libfd, so that the library's host code (argument checks, the
// plan, workspace carving; csrc/fd_api.cpp) can be built with the address and
// undefined-behaviour sanitizers and run without a GPU.
//
// The device reports 256 compute units and 160 KiB of LDS per CU.  A launch
// queues nothing: it checks the arguments it is given against what the
// kernels would touch, and records the launch.  For the token-balanced split
// stage it walks every work-group's share on the host (partition_plan.h, the
// same walk the kernel runs) with kv_lens read from host memory, so callers
// pass host arrays where the library takes device pointers, and checks that
// every piece's slot and every unit descriptor falls inside the workspace the
// plan carved.  A violation aborts.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fd_internal.h"
#include "partition_plan.h"
#include "stubs.h"

namespace {
HostLaunchLog g_log;

[[noreturn]] void die(const char *what) {
    std::fprintf(stderr, "stub launcher: %s\n", what);
    std::abort();
}
}  // namespace

HostLaunchLog &host_launch_log() { return g_log; }

extern "C" {
hipError_t hipGetDevice(int *device) {
    *device = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int device) {
    if (device != 0)
        return hipErrorInvalidDevice;
    switch (attr) {
    case hipDeviceAttributeMultiprocessorCount: *value = 256; return hipSuccess;
    case hipDeviceAttributeMaxSharedMemoryPerMultiprocessor: *value = 160 * 1024; return hipSuccess;
    default: return hipErrorInvalidValue;
    }
}
const char *hipGetErrorString(hipError_t) { return "stubbed HIP runtime"; }
}

namespace fd {
namespace {

// The token-balanced split stage over units of hx heads each (the matrix-core
// kernel: KV heads, gsz = heads_q / heads_kv query rows per slot; the vector
// kernel: query heads, one row per slot): every share walked on the host.
void check_balanced(const SplitArgs &a, int hx) {
    ++g_log.balanced;
    const long long units = (long long)a.batch * hx;
    const long long slots = (long long)a.num_wgs + units;
    // the layout the plan carved: o slots, LSE slots, descriptors
    const size_t gsz = (size_t)(a.heads_q / hx);
    const char *o0 = reinterpret_cast<const char *>(a.o_part);
    const char *l0 = reinterpret_cast<const char *>(a.lse_part);
    const char *d0 = reinterpret_cast<const char *>(a.unit_desc);
    if (l0 < o0 + slots * gsz * a.head_dim * sizeof(float) ||
        d0 < l0 + slots * gsz * sizeof(float))
        die("balanced workspace parts overlap");
    if (g_log.workspace_end && d0 + units * 2 * sizeof(int) > g_log.workspace_end)
        die("balanced descriptors run past the workspace");
    for (int blk = 0; blk < a.num_wgs; ++blk) {
        const int w = share_index(blk, hx, a.num_wgs);
        if (w < 0 || w >= a.num_wgs)
            die("share index out of range");
        PieceCursor c;
        if (!balanced_start_ref(a.kv_lens, a.batch, a.max_kv_len, hx, w, a.num_wgs, c))
            continue;
        walk_share(a.kv_lens, a.batch, a.max_kv_len, hx, w, c, [&](const Piece &p) {
            if (p.slot < 0 || p.slot >= slots)
                die("piece slot outside the slot arrays");
            if (p.t0 < 0 || p.t1 > p.n || p.t0 >= p.t1)
                die("piece token range outside its sequence");
            if (p.first && (p.desc_count < 1 || p.slot + p.desc_count > slots))
                die("unit descriptor outside the slot arrays");
            ++g_log.pieces;
        });
    }
}

}  // namespace

hipError_t launch_split_valu(const SplitArgs &a, int in_dtype, hipStream_t) {
    ++g_log.split_valu;
    if (a.balanced) {  // one unit per (sequence, group of valu_heads_per_wg query heads)
        check_balanced(a, a.heads_q / valu_heads_per_wg(in_dtype, a.head_dim, a.heads_q / a.heads_kv));
        return hipSuccess;
    }
    if (a.num_splits < 1 || a.split_len < 1 ||
        (long long)a.num_splits * a.split_len < a.max_kv_len)
        die("vector split launch with a partition that does not cover the cache");
    return hipSuccess;
}

hipError_t launch_split_mfma(const SplitArgs &a, int, hipStream_t) {
    ++g_log.split_mfma;
    if (!a.balanced) {
        if (a.num_splits < 1 || a.split_len < 1 ||
            (long long)a.num_splits * a.split_len < a.max_kv_len)
            die("matrix-core split launch with a partition that does not cover the cache");
        return hipSuccess;
    }
    check_balanced(a, a.heads_kv);
    return hipSuccess;
}

hipError_t launch_combine(const float *, const float *, int rows, int num_splits, int, void *,
                          int, float *, hipStream_t) {
    ++g_log.combine;
    if (rows < 1 || num_splits < 1)
        die("combine launch without rows or splits");
    return hipSuccess;
}

hipError_t launch_combine_mlo(const float *, const float *, const float *, int rows,
                              int num_splits, int, void *, int, float *, hipStream_t) {
    ++g_log.combine;
    if (rows < 1 || num_splits < 1)
        die("combine launch without rows or splits");
    return hipSuccess;
}

hipError_t launch_combine_slots(const SlotCombineArgs &c, hipStream_t) {
    ++g_log.combine;
    if ((long long)c.batch * c.heads_q > 0x7fffffffLL || c.gsz < 1 || c.heads_q % c.gsz)
        die("slot combine launch with a bad grid");
    return hipSuccess;
}

hipError_t scratch_buffer(void **ptr) {
    alignas(256) static char fake[256];
    *ptr = fake;  // never dereferenced: the stub launchers touch no memory
    return hipSuccess;
}

}  // namespace fd
