// host_checks.cpp -- CPU checks of libfd's host code, built with the address
// and undefined-behaviour sanitizers (tests/test_host_sanitized.py):
//   1. the token-balanced partition (partition_plan.h, the definitions and
//      the walk the split kernel runs) over seeded random ragged batches:
//      every granule of every non-empty (sequence, KV head) unit is covered
//      exactly once, a unit's pieces fill consecutive slots below
//      work-groups + units, the piece holding granule 0 carries the unit's
//      slot count, the share permutation is a bijection, and the start
//      cursor agrees with a brute-force walk of the flattened space;
//   2. fd_decode_plan for the five named workloads on 256 compute units;
//   3. fd_decode and fd_decode_cascade through the stub launchers
//      (stubs.cpp), which walk every balanced share against the workspace
//      the plan carved.
// Exit status 0 when every check passes; a failed check prints and aborts.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "fd.h"
#include "partition_plan.h"
#include "stubs.h"

namespace {

[[noreturn]] void fail(const char *what, long long a = 0, long long b = 0) {
    std::fprintf(stderr, "host check failed: %s (%lld, %lld)\n", what, a, b);
    std::abort();
}

struct Lcg {  // a fixed generator, so every run checks the same cases
    uint64_t s;
    explicit Lcg(uint64_t seed) : s(seed * 6364136223846793005ull + 1442695040888963407ull) {}
    uint32_t next() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (uint32_t)(s >> 33);
    }
    int range(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }
};

// The flattened space by brute force: position -> (x, b, t) in head-major order.
bool locate(const std::vector<int32_t> &lens, int max_kv_len, int hx, long long pos, int *x,
            int *b, int *t) {
    long long p = 0;
    for (int xx = 0; xx < hx; ++xx)
        for (int bb = 0; bb < (int)lens.size(); ++bb) {
            const int n = fd::unit_cost(lens.data(), bb, max_kv_len);
            if (pos < p + n) {
                *x = xx;
                *b = bb;
                *t = (int)(pos - p);
                return true;
            }
            p += n;
        }
    return false;
}

void check_partition_case(const std::vector<int32_t> &lens, int max_kv_len, int hx, int num_wgs,
                          bool brute) {
    const int batch = (int)lens.size();
    const long long units = (long long)batch * hx;
    // share permutation
    std::vector<char> seen(num_wgs, 0);
    for (int blk = 0; blk < num_wgs; ++blk) {
        const int w = fd::share_index(blk, hx, num_wgs);
        if (w < 0 || w >= num_wgs || seen[w])
            fail("share_index is not a bijection", blk, w);
        seen[w] = 1;
    }
    struct P {
        int lo, hi, slot, count;
        bool first;
    };
    std::map<long long, std::vector<P>> by_unit;
    std::vector<char> slot_used((size_t)(num_wgs + units), 0);
    for (int w = 0; w < num_wgs; ++w) {
        fd::PieceCursor c;
        if (!fd::balanced_start_ref(lens.data(), batch, max_kv_len, hx, w, num_wgs, c))
            continue;
        if (brute) {
            int x, b, t;
            if (!locate(lens, max_kv_len, hx, c.pos, &x, &b, &t) || x != c.x || b != c.b ||
                t != c.t)
                fail("start cursor differs from the brute-force walk", w, c.pos);
        }
        long long prev_end = -1;
        fd::walk_share(lens.data(), batch, max_kv_len, hx, w, c, [&](const fd::Piece &p) {
            if (p.slot < 0 || p.slot >= num_wgs + units)
                fail("slot out of range", p.slot, num_wgs + units);
            if (slot_used[p.slot])
                fail("slot written twice", p.slot);
            slot_used[p.slot] = 1;
            if (p.lo < 0 || p.hi <= p.lo || p.t1 > p.n || p.t0 != (long)p.lo * fd::kGranule)
                fail("bad piece range", p.lo, p.hi);
            const long long u = (long long)p.x * batch + p.b;  // head-major order
            if (u <= prev_end && prev_end >= 0 && u < prev_end)
                fail("pieces of a share out of order", u, prev_end);
            prev_end = u;
            by_unit[(long long)p.b * hx + p.x].push_back({p.lo, p.hi, p.slot, p.desc_count,
                                                           p.first});
        });
    }
    for (int b = 0; b < batch; ++b)
        for (int x = 0; x < hx; ++x) {
            const int g = fd::granules(lens.data(), b, max_kv_len);
            auto it = by_unit.find((long long)b * hx + x);
            if (g == 0) {
                if (it != by_unit.end())
                    fail("pieces for an empty sequence", b, x);
                continue;
            }
            if (it == by_unit.end())
                fail("unit without pieces", b, x);
            std::vector<P> ps = it->second;
            std::sort(ps.begin(), ps.end(), [](const P &l, const P &r) { return l.lo < r.lo; });
            if (ps.front().lo != 0 || ps.back().hi != g || !ps.front().first)
                fail("unit not covered from its first granule to its last", b, x);
            if (ps.front().count != (int)ps.size())
                fail("descriptor count differs from the unit's pieces", ps.front().count,
                     (long long)ps.size());
            for (size_t i = 1; i < ps.size(); ++i) {
                if (ps[i].lo != ps[i - 1].hi)
                    fail("granules not covered exactly once", b, x);
                if (ps[i].first)
                    fail("two pieces claim granule 0", b, x);
                if (ps[i].slot != ps.front().slot + (int)i)
                    fail("a unit's slots are not consecutive", ps[i].slot, ps.front().slot);
            }
        }
}

int check_partition() {
    Lcg rng(2024);
    const int hxs[] = {1, 2, 3, 4, 8, 16, 24};
    const int wgs[] = {1, 2, 5, 8, 64, 100, 256, 512, 1024, 2048};
    int cases = 0;
    for (int i = 0; i < 2500; ++i) {
        const int batch = i % 5 == 0 ? rng.range(60, 150) : rng.range(1, 40);
        const int hx = hxs[rng.next() % 7];
        const int num_wgs = wgs[rng.next() % 10];
        const int max_kv_len = i % 7 == 0 ? rng.range(0, 40) : rng.range(0, 6000);
        std::vector<int32_t> lens(batch);
        for (auto &n : lens) {
            const int r = rng.range(0, 9);
            n = r == 0 ? 0 : (r == 1 ? rng.range(-5, -1) : (r == 2 ? max_kv_len + rng.range(0, 9)
                                                                    : rng.range(0, max_kv_len)));
        }
        long long total = 0;
        for (int b = 0; b < batch; ++b)
            total += fd::unit_cost(lens.data(), b, max_kv_len);
        check_partition_case(lens, max_kv_len, hx, num_wgs, total * hx <= 20000);
        ++cases;
    }
    return cases;
}

void check_named_plans() {
    struct W {
        int batch, hq, hkv, n, d, dt, lens, B;
    } ws[] = {{1, 1, 1, 1024, 64, FD_F32, 0, 4},
              {8, 32, 32, 4096, 128, FD_BF16, 0, 0},
              {1, 32, 32, 65536, 128, FD_BF16, 0, 0},
              {16, 64, 8, 32768, 128, FD_BF16, 1, 0},
              {4, 16, 16, 131072, 256, FD_F16, 0, 0}};
    for (const W &w : ws) {
        fd_plan p;
        if (fd_decode_plan(w.batch, w.hq, w.hkv, w.n, w.d, w.dt, w.lens, 0, w.B, 0, 256, &p) !=
            FD_OK)
            fail("named workload has no plan", w.batch, w.hq);
        size_t bytes = 0;
        if (fd_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.n, w.d, w.dt, w.lens, w.B, 0,
                                      &bytes) != FD_OK || bytes != p.workspace_bytes)
            fail("workspace size differs from the plan's", (long long)bytes,
                 (long long)p.workspace_bytes);
        std::printf("plan b%d hq%d hkv%d n%d d%d: route %d kernel %d B %d L %d waves %d grid "
                    "%lld ws %zu\n",
                    w.batch, w.hq, w.hkv, w.n, w.d, p.route, p.kernel, p.num_splits, p.split_len,
                    p.waves_per_group, (long long)p.work_groups, p.workspace_bytes);
    }
}

void check_decode_through_stubs() {
    // the ragged grouped-query workload's shape with seeded lengths (host memory)
    Lcg rng(4);
    const int batch = 16, hq = 64, hkv = 8, d = 128;
    std::vector<int32_t> lens(batch);
    int n_max = 0;
    for (auto &n : lens) {
        n = rng.range(512, 32768);
        n_max = std::max(n_max, n);
    }
    size_t bytes = 0;
    if (fd_decode_workspace_bytes(batch, hq, hkv, n_max, d, FD_BF16, 1, 0, 0, &bytes) != FD_OK)
        fail("no workspace size");
    std::vector<char> ws(bytes + 256);
    char *ws0 = ws.data() + (256 - ((uintptr_t)ws.data() & 255));
    HostLaunchLog &log = host_launch_log();
    log.workspace_end = ws0 + bytes;
    alignas(256) static char fake[256];
    const long long before = log.balanced;
    if (fd_decode(fake, fake, fake, lens.data(), batch, hq, hkv, n_max, d, FD_BF16, FD_BF16,
                  0.0883883f, 0, 0, fake, (float *)fake, ws0, bytes, nullptr) != FD_OK)
        fail(fd_last_error());
    if (log.balanced != before + 1 || log.pieces == 0)
        fail("fd_decode did not take the balanced route", log.balanced, log.pieces);
    // cascade: a shared prefix plus ragged suffixes
    std::vector<int32_t> suf(batch);
    int s_max = 0;
    for (auto &n : suf) {
        n = rng.range(0, 4096);
        s_max = std::max(s_max, n);
    }
    if (fd_cascade_workspace_bytes(batch, hq, hkv, 16384, s_max, d, FD_BF16, 1, &bytes) != FD_OK)
        fail(fd_last_error());
    std::vector<char> cws(bytes + 256);
    char *c0 = cws.data() + (256 - ((uintptr_t)cws.data() & 255));
    log.workspace_end = c0 + bytes;
    if (fd_decode_cascade(fake, fake, fake, 16384, fake, fake, suf.data(), batch, hq, hkv, s_max,
                          d, FD_BF16, FD_BF16, 0.0883883f, fake, (float *)fake, c0, bytes,
                          nullptr) != FD_OK)
        fail(fd_last_error());
    // ragged multi-head and fp32 grouped batches: the balanced partition on the
    // vector kernel, one unit per (sequence, query head); and a cascade whose
    // ragged suffixes take it
    struct V {
        int hq, hkv, d, dt;
    } vs[] = {{32, 32, 128, FD_BF16}, {16, 16, 256, FD_F16}, {8, 2, 64, FD_F32}};
    for (const V &v : vs) {
        if (fd_decode_workspace_bytes(batch, v.hq, v.hkv, n_max, v.d, v.dt, 1, 0, 0, &bytes) !=
            FD_OK)
            fail(fd_last_error());
        std::vector<char> vws(bytes + 256);
        char *v0 = vws.data() + (256 - ((uintptr_t)vws.data() & 255));
        log.workspace_end = v0 + bytes;
        const long long b0 = log.balanced, s0 = log.split_valu;
        if (fd_decode(fake, fake, fake, lens.data(), batch, v.hq, v.hkv, n_max, v.d, v.dt, v.dt,
                      0.1f, 0, 0, fake, (float *)fake, v0, bytes, nullptr) != FD_OK)
            fail(fd_last_error());
        if (log.balanced != b0 + 1 || log.split_valu != s0 + 1)
            fail("fd_decode did not take the balanced vector route", v.hq, v.hkv);
    }
    if (fd_cascade_workspace_bytes(batch, 32, 32, 4096, s_max, 128, FD_BF16, 1, &bytes) != FD_OK)
        fail(fd_last_error());
    std::vector<char> mws(bytes + 256);
    char *m0 = mws.data() + (256 - ((uintptr_t)mws.data() & 255));
    log.workspace_end = m0 + bytes;
    const long long vb0 = log.balanced;
    if (fd_decode_cascade(fake, fake, fake, 4096, fake, fake, suf.data(), batch, 32, 32, s_max,
                          128, FD_BF16, FD_BF16, 0.0883883f, fake, (float *)fake, m0, bytes,
                          nullptr) != FD_OK)
        fail(fd_last_error());
    if (log.balanced != vb0 + 1)
        fail("multi-head cascade suffix did not take the balanced route", log.balanced);
    log.workspace_end = nullptr;
    // an undersized workspace is refused before any launch
    const long long launched = log.split_mfma;
    if (fd_decode(fake, fake, fake, lens.data(), batch, hq, hkv, n_max, d, FD_BF16, FD_BF16,
                  0.0883883f, 0, 0, fake, nullptr, ws0, 256, nullptr) != FD_ERR_WORKSPACE ||
        log.split_mfma != launched)
        fail("undersized workspace not refused");
}

}  // namespace

int main() {
    const int cases = check_partition();
    std::printf("partition: %d random cases passed\n", cases);
    check_named_plans();
    check_decode_through_stubs();
    const HostLaunchLog &log = host_launch_log();
    std::printf("stub launches: vector %lld, matrix-core %lld (balanced %lld, pieces %lld), "
                "combine %lld\n",
                log.split_valu, log.split_mfma, log.balanced, log.pieces, log.combine);
    std::printf("host checks passed\n");
    return 0;
}
