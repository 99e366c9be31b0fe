// Host planner of the multi-projection sweep: checks every projection, cuts
// the concatenated 16-row tiles of all projections into workgroup ranges of
// about equal weight bytes, and writes the device table image (header,
// projections, workgroup spans).  Host code only: nothing here touches the
// device.
#include <cstring>
#include <vector>

#include "twd_internal.h"

namespace twd {

namespace {

bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// LDS bytes of one staged token row: whole 256-wide slices, plus 16 bytes so
// that the 16 token rows of a B-operand read fall on different bank groups.
int stride_bytes(int K) { return ((K + 255) / 256) * 256 + 16; }

// Workgroups the planner aims for fill every compute unit with the
// resident waves the kernel is built for, fewer when the list is small, so that each wave
// still gets a few tiles.  A workgroup's staged activations may take its
// share of the compute unit's 160 KiB of LDS before the planner starts a new
// workgroup at a projection boundary (a single projection may take more).
constexpr int64_t kMinTilesPerWave = 2;
constexpr int kLdsHardCap = 160 * 1024;

// Outputs gathered in LDS and written after the stream.  A workgroup's tiles
// of one projection are consecutive, so for each token row its outputs form
// one run of 16 (t1 - t0) values: written at the end, each run goes out as
// whole lines in one pass, instead of 64-byte pieces of 16 token rows
// interleaved with the weight stream.  A workgroup keeps its outputs in LDS
// beside its staged activations: as the fp32 y (and int32 acc) values where
// all of them fit, else as each output's accumulator cut to 24 bits
// (|acc| <= 127 K < 2^20 for K <= 8192), three bytes instead of four for y
// or eight for acc and y, from which the write-out recomputes y exactly as
// the epilogue does -- for every tile where they fit, else for each span's
// first tiles, as many as fit, span after span, the later tiles storing in
// the stream.  (The packed form costs the write-out about 1 us at M = 4,
// where the fp32 values fit, so it is used only where they do not.)
int lay_out_deferred(SweepWork &w, const std::vector<SweepProj> &P, int m, int staged_end) {
    const int base = (staged_end + 15) & ~15;
    int off = base;
    for (int s = 0; s < w.nspan; ++s) {  // fp32 y and int32 acc rows
        SweepSpan &sp = w.span[s];
        const SweepProj &d = P[sp.q];
        const int bytes = 4 * m * 16 * (sp.t1 - sp.t0);
        sp.yoff = d.y ? off : -1;
        off += d.y ? bytes : 0;
        sp.aoff = d.acc ? off : -1;
        off += d.acc ? bytes : 0;
    }
    if (off <= kLdsHardCap) {
        w.defer = 1;
        return off;
    }
    off = base;
    int deferred = 0;
    const int per_tile = 3 * m * 16;  // a multiple of 16
    for (int s = 0; s < w.nspan; ++s) {  // 24-bit accumulators, as many tiles as fit
        SweepSpan &sp = w.span[s];
        const SweepProj &d = P[sp.q];
        sp.aoff = -1;
        const int room = kLdsHardCap - off;
        int nd = d.y || d.acc ? (room > 0 ? room / per_tile : 0) : 0;
        nd = nd < sp.t1 - sp.t0 ? nd : sp.t1 - sp.t0;
        sp.nd = nd;
        sp.yoff = nd > 0 ? off : -1;
        off += nd * per_tile;
        deferred += nd;
    }
    if (deferred > 0) {
        w.defer = 2;
        return off;
    }
    w.defer = 0;
    for (int s = 0; s < w.nspan; ++s)
        w.span[s].yoff = w.span[s].aoff = -1;
    return staged_end;
}

uint32_t fnv1a(const uint8_t *p, size_t n) {
    uint32_t h = 2166136261u;
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 16777619u;
    }
    return h;
}

twd_status check_proj(const twd_sweep_proj &p, int i, int64_t *N_out) {
    if (p.nseg < 1 || p.nseg > TWD_MAX_SEGMENTS)
        return set_error(TWD_ERR_INVALID_ARG, "sweep: projection %d has nseg=%lld", i,
                         (long long)p.nseg);
    int64_t N = 0;
    for (int s = 0; s < p.nseg; ++s) {
        if (p.seg_rows[s] < 0)
            return set_error(TWD_ERR_INVALID_ARG, "sweep: projection %d seg_rows[%d] < 0", i, s);
        N += p.seg_rows[s];
        if (N > (int64_t(1) << 30))
            return set_error(TWD_ERR_UNSUPPORTED, "sweep: projection %d has N > 2^30", i);
    }
    if (p.K < 64 || p.K > TWD_MAX_K || p.K % 64 != 0)
        return set_error(TWD_ERR_UNSUPPORTED,
                         "sweep: projection %d K=%lld must be a multiple of 64 in 64..%d", i,
                         (long long)p.K, TWD_MAX_K);
    *N_out = N;
    if (N == 0)
        return TWD_OK;
    if (!p.wpacked || !p.x_bf16)
        return set_error(TWD_ERR_INVALID_ARG, "sweep: projection %d has a null input", i);
    if (!p.acc && !p.y)
        return set_error(TWD_ERR_INVALID_ARG, "sweep: projection %d has no output", i);
    if (!aligned(p.wpacked, 16) || !aligned(p.x_bf16, 16))
        return set_error(TWD_ERR_INVALID_ARG,
                         "sweep: projection %d weights and activations must be 16-byte aligned",
                         i);
    if ((p.acc && !aligned(p.acc, 4)) || (p.y && !aligned(p.y, 4)))
        return set_error(TWD_ERR_INVALID_ARG, "sweep: projection %d outputs must be 4-byte aligned",
                         i);
    return TWD_OK;
}

}  // namespace

twd_status sweep_plan(const twd_sweep_proj *projs, int nproj, int64_t M, const void *table_dev,
                      void *table_host, int64_t table_bytes, int64_t *bytes_needed,
                      twd_sweep_plan *plan) {
    if (!projs || nproj < 1 || nproj > 65536)
        return set_error(TWD_ERR_INVALID_ARG, "sweep: need 1..65536 projections");
    if (M < 1 || M > TWD_MAX_M)
        return set_error(TWD_ERR_UNSUPPORTED, "sweep: M=%lld outside 1..%d", (long long)M,
                         TWD_MAX_M);
    const int m = static_cast<int>(M);

    std::vector<SweepProj> P(nproj);
    int64_t total = 0, tiles_total = 0;
    for (int i = 0; i < nproj; ++i) {
        int64_t N = 0;
        twd_status st = check_proj(projs[i], i, &N);
        if (st != TWD_OK)
            return st;
        SweepProj &d = P[i];
        std::memset(&d, 0, sizeof d);
        d.w = projs[i].wpacked;
        d.x = projs[i].x_bf16;
        d.acc = projs[i].acc;
        d.y = projs[i].y;
        d.K = static_cast<int>(projs[i].K);
        d.N = static_cast<int>(N);
        d.slices = (d.K + 255) / 256;
        d.passes = (d.slices + kSweepLP - 1) / kSweepLP;
        d.stride = stride_bytes(d.K);
        d.segs.nseg = static_cast<int>(projs[i].nseg);
        int64_t b = 0;
        for (int s = 0; s < d.segs.nseg; ++s) {
            b += projs[i].seg_rows[s];
            d.segs.bound[s] = static_cast<int>(b);
            d.segs.gamma[s] = projs[i].seg_gamma[s];
        }
        if (kSweepLdsHeader + m * d.stride > kLdsHardCap)
            return set_error(TWD_ERR_UNSUPPORTED,
                             "sweep: projection %d: M=%d rows of K=%d do not fit in LDS", i, m,
                             d.K);
        total += N * d.K / 4;
        tiles_total += (N + 15) / 16;
    }

    // Cut the tile sequence: a tile goes to the range of its first byte, and
    // a new workgroup also starts where one more projection would exceed the
    // span count or the LDS cap.
    const int nw = sweep_waves(m);
    const int cu_waves = 4 * sweep_simd_waves(m);
    const int64_t target = int64_t(kSweepCUs) * cu_waves / nw;
    const int lds_soft = kLdsHardCap * nw / cu_waves;
    int64_t groups = tiles_total / (kMinTilesPerWave * nw);
    groups = groups < 1 ? 1 : groups > target ? target : groups;
    std::vector<SweepWork> work;
    int lds_max = kSweepLdsHeader;
    // Where two neighbouring projections cannot be staged by one workgroup
    // (their rows exceed the LDS share together), a range must end between
    // them.  Such boundaries cut the list into segments, and each segment
    // gets a whole number of ranges in proportion to its bytes: ranges are
    // handed out one at a time to the segment with the most bytes per range.
    std::vector<int> seg_of(nproj);
    std::vector<int64_t> seg_bytes;
    {
        int prev = -1;
        for (int q = 0; q < nproj; ++q) {
            const int64_t b = static_cast<int64_t>(P[q].N) * P[q].K / 4;
            if (b == 0) {
                seg_of[q] = seg_bytes.empty() ? 0 : static_cast<int>(seg_bytes.size()) - 1;
                continue;
            }
            const bool forced = prev < 0 || kSweepLdsHeader + m * P[prev].stride +
                                                    m * P[q].stride > lds_soft;
            if (forced)
                seg_bytes.push_back(0);
            seg_of[q] = static_cast<int>(seg_bytes.size()) - 1;
            seg_bytes.back() += b;
            prev = q;
        }
        if (seg_bytes.empty())
            seg_bytes.push_back(0);
    }
    const int nsegs = static_cast<int>(seg_bytes.size());
    std::vector<int64_t> seg_ranges(nsegs), seg_base(nsegs);
    auto apportion = [&](int64_t g) {
        for (int i = 0; i < nsegs; ++i)
            seg_ranges[i] = 1;
        for (int64_t left = g - nsegs; left > 0; --left) {
            int best = 0;
            for (int i = 1; i < nsegs; ++i)  // bytes / ranges, compared exactly
                if (seg_bytes[i] * seg_ranges[best] > seg_bytes[best] * seg_ranges[i])
                    best = i;
            ++seg_ranges[best];
        }
        int64_t base = 0;
        for (int i = 0; i < nsegs; ++i) {
            seg_base[i] = base;
            base += seg_ranges[i];
        }
    };
    // Cut the tiles into about `g` ranges (per segment, of about equal
    // bytes); a range also closes early at the span or LDS limit, which adds
    // workgroups.
    auto cut = [&](int64_t g) {
        apportion(g);
        work.clear();
        lds_max = kSweepLdsHeader;
        SweepWork cur;
        std::memset(&cur, 0, sizeof cur);
        int cur_lds = kSweepLdsHeader;
        int64_t cur_target = -1;
        int64_t cum = 0;  // bytes before this tile in its segment
        int seg = -1;
        auto close = [&]() {
            if (cur.nspan > 0) {
                const int end = lay_out_deferred(cur, P, m, cur_lds);
                work.push_back(cur);
                if (end > lds_max)
                    lds_max = end;
            }
            std::memset(&cur, 0, sizeof cur);
            cur_lds = kSweepLdsHeader;
        };
        for (int q = 0; q < nproj; ++q) {
            const SweepProj &d = P[q];
            const int tiles = (d.N + 15) / 16;
            if (tiles > 0 && seg_of[q] != seg) {
                seg = seg_of[q];
                cum = 0;
            }
            for (int t = 0; t < tiles; ++t) {
                const int64_t sb = seg_bytes[seg];
                const int64_t range =
                    seg_base[seg] + (sb > 0 ? cum * seg_ranges[seg] / sb : 0);
                if (range != cur_target) {
                    close();
                    cur_target = range;
                }
                SweepSpan *last = cur.nspan ? &cur.span[cur.nspan - 1] : nullptr;
                if (!last || last->q != q) {
                    const int need = m * d.stride;
                    if (cur.nspan == kSweepMaxSpans ||
                        (cur.nspan > 0 && cur_lds + need > lds_soft))
                        close();
                    SweepSpan &sp = cur.span[cur.nspan++];
                    sp.q = q;
                    sp.t0 = t;
                    sp.t1 = t;
                    sp.xoff = cur_lds - kSweepLdsHeader;
                    cur_lds += need;
                    last = &sp;
                }
                last->t1 = t + 1;
                const int rows = d.N - 16 * t < 16 ? d.N - 16 * t : 16;
                cum += static_cast<int64_t>(rows) * d.K / 4;
            }
        }
        close();
    };
    // Workgroups past the resident count would run as a second round after
    // the first ones finish, so where the early closes push the count past
    // it, take the largest number of byte ranges that keeps it resident
    // (the count grows with g, so a bisection finds it).
    cut(groups);
    if (static_cast<int64_t>(work.size()) > target && groups > 1) {
        int64_t lo = 1, hi = groups - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            cut(mid);
            if (static_cast<int64_t>(work.size()) <= target)
                lo = mid;
            else
                hi = mid - 1;
        }
        cut(lo);
    }
    if (work.empty()) {
        // every projection is empty: one workgroup that stages nothing
        SweepWork w;
        std::memset(&w, 0, sizeof w);
        work.push_back(w);
    }

    const int64_t proj_off = kSweepHeaderBytes;
    const int64_t work_off = proj_off + static_cast<int64_t>(nproj) * sizeof(SweepProj);
    const int64_t need = work_off + static_cast<int64_t>(work.size()) * sizeof(SweepWork);
    if (need > (int64_t(1) << 31))
        return set_error(TWD_ERR_UNSUPPORTED, "sweep: table larger than 2 GiB");
    if (bytes_needed)
        *bytes_needed = need;
    if (!table_host)
        return TWD_OK;
    if (!plan)
        return set_error(TWD_ERR_INVALID_ARG, "sweep: null plan");
    if (!table_dev || !aligned(table_dev, 16))
        return set_error(TWD_ERR_INVALID_ARG, "sweep: the device table must be 16-byte aligned");
    if (table_bytes < need)
        return set_error(TWD_ERR_INVALID_ARG, "sweep: table of %lld bytes, %lld needed",
                         (long long)table_bytes, (long long)need);

    uint8_t *img = static_cast<uint8_t *>(table_host);
    std::memset(img, 0, static_cast<size_t>(need));
    SweepHeader h;
    std::memset(&h, 0, sizeof h);
    h.magic = kSweepMagic;
    h.check = 0;
    h.nproj = nproj;
    h.nwg = static_cast<int>(work.size());
    h.M = m;
    h.lds = lds_max;
    h.proj_off = static_cast<int>(proj_off);
    h.work_off = static_cast<int>(work_off);
    h.weight_bytes = total;
    std::memcpy(img, &h, sizeof h);
    std::memcpy(img + proj_off, P.data(), P.size() * sizeof(SweepProj));
    std::memcpy(img + work_off, work.data(), work.size() * sizeof(SweepWork));
    // the check value covers the whole image (its own field zero) and the
    // device address the image is bound to; never 0
    uint32_t check = fnv1a(img, static_cast<size_t>(need));
    const uintptr_t dev = reinterpret_cast<uintptr_t>(table_dev);
    check = fnv1a(reinterpret_cast<const uint8_t *>(&dev), sizeof dev) ^ check;
    if (check == 0)
        check = 1;
    std::memcpy(img + offsetof(SweepHeader, check), &check, sizeof check);

    std::memset(plan, 0, sizeof *plan);
    plan->table = table_dev;
    plan->table_bytes = need;
    plan->weight_bytes = total;
    plan->nproj = nproj;
    plan->M = m;
    plan->nwg = h.nwg;
    plan->lds_bytes = lds_max;
    plan->check = check;
    return TWD_OK;
}

}  // namespace twd
