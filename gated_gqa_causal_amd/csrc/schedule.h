// schedule.h -- which work item a workgroup of the attention kernel takes on
// each pass (used by the kernel; a CPU test builds it to check coverage).
//
// A work item is (64-row block, KV head, group of 4 query heads).  Row blocks
// are indexed heaviest first (rbi = 0 is the longest key walk).  The launch has
// P <= compute units workgroups; each takes one item per pass in a snake
// order (b, 2P-1-b, 2P+b, ...), so every pass pairs the heavy end of the list
// with the light end and the workgroups' totals stay level.
//
// Workgroups are dealt to the chip's eight XCDs in turn (workgroup b on XCD
// b % 8), each XCD with its own L2.  When the KV heads divide the XCDs evenly
// (Hkv in {1, 2, 4, 8}) and P is a multiple of 8, the items of KV head c go
// to that head's 8/Hkv XCDs only, so its K/V tiles are fetched into those L2s
// alone.  Within a head, the snake runs over slots u = 0 .. Q-1 (Q = the
// head's workgroups), and a slot's XCD is chosen so that the head groups of
// one row block (n_hg consecutive slots, taking consecutive items) sit on one
// XCD, walking the same tiles side by side, while successive row blocks go to
// the head's XCDs in turn (each XCD gets heavy and light walks alike; a
// contiguous share per XCD would give one XCD every heavy walk).  Otherwise
// items are numbered (row block, KV head, head group), head group fastest,
// over all workgroups.  Either way every item is taken exactly once, and what
// an item computes does not depend on which workgroup takes it.
//
// A launch may instead carry a table made on the host by sched_plan (below):
// per workgroup, the items it takes in order.  The snake keeps two rounds of
// items level but not a third partial one (672 items on 256 workgroups: the
// 160 that take a third item end up about 13% above the mean); the table
// packs each KV head's row blocks into that head's workgroups by first-fit
// decreasing against the smallest capacity that fits them all.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

namespace ga {

struct SchedItem {
    int rbi;    // row block, heaviest first
    int kvh;    // KV head
    int hg;     // group of four query heads
    int half;   // 0: the block's 64 rows; 1 / 2: only rows 0..31 / 32..63 (a split item)
};

__host__ __device__ inline bool sched_xcd_grouped(int P, int Hkv)
{
    return P % 8 == 0 && Hkv >= 1 && Hkv <= 8 && 8 % Hkv == 0;
}

// XCD-grouped form: the slot u (0 .. P/Hkv - 1) of workgroup b among the
// workgroups of its KV head (b % 8) / (8 / Hkv).  The first W1 = W - W % n_hg
// workgroups of every XCD (W = P / 8 on each) hold units of n_hg slots, unit
// t on the head's XCD t % (8 / Hkv); the rest take the last slots in turn.
__host__ __device__ inline int sched_slot(int b, int P, int Hkv, int n_hg)
{
    const int x = b % 8, k = b / 8, W = P / 8, xh = 8 / Hkv;
    const int W1 = W - W % n_hg, xp = x % xh;
    return (k < W1) ? ((k / n_hg) * xh + xp) * n_hg + k % n_hg : xh * W1 + (k - W1) * xh + xp;
}

// Item of workgroup b (of P) on pass `pass`; false once b has no more items
// (then on every later pass too).
__host__ __device__ inline bool sched_item(int b, int P, int pass, int nrb, int Hkv, int n_hg, SchedItem &it)
{
    if (sched_xcd_grouped(P, Hkv)) {
        const int x = b % 8, xh = 8 / Hkv;
        const int Q = xh * (P / 8);                     // workgroups of one KV head
        const int u = sched_slot(b, P, Hkv, n_hg);
        const int j = pass * Q + ((pass & 1) ? Q - 1 - u : u);
        if (j >= nrb * n_hg)
            return false;
        it.kvh = x / xh;
        it.rbi = j / n_hg;
        it.hg = j % n_hg;
        it.half = 0;
        return true;
    }
    const int per_rb = Hkv * n_hg;
    const int item = pass * P + ((pass & 1) ? P - 1 - b : b);
    if (item >= nrb * per_rb)
        return false;
    const int rem = item % per_rb;
    it.rbi = item / per_rb;
    it.kvh = rem / n_hg;
    it.hg = rem % n_hg;
    it.half = 0;
    return true;
}

// A table entry: the item packed into one int (n_hg <= 4 leaves bits 4..5 of
// the low byte for the half).
__host__ __device__ inline int sched_pack(int rbi, int kvh, int hg, int half = 0)
{
    return (rbi << 16) | (kvh << 8) | (half << 4) | hg;
}
__host__ __device__ inline SchedItem sched_unpack(int e)
{
    return SchedItem{e >> 16, (e >> 8) & 0xff, e & 0xf, (e >> 4) & 3};
}

// Host only.  A table for the launch (P workgroups, nrb row blocks, Hkv KV
// heads, n_hg head groups) when it is more even than the snake: weight of an
// item = tiles[rbi] (key tiles its row block walks) + overhead (its prologue
// and epilogue in tile units).  Per KV head in the XCD-grouped form (the
// whole launch otherwise, item by item), row blocks heaviest first go to the
// first unit with room under a capacity C: a unit is n_hg workgroups of
// consecutive slots on one XCD (sched_slot's units), which take the row
// block's n_hg items side by side as the snake does; a row block no unit has
// room for goes item by item to the head's remaining workgroups.  C is the
// smallest capacity that fits everything (binary search from max(heaviest
// item, mean) up to the snake's busiest).  table = P + 1 offsets, then per
// workgroup its entries (sched_pack) in walk order.  Returns false, table
// empty, when the snake's busiest workgroup is no heavier than the table's
// would be; *busiest_snake and *busiest_table report the busiest load of the
// snake and of the schedule kept (in weight units).
inline bool sched_plan(int P, int nrb, int Hkv, int n_hg, const int *tiles, int overhead, std::vector<int> &table,
                       long *busiest_snake = nullptr, long *busiest_table = nullptr)
{
    table.clear();
    if (P <= 0 || nrb <= 0)
        return false;
    const bool grouped = sched_xcd_grouped(P, Hkv);
    const int groups = grouped ? Hkv : 1;
    // The snake's loads.
    std::vector<long> snake(P, 0);
    for (int b = 0; b < P; ++b) {
        SchedItem it;
        for (int pass = 0; sched_item(b, P, pass, nrb, Hkv, n_hg, it); ++pass)
            snake[b] += tiles[it.rbi] + overhead;
    }
    const long snake_max = *std::max_element(snake.begin(), snake.end());
    if (busiest_snake)
        *busiest_snake = snake_max;
    if (busiest_table)
        *busiest_table = snake_max;
    // Workgroups of each group in slot order.
    std::vector<std::vector<int>> wg(groups);
    int g = 1, n_units = P;                              // unit size and units per group
    if (grouped) {
        const int xh = 8 / Hkv, W = P / 8;
        for (int c = 0; c < groups; ++c)
            wg[c].assign(P / Hkv, -1);
        for (int b = 0; b < P; ++b)
            wg[(b % 8) / xh][sched_slot(b, P, Hkv, n_hg)] = b;
        g = n_hg;
        n_units = xh * (W - W % n_hg) / n_hg;
    } else {
        for (int b = 0; b < P; ++b)
            wg[0].push_back(b);
    }
    std::vector<std::vector<int>> bins(P);
    long plan_max = 0;
    for (int c = 0; c < groups; ++c) {
        // Rows: a row block's items of this group placed together (grouped),
        // or single items; heaviest first (rbi ascending is weight descending).
        std::vector<std::vector<int>> rows;
        for (int rbi = 0; rbi < nrb; ++rbi) {
            if (grouped) {
                std::vector<int> r;
                for (int hg = 0; hg < n_hg; ++hg)
                    r.push_back(sched_pack(rbi, c, hg));
                rows.push_back(r);
            } else {
                for (int kvh = 0; kvh < Hkv; ++kvh)
                    for (int hg = 0; hg < n_hg; ++hg)
                        rows.push_back({sched_pack(rbi, kvh, hg)});
            }
        }
        std::stable_sort(rows.begin(), rows.end(), [&](const std::vector<int> &a, const std::vector<int> &b) {
            return tiles[sched_unpack(a[0]).rbi] > tiles[sched_unpack(b[0]).rbi];
        });
        const int Q = (int)wg[c].size();
        long total = 0, heaviest = 0, group_snake = 0;
        for (const auto &r : rows) {
            const long w = tiles[sched_unpack(r[0]).rbi] + overhead;
            total += w * (long)r.size();
            heaviest = std::max(heaviest, w);
        }
        for (int b : wg[c])
            group_snake = std::max(group_snake, snake[b]);
        std::vector<long> load(Q);                       // per slot
        std::vector<std::vector<int>> at(Q);             // entries per slot
        auto fits = [&](long cap) {
            std::fill(load.begin(), load.end(), 0);
            for (auto &a : at)
                a.clear();
            for (const auto &r : rows) {
                const long w = tiles[sched_unpack(r[0]).rbi] + overhead;
                int t = 0;
                while (t < n_units && load[t * g] + w > cap)
                    ++t;
                if (t < n_units && (int)r.size() == g) {
                    for (int i = 0; i < g; ++i) {
                        load[t * g + i] += w;
                        at[t * g + i].push_back(r[i]);
                    }
                    continue;
                }
                for (int e : r) {
                    int q = n_units * g;
                    while (q < Q && load[q] + w > cap)
                        ++q;
                    if (q == Q)
                        return false;
                    load[q] += w;
                    at[q].push_back(e);
                }
            }
            return true;
        };
        long lo = std::max(heaviest, (total + Q - 1) / Q), hi = group_snake;
        if (!fits(hi))
            return false;
        while (lo < hi) {
            const long mid = lo + (hi - lo) / 2;
            if (fits(mid))
                hi = mid;
            else
                lo = mid + 1;
        }
        fits(hi);
        plan_max = std::max(plan_max, *std::max_element(load.begin(), load.end()));
        for (int u = 0; u < Q; ++u)
            bins[wg[c][u]] = at[u];
    }
    if (plan_max >= snake_max)
        return false;
    if (busiest_table)
        *busiest_table = plan_max;
    table.reserve(P + 1 + (size_t)nrb * Hkv * n_hg);
    int off = 0;
    for (int b = 0; b < P; ++b) {
        table.push_back(off);
        off += (int)bins[b].size();
    }
    table.push_back(off);
    for (int b = 0; b < P; ++b)
        table.insert(table.end(), bins[b].begin(), bins[b].end());
    return true;
}

// Host only.  A causal or masked launch with fewer work items than the P workgroups
// (compute units) leaves workgroups idle while the longest walks run.  The
// table gives each workgroup at most one item and splits the heaviest items
// of each KV head into their two 32-row halves (sched_pack half 1 and 2; each
// half runs on one wave per SIMD, about 0.64 of the whole item's time) as far
// as the head's workgroups allow; row blocks with 32 rows or fewer (a ragged
// last block) stay whole.  rows_in_block[rbi] = the block's rows below S.
// Needs the XCD-grouped form (a head's items on its own XCDs); false, table
// empty, when there is nothing to split.
inline bool sched_plan_split(int P, int nrb, int Hkv, int n_hg, const int *rows_in_block, std::vector<int> &table)
{
    table.clear();
    const long items = (long)nrb * Hkv * n_hg;
    if (P <= 0 || items <= 0 || items >= P || !sched_xcd_grouped(P, Hkv))
        return false;
    const int xh = 8 / Hkv, Q = P / Hkv, per_head = nrb * n_hg;
    int splits = Q - per_head;                           // per head
    if (splits <= 0)
        return false;
    std::vector<std::vector<int>> bins(P);
    int done = 0;
    for (int c = 0; c < Hkv; ++c) {
        std::vector<int> wgs;                            // the head's workgroups
        for (int b = 0; b < P; ++b)
            if ((b % 8) / xh == c)
                wgs.push_back(b);
        int u = 0, left = splits;
        for (int rbi = 0; rbi < nrb; ++rbi)              // heaviest first
            for (int hg = 0; hg < n_hg; ++hg) {
                if (left > 0 && rows_in_block[rbi] > 32) {
                    bins[wgs[u++]].push_back(sched_pack(rbi, c, hg, 1));
                    bins[wgs[u++]].push_back(sched_pack(rbi, c, hg, 2));
                    --left;
                    ++done;
                } else {
                    bins[wgs[u++]].push_back(sched_pack(rbi, c, hg, 0));
                }
            }
    }
    if (done == 0)
        return false;
    int off = 0;
    for (int b = 0; b < P; ++b) {
        table.push_back(off);
        off += (int)bins[b].size();
    }
    table.push_back(off);
    for (int b = 0; b < P; ++b)
        table.insert(table.end(), bins[b].begin(), bins[b].end());
    return true;
}

}  // namespace ga
