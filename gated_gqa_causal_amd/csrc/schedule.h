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
// decreasing against the smallest capacity that fits them all.  A table by
// sched_plan_halves may also split items into their two 32-row halves (few
// items per workgroup, the heaviest far above the mean).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <functional>
#include <queue>
#include <utility>
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

// Host only.  Weight of one 32-row half of an item of weight w (key tiles
// plus overhead): a half runs on one wave per SIMD and takes about 0.64 of
// the whole item's time.
inline long sched_half_weight(long w)
{
    return (16 * w + 12) / 25;
}

// Host only.  A table that may split items into their two 32-row halves
// (sched_pack half 1 and 2; a half runs on waves 0..3), for launches whose
// whole items leave the busiest workgroup far above the mean: few items per
// workgroup, the heaviest walking much longer than the rest (a 2048-token
// pass, a short window over a long prefix).  The s heaviest splittable items
// (row blocks of more than 32 rows) are split, and the pieces go, heaviest
// first, to the least loaded of the KV head's P / Hkv workgroups (ties: the
// lowest slot); s is the count that gives the lightest busiest workgroup,
// scanned in steps of about 1/16 of the candidates, then one by one around
// the best step (counts that a lower bound rules out are skipped).  Every KV
// head gets the same plan on its own XCDs (slot q of head c is the head's
// q-th workgroup in index order).  tiles[rbi] and
// rows_in_block[rbi] as for sched_plan; weights in its units.  table = P + 1
// offsets, then per workgroup its entries in walk order (heaviest first);
// *busiest = the plan's busiest load.  Needs the XCD-grouped form and at most
// 2 P / Hkv items per KV head (beyond that whole items pack well and the scan
// would cost more host time); false, table empty, when no split makes the
// busiest workgroup lighter than whole items packed the same way.
inline bool sched_plan_halves(int P, int nrb, int Hkv, int n_hg, const int *tiles, const int *rows_in_block,
                              int overhead, std::vector<int> &table, long *busiest = nullptr)
{
    table.clear();
    if (P <= 0 || nrb <= 0 || n_hg <= 0 || !sched_xcd_grouped(P, Hkv))
        return false;
    const int Q = P / Hkv, xh = 8 / Hkv;
    const long per_head = (long)nrb * n_hg;
    if (per_head > 2L * Q)
        return false;
    struct Item {
        long w;
        int rbi, hg;
    };
    std::vector<Item> items;
    for (int rbi = 0; rbi < nrb; ++rbi)
        for (int hg = 0; hg < n_hg; ++hg)
            items.push_back({(long)tiles[rbi] + overhead, rbi, hg});
    std::stable_sort(items.begin(), items.end(), [](const Item &a, const Item &b) { return a.w > b.w; });
    std::vector<int> splittable;                          // item indices, heaviest first
    for (int i = 0; i < (int)items.size(); ++i)
        if (rows_in_block[items[i].rbi] > 32)
            splittable.push_back(i);
    struct Piece {
        long w;
        int item, half;
    };
    std::vector<Piece> pieces, halves, wholes;
    std::vector<int> slot_of;                             // per piece
    std::vector<std::pair<long, int>> heap;               // (load, slot), least on top
    pieces.reserve(2 * items.size());
    halves.reserve(2 * items.size());
    wholes.reserve(items.size());
    slot_of.reserve(2 * items.size());
    heap.reserve(Q);
    const auto later = std::greater<std::pair<long, int>>();
    // Split the first s splittable items and deal the pieces, heaviest first
    // (the halves and the whole items, each list already in weight order, are
    // merged; a whole item goes first on equal weight); returns the busiest
    // load, or stops as soon as it reaches `limit`.
    auto deal = [&](int s, long limit) {
        halves.clear();
        wholes.clear();
        int k = 0;
        for (int i = 0; i < (int)items.size(); ++i) {
            if (k < s && splittable[k] == i) {
                const long hw = sched_half_weight(items[i].w);
                halves.push_back({hw, i, 1});
                halves.push_back({hw, i, 2});
                ++k;
            } else {
                wholes.push_back({items[i].w, i, 0});
            }
        }
        pieces.resize(halves.size() + wholes.size());
        std::merge(wholes.begin(), wholes.end(), halves.begin(), halves.end(), pieces.begin(),
                   [](const Piece &a, const Piece &b) { return a.w > b.w; });
        // The first Q pieces take slots 0, 1, ... in turn (every load is still
        // 0 when each is dealt, and weights are positive); the rest go through
        // the heap.
        const size_t first = std::min(pieces.size(), (size_t)Q);
        slot_of.assign(pieces.size(), 0);
        heap.clear();
        long mx = 0;
        for (size_t m = 0; m < first; ++m) {
            slot_of[m] = (int)m;
            heap.push_back(std::make_pair(pieces[m].w, (int)m));
            mx = std::max(mx, pieces[m].w);
        }
        if (mx >= limit)
            return mx;
        for (int q = (int)first; q < Q; ++q)
            heap.push_back(std::make_pair(0L, q));
        std::make_heap(heap.begin(), heap.end(), later);
        for (size_t m = first; m < pieces.size(); ++m) {
            std::pop_heap(heap.begin(), heap.end(), later);
            heap.back().first += pieces[m].w;
            slot_of[m] = heap.back().second;
            mx = std::max(mx, heap.back().first);
            if (mx >= limit)
                return mx;
            std::push_heap(heap.begin(), heap.end(), later);
        }
        return mx;
    };
    // A lower bound on the busiest load with s splits (the heaviest piece, and
    // the mean load rounded up): a count whose bound is no lighter than the
    // best load found is not dealt, and dealing stops as soon as it reaches
    // that load.
    const int n_spl = (int)splittable.size();
    std::vector<long> bound(n_spl + 1);
    {
        long total = 0;
        for (const Item &it : items)
            total += it.w;
        int next_whole = 0;                               // first item not split
        std::vector<char> split(items.size(), 0);
        for (int s = 0; s <= n_spl; ++s) {
            if (s > 0) {
                const Item &it = items[splittable[s - 1]];
                total += 2 * sched_half_weight(it.w) - it.w;
                split[splittable[s - 1]] = 1;
            }
            while (next_whole < (int)items.size() && split[next_whole])
                ++next_whole;
            long heaviest = next_whole < (int)items.size() ? items[next_whole].w : 0;
            if (s > 0)
                heaviest = std::max(heaviest, sched_half_weight(items[splittable[0]].w));
            bound[s] = std::max(heaviest, (total + Q - 1) / Q);
        }
    }
    const long whole = deal(0, LONG_MAX);
    long best = whole;
    int best_s = 0;
    auto consider = [&](int s) {
        if (bound[s] >= best)
            return;
        const long m = deal(s, best);
        if (m < best) {
            best = m;
            best_s = s;
        }
    };
    const int step = std::max(1, n_spl / 16);
    for (int s = step; s <= n_spl; s += step)
        consider(s);
    const int lo = std::max(1, best_s - step + 1), hi = std::min(n_spl, best_s + step - 1);
    for (int s = lo; s <= hi; ++s)
        if (s % step != 0)
            consider(s);
    if (best_s == 0 || best >= whole)
        return false;
    deal(best_s, LONG_MAX);
    // Slot q of each head -> its workgroups in index order.
    std::vector<std::vector<int>> wgs(Hkv);
    for (int b = 0; b < P; ++b)
        wgs[(b % 8) / xh].push_back(b);
    std::vector<std::vector<int>> bins(P);
    for (int c = 0; c < Hkv; ++c)
        for (size_t k = 0; k < pieces.size(); ++k) {
            const Item &it = items[pieces[k].item];
            bins[wgs[c][slot_of[k]]].push_back(sched_pack(it.rbi, c, it.hg, pieces[k].half));
        }
    int off = 0;
    for (int b = 0; b < P; ++b) {
        table.push_back(off);
        off += (int)bins[b].size();
    }
    table.push_back(off);
    for (int b = 0; b < P; ++b)
        table.insert(table.end(), bins[b].begin(), bins[b].end());
    if (busiest)
        *busiest = best;
    return true;
}

}  // namespace ga
