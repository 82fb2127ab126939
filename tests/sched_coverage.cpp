// Checks the attention kernel's work schedule (csrc/schedule.h, the function
// the kernel runs) on the host: for each geometry, with P workgroups as the
// library launches them (min(items, compute units)), every work item is taken
// exactly once; in the XCD-grouped form every item of KV head c runs on one
// of that head's XCDs (workgroup b on XCD b % 8); and the busiest workgroup's
// load (key tiles walked plus 14 per item for its prologue and epilogue) is
// reported beside the mean.  Exit status 0 when every check holds.
#include "schedule.h"

#include <algorithm>
#include <cstdio>
#include <vector>

static int failures = 0;
#define CHECK(c, ...) do { if (!(c)) { ++failures; std::printf("FAIL: " __VA_ARGS__); std::printf("\n"); } } while (0)

// Key tiles walked by row block rb (causal pass over T keys from q_base).
static int tiles_of(int rb, int T, int q_base)
{
    const int p0 = q_base + 64 * rb;
    const int last = std::min(p0 + 63, T - 1);
    return last / 32 + 1;
}

static void check(int T, int q_base, int Hq, int Hkv, int cus, bool print)
{
    const int S = T - q_base, G = Hq / Hkv, n_hg = (G + 3) / 4, nrb = (S + 63) / 64;
    const long items = (long)nrb * Hkv * n_hg;
    const int P = (int)std::min<long>(items, cus);
    std::vector<int> seen((size_t)items, 0);
    std::vector<long> load(P, 0);
    const bool grouped = ga::sched_xcd_grouped(P, Hkv);
    for (int b = 0; b < P; ++b) {
        bool ended = false;
        for (int pass = 0; pass < 1 + (int)(items / P) + 2; ++pass) {
            ga::SchedItem it;
            const bool ok = ga::sched_item(b, P, pass, nrb, Hkv, n_hg, it);
            if (!ok) { ended = true; continue; }
            CHECK(!ended, "T=%d Hkv=%d: workgroup %d gets an item after its last", T, Hkv, b);
            CHECK(it.rbi >= 0 && it.rbi < nrb && it.kvh >= 0 && it.kvh < Hkv && it.hg >= 0 && it.hg < n_hg,
                  "T=%d Hkv=%d: item out of range (%d %d %d)", T, Hkv, it.rbi, it.kvh, it.hg);
            if (it.rbi < 0 || it.rbi >= nrb || it.kvh < 0 || it.kvh >= Hkv || it.hg < 0 || it.hg >= n_hg)
                continue;
            ++seen[((size_t)it.rbi * Hkv + it.kvh) * n_hg + it.hg];
            if (grouped)
                CHECK((b % 8) / (8 / Hkv) == it.kvh, "T=%d Hkv=%d: KV head %d on XCD %d", T, Hkv, it.kvh, b % 8);
            load[b] += tiles_of(nrb - 1 - it.rbi, T, q_base) + 14;
        }
    }
    long total = 0;
    for (size_t i = 0; i < seen.size(); ++i)
        CHECK(seen[i] == 1, "T=%d q_base=%d Hq=%d Hkv=%d cus=%d: item %zu taken %d times", T, q_base, Hq, Hkv, cus,
              i, seen[i]);
    long xcd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int b = 0; b < P; ++b) {
        total += load[b];
        xcd[b % 8] += load[b];
    }
    if (print)
        std::printf("T=%5d q_base=%4d %2d/%-2d cus=%3d: %5ld items on %3d workgroups (%s): busiest %ld, mean %.1f; "
                    "busiest XCD %ld, mean %.1f\n",
                    T, q_base, Hq, Hkv, cus, items, P, grouped ? "XCD-grouped" : "plain",
                    *std::max_element(load.begin(), load.end()), (double)total / P,
                    *std::max_element(xcd, xcd + 8), (double)total / std::min(P, 8));

    // The halves table (sched_plan_halves over every compute unit): every
    // item's two 32-row halves taken exactly once (a whole item takes both),
    // each KV head on its XCDs, no split of a block of 32 rows or fewer, and
    // the busiest load it reports is the one its entries give.
    {
        std::vector<int> rows(nrb), tl(nrb), split;
        for (int rbi = 0; rbi < nrb; ++rbi) {
            rows[rbi] = std::min(64, S - 64 * (nrb - 1 - rbi));
            tl[rbi] = tiles_of(nrb - 1 - rbi, T, q_base);
        }
        long hb = -1;
        const bool sp = ga::sched_plan_halves(cus, nrb, Hkv, n_hg, tl.data(), rows.data(), 14, split, &hb);
        if (sp) {
            CHECK(ga::sched_xcd_grouped(cus, Hkv), "T=%d Hkv=%d cus=%d: halves table without XCD grouping", T, Hkv,
                  cus);
            std::vector<int> halves((size_t)items * 2, 0);
            CHECK((int)split.size() >= cus + 1 && split[0] == 0, "T=%d Hkv=%d: halves table offsets", T, Hkv);
            int n_split = 0, max_per = 0;
            long busiest = 0;
            for (int b = 0; b < cus && (int)split.size() >= cus + 1; ++b) {
                long ld = 0;
                max_per = std::max(max_per, split[b + 1] - split[b]);
                for (int o = split[b]; o < split[b + 1]; ++o) {
                    const ga::SchedItem it = ga::sched_unpack(split[cus + 1 + o]);
                    const bool ok = it.rbi >= 0 && it.rbi < nrb && it.kvh >= 0 && it.kvh < Hkv && it.hg >= 0 &&
                                    it.hg < n_hg && it.half >= 0 && it.half <= 2;
                    CHECK(ok, "T=%d Hkv=%d: halves table item out of range", T, Hkv);
                    if (!ok)
                        continue;
                    CHECK((b % 8) / (8 / Hkv) == it.kvh, "T=%d Hkv=%d: halves table puts KV head %d on XCD %d", T,
                          Hkv, it.kvh, b % 8);
                    const size_t i = ((size_t)it.rbi * Hkv + it.kvh) * n_hg + it.hg;
                    if (it.half != 2)
                        ++halves[2 * i];
                    if (it.half != 1)
                        ++halves[2 * i + 1];
                    const long w = tl[it.rbi] + 14;
                    ld += it.half ? ga::sched_half_weight(w) : w;
                    if (it.half == 1) {
                        ++n_split;
                        CHECK(rows[it.rbi] > 32, "T=%d Hkv=%d: split of a block with %d rows", T, Hkv, rows[it.rbi]);
                    }
                }
                busiest = std::max(busiest, ld);
            }
            for (size_t i = 0; i < halves.size(); ++i)
                CHECK(halves[i] == 1, "T=%d q_base=%d Hq=%d Hkv=%d cus=%d: half %zu taken %d times", T, q_base, Hq,
                      Hkv, cus, i, halves[i]);
            CHECK(n_split > 0, "T=%d Hkv=%d: halves table with no split", T, Hkv);
            CHECK(busiest == hb, "T=%d Hkv=%d: halves table reports busiest %ld, entries give %ld", T, Hkv, hb,
                  busiest);
            if (print)
                std::printf("    halves table: %d of %ld items split, busiest %ld, up to %d entries a workgroup\n",
                            n_split, items, busiest, max_per);
        }
        // A 2048-token pass with 24 / 2 heads on 256 compute units gets one.
        if (T == 2048 && q_base == 0 && Hq == 24 && Hkv == 2 && cus == 256)
            CHECK(sp, "T=2048 24/2 on 256 compute units: no halves table");
    }

    // The host table (sched_plan), when it is more even than the snake.
    std::vector<int> tiles(nrb);
    for (int rbi = 0; rbi < nrb; ++rbi)
        tiles[rbi] = tiles_of(nrb - 1 - rbi, T, q_base);
    std::vector<int> table;
    long bs = 0, bt = 0;
    const bool use = ga::sched_plan(P, nrb, Hkv, n_hg, tiles.data(), 14, table, &bs, &bt);
    CHECK(bs == *std::max_element(load.begin(), load.end()), "T=%d Hkv=%d: plan's snake busiest %ld", T, Hkv, bs);
    if (!use) {
        CHECK(table.empty() && bt == bs, "T=%d Hkv=%d: table returned with the snake kept", T, Hkv);
        if (print)
            std::printf("    table: none\n");
        return;
    }
    CHECK(bt < bs, "T=%d Hkv=%d: table not more even (%ld vs %ld)", T, Hkv, bt, bs);
    CHECK((long)table.size() == P + 1 + items, "T=%d Hkv=%d: table size %zu", T, Hkv, table.size());
    if ((long)table.size() != P + 1 + items)
        return;
    std::vector<int> seen2((size_t)items, 0);
    long tmax = 0;
    CHECK(table[0] == 0 && table[P] == items, "T=%d Hkv=%d: table offsets", T, Hkv);
    for (int b = 0; b < P; ++b) {
        CHECK(table[b] <= table[b + 1], "T=%d Hkv=%d: offsets of workgroup %d", T, Hkv, b);
        long l = 0;
        for (int o = table[b]; o < table[b + 1]; ++o) {
            const ga::SchedItem it = ga::sched_unpack(table[P + 1 + o]);
            const bool ok = it.rbi >= 0 && it.rbi < nrb && it.kvh >= 0 && it.kvh < Hkv && it.hg >= 0 && it.hg < n_hg;
            CHECK(ok, "T=%d Hkv=%d: table item out of range", T, Hkv);
            if (!ok)
                continue;
            ++seen2[((size_t)it.rbi * Hkv + it.kvh) * n_hg + it.hg];
            if (grouped)
                CHECK((b % 8) / (8 / Hkv) == it.kvh, "T=%d Hkv=%d: table puts KV head %d on XCD %d", T, Hkv, it.kvh,
                      b % 8);
            l += tiles[it.rbi] + 14;
        }
        tmax = std::max(tmax, l);
    }
    for (size_t i = 0; i < seen2.size(); ++i)
        CHECK(seen2[i] == 1, "T=%d q_base=%d Hq=%d Hkv=%d cus=%d: table item %zu taken %d times", T, q_base, Hq, Hkv,
              cus, i, seen2[i]);
    CHECK(tmax == bt, "T=%d Hkv=%d: table busiest %ld, reported %ld", T, Hkv, tmax, bt);
    if (print)
        std::printf("    table: busiest %ld (snake %ld)\n", bt, bs);
}

int main()
{
    // The workloads (printed), then a sweep of shapes and launch sizes.
    check(64, 0, 24, 2, 256, true);
    check(2048, 0, 24, 2, 256, true);
    check(8192, 0, 16, 4, 256, true);
    check(8192, 1024, 24, 2, 256, true);
    check(8192, 0, 24, 2, 256, true);
    check(32768, 0, 4, 1, 256, true);
    const int Ts[] = {1, 31, 32, 33, 64, 65, 127, 128, 200, 511, 700, 2048, 4097, 8192, 16385, 32768};
    const int geo[][2] = {{24, 2}, {16, 4}, {4, 1}, {2, 2}, {32, 2}, {6, 1}, {12, 12}, {8, 8}, {16, 16}, {24, 3}, {48, 6}};
    const int cus[] = {256, 304, 80, 32, 8, 1};
    for (int T : Ts)
        for (auto &g : geo)
            for (int c : cus)
                for (int qb : {0, 128, 1024})
                    if (qb < T)
                        check(T, qb, g[0], g[1], c, false);
    std::printf("%s\n", failures ? "FAILED" : "schedule ok");
    return failures ? 1 : 0;
}
