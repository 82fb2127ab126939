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
#pragma once

#include <hip/hip_runtime.h>

namespace ga {

struct SchedItem {
    int rbi;    // row block, heaviest first
    int kvh;    // KV head
    int hg;     // group of four query heads
};

__host__ __device__ inline bool sched_xcd_grouped(int P, int Hkv)
{
    return P % 8 == 0 && Hkv >= 1 && Hkv <= 8 && 8 % Hkv == 0;
}

// Item of workgroup b (of P) on pass `pass`; false once b has no more items
// (then on every later pass too).
__host__ __device__ inline bool sched_item(int b, int P, int pass, int nrb, int Hkv, int n_hg, SchedItem &it)
{
    if (sched_xcd_grouped(P, Hkv)) {
        const int x = b % 8, k = b / 8, W = P / 8, xh = 8 / Hkv;
        const int Q = xh * W;                           // workgroups of one KV head
        // Slot of workgroup (XCD x, k-th on it): the first W1 = W - W % n_hg
        // workgroups of every XCD hold units of n_hg slots, unit t on the
        // head's XCD t % xh; the rest take the last slots in turn.
        const int W1 = W - W % n_hg, xp = x % xh;
        const int u = (k < W1) ? ((k / n_hg) * xh + xp) * n_hg + k % n_hg
                               : xh * W1 + (k - W1) * xh + xp;
        const int j = pass * Q + ((pass & 1) ? Q - 1 - u : u);
        if (j >= nrb * n_hg)
            return false;
        it.kvh = x / xh;
        it.rbi = j / n_hg;
        it.hg = j % n_hg;
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
    return true;
}

}  // namespace ga
