// Work queues of the persistent attention launches: the host-side table
// builder and the item decode that the kernels run (also built for the host,
// so that the mapping can be checked on a CPU).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

namespace mla {

constexpr int32_t kQueryTileRows = 256;  // queries per attention tile

// Work queues of a persistent attention launch, built on the host from the
// launch's lengths (build_work_queues) and stored in device memory:
//   perm[n]        sequences in the order they are dealt (longest first)
//   qtiles[n]      256-query tiles of each dealt sequence
//   prefix[X][n+1] queue x's items before dealt sequence r
//   counters       X ints, kCounterStride apart, zero before the launch
// The G = heads * splits groups of dealt sequence r are global groups
// t = r * G + g; group t belongs to queue t % X, and each group's items are
// consecutive in its queue (they stream the same keys, so they run together
// under one L2).  A non-causal item is one query tile.  A causal item is a
// pair of query tiles, the longest left with the shortest left (tiles Q-1-i
// and i of Q): every pair but a lone middle tile then costs Q + 1 key blocks.
constexpr int32_t kCounterStride = 16;       // ints between two queues' counters (64 bytes)
// table held in LDS by the kernel (the causal kernel's LDS holds it beside
// 144 KB of K ring and Q staging)
constexpr int32_t kMaxQueueTableInts = 4080;

struct WorkQueues {
    const int32_t* table = nullptr;  // work_table_ints(...) ints
    int32_t* counters = nullptr;
    int32_t num_seqs = 0;
    int32_t queues = 1;  // X
    int32_t items = 0;   // total items
};

// Ints of the table (counters excluded).
inline int64_t work_table_ints(int64_t n, int32_t queues) { return 2 * n + static_cast<int64_t>(queues) * (n + 1); }

// Writes the table for a launch over n sequences with q_lens / k_lens (k_lens
// unused when causal) to `out`; returns the number of items.  Sequences are
// dealt longest first: non-causal by key rows, causal by query rows (ties by
// index).
inline int64_t build_work_queues(const int32_t* q_lens, const int32_t* k_lens, int32_t n, int32_t heads,
                                 int32_t splits, bool causal, int32_t queues, int32_t* out) {
    int32_t* perm = out;
    int32_t* qtiles = out + n;
    int32_t* prefix = out + 2 * static_cast<int64_t>(n);
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    // longest first: non-causal by key rows (the length of every tile of the
    // sequence), causal by query rows (the length of each of its pairs)
    auto key = [&](int32_t i) { return causal ? q_lens[i] : k_lens[i]; };
    std::stable_sort(perm, perm + n, [&](int32_t x, int32_t y) { return key(x) > key(y); });
    const int64_t groups = static_cast<int64_t>(heads) * (causal ? 1 : splits);
    for (int32_t x = 0; x < queues; ++x) prefix[static_cast<int64_t>(x) * (n + 1)] = 0;
    int64_t items = 0;
    for (int32_t r = 0; r < n; ++r) {
        const int32_t ql = q_lens[perm[r]];
        qtiles[r] = ql > 0 ? (ql + kQueryTileRows - 1) / kQueryTileRows : 0;
        const int64_t per_group = causal ? (qtiles[r] + 1) / 2 : qtiles[r];
        const int64_t base = static_cast<int64_t>(r) * groups;
        for (int32_t x = 0; x < queues; ++x) {
            // groups t in [base, base + groups) with t % queues == x
            const int64_t first = base + ((x - base) % queues + queues) % queues;
            const int64_t cnt = first < base + groups ? (base + groups - 1 - first) / queues + 1 : 0;
            int32_t* pre = prefix + static_cast<int64_t>(x) * (n + 1);
            pre[r + 1] = static_cast<int32_t>(pre[r] + cnt * per_group);
        }
        items += groups * per_group;
    }
    return items;
}

// Last index i in [0, count) with a[i] <= v (a nondecreasing, a[0] <= v).
__host__ __device__ inline int32_t last_at_most(const int32_t* a, int32_t count, int32_t v) {
    int32_t lo = 0, hi = count - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (a[mid] <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Item j of queue `queue` (layout above) as (seq, head, split,
// qt, qt2): query tile qt, then (causal pairs) query tile qt2 unless it is
// negative.  False when j is past the queue's end.  groups = heads * splits.
__host__ __device__ inline bool decode_queue_item(const int32_t* table, int32_t n, int32_t queues, int32_t groups,
                                                  int32_t heads, bool causal, int32_t queue, int32_t j,
                                                  int32_t* item) {
    const int32_t* pre = table + 2 * n + queue * (n + 1);
    if (j < 0 || j >= pre[n]) return false;
    const int32_t r = last_at_most(pre, n, j);  // skips sequences without items on this queue
    const int32_t tiles = table[n + r];
    const int32_t per_group = causal ? (tiles + 1) / 2 : tiles;
    const int32_t o = j - pre[r], gi = o / per_group, i = o - gi * per_group;
    const int32_t base = r * groups;
    const int32_t t = base + ((queue - base) % queues + queues) % queues + gi * queues;
    const int32_t g = t - base;
    item[0] = table[r];
    item[1] = g % heads;
    item[2] = g / heads;
    item[3] = causal ? tiles - 1 - i : i;
    item[4] = causal && i != tiles - 1 - i ? i : -1;
    return true;
}

}  // namespace mla
