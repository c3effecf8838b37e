// Host check of the persistent attention's work queues (work_queues.h): for
// random launches, every (sequence, head, split, query tile) must come out of
// exactly one queue position, causal items must pair tile Q-1-i with tile i
// (a lone middle tile when Q is odd), each item's group must belong to its
// queue, and decoding past a queue's end must fail.  Prints "ok" or the first
// failures; exit status 0 on success.
#include <cstdio>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "work_queues.h"

int main() {
    std::mt19937 rng(1);
    int fails = 0, cases = 0;
    for (int it = 0; it < 4000 && fails < 10; ++it) {
        const int n = 1 + rng() % 40;
        const int heads = (it % 3 == 0) ? 128 : 1 + rng() % 20;
        const bool causal = rng() % 2;
        const int splits = causal ? 1 : 1 + rng() % 8;
        const int X = 1 + rng() % 8;
        std::vector<int32_t> ql(n), kl(n);
        for (int i = 0; i < n; ++i) {
            ql[i] = (rng() % 5 == 0) ? 0 : rng() % 3000;
            kl[i] = rng() % 100000;
        }
        if (mla::work_table_ints(n, X) > mla::kMaxQueueTableInts) continue;
        std::vector<int32_t> table(mla::work_table_ints(n, X));
        const int64_t items = mla::build_work_queues(ql.data(), kl.data(), n, heads, splits, causal, X, table.data());
        const int groups = heads * splits;
        std::vector<int> rank(n);
        for (int r = 0; r < n; ++r) rank[table[r]] = r;
        std::set<std::tuple<int, int, int, int>> seen;
        int64_t tiles_seen = 0, items_seen = 0;
        for (int q = 0; q < X; ++q) {
            const int32_t end = table[2 * n + q * (n + 1) + n];
            for (int j = 0; j <= end; ++j) {
                int32_t item[5];
                const bool ok = mla::decode_queue_item(table.data(), n, X, groups, heads, causal, q, j, item);
                if (j == end) {
                    if (ok) { ++fails; std::printf("case %d: decoded past the end\n", it); }
                    continue;
                }
                if (!ok) { ++fails; std::printf("case %d: item %d of queue %d missing\n", it, j, q); continue; }
                const int seq = item[0], h = item[1], sp = item[2], qt = item[3], qt2 = item[4];
                const int tl = ql[seq] > 0 ? (ql[seq] + 255) / 256 : 0;
                if (seq < 0 || seq >= n || h < 0 || h >= heads || sp < 0 || sp >= splits || qt < 0 || qt >= tl) {
                    ++fails; std::printf("case %d: invalid item\n", it); continue;
                }
                const int r = rank[seq];
                if ((static_cast<long>(r) * groups + static_cast<long>(sp) * heads + h) % X != q) {
                    ++fails; std::printf("case %d: item in the wrong queue\n", it);
                }
                ++items_seen;
                if (!seen.insert({seq, h, sp, qt}).second) { ++fails; std::printf("case %d: tile twice\n", it); }
                ++tiles_seen;
                if (causal) {
                    if (qt2 >= 0) {
                        if (qt2 + qt != tl - 1 || qt2 >= qt) { ++fails; std::printf("case %d: bad pair\n", it); }
                        if (!seen.insert({seq, h, sp, qt2}).second) { ++fails; std::printf("case %d: tile twice\n", it); }
                        ++tiles_seen;
                    } else if (2 * qt != tl - 1) {
                        ++fails; std::printf("case %d: lone tile not in the middle\n", it);
                    }
                } else if (qt2 >= 0) {
                    ++fails; std::printf("case %d: second tile in a non-causal item\n", it);
                }
            }
        }
        int64_t expect_tiles = 0, expect_items = 0;
        for (int i = 0; i < n; ++i) {
            const int tl = ql[i] > 0 ? (ql[i] + 255) / 256 : 0;
            expect_tiles += static_cast<int64_t>(groups) * tl;
            expect_items += static_cast<int64_t>(groups) * (causal ? (tl + 1) / 2 : tl);
        }
        if (tiles_seen != expect_tiles || items_seen != expect_items || items != expect_items) {
            ++fails;
            std::printf("case %d: %lld tiles %lld items, expected %lld and %lld (builder says %lld)\n", it,
                        static_cast<long long>(tiles_seen), static_cast<long long>(items_seen),
                        static_cast<long long>(expect_tiles), static_cast<long long>(expect_items),
                        static_cast<long long>(items));
        }
        // dealt longest first
        for (int r = 1; r < n; ++r) {
            const int a = table[r - 1], b = table[r];
            if ((causal ? ql[a] < ql[b] : kl[a] < kl[b])) { ++fails; std::printf("case %d: order\n", it); break; }
        }
        ++cases;
    }
    if (fails == 0) std::printf("ok %d cases\n", cases);
    return fails == 0 ? 0 : 1;
}
