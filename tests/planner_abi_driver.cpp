// Host driver for the planner's C ABI, built by the CPU tests with the address
// and undefined-behaviour sanitizers.  It reads cases from stdin and prints one
// result line per case.  Every output buffer is allocated with exactly the
// capacity the case gives (null when that capacity is 0), so a write past a
// caller's capacity is a heap overflow that the sanitizer reports.
//
// Case lines (whitespace separated):
//   P n budget cap align world interleave chunk_cap entry_cap ctx[n] q[n]
//       world = 0 calls mla_plan_context_chunks, else mla_plan_dcp_context_chunks.
//       Three calls: sizing (null buffers, capacities 0), the given capacities,
//       then the sizes the first call reported.  Prints
//       "P s1 nc1 ne1 s2 nc2 ne2 s3" and, when s3 is 0, the plan.
//   N n                      planner calls with null length arrays
//   T n empty_cap ctx[n] q[n]   mla_prefill_token_info
//   U n budget align ctx[n]     mla_plan_uniform_windows
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <memory>
#include <string>
#include <vector>

#include "mla_cc.h"

namespace {

template <class T>
std::unique_ptr<T[]> exact(int64_t n) {
    return n > 0 ? std::unique_ptr<T[]>(new T[n]) : nullptr;
}

std::vector<int32_t> read_ints(int64_t n) {
    std::vector<int32_t> v(n);
    for (auto& x : v) std::cin >> x;
    return v;
}

const int32_t* data_or_null(const std::vector<int32_t>& v) { return v.empty() ? nullptr : v.data(); }

int plan(int32_t world, int32_t il, const std::vector<int32_t>& ctx, const std::vector<int32_t>& q, int32_t n,
         int64_t budget, int64_t cap, int32_t align, int32_t ccap, int32_t ecap, int32_t* nc, int32_t* ne,
         mla_chunk_desc* chunks, int32_t* st, int32_t* ln, int32_t* lst, int32_t* lln) {
    if (world == 0)
        return mla_plan_context_chunks(data_or_null(ctx), data_or_null(q), n, budget, cap, align, chunks, ccap, nc, st,
                                       ln, ecap, ne);
    return mla_plan_dcp_context_chunks(data_or_null(ctx), data_or_null(q), n, budget, cap, align, world, il, chunks,
                                       ccap, nc, st, ln, lst, lln, ecap, ne);
}

void case_plan() {
    int32_t n, align, world, il, ccap, ecap;
    int64_t budget, cap;
    std::cin >> n >> budget >> cap >> align >> world >> il >> ccap >> ecap;
    const auto ctx = read_ints(n), q = read_ints(n);
    int32_t nc1 = -1, ne1 = -1, nc2 = -1, ne2 = -1, nc3 = -1, ne3 = -1;
    const int s1 = plan(world, il, ctx, q, n, budget, cap, align, 0, 0, &nc1, &ne1, nullptr, nullptr, nullptr,
                        nullptr, nullptr);
    {
        auto chunks = exact<mla_chunk_desc>(ccap);
        auto st = exact<int32_t>(ecap), ln = exact<int32_t>(ecap), lst = exact<int32_t>(ecap),
             lln = exact<int32_t>(ecap);
        const int s2 = plan(world, il, ctx, q, n, budget, cap, align, ccap, ecap, &nc2, &ne2, chunks.get(), st.get(),
                            ln.get(), lst.get(), lln.get());
        std::printf("P %d %d %d %d %d %d", s1, nc1, ne1, s2, nc2, ne2);
    }
    if (s1 != MLA_OK && s1 != MLA_ERR_CAPACITY) {
        std::printf(" -\n");
        return;
    }
    auto chunks = exact<mla_chunk_desc>(nc1);
    auto st = exact<int32_t>(ne1), ln = exact<int32_t>(ne1), lst = exact<int32_t>(ne1), lln = exact<int32_t>(ne1);
    const int s3 = plan(world, il, ctx, q, n, budget, cap, align, nc1, ne1, &nc3, &ne3, chunks.get(), st.get(),
                        ln.get(), lst.get(), lln.get());
    std::printf(" %d", s3);
    if (s3 == MLA_OK) {
        std::printf(" |");
        for (int32_t c = 0; c < nc3; ++c) {
            const mla_chunk_desc& d = chunks[c];
            std::printf(" %d %d %d %d %d %d %d %d %d %d ;", d.request_begin, d.request_end, d.token_begin, d.token_end,
                        d.entry_begin, d.num_entries, d.num_rows, d.max_seq_len, d.max_query_len, d.is_continuation);
        }
        std::printf(" |");
        for (int32_t e = 0; e < ne3; ++e) std::printf(" %d %d", st[e], ln[e]);
        if (world != 0) {
            std::printf(" |");
            for (int32_t e = 0; e < ne3; ++e) std::printf(" %d %d", lst[e], lln[e]);
        }
    }
    std::printf("\n");
}

void case_null() {
    int32_t n;
    std::cin >> n;
    int32_t nc = -1, ne = -1;
    const int s1 = mla_plan_context_chunks(nullptr, nullptr, n, 1024, 0, 64, nullptr, 0, &nc, nullptr, nullptr, 0, &ne);
    const int s2 = mla_plan_dcp_context_chunks(nullptr, nullptr, n, 1024, 0, 64, 2, 1, nullptr, 0, &nc, nullptr,
                                               nullptr, nullptr, nullptr, 0, &ne);
    int64_t prefix = -1;
    int32_t count = -1;
    const int s3 = mla_prefill_token_info(nullptr, nullptr, n, &prefix, nullptr, 0, &count);
    int64_t window = -1;
    int32_t iters = -1;
    const int s4 = mla_plan_uniform_windows(nullptr, n, 1024, 64, &window, &iters);
    std::printf("N %d %d %d %d\n", s1, s2, s3, s4);
}

void case_tokens() {
    int32_t n, ecap;
    std::cin >> n >> ecap;
    const auto ctx = read_ints(n), q = read_ints(n);
    auto slices = exact<int32_t>(2 * static_cast<int64_t>(ecap));
    int64_t prefix = -1;
    int32_t count = -1;
    const int s = mla_prefill_token_info(data_or_null(ctx), data_or_null(q), n, &prefix, slices.get(), ecap, &count);
    std::printf("T %d %lld %d |", s, static_cast<long long>(prefix), count);
    if (s == MLA_OK || s == MLA_ERR_CAPACITY)
        for (int32_t i = 0; i < count && i < ecap; ++i) std::printf(" %d %d", slices[2 * i], slices[2 * i + 1]);
    std::printf("\n");
}

void case_windows() {
    int32_t n, align;
    int64_t budget;
    std::cin >> n >> budget >> align;
    const auto ctx = read_ints(n);
    int64_t window = -1;
    int32_t iters = -1;
    const int s = mla_plan_uniform_windows(data_or_null(ctx), n, budget, align, &window, &iters);
    std::printf("U %d %lld %d\n", s, static_cast<long long>(window), iters);
}

}  // namespace

int main() {
    std::string kind;
    while (std::cin >> kind) {
        if (kind == "P") case_plan();
        else if (kind == "N") case_null();
        else if (kind == "T") case_tokens();
        else if (kind == "U") case_windows();
        else return 2;
        std::fflush(stdout);
    }
    return 0;
}
