// Chunked-context prefill driver (the _compute_prefill_context loop of the
// vLLM PR #50613 digest, 实现拆解 item 3, plus the final merge of the PR
// #36540 digest), native and stream-ordered:
//
//   host:   plan chunks, build per-chunk device metadata, one H2D upload
//   device: init the partial rows of requests without context (0, -inf)
//           for each chunk:
//             gather its context rows into the workspace
//             attention of its requests' queries against their rows; rows no
//             earlier chunk wrote go straight into the context partial, the
//             first request of a continuation chunk goes to a temporary and is
//             LSE-merged into the partial (accumulate_mla_context_chunk)
//           causal suffix attention over the new tokens
//           merge_attn_states(partial, suffix, prefix_num_tokens) -> out
//
// A single chunk that covers every token (the digest's early exit when one
// chunk covers all context) needs neither the init nor any accumulate: its
// attention output is the partial.
//
// Two more drivers share the pieces: the same loop with each chunk's rows
// assembled as under DCP (local gathers into the all-gather layout, then a
// reorganisation into request order), and the uniform-window scheduler that
// per-request packing replaced.
#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "device.h"
#include "planner.h"

// Scratch of mla_chunked_prefill_no_alloc: a fixed device buffer that every
// GPU the library runs on holds until the process ends.  Host code never
// passes this name to a kernel or a copy (on the host it is only a stand-in
// for the symbol): it uses the per-device address that
// hipGetSymbolAddress returns (no_alloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MLA_NO_ALLOC_SCRATCH_BYTES];

namespace mla {

namespace {

constexpr int64_t kAlign = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Plan {
    std::vector<mla_chunk_desc> chunks;
    std::vector<int32_t> starts, lens;
};

struct VecSink : PlanSink {
    Plan* p;
    void chunk(const mla_chunk_desc& c) override { p->chunks.push_back(c); }
    void entry(int32_t s, int32_t n) override {
        p->starts.push_back(s);
        p->lens.push_back(n);
    }
    int32_t entries_so_far() const override { return static_cast<int32_t>(p->starts.size()); }
};

// Key split of a chunk-attention launch whose longest workgroups outlast the
// average load of a CU, e.g. one long-context request with few queries, or a
// head shard of 16 heads per GPU: each sequence's key range is cut into
// `splits` slices of `split_keys` rows, one workgroup per slice, and the
// slices' states are LSE-merged (the merge_attn_states operator).
// The persistent launch deals its workgroups longest first to whichever CU
// frees up, so its length is that of list scheduling in that order.  Among
// S = 1 .. kMaxSplits slices of at least kMinSplitTiles key tiles each, the
// split with the shortest simulated schedule is taken (a longer split only
// if it gains kSplitGain), each workgroup costing its key tiles plus
// kItemOverheadTiles.  Launches whose longest workgroup stays within 1.2x
// the average CU load are not split.  CUs: the device's count.
constexpr int32_t kMaxSplits = kMaxSlices;  // slices one merge combines
constexpr int32_t kMinSplitTiles = 64; // 4096 keys per slice at least
constexpr int32_t kQueryTile = 256;    // queries per attention workgroup
constexpr int32_t kKeyTile = 64;       // keys per attention tile
constexpr int64_t kItemOverheadTiles = 1;
constexpr double kSplitGain = 0.97;
constexpr int64_t kMaxSimulatedItems = 1 << 16;

struct SplitPlan {
    int32_t splits = 1;
    int32_t split_keys = 0;
};

// Length in tile steps of list scheduling `cus` CUs over the workgroups of
// a launch cut into slices of `slice_tiles` key tiles (0: no split), in
// longest-first order; -1 past kMaxSimulatedItems workgroups.
int64_t simulated_length(const int32_t* q_lens, const int32_t* k_rows, int32_t n, int32_t heads, int32_t cus,
                         int32_t slices, int32_t slice_tiles) {
    std::vector<std::pair<int64_t, int64_t>> classes;  // (cost, count)
    int64_t items = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (q_lens[i] <= 0) continue;
        const int64_t kt = (k_rows[i] + kKeyTile - 1) / kKeyTile;
        const int64_t per_slice = static_cast<int64_t>((q_lens[i] + kQueryTile - 1) / kQueryTile) * heads;
        for (int32_t s = 0; s < slices; ++s) {
            const int64_t c = slices == 1 ? kt : std::max<int64_t>(0, std::min<int64_t>(kt - s * slice_tiles, slice_tiles));
            classes.emplace_back(c + kItemOverheadTiles, per_slice);
            items += per_slice;
        }
    }
    if (items > kMaxSimulatedItems) return -1;
    std::sort(classes.begin(), classes.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
    size_t m = 0;  // equal costs merged into one class
    for (size_t i = 0; i < classes.size(); ++i) {
        if (m > 0 && classes[m - 1].first == classes[i].first)
            classes[m - 1].second += classes[i].second;
        else
            classes[m++] = classes[i];
    }
    classes.resize(m);
    // a class of `count` equal workgroups: whole rounds of one per CU, then
    // the rest on the least loaded CUs (list scheduling gives each of them to
    // the CU that frees up first)
    std::vector<int64_t> load(static_cast<size_t>(cus), 0);
    int64_t base = 0;  // added to every CU
    for (const auto& [cost, count] : classes) {
        base += count / cus * cost;
        const int64_t rest = count % cus;
        if (rest == 0) continue;
        std::nth_element(load.begin(), load.begin() + (rest - 1), load.end());
        for (int64_t k = 0; k < rest; ++k) load[static_cast<size_t>(k)] += cost;
    }
    return base + *std::max_element(load.begin(), load.end());
}

// q_lens / k_rows: the launch's sequences (query rows, key rows)
SplitPlan plan_split(const int32_t* q_lens, const int32_t* k_rows, int32_t n, int32_t heads, int32_t cus) {
    int64_t work = 0;  // key tiles summed over the launch's live workgroups
    int32_t longest = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (q_lens[i] <= 0) continue;
        const int32_t kt = (k_rows[i] + kKeyTile - 1) / kKeyTile;
        work += static_cast<int64_t>((q_lens[i] + kQueryTile - 1) / kQueryTile) * kt * heads;
        longest = std::max(longest, kt);
    }
    if (work <= 0 || cus < 1) return {};
    const double avg = static_cast<double>(work) / cus;
    if (longest <= 1.2 * avg) return {};
    SplitPlan best;
    int64_t best_len = simulated_length(q_lens, k_rows, n, heads, cus, 1, 0);
    if (best_len < 0) return {};
    for (int32_t s = 2; s <= kMaxSplits && longest / s >= kMinSplitTiles; ++s) {
        const int32_t tiles = (longest + s - 1) / s;
        const int32_t slices = (longest + tiles - 1) / tiles;  // no slice starts past the longest range
        if (slices != s) continue;  // the same split as a smaller s
        const int64_t len = simulated_length(q_lens, k_rows, n, heads, cus, slices, tiles);
        if (len < 0) break;
        if (static_cast<double>(len) < kSplitGain * static_cast<double>(best_len)) {
            best_len = len;
            best.splits = slices;
            best.split_keys = tiles * kKeyTile;
        }
    }
    return best;
}

// Work queues of one persistent attention launch, as offsets (int32
// elements) into the meta block; table < 0: the launch's table does not fit
// the kernel's LDS copy and the launch takes one workgroup per tile instead.
struct QueuePlan {
    int64_t table = -1, counters = -1;
    int32_t n = 0, queues = 1, items = 0;
};

// Appends a launch's work table and its zeroed counters to the meta image
// (the upload zeroes the counters before every call's launches).
QueuePlan plan_queues(std::vector<int32_t>& meta, const int32_t* q_lens, const int32_t* k_lens, int32_t n,
                      int32_t heads, int32_t splits, bool causal, int32_t queues) {
    QueuePlan qp;
    if (n <= 0 || work_table_ints(n, queues) > kMaxQueueTableInts) return qp;
    qp.n = n;
    qp.queues = queues;
    qp.table = static_cast<int64_t>(meta.size());
    meta.resize(meta.size() + work_table_ints(n, queues), 0);
    const int64_t items = build_work_queues(q_lens, k_lens, n, heads, splits, causal, queues, meta.data() + qp.table);
    qp.items = static_cast<int32_t>(std::min<int64_t>(items, INT32_MAX));
    while (meta.size() % kCounterStride) meta.push_back(0);  // each counter on its own 64-byte line
    qp.counters = static_cast<int64_t>(meta.size());
    meta.resize(meta.size() + static_cast<size_t>(queues) * kCounterStride, 0);
    return qp;
}

// Device metadata of one chunk, as offsets (in int32 elements) into the meta
// block.  e_lstart / e_loff (local starts and offsets) exist only under DCP.
struct ChunkMeta {
    int64_t e_req, e_start, e_off, cu_q, e_lstart = 0, e_loff = 0;
    int32_t rows = 0;        // context rows (request order)
    int32_t local_rows = 0;  // padded local rows of one rank (DCP)
    SplitPlan split_cont;    // the continuation request's own launch
    SplitPlan split_direct;  // the launch over the other requests
    QueuePlan queues_cont, queues_direct;
};

struct Layout {
    int64_t ws_k, ws_v, part_out, part_lse, suf_out, suf_lse, tmp_out, tmp_lse, meta, g_k = 0, g_v = 0;
    int64_t split_out = 0, split_lse = 0;
    int64_t total;
    int64_t tmp_rows;        // rows of the continuation temporary
    int64_t meta_ints;       // int32 elements of metadata
    int64_t split_rows = 0;  // query rows of one split state (the largest split launch)
    int32_t split_max = 1;   // most splits of any launch
};

struct Problem {
    Plan plan;
    std::vector<int32_t> meta;  // host image of the device metadata
    std::vector<ChunkMeta> cmeta;
    int64_t suffix_cu;          // offset of the suffix query_start_loc
    QueuePlan queues_suffix;
    int64_t tokens = 0;
    int32_t max_q = 0;
    int64_t prefix_num_tokens = 0;
    std::vector<int32_t> empty;  // pairs
    int32_t world = 1, interleave = 1;
    Layout lay{};
};

int build_problem(const mla_chunked_prefill_params& p, Problem& pb, bool dcp = false, int32_t world = 1,
                  int32_t interleave = 1) {
    const int32_t n = p.num_requests;
    const DeviceShape shape = device_shape();
    VecSink sink;
    sink.p = &pb.plan;
    pb.world = world;
    pb.interleave = interleave;
    int st = plan_chunks(p.context_lens, p.query_lens, n, p.workspace_rows, p.max_context_chunk, p.split_alignment,
                         sink, world, interleave);
    if (st != MLA_OK) return st;
    int32_t n_empty = 0;
    st = token_info(p.context_lens, p.query_lens, n, &pb.prefix_num_tokens, nullptr, 0, &n_empty);
    if (st != MLA_OK && st != MLA_ERR_CAPACITY) return st;
    pb.empty.assign(2 * static_cast<size_t>(n_empty), 0);
    st = token_info(p.context_lens, p.query_lens, n, &pb.prefix_num_tokens, pb.empty.data(), n_empty, &n_empty);
    if (st != MLA_OK) return st;

    std::vector<int64_t> qsl(n + 1, 0);
    for (int32_t r = 0; r < n; ++r) {
        qsl[r + 1] = qsl[r] + p.query_lens[r];
        pb.max_q = std::max(pb.max_q, p.query_lens[r]);
    }
    pb.tokens = qsl[n];

    // metadata image: per chunk e_req[n], e_start[n], e_off[n+1], cu_q[n+1]
    int64_t tmp_rows = 0, split_rows = 0;
    int32_t split_max = 1;
    for (const auto& c : pb.plan.chunks) {
        ChunkMeta m{};
        const int32_t ne = c.num_entries;
        m.e_req = static_cast<int64_t>(pb.meta.size());
        for (int32_t i = 0; i < ne; ++i) pb.meta.push_back(c.request_begin + i);
        m.e_start = static_cast<int64_t>(pb.meta.size());
        for (int32_t i = 0; i < ne; ++i) pb.meta.push_back(pb.plan.starts[c.entry_begin + i]);
        m.e_off = static_cast<int64_t>(pb.meta.size());
        int32_t off = 0;
        pb.meta.push_back(0);
        for (int32_t i = 0; i < ne; ++i) {
            off += pb.plan.lens[c.entry_begin + i];
            pb.meta.push_back(off);
        }
        m.rows = off;
        m.cu_q = static_cast<int64_t>(pb.meta.size());
        for (int32_t i = 0; i <= ne; ++i)
            pb.meta.push_back(static_cast<int32_t>(qsl[c.request_begin + i] - qsl[c.request_begin]));
        if (dcp) {
            m.e_lstart = static_cast<int64_t>(pb.meta.size());
            for (int32_t i = 0; i < ne; ++i) pb.meta.push_back(pb.plan.starts[c.entry_begin + i] / world);
            m.e_loff = static_cast<int64_t>(pb.meta.size());
            int64_t loff = 0;
            pb.meta.push_back(0);
            for (int32_t i = 0; i < ne; ++i) {
                const int64_t s0 = pb.plan.starts[c.entry_begin + i], len = pb.plan.lens[c.entry_begin + i];
                loff += padded_local_rows(s0 + len, world, interleave) - s0 / world;
                pb.meta.push_back(static_cast<int32_t>(loff));
            }
            m.local_rows = static_cast<int32_t>(loff);
        }
        // key splits of the chunk's attention launches (see run_chunked)
        const int32_t first_direct = c.is_continuation ? 1 : 0;
        if (c.is_continuation && p.query_lens[c.request_begin] > 0) {
            m.split_cont = plan_split(&p.query_lens[c.request_begin], &pb.plan.lens[c.entry_begin], 1, p.num_heads,
                                      shape.cus);
            if (m.split_cont.splits > 1) {
                split_rows = std::max<int64_t>(split_rows, p.query_lens[c.request_begin]);
                split_max = std::max(split_max, m.split_cont.splits);
            }
            m.queues_cont = plan_queues(pb.meta, &p.query_lens[c.request_begin], &pb.plan.lens[c.entry_begin], 1,
                                        p.num_heads, m.split_cont.splits, false, shape.xcds);
        }
        if (ne > first_direct) {
            m.split_direct = plan_split(&p.query_lens[c.request_begin + first_direct],
                                        &pb.plan.lens[c.entry_begin + first_direct], ne - first_direct, p.num_heads,
                                        shape.cus);
            if (m.split_direct.splits > 1) {
                split_rows = std::max<int64_t>(split_rows, qsl[c.request_begin + ne] - qsl[c.request_begin]);
                split_max = std::max(split_max, m.split_direct.splits);
            }
            m.queues_direct = plan_queues(pb.meta, &p.query_lens[c.request_begin + first_direct],
                                          &pb.plan.lens[c.entry_begin + first_direct], ne - first_direct, p.num_heads,
                                          m.split_direct.splits, false, shape.xcds);
        }
        pb.cmeta.push_back(m);
        if (c.is_continuation) tmp_rows = std::max<int64_t>(tmp_rows, p.query_lens[c.request_begin]);
    }
    pb.suffix_cu = static_cast<int64_t>(pb.meta.size());
    for (int32_t r = 0; r <= n; ++r) pb.meta.push_back(static_cast<int32_t>(qsl[r]));
    pb.queues_suffix = plan_queues(pb.meta, p.query_lens, nullptr, n, p.num_heads, 1, true, shape.xcds);

    // scratch layout
    const int64_t H = p.num_heads, T = pb.tokens, W = p.workspace_rows;
    Layout& L = pb.lay;
    int64_t o = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = o;
        o = round_up(o + std::max<int64_t>(bytes, 0), kAlign);
        return at;
    };
    L.ws_k = take(W * H * kDk * 2);
    L.ws_v = take(W * H * kDv * 2);
    L.part_out = take(T * H * kDv * 2);
    L.part_lse = take(H * T * 4);
    L.suf_out = take(T * H * kDv * 2);
    L.suf_lse = take(H * T * 4);
    L.tmp_rows = tmp_rows;
    L.tmp_out = take(tmp_rows * H * kDv * 2);
    L.tmp_lse = take(H * tmp_rows * 4);
    L.meta_ints = static_cast<int64_t>(pb.meta.size());
    L.meta = take(L.meta_ints * 4);
    L.split_rows = split_rows;
    L.split_max = split_max;
    if (split_max > 1) {
        L.split_out = take(split_max * split_rows * H * kDv * 2);
        L.split_lse = take(split_max * H * split_rows * 4);
    }
    if (dcp) {
        int64_t g_rows = 0;
        for (const auto& m : pb.cmeta) g_rows = std::max<int64_t>(g_rows, static_cast<int64_t>(world) * m.local_rows);
        L.g_k = take(g_rows * H * kDk * 2);
        L.g_v = take(g_rows * H * kDv * 2);
    }
    L.total = o;
    return MLA_OK;
}

// Pinned staging for the metadata upload.  A slot is reused only after the
// copy that last read it has completed (its event), so calls can overlap.
struct StagingSlot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};
struct DevicePool {
    std::array<StagingSlot, 4> slots;
    int next = 0;
};
std::mutex g_pool_mu;
std::map<int, DevicePool> g_pools;

int upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
    if (bytes == 0) return MLA_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_pool_mu);
    DevicePool& pool = g_pools[dev];
    StagingSlot& s = pool.slots[pool.next];
    pool.next = (pool.next + 1) % static_cast<int>(pool.slots.size());
    if (s.pending) {
        if (hipEventSynchronize(s.ev) != hipSuccess) return MLA_ERR_HIP;
        s.pending = false;
    }
    if (s.ev == nullptr && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) return MLA_ERR_HIP;
    if (s.cap < bytes) {
        if (s.host != nullptr) hipHostFree(s.host);
        s.host = nullptr;
        s.cap = 0;
        const size_t cap = std::max<size_t>(bytes * 2, 1 << 16);
        if (hipHostMalloc(&s.host, cap, hipHostMallocDefault) != hipSuccess) return MLA_ERR_HIP;
        s.cap = cap;
    }
    std::memcpy(s.host, src, bytes);
    if (hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return MLA_ERR_HIP;
    if (hipEventRecord(s.ev, stream) != hipSuccess) return MLA_ERR_HIP;
    s.pending = true;
    return MLA_OK;
}

int check_params(const mla_chunked_prefill_params* p) {
    if (p == nullptr) return MLA_ERR_INVALID_ARG;
    if (p->num_requests < 0 || p->num_heads < 1 || p->num_heads > MLA_MAX_HEADS || p->block_size < 1 ||
        p->block_table_width < 0 ||
        p->num_blocks < 0 || p->workspace_rows < 1 || p->split_alignment < 1)
        return MLA_ERR_INVALID_ARG;
    if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return MLA_ERR_INVALID_ARG;
    if (p->num_requests > 0 && (p->context_lens == nullptr || p->query_lens == nullptr)) return MLA_ERR_INVALID_ARG;
    return MLA_OK;
}

#define MLA_TRY(expr)                     \
    do {                                  \
        const int st_ = (expr);           \
        if (st_ != MLA_OK) return st_;    \
    } while (0)

// ---------------------------------------------------------------------------
// Metadata upload without host staging: the metadata travels in the kernel
// arguments of small writer launches (kMetaPieceInts int32 each), so the
// no-allocation entry point needs neither pinned host memory nor a copy
// from pageable memory.

constexpr int kMetaPieceInts = 480;  // 1920 bytes of arguments per launch

struct MetaPiece {
    int32_t* dst;
    int32_t count;
    int32_t v[kMetaPieceInts];
};

__global__ __launch_bounds__(512) void write_meta_kernel(MetaPiece piece) {
    const int i = threadIdx.x;
    if (i < piece.count) piece.dst[i] = piece.v[i];
}

int write_meta_args(const int32_t* src, size_t count, int32_t* dst, hipStream_t stream) {
    for (size_t at = 0; at < count; at += kMetaPieceInts) {
        MetaPiece piece;
        piece.dst = dst + at;
        piece.count = static_cast<int32_t>(std::min<size_t>(kMetaPieceInts, count - at));
        std::memcpy(piece.v, src + at, static_cast<size_t>(piece.count) * sizeof(int32_t));
        hipLaunchKernelGGL(write_meta_kernel, dim3(1), dim3(512), 0, stream, piece);
    }
    return hip_status(hipGetLastError());
}

// Device address of `scratch` on each device, looked up once per device
// (with that device current) on the first no-allocation call there.
constexpr int kMaxDevices = 64;
std::mutex g_no_alloc_mu;
void* g_no_alloc_ptr[kMaxDevices] = {};

int no_alloc_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_no_alloc_mu);
    if (g_no_alloc_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MLA_ERR_HIP;
        g_no_alloc_ptr[dev] = ptr;
    }
    *out = g_no_alloc_ptr[dev];
    return MLA_OK;
}

// ---------------------------------------------------------------------------
// Uniform-window scheduler (the scheduling per-request packing replaced,
// PR #50613 digest, 功能与动机): every iteration covers the same window of
// every request and runs attention, mask and merge over the whole batch.

struct WindowProblem {
    int64_t window = 0;
    int32_t iterations = 0;
    std::vector<int32_t> meta;  // e_req[N], qsl[N+1], per iteration e_start[N] and e_off[N+1]
    int64_t e_req = 0, qsl = 0;
    std::vector<int64_t> it_start, it_off;
    std::vector<int32_t> it_rows;
    std::vector<QueuePlan> it_queues;  // each iteration's attention launch
    QueuePlan queues_suffix;
    std::vector<char> it_has_empty;
    int64_t tokens = 0;
    int32_t max_q = 0;
    int64_t prefix_num_tokens = 0;
    Layout lay{};
};

int build_window_problem(const mla_chunked_prefill_params& p, WindowProblem& pb) {
    const int32_t n = p.num_requests;
    MLA_TRY(uniform_windows(p.context_lens, n, p.workspace_rows, p.split_alignment, &pb.window, &pb.iterations));
    int32_t n_empty = 0;
    const int st = token_info(p.context_lens, p.query_lens, n, &pb.prefix_num_tokens, nullptr, 0, &n_empty);
    if (st != MLA_OK && st != MLA_ERR_CAPACITY) return st;

    pb.e_req = static_cast<int64_t>(pb.meta.size());
    for (int32_t r = 0; r < n; ++r) pb.meta.push_back(r);
    pb.qsl = static_cast<int64_t>(pb.meta.size());
    int64_t tok = 0;
    pb.meta.push_back(0);
    for (int32_t r = 0; r < n; ++r) {
        tok += p.query_lens[r];
        pb.meta.push_back(static_cast<int32_t>(tok));
        pb.max_q = std::max(pb.max_q, p.query_lens[r]);
    }
    pb.tokens = tok;

    int64_t max_rows = 0;
    const int64_t w = pb.window;
    const DeviceShape shape = device_shape();
    std::vector<int32_t> lens(static_cast<size_t>(n));
    for (int32_t it = 0; it < pb.iterations; ++it) {
        pb.it_start.push_back(static_cast<int64_t>(pb.meta.size()));
        for (int32_t r = 0; r < n; ++r) pb.meta.push_back(static_cast<int32_t>(it * w));
        pb.it_off.push_back(static_cast<int64_t>(pb.meta.size()));
        int64_t off = 0;
        bool empty = false;
        pb.meta.push_back(0);
        for (int32_t r = 0; r < n; ++r) {
            const int64_t len = std::max<int64_t>(0, std::min<int64_t>(p.context_lens[r], (it + 1) * w) - it * w);
            empty = empty || len == 0;
            off += len;
            lens[static_cast<size_t>(r)] = static_cast<int32_t>(len);
            pb.meta.push_back(static_cast<int32_t>(off));
        }
        pb.it_rows.push_back(static_cast<int32_t>(off));
        pb.it_has_empty.push_back(empty ? 1 : 0);
        max_rows = std::max(max_rows, off);
        // the same persistent launches as the chunked path, so that the two
        // schedulers differ only in their schedule
        pb.it_queues.push_back(plan_queues(pb.meta, p.query_lens, lens.data(), n, p.num_heads, 1, false, shape.xcds));
    }
    pb.queues_suffix = plan_queues(pb.meta, p.query_lens, nullptr, n, p.num_heads, 1, true, shape.xcds);

    const int64_t H = p.num_heads, T = pb.tokens;
    Layout& L = pb.lay;
    int64_t o = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = o;
        o = round_up(o + std::max<int64_t>(bytes, 0), kAlign);
        return at;
    };
    L.ws_k = take(max_rows * H * kDk * 2);
    L.ws_v = take(max_rows * H * kDv * 2);
    L.part_out = take(T * H * kDv * 2);
    L.part_lse = take(H * T * 4);
    L.suf_out = take(T * H * kDv * 2);
    L.suf_lse = take(H * T * 4);
    L.tmp_rows = pb.iterations > 1 ? T : 0;
    L.tmp_out = take(L.tmp_rows * H * kDv * 2);
    L.tmp_lse = take(H * L.tmp_rows * 4);
    L.meta_ints = static_cast<int64_t>(pb.meta.size());
    L.meta = take(L.meta_ints * 4);
    L.total = o;
    return MLA_OK;
}

// Pointer checks shared by both drivers.
int check_buffers(const mla_chunked_prefill_params& p, bool needs_cache, int64_t scratch_needed) {
    if (p.q == nullptr || p.k_new == nullptr || p.v_new == nullptr || p.out == nullptr || p.scratch == nullptr)
        return MLA_ERR_INVALID_ARG;
    if (!aligned16(p.q) || !aligned16(p.k_new) || !aligned16(p.v_new) || !aligned16(p.out) ||
        (reinterpret_cast<uintptr_t>(p.scratch) % kAlign) != 0)
        return MLA_ERR_INVALID_ARG;
    if (needs_cache && (p.k_cache == nullptr || p.v_cache == nullptr || p.block_table == nullptr ||
                        !aligned16(p.k_cache) || !aligned16(p.v_cache)))
        return MLA_ERR_INVALID_ARG;
    if (p.scratch_bytes < scratch_needed) return MLA_ERR_CAPACITY;
    return MLA_OK;
}

// The chunk loop shared by the single-device and DCP drivers: `gather`
// fills the workspace with a chunk's context rows in request order.
// `upload_meta(src, ints, dst, stream)` puts the metadata into the scratch.
template <class Gather, class UploadMeta>
int run_chunked(const mla_chunked_prefill_params& p, const Problem& pb, hipStream_t stream, Gather gather,
                UploadMeta upload_meta) {
    const int64_t T = pb.tokens;
    const int32_t H = p.num_heads;
    char* base = static_cast<char*>(p.scratch);
    const Layout& L = pb.lay;
    bf16_t* ws_k = reinterpret_cast<bf16_t*>(base + L.ws_k);
    bf16_t* ws_v = reinterpret_cast<bf16_t*>(base + L.ws_v);
    bf16_t* part_out = reinterpret_cast<bf16_t*>(base + L.part_out);
    float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
    bf16_t* suf_out = reinterpret_cast<bf16_t*>(base + L.suf_out);
    float* suf_lse = reinterpret_cast<float*>(base + L.suf_lse);
    bf16_t* tmp_out = reinterpret_cast<bf16_t*>(base + L.tmp_out);
    float* tmp_lse = reinterpret_cast<float*>(base + L.tmp_lse);
    int32_t* meta = reinterpret_cast<int32_t*>(base + L.meta);

    MLA_TRY(upload_meta(pb.meta.data(), pb.meta.size(), meta, stream));

    const bf16_t* q = static_cast<const bf16_t*>(p.q);
    const int64_t qrow = static_cast<int64_t>(H) * kDk;
    const int64_t orow = static_cast<int64_t>(H) * kDv;

    // context partial of requests without context (only rows the final merge reads)
    for (size_t i = 0; i + 1 < pb.empty.size(); i += 2) {
        const int64_t b = pb.empty[i], e = std::min<int64_t>(pb.empty[i + 1], pb.prefix_num_tokens);
        if (b < e) MLA_TRY(launch_init_partial(part_out, part_lse, T, b, e, H, kDv, stream));
    }

    bf16_t* split_out = reinterpret_cast<bf16_t*>(base + L.split_out);
    float* split_lse = reinterpret_cast<float*>(base + L.split_lse);
    // Chunk attention of n sequences whose queries are rows [rows_lo, rows_hi)
    // of the chunk, into dst (LSE head stride dst_stride).  A key-split launch
    // writes one state per slice, and one merge combines them into dst.
    // attention through the launch's work queues when it has them
    auto attend = [&](const bf16_t* qa, const bf16_t* ka, const bf16_t* va, const int32_t* cu_q, const int32_t* cu_k,
                      int32_t n, int32_t max_q, bool causal, bf16_t* dst, float* dst_lse, int64_t dst_stride,
                      const QueuePlan& qp, const AttnSplit& as) -> int {
        if (qp.table < 0)
            return launch_attention(qa, ka, va, cu_q, cu_k, n, max_q, H, p.scale, causal, dst, dst_lse, dst_stride,
                                    stream, as);
        WorkQueues wq;
        wq.table = meta + qp.table;
        wq.counters = meta + qp.counters;
        wq.num_seqs = qp.n;
        wq.queues = qp.queues;
        wq.items = qp.items;
        return launch_attention_persistent(qa, ka, va, cu_q, cu_k, n, H, p.scale, causal, dst, dst_lse, dst_stride,
                                           wq, stream, as);
    };
    auto chunk_attn = [&](const bf16_t* qc, const int32_t* cu_q, const int32_t* cu_k, int32_t n, int32_t max_q,
                          const SplitPlan& sp, int64_t rows_lo, int64_t rows_hi, bf16_t* dst, float* dst_lse,
                          int64_t dst_stride, const QueuePlan& qp) -> int {
        if (sp.splits <= 1)
            return attend(qc, ws_k, ws_v, cu_q, cu_k, n, max_q, false, dst, dst_lse, dst_stride, qp, AttnSplit{});
        const int64_t R = L.split_rows;
        AttnSplit as;
        as.splits = sp.splits;
        as.split_keys = sp.split_keys;
        as.out_stride = R * H * kDv;
        as.lse_stride = H * R;
        MLA_TRY(attend(qc, ws_k, ws_v, cu_q, cu_k, n, max_q, false, split_out, split_lse, R, qp, as));
        return launch_merge_slices(dst + rows_lo * orow, dst_lse + rows_lo, dst_stride, split_out + rows_lo * orow,
                                   split_lse + rows_lo, as.out_stride, as.lse_stride, R, rows_hi - rows_lo, H,
                                   sp.splits, stream);
    };

    for (size_t ci = 0; ci < pb.plan.chunks.size(); ++ci) {
        const mla_chunk_desc& c = pb.plan.chunks[ci];
        const ChunkMeta& m = pb.cmeta[ci];
        MLA_TRY(gather(c, m, meta, ws_k, ws_v, stream));
        const bf16_t* qc = q + c.token_begin * qrow;
        bf16_t* pc = part_out + c.token_begin * orow;
        float* lc = part_lse + c.token_begin;
        int32_t first_direct = 0;
        int64_t q0 = 0;
        if (c.is_continuation) {
            // the first request already holds the previous chunk's result
            q0 = p.query_lens[c.request_begin];
            if (q0 > 0) {
                MLA_TRY(chunk_attn(qc, meta + m.cu_q, meta + m.e_off, 1, static_cast<int32_t>(q0), m.split_cont, 0, q0,
                                   tmp_out, tmp_lse, L.tmp_rows, m.queues_cont));
                MLA_TRY(launch_merge(pc, lc, pc, lc, tmp_out, tmp_lse, q0, H, kDv, T, T, L.tmp_rows, q0, stream));
            }
            first_direct = 1;
        }
        if (c.num_entries > first_direct) {
            MLA_TRY(chunk_attn(qc, meta + m.cu_q + first_direct, meta + m.e_off + first_direct,
                               c.num_entries - first_direct, c.max_query_len, m.split_direct, q0,
                               c.token_end - c.token_begin, pc, lc, T, m.queues_direct));
        }
    }

    const int32_t* scu = meta + pb.suffix_cu;
    MLA_TRY(attend(q, static_cast<const bf16_t*>(p.k_new), static_cast<const bf16_t*>(p.v_new), scu, scu,
                   p.num_requests, pb.max_q, true, suf_out, suf_lse, T, pb.queues_suffix, AttnSplit{}));
    MLA_TRY(launch_merge(static_cast<bf16_t*>(p.out), p.out_lse, part_out, part_lse, suf_out, suf_lse, T, H, kDv,
                         T, T, T, pb.prefix_num_tokens, stream));
    return MLA_OK;
}

// Metadata upload through the pinned staging ring.
int staged_upload(const int32_t* src, size_t count, int32_t* dst, hipStream_t stream) {
    return upload(src, count * sizeof(int32_t), dst, stream);
}

}  // namespace

}  // namespace mla

extern "C" {

int mla_chunked_prefill_scratch_size(const mla_chunked_prefill_params* params, int64_t* bytes) {
    if (bytes == nullptr) return MLA_ERR_INVALID_ARG;
    MLA_TRY(mla::check_params(params));
    mla::Problem pb;
    MLA_TRY(mla::build_problem(*params, pb));
    *bytes = pb.lay.total;
    return MLA_OK;
}

int mla_chunked_prefill(const mla_chunked_prefill_params* params, void* stream_v) {
    using namespace mla;
    MLA_TRY(check_params(params));
    const mla_chunked_prefill_params& p = *params;
    Problem pb;
    MLA_TRY(build_problem(p, pb));
    if (pb.tokens == 0) return MLA_OK;
    MLA_TRY(check_buffers(p, !pb.plan.chunks.empty(), pb.lay.total));
    const int32_t H = p.num_heads;
    auto gather = [&](const mla_chunk_desc& c, const ChunkMeta& m, const int32_t* meta, bf16_t* ws_k, bf16_t* ws_v,
                      hipStream_t stream) {
        return launch_gather(static_cast<const bf16_t*>(p.k_cache), static_cast<const bf16_t*>(p.v_cache),
                             p.num_blocks, p.block_size, H, p.block_table, p.block_table_width, meta + m.e_req,
                             meta + m.e_start, meta + m.e_off, c.num_entries, m.rows, ws_k, ws_v, stream);
    };
    return run_chunked(p, pb, static_cast<hipStream_t>(stream_v), gather, staged_upload);
}

int mla_chunked_prefill_no_alloc(const mla_chunked_prefill_params* params, void* stream_v) {
    using namespace mla;
    MLA_TRY(check_params(params));
    Problem pb;
    MLA_TRY(build_problem(*params, pb));
    if (pb.tokens == 0) return MLA_OK;
    if (pb.lay.total > static_cast<int64_t>(MLA_NO_ALLOC_SCRATCH_BYTES)) return MLA_ERR_CAPACITY;
    mla_chunked_prefill_params p = *params;
    MLA_TRY(no_alloc_scratch(&p.scratch));
    p.scratch_bytes = static_cast<int64_t>(MLA_NO_ALLOC_SCRATCH_BYTES);
    MLA_TRY(check_buffers(p, !pb.plan.chunks.empty(), pb.lay.total));
    const int32_t H = p.num_heads;
    auto gather = [&](const mla_chunk_desc& c, const ChunkMeta& m, const int32_t* meta, bf16_t* ws_k, bf16_t* ws_v,
                      hipStream_t stream) {
        return launch_gather(static_cast<const bf16_t*>(p.k_cache), static_cast<const bf16_t*>(p.v_cache),
                             p.num_blocks, p.block_size, H, p.block_table, p.block_table_width, meta + m.e_req,
                             meta + m.e_start, meta + m.e_off, c.num_entries, m.rows, ws_k, ws_v, stream);
    };
    return run_chunked(p, pb, static_cast<hipStream_t>(stream_v), gather, write_meta_args);
}

int mla_dcp_chunked_prefill_scratch_size(const mla_chunked_prefill_params* params, const mla_dcp_ranks* ranks,
                                         int64_t* bytes) {
    if (bytes == nullptr || ranks == nullptr) return MLA_ERR_INVALID_ARG;
    MLA_TRY(mla::check_params(params));
    mla::Problem pb;
    MLA_TRY(mla::build_problem(*params, pb, true, ranks->world_size, ranks->interleave));
    *bytes = pb.lay.total;
    return MLA_OK;
}

int mla_dcp_chunked_prefill(const mla_chunked_prefill_params* params, const mla_dcp_ranks* ranks, void* stream_v) {
    using namespace mla;
    MLA_TRY(check_params(params));
    if (ranks == nullptr || ranks->world_size < 1 || ranks->interleave < 1) return MLA_ERR_INVALID_ARG;
    const mla_chunked_prefill_params& p = *params;
    const int32_t D = ranks->world_size;
    Problem pb;
    MLA_TRY(build_problem(p, pb, true, D, ranks->interleave));
    if (pb.tokens == 0) return MLA_OK;
    MLA_TRY(check_buffers(p, false, pb.lay.total));
    if (!pb.plan.chunks.empty()) {
        if (ranks->k_cache == nullptr || ranks->v_cache == nullptr || ranks->block_table == nullptr ||
            ranks->num_blocks == nullptr || ranks->block_table_width == nullptr)
            return MLA_ERR_INVALID_ARG;
        for (int32_t r = 0; r < D; ++r) {
            if (ranks->k_cache[r] == nullptr || ranks->v_cache[r] == nullptr || ranks->block_table[r] == nullptr ||
                !aligned16(ranks->k_cache[r]) || !aligned16(ranks->v_cache[r]) || ranks->num_blocks[r] < 0 ||
                ranks->block_table_width[r] < 0)
                return MLA_ERR_INVALID_ARG;
        }
    }
    const int32_t H = p.num_heads;
    char* base = static_cast<char*>(p.scratch);
    bf16_t* g_k = reinterpret_cast<bf16_t*>(base + pb.lay.g_k);
    bf16_t* g_v = reinterpret_cast<bf16_t*>(base + pb.lay.g_v);
    const int64_t krow = static_cast<int64_t>(H) * kDk, vrow = static_cast<int64_t>(H) * kDv;
    auto gather = [&](const mla_chunk_desc& c, const ChunkMeta& m, const int32_t* meta, bf16_t* ws_k, bf16_t* ws_v,
                      hipStream_t stream) {
        // each rank's padded local rows go where an all-gather would put them
        for (int32_t r = 0; r < D; ++r) {
            const int64_t at = static_cast<int64_t>(r) * m.local_rows;
            MLA_TRY(launch_gather(static_cast<const bf16_t*>(ranks->k_cache[r]),
                                  static_cast<const bf16_t*>(ranks->v_cache[r]), ranks->num_blocks[r], p.block_size,
                                  H, ranks->block_table[r], ranks->block_table_width[r], meta + m.e_req,
                                  meta + m.e_lstart, meta + m.e_loff, c.num_entries, m.local_rows, g_k + at * krow,
                                  g_v + at * vrow, stream));
        }
        return launch_dcp_reorganize(g_k, g_v, H, D, ranks->interleave, m.local_rows, meta + m.e_start,
                                     meta + m.e_off, meta + m.e_loff, c.num_entries, m.rows, ws_k, ws_v, stream);
    };
    return run_chunked(p, pb, static_cast<hipStream_t>(stream_v), gather, staged_upload);
}

}  // extern "C"

extern "C" {

int mla_uniform_window_prefill_scratch_size(const mla_chunked_prefill_params* params, int64_t* bytes) {
    if (bytes == nullptr) return MLA_ERR_INVALID_ARG;
    MLA_TRY(mla::check_params(params));
    mla::WindowProblem pb;
    MLA_TRY(mla::build_window_problem(*params, pb));
    *bytes = pb.lay.total;
    return MLA_OK;
}

int mla_uniform_window_prefill(const mla_chunked_prefill_params* params, void* stream_v) {
    using namespace mla;
    MLA_TRY(check_params(params));
    const mla_chunked_prefill_params& p = *params;
    WindowProblem pb;
    MLA_TRY(build_window_problem(p, pb));
    const int64_t T = pb.tokens;
    const int32_t H = p.num_heads, N = p.num_requests;
    if (T == 0) return MLA_OK;
    MLA_TRY(check_buffers(p, pb.iterations > 0, pb.lay.total));

    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    char* base = static_cast<char*>(p.scratch);
    const Layout& L = pb.lay;
    bf16_t* ws_k = reinterpret_cast<bf16_t*>(base + L.ws_k);
    bf16_t* ws_v = reinterpret_cast<bf16_t*>(base + L.ws_v);
    bf16_t* part_out = reinterpret_cast<bf16_t*>(base + L.part_out);
    float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
    bf16_t* suf_out = reinterpret_cast<bf16_t*>(base + L.suf_out);
    float* suf_lse = reinterpret_cast<float*>(base + L.suf_lse);
    bf16_t* tmp_out = reinterpret_cast<bf16_t*>(base + L.tmp_out);
    float* tmp_lse = reinterpret_cast<float*>(base + L.tmp_lse);
    int32_t* meta = reinterpret_cast<int32_t*>(base + L.meta);

    MLA_TRY(upload(pb.meta.data(), pb.meta.size() * sizeof(int32_t), meta, stream));
    const bf16_t* q = static_cast<const bf16_t*>(p.q);
    const int32_t* qsl = meta + pb.qsl;
    // attention over all N requests, through the launch's work queues when it has them
    auto window_attention = [&](const bf16_t* qa, const bf16_t* ka, const bf16_t* va, const int32_t* cu_q,
                                const int32_t* cu_k, bool causal, bf16_t* dst, float* dst_lse,
                                const QueuePlan& qp) -> int {
        if (qp.table < 0)
            return launch_attention(qa, ka, va, cu_q, cu_k, N, pb.max_q, H, p.scale, causal, dst, dst_lse, T, stream);
        WorkQueues wq;
        wq.table = meta + qp.table;
        wq.counters = meta + qp.counters;
        wq.num_seqs = qp.n;
        wq.queues = qp.queues;
        wq.items = qp.items;
        return launch_attention_persistent(qa, ka, va, cu_q, cu_k, N, H, p.scale, causal, dst, dst_lse, T, wq, stream);
    };

    for (int32_t it = 0; it < pb.iterations; ++it) {
        const int32_t* e_off = meta + pb.it_off[it];
        MLA_TRY(launch_gather(static_cast<const bf16_t*>(p.k_cache), static_cast<const bf16_t*>(p.v_cache),
                              p.num_blocks, p.block_size, H, p.block_table, p.block_table_width, meta + pb.e_req,
                              meta + pb.it_start[it], e_off, N, pb.it_rows[it], ws_k, ws_v, stream));
        // iteration 0 is the context state itself; later ones go through the temporary
        bf16_t* o = it == 0 ? part_out : tmp_out;
        float* l = it == 0 ? part_lse : tmp_lse;
        MLA_TRY(window_attention(q, ws_k, ws_v, qsl, e_off, false, o, l, pb.it_queues[it]));
        if (pb.it_has_empty[it]) MLA_TRY(launch_mask_empty_context(l, T, o, 2, qsl, e_off, N, T, H, kDv, stream));
        if (it > 0) MLA_TRY(launch_merge(part_out, part_lse, part_out, part_lse, tmp_out, tmp_lse, T, H, kDv, T, T, T,
                                         T, stream));
    }

    MLA_TRY(window_attention(q, static_cast<const bf16_t*>(p.k_new), static_cast<const bf16_t*>(p.v_new), qsl, qsl,
                             true, suf_out, suf_lse, pb.queues_suffix));
    MLA_TRY(launch_merge(static_cast<bf16_t*>(p.out), p.out_lse, part_out, part_lse, suf_out, suf_lse, T, H, kDv,
                         T, T, T, pb.prefix_num_tokens, stream));
    return MLA_OK;
}

}  // extern "C"
