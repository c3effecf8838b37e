// Bandwidth-bound kernels of MLA chunked-context prefill on gfx950:
//   * init of the context partial (output 0, LSE -inf),
//   * merge_attn_states (LSE-weighted merge, threshold copy, empty-state select),
//   * gather of a chunk's context rows out of the paged KV cache.
// All move 16-byte vectors; consecutive lanes touch consecutive vectors.
#include <algorithm>
#include <cmath>

#include "device.h"

namespace mla {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with a non-temporal hint (data read once)
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Blocks are dealt to the `xcds` XCDs round-robin.  For a copy whose rows all
// cost the same, this gives each XCD a contiguous range of block indices
// instead (blocks past the last full set of `xcds` keep their own), so the
// blocks of one XCD stream one contiguous stretch of rows through its L2: the
// gather measured +6-8%.  Kernels whose work is concentrated in a few rows
// (the empty-context mask) keep the round-robin spread.  A bijection on
// [0, gridDim.x).
__device__ __forceinline__ int64_t xcd_contiguous_block(int32_t xcds) {
    const int64_t b = blockIdx.x, per = gridDim.x / xcds;
    return b < per * xcds ? (b % xcds) * per + b / xcds : b;
}

// ---------------------------------------------------------------- init

__global__ __launch_bounds__(kThreads) void init_partial_kernel(uint4* out, float* lse, int64_t lse_stride,
                                                                int64_t row_begin, int64_t rows, int32_t heads,
                                                                int64_t vec_per_token) {
    const int64_t nvec = rows * vec_per_token;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (int64_t i = gid; i < nvec; i += stride) out[i] = make_uint4(0u, 0u, 0u, 0u);
    const int64_t nl = rows * heads;
    for (int64_t i = gid; i < nl; i += stride) {
        const int64_t h = i / rows;
        lse[h * lse_stride + row_begin + (i - h * rows)] = -INFINITY;
    }
}

// ---------------------------------------------------------------- merge

struct MergeArgs {
    uint4* out;
    float* out_lse;
    const uint4* p_out;
    const float* p_lse;
    const uint4* s_out;
    const float* s_lse;
    int64_t tokens;
    int32_t heads;
    int32_t vec_per_row;  // head_dim / 8
    int64_t out_stride, p_stride, s_stride;
    int64_t prefix_num_tokens;
};

// Merge of one 8-element vector of one (token, head) row, given both rows'
// vectors and LSEs.  An empty side (LSE -inf) is never used: the result is
// selected, not multiplied by zero, so NaN or garbage in it cannot leak.
__device__ __forceinline__ uint4 merge_values(float pl, float sl, const uint4& pv, const uint4& sv, float& ol) {
    const bool pe = pl == -INFINITY, se = sl == -INFINITY;
    if (pe && se) {
        ol = -INFINITY;
        return make_uint4(0u, 0u, 0u, 0u);
    }
    if (pe) {
        ol = sl;
        return sv;
    }
    if (se) {
        ol = pl;
        return pv;
    }
    const float m = fmaxf(pl, sl);
    const float wp = expf(pl - m), ws = expf(sl - m);
    const float tot = wp + ws;
    const float fp = wp / tot, fs = ws / tot;
    const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w};
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    uint32_t rw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = fp * bf16_to_f32(pw[k] & 0xffffu) + fs * bf16_to_f32(sw[k] & 0xffffu);
        const float hi = fp * bf16_to_f32(pw[k] >> 16) + fs * bf16_to_f32(sw[k] >> 16);
        rw[k] = pack_bf16x2(lo, hi);
    }
    ol = m + logf(tot);
    return make_uint4(rw[0], rw[1], rw[2], rw[3]);
}

// One vector of one row, for the generic kernel.  The prefix side is not
// read at or past the threshold.
__device__ __forceinline__ void merge_vec(const MergeArgs& a, int64_t t, int32_t h, int64_t vec_index,
                                          bool write_lse) {
    const float sl = a.s_lse[h * a.s_stride + t];
    const uint4 sv = a.s_out[vec_index];
    float ol;
    uint4 res;
    if (t >= a.prefix_num_tokens) {
        res = sv;
        ol = sl;
    } else {
        const float pl = a.p_lse[h * a.p_stride + t];
        const uint4 pv = a.p_out[vec_index];
        res = merge_values(pl, sl, pv, sv, ol);
    }
    a.out[vec_index] = res;
    if (write_lse && a.out_lse != nullptr) a.out_lse[h * a.out_stride + t] = ol;
}

// head_dim 128: (token, head) rows of 256 bytes are taken in memory order.
// A block of 512 lanes is 32 groups of 16 lanes; group g takes rows row0 + g
// and row0 + g + 32, so a block streams 64 consecutive rows (16 KB) of each
// array.  All loads of a lane are issued before any result is formed.  (A
// block of 16 tokens x 4 heads, whose rows lie 32 KB apart, measured 4.7
// TB/s; this order measures 6.1 TB/s.)
constexpr int kMergeThreads = 512;
constexpr int kMergeRowsPerGroup = 2;
constexpr int kMergeRowsPerBlock = kMergeThreads / 16 * kMergeRowsPerGroup;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel_d128(MergeArgs a) {
    const int lane_vec = threadIdx.x & 15;
    const int64_t total = a.tokens * a.heads;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kMergeRowsPerBlock + (threadIdx.x >> 4);
    uint4 pv[kMergeRowsPerGroup], sv[kMergeRowsPerGroup];
    float pl[kMergeRowsPerGroup], sl[kMergeRowsPerGroup];
#pragma unroll
    for (int i = 0; i < kMergeRowsPerGroup; ++i) {
        const int64_t row = row0 + i * (kMergeThreads / 16);
        if (row < total) {
            const int64_t t = row / a.heads;
            const int32_t h = static_cast<int32_t>(row - t * a.heads);
            sv[i] = load_nt(&a.s_out[row * 16 + lane_vec]);
            sl[i] = a.s_lse[h * a.s_stride + t];
            if (t < a.prefix_num_tokens) {  // the prefix is not read at or past the threshold
                pv[i] = load_nt(&a.p_out[row * 16 + lane_vec]);
                pl[i] = a.p_lse[h * a.p_stride + t];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kMergeRowsPerGroup; ++i) {
        const int64_t row = row0 + i * (kMergeThreads / 16);
        if (row < total) {
            const int64_t t = row / a.heads;
            const int32_t h = static_cast<int32_t>(row - t * a.heads);
            float ol = sl[i];
            const uint4 res = t < a.prefix_num_tokens ? merge_values(pl[i], sl[i], pv[i], sv[i], ol) : sv[i];
            a.out[row * 16 + lane_vec] = res;
            if (lane_vec == 0 && a.out_lse != nullptr) a.out_lse[h * a.out_stride + t] = ol;
        }
    }
}

// Merge of the key-slice states of one chunk-attention launch (head_dim 128):
// slice s of (token t, head h) is at parts[s * part_stride + (t * heads + h) *
// 16] with LSE part_lse[s * lse_slice_stride + h * lse_head_stride + t].  The
// slices cover disjoint keys, so the result is their LSE combination, formed
// in fp32 and rounded once.  A slice with LSE -inf (no keys) is not read.
struct SliceMergeArgs {
    uint4* out;
    float* out_lse;
    int64_t out_lse_stride;
    const uint4* parts;
    const float* part_lse;
    int64_t part_stride;  // 16-byte vectors between slices
    int64_t lse_slice_stride, lse_head_stride;
    int64_t tokens;
    int32_t heads;
    int32_t slices;
};

__global__ __launch_bounds__(kMergeThreads) void merge_slices_kernel(SliceMergeArgs a) {
    const int lane_vec = threadIdx.x & 15;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * (kMergeThreads / 16) + (threadIdx.x >> 4);
    if (row >= a.tokens * a.heads) return;
    const int64_t t = row / a.heads;
    const int32_t h = static_cast<int32_t>(row - t * a.heads);
    float l[kMaxSlices];
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s) {
        l[s] = s < a.slices ? a.part_lse[s * a.lse_slice_stride + h * a.lse_head_stride + t] : -INFINITY;
        m = fmaxf(m, l[s]);
    }
    uint4 v[kMaxSlices];
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s)
        if (l[s] != -INFINITY) v[s] = load_nt(&a.parts[s * a.part_stride + row * 16 + lane_vec]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s) {
        if (l[s] == -INFINITY) continue;
        const float w = expf(l[s] - m);
        tot += w;
        const uint32_t wd[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[2 * k] += w * bf16_to_f32(wd[k] & 0xffffu);
            acc[2 * k + 1] += w * bf16_to_f32(wd[k] >> 16);
        }
    }
    uint4 res = make_uint4(0u, 0u, 0u, 0u);
    float ol = -INFINITY;
    if (m != -INFINITY) {
        const float inv = 1.f / tot;
        res = make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                         pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
        ol = m + logf(tot);
    }
    a.out[row * 16 + lane_vec] = res;
    if (lane_vec == 0) a.out_lse[h * a.out_lse_stride + t] = ol;
}

// any head_dim that is a multiple of 8
__global__ __launch_bounds__(kThreads) void merge_kernel_generic(MergeArgs a) {
    const int64_t total = a.tokens * a.heads * a.vec_per_row;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total; i += stride) {
        const int64_t row = i / a.vec_per_row;
        const int32_t j = static_cast<int32_t>(i - row * a.vec_per_row);
        const int64_t t = row / a.heads;
        const int32_t h = static_cast<int32_t>(row - t * a.heads);
        merge_vec(a, t, h, i, j == 0);
    }
}

// ---------------------------------------------------------------- gather

constexpr int kGatherThreads = 512;  // one workspace row (H = 128: 80 KB) per block
constexpr int kGatherBatch = 16;     // 16-byte vectors in flight per lane (K and V of a row together)

// Rows per block: one row when a row holds more than 4 vectors per lane
// (H >= 52), else about 4 vectors per lane and at least 2 rows.  At 16 heads
// 3 rows per block (7.5 KB of loads in flight per lane group) measured
// 5.82-5.88 TB/s against 5.62-5.65 with 6 rows and 5.58-5.66 with 2 (one box).
inline int32_t gather_rows_per_block(int32_t heads) {
    const int32_t row_vectors = heads * (kDk + kDv) / 8;
    if (row_vectors > kGatherThreads * 4) return 1;
    return std::max<int32_t>(2, kGatherThreads * 4 / row_vectors);
}
constexpr int kGatherMaxRows = kGatherThreads * 4 / ((kDk + kDv) / 8);  // rows per block at one head

// Copy of `rows` consecutive workspace rows whose cache rows are src_rows[]
// (-1: write NaN): the rows' K and V vectors form one sequence of
// rows * (kvec + vvec) vectors, copied kGatherBatch per lane at a time.
__device__ __forceinline__ void copy_rows(const uint4* __restrict__ k_cache, const uint4* __restrict__ v_cache,
                                          const int64_t* src_rows, uint4* __restrict__ kdst,
                                          uint4* __restrict__ vdst, int32_t rows, int kvec, int vvec) {
    const uint4 nan4 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
    const int n = kvec + vvec;
    const int total = rows * n;
    for (int base = threadIdx.x; base < total; base += kGatherThreads * kGatherBatch) {
        uint4 r[kGatherBatch];
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
            const int idx = base + u * kGatherThreads;
            r[u] = nan4;
            if (idx < total) {
                const int rr = idx / n, v = idx - rr * n;
                const int64_t src = src_rows[rr];
                if (src >= 0) r[u] = v < kvec ? load_nt(&k_cache[src * kvec + v]) : load_nt(&v_cache[src * vvec + v - kvec]);
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
            const int idx = base + u * kGatherThreads;
            if (idx < total) {
                const int rr = idx / n, v = idx - rr * n;
                const u32x4_t val = {r[u].x, r[u].y, r[u].z, r[u].w};
                if (v < kvec)
                    __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(&kdst[static_cast<int64_t>(rr) * kvec + v]));
                else
                    __builtin_nontemporal_store(
                        val, reinterpret_cast<u32x4_t*>(&vdst[static_cast<int64_t>(rr) * vvec + v - kvec]));
            }
        }
    }
}

// Copy of one workspace row (its K vectors, then its V vectors, as one
// sequence of kvec + vvec 16-byte vectors): every lane issues up to
// kGatherBatch loads before its stores.  The cache is read once: non-temporal
// loads keep it from displacing lines that are reused.
__device__ __forceinline__ void copy_row(const uint4* __restrict__ ksrc, const uint4* __restrict__ vsrc,
                                         uint4* __restrict__ kdst, uint4* __restrict__ vdst, int kvec, int vvec,
                                         bool ok) {
    const uint4 nan4 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
    const int n = kvec + vvec;
    for (int base = threadIdx.x; base < n; base += kGatherThreads * kGatherBatch) {
        uint4 r[kGatherBatch];
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
            const int v = base + u * kGatherThreads;
            r[u] = nan4;
            if (ok && v < n) r[u] = v < kvec ? load_nt(&ksrc[v]) : load_nt(&vsrc[v - kvec]);
        }
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
            const int v = base + u * kGatherThreads;
            if (v < n) {
                const u32x4_t val = {r[u].x, r[u].y, r[u].z, r[u].w};
                if (v < kvec)
                    __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(&kdst[v]));
                else
                    __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(&vdst[v - kvec]));
            }
        }
    }
}

template <bool kMultiRow>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const uint4* __restrict__ k_cache, const uint4* __restrict__ v_cache, int64_t num_blocks, int32_t block_size,
    int32_t heads, const int32_t* __restrict__ block_table, int32_t bt_width, const int32_t* __restrict__ e_req,
    const int32_t* __restrict__ e_start, const int32_t* __restrict__ e_off, int32_t n_entries, int32_t num_rows,
    int32_t rows_per_block, int32_t xcds, uint4* __restrict__ ws_k, uint4* __restrict__ ws_v) {
    const int32_t row0 = static_cast<int32_t>(xcd_contiguous_block(xcds)) * rows_per_block;
    if (row0 >= num_rows) return;
    // entry owning row0: the last i with e_off[i] <= row0 (skips empty entries)
    int32_t lo = 0, hi = n_entries - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (e_off[mid] <= row0) lo = mid; else hi = mid - 1;
    }
    int32_t e = lo;
    const int kvec = heads * (kDk / 8), vvec = heads * (kDv / 8);
    // cache row of workspace row w (-1: the block table has no valid entry)
    auto source = [&](int32_t w) -> int64_t {
        while (e + 1 < n_entries && e_off[e + 1] <= w) ++e;
        const int32_t req = e_req[e];
        const int64_t p = static_cast<int64_t>(e_start[e]) + (w - e_off[e]);
        const int64_t lb = p / block_size;
        const int32_t slot = static_cast<int32_t>(p - lb * block_size);
        if (lb >= bt_width || req < 0) return -1;
        const int64_t blk = block_table[static_cast<int64_t>(req) * bt_width + lb];
        return blk >= 0 && blk < num_blocks ? blk * block_size + slot : -1;
    };
    if (!kMultiRow) {
        const int64_t src = source(row0);
        const int64_t s0 = src < 0 ? 0 : src;
        copy_row(k_cache + s0 * kvec, v_cache + s0 * vvec, ws_k + static_cast<int64_t>(row0) * kvec,
                 ws_v + static_cast<int64_t>(row0) * vvec, kvec, vvec, src >= 0);
        return;
    }
    // several short rows (small head counts): look every row's source up once,
    // then copy the rows as one sequence of vectors, so that each lane keeps up
    // to kGatherBatch loads in flight across rows
    __shared__ int64_t src_rows[kGatherMaxRows];
    const int32_t rows = min(rows_per_block, num_rows - row0);
    if (threadIdx.x == 0)
        for (int32_t rr = 0; rr < rows; ++rr) src_rows[rr] = source(row0 + rr);
    __syncthreads();
    copy_rows(k_cache, v_cache, src_rows, ws_k + static_cast<int64_t>(row0) * kvec,
              ws_v + static_cast<int64_t>(row0) * vvec, rows, kvec, vvec);
}

// ---------------------------------------------------------- DCP assembly

// Rows of an all-gathered DCP workspace back in request order.  The gathered
// buffer stacks `world` rank workspaces of `local_rows` rows each; rank r's
// block holds, for entry e, its local rows from local start e_start[e]/world
// at offset e_loff[e].  Output row w of entry e is context position
// p = e_start[e] + (w - e_off[e]), held by rank (p / il) % world at local index
// (p / (il * world)) * il + p % il.  Rows are copied like the gather; a source
// row outside the gathered buffer (inconsistent metadata) is written as NaN.
__global__ __launch_bounds__(kGatherThreads) void dcp_reorganize_kernel(
    const uint4* __restrict__ gk, const uint4* __restrict__ gv, int32_t heads, int32_t world, int32_t il,
    int32_t local_rows, const int32_t* __restrict__ e_start, const int32_t* __restrict__ e_off,
    const int32_t* __restrict__ e_loff, int32_t n_entries, int32_t num_rows, int32_t rows_per_block, int32_t xcds,
    uint4* __restrict__ ws_k, uint4* __restrict__ ws_v) {
    const int32_t row0 = static_cast<int32_t>(xcd_contiguous_block(xcds)) * rows_per_block;
    if (row0 >= num_rows) return;
    int32_t lo = 0, hi = n_entries - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (e_off[mid] <= row0) lo = mid; else hi = mid - 1;
    }
    int32_t e = lo;
    const int kvec = heads * (kDk / 8), vvec = heads * (kDv / 8);
    const int64_t total = static_cast<int64_t>(world) * local_rows;
    for (int rr = 0; rr < rows_per_block; ++rr) {
        const int32_t w = row0 + rr;
        if (w >= num_rows) break;
        while (e + 1 < n_entries && e_off[e + 1] <= w) ++e;
        const int64_t s = e_start[e];
        const int64_t p = s + (w - e_off[e]);
        const int64_t rank = (p / il) % world;
        const int64_t local = (p / (static_cast<int64_t>(il) * world)) * il + p % il;
        int64_t src = rank * local_rows + e_loff[e] + (local - s / world);
        const bool ok = src >= 0 && src < total;
        if (!ok) src = 0;
        copy_row(gk + src * kvec, gv + src * vvec, ws_k + static_cast<int64_t>(w) * kvec,
                 ws_v + static_cast<int64_t>(w) * vvec, kvec, vvec, ok);
    }
}

// ---------------------------------------------------------------- mask

// One wave per token row.  The row's request is found by a wavefront-parallel
// search over query_start_loc: lanes load a window of 64 consecutive entries
// and a ballot of (entry <= token) counts how many of them start at or before
// it; the last such entry is the request (requests with no queries share a
// start with their successor and are skipped by taking the last).  No
// per-token metadata is needed.
constexpr int kMaskWavesPerBlock = kThreads / 64;

__global__ __launch_bounds__(kThreads) void mask_empty_context_kernel(
    float* lse, int64_t lse_stride, uint32_t* out, int64_t row_words, bool vec16, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ csl, int32_t num_requests, int64_t num_tokens, int32_t heads) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kMaskWavesPerBlock + (threadIdx.x >> 6);
    if (t >= num_tokens) return;
    int32_t r = -1;
    for (int32_t base = 0; base <= num_requests; base += 64) {
        const int32_t idx = base + lane;
        const bool le = idx <= num_requests && qsl[idx] <= t;
        const uint64_t m = __builtin_amdgcn_ballot_w64(le);
        const int cnt = __builtin_popcountll(m);
        if (cnt > 0) r = base + cnt - 1;
        if (cnt < 64) break;
    }
    if (r < 0 || r >= num_requests) return;  // a row past the last request is left alone
    if (csl[r + 1] - csl[r] != 0) return;
    for (int h = lane; h < heads; h += 64) lse[h * lse_stride + t] = -INFINITY;
    uint32_t* row = out + t * row_words;
    if (vec16) {  // 16-byte aligned rows: one 16-byte store per lane per 1 KB
        uint4* row4 = reinterpret_cast<uint4*>(row);
        for (int64_t w = lane; w < row_words / 4; w += 64) row4[w] = make_uint4(0u, 0u, 0u, 0u);
    } else {
        for (int64_t w = lane; w < row_words; w += 64) row[w] = 0u;
    }
}

int grid_for(int64_t work, int64_t per_block, int64_t cap) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return static_cast<int>(g);
}

}  // namespace

int launch_init_partial(bf16_t* out, float* lse, int64_t lse_stride, int64_t row_begin, int64_t row_end,
                        int32_t heads, int32_t head_dim, hipStream_t stream) {
    const int64_t rows = row_end - row_begin;
    if (rows <= 0) return MLA_OK;
    const int64_t vpt = static_cast<int64_t>(heads) * head_dim / 8;
    uint4* o = reinterpret_cast<uint4*>(out + row_begin * heads * head_dim);
    const int grid = grid_for(rows * vpt, kThreads * 4, 8192);
    TimedLaunch timed(MLA_KERNEL_INIT, stream);
    hipLaunchKernelGGL(init_partial_kernel, dim3(grid), dim3(kThreads), 0, stream, o, lse, lse_stride, row_begin,
                       rows, heads, vpt);
    return hip_status(hipGetLastError());
}

int launch_merge_slices(bf16_t* out, float* out_lse, int64_t out_lse_stride, const bf16_t* parts,
                        const float* part_lse, int64_t part_stride, int64_t lse_slice_stride, int64_t lse_head_stride,
                        int64_t tokens, int32_t heads, int32_t slices, hipStream_t stream) {
    if (tokens <= 0) return MLA_OK;
    if (slices < 1 || slices > kMaxSlices || part_stride % 8 != 0) return MLA_ERR_INVALID_ARG;
    SliceMergeArgs a{reinterpret_cast<uint4*>(out), out_lse, out_lse_stride, reinterpret_cast<const uint4*>(parts),
                     part_lse, part_stride / 8, lse_slice_stride, lse_head_stride, tokens, heads, slices};
    const int64_t rows = tokens * heads;
    const unsigned grid = static_cast<unsigned>((rows + kMergeThreads / 16 - 1) / (kMergeThreads / 16));
    TimedLaunch timed(MLA_KERNEL_MERGE, stream);
    hipLaunchKernelGGL(merge_slices_kernel, dim3(grid), dim3(kMergeThreads), 0, stream, a);
    return hip_status(hipGetLastError());
}

int launch_merge(bf16_t* out, float* out_lse, const bf16_t* p_out, const float* p_lse, const bf16_t* s_out,
                 const float* s_lse, int64_t tokens, int32_t heads, int32_t head_dim, int64_t out_stride,
                 int64_t p_stride, int64_t s_stride, int64_t prefix_num_tokens, hipStream_t stream) {
    if (tokens <= 0) return MLA_OK;
    MergeArgs a{reinterpret_cast<uint4*>(out), out_lse, reinterpret_cast<const uint4*>(p_out), p_lse,
                reinterpret_cast<const uint4*>(s_out), s_lse, tokens, heads, head_dim / 8, out_stride, p_stride,
                s_stride, prefix_num_tokens};
    TimedLaunch timed(MLA_KERNEL_MERGE, stream);
    if (head_dim == 128) {
        const int64_t rows = tokens * heads;
        const unsigned grid = static_cast<unsigned>((rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock);
        hipLaunchKernelGGL(merge_kernel_d128, dim3(grid), dim3(kMergeThreads), 0, stream, a);
    } else {
        const int grid = grid_for(tokens * heads * (head_dim / 8), kThreads, 16384);
        hipLaunchKernelGGL(merge_kernel_generic, dim3(grid), dim3(kThreads), 0, stream, a);
    }
    return hip_status(hipGetLastError());
}

int launch_gather(const bf16_t* k_cache, const bf16_t* v_cache, int64_t num_blocks, int32_t block_size,
                  int32_t heads, const int32_t* block_table, int32_t bt_width, const int32_t* e_req,
                  const int32_t* e_start, const int32_t* e_off, int32_t n_entries, int32_t num_rows,
                  bf16_t* ws_k, bf16_t* ws_v, hipStream_t stream) {
    if (num_rows <= 0 || n_entries <= 0) return MLA_OK;
    const int32_t rows_per_block = gather_rows_per_block(heads);
    const unsigned grid = static_cast<unsigned>((num_rows + rows_per_block - 1) / rows_per_block);
    TimedLaunch timed(MLA_KERNEL_GATHER, stream);
    // one row per block (large head counts) and several short rows per block
    // are separate instantiations, so that each keeps its own register count
    auto kernel = rows_per_block == 1 ? gather_kernel<false> : gather_kernel<true>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kGatherThreads), 0, stream,
                       reinterpret_cast<const uint4*>(k_cache), reinterpret_cast<const uint4*>(v_cache), num_blocks,
                       block_size, heads, block_table, bt_width, e_req, e_start, e_off, n_entries, num_rows,
                       rows_per_block, device_shape().xcds, reinterpret_cast<uint4*>(ws_k),
                       reinterpret_cast<uint4*>(ws_v));
    return hip_status(hipGetLastError());
}

int launch_dcp_reorganize(const bf16_t* gk, const bf16_t* gv, int32_t heads, int32_t world, int32_t interleave,
                          int32_t local_rows, const int32_t* e_start, const int32_t* e_off, const int32_t* e_loff,
                          int32_t n_entries, int32_t num_rows, bf16_t* ws_k, bf16_t* ws_v, hipStream_t stream) {
    if (num_rows <= 0 || n_entries <= 0) return MLA_OK;
    const int32_t rows_per_block = gather_rows_per_block(heads);
    const unsigned grid = static_cast<unsigned>((num_rows + rows_per_block - 1) / rows_per_block);
    TimedLaunch timed(MLA_KERNEL_DCP_REORG, stream);
    hipLaunchKernelGGL(dcp_reorganize_kernel, dim3(grid), dim3(kGatherThreads), 0, stream,
                       reinterpret_cast<const uint4*>(gk), reinterpret_cast<const uint4*>(gv), heads, world,
                       interleave, local_rows, e_start, e_off, e_loff, n_entries, num_rows, rows_per_block,
                       device_shape().xcds, reinterpret_cast<uint4*>(ws_k), reinterpret_cast<uint4*>(ws_v));
    return hip_status(hipGetLastError());
}

int launch_mask_empty_context(float* lse, int64_t lse_stride, void* out, int32_t elem_bytes, const int32_t* qsl,
                              const int32_t* csl, int32_t num_requests, int64_t num_tokens, int32_t heads,
                              int32_t head_dim, hipStream_t stream) {
    if (num_tokens <= 0) return MLA_OK;
    const int64_t row_words = static_cast<int64_t>(heads) * head_dim * elem_bytes / 4;
    const bool vec16 = aligned16(out) && row_words % 4 == 0;
    const unsigned grid = static_cast<unsigned>((num_tokens + kMaskWavesPerBlock - 1) / kMaskWavesPerBlock);
    TimedLaunch timed(MLA_KERNEL_MASK, stream);
    hipLaunchKernelGGL(mask_empty_context_kernel, dim3(grid), dim3(kThreads), 0, stream, lse, lse_stride,
                       static_cast<uint32_t*>(out), row_words, vec16, qsl, csl, num_requests, num_tokens, heads);
    return hip_status(hipGetLastError());
}

}  // namespace mla

// ----------------------------------------------------------------------------
// C ABI

extern "C" {

int mla_init_context_partial(void* out, float* lse, int64_t lse_head_stride, int64_t row_begin, int64_t row_end,
                             int32_t num_heads, int32_t head_dim, void* stream) {
    if (row_begin < 0 || row_end < row_begin || num_heads < 1 || head_dim < 8 || head_dim % 8 != 0)
        return MLA_ERR_INVALID_ARG;
    if (row_end == row_begin) return MLA_OK;
    if (out == nullptr || lse == nullptr || !mla::aligned16(out) || lse_head_stride < row_end)
        return MLA_ERR_INVALID_ARG;
    return mla::launch_init_partial(static_cast<mla::bf16_t*>(out), lse, lse_head_stride, row_begin, row_end,
                                    num_heads, head_dim, static_cast<hipStream_t>(stream));
}

int mla_merge_attn_states(void* out, float* out_lse, const void* prefix_out, const float* prefix_lse,
                          const void* suffix_out, const float* suffix_lse, int64_t num_tokens, int32_t num_heads,
                          int32_t head_dim, int64_t out_lse_stride, int64_t prefix_lse_stride,
                          int64_t suffix_lse_stride, int64_t prefix_num_tokens, void* stream) {
    if (num_tokens < 0 || num_heads < 1 || head_dim < 8 || head_dim % 8 != 0 || prefix_num_tokens < 0)
        return MLA_ERR_INVALID_ARG;
    if (num_tokens == 0) return MLA_OK;
    if (out == nullptr || suffix_out == nullptr || suffix_lse == nullptr) return MLA_ERR_INVALID_ARG;
    if (prefix_num_tokens > 0 && (prefix_out == nullptr || prefix_lse == nullptr)) return MLA_ERR_INVALID_ARG;
    if (!mla::aligned16(out) || !mla::aligned16(suffix_out) || (prefix_out && !mla::aligned16(prefix_out)))
        return MLA_ERR_INVALID_ARG;
    if (suffix_lse_stride < num_tokens || (prefix_num_tokens > 0 && prefix_lse_stride < num_tokens) ||
        (out_lse != nullptr && out_lse_stride < num_tokens))
        return MLA_ERR_INVALID_ARG;
    return mla::launch_merge(static_cast<mla::bf16_t*>(out), out_lse, static_cast<const mla::bf16_t*>(prefix_out),
                             prefix_lse, static_cast<const mla::bf16_t*>(suffix_out), suffix_lse, num_tokens,
                             num_heads, head_dim, out_lse_stride, prefix_lse_stride, suffix_lse_stride,
                             prefix_num_tokens, static_cast<hipStream_t>(stream));
}

int mla_gather_context(const void* k_cache, const void* v_cache, int64_t num_blocks, int32_t block_size,
                       int32_t num_heads, const int32_t* block_table, int32_t block_table_width,
                       const int32_t* entry_request, const int32_t* entry_starts, const int32_t* entry_row_offsets,
                       int32_t num_entries, int32_t num_rows, void* ws_k, void* ws_v, void* stream) {
    if (num_blocks < 0 || block_size < 1 || num_heads < 1 || block_table_width < 0 || num_entries < 0 ||
        num_rows < 0)
        return MLA_ERR_INVALID_ARG;
    if (num_rows == 0) return MLA_OK;
    if (num_entries == 0 || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
        entry_request == nullptr || entry_starts == nullptr || entry_row_offsets == nullptr || ws_k == nullptr ||
        ws_v == nullptr)
        return MLA_ERR_INVALID_ARG;
    if (!mla::aligned16(k_cache) || !mla::aligned16(v_cache) || !mla::aligned16(ws_k) || !mla::aligned16(ws_v))
        return MLA_ERR_INVALID_ARG;
    return mla::launch_gather(static_cast<const mla::bf16_t*>(k_cache), static_cast<const mla::bf16_t*>(v_cache),
                              num_blocks, block_size, num_heads, block_table, block_table_width, entry_request,
                              entry_starts, entry_row_offsets, num_entries, num_rows,
                              static_cast<mla::bf16_t*>(ws_k), static_cast<mla::bf16_t*>(ws_v),
                              static_cast<hipStream_t>(stream));
}

}  // extern "C"

extern "C" int mla_mask_empty_context(float* lse, int64_t lse_head_stride, void* output, int32_t elem_bytes,
                                      const int32_t* query_start_loc, const int32_t* context_start_loc,
                                      int32_t num_requests, int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                                      void* stream) {
    if (num_requests < 0 || num_tokens < 0 || num_heads < 1 || head_dim < 1 || (elem_bytes != 2 && elem_bytes != 4))
        return MLA_ERR_INVALID_ARG;
    if ((static_cast<int64_t>(head_dim) * elem_bytes) % 4 != 0) return MLA_ERR_INVALID_ARG;
    if (num_tokens == 0) return MLA_OK;
    if (lse == nullptr || output == nullptr || query_start_loc == nullptr || context_start_loc == nullptr ||
        lse_head_stride < num_tokens || (reinterpret_cast<uintptr_t>(output) & 3u) != 0)
        return MLA_ERR_INVALID_ARG;
    return mla::launch_mask_empty_context(lse, lse_head_stride, output, elem_bytes, query_start_loc,
                                          context_start_loc, num_requests, num_tokens, num_heads, head_dim,
                                          static_cast<hipStream_t>(stream));
}

extern "C" int mla_dcp_reorganize_context(const void* gathered_k, const void* gathered_v, int32_t num_heads,
                                          int32_t world_size, int32_t interleave, int32_t local_rows,
                                          const int32_t* entry_starts, const int32_t* entry_row_offsets,
                                          const int32_t* entry_local_offsets, int32_t num_entries,
                                          int32_t num_rows, void* ws_k, void* ws_v, void* stream) {
    if (num_heads < 1 || world_size < 1 || interleave < 1 || local_rows < 0 || num_entries < 0 || num_rows < 0)
        return MLA_ERR_INVALID_ARG;
    if (num_rows == 0) return MLA_OK;
    if (num_entries == 0 || gathered_k == nullptr || gathered_v == nullptr || entry_starts == nullptr ||
        entry_row_offsets == nullptr || entry_local_offsets == nullptr || ws_k == nullptr || ws_v == nullptr)
        return MLA_ERR_INVALID_ARG;
    if (!mla::aligned16(gathered_k) || !mla::aligned16(gathered_v) || !mla::aligned16(ws_k) ||
        !mla::aligned16(ws_v))
        return MLA_ERR_INVALID_ARG;
    return mla::launch_dcp_reorganize(static_cast<const mla::bf16_t*>(gathered_k),
                                      static_cast<const mla::bf16_t*>(gathered_v), num_heads, world_size, interleave,
                                      local_rows, entry_starts, entry_row_offsets, entry_local_offsets, num_entries,
                                      num_rows, static_cast<mla::bf16_t*>(ws_k), static_cast<mla::bf16_t*>(ws_v),
                                      static_cast<hipStream_t>(stream));
}
