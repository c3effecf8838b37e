// Varlen attention with LSE for MLA prefill on gfx950 (qk dim 192, v dim 128).
//
// One kernel body serves both attention steps of the chunked prefill:
//   * chunk attention (non-causal): the prefill queries of each request in a
//     chunk against that request's gathered context rows
//     (run_prefill_context_chunk, vLLM PR #50613 digest, 实现拆解 item 4);
//   * suffix attention (causal): new tokens against the new tokens up to
//     themselves (the suffix merged by merge_attn_states, PR #36540 digest).
// Output: O = softmax(scale * q k^T) v in bf16 and LSE = ln sum exp(scale q.k)
// in fp32, stored head-major.
//
// Work decomposition
//   A workgroup owns 256 queries of one (sequence, head): 8 waves x 32
//   queries, two waves per SIMD.  Keys stream through LDS in tiles of 64 (K
//   row-major, V transposed), double-buffered: the next tile's global loads
//   are in flight while the current tile is computed, and one barrier per
//   tile separates the write of one buffer from the reads of the other.
//   The query tiles of one (sequence, head) run on the same XCD and share its
//   L2.  Two launch forms: one workgroup per tile (workgroup ids remapped so
//   that the tiles of a (sequence, head) land on one XCD), and a persistent
//   launch with one workgroup per CU that takes tiles from per-XCD queues,
//   longest first, and steals from the other XCDs' queues once its own is
//   empty (XCDs run at slightly different speeds, so equal shares finish at
//   different times).
//   K/V tiles are read with buffer loads whose descriptor covers exactly the
//   valid keys of the tile: keys past the end read as zero without branches,
//   and are masked to -inf before the softmax.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, wave64)
//   S^T = K Q^T : A = K tile rows from LDS, B = Q fragments held in registers.
//     The accumulator gives each lane one query column (lane & 31) and 16 of
//     each 32-key block's rows, so the running max / sum of a query live in
//     one lane pair (lane, lane ^ 32), combined with one v_permlane32_swap.
//   O^T = V^T P^T : B = P^T taken directly from the S^T accumulators
//     (converted to bf16); A = V^T from LDS.  The 8 keys a lane contributes
//     to one 16-key step are not contiguous in key order (accumulator rows
//     g*4+{0..3} and 8+g*4+{0..3}); V^T is stored in LDS with bits 2 and 3 of
//     the key index swapped so that those 8 keys are one 16-byte read.
//   Both operands of an MFMA use the same (lane group, slot) -> k mapping, so
//   the products are correct whatever order the hardware assigns to k.
//
// Softmax: base-2 exponentials with the scale folded in, p = 2^(s*c - m),
// c = scale * log2(e).  The reference max m of a query is raised only when a
// tile's max exceeds it by more than 2^8 (then O and the sum are rescaled);
// otherwise the stale m is kept, so p <= 256, which fp32 sums and bf16 P
// represent with the same relative precision.  The LSE is m + log2(sum)
// converted to natural log at the end.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQPerWave = 32;
constexpr int kBlockM = kWaves * kQPerWave;  // queries per workgroup
constexpr int kBlockN = 64;                  // keys per tile
constexpr int kKRowBytes = kDk * 2;         // K tile LDS row: 384 B, 24 chunks of 16 B, unpadded
constexpr int kVtStride = kBlockN + 8;       // V^T tile LDS row stride (elements): 144 B
constexpr int kKVecPerRow = kDk / 8;         // 24 16-byte vectors per K row
constexpr int kKLoads = kBlockN * kKVecPerRow / kThreads;  // 3 direct-to-LDS loads per lane
constexpr int kVLoads = 2;                                  // 2 keys x 8 dims per thread
constexpr int kKTileBytes = kBlockN * kKRowBytes;  // 24 KB
constexpr int kVtTileElems = kDv * kVtStride;
// Q rows of a tile reach LDS with direct-to-LDS loads over whole cache lines
// (like K) before they are read as MFMA fragments; the staging area holds the
// tile's 256 rows and doubles as the V^T ring.
constexpr int kQStageBytes = kBlockM * kKRowBytes;  // 96 KB
constexpr int kQStageWaveBytes = kQPerWave * kKRowBytes;  // 12 KB
static_assert(kQStageBytes >= 2 * kVtTileElems * 2, "the V^T ring lies inside the Q staging area");
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr int kBufferConfig = 0x00020000;  // dword 3 of a raw buffer descriptor on gfx9
// s_waitcnt immediate on gfx9: vmcnt in bits 3:0 (and 15:14), expcnt 6:4, lgkmcnt 11:8;
// this one waits for vector memory only
constexpr int kWaitVmcnt0 = 0x0F70;

static_assert(kBlockN * kKVecPerRow == kKLoads * kThreads, "K tile must split evenly over threads");
static_assert(kBlockM == kQueryTileRows, "work queues count query tiles of the kernel's size");
static_assert(kBlockN / 2 * (kDv / 8) == kThreads, "V tile mapping: 32 key pairs x 16 dim groups");

struct AttnArgs {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const int32_t* cu_q;
    const int32_t* cu_k;
    bf16_t* out;
    float* lse;
    int64_t lse_stride;
    int32_t num_seqs;
    int32_t q_tiles;
    int32_t heads;
    int32_t total_tiles;
    float scale_log2;  // scale * log2(e)
    // key split (non-causal only): split s of a sequence attends to keys
    // [s * split_keys, (s + 1) * split_keys) of it and writes its state at
    // out + s * split_out_stride, lse + s * split_lse_stride
    int32_t splits;
    int32_t split_keys;
    int64_t split_out_stride;
    int64_t split_lse_stride;
    int32_t num_xcd;  // XCDs of the device (workgroup b runs on XCD b % num_xcd)
};

// Work queues of a persistent launch (see WorkQueues in device.h).
struct QueueArgs {
    const int32_t* table;
    int32_t* counters;
    int32_t num_seqs;
    int32_t queues;
    int32_t table_ints;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Low (high) 16-bit halves of w0 and w1 packed as (w0 half, w1 half): one
// v_perm_b32 each (byte selector: 0-3 pick bytes of w0, 4-7 bytes of w1).
__device__ __forceinline__ uint32_t lo_halves(uint32_t w0, uint32_t w1) {
    return __builtin_amdgcn_perm(w1, w0, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t w0, uint32_t w1) {
    return __builtin_amdgcn_perm(w1, w0, 0x07060302u);
}

// Position of key (0..63) inside a V^T LDS row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// x of this lane and of lane ^ 32, via one cross-half swap (no LDS).
__device__ __forceinline__ float pair_max(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Workgroups are dealt to the X XCDs round-robin (XCD = bid % X, and each
// XCD starts its share in bid order).  Logical tiles are (group, q tile) with
// group = (sequence, head).  XCD x takes groups x, x + X, x + 2X, ... with all
// q tiles of a group back to back, so the tiles that stream the same K/V rows
// run together under one L2, and every sequence's heads are spread evenly
// over the XCDs whatever the sequence lengths.  Groups past the last full set
// of X keep the identity mapping.
__device__ __forceinline__ int32_t xcd_logical_tile(int32_t bid, int32_t total, int32_t q_tiles, int32_t xcds) {
    const int32_t groups = total / q_tiles;
    const int32_t full = groups / xcds * xcds;
    if (bid >= full * q_tiles) return bid;
    const int32_t x = bid % xcds, j = bid / xcds;
    return (x + xcds * (j / q_tiles)) * q_tiles + j % q_tiles;
}

// Per-item hook of the tile function: begin() runs first in every item,
// after_prologue() once the item's first loads have landed and the first
// barrier has passed (every thread has read the item's coordinates by then).
struct NoHook {
    __device__ void begin() {}
    __device__ void after_prologue() {}
};

// The tile a workgroup takes next, known before its current tile ends: the
// pair's second tile, or the next item (decoded into LDS during the current
// item's prologue).  Its first loads are fetched into L2 a few steps before
// the current tile ends, so that its prologue reads L2, not HBM.
struct NextTile {
    const int32_t* item;  // LDS: seq, head, split, qt of the next item (seq < 0: none), or null
    int32_t qt2;          // >= 0: the pair's second tile (same sequence, head and split, reversed)
};

constexpr int kPrefetchDumpBytes = kThreads / 64 * 256;  // LDS the prefetch loads land in (unread)
constexpr int kPrefetchLeadSteps = 4;                    // steps before a tile's end

// Issues the first loads of tile (seq, head, split, qt, reverse) as one-dword
// direct-to-LDS loads into `dump`, one per 128-byte line of its Q rows and of
// its first two key tiles' K and V rows: they only bring the lines into L2.
// Lines past the tile's rows fall outside the descriptors and read nothing.
template <bool kCausal>
__device__ __forceinline__ void prefetch_tile(const AttnArgs& a, int32_t seq, int32_t head, int32_t split,
                                              int32_t qt, bool reverse, unsigned char* dump) {
    const int32_t q_begin = a.cu_q[seq];
    const int32_t q_len = a.cu_q[seq + 1] - q_begin;
    int32_t k_begin = kCausal ? q_begin : a.cu_k[seq];
    int32_t k_len = kCausal ? q_len : a.cu_k[seq + 1] - k_begin;
    if (!kCausal && a.splits > 1) {
        const int32_t lo = split * a.split_keys;
        k_begin += lo;
        k_len = max(0, min(k_len - lo, a.split_keys));
    }
    const int32_t kv_end = kCausal ? min(k_len, (qt + 1) * kBlockM) : k_len;
    const int32_t n_tiles = (kv_end + kBlockN - 1) / kBlockN;
    const int32_t n_plain = kCausal ? min(n_tiles, qt * kBlockM / kBlockN) : n_tiles;
    // first key of the two first key tiles taken (see key0 in attention_tile)
    const int32_t kfirst = kCausal && reverse && n_plain > 0 ? max(0, n_plain - 2) * kBlockN : 0;
    const int32_t keys = max(0, min(2 * kBlockN, kv_end - kfirst));
    const int32_t rows = max(0, min(kBlockM, q_len - qt * kBlockM));
    const int32_t H = a.heads;
    const int t = threadIdx.x;
    unsigned char* dst = dump + (t >> 6) * 256;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(a.q + (static_cast<int64_t>(q_begin + qt * kBlockM) * H + head) * kDk), 0,
        rows * H * kDk * 2, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(a.k + (static_cast<int64_t>(k_begin + kfirst) * H + head) * kDk), 0,
        keys * H * kDk * 2, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(a.v + (static_cast<int64_t>(k_begin + kfirst) * H + head) * kDv), 0,
        keys * H * kDv * 2, kBufferConfig);
    // Q rows: 3 lines each (768 lines for 256 rows), two loads per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int l = i * kThreads + t;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)dst, 4,
                                                 (l / 3) * H * kDk * 2 + (l % 3) * 128, 0, 0, 0);
    }
    // K rows: 3 lines each (384 lines for 128 keys); V rows: 2 lines each
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)dst, 4,
                                             (t / 3) * H * kDk * 2 + (t % 3) * 128, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)dst, 4,
                                             (t / 2) * H * kDv * 2 + (t % 2) * 128, 0, 0, 0);
}

// One tile: 256 queries (tile qt) of sequence seq, head `head`, key slice
// `split`, against their keys.  Causal tiles take the key tiles below their
// diagonal block first and the diagonal ones last; reverse takes the former
// last to first.  The softmax does not depend on the order, and every query
// has unmasked keys in its wave's first active tile (below the diagonal, or
// key tile 0).
template <bool kCausal, class Hook>
__device__ __forceinline__ void attention_tile(const AttnArgs& a, int32_t seq, int32_t head, int32_t split,
                                               int32_t qt, bool reverse, unsigned char* k_lds, bf16_t* vt_lds,
                                               Hook& hook, const NextTile& next, unsigned char* dump,
                                               unsigned char* q_stage) {
    hook.begin();
    const int32_t q_begin = a.cu_q[seq];
    const int32_t q_len = a.cu_q[seq + 1] - q_begin;
    int32_t k_begin = kCausal ? q_begin : a.cu_k[seq];
    int32_t k_len = kCausal ? q_len : a.cu_k[seq + 1] - k_begin;
    bf16_t* out = a.out;
    float* lse_out = a.lse;
    if (!kCausal && a.splits > 1) {
        const int32_t lo = split * a.split_keys;
        k_begin += lo;
        k_len = max(0, min(k_len - lo, a.split_keys));  // an empty slice writes (0, -inf)
        out += split * a.split_out_stride;
        lse_out += split * a.split_lse_stride;
    }
    const int32_t kv_end = kCausal ? min(k_len, (qt + 1) * kBlockM) : k_len;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int H = a.heads;

    // ---- Q fragments (B operand of S^T = K Q^T), kept in registers.  A
    // fragment load straight from global memory would serve 32 rows (a lane
    // reads its own query's row) and touch 32 cache lines for 1 KB: a tile's Q
    // would then cost the memory pipeline about as much as all its other first
    // loads together.  Each wave instead copies its 32 rows (12 KB) into its
    // part of q_stage with direct-to-LDS loads of 1 KB each (about 9 lines), in
    // the K tile's swizzled row layout, and reads the fragments from there once
    // they land.
    const int32_t q_row = qt * kBlockM + wave * kQPerWave + l32;  // row inside the sequence
    const bool q_valid = q_row < q_len;
    bf16x8 qf[kDk / 16];
    {
        const int32_t rows = max(0, min(kQPerWave, q_len - (q_row - l32)));  // rows past the end read as zero
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(a.q + (static_cast<int64_t>(q_begin + q_row - l32) * H + head) * kDk), 0,
            rows * H * kDk * 2, kBufferConfig);
        unsigned char* dst = q_stage + wave * kQStageWaveBytes;
        // the lane-only offsets are computed here for every tile rather than
        // once per launch (they would be held in registers through the key loop)
        int lane_t = lane;
        asm volatile("" : "+v"(lane_t));
#pragma unroll
        for (int i = 0; i < kQStageWaveBytes / 1024; ++i) {
            // lane writes 16 bytes at i * 1024 + lane * 16: row r, position c ^ ((r >> 1) & 7) holds chunk c
            const int p = i * 64 + lane_t;
            const int r = p / kKVecPerRow;
            const int c = (p % kKVecPerRow) ^ ((r >> 1) & 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(dst + i * 1024),
                                                     16, r * H * kDk * 2 + c * 16, 0, 0, 0);
        }
    }

    f32x16 o_acc[kDv / 32];
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[db][r] = 0.f;
    float m_run = -INFINITY;  // reference max of s * c for this lane pair's query
    float l_run = 0.f;        // this lane's share of the sum of 2^(s*c - m_run)

    // ---- tile staging: per-thread offsets are fixed; the tile base moves
    const bf16_t* kseq = a.k + static_cast<int64_t>(k_begin) * H * kDk + static_cast<int64_t>(head) * kDk;
    const bf16_t* vseq = a.v + static_cast<int64_t>(k_begin) * H * kDv + static_cast<int64_t>(head) * kDv;
    const int32_t k_row_bytes = H * kDk * 2;
    const int32_t v_row_bytes = H * kDv * 2;
    // K tile in LDS: row r (key) holds its 24 16-byte chunks with chunk c at
    // position c ^ ((r >> 1) & 7).  Rows are 384 bytes, so rows of equal parity
    // start on the same bank; the swizzle gives the 16 rows that an MFMA
    // operand load serves together 16 distinct 16-byte bank groups (no
    // conflicts, no padding).  Each wave fills 3 KB of the tile
    // with direct-to-LDS loads (lane l writes 16 bytes at l * 16); the lane
    // picks the global chunk that belongs at that LDS position.
    int32_t k_goff[kKLoads];
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
        const int pbyte = (wave * kKLoads + i) * 1024 + lane * 16;
        const int row = pbyte / kKRowBytes;
        const int chunk = ((pbyte % kKRowBytes) >> 4) ^ ((row >> 1) & 7);
        k_goff[i] = row * k_row_bytes + chunk * 16;
    }
    const int vkp = tid & 31;  // keys 2*vkp, 2*vkp+1 of the tile
    const int vdc = tid >> 5;  // dims 8*vdc .. 8*vdc+7
    const int32_t v_goff = 2 * vkp * v_row_bytes + vdc * 16;
    const int v_lpos = vt_pos(2 * vkp);

    u32x4 vreg[kVLoads], vreg1[kVLoads];
    // K(k0 tile) straight into K buffer `buf` (no registers involved)
    auto load_k = [&](int32_t k0, int buf) {
        const int32_t keys = min(kBlockN, kv_end - k0);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(kseq + static_cast<int64_t>(k0) * H * kDk), 0, keys * k_row_bytes, kBufferConfig);
        unsigned char* dst = k_lds + buf * kKTileBytes + wave * kKLoads * 1024;
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, k_goff[i], 0, 0,
                0);
    };
    auto load_v_into = [&](int32_t k0, u32x4 (&dst)[kVLoads]) {
        const int32_t keys = min(kBlockN, kv_end - k0);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(vseq + static_cast<int64_t>(k0) * H * kDv), 0, keys * v_row_bytes, kBufferConfig);
#pragma unroll
        for (int u = 0; u < kVLoads; ++u)
            dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_goff + u * v_row_bytes, 0, 0);
    };
    auto load_v = [&](int32_t k0) { load_v_into(k0, vreg); };
    auto store_v = [&](int buf) {
        // transpose 2 keys x 8 dims into 8 rows (dims) of 2 keys
        bf16_t* vl = vt_lds + buf * kVtTileElems;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = vreg[0][i], w1 = vreg[1][i];
            const int d0 = vdc * 8 + 2 * i;
            *reinterpret_cast<uint32_t*>(&vl[d0 * kVtStride + v_lpos]) = lo_halves(w0, w1);
            *reinterpret_cast<uint32_t*>(&vl[(d0 + 1) * kVtStride + v_lpos]) = hi_halves(w0, w1);
        }
    };

    const int32_t n_tiles = (kv_end + kBlockN - 1) / kBlockN;
    // first key of the tile taken at step j
    // Causal: key tiles that end past the tile's first query meet its diagonal
    // block (the last n_tiles - n_plain in key order, n_plain a multiple of 4).
    // The others are taken first, in key order or, when reverse, last to first;
    // the diagonal tiles follow in key order.
    const int32_t n_plain = kCausal ? min(n_tiles, qt * kBlockM / kBlockN) : n_tiles;
    auto key0 = [&](int32_t j) { return (kCausal && reverse && j < n_plain ? n_plain - 1 - j : j) * kBlockN; };
    const int32_t wave_first_q = qt * kBlockM + wave * kQPerWave;
    const int32_t wave_last_q = wave_first_q + kQPerWave - 1;
    // per-lane LDS bases; every fragment read is base + a compile-time offset
    // per-lane K fragment addresses for the four values of ks & 3
    // (chunk 2*ks + g sits at (2*ks + g) ^ ((l32 >> 1) & 7) in row kb*32 + l32)
    const unsigned char* k_lane[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) k_lane[m] = k_lds + l32 * kKRowBytes + (((2 * m + g) ^ ((l32 >> 1) & 7)) << 4);
    const bf16_t* v_lane = vt_lds + l32 * kVtStride + g * 8;

    // S^T = K Q^T of one tile, from K buffer `kbuf` (compile-time)
    auto qk = [&](f32x16 (&s)[2], auto kbuf_tag) {
        constexpr int kbuf = decltype(kbuf_tag)::value;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 af = *reinterpret_cast<const bf16x8*>(
                    k_lane[ks & 3] + kbuf * kKTileBytes + kb * 32 * kKRowBytes + (ks >> 2) * 128);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], s[kb], 0, 0, 0);
            }
        // schedule: 6 fragment reads ahead, then alternate MFMA / read
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < 18; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    };

    // Software pipeline over key tiles.  Tile j's scores S(j) are computed one
    // iteration ahead: iteration j does the softmax of S(j) interleaved with
    // O += V(j) P(j) (each P fragment is produced just before the MFMAs that
    // consume it), then issues the MFMAs of S(j+1), whose results are only
    // needed after the barrier.
    // LDS: K runs one tile ahead of V, each in a ring of two buffers.  Iteration
    // j starts by storing V(j+1) (loaded into registers during iteration j-1)
    // over V(j-1), then issues K(j+2) straight into K(j)'s buffer and the
    // register loads of V(j+2); both buffers were last read in iteration j-1.
    // The barrier at the end of the iteration publishes them.
    // Prologue: one round trip.  Q, K(0), K(1) (straight into LDS), V(0) and
    // V(1) (registers) are all in flight together; V(0) is stored once they
    // have landed and every wave has read its Q rows out of the area the V^T
    // ring shares, V(1) at the start of iteration 0.
    f32x16 s_cur[2], s_nxt[2];
    if (n_tiles > 0) {
        load_k(key0(0), 0);
        if (n_tiles > 1) load_k(key0(1), 1);
        load_v(key0(0));
        if (n_tiles > 1) load_v_into(key0(1), vreg1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // direct-to-LDS loads have landed
    // the same wait as an instruction the compiler sees: the prologue's
    // register loads are then known complete on every path into the loop (the
    // prologue's conditional QK leaves a path where they are not, and the loop
    // would otherwise wait for all loads before its first QK MFMA)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    {
        // the same per-lane addresses as the K fragments (row l32 of the wave's
        // rows, the same swizzle), moved to the wave's staging rows
        const int32_t qs = static_cast<int32_t>(q_stage - k_lds) + wave * kQStageWaveBytes;
#pragma unroll
        for (int ks = 0; ks < kDk / 16; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(k_lane[ks & 3] + qs + (ks >> 2) * 128);
        __syncthreads();  // every wave's rows are read (and every K DMA has landed)
    }
    if (n_tiles > 0) store_v(0);
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) vreg[u] = vreg1[u];
    hook.after_prologue();
    if (n_tiles > 0 && (!kCausal || key0(0) <= wave_last_q)) qk(s_cur, std::integral_constant<int, 0>{});
    __syncthreads();  // K(0) is overwritten by K(2) at the end of iteration 0

    // kDiag: the tile meets the diagonal block of a causal query tile (some of
    // its keys lie past some of the tile's queries).  Every other tile runs
    // the plain step: all waves active, no causal mask, and the same basic
    // block structure as the non-causal kernel.
    auto step = [&](int32_t j, auto par_tag, auto diag_tag) {
        constexpr int par = decltype(par_tag)::value;  // j & 1
        constexpr bool kDiag = kCausal && decltype(diag_tag)::value;
        const int32_t k0 = key0(j);
        // V(j+1) over V(j-1); K(j+2) straight into the buffer that held K(j).
        // Both were last read in iteration j-1, before the previous barrier.
        if (j + 1 < n_tiles) store_v(par ^ 1);
        if (j + 2 < n_tiles) {
            load_k(key0(j + 2), par);
            load_v(key0(j + 2));  // stored at the start of iteration j+1
        }
        const bool active = !kDiag || k0 <= wave_last_q;  // a causal wave past this tile skips it

        // ---- mask keys of S(j) past the end (and above the diagonal when causal)
        if (active && ((k0 + kBlockN > kv_end) || (kDiag && k0 + kBlockN - 1 > wave_first_q))) {
            // element (kb, r) holds key k0 + g*4 + kb*32 + (r>>2)*8 + (r&3); the
            // lane's live keys end at min(kv_end - 1, its query row): one
            // compare of a constant against that limit per element
            const int32_t lim = (kDiag ? min(kv_end - 1, q_row) : kv_end - 1) - k0 - g * 4;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) s_cur[kb][r] = -INFINITY;
        }

        auto scores_next = [&]() {
            // ---- MFMAs of S(j+1).  Non-causal: issued unconditionally, so
            // that they share a basic block with the neighbouring VALU work;
            // on the last tile they read the other K buffer's stale (in-bounds)
            // contents and the result is never used.
            if (kDiag) {
                if (j + 1 < n_tiles && key0(j + 1) <= wave_last_q)
                    qk(s_nxt, std::integral_constant<int, par ^ 1>{});
            } else {
                qk(s_nxt, std::integral_constant<int, par ^ 1>{});
            }
        };
        auto softmax_pv = [&]() {
            if (active) {
                // ---- online softmax of S(j) (base 2), lazily raised reference max
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[kb][r]);
                const float m_tile = pair_max(mx) * a.scale_log2;
                const bool raise = m_tile > m_run + kRescaleThreshold;
                const bool any_raise = __builtin_amdgcn_ballot_w64(raise) != 0;
                const float m_new = raise ? m_tile : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 if kept, 0 if m_run was -inf
                m_run = m_new;
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                float psum = 0.f;
                bf16x8 pb[2][2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        uint32_t pk[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const float p0 =
                                __builtin_amdgcn_exp2f(fmaf(s_cur[kb][hh * 8 + 2 * jj], a.scale_log2, -m_use));
                            const float p1 =
                                __builtin_amdgcn_exp2f(fmaf(s_cur[kb][hh * 8 + 2 * jj + 1], a.scale_log2, -m_use));
                            psum += p0 + p1;
                            pk[jj] = pack_bf16x2(p0, p1);
                        }
                        pb[kb][hh] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
                    }
                l_run = l_run * alpha + psum;
                if (any_raise) {
#pragma unroll
                    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o_acc[db][r] *= alpha;
                }

                // ---- O^T += V(j)^T P(j)^T (4 independent accumulator chains)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int db = 0; db < kDv / 32; ++db) {
                            const bf16x8 af = *reinterpret_cast<const bf16x8*>(
                                &v_lane[par * kVtTileElems + db * 32 * kVtStride + kb * 32 + hh * 16]);
                            o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[kb][hh], o_acc[db], 0, 0, 0);
                        }
            }
        };
        // softmax and O update of tile j first; the MFMAs of S(j+1) then run
        // while the wave moves on to the end-of-tile wait and barrier.  The
        // softmax phase runs at raised wave priority: when the two waves of a
        // SIMD are in different phases, the one issuing VALU work goes first
        // and the other's long MFMAs fill in behind it (measured +5%; raising
        // the score phase instead, or both, is slower)
        __builtin_amdgcn_s_setprio(1);
        softmax_pv();
        __builtin_amdgcn_s_setprio(0);
        scores_next();

        // K(j+2) has landed in LDS (the barrier's fence also drains V(j+2))
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
    };
    // The plain tiles run the plain step, the diagonal ones the causal step,
    // each in a loop of its own taking steps in pairs (n_plain is even).
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int32_t j = 0;
    auto run = [&](int32_t j_end, auto diag_tag) {
        for (; j < j_end; j += 2) {
            step(j, P0{}, diag_tag);
            if (j + 1 < j_end) step(j + 1, P1{}, diag_tag);
        }
    };
    // the next tile's first loads go to L2 a few steps before this tile ends:
    // between loops, so that the steps' own code is untouched
    auto prefetch_next = [&]() {
        if (dump == nullptr) return;
        if (next.qt2 >= 0)
            prefetch_tile<kCausal>(a, seq, head, split, next.qt2, true, dump);
        else if (next.item != nullptr && next.item[0] >= 0)
            prefetch_tile<kCausal>(a, next.item[0], next.item[1], next.item[2], next.item[3], false, dump);
    };
    if (kCausal) {
        // (measured: the prefetch slows the suffix down, 1-8%)
        run(n_plain, std::false_type{});
        run(n_tiles, std::true_type{});
    } else {
        run(max(0, n_tiles - kPrefetchLeadSteps) & ~1, std::false_type{});
        prefetch_next();
        run(n_tiles, std::false_type{});
    }

    // ---- epilogue: normalise, write bf16 output rows and the LSE.
    // Every store instruction writes 32 rows (one per query of the wave), so
    // it costs the memory pipeline about one cycle per row whatever its width:
    // the rows are written 16 bytes per lane (eight instructions), not in the
    // accumulator's 8-byte pieces (sixteen).  A tile's stores are still in the
    // pipeline when the next tile's first loads are issued.
    const float l_tot = pair_sum(l_run);
    if (!q_valid) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    {
        // lane (l32, g) holds dims c*8 + g*4 .. +3 of every 8-dim chunk c of
        // its query; one swap across the lane pair per dword gives the lower
        // lane all of chunk 2m and the upper lane all of chunk 2m+1, written
        // as one 16-byte store each.
        bf16_t* orow = out + (static_cast<int64_t>(q_begin + q_row) * H + head) * kDv + g * 8;
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int r0 = 2 * m * 4, r1 = (2 * m + 1) * 4;  // accumulator slots of chunks 2m, 2m+1
                const uint32_t p0 = pack_bf16x2(o_acc[db][r0 + 0] * inv, o_acc[db][r0 + 1] * inv);
                const uint32_t p1 = pack_bf16x2(o_acc[db][r0 + 2] * inv, o_acc[db][r0 + 3] * inv);
                const uint32_t q0 = pack_bf16x2(o_acc[db][r1 + 0] * inv, o_acc[db][r1 + 1] * inv);
                const uint32_t q1 = pack_bf16x2(o_acc[db][r1 + 2] * inv, o_acc[db][r1 + 3] * inv);
                const auto s0 = __builtin_amdgcn_permlane32_swap(p0, q0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(p1, q1, false, false);
                // lower lanes: (own P, upper's P) = (p, s[1]); upper lanes: (lower's Q, own Q) = (s[0], q)
                const uint4 x = g == 0 ? make_uint4(p0, p1, s0[1], s1[1]) : make_uint4(s0[0], s1[0], q0, q1);
                *reinterpret_cast<uint4*>(orow + db * 32 + m * 16) = x;
            }
    }
    if (g == 0) {
        const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        lse_out[head * a.lse_stride + q_begin + q_row] = lse;
    }
}

// Grid form: workgroup bid computes one logical tile.
template <bool kCausal>
__device__ __forceinline__ void attention_grid(const AttnArgs& a, unsigned char* k_lds, bf16_t* vt_lds,
                                               unsigned char* q_stage) {
    const int32_t tile = xcd_logical_tile(blockIdx.x, a.total_tiles, a.q_tiles, a.num_xcd);
    int32_t qt = tile % a.q_tiles;
    int32_t rest = tile / a.q_tiles;
    const int32_t split = kCausal ? 0 : rest % a.splits;
    if (!kCausal) rest /= a.splits;
    const int32_t head = rest % a.heads;
    const int32_t seq = rest / a.heads;
    if (kCausal) qt = a.q_tiles - 1 - qt;  // longest causal tiles first
    if (qt * kBlockM >= a.cu_q[seq + 1] - a.cu_q[seq]) return;
    NoHook hook;
    attention_tile<kCausal>(a, seq, head, split, qt, false, k_lds, vt_lds, hook, NextTile{nullptr, -1}, nullptr,
                            q_stage);
}

// Persistent form.  Thread 0 takes items: one atomic increment of its
// queue's counter per item, issued when an item begins (so that it lands with
// the item's first loads) and decoded from the work table in LDS once the
// item's prologue barrier has passed, into s_next, which every thread reads
// when the item ends (two barriers later).  A queue whose counter has passed
// its item count is left for the next one; after all X queues the workgroup
// ends.  Every workgroup ends after at most (its items + X) increments.
struct QueueHook {
    const QueueArgs* w;
    const int32_t* table;  // LDS copy
    int32_t* s_next;       // LDS: seq, head, split, qt, qt2 (seq < 0: no more work)
    int32_t heads, groups;  // H, H * splits
    bool causal;
    int32_t queue, tried;   // thread 0's current queue and queues left behind
    int32_t pending;        // thread 0's in-flight increment result
    bool enabled;           // takes the next item in this tile (the first tile of an item)

    // System scope: the increment is performed at memory, past the XCDs'
    // separate L2s, so every XCD sees one counter (and the zero the upload
    // wrote before the launch).
    __device__ int32_t take(int32_t q) {
        return __hip_atomic_fetch_add(w->counters + q * kCounterStride, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // item j of the current queue (j may be past its end: move on)
    __device__ void decode(int32_t j) {
        const int32_t X = w->queues;
        for (;;) {
            int32_t item[5];
            if (decode_queue_item(table, w->num_seqs, X, groups, heads, causal, queue, j, item)) {
                for (int k = 0; k < 5; ++k) s_next[k] = item[k];
                return;
            }
            if (++tried >= X) {
                s_next[0] = -1;
                return;
            }
            queue = (queue + 1) % X;
            j = take(queue);
        }
    }
    __device__ void begin() {
        if (enabled && threadIdx.x == 0) pending = take(queue);
    }
    __device__ void after_prologue() {
        if (enabled && threadIdx.x == 0) decode(pending);
    }
};

template <bool kCausal>
__device__ __forceinline__ void attention_queues(const AttnArgs& a, const QueueArgs& w, unsigned char* k_lds,
                                                 bf16_t* vt_lds, int32_t* table, int32_t* s_next,
                                                 unsigned char* dump, unsigned char* q_stage) {
    for (int32_t i = threadIdx.x; i < w.table_ints; i += kThreads) table[i] = w.table[i];
    QueueHook hook;
    hook.w = &w;
    hook.table = table;
    hook.s_next = s_next;
    hook.heads = a.heads;
    hook.groups = a.heads * (kCausal ? 1 : a.splits);
    hook.causal = kCausal;
    hook.tried = 0;
    hook.pending = 0;
    hook.enabled = true;
    // this workgroup's XCD (hardware register XCC_ID, bits 3:0)
    hook.queue = static_cast<int32_t>(__builtin_amdgcn_s_getreg((3 << 11) | 20)) % w.queues;
    __syncthreads();  // the table is in LDS
    if (threadIdx.x == 0) hook.decode(hook.take(hook.queue));
    __syncthreads();
    for (;;) {
        const int32_t seq = s_next[0], head = s_next[1], split = s_next[2], qt = s_next[3], qt2 = s_next[4];
        if (seq < 0) break;
        // a causal pair's short tile runs its keys below the diagonal last to
        // first: the group's long tiles read key block tau at time tau and its
        // short tiles block Q - tau, so a group's workgroups share two key
        // blocks at a time in L2 instead of spreading over all of them.  One
        // call site for both tiles keeps one copy of the tile code.
        const int32_t n_items = kCausal && qt2 >= 0 ? 2 : 1;
        for (int32_t t = 0; t < n_items; ++t) {
            hook.enabled = t == 0;
            const NextTile next{s_next, t + 1 < n_items ? qt2 : -1};
            attention_tile<kCausal>(a, seq, head, split, t == 0 ? qt : qt2, t == 1, k_lds, vt_lds, hook, next, dump,
                                    q_stage);
        }
    }
}

// Distinct entry points so that profiles separate the two steps.
__global__ __launch_bounds__(kThreads, 1) void chunk_attention_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds[2 * kKTileBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vq_lds[kQStageBytes];  // V^T ring and Q staging
    attention_grid<false>(a, k_lds, reinterpret_cast<bf16_t*>(vq_lds), vq_lds);
}

__global__ __launch_bounds__(kThreads, 1) void suffix_attention_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds[2 * kKTileBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vq_lds[kQStageBytes];  // V^T ring and Q staging
    attention_grid<true>(a, k_lds, reinterpret_cast<bf16_t*>(vq_lds), vq_lds);
}

__global__ __launch_bounds__(kThreads, 1) void chunk_attention_queued_kernel(AttnArgs a, QueueArgs w) {
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds[2 * kKTileBytes];
    // V^T ring and Q staging; the next-tile prefetch lands past the V^T ring
    // (those loads complete within the step that issues them, before any
    // later tile stages its Q there)
    __shared__ __attribute__((aligned(1024))) unsigned char vq_lds[kQStageBytes];
    __shared__ int32_t table[kMaxQueueTableInts];
    __shared__ int32_t s_next[5];
    attention_queues<false>(a, w, k_lds, reinterpret_cast<bf16_t*>(vq_lds), table, s_next,
                            vq_lds + kQStageBytes - kPrefetchDumpBytes, vq_lds);
}

__global__ __launch_bounds__(kThreads, 1) void suffix_attention_queued_kernel(AttnArgs a, QueueArgs w) {
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds[2 * kKTileBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vq_lds[kQStageBytes];  // V^T ring and Q staging
    __shared__ int32_t table[kMaxQueueTableInts];
    __shared__ int32_t s_next[5];
    // no next-tile prefetch
    attention_queues<true>(a, w, k_lds, reinterpret_cast<bf16_t*>(vq_lds), table, s_next, nullptr, vq_lds);
}

}  // namespace

namespace {

int fill_args(AttnArgs& a, const bf16_t* q, const bf16_t* k, const bf16_t* v, const int32_t* cu_q,
              const int32_t* cu_k, int32_t num_seqs, int32_t max_q, int32_t heads, float scale, bool causal,
              bf16_t* out, float* lse, int64_t lse_stride, const AttnSplit& split) {
    if (split.splits < 1 || (split.splits > 1 && (causal || split.split_keys < kBlockN || split.split_keys % kBlockN)))
        return MLA_ERR_INVALID_ARG;
    a = AttnArgs{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu_q = cu_q;
    a.cu_k = causal ? cu_q : cu_k;
    a.out = out;
    a.lse = lse;
    a.lse_stride = lse_stride;
    a.num_seqs = num_seqs;
    a.q_tiles = (max_q + kBlockM - 1) / kBlockM;
    a.heads = heads;
    a.splits = split.splits;
    a.split_keys = split.split_keys;
    a.split_out_stride = split.out_stride;
    a.split_lse_stride = split.lse_stride;
    a.num_xcd = device_shape().xcds;
    const int64_t total = static_cast<int64_t>(num_seqs) * a.q_tiles * heads * split.splits;
    if (total > INT32_MAX) return MLA_ERR_UNSUPPORTED;
    a.total_tiles = static_cast<int32_t>(total);
    a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return MLA_OK;
}

}  // namespace

int launch_attention(const bf16_t* q, const bf16_t* k, const bf16_t* v, const int32_t* cu_q, const int32_t* cu_k,
                     int32_t num_seqs, int32_t max_q, int32_t heads, float scale, bool causal, bf16_t* out,
                     float* lse, int64_t lse_stride, hipStream_t stream, const AttnSplit& split) {
    if (num_seqs <= 0 || max_q <= 0) return MLA_OK;
    AttnArgs a;
    const int st = fill_args(a, q, k, v, cu_q, cu_k, num_seqs, max_q, heads, scale, causal, out, lse, lse_stride,
                             split);
    if (st != MLA_OK) return st;
    TimedLaunch timed(causal ? MLA_KERNEL_SUFFIX_ATTN : MLA_KERNEL_CHUNK_ATTN, stream);
    if (causal)
        hipLaunchKernelGGL(suffix_attention_kernel, dim3(a.total_tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(chunk_attention_kernel, dim3(a.total_tiles), dim3(kThreads), 0, stream, a);
    return hip_status(hipGetLastError());
}

int launch_attention_persistent(const bf16_t* q, const bf16_t* k, const bf16_t* v, const int32_t* cu_q,
                                const int32_t* cu_k, int32_t num_seqs, int32_t heads, float scale, bool causal,
                                bf16_t* out, float* lse, int64_t lse_stride, const WorkQueues& wq,
                                hipStream_t stream, const AttnSplit& split) {
    if (num_seqs <= 0 || wq.items <= 0) return MLA_OK;
    if (wq.queues < 1 || wq.queues > kMaxXcd || wq.num_seqs != num_seqs || wq.table == nullptr ||
        wq.counters == nullptr || work_table_ints(num_seqs, wq.queues) > kMaxQueueTableInts)
        return MLA_ERR_INVALID_ARG;
    AttnArgs a;
    const int st = fill_args(a, q, k, v, cu_q, cu_k, num_seqs, kBlockM, heads, scale, causal, out, lse, lse_stride,
                             split);
    if (st != MLA_OK) return st;
    QueueArgs w{wq.table, wq.counters, num_seqs, wq.queues, static_cast<int32_t>(work_table_ints(num_seqs, wq.queues))};
    const int32_t grid = std::min<int32_t>(device_shape().cus, wq.items);
    TimedLaunch timed(causal ? MLA_KERNEL_SUFFIX_ATTN : MLA_KERNEL_CHUNK_ATTN, stream);
    if (causal)
        hipLaunchKernelGGL(suffix_attention_queued_kernel, dim3(grid), dim3(kThreads), 0, stream, a, w);
    else
        hipLaunchKernelGGL(chunk_attention_queued_kernel, dim3(grid), dim3(kThreads), 0, stream, a, w);
    return hip_status(hipGetLastError());
}

}  // namespace mla

// ----------------------------------------------------------------------------
// C ABI

namespace {

int check_attention_args(const void* q, const void* k, const void* v, const int32_t* cu_q, int32_t num_seqs,
                         int32_t max_q, int32_t num_heads, float scale, const void* out, const float* lse,
                         int64_t lse_head_stride) {
    if (num_seqs < 0 || max_q < 0 || num_heads < 1 || num_heads > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
    if (num_seqs == 0 || max_q == 0) return MLA_OK;
    if (q == nullptr || k == nullptr || v == nullptr || cu_q == nullptr || out == nullptr || lse == nullptr)
        return MLA_ERR_INVALID_ARG;
    if (!mla::aligned16(q) || !mla::aligned16(k) || !mla::aligned16(v) || !mla::aligned16(out))
        return MLA_ERR_INVALID_ARG;
    if (lse_head_stride < 1) return MLA_ERR_INVALID_ARG;
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_context_chunk_attn(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                           int32_t num_seqs, int32_t max_q, int32_t num_heads, float scale, void* out, float* lse,
                           int64_t lse_head_stride, void* stream) {
    int st = check_attention_args(q, k, v, cu_q, num_seqs, max_q, num_heads, scale, out, lse, lse_head_stride);
    if (st != MLA_OK || num_seqs == 0 || max_q == 0) return st;
    if (cu_k == nullptr) return MLA_ERR_INVALID_ARG;
    return mla::launch_attention(static_cast<const mla::bf16_t*>(q), static_cast<const mla::bf16_t*>(k),
                                 static_cast<const mla::bf16_t*>(v), cu_q, cu_k, num_seqs, max_q, num_heads, scale,
                                 false, static_cast<mla::bf16_t*>(out), lse, lse_head_stride,
                                 static_cast<hipStream_t>(stream));
}

int mla_causal_suffix_attn(const void* q, const void* k_new, const void* v_new, const int32_t* cu_q,
                           int32_t num_seqs, int32_t max_q, int32_t num_heads, float scale, void* out, float* lse,
                           int64_t lse_head_stride, void* stream) {
    int st = check_attention_args(q, k_new, v_new, cu_q, num_seqs, max_q, num_heads, scale, out, lse,
                                  lse_head_stride);
    if (st != MLA_OK || num_seqs == 0 || max_q == 0) return st;
    return mla::launch_attention(static_cast<const mla::bf16_t*>(q), static_cast<const mla::bf16_t*>(k_new),
                                 static_cast<const mla::bf16_t*>(v_new), cu_q, cu_q, num_seqs, max_q, num_heads,
                                 scale, true, static_cast<mla::bf16_t*>(out), lse, lse_head_stride,
                                 static_cast<hipStream_t>(stream));
}

}  // extern "C"
