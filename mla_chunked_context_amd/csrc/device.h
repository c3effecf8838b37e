// Internal declarations shared by the HIP translation units of libmla_cc.so.
// gfx950 only: MFMA builtins and the bf16 conversion instructions of CDNA4
// are used directly.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_cc.h"
#include "work_queues.h"

namespace mla {

using bf16_t = uint16_t;  // storage type of bfloat16 tensors (raw bits)

constexpr int kDk = MLA_QK_HEAD_DIM;  // 192
constexpr int kDv = MLA_V_HEAD_DIM;   // 128
constexpr int kMaxXcd = 8;  // most XCDs a device may report here (MI355X has 8)

// Compute units and XCDs of the current device (hipDeviceAttributeMultiprocessorCount
// and hipDeviceAttributeNumberOfXccs), looked up once per device.  Workgroups are
// dealt to the XCDs round-robin (workgroup b runs on XCD b % xcds), each XCD with
// its own L2.  Without a visible device (host-only size queries) this is MI355X's
// 256 CUs in 8 XCDs.  xcds is clamped to [1, kMaxXcd].
struct DeviceShape {
    int32_t cus = 256;
    int32_t xcds = 8;
};
DeviceShape device_shape();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Optional event bracketing of launches (mla_kernel_timing_enable).  A
// TimedLaunch records a start event at construction and an end event at
// destruction when timing is on; it does nothing otherwise.
class TimedLaunch {
  public:
    TimedLaunch(int kind, hipStream_t stream);
    ~TimedLaunch();
    TimedLaunch(const TimedLaunch&) = delete;
    TimedLaunch& operator=(const TimedLaunch&) = delete;

  private:
    int kind_;
    hipStream_t stream_;
    int device_ = 0;
    hipEvent_t start_ = nullptr;
};

// Launchers used by both the C ABI wrappers (after argument checks) and the
// chunked-prefill driver.  They only enqueue work and report launch errors.
int launch_init_partial(bf16_t* out, float* lse, int64_t lse_stride, int64_t row_begin, int64_t row_end,
                        int32_t heads, int32_t head_dim, hipStream_t stream);

int launch_merge(bf16_t* out, float* out_lse, const bf16_t* p_out, const float* p_lse, const bf16_t* s_out,
                 const float* s_lse, int64_t tokens, int32_t heads, int32_t head_dim, int64_t out_stride,
                 int64_t p_stride, int64_t s_stride, int64_t prefix_num_tokens, hipStream_t stream);

// LSE merge of `slices` (at most kMaxSlices) key-slice states of head_dim 128
// into out: slice s of token row t is at parts + s * part_stride elements +
// t * heads * 128 with LSE part_lse[s * lse_slice_stride + h * lse_head_stride + t].
constexpr int kMaxSlices = 16;
int launch_merge_slices(bf16_t* out, float* out_lse, int64_t out_lse_stride, const bf16_t* parts,
                        const float* part_lse, int64_t part_stride, int64_t lse_slice_stride, int64_t lse_head_stride,
                        int64_t tokens, int32_t heads, int32_t slices, hipStream_t stream);

int launch_gather(const bf16_t* k_cache, const bf16_t* v_cache, int64_t num_blocks, int32_t block_size,
                  int32_t heads, const int32_t* block_table, int32_t bt_width, const int32_t* e_req,
                  const int32_t* e_start, const int32_t* e_off, int32_t n_entries, int32_t num_rows,
                  bf16_t* ws_k, bf16_t* ws_v, hipStream_t stream);

int launch_dcp_reorganize(const bf16_t* gk, const bf16_t* gv, int32_t heads, int32_t world, int32_t interleave,
                          int32_t local_rows, const int32_t* e_start, const int32_t* e_off, const int32_t* e_loff,
                          int32_t n_entries, int32_t num_rows, bf16_t* ws_k, bf16_t* ws_v, hipStream_t stream);
int launch_mask_empty_context(float* lse, int64_t lse_stride, void* out, int32_t elem_bytes, const int32_t* qsl,
                              const int32_t* csl, int32_t num_requests, int64_t num_tokens, int32_t heads,
                              int32_t head_dim, hipStream_t stream);

// Key split of a non-causal launch: split s of every sequence covers keys
// [s * split_keys, (s + 1) * split_keys) (split_keys a multiple of the 64-key
// tile) and writes its (output, LSE) state at out + s * out_stride elements and
// lse + s * lse_stride floats; the caller LSE-merges the splits.
struct AttnSplit {
    int32_t splits = 1;
    int32_t split_keys = 0;
    int64_t out_stride = 0;
    int64_t lse_stride = 0;
};

// Varlen attention.  causal: query i of a sequence sees keys 0..i of the same
// sequence (cu_k must then equal cu_q).  One workgroup per (sequence, 256-query
// tile, head, split); the query tiles of one (sequence, head, split) run on one
// XCD.
int launch_attention(const bf16_t* q, const bf16_t* k, const bf16_t* v, const int32_t* cu_q,
                     const int32_t* cu_k, int32_t num_seqs, int32_t max_q, int32_t heads, float scale,
                     bool causal, bf16_t* out, float* lse, int64_t lse_stride, hipStream_t stream,
                     const AttnSplit& split = AttnSplit{});

// The same attention as launch_attention, as a persistent launch: one
// workgroup per CU (at most one per item) takes items from its XCD's queue
// and then from the other queues, so the launch ends when the work does on
// every XCD.  Needs work_table_ints(num_seqs, queues) <= kMaxQueueTableInts.
int launch_attention_persistent(const bf16_t* q, const bf16_t* k, const bf16_t* v, const int32_t* cu_q,
                                const int32_t* cu_k, int32_t num_seqs, int32_t heads, float scale, bool causal,
                                bf16_t* out, float* lse, int64_t lse_stride, const WorkQueues& wq,
                                hipStream_t stream, const AttnSplit& split = AttnSplit{});

}  // namespace mla
