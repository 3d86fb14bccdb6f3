// Host-side launchers of the gfx950 kernels.  Arguments are validated by the C ABI
// layer before any of these is called; each returns the HIP launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dsv4 {

// log2 of a supported page size (32, 64 or 256 slots), -1 for any other.
inline int page_shift_of(int page_size) {
  return page_size == 32 ? 5 : page_size == 64 ? 6 : page_size == 256 ? 8 : -1;
}

hipError_t launch_combine(const int32_t* topk, int topk_stride, int topk_width,
                          const int32_t* topk_lens, const int32_t* qsl, const int32_t* seq_lens,
                          const int32_t* block_table, int bt_stride, int B, int T, int top_k,
                          int window, int page_shift, int32_t* combined, int combined_stride,
                          int32_t* combined_lens, hipStream_t stream);

// Compressed-cache form of the combine: indices into a per-request workspace of M rows.
hipError_t launch_combine_compressed(const int32_t* topk, int topk_stride, int topk_width,
                                     const int32_t* topk_lens, const int32_t* qsl,
                                     const int32_t* seq_lens, const int32_t* gather_lens, int B,
                                     int T, int top_k, int ratio, int window, int M, int N,
                                     int32_t* combined, int combined_stride,
                                     int32_t* combined_lens, hipStream_t stream);

// Fills that workspace (a cache of ws_num_pages pages) from the compressed and raw caches.
hipError_t launch_gather_workspace(const uint8_t* comp_cache, int comp_num_pages,
                                   const int32_t* comp_bt, int comp_bt_stride,
                                   const uint8_t* swa_cache, int swa_num_pages,
                                   const int32_t* swa_bt, int swa_bt_stride, int page_shift,
                                   const int32_t* seq_lens, const int32_t* gather_lens, int B,
                                   int ratio, int M, int N, uint8_t* ws, int ws_num_pages,
                                   hipStream_t stream);

// Indexer top-k: the top_k largest-logit causal candidates per token, ascending ids.
hipError_t launch_indexer_topk(const float* logits, int logits_stride, const int32_t* qsl,
                               const int32_t* seq_lens, int B, int T, int ratio, int top_k,
                               int32_t* topk, int topk_stride, int32_t* topk_lens,
                               hipStream_t stream);

hipError_t launch_insert(void* q, const void* kv, const int64_t* positions,
                         const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                         const void* weight, float eps, uint8_t* cache, int num_pages,
                         int page_shift, int kv_dtype, float kv_scale, int T, int H,
                         hipStream_t stream);

hipError_t launch_gather(const uint8_t* cache, int num_pages, int page_shift, int kv_dtype,
                         float kv_scale, const int32_t* slots, int n, void* out,
                         hipStream_t stream);

// The attention launchers below read a cache of dtype kv_dtype (kKvFp8Ds, kKvBf16 or
// kKvFp8E4m3; kv_scale is the fp8 cache's per-tensor scale, ignored otherwise).

// Decode / prefill over index rows from memory.  With a workspace of at least
// attention_workspace_bytes(T, H, idx_stride, prefill) bytes the call may cut rows into
// pieces (a decode batch too small to fill the compute units); workspace may be NULL.
hipError_t launch_attention(const void* q, const uint8_t* cache, int num_pages, int page_shift,
                            int kv_dtype, float kv_scale, const int32_t* indices, int idx_stride,
                            const int32_t* lens, const float* sinks, float softmax_scale, void* out, float* lse,
                            int T, int H, bool prefill, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
// Pieces per row the decode picks for T tokens, H heads and rows of `width` entries
// (1: no split), and the workspace that schedule needs (0 with no split).
int auto_splits(int T, int H, int width, bool prefill);
size_t attention_workspace_bytes(int T, int H, int width, bool prefill);

// Split-slot decode: the row of each token is cut into `splits` 64-aligned pieces whose
// partials go to `workspace` (split_workspace_bytes(T, H, splits) bytes) and are merged.
hipError_t launch_attention_split(const void* q, const uint8_t* cache, int num_pages,
                                  int page_shift, int kv_dtype, float kv_scale,
                                  const int32_t* indices, int idx_stride, const int32_t* lens,
                                  const float* sinks, float softmax_scale, void* out, float* lse,
                                  int T, int H, int splits, void* workspace, hipStream_t stream);
size_t split_workspace_bytes(int T, int H, int splits);

// The split decode's workspace for callers that cannot allocate: a static device array of
// kNoallocScratchBytes per GPU; *ptr receives its address on the current device (taken
// once per device).  Calls that overlap on one GPU share it and race.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// Decode that builds each token's combined index row itself from the combine step's
// inputs (top_k + window <= 4096).
hipError_t launch_attention_topk(const void* q, const uint8_t* cache, int num_pages,
                                 int page_shift, int kv_dtype, float kv_scale, const int32_t* topk,
                                 int topk_stride, int topk_width, const int32_t* topk_lens, const int32_t* qsl,
                                 const int32_t* seq_lens, const int32_t* block_table, int bt_stride,
                                 int B, int top_k, int window, const float* sinks,
                                 float softmax_scale, void* out, float* lse, int T, int H,
                                 hipStream_t stream);

// The insert step and the fused combine + decode in one launch (see sparse_mla_kernel);
// with splits > 1 each row is cut into pieces merged by their lse (workspace as for
// launch_attention_split).
hipError_t launch_attention_step(void* q, const void* kv, const int64_t* positions,
                                 const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                                 const void* q_norm_weight, float eps, uint8_t* cache,
                                 int num_pages, int page_shift, int kv_dtype, float kv_scale,
                                 const int32_t* topk, int topk_stride, int topk_width,
                                 const int32_t* topk_lens,
                                 const int32_t* qsl, const int32_t* seq_lens,
                                 const int32_t* block_table, int bt_stride, int B, int top_k,
                                 int window, const float* sinks, float softmax_scale, void* out,
                                 float* lse, int T, int H, int splits, void* workspace,
                                 hipStream_t stream);

}  // namespace dsv4
