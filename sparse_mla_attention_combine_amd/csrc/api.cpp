// C ABI of the library (declared in include/dsv4.h).  Every entry point checks its
// arguments on the host before launching anything; a failure returns a status and a
// thread-local reason string and touches no memory.  The error style follows the
// capability checks of PR #43477 (Key source excerpts, flashinfer_sparse.py
// supports_combination returning a reason string; NotImplementedError for an
// unsupported cache layout).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/dsv4.h"
#include "launch.hpp"
#include "peaks.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return DSV4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSV4_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_page(const char* fn, int page_size, int num_pages) {
  if (dsv4::page_shift_of(page_size) < 0)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: page_size %d not supported (32, 64 or 256)", fn, page_size);
  if (num_pages < 0) return fail(DSV4_ERR_SHAPE, "%s: num_pages %d < 0", fn, num_pages);
  if ((int64_t)num_pages * page_size >= ((int64_t)1 << 31))
    return fail(DSV4_ERR_SHAPE, "%s: num_pages * page_size exceeds the int32 slot range", fn);
  return DSV4_OK;
}

// The cache dtype and, for the per-tensor fp8 cache, its scale (kept where every
// E4M3 value times it, and 448 / it, stay normal fp32 numbers).
int check_kv(const char* fn, int kv_dtype, float kv_scale) {
  if (kv_dtype != DSV4_KV_FP8_DS_MLA && kv_dtype != DSV4_KV_BF16 && kv_dtype != DSV4_KV_FP8_E4M3)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: kv_dtype %d not supported (0 fp8_ds_mla, 1 bf16, 2 fp8_e4m3)",
                fn, kv_dtype);
  if (kv_dtype == DSV4_KV_FP8_E4M3 && !(kv_scale >= 0x1p-64f && kv_scale <= 0x1p64f))
    return fail(DSV4_ERR_SHAPE, "%s: kv_scale %g of the fp8 cache not in [2^-64, 2^64]", fn,
                (double)kv_scale);
  return DSV4_OK;
}

int check_attention(const char* fn, const void* q, const uint8_t* kv_cache, int num_pages,
                    int page_size, int kv_dtype, float kv_scale, const int32_t* indices, int idx_stride, const int32_t* lens,
                    const float* /*sinks*/, float softmax_scale, const void* out, int T, int H) {
  if (T < 0) return fail(DSV4_ERR_SHAPE, "%s: T = %d < 0", fn, T);
  if (H != 16 && H != 32 && H != 64 && H != 128)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: H = %d not in {16, 32, 64, 128}", fn, H);
  int st = check_page(fn, page_size, num_pages);
  if (!st) st = check_kv(fn, kv_dtype, kv_scale);
  if (st) return st;
  if (idx_stride < 0) return fail(DSV4_ERR_SHAPE, "%s: idx_stride %d < 0", fn, idx_stride);
  if (!(softmax_scale == softmax_scale)) return fail(DSV4_ERR_SHAPE, "%s: softmax_scale is NaN", fn);
  if (T == 0) return DSV4_OK;
  if (!q || !out || !lens || (!indices && idx_stride > 0) || (!kv_cache && num_pages > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || (kv_cache && !aligned(kv_cache, 16)))
    return fail(DSV4_ERR_ALIGN, "%s: q, out and kv_cache must be 16-byte aligned", fn);
  if (!aligned(lens, 4) || (indices && !aligned(indices, 4)))
    return fail(DSV4_ERR_ALIGN, "%s: indices and lens must be 4-byte aligned", fn);
  return DSV4_OK;
}

}  // namespace

extern "C" {

const char* dsv4_status_str(int status) {
  switch (status) {
    case DSV4_OK: return "DSV4_OK";
    case DSV4_ERR_NULL: return "DSV4_ERR_NULL";
    case DSV4_ERR_SHAPE: return "DSV4_ERR_SHAPE";
    case DSV4_ERR_ALIGN: return "DSV4_ERR_ALIGN";
    case DSV4_ERR_UNSUPPORTED: return "DSV4_ERR_UNSUPPORTED";
    case DSV4_ERR_WORKSPACE: return "DSV4_ERR_WORKSPACE";
    case DSV4_ERR_HIP: return "DSV4_ERR_HIP";
    default: return "DSV4_UNKNOWN_STATUS";
  }
}

const char* dsv4_last_error(void) { return g_err; }

size_t dsv4_cache_page_bytes(int page_size, int kv_dtype) {
  return page_size > 0 ? (size_t)page_size * (size_t)dsv4::kv_record_bytes_of(kv_dtype) : 0;
}

int dsv4_kv_insert(void* q, const void* kv, const int64_t* positions, const int64_t* slot_mapping,
                   const float* cos_sin, int max_pos, const void* q_norm_weight, float eps,
                   uint8_t* kv_cache, int num_pages, int page_size, int kv_dtype, float kv_scale,
                   int T, int H, void* stream) {
  const char* fn = "dsv4_kv_insert";
  if (T < 0 || H < 0 || H > 128) return fail(DSV4_ERR_SHAPE, "%s: T = %d, H = %d out of range (T >= 0, 0 <= H <= 128)", fn, T, H);
  int st = check_page(fn, page_size, num_pages);
  if (!st) st = check_kv(fn, kv_dtype, kv_scale);
  if (st) return st;
  if (max_pos < 0) return fail(DSV4_ERR_SHAPE, "%s: max_pos %d < 0", fn, max_pos);
  if (!(eps >= 0.f)) return fail(DSV4_ERR_SHAPE, "%s: eps must be >= 0", fn);
  if (T == 0) return ok();
  if (!kv || !positions || !slot_mapping || !cos_sin || (!kv_cache && num_pages > 0) ||
      (H > 0 && (!q || !q_norm_weight)))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if ((H > 0 && (!aligned(q, 16) || !aligned(q_norm_weight, 16))) || !aligned(kv, 16) ||
      (kv_cache && !aligned(kv_cache, 16)) || !aligned(cos_sin, 16) || !aligned(positions, 8) ||
      !aligned(slot_mapping, 8))
    return fail(DSV4_ERR_ALIGN, "%s: q, kv, q_norm_weight, cos_sin, kv_cache must be 16-byte aligned; positions, slot_mapping 8-byte", fn);
  return hip_status(dsv4::launch_insert(q, kv, positions, slot_mapping, cos_sin, max_pos,
                                        q_norm_weight, eps, kv_cache, num_pages,
                                        dsv4::page_shift_of(page_size), kv_dtype, kv_scale, T, H,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_combine_indices(const int32_t* topk, int topk_stride, int topk_width,
                         const int32_t* topk_lens, const int32_t* query_start_loc,
                         const int32_t* seq_lens, const int32_t* block_table,
                         int block_table_stride, int B, int T, int top_k, int window,
                         int page_size, int32_t* combined, int combined_stride,
                         int32_t* combined_lens, void* stream) {
  const char* fn = "dsv4_combine_indices";
  if (B < 0 || T < 0 || top_k < 0 || window < 0 || topk_width < 0 || topk_stride < topk_width ||
      block_table_stride < 0)
    return fail(DSV4_ERR_SHAPE, "%s: negative size or topk_stride < topk_width", fn);
  if (dsv4::page_shift_of(page_size) < 0)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: page_size %d not supported (32, 64 or 256)", fn, page_size);
  if (top_k > topk_width) return fail(DSV4_ERR_SHAPE, "%s: top_k %d > topk_width %d", fn, top_k, topk_width);
  const int64_t need = ((int64_t)top_k + window + DSV4_COMBINE_ALIGN - 1) / DSV4_COMBINE_ALIGN * DSV4_COMBINE_ALIGN;
  if (combined_stride < need)
    return fail(DSV4_ERR_SHAPE, "%s: combined_stride %d < round_up(top_k + window, 128) = %lld", fn,
                combined_stride, (long long)need);
  if (B == 0 || T == 0) return ok();
  if (!query_start_loc || !seq_lens || !combined || !combined_lens || (!topk && topk_width > 0) ||
      (!block_table && block_table_stride > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(combined, 4) || !aligned(combined_lens, 4) || (topk && !aligned(topk, 4)))
    return fail(DSV4_ERR_ALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  return hip_status(dsv4::launch_combine(topk, topk_stride, topk_width, topk_lens, query_start_loc,
                                         seq_lens, block_table, block_table_stride, B, T, top_k,
                                         window, dsv4::page_shift_of(page_size), combined,
                                         combined_stride, combined_lens,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_combine_indices_compressed(const int32_t* topk, int topk_stride, int topk_width,
                                    const int32_t* topk_lens, const int32_t* query_start_loc,
                                    const int32_t* seq_lens, const int32_t* gather_lens, int B,
                                    int T, int top_k, int compress_ratio, int window, int M, int N,
                                    int32_t* combined, int combined_stride, int32_t* combined_lens,
                                    void* stream) {
  const char* fn = "dsv4_combine_indices_compressed";
  if (B < 0 || T < 0 || top_k < 0 || window < 0 || topk_width < 0 || topk_stride < topk_width)
    return fail(DSV4_ERR_SHAPE, "%s: negative size or topk_stride < topk_width", fn);
  if (compress_ratio < 1) return fail(DSV4_ERR_SHAPE, "%s: compress_ratio %d < 1", fn, compress_ratio);
  if (N < 0 || M < N) return fail(DSV4_ERR_SHAPE, "%s: need 0 <= N <= M (N %d, M %d)", fn, N, M);
  if ((int64_t)B * M >= ((int64_t)1 << 31))
    return fail(DSV4_ERR_SHAPE, "%s: B * M exceeds the int32 index range", fn);
  if (top_k > topk_width) return fail(DSV4_ERR_SHAPE, "%s: top_k %d > topk_width %d", fn, top_k, topk_width);
  const int64_t need = ((int64_t)top_k + window + DSV4_COMBINE_ALIGN - 1) / DSV4_COMBINE_ALIGN * DSV4_COMBINE_ALIGN;
  if (combined_stride < need)
    return fail(DSV4_ERR_SHAPE, "%s: combined_stride %d < round_up(top_k + window, 128) = %lld", fn,
                combined_stride, (long long)need);
  if (B == 0 || T == 0) return ok();
  if (!query_start_loc || !seq_lens || !gather_lens || !combined || !combined_lens ||
      (!topk && topk_width > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(combined, 4) || !aligned(combined_lens, 4) || (topk && !aligned(topk, 4)))
    return fail(DSV4_ERR_ALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  return hip_status(dsv4::launch_combine_compressed(topk, topk_stride, topk_width, topk_lens,
                                                    query_start_loc, seq_lens, gather_lens, B, T,
                                                    top_k, compress_ratio, window, M, N, combined,
                                                    combined_stride, combined_lens,
                                                    static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_indexer_topk(const float* logits, int logits_stride, const int32_t* query_start_loc,
                      const int32_t* seq_lens, int B, int T, int compress_ratio, int top_k,
                      int32_t* topk, int topk_stride, int32_t* topk_lens, void* stream) {
  const char* fn = "dsv4_indexer_topk";
  if (B < 0 || T < 0 || top_k < 0 || logits_stride < 0)
    return fail(DSV4_ERR_SHAPE, "%s: negative size", fn);
  if (compress_ratio < 1) return fail(DSV4_ERR_SHAPE, "%s: compress_ratio %d < 1", fn, compress_ratio);
  if (topk_stride < top_k)
    return fail(DSV4_ERR_SHAPE, "%s: topk_stride %d < top_k %d", fn, topk_stride, top_k);
  if (B == 0 || T == 0) return ok();
  if (!query_start_loc || !seq_lens || (!topk && topk_stride > 0) || !topk_lens ||
      (!logits && logits_stride > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if ((logits && !aligned(logits, 4)) || !aligned(topk, 4) || !aligned(topk_lens, 4))
    return fail(DSV4_ERR_ALIGN, "%s: arrays must be 4-byte aligned", fn);
  return hip_status(dsv4::launch_indexer_topk(logits, logits_stride, query_start_loc, seq_lens, B,
                                              T, compress_ratio, top_k, topk, topk_stride,
                                              topk_lens, static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_gather_workspace(const uint8_t* comp_cache, int comp_num_pages,
                          const int32_t* comp_block_table, int comp_bt_stride,
                          const uint8_t* swa_cache, int swa_num_pages,
                          const int32_t* swa_block_table, int swa_bt_stride, int page_size,
                          const int32_t* seq_lens, const int32_t* gather_lens, int B,
                          int compress_ratio, int M, int N, uint8_t* ws_cache, int ws_num_pages,
                          void* stream) {
  const char* fn = "dsv4_gather_workspace";
  int st = check_page(fn, page_size, comp_num_pages);
  if (!st) st = check_page(fn, page_size, swa_num_pages);
  if (!st) st = check_page(fn, page_size, ws_num_pages);
  if (st) return st;
  if (B < 0 || comp_bt_stride < 0 || swa_bt_stride < 0)
    return fail(DSV4_ERR_SHAPE, "%s: negative size", fn);
  if (compress_ratio < 1) return fail(DSV4_ERR_SHAPE, "%s: compress_ratio %d < 1", fn, compress_ratio);
  if (N < 0 || M < N) return fail(DSV4_ERR_SHAPE, "%s: need 0 <= N <= M (N %d, M %d)", fn, N, M);
  if ((int64_t)B * M >= ((int64_t)1 << 31))
    return fail(DSV4_ERR_SHAPE, "%s: B * M exceeds the int32 index range", fn);
  if (B == 0 || M == 0 || ws_num_pages == 0) return ok();
  if (!seq_lens || !gather_lens || !ws_cache || (!comp_cache && comp_num_pages > 0) ||
      (!swa_cache && swa_num_pages > 0) || (!comp_block_table && comp_bt_stride > 0) ||
      (!swa_block_table && swa_bt_stride > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(ws_cache, 16) || (comp_cache && !aligned(comp_cache, 16)) ||
      (swa_cache && !aligned(swa_cache, 16)))
    return fail(DSV4_ERR_ALIGN, "%s: caches must be 16-byte aligned", fn);
  return hip_status(dsv4::launch_gather_workspace(comp_cache, comp_num_pages, comp_block_table,
                                                  comp_bt_stride, swa_cache, swa_num_pages,
                                                  swa_block_table, swa_bt_stride,
                                                  dsv4::page_shift_of(page_size), seq_lens,
                                                  gather_lens, B, compress_ratio, M, N, ws_cache,
                                                  ws_num_pages, static_cast<hipStream_t>(stream)),
                    fn);
}

// decode and prefill: the same checks, the workspace contract, then the launch
static int attention_checked(const char* fn, bool prefill, const void* q, const uint8_t* kv_cache,
                             int num_pages, int page_size, int kv_dtype, float kv_scale,
                             const int32_t* indices, int idx_stride,
                             const int32_t* lens, const float* sinks, float softmax_scale,
                             void* out, float* lse, int T, int H, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int st = check_attention(fn, q, kv_cache, num_pages, page_size, kv_dtype, kv_scale, indices,
                           idx_stride, lens, sinks, softmax_scale, out, T, H);
  if (st) return st;
  if (!workspace && workspace_bytes != 0)
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace is NULL but workspace_bytes is %zu", fn,
                workspace_bytes);
  if (workspace) {
    const size_t need = dsv4::attention_workspace_bytes(T, H, idx_stride, prefill);
    if (!aligned(workspace, 16) || workspace_bytes < need)
      return fail(DSV4_ERR_WORKSPACE,
                  "%s: a workspace must be 16-byte aligned and hold %zu bytes (got %zu)", fn, need,
                  workspace_bytes);
  }
  if (T == 0) return ok();
  return hip_status(dsv4::launch_attention(q, kv_cache, num_pages, dsv4::page_shift_of(page_size),
                                           kv_dtype, kv_scale, indices, idx_stride, lens, sinks,
                                           softmax_scale, out, lse, T, H, prefill, workspace,
                                           workspace_bytes,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_sparse_mla_decode(const void* q, const uint8_t* kv_cache, int num_pages, int page_size,
                           int kv_dtype, float kv_scale, const int32_t* indices, int idx_stride,
                           const int32_t* lens, const float* sinks, float softmax_scale, void* out,
                           float* lse, int T, int H, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return attention_checked("dsv4_sparse_mla_decode", false, q, kv_cache, num_pages, page_size,
                           kv_dtype, kv_scale, indices, idx_stride, lens, sinks, softmax_scale, out, lse, T, H,
                           workspace, workspace_bytes, stream);
}

size_t dsv4_sparse_mla_workspace_bytes(int T, int H, int width, int is_prefill) {
  if (T < 0 || width < 0 || (H != 16 && H != 32 && H != 64 && H != 128)) return 0;
  return dsv4::attention_workspace_bytes(T, H, width, is_prefill != 0);
}

size_t dsv4_sparse_mla_split_workspace_bytes(int T, int H, int splits) {
  if (T < 0 || H < 0 || splits < 0) return 0;
  return dsv4::split_workspace_bytes(T, H, splits);
}

int dsv4_sparse_mla_decode_split(const void* q, const uint8_t* kv_cache, int num_pages,
                                 int page_size, int kv_dtype, float kv_scale,
                                 const int32_t* indices, int idx_stride, const int32_t* lens,
                                 const float* sinks, float softmax_scale, void* out, float* lse,
                                 int T, int H, int splits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "dsv4_sparse_mla_decode_split";
  int st = check_attention(fn, q, kv_cache, num_pages, page_size, kv_dtype, kv_scale, indices,
                           idx_stride, lens, sinks, softmax_scale, out, T, H);
  if (st) return st;
  if (splits < 1 || splits > 64) return fail(DSV4_ERR_SHAPE, "%s: splits %d not in 1..64", fn, splits);
  if (T == 0) return ok();
  if (splits == 1)
    return hip_status(dsv4::launch_attention(q, kv_cache, num_pages, dsv4::page_shift_of(page_size),
                                             kv_dtype, kv_scale, indices, idx_stride, lens, sinks,
                                             softmax_scale, out, lse, T, H, false, nullptr, 0,
                                             static_cast<hipStream_t>(stream)),
                      fn);
  if ((int64_t)T * splits >= ((int64_t)1 << 31) / 8)
    return fail(DSV4_ERR_SHAPE, "%s: T * splits = %lld too large", fn, (long long)T * splits);
  const size_t need = dsv4::split_workspace_bytes(T, H, splits);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need)
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned and hold %zu bytes (got %zu%s)",
                fn, need, workspace_bytes, workspace ? "" : ", NULL");
  return hip_status(dsv4::launch_attention_split(q, kv_cache, num_pages,
                                                 dsv4::page_shift_of(page_size), kv_dtype,
                                                 kv_scale, indices, idx_stride, lens, sinks,
                                                 softmax_scale, out, lse, T, H, splits, workspace,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_sparse_mla_decode_split_noalloc(const void* q, const uint8_t* kv_cache, int num_pages,
                                         int page_size, int kv_dtype, float kv_scale,
                                         const int32_t* indices, int idx_stride,
                                         const int32_t* lens, const float* sinks,
                                         float softmax_scale, void* out, float* lse, int T, int H,
                                         int splits, void* stream) {
  const char* fn = "dsv4_sparse_mla_decode_split_noalloc";
  int st = check_attention(fn, q, kv_cache, num_pages, page_size, kv_dtype, kv_scale, indices,
                           idx_stride, lens, sinks, softmax_scale, out, T, H);
  if (st) return st;
  if (splits < 1 || splits > 64) return fail(DSV4_ERR_SHAPE, "%s: splits %d not in 1..64", fn, splits);
  if (T == 0) return ok();
  if (splits == 1)
    return hip_status(dsv4::launch_attention(q, kv_cache, num_pages, dsv4::page_shift_of(page_size),
                                             kv_dtype, kv_scale, indices, idx_stride, lens, sinks,
                                             softmax_scale, out, lse, T, H, false, nullptr, 0,
                                             static_cast<hipStream_t>(stream)),
                      fn);
  if ((int64_t)T * splits >= ((int64_t)1 << 31) / 8)
    return fail(DSV4_ERR_SHAPE, "%s: T * splits = %lld too large", fn, (long long)T * splits);
  const size_t need = dsv4::split_workspace_bytes(T, H, splits);
  if (need > dsv4::kNoallocScratchBytes)
    return fail(DSV4_ERR_WORKSPACE,
                "%s: T = %d, H = %d, splits = %d need %zu bytes of workspace, more than the %zu "
                "bytes of the library's static scratch array (use dsv4_sparse_mla_decode_split "
                "with a workspace of your own)",
                fn, T, H, splits, need, dsv4::kNoallocScratchBytes);
  void* ws = nullptr;
  hipError_t e = dsv4::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(DSV4_ERR_HIP, "%s: the address of the static scratch array: %s", fn,
                hipGetErrorString(e));
  return hip_status(dsv4::launch_attention_split(q, kv_cache, num_pages,
                                                 dsv4::page_shift_of(page_size), kv_dtype,
                                                 kv_scale, indices, idx_stride, lens, sinks,
                                                 softmax_scale, out, lse, T, H, splits, ws,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_sparse_mla_decode_topk(const void* q, const uint8_t* kv_cache, int num_pages, int page_size,
                                int kv_dtype, float kv_scale, const int32_t* topk, int topk_stride, int topk_width,
                                const int32_t* topk_lens, const int32_t* query_start_loc,
                                const int32_t* seq_lens, const int32_t* block_table,
                                int block_table_stride, int B, int top_k, int window,
                                const float* sinks, float softmax_scale, void* out, float* lse,
                                int T, int H, void* stream) {
  const char* fn = "dsv4_sparse_mla_decode_topk";
  if (T < 0 || B < 0 || top_k < 0 || window < 0 || topk_width < 0 || topk_stride < topk_width ||
      block_table_stride < 0)
    return fail(DSV4_ERR_SHAPE, "%s: negative size or topk_stride < topk_width", fn);
  if (H != 16 && H != 32 && H != 64 && H != 128)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: H = %d not in {16, 32, 64, 128}", fn, H);
  int st = check_page(fn, page_size, num_pages);
  if (!st) st = check_kv(fn, kv_dtype, kv_scale);
  if (st) return st;
  if (top_k > topk_width) return fail(DSV4_ERR_SHAPE, "%s: top_k %d > topk_width %d", fn, top_k, topk_width);
  if ((int64_t)top_k + window > 4096)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: top_k + window = %lld > 4096", fn, (long long)top_k + window);
  if (!(softmax_scale == softmax_scale)) return fail(DSV4_ERR_SHAPE, "%s: softmax_scale is NaN", fn);
  if (T == 0) return ok();
  if (!q || !out || !query_start_loc || !seq_lens || (!topk && topk_width > 0) ||
      (!block_table && block_table_stride > 0) || (!kv_cache && num_pages > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || (kv_cache && !aligned(kv_cache, 16)))
    return fail(DSV4_ERR_ALIGN, "%s: q, out and kv_cache must be 16-byte aligned", fn);
  if ((topk && !aligned(topk, 4)) || !aligned(query_start_loc, 4) || !aligned(seq_lens, 4))
    return fail(DSV4_ERR_ALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  return hip_status(dsv4::launch_attention_topk(q, kv_cache, num_pages, dsv4::page_shift_of(page_size),
                                                kv_dtype, kv_scale, topk, topk_stride, topk_width, topk_lens,
                                                query_start_loc, seq_lens, block_table,
                                                block_table_stride, B, top_k, window, sinks,
                                                softmax_scale, out, lse, T, H,
                                                static_cast<hipStream_t>(stream)),
                    fn);
}

constexpr int kMaxStepQueriesPerRequest = 64;

static int decode_step_checked(const char* fn, void* q, const void* kv, const int64_t* positions,
                               const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                               const void* q_norm_weight, float eps, uint8_t* kv_cache,
                               int num_pages, int page_size, int kv_dtype, float kv_scale,
                               const int32_t* topk, int topk_stride, int topk_width,
                               const int32_t* topk_lens, const int32_t* query_start_loc,
                               const int32_t* seq_lens, const int32_t* block_table,
                               int block_table_stride, int B, int top_k, int window,
                               const float* sinks, float softmax_scale, void* out, float* lse,
                               int T, int H, int splits, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (T < 0 || B < 0 || top_k < 0 || window < 0 || topk_width < 0 || topk_stride < topk_width ||
      block_table_stride < 0 || max_pos < 0)
    return fail(DSV4_ERR_SHAPE, "%s: negative size or topk_stride < topk_width", fn);
  if (H != 16 && H != 32 && H != 64 && H != 128)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: H = %d not in {16, 32, 64, 128}", fn, H);
  int st = check_page(fn, page_size, num_pages);
  if (!st) st = check_kv(fn, kv_dtype, kv_scale);
  if (st) return st;
  if (top_k > topk_width) return fail(DSV4_ERR_SHAPE, "%s: top_k %d > topk_width %d", fn, top_k, topk_width);
  if ((int64_t)top_k + window > 4096)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: top_k + window = %lld > 4096", fn, (long long)top_k + window);
  if (splits < 1 || splits > 64)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: splits %d not in 1..64", fn, splits);
  // every workgroup of a token re-quantises its request's new rows up to its own, so the
  // insert work grows with the square of a request's query count: decode batches only
  if ((int64_t)T > (int64_t)kMaxStepQueriesPerRequest * (B > 0 ? B : 1))
    return fail(DSV4_ERR_UNSUPPORTED,
                "%s: T = %d exceeds %d query tokens per request on average (B = %d); use "
                "dsv4_kv_insert + dsv4_sparse_mla_decode_topk for prefill-sized requests",
                fn, T, kMaxStepQueriesPerRequest, B);
  if (!(softmax_scale == softmax_scale)) return fail(DSV4_ERR_SHAPE, "%s: softmax_scale is NaN", fn);
  if (!(eps >= 0.f)) return fail(DSV4_ERR_SHAPE, "%s: eps must be >= 0", fn);
  if (T == 0) return ok();
  if (!q || !kv || !positions || !slot_mapping || !cos_sin || !q_norm_weight || !out ||
      !query_start_loc || !seq_lens || (!topk && topk_width > 0) ||
      (!block_table && block_table_stride > 0) || (!kv_cache && num_pages > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(q_norm_weight, 16) || !aligned(cos_sin, 16) ||
      !aligned(out, 16) || (kv_cache && !aligned(kv_cache, 16)))
    return fail(DSV4_ERR_ALIGN, "%s: q, kv, q_norm_weight, cos_sin, out and kv_cache must be 16-byte aligned", fn);
  if (!aligned(positions, 8) || !aligned(slot_mapping, 8) || (topk && !aligned(topk, 4)) ||
      !aligned(query_start_loc, 4) || !aligned(seq_lens, 4))
    return fail(DSV4_ERR_ALIGN, "%s: positions, slot_mapping 8-byte aligned; int32 arrays 4-byte", fn);
  if (splits > 1) {
    const size_t need = dsv4::split_workspace_bytes(T, H, splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
      return fail(DSV4_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) needed, got %zu",
                  fn, need, workspace ? workspace_bytes : (size_t)0);
  }
  return hip_status(dsv4::launch_attention_step(q, kv, positions, slot_mapping, cos_sin, max_pos,
                                                q_norm_weight, eps, kv_cache, num_pages,
                                                dsv4::page_shift_of(page_size), kv_dtype,
                                                kv_scale, topk, topk_stride,
                                                topk_width, topk_lens, query_start_loc, seq_lens,
                                                block_table, block_table_stride, B, top_k, window,
                                                sinks, softmax_scale, out, lse, T, H, splits,
                                                workspace, static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_sparse_mla_decode_step(void* q, const void* kv, const int64_t* positions,
                                const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                                const void* q_norm_weight, float eps, uint8_t* kv_cache,
                                int num_pages, int page_size, int kv_dtype, float kv_scale,
                                const int32_t* topk, int topk_stride, int topk_width,
                                const int32_t* topk_lens, const int32_t* query_start_loc,
                                const int32_t* seq_lens, const int32_t* block_table,
                                int block_table_stride, int B, int top_k, int window,
                                const float* sinks, float softmax_scale, void* out, float* lse,
                                int T, int H, void* stream) {
  return decode_step_checked("dsv4_sparse_mla_decode_step", q, kv, positions, slot_mapping,
                             cos_sin, max_pos, q_norm_weight, eps, kv_cache, num_pages, page_size,
                             kv_dtype, kv_scale, topk, topk_stride, topk_width, topk_lens, query_start_loc, seq_lens,
                             block_table, block_table_stride, B, top_k, window, sinks,
                             softmax_scale, out, lse, T, H, 1, nullptr, 0, stream);
}

int dsv4_sparse_mla_decode_step_split(
    void* q, const void* kv, const int64_t* positions, const int64_t* slot_mapping,
    const float* cos_sin, int max_pos, const void* q_norm_weight, float eps, uint8_t* kv_cache,
    int num_pages, int page_size, int kv_dtype, float kv_scale, const int32_t* topk,
    int topk_stride, int topk_width, const int32_t* topk_lens, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int block_table_stride, int B, int top_k,
    int window, const float* sinks, float softmax_scale, void* out, float* lse, int T, int H,
    int splits, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_step_checked("dsv4_sparse_mla_decode_step_split", q, kv, positions, slot_mapping,
                             cos_sin, max_pos, q_norm_weight, eps, kv_cache, num_pages, page_size,
                             kv_dtype, kv_scale, topk, topk_stride, topk_width, topk_lens, query_start_loc, seq_lens,
                             block_table, block_table_stride, B, top_k, window, sinks,
                             softmax_scale, out, lse, T, H, splits, workspace, workspace_bytes,
                             stream);
}

int dsv4_sparse_mla_prefill(const void* q, const uint8_t* kv_cache, int num_pages, int page_size,
                            int kv_dtype, float kv_scale, const int32_t* indices, int idx_stride,
                            const int32_t* lens, const float* sinks, float softmax_scale, void* out,
                            float* lse, int T, int H, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return attention_checked("dsv4_sparse_mla_prefill", true, q, kv_cache, num_pages, page_size,
                           kv_dtype, kv_scale, indices, idx_stride, lens, sinks, softmax_scale, out, lse, T, H,
                           workspace, workspace_bytes, stream);
}

int dsv4_gather_dequant(const uint8_t* kv_cache, int num_pages, int page_size, int kv_dtype,
                        float kv_scale, const int32_t* slots, int n, void* out, void* stream) {
  const char* fn = "dsv4_gather_dequant";
  if (n < 0) return fail(DSV4_ERR_SHAPE, "%s: n = %d < 0", fn, n);
  int st = check_page(fn, page_size, num_pages);
  if (!st) st = check_kv(fn, kv_dtype, kv_scale);
  if (st) return st;
  if (n == 0) return ok();
  if (!slots || !out || (!kv_cache && num_pages > 0))
    return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(out, 16) || (kv_cache && !aligned(kv_cache, 16)) || !aligned(slots, 4))
    return fail(DSV4_ERR_ALIGN, "%s: out and kv_cache must be 16-byte aligned, slots 4-byte", fn);
  return hip_status(dsv4::launch_gather(kv_cache, num_pages, dsv4::page_shift_of(page_size),
                                        kv_dtype, kv_scale, slots, n, out,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_peak_mfma(int shape, int workgroups, int iters, float* sink, double* flops,
                   void* stream) {
  const char* fn = "dsv4_peak_mfma";
  if (shape != 0 && shape != 1)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: shape %d not supported (0 32x32x16, 1 16x16x32)", fn, shape);
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20))
    return fail(DSV4_ERR_SHAPE, "%s: workgroups %d not in [1, 65536] or iters %d not in [1, 2^20]",
                fn, workgroups, iters);
  if (!sink || !flops) return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(sink, 4)) return fail(DSV4_ERR_ALIGN, "%s: sink must be 4-byte aligned", fn);
  return hip_status(dsv4::launch_peak_mfma(shape, workgroups, iters, sink, flops,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

int dsv4_peak_stream(const void* src, void* dst, size_t bytes, uint32_t* sink, int workgroups,
                     void* stream) {
  const char* fn = "dsv4_peak_stream";
  if (bytes % 16 != 0) return fail(DSV4_ERR_SHAPE, "%s: bytes %zu not a multiple of 16", fn, bytes);
  if (workgroups < 1 || workgroups > 65536)
    return fail(DSV4_ERR_SHAPE, "%s: workgroups %d not in [1, 65536]", fn, workgroups);
  if (!sink || (!src && bytes > 0)) return fail(DSV4_ERR_NULL, "%s: a required pointer is NULL", fn);
  if ((src && !aligned(src, 16)) || (dst && !aligned(dst, 16)) || !aligned(sink, 4))
    return fail(DSV4_ERR_ALIGN, "%s: src and dst must be 16-byte aligned, sink 4-byte", fn);
  return hip_status(dsv4::launch_peak_stream(src, dst, bytes, sink, workgroups,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
