// Index combining: top-k + sliding window -> one deduplicated, physical, -1-padded row
// per query token.  Follows the ROCm combine step of PR #43385 (Key source excerpts,
// rocm.py combine kernel: per-token top-k part, then the window part, then the length),
// with the logical -> physical mapping of PR #43477 (forward_mqa excerpt) fused in and
// the per-row topk_lens of PR #42953 (Implementation breakdown item 6).
//
// Schedule: workgroup (b, y) owns tokens y, y+Y, ... of request b; its 256 threads
// sweep one row at a time, so every load of the top-k row and every store of the
// combined row is a coalesced 1 KiB wave access.  Integer only: bit-exact by design.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

constexpr int kColsPerThread = 9;  // 2304 columns per pass covers the 2176-wide rows

__global__ void __launch_bounds__(256) combine_kernel(
    const int32_t* __restrict__ topk, int topk_stride, int topk_width,
    const int32_t* __restrict__ topk_lens, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table, int bt_stride,
    int T, int top_k, int window, int ps, int32_t* __restrict__ combined, int combined_stride,
    int32_t* __restrict__ combined_lens) {
  const int b = blockIdx.x;
  const int base = qsl[0];
  const int q0 = qsl[b] - base;
  const int qlen = qsl[b + 1] - qsl[b];
  const int seq_len = seq_lens[b];
  const int32_t* bt_row = block_table + (int64_t)b * bt_stride;
  for (int i = blockIdx.y; i < qlen; i += gridDim.y) {
    const int64_t t = (int64_t)q0 + i;
    if (t < 0 || t >= T) continue;
    const int64_t pos = (int64_t)seq_len - qlen + i;
    int64_t tk = min(pos + 1, (int64_t)top_k);
    if (topk_lens) tk = min(tk, (int64_t)topk_lens[t]);
    tk = max(tk, (int64_t)0);
    const int64_t sw = max(min(pos + 1, (int64_t)window), (int64_t)0);
    const int64_t lo = pos - sw + 1;
    const int32_t* trow = topk + t * topk_stride;
    int32_t* crow = combined + t * combined_stride;
    // columns j = threadIdx.x + 256k: all top-k loads, then all block-table loads, are
    // issued before any is consumed (one memory round trip each per row, not per column).
    // The loads are unconditional at clamped in-bounds addresses (only uniform conditions
    // skip one) and their values selected afterwards: a load under a per-lane condition
    // is waited for on the spot.
    const int kmax = (int)min(tk, (int64_t)topk_width);  // top-k columns that are read
    const int32_t* tsrc = kmax > 0 ? trow : qsl;          // any readable word when none is
    for (int jb = 0; jb < combined_stride; jb += 256 * kColsPerThread) {
      int32_t tv[kColsPerThread];
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k)  // every load first, then their use
        tv[k] = tsrc[kmax > 0 ? min(jb + (int)threadIdx.x + 256 * k, kmax - 1) : 0];
      int64_t x[kColsPerThread];
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int j = jb + threadIdx.x + 256 * k;
        const int64_t from_topk = j < topk_width ? (int64_t)tv[k] : -1;
        const int64_t from_window = j < tk + sw ? lo + (j - tk) : -1;
        const int64_t xx = j < tk ? from_topk : from_window;
        // top-k entries that are invalid, beyond pos, or inside the window -> -1
        x[k] = (j < tk && !(xx >= 0 && xx < lo)) ? -1 : xx;
      }
      int32_t pg[kColsPerThread];
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int64_t lp = x[k] >> ps;
        pg[k] = (jb + 256 * k < tk + sw && bt_stride > 0)
                    ? bt_row[lp < 0 ? 0 : (lp < bt_stride ? lp : bt_stride - 1)] : -1;
      }
      int32_t v[kColsPerThread];
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const bool ok = x[k] >= 0 && (x[k] >> ps) < bt_stride && pg[k] >= 0;
        v[k] = ok ? (int32_t)(((int64_t)pg[k] << ps) + (x[k] & ((1 << ps) - 1))) : -1;
      }
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int j = jb + threadIdx.x + 256 * k;
        if (j < combined_stride) crow[j] = v[k];
      }
    }
    if (threadIdx.x == 0) combined_lens[t] = (int32_t)(tk + sw);
  }
}

// Compressed-cache form (PR #43385, the same combine kernel with COMPRESS_RATIO, M, N
// and gather_lens): the indices address a per-request workspace of M rows, the first N
// holding compressed entries, the next the last gather_len raw tokens of the sequence.
// Per token at position pos: tk = min((pos+1) / ratio, top_k[, topk_lens[t]]) top-k
// entries e -> M*b + e (0 <= e < N, else -1), then sw = min(pos+1, window) window rows
// M*b + N + (pos-sw+1+r - gather_start), -1 when outside the gathered tokens or past the
// request's M rows; no dedup (two index spaces).  Integer only: bit-exact by design.
__global__ void __launch_bounds__(256) combine_compressed_kernel(
    const int32_t* __restrict__ topk, int topk_stride, int topk_width,
    const int32_t* __restrict__ topk_lens, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ gather_lens, int T,
    int top_k, int ratio, int window, int M, int N, int32_t* __restrict__ combined,
    int combined_stride, int32_t* __restrict__ combined_lens) {
  const int b = blockIdx.x;
  const int base = qsl[0];
  const int q0 = qsl[b] - base;
  const int qlen = qsl[b + 1] - qsl[b];
  const int seq_len = seq_lens[b];
  const int gl = gather_lens[b];
  const int64_t gather_start = (int64_t)seq_len - gl;
  const int64_t row0 = (int64_t)M * b;
  for (int i = blockIdx.y; i < qlen; i += gridDim.y) {
    const int64_t t = (int64_t)q0 + i;
    if (t < 0 || t >= T) continue;
    const int64_t pos = (int64_t)seq_len - qlen + i;
    int64_t tk = pos + 1 >= 0 ? (pos + 1) / ratio : 0;
    tk = min(tk, (int64_t)top_k);
    if (topk_lens) tk = min(tk, (int64_t)topk_lens[t]);
    tk = max(tk, (int64_t)0);
    const int64_t sw = max(min(pos + 1, (int64_t)window), (int64_t)0);
    const int64_t k0 = pos - sw + 1 - gather_start;  // gathered-token row of the first window entry
    const int kmax = (int)min(tk, (int64_t)topk_width);
    const int32_t* trow = topk + t * topk_stride;
    const int32_t* tsrc = kmax > 0 ? trow : qsl;  // any readable word when no column is
    int32_t* crow = combined + t * combined_stride;
    for (int jb = 0; jb < combined_stride; jb += 256 * kColsPerThread) {
      int32_t v[kColsPerThread];
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int j = jb + threadIdx.x + 256 * k;
        // unconditional load at a clamped column (see combine_kernel), selected after
        const int32_t tv = tsrc[kmax > 0 ? min(j, kmax - 1) : 0];
        const int64_t e = (j < tk && j < topk_width) ? (int64_t)tv : -1;
        v[k] = (e >= 0 && e < N) ? (int32_t)(row0 + e) : -1;
      }
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int j = jb + threadIdx.x + 256 * k;
        if (j >= tk && j < tk + sw) {
          const int64_t kk = k0 + (j - tk);
          v[k] = (kk >= 0 && kk < gl && N + kk < M) ? (int32_t)(row0 + N + kk) : -1;
        }
        if (j < combined_stride) crow[j] = v[k];
      }
    }
    if (threadIdx.x == 0) combined_lens[t] = (int32_t)(tk + sw);
  }
}

hipError_t launch_combine_compressed(const int32_t* topk, int topk_stride, int topk_width,
                                     const int32_t* topk_lens, const int32_t* qsl,
                                     const int32_t* seq_lens, const int32_t* gather_lens, int B,
                                     int T, int top_k, int ratio, int window, int M, int N,
                                     int32_t* combined, int combined_stride,
                                     int32_t* combined_lens, hipStream_t stream) {
  if (B == 0 || T == 0) return hipSuccess;
  int per_req = (T + B - 1) / B;
  int Y = per_req < 1 ? 1 : (per_req > 2048 ? 2048 : per_req);
  hipLaunchKernelGGL(combine_compressed_kernel, dim3(B, Y), dim3(256), 0, stream, topk,
                     topk_stride, topk_width, topk_lens, qsl, seq_lens, gather_lens, T, top_k,
                     ratio, window, M, N, combined, combined_stride, combined_lens);
  return hipGetLastError();
}

hipError_t launch_combine(const int32_t* topk, int topk_stride, int topk_width,
                          const int32_t* topk_lens, const int32_t* qsl, const int32_t* seq_lens,
                          const int32_t* block_table, int bt_stride, int B, int T, int top_k,
                          int window, int page_shift, int32_t* combined, int combined_stride,
                          int32_t* combined_lens, hipStream_t stream) {
  if (B == 0 || T == 0) return hipSuccess;
  // tokens per request are device data; size the second grid axis from the average
  int per_req = (T + B - 1) / B;
  int Y = per_req < 1 ? 1 : (per_req > 2048 ? 2048 : per_req);
  hipLaunchKernelGGL(combine_kernel, dim3(B, Y), dim3(256), 0, stream, topk, topk_stride,
                     topk_width, topk_lens, qsl, seq_lens, block_table, bt_stride, T, top_k,
                     window, page_shift, combined, combined_stride, combined_lens);
  return hipGetLastError();
}

}  // namespace dsv4
