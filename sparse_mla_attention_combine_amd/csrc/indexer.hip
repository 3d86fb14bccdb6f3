// The indexer's top-k selection, the step before index combining (PR #40860: the MLA
// layer integrates an Indexer whose top-k picks feed the sparse backend; PR #43385: the
// picks are compressed-entry ids below (pos+1) / COMPRESS_RATIO).  Per token at
// position pos the candidates are ids 0..n-1, n = min((pos+1) / ratio, logits_stride);
// the result is the min(n, top_k) ids with the largest logits, ties to the smaller id
// (a NaN logit counts as -inf), listed in ascending id order, -1 after them.
//
// One workgroup (4 waves) per token.  Logits map to order-preserving 32-bit keys; a
// radix select (four 8-bit digits, most significant first, histograms in LDS) finds the
// k-th largest key K and how many keys equal to K are taken (m); one ordered pass then
// emits every id with key > K and the first m ids with key == K.  Each thread owns 8
// consecutive candidates per pass, so a block-wide scan of its counts (packed into one
// 32-bit value) gives every thread its output position.  Integer decisions on fp32
// keys only: bit-exact with the oracle's fp32 comparisons.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

constexpr int kSelThreads = 256;
constexpr int kSelItems = 8;

// Larger key <=> larger logit; -0 and +0 share a key (they compare equal), NaN takes the
// key of -inf.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (v != v) u = 0xFF800000u;
  if (v == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over the 256 threads of the block (4 waves); `wsum` holds 4 ints.
__device__ __forceinline__ int block_inclusive_scan(int x, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) add += i < w ? wsum[i] : 0;
  __syncthreads();  // wsum may be reused by the next scan
  return x + add;
}

__global__ void __launch_bounds__(kSelThreads) indexer_topk_kernel(
    const float* __restrict__ logits, int logits_stride, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ seq_lens, int T, int ratio, int top_k, int32_t* __restrict__ topk,
    int topk_stride, int32_t* __restrict__ topk_lens) {
  __shared__ uint32_t hist[256];
  __shared__ int wsum[4];
  __shared__ uint32_t sh_digit, sh_above;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int base = qsl[0];
  const int q0 = qsl[b] - base;
  const int qlen = qsl[b + 1] - qsl[b];
  const int seq_len = seq_lens[b];
  for (int i = blockIdx.y; i < qlen; i += gridDim.y) {
    const int64_t t = (int64_t)q0 + i;
    if (t < 0 || t >= T) continue;
    const int64_t pos = (int64_t)seq_len - qlen + i;
    int64_t n64 = pos + 1 > 0 ? (pos + 1) / ratio : 0;
    const int n = (int)min(n64, (int64_t)logits_stride);
    const int k = min(n, top_k);
    const float* row = logits + t * (int64_t)logits_stride;
    int32_t* out = topk + t * (int64_t)topk_stride;
    if (k == n) {
      for (int j = tid; j < n; j += kSelThreads) out[j] = j;
    } else if (k > 0) {
      // radix select of the k-th largest key
      uint32_t prefix = 0, mask = 0;
      int remaining = k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kSelThreads) {
          const uint32_t key = order_key(row[j]);
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // thread d holds the count of digit 255-d; the inclusive scan gives, for digit
        // 255-d, the number of matching keys with that digit or a larger one
        const int c = (int)hist[255 - tid];
        const int incl = block_inclusive_scan(c, wsum);
        const int excl = incl - c;  // keys with a larger digit
        if (excl < remaining && incl >= remaining) {
          sh_digit = 255u - (uint32_t)tid;
          sh_above = (uint32_t)excl;
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        remaining -= (int)sh_above;
        __syncthreads();  // sh_digit / sh_above / hist are rewritten next pass
      }
      const uint32_t K = prefix;
      const int m = remaining;  // keys equal to K that are taken, the smallest ids first
      int gt_run = 0, eq_run = 0;
      for (int c0 = 0; c0 < n; c0 += kSelThreads * kSelItems) {
        const int first = c0 + tid * kSelItems;
        uint32_t key[kSelItems];
        int cgt = 0, ceq = 0;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
          key[j] = first + j < n ? order_key(row[first + j]) : 0u;
          cgt += (first + j < n && key[j] > K) ? 1 : 0;
          ceq += (first + j < n && key[j] == K) ? 1 : 0;
        }
        // counts of at most 2048 per pass: pack (gt, eq) into one scan
        const int packed = cgt | (ceq << 16);
        const int incl = block_inclusive_scan(packed, wsum);
        const int excl = incl - packed;
        const int gt_before = gt_run + (excl & 0xFFFF);
        const int eq_before = eq_run + (excl >> 16);
        int p = gt_before + min(eq_before, m);
        int eq_rank = eq_before;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
          if (first + j >= n) break;
          if (key[j] > K) {
            out[p++] = first + j;
          } else if (key[j] == K) {
            if (eq_rank < m) out[p++] = first + j;
            ++eq_rank;
          }
        }
        // block totals of this pass: the last thread's inclusive value
        if (tid == kSelThreads - 1) wsum[0] = incl;
        __syncthreads();
        const int tot = wsum[0];
        gt_run += tot & 0xFFFF;
        eq_run += tot >> 16;
        __syncthreads();
      }
    }
    for (int j = k + tid; j < topk_stride; j += kSelThreads) out[j] = -1;
    if (tid == 0) topk_lens[t] = k;
    __syncthreads();  // LDS reuse by the next token of this workgroup
  }
}

hipError_t launch_indexer_topk(const float* logits, int logits_stride, const int32_t* qsl,
                               const int32_t* seq_lens, int B, int T, int ratio, int top_k,
                               int32_t* topk, int topk_stride, int32_t* topk_lens,
                               hipStream_t stream) {
  if (B == 0 || T == 0) return hipSuccess;
  int per_req = (T + B - 1) / B;
  int Y = per_req < 1 ? 1 : (per_req > 4096 ? 4096 : per_req);
  hipLaunchKernelGGL(indexer_topk_kernel, dim3(B, Y), dim3(kSelThreads), 0, stream, logits,
                     logits_stride, qsl, seq_lens, T, ratio, top_k, topk, topk_stride, topk_lens);
  return hipGetLastError();
}

}  // namespace dsv4
