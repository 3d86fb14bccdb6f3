// Fused insert: per-head q RMSNorm + GPT-J RoPE in place, and FP8 E4M3 / UE8M0
// quantisation of the new latent rows into the paged cache.  Follows PR #42953
// (Implementation breakdown item 4: fused q per-head RMSNorm, GPT-J RoPE and FP8 UE8M0
// KV insert; Key source excerpts: called with q, kv, kv_cache, slot_mapping, positions)
// and the "RMSNorm+Rope+Quant" fused kernel of PR #40860 (Implementation breakdown 2).
//
// The q part is ~99% of the bytes (q read + written once), so it is an HBM-streaming
// kernel: a wave owns 8 head rows, each row spread over 8 lanes that read 16 B chunks
// c, c+8, ..., so every load/store instruction moves 8 full 128 B lines.  The row
// reduction is 3 xor-shuffles inside the 8 lanes.  fp32 arithmetic, one bf16 rounding.
//
// The kv part is one wave per token: lane l owns nope dims 8l..8l+7 (block l/8); the
// block amax is exact, the exponent is taken from the fp32 bit fields, the scaling by
// 2^-e is exact and the E4M3 rounding is gfx950's RNE conversion -> bit-exact bytes.
// The bf16 and per-tensor fp8 caches (PR #43477 Key source excerpts: the SM100
// backend's kv-cache dtypes) take the same lanes: one record of the 576 values per slot.
#include "device.hpp"
#include "insert_rows.hpp"
#include "launch.hpp"

namespace dsv4 {

template <int KV>
__device__ __forceinline__ void kv_quant_insert(
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ positions,
    const int64_t* __restrict__ slot_mapping, const float* __restrict__ cos_sin, int max_pos,
    uint8_t* __restrict__ cache, int64_t num_slots, int ps, float kv_scale, int T, int block) {
  const int lane = threadIdx.x & 63;
  const int64_t t = ((int64_t)block * blockDim.x + threadIdx.x) >> 6;
  if (t >= T) return;
  // the row is requested beside its position and slot
  const KvLane v = kv_lane_load(kv + t * kLatent, lane);
  const int64_t p = positions[t];
  const int64_t slot = slot_mapping[t];
  if (p < 0 || p >= max_pos || slot < 0 || slot >= num_slots) return;
  kv_store_row<KV>(v, rope_cs_load(cos_sin + p * kRope, lane), cache, slot, ps, kv_scale, lane);
}

// One launch: blocks [0, qblocks) stream the q rows, the remaining blocks quantise the
// new latent rows (4 tokens per block) into a cache of dtype KV.
template <int KV>
__global__ void __launch_bounds__(256) insert_kernel(
    uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int64_t* __restrict__ positions,
    const int64_t* __restrict__ slot_mapping, const float* __restrict__ cos_sin, int max_pos,
    const uint16_t* __restrict__ weight, float eps, uint8_t* __restrict__ cache, int64_t num_slots,
    int ps, float kv_scale, int T, int H, int qblocks) {
  if ((int)blockIdx.x < qblocks)
    q_norm_rope_rows(q, positions, cos_sin, max_pos, weight, eps, (int64_t)T * H, H,
                     (int)blockIdx.x, qblocks);
  else
    kv_quant_insert<KV>(kv, positions, slot_mapping, cos_sin, max_pos, cache, num_slots, ps,
                        kv_scale, T, (int)blockIdx.x - qblocks);
}

hipError_t launch_insert(void* q, const void* kv, const int64_t* positions,
                         const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                         const void* weight, float eps, uint8_t* cache, int num_pages,
                         int page_shift, int kv_dtype, float kv_scale, int T, int H,
                         hipStream_t stream) {
  // no valid position: every token is left untouched (and the cos/sin table may be empty)
  if (T == 0 || max_pos <= 0) return hipSuccess;
  const int64_t rows = (int64_t)T * H;
  const int64_t groups = (rows + 31) / 32;  // 32 q rows per 256-thread block per pass
  const int qblocks = rows > 0 ? (int)(groups < 8192 ? groups : 8192) : 0;
  const int kvblocks = (T + 3) / 4;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(qblocks + kvblocks), dim3(256), 0, stream,
                       static_cast<uint16_t*>(q), static_cast<const uint16_t*>(kv), positions,
                       slot_mapping, cos_sin, max_pos, static_cast<const uint16_t*>(weight), eps,
                       cache, (int64_t)num_pages << page_shift, page_shift, kv_scale, T, H,
                       qblocks);
    return hipGetLastError();
  };
  switch (kv_dtype) {
    case kKvFp8Ds: return go(insert_kernel<kKvFp8Ds>);
    case kKvBf16: return go(insert_kernel<kKvBf16>);
    case kKvFp8E4m3: return go(insert_kernel<kKvFp8E4m3>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsv4
