// Gather + dequantise cache slots into bf16 rows, the separately testable form of the
// step the attention kernels fuse.  Follows PR #42953 (Key source excerpts,
// _dequant_gather_slots_kernel): a negative slot gives a zero row; otherwise the slot
// is split into page and row, the E4M3 codes are decoded and multiplied by
// 2^(byte - 127), rounded to bf16, and the bf16 RoPE part is copied.  One wave per
// slot: lane l turns nope bytes 8l..8l+7 into one 16 B store; lanes 0..7 copy the rope.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

__global__ void __launch_bounds__(256) gather_dequant_kernel(const uint8_t* __restrict__ cache,
                                                             int64_t num_slots, int ps,
                                                             const int32_t* __restrict__ slots,
                                                             int n, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (i >= n) return;
  const int64_t slot = slots[i];
  uint16_t* row = out + i * kLatent;
  if (slot < 0 || slot >= num_slots) {
    *reinterpret_cast<uint4*>(row + 8 * lane) = make_uint4(0, 0, 0, 0);
    if (lane < 8) *reinterpret_cast<uint4*>(row + kNope + 8 * lane) = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint8_t* base = cache + page_base(slot >> ps, ps);
  const int off = (int)(slot & ((1 << ps) - 1));
  const uint2 codes = *reinterpret_cast<const uint2*>(base + nope_off(off) + 8 * lane);
  const float scale = e8m0_as_scale(base[scale_off(off, ps) + (lane >> 3)]);
  const bf16x8 v = dequant8(codes.x, codes.y, scale);
  *reinterpret_cast<bf16x8*>(row + 8 * lane) = v;
  if (lane < 8)
    *reinterpret_cast<uint4*>(row + kNope + 8 * lane) =
        *reinterpret_cast<const uint4*>(base + rope_off(off, ps) + 16 * lane);
}

hipError_t launch_gather(const uint8_t* cache, int num_pages, int page_shift, const int32_t* slots,
                         int n, void* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_dequant_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, cache,
                     (int64_t)num_pages << page_shift, page_shift, slots, n,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace dsv4
