// Gather + dequantise cache slots into bf16 rows, the separately testable form of the
// step the attention kernels fuse.  Follows PR #42953 (Key source excerpts,
// _dequant_gather_slots_kernel): a negative slot gives a zero row; otherwise the slot
// is split into page and row, the E4M3 codes are decoded and multiplied by
// 2^(byte - 127), rounded to bf16, and the bf16 RoPE part is copied.  One wave per
// slot: lane l turns nope bytes 8l..8l+7 into one 16 B store; lanes 0..7 copy the rope.
// The other cache dtypes (PR #43477 Key source excerpts: the SM100 backend's "bfloat16"
// and "fp8" caches; one record of the 576 values per slot): bf16 records are copied;
// E4M3 records with a per-tensor scale s give each value code * s rounded once to bf16.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

// bf16 (round to nearest even) of the exact product c * s for an E4M3 value c and an
// fp32 s whose products stay in fp32's normal range: p = fl(c * s) and e = fma(c, s, -p)
// satisfy p + e = c * s exactly.  p rounds to the same bf16 as c * s unless p lies
// exactly halfway between two bf16 values; then e's sign relative to p decides.
__device__ __forceinline__ uint32_t bf16_of_product(float c, float s) {
  const float p = c * s;
  const float e = __builtin_fmaf(c, s, -p);
  const uint32_t b = __float_as_uint(p);
  if ((b & 0xFFFF) == 0x8000 && e != 0.f) return (b >> 16) + (((e > 0.f) == (p > 0.f)) ? 1 : 0);
  return f32_to_bf16_bits(p);
}

// 8 E4M3 codes (memory order) -> 8 bf16 values code * s (the unscaled conversion is exact).
__device__ __forceinline__ uint4 fp8_row8(uint2 codes, float s) {
  bf16x2 v[4];
  dequant4(codes.x, 1.0f, v[0], v[1]);
  dequant4(codes.y, 1.0f, v[2], v[3]);
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = bf16_of_product((float)v[k][0], s) | (bf16_of_product((float)v[k][1], s) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int KV>
__global__ void __launch_bounds__(256) gather_dequant_kernel(const uint8_t* __restrict__ cache,
                                                             int64_t num_slots, int ps,
                                                             float kv_scale,
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
  if constexpr (KV == kKvBf16) {
    const uint8_t* rec = cache + slot * kv_record_bytes_of(KV);
    *reinterpret_cast<uint4*>(row + 8 * lane) = *reinterpret_cast<const uint4*>(rec + 16 * lane);
    if (lane < 8)
      *reinterpret_cast<uint4*>(row + kNope + 8 * lane) =
          *reinterpret_cast<const uint4*>(rec + 2 * kNope + 16 * lane);
    return;
  } else if constexpr (KV == kKvFp8E4m3) {
    const uint8_t* rec = cache + slot * kv_record_bytes_of(KV);
    *reinterpret_cast<uint4*>(row + 8 * lane) =
        fp8_row8(*reinterpret_cast<const uint2*>(rec + 8 * lane), kv_scale);
    if (lane < 8)
      *reinterpret_cast<uint4*>(row + kNope + 8 * lane) =
          fp8_row8(*reinterpret_cast<const uint2*>(rec + kNope + 8 * lane), kv_scale);
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

hipError_t launch_gather(const uint8_t* cache, int num_pages, int page_shift, int kv_dtype,
                         float kv_scale, const int32_t* slots, int n, void* out,
                         hipStream_t stream) {
  if (n == 0) return hipSuccess;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((n + 3) / 4), dim3(256), 0, stream, cache,
                       (int64_t)num_pages << page_shift, page_shift, kv_scale, slots, n,
                       static_cast<uint16_t*>(out));
    return hipGetLastError();
  };
  switch (kv_dtype) {
    case kKvFp8Ds: return go(gather_dequant_kernel<kKvFp8Ds>);
    case kKvBf16: return go(gather_dequant_kernel<kKvBf16>);
    case kKvFp8E4m3: return go(gather_dequant_kernel<kKvFp8E4m3>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsv4
