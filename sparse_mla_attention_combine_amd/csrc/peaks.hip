// Throughput probes for the measured peaks that the roofline is also reported against
// (not a step of the method): the matrix cores on back-to-back dense bf16 MFMAs of the
// two shapes the attention kernels use, and HBM on a streaming read or copy.
#include "device.hpp"
#include "peaks.hpp"

namespace dsv4 {

typedef float f32x16p __attribute__((ext_vector_type(16)));

// Each wave keeps kChains independent accumulators, so an MFMA never waits for the
// previous one's result; every lane holds the same operands, a_i = (i + 1) / 8 and
// b_i = 1 / 8, so each accumulator grows by an exactly representable constant per step
// (1.125 per element for 32x32x16, 2.25 for 16x16x32) whatever the lane layout.
// Accumulator k starts at k (equal starting values would let the compiler treat the
// chains as one value).  The lane's accumulators are summed into sink so that no MFMA
// can be dropped.
constexpr int kChains = 8;

template <int SHAPE>  // 0: v_mfma_f32_32x32x16_bf16, 1: v_mfma_f32_16x16x32_bf16
__global__ void __launch_bounds__(256) peak_mfma_kernel(float* __restrict__ sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((float)(i + 1) * 0.125f);
    b[i] = (__bf16)0.125f;
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x16p c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) c[k][j] = (float)k;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < kChains; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += c[k][j];
  } else {
    // The eight 16x16x32 MFMAs of an iteration are written as one asm statement with each
    // accumulator tied to its own AGPR tuple: with the builtin, the register allocator
    // rotates the 4-register tuples through copies every iteration, which measures the
    // copies rather than the matrix cores.  Consecutive MFMAs are independent; each tuple
    // is written again only after the seven others (accumulation forwarding needs no
    // wait), and the wait states before the results are read are inserted explicitly.
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0 + 1.f, c2 = c0 + 2.f, c3 = c0 + 3.f, c4 = c0 + 4.f,
          c5 = c0 + 5.f, c6 = c0 + 6.f, c7 = c0 + 7.f;
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");  // the tuples' initial writes land
    for (int it = 0; it < iters; ++it)
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
          "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
          "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
          "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
          "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
          : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
          : "v"(a), "v"(b));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    s = (t[0] + t[1]) + (t[2] + t[3]);
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride over 16-byte units with non-temporal loads (and stores): read-only keeps
// eight units in flight per lane per round (dst == nullptr: the lane's xor of everything
// it read goes to sink), the copy four.  Measured on this GPU, those are the fastest of
// 4 / 8 / 16 units, plain or non-temporal, at 1k-16k workgroups.
template <int U>
__device__ __forceinline__ void stream_round(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                             int64_t i, int64_t stride, uint32_t& acc) {
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (dst)
      __builtin_nontemporal_store(v[u], dst + i + u * stride);
    else
      acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
}

__global__ void __launch_bounds__(256) peak_stream_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  if (dst) {
    for (; i + 3 * stride < n16; i += 4 * stride) stream_round<4>(src, dst, i, stride, acc);
  } else {
    for (; i + 7 * stride < n16; i += 8 * stride) stream_round<8>(src, nullptr, i, stride, acc);
  }
  for (; i < n16; i += stride) stream_round<1>(src, dst, i, stride, acc);
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_peak_mfma(int shape, int workgroups, int iters, float* sink, double* flops,
                            hipStream_t stream) {
  const double per = shape == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 16 * 16 * 32;
  *flops = per * kChains * (double)iters * 4.0 * workgroups;
  if (shape == 0)
    hipLaunchKernelGGL(peak_mfma_kernel<0>, dim3(workgroups), dim3(256), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL(peak_mfma_kernel<1>, dim3(workgroups), dim3(256), 0, stream, sink, iters);
  return hipGetLastError();
}

hipError_t launch_peak_stream(const void* src, void* dst, size_t bytes, uint32_t* sink,
                              int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(peak_stream_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace dsv4
