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
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

__device__ __forceinline__ void q_norm_rope(
    uint16_t* __restrict__ q, const int64_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, const uint16_t* __restrict__ weight, float eps,
    int64_t rows, int H, int qblocks) {
  const int lane = threadIdx.x & 63;
  const int r8 = lane >> 3, c8 = lane & 7;
  // this lane always touches chunks c8 + 8k (k = 0..8) of a row: keep their weights
  float w[72];
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    uint4 v = *reinterpret_cast<const uint4*>(weight + 8 * (c8 + 8 * k));
    uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[8 * k + 2 * e] = bf16_bits_to_f32(u[e] & 0xFFFF);
      w[8 * k + 2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
    }
  }
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)qblocks * blockDim.x) >> 6;
  for (int64_t g = wave; g * 8 < rows; g += nwaves) {
    const int64_t row = g * 8 + r8;
    if (row >= rows) continue;
    const int64_t t = row / H;
    const int64_t p = positions[t];
    if (p < 0 || p >= max_pos) continue;  // token left untouched
    uint16_t* qr = q + row * kLatent;
    float x[72];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      uint4 v = *reinterpret_cast<const uint4*>(qr + 8 * (c8 + 8 * k));
      uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * k + 2 * e] = bf16_bits_to_f32(u[e] & 0xFFFF);
        x[8 * k + 2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 72; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 1, 8);
    ss += __shfl_xor(ss, 2, 8);
    ss += __shfl_xor(ss, 4, 8);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kLatent) + eps);
#pragma unroll
    for (int i = 0; i < 72; ++i) x[i] = x[i] * inv * w[i];
    // chunk k = 8 holds dims 512 + 8*c8 .. +7, i.e. rotary pairs 4*c8 .. 4*c8+3
    const float* cs = cos_sin + p * kRope + 4 * c8;
    const float4 cv = *reinterpret_cast<const float4*>(cs);
    const float4 sv = *reinterpret_cast<const float4*>(cs + kRope / 2);
    const float cc[4] = {cv.x, cv.y, cv.z, cv.w}, sn[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = x[64 + 2 * e], b = x[64 + 2 * e + 1];
      x[64 + 2 * e] = a * cc[e] - b * sn[e];
      x[64 + 2 * e + 1] = a * sn[e] + b * cc[e];
    }
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      uint4 v;
      v.x = pack_bf16x2(x[8 * k + 0], x[8 * k + 1]);
      v.y = pack_bf16x2(x[8 * k + 2], x[8 * k + 3]);
      v.z = pack_bf16x2(x[8 * k + 4], x[8 * k + 5]);
      v.w = pack_bf16x2(x[8 * k + 6], x[8 * k + 7]);
      *reinterpret_cast<uint4*>(qr + 8 * (c8 + 8 * k)) = v;
    }
  }
}

__device__ __forceinline__ void kv_quant_insert(
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ positions,
    const int64_t* __restrict__ slot_mapping, const float* __restrict__ cos_sin, int max_pos,
    uint8_t* __restrict__ cache, int64_t num_slots, int ps, int T, int block) {
  const int lane = threadIdx.x & 63;
  const int64_t t = ((int64_t)block * blockDim.x + threadIdx.x) >> 6;
  if (t >= T) return;
  const int64_t p = positions[t];
  const int64_t slot = slot_mapping[t];
  if (p < 0 || p >= max_pos || slot < 0 || slot >= num_slots) return;
  const int64_t page = slot >> ps;
  const int off = (int)(slot & ((1 << ps) - 1));
  uint8_t* base = cache + page_base(page, ps);
  const uint16_t* kr = kv + t * kLatent;

  // nope dims 8*lane .. 8*lane+7, block lane/8
  uint4 v = *reinterpret_cast<const uint4*>(kr + 8 * lane);
  uint32_t u[4] = {v.x, v.y, v.z, v.w};
  float k[8];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k[2 * e] = bf16_bits_to_f32(u[e] & 0xFFFF);
    k[2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(k[2 * e]), fabsf(k[2 * e + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
  // smallest e with amax <= 448 * 2^e: amax = m * 2^k, m in [1,2): e = k-8 if m <= 1.75
  // else k-7; zero and fp32-subnormal amax (< 2^-126 < 448 * 2^-127) give e = -127.
  const uint32_t ab = __float_as_uint(amax);
  const int fexp = (int)(ab >> 23);
  int e = -127;
  if (fexp != 0) {
    e = (fexp - 127) - 8 + ((ab & 0x7FFFFF) > 0x600000 ? 1 : 0);
    e = max(-127, min(127, e));
  }
  uint32_t codes[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int c = 0;
    c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(k[4 * h + 0], -e),
                                        __builtin_amdgcn_ldexpf(k[4 * h + 1], -e), c, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(k[4 * h + 2], -e),
                                        __builtin_amdgcn_ldexpf(k[4 * h + 3], -e), c, true);
    codes[h] = (uint32_t)c;
  }
  *reinterpret_cast<uint2*>(base + nope_off(off) + 8 * lane) = make_uint2(codes[0], codes[1]);
  if ((lane & 7) == 0) base[scale_off(off, ps) + (lane >> 3)] = (uint8_t)(e + 127);

  // rope dims 512 + 8*lane .. +7 for lanes 0..7, stored rotated (bf16)
  if (lane < 8) {
    uint4 rv = *reinterpret_cast<const uint4*>(kr + kNope + 8 * lane);
    uint32_t ru[4] = {rv.x, rv.y, rv.z, rv.w};
    const float* cs = cos_sin + p * kRope + 4 * lane;
    const float4 cv = *reinterpret_cast<const float4*>(cs);
    const float4 sv = *reinterpret_cast<const float4*>(cs + kRope / 2);
    const float cc[4] = {cv.x, cv.y, cv.z, cv.w}, sn[4] = {sv.x, sv.y, sv.z, sv.w};
    uint32_t o[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float a = bf16_bits_to_f32(ru[e2] & 0xFFFF), b = bf16_bits_to_f32(ru[e2] >> 16);
      o[e2] = pack_bf16x2(a * cc[e2] - b * sn[e2], a * sn[e2] + b * cc[e2]);
    }
    *reinterpret_cast<uint4*>(base + rope_off(off, ps) + 16 * lane) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// One launch: blocks [0, qblocks) stream the q rows, the remaining blocks quantise the
// new latent rows (4 tokens per block).
__global__ void __launch_bounds__(256) insert_kernel(
    uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int64_t* __restrict__ positions,
    const int64_t* __restrict__ slot_mapping, const float* __restrict__ cos_sin, int max_pos,
    const uint16_t* __restrict__ weight, float eps, uint8_t* __restrict__ cache, int64_t num_slots,
    int ps, int T, int H, int qblocks) {
  if ((int)blockIdx.x < qblocks)
    q_norm_rope(q, positions, cos_sin, max_pos, weight, eps, (int64_t)T * H, H, qblocks);
  else
    kv_quant_insert(kv, positions, slot_mapping, cos_sin, max_pos, cache, num_slots, ps, T,
                    (int)blockIdx.x - qblocks);
}

hipError_t launch_insert(void* q, const void* kv, const int64_t* positions,
                         const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                         const void* weight, float eps, uint8_t* cache, int num_pages,
                         int page_shift, int T, int H, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t rows = (int64_t)T * H;
  const int64_t groups = (rows + 31) / 32;  // 32 q rows per 256-thread block per pass
  const int qblocks = rows > 0 ? (int)(groups < 8192 ? groups : 8192) : 0;
  const int kvblocks = (T + 3) / 4;
  hipLaunchKernelGGL(insert_kernel, dim3(qblocks + kvblocks), dim3(256), 0, stream,
                     static_cast<uint16_t*>(q), static_cast<const uint16_t*>(kv), positions,
                     slot_mapping, cos_sin, max_pos, static_cast<const uint16_t*>(weight), eps,
                     cache, (int64_t)num_pages << page_shift, page_shift, T, H, qblocks);
  return hipGetLastError();
}

}  // namespace dsv4
