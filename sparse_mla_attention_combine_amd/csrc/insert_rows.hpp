// Per-row pieces of the fused insert (per-head q RMSNorm + GPT-J RoPE; FP8 E4M3 / UE8M0
// quantisation of a latent row into the cache), shared by the insert kernel and the
// decode kernel that performs the whole step, so that both compute identical bits.
// Follows PR #42953 (Implementation breakdown item 4; Key source excerpts:
// _fused_qnorm_rope_kv_insert called with q, kv, kv_cache, slot_mapping, positions).
#pragma once
#include "device.hpp"

namespace dsv4 {

// cos and sin of rotary pairs 4j .. 4j+3 (j = lane & 7) of a position's row of the
// table (64 floats: 32 cos then 32 sin).
struct RopeCs {
  float4 c;
  float4 s;
};

__device__ __forceinline__ RopeCs rope_cs_load(const float* __restrict__ row, int lane) {
  RopeCs r;
  r.c = *reinterpret_cast<const float4*>(row + 4 * (lane & 7));
  r.s = *reinterpret_cast<const float4*>(row + 4 * (lane & 7) + kRope / 2);
  return r;
}

// q row RMSNorm + RoPE.  8 lanes (lane & 7 = c8) hold chunks c8 + 8k (k = 0..8) of one
// head's 576 dims, i.e. dims 8(c8 + 8k) .. +7.  Two passes over the chunks, in k order:
//   ss  = qn_sum_sq(chunk k, ss) for k = 0..8   (squares added in dim order in the lane)
//   inv = qn_inv(ss, eps)                        (sum over the 8 lanes by xor-shuffles,
//                                                 eps inside the square root)
//   out = qn_chunk(chunk k, weight chunk k, inv, rot, k == 8)
// where qn_chunk multiplies by inv and the weight, rotates the GPT-J pairs of dims
// 512..575 (chunk 8; `rot` holds the position's cos/sin values, rope_cs_load) and rounds
// once to bf16.  The chunks may live in registers or in LDS: every caller runs this same
// sequence of operations, so all produce the same bits.
__device__ __forceinline__ float qn_sum_sq(u32x4 c, float ss) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = bf16_bits_to_f32(c[e] & 0xFFFF), b = bf16_bits_to_f32(c[e] >> 16);
    ss += a * a;
    ss += b * b;
  }
  return ss;
}

// Partner values within each aligned group of 8 lanes, in DPP moves (no LDS round
// trip): lane i ^ 1 and lane i ^ 2 (quad permutations), then lane 7 - i of the group
// (half-row mirror), which lies in the other quad.  After the two quad steps every lane
// of a quad holds the quad's result, so the mirror step gives every lane the same value
// as an xor-4 step would.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;

// All 8 lanes of a row must take part.
__device__ __forceinline__ float qn_inv(float ss, float eps) {
  ss += dpp_partner<kDppXor1>(ss);
  ss += dpp_partner<kDppXor2>(ss);
  ss += dpp_partner<kDppHalfMirror>(ss);
  return 1.0f / sqrtf(ss * (1.0f / kLatent) + eps);
}

__device__ __forceinline__ u32x4 qn_chunk(u32x4 c, u32x4 w, float inv, const RopeCs& rot,
                                          bool rope) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = bf16_bits_to_f32(c[e] & 0xFFFF) * inv * bf16_bits_to_f32(w[e] & 0xFFFF);
    y[2 * e + 1] = bf16_bits_to_f32(c[e] >> 16) * inv * bf16_bits_to_f32(w[e] >> 16);
  }
  if (rope) {
    // chunk 8 holds dims 512 + 8*c8 .. +7, i.e. rotary pairs 4*c8 .. 4*c8+3
    const float cc[4] = {rot.c.x, rot.c.y, rot.c.z, rot.c.w};
    const float sn[4] = {rot.s.x, rot.s.y, rot.s.z, rot.s.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = y[2 * e], b = y[2 * e + 1];
      y[2 * e] = a * cc[e] - b * sn[e];
      y[2 * e + 1] = a * sn[e] + b * cc[e];
    }
  }
  u32x4 o;
  o[0] = pack_bf16x2(y[0], y[1]);
  o[1] = pack_bf16x2(y[2], y[3]);
  o[2] = pack_bf16x2(y[4], y[5]);
  o[3] = pack_bf16x2(y[6], y[7]);
  return o;
}

// One lane's share of a latent row (576 bf16) for a wave of 64 lanes: nope dims
// 8*lane .. 8*lane+7 (quantisation block lane/8) and rope dims 512 + 8*(lane&7) .. +7
// (used by lanes 0..7; every lane loads, so no load sits under a per-lane condition).
struct KvLane {
  uint4 nope;
  uint4 rope;
};

__device__ __forceinline__ KvLane kv_lane_load(const uint16_t* __restrict__ kr, int lane) {
  KvLane v;
  v.nope = *reinterpret_cast<const uint4*>(kr + 8 * lane);
  v.rope = *reinterpret_cast<const uint4*>(kr + kNope + 8 * (lane & 7));
  return v;
}

// Rope dims 512 + 8j .. +7 (a lane's KvLane::rope, j = lane & 7) rotated by the GPT-J pairs
// of its position (rope_cs_load) and rounded to bf16.
__device__ __forceinline__ uint4 rope_rotate8(uint4 r, const RopeCs& rot) {
  const uint32_t ru[4] = {r.x, r.y, r.z, r.w};
  const float cc[4] = {rot.c.x, rot.c.y, rot.c.z, rot.c.w};
  const float sn[4] = {rot.s.x, rot.s.y, rot.s.z, rot.s.w};
  uint32_t o[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const float a = bf16_bits_to_f32(ru[e2] & 0xFFFF), b = bf16_bits_to_f32(ru[e2] >> 16);
    o[e2] = pack_bf16x2(a * cc[e2] - b * sn[e2], a * sn[e2] + b * cc[e2]);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Quantises the row held by a wave (kv_lane_load) into the record of slot `off` of the
// page at `base` (pages of 2^ps slots); `rot` holds the cos/sin values of the row's
// position (rope_cs_load).
// The block amax is exact, the exponent comes from the fp32 bit fields, the scaling by
// 2^-e is exact and the E4M3 rounding is gfx950's RNE conversion; lanes 0..7 rotate and
// store the rope dims.  All 64 lanes must take part.
__device__ __forceinline__ void kv_quant_store(const KvLane& v, const RopeCs& rot,
                                               uint8_t* __restrict__ base, int off, int ps,
                                               int lane) {
  const uint32_t u[4] = {v.nope.x, v.nope.y, v.nope.z, v.nope.w};
  float k[8];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k[2 * e] = bf16_bits_to_f32(u[e] & 0xFFFF);
    k[2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(k[2 * e]), fabsf(k[2 * e + 1])));
  }
  amax = fmaxf(amax, dpp_partner<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_partner<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_partner<kDppHalfMirror>(amax));
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
  if (lane < 8) *reinterpret_cast<uint4*>(base + rope_off(off, ps) + 16 * lane) = rope_rotate8(v.rope, rot);
}

// The other kv-cache dtypes (PR #43477 Key source excerpts: the SM100 backend's
// "bfloat16" and "fp8" caches of shape (num_blocks, block_size, head_size)): one record
// of the 576 values per slot in dim order, `rec` pointing at the slot's record.  The
// rope dims are rotated and rounded to bf16 exactly as for the packed record.  bf16:
// the values' bits.  fp8 (one scale s per cache): e4m3(z / s) for every dim, the
// quotient correctly rounded in fp32, saturated to +-448, converted with gfx950's
// round-to-nearest-even.  All 64 lanes must take part (lanes 0..7 store the rope dims).
__device__ __forceinline__ void kv_store_bf16(const KvLane& v, const RopeCs& rot,
                                              uint8_t* __restrict__ rec, int lane) {
  *reinterpret_cast<uint4*>(rec + 16 * lane) = v.nope;
  if (lane < 8) *reinterpret_cast<uint4*>(rec + 2 * kNope + 16 * lane) = rope_rotate8(v.rope, rot);
}

// 8 bf16 values (memory order) -> 8 E4M3 codes of z / s.
__device__ __forceinline__ uint2 e4m3_quot8(uint4 z, float s) {
  const uint32_t u[4] = {z.x, z.y, z.z, z.w};
  float k[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k[2 * e] = fminf(fmaxf(bf16_bits_to_f32(u[e] & 0xFFFF) / s, -448.f), 448.f);
    k[2 * e + 1] = fminf(fmaxf(bf16_bits_to_f32(u[e] >> 16) / s, -448.f), 448.f);
  }
  uint32_t codes[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int c = 0;
    c = __builtin_amdgcn_cvt_pk_fp8_f32(k[4 * h + 0], k[4 * h + 1], c, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(k[4 * h + 2], k[4 * h + 3], c, true);
    codes[h] = (uint32_t)c;
  }
  return make_uint2(codes[0], codes[1]);
}

__device__ __forceinline__ void kv_store_fp8(const KvLane& v, const RopeCs& rot, float s,
                                             uint8_t* __restrict__ rec, int lane) {
  *reinterpret_cast<uint2*>(rec + 8 * lane) = e4m3_quot8(v.nope, s);
  if (lane < 8) *reinterpret_cast<uint2*>(rec + kNope + 8 * lane) = e4m3_quot8(rope_rotate8(v.rope, rot), s);
}

// The row writer of a cache dtype (packed FP8/UE8M0, bf16, or fp8 with scale s)
// for slot `slot` of a cache of pages of 2^ps slots.
template <int KV>
__device__ __forceinline__ void kv_store_row(const KvLane& v, const RopeCs& rot, uint8_t* cache,
                                             int64_t slot, int ps, float s, int lane) {
  if constexpr (KV == kKvFp8Ds) {
    kv_quant_store(v, rot, cache + page_base(slot >> ps, ps), (int)(slot & ((1 << ps) - 1)), ps, lane);
  } else if constexpr (KV == kKvBf16) {
    kv_store_bf16(v, rot, cache + slot * (2 * kLatent), lane);
  } else {
    kv_store_fp8(v, rot, s, cache + slot * kLatent, lane);
  }
}

// q RMSNorm + RoPE in place over q rows [T*H][576] for the waves of `nblocks` blocks of
// 256 threads, this one being block `block`: wave k handles rows 8k .. 8k+7, then
// 8(k + nwaves) ..., each row over 8 lanes (the partition above).  A row whose token's
// position lies outside [0, max_pos) is left untouched.
__device__ __forceinline__ void q_norm_rope_rows(
    uint16_t* __restrict__ q, const int64_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, const uint16_t* __restrict__ weight, float eps,
    int64_t rows, int H, int block, int nblocks) {
  const int lane = threadIdx.x & 63;
  const int r8 = lane >> 3, c8 = lane & 7;
  // this lane always touches chunks c8 + 8k (k = 0..8) of a row: keep their weights
  u32x4 w[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) w[k] = *reinterpret_cast<const u32x4*>(weight + 8 * (c8 + 8 * k));
  const int64_t wave = ((int64_t)block * 256 + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)nblocks * 256) >> 6;
  for (int64_t g = wave; g * 8 < rows; g += nwaves) {
    const int64_t row = g * 8 + r8;
    if (row >= rows) continue;
    const int64_t t = row / H;
    const int64_t p = positions[t];
    uint16_t* qr = q + row * kLatent;
    // the row is requested together with its position; the position is only tested after
    // the row has been consumed, so the compiler keeps the loads side by side
    u32x4 x[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) x[k] = *reinterpret_cast<const u32x4*>(qr + 8 * (c8 + 8 * k));
    const bool ok = p >= 0 && p < max_pos;
    const RopeCs rot = rope_cs_load(cos_sin + (ok ? p : 0) * kRope, c8);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 9; ++k) ss = qn_sum_sq(x[k], ss);
    const float inv = qn_inv(ss, eps);
    if (!ok) continue;  // token left untouched
#pragma unroll
    for (int k = 0; k < 9; ++k)
      *reinterpret_cast<u32x4*>(qr + 8 * (c8 + 8 * k)) = qn_chunk(x[k], w[k], inv, rot, k == 8);
  }
}

}  // namespace dsv4
