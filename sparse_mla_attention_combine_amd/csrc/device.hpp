// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLatent = 576;
constexpr int kNope = 512;
constexpr int kRope = 64;
constexpr int kBlocks = 8;
constexpr int kRecord = 648;
constexpr int kMaxPage = 256;  // page sizes accepted by the launchers: 32, 64 and 256 slots

// kv-cache dtypes (the DSV4_KV_* values of the C header).  kKvFp8Ds: the packed record
// below (E4M3 codes, UE8M0 block scales, bf16 rope; pages split by field).  kKvBf16 and
// kKvFp8E4m3: one record of the 576 values per slot in dim order, records back to back
// (slot s at byte s * record bytes): bf16 values (1152 B), or E4M3 codes (576 B) with one
// scale for the whole cache (PR #43477 Key source excerpts: the SM100 backend's kv-cache
// dtypes "bfloat16" / "fp8" and its (num_blocks, block_size, head_size) cache shape).
constexpr int kKvFp8Ds = 0;
constexpr int kKvBf16 = 1;
constexpr int kKvFp8E4m3 = 2;
constexpr int kv_record_bytes_of(int kv_dtype) {
  return kv_dtype == kKvFp8Ds ? 648 : kv_dtype == kKvBf16 ? 2 * 576 : kv_dtype == kKvFp8E4m3 ? 576 : 0;
}

// A page of P = 2^ps slots holds the E4M3 codes [P][512] at byte 0, the bf16 rope rows
// [P][64] at P*512 and the UE8M0 scales [P][8] at P*640.  Byte offsets of a page and of
// the three fields of its slot `off`:
__device__ __forceinline__ int64_t page_base(int64_t page, int ps) { return (page * (int64_t)kRecord) << ps; }
__device__ __forceinline__ int nope_off(int off) { return off * kNope; }
__device__ __forceinline__ int rope_off(int off, int ps) { return (kNope << ps) + off * kRope * 2; }
__device__ __forceinline__ int scale_off(int off, int ps) { return ((kNope + 2 * kRope) << ps) + off * kBlocks; }

// UE8M0 byte -> an fp32 whose exponent field is that byte.  gfx950's scaled FP8
// conversions read only the exponent field of the scale operand as an E8M0 value
// (2^(field-127), field 0 included), so this is an exact 2^(byte-127) multiplier.
__device__ __forceinline__ float e8m0_as_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// 4 E4M3 codes in a dword -> 4 bf16 (code * scale), bytes in memory order.
__device__ __forceinline__ void dequant4(uint32_t codes, float scale, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, scale, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, scale, true);
}

// 8 E4M3 codes (two dwords, memory order) -> bf16x8.
__device__ __forceinline__ bf16x8 dequant8(uint32_t c0, uint32_t c1, float scale) {
  bf16x2 a, b, c, d;
  dequant4(c0, scale, a, b);
  dequant4(c1, scale, c, d);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)x);
}

// Two fp32 values -> two bf16 (round to nearest even) in one dword, a in the low half: one
// v_cvt_pk_bf16_f32 (two scalar conversions would also shift and merge the halves).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

}  // namespace dsv4
