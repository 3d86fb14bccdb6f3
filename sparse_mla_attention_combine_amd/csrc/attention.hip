// Sparse MQA-form MLA attention over the FP8/UE8M0 paged latent cache (decode and
// prefill entry points).  What is computed follows PR #42953 (Key source excerpts,
// xpu_sparse_decode_fp8: gather + dequantise the listed slots, then bf16 sparse MLA with
// per-row lengths) and PR #43477 (forward_mqa: physical indices in, (T, H, 512) out;
// supports_sink).  Unlike the XPU design, nothing is written back to a bf16 workspace:
// the gather, the dequantisation and both contractions are fused in one kernel.
//
// Work decomposition (gfx950, 256 CUs in 8 XCDs):
//   workgroup = (query token t, group of NH = 16*NHB heads); 4 waves; 1 workgroup/CU.
//   The head groups of a token get block ids with the same value mod 8, so they run on
//   the same XCD and the three later gathers of each slot hit that XCD's L2.
//   The listed slots are consumed in chunks of 64; wave w owns rows 16w..16w+15.
// Per chunk:
//   1. every lane holds its slot's 128 nope bytes, 32 rope bytes and 8 scale bytes in
//      registers (requested two chunks ahead, as soon as the buffer is consumed; the
//      token's index row is staged in LDS first and every load is branch-free, so the
//      wait before a chunk covers exactly that chunk), converts them with gfx950's scaled
//      FP8->bf16 instruction (exact: a power-of-two scale) into MFMA A-fragments, and
//      stages the 512 value dims as bf16 rows in an XOR-swizzled LDS tile;
//   2. S^T = K Q^T on bf16 MFMA 16x16x32 (Q^T fragments live in registers for the whole
//      kernel);
//   3. online softmax in the log2 domain: per-wave maxima through lane swaps
//      (permlane16/32), the chunk maximum across the 4 waves through LDS; the reference
//      maximum only moves (and O is rescaled) when a chunk beats it by more than 2^8;
//      probabilities are rounded to bf16 into LDS;
//   4. O^T += V^T P^T on bf16 MFMA 16x16x32: wave w owns output dims 128w..128w+127 for
//      all NH heads; V^T fragments come from the row-major LDS tile through gfx950's
//      transposing LDS read (ds_read_b64_tr_b16), P^T fragments are plain 16 B reads.
//   LDS buffers are double-buffered so chunk i+1's staging overlaps chunk i's P.V.
// Numerics: bf16 operands, fp32 accumulation and softmax, P rounded to bf16 for P.V;
// the per-head sink enters only the final denominator.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

constexpr int kChunk = 64;
constexpr int kVStride = 512;  // bf16 per LDS value row (1024 B, 16 B units XOR-swizzled)
constexpr int kPStride = 72;   // bf16 per LDS probability row: 144 B
// The running max is only moved (and O rescaled) when a chunk beats it by more than
// 2^8 in probability units; in between, probabilities up to 256 are exact in bf16/fp32.
constexpr float kRescaleSlack = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kIdxBlock = 4096;  // index entries staged in LDS at a time (64 chunks)

template <int NHB>
struct AttnSmem {
  __bf16 v[2][kChunk][kVStride];
  __bf16 p[2][16 * NHB][kPStride];
  float red[2][4][16 * NHB];
  float lsum[4][16 * NHB];
  int32_t idx[kIdxBlock];
};

// Source of the (all-zero) record read for an invalid or absent slot, so that every
// lane issues the same loads every chunk: branch-free loads let the compiler wait for
// exactly the chunk it is about to use while later chunks stay in flight.
__device__ __attribute__((aligned(64))) uint8_t g_zero_page[kPage * kRecord];

struct RawSlot {
  uint4 nope[8];  // 128 codes: dims 64u + 16g .. 64u + 16g + 15 for u = 0..7
  uint4 rope[2];  // rope dims 8g..8g+7 and 32+8g..32+8g+7 (bf16)
  uint2 sc;       // the slot's 8 scale bytes
  int valid;
};

__device__ __forceinline__ void load_raw(RawSlot& r, const uint8_t* __restrict__ cache,
                                         int64_t num_slots, const int32_t* idx_lds, int jj,
                                         int n_blk, int g) {
  const int64_t slot = jj < n_blk ? (int64_t)idx_lds[jj] : -1;
  r.valid = (slot >= 0 && slot < num_slots) ? 1 : 0;
  const uint8_t* base = r.valid ? cache + page_base(slot >> 6) : g_zero_page;
  const int off = r.valid ? (int)(slot & (kPage - 1)) : 0;
  const uint8_t* np = base + nope_off(off) + 16 * g;
#pragma unroll
  for (int u = 0; u < 8; ++u) r.nope[u] = *reinterpret_cast<const uint4*>(np + 64 * u);
  const uint8_t* rp = base + rope_off(off) + 16 * g;
  r.rope[0] = *reinterpret_cast<const uint4*>(rp);
  r.rope[1] = *reinterpret_cast<const uint4*>(rp + 64);
  r.sc = *reinterpret_cast<const uint2*>(base + scale_off(off));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

// V tile layout: row j of the chunk occupies 1024 B; its 16 B unit k (value dims
// 8k..8k+7) is stored at unit k ^ swz(j).  swz spreads the b128 row writes of a wave
// (16 rows x 4 k-groups) over all banks, and keeps the 4 rows x 2 units that one
// 16-lane group of a transposing read touches on distinct banks.
__device__ __forceinline__ int v_swz(int row) {
  return (2 * (row & 3)) | ((row >> 2) & 1) | (((row >> 3) & 1) << 3);
}
__device__ __forceinline__ int v_off(int row, int unit) {  // in bf16 elements
  return row * kVStride + ((unit ^ v_swz(row)) << 3);
}

// max / sum with the lane 16 (resp. 32) apart, without going through LDS: the swap
// hands each lane its partner's value in one of the two results and keeps its own in
// the other.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int NHB>
struct AttnState {
  bf16x8 qf[NHB][18];  // Q^T fragments (registers for the whole kernel)
  float m_run[NHB];    // running max per head (log2 domain), same in every wave
  float l_part[NHB];   // this lane's share of the softmax denominator
  f32x4 oacc[8][NHB];  // O^T for output dims 128w + 16mb + 4g + i, head l16 of block hb
};

// One chunk of 64 listed slots: dequantise + stage V + S^T = K Q^T, online softmax,
// O^T += V^T P^T.  `cur` holds this wave's 16 slots (row l16, k-group g) of the chunk.
template <int NHB>
__device__ __forceinline__ void chunk_step(AttnSmem<NHB>& sm, AttnState<NHB>& st,
                                           const RawSlot& cur, RawSlot& pf, int pf_jj, int n_blk,
                                           const uint8_t* __restrict__ cache, int64_t num_slots,
                                           int buf, int w, int l16, int g, float scale_log2) {
  // ---- dequantise, stage V, S^T = K Q^T
  f32x4 sacc[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  __bf16* vtile = &sm.v[buf][0][0];
  const int vr = 16 * w + l16;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t sb = ((u < 4 ? cur.sc.x : cur.sc.y) >> (8 * (u & 3))) & 0xFF;
    const float scale = e8m0_as_scale(sb);
    const bf16x8 k0 = dequant8(cur.nope[u].x, cur.nope[u].y, scale);
    const bf16x8 k1 = dequant8(cur.nope[u].z, cur.nope[u].w, scale);
    *reinterpret_cast<bf16x8*>(vtile + v_off(vr, 8 * u + 2 * g)) = k0;
    *reinterpret_cast<bf16x8*>(vtile + v_off(vr, 8 * u + 2 * g + 1)) = k1;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      sacc[hb] = mfma16(k0, st.qf[hb][2 * u], sacc[hb]);
      sacc[hb] = mfma16(k1, st.qf[hb][2 * u + 1], sacc[hb]);
    }
  }
  {
    const bf16x8 k16 = as_bf16x8(cur.rope[0]);
    const bf16x8 k17 = as_bf16x8(cur.rope[1]);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      sacc[hb] = mfma16(k16, st.qf[hb][16], sacc[hb]);
      sacc[hb] = mfma16(k17, st.qf[hb][17], sacc[hb]);
    }
  }

  // ---- request the records of a later chunk now that `cur` has been consumed
  const uint64_t vmask = __ballot(cur.valid);  // bit j (j < 16) = row j of this wave valid
  load_raw(pf, cache, num_slots, sm.idx, pf_jj, n_blk, g);

  // ---- online softmax (log2 domain). sacc[hb][i] = score of row 4g+i, head l16.
  float s[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (vmask >> (4 * g + i)) & 1;
      s[hb][i] = ok ? sacc[hb][i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[hb][i]);
    }
    mx = max_xor32(max_xor16(mx));
    if (g == 0) sm.red[buf][w][16 * hb + l16] = mx;
  }
  __syncthreads();
  float alpha[NHB];
  bool rescale = false;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float cm = sm.red[buf][0][16 * hb + l16];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) cm = fmaxf(cm, sm.red[buf][ww][16 * hb + l16]);
    // move the reference max only when this chunk beats it by more than the slack
    alpha[hb] = 1.f;
    if (cm > st.m_run[hb] + kRescaleSlack) {
      alpha[hb] = (st.m_run[hb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m_run[hb] - cm);
      st.m_run[hb] = cm;
      rescale = true;
    }
    const float mr = st.m_run[hb];
    float p[4], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = (s[hb][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[hb][i] - mr);
      sum += p[i];
    }
    st.l_part[hb] = st.l_part[hb] * alpha[hb] + sum;
    *reinterpret_cast<uint2*>(&sm.p[buf][16 * hb + l16][16 * w + 4 * g]) =
        make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  }
  if (__builtin_amdgcn_ballot_w64(rescale)) {  // wave-uniform, rare after the first chunk
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) st.oacc[mb][hb] *= alpha[hb];
  }
  __syncthreads();

  // ---- O^T[c][h] += V^T[c][j] P^T[j][h] for c in 128w..128w+127.  All LDS reads of a
  // 32-slot step are issued before its MFMAs, so their latencies overlap instead of
  // being paid one by one.
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 pf[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      pf[hb] = *reinterpret_cast<const bf16x8*>(&sm.p[buf][16 * hb + l16][32 * ks + 8 * g]);
    // transposing reads: input lane 4r+q of a 16-lane group addresses row j0+r, value
    // dims c0+4q..c0+4q+3 (unit c0/8 + q/2, half q&1); lane L receives dim c0+L of rows
    // j0..j0+3.  Rows j0 = 32ks+8g (+4 for the second read).
    const int j0 = 32 * ks + 8 * g + (l16 >> 2);
    const int q4 = l16 & 3;
    bf16x4 t0[8], t1[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int unit = 16 * w + 2 * mb + (q4 >> 1);
      t0[mb] = lds_read_tr16(vtile + v_off(j0, unit) + 4 * (q4 & 1));
      t1[mb] = lds_read_tr16(vtile + v_off(j0 + 4, unit) + 4 * (q4 & 1));
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      bf16x8 vf;
      vf[0] = t0[mb][0]; vf[1] = t0[mb][1]; vf[2] = t0[mb][2]; vf[3] = t0[mb][3];
      vf[4] = t1[mb][0]; vf[5] = t1[mb][1]; vf[6] = t1[mb][2]; vf[7] = t1[mb][3];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) st.oacc[mb][hb] = mfma16(vf, pf[hb], st.oacc[mb][hb]);
    }
  }
}

template <int NHB>
__global__ void __launch_bounds__(256) sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots,
    const int32_t* __restrict__ indices, int idx_stride, const int32_t* __restrict__ lens,
    const float* __restrict__ sinks, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int T, int H, int groups) {
  __shared__ AttnSmem<NHB> sm;

  int t, hg;
  if (groups == 1) {
    t = blockIdx.x;
    hg = 0;
  } else {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    hg = k % groups;
    t = (k / groups) * 8 + x;
  }
  if (t >= T) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int h0 = hg * 16 * NHB;
  int n = lens[t];
  n = n < idx_stride ? n : idx_stride;
  n = n > 0 ? n : 0;
  const int32_t* idx_row = indices + (int64_t)t * idx_stride;

  AttnState<NHB> st;
  // Q^T fragments: lane (head l16 of block hb, k-group g); k-step s pairs with the
  // K-fragment dims chosen in load_raw (nope: 64u+16g+8h, rope: 32r+8g).
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint16_t* qr = q + ((int64_t)t * H + h0 + 16 * hb + l16) * kLatent;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      st.qf[hb][2 * u] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 64 * u + 16 * g));
      st.qf[hb][2 * u + 1] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 64 * u + 16 * g + 8));
    }
    st.qf[hb][16] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kNope + 8 * g));
    st.qf[hb][17] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kNope + 32 + 8 * g));
    st.m_run[hb] = -INFINITY;
    st.l_part[hb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) st.oacc[mb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Index blocks of up to 4096 entries are staged in LDS; inside a block, the records of
  // chunk c+2 are requested as soon as chunk c's contraction has consumed its buffer,
  // so two register buffers keep two chunks in flight (2x unrolled, never copied).
  const int row = 16 * w + l16;
  int gch = 0;  // chunks done so far (parity of the LDS double buffers)
  for (int blk0 = 0; blk0 < n; blk0 += kIdxBlock) {
    const int n_blk = min(n - blk0, kIdxBlock);
    __syncthreads();  // the previous block's entries are no longer read
#pragma unroll 4
    for (int i = tid; i < n_blk; i += 256) sm.idx[i] = idx_row[blk0 + i];
    __syncthreads();
    const int nch = (n_blk + kChunk - 1) / kChunk;
    RawSlot A, B;
    load_raw(A, cache, num_slots, sm.idx, row, n_blk, g);
    load_raw(B, cache, num_slots, sm.idx, kChunk + row, n_blk, g);
    int c = 0;
    // chunk c computes from one buffer and refills it with chunk c+2 once consumed
    for (; c + 2 <= nch; c += 2) {
      chunk_step<NHB>(sm, st, A, A, (c + 2) * kChunk + row, n_blk, cache, num_slots,
                      (gch + c) & 1, w, l16, g, scale_log2);
      chunk_step<NHB>(sm, st, B, B, (c + 3) * kChunk + row, n_blk, cache, num_slots,
                      (gch + c + 1) & 1, w, l16, g, scale_log2);
    }
    if (c < nch)
      chunk_step<NHB>(sm, st, A, A, (c + 2) * kChunk + row, n_blk, cache, num_slots,
                      (gch + c) & 1, w, l16, g, scale_log2);
    gch += nch;
  }

  // ---- finalise: sum the waves' partial denominators, add the sink, normalise
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float lp = sum_xor32(sum_xor16(st.l_part[hb]));
    if (g == 0) sm.lsum[w][16 * hb + l16] = lp;
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int h = h0 + 16 * hb + l16;
    const float lt = sm.lsum[0][16 * hb + l16] + sm.lsum[1][16 * hb + l16] +
                     sm.lsum[2][16 * hb + l16] + sm.lsum[3][16 * hb + l16];
    const float mr = st.m_run[hb];
    const float z2 = sinks ? sinks[h] * kLog2e : -INFINITY;
    const float M = fmaxf(mr, z2);
    const float f = (mr == -INFINITY) ? 0.f : exp2f(mr - M);
    const float den = lt * f + ((z2 == -INFINITY) ? 0.f : exp2f(z2 - M));
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow = out + ((int64_t)t * H + h) * kNope + 128 * w + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const f32x4 o = st.oacc[mb][hb];
      *reinterpret_cast<uint2*>(orow + 16 * mb) =
          make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
    }
    if (lse && w == 0 && g == 0) lse[(int64_t)t * H + h] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_attention(const void* q, const uint8_t* cache, int num_pages,
                            const int32_t* indices, int idx_stride, const int32_t* lens,
                            const float* sinks, float softmax_scale, void* out, float* lse, int T,
                            int H, bool prefill, hipStream_t stream) {
  (void)prefill;  // one schedule serves both entry points for now
  if (T == 0) return hipSuccess;
  const int64_t num_slots = (int64_t)num_pages * kPage;
  const float scale_log2 = softmax_scale * kLog2e;
  if (H == 16) {
    hipLaunchKernelGGL(sparse_mla_kernel<1>, dim3(T), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), cache, num_slots, indices, idx_stride, lens,
                       sinks, scale_log2, static_cast<uint16_t*>(out), lse, T, H, 1);
  } else {
    const int groups = H / 32;
    const int grid = groups == 1 ? T : 8 * groups * ((T + 7) / 8);
    hipLaunchKernelGGL(sparse_mla_kernel<2>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), cache, num_slots, indices, idx_stride, lens,
                       sinks, scale_log2, static_cast<uint16_t*>(out), lse, T, H, groups);
  }
  return hipGetLastError();
}

}  // namespace dsv4
