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
//   1. every lane loads its slot's 128 nope bytes, 32 rope bytes and 8 scale bytes
//      straight from HBM into registers (issued one chunk ahead), converts them with
//      gfx950's scaled FP8->bf16 instruction (exact: a power-of-two scale) into MFMA
//      A-fragments, and stages the 512 value dims as bf16 rows in LDS;
//   2. S^T = K Q^T on bf16 MFMA 16x16x32 (Q^T fragments live in registers for the whole
//      kernel);
//   3. online softmax in the log2 domain: per-wave maxima over 3 xor-shuffles, the
//      chunk maximum across the 4 waves through LDS, then probabilities rounded to bf16
//      into LDS;
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
constexpr int kVStride = 528;  // bf16 per LDS value row: 1056 B, 32 B skew per row
constexpr int kPStride = 72;   // bf16 per LDS probability row: 144 B
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int NHB>
struct AttnSmem {
  __bf16 v[2][kChunk][kVStride];
  __bf16 p[2][16 * NHB][kPStride];
  float red[2][4][16 * NHB];
  float lsum[4][16 * NHB];
};

struct RawSlot {
  uint4 nope[8];  // 128 codes: dims 64u + 16g .. 64u + 16g + 15 for u = 0..7
  uint4 rope[2];  // rope dims 8g..8g+7 and 32+8g..32+8g+7 (bf16)
  uint2 sc;       // the slot's 8 scale bytes
  int valid;
};

__device__ __forceinline__ void load_raw(RawSlot& r, const uint8_t* __restrict__ cache,
                                         int64_t num_slots, const int32_t* __restrict__ idx_row,
                                         int jj, int n, int g) {
  int64_t slot = -1;
  if (jj < n) slot = idx_row[jj];
  r.valid = (slot >= 0 && slot < num_slots) ? 1 : 0;
  if (r.valid) {
    const uint8_t* base = cache + page_base(slot >> 6);
    const int off = (int)(slot & (kPage - 1));
    const uint8_t* np = base + nope_off(off) + 16 * g;
#pragma unroll
    for (int u = 0; u < 8; ++u) r.nope[u] = *reinterpret_cast<const uint4*>(np + 64 * u);
    const uint8_t* rp = base + rope_off(off) + 16 * g;
    r.rope[0] = *reinterpret_cast<const uint4*>(rp);
    r.rope[1] = *reinterpret_cast<const uint4*>(rp + 64);
    r.sc = *reinterpret_cast<const uint2*>(base + scale_off(off));
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) r.nope[u] = make_uint4(0, 0, 0, 0);
    r.rope[0] = r.rope[1] = make_uint4(0, 0, 0, 0);
    r.sc = make_uint2(0, 0);
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

template <int NHB>
__global__ void __launch_bounds__(256) sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots,
    const int32_t* __restrict__ indices, int idx_stride, const int32_t* __restrict__ lens,
    const float* __restrict__ sinks, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int T, int H, int groups) {
  constexpr int NH = 16 * NHB;
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
  const int h0 = hg * NH;
  int n = lens[t];
  n = n < idx_stride ? n : idx_stride;
  n = n > 0 ? n : 0;
  const int nch = (n + kChunk - 1) / kChunk;
  const int32_t* idx_row = indices + (int64_t)t * idx_stride;

  // Q^T fragments: lane (head l16 of block hb, k-group g); k-step s pairs with the
  // K-fragment dims chosen in load_raw (nope: 64u+16g+8h, rope: 32r+8g).
  bf16x8 qf[NHB][18];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint16_t* qr = q + ((int64_t)t * H + h0 + 16 * hb + l16) * kLatent;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      qf[hb][2 * u] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 64 * u + 16 * g));
      qf[hb][2 * u + 1] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 64 * u + 16 * g + 8));
    }
    qf[hb][16] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kNope + 8 * g));
    qf[hb][17] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kNope + 32 + 8 * g));
  }

  float m_run[NHB], l_part[NHB];
  f32x4 oacc[8][NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    m_run[hb] = -INFINITY;
    l_part[hb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) oacc[mb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  RawSlot cur, nxt;
  if (nch > 0) load_raw(cur, cache, num_slots, idx_row, 16 * w + l16, n, g);

  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nch) load_raw(nxt, cache, num_slots, idx_row, (ch + 1) * kChunk + 16 * w + l16, n, g);

    // ---- dequantise, stage V, S^T = K Q^T
    f32x4 sacc[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __bf16* vrow = &sm.v[buf][16 * w + l16][0];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t sb = ((u < 4 ? cur.sc.x : cur.sc.y) >> (8 * (u & 3))) & 0xFF;
      const float scale = e8m0_as_scale(sb);
      const bf16x8 k0 = dequant8(cur.nope[u].x, cur.nope[u].y, scale);
      const bf16x8 k1 = dequant8(cur.nope[u].z, cur.nope[u].w, scale);
      *reinterpret_cast<bf16x8*>(vrow + 64 * u + 16 * g) = k0;
      *reinterpret_cast<bf16x8*>(vrow + 64 * u + 16 * g + 8) = k1;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        sacc[hb] = mfma16(k0, qf[hb][2 * u], sacc[hb]);
        sacc[hb] = mfma16(k1, qf[hb][2 * u + 1], sacc[hb]);
      }
    }
    {
      const bf16x8 k16 = as_bf16x8(cur.rope[0]);
      const bf16x8 k17 = as_bf16x8(cur.rope[1]);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        sacc[hb] = mfma16(k16, qf[hb][16], sacc[hb]);
        sacc[hb] = mfma16(k17, qf[hb][17], sacc[hb]);
      }
    }

    // ---- online softmax (log2 domain). sacc[hb][i] = score of row 4g+i, head l16.
    const uint64_t vmask = __ballot(cur.valid);  // bit j (j < 16) = row j of this wave valid
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
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) sm.red[buf][w][16 * hb + l16] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float cm = sm.red[buf][0][16 * hb + l16];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) cm = fmaxf(cm, sm.red[buf][ww][16 * hb + l16]);
      const float mn = fmaxf(m_run[hb], cm);
      const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[hb] - mn);
      float p[4], sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (s[hb][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[hb][i] - mn);
        sum += p[i];
      }
      l_part[hb] = l_part[hb] * alpha + sum;
      m_run[hb] = mn;
      *reinterpret_cast<uint2*>(&sm.p[buf][16 * hb + l16][16 * w + 4 * g]) =
          make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) oacc[mb][hb] *= alpha;
    }
    __syncthreads();

    // ---- O^T[c][h] += V^T[c][j] P^T[j][h] for c in 128w..128w+127
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pf[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        pf[hb] = *reinterpret_cast<const bf16x8*>(&sm.p[buf][16 * hb + l16][32 * ks + 8 * g]);
      const __bf16* vbase = &sm.v[buf][32 * ks + 8 * g + (l16 >> 2)][128 * w + 4 * (l16 & 3)];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const bf16x4 t0 = lds_read_tr16(vbase + 16 * mb);
        const bf16x4 t1 = lds_read_tr16(vbase + 16 * mb + 4 * kVStride);
        bf16x8 vf;
        vf[0] = t0[0]; vf[1] = t0[1]; vf[2] = t0[2]; vf[3] = t0[3];
        vf[4] = t1[0]; vf[5] = t1[1]; vf[6] = t1[2]; vf[7] = t1[3];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) oacc[mb][hb] = mfma16(vf, pf[hb], oacc[mb][hb]);
      }
    }
    if (ch + 1 < nch) cur = nxt;
  }

  // ---- finalise: sum the waves' partial denominators, add the sink, normalise
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float lp = l_part[hb];
    lp += __shfl_xor(lp, 16);
    lp += __shfl_xor(lp, 32);
    if (g == 0) sm.lsum[w][16 * hb + l16] = lp;
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int h = h0 + 16 * hb + l16;
    const float lt = sm.lsum[0][16 * hb + l16] + sm.lsum[1][16 * hb + l16] +
                     sm.lsum[2][16 * hb + l16] + sm.lsum[3][16 * hb + l16];
    const float mr = m_run[hb];
    const float z2 = sinks ? sinks[h] * kLog2e : -INFINITY;
    const float M = fmaxf(mr, z2);
    const float f = (mr == -INFINITY) ? 0.f : exp2f(mr - M);
    const float den = lt * f + ((z2 == -INFINITY) ? 0.f : exp2f(z2 - M));
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow = out + ((int64_t)t * H + h) * kNope + 128 * w + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const f32x4 o = oacc[mb][hb];
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
