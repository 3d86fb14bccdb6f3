// The indexer's top-k selection, the step before index combining (PR #40860: the MLA
// layer integrates an Indexer whose top-k picks feed the sparse backend; PR #43385: the
// picks are compressed-entry ids below (pos+1) / COMPRESS_RATIO).  Per token at
// position pos the candidates are ids 0..n-1, n = min((pos+1) / ratio, logits_stride);
// the result is the min(n, top_k) ids with the largest logits, ties to the smaller id
// (a NaN logit counts as -inf), listed in ascending id order, -1 after them.
//
// One workgroup per token: 16 waves when there are few tokens, 4 waves (three
// workgroups per CU) when there are many.  Logits map to order-preserving 32-bit keys,
// staged in LDS by the first pass for rows of up to 32 keys per thread (32768 or 8192
// candidates; longer rows are read again by every pass); a radix select
// (digits of 11, 11 and 10 bits, most significant first, 2048-bin histograms in LDS:
// wide enough that similar logits rarely collide on one bin) finds the k-th largest
// key K and how many keys equal to K are taken (m); one ordered pass then emits every
// id with key > K and the first m ids with key == K.  Each thread owns 8 consecutive
// candidates per round, so a scan of per-wave counts (gt and eq packed into one 32-bit
// value) gives every thread its output position.  When few keys share K's first two
// digits, the third pass already counts the rest per wave and lists those few, and the
// emission needs no counting sweep.  Integer decisions on fp32 keys only: bit-exact
// with the oracle's fp32 comparisons.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

constexpr int kSelItems = 8;
// rows of up to 4 rounds of 8 keys per thread (32 NT candidates: 32768 with 1024 threads,
// 8192 with 256) keep their keys in LDS
template <int NT>
constexpr int stage_max() { return 4 * NT * 8; }
constexpr int kBins = 2048;       // radix digits of 11, 11 and 10 bits
constexpr int kListMax = 512;     // staged rows: keys sharing K's first two digits listed up to this many

// Larger key <=> larger logit; -0 and +0 share a key (they compare equal), NaN takes the
// key of -inf.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (v != v) u = 0xFF800000u;
  if (v == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over the 64 lanes of a wave, in DPP moves (no LDS round trip): shifts
// by 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside the row
// add 0), then row 0's total into row 1 and row 2's into row 3 (broadcast of lane 15 of
// each row to the next, rows 1 and 3 only), then lane 31's running total into rows 2
// and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Inclusive scan over the block of NT threads; `wsum` holds one int per wave.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int x, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_inclusive_scan(x);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) add += i < w ? wsum[i] : 0;
  __syncthreads();  // wsum may be reused by the next scan
  return x + add;
}

template <int NT, bool STAGE>
struct SelSmem {
  alignas(16) uint32_t keys[STAGE ? stage_max<NT>() : 1];
  uint32_t hist[kBins];
  int wsum[NT / 64];
  int wtab[NT / 64 * 4];   // compaction: (gt, eq) count of wave w in round r at 4w + r ...
  int wbase[NT / 64 * 4];  // ... and of everything before it in emission order
  uint32_t sh_digit, sh_above;
  uint32_t lkey[STAGE ? kListMax : 1];  // staged rows: the keys sharing K's first two digits
  int lidx[STAGE ? kListMax : 1];       // ... and their indices
  int lcount;
};

// One histogram pass that reads the keys from memory (rows that are not staged): ITEMS
// keys per thread are requested before any is used, at clamped indices (a load under a
// per-lane condition is waited for on the spot); entries past n are ignored.
template <int ITEMS, int NT, bool STAGE, typename KeyAt>
__device__ __forceinline__ void hist_from_memory(SelSmem<NT, STAGE>& sm, int n, int tid,
                                                 uint32_t mask, uint32_t prefix, int shift,
                                                 uint32_t dmask, KeyAt key_at) {
  for (int j0 = 0; j0 < n; j0 += NT * ITEMS) {
    uint32_t v[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) v[u] = key_at(min(j0 + u * NT + tid, n - 1));
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int j = j0 + u * NT + tid;
      if (j < n && (v[u] & mask) == prefix) atomicAdd(&sm.hist[(v[u] >> shift) & dmask], 1u);
    }
  }
}

// The first pass of a staged row: every key into LDS and its first digit into the
// histogram.  The row is read as a raw buffer of n floats whose whole offset is the
// range-checked vector offset, so a load past the row's end returns 0 and reads nothing
// (no index clamping, one offset register per load); eight loads per thread in flight
// (measured: 8 beat 4, 16 and 32 a round).
template <int NT>
__device__ __forceinline__ void stage_row(SelSmem<NT, true>& sm, const float* row, int n,
                                          int tid) {
  // the row address and n are the same in every lane; said so, the buffer resource is
  // built in scalar registers
  const uint64_t ra = reinterpret_cast<uint64_t>(row);
  const uint64_t ua =
      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ra >> 32)) << 32) |
      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ra);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<float*>(ua), (short)0, __builtin_amdgcn_readfirstlane(n) * 4, 0x00020000);
#pragma unroll 1
  for (int j0 = 0; j0 < n; j0 += NT * kSelItems) {
    float x[kSelItems];
#pragma unroll
    for (int u = 0; u < kSelItems; ++u)
      x[u] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, (j0 + u * NT + tid) * 4, 0, 0));
#pragma unroll
    for (int u = 0; u < kSelItems; ++u) {
      const int j = j0 + u * NT + tid;
      if (j < n) {
        const uint32_t v = order_key(x[u]);
        sm.keys[j] = v;
        atomicAdd(&sm.hist[v >> 21], 1u);
      }
    }
  }
}

// The k largest of n keys (0 < k < n) of `row`, ties to the smaller index j: a radix
// select of the k-th largest key K (digits of 11, 11 and 10 bits, most significant first)
// and how many keys equal to K are taken (m), then one ordered pass that calls
// emit(p, j) for every j with key > K and the first m with key == K, p = the pick's rank
// in ascending j.  With STAGE and n <= stage_max<NT>() the first pass keeps the keys in LDS
// for the other passes; otherwise every pass reads the row again.  NT threads, all of
// which must call; barriers inside.
template <int NT, bool STAGE, typename Emit>
__device__ __forceinline__ void radix_select(SelSmem<NT, STAGE>& sm,
                                             const float* __restrict__ row, int n, int k,
                                             Emit emit) {
  static_assert(kSelItems == 8 && NT <= 1024,
                "a staged row is at most 4 rounds of 8 keys per thread; the emission table "
                "(4 rounds x NT / 64 waves) is scanned by one wave");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool staged = STAGE && n <= stage_max<NT>();
  auto key_at = [&](int j) { return order_key(row[j]); };
  // staged rows are read in rounds of 8 consecutive keys per thread (keys
  // r * 8 NT + 8 tid ..+7 in round r), the emission's order; a thread's 8 keys as two
  // 16 B reads (8 single reads of one thread's consecutive keys put 64 lanes on 8
  // banks); entries past n hold stale keys and are masked
  const int rounds = (n + NT * kSelItems - 1) / (NT * kSelItems);
  auto keys8 = [&](int first, uint32_t (&key)[kSelItems]) {
    const uint4 a = *reinterpret_cast<const uint4*>(&sm.keys[first]);
    const uint4 b = *reinterpret_cast<const uint4*>(&sm.keys[first + 4]);
    key[0] = a.x; key[1] = a.y; key[2] = a.z; key[3] = a.w;
    key[4] = b.x; key[5] = b.y; key[6] = b.z; key[7] = b.w;
  };
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
  // List mode (staged rows where at most kListMax keys share K's first two digits, known
  // from the second histogram): the third pass also counts, per emission group (round,
  // wave), the keys whose first two digits beat K's (all larger than K) and lists the
  // keys that share them; the emission's counts then come from that list.
  bool use_list = false;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    for (int d = tid; d < kBins; d += NT) sm.hist[d] = 0;
    if (STAGE && tid == 0) sm.lcount = 0;
    __syncthreads();
    if (!staged) {
      hist_from_memory<kSelItems>(sm, n, tid, mask, prefix, shift, dmask, key_at);
    } else if constexpr (STAGE) {
      if (pass == 0) {
        stage_row<NT>(sm, row, n, tid);
      } else if (pass == 2 && use_list) {
        const uint32_t top = prefix >> 10;  // K's first two digits
#pragma unroll 1
        for (int r = 0; r < rounds; ++r) {
          const int first = r * NT * kSelItems + tid * kSelItems;
          uint32_t key[kSelItems];
          keys8(first, key);
          int ca = 0;
#pragma unroll
          for (int i = 0; i < kSelItems; ++i) {
            const bool valid = first + i < n;
            ca += (valid && (key[i] >> 10) > top) ? 1 : 0;
            if (valid && (key[i] >> 10) == top) {
              atomicAdd(&sm.hist[key[i] & 1023u], 1u);
              const int pos = atomicAdd(&sm.lcount, 1);
              if (pos < kListMax) {
                sm.lkey[pos] = key[i];
                sm.lidx[pos] = first + i;
              }
            }
          }
          const int incl = wave_inclusive_scan(ca);
          if (lane == 63) sm.wtab[4 * w + r] = incl;  // the group's (gt, eq) so far: eq 0
        }
      } else {
#pragma unroll 1
        for (int r = 0; r < rounds; ++r) {
          const int first = r * NT * kSelItems + tid * kSelItems;
          uint32_t key[kSelItems];
          keys8(first, key);
#pragma unroll
          for (int i = 0; i < kSelItems; ++i)
            if (first + i < n && (key[i] & mask) == prefix)
              atomicAdd(&sm.hist[(key[i] >> shift) & dmask], 1u);
        }
      }
    }
    __syncthreads();
    // thread i owns the kBins/NT digits below dmask - (kBins/NT)*i (from the top); after
    // the scan of its counts it knows how many matching keys have a larger digit than
    // each of them, and the one whose range covers `remaining` is the digit
    constexpr int kPer = kBins / NT;
    int cnt[kPer];
    int sum = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int d = (int)dmask - kPer * tid - r;
      cnt[r] = d >= 0 ? (int)sm.hist[d] : 0;
      sum += cnt[r];
    }
    const int incl = block_inclusive_scan<NT>(sum, sm.wsum);
    int above = incl - sum;  // keys with a digit larger than this thread's first
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int d = (int)dmask - kPer * tid - r;
      if (d >= 0 && above < remaining && above + cnt[r] >= remaining) {
        sm.sh_digit = (uint32_t)d;
        sm.sh_above = (uint32_t)above;
      }
      above += cnt[r];
    }
    __syncthreads();
    if (staged && pass == 1)  // how many keys share the first two digits of K
      use_list = (int)sm.hist[sm.sh_digit] <= kListMax;
    prefix |= sm.sh_digit << shift;
    mask |= dmask << shift;
    remaining -= (int)sm.sh_above;
    __syncthreads();  // sh_digit / sh_above / hist are rewritten next pass
  }
  const uint32_t K = prefix;
  const int m = remaining;  // keys equal to K that are taken, the smallest indices first
  if constexpr (STAGE) {
    if (staged) {
      // The ordered emission with the keys in LDS: every round's (gt, eq) counts per wave
      // first, one wave's scan of them in emission order (rounds outer, waves inner),
      // then the emission, each thread recounting its 8 keys.
      if (use_list) {
        // the listed keys that are picks join their groups' counts
        const int nl = sm.lcount;
        for (int i = tid; i < nl; i += NT) {
          const uint32_t v = sm.lkey[i];
          const int j = sm.lidx[i];
          const int r = j / (NT * kSelItems), ww = (j % (NT * kSelItems)) / (64 * kSelItems);
          if (v > K) atomicAdd(&sm.wtab[4 * ww + r], 1);
          else if (v == K) atomicAdd(&sm.wtab[4 * ww + r], 1 << 16);
        }
      } else {
#pragma unroll 1
        for (int r = 0; r < rounds; ++r) {
          const int first = r * NT * kSelItems + tid * kSelItems;
          uint32_t key[kSelItems];
          keys8(first, key);
          int cgt = 0, ceq = 0;
#pragma unroll
          for (int i = 0; i < kSelItems; ++i) {
            cgt += (first + i < n && key[i] > K) ? 1 : 0;
            ceq += (first + i < n && key[i] == K) ? 1 : 0;
          }
          // at most NT * kSelItems of each per round
          const int incl = wave_inclusive_scan(cgt | (ceq << 16));
          if (lane == 63) sm.wtab[4 * w + r] = incl;
        }
      }
      __syncthreads();
      if (tid < 64) {  // lane r * (NT / 64) + w: entry (r, w) of the emission order
        const int r = tid / (NT / 64), ww = tid % (NT / 64);
        const bool entry = r < 4;  // 4 rounds x NT / 64 waves: all 64 lanes at NT = 1024
        const int v = entry && r < rounds ? sm.wtab[4 * ww + r] : 0;
        const int e = wave_inclusive_scan(v) - v;  // totals stay below 2^16 each
        if (entry) sm.wbase[4 * ww + r] = e;
      }
      __syncthreads();
#pragma unroll 1
      for (int r = 0; r < rounds; ++r) {
        const int first = r * NT * kSelItems + tid * kSelItems;
        uint32_t key[kSelItems];
        keys8(first, key);
        uint32_t gtm = 0, eqm = 0;  // bit i: key first + i is above K / equal to K
#pragma unroll
        for (int i = 0; i < kSelItems; ++i) {
          const bool valid = first + i < n;
          gtm |= (valid && key[i] > K) ? 1u << i : 0u;
          eqm |= (valid && key[i] == K) ? 1u << i : 0u;
        }
        const int packed = __popc(gtm) | (__popc(eqm) << 16);
        const int excl = sm.wbase[4 * w + r] + wave_inclusive_scan(packed) - packed;
        const int gt_before = excl & 0xFFFF, eq_before = excl >> 16;
        // the thread's equal keys that are still wanted: the first m - eq_before of them
        const int want = m - eq_before;
        uint32_t pm = gtm;
        int seen = 0;
#pragma unroll
        for (int i = 0; i < kSelItems; ++i) {
          const bool e = (eqm >> i) & 1u;
          pm |= (e && seen < want) ? 1u << i : 0u;
          seen += e ? 1 : 0;
        }
        int p = gt_before + min(eq_before, m);
        while (pm) {  // the thread's picks in ascending index
          const int i = __builtin_ctz(pm);
          pm &= pm - 1u;
          emit(p++, first + i);
        }
      }
      return;
    }
  }
  int gt_run = 0, eq_run = 0;
  for (int c0 = 0; c0 < n; c0 += NT * kSelItems) {
    const int first = c0 + tid * kSelItems;
    uint32_t key[kSelItems];
    int cgt = 0, ceq = 0;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) key[j] = key_at(min(first + j, n - 1));
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
      cgt += (first + j < n && key[j] > K) ? 1 : 0;
      ceq += (first + j < n && key[j] == K) ? 1 : 0;
    }
    // at most 8192 of each per pass: pack (gt, eq) into one scan
    const int packed = cgt | (ceq << 16);
    const int incl = block_inclusive_scan<NT>(packed, sm.wsum);
    const int excl = incl - packed;
    const int gt_before = gt_run + (excl & 0xFFFF);
    const int eq_before = eq_run + (excl >> 16);
    int p = gt_before + min(eq_before, m);
    int eq_rank = eq_before;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
      if (first + j >= n) break;
      if (key[j] > K) {
        emit(p++, first + j);
      } else if (key[j] == K) {
        if (eq_rank < m) emit(p++, first + j);
        ++eq_rank;
      }
    }
    // block totals of this pass: the last thread's inclusive value
    if (tid == NT - 1) sm.wsum[0] = incl;
    __syncthreads();
    const int tot = sm.wsum[0];
    gt_run += tot & 0xFFFF;
    eq_run += tot >> 16;
    __syncthreads();
  }
}

// Token i of request b: its position and candidate count (the causal bound).
struct IdxTok {
  int64_t t;
  int n;
  int k;
};

__device__ __forceinline__ IdxTok indexer_token(const int32_t* __restrict__ qsl,
                                                const int32_t* __restrict__ seq_lens, int b,
                                                int i, int logits_stride, int ratio, int top_k) {
  const int base = qsl[0];
  const int q0 = qsl[b] - base;
  const int qlen = qsl[b + 1] - qsl[b];
  const int64_t pos = (int64_t)seq_lens[b] - qlen + i;
  const int64_t n64 = pos + 1 > 0 ? (pos + 1) / ratio : 0;
  IdxTok r;
  r.t = (int64_t)q0 + i;
  r.n = (int)min(n64, (int64_t)logits_stride);
  r.k = min(r.n, top_k);
  return r;
}

// NT threads per token; STAGE keeps the keys of rows up to 32 NT candidates in LDS
// (longer rows: every pass rereads the row from the caches).
template <int NT, bool STAGE>
__global__ void __launch_bounds__(NT) indexer_topk_kernel(
    const float* __restrict__ logits, int logits_stride, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ seq_lens, int T, int ratio, int top_k, int32_t* __restrict__ topk,
    int topk_stride, int32_t* __restrict__ topk_lens) {
  __shared__ SelSmem<NT, STAGE> sm;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int qlen = qsl[b + 1] - qsl[b];
  for (int i = blockIdx.y; i < qlen; i += gridDim.y) {
    const IdxTok tk = indexer_token(qsl, seq_lens, b, i, logits_stride, ratio, top_k);
    if (tk.t < 0 || tk.t >= T) continue;
    const int n = tk.n, k = tk.k;
    const float* row = logits + tk.t * (int64_t)logits_stride;
    int32_t* out = topk + tk.t * (int64_t)topk_stride;
    if (k == n) {
      for (int j = tid; j < n; j += NT) out[j] = j;
    } else if (k > 0) {
      radix_select<NT, STAGE>(sm, row, n, k, [&](int p, int j) { out[p] = j; });
    }
    for (int j = k + tid; j < topk_stride; j += NT) out[j] = -1;
    if (tid == 0) topk_lens[tk.t] = k;
    if (i + (int)gridDim.y < qlen) __syncthreads();  // LDS reuse by this workgroup's next token
  }
}

hipError_t launch_indexer_topk(const float* logits, int logits_stride, const int32_t* qsl,
                               const int32_t* seq_lens, int B, int T, int ratio, int top_k,
                               int32_t* topk, int topk_stride, int32_t* topk_lens,
                               hipStream_t stream) {
  if (B == 0 || T == 0) return hipSuccess;
  int per_req = (T + B - 1) / B;
  int Y = per_req < 1 ? 1 : (per_req > 4096 ? 4096 : per_req);
  // few tokens: one 16-wave workgroup per token, rows of up to 32768 candidates in LDS
  // (128 KB); many tokens: 4-wave workgroups, rows of up to 8192 in LDS (32 KB), three
  // workgroups per CU
  if (T < 1024)
    hipLaunchKernelGGL((indexer_topk_kernel<1024, true>), dim3(B, Y), dim3(1024), 0, stream,
                       logits, logits_stride, qsl, seq_lens, T, ratio, top_k, topk, topk_stride,
                       topk_lens);
  else
    hipLaunchKernelGGL((indexer_topk_kernel<256, true>), dim3(B, Y), dim3(256), 0, stream,
                       logits, logits_stride, qsl, seq_lens, T, ratio, top_k, topk, topk_stride,
                       topk_lens);
  return hipGetLastError();
}

}  // namespace dsv4
