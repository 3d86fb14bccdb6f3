// Helpers of the gfx950 sparse MLA attention kernel (attention.hip): the LDS layout, the
// gather of a chunk's records, the FP8 dequantisation into MFMA fragments and the value
// tile, the online-softmax pieces, the P.V fragments, and the combine step built into a
// workgroup's prologue (written for any thread count and any LDS layout with an index
// block and request fields).  See attention.hip for the arithmetic they implement and
// the pages it follows.
#pragma once
#include "device.hpp"
#include "insert_rows.hpp"
#include "launch.hpp"

namespace dsv4 {

constexpr int kChunk = 64;
constexpr int kVStride = 512;  // bf16 per LDS value row (1024 B, 16 B units XOR-swizzled)
constexpr int kPStride = 72;   // bf16 per LDS probability row: 144 B
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
  int req[4];  // fused combine: request of the token, its first token, its query count, its length
};

// Inputs of the combine step when the decode builds its index rows itself (the
// arguments of dsv4_combine_indices; the page geometry comes with the cache).
struct TopkIn {
  const int32_t* topk;
  int topk_stride;
  int topk_width;
  const int32_t* topk_lens;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int bt_stride;
  int B;
  int top_k;
  int window;
};

// Inputs of the insert step when the decode performs it too (the arguments of
// dsv4_kv_insert): q is normalised in place and the new latent rows go into the cache,
// which the decode then reads through `cache`.
struct StepIn {
  uint16_t* q;
  const uint16_t* kv;
  const int64_t* positions;
  const int64_t* slot_mapping;
  const float* cos_sin;
  int max_pos;
  const uint16_t* weight;
  float eps;
  uint8_t* cache;
  float kv_scale;  // the fp8 cache's per-tensor scale (other dtypes: unused)
};

// Source of the (all-zero) record read for an invalid or absent slot, so that every
// lane issues the same loads every chunk: branch-free loads let the compiler wait for
// exactly the chunk it is about to use while later chunks stay in flight.
static __device__ __attribute__((aligned(64))) uint8_t g_zero_page[kMaxPage * kRecord];

// The cache as the kernels see it: base pointer, number of slots, log2 of the page size.
struct CacheRef {
  const uint8_t* base;
  int64_t num_slots;
  int ps;
};

template <int KV>
constexpr int kv_record_bytes() {
  return kv_record_bytes_of(KV);
}

// One lane's share of a slot's record (row l16 of its wave's 16, k-group g): the dims
// 64u + 16g .. +15 (u = 0..7) and the rope dims 8g..8g+7, 32+8g..32+8g+7, the pieces the
// MFMA fragments of the QK product take.
template <int KV>
struct RawT;
template <>
struct RawT<kKvFp8Ds> {
  uint4 nope[8];  // 128 codes: dims 64u + 16g .. 64u + 16g + 15 for u = 0..7
  uint4 rope[2];  // rope dims 8g..8g+7 and 32+8g..32+8g+7 (bf16)
  uint2 sc;       // the slot's 8 scale bytes
  int valid;
};
template <>
struct RawT<kKvBf16> {
  uint4 nope[16];  // dims 64u + 16g .. +7 in nope[2u], +8 .. +15 in nope[2u + 1] (bf16)
  uint4 rope[2];   // rope dims 8g..8g+7 and 32+8g..32+8g+7 (bf16)
  int valid;
};
template <>
struct RawT<kKvFp8E4m3> {
  uint4 nope[8];  // 128 codes: dims 64u + 16g .. 64u + 16g + 15 for u = 0..7
  uint2 rope[2];  // codes of rope dims 8g..8g+7 and 32+8g..32+8g+7
  int valid;
};
using RawSlot = RawT<kKvFp8Ds>;

// Where this lane's pieces of a slot's record live (the zero page for an invalid slot).
struct RecPtr {
  const uint8_t* np;  // value dims 16g.. of the record (u = 0 piece)
  const uint8_t* rp;  // rope dims 8g.. of the record
  const uint8_t* sp;  // scale bytes (packed record only)
  int valid;
};
template <int KV = kKvFp8Ds>
__device__ __forceinline__ RecPtr rec_ptr(const CacheRef& c, int64_t slot, int g) {
  RecPtr p;
  p.valid = (slot >= 0 && slot < c.num_slots) ? 1 : 0;
  if constexpr (KV == kKvFp8Ds) {
    const uint8_t* base = p.valid ? c.base + page_base(slot >> c.ps, c.ps) : g_zero_page;
    const int off = p.valid ? (int)(slot & ((1 << c.ps) - 1)) : 0;
    p.np = base + nope_off(off) + 16 * g;
    p.rp = base + rope_off(off, c.ps) + 16 * g;
    p.sp = base + scale_off(off, c.ps);
  } else {
    const uint8_t* base = p.valid ? c.base + slot * kv_record_bytes<KV>() : g_zero_page;
    constexpr int esz = KV == kKvBf16 ? 2 : 1;  // bytes per value
    p.np = base + esz * 16 * g;
    p.rp = base + esz * (kNope + 8 * g);
    p.sp = base;
  }
  return p;
}

// Loads of piece u of the value dims, and of the rope dims (and scales), from p.
template <int KV>
__device__ __forceinline__ void load_nope_piece(RawT<KV>& r, const RecPtr& p, int u) {
  if constexpr (KV == kKvBf16) {
    r.nope[2 * u] = *reinterpret_cast<const uint4*>(p.np + 128 * u);
    r.nope[2 * u + 1] = *reinterpret_cast<const uint4*>(p.np + 128 * u + 16);
  } else {
    r.nope[u] = *reinterpret_cast<const uint4*>(p.np + 64 * u);
  }
}
template <int KV>
__device__ __forceinline__ void load_rope_piece(RawT<KV>& r, const RecPtr& p) {
  if constexpr (KV == kKvFp8E4m3) {
    r.rope[0] = *reinterpret_cast<const uint2*>(p.rp);
    r.rope[1] = *reinterpret_cast<const uint2*>(p.rp + 32);
  } else {
    r.rope[0] = *reinterpret_cast<const uint4*>(p.rp);
    r.rope[1] = *reinterpret_cast<const uint4*>(p.rp + 64);
  }
  if constexpr (KV == kKvFp8Ds) r.sc = *reinterpret_cast<const uint2*>(p.sp);
  r.valid = p.valid;
}

template <int KV>
__device__ __forceinline__ void load_raw(RawT<KV>& r, const CacheRef& c, int64_t slot, int g) {
  if constexpr (KV == kKvFp8Ds) {
    r.valid = (slot >= 0 && slot < c.num_slots) ? 1 : 0;
    const uint8_t* base = r.valid ? c.base + page_base(slot >> c.ps, c.ps) : g_zero_page;
    const int off = r.valid ? (int)(slot & ((1 << c.ps) - 1)) : 0;
    const uint8_t* np = base + nope_off(off) + 16 * g;
#pragma unroll
    for (int u = 0; u < 8; ++u) r.nope[u] = *reinterpret_cast<const uint4*>(np + 64 * u);
    const uint8_t* rp = base + rope_off(off, c.ps) + 16 * g;
    r.rope[0] = *reinterpret_cast<const uint4*>(rp);
    r.rope[1] = *reinterpret_cast<const uint4*>(rp + 64);
    r.sc = *reinterpret_cast<const uint2*>(base + scale_off(off, c.ps));
  } else {
    const RecPtr p = rec_ptr<KV>(c, slot, g);
#pragma unroll
    for (int u = 0; u < 8; ++u) load_nope_piece<KV>(r, p, u);
    load_rope_piece<KV>(r, p);
  }
}
__device__ __forceinline__ void load_raw_slot(RawSlot& r, const CacheRef& c, int64_t slot, int g) {
  load_raw<kKvFp8Ds>(r, c, slot, g);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// The bf16 K fragments of piece u (dims 64u + 16g .. +7 and +8 .. +15) and of the rope
// dims.  The packed record's codes are scaled by their block's 2^(byte-127) in the
// conversion (exact); the per-tensor fp8 codes convert unscaled (exact: E4M3 values are
// bf16 values) and the scale is applied to the scores and the output instead.
template <int KV>
__device__ __forceinline__ void k_frags(const RawT<KV>& r, int u, bf16x8& k0, bf16x8& k1) {
  if constexpr (KV == kKvBf16) {
    k0 = as_bf16x8(r.nope[2 * u]);
    k1 = as_bf16x8(r.nope[2 * u + 1]);
  } else {
    float scale = 1.0f;
    if constexpr (KV == kKvFp8Ds)
      scale = e8m0_as_scale(((u < 4 ? r.sc.x : r.sc.y) >> (8 * (u & 3))) & 0xFF);
    k0 = dequant8(r.nope[u].x, r.nope[u].y, scale);
    k1 = dequant8(r.nope[u].z, r.nope[u].w, scale);
  }
}
template <int KV>
__device__ __forceinline__ void k_frags_rope(const RawT<KV>& r, bf16x8& k16, bf16x8& k17) {
  if constexpr (KV == kKvFp8E4m3) {
    k16 = dequant8(r.rope[0].x, r.rope[0].y, 1.0f);
    k17 = dequant8(r.rope[1].x, r.rope[1].y, 1.0f);
  } else {
    k16 = as_bf16x8(r.rope[0]);
    k17 = as_bf16x8(r.rope[1]);
  }
}

// Entry jj of the staged index block (-1 past its end).  The read is unconditional (at a
// clamped index) and the value selected afterwards, so no branch surrounds it.
__device__ __forceinline__ int64_t idx_at(const int32_t* idx_lds, int jj, int n_blk) {
  const int32_t v = idx_lds[min(jj, kIdxBlock - 1)];
  return jj < n_blk ? (int64_t)v : -1;
}

// Entries [0, n_win) of an index block, this thread's share, all requested before the
// first wait (one memory latency per block instead of one per NT entries); then written
// into LDS.  In two parts so that other loads can be issued in between.  NT = threads of
// the workgroup.
template <int NT = 256>
__device__ __forceinline__ void stage_idx_load(int32_t (&v)[kIdxBlock / NT],
                                               const int32_t* __restrict__ src, int n_win,
                                               int tid) {
#pragma unroll
  for (int k = 0; k < kIdxBlock / NT; ++k)
    if (NT * k < n_win) v[k] = src[min(tid + NT * k, n_win - 1)];
}
template <int NT = 256>
__device__ __forceinline__ void stage_idx_store(int32_t* dst, const int32_t (&v)[kIdxBlock / NT],
                                                int n_win, int tid) {
#pragma unroll
  for (int k = 0; k < kIdxBlock / NT; ++k)
    if (tid + NT * k < n_win) dst[tid + NT * k] = v[k];
}
constexpr int kStagePer = kIdxBlock / 256;

// A vector (not scalar) load of a value at a uniform address: its wait is then ordered
// with the vector loads around it instead of joining every LDS wait (lgkmcnt).
template <class T>
__device__ __forceinline__ T vload(const T* p) {
  uint64_t a = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+v"(a));
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(a);
}

typedef __attribute__((address_space(3))) void lds_void;

// Entries [0, n) of a row into LDS at `dst`, memory to LDS without registers: wave w
// copies entries 256u + 64w .. +63 with one 4-byte load per lane (lanes past n copy
// entry n - 1 into slots up to the next multiple of 64, never read).  Complete after
// s_waitcnt vmcnt(0) and a barrier.
__device__ __forceinline__ void copy_row_to_lds(int32_t* dst, const int32_t* __restrict__ src,
                                                int n, int w, int lane) {
  for (int e0 = 64 * w; e0 < n; e0 += 256) {
    const int e = min(e0 + lane, n - 1);
    __builtin_amdgcn_global_load_lds((const void*)(src + e), (lds_void*)(dst + e0), 4, 0, 0);
  }
}

// The combine step for token t, written straight into the LDS index block (the rules of
// combine_kernel: valid top-k entries outside the window, then the window ascending, each
// mapped through the request's block table; -1 for the rest).  Every load is
// unconditional at a clamped, in-bounds address (only uniform conditions skip one) and
// its value is selected afterwards: a load under a per-lane condition is waited for on
// the spot, which would serialise them.  Vector loads complete in order, so the parts
// are issued by their caller in the order their values are needed:
//   combine_search_load  the request search's loads (thread r tests request r), first;
//   combine_topk_load    the top-k row (and whatever else the caller requests after it);
//   combine_find         waits for the search loads only, records the token's request
//                        in sm.req (two barriers);
//   combine_stage_bt     copies the request's block-table entries for logical pages
//                        0 .. pos >> ps into LDS (memory to LDS, no registers; at most
//                        kBtStage entries, else the lookups below go to memory): one
//                        contiguous row instead of a scattered lookup per entry;
//   combine_rows         after s_waitcnt vmcnt(0) and a barrier, builds the row into
//                        sm.idx and returns its length tk + sw (0 for a token of no
//                        request), the same in every thread.
constexpr int kCombPer = kIdxBlock / 256;
constexpr int kBtStage = 16384;  // block-table entries staged in LDS (64 KB)

struct CombSearch {
  int32_t base, lo, hi, len;  // qsl[0], and qsl[r], qsl[r+1], seq_lens[r] of request r
};

template <int NT = 256>
__device__ __forceinline__ CombSearch combine_search_load(const TopkIn& c, int tid) {
  CombSearch cs{0, 0, 0, 0};
  if (c.B > 0) {
    const int r = min(tid, c.B - 1);
    cs.base = vload(c.qsl);
    cs.lo = c.qsl[r];
    cs.hi = c.qsl[r + 1];
    cs.len = c.seq_lens[r];
  }
  return cs;
}

template <int NT = 256>
__device__ __forceinline__ void combine_topk_load(const TopkIn& c, int64_t t, int tid,
                                                  int32_t (&xv)[kIdxBlock / NT], int& tl) {
  constexpr int kPer = kIdxBlock / NT;
  const int kmax = min(c.top_k, c.topk_width);
  const int32_t* trow = c.topk + t * c.topk_stride;
  // Every load unconditional and none of the values touched here: entries j >= kmax
  // (clamped reads of entry kmax - 1, or of a zero word when the row is empty) are
  // ignored by combine_rows.  A branch around the loads would let the compiler convert
  // the values inside it, with a wait for each load.
  const int32_t* src = kmax > 0 ? trow : reinterpret_cast<const int32_t*>(g_zero_page);
  const int last = max(kmax - 1, 0);
#pragma unroll
  for (int u = 0; u < kPer; ++u) xv[u] = src[min(tid + NT * u, last)];
  tl = c.topk_lens ? vload(c.topk_lens + t) : c.top_k;
}

template <int NT = 256, class SM>
__device__ __forceinline__ void combine_find(SM& sm, const TopkIn& c, int64_t t, int tid,
                                             const CombSearch& cs) {
  if (tid == 0) sm.req[0] = -1;
  __syncthreads();
  // thread r tests request r and brings its length along, so the token's position is
  // known right after the first loads
  auto test = [&](int r, int lo, int hi, int L) {
    if (t >= lo && t < hi) {  // at most one request holds the token
      sm.req[0] = r;
      sm.req[1] = lo;
      sm.req[2] = hi - lo;
      sm.req[3] = L;
    }
  };
  if (tid < c.B) test(tid, cs.lo - cs.base, cs.hi - cs.base, cs.len);
  for (int r = tid + NT; r < c.B; r += NT)  // batches of more than NT requests
    test(r, c.qsl[r] - cs.base, c.qsl[r + 1] - cs.base, c.seq_lens[r]);
  __syncthreads();
}

// Returns whether the entries were staged (the same in every thread).
template <class SM>
__device__ __forceinline__ bool combine_stage_bt(SM& sm, const TopkIn& c, int64_t t, int ps,
                                                 int32_t* bt_lds, int w, int lane) {
  const int b = sm.req[0];
  if (b < 0 || c.bt_stride <= 0) return false;
  const int64_t pos = (int64_t)sm.req[3] - sm.req[2] + (t - sm.req[1]);
  const int64_t np = min((int64_t)c.bt_stride, (max(pos, (int64_t)0) >> ps) + 1);
  if (np > kBtStage) return false;
  copy_row_to_lds(bt_lds, c.block_table + (int64_t)b * c.bt_stride, (int)np, w, lane);
  return true;
}

template <int NT = 256, class SM>
__device__ __forceinline__ int combine_rows(SM& sm, const TopkIn& c, int64_t t, int ps,
                                           int tid, const int32_t (&xv)[kIdxBlock / NT], int tl,
                                           const int32_t* bt_lds, bool staged) {
  constexpr int kPer = kIdxBlock / NT;
  const int kmax = min(c.top_k, c.topk_width);
  const int b = __builtin_amdgcn_readfirstlane(sm.req[0]);
  if (b < 0) return 0;
  const int64_t pos = (int64_t)__builtin_amdgcn_readfirstlane(sm.req[3]) -
                      __builtin_amdgcn_readfirstlane(sm.req[2]) +
                      (t - __builtin_amdgcn_readfirstlane(sm.req[1]));
  int64_t tk = min(pos + 1, (int64_t)c.top_k);
  tk = min(tk, (int64_t)tl);
  tk = max(tk, (int64_t)0);
  const int64_t sw = max(min(pos + 1, (int64_t)c.window), (int64_t)0);
  const int n = (int)(tk + sw);
  if (n <= 0) return 0;
  // n > 0 means pos >= 0, and pos < 2^31 (seq_lens are int32): every position and page
  // below fits in 32 bits
  const int lo = (int)(pos - sw + 1), tk32 = (int)tk;
  const int32_t* bt_row = c.block_table + (int64_t)b * c.bt_stride;
  // staged entries: logical pages 0 .. np - 1 (every valid entry's page lies there)
  const int np = (int)min((int64_t)c.bt_stride, (pos >> ps) + 1);
  // per entry, branch-free: the value of a top-k entry or the window position, then
  // its page from the staged entries (or from memory), all lanes reading
  int32_t xs[kPer], pg[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = tid + NT * u;
    int x = j < kmax ? xv[u] : -1;
    x = (x >= 0 && x < lo) ? x : -1;  // invalid, beyond pos, or in the window
    x = j < tk32 ? x : lo + (j - tk32);
    xs[u] = j < n ? x : -1;
  }
  // the staged entries are read unconditionally (clamped into the staged range) and,
  // when the row was too long to stage, replaced by lookups in memory: an if / else
  // would let the compiler fold both into one generic-address (flat) path
  const int nps = min(np, kBtStage);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int lp = xs[u] >> ps;
    pg[u] = bt_lds[lp < 0 ? 0 : (lp < nps ? lp : nps - 1)];
  }
  if (!staged) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int lp = xs[u] >> ps;
      pg[u] = c.bt_stride > 0 ? bt_row[lp < 0 ? 0 : (lp < c.bt_stride ? lp : c.bt_stride - 1)] : -1;
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = tid + NT * u;
    const int x = xs[u];
    const bool ok = x >= 0 && (x >> ps) < c.bt_stride && pg[u] >= 0;
    if (j < n) sm.idx[j] = ok ? (int32_t)(((int64_t)pg[u] << ps) + (x & ((1 << ps) - 1))) : -1;
  }
  return n;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

// V tile layout: row j of the chunk occupies 1024 B; its 16 B unit k (value dims
// 8k..8k+7) is stored at unit k ^ swz(j), swz(j) = 4*(j & 3) + ((j >> 2) & 3).  The four
// rows that one 16-lane group of a transposing read touches then sit on disjoint banks,
// and the 16 rows of a wave's 16 B row writes are spread over all of them.
__device__ __forceinline__ int v_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
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

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A probability may exceed 1 by up to 2^kPLimit before the reference max must move:
// the reference agreed on after a chunk's barrier applies to the next chunk, and a
// chunk that beats it by more than this is recomputed (fp32/bf16 hold it exactly).
constexpr float kPLimit = 20.0f;
// Starting reference: finite, so that masked scores (-inf) give exp2(-inf) = 0 without a
// test, and below any real score, so the first valid chunk always moves it.
constexpr float kMFloor = -1.0e30f;

template <int NHB>
struct AttnState {
  bf16x8 qf[NHB][18];  // Q^T fragments (registers for the whole kernel)
  float m_run[NHB];    // reference max per head (log2 domain), same in every wave
  float l_part[NHB];   // this lane's share of the softmax denominator
  // O^T, per wave 128 of the 512 output dims:
  //   NHB == 1: o16[mb] = dims 128w + 16mb + 4g + i, head l16 (16x16 MFMA layout)
  //   NHB == 2: o32[mb] = dims 128mb + 32w + 8(r/4) + 4(lane/32) + r%4, head lane%32
  f32x4 o16[8];
  f32x16 o32[4];
};

// Dequantise this lane's slot of a chunk (row 16w + l16, k-group g), stage its value
// dims as bf16 into `vtile` and return S^T fragments: sacc[hb][i] = q.k of chunk row
// 16w + 4g + i and head 16hb + l16.  Two accumulator chains per head block.
template <int NHB, int KV = kKvFp8Ds>
__device__ __forceinline__ void stage_chunk(__bf16* __restrict__ vtile, const RawT<KV>& cur,
                                            const AttnState<NHB>& st, f32x4 (&sacc)[NHB], int w,
                                            int l16, int g) {
  f32x4 sa[NHB], sb[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    sa[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    sb[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int vr = 16 * w + l16;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    bf16x8 k0, k1;
    k_frags<KV>(cur, u, k0, k1);
    *reinterpret_cast<bf16x8*>(vtile + v_off(vr, 8 * u + 2 * g)) = k0;
    *reinterpret_cast<bf16x8*>(vtile + v_off(vr, 8 * u + 2 * g + 1)) = k1;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      sa[hb] = mfma16(k0, st.qf[hb][2 * u], sa[hb]);
      sb[hb] = mfma16(k1, st.qf[hb][2 * u + 1], sb[hb]);
    }
  }
  bf16x8 k16, k17;
  k_frags_rope<KV>(cur, k16, k17);
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    sa[hb] = mfma16(k16, st.qf[hb][16], sa[hb]);
    sb[hb] = mfma16(k17, st.qf[hb][17], sb[hb]);
    sacc[hb] = sa[hb] + sb[hb];
  }
}

// O^T[c][h] += V^T[c][j] P^T[j][h] over the 64 rows of a staged chunk, for this wave's
// 128 output dims.  Transposing reads: input lane 4r+q of a 16-lane group addresses row
// row0+r, dims col0+4q..col0+4q+3 (16 B unit col0/8 + q/2, half q&1); lane L of the
// group receives dim col0+L of rows row0..row0+3.
// NHB == 1: O^T[c][h] += V^T[c][j] P^T[j][h] over the 64 rows of a staged chunk for
// this wave's 128 output dims, on 16x16x32 MFMA: A = V^T (16 dims x 32 rows), B = P^T
// (32 rows x 16 heads).  Transposing reads: input lane 4r+q of a 16-lane group addresses
// row row0+r, dims col0+4q..col0+4q+3; lane L of the group receives dim col0+L of rows
// row0..row0+3.
template <int NHB>
__device__ __forceinline__ void pv_chunk(const __bf16* __restrict__ vtile,
                                         const __bf16 (*__restrict__ ptile)[kPStride],
                                         AttnState<NHB>& st, int w, int lane) {
  static_assert(NHB == 1, "the two-block path uses pv_reads2 / pv_mfma2");
  const int l16 = lane & 15, G = lane >> 4;
  const int r = l16 >> 2, q4 = l16 & 3;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 pf = *reinterpret_cast<const bf16x8*>(&ptile[l16][32 * ks + 8 * G]);
    const int row0 = 32 * ks + 8 * G + r;
    bf16x4 t0[8], t1[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int unit = 16 * w + 2 * mb + (q4 >> 1);
      t0[mb] = lds_read_tr16(vtile + v_off(row0, unit) + 4 * (q4 & 1));
      t1[mb] = lds_read_tr16(vtile + v_off(row0 + 4, unit) + 4 * (q4 & 1));
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      bf16x8 vf;
      vf[0] = t0[mb][0]; vf[1] = t0[mb][1]; vf[2] = t0[mb][2]; vf[3] = t0[mb][3];
      vf[4] = t1[mb][0]; vf[5] = t1[mb][1]; vf[6] = t1[mb][2]; vf[7] = t1[mb][3];
      st.o16[mb] = mfma16(vf, pf, st.o16[mb]);
    }
  }
}

// NHB == 2 pieces of a pipelined chunk step.  Output dims of wave w are the 32-dim
// blocks 128mb + 32w (mb = 0..3), so that in the transposing reads the lane-dependent
// part of the swizzle lands on the wave's own unit bits and every LDS access of a lane
// is one base register plus a compile-time constant.

// Staging of one chunk: dequantise this lane's slot (row 16w + l16, k-group g), write its
// value dims into `vn`, S^T fragments into sacc (two accumulator chains per head block).
// If REFILL, each piece of `cur` is re-requested for the chunk at `nxt` as soon as it has
// been converted, so the record loads of a chunk go out one by one across the staging
// work instead of as one burst: a burst fills the memory pipeline's queue and stalls
// the wave's in-order issue until it drains.
template <bool REFILL, int KV = kKvFp8Ds>
__device__ __forceinline__ void stage2(__bf16* __restrict__ vn, RawT<KV>& cur, const RecPtr& nxt,
                                       const AttnState<2>& st, f32x4 (&sacc)[2], int w,
                                       int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  const int vr = 16 * w + l16;
  // unit 8u + 2g + h of row vr goes to unit (8u + 2g + h) ^ swz(vr): bit 3 of swz flips
  // the parity of u, bit 0 flips h, bits 1-2 act on g only.
  const int sw = v_swz(vr);
  const int ub = (sw >> 3) & 1;
  const int c0 = (2 * g) ^ (sw & 6);
  __bf16* const rowp = vn + vr * kVStride + 8 * c0;
  __bf16* const wb[2][2] = {{rowp + 64 * ub + 8 * (sw & 1), rowp + 64 * ub + 8 * (1 - (sw & 1))},
                            {rowp - 64 * ub + 8 * (sw & 1), rowp - 64 * ub + 8 * (1 - (sw & 1))}};
  f32x4 sa[2], sb[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    sa[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    sb[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    bf16x8 k0, k1;
    k_frags<KV>(cur, u, k0, k1);
    if constexpr (REFILL) load_nope_piece<KV>(cur, nxt, u);
    *reinterpret_cast<bf16x8*>(wb[u & 1][0] + 64 * u) = k0;
    *reinterpret_cast<bf16x8*>(wb[u & 1][1] + 64 * u) = k1;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sa[hb] = mfma16(k0, st.qf[hb][2 * u], sa[hb]);
      sb[hb] = mfma16(k1, st.qf[hb][2 * u + 1], sb[hb]);
    }
  }
  bf16x8 k16, k17;
  k_frags_rope<KV>(cur, k16, k17);
  if constexpr (REFILL) load_rope_piece<KV>(cur, nxt);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    sa[hb] = mfma16(k16, st.qf[hb][16], sa[hb]);
    sb[hb] = mfma16(k17, st.qf[hb][17], sb[hb]);
    sacc[hb] = sa[hb] + sb[hb];
  }
}

// P.V operands of a staged chunk.  32x32x16 MFMA: A = V^T (32 dims x 16 rows), lane L
// holding dim L%32 of rows 8(L/32)..+7; B = P^T, lane L holding head L%32 of the same rows.
// Transposing read: input lane 4r+q of a 16-lane group addresses row row0+r, dims
// col0+4q..+3 (unit col0/8 + q/2, half q&1); lane L of the group receives dim col0+L of
// rows row0..row0+3.  Row 16ks + 8hi + r (+4) has swz 4r + 2hi (+1).
struct PvFrags {
  bf16x8 pf[4];
  bf16x4 t0[4][4], t1[4][4];
};
__device__ __forceinline__ void pv_reads2(const __bf16* __restrict__ vt,
                                          const __bf16 (*__restrict__ pt)[kPStride], PvFrags& f,
                                          int w, int lane) {
  const int l16 = lane & 15, G = lane >> 4, hi = lane >> 5;
  const int r = l16 >> 2, q4 = l16 & 3;
  const int lo = 2 * (G & 1) + (q4 >> 1);  // unit bits 0-1 before the swizzle
  const __bf16* const rb0 =
      vt + (8 * hi + r) * kVStride + 8 * (4 * (w ^ r) + (lo ^ (2 * hi))) + 4 * (q4 & 1);
  const __bf16* const rb1 =
      vt + (8 * hi + r + 4) * kVStride + 8 * (4 * (w ^ r) + (lo ^ (2 * hi + 1))) + 4 * (q4 & 1);
  const __bf16* const pb = &pt[lane & 31][8 * hi];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f.pf[ks] = *reinterpret_cast<const bf16x8*>(pb + 16 * ks);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f.t0[ks][mb] = lds_read_tr16(rb0 + 16 * ks * kVStride + 128 * mb);
      f.t1[ks][mb] = lds_read_tr16(rb1 + 16 * ks * kVStride + 128 * mb);
    }
  }
}
__device__ __forceinline__ void pv_mfma2(const PvFrags& f, AttnState<2>& st) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      bf16x8 vf;
      vf[0] = f.t0[ks][mb][0]; vf[1] = f.t0[ks][mb][1]; vf[2] = f.t0[ks][mb][2]; vf[3] = f.t0[ks][mb][3];
      vf[4] = f.t1[ks][mb][0]; vf[5] = f.t1[ks][mb][1]; vf[6] = f.t1[ks][mb][2]; vf[7] = f.t1[ks][mb][3];
      st.o32[mb] = mfma32(vf, f.pf[ks], st.o32[mb]);
    }
}

// Scores of the freshly staged chunk -> s (raw q.k, invalid rows -inf), this wave's
// per-head maxima (log2 domain) into `red`, probabilities against the current reference into
// `ptile` (clamped at 2^kPLimit; a chunk that needs more is recomputed after the
// barrier), and their per-lane sums into psum.
// SHIFT_MASK: the lane's four validity bits are taken from vmask >> 4g (one 64-bit shift
// a chunk) instead of being tested against four per-lane 64-bit masks, which a kernel
// short of registers would otherwise keep (or spill) across its loop.
template <int NHB, bool SHIFT_MASK = false>
__device__ __forceinline__ void softmax_local(__bf16 (*__restrict__ ptile)[kPStride],
                                              float (*__restrict__ red)[16 * NHB],
                                              const f32x4 (&sacc)[NHB], uint64_t vmask,
                                              const AttnState<NHB>& st, float scale_log2,
                                              float (&s)[NHB][4], float (&psum)[NHB], int w,
                                              int l16, int g) {
  const uint32_t vm = SHIFT_MASK ? (uint32_t)(vmask >> (4 * g)) : 0u;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (SHIFT_MASK)
        s[hb][i] = ((vm >> i) & 1u) ? sacc[hb][i] : -INFINITY;
      else
        s[hb][i] = ((vmask >> (4 * g + i)) & 1) ? sacc[hb][i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[hb][0], s[hb][1]), fmaxf(s[hb][2], s[hb][3]));
    mx = max_xor32(max_xor16(mx));
    // every lane stores (the 4 lanes of a head hold the same value): a lane condition here
    // would end the basic block, and with it the interleaving of the softmax with the
    // P.V MFMAs in pipelined_step
    red[w][16 * hb + l16] = mx * scale_log2;
    const float nmr = -st.m_run[hb];
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = __builtin_amdgcn_exp2f(fminf(__builtin_fmaf(s[hb][i], scale_log2, nmr), kPLimit));
    psum[hb] = (p[0] + p[1]) + (p[2] + p[3]);
    *reinterpret_cast<uint2*>(&ptile[16 * hb + l16][16 * w + 4 * g]) =
        make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  }
}

// After the barrier that publishes a chunk's maxima: if any head's chunk max beats the
// reference by more than kPLimit (always the case for the first chunk with a valid
// row), every wave moves the reference, rescales O and the denominator, rewrites the
// chunk's probabilities and meets at one more barrier.  The decision reads the same LDS
// words in every wave, so the workgroup takes the branch together.
template <int NHB>
__device__ __forceinline__ void resolve_chunk(__bf16 (*__restrict__ ptile)[kPStride],
                                              const float (*__restrict__ red)[16 * NHB],
                                              AttnState<NHB>& st, const float (&s)[NHB][4],
                                              float scale_log2, float (&psum)[NHB], int w, int l16,
                                              int g) {
  float cm[NHB];
  bool fix = false;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    cm[hb] = fmaxf(fmaxf(red[0][16 * hb + l16], red[1][16 * hb + l16]),
                   fmaxf(red[2][16 * hb + l16], red[3][16 * hb + l16]));
    fix |= cm[hb] > st.m_run[hb] + kPLimit;
  }
  if (__builtin_amdgcn_ballot_w64(fix)) {
    float alpha[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const float mn = fmaxf(st.m_run[hb], cm[hb]);
      alpha[hb] = __builtin_amdgcn_exp2f(st.m_run[hb] - mn);
      st.m_run[hb] = mn;
      st.l_part[hb] *= alpha[hb];
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = __builtin_amdgcn_exp2f(fminf(__builtin_fmaf(s[hb][i], scale_log2, -mn), kPLimit));
      psum[hb] = (p[0] + p[1]) + (p[2] + p[3]);
      *reinterpret_cast<uint2*>(&ptile[16 * hb + l16][16 * w + 4 * g]) =
          make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    }
    if constexpr (NHB == 2) {
      const float a = (g & 1) ? alpha[1] : alpha[0];  // this lane's head is lane % 32
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) st.o32[mb] *= a;
    } else {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) st.o16[mb] *= alpha[0];
    }
    __syncthreads();
  }
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) st.l_part[hb] += psum[hb];
}

// Chunk i's P.V (tiles vt/pt, published by the last barrier) in the same basic block as
// chunk i+1's staging (raw -> vn, scores), so the matrix cores, the LDS and the VALU
// work on both at once; then chunk i+1's softmax, the chunk's only barrier, and its
// reference check.
// One step of the chunk pipeline (see above), the next record to request given as a slot
// (read from the LDS index block by the caller; -1 for none).  SM: any LDS layout with
// the value tiles v, the probability tiles p and the maxima red.
template <int NHB, int KV = kKvFp8Ds, bool SHIFT_MASK = false, class SM>
__device__ __forceinline__ void pipelined_step_slot(SM& sm, int cb, AttnState<NHB>& st,
                                                    RawT<KV>& raw, int64_t next_slot,
                                                    const CacheRef& cr, int w, int lane,
                                                    float scale_log2) {
  const int l16 = lane & 15, g = lane >> 4;
  const int nb = cb ^ 1;
  f32x4 sacc[NHB];
  float s[NHB][4], psum[NHB];
  if constexpr (NHB == 2) {
    // staging + S first, so the scores are ready by the softmax; the P.V operands are
    // requested next and consumed last, so their MFMAs run across the barrier.
    const uint64_t vmask = __ballot(raw.valid);  // bit j (j < 16) = row 16w + j valid
    const RecPtr nxt = rec_ptr<KV>(cr, next_slot, g);
    stage2<true, KV>(&sm.v[nb][0][0], raw, nxt, st, sacc, w, lane);
    PvFrags f;
    pv_reads2(&sm.v[cb][0][0], sm.p[cb], f, w, lane);
    // With one wave per SIMD the wave issues in order, so left to itself the softmax
    // (VALU only) and the P.V MFMAs run one after the other.  Scheduled as one MFMA then
    // up to eight VALU operations, sixteen times, each P.V MFMA runs on the matrix core
    // while the next softmax operations issue (plain decode 64.3 -> 61.4 us, step 72.9
    // -> 70.8 us; 4, 5 and 6 VALU a group measured within 0.6 us of it).  The
    // scheduling barrier keeps the staging, whose own MFMAs and conversions are already
    // interleaved, out of that pattern.
    __builtin_amdgcn_sched_barrier(0);
    softmax_local<NHB, SHIFT_MASK>(sm.p[nb], sm.red[nb], sacc, vmask, st, scale_log2, s, psum, w,
                                   l16, g);
    pv_mfma2(f, st);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one P.V MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // then up to eight VALU
    }
  } else {
    stage_chunk<NHB, KV>(&sm.v[nb][0][0], raw, st, sacc, w, l16, g);
    pv_chunk<NHB>(&sm.v[cb][0][0], sm.p[cb], st, w, lane);
    const uint64_t vmask = __ballot(raw.valid);
    load_raw<KV>(raw, cr, next_slot, g);
    softmax_local<NHB, SHIFT_MASK>(sm.p[nb], sm.red[nb], sacc, vmask, st, scale_log2, s, psum, w,
                                   l16, g);
  }
  __syncthreads();
  resolve_chunk<NHB>(sm.p[nb], sm.red[nb], st, s, scale_log2, psum, w, l16, g);
}
template <int NHB, int KV = kKvFp8Ds, class SM>
__device__ __forceinline__ void pipelined_step(SM& sm, int cb, AttnState<NHB>& st,
                                               RawT<KV>& raw, int pf_jj, int n_blk,
                                               const CacheRef& cr, int w, int lane,
                                               float scale_log2) {
  pipelined_step_slot<NHB, KV>(sm, cb, st, raw, idx_at(sm.idx, pf_jj, n_blk), cr, w, lane,
                               scale_log2);
}
// The step's normalised q rows in LDS: rows padded by 16 B.  At a 1152 B stride the 16
// rows one Q-fragment read touches fall on the same banks in pairs (measured on this GPU:
// 94% of that read's LDS cycles in conflicts against 75% for lane-consecutive 16 B reads;
// 1168 B matches the consecutive reads).
constexpr int kQRow = kLatent + 8;  // bf16 per LDS q row
static_assert(32 * kQRow <= kChunk * kVStride, "32 q rows fit one value-tile buffer");
static_assert(32 * (kNope + 8) <= kChunk * kVStride, "32 staged output rows fit one value-tile buffer");
static_assert(32 * (kNope + 4) * 4 <= 2 * kChunk * kVStride * 2, "32 staged fp32 partial rows fit both value-tile buffers");

// Q^T fragments of one block of 16 heads from q row `qr` (global memory or LDS): lane
// (head l16, k-group g); k-step s pairs with the K-fragment dims chosen in load_raw
// (nope: 64u+16g+8h, rope: 32r+8g).
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[18], const uint16_t* qr, int g) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    qf[2 * u] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 64 * u + 16 * g));
    qf[2 * u + 1] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 64 * u + 16 * g + 8));
  }
  qf[16] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kNope + 8 * g));
  qf[17] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kNope + 32 + 8 * g));
}

// The block's last chunk: P.V only.
template <int NHB, class SM>
__device__ __forceinline__ void pv_last(SM& sm, int cb, AttnState<NHB>& st,
                                        int w, int lane) {
  if constexpr (NHB == 2) {
    PvFrags f;
    pv_reads2(&sm.v[cb][0][0], sm.p[cb], f, w, lane);
    pv_mfma2(f, st);
  } else {
    pv_chunk<NHB>(&sm.v[cb][0][0], sm.p[cb], st, w, lane);
  }
}

}  // namespace dsv4
