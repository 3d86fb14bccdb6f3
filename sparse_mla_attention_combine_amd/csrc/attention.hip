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
// Per chunk of 64 listed slots (a software pipeline: chunk i's P.V runs in the same step
// as chunk i+1's staging, with one workgroup barrier per chunk):
//   1. every lane holds its slot's 128 code bytes, 32 rope bytes and 8 scale bytes in
//      registers (the token's index row is staged in LDS, every load is branch-free, and
//      each piece is re-requested for the chunk two ahead right after it is converted, so
//      the loads leave one by one instead of as a burst that would stall in-order issue),
//      converts them with gfx950's scaled FP8->bf16 instruction (exact: a power-of-two
//      scale) into MFMA fragments, and stages the 512 value dims as bf16 rows in an
//      XOR-swizzled, double-buffered LDS tile;
//   2. S^T = K Q^T on bf16 MFMA 16x16x32 (Q^T fragments live in registers);
//   3. softmax in the log2 domain against a per-head reference maximum that all waves
//      share: probabilities exp2(s - ref) (up to 2^20) are rounded to bf16 into LDS and
//      each wave's chunk maxima (permlane16/32 swaps) go to LDS; after the barrier the
//      maxima are compared with the reference, and only when a chunk beats it by more
//      than 2^20 (always for the first chunk with a valid row) does the workgroup move
//      the reference, rescale O and the denominator, and rewrite that chunk's
//      probabilities behind one more barrier;
//   4. O^T += V^T P^T on bf16 MFMA 32x32x16: wave w owns output dims 128mb + 32w (mb =
//      0..3) for all NH heads; V^T fragments come from the row-major LDS tile through
//      gfx950's transposing LDS read (ds_read_b64_tr_b16), P^T fragments are plain 16 B
//      reads; these MFMAs are scheduled between the softmax operations of the next
//      chunk (one MFMA, then up to eight VALU operations), so the matrix core works
//      while the in-order wave issues the softmax.
// The output rows leave through LDS as whole rows (a lane's accumulators hold 4
// consecutive dims of one head), and the thread's indices in the epilogue come from an
// opaque copy of the thread id so that nothing stays live, or spilled, across the loop.
// Numerics: bf16 operands, fp32 accumulation and softmax, P rounded to bf16 for P.V;
// the per-head sink enters only the final denominator.
// Cache dtypes (template KV): the packed FP8/UE8M0 record above; bf16 records (the
// fragments are the loaded bits, nothing to convert); E4M3 records with one scale s per
// cache (PR #43477 Key source excerpts: the SM100 backend's "bfloat16" / "fp8" caches):
// the codes convert exactly to bf16 unscaled, s multiplies the softmax scale of the
// scores and the output (o_scale), the same values as scaling every K and V entry.
// Variants of one kernel: the index rows come from memory (decode, prefill, and pieces of
// rows for the split decode), or each workgroup builds its token's row in LDS from the
// combine step's inputs (PR #43385 combine kernel: top-k, window, block table), or it
// also performs the insert step first (PR #42953 Implementation breakdown item 4: q
// RMSNorm + GPT-J RoPE, FP8/UE8M0 insert of the new latent rows) so that one launch is
// the whole decode step.
#include <mutex>


#include "attention_core.hpp"

namespace dsv4 {

// FUSED: the index rows are built in the prologue from the combine step's inputs (`tin`)
// instead of read from `indices` / `lens` (one row per token, no pieces).
// STEP (with FUSED): the prologue also performs the insert step (`sti`) for what this
// workgroup reads: it normalises and rotates its own q heads (written back in place and
// kept in LDS for the Q fragments) and quantises into the cache the new latent rows of
// its request's tokens up to its own, plus its own row; `q` and `cache` are unused and
// the cache is read through sti.cache.  Only this workgroup reads what it wrote (other
// workgroups that write the same rows write the same bytes), so the barrier's
// workgroup-scope ordering suffices.
template <int NHB, bool FUSED, bool STEP, int KV>
__global__ void __launch_bounds__(256) sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots, int ps,
    const int32_t* __restrict__ indices, int idx_stride, const int32_t* __restrict__ lens,
    const float* __restrict__ sinks, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int T, int H, int groups, int splits, int split_len,
    float* __restrict__ part_o, float* __restrict__ part_ml, TopkIn tin, StepIn sti,
    float o_scale) {
  static_assert(FUSED || !STEP, "the step variant builds its index rows itself");
  __shared__ AttnSmem<NHB> sm;

  // work item vt = (query token, split); with one split it is the query token
  int vt, hg;
  if (groups == 1) {
    vt = blockIdx.x;
    hg = 0;
  } else {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    hg = k % groups;
    vt = (k / groups) * 8 + x;
  }
  if (vt >= T * splits) return;
  // Work items in reverse order: in a launch of many rounds (prefill) the longest rows,
  // which come last in a causal sequence, then start first and the last round is short
  // (longest processing time first).  The head groups of a token keep their common
  // block id mod 8, so they still share an XCD.
  vt = T * splits - 1 - vt;
  const int t = vt / splits, sp = vt - t * splits;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int h0 = hg * 16 * NHB;
  // The row length is read as a vector load issued next to the Q and index loads (the
  // address is moved to VGPRs), so that its latency overlaps theirs.
  int n_lens_v = 0;
  if constexpr (!FUSED) {
    uint64_t len_addr = reinterpret_cast<uint64_t>(lens + t);
    asm volatile("" : "+v"(len_addr));
    n_lens_v = *reinterpret_cast<const __attribute__((address_space(1))) int32_t*>(len_addr);
  }
  const int32_t* idx_row = indices + (int64_t)t * idx_stride;
  // this work item's piece [beg, lim) of the row, known before its length arrives
  const int beg = FUSED ? 0 : ((int64_t)sp * split_len < idx_stride ? sp * split_len : idx_stride);
  const int lim = FUSED ? kIdxBlock : beg + min(split_len, idx_stride - beg);

  AttnState<NHB> st;
  const int c8 = lane & 7;
  const float* const no_row = reinterpret_cast<const float*>(g_zero_page);  // unused values
  // Q^T fragments from memory (all but STEP): lane (head l16 of block hb, k-group g);
  // k-step s pairs with the K-fragment dims chosen in load_raw (nope: 64u+16g+8h, rope:
  // 32r+8g).  Requested after the loads that build the index row: vector-memory loads
  // complete in order, so a wait for the row would otherwise also wait for all of Q
  // (144 registers a lane), and the first gathers would leave later.
  auto load_q_global = [&]() {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const uint16_t* qr = q + ((int64_t)t * H + h0 + 16 * hb + l16) * kLatent;
      load_q_frags(st.qf[hb], qr, g);
    }
  };
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    st.m_run[hb] = kMFloor;
    st.l_part[hb] = 0.f;
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.o16[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o32[mb][r] = 0.f;


  // Index blocks of up to 4096 entries are staged in LDS.  Inside a block chunk c lives
  // in register buffer c&1 and LDS tiles c&1; a buffer is refilled with chunk c+2 as
  // soon as staging has consumed it, so two chunks of records are always in flight.
  // Rows from memory: the first block is requested together with the row length and
  // then Q (entries past the length are staged but never used), so the prologue waits
  // for memory only once, and only for the row.  Rows built here (FUSED): the request
  // search's loads, the top-k row and (STEP) the q rows, the first new latent row and
  // the norm weights take one round of memory, issued in the order their values are
  // needed; the block-table entries (one contiguous copy into LDS) and the cos/sin rows
  // a second.
  int end;
  if constexpr (STEP) {
    // Wave w < 2*NHB owns q heads h0 + 8w .. +7 (8 lanes a row, the insert kernel's
    // partition, so the bits match it); every wave w owns the new latent rows t - w,
    // t - w - 4, ... of the request.
    const CombSearch cs = combine_search_load(tin, tid);
    const int64_t t1 = t >= w ? t - w : t;  // in bounds; used only if in the request
    const int64_t qp = vload(sti.positions + t);
    const int64_t kvp = vload(sti.positions + t1);
    const int64_t kvs = vload(sti.slot_mapping + t1);
    int32_t xv[kCombPer];
    int tl;
    combine_topk_load(tin, t, tid, xv, tl);
    u32x4 qraw[9], wq[9];  // (native vectors: copies of a struct type would stay in memory)
    if (w < 2 * NHB) {  // chunk k of this lane's row: 16-byte unit c8 + 8k of the row
      const uint16_t* qr = sti.q + ((int64_t)t * H + h0 + 8 * w + (lane >> 3)) * kLatent;
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        qraw[k] = *reinterpret_cast<const u32x4*>(qr + 8 * (c8 + 8 * k));
        wq[k] = *reinterpret_cast<const u32x4*>(sti.weight + 8 * (c8 + 8 * k));
      }
    }
    const KvLane kvv = kv_lane_load(sti.kv + t1 * kLatent, lane);
    combine_find(sm, tin, t, tid, cs);
    // second round: the block-table entries into the first value tile (free until chunk
    // 0 is staged) and the cos/sin rows of the two positions
    const bool qok = qp >= 0 && qp < sti.max_pos;
    const RopeCs qrot = rope_cs_load(qok ? sti.cos_sin + qp * kRope : no_row, c8);
    const RopeCs kvrot =
        rope_cs_load(kvp >= 0 && kvp < sti.max_pos ? sti.cos_sin + kvp * kRope : no_row, lane);
    int32_t* const bt = reinterpret_cast<int32_t*>(&sm.v[0][0][0]);
    const bool staged = combine_stage_bt(sm, tin, t, ps, bt, w, lane);
    asm volatile("" ::: "memory");  // every load above is issued before the wait
    __builtin_amdgcn_s_waitcnt(0);  // (includes the copy into LDS)
    __syncthreads();
    end = __builtin_amdgcn_readfirstlane(combine_rows(sm, tin, t, ps, tid, xv, tl, bt, staged));
    // this wave's q rows normalised and rotated into LDS (for the Q fragments) and, when
    // the row is not cut into pieces, written back in place.  With pieces, the
    // workgroups of a token's other pieces may still be about to read the raw rows (a
    // grid of several dispatch rounds starts them at different times), so every piece
    // reads raw q and only the merge launch, stream-ordered after all of them, writes
    // the normalised rows.
    const bool q_writer = splits == 1;
    u32x4* ql = reinterpret_cast<u32x4*>(&sm.v[1][0][0]) + (8 * w + (lane >> 3)) * (kQRow / 8) + c8;
    if (w < 2 * NHB) {
      if (qok) {
        u32x4* qg = reinterpret_cast<u32x4*>(sti.q + ((int64_t)t * H + h0 + 8 * w + (lane >> 3)) *
                                                         kLatent) + c8;
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 9; ++k) ss = qn_sum_sq(qraw[k], ss);
        const float inv = qn_inv(ss, sti.eps);
#pragma unroll
        for (int k = 0; k < 9; ++k) {
          const u32x4 y = qn_chunk(qraw[k], wq[k], inv, qrot, k == 8);
          ql[8 * k] = y;
          if (q_writer) qg[8 * k] = y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 9; ++k) ql[8 * k] = qraw[k];  // token left untouched
      }
    }
    // the new rows this token may read: its request's tokens up to itself (only itself for
    // a token of no request, whose own row is inserted all the same)
    const int64_t first = sm.req[0] >= 0 ? (int64_t)max(sm.req[1], 0) : (int64_t)t;
    int64_t tt = (int64_t)t - w;
    if (tt >= first && kvp >= 0 && kvp < sti.max_pos && kvs >= 0 && kvs < num_slots)
      kv_store_row<KV>(kvv, kvrot, sti.cache, kvs, ps, sti.kv_scale, lane);
    for (tt -= 4; tt >= first; tt -= 4) {
      const KvLane v = kv_lane_load(sti.kv + tt * kLatent, lane);
      const int64_t p = sti.positions[tt], sl = sti.slot_mapping[tt];
      if (p >= 0 && p < sti.max_pos && sl >= 0 && sl < num_slots)
        kv_store_row<KV>(v, rope_cs_load(sti.cos_sin + p * kRope, lane), sti.cache, sl, ps,
                         sti.kv_scale, lane);
    }
  } else if constexpr (FUSED) {
    const CombSearch cs = combine_search_load(tin, tid);
    int32_t xv[kCombPer];
    int tl;
    combine_topk_load(tin, t, tid, xv, tl);
    combine_find(sm, tin, t, tid, cs);
    int32_t* const bt = reinterpret_cast<int32_t*>(&sm.v[0][0][0]);
    const bool staged = combine_stage_bt(sm, tin, t, ps, bt, w, lane);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);  // (includes the copy into LDS)
    __syncthreads();
    end = __builtin_amdgcn_readfirstlane(combine_rows(sm, tin, t, ps, tid, xv, tl, bt, staged));
    load_q_global();
  } else {
    int32_t iv[kStagePer];
    const int n_win = min(lim - beg, kIdxBlock);
    stage_idx_load(iv, idx_row + beg, n_win, tid);
    load_q_global();
    stage_idx_store(sm.idx, iv, n_win, tid);
    end = min(max(__builtin_amdgcn_readfirstlane(n_lens_v), 0), lim);
  }
  __syncthreads();  // (STEP: also the q rows in LDS and this workgroup's cache rows written)
  if constexpr (FUSED) {
    if (splits > 1) {
      // piece sp of the built row, [sp * split_len, +split_len), moves to the start of
      // the index block (every entry read before any is written)
      const int pb = min(sp * split_len, end);
      const int pn = min(split_len, end - pb);
      int32_t pv[kCombPer];
#pragma unroll
      for (int u = 0; u < kCombPer; ++u) pv[u] = sm.idx[min(pb + tid + 256 * u, kIdxBlock - 1)];
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kCombPer; ++u)
        if (tid + 256 * u < pn) sm.idx[tid + 256 * u] = pv[u];
      __syncthreads();
      end = pn;
    }
  }
  if constexpr (STEP) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      load_q_frags(st.qf[hb], reinterpret_cast<const uint16_t*>(&sm.v[1][0][0]) +
                                  (16 * hb + l16) * kQRow, g);
  }
  if constexpr (NHB == 2 && STEP) {
    // The step's prologue leaves more values live than the other variants, and the
    // register allocator would otherwise spill Q fragments to AGPRs and copy each one
    // back into VGPRs before every use (72 copies per chunk for the second head block,
    // then 12 for the first block's first three).  Placing the second block and the
    // first ten fragments of the first in AGPRs from the start lets the MFMAs read them
    // there directly (an MFMA accepts AGPR A/B operands); the empty asm only fixes the
    // register class.  Measured: step 63.9 -> 61.5 us (B = 64, H = 128), MTP step 581
    // -> 578 us; 3, 6 or 13 of the first block's fragments were slower, all 18 much
    // slower (66.7 us).
#pragma unroll
    for (int k = 0; k < 18; ++k) asm volatile("" : "+a"(st.qf[1][k]));
#pragma unroll
    for (int k = 0; k < 10; ++k) asm volatile("" : "+a"(st.qf[0][k]));
  }
  const int row = 16 * w + l16;
  const CacheRef cr{STEP ? sti.cache : cache, num_slots, ps};
  for (int blk0 = beg; blk0 < end; blk0 += kIdxBlock) {
    const int n_blk = min(end - blk0, kIdxBlock);
    if (blk0 != beg) {
      __syncthreads();  // the previous block's entries and tiles are no longer read
      for (int i = tid; i < n_blk; i += 256) sm.idx[i] = idx_row[blk0 + i];
      __syncthreads();
    }
    const int nch = (n_blk + kChunk - 1) / kChunk;
    // Chunks of records in flight per lane: two (buffers A and B, odd chunks in B), or
    // one for bf16 records at 32 heads (72 registers a chunk beside Q for 32 heads).
    constexpr int kAhead = (KV == kKvBf16 && NHB == 2) ? 1 : 2;
    RawT<KV> A, B;
    RawT<KV>& odd = kAhead == 2 ? B : A;
    load_raw<KV>(A, cr, idx_at(sm.idx, row, n_blk), g);
    if constexpr (kAhead == 2) load_raw<KV>(B, cr, idx_at(sm.idx, kChunk + row, n_blk), g);
    {  // prologue: stage chunk 0 and settle its probabilities
      f32x4 sacc[NHB];
      const uint64_t vmask = __ballot(A.valid);
      if constexpr (NHB == 2) {
        const RecPtr nxt = rec_ptr<KV>(cr, idx_at(sm.idx, kAhead * kChunk + row, n_blk), g);
        stage2<true, KV>(&sm.v[0][0][0], A, nxt, st, sacc, w, lane);
      } else {
        stage_chunk<NHB, KV>(&sm.v[0][0][0], A, st, sacc, w, l16, g);
        load_raw<KV>(A, cr, idx_at(sm.idx, kAhead * kChunk + row, n_blk), g);
      }
      float s[NHB][4], psum[NHB];
      softmax_local<NHB>(sm.p[0], sm.red[0], sacc, vmask, st, scale_log2, s, psum, w, l16, g);
      __syncthreads();
      resolve_chunk<NHB>(sm.p[0], sm.red[0], st, s, scale_log2, psum, w, l16, g);
    }
    int i = 0;
    for (; i + 2 < nch; i += 2) {
      pipelined_step<NHB, KV>(sm, 0, st, odd, (i + 1 + kAhead) * kChunk + row, n_blk, cr, w,
                              lane, scale_log2);
      pipelined_step<NHB, KV>(sm, 1, st, A, (i + 2 + kAhead) * kChunk + row, n_blk, cr, w, lane,
                              scale_log2);
    }
    if (i + 1 < nch) {
      pipelined_step<NHB, KV>(sm, 0, st, odd, (i + 1 + kAhead) * kChunk + row, n_blk, cr, w,
                              lane, scale_log2);
      pv_last<NHB>(sm, 1, st, w, lane);
    } else {
      pv_last<NHB>(sm, 0, st, w, lane);
    }
  }

  {  // the thread's indices are recomputed from an opaque copy of the thread id: shared
     // with the prologue, their address terms would stay live across the chunk loop
     // and be spilled
  int tid_e = threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  const int lane = tid_e & 63, w = tid_e >> 6, l16 = lane & 15, g = lane >> 4;
  // ---- finalise: sum the waves' partial denominators, add the sink, normalise
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float lp = sum_xor32(sum_xor16(st.l_part[hb]));
    if (g == 0) sm.lsum[w][16 * hb + l16] = lp;
  }
  __syncthreads();
  // this lane's output head: l16 (NHB == 1) or lane % 32 (NHB == 2)
  const int hl = NHB == 2 ? (lane & 31) : l16;
  const int h = h0 + hl;
  const float lt = sm.lsum[0][hl] + sm.lsum[1][hl] + sm.lsum[2][hl] + sm.lsum[3][hl];
  const float mr = (NHB == 2 && (g & 1)) ? st.m_run[NHB - 1] : st.m_run[0];
  if constexpr (KV == kKvFp8E4m3) {
    if (part_o) {  // the per-tensor scale of the values, before the partial leaves
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) st.o16[mb] *= o_scale;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) st.o32[mb] *= o_scale;
    }
  }
  if (part_o) {
    // one split of a row: the unnormalised O (relative to the reference mr), mr and the
    // denominator go to the workspace; the merge pass adds the sink and normalises
    float* po = part_o + ((int64_t)vt * H + h) * kNope;
    if constexpr (NHB == 2) {
      // staged through LDS (both value tiles, free after the barrier above; rows padded
      // by 16 B) so that each store instruction writes 1 KB of one row instead of 64
      // separate 16-byte pieces
      const int hi = lane >> 5;
      float* const ot = reinterpret_cast<float*>(&sm.v[0][0][0]);
      constexpr int kOStride = kNope + 4;  // fp32 per staged partial row
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& o = st.o32[mb];
          *reinterpret_cast<float4*>(ot + hl * kOStride + 128 * mb + 32 * w + 8 * qd + 4 * hi) =
              make_float4(o[4 * qd], o[4 * qd + 1], o[4 * qd + 2], o[4 * qd + 3]);
        }
      if (w == 0 && hi == 0) *reinterpret_cast<float2*>(part_ml + ((int64_t)vt * H + h) * 2) = make_float2(mr, lt);
      __syncthreads();
      float* const pb = part_o + ((int64_t)vt * H + h0) * kNope;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int hr = 8 * w + r;
          *reinterpret_cast<float4*>(pb + (int64_t)hr * kNope + 256 * half + 4 * lane) =
              *reinterpret_cast<const float4*>(ot + hr * kOStride + 256 * half + 4 * lane);
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const f32x4 o = st.o16[mb];
        *reinterpret_cast<float4*>(po + 128 * w + 16 * mb + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (w == 0 && g == 0) *reinterpret_cast<float2*>(part_ml + ((int64_t)vt * H + h) * 2) = make_float2(mr, lt);
    }
    return;
  }
  const float z2 = sinks ? sinks[h] * kLog2e : -INFINITY;
  const float M = fmaxf(mr, z2);
  const float f = exp2f(mr - M);
  const float den = lt * f + ((z2 == -INFINITY) ? 0.f : exp2f(z2 - M));
  float inv = den > 0.f ? f / den : 0.f;
  if constexpr (KV == kKvFp8E4m3) inv *= o_scale;  // the per-tensor scale of the values
  uint16_t* orow = out + ((int64_t)t * H + h) * kNope;
  if constexpr (NHB == 2) {
    // A lane holds 4 consecutive output dims of one head per register group, so direct
    // stores would write 8-byte pieces, 64 rows per instruction.  The normalised rows go
    // through LDS instead (the first value tile is free after the barrier above; rows
    // padded by 16 B so that the heads of a write spread over the banks) and leave as
    // whole 1 KB rows, one per store instruction.
    const int hi = lane >> 5;
    __bf16* const ot = &sm.v[0][0][0];
    constexpr int kOStride = kNope + 8;  // bf16 per staged output row
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x16& o = st.o32[mb];
        *reinterpret_cast<uint2*>(ot + hl * kOStride + 128 * mb + 32 * w + 8 * qd + 4 * hi) =
            make_uint2(pack_bf16x2(o[4 * qd] * inv, o[4 * qd + 1] * inv),
                       pack_bf16x2(o[4 * qd + 2] * inv, o[4 * qd + 3] * inv));
      }
    if (lse && w == 0 && hi == 0)
      lse[(int64_t)t * H + h] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
    __syncthreads();
    uint16_t* const ob = out + ((int64_t)t * H + h0) * kNope;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int hr = 8 * w + r;
      *reinterpret_cast<uint4*>(ob + (int64_t)hr * kNope + 8 * lane) =
          *reinterpret_cast<const uint4*>(ot + hr * kOStride + 8 * lane);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const f32x4 o = st.o16[mb];
      *reinterpret_cast<uint2*>(orow + 128 * w + 16 * mb + 4 * g) =
          make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
    }
    if (lse && w == 0 && g == 0)
      lse[(int64_t)t * H + h] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
  }
}

// Persistent prefill (dsv4_sparse_mla_prefill with many rows): one workgroup per compute
// unit loops over the (token, 32-head group) items of the one-shot launch, in the same
// order and XCD placement (item i runs on the XCD of block id i; tokens in reverse, so
// the longest causal rows come first).  What the loop buys is the prologue: while an
// item's chunks run, the next item's index row is copied from memory straight into the
// other of two LDS row buffers (no registers), and its Q fragments are requested as soon
// as the item's last chunk has been staged (Q is dead then), so the next item starts
// with its row in LDS and its Q in flight instead of paying two memory round trips.
// Rows of up to kPIdx entries.  Same arithmetic as the one-shot kernel, bit for bit.
constexpr int kPIdx = 2304;

struct AttnSmemP {
  __bf16 v[2][kChunk][kVStride];
  __bf16 p[2][32][kPStride];
  float red[2][4][32];
  float lsum[4][32];
  int32_t idx[2][kPIdx];
};
static_assert(sizeof(AttnSmemP) <= 160 * 1024, "fits the LDS of a compute unit");

// Entry jj of a row buffer of kPIdx entries (-1 at or past n).
__device__ __forceinline__ int64_t idx_at_p(const int32_t* idx, int jj, int n) {
  const int32_t v = idx[min(jj, kPIdx - 1)];
  return jj < n ? (int64_t)v : -1;
}

// The normalised output rows and lse of a (token, 32 heads) item: the waves' partial
// denominators summed, the sink added, O scaled and staged through LDS (first value
// tile) so that each store writes one 1 KB row.
template <int KV, class SM>
__device__ __forceinline__ void store_rows2(SM& sm, const AttnState<2>& st,
                                            const float* __restrict__ sinks,
                                            uint16_t* __restrict__ out, float* __restrict__ lse,
                                            int64_t t, int H, int h0, float o_scale) {
  int tid_e = threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  const int lane = tid_e & 63, w = tid_e >> 6, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float lp = sum_xor32(sum_xor16(st.l_part[hb]));
    if (g == 0) sm.lsum[w][16 * hb + l16] = lp;
  }
  __syncthreads();
  const int hl = lane & 31;
  const int h = h0 + hl;
  const float lt = sm.lsum[0][hl] + sm.lsum[1][hl] + sm.lsum[2][hl] + sm.lsum[3][hl];
  const float mr = (g & 1) ? st.m_run[1] : st.m_run[0];
  const float z2 = sinks ? sinks[h] * kLog2e : -INFINITY;
  const float M = fmaxf(mr, z2);
  const float f = exp2f(mr - M);
  const float den = lt * f + ((z2 == -INFINITY) ? 0.f : exp2f(z2 - M));
  float inv = den > 0.f ? f / den : 0.f;
  if constexpr (KV == kKvFp8E4m3) inv *= o_scale;
  const int hi = lane >> 5;
  __bf16* const ot = &sm.v[0][0][0];
  constexpr int kOStride = kNope + 8;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f32x16& o = st.o32[mb];
      *reinterpret_cast<uint2*>(ot + hl * kOStride + 128 * mb + 32 * w + 8 * qd + 4 * hi) =
          make_uint2(pack_bf16x2(o[4 * qd] * inv, o[4 * qd + 1] * inv),
                     pack_bf16x2(o[4 * qd + 2] * inv, o[4 * qd + 3] * inv));
    }
  if (lse && w == 0 && hi == 0)
    lse[t * H + h] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
  __syncthreads();
  uint16_t* const ob = out + (t * H + h0) * kNope;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int hr = 8 * w + r;
    *reinterpret_cast<uint4*>(ob + (int64_t)hr * kNope + 8 * lane) =
        *reinterpret_cast<const uint4*>(ot + hr * kOStride + 8 * lane);
  }
}

template <int KV>
__global__ void __launch_bounds__(256) sparse_mla_prefill_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots, int ps,
    const int32_t* __restrict__ indices, int idx_stride, const int32_t* __restrict__ lens,
    const float* __restrict__ sinks, float scale_log2, float o_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse, int T, int H, int groups, int n_items) {
  __shared__ AttnSmemP sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int row = 16 * w + l16;
  const CacheRef cr{cache, num_slots, ps};
  // item -> (token, head group), as the one-shot launch maps its block ids
  auto item = [&](int it, int64_t& t, int& h0, int& len) -> bool {
    const int x = it & 7, k = it >> 3;
    const int vt = (k / groups) * 8 + x;
    if (vt >= T) return false;
    t = T - 1 - vt;
    h0 = (k % groups) * 32;
    len = min(max(lens[t], 0), idx_stride);
    return true;
  };
  int it = blockIdx.x;
  int64_t t = 0;
  int h0 = 0, len = 0;
  while (it < n_items && !item(it, t, h0, len)) it += gridDim.x;
  if (it >= n_items) return;
  int buf = 0;
  AttnState<2> st;
  copy_row_to_lds(sm.idx[0], indices + t * idx_stride, len, w, lane);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
    load_q_frags(st.qf[hb], q + (t * H + h0 + 16 * hb + l16) * kLatent, g);
  __builtin_amdgcn_s_waitcnt(0);  // (includes the row's copy into LDS)
  __syncthreads();
  for (;;) {
    int nit = it + gridDim.x;
    int64_t nt = 0;
    int nh0 = 0, nlen = 0;
    while (nit < n_items && !item(nit, nt, nh0, nlen)) nit += gridDim.x;
    const bool has_next = nit < n_items;
    if (has_next) copy_row_to_lds(sm.idx[buf ^ 1], indices + nt * idx_stride, nlen, w, lane);
    // (the lane's indices from an opaque copy of the thread id: kept from the prologue,
    // their address terms would stay live across the chunk loop and be spilled)
    auto load_next_q = [&]() {
      if (has_next) {
        int tid_q = threadIdx.x;
        asm volatile("" : "+v"(tid_q));
        const int l16q = tid_q & 15, gq = (tid_q >> 4) & 3;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          load_q_frags(st.qf[hb], q + (nt * H + nh0 + 16 * hb + l16q) * kLatent, gq);
      }
    };
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      st.m_run[hb] = kMFloor;
      st.l_part[hb] = 0.f;
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o32[mb][r] = 0.f;
    const int32_t* cidx = sm.idx[buf];
    const int n_blk = len;
    const int nch = (n_blk + kChunk - 1) / kChunk;
    if (nch > 0) {
      constexpr int kAhead = KV == kKvBf16 ? 1 : 2;
      RawT<KV> A, B;
      RawT<KV>& odd = kAhead == 2 ? B : A;
      load_raw<KV>(A, cr, idx_at_p(cidx, row, n_blk), g);
      if constexpr (kAhead == 2) load_raw<KV>(B, cr, idx_at_p(cidx, kChunk + row, n_blk), g);
      {
        f32x4 sacc[2];
        const uint64_t vmask = __ballot(A.valid);
        const RecPtr nxt = rec_ptr<KV>(cr, idx_at_p(cidx, kAhead * kChunk + row, n_blk), g);
        stage2<true, KV>(&sm.v[0][0][0], A, nxt, st, sacc, w, lane);
        float s[2][4], psum[2];
        softmax_local<2, true>(sm.p[0], sm.red[0], sacc, vmask, st, scale_log2, s, psum, w, l16,
                               g);
        __syncthreads();
        resolve_chunk<2>(sm.p[0], sm.red[0], st, s, scale_log2, psum, w, l16, g);
      }
      int i = 0;
      for (; i + 2 < nch; i += 2) {
        pipelined_step_slot<2, KV, true>(sm, 0, st, odd,
                                   idx_at_p(cidx, (i + 1 + kAhead) * kChunk + row, n_blk), cr,
                                   w, lane, scale_log2);
        pipelined_step_slot<2, KV, true>(sm, 1, st, A,
                                   idx_at_p(cidx, (i + 2 + kAhead) * kChunk + row, n_blk), cr,
                                   w, lane, scale_log2);
      }
      if (i + 1 < nch) {
        pipelined_step_slot<2, KV, true>(sm, 0, st, odd,
                                   idx_at_p(cidx, (i + 1 + kAhead) * kChunk + row, n_blk), cr,
                                   w, lane, scale_log2);
        pv_last<2>(sm, 1, st, w, lane);
      } else {
        pv_last<2>(sm, 0, st, w, lane);
      }
    }
    load_next_q();  // in flight during the output rows' staging and stores
    store_rows2<KV>(sm, st, sinks, out, lse, t, H, h0, o_scale);
    __builtin_amdgcn_s_waitcnt(0);  // the next row's copy into LDS has landed
    __syncthreads();                // ... for every wave; the value tiles are free again
    if (!has_next) break;
    it = nit;
    t = nt;
    h0 = nh0;
    len = nlen;
    buf ^= 1;
  }
}

// Merge of the split partials of a row (LSE merge): with per-split reference maxima m_s
// (log2 domain), denominators l_s and unnormalised outputs O_s, and the sink z,
//   M = max(z, max_s m_s),  den = 2^(z-M) + sum_s l_s 2^(m_s-M),
//   out = sum_s O_s 2^(m_s-M) / den,  lse = (M + log2 den) ln 2.
// One wave per (token, head); lane l owns output dims 8l..8l+7.
// For the split form of the whole step, blocks past the merge's normalise and rotate q in
// place (the insert's q part, the same per-row arithmetic): the pieces read raw q, and
// this launch runs after all of them.
__global__ void __launch_bounds__(256) split_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const float* __restrict__ sinks, uint16_t* __restrict__ out, float* __restrict__ lse, int T,
    int H, int splits, int merge_blocks, int qblocks, StepIn sti) {
  if ((int)blockIdx.x >= merge_blocks) {
    q_norm_rope_rows(sti.q, sti.positions, sti.cos_sin, sti.max_pos, sti.weight, sti.eps,
                     (int64_t)T * H, H, (int)blockIdx.x - merge_blocks, qblocks);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * H + h
  if (row >= (int64_t)T * H) return;
  const int t = (int)(row / H), h = (int)(row - (int64_t)t * H);
  const float z2 = sinks ? sinks[h] * kLog2e : -INFINITY;
  // Up to 8 partials per round, every load of a round issued before the first is used
  // (at clamped indices): one memory round trip per 8 pieces instead of two per piece.
  // A later round rescales what the earlier ones summed (only with more than 8 pieces;
  // with at most 8 the arithmetic is the definition's, in its order).
  constexpr int kRound = 8;
  float M = z2, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += kRound) {
    float2 ml[kRound];
    float4 a[kRound], b[kRound];
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int64_t pr = ((int64_t)t * splits + min(s0 + j, splits - 1)) * H + h;
      ml[j] = *reinterpret_cast<const float2*>(part_ml + pr * 2);
      a[j] = *reinterpret_cast<const float4*>(part_o + pr * kNope + 8 * lane);
      b[j] = *reinterpret_cast<const float4*>(part_o + pr * kNope + 8 * lane + 4);
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kRound; ++j)
      if (s0 + j < splits) mb = fmaxf(mb, ml[j].x);
    if (s0 == 0) {
      den = (z2 == -INFINITY) ? 0.f : exp2f(z2 - mb);
    } else {
      const float c = exp2f(M - mb);
      den *= c;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= c;
    }
    M = mb;
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      if (s0 + j >= splits) break;
      const float wgt = exp2f(ml[j].x - M);
      den += ml[j].y * wgt;
      acc[0] += a[j].x * wgt; acc[1] += a[j].y * wgt; acc[2] += a[j].z * wgt; acc[3] += a[j].w * wgt;
      acc[4] += b[j].x * wgt; acc[5] += b[j].y * wgt; acc[6] += b[j].z * wgt; acc[7] += b[j].w * wgt;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint4 v;
  v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(out + row * kNope + 8 * lane) = v;
  if (lse && lane == 0) lse[row] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

size_t split_workspace_bytes(int T, int H, int splits) {
  return (size_t)T * splits * H * (kNope + 2) * sizeof(float);
}

template <bool FUSED, bool STEP, int KV>
static hipError_t launch_items_kv(const void* q, const uint8_t* cache, int num_pages, int ps,
                                  const int32_t* indices, int idx_stride, const int32_t* lens,
                                  const float* sinks, float scale_log2, float o_scale, void* out,
                                  float* lse, int T, int H, int splits, int split_len,
                                  float* part_o, float* part_ml, const TopkIn& tin,
                                  const StepIn& sti, hipStream_t stream) {
  const int64_t num_slots = (int64_t)num_pages << ps;
  const int items = T * splits;
  if (H == 16) {
    hipLaunchKernelGGL((sparse_mla_kernel<1, FUSED, STEP, KV>), dim3(items), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), cache, num_slots, ps, indices, idx_stride, lens,
                       sinks, scale_log2, static_cast<uint16_t*>(out), lse, T, H, 1, splits,
                       split_len, part_o, part_ml, tin, sti, o_scale);
  } else {
    const int groups = H / 32;
    const int grid = groups == 1 ? items : 8 * groups * ((items + 7) / 8);
    hipLaunchKernelGGL((sparse_mla_kernel<2, FUSED, STEP, KV>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), cache, num_slots, ps, indices, idx_stride, lens,
                       sinks, scale_log2, static_cast<uint16_t*>(out), lse, T, H, groups, splits,
                       split_len, part_o, part_ml, tin, sti, o_scale);
  }
  return hipGetLastError();
}

// The per-tensor fp8 cache folds its scale s into the scores' softmax scale and the
// output: the codes are K and V up to that factor.
template <bool FUSED, bool STEP>
static hipError_t launch_items(const void* q, const uint8_t* cache, int num_pages, int ps,
                               int kv_dtype, float kv_scale, const int32_t* indices,
                               int idx_stride, const int32_t* lens, const float* sinks,
                               float softmax_scale, void* out, float* lse, int T, int H,
                               int splits, int split_len, float* part_o, float* part_ml,
                               const TopkIn& tin, StepIn sti, hipStream_t stream) {
  const float scale_log2 = softmax_scale * kLog2e;
  sti.kv_scale = kv_scale;
  switch (kv_dtype) {
    case kKvFp8Ds:
      return launch_items_kv<FUSED, STEP, kKvFp8Ds>(q, cache, num_pages, ps, indices, idx_stride,
                                                    lens, sinks, scale_log2, 1.f, out, lse, T, H,
                                                    splits, split_len, part_o, part_ml, tin, sti,
                                                    stream);
    case kKvBf16:
      return launch_items_kv<FUSED, STEP, kKvBf16>(q, cache, num_pages, ps, indices, idx_stride,
                                                   lens, sinks, scale_log2, 1.f, out, lse, T, H,
                                                   splits, split_len, part_o, part_ml, tin, sti,
                                                   stream);
    case kKvFp8E4m3:
      return launch_items_kv<FUSED, STEP, kKvFp8E4m3>(
          q, cache, num_pages, ps, indices, idx_stride, lens, sinks, softmax_scale * kv_scale * kLog2e,
          kv_scale, out, lse, T, H, splits, split_len, part_o, part_ml, tin, sti, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_topk(const void* q, const uint8_t* cache, int num_pages,
                                 int page_shift, int kv_dtype, float kv_scale,
                                 const int32_t* topk, int topk_stride,
                                 int topk_width, const int32_t* topk_lens, const int32_t* qsl,
                                 const int32_t* seq_lens, const int32_t* block_table, int bt_stride,
                                 int B, int top_k, int window, const float* sinks,
                                 float softmax_scale, void* out, float* lse, int T, int H,
                                 hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const TopkIn tin{topk, topk_stride, topk_width, topk_lens, qsl, seq_lens, block_table,
                   bt_stride, B, top_k, window};
  return launch_items<true, false>(q, cache, num_pages, page_shift, kv_dtype, kv_scale, nullptr,
                                   0, nullptr, sinks,
                                   softmax_scale, out, lse, T, H, 1, kIdxBlock, nullptr, nullptr,
                                   tin, StepIn{}, stream);
}

hipError_t launch_attention_step(void* q, const void* kv, const int64_t* positions,
                                 const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                                 const void* q_norm_weight, float eps, uint8_t* cache,
                                 int num_pages, int page_shift, int kv_dtype, float kv_scale,
                                 const int32_t* topk,
                                 int topk_stride, int topk_width, const int32_t* topk_lens,
                                 const int32_t* qsl, const int32_t* seq_lens,
                                 const int32_t* block_table, int bt_stride, int B, int top_k,
                                 int window, const float* sinks, float softmax_scale, void* out,
                                 float* lse, int T, int H, int splits, void* workspace,
                                 hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const TopkIn tin{topk, topk_stride, topk_width, topk_lens, qsl, seq_lens, block_table,
                   bt_stride, B, top_k, window};
  const StepIn sti{static_cast<uint16_t*>(q), static_cast<const uint16_t*>(kv), positions,
                   slot_mapping, cos_sin, max_pos, static_cast<const uint16_t*>(q_norm_weight),
                   eps, cache};
  if (splits <= 1)
    return launch_items<true, true>(nullptr, nullptr, num_pages, page_shift, kv_dtype, kv_scale,
                                    nullptr, 0, nullptr,
                                    sinks, softmax_scale, out, lse, T, H, 1, kIdxBlock, nullptr,
                                    nullptr, tin, sti, stream);
  // pieces of the row as the split decode cuts a combined row of width
  // round_up(top_k + window, 128): 64-entry-aligned, trailing pieces may be empty
  const int width = (top_k + window + 127) / 128 * 128;
  const int per = (width + splits - 1) / splits;
  const int split_len = per > 0 ? ((per + kChunk - 1) / kChunk) * kChunk : kChunk;
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + (size_t)T * splits * H * kNope;
  hipError_t e = launch_items<true, true>(nullptr, nullptr, num_pages, page_shift, kv_dtype,
                                          kv_scale, nullptr, 0,
                                          nullptr, sinks, softmax_scale, out, lse, T, H, splits,
                                          split_len, part_o, part_ml, tin, sti, stream);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)T * H;
  const int merge_blocks = (int)((rows + 3) / 4);
  // the q rows, 32 per block per pass (the insert kernel's partition); positions outside
  // [0, max_pos) leave their rows untouched, and with no valid position none is touched
  const int64_t qgroups = (rows + 31) / 32;
  const int qblocks = max_pos > 0 ? (int)(qgroups < 8192 ? qgroups : 8192) : 0;
  hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)(merge_blocks + qblocks)), dim3(256), 0,
                     stream, part_o, part_ml, sinks, static_cast<uint16_t*>(out), lse, T, H,
                     splits, merge_blocks, qblocks, sti);
  return hipGetLastError();
}

static hipError_t launch_prefill_persistent(const void* q, const uint8_t* cache, int num_pages,
                                            int ps, int kv_dtype, float kv_scale,
                                            const int32_t* indices, int idx_stride,
                                            const int32_t* lens, const float* sinks,
                                            float softmax_scale, void* out, float* lse, int T,
                                            int H, int n_items, int grid, hipStream_t stream) {
  const int64_t num_slots = (int64_t)num_pages << ps;
  const float scale_log2 = softmax_scale * kLog2e * (kv_dtype == kKvFp8E4m3 ? kv_scale : 1.f);
  const float o_scale = kv_dtype == kKvFp8E4m3 ? kv_scale : 1.f;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), cache, num_slots, ps, indices, idx_stride,
                       lens, sinks, scale_log2, o_scale, static_cast<uint16_t*>(out), lse, T, H,
                       H / 32, n_items);
    return hipGetLastError();
  };
  switch (kv_dtype) {
    case kKvFp8Ds: return go(sparse_mla_prefill_kernel<kKvFp8Ds>);
    case kKvBf16: return go(sparse_mla_prefill_kernel<kKvBf16>);
    default: return go(sparse_mla_prefill_kernel<kKvFp8E4m3>);
  }
}

int auto_splits(int T, int H, int width, bool prefill) {
  // workgroups of the unsplit schedule: (token, 32 heads), or (token, 16 heads) at H = 16
  const int64_t wgs = (int64_t)T * (H == 16 ? 1 : H / 32);
  if (prefill || wgs <= 0 || wgs >= 160) return 1;
  int s = (int)(256 / wgs);
  s = s < 8 ? s : 8;                             // the merge's one-round maximum
  while (s > 1 && width < 256 * s) --s;          // pieces of at least 256 entries
  return s > 1 ? s : 1;
}

size_t attention_workspace_bytes(int T, int H, int width, bool prefill) {
  const int s = auto_splits(T, H, width, prefill);
  return s > 1 ? split_workspace_bytes(T, H, s) : 0;
}

hipError_t launch_attention(const void* q, const uint8_t* cache, int num_pages, int page_shift,
                            int kv_dtype, float kv_scale, const int32_t* indices, int idx_stride, const int32_t* lens,
                            const float* sinks, float softmax_scale, void* out, float* lse, int T,
                            int H, bool prefill, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int splits = auto_splits(T, H, idx_stride, prefill);
  if (splits > 1 && workspace && workspace_bytes >= split_workspace_bytes(T, H, splits))
    return launch_attention_split(q, cache, num_pages, page_shift, kv_dtype, kv_scale, indices,
                                  idx_stride, lens,
                                  sinks, softmax_scale, out, lse, T, H, splits, workspace, stream);
  if (prefill && H >= 32 && idx_stride <= kPIdx && kv_dtype >= 0 && kv_dtype <= 2) {
    // the persistent schedule, when the one-shot grid would run in several rounds
    static int n_cu = 0;
    if (n_cu == 0) {
      int dev = 0, v = 0;
      if (hipGetDevice(&dev) == hipSuccess &&
          hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        n_cu = v;
    }
    const int groups = H / 32;
    const int64_t n_items = 8LL * groups * ((T + 7) / 8);
    const int grid = (n_cu / 8) * 8;  // a multiple of 8: an item keeps its block id's XCD
    if (grid >= 8 && n_items > 2LL * grid && n_items < (1LL << 31))
      return launch_prefill_persistent(q, cache, num_pages, page_shift, kv_dtype, kv_scale,
                                       indices, idx_stride, lens, sinks, softmax_scale, out, lse,
                                       T, H, (int)n_items, grid, stream);
  }
  const int whole = idx_stride > 0 ? idx_stride : 1;
  return launch_items<false, false>(q, cache, num_pages, page_shift, kv_dtype, kv_scale, indices,
                                    idx_stride, lens,
                                    sinks, softmax_scale, out, lse, T, H, 1, whole, nullptr,
                                    nullptr, TopkIn{}, StepIn{}, stream);
}

// Workspace of the split decode for callers that cannot allocate: one static device array
// per GPU the library runs on (held until the process ends).  Host code never passes the
// array's name to a kernel or a copy: its host-side symbol is only a stand-in, so the
// device address is taken once per device, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attention_split(const void* q, const uint8_t* cache, int num_pages,
                                  int page_shift, int kv_dtype, float kv_scale,
                                  const int32_t* indices, int idx_stride, const int32_t* lens,
                                  const float* sinks, float softmax_scale, void* out, float* lse,
                                  int T, int H, int splits, void* workspace, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // 64-entry-aligned pieces of the row; trailing pieces may be empty
  const int per = (idx_stride + splits - 1) / splits;
  const int split_len = per > 0 ? ((per + kChunk - 1) / kChunk) * kChunk : kChunk;
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + (size_t)T * splits * H * kNope;
  hipError_t e = launch_items<false, false>(q, cache, num_pages, page_shift, kv_dtype, kv_scale,
                                            indices, idx_stride,
                                            lens, sinks, softmax_scale, out, lse, T, H, splits,
                                            split_len, part_o, part_ml, TopkIn{}, StepIn{}, stream);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)T * H;
  const int merge_blocks = (int)((rows + 3) / 4);
  hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)merge_blocks), dim3(256), 0, stream,
                     part_o, part_ml, sinks, static_cast<uint16_t*>(out), lse, T, H, splits,
                     merge_blocks, 0, StepIn{});
  return hipGetLastError();
}

}  // namespace dsv4
