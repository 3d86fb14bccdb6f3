/*
 * dsv4.h — C ABI of the MI355X (gfx950) sparse MLA hot path for DeepSeek-V4-style
 * attention over an FP8 paged latent KV cache.
 *
 * Sources (the four prhub.com.cn digests of vLLM pull requests):
 *   [p1] PR #40860 "DeepSeek V4 full model support" — Implementation breakdown, item 2
 *        (MLA wrapper calls a fused RMSNorm+RoPE+Quant kernel; indexer + sparse SWA backend).
 *   [p2] PR #42953 "feat: add DeepSeek-V4 XPU attention decode path" — Implementation
 *        breakdown, items 4 and 6; Key source excerpts (xpu_sparse.py forward_mqa,
 *        xpu_sparse_decode_fp8.py _dequant_gather_slots_kernel); Review highlights (FP8 type).
 *   [p3] PR #43385 "[ROCm][DSv4][Perf] Support DeepSeek v4 MTP" — Implementation breakdown,
 *        item 3; Key source excerpts (rocm.py _combine_topk_swa_indices_kernel).
 *   [p4] PR #43477 "Enable DeepSeek V4 and GLM-5.1 on SM120" — Key source excerpts
 *        (flashinfer_mla_sparse_sm120.py forward_mqa; flashinfer_sparse.py supports_sink,
 *        get_kv_cache_shape; flashinfer_mla_sparse.py supported_kv_cache_dtypes;
 *        supported kernel block sizes).
 *
 * Geometry (fixed): latent D = 576 = 512 no-PE ("nope") + 64 RoPE dims; value/output
 * Dv = kv_lora_rank = 512 [p4 forward_mqa output shape (T, H, kv_lora_rank)].
 *
 * ---------------------------------------------------------------------------------
 * KV cache byte layout (this library's own specification; the pages name the content
 * of a record but give no byte order, and disagree across architectures [p2 Motivation
 * vs p4 get_kv_cache_shape]).  The cache is an array of pages of P slots each
 * (P = page_size: 32, 64 or 256 [p4 get_supported_kernel_block_sizes: 32 and 64 for one
 * backend, 256 for the other]).  Page p starts at byte p * P * 648 and holds
 *     +0          nope codes  uint8 [P][512]   FP8 OCP E4M3 ("e4m3fn", max 448)
 *     +P*512      rope values bf16  [P][64]    stored already rotated
 *     +P*640      scale bytes uint8 [P][8]     UE8M0, one per 64 nope dims
 * Slot s lives in page s / P at row s % P [p2 dequant kernel: block_idx / pos_in_block].
 * Dequantised nope value d of slot s = e4m3(code) * 2^(scale[d/64] - 127) [p2 dequant
 * kernel], which is exactly representable in bf16.  648 bytes per token record.
 * This is kv_dtype DSV4_KV_FP8_DS_MLA [p4: the "fp8_ds_mla" cache of the SM120 backend].
 *
 * Other kv-cache dtypes [p4 Key source excerpts: the SM100 backend's supported kv-cache
 * dtypes "auto" / "bfloat16" / "fp8" / "fp8_e4m3", block sizes 32 and 64, and its cache
 * shape (num_blocks, block_size, head_size)]: a slot holds one record of the 576 values
 * in dim order, the records of a page back to back, so slot s starts at byte
 * s * record_bytes (page p at p * P * record_bytes):
 *   DSV4_KV_BF16      1152 B: the 576 values as bf16 (rope dims stored rotated).
 *   DSV4_KV_FP8_E4M3   576 B: OCP E4M3 codes of value / kv_scale, one fp32 scale
 *                     kv_scale for the whole cache (per tensor, a host argument):
 *                     value = e4m3(code) * kv_scale.
 * The entry points that read or write a cache take (kv_dtype, kv_scale) right after
 * page_size; kv_scale is used by DSV4_KV_FP8_E4M3 only and must lie in [2^-64, 2^64]
 * there (DSV4_ERR_SHAPE otherwise); an unknown kv_dtype is DSV4_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------------------
 *
 * Conventions for every entry point:
 *  - All array pointers are device pointers owned by the caller.  The library never
 *    allocates, frees or synchronises; it enqueues kernels on `stream` (a hipStream_t,
 *    NULL = the legacy default stream) and returns.  Results are visible after the
 *    stream is synchronised.
 *  - Host-side argument checks run before any launch.  On failure the call returns a
 *    non-zero dsv4_status, sets a thread-local reason string (dsv4_last_error) and
 *    touches no memory [p4 supports_combination returns a reason string].
 *  - A launch failure returns DSV4_ERR_HIP with the HIP error text as the reason.
 *  - Bad values inside device arrays are defined behaviour, never faults: out-of-range
 *    slots, -1 entries, entries at or beyond a row's length and causally invalid top-k
 *    entries contribute nothing; out-of-range positions leave a token untouched.
 *  - Non-finite floating inputs give unspecified (but memory-safe) results.
 *  - Calls on one stream are ordered; calls on different streams that touch the same
 *    buffers must be ordered by the caller.
 */
#ifndef DSV4_H_
#define DSV4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSV4_LATENT_DIM 576
#define DSV4_NOPE_DIM 512
#define DSV4_ROPE_DIM 64
#define DSV4_SCALE_BLOCK 64
#define DSV4_RECORD_BYTES 648
#define DSV4_KV_FP8_DS_MLA 0 /* the packed FP8/UE8M0 record above (648 B)          */
#define DSV4_KV_BF16 1       /* 576 bf16 values per slot (1152 B)                   */
#define DSV4_KV_FP8_E4M3 2   /* 576 E4M3 codes per slot (576 B), per-tensor scale   */
#define DSV4_COMBINE_ALIGN 128 /* [p3 rocm.py: top-k rows padded to a multiple of 128] */

typedef enum {
  DSV4_OK = 0,
  DSV4_ERR_NULL = 1,        /* a required pointer is NULL                         */
  DSV4_ERR_SHAPE = 2,       /* a size or stride is negative or inconsistent       */
  DSV4_ERR_ALIGN = 3,       /* a pointer is not aligned as documented             */
  DSV4_ERR_UNSUPPORTED = 4, /* a valid but unsupported configuration (H, P, ...)  */
  DSV4_ERR_WORKSPACE = 5,   /* the caller's workspace is missing or too small     */
  DSV4_ERR_HIP = 6          /* the HIP runtime reported an error at launch        */
} dsv4_status;

/* Name of a status code ("DSV4_OK", ...). Never NULL. */
const char* dsv4_status_str(int status);

/* Reason for the last failing call on this thread ("" after a successful call).
 * The pointer stays valid until the next dsv4_* call on the same thread. */
const char* dsv4_last_error(void);

/* Bytes of one cache page of `page_size` slots of kv_dtype (page_size * 648, 1152 or 576),
 * 0 if page_size <= 0 or kv_dtype is unknown. */
size_t dsv4_cache_page_bytes(int page_size, int kv_dtype);

/*
 * dsv4_kv_insert — fused per-head q RMSNorm + GPT-J RoPE, and FP8/UE8M0 insert of the
 * new latent rows into the cache [p2 Implementation breakdown item 4: fused q per-head
 * RMSNorm, GPT-J RoPE and FP8 UE8M0 KV insert; Key source excerpts xpu_sparse.py
 * _fused_qnorm_rope_kv_insert(q, kv, positions) writing at slot_mapping; p1 item 2].
 *
 *   q            bf16 [T][H][576], updated in place:
 *                  y = x / sqrt(mean(x^2) + eps) * w   over all 576 dims of a head,
 *                  then dims 512..575 rotated in GPT-J (interleaved) pairs
 *                  (y[512+2i], y[513+2i]) -> (a*c_i - b*s_i, a*s_i + b*c_i),
 *                  rounded once to bf16.
 *   kv           bf16 [T][576] (read only): dims 512..575 rotated the same way and
 *                  stored as bf16; dims 0..511 split into 8 blocks of 64, each block
 *                  stored as E4M3 codes of k * 2^-e with scale byte e + 127, where e is
 *                  the smallest integer with max|k| <= 448 * 2^e (clamped to [-127,127],
 *                  e = -127 for an all-zero block); round to nearest even, sign kept.
 *   positions    int64 [T]; cos_sin fp32 [max_pos][64] = cos[32] | sin[32] per
 *                  position (caller supplies the table). A token whose position is
 *                  outside [0, max_pos) is left untouched (q and cache).
 *   slot_mapping int64 [T]; the cache row written for token t; a value outside
 *                  [0, num_pages*page_size) (e.g. -1) skips the cache write only.
 *                  Duplicate slots: one of the writers wins (unspecified which).
 *   q_norm_weight bf16 [576], shared by all heads.
 *   kv_cache     uint8, num_pages pages in the layout above (16-byte aligned).
 *   kv_dtype, kv_scale  the cache's dtype.  The packed dtype stores the kv row as
 *                  above; DSV4_KV_BF16 stores dims 0..511 as given and the rotated rope
 *                  dims as bf16; DSV4_KV_FP8_E4M3 takes those same 576 bf16 values z and
 *                  stores e4m3(z / kv_scale), the quotient correctly rounded in fp32,
 *                  saturated to +-448, round to nearest even.
 * Supported: page_size in {32, 64, 256}, H in 1..128, T >= 0 (T == 0 is a no-op).
 * Alignment: q, kv, kv_cache 16-byte aligned.
 */
int dsv4_kv_insert(void* q, const void* kv, const int64_t* positions,
                   const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                   const void* q_norm_weight, float eps, uint8_t* kv_cache, int num_pages,
                   int page_size, int kv_dtype, float kv_scale, int T, int H, void* stream);

/*
 * dsv4_combine_indices — merge each query token's indexer top-k with its sliding
 * window into one index row, deduplicated, mapped to physical cache slots and padded
 * with -1 [p3 Key source excerpts: rocm.py _combine_topk_swa_indices_kernel;
 * p4 forward_mqa: per-request logical index -> physical slot through the block table;
 * p2 Implementation breakdown item 6: per-row topk_lens].
 *
 * For request b with qlen = qsl[b+1]-qsl[b] query tokens, its i-th token
 * t = qsl[b]-qsl[0]+i sits at position pos = seq_lens[b]-qlen+i and gets
 *   tk = max(0, min(pos+1, top_k, topk_lens[t] if topk_lens)),  sw = max(0, min(pos+1, window)),
 *   combined[t][j]    = phys(b, topk[t][j]) for j < tk, or -1 if that entry is < 0, > pos,
 *                       inside the window [pos-sw+1, pos] (the window supplies it), or
 *                       at a column >= topk_width;
 *   combined[t][tk+r] = phys(b, pos-sw+1+r) for r < sw (window, ascending);
 *   combined[t][j]    = -1 for tk+sw <= j < combined_stride;
 *   combined_lens[t]  = tk + sw,
 * where phys(b, x) = block_table[b][x/P]*P + x%P, or -1 if x/P >= block_table_stride or
 * the table entry is negative.  Tokens t >= T are skipped; rows of tokens that belong to
 * no request are not written.
 *   topk            int32 [T][topk_stride], topk_width <= topk_stride valid columns
 *   topk_lens       int32 [T] or NULL
 *   query_start_loc int32 [B+1]; seq_lens int32 [B]
 *   block_table     int32 [B][block_table_stride] (physical page ids)
 *   combined        int32 [T][combined_stride], combined_lens int32 [T]
 * Requires combined_stride >= round_up(top_k + window, 128) and top_k <= topk_width.
 */
int dsv4_combine_indices(const int32_t* topk, int topk_stride, int topk_width,
                         const int32_t* topk_lens, const int32_t* query_start_loc,
                         const int32_t* seq_lens, const int32_t* block_table,
                         int block_table_stride, int B, int T, int top_k, int window,
                         int page_size, int32_t* combined, int combined_stride,
                         int32_t* combined_lens, void* stream);

/*
 * dsv4_indexer_topk — the indexer's top-k selection that feeds the combine step
 * [p1 Implementation breakdown item 2 and Key files: the MLA layer integrates an Indexer
 * whose picks feed the sparse backend; p3 combine kernel: top-k ids are compressed
 * entries below (pos+1) / COMPRESS_RATIO].  For request b's i-th token t, at
 * pos = seq_lens[b]-qlen+i, the candidates are ids 0..n-1 with
 * n = min((pos+1) / compress_ratio, logits_stride) (floor; 0 when pos < 0):
 *   topk[t][0..k)   = the k = min(n, top_k) ids with the largest logits[t][id], ties
 *                     to the smaller id, a NaN counting as -inf, in ascending id order;
 *   topk[t][k..)    = -1 up to topk_stride;   topk_lens[t] = k.
 * (The pages name the step, not its tie rule or order: ascending ids make the result
 * unique.)  Tokens of no request are not written.  The output is the topk / topk_lens
 * input of dsv4_combine_indices (compress_ratio 1: ids are positions) and of
 * dsv4_combine_indices_compressed.
 *   logits int32-aligned fp32 [T][logits_stride]; topk int32 [T][topk_stride] (may be
 *   NULL when topk_stride is 0);
 *   topk_lens int32 [T]; query_start_loc int32 [B+1]; seq_lens int32 [B]
 * Requires compress_ratio >= 1, topk_stride >= top_k >= 0.
 */
int dsv4_indexer_topk(const float* logits, int logits_stride, const int32_t* query_start_loc,
                      const int32_t* seq_lens, int B, int T, int compress_ratio, int top_k,
                      int32_t* topk, int topk_stride, int32_t* topk_lens, void* stream);

/*
 * dsv4_combine_indices_compressed — the combine step for a compressed KV cache, where
 * top-k picks compressed entries and the window picks raw tokens: two index spaces
 * [p3 Key source excerpts: rocm.py combine kernel with COMPRESS_RATIO, M, N and
 * gather_lens].  The output indexes a per-request workspace of M rows (request b owns
 * rows M*b .. M*b+M-1: N compressed entries, then the last gather_lens[b] raw tokens of
 * the sequence, from position gather_start = seq_lens[b] - gather_lens[b]); see
 * dsv4_gather_workspace.  For request b's i-th token, at pos = seq_lens[b]-qlen+i:
 *   tk = max(0, min((pos+1) / compress_ratio, top_k, topk_lens[t] if topk_lens)),
 *   sw = max(0, min(pos+1, window)),
 *   combined[t][j]    = M*b + e for j < tk, e = topk[t][j], if 0 <= e < N, else -1;
 *   combined[t][tk+r] = M*b + N + k for r < sw, k = pos-sw+1+r - gather_start, or -1
 *                       when k < 0, k >= gather_lens[b] or N + k >= M;
 *   combined[t][j]    = -1 past tk+sw;  combined_lens[t] = tk + sw.
 * No dedup between the parts (different index spaces).  Arrays as for
 * dsv4_combine_indices, plus gather_lens int32 [B].  Requires compress_ratio >= 1,
 * 0 <= N <= M, B*M < 2^31, top_k <= topk_width, combined_stride >= round_up(top_k +
 * window, 128); errors otherwise as for dsv4_combine_indices.
 */
int dsv4_combine_indices_compressed(const int32_t* topk, int topk_stride, int topk_width,
                                    const int32_t* topk_lens, const int32_t* query_start_loc,
                                    const int32_t* seq_lens, const int32_t* gather_lens, int B,
                                    int T, int top_k, int compress_ratio, int window, int M, int N,
                                    int32_t* combined, int combined_stride, int32_t* combined_lens,
                                    void* stream);

/*
 * dsv4_gather_workspace — fills the workspace the compressed-form indices address, as a
 * cache of its own (ws_num_pages pages of page_size slots, the layout above; slot M*b+e
 * for row e of request b), so that dsv4_sparse_mla_prefill / _decode run over it with
 * those indices as slots [p3 Key source excerpts: the workspace rows M*b + ... of the
 * combine kernel; the page shows the indices, the filling is their plain reading]:
 *   e < N:      compressed entry e of request b, read from comp_cache at slot
 *               comp_block_table[b][e/P]*P + e%P, if e < seq_lens[b] / compress_ratio
 *               (the entries that exist), else a zero record;
 *   e = N + k:  the raw token at x = seq_lens[b] - gather_lens[b] + k, read from
 *               swa_cache at swa_block_table[b][x/P]*P + x%P, for k < gather_lens[b]
 *               and 0 <= x < seq_lens[b], else a zero record.
 * A negative page, a page index past the table's stride or a slot past the source
 * cache also give a zero record.  Records are copied exactly (codes, scales, rope).
 * Workspace slots >= B*M, and all of ws_cache past ws_num_pages pages, are untouched.
 *   comp_cache / swa_cache  caches of comp_num_pages / swa_num_pages pages (may be the
 *                           same buffer); block tables int32 [B][stride]
 *   seq_lens, gather_lens   int32 [B]
 * Requires page_size in {32, 64, 256} (all three caches), compress_ratio >= 1,
 * 0 <= N <= M, B*M < 2^31, 16-byte aligned caches.
 */
int dsv4_gather_workspace(const uint8_t* comp_cache, int comp_num_pages,
                          const int32_t* comp_block_table, int comp_bt_stride,
                          const uint8_t* swa_cache, int swa_num_pages,
                          const int32_t* swa_block_table, int swa_bt_stride, int page_size,
                          const int32_t* seq_lens, const int32_t* gather_lens, int B,
                          int compress_ratio, int M, int N, uint8_t* ws_cache, int ws_num_pages,
                          void* stream);

/*
 * dsv4_sparse_mla_decode — sparse MQA-form MLA attention of every head over the
 * listed cache slots [p2 Key source excerpts xpu_sparse_decode_fp8: dequantise the
 * gathered FP8 slots, then bf16 sparse MLA with topk_lens; p4 forward_mqa: output
 * (T, H, kv_lora_rank) from physical indices; p4 supports_sink].  For token t, head h:
 *   J      = { j < min(lens[t], idx_stride) : 0 <= indices[t][j] < num_pages*page_size }
 *            (a multiset: a repeated slot counts twice),
 *   K_j    = the 576 values of slot indices[t][j] (dequantised for the FP8 dtypes:
 *            e4m3(code) * 2^(scale-127), or e4m3(code) * kv_scale),  V_j = K_j[0:512],
 *   s_j    = softmax_scale * <q[t][h], K_j>,   z = sinks[h] (absent: -inf),
 *   m      = max(z, max_j s_j),  den = e^(z-m) + sum_j e^(s_j-m),
 *   out[t][h] = sum_j e^(s_j-m) V_j / den  (0 when den == 0),
 *   lse[t][h] = m + ln(den)  (-inf when den == 0).
 * The sink adds to the denominator only (logit units, not multiplied by softmax_scale).
 *   q        bf16 [T][H][576];  out bf16 [T][H][512];  lse fp32 [T][H] or NULL
 *   indices  int32 [T][idx_stride];  lens int32 [T];  sinks fp32 [H] or NULL
 * Arithmetic: bf16 operands, fp32 accumulation, probabilities rounded to bf16 for the
 * value product (the per-tensor fp8 scale multiplies the scores' scale and the output
 * instead of each value).  Supported: H in {16, 32, 64, 128}, page_size in {32, 64, 256},
 * every kv_dtype.
 * Alignment: q, out, kv_cache 16-byte aligned; indices 4-byte aligned.
 *
 * Workspace [p2 Review highlights: no allocation on the decode path, so scratch memory
 * is the caller's]: `workspace` may be NULL with workspace_bytes 0, and the call then
 * runs one workgroup per (token, head group).  Given at least
 * dsv4_sparse_mla_workspace_bytes(T, H, idx_stride, 0) bytes (16-byte aligned), a batch
 * too small to fill the GPU has its rows cut into pieces merged by their log-sum-exp, as
 * dsv4_sparse_mla_decode_split does with the piece count that function reports; the
 * result is the same up to rounding order.  The workspace carries nothing between calls;
 * calls sharing one workspace on different streams race.  A non-NULL workspace that is
 * misaligned or smaller than that size, or a NULL one with workspace_bytes != 0, is
 * DSV4_ERR_WORKSPACE.
 */
int dsv4_sparse_mla_decode(const void* q, const uint8_t* kv_cache, int num_pages,
                           int page_size, int kv_dtype, float kv_scale, const int32_t* indices,
                           int idx_stride, const int32_t* lens, const float* sinks,
                           float softmax_scale, void* out, float* lse, int T, int H,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsv4_sparse_mla_workspace_bytes — device workspace bytes that dsv4_sparse_mla_decode
 * (is_prefill 0) or dsv4_sparse_mla_prefill (is_prefill 1) may use for T query tokens,
 * H heads and index rows of `width` entries (idx_stride).  0 when the call's schedule
 * needs none: a decode batch that fills the GPU (T * H / 32 >= 160 workgroups) and every
 * prefill.  Otherwise the split workspace of the piece count the decode picks
 * (min(8, 256 / (T * max(1, H / 32))), lowered until every piece holds >= 256 entries).
 * Returns 0 for T < 0, width < 0 or an unsupported H.
 */
size_t dsv4_sparse_mla_workspace_bytes(int T, int H, int width, int is_prefill);

/*
 * dsv4_sparse_mla_decode_topk — dsv4_combine_indices followed by dsv4_sparse_mla_decode
 * in one launch: each workgroup builds its token's combined index row in LDS from the
 * combine step's inputs and attends over it, so the combined rows never go through
 * memory [p3 combine kernel + p4 forward_mqa, the same two steps].  The result (out, lse)
 * is the decode's on the rows dsv4_combine_indices would write; a token that belongs to
 * no request gets an empty row (out 0; lse -inf, or the sink alone).  Arguments: those of the two entry
 * points (the combine's topk / topk_lens / query_start_loc / seq_lens / block_table / B /
 * top_k / window, the decode's q / cache / sinks / scale / out / lse / T / H); no
 * combined_stride, since the row lives in LDS.  Requires top_k + window <= 4096
 * (DSV4_ERR_UNSUPPORTED otherwise) and what both entry points require.
 */
int dsv4_sparse_mla_decode_topk(const void* q, const uint8_t* kv_cache, int num_pages, int page_size,
                                int kv_dtype, float kv_scale, const int32_t* topk,
                                int topk_stride, int topk_width,
                                const int32_t* topk_lens, const int32_t* query_start_loc,
                                const int32_t* seq_lens, const int32_t* block_table,
                                int block_table_stride, int B, int top_k, int window,
                                const float* sinks, float softmax_scale, void* out, float* lse,
                                int T, int H, void* stream);

/*
 * dsv4_sparse_mla_decode_step — dsv4_kv_insert followed by dsv4_sparse_mla_decode_topk in
 * one launch, the whole decode step of the layer [p2 Implementation breakdown item 4, the
 * fused insert, feeding the sparse decode of Key source excerpts xpu_sparse_decode_fp8;
 * p3 combine kernel; p4 forward_mqa].  Each workgroup normalises and rotates its own q
 * heads (written back to q in place, as dsv4_kv_insert does) and quantises into the cache
 * the new latent rows of its request's tokens up to its own before it attends; a token of
 * no request inserts its own row only.  Arguments: those of dsv4_kv_insert (q, kv,
 * positions, slot_mapping, cos_sin / max_pos, q_norm_weight, eps, kv_cache) and of
 * dsv4_sparse_mla_decode_topk, in that order, sharing the cache and T / H.
 * Precondition for the result (q, cache bytes, out, lse) to equal the two calls in
 * sequence: a slot read by a token's combined row is written in this call only by
 * tokens of the same request at positions up to the token's own, i.e. slot_mapping and
 * positions agree with the block tables and the positions the combine derives from
 * query_start_loc and seq_lens, as in a decode step.  The inserted rows of a request are
 * quantised by every workgroup of each of its tokens (a request of n new tokens does
 * O(n^2) row insertions): meant for decode batches of a few tokens per request (MTP);
 * prefill-sized requests use the two entry points, and T > 64 * max(B, 1) is refused
 * with DSV4_ERR_UNSUPPORTED.  Requires what both entry points require.
 */
int dsv4_sparse_mla_decode_step(void* q, const void* kv, const int64_t* positions,
                                const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                                const void* q_norm_weight, float eps, uint8_t* kv_cache,
                                int num_pages, int page_size, int kv_dtype, float kv_scale,
                                const int32_t* topk, int topk_stride, int topk_width,
                                const int32_t* topk_lens,
                                const int32_t* query_start_loc, const int32_t* seq_lens,
                                const int32_t* block_table, int block_table_stride, int B,
                                int top_k, int window, const float* sinks, float softmax_scale,
                                void* out, float* lse, int T, int H, void* stream);

/*
 * dsv4_sparse_mla_decode_step_split — dsv4_sparse_mla_decode_step with each token's row
 * cut into `splits` pieces attended by separate workgroups and merged by their
 * log-sum-exp (the split decode's merge), for small batches where one workgroup per
 * (token, head group) leaves compute units idle.  The pieces are those
 * dsv4_sparse_mla_decode_split cuts from a combined row of width
 * round_up(top_k + window, 128), so out and lse equal dsv4_kv_insert +
 * dsv4_combine_indices (combined_stride = that width) + dsv4_sparse_mla_decode_split with
 * the same splits; q and the cache bytes equal dsv4_sparse_mla_decode_step's.  Every
 * piece reads the raw q rows; the merge launch, enqueued after all pieces, writes the
 * normalised rows back in place (a piece never writes q, since the pieces of one row
 * run at different times and a later one would otherwise read a normalised row).
 *   splits     1..64 (1: dsv4_sparse_mla_decode_step, no workspace)
 *   workspace  caller-owned device memory of at least
 *              dsv4_sparse_mla_split_workspace_bytes(T, H, splits) bytes, 16-byte
 *              aligned (DSV4_ERR_WORKSPACE otherwise); it carries nothing between calls
 * Other arguments and requirements as for dsv4_sparse_mla_decode_step.
 */
int dsv4_sparse_mla_decode_step_split(
    void* q, const void* kv, const int64_t* positions, const int64_t* slot_mapping,
    const float* cos_sin, int max_pos, const void* q_norm_weight, float eps, uint8_t* kv_cache,
    int num_pages, int page_size, int kv_dtype, float kv_scale, const int32_t* topk,
    int topk_stride, int topk_width, const int32_t* topk_lens, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int block_table_stride, int B, int top_k,
    int window, const float* sinks, float softmax_scale, void* out, float* lse, int T, int H,
    int splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsv4_sparse_mla_prefill — the same result as dsv4_sparse_mla_decode, scheduled for
 * many query tokens per call (prefill: each token of a long sequence attends its own
 * combined index row) [p3 Motivation/Implementation breakdown: sparse prefill index
 * combining; p4 decoder self-attention].  Same arguments, contract and limits; its
 * schedule needs no workspace (dsv4_sparse_mla_workspace_bytes(T, H, width, 1) == 0),
 * so NULL / 0 is the usual argument.
 */
int dsv4_sparse_mla_prefill(const void* q, const uint8_t* kv_cache, int num_pages,
                            int page_size, int kv_dtype, float kv_scale, const int32_t* indices,
                            int idx_stride, const int32_t* lens, const float* sinks,
                            float softmax_scale, void* out, float* lse, int T, int H,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsv4_sparse_mla_split_workspace_bytes — bytes of device workspace that
 * dsv4_sparse_mla_decode_split needs for T query tokens, H heads and `splits` pieces per
 * row: T * splits * H * 514 * 4 (fp32 partial outputs, maxima and denominators).
 * Returns 0 for a negative argument.
 */
size_t dsv4_sparse_mla_split_workspace_bytes(int T, int H, int splits);

/*
 * dsv4_sparse_mla_decode_split — the result of dsv4_sparse_mla_decode for batches too
 * small to fill the GPU, where one workgroup per (token, head group) leaves most compute
 * units idle [p4 forward_mqa: decode returns (output, None) where an lse would go; the
 * lse output makes the pieces mergeable].  Each token's row is cut into `splits`
 * contiguous pieces of a multiple of 64 entries; every (token, head group, piece) runs as
 * its own workgroup and leaves, per head, the unnormalised output, its reference maximum
 * and its denominator in `workspace`; a merge pass then forms
 *   M = max(z, max_s m_s),  den = e^(z-M) + sum_s l_s e^(m_s-M),
 *   out = sum_s O_s e^(m_s-M) / den,  lse = M + ln(den),
 * which is the same result as the unsplit call up to rounding order.
 *   Arguments as dsv4_sparse_mla_decode, plus
 *   splits     1..64 (1 runs the unsplit path and needs no workspace);
 *   workspace  caller-owned device memory of at least
 *              dsv4_sparse_mla_split_workspace_bytes(T, H, splits) bytes, 16-byte
 *              aligned; overwritten by the call; calls that share one workspace on
 *              different streams race.
 * Errors: DSV4_ERR_SHAPE for splits outside 1..64, DSV4_ERR_WORKSPACE for a NULL,
 * misaligned or too small workspace, and everything dsv4_sparse_mla_decode checks.
 */
int dsv4_sparse_mla_decode_split(const void* q, const uint8_t* kv_cache, int num_pages,
                                 int page_size, int kv_dtype, float kv_scale,
                                 const int32_t* indices, int idx_stride, const int32_t* lens,
                                 const float* sinks, float softmax_scale, void* out, float* lse,
                                 int T, int H, int splits, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * dsv4_sparse_mla_decode_split_noalloc — dsv4_sparse_mla_decode_split for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels, with the workspace in a static
 * device array that the library holds on each GPU it runs on until the process ends
 * (DSV4_NOALLOC_SCRATCH_BYTES = 32 MiB per GPU).  The call allocates nothing.
 *   Arguments as dsv4_sparse_mla_decode_split, without workspace / workspace_bytes.
 *   Result: bit-identical to dsv4_sparse_mla_decode_split with the same splits.
 *   Limit: dsv4_sparse_mla_split_workspace_bytes(T, H, splits) <= 32 MiB (e.g. 256
 *   workgroups' worth of pieces at H >= 32: T * splits <= 63 at H = 128), else
 *   DSV4_ERR_WORKSPACE with nothing launched.
 *   Every call on one GPU shares that GPU's array (the contents of the last call stay
 *   there; nothing in it needs to start at zero): calls that overlap on one GPU, i.e. on
 *   different streams without ordering, race and give wrong results.
 * Errors: as dsv4_sparse_mla_decode_split; DSV4_ERR_HIP if the array's device address
 * cannot be obtained.
 */
#define DSV4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int dsv4_sparse_mla_decode_split_noalloc(const void* q, const uint8_t* kv_cache, int num_pages,
                                         int page_size, int kv_dtype, float kv_scale,
                                         const int32_t* indices, int idx_stride,
                                         const int32_t* lens, const float* sinks,
                                         float softmax_scale, void* out, float* lse, int T, int H,
                                         int splits, void* stream);

/*
 * dsv4_gather_dequant — gather + dequantise slots into bf16 rows [p2 Key source
 * excerpts: _dequant_gather_slots_kernel, one program per slot; a negative slot gives
 * a zero row; FP8 -> fp32 times 2^(byte-127) -> bf16; the bf16 RoPE part is copied].
 * Slots >= num_pages*page_size also give zero rows.  The attention entry points fuse
 * this step; it is exported as a separately testable step.  DSV4_KV_BF16 records are
 * copied; DSV4_KV_FP8_E4M3 values are e4m3(code) * kv_scale rounded once to bf16.
 *   slots int32 [n];  out bf16 [n][576]
 */
int dsv4_gather_dequant(const uint8_t* kv_cache, int num_pages, int page_size, int kv_dtype,
                        float kv_scale, const int32_t* slots, int n, void* out, void* stream);

/*
 * ---------------------------------------------------------------------------------
 * Measurement probes (not steps of the method).  The roofline of each kernel is
 * reported against the chip's published peaks and, separately, against the peaks these
 * probes reach on the GPU at hand.
 *
 * dsv4_peak_mfma — matrix-core throughput: `workgroups` workgroups of 4 waves, each wave
 * issuing iters x 8 dense bf16 MFMAs with fp32 accumulation on 8 independent
 * accumulators (shape 0: v_mfma_f32_32x32x16_bf16, the P.V shape; shape 1:
 * v_mfma_f32_16x16x32_bf16, the QK^T shape).  Every lane holds the operands
 * a_i = (i + 1) / 8, b_i = 1 / 8 and accumulator k starts at k, so sink[j] =
 * 448 + 144 * iters (shape 0) or 112 + 72 * iters (shape 1) exactly.
 *   sink float [workgroups * 256] (device);  *flops (host) = the launch's dense FLOPs.
 *   workgroups in [1, 65536], iters in [1, 2^20]; shape outside {0, 1} is
 *   DSV4_ERR_UNSUPPORTED.
 *
 * dsv4_peak_stream — HBM throughput: reads `bytes` (a multiple of 16) from src in 16-byte
 * units, grid-stride over `workgroups` x 256 threads; dst == NULL: read only, sink[j] =
 * the xor of every 32-bit word thread j read; else copies src to dst (sink[j] = 0).
 *   src, dst 16-byte aligned device buffers; sink uint32 [workgroups * 256] (device).
 * ---------------------------------------------------------------------------------
 */
int dsv4_peak_mfma(int shape, int workgroups, int iters, float* sink, double* flops,
                   void* stream);
int dsv4_peak_stream(const void* src, void* dst, size_t bytes, uint32_t* sink, int workgroups,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSV4_H_ */
