/*
 * oracle.c — slow, plain, fp64 CPU reference of the sparse MLA hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file; only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
 * It includes no header of the HIP library and shares no code, table or constant
 * generator with it: the FP8 and bf16 codecs below are written from their published
 * definitions (OCP 8-bit floating point spec, E4M3 "fn" variant; bf16 = the top 16 bits
 * of an IEEE binary32 with round-to-nearest-even).
 *
 * Pages followed (prhub.com.cn digests of vLLM pull requests):
 *   [p1] PR #40860 "DeepSeek V4 full model support" — Implementation breakdown item 2.
 *   [p2] PR #42953 "feat: add DeepSeek-V4 XPU attention decode path" — Implementation
 *        breakdown items 4 and 6; Key source excerpts (xpu_sparse.py forward_mqa and
 *        _fused_qnorm_rope_kv_insert; xpu_sparse_decode_fp8.py dequant kernel).
 *   [p3] PR #43385 "[ROCm][DSv4][Perf] Support DeepSeek v4 MTP" — Key source excerpts
 *        (rocm.py _combine_topk_swa_indices_kernel).
 *   [p4] PR #43477 "Enable DeepSeek V4 and GLM-5.1 on SM120" — Key source excerpts
 *        (flashinfer_mla_sparse_sm120.py forward_mqa; flashinfer_sparse.py supports_sink;
 *        flashinfer_mla_sparse.py supported_kv_cache_dtypes; get_kv_cache_shape).
 *
 * Readings taken where the pages are silent are listed beside each function.
 * Every function here is pinned by the CPU test suite against closed forms, library
 * routines, invariants or brute force; none is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LATENT 576
#define NOPE 512
#define ROPE 64
#define NBLOCKS 8
#define BLOCK 64
#define RECORD 648

/* ------------------------------------------------------------------------------- */
/* Codecs                                                                          */
/* ------------------------------------------------------------------------------- */

/* OCP E4M3 ("fn") decode: sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent field 0 holds subnormals m * 2^-9.
 * Which E4M3: the XPU review debates float8e4nv vs float8e4m3fn, both OCP E4M3
 * [p2 Review highlights]. */
double oracle_e4m3_decode(int code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

/* OCP E4M3 encode with round-to-nearest, ties to even, sign kept (-0 -> 0x80).
 * Magnitudes above 448 saturate to 448 (never reached by the insert step, whose
 * inputs are scaled into [-448, 448]). */
int oracle_e4m3_encode(double x) {
  int sign = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  if (isnan(x)) return sign | 0x7F;
  if (a < 0x1p-6) { /* subnormal grid 2^-9; a result of 8 is the smallest normal */
    double m = nearbyint(ldexp(a, 9));
    return sign | (int)m;
  }
  int E = ilogb(a);                   /* a = f * 2^E, f in [1, 2) */
  double m = nearbyint(ldexp(a, 3 - E)); /* f * 8 rounded, in [8, 16] */
  if (m == 16.0) {
    m = 8.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && m > 14.0)) return sign | 0x7E;
  return sign | ((E + 7) << 3) | ((int)m - 8);
}

/* bf16 bits of a double, rounded once, to nearest, ties to even. */
uint16_t oracle_bf16_from_double(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x), r;
  if (a == 0.0) return sign;
  if (a < 0x1p-126) {
    r = ldexp(nearbyint(ldexp(a, 133)), -133); /* subnormal grid 2^-133 */
  } else {
    int E = ilogb(a);
    r = ldexp(nearbyint(ldexp(a, 7 - E)), E - 7); /* 8 significant bits */
  }
  if (r >= 0x1p128) return sign | 0x7F80;
  float f = (float)r; /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* UE8M0 block exponent: the smallest integer e with amax <= 448 * 2^e, clamped to
 * [-127, 127]; e = -127 for amax == 0.  The scale byte is e + 127 and decodes as
 * 2^(byte - 127) [p2 dequant kernel]. The choice of e is this build's reading (the
 * pages name UE8M0 scales but not how they are picked). */
int oracle_ue8m0_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int e = ilogb(amax) - 8;
  while (e < 127 && amax > ldexp(448.0, e)) ++e;
  while (e > -127 && amax <= ldexp(448.0, e - 1)) --e;
  return e;
}

/* ------------------------------------------------------------------------------- */
/* Cache record addressing (layout: pages of P slots; nope [P][512] at +0, rope bf16   */
/* [P][64] at +P*512, scales [P][8] at +P*640).  slot -> (slot / P, slot % P)          */
/* [p2 dequant kernel: block_idx and pos_in_block].                                   */
/* ------------------------------------------------------------------------------- */

static const uint8_t* rec_nope(const uint8_t* cache, int P, int64_t slot) {
  int64_t page = slot / P, off = slot % P;
  return cache + page * (int64_t)P * RECORD + off * NOPE;
}
static const uint8_t* rec_rope(const uint8_t* cache, int P, int64_t slot) {
  int64_t page = slot / P, off = slot % P;
  return cache + page * (int64_t)P * RECORD + (int64_t)P * NOPE + off * ROPE * 2;
}
static const uint8_t* rec_scale(const uint8_t* cache, int P, int64_t slot) {
  int64_t page = slot / P, off = slot % P;
  return cache + page * (int64_t)P * RECORD + (int64_t)P * (NOPE + ROPE * 2) + off * NBLOCKS;
}

static uint16_t load_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void store_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}

/* ------------------------------------------------------------------------------- */
/* Step 3 (gather + dequantise) [p2 Key source excerpts: _dequant_gather_slots_kernel] */
/* ------------------------------------------------------------------------------- */

/* One slot's 576 dequantised values as fp64 (each exactly a bf16 value after the
 * bf16 rounding of the product).  Returns 0 and writes zeros for an invalid slot
 * (negative per the page; >= num_pages*P is this build's addition). */
static int dequant_slot(const uint8_t* cache, int num_pages, int P, int64_t slot, double* out) {
  if (slot < 0 || slot >= (int64_t)num_pages * P) {
    for (int d = 0; d < LATENT; ++d) out[d] = 0.0;
    return 0;
  }
  const uint8_t* nope = rec_nope(cache, P, slot);
  const uint8_t* rope = rec_rope(cache, P, slot);
  const uint8_t* sc = rec_scale(cache, P, slot);
  for (int d = 0; d < NOPE; ++d) {
    double v = oracle_e4m3_decode(nope[d]) * ldexp(1.0, (int)sc[d / BLOCK] - 127);
    out[d] = oracle_bf16_to_double(oracle_bf16_from_double(v));
  }
  for (int i = 0; i < ROPE; ++i) out[NOPE + i] = oracle_bf16_to_double(load_u16(rope + 2 * i));
  return 1;
}

/* ------------------------------------------------------------------------------- */
/* The other kv-cache dtypes [p4 Key source excerpts: the SM100 backend lists "auto",   */
/* "float16", "bfloat16", "fp8" and "fp8_e4m3" as kv-cache dtypes (block sizes 32, 64)  */
/* and get_kv_cache_shape gives it a cache of shape (num_blocks, block_size,           */
/* head_size); the SM120 backend takes "fp8_ds_mla", the packed record above].          */
/* Readings: a slot of such a cache is one record of the 576 latent values in dim       */
/* order (head_size = 512 + 64), the records of a page back to back, so slot s starts   */
/* at byte s * record_bytes.                                                            */
/*   bf16: 1152 B, the values' bf16 bits (little-endian); value = that bf16 number.     */
/*   fp8:  576 B of OCP E4M3 codes and one fp32 scale s for the whole cache (per        */
/*         tensor); value = e4m3(code) * s.                                             */
/* ------------------------------------------------------------------------------- */

#define KV_FP8_DS 0
#define KV_BF16 1
#define KV_FP8_E4M3 2

int oracle_kv_record_bytes(int kv_dtype) {
  switch (kv_dtype) {
    case KV_FP8_DS: return RECORD;
    case KV_BF16: return LATENT * 2;
    case KV_FP8_E4M3: return LATENT;
    default: return 0;
  }
}

typedef struct {
  const uint8_t* cache;
  int num_pages, P, dtype;
  double scale; /* fp8 (per tensor) only */
} kv_view;

/* One slot's 576 values as fp64 (zeros and 0 for an invalid slot). */
static int read_slot(const kv_view* kv, int64_t slot, double* out) {
  if (kv->dtype == KV_FP8_DS) return dequant_slot(kv->cache, kv->num_pages, kv->P, slot, out);
  if (slot < 0 || slot >= (int64_t)kv->num_pages * kv->P) {
    for (int d = 0; d < LATENT; ++d) out[d] = 0.0;
    return 0;
  }
  const uint8_t* rec = kv->cache + slot * oracle_kv_record_bytes(kv->dtype);
  for (int d = 0; d < LATENT; ++d)
    out[d] = kv->dtype == KV_BF16 ? oracle_bf16_to_double(load_u16(rec + 2 * d))
                                  : oracle_e4m3_decode(rec[d]) * kv->scale;
  return 1;
}

/* The gather step's output: each slot's values rounded once to bf16 (exact for the
 * packed and bf16 caches; for fp8 the exact product code * s rounded once). */
void oracle_gather_dequant_kv(const uint8_t* cache, int num_pages, int P, int kv_dtype,
                              double kv_scale, const int32_t* slots, int n,
                              uint16_t* out_bf16 /* [n][576] */) {
  const kv_view kv = {cache, num_pages, P, kv_dtype, kv_scale};
  double row[LATENT];
  for (int i = 0; i < n; ++i) {
    read_slot(&kv, slots[i], row);
    for (int d = 0; d < LATENT; ++d) out_bf16[(int64_t)i * LATENT + d] = oracle_bf16_from_double(row[d]);
  }
}

void oracle_gather_dequant(const uint8_t* cache, int num_pages, int P, const int32_t* slots,
                           int n, uint16_t* out_bf16 /* [n][576] */) {
  oracle_gather_dequant_kv(cache, num_pages, P, KV_FP8_DS, 1.0, slots, n, out_bf16);
}

/* ------------------------------------------------------------------------------- */
/* Step 1 (combine) [p3 Key source excerpts: _combine_topk_swa_indices_kernel;        */
/* p4 forward_mqa: logical -> physical through the block table; p2 item 6: topk_lens] */
/* Readings: one cache, so the compress ratio is 1; a top-k entry is valid only when   */
/* 0 <= x <= pos (the page checks x < N); in-window top-k entries become -1 in place    */
/* (dedup, no compaction); the row tail is written with -1.                            */
/* ------------------------------------------------------------------------------- */

static int32_t phys_slot(const int32_t* block_table, int bt_stride, int b, int64_t x, int P) {
  int64_t lp = x / P;
  if (x < 0 || lp >= bt_stride) return -1;
  int32_t page = block_table[(int64_t)b * bt_stride + lp];
  if (page < 0) return -1;
  return (int32_t)((int64_t)page * P + x % P);
}

void oracle_combine(const int32_t* topk, int topk_stride, int topk_width, const int32_t* topk_lens,
                    const int32_t* qsl, const int32_t* seq_lens, const int32_t* block_table,
                    int bt_stride, int B, int T, int top_k, int window, int P, int32_t* combined,
                    int combined_stride, int32_t* combined_lens) {
  for (int b = 0; b < B; ++b) {
    int qlen = qsl[b + 1] - qsl[b];
    for (int i = 0; i < qlen; ++i) {
      int64_t t = (int64_t)qsl[b] - qsl[0] + i;
      if (t < 0 || t >= T) continue;
      int64_t pos = (int64_t)seq_lens[b] - qlen + i;
      int64_t tk = pos + 1 < top_k ? pos + 1 : top_k;
      if (topk_lens && topk_lens[t] < tk) tk = topk_lens[t];
      if (tk < 0) tk = 0;
      int64_t sw = pos + 1 < window ? pos + 1 : window;
      if (sw < 0) sw = 0;
      int64_t lo = pos - sw + 1;
      int32_t* row = combined + t * combined_stride;
      for (int64_t j = 0; j < tk; ++j) {
        int64_t x = j < topk_width ? topk[t * topk_stride + j] : -1;
        int32_t v;
        if (x < 0 || x > pos)
          v = -1;
        else if (x >= lo)
          v = -1; /* inside the window: the window part supplies it */
        else
          v = phys_slot(block_table, bt_stride, b, x, P);
        row[j] = v;
      }
      for (int64_t r = 0; r < sw; ++r) row[tk + r] = phys_slot(block_table, bt_stride, b, lo + r, P);
      for (int64_t j = tk + sw; j < combined_stride; ++j) row[j] = -1;
      combined_lens[t] = (int32_t)(tk + sw);
    }
  }
}

/* ------------------------------------------------------------------------------- */
/* Step 1, compressed-cache form [p3 Key source excerpts: the same combine kernel with */
/* COMPRESS_RATIO, M, N and gather_lens].  The indices address the rows of a per-      */
/* request workspace of M rows: request b owns rows M*b .. M*b+M-1; its first N rows   */
/* hold compressed entries 0..N-1, the next ones the last gather_lens[b] raw tokens of  */
/* the sequence, starting at position gather_start = seq_len - gather_len.  Per token  */
/* at position pos (request b):                                                         */
/*   tk = min((pos+1) / ratio, top_k[, topk_lens[t]]) (floor; at least 0),              */
/*   sw = min(pos+1, window),                                                           */
/*   row[j]    = M*b + e for j < tk, e = topk[t][j], if 0 <= e < N, else -1,            */
/*   row[tk+r] = M*b + N + (pos-sw+1+r - gather_start) for r < sw,                      */
/*   lens[t]   = tk + sw, the rest of the row -1.                                       */
/* Readings: no dedup between the two parts (they are different index spaces); a      */
/* window row outside the gathered tokens or beyond the request's M rows is -1 (the    */
/* page writes it unchecked; the two agree whenever gather_len covers the window and   */
/* N + gather_len <= M); topk_lens is optional (NULL: the page's kernel exactly).      */
/* ------------------------------------------------------------------------------- */

void oracle_combine_compressed(const int32_t* topk, int topk_stride, int topk_width,
                               const int32_t* topk_lens, const int32_t* qsl,
                               const int32_t* seq_lens, const int32_t* gather_lens, int B, int T,
                               int top_k, int ratio, int window, int M, int N, int32_t* combined,
                               int combined_stride, int32_t* combined_lens) {
  for (int b = 0; b < B; ++b) {
    int qlen = qsl[b + 1] - qsl[b];
    int64_t gather_start = (int64_t)seq_lens[b] - gather_lens[b];
    for (int i = 0; i < qlen; ++i) {
      int64_t t = (int64_t)qsl[b] - qsl[0] + i;
      if (t < 0 || t >= T) continue;
      int64_t pos = (int64_t)seq_lens[b] - qlen + i;
      int64_t tk = pos + 1 >= 0 ? (pos + 1) / ratio : 0;
      if (tk > top_k) tk = top_k;
      if (topk_lens && topk_lens[t] < tk) tk = topk_lens[t];
      if (tk < 0) tk = 0;
      int64_t sw = pos + 1 < window ? pos + 1 : window;
      if (sw < 0) sw = 0;
      int32_t* row = combined + t * combined_stride;
      for (int64_t j = 0; j < tk; ++j) {
        int64_t e = j < topk_width ? topk[t * topk_stride + j] : -1;
        row[j] = (e >= 0 && e < N) ? (int32_t)((int64_t)M * b + e) : -1;
      }
      for (int64_t r = 0; r < sw; ++r) {
        int64_t k = pos - sw + 1 + r - gather_start; /* row among the gathered tokens */
        int ok = k >= 0 && k < gather_lens[b] && N + k < M;
        row[tk + r] = ok ? (int32_t)((int64_t)M * b + N + k) : -1;
      }
      for (int64_t j = tk + sw; j < combined_stride; ++j) row[j] = -1;
      combined_lens[t] = (int32_t)(tk + sw);
    }
  }
}

/* The workspace those indices address, as a cache of its own (pages of P slots, slot */
/* M*b + e): row e < N of request b is a copy of compressed entry e (the entries       */
/* seq_len / ratio ... N-1 do not exist yet and are zero), row N + k (k < gather_len)  */
/* a copy of the raw token at position gather_start + k; rows without a source are     */
/* zero.  Compressed entry e lives in comp_cache at comp_bt[b][e / P] * P + e % P, raw */
/* position x in swa_cache at swa_bt[b][x / P] * P + x % P (a negative page or one     */
/* past the table also gives a zero row).  Readings: the page shows the indices, not   */
/* the step that fills the workspace; this is the plainest filling they imply.         */
static void copy_record(uint8_t* dst, int Pd, int64_t ds, const uint8_t* src, int Ps, int64_t ss) {
  uint8_t* dn = dst + (ds / Pd) * (int64_t)Pd * RECORD + (ds % Pd) * NOPE;
  uint8_t* dr = dst + (ds / Pd) * (int64_t)Pd * RECORD + (int64_t)Pd * NOPE + (ds % Pd) * ROPE * 2;
  uint8_t* dc = dst + (ds / Pd) * (int64_t)Pd * RECORD + (int64_t)Pd * (NOPE + ROPE * 2) + (ds % Pd) * NBLOCKS;
  if (!src) {
    memset(dn, 0, NOPE);
    memset(dr, 0, ROPE * 2);
    memset(dc, 0, NBLOCKS);
    return;
  }
  memcpy(dn, rec_nope(src, Ps, ss), NOPE);
  memcpy(dr, rec_rope(src, Ps, ss), ROPE * 2);
  memcpy(dc, rec_scale(src, Ps, ss), NBLOCKS);
}

void oracle_gather_workspace(const uint8_t* comp_cache, int comp_num_pages, const int32_t* comp_bt,
                             int comp_bt_stride, const uint8_t* swa_cache, int swa_num_pages,
                             const int32_t* swa_bt, int swa_bt_stride, int P,
                             const int32_t* seq_lens, const int32_t* gather_lens, int B, int ratio,
                             int M, int N, uint8_t* ws, int ws_num_pages) {
  for (int b = 0; b < B; ++b) {
    int64_t n_comp = seq_lens[b] / ratio;
    int64_t gather_start = (int64_t)seq_lens[b] - gather_lens[b];
    for (int64_t e = 0; e < M; ++e) {
      int64_t ds = (int64_t)M * b + e;
      if (ds >= (int64_t)ws_num_pages * P) continue;
      const uint8_t* src = NULL;
      int64_t ss = -1;
      if (e < N) {
        if (e < n_comp) {
          ss = phys_slot(comp_bt, comp_bt_stride, b, e, P);
          if (ss >= (int64_t)comp_num_pages * P) ss = -1;
          src = ss >= 0 ? comp_cache : NULL;
        }
      } else {
        int64_t k = e - N;
        int64_t x = gather_start + k;
        if (k < gather_lens[b] && x >= 0 && x < seq_lens[b]) {
          ss = phys_slot(swa_bt, swa_bt_stride, b, x, P);
          if (ss >= (int64_t)swa_num_pages * P) ss = -1;
          src = ss >= 0 ? swa_cache : NULL;
        }
      }
      copy_record(ws, P, ds, src, P, ss);
    }
  }
}

/* ------------------------------------------------------------------------------- */
/* Before step 1: the indexer's top-k selection [p1 item 2 and Key files: the MLA      */
/* layer integrates an Indexer whose top-k picks feed the sparse backend; p3 combine   */
/* kernel: top-k entries are compressed-entry ids below (pos+1) / COMPRESS_RATIO].     */
/* Per token at position pos: the candidates are ids 0 .. n-1, n = min((pos+1) /      */
/* ratio, logits_stride); the result is the set of the min(n, top_k) candidates with   */
/* the largest logits, ties going to the smaller id, listed in ascending id order,     */
/* then -1 up to topk_stride; topk_lens[t] = min(n, top_k).  Readings: the pages name  */
/* the step but not its tie rule or output order; ascending ids make the result unique */
/* (and the later gathers ordered); a NaN logit counts as -inf.                        */
/* ------------------------------------------------------------------------------- */

typedef struct {
  float v;
  int32_t id;
} scored;

static int by_score(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return x->id < y->id ? -1 : (x->id > y->id ? 1 : 0);
}

static int by_id(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}

void oracle_indexer_topk(const float* logits, int logits_stride, const int32_t* qsl,
                         const int32_t* seq_lens, int B, int T, int ratio, int top_k,
                         int32_t* topk, int topk_stride, int32_t* topk_lens) {
  scored* buf = (scored*)malloc(sizeof(scored) * (size_t)(logits_stride > 0 ? logits_stride : 1));
  for (int b = 0; b < B; ++b) {
    int qlen = qsl[b + 1] - qsl[b];
    for (int i = 0; i < qlen; ++i) {
      int64_t t = (int64_t)qsl[b] - qsl[0] + i;
      if (t < 0 || t >= T) continue;
      int64_t pos = (int64_t)seq_lens[b] - qlen + i;
      int64_t n = pos + 1 > 0 ? (pos + 1) / ratio : 0;
      if (n > logits_stride) n = logits_stride;
      for (int64_t c = 0; c < n; ++c) {
        float v = logits[t * (int64_t)logits_stride + c];
        buf[c].v = isnan(v) ? -INFINITY : v;
        buf[c].id = (int32_t)c;
      }
      qsort(buf, (size_t)n, sizeof(scored), by_score);
      int64_t k = n < top_k ? n : top_k;
      int32_t* row = topk + t * (int64_t)topk_stride;
      for (int64_t j = 0; j < k; ++j) row[j] = buf[j].id;
      qsort(row, (size_t)k, sizeof(int32_t), by_id);
      for (int64_t j = k; j < topk_stride; ++j) row[j] = -1;
      topk_lens[t] = (int32_t)k;
    }
  }
  free(buf);
}

/* ------------------------------------------------------------------------------- */
/* Step 4 (fused insert) [p2 Implementation breakdown item 4: per-head q RMSNorm,      */
/* GPT-J RoPE, FP8 UE8M0 KV insert; Key source excerpts: xpu_sparse.py calls it with   */
/* (q, kv, kv_cache, slot_mapping, positions); p1 item 2 "RMSNorm+Rope+Quant"].        */
/* Readings: RMSNorm over all 576 dims of a head with one shared weight, eps inside    */
/* the square root; GPT-J pairs (2i, 2i+1) of dims 512..575; q rounded once to bf16    */
/* after norm and rotation; kv is not normed; only the 512 nope dims are quantised;    */
/* the rotated rope dims are stored as bf16.  Position outside [0, max_pos): token     */
/* untouched; slot outside [0, num_pages*P): cache write skipped.                      */
/* ------------------------------------------------------------------------------- */

/* The cache write for the bf16 and fp8 dtypes [p4, as above]: the rope dims rotated and
 * rounded to bf16 as for the packed record (what the RoPE step hands on); bf16 stores
 * every value's bits; fp8 stores e4m3(z / s) for every dim z, the quotient rounded to
 * fp32 first (reading: the pages give no quantiser; both this and the GPU take the
 * rounding decision on the fp32 quotient), round-to-nearest-even, saturated to +-448. */
void oracle_kv_insert_kv(uint16_t* q, const uint16_t* kv, const int64_t* positions,
                         const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                         const uint16_t* weight, double eps, uint8_t* cache, int num_pages, int P,
                         int kv_dtype, double kv_scale, int T, int H) {
  double x[LATENT], y[LATENT], c[ROPE / 2], s[ROPE / 2];
  for (int64_t t = 0; t < T; ++t) {
    int64_t p = positions[t];
    if (p < 0 || p >= max_pos) continue;
    for (int i = 0; i < ROPE / 2; ++i) {
      c[i] = cos_sin[p * ROPE + i];
      s[i] = cos_sin[p * ROPE + ROPE / 2 + i];
    }
    for (int h = 0; h < H; ++h) {
      uint16_t* qh = q + (t * H + h) * LATENT;
      double ss = 0.0;
      for (int d = 0; d < LATENT; ++d) {
        x[d] = oracle_bf16_to_double(qh[d]);
        ss += x[d] * x[d];
      }
      double rms = sqrt(ss / LATENT + eps);
      for (int d = 0; d < LATENT; ++d) y[d] = x[d] / rms * oracle_bf16_to_double(weight[d]);
      for (int i = 0; i < ROPE / 2; ++i) {
        double a = y[NOPE + 2 * i], b = y[NOPE + 2 * i + 1];
        y[NOPE + 2 * i] = a * c[i] - b * s[i];
        y[NOPE + 2 * i + 1] = a * s[i] + b * c[i];
      }
      for (int d = 0; d < LATENT; ++d) qh[d] = oracle_bf16_from_double(y[d]);
    }
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= (int64_t)num_pages * P) continue;
    const uint16_t* kt = kv + t * LATENT;
    for (int d = 0; d < LATENT; ++d) x[d] = oracle_bf16_to_double(kt[d]);
    if (kv_dtype != KV_FP8_DS) {
      double z[LATENT];
      for (int d = 0; d < NOPE; ++d) z[d] = x[d];
      for (int i = 0; i < ROPE / 2; ++i) {
        double a = x[NOPE + 2 * i], b = x[NOPE + 2 * i + 1];
        z[NOPE + 2 * i] = oracle_bf16_to_double(oracle_bf16_from_double(a * c[i] - b * s[i]));
        z[NOPE + 2 * i + 1] = oracle_bf16_to_double(oracle_bf16_from_double(a * s[i] + b * c[i]));
      }
      uint8_t* rec = cache + slot * oracle_kv_record_bytes(kv_dtype);
      for (int d = 0; d < LATENT; ++d) {
        if (kv_dtype == KV_BF16)
          store_u16(rec + 2 * d, oracle_bf16_from_double(z[d]));
        else
          rec[d] = (uint8_t)oracle_e4m3_encode((double)(float)(z[d] / kv_scale));
      }
      continue;
    }
    uint8_t* rope = (uint8_t*)rec_rope(cache, P, slot);
    for (int i = 0; i < ROPE / 2; ++i) {
      double a = x[NOPE + 2 * i], b = x[NOPE + 2 * i + 1];
      store_u16(rope + 4 * i, oracle_bf16_from_double(a * c[i] - b * s[i]));
      store_u16(rope + 4 * i + 2, oracle_bf16_from_double(a * s[i] + b * c[i]));
    }
    uint8_t* nope = (uint8_t*)rec_nope(cache, P, slot);
    uint8_t* sc = (uint8_t*)rec_scale(cache, P, slot);
    for (int blk = 0; blk < NBLOCKS; ++blk) {
      double amax = 0.0;
      for (int i = 0; i < BLOCK; ++i) {
        double a = fabs(x[blk * BLOCK + i]);
        if (a > amax) amax = a;
      }
      int e = oracle_ue8m0_exponent(amax);
      sc[blk] = (uint8_t)(e + 127);
      for (int i = 0; i < BLOCK; ++i)
        nope[blk * BLOCK + i] = (uint8_t)oracle_e4m3_encode(ldexp(x[blk * BLOCK + i], -e));
    }
  }
}

void oracle_kv_insert(uint16_t* q, const uint16_t* kv, const int64_t* positions,
                      const int64_t* slot_mapping, const float* cos_sin, int max_pos,
                      const uint16_t* weight, double eps, uint8_t* cache, int num_pages, int P,
                      int T, int H) {
  oracle_kv_insert_kv(q, kv, positions, slot_mapping, cos_sin, max_pos, weight, eps, cache,
                      num_pages, P, KV_FP8_DS, 1.0, T, H);
}

/* ------------------------------------------------------------------------------- */
/* Steps 2+3 (sparse attention over the listed slots) — the plain definition:        */
/* softmax attention of each head over the valid listed slots, value = first 512 dims, */
/* optional per-head sink logit in the denominator [p2 xpu_sparse_decode_fp8: dequant  */
/* then bf16 sparse MLA with topk_lens; p4 forward_mqa output (T, H, kv_lora_rank);    */
/* p4 supports_sink].  Readings: a listed slot counts as often as it is listed; the    */
/* sink is a logit (not multiplied by the softmax scale) with no value vector; an      */
/* empty row without sink gives 0 and lse = -inf.                                      */
/* ------------------------------------------------------------------------------- */

typedef struct {
  const uint16_t* q;
  kv_view kv;
  const int32_t* idx;
  int idx_stride;
  const int32_t* lens;
  const float* sinks;
  double scale;
  double* out;
  double* lse;
  int T, H;
  int t0, t1;
} attn_job;

static void attend_token(const attn_job* jb, int t, double* K, double* sc) {
  int L = jb->lens[t];
  if (L > jb->idx_stride) L = jb->idx_stride;
  if (L < 0) L = 0;
  int n = 0;
  for (int j = 0; j < L; ++j) {
    int64_t slot = jb->idx[(int64_t)t * jb->idx_stride + j];
    if (read_slot(&jb->kv, slot, K + (int64_t)n * LATENT)) ++n;
  }
  for (int h = 0; h < jb->H; ++h) {
    const uint16_t* qh = jb->q + ((int64_t)t * jb->H + h) * LATENT;
    double qd[LATENT];
    for (int d = 0; d < LATENT; ++d) qd[d] = oracle_bf16_to_double(qh[d]);
    double z = jb->sinks ? (double)jb->sinks[h] : -INFINITY;
    double m = z;
    for (int j = 0; j < n; ++j) {
      const double* k = K + (int64_t)j * LATENT;
      double acc = 0.0;
      for (int d = 0; d < LATENT; ++d) acc += qd[d] * k[d];
      sc[j] = jb->scale * acc;
      if (sc[j] > m) m = sc[j];
    }
    double* o = jb->out + ((int64_t)t * jb->H + h) * NOPE;
    for (int c = 0; c < NOPE; ++c) o[c] = 0.0;
    if (m == -INFINITY) { /* nothing to attend, no sink */
      if (jb->lse) jb->lse[(int64_t)t * jb->H + h] = -INFINITY;
      continue;
    }
    double den = jb->sinks ? exp(z - m) : 0.0;
    for (int j = 0; j < n; ++j) {
      double w = exp(sc[j] - m);
      den += w;
      const double* v = K + (int64_t)j * LATENT;
      for (int c = 0; c < NOPE; ++c) o[c] += w * v[c];
    }
    for (int c = 0; c < NOPE; ++c) o[c] /= den;
    if (jb->lse) jb->lse[(int64_t)t * jb->H + h] = m + log(den);
  }
}

static void* attn_worker(void* arg) {
  attn_job* jb = (attn_job*)arg;
  int maxL = jb->idx_stride;
  double* K = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1) * LATENT);
  double* sc = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
  for (int t = jb->t0; t < jb->t1; ++t) attend_token(jb, t, K, sc);
  free(K);
  free(sc);
  return NULL;
}

/* out fp64 [T][H][512], lse fp64 [T][H] or NULL.  nthreads <= 1 runs on the caller's
 * thread; otherwise query tokens are split into contiguous ranges, one per thread. */
void oracle_sparse_mla_kv(const uint16_t* q, const uint8_t* cache, int num_pages, int P,
                          int kv_dtype, double kv_scale, const int32_t* idx, int idx_stride,
                          const int32_t* lens, const float* sinks, double scale, double* out,
                          double* lse, int T, int H, int nthreads) {
  attn_job base = {q, {cache, num_pages, P, kv_dtype, kv_scale}, idx, idx_stride, lens, sinks,
                   scale, out, lse, T, H, 0, T};
  if (nthreads <= 1 || T <= 1) {
    attn_worker(&base);
    return;
  }
  if (nthreads > T) nthreads = T;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  attn_job* jobs = (attn_job*)malloc(sizeof(attn_job) * nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].t0 = (int)((int64_t)T * i / nthreads);
    jobs[i].t1 = (int)((int64_t)T * (i + 1) / nthreads);
    pthread_create(&th[i], NULL, attn_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

void oracle_sparse_mla(const uint16_t* q, const uint8_t* cache, int num_pages, int P,
                       const int32_t* idx, int idx_stride, const int32_t* lens, const float* sinks,
                       double scale, double* out, double* lse, int T, int H, int nthreads) {
  oracle_sparse_mla_kv(q, cache, num_pages, P, KV_FP8_DS, 1.0, idx, idx_stride, lens, sinks,
                       scale, out, lse, T, H, nthreads);
}
