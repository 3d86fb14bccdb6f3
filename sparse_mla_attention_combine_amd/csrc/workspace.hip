// The workspace addressed by the compressed-cache form of the index combine (PR #43385,
// Key source excerpts: rocm.py combine kernel with COMPRESS_RATIO, M, N, gather_lens),
// built as a cache of its own: request b owns slots M*b .. M*b+M-1; slot M*b + e (e < N)
// is a copy of compressed entry e (zero when the sequence has fewer than e+1 compressed
// entries), slot M*b + N + k a copy of the raw token at position seq_len - gather_len + k
// (k < gather_len); every other slot is a zero record.  The attention kernels then read
// it like any cache.  Records are copied as they are (FP8 codes, scales, bf16 rope), so
// the copy is exact and costs 648 B read + 648 B written per slot.
//
// One wave per workspace slot, four per 256-thread block: lanes 0..31 move the 512 code
// bytes, lanes 32..39 the 128 rope bytes, lane 40 the 8 scale bytes, 16 B / 8 B each.
#include "device.hpp"
#include "launch.hpp"

namespace dsv4 {

__global__ void __launch_bounds__(256) gather_workspace_kernel(
    const uint8_t* __restrict__ comp_cache, int64_t comp_slots, const int32_t* __restrict__ comp_bt,
    int comp_bt_stride, const uint8_t* __restrict__ swa_cache, int64_t swa_slots,
    const int32_t* __restrict__ swa_bt, int swa_bt_stride, int ps,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ gather_lens, int B,
    int ratio, int M, int N, uint8_t* __restrict__ ws, int64_t ws_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t d = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;  // workspace slot
  if (d >= ws_slots || d >= (int64_t)B * M) return;
  const int b = (int)(d / M);
  const int e = (int)(d - (int64_t)b * M);
  const int seq_len = seq_lens[b];
  const int P = 1 << ps;
  // source slot of this row, or -1 for a zero record
  const uint8_t* src = nullptr;
  int64_t s = -1;
  if (e < N) {
    if (e < seq_len / ratio) {
      const int lp = e >> ps;
      const int32_t pg = lp < comp_bt_stride ? comp_bt[(int64_t)b * comp_bt_stride + lp] : -1;
      s = pg < 0 ? -1 : ((int64_t)pg << ps) + (e & (P - 1));
      if (s >= comp_slots) s = -1;
      src = comp_cache;
    }
  } else {
    const int gl = gather_lens[b];
    const int64_t k = e - N;
    const int64_t x = (int64_t)seq_len - gl + k;  // raw position
    if (k < gl && x >= 0 && x < seq_len) {
      const int64_t lp = x >> ps;
      const int32_t pg = lp < swa_bt_stride ? swa_bt[(int64_t)b * swa_bt_stride + lp] : -1;
      s = pg < 0 ? -1 : ((int64_t)pg << ps) + (x & (P - 1));
      if (s >= swa_slots) s = -1;
      src = swa_cache;
    }
  }
  uint8_t* dpage = ws + page_base(d >> ps, ps);
  const int doff = (int)(d & (P - 1));
  if (lane < 40) {
    // 16 B pieces: codes (lanes 0..31) then rope (lanes 32..39)
    const int soff_n = lane < 32 ? 16 * lane : 0;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s >= 0) {
      const uint8_t* spage = src + page_base(s >> ps, ps);
      const int soff = (int)(s & (P - 1));
      const uint8_t* from = lane < 32 ? spage + nope_off(soff) + soff_n
                                      : spage + rope_off(soff, ps) + 16 * (lane - 32);
      v = *reinterpret_cast<const uint4*>(from);
    }
    uint8_t* to = lane < 32 ? dpage + nope_off(doff) + soff_n
                            : dpage + rope_off(doff, ps) + 16 * (lane - 32);
    *reinterpret_cast<uint4*>(to) = v;
  } else if (lane == 40) {
    uint2 v = make_uint2(0, 0);
    if (s >= 0) {
      const uint8_t* spage = src + page_base(s >> ps, ps);
      v = *reinterpret_cast<const uint2*>(spage + scale_off((int)(s & (P - 1)), ps));
    }
    *reinterpret_cast<uint2*>(dpage + scale_off(doff, ps)) = v;
  }
}

hipError_t launch_gather_workspace(const uint8_t* comp_cache, int comp_num_pages,
                                   const int32_t* comp_bt, int comp_bt_stride,
                                   const uint8_t* swa_cache, int swa_num_pages,
                                   const int32_t* swa_bt, int swa_bt_stride, int page_shift,
                                   const int32_t* seq_lens, const int32_t* gather_lens, int B,
                                   int ratio, int M, int N, uint8_t* ws, int ws_num_pages,
                                   hipStream_t stream) {
  const int64_t ws_slots = (int64_t)ws_num_pages << page_shift;
  const int64_t rows = ws_slots < (int64_t)B * M ? ws_slots : (int64_t)B * M;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_workspace_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, comp_cache, (int64_t)comp_num_pages << page_shift, comp_bt,
                     comp_bt_stride, swa_cache, (int64_t)swa_num_pages << page_shift, swa_bt,
                     swa_bt_stride, page_shift, seq_lens, gather_lens, B, ratio, M, N, ws,
                     ws_slots);
  return hipGetLastError();
}

}  // namespace dsv4
