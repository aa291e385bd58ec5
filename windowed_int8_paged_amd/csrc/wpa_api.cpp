// C ABI of the library: host-side validation, then the kernel launchers.
// Every check runs before anything is enqueued, so a nonzero status means no
// work was queued and no output was touched.

#include <cmath>
#include <cstdint>

#include "wpa.h"
#include "wpa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long ceil_div(long a, long b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

const char* wpa_status_string(wpa_status s) {
  switch (s) {
    case WPA_OK: return "WPA_OK";
    case WPA_ERR_NULL: return "WPA_ERR_NULL: a required pointer is NULL";
    case WPA_ERR_SHAPE: return "WPA_ERR_SHAPE: a size, count or scale is out of range";
    case WPA_ERR_UNSUPPORTED: return "WPA_ERR_UNSUPPORTED: dtype, alignment or a size limit";
    case WPA_ERR_LAUNCH: return "WPA_ERR_LAUNCH: the HIP kernel launch failed";
    case WPA_ERR_TOO_LARGE:
      return "WPA_ERR_TOO_LARGE: the call needs more scratch than the fixed buffer holds (WPA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

wpa_status wpa_quantize_q_rows(const void* q, wpa_dtype q_dtype, int n_tokens, int n_q_heads, int8_t* q_i8,
                               float* q_scale, hipStream_t stream) {
  if (n_tokens < 0 || n_q_heads <= 0) return WPA_ERR_SHAPE;
  if (q_dtype != WPA_BF16 && q_dtype != WPA_F32) return WPA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return WPA_OK;
  if (!q || !q_i8 || !q_scale) return WPA_ERR_NULL;
  if (!aligned16(q) || !aligned16(q_i8)) return WPA_ERR_UNSUPPORTED;
  if ((long)n_tokens * n_q_heads * 32 > 0x7fffffffL * 256L) return WPA_ERR_UNSUPPORTED;
  if (wpa::launch_quantize_q_rows(q, q_dtype == WPA_BF16, n_tokens, n_q_heads, q_i8, q_scale, stream) !=
      hipSuccess)
    return WPA_ERR_LAUNCH;
  return WPA_OK;
}

wpa_status wpa_kv_write_i8(const void* k, const void* v, wpa_dtype dtype, int n_tokens, int n_kv_heads,
                           const int32_t* slots, int n_pool_pages, int8_t* k_pool, int8_t* v_pool, float* k_scale,
                           float* v_scale, hipStream_t stream) {
  if (n_tokens < 0 || n_kv_heads <= 0 || n_pool_pages < 0) return WPA_ERR_SHAPE;
  if (dtype != WPA_BF16 && dtype != WPA_F32) return WPA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return WPA_OK;
  if (!k || !v || !slots || !k_pool || !v_pool || !k_scale || !v_scale) return WPA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool)) return WPA_ERR_UNSUPPORTED;
  if (2L * n_tokens * n_kv_heads * 32 > 0x7fffffffL * 256L) return WPA_ERR_UNSUPPORTED;
  if (wpa::launch_kv_write(k, v, dtype == WPA_BF16, n_tokens, n_kv_heads, slots, n_pool_pages, k_pool, v_pool,
                           k_scale, v_scale, stream) != hipSuccess)
    return WPA_ERR_LAUNCH;
  return WPA_OK;
}

}  // extern "C"

namespace {

// q_bf16 == nullptr: Q comes as int8 codes and row scales; otherwise as bf16
// and the kernels quantize it.
wpa_status prefill_attn(const int8_t* q_i8, const float* q_scale, const uint16_t* q_bf16, const int8_t* k_pool,
                        const int8_t* v_pool, const float* k_scale, const float* v_scale,
                        const int32_t* page_table, int n_pool_pages, int q_start, int n_tokens, int n_q_heads,
                        int n_kv_heads, int window_blocks, int sink_blocks, float softmax_scale, void* out,
                        wpa_dtype out_dtype, hipStream_t stream) {
  if (n_tokens < 0 || q_start < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
    return WPA_ERR_SHAPE;
  if (sink_blocks < 0 || !std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return WPA_ERR_SHAPE;
  const long seq = (long)q_start + n_tokens;  // keys 0 .. seq-1 are in the pool
  if (n_pool_pages < 0 || n_pool_pages < ceil_div(seq, WPA_PAGE_TOKENS)) return WPA_ERR_SHAPE;
  if (out_dtype != WPA_BF16 && out_dtype != WPA_F32) return WPA_ERR_UNSUPPORTED;
  if (q_start % WPA_PAGE_TOKENS != 0 || seq > 0x7fffffffL - WPA_PAGE_TOKENS) return WPA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return WPA_OK;
  const bool have_q = q_bf16 ? true : (q_i8 && q_scale);
  if (!have_q || !k_pool || !v_pool || !k_scale || !v_scale || !page_table || !out) return WPA_ERR_NULL;
  if (!aligned16(q_bf16 ? (const void*)q_bf16 : (const void*)q_i8) || !aligned16(k_pool) || !aligned16(v_pool))
    return WPA_ERR_UNSUPPORTED;
  const long n_tiles = ceil_div(n_tokens, WPA_PAGE_TOKENS);
  if (wpa::prefill_grid(n_q_heads, n_kv_heads, q_start / WPA_PAGE_TOKENS, n_tiles).workgroups > 0x7fffffffL)
    return WPA_ERR_UNSUPPORTED;

  wpa::AttnArgs a = {};
  a.q_i8 = q_i8;
  a.q_scale = q_scale;
  a.q_bf16 = q_bf16;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.page_table = page_table;
  a.out = out;
  a.n_pool_pages = n_pool_pages;
  a.n_tokens = n_tokens;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.window_blocks = window_blocks;
  a.sink_blocks = sink_blocks;
  a.softmax_scale = softmax_scale;
  a.q_start = q_start;
  if (wpa::launch_prefill_attn(a, out_dtype == WPA_BF16, stream) != hipSuccess) return WPA_ERR_LAUNCH;
  return WPA_OK;
}

wpa_status mask_counts(int q_start, int n_tokens, int window_blocks, int sink_blocks, int32_t* counts,
                       hipStream_t stream) {
  if (n_tokens < 0 || q_start < 0 || sink_blocks < 0) return WPA_ERR_SHAPE;
  if ((long)q_start + n_tokens > 0x7fffffffL - WPA_PAGE_TOKENS) return WPA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return WPA_OK;
  if (!counts) return WPA_ERR_NULL;
  if (wpa::launch_mask_counts(q_start, n_tokens, window_blocks, sink_blocks, counts, stream) != hipSuccess)
    return WPA_ERR_LAUNCH;
  return WPA_OK;
}

}  // namespace

extern "C" {

wpa_status wpa_prefill_attn_i8(const int8_t* q_i8, const float* q_scale, const int8_t* k_pool,
                               const int8_t* v_pool, const float* k_scale, const float* v_scale,
                               const int32_t* page_table, int n_pool_pages, int n_tokens, int n_q_heads,
                               int n_kv_heads, int window_blocks, int sink_blocks, float softmax_scale,
                               void* out, wpa_dtype out_dtype, hipStream_t stream) {
  return prefill_attn(q_i8, q_scale, nullptr, k_pool, v_pool, k_scale, v_scale, page_table, n_pool_pages, 0,
                      n_tokens,
                      n_q_heads, n_kv_heads, window_blocks, sink_blocks, softmax_scale, out, out_dtype, stream);
}

wpa_status wpa_prefill_attn_i8_chunk(const int8_t* q_i8, const float* q_scale, const int8_t* k_pool,
                                     const int8_t* v_pool, const float* k_scale, const float* v_scale,
                                     const int32_t* page_table, int n_pool_pages, int q_start, int n_tokens,
                                     int n_q_heads, int n_kv_heads, int window_blocks, int sink_blocks,
                                     float softmax_scale, void* out, wpa_dtype out_dtype, hipStream_t stream) {
  return prefill_attn(q_i8, q_scale, nullptr, k_pool, v_pool, k_scale, v_scale, page_table, n_pool_pages,
                      q_start, n_tokens, n_q_heads, n_kv_heads, window_blocks, sink_blocks, softmax_scale, out, out_dtype,
                      stream);
}

wpa_status wpa_prefill_attn_fused_q(const void* q, wpa_dtype q_dtype, const int8_t* k_pool, const int8_t* v_pool,
                                    const float* k_scale, const float* v_scale, const int32_t* page_table,
                                    int n_pool_pages, int q_start, int n_tokens, int n_q_heads, int n_kv_heads,
                                    int window_blocks, int sink_blocks, float softmax_scale, void* out,
                                    wpa_dtype out_dtype, hipStream_t stream) {
  if (q_dtype != WPA_BF16) return WPA_ERR_UNSUPPORTED;
  // a NULL q reaches prefill_attn with no Q at all and fails its pointer check
  return prefill_attn(nullptr, nullptr, static_cast<const uint16_t*>(q), k_pool, v_pool, k_scale, v_scale,
                      page_table, n_pool_pages, q_start, n_tokens, n_q_heads, n_kv_heads, window_blocks, sink_blocks,
                      softmax_scale, out, out_dtype, stream);
}

wpa_status wpa_mask_counts(int n_tokens, int window_blocks, int sink_blocks, int32_t* counts,
                           hipStream_t stream) {
  return mask_counts(0, n_tokens, window_blocks, sink_blocks, counts, stream);
}

size_t wpa_decode_workspace_bytes(int batch, int n_q_heads, int max_blocks, int window_blocks, int sink_blocks) {
  if (batch <= 0 || n_q_heads <= 0 || max_blocks <= 0) return 0;
  const int splits = wpa::decode_splits(max_blocks, window_blocks, sink_blocks < 0 ? 0 : sink_blocks);
  return (size_t)batch * n_q_heads * splits * wpa::kWsRow * sizeof(float);
}

}  // extern "C"

namespace {

// Host checks shared by the two decode entry points (all but the workspace).
wpa_status decode_check(const int8_t* q_i8, const float* q_scale, const int8_t* k_pool, const int8_t* v_pool,
                        const float* k_scale, const float* v_scale, int n_pool_pages, const int32_t* page_tables,
                        int max_blocks, const int32_t* seq_lens, int batch, int n_q_heads, int n_kv_heads,
                        int window_blocks, int sink_blocks, float softmax_scale, const void* out,
                        wpa_dtype out_dtype) {
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return WPA_ERR_SHAPE;
  if (max_blocks <= 0 || n_pool_pages <= 0 || sink_blocks < 0) return WPA_ERR_SHAPE;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return WPA_ERR_SHAPE;
  if (out_dtype != WPA_BF16 && out_dtype != WPA_F32) return WPA_ERR_UNSUPPORTED;
  if (batch == 0) return WPA_OK;
  if (!q_i8 || !q_scale || !k_pool || !v_pool || !k_scale || !v_scale || !page_tables || !seq_lens || !out)
    return WPA_ERR_NULL;
  if (!aligned16(q_i8) || !aligned16(k_pool) || !aligned16(v_pool)) return WPA_ERR_UNSUPPORTED;
  const long splits = wpa::decode_splits(max_blocks, window_blocks, sink_blocks);
  const long head_groups = (n_q_heads / n_kv_heads + wpa::kMaxDecodeG - 1) / wpa::kMaxDecodeG;
  if ((long)batch * n_kv_heads * head_groups * splits > 0x7fffffffL || (long)batch * n_q_heads > 0x7fffffffL)
    return WPA_ERR_UNSUPPORTED;
  (void)window_blocks;
  return WPA_OK;
}

wpa_status decode_launch(const int8_t* q_i8, const float* q_scale, const int8_t* k_pool, const int8_t* v_pool,
                         const float* k_scale, const float* v_scale, int n_pool_pages, const int32_t* page_tables,
                         int max_blocks, const int32_t* seq_lens, int batch, int n_q_heads, int n_kv_heads,
                         int window_blocks, int sink_blocks, float softmax_scale, float* ws, void* out,
                         wpa_dtype out_dtype, hipStream_t stream) {
  wpa::DecodeArgs a = {};
  a.q_i8 = q_i8;
  a.q_scale = q_scale;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.page_tables = page_tables;
  a.seq_lens = seq_lens;
  a.ws = ws;
  a.out = out;
  a.n_pool_pages = n_pool_pages;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.window_blocks = window_blocks;
  a.sink_blocks = sink_blocks;
  a.softmax_scale = softmax_scale;
  if (wpa::launch_decode(a, out_dtype == WPA_BF16, stream) != hipSuccess) return WPA_ERR_LAUNCH;
  return WPA_OK;
}

}  // namespace

extern "C" {

wpa_status wpa_decode_attn_i8(const int8_t* q_i8, const float* q_scale, const int8_t* k_pool, const int8_t* v_pool,
                              const float* k_scale, const float* v_scale, int n_pool_pages,
                              const int32_t* page_tables, int max_blocks, const int32_t* seq_lens, int batch,
                              int n_q_heads, int n_kv_heads, int window_blocks, int sink_blocks, float softmax_scale,
                              void* workspace, size_t workspace_bytes, void* out, wpa_dtype out_dtype,
                              hipStream_t stream) {
  const wpa_status st = decode_check(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, n_pool_pages, page_tables,
                                     max_blocks, seq_lens, batch, n_q_heads, n_kv_heads, window_blocks, sink_blocks,
                                     softmax_scale, out, out_dtype);
  if (st != WPA_OK || batch == 0) return st;
  if (!workspace) return WPA_ERR_NULL;
  if (workspace_bytes < wpa_decode_workspace_bytes(batch, n_q_heads, max_blocks, window_blocks, sink_blocks))
    return WPA_ERR_SHAPE;
  if (!aligned16(workspace)) return WPA_ERR_UNSUPPORTED;
  return decode_launch(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, n_pool_pages, page_tables, max_blocks,
                       seq_lens, batch, n_q_heads, n_kv_heads, window_blocks, sink_blocks, softmax_scale,
                       static_cast<float*>(workspace), out, out_dtype, stream);
}

wpa_status wpa_decode_attn_i8_noalloc(const int8_t* q_i8, const float* q_scale, const int8_t* k_pool,
                                      const int8_t* v_pool, const float* k_scale, const float* v_scale,
                                      int n_pool_pages, const int32_t* page_tables, int max_blocks,
                                      const int32_t* seq_lens, int batch, int n_q_heads, int n_kv_heads,
                                      int window_blocks, int sink_blocks, float softmax_scale, void* out,
                                      wpa_dtype out_dtype, hipStream_t stream) {
  static_assert(WPA_NOALLOC_SCRATCH_BYTES == wpa::kNoAllocScratchBytes, "one stated size");
  const wpa_status st = decode_check(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, n_pool_pages, page_tables,
                                     max_blocks, seq_lens, batch, n_q_heads, n_kv_heads, window_blocks, sink_blocks,
                                     softmax_scale, out, out_dtype);
  if (st != WPA_OK || batch == 0) return st;
  // every check above and this one come before any HIP call
  if (wpa_decode_workspace_bytes(batch, n_q_heads, max_blocks, window_blocks, sink_blocks) >
      WPA_NOALLOC_SCRATCH_BYTES)
    return WPA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (wpa::noalloc_scratch(&ws) != hipSuccess) return WPA_ERR_LAUNCH;
  return decode_launch(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, n_pool_pages, page_tables, max_blocks,
                       seq_lens, batch, n_q_heads, n_kv_heads, window_blocks, sink_blocks, softmax_scale,
                       static_cast<float*>(ws), out, out_dtype, stream);
}

wpa_status wpa_mask_counts_chunk(int q_start, int n_tokens, int window_blocks, int sink_blocks, int32_t* counts,
                                 hipStream_t stream) {
  return mask_counts(q_start, n_tokens, window_blocks, sink_blocks, counts, stream);
}

}  // extern "C"
