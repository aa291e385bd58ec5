// Kernel launchers behind the C ABI (host side, arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <stdint.h>

namespace wpa {

struct AttnArgs {
  const int8_t* q_i8;       // int8 Q codes and row scales, or
  const float* q_scale;
  const uint16_t* q_bf16;   // bf16 Q, quantized by the attention kernels themselves
  const int8_t* k_pool;
  const int8_t* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* page_table;
  void* out;
  int n_pool_pages;  // page ids are clamped into [0, n_pool_pages)
  int n_tokens, n_q_heads, n_kv_heads;
  int window_blocks, sink_blocks;
  float softmax_scale;
  int q_start;  // sequence position of the call's first query row, a multiple of 16
  // filled in by the launcher
  int G, hgroups, n_tiles, tile0;
  float row_mul;
};

// Split-KV decode (wpa_decode.hip).
constexpr int kMaxDecodeG = 16;  // query heads per KV head
constexpr int kWsRow = 260;      // floats per (sequence, head, split): O[256], Z, l, 2 pad (16-byte rows)
struct DecodeArgs {
  const int8_t* q_i8;
  const float* q_scale;
  const int8_t* k_pool;
  const int8_t* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* page_tables;
  const int32_t* seq_lens;
  float* ws;
  void* out;
  int n_pool_pages, max_blocks, batch, n_q_heads, n_kv_heads;
  int window_blocks, sink_blocks;
  float softmax_scale;
  // filled in by the launcher
  int G, n_splits;
  float row_mul;
};
int decode_splits(int max_blocks, int window_blocks, int sink_blocks);
hipError_t launch_decode(const DecodeArgs& args, bool out_bf16, hipStream_t stream);

hipError_t launch_quantize_q_rows(const void* q, bool bf16, int n_tokens, int n_q_heads, int8_t* q_i8,
                                  float* q_scale, hipStream_t stream);
hipError_t launch_kv_write(const void* k, const void* v, bool bf16, int n_tokens, int n_kv_heads,
                           const int32_t* slots, int n_pool_pages, int8_t* k_pool, int8_t* v_pool, float* k_scale,
                           float* v_scale, hipStream_t stream);
hipError_t launch_mask_counts(int q_start, int n_tokens, int window_blocks, int sink_blocks, int32_t* counts,
                              hipStream_t stream);
// q_bf16 set: the kernels quantize Q as they load it (q_i8, q_scale unused).
hipError_t launch_prefill_attn(const AttnArgs& args, bool out_bf16, hipStream_t stream);

// Work decomposition of the prefill attention: a workgroup takes wpg query
// heads of one KV head (the largest of 4, 2, 1 dividing G) on 4/wpg
// consecutive query tiles, the groups of tiles counted from the sequence's
// first tile.  Workgroups of a call whose rows start at tile tile0:
struct PrefillGrid {
  int wpg, tpg, hgroups;
  long n_groups, workgroups;
};
inline PrefillGrid prefill_grid(int n_q_heads, int n_kv_heads, int tile0, long n_tiles) {
  PrefillGrid g;
  const int G = n_q_heads / n_kv_heads;
  g.wpg = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  g.tpg = 4 / g.wpg;
  g.hgroups = G / g.wpg;
  g.n_groups = n_tiles > 0 ? (tile0 + n_tiles - 1) / g.tpg - tile0 / g.tpg + 1 : 0;
  g.workgroups = g.n_groups * n_kv_heads * g.hgroups;
  return g;
}

}  // namespace wpa
