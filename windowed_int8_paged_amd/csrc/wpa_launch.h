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
  int n_groups, streams, xcd_r, xcd_q;
  int runs;          // with xcd_r: contiguous runs (else every xcd_r-th group)
  int run_start[9];  // run r holds groups run_start[r] .. run_start[r + 1] - 1
  float row_mul;
};

// Split-KV decode (wpa_decode.hip).
constexpr int kMaxDecodeG = 16;  // query heads of one KV head per workgroup
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
  int G, n_splits, n_hg;  // n_hg groups of up to kMaxDecodeG query heads per KV head
  float row_mul;
};
int decode_splits(int max_blocks, int window_blocks, int sink_blocks);
// The decode's fixed scratch for callers that cannot allocate: its size, and
// its device address on the current device (looked up on first use there).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** addr);
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

// Work decomposition of the prefill attention: a workgroup (eight waves)
// takes wpg query heads of one KV head (the largest of 4, 2, 1 dividing G)
// on 8/wpg consecutive query tiles, the groups of tiles counted from the sequence's
// first tile.  A stream is one (KV head, head group) pair; its groups are
// numbered from the last (longest key list) down.
//
// Workgroups are dispatched to the chip's eight XCDs in turn (workgroup b
// runs on XCD b % 8), and each XCD has its own L2.  The order below keeps
// each stream's consecutive tile groups on as few XCDs as possible, so the
// key pages a window shares between neighbouring tiles stay in one L2:
//   * streams dividing 8 (xcd_r = 8 / streams XCDs per stream): XCD x takes
//     stream x % streams.  With many groups (kRunGroups or more per XCD of
//     the stream), the stream's groups are cut into xcd_r contiguous runs of
//     equal work (key steps plus a fixed cost per group) and XCD x takes run
//     x / streams: its L2 then holds one stretch of the sequence.  With few,
//     it takes every xcd_r-th group from x / streams on, which spreads the
//     long and short lists evenly over the XCDs;
//   * 8 dividing streams (xcd_q = streams / 8 streams per XCD): XCD x takes
//     streams x, x + 8, ..., their groups in turn;
//   * otherwise streams in turn, then groups.
// Either way each XCD walks its groups longest first.
constexpr int kXcds = 8;
constexpr long kRunGroups = 256;
struct PrefillGrid {
  int wpg, tpg, hgroups, streams, xcd_r, xcd_q;
  long n_groups, workgroups;  // workgroups to launch (an upper bound with xcd_r); those past a run exit at once
};
inline PrefillGrid prefill_grid(int n_q_heads, int n_kv_heads, int tile0, long n_tiles) {
  PrefillGrid g;
  const int G = n_q_heads / n_kv_heads;
  g.wpg = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  g.tpg = 8 / g.wpg;
  g.hgroups = G / g.wpg;
  g.n_groups = n_tiles > 0 ? (tile0 + n_tiles - 1) / g.tpg - tile0 / g.tpg + 1 : 0;
  g.streams = n_kv_heads * g.hgroups;
  g.xcd_r = g.streams <= kXcds && kXcds % g.streams == 0 ? kXcds / g.streams : 0;
  g.xcd_q = g.streams > kXcds && g.streams % kXcds == 0 ? g.streams / kXcds : 0;
  // with contiguous runs the launcher sizes the grid by its longest run: at most kXcds * n_groups
  g.workgroups = g.xcd_r ? (g.n_groups >= kRunGroups * g.xcd_r ? kXcds * g.n_groups
                                                                 : kXcds * ((g.n_groups + g.xcd_r - 1) / g.xcd_r))
                         : g.n_groups * g.streams;
  return g;
}
// Stream and group (0 = the last, longest) of workgroup b; a workgroup past
// the end of its run gets a group past every run (it exits at once).
__device__ inline void prefill_item(long b, int streams, int xcd_r, int xcd_q, int runs, const int* run_start,
                                    long& stream, long& group) {
  const long x = b % kXcds, j = b / kXcds;
  if (xcd_r && runs) {
    stream = x % streams;
    const int r = (int)(x / streams);
    group = run_start[r] + j;
    if (group >= run_start[r + 1]) group = 1L << 40;
  } else if (xcd_r) {
    stream = x % streams;
    group = xcd_r * j + x / streams;
  } else if (xcd_q) {
    stream = x + kXcds * (j % xcd_q);
    group = j / xcd_q;
  } else {
    stream = b % streams;
    group = b / streams;
  }
}

}  // namespace wpa
