// Device-side pieces shared by the attention and mask-count kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wpa {

constexpr int kHeadDim = 256;
constexpr int kPage = 16;

// Key blocks visited by one 16-row query tile.  The query tile is aligned to
// the 16-token page, so the window start is one value for the whole tile and
// only the causal bound differs between its rows (int8 tensor-core prefill
// attention page, "Why the attention, and why tensor cores").  The list is
// the sink blocks [0, n_sink) followed by the window blocks
// [win_start, qt]; window_blocks <= 0 means every block up to the diagonal
// ("Relation to open PRs").  The diagonal block qt is always the last entry
// and is the only one that needs a per-row (causal) mask.
struct TileBlocks {
  int n_sink;     // leading sink blocks 0 .. n_sink-1
  int win_start;  // first window block
  int n_total;    // list length = n_sink + (qt - win_start + 1)

  __host__ __device__ int block(int i) const { return i < n_sink ? i : win_start + (i - n_sink); }
};

__host__ __device__ inline TileBlocks tile_blocks(int qt, int window_blocks, int sink_blocks) {
  TileBlocks tb;
  const int n_blk_q = qt + 1;  // (t + 16) / 16 for every row t of the tile
  if (window_blocks <= 0) {
    tb.n_sink = 0;
    tb.win_start = 0;
  } else {
    const int rsb = n_blk_q - window_blocks > 0 ? n_blk_q - window_blocks : 0;
    tb.win_start = rsb;
    tb.n_sink = sink_blocks < rsb ? sink_blocks : rsb;  // sink blocks left of the window
  }
  tb.n_total = tb.n_sink + (n_blk_q - tb.win_start);
  return tb;
}

// Per-row Q quantization (int8 tensor-core prefill attention page, "Why the
// attention, and why tensor cores": one scale per query row).  Every kernel
// that quantizes Q goes through these, so the separate quantize launch and the
// attention launches that quantize their own tile give the same bits.
__device__ inline float q_inv_of(float amax) { return amax > 0.f ? 127.0f / amax : 0.f; }
__device__ inline float q_scale_of(float amax) { return amax > 0.f ? amax / 127.0f : 0.f; }
// Four codes rint(v * inv), little-endian in one word.  The product is
// rounded to float first, as the definition states; adding 1.5 * 2^23 then
// rounds it half-to-even to an integer held in the low mantissa bits, whose
// low byte is the code in two's complement.  No clamp is needed: |v| <= amax
// gives |v * inv| <= 127 * (1 + 2^-23) < 127.5 for finite rows, so the code
// is never -128 and never above 127.
__device__ inline uint32_t q_code4(float v0, float v1, float v2, float v3, float inv) {
#pragma clang fp contract(off)
  constexpr float kRound = 12582912.0f;
  const uint32_t b0 = __float_as_uint(v0 * inv + kRound), b1 = __float_as_uint(v1 * inv + kRound);
  const uint32_t b2 = __float_as_uint(v2 * inv + kRound), b3 = __float_as_uint(v3 * inv + kRound);
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // bytes: b0.0, b1.0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

}  // namespace wpa
