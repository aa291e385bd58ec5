// Q row quantization, the KV-pool writer and mask counts: the small kernels
// of the path.
//
// Q quantization follows the int8 tensor-core prefill attention page, section
// "Why the attention, and why tensor cores" (one scale per query row).  It is
// a pure HBM stream: each row is 256 values, read once, written once as int8
// plus one float scale.  32 lanes take a row, 8 values per lane, so every
// lane issues one 16-byte load (bf16) and one 8-byte store per row.

#include "wpa_common.h"
#include "wpa_launch.h"

namespace wpa {

// Eight consecutive channels of a 256-channel row held by one of 32 lanes.
template <bool BF16>
__device__ inline void load8(const void* __restrict__ x, long row, int sub, float (&v)[8]) {
  if (BF16) {
    const uint4 raw = reinterpret_cast<const uint4*>(x)[row * 32 + sub];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(x) + row * 64 + sub * 2;
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Per-row quantization of a row spread over the 32 lanes of a half wave:
// amax by a shuffle reduction, then IEEE division and round-half-to-even, as
// the definition states.  Returns the lane's 8 codes and the row scale.
__device__ inline uint2 quant8(const float (&v)[8], float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
  const float inv = q_inv_of(amax);
  scale = q_scale_of(amax);
  return make_uint2(q_code4(v[0], v[1], v[2], v[3], inv), q_code4(v[4], v[5], v[6], v[7], inv));
}

// Each half wave takes kRowsPerHalf consecutive rows and issues all their
// loads before quantizing any, so a wave keeps 4 KB of reads in flight.
constexpr int kRowsPerHalf = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_q_rows_kernel(const void* __restrict__ q,
                                                              int8_t* __restrict__ q_i8,
                                                              float* __restrict__ q_scale,
                                                              long n_rows) {
  const long row0 = (((long)blockIdx.x * blockDim.x + threadIdx.x) >> 5) * kRowsPerHalf;
  const int sub = threadIdx.x & 31;  // 8 channels each
  if (row0 >= n_rows) return;        // whole half-waves drop out together
  float v[kRowsPerHalf][8];
#pragma unroll
  for (int i = 0; i < kRowsPerHalf; ++i) load8<BF16>(q, min(row0 + i, n_rows - 1), sub, v[i]);
#pragma unroll
  for (int i = 0; i < kRowsPerHalf; ++i) {
    const long row = row0 + i;
    float scale;
    const uint2 codes = quant8(v[i], scale);
    if (row < n_rows) {
      reinterpret_cast<uint2*>(q_i8)[row * 32 + sub] = codes;
      if (sub == 0) q_scale[row] = scale;
    }
  }
}

// KV-pool writer: half wave r takes rows kRowsPerHalf*r .. of K, or of V
// (half waves past the K rows), row = token * n_kv_heads + head, and stores
// each row's codes and scale at its token's pool slot.  Slots outside the
// pool are skipped.
template <bool BF16>
__global__ __launch_bounds__(256) void kv_write_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                       const int32_t* __restrict__ slots, int n_kv_heads,
                                                       long n_rows, long n_slots, int8_t* __restrict__ k_pool,
                                                       int8_t* __restrict__ v_pool, float* __restrict__ k_scale,
                                                       float* __restrict__ v_scale) {
  const long halves = (n_rows + kRowsPerHalf - 1) / kRowsPerHalf;  // per tensor
  long hr = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
  const int sub = threadIdx.x & 31;
  if (hr >= 2 * halves) return;
  const bool is_v = hr >= halves;
  if (is_v) hr -= halves;
  const long row0 = hr * kRowsPerHalf;
  float x[kRowsPerHalf][8];
  long slot[kRowsPerHalf];
#pragma unroll
  for (int i = 0; i < kRowsPerHalf; ++i) {
    const long r = min(row0 + i, n_rows - 1);
    slot[i] = slots[r / n_kv_heads];
    load8<BF16>(is_v ? v : k, r, sub, x[i]);
  }
#pragma unroll
  for (int i = 0; i < kRowsPerHalf; ++i) {
    const long r = row0 + i;
    float scale;
    const uint2 codes = quant8(x[i], scale);
    if (r >= n_rows || slot[i] < 0 || slot[i] >= n_slots) continue;  // the whole half wave together
    const long token = r / n_kv_heads;
    const long dst = slot[i] * n_kv_heads + (r - token * n_kv_heads);
    reinterpret_cast<uint2*>(is_v ? v_pool : k_pool)[dst * 32 + sub] = codes;
    if (sub == 0) (is_v ? v_scale : k_scale)[dst] = scale;
  }
}

// counts[i] = number of keys row t = q_start + i attends: every listed block
// but the diagonal one is attended whole, the diagonal contributes t%16 + 1 keys.
__global__ __launch_bounds__(256) void mask_counts_kernel(int q_start, int n_tokens, int window_blocks,
                                                          int sink_blocks, int32_t* __restrict__ counts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_tokens) return;
  const int t = q_start + i;
  const int qt = t / kPage;
  const TileBlocks tb = tile_blocks(qt, window_blocks, sink_blocks);
  counts[i] = kPage * (tb.n_total - 1) + (t - kPage * qt + 1);
}

hipError_t launch_quantize_q_rows(const void* q, bool bf16, int n_tokens, int n_q_heads, int8_t* q_i8,
                                  float* q_scale, hipStream_t stream) {
  const long n_rows = (long)n_tokens * n_q_heads;
  const long threads = (n_rows + kRowsPerHalf - 1) / kRowsPerHalf * 32;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(quantize_q_rows_kernel<true>, dim3(blocks), dim3(256), 0, stream, q, q_i8, q_scale, n_rows);
  else
    hipLaunchKernelGGL(quantize_q_rows_kernel<false>, dim3(blocks), dim3(256), 0, stream, q, q_i8, q_scale, n_rows);
  return hipGetLastError();
}

hipError_t launch_kv_write(const void* k, const void* v, bool bf16, int n_tokens, int n_kv_heads,
                           const int32_t* slots, int n_pool_pages, int8_t* k_pool, int8_t* v_pool, float* k_scale,
                           float* v_scale, hipStream_t stream) {
  const long n_rows = (long)n_tokens * n_kv_heads;
  const long n_slots = (long)n_pool_pages * kPage;
  const long threads = 2 * ((n_rows + kRowsPerHalf - 1) / kRowsPerHalf) * 32;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(kv_write_kernel<true>, dim3(blocks), dim3(256), 0, stream, k, v, slots, n_kv_heads, n_rows,
                       n_slots, k_pool, v_pool, k_scale, v_scale);
  else
    hipLaunchKernelGGL(kv_write_kernel<false>, dim3(blocks), dim3(256), 0, stream, k, v, slots, n_kv_heads, n_rows,
                       n_slots, k_pool, v_pool, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_mask_counts(int q_start, int n_tokens, int window_blocks, int sink_blocks, int32_t* counts,
                              hipStream_t stream) {
  const unsigned blocks = (unsigned)((n_tokens + 255) / 256);
  hipLaunchKernelGGL(mask_counts_kernel, dim3(blocks), dim3(256), 0, stream, q_start, n_tokens, window_blocks,
                     sink_blocks, counts);
  return hipGetLastError();
}

}  // namespace wpa
