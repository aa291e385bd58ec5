// Split-KV decode over the paged int8 pool: one query token per sequence (the
// sequence's last position), the prefill path's mask and int8 scheme.
//
// Method (int8 tensor-core prefill attention page, "Why the attention, and
// why tensor cores"; the scheme it credits to the int8 GQA flash-decode in
// "Relation to open PRs"): Q is int8 with one scale per row (here a row is
// one query head of one sequence), QK^T runs int8 x int8 -> int32 and the row
// Q scale, per-token K scale and softmax scale are applied to the int32; the
// per-token V scale is folded into P, P is quantized to int8 per 16-key block
// and PV runs int8 x int8 -> int32.  Keys: the sink and window blocks up to
// the query's own block, causally ("Relation to open PRs": a window <= 0 is
// full causal attention).
//
// Design
//   * A workgroup takes one (sequence, KV head, split): the G query heads of
//     the KV head share every K and V row it loads.  A split is 8 pages (128
//     keys) of the sequence's key list, so short batches still spread over
//     the chip; a second launch combines the splits.
//   * The P codes of a block depend only on the ratios of P*v_scale inside the
//     block, so each split can use its own maximum Z_s: it returns
//     O_s = sum_blocks ps * (codes . v) and l_s = sum P, both relative to
//     2^Z_s, and the combine weighs split s by 2^(Z_s - max Z).  The per-block
//     step ps is applied in float after each block's int32 sum, as the method
//     writes it; decode is bound by HBM, not by this vector work.
//   * QK^T uses v_dot4_i32_i8 on K rows read straight from the pool; V is
//     staged in LDS (16-byte chunks XOR-swizzled by key) for the PV reads.

#include "wpa_common.h"
#include "wpa_launch.h"

namespace wpa {

constexpr int kSplitPages = 8;
constexpr int kSplitKeys = kSplitPages * kPage;  // 128
constexpr float kLog2eD = 1.4426950408889634f;

__device__ inline int dswz(int r) { return r & 15; }  // chunk slot XOR of key r

__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ alignas(16) int8_t q_lds[kMaxDecodeG][kHeadDim];
  __shared__ alignas(16) int8_t v_lds[kSplitKeys][kHeadDim];
  __shared__ float rowf_lds[kMaxDecodeG];
  __shared__ float ks_lds[kSplitKeys], lv_lds[kSplitKeys], vs_lds[kSplitKeys];
  __shared__ float s_lds[kMaxDecodeG][kSplitKeys];  // acc * k_scale; -inf for masked keys
  __shared__ int8_t code_lds[kMaxDecodeG][kSplitKeys];
  __shared__ float ps_lds[kMaxDecodeG][kSplitPages];
  __shared__ float z_lds[kMaxDecodeG], l_lds[kMaxDecodeG];
  __shared__ int page_lds[kSplitPages], pos_lds[kSplitPages];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int u = blockIdx.x;
  const int sp = u % a.n_splits;
  u /= a.n_splits;
  const int kvh = u % a.n_kv_heads;
  const int b = u / a.n_kv_heads;
  const int G = a.G;
  float* ws = a.ws + ((long)b * a.n_q_heads + (long)kvh * G) * a.n_splits * kWsRow;

  // the query position; lengths beyond the page table are clamped to it
  const int len = min(a.seq_lens[b], kPage * a.max_blocks);
  const int t = len - 1;
  const TileBlocks tb = tile_blocks(t >= 0 ? t / kPage : 0, a.window_blocks, a.sink_blocks);
  const int first = sp * kSplitPages;
  const int nb = t < 0 ? 0 : min(kSplitPages, tb.n_total - first);
  if (nb <= 0) {  // nothing to attend in this split
    if (tid < G) {
      float* w = ws + ((long)tid * a.n_splits + sp) * kWsRow;
      w[kHeadDim] = -INFINITY;
      w[kHeadDim + 1] = 0.f;
    }
    return;
  }

  // ---- stage: page ids first, then every global load of the split is issued
  // before anything waits on one (Q rows, V rows, K rows, scales)
  if (tid < kSplitPages) {
    const int blk = tb.block(min(first + tid, tb.n_total - 1));
    const int pg = a.page_tables[(long)b * a.max_blocks + blk];
    page_lds[tid] = min(max(pg, 0), a.n_pool_pages - 1);  // a bad entry reads a wrong page, never out of bounds
    pos_lds[tid] = kPage * blk;
  }
  __syncthreads();
  const int r16 = tid >> 4, c16 = tid & 15;  // staging: key r16 of each page, 16-byte chunk c16
  const int j = tid >> 1, half = tid & 1;     // scores: key j of the split, half of the channels
  uint4 qv, vv[kSplitPages];
  int4 kr[8];
  float ksv = 0.f, vsv = 0.f;
  if (r16 < G) qv = *reinterpret_cast<const uint4*>(a.q_i8 + ((long)b * a.n_q_heads + kvh * G + r16) * kHeadDim +
                                                    16 * c16);
  // Straight-line loads: slots past the split's last page repeat a page of the
  // split (page_lds clamps), so every load is in bounds and none waits on a
  // branch; what they bring is masked or never read.
#pragma unroll
  for (int p = 0; p < kSplitPages; ++p) {
    const long row = ((long)page_lds[p] * kPage + r16) * a.n_kv_heads + kvh;
    vv[p] = *reinterpret_cast<const uint4*>(a.v_pool + row * kHeadDim + 16 * c16);
  }
  const bool have = j < kPage * nb;
  {
    const long row = ((long)page_lds[j >> 4] * kPage + (j & 15)) * a.n_kv_heads + kvh;
    const int4* src = reinterpret_cast<const int4*>(a.k_pool + row * kHeadDim + 128 * half);
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = src[i];
  }
  if (tid < kSplitKeys) {
    const long row = ((long)page_lds[tid >> 4] * kPage + (tid & 15)) * a.n_kv_heads + kvh;
    ksv = a.k_scale[row];
    vsv = a.v_scale[row];
  }
  const float rowf = tid < G ? a.q_scale[(long)b * a.n_q_heads + kvh * G + tid] * a.row_mul : 0.f;
  if (r16 < G) *reinterpret_cast<uint4*>(&q_lds[r16][16 * c16]) = qv;
#pragma unroll
  for (int p = 0; p < kSplitPages; ++p) {
    const int key = kPage * p + r16;
    *reinterpret_cast<uint4*>(&v_lds[key][16 * (c16 ^ dswz(key))]) = vv[p];
  }
  if (tid < kSplitKeys) {
    ks_lds[tid] = ksv;
    vs_lds[tid] = vsv;
    lv_lds[tid] = __builtin_amdgcn_logf(vsv);
  }
  if (tid < G) rowf_lds[tid] = rowf;
  __syncthreads();

  // ---- scores: thread (key j, half of the channels), int8 dot products
  {
    const int p = j >> 4;
    const bool valid = have && pos_lds[min(p, kSplitPages - 1)] + (j & 15) <= t && first + p < tb.n_total;
    for (int h = 0; h < G; ++h) {
      int acc = 0;
      if (have) {
        const int4* qq = reinterpret_cast<const int4*>(&q_lds[h][128 * half]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int4 q4 = qq[i];
          acc = __builtin_amdgcn_sdot4(kr[i].x, q4.x, acc, false);
          acc = __builtin_amdgcn_sdot4(kr[i].y, q4.y, acc, false);
          acc = __builtin_amdgcn_sdot4(kr[i].z, q4.z, acc, false);
          acc = __builtin_amdgcn_sdot4(kr[i].w, q4.w, acc, false);
        }
      }
      acc += __shfl_xor(acc, 1);
      if (half == 0) s_lds[h][j] = valid ? (float)acc * ks_lds[j] : -INFINITY;
    }
  }
  __syncthreads();

  // ---- per head: split max Z of z = s*rowf + log2(v_scale), e = exp2(s*rowf - Z),
  // l = sum e, P' = e * v_scale, per-page codes.  Wave w takes heads w, w+4, ...
  for (int h = wave; h < G; h += 4) {
    const float rowf = rowf_lds[h];
    float z = -INFINITY;
    for (int j = lane; j < kSplitKeys; j += 64) {
      const float s = s_lds[h][j];
      if (s != -INFINITY) z = fmaxf(z, fmaf(s, rowf, lv_lds[j]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z = fmaxf(z, __shfl_xor(z, off));
    float lsum = 0.f;
    for (int j0 = 0; j0 < kSplitKeys; j0 += 64) {
      const int j = j0 + lane;
      const float s = s_lds[h][j];
      const bool ok = s != -INFINITY;
      const float e = ok ? __builtin_amdgcn_exp2f(fmaf(s, rowf, -z)) : 0.f;
      const float pv = e * (ok ? vs_lds[j] : 0.f);
      lsum += e;
      float mx = pv;  // max over the 16 keys of this page (lanes 16k .. 16k+15)
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
      // code = rint(P' * 127 / max); a page whose P' are all zero gets codes 0 and step 0
      const float c = mx > 0.f ? rintf(pv * (127.0f / mx)) : 0.f;
      code_lds[h][j] = (int8_t)(int)c;
      if ((lane & 15) == 0) ps_lds[h][j >> 4] = mx * (1.0f / 127.0f);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    if (lane == 0) {
      z_lds[h] = z;
      l_lds[h] = lsum;
    }
  }
  __syncthreads();

  // ---- PV: thread task = (head, 4 channels); int32 sum per page, then ps * sum in float
  for (int task = tid; task < G * 64; task += 256) {
    const int h = task >> 6, c4 = 4 * (task & 63);
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < nb; ++p) {
      int acc[4] = {0, 0, 0, 0};
#pragma unroll 4
      for (int r = 0; r < kPage; ++r) {
        const int key = kPage * p + r;
        const int code = code_lds[h][key];
        const uint32_t vv =
            *reinterpret_cast<const uint32_t*>(&v_lds[key][16 * ((c4 >> 4) ^ dswz(key)) + (c4 & 15)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += code * (int)(int8_t)(vv >> (8 * i));
      }
      const float ps = ps_lds[h][p];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(ps, (float)acc[i], o[i]);
    }
    float* w = ws + ((long)h * a.n_splits + sp) * kWsRow;
    *reinterpret_cast<float4*>(w + c4) = make_float4(o[0], o[1], o[2], o[3]);
    if (c4 == 0) {
      w[kHeadDim] = z_lds[h];
      w[kHeadDim + 1] = l_lds[h];
    }
  }
}

// Combine the splits of one (sequence, query head): weights 2^(Z_s - max Z).
// One wave per row: the split maxima and weights are found lane-parallel (64
// splits at a time), then each lane sums 4 channels over the splits.  A
// sequence with no key to attend (length 0) gets a zero row.
template <bool OUT_BF16>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float f_lds[64];
  const long row = blockIdx.x;  // sequence * n_q_heads + head
  const int lane = threadIdx.x, c4 = 4 * lane;
  const float* w = a.ws + row * a.n_splits * kWsRow;
  float zmax = -INFINITY;
  for (int s = lane; s < a.n_splits; s += 64) zmax = fmaxf(zmax, w[(long)s * kWsRow + kHeadDim]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, off));
  float o[4] = {0.f, 0.f, 0.f, 0.f}, l = 0.f;
  if (zmax != -INFINITY) {
    for (int s0 = 0; s0 < a.n_splits; s0 += 64) {
      const int s = s0 + lane;
      float f = 0.f;
      if (s < a.n_splits) {
        const float z = w[(long)s * kWsRow + kHeadDim];
        if (z != -INFINITY) {  // an empty split wrote only Z and l; its O is not read
          f = __builtin_amdgcn_exp2f(z - zmax);
          l = fmaf(f, w[(long)s * kWsRow + kHeadDim + 1], l);
        }
      }
      __syncthreads();
      f_lds[lane] = f;
      __syncthreads();
      const int n = min(64, a.n_splits - s0);
#pragma unroll 4
      for (int i = 0; i < n; ++i) {
        const float fi = f_lds[i];
        if (fi == 0.f) continue;  // the same for every lane
        const float4 v = *reinterpret_cast<const float4*>(w + (long)(s0 + i) * kWsRow + c4);
        o[0] = fmaf(fi, v.x, o[0]);
        o[1] = fmaf(fi, v.y, o[1]);
        o[2] = fmaf(fi, v.z, o[2]);
        o[3] = fmaf(fi, v.w, o[3]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = o[i] * inv;
    if (OUT_BF16) {
      const uint32_t u32 = __float_as_uint(x);  // round to nearest even
      reinterpret_cast<uint16_t*>(a.out)[row * kHeadDim + c4 + i] =
          (uint16_t)((u32 + 0x7fffu + ((u32 >> 16) & 1u)) >> 16);
    } else {
      reinterpret_cast<float*>(a.out)[row * kHeadDim + c4 + i] = x;
    }
  }
}

int decode_splits(int max_blocks, int window_blocks, int sink_blocks) {
  long blocks = max_blocks;
  if (window_blocks > 0) blocks = std::min<long>(blocks, (long)window_blocks + sink_blocks);
  return (int)((blocks + kSplitPages - 1) / kSplitPages);
}

hipError_t launch_decode(const DecodeArgs& args_in, bool out_bf16, hipStream_t stream) {
  DecodeArgs a = args_in;
  a.G = a.n_q_heads / a.n_kv_heads;
  a.row_mul = a.softmax_scale * kLog2eD;
  a.n_splits = decode_splits(a.max_blocks, a.window_blocks, a.sink_blocks);
  const unsigned grid = (unsigned)((long)a.batch * a.n_kv_heads * a.n_splits);
  hipLaunchKernelGGL(decode_split_kernel, dim3(grid), dim3(256), 0, stream, a);
  const unsigned rows = (unsigned)((long)a.batch * a.n_q_heads);
  if (out_bf16) hipLaunchKernelGGL(decode_combine_kernel<true>, dim3(rows), dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(decode_combine_kernel<false>, dim3(rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wpa
