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
//   * A workgroup takes one (sequence, KV head, split) and up to 16 query
//     heads of the KV head, which share every K and V row it loads; a KV head
//     with more query heads takes one workgroup per group of 16.  A split is 8 pages (128
//     keys) of the sequence's key list, so short batches still spread over
//     the chip; a second launch combines the splits.
//   * The P codes of a block depend only on the ratios of P*v_scale inside the
//     block, so each split can use its own maximum Z_s: it returns
//     O_s = sum_blocks ps * (codes . v) and l_s = sum P, both relative to
//     2^Z_s, and the combine weighs split s by 2^(Z_s - max Z).  The per-block
//     step ps is applied in float to each block's int32 sum, as the method
//     writes it.
//   * Every load of a split is issued before any is waited on: page ids by
//     scalar loads, then Q and K straight into matrix-operand registers, V rows
//     and the scales.  The V rows are read whole (16 lanes over a key's 256
//     bytes) as non-temporal loads: read once, whole lines that skip L2
//     allocation stream faster on this part.  The K operand reads take half a
//     128-byte line per instruction (the other half comes with the next one),
//     which needs L2 to keep the line, so they stay ordinary loads.  QK^T runs on v_mfma_i32_16x16x64_i8 as S^T = K . Q^T
//     (wave w takes pages 2w, 2w+1 of the split; a lane then holds one head
//     and four keys per page).  PV runs on the same instruction with a block-diagonal P
//     operand: its 16 rows are (head, page) pairs, row (h, p) holding head
//     h's codes for the keys of page p and zeros elsewhere, so one product
//     over 64 keys returns the int32 sum of each page separately; wave w takes
//     16-channel tiles 4w .. 4w+3.  V is staged in LDS in the attention
//     kernel's swizzled 64-key tiles and read with the same transposing reads.

#include "wpa_common.h"
#include "wpa_lanes.h"
#include "wpa_launch.h"

#include <mutex>

namespace wpa {

constexpr int kSplitPages = 8;  // 4 and 16 measured slower
constexpr int kSplitKeys = kSplitPages * kPage;
constexpr int kPPW = kSplitPages / 4;  // pages per wave in QK^T and the softmax
constexpr int kTileKeys = 64;                    // keys of one PV product (four pages)
constexpr float kLog2eD = 1.4426950408889634f;

__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ alignas(16) int8_t v_lds[kSplitKeys / kTileKeys][kTileKeys * kHeadDim];
  __shared__ uint32_t code_lds[kMaxDecodeG][kSplitKeys / 4];  // four codes per word, keys 4m .. 4m+3
  __shared__ float ps_lds[kMaxDecodeG][kSplitPages];
  __shared__ float zpart[4][16], lpart[4][16];
  __shared__ float ks_lds[kSplitKeys], vs_lds[kSplitKeys], lv_lds[kSplitKeys];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  int u = blockIdx.x;
  const int sp = u % a.n_splits;
  u /= a.n_splits;
  const int hgi = u % a.n_hg;  // which group of kMaxDecodeG query heads of the KV head
  u /= a.n_hg;
  const int kvh = u % a.n_kv_heads;
  const int b = u / a.n_kv_heads;
  const int G = min(kMaxDecodeG, a.G - kMaxDecodeG * hgi);  // query heads of this workgroup
  // Q / ws row of the workgroup's first head
  const long head_row0 = (long)b * a.n_q_heads + (long)kvh * a.G + (long)kMaxDecodeG * hgi;
  float* ws = a.ws + head_row0 * a.n_splits * kWsRow;

  // the query position; lengths beyond the page table are clamped to it
  const int len = min(a.seq_lens[b], kPage * a.max_blocks);
  const int t = len - 1;
  const TileBlocks tb = tile_blocks(t >= 0 ? t / kPage : 0, a.window_blocks, a.sink_blocks);
  const int first = sp * kSplitPages;
  const int nb = t < 0 ? 0 : min(kSplitPages, tb.n_total - first);
  if (nb <= 0) {  // nothing to attend in this split: O = 0, Z = -inf, l = 0
    for (int h = 0; h < G; ++h) {
      float* w = ws + ((long)h * a.n_splits + sp) * kWsRow;
      w[tid] = 0.f;
      if (tid == 0) {
        w[kHeadDim] = -INFINITY;
        w[kHeadDim + 1] = 0.f;
      }
    }
    return;
  }

  // ---- page ids (scalar loads; slots past the split's last page repeat it,
  // and a bad entry is clamped into the pool: a wrong page, never out of bounds)
  const WPA_CONST int32_t* pt = (const WPA_CONST int32_t*)a.page_tables + (long)b * a.max_blocks;
  int page[kSplitPages], pos[kSplitPages];
#pragma unroll
  for (int p = 0; p < kSplitPages; ++p) {
    const int blk = tb.block(min(first + p, tb.n_total - 1));
    page[p] = min(max(pt[blk], 0), a.n_pool_pages - 1);
    pos[p] = kPage * blk;
  }

  // ---- every load of the split
  const int hq = min(n, G - 1);  // lanes of heads past G repeat the last head; never stored
  v4i qf[4], kf[kPPW][4];
  {
    const int8_t* qrow = a.q_i8 + (head_row0 + hq) * kHeadDim + 16 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *reinterpret_cast<const v4i*>(qrow + 64 * c);
  }
  const float rowf = a.q_scale[head_row0 + hq] * a.row_mul;
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const long row = ((long)page[kPPW * wave + pp] * kPage + n) * a.n_kv_heads + kvh;
    const int8_t* krow = a.k_pool + row * kHeadDim + 16 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) kf[pp][c] = *reinterpret_cast<const v4i*>(krow + 64 * c);
  }
  const int r16 = tid >> 4, c16 = tid & 15;  // V staging: key r16 of each page, 16-byte chunk c16
  v4i vv[kSplitPages];
#pragma unroll
  for (int p = 0; p < kSplitPages; ++p) {
    const long row = ((long)page[p] * kPage + r16) * a.n_kv_heads + kvh;
    vv[p] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(a.v_pool + row * kHeadDim + 16 * c16));
  }
  float ksv = 0.f, vsv = 0.f;
  if (tid < kSplitKeys) {
    const long row = ((long)page[tid >> 4] * kPage + (tid & 15)) * a.n_kv_heads + kvh;
    ksv = a.k_scale[row];
    vsv = a.v_scale[row];
  }
#pragma unroll
  for (int p = 0; p < kSplitPages; ++p) {
    const int key = kPage * (p & 3) + r16;  // key of its 64-key tile
    *reinterpret_cast<v4i*>(&v_lds[p >> 2][key * kHeadDim + 16 * (c16 ^ swz(key))]) = vv[p];
  }
  if (tid < kSplitKeys) {
    ks_lds[tid] = ksv;
    vs_lds[tid] = vsv;
    // floored as in the prefill kernel: keys of zero v_scale keep Z finite
    lv_lds[tid] = __builtin_amdgcn_logf(fmaxf(vsv, 0x1p-64f));
  }

  // ---- S^T = K . Q^T for this wave's pages: s[pp] register i is key 4g + i
  // of page kPPW*wave + pp for head n
  v4i s[kPPW];
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    s[pp] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c) s[pp] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[pp][c], qf[c], s[pp], 0, 0, 0);
  }
  __syncthreads();

  // ---- scores z = s*k_scale*rowf + log2(v_scale); the split maximum Z per head
  float sk[kPPW][4];
  bool ok[kPPW][4];
  float zmax = -INFINITY;
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const int p = kPPW * wave + pp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = kPage * p + 4 * g + i;
      ok[pp][i] = p < nb && pos[p] + 4 * g + i <= t;
      sk[pp][i] = (float)s[pp][i] * ks_lds[j];
      if (ok[pp][i]) zmax = fmaxf(zmax, fmaf(sk[pp][i], rowf, lv_lds[j]));
    }
  }
  zmax = rows_max(zmax);
  if (g == 0) zpart[wave][n] = zmax;
  __syncthreads();
  const float Z = fmaxf(fmaxf(zpart[0][n], zpart[1][n]), fmaxf(zpart[2][n], zpart[3][n]));

  // ---- e = exp2(s*k_scale*rowf - Z) = P, l = sum P, P' = P*v_scale, the
  // per-page codes rint(P' * 127 / max P') and steps max P' / 127
  float lsum = 0.f;
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const int p = kPPW * wave + pp;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = kPage * p + 4 * g + i;
      const float e = ok[pp][i] ? __builtin_amdgcn_exp2f(fmaf(sk[pp][i], rowf, -Z)) : 0.f;
      lsum += e;
      pv[i] = e * vs_lds[j];
    }
    const float mx = rows_max(fmaxf(fmaxf(pv[0], pv[1]), fmaxf(pv[2], pv[3])));
    const float inv = mx > 0.f ? 127.0f / mx : 0.f;  // a page with no attended key: codes 0, step 0
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= ((uint32_t)(int32_t)rintf(pv[i] * inv) & 0xffu) << (8 * i);
    code_lds[n][4 * p + g] = w;
    if (g == 0) ps_lds[n][p] = mx * (1.0f / 127.0f);
  }
  lsum = rows_sum(lsum);
  if (g == 0) lpart[wave][n] = lsum;
  __syncthreads();

  // ---- PV with a block-diagonal P operand: row r = 4*hl + pg of row tile rt
  // is head 4*rt + hl, page pg of the 64-key tile; output register i of lane
  // (g, n) is then head 4*rt + g, page i, channel 16*nt + n.
  const int rt_n = (G + 3) >> 2;
  float o[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int q = 0; q < 4; ++q) o[rt][q] = 0.f;
#pragma unroll
  for (int kt = 0; kt < kSplitKeys / kTileKeys; ++kt) {
    const VFrag read_v(v_lds[kt], lane);
    v4i vf[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vf[q] = read_v(4 * wave + q);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt >= rt_n) break;
      const int ha = 4 * rt + (n >> 2), pa = n & 3;  // this lane's row of the P operand
      const uint32_t cw = ha < G ? code_lds[ha][4 * (4 * kt + pa) + g] : 0u;
      v4i pa_op = v4i{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < 4; ++p) pa_op[p] = p == pa ? (int)cw : 0;
      const int hc = min(4 * rt + g, kMaxDecodeG - 1);  // this lane's head of the result
      float st[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) st[i] = ps_lds[hc][4 * kt + i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa_op, vf[q], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[rt][q] = fmaf(st[i], (float)c[i], o[rt][q]);
      }
    }
  }

  // ---- O_s, Z_s and l_s to the workspace.  The partial rows are written and
  // read back with non-temporal hints, since the combine reads each once: 2%
  // faster for the entry point at the 32k batch shape, the same bits (the
  // combine's loads give it; the stores alone gain a third of that).
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int h = 4 * rt + g;
    if (rt >= rt_n || h >= G) continue;
    float* w = ws + ((long)h * a.n_splits + sp) * kWsRow;
#pragma unroll
    for (int q = 0; q < 4; ++q) __builtin_nontemporal_store(o[rt][q], w + 16 * (4 * wave + q) + n);
  }
  if (wave == 0 && g == 0 && n < G) {
    float* w = ws + ((long)n * a.n_splits + sp) * kWsRow;
    __builtin_nontemporal_store(Z, w + kHeadDim);
    __builtin_nontemporal_store(lpart[0][n] + lpart[1][n] + lpart[2][n] + lpart[3][n], w + kHeadDim + 1);
  }
}

// Combine the splits of one (sequence, query head): weights 2^(Z_s - max Z).
// Thread c of the 256 sums channel c over the splits; the split weights are
// formed 256 splits at a time and shared through LDS.  Every split row holds
// a finite O (an empty split writes zeros and Z = -inf, weight 0), so the sum
// needs no branch and its loads can all be in flight.  A sequence with no key
// to attend (length 0) gets a zero row.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float f_lds[256];
  __shared__ float red[4];
  const long row = blockIdx.x;  // sequence * n_q_heads + head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* w = a.ws + row * a.n_splits * kWsRow;
  float zmax = -INFINITY;
  for (int s = tid; s < a.n_splits; s += 256) zmax = fmaxf(zmax, w[(long)s * kWsRow + kHeadDim]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, off));
  if (lane == 0) red[wave] = zmax;
  __syncthreads();
  zmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float o = 0.f, l = 0.f;
  if (zmax != -INFINITY) {
    for (int s0 = 0; s0 < a.n_splits; s0 += 256) {
      const int s = s0 + tid;
      float f = 0.f;
      if (s < a.n_splits) {
        const float z = w[(long)s * kWsRow + kHeadDim];
        f = __builtin_amdgcn_exp2f(z - zmax);  // 0 for an empty split
        l = fmaf(f, w[(long)s * kWsRow + kHeadDim + 1], l);
      }
      __syncthreads();  // the previous chunk's weights are no longer read
      f_lds[tid] = f;
      __syncthreads();
      const int m = min(256, a.n_splits - s0);
      const float* col = w + (long)s0 * kWsRow + tid;
      int i = 0;
      for (; i + 8 <= m; i += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(col + (long)(i + k) * kWsRow);
#pragma unroll
        for (int k = 0; k < 8; ++k) o = fmaf(f_lds[i + k], v[k], o);
      }
      for (; i < m; ++i) o = fmaf(f_lds[i], col[(long)i * kWsRow], o);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  __syncthreads();  // red[] is reused
  if (lane == 0) red[wave] = l;
  __syncthreads();
  l = red[0] + red[1] + red[2] + red[3];
  const float x = o * (l > 0.f ? 1.0f / l : 0.f);
  if (OUT_BF16) {
    const uint32_t u32 = __float_as_uint(x);  // round to nearest even
    reinterpret_cast<uint16_t*>(a.out)[row * kHeadDim + tid] = (uint16_t)((u32 + 0x7fffu + ((u32 >> 16) & 1u)) >> 16);
  } else {
    reinterpret_cast<float*>(a.out)[row * kHeadDim + tid] = x;
  }
}

// ---- The fixed device buffer of wpa_decode_attn_i8_noalloc: the split
// kernel's partial rows live here instead of in a caller workspace.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with that device current and kept;
// every launch gets that address.  Every GPU holds its own copy until the
// process ends; calls on one GPU share it.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_addr[kMaxDevices] = {};

hipError_t noalloc_scratch(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
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
  a.n_hg = (a.G + kMaxDecodeG - 1) / kMaxDecodeG;
  const unsigned grid = (unsigned)((long)a.batch * a.n_kv_heads * a.n_hg * a.n_splits);
  hipLaunchKernelGGL(decode_split_kernel, dim3(grid), dim3(256), 0, stream, a);
  const unsigned rows = (unsigned)((long)a.batch * a.n_q_heads);
  if (out_bf16) hipLaunchKernelGGL(decode_combine_kernel<true>, dim3(rows), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(decode_combine_kernel<false>, dim3(rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wpa
