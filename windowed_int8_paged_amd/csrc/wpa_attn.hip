// Windowed int8 paged prefill attention, head_dim 256, for gfx950.
//
// Method (int8 tensor-core prefill attention page, "Why the attention, and
// why tensor cores"): Q is int8 with one scale per row; QK^T runs int8 x int8
// -> int32 and the row Q scale, per-token K scale and softmax scale are
// applied to the int32; the per-token V scale is folded into P, P is
// quantized to int8 and PV runs int8 x int8 -> int32.  The mask is causal
// plus sink/window over 16-token key blocks ("Relation to open PRs": a window
// <= 0 is full causal attention).
//
// gfx950 design
//   * One workgroup = one 16-token query tile x one KV head x up to 8 of its
//     query heads.  Each wave owns 32 query rows (two heads x 16 tokens) and
//     every K/V page it stages in LDS serves all the workgroup's heads.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_i32_32x32x32_i8: a lane then holds 16 keys of ONE query row, so
//     the row max/sum are in-lane plus one v_permlane32_swap.
//   * P codes are exactly the per-(row, 16-key block) int8 codes of the
//     method.  Their weights ps*code are then written as one fixed-point
//     integer relative to the row's largest P*v_scale (found by a first QK
//     pass) and split into NPL signed int8 digit planes, so PV runs at the
//     full K = 32 rate with int32 accumulation across every block and no
//     per-block floating-point rescale; the planes are recombined once at the
//     end.  With NPL = 3 the fixed point has 22 bits.
//   * K pages are copied to LDS row-major with a 16-byte row pad; V pages are
//     transposed in registers (4x4 byte blocks) so a lane reads 16 keys of
//     one channel with one 16-byte LDS read.

#include "wpa_common.h"
#include "wpa_launch.h"

#ifndef WPA_NPL
#define WPA_NPL 3
#endif

namespace wpa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kItKeys = 32;    // keys per loop iteration (two pages)
constexpr int kKStride = 272;  // LDS bytes per staged key row: 256 + 16 pad
constexpr int kVStride = 48;   // LDS bytes per channel row of staged V^T: 32 + 16 pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMagic = 8388608.0f;  // 2^23: x + 2^23 has x in its low 23 bits

template <int NPL>
struct FixedPoint;
template <>
struct FixedPoint<3> {
  static constexpr float kXmax = 4194304.f;  // 2^22; top digit stays <= 64
};
template <>
struct FixedPoint<2> {
  static constexpr float kXmax = 32512.f;  // top digit (x + 128) >> 8 stays <= 127
};

struct alignas(16) Smem {
  int8_t k[kItKeys * kKStride];
  int8_t vt[kHeadDim * kVStride];
  float ks[kItKeys];   // k_scale
  float lvs[kItKeys];  // log2(v_scale)
  float rvs[kItKeys];  // 1 / v_scale
};

__device__ inline float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline uint32_t byte_of(uint32_t w, int k) { return (w >> (8 * k)) & 0xffu; }

// Stage the two pages of iteration `it` (list entries 2it, 2it+1) into LDS.
// Entries past the end of the list are staged as zero keys with zero scales;
// their scores are masked.
template <int NTHR, bool WITH_V>
__device__ inline void stage(Smem& sm, const AttnArgs& a, const TileBlocks& tb, int it, int kvh) {
  const int tid = threadIdx.x;
  const long row_elems = (long)a.n_kv_heads * kHeadDim;  // pool row stride (bytes)
  const int li0 = 2 * it;
  const bool ok1 = li0 + 1 < tb.n_total;
  const long phys0 = a.page_table[tb.block(li0)];
  const long phys1 = ok1 ? (long)a.page_table[tb.block(li0 + 1)] : 0;
  // K rows: 32 keys x 16 chunks of 16 bytes
#pragma unroll
  for (int c0 = 0; c0 < kItKeys * 16; c0 += NTHR) {
    const int c = c0 + tid;
    const int key = c >> 4, ch = c & 15;
    const bool second = key >= 16;
    uint4 val = {0u, 0u, 0u, 0u};
    if (!second || ok1) {
      const long phys = second ? phys1 : phys0;
      const int8_t* src = a.k_pool + (phys * kPage + (key & 15)) * row_elems + (long)kvh * kHeadDim + ch * 16;
      val = *reinterpret_cast<const uint4*>(src);
    }
    *reinterpret_cast<uint4*>(sm.k + key * kKStride + ch * 16) = val;
  }
  if (tid < kItKeys) {
    const int key = tid;
    const bool second = key >= 16;
    float k_s = 0.f, lv = 0.f, rv = 0.f;
    if (!second || ok1) {
      const long phys = second ? phys1 : phys0;
      const long idx = (phys * kPage + (key & 15)) * a.n_kv_heads + kvh;
      const float v_s = a.v_scale[idx];
      k_s = a.k_scale[idx];
      lv = log2f(v_s);
      rv = 1.0f / v_s;
    }
    sm.ks[key] = k_s;
    sm.lvs[key] = lv;
    sm.rvs[key] = rv;
  }
  if (!WITH_V) return;
  // V^T: 8 groups of 4 tokens x 16 chunks of 16 channels.  Keys of a channel
  // row are stored in the order the PV operand reads them: position
  // 16h + 4i + k holds key 8i + 4h + k.
#pragma unroll
  for (int u0 = 0; u0 < 128; u0 += NTHR) {
    const int u = u0 + tid;
    if (NTHR > 128 && u >= 128) break;
    const int tg = u >> 4, dc = u & 15;
    const int key0 = 4 * tg;
    const bool second = key0 >= 16;
    uint4 r[4] = {};
    if (!second || ok1) {
      const long phys = second ? phys1 : phys0;
      const int8_t* src = a.v_pool + (phys * kPage + (key0 & 15)) * row_elems + (long)kvh * kHeadDim + dc * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = *reinterpret_cast<const uint4*>(src + i * row_elems);
    }
    const int pos0 = 16 * (tg & 1) + 4 * (tg >> 1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = (&r[0].x)[w], a1 = (&r[1].x)[w], a2 = (&r[2].x)[w], a3 = (&r[3].x)[w];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t b = byte_of(a0, k) | (byte_of(a1, k) << 8) | (byte_of(a2, k) << 16) | (byte_of(a3, k) << 24);
        *reinterpret_cast<uint32_t*>(sm.vt + (dc * 16 + 4 * w + k) * kVStride + pos0) = b;
      }
    }
  }
}

// S^T for the 32 staged keys x this wave's 32 query rows.
__device__ inline v16i qk_tile(const Smem& sm, const v4i (&qf)[8], int lane) {
  v16i s = {};
  const int8_t* krow = sm.k + (lane & 31) * kKStride + 16 * (lane >> 5);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const v4i kf = *reinterpret_cast<const v4i*>(krow + 32 * c);
    s = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[c], s, 0, 0, 0);
  }
  return s;
}

// Per-lane constants of one wave.
struct RowCtx {
  int h;        // half of the wave (0/1)
  float rowf;   // q_scale * softmax_scale * log2(e) of this lane's row
  int t_mask;   // causal bound of this lane's row
};

// Which of the 16 score registers hold attended keys (only the last iteration
// of a tile can contain the diagonal block or an empty list slot).
__device__ inline uint32_t key_mask(const TileBlocks& tb, int it, const RowCtx& rc) {
  uint32_t m = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kap = 8 * (v >> 2) + 4 * rc.h + (v & 3);
    const int li = 2 * it + (kap >> 4);
    const int blk = li < tb.n_total ? tb.block(li) : 0;
    const bool ok = (li < tb.n_total) && (kPage * blk + (kap & 15) <= rc.t_mask);
    m |= (ok ? 1u : 0u) << v;
  }
  return m;
}

template <bool MASKED>
__device__ inline float pass1_iter(const Smem& sm, const v4i (&qf)[8], int lane, const RowCtx& rc,
                                   uint32_t kmask, float m2) {
  const v16i s = qk_tile(sm, qf, lane);
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 ks4 = *reinterpret_cast<const float4*>(sm.ks + 8 * i4 + 4 * rc.h);
    const float4 lv4 = *reinterpret_cast<const float4*>(sm.lvs + 8 * i4 + 4 * rc.h);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * i4 + k;
      float z = fmaf((float)s[v] * (&ks4.x)[k], rc.rowf, (&lv4.x)[k]);
      if (MASKED) z = ((kmask >> v) & 1u) ? z : -INFINITY;
      m2 = fmaxf(m2, z);
    }
  }
  return m2;
}

template <int NPL, bool MASKED>
__device__ inline void pass2_iter(const Smem& sm, const v4i (&qf)[8], int lane, const RowCtx& rc,
                                  uint32_t kmask, float m2, float& lsum, v16i (&acc)[NPL][8]) {
  constexpr float kXmax = FixedPoint<NPL>::kXmax;
  const v16i s = qk_tile(sm, qf, lane);
  float pp[16];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 ks4 = *reinterpret_cast<const float4*>(sm.ks + 8 * i4 + 4 * rc.h);
    const float4 lv4 = *reinterpret_cast<const float4*>(sm.lvs + 8 * i4 + 4 * rc.h);
    const float4 rv4 = *reinterpret_cast<const float4*>(sm.rvs + 8 * i4 + 4 * rc.h);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * i4 + k;
      const float z = fmaf((float)s[v] * (&ks4.x)[k], rc.rowf, (&lv4.x)[k]);
      float e = __builtin_amdgcn_exp2f(z - m2);
      float lp = e * (&rv4.x)[k];
      if (MASKED) {
        const bool ok = (kmask >> v) & 1u;
        e = ok ? e : 0.f;
        lp = ok ? lp : 0.f;
      }
      lsum += lp;
      pp[v] = e;
    }
  }
  // per-(row, page) max of P': page 0 is v = 0..7, page 1 is v = 8..15
  float mx0 = pp[0], mx1 = pp[8];
#pragma unroll
  for (int v = 1; v < 8; ++v) {
    mx0 = fmaxf(mx0, pp[v]);
    mx1 = fmaxf(mx1, pp[8 + v]);
  }
  mx0 = xhalf_max(mx0);
  mx1 = xhalf_max(mx1);
  const float inv0 = mx0 > 0.f ? 127.0f / mx0 : 0.f;
  const float inv1 = mx1 > 0.f ? 127.0f / mx1 : 0.f;
  const float f0 = mx0 * (kXmax / 127.0f);
  const float f1 = mx1 * (kXmax / 127.0f);

  v4i dig[NPL];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d[3] = {0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * w + k;
      const float code = rintf(pp[v] * (v < 8 ? inv0 : inv1));
      const uint32_t b = __float_as_uint(fmaf(code, v < 8 ? f0 : f1, kMagic));
      d[0] |= (b & 0xffu) << (8 * k);
      d[1] |= (((b + 128u) >> 8) & 0xffu) << (8 * k);
      if (NPL == 3) d[2] |= (((b + 32896u) >> 16) & 0xffu) << (8 * k);
    }
#pragma unroll
    for (int p = 0; p < NPL; ++p) dig[p][w] = (int)d[p];
  }

  const int8_t* vrow = sm.vt + (lane & 31) * kVStride + 16 * rc.h;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const v4i vf = *reinterpret_cast<const v4i*>(vrow + nt * 32 * kVStride);
#pragma unroll
    for (int p = 0; p < NPL; ++p) acc[p][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(dig[p], vf, acc[p][nt], 0, 0, 0);
  }
}

template <int NPL, int WPG, bool OUT_BF16>
__global__ __launch_bounds__(64 * WPG, 1) void prefill_attn_kernel(AttnArgs a) {
  constexpr int NTHR = 64 * WPG;
  __shared__ Smem sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rho = lane & 31;  // this lane's query row within the wave (S^T column)

  int u = blockIdx.x;
  const int hg = u % a.hgroups;
  u /= a.hgroups;
  const int kvh = u % a.n_kv_heads;
  const int qt = a.n_tiles - 1 - u / a.n_kv_heads;  // longest tiles first

  const int pair = hg * WPG + wave;                 // every wave has a pair: WPG divides n_pairs
  const int head_lo = 2 * pair;                     // within the KV group
  const int my_head_in_group = head_lo + (rho >> 4);
  const bool head_ok = my_head_in_group < a.G;      // odd G: the last pair's 2nd head is padding
  const int my_head = kvh * a.G + (head_ok ? my_head_in_group : 0);
  const int my_t = qt * kPage + (rho & 15);
  const bool row_ok = head_ok && my_t < a.n_tokens;

  RowCtx rc;
  rc.h = lane >> 5;
  rc.t_mask = my_t < a.n_tokens ? my_t : a.n_tokens - 1;
  rc.rowf = 0.f;

  // Q codes of this lane's row, in the B-operand layout (16 channels per chunk).
  v4i qf[8];
  {
    const int8_t* qrow = a.q_i8 + ((long)my_t * a.n_q_heads + my_head) * kHeadDim + 16 * rc.h;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = row_ok ? *reinterpret_cast<const v4i*>(qrow + 32 * c) : v4i{0, 0, 0, 0};
    if (row_ok) rc.rowf = a.q_scale[(long)my_t * a.n_q_heads + my_head] * a.row_mul;
  }

  const TileBlocks tb = tile_blocks(qt, a.window_blocks, a.sink_blocks);
  const int n_it = (tb.n_total + 1) >> 1;
  const uint32_t kmask = key_mask(tb, n_it - 1, rc);

  // ---- pass 1: M2 = max over attended keys of z = s*log2(e) + log2(v_scale)
  float m2 = -INFINITY;
  for (int it = 0; it < n_it - 1; ++it) {
    __syncthreads();
    stage<NTHR, false>(sm, a, tb, it, kvh);
    __syncthreads();
    m2 = pass1_iter<false>(sm, qf, lane, rc, 0u, m2);
  }
  __syncthreads();
  stage<NTHR, false>(sm, a, tb, n_it - 1, kvh);
  __syncthreads();
  m2 = pass1_iter<true>(sm, qf, lane, rc, kmask, m2);
  m2 = xhalf_max(m2);

  // ---- pass 2: P' = exp2(z - M2) <= 1, codes, fixed-point digits, PV
  v16i acc[NPL][8];
#pragma unroll
  for (int p = 0; p < NPL; ++p)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[p][nt] = v16i{};
  float lsum = 0.f;
  for (int it = 0; it < n_it - 1; ++it) {
    __syncthreads();
    stage<NTHR, true>(sm, a, tb, it, kvh);
    __syncthreads();
    pass2_iter<NPL, false>(sm, qf, lane, rc, 0u, m2, lsum, acc);
  }
  __syncthreads();
  stage<NTHR, true>(sm, a, tb, n_it - 1, kvh);
  __syncthreads();
  pass2_iter<NPL, true>(sm, qf, lane, rc, kmask, m2, lsum, acc);

  // ---- epilogue: recombine digit planes, divide by Xmax * l, store
  constexpr float kXmax = FixedPoint<NPL>::kXmax;
  lsum = xhalf_sum(lsum);
  const float rinv = 1.0f / (kXmax * lsum);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * rc.h + (v & 3);  // output row of register v
    const float rr = __shfl(rinv, r);
    const int hig = head_lo + (r >> 4);
    const int t = qt * kPage + (r & 15);
    if (hig >= a.G || t >= a.n_tokens) continue;
    const long base = ((long)t * a.n_q_heads + kvh * a.G + hig) * kHeadDim + rho;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      float x = (float)acc[0][nt][v];
      if (NPL >= 2) x = fmaf((float)acc[1][nt][v], 256.f, x);
      if (NPL >= 3) x = fmaf((float)acc[2][nt][v], 65536.f, x);
      const float o = x * rr;
      if (OUT_BF16) {
        const uint32_t u32 = __float_as_uint(o);  // round to nearest even
        const uint16_t hb = (uint16_t)((u32 + 0x7fffu + ((u32 >> 16) & 1u)) >> 16);
        reinterpret_cast<uint16_t*>(a.out)[base + 32 * nt] = hb;
      } else {
        reinterpret_cast<float*>(a.out)[base + 32 * nt] = o;
      }
    }
  }
}

template <int WPG>
static void launch_wpg(const AttnArgs& a, bool out_bf16, unsigned grid, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((prefill_attn_kernel<WPA_NPL, WPG, true>), dim3(grid), dim3(64 * WPG), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<WPA_NPL, WPG, false>), dim3(grid), dim3(64 * WPG), 0, stream, a);
}

hipError_t launch_prefill_attn(const AttnArgs& args_in, bool out_bf16, hipStream_t stream) {
  AttnArgs a = args_in;
  a.G = a.n_q_heads / a.n_kv_heads;
  a.n_pairs = (a.G + 1) / 2;
  // waves per workgroup: the largest of 4, 2, 1 that divides the pair count,
  // so no wave is ever idle
  const int wpg = a.n_pairs % 4 == 0 ? 4 : (a.n_pairs % 2 == 0 ? 2 : 1);
  a.hgroups = a.n_pairs / wpg;
  a.n_tiles = (a.n_tokens + kPage - 1) / kPage;
  a.row_mul = a.softmax_scale * kLog2e;
  const unsigned grid = (unsigned)((long)a.n_tiles * a.n_kv_heads * a.hgroups);
  if (wpg == 4) launch_wpg<4>(a, out_bf16, grid, stream);
  else if (wpg == 2) launch_wpg<2>(a, out_bf16, grid, stream);
  else launch_wpg<1>(a, out_bf16, grid, stream);
  return hipGetLastError();
}

}  // namespace wpa
