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
#define WPA_NPL 2
#endif

namespace wpa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
#define WPA_LDS __attribute__((address_space(3)))

constexpr int kItKeys = 32;                 // keys per loop iteration (two pages)
constexpr int kStage = kItKeys * kHeadDim;  // bytes of one staged K or V tile
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

// One stage buffer.  K and V tiles are row-major (row = key of the
// iteration, 256 bytes) with the 16-byte chunk c of row r stored in slot
// c ^ (r & 15), so the operand reads below hit all 64 banks once.  The two
// buffers are separate LDS objects so the compiler can tell that reads of one
// never alias the asynchronous copies into the other.
struct alignas(16) Stage {
  int8_t k[kStage];
  int8_t v[kStage];
  float sc[2][kItKeys];  // [k_scale, v_scale][key]
};

__device__ inline float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Physical pages of list entries 2it and 2it+1 (an empty second slot reuses
// the first page: its keys are masked).
struct PagePair {
  long p0, p1;
};
__device__ inline PagePair page_pair(const int32_t* __restrict__ pt, const TileBlocks& tb, int it) {
  const int li = 2 * it;
  const int b0 = tb.block(li);
  const int b1 = li + 1 < tb.n_total ? tb.block(li + 1) : b0;
  PagePair pp;
  pp.p0 = pt[b0];
  pp.p1 = pt[b1];
  return pp;
}

// Asynchronous global->LDS copy of 16 (or 4) bytes per lane: lane l's bytes
// land at lds_base + 16*l (4*l).  Issued as inline assembly so the compiler
// does not model the in-flight LDS write; the kernel orders it explicitly
// with wait_stage() and a workgroup barrier before any read of that buffer.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const WPA_LDS void*)p;
}
__device__ inline void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory", "m0");
}
__device__ inline void dma4(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_base) : "memory", "m0");
}

// Issue the copies of one iteration's two pages: 8 K and 8 V row groups of 4
// rows (1 KB, one 16-byte chunk per lane), shared out over the workgroup's
// waves, plus the 32 K and 32 V scales.
template <int WPG>
__device__ inline void issue_stage(Stage& st, const AttnArgs& a, int kvh, PagePair pg, int wave, int lane) {
  const long row_bytes = (long)a.n_kv_heads * kHeadDim;
  const int s = lane & 15;
#pragma unroll
  for (int j = 0; j < 16 / WPG; ++j) {
    const int g = wave + WPG * j;  // wave-uniform
    const bool isv = g >= 8;
    const int r0 = 4 * (g & 7);
    const int r = r0 + (lane >> 4);
    const long phys = r < 16 ? pg.p0 : pg.p1;
    const int8_t* src = (isv ? a.v_pool : a.k_pool) + (phys * kPage + (r & 15)) * row_bytes +
                        (long)kvh * kHeadDim + 16 * (s ^ (r & 15));
    dma16(src, lds_addr((isv ? st.v : st.k) + r0 * kHeadDim));
  }
  if (wave == 0) {
    const int key = lane & 31;
    const long phys = key < 16 ? pg.p0 : pg.p1;
    const float* src = (lane < 32 ? a.k_scale : a.v_scale) + (phys * kPage + (key & 15)) * a.n_kv_heads + kvh;
    dma4(src, lds_addr(&st.sc[0][0]));
  }
}

__device__ inline void wait_stage() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// S^T for the 32 staged keys x this wave's 32 query rows: lane l owns query
// row l%32 and keys 8(v/4) + 4(l/32) + v%4 of register v.  Both operands come
// from LDS tiles with the chunk swizzle c ^ (row & 15).
__device__ inline v16i qk_tile(const int8_t* kb, const int8_t* qb, int lane) {
  v16i s = {};
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int slot = (2 * c + h) ^ (r & 15);
    const v4i kf = *reinterpret_cast<const v4i*>(kb + r * kHeadDim + 16 * slot);
    const v4i qf = *reinterpret_cast<const v4i*>(qb + r * kHeadDim + 16 * slot);
    s = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf, s, 0, 0, 0);
  }
  return s;
}

// Per-lane constants of one wave.
struct RowCtx {
  int h;       // half of the wave (0/1)
  float rowf;  // q_scale * softmax_scale * log2(e) of this lane's row
  int t_mask;  // causal bound of this lane's row
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

// Pass 1: running max of u = acc * k_scale (the row's scores up to the
// positive factor rowf) and of z = u*rowf + log2(v_scale), whose max fixes the
// row's largest P*v_scale.
template <bool MASKED>
__device__ inline void pass1_iter(const Stage& st, const int8_t* qb, int lane, const RowCtx& rc,
                                  uint32_t kmask, float& umax, float& zmax) {
  const v16i s = qk_tile(st.k, qb, lane);
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 ks4 = *reinterpret_cast<const float4*>(&st.sc[0][8 * i4 + 4 * rc.h]);
    const float4 vs4 = *reinterpret_cast<const float4*>(&st.sc[1][8 * i4 + 4 * rc.h]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * i4 + k;
      float u = (float)s[v] * (&ks4.x)[k];
      float z = fmaf(u, rc.rowf, __builtin_amdgcn_logf((&vs4.x)[k]));
      if (MASKED) {
        const bool ok = (kmask >> v) & 1u;
        u = ok ? u : -INFINITY;
        z = ok ? z : -INFINITY;
      }
      umax = fmaxf(umax, u);
      zmax = fmaxf(zmax, z);
    }
  }
}

// Pass 2: P = exp2(u*rowf - Mt) <= 1, l += P, P' = P*v_scale, per-page codes,
// fixed-point digit planes relative to the row cap (largest P'), PV.
template <int NPL, bool MASKED>
__device__ inline void pass2_iter(const Stage& st, const int8_t* qb, int lane, const RowCtx& rc,
                                  uint32_t kmask, float neg_mt, float crow, float cap, float& lsum,
                                  v16i (&acc)[NPL][8]) {
  const v16i s = qk_tile(st.k, qb, lane);
  float pp[16];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 ks4 = *reinterpret_cast<const float4*>(&st.sc[0][8 * i4 + 4 * rc.h]);
    const float4 vs4 = *reinterpret_cast<const float4*>(&st.sc[1][8 * i4 + 4 * rc.h]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * i4 + k;
      const float u = (float)s[v] * (&ks4.x)[k];
      float p = __builtin_amdgcn_exp2f(fmaf(u, rc.rowf, neg_mt));
      float pv = p * (&vs4.x)[k];
      if (MASKED) {
        const bool ok = (kmask >> v) & 1u;
        p = ok ? p : 0.f;
        pv = ok ? pv : 0.f;
      }
      lsum += p;
      pp[v] = pv;
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
  // A block whose largest P' is below 2^-60 of the row cap weighs nothing at
  // this fixed-point resolution: its codes are irrelevant (and 127/mx could
  // overflow), so they are set to 0.
  const float inv0 = mx0 > 0x1p-60f * cap ? 127.0f / mx0 : 0.f;
  const float inv1 = mx1 > 0x1p-60f * cap ? 127.0f / mx1 : 0.f;
  const float f0 = mx0 * crow;  // ps * Xmax / cap of the row
  const float f1 = mx1 * crow;

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

  // V operand: 16 keys of one channel per lane, gathered by two transposing
  // reads; slot b holds key 8(b/4) + 4h + b%4, the same key as P's byte b.
  const int i = lane & 15;
  const int kk = i >> 1;
  const int key1 = 8 * (kk >> 2) + 4 * rc.h + (kk & 3);
  const int8_t* vb = st.v;
  const int8_t* row1 = vb + key1 * kHeadDim + 8 * (i & 1);
  const int8_t* row2 = row1 + 16 * kHeadDim;  // key1 + 16, same swizzle
  const int sw = key1 & 15;
  const int half16 = (lane >> 4) & 1;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int slot = (2 * nt + half16) ^ sw;
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((WPA_LDS v2i*)(row1 + 16 * slot));
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((WPA_LDS v2i*)(row2 + 16 * slot));
    const v4i vf = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int p = 0; p < NPL; ++p) acc[p][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(dig[p], vf, acc[p][nt], 0, 0, 0);
  }
}

template <int NPL, int WPG, bool OUT_BF16>
__global__ __launch_bounds__(64 * WPG, 1) void prefill_attn_kernel(AttnArgs a, const int32_t* __restrict__ pt) {
  __shared__ Stage st[2];
  __shared__ alignas(16) int8_t q_lds[WPG][32 * kHeadDim];  // each wave's 32 query rows
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  const TileBlocks tb = tile_blocks(qt, a.window_blocks, a.sink_blocks);
  const int n_it = (tb.n_total + 1) >> 1;
  const uint32_t kmask = key_mask(tb, n_it - 1, rc);

  // Start streaming the first pages before anything else.
  const PagePair pg0 = page_pair(pt, tb, 0);
  issue_stage<WPG>(st[0], a, kvh, pg0, wave, lane);

  // This wave's 32 query rows (codes) into LDS, same chunk swizzle as K.
  // Rows without a token or head (ragged tail, odd G) copy a valid row; their
  // row factor is 0 and they are never stored.
  {
    const int s16 = lane & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int hq = head_lo + (r >> 4) < a.G ? kvh * a.G + head_lo + (r >> 4) : kvh * a.G;
      const int tq = qt * kPage + (r & 15) < a.n_tokens ? qt * kPage + (r & 15) : a.n_tokens - 1;
      const int8_t* src = a.q_i8 + ((long)tq * a.n_q_heads + hq) * kHeadDim + 16 * (s16 ^ (r & 15));
      dma16(src, lds_addr(&q_lds[wave][4 * j * kHeadDim]));
    }
  }
  const int8_t* qb = q_lds[wave];
  if (row_ok) rc.rowf = a.q_scale[(long)my_t * a.n_q_heads + my_head] * a.row_mul;

  // The 2*n_it steps (pass 1, then pass 2 over the same page list) alternate
  // between the two buffers.  A step waits for its own copies, syncs (every
  // wave is then done with the other buffer), issues the next step's copies
  // into the other buffer, then computes on its own.
  const int n_steps = 2 * n_it;
  auto pages_of_step = [&](int step) { return page_pair(pt, tb, step < n_it ? step : step - n_it); };
  PagePair pg_next = pages_of_step(1 < n_steps ? 1 : 0);

  // ---- pass 1: row max of the scores and of score*log2e + log2(v_scale)
  float umax = -INFINITY, zmax = -INFINITY;
  int buf = 0;
  for (int it = 0; it + 1 < n_it; ++it) {
    wait_stage();
    __syncthreads();
    issue_stage<WPG>(st[buf ^ 1], a, kvh, pg_next, wave, lane);
    pg_next = pages_of_step(it + 2);
    pass1_iter<false>(st[buf], qb, lane, rc, 0u, umax, zmax);
    buf ^= 1;
  }
  wait_stage();
  __syncthreads();
  issue_stage<WPG>(st[buf ^ 1], a, kvh, pg_next, wave, lane);  // pass 2, entry 0
  pg_next = pages_of_step(n_it + 1 < n_steps ? n_it + 1 : n_it);
  pass1_iter<true>(st[buf], qb, lane, rc, kmask, umax, zmax);
  buf ^= 1;

  umax = xhalf_max(umax);
  zmax = xhalf_max(zmax);
  const float mt = umax * rc.rowf;
  const float neg_mt = -mt;
  // cap = largest P' of the row (with P = exp2(score*log2e - Mt) <= 1); the
  // small factor covers rounding between the two passes
  const float cap = __builtin_amdgcn_exp2f(zmax - mt) * (1.0f + 1.0f / 4096.0f);
  constexpr float kXmax = FixedPoint<NPL>::kXmax;
  const float crow = kXmax / (127.0f * cap);

  // ---- pass 2
  v16i acc[NPL][8];
#pragma unroll
  for (int p = 0; p < NPL; ++p)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[p][nt] = v16i{};
  float lsum = 0.f;
  for (int it = 0; it + 1 < n_it; ++it) {
    wait_stage();
    __syncthreads();
    issue_stage<WPG>(st[buf ^ 1], a, kvh, pg_next, wave, lane);
    if (n_it + it + 2 < n_steps) pg_next = pages_of_step(n_it + it + 2);
    pass2_iter<NPL, false>(st[buf], qb, lane, rc, 0u, neg_mt, crow, cap, lsum, acc);
    buf ^= 1;
  }
  wait_stage();
  __syncthreads();
  pass2_iter<NPL, true>(st[buf], qb, lane, rc, kmask, neg_mt, crow, cap, lsum, acc);

  // ---- epilogue: recombine digit planes, scale by cap / (Xmax * l), store
  lsum = xhalf_sum(lsum);
  const float rscale = cap / (kXmax * lsum);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * rc.h + (v & 3);  // output row of register v
    const float rr = __shfl(rscale, r);
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
    hipLaunchKernelGGL((prefill_attn_kernel<WPA_NPL, WPG, true>), dim3(grid), dim3(64 * WPG), 0, stream, a,
                       a.page_table);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<WPA_NPL, WPG, false>), dim3(grid), dim3(64 * WPG), 0, stream, a,
                       a.page_table);
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
