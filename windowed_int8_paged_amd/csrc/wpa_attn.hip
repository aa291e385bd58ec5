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
//   * One workgroup = one 16-token query tile x one KV head x up to 4 of its
//     query heads, one wave per head (16 query rows).  A wave needs at most
//     256 registers, so two waves share each SIMD and the hardware overlaps
//     one wave's matrix work with the other's vector work.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_i32_16x16x64_i8 per 16-key page: a lane holds 4 keys of one query
//     row per page, so row reductions are in-lane plus two lane swaps.
//   * A step covers 64 keys (four pages).  P codes are exactly the
//     per-(row, 16-key block) int8 codes of the method; their weights ps*code
//     are written as one fixed-point integer relative to the row's largest
//     P*v_scale (found by a first QK pass) and split into two signed int8
//     digit planes, so PV runs at the full K = 64 rate with int32 accumulation
//     across every block and no per-block floating-point rescale.
//   * K and V pages go global -> LDS by asynchronous LDS DMA into row-major
//     XOR-swizzled tiles, double-buffered; V operands are gathered with the
//     transposing read ds_read_b64_tr_b8.

#include "wpa_common.h"
#include "wpa_launch.h"

namespace wpa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
#define WPA_LDS __attribute__((address_space(3)))
#define WPA_CONST __attribute__((address_space(4)))

constexpr int kStepKeys = 64;                 // keys per step (four pages)
constexpr int kStage = kStepKeys * kHeadDim;  // bytes of one staged K or V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeysPerGroup = 4;              // keys (rows) of one 1 KB copy group
constexpr float kTwo23 = 8388608.0f;  // 2^23 + v rounds v to an integer held in the low mantissa bits
// Fixed point of the PV weights: full scale Xmax = 127 * 256, relative to a
// cap that bounds every P' of the row (P' <= 1 up to exp2/log2 rounding).
constexpr float kXmax = 32512.f;
constexpr float kCap = 1.0f + 1.0f / 4096.0f;
// F = rint(f * 2^16) with f = mx * Xmax / (127 * cap) = mx * 256 / cap
constexpr float kFScale = 16777216.0f / kCap;
constexpr uint32_t kDigitBias = (128u << 16) + (1u << 15);  // digit offset 128, rounding half
constexpr float kTiny = 0x1p-60f;

// One stage buffer.  K and V tiles are row-major (row = key of the step, 256
// bytes) with the 16-byte chunk c of row r stored in slot c ^ swz(r).  The
// operand reads below then touch every bank once per half wave: the K reads
// see 16 consecutive rows of one page (slots r%16 ^ const), the transposing V
// reads rows 8h..8h+7 and 16+8h..16+8h+7 (slots m and 8 + m).
__device__ inline int swz(int r) { return (r & 15) ^ (((r >> 4) & 1) << 3); }
struct alignas(16) Stage {
  int8_t k[kStage];
  int8_t v[kStage];
  float sc[2][kStepKeys];  // [k_scale, v_scale][key]
};

// ---- cross-lane helpers: rows of 16 lanes R0..R3
__device__ inline void swap16(float& a, float& b) {  // a <-> odd rows of b, as one instruction
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ inline void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// all-reduce over the four 16-lane rows (same query row, different keys)
__device__ inline float rows_max(float x) {
  float y = x;
  swap16(x, y);
  x = fmaxf(x, y);
  y = x;
  swap32(x, y);
  return fmaxf(x, y);
}
__device__ inline float rows_sum(float x) {
  float y = x;
  swap16(x, y);
  x = x + y;
  y = x;
  swap32(x, y);
  return x + y;
}

// Physical pages of list entries 4s .. 4s+3, read through the scalar cache
// (entries past the end clamp to the last one; their keys are masked).  Entry
// li is block li for the sink part and win_start + li - n_sink after it.
struct Pages {
  int p[4];
};
__device__ inline Pages step_pages(const WPA_CONST int32_t* pt, const TileBlocks& tb, int step) {
  Pages pg;
  const int li0 = 4 * step;
  const int shift = tb.win_start - tb.n_sink;
  if (li0 + 3 < tb.n_total && (li0 >= tb.n_sink || li0 + 3 < tb.n_sink)) {
    // four consecutive blocks: one 16-byte scalar load
    const int b0 = li0 + (li0 >= tb.n_sink ? shift : 0);
    const v4i v = *reinterpret_cast<const WPA_CONST v4i*>(pt + b0);
    pg.p[0] = v[0];
    pg.p[1] = v[1];
    pg.p[2] = v[2];
    pg.p[3] = v[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int li = min(li0 + i, tb.n_total - 1);
      pg.p[i] = pt[li + (li >= tb.n_sink ? shift : 0)];
    }
  }
  return pg;
}

// Asynchronous global->LDS copy of 16 (or 4) bytes per lane: lane l's bytes
// land at lds_base + 16*l (4*l).  Issued as inline assembly so the compiler
// does not model the in-flight LDS write; the kernel orders it explicitly
// with wait_stage() and a workgroup barrier before any read of that buffer.
// The 16-byte form takes a scalar base address and a 32-bit per-lane offset.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const WPA_LDS void*)p;
}
__device__ inline void dma16(uint32_t voff, const int8_t* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ inline void dma4(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_base) : "memory", "m0");
}
__device__ inline void wait_stage() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row groups of 4 keys (1 KB of one page, one 16-byte chunk per lane) that a
// wave copies each step: g = wave + WPG*j for j < 16/WPG (K; V uses the same
// g + 16).  Their in-page byte offsets are per-lane constants, kept in
// registers so a copy costs no vector arithmetic.
template <int WPG>
struct DmaPlan {
  static constexpr int NJ = 16 / WPG;
  uint32_t voff[NJ];
};
template <int WPG>
__device__ inline void make_plan(DmaPlan<WPG>& pl, int row_bytes, int kvh, int wave, int lane) {
  const int q = lane >> 4, s = lane & 15;
#pragma unroll
  for (int j = 0; j < DmaPlan<WPG>::NJ; ++j) {
    const int g = wave + WPG * j;
    const int page = (WPG * j) >> 2;  // WPG divides 4, so this is g / 4
    const int rr = 4 * (g & 3) + q;   // row inside the page
    const int r = 16 * page + rr;     // row of the tile
    pl.voff[j] = (uint32_t)(rr * row_bytes + kvh * kHeadDim + 16 * (s ^ swz(r)));
  }
}

// Issue the copies of one step's four pages: K (and, for pass 2, V) row groups
// shared over the waves, plus the 64 K and 64 V scales.
template <int WPG, bool WITH_V>
__device__ inline void issue_stage(Stage& st, const AttnArgs& a, const DmaPlan<WPG>& pl, long page_bytes, int kvh,
                                   const Pages& pg, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < DmaPlan<WPG>::NJ; ++j) {
    const int page = (WPG * j) >> 2;
    const int g = wave + WPG * j;
    const long pbase = (long)pg.p[page] * page_bytes;
    dma16(pl.voff[j], a.k_pool + pbase, lds_addr(st.k + kKeysPerGroup * kHeadDim * g));
    if (WITH_V) dma16(pl.voff[j], a.v_pool + pbase, lds_addr(st.v + kKeysPerGroup * kHeadDim * g));
  }
  // k_scale by wave 0, v_scale by wave 1 (both by wave 0 when WPG == 1):
  // lane l copies the scale of key l, page l/16
  const int q = lane >> 4, s = lane & 15;
  const int odd = -(q & 1), high = -((q >> 1) & 1);
  const int lo = pg.p[0] ^ ((pg.p[0] ^ pg.p[1]) & odd);
  const int hi = pg.p[2] ^ ((pg.p[2] ^ pg.p[3]) & odd);
  const int ppage = lo ^ ((lo ^ hi) & high);
  const long sidx = ((long)ppage * kPage + s) * a.n_kv_heads + kvh;
  if (wave == 0) dma4(a.k_scale + sidx, lds_addr(&st.sc[0][0]));
  if (wave == (WPG > 1 ? 1 : 0)) dma4(a.v_scale + sidx, lds_addr(&st.sc[1][0]));
}

// S^T of the step: for page p, lane l holds query row l%16 and keys
// 4(l/16) + i of that page in register i.
__device__ inline void qk_step(const int8_t* kb, const v4i (&qf)[4], int lane, v4i (&s)[4]) {
  const int g = lane >> 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 16 * p + (lane & 15);
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int slot = (4 * c + g) ^ swz(r);
      const v4i kf = *reinterpret_cast<const v4i*>(kb + r * kHeadDim + 16 * slot);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf, qf[c], acc, 0, 0, 0);
    }
    s[p] = acc;
  }
}

// Per-lane constants of one wave.
struct RowCtx {
  int g;       // 16-lane row of the wave (0..3)
  float rowf;  // q_scale * softmax_scale * log2(e) of this lane's query row
  int t_mask;  // causal bound of this lane's query row
};

// Attended keys among the 16 score registers (p, i) of a step; only the last
// step of a tile holds the diagonal block or empty list slots.
__device__ inline uint32_t key_mask(const TileBlocks& tb, int step, const RowCtx& rc) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int li = 4 * step + p;
    const int blk = li < tb.n_total ? tb.block(li) : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (li < tb.n_total) && (kPage * blk + 4 * rc.g + i <= rc.t_mask);
      m |= (ok ? 1u : 0u) << (4 * p + i);
    }
  }
  return m;
}

// Pass 1: running max of z = score*log2(e) + log2(v_scale) = (acc*k_scale)*rowf
// + log2(v_scale).  Its row maximum Z makes P' = exp2(z - Z) <= 1 in pass 2,
// so the row's largest P' is 1 and fixes the fixed-point scale.  Each lane
// takes one log2 (key = lane) and the wave shares them through its own LDS
// slice.
template <bool MASKED>
__device__ inline void pass1_step(const Stage& st, float* lvs_w, const v4i (&qf)[4], int lane, const RowCtx& rc,
                                  uint32_t kmask, float& zmax) {
  lvs_w[lane] = __builtin_amdgcn_logf(st.sc[1][lane]);
  v4i s[4];
  qk_step(st.k, qf, lane, s);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float4 ks4 = *reinterpret_cast<const float4*>(&st.sc[0][16 * p + 4 * rc.g]);
    const float4 lv4 = *reinterpret_cast<const float4*>(&lvs_w[16 * p + 4 * rc.g]);
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = fmaf((float)s[p][i] * (&ks4.x)[i], rc.rowf, (&lv4.x)[i]);
      if (MASKED) z[i] = ((kmask >> (4 * p + i)) & 1u) ? z[i] : -INFINITY;
    }
    zmax = fmaxf(fmaxf(zmax, fmaxf(z[0], z[1])), fmaxf(z[2], z[3]));
  }
  __builtin_amdgcn_wave_barrier();
}

// Pass 2: e = exp2(z - Z - log2 v_scale) = P, l += P, P' = P * v_scale <= 1,
// per-page codes code = rint(P' * 127 / max P'), their weights ps * code as
// the fixed-point integer x = rint(code * f), f = max P' * Xmax / (127 * cap),
// split into two signed int8 digit planes x = d0 + 256 d1, then PV.
//
// code * f is formed as (code * F + 2^15) >> 16 with F = rint(f * 2^16) < 2^24
// by one 24-bit multiply-add; with a bias of 128 in the upper half, bytes 2
// and 3 of the result are d0 + 128 and d1.
template <bool MASKED>
__device__ inline void pass2_step(const Stage& st, const v4i (&qf)[4], int lane, const RowCtx& rc, uint32_t kmask,
                                  float neg_z, float& lsum, v4i (&acc)[2][16]) {
  v4i s[4];
  qk_step(st.k, qf, lane, s);
  float pp[4][4];
  float mx[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float4 ks4 = *reinterpret_cast<const float4*>(&st.sc[0][16 * p + 4 * rc.g]);
    const float4 vs4 = *reinterpret_cast<const float4*>(&st.sc[1][16 * p + 4 * rc.g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e = __builtin_amdgcn_exp2f(fmaf((float)s[p][i] * (&ks4.x)[i], rc.rowf, neg_z));
      float pv = e * (&vs4.x)[i];
      if (MASKED) {
        const bool ok = (kmask >> (4 * p + i)) & 1u;
        e = ok ? e : 0.f;
        pv = ok ? pv : 0.f;
      }
      lsum += e;
      pp[p][i] = pv;
    }
    mx[p] = fmaxf(fmaxf(pp[p][0], pp[p][1]), fmaxf(pp[p][2], pp[p][3]));
  }
  // page maxima over the four 16-lane rows: afterwards every lane holds all four
  {
    float a = mx[0], b = mx[1], c = mx[2], d = mx[3];
    swap16(a, b);
    const float x01 = fmaxf(a, b);  // R0: p0(R0,R1)  R1: p1(R0,R1)  R2: p0(R2,R3)  R3: p1(R2,R3)
    swap16(c, d);
    const float x23 = fmaxf(c, d);
    float e0 = x01, e1 = x23;
    swap32(e0, e1);
    const float y = fmaxf(e0, e1);  // row Rk holds the full max of page k
    float g0 = y, g1 = y;
    swap16(g0, g1);  // rows 0,1: (M0, M1); rows 2,3: (M2, M3)
    float m0 = g0, m2 = g0, m1 = g1, m3 = g1;
    swap32(m0, m2);  // every lane: m0 = M0, m2 = M2
    swap32(m1, m3);
    mx[0] = m0;
    mx[1] = m1;
    mx[2] = m2;
    mx[3] = m3;
  }
  v4i dig[2];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // pages weighing below 2^-60 of the cap round to zero in this fixed point
    const bool live = mx[p] > kTiny;
    const float inv = live ? 127.0f * __builtin_amdgcn_rcpf(mx[p]) : 0.f;
    const uint32_t F = (uint32_t)fmaf(mx[p], kFScale, 0.5f);
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t code = __float_as_uint(fmaf(pp[p][i], inv, kTwo23));  // 2^23 + rint(P' * inv)
      r[i] = __umul24(code, F) + kDigitBias;
    }
    const uint32_t w01 = __builtin_amdgcn_perm(r[1], r[0], 0x07060302u);
    const uint32_t w23 = __builtin_amdgcn_perm(r[3], r[2], 0x07060302u);
    dig[0][p] = (int)(__builtin_amdgcn_perm(w23, w01, 0x06040200u) ^ 0x80808080u);  // low digit, signed
    dig[1][p] = (int)__builtin_amdgcn_perm(w23, w01, 0x07050301u);                 // high digit
  }

  // V operand: lane (row g, column j) needs 16 keys of channel 16nt + j in the
  // slot order of P: slot b holds key 16(b/4) + 4g + b%4.  Two transposing
  // reads give slots 0-7 (pages 0, 1) and 8-15 (pages 2, 3).
  const int j = lane & 15;
  const int kk = j >> 1;
  const int key1 = 16 * (kk >> 2) + 4 * rc.g + (kk & 3);
  const int8_t* row1 = st.v + key1 * kHeadDim + 8 * (j & 1);
  const int8_t* row2 = row1 + 32 * kHeadDim;  // key1 + 32
  const int sw = swz(key1);
  const int sw2 = swz(key1 + 32);
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) {
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((WPA_LDS v2i*)(row1 + 16 * (nt ^ sw)));
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((WPA_LDS v2i*)(row2 + 16 * (nt ^ sw2)));
    const v4i vf = {lo.x, lo.y, hi.x, hi.y};
    acc[0][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dig[0], vf, acc[0][nt], 0, 0, 0);
    acc[1][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dig[1], vf, acc[1][nt], 0, 0, 0);
  }
}

template <int WPG, bool OUT_BF16>
__global__ __launch_bounds__(64 * WPG, 2) void prefill_attn_kernel(AttnArgs a, const int32_t* __restrict__ pt_arg) {
  __shared__ Stage st[2];
  __shared__ alignas(16) float lvs[WPG][kStepKeys];  // per-wave log2(v_scale) of the step
  const WPA_CONST int32_t* pt = (const WPA_CONST int32_t*)pt_arg;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  int u = blockIdx.x;
  const int hg = u % a.hgroups;
  u /= a.hgroups;
  const int kvh = u % a.n_kv_heads;
  const int qt = a.n_tiles - 1 - u / a.n_kv_heads;  // longest tiles first

  const int head = kvh * a.G + hg * WPG + wave;  // WPG divides G: every wave has a head
  const int my_t = qt * kPage + (lane & 15);
  const bool row_ok = my_t < a.n_tokens;

  RowCtx rc;
  rc.g = lane >> 4;
  rc.t_mask = row_ok ? my_t : a.n_tokens - 1;

  const TileBlocks tb = tile_blocks(qt, a.window_blocks, a.sink_blocks);
  const int n_st = (tb.n_total + 3) >> 2;
  const uint32_t kmask = key_mask(tb, n_st - 1, rc);

  const int row_bytes = a.n_kv_heads * kHeadDim;
  const long page_bytes = (long)kPage * row_bytes;
  DmaPlan<WPG> plan;
  make_plan<WPG>(plan, row_bytes, kvh, wave, lane);

  // Start streaming the first pages before anything else.
  const Pages pg0 = step_pages(pt, tb, 0);
  issue_stage<WPG, false>(st[0], a, plan, page_bytes, kvh, pg0, wave, lane);

  // Q codes of this lane's row in the B-operand layout (16 channels per chunk);
  // rows past the end read the last token and are never stored.
  v4i qf[4];
  {
    const int tq = row_ok ? my_t : a.n_tokens - 1;
    const int8_t* qrow = a.q_i8 + ((long)tq * a.n_q_heads + head) * kHeadDim + 16 * rc.g;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *reinterpret_cast<const v4i*>(qrow + 64 * c);
    rc.rowf = row_ok ? a.q_scale[(long)tq * a.n_q_heads + head] * a.row_mul : 0.f;
  }

  // The 2*n_st steps (pass 1, then pass 2 over the same page list) alternate
  // between the two buffers.  A step waits for its own copies, syncs (every
  // wave is then done with the other buffer), issues the next step's copies
  // into the other buffer, then computes on its own.
  const int n_all = 2 * n_st;
  auto pages_of = [&](int step) { return step_pages(pt, tb, step < n_st ? step : step - n_st); };
  Pages pg_next = pages_of(1 < n_all ? 1 : 0);
  float* lvs_w = lvs[wave];

  // ---- pass 1: row max of score*log2e + log2(v_scale)
  float zmax = -INFINITY;
  int buf = 0;
  for (int it = 0; it + 1 < n_st; ++it) {
    wait_stage();
    __syncthreads();
    issue_stage<WPG, false>(st[buf ^ 1], a, plan, page_bytes, kvh, pg_next, wave, lane);
    pg_next = pages_of(it + 2);
    pass1_step<false>(st[buf], lvs_w, qf, lane, rc, 0u, zmax);
    buf ^= 1;
  }
  wait_stage();
  __syncthreads();
  issue_stage<WPG, true>(st[buf ^ 1], a, plan, page_bytes, kvh, pg_next, wave, lane);  // pass 2, first step
  pg_next = pages_of(n_st + 1 < n_all ? n_st + 1 : n_st);
  pass1_step<true>(st[buf], lvs_w, qf, lane, rc, kmask, zmax);
  buf ^= 1;

  const float neg_z = -rows_max(zmax);

  // ---- pass 2
  v4i acc[2][16];
#pragma unroll
  for (int pl = 0; pl < 2; ++pl)
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) acc[pl][nt] = v4i{0, 0, 0, 0};
  float lsum = 0.f;
  for (int it = 0; it + 1 < n_st; ++it) {
    wait_stage();
    __syncthreads();
    issue_stage<WPG, true>(st[buf ^ 1], a, plan, page_bytes, kvh, pg_next, wave, lane);
    if (n_st + it + 2 < n_all) pg_next = pages_of(n_st + it + 2);
    pass2_step<false>(st[buf], qf, lane, rc, 0u, neg_z, lsum, acc);
    buf ^= 1;
  }
  wait_stage();
  __syncthreads();
  pass2_step<true>(st[buf], qf, lane, rc, kmask, neg_z, lsum, acc);

  // ---- epilogue: recombine the digit planes, scale by cap / (Xmax * l), store.
  // Output register i of tile nt is row 4g + i, channel 16nt + lane%16.
  lsum = rows_sum(lsum);
  const float rscale = kCap / (kXmax * lsum);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * rc.g + i;
    const float rr = __shfl(rscale, r);
    const int t = qt * kPage + r;
    if (t >= a.n_tokens) continue;
    const long base = ((long)t * a.n_q_heads + head) * kHeadDim + (lane & 15);
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      const float x = fmaf((float)acc[1][nt][i], 256.f, (float)acc[0][nt][i]);
      const float o = x * rr;
      if (OUT_BF16) {
        const uint32_t u32 = __float_as_uint(o);  // round to nearest even
        const uint16_t hb = (uint16_t)((u32 + 0x7fffu + ((u32 >> 16) & 1u)) >> 16);
        reinterpret_cast<uint16_t*>(a.out)[base + 16 * nt] = hb;
      } else {
        reinterpret_cast<float*>(a.out)[base + 16 * nt] = o;
      }
    }
  }
}

template <int WPG>
static void launch_wpg(const AttnArgs& a, bool out_bf16, unsigned grid, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((prefill_attn_kernel<WPG, true>), dim3(grid), dim3(64 * WPG), 0, stream, a, a.page_table);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<WPG, false>), dim3(grid), dim3(64 * WPG), 0, stream, a, a.page_table);
}

hipError_t launch_prefill_attn(const AttnArgs& args_in, bool out_bf16, hipStream_t stream) {
  AttnArgs a = args_in;
  a.G = a.n_q_heads / a.n_kv_heads;
  // waves (query heads) per workgroup: the largest of 4, 2, 1 dividing G
  const int wpg = a.G % 4 == 0 ? 4 : (a.G % 2 == 0 ? 2 : 1);
  a.hgroups = a.G / wpg;
  a.n_tiles = (a.n_tokens + kPage - 1) / kPage;
  a.row_mul = a.softmax_scale * kLog2e;
  const unsigned grid = (unsigned)((long)a.n_tiles * a.n_kv_heads * a.hgroups);
  if (wpg == 4) launch_wpg<4>(a, out_bf16, grid, stream);
  else if (wpg == 2) launch_wpg<2>(a, out_bf16, grid, stream);
  else launch_wpg<1>(a, out_bf16, grid, stream);
  return hipGetLastError();
}

}  // namespace wpa
