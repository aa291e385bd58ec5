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
//   * One launch.  A workgroup = four waves on one KV head: 4 of its query
//     heads on one 16-token query tile, or, with 2 (1) query heads per
//     workgroup, 2 heads on 2 consecutive tiles (1 head on 4 tiles) walking
//     the union of their key lists, so every staged K/V page feeds four
//     waves whatever the GQA ratio.  A wave takes one head of one tile (16
//     query rows) and needs at most 256 registers, so two waves share each
//     SIMD.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_i32_16x16x64_i8 per 16-key page: a lane holds 4 keys of one query
//     row per page, so row reductions are in-lane plus lane swaps.
//   * A step covers 64 keys (four pages).  P codes are exactly the
//     per-(row, 16-key block) int8 codes of the method; their weights ps*code
//     are written as one fixed-point integer relative to a per-row reference
//     2^zref and split into two signed int8 digit planes, so PV runs at the
//     full K = 64 rate with int32 accumulation across every block and no
//     per-block floating-point rescale.
//   * The reference is raised as the scores come in: before a step's weights
//     are formed, a row whose largest z = score*log2(e) + log2(v_scale) passes
//     zref gets zref = ceil(z) + 1, and what the row has accumulated (two
//     int32 planes, l) is shifted right by the whole number of bits zref
//     moved.  So every P*v_scale stays <= 1 and the row's largest lies within
//     a factor 4 of it.  P codes depend only on ratios inside their block, so
//     the reference does not change them.
//   * K and V pages go global -> LDS by asynchronous LDS DMA (each wave copies
//     whole pages) into row-major XOR-swizzled tiles, double-buffered; LDS
//     fragment reads are software-pipelined ahead of their matrix products;
//     V operands are gathered with the transposing read ds_read_b64_tr_b8.
//   * From bf16 Q (the fused entry point) each wave quantizes its own rows as
//     it loads them, by the same formula as the separate quantize kernel.

#include "wpa_common.h"
#include "wpa_lanes.h"
#include "wpa_launch.h"

namespace wpa {

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
// The per-row reference: raised to ceil(row max) + kRefHeadroom when the
// row's maximum passes it.  The two int32 planes of a row hold the value
// 256 hi + lo; it is divided by 2^d with floor, exactly, in stages of at most
// kStageShift bits (the carried remainder << 8 stays in int32).  With
// |256 hi + lo| < 2^40, two stages (kMaxShift bits) take any value to 0 or -1,
// which is what any larger floor shift gives.
constexpr float kRefHeadroom = 1.f;
constexpr int kStageShift = 22;
constexpr float kMaxShift = 2.f * kStageShift;
// log2(v_scale) enters the reference as log2(max(v_scale, kVsFloor)): a zero
// v_scale (the KV writer's scale of an all-zero V row) still sets a finite
// reference, and every e = exp2(score * log2(e) - zref) stays below 2^63
// (P' = e * v_scale is unchanged).
constexpr float kVsFloor = 0x1p-64f;

// Scales of page p of the step: sc[p][0..15] k_scale, sc[p][16..31] v_scale
// of its 16 keys (one 256-byte copy per page; slots 32..63 repeat them, and
// slots 32..47 then take log2(v_scale) of the keys).
struct alignas(16) Stage {
  int8_t k[kStage];
  int8_t v[kStage];
  float sc[4][64];
};
// Each wave copies 4/WPG whole pages of a step: list entries
// 4s + wave*PPW + i.  Their physical pages are read through the scalar cache
// (entries past the end clamp to the last one; their keys are masked).  The
// copies clamp the page ids themselves into the pool.
template <int WPG>
struct WavePages {
  static constexpr int PPW = 4 / WPG;
  int p[PPW];
};
template <int WPG>
__device__ inline WavePages<WPG> wave_pages(const WPA_CONST int32_t* pt, const TileBlocks& tb, int step, int wave) {
  WavePages<WPG> pg;
#pragma unroll
  for (int i = 0; i < WavePages<WPG>::PPW; ++i) {
    const int li = min(4 * step + wave * WavePages<WPG>::PPW + i, tb.n_total - 1);
    pg.p[i] = pt[tb.block(li)];
  }
  return pg;
}

// Asynchronous global->LDS copy of 16 (or 4) bytes per lane: lane l's bytes
// land at lds_base + 16*l (4*l).  Issued as inline assembly so the compiler
// does not model the in-flight LDS write; the kernel orders it explicitly
// with wait_stage() and a workgroup barrier before any read of that buffer.
// The 16-byte form takes a scalar base address and a 32-bit per-lane offset.
// m0 carries the LDS address and is set right before each copy; the compiler
// warns about clobbering a reserved register, but on gfx950 nothing it emits
// in these kernels reads m0 (every m0 in their assembly belongs to a copy).
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
// vmcnt(0) through the builtin, so the compiler's own wait tracking sees it:
// registers filled by earlier vector loads (Q codes, scales) then count as
// ready, and no wait on the in-flight copies is inserted before their uses.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline void wait_stage() {
  asm volatile("" ::: "memory");
  wait_vmem();
  asm volatile("" ::: "memory");
}

// A wave's copies per step: for each of its pages, four 1 KB row groups
// (keys 4j .. 4j+3, one 16-byte chunk per lane) of K (and V), and one 256-byte
// copy of the page's 16 k_scales and 16 v_scales.  The per-lane parts of the
// addresses are constants kept in registers, so a copy costs one scalar
// base per page and no vector arithmetic.
template <int WPG>
struct DmaPlan {
  static constexpr int PPW = 4 / WPG;
  uint32_t voff[4 * PPW];  // byte offset inside a page, LDS swizzle applied
  const float* sptr;       // lane l: k_scale (l/16 even) or v_scale (odd) of key l%16 of page 0
};
template <int WPG>
__device__ inline void make_plan(DmaPlan<WPG>& pl, const AttnArgs& a, int kvh, int wave, int lane) {
  constexpr int PPW = DmaPlan<WPG>::PPW;
  const int q = lane >> 4, s = lane & 15;
  const int row_bytes = a.n_kv_heads * kHeadDim;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int p = wave * PPW + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 4 * j + q;  // key inside the page
      pl.voff[4 * i + j] = (uint32_t)(rr * row_bytes + kvh * kHeadDim + 16 * (s ^ swz(16 * p + rr)));
    }
  }
  pl.sptr = ((q & 1) ? a.v_scale : a.k_scale) + s * a.n_kv_heads + kvh;
}

template <int WPG, bool WITH_V, class S>
__device__ inline void issue_stage(S& st, const AttnArgs& a, const DmaPlan<WPG>& pl, uint32_t page_bytes,
                                   uint32_t scale_stride, const WavePages<WPG>& pg, int wave) {
  constexpr int PPW = DmaPlan<WPG>::PPW;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int p = wave * PPW + i;
    // a page id outside the pool is clamped into it: a wrong page, never memory outside
    const uint32_t page = (uint32_t)min(max(pg.p[i], 0), a.n_pool_pages - 1);
    const uint64_t off = (uint64_t)page * page_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dma16(pl.voff[4 * i + j], a.k_pool + off, lds_addr(st.k + kKeysPerGroup * kHeadDim * (4 * p + j)));
      if constexpr (WITH_V)
        dma16(pl.voff[4 * i + j], a.v_pool + off, lds_addr(st.v + kKeysPerGroup * kHeadDim * (4 * p + j)));
    }
    dma4(pl.sptr + (uint64_t)page * scale_stride, lds_addr(&st.sc[p][0]));
  }
}

// Per-lane constants of one wave.
struct RowCtx {
  int g;       // 16-lane row of the wave (0..3)
  int t_mask;  // causal bound of this lane's query row
};

// Attended keys among the 16 score registers (p, i) of step `step` of the
// group's key list tb, for a lane of a wave whose own tile is tw: a block
// counts if it is one of tw's sinks or lies in tw's window, and a key if it is
// not after the lane's row.  Only a wave's first and last steps need it.
__device__ inline uint32_t key_mask(const TileBlocks& tb, const TileBlocks& tw, int step, const RowCtx& rc) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int li = 4 * step + p;
    const bool listed = li < tb.n_total;
    const int blk = listed ? tb.block(li) : 0;
    const bool bok = listed && (blk >= tw.win_start || blk < tw.n_sink);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = bok && (kPage * blk + 4 * rc.g + i <= rc.t_mask);
      m |= (ok ? 1u : 0u) << (4 * p + i);
    }
  }
  return m;
}

// S^T = K . Q^T for HPW query heads and NP pages (p0 ..) of a step: each K
// fragment (16 keys x 64 channels, one ds_read_b128) feeds HPW products.
// Afterwards s[h][pp] register i of lane l holds query row l%16 and key
// 4(l/16) + i of page p0 + pp.  The fragment reads are software-pipelined D
// fragments ahead of their products; the scheduling fences keep the compiler
// from sinking them back next to their uses (it would otherwise reuse one
// register set and wait out the full LDS latency before every product).
template <int HPW, int NP, int D>
__device__ inline void qk_pages_pipelined(const int8_t* kb, const v4i (&qf)[HPW][4], int p0, int lane,
                                          v4i (&s)[HPW][NP]) {
  constexpr int NF = 4 * NP;  // fragments: f = 4 * pp + c
  const int g = lane >> 4;
  auto read = [&](int f) {
    const int r = 16 * (p0 + f / 4) + (lane & 15);
    const int slot = (4 * (f % 4) + g) ^ swz(r);
    return *reinterpret_cast<const v4i*>(kb + r * kHeadDim + 16 * slot);
  };
  v4i kf[NF];
#pragma unroll
  for (int f = 0; f < D; ++f) {
    kf[f] = read(f);
    __builtin_amdgcn_sched_barrier(0);  // issue in order: the first product waits for the first read only
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + D < NF) kf[f + D] = read(f + D);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < HPW; ++h)
      s[h][f / 4] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[f], qf[h][f % 4], f % 4 ? s[h][f / 4] : v4i{0, 0, 0, 0},
                                                          0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Register i of both planes (one accumulator row per 16 lanes) becomes
// floor((256 hi + lo) / 2^d), exactly, for 0 <= d <= kStageShift: hi keeps
// its high part and its low d bits move down into lo.  For d >= 1 the sum
// lo + 256 (hi mod 2^d) is halved first (256 (hi mod 2^d) is even, so
// floor(lo / 2) + 128 (hi mod 2^d) is the exact half, floored), which keeps
// every intermediate below 2^31 for any int32 hi and lo; then it is shifted
// by the remaining d - 1 bits.
__device__ inline void shift_planes(v4i (&acc)[2][16], int i, int d) {
  const int m = (1 << d) - 1;
  const int s1 = min(d, 1);
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) {
    const int hi = acc[1][nt][i], lo = acc[0][nt][i];
    acc[1][nt][i] = hi >> d;
    acc[0][nt][i] = (int)((uint32_t)(lo >> s1) + ((uint32_t)(hi & m) << (8 - s1))) >> (d - s1);
  }
}

// One step for HPW heads.  z = acc*k_scale*rowf + log2(v_scale) (rowf = q
// scale * softmax scale * log2 e); the row maximum of z over the step raises
// the reference zref when it passes it (the accumulators and l of a raised
// row are shifted right by the difference).  Then e = exp2(z - log2 v_scale -
// zref) = P relative to 2^zref, l += P, P' = P * v_scale <= 1, per-page codes
// code = rint(P' * 127 / max P'), their weights ps * code as the fixed-point
// integer x = rint(code * f), f = max P' * Xmax / (127 * cap), split into two
// signed int8 digit planes x = d0 + 256 d1, then PV.  Every K and V fragment
// read serves HPW heads.
//
// code * f is formed as (code * F + 2^15) >> 16 with F = rint(f * 2^16) < 2^24
// by one 24-bit multiply-add; with a bias of 128 in the upper half, bytes 2
// and 3 of the result are d0 + 128 and d1.
template <int HPW, bool MASKED>
__device__ inline void attn_step(Stage& st, const v4i (&qf)[HPW][4], int lane, int g, const float (&rowf)[HPW],
                                    uint32_t kmask, float (&zref)[HPW], float (&lsum)[HPW], v4i (&acc)[HPW][2][16]) {
  v4i s[HPW][4];
  qk_pages_pipelined<HPW, 4, 8>(st.k, qf, 0, lane, s);
  v4i dig[HPW][2];
  // log2(v_scale) of the step's 64 keys, one per lane, into the spare scale
  // slots (every wave writes the same values)
  st.sc[lane >> 4][32 + (lane & 15)] = __builtin_amdgcn_logf(fmaxf(st.sc[lane >> 4][16 + (lane & 15)], kVsFloor));
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    float sk[4][4];
    float zm = -INFINITY;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float4 ks4 = *reinterpret_cast<const float4*>(&st.sc[p][4 * g]);
      const float4 lv4 = *reinterpret_cast<const float4*>(&st.sc[p][32 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sk[p][i] = (float)s[h][p][i] * (&ks4.x)[i];
        float z = fmaf(sk[p][i], rowf[h], (&lv4.x)[i]);
        if (MASKED) z = ((kmask >> (4 * p + i)) & 1u) ? z : -INFINITY;
        zm = fmaxf(zm, z);
      }
    }
    zm = rows_max(zm);
    // a row whose maximum passes its reference raises it to a whole power of
    // two plus headroom and scales what it has accumulated by the difference
    if (__builtin_amdgcn_ballot_w64(zm > zref[h]) != 0) {
      const bool first = zref[h] == -INFINITY;  // every row starts there: the first step's event
      const float znew = zm > zref[h] ? ceilf(zm) + kRefHeadroom : zref[h];
      const float dz = first ? 0.f : znew - zref[h];  // a whole number of bits
      lsum[h] = __builtin_amdgcn_ldexpf(lsum[h], -(int)fminf(dz, 255.f));
      const int dl = (int)fminf(dz, kMaxShift);
      zref[h] = znew;
      if (!first) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int di = __shfl(dl, 4 * g + i);  // shift of accumulator row 4g + i
          if (__builtin_amdgcn_ballot_w64(di != 0) != 0) {
            const int d1 = min(di, kStageShift), d2 = di - d1;
            shift_planes(acc[h], i, d1);
            if (__builtin_amdgcn_ballot_w64(d2 != 0) != 0) shift_planes(acc[h], i, d2);
          }
        }
      }
    }
    const float negz = -zref[h];
    float pp[4][4];
    uint32_t mx[4];  // bit patterns of the page maxima of P' >= 0
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float4 vs4 = *reinterpret_cast<const float4*>(&st.sc[p][16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e = __builtin_amdgcn_exp2f(fmaf(sk[p][i], rowf[h], negz));
        float pv = e * (&vs4.x)[i];
        if (MASKED) {
          const bool ok = (kmask >> (4 * p + i)) & 1u;
          e = ok ? e : 0.f;
          pv = ok ? pv : 0.f;
        }
        lsum[h] += e;
        pp[p][i] = pv;
      }
      mx[p] = max(max(__float_as_uint(pp[p][0]), __float_as_uint(pp[p][1])),
                  max(__float_as_uint(pp[p][2]), __float_as_uint(pp[p][3])));
    }
    page_maxima(mx);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // a page whose P' all lie below 2^-60 (masked ones are 0) gets F = 0 and
      // finite codes, so its weights are exactly zero
      const float inv = 127.0f * __builtin_amdgcn_rcpf(__uint_as_float(max(mx[p], __float_as_uint(kTiny))));
      const uint32_t F = (uint32_t)fmaf(__uint_as_float(mx[p]), kFScale, 0.5f);
      uint32_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t code = __float_as_uint(fmaf(pp[p][i], inv, kTwo23));  // 2^23 + rint(P' * inv)
        r[i] = __umul24(code, F) + kDigitBias;
      }
      const uint32_t w01 = __builtin_amdgcn_perm(r[1], r[0], 0x07060302u);
      const uint32_t w23 = __builtin_amdgcn_perm(r[3], r[2], 0x07060302u);
      dig[h][0][p] = (int)(__builtin_amdgcn_perm(w23, w01, 0x06040200u) ^ 0x80808080u);  // low digit, signed
      dig[h][1][p] = (int)__builtin_amdgcn_perm(w23, w01, 0x07050301u);                 // high digit
    }
  }

  // V operand (see VFrag): reads run two column tiles ahead of their products
  // (see qk_pages_pipelined)
  constexpr int DV = 2;
  const VFrag read_v(st.v, lane);
  v4i vf[16];
#pragma unroll
  for (int nt = 0; nt < DV; ++nt) {
    vf[nt] = read_v(nt);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) {
    if (nt + DV < 16) vf[nt + DV] = read_v(nt + DV);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      acc[h][0][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dig[h][0], vf[nt], acc[h][0][nt], 0, 0, 0);
      acc[h][1][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dig[h][1], vf[nt], acc[h][1][nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Where the attention finds its Q rows: int8 codes and row scales from the
// caller, or bf16 from the caller, quantized on load.
enum class QSrc { kInt8, kBf16 };

// What a wave knows about its work item.  A workgroup is four waves over
// TPG = 4/WPG consecutive query tiles and WPG query heads of one KV head:
// wave w takes head w % WPG of tile T0 + w / WPG (16 query rows), where the
// group's first tile T0 is a multiple of TPG in the sequence's numbering.
// The group walks the union of its tiles' key lists, from T0's sinks and
// window start to the diagonal block of its last tile in the call, so all
// four waves share every staged page; a wave masks the blocks its own tile
// does not attend, which can only happen in its first and last steps.
// Because T0 does not depend on where a call starts, a tile's keys sit at the
// same list entries in a chunked call as in a whole-sequence call, and its
// result is the same bits.  The call's rows start at tile a.tile0 of the
// sequence; my_t is the lane's row within the call's Q and out.  A wave whose
// tile is outside the call repeats a tile of the call and stores nothing.
template <int WPG>
struct Work {
  static constexpr int TPG = 4 / WPG;
  int lane, wave, kvh, qt_local, head0, my_t;
  bool wave_ok, row_ok;
  RowCtx rc;
  TileBlocks tb;  // the group's key list
  TileBlocks tw;  // this wave's tile: its sinks and window start
  int n_st;       // steps of 64 keys
  int m_early, m_late;  // steps before m_early and from m_late on need key masks
  uint32_t page_bytes, scale_stride;
  DmaPlan<4> plan;
  __device__ Work(const AttnArgs& a) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int u = blockIdx.x;
    const int hg = u % a.hgroups;
    u /= a.hgroups;
    kvh = u % a.n_kv_heads;
    // tiles in the sequence's numbering; groups of the call, longest first
    const int t_end = a.tile0 + a.n_tiles - 1;
    const int t0 = (t_end / TPG - u / a.n_kv_heads) * TPG;
    const int ta = max(t0, a.tile0), tz = min(t0 + TPG - 1, t_end);  // the group's tiles in the call
    const int tt = t0 + wave / WPG;
    wave_ok = tt >= ta && tt <= tz;
    const int qt = min(max(tt, ta), tz);
    qt_local = qt - a.tile0;
    head0 = kvh * a.G + hg * WPG + wave % WPG;
    my_t = qt_local * kPage + (lane & 15);
    row_ok = wave_ok && my_t < a.n_tokens;
    rc.g = lane >> 4;
    rc.t_mask = kPage * a.tile0 + min(my_t, a.n_tokens - 1);
    tb = tile_blocks(t0, a.window_blocks, a.sink_blocks);
    tb.n_total = tb.n_sink + (tz + 1 - tb.win_start);
    tw = tile_blocks(qt, a.window_blocks, a.sink_blocks);
    n_st = (tb.n_total + 3) >> 2;
    // list entries of the window blocks before tw's window, and of tw's diagonal block
    m_early = tw.win_start > tb.win_start ? (tb.n_sink + tw.win_start - tb.win_start + 3) >> 2 : 0;
    m_late = (tb.n_sink + qt - tb.win_start) >> 2;
    page_bytes = (uint32_t)(kPage * a.n_kv_heads * kHeadDim);
    scale_stride = (uint32_t)(kPage * a.n_kv_heads);
    make_plan<4>(plan, a, kvh, wave, lane);
  }
  // Q codes of this lane's row for heads hd0 .. in the B-operand layout (16
  // channels per chunk) and rowf = q_scale * softmax_scale * log2(e); rows
  // past the end read the last token and are never stored.  From bf16 the
  // lane reads the same 64 channels and the four lanes of a row (lane, +16,
  // +32, +48) share their maximum to quantize the row.
  template <int H, QSrc QS>
  __device__ void load_q(const AttnArgs& a, int hd0, v4i (&qf)[H][4], float (&rowf)[H], float (&qscale)[H]) const {
    const int tq = row_ok ? my_t : a.n_tokens - 1;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const long row = (long)tq * a.n_q_heads + hd0 + h;
      if (QS == QSrc::kBf16) {
        const uint4* qrow = reinterpret_cast<const uint4*>(a.q_bf16 + row * kHeadDim + 16 * rc.g);
        uint4 raw[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          raw[c][0] = qrow[8 * c];
          raw[c][1] = qrow[8 * c + 1];
        }
        // |x| of finite values ordered as the unsigned magnitude bits; the
        // packed words stay in registers and are widened only once, below
        uint32_t mlo = 0, mhi = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t w[4] = {raw[c][k].x, raw[c][k].y, raw[c][k].z, raw[c][k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              mlo = max(mlo, w[i] & 0x7fffu);
              mhi = max(mhi, w[i] & 0x7fff0000u);
            }
          }
        uint32_t mbits = max(mlo << 16, mhi);
        mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 16));
        mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 32));
        const float amax = __uint_as_float(mbits);
        const float inv = q_inv_of(amax);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t cw[4];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t w[4] = {raw[c][k].x, raw[c][k].y, raw[c][k].z, raw[c][k].w};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t lo = w[2 * i], hi = w[2 * i + 1];
              cw[2 * k + i] = q_code4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                                      __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u), inv);
            }
          }
          qf[h][c] = v4i{(int)cw[0], (int)cw[1], (int)cw[2], (int)cw[3]};
        }
        qscale[h] = q_scale_of(amax);
        rowf[h] = row_ok ? qscale[h] * a.row_mul : 0.f;
        // one head's bf16 row in registers at a time
        asm volatile("" ::: "memory");
      } else {
        const int8_t* qrow = a.q_i8 + row * kHeadDim + 16 * rc.g;
#pragma unroll
        for (int c = 0; c < 4; ++c) qf[h][c] = *reinterpret_cast<const v4i*>(qrow + 64 * c);
        qscale[h] = a.q_scale[row];
        rowf[h] = row_ok ? qscale[h] * a.row_mul : 0.f;
      }
    }
  }
};

// The attention: the group's key list walked four pages at a time with K and
// V staged, the running reference, P codes, digit planes and PV, then the
// epilogue.  One head per wave (HPW = 1): a wave holding two heads'
// accumulators runs alone on its SIMD and measured slower than two waves per
// SIMD.
template <int WPG, bool OUT_BF16, bool QF>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(AttnArgs a, const int32_t* __restrict__ pt_arg) {
  constexpr int HPW = 1;
  __shared__ Stage st[2];
  const WPA_CONST int32_t* pt = (const WPA_CONST int32_t*)pt_arg;
  Work<WPG> w(a);
  issue_stage<4, true>(st[0], a, w.plan, w.page_bytes, w.scale_stride, wave_pages<4>(pt, w.tb, 0, w.wave), w.wave);
  v4i qf[HPW][4];
  float rowf[HPW], zref[HPW], lsum[HPW];
  float qscale[HPW];
  w.template load_q<HPW, QF ? QSrc::kBf16 : QSrc::kInt8>(a, w.head0, qf, rowf, qscale);
  // rows past the end read the last token with rowf = 0; their results stay
  // in their own accumulator rows and are never stored
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    zref[h] = -INFINITY;  // raised by the first step
    lsum[h] = 0.f;
  }
  wait_vmem();
  // page ids two steps ahead: a scalar load still in flight holds up the
  // step's first LDS wait (both count on lgkmcnt), so it must be issued early
  // enough to have returned; entries past the list clamp to its last page
  WavePages<4> pg1 = wave_pages<4>(pt, w.tb, 1, w.wave), pg2 = wave_pages<4>(pt, w.tb, 2, w.wave);

  v4i acc[HPW][2][16];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) acc[h][pl][nt] = v4i{0, 0, 0, 0};
  int buf = 0;
  // every wave runs n_st steps with one barrier each; only which steps are
  // masked differs between the waves
  auto next_stage = [&](int it) {
    wait_stage();
    __syncthreads();
    if (it + 1 < w.n_st) issue_stage<4, true>(st[buf ^ 1], a, w.plan, w.page_bytes, w.scale_stride, pg1, w.wave);
    pg1 = pg2;
    pg2 = wave_pages<4>(pt, w.tb, it + 3, w.wave);
  };
  int it = 0;
  for (; it < min(w.m_early, w.n_st); ++it) {
    next_stage(it);
    attn_step<HPW, true>(st[buf], qf, w.lane, w.rc.g, rowf, key_mask(w.tb, w.tw, it, w.rc), zref, lsum, acc);
    buf ^= 1;
  }
  for (; it < w.m_late; ++it) {
    next_stage(it);
    attn_step<HPW, false>(st[buf], qf, w.lane, w.rc.g, rowf, 0u, zref, lsum, acc);
    buf ^= 1;
  }
  for (; it < w.n_st; ++it) {
    next_stage(it);
    attn_step<HPW, true>(st[buf], qf, w.lane, w.rc.g, rowf, key_mask(w.tb, w.tw, it, w.rc), zref, lsum, acc);
    buf ^= 1;
  }

  // ---- epilogue: recombine the digit planes, scale by cap / (Xmax * l), store.
  // Output register i of tile nt is row 4g + i, channel 16nt + lane%16.
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float rscale = kCap / (kXmax * rows_sum(lsum[h]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * w.rc.g + i;
      const float rr = __shfl(rscale, r);
      const int t = w.qt_local * kPage + r;
      if (!w.wave_ok || t >= a.n_tokens) continue;
      const long base = ((long)t * a.n_q_heads + w.head0 + h) * kHeadDim + (w.lane & 15);
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) {
        const float x = fmaf((float)acc[h][1][nt][i], 256.f, (float)acc[h][0][nt][i]);
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
}

template <int WPG, bool OUT_BF16, bool QF>
static void launch_wpg(const AttnArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_attn_kernel<WPG, OUT_BF16, QF>), dim3(grid), dim3(256), 0, stream, a, a.page_table);
}
template <int WPG>
static void launch_wpg(const AttnArgs& a, bool out_bf16, unsigned grid, hipStream_t stream) {
  const bool qf = a.q_bf16 != nullptr;
  if (out_bf16) {
    if (qf) launch_wpg<WPG, true, true>(a, grid, stream);
    else launch_wpg<WPG, true, false>(a, grid, stream);
  } else {
    if (qf) launch_wpg<WPG, false, true>(a, grid, stream);
    else launch_wpg<WPG, false, false>(a, grid, stream);
  }
}

hipError_t launch_prefill_attn(const AttnArgs& args_in, bool out_bf16, hipStream_t stream) {
  AttnArgs a = args_in;
  a.G = a.n_q_heads / a.n_kv_heads;
  a.n_tiles = (a.n_tokens + kPage - 1) / kPage;
  a.tile0 = a.q_start / kPage;
  a.row_mul = a.softmax_scale * kLog2e;
  // groups of tiles counted from the sequence's first tile, so that a
  // chunk's tiles fall in the same groups as in a whole-sequence call
  const PrefillGrid pg = prefill_grid(a.n_q_heads, a.n_kv_heads, a.tile0, a.n_tiles);
  a.hgroups = pg.hgroups;
  const unsigned grid = (unsigned)pg.workgroups;
  if (pg.wpg == 4) launch_wpg<4>(a, out_bf16, grid, stream);
  else if (pg.wpg == 2) launch_wpg<2>(a, out_bf16, grid, stream);
  else launch_wpg<1>(a, out_bf16, grid, stream);
  return hipGetLastError();
}

}  // namespace wpa
