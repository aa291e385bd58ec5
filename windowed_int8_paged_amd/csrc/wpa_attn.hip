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
//   * One launch.  A workgroup = eight waves on one KV head: 4 of its query
//     heads on two consecutive 16-token query tiles, or, with 2 (1) query
//     heads per workgroup, 2 heads on 4 tiles (1 head on 8 tiles), walking
//     the union of their key lists, so every staged K/V page feeds eight
//     waves whatever the GQA ratio.  A wave takes one head of one tile (16
//     query rows) and needs at most 256 registers, so two waves share each
//     SIMD and one workgroup fills a CU.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_i32_16x16x64_i8.  The 16 keys of each product are taken four
//     from each page of the step, so that afterwards a lane holds one query
//     row and all 16 keys of one page: a page's maximum is an in-lane
//     reduction, and the lane's 16 P codes are exactly the A operand of the
//     PV product (page g of the step in its K-slice 16g .. 16g+15).
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
//   * K and V pages go global -> LDS by asynchronous LDS DMA into row-major
//     XOR-swizzled tiles, in a ring of four stages filled two steps ahead,
//     with one workgroup barrier every second step.  Each wave issues five
//     copies per step (one page of K or of V and its scales), spread among
//     its PV products, so a page is fetched once for all eight waves.  LDS fragment reads are software-pipelined ahead of
//     their matrix products; V operands are gathered with the transposing
//     read ds_read_b64_tr_b8.  The unmasked steps run with their ring stage
//     known, so every LDS read is a register holding the lane's address plus
//     an immediate: no address arithmetic in the step.
//   * From bf16 Q (the fused entry point) each wave quantizes its own rows as
//     it loads them, by the same formula as the separate quantize kernel.

#include "wpa_common.h"
#include "wpa_lanes.h"
#include "wpa_launch.h"

namespace wpa {

constexpr int kStepKeys = 64;                 // keys per step (four pages)
constexpr int kStage = kStepKeys * kHeadDim;  // bytes of one staged K or V tile
constexpr int kWaves = 8;                     // waves per workgroup
constexpr int kStages = 4;                    // LDS ring depth
constexpr int kLead = 2;                      // a step's copies are issued this many steps before it runs
constexpr int kCopies = 5;                    // copies per wave and step (4 x 1 KB rows + 1 scale row)
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
// 8 bits (floor divisions compose).  With |256 hi + lo| < 2^40, kMaxShift bits
// take any value to 0 or -1, which is what any larger floor shift gives.
constexpr float kRefHeadroom = 1.f;
constexpr float kMaxShift = 40.f;
// log2(v_scale) enters the reference as log2(max(v_scale, kVsFloor)): a zero
// v_scale (the KV writer's scale of an all-zero V row) still sets a finite
// reference, and every e = exp2(score * log2(e) - zref) stays below 2^63
// (P' = e * v_scale is unchanged).
constexpr float kVsFloor = 0x1p-64f;

// The LDS ring.  Stage s holds the step's four pages of K and of V (row
// 16p + r is key r of page p) and their scales: ks[p][r] and vs[p][r] for
// slot r < 16 (each 256-byte copy repeats the page's 16 scales four times),
// with vs[p][16 + r] then overwritten by log2(v_scale).  The K tiles of the
// four stages fill the first 64 KB, their V tiles the next 64 KB and the
// scale rows follow, so a stage's place inside a region fits the 16-bit
// immediate offset of an LDS read: with the lane's part of every operand
// address held in a register, a step with a known stage reads LDS with no
// address arithmetic.  The scale rows are 272 bytes apart, so that the four
// lane groups reading the same slots of their four pages hit four different
// sets of banks.
constexpr int kScaleRow = 68;                                    // floats per scale row: 64 copied + 4 of padding
constexpr uint32_t kRegionV = kStages * kStage;                  // V tiles
constexpr uint32_t kRegionSc = 2 * kStages * kStage;             // scale rows
constexpr uint32_t kScRows = 4 * kScaleRow * sizeof(float);      // the four k (or v) scale rows of a stage
constexpr uint32_t kScStage = 2 * kScRows;                       // k rows, then v rows
constexpr uint32_t kLdsBytes = kRegionSc + kStages * kScStage;
static_assert(kStages * kStage <= 65536, "a stage offset inside a region fits an LDS immediate");

// LDS swizzle of the staged tiles: the 16-byte chunk c of row r sits in slot
// c ^ swz_pg(r).  The score operand reads (rows 16q + 4t + i, q, i = 0..3, for
// one t) and the transposing V reads (rows 16q + 8h + 0..7 of two adjacent
// pages q) then touch every bank once per read.  Bit 3 of r does not enter,
// so the two halves of a V operand (slots k and 8 + k of a page) share one
// swizzle and one address computation.
__device__ inline int swz_pg(int r) {
  return (r & 3) | ((((r >> 2) ^ (r >> 5)) & 1) << 2) | (((r >> 4) & 1) << 3);
}

// Asynchronous global->LDS copy of 16 (or 4) bytes per lane through a buffer
// resource: lane l reads at its byte offset inside the resource and its
// bytes land at lds_base + 16*l (4*l).  The resource covers one page (or one
// page's scales), and an offset past its size reads zeros instead of memory
// outside it.  Issued as inline assembly so the compiler does not model the
// in-flight LDS write; the kernel orders it explicitly with its vmcnt waits
// and a workgroup barrier before any read of that buffer.  m0 carries the LDS
// address and is set right before each copy; the compiler warns about
// clobbering a reserved register, but on gfx950 nothing it emits in these
// kernels reads m0 (every m0 in their assembly belongs to a copy).  The
// buffer form measured 0.6% faster than the global form with the same bits.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const WPA_LDS void*)p;
}
typedef int sv4 __attribute__((ext_vector_type(4)));
// Raw buffer resource over `bytes` bytes from `base` (no stride, 32-bit
// data format as gfx9 raw loads take it).
__device__ inline sv4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return sv4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)bytes, 0x00020000};
}
__device__ inline void dma16(uint32_t voff, sv4 rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}
__device__ inline void dma4(uint32_t voff, sv4 rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}
// Waits until at most N of the wave's vector memory operations are in
// flight, through the builtin so the compiler's own wait tracking sees it
// (registers filled by earlier vector loads then count as ready).  The
// immediate holds vmcnt in bits 3:0 (N < 16 here), with expcnt and lgkmcnt
// left at their maxima.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  asm volatile("" ::: "memory");
}

// The copies of one wave: wave w takes page w % 4 of each step, K for waves
// 0-3 and V for waves 4-7, as four 1 KB row groups (keys 4j .. 4j+3, one
// 16-byte chunk per lane) and one 256-byte copy of the page's 16 scales.
// The per-lane parts of the addresses are constants kept in registers, so a
// copy costs one scalar base per page and no vector arithmetic.
struct DmaPlan {
  uint32_t voff[4];     // byte offset inside a page, swizzle applied
  uint32_t lds_rows;    // LDS offset of the wave's page rows in stage 0
  uint32_t lds_sc;      // LDS offset of the wave's page scales in stage 0
  const int8_t* pool;   // k_pool or v_pool
  const float* scales;  // k_scale or v_scale
  uint32_t soff;        // lane l: byte offset of the scale of slot l % 16 inside a page's scales
  int page;             // page of the step this wave copies (0..3)
};
__device__ inline void make_plan(DmaPlan& pl, const AttnArgs& a, int kvh, int wave, int lane) {
  const int q = lane >> 4, s = lane & 15;
  const int p = wave & 3;
  const bool is_v = wave >= 4;
  const int row_bytes = a.n_kv_heads * kHeadDim;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = 4 * j + q;  // key inside the page
    pl.voff[j] = (uint32_t)(rr * row_bytes + kvh * kHeadDim + 16 * (s ^ swz_pg(16 * p + rr)));
  }
  pl.lds_rows = (is_v ? kRegionV : 0u) + (uint32_t)(16 * p * kHeadDim);
  pl.lds_sc = kRegionSc + (is_v ? kScRows : 0u) + (uint32_t)(kScaleRow * sizeof(float) * p);
  pl.pool = is_v ? a.v_pool : a.k_pool;
  pl.scales = is_v ? a.v_scale : a.k_scale;
  pl.soff = (uint32_t)((s * a.n_kv_heads + kvh) * sizeof(float));
  pl.page = p;
}
// The copies a wave owes for a later step into the stage at LDS address
// `stage`.  Inside the loop they are issued one at a time among the current
// step's PV products rather than in a burst after the barrier: a burst of
// LDS copies from every wave at once holds up the waves' own operand reads.
// A page id outside the pool is clamped into it: a wrong page, never memory
// outside the pool.
struct CopyJob {
  bool on;              // wave-uniform: is there a step to copy for
  sv4 rows;             // the page's rows in the pool
  sv4 sc;               // the page's scales
  uint32_t lds_rows;    // LDS destinations
  uint32_t lds_sc;
};
__device__ inline CopyJob make_job(bool on, uint32_t ring, int stage, const AttnArgs& a, const DmaPlan& pl,
                                   uint32_t page_bytes, uint32_t scale_stride, int page_id) {
  const uint32_t page = (uint32_t)min(max(page_id, 0), a.n_pool_pages - 1);
  CopyJob c;
  c.on = on;
  c.rows = buffer_rsrc(pl.pool + (uint64_t)page * page_bytes, page_bytes);
  c.sc = buffer_rsrc(pl.scales + (uint64_t)page * scale_stride, scale_stride * (uint32_t)sizeof(float));
  c.lds_rows = ring + pl.lds_rows + (uint32_t)stage * kStage;
  c.lds_sc = ring + pl.lds_sc + (uint32_t)stage * kScStage;
  return c;
}
__device__ inline void copy_part(const CopyJob& c, const DmaPlan& pl, int j) {
  if (j < 4) dma16(pl.voff[j], c.rows, c.lds_rows + kKeysPerGroup * kHeadDim * j);
  else dma4(pl.soff, c.sc, c.lds_sc);
}

// Physical page of list entry 4*step + p, read through the scalar cache;
// entries past the end clamp to the last one (their keys are masked).
__device__ inline int step_page(const WPA_CONST int32_t* pt, const TileBlocks& tb, int step, int p) {
  return pt[tb.block(min(4 * step + p, tb.n_total - 1))];
}

// Per-lane constants of one wave.
struct RowCtx {
  int g;       // 16-lane row of the wave (0..3); after the scores, also the page it holds
  int t_mask;  // causal bound of this lane's query row
};

// Attended keys among the lane's 16 scores of step `step` (page g of the
// step, slot 4t + i in bit 4t + i) of the group's key list tb, for a wave
// whose own tile is tw: the block counts if it is one of tw's sinks or lies
// in tw's window, and a key if it is not after the lane's row.  Only a wave's
// first and last steps need it.
__device__ inline uint32_t key_mask(const TileBlocks& tb, const TileBlocks& tw, int step, const RowCtx& rc) {
  const int li = 4 * step + rc.g;
  if (li >= tb.n_total) return 0u;
  const int blk = tb.block(li);
  if (blk < tw.win_start && blk >= tw.n_sink) return 0u;
  const int lim = rc.t_mask - kPage * blk;  // last attended slot
  return lim >= 15 ? 0xffffu : (lim < 0 ? 0u : (2u << lim) - 1u);
}

// S^T = K . Q^T for the 64 keys of a step.  Product t takes, as its 16 keys
// m = 0..15, slot 4t + m%4 of page m/4, so that afterwards register i of
// s[t] in lane l holds query row l%16 and slot 4t + i of page l/16.  Each K
// fragment (16 keys x 64 channels) is one ds_read_b128.  The fragment reads
// are software-pipelined D fragments ahead of their products; the scheduling
// fences keep the compiler from sinking them back next to their uses (it
// would otherwise reuse one register set and wait out the full LDS latency
// before every product).
// The lane's part of every LDS address a step reads, for stage 0; stage s
// adds s * kStage (tiles) or s * kScStage (scales), an immediate when s is
// known.  The values pass through an empty asm so that the compiler keeps
// them as they are rather than splitting them into a shared base and per-use
// offsets again.
struct LdsAddr {
  uint32_t k[8];   // K fragment of product t, chunk c at k[4 (t % 2) + c], + 2048 for t >= 2
  uint32_t v[16];  // V operand of column tile nt (keys of the first half; the second is 2048 on)
  uint32_t ks, vs;   // the lane's page row of k and v scales
  uint32_t lw, lr;   // log2(v_scale) slot this lane writes, and the v_scale it reads for it
};
__device__ inline void make_addr(LdsAddr& A, uint32_t ring, int lane) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = 16 * (m >> 2) + 4 * t + (m & 3);  // r + 8 (products 2, 3) has the same swizzle
      A.k[4 * t + c] = ring + (uint32_t)(r * kHeadDim + 16 * ((4 * c + g) ^ swz_pg(r)));
    }
  const int key1 = 16 * g + (m >> 1);  // key1 + 8 has the same swizzle
#pragma unroll
  for (int nt = 0; nt < 16; ++nt)
    A.v[nt] = ring + kRegionV + (uint32_t)(key1 * kHeadDim + 8 * (m & 1) + 16 * (nt ^ swz_pg(key1)));
  A.ks = ring + kRegionSc + (uint32_t)(g * kScaleRow * 4);
  A.vs = A.ks + kScRows;
  A.lr = ring + kRegionSc + kScRows + (uint32_t)(g * kScaleRow * 4 + 4 * m);
  A.lw = A.lr + 16 * 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(A.k[i]));
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(A.v[i]));
  asm volatile("" : "+v"(A.ks), "+v"(A.vs), "+v"(A.lw), "+v"(A.lr));
}
typedef float v4f __attribute__((ext_vector_type(4)));  // 16-byte aligned, unlike float4
template <typename T>
__device__ inline T lds_read(uint32_t addr) {
  return *reinterpret_cast<const WPA_LDS T*>((uintptr_t)addr);
}

template <int D>
__device__ inline void qk_step(const LdsAddr& A, int st, const v4i (&qf)[4], v4i (&s)[4]) {
  auto read = [&](int f) {  // fragment f = 4t + c: product t, channel chunk c
    const int t = f >> 2, c = f & 3;
    return lds_read<v4i>(A.k[4 * (t & 1) + c] + (uint32_t)(2048 * (t >> 1) + st * kStage));
  };
  v4i kf[16];
#pragma unroll
  for (int f = 0; f < D; ++f) {
    kf[f] = read(f);
    __builtin_amdgcn_sched_barrier(0);  // issue in order: the first product waits for the first read only
  }
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    if (f + D < 16) kf[f + D] = read(f + D);
    __builtin_amdgcn_sched_barrier(0);
    s[f >> 2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[f], qf[f & 3], (f & 3) ? s[f >> 2] : v4i{0, 0, 0, 0}, 0,
                                                     0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// B operand of a PV product over one staged 64-key V tile: lane (column j,
// row group g) gets channel 16 nt + j of the 16 keys of page g in slot order,
// which is the order of the lane's P operand.  Within a 16-lane group, the
// transposing read gives lane j byte j%8 of the 8-byte blocks addressed by
// lanes 2k + j/8 (k = 0..7); lane L here addresses slot L/2 of page g (slot
// 8 + L/2 in the second read) at channel 16 nt + 8 (L%2).
__device__ inline v4i read_v(const LdsAddr& A, int st, int nt) {
  const uint32_t p = A.v[nt] + (uint32_t)(st * kStage);
  const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<WPA_LDS v2i*>((uintptr_t)p));
  const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<WPA_LDS v2i*>((uintptr_t)(p + 8 * kHeadDim)));
  return v4i{lo.x, lo.y, hi.x, hi.y};
}

// Register i of both planes (one accumulator row per 16 lanes) becomes
// floor((256 hi + lo) / 2^d), exactly, for 0 <= d <= 8: hi keeps its high
// part and its low d bits move down into lo.  256 (hi mod 2^d) / 2^d is a
// whole number, so floor((lo + 256 (hi mod 2^d)) / 2^d) = (lo >> d) + (hi mod
// 2^d) 2^(8-d), and that sum stays in int32 for any int32 hi and lo.
__device__ inline void shift_planes(v4i (&acc)[2][16], int i, int d) {
  const int m = (1 << d) - 1;
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) {
    const int hi = acc[1][nt][i], lo = acc[0][nt][i];
    acc[1][nt][i] = hi >> d;
    acc[0][nt][i] = (int)((uint32_t)(lo >> d) + ((uint32_t)(hi & m) << (8 - d)));
  }
}

// Range guard of the int32 planes, for rows of any length.  A key adds at
// most 128 * 127 to a plane element, so kGuardSteps steps of 64 keys (plus the
// few masked steps around them) add less than 2^26.  Every kGuardSteps steps,
// a row holding a plane element of magnitude 2^30 or more has its reference
// raised by one bit: its planes are shifted right by one (exactly, as for any
// raise) and l is halved, so every element stays below 2^31 whatever the
// row's length.  Accumulator register i of lane (column c, group g) is row
// 4g + i; the softmax state of row r sits in lanes r, r + 16, r + 32, r + 48.
constexpr int kGuardSteps = 64;
// The fixed cost of a workgroup (Q load, epilogue) in key steps, for
// balancing the runs of tile groups across XCDs.
constexpr long kGroupCost = 2;
__device__ inline void guard_planes(v4i (&acc)[2][16], int lane, float& zref, float& lsum) {
  uint64_t big[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int hi = INT32_MIN, lo = INT32_MAX;
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        hi = max(hi, acc[pl][nt][i]);
        lo = min(lo, acc[pl][nt][i]);
      }
    big[i] = __builtin_amdgcn_ballot_w64(hi >= (1 << 30) || lo <= -(1 << 30));
  }
  if ((big[0] | big[1] | big[2] | big[3]) == 0) return;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) shift_planes(acc, i, ((big[i] >> (16 * g)) & 0xffffu) ? 1 : 0);
  const uint64_t mine = big[r & 3] >> (16 * (r >> 2));  // this lane's softmax row r = 4 (r/4) + r%4
  if (mine & 0xffffu) {
    zref += 1.f;
    lsum *= 0.5f;
  }
}

// One step of one wave.  z = acc*k_scale*rowf + log2(v_scale) (rowf = q
// scale * softmax scale * log2 e); the row maximum of z over the step raises
// the reference zref when it passes it (the accumulators and l of a raised
// row are shifted right by the difference).  Then e = exp2(z - log2 v_scale -
// zref) = P relative to 2^zref, l += P, P' = P * v_scale <= 1, per-page codes
// code = rint(P' * 127 / max P'), their weights ps * code as the fixed-point
// integer x = rint(code * f), f = max P' * Xmax / (127 * cap), split into two
// signed int8 digit planes x = d0 + 256 d1, then PV.
//
// code * f is formed as (code * F + 2^15) >> 16 with F = rint(f * 2^16) < 2^24
// by one 24-bit multiply-add; with a bias of 128 in the upper half, bytes 2
// and 3 of the result are d0 + 128 and d1.
template <bool MASKED>
__device__ __attribute__((always_inline)) inline void attn_step(const LdsAddr& A, int st, const v4i (&qf)[4], int lane, int g, float rowf, uint32_t kmask,
                                 float& zref, float& lsum, v4i (&acc)[2][16], const CopyJob& job,
                                 const DmaPlan& plan) {
  v4i s[4];
  qk_step<8>(A, st, qf, s);
  // The weights run at a raised wave priority, the products at the normal
  // one: where the two waves of a SIMD are in different phases, the arbiter
  // issues the vector work first.  Measured 0.5-1% faster at 32k, 64k and
  // 16k full causal and about 4% at 4k, with the same bits.
  __builtin_amdgcn_s_setprio(1);
  const uint32_t sc = (uint32_t)(st * kScStage);
  // log2(v_scale) of the step's 64 keys, one per lane, into the spare scale
  // slots (every wave writes the same values)
  *reinterpret_cast<WPA_LDS float*>((uintptr_t)(A.lw + sc)) =
      __builtin_amdgcn_logf(fmaxf(lds_read<float>(A.lr + sc), kVsFloor));
  __builtin_amdgcn_wave_barrier();
  float sk[4][4];
  float zm = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v4f ks4 = lds_read<v4f>(A.ks + sc + 16 * t);
    const v4f lv4 = lds_read<v4f>(A.vs + sc + 64 + 16 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sk[t][i] = (float)s[t][i] * ks4[i];
      float z = fmaf(sk[t][i], rowf, lv4[i]);
      if (MASKED) z = ((kmask >> (4 * t + i)) & 1u) ? z : -INFINITY;
      zm = fmaxf(zm, z);
    }
  }
  zm = rows_max(zm);
  // a row whose maximum passes its reference raises it to a whole power of
  // two plus headroom and scales what it has accumulated by the difference
  if (__builtin_amdgcn_ballot_w64(zm > zref) != 0) {
    const bool first = zref == -INFINITY;  // every row starts there: the first step's event
    const float znew = zm > zref ? ceilf(zm) + kRefHeadroom : zref;
    const float dz = first ? 0.f : znew - zref;  // a whole number of bits
    lsum = __builtin_amdgcn_ldexpf(lsum, -(int)fminf(dz, 255.f));
    const int dl = (int)fminf(dz, kMaxShift);
    zref = znew;
    if (!first) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int di = __shfl(dl, 4 * g + i);  // shift of accumulator row 4g + i
        if (__builtin_amdgcn_ballot_w64(di != 0) != 0) {
          int rem = di;  // in stages of at most 8 bits
          do {
            const int dd = min(rem, 8);
            shift_planes(acc, i, dd);
            rem -= dd;
          } while (__builtin_amdgcn_ballot_w64(rem != 0) != 0);
        }
      }
    }
  }
  const float negz = -zref;
  float pp[4][4];
  uint32_t mx = 0;  // bit pattern of the page maximum of P' >= 0
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v4f vs4 = lds_read<v4f>(A.vs + sc + 16 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e = __builtin_amdgcn_exp2f(fmaf(sk[t][i], rowf, negz));
      float pv = e * vs4[i];
      if (MASKED) {
        const bool ok = (kmask >> (4 * t + i)) & 1u;
        e = ok ? e : 0.f;
        pv = ok ? pv : 0.f;
      }
      lsum += e;
      pp[t][i] = pv;
    }
    mx = max(mx, max(max(__float_as_uint(pp[t][0]), __float_as_uint(pp[t][1])),
                     max(__float_as_uint(pp[t][2]), __float_as_uint(pp[t][3]))));
  }
  // inv = 127 / max P' by IEEE division, the method's float32 step.  A page
  // whose P' all lie below 2^-60 (masked ones are 0) gets F = 0 and finite
  // codes, so its weights are exactly zero.  F is clamped to 24 bits: P' <= cap
  // holds only up to the rounding of z, which can pass the cap's margin when
  // |z| is huge (scores of order 2^13 bits), and a wrapped F would drop the
  // page's largest weights.
  const float inv = 127.0f / __uint_as_float(max(mx, __float_as_uint(kTiny)));
  const uint32_t F = min((uint32_t)fmaf(__uint_as_float(mx), kFScale, 0.5f), 0xFFFFFFu);
  v4i dig[2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t code = __float_as_uint(fmaf(pp[t][i], inv, kTwo23));  // 2^23 + rint(P' * inv)
      r[i] = __umul24(code, F) + kDigitBias;
    }
    const uint32_t w01 = __builtin_amdgcn_perm(r[1], r[0], 0x07060302u);
    const uint32_t w23 = __builtin_amdgcn_perm(r[3], r[2], 0x07060302u);
    dig[0][t] = (int)(__builtin_amdgcn_perm(w23, w01, 0x06040200u) ^ 0x80808080u);  // low digit, signed
    dig[1][t] = (int)__builtin_amdgcn_perm(w23, w01, 0x07050301u);                 // high digit
  }

  __builtin_amdgcn_s_setprio(0);
  // V operand (see read_v): reads run two column tiles ahead of their
  // products (see qk_step)
  constexpr int DV = 2;
  v4i vf[16];
#pragma unroll
  for (int nt = 0; nt < DV; ++nt) {
    vf[nt] = read_v(A, st, nt);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) {
    if (nt + DV < 16) vf[nt + DV] = read_v(A, st, nt + DV);
    __builtin_amdgcn_sched_barrier(0);
    acc[0][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dig[0], vf[nt], acc[0][nt], 0, 0, 0);
    acc[1][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dig[1], vf[nt], acc[1][nt], 0, 0, 0);
    if (nt % 3 == 2 && job.on) copy_part(job, plan, nt / 3);  // nt = 2, 5, 8, 11, 14: the five copies
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Where the attention finds its Q rows: int8 codes and row scales from the
// caller, or bf16 from the caller, quantized on load.
enum class QSrc { kInt8, kBf16 };

// What a wave knows about its work item.  A workgroup is eight waves over
// TPG = 8/WPG consecutive query tiles and WPG query heads of one KV head:
// wave w takes head w % WPG of tile T0 + w / WPG (16 query rows), where the
// group's first tile T0 is a multiple of TPG in the sequence's numbering.
// The group walks the union of its tiles' key lists, from T0's sinks and
// window start to the diagonal block of its last tile in the call, so all
// eight waves share every staged page; a wave masks the blocks its own tile
// does not attend, which can only happen in its first and last steps.
// Because T0 does not depend on where a call starts, a tile's keys sit at the
// same list entries in a chunked call as in a whole-sequence call, and its
// result is the same bits.  The call's rows start at tile a.tile0 of the
// sequence; my_t is the lane's row within the call's Q and out.  A wave whose
// tile is outside the call repeats a tile of the call and stores nothing.
template <int WPG>
struct Work {
  static constexpr int TPG = kWaves / WPG;
  int lane, wave, kvh, qt_local, head0, my_t;
  bool valid;  // false for the few padding workgroups past the last group
  bool wave_ok, row_ok;
  RowCtx rc;
  TileBlocks tb;  // the group's key list
  TileBlocks tw;  // this wave's tile: its sinks and window start
  int n_st;       // steps of 64 keys
  int m_early, m_late;  // steps before m_early and from m_late on need key masks
  uint32_t page_bytes, scale_stride;
  DmaPlan plan;
  __device__ Work(const AttnArgs& a) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    long stream, group;
    prefill_item(blockIdx.x, a.streams, a.xcd_r, a.xcd_q, a.runs, a.run_start, stream, group);
    valid = group < a.n_groups;
    const int hg = (int)stream % a.hgroups;
    kvh = (int)stream / a.hgroups;
    // tiles in the sequence's numbering; groups of the call, longest first
    const int t_end = a.tile0 + a.n_tiles - 1;
    const int t0 = (t_end / TPG - (int)min(group, (long)a.n_groups - 1)) * TPG;
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
    make_plan(plan, a, kvh, wave, lane);
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
        const v4i* qrow = reinterpret_cast<const v4i*>(a.q_bf16 + row * kHeadDim + 16 * rc.g);
        v4i raw[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          raw[c][0] = __builtin_nontemporal_load(qrow + 8 * c);  // read once: keep it out of L2's way
          raw[c][1] = __builtin_nontemporal_load(qrow + 8 * c + 1);
        }
        // |x| of finite values ordered as the unsigned magnitude bits; the
        // packed words stay in registers and are widened only once, below
        uint32_t mlo = 0, mhi = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t w[4] = {(uint32_t)raw[c][k][0], (uint32_t)raw[c][k][1], (uint32_t)raw[c][k][2],
                                   (uint32_t)raw[c][k][3]};
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
            const uint32_t w[4] = {(uint32_t)raw[c][k][0], (uint32_t)raw[c][k][1], (uint32_t)raw[c][k][2],
                                   (uint32_t)raw[c][k][3]};
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
        for (int c = 0; c < 4; ++c) qf[h][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(qrow + 64 * c));
        qscale[h] = a.q_scale[row];
        rowf[h] = row_ok ? qscale[h] * a.row_mul : 0.f;
      }
    }
  }
};

// The attention: the group's key list walked four pages at a time through
// the LDS ring, the running reference, P codes, digit planes and PV, then the
// epilogue.  One head per wave: a wave holding two heads' accumulators would
// run alone on its SIMD.
template <int WPG, bool OUT_BF16, bool QF>
__global__ __launch_bounds__(512, 1) void prefill_attn_kernel(AttnArgs a, const int32_t* __restrict__ pt_arg) {
  constexpr int HPW = 1;
  __shared__ alignas(16) int8_t lds[kLdsBytes];
  const WPA_CONST int32_t* pt = (const WPA_CONST int32_t*)pt_arg;
  Work<WPG> w(a);
  if (!w.valid) return;  // uniform over the workgroup, before any copy or barrier
  const uint32_t ring = lds_addr(&lds[0]);
  // the first kLead steps' copies, then Q; the wait for Q also covers them
#pragma unroll
  for (int i = 0; i < kLead; ++i) {
    const CopyJob c = make_job(i < w.n_st, ring, i, a, w.plan, w.page_bytes, w.scale_stride,
                               step_page(pt, w.tb, i, w.plan.page));
    if (c.on)
#pragma unroll
      for (int j = 0; j < kCopies; ++j) copy_part(c, w.plan, j);
  }
  v4i qf[HPW][4];
  float rowf[HPW], qscale[HPW];
  w.template load_q<HPW, QF ? QSrc::kBf16 : QSrc::kInt8>(a, w.head0, qf, rowf, qscale);
  // rows past the end read the last token with rowf = 0; their results stay
  // in their own accumulator rows and are never stored
  float zref = -INFINITY;  // raised by the first step
  float lsum = 0.f;
  wait_vm<0>();
  // page ids two steps before their copies are issued: a scalar load still
  // in flight holds up the step's first LDS wait (both count on lgkmcnt), so
  // it must be issued early enough to have returned
  int pg1 = step_page(pt, w.tb, kLead, w.plan.page), pg2 = step_page(pt, w.tb, kLead + 1, w.plan.page);

  LdsAddr A;
  make_addr(A, ring, w.lane);
  v4i acc[2][16];
#pragma unroll
  for (int pl = 0; pl < 2; ++pl)
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) acc[pl][nt] = v4i{0, 0, 0, 0};
  // every wave runs the same n_st steps; only which steps are masked differs
  // between the waves.  A barrier comes before every even step: there each
  // wave waits for all its copies in flight (those of this step and the
  // next, issued in the two steps before), and the barrier makes every
  // wave's copies visible for both steps.  It also means every wave has
  // finished the two steps before, so their stages are free: the copies a
  // step issues (kLead = 2 steps ahead) go into the stage read two steps
  // earlier, and a ring of four stages holds the two steps being read and
  // the two being filled.
  static_assert(kLead == 2 && kStages == 4, "a barrier every second step");
  CopyJob job;
  // `sj` = (it + kLead) % kStages, the stage that takes the copies issued in
  // step it; `even`: it is even, the step starts with a barrier
  auto next_stage = [&](int it, int sj, bool even) __attribute__((always_inline)) {
    if (even) {
      wait_vm<0>();
      __syncthreads();
    }
    job = make_job(it + kLead < w.n_st, ring, sj, a, w.plan, w.page_bytes, w.scale_stride, pg1);
    pg1 = pg2;
    pg2 = step_page(pt, w.tb, it + kLead + 2, w.plan.page);
  };
  auto plain_step = [&](int it, int st) __attribute__((always_inline)) {
    next_stage(it, (st + kLead) % kStages, st % 2 == 0);
    attn_step<false>(A, st, qf[0], w.lane, w.rc.g, rowf[0], 0u, zref, lsum, acc, job, w.plan);
  };
  auto masked_step = [&](int it) __attribute__((always_inline)) {
    next_stage(it, (it + kLead) % kStages, it % 2 == 0);
    attn_step<true>(A, it % kStages, qf[0], w.lane, w.rc.g, rowf[0], key_mask(w.tb, w.tw, it, w.rc), zref, lsum,
                    acc, job, w.plan);
  };
  int it = 0;
  for (; it < min(w.m_early, w.n_st); ++it) masked_step(it);
  // the unmasked steps lo .. hi-1, with their stages known: the loop walks
  // the aligned groups of four steps that hold them (step 4j + i is at stage
  // i) and runs the ones in range.  The range guard runs after steps 63,
  // 127, ...: a step there is at stage 3.
  static_assert(kStages == 4 && kGuardSteps % kStages == 0, "four steps, one per stage");
  {
    const int lo = it, hi = w.m_late;
    for (int i0 = lo & ~(kStages - 1); i0 < hi; i0 += kStages) {
      if (i0 >= lo) plain_step(i0, 0);
      if (i0 + 1 >= lo && i0 + 1 < hi) plain_step(i0 + 1, 1);
      if (i0 + 2 >= lo && i0 + 2 < hi) plain_step(i0 + 2, 2);
      if (i0 + 3 >= lo && i0 + 3 < hi) {
        plain_step(i0 + 3, 3);
        if ((i0 + 3) % kGuardSteps == kGuardSteps - 1) guard_planes(acc, w.lane, zref, lsum);
      }
    }
    it = max(lo, hi);
  }
  for (; it < w.n_st; ++it) masked_step(it);

  // ---- epilogue: recombine the digit planes, scale by cap / (Xmax * l), store.
  // Output register i of tile nt is row 4g + i, channel 16nt + lane%16.
  const float rscale = kCap / (kXmax * rows_sum(lsum));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * w.rc.g + i;
    const float rr = __shfl(rscale, r);
    const int t = w.qt_local * kPage + r;
    if (!w.wave_ok || t >= a.n_tokens) continue;
    const long base = ((long)t * a.n_q_heads + w.head0) * kHeadDim + (w.lane & 15);
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      const float x = fmaf((float)acc[1][nt][i], 256.f, (float)acc[0][nt][i]);
      const float o = x * rr;
      if (OUT_BF16) {
        const uint32_t u32 = __float_as_uint(o);  // round to nearest even
        const uint16_t hb = (uint16_t)((u32 + 0x7fffu + ((u32 >> 16) & 1u)) >> 16);
        __builtin_nontemporal_store(hb, reinterpret_cast<uint16_t*>(a.out) + base + 16 * nt);
      } else {
        __builtin_nontemporal_store(o, reinterpret_cast<float*>(a.out) + base + 16 * nt);
      }
    }
  }
}

template <int WPG, bool OUT_BF16, bool QF>
static void launch_wpg(const AttnArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_attn_kernel<WPG, OUT_BF16, QF>), dim3(grid), dim3(64 * kWaves), 0, stream, a,
                     a.page_table);
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
  a.n_groups = (int)pg.n_groups;
  a.streams = pg.streams;
  a.xcd_r = pg.xcd_r;
  a.xcd_q = pg.xcd_q;
  long workgroups = pg.workgroups;
  a.runs = pg.xcd_r && pg.n_groups >= kRunGroups * pg.xcd_r;
  if (a.runs) {
    // runs of equal work: group g's key steps (its longest list) plus a fixed
    // cost, the list as the kernel forms it
    static_assert(kXcds + 1 <= (int)(sizeof(a.run_start) / sizeof(a.run_start[0])), "run bounds");
    const int t_end = a.tile0 + a.n_tiles - 1;
    auto work = [&](long g) {
      const int t0 = (int)((t_end / pg.tpg - g) * pg.tpg);
      const int tz = std::min(t0 + pg.tpg - 1, t_end);
      const TileBlocks tb = tile_blocks(t0, a.window_blocks, a.sink_blocks);
      return (long)((tb.n_sink + (tz + 1 - tb.win_start) + 3) >> 2) + kGroupCost;
    };
    long total = 0;
    for (long g = 0; g < pg.n_groups; ++g) total += work(g);
    long acc = 0, g = 0, longest = 0;
    a.run_start[0] = 0;
    for (int r = 1; r <= pg.xcd_r; ++r) {
      const long goal = r == pg.xcd_r ? total : total * r / pg.xcd_r;
      while (g < pg.n_groups && acc + work(g) <= goal) acc += work(g++);
      if (r == pg.xcd_r) g = pg.n_groups;
      a.run_start[r] = (int)g;
      longest = std::max(longest, (long)(a.run_start[r] - a.run_start[r - 1]));
    }
    workgroups = (long)kXcds * longest;
  }
  const unsigned grid = (unsigned)workgroups;
  if (pg.wpg == 4) launch_wpg<4>(a, out_bf16, grid, stream);
  else if (pg.wpg == 2) launch_wpg<2>(a, out_bf16, grid, stream);
  else launch_wpg<1>(a, out_bf16, grid, stream);
  return hipGetLastError();
}

}  // namespace wpa
