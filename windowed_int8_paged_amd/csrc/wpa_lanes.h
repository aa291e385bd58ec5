// Wave-level helpers shared by the attention and decode kernels: operand
// types, the LDS tile swizzle, the transposing V-operand read and reductions
// over the four 16-lane rows of a wave.
#pragma once

#include "wpa_common.h"

namespace wpa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
#define WPA_LDS __attribute__((address_space(3)))
#define WPA_CONST __attribute__((address_space(4)))

// Staged K and V tiles are row-major (row = key of a 64-key tile, 256 bytes)
// with the 16-byte chunk c of row r stored in slot c ^ swz(r).  The
// operand reads below then touch every bank once per half wave: the K reads
// see 16 consecutive rows of one page (slots r%16 ^ const), the transposing V
// reads rows 8h..8h+7 and 16+8h..16+8h+7 (slots m and 8 + m).
__device__ inline int swz(int r) { return (r & 15) ^ (((r >> 4) & 1) << 3); }

// B operand of a PV product over one 64-key tile staged as above: lane
// (column j, row group g) gets 16 keys of channel 16 nt + j in the order of
// the P operand, slot b holding key 16(b/4) + 4g + b%4.  Two transposing reads
// give slots 0-7 (pages 0, 1) and 8-15 (pages 2, 3).
struct VFrag {
  const int8_t* row1;
  const int8_t* row2;
  int sw, sw2;
  __device__ VFrag(const int8_t* tile, int lane) {
    const int g = lane >> 4, j = lane & 15, kk = j >> 1;
    const int key1 = 16 * (kk >> 2) + 4 * g + (kk & 3);
    row1 = tile + key1 * kHeadDim + 8 * (j & 1);
    row2 = row1 + 32 * kHeadDim;  // key1 + 32
    sw = swz(key1);
    sw2 = swz(key1 + 32);
  }
  __device__ v4i operator()(int nt) const {
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((WPA_LDS v2i*)(row1 + 16 * (nt ^ sw)));
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((WPA_LDS v2i*)(row2 + 16 * (nt ^ sw2)));
    return v4i{lo.x, lo.y, hi.x, hi.y};
  }
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

// Page maxima over the four 16-lane rows for the four pages at once:
// afterwards every lane holds all four.  The values are the bit patterns of
// non-negative floats, whose unsigned order is their float order, so the
// maxima are integer maxima (no NaN-quieting canonicalisations).
__device__ inline uint32_t swap16u(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
  return a;
}
__device__ inline void swap32u(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ inline void page_maxima(uint32_t (&mx)[4]) {
  uint32_t a = mx[0], b = mx[1], c = mx[2], d = mx[3];
  swap16u(a, b);
  const uint32_t x01 = max(a, b);  // R0: p0(R0,R1)  R1: p1(R0,R1)  R2: p0(R2,R3)  R3: p1(R2,R3)
  swap16u(c, d);
  const uint32_t x23 = max(c, d);
  uint32_t e0 = x01, e1 = x23;
  swap32u(e0, e1);
  const uint32_t y = max(e0, e1);  // row Rk holds the full max of page k
  uint32_t g0 = y, g1 = y;
  swap16u(g0, g1);  // rows 0,1: (M0, M1); rows 2,3: (M2, M3)
  uint32_t m0 = g0, m2 = g0, m1 = g1, m3 = g1;
  swap32u(m0, m2);  // every lane: m0 = M0, m2 = M2
  swap32u(m1, m3);
  mx[0] = m0;
  mx[1] = m1;
  mx[2] = m2;
  mx[3] = m3;
}

}  // namespace wpa
