// Device helpers shared by the small-M and the large-M GEMM kernels: column
// maps of the weight layouts, per-lane weight addressing and buffer loads.
#pragma once

#include "la_internal.hpp"

namespace la {

// ---------------------------------------------------------------- column maps

// Weight row read by operand column c (0..15) of column tile `tile`.
// INT4 weights in the matrix cores: a dword w of 8 nibbles becomes 4 dwords of
// two bf16 each, nibbles k and k + 4 as 128 + q (bf16 0x4300 | q), so a group's
// products carry 128 times the activation sum, removed with the group sums.
// The bias lives in a vector register that the compiler cannot see into (an
// empty asm), so shift, mask and bias are one v_lshrrev and one v_and_or_b32
// per dword (gfx9 reads at most one scalar or literal operand per vector op).
__device__ __forceinline__ uint32_t int4_bias_reg() {
  uint32_t b = 0x43004300u;
  asm volatile("" : "+v"(b));
  return b;
}
__device__ __forceinline__ u32x4 int4_to_bf16x8(uint32_t w, uint32_t bias) {
  u32x4 bb;
  bb[0] = (w & 0x000F000Fu) | bias;
  bb[1] = ((w >> 4) & 0x000F000Fu) | bias;
  bb[2] = ((w >> 8) & 0x000F000Fu) | bias;
  bb[3] = ((w >> 12) & 0x000F000Fu) | bias;
  return bb;
}

template <int EPI>
__device__ __forceinline__ int col_row(int N, int tile, int c) {
  if (EPI == EPI_SILU) {
    // columns 0..7: gate rows, 8..15: the matching up rows
    return c < 8 ? tile * 8 + c : N / 2 + tile * 8 + (c - 8);
  } else if (EPI == EPI_QKV) {
    // tile = (head, sub): dims sub*8 + c and 64 + sub*8 + c of one head, so each
    // RoPE pair (i, i + 64) stays inside the tile
    const int head = tile >> 3, sub = tile & 7;
    return head * kHeadDim + (c < 8 ? sub * 8 + c : 64 + sub * 8 + (c - 8));
  } else {
    return tile * 16 + c;
  }
}

__host__ __device__ __forceinline__ int layout_row(int layout, int N, int tile, int c) {
  if (layout == LA_LAYOUT_TILED_GU) return c < 8 ? tile * 8 + c : N / 2 + tile * 8 + (c - 8);
  if (layout == LA_LAYOUT_TILED_QKV) {
    const int head = tile >> 3, sub = tile & 7;
    return head * kHeadDim + (c < 8 ? sub * 8 + c : 64 + sub * 8 + (c - 8));
  }
  return tile * 16 + c;
}

// Weight location of this lane for a work item, as byte offsets into the
// weight (and INT4 scale) buffer resources.
struct WPtr {
  uint32_t w;           // unit 0 of this lane
  uint32_t ustride;     // between consecutive units
  uint32_t s;           // INT4: scale of unit 0 for this lane
  uint32_t sstride;     // INT4: between consecutive units
};

template <bool INT4, int EPI>
__device__ __forceinline__ WPtr wptr(const GemmArgs& a, int tile) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  WPtr p;
  p.s = 0;
  p.sstride = 0;
  if (a.layout != LA_LAYOUT_ROWS) {
    const int UT = INT4 ? (a.K >> 7) : (a.K >> 5);
    p.w = ((uint32_t)tile * UT * 64 + lane) * 16;
    p.ustride = 1024;
    if (INT4) {
      p.s = ((uint32_t)tile * UT * 16 + c) * 2;
      p.sstride = 32;
    }
  } else {
    int r = col_row<EPI>(a.N, tile, c);
    if (r >= a.N) r = a.N - 1;  // lm_head tail columns: read a valid row, drop the result
    if (!INT4) {
      p.w = ((uint32_t)r * a.K + g * 8) * 2;
      p.ustride = 64;
    } else {
      p.w = (uint32_t)r * (a.K >> 1) + g * 16;
      p.ustride = 64;
      p.s = (uint32_t)r * (a.K >> 7) * 2;
      p.sstride = 2;
    }
  }
  return p;
}

// Running top-2 of a row: (v1, i1) the best value and its column (lowest index
// on ties), v2 the second best value.
// Repetition penalty of a used token's logit: divided by theta when
// positive, multiplied otherwise (a positive per-row scale applied before or
// after gives the same ranking).
__device__ __forceinline__ float rep_penalise(float v, float theta) {
  return v > 0.f ? v / theta : v * theta;
}

// The bitmap word of row m holding vocabulary id n (bit n % 32), 0 without a
// bitmap.
__device__ __forceinline__ uint32_t rep_word(const GemmArgs& a, int m, int n) {
  return a.rep_bits ? a.rep_bits[(size_t)(m / a.rep_rows) * a.rep_words + (n >> 5)] : 0u;
}

struct Top2 {
  float v1, v2;
  int i1;
};

__device__ __forceinline__ void top2_merge(float& v1, int& i1, float& v2, float b1, int bi,
                                           float b2) {
  if (b1 > v1 || (b1 == v1 && bi < i1)) {
    v2 = fmaxf(b2, v1);
    v1 = b1;
    i1 = bi;
  } else {
    v2 = fmaxf(v2, b1);
  }
}

}  // namespace la
