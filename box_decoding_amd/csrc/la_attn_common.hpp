// Device pieces of the window attention shared by the attention kernels and
// the persistent front-half kernel: page staging in LDS, the per-pair score
// and value products with the online softmax.
#pragma once

#include "la_internal.hpp"

namespace la {

// Real window rows of sequence b (1 .. W).
__device__ __forceinline__ int attn_wlen(const AttnArgs& a, int b) {
  return a.window_len ? min(max(a.window_len[b], 1), a.W) : a.W;
}

__device__ __forceinline__ int attn_keys(const AttnArgs& a, int b) {
  int n = a.prefix_len[b] + attn_wlen(a, b);
  if (n > a.cap) n = a.cap;
  if (n < 0) n = 0;
  return n;
}

// A page in LDS: K [16 keys][128 dims] with the 16-byte chunks of key k
// rotated by XOR with k (so the 16 lanes that read one chunk of 16 different
// keys hit 16 different bank groups), then V^T [128 dims][16 keys] as stored.
constexpr int kPageBytes = 2 * kBlock * kHeadDim * 2;  // 8 KB
constexpr int kPairBytes = 2 * kPageBytes;

// Piece q (0..7, 1 KB each) of a page: the 16-byte granule lane l writes in
// LDS (q * 64 + l) and where it comes from in the cache page.
__device__ __forceinline__ uint32_t page_piece_src(int q, int lane) {
  const int p = (q & 3) * 64 + lane;  // granule within the K or V half
  if (q < 4) {
    const int k = p >> 4, cch = (p & 15) ^ (k & 15);
    return (uint32_t)(k * 256 + cch * 16);
  }
  return (uint32_t)p * 16;
}

// K of two pages and V^T of both for this lane.  The products run over the 32
// keys of the pair in one step; key slot 8g + e of lane group g is key 4g + e
// of the first page for e < 4 and key 4g + e - 4 of the second page for e >= 4,
// which is where the score accumulators of the two pages leave them.
struct PairRegs {
  bf16x8 ka[4], kb[4];
  s16x4 va[8], vb[8];
};

__device__ __forceinline__ void read_pair(const unsigned char* pr_lds, PairRegs& pr) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int off = r * 256 + (((kb * 4 + g) ^ r) * 16);
    pr.ka[kb] = *(const bf16x8*)(pr_lds + off);
    pr.kb[kb] = *(const bf16x8*)(pr_lds + kPageBytes + off);
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int off = 4096 + (dt * 16 + r) * 32 + g * 8;
    pr.va[dt] = *(const s16x4*)(pr_lds + off);
    pr.vb[dt] = *(const s16x4*)(pr_lds + kPageBytes + off);
  }
}

// Running state of one wave: online-softmax reference max and sum of its 16
// query columns and the unnormalised O^T tile (dims x queries).
struct AttnState {
  float m, l;
  f32x4 acc[8];
};

// The reference max moves only when a score exceeds it by more than this
// (log2 units): exp2 of at most 2^8 stays far inside fp32, and most pages then
// need no cross-lane max and no rescale.  The result is the same softmax.
constexpr float kLazyMax = 8.f;

__device__ __forceinline__ bf16x8 cat_s16x4(s16x4 a, s16x4 b) {
  const uint32_t x0 = (uint32_t)(uint16_t)a[0] | ((uint32_t)(uint16_t)a[1] << 16);
  const uint32_t x1 = (uint32_t)(uint16_t)a[2] | ((uint32_t)(uint16_t)a[3] << 16);
  const uint32_t x2 = (uint32_t)(uint16_t)b[0] | ((uint32_t)(uint16_t)b[1] << 16);
  const uint32_t x3 = (uint32_t)(uint16_t)b[2] | ((uint32_t)(uint16_t)b[3] << 16);
  const u32x4 u = {x0, x1, x2, x3};
  return __builtin_bit_cast(bf16x8, u);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// bf16 of a and b (round to nearest even, one hardware conversion), a in the
// low half.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// One pair of pages (keys p0 .. p0 + nvalid - 1 valid, nvalid >= 1) into the
// running state; this lane's query column sees the first nsc <= nvalid of
// them (fewer under the causal window, possibly none).
__device__ __forceinline__ void attn_pair(PairRegs& pr, int nvalid, int nsc, const bf16x8 (&qh)[4],
                                          const bf16x8 (&ql)[4], AttnState& st) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const float sl2 = 0.08838834764831845f * 1.4426950408889634f;  // log2(e) / sqrt(128)
  if (nvalid < 2 * kBlock) {
    // keys past the bound: zero their values (unused slots may hold anything)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (4 * g + e >= nvalid) pr.va[dt][e] = 0;
        if (kBlock + 4 * g + e >= nvalid) pr.vb[dt][e] = 0;
      }
  }
  f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = ah, bh = ah, bl = ah;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    ah = mfma_16x16x32(pr.ka[kb], qh[kb], ah);
    bh = mfma_16x16x32(pr.kb[kb], qh[kb], bh);
    al = mfma_16x16x32(pr.ka[kb], ql[kb], al);
    bl = mfma_16x16x32(pr.kb[kb], ql[kb], bl);
  }
  float sc[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sc[e] = 4 * g + e < nsc ? (ah[e] + al[e]) * sl2 : -INFINITY;
    sc[4 + e] = kBlock + 4 * g + e < nsc ? (bh[e] + bl[e]) * sl2 : -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                   fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazyMax) != 0) {  // uniform over the wave
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(st.m, mx);
    // 0 while st.m is -inf (mnew too may be -inf: a column that saw no key yet)
    const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt] *= alpha;
    st.m = mnew;
  }
  float p[8], ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = sc[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[e] - st.m);
    ps += p[e];
  }
  st.l += ps;
  // P^T operand, bf16 hi (truncated) + lo (the exact remainder, rounded)
  u32x4 H, L;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b0 = __float_as_uint(p[2 * i]), b1 = __float_as_uint(p[2 * i + 1]);
    const uint32_t h0 = b0 & 0xFFFF0000u, h1 = b1 & 0xFFFF0000u;
    H[i] = (h0 >> 16) | h1;
    L[i] = cvt_bf16x2(p[2 * i] - __uint_as_float(h0), p[2 * i + 1] - __uint_as_float(h1));
  }
  const bf16x8 ph = __builtin_bit_cast(bf16x8, H), pl = __builtin_bit_cast(bf16x8, L);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const bf16x8 v = cat_s16x4(pr.va[dt], pr.vb[dt]);
    st.acc[dt] = mfma_16x16x32(v, ph, st.acc[dt]);
    st.acc[dt] = mfma_16x16x32(v, pl, st.acc[dt]);
  }
}

}  // namespace la
