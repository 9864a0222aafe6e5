// Shared device helpers of the gfx950 PBD step library: types, bf16 and fp16
// conversions, matrix-core wrappers and the packed activation layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/la_pbd.h"

namespace la {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kWave = 64;
constexpr int kHeadDim = 128;
constexpr int kBlock = 16;   // KV page size in tokens

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fp16_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

// Split x into bf16 hi + lo: hi = bf16(x), lo = bf16(x - hi).  hi + lo carries
// about 16 significant bits of x, enough for fp32-grade products with exact bf16
// weights on the matrix cores.
__device__ __forceinline__ void split_hi_lo(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
}

// ---------------------------------------------------------------- buffer loads

// Buffer loads: an offset at or past the end of the resource reads zero and
// touches no memory, which masks a unit without a branch.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kCfgDword = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kNonTemporal = 2;        // cache policy: streaming

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kCfgDword);
}

template <int POLICY>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}

// Direct-to-LDS copies through a buffer resource: lane l's bytes at voff +
// soff land at lds_dst + l * size.  (The buffer form keeps these loads in the
// same in-order class as the weight loads, so the compiler's waits on the
// weights stay exact.)  The LDS address-space cast lives here, in device-only
// code.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds_dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds_dst, 4, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------- matrix cores

// D[16x16] += A[16x32] . B[32x16]; lane l holds A row l%16, B column l%16 and
// 8 k-values selected by l/16; D lane l holds rows 4*(l/16)+e, column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same with 4 k-values per lane (k = 4*(l/16) + e).
__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- packed activations
//
// "Apack": the matrix-core A operand of a small-M GEMM.  Rows are grouped in
// tiles of 8 real rows; a tile holds 16 operand rows: rows 0..7 the bf16 hi part
// of real rows 8*mt .. 8*mt+7, rows 8..15 their lo part (absent rows are zero).
// Layout: uint16 [MT][K/8][16][8]: for every 8-wide k chunk, 16 rows of 8
// values, so that one 16-byte load per lane fetches a whole operand fragment.
// For INT4 weights the 8 values of a chunk are stored in the order
// k0 k4 k1 k5 k2 k6 k3 k7, the order in which the weight nibbles are expanded.

__host__ __device__ __forceinline__ size_t apack_elems(int M, int K) {
  return (size_t)((M + 7) / 8) * (size_t)K * 16;
}

__device__ __forceinline__ int apack_perm_pos(int e, bool int4) {
  return int4 ? ((e & 3) * 2 + (e >> 2)) : e;
}

// Pack one 8-wide chunk (values v[0..7] = k0..k7 of real row m, chunk kc).
__device__ __forceinline__ void apack_store_chunk(uint16_t* ap, int K, int m, int kc,
                                                  const float v[8], bool int4) {
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t h, l;
    split_hi_lo(v[e], h, l);
    const int p = apack_perm_pos(e, int4);
    hi[p] = h;
    lo[p] = l;
  }
  const int mt = m >> 3, r = m & 7;
  const size_t base = (((size_t)mt * (K / 8) + kc) * 16 + r) * 8;
  u32x4 H = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
             hi[6] | (hi[7] << 16)};
  u32x4 L = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
             lo[6] | (lo[7] << 16)};
  *(u32x4*)(ap + base) = H;
  *(u32x4*)(ap + base + 8 * 8) = L;
}

__device__ __forceinline__ void apack_store_zero_chunk(uint16_t* ap, int K, int m, int kc) {
  const int mt = m >> 3, r = m & 7;
  const size_t base = (((size_t)mt * (K / 8) + kc) * 16 + r) * 8;
  u32x4 z = {0u, 0u, 0u, 0u};
  *(u32x4*)(ap + base) = z;
  *(u32x4*)(ap + base + 64) = z;
}

// ---------------------------------------------------------------- misc

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float silu_f(float z) {
  return z / (1.0f + expf(-z));
}

}  // namespace la
