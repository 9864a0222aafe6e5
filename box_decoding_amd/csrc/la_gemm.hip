// Small-M weight-streaming GEMMs on the gfx950 matrix cores, their activation
// packing (with the fused RMSNorm) and their epilogues (bias + residual, SiLU
// gate, QKV bias + RoPE + bf16 KV-cache write, lm_head top-2).
//
// Why the matrix cores at M = 6: every weight is used by only 6 rows, so the
// work is a weight stream (6 FLOP per weight byte).  On the vector ALUs each
// bf16 weight costs a conversion plus 6 FMAs, about 70% of the chip's vector
// issue rate at the HBM rate; on the matrix cores the weight goes straight from
// HBM into the B operand and the 6 rows, split into bf16 hi and lo parts, fill
// 12 of the 16 operand rows.  The vector ALUs are left for the epilogues.
//
// Work decomposition: a workgroup owns `nt` tiles of 16 output columns over the
// whole reduction; its `nw` waves split the tiles and then K, and combine their
// partial sums through LDS.  No workgroup ever waits for another (device-wide
// fences cost far more than a kernel boundary on this chip), so each kernel's
// output is complete when it ends.  When M <= 8 the workgroup packs the
// activations itself (RMSNorm included) into LDS while its first weight loads
// are in flight; larger M reads activations packed once in global memory.
#include "la_internal.hpp"

namespace la {

// Rows per GEMM launch: four 8-row tiles keep the accumulators and the operand
// fragments of a wave in registers.
constexpr int kRowsPerLaunch = 32;

// ---------------------------------------------------------------- column maps

// Weight row read by operand column c (0..15) of column tile `tile`.
template <int EPI>
__device__ __forceinline__ int col_row(const GemmArgs& a, int tile, int c) {
  if (EPI == EPI_SILU) {
    // columns 0..7: gate rows, 8..15: the matching up rows
    const int half = a.N / 2;
    return c < 8 ? tile * 8 + c : half + tile * 8 + (c - 8);
  } else if (EPI == EPI_QKV) {
    // tile = (head, sub): dims sub*8 + c and 64 + sub*8 + c of one head, so each
    // RoPE pair (i, i + 64) stays inside the tile
    const int head = tile >> 3, sub = tile & 7;
    return head * kHeadDim + (c < 8 ? sub * 8 + c : 64 + sub * 8 + (c - 8));
  } else {
    return tile * 16 + c;
  }
}

// ---------------------------------------------------------------- weight blocks

// One pipeline stage of weights for one lane: U units of 32 (bf16) or 128
// (INT4) reduction elements of the lane's column.
template <bool INT4, int U>
struct WBlock {
  u32x4 w[U];
  float s[U];  // INT4 group scale
};

template <bool INT4, int U>
__device__ __forceinline__ void load_block(WBlock<INT4, U>& b, const GemmArgs& a, int wrow, int u,
                                           int u1) {
  const int g = (threadIdx.x & 63) >> 4;
  if (!INT4) {
    const uint16_t* wp = (const uint16_t*)a.w + (size_t)wrow * a.K + g * 8;
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (u + i < u1) b.w[i] = __builtin_nontemporal_load((const u32x4*)(wp + (size_t)(u + i) * 32));
  } else {
    const uint8_t* wp = (const uint8_t*)a.w + (size_t)wrow * (a.K >> 1) + g * 16;
    const uint16_t* sp = a.wscale + (size_t)wrow * (a.K >> 7);
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (u + i < u1) {
        b.w[i] = __builtin_nontemporal_load((const u32x4*)(wp + (size_t)(u + i) * 64));
        b.s[i] = fp16_to_f32(sp[u + i]);
      }
  }
}

// Activation fragment of row tile mt, 8-wide chunk kc, for this lane (row l%16).
__device__ __forceinline__ bf16x8 a_frag(const uint16_t* ap, int K8, int mt, int kc) {
  return *(const bf16x8*)(ap + ((size_t)mt * K8 + kc) * 128);
}

template <int MT, bool INT4, int U>
__device__ __forceinline__ void compute_block(const WBlock<INT4, U>& b, const uint16_t* ap,
                                              const float* asp, int K8, int KG, int u, int u1,
                                              int mtv, f32x4 (&acc)[MT]) {
  const int g = (threadIdx.x & 63) >> 4;
  if (!INT4) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (u + i < u1) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, b.w[i]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < mtv) acc[mt] = mfma_16x16x32(a_frag(ap, K8, mt, (u + i) * 4 + g), bv, acc[mt]);
      }
    }
  } else {
    // Every 4-byte word expands with two masks and an OR into four bf16 pairs
    // holding 128 + q (k0 k4 | k1 k5 | k2 k6 | k3 k7), the order the packed
    // activations use.  Per group: acc += scale * (sum - 136 * sum_k a_k), since
    // sum a_k (128 + q_k) - 136 sum a_k = sum a_k (q_k - 8).
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (u + i < u1) {
        f32x4 t[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = b.w[i][j];
          u32x4 bb;
          bb[0] = (w & 0x000F000Fu) | 0x43004300u;
          bb[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
          bb[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
          bb[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
          const bf16x8 bv = __builtin_bit_cast(bf16x8, bb);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < mtv) t[mt] = mfma_16x16x32(a_frag(ap, K8, mt, (u + i) * 16 + g * 4 + j), bv, t[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mtv) {
            const f32x4 as = *(const f32x4*)(asp + ((size_t)mt * KG + (u + i)) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mt][e] += b.s[i] * (t[mt][e] - 136.0f * as[e]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- LDS packing

// Pack rows m_base .. m_base+MT*8-1 of x (RMSNorm'd when a gain is given) into
// the LDS operand layout; INT4 consumers also get per-group sums.
template <int MT, bool INT4>
__device__ void pack_rows_lds(const GemmArgs& a, uint16_t* ap, float* asp, float* inv_s) {
  const int nthr = a.nw * 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int K = a.K, K8 = K >> 3;
  const int rows = min(a.M - a.m_base, MT * 8);
  for (int m = wave; m < MT * 8; m += a.nw) {
    float inv = 1.0f;
    if (m < rows && a.gain) {
      const float* xr = a.x + (size_t)(a.m_base + m) * a.ldx;
      float ss = 0.f;
      for (int k = lane * 4; k < K; k += 256) {
        const float4 v = *(const float4*)(xr + k);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = warp_sum(ss);
      inv = 1.0f / sqrtf(ss / (float)K + a.eps);
    }
    if (lane == 0) inv_s[m] = inv;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 8 * K8; idx += nthr) {
    const int m = idx / K8, kc = idx - m * K8;
    float v[8];
    if (m < rows) {
      const float* xr = a.x + (size_t)(a.m_base + m) * a.ldx + kc * 8;
      const float4 v0 = *(const float4*)xr, v1 = *(const float4*)(xr + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
      if (a.gain) {
        const float inv = inv_s[m];
        const uint4 gg = *(const uint4*)(a.gain + kc * 8);
        const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * inv * bf16_to_f32((gw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    apack_store_chunk(ap, K, m, kc, v, INT4);
  }
  if (INT4) {
    __syncthreads();
    // per (operand row, 128-group) sums of the stored bf16 values
    const int KG = K >> 7;
    for (int idx = threadIdx.x; idx < MT * 16 * KG; idx += nthr) {
      const int mt = idx / (16 * KG), rem = idx - mt * 16 * KG;
      const int gi = rem >> 4, r = rem & 15;
      float s = 0.f;
      for (int c = 0; c < 16; ++c) {
        const u32x4 q = *(const u32x4*)(ap + (((size_t)mt * K8 + gi * 16 + c) * 16 + r) * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) s += bf16_to_f32(q[j] & 0xFFFFu) + bf16_to_f32(q[j] >> 16);
      }
      asp[((size_t)mt * KG + gi) * 16 + r] = s;
    }
  }
}

// ---------------------------------------------------------------- epilogues

template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int tile0, int nt_valid, int rows,
                                         const float* outv, int ldo) {
  // outv[(t * ldo + row) * 17 + c] for column tile t of this workgroup
  const int tid = threadIdx.x, nthr = a.nw * 64;
  if (EPI == EPI_STORE) {
    for (int idx = tid; idx < nt_valid * rows * 16; idx += nthr) {
      const int t = idx / (rows * 16), rem = idx - t * rows * 16;
      const int ml = rem >> 4, c = rem & 15;
      const int m = a.m_base + ml;
      const int n = (tile0 + t) * 16 + c;
      if (n >= a.N) continue;
      float v = outv[(t * ldo + ml) * 17 + c];
      if (a.bias) v += bf16_to_f32(a.bias[n]);
      if (a.residual) v += a.residual[(size_t)m * a.ldy + n];
      a.y[(size_t)m * a.ldy + n] = v;
    }
  } else if (EPI == EPI_SILU) {
    const int F = a.N / 2;
    for (int idx = tid; idx < nt_valid * rows * 8; idx += nthr) {
      const int t = idx / (rows * 8), rem = idx - t * rows * 8;
      const int ml = rem >> 3, c = rem & 7;
      const int m = a.m_base + ml;
      const float* o = outv + (t * ldo + ml) * 17;
      const float v = silu_f(o[c]) * o[c + 8];
      const int n = (tile0 + t) * 8 + c;
      if (a.y) a.y[(size_t)m * a.ldy + n] = v;
      if (a.y_apack) {
        // hi/lo bf16 straight into the packed operand of the next GEMM (K = F)
        uint32_t h, l;
        split_hi_lo(v, h, l);
        const size_t base = (((size_t)(m >> 3) * (F / 8) + (n >> 3)) * 16 + (m & 7)) * 8 + (n & 7);
        a.y_apack[base] = (uint16_t)h;
        a.y_apack[base + 64] = (uint16_t)l;
      }
    }
  } else if (EPI == EPI_QKV) {
    const int Hq = a.n_heads, Hkv = a.n_kv_heads;
    for (int idx = tid; idx < nt_valid * rows * 8; idx += nthr) {
      const int t = idx / (rows * 8), rem = idx - t * rows * 8;
      const int ml = rem >> 3, c = rem & 7;
      const int tile = tile0 + t;
      const int head = tile >> 3, sub = tile & 7;
      const int m = a.m_base + ml;
      const int i = sub * 8 + c;  // rotary pair index
      const int r1 = head * kHeadDim + i, r2 = r1 + 64;
      const float* o = outv + (t * ldo + ml) * 17;
      float x1 = o[c], x2 = o[c + 8];
      if (a.bias) {
        x1 += bf16_to_f32(a.bias[r1]);
        x2 += bf16_to_f32(a.bias[r2]);
      }
      if (head < Hq + Hkv) {
        const float2 cs = a.rope[(size_t)m * 64 + i];
        const float y1 = x1 * cs.x - x2 * cs.y;
        const float y2 = x2 * cs.x + x1 * cs.y;
        x1 = y1;
        x2 = y2;
      }
      if (head < Hq) {
        a.y[(size_t)m * a.ldy + r1] = x1;
        a.y[(size_t)m * a.ldy + r2] = x2;
        continue;
      }
      if (a.flags && a.flags[m] != 0) continue;
      const int b = m / a.W, j = m - b * a.W;
      const int pos = a.prefix_len[b] + j;
      if (pos < 0 || pos >= a.max_blocks * kBlock) continue;
      const int blk = a.block_table[(size_t)b * a.max_blocks + pos / kBlock];
      if (blk < 0 || blk >= a.num_blocks) continue;
      const int slot = pos % kBlock;
      if (head < Hq + Hkv) {
        const int kvh = head - Hq;
        uint16_t* kp = a.kc + (((size_t)blk * Hkv + kvh) * kBlock + slot) * kHeadDim;
        kp[i] = (uint16_t)f32_to_bf16_rne(x1);
        kp[i + 64] = (uint16_t)f32_to_bf16_rne(x2);
      } else {
        const int kvh = head - Hq - Hkv;
        uint16_t* vp = a.vc + ((size_t)blk * Hkv + kvh) * kHeadDim * kBlock;
        vp[(size_t)i * kBlock + slot] = (uint16_t)f32_to_bf16_rne(x1);
        vp[(size_t)(i + 64) * kBlock + slot] = (uint16_t)f32_to_bf16_rne(x2);
      }
    }
  } else {  // EPI_ARGMAX: per row top-2 over the workgroup's valid columns
    for (int ml = tid; ml < rows; ml += nthr) {
      const int m = a.m_base + ml;
      float v1 = -INFINITY, v2 = -INFINITY;
      int i1 = 0x7FFFFFFF;
      for (int t = 0; t < nt_valid; ++t) {
        for (int c = 0; c < 16; ++c) {
          const int n = (tile0 + t) * 16 + c;
          if (n >= a.N) break;
          const float v = outv[(t * ldo + ml) * 17 + c];
          if (v > v1) {
            v2 = v1;
            v1 = v;
            i1 = n;
          } else {
            v2 = fmaxf(v2, v);
          }
        }
      }
      float* o = a.amax + ((size_t)m * a.n_parts + blockIdx.x) * 3;
      o[0] = v1;
      o[1] = __int_as_float(i1);
      o[2] = v2;
    }
  }
}

// ---------------------------------------------------------------- GEMM kernel

template <int MT, bool INT4, bool LDSA, int EPI>
__global__ __launch_bounds__(512) void k_gemm(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float inv_s[64];
  constexpr int U = INT4 ? (MT <= 2 ? 4 : 2) : (MT <= 2 ? 8 : 4);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nt = a.nt, nks = a.nw / a.nt;
  const int tile0 = blockIdx.x * nt;
  const int nt_valid = min(nt, a.n_tiles - tile0);
  const int tw = wave % nt, ks = wave / nt;
  const int tile = tile0 + min(tw, nt_valid - 1);
  const int K8 = a.K >> 3, KG = a.K >> 7;
  const int units = INT4 ? (a.K >> 7) : (a.K >> 5);
  const int u0 = units * ks / nks, u1 = units * (ks + 1) / nks;
  const bool active = tw < nt_valid;
  int wrow = col_row<EPI>(a, tile, lane & 15);
  if (wrow >= a.N) wrow = a.N - 1;  // tail columns of the lm_head: read a valid row, drop the result
  const int rows = min(min(kRowsPerLaunch, a.M - a.m_base), MT * 8);
  const int mtv = (rows + 7) >> 3;

  // the first weight stage goes out before the activations are packed
  WBlock<INT4, U> b0, b1;
  int u = u0;
  if (active) load_block<INT4, U>(b0, a, wrow, u, u1);

  const uint16_t* ap;
  const float* asp;
  const int lane_off = (lane & 15) * 8;  // operand row; the k chunk is added per step
  if (LDSA) {
    uint16_t* lds_a = (uint16_t*)smem;
    float* lds_as = (float*)(smem + (size_t)MT * a.K * 32);
    pack_rows_lds<MT, INT4>(a, lds_a, lds_as, inv_s);
    __syncthreads();
    ap = lds_a + lane_off;
    asp = lds_as + 4 * (lane >> 4);
  } else {
    ap = a.apack + (size_t)(a.m_base >> 3) * K8 * 128 + lane_off;
    asp = a.asum ? a.asum + (size_t)(a.m_base >> 3) * KG * 16 + 4 * (lane >> 4) : nullptr;
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (active) {
    while (true) {
      if (u + U < u1) load_block<INT4, U>(b1, a, wrow, u + U, u1);
      compute_block<MT, INT4, U>(b0, ap, asp, K8, KG, u, u1, mtv, acc);
      u += U;
      if (u >= u1) break;
      if (u + U < u1) load_block<INT4, U>(b0, a, wrow, u + U, u1);
      compute_block<MT, INT4, U>(b1, ap, asp, K8, KG, u, u1, mtv, acc);
      u += U;
      if (u >= u1) break;
    }
  }

  // ---- combine waves (the LDS operand area is reused)
  f32x4* red = (f32x4*)smem;                                   // [nw][MT][64]
  float* outv = (float*)(smem + (size_t)a.nw * MT * 64 * 16);  // [nt][MT*8][17]
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[((size_t)wave * MT + mt) * 64 + lane] = acc[mt];
  __syncthreads();
  // real row r of tile mt = operand row r (hi) + operand row r + 8 (lo)
  const int ldo = MT * 8;
  for (int idx = threadIdx.x; idx < nt * MT * 128; idx += a.nw * 64) {
    const int t = idx / (MT * 128), rem = idx - t * MT * 128;
    const int mt = rem >> 7, r = (rem >> 4) & 7, c = rem & 15;
    const int lh = (r >> 2) * 16 + c, ll = ((r + 8) >> 2) * 16 + c, e = r & 3;
    float v = 0.f;
    for (int s = 0; s < nks; ++s) {
      const int w = s * nt + t;
      v += red[((size_t)w * MT + mt) * 64 + lh][e] + red[((size_t)w * MT + mt) * 64 + ll][e];
    }
    outv[(t * ldo + mt * 8 + r) * 17 + c] = v;
  }
  __syncthreads();
  epilogue<EPI>(a, tile0, nt_valid, rows, outv, ldo);
}

// ---------------------------------------------------------------- packing kernel

// One workgroup per operand row: optional RMSNorm, then bf16 hi/lo split into the
// packed layout (plus per-group sums for INT4 consumers).
__global__ __launch_bounds__(256) void k_pack(PackArgs a) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int K8 = a.K >> 3;
  if (m >= a.M) {
    for (int kc = threadIdx.x; kc < K8; kc += 256) apack_store_zero_chunk(a.apack, a.K, m, kc);
    if (a.int4 && a.asum) {
      const int KG = a.K >> 7;
      for (int gi = threadIdx.x; gi < KG; gi += 256) {
        float* as = a.asum + ((size_t)(m >> 3) * KG + gi) * 16;
        as[m & 7] = 0.f;
        as[(m & 7) + 8] = 0.f;
      }
    }
    return;
  }
  const float* x = a.x + (size_t)m * a.ldx;
  float inv = 1.0f;
  if (a.gain) {
    float ss = 0.f;
    for (int k = threadIdx.x * 4; k < a.K; k += 1024) {
      const float4 v = *(const float4*)(x + k);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = warp_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
  }
  const int KG = a.K >> 7;
  for (int kc0 = 0; kc0 < K8; kc0 += 256) {
    const int kc = kc0 + threadIdx.x;
    float hs = 0.f, ls = 0.f;
    if (kc < K8) {
      float v[8];
      const float4 v0 = *(const float4*)(x + kc * 8);
      const float4 v1 = *(const float4*)(x + kc * 8 + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
      if (a.gain) {
        const uint4 gg = *(const uint4*)(a.gain + kc * 8);
        const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t gb = (gw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          v[e] = v[e] * inv * bf16_to_f32(gb);
        }
      }
      apack_store_chunk(a.apack, a.K, m, kc, v, a.int4);
      if (a.int4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t h, l;
          split_hi_lo(v[e], h, l);
          hs += bf16_to_f32(h);
          ls += bf16_to_f32(l);
        }
      }
    }
    if (a.int4 && a.asum) {
      // 16 consecutive chunks form one 128-wide group
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        hs += __shfl_xor(hs, o);
        ls += __shfl_xor(ls, o);
      }
      if (kc < K8 && (kc & 15) == 0) {
        float* as = a.asum + ((size_t)(m >> 3) * KG + (kc >> 4)) * 16;
        as[m & 7] = hs;
        as[(m & 7) + 8] = ls;
      }
    }
  }
}

// ---------------------------------------------------------------- argmax reduce

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

__global__ __launch_bounds__(1024) void k_argmax_reduce(const float* amax, int n_parts,
                                                        const int32_t* flags, int32_t* ids,
                                                        float* top1, float* gap, int32_t* err) {
  __shared__ float s1[1024], s2[1024];
  __shared__ int si[1024];
  const int m = blockIdx.x;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7FFFFFFF;
  for (int t = threadIdx.x; t < n_parts; t += 1024) {
    const float* p = amax + ((size_t)m * n_parts + t) * 3;
    top2_merge(v1, i1, v2, p[0], __float_as_int(p[1]), p[2]);
  }
  s1[threadIdx.x] = v1;
  s2[threadIdx.x] = v2;
  si[threadIdx.x] = i1;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      float a1 = s1[threadIdx.x], a2 = s2[threadIdx.x];
      int ai = si[threadIdx.x];
      top2_merge(a1, ai, a2, s1[threadIdx.x + o], si[threadIdx.x + o], s2[threadIdx.x + o]);
      s1[threadIdx.x] = a1;
      s2[threadIdx.x] = a2;
      si[threadIdx.x] = ai;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int f = flags ? flags[m] : 0;
    ids[m] = f ? -1 : si[0];
    if (top1) top1[m] = s1[0];
    if (gap) gap[m] = s1[0] - s2[0];
    if (f && err) atomicOr(err, f);
  }
}

// ---------------------------------------------------------------- host side

static size_t gemm_smem(const GemmPlan& p, int K, bool int4) {
  const size_t red = (size_t)p.nw * p.mt * 64 * 16 + (size_t)p.nt * p.mt * 8 * 17 * 4;
  const size_t opnd =
      p.lds ? (size_t)p.mt * K * 32 + (int4 ? (size_t)p.mt * (K / 128) * 16 * 4 : 0) : 0;
  return red > opnd ? red : opnd;
}

// Largest dynamic LDS a workgroup may use (queried once; static LDS is small).
static size_t lds_limit() {
  static size_t lim = 0;
  if (!lim) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
      lim = (size_t)v;
    else
      lim = 64 * 1024;
  }
  return lim - 1024;  // headroom for the kernels' static LDS
}

GemmPlan plan_gemm(int M, int N, int K, bool int4, int epi, bool x_available) {
  GemmPlan p;
  p.n_tiles = (epi == EPI_SILU) ? (N / 2) / 8 : (N + 15) / 16;
  const int rows = M < kRowsPerLaunch ? M : kRowsPerLaunch;
  const int mt = (rows + 7) / 8;
  p.mt = mt <= 1 ? 1 : mt <= 2 ? 2 : 4;
  p.launches = (M + kRowsPerLaunch - 1) / kRowsPerLaunch;
  // pack in LDS when one row tile covers M and the operand fits in 64 KB
  p.lds = x_available && M <= 8 &&
          (size_t)K * 32 + (int4 ? (size_t)(K / 128) * 64 : 0) <= lds_limit();
  switch (epi) {
    case EPI_SILU: p.nt = 4; break;
    case EPI_ARGMAX: p.nt = 4; break;
    default: p.nt = 1; break;
  }
  p.nw = 8;
  // keep enough workgroups to cover the chip
  while (p.nt > 1 && (p.n_tiles + p.nt - 1) / p.nt < 256) p.nt >>= 1;
  p.grid = (p.n_tiles + p.nt - 1) / p.nt;
  p.smem = gemm_smem(p, K, int4);
  return p;
}

template <int MT, bool INT4, bool LDSA>
static hipError_t launch_gemm_mt(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  const dim3 grid(p.grid), block(p.nw * 64);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<MT, INT4, LDSA, EPI_STORE>), grid, block, p.smem, s, a); break;
    case EPI_SILU: hipLaunchKernelGGL((k_gemm<MT, INT4, LDSA, EPI_SILU>), grid, block, p.smem, s, a); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemm<MT, INT4, LDSA, EPI_QKV>), grid, block, p.smem, s, a); break;
    default: hipLaunchKernelGGL((k_gemm<MT, INT4, LDSA, EPI_ARGMAX>), grid, block, p.smem, s, a); break;
  }
  return hipGetLastError();
}

template <bool INT4>
static hipError_t launch_gemm_fmt(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  if (p.lds) return launch_gemm_mt<1, INT4, true>(a, epi, p, s);
  switch (p.mt) {
    case 1: return launch_gemm_mt<1, INT4, false>(a, epi, p, s);
    case 2: return launch_gemm_mt<2, INT4, false>(a, epi, p, s);
    default: return launch_gemm_mt<4, INT4, false>(a, epi, p, s);
  }
}

hipError_t launch_gemm(GemmArgs a, int epi, bool int4, hipStream_t s) {
  const GemmPlan p = plan_gemm(a.M, a.N, a.K, int4, epi, a.x != nullptr);
  a.n_tiles = p.n_tiles;
  a.nt = p.nt;
  a.nw = p.nw;
  a.n_parts = p.grid;
  for (int l = 0; l < p.launches; ++l) {
    a.m_base = l * kRowsPerLaunch;
    const int rows = (a.M - a.m_base) < kRowsPerLaunch ? (a.M - a.m_base) : kRowsPerLaunch;
    const int mt8 = (rows + 7) / 8;
    GemmPlan pl = p;
    pl.mt = mt8 <= 1 ? 1 : mt8 <= 2 ? 2 : 4;
    pl.smem = gemm_smem(pl, a.K, int4);
    hipError_t e = int4 ? launch_gemm_fmt<true>(a, epi, pl, s) : launch_gemm_fmt<false>(a, epi, pl, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  // every operand row of the last tile is written (rows >= M become zero)
  const int rows = ((a.M + 7) / 8) * 8;
  hipLaunchKernelGGL(k_pack, dim3(rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(const float* amax, int M, int n_parts, const int32_t* flags,
                                int32_t* ids, float* top1, float* gap, int32_t* err,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_reduce, dim3(M), dim3(1024), 0, s, amax, n_parts, flags, ids, top1,
                     gap, err);
  return hipGetLastError();
}

}  // namespace la
