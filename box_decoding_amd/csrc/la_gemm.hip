// Small-M weight-streaming GEMMs on the gfx950 matrix cores, the activation
// packing kernel (with the fused residual sum and RMSNorm) and the epilogues
// (bias + residual, SiLU gate, QKV bias + RoPE + bf16 KV-cache write, lm_head
// top-2).
//
// Why the matrix cores at M = 6: every weight is used by only 6 rows, so the
// work is a weight stream (6 FLOP per weight byte).  On the vector ALUs each
// bf16 weight costs a conversion plus 6 FMAs, about 70% of the chip's vector
// issue rate at the HBM rate; on the matrix cores the weight goes straight from
// HBM into the B operand and the 6 rows, split into bf16 hi and lo parts, fill
// 12 of the 16 operand rows.  The vector ALUs are left for the epilogues.
//
// Work decomposition: a work item is one tile of 16 operand columns (weight
// rows) and one slice of K; a workgroup walks the items blockIdx.x,
// blockIdx.x + gridDim.x, ... and its waves split the item's K range, then
// combine their partial sums through LDS.  No workgroup ever waits for
// another: a device-wide fence costs more than a kernel boundary on this chip,
// so a K-sliced GEMM writes partial sums that the next kernel adds up.  A
// wave's weight loads form one stream across work items (two stages in
// flight); loads are branch-free (clamped address, masked value) so that the
// compiler never drains the stream.
#include "la_internal.hpp"

namespace la {

// Rows per GEMM launch: four 8-row tiles keep the accumulators and the operand
// fragments of a wave in registers.
constexpr int kRowsPerLaunch = 32;

// ---------------------------------------------------------------- column maps

// Weight row read by operand column c (0..15) of column tile `tile`.
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

// ---------------------------------------------------------------- stages

// One pipeline stage for one lane: U units of 32 (bf16) or 128 (INT4) reduction
// elements of the lane's weight column, plus (bf16) the matching activation
// fragments, so that neither waits on its load.
template <bool INT4, int MT, int U>
struct Stage {
  u32x4 w[U];
  float s[INT4 ? U : 1];
  bf16x8 af[INT4 ? 1 : U][MT];
};

// Weight location of this lane for a work item: base pointers for the unit loop.
struct WPtr {
  const uint8_t* w;     // byte address of unit 0 for this lane
  size_t ustride;       // bytes between consecutive units
  const uint16_t* s;    // INT4: scale of unit 0 for this lane
  int sstride;          // INT4: scale elements between consecutive units
};

template <bool INT4, int EPI>
__device__ __forceinline__ WPtr wptr(const GemmArgs& a, int tile) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  WPtr p;
  p.s = nullptr;
  p.sstride = 0;
  if (a.layout != LA_LAYOUT_ROWS) {
    const int UT = INT4 ? (a.K >> 7) : (a.K >> 5);
    p.w = (const uint8_t*)a.w + ((size_t)tile * UT * 64 + lane) * 16;
    p.ustride = 1024;
    if (INT4) {
      p.s = a.wscale + (size_t)tile * UT * 16 + c;
      p.sstride = 16;
    }
  } else {
    int r = col_row<EPI>(a.N, tile, c);
    if (r >= a.N) r = a.N - 1;  // lm_head tail columns: read a valid row, drop the result
    if (!INT4) {
      p.w = (const uint8_t*)a.w + ((size_t)r * a.K + g * 8) * 2;
      p.ustride = 64;
    } else {
      p.w = (const uint8_t*)a.w + (size_t)r * (a.K >> 1) + g * 16;
      p.ustride = 64;
      p.s = a.wscale + (size_t)r * (a.K >> 7);
      p.sstride = 1;
    }
  }
  return p;
}

// Loads are branch-free: a unit past the wave's range reads a clamped (valid)
// address and is masked to zero at compute time.
template <bool INT4, int MT, int U>
__device__ __forceinline__ void load_stage(Stage<INT4, MT, U>& b, const WPtr& wp,
                                           const uint16_t* ap, int K8, int u, int ulo, int uhi,
                                           int mtv) {
  const int g = (threadIdx.x & 63) >> 4;
  const int ulast = uhi > ulo ? uhi - 1 : ulo;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int uu = min(u + i, ulast);
    b.w[i] = __builtin_nontemporal_load((const u32x4*)(wp.w + (size_t)uu * wp.ustride));
    if (INT4) b.s[INT4 ? i : 0] = fp16_to_f32(wp.s[(size_t)uu * wp.sstride]);
    if (!INT4) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        b.af[INT4 ? 0 : i][mt] = *(const bf16x8*)(ap + ((size_t)min(mt, mtv - 1) * K8 + uu * 4 + g) * 128);
    }
  }
}

// Activation fragment of row tile mt, 8-wide chunk kc, for this lane (row l%16).
__device__ __forceinline__ bf16x8 a_frag(const uint16_t* ap, int K8, int mt, int kc) {
  return *(const bf16x8*)(ap + ((size_t)mt * K8 + kc) * 128);
}

template <int MT, bool INT4, int U>
__device__ __forceinline__ void compute_stage(const Stage<INT4, MT, U>& b, const uint16_t* ap,
                                              const float* asp, int K8, int KG, int u, int ulo,
                                              int uhi, int mtv, f32x4 (&acc)[MT]) {
  const int g = (threadIdx.x & 63) >> 4;
  const int ulast = uhi > ulo ? uhi - 1 : ulo;
  if (!INT4) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const uint32_t keep = (u + i < uhi) ? 0xFFFFFFFFu : 0u;  // wave-uniform
      const bf16x8 bv = __builtin_bit_cast(bf16x8, b.w[i] & keep);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_16x16x32(b.af[INT4 ? 0 : i][mt], bv, acc[mt]);
    }
  } else {
    // Every 4-byte word expands with two masks and an OR into four bf16 pairs
    // holding 128 + q (k0 k4 | k1 k5 | k2 k6 | k3 k7), the order the packed
    // activations use.  Per group: acc += scale * (sum - 136 * sum_k a_k), since
    // sum a_k (128 + q_k) - 136 sum a_k = sum a_k (q_k - 8).
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const float sc = (u + i < uhi) ? b.s[INT4 ? i : 0] : 0.f;  // wave-uniform mask
      const int uu = min(u + i, ulast);
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
          t[mt] = mfma_16x16x32(a_frag(ap, K8, min(mt, mtv - 1), uu * 16 + g * 4 + j), bv, t[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 as = *(const f32x4*)(asp + ((size_t)min(mt, mtv - 1) * KG + uu) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][e] += sc * (t[mt][e] - 136.0f * as[e]);
      }
    }
  }
}

// ---------------------------------------------------------------- epilogues

struct Top2 {
  float v1, v2;
  int i1;
};

template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int tile, int ks, int rows,
                                         const float* outv, Top2& t2) {
  // outv[row * 17 + c]: operand column c of output row m_base + row
  const int tid = threadIdx.x, nthr = a.nw * 64;
  if (EPI == EPI_STORE) {
    for (int idx = tid; idx < rows * 16; idx += nthr) {
      const int ml = idx >> 4, c = idx & 15;
      const int m = a.m_base + ml;
      const int n = tile * 16 + c;
      if (n >= a.N) continue;
      float v = outv[ml * 17 + c];
      if (a.ksplit > 1) {
        a.partial[((size_t)ks * a.M + m) * a.N + n] = v;
      } else {
        if (a.bias) v += bf16_to_f32(a.bias[n]);
        if (a.residual) v += a.residual[(size_t)m * a.ldy + n];
        a.y[(size_t)m * a.ldy + n] = v;
      }
    }
  } else if (EPI == EPI_SILU) {
    const int F = a.N / 2;
    for (int idx = tid; idx < rows * 8; idx += nthr) {
      const int ml = idx >> 3, c = idx & 7;
      const int m = a.m_base + ml;
      const float* o = outv + ml * 17;
      const float v = silu_f(o[c]) * o[c + 8];
      const int n = tile * 8 + c;
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
    const int head = tile >> 3, sub = tile & 7;
    for (int idx = tid; idx < rows * 8; idx += nthr) {
      const int ml = idx >> 3, c = idx & 7;
      const int m = a.m_base + ml;
      const int i = sub * 8 + c;  // rotary pair index
      const int r1 = head * kHeadDim + i, r2 = r1 + 64;
      const float* o = outv + ml * 17;
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
  } else {  // EPI_ARGMAX: running per-row top-2 over this workgroup's columns
    if (tid < rows) {
      for (int c = 0; c < 16; ++c) {
        const int n = tile * 16 + c;
        if (n >= a.N) break;
        const float v = outv[tid * 17 + c];
        if (v > t2.v1) {
          t2.v2 = t2.v1;
          t2.v1 = v;
          t2.i1 = n;
        } else {
          t2.v2 = fmaxf(t2.v2, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- GEMM kernel

template <int MT, bool INT4, int EPI>
__global__ __launch_bounds__(512) void k_gemm(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int U = INT4 ? (MT <= 2 ? 4 : 2) : (MT <= 2 ? 8 : 4);
  // the wave index is made provably uniform: segment bounds live in scalar
  // registers and every branch on them is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nw = a.nw;
  const int K8 = a.K >> 3, KG = a.K >> 7;
  const int units = INT4 ? (a.K >> 7) : (a.K >> 5);
  const int ks_units = units / a.ksplit;  // K slice length (ksplit divides units)
  const int w0 = ks_units * wave / nw, w1 = ks_units * (wave + 1) / nw;  // within a slice
  const int nb = ((ks_units + nw - 1) / nw + U - 1) / U;  // same stage count for every wave
  const int n_items = a.n_tiles * a.ksplit;
  const int n_my = (n_items - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int total = n_my * nb;
  const int rows = min(min(kRowsPerLaunch, a.M - a.m_base), MT * 8);
  const int mtv = (rows + 7) >> 3;

  f32x4* red = (f32x4*)smem;                                    // [nw][MT][64]
  float* outv = (float*)(smem + (size_t)nw * MT * 64 * 16);     // [MT*8][17]

  const uint16_t* ap = a.apack + (size_t)(a.m_base >> 3) * K8 * 128 + (lane & 15) * 8;
  const float* asp = a.asum ? a.asum + (size_t)(a.m_base >> 3) * KG * 16 + 4 * (lane >> 4) : nullptr;

  auto item_of = [&](int bi) { return (int)blockIdx.x + (bi / nb) * (int)gridDim.x; };
  auto u_of = [&](int bi, int ks) { return ks * ks_units + w0 + (bi % nb) * U; };

  Stage<INT4, MT, U> s0, s1;
  WPtr p0, p1;
  int it0 = 0, it1 = 0;
  if (total > 0) {
    it0 = item_of(0);
    p0 = wptr<INT4, EPI>(a, it0 / a.ksplit);
    const int ks = it0 % a.ksplit;
    load_stage<INT4, MT, U>(s0, p0, ap, K8, u_of(0, ks), ks * ks_units + w0, ks * ks_units + w1, mtv);
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  Top2 t2 = {-INFINITY, -INFINITY, 0x7FFFFFFF};

  auto finish_item = [&](int item) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      red[((size_t)wave * MT + mt) * 64 + lane] = acc[mt];
      acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    // real row r of tile mt = operand row r (hi) + operand row r + 8 (lo)
    for (int idx = threadIdx.x; idx < MT * 128; idx += nw * 64) {
      const int mt = idx >> 7, r = (idx >> 4) & 7, c = idx & 15;
      const int lh = (r >> 2) * 16 + c, ll = ((r + 8) >> 2) * 16 + c, e = r & 3;
      float v = 0.f;
      for (int w = 0; w < nw; ++w)
        v += red[((size_t)w * MT + mt) * 64 + lh][e] + red[((size_t)w * MT + mt) * 64 + ll][e];
      outv[(mt * 8 + r) * 17 + c] = v;
    }
    __syncthreads();
    epilogue<EPI>(a, item / a.ksplit, item % a.ksplit, rows, outv, t2);
  };

  for (int bi = 0; bi < total;) {
    if (bi + 1 < total) {
      const int it = item_of(bi + 1);
      p1 = (it != it0) ? wptr<INT4, EPI>(a, it / a.ksplit) : p0;
      it1 = it;
      const int ks = it % a.ksplit;
      load_stage<INT4, MT, U>(s1, p1, ap, K8, u_of(bi + 1, ks), ks * ks_units + w0, ks * ks_units + w1, mtv);
    }
    {
      const int ks = it0 % a.ksplit;
      compute_stage<MT, INT4, U>(s0, ap, asp, K8, KG, u_of(bi, ks), ks * ks_units + w0, ks * ks_units + w1, mtv, acc);
    }
    if (bi % nb == nb - 1) finish_item(it0);
    if (++bi >= total) break;
    if (bi + 1 < total) {
      const int it = item_of(bi + 1);
      p0 = (it != it1) ? wptr<INT4, EPI>(a, it / a.ksplit) : p1;
      it0 = it;
      const int ks = it % a.ksplit;
      load_stage<INT4, MT, U>(s0, p0, ap, K8, u_of(bi + 1, ks), ks * ks_units + w0, ks * ks_units + w1, mtv);
    }
    {
      const int ks = it1 % a.ksplit;
      compute_stage<MT, INT4, U>(s1, ap, asp, K8, KG, u_of(bi, ks), ks * ks_units + w0, ks * ks_units + w1, mtv, acc);
    }
    if (bi % nb == nb - 1) finish_item(it1);
    ++bi;
  }
  if (EPI == EPI_ARGMAX && (int)threadIdx.x < rows) {
    float* o = a.amax + ((size_t)(a.m_base + threadIdx.x) * a.n_parts + blockIdx.x) * 3;
    o[0] = t2.v1;
    o[1] = __int_as_float(t2.i1);
    o[2] = t2.v2;
  }
}

// ---------------------------------------------------------------- packing kernel

// One workgroup per operand row: v = x + sum of partial sums (fixed order),
// optionally written back, then RMSNorm (optional) and the bf16 hi/lo split into
// the packed layout (plus per-group sums for INT4 consumers).
__global__ __launch_bounds__(256) void k_pack(PackArgs a) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int K8 = a.K >> 3;
  const int KG = a.K >> 7;
  if (m >= a.M) {
    if (a.apack)
      for (int kc = threadIdx.x; kc < K8; kc += 256) apack_store_zero_chunk(a.apack, a.K, m, kc);
    if (a.int4 && a.asum) {
      for (int gi = threadIdx.x; gi < KG; gi += 256) {
        float* as = a.asum + ((size_t)(m >> 3) * KG + gi) * 16;
        as[m & 7] = 0.f;
        as[(m & 7) + 8] = 0.f;
      }
    }
    return;
  }
  // every thread keeps its chunks in registers: K <= 256 * 8 * 8
  constexpr int MAXC = 8;
  float v[MAXC][8];
  const float* x = a.x + (size_t)m * a.ldx;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int kc = threadIdx.x + j * 256;
    if (kc < K8) {
      const float4 v0 = *(const float4*)(x + kc * 8), v1 = *(const float4*)(x + kc * 8 + 4);
      v[j][0] = v0.x; v[j][1] = v0.y; v[j][2] = v0.z; v[j][3] = v0.w;
      v[j][4] = v1.x; v[j][5] = v1.y; v[j][6] = v1.z; v[j][7] = v1.w;
      for (int s = 0; s < a.n_parts; ++s) {
        const float* pp = a.parts + ((size_t)s * a.M + m) * a.K + kc * 8;
        const float4 p0 = *(const float4*)pp, p1 = *(const float4*)(pp + 4);
        v[j][0] += p0.x; v[j][1] += p0.y; v[j][2] += p0.z; v[j][3] += p0.w;
        v[j][4] += p1.x; v[j][5] += p1.y; v[j][6] += p1.z; v[j][7] += p1.w;
      }
      if (a.h_out) {
        float* ho = a.h_out + (size_t)m * a.ldx + kc * 8;
        *(float4*)ho = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
        *(float4*)(ho + 4) = make_float4(v[j][4], v[j][5], v[j][6], v[j][7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    }
  }
  if (!a.apack) return;
  float inv = 1.0f;
  if (a.gain) {
    ss = warp_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
  }
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int kc = threadIdx.x + j * 256;
    float hs = 0.f, ls = 0.f;
    if (kc < K8) {
      if (a.gain) {
        const uint4 gg = *(const uint4*)(a.gain + kc * 8);
        const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = v[j][e] * inv * bf16_to_f32((gw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
      }
      apack_store_chunk(a.apack, a.K, m, kc, v[j], a.int4);
      if (a.int4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t h, l;
          split_hi_lo(v[j][e], h, l);
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

// ---------------------------------------------------------------- weight packing

// One thread per 16-byte entry of the tiled layout; rows past n read as zero.
__global__ __launch_bounds__(256) void k_pack_weight(la_weight src, int layout, uint8_t* dst,
                                                     uint16_t* dst_scales, size_t entries) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= entries) return;
  const int lane = (int)(e & 63), c = lane & 15, g = lane >> 4;
  const bool int4 = src.fmt == LA_W_INT4;
  const int UT = int4 ? src.k / 128 : src.k / 32;
  const size_t tu = e >> 6;
  const int t = (int)(tu / UT), u = (int)(tu % UT);
  const int row = layout_row(layout, src.n, t, c);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < src.n) {
    const size_t off = int4 ? (size_t)row * (src.k / 2) + (size_t)u * 64 + g * 16
                            : ((size_t)row * src.k + (size_t)u * 32 + g * 8) * 2;
    v = *(const u32x4*)((const uint8_t*)src.data + off);
  }
  *(u32x4*)(dst + e * 16) = v;
  if (int4 && g == 0) {
    const uint16_t sv = row < src.n ? ((const uint16_t*)src.scales)[(size_t)row * (src.k / 128) + u] : (uint16_t)0;
    dst_scales[tu * 16 + c] = sv;
  }
}

hipError_t launch_pack_weight(const la_weight& src, int layout, void* dst, void* dst_scales,
                              hipStream_t s) {
  const int n_tiles = layout == LA_LAYOUT_TILED_GU ? (src.n / 2 + 7) / 8 : (src.n + 15) / 16;
  const int UT = src.fmt == LA_W_INT4 ? src.k / 128 : src.k / 32;
  const size_t entries = (size_t)n_tiles * UT * 64;
  hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, src,
                     layout, (uint8_t*)dst, (uint16_t*)dst_scales, entries);
  return hipGetLastError();
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

static int cu_count() {
  static int n = 0;
  if (!n) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

static size_t gemm_smem(int nw, int mt) {
  return (size_t)nw * mt * 64 * 16 + (size_t)mt * 8 * 17 * 4;
}

GemmPlan plan_gemm(int M, int N, int K, bool int4, int epi, bool allow_split) {
  GemmPlan p;
  p.n_tiles = (epi == EPI_SILU) ? (N / 2) / 8 : (N + 15) / 16;
  const int rows = M < kRowsPerLaunch ? M : kRowsPerLaunch;
  const int mt = (rows + 7) / 8;
  p.mt = mt <= 1 ? 1 : mt <= 2 ? 2 : 4;
  p.launches = (M + kRowsPerLaunch - 1) / kRowsPerLaunch;
  p.nw = 8;
  const int units = int4 ? K / 128 : K / 32;
  const int cus = cu_count();
  // K slices so that narrow GEMMs still cover every compute unit; a slice keeps
  // at least 4 units per wave and the slices divide K evenly
  p.ksplit = 1;
  if (allow_split && epi == EPI_STORE) {
    while (p.n_tiles * p.ksplit < cus && units % (p.ksplit * 2) == 0 &&
           units / (p.ksplit * 2) >= 4 * p.nw)
      p.ksplit *= 2;
  }
  // one 8-wave workgroup per compute unit; the items are dealt out evenly
  const int items = p.n_tiles * p.ksplit;
  const int per = (items + cus - 1) / cus;
  p.grid = (items + per - 1) / per;
  p.smem = gemm_smem(p.nw, p.mt);
  return p;
}

template <int MT, bool INT4, int EPI>
static hipError_t launch_one(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm<MT, INT4, EPI>), dim3(p.grid), dim3(p.nw * 64), p.smem, s, a);
  return hipGetLastError();
}

template <int MT, bool INT4>
static hipError_t launch_gemm_mt(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_one<MT, INT4, EPI_STORE>(a, p, s);
    case EPI_SILU: return launch_one<MT, INT4, EPI_SILU>(a, p, s);
    case EPI_QKV: return launch_one<MT, INT4, EPI_QKV>(a, p, s);
    default: return launch_one<MT, INT4, EPI_ARGMAX>(a, p, s);
  }
}

template <bool INT4>
static hipError_t launch_gemm_fmt(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  switch (p.mt) {
    case 1: return launch_gemm_mt<1, INT4>(a, epi, p, s);
    case 2: return launch_gemm_mt<2, INT4>(a, epi, p, s);
    default: return launch_gemm_mt<4, INT4>(a, epi, p, s);
  }
}

hipError_t launch_gemm(GemmArgs a, int epi, bool int4, hipStream_t s) {
  const GemmPlan p = plan_gemm(a.M, a.N, a.K, int4, epi, a.partial != nullptr);
  a.n_tiles = p.n_tiles;
  a.ksplit = p.ksplit;
  a.nw = p.nw;
  a.n_parts = p.grid;
  for (int l = 0; l < p.launches; ++l) {
    a.m_base = l * kRowsPerLaunch;
    const int rows = (a.M - a.m_base) < kRowsPerLaunch ? (a.M - a.m_base) : kRowsPerLaunch;
    const int mt8 = (rows + 7) / 8;
    GemmPlan pl = p;
    pl.mt = mt8 <= 1 ? 1 : mt8 <= 2 ? 2 : 4;
    pl.smem = gemm_smem(pl.nw, pl.mt);
    hipError_t e = int4 ? launch_gemm_fmt<true>(a, epi, pl, s) : launch_gemm_fmt<false>(a, epi, pl, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  // every operand row of the last tile is written (rows >= M become zero)
  const int rows = a.apack ? ((a.M + 7) / 8) * 8 : a.M;
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
