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
// rows) and one slice of K; workgroup b takes slice b % ksplit and every
// (gridDim.x / ksplit)-th tile, and its loading waves split the slice, then
// combine their partial sums through LDS; one more wave per workgroup runs the
// epilogues.  No workgroup ever waits for another: a device-wide fence costs
// more than a kernel boundary on this chip, so a K-sliced GEMM writes partial
// sums that the next kernel adds up.  A loading wave's weight loads form one
// stream across its work items with up to 7 stages in flight; the loads are
// raw buffer loads whose masked units carry an out-of-range offset (they read
// zero and touch no memory), so no branch ever splits the stream and the
// loading waves never store to global memory: the compiler counts the loads
// in flight exactly and never drains the ring.
#include "la_gemm_common.hpp"

#include <string.h>

namespace la {

// Rows per GEMM launch: four 8-row tiles keep the accumulators and the operand
// fragments of a wave in registers.
constexpr int kRowsPerLaunch = 32;

// Activation pieces (16 bytes) per thread of the one-batch LDS copy, and the
// INT4 group sums per thread.
__host__ __device__ constexpr int copy_batch(int mt) { return mt == 1 ? 12 : 16; }
constexpr int kCopySums = 2;

// LDS of the cross-wave reduction: [nw][MT][64] f32x4 partial tiles plus the
// [MT*8][17] output tile, rounded up to 16 bytes.
__host__ __device__ constexpr size_t gemm_red_bytes(int nw, int mt) {
  return ((size_t)nw * mt * 64 * 16 + (size_t)mt * 8 * 17 * 4 + 15) / 16 * 16;
}

// ---------------------------------------------------------------- stages

// Kernel modes, chosen by the host per GEMM:
//   single: every wave has exactly one stage; its activations are loaded with
//           its weights (QKV and O projections at small M)
//   ring:   a 2-deep ring, activations loaded with every stage (4 row tiles)
//   lds:    the workgroup's activation slice is copied to LDS once and a deep
//           ring of weight-only stages streams through it (gate/up, down,
//           lm_head)
// Every load instruction costs address-unit time even when it fetches
// nothing, so the modes avoid loads that carry no data.
constexpr int kModeSingle = 0;
constexpr int kModeRing = 1;
constexpr int kModeLds = 2;

// Chunks of 8 reduction elements per unit (a unit is 32 bf16 or 128 INT4 k).
template <bool INT4>
__host__ __device__ constexpr int unit_chunks() { return INT4 ? 16 : 4; }

// Units per stage and stages in the ring.
// The lds mode streams bf16 weights in stages of 4 units (4 KB per wave) with
// two stages in flight: measured at batch 1, gate/up 18.2 us and down 11.6 us
// against 20.2 and 13.1 with 8-unit stages three deep, and 18-20 us / 12-14 us
// for the other depths and sizes tried; more bytes in flight per compute unit
// make the weight stream slower, not faster.
template <bool INT4, int MT, int MODE>
__host__ __device__ constexpr int stage_units() {
  return INT4 ? 2 : (MODE == kModeRing ? (MT == 4 ? 2 : 4) : MODE == kModeLds ? 4 : 8);
}
template <bool INT4, int MT, int MODE>
__host__ __device__ constexpr int ring_depth() {
  return MODE == kModeSingle ? 1
         : MODE == kModeRing ? ((MT == 1 && !INT4) ? 4 : 2)
                             : (INT4 ? 8 : 3);
}
// Activation fragments travel in the stage (else: LDS, or for INT4 in the
// 2-deep ring, global loads at multiply time).
template <bool INT4, int MODE>
__host__ __device__ constexpr bool a_in_stage() {
  return MODE == kModeSingle || (MODE == kModeRing && !INT4);
}

// One pipeline stage for one lane: U units of the lane's weight column, their
// INT4 scales and, when a_in_stage, the matching activation fragments (and
// INT4 group sums).
template <bool INT4, int MT, int U, bool AIN>
struct Stage {
  u32x4 w[U];
  uint16_t s[INT4 ? U : 1];  // fp16 bits, converted at multiply time
  bf16x8 af[AIN ? (INT4 ? 4 * U : U) : 1][MT];
  f32x4 as[(AIN && INT4) ? U : 1][MT];
};

// Where a stage reads its activations when they are not in the stage: the
// workgroup's LDS copy of the K slice (chunk index relative to the slice start)
// or the packed rows in global memory.
struct ASrc {
  const uint16_t* p;    // lane base (row l%16 folded in)
  const float* s;       // INT4 group sums, lane base (4 (l/16) folded in)
  int tstride;          // elements between row tiles
  int sts;              // group-sum floats between row tiles
  int c0;               // chunk index of the slice start (0 for global)
  int u0;               // unit index of the slice start (0 for global)
  int mtv;              // valid row tiles
};

__device__ __forceinline__ bf16x8 a_frag(const ASrc& A, int mt, int kc) {
  return *(const bf16x8*)(A.p + (size_t)min(mt, A.mtv - 1) * A.tstride + (size_t)(kc - A.c0) * 128);
}
__device__ __forceinline__ f32x4 a_sums(const ASrc& A, int mt, int uu) {
  return *(const f32x4*)(A.s + (size_t)min(mt, A.mtv - 1) * A.sts + (size_t)(uu - A.u0) * 16);
}

// Loads are branch-free: a unit past the wave's range (or a stage past the
// end) reads zero weights and a zero scale; its activation loads repeat the
// wave's last unit.
template <bool INT4, int MT, int U, bool AIN>
__device__ __forceinline__ void load_stage(Stage<INT4, MT, U, AIN>& b, const WPtr& wp,
                                           __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rs,
                                           const ASrc& G, int u, int ulo, int uhi) {
  const int g = (threadIdx.x & 63) >> 4;
  const int ulast = uhi > ulo ? uhi - 1 : ulo;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    // a masked unit gets bit 31 set (offsets of real units stay below 2^31):
    // arithmetic, not a select, so that no branch ever splits the stream
    const uint32_t dead = (uint32_t)(u + i >= uhi) << 31;  // wave-uniform
    const int uu = min(u + i, ulast);
    b.w[i] = bload16<kNonTemporal>(rw, (wp.w + (uint32_t)uu * wp.ustride) | dead);
    if (INT4) {
      const uint32_t so = (wp.s + (uint32_t)uu * wp.sstride) | dead;
      b.s[INT4 ? i : 0] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
    }
    if (AIN) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (INT4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) b.af[AIN ? (INT4 ? 4 * i + j : i) : 0][mt] = a_frag(G, mt, uu * 16 + g * 4 + j);
          b.as[(AIN && INT4) ? i : 0][mt] = a_sums(G, mt, uu);
        } else {
          b.af[AIN ? i : 0][mt] = a_frag(G, mt, uu * 4 + g);
        }
      }
    }
  }
}

template <int MT, bool INT4, int U, bool AIN>
__device__ __forceinline__ void compute_stage(const Stage<INT4, MT, U, AIN>& b, const ASrc& A,
                                              int u, int ulo, int uhi, f32x4 (&acc)[MT], uint32_t i4bias) {
  const int g = (threadIdx.x & 63) >> 4;
  const int ulast = uhi > ulo ? uhi - 1 : ulo;
  if (!INT4) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, b.w[i]);  // zero for a masked unit
      const int uu = min(u + i, ulast);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 af = AIN ? b.af[AIN ? i : 0][mt] : a_frag(A, mt, uu * 4 + g);
        acc[mt] = mfma_16x16x32(af, bv, acc[mt]);
      }
    }
  } else {
    // Every 4-byte word expands (int4_to_bf16x8) into four bf16 pairs holding
    // 128 + q (k0 k4 | k1 k5 | k2 k6 | k3 k7), the order the packed activations
    // use.  Per group: acc += scale * (sum - 136 * sum_k a_k), since
    // sum a_k (128 + q_k) - 136 sum a_k = sum a_k (q_k - 8).
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const float sc = fp16_to_f32(b.s[INT4 ? i : 0]);  // zero for a masked unit
      const int uu = min(u + i, ulast);
      f32x4 t[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) t[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, int4_to_bf16x8(b.w[i][j], i4bias));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 af = AIN ? b.af[AIN ? (INT4 ? 4 * i + j : i) : 0][mt] : a_frag(A, mt, uu * 16 + g * 4 + j);
          t[mt] = mfma_16x16x32(af, bv, t[mt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 as = AIN ? b.as[(AIN && INT4) ? i : 0][mt] : a_sums(A, mt, uu);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][e] += sc * (t[mt][e] - 136.0f * as[e]);
      }
    }
  }
}

// ---------------------------------------------------------------- epilogues

// The epilogue wave's operands, loaded before it waits for a work item: per
// lane and iteration (idx = lane + 64 * it) two values, and per row (lane =
// row) where its K/V goes.
constexpr int kEpiIters = kRowsPerLaunch * 16 / 64;
struct EpiPre {
  float p0[kEpiIters], p1[kEpiIters], p2[kEpiIters];
  float2 cs[kEpiIters];
  float inv[kRowsPerLaunch / 8];  // 1/rms of rows 8 rb + (lane >> 3)
  int blk;       // QKV: page of the row's cache position (-1: no write)
  int slot;      // QKV: slot within the page
};

// Per-row cache location (QKV): row m writes position prefix_len[b] + j of
// sequence b unless it is flagged or the position has no valid page.
__device__ __forceinline__ void epi_rows(const GemmArgs& a, int rows, EpiPre& e) {
  const int lane = threadIdx.x & 63;
  e.blk = -1;
  e.slot = 0;
  if (lane >= rows) return;
  const int m = a.m_base + lane;
  const int b = m / a.W, j = m - b * a.W;
  const int pos = a.prefix_len[b] + j;
  const int f = a.flags ? a.flags[m] : 0;
  if (f != 0 || pos < 0 || pos >= a.max_blocks * kBlock) return;
  const int blk = a.block_table[(size_t)b * a.max_blocks + pos / kBlock];
  if (blk < 0 || blk >= a.num_blocks) return;
  e.blk = blk;
  e.slot = pos % kBlock;
}

// 1/rms of the launch's rows from the producer's per-tile sums of squares:
// lane l sums tiles (l & 7), (l & 7) + 8, ... of row 8 rb + (l >> 3), then the
// 8 lanes of a row combine in a fixed butterfly.
__device__ __forceinline__ void epi_inv(const GemmArgs& a, int rows, EpiPre& e) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < kRowsPerLaunch / 8; ++rb) e.inv[rb] = 1.f;
  if (!a.ss_in) return;
#pragma unroll
  for (int rb = 0; rb < kRowsPerLaunch / 8; ++rb) {
    if (rb * 8 >= rows) break;  // uniform
    const int row = min(rb * 8 + (lane >> 3), rows - 1);
    const float* src = a.ss_in + (size_t)(a.m_base + row) * a.ss_tiles;
    // 16 loads at a time, all in flight together (128 tiles: one batch)
    float sum = 0.f;
    for (int t0 = 0; t0 < a.ss_tiles; t0 += 128) {
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int t = t0 + (lane & 7) + 8 * k;
        v[k] = src[min(t, a.ss_tiles - 1)];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (t0 + (lane & 7) + 8 * k < a.ss_tiles) sum += v[k];
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    e.inv[rb] = 1.0f / sqrtf(sum / (float)a.K + a.eps);
  }
}

// 1/rms of row ml (any lane may ask for any row < 32).
__device__ __forceinline__ float row_inv(const EpiPre& e, int ml) {
  float iv = 1.f;
#pragma unroll
  for (int rb = 0; rb < kRowsPerLaunch / 8; ++rb) {
    const float t = __shfl(e.inv[rb], (ml & 7) * 8);
    if ((ml >> 3) == rb) iv = t;
  }
  return iv;
}

template <int EPI>
__device__ __forceinline__ void epi_prefetch(const GemmArgs& a, int tile, int rows, EpiPre& e) {
  const int lane = threadIdx.x & 63;
  if (EPI == EPI_STORE) {
    if (a.ksplit > 1) return;
#pragma unroll
    for (int it = 0; it < kEpiIters; ++it) {
      const int idx = lane + it * 64;
      const int ml = min(idx >> 4, rows - 1), c = idx & 15;
      const int n = min(tile * 16 + c, a.N - 1);
      e.p0[it] = a.residual ? a.residual[(size_t)(a.m_base + ml) * a.ldy + n] : 0.f;
      e.p1[it] = a.bias ? bf16_to_f32(a.bias[n]) : 0.f;
      e.p2[it] = a.out_gain ? bf16_to_f32(a.out_gain[n]) : 0.f;
    }
  } else if (EPI == EPI_QKV) {
    const int head = tile >> 3, sub = tile & 7;
#pragma unroll
    for (int it = 0; it < kEpiIters / 2; ++it) {
      const int idx = lane + it * 64;
      const int ml = min(idx >> 3, rows - 1), c = idx & 7;
      const int i = sub * 8 + c;
      const int r1 = head * kHeadDim + i, r2 = r1 + 64;
      e.cs[it] = a.rope[(size_t)(a.m_base + ml) * 64 + i];
      e.p0[it] = a.bias ? bf16_to_f32(a.bias[r1]) : 0.f;
      e.p1[it] = a.bias ? bf16_to_f32(a.bias[r2]) : 0.f;
    }
  }
}

// outv[row * 17 + c]: operand column c of output row m_base + row; run by the
// workgroup's epilogue wave with the operands it prefetched.
template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int tile, int ks, int rows,
                                         const float* outv, const EpiPre& e, Top2& t2) {
  const int lane = threadIdx.x & 63;
  if (EPI == EPI_STORE) {
#pragma unroll
    for (int it = 0; it < kEpiIters; ++it) {
      const int idx = lane + it * 64;
      const int ml = idx >> 4, c = idx & 15;
      const int m = a.m_base + ml;
      const int n = tile * 16 + c;
      const bool ok = ml < rows && n < a.N;
      float v = ok ? outv[ml * 17 + c] : 0.f;
      if (a.ksplit > 1) {
        if (ok) a.partial[((size_t)ks * a.M + m) * a.N + n] = v;
        continue;
      }
      v = v + e.p1[it] + e.p0[it];
      if (ok) a.y[(size_t)m * a.ldy + n] = v;
      if (a.ss_out) {
        // this tile's share of the row's sum of squares (16 lanes, fixed order)
        float q = ok ? v * v : 0.f;
        q += __shfl_xor(q, 1);
        q += __shfl_xor(q, 2);
        q += __shfl_xor(q, 4);
        q += __shfl_xor(q, 8);
        if (ml < rows && c == 0) a.ss_out[(size_t)m * a.n_tiles + tile] = q;
      }
      if (a.y_apack && ok) {
        // y * gain as bf16 hi/lo into the next GEMM's packed operand (K = N)
        uint32_t h, l;
        split_hi_lo(v * e.p2[it], h, l);
        const size_t base = (((size_t)(m >> 3) * (a.N / 8) + (n >> 3)) * 16 + (m & 7)) * 8 + (n & 7);
        a.y_apack[base] = (uint16_t)h;
        a.y_apack[base + 64] = (uint16_t)l;
      }
    }
  } else if (EPI == EPI_SILU) {
    const int F = a.N / 2;
#pragma unroll
    for (int it = 0; it < kEpiIters / 2; ++it) {
      const int idx = lane + it * 64;
      const int ml = idx >> 3, c = idx & 7;
      const float iv = row_inv(e, ml);
      if (ml >= rows) continue;
      const int m = a.m_base + ml;
      const float* o = outv + ml * 17;
      const float v = silu_f(o[c] * iv) * (o[c + 8] * iv);
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
#pragma unroll
    for (int it = 0; it < kEpiIters / 2; ++it) {
      const int idx = lane + it * 64;
      const int ml = idx >> 3, c = idx & 7;
      // the row's cache location lives in lane ml
      const int blk = __shfl(e.blk, ml & 63), slot = __shfl(e.slot, ml & 63);
      const float iv = row_inv(e, ml);
      if (ml >= rows) continue;
      const int m = a.m_base + ml;
      const int i = sub * 8 + c;  // rotary pair index
      const int r1 = head * kHeadDim + i, r2 = r1 + 64;
      const float* o = outv + ml * 17;
      float x1 = o[c] * iv + e.p0[it], x2 = o[c + 8] * iv + e.p1[it];
      if (head < Hq + Hkv) {
        const float2 cs = e.cs[it];
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
      if (blk < 0) continue;
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
    if (lane < rows) {
      // the tile's 16 bits of this row's bitmap (repetition penalty)
      const uint32_t used = rep_word(a, a.m_base + lane, tile * 16) >> ((tile * 16) & 31);
      for (int c = 0; c < 16; ++c) {
        const int n = tile * 16 + c;
        if (n >= a.N) break;
        float v = outv[lane * 17 + c];
        if ((used >> c) & 1u) v = rep_penalise(v, a.rep_theta);
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

// Workgroup b takes K slice b % ksplit and the column tiles b / ksplit,
// b / ksplit + gridDim.x / ksplit, ...; its nw loading waves split the slice
// and one more wave runs the epilogues.  A loading wave's stages run through
// its tiles in order, ring_depth - 1 of them in flight while one is
// multiplied; it never stores to global memory, so the compiler can count its
// loads in flight exactly and never has to drain the ring.
template <int MT, bool INT4, int EPI, int MODE>
__global__ __launch_bounds__(576) __attribute__((amdgpu_waves_per_eu(1, 3)))
void k_gemm(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr bool ALDS = MODE == kModeLds;
  constexpr bool AIN = a_in_stage<INT4, MODE>();
  constexpr int U = stage_units<INT4, MT, MODE>();
  constexpr int D = ring_depth<INT4, MT, MODE>();
  constexpr int CPU = unit_chunks<INT4>();
  constexpr int CB = copy_batch(MT);
  // the wave index is made provably uniform: segment bounds live in scalar
  // registers and every branch on them is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nw = a.nw, nthr = nw * 64;
  const int K8 = a.K >> 3, KG = a.K >> 7;
  const int units = INT4 ? (a.K >> 7) : (a.K >> 5);
  const int ks = (int)blockIdx.x % a.ksplit;
  const int tb = (int)blockIdx.x / a.ksplit, gt = (int)gridDim.x / a.ksplit;
  const int s_lo = units * ks / a.ksplit, s_hi = units * (ks + 1) / a.ksplit;
  const int s_len = s_hi - s_lo;
  const int nb = ((s_len + nw - 1) / nw + U - 1) / U;  // same stage count for every wave
  const int n_my = (a.n_tiles - tb + gt - 1) / gt;
  const int total = n_my * nb;
  if (total <= 0) return;  // uniform over the workgroup
  const int rows = min(min(kRowsPerLaunch, a.M - a.m_base), MT * 8);
  const int mtv = (rows + 7) >> 3;

  f32x4* red = (f32x4*)smem;                                    // [nw][MT][64]
  float* outv = (float*)(smem + (size_t)nw * MT * 64 * 16);     // [MT*8][17]
  uint16_t* lds_a = (uint16_t*)(smem + gemm_red_bytes(nw, MT)); // [MT][s_len*CPU][16][8]
  float* lds_s = (float*)(lds_a + (size_t)MT * s_len * CPU * 128);  // [MT][s_len][16]

  if (wave == nw) {
    // the epilogue wave: the same barriers as the loading waves (the LDS
    // copy, then two per work item), an epilogue after each item
    EpiPre e;
    if (EPI == EPI_QKV) epi_rows(a, rows, e);
    if (EPI != EPI_STORE) epi_inv(a, rows, e);
    if (ALDS) __syncthreads();
    Top2 t2 = {-INFINITY, -INFINITY, 0x7FFFFFFF};
    for (int it = 0; it < n_my; ++it) {
      epi_prefetch<EPI>(a, tb + it * gt, rows, e);  // in flight during the item
      __syncthreads();
      __syncthreads();
      epilogue<EPI>(a, tb + it * gt, ks, rows, outv, e, t2);
    }
    if (EPI == EPI_ARGMAX) {
      // the row scale is positive: it changes no ranking, only the values
      const float iv = row_inv(e, lane);
      if (lane < rows) {
        float* o = a.amax + ((size_t)(a.m_base + lane) * a.n_parts + blockIdx.x) * 3;
        o[0] = t2.v1 * iv;
        o[1] = __int_as_float(t2.i1);
        o[2] = t2.v2 * iv;
      }
    }
    return;
  }

  const int ulo = s_lo + s_len * wave / nw, uhi = s_lo + s_len * (wave + 1) / nw;

  // activations in global memory (for the stage loads) and where the multiply
  // reads them when they are not in the stage
  ASrc G;
  G.p = a.apack + (size_t)(a.m_base >> 3) * K8 * 128 + (lane & 15) * 8;
  G.s = a.asum ? a.asum + (size_t)(a.m_base >> 3) * KG * 16 + 4 * (lane >> 4) : nullptr;
  G.tstride = K8 * 128;
  G.sts = KG * 16;
  G.c0 = 0;
  G.u0 = 0;
  G.mtv = mtv;
  ASrc A = G;
  if (ALDS) {
    A.p = lds_a + (lane & 15) * 8;
    A.s = lds_s + 4 * (lane >> 4);
    A.tstride = s_len * CPU * 128;
    A.sts = s_len * 16;
    A.c0 = s_lo * CPU;
    A.u0 = s_lo;
  }

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(INT4 ? (const void*)a.wscale : a.w, INT4 ? a.s_bytes : 0u);

  // lds mode: copy this slice of the packed rows (and INT4 group sums) in one
  // batch of unconditional loads, issued before the weights so that storing
  // them waits for nothing else (the host guarantees the batch suffices)
  const int n16 = s_len * CPU * 16;  // 16-byte pieces per row tile
  u32x4 cbuf[ALDS ? CB : 1];
  float sbuf[ALDS && INT4 ? kCopySums : 1];
  if (ALDS) {
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(a.apack + (size_t)(a.m_base >> 3) * K8 * 128, (uint32_t)mtv * K8 * 256);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int p = i * nthr + (int)threadIdx.x;
      const int mt = p / n16, q = p - mt * n16;
      const uint32_t off = ((uint32_t)min(mt, mtv - 1) * K8 + (uint32_t)s_lo * CPU) * 256 + (uint32_t)q * 16;
      cbuf[i] = bload16<0>(ra, p < MT * n16 ? off : kOOB);
    }
    if (INT4) {
      const __amdgpu_buffer_rsrc_t rg =
          make_rsrc(a.asum + (size_t)(a.m_base >> 3) * KG * 16, (uint32_t)mtv * KG * 64);
      const int ns = s_len * 16;
#pragma unroll
      for (int i = 0; i < (ALDS && INT4 ? kCopySums : 1); ++i) {
        const int p = i * nthr + (int)threadIdx.x;
        const int mt = p / ns, q = p - mt * ns;
        const uint32_t off = (((uint32_t)min(mt, mtv - 1) * KG + s_lo) * 16 + q) * 4;
        sbuf[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, p < MT * ns ? off : kOOB, 0, 0));
      }
    }
  }

  auto tile_of = [&](int bi) { return tb + (bi / nb) * gt; };
  // stage bi's first unit; past the end it is uhi, so every unit is masked
  auto u_of = [&](int bi) { return bi < total ? ulo + (bi % nb) * U : uhi; };
  Stage<INT4, MT, U, AIN> st[D];
  auto issue = [&](int bi, Stage<INT4, MT, U, AIN>& s) {
    const WPtr wp = wptr<INT4, EPI>(a, tile_of(min(bi, total - 1)));
    load_stage<INT4, MT, U, AIN>(s, wp, rw, rs, G, u_of(bi), ulo, uhi);
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, st[j]);
  // every load of a stage goes out before the multiplies (with four row tiles
  // the registers do not allow it; the compiler interleaves instead)
  if (MT <= 2) __builtin_amdgcn_sched_barrier(0);

  if (ALDS) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int p = i * nthr + (int)threadIdx.x;
      if (p < MT * n16) *(u32x4*)(lds_a + (size_t)p * 8) = cbuf[i];
    }
    if (INT4) {
#pragma unroll
      for (int i = 0; i < (ALDS && INT4 ? kCopySums : 1); ++i) {
        const int p = i * nthr + (int)threadIdx.x;
        if (p < MT * s_len * 16) lds_s[p] = sbuf[i];
      }
    }
    __syncthreads();
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const uint32_t i4bias = INT4 ? int4_bias_reg() : 0u;

  // a work item's partial sums: through LDS to one output tile (outv), which
  // the epilogue wave takes after the second barrier
  auto finish_item = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      red[((size_t)wave * MT + mt) * 64 + lane] = acc[mt];
      acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    // real row r of tile mt = operand row r (hi) + operand row r + 8 (lo)
    for (int idx = threadIdx.x; idx < MT * 128; idx += nthr) {
      const int mt = idx >> 7, r = (idx >> 4) & 7, c = idx & 15;
      const int lh = (r >> 2) * 16 + c, ll = ((r + 8) >> 2) * 16 + c, e = r & 3;
      float v = 0.f;
      for (int w = 0; w < nw; ++w)
        v += red[((size_t)w * MT + mt) * 64 + lh][e] + red[((size_t)w * MT + mt) * 64 + ll][e];
      outv[(mt * 8 + r) * 17 + c] = v;
    }
    __syncthreads();
  };

  // the ring: stage bi is multiplied while stages bi+1 .. bi+D-1 are in
  // flight; past the last stage the loop is left at once (the loads issued
  // for stages past the end are masked and read nothing)
  for (int bi0 = 0;; bi0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int bi = bi0 + j;
      if (D > 1) issue(bi + D - 1, st[(j + D - 1) % D]);
      else issue(bi, st[0]);
      if (MT <= 2) __builtin_amdgcn_sched_barrier(0);
      compute_stage<MT, INT4, U, AIN>(st[j], A, u_of(bi), ulo, uhi, acc, i4bias);
      if (bi % nb == nb - 1) finish_item();
      if (bi + 1 >= total) return;  // uniform
    }
  }
}

// ---------------------------------------------------------------- packing kernel

// One workgroup per operand row: v = x + sum of NP partial sums (fixed order),
// optionally written back, then RMSNorm (optional) and the bf16 hi/lo split into
// the packed layout (plus per-group sums for INT4 consumers).  A thread holds C
// chunks of 8 values; every load of the row (x, partial sums, gain) is issued
// before the first is used, so the kernel waits on memory once.  Without the
// norm (no row-wide sum) a row may be split over gridDim.y workgroups, each
// taking blockDim.x * C consecutive chunks (a multiple of 16: whole groups).
template <int NP, int C>
__global__ __launch_bounds__(1024) void k_pack(PackArgs a) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int K8 = a.K >> 3;
  const int KG = a.K >> 7;
  const int bd = blockDim.x;
  const int k0 = (int)blockIdx.y * bd * C;  // first chunk of this workgroup's part of the row
  const int k1 = min(K8, k0 + bd * C);
  if (m >= a.M) {
    // padding rows of the last tile: zero operand rows and group sums
    if (a.apack)
      for (int kc = k0 + (int)threadIdx.x; kc < k1; kc += bd) apack_store_zero_chunk(a.apack, a.K, m, kc);
    if (a.int4 && a.asum) {
      for (int gi = k0 / 16 + (int)threadIdx.x; gi < min(KG, (k1 + 15) / 16); gi += bd) {
        float* as = a.asum + ((size_t)(m >> 3) * KG + gi) * 16;
        as[m & 7] = 0.f;
        as[(m & 7) + 8] = 0.f;
      }
    }
    return;
  }
  float v[C][8];
  uint4 gg[C];
  const float* x = a.x + (size_t)m * a.ldx;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int kc = min(k0 + (int)threadIdx.x + j * bd, K8 - 1);  // clamped; masked below
    float4 p[2 * NP + 2];
    p[0] = *(const float4*)(x + kc * 8);
    p[1] = *(const float4*)(x + kc * 8 + 4);
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      // NP bounds the count; slices past a.n_parts read the last one and
      // add it times zero (no branch, so every load is in flight at once)
      const float* pp = a.parts + ((size_t)min(s, a.n_parts - 1) * a.M + m) * a.K + kc * 8;
      const float on = s < a.n_parts ? 1.f : 0.f;
      const float4 q0 = *(const float4*)pp, q1 = *(const float4*)(pp + 4);
      p[2 * s + 2] = make_float4(q0.x * on, q0.y * on, q0.z * on, q0.w * on);
      p[2 * s + 3] = make_float4(q1.x * on, q1.y * on, q1.z * on, q1.w * on);
    }
    if (a.gain) gg[j] = *(const uint4*)(a.gain + kc * 8);
    // x first, then the partial sums in order
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float4 t = p[h];
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const float4 q = p[2 * s + 2 + h];
        t.x += q.x; t.y += q.y; t.z += q.z; t.w += q.w;
      }
      v[j][4 * h + 0] = t.x; v[j][4 * h + 1] = t.y; v[j][4 * h + 2] = t.z; v[j][4 * h + 3] = t.w;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int kc = k0 + (int)threadIdx.x + j * bd;
    if (kc < k1) {
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
    ss = 0.f;
    for (int w = 0; w < (bd >> 6); ++w) ss += red[w];  // fixed order
    inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int kc = k0 + (int)threadIdx.x + j * bd;
    float hs = 0.f, ls = 0.f;
    if (kc < k1) {
      if (a.gain) {
        const uint32_t gw[4] = {gg[j].x, gg[j].y, gg[j].z, gg[j].w};
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
      // 16 consecutive chunks (consecutive lanes) form one 128-wide group
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        hs += __shfl_xor(hs, o);
        ls += __shfl_xor(ls, o);
      }
      if (kc < k1 && (kc & 15) == 0) {
        float* as = a.asum + ((size_t)(m >> 3) * KG + (kc >> 4)) * 16;
        as[m & 7] = hs;
        as[(m & 7) + 8] = ls;
      }
    }
  }
}

// ---------------------------------------------------------------- w8a8

// w8a8 (the RK3588 conversion's format; read as int8 weight codes with one
// fp32 scale per output channel, int8 activations with one scale per row):
// the packed activations are int8 [M/16][K/64][64 lanes][16 bytes] (lane l:
// row l % 16, k = 64 u + 16 (l / 16) .. + 15) plus fp32 row scales (in the
// asum buffer); tiled weights are int8 [n_tiles][K/64][64 lanes][16 bytes]
// in the same lane order, so one 16-byte load per lane is one operand of
// v_mfma_i32_16x16x64_i8 on either side.
typedef __attribute__((ext_vector_type(4))) int i32x4;

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

constexpr int kW8Waves = 8;   // loading waves; one more runs the epilogues
constexpr int kW8Units = 4;   // K units of 64 per stage and wave

// One workgroup per row (rows M .. 16-padded become zero): v = x + the NP
// partial sums in order (optionally written back), RMSNorm with gain
// (optional), then s = max|v| / 127 and q = round-half-even(v / s) clamped to
// [-127, 127] (s = 0: q = 0), every decision in fp32.  A thread takes 16
// consecutive k.
template <int NP>
__global__ __launch_bounds__(1024) void k_pack_w8(PackArgs a) {
  __shared__ float red[16];
  const int m = blockIdx.x, t = threadIdx.x, nw = blockDim.x >> 6;
  const int K16 = a.K >> 4, U64 = a.K >> 6;
  const bool live = m < a.M && t < K16;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = 0.f;
  if (live) {
    const float* x = a.x + (size_t)m * a.ldx + t * 16;
    float4 p[4 * (NP + 1)];
#pragma unroll
    for (int h = 0; h < 4; ++h) p[h] = *(const float4*)(x + 4 * h);
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      const float* pp = a.parts + ((size_t)min(s, a.n_parts - 1) * a.M + m) * a.K + t * 16;
      const float on = s < a.n_parts ? 1.f : 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float4 q = *(const float4*)(pp + 4 * h);
        p[4 * s + 4 + h] = make_float4(q.x * on, q.y * on, q.z * on, q.w * on);
      }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float4 tt = p[h];
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const float4 q = p[4 * s + 4 + h];
        tt.x += q.x; tt.y += q.y; tt.z += q.z; tt.w += q.w;
      }
      v[4 * h] = tt.x; v[4 * h + 1] = tt.y; v[4 * h + 2] = tt.z; v[4 * h + 3] = tt.w;
    }
    if (a.h_out) {
      float* ho = a.h_out + (size_t)m * a.ldx + t * 16;
#pragma unroll
      for (int h = 0; h < 4; ++h) *(float4*)(ho + 4 * h) = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
    }
  }
  if (!a.apack) return;
  if (a.gain) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += v[e] * v[e];
    ss = warp_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    ss = 0.f;
    for (int w = 0; w < nw; ++w) ss += red[w];  // fixed order
    const float inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    __syncthreads();
    if (live) {
      const uint4 g0 = *(const uint4*)(a.gain + t * 16), g1 = *(const uint4*)(a.gain + t * 16 + 8);
      const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = v[e] * inv * bf16_to_f32((gw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(v[e]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = 0.f;
  for (int w = 0; w < nw; ++w) mx = fmaxf(mx, red[w]);
  const float sc = mx / 127.0f;
  if (t < K16) {
    uint32_t w4[4] = {0u, 0u, 0u, 0u};
    if (sc > 0.f) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float q = fminf(fmaxf(__builtin_rintf(v[e] / sc), -127.f), 127.f);
        w4[e >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (e & 3));
      }
    }
    const int u = t >> 2, g = t & 3;
    const size_t off = (((size_t)(m >> 4) * U64 + u) * 64 + g * 16 + (m & 15)) * 16;
    *(uint4*)((uint8_t*)a.apack + off) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  if (t == 0 && a.asum) a.asum[m] = sc;
}

// w8a8 GEMM for up to 16 MT rows per launch: work items are (column tile, K
// slice); 8 loading waves split a slice's 64-k units and stream stages of
// kW8Units units (their weight and activation fragments) D deep; int32 sums
// meet exactly in LDS, are scaled by the row's and the column's scale into the
// fp32 output tile, and the epilogue wave finishes the item with the same
// epilogues as the bf16 kernel (bias, RoPE and the K/V write, SiLU, residual,
// partial sums, running top-2).
template <int MT, int EPI>
__global__ __launch_bounds__((kW8Waves + 1) * 64) void k_gemm_w8(GemmArgs a) {
  constexpr int D = MT == 1 ? 3 : 2;
  __shared__ __align__(16) i32x4 red[kW8Waves * MT * 64];
  __shared__ float outv[MT * 16 * 17];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int units = a.K >> 6;
  const int ks = (int)blockIdx.x % a.ksplit;
  const int tb = (int)blockIdx.x / a.ksplit, gt = (int)gridDim.x / a.ksplit;
  const int s_lo = units * ks / a.ksplit, s_hi = units * (ks + 1) / a.ksplit;
  const int s_len = s_hi - s_lo;
  const int nb = ((s_len + kW8Waves - 1) / kW8Waves + kW8Units - 1) / kW8Units;  // stages per item
  const int n_my = (a.n_tiles - tb + gt - 1) / gt;
  const int total = n_my * nb;
  if (total <= 0) return;  // uniform over the workgroup
  const int rows = min(min(kRowsPerLaunch, a.M - a.m_base), MT * 16);
  const int mtv = (rows + 15) >> 4;

  if (wave == kW8Waves) {
    EpiPre e;
    if (EPI == EPI_QKV) epi_rows(a, rows, e);
    if (EPI != EPI_STORE) epi_inv(a, rows, e);
    Top2 t2 = {-INFINITY, -INFINITY, 0x7FFFFFFF};
    for (int it = 0; it < n_my; ++it) {
      epi_prefetch<EPI>(a, tb + it * gt, rows, e);
      __syncthreads();
      __syncthreads();
      epilogue<EPI>(a, tb + it * gt, ks, rows, outv, e, t2);
    }
    if (EPI == EPI_ARGMAX) {
      const float iv = row_inv(e, lane);
      if (lane < rows) {
        float* o = a.amax + ((size_t)(a.m_base + lane) * a.n_parts + blockIdx.x) * 3;
        o[0] = t2.v1 * iv;
        o[1] = __int_as_float(t2.i1);
        o[2] = t2.v2 * iv;
      }
    }
    return;
  }

  const int ulo = s_lo + s_len * wave / kW8Waves, uhi = s_lo + s_len * (wave + 1) / kW8Waves;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.apack, (uint32_t)((a.M + 15) >> 4) * units * 1024);
  const int mt0 = a.m_base >> 4;
  const float* sw = (const float*)a.wscale;

  struct St {
    u32x4 w[kW8Units];
    u32x4 x[kW8Units][MT];
  };
  auto tile_of = [&](int bi) { return tb + (bi / nb) * gt; };
  auto issue = [&](int bi, St& st) {
    const int tile = tile_of(min(bi, total - 1));
    const int u0 = ulo + (bi % nb) * kW8Units;
    uint32_t wrow = 0;
    if (a.layout == LA_LAYOUT_ROWS) wrow = (uint32_t)min(col_row<EPI>(a.N, tile, lane & 15), a.N - 1) * a.K + (lane >> 4) * 16;
#pragma unroll
    for (int j = 0; j < kW8Units; ++j) {
      const int u = u0 + j;
      const bool ok = bi < total && u < uhi;
      const uint32_t wo = a.layout == LA_LAYOUT_ROWS ? wrow + (uint32_t)u * 64
                                                     : (((uint32_t)tile * units + u) * 64 + lane) * 16;
      st.w[j] = bload16<kNonTemporal>(rw, ok ? wo : kOOB);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t xo = (((uint32_t)(mt0 + mt) * units + u) * 64 + lane) * 16;
        st.x[j][mt] = bload16<0>(ra, ok && mt < mtv ? xo : kOOB);
      }
    }
  };
  i32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (i32x4){0, 0, 0, 0};
  auto compute = [&](const St& st) {
#pragma unroll
    for (int j = 0; j < kW8Units; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_i8(st.x[j][mt], st.w[j], acc[mt]);
  };
  // an item's int32 sums: exact across the waves, then both scales
  auto finish_item = [&](int bi) {
    const int tile = tile_of(bi);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      red[(wave * MT + mt) * 64 + lane] = acc[mt];
      acc[mt] = (i32x4){0, 0, 0, 0};
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * 256; idx += kW8Waves * 64) {
      const int mt = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
      const int src = (r >> 2) * 16 + c, e = r & 3;
      int sum = 0;
      for (int w = 0; w < kW8Waves; ++w) sum += red[(w * MT + mt) * 64 + src][e];
      const int ml = mt * 16 + r;
      const float sa = ml < rows ? a.asum[a.m_base + ml] : 0.f;
      const float sc = sw[min(col_row<EPI>(a.N, tile, c), a.N - 1)];
      outv[ml * 17 + c] = (float)sum * sa * sc;
    }
    __syncthreads();
  };

  St st[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, st[j]);
  __builtin_amdgcn_sched_barrier(0);
  for (int bi0 = 0;; bi0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int bi = bi0 + j;
      issue(bi + D - 1, st[(j + D - 1) % D]);
      __builtin_amdgcn_sched_barrier(0);
      compute(st[j]);
      if (bi % nb == nb - 1) finish_item(bi);
      if (bi + 1 >= total) return;  // uniform
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
  const bool int4 = src.fmt == LA_W_INT4, w8 = src.fmt == LA_W_W8A8;
  const int UT = int4 ? src.k / 128 : w8 ? src.k / 64 : src.k / 32;
  const size_t tu = e >> 6;
  const int t = (int)(tu / UT), u = (int)(tu % UT);
  const int row = layout_row(layout, src.n, t, c);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < src.n) {
    const size_t off = int4 ? (size_t)row * (src.k / 2) + (size_t)u * 64 + g * 16
                       : w8 ? (size_t)row * src.k + (size_t)u * 64 + g * 16
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
  const int UT = src.fmt == LA_W_INT4 ? src.k / 128 : src.fmt == LA_W_W8A8 ? src.k / 64 : src.k / 32;
  const size_t entries = (size_t)n_tiles * UT * 64;
  if (src.fmt == LA_W_W8A8 && dst_scales) {
    // per-channel scales stay indexed by weight row
    const hipError_t e = hipMemcpyAsync(dst_scales, src.scales, (size_t)src.n * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, src,
                     layout, (uint8_t*)dst, (uint16_t*)dst_scales, entries);
  return hipGetLastError();
}

// ---------------------------------------------------------------- argmax reduce

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

int cu_count() {
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

// LDS of the activation slice (and INT4 group sums) of a K slice of `len` units.
static size_t gemm_alds_bytes(int mt, int len, bool int4) {
  return (size_t)mt * len * (int4 ? 16 : 4) * 256 + (int4 ? (size_t)mt * len * 64 : 0);
}

constexpr size_t kLdsBudget = 160 * 1024;

// The lds mode holds one or two row tiles, and its copy is one batch: at most
// copy_batch pieces (and kCopySums group sums) per thread.
static bool alds_fits(int mt, int len, bool int4, int nw) {
  const long pieces = (long)mt * len * (int4 ? 16 : 4) * 16;
  const long sums = int4 ? (long)mt * len * 16 : 0;
  return mt <= 2 && gemm_red_bytes(nw, mt) + gemm_alds_bytes(mt, len, int4) <= kLdsBudget &&
         pieces <= (long)copy_batch(mt) * nw * 64 && sums <= (long)kCopySums * nw * 64;
}

static int mode_units(bool int4, int mt, int mode) {
  if (int4) return stage_units<true, 1, kModeSingle>();
  if (mode != kModeRing) return stage_units<false, 1, kModeSingle>();
  return mt == 4 ? stage_units<false, 4, kModeRing>()
                 : mt == 2 ? stage_units<false, 2, kModeRing>() : stage_units<false, 1, kModeRing>();
}

// Mode, waves and shared memory of one launch with `mt` row tiles, given the
// column tiles, K slices and tiles per workgroup.
static void plan_launch(GemmPlan& p, int mt, int units, bool int4, int per) {
  p.mt = mt;
  const int len = (units + p.ksplit - 1) / p.ksplit;
  const int us = mode_units(int4, mt, kModeSingle);
  if (per == 1 && len <= 8 * us) {
    // one stage per wave: as many waves as the slice needs
    p.mode = kModeSingle;
    p.nw = (len + us - 1) / us;
  } else {
    p.nw = 8;
    p.mode = alds_fits(mt, len, int4, p.nw) ? kModeLds : kModeRing;
  }
  p.smem = gemm_red_bytes(p.nw, mt) + (p.mode == kModeLds ? gemm_alds_bytes(mt, len, int4) : 0);
}

GemmPlan plan_gemm(int M, int N, int K, bool int4, int epi, bool allow_split) {
  GemmPlan p;
  p.n_tiles = (epi == EPI_SILU) ? (N / 2) / 8 : (N + 15) / 16;
  const int rows = M < kRowsPerLaunch ? M : kRowsPerLaunch;
  const int mt8 = (rows + 7) / 8;
  const int mt = mt8 <= 1 ? 1 : mt8 <= 2 ? 2 : 4;
  p.launches = (M + kRowsPerLaunch - 1) / kRowsPerLaunch;
  const int units = int4 ? K / 128 : K / 32;
  const int cus = cu_count();
  // K slices (partial sums for the next kernel, EPI_STORE only) so that narrow
  // GEMMs still cover every compute unit and, for one or two row tiles, the
  // activation slice fits in LDS; every wave keeps at least one unit
  p.ksplit = 1;
  if (allow_split && epi == EPI_STORE) {
    while (p.ksplit < 16 &&
           (p.n_tiles * p.ksplit < cus ||
            (mt <= 2 && !alds_fits(mt, (units + p.ksplit - 1) / p.ksplit, int4, 8))) &&
           units / (p.ksplit * 2) >= 8)
      p.ksplit *= 2;
  }
  // workgroups per slice: the slice's tiles dealt out evenly over cus/ksplit
  const int per_slice = cus / p.ksplit > 0 ? cus / p.ksplit : 1;
  p.per = (p.n_tiles + per_slice - 1) / per_slice;
  const int gt = (p.n_tiles + p.per - 1) / p.per;
  p.grid = gt * p.ksplit;
  plan_launch(p, mt, units, int4, p.per);
  return p;
}

template <int MT, bool INT4, int EPI, int MODE>
static hipError_t launch_one(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
  static bool attr = false;  // allow the full LDS once per instantiation
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm<MT, INT4, EPI, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBudget);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm<MT, INT4, EPI, MODE>), dim3(p.grid), dim3(p.nw * 64 + 64), p.smem, s, a);
  return hipGetLastError();
}

template <int MT, bool INT4, int MODE>
static hipError_t launch_gemm_epi(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_one<MT, INT4, EPI_STORE, MODE>(a, p, s);
    case EPI_SILU: return launch_one<MT, INT4, EPI_SILU, MODE>(a, p, s);
    case EPI_QKV: return launch_one<MT, INT4, EPI_QKV, MODE>(a, p, s);
    default: return launch_one<MT, INT4, EPI_ARGMAX, MODE>(a, p, s);
  }
}

template <bool INT4>
static hipError_t launch_gemm_fmt(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  if (p.mode == kModeLds) {
    if (p.mt == 1) return launch_gemm_epi<1, INT4, kModeLds>(a, epi, p, s);
    return launch_gemm_epi<2, INT4, kModeLds>(a, epi, p, s);
  }
  if (p.mode == kModeSingle) {
    switch (p.mt) {
      case 1: return launch_gemm_epi<1, INT4, kModeSingle>(a, epi, p, s);
      case 2: return launch_gemm_epi<2, INT4, kModeSingle>(a, epi, p, s);
      default: return launch_gemm_epi<4, INT4, kModeSingle>(a, epi, p, s);
    }
  }
  switch (p.mt) {
    case 1: return launch_gemm_epi<1, INT4, kModeRing>(a, epi, p, s);
    case 2: return launch_gemm_epi<2, INT4, kModeRing>(a, epi, p, s);
    default: return launch_gemm_epi<4, INT4, kModeRing>(a, epi, p, s);
  }
}

// ---------------------------------------------------------------- w8a8 host side

GemmPlan plan_gemm_w8(int M, int N, int K, int epi, bool allow_split) {
  GemmPlan p;
  memset(&p, 0, sizeof(p));
  p.n_tiles = epi == EPI_SILU ? N / 16 : (N + 15) / 16;
  const int units = K / 64, cus = cu_count();
  int ks = 1;
  if (allow_split && epi == EPI_STORE && p.n_tiles < cus) ks = std::min(8, std::max(1, cus / p.n_tiles));
  ks = std::max(1, std::min(ks, units / kW8Waves));
  p.ksplit = ks;
  p.grid = std::max(1, std::min(p.n_tiles, cus / ks)) * ks;
  p.launches = (M + kRowsPerLaunch - 1) / kRowsPerLaunch;
  return p;
}

template <int MT, int EPI>
static hipError_t launch_w8_one(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_w8<MT, EPI>), dim3(grid), dim3((kW8Waves + 1) * 64), 0, s, a);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_w8_epi(const GemmArgs& a, int epi, int grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_w8_one<MT, EPI_STORE>(a, grid, s);
    case EPI_SILU: return launch_w8_one<MT, EPI_SILU>(a, grid, s);
    case EPI_QKV: return launch_w8_one<MT, EPI_QKV>(a, grid, s);
    case EPI_ARGMAX: return launch_w8_one<MT, EPI_ARGMAX>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_gemm_w8(GemmArgs a, int epi, hipStream_t s) {
  if (a.K % 64 || !a.asum || !a.wscale) return hipErrorInvalidValue;
  const GemmPlan p = plan_gemm_w8(a.M, a.N, a.K, epi, a.partial != nullptr);
  a.n_tiles = p.n_tiles;
  a.ksplit = p.ksplit;
  a.n_parts = p.grid;
  for (int l = 0; l < p.launches; ++l) {
    a.m_base = l * kRowsPerLaunch;
    const int rows = std::min(kRowsPerLaunch, a.M - a.m_base);
    const hipError_t e = rows <= 16 ? launch_w8_epi<1>(a, epi, p.grid, s) : launch_w8_epi<2>(a, epi, p.grid, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(GemmArgs a, int epi, int fmt, hipStream_t s) {
  if (fmt == LA_W_W8A8) return launch_gemm_w8(a, epi, s);
  const bool int4 = fmt == LA_W_INT4;
  if (use_big_gemm(a.M, int4, epi, a.layout != LA_LAYOUT_ROWS)) return launch_gemm_big(a, epi, int4, s);
  const GemmPlan p = plan_gemm(a.M, a.N, a.K, int4, epi, a.partial != nullptr);
  a.n_tiles = p.n_tiles;
  a.ksplit = p.ksplit;
  a.n_parts = p.grid;
  const int units = int4 ? a.K / 128 : a.K / 32;
  for (int l = 0; l < p.launches; ++l) {
    a.m_base = l * kRowsPerLaunch;
    const int rows = (a.M - a.m_base) < kRowsPerLaunch ? (a.M - a.m_base) : kRowsPerLaunch;
    // the last launch may hold fewer rows: fewer row tiles, perhaps another mode
    const int mt8 = (rows + 7) / 8;
    GemmPlan pl = p;
    plan_launch(pl, mt8 <= 1 ? 1 : mt8 <= 2 ? 2 : 4, units, int4, p.per);
    a.nw = pl.nw;
    hipError_t e = int4 ? launch_gemm_fmt<true>(a, epi, pl, s) : launch_gemm_fmt<false>(a, epi, pl, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

constexpr int kPackSplitChunks = 256;  // chunks of 8 values per workgroup of a split row

template <int NP>
static hipError_t launch_pack_np(const PackArgs& a, int rows, hipStream_t s) {
  const int K8 = a.K / 8;
  if (!a.gain && K8 > kPackSplitChunks) {
    // no row-wide sum: parts of kPackSplitChunks chunks, so that the rows of a
    // small batch spread over many compute units (the INT4 down operand at 48
    // rows: 48 workgroups of 88 KB each were bound by the per-CU load rate)
    const dim3 grid(rows, (K8 + kPackSplitChunks - 1) / kPackSplitChunks);
    hipLaunchKernelGGL((k_pack<NP, 1>), grid, dim3(kPackSplitChunks), 0, s, a);
    return hipGetLastError();
  }
  const int C = K8 <= 1024 ? 1 : 2;
  const int bd = ((K8 + C - 1) / C + 63) / 64 * 64;
  if (C == 1) hipLaunchKernelGGL((k_pack<NP, 1>), dim3(rows), dim3(bd), 0, s, a);
  else hipLaunchKernelGGL((k_pack<NP, 2>), dim3(rows), dim3(bd), 0, s, a);
  return hipGetLastError();
}

template <int NP>
static hipError_t launch_pack_w8(const PackArgs& a, hipStream_t s) {
  const int rows = a.apack ? ((a.M + 15) / 16) * 16 : a.M;
  const int bd = ((a.K / 16) + 63) / 64 * 64;
  hipLaunchKernelGGL((k_pack_w8<NP>), dim3(rows), dim3(bd), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  if (a.w8) {
    // int8 rows and their scales; every row of the last 16-row tile is written
    if (a.K % 64 || a.K / 16 > 1024) return hipErrorInvalidValue;
    const int n = a.parts ? a.n_parts : 0;
    if (n < 0 || n > 8) return hipErrorInvalidValue;
    if (n == 0) return launch_pack_w8<0>(a, s);
    if (n <= 2) return launch_pack_w8<2>(a, s);
    if (n <= 4) return launch_pack_w8<4>(a, s);
    return launch_pack_w8<8>(a, s);
  }
  // every operand row of the last tile is written (rows >= M become zero)
  const int rows = a.apack ? ((a.M + 7) / 8) * 8 : a.M;
  if (a.K / 8 > 2048) return hipErrorInvalidValue;
  const int n = a.parts ? a.n_parts : 0;
  if (n < 0 || n > 16) return hipErrorInvalidValue;
  if (n == 0) return launch_pack_np<0>(a, rows, s);
  if (n == 1) return launch_pack_np<1>(a, rows, s);
  if (n == 2) return launch_pack_np<2>(a, rows, s);
  if (n <= 4) return launch_pack_np<4>(a, rows, s);
  if (n <= 8) return launch_pack_np<8>(a, rows, s);
  if (n <= 12) return launch_pack_np<12>(a, rows, s);
  return launch_pack_np<16>(a, rows, s);
}

hipError_t launch_argmax_reduce(const float* amax, int M, int n_parts, const int32_t* flags,
                                int32_t* ids, float* top1, float* gap, int32_t* err,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_reduce, dim3(M), dim3(1024), 0, s, amax, n_parts, flags, ids, top1,
                     gap, err);
  return hipGetLastError();
}

}  // namespace la
