// Weight-streaming GEMMs for 33 .. 192 rows (batched PBD windows) on the gfx950
// matrix cores.
//
// At M = 6 x batch rows in the hundreds every weight must meet every row while
// it is in registers: a weight fragment read once from HBM feeds one
// 16x16x32 step per 8-row tile of the launch (24 steps at 192 rows), so the
// stream stays near the HBM rate while the matrix cores do the hi + lo work.
//
// Work decomposition: workgroup b takes K slice b % ksplit and column blocks
// b / ksplit, b / ksplit + gridDim.x / ksplit, ...; a column block is CW pairs
// of 16-column tiles.  Its consumer waves form an RW x CW grid: wave (rw, cw)
// keeps the accumulators of RT row tiles x 2 column tiles, loads the weights of
// its two column tiles through a deep ring of registers (raw buffer loads; a
// masked unit reads zero), and reads the activation fragments from LDS.  One
// producer wave copies each K unit of the packed activations (all row tiles of
// the launch) into a ring of LDS slots with direct-to-LDS loads; the waves
// meet at one barrier per unit.  The producer keeps its own load counter, so a
// consumer only ever waits for its weights.  Epilogues run in the consumer
// waves straight from the accumulators.
#include <algorithm>
#include <type_traits>

#include "la_gemm_common.hpp"

namespace la {

constexpr int kBigSlots = 5;  // LDS slots of the activation ring

template <bool INT4>
__host__ __device__ constexpr int big_depth() { return INT4 ? 3 : 5; }

// LDS bytes of one activation slot: RTW row tiles x one K unit (+ INT4 group sums).
__host__ __device__ constexpr int big_slot_bytes(int rtw, bool int4) {
  return rtw * (int4 ? 16 : 4) * 256 + (int4 ? (rtw + 3) / 4 * 256 : 0);
}

// Two producer waves split the copies of a unit: producer 0 the first half of
// the row tiles, producer 1 the rest (and the INT4 group sums).  Each issues a
// fixed count per unit, so its waits are compile-time constants.
constexpr int kBigProducers = 2;

template <int RTW, bool INT4>
__host__ __device__ constexpr int big_tiles_of(int p) {
  return p == 0 ? RTW / 2 : RTW - RTW / 2;
}
template <int RTW, bool INT4>
__host__ __device__ constexpr int big_copies(int p) {
  return big_tiles_of<RTW, INT4>(p) * (INT4 ? 4 : 1) + ((INT4 && p == 1) ? (RTW + 3) / 4 : 0);
}

__device__ __forceinline__ void lds_copy16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)lds_dst, 4, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// At most 3 column-pair waves per row of waves, plus the producer.
constexpr int kBigMaxCW = 3;

// The per-unit meeting point of producers and consumers.  A plain
// __syncthreads would make the producers drain every copy in flight (its
// release fence waits for all LDS-bound loads); instead each side waits for
// exactly what it must before the hardware barrier: the producers for the unit
// the consumers read next (wait_vmcnt), the consumers for their own LDS reads.
__device__ __forceinline__ void stage_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int RT, int RW, bool INT4, int EPI>
__global__ __launch_bounds__((RW * kBigMaxCW + kBigProducers) * 64) void k_gemm_big(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int RTW = RT * RW;
  constexpr int CPU = INT4 ? 16 : 4;
  constexpr int D = big_depth<INT4>();
  constexpr int SLOT = big_slot_bytes(RTW, INT4);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int CW = a.nw;  // column-pair waves per row of waves
  const int n_cons = RW * CW;
  const int K8 = a.K >> 3, KG = a.K >> 7;
  const int units = INT4 ? (a.K >> 7) : (a.K >> 5);
  const int ks = (int)blockIdx.x % a.ksplit;
  const int cb0 = (int)blockIdx.x / a.ksplit, gt = (int)gridDim.x / a.ksplit;
  const int s_lo = units * ks / a.ksplit, s_hi = units * (ks + 1) / a.ksplit;
  const int nu = s_hi - s_lo;
  // an item's stages are padded to whole turns of the weight ring (the padding
  // stages read zero weights), so items end where a turn ends
  const int nup = (nu + D - 1) / D * D;
  const int n_cb = (a.n_tiles + 2 * CW - 1) / (2 * CW);
  const int n_my = (n_cb - cb0 + gt - 1) / gt;
  const int total = n_my * nup;
  if (total <= 0) return;  // uniform over the workgroup
  const int rows = min(a.M - a.m_base, RTW * 8);
  const int mtv = (rows + 7) >> 3;
  unsigned char* slots = smem;                                  // [kBigSlots][SLOT]
  float* stage_lds = (float*)(smem + kBigSlots * SLOT);         // [n_cons][3*8][33]
  float* amax_lds = stage_lds + (size_t)n_cons * 3 * 8 * 33;    // ARGMAX: [n_cons][RT*8][3]

  auto slot_of = [&](int bi) { return slots + (bi % kBigSlots) * SLOT; };
  // unit of stage bi (a padding stage repeats the item's last unit)
  auto unit_of = [&](int bi) { return s_lo + min(bi % nup, nu - 1); };
  auto live_of = [&](int bi) { return bi < total && bi % nup < nu; };
  auto cblock_of = [&](int bi) { return cb0 + (bi / nup) * gt; };

  if (wave >= n_cons) {
    // ---------------------------------------------------------------- producers
    const int pw = wave - n_cons;  // 0 or 1
    const uint16_t* ap = a.apack + (size_t)(a.m_base >> 3) * K8 * 128;
    const float* asp = INT4 ? a.asum + (size_t)(a.m_base >> 3) * KG * 16 : nullptr;
    auto copy_unit = [&](auto pc, int bi) {
      constexpr int P = decltype(pc)::value;
      constexpr int T0 = P == 0 ? 0 : RTW / 2;
      constexpr int NT = big_tiles_of<RTW, INT4>(P);
      // a stage past the end re-copies the last one into a slot nobody reads again
      const int b = min(bi, total - 1);
      const int u = unit_of(b);
      unsigned char* dst = slot_of(bi);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int t = T0 + tt;
        const uint16_t* src = ap + ((size_t)min(t, mtv - 1) * K8 + (size_t)u * CPU) * 128;
#pragma unroll
        for (int q = 0; q < CPU / 4; ++q)
          lds_copy16(src + q * 512 + lane * 8, dst + (t * CPU + q * 4) * 256);
      }
      if (INT4 && P == 1) {
        float* sdst = (float*)(dst + RTW * CPU * 256);
#pragma unroll
        for (int q = 0; q < (RTW + 3) / 4; ++q) {
          const int t = min(q * 4 + (lane >> 4), RTW - 1);
          lds_copy4(asp + ((size_t)min(t, mtv - 1) * KG + u) * 16 + (lane & 15), sdst + q * 64);
        }
      }
    };
    auto run = [&](auto pc) {
      constexpr int P = decltype(pc)::value;
      constexpr int WAIT = (kBigSlots - 2) * big_copies<RTW, INT4>(P);
#pragma unroll
      for (int j = 0; j < kBigSlots - 1; ++j) copy_unit(pc, j);
      wait_vmcnt<WAIT>();
      stage_barrier();
      for (int bi = 0; bi < total; ++bi) {
        copy_unit(pc, bi + kBigSlots - 1);
        wait_vmcnt<WAIT>();  // unit bi + 1 has landed
        stage_barrier();
      }
      // Both roles end on a full barrier.  Without it the compiler may share
      // the final stage barrier between the roles, and the consumers' loop then
      // inherits the producers' outstanding LDS copies: it waits for all
      // memory (weights included) once per ring turn.
      __syncthreads();
    };
    if (pw == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
    return;
  }

  // ---------------------------------------------------------------- consumers
  const int rw = wave / CW, cw = wave - rw * CW;
  const int g = lane >> 4, c = lane & 15;
  const __amdgpu_buffer_rsrc_t rwt = make_rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(INT4 ? (const void*)a.wscale : a.w, INT4 ? a.s_bytes : 0u);

  struct WStage {
    u32x4 w[2];
    uint16_t s[INT4 ? 2 : 1];
  };
  WStage st[D];
  auto issue = [&](int bi, WStage& s) {
    const int b = min(bi, total - 1);
    const int u = unit_of(b);
    const int tile0 = (cblock_of(b) * CW + cw) * 2;
    const bool live_stage = live_of(bi);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tile = tile0 + t;
      const bool live = live_stage && tile < a.n_tiles;  // wave-uniform
      const WPtr wp = wptr<INT4, EPI>(a, min(tile, a.n_tiles - 1));
      const uint32_t dead = (uint32_t)(!live) << 31;  // out of range: reads zero
      s.w[t] = bload16<kNonTemporal>(rwt, (wp.w + (uint32_t)u * wp.ustride) | dead);
      if (INT4) s.s[INT4 ? t : 0] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (wp.s + (uint32_t)u * wp.sstride) | dead, 0, 0);
    }
  };

  f32x4 acc[RT][2];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WStage& s, const unsigned char* slot) {
    const uint16_t* A = (const uint16_t*)slot + (size_t)(rw * RT) * CPU * 128 + c * 8;
    if (!INT4) {
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, s.w[0]);
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, s.w[1]);
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const bf16x8 af = *(const bf16x8*)(A + (i * CPU + g) * 128);
        acc[i][0] = mfma_16x16x32(af, b0, acc[i][0]);
        acc[i][1] = mfma_16x16x32(af, b1, acc[i][1]);
      }
    } else {
      // 128 + q as bf16 from two masks and an OR; per group:
      // acc += scale * (sum - 136 * sum_k a_k)
      const float* AS = (const float*)(slot + RTW * CPU * 256) + (size_t)(rw * RT) * 16 + 4 * g;
      f32x4 tacc[RT][2];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) tacc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 bv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t w = s.w[t][j];
          u32x4 bb;
          bb[0] = (w & 0x000F000Fu) | 0x43004300u;
          bb[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
          bb[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
          bb[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
          bv[t] = __builtin_bit_cast(bf16x8, bb);
        }
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          const bf16x8 af = *(const bf16x8*)(A + (i * CPU + g * 4 + j) * 128);
          tacc[i][0] = mfma_16x16x32(af, bv[0], tacc[i][0]);
          tacc[i][1] = mfma_16x16x32(af, bv[1], tacc[i][1]);
        }
        // the next step's fragments are not read ahead of time (registers)
        __builtin_amdgcn_sched_barrier(0);
      }
      const float sc0 = fp16_to_f32(s.s[0]), sc1 = fp16_to_f32(s.s[INT4 ? 1 : 0]);
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const f32x4 as = *(const f32x4*)(AS + i * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][0][e] += sc0 * (tacc[i][0][e] - 136.0f * as[e]);
          acc[i][1][e] += sc1 * (tacc[i][1][e] - 136.0f * as[e]);
        }
      }
    }
  };

  // Epilogue of one column block.  The accumulators go through this wave's
  // small LDS staging area RP row tiles at a time (hi + lo rows added; lanes
  // 0..31 hold real rows 4g + e, column c), and one rolled loop does the
  // epilogue of each part, so its code exists once.
  constexpr int RP = 3;  // row tiles per staged part
  constexpr int NPART = RT / RP;
  static_assert(RT % RP == 0, "parts");
  float* stage = stage_lds + (size_t)wave * RP * 8 * 33;
  float* my_amax = EPI == EPI_ARGMAX ? amax_lds + (size_t)wave * RT * 8 * 3 : nullptr;
  if (EPI == EPI_ARGMAX) {
    for (int i = lane; i < RT * 8; i += 64) {
      my_amax[i * 3 + 0] = -INFINITY;
      my_amax[i * 3 + 1] = __int_as_float(0x7FFFFFFF);
      my_amax[i * 3 + 2] = -INFINITY;
    }
  }
  auto stage_part = [&](auto pc) {
    constexpr int P = decltype(pc)::value;
#pragma unroll
    for (int ii = 0; ii < RP; ++ii) {
      constexpr int dummy = 0;
      (void)dummy;
      const int i = P * RP + ii;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[P * RP + ii][t][e] + __shfl_xor(acc[P * RP + ii][t][e], 32);
          if (g < 2) stage[(ii * 8 + 4 * g + e) * 33 + t * 16 + c] = v;
        }
        acc[P * RP + ii][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
      (void)i;
    }
  };
  auto epi_part = [&](int cblock, int part) {
    const int tile0 = (cblock * CW + cw) * 2;
    const int row0 = rw * RT * 8 + part * RP * 8;  // first staged row within the launch
    if (EPI == EPI_ARGMAX) {
      // lane r < RP*8 takes staged row r: its 32 columns into the row's state
      if (lane < RP * 8) {
        const float* src = stage + lane * 33;
        float* s3 = my_amax + (part * RP * 8 + lane) * 3;
        float v1 = s3[0], v2 = s3[2];
        int i1 = __float_as_int(s3[1]);
        for (int cc = 0; cc < 32; ++cc) {
          const int tile = tile0 + (cc >> 4);
          const int n = tile * 16 + (cc & 15);
          if (tile >= a.n_tiles || n >= a.N) break;
          top2_merge(v1, i1, v2, src[cc], n, -INFINITY);
        }
        s3[0] = v1;
        s3[1] = __int_as_float(i1);
        s3[2] = v2;
      }
      return;
    }
    for (int idx = lane; idx < RP * 8 * 32; idx += 64) {
      const int r = idx >> 5, cc = idx & 31;
      const int t = cc >> 4, cl = cc & 15;
      const int tile = tile0 + t;
      const int ml = row0 + r;
      if (tile >= a.n_tiles || ml >= rows) continue;
      const int m = a.m_base + ml;
      const float v = stage[r * 33 + cc];
      if (EPI == EPI_STORE) {
        const int n = tile * 16 + cl;
        if (n >= a.N) continue;
        if (a.ksplit > 1) {
          a.partial[((size_t)ks * a.M + m) * a.N + n] = v;
        } else {
          float y = v;
          if (a.bias) y += bf16_to_f32(a.bias[n]);
          if (a.residual) y += a.residual[(size_t)m * a.ldy + n];
          a.y[(size_t)m * a.ldy + n] = y;
        }
      } else if (EPI == EPI_SILU) {
        // columns 0..7: gate rows tile*8 + c, 8..15: the matching up rows
        if (cl >= 8) continue;
        const int F = a.N / 2;
        const int n = tile * 8 + cl;
        const float y = silu_f(v) * stage[r * 33 + cc + 8];
        if (a.y) a.y[(size_t)m * a.ldy + n] = y;
        if (a.y_apack) {
          uint32_t h, l;
          split_hi_lo(y, h, l);
          const size_t base = (((size_t)(m >> 3) * (F / 8) + (n >> 3)) * 16 + (m & 7)) * 8 + (n & 7);
          a.y_apack[base] = (uint16_t)h;
          a.y_apack[base + 64] = (uint16_t)l;
        }
      } else if (EPI == EPI_QKV) {
        // tile = (head, sub): columns c < 8 are dims sub*8 + c, c >= 8 the
        // RoPE partners 64 + sub*8 + c - 8
        if (cl >= 8) continue;
        const int Hq = a.n_heads, Hkv = a.n_kv_heads;
        const int head = tile >> 3, sub = tile & 7;
        const int i2 = sub * 8 + cl;
        const int r1 = head * kHeadDim + i2, r2 = r1 + 64;
        float x1 = v, x2 = stage[r * 33 + cc + 8];
        if (a.bias) {
          x1 += bf16_to_f32(a.bias[r1]);
          x2 += bf16_to_f32(a.bias[r2]);
        }
        if (head < Hq + Hkv) {
          const float2 cs = a.rope[(size_t)m * 64 + i2];
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
        const int b = m / a.W, jw = m - b * a.W;
        const int pos = a.prefix_len[b] + jw;
        if (pos < 0 || pos >= a.max_blocks * kBlock) continue;
        const int blk = a.block_table[(size_t)b * a.max_blocks + pos / kBlock];
        if (blk < 0 || blk >= a.num_blocks) continue;
        const int slot = pos % kBlock;
        if (head < Hq + Hkv) {
          uint16_t* kp = a.kc + (((size_t)blk * Hkv + (head - Hq)) * kBlock + slot) * kHeadDim;
          kp[i2] = (uint16_t)f32_to_bf16_rne(x1);
          kp[i2 + 64] = (uint16_t)f32_to_bf16_rne(x2);
        } else {
          uint16_t* vp = a.vc + ((size_t)blk * Hkv + (head - Hq - Hkv)) * kHeadDim * kBlock;
          vp[(size_t)i2 * kBlock + slot] = (uint16_t)f32_to_bf16_rne(x1);
          vp[(size_t)(i2 + 64) * kBlock + slot] = (uint16_t)f32_to_bf16_rne(x2);
        }
      }
    }
  };
  auto epilogue = [&](int cblock) {
    for (int part = 0; part < NPART; ++part) {
      switch (part) {  // each case stages fixed accumulators
        case 0: stage_part(std::integral_constant<int, 0>{}); break;
        case 1: stage_part(std::integral_constant<int, 1 % NPART>{}); break;
        case 2: stage_part(std::integral_constant<int, 2 % NPART>{}); break;
        default: stage_part(std::integral_constant<int, 3 % NPART>{}); break;
      }
      epi_part(cblock, part);
    }
  };

  // the weight ring: stage bi is multiplied while stages bi+1 .. bi+D-1 are in
  // flight; one barrier per stage pairs the consumers with the producer.  An
  // item is a whole number of ring turns, so its epilogue has one site.
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, st[j]);
  __builtin_amdgcn_sched_barrier(0);
  stage_barrier();
  for (int it = 0; it < n_my; ++it) {
    for (int u0 = 0; u0 < nup; u0 += D) {
      const int bb = it * nup + u0;
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int bi = bb + j;
        issue(bi + D - 1, st[(j + D - 1) % D]);
        __builtin_amdgcn_sched_barrier(0);
        compute(st[j], slot_of(bi));
        stage_barrier();
      }
    }
    epilogue(cblock_of(it * nup));
  }
  __syncthreads();  // pairs with the producers' last barrier
  if (EPI == EPI_ARGMAX) {
    // merge the column waves' row states (fixed order) and write one partial
    // per row and workgroup
    if (cw == 0) {
      for (int r = lane; r < RT * 8; r += 64) {
        const int ml = (rw * RT) * 8 + r;
        float v1 = -INFINITY, v2 = -INFINITY;
        int i1 = 0x7FFFFFFF;
        for (int w = 0; w < CW; ++w) {
          const float* s3 = amax_lds + ((size_t)(rw * CW + w) * RT * 8 + r) * 3;
          top2_merge(v1, i1, v2, s3[0], __float_as_int(s3[1]), s3[2]);
        }
        if (ml < rows) {
          float* o = a.amax + ((size_t)(a.m_base + ml) * a.n_parts + blockIdx.x) * 3;
          o[0] = v1;
          o[1] = __int_as_float(i1);
          o[2] = v2;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- host side

static int big_cus() {
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

static size_t big_smem(const BigPlan& p, bool int4, int epi) {
  const size_t waves = (size_t)p.rw * p.cw;
  return (size_t)kBigSlots * big_slot_bytes(p.rt * p.rw, int4) + waves * 3 * 8 * 33 * 4 +
         (epi == EPI_ARGMAX ? waves * p.rt * 8 * 3 * 4 : 0);
}

// Rows per launch: 192 (bf16) or 48 (INT4).
int big_rows_per_launch(bool int4) { return int4 ? 48 : 192; }

// The large-M kernel serves every M > 32 rows.
bool use_big_gemm(int M, int K, bool int4) {
  (void)K;
  (void)int4;
  return M > 32;
}

BigPlan plan_gemm_big(int rows, int N, int K, bool int4, int epi, bool allow_split) {
  BigPlan p;
  p.n_tiles = (epi == EPI_SILU) ? (N / 2) / 8 : (N + 15) / 16;
  const int mt = (rows + 7) / 8;
  if (int4) {
    p.rt = 6;
    p.rw = 1;
  } else if (mt <= 6) {
    p.rt = 6;
    p.rw = 1;
  } else if (mt <= 12) {
    p.rt = 12;
    p.rw = 1;
  } else {
    p.rt = 12;
    p.rw = 2;
  }
  const int cus = big_cus();
  const int units = int4 ? K / 128 : K / 32;
  // column-pair waves per row of waves and K slices: the fewest rounds of
  // column blocks times the work of one block (columns x units of its slice);
  // on a tie the wider block, which reuses each activation unit for more
  // columns
  double best = 1e30;
  p.cw = 1;
  p.ksplit = 1;
  for (int cw = 1; cw <= kBigMaxCW; ++cw) {
    const int n_cb = (p.n_tiles + 2 * cw - 1) / (2 * cw);
    for (int ks = 1; ks <= 16; ks *= 2) {
      if (ks > 1 && !(allow_split && epi == EPI_STORE)) break;
      if (ks > 1 && units / ks < 8) break;
      const int per_slice = cus / ks > 0 ? cus / ks : 1;
      const int rounds = (n_cb + per_slice - 1) / per_slice;
      // partial sums cost a write and a read of the output per slice
      const double cost = (double)rounds * cw * ((units + ks - 1) / ks) * (1.0 + 0.02 * (ks - 1));
      if (cost < best - 1e-9 || (cost < best + 1e-9 && cw > p.cw)) {
        best = cost;
        p.cw = cw;
        p.ksplit = ks;
      }
    }
  }
  const int n_cb = (p.n_tiles + 2 * p.cw - 1) / (2 * p.cw);
  const int per_slice = cus / p.ksplit > 0 ? cus / p.ksplit : 1;
  const int per = (n_cb + per_slice - 1) / per_slice;
  const int gt = (n_cb + per - 1) / per;
  p.grid = gt * p.ksplit;
  p.threads = (p.rw * p.cw + kBigProducers) * 64;
  p.smem = big_smem(p, int4, epi);
  return p;
}

template <int RT, int RW, bool INT4, int EPI>
static hipError_t launch_big_one(const GemmArgs& a, const BigPlan& p, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_big<RT, RW, INT4, EPI>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm_big<RT, RW, INT4, EPI>), dim3(p.grid), dim3(p.threads), p.smem, s, a);
  return hipGetLastError();
}

template <int RT, int RW, bool INT4>
static hipError_t launch_big_epi(const GemmArgs& a, int epi, const BigPlan& p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_big_one<RT, RW, INT4, EPI_STORE>(a, p, s);
    case EPI_SILU: return launch_big_one<RT, RW, INT4, EPI_SILU>(a, p, s);
    case EPI_QKV: return launch_big_one<RT, RW, INT4, EPI_QKV>(a, p, s);
    default: return launch_big_one<RT, RW, INT4, EPI_ARGMAX>(a, p, s);
  }
}

hipError_t launch_gemm_big(GemmArgs a, int epi, bool int4, hipStream_t s) {
  const int per_launch = big_rows_per_launch(int4);
  const BigPlan p0 = plan_gemm_big(std::min(a.M, per_launch), a.N, a.K, int4, epi, a.partial != nullptr);
  for (int m0 = 0; m0 < a.M; m0 += per_launch) {
    const int rows = std::min(a.M - m0, per_launch);
    BigPlan p = plan_gemm_big(rows, a.N, a.K, int4, epi, a.partial != nullptr);
    // one plan of K slices and workgroups for every launch (the partial sums
    // and the lm_head parts are laid out by the first)
    p.ksplit = p0.ksplit;
    p.cw = p0.cw;
    p.grid = p0.grid;
    p.threads = (p.rw * p.cw + kBigProducers) * 64;
    p.smem = big_smem(p, int4, epi);
    GemmArgs g = a;
    g.m_base = m0;
    g.n_tiles = p.n_tiles;
    g.ksplit = p.ksplit;
    g.nw = p.cw;
    g.n_parts = p.grid;
    hipError_t e;
    if (int4) e = launch_big_epi<6, 1, true>(g, epi, p, s);
    else if (p.rt == 6) e = launch_big_epi<6, 1, false>(g, epi, p, s);
    else if (p.rw == 1) e = launch_big_epi<12, 1, false>(g, epi, p, s);
    else e = launch_big_epi<12, 2, false>(g, epi, p, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace la
