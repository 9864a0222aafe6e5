// The front half of a decoder layer for at most 8 window rows, as one
// persistent launch: input RMSNorm, the QKV projection with bias, RoPE and
// the bf16 K/V write, the window attention over the paged cache with its
// log-sum-exp merge, and the O projection with the residual and the packed,
// post-normed operand of the gate/up projection.
//
// Why one launch: at a handful of rows every one of these steps is short and
// latency bound, and as separate kernels each pays a launch boundary and a
// full HBM round trip before its first product.  Here everything that does
// not depend on another step is in flight from the first cycle: the QKV
// weight tiles, the rows and the pending K-slice sums, and every cache page
// that holds only keys older than this step.
//
// The RMSNorm is folded into the QKV product: the operand is (h + pending
// sums) * in_norm, split into bf16 hi / lo, and the epilogue scales row r by
// 1 / rms_r, so packing a slice of K needs nothing from the rest of the row.
//
// One workgroup per compute unit (the grid never exceeds the compute units,
// and all its workgroups are resident together); each takes fixed roles:
//   QKV tile t:     workgroup t, 8 waves split K, wave 0 runs the epilogue;
//   O tile t:       workgroup t, after its QKV tile (its O weights load while
//                   the attention runs);
//   pack slice p:   the 64 workgroups after the QKV tiles, 32 columns of K
//                   each: the operand slice and its rows' sums of squares;
//   attention item: workgroups from the top of the grid, one run of at most
//                   kFrontMaxRunPages pages of one (sequence, KV head) for one
//                   16-column query tile each, the whole run staged in LDS and
//                   its page pairs spread one per wave; once every run of the
//                   tile has stored its partial result, run r merges a slice
//                   of the tile's columns.  (A workgroup may be both a pack
//                   slice and an item: it packs while its pages load.)
// Hand-offs.  Data that a few workgroups read (q and the window's K / V for
// the attention items, the runs' partial results for their merge) travels as
// 8-byte words {32-bit datum, epoch}: one agent-scope (cross-XCD coherent)
// store per word, read with agent-scope loads until every word it needs holds
// the launch's epoch (the layer index + 1; the step's prologue zeroes the
// words).  An aligned 8-byte access is never split, so a word is wholly old or
// wholly new, and the consumer sees the data one memory trip after it is
// written: no store has to complete before a flag, and no flag is read first.
// Data that 128 or more workgroups read in full (the packed QKV operand, the
// attention output) goes as plain data plus flag words: each producer stores
// with agent-scope stores, waits for them to complete (s_waitcnt) and sets its
// own int32 word to the epoch (no two producers write one word, no atomic);
// these flag arrays have a copy per XCD (each waiter polls the copy of its
// XCD) and a waiter reads a whole array with one vector load per poll.  Every
// wait is bounded: a wait that runs out sets LA_DERR_SYNC in the error word and
// goes on, so the launch always ends.
#include "la_attn_common.hpp"

namespace la {

namespace {

constexpr int kFrontWaves = 8;
constexpr int kFrontThreads = kFrontWaves * 64;
constexpr int kFrontUnits = 8;               // 32-k units per wave (K = 2048)
constexpr int kFrontK = 2048;
constexpr int kFrontMaxParts = 4;            // pending K-slice sums read in one pass
constexpr int kFrontMaxRuns = 16;            // runs of one (sequence, KV head)
constexpr int kSliceK = kFrontK / kFrontPackSlices;  // columns of one pack slice
constexpr int kFlagCopies = 8;               // copies of a widely waited flag array (one per XCD)
constexpr int kSpinLimit = 1 << 21;
constexpr int kCoherent = 16;                // cache policy of agent-scope coherent buffer accesses
constexpr uint32_t kNoRow = 0x80000000u;     // buffer offset past every range: the load reads zeros
static_assert(kSliceK == 32, "a pack slice is 4 chunks of 8 columns");

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// LDS: the attention role's page ring, or (once a workgroup's front roles are
// done) its first kGuPreload gate/up weight tiles; then the reduction tiles.
constexpr int kTileBytes = kFrontK / 32 * 1024;  // one 16-column tile of a tiled weight (K = 2048)
constexpr int kGuPreload = 2;
constexpr int kRingBytes = kFrontMaxRunPages * kPageBytes;
constexpr int kRedOff = kRingBytes > kGuPreload * kTileBytes ? kRingBytes : kGuPreload * kTileBytes;
constexpr int kOutvOff = kRedOff + kFrontWaves * 64 * 16;
constexpr int kQOff = kOutvOff + 8 * 17 * 4;                 // an attention item's q (hi, lo fragments)
constexpr int kFrontLds = kQOff + 64 * 8 * 16;

__device__ __forceinline__ void set_flag(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u16(uint16_t* p, uint32_t v) {
  __hip_atomic_store((short*)p, (short)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Stores made so far have reached the coherent level.
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ u32x4 pack8(const uint32_t (&x)[8]) {
  const u32x4 v = {x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16), x[6] | (x[7] << 16)};
  return v;
}

// Flag arrays (ints): pack [kFlagCopies][64] (slice), ready [kFlagCopies][128]
// (item), O done [kFlagCopies][128] (O tile), gate/up done [kFlagCopies][256]
// (workgroup).
__device__ __forceinline__ int32_t* fl_pack(const FrontArgs& f, int copy) { return f.sync + copy * 64; }
__device__ __forceinline__ int32_t* fl_ready(const FrontArgs& f, int copy) {
  return f.sync + kFlagCopies * 64 + copy * 128;
}
__device__ __forceinline__ int32_t* fl_odone(const FrontArgs& f, int copy) {
  return f.sync + kFlagCopies * (64 + 128) + copy * 128;
}
__device__ __forceinline__ int32_t* fl_gdone(const FrontArgs& f, int copy) {
  return f.sync + kFlagCopies * (64 + 128 + 128) + copy * 256;
}
static_assert(kFlagCopies * (64 + 128 + 128 + 256) == kFrontSyncWords, "flag words the step carves");

// One 8-byte word {datum, epoch}.
__device__ __forceinline__ void ll_store(uint64_t* p, uint32_t d, int epoch) {
  __hip_atomic_store(p, ((uint64_t)(uint32_t)epoch << 32) | d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two words {d0, epoch}, {d1, epoch} as one 16-byte agent-scope store.
__device__ __forceinline__ void ll_store2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t d0, uint32_t d1, int epoch) {
  const u32x4 v = {d0, (uint32_t)epoch, d1, (uint32_t)epoch};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCoherent);
}
__device__ __forceinline__ u32x4 ll_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ bool ll_ok(u32x4 v, uint32_t epoch) { return v[1] == epoch && v[3] == epoch; }

// End of a poll round of one wave: true once no active lane still misses a
// word; false after a short sleep otherwise (the spin limit ends the wait with
// LA_DERR_SYNC).
__device__ __forceinline__ bool ll_round(const FrontArgs& f, bool ok, int& spins) {
  if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
  if (++spins >= kSpinLimit) {
    // the first active lane reports
    if (f.err && (threadIdx.x & 63) == (int)__builtin_amdgcn_readfirstlane(threadIdx.x & 63)) atomicOr(f.err, LA_DERR_SYNC);
    return true;
  }
  __builtin_amdgcn_s_sleep(1);
  return false;
}

// The whole workgroup waits until p[0 .. n) (n <= 128) all hold the epoch
// (wave 0 polls, two words per lane at most).  One poll in flight: more polls
// of the same lines from the same waiters make the flag land later.
__device__ __forceinline__ void wait_flags(const FrontArgs& f, const int32_t* p, int n) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p, (uint32_t)n * 4);
    const uint32_t o0 = lane < n ? (uint32_t)lane * 4 : kNoRow;
    const uint32_t o1 = lane + 64 < n ? (uint32_t)(lane + 64) * 4 : kNoRow;
    const uint32_t ep = (uint32_t)f.epoch;
    for (int spins = 0;;) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // every poll is a fresh load
      const uint32_t a = __builtin_amdgcn_raw_buffer_load_b32(r, o0, 0, kCoherent);
      const uint32_t b = __builtin_amdgcn_raw_buffer_load_b32(r, o1, 0, kCoherent);
      // words past n read as zero and count as set
      if (__builtin_amdgcn_ballot_w64((lane < n && a != ep) || (lane + 64 < n && b != ep)) == 0) break;
      if (++spins >= kSpinLimit) {
        if (lane == 0 && f.err) atomicOr(f.err, LA_DERR_SYNC);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// wait_flags for up to 256 words (four per lane).
__device__ __forceinline__ void wait_flags_wide(const FrontArgs& f, const int32_t* p, int n) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p, (uint32_t)n * 4);
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = lane + 64 * k < n ? (uint32_t)(lane + 64 * k) * 4 : kNoRow;
    const uint32_t ep = (uint32_t)f.epoch;
    for (int spins = 0;;) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // every poll is a fresh load
      uint32_t v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = __builtin_amdgcn_raw_buffer_load_b32(r, o[k], 0, kCoherent);
      bool miss = false;
#pragma unroll
      for (int k = 0; k < 4; ++k) miss |= lane + 64 * k < n && v[k] != ep;
      if (__builtin_amdgcn_ballot_w64(miss) == 0) break;
      if (++spins >= kSpinLimit) {
        if (lane == 0 && f.err) atomicOr(f.err, LA_DERR_SYNC);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// This wave's 8 weight fragments of tile t of a tiled bf16 weight with K = 2048.
__device__ __forceinline__ void load_tile_weights(const void* w, uint32_t bytes, int t, int wave, u32x4 (&wf)[kFrontUnits]) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, bytes);
  constexpr int UT = kFrontK / 32;
#pragma unroll
  for (int i = 0; i < kFrontUnits; ++i) {
    const uint32_t u = (uint32_t)wave * kFrontUnits + i;
    wf[i] = bload16<kNonTemporal>(rw, (((uint32_t)t * UT + u) * 64 + lane) * 16);
  }
}

// The 8 x 16 product tile from this wave's A and weight fragments: partial
// tiles through LDS, real row r = operand row r (hi) + operand row r + 8 (lo),
// into outv[8][17].
__device__ __forceinline__ void tile_reduce(const bf16x8 (&af)[kFrontUnits], const u32x4 (&wf)[kFrontUnits], int wave,
                                            f32x4* red, float* outv) {
  const int lane = threadIdx.x & 63;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kFrontUnits; ++i) acc = mfma_16x16x32(af[i], __builtin_bit_cast(bf16x8, wf[i]), acc);
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (threadIdx.x < 128) {
    const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
    const int lh = (r >> 2) * 16 + c, ll = ((r + 8) >> 2) * 16 + c, e = r & 3;
    float v = 0.f;
    for (int w = 0; w < kFrontWaves; ++w) v += red[w * 64 + lh][e] + red[w * 64 + ll][e];
    outv[r * 17 + c] = v;
  }
  __syncthreads();
}

// 1 / rms of window row ml (rows of lanes 8 ml .. 8 ml + 7 of wave 0): the 64
// pack slices' sums of squares, 8 per lane, then a fixed butterfly.
__device__ __forceinline__ float row_inv_rms(const FrontArgs& f, u32x4 s0, u32x4 s1) {
  float t = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) t += __uint_as_float(s0[e]);
#pragma unroll
  for (int e = 0; e < 4; ++e) t += __uint_as_float(s1[e]);
  t += __shfl_xor(t, 1);
  t += __shfl_xor(t, 2);
  t += __shfl_xor(t, 4);
  return 1.0f / sqrtf(t / (float)f.H + f.eps);
}

// What the QKV epilogue of tile t needs besides the product, read before the
// product so that its latency hides behind the weights (wave 0, lane (row
// ml = lane / 8, column c = lane % 8)): the bias, the RoPE rotation and, for
// K and V tiles, where the row's two values go in the cache (null: not written).
struct QkvEpi {
  float b1, b2;
  float2 cs;
  uint16_t* p1;
  uint16_t* p2;
};

__device__ QkvEpi qkv_epi_prepare(const FrontArgs& f, int t) {
  const AttnArgs& a = f.at;
  const int lane = threadIdx.x & 63;
  const int head = t >> 3, sub = t & 7;
  const int ml = lane >> 3, c = lane & 7;
  const int i = sub * 8 + c;
  const int r1 = head * kHeadDim + i, r2 = r1 + 64;
  QkvEpi e;
  e.b1 = e.b2 = 0.f;
  e.cs = make_float2(1.f, 0.f);
  e.p1 = e.p2 = nullptr;
  if (ml >= f.T) return e;
  if (f.qkv_bias) {
    e.b1 = bf16_to_f32(f.qkv_bias[r1]);
    e.b2 = bf16_to_f32(f.qkv_bias[r2]);
  }
  if (head < a.Hq + a.Hkv) e.cs = f.rope[(size_t)ml * 64 + i];
  if (head < a.Hq) return e;
  const int b = ml / a.W, j = ml - b * a.W;
  const int pos = a.prefix_len[b] + j;
  if ((f.flags && f.flags[ml]) || pos < 0 || pos >= a.max_blocks * kBlock) return e;
  const int blk = a.block_table[(size_t)b * a.max_blocks + pos / kBlock];
  if (blk < 0 || blk >= a.num_blocks) return e;
  const int slot = pos % kBlock;
  if (head < a.Hq + a.Hkv) {
    uint16_t* kp = const_cast<uint16_t*>(a.kc) + (((size_t)blk * a.Hkv + (head - a.Hq)) * kBlock + slot) * kHeadDim;
    e.p1 = kp + i;
    e.p2 = kp + i + 64;
  } else {
    uint16_t* vp = const_cast<uint16_t*>(a.vc) + ((size_t)blk * a.Hkv + (head - a.Hq - a.Hkv)) * kHeadDim * kBlock;
    e.p1 = vp + (size_t)i * kBlock + slot;
    e.p2 = vp + (size_t)(i + 64) * kBlock + slot;
  }
  return e;
}

// QKV epilogue of tile t (wave 0): 1 / rms, bias, RoPE; q as words for the
// attention, the window's K and V as words for the attention and as bf16 into
// the cache (for later steps).
__device__ void qkv_epilogue(const FrontArgs& f, int t, const float* outv, float inv, const QkvEpi& e) {
  const AttnArgs& a = f.at;
  const int lane = threadIdx.x & 63;
  const int head = t >> 3, sub = t & 7;
  const int ml = lane >> 3, c = lane & 7;
  if (ml >= f.T) return;
  const int i = sub * 8 + c;
  const int r1 = head * kHeadDim + i, r2 = r1 + 64;
  float x1 = outv[ml * 17 + c] * inv + e.b1, x2 = outv[ml * 17 + c + 8] * inv + e.b2;
  if (head < a.Hq + a.Hkv) {
    const float y1 = x1 * e.cs.x - x2 * e.cs.y, y2 = x2 * e.cs.x + x1 * e.cs.y;
    x1 = y1;
    x2 = y2;
  }
  if (head < a.Hq) {
    uint64_t* q = f.ll_q + (size_t)ml * a.Hq * kHeadDim;
    ll_store(q + r1, __float_as_uint(x1), f.epoch);
    ll_store(q + r2, __float_as_uint(x2), f.epoch);
    return;
  }
  const uint32_t b1 = f32_to_bf16_rne(x1), b2 = f32_to_bf16_rne(x2);
  const int kv = head < a.Hq + a.Hkv ? 0 : 1, g = head - a.Hq - kv * a.Hkv;
  ll_store(f.ll_kv + ((size_t)(ml * a.Hkv + g) * 2 + kv) * 64 + i, b1 | (b2 << 16), f.epoch);
  if (e.p1) {
    *e.p1 = (uint16_t)b1;
    *e.p2 = (uint16_t)b2;
  }
}

// h + the pending K-slice sums (slice order) at columns n of rows ml, read
// through buffer ranges that end at the last valid byte: rows past T and
// slices past n_parts read as zeros.
__device__ __forceinline__ void load_rows(const FrontArgs& f, int ml, int n, float (&x)[1 + kFrontMaxParts]) {
  const uint32_t row_bytes = (uint32_t)f.H * 4;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(f.h, (uint32_t)f.T * row_bytes);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(f.parts, f.parts ? (uint32_t)f.n_parts * f.T * row_bytes : 0u);
  const bool live = ml < f.T;
  x[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rh, live ? (uint32_t)ml * row_bytes + n * 4 : kNoRow, 0, 0));
#pragma unroll
  for (int s = 0; s < kFrontMaxParts; ++s)
    x[1 + s] = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rp, live ? ((uint32_t)s * f.T + ml) * row_bytes + n * 4 : kNoRow, 0, 0));
}

// O epilogue of tile t (wave 0): h1 = (h + pending sums) + o, the tile's sums
// of squares, h1 * post_norm packed.  res: this lane's two residual columns,
// gain: post_norm at its column.
__device__ void o_epilogue(const FrontArgs& f, int t, const float (&res)[2][1 + kFrontMaxParts], float gain,
                           const float* outv) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = lane + it * 64;
    const int ml = idx >> 4, c = idx & 15;
    const int n = t * 16 + c;
    const bool ok = ml < f.T;
    float v = 0.f;
    if (ok) {
      float hv = res[it][0];
#pragma unroll
      for (int s = 0; s < kFrontMaxParts; ++s) hv += res[it][1 + s];
      v = hv + outv[ml * 17 + c];
      f.h[(size_t)ml * f.H + n] = v;
    }
    float q = ok ? v * v : 0.f;
    q += __shfl_xor(q, 1);
    q += __shfl_xor(q, 2);
    q += __shfl_xor(q, 4);
    q += __shfl_xor(q, 8);
    // read by the gate/up tiles of this launch when it runs them (agent-scope
    // stores), else by the next kernel
    if (ok && c == 0) {
      if (f.wgu) st_f32(f.ss + (size_t)ml * (f.H / 16) + t, q);
      else f.ss[(size_t)ml * (f.H / 16) + t] = q;
    }
    if (ok) {
      uint32_t hb, lb;
      split_hi_lo(v * gain, hb, lb);
      const size_t base = ((size_t)(n >> 3) * 16 + ml) * 8 + (n & 7);
      if (f.wgu) {
        st_u16(f.gpack + base, hb);
        st_u16(f.gpack + base + 64, lb);
      } else {
        f.gpack[base] = (uint16_t)hb;
        f.gpack[base + 64] = (uint16_t)lb;
      }
    }
  }
}

// Pack slice p (wave 0, lanes 0..31: row lane / 4, chunk 4p + lane % 4):
// (h + pending sums) * in_norm as bf16 hi (operand row r) and lo (row r + 8),
// written as one contiguous kilobyte; the rows' sums of squares over the slice
// into ss_part[row][p].
__device__ void front_pack(const FrontArgs& f, int p) {
  const int lane = threadIdx.x & 63;
  const int r = (lane >> 2) & 7, kc = p * (kSliceK / 8) + (lane & 3);
  const uint32_t row_bytes = (uint32_t)f.H * 4;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(f.h, (uint32_t)f.T * row_bytes);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(f.parts, f.parts ? (uint32_t)f.n_parts * f.T * row_bytes : 0u);
  const bool live = r < f.T && lane < 32;
  const uint32_t oh = live ? (uint32_t)r * row_bytes + (uint32_t)kc * 32 : kNoRow;
  u32x4 x[1 + kFrontMaxParts][2];
  x[0][0] = bload16<0>(rh, oh);
  x[0][1] = bload16<0>(rh, oh + 16);
#pragma unroll
  for (int s = 0; s < kFrontMaxParts; ++s) {
    const uint32_t op = live ? ((uint32_t)s * f.T + r) * row_bytes + (uint32_t)kc * 32 : kNoRow;
    x[1 + s][0] = bload16<0>(rp, op);
    x[1 + s][1] = bload16<0>(rp, op + 16);
  }
  const uint4 gw = *(const uint4*)(f.in_norm + kc * 8);
  const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
  float v[8], ss = 0.f;
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = __uint_as_float(x[0][e >> 2][e & 3]);
#pragma unroll
    for (int s = 0; s < kFrontMaxParts; ++s) v[e] += __uint_as_float(x[1 + s][e >> 2][e & 3]);
    ss += v[e] * v[e];
    split_hi_lo(v[e] * bf16_to_f32((gg[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu), hi[e], lo[e]);
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  if (lane < 32) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(f.xpack, kFrontK / 8 * 256);
    const uint32_t off = ((uint32_t)kc * 16 + r) * 16;
    __builtin_amdgcn_raw_buffer_store_b128(pack8(hi), rx, off, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b128(pack8(lo), rx, off + 128, 0, kCoherent);
    if ((lane & 3) == 0) st_f32(f.ss_part + r * kFrontPackSlices + p, ss);
  }
  stores_done();
  if (lane < kFlagCopies) set_flag(fl_pack(f, lane) + p, f.epoch);
}

// The projection role of tile t: the packed operand
// (read coherently once every pack slice is in), the product, the epilogue.
// An O tile's weights (tile t of O, t < n_o_tiles) are requested into wo at
// the first cycle with the QKV weights: they arrive long before the attention
// is done, and the gate/up loads issued after the QKV product no longer queue
// ahead of them.
__device__ __forceinline__ void front_qkv(const FrontArgs& f, int t, unsigned char* smem, u32x4 (&wo)[kFrontUnits]) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4 wq[kFrontUnits];
  load_tile_weights(f.wqkv, f.wqkv_bytes, t, wave, wq);
  if (t < f.n_o_tiles) load_tile_weights(f.wo, f.wo_bytes, t, wave, wo);
  QkvEpi epi;
  if (wave == 0) epi = qkv_epi_prepare(f, t);
  wait_flags(f, fl_pack(f, blockIdx.x % kFlagCopies), kFrontPackSlices);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(f.xpack, kFrontK / 8 * 256);
  const bool live = (lane & 7) < f.T;  // operand rows r (hi) and r + 8 (lo) of window row r
  bf16x8 af[kFrontUnits];
#pragma unroll
  for (int i = 0; i < kFrontUnits; ++i) {
    const uint32_t kc = (uint32_t)(wave * kFrontUnits + i) * 4 + g4;
    af[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, live ? (kc * 16 + (lane & 15)) * 16 : kNoRow, 0, kCoherent));
  }
  // wave 0: this lane's 8 of the 64 sums of squares of row lane / 8
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(f.ss_part, 8 * kFrontPackSlices * 4);
  u32x4 s0 = {0u, 0u, 0u, 0u}, s1 = s0;
  if (wave == 0) {
    const uint32_t so = (uint32_t)((lane >> 3) * kFrontPackSlices + (lane & 7) * 8) * 4;
    s0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, so, 0, kCoherent));
    s1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, so + 16, 0, kCoherent));
  }
  __builtin_amdgcn_sched_barrier(0);  // every request in flight before the first product
  float* outv = (float*)(smem + kOutvOff);
  tile_reduce(af, wq, wave, (f32x4*)(smem + kRedOff), outv);
  if (wave == 0) qkv_epilogue(f, t, outv, row_inv_rms(f, s0, s1), epi);
  __syncthreads();  // the epilogue's stores go out before the O weight loads
}

// The O role of tile t: waits for every attention item, reads the packed
// attention output coherently, multiplies, runs the epilogue.
__device__ __forceinline__ void front_o(const FrontArgs& f, int t, const u32x4 (&wo)[kFrontUnits], unsigned char* smem) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float res[2][1 + kFrontMaxParts];
  float gain = 0.f;
  if (wave == 0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) load_rows(f, (lane + it * 64) >> 4, t * 16 + (lane & 15), res[it]);
    gain = bf16_to_f32(f.post_norm[t * 16 + (lane & 15)]);
  }
  wait_flags(f, fl_ready(f, blockIdx.x % kFlagCopies), f.n_items);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(f.at.out_apack, kFrontK / 8 * 256);
  const bool live = (lane & 7) < f.T;  // operand rows r (hi) and r + 8 (lo) of window row r
  bf16x8 af[kFrontUnits];
#pragma unroll
  for (int i = 0; i < kFrontUnits; ++i) {
    const uint32_t kc = (uint32_t)(wave * kFrontUnits + i) * 4 + g4;
    af[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, live ? (kc * 16 + (lane & 15)) * 16 : kNoRow, 0, kCoherent));
  }
  __builtin_amdgcn_sched_barrier(0);  // all 8 requests in flight before the first product
  float* outv = (float*)(smem + kOutvOff);
  tile_reduce(af, wo, wave, (f32x4*)(smem + kRedOff), outv);
  if (wave == 0) {
    o_epilogue(f, t, res, gain, outv);
    if (f.wgu) {
      stores_done();
      if (lane < kFlagCopies) set_flag(fl_odone(f, lane) + t, f.epoch);
    }
  }
}

// The first kGuPreload gate/up tiles of this workgroup (tiles blockIdx.x,
// blockIdx.x + gridDim.x, ...) copied into LDS in the tiled weight's byte
// order (direct-to-LDS loads; wave w copies units 8w .. 8w + 7).  The caller's
// roles no longer use LDS below kRedOff.
__device__ void gu_preload(const FrontArgs& f, unsigned char* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.wgu, f.wgu_bytes);
  for (int p = 0; p < kGuPreload; ++p) {
    const int j = (int)blockIdx.x + p * (int)gridDim.x;
    if (j >= f.n_gu_tiles) break;  // uniform
#pragma unroll
    for (int i = 0; i < kFrontUnits; ++i) {
      const uint32_t u = (uint32_t)wave * kFrontUnits + i;
      void __attribute__((address_space(3)))* dst =
          (void __attribute__((address_space(3)))*)(smem + p * kTileBytes + u * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, (uint32_t)lane * 16, ((uint32_t)j * (kFrontK / 32) + u) * 1024,
                                               0, kNonTemporal);
    }
  }
}

// Gate/up epilogue of tile j (wave 0, lane (row lane / 8, column lane % 8)):
// silu(gate / rms) * (up / rms) as bf16 hi / lo into the down operand.
__device__ __forceinline__ void gu_epilogue(const FrontArgs& f, int j, const float* outv, float inv) {
  const int lane = threadIdx.x & 63, ml = lane >> 3, c = lane & 7;
  if (ml >= f.T) return;
  const float v = silu_f(outv[ml * 17 + c] * inv) * (outv[ml * 17 + c + 8] * inv);
  const int n = j * 8 + c;
  uint32_t h, l;
  split_hi_lo(v, h, l);
  const size_t base = ((size_t)(n >> 3) * 16 + ml) * 8 + (n & 7);
  if (f.wdn) {
    // read by this launch's down projection on other compute units
    st_u16(f.mpack + base, h);
    st_u16(f.mpack + base + 64, l);
  } else {
    f.mpack[base] = (uint16_t)h;
    f.mpack[base + 64] = (uint16_t)l;
  }
}

// The down projection's share of this workgroup when the launch runs it: K
// slice s of kFrontDownSlices (units u0 .. u0 + nu - 1 of 32 k), output tiles
// t0 and t0 + 1 (per = gridDim.x / kFrontDownSlices workgroups a slice, the
// host makes 2 per = H / 16); wave w takes units u0 + w + 8 i.
struct DnShare {
  int s, t0, u0, nu, U;
};
__device__ __forceinline__ DnShare dn_share(const FrontArgs& f) {
  DnShare d;
  const int per = gridDim.x / kFrontDownSlices;
  d.s = blockIdx.x / per;
  d.t0 = 2 * (blockIdx.x % per);
  d.U = f.F / 32;
  const int spu = (d.U + kFrontDownSlices - 1) / kFrontDownSlices;
  d.u0 = d.s * spu;
  d.nu = min(spu, d.U - d.u0);
  return d;
}
constexpr int kDnLds = 8;  // units per wave and tile staged in LDS: 2 x 8 x 8 KB = 128 KB
constexpr int kDnReg = 3;  // further units per wave and tile in registers
static_assert(8 * (kDnLds + kDnReg) == kFrontDownUnits, "units of one slice");
static_assert(2 * kDnLds * kFrontWaves * 1024 <= kGuPreload * kTileBytes, "down weights in the preload LDS");

// The first kDnLds units per wave of both down tiles into LDS (direct-to-LDS
// loads; unit (tile k, i) of wave w at ((k kDnLds + i) 8 + w) KB), once the
// preloaded gate/up tiles have been read.
__device__ void dn_preload(const FrontArgs& f, unsigned char* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const DnShare d = dn_share(f);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.wdn, f.wdn_bytes);
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int i = 0; i < kDnLds; ++i) {
      const int ui = wave + 8 * i;
      if (ui < d.nu) {  // uniform
        void __attribute__((address_space(3)))* dst =
            (void __attribute__((address_space(3)))*)(smem + ((k * kDnLds + i) * kFrontWaves + wave) * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, (uint32_t)lane * 16,
                                                 ((uint32_t)(d.t0 + k) * d.U + d.u0 + ui) * 1024, 0, kNonTemporal);
      }
    }
}

// The rest of this wave's down units (kDnReg per tile) into registers.
__device__ __forceinline__ void dn_issue_regs(const FrontArgs& f, int wave, u32x4 (&wd)[2 * kDnReg]) {
  const int lane = threadIdx.x & 63;
  const DnShare d = dn_share(f);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.wdn, f.wdn_bytes);
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int i = 0; i < kDnReg; ++i) {
      const int ui = wave + 8 * (kDnLds + i);
      const uint32_t off = ui < d.nu ? ((((uint32_t)(d.t0 + k) * d.U + d.u0 + ui) * 64 + lane) * 16) : kNoRow;
      wd[k * kDnReg + i] = bload16<kNonTemporal>(rw, off);
    }
}

// The down role of every workgroup: once every workgroup's gate/up outputs
// are in (the packed SiLU operand, agent-scope stores), its two output tiles
// over its K slice; the waves' partial tiles meet in LDS (the same sums in the
// same order as tile_reduce), and the K-slice sums go to dparts for the next
// pack.
__device__ __forceinline__ void front_down(const FrontArgs& f, unsigned char* smem, const u32x4 (&wd)[2 * kDnReg]) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const DnShare d = dn_share(f);
  wait_flags_wide(f, fl_gdone(f, blockIdx.x % kFlagCopies), gridDim.x);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(f.mpack, (uint32_t)(f.F / 8) * 256);
  const bool live = (lane & 7) < f.T;  // operand rows r (hi) and r + 8 (lo) of window row r
  bf16x8 af[kDnLds + kDnReg];
#pragma unroll
  for (int i = 0; i < kDnLds + kDnReg; ++i) {
    const int ui = wave + 8 * i;
    const uint32_t kc = (uint32_t)(d.u0 + ui) * 4 + g4;
    af[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                           ra, ui < d.nu && live ? (kc * 16 + (lane & 15)) * 16 : kNoRow, 0, kCoherent));
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS copies (each wave reads only its own units)
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < kDnLds + kDnReg; ++i) {
    if (wave + 8 * i < d.nu) {  // uniform
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4 w = i < kDnLds ? *(const u32x4*)(smem + ((k * kDnLds + i) * kFrontWaves + wave) * 1024 + lane * 16)
                                   : wd[k * kDnReg + (i < kDnLds ? 0 : i - kDnLds)];
        acc[k] = mfma_16x16x32(af[i], __builtin_bit_cast(bf16x8, w), acc[k]);
      }
    }
  }
  __syncthreads();  // every wave is done with the LDS weights
  f32x4* red = (f32x4*)smem;  // [tile][wave][lane]
#pragma unroll
  for (int k = 0; k < 2; ++k) red[(k * kFrontWaves + wave) * 64 + lane] = acc[k];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int k = threadIdx.x >> 7, o = threadIdx.x & 127, r = o >> 4, c = o & 15;
    const int lh = (r >> 2) * 16 + c, ll = ((r + 8) >> 2) * 16 + c, e = r & 3;
    float v = 0.f;
    for (int w = 0; w < kFrontWaves; ++w)
      v += red[(k * kFrontWaves + w) * 64 + lh][e] + red[(k * kFrontWaves + w) * 64 + ll][e];
    if (r < f.T) f.dparts[((size_t)d.s * f.T + r) * f.H + (d.t0 + k) * 16 + c] = v;
  }
}

// After this workgroup's gate/up tiles: its flag (once wave 0's stores of the
// packed SiLU operand are out), the down weights' register part, the down role.
__device__ __forceinline__ void front_dn_tail(const FrontArgs& f, unsigned char* smem, u32x4 (&wd)[2 * kDnReg],
                                              bool wd_issued) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0) {
    stores_done();
    if (lane < kFlagCopies) set_flag(fl_gdone(f, lane) + blockIdx.x, f.epoch);
  }
  if (!wd_issued) dn_issue_regs(f, wave, wd);
  front_down(f, smem, wd);
}

// This workgroup's gate/up tiles after the kGuPreload preloaded ones: the
// first three are requested into the register buffers.
__device__ __forceinline__ void gu_issue(const FrontArgs& f, int wave, u32x4 (&wa)[kFrontUnits],
                                         u32x4 (&wb)[kFrontUnits], u32x4 (&wc)[kFrontUnits]) {
  const int G = gridDim.x, js = (int)blockIdx.x + kGuPreload * G;
  if (js < f.n_gu_tiles) load_tile_weights(f.wgu, f.wgu_bytes, js, wave, wa);
  if (js + G < f.n_gu_tiles) load_tile_weights(f.wgu, f.wgu_bytes, js + G, wave, wb);
  if (js + 2 * G < f.n_gu_tiles) load_tile_weights(f.wgu, f.wgu_bytes, js + 2 * G, wave, wc);
}

// The gate/up role of every workgroup: its tiles blockIdx.x + k gridDim.x.
// Three streamed tiles' weights are requested before the wait (by gu_issue,
// here unless the caller did it earlier); once every O tile is done the packed
// post-norm operand and the rows' 1 / rms are read (agent scope), the
// preloaded tiles multiply from LDS and the rest stream through the three
// register buffers.
__device__ __forceinline__ void front_gateup(const FrontArgs& f, unsigned char* smem, u32x4 (&wa)[kFrontUnits],
                                             u32x4 (&wb)[kFrontUnits], u32x4 (&wc)[kFrontUnits], bool issued,
                                             u32x4 (&wd)[2 * kDnReg], bool& wd_issued) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x, j0 = blockIdx.x;
  if (j0 >= f.n_gu_tiles) {  // uniform
    if (f.wdn) dn_preload(f, smem);
    return;
  }
  const int js = j0 + kGuPreload * G;  // first streamed tile
  if (!issued) gu_issue(f, wave, wa, wb, wc);
  wait_flags(f, fl_odone(f, blockIdx.x % kFlagCopies), f.n_o_tiles);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(f.gpack, kFrontK / 8 * 256);
  const bool live = (lane & 7) < f.T;  // operand rows r (hi) and r + 8 (lo) of window row r
  bf16x8 af[kFrontUnits];
#pragma unroll
  for (int i = 0; i < kFrontUnits; ++i) {
    const uint32_t kc = (uint32_t)(wave * kFrontUnits + i) * 4 + g4;
    af[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, live ? (kc * 16 + (lane & 15)) * 16 : kNoRow, 0, kCoherent));
  }
  // wave 0: 1 / rms of row lane / 8 from the O tiles' 128 sums of squares
  float inv = 0.f;
  if (wave == 0) {
    const int ml = lane >> 3;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(f.ss, (uint32_t)f.T * (f.H / 16) * 4);
    const uint32_t so = ml < f.T ? ((uint32_t)ml * (f.H / 16) + (lane & 7) * 16) * 4 : kNoRow;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, so + k * 16, 0, kCoherent));
#pragma unroll
      for (int e = 0; e < 4; ++e) t += __uint_as_float(v[e]);
    }
    t += __shfl_xor(t, 1);
    t += __shfl_xor(t, 2);
    t += __shfl_xor(t, 4);
    inv = 1.0f / sqrtf(t / (float)f.H + f.eps);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's preload copies (and everything before them)
  __syncthreads();
  float* outv = (float*)(smem + kOutvOff);
  f32x4* red = (f32x4*)(smem + kRedOff);
  for (int p = 0; p < kGuPreload; ++p) {
    const int j = j0 + p * G;
    if (j >= f.n_gu_tiles) break;  // uniform: no streamed tile either
    u32x4 wf[kFrontUnits];
#pragma unroll
    for (int i = 0; i < kFrontUnits; ++i)
      wf[i] = *(const u32x4*)(smem + p * kTileBytes + (((uint32_t)wave * kFrontUnits + i) * 64 + lane) * 16);
    tile_reduce(af, wf, wave, red, outv);
    if (wave == 0) gu_epilogue(f, j, outv, inv);
  }
  // the preloaded tiles' LDS now takes the down projection's weights
  if (f.wdn) dn_preload(f, smem);
  // three tiles in flight: each buffer is refilled right after its product
  for (int j = js; j < f.n_gu_tiles; j += 3 * G) {
    tile_reduce(af, wa, wave, red, outv);
    if (j + 3 * G < f.n_gu_tiles) load_tile_weights(f.wgu, f.wgu_bytes, j + 3 * G, wave, wa);
    if (wave == 0) gu_epilogue(f, j, outv, inv);
    if (j + G >= f.n_gu_tiles) break;  // uniform
    tile_reduce(af, wb, wave, red, outv);
    if (j + 4 * G < f.n_gu_tiles) load_tile_weights(f.wgu, f.wgu_bytes, j + 4 * G, wave, wb);
    if (wave == 0) gu_epilogue(f, j + G, outv, inv);
    if (j + 2 * G >= f.n_gu_tiles) break;  // uniform
    tile_reduce(af, wc, wave, red, outv);
    if (j + 5 * G < f.n_gu_tiles) load_tile_weights(f.wgu, f.wgu_bytes, j + 5 * G, wave, wc);
    // the down weights' register part once three buffers' tiles are done
    // (wave 0 after its flag: its stores must not wait for these loads)
    if (f.wdn && wave != 0 && !wd_issued) {
      dn_issue_regs(f, wave, wd);
      wd_issued = true;
    }
    if (wave == 0) gu_epilogue(f, j + 2 * G, outv, inv);
  }
}

// One attention item: sequence b, KV head g, query tile qt (query columns
// 16 qt .. 16 qt + 15, column i being window row i / G of query head g G + i %
// G), run r of a.pages_per_split pages.  Every page is copied into LDS at
// once; the keys of the window rows (written by this launch) then come from
// their K / V words, and q from its words (wave 0 polls them and hands the hi /
// lo fragments on through LDS).  Wave w takes pairs w, w + 8, ..., and wave 0
// combines the waves' states.  A single-run sequence writes its normalised
// output; otherwise every run stores its (max, sum, unnormalised O) as words
// and merges a slice of the tile's columns from every run's words.
__device__ void front_attention(const FrontArgs& f, int b, int g, int qt, int r, unsigned char* smem, int slice) {
  const AttnArgs& a = f.at;
  unsigned char* ring = smem;
  const int lane = threadIdx.x & 63, gl = lane >> 4, rr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.Hq / a.Hkv, NQ = a.W * G;
  const int q0 = qt * 16;
  const int kps = a.pages_per_split * kBlock;
  const int n_keys = attn_keys(a, b);
  const int nruns = (n_keys + kps - 1) / kps;
  const int k0 = r * kps;
  const uint32_t ep = (uint32_t)f.epoch;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out_apack, (uint32_t)(a.Hq * kHeadDim / 8) * 256);
  if (k0 >= n_keys) {
    if (slice >= 0 && threadIdx.x < 64) front_pack(f, slice);
    if (n_keys == 0 && r == 0) {
      // no key at all (a prefix the step flags as invalid): zero output
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int idx = threadIdx.x; idx < 16 * 16; idx += kFrontThreads) {
        const int qi = q0 + (idx >> 4), ch = idx & 15;
        if (qi >= NQ) continue;
        const int wr = qi / G, hg = qi - wr * G;
        const int row = b * a.W + wr, col = (g * G + hg) * kHeadDim + ch * 8;
        const uint32_t off = ((uint32_t)(col >> 3) * 16 + row) * 16;
        __builtin_amdgcn_raw_buffer_store_b128(z, ro, off, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b128(z, ro, off + 128, 0, kCoherent);
      }
    }
    return;  // uniform: this run holds no keys
  }
  const int k1 = min(n_keys, k0 + kps);
  const int npages = (k1 - k0 + kBlock - 1) / kBlock;
  const int npairs = (npages + 1) >> 1;
  const int first = k0 / kBlock;
  int bt = a.block_table[(size_t)b * a.max_blocks + min(first + min(lane, npages - 1), a.max_blocks - 1)];
  bt = bt < 0 ? 0 : (bt >= a.num_blocks ? a.num_blocks - 1 : bt);
  const uint32_t cache_bytes = (uint32_t)a.num_blocks * a.Hkv * (kPageBytes / 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.kc, cache_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vc, cache_bytes);
  // wave 0 packs its slice first (the pack's wait for its own stores would
  // otherwise also wait for the page copies)
  if (slice >= 0) {
    if (wave == 0) front_pack(f, slice);
    __syncthreads();  // the pages wait: the pack is on the QKV tiles' path, the pages are not
  }
  // page j: wave w copies 1 KB piece w (pieces 0..3 of K, 4..7 of V^T); the
  // slots of window rows are overwritten below
  for (int j = 0; j < npages; ++j) {
    const int blk = __builtin_amdgcn_readlane(bt, j);
    const uint32_t base = ((uint32_t)blk * a.Hkv + g) * (kPageBytes / 2);
    void __attribute__((address_space(3)))* dst =
        (void __attribute__((address_space(3)))*)(ring + j * kPageBytes + wave * 1024);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 4 ? rk : rv, dst, 16, page_piece_src(wave, lane), base, 0, 0);
  }

  // keys [wlo, wlo + nwin) of this run are window rows of this launch: thread
  // t < 64 nwin takes two words (K if bit 5 of t is clear, else V) of key
  // wlo + t / 64
  const int P = a.prefix_len[b];
  const int wlo = max(P, k0), nwin = max(0, k1 - wlo);
  const bool kvt = (int)threadIdx.x < nwin * 64;
  const int wkey = wlo + (threadIdx.x >> 6), kvh = (threadIdx.x >> 5) & 1, i2 = (threadIdx.x & 31) * 2;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.ll_kv, (uint32_t)(f.T * a.Hkv * 128) * 8);
  const uint32_t kvoff =
      kvt ? ((uint32_t)(((b * a.W + wkey - P) * a.Hkv + g) * 2 + kvh) * 64 + i2) * 8 : 0u;
  // q of column q0 + rr (lane (gl, rr) of wave 0: dims 32 kb + 8 gl .. + 7)
  const int qi = q0 + rr;
  const int qc = qi < NQ ? qi : 0;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(f.ll_q, (uint32_t)(f.T * a.Hq * kHeadDim) * 8);
  const uint32_t qoff =
      ((uint32_t)((b * a.W + qc / G) * a.Hq + g * G + qc % G) * kHeadDim + gl * 8) * 8;
  u32x4 xq[4][4], xw = {0u, 0u, 0u, 0u};
  for (int spins = 0;;) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // every poll is a fresh load
    bool ok = true;
    if (wave == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int n = 0; n < 4; ++n) xq[kb][n] = ll_load2(rq, qoff + (kb * 32 + 2 * n) * 8);
    }
    if (kvt) xw = ll_load2(rw, kvoff);
    if (wave == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int n = 0; n < 4; ++n) ok = ok && ll_ok(xq[kb][n], ep);
    }
    if (kvt) ok = ok && ll_ok(xw, ep);
    if (ll_round(f, ok, spins)) break;
  }
  u32x4* qs = (u32x4*)(smem + kQOff);  // [8 fragments][64 lanes]
  if (wave == 0) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        split_hi_lo(qi < NQ ? __uint_as_float(xq[kb][e >> 1][(e & 1) * 2]) : 0.f, hi[e], lo[e]);
      qs[kb * 64 + lane] = pack8(hi);
      qs[(4 + kb) * 64 + lane] = pack8(lo);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's pieces of every page
  __syncthreads();
  if (kvt) {
    // the window key's K (chunk c of key k sits at 16-byte slot c ^ k) or V^T
    const int kk = wkey - k0, sl = kk & 15;
    unsigned char* pg = ring + (kk >> 4) * kPageBytes;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t d = xw[2 * u];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int dim = i2 + u + 64 * h;
        const uint16_t v = (uint16_t)(d >> (16 * h));
        if (kvh == 0)
          *(uint16_t*)(pg + sl * 256 + (((dim >> 3) ^ sl) * 16) + (dim & 7) * 2) = v;
        else
          *(uint16_t*)(pg + 4096 + dim * 32 + sl * 2) = v;
      }
    }
  }
  __syncthreads();

  AttnState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int crows = a.causal_rows ? min(max(a.causal_rows[b], 0), a.W) : (a.causal ? a.W : 0);
  const int wrow = qc / G;
  const int kcol = wrow < crows ? max(min(n_keys, P + wrow + 1), min(n_keys, 1)) : n_keys;
  if (wave < npairs) {
    bf16x8 qh[4], ql[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      qh[kb] = __builtin_bit_cast(bf16x8, qs[kb * 64 + lane]);
      ql[kb] = __builtin_bit_cast(bf16x8, qs[(4 + kb) * 64 + lane]);
    }
    for (int c = wave; c < npairs; c += kFrontWaves) {
      PairRegs pr;
      read_pair(ring + c * kPairBytes, pr);
      const int p0 = k0 + 2 * c * kBlock;
      attn_pair(pr, k1 - p0, min(k1, kcol) - p0, qh, ql, st);
    }
  }
  // the waves' states meet through the ring (every wave is done with the
  // pages): wave w then combines slice dt = w of the output dims over the
  // states in wave order, and stores it
  const int nw = min(npairs, kFrontWaves);  // waves that hold a state
  constexpr int kStateFloats = 8 * 4 + 2;
  float* gs = (float*)ring;
  __syncthreads();
  if (wave < nw) {
    float* d = gs + wave * kStateFloats * 64 + lane;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) d[(dt * 4 + e) * 64] = st.acc[dt][e];
    d[32 * 64] = st.m;
    d[33 * 64] = st.l;
  }
  __syncthreads();
  const int dt = wave;
  float M = -INFINITY;
  for (int w2 = 0; w2 < nw; ++w2) M = fmaxf(M, gs[w2 * kStateFloats * 64 + 32 * 64 + lane]);
  float lw = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int w2 = 0; w2 < nw; ++w2) {
    const float* sp = gs + w2 * kStateFloats * 64 + lane;
    const float m2 = sp[32 * 64];
    const float w = m2 == -INFINITY ? 0.f : exp2f(m2 - M);
    lw += w * sp[33 * 64];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += w * sp[(dt * 4 + e) * 64];
  }
  float lsum = lw;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (nruns == 1) {
    const float inv = 1.f / lsum;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = acc[e] * inv;
      v[4 + e] = __shfl_xor(v[e], 16);
    }
    if (qi < NQ && (gl & 1) == 0) {
      const int wr = qi / G, hg = qi - wr * G;
      const int row = b * a.W + wr, col = (g * G + hg) * kHeadDim + dt * 16 + 4 * gl;
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_hi_lo(v[e], hi[e], lo[e]);
      const uint32_t off = ((uint32_t)(col >> 3) * 16 + row) * 16;
      __builtin_amdgcn_raw_buffer_store_b128(pack8(hi), ro, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(pack8(lo), ro, off + 128, 0, kCoherent);
    }
    return;
  }

  // partial result of this run as words: unit ((b, g) run, query column)
  const uint32_t ubase = (uint32_t)((b * a.Hkv + g) * f.runs);
  const uint32_t units = (uint32_t)(a.B * a.Hkv * f.runs * a.nqp);
  const __amdgpu_buffer_rsrc_t rml = make_rsrc(f.ll_ml, units * 16);
  const __amdgpu_buffer_rsrc_t rpo = make_rsrc(f.ll_po, units * kHeadDim * 8);
  {
    const uint32_t u = (ubase + r) * a.nqp + qi;
    if (wave == 0 && gl == 0) ll_store2(rml, u * 16, __float_as_uint(M), __float_as_uint(lsum), f.epoch);
    const uint32_t o = (u * kHeadDim + dt * 16 + 4 * gl) * 8;
    ll_store2(rpo, o, __float_as_uint(acc[0]), __float_as_uint(acc[1]), f.epoch);
    ll_store2(rpo, o + 16, __float_as_uint(acc[2]), __float_as_uint(acc[3]), f.epoch);
  }

  // merge of the tile's columns [qa, qb): thread (column, 4-dim chunk c4,
  // half hf) combines runs hf * 8 .. hf * 8 + 7 in run order, the two halves
  // meet (half 0 first), and the column is normalised and packed (with the
  // neighbouring chunk)
  const int qa = q0 + r * 16 / nruns, qb = min(q0 + (r + 1) * 16 / nruns, NQ);
  for (int idx = threadIdx.x; idx < (qb - qa) * 64; idx += kFrontThreads) {
    const int q = qa + (idx >> 6), c4 = (idx >> 1) & 31, hf = idx & 1;
    const int s0 = hf * 8, ns = min(8, nruns - s0);  // ns <= 0: no run in this half
    u32x4 mlw[8], o0[8], o1[8];
    for (int spins = 0;;) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // every poll is a fresh load
      bool ok = true;
      if (ns > 0) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t u = (ubase + s0 + min(s, ns - 1)) * a.nqp + q;
          mlw[s] = ll_load2(rml, u * 16);
          o0[s] = ll_load2(rpo, (u * kHeadDim + 4 * c4) * 8);
          o1[s] = ll_load2(rpo, (u * kHeadDim + 4 * c4) * 8 + 16);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) ok = ok && ll_ok(mlw[s], ep) && ll_ok(o0[s], ep) && ll_ok(o1[s], ep);
      }
      if (ll_round(f, ok, spins)) break;
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < ns) M = fmaxf(M, __uint_as_float(mlw[s][0]));
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < ns) {
        const float ms = __uint_as_float(mlw[s][0]);
        const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
        den += w * __uint_as_float(mlw[s][2]);
        const f32x4 os = {__uint_as_float(o0[s][0]), __uint_as_float(o0[s][2]), __uint_as_float(o1[s][0]),
                          __uint_as_float(o1[s][2])};
        num += w * os;
      }
    }
    // the two halves (lanes idx, idx ^ 1): half 0's terms first
    const float Mo = __shfl_xor(M, 1), deno = __shfl_xor(den, 1);
    f32x4 numo;
#pragma unroll
    for (int e = 0; e < 4; ++e) numo[e] = __shfl_xor(num[e], 1);
    const float Mt = fmaxf(M, Mo);
    const float wa = M == -INFINITY ? 0.f : exp2f(M - Mt), wb = Mo == -INFINITY ? 0.f : exp2f(Mo - Mt);
    const float w0 = hf == 0 ? wa : wb, w1 = hf == 0 ? wb : wa;
    const float d0 = hf == 0 ? den : deno, d1 = hf == 0 ? deno : den;
    const float dtot = w0 * d0 + w1 * d1;
    const float inv = dtot > 0.f ? 1.f / dtot : 0.f;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float n0 = hf == 0 ? num[e] : numo[e], n1 = hf == 0 ? numo[e] : num[e];
      v[e] = (w0 * n0 + w1 * n1) * inv;
    }
    float w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = __shfl_xor(v[e], 2);  // the neighbouring chunk
    if (hf == 0 && (c4 & 1) == 0) {
      const float xv[8] = {v[0], v[1], v[2], v[3], w4[0], w4[1], w4[2], w4[3]};
      const int wr = q / G, hg = q - wr * G;
      const int row = b * a.W + wr, col = (g * G + hg) * kHeadDim + 4 * c4;
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_hi_lo(xv[e], hi[e], lo[e]);
      const uint32_t off = ((uint32_t)(col >> 3) * 16 + row) * 16;
      __builtin_amdgcn_raw_buffer_store_b128(pack8(hi), ro, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(pack8(lo), ro, off + 128, 0, kCoherent);
    }
  }
}

}  // namespace

__global__ __launch_bounds__(kFrontThreads) void k_front(FrontArgs f) {
  extern __shared__ __align__(16) unsigned char smem[];
  const AttnArgs& a = f.at;
  const int w = blockIdx.x, G = gridDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = G - 1 - w;
  const int slice = w - f.n_qkv_tiles;

  if (w < f.n_qkv_tiles) {
    u32x4 wo[kFrontUnits];
    front_qkv(f, w, smem, wo);
    if (w < f.n_o_tiles) {
      // the O weights are in flight since the first cycle; the first gate/up
      // tiles go into LDS and the next three into registers while the
      // attention runs (so that they land before the O tile is done:
      // requested after it, they were the tail of the launch)
      u32x4 wa[kFrontUnits], wb[kFrontUnits], wc[kFrontUnits];
      if (f.wgu) {
        gu_preload(f, smem);
        gu_issue(f, wave, wa, wb, wc);
      }
      front_o(f, w, wo, smem);
      u32x4 wd[2 * kDnReg];
      bool wd_issued = false;
      if (f.wgu) front_gateup(f, smem, wa, wb, wc, true, wd, wd_issued);
      if (f.wdn) front_dn_tail(f, smem, wd, wd_issued);
      return;
    } else if (f.wgu) {
      gu_preload(f, smem);
    }
  } else {
    const bool has_item = item >= 0 && item < f.n_items;
    const bool has_slice = slice < kFrontPackSlices;
    if (has_item) {
      // the host keeps these workgroups free of QKV and O tiles; item =
      // ((b * Hkv + g) * tiles + qt) * runs + r
      const int tiles = a.nqp / 16;
      const int r = item % f.runs, rest = item / f.runs;
      const int qt = rest % tiles, bg = rest / tiles;
      front_attention(f, bg / a.Hkv, bg % a.Hkv, qt, r, smem, has_slice ? slice : -1);
      stores_done();
      __syncthreads();  // every wave is also done with the page ring
      if (threadIdx.x < kFlagCopies) set_flag(fl_ready(f, threadIdx.x) + item, f.epoch);
    } else if (has_slice) {
      if (wave == 0) front_pack(f, slice);
      // the other waves' gate/up loads wait: in the same compute unit they
      // would queue ahead of the pack's, which every QKV tile waits for
      __syncthreads();
    }
    if (f.wgu) gu_preload(f, smem);
  }
  u32x4 wa[kFrontUnits], wb[kFrontUnits], wc[kFrontUnits];
  u32x4 wd[2 * kDnReg];
  bool wd_issued = false;
  if (f.wgu) front_gateup(f, smem, wa, wb, wc, false, wd, wd_issued);
  if (f.wdn) front_dn_tail(f, smem, wd, wd_issued);
}

hipError_t launch_front(const FrontArgs& f, int grid, hipStream_t s) {
  if (!f.ll_q || !f.ll_kv || !f.ll_ml || !f.ll_po) return hipErrorInvalidValue;
  if (f.wgu && (!f.mpack || f.F != f.n_gu_tiles * 8 || f.n_gu_tiles < 1 ||
                (size_t)f.n_gu_tiles * kTileBytes > f.wgu_bytes))
    return hipErrorInvalidValue;
  // the down projection: every workgroup two output tiles of one K slice, at
  // most kFrontDownUnits units a slice, one gate/up-done flag per workgroup
  if (f.wdn && (!f.wgu || !f.dparts || f.H % 16 || grid != (f.H / 16) * kFrontDownSlices / 2 || grid > 256 ||
                f.F % 32 || (f.F / 32 + kFrontDownSlices - 1) / kFrontDownSlices > kFrontDownUnits ||
                (size_t)(f.H / 16) * (f.F / 32) * 1024 > f.wdn_bytes))
    return hipErrorInvalidValue;
  if (f.runs > kFrontMaxRuns || f.n_parts > kFrontMaxParts || f.at.pages_per_split > kFrontMaxRunPages ||
      f.H != kFrontK || f.HQ != kFrontK || f.T > 8 || f.n_o_tiles > f.n_qkv_tiles || f.at.nqp % 16 ||
      f.at.nqp < 16 || f.at.nqp > 64 || f.n_items != f.at.B * f.at.Hkv * (f.at.nqp / 16) * f.runs ||
      f.n_qkv_tiles + kFrontPackSlices > grid || f.n_qkv_tiles + f.n_items > grid || f.n_items > 128 || f.epoch <= 0)
    return hipErrorInvalidValue;
  static bool attr = false;  // allow the LDS beyond the static default once
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_front, hipFuncAttributeMaxDynamicSharedMemorySize, kFrontLds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(k_front, dim3(grid), dim3(kFrontThreads), kFrontLds, s, f);
  return hipGetLastError();
}

}  // namespace la
