// Block-masked GQA attention of the window rows over the paged bf16 KV cache.
//
// Every window row of sequence b attends to cache slots 0 .. P_b+W-1: the
// prefix lies before it and the window is bidirectional, so one key bound
// serves all rows and no per-element mask exists ("LocateAnything-3B for RK3588
// (RKLLM + RKNN)", "How it differs from the original", item 1; the Jetson
// page, section 1.3, block mask).  The causal window that RK3588 conversion
// runs instead (same item) is a per-row bound: row j sees slots 0 .. P_b+j.
// So is a re-fed window, whose first c_b rows re-send accepted tokens
// causally (row j < c_b sees slots 0 .. P_b+j) before the block, whose rows
// see slots 0 .. P_b+w_b-1 (w_b real rows; rows past them are padding).
//
// Work split: a workgroup takes one run of pages of one (sequence, KV head),
// one wave per tile of 16 query columns.  The 8 query heads of a KV head times
// W window rows form up to 128 query columns that share every K/V page:
//   S^T[key, query] = K_page . Q^T        16x16x32 bf16 matrix-core steps, Q split
//                                         into bf16 hi + lo columns (K is exact bf16)
//   online softmax per query column       exp2 on pre-scaled scores, a reference max
//                                         that moves only when a score passes it by 2^8
//   O^T[d, query] += V_pair^T . P^T       16x16x32 steps over the 32 keys of two
//                                         pages; P split into hi + lo; the two pages'
//                                         S^T accumulators are exactly the P^T
//                                         operand, so P never leaves registers
// V pages are stored dim-major ([D][16 keys]) so a V^T operand half is one
// 8-byte load.  The step is latency bound (a layer reads about a megabyte of KV
// at batch 1), so a run is short and issues all of its loads before it waits.
// Each run writes (max, sum, unnormalised O); a merge kernel combines the runs
// with log-sum-exp rescaling in a fixed order.  A sequence that fits one run
// is normalised and stored directly.
#include "la_attn_common.hpp"

namespace la {

// Store the normalised output of query column qi, dims [d0, d0 + 8).
__device__ __forceinline__ void attn_store8(const AttnArgs& a, int b, int kvh, int qi, int d0,
                                            const float v[8]) {
  const int G = a.Hq / a.Hkv;
  const int wr = qi / G, hg = qi - wr * G;
  const int row = b * a.W + wr;
  const int h = kvh * G + hg;
  const int ldo = a.Hq * kHeadDim;
  if (a.out) {
    float* o = a.out + (size_t)row * ldo + h * kHeadDim + d0;
    *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  if (a.out_apack) apack_store_chunk(a.out_apack, ldo, row, (h * kHeadDim + d0) / 8, v, a.out_int4);
}

// One workgroup per (run of pages_per_split pages, KV head, sequence); wave qt
// takes query tile qt.  The run's pages stream in pairs through a ring of
// LA + 1 LDS pair slots with direct-to-LDS loads, LA pairs ahead; each wave
// copies a share of every pair (16 pieces of 1 KB) and the waves meet at one
// barrier per pair, after which that pair is complete and the slot being
// refilled has been read by everybody.  With a single run per sequence the result is
// normalised and stored here; otherwise (max, sum, unnormalised O) goes to
// the run's partial slot.
template <int NQT, int LA>
__global__ __launch_bounds__(NQT > 4 ? 512 : 256)
__attribute__((amdgpu_waves_per_eu(LA == 1 && NQT > 1 ? 3 : (NQT > 4 ? 2 : 1)))) void k_attn_split(AttnArgs a) {
  constexpr int NSP = LA + 1;
  constexpr int PPW = (16 + NQT - 1) / NQT;  // pieces per wave and pair
  __shared__ __align__(16) unsigned char ring[NSP * kPairBytes];
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  // sequences vary fastest, so the runs that exist (all first runs, then the
  // second runs of longer sequences, ...) come first in dispatch order
  const int b = blockIdx.x, split = blockIdx.y, kvh = blockIdx.z;
  const int qt = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.Hq / a.Hkv;
  const int NQ = a.W * G;
  const bool direct = a.max_splits == 1;
  const int kps = a.pages_per_split * kBlock;
  const int k0 = split * kps;
  const int qi = qt * 16 + r;
  const int first = k0 / kBlock;
  // the block ids of the run's pages (one per lane, clamped to the table) and
  // the Q fragments are loaded together with the sequence length, not after it
  const int bt_row = a.bt_div > 1 ? b / a.bt_div : b;
  int bt = a.block_table[(size_t)bt_row * a.max_blocks +
                         min(first + min(lane, a.pages_per_split - 1), a.max_blocks - 1)];

  // Q^T operand of this wave's tile: lane (g, r) holds dims kb*32 + 8g .. +8 of
  // query column qi as bf16 hi and lo (absent columns: zeros).  The loads go
  // out before the run is known to exist; a run past the sequence leaves
  // without waiting for them.
  float4 v[8];
  {
    const int qc = qi < NQ ? qi : 0;
    const int wr = qc / G, hg = qc - wr * G;
    const float* src = a.q + ((size_t)(b * a.W + wr) * a.Hq + kvh * G + hg) * kHeadDim + g * 8;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      v[2 * kb] = *(const float4*)(src + kb * 32);
      v[2 * kb + 1] = *(const float4*)(src + kb * 32 + 4);
    }
  }
  const int n_keys = attn_keys(a, b);
  // keys this lane's query column sees: all of them, or for a causal row (the
  // causal window, the re-fed rows) the prefix and the window rows up to its
  // own (at least one key)
  const int crows = a.causal_rows ? min(max(a.causal_rows[b], 0), a.W) : (a.causal ? a.W : 0);
  const int wrow = (qi < NQ ? qi : 0) / G;
  const int kcol = wrow < crows ? max(min(n_keys, a.prefix_len[b] + wrow + 1), min(n_keys, 1)) : n_keys;
  if (k0 >= n_keys) {  // uniform over the workgroup
    if (direct && qi < NQ && (g & 1) == 0) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int dt = 0; dt < 8; ++dt) attn_store8(a, b, kvh, qi, dt * 16 + 4 * g, z);
    }
    return;
  }
  bf16x8 qh[4], ql[4];
  {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float x[8] = {v[2 * kb].x, v[2 * kb].y, v[2 * kb].z, v[2 * kb].w,
                          v[2 * kb + 1].x, v[2 * kb + 1].y, v[2 * kb + 1].z, v[2 * kb + 1].w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_hi_lo(qi < NQ ? x[e] : 0.f, hi[e], lo[e]);
      const u32x4 H = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                       hi[6] | (hi[7] << 16)};
      const u32x4 L = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                       lo[6] | (lo[7] << 16)};
      qh[kb] = __builtin_bit_cast(bf16x8, H);
      ql[kb] = __builtin_bit_cast(bf16x8, L);
    }
  }
  const int k1 = min(n_keys, k0 + kps);
  const int npages = (k1 - k0 + kBlock - 1) / kBlock;  // 1 .. pages_per_split (<= 64)
  bt = bt < 0 ? 0 : (bt >= a.num_blocks ? a.num_blocks - 1 : bt);

  // copies: this wave's pieces of pair c (a page past the run repeats the
  // last one into a slot nobody reads before it is refilled, or that only
  // masked keys read)
  const int npairs = (npages + 1) >> 1;
  const uint32_t cache_bytes = (uint32_t)a.num_blocks * a.Hkv * (kPageBytes / 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.kc, cache_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vc, cache_bytes);
  uint32_t psrc[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) psrc[i] = page_piece_src(min(qt + NQT * i, 15) & 7, lane);
  auto copy_pair = [&](int c) {
    unsigned char* slot = ring + (c % NSP) * kPairBytes;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int piece = min(qt + NQT * i, 15);
      const int h = piece >> 3, q = piece & 7;
      const int blk = __builtin_amdgcn_readlane(bt, min(2 * c + h, npages - 1));
      const uint32_t base = ((uint32_t)blk * a.Hkv + kvh) * (kPageBytes / 2);
      if (q < 4) lds_copy16(rk, psrc[i], base, slot + h * kPageBytes + q * 1024);
      else lds_copy16(rv, psrc[i], base, slot + h * kPageBytes + q * 1024);
    }
  };

  AttnState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < LA; ++c) copy_pair(c);
  for (int c = 0; c < npairs; ++c) {
    wait_vmcnt<(LA - 1) * PPW>();  // my pieces of pair c (LA - 1 pairs' pieces follow them)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): my reads of pair c - 1 are done
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    copy_pair(c + LA);  // into the slot of pair c - 1
    PairRegs pr;
    read_pair(ring + (c % NSP) * kPairBytes, pr);
    const int p0 = k0 + 2 * c * kBlock;
    attn_pair(pr, k1 - p0, min(k1, kcol) - p0, qh, ql, st);
  }
  float lsum = st.l;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  if (direct) {
    // lane (g, r) holds dims dt*16 + 4g .. +4 of column qi; even g lanes take
    // the next 4 dims from lane (g+1, r) and store 8
    const float inv = 1.f / lsum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = st.acc[dt][e] * inv;
        v[4 + e] = __shfl_xor(v[e], 16);
      }
      if (qi < NQ && (g & 1) == 0) attn_store8(a, b, kvh, qi, dt * 16 + 4 * g, v);
    }
  } else {
    const size_t unit = ((size_t)b * a.Hkv + kvh) * a.max_splits + split;
    if (g == 0) {
      float2* ml = (float2*)a.part_ml + unit * a.nqp + qi;
      *ml = make_float2(st.m, lsum);
    }
    float* po = a.part_o + (unit * a.nqp + qi) * kHeadDim + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *(f32x4*)(po + dt * 16) = st.acc[dt];
  }
  // copies still in flight land in LDS this workgroup owns until it ends
  __builtin_amdgcn_s_waitcnt(0);
}

// Merge of the runs.  A workgroup of 256 threads takes one query column of a
// (sequence, KV head): thread (chunk c of 4 dims, group j of 8) combines runs
// j, j+8, j+16, ... (eight at a time, all loads of a group in flight together),
// then the 8 groups are combined across lanes in a fixed butterfly, so the
// result does not depend on timing.  Combination is the usual log-sum-exp
// rescaling of (max, sum, unnormalised O).
constexpr int kMergeGroups = 8;
// Up to this many runs per sequence the column-group merge serves.
constexpr int kMergeColsMaxRuns = 32;

struct MergeAcc {
  float m, den;
  float4 num;
};

__device__ __forceinline__ MergeAcc merge_pair(const MergeAcc& x, const MergeAcc& y) {
  MergeAcc r;
  r.m = fmaxf(x.m, y.m);
  const float sx = x.m == -INFINITY ? 0.f : exp2f(x.m - r.m);
  const float sy = y.m == -INFINITY ? 0.f : exp2f(y.m - r.m);
  r.den = x.den * sx + y.den * sy;
  r.num.x = x.num.x * sx + y.num.x * sy;
  r.num.y = x.num.y * sx + y.num.y * sy;
  r.num.z = x.num.z * sx + y.num.z * sy;
  r.num.w = x.num.w * sx + y.num.w * sy;
  return r;
}

__device__ __forceinline__ MergeAcc shfl_xor_acc(const MergeAcc& x, int mask) {
  MergeAcc r;
  r.m = __shfl_xor(x.m, mask);
  r.den = __shfl_xor(x.den, mask);
  r.num.x = __shfl_xor(x.num.x, mask);
  r.num.y = __shfl_xor(x.num.y, mask);
  r.num.z = __shfl_xor(x.num.z, mask);
  r.num.w = __shfl_xor(x.num.w, mask);
  return r;
}

// MB: runs per group loaded at once (the host picks the smallest power of two
// with MB * kMergeGroups >= max_splits, so no group loads clamped duplicates
// beyond its last batch).
template <int MB>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  constexpr int kMergeBatch = MB;
  const int qi = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 3;                              // run group
  const int c4 = (threadIdx.x >> 6) * 8 + (lane & 7);  // 4-dim chunk
  const int kps = a.pages_per_split * kBlock;
  const size_t base = ((size_t)b * a.Hkv + kvh) * a.max_splits;
  const float2* ml = (const float2*)a.part_ml;
  MergeAcc acc;
  acc.m = -INFINITY;
  acc.den = 0.f;
  acc.num = make_float4(0.f, 0.f, 0.f, 0.f);
  // slot addresses do not depend on the sequence length (it only masks), so
  // the loads need not wait for it
  const int ns = (attn_keys(a, b) + kps - 1) / kps;
  for (int s0 = j; s0 < a.max_splits; s0 += kMergeGroups * kMergeBatch) {
    float2 m[kMergeBatch];
    float4 o[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int s = s0 + i * kMergeGroups;
      const size_t u = base + (s < a.max_splits ? s : 0);  // a slot inside the buffer
      m[i] = ml[u * a.nqp + qi];
      o[i] = *(const float4*)(a.part_o + (u * a.nqp + qi) * kHeadDim + 4 * c4);
    }
    float bm = acc.m;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (s0 + i * kMergeGroups < ns) bm = fmaxf(bm, m[i].x);
    const float sc = acc.m == -INFINITY ? 0.f : exp2f(acc.m - bm);
    acc.den *= sc;
    acc.num.x *= sc; acc.num.y *= sc; acc.num.z *= sc; acc.num.w *= sc;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (s0 + i * kMergeGroups < ns) {
        const float w = m[i].x == -INFINITY ? 0.f : exp2f(m[i].x - bm);
        acc.den += w * m[i].y;
        acc.num.x += w * o[i].x; acc.num.y += w * o[i].y;
        acc.num.z += w * o[i].z; acc.num.w += w * o[i].w;
      }
    }
    acc.m = bm;
  }
  // groups j and j^1, j^2, j^4 (lanes 8, 16, 32 apart); both partners compute
  // the same sums, so every lane of a chunk ends with one identical result
  acc = merge_pair(acc, shfl_xor_acc(acc, 8));
  acc = merge_pair(acc, shfl_xor_acc(acc, 16));
  acc = merge_pair(acc, shfl_xor_acc(acc, 32));
  const float inv = acc.den > 0.f ? 1.f / acc.den : 0.f;
  float v[8];
  v[0] = acc.num.x * inv; v[1] = acc.num.y * inv; v[2] = acc.num.z * inv; v[3] = acc.num.w * inv;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[4 + e] = __shfl_xor(v[e], 1);
  if (j == 0 && (c4 & 1) == 0) attn_store8(a, b, kvh, qi, 4 * c4, v);
}

// Merge for few runs (at most 16, or 32 with 16 sequences and more): a
// workgroup takes 8 query columns of a (sequence, KV head); thread (column j
// of 8, chunk of 4 dims) combines every run of its column in run order, MB
// runs' loads in flight together.  Many short workgroups of one column each
// (k_attn_merge) cost more dispatch than they save once the runs are few.
template <int MB>
__global__ __launch_bounds__(256) void k_attn_merge_cols(AttnArgs a) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int qi = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int c4 = threadIdx.x & 31;
  const int NQ = a.W * (a.Hq / a.Hkv);
  const int kps = a.pages_per_split * kBlock;
  const size_t base = ((size_t)b * a.Hkv + kvh) * a.max_splits;
  const float2* ml = (const float2*)a.part_ml;
  const int ns = (attn_keys(a, b) + kps - 1) / kps;
  const int q = qi < NQ ? qi : NQ - 1;  // a column past the last repeats it (not stored)
  float bm = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ns; s0 += MB) {
    float2 m[MB];
    float4 o[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const size_t u = base + (s0 + i < a.max_splits ? s0 + i : 0);
      m[i] = ml[u * a.nqp + q];
      o[i] = *(const float4*)(a.part_o + (u * a.nqp + q) * kHeadDim + 4 * c4);
    }
    float nm = bm;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (s0 + i < ns) nm = fmaxf(nm, m[i].x);
    const float sc = bm == -INFINITY ? 0.f : exp2f(bm - nm);
    den *= sc;
    num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (s0 + i < ns) {
        const float w = m[i].x == -INFINITY ? 0.f : exp2f(m[i].x - nm);
        den += w * m[i].y;
        num.x += w * o[i].x; num.y += w * o[i].y;
        num.z += w * o[i].z; num.w += w * o[i].w;
      }
    }
    bm = nm;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float v[8];
  v[0] = num.x * inv; v[1] = num.y * inv; v[2] = num.z * inv; v[3] = num.w * inv;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[4 + e] = __shfl_xor(v[e], 1);
  if (qi < NQ && (c4 & 1) == 0) attn_store8(a, b, kvh, qi, 4 * c4, v);
}

// Runs of pages_per_split pages: two pages per run while that keeps the grid
// within about 640 workgroups, longer runs beyond.  Many short runs cost
// workgroup launches and partial results (24 KB each, written and merged);
// few long ones leave compute units idle and make long dependent chains.
void plan_attention(int B, int Hkv, int max_len, int* pages_per_split, int* max_splits) {
  const int max_pages = (max_len + kBlock - 1) / kBlock;
  int pps = 2;
  // a single sequence has no empty runs in its grid: keep it within the 512
  // workgroups that are resident together (two per compute unit), so that no
  // run waits for a second round (prefix 32768: 514 runs of 8 pages, the step
  // 2.78 ms, against 258 of 16, 2.71 ms)
  const long lim = B == 1 ? 2L * cu_count() : 640;
  while (pps < 64 && (long)B * Hkv * ((max_pages + pps - 1) / pps) > lim) pps *= 2;
  // at least 8 pages per run while 128 runs remain: INT4 batch 8 at P 1280
  // (336 runs of 4 pages) measured 4.15 -> 4.07 ms per step with runs of 8
  while (pps < 8 && (long)B * Hkv * ((max_pages + 2 * pps - 1) / (2 * pps)) >= 128) pps *= 2;
  if (pps > max_pages) pps = max_pages;
  if (pps < 1) pps = 1;
  *pages_per_split = pps;
  *max_splits = (max_pages + pps - 1) / pps;
}

template <int NQT>
static void launch_split(const AttnArgs& a, bool deep, dim3 grid, dim3 block, hipStream_t s) {
  if (deep) hipLaunchKernelGGL((k_attn_split<NQT, 3>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_attn_split<NQT, 1>), grid, block, 0, s, a);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int nqt = a.nqp / 16;
  const dim3 grid(a.B, a.max_splits, a.Hkv), block(nqt * 64);
  // a deep ring for long runs, a short one for the two-page runs of short
  // sequences
  const bool deep = a.pages_per_split > 2;
  switch (nqt) {
    case 1: launch_split<1>(a, deep, grid, block, s); break;
    case 2: launch_split<2>(a, deep, grid, block, s); break;
    case 3: launch_split<3>(a, deep, grid, block, s); break;
    case 4: launch_split<4>(a, deep, grid, block, s); break;
    case 5: launch_split<5>(a, deep, grid, block, s); break;
    case 6: launch_split<6>(a, deep, grid, block, s); break;
    case 7: launch_split<7>(a, deep, grid, block, s); break;
    default: launch_split<8>(a, deep, grid, block, s); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  const int NQ = a.W * (a.Hq / a.Hkv);
  // the column-group merge for few runs, or for up to 32 where the per-column
  // grid is large (measured: batch 8 with 21 runs 6.3 against 4.8 us per-column,
  // batch 16 with 18 runs faster by column groups)
  if (a.max_splits <= kMergeColsMaxRuns / 2 || (a.max_splits <= kMergeColsMaxRuns && a.B >= 16)) {
    const dim3 cgrid((NQ + 7) / 8, a.Hkv, a.B);
    if (a.max_splits <= 4) hipLaunchKernelGGL(k_attn_merge_cols<4>, cgrid, dim3(256), 0, s, a);
    else if (a.max_splits <= 8) hipLaunchKernelGGL(k_attn_merge_cols<8>, cgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_attn_merge_cols<16>, cgrid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const dim3 mgrid(NQ, a.Hkv, a.B);
  const int per_group = (a.max_splits + kMergeGroups - 1) / kMergeGroups;
  if (per_group <= 1) hipLaunchKernelGGL(k_attn_merge<1>, mgrid, dim3(256), 0, s, a);
  else if (per_group <= 2) hipLaunchKernelGGL(k_attn_merge<2>, mgrid, dim3(256), 0, s, a);
  else if (per_group <= 4) hipLaunchKernelGGL(k_attn_merge<4>, mgrid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_attn_merge<8>, mgrid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace la
