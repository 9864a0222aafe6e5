// Block-masked GQA attention of the window rows over the paged bf16 KV cache.
//
// Every window row of sequence b attends to cache slots 0 .. P_b+W-1: the
// prefix lies before it and the window is bidirectional, so one key bound
// serves all rows and no per-element mask exists ("LocateAnything-3B for RK3588
// (RKLLM + RKNN)", "How it differs from the original", item 1; the Jetson
// page, section 1.3, block mask).
//
// Work split: one wave per (sequence, KV head, run of pages).  The 8 query
// heads of a KV head times W window rows form up to 64 query columns that share
// every K/V page, so a page is read once for all of them:
//   S^T[key, query] = K_page . Q^T        16x16x32 bf16 matrix-core steps, Q split
//                                         into bf16 hi + lo columns (K is exact bf16)
//   online softmax per query column       exp2 on pre-scaled scores, one max per page
//   O^T[d, query] += V_page^T . P^T       16x16x16 steps; P split into hi + lo; the
//                                         S^T accumulator layout is exactly the P^T
//                                         operand layout, so P never leaves registers
// V pages are stored dim-major ([D][16 keys]) so a V^T operand fragment is one
// 8-byte load.  Each wave writes (max, sum, unnormalised O) for its run; a merge
// kernel combines the runs with the usual log-sum-exp rescaling in a fixed order.
#include "la_internal.hpp"

namespace la {

__device__ __forceinline__ int attn_keys(const AttnArgs& a, int b) {
  int n = a.prefix_len[b] + a.W;
  if (n > a.cap) n = a.cap;
  if (n < 0) n = 0;
  return n;
}

template <int NQT>
__global__ __launch_bounds__(256) void k_attn_partial(AttnArgs a) {
  __shared__ bf16x8 qf[2 * NQT][4][64];
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int G = a.Hq / a.Hkv;
  const int NQ = a.W * G;
  const int D = kHeadDim;
  const int n_keys = attn_keys(a, b);
  const int kps = a.pages_per_split * kBlock;
  const int split0 = blockIdx.x * 4;
  if (split0 * kps >= n_keys) return;  // uniform over the workgroup

  // Q^T operand fragments, hi tiles [0, NQT) and lo tiles [NQT, 2 NQT).
  for (int idx = threadIdx.x; idx < NQT * 16 * 16; idx += 256) {
    const int qi = idx >> 4, c = idx & 15;
    const int kb = c >> 2, gg = c & 3;
    float v[8];
    if (qi < NQ) {
      const int wr = qi / G, hg = qi - wr * G;
      const float* src = a.q + ((size_t)(b * a.W + wr) * a.Hq + kvh * G + hg) * D + c * 8;
      const float4 v0 = *(const float4*)src, v1 = *(const float4*)(src + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_hi_lo(v[e], hi[e], lo[e]);
    const u32x4 H = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                     hi[6] | (hi[7] << 16)};
    const u32x4 L = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                     lo[6] | (lo[7] << 16)};
    const int ct = qi >> 4, fl = gg * 16 + (qi & 15);
    qf[ct][kb][fl] = __builtin_bit_cast(bf16x8, H);
    qf[NQT + ct][kb][fl] = __builtin_bit_cast(bf16x8, L);
  }
  __syncthreads();

  const int split = split0 + wave;
  const int k0 = split * kps;
  if (k0 >= n_keys) return;
  const int k1 = min(n_keys, k0 + kps);
  const float sl2 = 0.08838834764831845f * 1.4426950408889634f;  // log2(e) / sqrt(128)

  float mrun[NQT], lrun[NQT];
  f32x4 acc[8][NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // K and V of one page for this lane: K rows are keys, V^T rows are dims
  auto load_page = [&](int p0, bf16x8 (&ka)[4], s16x4 (&va)[8]) {
    int blk = a.block_table[(size_t)b * a.max_blocks + p0 / kBlock];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const uint16_t* Kp = a.kc + ((size_t)blk * a.Hkv + kvh) * kBlock * D;
    const uint16_t* Vp = a.vc + ((size_t)blk * a.Hkv + kvh) * D * kBlock;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) ka[kb] = *(const bf16x8*)(Kp + r * D + kb * 32 + g * 8);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = *(const s16x4*)(Vp + (dt * 16 + r) * kBlock + 4 * g);
  };
  bf16x8 ka[4], kn[4];
  s16x4 va[8], vn[8];
  load_page(k0, ka, va);
  for (int p0 = k0; p0 < k1; p0 += kBlock) {
    // the next page is in flight while this one is processed
    if (p0 + kBlock < k1) load_page(p0 + kBlock, kn, vn);
    const int nvalid = k1 - p0;
    if (nvalid < kBlock) {
      // keys past the bound: zero their values (unused slots may hold anything)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g + e >= nvalid) va[dt][e] = 0;
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x4 sh = {0.f, 0.f, 0.f, 0.f}, sl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sh = mfma_16x16x32(ka[kb], qf[qt][kb][lane], sh);
        sl = mfma_16x16x32(ka[kb], qf[NQT + qt][kb][lane], sl);
      }
      float s[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = (sh[e] + sl[e]) * sl2;
        if (4 * g + e >= nvalid) s[e] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[qt], mx);
      const float alpha = exp2f(mrun[qt] - mnew);
      float p[4], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = exp2f(s[e] - mnew);
        ps += p[e];
      }
      lrun[qt] = lrun[qt] * alpha + ps;
      mrun[qt] = mnew;
      s16x4 ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t h, l;
        split_hi_lo(p[e], h, l);
        ph[e] = (short)h;
        pl[e] = (short)l;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        acc[dt][qt] *= alpha;
        acc[dt][qt] = mfma_16x16x16(va[dt], ph, acc[dt][qt]);
        acc[dt][qt] = mfma_16x16x16(va[dt], pl, acc[dt][qt]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) ka[kb] = kn[kb];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = vn[dt];
  }

  const size_t unit = ((size_t)b * a.Hkv + kvh) * a.max_splits + split;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float l = lrun[qt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int qi = qt * 16 + r;
    if (g == 0) {
      float2* ml = (float2*)a.part_ml + unit * a.nqp + qi;
      *ml = make_float2(mrun[qt], l);
    }
    float* po = a.part_o + (unit * a.nqp + qi) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *(f32x4*)(po + dt * 16) = acc[dt][qt];
  }
}

// One workgroup per (query column, KV head, sequence): 512 threads = 128 dims x
// 4 interleaved subsets of the splits; the log-sum-exp weights are computed once
// in LDS and the four partial sums are added in a fixed order.
__global__ __launch_bounds__(512) void k_attn_merge(AttnArgs a) {
  extern __shared__ float wsh[];  // [max_splits] weights
  __shared__ float red[512];
  __shared__ float so[kHeadDim];
  __shared__ float s_M, s_den;
  const int qi = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, d = tid & 127, part = tid >> 7;
  const int G = a.Hq / a.Hkv;
  const int n_keys = attn_keys(a, b);
  const int kps = a.pages_per_split * kBlock;
  const int ns = (n_keys + kps - 1) / kps;
  const size_t base = ((size_t)b * a.Hkv + kvh) * a.max_splits;
  const float2* ml = (const float2*)a.part_ml;
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += 512) mx = fmaxf(mx, ml[(base + s) * a.nqp + qi].x);
  red[tid] = mx;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float den = 0.f;
  for (int s = tid; s < ns; s += 512) {
    const float2 v = ml[(base + s) * a.nqp + qi];
    const float w = exp2f(v.x - M);
    wsh[s] = w;
    den += w * v.y;
  }
  red[tid] = den;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) s_den = red[0];
  __syncthreads();
  float num = 0.f;
  const float* po = a.part_o + ((base)*a.nqp + qi) * kHeadDim + d;
  const size_t sstride = (size_t)a.nqp * kHeadDim;
  int s = part;
  for (; s + 12 < ns; s += 16) {
    const float o0 = po[(size_t)s * sstride], o1 = po[(size_t)(s + 4) * sstride];
    const float o2 = po[(size_t)(s + 8) * sstride], o3 = po[(size_t)(s + 12) * sstride];
    num += wsh[s] * o0;
    num += wsh[s + 4] * o1;
    num += wsh[s + 8] * o2;
    num += wsh[s + 12] * o3;
  }
  for (; s < ns; s += 4) num += wsh[s] * po[(size_t)s * sstride];
  red[tid] = num;
  __syncthreads();
  (void)s_M;
  if (part == 0) {
    const float o = ns > 0 ? (red[d] + red[d + 128] + red[d + 256] + red[d + 384]) / s_den : 0.f;
    const int wr = qi / G, hg = qi - wr * G;
    const int row = b * a.W + wr;
    const int h = kvh * G + hg;
    const int ldo = a.Hq * kHeadDim;
    if (a.out) a.out[(size_t)row * ldo + h * kHeadDim + d] = o;
    so[d] = o;
  }
  if (a.out_apack) {
    __syncthreads();
    if (tid < 16) {
      const int wr = qi / G, hg = qi - wr * G;
      const int row = b * a.W + wr;
      const int h = kvh * G + hg;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = so[tid * 8 + e];
      apack_store_chunk(a.out_apack, a.Hq * kHeadDim, row, (h * kHeadDim) / 8 + tid, v, a.out_int4);
    }
  }
}

void plan_attention(int B, int Hkv, int max_len, int* pages_per_split, int* max_splits) {
  const int max_pages = (max_len + kBlock - 1) / kBlock;
  const long total = (long)B * Hkv * max_pages;
  int pps = (int)((total + 1023) / 1024);  // about 1024 waves in flight
  if (pps < 2) pps = 2;                     // at least two pages: the second overlaps the first
  if (pps > max_pages) pps = max_pages > 0 ? max_pages : 1;
  *pages_per_split = pps;
  *max_splits = (max_pages + pps - 1) / pps;
  if (*max_splits < 1) *max_splits = 1;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int nqt = a.nqp / 16;
  const dim3 grid((a.max_splits + 3) / 4, a.Hkv, a.B);
  switch (nqt) {
    case 1: hipLaunchKernelGGL(k_attn_partial<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_attn_partial<2>, grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_attn_partial<3>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_attn_partial<4>, grid, dim3(256), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int NQ = a.W * (a.Hq / a.Hkv);
  hipLaunchKernelGGL(k_attn_merge, dim3(NQ, a.Hkv, a.B), dim3(512), (size_t)a.max_splits * 4, s, a);
  return hipGetLastError();
}

}  // namespace la
