// Sampled selection at the end of a window step: temperature, top-p (nucleus)
// and a counter-based random draw, in place of the greedy argmax.
//
// The RK3588 page ("LocateAnything-3B for RK3588 (RKLLM + RKNN)", "Usage (on
// the board)" and "Evaluation") runs the model with temperature 0.7, top-p 0.9
// and repetition penalty 1.1, and the Jetson page (Part 1 section 1.4) notes
// that the sampler falls back to the argmax when the temperature is not
// positive.  Per row of logits z (after the repetition penalty):
//   p_v ~ exp(z_v / T);
//   the nucleus is the shortest run of the vocabulary ordered by z descending
//   (equal logits: lower id first) whose probability reaches top_p;
//   a uniform u in [0, 1) selects, among the kept ids in ascending id order,
//   the first whose running kept probability exceeds u times the kept total.
// u is the top 24 bits of the first word of Philox4x32-10 (Salmon et al.,
// SC 2011) at counter (row, offset lo, offset hi, 0) and key (seed lo, seed hi).
//
// One workgroup of 16 waves per row.  Probabilities are exp2 of the scaled
// logit distance to the row's maximum, held as 40-bit fixed point in 64-bit
// integers, so every sum is exact and the result does not depend on the order
// of the additions.  The nucleus boundary is found by radix selection over the
// order-preserving 32-bit key of z, four bits per pass, each thread keeping its
// 16 bin sums in private LDS slots (bin-major, so the lanes of a wave hit
// distinct banks whatever their digits: one read-modify-write per element);
// wave b then sums bin b over the threads.  Ties on the boundary key and the
// final draw are located by per-wave contiguous scans in id order.  Every
// pass reads the row (V fp32) again from L2.
#include "la_internal.hpp"

namespace la {

namespace {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;
constexpr float kFix = 1099511627776.0f;  // 2^40
constexpr size_t kSampleLds = (size_t)16 * kSampleThreads * 8;  // private bins [16][threads] uint64

__device__ __forceinline__ uint32_t philox_first_word(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                      uint32_t k0, uint32_t k1) {
  // ten rounds; the key advances between rounds
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  return c0;
}

// Order-preserving key of a finite float: a larger value gives a larger key.
__device__ __forceinline__ uint32_t zkey(float z) {
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d), hi = __shfl_up((uint32_t)(v >> 32), d);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor_u64(v, o);
  return v;
}
// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t t = shfl_up_u64(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

struct SampleShared {
  float fmax[kSampleWaves];
  int imax[kSampleWaves];
  uint64_t bins[16];
  uint64_t wsum[kSampleWaves];
  uint64_t total;
  float zmax;
  int arg;
  uint32_t prefix, pmask;
  uint64_t above, target;
  int seg_wave;    // the segment holding a crossing
  uint64_t seg_run;
  int found;       // the id found there, and the running mass at it
  uint64_t found_run;
};

}  // namespace

__global__ __launch_bounds__(kSampleThreads) void k_sample(SampleArgs a) {
  __shared__ SampleShared sh;
  extern __shared__ __align__(16) uint64_t pbins[];  // [16][kSampleThreads]
  const int m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = a.V;
  if (a.flags && a.flags[m]) {
    if (tid == 0) {
      a.ids[m] = -1;
      if (a.sel_gap) a.sel_gap[m] = 0.f;
      if (a.err) atomicOr(a.err, a.flags[m]);
    }
    return;
  }
  const float* zr = a.logits + (size_t)m * a.ldz;
  const uint32_t* bits = a.rep_bits ? a.rep_bits + (size_t)(m / a.rep_rows) * a.rep_words : nullptr;
  auto zpen = [&](int v) {
    float z = zr[v];
    if (bits && ((bits[v >> 5] >> (v & 31)) & 1u)) z = z > 0.f ? z / a.rep_theta : z * a.rep_theta;
    return z;
  };

  // pass 0: the row's largest logit (lowest id on a tie)
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int v = tid; v < V; v += kSampleThreads) {
    const float z = zpen(v);
    if (z > best) {  // ids rise along a thread's stride: the first of a tie stays
      best = z;
      bi = v;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(bi, o);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (lane == 0) {
    sh.fmax[wave] = best;
    sh.imax[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float b = -INFINITY;
    int i = 0x7FFFFFFF;
    for (int w = 0; w < kSampleWaves; ++w)
      if (sh.fmax[w] > b || (sh.fmax[w] == b && sh.imax[w] < i)) {
        b = sh.fmax[w];
        i = sh.imax[w];
      }
    sh.zmax = b;
    sh.arg = i;
  }
  __syncthreads();
  const float zmax = sh.zmax;
  if (!(a.temperature > 0.f)) {  // greedy
    if (tid == 0) {
      a.ids[m] = sh.arg;
      if (a.sel_gap) a.sel_gap[m] = 0.f;
    }
    return;
  }
  const float scale = 1.4426950408889634f / a.temperature;  // log2(e) / T
  auto qfix = [&](float z) -> uint64_t {
    const float p = __builtin_amdgcn_exp2f((z - zmax) * scale);  // in [0, 1]
    return (uint64_t)(p * kFix);
  };

  // passes 1..8: radix selection of the nucleus boundary key, 4 bits a pass
  // (pass 1 also yields the total)
  uint32_t prefix = 0, pmask = 0;
  uint64_t above = 0, target = 0;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 28 - 4 * pass;
#pragma unroll
    for (int b = 0; b < 16; ++b) pbins[b * kSampleThreads + tid] = 0;
    for (int v = tid; v < V; v += kSampleThreads) {
      const float z = zpen(v);
      const uint32_t k = zkey(z);
      if ((k & pmask) != prefix) continue;
      const uint32_t d = (k >> shift) & 15u;
      pbins[d * kSampleThreads + tid] += qfix(z);
    }
    __syncthreads();
    {
      // wave b: bin b over every thread (16 slots per lane, fixed order)
      static_assert(kSampleWaves == 16, "one wave per bin");
      uint64_t s = 0;
#pragma unroll
      for (int i = 0; i < kSampleThreads / 64; ++i) s += pbins[wave * kSampleThreads + i * 64 + lane];
      s = wave_sum_u64(s);
      if (lane == 0) sh.bins[wave] = s;
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t H[16], all = 0;
      for (int b = 0; b < 16; ++b) {
        H[b] = sh.bins[b];
        all += H[b];
      }
      if (pass == 0) {
        // the nucleus must hold ceil(top_p * total) of the fixed-point mass
        double t = ceil((double)a.top_p * (double)all);
        uint64_t tt = t < 1.0 ? 1ull : (uint64_t)t;
        if (tt > all) tt = all;
        sh.total = all;
        sh.target = tt;
        sh.above = 0;
      }
      uint64_t cum = sh.above;
      int chosen = 0;
      for (int b = 15; b >= 0; --b) {
        if (cum + H[b] >= sh.target) {
          chosen = b;
          break;
        }
        cum += H[b];
      }
      sh.above = cum;
      sh.prefix = prefix | ((uint32_t)chosen << shift);
      sh.pmask = pmask | (15u << shift);
    }
    __syncthreads();
    prefix = sh.prefix;
    pmask = sh.pmask;
    above = sh.above;
    target = sh.target;
  }
  const uint32_t kappa = prefix;

  // Per-wave contiguous segments in id order: wave w scans ids
  // [w * seg, (w + 1) * seg) 64 at a time.  find_first returns the first id
  // whose running mass (mass(v) summed over ids up to v, plus `base`)
  // reaches `need`, and that running mass.
  const int seg = ((V + kSampleWaves - 1) / kSampleWaves + 63) / 64 * 64;
  auto find_first = [&](auto mass, uint64_t base, uint64_t need, int& out_id, uint64_t& out_run) {
    // segment totals
    const int v0 = wave * seg, v1 = min(V, v0 + seg);
    uint64_t s = 0;
    for (int v = v0 + lane; v < v1; v += 64) s += mass(v);
    s = wave_sum_u64(s);
    if (lane == 0) sh.wsum[wave] = s;
    __syncthreads();
    if (tid == 0) {
      // the segment holding the crossing, and the mass before it
      uint64_t run = base;
      int w = 0;
      for (; w < kSampleWaves - 1; ++w) {
        if (run + sh.wsum[w] >= need) break;
        run += sh.wsum[w];
      }
      sh.seg_wave = w;
      sh.seg_run = run;
    }
    __syncthreads();
    if (wave == sh.seg_wave) {
      uint64_t run = sh.seg_run;
      int id = -1;
      uint64_t at = 0;
      for (int vb = v0; vb < v1 && id < 0; vb += 64) {
        const int v = vb + lane;
        const uint64_t q = v < v1 ? mass(v) : 0ull;
        const uint64_t inc = wave_scan_u64(q) + run;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(v < v1 && q > 0 && inc >= need);
        if (hit) {
          const int l = __builtin_ffsll((long long)hit) - 1;
          id = vb + l;
          const uint32_t lo = __shfl((uint32_t)inc, l), hi = __shfl((uint32_t)(inc >> 32), l);
          at = ((uint64_t)hi << 32) | lo;
        }
        const uint32_t lo = __shfl((uint32_t)inc, 63), hi = __shfl((uint32_t)(inc >> 32), 63);
        run = ((uint64_t)hi << 32) | lo;
      }
      if (lane == 0) {
        sh.found = id;
        sh.found_run = at;
      }
    }
    __syncthreads();
    out_id = sh.found;
    out_run = sh.found_run;
    __syncthreads();
  };

  // ties on the boundary key: the lowest ids first, until the nucleus mass
  int cut_id;
  uint64_t kept_total;
  find_first([&](int v) -> uint64_t {
               const float z = zpen(v);
               return zkey(z) == kappa ? qfix(z) : 0ull;
             },
             above, target, cut_id, kept_total);

  // the draw
  uint64_t off = a.offset_dev ? *a.offset_dev : a.offset;
  const uint32_t u24 = philox_first_word((uint32_t)m, (uint32_t)off, (uint32_t)(off >> 32), 0u,
                                         (uint32_t)a.seed, (uint32_t)(a.seed >> 32)) >> 8;
  // floor(u * kept_total) with u = u24 / 2^24, exactly: kept_total = A 2^24 + B
  const uint64_t t = (kept_total >> 24) * u24 + (((kept_total & 0xFFFFFFull) * u24) >> 24);
  int sel;
  uint64_t run_at;
  find_first([&](int v) -> uint64_t {
               const float z = zpen(v);
               const uint32_t k = zkey(z);
               const bool kept = k > kappa || (k == kappa && v <= cut_id);
               return kept ? qfix(z) : 0ull;
             },
             0ull, t + 1, sel, run_at);
  if (tid == 0) {
    a.ids[m] = sel;
    if (a.sel_gap) a.sel_gap[m] = sel >= 0 ? zpen(sel) - zmax : 0.f;
  }
}

__global__ void k_offset_advance(uint64_t* offset) {
  if (threadIdx.x == 0) *offset += 1;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  static bool attr = false;  // the private bins need LDS beyond the static default
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_sample, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kSampleLds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(k_sample, dim3(a.M), dim3(kSampleThreads), kSampleLds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.offset_dev || !(a.temperature > 0.f)) return e;
  hipLaunchKernelGGL(k_offset_advance, dim3(1), dim3(64), 0, s, const_cast<uint64_t*>(a.offset_dev));
  return hipGetLastError();
}

}  // namespace la
