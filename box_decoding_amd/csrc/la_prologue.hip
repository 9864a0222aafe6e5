// Step prologue: embedding gather (bf16 rows or INT4 group-32 rows), the RoPE
// cos/sin of every window position and per-row data-error flags.
#include "la_internal.hpp"

namespace la {

// Where row t's input comes from: its index in ids / embeds, or -1 for a
// padding row of a prefill (rows past in_w of each sequence).
__device__ __forceinline__ int prologue_src(const PrologueArgs& a, int t) {
  if (a.in_w <= 0) return t;
  const int b = t / a.W, j = t - b * a.W;
  return j < a.in_w ? b * a.in_w + j : -1;
}

// A window id's data error: outside [0, vocab), except a negative id that
// takes a spliced input row.
__device__ __forceinline__ bool prologue_id_bad(const PrologueArgs& a, int id) {
  return id >= a.emb.n || (id < 0 && !a.embeds);
}

// One workgroup per window row t.
__global__ __launch_bounds__(256) void k_prologue(PrologueArgs a) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (t >= a.T) {
    // the extra workgroups clear the front-half launch's flags and words
    const int n4 = a.n_zero / 4, nb = gridDim.x - a.T;
    uint4* z = (uint4*)a.zero;
    for (int i = (t - a.T) * 256 + tid; i < n4; i += nb * 256) z[i] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  int id_bad = 0;
  if (a.ids) {
    const int src = prologue_src(a, t);
    const int id = src >= 0 ? a.ids[src] : 0;
    const int K = a.emb.k;
    float* out = a.out + (size_t)t * K;
    id_bad = src >= 0 && prologue_id_bad(a, id);
    if (src >= 0 && id < 0 && a.embeds) {
      // a spliced input row (the vision features at an image-token position)
      const float* e = a.embeds + (size_t)src * K;
      for (int k = tid * 4; k < K; k += 1024) *(float4*)(out + k) = *(const float4*)(e + k);
    } else if (src < 0 || id_bad) {
      for (int k = tid * 4; k < K; k += 1024) *(float4*)(out + k) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else if (a.emb.fmt == LA_W_BF16) {
      const uint16_t* base = (const uint16_t*)a.emb.data;
      const int UT = K / 32;
      for (int k = tid * 8; k < K; k += 2048) {
        // row-major, or the 16-row tiled layout of the tied lm_head
        const size_t off = a.emb.layout == LA_LAYOUT_ROWS
                               ? (size_t)id * K + k
                               : (((size_t)(id >> 4) * UT + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (id & 15)) * 8;
        const uint4 w = *(const uint4*)(base + off);
        *(float4*)(out + k) = make_float4(bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16),
                                          bf16_to_f32(w.y & 0xFFFFu), bf16_to_f32(w.y >> 16));
        *(float4*)(out + k + 4) = make_float4(bf16_to_f32(w.z & 0xFFFFu), bf16_to_f32(w.z >> 16),
                                              bf16_to_f32(w.w & 0xFFFFu), bf16_to_f32(w.w >> 16));
      }
    } else {
      // INT4: element j = (q_j - 8) * scale[j / group], q_j the low nibble of byte
      // j/2 for even j and its high nibble for odd j (exact in fp32).
      const uint8_t* row = (const uint8_t*)a.emb.data + (size_t)id * (K / 2);
      const uint16_t* sc = (const uint16_t*)a.emb.scales + (size_t)id * (K / a.emb.group);
      for (int k = tid * 8; k < K; k += 2048) {
        const uint32_t w = *(const uint32_t*)(row + k / 2);
        const float s = fp16_to_f32(sc[k / a.emb.group]);
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (float)((int)((w >> (4 * j)) & 0xFu) - 8) * s;
        *(float4*)(out + k) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)(out + k + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }

  if (a.prefix_len) {
    const int b = t / a.W, j = t - b * a.W;
    const int P = a.prefix_len[b];
    const long pos = (long)P + j;
    if (a.rope && tid < 64) {
      // angle = pos * theta^(-2i/128), evaluated in fp64, stored as fp32 cos/sin
      const double inv_freq = pow(a.rope_theta, -2.0 * (double)tid / (double)kHeadDim);
      const double ang = (double)pos * inv_freq;
      a.rope[(size_t)t * 64 + tid] = make_float2((float)cos(ang), (float)sin(ang));
    }
    if (a.flags) {
      // a data error anywhere in the window poisons the whole sequence (its rows
      // attend to each other)
      int f = 0;
      if (a.ids) {
        const int nw = a.in_w > 0 ? a.in_w : a.W;
        for (int jj = tid; jj < nw; jj += 256)
          if (prologue_id_bad(a, a.ids[b * nw + jj])) f = LA_DERR_TOKEN_ID;
        if (__syncthreads_or(f)) f = LA_DERR_TOKEN_ID;
      }
      const long n = (long)P + a.W;
      if (P < 0 || n > a.cap) f |= LA_DERR_CAPACITY;
      if (a.causal_rows || a.window_len) {
        // a re-fed window: c causal rows, then the block up to w real rows
        const int c = a.causal_rows ? a.causal_rows[b] : 0;
        const int w = a.window_len ? a.window_len[b] : a.W;
        if (w < 1 || w > a.W || c < 0 || c > w) f |= LA_DERR_WINDOW;
      }
      int blk_bad = 0;
      if (!(f & LA_DERR_CAPACITY)) {
        const int pages = (int)((n + kBlock - 1) / kBlock);
        for (int p = tid; p < pages; p += 256) {
          const int blk = a.block_table[(size_t)b * a.max_blocks + p];
          if (blk < 0 || blk >= a.num_blocks) blk_bad = 1;
        }
      }
      if (__syncthreads_or(blk_bad)) f |= LA_DERR_BLOCK_ID;
      if (tid == 0) {
        a.flags[t] = f;
        if (f && a.err) atomicOr(a.err, f);
      }
    }
  } else if (id_bad && a.err && tid == 0) {
    atomicOr(a.err, LA_DERR_TOKEN_ID);
  }
}

// The attention's view of a prefill of L rows per sequence: window k of
// sequence b holds prompt rows 16k .. 16k + 15 at prefix P_b + 16k, every row
// causal, min(16, L - 16k) of them real.
__global__ __launch_bounds__(256) void k_prefill_views(const int32_t* prefix_len, int B, int L, int chunks,
                                                       int32_t* pp, int32_t* pc, int32_t* pw) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * chunks) return;
  const int b = i / chunks, k = i - b * chunks;
  pp[i] = prefix_len[b] + 16 * k;
  pc[i] = 16;
  pw[i] = min(16, L - 16 * k);
}

hipError_t launch_prefill_views(const int32_t* prefix_len, int B, int L, int chunks, int32_t* pp,
                                int32_t* pc, int32_t* pw, hipStream_t s) {
  hipLaunchKernelGGL(k_prefill_views, dim3((B * chunks + 255) / 256), dim3(256), 0, s, prefix_len, B, L,
                     chunks, pp, pc, pw);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  if (a.zero && ((uintptr_t)a.zero % 16 || a.n_zero % 4 || a.zero_blocks < 1)) return hipErrorInvalidValue;
  const int zb = a.zero ? a.zero_blocks : 0;
  hipLaunchKernelGGL(k_prologue, dim3(a.T + zb), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Commit of a fully accepted window: one thread per window slot of each
// sequence; the slot-0 thread also advances the prefix length.
__global__ __launch_bounds__(1024) void k_commit(const int32_t* out_ids, int32_t* window_ids,
                                                 int32_t* prefix_len, int B, int W, int mask_id) {
  const int t = threadIdx.x;
  if (t >= B * W) return;
  const int b = t / W, j = t - b * W;
  window_ids[t] = j == 0 ? out_ids[b * W + W - 1] : mask_id;
  if (j == 0) prefix_len[b] += W;
}

hipError_t launch_commit(const int32_t* out_ids, int32_t* window_ids, int32_t* prefix_len, int B,
                         int W, int mask_id, hipStream_t s) {
  hipLaunchKernelGGL(k_commit, dim3(1), dim3(((B * W + 63) / 64) * 64), 0, s, out_ids, window_ids,
                     prefix_len, B, W, mask_id);
  return hipGetLastError();
}

// Commit of a re-fed window.  Sequence b accepts the first n_b outputs of its
// block (rows c_b .. w_b - 1; n_b clamped to 1 .. w_b - c_b and to
// W - block + 1); every row up to the block's first is final, so the prefix
// becomes P_b + c_b + 1, and the next window re-feeds the accepted tokens, the
// last of them opening a block of `block` rows with block - 1 mask tokens:
// [out[c_b] .. out[c_b + n_b - 1], mask ...], c' = n_b - 1, w' = n_b + block - 1.
// Every thread reads before any writes (the state is updated in place).
__global__ __launch_bounds__(1024) void k_commit_refeed(const int32_t* out_ids, const int32_t* n_accept,
                                                        int32_t* window_ids, int32_t* prefix_len,
                                                        int32_t* causal_rows, int32_t* window_len,
                                                        int B, int W, int block, int mask_id) {
  const int t = threadIdx.x;
  const bool live = t < B * W;
  const int b = live ? t / W : 0, j = t - b * W;
  int c = 0, n = 1, P = 0, id = mask_id;
  if (live) {
    c = min(max(causal_rows[b], 0), W - 1);
    const int w = min(max(window_len[b], c + 1), W);
    const int S = w - c;
    n = n_accept ? min(max(n_accept[b], 1), S) : S;
    n = min(n, W - block + 1);
    P = prefix_len[b];
    if (j < n) id = out_ids[b * W + c + j];
  }
  __syncthreads();
  if (live) {
    window_ids[t] = id;
    if (j == 0) {
      prefix_len[b] = P + c + 1;
      causal_rows[b] = n - 1;
      window_len[b] = n + block - 1;
    }
  }
}

hipError_t launch_commit_refeed(const int32_t* out_ids, const int32_t* n_accept, int32_t* window_ids,
                                int32_t* prefix_len, int32_t* causal_rows, int32_t* window_len, int B,
                                int W, int block, int mask_id, hipStream_t s) {
  hipLaunchKernelGGL(k_commit_refeed, dim3(1), dim3(((B * W + 63) / 64) * 64), 0, s, out_ids, n_accept,
                     window_ids, prefix_len, causal_rows, window_len, B, W, block, mask_id);
  return hipGetLastError();
}

// Set the bitmap bit of every selected window id: ids[b][j] for first[b] <= j
// < first[b] + count[b] (defaults 0 and W); ids outside [0, vocab) are skipped.
__global__ __launch_bounds__(256) void k_mark_tokens(const int32_t* ids, int B, int W, const int32_t* first,
                                                     const int32_t* count, uint32_t* bits, int words,
                                                     int vocab) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * W) return;
  const int b = t / W, j = t - b * W;
  const int j0 = first ? first[b] : 0;
  const int n = count ? count[b] : W;
  if (j < j0 || j >= j0 + n) return;
  const int id = ids[t];
  if (id < 0 || id >= vocab) return;
  atomicOr(bits + (size_t)b * words + (id >> 5), 1u << (id & 31));
}

hipError_t launch_mark_tokens(const int32_t* ids, int B, int W, const int32_t* first, const int32_t* count,
                              uint32_t* bits, int words, int vocab, hipStream_t s) {
  hipLaunchKernelGGL(k_mark_tokens, dim3((B * W + 255) / 256), dim3(256), 0, s, ids, B, W, first, count,
                     bits, words, vocab);
  return hipGetLastError();
}

}  // namespace la
