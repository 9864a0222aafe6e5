// C ABI of the PBD window step: host-side validation, workspace carving and the
// launch sequence of every entry point declared in include/la_pbd.h.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "la_internal.hpp"

using namespace la;

namespace {

constexpr size_t kAlign = 256;

size_t al(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base((char*)p) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += al(count * sizeof(T));
    return p;
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// `tiled`: the tiled layout this use accepts besides row-major (-1: none).
// Bytes of a weight's data and INT4 scales in its layout.
void weight_storage(const la_weight* w, size_t* data, size_t* scales) {
  const bool int4 = w->fmt == LA_W_INT4;
  if (w->fmt == LA_W_W8A8) {
    // int8 codes (tiled: 16-row tiles, zero past n) and fp32 scales per row
    const size_t rows = w->layout == LA_LAYOUT_ROWS ? (size_t)w->n
                        : w->layout == LA_LAYOUT_TILED_GU ? (size_t)(w->n / 2 + 7) / 8 * 16
                                                          : (size_t)(w->n + 15) / 16 * 16;
    *data = rows * (size_t)w->k;
    *scales = (size_t)w->n * 4;
    return;
  }
  if (w->layout == LA_LAYOUT_ROWS) {
    *data = int4 ? (size_t)w->n * (w->k / 2) : (size_t)w->n * w->k * 2;
    *scales = int4 && w->group > 0 ? (size_t)w->n * (w->k / w->group) * 2 : 0;
    return;
  }
  const size_t n_tiles = w->layout == LA_LAYOUT_TILED_GU ? (size_t)(w->n / 2 + 7) / 8
                                                         : (size_t)(w->n + 15) / 16;
  *data = int4 ? n_tiles * 16 * (size_t)(w->k / 2) : n_tiles * 16 * (size_t)w->k * 2;
  *scales = int4 ? n_tiles * (w->k / 128) * 16 * 2 : 0;
}

// The kernels address a weight with 32-bit offsets.
constexpr size_t kMaxWeightBytes = (size_t)1 << 31;
// Window rows, and window rows times query heads per KV head (one attention
// wave per 16 of them, at most 8 waves).
constexpr int kMaxWindow = 16;
constexpr int kMaxQueryCols = 128;
// Rows of one prefill call (B times the prompt length rounded up to 16).
constexpr int64_t kMaxPrefillRows = 8192;

la_status attention_entry(const float* q, const la_kv_cache* kv, int32_t layer, int32_t n_heads,
                          int32_t n_kv_heads, int32_t head_dim, const int32_t* prefix_len,
                          bool causal, const int32_t* causal_rows, const int32_t* window_len,
                          int32_t B, int32_t W, int32_t max_len, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

// allow_int4: the quantised formats (INT4 with group int4_group, w8a8) are accepted.
la_status check_weight(const la_weight* w, int n, int k, bool allow_int4, int int4_group,
                       int tiled) {
  if (!w || !w->data) return LA_ERR_ARG;
  if (w->n != n || w->k != k) return LA_ERR_SHAPE;
  {
    size_t wb, sb;
    weight_storage(w, &wb, &sb);
    if (wb >= kMaxWeightBytes) return LA_ERR_SHAPE;
  }
  if (!aligned16(w->data)) return LA_ERR_ARG;
  if (w->layout != LA_LAYOUT_ROWS && w->layout != tiled) return LA_ERR_UNSUPPORTED;
  if (w->layout != LA_LAYOUT_ROWS && k % 128) return LA_ERR_SHAPE;
  if (w->fmt == LA_W_BF16) return LA_OK;
  if (w->fmt == LA_W_W8A8) {
    if (!allow_int4) return LA_ERR_UNSUPPORTED;
    if (!w->scales || k % 64) return LA_ERR_SHAPE;
    return LA_OK;
  }
  if (w->fmt != LA_W_INT4) return LA_ERR_ARG;
  if (!allow_int4) return LA_ERR_UNSUPPORTED;
  if (!w->scales || w->group != int4_group || k % int4_group) return LA_ERR_SHAPE;
  return LA_OK;
}

la_status check_gemm_weight(const la_weight* w, int tiled) {
  if (!w || !w->data) return LA_ERR_ARG;
  if (w->n < 1 || w->k < 256 || w->k % 256) return LA_ERR_SHAPE;
  return check_weight(w, w->n, w->k, true, 128, tiled);
}

// ---------------------------------------------------------------- workspace plans

// Launch plans as launch_gemm makes them: up to 32 rows the small-M kernel,
// beyond that the large-M kernel (whose first launch fixes the plan).
int gemm_parts(int M, const la_weight* w, int epi) {
  if (w->fmt == LA_W_W8A8) return plan_gemm_w8(M, w->n, w->k, epi, false).grid;
  const bool int4 = w->fmt == LA_W_INT4;
  if (use_big_gemm(M, int4, epi, w->layout != LA_LAYOUT_ROWS))
    return plan_gemm_big(std::min(M, big_rows_per_launch(int4)), w->n, w->k, int4, epi, false).grid;
  return plan_gemm(M, w->n, w->k, int4, epi, false).grid;
}

int gemm_ksplit(int M, const la_weight* w) {
  if (w->fmt == LA_W_W8A8) return plan_gemm_w8(M, w->n, w->k, EPI_STORE, true).ksplit;
  const bool int4 = w->fmt == LA_W_INT4;
  if (use_big_gemm(M, int4, EPI_STORE, w->layout != LA_LAYOUT_ROWS))
    return plan_gemm_big(std::min(M, big_rows_per_launch(int4)), w->n, w->k, int4, EPI_STORE, true).ksplit;
  return plan_gemm(M, w->n, w->k, int4, EPI_STORE, true).ksplit;
}

// K slices of the QKV projection: past 32 rows it writes slice sums that a
// finishing kernel turns into q and the window's K/V (0: no slice buffer).
int qkv_ksplit(int M, const la_weight* w) {
  if (w->fmt == LA_W_W8A8) return 0;
  const bool int4 = w->fmt == LA_W_INT4;
  if (!use_big_gemm(M, int4, EPI_QKV, w->layout != LA_LAYOUT_ROWS)) return 0;
  return plan_gemm_big(std::min(M, big_rows_per_launch(int4)), w->n, w->k, int4, EPI_QKV, true).ksplit;
}

// The front-half launch's attention runs for B sequences of W rows with keys
// up to max_len: pages per run and runs per (sequence, KV head), every run of
// every 16-column query tile beside the QKV tiles on its own compute unit (at
// most 16 runs of at most kFrontMaxRunPages pages); false when the shape does not fit the launch
// (at most 8 bf16 rows, hidden and heads x 128 both 2048, the 64 pack slices
// beside the QKV tiles).
bool front_shape(const la_model* m, int B, int W, int max_len, int* pps_out, int* runs_out) {
  const int T = B * W, H = m->hidden, HQ = m->n_heads * m->head_dim;
  const int NQKV = (m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
  if (T < 1 || T > 8 || H != 2048 || HQ != 2048 || m->layers[0].qkv.fmt != LA_W_BF16) return false;
  if (attn_nqp(W, m->n_heads / m->n_kv_heads) > 64) return false;
  const int G = cu_count(), n_qkv = NQKV / 16;
  const int free_wgs = G - n_qkv;
  const int units = B * m->n_kv_heads * attn_nqp(W, m->n_heads / m->n_kv_heads) / 16;  // items per run
  if (n_qkv + kFrontPackSlices > G || H / 16 > n_qkv || free_wgs < units) return false;
  const int max_pages = (max_len + kBlock - 1) / kBlock;
  const int runs_max = std::min(std::min(16, free_wgs / units), 128 / units);
  const int pps = std::max(2, (max_pages + runs_max - 1) / runs_max);
  if (pps > kFrontMaxRunPages) return false;
  *pps_out = pps;
  *runs_out = (max_pages + pps - 1) / pps;
  return true;
}

struct StepWs {
  float* h;
  float* q;
  float* o;
  float* mlp;
  uint16_t* apack;    // packed operand with K <= max(hidden, heads * head_dim)
  uint16_t* apack_o;  // packed attention output (K = heads * head_dim), bf16 path
  float* ss;          // [T][hidden / 16] per-tile sums of squares of h, bf16 path
  float* asum;
  uint16_t* apack_m;  // packed MLP activations (K = inter)
  float* asum_m;
  float2* rope;
  int32_t* flags;
  float* part_o;
  float* part_ml;
  float* amax;
  float* parts;       // K-slice partial sums of the O and down projections
  int32_t* sync;      // the front-half launch's flag words, then its 8-byte words
  int n_sync;         // (all zeroed by the prologue: n_sync int32 words)
  uint64_t* ll_q;
  uint64_t* ll_kv;
  uint64_t* ll_ml;
  uint64_t* ll_po;
  float* front_ss;    // the front-half launch's per-slice sums of squares
  int32_t* err;       // the step's error word (nullable)
  // prefill: the attention's view of the prompt as 16-row windows, the
  // per-sequence flags and the last rows
  int32_t* pre_prefix;
  int32_t* pre_causal;
  int32_t* pre_wlen;
  int32_t* pre_flags;
  float* h_last;
  int pps, max_splits, nqp, vocab_parts;
  size_t bytes;
};

// Rows of one attention window of a prefill (the attention sees the prompt as
// windows of this many causal rows).
constexpr int kPrefillChunk = 16;

// Workspace of a step (chunks = 0) or of a prefill of B sequences of W =
// 16 * chunks rows, whose attention runs as B * chunks windows of 16 rows and
// whose lm_head takes one row per sequence.
StepWs carve_step(const la_model* m, int B, int W, int max_len, void* ws, bool lm_head,
                  int chunks = 0) {
  StepWs s;
  memset(&s, 0, sizeof(s));
  Carver c(ws);
  const int T = B * W;
  const int aB = chunks ? B * chunks : B, aW = chunks ? kPrefillChunk : W;
  const int lm_rows = chunks ? B : T;
  const int H = m->hidden, HQ = m->n_heads * m->head_dim, F = m->inter;
  const int Kx = H > HQ ? H : HQ;
  s.h = c.take<float>((size_t)T * H);
  s.q = c.take<float>((size_t)T * HQ);
  s.o = c.take<float>((size_t)T * HQ);
  s.mlp = c.take<float>((size_t)T * F);
  s.apack = c.take<uint16_t>(apack_elems(T, Kx));
  s.apack_o = c.take<uint16_t>(apack_elems(T, HQ));
  s.ss = c.take<float>((size_t)T * (H / 16));
  s.asum = c.take<float>((size_t)((T + 7) / 8) * (Kx / 128) * 16);
  s.apack_m = c.take<uint16_t>(apack_elems(T, F));
  s.asum_m = c.take<float>((size_t)((T + 7) / 8) * (F / 128) * 16);
  s.rope = c.take<float2>((size_t)T * 64);
  s.flags = c.take<int32_t>(T);
  plan_attention(aB, m->n_kv_heads, max_len, &s.pps, &s.max_splits);
  s.nqp = attn_nqp(aW, m->n_heads / m->n_kv_heads);
  const size_t units = (size_t)aB * m->n_kv_heads * s.max_splits * s.nqp;
  s.part_o = c.take<float>(units * kHeadDim);
  s.part_ml = c.take<float>(units * 2);
  const la_weight* lm = m->lm_head.data ? &m->lm_head : &m->embed;
  s.vocab_parts = gemm_parts(lm_rows, lm, EPI_ARGMAX);
  s.amax = lm_head ? c.take<float>((size_t)lm_rows * s.vocab_parts * 3) : nullptr;
  if (chunks) {
    s.pre_prefix = c.take<int32_t>(aB);
    s.pre_causal = c.take<int32_t>(aB);
    s.pre_wlen = c.take<int32_t>(aB);
    s.pre_flags = c.take<int32_t>(B);
    s.h_last = c.take<float>((size_t)B * H);
  }
  // (at least the front launch's down slices)
  const int ksp = std::max(std::max(gemm_ksplit(T, &m->layers[0].o), gemm_ksplit(T, &m->layers[0].down)),
                           kFrontDownSlices);
  const int NQKV = (m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
  const size_t qkv_parts = (size_t)qkv_ksplit(T, &m->layers[0].qkv) * T * NQKV;
  s.parts = c.take<float>(std::max((size_t)ksp * T * H, qkv_parts));
  const size_t sync_off = c.off;
  s.sync = c.take<int32_t>(kFrontSyncWords);
  int fpps, fruns;
  if (!chunks && front_shape(m, B, W, max_len, &fpps, &fruns)) {
    const size_t units = (size_t)B * m->n_kv_heads * fruns * s.nqp;
    s.ll_q = c.take<uint64_t>((size_t)T * HQ);
    s.ll_kv = c.take<uint64_t>((size_t)T * m->n_kv_heads * 2 * 64);
    s.ll_ml = c.take<uint64_t>(units * 2);
    s.ll_po = c.take<uint64_t>(units * kHeadDim);
  }
  s.n_sync = (int)((c.off - sync_off) / 4);
  s.front_ss = c.take<float>(8 * kFrontPackSlices);
  s.bytes = c.off;
  return s;
}

la_status check_model(const la_model* m) {
  if (!m || !m->layers) return LA_ERR_ARG;
  if (m->head_dim != kHeadDim || m->n_kv_heads < 1 || m->n_heads < m->n_kv_heads ||
      m->n_heads % m->n_kv_heads || m->hidden < 256 || m->hidden % 256 ||
      (m->n_heads * m->head_dim) % 256 || m->inter < 256 || m->inter % 256 || m->n_layers < 1 ||
      m->vocab < 1 || !(m->rms_eps > 0.f) || !(m->rope_theta > 1.f))
    return LA_ERR_SHAPE;
  const int H = m->hidden, HQ = m->n_heads * m->head_dim;
  const int NQKV = (m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
  const int fmt = m->layers[0].qkv.fmt;
  if (fmt != LA_W_BF16 && fmt != LA_W_INT4 && fmt != LA_W_W8A8) return LA_ERR_ARG;
  if (m->window_mask != LA_MASK_BIDIRECTIONAL && m->window_mask != LA_MASK_CAUSAL) return LA_ERR_ARG;
  for (int l = 0; l < m->n_layers; ++l) {
    const la_layer& L = m->layers[l];
    if (!L.in_norm || !L.post_norm) return LA_ERR_ARG;
    if (!aligned16(L.in_norm) || !aligned16(L.post_norm)) return LA_ERR_ARG;
    la_status st;
    if ((st = check_weight(&L.qkv, NQKV, H, true, 128, LA_LAYOUT_TILED_QKV)) != LA_OK) return st;
    if ((st = check_weight(&L.o, H, HQ, true, 128, LA_LAYOUT_TILED)) != LA_OK) return st;
    if ((st = check_weight(&L.gate_up, 2 * m->inter, H, true, 128, LA_LAYOUT_TILED_GU)) != LA_OK)
      return st;
    if ((st = check_weight(&L.down, H, m->inter, true, 128, LA_LAYOUT_TILED)) != LA_OK) return st;
    if (L.qkv.fmt != fmt || L.o.fmt != fmt || L.gate_up.fmt != fmt || L.down.fmt != fmt)
      return LA_ERR_UNSUPPORTED;
  }
  if (!m->final_norm || !aligned16(m->final_norm)) return LA_ERR_ARG;
  if (fmt == LA_W_BF16) {
    la_status st = check_weight(&m->embed, m->vocab, H, false, 0, LA_LAYOUT_TILED);
    if (st != LA_OK) return st;
    if (m->lm_head.data) {
      if ((st = check_weight(&m->lm_head, m->vocab, H, false, 0, LA_LAYOUT_TILED)) != LA_OK) return st;
    }
  } else if (fmt == LA_W_W8A8) {
    // bf16 embedding; the lm_head is the w8a8 copy of the tied matrix
    la_status st = check_weight(&m->embed, m->vocab, H, false, 0, LA_LAYOUT_TILED);
    if (st != LA_OK) return st;
    if (!m->lm_head.data || m->lm_head.fmt != LA_W_W8A8) return LA_ERR_ARG;
    if ((st = check_weight(&m->lm_head, m->vocab, H, true, 0, LA_LAYOUT_TILED)) != LA_OK) return st;
  } else {
    la_status st = check_weight(&m->embed, m->vocab, H, true, 32, -1);
    if (st != LA_OK) return st;
    if (!m->lm_head.data) return LA_ERR_ARG;
    if ((st = check_weight(&m->lm_head, m->vocab, H, true, 128, LA_LAYOUT_TILED)) != LA_OK) return st;
  }
  return LA_OK;
}

la_status check_cache(const la_kv_cache* kv, const la_model* m, int B) {
  if (!kv || !kv->k || !kv->v || !kv->block_table) return LA_ERR_ARG;
  if (kv->block_size != kBlock || kv->num_blocks < 1 || kv->max_blocks < 1) return LA_ERR_SHAPE;
  if (m && kv->n_layers < m->n_layers) return LA_ERR_SHAPE;
  if (!aligned16(kv->k) || !aligned16(kv->v)) return LA_ERR_ARG;
  (void)B;
  return LA_OK;
}

la_status check_step_shape(const la_model* m, int B, int W, int max_len) {
  if (B < 1 || B > 64 || W < 1 || W > kMaxWindow || max_len < W) return LA_ERR_SHAPE;
  if (W * (m->n_heads / m->n_kv_heads) > kMaxQueryCols) return LA_ERR_SHAPE;
  return LA_OK;
}

la_status hip_status(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

#define LA_TRY(expr)                          \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return LA_ERR_HIP;  \
  } while (0)

size_t kv_layer_elems(const la_kv_cache* kv, const la_model* m) {
  return (size_t)kv->num_blocks * m->n_kv_heads * kBlock * kHeadDim;
}

GemmArgs base_gemm(const la_weight* w, int M) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.w = w->data;
  g.wscale = (const uint16_t*)w->scales;
  size_t wb, sb;
  weight_storage(w, &wb, &sb);
  g.w_bytes = (uint32_t)wb;
  g.s_bytes = (uint32_t)sb;
  g.layout = w->layout;
  g.M = M;
  g.N = w->n;
  g.K = w->k;
  return g;
}

// Pack fp32 rows (h plus pending partial sums, RMSNorm'd when gain != NULL)
// into the matrix-core operand; the summed rows are written back to h_out.
// fmt: the consumer's weight format (LA_W_*), which fixes the operand's form.
la_status pack_rows(const float* x, int ldx, int M, int K, const uint16_t* gain, float eps,
                    uint16_t* apack, float* asum, int fmt, const float* parts, int n_parts,
                    float* h_out, hipStream_t st) {
  PackArgs p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.ldx = ldx;
  p.M = M;
  p.K = K;
  p.gain = gain;
  p.eps = eps;
  p.apack = apack;
  p.asum = asum;
  p.int4 = fmt == LA_W_INT4;
  p.w8 = fmt == LA_W_W8A8;
  p.parts = parts;
  p.n_parts = parts ? n_parts : 0;
  p.h_out = h_out;
  LA_TRY(launch_pack(p, st));
  return LA_OK;
}

la_status gemm_from_rows(GemmArgs g, const float* x, int ldx, const uint16_t* gain, float eps,
                         uint16_t* apack, float* asum, int epi, int fmt, hipStream_t st) {
  la_status rs = pack_rows(x, ldx, g.M, g.K, gain, eps, apack, asum, fmt, nullptr, 0, nullptr, st);
  if (rs != LA_OK) return rs;
  g.apack = apack;
  g.asum = asum;
  LA_TRY(launch_gemm(g, epi, fmt, st));
  return LA_OK;
}

// What the previous kernel left for the next layer's input: `pending` K-slice
// partial sums still to be added to h (INT4 path), or `packed`: the operand of
// h * in_norm is in s.apack and the per-tile sums of squares of h in s.ss, so
// the QKV projection applies 1/rms itself (bf16 path).
struct Carry {
  int pending = 0;
  bool packed = false;
};

// One decoder layer on the rows in s.h.  bf16 weights: the O projection (and
// the down projection when it is not K-sliced) adds the residual, keeps h,
// packs h * gain for the next GEMM and leaves per-tile sums of squares; the
// next GEMM scales its outputs by 1/rms, so no normalisation kernel runs.  `next_gain` is the RMSNorm gain after this
// layer (the next layer's input norm or the final norm; NULL: h only).
// The attention's view of the rows when it differs from the layer's (a
// prefill: B sequences of W rows seen as windows of kPrefillChunk rows).
struct AttnView {
  int B, W;
  const int32_t* prefix_len;
  const int32_t* causal_rows;
  const int32_t* window_len;
  int bt_div;  // windows per block-table row
};

// The front half of a layer (RMSNorm, QKV, attention, O) runs as one
// persistent launch for at most 8 bf16 rows with K = 2048 tiled weights and at
// most 4 pending K-slice sums, when the attention runs of every (sequence, KV
// head) fit beside the QKV tiles on the compute units (at most 16 runs of at
// most kFrontMaxRunPages pages each); otherwise (and with LA_PBD_FRONT=0 in the
// environment, a diagnostic switch) each step is a kernel of its own.
struct FrontPlan {
  int grid = 0, pps = 0, runs = 0, items = 0;
  bool gate_up = false;  // the launch also runs gate/up (LA_PBD_FRONT_GU=0 in the environment turns it off)
  bool down = false;     // and the down projection (LA_PBD_FRONT_DOWN=0 turns it off)
};

FrontPlan plan_front(const la_model* m, const la_layer& L, int B, int W, int max_len, const StepWs& s,
                     const AttnView* av, const float* attn_out, int pending) {
  FrontPlan f;
  const char* env = getenv("LA_PBD_FRONT");
  if (env && env[0] == '0') return f;
  if (av || attn_out || pending > 4 || L.qkv.fmt != LA_W_BF16 || !s.ll_q) return f;
  if (L.qkv.layout != LA_LAYOUT_TILED_QKV || L.o.layout != LA_LAYOUT_TILED) return f;
  int pps, runs;
  if (!front_shape(m, B, W, max_len, &pps, &runs)) return f;
  f.grid = cu_count();
  f.pps = pps;
  f.runs = runs;
  f.items = B * m->n_kv_heads * (s.nqp / 16) * runs;
  const char* gu = getenv("LA_PBD_FRONT_GU");
  f.gate_up = !(gu && gu[0] == '0') && L.gate_up.fmt == LA_W_BF16 && L.gate_up.layout == LA_LAYOUT_TILED_GU &&
              L.gate_up.k == m->hidden && m->inter % 8 == 0;
  // the down projection as K-slice sums, two output tiles of one slice per
  // workgroup: the grid must hold H / 16 x kFrontDownSlices / 2 workgroups
  const char* dn = getenv("LA_PBD_FRONT_DOWN");
  const int U = m->inter / 32;
  f.down = f.gate_up && !(dn && dn[0] == '0') && L.down.fmt == LA_W_BF16 && L.down.layout == LA_LAYOUT_TILED &&
           L.down.k == m->inter && L.down.n == m->hidden && m->inter % 32 == 0 && m->hidden % 16 == 0 &&
           f.grid == (m->hidden / 16) * kFrontDownSlices / 2 && f.grid <= 256 &&
           (U + kFrontDownSlices - 1) / kFrontDownSlices <= kFrontDownUnits;
  return f;
}

la_status run_layer(const la_model* m, int l, const la_kv_cache* kv, const int32_t* prefix_len,
                    const int32_t* causal_rows, const int32_t* window_len, int B, int W,
                    int max_len, const StepWs& s, float* attn_out, Carry* carry,
                    const uint16_t* next_gain, hipStream_t st, const AttnView* av = nullptr,
                    const hipEvent_t* ev = nullptr) {
  const la_layer& L = m->layers[l];
  const int T = B * W;
  const int H = m->hidden, HQ = m->n_heads * m->head_dim;
  // quantised weights (INT4, w8a8): every GEMM writes fp32 and a packing kernel
  // prepares the next operand (a w8a8 operand's per-row scale needs the whole row)
  const int wf = L.qkv.fmt;
  const bool quant = wf != LA_W_BF16;
  const size_t le = kv_layer_elems(kv, m);
  la_status rs;
  const FrontPlan fp = plan_front(m, L, B, W, max_len, s, av, attn_out, carry->pending);
  GemmArgs g;
  // timing events around the attention block (input norm .. O projection)
  if (ev) LA_TRY(hipEventRecord(ev[0], st));
  if (fp.grid) {
    FrontArgs f;
    memset(&f, 0, sizeof(f));
    AttnArgs& at = f.at;
    at.kc = (uint16_t*)kv->k + (size_t)l * le;
    at.vc = (uint16_t*)kv->v + (size_t)l * le;
    at.block_table = kv->block_table;
    at.prefix_len = prefix_len;
    at.B = B;
    at.W = W;
    at.Hq = m->n_heads;
    at.Hkv = m->n_kv_heads;
    at.num_blocks = kv->num_blocks;
    at.max_blocks = kv->max_blocks;
    at.cap = std::min(max_len, kv->max_blocks * kBlock);
    at.pages_per_split = fp.pps;
    at.max_splits = fp.runs;
    at.out_apack = s.apack_o;
    at.nqp = s.nqp;
    at.causal = m->window_mask == LA_MASK_CAUSAL;
    at.causal_rows = causal_rows;
    at.window_len = window_len;
    at.bt_div = 1;
    f.T = T;
    f.H = H;
    f.HQ = HQ;
    f.h = s.h;
    f.parts = carry->pending ? s.parts : nullptr;
    f.n_parts = carry->pending;
    f.in_norm = L.in_norm;
    f.eps = m->rms_eps;
    f.xpack = s.apack;
    f.ss_part = s.front_ss;
    size_t wb, sb;
    weight_storage(&L.qkv, &wb, &sb);
    f.wqkv = L.qkv.data;
    f.wqkv_bytes = (uint32_t)wb;
    f.qkv_bias = L.qkv_bias;
    f.rope = s.rope;
    f.flags = s.flags;
    weight_storage(&L.o, &wb, &sb);
    f.wo = L.o.data;
    f.wo_bytes = (uint32_t)wb;
    f.post_norm = L.post_norm;
    f.gpack = s.apack;
    f.ss = s.ss;
    f.n_qkv_tiles = (m->n_heads + 2 * m->n_kv_heads) * m->head_dim / 16;
    f.n_o_tiles = H / 16;
    f.n_items = fp.items;
    f.runs = fp.runs;
    if (fp.gate_up) {
      weight_storage(&L.gate_up, &wb, &sb);
      f.wgu = L.gate_up.data;
      f.wgu_bytes = (uint32_t)wb;
      f.F = m->inter;
      f.n_gu_tiles = m->inter / 8;
      f.mpack = s.apack_m;
    }
    if (fp.down) {
      weight_storage(&L.down, &wb, &sb);
      f.wdn = L.down.data;
      f.wdn_bytes = (uint32_t)wb;
      f.dparts = s.parts;
    }
    f.sync = s.sync;
    f.ll_q = s.ll_q;
    f.ll_kv = s.ll_kv;
    f.ll_ml = s.ll_ml;
    f.ll_po = s.ll_po;
    f.epoch = l + 1;
    f.err = s.err;
    LA_TRY(launch_front(f, fp.grid, st));
    carry->pending = 0;
    carry->packed = false;
    if (fp.down) {
      // the launch wrote the down projection's K-slice sums (the next pack adds them)
      if (ev) LA_TRY(hipEventRecord(ev[1], st));
      carry->pending = kFrontDownSlices;
      return LA_OK;
    }
  } else {

  // input operand: h (+ pending partial sums), RMSNorm, pack, unless the
  // previous projection already packed it
  const bool in_packed = carry->packed;
  if (!in_packed) {
    if ((rs = pack_rows(s.h, H, T, H, L.in_norm, m->rms_eps, s.apack, s.asum, wf, s.parts,
                        carry->pending, carry->pending ? s.h : nullptr, st)) != LA_OK)
      return rs;
  }
  carry->pending = 0;
  carry->packed = false;

  // QKV + bias + RoPE + K/V write
  g = base_gemm(&L.qkv, T);
  g.apack = s.apack;
  g.asum = s.asum;
  if (in_packed) {
    g.ss_in = s.ss;
    g.ss_tiles = H / 16;
    g.eps = m->rms_eps;
  }
  g.bias = L.qkv_bias;
  g.y = s.q;
  g.ldy = HQ;
  g.rope = s.rope;
  g.prefix_len = prefix_len;
  g.flags = s.flags;
  g.W = W;
  g.n_heads = m->n_heads;
  g.n_kv_heads = m->n_kv_heads;
  g.block_table = kv->block_table;
  g.max_blocks = kv->max_blocks;
  g.num_blocks = kv->num_blocks;
  g.kc = (uint16_t*)kv->k + (size_t)l * le;
  g.vc = (uint16_t*)kv->v + (size_t)l * le;
  if (qkv_ksplit(T, &L.qkv) > 0) g.partial = s.parts;  // slice sums + finishing kernel
  LA_TRY(launch_gemm(g, EPI_QKV, wf, st));

  // window attention -> packed O-projection operand
  AttnArgs at;
  memset(&at, 0, sizeof(at));
  at.q = s.q;
  at.kc = g.kc;
  at.vc = g.vc;
  at.block_table = kv->block_table;
  at.prefix_len = prefix_len;
  at.B = B;
  at.W = W;
  at.Hq = m->n_heads;
  at.Hkv = m->n_kv_heads;
  at.num_blocks = kv->num_blocks;
  at.max_blocks = kv->max_blocks;
  at.cap = std::min(max_len, kv->max_blocks * kBlock);
  at.pages_per_split = s.pps;
  at.max_splits = s.max_splits;
  at.part_o = s.part_o;
  at.part_ml = s.part_ml;
  at.nqp = s.nqp;
  at.out = (quant || attn_out) ? (attn_out ? attn_out : s.o) : nullptr;
  at.out_apack = quant ? nullptr : s.apack_o;
  at.out_int4 = false;
  at.causal = m->window_mask == LA_MASK_CAUSAL;
  at.causal_rows = causal_rows;
  at.window_len = window_len;
  at.bt_div = 1;
  if (av) {
    at.B = av->B;
    at.W = av->W;
    at.prefix_len = av->prefix_len;
    at.causal_rows = av->causal_rows;
    at.window_len = av->window_len;
    at.bt_div = av->bt_div;
  }
  LA_TRY(launch_attention(at, st));
  if (quant)
    if ((rs = pack_rows(at.out, HQ, T, HQ, nullptr, 0.f, s.apack, s.asum, wf, nullptr, 0, nullptr,
                        st)) != LA_OK)
      return rs;
  }

  const int F = m->inter;
  if (!quant && T <= 32) {
    if (!fp.grid) {
      // O projection: h += attn . Wo^T, h * post_norm packed for gate/up
      g = base_gemm(&L.o, T);
      g.apack = s.apack_o;
      g.residual = s.h;
      g.y = s.h;
      g.ldy = H;
      g.y_apack = s.apack;
      g.out_gain = L.post_norm;
      g.ss_out = s.ss;
      LA_TRY(launch_gemm(g, EPI_STORE, LA_W_BF16, st));
    }
    if (ev) LA_TRY(hipEventRecord(ev[1], st));
    if (!fp.gate_up) {
      // gate/up + 1/rms + SiLU, packed straight into the down operand
      g = base_gemm(&L.gate_up, T);
      g.apack = s.apack;
      g.ss_in = s.ss;
      g.ss_tiles = H / 16;
      g.eps = m->rms_eps;
      g.y_apack = s.apack_m;
      LA_TRY(launch_gemm(g, EPI_SILU, LA_W_BF16, st));
    }
    // down projection: K-slice partial sums when its plan splits K (a sliced
    // stream over every compute unit beats an unsplit one; the next input
    // packing adds them up), else h += directly with h * next_gain packed for
    // the next GEMM
    const int ks_d = gemm_ksplit(T, &L.down);
    g = base_gemm(&L.down, T);
    g.apack = s.apack_m;
    if (ks_d > 1) {
      g.partial = s.parts;
      carry->pending = ks_d;
    } else {
      g.residual = s.h;
      g.y = s.h;
      g.ldy = H;
      if (next_gain) {
        g.y_apack = s.apack;
        g.out_gain = next_gain;
        g.ss_out = s.ss;
        carry->packed = true;
      }
    }
    LA_TRY(launch_gemm(g, EPI_STORE, LA_W_BF16, st));
    return LA_OK;
  }

  // INT4, or more than 32 rows: O projection as K-slice partial sums (or h +=
  // directly), then a packing kernel adds them and normalises
  const int ks_o = gemm_ksplit(T, &L.o);
  g = base_gemm(&L.o, T);
  g.apack = quant ? s.apack : s.apack_o;  // bf16: packed by the attention merge
  g.asum = s.asum;
  if (ks_o > 1) {
    g.partial = s.parts;
  } else {
    g.residual = s.h;
    g.y = s.h;
    g.ldy = H;
  }
  LA_TRY(launch_gemm(g, EPI_STORE, wf, st));

  // h += O partial sums; RMSNorm; gate/up + SiLU (bf16: packed straight into
  // the down operand)
  if (ev) LA_TRY(hipEventRecord(ev[1], st));
  if ((rs = pack_rows(s.h, H, T, H, L.post_norm, m->rms_eps, s.apack, s.asum, wf, s.parts,
                      ks_o > 1 ? ks_o : 0, ks_o > 1 ? s.h : nullptr, st)) != LA_OK)
    return rs;
  g = base_gemm(&L.gate_up, T);
  g.apack = s.apack;
  g.asum = s.asum;
  if (quant) {
    g.y = s.mlp;
    g.ldy = F;
  } else {
    g.y_apack = s.apack_m;
  }
  LA_TRY(launch_gemm(g, EPI_SILU, wf, st));
  if (quant)
    if ((rs = pack_rows(s.mlp, F, T, F, nullptr, 0.f, s.apack_m, s.asum_m, wf, nullptr, 0, nullptr,
                        st)) != LA_OK)
      return rs;

  // down projection: K-slice partial sums left for the next packing
  const int ks_d = gemm_ksplit(T, &L.down);
  g = base_gemm(&L.down, T);
  g.apack = s.apack_m;
  g.asum = s.asum_m;
  if (ks_d > 1) {
    g.partial = s.parts;
  } else {
    g.residual = s.h;
    g.y = s.h;
    g.ldy = H;
  }
  LA_TRY(launch_gemm(g, EPI_STORE, wf, st));
  carry->pending = ks_d > 1 ? ks_d : 0;
  return LA_OK;
}

PrologueArgs base_prologue(const la_model* m, const la_kv_cache* kv, const int32_t* prefix_len,
                           int B, int W, int max_len, const StepWs& s) {
  PrologueArgs p;
  memset(&p, 0, sizeof(p));
  p.T = B * W;
  p.prefix_len = prefix_len;
  p.W = W;
  p.rope = s.rope;
  p.rope_theta = m->rope_theta;
  p.flags = s.flags;
  p.block_table = kv->block_table;
  p.max_blocks = kv->max_blocks;
  p.num_blocks = kv->num_blocks;
  p.cap = std::min(max_len, kv->max_blocks * kBlock);
  p.zero = s.sync;
  p.n_zero = s.n_sync;
  p.zero_blocks = std::min(64, std::max(1, (int)(((size_t)s.n_sync * 4 + 32767) / 32768)));
  return p;
}

la_status check_sampling(const la_sampling* smp) {
  if (!smp) return LA_ERR_ARG;
  if (!(smp->top_p > 0.f) || !(smp->top_p <= 1.f)) return LA_ERR_ARG;
  if (!(smp->temperature < INFINITY) || !(smp->temperature > -INFINITY)) return LA_ERR_ARG;
  return LA_OK;
}

SampleArgs sample_args(const la_sampling* smp, const float* logits, int M, int V, int ld) {
  SampleArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.logits = logits;
  sa.M = M;
  sa.V = V;
  sa.ldz = ld;
  sa.rep_rows = 1;
  sa.rep_theta = 1.f;
  sa.temperature = smp->temperature;
  sa.top_p = smp->top_p;
  sa.seed = smp->seed;
  sa.offset = smp->offset;
  sa.offset_dev = smp->offset_dev;
  return sa;
}

}  // namespace

extern "C" {

const char* la_status_str(int32_t status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_ERR_ARG: return "invalid argument";
    case LA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_UNSUPPORTED: return "unsupported request";
    case LA_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

la_status la_int4_embed_gather(const int32_t* ids, int32_t T, const la_weight* emb, float* out,
                               int32_t* err, hipStream_t stream) {
  if (!ids || !emb || !out || !emb->data || T < 0) return LA_ERR_ARG;
  if (emb->k < 8 || emb->k % 8 || emb->n < 1) return LA_ERR_SHAPE;
  if (emb->fmt == LA_W_INT4) {
    if (!emb->scales || emb->group < 8 || emb->group % 8 || emb->k % emb->group) return LA_ERR_SHAPE;
    if (emb->layout != LA_LAYOUT_ROWS) return LA_ERR_UNSUPPORTED;
  } else if (emb->fmt != LA_W_BF16) {
    return LA_ERR_ARG;
  } else if (emb->layout != LA_LAYOUT_ROWS && (emb->layout != LA_LAYOUT_TILED || emb->k % 32)) {
    return LA_ERR_UNSUPPORTED;
  }
  if (!aligned16(out) || !aligned16(emb->data)) return LA_ERR_ARG;
  if (T == 0) return LA_OK;
  PrologueArgs p;
  memset(&p, 0, sizeof(p));
  p.ids = ids;
  p.T = T;
  p.emb = *emb;
  p.out = out;
  p.err = err;
  return hip_status(launch_prologue(p, stream));
}

size_t la_packed_rows_bytes(int32_t M, int32_t K) {
  if (M < 1 || K < 256 || K % 256) return 0;
  Carver c(nullptr);
  c.take<uint16_t>(apack_elems(M, K));
  c.take<float>((size_t)((M + 7) / 8) * (K / 128) * 16);
  return c.off;
}

la_status la_pack_rows(const float* x, int32_t M, int32_t K, const uint16_t* norm_gain,
                       float rms_eps, int32_t fmt, void* packed, size_t packed_bytes,
                       hipStream_t stream) {
  if (!x || !packed) return LA_ERR_ARG;
  if (fmt != LA_W_BF16 && fmt != LA_W_INT4 && fmt != LA_W_W8A8) return LA_ERR_ARG;
  if (M < 1 || M > 512 || K < 256 || K % 256 || K > 16384) return LA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(packed) || (norm_gain && !aligned16(norm_gain))) return LA_ERR_ARG;
  if (norm_gain && !(rms_eps > 0.f)) return LA_ERR_ARG;
  if (packed_bytes < la_packed_rows_bytes(M, K)) return LA_ERR_WORKSPACE;
  Carver c(packed);
  uint16_t* apack = c.take<uint16_t>(apack_elems(M, K));
  float* asum = c.take<float>((size_t)((M + 7) / 8) * (K / 128) * 16);
  return pack_rows(x, K, M, K, norm_gain, rms_eps, apack, asum, fmt, nullptr, 0, nullptr, stream);
}

la_status la_wgemm_packed(const void* packed, int32_t M, const la_weight* w, const uint16_t* bias,
                          const float* residual, int32_t epilogue, float* y, hipStream_t stream) {
  if (!packed || !y || !w) return LA_ERR_ARG;
  if (epilogue != LA_EPI_NONE && epilogue != LA_EPI_SILU_GATE) return LA_ERR_ARG;
  if (M < 1 || M > 512) return LA_ERR_SHAPE;
  const int epi = epilogue == LA_EPI_SILU_GATE ? EPI_SILU : EPI_STORE;
  la_status st = check_gemm_weight(w, epi == EPI_SILU ? LA_LAYOUT_TILED_GU : LA_LAYOUT_TILED);
  if (st != LA_OK) return st;
  if (epi == EPI_SILU && (w->n % 16 || bias || residual)) return LA_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(y)) return LA_ERR_ARG;
  Carver c(const_cast<void*>(packed));
  GemmArgs g = base_gemm(w, M);
  g.apack = c.take<uint16_t>(apack_elems(M, w->k));
  g.asum = c.take<float>((size_t)((M + 7) / 8) * (w->k / 128) * 16);
  g.bias = bias;
  g.residual = residual;
  g.y = y;
  g.ldy = epi == EPI_SILU ? w->n / 2 : w->n;
  return hip_status(launch_gemm(g, epi, w->fmt, stream));
}

size_t la_wgemm_workspace(int32_t M, const la_weight* w, int32_t epilogue) {
  if (!w) return 0;
  (void)epilogue;
  return la_packed_rows_bytes(M, w->k);
}

la_status la_wgemm(const float* x, int32_t M, const la_weight* w, const uint16_t* norm_gain,
                   float rms_eps, const uint16_t* bias, const float* residual, int32_t epilogue,
                   float* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !y || !w) return LA_ERR_ARG;
  if (epilogue != LA_EPI_NONE && epilogue != LA_EPI_SILU_GATE) return LA_ERR_ARG;
  if (M < 1 || M > 512) return LA_ERR_SHAPE;
  const int epi = epilogue == LA_EPI_SILU_GATE ? EPI_SILU : EPI_STORE;
  la_status st = check_gemm_weight(w, epi == EPI_SILU ? LA_LAYOUT_TILED_GU : LA_LAYOUT_TILED);
  if (st != LA_OK) return st;
  if (epi == EPI_SILU && (w->n % 16 || bias || residual)) return LA_ERR_SHAPE;
  if (!aligned16(x) || (norm_gain && !aligned16(norm_gain))) return LA_ERR_ARG;
  if (norm_gain && !(rms_eps > 0.f)) return LA_ERR_ARG;
  const size_t need = la_wgemm_workspace(M, w, epilogue);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  if ((st = la_pack_rows(x, M, w->k, norm_gain, rms_eps, w->fmt, workspace, workspace_bytes,
                         stream)) != LA_OK)
    return st;
  return la_wgemm_packed(workspace, M, w, bias, residual, epilogue, y, stream);
}

size_t la_pbd_attention_workspace(int32_t B, int32_t W, int32_t n_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t max_len) {
  if (B < 1 || W < 1 || n_kv_heads < 1 || n_heads < n_kv_heads || head_dim != kHeadDim ||
      max_len < 1)
    return 0;
  int pps, ms;
  plan_attention(B, n_kv_heads, max_len, &pps, &ms);
  const size_t units = (size_t)B * n_kv_heads * ms * attn_nqp(W, n_heads / n_kv_heads);
  Carver c(nullptr);
  c.take<float>(units * kHeadDim);
  c.take<float>(units * 2);
  return c.off;
}

la_status la_pbd_attention(const float* q, const la_kv_cache* kv, int32_t layer, int32_t n_heads,
                           int32_t n_kv_heads, int32_t head_dim, const int32_t* prefix_len,
                           int32_t B, int32_t W, int32_t max_len, float* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return la_pbd_attention_masked(q, kv, layer, n_heads, n_kv_heads, head_dim, prefix_len, B, W,
                                 max_len, LA_MASK_BIDIRECTIONAL, out, workspace, workspace_bytes,
                                 stream);
}

la_status la_pbd_attention_masked(const float* q, const la_kv_cache* kv, int32_t layer,
                                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                  const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len,
                                  int32_t window_mask, float* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (window_mask != LA_MASK_BIDIRECTIONAL && window_mask != LA_MASK_CAUSAL) return LA_ERR_ARG;
  return attention_entry(q, kv, layer, n_heads, n_kv_heads, head_dim, prefix_len,
                         window_mask == LA_MASK_CAUSAL, nullptr, nullptr, B, W, max_len, out,
                         workspace, workspace_bytes, stream);
}

la_status la_pbd_attention_refeed(const float* q, const la_kv_cache* kv, int32_t layer,
                                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                  const int32_t* prefix_len, const int32_t* causal_rows,
                                  const int32_t* window_len, int32_t B, int32_t W, int32_t max_len,
                                  float* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (!causal_rows || !window_len) return LA_ERR_ARG;
  return attention_entry(q, kv, layer, n_heads, n_kv_heads, head_dim, prefix_len, false,
                         causal_rows, window_len, B, W, max_len, out, workspace, workspace_bytes,
                         stream);
}

}  // extern "C"

namespace {

la_status attention_entry(const float* q, const la_kv_cache* kv, int32_t layer, int32_t n_heads,
                          int32_t n_kv_heads, int32_t head_dim, const int32_t* prefix_len,
                          bool causal, const int32_t* causal_rows, const int32_t* window_len,
                          int32_t B, int32_t W, int32_t max_len, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (!q || !out || !prefix_len) return LA_ERR_ARG;
  la_status st = check_cache(kv, nullptr, B);
  if (st != LA_OK) return st;
  if (head_dim != kHeadDim || n_kv_heads < 1 || n_heads < n_kv_heads || n_heads % n_kv_heads)
    return LA_ERR_SHAPE;
  if (B < 1 || B > 64 || W < 1 || W > kMaxWindow || W * (n_heads / n_kv_heads) > kMaxQueryCols ||
      max_len < 1)
    return LA_ERR_SHAPE;
  if (layer < 0 || layer >= kv->n_layers) return LA_ERR_ARG;
  if (!aligned16(q) || !aligned16(out)) return LA_ERR_ARG;
  const size_t need = la_pbd_attention_workspace(B, W, n_heads, n_kv_heads, head_dim, max_len);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  AttnArgs at;
  memset(&at, 0, sizeof(at));
  const size_t le = (size_t)kv->num_blocks * n_kv_heads * kBlock * kHeadDim;
  at.q = q;
  at.kc = (const uint16_t*)kv->k + (size_t)layer * le;
  at.vc = (const uint16_t*)kv->v + (size_t)layer * le;
  at.block_table = kv->block_table;
  at.prefix_len = prefix_len;
  at.B = B;
  at.W = W;
  at.Hq = n_heads;
  at.Hkv = n_kv_heads;
  at.num_blocks = kv->num_blocks;
  at.max_blocks = kv->max_blocks;
  at.cap = std::min(max_len, kv->max_blocks * kBlock);
  plan_attention(B, n_kv_heads, max_len, &at.pages_per_split, &at.max_splits);
  at.nqp = attn_nqp(W, n_heads / n_kv_heads);
  Carver c(workspace);
  const size_t units = (size_t)B * n_kv_heads * at.max_splits * at.nqp;
  at.part_o = c.take<float>(units * kHeadDim);
  at.part_ml = c.take<float>(units * 2);
  at.out = out;
  at.bt_div = 1;
  at.causal = causal;
  at.causal_rows = causal_rows;
  at.window_len = window_len;
  return hip_status(launch_attention(at, stream));
}

}  // namespace

extern "C" {

size_t la_lm_head_argmax_workspace(int32_t M, const la_weight* lm) {
  if (!lm || M < 1 || lm->k < 256) return 0;
  Carver c(nullptr);
  c.take<uint16_t>(apack_elems(M, lm->k));
  c.take<float>((size_t)((M + 7) / 8) * (lm->k / 128) * 16);
  c.take<float>((size_t)M * gemm_parts(M, lm, EPI_ARGMAX) * 3);
  return c.off;
}

la_status la_lm_head_argmax(const float* h, int32_t M, const la_weight* lm,
                            const uint16_t* norm_gain, float rms_eps, int32_t* ids, float* top1,
                            float* gap, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return la_lm_head_argmax_penalized(h, M, lm, norm_gain, rms_eps, nullptr, 0, 1, 1.f, ids, top1,
                                     gap, workspace, workspace_bytes, stream);
}

la_status la_lm_head_argmax_penalized(const float* h, int32_t M, const la_weight* lm,
                                      const uint16_t* norm_gain, float rms_eps,
                                      const uint32_t* rep_bits, int32_t rep_words,
                                      int32_t rep_rows, float rep_penalty, int32_t* ids,
                                      float* top1, float* gap, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!h || !ids || !lm) return LA_ERR_ARG;
  if (rep_bits && (rep_rows < 1 || (int64_t)rep_words * 32 < (int64_t)lm->n ||
                   !(rep_penalty > 0.f) || !(rep_penalty < INFINITY)))
    return LA_ERR_ARG;
  if (M < 1 || M > 512) return LA_ERR_SHAPE;
  la_status st = check_gemm_weight(lm, LA_LAYOUT_TILED);
  if (st != LA_OK) return st;
  if (!aligned16(h) || (norm_gain && !aligned16(norm_gain))) return LA_ERR_ARG;
  if (norm_gain && !(rms_eps > 0.f)) return LA_ERR_ARG;
  const size_t need = la_lm_head_argmax_workspace(M, lm);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  Carver c(workspace);
  uint16_t* apack = c.take<uint16_t>(apack_elems(M, lm->k));
  float* asum = c.take<float>((size_t)((M + 7) / 8) * (lm->k / 128) * 16);
  const int parts = gemm_parts(M, lm, EPI_ARGMAX);
  float* amax = c.take<float>((size_t)M * parts * 3);
  GemmArgs g = base_gemm(lm, M);
  g.amax = amax;
  g.rep_bits = rep_bits;
  g.rep_words = rep_words;
  g.rep_rows = rep_rows;
  g.rep_theta = rep_penalty;
  if ((st = gemm_from_rows(g, h, lm->k, norm_gain, rms_eps, apack, asum, EPI_ARGMAX, lm->fmt, stream)) != LA_OK)
    return st;
  return hip_status(launch_argmax_reduce(amax, M, parts, nullptr, ids, top1, gap, nullptr, stream));
}

la_status la_sample_logits(const float* logits, int32_t M, int32_t V, int32_t ld,
                           const uint32_t* rep_bits, int32_t rep_words, int32_t rep_rows,
                           float rep_penalty, const la_sampling* smp, int32_t* ids, float* sel_gap,
                           hipStream_t stream) {
  if (!logits || !ids || !smp) return LA_ERR_ARG;
  la_status st = check_sampling(smp);
  if (st != LA_OK) return st;
  if (M < 1 || M > 65535 || V < 1 || ld < V) return LA_ERR_SHAPE;
  if (rep_bits && (rep_rows < 1 || (int64_t)rep_words * 32 < (int64_t)V || !(rep_penalty > 0.f) ||
                   !(rep_penalty < INFINITY)))
    return LA_ERR_ARG;
  SampleArgs sa = sample_args(smp, logits, M, V, ld);
  if (rep_bits) {
    sa.rep_bits = rep_bits;
    sa.rep_words = rep_words;
    sa.rep_rows = rep_rows;
    sa.rep_theta = rep_penalty;
  }
  sa.ids = ids;
  sa.sel_gap = sel_gap;
  return hip_status(launch_sample(sa, stream));
}

la_status la_pbd_layer(const la_model* m, int32_t layer, const la_kv_cache* kv, const float* x,
                       const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len, float* y,
                       float* attn_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  la_status st = check_model(m);
  if (st != LA_OK) return st;
  if ((st = check_cache(kv, m, B)) != LA_OK) return st;
  if ((st = check_step_shape(m, B, W, max_len)) != LA_OK) return st;
  if (!x || !y || !prefix_len) return LA_ERR_ARG;
  if (layer < 0 || layer >= m->n_layers) return LA_ERR_ARG;
  if (!aligned16(x) || !aligned16(y) || (attn_out && !aligned16(attn_out))) return LA_ERR_ARG;
  const size_t need = carve_step(m, B, W, max_len, nullptr, false).bytes;
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  StepWs s = carve_step(m, B, W, max_len, workspace, false);
  const int T = B * W;
  const int H = m->hidden;
  s.h = y;  // the layer runs in place on y
  if (y != x) LA_TRY(hipMemcpyAsync(y, x, (size_t)T * H * sizeof(float), hipMemcpyDeviceToDevice, stream));
  PrologueArgs p = base_prologue(m, kv, prefix_len, B, W, max_len, s);
  LA_TRY(launch_prologue(p, stream));
  Carry carry;
  if ((st = run_layer(m, layer, kv, prefix_len, nullptr, nullptr, B, W, max_len, s, attn_out,
                      &carry, nullptr, stream)) != LA_OK)
    return st;
  if (carry.pending)
    return pack_rows(y, H, T, H, nullptr, 0.f, nullptr, nullptr, LA_W_BF16, s.parts, carry.pending, y,
                     stream);
  return LA_OK;
}

size_t la_pbd_step_workspace(const la_model* m, int32_t B, int32_t W, int32_t max_len) {
  if (check_model(m) != LA_OK || B < 1 || W < 1 || max_len < W) return 0;
  return carve_step(m, B, W, max_len, nullptr, true).bytes;
}

la_status la_pbd_step(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                      const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len,
                      int32_t* out_ids, float* out_gap, float* out_hidden, void* workspace,
                      size_t workspace_bytes, int32_t* err, hipStream_t stream) {
  return la_pbd_step_opts(m, kv, window_ids, prefix_len, nullptr, B, W, max_len, out_ids, out_gap,
                          out_hidden, workspace, workspace_bytes, err, stream);
}

la_status la_pbd_step_refeed(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                             const int32_t* prefix_len, const int32_t* causal_rows,
                             const int32_t* window_len, int32_t B, int32_t W, int32_t max_len,
                             int32_t* out_ids, float* out_gap, float* out_hidden, void* workspace,
                             size_t workspace_bytes, int32_t* err, hipStream_t stream) {
  la_step_opts o;
  memset(&o, 0, sizeof(o));
  o.causal_rows = causal_rows;
  o.window_len = window_len;
  o.rep_penalty = 1.f;
  return la_pbd_step_opts(m, kv, window_ids, prefix_len, &o, B, W, max_len, out_ids, out_gap,
                          out_hidden, workspace, workspace_bytes, err, stream);
}

la_status la_pbd_step_opts(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                           const int32_t* prefix_len, const la_step_opts* opts, int32_t B, int32_t W,
                           int32_t max_len, int32_t* out_ids, float* out_gap, float* out_hidden,
                           void* workspace, size_t workspace_bytes, int32_t* err,
                           hipStream_t stream) {
  la_status st = check_model(m);
  if (st != LA_OK) return st;
  const int32_t* causal_rows = opts ? opts->causal_rows : nullptr;
  const int32_t* window_len = opts ? opts->window_len : nullptr;
  const la_sampling* smp = opts ? opts->sampling : nullptr;
  if (smp && (st = check_sampling(smp)) != LA_OK) return st;
  const bool sampled = smp && smp->temperature > 0.f;
  if (sampled && (!smp->logits || !aligned16(smp->logits))) return LA_ERR_ARG;
  if (opts && opts->rep_bits &&
      (!(opts->rep_penalty > 0.f) || !(opts->rep_penalty < INFINITY) ||
       (int64_t)opts->rep_words * 32 < (int64_t)(m->lm_head.data ? m->lm_head.n : m->embed.n)))
    return LA_ERR_ARG;
  if ((st = check_cache(kv, m, B)) != LA_OK) return st;
  if ((st = check_step_shape(m, B, W, max_len)) != LA_OK) return st;
  if (!window_ids || !prefix_len || !out_ids) return LA_ERR_ARG;
  if (out_hidden && !aligned16(out_hidden)) return LA_ERR_ARG;
  const size_t need = carve_step(m, B, W, max_len, nullptr, true).bytes;
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  StepWs s = carve_step(m, B, W, max_len, workspace, true);
  s.err = err;
  const int T = B * W;
  const int H = m->hidden;

  PrologueArgs p = base_prologue(m, kv, prefix_len, B, W, max_len, s);
  p.ids = window_ids;
  p.emb = m->embed;
  p.out = s.h;
  p.err = err;
  p.causal_rows = causal_rows;
  p.window_len = window_len;
  LA_TRY(launch_prologue(p, stream));
  Carry carry;
  const la_weight* lm = m->lm_head.data ? &m->lm_head : &m->embed;
  const bool quant_lm = lm->fmt != LA_W_BF16;
  for (int l = 0; l < m->n_layers; ++l) {
    // the gain after layer l: the next input norm, or the final norm when the
    // lm_head takes the packed rows directly (bf16)
    // (sampling stores the logits themselves: the final norm is applied by the
    // packing below, not folded into the lm_head's epilogue)
    const uint16_t* next_gain = l + 1 < m->n_layers ? m->layers[l + 1].in_norm
                                                    : (quant_lm || sampled ? nullptr : m->final_norm);
    const hipEvent_t* ev = opts && opts->block_events ? opts->block_events + 2 * l : nullptr;
    st = run_layer(m, l, kv, prefix_len, causal_rows, window_len, B, W, max_len, s, nullptr, &carry,
                   next_gain, stream, nullptr, ev);
    if (st != LA_OK) return st;
  }
  if (!carry.packed) {
    // h += last partial sums (written back for out_hidden); final RMSNorm; pack
    if ((st = pack_rows(s.h, H, T, H, m->final_norm, m->rms_eps, s.apack, s.asum, lm->fmt, s.parts,
                        carry.pending, carry.pending ? s.h : nullptr, stream)) != LA_OK)
      return st;
  }
  if (out_hidden)
    LA_TRY(hipMemcpyAsync(out_hidden, s.h, (size_t)T * H * sizeof(float), hipMemcpyDeviceToDevice,
                          stream));
  if (sampled) {
    // the logits of every row, then the sampled selection
    GemmArgs g = base_gemm(lm, T);
    g.apack = s.apack;
    g.asum = s.asum;
    g.y = smp->logits;
    g.ldy = lm->n;
    LA_TRY(launch_gemm(g, EPI_STORE, lm->fmt, stream));
    SampleArgs sa = sample_args(smp, smp->logits, T, lm->n, lm->n);
    if (opts->rep_bits) {
      sa.rep_bits = opts->rep_bits;
      sa.rep_words = opts->rep_words;
      sa.rep_rows = W;
      sa.rep_theta = opts->rep_penalty;
    }
    sa.flags = s.flags;
    sa.ids = out_ids;
    sa.sel_gap = out_gap;
    sa.err = err;
    return hip_status(launch_sample(sa, stream));
  }
  GemmArgs g = base_gemm(lm, T);
  g.amax = s.amax;
  g.apack = s.apack;
  g.asum = s.asum;
  if (opts && opts->rep_bits) {
    g.rep_bits = opts->rep_bits;
    g.rep_words = opts->rep_words;
    g.rep_rows = W;
    g.rep_theta = opts->rep_penalty;
  }
  if (carry.packed) {
    g.ss_in = s.ss;
    g.ss_tiles = H / 16;
    g.eps = m->rms_eps;
  }
  LA_TRY(launch_gemm(g, EPI_ARGMAX, lm->fmt, stream));
  return hip_status(launch_argmax_reduce(s.amax, T, s.vocab_parts, s.flags, out_ids, nullptr, out_gap,
                                         nullptr, stream));
}

size_t la_pbd_prefill_workspace(const la_model* m, int32_t B, int32_t L, int32_t max_len) {
  if (check_model(m) != LA_OK || B < 1 || B > 64 || L < 1) return 0;
  const int chunks = (L + kPrefillChunk - 1) / kPrefillChunk, Lp = chunks * kPrefillChunk;
  if (max_len < Lp || (int64_t)B * Lp > kMaxPrefillRows) return 0;
  return carve_step(m, B, Lp, max_len, nullptr, true, chunks).bytes;
}

la_status la_pbd_prefill(const la_model* m, const la_kv_cache* kv, const int32_t* ids,
                         const float* embeds, const int32_t* prefix_len, int32_t B, int32_t L,
                         int32_t max_len, int32_t* out_ids, float* out_gap, float* out_hidden,
                         void* workspace, size_t workspace_bytes, int32_t* err,
                         hipStream_t stream) {
  la_status st = check_model(m);
  if (st != LA_OK) return st;
  if ((st = check_cache(kv, m, B)) != LA_OK) return st;
  if (B < 1 || B > 64 || L < 1) return LA_ERR_SHAPE;
  const int chunks = (L + kPrefillChunk - 1) / kPrefillChunk, Lp = chunks * kPrefillChunk;
  if (max_len < Lp || (int64_t)B * Lp > kMaxPrefillRows) return LA_ERR_SHAPE;
  if (!ids || !prefix_len || !out_ids) return LA_ERR_ARG;
  if ((embeds && !aligned16(embeds)) || (out_hidden && !aligned16(out_hidden))) return LA_ERR_ARG;
  const size_t need = carve_step(m, B, Lp, max_len, nullptr, true, chunks).bytes;
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  const StepWs s = carve_step(m, B, Lp, max_len, workspace, true, chunks);
  const int T = B * Lp;
  const int H = m->hidden;

  // the prompt rows: gathered or spliced, RoPE at P_b + j, flags; the
  // attention's 16-row windows
  LA_TRY(launch_prefill_views(prefix_len, B, L, chunks, s.pre_prefix, s.pre_causal, s.pre_wlen, stream));
  PrologueArgs p = base_prologue(m, kv, prefix_len, B, Lp, max_len, s);
  p.ids = ids;
  p.emb = m->embed;
  p.out = s.h;
  p.err = err;
  p.in_w = L;
  p.embeds = embeds;
  LA_TRY(launch_prologue(p, stream));
  const AttnView av{B * chunks, kPrefillChunk, s.pre_prefix, s.pre_causal, s.pre_wlen, chunks};
  Carry carry;
  for (int l = 0; l < m->n_layers; ++l) {
    const uint16_t* next_gain = l + 1 < m->n_layers ? m->layers[l + 1].in_norm : nullptr;
    st = run_layer(m, l, kv, prefix_len, nullptr, nullptr, B, Lp, max_len, s, nullptr, &carry,
                   next_gain, stream, &av);
    if (st != LA_OK) return st;
  }
  if (carry.pending &&
      (st = pack_rows(s.h, H, T, H, nullptr, 0.f, nullptr, nullptr, LA_W_BF16, s.parts, carry.pending,
                      s.h, stream)) != LA_OK)
    return st;
  // each sequence's last prompt row (and its flags) -> final norm, lm_head, argmax
  LA_TRY(hipMemcpy2DAsync(s.h_last, (size_t)H * sizeof(float), s.h + (size_t)(L - 1) * H,
                          (size_t)Lp * H * sizeof(float), (size_t)H * sizeof(float), B,
                          hipMemcpyDeviceToDevice, stream));
  LA_TRY(hipMemcpy2DAsync(s.pre_flags, sizeof(int32_t), s.flags + (L - 1), (size_t)Lp * sizeof(int32_t),
                          sizeof(int32_t), B, hipMemcpyDeviceToDevice, stream));
  if (out_hidden)
    LA_TRY(hipMemcpyAsync(out_hidden, s.h_last, (size_t)B * H * sizeof(float), hipMemcpyDeviceToDevice,
                          stream));
  const la_weight* lm = m->lm_head.data ? &m->lm_head : &m->embed;
  GemmArgs g = base_gemm(lm, B);
  g.amax = s.amax;
  if ((st = gemm_from_rows(g, s.h_last, H, m->final_norm, m->rms_eps, s.apack, s.asum, EPI_ARGMAX,
                           lm->fmt, stream)) != LA_OK)
    return st;
  return hip_status(launch_argmax_reduce(s.amax, B, s.vocab_parts, s.pre_flags, out_ids, nullptr,
                                         out_gap, nullptr, stream));
}

size_t la_pack_weight_bytes(const la_weight* src, int32_t layout, int32_t scales) {
  if (!src || src->layout != LA_LAYOUT_ROWS || src->n < 1 || src->k < 128 || src->k % 128) return 0;
  if (layout != LA_LAYOUT_TILED && layout != LA_LAYOUT_TILED_GU && layout != LA_LAYOUT_TILED_QKV) return 0;
  if (src->fmt != LA_W_BF16 && src->fmt != LA_W_W8A8 && !(src->fmt == LA_W_INT4 && src->group == 128)) return 0;
  if (layout == LA_LAYOUT_TILED_GU && src->n % 16) return 0;
  if (layout == LA_LAYOUT_TILED_QKV && src->n % kHeadDim) return 0;
  const size_t n_tiles = layout == LA_LAYOUT_TILED_GU ? (size_t)(src->n / 2 + 7) / 8 : (size_t)(src->n + 15) / 16;
  if (scales) return src->fmt == LA_W_INT4 ? n_tiles * (src->k / 128) * 16 * 2 : src->fmt == LA_W_W8A8 ? (size_t)src->n * 4 : 0;
  return src->fmt == LA_W_INT4 ? n_tiles * 16 * (size_t)(src->k / 2)
         : src->fmt == LA_W_W8A8 ? n_tiles * 16 * (size_t)src->k : n_tiles * 16 * (size_t)src->k * 2;
}

la_status la_pack_weight(const la_weight* src, int32_t layout, void* dst, void* dst_scales,
                         hipStream_t stream) {
  if (!src || !src->data || !dst) return LA_ERR_ARG;
  if (la_pack_weight_bytes(src, layout, 0) == 0) return LA_ERR_SHAPE;
  if (src->fmt != LA_W_BF16 && (!src->scales || !dst_scales)) return LA_ERR_ARG;
  if (!aligned16(src->data) || !aligned16(dst)) return LA_ERR_ARG;
  return hip_status(launch_pack_weight(*src, layout, dst, dst_scales, stream));
}

la_status la_pbd_commit(const int32_t* out_ids, int32_t* window_ids, int32_t* prefix_len,
                        int32_t B, int32_t W, int32_t mask_id, hipStream_t stream) {
  if (!out_ids || !window_ids || !prefix_len) return LA_ERR_ARG;
  if ((const void*)out_ids == (const void*)window_ids) return LA_ERR_ARG;
  if (B < 1 || B > 64 || W < 1 || W > kMaxWindow) return LA_ERR_SHAPE;
  return hip_status(launch_commit(out_ids, window_ids, prefix_len, B, W, mask_id, stream));
}

la_status la_pbd_mark_tokens(const int32_t* ids, int32_t B, int32_t W, const int32_t* first,
                             const int32_t* count, uint32_t* bits, int32_t words, int32_t vocab,
                             hipStream_t stream) {
  if (!ids || !bits) return LA_ERR_ARG;
  if (B < 1 || B > 64 || W < 1 || W > kMaxWindow || vocab < 1 || (int64_t)words * 32 < vocab)
    return LA_ERR_SHAPE;
  return hip_status(launch_mark_tokens(ids, B, W, first, count, bits, words, vocab, stream));
}

la_status la_pbd_commit_refeed(const int32_t* out_ids, const int32_t* n_accept, int32_t* window_ids,
                               int32_t* prefix_len, int32_t* causal_rows, int32_t* window_len,
                               int32_t B, int32_t W, int32_t block, int32_t mask_id,
                               hipStream_t stream) {
  if (!out_ids || !window_ids || !prefix_len || !causal_rows || !window_len) return LA_ERR_ARG;
  const void* state[4] = {window_ids, prefix_len, causal_rows, window_len};
  for (const void* p : state)
    if (p == (const void*)out_ids || (n_accept && p == (const void*)n_accept)) return LA_ERR_ARG;
  if (B < 1 || B > 64 || W < 1 || W > kMaxWindow || block < 1 || block > W) return LA_ERR_SHAPE;
  return hip_status(launch_commit_refeed(out_ids, n_accept, window_ids, prefix_len, causal_rows,
                                         window_len, B, W, block, mask_id, stream));
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free step
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it): the step's scratch lives in
// a fixed array of this library, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it resolves the array's device address
// once per device with hipGetSymbolAddress and uses that address.

namespace {

constexpr size_t kStepScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStepScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (resolved on the first call on that
// device, with that device current).
la_status step_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace

extern "C" la_status la_pbd_step_noalloc(const la_model* m, const la_kv_cache* kv,
                                         const int32_t* window_ids, const int32_t* prefix_len,
                                         int32_t B, int32_t W, int32_t max_len, int32_t* out_ids,
                                         float* out_gap, float* out_hidden, int32_t* err,
                                         hipStream_t stream) {
  la_status st = check_model(m);
  if (st != LA_OK) return st;
  if ((st = check_step_shape(m, B, W, max_len)) != LA_OK) return st;
  const size_t need = carve_step(m, B, W, max_len, nullptr, true).bytes;
  if (need > kStepScratchBytes) return LA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = step_scratch(&ws)) != LA_OK) return st;
  return la_pbd_step(m, kv, window_ids, prefix_len, B, W, max_len, out_ids, out_gap, out_hidden, ws,
                     kStepScratchBytes, err, stream);
}
