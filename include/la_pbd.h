/*
 * la_pbd.h — C ABI of the MI355X (gfx950) Parallel Box Decoding window step.
 *
 * The step: a window of W tokens (the last accepted token followed by mask
 * tokens) sits at positions P_b .. P_b+W-1 after a cached prefix of P_b tokens.
 * Its rows go through a Qwen2-style decoder whose attention is causal to the
 * cached prefix and bidirectional inside the window, and the step ends with a
 * per-position argmax over the lm_head tied to the input embedding.
 * Sources: "LocateAnything-3B for RK3588 (RKLLM + RKNN)", section "How it
 * differs from the original", item 1 (window make-up, bidirectional window,
 * prefix KV reuse without rollback, original positions); "LocateAnything-3B on
 * Jetson Orin Nano", Part 1 sections 1.2-1.4 (Qwen2 decoder, block mask, greedy
 * selection); "LocateAnything-3B — ONNX WebGPU (INT4 + 4-bit embeddings)",
 * sections "Why this repo exists", "Files", "Embedding gather / dequant (JS
 * reference)" and "KV-cache graph for in-browser use" (tied lm_head, INT4
 * formats, GQA KV of 2 heads x 128).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *    buffer; the library allocates and frees nothing and keeps no pointer after
 *    a call returns.
 *  - Every call only enqueues work on `stream` and returns; nothing is
 *    synchronised.  Results are valid once the stream has reached that point.
 *  - Shape and argument errors are detected on the host before any launch and
 *    returned as la_status; nothing is enqueued then.  Launch failures return
 *    LA_ERR_HIP.
 *  - bf16 values are passed as uint16 bit patterns; fp16 scales likewise.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - Supported model shapes: head_dim 128, n_heads a multiple of n_kv_heads,
 *    hidden, n_heads*head_dim and inter multiples of 256, KV block size 16,
 *    window 1 <= W <= 16 with W * (n_heads / n_kv_heads) <= 128, batch 1..64.
 */
#ifndef LA_PBD_H
#define LA_PBD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_ARG = -1,         /* NULL where required, negative size, bad enum */
  LA_ERR_SHAPE = -2,       /* shape outside the supported set */
  LA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than the *_workspace() size */
  LA_ERR_UNSUPPORTED = -4, /* valid request this build does not implement */
  LA_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} la_status;

/* Weight formats. */
enum { LA_W_BF16 = 0, LA_W_INT4 = 1, LA_W_W8A8 = 2 };

/* Weight layouts.  LA_LAYOUT_ROWS is the plain row-major matrix.  The tiled
 * layouts hold the same values regrouped in tiles of 16 rows so that the
 * matrix-core operand of one wave is one contiguous 1 KB block; they are
 * written once by la_pack_weight.  Which 16 rows form tile t:
 *   LA_LAYOUT_TILED     rows 16t .. 16t+15 (rows >= n are zero);
 *   LA_LAYOUT_TILED_GU  rows 8t .. 8t+7 and n/2 + 8t .. n/2 + 8t+7 (the gate
 *                       rows and the matching up rows of a [gate | up] matrix);
 *   LA_LAYOUT_TILED_QKV for head h = t / 8, s = t % 8: rows 128h + 8s .. +7
 *                       and 128h + 64 + 8s .. +7 (the RoPE pairs of a head).
 * bf16 tiled: data = bf16 [n_tiles][k/32][64][8]; entry [t][u][16g + c][e] is
 *   row c of tile t at column 32u + 8g + e.
 * INT4 tiled (group 128): data = uint8 [n_tiles][k/128][64][16]; entry
 *   [t][u][16g + c] holds the 32 codes of row c of tile t at columns
 *   128u + 32g .. +31 packed as in row-major storage; scales = fp16
 *   [n_tiles][k/128][16] (scale of row c of tile t, group u).
 * w8a8 tiled: data = int8 [n_tiles][k/64][64][16]; entry [t][u][16g + c] holds
 *   row c of tile t at columns 64u + 16g .. +15; scales stay fp32 [n], indexed
 *   by weight row. */
enum { LA_LAYOUT_ROWS = 0, LA_LAYOUT_TILED = 1, LA_LAYOUT_TILED_GU = 2, LA_LAYOUT_TILED_QKV = 3 };

/* A weight matrix W[n, k] (y = x . W^T).
 *  LA_W_BF16: data = bf16 [n][k] row-major, scales = NULL, group ignored.
 *  LA_W_INT4: group-wise symmetric INT4 (WebGPU page, "Embedding gather /
 *    dequant"): data = uint8 [n][k/2], byte i of a row holds element 2i in its
 *    low nibble and element 2i+1 in its high nibble; scales = fp16 [n][k/group];
 *    element j of row r is (q - 8) * scales[r][j / group].  group is 32 for the
 *    embedding and 128 for the linears and the lm_head.
 *  LA_W_W8A8: the RK3588 conversion's format ("LocateAnything-3B for RK3588
 *    (RKLLM + RKNN)", "Files"; "How it differs from the original", item 3),
 *    read as: data = int8 [n][k] codes, scales = fp32 [n], element j of row r
 *    is q * scales[r]; the activations entering the product are quantised per
 *    row to int8 (s = max|x| / 127, q = round-half-even(x / s) clamped to
 *    [-127, 127], decided in fp32) and the int32 sums are scaled by both
 *    scales.  group ignored; k a multiple of 64.  A w8a8 model has w8a8
 *    linears, a bf16 embedding and a w8a8 lm_head (the tied matrix's copy).
 *  layout: one of LA_LAYOUT_*, as above. */
typedef struct {
  int32_t fmt;
  int32_t n;
  int32_t k;
  int32_t group;
  int32_t layout;
  int32_t reserved;
  const void* data;
  const void* scales;
} la_weight;

/* One decoder layer.  qkv is [q | k | v] stacked along n (n = (Hq + 2 Hkv) D);
 * gate_up is [gate | up] stacked along n (n = 2 F); o is [H, Hq D]; down is
 * [H, F].  Gains are bf16 [H]; qkv_bias is bf16 [(Hq + 2 Hkv) D] or NULL. */
typedef struct {
  const uint16_t* in_norm;
  const uint16_t* post_norm;
  la_weight qkv;
  const uint16_t* qkv_bias;
  la_weight o;
  la_weight gate_up;
  la_weight down;
} la_layer;

/* The decoder.  `layers` is a HOST array of n_layers entries (its device
 * pointers are read during the call only).  The lm_head is tied: with
 * lm_head.data == NULL the (bf16) embedding matrix is the lm_head; an INT4
 * model passes its group-128 copy of the tied matrix in lm_head. */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, inter, n_layers, vocab;
  float rms_eps;
  float rope_theta;
  const la_layer* layers;
  la_weight embed;
  la_weight lm_head;
  const uint16_t* final_norm;
  int32_t window_mask;  /* LA_MASK_BIDIRECTIONAL (0) or LA_MASK_CAUSAL */
} la_model;

/* Attention mask inside the window.  Bidirectional is the PBD window of the
 * original model (Jetson page, Part 1 section 1.3); causal is the mask the
 * RK3588 conversion evaluates it with ("LocateAnything-3B for RK3588 (RKLLM +
 * RKNN)", "How it differs from the original", item 1): window row j sees the
 * prefix and window rows 0..j. */
enum { LA_MASK_BIDIRECTIONAL = 0, LA_MASK_CAUSAL = 1 };

/* Paged bf16 KV cache (the pages' KV graph keeps [1, 2, seq, 128] per layer;
 * here the sequence axis is paged in blocks of `block_size` = 16 tokens):
 *   k: bf16 [n_layers][num_blocks][n_kv_heads][block_size][head_dim]
 *   v: bf16 [n_layers][num_blocks][n_kv_heads][head_dim][block_size]  (dim-major page)
 *   block_table: int32 [B][max_blocks]; token t of sequence b lives in block
 *   block_table[b][t / 16] at offset t % 16. */
typedef struct {
  void* k;
  void* v;
  const int32_t* block_table;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t block_size;
  int32_t n_layers;
} la_kv_cache;

/* Error bits written (OR-ed) into the optional device word `err`. */
enum {
  LA_DERR_TOKEN_ID = 1,   /* a window id outside [0, vocab) */
  LA_DERR_CAPACITY = 2,   /* P_b + W exceeds max_len or max_blocks * 16 */
  LA_DERR_BLOCK_ID = 4,   /* a block-table entry needed by the step is outside [0, num_blocks) */
  LA_DERR_WINDOW = 8,     /* re-fed window: window_len[b] outside 1..W or causal_rows[b] outside 0..window_len[b] */
  LA_DERR_SYNC = 16       /* a step's persistent front-half launch timed out waiting for its own
                             workgroups (the device did not run them all together); results invalid */
};

/* la_pbd_step epilogue selectors for la_wgemm. */
enum {
  LA_EPI_NONE = 0,      /* y[M][n] = x' . W^T (+ bias) (+ residual) */
  LA_EPI_SILU_GATE = 1  /* y[M][n/2] = SiLU(g) * u, g = columns [0, n/2), u = [n/2, n) */
};

/* Embedding gather: out[t][:] = E[ids[t]] as fp32, from a bf16 table or an INT4
 * group-32 table decoded as (q - 8) * scale (WebGPU page, "Embedding gather /
 * dequant (JS reference)").  ids int32 [T]; out fp32 [T][emb->k].  An id outside
 * [0, emb->n) yields a zero row and sets LA_DERR_TOKEN_ID in *err (err may be
 * NULL).  Exact: no rounding happens. */
la_status la_int4_embed_gather(const int32_t* ids, int32_t T, const la_weight* emb, float* out,
                               int32_t* err, hipStream_t stream);

/* Weight-streaming GEMM for small M (M = 6 x batch rows): one linear layer of
 * the decoder, y = x' . W^T, as the standard Qwen2 layers apply them ("LocateAnything-3B
 * on Jetson Orin Nano", Part 1 section 1.2: the language model is a plain Qwen2
 * causal LM; its projections are the QKV, O, gate/up and down linears, with
 * group-wise INT4 weights as in "LocateAnything-3B — ONNX WebGPU (INT4 + 4-bit
 * embeddings)", section "Files", block 128):
 *   x' = RMSNorm(x; norm_gain, rms_eps) if norm_gain != NULL, else x;
 *   LA_EPI_NONE:      y = x' . W^T + bias + residual  (bias bf16 [n] / residual fp32 [M][n], each nullable)
 *   LA_EPI_SILU_GATE: y = SiLU(x' . Wg^T) * (x' . Wu^T), Wg / Wu the two halves of W's rows.
 * x fp32 [M][w->k]; y fp32 [M][n] (or [M][n/2]).  y may alias residual.
 * Arithmetic: weights exact, activations split into bf16 hi + lo parts, fp32
 * accumulation on the matrix cores.  1 <= M <= 64. */
size_t la_wgemm_workspace(int32_t M, const la_weight* w, int32_t epilogue);
la_status la_wgemm(const float* x, int32_t M, const la_weight* w, const uint16_t* norm_gain,
                   float rms_eps, const uint16_t* bias, const float* residual, int32_t epilogue,
                   float* y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two halves of la_wgemm, for callers that reuse one packed operand or
 * time the GEMM alone.  la_pack_rows writes x' (as above) for a weight of
 * format fmt (LA_W_BF16 / LA_W_INT4 / LA_W_W8A8: the operand layout differs) into `packed`
 * (caller-owned device memory of la_packed_rows_bytes(M, K) bytes, 16-byte
 * aligned; x fp32 [M][K], 256 <= K <= 16384, K % 256 == 0).  la_wgemm_packed
 * runs the GEMM and epilogue of la_wgemm on such an operand; w->k must equal
 * the K it was packed with and w->fmt its fmt (not checkable: the operand
 * carries no header).  Errors as la_wgemm; no workspace is needed. */
size_t la_packed_rows_bytes(int32_t M, int32_t K);
la_status la_pack_rows(const float* x, int32_t M, int32_t K, const uint16_t* norm_gain,
                       float rms_eps, int32_t fmt, void* packed, size_t packed_bytes,
                       hipStream_t stream);
la_status la_wgemm_packed(const void* packed, int32_t M, const la_weight* w, const uint16_t* bias,
                          const float* residual, int32_t epilogue, float* y, hipStream_t stream);

/* Block-masked GQA attention of the window rows over the paged cache of one
 * layer: the window rows attend to the whole cached prefix and to every row of
 * the window ("LocateAnything-3B on Jetson Orin Nano", Part 1 section 1.3: a
 * block mask instead of a strictly causal one; "LocateAnything-3B for RK3588
 * (RKLLM + RKNN)", "How it differs from the original", item 1: the prefix KV is
 * reused and the window sits at the original positions after it).  q fp32 [B][W][n_heads][head_dim] (RoPE already applied); the keys of
 * sequence b are cache slots 0 .. P_b+W-1 (the window's own K/V must already be
 * stored at P_b .. P_b+W-1): every window row sees all of them (prefix causal,
 * window bidirectional).  out fp32 [B][W][n_heads][head_dim] =
 * softmax(q.K^T / sqrt(D)) . V, query head h reading KV head h / (n_heads /
 * n_kv_heads).  prefix_len int32 [B] (device); max_len (host) is an upper bound
 * of every P_b + W and sizes the split-K grid; keys beyond the cache capacity
 * are ignored. */
/* Workspace of la_pbd_attention (and its masked / re-fed forms): the split-K
 * partial results (per run: running max, sum and unnormalised output) that the
 * log-sum-exp merge combines; 0 for an unsupported shape. */
size_t la_pbd_attention_workspace(int32_t B, int32_t W, int32_t n_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t max_len);
/* The same with the window mask chosen: LA_MASK_BIDIRECTIONAL (as
 * la_pbd_attention) or LA_MASK_CAUSAL (window row j sees slots 0 .. P_b + j).
 * Any other value returns LA_ERR_ARG. */
la_status la_pbd_attention_masked(const float* q, const la_kv_cache* kv, int32_t layer,
                                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                  const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len,
                                  int32_t window_mask, float* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);
la_status la_pbd_attention(const float* q, const la_kv_cache* kv, int32_t layer, int32_t n_heads,
                           int32_t n_kv_heads, int32_t head_dim, const int32_t* prefix_len,
                           int32_t B, int32_t W, int32_t max_len, float* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);
/* Re-fed window ("LocateAnything-3B for RK3588 (RKLLM + RKNN)", "How it
 * differs from the original", item 1: each step sends the accepted tokens
 * again together with the mask tokens).  causal_rows and window_len are int32
 * [B] device arrays (both required).  The first c_b = causal_rows[b] rows of
 * sequence b re-feed accepted tokens causally: row j < c_b sees slots
 * 0 .. P_b + j.  Rows c_b .. w_b - 1 (w_b = window_len[b]) form the
 * bidirectional block: each sees slots 0 .. P_b + w_b - 1.  Rows from w_b to W
 * are padding; no real row sees them, and they see what the block sees.
 * Values outside 1 <= w_b <= W, 0 <= c_b <= W are clamped into them.  c_b = 0,
 * w_b = W is la_pbd_attention; c_b = W is the causal window.  Same workspace
 * and errors as la_pbd_attention. */
la_status la_pbd_attention_refeed(const float* q, const la_kv_cache* kv, int32_t layer,
                                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                  const int32_t* prefix_len, const int32_t* causal_rows,
                                  const int32_t* window_len, int32_t B, int32_t W, int32_t max_len,
                                  float* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Tied lm_head with per-row argmax (greedy selection; Jetson page, section 1.4).
 * f = RMSNorm(h; norm_gain, rms_eps) if norm_gain != NULL else h; logits =
 * f . E^T over the lm->n vocabulary rows (never stored).  ids int32 [M] = argmax
 * (lowest index on an exact tie); top1 fp32 [M] = max logit; gap fp32 [M] =
 * top1 - second largest logit (0 on a tie).  top1 / gap nullable. */
size_t la_lm_head_argmax_workspace(int32_t M, const la_weight* lm);
la_status la_lm_head_argmax(const float* h, int32_t M, const la_weight* lm,
                            const uint16_t* norm_gain, float rms_eps, int32_t* ids, float* top1,
                            float* gap, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
/* The same with a repetition penalty (the Jetson page's generate call, Part 1
 * section 1.4, passes repetition_penalty=1.1 beside greedy selection; the pages
 * give no formula, and this is the plain one): row m's logit z of a vocabulary
 * id whose bit is set in bitmap m / rep_rows is ranked as z / rep_penalty when
 * z > 0 and z * rep_penalty otherwise; top1 and gap are the penalised values.
 * rep_bits uint32 [ceil(M / rep_rows)][rep_words] (id v is bit v % 32 of word
 * v / 32), or NULL for none.  LA_ERR_ARG when rep_bits is given with rep_rows
 * < 1, rep_words * 32 < lm->n, or rep_penalty not positive and finite. */
la_status la_lm_head_argmax_penalized(const float* h, int32_t M, const la_weight* lm,
                                      const uint16_t* norm_gain, float rms_eps,
                                      const uint32_t* rep_bits, int32_t rep_words,
                                      int32_t rep_rows, float rep_penalty, int32_t* ids,
                                      float* top1, float* gap, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* One decoder layer for the window rows (RMSNorm, QKV + bias, RoPE at positions
 * P_b + j, bf16 K/V written to the cache at slots P_b + j, window attention, O
 * projection + residual, RMSNorm, SiLU-gated MLP + residual).  x, y fp32
 * [B*W][hidden] (y may alias x); attn_out (nullable) fp32 [B*W][n_heads*head_dim]
 * receives the attention output. */
la_status la_pbd_layer(const la_model* m, int32_t layer, const la_kv_cache* kv, const float* x,
                       const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len, float* y,
                       float* attn_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* The whole PBD window step ("LocateAnything-3B for RK3588 (RKLLM + RKNN)", "How
 * it differs from the original", item 1: each step sends the last accepted token
 * and the mask tokens over the reused prefix, at their original positions, and
 * reads one prediction per window position; "LocateAnything-3B on Jetson Orin
 * Nano", Part 1 sections 1.2-1.4: a Qwen2 decoder, the block mask, greedy
 * selection): embedding gather of window_ids int32 [B][W]; all
 * layers (writing each window's K/V into the cache at slots P_b .. P_b+W-1);
 * final RMSNorm; tied lm_head argmax.  out_ids int32 [B][W]; out_gap (nullable)
 * fp32 [B][W] top-2 logit gaps; out_hidden (nullable) fp32 [B*W][hidden] final
 * hidden state before the final norm.  prefix_len is not modified: the caller
 * commits accepted tokens by advancing it (nothing to roll back otherwise; the
 * next step overwrites the slots).  Rows of a sequence with a data error get
 * out_ids = -1 and set bits in *err (nullable; OR-ed, never cleared). */
/* Workspace of la_pbd_step (and la_pbd_step_refeed / la_pbd_step_opts / la_pbd_layer)
 * for B sequences of W window rows and keys up to max_len: the residual stream,
 * packed operands, attention partials and lm_head partials of the step above;
 * 0 for an invalid model or shape. */
size_t la_pbd_step_workspace(const la_model* m, int32_t B, int32_t W, int32_t max_len);
la_status la_pbd_step(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                      const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len,
                      int32_t* out_ids, float* out_gap, float* out_hidden, void* workspace,
                      size_t workspace_bytes, int32_t* err, hipStream_t stream);
/* la_pbd_step without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The step's scratch is a fixed array inside this
 * library: 64 MiB on each GPU the library runs on, held until the process
 * ends (its device address is resolved once per device, on the first call
 * made with that device current; the calling thread's current device must be
 * the stream's).  The call allocates and frees nothing.  Shapes whose
 * la_pbd_step_workspace() exceeds 64 MiB return LA_ERR_WORKSPACE (e.g. batch 1
 * up to a 32K-token context, or 16 sequences of 11 rows up to max_len 4102,
 * fit).  Every call on one GPU uses the same array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that may overlap on one
 * GPU (two streams, two threads) race and must be serialised by the caller.
 * Otherwise exactly la_pbd_step: the same arguments, results and errors. */
la_status la_pbd_step_noalloc(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                              const int32_t* prefix_len, int32_t B, int32_t W, int32_t max_len,
                              int32_t* out_ids, float* out_gap, float* out_hidden, int32_t* err,
                              hipStream_t stream);

/* Sampled selection in place of the greedy argmax (the RK3588 page, "LocateAnything-3B
 * for RK3588 (RKLLM + RKNN)", sections "Usage (on the board)" and "Evaluation",
 * runs the model with temperature 0.7, top-p 0.9 and repetition penalty 1.1; the
 * Jetson page, Part 1 section 1.4, notes that a temperature that is not positive
 * means greedy selection).  Per row of logits z (after the repetition penalty,
 * when one is given): p_v ~ exp(z_v / temperature); the nucleus is the shortest
 * run of the vocabulary ordered by z descending (equal logits: lower id first)
 * whose probability reaches top_p; a uniform draw u in [0, 1) selects, among the
 * kept ids in ascending id order, the first whose running kept probability
 * exceeds u times the kept total.  u is the top 24 bits of the first output word
 * of Philox4x32-10 at counter (row, offset mod 2^32, offset / 2^32, 0) and key
 * (seed mod 2^32, seed / 2^32), times 2^-24; row is the call's row index (b * W
 * + j for a step).  Probabilities are summed as 40-bit fixed point, exactly, so
 * the result is deterministic.  temperature <= 0 selects the argmax (lowest id
 * on a tie).  top_p must lie in (0, 1]. */
typedef struct {
  float temperature;
  float top_p;
  uint64_t seed;
  uint64_t offset;      /* the draw counter of this call */
  uint64_t* offset_dev; /* nullable device word: when given, its value is used instead
                           of `offset` and the call adds 1 to it afterwards (for a
                           loop replayed from one captured graph) */
  float* logits;        /* la_pbd_step_opts only: device fp32 [B*W][vocab] scratch,
                           caller-owned, 16-byte aligned; holds the step's logits
                           (before the penalty) when the call has run */
} la_sampling;

/* Sampled selection from given logits: ids int32 [M] for logits fp32 [M][ld]
 * (the first V of each row), with the repetition penalty of
 * la_lm_head_argmax_penalized when rep_bits is given (bitmap m / rep_rows for
 * row m).  sel_gap (nullable) fp32 [M] receives the selected logit minus the
 * row's largest (after the penalty).  LA_ERR_ARG for NULL logits, ids or s,
 * top_p outside (0, 1], a temperature that is not finite, or a bad penalty;
 * LA_ERR_SHAPE outside 1 <= M <= 65535, 1 <= V <= ld. */
la_status la_sample_logits(const float* logits, int32_t M, int32_t V, int32_t ld,
                           const uint32_t* rep_bits, int32_t rep_words, int32_t rep_rows,
                           float rep_penalty, const la_sampling* s, int32_t* ids, float* sel_gap,
                           hipStream_t stream);

/* Options of la_pbd_step_opts (zero-initialise, then set what is used):
 *  - causal_rows, window_len: int32 [B] device arrays of a re-fed window
 *    (la_pbd_step_refeed), or NULL;
 *  - rep_bits: uint32 [B][rep_words] device bitmaps of the vocabulary ids
 *    already in each sequence (id v is bit v % 32 of word v / 32), or NULL;
 *    every window row of sequence b ranks its logits with those ids'
 *    penalised by rep_penalty as in la_lm_head_argmax_penalized;
 *    rep_words * 32 >= the lm_head's vocabulary, rep_penalty positive and
 *    finite (else LA_ERR_ARG);
 *  - sampling: NULL for greedy selection; else the sampled selection above
 *    over the step's logits (with the repetition bitmaps when given).  Then
 *    out_gap (nullable) receives each row's selected logit minus its largest
 *    instead of the top-2 gap.  LA_ERR_ARG when sampling->logits is NULL or
 *    misaligned, or the parameters are out of range;
 *  - block_events: NULL, or 2 * n_layers events (created by the caller) for
 *    timing: block_events[2 l] is recorded on the stream before layer l's
 *    attention block (input RMSNorm, QKV, attention, O projection) and
 *    block_events[2 l + 1] after the launch that ends it (with bf16 tiled
 *    weights at up to 8 rows that one launch also runs the gate/up and down
 *    projections, the whole layer, unless LA_PBD_FRONT_GU=0 or
 *    LA_PBD_FRONT_DOWN=0 in the environment stops it earlier). */
typedef struct {
  const int32_t* causal_rows;
  const int32_t* window_len;
  const uint32_t* rep_bits;
  int32_t rep_words;
  float rep_penalty;
  const la_sampling* sampling;
  const hipEvent_t* block_events;
} la_step_opts;
la_status la_pbd_step_opts(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                           const int32_t* prefix_len, const la_step_opts* opts, int32_t B, int32_t W,
                           int32_t max_len, int32_t* out_ids, float* out_gap, float* out_hidden,
                           void* workspace, size_t workspace_bytes, int32_t* err,
                           hipStream_t stream);

/* Prefill of a prompt of L positions per sequence after its cached prefix of
 * P_b (the fixed cost before decoding in the Jetson page's latency breakdown,
 * section 3.1).  ids int32 [B][L]: a token id, or a negative id for a row
 * that takes its input from embeds fp32 [B][L][hidden] (the vision encoder's
 * features spliced in over the image-token positions, as the WebGPU page's
 * language graph takes them: "LocateAnything-3B — ONNX WebGPU (INT4 + 4-bit
 * embeddings)", sections "Why this repo exists" and "Embedding gather /
 * dequant (JS reference)"); embeds may be NULL when every id is a token.  Every
 * row attends causally to the prefix and the prompt rows up to its own (a
 * plain causal pass), and its K/V go to slots P_b .. P_b+L-1 of every layer.
 * out_ids int32 [B] = the argmax of each sequence's last prompt row (the first
 * generated token); out_gap fp32 [B] and out_hidden fp32 [B][hidden] (its
 * final hidden state before the final norm) are nullable.  prefix_len is not
 * modified.  Rows are processed in windows of 16: max_len >= P_b +
 * ceil(L/16)*16 and the cache must hold that many slots (the slots past L are
 * written and lie past the prompt).  B*ceil(L/16)*16 <= 8192, B <= 64.  Data
 * errors as la_pbd_step (out_ids -1 and bits in *err); a negative id with
 * embeds NULL is LA_DERR_TOKEN_ID. */
size_t la_pbd_prefill_workspace(const la_model* m, int32_t B, int32_t L, int32_t max_len);
la_status la_pbd_prefill(const la_model* m, const la_kv_cache* kv, const int32_t* ids,
                         const float* embeds, const int32_t* prefix_len, int32_t B, int32_t L,
                         int32_t max_len, int32_t* out_ids, float* out_gap, float* out_hidden,
                         void* workspace, size_t workspace_bytes, int32_t* err,
                         hipStream_t stream);

/* Mark tokens in the repetition bitmaps (uint32 [B][words], device): for
 * each sequence b, ids[b][j] for first[b] <= j < first[b] + count[b] (first
 * NULL: 0; count NULL: W) gets its bit set; ids outside [0, vocab) are
 * skipped.  ids int32 [B][W].  For a decode loop: mark the tokens it accepts.
 * Only enqueues (graph-capturable).  LA_ERR_ARG for NULL ids or bits,
 * LA_ERR_SHAPE outside 1 <= B <= 64, 1 <= W <= 16, words * 32 >= vocab >= 1. */
la_status la_pbd_mark_tokens(const int32_t* ids, int32_t B, int32_t W, const int32_t* first,
                             const int32_t* count, uint32_t* bits, int32_t words, int32_t vocab,
                             hipStream_t stream);

/* The step on a re-fed window (la_pbd_attention_refeed): causal_rows and
 * window_len are int32 [B] device arrays; either may be NULL (then 0 re-fed
 * rows, or m->window_mask decides; W real rows).  Every row, padding
 * included, is computed and writes its K/V at slot P_b + j, so P_b + W must
 * fit the cache; padding rows' slots lie past the window and are rewritten
 * before any later prefix covers them.  A sequence whose w_b is outside 1..W
 * or whose c_b is outside 0..w_b sets LA_DERR_WINDOW and gets out_ids = -1.
 * Workspace as la_pbd_step_workspace. */
la_status la_pbd_step_refeed(const la_model* m, const la_kv_cache* kv, const int32_t* window_ids,
                             const int32_t* prefix_len, const int32_t* causal_rows,
                             const int32_t* window_len, int32_t B, int32_t W, int32_t max_len,
                             int32_t* out_ids, float* out_gap, float* out_hidden, void* workspace,
                             size_t workspace_bytes, int32_t* err, hipStream_t stream);

/* Commit a fully accepted window and form the next one without re-feeding:
 * prefix_len[b] += W, and window_ids[b] becomes [out_ids[b][W-1], mask_id
 * x (W-1)].  The K/V that stay in the cache at slots P_b .. P_b+W-1 are the
 * ones la_pbd_step wrote: those of the window's own inputs.  With W = 1 (plain
 * token-by-token decoding, the slow mode) that input is the accepted token, so
 * the cache is exact.  With W > 1 slots P_b+1 .. P_b+W-1 keep the mask tokens'
 * K/V instead of the accepted tokens': a cheaper approximation of the method
 * that serves as a throughput proxy.  The method's loop re-feeds the accepted
 * tokens so that their K/V enter the cache: la_pbd_step_refeed with
 * la_pbd_commit_refeed below.  out_ids and window_ids int32 [B][W] (distinct
 * buffers), prefix_len int32 [B], all device memory owned by the caller.  Only
 * enqueues on the stream (graph-capturable).  Returns LA_ERR_ARG for NULL
 * pointers or aliased ids, LA_ERR_SHAPE outside 1 <= B <= 64, 1 <= W <= 16 (the
 * step's limits). */
la_status la_pbd_commit(const int32_t* out_ids, int32_t* window_ids, int32_t* prefix_len,
                        int32_t B, int32_t W, int32_t mask_id, hipStream_t stream);

/* Commit of a re-fed window step, with partial acceptance (same page and item:
 * the accepted tokens are sent again with the mask tokens, over the reused
 * prefix).  Window row i of sequence b sits at position P_b + i and its argmax
 * is read as the token at P_b + i + 1, so the block (rows c_b .. w_b - 1)
 * predicts the tokens after position P_b + c_b.  Sequence b accepts the first
 * n_b of them: n_accept[b] clamped to 1 .. w_b - c_b and to W - block + 1
 * (n_accept NULL: the whole block).  Rows up to the block's first are then
 * final, and the state becomes, in place:
 *   window_ids[b] = [out_ids[b][c_b] .. out_ids[b][c_b + n_b - 1], mask_id ...]
 *   prefix_len[b] += c_b + 1;  causal_rows[b] = n_b - 1;  window_len[b] = n_b + block - 1
 * i.e. the accepted tokens are re-fed causally and the last of them opens a
 * new block of `block` rows (it and block - 1 mask tokens).  The K/V of the
 * final rows are already in the cache (la_pbd_step_refeed wrote them).  All
 * arrays are int32 device memory: out_ids, window_ids [B][W]; n_accept,
 * prefix_len, causal_rows, window_len [B]; out_ids and n_accept must not alias
 * the state arrays.  Stored c_b, w_b are clamped (c_b to 0 .. W - 1, w_b to
 * c_b + 1 .. W) before use.  Only enqueues (graph-capturable).  Returns
 * LA_ERR_ARG for NULL or aliased pointers, LA_ERR_SHAPE outside 1 <= B <= 64,
 * 1 <= W <= 16, 1 <= block <= W. */
la_status la_pbd_commit_refeed(const int32_t* out_ids, const int32_t* n_accept, int32_t* window_ids,
                               int32_t* prefix_len, int32_t* causal_rows, int32_t* window_len,
                               int32_t B, int32_t W, int32_t block, int32_t mask_id,
                               hipStream_t stream);

/* Repack a row-major weight (src->layout == LA_LAYOUT_ROWS) into one of the
 * tiled layouts (bf16, or INT4 with group 128).  dst receives
 * la_pack_weight_bytes(src, layout, 0) bytes of data and dst_scales (INT4
 * only) la_pack_weight_bytes(src, layout, 1) bytes of scales; the caller then
 * describes the copy with the same fmt/n/k/group and the new layout.  The values
 * are copied bit for bit. */
size_t la_pack_weight_bytes(const la_weight* src, int32_t layout, int32_t scales);
la_status la_pack_weight(const la_weight* src, int32_t layout, void* dst, void* dst_scales,
                         hipStream_t stream);

/* Static text for a status code. */
const char* la_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* LA_PBD_H */
