// Internal launch interface shared by the kernels' translation units and the
// C ABI layer.  Everything here is host code plus argument structs.
#pragma once

#include "la_common.hpp"

namespace la {

enum GemmEpi { EPI_STORE = 0, EPI_SILU = 1, EPI_QKV = 2, EPI_ARGMAX = 3 };

// Arguments of one small-M GEMM launch (rows m_base .. m_base+31 at most).
struct GemmArgs {
  const uint16_t* apack;     // packed activations of all M rows
  const float* asum;         // INT4: [MT][K/128][16] per-group sums of the packed rows;
                             // w8a8: the rows' scales [M]
  const void* w;             // weight data
  const uint16_t* wscale;    // INT4 scales (fp16); w8a8: per-channel fp32 scales
  uint32_t w_bytes;          // size of the weight data (buffer range)
  uint32_t s_bytes;          // size of the INT4 scales
  int layout;                // LA_LAYOUT_* of w
  int M;                     // total rows of the problem
  int m_base;                // first row handled by this launch (multiple of 32)
  int N, K;                  // weight rows / reduction length
  int n_tiles;               // column tiles (16 operand columns each)
  int ksplit;                // K slices per tile (> 1: partial sums go to `partial`);
                             // slice s covers units [units*s/ksplit, units*(s+1)/ksplit)
  int nw;                    // waves per workgroup (they split a work item's K range)
  float* partial;            // [ksplit][M][N] partial sums when ksplit > 1
  // epilogue
  const uint16_t* bias;      // bf16, indexed by weight row (nullable)
  const float* residual;     // fp32 [M][ldy] (nullable)
  float* y;                  // fp32 [M][ldy]
  int ldy;
  uint16_t* y_apack;         // SiLU: also pack the output rows here; STORE (ksplit 1):
                             // pack y * out_gain for the next bf16 GEMM (nullable)
  const uint16_t* out_gain;  // STORE: RMSNorm gain of the next consumer (with y_apack)
  float* ss_out;             // STORE (ksplit 1): [M][n_tiles] sums of squares of y per tile
  // consumers of an RMSNorm'd operand whose 1/rms is not applied yet: outputs
  // are scaled by 1/sqrt(sum(ss_in[m][*]) / K + eps) (nullable)
  const float* ss_in;
  int ss_tiles;
  float eps;
  // QKV epilogue
  const float2* rope;        // [M][64] (cos, sin) of the row's position
  const int32_t* prefix_len; // [B]
  const int32_t* flags;      // [M] nonzero: row must not write the cache (nullable)
  int W, n_heads, n_kv_heads;
  const int32_t* block_table;
  int max_blocks, num_blocks;
  uint16_t* kc;              // layer base of the K pages
  uint16_t* vc;              // layer base of the V pages
  // ARGMAX epilogue
  float* amax;               // [M][n_parts][3] (top1, index bits, top2), one part per workgroup
  int n_parts;
  // repetition penalty of the ARGMAX epilogue (rep_bits nullable): row m ranks
  // its logits with those of the tokens set in bitmap m / rep_rows penalised
  const uint32_t* rep_bits;  // [M / rep_rows][rep_words] vocabulary bitmaps
  int rep_words, rep_rows;
  float rep_theta;
};

// Row packing: v = x[m] + sum_s parts[s][m] (fixed order), optionally stored to
// h_out, then RMSNorm'd (when gain != NULL) and packed into the operand layout.
struct PackArgs {
  const float* x;
  int ldx;
  int M, K;
  const uint16_t* gain;  // nullable: no RMSNorm
  float eps;
  uint16_t* apack;       // nullable: no packing
  float* asum;           // INT4: group sums; w8a8: the rows' scales (nullable otherwise)
  bool int4;
  bool w8;               // w8a8: int8 rows and per-row scales instead of bf16 hi/lo
  const float* parts;    // nullable: [n_parts][M][K] partial sums to add
  int n_parts;
  float* h_out;          // nullable: receives v (may alias x)
};

struct AttnArgs {
  const float* q;            // [B*W][Hq*D]
  const uint16_t* kc;        // layer base of the K pages
  const uint16_t* vc;        // layer base of the V pages
  const int32_t* block_table;
  const int32_t* prefix_len;
  int B, W, Hq, Hkv;
  int num_blocks, max_blocks;
  int cap;                   // key capacity bound (min(max_len, max_blocks*16))
  int pages_per_split;
  int max_splits;            // splits per (b, kv head)
  float* part_o;             // [B][Hkv][max_splits][NQP][D]
  float* part_ml;            // [B][Hkv][max_splits][NQP][2]
  float* out;                // fp32 [B*W][Hq*D] (nullable)
  uint16_t* out_apack;       // packed output for the next GEMM (nullable)
  bool out_int4;
  int nqp;                   // padded queries per kv head (multiple of 16)
  int causal;                // nonzero: window row j sees slots 0 .. P_b + j only
  const int32_t* causal_rows; // [B] re-fed rows (nullable; overrides `causal`)
  const int32_t* window_len;  // [B] real window rows (nullable: W)
  int bt_div;                 // windows per block-table row (a prefill's 16-row windows)
};

struct PrologueArgs {
  const int32_t* ids;        // [T] (nullable: no gather)
  int T;
  la_weight emb;
  float* out;                // fp32 [T][H]
  int32_t* err;              // nullable
  // step bookkeeping (all nullable)
  const int32_t* prefix_len; // [B]
  int W;
  float2* rope;              // [T][64]
  double rope_theta;
  int32_t* flags;            // [T]
  const int32_t* causal_rows; // [B] re-fed rows (nullable)
  const int32_t* window_len;  // [B] real window rows (nullable)
  const int32_t* block_table;
  int max_blocks, num_blocks, cap;
  int32_t* zero;             // nullable: n_zero words cleared (the front kernel's flags and words;
  int n_zero;                 // 16-byte aligned, n_zero a multiple of 4) by zero_blocks extra workgroups
  int zero_blocks;
  // prefill: ids / embeds hold in_w rows per sequence (rows j >= in_w of the
  // W are padding: zero input, no error); a negative id takes its row of
  // embeds ([B][in_w][H] fp32, nullable)
  int in_w;
  const float* embeds;
};

struct GemmPlan {
  int n_tiles;
  int ksplit;
  int nw;
  int mt;        // row tiles per launch (1, 2 or 4)
  int launches;  // ceil(M / 32)
  int grid;      // workgroups per launch
  int per;       // column tiles per workgroup (at most)
  int mode;      // kernel mode (single stage, 2-deep ring, LDS-staged ring)
  size_t smem;   // dynamic LDS bytes
};

// allow_split: the caller takes K-slice partial sums (EPI_STORE only)
GemmPlan plan_gemm(int M, int N, int K, bool int4, int epi, bool allow_split);
hipError_t launch_pack_weight(const la_weight& src, int layout, void* dst, void* dst_scales,
                              hipStream_t s);

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s);
hipError_t launch_commit(const int32_t* out_ids, int32_t* window_ids, int32_t* prefix_len, int B,
                         int W, int mask_id, hipStream_t s);
hipError_t launch_prefill_views(const int32_t* prefix_len, int B, int L, int chunks, int32_t* pp,
                                int32_t* pc, int32_t* pw, hipStream_t s);
hipError_t launch_mark_tokens(const int32_t* ids, int B, int W, const int32_t* first, const int32_t* count,
                              uint32_t* bits, int words, int vocab, hipStream_t s);
hipError_t launch_commit_refeed(const int32_t* out_ids, const int32_t* n_accept, int32_t* window_ids,
                                int32_t* prefix_len, int32_t* causal_rows, int32_t* window_len, int B,
                                int W, int block, int mask_id, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
// fmt: LA_W_BF16, LA_W_INT4 or LA_W_W8A8 (the weight's format; the operand was
// packed for it)
hipError_t launch_gemm(GemmArgs a, int epi, int fmt, hipStream_t s);
GemmPlan plan_gemm_w8(int M, int N, int K, int epi, bool allow_split);
hipError_t launch_argmax_reduce(const float* amax, int M, int n_tiles, const int32_t* flags,
                                int32_t* ids, float* top1, float* gap, int32_t* err,
                                hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// Large-M GEMMs (more than 32 rows): every weight fragment meets all rows of a
// launch (up to 192 bf16 / 64 INT4 rows) while it is in registers.  QKV goes
// through K-slice sums in `partial` and a finishing kernel.
struct BigPlan {
  int n_tiles;
  int lay;     // wave grid
  int rt;      // row tiles per row wave
  int ksplit;
  int grid, threads;
  size_t smem;
};
int big_rows_per_launch(bool int4);
bool use_big_gemm(int M, bool int4, int epi, bool tiled);
BigPlan plan_gemm_big(int rows, int N, int K, bool int4, int epi, bool allow_split);
hipError_t launch_gemm_big(GemmArgs a, int epi, bool int4, hipStream_t s);

// Sampled selection (temperature, top-p, Philox draw) from stored logits, one
// workgroup per row.
struct SampleArgs {
  const float* logits;         // [M][ldz]
  int M, V, ldz;
  const uint32_t* rep_bits;    // [M / rep_rows][rep_words] (nullable)
  int rep_words, rep_rows;
  float rep_theta;
  float temperature, top_p;    // temperature <= 0: argmax
  uint64_t seed, offset;
  const uint64_t* offset_dev;  // nullable: replaces offset and is advanced by 1 afterwards
  const int32_t* flags;        // [M] nullable: nonzero rows get id -1
  int32_t* ids;                // [M]
  float* sel_gap;              // [M] nullable: selected logit minus the row's largest
  int32_t* err;                // nullable
};
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);

// The front half of a layer (RMSNorm + pack, QKV, attention, O) for up to 8
// window rows with bf16 tiled weights and K = 2048, as one persistent launch
// (la_front.hip).
struct FrontArgs {
  AttnArgs at;                // the attention (q, kc, vc, partials, out_apack = the O operand)
  int T, H, HQ;               // window rows, hidden (QKV K, O N), heads x 128 (O K)
  float* h;                   // [T][H] residual stream, updated in place
  const float* parts;         // [n_parts][T][H] K-slice sums still to add (nullable)
  int n_parts;
  const uint16_t* in_norm;
  float eps;
  uint16_t* xpack;            // packed QKV operand (one row tile): (h + sums) * in_norm
  float* ss_part;             // [8][kFrontPackSlices] sums of squares of the rows per pack slice
  const void* wqkv;           // tiled QKV weight
  uint32_t wqkv_bytes;
  const uint16_t* qkv_bias;   // nullable
  const float2* rope;         // [T][64]
  const int32_t* flags;       // [T] nonzero: the row writes no K/V
  const void* wo;             // tiled O weight
  uint32_t wo_bytes;
  const uint16_t* post_norm;
  uint16_t* gpack;            // packed gate/up operand: h1 * post_norm
  float* ss;                  // [T][H / 16] per-tile sums of squares of h1
  // gate/up in the same launch (nullable wgu: the launch ends after O): the
  // tiled gate/up weight, F / 8 tiles of 8 gate and 8 up columns, the packed
  // down operand silu(gate) * up it writes (bf16 hi / lo, K = F)
  const void* wgu;
  uint32_t wgu_bytes;
  int n_gu_tiles, F;
  uint16_t* mpack;
  // the down projection in the same launch too (nullable wdn: a kernel of its
  // own): the tiled down weight (H / 16 tiles of F / 32 units), its output as
  // kFrontDownSlices K-slice sums [slice][T][H] that the next pack adds
  const void* wdn;
  uint32_t wdn_bytes;
  float* dparts;
  int n_qkv_tiles, n_o_tiles, n_items, runs;  // attention items = B * Hkv * runs
  int32_t* sync;              // flag words (the step's prologue zeroes them)
  // Data handed from a few producers to a few consumers inside the launch, as
  // 8-byte words {32-bit datum (low half), epoch (high half)} (the step's
  // prologue zeroes them):
  uint64_t* ll_q;             // [T][HQ] q after bias and RoPE (fp32 bits)
  uint64_t* ll_kv;            // [T][Hkv][2 (K, V)][64]: bf16 of dims i (low) and i + 64 (high)
  uint64_t* ll_ml;            // [units][2] per run and query column: max, sum
  uint64_t* ll_po;            // [units][128] per run and query column: unnormalised O
  int epoch;                  // the value this launch's flags and words take: layer index + 1
  int32_t* err;               // nullable
};
// Pages of one attention run of the front-half launch (the whole run sits in
// LDS), and the slices its operand packing splits K = 2048 into.
constexpr int kFrontMaxRunPages = 12;
constexpr int kFrontPackSlices = 64;
// K slices of the down projection when the front-half launch runs it: each
// workgroup takes two output tiles of one slice (grid = 2 x slices x ... =
// H / 16 x slices / 2 workgroups), at most kFrontDownUnits units of 32 k.
constexpr int kFrontDownSlices = 4;
constexpr int kFrontDownUnits = 88;
// Flag words of the front-half launch: pack [8 copies][64 slices], ready [8
// copies][128 items], O tiles done [8 copies][128 tiles], gate/up done [8
// copies][256 workgroups].
constexpr int kFrontSyncWords = 8 * 64 + 8 * 128 + 8 * 128 + 8 * 256;
hipError_t launch_front(const FrontArgs& f, int grid, hipStream_t s);
// Compute units of the current device (256 when the query fails).
int cu_count();

// attention split planning
void plan_attention(int B, int Hkv, int max_len, int* pages_per_split, int* max_splits);
inline int attn_nqp(int W, int G) { return ((W * G + 15) / 16) * 16; }

}  // namespace la
