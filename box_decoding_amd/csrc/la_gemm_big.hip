// Weight-streaming GEMMs for 33 .. 192 rows (batched PBD windows) on the gfx950
// matrix cores.
//
// At M = 6 x batch rows in the hundreds the contraction is dense enough for the
// matrix cores to set the pace: 192 rows in bf16 hi + lo halves are 384
// operand rows, so every weight fragment feeds a dozen 32x32x16 products.
//
// One workgroup is four waves, one per SIMD, so each wave may hold 512
// registers; the 32x32x16 product keeps a lone wave's matrix core near its
// peak (the 16x16x32 one does not).  Waves (rw, cw) form a 2 x 2 grid: rw takes
// half of the operand rows, cw half of a work item's 128 columns; an item is
// those 128 columns over one K slice.  Per K unit (32 columns of K for bf16,
// one 128-group for INT4) a stage
//   - waits for this wave's copies of the unit read next and meets the other
//     waves at one barrier, after which that unit is complete in LDS,
//   - runs the stage's products, and among them
//   - reads the next unit's activation fragments into registers (bf16),
//   - copies a later unit of the packed activations into a ring of NS LDS
//     slots with direct-to-LDS loads (each wave a quarter of it), into the
//     slot whose reads completed before the barrier,
//   - issues the weight loads of stage bi + DW into a register ring (raw
//     buffer loads; a masked stage reads zero).
// Loads complete in issue order, so a wave that waits for its copies has also
// received every weight issued before them.  An item's stages are padded to
// whole turns of the weight ring; its epilogue goes through a small LDS
// staging area 8 rows at a time.  INT4 weights keep the 16x16x32 product
// (its dequantisation runs between the steps) and the same item shape.
#include <algorithm>
#include <type_traits>

#include "la_gemm_common.hpp"

namespace la {

constexpr int kPfSink = 1024;  // LDS bytes the L2 prefetches land in (never read)

// Wave grids (LAY): 0: 2 row waves x 2 column waves (bf16 2 tiles of 32
// columns each, INT4 4 tiles of 16: items of 128 columns); 1 (bf16): 4 row
// waves x 1 column wave of 3 tiles of 32 (items of 96 columns, so more
// workgroups for a GEMM that cannot take K slices); 2: 4 x 2, eight waves
// (two per SIMD, so one wave's other instructions run beside another's
// products); 3 (INT4): 4 x 2 with 3 tiles of 16 columns per column wave
// (items of 96 columns: more workgroups for the gate/up projection); 4
// (INT4, up to 48 rows): 2 row waves of 3 row tiles x 2 column waves of 3
// tiles, four waves (the launch's rows fill the row tiles exactly, and each
// expanded weight fragment feeds three products).
constexpr int lay_row_waves(int lay) { return lay == 0 || lay == 4 ? 2 : 4; }
constexpr int lay_col_waves(int lay) { return lay == 1 ? 1 : 2; }
constexpr int lay_threads(int lay) { return lay_row_waves(lay) * lay_col_waves(lay) * 64; }
constexpr int lay_waves_per_eu(int lay) { return lay == 2 || lay == 3 ? 2 : 1; }

template <int RT, bool INT4, int LAY = 0>
struct Wide {
  // bf16: RT tiles of 32 operand rows (16 real rows) per row wave, CT tiles
  // of 32 columns per column wave.  INT4: RT tiles of 16 operand rows (8 real
  // rows), CT = 4 tiles of 16 columns.
  static constexpr int RWV = lay_row_waves(LAY), CW = lay_col_waves(LAY), WAVES = RWV * CW;
  static constexpr int RTW = RWV * RT * (INT4 ? 1 : 2);  // packed 16-row tiles of a launch
  static constexpr int NP = INT4 ? RT : 2 * RT;       // epilogue parts of 8 real rows per row wave
  static constexpr int CT = INT4 ? (LAY >= 3 ? 3 : 4) : (LAY == 1 ? 3 : 2);
  static constexpr int TPW = INT4 ? CT : 2 * CT;      // 16-column tiles per column wave
  static constexpr int ITEM = CW * TPW;               // 16-column tiles per work item
  static constexpr int SW = TPW * 16;                 // staged columns per wave
  static constexpr int NG = SW / 8;                   // 8-column epilogue groups per staged row
  static constexpr int CPU = INT4 ? 16 : 4;           // 256-byte chunks per packed tile and K unit
  static constexpr int FR = INT4 ? RT : 2 * RT;       // fragments per bf16 stage / INT4 K step
  // staged rows of an epilogue part: the INT4 exact-fit grid stages the hi
  // and the lo operand rows apart and adds them when it reads (no cross-lane
  // exchange); the eight-wave INT4 grids have no LDS left for that
  static constexpr bool SPLIT_HL = INT4 && LAY == 4;
  static constexpr int SROWS = SPLIT_HL ? 16 : 8;
  static constexpr int SUMP = (RTW + 3) / 4;           // INT4 group-sum pieces of 256 B (4 row tiles each)
  static constexpr int SUMS = INT4 ? SUMP * 256 : 0;  // INT4 group sums of a slot (bytes)
  // INT4 scales of the stage's item tiles (16 fp16 per tile), copied into the
  // slot beside the sums: carried in registers through the weight ring they
  // made the compiler wait for nearly every load at each turn of the ring
  static constexpr int SCB = INT4 ? 256 : 0;
  static constexpr int SLOT = RTW * CPU * 256 + SUMS + SCB;
  static constexpr int NS = INT4 ? 4 : 6;             // LDS slots
  // bf16 reads the next stage's fragments during a stage (registers for two
  // stages); INT4 reads its own stage's, one K step ahead
  static constexpr bool PREFETCH = !INT4;
  static constexpr int LA = NS - 1;                   // copy lead (stages)
  // weight ring entries (and loop unroll): INT4 stages are short at 48-64 rows,
  // so the gate/up layout keeps 3 stages ahead; the lm_head's layout (more
  // accumulators) has registers for 2
  static constexpr int R = INT4 && LAY != 3 ? 3 : 4;
  static constexpr int DW = R - 1;                    // weight lead (stages)
  static constexpr int NCOPY = RTW * CPU / 4 / WAVES;  // 1 KB copies per wave and stage
  static constexpr int NC = NCOPY + (INT4 ? 2 : 0);  // INT4: + group sums + scales
  static constexpr int NW = INT4 ? CT : 2 * CT;       // bf16: CT tiles x 2 K steps
  // Optional L2 prefetch: the weights of stage s + PF pulled into L2 at stage
  // s (direct-to-LDS loads into a scratch kilobyte nobody reads).  Measured
  // slower at PF 8..16 (the loop is not waiting on weights: with every
  // workgroup reading the same L2-resident weights it runs no faster), so off.
  // INT4 (the row waves of a column wave split the stage's tiles) measured
  // slower too: gate/up at 48 rows with the exact-fit grid 29.6 against 25.6
  // us at PF 8.
  static constexpr int PF = 0;
  static constexpr int NPF = PF > DW ? (INT4 ? (CT + RWV - 1) / RWV : CT) : 0;  // prefetch loads per wave and stage
  // A wave waits for its own copies of the unit read next before the barrier
  // (loads complete in issue order).  The wait counts come from a replay of
  // the issue order: the prologue (L2 prefetches, DW stages of weights,
  // CLEAD stages of copies), then per stage one copy batch, one weight batch
  // and one prefetch batch.  At each
  // stage's wait it counts the loads issued after the last copy of the unit
  // read next; the smallest count over the first stages (after which the
  // pattern repeats) is the wait of every stage, and the prologue's own
  // count is the wait before the first fragment reads.
  static constexpr int CLEAD = PREFETCH ? LA + 1 : LA;  // copies of stage s + CLEAD at stage s
  struct Waits {
    int first, loop;
  };
  static constexpr Waits waits() {
    int endc[64] = {};
    int e = 0, cp = 0;
    for (int s = -DW; s < 0; ++s) {
      e += NC;  // a copy (of stage 0's bytes when no real copy is due yet)
      if (s + CLEAD >= 0) endc[cp++] = e;
      e += NW;
    }
    for (int s = DW; s < CLEAD; ++s) {
      e += NC;
      endc[cp++] = e;
    }
    Waits r{PREFETCH ? e - endc[0] : 0, 1 << 20};
    for (int j = 0; j < 2 * NS + 2 * R; ++j) {
      const int after = e - endc[PREFETCH ? j + 1 : j];
      r.loop = after < r.loop ? after : r.loop;
      e += NC;
      endc[cp++] = e;
      e += NW + NPF;
    }
    return r;
  }
  static constexpr int WAIT = waits().loop;
  static constexpr int WAIT0 = waits().first;
  static_assert((RTW % 4 == 0 || (INT4 && RTW % 2 == 0)) && (R % 2 == 0 || !PREFETCH) && DW >= 1,
                "wide GEMM shape");
  static_assert((RTW * CPU / 4) % WAVES == 0 && (!INT4 || LAY != 1), "wide GEMM shape");
  static_assert(WAIT >= 0 && WAIT0 >= 0 && WAIT < 64 && WAIT0 < 64, "vmcnt range");
  static_assert(NG <= 16 && SW % 8 == 0, "item shape");
  static_assert(!INT4 || ITEM * 8 <= 64, "one lane per scale dword of an item");
};

// The per-stage meeting point: this wave's LDS reads are complete, then the
// hardware barrier.  Unlike __syncthreads it does not wait for the copies in
// flight (each wave waits for exactly its own before arriving).
__device__ __forceinline__ void stage_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

// D[32x32] += A[32x16] . B[16x32]: lane l holds A row l%32 and B column l%32
// with k = 8*(l/32) .. +7; D lane l holds column l%32, rows 8*(q/4) + 4*(l/32)
// + q%4 for q = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>)
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <int RT, bool INT4, int EPI, int LAY>
__global__ __launch_bounds__(lay_threads(LAY))
__attribute__((amdgpu_waves_per_eu(lay_waves_per_eu(LAY), lay_waves_per_eu(LAY))))
void k_gemm_big(GemmArgs a) {
  using C = Wide<RT, INT4, LAY>;
  constexpr int RTW = C::RTW, NP = C::NP, CT = C::CT, CPU = C::CPU, FR = C::FR, NS = C::NS,
                LA = C::LA, DW = C::DW, SLOT = C::SLOT, WAVES = C::WAVES, CW = C::CW,
                TPW = C::TPW, ITEM = C::ITEM;
  using AccT = std::conditional_t<INT4, f32x4, f32x16>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rw = wave / CW, cw = wave % CW;
  const int g = lane >> 4, c = lane & 15;
  const int K8 = a.K >> 3, KG = a.K >> 7;
  const int units = INT4 ? (a.K >> 7) : (a.K >> 5);
  const int ks = (int)blockIdx.x % a.ksplit;
  const int cb0 = (int)blockIdx.x / a.ksplit, gt = (int)gridDim.x / a.ksplit;
  const int s_lo = units * ks / a.ksplit, s_hi = units * (ks + 1) / a.ksplit;
  const int nu = s_hi - s_lo;
  const int nup = (nu + C::R - 1) / C::R * C::R;  // stages per item: whole ring turns
  const int n_cb = (a.n_tiles + ITEM - 1) / ITEM;
  const int n_my = cb0 < n_cb ? (n_cb - cb0 + gt - 1) / gt : 0;
  const int total = n_my * nup;
  const int rows = min(a.M - a.m_base, RTW * 8);
  const int mtv = (rows + 7) >> 3;

  constexpr int SW = C::SW;      // columns of a column wave
  constexpr int SROW = SW + 4;  // 16-byte aligned rows, column writes spread over banks
  constexpr int SR = C::SROWS;  // staged rows per wave (INT4: the hi rows, then the lo rows)
  unsigned char* slots = smem;                                              // [NS][SLOT]
  unsigned char* pf_sink = smem + NS * SLOT;                                // [kPfSink]
  float* stage = (float*)(pf_sink + kPfSink) + (size_t)wave * SR * SROW;    // [SR][SROW] per wave
  float* amax_lds = (float*)(pf_sink + kPfSink) + (size_t)WAVES * SR * SROW;
  float* my_amax = amax_lds + (size_t)wave * NP * 8 * 3;                    // ARGMAX: [NP*8][3]
  if (EPI == EPI_ARGMAX) {
    for (int i = lane; i < NP * 8; i += 64) {
      my_amax[i * 3 + 0] = -INFINITY;
      my_amax[i * 3 + 1] = __int_as_float(0x7FFFFFFF);
      my_amax[i * 3 + 2] = -INFINITY;
    }
  }

  // A stream walks the stages in order: item `it`, stage `uu` of the item's
  // nup, LDS slot.  Stepping is scalar and branch-free.  Past the last item
  // a stream keeps producing valid (unused) stages.
  struct Pos {
    int it, uu, slot;
  };
  auto step = [&](Pos& q) {
    const bool wrap = q.uu + 1 == nup;
    q.uu = wrap ? 0 : q.uu + 1;
    q.it += wrap ? 1 : 0;
    q.slot = q.slot + 1 == NS ? 0 : q.slot + 1;
  };
  auto slot_ptr = [&](int slot) { return slots + slot * SLOT; };

  // ---- activation copies: 1 KB pieces wave, wave + 4, ... of the unit
  const __amdgpu_buffer_rsrc_t rap =
      make_rsrc(a.apack + (size_t)(a.m_base >> 3) * K8 * 128, (uint32_t)mtv * K8 * 256);
  const __amdgpu_buffer_rsrc_t ras =
      make_rsrc(INT4 ? (const void*)(a.asum + (size_t)(a.m_base >> 3) * KG * 16) : a.apack,
                INT4 ? (uint32_t)mtv * KG * 64 : 0u);
  // INT4 group sums: RTW packed tiles x 16 floats in SUMP pieces of 256 B (a
  // last piece's tiles past RTW repeat the last tile into the slot's padding);
  // waves beyond the piece count repeat the first ones (same bytes, same place)
  static_assert(!INT4 || C::SUMP <= 4, "sum pieces");
  const int sum_q = INT4 ? wave % C::SUMP : 0;
  const uint32_t sum_voff =
      INT4 ? ((uint32_t)min(min(sum_q * 4 + (lane >> 4), RTW - 1), mtv - 1) * KG * 16 + (lane & 15)) * 4 : 0u;
  // INT4 scale copy: lane l < 8 ITEM takes dword l % 8 of item tile l / 8
  // (tiled scales: [tile][unit][16] fp16); the other lanes read past the end
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(INT4 ? (const void*)a.wscale : a.w, INT4 ? a.s_bytes : 0u);
  const uint32_t sc_voff = lane < 8 * ITEM ? (uint32_t)(lane >> 3) * (uint32_t)units * 32 + (lane & 7) * 4 : 0x40000000u;
  auto copy_stage = [&](const Pos& q) {
    const uint32_t u = (uint32_t)(s_lo + min(q.uu, nu - 1));
    unsigned char* dst = slot_ptr(q.slot);
#pragma unroll
    for (int k = 0; k < C::NCOPY; ++k) {
      const int p = wave + WAVES * k;
      const int t = p / (CPU / 4), part = p % (CPU / 4);
      const uint32_t soff = ((uint32_t)min(t, mtv - 1) * K8 + u * CPU + part * 4) * 256;
      lds_copy16(rap, lane * 16, soff, dst + (t * CPU + part * 4) * 256);
    }
    if (INT4) {
      lds_copy4(ras, sum_voff, u * 64, dst + RTW * CPU * 256 + sum_q * 256);
      // the item's tile scales for unit u (tiles past the weight read zero);
      // a stage whose weights are dead (ring padding, past the last item)
      // gets zero scales too, so its group correction adds nothing
      const bool live_stage = q.it < n_my && q.uu < nu;
      const uint32_t item_tile = (uint32_t)(cb0 + q.it * gt) * ITEM;
      const uint32_t so = live_stage ? (item_tile * (uint32_t)units + u) * 32 : 0x7FFFFFFFu;
      lds_copy4(rsc, sc_voff, so, dst + RTW * CPU * 256 + C::SUMS);
    }
  };

  // ---- weights of the column wave's 16-column tiles tile0 .. tile0 + 3.  A
  // lane's offset is a fixed part (which operand column and K slice it holds)
  // plus a wave-uniform part (tile and unit), so a load needs no vector
  // arithmetic.  bf16 (32x32x16): lane l holds column l%32 of a 32-column
  // tile (16-column tile 2T + (l/16)%2, column l%16) and K values
  // 16*kk + 8*(l/32) .. +7 of the unit; in the 16-column tile's layout those
  // are lane (2*kk + l/32)*16 + l%16's bytes.
  const __amdgpu_buffer_rsrc_t rwt = make_rsrc(a.w, a.w_bytes);
  const bool tiled = a.layout != LA_LAYOUT_ROWS;
  const int UT = units;
  // row layout: weight row of operand column c of a tile = row_of_tile + row_of_lane
  const int row_of_lane = EPI == EPI_SILU ? (c < 8 ? c : a.N / 2 + c - 8)
                          : EPI == EPI_QKV ? (c < 8 ? c : 56 + c) : c;
  const int odd = (lane >> 4) & 1;  // bf16: second 16-column tile of the pair
  const int tile_rows = EPI == EPI_STORE || EPI == EPI_ARGMAX ? 16 : 8;  // row step of a 16-column tile
  uint32_t w_lane;
  if (INT4) {
    w_lane = tiled ? (uint32_t)lane * 16 : (uint32_t)row_of_lane * (a.K >> 1) + g * 16;
  } else {
    w_lane = tiled ? (uint32_t)((lane >> 5) * 16 + c) * 16 + (uint32_t)odd * UT * 1024
                   : ((uint32_t)(row_of_lane + odd * tile_rows) * a.K + (lane >> 5) * 8) * 2;
  }
  const uint32_t kk_step = tiled ? 512u : 32u;  // bf16: second K step of the unit
  const uint32_t ustride = tiled ? 1024u : 64u;
  auto tile_row = [&](int tile) {
    return EPI == EPI_SILU ? tile * 8 : EPI == EPI_QKV ? (tile >> 3) * 128 + (tile & 7) * 8 : tile * 16;
  };
  auto tile_w = [&](int tile) -> uint32_t {
    if (tiled) return (uint32_t)tile * UT * 1024;
    return INT4 ? (uint32_t)tile_row(tile) * (a.K >> 1) : (uint32_t)tile_row(tile) * a.K * 2;
  };
  struct WStage {
    u32x4 w[2 * CT / (INT4 ? 2 : 1)];  // bf16: [tile][K step]; INT4: [tile]
  };
  WStage st[C::R];
  auto issue_w = [&](const Pos& q, WStage& d) {
    const bool live_stage = q.it < n_my && q.uu < nu;
    const uint32_t u = (uint32_t)(s_lo + min(q.uu, nu - 1));
    const int tile0 = ((cb0 + q.it * gt) * CW + cw) * TPW;
    if (INT4) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const int tile = tile0 + t;
        const bool live = live_stage && tile < a.n_tiles;  // wave-uniform
        // a dead load starts past the end of the buffer and reads zero
        const uint32_t so = live ? tile_w(tile) + u * ustride : 0x7FFFFFFFu;
        d.w[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwt, w_lane, so, kNonTemporal));
      }
    } else {
#pragma unroll
      for (int T = 0; T < CT; ++T) {
        const int tile = tile0 + 2 * T;
        // both 16-column tiles of the pair live or dead together (n_tiles is
        // even for every bf16 weight with N % 32 == 0; the tail of an odd one
        // reads past its end, which is zero)
        const bool live = live_stage && tile < a.n_tiles;
        const uint32_t so = live ? tile_w(tile) + u * ustride : 0x7FFFFFFFu;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          d.w[T * 2 + kk] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwt, w_lane + kk * kk_step, so, kNonTemporal));
      }
    }
  };

  // L2 prefetch of a stage's bf16 weights: this wave takes loads rw*CT ..
  // rw*CT + CT - 1 (load T*2 + kk) of its column wave's stage
  auto issue_pf = [&](const Pos& q) {
    if constexpr (C::NPF > 0) {
      const bool live_stage = q.it < n_my && q.uu < nu;
      const uint32_t u = (uint32_t)(s_lo + min(q.uu, nu - 1));
      const int tile0 = ((cb0 + q.it * gt) * CW + cw) * TPW;
#pragma unroll
      for (int i = 0; i < C::NPF; ++i) {
        if (INT4) {
          // tiles rw, rw + RWV, ... of the column wave's CT
          const int t = rw + C::RWV * i;
          const int tile = tile0 + t;
          const bool live = live_stage && t < CT && tile < a.n_tiles;
          const uint32_t so = live ? tile_w(tile) + u * ustride : 0x7FFFFFFFu;
          lds_copy16(rwt, w_lane, so, pf_sink);
        } else {
          const int idx = rw * CT + i, T = idx >> 1, kk = idx & 1;
          const int tile = tile0 + 2 * T;
          const bool live = live_stage && tile < a.n_tiles;
          const uint32_t so = live ? tile_w(tile) + u * ustride : 0x7FFFFFFFu;
          lds_copy16(rwt, w_lane + kk * kk_step, so, pf_sink);
        }
      }
    }
  };

  // ---- activation fragments.  bf16: fragment 2i + kk is row tile i (packed
  // tiles 2i, 2i + 1 of the wave's rows), K step kk; INT4: row tile i of K
  // step j.
  const uint32_t a_lane = INT4 ? (uint32_t)(rw * RT) * CPU * 256 + c * 16
                               : ((uint32_t)((2 * rw * RT + odd) * CPU + (lane >> 5)) * 16 + c) * 16;
  auto frag_base = [&](int slot) { return (const unsigned char*)(slot_ptr(slot) + a_lane); };
  auto read_frags = [&](const unsigned char* A, int j, bf16x8 (&d)[FR]) {
    if (INT4) {
#pragma unroll
      for (int i = 0; i < RT; ++i) d[i] = *(const bf16x8*)(A + (i * CPU + g * 4 + j) * 256);
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) d[2 * i + kk] = *(const bf16x8*)(A + (2 * i * CPU + 2 * kk) * 256);
    }
  };

  AccT acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[i][t] = AccT{};

  // bf16: the products of one stage from fragments read one stage earlier
  auto compute_bf16 = [&](const WStage& s, const bf16x8 (&f)[FR]) {
    if constexpr (!INT4) {
      // K step outermost: consecutive products go to different accumulators
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int T = 0; T < CT; ++T)
            acc[i][T] = mfma_32x32x16(f[2 * i + kk], __builtin_bit_cast(bf16x8, s.w[T * 2 + kk]), acc[i][T]);
    }
  };
  // INT4: one 128-group per stage, per group
  //   acc += scale * (sum_k a_k (128 + q_k) - 136 * sum_k a_k),
  // the fragments of step j + 1 read while step j multiplies
  const uint32_t i4bias = INT4 ? int4_bias_reg() : 0u;
  auto compute_int4 = [&](int slot, const WStage& s) {
    if constexpr (INT4) {
      const unsigned char* A = frag_base(slot);
      const float* AS = (const float*)(slot_ptr(slot) + RTW * CPU * 256) + (size_t)(rw * RT) * 16 + 4 * g;
      f32x4 sums[RT];
#pragma unroll
      for (int i = 0; i < RT; ++i) sums[i] = *(const f32x4*)(AS + i * 16);
      bf16x8 fa[2][FR];
      read_frags(A, 0, fa[0]);
      f32x4 tacc[RT][CT];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int t = 0; t < CT; ++t) tacc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < 3) read_frags(A, j + 1, fa[(j + 1) & 1]);
        bf16x8 bv[CT];
#pragma unroll
        for (int t = 0; t < CT; ++t) bv[t] = __builtin_bit_cast(bf16x8, int4_to_bf16x8(s.w[t][j], i4bias));
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int t = 0; t < CT; ++t) tacc[i][t] = mfma_16x16x32(fa[j & 1][i], bv[t], tacc[i][t]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const float sc = fp16_to_f32(*(const uint16_t*)(slot_ptr(slot) + RTW * CPU * 256 + C::SUMS +
                                                        ((cw * TPW + t) * 16 + c) * 2));
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][t][e] += sc * (tacc[i][t][e] - 136.0f * sums[i][e]);
      }
    }
  };

  // ---- epilogue of one column block, 8 real rows (a part) at a time: the
  // part's accumulators go through this wave's LDS staging rows (hi + lo
  // added), and one rolled loop does the per-element work, so its code exists
  // once.
  auto stage_part = [&](auto pc) {
    constexpr int P = decltype(pc)::value;
    if constexpr (C::SPLIT_HL) {
      // 16x16x32: lane l holds operand rows 4 (l / 16) + e: real row
      // 4 ((l / 16) % 2) + e, hi for l < 32 and lo beyond (staged 8 rows on)
#pragma unroll
      for (int t = 0; t < CT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) stage[(4 * g + e) * SROW + t * 16 + c] = acc[P][t][e];
        acc[P][t] = AccT{};
      }
    } else if constexpr (INT4) {
      // 16x16x32: lanes g < 2 hold real rows 4g + e after the xor-32 exchange
#pragma unroll
      for (int t = 0; t < CT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[P][t][e] + __shfl_xor(acc[P][t][e], 32);
          if (g < 2) stage[(4 * g + e) * SROW + t * 16 + c] = v;
        }
        acc[P][t] = AccT{};
      }
    } else {
      // 32x32x16: rows 8h + 4*(l/32) + e (hi) and 8h + 8 + ... (lo) of tile
      // P/2 sit in the same lane at q = 8*(P%2) + e and q + 4
      constexpr int i = P / 2, h = P % 2;
#pragma unroll
      for (int T = 0; T < CT; ++T) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          stage[((lane >> 5) * 4 + e) * SROW + T * 32 + (lane & 31)] = acc[i][T][8 * h + e] + acc[i][T][8 * h + e + 4];
        if (h == 1) acc[i][T] = AccT{};
      }
    }
  };
  // A staged value (split staging: the row's hi and lo halves, 8 staged rows
  // apart, added in that order)
  auto st4 = [&](const float* p) -> f32x4 {
    f32x4 v = *(const f32x4*)p;
    if constexpr (C::SPLIT_HL) v += *(const f32x4*)(p + 8 * SROW);
    return v;
  };
  auto st1 = [&](const float* p, int e) -> float { return C::SPLIT_HL ? p[e] + p[e + 8 * SROW] : p[e]; };
  // One lane per 8 consecutive staged columns of a row (r = lane / 8, column
  // group lane % 8, + 8 in a second pass when a wave stages 96 columns: the
  // group's 16-column tile is group / 2, its half group % 2), so the outputs
  // go out as 16-byte pieces.
  auto epi_part = [&](int cblock, int part) {
    const int tile0 = (cblock * CW + cw) * TPW;
    const int r = lane >> 3;
    const int ml = (rw * NP + part) * 8 + r;  // row within the launch
    const bool row_ok = ml < rows;
    const int m = a.m_base + ml;
    if (EPI == EPI_ARGMAX) {
      float v1 = -INFINITY, v2 = -INFINITY;
      int i1 = 0x7FFFFFFF;
#pragma unroll
      for (int gp = 0; gp < (C::NG + 7) / 8; ++gp) {
        const int grp = gp * 8 + (lane & 7);
        const int tile = tile0 + (grp >> 1), half = grp & 1;
        if (grp < C::NG && tile < a.n_tiles) {
          const float* src = stage + r * SROW + grp * 8;
          const f32x4 x0 = st4(src), x1 = st4(src + 4);
          const int n0 = tile * 16 + half * 8;
          // the group's 8 bits of this row's bitmap (repetition penalty)
          const uint32_t used = row_ok ? rep_word(a, m, n0) >> (n0 & 31) : 0u;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int n = n0 + e;
            float x = e < 4 ? x0[e] : x1[e - 4];
            if ((used >> e) & 1u) x = rep_penalise(x, a.rep_theta);
            if (n < a.N) top2_merge(v1, i1, v2, x, n, -INFINITY);
          }
        }
      }
#pragma unroll
      for (int x = 1; x < 8; x <<= 1) {
        const float o1 = __shfl_xor(v1, x), o2 = __shfl_xor(v2, x);
        const int oi = __shfl_xor(i1, x);
        top2_merge(v1, i1, v2, o1, oi, o2);
      }
      if ((lane & 7) == 0) {
        float* s3 = my_amax + (part * 8 + r) * 3;
        float w1 = s3[0], w2 = s3[2];
        int wi = __float_as_int(s3[1]);
        top2_merge(w1, wi, w2, v1, i1, v2);
        s3[0] = w1;
        s3[1] = __int_as_float(wi);
        s3[2] = w2;
      }
    } else if (EPI == EPI_SILU) {
      // lanes 0 .. 8 TPW - 1: row lane / TPW, tile lane % TPW; columns 0..7 of
      // the tile are gate rows tile*8 + c, 8..15 the matching up rows
      const int rs = lane / TPW, ts = lane % TPW;
      const int tile_s = tile0 + ts;
      const int ml_s = (rw * NP + part) * 8 + rs;
      if (lane < 8 * TPW && tile_s < a.n_tiles && ml_s < rows) {
        const int ms = a.m_base + ml_s;
        const float* gsrc = stage + rs * SROW + ts * 16;
        const int F = a.N / 2;
        const int n0 = tile_s * 8;
        uint16_t* base = a.y_apack ? a.y_apack + (((size_t)(ms >> 3) * (F / 8) + tile_s) * 16 + (ms & 7)) * 8 : nullptr;
        // two halves of 4 columns: 8-byte hi and lo pieces
#pragma unroll 1
        for (int hf = 0; hf < 2; ++hf) {
          const f32x4 gv = st4(gsrc + 4 * hf), uv = st4(gsrc + 8 + 4 * hf);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = silu_f(gv[e]) * uv[e];
          if (a.y) {
            float* yo = a.y + (size_t)ms * a.ldy + n0 + 4 * hf;
#pragma unroll
            for (int e = 0; e < 4; ++e) yo[e] = y[e];
          }
          if (base) {
            u32x2 hi, lo;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              uint32_t h0, l0, h1, l1;
              split_hi_lo(y[2 * e], h0, l0);
              split_hi_lo(y[2 * e + 1], h1, l1);
              hi[e] = h0 | (h1 << 16);
              lo[e] = l0 | (l1 << 16);
            }
            *(u32x2*)(base + 4 * hf) = hi;
            *(u32x2*)(base + 64 + 4 * hf) = lo;
          }
        }
      }
    } else {
#pragma unroll
      for (int gp = 0; gp < (C::NG + 7) / 8; ++gp) {
        const int grp = gp * 8 + (lane & 7);
        const int tile = tile0 + (grp >> 1), half = grp & 1;
        if (grp >= C::NG || !row_ok || tile >= a.n_tiles) continue;
        const float* src = stage + r * SROW + grp * 8;
        if (EPI == EPI_QKV || a.partial) {
          // K-slice partial sums (QKV: at the natural column of the operand;
          // the 8 columns of a half tile are consecutive there)
          const int n0 = EPI == EPI_QKV ? col_row<EPI_QKV>(a.N, tile, half * 8) : tile * 16 + half * 8;
          float* po = a.partial + ((size_t)ks * a.M + m) * a.N + n0;
          if (n0 + 8 <= a.N && (a.N & 3) == 0) {
            *(f32x4*)po = st4(src);
            *(f32x4*)(po + 4) = st4(src + 4);
          } else {
            for (int e = 0; e < 8 && n0 + e < a.N; ++e) po[e] = st1(src, e);
          }
        } else {
          // y = v (+ bias + residual)
          const int n0 = tile * 16 + half * 8;
#pragma unroll 1
          for (int e = 0; e < 8; ++e) {
            const int n = n0 + e;
            if (n >= a.N) break;
            float y = st1(src, e);
            if (a.bias) y += bf16_to_f32(a.bias[n]);
            if (a.residual) y += a.residual[(size_t)m * a.ldy + n];
            a.y[(size_t)m * a.ldy + n] = y;
          }
        }
      }
    }
  };
  // parts in straight-line order, so each reads only its own accumulators
  // (a rolled loop over parts makes the compiler copy all of them out first)
  auto epilogue = [&](int cblock) {
    static_for<NP>([&](auto pc) {
      stage_part(pc);
      epi_part(cblock, decltype(pc)::value);
      __builtin_amdgcn_sched_barrier(0);  // one part's temporaries live at a time
    });
  };

  if (total > 0) {
    // Stage bi: wait for my copies of the unit read next, barrier, then the
    // products of stage bi with the next unit's fragment reads (PREFETCH),
    // the copies of a later unit and the weights of stage bi + DW issued
    // among them.  The copies of stage bi + LA (+ 1 with PREFETCH) go to
    // the slot whose reads completed before this barrier.
    Pos cpos{0, 0, 0}, wpos{0, 0, 0}, ppos{0, 0, 0};
    int rslot = 0;  // slot of stage bi
    // ---- L2 prefetches of the stages whose weights the loop loads first
    if constexpr (C::NPF > 0) {
#pragma unroll
      for (int s = 0; s < DW; ++s) step(ppos);
#pragma unroll
      for (int s = DW; s < C::PF; ++s) {
        issue_pf(ppos);
        step(ppos);
      }
    }
    // ---- prologue: DW stages' loads in the loop's pattern (a stage with no
    // copy due repeats stage 0's: same bytes to the same place)
    constexpr int CLEAD = C::CLEAD;
#pragma unroll
    for (int s = -DW; s < 0; ++s) {
      if (s + CLEAD >= 0) {
        copy_stage(cpos);
        step(cpos);
      } else {
        copy_stage(Pos{0, 0, 0});
      }
      issue_w(wpos, st[s + DW]);
      step(wpos);
    }
    // copy streams still owed before stage 0 (a lead beyond DW stages)
#pragma unroll
    for (int s = DW; s < CLEAD; ++s) {
      copy_stage(cpos);
      step(cpos);
    }
    bf16x8 af[2][FR];  // PREFETCH: fragments of the current and the next stage
    if (C::PREFETCH) {
      wait_vmcnt<C::WAIT0>();
      stage_barrier();
      read_frags(frag_base(0), 0, af[0]);
    }

    for (int it = 0; it < n_my; ++it) {
      for (int u0 = 0; u0 < nup; u0 += C::R) {
#pragma unroll
        for (int j = 0; j < C::R; ++j) {
          wait_vmcnt<C::WAIT>();
          stage_barrier();
          const int nslot = rslot + 1 == NS ? 0 : rslot + 1;
          if (C::PREFETCH) read_frags(frag_base(nslot), 0, af[(j + 1) & 1]);
          copy_stage(cpos);
          step(cpos);
          issue_w(wpos, st[(j + DW) % C::R]);
          step(wpos);
          if constexpr (C::NPF > 0) {
            issue_pf(ppos);
            step(ppos);
          }
          if (C::PREFETCH) {
            compute_bf16(st[j], af[j & 1]);
            // one lone wave per SIMD: spread the stage's other instructions
            // between the products so they issue in the matrix core's shadow
#pragma unroll
            for (int k = 0; k < 2 * RT * CT; ++k) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // an LDS read
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // a global load
              __builtin_amdgcn_sched_group_barrier(0x004, 3, 0);  // scalar work
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // vector work
            }
          } else {
            compute_int4(rslot, st[j]);
          }
          rslot = nslot;
        }
      }
      epilogue(cb0 + it * gt);
    }
  }

  if (EPI == EPI_ARGMAX) {
    // merge the column waves' row states (fixed order) and write one partial
    // per row and workgroup (a workgroup without items writes -inf)
    __syncthreads();
    if (cw == 0) {
      for (int r = lane; r < NP * 8; r += 64) {
        const int ml = (rw * NP) * 8 + r;
        float v1 = -INFINITY, v2 = -INFINITY;
        int i1 = 0x7FFFFFFF;
        for (int w = 0; w < CW; ++w) {
          const float* s3 = amax_lds + ((size_t)(rw * CW + w) * NP * 8 + r) * 3;
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

// QKV from K-slice partial sums: bias, RoPE, q rows to y, window K/V (bf16)
// into the cache pages.  One workgroup per row and head, lane i2 < 64 takes the
// RoPE pair (i2, i2 + 64).
__global__ __launch_bounds__(64) void k_qkv_finish(GemmArgs a) {
  const int m = blockIdx.x, head = blockIdx.y, i2 = threadIdx.x;
  const int Hq = a.n_heads, Hkv = a.n_kv_heads;
  const int r1 = head * kHeadDim + i2, r2 = r1 + 64;
  float x1 = 0.f, x2 = 0.f;
  for (int s = 0; s < a.ksplit; ++s) {
    const float* p = a.partial + ((size_t)s * a.M + m) * a.N;
    x1 += p[r1];
    x2 += p[r2];
  }
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
    return;
  }
  if (a.flags && a.flags[m] != 0) return;
  const int b = m / a.W, jw = m - b * a.W;
  const int pos = a.prefix_len[b] + jw;
  if (pos < 0 || pos >= a.max_blocks * kBlock) return;
  const int blk = a.block_table[(size_t)b * a.max_blocks + pos / kBlock];
  if (blk < 0 || blk >= a.num_blocks) return;
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

template <int RT, bool INT4, int LAY>
static constexpr size_t wide_smem(int epi) {
  using C = Wide<RT, INT4, LAY>;
  return (size_t)C::NS * C::SLOT + kPfSink + (size_t)C::WAVES * C::SROWS * (C::SW + 4) * 4 +
         (epi == EPI_ARGMAX ? (size_t)C::WAVES * C::NP * 8 * 3 * 4 : 0);
}

// Rows per launch: 192 (bf16) or 64 (INT4).
int big_rows_per_launch(bool int4) { return int4 ? 64 : 192; }

// The large-M kernel serves bf16 GEMMs of more than 32 rows and INT4 ones of
// more than 32 except QKV, O and down at 49..64 rows, which the small-M
// kernel's two launches of 32 rows serve.  Up to 48 INT4 rows every
// projection takes one launch of the exact-fit grid (4): the INT4 step at
// batch 8 measured 4.09 -> 4.00 ms against two small-M launches each for QKV,
// O and down.
bool use_big_gemm(int M, bool int4, int epi, bool tiled) {
  if (!int4) return M > 32;
  if (!tiled) return false;  // INT4 scales are copied per item tile: tiled weights only
  return M > 64 || (M > 32 && (M <= 48 || epi == EPI_SILU || epi == EPI_ARGMAX));
}

// Wave grid of a GEMM (see Wide).  Measured at 192 rows: 96-column items
// (4 x 1) for the projections (gate/up 56.5 -> 51.8 us; O, down and QKV a
// little faster), 128-column items (2 x 2) for the lm_head (282 against 367 us).
// INT4 runs eight waves (4 x 2): the dequantisation and per-group scaling of
// one wave run beside the products of the other wave on its SIMD.
static int big_lay(int rows, bool int4, int epi) {
  // INT4 gate/up cannot take K slices: 96-column items (at 48 rows 30.7 us
  // against 37.2 with 128-column items; the lm_head is faster with 128); up
  // to 48 rows every INT4 GEMM takes the exact-fit grid (4), whose row tiles
  // hold the rows without padding (gate/up at 48 rows 26.7 -> 24.2 us; the
  // lm_head too once its scales came through LDS: the step 3.657 -> 3.645 ms)
  if (int4) return rows <= 48 ? 4 : epi == EPI_SILU ? 3 : 2;
  // 65..96 rows fill three 2 x 2 row tiles exactly, where 4 x 1 would pad to 128
  const int mt = (rows + 7) / 8;
  return epi == EPI_ARGMAX || (mt > 8 && mt <= 12) ? 0 : 1;
}

// Row tiles per row wave for a launch of `rows` rows: INT4 tiles of 16
// operand rows (64 rows in all); bf16 tiles of 32 operand rows (16 real rows).
static int big_rt(int rows, bool int4, int lay) {
  const int mt = (rows + 7) / 8;
  if (int4) return lay == 4 ? 3 : 2;
  if (lay == 0) return mt <= 8 ? 2 : mt <= 12 ? 3 : 6;
  return mt <= 8 ? 1 : mt <= 16 ? 2 : 3;
}

template <bool INT4, int LAY>
static size_t big_smem(int rt, int epi) {
  if (INT4) return LAY == 4 ? wide_smem<3, true, 4>(epi) : LAY == 3 ? wide_smem<2, true, 3>(epi)
                                                                    : wide_smem<2, true, 2>(epi);
  if (LAY == 0) return rt == 2 ? wide_smem<2, false, 0>(epi) : rt == 3 ? wide_smem<3, false, 0>(epi)
                                                                     : wide_smem<6, false, 0>(epi);
  return rt == 1 ? wide_smem<1, false, 1>(epi) : rt == 2 ? wide_smem<2, false, 1>(epi)
                                                         : wide_smem<3, false, 1>(epi);
}

BigPlan plan_gemm_big(int rows, int N, int K, bool int4, int epi, bool allow_split) {
  BigPlan p;
  p.lay = big_lay(rows, int4, epi);
  p.rt = big_rt(rows, int4, p.lay);
  p.n_tiles = (epi == EPI_SILU) ? (N / 2) / 8 : (N + 15) / 16;
  const int item = int4 ? (p.lay == 4 ? Wide<3, true, 4>::ITEM : p.lay == 3 ? Wide<2, true, 3>::ITEM
                                                                           : Wide<2, true, 2>::ITEM)
                        : p.lay == 1 ? Wide<3, false, 1>::ITEM : Wide<6, false, 0>::ITEM;
  const int n_cb = (p.n_tiles + item - 1) / item;
  const int cus = big_cus();
  const int units = int4 ? K / 128 : K / 32;
  const int dw = int4 ? (p.lay == 4 ? Wide<3, true, 4>::R : p.lay == 3 ? Wide<2, true, 3>::R
                                                                       : Wide<2, true, 2>::R)
                      : Wide<6, false>::R;  // stages per ring turn
  // K slices (QKV always writes slice sums; STORE when the caller takes them):
  // the fewest rounds of items times the padded stages of one item, plus the
  // slice sums' write and read-back counted in stage times (a stage of 192
  // rows measured at about 0.73 us; slice traffic at about 3 TB/s); on a tie
  // the fewer slices
  const bool can_split = epi == EPI_QKV || (allow_split && epi == EPI_STORE);
  const double stage_us = 0.73 * std::max(rows, 32) / 192.0;
  const double slice_stages = (double)rows * N * 8 / 3e6 / stage_us;
  double best = -1;
  p.ksplit = 1;
  // at most 12 slices: the next pack reads every slice's sums, and beyond about
  // a dozen that read costs more than the shorter items gain (measured on the
  // down projection at 192 rows: 11 slices 42 us with its pack, 15 slices 45)
  for (int ks = 1; ks <= (can_split ? 12 : 1); ++ks) {
    if (ks > 1 && units / ks < 4) break;
    const long items = (long)n_cb * ks;
    const long rounds = (items + cus - 1) / cus;
    const int per = (units + ks - 1) / ks;
    const double cost = (double)rounds * ((per + dw - 1) / dw * dw) + (ks > 1 ? ks * slice_stages : 0.0);
    if (best < 0 || cost < best - 1e-9) {
      best = cost;
      p.ksplit = ks;
    }
  }
  const int per_slice = std::max(1, cus / p.ksplit);
  const int per = (n_cb + per_slice - 1) / per_slice;
  const int gt = (n_cb + per - 1) / per;
  p.grid = gt * p.ksplit;
  p.threads = lay_threads(p.lay);
  p.smem = int4 ? (p.lay == 4 ? big_smem<true, 4>(p.rt, epi)
                   : p.lay == 3 ? big_smem<true, 3>(p.rt, epi) : big_smem<true, 2>(p.rt, epi))
                : (p.lay == 0 ? big_smem<false, 0>(p.rt, epi) : big_smem<false, 1>(p.rt, epi));
  return p;
}

template <int RT, bool INT4, int EPI, int LAY>
static hipError_t launch_big_one(const GemmArgs& a, const BigPlan& p, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_big<RT, INT4, EPI, LAY>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm_big<RT, INT4, EPI, LAY>), dim3(p.grid), dim3(p.threads), p.smem, s, a);
  return hipGetLastError();
}

template <int RT, bool INT4, int LAY>
static hipError_t launch_big_epi(const GemmArgs& a, int epi, const BigPlan& p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_big_one<RT, INT4, EPI_STORE, LAY>(a, p, s);
    case EPI_SILU: return launch_big_one<RT, INT4, EPI_SILU, LAY>(a, p, s);
    case EPI_QKV: return launch_big_one<RT, INT4, EPI_QKV, LAY>(a, p, s);
    default: return launch_big_one<RT, INT4, EPI_ARGMAX, LAY>(a, p, s);
  }
}

static hipError_t launch_big_plan(const GemmArgs& g, int epi, bool int4, const BigPlan& p,
                                  hipStream_t s) {
  if (int4) {
    if (p.lay == 4) return launch_big_epi<3, true, 4>(g, epi, p, s);
    return p.lay == 3 ? launch_big_epi<2, true, 3>(g, epi, p, s) : launch_big_epi<2, true, 2>(g, epi, p, s);
  }
  if (p.lay == 0) {
    if (p.rt == 2) return launch_big_epi<2, false, 0>(g, epi, p, s);
    if (p.rt == 3) return launch_big_epi<3, false, 0>(g, epi, p, s);
    return launch_big_epi<6, false, 0>(g, epi, p, s);
  }
  if (p.rt == 1) return launch_big_epi<1, false, 1>(g, epi, p, s);
  if (p.rt == 2) return launch_big_epi<2, false, 1>(g, epi, p, s);
  return launch_big_epi<3, false, 1>(g, epi, p, s);
}

hipError_t launch_gemm_big(GemmArgs a, int epi, bool int4, hipStream_t s) {
  // QKV writes K-slice sums and a finishing kernel does bias, RoPE and the
  // cache writes; its caller provides the slice buffer
  if (epi == EPI_QKV && !a.partial) return hipErrorInvalidValue;
  if (a.y_apack && epi == EPI_STORE) return hipErrorInvalidValue;  // fused RMSNorm: small M only
  if (a.ss_in) return hipErrorInvalidValue;
  const int per_launch = big_rows_per_launch(int4);
  // one plan for every launch (the slice sums and the lm_head parts are laid
  // out by it); a shorter last launch pads its row tiles
  const BigPlan p = plan_gemm_big(std::min(a.M, per_launch), a.N, a.K, int4, epi, a.partial != nullptr);
  for (int m0 = 0; m0 < a.M; m0 += per_launch) {
    GemmArgs g = a;
    g.m_base = m0;
    g.n_tiles = p.n_tiles;
    g.ksplit = p.ksplit;
    g.n_parts = p.grid;
    const hipError_t e = launch_big_plan(g, epi, int4, p, s);
    if (e != hipSuccess) return e;
  }
  if (epi == EPI_QKV) {
    GemmArgs g = a;
    g.ksplit = p.ksplit;
    const int heads = a.n_heads + 2 * a.n_kv_heads;
    hipLaunchKernelGGL(k_qkv_finish, dim3(a.M, heads), dim3(64), 0, s, g);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace la
