// One MFMA GEMM family for every matrix product of the layer.
//
//   out[m, n] = sum_k A[m, k] * B[n, k]      (A rows and B rows both K-contiguous,
//                                             B stored like an nn.Linear weight)
//
// Workgroup: 4 or 8 wave64s in a WGM x WGN grid; block tile BM x BN;
// K advances 64 bytes per step (32 bf16/fp16 or 16 fp32).  Operand tiles go
// straight from global memory into LDS with gfx950's LDS-DMA loads
// (global_load_lds_dwordx4) through a 4-stage ring, one barrier per K step.
//
// Matrix cores: v_mfma_f32_32x32x16_bf16 / _f16 (gfx950) for 2-byte operands,
// v_mfma_f32_32x32x2f32 for fp32.  With an fp16 A operand and bf16 weights the
// B fragments are widened bf16 -> fp16 in registers after the LDS read.
// Lane l supplies row (l % 32) of A and column (l % 32) of B with the K slice
// selected by (l / 32); the 16 accumulator values of lane l are rows
// 8*(v/4) + 4*(l/32) + (v%4), column l % 32 of the 32x32 sub-tile.
//
// Variants (template parameters):
//   A_DENSE   A row m of a dense matrix
//   A_GATHER  grouped by expert: A row = z[order[offsets[e] + r] / k]   (routed, no padded copy)
//   A_PADDED  grouped by expert: A row = padded[e * C + r]              (pages' [R, C, l] layout)
//   A_SORTED  grouped by expert: A row = h[offsets[e] + r]              (rows in sorted pair order)
//   B_SINGLE  one weight matrix (per expert in grouped mode)
//   B_DUAL    gate and up matrices interleaved per tile (BN/2 rows of each)
//   B_KSEG    B concatenated along K from up to kMaxSeg separate matrices
//   E_STORE   plain store (fp32 or storage dtype), masked to valid rows/cols
//   E_SITU    SiTU-GLU hidden of the (gate, up) accumulator pair, stored as OutT
//   E_SLOTS   p-weighted result of sorted pair q written to its own slot row q
#pragma once

#include "lmoe_common.h"

namespace lmoe {

enum { A_DENSE = 0, A_GATHER = 1, A_PADDED = 2, A_SORTED = 3 };
enum { B_SINGLE = 0, B_DUAL = 1, B_KSEG = 2 };
enum { E_STORE = 0, E_SITU = 1, E_SLOTS = 2 };

template <int V>
struct IntC {
  static constexpr int value = V;
};

constexpr int kMaxSeg = 17;
constexpr int kKStepBytes = 64;  // bytes of every tile row consumed per K step

struct GemmArgs {
  int M;        // dense: rows of A / out
  int N;        // valid output columns
  int K;        // reduction length (elements)
  int m_tiles;  // dense: ceil(M / BM); grouped: bound on the tile list length
  int n_tiles;
  // A
  const char* a;
  int64_t lda;  // bytes
  const int32_t* order;
  int top_k;
  int64_t cap;  // A_PADDED: rows per expert
  // grouped tiles
  const int32_t* tile_list;  // (expert, m0) pairs
  const int32_t* tile_count;
  const int32_t* counts;
  const int32_t* offsets;
  // B
  const char* b0;
  const char* b1;
  int64_t ldb;            // bytes
  int64_t b_expert_stride;  // bytes
  int nb_rows;            // rows of each B matrix (clamp)
  int nseg;
  const char* seg_base[kMaxSeg];
  int64_t seg_ld[kMaxSeg];
  int seg_kt0[kMaxSeg + 1];  // first K step (of kKStepBytes per row) of each segment
  // out
  char* out;
  int64_t ldo;  // bytes (E_SLOTS: fp32 elements per slot row * 4)
  const float* probs;
  float beta1, beta2;
};

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; expcnt / lgkmcnt left at "no wait").
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

typedef __attribute__((address_space(3))) void lds_void_t;

template <typename TA, typename TB, typename OutT, int BM, int BN, int WGM, int WGN, int AMODE,
          int BMODE, int EMODE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(const GemmArgs args) {
  static_assert(sizeof(TA) == sizeof(TB), "operand element sizes must match");
  constexpr bool kHalf = sizeof(TA) == 2;  // 16-bit operands
  constexpr bool kF16 = __is_same(TA, f16_t);
  constexpr bool kWiden = kF16 && __is_same(TB, bf16_t);
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr bool GROUPED = AMODE != A_DENSE;
  // K step: 64 bytes of every tile row.  One LDS-DMA wave instruction moves
  // 64 lanes x 16 bytes = 16 tile rows.
  constexpr int ROWB = kKStepBytes;
  constexpr int A_INST = BM / 16, B_INST = BN / 16;
  constexpr int INST = (A_INST + B_INST) / NW;  // DMA instructions per wave per K step
  constexpr int STAGES = 4;
  constexpr int kStage = (BM + BN) * ROWB;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "32x32 sub-tiles");
  static_assert(BMODE != B_DUAL || TN % 2 == 0, "dual tile needs gate and up sub-tiles");
  static_assert((A_INST + B_INST) % NW == 0 && BM % 16 == 0 && BN % 16 == 0, "DMA split");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, lh = lane >> 5;

  int mt, nt;
  if constexpr (GROUPED) {
    // The grid is sized by a bound on the tile list; only the first
    // tile_count * n_tiles workgroup ids carry work.  Those ids reach the
    // XCDs round-robin, so renumbering over the real count keeps every XCD
    // busy.  N tiles of one expert tile are neighbours: they share its A rows.
    const int total = *args.tile_count * args.n_tiles;
    if ((int)blockIdx.x >= total) return;  // uniform over the workgroup
    const int L = xcd_contiguous_id(blockIdx.x, total);
    mt = L / args.n_tiles;
    nt = L % args.n_tiles;
  } else {
    const int total = args.m_tiles * args.n_tiles;
    const int L = xcd_contiguous_id(blockIdx.x, total);
    constexpr int GM = 8;  // raster: groups of 8 M tiles sweep all N tiles
    const int group = L / (GM * args.n_tiles);
    const int first_m = group * GM;
    const int gsize = min(args.m_tiles - first_m, GM);
    const int in = L - group * GM * args.n_tiles;
    mt = first_m + in % gsize;
    nt = in / gsize;
  }

  int m0, rows_valid, e = 0;
  int64_t off = 0;
  if constexpr (GROUPED) {
    e = args.tile_list[2 * mt];
    m0 = args.tile_list[2 * mt + 1];
    rows_valid = min(BM, args.counts[e] - m0);
    off = args.offsets[e];
  } else {
    m0 = mt * BM;
    rows_valid = min(BM, args.M - m0);
  }

  // ---- DMA plan.  Wave `wave` moves tile-row blocks (wave*INST + ii)*16 ...
  // of the stacked [A rows | B rows] tile.  Lane l carries tile row
  // block*16 + l/4 and lands at LDS slot l%4 of that row; it fetches global
  // 16-byte chunk (l%4) ^ ((l>>4)&3), i.e. rows are XOR-swizzled so that the
  // fragment reads of 16 consecutive rows hit 16 distinct bank groups.
  // Rows past the valid range are clamped to the last valid row: every DMA
  // instruction is always issued, which keeps the vmcnt accounting exact.
  const uint32_t lane_chunk = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  constexpr int H = BMODE == B_DUAL ? BN / 2 : BN;  // rows of one B matrix per tile
  const int b_rows_here = min(H, args.nb_rows - nt * H);
  const char* dma_base[INST];  // workgroup-uniform
  uint32_t dma_off[INST];      // per lane, K step 0
  int dma_brow[INST];          // B_KSEG: clamped row inside the tile's slice
  bool dma_is_b[INST];
#pragma unroll
  for (int ii = 0; ii < INST; ++ii) {
    const int blk = wave * INST + ii;
    const int trow = blk * 16 + (lane >> 2);
    dma_brow[ii] = 0;
    if (blk < A_INST) {
      dma_is_b[ii] = false;
      const int rr = min(trow, rows_valid - 1);
      int64_t row = rr;
      if constexpr (AMODE == A_GATHER) {
        row = args.order[off + m0 + rr] / args.top_k;
        dma_base[ii] = args.a;
      } else if constexpr (AMODE == A_PADDED) {
        dma_base[ii] = args.a + ((int64_t)e * args.cap + m0) * args.lda;
      } else if constexpr (AMODE == A_SORTED) {
        dma_base[ii] = args.a + (off + m0) * args.lda;
      } else {
        dma_base[ii] = args.a + (int64_t)m0 * args.lda;
      }
      dma_off[ii] = (uint32_t)(row * args.lda) + lane_chunk;
    } else {
      dma_is_b[ii] = true;
      const int r = trow - BM;
      const bool up = BMODE == B_DUAL && r >= H;
      const int br = min(up ? r - H : r, b_rows_here - 1);
      dma_brow[ii] = br;
      dma_base[ii] = (up ? args.b1 : args.b0) + (int64_t)e * args.b_expert_stride +
                     (int64_t)nt * H * args.ldb;
      dma_off[ii] = (uint32_t)(br * args.ldb) + lane_chunk;
    }
  }

  auto issue_dma = [&](int kt, char* stage) {
    if constexpr (BMODE == B_KSEG) {
      int s = 0;
      while (s + 1 < args.nseg && kt >= args.seg_kt0[s + 1]) ++s;
      const int64_t ld = args.seg_ld[s];
      const char* bbase = args.seg_base[s] + (int64_t)nt * BN * ld + (int64_t)(kt - args.seg_kt0[s]) * ROWB;
#pragma unroll
      for (int ii = 0; ii < INST; ++ii) {
        const int blk = wave * INST + ii;
        const char* g = dma_is_b[ii] ? bbase + ((uint32_t)(dma_brow[ii] * ld) + lane_chunk)
                                     : dma_base[ii] + (dma_off[ii] + (uint32_t)kt * ROWB);
        __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + blk * 16 * ROWB), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < INST; ++ii) {
        const int blk = wave * INST + ii;
        const char* g = dma_base[ii] + (dma_off[ii] + (uint32_t)kt * ROWB);
        __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + blk * 16 * ROWB), 16, 0, 0);
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto b_tile_row = [&](int j) -> int {
    if constexpr (BMODE == B_DUAL) {
      constexpr int HW = WTN / 2;
      return j < TN / 2 ? wn * HW + j * 32 : H + wn * HW + (j - TN / 2) * 32;
    } else {
      return wn * WTN + j * 32;
    }
  };
  // physical byte offset of logical 16-byte chunk c of tile row `row`
  auto swz = [](int row, int c) -> int { return row * ROWB + ((c ^ ((row >> 2) & 3)) << 4); };

  // Multiply one K step held in LDS.  NA = number of this wave's 32-row
  // sub-tiles that hold valid rows (a wave-uniform constant of the
  // instantiation, so the step is straight-line code).
  auto compute = [&](const char* As, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const char* Bs = As + BM * ROWB;
    // two fragment chunks per lane per K step:
    //   16-bit: chunk lh holds k 8lh..8lh+7 of step 0, chunk 2+lh those of step 1
    //   fp32:   chunks 2lh and 2lh+1 hold k 8lh..8lh+7, one k per MFMA
    u32x4 fa[2][NA > 0 ? NA : 1], fb[2][TN];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = kHalf ? (2 * c + lh) : (2 * lh + c);
#pragma unroll
      for (int i = 0; i < NA; ++i) fa[c][i] = *(const u32x4*)(As + swz(wm * WTM + i * 32 + lr, ch));
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[c][j] = *(const u32x4*)(Bs + swz(b_tile_row(j) + lr, ch));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if constexpr (kWiden) fb[c][j] = bf16x8_to_f16x8(fb[c][j]);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (kF16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa[c][i]),
                                                               __builtin_bit_cast(f16x8, fb[c][j]),
                                                               acc[i][j], 0, 0, 0);
          } else if constexpr (kHalf) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[c][i]),
                                                                __builtin_bit_cast(bf16x8, fb[c][j]),
                                                                acc[i][j], 0, 0, 0);
          } else {
            const f32x4 a4 = __builtin_bit_cast(f32x4, fa[c][i]);
            const f32x4 b4 = __builtin_bit_cast(f32x4, fb[c][j]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[q], b4[q], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---- main loop: a 4-deep LDS ring.  Tile t sits in stage t % 4; the DMA
  // of tile t + 3 is issued right after the barrier that opens step t, so
  // three K steps of loads are in flight while one is multiplied.  The
  // stage it overwrites (t - 1) was released by that same barrier.
  const int KT = args.K * (int)sizeof(TA) / ROWB;
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    if (t < KT) issue_dma(t, smem + t * kStage);
  // wait for this wave's DMAs of tile kt with `later` newer tiles still in
  // flight, then make every wave's DMAs of tile kt visible
  auto sync_tile = [&](auto later_c) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(later_c)::value * INST));
    asm volatile("" ::: "memory");  // no LDS access may move across the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  using C0 = IntC<0>;
  using C1 = IntC<1>;
  using C2 = IntC<2>;
  const int n_steady = KT > 2 ? KT - 2 : 0;
  auto main_loop = [&](auto na_c) {
    // steady steps kt = 0 .. KT-3 (two newer tiles in flight), static stages
    auto steady = [&](int kt, char* cur, char* refill) {
      sync_tile(C2{});
      if (kt + 3 < KT) issue_dma(kt + 3, refill);
      compute(cur, na_c);
    };
    for (int kt = 0; kt < n_steady; kt += STAGES) {
      steady(kt, smem + 0 * kStage, smem + 3 * kStage);
      if (kt + 1 < n_steady) steady(kt + 1, smem + 1 * kStage, smem + 0 * kStage);
      if (kt + 2 < n_steady) steady(kt + 2, smem + 2 * kStage, smem + 1 * kStage);
      if (kt + 3 < n_steady) steady(kt + 3, smem + 3 * kStage, smem + 2 * kStage);
    }
    // last two steps: one, then no newer tile in flight
    if (KT >= 2) {
      sync_tile(C1{});
      compute(smem + ((KT - 2) & 3) * kStage, na_c);
    }
    sync_tile(C0{});
    compute(smem + ((KT - 1) & 3) * kStage, na_c);
  };
  if constexpr (GROUPED) {
    // sub-tiles of this wave that hold valid rows (uniform across the wave)
    const int na = __builtin_amdgcn_readfirstlane(
        max(0, min(TM, (rows_valid - wm * WTM + 31) / 32)));
    static_assert(TM <= 8, "sub-tile dispatch covers up to 8");
    switch (na) {
      case 0: main_loop(IntC<0>{}); break;
      case 1: if constexpr (TM >= 1) main_loop(IntC<1>{}); break;
      case 2: if constexpr (TM >= 2) main_loop(IntC<2>{}); break;
      case 3: if constexpr (TM >= 3) main_loop(IntC<3>{}); break;
      case 4: if constexpr (TM >= 4) main_loop(IntC<4>{}); break;
      case 5: if constexpr (TM >= 5) main_loop(IntC<5>{}); break;
      case 6: if constexpr (TM >= 6) main_loop(IntC<6>{}); break;
      case 7: if constexpr (TM >= 7) main_loop(IntC<7>{}); break;
      default: if constexpr (TM >= 8) main_loop(IntC<8>{}); break;
    }
  } else {
    main_loop(IntC<TM>{});
  }

  // ---- epilogue
  constexpr int TJ = (BMODE == B_DUAL) ? TN / 2 : TN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      int col;
      if constexpr (BMODE == B_DUAL) col = nt * (BN / 2) + wn * (WTN / 2) + j * 32 + lr;
      else col = nt * BN + wn * WTN + j * 32 + lr;
      if (col >= args.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (r >= rows_valid) continue;
        if constexpr (EMODE == E_SLOTS) {
          const int q = args.order[off + m0 + r];
          Elem<OutT>::store((OutT*)(args.out + (int64_t)q * args.ldo) + col, args.probs[q] * acc[i][j][v]);
        } else {
          const int64_t orow = GROUPED ? off + m0 + r : (int64_t)(m0 + r);
          float val;
          if constexpr (EMODE == E_SITU)
            val = situ_hidden(acc[i][j][v], acc[i][j + TN / 2][v], args.beta1, args.beta2);
          else val = acc[i][j][v];
          Elem<OutT>::store((OutT*)(args.out + orow * args.ldo) + col, val);
        }
      }
    }
  }
}

}  // namespace lmoe
