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

constexpr int gcd_(int a, int b) { return b == 0 ? a : gcd_(b, a % b); }

template <typename TA, typename TB, typename OutT, int BM, int BN, int WGM, int WGN, int AMODE,
          int BMODE, int EMODE, int SA, int SB>
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
  constexpr int A_W = A_INST / NW, B_W = B_INST / NW;  // DMA instructions per wave per K step
  // Two LDS rings: SA stages of A rows and SB >= SA stages of B rows (the
  // B ring is deeper where B is the HBM-streamed weight matrix).
  constexpr int kStageA = BM * ROWB, kStageB = BN * ROWB;
  constexpr int RING = SA * kStageA + SB * kStageB;
  constexpr int UNROLL = SA * SB / gcd_(SA, SB);
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "32x32 sub-tiles");
  static_assert(BMODE != B_DUAL || TN % 2 == 0, "dual tile needs gate and up sub-tiles");
  static_assert(A_INST % NW == 0 && B_INST % NW == 0 && BM % 16 == 0 && BN % 16 == 0, "DMA split");
  static_assert(SA >= 2 && SB >= SA && UNROLL <= 8, "ring shape");
  __shared__ __attribute__((aligned(1024))) char smem[RING];
  char* const ringA = smem;
  char* const ringB = smem + SA * kStageA;

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

  // ---- DMA plan.  For each operand, wave `wave` moves 16-row blocks
  // wave*X_W + ii of the tile.  Lane l carries tile row block*16 + l/4 and
  // lands at LDS slot l%4 of that row; it fetches global 16-byte chunk
  // (l%4) ^ ((l>>4)&3), i.e. rows are XOR-swizzled so that the fragment
  // reads of 16 consecutive rows hit 16 distinct bank groups.  Rows past the
  // valid range are clamped to the last valid row: every DMA instruction is
  // always issued, which keeps the vmcnt accounting exact.
  const uint32_t lane_chunk = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  constexpr int H = BMODE == B_DUAL ? BN / 2 : BN;  // rows of one B matrix per tile
  const int b_rows_here = min(H, args.nb_rows - nt * H);
  const char* a_base;
  uint32_t a_off[A_W];
  if constexpr (AMODE == A_GATHER) a_base = args.a;
  else if constexpr (AMODE == A_PADDED) a_base = args.a + ((int64_t)e * args.cap + m0) * args.lda;
  else if constexpr (AMODE == A_SORTED) a_base = args.a + (off + m0) * args.lda;
  else a_base = args.a + (int64_t)m0 * args.lda;
#pragma unroll
  for (int ii = 0; ii < A_W; ++ii) {
    const int rr = min((wave * A_W + ii) * 16 + (lane >> 2), rows_valid - 1);
    int64_t row = rr;
    if constexpr (AMODE == A_GATHER) row = args.order[off + m0 + rr] / args.top_k;
    a_off[ii] = (uint32_t)(row * args.lda) + lane_chunk;
  }
  const char* b_base[B_W];  // workgroup-uniform
  uint32_t b_off[B_W];      // per lane, K step 0
  int b_brow[B_W];          // clamped row inside the tile's slice of its matrix
#pragma unroll
  for (int ii = 0; ii < B_W; ++ii) {
    const int r = (wave * B_W + ii) * 16 + (lane >> 2);
    const bool up = BMODE == B_DUAL && r >= H;
    const int br = min(up ? r - H : r, b_rows_here - 1);
    b_brow[ii] = br;
    b_base[ii] = (up ? args.b1 : args.b0) + (int64_t)e * args.b_expert_stride + (int64_t)nt * H * args.ldb;
    b_off[ii] = (uint32_t)(br * args.ldb) + lane_chunk;
  }

  auto issue_a = [&](int kt, char* stage) {
#pragma unroll
    for (int ii = 0; ii < A_W; ++ii) {
      const char* g = a_base + (a_off[ii] + (uint32_t)kt * ROWB);
      __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + (wave * A_W + ii) * 16 * ROWB), 16, 0, 0);
    }
  };
  auto issue_b = [&](int kt, char* stage) {
    if constexpr (BMODE == B_KSEG) {
      int s = 0;
      while (s + 1 < args.nseg && kt >= args.seg_kt0[s + 1]) ++s;
      const int64_t ld = args.seg_ld[s];
      const char* bbase = args.seg_base[s] + (int64_t)nt * BN * ld + (int64_t)(kt - args.seg_kt0[s]) * ROWB;
#pragma unroll
      for (int ii = 0; ii < B_W; ++ii) {
        const char* g = bbase + ((uint32_t)(b_brow[ii] * ld) + lane_chunk);
        __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + (wave * B_W + ii) * 16 * ROWB), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < B_W; ++ii) {
        const char* g = b_base[ii] + (b_off[ii] + (uint32_t)kt * ROWB);
        __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + (wave * B_W + ii) * 16 * ROWB), 16, 0, 0);
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
  auto compute = [&](const char* As, const char* Bs, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
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

  // ---- main loop.  Tile t of A sits in A stage t % SA, of B in B stage
  // t % SB.  Step s issues, right after its barrier, the B DMA of tile
  // s + SB - 1 and then the A DMA of tile s + SA - 1; each overwrites the
  // stage that step s - 1 read, which that same barrier released.  With B
  // issued first in every step (and SB >= SA), waiting for A of tile kt also
  // covers B of tile kt, so one vmcnt per step suffices: the operations
  // issued after A(kt) are B tiles kt+SB-SA+1 .. kt+SB-2 and A tiles
  // kt+1 .. kt+SA-2 (SA-2 of each).
  const int KT = args.K * (int)sizeof(TA) / ROWB;
  constexpr int kNewer = (SA - 2) * (B_W + A_W);  // steady-state vmcnt
#pragma unroll
  for (int s = -(SB - 1); s < 0; ++s) {  // the steps before step 0, issue part only
    const int tb = s + SB - 1, ta = s + SA - 1;
    if (tb >= 0 && tb < KT) issue_b(tb, ringB + tb * kStageB);
    if (ta >= 0 && ta < KT) issue_a(ta, ringA + ta * kStageA);
  }
  auto barrier = [&]() {
    asm volatile("" ::: "memory");  // no LDS access may move across the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // steady steps: every tile counted in kNewer exists (kt + SB - 2 < KT)
  const int n_steady = KT - SB + 2 > 0 ? KT - SB + 2 : 0;
  auto main_loop = [&](auto na_c) {
    auto steady = [&](int kt, auto u_c) {
      constexpr int u = decltype(u_c)::value;  // kt % UNROLL, stages are static
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kNewer));
      barrier();
      if (kt + SB - 1 < KT) issue_b(kt + SB - 1, ringB + ((u + SB - 1) % SB) * kStageB);
      if (kt + SA - 1 < KT) issue_a(kt + SA - 1, ringA + ((u + SA - 1) % SA) * kStageA);
      compute(ringA + (u % SA) * kStageA, ringB + (u % SB) * kStageB, na_c);
    };
    for (int kt = 0; kt < n_steady; kt += UNROLL) {
      steady(kt, IntC<0>{});
      if constexpr (UNROLL > 1) if (kt + 1 < n_steady) steady(kt + 1, IntC<1>{});
      if constexpr (UNROLL > 2) if (kt + 2 < n_steady) steady(kt + 2, IntC<2>{});
      if constexpr (UNROLL > 3) if (kt + 3 < n_steady) steady(kt + 3, IntC<3>{});
      if constexpr (UNROLL > 4) if (kt + 4 < n_steady) steady(kt + 4, IntC<4>{});
      if constexpr (UNROLL > 5) if (kt + 5 < n_steady) steady(kt + 5, IntC<5>{});
      if constexpr (UNROLL > 6) if (kt + 6 < n_steady) steady(kt + 6, IntC<6>{});
      if constexpr (UNROLL > 7) if (kt + 7 < n_steady) steady(kt + 7, IntC<7>{});
    }
    // last SB-2 steps: full waits (stage indices are no longer static here)
    for (int kt = n_steady; kt < KT; ++kt) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      barrier();
      if (kt + SA - 1 < KT) issue_a(kt + SA - 1, ringA + ((kt + SA - 1) % SA) * kStageA);
      compute(ringA + (kt % SA) * kStageA, ringB + (kt % SB) * kStageB, na_c);
    }
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

  // ---- epilogue.  Each wave stages its finished output tile in LDS (the
  // operand ring is free once every wave has passed the barrier below) and
  // writes it back as 16-byte row chunks; falls back to per-element stores
  // when the staged tile would not fit.
  constexpr int TJ = (BMODE == B_DUAL) ? TN / 2 : TN;
  constexpr int OCOLS = TJ * 32;  // output columns of one wave
  constexpr int OES = (int)sizeof(OutT);
  constexpr int CPR = OCOLS * OES / 16;  // 16-byte chunks per staged row
  constexpr bool kPad = WTM * (OCOLS * OES + 16) * NW <= RING;
  constexpr bool kSwz = !kPad && WTM * OCOLS * OES * NW <= RING && CPR >= 8;
  constexpr bool kStaged = (kPad || kSwz) && (OCOLS * OES) % 16 == 0;
  constexpr int EROW = OCOLS * OES + (kPad ? 16 : 0);
  const float inv_b1 = 1.0f / args.beta1, inv_b2 = 1.0f / args.beta2;
  const int col0 = BMODE == B_DUAL ? nt * (BN / 2) + wn * (WTN / 2) : nt * BN + wn * WTN;

  auto value = [&](int i, int j, int v) -> float {
    if constexpr (EMODE == E_SITU)
      return situ_hidden(acc[i][j][v], acc[i][j + TN / 2][v], args.beta1, args.beta2, inv_b1, inv_b2);
    else
      return acc[i][j][v];
  };
  auto out_row = [&](int r) -> int64_t {  // r: row inside the block tile
    if constexpr (EMODE == E_SLOTS) return args.order[off + m0 + r];
    else return GROUPED ? off + m0 + r : (int64_t)(m0 + r);
  };

  if constexpr (kStaged) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // every wave is done reading the ring
    asm volatile("" ::: "memory");
    char* E = smem + wave * (WTM * EROW);
    auto pos = [](int rl, int c) -> int { return rl * EROW + ((kSwz ? (c ^ (rl & 7)) : c) << 4); };
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float ps[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        ps[v] = 1.f;
        if constexpr (EMODE == E_SLOTS) {
          const int r = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          ps[v] = r < rows_valid ? args.probs[args.order[off + m0 + r]] : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int cb = (j * 32 + lr) * OES;  // byte column inside the staged row
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          float val = value(i, j, v);
          if constexpr (EMODE == E_SLOTS) val *= ps[v];
          Elem<OutT>::store((OutT*)(E + pos(rl, cb >> 4) + (cb & 15)), val);
        }
      }
    }
    const bool aligned = (((uintptr_t)args.out | (uintptr_t)args.ldo) & 15) == 0;
    constexpr int EPC = 16 / OES;  // elements per chunk
    for (int id = lane; id < WTM * CPR; id += 64) {
      const int rl = id / CPR, c = id % CPR;
      const int r = wm * WTM + rl;
      const int col = col0 + c * EPC;
      if (r >= rows_valid || col >= args.N) continue;
      const char* src = E + pos(rl, c);
      OutT* dst = (OutT*)(args.out + out_row(r) * args.ldo) + col;
      if (aligned && col + EPC <= args.N) {
        *(u32x4*)dst = *(const u32x4*)src;
      } else {
        for (int q = 0; q < EPC && col + q < args.N; ++q) dst[q] = ((const OutT*)src)[q];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = col0 + j * 32 + lr;
        if (col >= args.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          if (r >= rows_valid) continue;
          float val = value(i, j, v);
          if constexpr (EMODE == E_SLOTS) val *= args.probs[args.order[off + m0 + r]];
          Elem<OutT>::store((OutT*)(args.out + out_row(r) * args.ldo) + col, val);
        }
      }
    }
  }
}

}  // namespace lmoe
