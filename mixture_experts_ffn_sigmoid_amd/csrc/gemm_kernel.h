// One MFMA GEMM family for every matrix product of the layer.
//
//   out[m, n] = sum_k A[m, k] * B[n, k]      (A rows and B rows both K-contiguous,
//                                             B stored like an nn.Linear weight)
//
// Workgroup: 256 threads = 4 wave64s in a WGM x WGN grid; block tile BM x BN;
// K advances 128 bytes per step (64 bf16 or 32 fp32).  Operand tiles go
// global -> registers -> LDS (double buffered, one barrier per K step); the
// next K step's global loads are in flight while the current one is
// multiplied.  LDS rows are padded to 144 bytes so that the 16-byte fragment
// reads of 32 consecutive rows hit distinct banks.
//
// Matrix cores: v_mfma_f32_32x32x16_bf16 / _f16 (gfx950) for 2-byte operands,
// v_mfma_f32_32x32x2f32 for fp32.  With an fp16 A operand and bf16 weights the
// B tile is widened bf16 -> fp16 on its way into LDS.  Lane l supplies row (l % 32) of A and column (l % 32) of B with
// the K slice selected by (l / 32); the 16 accumulator values of lane l are
// rows 8*(v/4) + 4*(l/32) + (v%4), column l % 32 of the 32x32 sub-tile.
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

constexpr int kMaxSeg = 17;
constexpr int kLdsRow = 144;  // bytes per LDS tile row: 128 data + 16 pad

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
  int seg_kt0[kMaxSeg + 1];
  // out
  char* out;
  int64_t ldo;  // bytes (E_SLOTS: fp32 elements per slot row * 4)
  const float* probs;
  float beta1, beta2;
};

template <typename TA, typename TB, typename OutT, int BM, int BN, int WGM, int WGN, int AMODE,
          int BMODE, int EMODE>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs args) {
  static_assert(sizeof(TA) == sizeof(TB), "operand element sizes must match");
  constexpr bool kHalf = sizeof(TA) == 2;  // 16-bit operands
  constexpr bool kF16 = __is_same(TA, f16_t);
  constexpr bool kWiden = kF16 && __is_same(TB, bf16_t);
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_LD = BM / 32, B_LD = BN / 32;
  constexpr bool GROUPED = AMODE != A_DENSE;
  static_assert(WGM * WGN == 4, "4 waves per workgroup");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "32x32 sub-tiles");
  static_assert(BMODE != B_DUAL || TN % 2 == 0, "dual tile needs gate and up sub-tiles");
  constexpr int kStage = (BM + BN) * kLdsRow;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, lh = lane >> 5;
  const int chunk = tid & 7, trow = tid >> 3;

  const int total = args.m_tiles * args.n_tiles;
  const int L = xcd_contiguous_id(blockIdx.x, total);
  int mt, nt;
  if constexpr (GROUPED) {
    mt = L % args.m_tiles;
    nt = L / args.m_tiles;
  } else {
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
    if (mt >= *args.tile_count) return;  // uniform over the workgroup
    e = args.tile_list[2 * mt];
    m0 = args.tile_list[2 * mt + 1];
    rows_valid = min(BM, args.counts[e] - m0);
    off = args.offsets[e];
  } else {
    m0 = mt * BM;
    rows_valid = min(BM, args.M - m0);
  }

  // ---- per-thread global row pointers (rows past the valid range are clamped
  // to the last valid row; their results are never stored)
  const char* a_ptr[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int rr = min(trow + 32 * i, rows_valid - 1);
    int64_t row;
    if constexpr (AMODE == A_DENSE) row = m0 + rr;
    else if constexpr (AMODE == A_GATHER) row = args.order[off + m0 + rr] / args.top_k;
    else if constexpr (AMODE == A_PADDED) row = (int64_t)e * args.cap + m0 + rr;
    else row = off + m0 + rr;
    a_ptr[i] = args.a + row * args.lda + chunk * 16;
  }
  const char* b_ptr[B_LD];
  int64_t b_row[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = trow + 32 * i;
    if constexpr (BMODE == B_DUAL) {
      constexpr int H = BN / 2;
      const bool up = r >= H;
      const int n = min(nt * H + (up ? r - H : r), args.nb_rows - 1);
      b_ptr[i] = (up ? args.b1 : args.b0) + (int64_t)e * args.b_expert_stride + n * args.ldb + chunk * 16;
      b_row[i] = n;
    } else {
      const int n = min(nt * BN + r, args.nb_rows - 1);
      b_ptr[i] = args.b0 + (int64_t)e * args.b_expert_stride + n * args.ldb + chunk * 16;
      b_row[i] = n;
    }
  }

  u32x4 ra[A_LD], rb[B_LD];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4*)(a_ptr[i] + (int64_t)kt * 128);
    if constexpr (BMODE == B_KSEG) {
      int s = 0;
      while (s + 1 < args.nseg && kt >= args.seg_kt0[s + 1]) ++s;
      const char* base = args.seg_base[s] + (int64_t)(kt - args.seg_kt0[s]) * 128 + chunk * 16;
      const int64_t ld = args.seg_ld[s];
#pragma unroll
      for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4*)(base + b_row[i] * ld);
    } else {
#pragma unroll
      for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4*)(b_ptr[i] + (int64_t)kt * 128);
    }
  };
  auto store_tile = [&](int buf) {
    char* As = smem + buf * kStage;
    char* Bs = As + BM * kLdsRow;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4*)(As + (trow + 32 * i) * kLdsRow + chunk * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      u32x4 v = rb[i];
      if constexpr (kWiden) v = bf16x8_to_f16x8(v);
      *(u32x4*)(Bs + (trow + 32 * i) * kLdsRow + chunk * 16) = v;
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
      constexpr int H = BN / 2, HW = WTN / 2;
      return j < TN / 2 ? wn * HW + j * 32 : H + wn * HW + (j - TN / 2) * 32;
    } else {
      return wn * WTN + j * 32;
    }
  };

  auto compute = [&](int buf) {
    const char* As = smem + buf * kStage;
    const char* Bs = As + BM * kLdsRow;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int koff = kHalf ? (c * 32 + lh * 16) : (lh * 64 + c * 16);
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = *(const u32x4*)(As + (wm * WTM + i * 32 + lr) * kLdsRow + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = *(const u32x4*)(Bs + (b_tile_row(j) + lr) * kLdsRow + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (GROUPED && wm * WTM + i * 32 >= rows_valid) continue;  // all 32 rows are padding
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (kF16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa[i]),
                                                               __builtin_bit_cast(f16x8, fb[j]),
                                                               acc[i][j], 0, 0, 0);
          } else if constexpr (kHalf) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[i]),
                                                                __builtin_bit_cast(bf16x8, fb[j]),
                                                                acc[i][j], 0, 0, 0);
          } else {
            const f32x4 a4 = __builtin_bit_cast(f32x4, fa[i]);
            const f32x4 b4 = __builtin_bit_cast(f32x4, fb[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[q], b4[q], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  const int KT = args.K * (int)sizeof(TA) / 128;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    compute(cur);
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
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
          float* dst = (float*)(args.out + (int64_t)q * args.ldo) + col;
          *dst = args.probs[q] * acc[i][j][v];
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
