// Per-expert weight gradients with a short reduction:
//
//   dW[e] (M x N, row-major) = sum over the expert's pairs q of a_q^T b_q,
//
// a_q (M values) and b_q (N values) rows of pair-row buffers as stored
// (K-major operands: the reduction runs over rows): a_q = row off_e + q of
// `a` at column offset 0, b_q = row off_e + q of `b`, or, gathered, the
// token's row order[off_e + q] / top_k.  K_e = counts[e] <= 192 pairs,
// padded to a multiple of 64 (the padded rows of the A strip are zeroed in
// LDS; those of B repeat its last pair row, finite, multiplied by zero).  M
// is a multiple of 256 and N of 64; 16-bit operands (a bf16 b is widened to
// fp16 in registers), fp32 accumulation.
//
// A general GEMM tile spends most of its life waiting for its few K steps'
// operands.  Here one workgroup (4 waves, one per 64-row quarter) owns an
// expert's 256-row strip of M: the strip passes through LDS into registers
// once (the A fragments of every K step, at most 96 VGPRs per lane; two
// 128-row halves in turn), then the workgroup sweeps all N / 64 column tiles.
// Two LDS buffers alternate for the B tiles: tile t+1 streams in (LDS-DMA)
// while tile t is multiplied, staged in a third buffer and written back as
// 128-byte row pieces.  At 80 KB of LDS two workgroups share a compute unit,
// so one's stores can run while the other multiplies; each reads a B tile
// once per 32 KB of output.
//
// LDS images of the operands hold K-row k (one pair row's 128 strip columns
// or 64 tile columns) at k * ROWK, 16-byte chunks XOR-swizzled per K-row;
// MFMA fragments come out through gfx950's transposing LDS read
// ds_read_b64_tr_b16: within each 16-lane group, lanes 4j..4j+3 name 4
// consecutive values of K-row j and lane i receives column i of the 4 rows.
#pragma once

#include "lmoe_common.h"

namespace lmoe {

constexpr int kWgradKMax = 192;    // largest K_e this kernel takes
constexpr int kWgradTile = 64;     // columns of an output tile (of a B tile's K-rows)
constexpr int kWgradStrip = 256;   // rows of an output tile (columns of the A strip)
constexpr int kWgradHalf = 128;    // strip columns per A image (the strip passes in two halves)
constexpr int kWgradBuf = kWgradTile * kWgradKMax * 2;     // one B tile (24 KB)
constexpr int kWgradStage = kWgradStrip * kWgradTile * 2;  // one staged output tile (32 KB)
constexpr int kWgradLds = 2 * kWgradBuf + kWgradStage;    // 80 KB: two workgroups per CU
static_assert(kWgradHalf * kWgradKMax * 2 <= 2 * kWgradBuf, "an A half image fits the two B buffers");
constexpr int kWgradWaves = 4;
constexpr int kWgradThreads = 64 * kWgradWaves;

typedef __attribute__((address_space(3))) void wg_lds_void_t;

// gfx9 s_waitcnt immediates (expcnt / the counter not named left at "no wait")
constexpr int wg_vmcnt(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int wg_lgkm0() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Byte of value (K-row r, column n) in an operand image of ROWK bytes per
// K-row.  The swizzle makes a transposing read, which takes 64 bytes from each
// of K-rows 0-3 and 8-11 of a 16-row group, hit distinct banks.
// For 256-byte K-rows (16 chunks) the 8 K-rows of one read (0-3 and 8-11 of a
// 16-row group, 64 bytes each) start at chunks 0, 4, 8, 12 (+16 for 8-11: the
// same banks a row later, in the read's other half); for 128-byte K-rows (8
// chunks, two K-rows per 256-byte bank row) K-rows 2 and 3 of each 4 move by
// 64 bytes, so K-rows 0-3 cover the 64 banks once.
template <int ROWK>
__device__ __forceinline__ int wk_sw(int r) {
  if constexpr (ROWK == 128) return 4 * ((r >> 1) & 1);
  else return (4 * (r & 3) + 16 * ((r >> 3) & 1)) & (ROWK / 16 - 1);
}
template <int ROWK>
__device__ __forceinline__ int wk_pos(int r, int n) { return r * ROWK + (((n >> 3) ^ wk_sw<ROWK>(r)) << 4) + (n & 7) * 2; }

// Two MFMA fragments (32 columns x 16 K each) from an operand image:
// lane l = 16 g + q reads 4 columns of K-row rb (rb = 8 (g / 2) + q / 4) at
// LDS byte p (K-rows 0-3 / 8-11) and p + 4 ROWK (K-rows 4-7 / 12-15); the
// transposing read hands it column l % 32 of K values 8 (l / 32) .. + 7.
// The reads wait for themselves (lgkmcnt 0) in the same asm block: through
// the builtin, which carries no alias information, the compiler would wait
// for every LDS-DMA and store in flight first.
template <int ROWK, int OFF>
__device__ __forceinline__ void wk_read2(uint32_t p0, uint32_t p1, u32x4& f0, u32x4& f1) {
  u32x2 r00, r01, r10, r11;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r00), "=&v"(r01), "=&v"(r10), "=&v"(r11)
      : "v"(p0), "v"(p1), "i"(OFF), "i"(OFF + 4 * ROWK));
  f0 = u32x4{r00[0], r00[1], r01[0], r01[1]};
  f1 = u32x4{r10[0], r10[1], r11[0], r11[1]};
}

// Staged output tile: 256 rows of 128 bytes, 16-byte chunk c of row r at
// chunk c ^ (r % 8).
__device__ __forceinline__ int wg_spos(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Operand rows of one expert: row k (< cnt) at base + row(k) * ld bytes,
// row(k) = off + k, or order[off + k] / top_k when gathered.
struct WgRows {
  const char* base;
  int64_t ld;
  const int32_t* order;  // NULL: rows in sorted pair order
  int top_k;
  __device__ __forceinline__ const char* row(int off, int k) const {
    const int64_t r = order ? (int64_t)(order[off + k] / top_k) : (int64_t)(off + k);
    return base + r * ld;
  }
};

template <typename TB, typename TO, int KG>
__device__ __forceinline__ void wgrad_strip(const WgRows A, const WgRows B, int off, int cnt, int m0, int N,
                                            char* out, int64_t ldo, char* smem) {
  constexpr int NWAVE = kWgradWaves, NTHR = kWgradThreads;
  constexpr int KS = 2 * KG;              // MFMA K steps of 16
  constexpr int KP = 32 * KG;             // padded K (pair rows)
  constexpr int kDma = KG * (4 / NWAVE);  // DMA instructions per wave for a B tile (an A half image: 2 kDma)
  constexpr int ROWA = 2 * kWgradHalf, ROWB = 2 * kWgradTile;  // bytes per K-row of the images
  constexpr bool kWidenB = __is_same(TB, bf16_t);
  // (the wave index is uniform: readfirstlane keeps the DMA destinations scalar)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave wm owns rows wm * 64 .. + 64 of the strip and all 64 columns of a tile
  const int wm = wave;
  const int NT = N / kWgradTile;
  auto bbuf = [&](int t) { return smem + (t & 1) * kWgradBuf; };  // column tile t's B buffer
  char* const S = smem + 2 * kWgradBuf;                           // staged output tile
  char* const Aimg = smem;  // an A half image: KP K-rows of 256 bytes over both B buffers
  typedef __attribute__((address_space(3))) const char* lds_cptr;
  auto lds_addr = [](const char* p) -> uint32_t { return (uint32_t)(size_t)(lds_cptr)p; };

  // DMA plan.  Instruction i of an image fills its bytes [1024 i, +1024):
  // lane l lands at byte 16 l, i.e. K-row (1024 i + 16 l) / ROWK and physical
  // chunk (16 l % ROWK) / 16, and fetches the logical chunk swizzled there.
  // K-rows past the expert's pairs reload its last pair row.  Wave w issues
  // instructions w, w + 4, ...
  // B tile: K-row 8 i + l / 8; its swizzle depends on (l / 16) % 2 only.
  const int bchunk = ((lane & 7) ^ (4 * ((lane >> 4) & 1))) * 16;
  const char* brow[kDma];
#pragma unroll
  for (int ii = 0; ii < kDma; ++ii) brow[ii] = B.row(off, min(8 * (wave + NWAVE * ii) + (lane >> 3), cnt - 1)) + bchunk;
  auto dma_b = [&](int t, char* buf) {
#pragma unroll
    for (int ii = 0; ii < kDma; ++ii)
      __builtin_amdgcn_global_load_lds((const void*)(brow[ii] + (int64_t)t * (kWgradTile * 2)),
                                       (wg_lds_void_t*)(buf + (wave + NWAVE * ii) * 1024), 16, 0, 0);
  };
  // fragment addresses: K-row rb of columns c0 + 16 (g % 2) + 4 (q % 4) (the
  // swizzle of K-row 16 s + rb (+ 4) equals that of rb)
  const int rb = 8 * (lane >> 5) + ((lane >> 2) & 3);
  const int cl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // The A strip in two halves of 128 columns (K-row 4 i + l / 16 of a half
  // image; its swizzle depends on (l / 16) % 4 only): each half is loaded,
  // its padded K-rows zeroed (they multiply the repeated B rows), and the
  // two waves whose rows it holds read their fragments into registers.
  u32x4 fa[KS][2];
  const int achunk = (lane & 15) ^ (4 * ((lane >> 4) & 3));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2 * kDma; ++ii) {
      const int inst = wave + NWAVE * ii, r = 4 * inst + (lane >> 4);
      const char* src = A.row(off, min(r, cnt - 1)) + (int64_t)(m0 + kWgradHalf * h + 8 * achunk) * 2;
      __builtin_amdgcn_global_load_lds((const void*)src, (wg_lds_void_t*)(Aimg + inst * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(wg_vmcnt(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int id = tid; id < (KP - cnt) * (ROWA / 16); id += NTHR) *(u32x4*)(Aimg + cnt * ROWA + id * 16) = z;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wg_lgkm0());
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if ((wm >> 1) == h) {  // uniform per wave
      const uint32_t a0 = lds_addr(Aimg + wk_pos<ROWA>(rb, (wm & 1) * 64 + cl));
      const uint32_t a1 = lds_addr(Aimg + wk_pos<ROWA>(rb, (wm & 1) * 64 + 32 + cl));
#pragma unroll
      for (int s = 0; s < KS; ++s) wk_read2<ROWA, 0>(a0 + s * 16 * ROWA, a1 + s * 16 * ROWA, fa[s][0], fa[s][1]);
    }
    // every wave is done with this half image before the next DMA overwrites it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  dma_b(0, bbuf(0));
  const uint32_t b0 = lds_addr(smem + wk_pos<ROWB>(rb, cl));
  const uint32_t b1 = lds_addr(smem + wk_pos<ROWB>(rb, 32 + cl));

  // The MFMAs take the B fragment first, so each 32 x 32 accumulator holds
  // the transposed sub-tile: lane l has output row l % 32 and columns
  // 8 (v / 4) + 4 (l / 32) + v % 4, i.e. four runs of four consecutive
  // columns, each staged with one 8-byte LDS write.
  const int lr = lane & 31, lh = lane >> 5;
  constexpr int kStores = kWgradStrip * (kWgradTile * 2) / 16 / NTHR;  // 16-byte stores per thread per tile
  for (int t = 0; t < NT; ++t) {
    const uint32_t bofs = (t & 1) * kWgradBuf;
    // B tile t has landed (issued after it: the stores of tile t-1, none
    // before tile 0), and every wave is done reading the staged tile t-1 and
    // B tile t-1: B tile t+1 may stream into the other buffer and tile t may
    // be staged
    if (t == 0) __builtin_amdgcn_s_waitcnt(wg_vmcnt(0) & wg_lgkm0());
    else __builtin_amdgcn_s_waitcnt(wg_vmcnt(kStores) & wg_lgkm0());
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 1 < NT) dma_b(t + 1, bbuf(t + 1));
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // step s's MFMAs are issued before step s + 1's fragment reads, whose
    // wait then overlaps them
    u32x4 fb[2][2];
    auto read_b = [&](auto s_c, u32x4* f) {
      constexpr int s = decltype(s_c)::value;
      wk_read2<ROWB, s * 16 * ROWB>(b0 + bofs, b1 + bofs, f[0], f[1]);
      if constexpr (kWidenB) {
        f[0] = bf16x8_to_f16x8(f[0]);
        f[1] = bf16x8_to_f16x8(f[1]);
      }
    };
    read_b(IntC<0>{}, fb[0]);
    sfor<KS>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fb[s & 1][j]),
                                                             __builtin_bit_cast(f16x8, fa[s][i]), acc[i][j], 0, 0, 0);
      if constexpr (s + 1 < KS) {
        __builtin_amdgcn_sched_barrier(0);
        read_b(IntC<s + 1>{}, fb[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // columns j*32 + 8q + 4lh + (0..3): bytes 8 lh.. of chunk j*4 + q
          TO four[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) Elem<TO>::store(&four[u], acc[i][j][4 * q + u]);
          u32x2 w;
          __builtin_memcpy(&w, four, 8);
          *(u32x2*)(S + wg_spos(row, j * 4 + q) + 8 * lh) = w;
        }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wg_lgkm0());
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    char* otile = out + (int64_t)t * kWgradTile * 2;
#pragma unroll
    for (int q = 0; q < kStores; ++q) {
      const int id = q * NTHR + tid, row = id >> 3, c = id & 7;
      *(u32x4*)(otile + row * ldo + c * 16) = *(const u32x4*)(S + wg_spos(row, c));
    }
  }
  // no LDS-DMA may still be writing when the workgroup's LDS is handed on
  __builtin_amdgcn_s_waitcnt(wg_vmcnt(0));
}

// dW[e] = A_e^T B_e for every expert e (grid: experts x M / 256 strips).
// a: pair rows of M values (row stride lda bytes), b: rows of N values (ldb
// bytes), gathered through b_order / top_k when b_order is not NULL.
template <typename TA, typename TB, typename TO>
__global__ __launch_bounds__(kWgradThreads, 2) void wgrad_kernel(const TA* __restrict__ a, int64_t lda,
                                                    const TB* __restrict__ b, int64_t ldb,
                                                    const int32_t* __restrict__ b_order, int top_k,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets, int M, int N,
                                                    TO* __restrict__ out) {
  static_assert(__is_same(TA, f16_t) && sizeof(TB) == 2 && sizeof(TO) == 2, "fp16 A, 16-bit B and output");
  __shared__ __attribute__((aligned(1024))) char smem[kWgradLds];
  const int strips = M / kWgradStrip;
  // the strips of one expert are neighbours on one XCD: they share B_e in its L2
  const int L = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int e = L / strips, ms = L % strips;
  const int cnt = counts[e], off = offsets[e];
  const int64_t ldo = (int64_t)N * 2;
  char* o = (char*)(out + ((int64_t)e * M + (int64_t)ms * kWgradStrip) * N);
  const WgRows A{(const char*)a, lda, nullptr, 1};
  const WgRows B{(const char*)b, ldb, b_order, top_k};
  const int m0 = ms * kWgradStrip;
  switch ((cnt + 63) / 64) {
    case 1: wgrad_strip<TB, TO, 2>(A, B, off, cnt, m0, N, o, ldo, smem); break;
    case 2: wgrad_strip<TB, TO, 4>(A, B, off, cnt, m0, N, o, ldo, smem); break;
    case 3: wgrad_strip<TB, TO, 6>(A, B, off, cnt, m0, N, o, ldo, smem); break;
    default: {  // no pairs: a zero gradient (more than kWgradKMax never reaches here)
      const u32x4 z = {0u, 0u, 0u, 0u};
      const int chunks = N / 8;  // 16-byte chunks per row
      for (int id = threadIdx.x; id < kWgradStrip * chunks; id += kWgradThreads)
        *(u32x4*)(o + (int64_t)(id / chunks) * ldo + (id % chunks) * 16) = z;
    }
  }
}

}  // namespace lmoe
