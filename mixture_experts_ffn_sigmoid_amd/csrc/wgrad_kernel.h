// Per-expert weight gradients with a short reduction:
//
//   dW[e] (M x N, row-major) = A_e B_e^T,
//
// A_e the row-major [M, K_e] block at element kr_off[e] * M of `a`, B_e the
// [N, K_e] block at kr_off[e] * N of `b`, K_e = kr_len[e] in {0, 64, 128, 192}
// (an expert's pairs, zero-padded to a multiple of 64).  M is a multiple of
// 256 and N of 128; 16-bit operands, fp32 accumulation.
//
// A general GEMM tile spends most of its life waiting for its few K steps'
// operands.  Here one workgroup (8 waves, 4 x 2) owns an expert's 256-row
// strip of M: the strip passes through LDS into registers once (the A
// fragments of every K step, at most 96 VGPRs per lane), then the workgroup
// sweeps all N / 128 column tiles.  Two LDS buffers alternate for the B tiles:
// tile t+1 streams in (LDS-DMA) while tile t is multiplied, staged in a third
// buffer and written back as 16-byte row chunks.  The loads of a CU queue with
// its stores; a 256-row strip reads each B tile once per 64 KB of output.
#pragma once

#include "lmoe_common.h"

namespace lmoe {

constexpr int kWgradKMax = 192;    // largest K_e this kernel takes
constexpr int kWgradTile = 128;    // columns of an output tile, rows of a B tile
constexpr int kWgradStrip = 256;   // rows of an A strip and of an output tile
constexpr int kWgradBuf = kWgradTile * kWgradKMax * 2;     // one B tile (48 KB)
constexpr int kWgradStage = kWgradStrip * kWgradTile * 2;  // one staged output tile (64 KB)
constexpr int kWgradLds = 2 * kWgradBuf + kWgradStage;    // 160 KB: one workgroup per CU
constexpr int kWgradWaves = 8;
constexpr int kWgradThreads = 64 * kWgradWaves;

typedef __attribute__((address_space(3))) void wg_lds_void_t;

// gfx9 s_waitcnt immediates (expcnt / the counter not named left at "no wait")
constexpr int wg_vmcnt(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int wg_lgkm0() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// LDS operand layout: KG groups of 32 K values; group g holds the tile's 128
// rows x 64 bytes at g * 8 KB, row r's four 16-byte chunks XOR-swizzled by
// (r / 4) % 4 so that a fragment read of 32 consecutive rows hits every bank
// group evenly.
__device__ __forceinline__ int wg_pos(int g, int row, int chunk) {
  return g * (kWgradTile * 64) + row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// LDS-DMA of the [128, K] row slice at `blk` (row stride K elements) into an
// operand buffer.  Group g is 8 instructions of 1 KB; wave w of NWAVE issues
// instructions w, w + NWAVE, ...  Instruction i lands rows 16 i .. 16 i + 15:
// lane l takes row 16 i + l / 4 and the global chunk (l % 4) ^ ((l / 16) % 4),
// its row's swizzle, so one per-lane byte offset serves every instruction.
template <int KG, int NWAVE>
__device__ __forceinline__ void wg_dma(const char* blk, int K, char* buf, int wave, uint32_t lane_off) {
#pragma unroll
  for (int g = 0; g < KG; ++g) {
#pragma unroll
    for (int ii = 0; ii < 8 / NWAVE; ++ii) {
      const int inst = wave + NWAVE * ii;
      const char* src = blk + ((int64_t)inst * 16 * K * 2 + g * 64) + lane_off;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (wg_lds_void_t*)(buf + g * (kWgradTile * 64) + inst * 1024), 16, 0, 0);
    }
  }
}

// Staged output tile: 256 rows of 256 bytes, 16-byte chunk c of row r at
// chunk c ^ (r % 16).
__device__ __forceinline__ int wg_spos(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

template <typename TO, int KG>
__device__ __forceinline__ void wgrad_strip(const char* a_blk, const char* b_blk, int K, int N, char* out,
                                            int64_t ldo, char* smem) {
  constexpr int NWAVE = kWgradWaves, NTHR = kWgradThreads;
  constexpr int KS = 2 * KG;              // MFMA K steps of 16
  constexpr int kDma = KG * (8 / NWAVE);  // DMA instructions per wave per 128-row block
  // (the wave index is uniform: readfirstlane keeps the DMA destinations scalar)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves 4 (rows) x 2 (columns): 64 x 64 of the tile each
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
  const int NT = N / kWgradTile;
  auto bbuf = [&](int t) { return smem + (t & 1) * kWgradBuf; };  // column tile t's B buffer
  char* const S = smem + 2 * kWgradBuf;                           // staged output tile
  auto b_tile = [&](int t) { return b_blk + (int64_t)t * kWgradTile * K * 2; };
  const uint32_t lane_off = (uint32_t)((lane >> 2) * K * 2 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4));

  // the A strip's two 128-row blocks into B buffer 1 and the staging buffer
  // (contiguous), B tile 0 into B buffer 0; then the strip into registers
  wg_dma<KG, NWAVE>(a_blk, K, bbuf(1), wave, lane_off);
  wg_dma<KG, NWAVE>(a_blk + (int64_t)kWgradTile * K * 2, K, bbuf(1) + kWgradBuf, wave, lane_off);
  wg_dma<KG, NWAVE>(b_tile(0), K, bbuf(0), wave, lane_off);
  __builtin_amdgcn_s_waitcnt(wg_vmcnt(kDma));  // issued after the strip: B tile 0 only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  u32x4 fa[KS][2];
  {
    const char* Ab = bbuf(1) + (wm >> 1) * kWgradBuf;  // this wave's 64 rows lie in one block
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[s][i] = *(const u32x4*)(Ab + wg_pos(s >> 1, (wm & 1) * 64 + i * 32 + lr, 2 * (s & 1) + lh));
  }

  // The MFMAs take the B fragment first, so each 32 x 32 accumulator holds
  // the transposed sub-tile: lane l has output row lr and columns
  // 8 (v / 4) + 4 lh + v % 4, i.e. four runs of four consecutive columns,
  // each staged with one 8-byte LDS write.
  constexpr int kStores = kWgradStrip * 256 / 16 / NTHR;  // 16-byte stores per thread per tile
  for (int t = 0; t < NT; ++t) {
    const char* const B = bbuf(t);
    // B tile t has landed (issued after it: the stores of tile t-1, none
    // before tile 0), and every wave is done reading the A strip or the
    // staged tile t-1 and B tile t-1: B tile t+1 may stream into the other
    // buffer and tile t may be staged
    if (t == 0) __builtin_amdgcn_s_waitcnt(wg_vmcnt(0) & wg_lgkm0());
    else __builtin_amdgcn_s_waitcnt(wg_vmcnt(kStores) & wg_lgkm0());
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 1 < NT) wg_dma<KG, NWAVE>(b_tile(t + 1), K, bbuf(t + 1), wave, lane_off);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 fb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *(const u32x4*)(B + wg_pos(s >> 1, wn * 64 + j * 32 + lr, 2 * (s & 1) + lh));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fb[j]),
                                                             __builtin_bit_cast(f16x8, fa[s][i]), acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // columns wn*64 + j*32 + 8q + 4lh + (0..3): bytes 8 lh.. of chunk wn*8 + j*4 + q
          TO four[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) Elem<TO>::store(&four[u], acc[i][j][4 * q + u]);
          u32x2 w;
          __builtin_memcpy(&w, four, 8);
          *(u32x2*)(S + wg_spos(row, wn * 8 + j * 4 + q) + 8 * lh) = w;
        }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wg_lgkm0());
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    char* otile = out + (int64_t)t * kWgradTile * 2;
#pragma unroll
    for (int q = 0; q < kStores; ++q) {
      const int id = q * NTHR + tid, row = id >> 4, c = id & 15;
      *(u32x4*)(otile + row * ldo + c * 16) = *(const u32x4*)(S + wg_spos(row, c));
    }
  }
  // no LDS-DMA may still be writing when the workgroup's LDS is handed on
  __builtin_amdgcn_s_waitcnt(wg_vmcnt(0));
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kWgradThreads) void wgrad_kernel(const TI* __restrict__ a, const TI* __restrict__ b,
                                                    const int32_t* __restrict__ kr_off,
                                                    const int32_t* __restrict__ kr_len, int M, int N,
                                                    TO* __restrict__ out) {
  static_assert(sizeof(TI) == 2 && sizeof(TO) == 2, "16-bit operands and output");
  __shared__ __attribute__((aligned(1024))) char smem[kWgradLds];
  const int strips = M / kWgradStrip;
  // the strips of one expert are neighbours on one XCD: they share B_e in its L2
  const int L = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int e = L / strips, ms = L % strips;
  const int K = kr_len[e];
  const int64_t ldo = (int64_t)N * 2;
  char* o = (char*)(out + ((int64_t)e * M + (int64_t)ms * kWgradStrip) * N);
  const char* ab = (const char*)(a + (int64_t)kr_off[e] * M + (int64_t)ms * kWgradStrip * K);
  const char* bb = (const char*)(b + (int64_t)kr_off[e] * N);
  switch (K) {
    case 64: wgrad_strip<TO, 2>(ab, bb, K, N, o, ldo, smem); break;
    case 128: wgrad_strip<TO, 4>(ab, bb, K, N, o, ldo, smem); break;
    case 192: wgrad_strip<TO, 6>(ab, bb, K, N, o, ldo, smem); break;
    default: {  // no pairs: a zero gradient (K above the maximum never reaches here)
      const u32x4 z = {0u, 0u, 0u, 0u};
      const int chunks = N / 8;  // 16-byte chunks per row
      for (int id = threadIdx.x; id < kWgradStrip * chunks; id += kWgradThreads)
        *(u32x4*)(o + (int64_t)(id / chunks) * ldo + (id % chunks) * 16) = z;
    }
  }
}

}  // namespace lmoe
