// Element-wise, reduction and layout kernels of the routed-block backward.
// The matrix products run on the GEMM family (gemm_kernel.h).
#pragma once

#include "lmoe_common.h"

namespace lmoe {
// Internal linkage: every translation unit that launches these kernels
// carries its own copy.
namespace {

// Zero n 4-byte words.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Batched transpose through a 64 x 64 LDS tile: out[b][c][col0 + r] = in[b][r][c]
// for r < rows, c < cols (leading dimensions in elements).  Batches with
// counts[b] == 0 are skipped when counts is given.  Grid: (ceil(cols/64),
// ceil(rows/64), batches), 256 threads.
template <typename T>
__global__ __launch_bounds__(256) void transpose_batched_kernel(const T* __restrict__ in, int64_t in_bstride,
                                                                int ld_in, int rows, int cols,
                                                                T* __restrict__ out, int64_t out_bstride,
                                                                int ld_out, int col0,
                                                                const int32_t* __restrict__ counts) {
  const int b = blockIdx.z;
  if (counts && counts[b] == 0) return;
  __shared__ T tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const T* src = in + (int64_t)b * in_bstride;
  T* dst = out + (int64_t)b * out_bstride;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(int64_t)r * ld_in + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(int64_t)c * ld_out + col0 + r] = tile[tx][i];
  }
}

// The same transpose for 16-bit elements with 16-byte global accesses: a
// 64 x 64 tile is read as 8-element row chunks and written as 8-element
// column chunks.  rows, cols, ld_in, ld_out and col0 are multiples of 8 and
// the buffers 16-byte aligned.
__global__ __launch_bounds__(256) void transpose16_batched_kernel(const uint16_t* __restrict__ in,
                                                                  int64_t in_bstride, int ld_in, int rows,
                                                                  int cols, uint16_t* __restrict__ out,
                                                                  int64_t out_bstride, int ld_out, int col0,
                                                                  const int32_t* __restrict__ counts) {
  const int b = blockIdx.z;
  if (counts && counts[b] == 0) return;
  constexpr int LD = 72;  // padded row of the LDS tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LD];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const uint16_t* src = in + (int64_t)b * in_bstride;
  uint16_t* dst = out + (int64_t)b * out_bstride;
  const int t = threadIdx.x, q = t & 7;
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 64 rows x 8 chunks
    const int r = (t >> 3) + 32 * i;
    if (r0 + r < rows && c0 + q * 8 < cols)
      *(u32x4*)(tile + r * LD + q * 8) = *(const u32x4*)(src + (int64_t)(r0 + r) * ld_in + c0 + q * 8);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 64 output rows (columns c) x 8 chunks of 8 r
    const int c = (t >> 3) + 32 * i;
    if (c0 + c >= cols || r0 + q * 8 >= rows) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[(q * 8 + 2 * j) * LD + c] | ((uint32_t)tile[(q * 8 + 2 * j + 1) * LD + c] << 16);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(dst + (int64_t)(c0 + c) * ld_out + col0 + r0 + q * 8) = v;
  }
}

// Per-expert padded K ranges of the weight-gradient products:
// kr_len[e] = counts[e] rounded up to 64, kr_off[e] = sum of kr_len[e'] for e' < e.
// One workgroup of 1024 threads; R <= 4096.
__global__ __launch_bounds__(1024) void padded_ranges_kernel(const int32_t* __restrict__ counts, int R,
                                                             int32_t* __restrict__ kr_off,
                                                             int32_t* __restrict__ kr_len) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int per = (R + 1023) / 1024;
  const int e0 = t * per, e1 = min(R, e0 + per);
  int32_t s = 0;
  for (int e = e0; e < e1; ++e) s += (counts[e] + 63) & ~63;
  part[t] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan of the partial sums
    const int32_t v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = part[t] - s;
  for (int e = e0; e < e1; ++e) {
    const int32_t len = (counts[e] + 63) & ~63;
    kr_off[e] = run;
    kr_len[e] = len;
    run += len;
  }
}

// Expert-segment transpose with zero padding: for expert e (blockIdx.z) and
// segment row r < kr_len[e] (pairs of e in sorted order, r >= counts[e] pad),
// expert e's block of out is row-major [ncols, kr_len[e]] at element
// kr_off[e] * ncols:
//   block[c * kr_len[e] + r] = r < counts[e] ? src_row(e, r)[col_off + c] : 0
// src_row(e, r) = src + row * ld_src with row = offsets[e] + r (sorted rows)
// or, when order is given, row = order[offsets[e] + r] / top_k (token rows).
// Grid: (ceil(ncols/64), ceil(max_len/64), R), 256 threads.
template <typename TS, typename TD>
__global__ __launch_bounds__(256) void segment_transpose_kernel(
    const TS* __restrict__ src, int64_t ld_src, int col_off, int ncols, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ order, int top_k,
    const int32_t* __restrict__ kr_off, const int32_t* __restrict__ kr_len, TD* __restrict__ out) {
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (r0 >= kr_len[e]) return;
  __shared__ float tile[64][65];
  const int cnt = counts[e];
  const int64_t base = offsets[e];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    float v = 0.f;
    if (r < cnt && c < ncols) {
      const int64_t row = order ? (int64_t)(order[base + r] / top_k) : base + r;
      v = Elem<TS>::load(src + row * ld_src + col_off + c);
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  const int64_t ld = kr_len[e];
  TD* blk = out + (int64_t)kr_off[e] * ncols;
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < ncols) Elem<TD>::store(blk + (int64_t)c * ld + r, tile[tx][i]);
  }
}

// The same segment transpose for 16-bit elements with 16-byte global accesses
// (TS -> TD converted as the tile is loaded): the 64 x 64 tile is read as
// 8-element chunks of its source rows and written as 8-element chunks of the
// block's rows.  ncols, col_off and ld_src are multiples of 8, the buffers
// 16-byte aligned (kr_len and kr_off are multiples of 64).
template <typename TS, typename TD>
__global__ __launch_bounds__(256) void segment_transpose16_kernel(
    const TS* __restrict__ src, int64_t ld_src, int col_off, int ncols, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ order, int top_k,
    const int32_t* __restrict__ kr_off, const int32_t* __restrict__ kr_len, TD* __restrict__ out) {
  static_assert(sizeof(TS) == 2 && sizeof(TD) == 2, "16-bit elements");
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (r0 >= kr_len[e]) return;
  constexpr int LD = 72;  // padded row of the LDS tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LD];
  const int cnt = counts[e];
  const int64_t base = offsets[e];
  const int t = threadIdx.x, q = t & 7;
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 64 segment rows x 8 chunks of 8 columns
    const int r = (t >> 3) + 32 * i, c = c0 + q * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + r < cnt && c < ncols) {
      const int64_t row = order ? (int64_t)(order[base + r0 + r] / top_k) : base + r0 + r;
      v = *(const u32x4*)(src + row * ld_src + col_off + c);
      if constexpr (!__is_same(TS, TD)) {
        const TS* in = (const TS*)&v;
        TD cv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) Elem<TD>::store(cv + j, Elem<TS>::load(in + j));
        v = *(const u32x4*)cv;
      }
    }
    *(u32x4*)(tile + r * LD + q * 8) = v;
  }
  __syncthreads();
  const int64_t ld = kr_len[e];
  TD* blk = out + (int64_t)kr_off[e] * ncols;
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 64 block rows (columns c) x 8 chunks of 8 segment rows
    const int c = (t >> 3) + 32 * i;
    if (c0 + c >= ncols) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[(q * 8 + 2 * j) * LD + c] | ((uint32_t)tile[(q * 8 + 2 * j + 1) * LD + c] << 16);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(blk + (int64_t)(c0 + c) * ld + r0 + q * 8) = v;
  }
}

// Pair gradients from v = W_o^T du (the product of du's row with the pair's
// W_o, one row per sorted pair q', q = order[q'], token n = q / k):
//   dprobs[q] = <v[q'], h[q']>  (= <du[n], W_o h[q']>, the pair's output o
//   never formed),  dout[q'] = probs[q] * du[n]  (for dW_o),  sp[q'] = probs[q].
// The gradient of the hidden is dh = p v, applied by the SiTU backward.
template <typename TD>
__global__ __launch_bounds__(256) void pair_vh_kernel(const float* __restrict__ v, const TD* __restrict__ h,
                                                      const float* __restrict__ du, const float* __restrict__ probs,
                                                      const int32_t* __restrict__ order, int top_k, int ell, int f,
                                                      float* __restrict__ dprobs, TD* __restrict__ dout,
                                                      float* __restrict__ sp) {
  const int64_t qs = blockIdx.x;
  const int32_t q = order[qs];
  const float pq = probs[q];
  const float* vrow = v + qs * f;
  const TD* hrow = h + qs * f;
  const float* dur = du + (int64_t)(q / top_k) * ell;
  TD* drow = dout + qs * ell;
  float acc = 0.f;
  // uniform: four values per thread and access (rows stay aligned; v, h and
  // dout are workspace buffers, du the caller's)
  if ((f & 3) == 0 && (ell & 3) == 0 && (((uintptr_t)du) & 15) == 0) {
    for (int c = 4 * (int)threadIdx.x; c < f; c += 4 * 256) {
      const f32x4 vv = *(const f32x4*)(vrow + c);
      TD hv[4];
      if constexpr (sizeof(TD) == 2) {
        const u32x2 w = *(const u32x2*)(hrow + c);
        __builtin_memcpy(hv, &w, 8);
      } else {
        const f32x4 w = *(const f32x4*)(hrow + c);
        __builtin_memcpy(hv, &w, 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += vv[j] * Elem<TD>::load(&hv[j]);
    }
    for (int c = 4 * (int)threadIdx.x; c < ell; c += 4 * 256) {
      const f32x4 dv = *(const f32x4*)(dur + c);
      TD ov[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) Elem<TD>::store(&ov[j], pq * dv[j]);
      if constexpr (sizeof(TD) == 2) {
        u32x2 w;
        __builtin_memcpy(&w, ov, 8);
        *(u32x2*)(drow + c) = w;
      } else {
        f32x4 w;
        __builtin_memcpy(&w, ov, 16);
        *(f32x4*)(drow + c) = w;
      }
    }
  } else {
    for (int c = threadIdx.x; c < f; c += 256) acc += vrow[c] * Elem<TD>::load(hrow + c);
    for (int c = threadIdx.x; c < ell; c += 256) Elem<TD>::store(drow + c, pq * dur[c]);
  }
  __shared__ float red[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    dprobs[q] = (red[0] + red[1]) + (red[2] + red[3]);
    sp[qs] = pq;
  }
}

// Elementwise fp32 -> TD (n values).
template <typename TD>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ in, int64_t n, TD* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    Elem<TD>::store(out + i, in[i]);
}

// SiTU-GLU backward through the hidden: with G(a) = b1 tanh(a/b1) sigmoid(a)
// and U(a) = b2 tanh(a/b2),
//   dg = dh * G'(g) U(u),  du = dh * G(g) U'(u)
//   G'(a) = (1 - tanh(a/b1)^2) sigmoid(a) + b1 tanh(a/b1) sigmoid(a) (1 - sigmoid(a)),
//   U'(a) = 1 - tanh(a/b2)^2.
// Row q of dgu (leading dimension ld, starting at column col0) holds
// [dg | du] (f columns each) for row q of the rows x f pre-activations; with
// row_scale, row q's dh is multiplied by row_scale[q] first.
// Workgroups stride over rows and threads over columns (no index division);
// tanh and sigma from the hardware exp and reciprocal (absolute error ~1e-7).
// TP: type of the stored pre-activations (read as fp32).
template <typename TP, typename TD>
__global__ __launch_bounds__(256) void situ_backward_kernel(const float* __restrict__ dh, const TP* __restrict__ g,
                                                            const TP* __restrict__ u, int64_t rows, int f,
                                                            float beta1, float beta2, TD* __restrict__ dgu,
                                                            int64_t ld, int64_t col0,
                                                            const float* __restrict__ row_scale) {
  const float ib1 = 1.0f / beta1, ib2 = 1.0f / beta2;
  for (int64_t q = blockIdx.x; q < rows; q += gridDim.x) {
    const TP* gq = g + q * f;
    const TP* uq = u + q * f;
    const float* dq = dh + q * f;
    const float rs = row_scale ? row_scale[q] : 1.0f;
    TD* out = dgu + q * ld + col0;
    for (int j = threadIdx.x; j < f; j += 256) {
      const float a = Elem<TP>::load(gq + j), b = Elem<TP>::load(uq + j), d = dq[j] * rs;
      const float tg = tanh_fast(a * ib1), tu = tanh_fast(b * ib2);
      const float sg = rcp_fast(1.0f + __expf(-a));
      const float gate = beta1 * tg * sg, up = beta2 * tu;
      const float dgate = (1.0f - tg * tg) * sg + beta1 * tg * sg * (1.0f - sg);
      const float dup = 1.0f - tu * tu;
      Elem<TD>::store(out + j, d * dgate * up);
      Elem<TD>::store(out + f + j, d * gate * dup);
    }
  }
}

// inv[order[q']] = q'
__global__ __launch_bounds__(256) void inverse_order_kernel(const int32_t* __restrict__ order, int64_t pairs,
                                                            int32_t* __restrict__ inv) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < pairs) inv[order[i]] = (int32_t)i;
}

// dz[n] (row stride ld) = sum over slots j (in slot order) of rows[inv[n k + j]]
// (rows of type TS, summed in fp32), one workgroup per token; top_k <= 64.
// Four-element row loads where rows and ell allow them.
template <typename TS, typename TD>
__global__ __launch_bounds__(256) void pair_sum_kernel(const TS* __restrict__ rows, const int32_t* __restrict__ inv,
                                                       int top_k, int ell, TD* __restrict__ dz, int64_t ld) {
  const int64_t n = blockIdx.x;
  __shared__ int64_t src[64];  // first element of each slot's row
  if ((int)threadIdx.x < top_k) src[threadIdx.x] = (int64_t)inv[n * top_k + threadIdx.x] * ell;
  __syncthreads();
  TD* out = dz + n * ld;
  if ((((uintptr_t)rows) & (4 * sizeof(TS) - 1)) == 0 && (ell & 3) == 0) {  // uniform
    for (int c = 4 * (int)threadIdx.x; c < ell; c += 4 * 256) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int j = 0; j < top_k; ++j) {
        const TS* p = rows + src[j] + c;
        f32x4 v;
        if constexpr (sizeof(TS) == 4) {
          v = *(const f32x4*)p;
        } else {
          TS t4[4];
          *(u32x2*)t4 = *(const u32x2*)p;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = Elem<TS>::load(t4 + q);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += v[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) Elem<TD>::store(out + c + q, acc[q]);
    }
  } else {
    for (int c = threadIdx.x; c < ell; c += 256) {
      float acc = 0.f;
      for (int j = 0; j < top_k; ++j) acc += Elem<TS>::load(rows + src[j] + c);
      Elem<TD>::store(out + c, acc);
    }
  }
}

// RMSNorm backward, one workgroup per token (r = w u rho, rho = (mean(u^2) + eps)^(-1/2);
// w NULL = ones):
//   du_j = w_j dr_j rho - rho^3 u_j / l * sum_i dr_i w_i u_i ;  rho_out[n] = rho
__global__ __launch_bounds__(256) void rmsnorm_backward_kernel(const float* __restrict__ u, const float* __restrict__ dr,
                                                               const float* __restrict__ w, int ell, float eps,
                                                               float* __restrict__ du, float* __restrict__ rho_out) {
  const int64_t n = blockIdx.x;
  const float* ur = u + n * ell;
  const float* dr_r = dr + n * ell;
  float ss = 0.f, dot = 0.f;
  for (int c = threadIdx.x; c < ell; c += 256) {
    const float v = ur[c];
    ss += v * v;
    dot += dr_r[c] * (w ? w[c] : 1.f) * v;
  }
  __shared__ float red[2][4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off);
    dot += __shfl_xor(dot, off);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = ss;
    red[1][threadIdx.x >> 6] = dot;
  }
  __syncthreads();
  ss = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  dot = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const float rho = 1.0f / sqrtf(ss / ell + eps);
  const float c3 = rho * rho * rho * dot / ell;
  for (int c = threadIdx.x; c < ell; c += 256) du[n * ell + c] = (w ? w[c] : 1.f) * dr_r[c] * rho - c3 * ur[c];
  if (threadIdx.x == 0) rho_out[n] = rho;
}

// dw[c] = sum over tokens n of dr[n, c] u[n, c] rho[n], in two passes with a
// fixed order: pass 1 sums chunks of `chunk` tokens into part[chunk index, c]
// (grid: column blocks x chunks), pass 2 adds the chunks in order.
constexpr int kWgradChunk = 64;  // tokens per chunk (more past 65535 chunks)
__global__ __launch_bounds__(256) void rmsnorm_wgrad_partial_kernel(const float* __restrict__ u,
                                                                    const float* __restrict__ dr,
                                                                    const float* __restrict__ rho, int64_t N,
                                                                    int64_t chunk, int ell,
                                                                    float* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ell) return;
  const int64_t n0 = (int64_t)blockIdx.y * chunk;
  const int64_t n1 = n0 + chunk < N ? n0 + chunk : N;
  float acc = 0.f;
  for (int64_t n = n0; n < n1; ++n) acc += dr[n * ell + c] * u[n * ell + c] * rho[n];
  part[(int64_t)blockIdx.y * ell + c] = acc;
}

__global__ __launch_bounds__(256) void rmsnorm_wgrad_final_kernel(const float* __restrict__ part, int nchunks,
                                                                  int ell, float* __restrict__ dw) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ell) return;
  float acc = 0.f;
  for (int i = 0; i < nchunks; ++i) acc += part[(int64_t)i * ell + c];
  dw[c] = acc;
}

// Router backward, one wave per token: with s = sigmoid(logits) at the token's
// k selected experts, S = sum s and p = s / S,
//   ds_i = dp_i / S - (sum_j dp_j s_j) / S^2   (ds = dp / 1e-9 under the clamp S < 1e-9)
//   dl_i = ds_i s_i (1 - s_i)
// The dl row (leading dimension ld, R columns plus zero padding up to rpad) is
// zero except at the selected experts.
template <typename TD>
__global__ __launch_bounds__(256) void router_backward_kernel(const float* __restrict__ logits,
                                                              const int32_t* __restrict__ ids,
                                                              const float* __restrict__ dprobs, int64_t N, int R,
                                                              int k, int rpad, TD* __restrict__ dl, int64_t ld) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  TD* row = dl + n * ld;
  float s = 0.f, dp = 0.f;
  int e = 0;
  if (lane < k) {
    e = ids[n * k + lane];
    s = 1.0f / (1.0f + expf(-logits[n * R + e]));
    dp = dprobs[n * k + lane];
  }
  float S = s, dot = dp * s;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S += __shfl_xor(S, off);
    dot += __shfl_xor(dot, off);
  }
  const float Sc = fmaxf(S, 1e-9f);
  const float ds = dp / Sc - (S >= 1e-9f ? dot / (Sc * Sc) : 0.f);
  const float g = lane < k ? ds * s * (1.0f - s) : 0.f;
  // every column written once: the selected experts' dl, zero elsewhere
  for (int c0 = 0; c0 < rpad; c0 += 64) {
    const int c = c0 + lane;
    float v = 0.f;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e, j);
      const float gj = __shfl(g, j);
      if (ej == c) v = gj;
    }
    if (c < rpad) Elem<TD>::store(row + c, v);
  }
}

// Four ints into device memory (parameters of a one-segment transpose).
__global__ void set_ints_kernel(int32_t* __restrict__ p, int32_t a, int32_t b, int32_t c, int32_t d) {
  if (threadIdx.x == 0) {
    p[0] = a;
    p[1] = b;
    p[2] = c;
    p[3] = d;
  }
}

}  // namespace
}  // namespace lmoe
