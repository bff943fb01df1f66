// K3 sigmoid routing after the logits GEMM, and the permute-dispatch
// bookkeeping (histogram -> scan -> stable scatter) on the device.
#pragma once

#include "lmoe_common.h"

namespace lmoe {
// Internal linkage: every translation unit that launches these kernels
// carries its own copy.
namespace {

constexpr int kMaxRouted = 4096;
constexpr int kMaxTopK = 64;
constexpr int kDispatchChunk = 1024;  // pairs per histogram / scatter chunk

// ---------------------------------------------------------------------------
// One wave64 per token: s = sigmoid(l) over the R experts, k rounds of a
// wave-wide arg-max of v = s + b (larger v first, equal v -> lower id), then
// p_i = s_i / max(sum_T s, 1e-9).  v lives in LDS (R floats per wave), each
// lane keeps the best of its own experts so that a round rescans one lane.
// kSoftmax selects the legacy router instead: v = the raw logits, and the k
// winners are weighted by a softmax over their logits.
template <bool kSoftmax>
__global__ __launch_bounds__(256) void topk_route_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ bias, int64_t N,
                                                         int R, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ probs) {
  extern __shared__ float vbuf[];  // [4][R]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  if (n >= N) return;  // no block-level barrier below: waves are independent
  float* v = vbuf + wave * R;
  const float* lrow = logits + n * R;

  float best = -INFINITY;
  int best_id = 0x7fffffff;
#pragma unroll 8
  for (int e = lane; e < R; e += 64) {
    const float ve = kSoftmax ? lrow[e] : sigmoidf_(lrow[e]) + (bias ? bias[e] : 0.f);
    v[e] = ve;
    if (ve > best) {  // ascending e per lane: strict > keeps the lower id on ties
      best = ve;
      best_id = e;
    }
  }

  int my_id = 0;  // lane j keeps the j-th winner
  for (int j = 0; j < k; ++j) {
    float bv = best;
    int bi = best_id;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi >= R) bi = 0;  // only reachable with NaN scores; keeps every index in range
    if (lane == j) my_id = bi;
    if ((bi & 63) == lane) {  // owner lane removes the winner and rescans its experts
      v[bi] = -INFINITY;
      best = -INFINITY;
      best_id = 0x7fffffff;
#pragma unroll 8
      for (int e = lane; e < R; e += 64) {
        const float ve = v[e];
        if (ve > best) {
          best = ve;
          best_id = e;
        }
      }
    }
  }
  // weights of the k winners, lane j holding winner j: s_j (softmax: exp of the
  // logit minus the first winner's, the largest) over their sum, which is
  // reduced across the wave in a fixed order and taken from lane 0
  float w = 0.f;
  if (lane < k) w = kSoftmax ? lrow[my_id] : sigmoidf_(lrow[my_id]);
  if constexpr (kSoftmax) {
    const float lmax = __shfl(w, 0);
    w = lane < k ? expf(w - lmax) : 0.f;
  }
  float ssum = w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ssum += __shfl_xor(ssum, off);
  ssum = __shfl(ssum, 0);
  if (lane < k) {
    ids[n * k + lane] = my_id;
    probs[n * k + lane] = kSoftmax ? w / ssum : w / fmaxf(ssum, 1e-9f);
  }
}

// ---------------------------------------------------------------------------
// Router statistics for the Switch/GShard auxiliary loss and the router
// z-loss.  Pass 1, one workgroup per block of kLossTokens tokens:
//   colsum[blk, e] = sum over the block's tokens of sigmoid(l_te)
//   lse2[blk]      = sum over the block's tokens of (logsumexp_e l_te)^2
// (fixed summation order: deterministic).
constexpr int kLossTokens = 64;
__global__ __launch_bounds__(256) void router_stats_kernel(const float* __restrict__ logits, int64_t N,
                                                           int R, float* __restrict__ colsum,
                                                           float* __restrict__ lse2) {
  __shared__ float part[4];
  const int64_t t0 = (int64_t)blockIdx.x * kLossTokens;
  const int64_t t1 = min(t0 + kLossTokens, N);
  for (int e = threadIdx.x; e < R; e += 256) {
    float acc = 0.f;
    for (int64_t t = t0; t < t1; ++t) acc += sigmoidf_(logits[t * R + e]);
    colsum[(int64_t)blockIdx.x * R + e] = acc;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float wsum = 0.f;
  for (int64_t t = t0 + wave; t < t1; t += 4) {
    const float* l = logits + t * R;
    float m = -INFINITY;
    for (int e = lane; e < R; e += 64) m = fmaxf(m, l[e]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float se = 0.f;
    for (int e = lane; e < R; e += 64) se += expf(l[e] - m);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) se += __shfl_xor(se, off);
    const float lse = m + logf(se);
    wsum += lse * lse;  // wave-uniform
  }
  if (lane == 0) part[wave] = wsum;
  __syncthreads();
  if (threadIdx.x == 0) lse2[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

// Pass 2 (one workgroup; nblk may be 0): f_e = counts_e / max(sum counts, 1), P_e = colsum_e / N,
// out[0] = R * sum_e f_e P_e, out[1] = sum lse^2 / N.
__global__ __launch_bounds__(1024) void router_losses_kernel(const float* __restrict__ colsum,
                                                             const float* __restrict__ lse2, int nblk,
                                                             int64_t N, int R,
                                                             const int32_t* __restrict__ counts,
                                                             float* __restrict__ out) {
  __shared__ float red_a[1024], red_z[1024];
  __shared__ long long red_c[1024];
  const int t = threadIdx.x;
  float a = 0.f;
  long long c = 0;
  for (int e = t; e < R; e += 1024) {
    float pe = 0.f;
    for (int b = 0; b < nblk; ++b) pe += colsum[(int64_t)b * R + e];
    a += (float)counts[e] * pe;
    c += counts[e];
  }
  float z = 0.f;
  for (int b = t; b < nblk; b += 1024) z += lse2[b];
  red_a[t] = a;
  red_z[t] = z;
  red_c[t] = c;
  __syncthreads();
  for (int s = 512; s >= 1; s >>= 1) {
    if (t < s) {
      red_a[t] += red_a[t + s];
      red_z[t] += red_z[t + s];
      red_c[t] += red_c[t + s];
    }
    __syncthreads();
  }
  if (t == 0) {  // an empty batch has both losses 0
    const double tot = red_c[0] > 0 ? (double)red_c[0] : 1.0;
    const double n = N > 0 ? (double)N : 1.0;
    out[0] = (float)((double)R * (double)red_a[0] / (tot * n));
    out[1] = (float)((double)red_z[0] / n);
  }
}

// ---------------------------------------------------------------------------
// Dispatch step 1: per-chunk expert histogram of the flattened pair ids.
// Expert ids outside [0, R) are not counted; chunk_bad[chunk] records how many.
__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                            int64_t pairs, int R,
                                                            int32_t* __restrict__ chunk_hist,
                                                            int32_t* __restrict__ chunk_bad) {
  extern __shared__ int32_t hist[];  // [R] + 1 bad counter
  for (int e = threadIdx.x; e <= R; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t q0 = (int64_t)blockIdx.x * kDispatchChunk;
  const int64_t q1 = min(q0 + kDispatchChunk, pairs);
  for (int64_t q = q0 + threadIdx.x; q < q1; q += 256) {
    const int e = ids[q];
    atomicAdd(&hist[(e >= 0 && e < R) ? e : R], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < R; e += 256) chunk_hist[(int64_t)blockIdx.x * R + e] = hist[e];
  if (threadIdx.x == 0) chunk_bad[blockIdx.x] = hist[R];
}

// Dispatch step 2 (one workgroup of 1024 threads): per expert, a running sum
// over chunks turns chunk_hist into each chunk's first sorted position;
// counts, offsets (exclusive scan over experts), meta[0] = C = max counts and
// meta[2] = number of ids outside [0, R).  Each thread walks its experts'
// chunk counts kScanBatch at a time (the loads of a batch are independent, so
// their latencies overlap instead of adding up chunk by chunk).
constexpr int kScanBatch = 16;
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ chunk_hist,
                                                             int nchunks, int R,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ chunk_bad,
                                                             int32_t* __restrict__ meta) {
  __shared__ int32_t part[1024];
  __shared__ int32_t cmax[1024];
  __shared__ int32_t bad_part[1024];
  const int t = threadIdx.x;
  int bad = 0;
  for (int c = t; c < nchunks; c += 1024) bad += chunk_bad[c];
  bad_part[t] = bad;
  const int ept = (R + 1023) / 1024;  // experts per thread, contiguous
  const int e0 = min(t * ept, R), e1 = min(e0 + ept, R);
  int my_total = 0, my_max = 0;
  for (int e = e0; e < e1; ++e) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) h[i] = c0 + i < nchunks ? chunk_hist[(int64_t)(c0 + i) * R + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (c0 + i < nchunks) chunk_hist[(int64_t)(c0 + i) * R + e] = run;
        run += h[i];
      }
    }
    counts[e] = run;
    my_total += run;
    my_max = max(my_max, run);
  }
  part[t] = my_total;
  cmax[t] = my_max;
  __syncthreads();
  for (int s = 1; s < 1024; s <<= 1) {  // inclusive scan (sum), suffix max, total of bad ids
    const int a = t >= s ? part[t - s] : 0;
    const int m = t + s < 1024 ? cmax[t + s] : 0;
    const int b = t + s < 1024 ? bad_part[t + s] : 0;
    __syncthreads();
    part[t] += a;
    cmax[t] = max(cmax[t], m);
    bad_part[t] += b;
    __syncthreads();
  }
  int base = part[t] - my_total;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = base;
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) h[i] = c0 + i < nchunks ? chunk_hist[(int64_t)(c0 + i) * R + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (c0 + i < nchunks) chunk_hist[(int64_t)(c0 + i) * R + e] = h[i] + base;
    }
    base += counts[e];
  }
  if (t == 0) {
    meta[0] = cmax[0];
    meta[2] = bad_part[0];
  }
}

// Grouped-GEMM work list (one workgroup of 1024 threads): every expert with
// pairs contributes ceil(counts[e] / tile_m) row tiles (expert, first row), in
// expert order.  meta[1] = number of tiles.
__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ counts, int R,
                                                         int tile_m, int32_t* __restrict__ tile_list,
                                                         int32_t* __restrict__ meta) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int ept = (R + 1023) / 1024;
  const int e0 = min(t * ept, R), e1 = min(e0 + ept, R);
  int mine = 0;
  for (int e = e0; e < e1; ++e) mine += (counts[e] + tile_m - 1) / tile_m;
  part[t] = mine;
  __syncthreads();
  for (int s = 1; s < 1024; s <<= 1) {
    const int a = t >= s ? part[t - s] : 0;
    __syncthreads();
    part[t] += a;
    __syncthreads();
  }
  int tb = part[t] - mine;
  for (int e = e0; e < e1; ++e) {
    for (int m = 0; m < counts[e]; m += tile_m) {
      tile_list[2 * tb] = e;
      tile_list[2 * tb + 1] = m;
      ++tb;
    }
  }
  if (t == 1023) meta[1] = part[1023];
}

// Dispatch step 3: stable scatter.  One workgroup of kDispatchChunk / 64
// waves per chunk, wave w owning the chunk's pairs 64 w .. 64 w + 63 (one per
// lane).  Each wave first ranks its pairs among the wave's pairs of the same
// expert (lanes grouped by expert with ballots, one round per distinct
// expert in the wave); then the waves, in order, add their ranks to
// per-expert cursors in LDS (seeded with the chunk's first positions), so
// pairs of one expert land in ascending pair order.
constexpr int kScatterWaves = kDispatchChunk / 64;
__global__ __launch_bounds__(kDispatchChunk) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                                          int64_t pairs, int R,
                                                                          const int32_t* __restrict__ chunk_base,
                                                                          int32_t* __restrict__ order) {
  extern __shared__ int32_t cursor[];  // [R]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* base = chunk_base + (int64_t)blockIdx.x * R;
  for (int e = tid; e < R; e += kDispatchChunk) cursor[e] = base[e];
  const int64_t q = (int64_t)blockIdx.x * kDispatchChunk + tid;
  int e = -1;  // past the end, or an id outside [0, R): not placed (not counted by the histogram)
  if (q < pairs) {
    const int v = ids[q];
    e = (v >= 0 && v < R) ? v : -1;
  }
  int before = 0;     // lanes below with the same expert
  bool last = true;   // no lane above with the same expert
  uint64_t todo = __ballot(e >= 0);  // wave-uniform
  while (todo) {
    const int lead = __ffsll((unsigned long long)todo) - 1;
    const int el = __builtin_amdgcn_readlane(e, lead);
    const uint64_t m = __ballot(e == el);
    if (e == el) {
      before = __popcll(m & ((1ull << lane) - 1));
      last = (m >> lane) == 1ull;
    }
    todo &= ~m;
  }
  __syncthreads();  // cursors seeded
  for (int w = 0; w < kScatterWaves; ++w) {
    if (wave == w && e >= 0) {
      const int pos = cursor[e] + before;
      order[pos] = (int32_t)q;
      if (last) cursor[e] = pos + 1;  // the wave's last pair of expert e
    }
    __syncthreads();
  }
}

// Padded copy of the pages' layout: padded[e, r] = z[order[offsets[e] + r] / k]
// for r < counts[e], zeros up to C.  One workgroup per padded row.
template <typename T>
__global__ __launch_bounds__(256) void padded_gather_kernel(const T* __restrict__ z, int ell,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ order,
                                                            int k, int64_t C, T* __restrict__ padded) {
  const int64_t row = blockIdx.x;  // e * C + r
  const int e = (int)(row / C), r = (int)(row % C);
  T* dst = padded + row * ell;
  const int vec = 16 / (int)sizeof(T);
  if (r < counts[e]) {
    const int64_t tok = order[offsets[e] + r] / k;
    const T* src = z + tok * ell;
    for (int c = threadIdx.x * vec; c < ell; c += 256 * vec) *(u32x4*)(dst + c) = *(const u32x4*)(src + c);
  } else {
    for (int c = threadIdx.x * vec; c < ell; c += 256 * vec) *(u32x4*)(dst + c) = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace
}  // namespace lmoe
