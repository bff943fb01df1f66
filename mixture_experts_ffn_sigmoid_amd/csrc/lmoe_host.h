// Host side of the C ABI shared by its translation units (forward.hip,
// backward.hip): status helpers, argument checks, workspace carving and the
// GEMM launch table.  Everything here has internal linkage (one copy per
// unit) except the per-thread error text, which all units share.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "latentmoe.h"
#include "backward_kernels.h"
#include "gemm_kernel.h"
#include "merge_kernels.h"
#include "route_kernels.h"
#include "wgrad_kernel.h"

namespace lmoe {
constexpr size_t kErrorBufferBytes = 512;
// The calling thread's description of its last failure (defined once, in forward.hip).
char* error_buffer();
}  // namespace lmoe

using namespace lmoe;

namespace {


lmoe_status fail(lmoe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(lmoe::error_buffer(), lmoe::kErrorBufferBytes, fmt, ap);
  va_end(ap);
  return s;
}

#define LMOE_HIP(call)                                                                      \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(LMOE_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, \
                  __LINE__);                                                                \
  } while (0)

// Stream of an entry point's launches.  Also clears the calling thread's last
// HIP error, which earlier calls of the caller (a failed pointer query, say)
// may have left behind, so that the launch checks report this library's own
// launches only.
hipStream_t launch_stream(void* stream) {
  (void)hipGetLastError();
  return (hipStream_t)stream;
}

// ----------------------------------------------------------------- sizes
struct Plan {
  int64_t N, pairs;
  int d, l, R, k, ns, fr, fs;
  bool bf16;
  int es;  // bytes per stored element
  int nchunks;
  int tile_m;  // rows per grouped-GEMM tile
  int64_t tile_bound;
  int64_t ldh;  // elements per row of the [h_shared | u_normed] buffer
};

// Row-tile height of the grouped expert GEMMs from the mean rows per expert:
// 64 for a handful (weight streaming), 192 from ~100 rows on (one tile usually
// holds a whole expert's rows, so its weights are read once), 128 in between.
int routed_tile_m(int64_t pairs, int R) {
  const int64_t mean = pairs / R;
  return mean < 48 ? 64 : mean < 96 ? 128 : 192;
}

// Matrices and workspace buffers are moved 16 bytes at a time (LDS-DMA
// operand tiles, 16-byte epilogue and weight-gradient stores), so every
// matrix pointer and the workspace must be 16-byte aligned (hipMalloc and
// torch allocations are).  NULL passes: it is checked on its own.
bool misaligned(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (((uintptr_t)q) & 15) return true;
  return false;
}
constexpr const char* kAlignMsg = "matrix pointers and the workspace must be 16-byte aligned";

lmoe_status check_dims(const lmoe_dims* dm, Plan* p) {
  if (!dm) return fail(LMOE_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (dm->n_tokens < 0) return fail(LMOE_ERR_INVALID_ARGUMENT, "n_tokens < 0");
  if (dm->d_model <= 0 || dm->d_latent <= 0 || dm->n_routed <= 0 || dm->ff_routed <= 0)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "non-positive layer width");
  if (dm->n_shared < 0 || (dm->n_shared > 0 && dm->ff_shared <= 0))
    return fail(LMOE_ERR_INVALID_ARGUMENT, "bad shared expert sizes");
  if (dm->top_k < 1 || dm->top_k > dm->n_routed)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "top_k must satisfy 1 <= k <= R (k=%d, R=%d)", dm->top_k,
                dm->n_routed);
  if (!(dm->beta1 > 0.f) || !(dm->beta2 > 0.f)) return fail(LMOE_ERR_INVALID_ARGUMENT, "beta <= 0");
  if (!(dm->rms_eps >= 0.f)) return fail(LMOE_ERR_INVALID_ARGUMENT, "rms_eps < 0");
  if (dm->dtype != LMOE_F32 && dm->dtype != LMOE_BF16)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "unknown dtype %d", dm->dtype);
  // bf16 storage keeps the SiTU hidden in fp16: its bound beta1 * beta2 must fit
  if (dm->dtype == LMOE_BF16 && !((double)dm->beta1 * (double)dm->beta2 < 65504.0))
    return fail(LMOE_ERR_UNSUPPORTED, "beta1 * beta2 must stay below 65504 with bf16 storage");
  if (dm->d_model % 64 || dm->d_latent % 64 || dm->ff_routed % 64 ||
      (dm->n_shared > 0 && dm->ff_shared % 64))
    return fail(LMOE_ERR_UNSUPPORTED, "d, l, f_r, f_s must be multiples of 64");
  if (dm->n_routed > kMaxRouted) return fail(LMOE_ERR_UNSUPPORTED, "n_routed > %d", kMaxRouted);
  if (dm->top_k > kMaxTopK) return fail(LMOE_ERR_UNSUPPORTED, "top_k > %d", kMaxTopK);
  if (dm->n_shared > kMaxSeg - 1) return fail(LMOE_ERR_UNSUPPORTED, "n_shared > %d", kMaxSeg - 1);
  if (dm->d_latent > kMaxLatent) return fail(LMOE_ERR_UNSUPPORTED, "d_latent > %d", kMaxLatent);
  const int64_t pairs = dm->n_tokens * dm->top_k;
  const int64_t es = dm->dtype == LMOE_BF16 ? 2 : 4;
  // gathered expert rows are addressed with 32-bit offsets into z
  if (pairs > (int64_t)INT32_MAX / 2 || dm->n_tokens * dm->d_latent * es >= ((int64_t)1 << 32))
    return fail(LMOE_ERR_UNSUPPORTED, "too many tokens (N * l * element size must stay below 4 GiB)");
  p->N = dm->n_tokens;
  p->pairs = pairs;
  p->d = dm->d_model;
  p->l = dm->d_latent;
  p->R = dm->n_routed;
  p->k = dm->top_k;
  p->ns = dm->n_shared;
  p->fr = dm->ff_routed;
  p->fs = dm->n_shared > 0 ? dm->ff_shared : 0;
  p->bf16 = dm->dtype == LMOE_BF16;
  p->es = p->bf16 ? 2 : 4;
  p->nchunks = (int)((pairs + kDispatchChunk - 1) / kDispatchChunk);
  p->tile_m = routed_tile_m(pairs, p->R);
  p->tile_bound = (pairs + (int64_t)p->R * (p->tile_m - 1)) / p->tile_m;
  p->ldh = (int64_t)p->ns * p->fs + p->l;
  return LMOE_OK;
}

// Bump allocator over the caller's workspace (256-byte aligned regions).
// Split K for few-row dense products (the 64-row tile): with M <= 64 a
// product has only N / 128 tiles, too few to stream its weights at HBM rate,
// so K is cut into S slices (>= 8 K steps each) until about 512 workgroups
// run; each slice stores an fp32 partial product and one pass sums them in
// slice order.  Returns the slice count (1: no split) and its workspace bytes.
int splitk_slices(int64_t M, int64_t N, int64_t k_bytes, int64_t part_bytes, int* kslice) {
  const int64_t steps = k_bytes / 128;  // K steps of the 64-row tile
  const int64_t tiles = ((M + 63) / 64) * ((N + 127) / 128);
  int64_t S = std::min<int64_t>({(512 + tiles - 1) / tiles, steps / 8, 32});
  while (S > 1 && S * M * N * 4 > part_bytes) --S;
  if (S < 2) return 1;
  const int64_t per = (steps + S - 1) / S;
  *kslice = (int)per;
  return (int)((steps + per - 1) / per);  // every slice non-empty
}
int64_t splitk_bytes(int64_t M, int64_t N, int64_t k_bytes) {
  int kslice = 0;
  const int S = splitk_slices(M, N, k_bytes, INT64_MAX, &kslice);
  return S > 1 ? (int64_t)S * M * N * 4 : 0;
}

// Block tiles (rows x cols, waves, A / B LDS stages, bytes of K per step):
//   S  64 x 128 (256 for gate/up pairs), 4 waves, 3/3, 128: few-row dense products
//   M 128 x 128, 4 waves, 3/3, 128
//   L 256 x 256, 8 waves, 2/2, 128 (128 KB of LDS): large dense products
//   W 192 x 256, 8 waves, 2/3, 128 (144 KB): grouped expert products that
//     stream their weights (B) from HBM; the B ring is one stage deeper than
//     the ring of the (L2-resident) A rows
//   V  64 x 256, 4 waves, 2/3, 128: the same for a handful of rows per expert
//   V2 64 x 256, 4 waves, 2/3, 64 (56 KB, two workgroups per CU): the routed
//     down projection with a handful of rows per expert, whose tiles have few
//     K steps: one workgroup's ring fill overlaps the other's streaming
//   M2 128 x 128, 4 waves, 3/3, 64 (48 KB, three workgroups per CU): short-K
//     products whose time goes into storing the output tile
enum Tile { TILE_S = 0, TILE_M = 1, TILE_L = 2, TILE_W = 3, TILE_V = 4, TILE_M2 = 5, TILE_V2 = 6 };

// Dense products: 32-row tiles for a handful of tokens, 256 x 256 when that
// still gives about one tile per compute unit, else 128 x 128.
Tile dense_tile(int64_t M, int64_t cols, bool dual) {
  if (M <= 64) return TILE_S;
  const int64_t big = ((M + 255) / 256) * ((cols + (dual ? 127 : 255)) / (dual ? 128 : 256));
  return big >= 240 ? TILE_L : TILE_M;
}

// Compute units per XCD of the current device (8 XCDs), 32 (gfx950's 256 /
// 8) when no device answers.  Cached per device.
int cus_per_xcd() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) return 32;
    n = cus / 8;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tail split of a large dense product (256 x 256 tiles, GemmArgs tsplit):
// each XCD runs P tiles on its `cus` compute units, so its last wave holds
// rem = P mod cus tiles and leaves the other units idle.  Cutting those tiles
// into S = cus / rem K slices (S <= 4, >= 8 K steps each) turns that wave
// into one of 1 / S of the time, for S fp32 partial blocks per tail tile
// (summed by tail_reduce_kernel).  Applies to 16-bit operands when the tile
// count is a multiple of 8 and rem <= cus / 2.
struct TailPlan {
  int S = 1, whole = 0, kslice = 0, tail_tiles = 0;
  int64_t bytes = 0;
};
constexpr int kTailTile = 256;            // the tile the tail split runs on
constexpr int64_t kTailBlocksMax = 8 * 32;  // partial blocks the forward workspace reserves
constexpr int64_t kTailBlockBytes = (int64_t)kTailTile * kTailTile * 4;
TailPlan tail_split_plan(int64_t m_tiles, int64_t n_tiles, int64_t steps, int cus) {
  TailPlan tp;
  const int64_t per = m_tiles * n_tiles;
  if (per <= 0 || per % 8 != 0 || cus < 2) return tp;
  const int64_t P = per / 8, rem = P % cus;
  if (rem == 0) return tp;
  const int64_t S = std::min<int64_t>(cus / rem, 4);
  if (S < 2 || steps / S < 8) return tp;
  const int64_t kslice = (steps + S - 1) / S;
  tp.S = (int)((steps + kslice - 1) / kslice);  // every slice non-empty
  tp.kslice = (int)kslice;
  tp.whole = (int)(P - rem);
  tp.tail_tiles = (int)(8 * rem);
  tp.bytes = 8 * rem * tp.S * kTailBlockBytes;
  return tp;
}

struct Carver {
  char* base;
  size_t off = 0;
  template <typename X>
  X* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    X* r = base ? (X*)(base + off) : nullptr;
    off += bytes;
    return r;
  }
};

struct RouteWs {
  float* logits;
};
struct DispatchWs {
  int32_t* chunk_hist;
  int32_t* chunk_bad;
  int32_t* meta;
};
struct ExpertsWs {
  int32_t* tile_list;
  int32_t* meta;
  char* h;
  char* slots;
};
struct ForwardWs {
  char* z;
  float* logits;
  int32_t* chunk_hist;
  int32_t* chunk_bad;
  int32_t* meta;
  int32_t* offsets;
  int32_t* order;
  int32_t* tile_list;
  char* h;
  char* slots;
  char* hcat;
  char* part;  // fp32 K-slice partials of the few-row dense products
  int64_t part_bytes;
};

size_t carve_route(const Plan& p, char* b, RouteWs* w) {
  Carver c{b};
  w->logits = c.take<float>((size_t)p.N * p.R * 4);
  return c.off;
}
size_t carve_dispatch(const Plan& p, char* b, DispatchWs* w) {
  Carver c{b};
  w->chunk_hist = c.take<int32_t>((size_t)p.nchunks * p.R * 4);
  w->chunk_bad = c.take<int32_t>((size_t)p.nchunks * 4);
  w->meta = c.take<int32_t>(64);
  return c.off;
}
size_t carve_experts(const Plan& p, char* b, ExpertsWs* w) {
  Carver c{b};
  w->tile_list = c.take<int32_t>((size_t)p.tile_bound * 8);
  w->meta = c.take<int32_t>(64);
  w->h = c.take<char>((size_t)p.pairs * p.fr * p.es);
  w->slots = c.take<char>((size_t)p.pairs * p.l * p.es);
  return c.off;
}
size_t carve_forward(const Plan& p, char* b, ForwardWs* w) {
  Carver c{b};
  w->z = c.take<char>((size_t)p.N * p.l * p.es);
  w->logits = c.take<float>((size_t)p.N * p.R * 4);
  w->chunk_hist = c.take<int32_t>((size_t)p.nchunks * p.R * 4);
  w->chunk_bad = c.take<int32_t>((size_t)p.nchunks * 4);
  w->meta = c.take<int32_t>(64);
  w->offsets = c.take<int32_t>((size_t)p.R * 4);
  w->order = c.take<int32_t>((size_t)p.pairs * 4);
  w->tile_list = c.take<int32_t>((size_t)p.tile_bound * 8);
  w->h = c.take<char>((size_t)p.pairs * p.fr * p.es);
  w->slots = c.take<char>((size_t)p.pairs * p.l * p.es);
  w->hcat = c.take<char>((size_t)p.N * p.ldh * p.es);
  // split-K partials of the latent, router and merge products (used up to 64
  // rows; sized for min(N, 64) rows so the workspace never shrinks as N grows)
  const int64_t pr = std::min<int64_t>(p.N, 64);
  w->part_bytes = std::max({splitk_bytes(pr, p.l, (int64_t)p.d * p.es), splitk_bytes(pr, p.R, (int64_t)p.d * p.es),
                            splitk_bytes(pr, p.d, p.ldh * p.es)});
  // the tail split of the latent and merge products on 256 x 256 tiles
  // (a fixed reservation, so the workspace never shrinks as N grows)
  if (dense_tile(p.N, p.l, false) == TILE_L || dense_tile(p.N, p.d, false) == TILE_L)
    w->part_bytes = std::max(w->part_bytes, kTailBlocksMax * kTailBlockBytes);
  w->part = c.take<char>((size_t)w->part_bytes);
  return c.off;
}

// Routed-block backward.  Rows of the [pairs, *] buffers are in sorted pair
// order; the transposed buffers hold, per expert, a row-major [cols, kr_len]
// block of its pairs zero-padded to a multiple of 64 (kpad bounds the total
// of kr_len).
struct RoutedBwdWs {
  int32_t *counts, *offsets, *order, *chunk_hist, *chunk_bad, *meta, *tile_list, *inv, *kr_off, *kr_len;
  char *g, *up;  // gate / up pre-activations (intermediate type)
  char* o;       // the layer backward's slot rows, then the dz rows (intermediate type)
  float* dh;     // v = W_o^T du per pair
  float* sp;               // probs of the sorted pairs
  char* du16;              // du in the intermediate type (16-bit operands of v)
  char *hs, *dout, *dgu;   // intermediate type
  char *w_oT, *w_guT;      // storage type
  char *doutT, *hT, *dgT, *duT, *zT;
  int64_t kpad;
};
size_t carve_routed_backward(const Plan& p, char* b, RoutedBwdWs* w) {
  Carver c{b};
  const int64_t P = p.pairs, ei = p.es;  // intermediates: fp16 with bf16 storage, fp32 with fp32
  w->kpad = P + 63 * (int64_t)p.R;
  w->counts = c.take<int32_t>((size_t)p.R * 4);
  w->offsets = c.take<int32_t>((size_t)p.R * 4);
  w->order = c.take<int32_t>((size_t)P * 4);
  w->chunk_hist = c.take<int32_t>((size_t)p.nchunks * p.R * 4);
  w->chunk_bad = c.take<int32_t>((size_t)p.nchunks * 4);
  w->meta = c.take<int32_t>(64);
  w->tile_list = c.take<int32_t>((size_t)p.tile_bound * 8);
  w->inv = c.take<int32_t>((size_t)P * 4);
  w->kr_off = c.take<int32_t>((size_t)p.R * 4);
  w->kr_len = c.take<int32_t>((size_t)p.R * 4);
  w->g = c.take<char>((size_t)P * p.fr * ei);
  w->up = c.take<char>((size_t)P * p.fr * ei);
  w->o = c.take<char>((size_t)P * p.l * ei);
  w->dh = c.take<float>((size_t)P * p.fr * 4);
  w->sp = c.take<float>((size_t)P * 4);
  w->du16 = c.take<char>(ei == 2 ? (size_t)p.N * p.l * ei : 0);
  w->hs = c.take<char>((size_t)P * p.fr * ei);
  w->dout = c.take<char>((size_t)P * p.l * ei);
  w->dgu = c.take<char>((size_t)P * 2 * p.fr * ei);
  // transposed routed weights: fp32 only (16-bit weights are read K-major)
  const bool transposed = p.es == 4;
  w->w_oT = c.take<char>(transposed ? (size_t)p.R * p.fr * p.l * p.es : 0);
  w->w_guT = c.take<char>(transposed ? (size_t)p.R * p.l * 2 * p.fr * p.es : 0);
  w->doutT = c.take<char>((size_t)p.l * w->kpad * ei);
  w->hT = c.take<char>((size_t)p.fr * w->kpad * ei);
  w->dgT = c.take<char>((size_t)p.fr * w->kpad * ei);
  w->duT = c.take<char>((size_t)p.fr * w->kpad * ei);
  w->zT = c.take<char>((size_t)p.l * w->kpad * ei);
  return c.off;
}

// Whole-layer backward: the routed block's workspace plus the dense parts.
// dcat [N, kcat] = [dz | dl (R padded to rpad) | dg_shared | du_shared] feeds
// one K-segmented product for dx; the [cols, npad] transposes (N zero-padded
// to a multiple of 64) feed the dense weight gradients.
struct LayerBwdWs {
  RoutedBwdWs rw;
  int64_t rpad, nsf, kcat, npad, rms_chunk;
  char *z, *rn, *hs, *dcat;            // intermediate type
  float *logits, *u, *dr, *dhs, *du, *rho, *dprobs, *rms_part;
  char *ag, *au;  // shared gate / up pre-activations (intermediate type)
  char *w_upT, *shoT, *w_downT, *w_rT, *sgT, *suT;  // storage type
  int32_t* seg;
  char *dyT, *rnT, *hsT, *dcatT, *xT;  // intermediate type
  char* tpart;  // fp32 partial blocks of dx's tail split (NULL: none)
  int64_t tpart_bytes;
};
size_t carve_layer_backward(const Plan& p, char* b, LayerBwdWs* w) {
  Carver c{b};
  const size_t rsz = carve_routed_backward(p, nullptr, &w->rw);
  char* rbase = c.take<char>(rsz);
  if (b) carve_routed_backward(p, rbase, &w->rw);
  const int64_t N = p.N, ei = p.es, es = p.es;
  w->rpad = (p.R + 63) / 64 * 64;
  w->nsf = (int64_t)p.ns * p.fs;
  w->kcat = p.l + w->rpad + 2 * w->nsf;
  w->npad = (N + 63) / 64 * 64;
  w->z = c.take<char>((size_t)N * p.l * ei);
  w->rn = c.take<char>((size_t)N * p.l * ei);
  w->hs = c.take<char>((size_t)N * w->nsf * ei);
  w->dcat = c.take<char>((size_t)N * w->kcat * ei);
  w->logits = c.take<float>((size_t)N * p.R * 4);
  w->u = c.take<float>((size_t)N * p.l * 4);
  w->ag = c.take<char>((size_t)N * w->nsf * p.es);
  w->au = c.take<char>((size_t)N * w->nsf * p.es);
  w->dr = c.take<float>((size_t)N * p.l * 4);
  w->dhs = c.take<float>((size_t)N * w->nsf * 4);
  w->du = c.take<float>((size_t)N * p.l * 4);
  w->rho = c.take<float>((size_t)N * 4);
  w->dprobs = c.take<float>((size_t)N * p.k * 4);
  w->rms_chunk = std::max<int64_t>(kWgradChunk, (N + 65534) / 65535);
  w->rms_part = c.take<float>((size_t)((N + w->rms_chunk - 1) / w->rms_chunk) * p.l * 4);
  w->w_upT = c.take<char>((size_t)p.l * p.d * es);
  w->shoT = c.take<char>((size_t)w->nsf * p.d * es);
  w->w_downT = c.take<char>((size_t)p.d * p.l * es);
  w->w_rT = c.take<char>((size_t)p.d * w->rpad * es);
  w->sgT = c.take<char>((size_t)p.d * w->nsf * es);
  w->suT = c.take<char>((size_t)p.d * w->nsf * es);
  w->seg = c.take<int32_t>(16);
  w->dyT = c.take<char>((size_t)p.d * w->npad * ei);
  w->rnT = c.take<char>((size_t)p.l * w->npad * ei);
  w->hsT = c.take<char>((size_t)w->nsf * w->npad * ei);
  w->dcatT = c.take<char>((size_t)w->kcat * w->npad * ei);
  w->xT = c.take<char>((size_t)p.d * w->npad * ei);
  // dx on 256 x 256 tiles with 16-bit operands may take the tail split
  w->tpart_bytes = (ei == 2 && dense_tile(N, p.d, false) == TILE_L) ? kTailBlocksMax * kTailBlockBytes : 0;
  w->tpart = w->tpart_bytes ? c.take<char>((size_t)w->tpart_bytes) : nullptr;
  return c.off;
}

// Words of a workspace's meta block: C (dispatch), the grouped tile count,
// the count of expert ids outside [0, R), and the range flag (set when an
// fp16 intermediate of the forward left fp16's range).
constexpr int kMetaC = 0, kMetaTiles = 1, kMetaBadIds = 2, kMetaRange = 3;

// The shared-expert gate/up GEMM runs on the second stream while its
// multiply-adds N d n_s f_s stay at or below those of 2048 tokens at the
// full-K3 widths (d = 7168, one shared expert of f_s = 18432): up to there the
// layer's GEMMs leave compute units idle between launches; past it each fills
// the chip alone and their 128-144 KB LDS tiles cannot share a CU.
constexpr double kOverlapMaxSharedMacs = 2048.0 * 7168.0 * 18432.0;
inline bool shared_overlaps(const Plan& p) {
  return p.ns > 0 && (double)p.N * p.d * p.ns * p.fs <= kOverlapMaxSharedMacs;
}

// A second stream on which the shared-expert GEMM overlaps the routed
// experts: default priority, non-blocking, created on first use for each
// (host thread, device) and kept until the process ends.  Per thread, so
// that one thread capturing a forward into a graph never captures (or
// breaks) another thread's forward on the same device.
lmoe_status side_stream(hipStream_t* out) {
  thread_local hipStream_t streams[64] = {};
  int dev = 0;
  LMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(LMOE_ERR_UNSUPPORTED, "device index %d", dev);
  if (!streams[dev]) LMOE_HIP(hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking));
  *out = streams[dev];
  return LMOE_OK;
}

// ------------------------------------------------------------ GEMM launches
template <typename TA, typename TB, typename OutT, int BM, int BN, int WGM, int WGN, int AM, int BMD,
          int EM, int SA, int SB, int KB>
lmoe_status launch_gemm(GemmArgs a, hipStream_t st) {
  const int64_t per = (int64_t)a.m_tiles * a.n_tiles;
  const int64_t grid = a.tsplit > 1 ? 8 * (a.twhole + (per / 8 - a.twhole) * (int64_t)a.tsplit)
                                    : per * (AM == A_KBATCH ? a.nbatch : a.ksplit > 1 ? a.ksplit : 1);
  if (grid <= 0) return LMOE_OK;
  if (grid > INT32_MAX) return fail(LMOE_ERR_UNSUPPORTED, "GEMM grid too large");
  gemm_kernel<TA, TB, OutT, BM, BN, WGM, WGN, AM, BMD, EM, SA, SB, KB>
      <<<(unsigned)grid, 64 * WGM * WGN, 0, st>>>(a);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}


template <typename TA, typename TB, typename OutT, int AM, int BMD, int EM, int BM, int BN, int WGM,
          int WGN, int SA, int SB, int KB = 64>
lmoe_status gemm_cfg(GemmArgs a, hipStream_t st) {
  constexpr int cols = BMD == B_DUAL ? BN / 2 : BN;
  a.n_tiles = (a.N + cols - 1) / cols;
  if (AM == A_DENSE || AM == A_KBATCH) a.m_tiles = (a.M + BM - 1) / BM;
  if ((int64_t)a.K * (int64_t)sizeof(TA) % KB != 0) return fail(LMOE_ERR_UNSUPPORTED, "K not a multiple of the K step");
  if constexpr (BMD == B_KMAJOR) {
    if (a.nb_rows < 8 || a.nb_rows % 8 != 0) return fail(LMOE_ERR_UNSUPPORTED, "K-major B needs a multiple of 8 columns");
    if (a.kmaj_split % (KB / (int)sizeof(TB)) != 0 && a.kmaj_split < a.K)
      return fail(LMOE_ERR_UNSUPPORTED, "K-major B split not a multiple of the K step");
  }
  if (BMD == B_KSEG)
    for (int s = 0; s <= a.nseg; ++s)
      if (a.seg_kt0[s] % (KB / kSegUnit) != 0) return fail(LMOE_ERR_UNSUPPORTED, "K segment not a multiple of the K step");
  return launch_gemm<TA, TB, OutT, BM, BN, WGM, WGN, AM, BMD, EM, SA, SB, KB>(a, st);
}

template <typename TA, typename TB, typename OutT, int AM, int BMD, int EM>
lmoe_status gemm(GemmArgs a, Tile t, hipStream_t st) {
  constexpr bool dual = BMD == B_DUAL;
  if constexpr (AM == A_DENSE && EM == E_STORE && !dual) {
    int kslice = 0;
    const int S = (t == TILE_S && a.part && a.M <= 64)
                      ? splitk_slices(a.M, a.N, (int64_t)a.K * sizeof(TA), a.part_bytes, &kslice)
                      : 1;
    if (S > 1) {
      GemmArgs g = a;
      g.out = a.part;
      g.ldo = (int64_t)a.N * 4;
      g.o_batch_stride = (int64_t)a.M * a.N * 4;
      g.ksplit = S;
      g.kslice = kslice;
      g.part = nullptr;
      const lmoe_status ps = gemm_cfg<TA, TB, float, AM, BMD, EM, 64, 128, 1, 4, 3, 3, 128>(g, st);
      if (ps != LMOE_OK) return ps;
      const int64_t mn = (int64_t)a.M * a.N;
      splitk_reduce_kernel<OutT><<<(unsigned)std::min<int64_t>((mn + 1023) / 1024, 2048), 256, 0, st>>>(
          (const float*)a.part, S, a.M, a.N, a.out, a.ldo, a.range_flag);
      LMOE_HIP(hipGetLastError());
      return LMOE_OK;
    }
    if (sizeof(TA) == 2 && t == TILE_L && a.part && a.M > 0 && a.N > 0 && (int64_t)a.K * 2 % 128 == 0) {
      GemmArgs g = a;
      g.m_tiles = (a.M + kTailTile - 1) / kTailTile;
      g.n_tiles = (a.N + kTailTile - 1) / kTailTile;
      const TailPlan tp = tail_split_plan(g.m_tiles, g.n_tiles, (int64_t)a.K * sizeof(TA) / 128, cus_per_xcd());
      if (tp.S > 1 && tp.bytes <= a.part_bytes) {
        g.tsplit = tp.S;
        g.twhole = tp.whole;
        g.kslice = tp.kslice;
        g.tpart = a.part;
        g.part = nullptr;
        const lmoe_status ts = gemm_cfg<TA, TB, OutT, AM, BMD, EM, kTailTile, kTailTile, 2, 4, 2, 2, 128>(g, st);
        if (ts != LMOE_OK) return ts;
        tail_reduce_kernel<OutT, kTailTile, kTailTile><<<(unsigned)tp.tail_tiles * (kTailTile / 16), 256, 0, st>>>(g);
        LMOE_HIP(hipGetLastError());
        return LMOE_OK;
      }
    }
  }
  if constexpr (AM == A_DENSE || AM == A_KBATCH) {
    switch (t) {
      case TILE_S: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 64, dual ? 256 : 128, 1, 4, 3, 3, 128>(a, st);
      case TILE_M: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 128, 128, 2, 2, 3, 3, 128>(a, st);
      case TILE_M2: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 128, 128, 2, 2, 3, 3, 64>(a, st);
      default: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 256, 256, 2, 4, 2, 2, 128>(a, st);
    }
  } else {
    switch (t) {
      case TILE_V: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 64, 256, 1, 4, 2, 3, 128>(a, st);
      case TILE_V2: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 64, 256, 1, 4, 2, 3, 64>(a, st);
      case TILE_M: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 128, 128, 2, 2, 3, 3, 128>(a, st);
      default: return gemm_cfg<TA, TB, OutT, AM, BMD, EM, 192, 256, 2, 4, 2, 3, 128>(a, st);
    }
  }
}


GemmArgs base_args(const lmoe_dims* dm) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.beta1 = dm->beta1;
  a.beta2 = dm->beta2;
  a.nseg = 1;
  return a;
}

#define LMOE_TRY(x)                       \
  do {                                    \
    lmoe_status s_ = (x);                 \
    if (s_ != LMOE_OK) return s_;         \
  } while (0)

// counts / offsets / stable order (+ C in meta[0]).
lmoe_status run_dispatch(const Plan& p, const int32_t* ids, int32_t* chunk_hist, int32_t* chunk_bad,
                         int32_t* counts, int32_t* offsets, int32_t* order, int32_t* meta,
                         hipStream_t st) {
  dispatch_hist_kernel<<<p.nchunks, 256, (p.R + 1) * sizeof(int32_t), st>>>(ids, p.pairs, p.R,
                                                                            chunk_hist, chunk_bad);
  LMOE_HIP(hipGetLastError());
  dispatch_scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, p.nchunks, p.R, counts, offsets, chunk_bad, meta);
  LMOE_HIP(hipGetLastError());
  dispatch_scatter_kernel<<<p.nchunks, kDispatchChunk, p.R * sizeof(int32_t), st>>>(ids, p.pairs, p.R,
                                                                                          chunk_hist, order);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}
}  // namespace
