// C ABI of the gfx950 Stable LatentMoE forward: argument checks, workspace
// carving and the launch sequence of each entry point (see latentmoe.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "latentmoe.h"
#include "backward_kernels.h"
#include "gemm_kernel.h"
#include "merge_kernels.h"
#include "route_kernels.h"
#include "wgrad_kernel.h"

using namespace lmoe;

namespace {

thread_local char g_err[512] = "";

lmoe_status fail(lmoe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
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
  w->part = c.take<char>((size_t)w->part_bytes);
  return c.off;
}

// Routed-block backward.  Rows of the [pairs, *] buffers are in sorted pair
// order; the transposed buffers hold, per expert, a row-major [cols, kr_len]
// block of its pairs zero-padded to a multiple of 64 (kpad bounds the total
// of kr_len).
struct RoutedBwdWs {
  int32_t *counts, *offsets, *order, *chunk_hist, *chunk_bad, *meta, *tile_list, *inv, *kr_off, *kr_len;
  float *g, *up, *o, *dh;  // o also holds the dz rows once it is consumed
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
  w->g = c.take<float>((size_t)P * p.fr * 4);
  w->up = c.take<float>((size_t)P * p.fr * 4);
  w->o = c.take<float>((size_t)P * p.l * 4);
  w->dh = c.take<float>((size_t)P * p.fr * 4);
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
  float *logits, *u, *ag, *au, *dr, *dhs, *du, *rho, *dprobs, *rms_part;
  char *w_upT, *shoT, *w_downT, *w_rT, *sgT, *suT;  // storage type
  int32_t* seg;
  char *dyT, *rnT, *hsT, *dcatT, *xT;  // intermediate type
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
  w->ag = c.take<float>((size_t)N * w->nsf * 4);
  w->au = c.take<float>((size_t)N * w->nsf * 4);
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
  return c.off;
}

// Largest batch whose shared-expert GEMM runs on the second stream.
constexpr int64_t kOverlapMaxTokens = 2048;

// A second stream per device on which the shared-expert GEMM overlaps the
// routed experts (default priority, non-blocking, created once per device).
lmoe_status side_stream(hipStream_t* out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  LMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(LMOE_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) LMOE_HIP(hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking));
  *out = streams[dev];
  return LMOE_OK;
}

// ------------------------------------------------------------ GEMM launches
template <typename TA, typename TB, typename OutT, int BM, int BN, int WGM, int WGN, int AM, int BMD,
          int EM, int SA, int SB, int KB>
lmoe_status launch_gemm(GemmArgs a, hipStream_t st) {
  const int64_t grid = (int64_t)a.m_tiles * a.n_tiles * (AM == A_KBATCH ? a.nbatch : a.ksplit > 1 ? a.ksplit : 1);
  if (grid <= 0) return LMOE_OK;
  if (grid > INT32_MAX) return fail(LMOE_ERR_UNSUPPORTED, "GEMM grid too large");
  gemm_kernel<TA, TB, OutT, BM, BN, WGM, WGN, AM, BMD, EM, SA, SB, KB>
      <<<(unsigned)grid, 64 * WGM * WGN, 0, st>>>(a);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
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
          (const float*)a.part, S, a.M, a.N, a.out, a.ldo);
      LMOE_HIP(hipGetLastError());
      return LMOE_OK;
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

// Dense products: 32-row tiles for a handful of tokens, 256 x 256 when that
// still gives about one tile per compute unit, else 128 x 128.
Tile dense_tile(int64_t M, int64_t cols, bool dual) {
  if (M <= 64) return TILE_S;
  const int64_t big = ((M + 255) / 256) * ((cols + (dual ? 127 : 255)) / (dual ? 128 : 256));
  return big >= 240 ? TILE_L : TILE_M;
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

// ---------------------------------------------------------- step launchers
// logits = x W_r^T (fp32), then the sigmoid / top-k / renormalisation kernel.
template <typename T>
lmoe_status run_route(const Plan& p, const lmoe_dims* dm, const void* x, const void* w_router,
                      const float* bias, int32_t* ids, float* probs, float* logits, hipStream_t st,
                      bool softmax = false, char* part = nullptr, int64_t part_bytes = 0) {
  GemmArgs a = base_args(dm);
  a.M = (int)p.N;
  a.N = p.R;
  a.K = p.d;
  a.a = (const char*)x;
  a.lda = (int64_t)p.d * p.es;
  a.b0 = (const char*)w_router;
  a.ldb = (int64_t)p.d * p.es;
  a.nb_rows = p.R;
  a.out = (char*)logits;
  a.ldo = (int64_t)p.R * 4;
  a.part = part;
  a.part_bytes = part_bytes;
  LMOE_TRY((gemm<T, T, float, A_DENSE, B_SINGLE, E_STORE>(a, dense_tile(p.N, p.R, false), st)));
  const unsigned blocks = (unsigned)((p.N + 3) / 4);
  if (softmax)
    topk_route_kernel<true><<<blocks, 256, 4 * p.R * sizeof(float), st>>>(logits, nullptr, p.N, p.R, p.k,
                                                                          ids, probs);
  else
    topk_route_kernel<false><<<blocks, 256, 4 * p.R * sizeof(float), st>>>(logits, bias, p.N, p.R, p.k,
                                                                           ids, probs);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

// counts / offsets / stable order (+ C in meta[0]).
lmoe_status run_dispatch(const Plan& p, const int32_t* ids, int32_t* chunk_hist, int32_t* chunk_bad,
                         int32_t* counts, int32_t* offsets, int32_t* order, int32_t* meta,
                         hipStream_t st) {
  dispatch_hist_kernel<<<p.nchunks, 256, (p.R + 1) * sizeof(int32_t), st>>>(ids, p.pairs, p.R,
                                                                            chunk_hist, chunk_bad);
  LMOE_HIP(hipGetLastError());
  dispatch_scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, p.nchunks, p.R, counts, offsets, chunk_bad, meta);
  LMOE_HIP(hipGetLastError());
  dispatch_scatter_kernel<<<p.nchunks, 64, p.R * sizeof(int32_t), st>>>(ids, p.pairs, p.R,
                                                                              chunk_hist, order);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

// Routed experts: tile list, gate/up grouped GEMM with the SiTU epilogue into
// h (sorted pair rows, type TH), down grouped GEMM with the p-weighted slot
// epilogue.  TA: type of the gathered rows, TW: weight storage type.
template <typename TA, typename TW, typename TH, int AM, typename Mark = lmoe_status (*)()>
lmoe_status run_experts(const Plan& p, const lmoe_dims* dm, const void* a_src, int64_t cap,
                        const int32_t* counts, const int32_t* offsets, const int32_t* order,
                        const float* probs, const void* w_g, const void* w_u, const void* w_o,
                        int32_t* tile_list, int32_t* meta, char* h, char* slots, hipStream_t st,
                        Mark* mark = nullptr) {
  tile_list_kernel<<<1, 1024, 0, st>>>(counts, p.R, p.tile_m, tile_list, meta);
  LMOE_HIP(hipGetLastError());
  const Tile tile = p.tile_m == 64 ? TILE_V : p.tile_m == 128 ? TILE_M : TILE_W;
  GemmArgs a = base_args(dm);
  a.N = p.fr;
  a.K = p.l;
  a.m_tiles = (int)p.tile_bound;
  a.a = (const char*)a_src;
  a.lda = (int64_t)p.l * sizeof(TA);
  a.order = order;
  a.top_k = p.k;
  a.cap = cap;
  a.tile_list = tile_list;
  a.tile_count = meta + 1;
  a.counts = counts;
  a.offsets = offsets;
  a.b0 = (const char*)w_g;
  a.b1 = (const char*)w_u;
  a.ldb = (int64_t)p.l * p.es;
  a.b_expert_stride = (int64_t)p.fr * p.l * p.es;
  a.nb_rows = p.fr;
  a.out = h;
  a.ldo = (int64_t)p.fr * p.es;
  LMOE_TRY((gemm<TA, TW, TH, AM, B_DUAL, E_SITU>(a, tile, st)));
  if (mark) LMOE_TRY((*mark)());

  GemmArgs b = base_args(dm);
  b.N = p.l;
  b.K = p.fr;
  b.m_tiles = (int)p.tile_bound;
  b.a = h;
  b.lda = (int64_t)p.fr * p.es;
  b.order = order;
  b.top_k = p.k;
  b.tile_list = tile_list;
  b.tile_count = meta + 1;
  b.counts = counts;
  b.offsets = offsets;
  b.b0 = (const char*)w_o;
  b.ldb = (int64_t)p.fr * p.es;
  b.b_expert_stride = (int64_t)p.l * p.fr * p.es;
  b.nb_rows = p.l;
  b.out = slots;
  b.ldo = (int64_t)p.l * sizeof(TH);
  b.probs = probs;
  return gemm<TH, TW, TH, A_SORTED, B_SINGLE, E_SLOTS>(b, tile == TILE_V ? TILE_V2 : tile, st);
}

// Batched transpose out[b][c][col0 + r] = in[b][r][c] (16-byte accesses for
// 16-bit elements), skipping batches without pairs.
template <typename T>
lmoe_status transpose_batched(const T* in, int64_t in_bstride, int ld_in, int rows, int cols, T* out,
                              int64_t out_bstride, int ld_out, int col0, int nbatch, const int32_t* counts,
                              hipStream_t st) {
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64, nbatch);
  if constexpr (sizeof(T) == 2)
    transpose16_batched_kernel<<<grid, 256, 0, st>>>((const uint16_t*)in, in_bstride, ld_in, rows, cols,
                                                     (uint16_t*)out, out_bstride, ld_out, col0, counts);
  else
    transpose_batched_kernel<T><<<grid, 256, 0, st>>>(in, in_bstride, ld_in, rows, cols, out, out_bstride,
                                                      ld_out, col0, counts);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

// Expert-segment transpose (see segment_transpose_kernel); 16-bit data with
// 8-element-aligned columns and strides goes through the 16-byte kernel.
template <typename TS, typename TD>
lmoe_status segment_transpose(dim3 grid, const TS* src, int64_t ld_src, int col_off, int ncols,
                              const int32_t* counts, const int32_t* offsets, const int32_t* order, int top_k,
                              const int32_t* kr_off, const int32_t* kr_len, TD* out, hipStream_t st) {
  if constexpr (sizeof(TS) == 2 && sizeof(TD) == 2) {
    if (ncols % 8 == 0 && col_off % 8 == 0 && ld_src % 8 == 0 && (((uintptr_t)src | (uintptr_t)out) & 15) == 0) {
      segment_transpose16_kernel<TS, TD><<<grid, 256, 0, st>>>(src, ld_src, col_off, ncols, counts, offsets,
                                                               order, top_k, kr_off, kr_len, out);
      LMOE_HIP(hipGetLastError());
      return LMOE_OK;
    }
  }
  segment_transpose_kernel<TS, TD><<<grid, 256, 0, st>>>(src, ld_src, col_off, ncols, counts, offsets, order,
                                                         top_k, kr_off, kr_len, out);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

// Grouped-GEMM arguments over the routed pairs of a backward workspace.
GemmArgs routed_grouped(const Plan& p, const lmoe_dims* dm, const RoutedBwdWs& w, const void* a, int64_t lda,
                        const void* bw, int64_t ldb, int64_t bstride, int nrows, int K, void* out, int64_t ldo) {
  GemmArgs g = base_args(dm);
  g.N = nrows;
  g.K = K;
  g.m_tiles = (int)p.tile_bound;
  g.a = (const char*)a;
  g.lda = lda;
  g.order = w.order;
  g.top_k = p.k;
  g.tile_list = w.tile_list;
  g.tile_count = w.meta + 1;
  g.counts = w.counts;
  g.offsets = w.offsets;
  g.b0 = (const char*)bw;
  g.ldb = ldb;
  g.b_expert_stride = bstride;
  g.nb_rows = nrows;
  g.out = (char*)out;
  g.ldo = ldo;
  return g;
}

Tile routed_tile(const Plan& p) { return p.tile_m == 64 ? TILE_V : p.tile_m == 128 ? TILE_M : TILE_W; }

// Forward part of the routed-block backward: the dispatch bookkeeping, the
// pre-activations g = z W_g^T and up = z W_u^T (fp32), the hidden h (TI) and
// the expert outputs o = h W_o^T (fp32), all in sorted pair order.  Returns
// the capacity C (one host read-back).  T: storage type of the weights;
// TI: intermediate type; TZ: type of z.
template <typename T, typename TI, typename TZ>
lmoe_status routed_recompute(const Plan& p, const lmoe_dims* dm, const void* z, const int32_t* ids,
                             const void* w_g, const void* w_u, const void* w_o, const RoutedBwdWs& w,
                             int* C_out, hipStream_t st) {
  const int64_t P = p.pairs;
  const int f = p.fr, l = p.l, R = p.R;
  const int64_t es = sizeof(T), ei = sizeof(TI);
  auto blocks = [](int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); };
  // 1. bookkeeping: counts, offsets, stable order, C, tile list, inverse order, padded K ranges
  LMOE_TRY(run_dispatch(p, ids, w.chunk_hist, w.chunk_bad, w.counts, w.offsets, w.order, w.meta, st));
  tile_list_kernel<<<1, 1024, 0, st>>>(w.counts, R, p.tile_m, w.tile_list, w.meta);
  LMOE_HIP(hipGetLastError());
  int32_t meta[4] = {0, 0, 0, 0};
  LMOE_HIP(hipMemcpyAsync(meta, w.meta, sizeof(meta), hipMemcpyDeviceToHost, st));
  LMOE_HIP(hipStreamSynchronize(st));
  if (meta[2] != 0) return fail(LMOE_ERR_INVALID_ARGUMENT, "%d expert ids outside [0, R)", meta[2]);
  *C_out = meta[0];
  inverse_order_kernel<<<(unsigned)((P + 255) / 256), 256, 0, st>>>(w.order, P, w.inv);
  LMOE_HIP(hipGetLastError());
  padded_ranges_kernel<<<1, 1024, 0, st>>>(w.counts, R, w.kr_off, w.kr_len);
  LMOE_HIP(hipGetLastError());
  const Tile tile = routed_tile(p);
  auto grouped = [&](const void* a, int64_t lda, const void* bw, int64_t ldb, int64_t bstride, int nrows,
                     int K, void* out, int64_t ldo) {
    return routed_grouped(p, dm, w, a, lda, bw, ldb, bstride, nrows, K, out, ldo);
  };
  // 2. pre-activations of every pair: g = z W_g^T, up = z W_u^T (fp32, sorted rows)
  const int64_t ez = sizeof(TZ);
  LMOE_TRY((gemm<TZ, T, float, A_GATHER, B_SINGLE, E_STORE>(
      grouped(z, l * ez, w_g, l * es, (int64_t)f * l * es, f, l, w.g, (int64_t)f * 4), tile, st)));
  LMOE_TRY((gemm<TZ, T, float, A_GATHER, B_SINGLE, E_STORE>(
      grouped(z, l * ez, w_u, l * es, (int64_t)f * l * es, f, l, w.up, (int64_t)f * 4), tile, st)));
  situ_hidden_kernel<TI><<<blocks(P * f), 256, 0, st>>>(w.g, w.up, P * f, dm->beta1, dm->beta2, (TI*)w.hs);
  LMOE_HIP(hipGetLastError());
  // 3. expert outputs o = h W_o^T (fp32, sorted rows)
  return gemm<TI, T, float, A_SORTED, B_SINGLE, E_STORE>(
      grouped(w.hs, f * ei, w_o, f * es, (int64_t)l * f * es, l, f, w.o, (int64_t)l * 4), tile, st);
}

// Gradient part of the routed-block backward, on the quantities
// routed_recompute left in the workspace.  dz is written as TDZ with row
// stride ld_dz.
template <typename T, typename TI, typename TZ, typename TDZ>
lmoe_status routed_gradients(const Plan& p, const lmoe_dims* dm, const void* z, const float* probs,
                             const void* w_g, const void* w_u, const void* w_o, const float* du, void* dz,
                             int64_t ld_dz, float* dprobs, void* dw_g, void* dw_u, void* dw_o, const RoutedBwdWs& w,
                             int C, hipStream_t st) {
  const int64_t P = p.pairs;
  const int f = p.fr, l = p.l, R = p.R;
  const int64_t es = sizeof(T), ei = sizeof(TI);
  auto blocks = [](int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); };
  const Tile tile = routed_tile(p);
  auto grouped = [&](const void* a, int64_t lda, const void* bw, int64_t ldb, int64_t bstride, int nrows,
                     int K, void* out, int64_t ldo) {
    return routed_grouped(p, dm, w, a, lda, bw, ldb, bstride, nrows, K, out, ldo);
  };
  // 3b. dprobs and dout = p * du (sorted rows)
  pair_grad_kernel<TI><<<(unsigned)P, 256, 0, st>>>(du, w.o, probs, w.order, p.k, l, dprobs, (TI*)w.dout);
  LMOE_HIP(hipGetLastError());
  // 4. dh = dout W_o, then the SiTU backward -> [dg | du].  16-bit weights are
  // read as stored (K-major B: K-row k of W_o[e] is its latent row k); fp32
  // ones through a transposed copy W_o^T [R, f, l]
  if constexpr (sizeof(T) == 2) {
    GemmArgs g = grouped(w.dout, l * ei, w_o, f * es, (int64_t)l * f * es, f, l, w.dh, (int64_t)f * 4);
    g.kmaj_split = l;
    LMOE_TRY((gemm<TI, T, float, A_SORTED, B_KMAJOR, E_STORE>(g, tile, st)));
  } else {
    LMOE_TRY(transpose_batched<T>((const T*)w_o, (int64_t)l * f, f, l, f, (T*)w.w_oT, (int64_t)f * l, l, 0, R,
                                   w.counts, st));
    LMOE_TRY((gemm<TI, T, float, A_SORTED, B_SINGLE, E_STORE>(
        grouped(w.dout, l * ei, w.w_oT, l * es, (int64_t)f * l * es, f, l, w.dh, (int64_t)f * 4), tile, st)));
  }
  situ_backward_kernel<TI><<<(unsigned)std::min<int64_t>(P, 65536), 256, 0, st>>>(
      w.dh, w.g, w.up, P, f, dm->beta1, dm->beta2, (TI*)w.dgu, 2 * (int64_t)f, 0);
  LMOE_HIP(hipGetLastError());
  // 5. dz rows = [dg | du] [W_g ; W_u] (K = 2f: W_g's rows, then W_u's), summed per token
  float* dzrows = w.o;  // o is consumed
  if constexpr (sizeof(T) == 2) {
    GemmArgs g = grouped(w.dgu, 2 * f * ei, w_g, l * es, (int64_t)f * l * es, l, 2 * f, dzrows, (int64_t)l * 4);
    g.b1 = (const char*)w_u;
    g.kmaj_split = f;
    LMOE_TRY((gemm<TI, T, float, A_SORTED, B_KMAJOR, E_STORE>(g, tile, st)));
  } else {
    LMOE_TRY(transpose_batched<T>((const T*)w_g, (int64_t)f * l, l, f, l, (T*)w.w_guT, (int64_t)l * 2 * f,
                                   2 * f, 0, R, w.counts, st));
    LMOE_TRY(transpose_batched<T>((const T*)w_u, (int64_t)f * l, l, f, l, (T*)w.w_guT, (int64_t)l * 2 * f,
                                   2 * f, f, R, w.counts, st));
    LMOE_TRY((gemm<TI, T, float, A_SORTED, B_SINGLE, E_STORE>(
        grouped(w.dgu, 2 * f * ei, w.w_guT, 2 * f * es, (int64_t)l * 2 * f * es, l, 2 * f, dzrows,
                (int64_t)l * 4),
        tile, st)));
  }
  pair_sum_kernel<TDZ><<<(unsigned)p.N, 256, 0, st>>>(dzrows, w.inv, p.k, l, nullptr, (TDZ*)dz, ld_dz);
  LMOE_HIP(hipGetLastError());
  // 6. weight gradients: per expert, products over its pairs (K = padded pair range)
  const unsigned ysegs = (unsigned)((C + 63) / 64);
  if (ysegs > 0) {
    const dim3 gl(l / 64, ysegs, R), gf(f / 64, ysegs, R);
    LMOE_TRY((segment_transpose<TI, TI>(gl, (const TI*)w.dout, l, 0, l, w.counts, w.offsets, nullptr, p.k,
                                        w.kr_off, w.kr_len, (TI*)w.doutT, st)));
    LMOE_TRY((segment_transpose<TI, TI>(gf, (const TI*)w.hs, f, 0, f, w.counts, w.offsets, nullptr, p.k,
                                        w.kr_off, w.kr_len, (TI*)w.hT, st)));
    LMOE_TRY((segment_transpose<TI, TI>(gf, (const TI*)w.dgu, 2 * f, 0, f, w.counts, w.offsets, nullptr, p.k,
                                        w.kr_off, w.kr_len, (TI*)w.dgT, st)));
    LMOE_TRY((segment_transpose<TI, TI>(gf, (const TI*)w.dgu, 2 * f, f, f, w.counts, w.offsets, nullptr, p.k,
                                        w.kr_off, w.kr_len, (TI*)w.duT, st)));
    LMOE_TRY((segment_transpose<TZ, TI>(gl, (const TZ*)z, l, 0, l, w.counts, w.offsets, w.order, p.k,
                                        w.kr_off, w.kr_len, (TI*)w.zT, st)));
  }
  auto batched = [&](const char* a, int M, const char* b, int N, void* out) {
    GemmArgs g = base_args(dm);
    g.M = M;
    g.N = N;
    g.K = 64;  // per-batch K comes from kr_len
    g.a = a;
    g.b0 = b;
    g.nb_rows = N;
    g.kr_off = w.kr_off;
    g.kr_len = w.kr_len;
    g.nbatch = R;
    g.out = (char*)out;
    g.ldo = (int64_t)N * es;
    g.o_batch_stride = (int64_t)M * N * es;
    return g;
  };
  // Every expert's K is its padded pair count (at most C rounded up to 64).
  // Up to kWgradKMax, with 16-bit operands and 256-multiple widths, one
  // workgroup per 256-row strip keeps its A fragments in registers and sweeps
  // the columns; otherwise batched GEMM tiles (128 x 128, 64-byte K steps in
  // a 3-stage ring: 48 KB of LDS, three tiles per compute unit).
  if constexpr (sizeof(TI) == 2 && sizeof(T) == 2) {
    if ((C + 63) / 64 * 64 <= kWgradKMax && l % kWgradStrip == 0 && f % kWgradStrip == 0) {
      auto strips = [&](const void* a, int M, const void* b, int N, void* out) -> lmoe_status {
        wgrad_kernel<TI, T><<<(unsigned)((int64_t)R * (M / kWgradStrip)), kWgradThreads, 0, st>>>(
            (const TI*)a, (const TI*)b, w.kr_off, w.kr_len, M, N, (T*)out);
        LMOE_HIP(hipGetLastError());
        return LMOE_OK;
      };
      LMOE_TRY(strips(w.doutT, l, w.hT, f, dw_o));
      LMOE_TRY(strips(w.dgT, f, w.zT, l, dw_g));
      LMOE_TRY(strips(w.duT, f, w.zT, l, dw_u));
      return LMOE_OK;
    }
  }
  constexpr Tile kWgradGemmTile = TILE_M2;
  LMOE_TRY((gemm<TI, TI, T, A_KBATCH, B_SINGLE, E_STORE>(batched(w.doutT, l, w.hT, f, dw_o), kWgradGemmTile, st)));
  LMOE_TRY((gemm<TI, TI, T, A_KBATCH, B_SINGLE, E_STORE>(batched(w.dgT, f, w.zT, l, dw_g), kWgradGemmTile, st)));
  LMOE_TRY((gemm<TI, TI, T, A_KBATCH, B_SINGLE, E_STORE>(batched(w.duT, f, w.zT, l, dw_u), kWgradGemmTile, st)));
  return LMOE_OK;
}

// Routed-block backward (see latentmoe_routed_backward).  T: storage type of
// the weights and the weight gradients; TI: intermediate type; TZ: type of z.
template <typename T, typename TI, typename TZ, typename TDZ>
lmoe_status run_routed_backward(const Plan& p, const lmoe_dims* dm, const void* z, const int32_t* ids,
                                const float* probs, const void* w_g, const void* w_u, const void* w_o,
                                const float* du, void* dz, int64_t ld_dz, float* dprobs, void* dw_g,
                                void* dw_u, void* dw_o, const RoutedBwdWs& w, hipStream_t st) {
  int C = 0;
  LMOE_TRY((routed_recompute<T, TI, TZ>(p, dm, z, ids, w_g, w_u, w_o, w, &C, st)));
  return routed_gradients<T, TI, TZ, TDZ>(p, dm, z, probs, w_g, w_u, w_o, du, dz, ld_dz, dprobs, dw_g, dw_u,
                                          dw_o, w, C, st);
}

// Whole-layer backward (see latentmoe_backward).  T: storage type; TI: intermediate type.
template <typename T, typename TI>
lmoe_status run_layer_backward(const Plan& p, const lmoe_dims* dm, const lmoe_weights* W, const void* x,
                               const int32_t* ids, const float* probs, const void* dy, float* dx,
                               const lmoe_grads* G, const LayerBwdWs& w, hipStream_t st) {
  const int64_t N = p.N, es = sizeof(T), ei = sizeof(TI);
  const int d = p.d, l = p.l, R = p.R;
  const int nsf = (int)w.nsf, rpad = (int)w.rpad;
  const int64_t kcat = w.kcat, npad = w.npad;
  auto blocks = [](int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); };
  auto dense = [&](const void* a, int64_t lda, int M, const void* b, int64_t ldb, int Ncols, int K, void* out,
                   int64_t ldo) {
    GemmArgs g = base_args(dm);
    g.M = M;
    g.N = Ncols;
    g.K = K;
    g.a = (const char*)a;
    g.lda = lda;
    g.b0 = (const char*)b;
    g.ldb = ldb;
    g.nb_rows = Ncols;
    g.out = (char*)out;
    g.ldo = ldo;
    return g;
  };
  // ---- recompute the forward quantities the gradients need
  LMOE_TRY((gemm<T, T, TI, A_DENSE, B_SINGLE, E_STORE>(dense(x, d * es, (int)N, W->w_down, d * es, l, d, w.z, l * ei),
                                                       dense_tile(N, l, false), st)));
  LMOE_TRY((gemm<T, T, float, A_DENSE, B_SINGLE, E_STORE>(
      dense(x, d * es, (int)N, W->w_router, d * es, R, d, w.logits, (int64_t)R * 4), dense_tile(N, R, false), st)));
  // the routed block's forward quantities (pre-activations, hidden, expert
  // outputs), kept for its gradients below
  const RoutedBwdWs& rw = w.rw;
  int C = 0;
  LMOE_TRY((routed_recompute<T, TI, TI>(p, dm, w.z, ids, W->w_g, W->w_u, W->w_o, rw, &C, st)));
  // u = sum over the token's pairs (slot order) of p o, then RMSNorm(u)
  pair_sum_kernel<float><<<(unsigned)N, 256, 0, st>>>(rw.o, rw.inv, p.k, l, probs, w.u, l);
  LMOE_HIP(hipGetLastError());
  combine_rmsnorm_kernel<float, TI><<<(unsigned)N, 256, 0, st>>>(w.u, 1, l, nullptr, W->rms_w, dm->rms_eps,
                                                                 (TI*)w.rn, l);
  LMOE_HIP(hipGetLastError());
  if (nsf > 0) {
    LMOE_TRY((gemm<T, T, float, A_DENSE, B_SINGLE, E_STORE>(
        dense(x, d * es, (int)N, W->sh_g, d * es, nsf, d, w.ag, (int64_t)nsf * 4), dense_tile(N, nsf, false), st)));
    LMOE_TRY((gemm<T, T, float, A_DENSE, B_SINGLE, E_STORE>(
        dense(x, d * es, (int)N, W->sh_u, d * es, nsf, d, w.au, (int64_t)nsf * 4), dense_tile(N, nsf, false), st)));
    situ_hidden_kernel<TI><<<blocks(N * nsf), 256, 0, st>>>(w.ag, w.au, N * nsf, dm->beta1, dm->beta2, (TI*)w.hs);
    LMOE_HIP(hipGetLastError());
  }
  // ---- step 5 backward: dr = dy W_up, dh_shared = dy [S_o^j], RMSNorm backward
  LMOE_TRY(transpose_batched<T>((const T*)W->w_up, 0, l, d, l, (T*)w.w_upT, 0, d, 0, 1, nullptr, st));
  LMOE_TRY((gemm<T, T, float, A_DENSE, B_SINGLE, E_STORE>(dense(dy, d * es, (int)N, w.w_upT, d * es, l, d, w.dr,
                                                                (int64_t)l * 4),
                                                          dense_tile(N, l, false), st)));
  rmsnorm_backward_kernel<<<(unsigned)N, 256, 0, st>>>(w.u, w.dr, W->rms_w, l, dm->rms_eps, w.du, w.rho);
  LMOE_HIP(hipGetLastError());
  {
    const int nch = (int)((N + w.rms_chunk - 1) / w.rms_chunk);
    rmsnorm_wgrad_partial_kernel<<<dim3((l + 255) / 256, nch), 256, 0, st>>>(w.u, w.dr, w.rho, N, w.rms_chunk, l,
                                                                              w.rms_part);
    LMOE_HIP(hipGetLastError());
    rmsnorm_wgrad_final_kernel<<<(unsigned)((l + 255) / 256), 256, 0, st>>>(w.rms_part, nch, l, G->rms_w);
    LMOE_HIP(hipGetLastError());
  }
  if (nsf > 0) {
    LMOE_TRY(transpose_batched<T>((const T*)W->sh_o, (int64_t)d * p.fs, p.fs, d, p.fs, (T*)w.shoT,
                                   (int64_t)p.fs * d, d, 0, p.ns, nullptr, st));
    LMOE_TRY((gemm<T, T, float, A_DENSE, B_SINGLE, E_STORE>(dense(dy, d * es, (int)N, w.shoT, d * es, nsf, d,
                                                                  w.dhs, (int64_t)nsf * 4),
                                                            dense_tile(N, nsf, false), st)));
    situ_backward_kernel<TI><<<(unsigned)std::min<int64_t>(N, 65536), 256, 0, st>>>(
        w.dhs, w.ag, w.au, N, nsf, dm->beta1, dm->beta2, (TI*)w.dcat, kcat, l + rpad);
    LMOE_HIP(hipGetLastError());
  }
  // ---- step 3 backward (routed block) -> dz into dcat[:, :l], dprobs
  LMOE_TRY((routed_gradients<T, TI, TI, TI>(p, dm, w.z, probs, W->w_g, W->w_u, W->w_o, w.du, w.dcat, kcat,
                                            w.dprobs, G->w_g, G->w_u, G->w_o, rw, C, st)));
  // ---- step 2 backward -> dl into dcat[:, l:l+rpad]
  router_backward_kernel<TI><<<(unsigned)((N + 3) / 4), 256, 0, st>>>(w.logits, ids, w.dprobs, N, R, p.k, rpad,
                                                                      (TI*)w.dcat + l, kcat);
  LMOE_HIP(hipGetLastError());
  // ---- dx = [dz | dl | dg_sh | du_sh] [W_down ; W_r ; S_g ; S_u]  (K-segmented, transposed weights)
  LMOE_TRY(transpose_batched<T>((const T*)W->w_down, 0, d, l, d, (T*)w.w_downT, 0, l, 0, 1, nullptr, st));
  zero_words_kernel<<<256, 256, 0, st>>>((uint32_t*)w.w_rT, (int64_t)d * rpad * es / 4);
  LMOE_HIP(hipGetLastError());
  LMOE_TRY(transpose_batched<T>((const T*)W->w_router, 0, d, R, d, (T*)w.w_rT, 0, rpad, 0, 1, nullptr, st));
  GemmArgs f = base_args(dm);
  f.M = (int)N;
  f.N = d;
  f.K = (int)kcat;
  f.a = w.dcat;
  f.lda = kcat * ei;
  f.nb_rows = d;
  f.nseg = 0;
  auto seg = [&](const char* base, int64_t kseg, int64_t k0) {
    f.seg_base[f.nseg] = base;
    f.seg_ld[f.nseg] = kseg * es;
    f.seg_kt0[f.nseg] = (int)(k0 * ei / kSegUnit);
    ++f.nseg;
  };
  seg(w.w_downT, l, 0);
  seg(w.w_rT, rpad, l);
  if (nsf > 0) {
    LMOE_TRY(transpose_batched<T>((const T*)W->sh_g, 0, d, nsf, d, (T*)w.sgT, 0, nsf, 0, 1, nullptr, st));
    LMOE_TRY(transpose_batched<T>((const T*)W->sh_u, 0, d, nsf, d, (T*)w.suT, 0, nsf, 0, 1, nullptr, st));
    seg(w.sgT, nsf, l + rpad);
    seg(w.suT, nsf, l + rpad + nsf);
  }
  f.seg_kt0[f.nseg] = (int)(kcat * ei / kSegUnit);
  f.out = (char*)dx;
  f.ldo = (int64_t)d * 4;
  LMOE_TRY((gemm<TI, T, float, A_DENSE, B_KSEG, E_STORE>(f, dense_tile(N, d, false), st)));
  // ---- dense weight gradients: products over tokens (K = npad, zero-padded transposes)
  set_ints_kernel<<<1, 64, 0, st>>>(w.seg, (int32_t)N, 0, 0, (int32_t)npad);
  LMOE_HIP(hipGetLastError());
  const int32_t *cnt = w.seg, *off = w.seg + 1, *kro = w.seg + 2, *krl = w.seg + 3;
  const unsigned ny = (unsigned)(npad / 64);
  auto tr = [&](auto src_c, int64_t ld_src, int64_t col0, int ncols, char* out) -> lmoe_status {
    using TS = std::remove_const_t<std::remove_pointer_t<decltype(src_c)>>;
    return segment_transpose<TS, TI>(dim3((ncols + 63) / 64, ny, 1), src_c, ld_src, (int)col0, ncols, cnt, off,
                                     nullptr, 1, kro, krl, (TI*)out, st);
  };
  LMOE_TRY(tr((const T*)dy, d, 0, d, w.dyT));
  LMOE_TRY(tr((const TI*)w.rn, l, 0, l, w.rnT));
  LMOE_TRY(tr((const TI*)w.dcat, kcat, 0, (int)kcat, w.dcatT));
  LMOE_TRY(tr((const T*)x, d, 0, d, w.xT));
  const int64_t ldt = npad * ei;
  auto wgrad = [&](const char* a, int M, const char* b, int Ncols, void* out) {
    return gemm<TI, TI, T, A_DENSE, B_SINGLE, E_STORE>(dense(a, ldt, M, b, ldt, Ncols, (int)npad, out,
                                                             (int64_t)Ncols * es),
                                                       dense_tile(M, Ncols, false), st);
  };
  LMOE_TRY(wgrad(w.dyT, d, w.rnT, l, G->w_up));
  LMOE_TRY(wgrad(w.dcatT, l, w.xT, d, G->w_down));
  LMOE_TRY(wgrad(w.dcatT + (int64_t)l * ldt, R, w.xT, d, G->w_router));
  if (nsf > 0) {
    LMOE_TRY(tr((const TI*)w.hs, nsf, 0, nsf, w.hsT));
    for (int j = 0; j < p.ns; ++j)
      LMOE_TRY(wgrad(w.dyT, d, w.hsT + (int64_t)j * p.fs * ldt, p.fs, (char*)G->sh_o + (int64_t)j * d * p.fs * es));
    LMOE_TRY(wgrad(w.dcatT + (int64_t)(l + rpad) * ldt, nsf, w.xT, d, G->sh_g));
    LMOE_TRY(wgrad(w.dcatT + (int64_t)(l + rpad + nsf) * ldt, nsf, w.xT, d, G->sh_u));
  }
  return LMOE_OK;
}

// Shared experts' gate/up GEMM with the SiTU epilogue -> hcat[:, :n_s f_s].
template <typename T, typename TI>
lmoe_status run_shared(const Plan& p, const lmoe_dims* dm, const lmoe_weights* W, const void* x,
                       const ForwardWs& w, hipStream_t st) {
  GemmArgs s = base_args(dm);
  s.M = (int)p.N;
  s.N = p.ns * p.fs;
  s.K = p.d;
  s.a = (const char*)x;
  s.lda = (int64_t)p.d * p.es;
  s.b0 = (const char*)W->sh_g;
  s.b1 = (const char*)W->sh_u;
  s.ldb = (int64_t)p.d * p.es;
  s.nb_rows = p.ns * p.fs;
  s.out = w.hcat;
  s.ldo = p.ldh * p.es;
  return gemm<T, T, TI, A_DENSE, B_DUAL, E_SITU>(s, dense_tile(p.N, s.N, true), st);
}

// T: storage type (x, weights, y); TI: intermediate type of z, h and the
// normalised u (fp32 with fp32 storage, fp16 with bf16 storage).
template <typename T, typename TI>
lmoe_status run_forward(const Plan& p, const lmoe_dims* dm, const lmoe_weights* W, const void* x,
                        void* y, int32_t* ids, float* probs, int32_t* counts, const ForwardWs& w,
                        hipStream_t st, hipEvent_t* ev) {
  int step = 0;
  auto mark = [&]() -> lmoe_status {  // optional per-step timing events
    if (ev) LMOE_HIP(hipEventRecord(ev[step], st));
    ++step;
    return LMOE_OK;
  };
  LMOE_TRY(mark());
  // The shared experts depend on x only.  For small batches (whose GEMMs
  // leave most CUs idle) and without timing marks they run on a second
  // stream, next to steps 1-3 and the routed experts; the merge GEMM waits
  // for both.  Large batches fill the chip with each GEMM alone, and their
  // 128-132 KB LDS tiles cannot share a CU, so there they run in order.
  hipStream_t side = st;
  struct Events {
    hipEvent_t fork = nullptr, join = nullptr;
    ~Events() {
      if (fork) (void)hipEventDestroy(fork);
      if (join) (void)hipEventDestroy(join);
    }
  } evs;
  const bool overlap = ev == nullptr && p.ns > 0 && p.N <= kOverlapMaxTokens;
  if (overlap) {
    LMOE_TRY(side_stream(&side));
    LMOE_HIP(hipEventCreateWithFlags(&evs.fork, hipEventDisableTiming));
    LMOE_HIP(hipEventCreateWithFlags(&evs.join, hipEventDisableTiming));
    LMOE_HIP(hipEventRecord(evs.fork, st));
    LMOE_HIP(hipStreamWaitEvent(side, evs.fork, 0));
    LMOE_TRY((run_shared<T, TI>(p, dm, W, x, w, side)));
    LMOE_HIP(hipEventRecord(evs.join, side));
  }
  // 1. z = W_down x
  GemmArgs a = base_args(dm);
  a.M = (int)p.N;
  a.N = p.l;
  a.K = p.d;
  a.a = (const char*)x;
  a.lda = (int64_t)p.d * p.es;
  a.b0 = (const char*)W->w_down;
  a.ldb = (int64_t)p.d * p.es;
  a.nb_rows = p.l;
  a.out = w.z;
  a.ldo = (int64_t)p.l * p.es;
  a.part = w.part;
  a.part_bytes = w.part_bytes;
  LMOE_TRY((gemm<T, T, TI, A_DENSE, B_SINGLE, E_STORE>(a, dense_tile(p.N, p.l, false), st)));
  LMOE_TRY(mark());
  // 2. routing
  LMOE_TRY(run_route<T>(p, dm, x, W->w_router, W->bias, ids, probs, w.logits, st, false, w.part, w.part_bytes));
  LMOE_TRY(mark());
  // 3a. dispatch bookkeeping
  LMOE_TRY(run_dispatch(p, ids, w.chunk_hist, w.chunk_bad, counts, w.offsets, w.order, w.meta, st));
  LMOE_TRY(mark());
  // 4. shared experts gate/up -> h_shared = hcat[:, :n_s f_s] (in order when timed)
  if (!overlap && p.ns > 0) LMOE_TRY((run_shared<T, TI>(p, dm, W, x, w, st)));
  LMOE_TRY(mark());
  // 3b. routed experts straight from z -> slots
  LMOE_TRY((run_experts<TI, T, TI, A_GATHER>(p, dm, w.z, 0, counts, w.offsets, w.order, probs, W->w_g,
                                     W->w_u, W->w_o, w.tile_list, w.meta, w.h, w.slots, st,
                                     ev ? &mark : nullptr)));
  LMOE_TRY(mark());
  // 5a. u = sum of slots, RMSNorm -> hcat[:, n_s f_s:]
  combine_rmsnorm_kernel<TI, TI><<<(unsigned)p.N, 256, 0, st>>>(
      (const TI*)w.slots, p.k, p.l, nullptr, W->rms_w, dm->rms_eps,
      (TI*)(w.hcat + (int64_t)p.ns * p.fs * p.es), p.ldh);
  LMOE_HIP(hipGetLastError());
  LMOE_TRY(mark());
  if (overlap) LMOE_HIP(hipStreamWaitEvent(st, evs.join, 0));
  // 5b. y = [h_shared | RMSNorm(u)] [sh_o_0 | ... | sh_o_{n_s-1} | W_up]^T
  GemmArgs f = base_args(dm);
  f.M = (int)p.N;
  f.N = p.d;
  f.K = (int)p.ldh;
  f.a = w.hcat;
  f.lda = p.ldh * p.es;
  f.nb_rows = p.d;
  const int kt_per_fs = p.fs * p.es / kSegUnit;
  f.nseg = p.ns + 1;
  for (int j = 0; j < p.ns; ++j) {
    f.seg_base[j] = (const char*)W->sh_o + (int64_t)j * p.d * p.fs * p.es;
    f.seg_ld[j] = (int64_t)p.fs * p.es;
    f.seg_kt0[j] = j * kt_per_fs;
  }
  f.seg_base[p.ns] = (const char*)W->w_up;
  f.seg_ld[p.ns] = (int64_t)p.l * p.es;
  f.seg_kt0[p.ns] = p.ns * kt_per_fs;
  f.seg_kt0[p.ns + 1] = (int)(p.ldh * p.es / kSegUnit);
  f.out = (char*)y;
  f.ldo = (int64_t)p.d * p.es;
  f.part = w.part;
  f.part_bytes = w.part_bytes;
  LMOE_TRY((gemm<TI, T, T, A_DENSE, B_KSEG, E_STORE>(f, dense_tile(p.N, p.d, false), st)));
  return mark();
}

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* latentmoe_status_string(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LMOE_ERR_UNSUPPORTED: return "unsupported shape";
    case LMOE_ERR_CAPACITY: return "padded capacity smaller than C";
    case LMOE_ERR_WORKSPACE: return "workspace too small";
    case LMOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* latentmoe_last_error(void) { return g_err; }

size_t latentmoe_workspace_bytes(const lmoe_dims* dims, int32_t entry) {
  Plan p;
  if (check_dims(dims, &p) != LMOE_OK) return 0;
  switch (entry) {
    case LMOE_ENTRY_ROUTE: {
      RouteWs w;
      return carve_route(p, nullptr, &w);
    }
    case LMOE_ENTRY_DISPATCH: {
      DispatchWs w;
      return carve_dispatch(p, nullptr, &w);
    }
    case LMOE_ENTRY_EXPERTS: {
      ExpertsWs w;
      return carve_experts(p, nullptr, &w);
    }
    case LMOE_ENTRY_FORWARD: {
      ForwardWs w;
      return carve_forward(p, nullptr, &w);
    }
    case LMOE_ENTRY_ROUTED_BACKWARD: {
      RoutedBwdWs w;
      return carve_routed_backward(p, nullptr, &w);
    }
    case LMOE_ENTRY_BACKWARD: {
      LayerBwdWs w;
      return carve_layer_backward(p, nullptr, &w);
    }
  }
  return 0;
}

lmoe_status latentmoe_route(const lmoe_dims* dims, const void* x, const void* w_router,
                            const float* bias, int32_t* ids, float* probs, float* logits,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (p.N == 0) return LMOE_OK;
  if (!x || !w_router || !ids || !probs) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  if (misaligned({x, w_router, workspace})) return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  RouteWs w{};
  if (!logits) {
    const size_t need = carve_route(p, nullptr, &w);
    if (!workspace || workspace_bytes < need)
      return fail(LMOE_ERR_WORKSPACE, "route needs %zu workspace bytes", need);
    carve_route(p, (char*)workspace, &w);
    logits = w.logits;
  }
  hipStream_t st = launch_stream(stream);
  if (p.bf16) return run_route<bf16_t>(p, dims, x, w_router, bias, ids, probs, logits, st);
  return run_route<float>(p, dims, x, w_router, bias, ids, probs, logits, st);
}

lmoe_status latentmoe_route_softmax(const lmoe_dims* dims, const void* x, const void* w_router,
                                    int32_t* ids, float* probs, float* logits, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (p.N == 0) return LMOE_OK;
  if (!x || !w_router || !ids || !probs) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  if (misaligned({x, w_router, workspace})) return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  RouteWs w{};
  if (!logits) {
    const size_t need = carve_route(p, nullptr, &w);
    if (!workspace || workspace_bytes < need)
      return fail(LMOE_ERR_WORKSPACE, "route needs %zu workspace bytes", need);
    carve_route(p, (char*)workspace, &w);
    logits = w.logits;
  }
  hipStream_t st = launch_stream(stream);
  if (p.bf16) return run_route<bf16_t>(p, dims, x, w_router, nullptr, ids, probs, logits, st, true);
  return run_route<float>(p, dims, x, w_router, nullptr, ids, probs, logits, st, true);
}

size_t latentmoe_router_losses_workspace_bytes(const lmoe_dims* dims) {
  Plan p;
  if (check_dims(dims, &p) != LMOE_OK) return 0;
  const int64_t nblk = (p.N + kLossTokens - 1) / kLossTokens;
  return (size_t)(nblk * p.R + nblk) * sizeof(float) + 256;
}

lmoe_status latentmoe_router_losses(const lmoe_dims* dims, const float* logits, const int32_t* counts,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (!out || !counts || (p.N > 0 && !logits)) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  hipStream_t st = launch_stream(stream);
  const int64_t nblk = (p.N + kLossTokens - 1) / kLossTokens;
  const size_t need = latentmoe_router_losses_workspace_bytes(dims);
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "router losses need %zu workspace bytes", need);
  if (nblk > INT32_MAX) return fail(LMOE_ERR_UNSUPPORTED, "too many tokens");
  float* colsum = (float*)workspace;
  float* lse2 = colsum + nblk * p.R;
  if (nblk > 0) {
    router_stats_kernel<<<(unsigned)nblk, 256, 0, st>>>(logits, p.N, p.R, colsum, lse2);
    LMOE_HIP(hipGetLastError());
  }
  router_losses_kernel<<<1, 1024, 0, st>>>(colsum, lse2, (int)nblk, p.N, p.R, counts, out);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

lmoe_status latentmoe_dispatch(const lmoe_dims* dims, const int32_t* ids, const void* z,
                               int32_t* counts, int32_t* offsets, int32_t* order, void* padded,
                               int64_t capacity, int64_t* C_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (!C_out || !counts || !offsets || (p.N > 0 && (!ids || !order)))
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL argument");
  if (padded && !z) return fail(LMOE_ERR_INVALID_ARGUMENT, "padded output needs z");
  if (capacity < 0) return fail(LMOE_ERR_INVALID_ARGUMENT, "capacity < 0");
  if (misaligned({z, padded, workspace})) return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  hipStream_t st = launch_stream(stream);
  *C_out = 0;
  if (p.N == 0) {
    for (int32_t* v : {counts, offsets}) {  // a fill kernel, no memset node if the caller captures
      zero_words_kernel<<<(unsigned)((p.R + 255) / 256), 256, 0, st>>>((uint32_t*)v, p.R);
      LMOE_HIP(hipGetLastError());
    }
    LMOE_HIP(hipStreamSynchronize(st));
    return LMOE_OK;
  }
  DispatchWs w{};
  const size_t need = carve_dispatch(p, nullptr, &w);
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "dispatch needs %zu workspace bytes", need);
  carve_dispatch(p, (char*)workspace, &w);
  LMOE_TRY(run_dispatch(p, ids, w.chunk_hist, w.chunk_bad, counts, offsets, order, w.meta, st));
  int32_t meta[4] = {0, 0, 0, 0};
  LMOE_HIP(hipMemcpyAsync(meta, w.meta, sizeof(meta), hipMemcpyDeviceToHost, st));
  LMOE_HIP(hipStreamSynchronize(st));
  const int32_t C = meta[0];
  *C_out = C;
  if (meta[2] != 0)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "%d expert ids outside [0, R)", meta[2]);
  if (!padded) return LMOE_OK;
  if (C > capacity) return fail(LMOE_ERR_CAPACITY, "C = %d exceeds capacity %lld", C, (long long)capacity);
  if (C == 0) return LMOE_OK;
  const unsigned rows = (unsigned)((int64_t)p.R * C);
  if (p.bf16)
    padded_gather_kernel<bf16_t><<<rows, 256, 0, st>>>((const bf16_t*)z, p.l, counts, offsets, order,
                                                       p.k, C, (bf16_t*)padded);
  else
    padded_gather_kernel<float><<<rows, 256, 0, st>>>((const float*)z, p.l, counts, offsets, order, p.k,
                                                      C, (float*)padded);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

lmoe_status latentmoe_experts(const lmoe_dims* dims, const void* padded, int64_t C,
                              const int32_t* counts, const int32_t* offsets, const int32_t* order,
                              const float* probs, const void* w_g, const void* w_u,
                              const void* w_o, float* u, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (p.N == 0) return LMOE_OK;
  if (!padded || !counts || !offsets || !order || !probs || !w_g || !w_u || !w_o || !u)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  if (C < 1 || C > p.N) return fail(LMOE_ERR_INVALID_ARGUMENT, "C must be in [1, N]");
  if (misaligned({padded, w_g, w_u, w_o, u, workspace})) return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  ExpertsWs w{};
  const size_t need = carve_experts(p, nullptr, &w);
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "experts needs %zu workspace bytes", need);
  carve_experts(p, (char*)workspace, &w);
  hipStream_t st = launch_stream(stream);
  if (p.bf16)
    LMOE_TRY((run_experts<bf16_t, bf16_t, f16_t, A_PADDED>(p, dims, padded, C, counts, offsets, order, probs, w_g,
                                            w_u, w_o, w.tile_list, w.meta, w.h, w.slots, st)));
  else
    LMOE_TRY((run_experts<float, float, float, A_PADDED>(p, dims, padded, C, counts, offsets, order, probs, w_g, w_u,
                                           w_o, w.tile_list, w.meta, w.h, w.slots, st)));
  if (p.bf16)
    combine_rmsnorm_kernel<f16_t, f16_t><<<(unsigned)p.N, 256, 0, st>>>(
        (const f16_t*)w.slots, p.k, p.l, u, nullptr, 0.f, nullptr, 0);
  else
    combine_rmsnorm_kernel<float, float><<<(unsigned)p.N, 256, 0, st>>>(
        (const float*)w.slots, p.k, p.l, u, nullptr, 0.f, nullptr, 0);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

}  // extern "C"

namespace {
lmoe_status forward_impl(const lmoe_dims* dims, const lmoe_weights* weights, const void* x, void* y,
                         int32_t* ids, float* probs, int32_t* counts, int64_t* C_host,
                         void* workspace, size_t workspace_bytes, void* stream, hipEvent_t* ev) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (C_host) *C_host = 0;
  if (p.N == 0) return LMOE_OK;
  if (!weights || !x || !y || !ids || !probs || !counts)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  const lmoe_weights* W = weights;
  if (!W->w_down || !W->w_router || !W->w_g || !W->w_u || !W->w_o || !W->w_up)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL weight");
  if (p.ns > 0 && (!W->sh_g || !W->sh_u || !W->sh_o))
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL shared expert weight");
  if (misaligned({x, y, W->w_down, W->w_router, W->w_g, W->w_u, W->w_o, W->sh_g, W->sh_u, W->sh_o, W->w_up,
                  workspace}))
    return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  ForwardWs w{};
  const size_t need = carve_forward(p, nullptr, &w);
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "forward needs %zu workspace bytes", need);
  carve_forward(p, (char*)workspace, &w);
  hipStream_t st = launch_stream(stream);
  if (p.bf16) LMOE_TRY((run_forward<bf16_t, f16_t>(p, dims, W, x, y, ids, probs, counts, w, st, ev)));
  else LMOE_TRY((run_forward<float, float>(p, dims, W, x, y, ids, probs, counts, w, st, ev)));
  if (C_host) {
    int32_t C = 0;
    LMOE_HIP(hipMemcpyAsync(&C, w.meta, sizeof(int32_t), hipMemcpyDeviceToHost, st));
    LMOE_HIP(hipStreamSynchronize(st));
    *C_host = C;
  }
  return LMOE_OK;
}

}  // namespace

extern "C" {

lmoe_status latentmoe_forward(const lmoe_dims* dims, const lmoe_weights* weights, const void* x,
                              void* y, int32_t* ids, float* probs, int32_t* counts,
                              int64_t* C_host, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return forward_impl(dims, weights, x, y, ids, probs, counts, C_host, workspace, workspace_bytes,
                      stream, nullptr);
}

lmoe_status latentmoe_forward_timed(const lmoe_dims* dims, const lmoe_weights* weights,
                                    const void* x, void* y, int32_t* ids, float* probs,
                                    int32_t* counts, void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* events, int32_t n_events) {
  if (!events || n_events != LMOE_FORWARD_TIMING_EVENTS)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "need %d events", LMOE_FORWARD_TIMING_EVENTS);
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL event");
  return forward_impl(dims, weights, x, y, ids, probs, counts, nullptr, workspace, workspace_bytes,
                      stream, (hipEvent_t*)events);
}

lmoe_status latentmoe_routed_backward(const lmoe_dims* dims, const void* z, const int32_t* ids,
                                      const float* probs, const void* w_g, const void* w_u,
                                      const void* w_o, const float* du, float* dz, float* dprobs,
                                      void* dw_g, void* dw_u, void* dw_o, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (!w_g || !w_u || !w_o || !dw_g || !dw_u || !dw_o) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL weight");
  if (p.N > 0 && (!z || !ids || !probs || !du || !dz || !dprobs))
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  if (misaligned({z, w_g, w_u, w_o, du, dz, dw_g, dw_u, dw_o, workspace}))
    return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  RoutedBwdWs w{};
  const size_t need = carve_routed_backward(p, nullptr, &w);
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "routed backward needs %zu workspace bytes", need);
  carve_routed_backward(p, (char*)workspace, &w);
  hipStream_t st = launch_stream(stream);
  if (p.N == 0) {  // no pairs: every weight gradient is zero
    const int64_t words = (int64_t)p.R * p.fr * p.l * p.es / 4;
    for (void* d : {dw_g, dw_u, dw_o}) {
      zero_words_kernel<<<1024, 256, 0, st>>>((uint32_t*)d, words);
      LMOE_HIP(hipGetLastError());
    }
    return LMOE_OK;
  }
  if (p.bf16)
    return run_routed_backward<bf16_t, f16_t, bf16_t, float>(p, dims, z, ids, probs, w_g, w_u, w_o, du, dz, p.l,
                                                             dprobs, dw_g, dw_u, dw_o, w, st);
  return run_routed_backward<float, float, float, float>(p, dims, z, ids, probs, w_g, w_u, w_o, du, dz, p.l,
                                                         dprobs, dw_g, dw_u, dw_o, w, st);
}

lmoe_status latentmoe_backward(const lmoe_dims* dims, const lmoe_weights* weights, const void* x,
                               const int32_t* ids, const float* probs, const void* dy, float* dx,
                               const lmoe_grads* grads, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (!weights || !grads) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL weights or gradients");
  const lmoe_weights* W = weights;
  const lmoe_grads* G = grads;
  if (!W->w_down || !W->w_router || !W->w_g || !W->w_u || !W->w_o || !W->w_up)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL weight");
  if (!G->w_down || !G->w_router || !G->w_g || !G->w_u || !G->w_o || !G->w_up || !G->rms_w)
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL gradient");
  if (p.ns > 0 && (!W->sh_g || !W->sh_u || !W->sh_o || !G->sh_g || !G->sh_u || !G->sh_o))
    return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL shared expert weight or gradient");
  if (p.N > 0 && (!x || !ids || !probs || !dy || !dx)) return fail(LMOE_ERR_INVALID_ARGUMENT, "NULL tensor");
  if (misaligned({x, dy, dx, W->w_down, W->w_router, W->w_g, W->w_u, W->w_o, W->sh_g, W->sh_u, W->sh_o, W->w_up,
                  G->w_down, G->w_router, G->w_g, G->w_u, G->w_o, G->sh_g, G->sh_u, G->sh_o, G->w_up, workspace}))
    return fail(LMOE_ERR_INVALID_ARGUMENT, kAlignMsg);
  LayerBwdWs w{};
  const size_t need = carve_layer_backward(p, nullptr, &w);
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "backward needs %zu workspace bytes", need);
  carve_layer_backward(p, (char*)workspace, &w);
  hipStream_t st = launch_stream(stream);
  if (p.N == 0) {  // no tokens: every gradient is zero
    auto zero = [&](void* ptr, int64_t bytes) -> lmoe_status {
      if (bytes <= 0) return LMOE_OK;
      zero_words_kernel<<<1024, 256, 0, st>>>((uint32_t*)ptr, bytes / 4);
      LMOE_HIP(hipGetLastError());
      return LMOE_OK;
    };
    const int64_t es = p.es, nsf = (int64_t)p.ns * p.fs;
    LMOE_TRY(zero(G->w_down, (int64_t)p.l * p.d * es));
    LMOE_TRY(zero(G->w_router, (int64_t)p.R * p.d * es));
    for (void* g : {G->w_g, G->w_u, G->w_o}) LMOE_TRY(zero(g, (int64_t)p.R * p.fr * p.l * es));
    if (nsf > 0)
      for (void* g : {G->sh_g, G->sh_u, G->sh_o}) LMOE_TRY(zero(g, nsf * p.d * es));
    LMOE_TRY(zero(G->w_up, (int64_t)p.d * p.l * es));
    LMOE_TRY(zero(G->rms_w, (int64_t)p.l * 4));
    return LMOE_OK;
  }
  if (p.bf16) return run_layer_backward<bf16_t, f16_t>(p, dims, W, x, ids, probs, dy, dx, G, w, st);
  return run_layer_backward<float, float>(p, dims, W, x, ids, probs, dy, dx, G, w, st);
}

}  // extern "C"
