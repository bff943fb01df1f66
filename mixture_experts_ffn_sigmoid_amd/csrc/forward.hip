// C ABI of the gfx950 Stable LatentMoE forward: the entry points of
// routing, dispatch, the routed experts and the whole layer, with their
// launch sequences (see latentmoe.h).
#include "lmoe_host.h"

char* lmoe::error_buffer() {
  thread_local char buf[kErrorBufferBytes] = "";
  return buf;
}

namespace {

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

// Routed experts: tile list, gate/up grouped GEMM with the SiTU epilogue into
// h (sorted pair rows, type TH), down grouped GEMM with the p-weighted slot
// epilogue.  TA: type of the gathered rows, TW: weight storage type.
template <typename TA, typename TW, typename TH, int AM, typename Mark = lmoe_status (*)()>
lmoe_status run_experts(const Plan& p, const lmoe_dims* dm, const void* a_src, int64_t cap,
                        const int32_t* counts, const int32_t* offsets, const int32_t* order,
                        const float* probs, const void* w_g, const void* w_u, const void* w_o,
                        int32_t* tile_list, int32_t* meta, char* h, char* slots, hipStream_t st,
                        int32_t* range_flag, Mark* mark = nullptr) {
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
  b.cap = AM == A_PADDED ? cap : 0;  // pairs past the padded capacity are dropped
  b.range_flag = range_flag;
  return gemm<TH, TW, TH, A_SORTED, B_SINGLE, E_SLOTS>(b, tile == TILE_V ? TILE_V2 : tile, st);
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
                        hipStream_t st, hipEvent_t* ev, bool one_stream) {
  int step = 0;
  auto mark = [&]() -> lmoe_status {  // optional per-step timing events
    if (ev) LMOE_HIP(hipEventRecord(ev[step], st));
    ++step;
    return LMOE_OK;
  };
  LMOE_TRY(mark());
  // meta: C, tile count, bad ids, range flag -- all cleared (a fill kernel,
  // not a memset node, so a captured forward replays correctly)
  set_ints_kernel<<<1, 64, 0, st>>>(w.meta, 0, 0, 0, 0);
  LMOE_HIP(hipGetLastError());
  // The shared experts depend on x only.  For small products (whose GEMMs
  // leave CUs idle; shared_overlaps) and without timing marks they run on a
  // second stream, next to steps 1-3 and the routed experts; the merge GEMM
  // waits for both.  Large ones fill the chip with each GEMM alone, and their
  // 128-144 KB LDS tiles cannot share a CU, so there they run in order.
  hipStream_t side = st;
  struct Events {
    hipEvent_t fork = nullptr, join = nullptr;
    ~Events() {
      if (fork) (void)hipEventDestroy(fork);
      if (join) (void)hipEventDestroy(join);
    }
  } evs;
  const bool overlap = ev == nullptr && !one_stream && shared_overlaps(p);
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
  a.range_flag = w.meta + kMetaRange;
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
                                     w.meta + kMetaRange, ev ? &mark : nullptr)));
  LMOE_TRY(mark());
  // 5a. u = sum of slots, RMSNorm -> hcat[:, n_s f_s:]
  combine_rmsnorm_kernel<TI, TI><<<(unsigned)p.N, 256, 0, st>>>(
      (const TI*)w.slots, p.k, p.l, nullptr, W->rms_w, dm->rms_eps,
      (TI*)(w.hcat + (int64_t)p.ns * p.fs * p.es), p.ldh, w.meta + kMetaRange);
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

extern "C" {

const char* latentmoe_status_string(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LMOE_ERR_UNSUPPORTED: return "unsupported shape";
    case LMOE_ERR_CAPACITY: return "padded capacity smaller than C";
    case LMOE_ERR_WORKSPACE: return "workspace too small";
    case LMOE_ERR_HIP: return "HIP runtime error";
    case LMOE_ERR_RANGE: return "an fp16 intermediate left fp16's range";
  }
  return "unknown status";
}

const char* latentmoe_last_error(void) { return lmoe::error_buffer(); }

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
                                            w_u, w_o, w.tile_list, w.meta, w.h, w.slots, st, nullptr)));
  else
    LMOE_TRY((run_experts<float, float, float, A_PADDED>(p, dims, padded, C, counts, offsets, order, probs, w_g, w_u,
                                           w_o, w.tile_list, w.meta, w.h, w.slots, st, nullptr)));
  if (p.bf16)
    combine_rmsnorm_kernel<f16_t, f16_t><<<(unsigned)p.N, 256, 0, st>>>(
        (const f16_t*)w.slots, p.k, p.l, u, nullptr, 0.f, nullptr, 0, nullptr);
  else
    combine_rmsnorm_kernel<float, float><<<(unsigned)p.N, 256, 0, st>>>(
        (const float*)w.slots, p.k, p.l, u, nullptr, 0.f, nullptr, 0, nullptr);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}

}  // extern "C"

namespace {
// Fixed device scratch of latentmoe_forward_noalloc (for callers that cannot
// allocate).  Each device holds its own copy for the life of the process; in
// host code the array's name is only a stand-in, so its device address is
// looked up once per device and used everywhere instead.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device.
lmoe_status scratch_ptr(char** out) {
  static std::mutex mu;
  static char* ptrs[kMaxDevices] = {};
  int dev = 0;
  LMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(LMOE_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(LMOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    ptrs[dev] = (char*)ptr;
  }
  *out = ptrs[dev];
  return LMOE_OK;
}

lmoe_status forward_impl(const lmoe_dims* dims, const lmoe_weights* weights, const void* x, void* y,
                         int32_t* ids, float* probs, int32_t* counts, int64_t* C_host,
                         void* workspace, size_t workspace_bytes, void* stream, hipEvent_t* ev,
                         bool one_stream = false) {
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
  if (p.bf16) LMOE_TRY((run_forward<bf16_t, f16_t>(p, dims, W, x, y, ids, probs, counts, w, st, ev, one_stream)));
  else LMOE_TRY((run_forward<float, float>(p, dims, W, x, y, ids, probs, counts, w, st, ev, one_stream)));
  if (C_host) {
    int32_t meta[4] = {0, 0, 0, 0};
    LMOE_HIP(hipMemcpyAsync(meta, w.meta, sizeof(meta), hipMemcpyDeviceToHost, st));
    LMOE_HIP(hipStreamSynchronize(st));
    *C_host = meta[kMetaC];
    if (meta[kMetaRange])
      return fail(LMOE_ERR_RANGE, "an fp16 intermediate (z, a p-weighted expert output or RMSNorm(u)) "
                                  "left fp16's range; y is unspecified");
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

lmoe_status latentmoe_forward_noalloc(const lmoe_dims* dims, const lmoe_weights* weights, const void* x,
                                      void* y, int32_t* ids, float* probs, int32_t* counts, void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (p.N == 0) return LMOE_OK;
  ForwardWs w{};
  const size_t need = carve_forward(p, nullptr, &w);
  if (need > kScratchBytes)
    return fail(LMOE_ERR_WORKSPACE, "the forward needs %zu bytes of scratch; the fixed scratch holds %zu "
                                    "(use latentmoe_forward with a workspace)", need, kScratchBytes);
  char* ws = nullptr;
  LMOE_TRY(scratch_ptr(&ws));
  return forward_impl(dims, weights, x, y, ids, probs, counts, nullptr, ws, kScratchBytes, stream, nullptr,
                      /*one_stream=*/true);
}

lmoe_status latentmoe_forward_check(const lmoe_dims* dims, const void* workspace, size_t workspace_bytes,
                                    void* stream) {
  Plan p;
  LMOE_TRY(check_dims(dims, &p));
  if (p.N == 0) return LMOE_OK;
  ForwardWs w{};
  const size_t need = carve_forward(p, nullptr, &w);
  if (!workspace && need <= kScratchBytes) {  // the fixed scratch of latentmoe_forward_noalloc
    char* ws = nullptr;
    LMOE_TRY(scratch_ptr(&ws));
    workspace = ws;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "forward needs %zu workspace bytes", need);
  carve_forward(p, (char*)workspace, &w);
  hipStream_t st = launch_stream(stream);
  int32_t flag = 0;
  LMOE_HIP(hipMemcpyAsync(&flag, w.meta + kMetaRange, sizeof(flag), hipMemcpyDeviceToHost, st));
  LMOE_HIP(hipStreamSynchronize(st));
  if (flag)
    return fail(LMOE_ERR_RANGE, "an fp16 intermediate (z, a p-weighted expert output or RMSNorm(u)) "
                                "left fp16's range; y is unspecified");
  return LMOE_OK;
}

}  // extern "C"
