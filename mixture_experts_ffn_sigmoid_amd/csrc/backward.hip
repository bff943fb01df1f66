// C ABI of the backward of the gfx950 Stable LatentMoE layer: the routed
// block's and the whole layer's gradients (see latentmoe.h).
#include "lmoe_host.h"

namespace {

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
// pre-activations g = z W_g^T and up = z W_u^T (fp32) and the hidden h (TI),
// in sorted pair order.  Returns the capacity C (one host read-back).  T:
// storage type of the weights; TI: intermediate type; TZ: type of z.
template <typename T, typename TI, typename TZ>
lmoe_status routed_recompute(const Plan& p, const lmoe_dims* dm, const void* z, const int32_t* ids,
                             const void* w_g, const void* w_u, const RoutedBwdWs& w, int* C_out,
                             hipStream_t st) {
  const int64_t P = p.pairs;
  const int f = p.fr, l = p.l, R = p.R;
  const int64_t es = sizeof(T), ei = sizeof(TI);
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
  // 2. pre-activations of every pair, g = z W_g^T and up = z W_u^T (type TI,
  // sorted rows), and the hidden h from one dual (gate, up) product
  const int64_t ez = sizeof(TZ);
  GemmArgs g = grouped(z, l * ez, w_g, l * es, (int64_t)f * l * es, f, l, w.hs, (int64_t)f * ei);
  g.b1 = (const char*)w_u;
  g.pre_g = w.g;
  g.pre_u = w.up;
  g.pre_ld = (int64_t)f * ei;
  return gemm<TZ, T, TI, A_GATHER, B_DUAL, E_PRE>(g, tile, st);
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
  // 3b-4. v = W_o^T du per pair (du's row times the pair's W_o; 16-bit
  // weights read as stored, K-major: K-row k of W_o[e] is its latent row k;
  // fp32 ones through a transposed copy W_o^T [R, f, l]).  Then
  // dprobs = <du, W_o h> = <v, h>, the hidden's gradient dh = p v (applied
  // by the SiTU backward) and dout = p du (for dW_o): the expert outputs
  // themselves are not needed.
  if constexpr (sizeof(T) == 2) {
    convert_kernel<TI><<<blocks((int64_t)p.N * l), 256, 0, st>>>(du, (int64_t)p.N * l, (TI*)w.du16);
    LMOE_HIP(hipGetLastError());
    GemmArgs g = grouped(w.du16, l * ei, w_o, f * es, (int64_t)l * f * es, f, l, w.dh, (int64_t)f * 4);
    g.kmaj_split = l;
    LMOE_TRY((gemm<TI, T, float, A_GATHER, B_KMAJOR, E_STORE>(g, tile, st)));
  } else {
    LMOE_TRY(transpose_batched<T>((const T*)w_o, (int64_t)l * f, f, l, f, (T*)w.w_oT, (int64_t)f * l, l, 0, R,
                                   w.counts, st));
    LMOE_TRY((gemm<float, T, float, A_GATHER, B_SINGLE, E_STORE>(
        grouped(du, l * 4, w.w_oT, l * es, (int64_t)f * l * es, f, l, w.dh, (int64_t)f * 4), tile, st)));
  }
  pair_vh_kernel<TI><<<(unsigned)P, 256, 0, st>>>(w.dh, (const TI*)w.hs, du, probs, w.order, p.k, l, f, dprobs,
                                                  (TI*)w.dout, w.sp);
  LMOE_HIP(hipGetLastError());
  situ_backward_kernel<TI, TI><<<(unsigned)std::min<int64_t>(P, 65536), 256, 0, st>>>(
      w.dh, (const TI*)w.g, (const TI*)w.up, P, f, dm->beta1, dm->beta2, (TI*)w.dgu, 2 * (int64_t)f, 0, w.sp);
  LMOE_HIP(hipGetLastError());
  // 5. dz rows = [dg | du] [W_g ; W_u] (K = 2f: W_g's rows, then W_u's; type
  // TI), summed per token in fp32
  TI* dzrows = (TI*)w.o;
  if constexpr (sizeof(T) == 2) {
    GemmArgs g = grouped(w.dgu, 2 * f * ei, w_g, l * es, (int64_t)f * l * es, l, 2 * f, dzrows, (int64_t)l * ei);
    g.b1 = (const char*)w_u;
    g.kmaj_split = f;
    LMOE_TRY((gemm<TI, T, TI, A_SORTED, B_KMAJOR, E_STORE>(g, tile, st)));
  } else {
    LMOE_TRY(transpose_batched<T>((const T*)w_g, (int64_t)f * l, l, f, l, (T*)w.w_guT, (int64_t)l * 2 * f,
                                   2 * f, 0, R, w.counts, st));
    LMOE_TRY(transpose_batched<T>((const T*)w_u, (int64_t)f * l, l, f, l, (T*)w.w_guT, (int64_t)l * 2 * f,
                                   2 * f, f, R, w.counts, st));
    LMOE_TRY((gemm<TI, T, TI, A_SORTED, B_SINGLE, E_STORE>(
        grouped(w.dgu, 2 * f * ei, w.w_guT, 2 * f * es, (int64_t)l * 2 * f * es, l, 2 * f, dzrows,
                (int64_t)l * ei),
        tile, st)));
  }
  pair_sum_kernel<TI, TDZ><<<(unsigned)p.N, 256, 0, st>>>(dzrows, w.inv, p.k, l, (TDZ*)dz, ld_dz);
  LMOE_HIP(hipGetLastError());
  // 6. weight gradients: per expert, products over its pairs.  Up to
  // kWgradKMax pairs per expert, with 16-bit operands and 256-multiple
  // widths, one workgroup per 256-row strip reads the pair rows as stored
  // (K-major), keeps its A fragments in registers and sweeps the columns;
  // otherwise the pair rows are transposed into zero-padded per-expert
  // segments for batched GEMM tiles (128 x 128, 64-byte K steps in a 3-stage
  // ring: 48 KB of LDS, three tiles per compute unit).
  if constexpr (sizeof(TI) == 2 && sizeof(T) == 2 && sizeof(TZ) == 2) {
    if ((C + 63) / 64 * 64 <= kWgradKMax && l % kWgradStrip == 0 && f % kWgradStrip == 0) {
      auto strips = [&](const TI* a, int64_t lda, int M, const auto* b, int64_t ldb, const int32_t* b_order, int N,
                        void* out) -> lmoe_status {
        wgrad_kernel<<<(unsigned)((int64_t)R * (M / kWgradStrip)), kWgradThreads, 0, st>>>(
            a, lda, b, ldb, b_order, p.k, w.counts, w.offsets, M, N, (T*)out);
        LMOE_HIP(hipGetLastError());
        return LMOE_OK;
      };
      const TI* dgu = (const TI*)w.dgu;
      LMOE_TRY(strips((const TI*)w.dout, l * ei, l, (const TI*)w.hs, f * ei, nullptr, f, dw_o));
      LMOE_TRY(strips(dgu, 2 * f * ei, f, (const TZ*)z, l * (int64_t)sizeof(TZ), w.order, l, dw_g));
      LMOE_TRY(strips(dgu + f, 2 * f * ei, f, (const TZ*)z, l * (int64_t)sizeof(TZ), w.order, l, dw_u));
      return LMOE_OK;
    }
  }
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
  LMOE_TRY((routed_recompute<T, TI, TZ>(p, dm, z, ids, w_g, w_u, w, &C, st)));
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
  // the routed block's forward quantities (pre-activations, hidden), kept
  // for its gradients below
  const RoutedBwdWs& rw = w.rw;
  int C = 0;
  LMOE_TRY((routed_recompute<T, TI, TI>(p, dm, w.z, ids, W->w_g, W->w_u, rw, &C, st)));
  // u and RMSNorm(u) formed as the forward forms them: the down product
  // writes each pair's p-weighted output (type TI) into the token's slot row
  // (rw.o's space, free until the dz rows), the slots are summed in slot
  // order into u (fp32, kept for the RMSNorm backward) and normalised
  {
    const Tile tile = routed_tile(p);
    GemmArgs g = routed_grouped(p, dm, rw, rw.hs, (int64_t)p.fr * ei, W->w_o, (int64_t)p.fr * es,
                                (int64_t)l * p.fr * es, l, p.fr, rw.o, (int64_t)l * ei);
    g.probs = probs;
    LMOE_TRY((gemm<TI, T, TI, A_SORTED, B_SINGLE, E_SLOTS>(g, tile == TILE_V ? TILE_V2 : tile, st)));
  }
  combine_rmsnorm_kernel<TI, TI><<<(unsigned)N, 256, 0, st>>>((const TI*)rw.o, p.k, l, w.u, W->rms_w,
                                                              dm->rms_eps, (TI*)w.rn, l, nullptr);
  LMOE_HIP(hipGetLastError());
  if (nsf > 0) {  // the shared pre-activations and hidden (type TI) from one dual (gate, up) product
    GemmArgs g = dense(x, d * es, (int)N, W->sh_g, d * es, nsf, d, w.hs, (int64_t)nsf * ei);
    g.b1 = (const char*)W->sh_u;
    g.pre_g = w.ag;
    g.pre_u = w.au;
    g.pre_ld = (int64_t)nsf * ei;
    LMOE_TRY((gemm<T, T, TI, A_DENSE, B_DUAL, E_PRE>(g, dense_tile(N, nsf, true), st)));
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
    situ_backward_kernel<TI, TI><<<(unsigned)std::min<int64_t>(N, 65536), 256, 0, st>>>(
        w.dhs, (const TI*)w.ag, (const TI*)w.au, N, nsf, dm->beta1, dm->beta2, (TI*)w.dcat, kcat, l + rpad, nullptr);
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
  f.part = w.tpart;  // partial blocks for the tail split (NULL unless dx runs on 256 x 256 tiles)
  f.part_bytes = w.tpart_bytes;
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

}  // namespace

extern "C" {

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
