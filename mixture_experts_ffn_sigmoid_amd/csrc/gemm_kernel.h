// One MFMA GEMM family for every matrix product of the layer.
//
//   out[m, n] = sum_k A[m, k] * B[n, k]      (A rows and B rows both K-contiguous,
//                                             B stored like an nn.Linear weight)
//
// Workgroup: 4 or 8 wave64s in a WGM x WGN grid; block tile BM x BN;
// K advances KB = 64 or 128 bytes of every tile row per step (KB = 128: each
// row's step is one whole 128-byte cache line, so every L2 request is a full
// line).  Operand tiles go straight from global memory into LDS with
// gfx950's LDS-DMA loads (global_load_lds_dwordx4) through rings of SA (A)
// and SB (B) stages, one barrier per K step.
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
//   A_KBATCH  batched over experts e with their own K = kr_len[e]: A is the
//             row-major [M, kr_len[e]] block at element kr_off[e] * M of a,
//             B the [nb_rows, kr_len[e]] block at kr_off[e] * nb_rows of b0;
//             the product goes to out + e * o_batch_stride
//   B_SINGLE  one weight matrix (per expert in grouped mode)
//   B_DUAL    gate and up matrices interleaved per tile (BN/2 rows of each)
//   B_KSEG    B concatenated along K from up to kMaxSeg separate matrices
//   B_KMAJOR  B stored K-major: element (n, k) at b[k * ldb + n] (a weight used
//             through its transpose), per expert at b_expert_stride; K rows
//             from kmaj_split on come from b1 (two matrices stacked along K).
//             LDS holds the tile as KB/2 K-rows of BN values and the MFMA
//             fragments come out of it through gfx950's transposing LDS read
//             (ds_read_b64_tr_b16); 16-bit operands only
//   E_STORE   plain store (fp32 or storage dtype), masked to valid rows/cols
//   E_SITU    SiTU-GLU hidden of the (gate, up) accumulator pair, stored as OutT
//   E_PRE     E_SITU that also stores the gate and up accumulators themselves
//             (pre-activations at pre_g / pre_u in the hidden's type, rows like
//             the hidden's)
//   E_SLOTS   p-weighted result of sorted pair q written to its own slot row q
// Runtime options (A_DENSE with E_STORE):
//   split K (ksplit > 1): the grid also runs over K slices of kslice steps,
//     each storing an fp32 partial product (summed afterwards by
//     splitk_reduce_kernel);
//   tail split (tsplit > 1, 16-bit operands): only the tiles of each XCD's
//     last, partly filled wave are cut into K slices, so that wave's compute
//     units all have work (fp32 partial blocks summed afterwards by
//     tail_reduce_kernel).
#pragma once

#include "lmoe_common.h"

namespace lmoe {

enum { A_DENSE = 0, A_GATHER = 1, A_PADDED = 2, A_SORTED = 3, A_KBATCH = 4 };
enum { B_SINGLE = 0, B_DUAL = 1, B_KSEG = 2, B_KMAJOR = 3 };
enum { E_STORE = 0, E_SITU = 1, E_SLOTS = 2, E_PRE = 3 };

constexpr int kMaxSeg = 17;
constexpr int kSegUnit = 64;  // B_KSEG segment boundaries are given in 64-byte units of K

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
  int64_t cap;  // A_PADDED: rows per expert; E_SLOTS: pairs kept per expert (0: all)
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
  int kmaj_split;           // B_KMAJOR: first K row taken from b1 (a multiple of KB / 2)
  int nb_rows;            // rows of each B matrix (clamp)
  int nseg;
  const char* seg_base[kMaxSeg];
  int64_t seg_ld[kMaxSeg];
  int seg_kt0[kMaxSeg + 1];  // first K byte of each segment / kSegUnit (a multiple of KB / kSegUnit)
  // A_KBATCH: per-batch K length and block start (elements; kr_len a multiple of KB / element size)
  const int32_t* kr_off;
  const int32_t* kr_len;
  int nbatch;
  int64_t o_batch_stride;  // bytes (A_KBATCH: per batch; split K: per K slice)
  // split K (A_DENSE with E_STORE, ksplit > 1): slice s covers K steps
  // [s * kslice, min((s + 1) * kslice, K steps)) and stores its partial
  // product at out + s * o_batch_stride
  int ksplit;
  int kslice;
  // tail split (A_DENSE with E_STORE, 16-bit operands, tsplit > 1, m_tiles *
  // n_tiles a multiple of 8): XCD x owns logical tiles [x P, (x + 1) P), P = m_tiles *
  // n_tiles / 8, and takes workgroups 8 j + x, j = 0, 1, ...  Its first twhole
  // tiles run whole (j < twhole); each of its other P - twhole tiles runs as
  // tsplit K slices of kslice steps (j = twhole + tsplit * t + slice), which
  // store their fp32 partial products as BM x BN blocks (tile-local rows and
  // columns, row-major) at tpart, block (tail tile, slice), tail tile
  // x (P - twhole) + t.  Grid: 8 (twhole + tsplit (P - twhole)).
  int tsplit;
  int twhole;
  char* tpart;
  // host side only: fp32 workspace for the K slices of few-row products
  // (NULL: no split)
  char* part;
  int64_t part_bytes;
  // out
  char* out;
  int64_t ldo;  // bytes per output row (E_SLOTS: per slot row)
  const float* probs;
  float beta1, beta2;
  // E_PRE: gate / up pre-activations (type OutT), row stride pre_ld bytes
  char* pre_g;
  char* pre_u;
  int64_t pre_ld;
  // E_STORE / E_SLOTS with fp16 output: set to 1 when a stored value leaves
  // fp16's range (|v| >= 65520 rounds to inf) or is NaN (NULL: no check)
  int32_t* range_flag;
};

// A value whose fp16 rounding is not finite.
__device__ __forceinline__ bool f16_out_of_range(float v) { return !(fabsf(v) < 65520.0f); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; expcnt / lgkmcnt left at "no wait").
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate that also waits for every LDS operation of this wave (lgkmcnt 0).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4); }

// Instruction order of one scheduling region (scheduling-group barriers;
// masks 0x008 MFMA, 0x100 LDS read, 0x020 VMEM read = LDS-DMA): NM MFMAs,
// with the region's NR fragment reads and then its ND DMA instructions (in
// that program order) spread evenly over them; memory operation m follows
// MFMA ceil((m + 1) * NM / (NR + ND)) - 1.
template <int NM, int NR, int ND, int Q = 0>
__device__ __forceinline__ void sched_interleave() {
  constexpr int NMEM = NR + ND;
  if constexpr (NM == 0) {
    if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    if constexpr (ND > 0) __builtin_amdgcn_sched_group_barrier(0x020, ND, 0);
  } else if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int lo = (Q * NMEM + NM - 1) / NM, hi = ((Q + 1) * NMEM + NM - 1) / NM;
    constexpr int r_lo = lo < NR ? lo : NR, r_hi = hi < NR ? hi : NR;
    if constexpr (r_hi > r_lo) __builtin_amdgcn_sched_group_barrier(0x100, r_hi - r_lo, 0);
    constexpr int d = (hi - lo) - (r_hi - r_lo);  // DMA instructions among them
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x020, d, 0);
    sched_interleave<NM, NR, ND, Q + 1>();
  }
}

constexpr int gcd_(int a, int b) { return b == 0 ? a : gcd_(b, a % b); }

// Logical dense tile L -> (M tile, N tile): groups of 4 M tiles sweep all N
// tiles, so neighbouring ids share A and B panels (groups of 4 and 8 measure
// alike; 16 and 32 slower).
__device__ __forceinline__ void dense_tile_coords(int L, int m_tiles, int n_tiles, int* mt, int* nt) {
  constexpr int GM = 4;
  const int group = L / (GM * n_tiles);
  const int first_m = group * GM;
  const int gsize = min(m_tiles - first_m, GM);
  const int in = L - group * GM * n_tiles;
  *mt = first_m + in % gsize;
  *nt = in / gsize;
}

template <typename TA, typename TB, typename OutT, int BM, int BN, int WGM, int WGN, int AMODE,
          int BMODE, int EMODE, int SA, int SB, int KB>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(const GemmArgs args) {
  static_assert(sizeof(TA) == sizeof(TB), "operand element sizes must match");
  constexpr bool kHalf = sizeof(TA) == 2;  // 16-bit operands
  constexpr bool kF16 = __is_same(TA, f16_t);
  constexpr bool kWiden = kF16 && __is_same(TB, bf16_t);
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr bool GROUPED = AMODE == A_GATHER || AMODE == A_PADDED || AMODE == A_SORTED;
  constexpr bool KBATCH = AMODE == A_KBATCH;
  const bool split_all = AMODE == A_DENSE && EMODE == E_STORE && args.ksplit > 1;  // uniform
  // the tail split exists for 16-bit operands only (the fp32 tile has no
  // registers to spare for it)
  constexpr bool kTail = AMODE == A_DENSE && EMODE == E_STORE && kHalf;
  // K step: KB bytes of every tile row = NCH 16-byte chunks.  One LDS-DMA
  // wave instruction moves 64 lanes x 16 bytes = RPI tile rows.
  static_assert(KB == 64 || KB == 128, "K step of 64 or 128 bytes");
  constexpr int ROWB = KB;
  constexpr int NCH = KB / 16, RPI = 64 / NCH;
  constexpr int RSH = 16 / NCH;  // consecutive rows sharing one chunk swizzle
  constexpr int A_INST = BM / RPI, B_INST = BN / RPI;
  constexpr int A_W = A_INST / NW, B_W = B_INST / NW;  // DMA instructions per wave per K step
  // Two LDS rings: SA stages of A rows and SB >= SA stages of B rows (the
  // B ring is deeper where B is the HBM-streamed weight matrix).
  constexpr int kStageA = BM * ROWB, kStageB = BN * ROWB;
  constexpr int RING = SA * kStageA + SB * kStageB;
  constexpr int UNROLL = SA * SB / gcd_(SA, SB);
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "32x32 sub-tiles");
  static_assert(BMODE != B_DUAL || TN % 2 == 0, "dual tile needs gate and up sub-tiles");
  static_assert(BMODE != B_KMAJOR || (kHalf && (1024 % (2 * BN) == 0 || (2 * BN) % 1024 == 0)),
                "K-major B: 16-bit operands, whole K rows per DMA instruction");
  static_assert(A_INST % NW == 0 && B_INST % NW == 0 && BM % RPI == 0 && BN % RPI == 0, "DMA split");
  static_assert(SA >= 2 && SB >= SA && UNROLL <= 8, "ring shape");
  // Dense 16-bit products on two-stage rings take the one-barrier schedule
  // (main loop below); the others the two-phase one.
  constexpr bool k1Bar = SA == 2 && SB == 2 && !GROUPED && kHalf && BMODE != B_KMAJOR;
  // One LDS object for everything (the operand rings and, for E_SLOTS, the
  // slot rows and weights after them): with a second __shared__ object the
  // compiler can no longer tell which object an LDS-DMA writes, and it waits
  // for every DMA in flight (vmcnt 0) before each fragment read.
  constexpr int kSlotBytes = EMODE == E_SLOTS ? BM * 8 : 0;
  __shared__ __attribute__((aligned(1024))) char smem[RING + kSlotBytes];
  char* const ringA = smem;
  char* const ringB = smem + SA * kStageA;

  // the wave index is uniform across the wave: saying so keeps the LDS-DMA
  // destinations (M0) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, lh = lane >> 5;

  int mt, nt, e_batch = 0;
  int tail_id = -1;  // tail split: this workgroup's tail tile (-1: a whole tile)
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
    const int per = args.m_tiles * args.n_tiles;
    int L;
    if (kTail && args.tsplit > 1) {
      const int x = blockIdx.x % 8, j = blockIdx.x / 8, P = per / 8;
      if (j < args.twhole) {
        L = x * P + j;
      } else {
        const int t = (j - args.twhole) / args.tsplit;
        e_batch = (j - args.twhole) % args.tsplit;  // K slice
        tail_id = x * (P - args.twhole) + t;
        L = x * P + args.twhole + t;
      }
    } else {
      const int total = per * (KBATCH ? args.nbatch : split_all ? args.ksplit : 1);
      L = xcd_contiguous_id(blockIdx.x, total);
      if (KBATCH || split_all) {  // batch / K slice
        e_batch = L / per;
        L -= e_batch * per;
      }
    }
    dense_tile_coords(L, args.m_tiles, args.n_tiles, &mt, &nt);
  }
  const bool tail = tail_id >= 0;           // uniform
  const bool split = split_all || tail;     // this workgroup covers one K slice

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
  // K range of this workgroup (A_KBATCH: its batch's range), in elements
  const int kbeg = KBATCH ? args.kr_off[e_batch] : 0;
  const int klen = KBATCH ? args.kr_len[e_batch] : args.K;
  const int64_t lda = KBATCH ? (int64_t)klen * (int64_t)sizeof(TA) : args.lda;  // bytes
  const int64_t ldb = KBATCH ? (int64_t)klen * (int64_t)sizeof(TB) : args.ldb;
  char* const outp = tail ? args.tpart + ((int64_t)tail_id * args.tsplit + e_batch) * (BM * BN * 4)
                          : args.out + ((KBATCH || split_all) ? e_batch * args.o_batch_stride : 0);
  const int kt0 = split ? e_batch * args.kslice : 0;  // first K step of this workgroup's slice
  const int64_t k0b = (int64_t)kt0 * ROWB;
  // E_SLOTS: slot row q and weight p_q of every tile row, fetched now (their
  // latency hides behind the main loop) into LDS outside the operand ring;
  // the main loop's barriers publish them to every wave.  With cap > 0 the
  // pairs at positions >= cap of their expert are dropped: weight 0.
  int* const slot_row = (int*)(smem + RING);              // E_SLOTS: [BM]
  float* const slot_p = (float*)(smem + RING + BM * 4);  // E_SLOTS: [BM]
  if constexpr (EMODE == E_SLOTS) {
    for (int r = tid; r < BM; r += 64 * NW) {
      const int q = r < rows_valid ? args.order[off + m0 + r] : 0;
      const bool kept = r < rows_valid && (args.cap == 0 || m0 + r < args.cap);
      slot_row[r] = q;
      slot_p[r] = kept ? args.probs[q] : 0.f;
    }
  }

  // ---- DMA plan.  For each operand, wave `wave` moves RPI-row blocks
  // wave*X_W + ii of the tile.  Lane l carries tile row r = block*RPI + l/NCH
  // and lands at LDS slot l%NCH of that row; it fetches global 16-byte chunk
  // (l%NCH) ^ sw(r), sw(r) = (r / RSH) % NCH: rows are XOR-swizzled so that
  // the fragment reads of 16 consecutive rows hit 16 distinct 16-byte bank
  // groups.  Rows past the valid range are clamped to the last valid row:
  // every DMA instruction is always issued, which keeps the vmcnt accounting
  // exact.
  auto lane_chunk = [&](int block) -> uint32_t {
    const int r = block * RPI + lane / NCH;
    return (uint32_t)(((lane % NCH) ^ ((r / RSH) % NCH)) * 16);
  };
  constexpr int H = BMODE == B_DUAL ? BN / 2 : BN;  // rows of one B matrix per tile
  const int b_rows_here = min(H, args.nb_rows - nt * H);
  const char* a_base;
  uint32_t a_off[A_W];
  if constexpr (AMODE == A_GATHER) a_base = args.a;
  else if constexpr (AMODE == A_PADDED) a_base = args.a + (int64_t)e * args.cap * args.lda;
  else if constexpr (AMODE == A_SORTED) a_base = args.a + (off + m0) * args.lda;
  else a_base = args.a + (int64_t)kbeg * args.M * (int64_t)sizeof(TA) + (int64_t)m0 * lda + k0b;
#pragma unroll
  for (int ii = 0; ii < A_W; ++ii) {
    const int rr = min((wave * A_W + ii) * RPI + lane / NCH, rows_valid - 1);
    int64_t row = rr;
    if constexpr (AMODE == A_GATHER) row = args.order[off + m0 + rr] / args.top_k;
    // the padded buffer holds an expert's first cap pairs: later pairs
    // (dropped, weighted 0 by the down projection) reread row cap - 1
    if constexpr (AMODE == A_PADDED) row = min(m0 + rr, (int)args.cap - 1);
    a_off[ii] = (uint32_t)(row * lda) + lane_chunk(wave * A_W + ii);
  }
  // B_KMAJOR stage: KE = KB / 2 K-rows of BN values (ROWK bytes, NCR 16-byte
  // chunks each).  DMA instruction `block` of a step fills bytes
  // [block * 1024, +1024) of it: lane l lands at byte l * 16 and fetches the
  // global chunk that belongs there.  Chunks are XOR-swizzled per K-row
  // (kmaj_sw) so that a transposing fragment read, which takes 64 bytes from
  // each of 8 K-rows (0-3 and 8-11 of a 16-row group), hits distinct banks.
  constexpr int KE = KB / 2, ROWK = 2 * BN, NCR = ROWK / 16;
  auto kmaj_sw = [](int r) -> int { return (4 * (r & 3) + 16 * ((r >> 3) & 1)) & (NCR - 1); };
  auto kmaj_pos = [&](int r, int n) -> int {  // LDS byte of value (K-row r, column n)
    return r * ROWK + (((n >> 3) ^ kmaj_sw(r)) << 4) + (n & 7) * 2;
  };
  const char* kmaj_b0 = args.b0 + (int64_t)e * args.b_expert_stride;
  const char* kmaj_b1 = args.b1 ? args.b1 + (int64_t)e * args.b_expert_stride : kmaj_b0;

  const char* b_base[B_W];  // workgroup-uniform
  uint32_t b_off[B_W];      // per lane, K step 0
  uint32_t b_chunk[B_W];    // per lane swizzled chunk offset
  int b_brow[B_W];          // clamped row inside the tile's slice of its matrix
#pragma unroll
  for (int ii = 0; ii < B_W; ++ii) {
    if constexpr (BMODE == B_KMAJOR) {
      const int byte = (wave * B_W + ii) * 1024 + lane * 16;
      const int r = byte / ROWK, c = (byte % ROWK) / 16;
      // first column of the chunk, clamped to the last valid chunk (nb_rows % 8 == 0)
      const int n = min(nt * BN + ((c ^ kmaj_sw(r)) << 3), args.nb_rows - 8);
      b_base[ii] = kmaj_b0;
      b_off[ii] = (uint32_t)((int64_t)r * ldb + (int64_t)n * 2);
      b_chunk[ii] = 0;
      b_brow[ii] = 0;
      continue;
    }
    const int r = (wave * B_W + ii) * RPI + lane / NCH;
    const bool up = BMODE == B_DUAL && r >= H;
    const int br = min(up ? r - H : r, b_rows_here - 1);
    b_brow[ii] = br;
    b_base[ii] = (up ? args.b1 : args.b0) + (int64_t)e * args.b_expert_stride +
                 (int64_t)kbeg * args.nb_rows * (int64_t)sizeof(TB) + (int64_t)nt * H * ldb + k0b;
    b_chunk[ii] = lane_chunk(wave * B_W + ii);
    b_off[ii] = (uint32_t)(br * ldb) + b_chunk[ii];
  }

  // DMA of one K step.  dma_a / dma_b issue instruction ii of this wave for
  // A / B tile kt into `stage`.
  struct BStep {  // per-step B source of B_KSEG (segment lookup)
    const char* base;
    int64_t ld;
  };
  // B_KSEG: the segment of the K step being fetched is kept as a cursor.  The
  // DMA walks B's K steps in order (clamped steps repeat the last one), so the
  // segment table in the kernel arguments is read, and the lanes' row offsets
  // in the segment computed, only when a boundary is passed (b_seek, at the
  // top of a step, outside its scheduling regions).  Searching the table at
  // every step put a scalar load and its wait into every K step.
  int seg_i = 0, seg_next = 0;       // current segment; its end (kSegUnit units)
  const char* seg_row0 = nullptr;    // segment base at this tile's rows, minus the segment's first K byte
  int64_t seg_ldv = 0;
  uint32_t seg_off[BMODE == B_KSEG ? B_W : 1];  // per lane: row and chunk offset in the segment
  auto seg_enter = [&](int i) {
    seg_i = i;
    seg_ldv = args.seg_ld[i];
    seg_row0 = args.seg_base[i] + (int64_t)nt * BN * seg_ldv - (int64_t)args.seg_kt0[i] * kSegUnit;
    seg_next = i + 1 < args.nseg ? args.seg_kt0[i + 1] : 0x7fffffff;
#pragma unroll
    for (int ii = 0; ii < (BMODE == B_KSEG ? B_W : 1); ++ii)
      seg_off[ii] = (uint32_t)(b_brow[ii] * seg_ldv) + b_chunk[ii];
  };
  if constexpr (BMODE == B_KSEG) seg_enter(0);
  auto b_seek = [&](int kt) {  // before the DMA of B K step kt
    if constexpr (BMODE == B_KSEG) {
      constexpr int U = KB / kSegUnit;  // segment units per K step
      while ((kt + kt0) * U >= seg_next) seg_enter(seg_i + 1);
    }
  };
  auto b_step = [&](int kt) -> BStep {
    if constexpr (BMODE == B_KSEG) {
      return {seg_row0 + (int64_t)(kt + kt0) * ROWB, seg_ldv};
    } else {
      return {nullptr, 0};
    }
  };
  auto dma_a = [&](int kt, char* stage, int ii) {
    const char* g = a_base + (a_off[ii] + (uint32_t)kt * ROWB);
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + (wave * A_W + ii) * RPI * ROWB), 16, 0, 0);
  };
  auto dma_b = [&](int kt, const BStep& bs, char* stage, int ii) {
    const char* g;
    if constexpr (BMODE == B_KSEG) {
      g = bs.base + seg_off[ii];
    } else if constexpr (BMODE == B_KMAJOR) {
      const int k0 = (kt + kt0) * KE;  // first K row of the step (workgroup-uniform)
      const char* rows = k0 < args.kmaj_split ? kmaj_b0 + (int64_t)k0 * ldb
                                              : kmaj_b1 + (int64_t)(k0 - args.kmaj_split) * ldb;
      g = rows + b_off[ii];
    } else {
      g = b_base[ii] + (b_off[ii] + (uint32_t)kt * ROWB);
    }
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(stage + (wave * B_W + ii) * RPI * ROWB), 16, 0, 0);
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
  // B_KMAJOR fragment reads.  Lane = 16 g + q: the 16 lanes of group g read
  // K-rows r..r+3 (4 columns each) and the transposing read hands lane q
  // column n0 + q of those rows; g / 2 picks the MFMA's K half, g % 2 the
  // column half of the 32-column sub-tile.  The swizzle of K-row
  // 16 c + rb (+ 4) equals that of rb, so one byte offset per sub-tile
  // serves every chunk c (+ 16 c K-rows) and both reads (+ 4 K-rows).
  uint32_t kmaj_frag[BMODE == B_KMAJOR ? TN : 1];
  if constexpr (BMODE == B_KMAJOR) {
    const int rb = 8 * (lane >> 5) + ((lane >> 2) & 3);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      kmaj_frag[j] = (uint32_t)kmaj_pos(rb, b_tile_row(j) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  }
  // physical byte offset of logical 16-byte chunk c of tile row `row`
  auto swz = [](int row, int c) -> int { return row * ROWB + ((c ^ ((row / RSH) % NCH)) << 4); };

  // ---- main loop.  Tile t of A sits in A stage t % SA, of B in B stage
  // t % SB.  A K step kt has two phases split by the workgroup barrier:
  //   phase 1: MFMAs on fragment chunks 0..H-1 of tile kt (already in
  //            registers) while chunks H..NC-1 of tile kt are read from LDS;
  //   wait:    this wave's reads of tile kt are done (lgkmcnt 0) and its DMA
  //            of tile kt+1 has landed (vmcnt), then the barrier: tile kt's
  //            stages are free and tile kt+1 is visible to every wave;
  //   phase 2: MFMAs on chunks H..NC-1 of tile kt while chunks 0..H-1 of tile
  //            kt+1 are read and the DMA of A tile kt+SA / B tile kt+SB is
  //            issued into the stages tile kt just released.
  // Every MFMA after the barrier has its operands in registers already, so
  // the barrier costs no LDS round trip.  Tiles past the end (t >= KT) reload
  // tile KT-1 into their stage (no later step reads it): every step issues the
  // same instructions, the steps are branch-free and the vmcnt accounting is
  // exact.  B is issued after A when SB > SA (B runs further ahead) and before
  // it when SB == SA; either way B(t) is issued before A(t), so waiting for
  // A(kt+1) covers B(kt+1): the DMA instructions issued after A(kt+1) are
  // those of the SA-2 later steps, plus B(kt+1-SA+SB) when SB > SA.
  constexpr bool kAFirst = SB > SA;
  constexpr int NI = A_W + B_W;                                 // DMA instructions per step
  constexpr int kNewer = (kAFirst ? B_W : 0) + (SA - 2) * NI;  // vmcnt at the barrier of a step
  constexpr int kNewer0 = kNewer + NI;                          // vmcnt before step 0
  static_assert(kNewer0 < 64, "vmcnt range");
  const int KT_all = klen * (int)sizeof(TA) / ROWB;  // 0 only for an empty A_KBATCH range
  const int KT = split ? min(args.kslice, KT_all - kt0) : KT_all;  // K steps of this workgroup
  auto clampt = [&](int t) { return t < KT ? t : KT - 1; };
  // issue the DMA of A tile ta into A stage sa and B tile tb into B stage sb
  auto dma_step = [&](int ta, char* sa, int tb, char* sb) {
    const BStep bs = b_step(tb);
    if constexpr (!kAFirst) {
#pragma unroll
      for (int ii = 0; ii < B_W; ++ii) dma_b(tb, bs, sb, ii);
    }
#pragma unroll
    for (int ii = 0; ii < A_W; ++ii) dma_a(ta, sa, ii);
    if constexpr (kAFirst) {
#pragma unroll
      for (int ii = 0; ii < B_W; ++ii) dma_b(tb, bs, sb, ii);
    }
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");  // no LDS access may move across the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // prologue: the DMA of virtual steps -SB..-1 (A tiles 0..SA-1, B tiles 0..SB-1);
  // an empty K range (KT == 0, uniform over the workgroup) has no DMA and no
  // main loop: its tile is stored as zeros
  if constexpr (k1Bar) {
    if (KT > 0) {  // step 0 only; step kt + 1 loads during step kt
      b_seek(0);
      dma_step(0, ringA, 0, ringB);
    }
  } else
#pragma unroll
  for (int s = -SB; s < 0 && KT > 0; ++s) {
    const int ta = s + SA, tb = s + SB;
    b_seek(clampt(tb));
    const BStep bs = b_step(clampt(tb));
    if constexpr (!kAFirst) {
#pragma unroll
      for (int ii = 0; ii < B_W; ++ii) dma_b(clampt(tb), bs, ringB + tb * kStageB, ii);
    }
    if (ta >= 0) {
#pragma unroll
      for (int ii = 0; ii < A_W; ++ii) dma_a(clampt(ta), ringA + ta * kStageA, ii);
    }
    if constexpr (kAFirst) {
#pragma unroll
      for (int ii = 0; ii < B_W; ++ii) dma_b(clampt(tb), bs, ringB + tb * kStageB, ii);
    }
  }

  // NA = number of this wave's 32-row sub-tiles that hold valid rows (a
  // wave-uniform constant of the instantiation, so every step is
  // straight-line code).
  auto main_loop = [&](auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    // NC = NCH / 2 fragment chunks per lane per K step:
    //   16-bit: chunk c holds k 8lh..8lh+7 of MFMA c (LDS chunk 2c + lh)
    //   fp32:   chunk c is LDS chunk NC*lh + c (this lane's K half), one k per MFMA
    constexpr int NC = NCH / 2, H = NC / 2;
    constexpr int NAr = NA > 0 ? NA : 1;
    u32x4 fa[NC][NAr], fb[NC][TN];
    auto read_chunk = [&](const char* As, const char* Bs, auto c_c) {
      constexpr int c = decltype(c_c)::value;
      const int ch = kHalf ? (2 * c + lh) : (NC * lh + c);
#pragma unroll
      for (int i = 0; i < NA; ++i) fa[c][i] = *(const u32x4*)(As + swz(wm * WTM + i * 32 + lr, ch));
      if constexpr (BMODE != B_KMAJOR) {  // (K-major B: read_b_kmaj)
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[c][j] = *(const u32x4*)(Bs + swz(b_tile_row(j) + lr, ch));
      }
    };
    // B_KMAJOR: the B fragments of chunks C0 .. C0+CN-1 through gfx950's
    // transposing LDS read (ds_read_b64_tr_b16), issued together and waited
    // for in the same asm block.  The builtin for this read carries no alias
    // information, and the compiler then waits for every LDS-DMA in flight
    // (vmcnt 0) before each such read; here the wave waits only for its own
    // LDS reads.
    auto read_b_kmaj = [&](const char* Bs, auto c0_c, auto cn_c) {
      constexpr int C0 = decltype(c0_c)::value, CN = decltype(cn_c)::value;
      if constexpr (BMODE == B_KMAJOR && CN > 0) {
        static_assert(TN == 2 && CN <= 2, "K-major B: two 32-column sub-tiles per wave, one or two chunks");
        typedef __attribute__((address_space(3))) const char* lds_cptr;
        const uint32_t a0 = (uint32_t)(size_t)(lds_cptr)(Bs + kmaj_frag[0]);
        const uint32_t a1 = (uint32_t)(size_t)(lds_cptr)(Bs + kmaj_frag[1]);
        u32x2 r[CN][TN][2];  // [chunk][sub-tile][K-rows 0-3 | 8-11 of the 16-row group]
        if constexpr (CN == 1) {
          asm volatile(
              "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
              "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
              "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
              "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(r[0][0][0]), "=&v"(r[0][0][1]), "=&v"(r[0][1][0]), "=&v"(r[0][1][1])
              : "v"(a0), "v"(a1), "i"(C0 * 16 * ROWK), "i"(C0 * 16 * ROWK + 4 * ROWK));
        } else {
          asm volatile(
              "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
              "ds_read_b64_tr_b16 %1, %8 offset:%11\n\t"
              "ds_read_b64_tr_b16 %2, %9 offset:%10\n\t"
              "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
              "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
              "ds_read_b64_tr_b16 %5, %8 offset:%13\n\t"
              "ds_read_b64_tr_b16 %6, %9 offset:%12\n\t"
              "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(r[0][0][0]), "=&v"(r[0][0][1]), "=&v"(r[0][1][0]), "=&v"(r[0][1][1]),
                "=&v"(r[1][0][0]), "=&v"(r[1][0][1]), "=&v"(r[1][1][0]), "=&v"(r[1][1][1])
              : "v"(a0), "v"(a1), "i"(C0 * 16 * ROWK), "i"(C0 * 16 * ROWK + 4 * ROWK),
                "i"((C0 + 1) * 16 * ROWK), "i"((C0 + 1) * 16 * ROWK + 4 * ROWK));
        }
#pragma unroll
        for (int c = 0; c < CN; ++c)
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[C0 + c][j] = u32x4{r[c][j][0][0], r[c][j][0][1], r[c][j][1][0], r[c][j][1][1]};
      }
    };
    auto mfma_chunk = [&](auto c_c) {
      constexpr int c = decltype(c_c)::value;
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
    };
    constexpr int MPC = NA * TN * (kHalf ? 1 : 4);  // MFMAs per chunk
    constexpr int RPC = NA + (BMODE == B_KMAJOR ? 0 : TN);  // compiler-visible fragment reads per chunk
    if constexpr (k1Bar) {
      // One barrier per K step.  Step kt's tiles sit in stage kt % 2, and
      // during the step the DMA fills the other stage with step kt + 1 (a
      // whole step to land, where the two-phase schedule gives a two-stage
      // ring half a step).  The MFMAs of a step's last chunk run after the
      // barrier, while the next step's first fragments are read, so the
      // matrix cores have work across it.  Results are bit-identical to the
      // two-phase schedule (same MFMAs in the same order per accumulator).
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      barrier();
      auto step1 = [&](int kt, auto u_c, auto first_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr bool first = decltype(first_c)::value;
        b_seek(clampt(kt + 1));
        const char* As = ringA + u * kStageA;
        const char* Bs = ringB + u * kStageB;
        read_chunk(As, Bs, IntC<0>{});
        if constexpr (!first) mfma_chunk(IntC<NC - 1>{});  // the previous step's last chunk
        // the stage of step kt - 1 is free: every wave passed the barrier after reading it
        dma_step(clampt(kt + 1), ringA + (1 - u) * kStageA, clampt(kt + 1), ringB + (1 - u) * kStageB);
        if constexpr (first) {
          __builtin_amdgcn_sched_group_barrier(0x100, RPC, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, NI, 0);
        } else {
          sched_interleave<MPC, RPC, NI>();
        }
        __builtin_amdgcn_sched_barrier(0);
        sfor<NC - 1>([&](auto c_c) {
          constexpr int c = decltype(c_c)::value;
          read_chunk(As, Bs, IntC<c + 1>{});
          mfma_chunk(IntC<c>{});
          sched_interleave<MPC, RPC, 0>();
          __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));  // step kt + 1 landed, this step's reads done
        barrier();
        __builtin_amdgcn_sched_barrier(0);
      };
      step1(0, IntC<0>{}, IntC<true>{});
      for (int kt = 1; kt < KT; kt += 2) {
        step1(kt, IntC<1>{}, IntC<false>{});
        if (kt + 1 < KT) step1(kt + 1, IntC<0>{}, IntC<false>{});
      }
      mfma_chunk(IntC<NC - 1>{});
      return;
    }
    // tile 0 landed and visible; its first chunks into registers
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kNewer0));
    barrier();
    sfor<H>([&](auto c_c) { read_chunk(ringA, ringB, c_c); });
    read_b_kmaj(ringB, IntC<0>{}, IntC<H>{});

    auto one = [&](int kt, auto u_c) {
      constexpr int u = decltype(u_c)::value;  // kt % UNROLL: stages are static
      b_seek(clampt(kt + SB));
      const char* As = ringA + (u % SA) * kStageA;
      const char* Bs = ringB + (u % SB) * kStageB;
      // phase 1
      sfor<NC - H>([&](auto c_c) { read_chunk(As, Bs, IntC<H + decltype(c_c)::value>{}); });
      read_b_kmaj(Bs, IntC<H>{}, IntC<NC - H>{});
      sfor<H>([&](auto c_c) { mfma_chunk(c_c); });
      // one MFMA (its operands were read in the previous phase), then the
      // reads, which must be complete at the barrier, then the other MFMAs;
      // nothing crosses the barrier
      if constexpr (H * MPC > 0) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (NC - H) * RPC, 0);
      if constexpr (H * MPC > 1) __builtin_amdgcn_sched_group_barrier(0x008, H * MPC - 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kNewer));
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      // phase 2 (program order: reads of tile kt+1, then the DMA into tile kt's stages)
      sfor<H>([&](auto c_c) {
        read_chunk(ringA + ((u + 1) % SA) * kStageA, ringB + ((u + 1) % SB) * kStageB, c_c);
      });
      read_b_kmaj(ringB + ((u + 1) % SB) * kStageB, IntC<0>{}, IntC<H>{});
      dma_step(clampt(kt + SA), ringA + (u % SA) * kStageA, clampt(kt + SB), ringB + (u % SB) * kStageB);
      sfor<NC - H>([&](auto c_c) { mfma_chunk(IntC<H + decltype(c_c)::value>{}); });
      // the next tile's reads first (phase 1 of the next step needs them at once),
      // then the DMA spread over the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, H * RPC, 0);
      sched_interleave<(NC - H) * MPC, 0, NI>();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < KT; kt += UNROLL) {
      one(kt, IntC<0>{});
      if constexpr (UNROLL > 1) if (kt + 1 < KT) one(kt + 1, IntC<1>{});
      if constexpr (UNROLL > 2) if (kt + 2 < KT) one(kt + 2, IntC<2>{});
      if constexpr (UNROLL > 3) if (kt + 3 < KT) one(kt + 3, IntC<3>{});
      if constexpr (UNROLL > 4) if (kt + 4 < KT) one(kt + 4, IntC<4>{});
      if constexpr (UNROLL > 5) if (kt + 5 < KT) one(kt + 5, IntC<5>{});
      if constexpr (UNROLL > 6) if (kt + 6 < KT) one(kt + 6, IntC<6>{});
      if constexpr (UNROLL > 7) if (kt + 7 < KT) one(kt + 7, IntC<7>{});
    }
    // the reloads past the end land before the ring is reused by the epilogue
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
  };
  if (KT == 0) {
  } else if constexpr (GROUPED) {
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

  // ---- epilogue.  A tail-split K slice stores its fp32 partial product as
  // the tile's BM x BN block (every row and column: values past the valid
  // range come from clamped operand rows, finite, and are never read).
  if constexpr (kTail) {
    if (tail) {
      float* const tp = (float*)outp;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            tp[(wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3)) * BN + wn * WTN + j * 32 + lr] = acc[i][j][v];
      return;
    }
  }
  // Each wave stages its finished output tile in LDS (the
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
    if constexpr (EMODE == E_SITU || EMODE == E_PRE)
      return situ_hidden(acc[i][j][v], acc[i][j + TN / 2][v], args.beta1, args.beta2, inv_b1, inv_b2);
    else
      return acc[i][j][v];
  };
  auto out_row = [&](int r) -> int64_t {  // r: row inside the block tile
    if constexpr (EMODE == E_SLOTS) return slot_row[r];
    else return GROUPED ? off + m0 + r : (int64_t)(m0 + r);
  };

  constexpr bool kRangeCheck = EMODE != E_SITU && EMODE != E_PRE && __is_same(OutT, f16_t);
  if constexpr (EMODE == E_PRE) {
    static_assert(BMODE == B_DUAL, "pre-activations of a (gate, up) pair");
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = col0 + j * 32 + lr;
        if (col >= args.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          if (r >= rows_valid) continue;
          const int64_t o = out_row(r) * args.pre_ld + (int64_t)col * (int64_t)sizeof(OutT);
          Elem<OutT>::store((OutT*)(args.pre_g + o), acc[i][j][v]);
          Elem<OutT>::store((OutT*)(args.pre_u + o), acc[i][j + TN / 2][v]);
        }
      }
  }
  bool out_of_range = false;
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
        if constexpr (EMODE == E_SLOTS) ps[v] = slot_p[wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3)];
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int cb = (j * 32 + lr) * OES;  // byte column inside the staged row
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          float val = value(i, j, v);
          if constexpr (EMODE == E_SLOTS) val *= ps[v];
          if constexpr (kRangeCheck) out_of_range |= f16_out_of_range(val);
          Elem<OutT>::store((OutT*)(E + pos(rl, cb >> 4) + (cb & 15)), val);
        }
      }
    }
    const bool aligned = (((uintptr_t)outp | (uintptr_t)args.ldo) & 15) == 0;
    constexpr int EPC = 16 / OES;  // elements per chunk
    for (int id = lane; id < WTM * CPR; id += 64) {
      const int rl = id / CPR, c = id % CPR;
      const int r = wm * WTM + rl;
      const int col = col0 + c * EPC;
      if (r >= rows_valid || col >= args.N) continue;
      const char* src = E + pos(rl, c);
      OutT* dst = (OutT*)(outp + out_row(r) * args.ldo) + col;
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
          if constexpr (EMODE == E_SLOTS) val *= slot_p[r];
          if constexpr (kRangeCheck) out_of_range |= f16_out_of_range(val);
          Elem<OutT>::store((OutT*)(outp + out_row(r) * args.ldo) + col, val);
        }
      }
    }
  }
  // rows past the valid range hold finite (clamped-row) values, so a flag
  // raised by them is raised by a valid row too
  if constexpr (kRangeCheck)
    if (out_of_range && args.range_flag) *args.range_flag = 1;  // any lane: every writer stores 1
}

// Sum of the K slices' fp32 partial products in slice order, stored as OutT:
// out[m, n] = sum over s of part[s][m][n]  (part [S, M, N], out row stride ldo bytes).
// Four consecutive columns per thread (N % 4 == 0: 16-byte loads), the slice
// loads issued four at a time.
template <typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            char* __restrict__ out, int64_t ldo,
                                                            int32_t* __restrict__ range_flag) {
  constexpr bool kRangeCheck = __is_same(OutT, f16_t);
  bool out_of_range = false;
  const int64_t MN = (int64_t)M * N;
  const bool vec = (N & 3) == 0;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < MN; i += (int64_t)gridDim.x * 1024) {
    const int64_t m = i / N, n = i % N;
    OutT* dst = (OutT*)(out + m * ldo) + n;
    if (vec) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int sl = 0;
      for (; sl + 4 <= S; sl += 4) {
        const f32x4 a = *(const f32x4*)(part + sl * MN + i), b = *(const f32x4*)(part + (sl + 1) * MN + i);
        const f32x4 c = *(const f32x4*)(part + (sl + 2) * MN + i), d = *(const f32x4*)(part + (sl + 3) * MN + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = (((acc[q] + a[q]) + b[q]) + c[q]) + d[q];
      }
      for (; sl < S; ++sl) {
        const f32x4 a = *(const f32x4*)(part + sl * MN + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += a[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kRangeCheck) out_of_range |= f16_out_of_range(acc[q]);
        Elem<OutT>::store(dst + q, acc[q]);
      }
    } else {
      for (int64_t j = i; j < i + 4 && j < MN; ++j) {
        float acc = 0.f;
        for (int sl = 0; sl < S; ++sl) acc += part[sl * MN + j];
        if constexpr (kRangeCheck) out_of_range |= f16_out_of_range(acc);
        Elem<OutT>::store((OutT*)(out + (j / N) * ldo) + j % N, acc);
      }
    }
  }
  if (out_of_range && range_flag) *range_flag = 1;
}

// The tail tiles of a tail-split product (GemmArgs: tsplit, twhole, tpart):
// out tile = sum of its K slices' fp32 partial blocks in slice order, stored
// as OutT (row stride ldo bytes) within M x N.  One workgroup per 16 rows of
// a tail tile; thread t sums BN / 16 consecutive columns of row t / 16.
template <typename OutT, int BM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const GemmArgs a) {
  static_assert(BM % 16 == 0 && BN % 64 == 0, "16-row blocks, 4-column groups");
  constexpr int CW = BN / 16;  // columns per thread
  constexpr bool kRangeCheck = __is_same(OutT, f16_t);
  const int tail_id = blockIdx.x / (BM / 16), rb = blockIdx.x % (BM / 16);
  const int P = a.m_tiles * a.n_tiles / 8, rem = P - a.twhole;
  int mt, nt;
  dense_tile_coords((tail_id / rem) * P + a.twhole + tail_id % rem, a.m_tiles, a.n_tiles, &mt, &nt);
  const int r = rb * 16 + (int)threadIdx.x / 16, c0 = ((int)threadIdx.x % 16) * CW;
  const int m = mt * BM + r, n0 = nt * BN + c0;
  if (m >= a.M || n0 >= a.N) return;
  const float* src = (const float*)a.tpart + (int64_t)tail_id * a.tsplit * (BM * BN) + r * BN + c0;
  f32x4 acc[CW / 4];
#pragma unroll
  for (int q = 0; q < CW / 4; ++q) acc[q] = *(const f32x4*)(src + 4 * q);
  for (int sl = 1; sl < a.tsplit; ++sl) {
    const float* s = src + (int64_t)sl * (BM * BN);
    f32x4 b[CW / 4];
#pragma unroll
    for (int q = 0; q < CW / 4; ++q) b[q] = *(const f32x4*)(s + 4 * q);
#pragma unroll
    for (int q = 0; q < CW / 4; ++q) acc[q] += b[q];
  }
  bool out_of_range = false;
  OutT* dst = (OutT*)(a.out + (int64_t)m * a.ldo) + n0;
  const bool whole = n0 + CW <= a.N && (((uintptr_t)a.out | (uintptr_t)a.ldo) & 15) == 0;
  if (whole) {
    // CW values as 16-byte stores (n0 * sizeof(OutT) is a multiple of 32)
    OutT vals[CW];
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      const float v = acc[q / 4][q % 4];
      if constexpr (kRangeCheck) out_of_range |= f16_out_of_range(v);
      Elem<OutT>::store(&vals[q], v);
    }
    constexpr int NV = CW * (int)sizeof(OutT) / 16;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      u32x4 w;
      __builtin_memcpy(&w, (const char*)vals + 16 * q, 16);
      *((u32x4*)dst + q) = w;
    }
  } else {
    for (int q = 0; q < CW && n0 + q < a.N; ++q) {
      const float v = acc[q / 4][q % 4];
      if constexpr (kRangeCheck) out_of_range |= f16_out_of_range(v);
      Elem<OutT>::store(dst + q, v);
    }
  }
  if (kRangeCheck && out_of_range && a.range_flag) *a.range_flag = 1;
}

}  // namespace lmoe
