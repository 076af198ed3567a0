// One MFMA GEMM template for every quantised contraction on the path.
//
// The pages' fused dequantize-and-multiply (llama.cpp-style MMQ, dense and
// grouped, page 2 "Show HN: LoRA over GGUF", section "Things involved in
// the training"; the ai-manual.ru article describes the fused kernel as
// decoding the compressed weights in registers and multiplying at once, with
// no fp16 copy of W) is built here for CDNA4:
//
//  * 256 threads = 4 wave64s in a 2x2 grid (block tile BM x 128, k-step 64),
//    or 512 threads in two k-groups of four waves that take alternate
//    k-steps and add their accumulators through LDS (split-K inside the
//    workgroup, for launches of at most one tile per CU).
//  * Activations (bf16) are staged global -> registers -> LDS; weight blocks
//    are loaded raw (scale + unaligned payload loads), decoded to bf16 in
//    registers and written to LDS -- the only full-precision copy of W is the
//    64-deep LDS slice of the current tile.
//  * NT (forward): the reduction runs along the weight's block dimension, the
//    decoded tile is stored [n][k].  NN (backward, dX = dY deq(W)): the
//    reduction runs along the weight's rows; the decoded rows are stored
//    row-major and read back transposed (ds_read_b64_tr_b16) into the same
//    MFMA operand layout (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//  * Double-buffered LDS, one barrier per k-step, prefetch depth 2; the
//    steady-state loop is one basic block, and full tiles run a copy of it
//    without masks.
//  * Grouped (MoE) launches map m-tile slots to experts through a device
//    prefix of per-expert tile counts: no host sync, idle experts' blocks are
//    never read.
//  * Workgroups are renumbered so that each XCD (8 per MI355X, dispatched
//    round-robin) works on a contiguous run of tiles; dense launches order
//    that run as 4 m-tiles by a band of n-tiles (L2 reuse of both operands).
//  * Epilogues fold in the rank-r adapter term and the fused consumers
//    (SwiGLU, the cross-entropy partials, the SwiGLU backward), with row and
//    column reductions staged through LDS in a fixed order (deterministic).
#pragma once
#include <math.h>

#include "gq_dev.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int BK = GEMM_BK;  // 64 = two quant blocks along k
constexpr int LDK = BK + 8;  // padded LDS row (bf16): 144 B keeps ds_read_b128 conflict-free
constexpr int NTHR = 256;

template <int BM, int BN, bool STAGE, bool NN, int KS>
struct Geom {
  static constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_CHUNKS = BM * BK / 8 / NTHR;  // 16-byte chunks per thread
  // weight tile in LDS (bf16 elements): NT [BN][LDK] (k contiguous);
  // NN [64][PN] row-major (columns contiguous), read with transposing loads;
  // unpadded rows whose 16-byte chunks are XOR-swizzled by the row (see
  // nn_chunk below)
  static constexpr int PN = BN;
  static constexpr int B_TILE = NN ? BK * PN : BN * LDK;
  static constexpr int SMEM_MAIN = 2 * (BM * LDK + B_TILE) * 2;
  static constexpr int ZP = BN + 1;  // pitch (floats) of the staged epilogue tile
  // staged tile with 16-byte aligned rows (BN + 4 floats) plus two [BN][8]
  // rank-vector slices (the SwiGLU-backward epilogue); covers the ZP layout
  static constexpr int SMEM_Z = STAGE ? BM * (BN + 4) * 4 + 2 * BN * 8 * 4 : 0;
  // KS groups of four waves, each with its own double-buffered stages; the
  // cross-group reduction of the accumulators reuses the same memory
  static constexpr int SMEM_K = KS * SMEM_MAIN;
  static constexpr int SMEM_RED = KS > 1 ? BM * BN * 4 : 0;
  static constexpr int SMEM_KR = SMEM_K > SMEM_RED ? SMEM_K : SMEM_RED;
  static constexpr int SMEM = SMEM_KR > SMEM_Z ? SMEM_KR : SMEM_Z;
};

// epilogues that stage the output tile through LDS
constexpr bool epi_stages(int epi) {
  return epi == EPI_CE_FWD || epi == EPI_CE_BWD || epi == EPI_DOWN_BWD;
}

// logistic function with the hardware reciprocal (about 1 ulp, no division
// sequence)
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// all-ones / all-zeros mask the optimiser cannot see through (an empty
// register-only asm), so a load whose result is masked is never turned back
// into a branch around the load
__device__ __forceinline__ uint32_t opaque_mask(bool keep) {
  uint32_t m = keep ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(m));
  return m;
}

// NN weight tile: the 16-byte chunk c (8 columns) of reduction row `row` is
// stored at chunk c ^ (5 * (row & 3)).  With 256-byte rows this makes both
// LDS access patterns of the tile free of bank conflicts (64 banks of 4
// bytes): a 16-lane pass of the decode's 16-byte writes covers rows R..R+3
// (R % 4 == 0) x 4 blocks at one chunk position q, whose swizzled chunks
// 4(kb ^ (row&3)) + (q ^ (row&3)) are all distinct; a 32-lane pass of the
// transposing 8-byte reads covers rows t (mod 4) x chunks base+0..3, whose
// swizzled chunks (base/4 ^ t, tc ^ t) are all distinct.
__device__ __forceinline__ int nn_chunk(int row, int c) { return c ^ (5 * (row & 3)); }

template <bool B> struct BoolC { static constexpr bool value = B; };
template <int I> struct IntC { static constexpr int value = I; };

// r (<= R) rank values at p: R/4 vector loads when r == R (rank vectors of
// r = R floats are 16-byte aligned), else guarded scalar loads.
template <int R>
__device__ __forceinline__ void load_rank(const float* p, int r, float (&v)[R]) {
  if (r == R) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const float4 f = reinterpret_cast<const float4*>(p)[q];
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = j < r ? p[j] : 0.f;
  }
}

// Row reduction of the staged tile Z [BM][ZP]:
//   out[j] = sum_{c : n0 + c < ncols} Z[row][c] * W[(n0 + c) * r + j],  j < r <= R
// The tile's rank vectors are first staged in LDS (S: BN x R floats) by all
// threads, so the reduction loop reads only LDS.  Thread (row = tid % BM,
// seg = tid / BM) sums one column segment; segments are combined in order
// through LDS.  sink(row, out) runs on segment 0.  Caller has synchronised
// after writing Z; returns synchronised.
template <int BM, int BN, int R, class Sink>
__device__ __forceinline__ void z_row_reduce(float* Z, float* S, const float* W, int r, int n0,
                                             int ncols, Sink sink) {
  constexpr int NSEG = NTHR / BM, SEGC = BN / NSEG, ZP = BN + 1, XP = R + 1;
  const int tid = threadIdx.x;
  const int row = tid % BM, seg = tid / BM;
  for (int i = tid; i < BN * R; i += NTHR) {
    const int c = i / R, j = i % R;
    S[i] = (j < r && n0 + c < ncols) ? W[(int64_t)(n0 + c) * r + j] : 0.f;
  }
  __syncthreads();
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;
#pragma unroll 4
  for (int c = seg * SEGC; c < (seg + 1) * SEGC; ++c) {
    const float z = Z[row * ZP + c];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] += z * S[c * R + j];
  }
  __syncthreads();
  float* X = Z;  // reuse: [NSEG][BM][R + 1]
  if (seg > 0) {
#pragma unroll
    for (int j = 0; j < R; ++j) X[(seg * BM + row) * XP + j] = acc[j];
  }
  __syncthreads();
  if (seg == 0) {
    for (int sg = 1; sg < NSEG; ++sg) {
#pragma unroll
      for (int j = 0; j < R; ++j) acc[j] += X[(sg * BM + row) * XP + j];
    }
    sink(row, acc);
  }
  __syncthreads();
}

// Column reduction of Z: out[j] = sum_{row : r0 + row < r1} Z[row][col] * X[(r0+row)*r + j],
// the tile's rank vectors staged in LDS (S: BM x R floats) first.
template <int BM, int BN, int R, class Sink>
__device__ __forceinline__ void z_col_reduce(float* Z, float* S, const float* X, int r, int64_t r0,
                                             int64_t r1, Sink sink) {
  constexpr int NSEG = NTHR / BN, SEGR = BM / NSEG, ZP = BN + 1, XP = R + 1;
  const int tid = threadIdx.x;
  const int col = tid % BN, seg = tid / BN;
  for (int i = tid; i < BM * R; i += NTHR) {
    const int rr = i / R, j = i % R;
    S[i] = (j < r && r0 + rr < r1) ? X[(r0 + rr) * r + j] : 0.f;
  }
  __syncthreads();
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;
#pragma unroll 4
  for (int rr = seg * SEGR; rr < (seg + 1) * SEGR; ++rr) {
    const float z = Z[rr * ZP + col];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] += z * S[rr * R + j];
  }
  __syncthreads();
  float* Xs = Z;
  if (seg > 0) {
#pragma unroll
    for (int j = 0; j < R; ++j) Xs[(seg * BN + col) * XP + j] = acc[j];
  }
  __syncthreads();
  if (seg == 0) {
    for (int sg = 1; sg < NSEG; ++sg) {
#pragma unroll
      for (int j = 0; j < R; ++j) acc[j] += Xs[(sg * BN + col) * XP + j];
    }
    sink(col, acc);
  }
  __syncthreads();
}

// Instruction interleave for the steady-state k-step: LEAD LDS reads first
// (the first MFMA operands), then per MFMA NV VALU ops (the decode of the
// next tile) and ND LDS ops, so the decode issues in the shadow of the
// matrix cores instead of in clusters (measured ~10% on the dense forward;
// the NN path, with two transposing reads per B fragment, takes 4 LDS ops
// per MFMA: ~5% on the dX launch).
template <int NM, int NV, int ND, int LEAD>
__device__ __forceinline__ void mfma_interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    __builtin_amdgcn_sched_group_barrier(0x080, ND, 0);
  }
}

// The tile GEMM of one workgroup: `block` of `nblocks` (the workgroup's
// position in its launch, or in its part of a launch that runs two kinds of
// tiles), `smem` the workgroup's LDS (at least Geom::SMEM bytes).
template <int QT, int EPI, int BM, int BN, int KS>
__device__ __forceinline__ void gemm_body(const GemmArgs& p, uint8_t* smem, const int block,
                                          const int nblocks) {
  constexpr bool NN = EPI >= EPI_LIN_BWD;
  using G = Geom<BM, BN, epi_stages(EPI), NN, KS>;
  constexpr int BS = QTraits<QT>::BS;
  constexpr int TM = G::TM, TN = G::TN, WTM = G::WTM, WTN = G::WTN, ZP = G::ZP;
  static_assert(BN == 128 || BN == 256, "weight items: 2*BN blocks per k-step");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate/up n-subtiles");
  static_assert(KS == 1 || (KS == 2 && !epi_stages(EPI)),
                "split-K groups: the reduction leaves one group for a barrier-free epilogue");

  // group `grp` of four waves takes k-steps grp, grp + KS, grp + 2KS, ...
  const int grp = KS > 1 ? (int)(threadIdx.x / NTHR) : 0;
  uint16_t* As = reinterpret_cast<uint16_t*>(smem + grp * G::SMEM_MAIN);
  uint16_t* Bs = As + 2 * BM * LDK;
  constexpr int B_TILE = G::B_TILE, PN = G::PN;

  const int tid = threadIdx.x % NTHR;  // thread within the group
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- workgroup -> tile, XCD-contiguous runs of tiles.  Workgroup ids go
  // round-robin over the 8 XCDs; renumbering them so that each XCD owns a
  // contiguous run of tile ids keeps the tiles that share operands in one L2.
  auto xcd_run = [](int id, int count) {
    const int q = count >> 3, rem = count & 7, xcd = id & 7, loc = id >> 3;
    return (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + loc;
  };
  // Grouped launches: the grid covers the largest possible number of m-slots;
  // only the first tile_start[E] hold rows.  The runs are laid over those
  // (the rest exit here), n-tiles fastest, so the n-tiles of one m-slot,
  // which share its gathered activation rows, run together on one XCD.
  // Dense launches: each XCD's run covers GM m-tiles by a band of n-tiles,
  // so its L2 holds the activation rows of GM m-tiles and the weight columns
  // of the band instead of every m-tile.
  int mslot, ntile;
  int ksidx = 0;
  if (p.offsets) {
    const int used = p.tile_start[p.E] * p.ntiles;
    if (block >= used) return;
    const int bid = xcd_run(block, used);
    mslot = bid / p.ntiles;
    ntile = bid - mslot * p.ntiles;
  } else {
    int bid = xcd_run(block, nblocks);
    if (p.ksplit > 1) {  // consecutive ids: the k-ranges of one tile
      ksidx = bid % p.ksplit;
      bid /= p.ksplit;
    }
    constexpr int GM = 4;
    const int gsize = GM * p.ntiles;
    const int g = bid / gsize;
    const int m_first = g * GM;
    const int gm = min(p.mtiles - m_first, GM);
    const int idx = bid - g * gsize;
    mslot = m_first + idx % gm;
    ntile = idx / gm;
  }
  int e = 0;
  int64_t r0, r1;
  if (p.offsets) {
    const int32_t* ts = p.tile_start;
    if (mslot >= ts[p.E]) return;
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ts[mid] <= mslot) lo = mid; else hi = mid;
    }
    e = lo;
    r0 = (int64_t)p.offsets[e] + (int64_t)(mslot - ts[e]) * BM;
    r1 = min((int64_t)p.offsets[e + 1], r0 + BM);
  } else {
    r0 = (int64_t)mslot * BM;
    if (r0 >= p.M) return;
    r1 = min(p.M, r0 + BM);
  }
  const int n0 = ntile * BN;
  // k-steps of this workgroup: all of them, or split ksidx's contiguous range
  const int nkall = (p.K + BK - 1) / BK;
  const int kb0 = p.ksplit > 1 ? (int)((int64_t)ksidx * nkall / p.ksplit) : 0;
  const int nk = p.ksplit > 1 ? (int)((int64_t)(ksidx + 1) * nkall / p.ksplit) - kb0 : nkall;
  const int nkl = (nk + KS - 1) / KS;   // k-steps of each group
  auto KT = [&](int ls) { return kb0 + ls * KS + grp; };
  auto LCb = [&](int b) { return wn * WTN + b * 32 + (lane & 31); };

  // ---- main loop
  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // NN operand B from the row-major tile with ds_read_b64_tr_b16: within
  // each 16-lane group g, output lane 16g + j slot t receives element j % 4
  // of the 4-element chunk addressed by lane 16g + 4t + j / 4.  Lane
  // 16g + 4t + q therefore addresses reduction row 8*(g/2) + t (+4 for the
  // second half) at column 16*(g%2) + 4q of its 32-column subtile, and lane
  // L ends up with rows 8*(L/32) .. +8 of column L % 32 -- the MFMA B layout.
  const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // this lane's element offset of subtile b in the swizzled tile, at rows
  // tr_row + 16kk (+4): the swizzle depends on row & 3 only, equal for all
  int tr_off[TN];
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int col = wn * WTN + b * 32 + tr_col;
    tr_off[b] = tr_row * PN + nn_chunk(tr_row, col >> 3) * 8 + (col & 7);
  }
  // NA = the wave's 32-row sub-tiles that hold rows of the tile (a partly
  // filled MoE tile leaves whole sub-tiles empty: no MFMAs for them)
  auto compute = [&](int cur, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const uint16_t* A = As + cur * BM * LDK;
    const uint16_t* B = Bs + cur * B_TILE;
    if constexpr (NA == 0) return;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int a = 0; a < NA; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(A + (wm * WTM + a * 32 + (lane & 31)) * LDK +
                                                 kk * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        if constexpr (NN) {
          typedef short v4i16 __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
          const uint16_t* base = B + kk * 16 * PN + tr_off[b];
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(__attribute__((address_space(3))) void*)(base));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(__attribute__((address_space(3))) void*)(base + 4 * PN));
          typedef short v8i16 __attribute__((ext_vector_type(8)));
          const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          bfr[b] = __builtin_bit_cast(bf16x8, both);
        } else {
          bfr[b] = *reinterpret_cast<const bf16x8*>(B + (wn * WTN + b * 32 + (lane & 31)) * LDK +
                                                    kk * 16 + (lane >> 5) * 8);
        }
      }
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  };

  // ---- activation operand: fixed rows per thread
  int64_t aoff[G::A_CHUNKS];
  bool aval[G::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < G::A_CHUNKS; ++i) {
    const int c = tid + NTHR * i;
    const int64_t pr = r0 + (c >> 3);
    aval[i] = pr < r1;
    int64_t src = pr;
    if (aval[i] && p.gather) src = p.gather[pr] / p.gdiv;
    aoff[i] = aval[i] ? src * p.lda + (c & 7) * 8 : 0;
  }

  // ---- weight operand: WPT = 2*BN/256 blocks per thread per k-step.
  // Item it = tid + 256*i; consecutive lanes read consecutive blocks of a row:
  // NT: (row = it >> 1, kb = it & 1): block 2kt + kb of weight row `row`
  // NN: (row = it / NB, kb = it % NB), NB = BN/32 blocks per row: block
  //     n0/32 + kb of reduction row kt*64 + row
  constexpr int WPT = 2 * BN / NTHR;
  constexpr int NB = BN / 32;
  int w_it_row[WPT], w_it_kb[WPT];
  const uint8_t* wptr[WPT];  // NT: row base + kb*BS;  NN: block of k-step 0 in w0
  bool wrow_ok[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int it = tid + NTHR * i;
    w_it_row[i] = NN ? (it / NB) : (it >> 1);
    w_it_kb[i] = NN ? (it % NB) : (it & 1);
    if constexpr (!NN) {
      const uint8_t* src = p.w0;
      int nrow;
      if constexpr (EPI == EPI_SWIGLU) {
        const int proj = (w_it_row[i] >> 5) & 1;
        nrow = (n0 >> 1) + (w_it_row[i] >> 6) * 32 + (w_it_row[i] & 31);
        src = proj ? p.w1 : p.w0;
      } else {
        nrow = n0 + w_it_row[i];
      }
      wrow_ok[i] = nrow < p.w_rows;
      wptr[i] = src + (int64_t)e * p.w_estride + (int64_t)(p.w_row0 + nrow) * p.w_rowbytes +
                w_it_kb[i] * BS;
    } else {
      wrow_ok[i] = ((n0 >> 5) + w_it_kb[i]) < p.w_nb;
      wptr[i] = p.w0 + (int64_t)e * p.w_estride + (int64_t)(p.w_row0 + w_it_row[i]) * p.w_rowbytes +
                (int64_t)((n0 >> 5) + w_it_kb[i]) * BS;
    }
  }
  // NN: byte offset of k-step kt from wptr -- uniform across the workgroup.
  // Rows at or past wsplit (a multiple of 64) come from w1.
  auto nn_koff = [&](int kt) {
    const int k0 = kt * BK;
    const int64_t delta = (int64_t)((uintptr_t)p.w1 - (uintptr_t)p.w0) - (int64_t)p.wsplit * p.w_rowbytes;
    // select by mask: a branch here would split the pipelined loop
    return (int64_t)k0 * p.w_rowbytes + (delta & -(int64_t)(k0 >= p.wsplit));
  };

  // A workgroup whose tile has every row, every weight column and only whole
  // k-steps runs the pipeline without masks or clamped addresses.
  bool full = (r1 - r0 == BM) && (p.K % (BK * KS) == 0);
  if constexpr (NN) {
    full = full && ((n0 >> 5) + NB <= p.w_nb);
  } else if constexpr (EPI == EPI_SWIGLU) {
    full = full && ((n0 >> 1) + BN / 2 <= p.w_rows);
  } else {
    full = full && (n0 + BN <= p.w_rows);
  }

  // ---- rank-r adapter term, folded into the accumulators on the MFMA:
  //   acc[row][col] += sum_j X(row, j) * s * Y(col, j)
  // over one k16 slice per 16 adapter ranks.  X and s*Y are split into bf16
  // hi + lo parts and accumulated as hi*hi + hi*lo + lo*hi (about 16
  // significant bits, far inside the bf16 output precision).  Row / column
  // operands follow the MFMA layout: lane l holds row (col) l%32 and ranks
  // 8*(l/32) .. +8 of the slice.
  const int r = p.r;
  const float s = p.s;
  constexpr int NSET = EPI == EPI_SWIGLU ? 2 : 1;
  constexpr bool FOLD = EPI != EPI_DH_ACC;
  // (split-K parts get the adapter term in the fixup instead).  It runs
  // before the main loop, right after the first tiles' loads are issued,
  // so the latency of its operand loads hides behind theirs; with two
  // k-groups only the first group adds it.
  auto fold_adapter = [&]() __attribute__((always_inline)) {
  if constexpr (FOLD) if (p.ksplit <= 1 && grp == 0) {
    const int rtot = EPI == EPI_GATEUP_BWD ? 2 * r : r;
    const float* Y0;
    const float* Y1 = nullptr;
    if constexpr (EPI == EPI_LIN_BWD || EPI == EPI_DOWN_BWD || EPI == EPI_GATEUP_BWD) {
      Y0 = p.lA0 + (int64_t)e * p.lA_estride;  // A [r][N]: Y(c, j) = A[j*N + c]
      if constexpr (EPI == EPI_GATEUP_BWD) Y1 = p.lA1 + (int64_t)e * p.lA_estride;
    } else if constexpr (EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) {
      Y0 = p.lB0 + (int64_t)p.w_row0 * r;      // B [V][r], columns from w_row0
    } else {
      Y0 = p.lB0 + (int64_t)e * p.lB_estride;  // B [N][r]
      if constexpr (EPI == EPI_SWIGLU) Y1 = p.lB1 + (int64_t)e * p.lB_estride;
    }
    auto split8 = [](const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)v[i];
        hi[i] = h;
        lo[i] = (__bf16)(v[i] - (float)h);
      }
    };
    for (int q = 0; q * 16 < rtot; ++q) {
      const int j0 = q * 16 + (lane >> 5) * 8;
      bf16x8 ah[TM][NSET], al[TM][NSET];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int64_t row = r0 + wm * WTM + a * 32 + (lane & 31);
        const bool ok = row < r1;
#pragma unroll
        for (int st = 0; st < NSET; ++st) {
          const float* X = st == 0 ? p.rv0 : p.rv1;
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int j = j0 + i;
            float x = 0.f;
            if (ok && j < rtot) {
              if constexpr (EPI == EPI_GATEUP_BWD) {
                x = j < r ? p.rv0[row * r + j] : p.rv1[row * r + j - r];
              } else if constexpr (EPI == EPI_LIN_BWD || EPI == EPI_LIN) {
                x = X[row * r + j];
                for (int sp = 1; sp < p.rv_parts; ++sp) x += X[sp * p.M * r + row * r + j];
                if (p.rv_out && ntile == 0 && wn == 0) p.rv_out[row * r + j] = x;
              } else {
                x = X[row * r + j];
              }
            }
            v[i] = x;
          }
          split8(v, ah[a][st], al[a][st]);
        }
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int st = EPI == EPI_SWIGLU ? (b & 1) : 0;
        int col;
        bool ok;
        if constexpr (EPI == EPI_SWIGLU) {
          col = (n0 >> 1) + (wn * (TN / 2) + (b >> 1)) * 32 + (lane & 31);
          ok = col < p.w_rows;
        } else if constexpr (EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) {
          col = n0 + LCb(b);
          ok = col < p.w_rows;
        } else {
          col = n0 + LCb(b);
          ok = col < p.N;
        }
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = j0 + i;
          float y = 0.f;
          if (ok && j < rtot) {
            if constexpr (EPI == EPI_LIN_BWD || EPI == EPI_DOWN_BWD)
              y = Y0[(int64_t)j * p.N + col];
            else if constexpr (EPI == EPI_GATEUP_BWD)
              y = j < r ? Y0[(int64_t)j * p.N + col] : Y1[(int64_t)(j - r) * p.N + col];
            else
              y = (st == 0 ? Y0 : Y1)[(int64_t)col * r + j];
          }
          v[i] = s * y;
        }
        bf16x8 bh, bl;
        split8(v, bh, bl);
#pragma unroll
        for (int a = 0; a < TM; ++a) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a][st], bh, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a][st], bl, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[a][st], bh, acc[a][b], 0, 0, 0);
        }
      }
    }
  }
  };

  auto pipeline = [&](auto full_c, auto na_c) {
    constexpr bool FULL = decltype(full_c)::value;
    constexpr int NA = decltype(na_c)::value;
    uint4 areg0[G::A_CHUNKS], areg1[G::A_CHUNKS];
    uint32_t amsk0[G::A_CHUNKS], amsk1[G::A_CHUNKS];
    auto load_a = [&](int kt, uint4 (&areg)[G::A_CHUNKS], uint32_t (&amsk)[G::A_CHUNKS]) {
      int k0 = kt * BK;
      const uint16_t* base = p.a0;
      if (k0 >= p.asplit) { base = p.a1; k0 -= p.asplit; }
#pragma unroll
      for (int i = 0; i < G::A_CHUNKS; ++i) {
        if constexpr (FULL) {
          areg[i] = *reinterpret_cast<const uint4*>(base + aoff[i] + k0);
        } else {
          // unconditional load from a clamped address, zeroed at the LDS
          // store (so nothing waits for it here), so the steady-state loop
          // stays one basic block
          const int kc = kt * BK + ((tid + NTHR * i) & 7) * 8;
          const bool ok = aval[i] && kc < p.K;
          areg[i] = *reinterpret_cast<const uint4*>(ok ? base + aoff[i] + k0 : p.a0);
          amsk[i] = opaque_mask(ok);
        }
      }
    };
    auto store_a = [&](int buf, const uint4 (&areg)[G::A_CHUNKS], const uint32_t (&amsk)[G::A_CHUNKS]) {
      uint16_t* A = As + buf * BM * LDK;
#pragma unroll
      for (int i = 0; i < G::A_CHUNKS; ++i) {
        const int c = tid + NTHR * i;
        uint4 v = areg[i];
        if constexpr (!FULL) {
          const uint32_t m = amsk[i];
          v = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
        }
        *reinterpret_cast<uint4*>(A + (c >> 3) * LDK + (c & 7) * 8) = v;
      }
    };
    RawBlock<QT> wr0[WPT], wr1[WPT];
    uint32_t wmsk0[WPT], wmsk1[WPT];
    auto load_w = [&](int kt, RawBlock<QT> (&wr)[WPT], uint32_t (&wmsk)[WPT]) {
      const int64_t koff = NN ? nn_koff(kt) : (int64_t)kt * 2 * BS;
#pragma unroll
      for (int i = 0; i < WPT; ++i) {
        if constexpr (FULL) {
          load_block<QT>(wptr[i] + koff, wr[i]);
        } else {
          // unconditional load (block 0 of w0 when out of range), zeroed at
          // the store; branch-free address selection keeps the loop one block
          // NT: block 2kt + kb of the row must exist (a reduction of an odd
          // number of blocks ends in a half k-step)
          const bool ok = wrow_ok[i] && (NN ? kt * BK + w_it_row[i] < p.K : 2 * kt + w_it_kb[i] < p.w_nb);
          load_block<QT>(ok ? wptr[i] + koff : p.w0, wr[i]);
          wmsk[i] = opaque_mask(ok);
        }
      }
    };
    auto store_w = [&](int buf, const RawBlock<QT> (&wraw)[WPT], const uint32_t (&wmsk)[WPT]) {
      uint16_t* B = Bs + buf * B_TILE;
#pragma unroll
      for (int i = 0; i < WPT; ++i) {
        RawBlock<QT> wr = wraw[i];
        if constexpr (!FULL) {
          wr.hdr &= wmsk[i];
#pragma unroll
          for (int q = 0; q < RawBlock<QT>::NQ; ++q) wr.q[q] &= wmsk[i];
        }
        uint32_t o[16];
        decode_block_bf16<QT>(wr, o);
        // NT: row w_it_row of the [n][k] tile, k = kb*32 .. +32
        // NN: reduction row w_it_row of the row-major tile, columns kb*32 .. +32
        uint4* dst = reinterpret_cast<uint4*>(B + w_it_row[i] * (NN ? PN : LDK));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = w_it_kb[i] * 4 + q;
          dst[NN ? nn_chunk(w_it_row[i], c) : c] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        }
      }
    };

    // Software pipeline, prefetch depth 2: tile kt+2 is loaded into the
    // register set that tile kt was stored from, while the MFMAs of tile kt
    // run and tile kt+1 (loaded one step earlier) waits in the other set.
    load_a(KT(0), areg0, amsk0);
    load_w(KT(0), wr0, wmsk0);
    if (nkl > 1) {
      load_a(KT(1), areg1, amsk1);
      load_w(KT(1), wr1, wmsk1);
    }
    fold_adapter();
    store_a(0, areg0, amsk0);
    store_w(0, wr0, wmsk0);
    __syncthreads();
    int kt = 0;
    // steady state without branches, so the decode of the next tile can be
    // scheduled among the MFMAs of the current one (the scheduling fence
    // keeps the loads ahead of the decode of the other set, which would
    // otherwise wait for them)
    for (; kt + 3 < nkl; kt += 2) {
      load_a(KT(kt + 2), areg0, amsk0);
      load_w(KT(kt + 2), wr0, wmsk0);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, na_c);
      store_a(1, areg1, amsk1);
      store_w(1, wr1, wmsk1);
      mfma_interleave<NA * TN * (BK / 16), 6, NN ? 4 : 2, 8>();
      __syncthreads();
      load_a(KT(kt + 3), areg1, amsk1);
      load_w(KT(kt + 3), wr1, wmsk1);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, na_c);
      store_a(0, areg0, amsk0);
      store_w(0, wr0, wmsk0);
      mfma_interleave<NA * TN * (BK / 16), 6, NN ? 4 : 2, 8>();
      __syncthreads();
    }
    // tail: tiles kt .. nkl-1 (at most three)
    for (; kt < nkl; kt += 2) {
      if (kt + 2 < nkl) {
        load_a(KT(kt + 2), areg0, amsk0);
        load_w(KT(kt + 2), wr0, wmsk0);
      }
      compute(0, na_c);
      if (kt + 1 < nkl) {
        store_a(1, areg1, amsk1);
        store_w(1, wr1, wmsk1);
      }
      __syncthreads();
      if (kt + 1 >= nkl) break;
      compute(1, na_c);
      if (kt + 2 < nkl) {
        store_a(0, areg0, amsk0);
        store_w(0, wr0, wmsk0);
      }
      __syncthreads();
    }
  };
  if (full) {
    pipeline(BoolC<true>{}, IntC<TM>{});
  } else {
    // this wave's rows wm*WTM .. +WTM of the tile, in 32-row sub-tiles
    const int64_t left = r1 - r0 - (int64_t)wm * WTM;
    const int nact = left <= 0 ? 0 : (left >= WTM ? TM : (int)((left + 31) / 32));
    if (nact >= TM)
      pipeline(BoolC<false>{}, IntC<TM>{});
    else if (TM == 2 && nact == 1)
      pipeline(BoolC<false>{}, IntC<(TM > 1 ? 1 : TM)>{});
    else
      pipeline(BoolC<false>{}, IntC<0>{});
  }

  if constexpr (KS > 1) {
    // fold the second group's partial sums into the first group's
    // accumulators (fixed order: deterministic), then retire the second
    // group; everything below is barrier-free
    __syncthreads();
    float4* red = reinterpret_cast<float4*>(smem);
    const int slot0 = wave * TM * TN;
    if (grp == 1) {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            red[((slot0 + a * TN + b) * 4 + v4) * 64 + lane] =
                make_float4(acc[a][b][4 * v4], acc[a][b][4 * v4 + 1], acc[a][b][4 * v4 + 2],
                            acc[a][b][4 * v4 + 3]);
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 q = red[((slot0 + a * TN + b) * 4 + v4) * 64 + lane];
          acc[a][b][4 * v4] += q.x;
          acc[a][b][4 * v4 + 1] += q.y;
          acc[a][b][4 * v4 + 2] += q.z;
          acc[a][b][4 * v4 + 3] += q.w;
        }
  }

  // ---- epilogues.  acc[a][b][v] sits at local row
  //   lr = wm*WTM + a*32 + (v>>2)*8 + (lane>>5)*4 + (v&3), local col lc = wn*WTN + b*32 + (lane&31)
  auto LR = [&](int a, int v) { return wm * WTM + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); };
  auto LC = [&](int b) { return LCb(b); };

  if constexpr (EPI == EPI_LIN || EPI == EPI_LIN_BWD) {
    if (p.ksplit > 1) {
      // this k-range's fp32 sums, summed with the others by the fixup
      float* P = p.part + (int64_t)ksidx * p.M * p.N;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int n = n0 + LC(b);
        if (n >= p.N) continue;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t pr = r0 + LR(a, v);
            if (pr < r1) P[pr * p.N + n] = acc[a][b][v];
          }
      }
      return;
    }
  }
  if constexpr (EPI == EPI_LIN || EPI == EPI_LIN_BWD || EPI == EPI_GATEUP_BWD) {
    // the wave's WTM x WTN output tile goes through a wave-private LDS
    // region (rows of WTN + 8 bf16) and leaves as 16-byte row stores (8
    // lanes per 128-byte row segment) -- when the output rows allow 16-byte
    // stores; else one 2-byte store per value.  The region lies past the
    // split-K reduction buffer, which other waves may still be reading.
    const bool vec = ((uintptr_t)p.o0 % 16 == 0) && (p.ldo % 8 == 0) && (p.N % 8 == 0);
    if (vec) {
      constexpr int SP = WTN + 8;
      uint16_t* Ws = reinterpret_cast<uint16_t*>(smem + (KS > 1 ? BM * BN * 4 : 0)) + wave * WTM * SP;
      static_assert((KS > 1 ? BM * BN * 4 : 0) + 4 * WTM * SP * 2 <= G::SMEM, "staging fits");
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            Ws[(a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * SP + b * 32 + (lane & 31)] =
                f2bf(acc[a][b][v]);
      // (the wave's own region: its LDS writes complete before these reads)
      constexpr int CH = WTN / 8;
      const int64_t rbase = r0 + wm * WTM;
      const int cbase = n0 + wn * WTN;
#pragma unroll
      for (int i = lane; i < WTM * CH; i += 64) {
        const int rr = i / CH, cc = (i % CH) * 8;
        const int64_t pr = rbase + rr;
        const int n = cbase + cc;
        if (pr < r1 && n < p.N)
          *reinterpret_cast<uint4*>(p.o0 + pr * p.ldo + n) = *reinterpret_cast<const uint4*>(Ws + rr * SP + cc);
      }
    } else {
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int n = n0 + LC(b);
        if (n >= p.N) continue;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t pr = r0 + LR(a, v);
            if (pr < r1) p.o0[pr * p.ldo + n] = f2bf(acc[a][b][v]);
          }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // n-subtiles come in (gate, up) pairs over the same 32 intermediate
    // rows.  h, g, u of the wave's WTM x IW block go through a wave-private
    // LDS region (three arrays, rows of IW + 8 bf16, past the split-K
    // reduction buffer) and leave as 16-byte row stores when the rows allow
    // it; else one 2-byte store per value.
    constexpr int IW = TN / 2 * 32;  // intermediate columns of the wave
    const int ibase = (n0 >> 1) + wn * IW;
    const bool vec = ((uintptr_t)p.o0 % 16 == 0) && ((uintptr_t)p.o1 % 16 == 0) &&
                     ((uintptr_t)p.o2 % 16 == 0) && (p.ldo % 8 == 0) && (p.w_rows % 8 == 0);
    if (vec) {
      constexpr int SPI = IW + 8;
      uint16_t* Ws = reinterpret_cast<uint16_t*>(smem + (KS > 1 ? BM * BN * 4 : 0)) + wave * 3 * WTM * SPI;
      static_assert((KS > 1 ? BM * BN * 4 : 0) + 4 * 3 * WTM * SPI * 2 <= G::SMEM, "staging fits");
#pragma unroll
      for (int b2 = 0; b2 < TN / 2; ++b2)
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int lw = a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            const float g = acc[a][2 * b2][v];
            const float u = acc[a][2 * b2 + 1][v];
            const float h = g * sigmoidf_(g) * u;
            const int c = b2 * 32 + (lane & 31);
            Ws[lw * SPI + c] = f2bf(h);
            Ws[(WTM + lw) * SPI + c] = f2bf(g);
            Ws[(2 * WTM + lw) * SPI + c] = f2bf(u);
          }
      // (the wave's own region: its LDS writes complete before these reads)
      constexpr int CH = IW / 8;
#pragma unroll
      for (int i = lane; i < 3 * WTM * CH; i += 64) {
        const int arr = i / (WTM * CH), q = i % (WTM * CH), rr = q / CH, cc = (q % CH) * 8;
        const int64_t pr = r0 + wm * WTM + rr;
        const int ic = ibase + cc;
        if (pr < r1 && ic < p.w_rows) {
          uint16_t* dst = arr == 0 ? p.o0 : (arr == 1 ? p.o1 : p.o2);
          *reinterpret_cast<uint4*>(dst + pr * p.ldo + ic) =
              *reinterpret_cast<const uint4*>(Ws + (arr * WTM + rr) * SPI + cc);
        }
      }
    } else {
#pragma unroll
      for (int b2 = 0; b2 < TN / 2; ++b2) {
        const int i = ibase + b2 * 32 + (lane & 31);
        if (i >= p.w_rows) continue;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t pr = r0 + LR(a, v);
            if (pr < r1) {
              const float g = acc[a][2 * b2][v];
              const float u = acc[a][2 * b2 + 1][v];
              const float h = g * sigmoidf_(g) * u;
              const int64_t o = pr * p.ldo + i;
              p.o0[o] = f2bf(h);
              p.o1[o] = f2bf(g);
              p.o2[o] = f2bf(u);
            }
          }
      }
    }
  } else if constexpr (EPI == EPI_DH_ACC) {
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int c = n0 + LC(b);
      if (c >= p.N) continue;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t pr = r0 + LR(a, v);
          if (pr < r1) {
            float* d = p.f0 + pr * p.ldf + c;
            *d = p.accum ? *d + acc[a][b][v] : acc[a][b][v];
          }
        }
    }
  } else if constexpr (EPI == EPI_DOWN_BWD) {
    // Columns are the expert's intermediate index i (< N = I); acc holds
    // e = dY deq(Wd) + s (dY Bd) Ad.  e is staged row-major in LDS; 4
    // threads then share a row, 8 columns at a time: 16-byte loads of the
    // saved g, u, the SwiGLU backward, 16-byte stores of dg, du (bf16), and
    // the row partials of this column tile: dw = sum e*silu(g)*u, dgB =
    // sum dg*Bg, duB = sum du*Bu (with the stored bf16 dg, du).  Bg, Bu of
    // the tile's columns sit in LDS, 8 ranks at a time: rank 16 takes a
    // second pass over the rows for ranks 8..15 (recomputing dg, du, no
    // stores).
    constexpr int ZD = BN + 4;
    float* Z = reinterpret_cast<float*>(smem);
    float* Bst = Z + BM * ZD;  // [2][BN][8]
    const int width = 1 + 2 * r;
    const float* Bg = p.lB1 + (int64_t)e * p.lB_estride;
    const float* Bu = p.lB2 + (int64_t)e * p.lB_estride;
    constexpr int BSTN = 2 * BN * 8 / NTHR;  // Bst values per thread
    auto bst_value = [&](int idx, int jb) {
      const int mat = idx / (BN * 8), c = (idx >> 3) % BN, j = idx & 7;
      const int col = n0 + c;
      return (jb + j < r && col < p.N) ? (mat ? Bu : Bg)[(int64_t)col * r + jb + j] : 0.f;
    };
    // the first 8 ranks of Bg, Bu are loaded before the LDS staging (their
    // latency overlaps it)
    float bsv[BSTN];
#pragma unroll
    for (int i = 0; i < BSTN; ++i) bsv[i] = bst_value(tid + NTHR * i, 0);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) Z[LR(a, v) * ZD + LC(b)] = acc[a][b][v];
    // TPR threads per tile row (2 for 128-row tiles, one pass over the
    // rows; 4 for 64-row tiles), CPT chunks of 8 columns each, RPP rows per
    // pass; the row partials are summed over the row's threads with xor
    // shuffles (fixed order) and written by its first thread
    constexpr int TPR = BM >= 128 ? 2 : 4, RPP = NTHR / TPR, CPT = BN / TPR / 8;
    static_assert(BM % RPP == 0, "whole row passes");
    const int cq = tid % TPR, rsub = tid / TPR;
    auto segment = [&](auto rc, const int jb) {
      constexpr int R = decltype(rc)::value;
      const bool first = jb == 0;
      for (int pass = 0; pass < BM / RPP; ++pass) {
        if (r0 + pass * RPP >= r1) break;  // workgroup-uniform: no rows left
        const int row = pass * RPP + rsub;
        const int64_t pr = r0 + row;
        float dw = 0.f, ag[R], au[R];
#pragma unroll
        for (int j = 0; j < R; ++j) ag[j] = au[j] = 0.f;
        const float wp = pr < r1 ? p.wflat[p.sorted[pr]] : 0.f;
#pragma unroll
        for (int ch = 0; ch < CPT; ++ch) {
          const int lc = (ch * TPR + cq) * 8;
          const int c = n0 + lc;
          const bool ok = pr < r1 && c < p.N;  // N % 8 == 0: whole 8-column chunks
          if (ok) {
            const int64_t o = pr * p.ldo + c;
            const uint4 g8 = *reinterpret_cast<const uint4*>(p.s0 + o);
            const uint4 u8 = *reinterpret_cast<const uint4*>(p.s1 + o);
            const float4 e0 = *reinterpret_cast<const float4*>(Z + row * ZD + lc);
            const float4 e1 = *reinterpret_cast<const float4*>(Z + row * ZD + lc + 4);
            const uint32_t gw[4] = {g8.x, g8.y, g8.z, g8.w}, uw[4] = {u8.x, u8.y, u8.z, u8.w};
            const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
            uint32_t dgp[4], dup[4];
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
              float dgv[2], duv[2];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float gg = bf2f((uint16_t)(gw[t2] >> (16 * h)));
                const float uu = bf2f((uint16_t)(uw[t2] >> (16 * h)));
                const float eh = ev[2 * t2 + h];
                const float sg = sigmoidf_(gg);
                const float silu = gg * sg;
                const float dh = wp * eh;
                dgv[h] = dh * uu * sg * (1.f + gg * (1.f - sg));
                duv[h] = dh * silu;
                dw += eh * silu * uu;
              }
              dgp[t2] = pack_bf2(dgv[0], dgv[1]);
              dup[t2] = pack_bf2(duv[0], duv[1]);
            }
            if (first) {
              *reinterpret_cast<uint4*>(p.o0 + o) = make_uint4(dgp[0], dgp[1], dgp[2], dgp[3]);
              *reinterpret_cast<uint4*>(p.o1 + o) = make_uint4(dup[0], dup[1], dup[2], dup[3]);
            }
            // rank partials of the eight columns (with the stored bf16 dg, du)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const float dq = __builtin_bit_cast(float, (dgp[t >> 1] >> (16 * (t & 1))) << 16);
              const float uq = __builtin_bit_cast(float, (dup[t >> 1] >> (16 * (t & 1))) << 16);
#pragma unroll
              for (int j = 0; j < R; ++j) {
                ag[j] += dq * Bst[(lc + t) * 8 + j];
                au[j] += uq * Bst[(BN + lc + t) * 8 + j];
              }
            }
          }
        }
#pragma unroll
        for (int o2 = 1; o2 < TPR; o2 <<= 1) {
          dw += __shfl_xor(dw, o2, TPR);
#pragma unroll
          for (int j = 0; j < R; ++j) {
            ag[j] += __shfl_xor(ag[j], o2, TPR);
            au[j] += __shfl_xor(au[j], o2, TPR);
          }
        }
        if (cq == 0 && pr < r1) {
          float* dst = p.f0 + ((int64_t)ntile * p.M + pr) * width;
          if (first) dst[0] = dw;
#pragma unroll
          for (int j = 0; j < R; ++j) {
            if (jb + j < r) {
              dst[1 + jb + j] = ag[j];
              dst[1 + r + jb + j] = au[j];
            }
          }
        }
      }
    };
    for (int jb = 0; jb < r; jb += 8) {
      if (jb) {
        __syncthreads();  // the previous pass is done with Bst
#pragma unroll
        for (int i = 0; i < BSTN; ++i) bsv[i] = bst_value(tid + NTHR * i, jb);
      }
#pragma unroll
      for (int i = 0; i < BSTN; ++i) Bst[tid + NTHR * i] = bsv[i];
      __syncthreads();
      if (r - jb <= 4)
        segment(IntC<4>{}, jb);
      else
        segment(IntC<8>{}, jb);
    }
  } else if constexpr (EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) {
    // acc holds the logits z of this tile (adapter term included)
    float* Z = reinterpret_cast<float*>(smem);
    const int64_t V = p.V;
    const int64_t c0 = p.w_row0;  // vocab offset of this launch's columns
    float coef = 0.f;
    if constexpr (EPI == EPI_CE_BWD) {
      const float nv = *p.nvalid;
      coef = nv > 0.f ? p.coef / nv : 0.f;
    }
    // the gradient tile G (bwd) or the logits (fwd), staged in Z
    auto gval = [&](int a, int b, int v, int64_t pr, int n) {
      const int64_t vv = c0 + n;
      const int64_t lab = p.labels[pr];
      const bool valid = lab != p.ignore_index && lab >= 0 && lab < V;
      if (!valid || n >= p.w_rows) return 0.f;
      return coef * (__expf(acc[a][b][v] - p.lse[pr]) - (vv == lab ? 1.f : 0.f));
    };
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int lc = LC(b);
      const int n = n0 + lc;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = LR(a, v);
          const int64_t pr = r0 + lr;
          float zv;
          if constexpr (EPI == EPI_CE_FWD) {
            zv = (pr < r1 && n < p.w_rows) ? acc[a][b][v] : -INFINITY;
          } else {
            zv = pr < r1 ? gval(a, b, v, pr, n) : 0.f;
            acc[a][b][v] = zv;  // G, restaged below without recomputing
          }
          Z[lr * ZP + lc] = zv;
        }
    }
    __syncthreads();
    if constexpr (EPI == EPI_CE_FWD) {
      // per-row online (max, sumexp) over this tile, label logit pick
      constexpr int NSEG = NTHR / BM, SEGC = BN / NSEG;
      const int row = tid % BM, seg = tid / BM;
      float m = -INFINITY, l = 0.f;
      for (int c = seg * SEGC; c < (seg + 1) * SEGC; ++c) m = fmaxf(m, Z[row * ZP + c]);
      if (m != -INFINITY)
        for (int c = seg * SEGC; c < (seg + 1) * SEGC; ++c) l += __expf(Z[row * ZP + c] - m);
      const int64_t pr = r0 + row;
      float zl = 0.f;
      bool have_lab = false;
      if (pr < r1) {
        const int64_t lab = p.labels[pr];
        const int64_t lc = lab - c0 - n0;
        if (lab != p.ignore_index && lab >= 0 && lab < V && lc >= seg * SEGC &&
            lc < (seg + 1) * SEGC) {
          zl = Z[row * ZP + lc];
          have_lab = true;
        }
      }
      __syncthreads();
      float* X = Z;
      if (seg > 0) {
        X[(seg * BM + row) * 2 + 0] = m;
        X[(seg * BM + row) * 2 + 1] = l;
      }
      __syncthreads();
      if (seg == 0) {
        for (int sg = 1; sg < NSEG; ++sg) {
          const float m2 = X[(sg * BM + row) * 2 + 0], l2 = X[(sg * BM + row) * 2 + 1];
          const float mn = fmaxf(m, m2);
          if (mn != -INFINITY) {
            l = (m == -INFINITY ? 0.f : l * __expf(m - mn)) + (m2 == -INFINITY ? 0.f : l2 * __expf(m2 - mn));
            m = mn;
          }
        }
        if (pr < r1) {
          float* dst = p.f0 + ((int64_t)(p.ntile_base + ntile) * p.M + pr) * 2;
          dst[0] = m;
          dst[1] = l;
        }
      }
      if (have_lab) p.f1[pr] = zl;
    } else {
      // the G tile to bf16, rows stored with 16-byte stores from the staged
      // copy (two threads per row, 8 columns per store)
      {
        const int row = tid >> 1, half = tid & 1;
        const int64_t pr = r0 + row;
        if (pr < r1) {
#pragma unroll
          for (int q8 = 0; q8 < BN / 16; ++q8) {
            const int c = half * (BN / 2) + q8 * 8;
            if (n0 + c < p.ldo) {
              const float* z = Z + row * ZP + c;
              *reinterpret_cast<uint4*>(p.o0 + pr * p.ldo + n0 + c) =
                  make_uint4(pack_bf2(z[0], z[1]), pack_bf2(z[2], z[3]), pack_bf2(z[4], z[5]),
                             pack_bf2(z[6], z[7]));
            }
          }
        }
      }
      // G . B over this tile's vocab columns -> part_GB[ntile][T][r], then
      // G^T . xa over this tile's rows -> part_dB[mtile][V][r] (G restaged
      // from the accumulators); the rank vectors go through the LDS area
      // behind the staged tile
      float* S = reinterpret_cast<float*>(smem + BM * (BN + 4) * 4);
      auto reductions = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        static_assert(BN * R * 4 <= 2 * BN * 8 * 4 && BM * R * 4 <= 2 * BN * 8 * 4, "staging fits");
        z_row_reduce<BM, BN, R>(Z, S, p.lB0 + c0 * r, r, n0, p.w_rows, [&](int row, float(&out)[R]) {
          const int64_t pr = r0 + row;
          if (pr < r1) {
            float* dst = p.f1 + ((int64_t)(p.ntile_base + ntile) * p.M + pr) * r;
#pragma unroll
            for (int j = 0; j < R; ++j)
              if (j < r) dst[j] = out[j];
          }
        });
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int v = 0; v < 16; ++v) Z[LR(a, v) * ZP + LC(b)] = acc[a][b][v];
        __syncthreads();
        z_col_reduce<BM, BN, R>(Z, S, p.rv0, r, r0, r1, [&](int col, float(&out)[R]) {
          const int n = n0 + col;
          if (n < p.w_rows) {
            float* dst = p.f2 + ((int64_t)mslot * V + c0 + n) * r;
#pragma unroll
            for (int j = 0; j < R; ++j)
              if (j < r) dst[j] = out[j];
          }
        });
      };
      if (r <= 4)
        reductions(IntC<4>{});
      else if (r <= 8)
        reductions(IntC<8>{});
      else
        reductions(IntC<16>{});
    }
  }
}

template <int QT, int EPI, int BM, int BN, int KS>
__global__ __launch_bounds__(NTHR * KS, (KS > 1 || BM * BN >= 256 * 256) ? 1 : 2) void gemm_kernel(
    const GemmArgs p) {
  using G = Geom<BM, BN, epi_stages(EPI), EPI >= EPI_LIN_BWD, KS>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::SMEM];
  gemm_body<QT, EPI, BM, BN, KS>(p, smem, (int)blockIdx.x, (int)gridDim.x);
}

// LM-head backward, two chunks in one launch: the first `nce` workgroups
// are the gradient tiles of chunk c (EPI_CE_BWD, writing one G buffer), the
// rest the dh tiles of chunk c-1 (EPI_DH_ACC, reading the other G buffer).
// The two kinds share nothing, so the dh tiles fill the CUs while the
// gradient tiles' epilogues run, instead of two single-round launches
// back to back.
template <int QT>
__global__ __launch_bounds__(NTHR, 2) void ce_bwd_dh_kernel(const GemmArgs pce, const GemmArgs pdh,
                                                            const int nce) {
  using GC = Geom<128, 128, true, false, 1>;
  using GD = Geom<128, 128, false, true, 1>;
  constexpr int SM = GC::SMEM > GD::SMEM ? GC::SMEM : GD::SMEM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM];
  if ((int)blockIdx.x < nce)
    gemm_body<QT, EPI_CE_BWD, 128, 128, 1>(pce, smem, (int)blockIdx.x, nce);
  else
    gemm_body<QT, EPI_DH_ACC, 128, 128, 1>(pdh, smem, (int)blockIdx.x - nce, (int)gridDim.x - nce);
}

template <int QT, int EPI>
hipError_t launch_skinny(int rg, const GemmArgs& a, hipStream_t st);
template <int QT, int EPI>
hipError_t launch_skinny_nn(int rg, const GemmArgs& a, hipStream_t st);

template <int QT, int EPI>
hipError_t launch_wide(const GemmArgs& a, hipStream_t st);
template <int QT, int EPI>
hipError_t launch_wide_nn(const GemmArgs& a, hipStream_t st);

template <int QT, int EPI>
hipError_t launch_q(int tilecfg, const GemmArgs& a, hipStream_t st) {
  if (tilecfg == TILE_WIDE_NN) {
    if constexpr (EPI == EPI_DH_ACC && QT != QT_Q2_DM) {
      // dense, one or two reduction ranges (a range without k-steps stores
      // zero sums), activation rows holding K rounded up to 64 columns
      const int64_t nkall = ((int64_t)a.K + GEMM_BK - 1) / GEMM_BK;
      if (a.offsets || a.gather || a.K < 1 || a.ksplit > 2 || a.lda < nkall * GEMM_BK || a.asplit < a.K ||
          a.wsplit < a.K || a.N > 32 * a.w_nb || a.N % 4)
        return hipErrorInvalidValue;
      // the range sums leave as 16-byte row pieces
      if (!a.f0 || (uintptr_t)a.f0 % 16 || a.ldf % 4) return hipErrorInvalidValue;
      return launch_wide_nn<QT, EPI>(a, st);
    }
    return hipErrorInvalidValue;
  }
  const unsigned splits = a.ksplit > 1 ? (unsigned)a.ksplit : 1u;
  if (splits > 1) {  // dense EPI_LIN / EPI_LIN_BWD on one group of four waves, whole k-steps
    if (a.offsets || a.K % GEMM_BK || tilecfg == TILE_128x128_K2 || tile_skinny(tilecfg) ||
        tilecfg == TILE_WIDE || !(EPI == EPI_LIN || EPI == EPI_LIN_BWD) || !a.part)
      return hipErrorInvalidValue;
  }
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles * splits);
  if (tilecfg == TILE_WIDE) {
    if constexpr ((EPI == EPI_LIN || EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) && QT != QT_Q2_DM) {
      if (a.offsets || a.gather || a.K % GEMM_BK || a.r > WIDE_MAX_RANK) return hipErrorInvalidValue;
      return launch_wide<QT, EPI>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (EPI == EPI_LIN || EPI == EPI_SWIGLU || EPI == EPI_CE_FWD) {
    if (tile_skinny(tilecfg)) return launch_skinny<QT, EPI>(tile_bm(tilecfg) / 16, a, st);
  }
  if constexpr (EPI == EPI_LIN_BWD || EPI == EPI_GATEUP_BWD || EPI == EPI_DOWN_BWD) {
    if (tile_skinny(tilecfg)) {
      if (tile_bm(tilecfg) > 32) return hipErrorInvalidValue;
      return launch_skinny_nn<QT, EPI>(tile_bm(tilecfg) / 16, a, st);
    }
  }
  if constexpr (!epi_stages(EPI)) {
    if (tilecfg == TILE_128x128_K2) {
      mmq_launch((gemm_kernel<QT, EPI, 128, 128, 2>), grid, dim3(2 * NTHR), st, a);
      return hipGetLastError();
    }
  }
  if (tilecfg == TILE_128x128)
    mmq_launch((gemm_kernel<QT, EPI, 128, 128, 1>), grid, dim3(NTHR), st, a);
  else
    mmq_launch((gemm_kernel<QT, EPI, 64, 128, 1>), grid, dim3(NTHR), st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace gq
