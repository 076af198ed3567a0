// Wide-tile MMQ for large dense forward launches (the reduction runs along
// the weight's block dimension): 256 x 192 output tiles on 512 threads, for
// the linear forward and the LM head's logits pass.
//
// The tile GEMM in gq_gemm_impl.h decodes each 64-deep weight slice for 128
// activation rows; here every decoded slice feeds 256 rows, which halves the
// block-decode VALU per MFMA, and each wave's 64 x 96 share of the tile needs
// 0.83 KB of LDS operand reads per 32x32x16 MFMA instead of 1 KB.  Eight
// waves (two per SIMD) keep the decode of the next slice overlapped with the
// matrix cores, and a 2048 x 6144 output is exactly one tile per CU.
//
//  * Activations: 256 rows x 64 bf16 per k-step, four coalesced 16-byte loads
//    per thread into registers, stored into a padded LDS tile one step later.
//  * Weights: the 192 rows x 2 blocks of a k-step as quarter-block items
//    (three per thread): the fp16 scale plus one quarter of the payload,
//    decoded to bf16 into the [n][k] LDS tile.
//  * Double-buffered LDS, one barrier per k-step, loads two steps ahead.
//  * Rows past M and weight rows past N are clamped to the last valid row
//    (their results are never stored), so the pipeline has no masks; K must
//    be a multiple of 64.
//  * The rank-r adapter term is folded into the accumulators as extra k16
//    MFMA slices (bf16 hi + lo parts), as in the tile GEMM.
//  * The LM head's backward uses the same tile for its gradient tiles
//    (EPI_CE_BWD): several vocabulary chunks per launch, so that the tiles
//    fill whole rounds of the chip.
#pragma once
#include "gq_dev.h"
#include "gq_internal.h"

namespace gq {
namespace wide {

constexpr int BM = 256, BN = 192, BK = 64, LDK = BK + 8, NTHR = 512;
constexpr int TM = 2, TN = 3;      // 32x32 sub-tiles per wave (64 x 96)
constexpr int WTM = 64, WTN = 96;  // wave tile
constexpr int A_ST = BM * LDK, B_ST = BN * LDK;
constexpr int SMEM_MAIN = (2 * A_ST + 2 * B_ST) * 2;
constexpr int SP = WTN + 8;  // staged epilogue row pitch (bf16)
constexpr int SMEM_EPI = 8 * WTM * SP * 2;
constexpr int SMEM = SMEM_MAIN > SMEM_EPI ? SMEM_MAIN : SMEM_EPI;
static_assert(BM * 2 * 16 * 8 + (BM + 64) * 4 <= SMEM, "CE partial pairs and label logits fit the LDS");
// CE gradient epilogue: one wave column's half of the tile as fp32 [BM][HP],
// then four ranks of the tile rows' xa (BM x 4) and of the half's B rows
// (WTN x 4)
constexpr int HP = WTN + 1;
constexpr int CEB_Z = BM * HP * 4, CEB_X = BM * 4 * 4, CEB_B = WTN * 4 * 4;
static_assert(CEB_Z + CEB_X + CEB_B <= SMEM, "CE gradient staging fits the LDS");
static_assert(3 * WTN * 5 * 4 <= CEB_Z, "column partials fit the staged half");
// Past the pipeline / epilogue area, written before the main loop and read
// after it: the adapter-fold operands of the tile (xa rows and s*B rows as
// bf16 hi + lo, 16 ranks, zero past the rank or the tile's valid rows /
// columns), and per row the label's column relative to the tile (-1 or BN
// when it lies in another tile, NO_LABEL when the label is ignored) and the
// row's log-sum-exp.
constexpr int FR = WIDE_MAX_RANK;
constexpr int FOLD_OFF = SMEM;
constexpr int FOLD_BYTES = (2 * BM * FR + 2 * BN * FR) * 2;
constexpr int ROW_OFF = FOLD_OFF + FOLD_BYTES;
constexpr int SMEM_ALL = ROW_OFF + BM * 8;
static_assert(FR == 16, "one k16 slice of adapter ranks");
constexpr int32_t NO_LABEL = -(1 << 20);
static_assert(SMEM_ALL <= 160 * 1024, "fits the CU's LDS");

// A quarter of a block: its fp16 scale (low 16 bits of hdr) and payload
// bytes [q*NB, q*NB + NB) with NB = 4 (Q4_0) or 8 (Q8_0).
template <int QT> struct QuarterBytes;
template <> struct QuarterBytes<QT_Q4_0> { static constexpr int NQ = 1; };
template <> struct QuarterBytes<QT_Q8_0> { static constexpr int NQ = 2; };
template <int QT> struct RawQuarter {
  uint32_t hdr;
  uint32_t q[QuarterBytes<QT>::NQ];
};

template <int QT>
__device__ __forceinline__ void load_quarter(const uint8_t* blk, int qq, RawQuarter<QT>& r) {
  typedef const __attribute__((address_space(1))) uint16_t g_u16;
  typedef const __attribute__((address_space(1))) u32_a2 g_u32a2;
  r.hdr = *(const g_u16*)blk;
  const g_u32a2* q = (const g_u32a2*)(blk + 2 + 4 * QuarterBytes<QT>::NQ * qq);
#pragma unroll
  for (int i = 0; i < QuarterBytes<QT>::NQ; ++i) r.q[i] = q[i];
}

// Decode one quarter and store it into the [n][k] tile row `base` (the
// block's first element).  Same arithmetic as decode_block_fast: every
// product is exact, the bf16 value is d*q rounded once.
//  Q4_0 quarter qq: bytes 4qq..4qq+3 -> elements 4qq.. (low nibbles) and
//                   16+4qq.. (high nibbles)
//  Q8_0 quarter qq: bytes 8qq..8qq+7 -> elements 8qq..8qq+7
template <int QT>
__device__ __forceinline__ void store_quarter(uint16_t* base, int qq, const RawQuarter<QT>& r) {
  const float d = h2f(r.hdr & 0xffffu);
  if constexpr (QT == QT_Q4_0) {
    const float off = -8.f * d;
    const uint32_t lo = r.q[0] & 0x0f0f0f0fu, hi = (r.q[0] >> 4) & 0x0f0f0f0fu;
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __builtin_fmaf(ubyte(lo, i), d, off);
      b[i] = __builtin_fmaf(ubyte(hi, i), d, off);
    }
    *reinterpret_cast<uint2*>(base + 4 * qq) = make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
    *reinterpret_cast<uint2*>(base + 16 + 4 * qq) = make_uint2(pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3]));
  } else {
    const float off = -128.f * d;
    float v[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t u = r.q[h] ^ 0x80808080u;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * h + i] = __builtin_fmaf(ubyte(u, i), d, off);
    }
    *reinterpret_cast<uint4*>(base + 8 * qq) =
        make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
  }
}

// Merge of two (max, sum of exp) pairs into (m, l) with one exp and no
// branch; a pair with max -inf has sum 0.
__device__ __forceinline__ void ml_merge1(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  const float e = __expf(mn == -INFINITY ? 0.f : -fabsf(m - m2));
  l = m >= m2 ? l + l2 * e : l * e + l2;
  m = mn;
}

// CE gradient epilogue of a 256 x 192 tile.  The accumulators hold the
// logits z of the tile (adapter term included); they are turned into G in
// place, then each wave column's 96-column half goes through LDS as fp32:
// its bf16 rows go out as 16-byte stores, the row sums G . B accumulate
// over both halves (two threads per row, 48 columns each, added at the
// end), and the column sums G^T . xa of the half (four threads per column,
// 64 rows each, added in a fixed order) are written.  Ranks are taken four
// at a time (one pass for rank <= 4), which keeps the kernel within its
// registers.
__device__ __forceinline__ void ce_grad_epilogue(const GemmArgs& p, f32x16 (&acc)[TM][TN], uint8_t* smem,
                                                 int64_t r0, int n0, int mt, int nt) {
  constexpr int R = 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int r = p.r;
  const int64_t V = p.V, c0 = p.w_row0;
  const float nv = *p.nvalid;
  const float coef = nv > 0.f ? p.coef / nv : 0.f;
  const int32_t* LBL = reinterpret_cast<const int32_t*>(smem + ROW_OFF);
  const float* LSE = reinterpret_cast<const float*>(smem + ROW_OFF + BM * 4);
  // z -> G in the accumulators (rows past M, ignored labels and columns past
  // w_rows give 0); the rows' label column and lse come from LDS
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lr = wm * WTM + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      const int32_t rel = LBL[lr];
      const float lse = LSE[lr];
      const bool valid = rel != NO_LABEL;  // also false for rows past M
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int lc = wn * WTN + b * 32 + (lane & 31);
        float gv = 0.f;
        if (valid && n0 + lc < p.w_rows) gv = coef * (__expf(acc[a][b][v] - lse) - (lc == rel ? 1.f : 0.f));
        acc[a][b][v] = gv;
      }
    }

  float* Z = reinterpret_cast<float*>(smem);
  float* Sx = reinterpret_cast<float*>(smem + CEB_Z);
  float* Sb = reinterpret_cast<float*>(smem + CEB_Z + CEB_X);
  const int row = tid >> 1, hh = tid & 1;        // row sums: 48 columns per thread
  const int ccol = tid % WTN, cseg = tid / WTN;  // column sums: 64 rows per thread (tid < 384)
  const bool vec = ((uintptr_t)p.o0 % 16 == 0) && (p.ldo % 8 == 0);
  for (int jb = 0; jb < r; jb += R) {
    __syncthreads();  // operand stages (first pass) or the previous pass's LDS reads are done
    for (int i = tid; i < BM * R; i += NTHR) {
      const int rr = i / R, j = jb + i % R;
      Sx[i] = (j < r && r0 + rr < p.M) ? p.rv0[(r0 + rr) * r + j] : 0.f;
    }
    float racc[R];
#pragma unroll
    for (int j = 0; j < R; ++j) racc[j] = 0.f;
    for (int h = 0; h < 2; ++h) {
      const int hc0 = n0 + h * WTN;  // first column of this half
      if (h) __syncthreads();        // the previous half's column partials are summed
      if (wn == h) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              Z[(wm * WTM + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * HP + b * 32 + (lane & 31)] =
                  acc[a][b][v];
      }
      for (int i = tid; i < WTN * R; i += NTHR) {
        const int c = i / R, j = jb + i % R;
        Sb[i] = (j < r && hc0 + c < p.w_rows) ? p.lB0[(c0 + hc0 + c) * r + j] : 0.f;
      }
      __syncthreads();
      if (jb == 0) {
        // G rows as bf16: 12 pieces of 8 columns per row
        for (int i = tid; i < BM * (WTN / 8); i += NTHR) {
          const int rr = i / (WTN / 8), cc = (i % (WTN / 8)) * 8;
          const int64_t pr = r0 + rr;
          const int n = hc0 + cc;
          if (pr >= p.M || n >= p.ldo) continue;
          const float* z = Z + rr * HP + cc;
          if (vec) {
            *reinterpret_cast<uint4*>(p.o0 + pr * p.ldo + n) = make_uint4(
                pack_bf2(z[0], z[1]), pack_bf2(z[2], z[3]), pack_bf2(z[4], z[5]), pack_bf2(z[6], z[7]));
          } else {
            for (int c = 0; c < 8 && n + c < p.ldo; ++c) p.o0[pr * p.ldo + n + c] = f2bf(z[c]);
          }
        }
      }
#pragma unroll 4
      for (int c = hh * (WTN / 2); c < (hh + 1) * (WTN / 2); ++c) {
        const float z = Z[row * HP + c];
#pragma unroll
        for (int j = 0; j < R; ++j) racc[j] += z * Sb[c * R + j];
      }
      float cacc[R];
#pragma unroll
      for (int j = 0; j < R; ++j) cacc[j] = 0.f;
      if (cseg < 4) {
#pragma unroll 4
        for (int rr = cseg * 64; rr < cseg * 64 + 64; ++rr) {
          const float z = Z[rr * HP + ccol];
#pragma unroll
          for (int j = 0; j < R; ++j) cacc[j] += z * Sx[rr * R + j];
        }
      }
      __syncthreads();
      float* Xs = Z;  // [3][WTN][R + 1] partials of segments 1..3
      if (cseg >= 1 && cseg < 4) {
#pragma unroll
        for (int j = 0; j < R; ++j) Xs[((cseg - 1) * WTN + ccol) * (R + 1) + j] = cacc[j];
      }
      __syncthreads();
      if (cseg == 0) {
#pragma unroll
        for (int sg = 0; sg < 3; ++sg)
#pragma unroll
          for (int j = 0; j < R; ++j) cacc[j] += Xs[(sg * WTN + ccol) * (R + 1) + j];
        const int n = hc0 + ccol;
        if (n < p.w_rows) {
          float* dst = p.f2 + ((int64_t)mt * V + c0 + n) * r + jb;
#pragma unroll
          for (int j = 0; j < R; ++j)
            if (jb + j < r) dst[j] = cacc[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) racc[j] += __shfl_xor(racc[j], 1);
    if (hh == 0 && r0 + row < p.M) {
      float* dst = p.f1 + ((int64_t)(p.ntile_base + nt) * p.M + r0 + row) * r + jb;
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (jb + j < r) dst[j] = racc[j];
    }
  }
}

// Dense forward: z[p][n] = sum_k a0[p][k] deq(W)[n][k] + s * rv0[p] . lB0[n].
// Geometry from GemmArgs: M rows, N = w_rows output columns, K.
//   EPI_LIN:    z stored as bf16 (o0, ldo).
//   EPI_CE_FWD: z never leaves the chip: per row and tile the online
//               (max, sum exp) over the tile's columns below w_rows goes to
//               f0[(tile column index) * M + row], and the row's label logit,
//               when the label column is in this tile, to f1[row].
//   EPI_CE_BWD: the columns are vocabulary rows w_row0 .. w_row0 + w_rows;
//               G = coef/nvalid * (exp(z - lse[row]) - [col == label]) (zero
//               for ignored labels and columns past w_rows) goes to o0 as
//               bf16 (ldo, columns below ldo), the tile's G . B rows to
//               f1[((ntile_base + tile column) * M + row) * r + j] and its
//               G^T . xa columns to f2[(tile row * V + w_row0 + col) * r + j].
template <int QT, int EPI>
__global__ __launch_bounds__(NTHR, 1) void wide_kernel(const GemmArgs p) {
  static_assert(EPI == EPI_LIN || EPI == EPI_CE_FWD || EPI == EPI_CE_BWD, "wide epilogues");
  constexpr int BS = QTraits<QT>::BS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_ALL];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * A_ST;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;

  // XCD-contiguous runs of tiles (ids go round-robin over the 8 XCDs), each
  // run laid out as GM m-tiles by a band of n-tiles
  const int count = gridDim.x;
  const int q8 = count >> 3, rem = count & 7, xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int bid = (xcd < rem ? xcd * (q8 + 1) : rem * (q8 + 1) + (xcd - rem) * q8) + loc;
  constexpr int GM = 4;
  const int g = bid / (GM * p.ntiles), m_first = g * GM, gm = min(p.mtiles - m_first, GM);
  const int idx = bid - g * GM * p.ntiles;
  const int mt = m_first + idx % gm, nt = idx / gm;
  const int64_t r0 = (int64_t)mt * BM;
  const int n0 = nt * BN;
  if (r0 >= p.M || n0 >= p.w_rows) return;
  const int nk = p.K / BK;

  // activation rows of this thread's four 16-byte chunks (c = tid + 512 i:
  // row c >> 3, chunk c & 7), clamped to the last row
  const uint16_t* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = min(r0 + (tid >> 3) + 64 * i, p.M - 1);
    ap[i] = p.a0 + row * p.lda + (tid & 7) * 8;
  }
  // weight quarter items it = tid + 512 i: row it >> 3, block (it >> 2) & 1,
  // quarter it & 3 (eight consecutive lanes cover a row's two blocks)
  int w_row[3], w_blk[3], w_q[3];
  const uint8_t* wp[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int it = tid + NTHR * i;
    w_row[i] = it >> 3;
    w_blk[i] = (it >> 2) & 1;
    w_q[i] = it & 3;
    const int nrow = min(n0 + w_row[i], p.w_rows - 1);
    wp[i] = p.w0 + (int64_t)(p.w_row0 + nrow) * p.w_rowbytes + w_blk[i] * BS;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  uint4 a00, a01, a02, a03, a10, a11, a12, a13;
  RawQuarter<QT> W0[3], W1[3];
#define GQW_LOAD_A(KT, X0, X1, X2, X3)                           \
  {                                                              \
    const int k_ = min((KT), nk - 1) * BK;                       \
    X0 = *reinterpret_cast<const uint4*>(ap[0] + k_);            \
    X1 = *reinterpret_cast<const uint4*>(ap[1] + k_);            \
    X2 = *reinterpret_cast<const uint4*>(ap[2] + k_);            \
    X3 = *reinterpret_cast<const uint4*>(ap[3] + k_);            \
  }
#define GQW_STORE_A(ST, X0, X1, X2, X3)                                            \
  {                                                                                \
    uint16_t* d_ = As + (ST) * A_ST + (tid >> 3) * LDK + (tid & 7) * 8;            \
    *reinterpret_cast<uint4*>(d_) = X0;                                            \
    *reinterpret_cast<uint4*>(d_ + 64 * LDK) = X1;                                 \
    *reinterpret_cast<uint4*>(d_ + 128 * LDK) = X2;                                \
    *reinterpret_cast<uint4*>(d_ + 192 * LDK) = X3;                                \
  }
  auto load_w = [&](int kt, RawQuarter<QT> (&Wr)[3]) {
    const int64_t koff = (int64_t)min(kt, nk - 1) * 2 * BS;
#pragma unroll
    for (int i = 0; i < 3; ++i) load_quarter<QT>(wp[i] + koff, w_q[i], Wr[i]);
  };
  auto store_w = [&](int st, const RawQuarter<QT> (&Wr)[3]) {
#pragma unroll
    for (int i = 0; i < 3; ++i) store_quarter<QT>(Bs + st * B_ST + w_row[i] * LDK + w_blk[i] * 32, w_q[i], Wr[i]);
  };
  auto compute = [&](int st) {
    const uint16_t* A = As + st * A_ST;
    const uint16_t* B = Bs + st * B_ST + wn * WTN * LDK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(A + (wm * WTM + a * 32 + (lane & 31)) * LDK + kk * 16 +
                                                 (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8*>(B + (b * 32 + (lane & 31)) * LDK + kk * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  };

  // prologue: slices 0 and 1 in registers, slice 0 into stage 0; the fold
  // operands and the per-row label / lse go to their LDS area meanwhile (so
  // their latency hides behind the pipeline instead of after it)
  const int r = p.r;
  const float s = p.s;
  auto split8 = [](const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)v[i];
      hi[i] = h;
      lo[i] = (__bf16)(v[i] - (float)h);
    }
  };
  uint16_t* XH = reinterpret_cast<uint16_t*>(smem + FOLD_OFF);  // [BM][FR]
  uint16_t* XL = XH + BM * FR;
  uint16_t* YH = XL + BM * FR;                                   // [BN][FR]
  uint16_t* YL = YH + BN * FR;
  int32_t* LBL = reinterpret_cast<int32_t*>(smem + ROW_OFF);     // [BM]
  float* LSE = reinterpret_cast<float*>(smem + ROW_OFF + BM * 4);  // [BM]
  {
    // thread t: xa row t >> 1 and (t < 2 BN) s*B row t >> 1, ranks 8 (t & 1) .. +8
    const int j0 = (tid & 1) * 8;
    const int64_t pr = r0 + (tid >> 1);
    float xv[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = 0.f;
      if (pr < p.M && j0 + i < r) {
        x = p.rv0[pr * r + j0 + i];
        // xa as rv_parts column-range partials: summed here; the tiles of
        // column 0 store the sum
        for (int sp = 1; sp < p.rv_parts; ++sp) x += p.rv0[sp * p.M * r + pr * r + j0 + i];
        if (p.rv_out && nt == 0) p.rv_out[pr * r + j0 + i] = x;
      }
      xv[i] = x;
    }
    const int col = n0 + (tid >> 1);
    const bool bt = tid < 2 * BN;
    const float* Bw = p.lB0 + (int64_t)(p.w_row0 + col) * r;
#pragma unroll
    for (int i = 0; i < 8; ++i) bv[i] = (bt && col < p.w_rows && j0 + i < r) ? s * Bw[j0 + i] : 0.f;
    int32_t rel = NO_LABEL;
    float ls = 0.f;
    if constexpr (EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) {
      if (tid < BM && r0 + tid < p.M) {
        const int64_t lab = p.labels[r0 + tid];
        if (lab != p.ignore_index && lab >= 0 && lab < p.V) {
          const int64_t rc = lab - p.w_row0 - n0;
          rel = rc < 0 ? -1 : (rc >= BN ? BN : (int32_t)rc);
        }
        if constexpr (EPI == EPI_CE_BWD) ls = p.lse[r0 + tid];
      }
    }
    GQW_LOAD_A(0, a00, a01, a02, a03)
    load_w(0, W0);
    GQW_LOAD_A(1, a10, a11, a12, a13)
    load_w(1, W1);
    bf16x8 h8, l8;
    split8(xv, h8, l8);
    *reinterpret_cast<bf16x8*>(XH + (tid >> 1) * FR + j0) = h8;
    *reinterpret_cast<bf16x8*>(XL + (tid >> 1) * FR + j0) = l8;
    if (bt) {
      split8(bv, h8, l8);
      *reinterpret_cast<bf16x8*>(YH + (tid >> 1) * FR + j0) = h8;
      *reinterpret_cast<bf16x8*>(YL + (tid >> 1) * FR + j0) = l8;
    }
    if constexpr (EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) {
      if (tid < BM) {
        LBL[tid] = rel;
        LSE[tid] = ls;
      }
    }
  }
  GQW_STORE_A(0, a00, a01, a02, a03)
  store_w(0, W0);
  __syncthreads();
  // step kt (stage S = kt & 1): slice kt+2 is loaded into the register set
  // slice kt was stored from, slice kt+1 (loaded a step earlier) goes into
  // the other stage while the MFMAs of slice kt run
#define GQW_STEP(KT, S, C0, C1, C2, C3, N0, N1, N2, N3, WC, WN) \
  GQW_LOAD_A((KT) + 2, C0, C1, C2, C3)                          \
  load_w((KT) + 2, WC);                                         \
  __builtin_amdgcn_sched_barrier(0);                            \
  compute(S);                                                   \
  GQW_STORE_A(1 - (S), N0, N1, N2, N3)                          \
  store_w(1 - (S), WN);                                         \
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    GQW_STEP(kt, 0, a00, a01, a02, a03, a10, a11, a12, a13, W0, W1)
    GQW_STEP(kt + 1, 1, a10, a11, a12, a13, a00, a01, a02, a03, W1, W0)
  }
  if (kt < nk) {
    GQW_STEP(kt, 0, a00, a01, a02, a03, a10, a11, a12, a13, W0, W1)
  }
#undef GQW_STEP
#undef GQW_LOAD_A
#undef GQW_STORE_A

  // ---- rank-r adapter term on the MFMA: acc[row][col] += sum_j xa[row][j] *
  // s * B[col][j], one k16 slice (rank <= 16) from the LDS copies, bf16 hi +
  // lo parts (three products: hi*hi + hi*lo + lo*hi)
  {
    const int jo = (lane >> 5) * 8;
    bf16x8 ah[TM], al[TM];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int row = wm * WTM + a * 32 + (lane & 31);
      ah[a] = *reinterpret_cast<const bf16x8*>(XH + row * FR + jo);
      al[a] = *reinterpret_cast<const bf16x8*>(XL + row * FR + jo);
    }
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int col = wn * WTN + b * 32 + (lane & 31);
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(YH + col * FR + jo);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(YL + col * FR + jo);
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bh, acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bl, acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[a], bh, acc[a][b], 0, 0, 0);
      }
    }
  }

  if constexpr (EPI == EPI_CE_FWD) {
    // Branch-free per (row, lane pair): the pair's six columns give the max
    // (one xor-1 exchange) and the sum of exp against it (three exps per
    // lane, one exchange); the 16
    // pairs of each wave's half row go through LDS ([256 rows][2 wave
    // columns][16] pairs, 64 KB), and two threads per row combine them (max
    // first, then the rescaled sum) and then the two halves.  A lane holding
    // the row's label column writes that logit to an LDS slot of the row,
    // every other lane to a slot of its own, so the loop has no branches.
    __syncthreads();  // every wave is done reading the operand stages
    float2* P = reinterpret_cast<float2*>(smem);
    float* ZL = reinterpret_cast<float*>(smem + BM * 2 * 16 * 8);  // [BM] label logits + [64] dump slots
    const int lcol0 = wn * WTN + (lane & 31);  // this lane's first column in the tile
    bool cok[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b) cok[b] = n0 + lcol0 + b * 32 < p.w_rows;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = wm * WTM + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        float z[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) z[b] = cok[b] ? acc[a][b][v] : -INFINITY;
        float m = z[0];
#pragma unroll
        for (int b = 1; b < TN; ++b) m = fmaxf(m, z[b]);
        m = fmaxf(m, __shfl_xor(m, 1));  // the pair's max: the two sums share it
        const float ms = m == -INFINITY ? 0.f : m;
        float l = 0.f;
#pragma unroll
        for (int b = 0; b < TN; ++b) l += __expf(z[b] - ms);
        const int lc = LBL[lr] - lcol0;
        const bool hit = lc >= 0 && lc < 32 * TN && (lc & 31) == 0;
        ZL[hit ? lr : BM + lane] = lc == 0 ? acc[a][0][v] : (lc == 32 ? acc[a][1][v] : acc[a][2][v]);
        l += __shfl_xor(l, 1);
        P[(lr * 2 + wn) * 16 + ((lane & 31) >> 1)] = make_float2(m, l);  // both lanes: same pair
      }
    __syncthreads();
    const int row = tid >> 1, h = tid & 1;
    float2 q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = P[(row * 2 + h) * 16 + i];
    float m = q[0].x;
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, q[i].x);
    const float ms = m == -INFINITY ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) l += q[i].y * __expf(q[i].x - ms);  // q.y = 0 where q.x = -inf
    const float m2 = __shfl_xor(m, 1), l2 = __shfl_xor(l, 1);
    if (h == 0 && r0 + row < p.M) {
      ml_merge1(m, l, m2, l2);  // wave column 0, then 1
      float* dst = p.f0 + ((int64_t)(p.ntile_base + nt) * p.M + r0 + row) * 2;
      dst[0] = m;
      dst[1] = l;
    }
    if (tid < BM && LBL[tid] >= 0 && LBL[tid] < BN && r0 + tid < p.M) p.f1[r0 + tid] = ZL[tid];
    return;
  }

  if constexpr (EPI == EPI_CE_BWD) {
    ce_grad_epilogue(p, acc, smem, r0, n0, mt, nt);
    return;
  }

  // ---- epilogue: the wave's 64 x 96 tile through its own LDS region (rows
  // of 104 bf16), stored as 16-byte row pieces (12 lanes per row) when the
  // output rows allow it, else one 2-byte store per value
  __syncthreads();  // every wave is done reading the operand stages
  uint16_t* Ws = reinterpret_cast<uint16_t*>(smem) + wave * WTM * SP;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        Ws[(a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * SP + b * 32 + (lane & 31)] = f2bf(acc[a][b][v]);
  const int64_t rbase = r0 + wm * WTM;
  const int cbase = n0 + wn * WTN;
  const bool vec = ((uintptr_t)p.o0 % 16 == 0) && (p.ldo % 8 == 0) && (p.N % 8 == 0);
  constexpr int CH = WTN / 8;
  for (int i = lane; i < WTM * CH; i += 64) {
    const int rr = i / CH, cc = (i % CH) * 8;
    const int64_t pr = rbase + rr;
    const int n = cbase + cc;
    if (pr >= p.M || n >= p.N) continue;
    const uint16_t* src = Ws + rr * SP + cc;
    if (vec) {
      *reinterpret_cast<uint4*>(p.o0 + pr * p.ldo + n) = *reinterpret_cast<const uint4*>(src);
    } else {
      for (int c = 0; c < 8 && n + c < p.N; ++c) p.o0[pr * p.ldo + n + c] = src[c];
    }
  }
}

}  // namespace wide

namespace {
// Launch of the wide-tile forward (EPI_LIN or EPI_CE_FWD, dense, Q8_0 /
// Q4_0, K % 64 == 0); declared beside launch_q in gq_gemm_impl.h.
template <int QT, int EPI>
hipError_t launch_wide(const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles);
  mmq_launch((wide::wide_kernel<QT, EPI>), grid, dim3(wide::NTHR), st, a);
  return hipGetLastError();
}
}  // namespace

}  // namespace gq
