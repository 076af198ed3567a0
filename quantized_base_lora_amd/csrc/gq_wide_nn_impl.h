// Wide-tile MMQ in the backward (NN) direction for the LM head's dh =
// G deq(W): the reduction runs along the weight (vocabulary) rows and the
// output columns along the blocks of a row.  256 x 128 output tiles on 512
// threads, the reduction of every tile cut into `ksplit` (1 or 2) contiguous
// ranges, one workgroup each, each range summing into its own fp32 array.
//
// The 128 x 128 tile of gq_gemm_impl.h gives a 2048 x 2048 output one round
// of workgroups by running two groups of four waves on alternate k-steps of
// the same tile, so each decoded weight slice feeds 128 rows.  Here the same
// number of workgroups comes from two reduction ranges of a 256-row tile:
// every decoded slice feeds 256 rows (half the decode VALU per MFMA) at the
// same LDS operand reads per MFMA (each wave owns a 64 x 64 share of the
// tile).  The dh sums are read and written once per launch anyway, so the
// two ranges cost a second array, not an extra pass.  (For dX the range
// sums would need a fixup pass over 2 x T x n_in floats, which costs more
// than the tile saves.)
//
//  * Activations: 256 rows x 64 bf16 per k-step, four coalesced 16-byte
//    loads per thread, stored into a padded LDS tile one step later.
//  * Weights: the 64 reduction rows x 4 blocks of a k-step as quarter-block
//    items (two per thread), decoded to bf16 into the row-major [k][n] tile
//    (16-byte chunks XOR-swizzled by row), read back as the B operand with
//    transposing LDS reads (ds_read_b64_tr_b16).
//  * Double-buffered LDS, one barrier per k-step, loads two steps ahead.
//  * Rows past M and blocks past the row are clamped to the last valid one
//    (never stored).  With K % 64 != 0 (the RAGGED instance) reduction rows
//    past K decode to zero (scale 0) and the activation columns past K are
//    zeroed (the activation rows must hold K rounded up to 64 columns); the
//    other instance has no masks in its loop.
//  * Range s accumulates its fp32 sums into f0 + s * M * ldf (or sets them
//    when accum == 0), no adapter term; the consumer adds the ranges in
//    order.  Ranges are never added between workgroups, so the result does
//    not depend on their timing.
#pragma once
#include "gq_dev.h"
#include "gq_internal.h"
#include "gq_wide_impl.h"

namespace gq {
namespace wnn {

constexpr int BM = WIDE_NN_BM, BN = WIDE_NN_BN, BK = 64, LDK = BK + 8, NTHR = 512;
constexpr int TM = 2, TN = 2;      // 32x32 sub-tiles per wave (64 x 64)
constexpr int WTM = 64, WTN = 64;  // wave tile
constexpr int PN = BN;             // [k][n] weight tile pitch: 16 chunks of 8, swizzled
constexpr int A_ST = BM * LDK, B_ST = BK * PN;
constexpr int SMEM = (2 * A_ST + 2 * B_ST) * 2;
constexpr int ZP = 40;  // epilogue staging pitch (fp32)
static_assert(BN == 128 && PN / 8 == 16, "one 16-chunk swizzle group per weight row");
static_assert(8 * WTM * ZP * 4 <= SMEM, "epilogue staging fits the operand stages");
static_assert(SMEM <= 160 * 1024, "fits the CU's LDS");

using wide::RawQuarter;
using wide::QuarterBytes;
using wide::load_quarter;

// Element offset of column `col` of reduction row `row` in the [k][n] tile:
// the 16-byte chunk index is XORed with 5 * (row % 4), which spreads the
// transposing reads of four consecutive rows over the banks.
__device__ __forceinline__ int swz(int row, int col) {
  return ((((col >> 3) ^ (5 * (row & 3))) & 15) << 3) | (col & 7);
}

// Decode one quarter of the block whose first column is `col0` into
// reduction row `row` of the tile.  Same arithmetic as decode_block_fast:
// every product is exact, each bf16 value is d*q rounded once.
//  Q4_0 quarter qq: bytes 4qq..4qq+3 -> columns 4qq.. (low nibbles) and
//                   16+4qq.. (high nibbles)
//  Q8_0 quarter qq: bytes 8qq..8qq+7 -> columns 8qq..8qq+7
template <int QT>
__device__ __forceinline__ void store_quarter_nn(uint16_t* tile, int row, int col0, int qq, const RawQuarter<QT>& r) {
  const float d = h2f(r.hdr & 0xffffu);
  uint16_t* rp = tile + row * PN;
  if constexpr (QT == QT_Q4_0) {
    const float off = -8.f * d;
    const uint32_t lo = r.q[0] & 0x0f0f0f0fu, hi = (r.q[0] >> 4) & 0x0f0f0f0fu;
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __builtin_fmaf(ubyte(lo, i), d, off);
      b[i] = __builtin_fmaf(ubyte(hi, i), d, off);
    }
    *reinterpret_cast<uint2*>(rp + swz(row, col0 + 4 * qq)) = make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
    *reinterpret_cast<uint2*>(rp + swz(row, col0 + 16 + 4 * qq)) = make_uint2(pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3]));
  } else {
    const float off = -128.f * d;
    float v[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t u = r.q[h] ^ 0x80808080u;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * h + i] = __builtin_fmaf(ubyte(u, i), d, off);
    }
    *reinterpret_cast<uint4*>(rp + swz(row, col0 + 8 * qq)) =
        make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
  }
}

// Geometry from GemmArgs (dense only): M rows, N output columns (N <= 32 *
// w_nb), K reduction rows; activations a0 (lda >= K rounded up to 64),
// weights w0 from reduction row w_row0, w_rowbytes per row.  Grid: mtiles *
// ntiles * ksplit workgroups.
template <int QT, int EPI, bool RAGGED>
__global__ __launch_bounds__(NTHR, 1) void wide_nn_kernel(const GemmArgs p) {
  static_assert(EPI == EPI_DH_ACC, "fp32 range sums");
  constexpr int BS = QTraits<QT>::BS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * A_ST;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;

  // XCD-contiguous runs of workgroups (ids go round-robin over the 8 XCDs);
  // within a run the ranges of a tile are adjacent and the tiles n-fastest,
  // so an XCD works on few activation row blocks
  const int count = gridDim.x;
  const int q8 = count >> 3, rem = count & 7, xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int bid = (xcd < rem ? xcd * (q8 + 1) : rem * (q8 + 1) + (xcd - rem) * q8) + loc;
  const int KS = p.ksplit > 1 ? p.ksplit : 1;
  const int ks = bid % KS, tile = bid / KS;
  const int mt = tile / p.ntiles, nt = tile % p.ntiles;
  const int64_t r0 = (int64_t)mt * BM;
  const int n0 = nt * BN;
  if (r0 >= p.M || n0 >= p.N) return;
  const int nkall = (p.K + BK - 1) / BK;
  const int kb0 = (int)((int64_t)ks * nkall / KS);
  const int nk = (int)((int64_t)(ks + 1) * nkall / KS) - kb0;

  // activation rows of this thread's four 16-byte chunks (c = tid + 512 i:
  // row c >> 3, chunk c & 7), clamped to the last row
  const uint16_t* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = min(r0 + (tid >> 3) + 64 * i, p.M - 1);
    ap[i] = p.a0 + row * p.lda + (int64_t)kb0 * BK + (tid & 7) * 8;
  }
  // weight quarter items it = tid + 512 i: reduction row it / 16 of the
  // k-step, block (it % 16) / 4 of the tile's four, quarter it % 4
  int w_row[2], w_blk[2], w_q[2];
  const uint8_t* wp[2];
  const uint8_t* wlast[2];  // RAGGED: the same block in reduction row K - 1
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int it = tid + NTHR * i;
    w_row[i] = it / 16;
    w_blk[i] = (it % 16) >> 2;
    w_q[i] = it & 3;
    const int nb = min((n0 >> 5) + w_blk[i], p.w_nb - 1);
    wp[i] = p.w0 + ((int64_t)p.w_row0 + (int64_t)kb0 * BK + w_row[i]) * p.w_rowbytes + (int64_t)nb * BS;
    wlast[i] = p.w0 + ((int64_t)p.w_row0 + p.K - 1) * p.w_rowbytes + (int64_t)nb * BS;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  if (nk > 0) {
    uint4 a00, a01, a02, a03, a10, a11, a12, a13;
    RawQuarter<QT> W0[2], W1[2];
    // k-step kt of the range (clamped to its last); in the reduction's last
    // k-step of a ragged K the columns past K read as zero
    auto load_a = [&](int kt, uint4& x0, uint4& x1, uint4& x2, uint4& x3) __attribute__((always_inline)) {
      const int kk = min(kt, nk - 1);
      const int k_ = kk * BK;
      x0 = *reinterpret_cast<const uint4*>(ap[0] + k_);
      x1 = *reinterpret_cast<const uint4*>(ap[1] + k_);
      x2 = *reinterpret_cast<const uint4*>(ap[2] + k_);
      x3 = *reinterpret_cast<const uint4*>(ap[3] + k_);
      if (RAGGED && kb0 + kk == nkall - 1) {
        const int valid = p.K - (kb0 + kk) * BK - (tid & 7) * 8;  // columns of the chunk below K
        auto cut = [&](uint4& x) {
          uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep = (2 * e + 1 < valid ? 0xffff0000u : 0u) | (2 * e < valid ? 0xffffu : 0u);
            w[e] &= keep;
          }
          x = make_uint4(w[0], w[1], w[2], w[3]);
        };
        cut(x0);
        cut(x1);
        cut(x2);
        cut(x3);
      }
    };
    auto store_a = [&](int st, const uint4& x0, const uint4& x1, const uint4& x2, const uint4& x3)
        __attribute__((always_inline)) {
      uint16_t* d_ = As + st * A_ST + (tid >> 3) * LDK + (tid & 7) * 8;
      *reinterpret_cast<uint4*>(d_) = x0;
      *reinterpret_cast<uint4*>(d_ + 64 * LDK) = x1;
      *reinterpret_cast<uint4*>(d_ + 128 * LDK) = x2;
      *reinterpret_cast<uint4*>(d_ + 192 * LDK) = x3;
    };
    auto load_w = [&](int kt, RawQuarter<QT> (&Wr)[2]) __attribute__((always_inline)) {
      const int kk = min(kt, nk - 1);
      const int64_t koff = (int64_t)kk * BK * p.w_rowbytes;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (RAGGED) {
          const bool ok = (kb0 + kk) * BK + w_row[i] < p.K;
          load_quarter<QT>(ok ? wp[i] + koff : wlast[i], w_q[i], Wr[i]);
          if (!ok) Wr[i].hdr = 0u;  // scale 0: the row decodes to zeros
        } else {
          load_quarter<QT>(wp[i] + koff, w_q[i], Wr[i]);
        }
      }
    };
    auto store_w = [&](int st, const RawQuarter<QT> (&Wr)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) store_quarter_nn<QT>(Bs + st * B_ST, w_row[i], w_blk[i] * 32, w_q[i], Wr[i]);
    };
    // transposing reads: lane l reads 4 columns of rows tr_row and tr_row + 4
    // of each k16 slice (rows with equal row % 4, so one swizzle)
    const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int tr_off[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b) tr_off[b] = tr_row * PN + swz(tr_row, wn * WTN + b * 32 + tr_col);
    auto compute = [&](int st) __attribute__((always_inline)) {
      const uint16_t* A = As + st * A_ST;
      const uint16_t* B = Bs + st * B_ST;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[TM], bfr[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          af[a] = *reinterpret_cast<const bf16x8*>(A + (wm * WTM + a * 32 + (lane & 31)) * LDK + kk * 16 +
                                                   (lane >> 5) * 8);
#pragma unroll
        for (int b = 0; b < TN; ++b) {
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
        }
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
      }
    };

    // prologue: steps 0 and 1 in registers, step 0 into stage 0
    load_a(0, a00, a01, a02, a03);
    load_w(0, W0);
    load_a(1, a10, a11, a12, a13);
    load_w(1, W1);
    store_a(0, a00, a01, a02, a03);
    store_w(0, W0);
    __syncthreads();
    // step kt (stage S = kt & 1): step kt+2 is loaded into the register set
    // step kt was stored from, step kt+1 (loaded a step earlier) goes into
    // the other stage while the MFMAs of step kt run
#define GQN_STEP(KT, S, C0, C1, C2, C3, N0, N1, N2, N3, WC, WN) \
  load_a((KT) + 2, C0, C1, C2, C3);                             \
  load_w((KT) + 2, WC);                                         \
  __builtin_amdgcn_sched_barrier(0);                            \
  compute(S);                                                   \
  store_a(1 - (S), N0, N1, N2, N3);                             \
  store_w(1 - (S), WN);                                         \
  __syncthreads();
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      GQN_STEP(kt, 0, a00, a01, a02, a03, a10, a11, a12, a13, W0, W1)
      GQN_STEP(kt + 1, 1, a10, a11, a12, a13, a00, a01, a02, a03, W1, W0)
    }
    if (kt < nk) {
      GQN_STEP(kt, 0, a00, a01, a02, a03, a10, a11, a12, a13, W0, W1)
    }
#undef GQN_STEP
  }

  // ---- fp32 sums of this range.  acc[a][b][v] sits at tile row
  // wm*64 + a*32 + (v>>2)*8 + (lane>>5)*4 + (v&3), column wn*64 + b*32 + (lane&31)
  float* dst = p.f0 + (int64_t)ks * p.M * p.ldf;
  const int64_t ld = p.ldf;
  const bool add = p.accum != 0;
  // The wave's 64 x 64 share goes out through its own LDS region, one
  // 32-column half at a time ([64][ZP] fp32; ZP = 40 puts rows four apart
  // 32 banks apart), as 16-byte row pieces (8 lanes per 128-byte row piece);
  // the accumulating form reads the old sums the same way.
  __syncthreads();  // every wave is done reading the operand stages
  float* Z = reinterpret_cast<float*>(smem) + wave * WTM * ZP;
  const int64_t rbase = r0 + wm * WTM;
#pragma unroll
  for (int b = 0; b < TN; ++b) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        Z[(a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * ZP + (lane & 31)] = acc[a][b][v];
    // (the wave's own region: its LDS writes complete before these reads)
    const int cb = n0 + wn * WTN + b * 32;
#pragma unroll
    for (int i = lane; i < WTM * 8; i += 64) {
      const int rr = i >> 3, c4 = (i & 7) * 4;
      const int64_t pr = rbase + rr;
      const int n = cb + c4;
      if (pr >= p.M || n >= p.N) continue;
      float4 val = *reinterpret_cast<const float4*>(Z + rr * ZP + c4);
      float4* d = reinterpret_cast<float4*>(dst + pr * ld + n);
      if (add) {
        const float4 o = *d;
        val.x = o.x + val.x;
        val.y = o.y + val.y;
        val.z = o.z + val.z;
        val.w = o.w + val.w;
      }
      *d = val;
    }
  }
}

}  // namespace wnn

namespace {
// Launch of the wide NN tile (EPI_DH_ACC, dense, Q8_0 / Q4_0); declared
// beside launch_q in gq_gemm_impl.h.
template <int QT, int EPI>
hipError_t launch_wide_nn(const GemmArgs& a, hipStream_t st) {
  const unsigned ks = a.ksplit > 1 ? (unsigned)a.ksplit : 1u;
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles * ks);
  if (a.K % wnn::BK)
    mmq_launch((wnn::wide_nn_kernel<QT, EPI, true>), grid, dim3(wnn::NTHR), st, a);
  else
    mmq_launch((wnn::wide_nn_kernel<QT, EPI, false>), grid, dim3(wnn::NTHR), st, a);
  return hipGetLastError();
}
}  // namespace

}  // namespace gq
