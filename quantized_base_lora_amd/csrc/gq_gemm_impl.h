// One MFMA GEMM template for every quantised contraction on the path.
//
// The pages' fused dequantize-and-multiply ("MMQ and grouped MMQ like
// llama.cpp", page 2 "Show HN: LoRA over GGUF", section "Things involved in
// the training"; the ai-manual.ru article describes the fused kernel as
// decoding the compressed weights in registers and multiplying at once, with
// no fp16 copy of W) is built here for CDNA4:
//
//  * 256 threads = 4 wave64s in a 2x2 grid; block tile BM x 128, k-step 64.
//  * Activations (bf16) are staged global -> registers -> LDS; weight blocks
//    are loaded raw (dword loads + byte realignment), decoded to bf16 in
//    registers and written to LDS -- the only full-precision copy of W is the
//    64-deep LDS slice of the current tile.
//  * NT (forward): the reduction runs along the weight's block dimension, the
//    decoded tile is stored [n][k].  NN (backward, dX = dY deq(W)): the
//    reduction runs along the weight's rows; the decode writes the tile
//    transposed, so both modes feed v_mfma_f32_32x32x16_bf16 from identical
//    [col][k] LDS layouts (fp32 accumulation).
//  * Double-buffered LDS, one barrier per k-step; the next tile's global
//    loads are in flight while the MFMAs of the current one run.
//  * Grouped (MoE) launches map m-tile slots to experts through a device
//    prefix of per-expert tile counts: no host sync, idle experts' blocks are
//    never read.
//  * Workgroups are renumbered so that each XCD (8 per MI355X, dispatched
//    round-robin) works on a contiguous run of tiles that share weight tiles
//    in its own L2.
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

template <int BM, int BN>
struct Geom {
  static constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_CHUNKS = BM * BK / 8 / NTHR;  // 16-byte chunks per thread
  static constexpr int SMEM_MAIN = 2 * (BM + BN) * LDK * 2;
  static constexpr int ZP = BN + 1;  // pitch (floats) of the staged epilogue tile
  static constexpr int SMEM_Z = BM * ZP * 4;
  static constexpr int SMEM = SMEM_MAIN > SMEM_Z ? SMEM_MAIN : SMEM_Z;
};

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Row reduction of the staged tile Z [BM][ZP]:
//   out[j] = sum_{c : n0 + c < ncols} Z[row][c] * (W ? W[(n0 + c) * r + j] : 1),  j < nv
// Thread (row = tid % BM, seg = tid / BM) sums one column segment; segments
// are combined in order through LDS.  sink(row, out) runs on segment 0.
// Caller has synchronised after writing Z; returns synchronised.
template <int BM, int BN, class Sink>
__device__ __forceinline__ void z_row_reduce(float* Z, const float* W, int r, int nv, int n0,
                                             int ncols, Sink sink) {
  constexpr int NSEG = NTHR / BM, SEGC = BN / NSEG, ZP = BN + 1;
  const int tid = threadIdx.x;
  const int row = tid % BM, seg = tid / BM;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  const int cend = min((seg + 1) * SEGC, ncols - n0);
  for (int c = seg * SEGC; c < cend; ++c) {
    const float z = Z[row * ZP + c];
    if (W) {
      const float* w = W + (int64_t)(n0 + c) * r;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < nv) acc[j] += z * w[j];
    } else {
      acc[0] += z;
    }
  }
  __syncthreads();
  float* X = Z;  // reuse: [NSEG][BM][17]
  if (seg > 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < nv) X[(seg * BM + row) * 17 + j] = acc[j];
  }
  __syncthreads();
  if (seg == 0) {
    for (int sg = 1; sg < NSEG; ++sg) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < nv) acc[j] += X[(sg * BM + row) * 17 + j];
    }
    sink(row, acc);
  }
  __syncthreads();
}

// Column reduction of Z: out[j] = sum_{row : r0 + row < r1} Z[row][col] * X[(r0+row)*r + j]
template <int BM, int BN, class Sink>
__device__ __forceinline__ void z_col_reduce(float* Z, const float* X, int r, int64_t r0,
                                             int64_t r1, Sink sink) {
  constexpr int NSEG = NTHR / BN, SEGR = BM / NSEG, ZP = BN + 1;
  const int tid = threadIdx.x;
  const int col = tid % BN, seg = tid / BN;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  const int rend = (int)min((int64_t)(seg + 1) * SEGR, r1 - r0);
  for (int rr = seg * SEGR; rr < rend; ++rr) {
    const float z = Z[rr * ZP + col];
    const float* x = X + (r0 + rr) * r;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) acc[j] += z * x[j];
  }
  __syncthreads();
  float* Xs = Z;
  if (seg > 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) Xs[(seg * BN + col) * 17 + j] = acc[j];
  }
  __syncthreads();
  if (seg == 0) {
    for (int sg = 1; sg < NSEG; ++sg) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < r) acc[j] += Xs[(sg * BN + col) * 17 + j];
    }
    sink(col, acc);
  }
  __syncthreads();
}

template <int QT, int EPI, int BM, int BN>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(const GemmArgs p) {
  using G = Geom<BM, BN>;
  constexpr bool NN = EPI >= EPI_LIN_BWD;
  constexpr int BS = QTraits<QT>::BS;
  constexpr int TM = G::TM, TN = G::TN, WTM = G::WTM, WTN = G::WTN, ZP = G::ZP;
  static_assert(BN == 128, "weight item mapping assumes 256 blocks per k-step");
  static_assert(EPI != EPI_SWIGLU || TN == 2, "SwiGLU pairs gate/up n-subtiles");

  __shared__ __attribute__((aligned(16))) uint8_t smem[G::SMEM];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * BM * LDK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- workgroup -> tile, XCD-contiguous runs of tiles
  int bid;
  {
    const int nblk = gridDim.x, q = nblk >> 3, rem = nblk & 7;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    bid = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + loc;
  }
  const int mslot = bid % p.mtiles;
  const int ntile = bid / p.mtiles;
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
  uint4 areg[G::A_CHUNKS];
  auto load_a = [&](int kt) {
    int k0 = kt * BK;
    const uint16_t* base = p.a0;
    if (k0 >= p.asplit) { base = p.a1; k0 -= p.asplit; }
#pragma unroll
    for (int i = 0; i < G::A_CHUNKS; ++i) {
      const int kc = kt * BK + ((tid + NTHR * i) & 7) * 8;
      if (aval[i] && kc < p.K)
        areg[i] = *reinterpret_cast<const uint4*>(base + aoff[i] + k0);
      else
        areg[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
    uint16_t* A = As + buf * BM * LDK;
#pragma unroll
    for (int i = 0; i < G::A_CHUNKS; ++i) {
      const int c = tid + NTHR * i;
      *reinterpret_cast<uint4*>(A + (c >> 3) * LDK + (c & 7) * 8) = areg[i];
    }
  };

  // ---- weight operand: one block per thread per k-step
  // NT: item (row = tid >> 1, kb = tid & 1): blocks 2kt + kb of weight row `wrow_n`
  // NN: item (kb = tid >> 6, row = tid & 63): block n0/32 + kb of reduction row kt*64 + row
  const int w_it_row = NN ? (tid & 63) : (tid >> 1);
  const int w_it_kb = NN ? (tid >> 6) : (tid & 1);
  const uint8_t* wptr = nullptr;  // NT: row base + kb*BS
  bool wrow_ok = false;
  if constexpr (!NN) {
    const uint8_t* src = p.w0;
    int nrow;
    if constexpr (EPI == EPI_SWIGLU) {
      const int proj = (w_it_row >> 5) & 1;
      nrow = (n0 >> 1) + (w_it_row >> 6) * 32 + (w_it_row & 31);
      src = proj ? p.w1 : p.w0;
    } else {
      nrow = n0 + w_it_row;
    }
    wrow_ok = nrow < p.w_rows;
    wptr = src + (int64_t)e * p.w_estride + (int64_t)(p.w_row0 + nrow) * p.w_rowbytes +
           w_it_kb * BS;
  } else {
    wrow_ok = ((n0 >> 5) + w_it_kb) < p.w_nb;
  }
  RawBlock<QT> wr;
  auto load_w = [&](int kt) {
    const uint8_t* blk = nullptr;
    if constexpr (!NN) {
      if (wrow_ok) blk = wptr + (int64_t)kt * 2 * BS;
    } else {
      const int rg = kt * BK + w_it_row;
      if (wrow_ok && rg < p.K) {
        const bool second = rg >= p.wsplit;
        const uint8_t* src = second ? p.w1 : p.w0;
        const int rr = second ? rg - p.wsplit : rg;
        blk = src + (int64_t)e * p.w_estride + (int64_t)(p.w_row0 + rr) * p.w_rowbytes +
              (int64_t)((n0 >> 5) + w_it_kb) * BS;
      }
    }
    if (blk) {
      load_block<QT>(blk, wr);
    } else {
      wr.hdr = 0;
#pragma unroll
      for (int i = 0; i < RawBlock<QT>::NQ; ++i) wr.q[i] = 0;
    }
  };
  auto store_w = [&](int buf) {
    float w[32];
    decode_block<QT>(wr, w);
    uint16_t* B = Bs + buf * BN * LDK;
    if constexpr (!NN) {
      uint4* dst = reinterpret_cast<uint4*>(B + w_it_row * LDK + w_it_kb * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_uint4(pack_bf2(w[8 * i + 0], w[8 * i + 1]), pack_bf2(w[8 * i + 2], w[8 * i + 3]),
                            pack_bf2(w[8 * i + 4], w[8 * i + 5]), pack_bf2(w[8 * i + 6], w[8 * i + 7]));
    } else {
      uint16_t* dst = B + (w_it_kb * 32) * LDK + w_it_row;
#pragma unroll
      for (int i = 0; i < 32; ++i) dst[i * LDK] = f2bf(w[i]);
    }
  };

  // ---- main loop
  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  const int nk = (p.K + BK - 1) / BK;
  load_a(0);
  load_w(0);
  store_a(0);
  store_w(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_a(kt + 1);
      load_w(kt + 1);
    }
    const uint16_t* A = As + cur * BM * LDK;
    const uint16_t* B = Bs + cur * BN * LDK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(A + (wm * WTM + a * 32 + (lane & 31)) * LDK +
                                                 kk * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8*>(B + (wn * WTN + b * 32 + (lane & 31)) * LDK +
                                                  kk * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    if (more) {
      store_a(cur ^ 1);
      store_w(cur ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogues.  acc[a][b][v] sits at local row
  //   lr = wm*WTM + a*32 + (v>>2)*8 + (lane>>5)*4 + (v&3), local col lc = wn*WTN + b*32 + (lane&31)
  const int r = p.r;
  const float s = p.s;
  auto LR = [&](int a, int v) { return wm * WTM + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); };
  auto LC = [&](int b) { return wn * WTN + b * 32 + (lane & 31); };
  auto dotr = [&](const float* x, const float* y) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) t += x[j] * y[j];
    return t;
  };

  if constexpr (EPI == EPI_LIN) {
    const float* Bm = p.lB0 + (int64_t)e * p.lB_estride;
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int n = n0 + LC(b);
      if (n >= p.N) continue;
      float bv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) bv[j] = j < r ? Bm[(int64_t)n * r + j] : 0.f;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t pr = r0 + LR(a, v);
          if (pr < r1) {
            const float val = acc[a][b][v] + s * dotr(p.rv0 + pr * r, bv);
            p.o0[pr * p.ldo + n] = f2bf(val);
          }
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int i = (n0 >> 1) + wn * 32 + (lane & 31);
    if (i < p.w_rows) {
      const float* Bg = p.lB0 + (int64_t)e * p.lB_estride + (int64_t)i * r;
      const float* Bu = p.lB1 + (int64_t)e * p.lB_estride + (int64_t)i * r;
      float bg[16], bu[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        bg[j] = j < r ? Bg[j] : 0.f;
        bu[j] = j < r ? Bu[j] : 0.f;
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t pr = r0 + LR(a, v);
          if (pr < r1) {
            const float g = acc[a][0][v] + s * dotr(p.rv0 + pr * r, bg);
            const float u = acc[a][1][v] + s * dotr(p.rv1 + pr * r, bu);
            const float h = g * sigmoidf_(g) * u;
            const int64_t o = pr * p.ldo + i;
            p.o0[o] = f2bf(h);
            p.o1[o] = f2bf(g);
            p.o2[o] = f2bf(u);
          }
        }
    }
  } else if constexpr (EPI == EPI_LIN_BWD || EPI == EPI_GATEUP_BWD) {
    constexpr bool DUAL = EPI == EPI_GATEUP_BWD;
    const float* A0 = p.lA0 + (int64_t)e * p.lA_estride;
    const float* A1 = DUAL ? p.lA1 + (int64_t)e * p.lA_estride : nullptr;
    float av0[TN][16], av1[TN][16];
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int c = n0 + LC(b);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        av0[b][j] = (c < p.N && j < r) ? A0[(int64_t)j * p.N + c] : 0.f;
        av1[b][j] = (DUAL && c < p.N && j < r) ? A1[(int64_t)j * p.N + c] : 0.f;
      }
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t pr = r0 + LR(a, v);
        if (pr >= r1) continue;
        float x0[16], x1[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          x0[j] = j < r ? p.rv0[pr * r + j] : 0.f;
          x1[j] = (DUAL && j < r) ? p.rv1[pr * r + j] : 0.f;
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int c = n0 + LC(b);
          if (c >= p.N) continue;
          float t = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            t += x0[j] * av0[b][j];
            if (DUAL) t += x1[j] * av1[b][j];
          }
          p.o0[pr * p.ldo + c] = f2bf(acc[a][b][v] + s * t);
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
    // columns are the expert's intermediate index i (< N = I).  Pass 0 writes
    // dg, du (bf16) and stages e*h for the dw row sums; passes 1 and 2 read
    // back this thread's own dg / du and stage them for the row dots with
    // Bg / Bu (the same rounded values the gate/up backward consumes).
    float* Z = reinterpret_cast<float*>(smem);
    const float* Ad = p.lA0 + (int64_t)e * p.lA_estride;
    const int width = 1 + 2 * r;
    {
      float av[TN][16];
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int c = n0 + LC(b);
#pragma unroll
        for (int j = 0; j < 16; ++j) av[b][j] = (c < p.N && j < r) ? Ad[(int64_t)j * p.N + c] : 0.f;
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = LR(a, v);
          const int64_t pr = r0 + lr;
          const bool rok = pr < r1;
          float x[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) x[j] = (rok && j < r) ? p.rv0[pr * r + j] : 0.f;
          const float wp = rok ? p.wflat[p.sorted[pr]] : 0.f;
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const int lc = LC(b);
            const int c = n0 + lc;
            float zv = 0.f;
            if (rok && c < p.N) {
              float t = 0.f;
#pragma unroll
              for (int j = 0; j < 16; ++j) t += x[j] * av[b][j];
              const float ev = acc[a][b][v] + s * t;
              const int64_t o = pr * p.ldo + c;
              const float gg = bf2f(p.s0[o]), uu = bf2f(p.s1[o]);
              const float sg = sigmoidf_(gg);
              const float silu = gg * sg;
              const float dh = wp * ev;
              p.o0[o] = f2bf(dh * uu * sg * (1.f + gg * (1.f - sg)));
              p.o1[o] = f2bf(dh * silu);
              zv = ev * silu * uu;
            }
            Z[lr * ZP + lc] = zv;
          }
        }
    }
    __syncthreads();
    z_row_reduce<BM, BN>(Z, nullptr, r, 1, n0, p.N, [&](int row, float(&out)[16]) {
      const int64_t pr = r0 + row;
      if (pr < r1) p.f0[((int64_t)ntile * p.M + pr) * width] = out[0];
    });
#pragma unroll 1
    for (int pass = 1; pass < 3; ++pass) {
      const uint16_t* src = pass == 1 ? p.o0 : p.o1;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = LR(a, v);
          const int64_t pr = r0 + lr;
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const int lc = LC(b);
            const int c = n0 + lc;
            Z[lr * ZP + lc] = (pr < r1 && c < p.N) ? bf2f(src[pr * p.ldo + c]) : 0.f;
          }
        }
      __syncthreads();
      const float* Wc = (pass == 1 ? p.lB1 : p.lB2) + (int64_t)e * p.lB_estride;
      const int off = pass == 1 ? 1 : 1 + r;
      z_row_reduce<BM, BN>(Z, Wc, r, r, n0, p.N, [&](int row, float(&out)[16]) {
        const int64_t pr = r0 + row;
        if (pr < r1) {
          float* dst = p.f0 + ((int64_t)ntile * p.M + pr) * width + off;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (j < r) dst[j] = out[j];
        }
      });
    }
  } else if constexpr (EPI == EPI_CE_FWD || EPI == EPI_CE_BWD) {
    float* Z = reinterpret_cast<float*>(smem);
    const int64_t V = p.V;
    const int64_t c0 = p.w_row0;  // vocab offset of this launch's columns
    const float* Bm = p.lB0;
    float coef = 0.f;
    if constexpr (EPI == EPI_CE_BWD) {
      const float nv = *p.nvalid;
      coef = nv > 0.f ? p.coef / nv : 0.f;
    }
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int lc = LC(b);
      const int n = n0 + lc;
      const int64_t vv = c0 + n;
      const bool vok = n < p.w_rows;  // inside this launch's vocab range
      float bv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) bv[j] = (vok && j < r) ? Bm[vv * r + j] : 0.f;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = LR(a, v);
          const int64_t pr = r0 + lr;
          float zv;
          if constexpr (EPI == EPI_CE_FWD) {
            zv = -INFINITY;
            if (pr < r1 && vok) zv = acc[a][b][v] + s * dotr(p.rv0 + pr * r, bv);
          } else {
            zv = 0.f;
            if (pr < r1) {
              const int64_t lab = p.labels[pr];
              const bool valid = lab != p.ignore_index && lab >= 0 && lab < V;
              if (valid && vok) {
                const float z = acc[a][b][v] + s * dotr(p.rv0 + pr * r, bv);
                zv = coef * (__expf(z - p.lse[pr]) - (vv == lab ? 1.f : 0.f));
              }
              if (n < p.ldo) p.o0[pr * p.ldo + n] = f2bf(zv);
            }
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
      // G . B over this tile's vocab columns -> part_GB[ntile][T][r]
      z_row_reduce<BM, BN>(Z, Bm + c0 * r, r, r, n0, p.w_rows, [&](int row, float(&out)[16]) {
        const int64_t pr = r0 + row;
        if (pr < r1) {
          float* dst = p.f1 + ((int64_t)(p.ntile_base + ntile) * p.M + pr) * r;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (j < r) dst[j] = out[j];
        }
      });
      // G^T . xa over this tile's rows -> part_dB[mtile][V][r]  (rewrite Z first)
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
            float zv = 0.f;
            if (pr < r1 && n < p.w_rows) {
              const int64_t lab = p.labels[pr];
              const bool valid = lab != p.ignore_index && lab >= 0 && lab < V;
              if (valid) {
                const int64_t vv = c0 + n;
                const float z = acc[a][b][v] + s * dotr(p.rv0 + pr * r, Bm + vv * r);
                zv = coef * (__expf(z - p.lse[pr]) - (vv == lab ? 1.f : 0.f));
              }
            }
            Z[lr * ZP + lc] = zv;
          }
      }
      __syncthreads();
      z_col_reduce<BM, BN>(Z, p.rv0, r, r0, r1, [&](int col, float(&out)[16]) {
        const int n = n0 + col;
        if (n < p.w_rows) {
          float* dst = p.f2 + ((int64_t)mslot * V + c0 + n) * r;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (j < r) dst[j] = out[j];
        }
      });
    }
  }
}

template <int QT, int EPI>
hipError_t launch_q(int tilecfg, const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles), block(NTHR);
  if (tilecfg == TILE_128x128)
    hipLaunchKernelGGL((gemm_kernel<QT, EPI, 128, 128>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((gemm_kernel<QT, EPI, 64, 128>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace gq
