// Skinny MMQ for few rows per weight (small token counts, MoE experts with a
// handful of routed tokens): the same fused dequantize-and-multiply as the
// tile GEMM (page 2 "Show HN: LoRA over GGUF", section "Things involved in
// the training": MMQ and grouped MMQ over GGUF blocks), shaped for the case
// where every weight block is used by at most 16 * RG rows and the launch is
// bound by streaming the blocks from HBM.
//
//  * A workgroup is 8 waves; each wave owns 16 weight rows (SwiGLU: waves
//    0-3 the gate rows, waves 4-7 the up rows of the same 64 intermediate
//    indices).  v_mfma_f32_16x16x32_bf16: MFMA rows are activation rows (RG
//    groups of 16), MFMA columns are the wave's weight rows, one 32-wide
//    reduction step is one quant block per weight row.
//  * K is walked in super-steps of 8 blocks.  A weight row's 8 blocks are
//    one 16-byte aligned segment (272 / 144 / 96 bytes), so a wave reads its
//    16 segments with fully coalesced 16-byte loads (lane i of load j takes
//    chunk 64j + i), stores them unchanged in its own LDS region and then
//    every lane reads back the blocks it decodes.  Per-lane block loads from
//    HBM (16 rows x 34 bytes per instruction) reach half the bandwidth of
//    these.
//  * The activation tile of a super-step (16 * RG rows x 256 values) is
//    loaded once per workgroup into a double-buffered LDS tile (one barrier
//    per super-step); rows past the tile end are zero-filled, so no masking
//    is needed in the k loop.  The next super-step's loads are in flight
//    while the current one is multiplied.
//  * Q8_0 / Q4_0: lane (n, q) decodes whole blocks (row n, steps q and
//    4 + q) to bf16; the MFMA reduction order is permuted to match (in MFMA j
//    of a 4-step group lane (n, q) supplies values 8j .. 8j+7 of its block).
//  * Q2 scale/min: the decode is the costly part for 2-bit blocks, so the
//    B operand is the raw bit pair as the exact bf16 value 128 + u (one byte
//    permute per 2 values) and the block's scale and min are applied in
//    fp32 after the MFMA: acc += d * (x . (128 + u)) per block, and
//    sum_s (m_s - 128 d_s) * (sum of the block's 32 x values) once per 4
//    steps as a v_mfma_f32_16x16x4_f32 over per-(row, step) activation sums.
//  * The rank-r adapter term is added in fp32 in the epilogue
//    (y += s * xa[row] . B[col]).
//  * Epilogues: linear (bf16 store), SwiGLU (up values handed to the gate
//    waves through LDS), and the cross-entropy logits pass (per-row max /
//    sum-exp partials of the workgroup's 128 vocabulary rows, label logit).
//  Requires K % 256 == 0 and 16-byte aligned weight and activation rows;
//  the host falls back to the tile GEMM otherwise.
#pragma once
#include "gq_gemm_impl.h"

namespace gq {
namespace {

constexpr int SK_WAVES = 8;
constexpr int SK_COLS = 16 * SK_WAVES;  // weight rows (GEMM columns) per workgroup

template <int QT, int EPI, int RG>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_kernel(const GemmArgs p) {
  static_assert(EPI == EPI_LIN || EPI == EPI_SWIGLU || EPI == EPI_CE_FWD, "forward epilogues");
  constexpr bool RAW = QT == QT_Q2_DM;
  constexpr int BS = QTraits<QT>::BS;
  constexpr int SEGB = 8 * BS;              // bytes of one row's super-step segment
  constexpr int SEGQ = SEGB / 16;           // its 16-byte chunks
  constexpr int NCH = 16 * SEGQ;            // chunks per wave and super-step
  constexpr int NI = (NCH + 63) / 64;       // load instructions per wave and super-step
  constexpr int WREG = NCH * 16 + 16;       // per-wave LDS bytes (tail read slack)
  constexpr int NQ = RawBlock<QT>::NQ;
  constexpr int RT = 16 * RG;               // activation rows per tile
  constexpr int XROW = 80;                  // LDS bytes per (step, row): 64 + 16 pad
  constexpr int XBUF = 8 * RT * XROW;
  constexpr int NTHR = 64 * SK_WAVES;
  constexpr int XCH = RT * 32;              // 16-byte activation pieces per super-step
  constexpr int XI = XCH / NTHR;
  static_assert(XCH % NTHR == 0, "whole activation pieces per thread");
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[SK_WAVES][WREG];
  __shared__ __attribute__((aligned(16))) uint8_t lds_x[2][XBUF];
  __shared__ float lds_s[2][RAW ? 8 * RT : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, q = lane >> 4;

  int bid;
  {
    const int nblk = gridDim.x, qq = nblk >> 3, rem = nblk & 7;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    bid = (xcd < rem ? xcd * (qq + 1) : rem * (qq + 1) + (xcd - rem) * qq) + loc;
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
    r0 = (int64_t)p.offsets[e] + (int64_t)(mslot - ts[e]) * RT;
    r1 = min((int64_t)p.offsets[e + 1], r0 + RT);
  } else {
    r0 = (int64_t)mslot * RT;
    if (r0 >= p.M) return;
    r1 = min(p.M, r0 + RT);
  }

  // this wave's 16 weight rows
  const uint8_t* wsrc = p.w0;
  int wbase;
  if constexpr (EPI == EPI_SWIGLU) {
    wbase = ntile * (SK_COLS / 2) + (wave & 3) * 16;
    if (wave >= 4) wsrc = p.w1;
  } else {
    wbase = ntile * SK_COLS + wave * 16;
  }
  const int wrow = wbase + nl;  // the weight row of this lane's output column
  const bool wok = wrow < p.w_rows;
  const uint8_t* wmat = wsrc + (int64_t)e * p.w_estride + (int64_t)p.w_row0 * p.w_rowbytes;
  const uint8_t* gsrc[NI];
  bool cvalid[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = i * 64 + lane;
    cvalid[i] = c < NCH;
    const int cc = cvalid[i] ? c : 0;
    const int row = min(wbase + cc / SEGQ, p.w_rows - 1);  // rows past the end: re-read the last
    gsrc[i] = wmat + (int64_t)row * p.w_rowbytes + (cc % SEGQ) * 16;
  }
  uint8_t* wl = lds_w[wave];

  // activation pieces of this thread: row t / 32, values 8 (t % 32) .. +8
  // of the super-step; zero for rows past the tile
  const uint16_t* xsrc[XI];
  bool xok[XI];
  int xdst[XI], xsd[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int t = i * NTHR + tid;
    const int rr = t / 32, piece = t % 32;
    const int64_t pr = r0 + rr;
    xok[i] = pr < r1;
    int64_t src = xok[i] ? pr : r0;
    if (p.gather) src = p.gather[src] / p.gdiv;
    xsrc[i] = p.a0 + src * p.lda + piece * 8;
    xdst[i] = ((piece >> 2) * RT + rr) * XROW + (piece & 3) * 16;
    xsd[i] = (piece >> 2) * RT + rr;
  }

  const int nss = p.K / 256;
  f32x4 acc[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
  u32x4 wr[NI];
  uint4 xr[XI];
  auto gload = [&](int ss) {
#pragma unroll
    for (int i = 0; i < NI; ++i) wr[i] = *(g_u32x4*)(gsrc[i] + (int64_t)ss * SEGB);
#pragma unroll
    for (int i = 0; i < XI; ++i)
      xr[i] = xok[i] ? *reinterpret_cast<const uint4*>(xsrc[i] + ss * 256) : make_uint4(0, 0, 0, 0);
  };

  gload(0);
  for (int ss = 0; ss < nss; ++ss) {
    uint8_t* xl = lds_x[ss & 1];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const uint4 v = xr[i];
      *reinterpret_cast<uint4*>(xl + xdst[i]) = v;
      if constexpr (RAW) {
        // sum of the 32 values of (row, step): 4 consecutive threads
        float sum = bf2f(v.x & 0xffff) + bf2f(v.x >> 16) + bf2f(v.y & 0xffff) + bf2f(v.y >> 16) +
                    bf2f(v.z & 0xffff) + bf2f(v.z >> 16) + bf2f(v.w & 0xffff) + bf2f(v.w >> 16);
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        if ((tid & 3) == 0) lds_s[ss & 1][xsd[i]] = sum;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (cvalid[i]) *reinterpret_cast<u32x4*>(wl + (i * 64 + lane) * 16) = wr[i];
    gload(min(ss + 1, nss - 1));
    __syncthreads();

    if constexpr (!RAW) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        // block (row nl, step 4g + q) of the segment
        const int off = nl * SEGB + (4 * g + q) * BS;
        RawBlock<QT> rb;
        rb.hdr = *reinterpret_cast<const uint16_t*>(wl + off);
        const int sh = (off + 2) & 3;
        const uint32_t* d = reinterpret_cast<const uint32_t*>(wl + off + 2 - sh);
        uint32_t D[NQ + 1];
#pragma unroll
        for (int t = 0; t <= NQ; ++t) D[t] = d[t];
#pragma unroll
        for (int t = 0; t < NQ; ++t) rb.q[t] = __builtin_amdgcn_alignbyte(D[t + 1], D[t], sh);
        float w[32];
        decode_block_fast<QT>(rb, w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, make_uint4(pack_bf2(w[8 * j], w[8 * j + 1]), pack_bf2(w[8 * j + 2], w[8 * j + 3]),
                                 pack_bf2(w[8 * j + 4], w[8 * j + 5]), pack_bf2(w[8 * j + 6], w[8 * j + 7])));
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            const uint4 av =
                *reinterpret_cast<const uint4*>(xl + ((4 * g + q) * RT + rg * 16 + nl) * XROW + 16 * j);
            acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), b, acc[rg], 0, 0, 0);
          }
        }
      }
    } else {
      const float* sl = lds_s[ss & 1];
      const uint32_t MAG = 0x43434343u;  // bf16 128 + byte, two per dword
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = 4 * g + j;
          const uint32_t* dp = reinterpret_cast<const uint32_t*>(wl + nl * SEGB + s * BS);
          const float dd = h2f(dp[0] & 0xffffu);
          // values 8q .. 8q+7 of the block: bit pair q of its 8 bytes
          const uint32_t u0 = (dp[1] >> (2 * q)) & 0x03030303u;
          const uint32_t u1 = (dp[2] >> (2 * q)) & 0x03030303u;
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, make_uint4(__builtin_amdgcn_perm(MAG, u0, 0x04010400u), __builtin_amdgcn_perm(MAG, u0, 0x04030402u),
                                 __builtin_amdgcn_perm(MAG, u1, 0x04010400u), __builtin_amdgcn_perm(MAG, u1, 0x04030402u)));
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            const uint4 av = *reinterpret_cast<const uint4*>(xl + (s * RT + rg * 16 + nl) * XROW + 16 * q);
            const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), b,
                                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[rg][v] = __builtin_fmaf(dd, t[v], acc[rg][v]);
          }
        }
        // sum over steps 4g .. 4g+3 of xsum[row][s] * (m - 128 d)[col][s]
        const int s = 4 * g + q;
        const uint32_t h = *reinterpret_cast<const uint32_t*>(wl + nl * SEGB + s * BS);
        const float c = h2f(h >> 16) - 128.f * h2f(h & 0xffffu);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x4f32(sl[s * RT + rg * 16 + nl], c, acc[rg], 0, 0, 0);
      }
    }
  }

  // ---- epilogue.  acc[rg][v] sits at row r0 + rg*16 + 4q + v, weight row
  // wrow.  Adapter term in fp32.
  const int r = p.r;
  const float s_ = p.s;
  auto fold = [&](auto rc) {
    constexpr int R = decltype(rc)::value;
    if (!wok) return;
    const float* Bm;
    const float* X;
    if constexpr (EPI == EPI_SWIGLU) {
      Bm = (wave < 4 ? p.lB0 : p.lB1) + (int64_t)e * p.lB_estride;
      X = wave < 4 ? p.rv0 : p.rv1;
    } else if constexpr (EPI == EPI_CE_FWD) {
      Bm = p.lB0 + (int64_t)p.w_row0 * r;
      X = p.rv0;
    } else {
      Bm = p.lB0 + (int64_t)e * p.lB_estride;
      X = p.rv0;
    }
    float bv[R];
    load_rank<R>(Bm + (int64_t)wrow * r, r, bv);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll 1
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = r0 + rg * 16 + 4 * q + v;
        if (pr >= r1) continue;
        float xv[R];
        load_rank<R>(X + pr * r, r, xv);
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < R; ++j) t += xv[j] * bv[j];
        acc[rg][v] += s_ * t;
      }
  };
  if (r <= 4)
    fold(IntC<4>{});
  else if (r <= 8)
    fold(IntC<8>{});
  else
    fold(IntC<16>{});

  if constexpr (EPI == EPI_LIN) {
    if (!wok) return;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = r0 + rg * 16 + 4 * q + v;
        if (pr < r1) p.o0[pr * p.ldo + wrow] = f2bf(acc[rg][v]);
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // up waves hand their values to the gate waves of the same indices
    __syncthreads();  // every wave is done with the activation tiles
    float* xch = reinterpret_cast<float*>(&lds_x[0][0]);
    static_assert(4 * 64 * 4 * RG * sizeof(float) <= XBUF, "exchange fits");
    if (wave >= 4) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) xch[(((wave - 4) * RG + rg) * 4 + v) * 64 + lane] = acc[rg][v];
    }
    __syncthreads();
    if (wave >= 4 || !wok) return;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = r0 + rg * 16 + 4 * q + v;
        if (pr < r1) {
          const float g = acc[rg][v], u = xch[((wave * RG + rg) * 4 + v) * 64 + lane];
          const float h = g / (1.0f + __expf(-g)) * u;
          const int64_t o = pr * p.ldo + wrow;
          p.o0[o] = f2bf(h);
          p.o1[o] = f2bf(g);
          p.o2[o] = f2bf(u);
        }
      }
  } else {
    // cross-entropy logits: per row, online (max, sum exp) over this
    // workgroup's 128 vocabulary rows; the 16 lanes of one quarter hold the
    // same rows (xor shuffles), then the 8 waves in order through LDS; the
    // label logit is written by its lane
    __shared__ float2 part[SK_WAVES][RT];
    const int64_t V = p.V;
    const int64_t c0 = p.w_row0;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int lr = rg * 16 + 4 * q + v;
        const int64_t pr = r0 + lr;
        float m = wok ? acc[rg][v] : -INFINITY;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
        float l = (wok && m != -INFINITY) ? __expf(acc[rg][v] - m) : 0.f;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 16);
        if (nl == 0) part[wave][lr] = make_float2(m, l);
        if (pr < r1 && wok) {
          const int64_t lab = p.labels[pr];
          if (lab != p.ignore_index && lab >= 0 && lab < V && c0 + wrow == lab) p.f1[pr] = acc[rg][v];
        }
      }
    __syncthreads();
    if (tid < RT) {
      const int lr = tid;
      const int64_t pr = r0 + lr;
      if (pr < r1) {
        float m = part[0][lr].x, l = part[0][lr].y;
#pragma unroll
        for (int w = 1; w < SK_WAVES; ++w) {
          const float m2 = part[w][lr].x, l2 = part[w][lr].y;
          if (m2 == -INFINITY) continue;
          if (m2 > m) {
            l = (m == -INFINITY ? 0.f : l * __expf(m - m2)) + l2;
            m = m2;
          } else {
            l += l2 * __expf(m2 - m);
          }
        }
        float* dst = p.f0 + ((int64_t)(p.ntile_base + ntile) * p.M + pr) * 2;
        dst[0] = m;
        dst[1] = l;
      }
    }
  }
}

template <int QT, int EPI>
hipError_t launch_skinny(int rg, const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles), block(64 * SK_WAVES);
  if (rg == 1)
    hipLaunchKernelGGL((skinny_kernel<QT, EPI, 1>), grid, block, 0, st, a);
  else if (rg == 2)
    hipLaunchKernelGGL((skinny_kernel<QT, EPI, 2>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((skinny_kernel<QT, EPI, 4>), grid, block, 0, st, a);
  return hipGetLastError();
}


// Skinny NN MMQ (backward dX = dY deq(W) for few rows per weight): the
// reduction runs over weight rows, the outputs over a row's elements.  A
// workgroup (8 waves) owns 16 * RG output rows by 256 output columns (8
// blocks of every weight row, one 16-byte aligned segment); wave w owns the
// 32 columns of block w.  Per step of 64 weight rows:
//  * the 64 row segments are read with coalesced 16-byte loads into a shared
//    LDS tile (double-buffered, one barrier per step; the next step's loads
//    are in flight meanwhile);
//  * lane l of wave w decodes block w of step row l and writes its 32 bf16
//    values row-major into the wave's own LDS region, read back transposed
//    (ds_read_b64_tr_b16) as the B operand of v_mfma_f32_16x16x32_bf16;
//  * the A operand (activation rows x 32 reduction rows) is read straight
//    from global memory; rows past the tile or the reduction are zero.
// The adapter term s * (X . A[:, col]) is added in fp32 in the epilogue.
// Epilogues: EPI_LIN_BWD (bf16 dX) and EPI_GATEUP_BWD (reduction over the
// gate rows with dg, then the up rows with du; bf16 dX rows).
constexpr int SKN_COLS = 256;  // output columns per workgroup

template <int QT, int EPI, int RG>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_nn_kernel(const GemmArgs p) {
  static_assert(EPI == EPI_LIN_BWD || EPI == EPI_GATEUP_BWD, "NN epilogues");
  constexpr int BS = QTraits<QT>::BS;
  constexpr int SEGB = 8 * BS;             // bytes of a row's 8-block segment
  constexpr int SEGQ = SEGB / 16;
  constexpr int NCH = 64 * SEGQ;           // 16-byte chunks per step
  constexpr int NTHR = 64 * SK_WAVES;
  constexpr int CI = (NCH + NTHR - 1) / NTHR;
  constexpr int RAWB = 64 * SEGB + 16;     // raw tile bytes (tail read slack)
  constexpr int DP = 40;                   // decoded row pitch (bf16): 32 + 8
  constexpr int NQ = RawBlock<QT>::NQ;
  constexpr int RT = 16 * RG;
  __shared__ __attribute__((aligned(16))) uint8_t raw[2][RAWB];
  __shared__ __attribute__((aligned(16))) uint16_t dec[SK_WAVES][64 * DP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, q = lane >> 4;

  int bid;
  {
    const int nblk = gridDim.x, qq = nblk >> 3, rem = nblk & 7;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    bid = (xcd < rem ? xcd * (qq + 1) : rem * (qq + 1) + (xcd - rem) * qq) + loc;
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
    r0 = (int64_t)p.offsets[e] + (int64_t)(mslot - ts[e]) * RT;
    r1 = min((int64_t)p.offsets[e + 1], r0 + RT);
  } else {
    r0 = (int64_t)mslot * RT;
    if (r0 >= p.M) return;
    r1 = min(p.M, r0 + RT);
  }
  const int c0 = ntile * SKN_COLS;  // first output column (weight row element)
  const int Kr = p.K;               // reduction length (weight rows)
  const int nsteps = (Kr + 63) / 64;

  // raw chunk loads: chunk t = row t / SEGQ of the step, bytes 16 (t % SEGQ)
  // of the row's segment; rows past the reduction re-read row 0
  const uint8_t* wbase0 = p.w0 + (int64_t)e * p.w_estride + (int64_t)ntile * SEGB;
  const uint8_t* wbase1 = p.w1 ? p.w1 + (int64_t)e * p.w_estride + (int64_t)ntile * SEGB : wbase0;
  int crow[CI], coff[CI];
  bool cval[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int t = i * NTHR + tid;
    cval[i] = t < NCH;
    const int tt = cval[i] ? t : 0;
    crow[i] = tt / SEGQ;
    coff[i] = (tt % SEGQ) * 16;
  }
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
  u32x4 wr[CI];
  auto load_w = [&](int st) {
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      int n = st * 64 + crow[i];
      if (n >= Kr) n = 0;
      const uint8_t* b = n >= p.wsplit ? wbase1 + (int64_t)(n - p.wsplit) * p.w_rowbytes
                                       : wbase0 + (int64_t)n * p.w_rowbytes;
      wr[i] = *(g_u32x4*)(b + coff[i]);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CI; ++i)
      if (cval[i]) *reinterpret_cast<u32x4*>(&raw[buf][crow[i] * SEGB + coff[i]]) = wr[i];
  };

  // A fragments: lane (m, q) holds A[row 16 rg + m][n0 + 32 ks + 8q .. +8]
  const uint16_t* arow[RG];
  bool aok[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int64_t pr = r0 + rg * 16 + nl;
    aok[rg] = pr < r1;
    int64_t src = aok[rg] ? pr : r0;
    if (p.gather) src = p.gather[src] / p.gdiv;
    arow[rg] = p.a0 + src * p.lda;
  }
  const uint16_t* arow1[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) arow1[rg] = p.a1 ? arow[rg] - p.a0 + p.a1 : arow[rg];
  auto load_a = [&](int st, int ks, int rg) -> bf16x8 {
    const int n = st * 64 + ks * 32 + 8 * q;  // 8 reduction rows n .. n+7
    const bool ok = aok[rg] && n < Kr;
    const uint16_t* src = n >= p.asplit ? arow1[rg] + (n - p.asplit) : arow[rg] + n;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = *reinterpret_cast<const uint4*>(src);
    return __builtin_bit_cast(bf16x8, v);
  };

  // transposed reads: lane 16g + 4t + m addresses decoded row 8g + t (+4),
  // columns 4m .. +4 of a 16-column group; lane 16g + c then holds rows
  // 8g .. 8g+7 of column c
  const int tr_row = 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3);
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  uint16_t* D = dec[wave];

  f32x4 acc[RG][2];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[rg][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_w(0);
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    store_w(buf);
    if (st + 1 < nsteps) load_w(st + 1);
    bf16x8 af[2][RG];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) af[ks][rg] = load_a(st, ks, rg);
    __syncthreads();
    // decode block `wave` of step row `lane` into the wave's region
    {
      const int off = lane * SEGB + wave * BS;
      RawBlock<QT> rb;
      if constexpr (QT == QT_Q2_DM) {
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&raw[buf][off]);
        rb.hdr = d[0]; rb.q[0] = d[1]; rb.q[1] = d[2];
      } else {
        rb.hdr = *reinterpret_cast<const uint16_t*>(&raw[buf][off]);
        const int sh = (off + 2) & 3;
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&raw[buf][off + 2 - sh]);
        uint32_t Dw[NQ + 1];
#pragma unroll
        for (int t = 0; t <= NQ; ++t) Dw[t] = d[t];
#pragma unroll
        for (int t = 0; t < NQ; ++t) rb.q[t] = __builtin_amdgcn_alignbyte(Dw[t + 1], Dw[t], sh);
      }
      float w[32];
      decode_block_fast<QT>(rb, w);
      uint4* dst = reinterpret_cast<uint4*>(D + lane * DP);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        dst[q4] = make_uint4(pack_bf2(w[8 * q4 + 0], w[8 * q4 + 1]), pack_bf2(w[8 * q4 + 2], w[8 * q4 + 3]),
                             pack_bf2(w[8 * q4 + 4], w[8 * q4 + 5]), pack_bf2(w[8 * q4 + 6], w[8 * q4 + 7]));
    }
    // (the wave's own region: the LDS writes above complete before the
    // reads below in this wave's program order)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint16_t* base = D + (ks * 32 + tr_row) * DP + g * 16 + tr_col;
        const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(__attribute__((address_space(3))) void*)(base));
        const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(__attribute__((address_space(3))) void*)(base + 4 * DP));
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 both = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        const bf16x8 b = __builtin_bit_cast(bf16x8, both);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          acc[rg][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][rg], b, acc[rg][g], 0, 0, 0);
      }
  }

  // ---- epilogue: acc[rg][g][v] at row r0 + 16 rg + 4q + v, column
  // c0 + 32 wave + 16 g + nl.  Adapter term in fp32:
  //   + s * sum_j X(row, j) * A[j][col]   (GATEUP: both projections)
  const int r = p.r;
  const float s_ = p.s;
  const float* Y0 = p.lA0 + (int64_t)e * p.lA_estride;
  const float* Y1 = EPI == EPI_GATEUP_BWD ? p.lA1 + (int64_t)e * p.lA_estride : nullptr;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int col = c0 + 32 * wave + 16 * g + nl;
    if (col >= p.N) continue;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll 1
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = r0 + rg * 16 + 4 * q + v;
        if (pr >= r1) continue;
        float t = 0.f;
        for (int j = 0; j < r; ++j) t += p.rv0[pr * r + j] * Y0[(int64_t)j * p.N + col];
        if constexpr (EPI == EPI_GATEUP_BWD)
          for (int j = 0; j < r; ++j) t += p.rv1[pr * r + j] * Y1[(int64_t)j * p.N + col];
        p.o0[pr * p.ldo + col] = f2bf(acc[rg][g][v] + s_ * t);
      }
  }
}

template <int QT, int EPI>
hipError_t launch_skinny_nn(int rg, const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles), block(64 * SK_WAVES);
  if (rg == 1)
    hipLaunchKernelGGL((skinny_nn_kernel<QT, EPI, 1>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((skinny_nn_kernel<QT, EPI, 2>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace gq
