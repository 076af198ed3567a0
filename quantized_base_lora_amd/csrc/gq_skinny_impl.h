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

}  // namespace
}  // namespace gq
