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
//
// The second kernel in this file, skinny_nn_kernel, is the transposed (NN)
// counterpart for the backward data gradient; its own comment describes it.
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
  // adapter-fold rows (xa, or xa_g / xa_u) of the tile, 16 ranks each, and
  // the rows' label columns (the LM head): written before the main loop
  constexpr int NXS = EPI == EPI_SWIGLU ? 2 : 1;
  __shared__ float lds_xa[NXS][RT * 16];
  __shared__ int32_t lds_lab[EPI == EPI_CE_FWD ? RT : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, q = lane >> 4;

  // workgroup -> tile in XCD-contiguous runs (ids go round-robin over the 8
  // XCDs).  Grouped launches lay the runs over the m-slots that hold rows
  // (tile_start[E] of them; the rest exit), n-tiles fastest, so the n-tiles
  // of one m-slot run together on one XCD; dense launches keep m fastest.
  auto xcd_run = [](int id, int count) {
    const int qq = count >> 3, rem = count & 7, xcd = id & 7, loc = id >> 3;
    return (xcd < rem ? xcd * (qq + 1) : rem * (qq + 1) + (xcd - rem) * qq) + loc;
  };
  int mslot, ntile;
  if (p.offsets) {
    const int used = p.tile_start[p.E] * p.ntiles;
    if ((int)blockIdx.x >= used) return;
    const int bid = xcd_run(blockIdx.x, used);
    mslot = bid / p.ntiles;
    ntile = bid - mslot * p.ntiles;
  } else {
    const int bid = xcd_run(blockIdx.x, gridDim.x);
    mslot = bid % p.mtiles;
    ntile = bid / p.mtiles;
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
    r0 = (int64_t)p.offsets[e] + (int64_t)(mslot - ts[e]) * RT;
    if (p.spill_bm > 0) {  // past the expert's full tiles (run by the tile MMQ)
      const int cnt = p.offsets[e + 1] - p.offsets[e];
      r0 += cnt - cnt % p.spill_bm;
    }
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

  // the adapter fold's operands and the label columns, loaded before the
  // main loop (their latency hides behind it): rows into LDS, this lane's
  // B row (its weight row, 16 ranks) into registers
  const int r = p.r;
  const float s_ = p.s;
  for (int i = tid; i < NXS * RT * 16; i += NTHR) {
    const int set = i / (RT * 16), rr = (i / 16) % RT, j = i % 16;
    const float* X = set ? p.rv1 : p.rv0;
    const int64_t pr = r0 + rr;
    lds_xa[set][rr * 16 + j] = (j < r && pr < r1) ? X[pr * r + j] : 0.f;
  }
  if constexpr (EPI == EPI_CE_FWD) {
    for (int i = tid; i < RT; i += NTHR) {
      const int64_t pr = r0 + i;
      int32_t rel = INT_MIN;  // ignored label (or no row)
      if (pr < r1) {
        const int64_t lab = p.labels[pr];
        if (lab != p.ignore_index && lab >= 0 && lab < p.V) rel = (int32_t)(lab - p.w_row0);
      }
      lds_lab[i] = rel;
    }
  }
  float bq[16];
  {
    const float* Bm;
    if constexpr (EPI == EPI_SWIGLU)
      Bm = (wave < 4 ? p.lB0 : p.lB1) + (int64_t)e * p.lB_estride;
    else if constexpr (EPI == EPI_CE_FWD)
      Bm = p.lB0 + (int64_t)p.w_row0 * r;
    else
      Bm = p.lB0 + (int64_t)e * p.lB_estride;
    Bm += (int64_t)(wok ? wrow : 0) * r;
#pragma unroll
    for (int j = 0; j < 16; ++j) bq[j] = (wok && j < r) ? Bm[j] : 0.f;
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
  // wrow.  Adapter term in fp32, from the rows staged in LDS and this lane's
  // B row in registers (ranks past r are zero in both).
  if (wok) {
    const float* X = lds_xa[EPI == EPI_SWIGLU && wave >= 4 ? 1 : 0];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float* xr = X + (rg * 16 + 4 * q + v) * 16;
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) t += xr[j] * bq[j];
        if (r0 + rg * 16 + 4 * q + v < r1) acc[rg][v] += s_ * t;
      }
  }

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
        if (wok && lds_lab[lr] == wrow) p.f1[pr] = acc[rg][v];  // (no label / no row: INT_MIN)
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
  if (a.r > 16) return hipErrorInvalidValue;  // the fold stages 16 ranks
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles), block(64 * SK_WAVES);
  if (rg == 1)
    mmq_launch((skinny_kernel<QT, EPI, 1>), grid, block, st, a);
  else if (rg == 2)
    mmq_launch((skinny_kernel<QT, EPI, 2>), grid, block, st, a);
  else
    mmq_launch((skinny_kernel<QT, EPI, 4>), grid, block, st, a);
  return hipGetLastError();
}


// Skinny NN MMQ (backward dX = dY deq(W) for few rows per weight): the
// reduction runs over weight rows, the outputs over a row's elements.  A
// workgroup (8 waves) owns 16 * RG output rows by 128 output columns (4
// blocks of every weight row); wave w owns the 32 columns of block w % 4 in
// reduction group w / 4.  Per step of 128 weight rows:
//  * the 128 row segments are read with coalesced 8-byte loads into a
//    shared LDS tile (double-buffered, one barrier per step; the next
//    step's loads are in flight meanwhile);
//  * lane l of wave w decodes block w % 4 of step row 64 (w / 4) + l and
//    writes its 32 bf16 values row-major into the wave's own LDS region,
//    read back transposed (ds_read_b64_tr_b16) as the B operand of
//    v_mfma_f32_16x16x32_bf16: reduction group g takes rows 64g .. 64g+63
//    of every step;
//  * the A operand (activation rows x 32 reduction rows) is read straight
//    from global memory; rows past the tile or the reduction are zero.
// The two groups' partial sums meet in LDS (group 0 + group 1, a fixed
// order).  A launch has twice the workgroups and half the sequential steps
// of one with 256 columns and 64-row steps: these launches are short grids
// whose time is the latency of each workgroup's chain of steps.
// The adapter term s * (X . A[:, col]) is added in fp32 in the epilogue.
// Epilogues: EPI_LIN_BWD (bf16 dX), EPI_GATEUP_BWD (reduction over the
// gate rows with dg, then the up rows with du; bf16 dX rows) and
// EPI_DOWN_BWD (the SwiGLU backward on the tile's e = dY deq(Wd) + adapter:
// e staged in LDS, one thread per 8 columns of a row with 16-byte g/u loads
// and dg/du stores, row partials dw, dg.Bg, du.Bu of the 128 columns summed
// over the row's 16 threads by xor shuffles in a fixed order).
constexpr int SKN_COLS = 128;  // output columns per workgroup
constexpr int SKN_ROWS = 128;  // reduction rows per step (two groups of 64)

// Adapter term of a skinny NN tile, s * sum_j X[row][j] * Y[j][col] (TWO:
// plus the second projection's X1, Y1), at the accumulator positions of a
// group-0 lane (row r0 + 16 rg + 4q + v, column c0 + 32 wave + 16 g + nl);
// zero outside the tile.
template <int RG, bool TWO>
__device__ __forceinline__ void nn_adapter(const GemmArgs& p, const float* Y0, const float* Y1,
                                           int64_t r0, int64_t r1, int c0, float (&ad)[RG][2][4]) {
  const int lane = threadIdx.x & 63, cg = (threadIdx.x >> 6) & 3;
  const int nl = lane & 15, q = lane >> 4;
  const int r = p.r;
  float t[RG][2][4];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) t[rg][g][v] = 0.f;
  // four ranks at a time, every load of a chunk issued together
#pragma unroll 1
  for (int jc = 0; jc < r; jc += 4) {
    float y0[2][4], y1[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int col = c0 + 32 * cg + 16 * g + nl;
      const bool okc = col < p.N;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bool ok = okc && jc + jj < r;
        y0[g][jj] = ok ? Y0[(int64_t)(jc + jj) * p.N + col] : 0.f;
        if constexpr (TWO) y1[g][jj] = ok ? Y1[(int64_t)(jc + jj) * p.N + col] : 0.f;
      }
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = r0 + rg * 16 + 4 * q + v;
        const bool okr = pr < r1;
        float x0[4], x1[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const bool ok = okr && jc + jj < r;
          x0[jj] = ok ? p.rv0[pr * r + jc + jj] : 0.f;
          if constexpr (TWO) x1[jj] = ok ? p.rv1[pr * r + jc + jj] : 0.f;
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            t[rg][g][v] += x0[jj] * y0[g][jj];
            if constexpr (TWO) t[rg][g][v] += x1[jj] * y1[g][jj];
          }
      }
  }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) ad[rg][g][v] = p.s * t[rg][g][v];
}

// SwiGLU backward on a skinny NN tile (RT = 16 RG rows x 128 columns of the
// intermediate index).  acc (valid in the group-0 waves) holds dY deq(Wd);
// Z (LDS, [RT][128 + 4] floats) and Bst (LDS, [2][128][8]) are free when
// this runs; every thread of the workgroup calls it.
template <int RG>
__device__ __forceinline__ void skinny_down_epilogue(const GemmArgs& p, const f32x4 (&acc)[RG][2],
                                                     int e, int64_t r0, int64_t r1, int c0,
                                                     int ntile, float* Z, float* Bst) {
  constexpr int RT = 16 * RG, ZD = SKN_COLS + 4, NT = 64 * SK_WAVES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, q = lane >> 4;
  const int r = p.r;
  const float* Ad = p.lA0 + (int64_t)e * p.lA_estride;
  const float* Bg = p.lB1 + (int64_t)e * p.lB_estride;
  const float* Bu = p.lB2 + (int64_t)e * p.lB_estride;
  // e = acc + s (dY Bd)[row] . Ad[:, col], staged by the group-0 waves
  if (wave < 4) {
    float ad[RG][2][4];
    nn_adapter<RG, false>(p, Ad, nullptr, r0, r1, c0, ad);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int lc = 32 * wave + 16 * g + nl;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) Z[(rg * 16 + 4 * q + v) * ZD + lc] = acc[rg][g][v] + ad[rg][g][v];
    }
  }
  // 16 threads per row (8 columns each), NT / 16 rows per pass
  constexpr int TPR = SKN_COLS / 8, RPP = NT / TPR;
  static_assert(RT <= RPP, "one pass covers the tile's rows");
  const int cq = tid % TPR, row = tid / TPR;
  const int width = 1 + 2 * r;
  auto rows = [&](auto rc, const int jb) {
    constexpr int R = decltype(rc)::value;
    const bool first = jb == 0;
    const int64_t pr = r0 + row;
    float dw = 0.f, ag[R], au[R];
#pragma unroll
    for (int j = 0; j < R; ++j) ag[j] = au[j] = 0.f;
    const int lc = cq * 8;
    const int c = c0 + lc;
    if (row < RT && pr < r1 && c < p.N) {  // N % 8 == 0: whole 8-column chunks
      const float wp = p.wflat[p.sorted[pr]];
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
      // rank partials with the stored bf16 dg, du
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float dq = __builtin_bit_cast(float, (dgp[t >> 1] >> (16 * (t & 1))) << 16);
        const float uq = __builtin_bit_cast(float, (dup[t >> 1] >> (16 * (t & 1))) << 16);
#pragma unroll
        for (int j = 0; j < R; ++j) {
          ag[j] += dq * Bst[(lc + t) * 8 + j];
          au[j] += uq * Bst[(SKN_COLS + lc + t) * 8 + j];
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
    if (cq == 0 && row < RT && pr < r1) {
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
  };
  // Bg, Bu of the tile's columns in LDS, 8 ranks at a time: rank 16 takes a
  // second pass over the rows for ranks 8..15 (dg, du recomputed, not stored)
  for (int jb = 0; jb < r; jb += 8) {
    if (jb) __syncthreads();  // the previous pass is done with Bst
    for (int idx = tid; idx < 2 * SKN_COLS * 8; idx += NT) {
      const int mat = idx / (SKN_COLS * 8), c = (idx >> 3) % SKN_COLS, j = idx & 7;
      const int col = c0 + c;
      Bst[idx] = (jb + j < r && col < p.N) ? (mat ? Bu : Bg)[(int64_t)col * r + jb + j] : 0.f;
    }
    __syncthreads();  // (first pass: also Z)
    if (r - jb <= 4)
      rows(IntC<4>{}, jb);
    else
      rows(IntC<8>{}, jb);
  }
}

template <int QT, int EPI, int RG>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_nn_kernel(const GemmArgs p) {
  static_assert(EPI == EPI_LIN_BWD || EPI == EPI_GATEUP_BWD || EPI == EPI_DOWN_BWD, "NN epilogues");
  static_assert(SK_WAVES == 8, "four column groups x two reduction groups");
  constexpr int BS = QTraits<QT>::BS;
  constexpr int SEGB = 4 * BS;             // bytes of a row's 4-block segment (8-byte multiple)
  constexpr int SEG8 = SEGB / 8;
  constexpr int NCH = SKN_ROWS * SEG8;     // 8-byte chunks per step
  constexpr int NTHR = 64 * SK_WAVES;
  constexpr int CI = (NCH + NTHR - 1) / NTHR;
  constexpr int RAWB = SKN_ROWS * SEGB + 16;  // raw tile bytes (tail read slack)
  constexpr int DP = 40;                   // decoded row pitch (bf16): 32 + 8
  constexpr int NQ = RawBlock<QT>::NQ;
  constexpr int RT = 16 * RG;
  static_assert(SEGB % 8 == 0, "8-byte chunks");
  __shared__ __attribute__((aligned(16))) uint8_t raw[2][RAWB];
  __shared__ __attribute__((aligned(16))) uint16_t dec[SK_WAVES][64 * DP];
  // SwiGLU backward: Bg, Bu rows of the tile's 128 columns (8 ranks at a time)
  __shared__ __attribute__((aligned(16))) float bst[EPI == EPI_DOWN_BWD ? 2 * SKN_COLS * 8 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = wave & 3, kg = wave >> 2;  // column group, reduction group
  const int nl = lane & 15, q = lane >> 4;

  // workgroup -> tile in XCD-contiguous runs (ids go round-robin over the 8
  // XCDs).  Grouped launches lay the runs over the m-slots that hold rows
  // (tile_start[E] of them; the rest exit), n-tiles fastest, so the n-tiles
  // of one m-slot run together on one XCD; dense launches keep m fastest.
  auto xcd_run = [](int id, int count) {
    const int qq = count >> 3, rem = count & 7, xcd = id & 7, loc = id >> 3;
    return (xcd < rem ? xcd * (qq + 1) : rem * (qq + 1) + (xcd - rem) * qq) + loc;
  };
  int mslot, ntile;
  if (p.offsets) {
    const int used = p.tile_start[p.E] * p.ntiles;
    if ((int)blockIdx.x >= used) return;
    const int bid = xcd_run(blockIdx.x, used);
    mslot = bid / p.ntiles;
    ntile = bid - mslot * p.ntiles;
  } else {
    const int bid = xcd_run(blockIdx.x, gridDim.x);
    mslot = bid % p.mtiles;
    ntile = bid / p.mtiles;
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
    r0 = (int64_t)p.offsets[e] + (int64_t)(mslot - ts[e]) * RT;
    if (p.spill_bm > 0) {  // past the expert's full tiles (run by the tile MMQ)
      const int cnt = p.offsets[e + 1] - p.offsets[e];
      r0 += cnt - cnt % p.spill_bm;
    }
    r1 = min((int64_t)p.offsets[e + 1], r0 + RT);
  } else {
    r0 = (int64_t)mslot * RT;
    if (r0 >= p.M) return;
    r1 = min(p.M, r0 + RT);
  }
  const int c0 = ntile * SKN_COLS;  // first output column (weight row element)
  const int Kr = p.K;               // reduction length (weight rows)
  const int nsteps = (Kr + SKN_ROWS - 1) / SKN_ROWS;

  // raw chunk loads: chunk t = row t / SEG8 of the step, bytes 8 (t % SEG8)
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
    crow[i] = tt / SEG8;
    coff[i] = (tt % SEG8) * 8;
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) u32x2 g_u32x2;
  // a step whose rows all lie below Kr and on one side of wsplit (the
  // common case, uniform across the workgroup) adds one scalar row offset to
  // a per-thread chunk offset; other steps take each chunk's row apart
  int64_t woff[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) woff[i] = (int64_t)crow[i] * p.w_rowbytes + coff[i];
  auto load_w = [&](int st, u32x2 (&wr)[CI]) {
    const int n0s = st * SKN_ROWS;
    if (n0s + SKN_ROWS <= Kr && (n0s + SKN_ROWS <= p.wsplit || n0s >= p.wsplit)) {
      const uint8_t* sb = n0s >= p.wsplit ? wbase1 + (int64_t)(n0s - p.wsplit) * p.w_rowbytes
                                          : wbase0 + (int64_t)n0s * p.w_rowbytes;
#pragma unroll
      for (int i = 0; i < CI; ++i) wr[i] = *(g_u32x2*)(sb + woff[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      int n = n0s + crow[i];
      if (n >= Kr) n = 0;
      const uint8_t* b = n >= p.wsplit ? wbase1 + (int64_t)(n - p.wsplit) * p.w_rowbytes
                                       : wbase0 + (int64_t)n * p.w_rowbytes;
      wr[i] = *(g_u32x2*)(b + coff[i]);
    }
  };
  auto store_w = [&](int buf, const u32x2 (&wr)[CI]) {
#pragma unroll
    for (int i = 0; i < CI; ++i)
      if (cval[i]) *reinterpret_cast<u32x2*>(&raw[buf][crow[i] * SEGB + coff[i]]) = wr[i];
  };

  // A fragments: lane (m, q) holds A[row 16 rg + m][step rows 64 kg + 32 ks + 8q .. +8]
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
  uint32_t amask[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    arow1[rg] = p.a1 ? arow[rg] - p.a0 + p.a1 : arow[rg];
    amask[rg] = opaque_mask(aok[rg]);
  }
  auto arow_n = [&](int st, int ks) { return st * SKN_ROWS + kg * 64 + ks * 32 + 8 * q; };
  auto load_a = [&](int st, bf16x8 (&af)[2][RG]) {
    const int n0s = st * SKN_ROWS;
    if (n0s + SKN_ROWS <= Kr && (n0s + SKN_ROWS <= p.asplit || n0s >= p.asplit)) {
      // whole step below Kr, one side of asplit: every lane reads its own
      // rows (rows past the tile read row r0's columns and are zeroed at use)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const int n = n0s + kg * 64 + ks * 32 + 8 * q;
          const uint16_t* src = n0s >= p.asplit ? arow1[rg] + (n - p.asplit) : arow[rg] + n;
          af[ks][rg] = *reinterpret_cast<const bf16x8*>(src);
        }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const int n = arow_n(st, ks);  // 8 reduction rows n .. n+7
        const bool ok = aok[rg] && n < Kr;
        const uint16_t* src = n >= p.asplit ? arow1[rg] + (n - p.asplit) : arow[rg] + n;
        // unconditional load (from the row start when out of range), zeroed
        // at its use: a conditional load, or a mask applied here, would make
        // the loads wait right away or with the weight loads issued later
        af[ks][rg] = *reinterpret_cast<const bf16x8*>(ok ? src : arow[rg]);
      }
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

  // one step of 128 reduction rows whose raw segments sit in raw[st & 1]
  auto compute_step = [&](int st, const bf16x8 (&af)[2][RG]) {
    const int buf = st & 1;
    __syncthreads();
    // decode block cg of step row 64 kg + lane into the wave's region
    {
      const int off = (kg * 64 + lane) * SEGB + cg * BS;
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
      uint32_t o[16];
      decode_block_bf16<QT>(rb, o);
      uint4* dst = reinterpret_cast<uint4*>(D + lane * DP);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) dst[q4] = make_uint4(o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]);
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
        for (int rg = 0; rg < RG; ++rg) {
          // rows past the tile or the reduction: zero A fragments (the
          // reduction test only matters in the last step)
          const uint32_t m = st * SKN_ROWS + SKN_ROWS <= Kr ? amask[rg] : opaque_mask(aok[rg] && arow_n(st, ks) < Kr);
          u32x4 av = __builtin_bit_cast(u32x4, af[ks][rg]);
          av &= m;
          acc[rg][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), b,
                                                               acc[rg][g], 0, 0, 0);
        }
      }
  };

  // Two-slot register ring: step s's weight chunks and A fragments sit in
  // slot s & 1 and are loaded one step ahead.  Loads past the last step
  // re-read it.
  u32x2 wr[2][CI];
  bf16x8 af[2][2][RG];
  load_w(0, wr[0]);
  load_a(0, af[0]);
  int st = 0;
  for (; st + 2 <= nsteps; st += 2) {
    store_w(0, wr[0]);
    load_w(min(st + 1, nsteps - 1), wr[1]);
    load_a(min(st + 1, nsteps - 1), af[1]);
    compute_step(st, af[0]);
    store_w(1, wr[1]);
    load_w(min(st + 2, nsteps - 1), wr[0]);
    load_a(min(st + 2, nsteps - 1), af[0]);
    compute_step(st + 1, af[1]);
  }
  if (st < nsteps) {
    store_w(0, wr[0]);
    compute_step(st, af[0]);
  }

  // ---- the two reduction groups meet: group 1's sums through LDS, added
  // to group 0's (fixed order)
  __syncthreads();  // every wave is done with the raw and decode regions
  float* red = reinterpret_cast<float*>(&dec[0][0]);  // [4][RG * 8][64]
  if (kg == 1) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((cg * RG + rg) * 8 + g * 4 + v) * 64 + lane] = acc[rg][g][v];
  }
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rg][g][v] += red[((cg * RG + rg) * 8 + g * 4 + v) * 64 + lane];
  }

  // ---- epilogue: group 0's acc[rg][g][v] at row r0 + 16 rg + 4q + v,
  // column c0 + 32 cg + 16 g + nl.  Adapter term in fp32:
  //   + s * sum_j X(row, j) * A[j][col]   (GATEUP: both projections)
  const float* Y0 = p.lA0 + (int64_t)e * p.lA_estride;
  const float* Y1 = EPI == EPI_GATEUP_BWD ? p.lA1 + (int64_t)e * p.lA_estride : nullptr;
  if constexpr (EPI == EPI_DOWN_BWD) {
    __syncthreads();  // group 0 is done reading the partial sums
    skinny_down_epilogue<RG>(p, acc, e, r0, r1, c0, ntile, reinterpret_cast<float*>(&dec[0][0]), bst);
    return;
  }
  if (kg != 0) return;
  float ad[RG][2][4];
  nn_adapter<RG, EPI == EPI_GATEUP_BWD>(p, Y0, Y1, r0, r1, c0, ad);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int col = c0 + 32 * cg + 16 * g + nl;
    if (col >= p.N) continue;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pr = r0 + rg * 16 + 4 * q + v;
        if (pr < r1) p.o0[pr * p.ldo + col] = f2bf(acc[rg][g][v] + ad[rg][g][v]);
      }
  }
}

template <int QT, int EPI>
hipError_t launch_skinny_nn(int rg, const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.mtiles * (unsigned)a.ntiles), block(64 * SK_WAVES);
  if (rg == 1)
    mmq_launch((skinny_nn_kernel<QT, EPI, 1>), grid, block, st, a);
  else
    mmq_launch((skinny_nn_kernel<QT, EPI, 2>), grid, block, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace gq
