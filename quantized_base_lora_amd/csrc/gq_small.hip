// Small (HBM- or latency-bound) kernels around the MFMA GEMMs.
//
//  * block decode export (gq_dequant)
//  * rank-r adapter passes: row dots (x A^T, dY B) one wave per row with a
//    shuffle reduction; column outer-product reductions (dA, dB) over fixed
//    row chunks with partials summed in chunk order (deterministic, no float
//    atomics)
//  * MoE routing after OpenAI's triton-kernels (page 2 "Show HN: LoRA over
//    GGUF", section "Things involved in the training"): wave-per-token top-k,
//    a stable counting sort by expert (per-chunk histograms, a scan, and
//    in-chunk ranks from an LDS key scan) -- positions never come from atomics
//  * the sparse combine of the experts' outputs and its backward
//  * the online log-sum-exp merge of the chunked cross entropy
#include <math.h>
#include <string.h>
#include <type_traits>

#include "gq_dev.h"
#include "gq_internal.h"

namespace gq {

namespace {

// ---------------------------------------------------------------- dequant
template <int QT>
__global__ void dequant_kernel(const uint8_t* __restrict__ blocks, int64_t nblocks,
                               int out_bf16, void* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  constexpr int BS = QTraits<QT>::BS;
  // 2-byte loads only: blocks are 2-byte aligned and may end the buffer
  const uint16_t* h = reinterpret_cast<const uint16_t*>(blocks + b * BS);
  RawBlock<QT> rb;
  if constexpr (QT == QT_Q2_DM) {
    rb.hdr = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
#pragma unroll
    for (int i = 0; i < RawBlock<QT>::NQ; ++i)
      rb.q[i] = (uint32_t)h[2 + 2 * i] | ((uint32_t)h[3 + 2 * i] << 16);
  } else {
    rb.hdr = h[0];
#pragma unroll
    for (int i = 0; i < RawBlock<QT>::NQ; ++i)
      rb.q[i] = (uint32_t)h[1 + 2 * i] | ((uint32_t)h[2 + 2 * i] << 16);
  }
  float w[32];
  decode_block<QT>(rb, w);
  if (out_bf16) {
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = make_uint4(pack_bf2(w[8 * i], w[8 * i + 1]), pack_bf2(w[8 * i + 2], w[8 * i + 3]),
                        pack_bf2(w[8 * i + 4], w[8 * i + 5]), pack_bf2(w[8 * i + 6], w[8 * i + 7]));
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  }
}

// ------------------------------------------------------ tile prefix (E <= 1024)
// Exclusive prefix over experts of ceil(rows_e / bm[q]) for up to three tile
// or chunk heights at once (one launch instead of one per height):
// ts_q[e] = first tile of expert e, ts_q[E] = number of tiles.
// The offsets are checked on the way: offsets[0] == 0, non-decreasing,
// offsets[E] == M.  Invalid offsets (e.g. from expert ids outside [0, E))
// set *err to 1 and make every prefix zero, so the launches that follow
// process no rows (nothing is read or written out of bounds); valid ones
// set *err to 0.
__global__ __launch_bounds__(1024) void tile_start_kernel(const int32_t* __restrict__ offsets,
                                                          int32_t E, int64_t M, int3 bm, int32_t* ts0,
                                                          int32_t* ts1, int32_t* ts2,
                                                          int32_t* __restrict__ err, int32_t spill,
                                                          int32_t spill_whole, int32_t* ts3) {
  __shared__ int32_t sh[4][1024];
  const int t = threadIdx.x;
  const int bms[3] = {bm.x, bm.y, bm.z};
  int32_t* outs[4] = {ts0, ts1, ts2, ts3};
  int cnt = t < E ? offsets[t + 1] - offsets[t] : 0;
  bool bad_t = cnt < 0;
  if (t == 0) bad_t = bad_t || offsets[0] != 0 || (int64_t)offsets[E] != M;
  const bool bad = __syncthreads_or(bad_t) != 0;
  if (bad) cnt = 0;
  if (t == 0 && err) *err = bad ? 1 : 0;
#pragma unroll
  for (int q = 0; q < 3; ++q) sh[q][t] = (t < E && outs[q]) ? (cnt + bms[q] - 1) / bms[q] : 0;
  // spill rows: a remainder of 1..spill rows past the full bm0-row tiles
  // (spill_whole: only an expert's whole 1..spill rows) leaves the tile MMQ
  // for ceil(rem / spill) skinny tiles
  const int rem = cnt % bms[0];
  const bool sp = ts3 && spill > 0 && rem > 0 && rem <= spill && (!spill_whole || cnt <= spill);
  if (sp) sh[0][t] -= 1;
  sh[3][t] = sp ? (rem + spill - 1) / spill : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int add[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) add[q] = t >= o ? sh[q][t - o] : 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) sh[q][t] += add[q];
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!outs[q]) continue;
    if (t < E) outs[q][t + 1] = sh[q][t];
    if (t == 0) outs[q][0] = 0;
  }
}

__device__ __forceinline__ int find_expert(const int32_t* offsets, int E, int64_t p) {
  int lo = 0, hi = E;  // offsets[lo] <= p < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------- row dots
// out[o][p][j] = sum_c act(p)[c] * W_o(e_p)[j][c], j < r <= 16, on the
// 16x16x32 bf16 MFMA: rows p are the MFMA rows, ranks j its columns, the
// activation columns c its reduction.  A block owns 16 consecutive rows and
// its eight waves take every eighth 32-column step; the fp32 rank vectors
// enter as bf16 hi + lo parts (about 16 significant bits).  Rows of a block
// that belong to different experts (sorted grouped rows) are covered by one
// pass per expert with the other rows masked.  The eight wave partials are
// added in wave order through LDS (deterministic).
// WT: W stored [C][r] (a LoRA B matrix) instead of [r][C] (an A matrix).
constexpr int RD_WAVES = 8;

// CS: dense rows over a.csplit column ranges (one workgroup each).
template <int NOUT, bool WT, bool CS>
__global__ __launch_bounds__(64 * RD_WAVES) void rowdot_kernel(const RowDotArgs a) {
  __shared__ f32x4 red[RD_WAVES - 1][NOUT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = a.r;
  const int cs = CS ? a.csplit : 1;  // column ranges (dense only)
  // rows p0 .. p1-1 of one expert: grouped rows come in expert-aligned
  // 16-row tiles (prefix tile16), so every block makes one pass with one
  // expert's rank vectors
  int64_t p0, p1;
  int e = 0;
  if (a.tile16) {
    // XCD-contiguous runs over the used tiles (ids go round-robin over the
    // 8 XCDs): the tiles of one expert, which read its rank vectors, share
    // an L2
    const int used = a.tile16[a.E];
    if ((int)blockIdx.x >= used) return;
    const int q8 = used >> 3, rem = used & 7, xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const int tile = (xcd < rem ? xcd * (q8 + 1) : rem * (q8 + 1) + (xcd - rem) * q8) + loc;
    e = find_expert(a.tile16, a.E, tile);
    p0 = (int64_t)a.offsets[e] + (int64_t)(tile - a.tile16[e]) * 16;
    p1 = min((int64_t)a.offsets[e + 1], p0 + 16);
  } else {
    p0 = (int64_t)(CS ? blockIdx.x / cs : blockIdx.x) * 16;
    p1 = min(a.M, p0 + 16);
  }
  // this workgroup's column range (whole 256-column groups)
  int part = 0, c_lo = 0, c_hi = a.C;
  if constexpr (CS) {
    part = (int)blockIdx.x % cs;
    const int ngrp = (a.C + 32 * RD_WAVES - 1) / (32 * RD_WAVES);
    c_lo = part * ngrp / cs * 32 * RD_WAVES;
    c_hi = min(a.C, (part + 1) * ngrp / cs * 32 * RD_WAVES);
  }
  // the activation row this lane feeds into the MFMA (row lane % 16)
  const int64_t pa = p0 + (lane & 15);
  const bool pav = pa < p1;
  const int64_t src = !pav ? 0 : (a.gather ? (int64_t)(a.gather[pa] / a.gdiv) : pa);
  const uint16_t* arow = a.act + src * a.lda + 8 * (lane >> 4);
  const int j = lane & 15;  // rank column this lane feeds (B operand)
  const bool jok = j < r;
  const int jc = jok ? j : 0;  // clamped: every load below stays in bounds
  f32x4 acc[NOUT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o) acc[o] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int UNR = 4;  // 32-column steps whose loads are issued together
  {
    const bool rowok = pav;
    const float* Wb[NOUT];
#pragma unroll
    for (int o = 0; o < NOUT; ++o) Wb[o] = a.W[o] + (int64_t)e * a.w_estride + (int64_t)jc * a.w_jstride;
    for (int cb = c_lo + wave * 32; cb < c_hi; cb += 32 * RD_WAVES * UNR) {
      uint4 raw[UNR];
      float w8[UNR][NOUT][8];
      bool aok[UNR], wok[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = cb + u * 32 * RD_WAVES + 8 * (lane >> 4);
        const bool cok = c < c_hi;  // C % 8 == 0: whole 8-column chunks
        const int cc = cok ? c : 0;
        aok[u] = rowok && cok;
        wok[u] = jok && cok;
        raw[u] = *reinterpret_cast<const uint4*>(aok[u] ? arow + (c - 8 * (lane >> 4)) : a.act);
#pragma unroll
        for (int o = 0; o < NOUT; ++o) {
          if constexpr (WT) {
#pragma unroll
            for (int t = 0; t < 8; ++t) w8[u][o][t] = Wb[o][(int64_t)(cc + t) * a.w_cstride];
          } else {
            const float4 lo = *reinterpret_cast<const float4*>(Wb[o] + cc);
            const float4 hi = *reinterpret_cast<const float4*>(Wb[o] + cc + 4);
            w8[u][o][0] = lo.x; w8[u][o][1] = lo.y; w8[u][o][2] = lo.z; w8[u][o][3] = lo.w;
            w8[u][o][4] = hi.x; w8[u][o][5] = hi.y; w8[u][o][6] = hi.z; w8[u][o][7] = hi.w;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint4 rv = aok[u] ? raw[u] : make_uint4(0u, 0u, 0u, 0u);
        const bf16x8 av = __builtin_bit_cast(bf16x8, rv);
#pragma unroll
        for (int o = 0; o < NOUT; ++o) {
          bf16x8 wh, wl;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float w = wok[u] ? w8[u][o][t] : 0.f;
            const __bf16 h = (__bf16)w;
            wh[t] = h;
            wl[t] = (__bf16)(w - (float)h);
          }
          acc[o] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wh, acc[o], 0, 0, 0);
          acc[o] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wl, acc[o], 0, 0, 0);
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o) red[wave - 1][o][lane] = acc[o];
  }
  __syncthreads();
  if (wave == 0 && jok) {
    // D layout: lane holds rank column lane % 16 of rows 4*(lane/16) .. +4
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
      f32x4 v = acc[o];
#pragma unroll
      for (int w = 0; w < RD_WAVES - 1; ++w) v += red[w][o][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t p = p0 + 4 * (lane >> 4) + q;
        if (p < p1) {
          a.out[o][(CS ? (int64_t)part * a.M * r : 0) + p * r + j] = v[q];
          if (o == 0 && a.out2) a.out2[p * r + j] = a.wflat[a.sorted[p]] * v[q];
          if (o == 0 && a.wout) a.wout[p * r + j] = a.wflat[a.sorted[p]] * a.win[p * r + j];
        }
      }
    }
  }
}

// ------------------------------------------------ down-backward row sums
// Row p of the grouped down MMQ's partials (one record of 1 + 2r floats per
// n-tile: dw, dg.Bg, du.Bu over that tile's columns), summed over the
// n-tiles in order.
__device__ void down_finish_row(const float* __restrict__ part, int32_t ntiles, int64_t M, int32_t r,
                                int64_t p, const int32_t* __restrict__ sorted, float* __restrict__ dw_flat,
                                float* __restrict__ dgB, float* __restrict__ duB) {
  const int width = 1 + 2 * r;
  float dw = 0.f, g[16], u[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) g[j] = u[j] = 0.f;
  for (int nt = 0; nt < ntiles; ++nt) {
    const float* src = part + ((int64_t)nt * M + p) * width;
    dw += src[0];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) {
        g[j] += src[1 + j];
        u[j] += src[1 + r + j];
      }
  }
  dw_flat[sorted[p]] = dw;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < r) {
      dgB[p * r + j] = g[j];
      duB[p * r + j] = u[j];
    }
}

// ---------------------------------------------------- column reductions
// part[slot][c][j] = sum_{rows p of slot} U(p)[c] * V[p][j]  (j < r <= 16),
// as D[j][c] = V^T U on v_mfma_f32_16x16x32_bf16: the reduction over rows is
// the MFMA k dimension.  A workgroup (4 waves) owns one slot and CR_COLS
// columns; rows go in steps of 32: the U rows (bf16, exact) are loaded with
// 16-byte coalesced loads into an LDS tile and read back transposed
// (ds_read_b64_tr_b16) as the B operand; the rank vectors enter as A in
// bf16 hi + lo parts (about 16 significant bits), two MFMAs per product.
// Each wave owns 64 columns (four 16-column MFMA tiles).  The next step's
// U loads are in flight while the current step is multiplied.  NV = 2: a
// second rank-vector array V2 over the same U rows (one pass over U for two
// reductions).  blockIdx.z picks one of two independent jobs sharing the
// launch (same rows and slots).
constexpr int CR_COLS = 256;
constexpr int CR_PITCH = CR_COLS + 8;  // bf16 elements per LDS tile row

// VS: job 1's rank vectors come as a.vsplit_1 partial arrays, summed on load.
template <int NV, bool VS>
__global__ __launch_bounds__(256) void colred_kernel(const ColRedArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][32 * CR_PITCH];
  const bool z1 = blockIdx.z == 1;
  const int32_t C = z1 ? a.C_1 : a.C;
  const uint16_t* const U = z1 ? a.U_1 : a.U;
  const int64_t ldu = z1 ? a.ldu_1 : a.ldu;
  const int32_t* const gather = z1 ? a.gather_1 : a.gather;
  const int32_t gdiv = z1 ? a.gdiv_1 : a.gdiv;
  const float* const V0 = z1 ? a.Vv_1 : a.Vv;
  const int vs = VS && z1 ? a.vsplit_1 : 1;  // partial arrays summed on load
  const int64_t vstride = a.M * a.r;
  float* const part0 = z1 ? a.part_1 : a.part;
  const int slot = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * CR_COLS;
  if (c0 >= C) return;  // this job has fewer columns
  int64_t r0, r1;
  if (a.offsets) {
    const int32_t* cs = a.chunk_start;
    if (slot >= cs[a.E]) return;
    const int e = find_expert(cs, a.E, slot);
    r0 = (int64_t)a.offsets[e] + (int64_t)(slot - cs[e]) * a.rc;
    r1 = min((int64_t)a.offsets[e + 1], r0 + a.rc);
  } else {
    r0 = (int64_t)slot * a.rc;
    r1 = min(a.M, r0 + a.rc);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  if (VS && z1 && a.vfinal_1) {
    // side job: the summed rank vectors of this slot's rows, spread over the
    // slot's column blocks of this job (every row lies in one slot)
    const int64_t nv = (r1 - r0) * r;
    const int nb = (C + CR_COLS - 1) / CR_COLS;
    const int64_t q0 = nv * blockIdx.y / nb, q1 = nv * (blockIdx.y + 1) / nb;
    for (int64_t q = q0 + tid; q < q1; q += 256) {
      const int64_t p = r0 + q / r;
      const int j = (int)(q % r);
      float v = V0[p * r + j];
      for (int sp = 1; sp < vs; ++sp) v += V0[sp * vstride + p * r + j];
      a.vfinal_1[p * r + j] = v;
    }
  }
  if (a.dfin_part && blockIdx.y == 0 && !z1) {
    // side job: every row lies in exactly one slot, and every slot has a
    // workgroup with column block 0 and job 0
    for (int64_t p = r0 + tid; p < r1; p += 256)
      down_finish_row(a.dfin_part, a.dfin_ntiles, a.M, r, p, a.dfin_sorted, a.dfin_dw, a.dfin_dgB,
                      a.dfin_duB);
  }

  // U tile loads: 32 rows x 256 columns = 1024 16-byte chunks, 4 per thread
  // (chunk t: row t / 32, columns 8 (t % 32) .. +8); zero past r1 or C
  constexpr int UCH = 4;
  int64_t uoff[UCH];
  int urow[UCH], ucol[UCH];
  bool ucok[UCH];
#pragma unroll
  for (int i = 0; i < UCH; ++i) {
    const int t = i * 256 + tid;
    urow[i] = t >> 5;
    ucol[i] = (t & 31) * 8;
    ucok[i] = c0 + ucol[i] < C;
    uoff[i] = c0 + (ucok[i] ? ucol[i] : 0);
  }
  uint4 ur[UCH];
  // source rows of the next load_u: gathered row indices are read one step
  // before the rows themselves, so the index load's latency is not paid in
  // series with the row load's
  int64_t srow[UCH];
  auto rows_for = [&](int64_t p0) {
#pragma unroll
    for (int i = 0; i < UCH; ++i) {
      const int64_t p = p0 + urow[i];
      const int64_t pc = p < r1 ? p : r0;
      srow[i] = gather ? (int64_t)(gather[pc] / gdiv) : pc;
    }
  };
  auto load_u = [&](int64_t p0) {
#pragma unroll
    for (int i = 0; i < UCH; ++i) {
      const int64_t p = p0 + urow[i];
      const bool ok = p < r1 && ucok[i];
      ur[i] = *reinterpret_cast<const uint4*>(U + srow[i] * ldu + uoff[i]);
      if (!ok) ur[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_u = [&](int buf) {
#pragma unroll
    for (int i = 0; i < UCH; ++i)
      *reinterpret_cast<uint4*>(&tile[buf][urow[i] * CR_PITCH + ucol[i]]) = ur[i];
  };

  // A operand: lane (j = lane % 16, q = lane / 16) holds V[p0 + 8q + i][j],
  // i < 8, as bf16 hi and lo
  const int aj = lane & 15, aq = lane >> 4;
  auto load_a = [&](const float* V, int64_t p0, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t p = p0 + 8 * aq + i;
      float v = 0.f;
      if (p < r1 && aj < r) {
        v = V[p * r + aj];
        if constexpr (VS)
          for (int sp = 1; sp < vs; ++sp) v += V[sp * vstride + p * r + aj];
      }
      const __bf16 h = (__bf16)v;
      hi[i] = h;
      lo[i] = (__bf16)(v - (float)h);
    }
  };

  // B operand (transposing reads): lane L = 16g + 4t + m addresses row
  // 8g + t (+4 for the second read) at column 4m of its 16-column tile;
  // lane 16g + c then holds rows 8g .. 8g+7 of column c
  const int tr_row = 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3);

  f32x4 acc[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[v][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  int buf = 0;
  rows_for(r0);
  load_u(r0);
  rows_for(r0 + 32);
  for (int64_t p0 = r0; p0 < r1; p0 += 32) {
    store_u(buf);
    if (p0 + 32 < r1) {
      load_u(p0 + 32);
      rows_for(p0 + 64);
    }
    bf16x8 ahi[NV], alo[NV];
    load_a(V0, p0, ahi[0], alo[0]);
    if constexpr (NV == 2) load_a(a.Vv2, p0, ahi[1], alo[1]);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint16_t* base = &tile[buf][tr_row * CR_PITCH + wave * 64 + g * 16 + tr_col];
      const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(__attribute__((address_space(3))) void*)(base));
      const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(__attribute__((address_space(3))) void*)(base + 4 * CR_PITCH));
      typedef short v8i16 __attribute__((ext_vector_type(8)));
      const v8i16 both = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      const bf16x8 b = __builtin_bit_cast(bf16x8, both);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        acc[v][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[v], b, acc[v][g], 0, 0, 0);
        acc[v][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[v], b, acc[v][g], 0, 0, 0);
      }
    }
    buf ^= 1;
  }
  // D layout: lane holds column lane % 16 of its tile, ranks 4 (lane / 16) .. +4
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    float* dst = v == 0 ? part0 : a.part2;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t c = c0 + wave * 64 + g * 16 + (lane & 15);
      if (c >= C) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 4 * (lane >> 4) + q;
        if (j < r) dst[((int64_t)slot * C + c) * r + j] = acc[v][g][q];
      }
    }
  }
}

// out[e] = s * sum_{slots of e} part[slot].  A block covers 256/SL outputs
// (c, j) of one expert with SL slot lanes each: lane g adds slots g, g+SL,
// ... in order, and the SL lane sums are added in lane order through LDS
// (deterministic), so many slots are read with many loads in flight.
template <int SL>
__global__ __launch_bounds__(256) void colred_finish_kernel(const ColFinJobs jb,
                                                            int32_t nslots, int32_t r, float s) {
  constexpr int NO = 256 / SL;
  __shared__ float red[SL][NO];
  const int z = blockIdx.z;
  const int32_t C = jb.C[z];
  const float* __restrict__ part = jb.part[z];
  const int oi = threadIdx.x % NO, g = threadIdx.x / NO;
  const int64_t n = (int64_t)C * r;
  const int64_t i = (int64_t)blockIdx.x * NO + oi;
  if ((int64_t)blockIdx.x * NO >= n) return;  // this job has fewer outputs
  float acc = 0.f;
  if (i < n) {
#pragma unroll 4
    for (int sl = g; sl < nslots; sl += SL) acc += part[(int64_t)sl * n + i];
  }
  red[g][oi] = acc;
  __syncthreads();
  if (g == 0 && i < n) {
    float t = red[0][oi];
#pragma unroll
    for (int k = 1; k < SL; ++k) t += red[k][oi];
    const int64_t c = i / r, jj = i % r;
    if (jb.transpose[z])
      jb.out[z][jj * C + c] = s * t;
    else
      jb.out[z][i] = s * t;
  }
}

// ----------------------------------------------------------------- routing
constexpr int ROUTE_CHUNK = 256;

// Selection key of logit v of expert ex: larger key = larger logit, ties to
// the lower expert index (the low word holds the complement of the index).
// -0 counts as +0; NaN ranks below every number.
__device__ __forceinline__ uint64_t topk_key(float v, int ex) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  if (v != v) o = 0u;
  return ((uint64_t)o << 32) | (uint32_t)(0xffffffffu - (uint32_t)ex);
}

// Maximum of a 64-bit value over the wave, returned to every lane: DPP
// exchanges within each 16-lane row (xor 1, xor 2, half mirror, mirror),
// then the four row maxima read as scalars.  No LDS traffic, so a round
// costs a few dozen cycles instead of six LDS permute round trips.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto step = [&](auto ctrl_c) {
    constexpr int CTRL = decltype(ctrl_c)::value;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, true);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  };
  step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{});  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    m = o > m ? o : m;
  }
  return m;
}

// One wave selects the top k of the E <= 64 NQ logits at row: k rounds of a
// wave arg-max over 64-bit keys, no branches.  Lane j < k returns selection j
// (expert and weight); every lane accumulates the softmax denominator in
// selection order, so all lanes hold the same value.
template <int NQ>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int32_t E, int32_t k,
                                          int lane, int& my_ex, float& my_w) {
  uint64_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int ex = lane + 64 * q;
    key[q] = ex < E ? topk_key(row[ex], ex) : 0ull;
  }
  float v0 = 0.f, sum = 0.f, my_v = 0.f;
  my_ex = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q) best = key[q] > best ? key[q] : best;
    best = wave_max_u64(best);
    const int ex = (int)(0xffffffffu - (uint32_t)best);
    // the logit back from the key (NaN came in as key 0: reported as NaN)
    const uint32_t o = (uint32_t)(best >> 32);
    const float v = o == 0u ? __builtin_nanf("") : __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
    if (j == 0) v0 = v;
    sum += __expf(v - v0);
    if (lane == j) { my_ex = ex; my_v = v; }
    // retire the winner (its owner lane clears the key)
#pragma unroll
    for (int q = 0; q < NQ; ++q) key[q] = key[q] == best ? 0ull : key[q];
  }
  my_w = __expf(my_v - v0) / sum;
}

template <class F>
__device__ __forceinline__ void with_nq(int32_t E, F&& f) {
  if (E <= 64) f(std::integral_constant<int, 1>{});
  else if (E <= 128) f(std::integral_constant<int, 2>{});
  else if (E <= 256) f(std::integral_constant<int, 4>{});
  else if (E <= 512) f(std::integral_constant<int, 8>{});
  else f(std::integral_constant<int, 16>{});
}

// one wave per token
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int32_t E, int32_t k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int ex;
  float wv;
  with_nq(E, [&](auto nq) { wave_topk<decltype(nq)::value>(logits + t * E, E, k, lane, ex, wv); });
  if (lane < k) {
    ids[t * k + lane] = ex;
    w[t * k + lane] = wv;
  }
}

// Few assignments (T k <= 256): the whole routing in one block of 1024
// threads -- top-k per token (one wave per token), expert counts, offsets,
// and the stable scatter (an assignment's rank among the earlier ones of its
// expert, counted over the assignment list in LDS; linear in T k, which is
// why larger counts take the chunked kernels).
constexpr int ROUTE_SMALL = 256;
__global__ __launch_bounds__(1024) void route_small_kernel(const float* __restrict__ logits,
                                                           int64_t T, int32_t E, int32_t k,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ w,
                                                           int32_t* __restrict__ sorted,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ pos) {
  __shared__ int32_t sid[ROUTE_SMALL];
  __shared__ int32_t cnt[1024];
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = (int)(T * k);
  for (int e = tid; e < 1024; e += 1024) cnt[e] = 0;
  for (int64_t t = wave; t < T; t += 16) {
    int ex;
    float wv;
    with_nq(E, [&](auto nq) { wave_topk<decltype(nq)::value>(logits + t * E, E, k, lane, ex, wv); });
    if (lane < k) {
      ids[t * k + lane] = ex;
      w[t * k + lane] = wv;
      sid[t * k + lane] = ex;
    }
  }
  __syncthreads();
  if (tid < n) atomicAdd(&cnt[sid[tid]], 1);  // integer counts: order-independent
  __syncthreads();
  // inclusive scan over the (up to 1024) experts
  const int c = tid < E ? cnt[tid] : 0;
  scan[tid] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  if (tid < E) offsets[tid] = scan[tid] - c;
  if (tid == 0) offsets[E] = scan[1023];
  if (tid < n) {
    const int key = sid[tid];
    int rank = 0;
    for (int j = 0; j < tid; ++j) rank += sid[j] == key;
    const int p = scan[key] - cnt[key] + rank;
    sorted[p] = tid;
    pos[tid] = p;
  }
}

__global__ void route_hist_kernel(const int32_t* __restrict__ ids, int64_t n, int32_t E,
                                  int32_t* __restrict__ counts) {
  __shared__ int32_t hist[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t a = (int64_t)blockIdx.x * ROUTE_CHUNK + threadIdx.x;
  if (a < n) atomicAdd(&hist[ids[a]], 1);  // integer counts: order-independent
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// one block of 1024 threads: per-expert running bases over chunks, then the
// exclusive scan over experts.  The chunk counts of an expert are read 8 at a
// time (independent loads in flight) in both passes.
__global__ void route_scan_kernel(int32_t* __restrict__ counts, int32_t nchunks, int32_t E,
                                  int32_t* __restrict__ offsets) {
  __shared__ int32_t sh[1024];
  constexpr int G = 8;
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += G) {
      int v[G];
#pragma unroll
      for (int i = 0; i < G; ++i) v[i] = c0 + i < nchunks ? counts[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < G; ++i) tot += v[i];
    }
  }
  sh[e] = tot;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = e >= o ? sh[e - o] : 0;
    __syncthreads();
    sh[e] += add;
    __syncthreads();
  }
  const int excl = sh[e] - tot;
  if (e < E) {
    offsets[e] = excl;
    int run = excl;
    for (int c0 = 0; c0 < nchunks; c0 += G) {
      int v[G];
#pragma unroll
      for (int i = 0; i < G; ++i) v[i] = c0 + i < nchunks ? counts[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (c0 + i < nchunks) counts[(int64_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
  }
  if (e == 0) offsets[E] = sh[1023];
}

__global__ void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t n, int32_t E,
                                     const int32_t* __restrict__ base, int32_t* __restrict__ sorted,
                                     int32_t* __restrict__ pos) {
  __shared__ int32_t keys[ROUTE_CHUNK];
  const int t = threadIdx.x;
  const int64_t a = (int64_t)blockIdx.x * ROUTE_CHUNK + t;
  const int key = a < n ? ids[a] : -1;
  keys[t] = key;
  __syncthreads();
  if (a >= n) return;
  int rank = 0;
  for (int j = 0; j < t; ++j) rank += keys[j] == key;
  const int p = base[(int64_t)blockIdx.x * E + key] + rank;
  sorted[p] = (int32_t)a;
  pos[a] = p;
}

__global__ __launch_bounds__(256) void route_bwd_kernel(const int32_t* __restrict__ ids,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ dw, int64_t T,
                                                        int32_t E, int32_t k,
                                                        float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float inner = 0.f;
  for (int j = 0; j < k; ++j) inner += w[t * k + j] * dw[t * k + j];
  for (int ex = lane; ex < E; ex += 64) {
    float v = 0.f;
    for (int j = 0; j < k; ++j)
      if (ids[t * k + j] == ex) v = w[t * k + j] * (dw[t * k + j] - inner);
    dl[t * E + ex] = v;
  }
}

// y[t][c..c+8) = sum_j w[t][j] rows[pos[t*k+j]][c..c+8)   (w == nullptr: weight 1)
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ rows,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ pos, int64_t T,
                                                      int32_t k, int64_t H,
                                                      uint16_t* __restrict__ out) {
  const int64_t nxb = (H + 2047) / 2048;  // column blocks per token
  const int64_t t = blockIdx.x / nxb;
  const int64_t c = ((blockIdx.x % nxb) * 256 + threadIdx.x) * 8;
  if (t >= T || c >= H) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t pr = pos[t * k + j];
    const float wj = w ? w[t * k + j] : 1.f;
    const uint4 raw = *reinterpret_cast<const uint4*>(rows + pr * H + c);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += wj * bf2f((uint16_t)(rw[q] & 0xffffu));
      acc[2 * q + 1] += wj * bf2f((uint16_t)(rw[q] >> 16));
    }
  }
  *reinterpret_cast<uint4*>(out + t * H + c) =
      make_uint4(pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]),
                 pack_bf2(acc[6], acc[7]));
}

// --------------------------------------------------------- cross entropy
// Online (max, sum exp) merge of log-sum-exp partials.
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  if (m2 == -INFINITY) return;
  if (m2 > m) {
    l = (m == -INFINITY ? 0.f : l * __expf(m - m2)) + l2;
    m = m2;
  } else {
    l += l2 * __expf(m2 - m);
  }
}

// Merge the per-tile (max, sum exp) partials [ntiles][T][2] of each token
// into lse.  A block of NT threads takes NT/LPT tokens with LPT lanes each;
// lane g merges tiles g, g+LPT, ... in order (eight loads in flight), and the
// LPT lane results are merged by a fixed pairwise tree in LDS, so the result
// does not depend on scheduling.  term[t] = lse - z[label] for a valid label.
template <int NT, int LPT>
__device__ __forceinline__ void ce_merge_tokens(const float* __restrict__ part, int32_t ntiles,
                                                int64_t T, int64_t t0,
                                                const float* __restrict__ zlab,
                                                const int64_t* __restrict__ labels, int64_t V,
                                                int64_t ignore_index, float* __restrict__ lse,
                                                float* __restrict__ term, float2* red) {
  constexpr int TPB = NT / LPT;
  const int ti = threadIdx.x % TPB, seg = threadIdx.x / TPB;
  const int64_t t = t0 + ti;
  float m = -INFINITY, l = 0.f;
  if (t < T) {
    for (int nb = seg; nb < ntiles; nb += 8 * LPT) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int nt = nb + u * LPT;
        v[u] = nt < ntiles ? *reinterpret_cast<const float2*>(part + ((int64_t)nt * T + t) * 2)
                           : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) lse_merge(m, l, v[u].x, v[u].y);
    }
  }
  red[threadIdx.x] = make_float2(m, l);
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) {
    __syncthreads();
    if (seg < o) {
      const float2 q = red[(seg + o) * TPB + ti];
      lse_merge(m, l, q.x, q.y);
      red[threadIdx.x] = make_float2(m, l);
    }
  }
  if (seg == 0 && t < T) {
    const float v = m + __logf(l);
    lse[t] = v;
    const int64_t lab = labels[t];
    term[t] = (lab != ignore_index && lab >= 0 && lab < V) ? v - zlab[t] : 0.f;
  }
}

template <int LPT>
__global__ __launch_bounds__(256) void ce_merge_kernel(const float* __restrict__ part,
                                                       int32_t ntiles, int64_t T,
                                                       const float* __restrict__ zlab,
                                                       const int64_t* __restrict__ labels, int64_t V,
                                                       int64_t ignore_index, float* __restrict__ lse,
                                                       float* __restrict__ term) {
  __shared__ float2 red[256];
  ce_merge_tokens<256, LPT>(part, ntiles, T, (int64_t)blockIdx.x * (256 / LPT), zlab, labels, V,
                            ignore_index, lse, term, red);
}

// Loss over the per-token terms, with the label checks: nvalid = number of
// labels in [0, V); err = 1 if a label is neither valid nor ignore_index.
// Fixed-order sums (one thread per strided subset, then a tree).
template <int NT>
__device__ __forceinline__ void ce_loss_block(const float* __restrict__ term,
                                              const int64_t* __restrict__ labels, int64_t T,
                                              int64_t V, int64_t ignore_index,
                                              int32_t* __restrict__ err, float* __restrict__ nvalid,
                                              float* __restrict__ loss, float* sh, int* shc) {
  float acc = 0.f;
  int c = 0, b = 0;
  for (int64_t t = threadIdx.x; t < T; t += NT) {
    acc += term[t];
    const int64_t lab = labels[t];
    if (lab == ignore_index) continue;
    if (lab >= 0 && lab < V) ++c; else ++b;
  }
  sh[threadIdx.x] = acc;
  shc[threadIdx.x] = c;
  shc[NT + threadIdx.x] = b;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      sh[threadIdx.x] += sh[threadIdx.x + o];
      shc[threadIdx.x] += shc[threadIdx.x + o];
      shc[NT + threadIdx.x] += shc[NT + threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float nv = (float)shc[0];
    *nvalid = nv;
    *err = shc[NT] ? 1 : 0;
    *loss = nv > 0.f ? sh[0] / nv : 0.f;
  }
}

__global__ __launch_bounds__(1024) void ce_loss_kernel(const float* __restrict__ term,
                                                       const int64_t* __restrict__ labels,
                                                       int64_t T, int64_t V, int64_t ignore_index,
                                                       int32_t* __restrict__ err,
                                                       float* __restrict__ nvalid,
                                                       float* __restrict__ loss) {
  __shared__ float sh[1024];
  __shared__ int shc[2048];
  ce_loss_block<1024>(term, labels, T, V, ignore_index, err, nvalid, loss, sh, shc);
}

// Few tokens: merge, loss and label checks in one block of 1024 threads.
template <int LPT>
__global__ __launch_bounds__(1024) void ce_merge_loss_kernel(
    const float* __restrict__ part, int32_t ntiles, int64_t T, const float* __restrict__ zlab,
    const int64_t* __restrict__ labels, int64_t V, int64_t ignore_index, float* __restrict__ lse,
    float* __restrict__ term, int32_t* __restrict__ err, float* __restrict__ nvalid,
    float* __restrict__ loss) {
  __shared__ float2 red[1024];
  __shared__ int shc[2048];
  ce_merge_tokens<1024, LPT>(part, ntiles, T, 0, zlab, labels, V, ignore_index, lse, term, red);
  __threadfence_block();
  __syncthreads();
  ce_loss_block<1024>(term, labels, T, V, ignore_index, err, nvalid, loss,
                      reinterpret_cast<float*>(red), shc);
}

__global__ void ce_final_dh_kernel(const float* __restrict__ dh_acc, int32_t nacc, const float* __restrict__ GB,
                                   const float* __restrict__ A, int64_t T, int32_t H, int32_t r,
                                   float s, uint16_t* __restrict__ dh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * H) return;
  const int64_t t = i / H, c = i % H;
  float v = 0.f;
  for (int j = 0; j < r; ++j) v += GB[t * r + j] * A[(int64_t)j * H + c];
  float acc = dh_acc[i];
  for (int q = 1; q < nacc; ++q) acc += dh_acc[q * T * H + i];
  dh[i] = f2bf(acc + s * v);
}

// out[p][j] = wflat[sorted[p]] * in[p][j]
__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void fill_u16_kernel(uint16_t* p, int64_t n, uint16_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

// ================================================================ launchers
hipError_t launch_dequant(int qtype, const void* blocks, int64_t rows, int64_t cols, int out_bf16,
                          void* out, hipStream_t st) {
  const int64_t nb = rows * (cols / 32);
  if (nb == 0) return hipSuccess;
  const dim3 g(blocks_for(nb, 256)), b(256);
  const uint8_t* bl = static_cast<const uint8_t*>(blocks);
  switch (qtype) {
    case QT_Q8_0: hipLaunchKernelGGL(dequant_kernel<QT_Q8_0>, g, b, 0, st, bl, nb, out_bf16, out); break;
    case QT_Q4_0: hipLaunchKernelGGL(dequant_kernel<QT_Q4_0>, g, b, 0, st, bl, nb, out_bf16, out); break;
    case QT_Q2_DM: hipLaunchKernelGGL(dequant_kernel<QT_Q2_DM>, g, b, 0, st, bl, nb, out_bf16, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tile_starts(const int32_t* offsets, int32_t E, int64_t M, int32_t* err,
                              int32_t bm0, int32_t* ts0, int32_t bm1, int32_t* ts1, int32_t bm2,
                              int32_t* ts2, hipStream_t st, int32_t spill, int32_t* ts_sp,
                              bool spill_whole) {
  if (ts_sp && (spill < 1 || spill > bm0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_start_kernel, dim3(1), dim3(1024), 0, st, offsets, E, M,
                     make_int3(bm0, bm1, bm2), ts0, ts1, ts2, err, spill, spill_whole ? 1 : 0, ts_sp);
  return hipGetLastError();
}

int rowdot_csplit(int64_t M, int64_t C) {
  const int64_t nwg = (M + 15) / 16;
  int cs = 1;
  while (cs < 4 && nwg * cs * 2 <= 256 && C / (cs * 2) >= 768) cs *= 2;
  return cs;
}

hipError_t launch_rowdot(const RowDotArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const unsigned cs = a.csplit > 1 ? (unsigned)a.csplit : 1u;
  if (cs > 1 && (a.tile16 || a.out2 || a.wout)) return hipErrorInvalidValue;
  // grouped: at most M/16 + E expert-aligned tiles; dense: cs per 16 rows
  const dim3 g(blocks_for(a.M, 16) * cs + (a.tile16 ? (unsigned)a.E : 0u)), b(64 * RD_WAVES);
  const bool wt = a.w_jstride == 1;
  if (cs > 1) {
    if (a.nout != 1) return hipErrorInvalidValue;
    if (wt) hipLaunchKernelGGL((rowdot_kernel<1, true, true>), g, b, 0, st, a);
    else hipLaunchKernelGGL((rowdot_kernel<1, false, true>), g, b, 0, st, a);
  } else if (a.nout == 2) {
    if (wt) hipLaunchKernelGGL((rowdot_kernel<2, true, false>), g, b, 0, st, a);
    else hipLaunchKernelGGL((rowdot_kernel<2, false, false>), g, b, 0, st, a);
  } else {
    if (wt) hipLaunchKernelGGL((rowdot_kernel<1, true, false>), g, b, 0, st, a);
    else hipLaunchKernelGGL((rowdot_kernel<1, false, false>), g, b, 0, st, a);
  }
  return hipGetLastError();
}

// Split-K fixup: two output columns per thread (enough threads to hide the
// latency of the few dependent loads), the parts summed in split order.
__global__ __launch_bounds__(256) void split_fixup_kernel(const float* __restrict__ part, int ksplit, int64_t M,
                                                          int32_t N, const float* __restrict__ X, int32_t r,
                                                          const float* __restrict__ Y, int64_t ys_n, int64_t ys_j,
                                                          float scale, uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nc = N / 2;
  if (i >= M * nc) return;
  const int64_t t = i / nc;
  const int n = (int)(i % nc) * 2;
  float v0 = 0.f, v1 = 0.f;
  for (int k = 0; k < ksplit; ++k) {
    const float2 a = *reinterpret_cast<const float2*>(part + ((int64_t)k * M + t) * N + n);
    v0 += a.x;
    v1 += a.y;
  }
  for (int j = 0; j < r; ++j) {
    const float xj = scale * X[t * r + j];
    v0 = __builtin_fmaf(xj, Y[(int64_t)n * ys_n + (int64_t)j * ys_j], v0);
    v1 = __builtin_fmaf(xj, Y[(int64_t)(n + 1) * ys_n + (int64_t)j * ys_j], v1);
  }
  *reinterpret_cast<uint32_t*>(out + t * ldo + n) = pack_bf2(v0, v1);
}

hipError_t launch_split_fixup(const float* part, int ksplit, int64_t M, int32_t N, const float* X, int32_t r,
                              const float* Y, int64_t ys_n, int64_t ys_j, float scale, uint16_t* out,
                              int64_t ldo, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (N % 2 || ldo % 2 || (uintptr_t)out % 4 || (uintptr_t)part % 8) return hipErrorInvalidValue;
  const int64_t n = M * (N / 2);
  hipLaunchKernelGGL(split_fixup_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, part, ksplit, M, N, X, r,
                     Y, ys_n, ys_j, scale, out, ldo);
  return hipGetLastError();
}

int colred_cols_per_block(int) { return CR_COLS; }

hipError_t launch_colred(const ColRedArgs& a, hipStream_t st) {
  if (a.slots == 0) return hipSuccess;
  if (a.r > 16) return hipErrorInvalidValue;
  const bool two = a.njobs == 2;
  const int32_t cmax = two && a.C_1 > a.C ? a.C_1 : a.C;
  const dim3 g((unsigned)a.slots, blocks_for(cmax, CR_COLS), two ? 2 : 1), b(256);
  const bool vsum = two && a.vsplit_1 > 1;
  if (a.Vv2) {
    if (two) return hipErrorInvalidValue;
    hipLaunchKernelGGL((colred_kernel<2, false>), g, b, 0, st, a);
  } else if (vsum) {
    hipLaunchKernelGGL((colred_kernel<1, true>), g, b, 0, st, a);
  } else {
    hipLaunchKernelGGL((colred_kernel<1, false>), g, b, 0, st, a);
  }
  return hipGetLastError();
}

// Grouped finish: out[e] = s * sum of expert e's slots, in slot order.  A
// thread owns four consecutive outputs (one 16-byte load per slot); experts
// with no slots get zeros.  blockIdx.z = job.
__global__ __launch_bounds__(256) void colred_finish_grp_kernel(const ColFinJobs jb,
                                                                const int32_t* __restrict__ cs,
                                                                int32_t r, float s) {
  const int z = blockIdx.z;
  const int e = blockIdx.y;
  const int32_t C = jb.C[z];
  const float* __restrict__ part = jb.part[z];
  const int transpose = jb.transpose[z];
  const int64_t n = (int64_t)C * r;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const int s0 = cs[e], s1 = cs[e + 1];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int sl = s0; sl < s1; ++sl) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)sl * n + i);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
  float* o = jb.out[z] + (int64_t)e * n;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t ii = i + q;
    if (transpose)
      o[(ii % r) * C + ii / r] = s * a4[q];
    else
      o[ii] = s * a4[q];
  }
}

hipError_t launch_colred_finish_grp(const ColFinJobs& j, const int32_t* chunk_start, int32_t E,
                                    int32_t r, float s, hipStream_t st) {
  if (j.n < 1 || j.n > 4) return hipErrorInvalidValue;
  int64_t nmax = 0;
  for (int z = 0; z < j.n; ++z) {
    const int64_t n = (int64_t)j.C[z] * r;  // a multiple of 4: C % 8 == 0
    if (n > nmax) nmax = n;
  }
  const dim3 g(blocks_for(nmax, 1024), (unsigned)E, (unsigned)j.n), b(256);
  hipLaunchKernelGGL(colred_finish_grp_kernel, g, b, 0, st, j, chunk_start, r, s);
  return hipGetLastError();
}

hipError_t launch_colred_finish(const float* part, const int32_t* chunk_start, int32_t E,
                                int32_t nslots_dense, int32_t C, int32_t r, float s, int transpose,
                                float* out, hipStream_t st) {
  if (chunk_start) {
    ColFinJobs j;
    memset(&j, 0, sizeof j);
    j.n = 1; j.part[0] = part; j.out[0] = out; j.C[0] = C; j.transpose[0] = transpose;
    return launch_colred_finish_grp(j, chunk_start, E, r, s, st);
  }
  ColFinJobs j;
  memset(&j, 0, sizeof j);
  j.n = 1; j.part[0] = part; j.out[0] = out; j.C[0] = C; j.transpose[0] = transpose;
  return launch_colred_finish_dense(j, nslots_dense, r, s, st);
}

hipError_t launch_colred_finish_dense(const ColFinJobs& j, int32_t nslots, int32_t r, float s,
                                      hipStream_t st) {
  if (j.n < 1 || j.n > 4) return hipErrorInvalidValue;
  int64_t nmax = 0;
  for (int z = 0; z < j.n; ++z) {
    const int64_t n = (int64_t)j.C[z] * r;
    if (n > nmax) nmax = n;
  }
  // many slots per output (long reductions): 32 slot lanes
  if (nslots > 64) {
    const dim3 g(blocks_for(nmax, 8), 1, (unsigned)j.n), b(256);
    hipLaunchKernelGGL(colred_finish_kernel<32>, g, b, 0, st, j, nslots, r, s);
  } else {
    const dim3 g(blocks_for(nmax, 32), 1, (unsigned)j.n), b(256);
    hipLaunchKernelGGL(colred_finish_kernel<8>, g, b, 0, st, j, nslots, r, s);
  }
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* part, int32_t nparts, int64_t rows, int32_t width,
                            float scale, float* out, hipStream_t st) {
  if (rows * width == 0) return hipSuccess;
  return launch_colred_finish(part, nullptr, 1, nparts, (int32_t)rows, width, scale, 0, out, st);
}

size_t route_ws_bytes(int64_t T, int32_t E, int32_t k) {
  const int64_t n = T * k;
  const int64_t nch = (n + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  return (size_t)(nch * E * sizeof(int32_t));
}

hipError_t launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                        float* w, int32_t* sorted, int32_t* offsets, int32_t* pos, void* ws,
                        hipStream_t st) {
  const int64_t n = T * k;
  if (n <= ROUTE_SMALL) {
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(1024), 0, st, logits, T, E, k, ids, w,
                       sorted, offsets, pos);
    return hipGetLastError();
  }
  const int nch = (int)((n + ROUTE_CHUNK - 1) / ROUTE_CHUNK);
  int32_t* counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(topk_kernel, dim3(blocks_for(T, 4)), dim3(256), 0, st, logits, T, E, k, ids, w);
  hipLaunchKernelGGL(route_hist_kernel, dim3(nch), dim3(ROUTE_CHUNK), 0, st, ids, n, E, counts);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, st, counts, nch, E, offsets);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nch), dim3(ROUTE_CHUNK), 0, st, ids, n, E, counts,
                     sorted, pos);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const int32_t* ids, const float* w, const float* dw, int64_t T,
                            int32_t E, int32_t k, float* dlogits, hipStream_t st) {
  hipLaunchKernelGGL(route_bwd_kernel, dim3(blocks_for(T, 4)), dim3(256), 0, st, ids, w, dw, T, E,
                     k, dlogits);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* rows, const float* w, const int32_t* pos, int64_t T,
                          int32_t k, int64_t H, uint16_t* out, hipStream_t st) {
  const dim3 g((unsigned)(blocks_for(H, 2048) * T)), b(256);
  hipLaunchKernelGGL(combine_kernel, g, b, 0, st, rows, w, pos, T, k, H, out);
  return hipGetLastError();
}


hipError_t launch_ce_merge(const float* part_ml, int32_t ntiles, int64_t T, const float* zlab,
                           const int64_t* labels, int64_t V, int64_t ignore_index, float* lse,
                           float* term, int32_t* err, float* nvalid, float* loss,
                           hipStream_t st) {
  int lpt1 = 256;
  while ((int64_t)lpt1 * T > 1024) lpt1 /= 2;
  if (T <= 64 && (int64_t)lpt1 * 24 >= ntiles) {
    // few tokens and partials: one block of 1024 threads, lpt1 lanes per token
    const int lpt = lpt1;
#define GQ_CE1(L) \
  hipLaunchKernelGGL(ce_merge_loss_kernel<L>, dim3(1), dim3(1024), 0, st, part_ml, ntiles, T, zlab, \
                     labels, V, ignore_index, lse, term, err, nvalid, loss)
    switch (lpt) {
      case 16: GQ_CE1(16); break;
      case 32: GQ_CE1(32); break;
      case 64: GQ_CE1(64); break;
      case 128: GQ_CE1(128); break;
      default: GQ_CE1(256); break;
    }
#undef GQ_CE1
    return hipGetLastError();
  }
  // lanes per token: enough that each lane merges at most ~16 partials
  int lpt = 16;
  while (lpt < 256 && (int64_t)lpt * 16 < ntiles) lpt *= 2;
  const dim3 g((unsigned)blocks_for(T, 256 / lpt)), b(256);
#define GQ_CEM(L) \
  hipLaunchKernelGGL(ce_merge_kernel<L>, g, b, 0, st, part_ml, ntiles, T, zlab, labels, V, \
                     ignore_index, lse, term)
  switch (lpt) {
    case 16: GQ_CEM(16); break;
    case 32: GQ_CEM(32); break;
    case 64: GQ_CEM(64); break;
    case 128: GQ_CEM(128); break;
    default: GQ_CEM(256); break;
  }
#undef GQ_CEM
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(1024), 0, st, term, labels, T, V, ignore_index,
                     err, nvalid, loss);
  return hipGetLastError();
}

hipError_t launch_ce_final_dh(const float* dh_acc, int32_t nacc, const float* GB, const float* A, int64_t T,
                              int32_t H, int32_t r, float s, uint16_t* dh, hipStream_t st) {
  const int64_t n = T * H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_final_dh_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, dh_acc, nacc, GB, A,
                     T, H, r, s, dh);
  return hipGetLastError();
}


hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* p, int64_t n, uint16_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u16_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace gq
