// Internal launch interface between the C ABI (gq_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace gq {

// GEMM epilogues of the one MFMA kernel template (gq_gemm.hip).
//   NT = the reduction runs along the weight's block dimension (forward):
//        C[p][n] = sum_k act[p][k] * deq(W)[n][k]
//   NN = the reduction runs along the weight's rows (backward):
//        C[p][c] = sum_n act[p][n] * deq(W)[n][c]
enum Epi {
  EPI_LIN = 0,      // NT: out = C + s * rv0[p] . lB0[n]            -> bf16
  EPI_SWIGLU,       // NT: gate/up pair, h = silu(g) u               -> bf16 g,u,h
  EPI_CE_FWD,       // NT: per-row (max, sumexp) partials + label logit
  EPI_CE_BWD,       // NT: G tile -> bf16, partial G.B and G^T.xa
  EPI_LIN_BWD,      // NN: out = C + s * rv0[p] . lA0[:, c]          -> bf16
  EPI_DOWN_BWD,     // NN: MoE down backward + SwiGLU backward
  EPI_GATEUP_BWD,   // NN: dxrows = C + s (rv0 . lA0 + rv1 . lA1)    -> bf16
  EPI_DH_ACC,       // NN: f0 (+)= C                                  fp32
  EPI_COUNT
};

struct GemmArgs {
  // geometry: M rows, N output columns, K reduction length
  int64_t M;
  int32_t N;
  int32_t K;
  // activation operand (bf16 rows); a1 serves reduction indices >= asplit
  const uint16_t* a0;
  const uint16_t* a1;
  int64_t lda;
  int32_t asplit;
  const int32_t* gather;  // row p reads a[gather[p] / gdiv]
  int32_t gdiv;
  // weights: raw blocks, w1 = second projection (gate/up pairs)
  const uint8_t* w0;
  const uint8_t* w1;
  int64_t w_estride;   // bytes between experts
  int64_t w_rowbytes;  // bytes per weight row
  int32_t w_nb;        // blocks per weight row
  int32_t w_rows;      // rows per weight source (NN: bound on the reduction rows)
  int32_t wsplit;      // NN: reduction index where w1 starts
  int32_t w_row0;      // first weight row (chunk offset)
  // grouping (offsets == nullptr: dense)
  int32_t E;
  const int32_t* offsets;
  const int32_t* tile_start;
  int32_t mtiles;      // m-tile slots in the grid
  int32_t ntiles;
  // epilogue
  float s;
  int32_t r;
  const float* lA0;
  const float* lA1;
  const float* lB0;
  const float* lB1;
  const float* lB2;
  int64_t lA_estride;  // floats between experts
  int64_t lB_estride;
  const float* rv0;    // per-row rank vectors [M][r]
  const float* rv1;
  // EPI_LIN_BWD: rv0 as rv_parts partial arrays (rv0 + s * M * r) summed by
  // the adapter fold; with rv_out, the workgroups of column tile 0 store
  // that sum (rv_out[p][j]).  0 or 1: one array.
  int32_t rv_parts;
  float* rv_out;
  uint16_t* o0;
  uint16_t* o1;
  uint16_t* o2;
  int64_t ldo;
  float* f0;
  float* f1;
  float* f2;
  int64_t ldf;
  const uint16_t* s0;  // saved g
  const uint16_t* s1;  // saved u
  const float* wflat;
  const int32_t* sorted;
  const int64_t* labels;
  const float* lse;
  float coef;
  int64_t ignore_index;
  int32_t V;
  int32_t ntile_base;  // global n-tile index of this launch's first n-tile
  int32_t accum;       // EPI_DH_ACC: add into f0
  const float* nvalid; // EPI_CE_BWD: device count of valid labels
  // split-K (dense EPI_LIN / EPI_LIN_BWD, one group of waves, K % 64 == 0):
  // ksplit > 1 workgroups per tile take contiguous k-step ranges and store
  // their fp32 sums in part[split][M][N] (no adapter term, no bf16 output);
  // launch_split_fixup then adds the parts, the adapter term, and rounds.
  int32_t ksplit;
  float* part;
  // grouped skinny launch over spill rows: each expert's rows start after its
  // full spill_bm-row tiles (those run on the tile MMQ); 0 = all its rows
  int32_t spill_bm;
};

// TILE_128x128_K2: 128x128 tiles computed by 512 threads, two groups of four
// waves taking alternate k-steps (split-K inside the workgroup), reduced in
// LDS; only for the epilogues that do not stage through LDS.
// TILE_SKINNY{16,32,64}: the forward-only skinny MMQ for few rows per
// weight (16, 32 or 64 rows per tile, 128 weight rows per workgroup;
// K % 256 == 0).
// TILE_WIDE: 256 x 192 tiles on 512 threads (gq_wide_impl.h), dense
// forward launches and the LM head's gradient tiles, with Q8_0 / Q4_0
// weights, K % 64 == 0 and rank <= WIDE_MAX_RANK only.
// TILE_WIDE_NN: 256 x 128 backward (NN) tiles on 512 threads, the reduction
// cut into ksplit (1 or 2) ranges of one workgroup each, fp32 sums per range
// (gq_wide_nn_impl.h): the LM head's dh, Q8_0 / Q4_0 weights.
enum TileCfg {
  TILE_128x128 = 0,
  TILE_64x128 = 1,
  TILE_128x128_K2 = 2,
  TILE_SKINNY16 = 3,
  TILE_SKINNY32 = 4,
  TILE_SKINNY64 = 5,
  TILE_WIDE = 6,
  TILE_WIDE_NN = 7
};
constexpr int WIDE_BM = 256, WIDE_BN = 192;
constexpr int WIDE_NN_BM = 256, WIDE_NN_BN = 128;
constexpr int WIDE_MAX_RANK = 16;  // adapter rank the wide tile stages in LDS

inline bool tile_skinny(int cfg) { return cfg >= TILE_SKINNY16 && cfg <= TILE_SKINNY64; }
inline int tile_bm(int cfg) {
  switch (cfg) {
    case TILE_WIDE: return WIDE_BM;
    case TILE_WIDE_NN: return WIDE_NN_BM;
    case TILE_64x128: return 64;
    case TILE_SKINNY16: return 16;
    case TILE_SKINNY32: return 32;
    case TILE_SKINNY64: return 64;
    default: return 128;
  }
}
inline int tile_bn(int) { return 128; }
constexpr int TILE_BN = 128;
constexpr int GEMM_BK = 64;

hipError_t launch_gemm(int qtype, int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
// One launch of EPI_CE_BWD tiles (`ce`, 128 x 128, TILE_128x128) followed by
// EPI_DH_ACC tiles (`dh`, 128 x 128, one group of four waves).
hipError_t launch_ce_bwd_dh(int qtype, const GemmArgs& ce, const GemmArgs& dh, hipStream_t st);
// thread-local timing events of the MMQ launches (nullptr: off)
void set_profile_events(hipEvent_t start, hipEvent_t stop);
hipEvent_t profile_event(int stop);

// Every MMQ kernel is launched through this: with the thread's timing events
// set, through hipExtLaunchKernelGGL, whose dispatch itself stamps `start`
// when the kernel begins and `stop` when it ends (no queue time between an
// event and the kernel); a plain launch otherwise.
template <typename F, typename... Args>
inline void mmq_launch(F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  const hipEvent_t a = profile_event(0), b = profile_event(1);
  if (a && b)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// ---- small kernels (gq_small.hip) ----
hipError_t launch_dequant(int qtype, const void* blocks, int64_t rows, int64_t cols,
                          int out_bf16, void* out, hipStream_t st);

// Up to three tile prefixes in one launch (ts1 / ts2 nullable):
// ts_q[e] = sum_{e' < e} ceil(cnt(e') / bm_q), E + 1 entries.  The offsets
// are checked (offsets[0] == 0, non-decreasing, offsets[E] == M): invalid
// ones set *err (nullable) to 1 and every prefix to zero, valid ones *err = 0.
// With spill > 0 and ts_sp non-null, an expert whose rows leave a remainder
// rem = cnt mod bm0 of 1..spill rows (spill_whole: an expert of 1..spill rows
// in all) counts only its full bm0-row tiles in ts0 and ceil(rem / spill)
// tiles of `spill` rows in ts_sp (others: 0).
hipError_t launch_tile_starts(const int32_t* offsets, int32_t E, int64_t M, int32_t* err,
                              int32_t bm0, int32_t* ts0, int32_t bm1, int32_t* ts1, int32_t bm2,
                              int32_t* ts2, hipStream_t st, int32_t spill = 0,
                              int32_t* ts_sp = nullptr, bool spill_whole = false);

// out[p][j] = sum_c act(p)[c] * W(e)[j][c]   (W [r][C] if w_jstride == C, or
// [C][r] if w_jstride == 1, w_cstride == r); act rows via gather; e via offsets.
// out2 (optional): out2[p][j] = wflat[sorted[p]] * out[p][j]
// wout (optional): wout[p][j] = wflat[sorted[p]] * win[p][j] over the same rows
struct RowDotArgs {
  int64_t M;
  int32_t C;
  int32_t r;
  const uint16_t* act;
  int64_t lda;
  const int32_t* gather;
  int32_t gdiv;
  const int32_t* offsets;
  int32_t E;
  const int32_t* tile16;  // grouped: prefix of 16-row tiles per expert (launch_tile_starts)
  const float* W[2];
  int64_t w_estride;
  int64_t w_jstride;
  int64_t w_cstride;
  float* out[2];
  int32_t nout;
  float* out2;  // weighted copy of out[0]
  const float* wflat;
  const int32_t* sorted;
  const float* win;  // optional side job: wout[p][j] = wflat[sorted[p]] * win[p][j]
  float* wout;       // over the same rows (needs wflat, sorted)
  // dense only (no tile16, out2, wout): the columns are cut into csplit
  // ranges, one workgroup each, and range s writes its partial sums to
  // out[o] + s * M * r (the consumer adds the csplit partials); 0 or 1 = no cut
  int32_t csplit;
};
// Column ranges for a dense row-dot: enough workgroups to give every CU one
// (at most 4 ranges, each at least 768 columns).
int rowdot_csplit(int64_t M, int64_t C);
hipError_t launch_rowdot(const RowDotArgs& a, hipStream_t st);

// out[t][n] = bf16( sum_{s < ksplit} part[s][t][n] + scale * sum_{j < r} X[t][j] * Y[n*ys_n + j*ys_j] )
// for t < M, n < N (N even, out 4-byte aligned).
hipError_t launch_split_fixup(const float* part, int ksplit, int64_t M, int32_t N, const float* X, int32_t r,
                              const float* Y, int64_t ys_n, int64_t ys_j, float scale, uint16_t* out,
                              int64_t ldo, hipStream_t st);

// Partial outer-product reductions over row chunks:
//   part[slot][c][j] = sum_{rows p of slot} U(p)[c] * Vv[p][j]
// slots: chunks of `rc` rows within each expert (chunk_start from
// launch_tile_starts with bm = rc).  U rows via gather.
struct ColRedArgs {
  int64_t M;
  int32_t C;
  int32_t r;
  const uint16_t* U;
  int64_t ldu;
  const int32_t* gather;
  int32_t gdiv;
  const float* Vv;
  const int32_t* offsets;   // nullptr = dense
  const int32_t* chunk_start;
  int32_t E;
  int32_t rc;
  int32_t slots;
  float* part;              // [slots][C][r]
  // optional second rank-vector array over the same U (one pass, two
  // partial sets); only with njobs <= 1
  const float* Vv2;
  float* part2;
  // optional second independent reduction in the same launch (blockIdx.z
  // == 1) over the same rows and slots: its own U, C, gather and V
  int32_t njobs;            // 0 or 1: one job
  int32_t C_1;
  const uint16_t* U_1;
  int64_t ldu_1;
  const int32_t* gather_1;
  int32_t gdiv_1;
  const float* Vv_1;
  float* part_1;
  // job 1's rank vectors as vsplit_1 partial arrays (Vv_1 + s * M * r) that
  // are summed on load (0 or 1: one array); with vfinal_1, workgroups of
  // column block 0 also store that sum for their rows (vfinal_1[p][j])
  int32_t vsplit_1;
  float* vfinal_1;
  // optional side job over the same slots (workgroups of column block 0,
  // job 0): the row sums of the grouped down MMQ's per-n-tile partials
  // (dfin_part [ntiles][M][1 + 2r] -> dw_flat[sorted[p]], dgB[p], duB[p])
  const float* dfin_part;
  int32_t dfin_ntiles;
  const int32_t* dfin_sorted;
  float* dfin_dw;
  float* dfin_dgB;
  float* dfin_duB;
};
hipError_t launch_colred(const ColRedArgs& a, hipStream_t st);
// columns covered by one launch_colred workgroup
int colred_cols_per_block(int r);

// Up to four grouped finishes in one launch (blockIdx.z = job): out[j] =
// s * sum over an expert's slots (in order) of part[j], as
// launch_colred_finish with chunk_start.
struct ColFinJobs {
  int32_t n;
  const float* part[4];
  float* out[4];
  int32_t C[4];
  int32_t transpose[4];
};
hipError_t launch_colred_finish_grp(const ColFinJobs& j, const int32_t* chunk_start, int32_t E,
                                    int32_t r, float s, hipStream_t st);
// Up to four dense finishes (one group of nslots slots) in one launch.
hipError_t launch_colred_finish_dense(const ColFinJobs& j, int32_t nslots, int32_t r, float s,
                                      hipStream_t st);

// out = s * sum over an expert's slots (in order) of part; experts with no
// rows get zeros.  transpose: out[e][j][c] instead of out[e][c][j].
// chunk_start == nullptr: one dense group of nslots_dense slots.
hipError_t launch_colred_finish(const float* part, const int32_t* chunk_start, int32_t E,
                                int32_t nslots_dense, int32_t C, int32_t r, float s,
                                int transpose, float* out, hipStream_t st);

// out[i][j] = sum_{t < nparts} part[t][i][j] (fixed order); i < rows, j < width
hipError_t launch_sum_parts(const float* part, int32_t nparts, int64_t rows, int32_t width,
                            float scale, float* out, hipStream_t st);

// routing
hipError_t launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                        float* w, int32_t* sorted, int32_t* offsets, int32_t* pos, void* ws,
                        hipStream_t st);
size_t route_ws_bytes(int64_t T, int32_t E, int32_t k);
hipError_t launch_route_bwd(const int32_t* ids, const float* w, const float* dw, int64_t T,
                            int32_t E, int32_t k, float* dlogits, hipStream_t st);
hipError_t launch_combine(const uint16_t* rows, const float* w, const int32_t* pos, int64_t T,
                          int32_t k, int64_t H, uint16_t* out, hipStream_t st);

// MoE down-backward partial finish: from part [ntiles][M][1 + 2r]
//   dw_flat[sorted[p]] = sum part[.][p][0]; dgB[p][j] = sum part[.][p][1+j];
//   duB[p][j] = sum part[.][p][1+r+j]

// LM head helpers
// term: [T] scratch for the per-token loss terms.  Also writes nvalid (the
// number of labels in [0, V)), err (1 if a label is neither valid nor the
// ignore index) and the loss; lse and the gradient passes read nothing else.
hipError_t launch_ce_merge(const float* part_ml, int32_t ntiles, int64_t T, const float* zlab,
                           const int64_t* labels, int64_t V, int64_t ignore_index, float* lse,
                           float* term, int32_t* err, float* nvalid, float* loss,
                           hipStream_t st);
// AdamW step with 8-bit block-wise states (blocks of 256 elements)
hipError_t launch_adamw8bit(float* p, const float* g, uint8_t* mq, uint8_t* vq, float* sm, float* sv,
                            int64_t n, int64_t t, float lr, float beta1, float beta2, float eps,
                            float wd, hipStream_t st);
// RMS normalisation (y = x rstd w) and its input gradient; H % 8 == 0
hipError_t launch_rmsnorm_fwd(const uint16_t* x, const float* w, int64_t T, int32_t H, float eps,
                              uint16_t* y, float* rstd, hipStream_t st);
hipError_t launch_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const float* w,
                              const float* rstd, int64_t T, int32_t H, uint16_t* dx,
                              hipStream_t st);
// dh[t][c] = bf16( sum_{q < nacc} dh_acc[q][t][c] (in order) + s * sum_j GB[t][j] A[j][c] )
hipError_t launch_ce_final_dh(const float* dh_acc, int32_t nacc, const float* GB, const float* A, int64_t T,
                              int32_t H, int32_t r, float s, uint16_t* dh, hipStream_t st);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
hipError_t launch_fill_u16(uint16_t* p, int64_t n, uint16_t v, hipStream_t st);

}  // namespace gq
