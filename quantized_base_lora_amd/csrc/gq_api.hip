// C ABI of libgq: argument validation (before any HIP call), workspace
// planning and launch sequencing.  Every step of the computation runs in the
// HIP kernels of gq_gemm.hip / gq_small.hip on the caller's stream.
#include <dlfcn.h>
#include <limits.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/gq.h"
#include "gq_internal.h"

using namespace gq;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                  \
  do {                                       \
    hipError_t _e = (expr);                  \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// Environment switches, read once per process:
//   GQ_TRACE=1  each entry point runs inside a roctx range named after it
//               (visible to rocprofv3 --marker-trace); GQ_TRACE=2 also
//               prints one line per call (name, status, error text) to
//               stderr.
//   GQ_DEBUG=1  after an entry point has queued its work, synchronise its
//               stream and turn an asynchronous HIP error, or a nonzero
//               device error word, into the call's own return code
//               (GQ_EHIP / GQ_EDEVICE) instead of leaving it for the caller
//               to find.  This serialises the caller with the GPU: a
//               debugging aid, never for timing.
struct Switches {
  int trace = 0;
  bool debug = false;
};

const Switches& switches() {
  static const Switches s = [] {
    Switches v;
    if (const char* t = getenv("GQ_TRACE")) v.trace = atoi(t);
    if (const char* d = getenv("GQ_DEBUG")) v.debug = atoi(d) != 0;
    return v;
  }();
  return s;
}

// roctx is looked up at run time so that the library has no link-time
// dependency on the tracer; without it the ranges are simply not emitted.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx v;
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so", "libroctx64.so.4",
                            "libroctx64.so"}) {
      void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (!h) continue;
      v.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
      v.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
      if (v.push && v.pop) break;
      v.push = nullptr;
      v.pop = nullptr;
    }
    return v;
  }();
  return r;
}

int debug_check(const char* name, void* stream, const void* err_word) {
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(GQ_EHIP, "%s (GQ_DEBUG): %s", name, hipGetErrorString(e));
  if (err_word) {
    int32_t w = 0;
    e = hipMemcpy(&w, err_word, sizeof w, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(GQ_EHIP, "%s (GQ_DEBUG): reading the error word: %s", name, hipGetErrorString(e));
    if (w != 0) return fail(GQ_EDEVICE, "%s (GQ_DEBUG): device error word %d", name, (int)w);
  }
  return GQ_OK;
}

// Runs one entry point's body under the GQ_TRACE / GQ_DEBUG switches;
// err_word is the workspace word the body's kernels report data errors in
// (nullptr for entry points without one).
template <class Body>
int traced_call(const char* name, void* stream, const void* err_word, Body&& body) {
  const Switches& sw = switches();
  if (!sw.trace && !sw.debug) return body();
  const Roctx& rx = roctx();
  if (sw.trace && rx.push) rx.push(name);
  int rc = body();
  if (rc == GQ_OK && sw.debug) rc = debug_check(name, stream, err_word);
  if (sw.trace && rx.pop) rx.pop();
  if (sw.trace >= 2)
    fprintf(stderr, "[gq] %s -> %d%s%s\n", name, rc, rc ? ": " : "", rc ? g_err.c_str() : "");
  return rc;
}

int64_t block_bytes(int qtype) {
  switch (qtype) {
    case GQ_Q8_0: return 34;
    case GQ_Q4_0: return 18;
    case GQ_Q2_DM: return 12;
    default: return -1;
  }
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Alignment check of one (non-NULL) array argument, naming it in the error.
#define REQ_ALIGN(ptr, a, fn)                                                             \
  do {                                                                                    \
    if ((ptr) && !aligned((ptr), (a)))                                                    \
      return fail(GQ_EINVAL, "%s: %s must be %d-byte aligned", (fn), #ptr, (int)(a));     \
  } while (0)

// Bump allocator over the caller's workspace (256-byte aligned pieces).
// With base == nullptr it only measures.
struct Ws {
  uint8_t* base;
  size_t off = 0;
  explicit Ws(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <class T>
  T* take(int64_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)count * sizeof(T);
    return p;
  }
  size_t size() const { return (off + 255) & ~(size_t)255; }
};

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return GQ_OK;
  if (!ws) return fail(GQ_EWORKSPACE, "workspace is NULL but %zu bytes are required", need);
  if (!aligned(ws, 256)) return fail(GQ_EINVAL, "workspace must be 256-byte aligned");
  if (have < need)
    return fail(GQ_EWORKSPACE, "workspace too small: %zu bytes given, %zu required", have, need);
  return GQ_OK;
}

// out8: the layer's backward reads activation rows of n_out bf16 with
// 16-byte loads (not the LM head: its vocabulary rows are only walked by
// masked tiles and a padded gradient chunk)
int check_proj(const gq_lora_linear* L, const char* name, bool grouped, bool out8 = true) {
  if (!L) return fail(GQ_EINVAL, "%s: NULL projection", name);
  if (block_bytes(L->qtype) < 0) return fail(GQ_EINVAL, "%s: unknown qtype %d", name, L->qtype);
  if (L->rank < 1 || L->rank > 16) return fail(GQ_EINVAL, "%s: rank %d not in [1, 16]", name, L->rank);
  if (L->n_in < 32 || L->n_in % 32)
    return fail(GQ_ENOTSUP, "%s: n_in %lld must be a positive multiple of 32", name,
                (long long)L->n_in);
  if (L->n_out < 1 || (out8 && (L->n_out < 8 || L->n_out % 8)))
    return fail(GQ_ENOTSUP, "%s: n_out %lld must be a positive multiple of 8", name,
                (long long)L->n_out);
  if (L->n_in > INT_MAX / 2 || L->n_out > INT_MAX / 2)
    return fail(GQ_ENOTSUP, "%s: dimension too large", name);
  if (!grouped && L->n_experts != 1)
    return fail(GQ_EINVAL, "%s: n_experts must be 1 here (got %d)", name, L->n_experts);
  if (L->n_experts < 1 || L->n_experts > 1024)
    return fail(GQ_EINVAL, "%s: n_experts %d not in [1, 1024]", name, L->n_experts);
  if (!L->w_blocks || !L->A || !L->B) return fail(GQ_EINVAL, "%s: NULL weight or adapter", name);
  REQ_ALIGN(L->w_blocks, 4, name);
  REQ_ALIGN(L->A, 16, name);
  REQ_ALIGN(L->B, 16, name);
  return GQ_OK;
}

int64_t rowbytes(const gq_lora_linear* L) { return (L->n_in / 32) * block_bytes(L->qtype); }
int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// tile configuration: 128-row tiles unless that leaves the chip underfilled
// 128x128 tiles decode each weight tile for twice the rows of 64x128 ones
// and run faster per flop even at one workgroup per CU; halve the rows only
// when 128-row tiles would leave most of the 256 CUs idle.
// A launch of at most one 128x128 tile per CU with a long reduction runs each
// tile on eight waves (two k-groups), which keeps two waves per SIMD busy;
// `k2ok` marks the epilogues that allow it.
int pick_tile(int64_t rows_est, int64_t ntiles, int64_t K = 0, bool k2ok = false) {
  const int64_t t128 = (int64_t)cdiv(rows_est, 128) * ntiles;
  if (k2ok && t128 <= 256 && K >= 1024) return TILE_128x128_K2;
  return t128 < 192 ? TILE_64x128 : TILE_128x128;
}

GemmArgs gemm_defaults() {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.asplit = INT_MAX;
  a.wsplit = INT_MAX;
  a.gdiv = 1;
  a.E = 1;
  return a;
}

// Rows per chunk of the adapter-gradient column reductions: the largest
// power of two (32..1024) that still gives >= 256 workgroups, so that the
// reduction fills the chip without multiplying the partial-sum traffic
// (C x r floats per chunk, written and read once more by the finish).
int pick_rc(int64_t M, int64_t C, int r, int E) {
  // grouped: per-expert chunks of 256 rows -- most experts are one chunk
  // (one partial set each), the Zipf head experts are still split
  if (E > 1) return 256;
  const int64_t cb = cdiv(C, colred_cols_per_block(r));
  int rc = 32;
  while (rc < 1024 && cdiv(M, rc * 2) * cb >= 256) rc *= 2;
  return rc;
}
// Forward launches with few rows per weight row run the skinny MMQ (each
// block streamed once per 16/32/64-row tile with coalesced loads), when its
// layout conditions hold: K a multiple of 256 (whole 8-block segments) and
// 16-byte aligned weights.  rows_per_w = rows sharing one weight (tokens, or
// routed rows per expert on average).
int pick_fwd_tile(int64_t rows_per_w, int64_t rows_est, int64_t ntiles128, int64_t K,
                  bool w_aligned, bool k2ok = false) {
  if (K % 256 == 0 && w_aligned) {
    if (rows_per_w <= 16) return TILE_SKINNY16;
    if (rows_per_w <= 32) return TILE_SKINNY32;
    if (rows_per_w <= 64) return TILE_SKINNY64;
  }
  return pick_tile(rows_est, ntiles128, K, k2ok);
}

// Grouped launches: an expert's rows fill ceil(rows / BM) m-tiles.  With at
// most 64 rows per expert on average, 64-row tiles waste less padding; at
// 128 rows per expert the 128-row tiles measured faster despite it.
int pick_grp_tile(int64_t M, int E, int64_t ntiles) {
  if (M <= (int64_t)E * 64) return TILE_64x128;
  return pick_tile(M, ntiles);
}

// Backward (NN) launches with few rows per weight run the skinny NN MMQ
// (16 or 32 rows per tile, 128 output columns per workgroup) when the
// output row length is a multiple of 128 (whole 4-block segments) and the
// weights are 16-byte aligned.
int pick_nn_tile(int64_t rows_per_w, int64_t rows_est, int64_t ntiles128, int64_t Nout,
                 bool w_aligned, int64_t Kred, bool k2ok = false) {
  if (Nout % 128 == 0 && w_aligned) {
    if (rows_per_w <= 16) return TILE_SKINNY16;
    if (rows_per_w <= 32) return TILE_SKINNY32;
  }
  return pick_tile(rows_est, ntiles128, Kred, k2ok);
}
int nn_tile_bn(int tc) { (void)tc; return TILE_BN; }  // 128 for the tile and the skinny NN MMQ

// Grouped tile launches: an expert's last few rows past its full tiles (a
// nearly empty tile that still decodes the expert's whole weight slice) run
// on a second, skinny launch, which streams each such slice once.  Forward:
// remainders of up to 32 rows.  Backward (NN): only experts of at most 8 rows
// in all, and only beside 128-row tiles -- the skinny NN MMQ is VALU-bound on
// its decode and gets few workgroups from a handful of remainders (measured
// slower than the tiles it saves), and beside 64-row tiles (few rows per
// expert) spilling measured slower too.  Needs the
// skinny layout: reduction a multiple of 256 (forward) / output row a
// multiple of 128 (backward), 16-byte aligned weights.  Returns the spill
// threshold in rows, 0 = no spill launch.
int spill_rows(int tc, int E, bool nn, int64_t kdim_or_nout, bool w_aligned) {
  if (tile_skinny(tc) || E < 2 || !w_aligned) return 0;
  if (nn) return kdim_or_nout % 128 == 0 && tile_bm(tc) == 128 ? 8 : 0;
  return kdim_or_nout % 256 == 0 ? 32 : 0;
}
int spill_tile(int rows) { return rows <= 16 ? TILE_SKINNY16 : TILE_SKINNY32; }

int64_t colred_slots(int64_t M, int rc, int E) { return cdiv(M, rc) + (E > 1 ? E : 0); }

// Dense forward launches with Q8_0 / Q4_0 weights and K % 64 == 0 run the
// 256 x 192 wide tiles when those fill the chip: their rows at least three
// quarters used (clamped rows cost as much as real ones), at least 192
// tiles, and the last round of one tile per CU at least three quarters full.
bool wide_pays(int qtype, int64_t M, int64_t N, int64_t K, int r) {
  if (qtype == GQ_Q2_DM || K % GEMM_BK || r > WIDE_MAX_RANK) return false;
  if (M * 4 < (int64_t)cdiv(M, WIDE_BM) * WIDE_BM * 3) return false;
  const int64_t tiles = (int64_t)cdiv(M, WIDE_BM) * cdiv(N, WIDE_BN);
  if (tiles < 192) return false;
  const int64_t rounds = (tiles + 255) / 256;
  return tiles * 4 >= rounds * 256 * 3;
}

// Split-K for small dense launches: when even 64-row tiles leave most CUs
// idle, each tile's reduction is cut into ksplit contiguous ranges (at least
// two k-steps each), one workgroup per range writing fp32 sums that a fixup
// pass adds up with the adapter term.  1 = no split.
int small_split(int64_t M, int64_t N, int64_t K) {
  if (K % GEMM_BK || N % 8) return 1;
  const int64_t tiles = (int64_t)cdiv(M, 64) * cdiv(N, TILE_BN);
  const int64_t nk = K / GEMM_BK;
  if (tiles * 4 > 256 || nk < 4) return 1;
  const int64_t ks = std::min<int64_t>(256 / tiles, nk / 2);
  return ks > 1 ? (int)ks : 1;
}

hipStream_t S(void* st) { return static_cast<hipStream_t>(st); }

}  // namespace

extern "C" {

int gq_version(void) { return 100; }

const char* gq_last_error(void) { return g_err.c_str(); }

int64_t gq_block_bytes(int qtype) { return block_bytes(qtype); }

void gq_profile_mmq_events(void* start, void* stop) {
  set_profile_events(static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
}

// ------------------------------------------------------------------ dequant
static int dequant_impl(int qtype, const void* blocks, int64_t rows, int64_t cols, int out_dtype, void* out,
               void* stream) {
  g_err.clear();
  if (block_bytes(qtype) < 0) return fail(GQ_EINVAL, "gq_dequant: unknown qtype %d", qtype);
  if (rows < 0 || cols <= 0 || cols % 32)
    return fail(GQ_EINVAL, "gq_dequant: rows >= 0 and cols a positive multiple of 32 required");
  if (out_dtype != GQ_F32 && out_dtype != GQ_BF16)
    return fail(GQ_EINVAL, "gq_dequant: unknown out_dtype %d", out_dtype);
  if (rows == 0) return GQ_OK;
  if (!blocks || !out) return fail(GQ_EINVAL, "gq_dequant: NULL pointer");
  REQ_ALIGN(blocks, 2, "gq_dequant");
  REQ_ALIGN(out, 16, "gq_dequant");
  HIP_TRY(launch_dequant(qtype, blocks, rows, cols, out_dtype == GQ_BF16, out, S(stream)),
          "gq_dequant");
  return GQ_OK;
}

// ------------------------------------------------------------------- linear
size_t gq_linear_lora_fwd_workspace_size(const gq_lora_linear* L, int64_t T) {
  if (!L || T <= 0 || L->n_in <= 0 || L->n_out <= 0) return 0;
  const int ks = small_split(T, L->n_out, L->n_in);
  const int cs = rowdot_csplit(T, L->n_in);
  if (ks <= 1 && cs <= 1) return 0;
  Ws w(nullptr);
  if (ks > 1) w.take<float>((int64_t)ks * T * L->n_out);
  if (cs > 1) w.take<float>((int64_t)cs * T * L->rank);
  return w.size();
}

static int linear_lora_fwd_impl(const gq_lora_linear* L, const uint16_t* x, int64_t T, uint16_t* y,
                       float* xa, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_proj(L, "gq_linear_lora_fwd", false);
  if (rc) return rc;
  if (T < 0 || T > INT_MAX) return fail(GQ_EINVAL, "gq_linear_lora_fwd: bad T %lld", (long long)T);
  if (T == 0) return GQ_OK;
  if (!x || !y || !xa) return fail(GQ_EINVAL, "gq_linear_lora_fwd: NULL x, y or xa");
  REQ_ALIGN(x, 16, "gq_linear_lora_fwd");
  REQ_ALIGN(y, 2, "gq_linear_lora_fwd");
  REQ_ALIGN(xa, 4, "gq_linear_lora_fwd");
  const hipStream_t st = S(stream);
  const int r = L->rank, K = (int)L->n_in, N = (int)L->n_out;

  GemmArgs g = gemm_defaults();
  g.M = T; g.N = N; g.K = K;
  g.a0 = x; g.lda = K;
  g.w0 = static_cast<const uint8_t*>(L->w_blocks);
  g.w_rowbytes = rowbytes(L); g.w_nb = K / 32; g.w_rows = N;
  g.ntiles = cdiv(N, TILE_BN);
  int tc = pick_fwd_tile(T, T, g.ntiles, K, aligned(L->w_blocks, 16), true);
  if (!tile_skinny(tc) && wide_pays(L->qtype, T, N, K, L->rank)) {
    tc = TILE_WIDE;
    g.ntiles = cdiv(N, WIDE_BN);
  }
  // small launches: split the reduction (needs the workspace and 4-byte
  // aligned y for the fixup's stores; else the unsplit tile)
  const int ks = (tile_skinny(tc) || tc == TILE_WIDE || !aligned(y, 4)) ? 1 : small_split(T, N, K);
  Ws w(ws);
  if (ks > 1) {
    if ((rc = check_ws(ws, ws_bytes, gq_linear_lora_fwd_workspace_size(L, T)))) return rc;
    tc = TILE_64x128;
    g.ksplit = ks;
    g.part = w.take<float>((int64_t)ks * T * N);
  }
  g.mtiles = cdiv(T, tile_bm(tc));
  g.s = L->scale; g.r = r; g.lB0 = L->B; g.rv0 = xa;
  g.o0 = y; g.ldo = N;
  // x A^T over column ranges when 16-row workgroups alone leave CUs idle
  // (tile launches only, and only with the workspace for the partials): the
  // MMQ's adapter fold adds them and stores xa
  int cs = (tile_skinny(tc) || ks > 1) ? 1 : rowdot_csplit(T, K);
  float* xa_part = nullptr;
  if (cs > 1) {
    const size_t need = gq_linear_lora_fwd_workspace_size(L, T);
    if (ws && ws_bytes >= need) {
      xa_part = w.take<float>((int64_t)cs * T * r);
      g.rv0 = xa_part; g.rv_parts = cs; g.rv_out = xa;
    } else {
      cs = 1;
    }
  }

  RowDotArgs rd;
  memset(&rd, 0, sizeof rd);
  rd.M = T; rd.C = K; rd.r = r; rd.act = x; rd.lda = K; rd.gdiv = 1; rd.E = 1;
  rd.W[0] = L->A; rd.w_jstride = K; rd.w_cstride = 1; rd.nout = 1;
  rd.out[0] = cs > 1 ? xa_part : xa; rd.csplit = cs;
  HIP_TRY(launch_rowdot(rd, st), "gq_linear_lora_fwd: x A^T");
  HIP_TRY(launch_gemm(L->qtype, EPI_LIN, tc, g, st), "gq_linear_lora_fwd: MMQ");
  if (ks > 1)
    HIP_TRY(launch_split_fixup(g.part, ks, T, N, xa, r, L->B, r, 1, L->scale, y, N, st),
            "gq_linear_lora_fwd: split sums");
  return GQ_OK;
}

namespace {
struct LinBwdWs {
  float* dyB;
  float* dyB_part;  // column-range partials of dY B when the row-dot is cut (else nullptr)
  float* part_dB;
  float* part_dA;
  float* part_dx;  // split-K sums of a small dX launch (else nullptr)
  int ks_dx;
  int cs_dyB;      // column ranges of the dY B row-dot (1 = one)
};
int lin_rc(const gq_lora_linear* L, int64_t T) {
  return pick_rc(T, L->n_in > L->n_out ? L->n_in : L->n_out, L->rank, 1);
}
LinBwdWs plan_lin_bwd(Ws& w, const gq_lora_linear* L, int64_t T) {
  LinBwdWs p;
  const int64_t slots = colred_slots(T, lin_rc(L, T), 1);
  p.dyB = w.take<float>(T * L->rank);
  // dY B over column ranges when 16-row workgroups alone leave CUs idle;
  // the dX MMQ's adapter fold (tile path, unsplit) or else the dB / dA
  // reduction adds the partials and stores dY B for the other
  p.cs_dyB = rowdot_csplit(T, L->n_out);
  p.dyB_part = p.cs_dyB > 1 ? w.take<float>((int64_t)p.cs_dyB * T * L->rank) : nullptr;
  p.part_dB = w.take<float>(slots * L->n_out * L->rank);
  p.part_dA = w.take<float>(slots * L->n_in * L->rank);
  p.ks_dx = small_split(T, L->n_in, L->n_out);
  p.part_dx = p.ks_dx > 1 ? w.take<float>((int64_t)p.ks_dx * T * L->n_in) : nullptr;
  return p;
}
}  // namespace

size_t gq_linear_lora_bwd_workspace_size(const gq_lora_linear* L, int64_t T) {
  if (!L || T <= 0 || L->rank < 1 || L->rank > 16) return 0;
  Ws w(nullptr);
  plan_lin_bwd(w, L, T);
  return w.size();
}

static int linear_lora_bwd_impl(const gq_lora_linear* L, const uint16_t* x, const float* xa,
                       const uint16_t* dy, int64_t T, uint16_t* dx, float* dA, float* dB, void* ws,
                       size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_proj(L, "gq_linear_lora_bwd", false);
  if (rc) return rc;
  if (T < 0 || T > INT_MAX) return fail(GQ_EINVAL, "gq_linear_lora_bwd: bad T %lld", (long long)T);
  if (!dA || !dB) return fail(GQ_EINVAL, "gq_linear_lora_bwd: NULL dA or dB");
  const hipStream_t st = S(stream);
  const int r = L->rank, K = (int)L->n_in, N = (int)L->n_out;
  REQ_ALIGN(dA, 4, "gq_linear_lora_bwd");
  REQ_ALIGN(dB, 4, "gq_linear_lora_bwd");
  if (T == 0) {
    HIP_TRY(launch_fill_f32(dA, (int64_t)r * K, 0.f, st), "gq_linear_lora_bwd: zero dA");
    HIP_TRY(launch_fill_f32(dB, (int64_t)N * r, 0.f, st), "gq_linear_lora_bwd: zero dB");
    return GQ_OK;
  }
  if (!x || !xa || !dy) return fail(GQ_EINVAL, "gq_linear_lora_bwd: NULL x, xa or dy");
  REQ_ALIGN(x, 16, "gq_linear_lora_bwd");
  REQ_ALIGN(dy, 16, "gq_linear_lora_bwd");
  REQ_ALIGN(dx, 2, "gq_linear_lora_bwd");
  REQ_ALIGN(xa, 4, "gq_linear_lora_bwd");
  REQ_ALIGN(dA, 4, "gq_linear_lora_bwd");
  REQ_ALIGN(dB, 4, "gq_linear_lora_bwd");
  Ws meas(nullptr);
  plan_lin_bwd(meas, L, T);
  if ((rc = check_ws(ws, ws_bytes, meas.size()))) return rc;
  Ws w(ws);
  const LinBwdWs P = plan_lin_bwd(w, L, T);
  const int rcl = lin_rc(L, T);
  const int slots = (int)colred_slots(T, rcl, 1);

  RowDotArgs rd;
  memset(&rd, 0, sizeof rd);
  rd.M = T; rd.C = N; rd.r = r; rd.act = dy; rd.lda = N; rd.gdiv = 1; rd.E = 1;
  rd.W[0] = L->B; rd.w_jstride = 1; rd.w_cstride = r; rd.nout = 1;
  rd.out[0] = P.cs_dyB > 1 ? P.dyB_part : P.dyB; rd.csplit = P.cs_dyB;
  HIP_TRY(launch_rowdot(rd, st), "gq_linear_lora_bwd: dY B");

  // dX MMQ.  With dY B as column-range partials, the tile path's adapter
  // fold adds them and stores dY B, and runs before the dB / dA reductions;
  // otherwise (split or skinny launches, or no dx) the reductions do.
  const int tc0 = pick_nn_tile(T, T, cdiv(K, TILE_BN), K, aligned(L->w_blocks, 16), N, true);
  const bool split = dx && P.ks_dx > 1 && !tile_skinny(tc0) && aligned(dx, 4);
  const bool fold_sums = dx && P.cs_dyB > 1 && !split && !tile_skinny(tc0);
  auto launch_dx = [&]() -> int {
    GemmArgs g = gemm_defaults();
    g.M = T; g.N = K; g.K = N;
    g.a0 = dy; g.lda = N;
    g.w0 = static_cast<const uint8_t*>(L->w_blocks);
    g.w_rowbytes = rowbytes(L); g.w_nb = K / 32; g.w_rows = N;
    int tc = tc0;
    if (split) {
      tc = TILE_64x128;
      g.ksplit = P.ks_dx;
      g.part = P.part_dx;
    }
    g.ntiles = cdiv(K, nn_tile_bn(tc));
    g.mtiles = cdiv(T, tile_bm(tc));
    g.s = L->scale; g.r = r; g.lA0 = L->A; g.rv0 = P.dyB;
    if (fold_sums) {
      g.rv0 = P.dyB_part; g.rv_parts = P.cs_dyB; g.rv_out = P.dyB;
    }
    g.o0 = dx; g.ldo = K;
    HIP_TRY(launch_gemm(L->qtype, EPI_LIN_BWD, tc, g, st), "gq_linear_lora_bwd: dX MMQ");
    if (split)  // adapter term s (dY B) A: A is [r][n_in]
      HIP_TRY(launch_split_fixup(P.part_dx, P.ks_dx, T, K, P.dyB, r, L->A, 1, K, L->scale, dx, K, st),
              "gq_linear_lora_bwd: dX split sums");
    return GQ_OK;
  };
  if (fold_sums && (rc = launch_dx())) return rc;

  // dB = s dY^T xa and dA = s (dY B)^T x: both reductions in one launch,
  // both finishes in one launch
  ColRedArgs cr;
  memset(&cr, 0, sizeof cr);
  cr.M = T; cr.C = N; cr.r = r; cr.U = dy; cr.ldu = N; cr.gdiv = 1; cr.Vv = xa;
  cr.E = 1; cr.rc = rcl; cr.slots = slots; cr.part = P.part_dB;
  cr.njobs = 2;
  cr.C_1 = K; cr.U_1 = x; cr.ldu_1 = K; cr.gdiv_1 = 1; cr.part_1 = P.part_dA;
  if (P.cs_dyB > 1 && !fold_sums) {  // the partials summed here, dY B stored for the dX MMQ
    cr.Vv_1 = P.dyB_part; cr.vsplit_1 = P.cs_dyB; cr.vfinal_1 = P.dyB;
  } else {
    cr.Vv_1 = P.dyB;
  }
  HIP_TRY(launch_colred(cr, st), "gq_linear_lora_bwd: dB, dA partials");
  ColFinJobs fj;
  memset(&fj, 0, sizeof fj);
  fj.n = 2;
  fj.part[0] = P.part_dB; fj.out[0] = dB; fj.C[0] = N; fj.transpose[0] = 0;
  fj.part[1] = P.part_dA; fj.out[1] = dA; fj.C[1] = K; fj.transpose[1] = 1;
  HIP_TRY(launch_colred_finish_dense(fj, slots, r, L->scale, st), "gq_linear_lora_bwd: dB, dA");

  if (dx && !fold_sums && (rc = launch_dx())) return rc;
  return GQ_OK;
}

// ------------------------------------------------ linear backward, no allocation
}  // extern "C"

namespace {
// Scratch of gq_linear_lora_bwd_noalloc: a file-scope device array (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// never passes `scratch` itself to a kernel -- in host code that name is a
// stand-in, not a device address; the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)GQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// device address of this device's scratch array (the current device must be
// the one the stream belongs to)
int scratch_for_current_device(void** out, const char* name) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, name);
  if (dev < 0 || dev >= kMaxDevices) return fail(GQ_ENOTSUP, "%s: device %d beyond %d", name, dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], name);
  *out = g_scratch_ptr[dev];
  return GQ_OK;
}
}  // namespace

extern "C" {

size_t gq_noalloc_scratch_bytes(void) { return kScratchBytes; }

static int linear_lora_bwd_noalloc_impl(const gq_lora_linear* L, const uint16_t* x, const float* xa,
                               const uint16_t* dy, int64_t T, uint16_t* dx, float* dA, float* dB,
                               void* stream) {
  g_err.clear();
  const char* name = "gq_linear_lora_bwd_noalloc";
  int rc = check_proj(L, name, false);
  if (rc) return rc;
  if (T < 0 || T > INT_MAX) return fail(GQ_EINVAL, "%s: bad T %lld", name, (long long)T);
  const size_t need = T > 0 ? gq_linear_lora_bwd_workspace_size(L, T) : 0;
  if (need > kScratchBytes)
    return fail(GQ_EWORKSPACE, "%s: needs %zu bytes of scratch, the fixed maximum is %zu", name, need,
                kScratchBytes);
  void* ws = nullptr;
  if (need > 0 && (rc = scratch_for_current_device(&ws, name))) return rc;
  // the same kernels as gq_linear_lora_bwd; every scratch word they read is
  // written earlier in the same call, so nothing needs clearing
  rc = gq_linear_lora_bwd(L, x, xa, dy, T, dx, dA, dB, ws, kScratchBytes, stream);
  if (rc) {
    std::string msg = g_err;
    return fail(rc, "%s", msg.c_str());
  }
  return GQ_OK;
}

// ------------------------------------------------------------------ routing
size_t gq_moe_route_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T <= 0 || E < 1 || k < 1) return 0;
  return (route_ws_bytes(T, E, k) + 255) & ~(size_t)255;
}

static int moe_route_impl(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                 int32_t* sorted, int32_t* offsets, int32_t* pos, void* ws, size_t ws_bytes,
                 void* stream) {
  g_err.clear();
  if (E < 1 || E > 1024) return fail(GQ_EINVAL, "gq_moe_route: E %d not in [1, 1024]", E);
  if (k < 1 || k > 16 || k > E) return fail(GQ_EINVAL, "gq_moe_route: k %d not in [1, min(E, 16)]", k);
  if (T < 0 || T * k > INT_MAX) return fail(GQ_EINVAL, "gq_moe_route: bad T %lld", (long long)T);
  if (!offsets) return fail(GQ_EINVAL, "gq_moe_route: NULL offsets");
  const hipStream_t st = S(stream);
  REQ_ALIGN(offsets, 4, "gq_moe_route");
  if (T == 0) {
    HIP_TRY(launch_fill_f32(reinterpret_cast<float*>(offsets), E + 1, 0.f, st), "gq_moe_route");
    return GQ_OK;
  }
  if (!logits || !ids || !w || !sorted || !pos) return fail(GQ_EINVAL, "gq_moe_route: NULL pointer");
  REQ_ALIGN(logits, 4, "gq_moe_route");
  REQ_ALIGN(ids, 4, "gq_moe_route");
  REQ_ALIGN(w, 4, "gq_moe_route");
  REQ_ALIGN(sorted, 4, "gq_moe_route");
  REQ_ALIGN(offsets, 4, "gq_moe_route");
  REQ_ALIGN(pos, 4, "gq_moe_route");
  int rc = check_ws(ws, ws_bytes, gq_moe_route_workspace_size(T, E, k));
  if (rc) return rc;
  HIP_TRY(launch_route(logits, T, E, k, ids, w, sorted, offsets, pos, ws, st), "gq_moe_route");
  return GQ_OK;
}

static int moe_route_bwd_impl(const int32_t* ids, const float* w, const float* dw, int64_t T, int32_t E,
                     int32_t k, float* dlogits, void* stream) {
  g_err.clear();
  if (E < 1 || E > 1024 || k < 1 || k > 16 || k > E)
    return fail(GQ_EINVAL, "gq_moe_route_bwd: bad E %d / k %d", E, k);
  if (T < 0) return fail(GQ_EINVAL, "gq_moe_route_bwd: bad T");
  if (T == 0) return GQ_OK;
  if (!ids || !w || !dw || !dlogits) return fail(GQ_EINVAL, "gq_moe_route_bwd: NULL pointer");
  REQ_ALIGN(ids, 4, "gq_moe_route_bwd");
  REQ_ALIGN(w, 4, "gq_moe_route_bwd");
  REQ_ALIGN(dw, 4, "gq_moe_route_bwd");
  REQ_ALIGN(dlogits, 4, "gq_moe_route_bwd");
  HIP_TRY(launch_route_bwd(ids, w, dw, T, E, k, dlogits, S(stream)), "gq_moe_route_bwd");
  return GQ_OK;
}

static int moe_combine_fwd_impl(const uint16_t* o, const float* w, const int32_t* pos, int64_t T, int32_t k,
                       int64_t H, uint16_t* y, void* stream) {
  g_err.clear();
  if (T < 0 || k < 1 || k > 16 || H < 8 || H % 8 || T * ((H + 2047) / 2048) > INT_MAX)
    return fail(GQ_EINVAL, "gq_moe_combine_fwd: bad T/k/H (H must be a multiple of 8)");
  if (T == 0) return GQ_OK;
  if (!o || !w || !pos || !y) return fail(GQ_EINVAL, "gq_moe_combine_fwd: NULL pointer");
  REQ_ALIGN(o, 16, "gq_moe_combine_fwd");
  REQ_ALIGN(y, 16, "gq_moe_combine_fwd");
  REQ_ALIGN(w, 4, "gq_moe_combine_fwd");
  REQ_ALIGN(pos, 4, "gq_moe_combine_fwd");
  HIP_TRY(launch_combine(o, w, pos, T, k, H, y, S(stream)), "gq_moe_combine_fwd");
  return GQ_OK;
}

static int adamw8bit_step_impl(float* p, const float* g, uint8_t* m_codes, uint8_t* v_codes, float* m_scale,
                      float* v_scale, int64_t n, int64_t step, float lr, float beta1, float beta2,
                      float eps, float weight_decay, void* stream) {
  g_err.clear();
  if (n < 0 || (n + 255) / 256 > INT_MAX) return fail(GQ_EINVAL, "gq_adamw8bit_step: bad n");
  if (step < 1) return fail(GQ_EINVAL, "gq_adamw8bit_step: step must be >= 1");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f) ||
      !(lr >= 0.f) || !(weight_decay >= 0.f))
    return fail(GQ_EINVAL, "gq_adamw8bit_step: need 0 <= beta < 1, eps > 0, lr >= 0, weight_decay >= 0");
  if (n == 0) return GQ_OK;
  if (!p || !g || !m_codes || !v_codes || !m_scale || !v_scale)
    return fail(GQ_EINVAL, "gq_adamw8bit_step: NULL pointer");
  REQ_ALIGN(p, 4, "gq_adamw8bit_step");
  REQ_ALIGN(g, 4, "gq_adamw8bit_step");
  REQ_ALIGN(m_scale, 4, "gq_adamw8bit_step");
  REQ_ALIGN(v_scale, 4, "gq_adamw8bit_step");
  HIP_TRY(launch_adamw8bit(p, g, m_codes, v_codes, m_scale, v_scale, n, step, lr, beta1, beta2, eps,
                           weight_decay, S(stream)),
          "gq_adamw8bit_step");
  return GQ_OK;
}

static int rmsnorm_fwd_impl(const uint16_t* x, const float* w, int64_t T, int64_t H, float eps, uint16_t* y,
                   float* rstd, void* stream) {
  g_err.clear();
  if (T < 0 || H < 8 || H % 8 || H > INT_MAX || (T + 3) / 4 > INT_MAX)
    return fail(GQ_EINVAL, "gq_rmsnorm_fwd: bad T/H (H must be a positive multiple of 8)");
  if (!(eps >= 0.f)) return fail(GQ_EINVAL, "gq_rmsnorm_fwd: eps must be >= 0");
  if (T == 0) return GQ_OK;
  if (!x || !w || !y || !rstd) return fail(GQ_EINVAL, "gq_rmsnorm_fwd: NULL pointer");
  REQ_ALIGN(x, 16, "gq_rmsnorm_fwd");
  REQ_ALIGN(w, 16, "gq_rmsnorm_fwd");
  REQ_ALIGN(y, 16, "gq_rmsnorm_fwd");
  REQ_ALIGN(rstd, 4, "gq_rmsnorm_fwd");
  HIP_TRY(launch_rmsnorm_fwd(x, w, T, (int32_t)H, eps, y, rstd, S(stream)), "gq_rmsnorm_fwd");
  return GQ_OK;
}

static int rmsnorm_bwd_impl(const uint16_t* dy, const uint16_t* x, const float* w, const float* rstd,
                   int64_t T, int64_t H, uint16_t* dx, void* stream) {
  g_err.clear();
  if (T < 0 || H < 8 || H % 8 || H > INT_MAX || (T + 3) / 4 > INT_MAX)
    return fail(GQ_EINVAL, "gq_rmsnorm_bwd: bad T/H (H must be a positive multiple of 8)");
  if (T == 0) return GQ_OK;
  if (!dy || !x || !w || !rstd || !dx) return fail(GQ_EINVAL, "gq_rmsnorm_bwd: NULL pointer");
  REQ_ALIGN(dy, 16, "gq_rmsnorm_bwd");
  REQ_ALIGN(x, 16, "gq_rmsnorm_bwd");
  REQ_ALIGN(w, 16, "gq_rmsnorm_bwd");
  REQ_ALIGN(dx, 16, "gq_rmsnorm_bwd");
  REQ_ALIGN(rstd, 4, "gq_rmsnorm_bwd");
  HIP_TRY(launch_rmsnorm_bwd(dy, x, w, rstd, T, (int32_t)H, dx, S(stream)), "gq_rmsnorm_bwd");
  return GQ_OK;
}

static int moe_combine_bwd_impl(const uint16_t* dxrows, const int32_t* pos, int64_t T, int32_t k, int64_t H,
                       uint16_t* dx, void* stream) {
  g_err.clear();
  if (T < 0 || k < 1 || k > 16 || H < 8 || H % 8)
    return fail(GQ_EINVAL, "gq_moe_combine_bwd: bad T/k/H (H must be a multiple of 8)");
  if (T == 0) return GQ_OK;
  if (!dxrows || !pos || !dx) return fail(GQ_EINVAL, "gq_moe_combine_bwd: NULL pointer");
  REQ_ALIGN(dxrows, 16, "gq_moe_combine_bwd");
  REQ_ALIGN(dx, 16, "gq_moe_combine_bwd");
  REQ_ALIGN(pos, 4, "gq_moe_combine_bwd");
  HIP_TRY(launch_combine(dxrows, nullptr, pos, T, k, H, dx, S(stream)), "gq_moe_combine_bwd");
  return GQ_OK;
}

// ------------------------------------------------------------ grouped MMQ
namespace {
int check_group(const gq_lora_linear* P, int nproj, const char* name) {
  for (int i = 0; i < nproj; ++i) {
    int rc = check_proj(&P[i], name, true);
    if (rc) return rc;
  }
  return GQ_OK;
}
bool same_shape(const gq_lora_linear& a, const gq_lora_linear& b) {
  return a.qtype == b.qtype && a.rank == b.rank && a.n_out == b.n_out && a.n_in == b.n_in &&
         a.n_experts == b.n_experts && a.scale == b.scale;
}
int64_t grouped_mtiles(int64_t M, int E, int bm) { return cdiv(M, bm) + E; }
}  // namespace

size_t gq_grouped_mmq_lora_fwd_workspace_size(const gq_lora_linear* P, int32_t, int64_t) {
  if (!P) return 0;
  Ws w(nullptr);
  w.take<int32_t>(64);                // device error word (first 4 bytes)
  w.take<int32_t>(P->n_experts + 1);  // GEMM tiles
  w.take<int32_t>(P->n_experts + 1);  // 16-row tiles of the row dots
  w.take<int32_t>(P->n_experts + 1);  // skinny tiles of the spill rows
  return w.size();
}

static int grouped_mmq_lora_fwd_impl(const gq_lora_linear* P, int32_t nproj, int32_t epilogue,
                            const gq_grouped_fwd_args* a, void* ws, size_t ws_bytes,
                            void* stream) {
  g_err.clear();
  if (!P || !a) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: NULL argument");
  if (!((epilogue == GQ_EPI_NONE && nproj == 1) || (epilogue == GQ_EPI_SWIGLU && nproj == 2)))
    return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: epilogue %d needs nproj %d", epilogue,
                epilogue == GQ_EPI_SWIGLU ? 2 : 1);
  int rc = check_group(P, nproj, "gq_grouped_mmq_lora_fwd");
  if (rc) return rc;
  if (nproj == 2 && !same_shape(P[0], P[1]))
    return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: gate and up projections differ in shape");
  const int64_t M = a->M;
  if (M < 0 || M > INT_MAX) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: bad M");
  if (!a->offsets) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: NULL offsets");
  if (M == 0) return GQ_OK;
  if (!a->in || !a->out || !a->xa) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: NULL in/out/xa");
  if (epilogue == GQ_EPI_SWIGLU && (!a->save_g || !a->save_u))
    return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: SWIGLU needs save_g and save_u");
  if (a->gather_div < 1) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_fwd: gather_div < 1");
  {
    const char* fn = "gq_grouped_mmq_lora_fwd";
    REQ_ALIGN(a->in, 16, fn);
    REQ_ALIGN(a->out, 2, fn);
    REQ_ALIGN(a->save_g, 2, fn);
    REQ_ALIGN(a->save_u, 2, fn);
    REQ_ALIGN(a->xa, 4, fn);
    REQ_ALIGN(a->gather, 4, fn);
    REQ_ALIGN(a->offsets, 4, fn);
  }
  if ((rc = check_ws(ws, ws_bytes, gq_grouped_mmq_lora_fwd_workspace_size(P, nproj, M)))) return rc;
  const hipStream_t st = S(stream);
  const int E = P->n_experts, r = P->rank, K = (int)P->n_in, N = (int)P->n_out;
  Ws w(ws);
  int32_t* err = w.take<int32_t>(64);
  int32_t* ts = w.take<int32_t>(E + 1);
  int32_t* ts16 = w.take<int32_t>(E + 1);
  int32_t* tsp = w.take<int32_t>(E + 1);
  const int ncols = epilogue == GQ_EPI_SWIGLU ? 2 * N : N;  // GEMM columns
  const bool w_al = aligned(P[0].w_blocks, 16) && (nproj < 2 || aligned(P[1].w_blocks, 16));
  const int tc = cdiv(M, E) <= 64 ? pick_fwd_tile(cdiv(M, E), M, cdiv(ncols, TILE_BN), K, w_al)
                                   : pick_grp_tile(M, E, cdiv(ncols, TILE_BN));
  const int spill = spill_rows(tc, E, false, K, w_al);
  HIP_TRY(launch_tile_starts(a->offsets, E, M, err, tile_bm(tc), ts, 16, ts16, 1, nullptr, st,
                             spill, spill ? tsp : nullptr),
          "gq_grouped_mmq_lora_fwd: tiles");

  RowDotArgs rd;
  memset(&rd, 0, sizeof rd);
  rd.M = M; rd.C = K; rd.r = r; rd.act = a->in; rd.lda = K; rd.gather = a->gather;
  rd.gdiv = a->gather_div; rd.offsets = a->offsets; rd.E = E; rd.tile16 = ts16;
  rd.w_estride = (int64_t)r * K; rd.w_jstride = K; rd.w_cstride = 1; rd.nout = nproj;
  for (int i = 0; i < nproj; ++i) {
    rd.W[i] = P[i].A;
    rd.out[i] = a->xa + (int64_t)i * M * r;
  }
  HIP_TRY(launch_rowdot(rd, st), "gq_grouped_mmq_lora_fwd: in A^T");

  GemmArgs g = gemm_defaults();
  g.M = M; g.K = K;
  g.a0 = a->in; g.lda = K; g.gather = a->gather; g.gdiv = a->gather_div;
  g.w0 = static_cast<const uint8_t*>(P[0].w_blocks);
  g.w1 = nproj == 2 ? static_cast<const uint8_t*>(P[1].w_blocks) : nullptr;
  g.w_rowbytes = rowbytes(P); g.w_estride = (int64_t)N * g.w_rowbytes; g.w_nb = K / 32;
  g.w_rows = N;
  g.E = E; g.offsets = a->offsets; g.tile_start = ts;
  g.s = P->scale; g.r = r;
  g.lB0 = P[0].B; g.lB1 = nproj == 2 ? P[1].B : nullptr; g.lB_estride = (int64_t)N * r;
  g.rv0 = a->xa; g.rv1 = nproj == 2 ? a->xa + M * r : nullptr;
  g.o0 = a->out; g.o1 = a->save_g; g.o2 = a->save_u; g.ldo = N;
  int epi;
  if (epilogue == GQ_EPI_SWIGLU) {
    g.N = 2 * N;
    g.ntiles = cdiv(2 * N, tile_bn(tc));
    epi = EPI_SWIGLU;
  } else {
    g.N = N;
    g.ntiles = cdiv(N, tile_bn(tc));
    epi = EPI_LIN;
  }
  g.mtiles = (int)grouped_mtiles(M, E, tile_bm(tc));
  HIP_TRY(launch_gemm(P->qtype, epi, tc, g, st), "gq_grouped_mmq_lora_fwd: grouped MMQ");
  if (spill) {  // at most one spill tile per expert
    g.tile_start = tsp;
    g.mtiles = E;
    g.spill_bm = tile_bm(tc);
    HIP_TRY(launch_gemm(P->qtype, epi, spill_tile(spill), g, st), "gq_grouped_mmq_lora_fwd: spill rows");
  }
  return GQ_OK;
}

namespace {
struct GrpBwdWs {
  int32_t* err;
  int32_t* ts;
  int32_t* cs;
  int32_t* ts16;
  int32_t* tsp;  // skinny tiles of the spill rows
  float* dyB;
  float* wdyB;
  float* wxa;
  float* part_down;
  float* part[4];  // colred partials, one set per adapter gradient
};
int grp_rc(const gq_lora_linear* P, int64_t M) {
  const int64_t H = P[0].n_in > P[0].n_out ? P[0].n_in : P[0].n_out;
  return pick_rc(M, H, P[0].rank, P[0].n_experts);
}
GrpBwdWs plan_grp_bwd(Ws& w, const gq_lora_linear* P, int mode, int64_t M) {
  GrpBwdWs p;
  memset(&p, 0, sizeof p);
  const int E = P->n_experts, r = P->rank;
  p.err = w.take<int32_t>(64);  // device error word (first 4 bytes)
  p.ts = w.take<int32_t>(E + 1);
  p.cs = w.take<int32_t>(E + 1);
  p.ts16 = w.take<int32_t>(E + 1);
  p.tsp = w.take<int32_t>(E + 1);
  const int64_t slots = colred_slots(M, grp_rc(P, M), E);
  if (mode == GQ_BWD_DOWN_SWIGLU) {
    const int64_t H = P[0].n_out, I = P[0].n_in;
    p.dyB = w.take<float>(M * r);
    p.wdyB = w.take<float>(M * r);
    p.wxa = w.take<float>(M * r);
    p.part_down = w.take<float>((int64_t)cdiv(I, TILE_BN) * M * (1 + 2 * r));
    p.part[0] = w.take<float>(slots * I * r);  // dA_d
    p.part[1] = w.take<float>(slots * H * r);  // dB_d
  } else {
    const int64_t H = P[0].n_in, I = P[0].n_out;
    p.part[0] = w.take<float>(slots * H * r);  // dA_g
    p.part[1] = w.take<float>(slots * H * r);  // dA_u
    p.part[2] = w.take<float>(slots * I * r);  // dB_g
    p.part[3] = w.take<float>(slots * I * r);  // dB_u
  }
  return p;
}
}  // namespace

size_t gq_grouped_mmq_lora_bwd_workspace_size(const gq_lora_linear* P, int32_t nproj,
                                              int32_t mode, int64_t M) {
  if (!P || M <= 0 || nproj < 1) return 0;
  Ws w(nullptr);
  plan_grp_bwd(w, P, mode, M);
  return w.size();
}

static int grouped_mmq_lora_bwd_impl(const gq_lora_linear* P, int32_t nproj, int32_t mode,
                            const gq_grouped_bwd_args* a, void* ws, size_t ws_bytes,
                            void* stream) {
  g_err.clear();
  if (!P || !a) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: NULL argument");
  const hipStream_t st = S(stream);
  const int64_t M = a->M;
  if (M < 0 || M > INT_MAX) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: bad M");
  if (!a->offsets) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: NULL offsets");
  if (a->gather_div < 1) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: gather_div < 1");
  int rc;
  if (mode == GQ_BWD_DOWN_SWIGLU) {
    if (nproj != 3) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: DOWN_SWIGLU needs nproj 3");
    if ((rc = check_group(P, 3, "gq_grouped_mmq_lora_bwd"))) return rc;
    if (!same_shape(P[1], P[2]) || P[0].n_in != P[1].n_out || P[0].n_out != P[1].n_in ||
        P[0].rank != P[1].rank || P[0].n_experts != P[1].n_experts || P[0].scale != P[1].scale)
      return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: down/gate/up shapes do not form an FFN");
  } else if (mode == GQ_BWD_GATEUP) {
    if (nproj != 2) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: GATEUP needs nproj 2");
    if ((rc = check_group(P, 2, "gq_grouped_mmq_lora_bwd"))) return rc;
    if (!same_shape(P[0], P[1]))
      return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: gate and up projections differ in shape");
  } else {
    return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: unknown mode %d", mode);
  }
  const int E = P->n_experts, r = P->rank;
  const float s = P->scale;
  {
    const char* fn = "gq_grouped_mmq_lora_bwd";
    REQ_ALIGN(a->dA_d, 4, fn);
    REQ_ALIGN(a->dB_d, 4, fn);
    REQ_ALIGN(a->dA_g, 4, fn);
    REQ_ALIGN(a->dB_g, 4, fn);
    REQ_ALIGN(a->dA_u, 4, fn);
    REQ_ALIGN(a->dB_u, 4, fn);
  }
  if (M == 0) {
    // no rows: every adapter gradient is exactly zero
    if (mode == GQ_BWD_DOWN_SWIGLU) {
      const int64_t H = P[0].n_out, I = P[0].n_in;
      if (!a->dA_d || !a->dB_d) return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: NULL dA_d/dB_d");
      HIP_TRY(launch_fill_f32(a->dA_d, (int64_t)E * r * I, 0.f, st), "zero dA_d");
      HIP_TRY(launch_fill_f32(a->dB_d, (int64_t)E * H * r, 0.f, st), "zero dB_d");
    } else {
      const int64_t H = P[0].n_in, I = P[0].n_out;
      if (!a->dA_g || !a->dB_g || !a->dA_u || !a->dB_u)
        return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: NULL adapter gradient");
      HIP_TRY(launch_fill_f32(a->dA_g, (int64_t)E * r * H, 0.f, st), "zero dA_g");
      HIP_TRY(launch_fill_f32(a->dA_u, (int64_t)E * r * H, 0.f, st), "zero dA_u");
      HIP_TRY(launch_fill_f32(a->dB_g, (int64_t)E * I * r, 0.f, st), "zero dB_g");
      HIP_TRY(launch_fill_f32(a->dB_u, (int64_t)E * I * r, 0.f, st), "zero dB_u");
    }
    return GQ_OK;
  }
  if ((rc = check_ws(ws, ws_bytes, gq_grouped_mmq_lora_bwd_workspace_size(P, nproj, mode, M))))
    return rc;
  // every argument check before the first launch
  if (mode == GQ_BWD_DOWN_SWIGLU) {
    if (!a->dy || !a->w_flat || !a->sorted || !a->g || !a->u || !a->h || !a->xa_d || !a->dw_flat ||
        !a->dA_d || !a->dB_d || !a->dg || !a->du || !a->dgB || !a->duB)
      return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: NULL pointer for DOWN_SWIGLU");
    const char* fn = "gq_grouped_mmq_lora_bwd";
    REQ_ALIGN(a->dy, 16, fn);
    REQ_ALIGN(a->g, 16, fn);
    REQ_ALIGN(a->u, 16, fn);
    REQ_ALIGN(a->h, 16, fn);
    REQ_ALIGN(a->dg, 16, fn);
    REQ_ALIGN(a->du, 16, fn);
    REQ_ALIGN(a->w_flat, 4, fn);
    REQ_ALIGN(a->sorted, 4, fn);
    REQ_ALIGN(a->xa_d, 4, fn);
    REQ_ALIGN(a->dw_flat, 4, fn);
    REQ_ALIGN(a->dA_d, 4, fn);
    REQ_ALIGN(a->dB_d, 4, fn);
    REQ_ALIGN(a->dgB, 4, fn);
    REQ_ALIGN(a->duB, 4, fn);
    REQ_ALIGN(a->gather, 4, fn);
    REQ_ALIGN(a->offsets, 4, fn);
  } else {
    if (!a->x || !a->xa || !a->dg || !a->du || !a->dgB || !a->duB || !a->dxrows || !a->dA_g ||
        !a->dB_g || !a->dA_u || !a->dB_u)
      return fail(GQ_EINVAL, "gq_grouped_mmq_lora_bwd: NULL pointer for GATEUP");
    {
      const char* fn = "gq_grouped_mmq_lora_bwd";
      REQ_ALIGN(a->x, 16, fn);
      REQ_ALIGN(a->dg, 16, fn);
      REQ_ALIGN(a->du, 16, fn);
      REQ_ALIGN(a->dxrows, 2, fn);
      REQ_ALIGN(a->xa, 4, fn);
      REQ_ALIGN(a->dgB, 4, fn);
      REQ_ALIGN(a->duB, 4, fn);
      REQ_ALIGN(a->dA_g, 4, fn);
      REQ_ALIGN(a->dB_g, 4, fn);
      REQ_ALIGN(a->dA_u, 4, fn);
      REQ_ALIGN(a->dB_u, 4, fn);
      REQ_ALIGN(a->gather, 4, fn);
      REQ_ALIGN(a->offsets, 4, fn);
    }
    if (P[0].n_out % GEMM_BK)
      return fail(GQ_ENOTSUP, "gq_grouped_mmq_lora_bwd: intermediate size must be a multiple of 64");
  }
  Ws w(ws);
  const GrpBwdWs W = plan_grp_bwd(w, P, mode, M);
  const int rcg = grp_rc(P, M);
  const int slots = (int)colred_slots(M, rcg, E);
  // GEMM tiles (the backward MMQ's tile height), column-reduction chunks and
  // 16-row row-dot tiles of every expert, in one launch
  const int ntiles_bwd = cdiv(P[0].n_in, TILE_BN);  // N of both backward MMQs
  int tc = pick_grp_tile(M, E, ntiles_bwd);
  // backward MMQ with at most 8 rows per expert on average: the skinny NN
  // MMQ (with more, experts spill into second 16-row tiles that re-read the
  // weights, and the 64-row tile measured faster)
  const bool w_al = aligned(P[0].w_blocks, 16) && (mode != GQ_BWD_GATEUP || aligned(P[1].w_blocks, 16));
  if (cdiv(M, E) <= 8 && w_al) {
    const int tn = pick_nn_tile(cdiv(M, E), M, ntiles_bwd, P[0].n_in, true, 0);
    if (tile_skinny(tn)) tc = tn;
  }
  // output row of both backward MMQs: I (down) or H (gate/up) = P[0].n_in
  const int spill = spill_rows(tc, E, true, P[0].n_in, w_al);
  HIP_TRY(launch_tile_starts(a->offsets, E, M, W.err, tile_bm(tc), W.ts, rcg, W.cs, 16,
                             mode == GQ_BWD_DOWN_SWIGLU ? W.ts16 : nullptr, st,
                             spill, spill ? W.tsp : nullptr, true),
          "gq_grouped_mmq_lora_bwd: tiles");

  ColRedArgs cr;
  memset(&cr, 0, sizeof cr);
  cr.M = M; cr.r = r; cr.offsets = a->offsets; cr.chunk_start = W.cs; cr.E = E; cr.rc = rcg;
  cr.slots = slots; cr.gdiv = 1;

  if (mode == GQ_BWD_DOWN_SWIGLU) {
    const int H = (int)P[0].n_out, I = (int)P[0].n_in;
    // dY Bd (unweighted) and its gate-weighted copy
    RowDotArgs rd;
    memset(&rd, 0, sizeof rd);
    rd.M = M; rd.C = H; rd.r = r; rd.act = a->dy; rd.lda = H; rd.gather = a->gather;
    rd.gdiv = a->gather_div; rd.offsets = a->offsets; rd.E = E; rd.tile16 = W.ts16;
    rd.W[0] = P[0].B; rd.w_estride = (int64_t)H * r; rd.w_jstride = 1; rd.w_cstride = r;
    rd.out[0] = W.dyB; rd.nout = 1; rd.out2 = W.wdyB; rd.wflat = a->w_flat; rd.sorted = a->sorted;
    rd.win = a->xa_d; rd.wout = W.wxa;  // the gate-weighted xa_d rows, in the same pass
    HIP_TRY(launch_rowdot(rd, st), "gq_grouped_mmq_lora_bwd: dY Bd, w xa_d");

    GemmArgs g = gemm_defaults();
    g.M = M; g.N = I; g.K = H;
    g.a0 = a->dy; g.lda = H; g.gather = a->gather; g.gdiv = a->gather_div;
    g.w0 = static_cast<const uint8_t*>(P[0].w_blocks);
    g.w_rowbytes = rowbytes(&P[0]); g.w_estride = (int64_t)H * g.w_rowbytes; g.w_nb = I / 32;
    g.w_rows = H;
    g.E = E; g.offsets = a->offsets; g.tile_start = W.ts;
    g.ntiles = cdiv(I, nn_tile_bn(tc));
    g.mtiles = (int)grouped_mtiles(M, E, tile_bm(tc));
    g.s = s; g.r = r;
    g.lA0 = P[0].A; g.lA_estride = (int64_t)r * I;
    g.lB1 = P[1].B; g.lB2 = P[2].B; g.lB_estride = (int64_t)I * r;
    g.rv0 = W.dyB; g.s0 = a->g; g.s1 = a->u; g.wflat = a->w_flat; g.sorted = a->sorted;
    g.o0 = a->dg; g.o1 = a->du; g.ldo = I; g.f0 = W.part_down;
    HIP_TRY(launch_gemm(P[0].qtype, EPI_DOWN_BWD, tc, g, st), "gq_grouped_mmq_lora_bwd: down MMQ");
    if (spill) {
      GemmArgs gs = g;
      gs.tile_start = W.tsp;
      gs.mtiles = E;
      gs.spill_bm = tile_bm(tc);
      HIP_TRY(launch_gemm(P[0].qtype, EPI_DOWN_BWD, spill_tile(spill), gs, st),
              "gq_grouped_mmq_lora_bwd: down spill rows");
    }

    // dA_d[e] = s sum_p (w dY Bd)^T h ;  dB_d[e] = s sum_p dY^T (w xa_d):
    // both reductions in one launch, both finishes in one launch
    cr.C = I; cr.U = a->h; cr.ldu = I; cr.Vv = W.wdyB; cr.part = W.part[0];
    cr.njobs = 2;
    cr.C_1 = H; cr.U_1 = a->dy; cr.ldu_1 = H; cr.gather_1 = a->gather; cr.gdiv_1 = a->gather_div;
    cr.Vv_1 = W.wxa; cr.part_1 = W.part[1];
    // dw, dgB, duB: the row sums of the down MMQ partials, as a side job
    cr.dfin_part = W.part_down; cr.dfin_ntiles = g.ntiles; cr.dfin_sorted = a->sorted;
    cr.dfin_dw = a->dw_flat; cr.dfin_dgB = a->dgB; cr.dfin_duB = a->duB;
    HIP_TRY(launch_colred(cr, st), "dA_d, dB_d partials; dw, dgB, duB");
    ColFinJobs fj;
    memset(&fj, 0, sizeof fj);
    fj.n = 2;
    fj.part[0] = W.part[0]; fj.out[0] = a->dA_d; fj.C[0] = I; fj.transpose[0] = 1;
    fj.part[1] = W.part[1]; fj.out[1] = a->dB_d; fj.C[1] = H; fj.transpose[1] = 0;
    HIP_TRY(launch_colred_finish_grp(fj, W.cs, E, r, s, st), "dA_d, dB_d");
    return GQ_OK;
  }

  // GATEUP
  const int H = (int)P[0].n_in, I = (int)P[0].n_out;
  GemmArgs g = gemm_defaults();
  g.M = M; g.N = H; g.K = 2 * I;
  g.a0 = a->dg; g.a1 = a->du; g.lda = I; g.asplit = I;
  g.w0 = static_cast<const uint8_t*>(P[0].w_blocks);
  g.w1 = static_cast<const uint8_t*>(P[1].w_blocks);
  g.w_rowbytes = rowbytes(&P[0]); g.w_estride = (int64_t)I * g.w_rowbytes; g.w_nb = H / 32;
  g.w_rows = I; g.wsplit = I;
  g.E = E; g.offsets = a->offsets; g.tile_start = W.ts;
  g.ntiles = cdiv(H, nn_tile_bn(tc));
  g.mtiles = (int)grouped_mtiles(M, E, tile_bm(tc));
  g.s = s; g.r = r;
  g.lA0 = P[0].A; g.lA1 = P[1].A; g.lA_estride = (int64_t)r * H;
  g.rv0 = a->dgB; g.rv1 = a->duB;
  g.o0 = a->dxrows; g.ldo = H;
  HIP_TRY(launch_gemm(P[0].qtype, EPI_GATEUP_BWD, tc, g, st), "gq_grouped_mmq_lora_bwd: gate/up MMQ");
  if (spill) {
    g.tile_start = W.tsp;
    g.mtiles = E;
    g.spill_bm = tile_bm(tc);
    HIP_TRY(launch_gemm(P[0].qtype, EPI_GATEUP_BWD, spill_tile(spill), g, st),
            "gq_grouped_mmq_lora_bwd: gate/up spill rows");
  }

  // dA_g and dA_u in one pass over the gathered x rows
  cr.C = H; cr.U = a->x; cr.ldu = H; cr.gather = a->gather; cr.gdiv = a->gather_div;
  cr.Vv = a->dgB; cr.part = W.part[0];
  cr.Vv2 = a->duB; cr.part2 = W.part[1];
  HIP_TRY(launch_colred(cr, st), "dA_g, dA_u partials");
  // dB_g and dB_u in one launch
  cr.Vv2 = nullptr; cr.part2 = nullptr;
  cr.C = I; cr.U = a->dg; cr.ldu = I; cr.gather = nullptr; cr.gdiv = 1; cr.Vv = a->xa;
  cr.part = W.part[2];
  cr.njobs = 2;
  cr.C_1 = I; cr.U_1 = a->du; cr.ldu_1 = I; cr.gather_1 = nullptr; cr.gdiv_1 = 1;
  cr.Vv_1 = a->xa + M * r; cr.part_1 = W.part[3];
  HIP_TRY(launch_colred(cr, st), "dB_g, dB_u partials");
  ColFinJobs fj;
  memset(&fj, 0, sizeof fj);
  fj.n = 4;
  fj.part[0] = W.part[0]; fj.out[0] = a->dA_g; fj.C[0] = H; fj.transpose[0] = 1;
  fj.part[1] = W.part[1]; fj.out[1] = a->dA_u; fj.C[1] = H; fj.transpose[1] = 1;
  fj.part[2] = W.part[2]; fj.out[2] = a->dB_g; fj.C[2] = I; fj.transpose[2] = 0;
  fj.part[3] = W.part[3]; fj.out[3] = a->dB_u; fj.C[3] = I; fj.transpose[3] = 0;
  HIP_TRY(launch_colred_finish_grp(fj, W.cs, E, r, s, st), "dA_g, dA_u, dB_g, dB_u");
  return GQ_OK;
}

// ---------------------------------------------------------------- LM head
namespace {
struct CeWs {
  int32_t* err;
  float* nvalid;
  float* xa;
  float* part_ml;
  float* zlab;
  float* term;
  uint16_t* G;
  uint16_t* G2;  // second gradient buffer when chunks are paired, else nullptr
  float* dh_acc;  // dh_nacc fp32 [T][H] sums, added in order at the end
  int dh_nacc;
  float* part_GB;
  float* part_dB;
  float* GB;
  float* part;
  int64_t ldG;
  int64_t span;  // vocabulary rows per backward step (one or more chunks)
  int mt;
  int ntiles_bwd;
  int tc_fwd, tc_bwd, tc_dh;
};
// Chunks per backward step when the gradient tiles run on the 256 x 192
// tile: the fewest (up to six) that give four full rounds of tiles, kept
// only if the tiles fill the chip (wide_pays); 0 = 128 x 128 gradient tiles.
// Longer steps mean fewer dh launches, each of which reads and writes the
// T x H fp32 sums once.
int64_t ce_wide_chunks(int qtype, int64_t T, int64_t V, int64_t H, int r, int64_t C) {
  const int64_t nchunks = (V + C - 1) / C;
  int64_t g = 1;
  while (g < 6 && g < nchunks && (int64_t)cdiv(T, WIDE_BM) * cdiv(std::min(g * C, V), WIDE_BN) < 1024) ++g;
  return wide_pays(qtype, T, std::min(g * C, V), H, r) ? g : 0;
}
CeWs plan_ce(Ws& w, const gq_lora_linear* L, int64_t T, int64_t chunk, bool grad) {
  CeWs p;
  memset(&p, 0, sizeof p);
  const int64_t V = L->n_out, H = L->n_in, r = L->rank;
  p.err = w.take<int32_t>(64);
  p.nvalid = w.take<float>(64);
  p.xa = w.take<float>(T * r);
  const int nt_v = cdiv(V, TILE_BN);
  p.tc_fwd = pick_fwd_tile(T, T, nt_v, H, aligned(L->w_blocks, 16));
  // 256 x 192 tiles when they fill the chip (part_ml, sized for 128-column
  // tiles, holds their fewer partials)
  if (!tile_skinny(p.tc_fwd) && wide_pays(L->qtype, T, V, H, (int)r)) p.tc_fwd = TILE_WIDE;
  p.part_ml = w.take<float>((int64_t)nt_v * T * 2);
  p.zlab = w.take<float>(T);
  p.term = w.take<float>(T);
  if (grad) {
    const int64_t C = chunk < V ? chunk : V;
    // gradient tiles on the 256 x 192 tile, several chunks per step, when
    // they fill the chip; else 128 x 128 tiles, one chunk per step
    const int64_t gw = ce_wide_chunks(L->qtype, T, V, H, (int)r, C);
    p.span = gw ? std::min(gw * C, V) : C;
    const int bn = gw ? WIDE_BN : TILE_BN;
    p.ldG = (p.span + 63) / 64 * 64;
    p.G = w.take<uint16_t>(T * p.ldG);
    // dh tiles: with the wide gradient tiles, 256 x 128 backward tiles whose
    // two reduction ranges (halves of the step's vocabulary rows) sum into
    // two accumulators; else the 128-row tiles and one accumulator
    p.tc_dh = pick_tile(T, cdiv(H, TILE_BN), p.span, true);
    p.dh_nacc = 1;
    if (gw && L->qtype != GQ_Q2_DM) {
      p.tc_dh = TILE_WIDE_NN;
      p.dh_nacc = 2;
    }
    p.dh_acc = w.take<float>(p.dh_nacc * T * H);
    int64_t ntb = 0;
    for (int64_t c0 = 0; c0 < V; c0 += p.span) ntb += cdiv(std::min(p.span, V - c0), bn);
    p.ntiles_bwd = (int)ntb;
    p.part_GB = w.take<float>(ntb * T * r);
    p.tc_bwd = gw ? TILE_WIDE : pick_tile(T, cdiv(C, TILE_BN));
    p.mt = cdiv(T, tile_bm(p.tc_bwd));
    p.part_dB = w.take<float>((int64_t)p.mt * V * r);
    p.GB = w.take<float>(T * r);
    p.part = w.take<float>(colred_slots(T, pick_rc(T, H, (int)r, 1), 1) * H * r);
    // two or more chunks with 128-row tiles on both passes: chunk c's
    // gradient tiles share a launch with chunk c-1's dh tiles, which needs a
    // second gradient buffer
    const int64_t nsteps = (V + p.span - 1) / p.span;
    if (nsteps >= 2 && p.tc_bwd == TILE_128x128 && tile_bm(p.tc_dh) == 128)
      p.G2 = w.take<uint16_t>(T * p.ldG);
  }
  return p;
}
}  // namespace

size_t gq_lmhead_chunked_ce_workspace_size(const gq_lora_linear* L, int64_t T, int64_t chunk) {
  if (!L || T <= 0 || chunk < 1 || L->rank < 1 || L->n_out < 1) return 0;
  Ws w(nullptr);
  plan_ce(w, L, T, chunk, true);
  return w.size();
}

static int lmhead_chunked_ce_impl(const gq_lora_linear* L, const uint16_t* h, const int64_t* labels,
                         int64_t T, int64_t chunk, int64_t ignore_index, float grad_scale,
                         float* loss, float* lse, uint16_t* dh, float* dA, float* dB, void* ws,
                         size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_proj(L, "gq_lmhead_chunked_ce", false, false);
  if (rc) return rc;
  if (T < 0 || T > INT_MAX) return fail(GQ_EINVAL, "gq_lmhead_chunked_ce: bad T");
  if (chunk < 1) return fail(GQ_EINVAL, "gq_lmhead_chunked_ce: chunk_rows must be >= 1");
  if (!loss) return fail(GQ_EINVAL, "gq_lmhead_chunked_ce: NULL loss");
  const bool grad = dh != nullptr;
  if (grad && (!dA || !dB)) return fail(GQ_EINVAL, "gq_lmhead_chunked_ce: dh needs dA and dB");
  const hipStream_t st = S(stream);
  const int64_t V = L->n_out;
  const int H = (int)L->n_in, r = L->rank;
  REQ_ALIGN(loss, 4, "gq_lmhead_chunked_ce");
  REQ_ALIGN(dA, 4, "gq_lmhead_chunked_ce");
  REQ_ALIGN(dB, 4, "gq_lmhead_chunked_ce");
  if (T == 0) {
    HIP_TRY(launch_fill_f32(loss, 1, 0.f, st), "gq_lmhead_chunked_ce");
    if (grad) {
      HIP_TRY(launch_fill_f32(dA, (int64_t)r * H, 0.f, st), "gq_lmhead_chunked_ce");
      HIP_TRY(launch_fill_f32(dB, V * r, 0.f, st), "gq_lmhead_chunked_ce");
    }
    return GQ_OK;
  }
  if (!h || !labels || !lse) return fail(GQ_EINVAL, "gq_lmhead_chunked_ce: NULL h, labels or lse");
  REQ_ALIGN(h, 16, "gq_lmhead_chunked_ce");
  REQ_ALIGN(dh, 2, "gq_lmhead_chunked_ce");
  REQ_ALIGN(labels, 8, "gq_lmhead_chunked_ce");
  REQ_ALIGN(loss, 4, "gq_lmhead_chunked_ce");
  REQ_ALIGN(lse, 4, "gq_lmhead_chunked_ce");
  REQ_ALIGN(dA, 4, "gq_lmhead_chunked_ce");
  REQ_ALIGN(dB, 4, "gq_lmhead_chunked_ce");
  if (chunk > V) chunk = V;
  if (chunk > INT_MAX / 2) return fail(GQ_ENOTSUP, "gq_lmhead_chunked_ce: chunk too large");
  Ws meas(nullptr);
  plan_ce(meas, L, T, chunk, grad);
  if ((rc = check_ws(ws, ws_bytes, meas.size()))) return rc;
  Ws w(ws);
  const CeWs P = plan_ce(w, L, T, chunk, grad);

  RowDotArgs rd;
  memset(&rd, 0, sizeof rd);
  rd.M = T; rd.C = H; rd.r = r; rd.act = h; rd.lda = H; rd.gdiv = 1; rd.E = 1;
  rd.W[0] = L->A; rd.w_jstride = H; rd.w_cstride = 1; rd.out[0] = P.xa; rd.nout = 1;
  HIP_TRY(launch_rowdot(rd, st), "ce: h A^T");

  const uint8_t* wb = static_cast<const uint8_t*>(L->w_blocks);
  GemmArgs g = gemm_defaults();
  g.M = T; g.N = (int)V; g.K = H;
  g.a0 = h; g.lda = H;
  g.w0 = wb; g.w_rowbytes = rowbytes(L); g.w_nb = H / 32; g.w_rows = (int)V; g.w_row0 = 0;
  g.ntiles = cdiv(V, P.tc_fwd == TILE_WIDE ? WIDE_BN : tile_bn(P.tc_fwd));
  g.mtiles = cdiv(T, tile_bm(P.tc_fwd));
  g.s = L->scale; g.r = r; g.lB0 = L->B; g.rv0 = P.xa;
  g.f0 = P.part_ml; g.f1 = P.zlab; g.labels = labels; g.ignore_index = ignore_index;
  g.V = (int)V; g.ntile_base = 0;
  HIP_TRY(launch_gemm(L->qtype, EPI_CE_FWD, P.tc_fwd, g, st), "ce: logits pass");
  HIP_TRY(launch_ce_merge(P.part_ml, g.ntiles, T, P.zlab, labels, V, ignore_index, lse, P.term,
                          P.err, P.nvalid, loss, st),
          "ce: log-sum-exp merge, loss");
  if (!grad) return GQ_OK;

  // Step after step (one chunk, or up to six on the 256 x 192 gradient
  // tile): the gradient tiles write G for the step's vocabulary rows (plus
  // the G.B and dB partials), the dh tiles accumulate G deq(W) of the step
  // into dh_acc (step order fixed: deterministic; with the 256 x 128 dh
  // tiles the first and second half of the step's rows into two sums).  With two gradient
  // buffers, step c's gradient tiles and step c-1's dh tiles run in one
  // launch.
  const bool pair = P.G2 != nullptr;
  GemmArgs dprev = gemm_defaults();
  bool have_prev = false;
  int ntile_base = 0;
  int ci = 0;
  for (int64_t c0 = 0; c0 < V; c0 += P.span, ++ci) {
    const int C = (int)std::min(P.span, V - c0);
    uint16_t* Gc = (pair && (ci & 1)) ? P.G2 : P.G;
    GemmArgs b = gemm_defaults();
    b.M = T; b.N = C; b.K = H;
    b.a0 = h; b.lda = H;
    b.w0 = wb; b.w_rowbytes = rowbytes(L); b.w_nb = H / 32; b.w_rows = C; b.w_row0 = (int)c0;
    b.ntiles = cdiv(C, P.tc_bwd == TILE_WIDE ? WIDE_BN : TILE_BN);
    b.mtiles = cdiv(T, tile_bm(P.tc_bwd));
    b.s = L->scale; b.r = r; b.lB0 = L->B; b.rv0 = P.xa;
    b.o0 = Gc; b.ldo = P.ldG;
    b.f1 = P.part_GB; b.f2 = P.part_dB;
    b.labels = labels; b.ignore_index = ignore_index; b.lse = lse; b.coef = grad_scale;
    b.nvalid = P.nvalid; b.V = (int)V; b.ntile_base = ntile_base;
    ntile_base += b.ntiles;

    GemmArgs d = gemm_defaults();
    d.M = T; d.N = H; d.K = C;
    d.a0 = Gc; d.lda = P.ldG;
    d.w0 = wb; d.w_rowbytes = rowbytes(L); d.w_nb = H / 32; d.w_rows = C; d.w_row0 = (int)c0;
    d.ntiles = cdiv(H, P.tc_dh == TILE_WIDE_NN ? WIDE_NN_BN : TILE_BN);
    d.mtiles = cdiv(T, tile_bm(P.tc_dh));
    d.f0 = P.dh_acc; d.ldf = H; d.accum = c0 > 0;
    d.ksplit = P.dh_nacc;
    if (!pair) {
      HIP_TRY(launch_gemm(L->qtype, EPI_CE_BWD, P.tc_bwd, b, st), "ce: gradient tile pass");
      HIP_TRY(launch_gemm(L->qtype, EPI_DH_ACC, P.tc_dh, d, st), "ce: dh pass");
      continue;
    }
    if (have_prev) {
      GemmArgs dk = dprev;
      dk.mtiles = cdiv(T, 128);  // one group of four waves per 128 x 128 tile
      HIP_TRY(launch_ce_bwd_dh(L->qtype, b, dk, st), "ce: gradient tiles + previous chunk's dh tiles");
    } else {
      HIP_TRY(launch_gemm(L->qtype, EPI_CE_BWD, P.tc_bwd, b, st), "ce: gradient tile pass");
    }
    dprev = d;
    have_prev = true;
  }
  if (pair && have_prev) HIP_TRY(launch_gemm(L->qtype, EPI_DH_ACC, P.tc_dh, dprev, st), "ce: dh pass");
  HIP_TRY(launch_sum_parts(P.part_GB, P.ntiles_bwd, T, r, 1.f, P.GB, st), "ce: G B");
  HIP_TRY(launch_sum_parts(P.part_dB, P.mt, V, r, L->scale, dB, st), "ce: dB");
  HIP_TRY(launch_ce_final_dh(P.dh_acc, P.dh_nacc, P.GB, L->A, T, H, r, L->scale, dh, st), "ce: dh");
  ColRedArgs cr;
  memset(&cr, 0, sizeof cr);
  cr.M = T; cr.C = H; cr.r = r; cr.U = h; cr.ldu = H; cr.gdiv = 1; cr.Vv = P.GB; cr.E = 1;
  cr.rc = pick_rc(T, H, r, 1); cr.slots = (int)colred_slots(T, cr.rc, 1); cr.part = P.part;
  HIP_TRY(launch_colred(cr, st), "ce: dA partials");
  HIP_TRY(launch_colred_finish(P.part, nullptr, 1, cr.slots, H, r, L->scale, 1, dA, st), "ce: dA");
  return GQ_OK;
}

}  // extern "C"

// Exported entry points: each runs its implementation above inside
// traced_call (GQ_TRACE ranges, GQ_DEBUG checks; both off by default).
extern "C" {

int gq_dequant(int qtype, const void* blocks, int64_t rows, int64_t cols, int out_dtype, void* out,
               void* stream) {
  return traced_call("gq_dequant", stream, nullptr,
                    [&] { return dequant_impl(qtype, blocks, rows, cols, out_dtype, out, stream); });
}

int gq_linear_lora_fwd(const gq_lora_linear* L, const uint16_t* x, int64_t T, uint16_t* y,
                       float* xa, void* ws, size_t ws_bytes, void* stream) {
  return traced_call("gq_linear_lora_fwd", stream, nullptr,
                    [&] { return linear_lora_fwd_impl(L, x, T, y, xa, ws, ws_bytes, stream); });
}

int gq_linear_lora_bwd(const gq_lora_linear* L, const uint16_t* x, const float* xa,
                       const uint16_t* dy, int64_t T, uint16_t* dx, float* dA, float* dB, void* ws,
                       size_t ws_bytes, void* stream) {
  return traced_call("gq_linear_lora_bwd", stream, nullptr,
                    [&] { return linear_lora_bwd_impl(L, x, xa, dy, T, dx, dA, dB, ws, ws_bytes, stream); });
}

int gq_linear_lora_bwd_noalloc(const gq_lora_linear* L, const uint16_t* x, const float* xa,
                               const uint16_t* dy, int64_t T, uint16_t* dx, float* dA, float* dB,
                               void* stream) {
  return traced_call("gq_linear_lora_bwd_noalloc", stream, nullptr,
                    [&] { return linear_lora_bwd_noalloc_impl(L, x, xa, dy, T, dx, dA, dB, stream); });
}

int gq_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                 int32_t* sorted, int32_t* offsets, int32_t* pos, void* ws, size_t ws_bytes,
                 void* stream) {
  return traced_call("gq_moe_route", stream, nullptr,
                    [&] { return moe_route_impl(logits, T, E, k, ids, w, sorted, offsets, pos, ws, ws_bytes, stream); });
}

int gq_moe_route_bwd(const int32_t* ids, const float* w, const float* dw, int64_t T, int32_t E,
                     int32_t k, float* dlogits, void* stream) {
  return traced_call("gq_moe_route_bwd", stream, nullptr,
                    [&] { return moe_route_bwd_impl(ids, w, dw, T, E, k, dlogits, stream); });
}

int gq_moe_combine_fwd(const uint16_t* o, const float* w, const int32_t* pos, int64_t T, int32_t k,
                       int64_t H, uint16_t* y, void* stream) {
  return traced_call("gq_moe_combine_fwd", stream, nullptr,
                    [&] { return moe_combine_fwd_impl(o, w, pos, T, k, H, y, stream); });
}

int gq_adamw8bit_step(float* p, const float* g, uint8_t* m_codes, uint8_t* v_codes, float* m_scale,
                      float* v_scale, int64_t n, int64_t step, float lr, float beta1, float beta2,
                      float eps, float weight_decay, void* stream) {
  return traced_call("gq_adamw8bit_step", stream, nullptr,
                    [&] { return adamw8bit_step_impl(p, g, m_codes, v_codes, m_scale, v_scale, n, step, lr, beta1, beta2, eps, weight_decay, stream); });
}

int gq_rmsnorm_fwd(const uint16_t* x, const float* w, int64_t T, int64_t H, float eps, uint16_t* y,
                   float* rstd, void* stream) {
  return traced_call("gq_rmsnorm_fwd", stream, nullptr,
                    [&] { return rmsnorm_fwd_impl(x, w, T, H, eps, y, rstd, stream); });
}

int gq_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const float* w, const float* rstd,
                   int64_t T, int64_t H, uint16_t* dx, void* stream) {
  return traced_call("gq_rmsnorm_bwd", stream, nullptr,
                    [&] { return rmsnorm_bwd_impl(dy, x, w, rstd, T, H, dx, stream); });
}

int gq_moe_combine_bwd(const uint16_t* dxrows, const int32_t* pos, int64_t T, int32_t k, int64_t H,
                       uint16_t* dx, void* stream) {
  return traced_call("gq_moe_combine_bwd", stream, nullptr,
                    [&] { return moe_combine_bwd_impl(dxrows, pos, T, k, H, dx, stream); });
}

int gq_grouped_mmq_lora_fwd(const gq_lora_linear* P, int32_t nproj, int32_t epilogue,
                            const gq_grouped_fwd_args* a, void* ws, size_t ws_bytes,
                            void* stream) {
  return traced_call("gq_grouped_mmq_lora_fwd", stream, a && a->M > 0 ? ws : nullptr,
                    [&] { return grouped_mmq_lora_fwd_impl(P, nproj, epilogue, a, ws, ws_bytes, stream); });
}

int gq_grouped_mmq_lora_bwd(const gq_lora_linear* P, int32_t nproj, int32_t mode,
                            const gq_grouped_bwd_args* a, void* ws, size_t ws_bytes,
                            void* stream) {
  return traced_call("gq_grouped_mmq_lora_bwd", stream, a && a->M > 0 ? ws : nullptr,
                    [&] { return grouped_mmq_lora_bwd_impl(P, nproj, mode, a, ws, ws_bytes, stream); });
}

int gq_lmhead_chunked_ce(const gq_lora_linear* L, const uint16_t* h, const int64_t* labels,
                         int64_t T, int64_t chunk, int64_t ignore_index, float grad_scale,
                         float* loss, float* lse, uint16_t* dh, float* dA, float* dB, void* ws,
                         size_t ws_bytes, void* stream) {
  return traced_call("gq_lmhead_chunked_ce", stream, T > 0 ? ws : nullptr,
                    [&] { return lmhead_chunked_ce_impl(L, h, labels, T, chunk, ignore_index, grad_scale, loss, lse, dh, dA, dB, ws, ws_bytes, stream); });
}

}  // extern "C"
