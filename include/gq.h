/*
 * gq.h -- C ABI of libgq: LoRA over a frozen GGUF block-quantised base on
 * AMD MI355X (gfx950).
 *
 * The method (page 2, "Show HN: LoRA over GGUF - Train Qwen3.8-Flash-Next in
 * 40G VRAM", section "Things involved in the training"): the base weights
 * stay in GGUF blocks and are multiplied without being expanded, after
 * llama.cpp's MMQ, dense and grouped by expert; a LoRA adapter is folded
 * into the same layer and trained with Unsloth's fast backward formula for
 * linear and MoE layers; MoE routing is softmax top-k after OpenAI's
 * triton-kernels; the LM head feeds a chunked cross entropy after Liger
 * Kernel's that consumes the MMQ output; no load-balancing loss.
 *
 * Conventions shared by every entry point
 *  - All array pointers are DEVICE pointers to contiguous row-major data
 *    unless a parameter says "host".  bf16 arrays are passed as uint16_t bit
 *    patterns.  The caller owns all memory; the library never allocates.
 *    Temporary storage comes from a caller-provided workspace sized by the
 *    matching *_workspace_size() query (bytes, 256-byte aligned pointer).
 *  - Alignment (checked on the host; GQ_EINVAL names the argument): bf16
 *    arrays read or written with 16-byte accesses must be 16-byte aligned --
 *    x, dy of the linear layer, `in` of the grouped forward, dy, g, u, h, x,
 *    dg, du of the grouped backward, o, y, dxrows, dx of the combines, h of
 *    the LM head, every array of the RMS normalisation (w included), the
 *    dequant output; the other bf16 outputs (y, dx of the linear layer,
 *    out/save_g/save_u, dxrows of the grouped calls, dh) 2-byte aligned;
 *    float32 and int32 arrays 4-byte; int64 labels 8-byte; w_blocks 4-byte
 *    (2-byte for gq_dequant); A and B 16-byte; the workspace 256-byte.
 *  - `stream` is a hipStream_t (0 = the default stream).  Every call only
 *    enqueues work on it and returns; nothing synchronises, nothing copies
 *    between host and device.  Results are stream-ordered.
 *  - Return value: GQ_OK (0) or a negative GQ_E* code.  Argument errors are
 *    found on the host before any HIP call; gq_last_error() then returns a
 *    thread-local message.  A failed launch returns GQ_EHIP.
 *  - Results are bitwise deterministic from run to run (no float atomics;
 *    every reduction has a fixed order).
 *  - No full-precision copy of a quantised weight is ever written: the
 *    blocks are decoded into registers / LDS inside the kernels.
 *  - Calls are reentrant; there is no global mutable state besides the
 *    thread-local error text, the thread-local event pair that
 *    gq_profile_mmq_events installs (see there), the two environment
 *    switches below (read once per process) and the fixed device scratch
 *    array of gq_linear_lora_bwd_noalloc (see there).
 *  - Environment switches (both off when unset or 0):
 *      GQ_TRACE=1  every entry point runs inside a roctx range named after
 *                  it (rocprofv3 --marker-trace shows them; without the
 *                  roctx library nothing is emitted); GQ_TRACE=2 also
 *                  prints "[gq] <name> -> <status>[: <error text>]" to
 *                  stderr for each call.
 *      GQ_DEBUG=1  after queuing its work an entry point synchronises its
 *                  stream, returns GQ_EHIP for an asynchronous HIP error
 *                  and, for the calls that keep a device error word in the
 *                  workspace, GQ_EDEVICE when that word is nonzero.  This
 *                  breaks the "never synchronises" rule above on purpose:
 *                  a debugging aid, not for timing or graph capture.
 *
 * Block formats (32 weights per block, little-endian fields, the blocks of
 * one row contiguous, rows contiguous):
 *   GQ_Q8_0  34 B: fp16 d, int8 q[32]                 w_i = d*q_i
 *   GQ_Q4_0  18 B: fp16 d, u8 qs[16]; byte j holds element j (low nibble)
 *            and element j+16 (high nibble)            w_i = d*(q_i - 8)
 *   GQ_Q2_DM 12 B: fp16 d, fp16 m, u8 qs[8]; byte j holds element j+8p in
 *            bits [2p, 2p+2)                           w_i = d*q_i + m
 * (Q8_0 / Q4_0 are GGUF's formats; the 2-bit scale/min format stands in for
 * the pages' 2-bit bases, page 2 sections "DeepSeek-specific" and
 * "Qwen4-Exp-specific".)
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define GQ_OK 0
#define GQ_EINVAL (-1)     /* bad argument (null pointer, size, alignment) */
#define GQ_ENOTSUP (-2)    /* valid but unsupported shape or type */
#define GQ_EWORKSPACE (-3) /* workspace missing or smaller than required */
#define GQ_EHIP (-4)       /* a HIP launch or runtime call failed */
#define GQ_EDEVICE (-5)    /* device-detected data error: reported through the
                              workspace's first 32-bit word (labels outside
                              [0, V); inconsistent expert offsets) */

/* quant types */
#define GQ_Q8_0 0
#define GQ_Q4_0 1
#define GQ_Q2_DM 2

/* output dtypes of gq_dequant */
#define GQ_F32 0
#define GQ_BF16 1

/* grouped forward epilogues */
#define GQ_EPI_NONE 0   /* out = o = in deq(W)^T + s (in A^T) B^T           */
#define GQ_EPI_SWIGLU 1 /* two projections (gate, up): out = silu(g) * u    */

/* grouped backward modes */
#define GQ_BWD_DOWN_SWIGLU 0
#define GQ_BWD_GATEUP 1

/* Library version: major*10000 + minor*100 + patch. */
int gq_version(void);

/* Thread-local text of the last error returned on this thread ("" if none). */
const char* gq_last_error(void);

/* Bytes per 32-weight block of `qtype`, or -1 for an unknown type. */
int64_t gq_block_bytes(int qtype);

/*
 * Timing hook for profilers and benchmarks (not part of the method): while
 * `start` / `stop` are non-NULL hipEvent_t handles (created with timing
 * enabled), every fused MMQ kernel this thread launches is dispatched with
 * them through hipExtLaunchKernel, which stamps `start` when the kernel
 * begins executing and `stop` when it ends, so hipEventElapsedTime(start,
 * stop) is that kernel's duration without the queue time around it.  Pass
 * NULL, NULL to switch it off.  The events belong to the caller; they are
 * stamped again by each later MMQ launch.
 */
void gq_profile_mmq_events(void* start, void* stop);

/*
 * Block decode (the primitive inside every MMQ; a test/debug export).
 * blocks: [rows][cols/32] blocks of `qtype`.  out: [rows][cols] float32
 * (out_dtype GQ_F32) or bf16 (GQ_BF16).  The float32 result is the weight's
 * exact value rounded once to nearest-even (exact for Q8_0 / Q4_0); bf16 is
 * that float32 rounded to nearest-even.  fp16 subnormal scales are honoured.
 * cols % 32 == 0.  rows == 0 is a no-op.
 */
int gq_dequant(int qtype, const void* blocks, int64_t rows, int64_t cols, int out_dtype,
               void* out, void* stream);

/*
 * A quantised projection with its LoRA adapter (one layer, or E stacked
 * experts when n_experts > 1):
 *   w_blocks  [E][n_out][n_in/32] blocks of `qtype`
 *   A         [E][rank][n_in]  float32
 *   B         [E][n_out][rank] float32
 *   scale     s = alpha / rank
 * Pointers: w_blocks 4-byte aligned, A and B 16-byte aligned (rows of an
 * odd number of Q8_0 / Q4_0 blocks start only 2-byte aligned: the kernels
 * read blocks with 2-byte aligned loads).
 * Constraints: n_in % 32 == 0 (whole blocks), n_out % 8 == 0 (the backward
 * reads activation rows of n_out bf16 with 16-byte loads), 1 <= rank <= 16,
 * 1 <= n_experts <= 1024.  The grouped GATEUP backward also needs the expert
 * intermediate size (gate/up n_out) % 64 == 0: it reduces over [dg | du]
 * in 64-deep steps and switches operands at a step boundary.
 */
typedef struct gq_lora_linear {
    int32_t qtype;
    int32_t rank;
    int64_t n_out;
    int64_t n_in;
    const void* w_blocks;
    const float* A;
    const float* B;
    float scale;
    int32_t n_experts;
} gq_lora_linear;

/*
 * Fused linear forward (one layer; n_experts must be 1):
 *   xa = x A^T                 [T][rank] float32 (saved for the backward)
 *   y  = x deq(W)^T + s xa B^T [T][n_out] bf16
 * x [T][n_in] bf16.  T == 0 is a no-op.
 * Workspace: gq_linear_lora_fwd_workspace_size() bytes, zero except for
 * launches too small to fill the GPU with output tiles, whose reduction is
 * split over workgroups (their fp32 partial sums live there), and for T
 * whose x A^T row-dot runs over column ranges (its fp32 partials, summed by
 * the MMQ).  Without that much workspace the row-dot runs uncut (same
 * results up to rounding); the split launches need it.
 */
size_t gq_linear_lora_fwd_workspace_size(const gq_lora_linear* L, int64_t T);
int gq_linear_lora_fwd(const gq_lora_linear* L, const uint16_t* x, int64_t T, uint16_t* y,
                       float* xa, void* ws, size_t ws_bytes, void* stream);

/*
 * Fast LoRA backward (the frozen W gets no gradient):
 *   dX = dY deq(W) + s (dY B) A     [T][n_in] bf16  (dx may be NULL: skipped)
 *   dB = s dY^T xa                  [n_out][rank] float32 (overwritten)
 *   dA = s (dY B)^T x               [rank][n_in]  float32 (overwritten)
 * x [T][n_in] bf16, xa [T][rank] float32 from the forward, dy [T][n_out] bf16.
 */
size_t gq_linear_lora_bwd_workspace_size(const gq_lora_linear* L, int64_t T);
int gq_linear_lora_bwd(const gq_lora_linear* L, const uint16_t* x, const float* xa,
                       const uint16_t* dy, int64_t T, uint16_t* dx, float* dA, float* dB,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the fast LoRA backward of
 * gq_linear_lora_bwd with its scratch taken from a fixed device array inside
 * the library instead of a caller workspace.  Same arguments, results and
 * kernels as gq_linear_lora_bwd (bitwise equal outputs); it allocates
 * nothing (no hipMalloc/hipFree, no allocating library call).
 *  - The array holds GQ_NOALLOC_SCRATCH_BYTES bytes on each GPU the library
 *    runs on, from the first call on that GPU until the process ends.  A
 *    shape whose gq_linear_lora_bwd_workspace_size() exceeds it is rejected
 *    with GQ_EWORKSPACE before any launch.
 *  - The first call on a device looks up the array's device address
 *    (hipGetSymbolAddress) with that device current: the stream must belong
 *    to the current device.
 *  - Every call on one GPU shares that GPU's array and leaves its contents
 *    behind; calls that overlap in time on one GPU (different streams or
 *    threads without ordering) race on it and give undefined results.
 *    Calls ordered on one stream are safe.
 * gq_noalloc_scratch_bytes() returns the array's size.
 */
#define GQ_NOALLOC_SCRATCH_BYTES (32u << 20)
size_t gq_noalloc_scratch_bytes(void);
int gq_linear_lora_bwd_noalloc(const gq_lora_linear* L, const uint16_t* x, const float* xa,
                               const uint16_t* dy, int64_t T, uint16_t* dx, float* dA, float* dB,
                               void* stream);

/*
 * MoE routing, softmax top-k.  For each token t over logits [T][E] (fp32):
 *   ids[t][0..k)  the k largest logits, ties to the lower expert index, in
 *                 that order;
 *   w[t][0..k)    softmax over the k selected logits (fp32);
 *   sorted[T*k]   assignment indices a = t*k + j sorted stably by expert;
 *   offsets[E+1]  offsets[e] = number of assignments with expert < e;
 *   pos[T*k]      pos[sorted[p]] = p.
 * 1 <= k <= min(E, 16), E <= 1024.  NaN logits give an unspecified order.
 */
size_t gq_moe_route_workspace_size(int64_t T, int32_t E, int32_t k);
int gq_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                 int32_t* sorted, int32_t* offsets, int32_t* pos, void* ws, size_t ws_bytes,
                 void* stream);

/* Router backward (no load-balancing term): dlogits [T][E] fp32 (overwritten),
 * dlogits[t][ids[t][j]] = w[t][j] (dw[t][j] - sum_i w[t][i] dw[t][i]), else 0.
 * dw [T][k] fp32.  An id outside [0, E) matches no column: its term is
 * dropped and nothing is written outside dlogits (there is no workspace to
 * report it in; gq_moe_route never produces such ids). */
int gq_moe_route_bwd(const int32_t* ids, const float* w, const float* dw, int64_t T, int32_t E,
                     int32_t k, float* dlogits, void* stream);

/* Combine: y[t] = sum_{j<k} w[t][j] o[pos[t*k+j]]  (fp32 sum in slot order).
 * o [T*k][H] bf16 rows in sorted order; y [T][H] bf16.  H % 8 == 0. */
int gq_moe_combine_fwd(const uint16_t* o, const float* w, const int32_t* pos, int64_t T,
                       int32_t k, int64_t H, uint16_t* y, void* stream);

/* Combine backward for the activations: dx[t] = sum_j dxrows[pos[t*k+j]]
 * (fp32 sum in slot order).  dxrows [T*k][H] bf16; dx [T][H] bf16. */
int gq_moe_combine_bwd(const uint16_t* dxrows, const int32_t* pos, int64_t T, int32_t k,
                       int64_t H, uint16_t* dx, void* stream);

/*
 * Grouped MMQ + LoRA forward over routed rows.  P[0..nproj) are stacked
 * expert projections with identical shapes (n_experts = E).  Row p
 * (0 <= p < M) belongs to expert e with offsets[e] <= p < offsets[e+1]
 * (offsets [E+1], device) and reads activation row
 *   in[gather[p] / gather_div]   (gather may be NULL: row p reads in[p]).
 *   GQ_EPI_NONE   (nproj 1): out[p] = in_p deq(W_e)^T + s (in_p A_e^T) B_e^T
 *                            xa[p]  = in_p A_e^T
 *   GQ_EPI_SWIGLU (nproj 2, P[0] = gate, P[1] = up):
 *                 g, u as above; out[p] = silu(g) * u;
 *                 save_g[p] = g, save_u[p] = u (bf16); xa = [2][M][rank].
 * Only experts that own rows read their blocks.
 * The offsets are checked on the device (offsets[0] == 0, non-decreasing,
 * offsets[E] == M; expert ids outside [0, E) in the routing that produced
 * them break this): invalid offsets set the workspace's first 32-bit word
 * to nonzero (GQ_EDEVICE condition, readable after synchronising) and no
 * row is processed, so the outputs are left unspecified but nothing is read
 * or written out of bounds; valid offsets set it to 0.
 */
typedef struct gq_grouped_fwd_args {
    const uint16_t* in;      /* activations [*][n_in] bf16 */
    const int32_t* gather;   /* [M] or NULL */
    int32_t gather_div;      /* >= 1 */
    const int32_t* offsets;  /* [E+1] */
    int64_t M;               /* total rows */
    uint16_t* out;           /* [M][n_out] bf16 */
    uint16_t* save_g;        /* SWIGLU only */
    uint16_t* save_u;        /* SWIGLU only */
    float* xa;               /* [nproj][M][rank] */
} gq_grouped_fwd_args;

size_t gq_grouped_mmq_lora_fwd_workspace_size(const gq_lora_linear* P, int32_t nproj,
                                              int64_t M);
int gq_grouped_mmq_lora_fwd(const gq_lora_linear* P, int32_t nproj, int32_t epilogue,
                            const gq_grouped_fwd_args* a, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Grouped fast-LoRA backward of a routed SwiGLU expert FFN, in two calls.
 *
 * GQ_BWD_DOWN_SWIGLU, nproj 3: P[0] = down, P[1] = gate, P[2] = up.
 *   For row p of expert e with token t = gather[p] / gather_div and gate
 *   weight wp = w_flat[sorted[p]]:
 *     e_p   = dy[t] deq(Wd_e) + s (dy[t] Bd_e) Ad_e          (unweighted)
 *     dh    = wp e_p;  sg = sigmoid(g);  dg = dh u sg (1 + g (1 - sg));
 *     du    = dh g sg                       -> dg, du [M][I] bf16
 *     dw_flat[sorted[p]] = <e_p, silu(g) u>  (= <dy[t], o_p>)   fp32
 *     dgB[p] = dg Bg_e, duB[p] = du Bu_e     [M][rank] fp32
 *     dA_d[e] = s sum_p (wp dy[t] Bd_e)^T h_p,  dB_d[e] = s sum_p (wp dy[t])^T xa_d[p]
 *   Inputs: dy [T][H], g, u, h [M][I] bf16 (saved), xa_d [M][rank].
 * GQ_BWD_GATEUP, nproj 2: P[0] = gate, P[1] = up.
 *   dxrows[p] = dg deq(Wg_e) + du deq(Wu_e) + s (dgB[p] Ag_e + duB[p] Au_e)  bf16
 *   dA_g[e] = s sum_p dgB[p]^T x_p,  dB_g[e] = s sum_p dg[p]^T xa_g[p]; same for up.
 *   Inputs: x (activation rows via gather), dg, du, dgB, duB, xa (= [2][M][rank]).
 * Adapter gradients of experts without rows are written as exact zeros.
 * Offsets are checked on the device as in the forward (the workspace's
 * first 32-bit word: 0 valid, nonzero invalid; with invalid offsets the
 * adapter gradients are zero and the row outputs unspecified).
 * All bf16 row arrays (dy, x, g, u, h, dg, du, dxrows) must be 16-byte
 * aligned (GQ_EINVAL otherwise).
 */
typedef struct gq_grouped_bwd_args {
    const int32_t* offsets;  /* [E+1] */
    int64_t M;
    const int32_t* gather;   /* [M] row -> activation row * gather_div, or NULL */
    int32_t gather_div;
    /* DOWN_SWIGLU */
    const uint16_t* dy;      /* [*][H] bf16, read through gather */
    const float* w_flat;     /* [M] gate weights by assignment */
    const int32_t* sorted;   /* [M] */
    const uint16_t* g;       /* [M][I] */
    const uint16_t* u;
    const uint16_t* h;
    const float* xa_d;       /* [M][rank] */
    float* dw_flat;          /* [M] by assignment */
    float* dA_d;             /* [E][rank][I] */
    float* dB_d;             /* [E][H][rank] */
    /* shared between the two modes */
    uint16_t* dg;            /* [M][I] (written by DOWN_SWIGLU, read by GATEUP) */
    uint16_t* du;
    float* dgB;              /* [M][rank] */
    float* duB;
    /* GATEUP */
    const uint16_t* x;       /* [*][H] bf16, read through gather */
    const float* xa;         /* [2][M][rank] (xa_g, xa_u) */
    uint16_t* dxrows;        /* [M][H] bf16 */
    float* dA_g;             /* [E][rank][H] */
    float* dB_g;             /* [E][I][rank] */
    float* dA_u;
    float* dB_u;
} gq_grouped_bwd_args;

size_t gq_grouped_mmq_lora_bwd_workspace_size(const gq_lora_linear* P, int32_t nproj,
                                              int32_t mode, int64_t M);
int gq_grouped_mmq_lora_bwd(const gq_lora_linear* P, int32_t nproj, int32_t mode,
                            const gq_grouped_bwd_args* a, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * LM head + chunked cross entropy (head->n_experts must be 1; n_out = V
 * vocabulary rows, n_in = H):
 *   z     = h deq(W)^T + s (h A^T) B^T   (never stored whole)
 *   lse   [T] fp32 log-sum-exp of each row of z (online over the vocabulary)
 *   loss  (device scalar) = (1/N_valid) sum_{valid t} (lse_t - z[t][label_t])
 * If dh != NULL also (the vocabulary walked in chunks of chunk_rows rows;
 * G = grad_scale/N_valid (softmax(z) - onehot(label)), zero rows for ignored
 * tokens):
 *   dh [T][H] bf16 = G deq(W) + s (G B) A;  dA [rank][H] = s (G B)^T h;
 *   dB [V][rank] = s G^T (h A^T)            (fp32, overwritten)
 * V (n_out) may be any positive size (no multiple-of-8 constraint here).
 * labels [T] int64, each in [0, V) or == ignore_index.  With no valid label
 * the loss and gradients are zero.  A label outside [0, V) that is not
 * ignore_index is treated as ignored and sets the workspace's first 32-bit
 * word to nonzero (GQ_EDEVICE condition, readable after synchronising).
 * chunk_rows >= 1.  The workspace holds the gradient rows of at most six
 * chunks (T x 6 chunk_rows bf16): of one chunk; of two when the backward
 * runs one chunk's gradient tiles beside the previous chunk's dh tiles
 * (two or more chunks with 128-row tiles); of up to six when the gradient
 * tiles run 256 x 192 and one launch covers the fewest chunks (at most
 * six) that give it four full rounds of tiles.  Plus O(T x (H + r) + V x r)
 * floats (two T x H fp32 dh sums with the 256 x 192 gradient tiles); it
 * never holds T x V values.
 */
size_t gq_lmhead_chunked_ce_workspace_size(const gq_lora_linear* head, int64_t T,
                                           int64_t chunk_rows);
int gq_lmhead_chunked_ce(const gq_lora_linear* head, const uint16_t* h, const int64_t* labels,
                         int64_t T, int64_t chunk_rows, int64_t ignore_index, float grad_scale,
                         float* loss, float* lse, uint16_t* dh, float* dA, float* dB, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * One AdamW step for adapter parameters with 8-bit block-wise quantised
 * optimizer states (page 2 "Show HN: LoRA over GGUF", section "Things
 * involved in the training": bitsandbytes' 8-bit AdamW; the pages give no
 * formulas, the definition here is this library's reading):
 *   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2        (float32, no FMA)
 *   d = sqrt(v) k2 + eps;   p = p kd - s1 (m / d)
 * with k2 = 1 / sqrt(1 - b2^step), kd = 1 - lr weight_decay and
 * s1 = lr / (1 - b1^step) formed in double from the float32 arguments and
 * rounded once (the textbook AdamW step with the bias corrections moved into
 * constants).  p fp32 [n] (updated in place), g fp32 [n].  The states are
 * stored in blocks of 256 elements: m_codes, v_codes uint8 [n] and m_scale,
 * v_scale fp32 [ceil(n / 256)]; an element's state = book[code] * its
 * block's scale, the scale being the block's largest |m| (largest v) after
 * the update and the code the book entry nearest to the state times the
 * float32 reciprocal of the scale (ties to the smaller magnitude; a scale
 * below 2^-126 stores code 0).  Books: "dynamic tree" codes -- optional sign
 * bit, e zero bits, a one bit, f fraction bits i -- value
 * 10^-e (0.1 + 0.9 (i + 1) / 2^f), all-zero magnitude 0; m signed (7
 * magnitude bits), v unsigned (8 bits).
 * Zero-filled codes and scales are the initial (zero) state.  step >= 1;
 * 0 <= beta < 1, eps > 0, lr >= 0, weight_decay >= 0; n = 0 is a no-op.
 * No workspace; bitwise deterministic.
 */
int gq_adamw8bit_step(float* p, const float* g, uint8_t* m_codes, uint8_t* v_codes, float* m_scale,
                      float* v_scale, int64_t n, int64_t step, float lr, float beta1, float beta2,
                      float eps, float weight_decay, void* stream);

/*
 * RMS normalisation before a quantised linear layer, emitting the bf16
 * activation the MMQ consumes (page 2 "Show HN: LoRA over GGUF", section
 * "Things involved in the training": Liger Kernel's RMSNorm is on the
 * training path; the pages give no formula, this is the usual definition):
 *   rstd[t] = 1 / sqrt(mean_i x[t][i]^2 + eps)      fp32 [T] (saved for the backward)
 *   y[t][i] = bf16(x[t][i] * rstd[t] * w[i])          bf16 [T][H]
 * x bf16 [T][H], w fp32 [H] (the frozen base's norm weight).  The backward
 * returns the input gradient only (w receives none):
 *   dx[t][j] = rstd w_j dy[t][j] - (rstd^3 / H) x[t][j] sum_i dy[t][i] w_i x[t][i]
 * H a positive multiple of 8; x, y, dy, dx and w 16-byte aligned; eps >= 0;
 * T = 0 is a no-op.  No workspace.  Row sums have a fixed order.
 */
int gq_rmsnorm_fwd(const uint16_t* x, const float* w, int64_t T, int64_t H, float eps, uint16_t* y,
                   float* rstd, void* stream);
int gq_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const float* w, const float* rstd,
                   int64_t T, int64_t H, uint16_t* dx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
