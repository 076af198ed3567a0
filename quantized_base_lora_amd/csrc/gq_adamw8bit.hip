// AdamW step for the adapters with 8-bit block-wise quantised states (page 2
// "Show HN: LoRA over GGUF", section "Things involved in the training":
// bitsandbytes' 8-bit AdamW is the optimizer).  One wave per block of 256
// elements (lane l holds elements l, l+64, l+128, l+192): dequantise m and v
// (code book value x the block's scale), update in float32 (no fused
// multiply-adds: the stored codes are decided by these values), write p, then
// the block's new scales (largest |m|, largest v) and the nearest 8-bit codes
// of the states times the reciprocal scales.  The update is the textbook AdamW
// step with the bias corrections moved into host constants:
//   d = sqrt(v) k2 + eps,  p = p kd - s1 (m / d),
//   k2 = 1 / sqrt(1 - b2^t),  kd = 1 - lr wd,  s1 = lr / (1 - b1^t).
//
// Code books ("dynamic tree" layout): an optional sign bit, e zero bits, a
// one bit and f fraction bits i; value 10^-e (0.1 + 0.9 (i + 1) / 2^f), the
// all-zero magnitude 0.  m uses the signed book (7 magnitude bits), v the
// unsigned one (8 bits).  The books are built at compile time from that rule
// in double precision and rounded to float.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "gq_internal.h"

#pragma clang fp contract(off)

namespace gq {
namespace adamw8 {

constexpr int AB = 256;     // elements per quantisation block (one wave)
constexpr int WAVES = 4;    // blocks per workgroup
constexpr int PAD = 2;      // entries past the end of a staged book, +infinity

constexpr double kDecade[8] = {1.0, 0.1, 0.01, 0.001, 0.0001, 0.00001, 0.000001, 0.0000001};

struct CodeBook {
  float v[256];
};

// magnitude code c of a `bits`-bit book
constexpr float book_value(int bits, int c) {
  if (c == 0) return 0.0f;
  int top = 0;
  while ((c >> (top + 1)) != 0) ++top;  // position of the leading one
  const int e = bits - 1 - top, f = top, i = c - (1 << top);
  return (float)(kDecade[e] * (0.1 + 0.9 * ((double)(i + 1) / (double)(1 << f))));
}

constexpr CodeBook make_book(int bits) {
  CodeBook b{};
  for (int c = 0; c < (1 << bits); ++c) b.v[c] = book_value(bits, c);
  return b;
}

__constant__ CodeBook c_mag7 = make_book(7);  // |m| codes 0..127
__constant__ CodeBook c_mag8 = make_book(8);  // v codes 0..255

// Per decade, indexed by f + 1 for the leading-one position f (index 0: a
// below the first non-zero code): the slope and offset of the fraction index
// i as a linear function of the value inside that decade (the book is linear
// in i there), lowered by kBias so that the estimate never lies above the
// answer; the largest i; and the decade's first code.
constexpr double kBias = 1.0 / 32;

struct Decade {
  float slope, off, top;
  int base;
};
struct DecadeTable {
  Decade d[9];
};

constexpr DecadeTable make_decades(int bits) {
  DecadeTable t{};
  t.d[0] = Decade{0.f, 0.f, 0.f, 0};  // window at codes 0, 1
  for (int f = 0; f < bits; ++f) {
    const double w = (double)(1 << f);
    t.d[f + 1] = Decade{(float)(w / (0.9 * kDecade[bits - 1 - f])), (float)(-0.1 * w / 0.9 - 1.0 - kBias),
                        (float)(w - 1.0), 1 << f};
  }
  return t;
}

// Per binary octave [2^(E-127), 2^(E-126)) of a float with exponent field E
// (E = 0: zero and the subnormals): the number of decade edges (first
// non-zero code of each leading-one position) at or below the octave's lower
// end, and the one edge inside the octave, if any (+infinity otherwise).
// Consecutive edges are more than a factor 2 apart, so an octave holds at
// most one; f + 1 of a value a is then cnt + (a >= edge).
struct Octave {
  float edge;
  int cnt;
};
struct OctaveTable {
  Octave o[128];
};

constexpr double pow2(int k) {
  double r = 1.0;
  for (; k > 0; --k) r *= 2.0;
  for (; k < 0; ++k) r *= 0.5;
  return r;
}

constexpr OctaveTable make_octaves(int bits) {
  OctaveTable t{};
  for (int e = 0; e < 128; ++e) {
    const double lo = e == 0 ? 0.0 : pow2(e - 127), hi = pow2(e - 126);
    t.o[e] = Octave{__builtin_inff(), 0};
    for (int f = 0; f < bits; ++f) {
      const double edge = (double)book_value(bits, 1 << f);
      if (edge <= lo) ++t.o[e].cnt;
      else if (edge < hi) t.o[e].edge = (float)edge;
    }
  }
  return t;
}

// Nearest magnitude code of a in [0, 1] (a little above 1 gives the top code)
// in the increasing `BITS`-bit book, ties to the smaller magnitude.  The
// decade comes from the octave table, the fraction index from the linear
// estimate, which is the largest code <= a or the one below it; reading the
// book at k0 .. k0+2 decides which, and the nearest of the two neighbours.
// `book` holds 2^BITS values and PAD entries of +infinity after them, `oct`
// is make_octaves(BITS) and `dec` make_decades(BITS).  Host-callable so that
// it can be checked on every float in [0, 1] against a plain bisection of
// the same book.  A NaN lands in the top octave and gets some code
// (non-finite states are not meaningful).
template <int BITS>
__host__ __device__ __forceinline__ int nearest_code(const float* book, const Octave* oct, const Decade* dec,
                                                     float a) {
  const uint32_t ex = (__builtin_bit_cast(uint32_t, a) >> 23) & 0x7f;  // a >= 0
  const Octave o = oct[ex];
  const Decade d = dec[o.cnt + (a >= o.edge ? 1 : 0)];
  float x = a * d.slope + d.off;
  x = fminf(fmaxf(x, 0.f), d.top);
  const int k0 = d.base + (int)floorf(x);
  const float b0 = book[k0], b1 = book[k0 + 1], b2 = book[k0 + 2];
  const bool up = b1 <= a;  // the largest code <= a is k0 + 1
  const float dlo = a - (up ? b1 : b0);
  const float dhi = (up ? b2 : b1) - a;  // +infinity past the last code
  return k0 + (up ? 1 : 0) + (dhi < dlo ? 1 : 0);
}

__constant__ DecadeTable c_dec7 = make_decades(7);
__constant__ DecadeTable c_dec8 = make_decades(8);
__constant__ OctaveTable c_oct7 = make_octaves(7);
__constant__ OctaveTable c_oct8 = make_octaves(8);

#ifdef __HIP_DEVICE_COMPILE__
__device__ __forceinline__ float wave_max_f32(float v) {
  auto step = [&](auto ctrl_c) {
    constexpr int CTRL = decltype(ctrl_c)::value;
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true)));
  };
  step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{});  // row_mirror
  float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
#pragma unroll
  for (int r = 1; r < 4; ++r)
    s = fmaxf(s, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r)));
  return s;
}
#endif

struct AdamArgs {
  float b1, b2, om1, om2, k2, kd, s1, eps;
};

// One block of 256 elements on one wave, in two phases around the workgroup
// barrier that stages the books.  FULL: the block lies inside [0, n).
// Out-of-range elements of the last block take code 0 and gradient 0, so
// m = v = 0 there, which leaves the block maxima unchanged; they are not
// stored.
struct BlockRegs {
  float g[4], p[4], sm, sv;
  uint32_t cm[4], cv[4];
};

template <bool FULL>
__device__ __forceinline__ void adam_load(BlockRegs& r, const float* __restrict__ p, const float* __restrict__ g,
                                          const uint8_t* __restrict__ mq, const uint8_t* __restrict__ vq,
                                          const float* __restrict__ sm, const float* __restrict__ sv, int64_t n,
                                          int64_t blk, int lane) {
  const int64_t i0 = blk * AB + lane;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = i0 + 64 * j;
    if (FULL || i < n) {
      r.g[j] = g[i];
      r.p[j] = p[i];
      r.cm[j] = mq[i];
      r.cv[j] = vq[i];
    }
  }
  r.sm = sm[blk];
  r.sv = sv[blk];
}

template <bool FULL>
__device__ __forceinline__ void adam_finish(BlockRegs& r, float* __restrict__ p, uint8_t* __restrict__ mq,
                                            uint8_t* __restrict__ vq, float* __restrict__ sm,
                                            float* __restrict__ sv, int64_t n, int64_t blk, int lane,
                                            const AdamArgs& a, const float* sbook, const float* book7,
                                            const float* book8, const Octave* oct7, const Octave* oct8, const Decade* dec7,
                                            const Decade* dec8) {
#ifdef __HIP_DEVICE_COMPILE__
  const int64_t i0 = blk * AB + lane;
  float m[4], v[4], am = 0.f, av = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = sbook[r.cm[j]] * r.sm;
    v[j] = book8[r.cv[j]] * r.sv;
    m[j] = a.b1 * m[j] + a.om1 * r.g[j];
    v[j] = a.b2 * v[j] + a.om2 * (r.g[j] * r.g[j]);
    const float d = sqrtf(v[j]) * a.k2 + a.eps;
    r.p[j] = r.p[j] * a.kd - a.s1 * (m[j] / d);
    am = fmaxf(am, fabsf(m[j]));
    av = fmaxf(av, v[j]);
  }
  // block scales: largest |m| and largest v (max: order-independent)
  am = wave_max_f32(am);
  av = wave_max_f32(av);
  if (lane == 0) {
    sm[blk] = am;
    sv[blk] = av;
  }
  // reciprocal scales; a scale below the smallest normal float (zero
  // included) normalises the block to 0, as its reciprocal would overflow
  const float rm = am >= 0x1p-126f ? 1.0f / am : 0.f;
  const float rv = av >= 0x1p-126f ? 1.0f / av : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float xm = m[j] * rm;
    const float xv = v[j] * rv;
    const int c = nearest_code<7>(book7, oct7, dec7, fabsf(xm));
    const int cvj = nearest_code<8>(book8, oct8, dec8, xv);
    const int64_t i = i0 + 64 * j;
    if (FULL || i < n) {
      p[i] = r.p[j];
      mq[i] = (uint8_t)(xm < 0.f && c != 0 ? (0x80 | c) : c);
      vq[i] = (uint8_t)cvj;
    }
  }
#endif
}

__global__ __launch_bounds__(64 * WAVES) void adamw8bit_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                               uint8_t* __restrict__ mq, uint8_t* __restrict__ vq,
                                                               float* __restrict__ sm, float* __restrict__ sv,
                                                               int64_t n, int64_t nblk, const AdamArgs a) {
#ifdef __HIP_DEVICE_COMPILE__
  __shared__ float sbook[256];  // signed m codes: magnitude, then negated
  __shared__ float book7[128 + PAD], book8[256 + PAD];
  __shared__ Decade dec7[8], dec8[9];
  __shared__ Octave oct7[128], oct8[128];
  const int tid = threadIdx.x, lane = tid & 63;
  book8[tid] = c_mag8.v[tid];
  sbook[tid] = tid < 128 ? c_mag7.v[tid] : -c_mag7.v[tid - 128];
  if (tid < 128) {
    book7[tid] = c_mag7.v[tid];
    oct7[tid] = c_oct7.o[tid];
    oct8[tid] = c_oct8.o[tid];
  }
  if (tid < PAD) {
    book7[128 + tid] = __builtin_inff();
    book8[256 + tid] = __builtin_inff();
  }
  if (tid < 8) dec7[tid] = c_dec7.d[tid];
  if (tid < 9) dec8[tid] = c_dec8.d[tid];
  // the wave's block, kept in scalar registers so that the branches are uniform
  const int64_t blk = (int64_t)blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool full = blk + 1 < nblk || (blk + 1 == nblk && n % AB == 0);
  const bool live = blk < nblk;
  BlockRegs r = {};  // zeros stand for the elements past n
  if (full)
    adam_load<true>(r, p, g, mq, vq, sm, sv, n, blk, lane);
  else if (live)
    adam_load<false>(r, p, g, mq, vq, sm, sv, n, blk, lane);
  __syncthreads();  // books staged
  if (full)
    adam_finish<true>(r, p, mq, vq, sm, sv, n, blk, lane, a, sbook, book7, book8, oct7, oct8, dec7, dec8);
  else if (live)
    adam_finish<false>(r, p, mq, vq, sm, sv, n, blk, lane, a, sbook, book7, book8, oct7, oct8, dec7, dec8);
#endif
}

}  // namespace adamw8

hipError_t launch_adamw8bit(float* p, const float* g, uint8_t* mq, uint8_t* vq, float* sm, float* sv,
                            int64_t n, int64_t t, float lr, float beta1, float beta2, float eps,
                            float wd, hipStream_t st) {
  using namespace adamw8;
  // derived constants from the float32 hyper-parameters, in double, rounded once
  const double l = lr, b1d = beta1, b2d = beta2;
  AdamArgs a;
  a.b1 = beta1;
  a.b2 = beta2;
  a.om1 = (float)(1.0 - b1d);
  a.om2 = (float)(1.0 - b2d);
  a.k2 = (float)(1.0 / sqrt(1.0 - pow(b2d, (double)t)));
  a.kd = (float)(1.0 - l * (double)wd);
  a.s1 = (float)(l / (1.0 - pow(b1d, (double)t)));
  a.eps = eps;
  const int64_t nblk = (n + AB - 1) / AB;
  const int64_t nwg = (nblk + WAVES - 1) / WAVES;
  hipLaunchKernelGGL(adamw8bit_kernel, dim3((unsigned)nwg), dim3(64 * WAVES), 0, st, p, g, mq, vq, sm, sv, n,
                     nblk, a);
  return hipGetLastError();
}

}  // namespace gq
