// Device-side helpers shared by the gq kernels (gfx950 / CDNA4).
//
// Block decode follows the block definitions of GGUF Q8_0 / Q4_0 and the
// 2-bit scale/min format (page 2 "Show HN: LoRA over GGUF", section "Things
// involved in the training": MMQ over GGUF weights).  Blocks are read with
// dword loads from the 4-byte-aligned address at or below the block (blocks
// are only 2-byte aligned: 34 and 18 bytes) and realigned in registers, then
// decoded straight to bf16 pairs -- no full-precision weight is ever stored.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { QT_Q8_0 = 0, QT_Q4_0 = 1, QT_Q2_DM = 2 };

template <int QT> struct QTraits;
template <> struct QTraits<QT_Q8_0> { static constexpr int BS = 34, NDW = 9; };
template <> struct QTraits<QT_Q4_0> { static constexpr int BS = 18, NDW = 5; };
template <> struct QTraits<QT_Q2_DM> { static constexpr int BS = 12, NDW = 3; };

__device__ __forceinline__ float h2f(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// round-to-nearest-even float -> bf16 bits (hardware v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Raw bytes of one block, realigned: hdr = first 4 bytes of the block
// (d, and m for Q2_DM), q[] = the payload as dwords.
template <int QT> struct RawBlock {
  static constexpr int NQ = QT == QT_Q8_0 ? 8 : (QT == QT_Q4_0 ? 4 : 2);
  uint32_t hdr;
  uint32_t q[NQ];
};

// Load the block at byte address `blk` (2-byte aligned).  The dword window
// [blk & ~3, (blk & ~3) + 4*NDW) stays inside the block for a block that
// starts 2 bytes past a dword boundary, and runs at most 2 bytes past its end
// otherwise; callers only issue the latter kind when another block follows
// in the same row (rows of an even number of blocks start dword-aligned).
template <int QT> struct BlockWindow {
  uint32_t dw[QTraits<QT>::NDW];
  uint32_t sh;  // nonzero: the block starts at byte 2 of dw[0]
};

// Issue the dword loads of one block and nothing else, so that a prefetch
// does not pull the realignment (which waits for the data) up to the load.
template <int QT>
__device__ __forceinline__ void load_window(const uint8_t* blk, BlockWindow<QT>& w) {
  const uintptr_t a = (uintptr_t)blk;
  // global address space explicitly: a generic (flat) load would also count
  // against the LDS wait counter and serialise with the LDS reads
  const __attribute__((address_space(1))) uint32_t* p =
      (const __attribute__((address_space(1))) uint32_t*)(a & ~(uintptr_t)3);
#pragma unroll
  for (int i = 0; i < QTraits<QT>::NDW; ++i) w.dw[i] = p[i];
  w.sh = (uint32_t)(a & 2);
}

// Realign a loaded window to hdr + payload dwords, ANDed with `mask`.
template <int QT>
__device__ __forceinline__ void realign(const BlockWindow<QT>& w, uint32_t mask, RawBlock<QT>& rb) {
  if constexpr (QT == QT_Q2_DM) {
    // 12-byte blocks in dword-aligned rows are always dword-aligned
    rb.hdr = w.dw[0] & mask;
    rb.q[0] = w.dw[1] & mask;
    rb.q[1] = w.dw[2] & mask;
  } else {
    const bool sh = w.sh != 0;
    rb.hdr = (sh ? (w.dw[0] >> 16) : (w.dw[0] & 0xffffu)) & mask;
#pragma unroll
    for (int i = 0; i < RawBlock<QT>::NQ; ++i)
      rb.q[i] = (sh ? w.dw[i + 1] : __builtin_amdgcn_alignbyte(w.dw[i + 1], w.dw[i], 2)) & mask;
  }
}

template <int QT>
__device__ __forceinline__ void load_block(const uint8_t* blk, RawBlock<QT>& rb) {
  BlockWindow<QT> w;
  load_window<QT>(blk, w);
  realign<QT>(w, 0xffffffffu, rb);
}

// Decode to 32 floats in element order (exact value rounded once to fp32).
template <int QT>
__device__ __forceinline__ void decode_block(const RawBlock<QT>& rb, float (&w)[32]) {
  const float d = h2f(rb.hdr & 0xffffu);
  if constexpr (QT == QT_Q8_0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int q = (int)(int8_t)(uint8_t)(rb.q[i] >> (8 * b));
        w[4 * i + b] = d * (float)q;
      }
    }
  } else if constexpr (QT == QT_Q4_0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (rb.q[i] >> (8 * b)) & 0xffu;
        w[4 * i + b] = d * (float)((int)(byte & 15u) - 8);
        w[16 + 4 * i + b] = d * (float)((int)(byte >> 4) - 8);
      }
    }
  } else {
    const float m = h2f(rb.hdr >> 16);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t byte = (rb.q[j >> 2] >> (8 * (j & 3))) & 0xffu;
        const float q = (float)((byte >> (2 * p)) & 3u);
        w[8 * p + j] = __builtin_fmaf(d, q, m);
      }
    }
  }
}

// Decode for the MMQ kernels: the same values as decode_block for every
// finite scale, with fewer VALU ops.  Bytes are converted with the
// byte-select conversions (v_cvt_f32_ubyte0..3) and the offset folded into
// one FMA:
//   Q8_0: u = q + 128 (xor 0x80 per byte)  w = u*d - 128*d
//   Q4_0: u = nibble                        w = u*d - 8*d
//   Q2:   u = bit pair                      w = u*d + m
// Every product and sum is exact (fp16 d times an 8-bit integer), so the
// result is bit-identical to d*q.  With an infinite scale the biased form
// yields NaN where d*q would be +-inf.
// byte b of x as float: one v_cvt_f32_ubyte{b} (register-only asm; the
// optimiser would otherwise split it into a bit-field extract plus convert)
__device__ __forceinline__ float ubyte(uint32_t x, int b) {
  float r;
  switch (b) {
    case 0: asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x)); break;
    case 1: asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x)); break;
    case 2: asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x)); break;
    default: asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x)); break;
  }
  return r;
}

template <int QT>
__device__ __forceinline__ void decode_block_fast(const RawBlock<QT>& rb, float (&w)[32]) {
  const float d = h2f(rb.hdr & 0xffffu);
  if constexpr (QT == QT_Q8_0) {
    const float off = -128.f * d;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = rb.q[i] ^ 0x80808080u;
#pragma unroll
      for (int b = 0; b < 4; ++b) w[4 * i + b] = __builtin_fmaf(ubyte(u, b), d, off);
    }
  } else if constexpr (QT == QT_Q4_0) {
    const float off = -8.f * d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = rb.q[i] & 0x0f0f0f0fu;
      const uint32_t hi = (rb.q[i] >> 4) & 0x0f0f0f0fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        w[4 * i + b] = __builtin_fmaf(ubyte(lo, b), d, off);
        w[16 + 4 * i + b] = __builtin_fmaf(ubyte(hi, b), d, off);
      }
    }
  } else {
    const float m = h2f(rb.hdr >> 16);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t u = (rb.q[h] >> (2 * pp)) & 0x03030303u;
#pragma unroll
        for (int b = 0; b < 4; ++b) w[8 * pp + 4 * h + b] = __builtin_fmaf(ubyte(u, b), d, m);
      }
    }
  }
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace gq
