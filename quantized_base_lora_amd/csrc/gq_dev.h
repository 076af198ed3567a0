// Device-side helpers shared by the gq kernels (gfx950 / CDNA4).
//
// Block decode follows the block definitions of GGUF Q8_0 / Q4_0 and the
// 2-bit scale/min format (page 2 "Show HN: LoRA over GGUF", section "Things
// involved in the training": MMQ over GGUF weights).  A block (only 2-byte
// aligned: 34 and 18 bytes) is read as its fp16 scale plus the payload with
// unaligned dword loads, then decoded straight to bf16 pairs -- no
// full-precision weight is ever stored.
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

// Raw bytes of one block: hdr = the scale (low 16 bits; d and m for Q2_DM),
// q[] = the payload as dwords.
template <int QT> struct RawBlock {
  static constexpr int NQ = QT == QT_Q8_0 ? 8 : (QT == QT_Q4_0 ? 4 : 2);
  uint32_t hdr;
  uint32_t q[NQ];
};

// Issue the loads of the block at byte address `blk` (2-byte aligned): the
// fp16 scale and the payload.  The payload of a 2-byte aligned block is read
// with unaligned dword loads straight into place (global memory accepts
// them on this target), so nothing waits for the data before its use.
// Global address space explicitly: a generic (flat) load would also count
// against the LDS wait counter and serialise with the LDS reads.
typedef uint32_t u32_a2 __attribute__((aligned(2)));
template <int QT>
__device__ __forceinline__ void load_block(const uint8_t* blk, RawBlock<QT>& rb) {
  typedef const __attribute__((address_space(1))) uint16_t g_u16;
  typedef const __attribute__((address_space(1))) uint32_t g_u32;
  typedef const __attribute__((address_space(1))) u32_a2 g_u32a2;
  if constexpr (QT == QT_Q2_DM) {
    // 12-byte blocks in dword-aligned rows are always dword-aligned
    const g_u32* p = (const g_u32*)blk;
    rb.hdr = p[0];
    rb.q[0] = p[1];
    rb.q[1] = p[2];
  } else {
    rb.hdr = *(const g_u16*)blk;
    const g_u32a2* q = (const g_u32a2*)(blk + 2);
#pragma unroll
    for (int i = 0; i < RawBlock<QT>::NQ; ++i) rb.q[i] = q[i];
  }
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
// result is bit-identical to d*q, except that a zero weight comes out as +0
// where d*0 is -0 for a negative d.  With an infinite scale the biased form
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

// Decode straight to packed bf16 pairs: o[i] = (bf16(w[2i]), bf16(w[2i+1]))
// with w as decode_block_fast gives it (bit-identical).  For the 2-bit
// scale/min block the four values d*u + m (u = 0..3) are rounded to bf16
// once per block and kept as two byte planes (low bytes, high bytes); each
// group of four bit pairs then takes a mask, two table permutes and two
// byte interleaves, 1.5 VALU per weight instead of 3 (bit-field extract,
// convert, FMA and half a pack).
template <int QT>
__device__ __forceinline__ void decode_block_bf16(const RawBlock<QT>& rb, uint32_t (&o)[16]) {
  if constexpr (QT == QT_Q2_DM) {
    const float d = h2f(rb.hdr & 0xffffu), m = h2f(rb.hdr >> 16);
    const uint32_t p01 = pack_bf2(__builtin_fmaf(0.f, d, m), __builtin_fmaf(1.f, d, m));
    const uint32_t p23 = pack_bf2(__builtin_fmaf(2.f, d, m), __builtin_fmaf(3.f, d, m));
    // v_perm_b32 picks bytes of {src0 : src1} (src1 = bytes 0-3)
    const uint32_t lo = __builtin_amdgcn_perm(p23, p01, 0x06040200u);  // low bytes of the 4 values
    const uint32_t hi = __builtin_amdgcn_perm(p23, p01, 0x07050301u);  // high bytes
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // elements 8pp + 4h + b, b = 0..3: bit pair pp of byte b of q[h]
        const uint32_t u = (rb.q[h] >> (2 * pp)) & 0x03030303u;
        const uint32_t vl = __builtin_amdgcn_perm(0u, lo, u);
        const uint32_t vh = __builtin_amdgcn_perm(0u, hi, u);
        o[4 * pp + 2 * h] = __builtin_amdgcn_perm(vh, vl, 0x05010400u);
        o[4 * pp + 2 * h + 1] = __builtin_amdgcn_perm(vh, vl, 0x07030602u);
      }
    }
  } else {
    float w[32];
    decode_block_fast<QT>(rb, w);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = pack_bf2(w[2 * i], w[2 * i + 1]);
  }
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace gq
