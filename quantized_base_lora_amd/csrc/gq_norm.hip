// RMS normalisation before a quantised linear layer (page 2 "Show HN: LoRA
// over GGUF", section "Things involved in the training": Liger Kernel's
// RMSNorm on the training path), emitting the bf16 activation the MMQ
// consumes.  y = x * rstd * w with rstd = 1/sqrt(mean(x^2) + eps) per row,
// and the input gradient dx = rstd w dy - (rstd^3 / H) x sum(dy w x) (the
// weight is part of the frozen base).
//
// One wave per row, 8 elements per lane per 16-byte load: a row of up to
// 64 * 8 * NC_MAX elements stays in registers between the reduction and the
// output (one read of x); longer rows read x a second time (from L2).  The
// row sums use a fixed butterfly (DPP within 16-lane rows, then the four row
// results in lane order), so results do not depend on scheduling.  HBM-bound:
// the forward reads x and writes y (2 H bytes each per row), the backward
// reads x, dy and writes dx.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gq_dev.h"
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int NORM_WAVES = 4;  // rows per workgroup
constexpr int NC_MAX = 8;      // 16-byte chunks per lane kept in registers (H <= 4096)

// sum over the wave, the same value in every lane
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto step = [&](auto ctrl_c) {
    constexpr int CTRL = decltype(ctrl_c)::value;
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
  };
  step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{});  // row_mirror
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r));
  return s;
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, u[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load_w8(const float* w, int c, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(w + c);
  const float4 b = *reinterpret_cast<const float4*>(w + c + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

template <bool REG>
__global__ __launch_bounds__(64 * NORM_WAVES) void rmsnorm_fwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w, int64_t T, int32_t H, float eps,
    uint16_t* __restrict__ y, float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * NORM_WAVES + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* xr = x + t * H;
  uint16_t* yr = y + t * H;
  const int nc = H / 8;  // 16-byte chunks in the row; lane takes chunks lane, lane + 64, ...
  uint4 reg[NC_MAX];
  float ss = 0.f;
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NC_MAX; ++i) {
      const int c = lane + 64 * i;
      reg[i] = c < nc ? *reinterpret_cast<const uint4*>(xr + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NC_MAX; ++i) {
      float f[8];
      unpack8(reg[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    }
  } else {
    for (int c = lane; c < nc; c += 64) {
      float f[8];
      unpack8(*reinterpret_cast<const uint4*>(xr + 8 * c), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    }
  }
  const float r = 1.0f / sqrtf(wave_sum_f32(ss) / (float)H + eps);
  if (lane == 0) rstd[t] = r;
  auto emit = [&](int c, const uint4 v) {
    float f[8], wv[8];
    unpack8(v, f);
    load_w8(w, 8 * c, wv);
    *reinterpret_cast<uint4*>(yr + 8 * c) =
        make_uint4(pack_bf2(f[0] * r * wv[0], f[1] * r * wv[1]), pack_bf2(f[2] * r * wv[2], f[3] * r * wv[3]),
                   pack_bf2(f[4] * r * wv[4], f[5] * r * wv[5]), pack_bf2(f[6] * r * wv[6], f[7] * r * wv[7]));
  };
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NC_MAX; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) emit(c, reg[i]);
    }
  } else {
    for (int c = lane; c < nc; c += 64) emit(c, *reinterpret_cast<const uint4*>(xr + 8 * c));
  }
}

template <bool REG>
__global__ __launch_bounds__(64 * NORM_WAVES) void rmsnorm_bwd_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ rstd, int64_t T, int32_t H, uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * NORM_WAVES + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* xr = x + t * H;
  const uint16_t* gr = dy + t * H;
  uint16_t* dr = dx + t * H;
  const int nc = H / 8;
  uint4 rx[NC_MAX], rg[NC_MAX];
  float s = 0.f;
  auto accum = [&](int c, const uint4 vx, const uint4 vg) {
    float fx[8], fg[8], wv[8];
    unpack8(vx, fx);
    unpack8(vg, fg);
    load_w8(w, 8 * c, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += fg[j] * wv[j] * fx[j];
  };
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NC_MAX; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nc;
      rx[i] = ok ? *reinterpret_cast<const uint4*>(xr + 8 * c) : make_uint4(0, 0, 0, 0);
      rg[i] = ok ? *reinterpret_cast<const uint4*>(gr + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NC_MAX; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) accum(c, rx[i], rg[i]);
    }
  } else {
    for (int c = lane; c < nc; c += 64)
      accum(c, *reinterpret_cast<const uint4*>(xr + 8 * c), *reinterpret_cast<const uint4*>(gr + 8 * c));
  }
  const float r = rstd[t];
  const float k = r * r * r * wave_sum_f32(s) / (float)H;
  auto emit = [&](int c, const uint4 vx, const uint4 vg) {
    float fx[8], fg[8], wv[8], o[8];
    unpack8(vx, fx);
    unpack8(vg, fg);
    load_w8(w, 8 * c, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = r * wv[j] * fg[j] - k * fx[j];
    *reinterpret_cast<uint4*>(dr + 8 * c) = make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]),
                                                       pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7]));
  };
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NC_MAX; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) emit(c, rx[i], rg[i]);
    }
  } else {
    for (int c = lane; c < nc; c += 64)
      emit(c, *reinterpret_cast<const uint4*>(xr + 8 * c), *reinterpret_cast<const uint4*>(gr + 8 * c));
  }
}

}  // namespace

hipError_t launch_rmsnorm_fwd(const uint16_t* x, const float* w, int64_t T, int32_t H, float eps,
                              uint16_t* y, float* rstd, hipStream_t st) {
  const dim3 g((unsigned)((T + NORM_WAVES - 1) / NORM_WAVES)), b(64 * NORM_WAVES);
  if (H / 8 <= 64 * NC_MAX)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<true>, g, b, 0, st, x, w, T, H, eps, y, rstd);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<false>, g, b, 0, st, x, w, T, H, eps, y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const float* w,
                              const float* rstd, int64_t T, int32_t H, uint16_t* dx,
                              hipStream_t st) {
  const dim3 g((unsigned)((T + NORM_WAVES - 1) / NORM_WAVES)), b(64 * NORM_WAVES);
  if (H / 8 <= 64 * NC_MAX)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<true>, g, b, 0, st, dy, x, w, rstd, T, H, dx);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<false>, g, b, 0, st, dy, x, w, rstd, T, H, dx);
  return hipGetLastError();
}

}  // namespace gq
