// Device helpers shared by the SOCKET kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace socketlsh {

constexpr int kHead = 128;       // supported head dimension
constexpr int kHistBins = 1024;  // first top-k digit: float bits >> 21 (non-negative floats)
constexpr int kHistShift = 21;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 packed in a uint4 -> 8 floats (exact widening).
__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// DPP move within rows of 16 lanes (row_ror:n is control 0x120 + n).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Butterfly sum over each row of 16 lanes; every lane of the row gets the
// same total (each level adds the same two operands in every lane).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0x128>(x);
  x += dpp_f32<0x124>(x);
  x += dpp_f32<0x122>(x);
  x += dpp_f32<0x121>(x);
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));
  x = fmaxf(x, dpp_f32<0x124>(x));
  x = fmaxf(x, dpp_f32<0x122>(x));
  x = fmaxf(x, dpp_f32<0x121>(x));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ uint64_t lanemask_lt64() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace socketlsh
