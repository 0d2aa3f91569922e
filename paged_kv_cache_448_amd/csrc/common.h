// Device-side helpers shared by the kernels of the paged KV-cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kSubTile = 16;  // tokens per cache sub-tile

struct Bf16 {};
struct Fp16 {};

// The two 16-bit values packed in w, as fp32 (exact conversions).
template <typename T> __device__ __forceinline__ float lo_f32(uint32_t w);
template <typename T> __device__ __forceinline__ float hi_f32(uint32_t w);

template <> __device__ __forceinline__ float lo_f32<Bf16>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float hi_f32<Bf16>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo_f32<Fp16>(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
template <> __device__ __forceinline__ float hi_f32<Fp16>(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// 8 elements (16 bytes) of 16-bit input to 8 E4M3 codes (8 bytes): each value
// times inv_scale in fp32, clamped to +-448 so that the conversion saturates
// (the hardware conversion rounds to nearest even and returns NaN past the
// range), NaN kept NaN and given the code 0x7F.
template <typename T>
__device__ __forceinline__ uint2 to_e4m3(uint4 w, float inv_scale) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = lo_f32<T>(ws[e]) * inv_scale, b = hi_f32<T>(ws[e]) * inv_scale;
    const float ca = a != a ? a : fminf(fmaxf(a, -448.f), 448.f);
    const float cb = b != b ? b : fminf(fmaxf(b, -448.f), 448.f);
    uint32_t pk = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false)) & 0xffffu;
    if (a != a) pk = (pk & 0xff00u) | 0x7fu;
    if (b != b) pk = (pk & 0x00ffu) | 0x7f00u;
    out[e >> 1] |= pk << (16 * (e & 1));
  }
  return uint2{out[0], out[1]};
}

// Quiet-NaN bit pattern of each storage type.
template <typename T> inline constexpr uint16_t kNanBits = 0;
template <> inline constexpr uint16_t kNanBits<Bf16> = 0x7fc0;
template <> inline constexpr uint16_t kNanBits<Fp16> = 0x7e00;

// fp32 -> 16-bit storage, round to nearest even.
template <typename T> __device__ __forceinline__ uint16_t to_bits(float f);
template <> __device__ __forceinline__ uint16_t to_bits<Bf16>(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays a quiet NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
template <> __device__ __forceinline__ uint16_t to_bits<Fp16>(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Workgroups are dispatched round-robin over the 8 XCDs (bid % 8).  Give each
// XCD a contiguous range of work items instead, so items that touch the same
// data (a sequence's partitions, sequences sharing prefix blocks) share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int nx = n >> 3, rem = n & 7, x = bid & 7, k = bid >> 3;
  return x * nx + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// max / sum of v over lanes l and l^16 (l^32), with the gfx950 row-swap
// instructions instead of an LDS permute: a swap of v with itself returns v
// with odd rows taking the even rows' values and v with even rows taking the
// odd rows' values, so combining the two gives every lane the pair it needs.
// Both lanes of a pair combine the same two operands in the same order.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
