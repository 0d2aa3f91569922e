// KV append: copy the K/V of new tokens into their cache slots.
//
// New K/V go only into the blocks a sequence already holds, one slot per
// token ("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린 서빙 엔진",
// section "PagedAttention -- OS 가상 메모리에서 영감"; section "KV Cache가 왜
// 병목인가" for why past K/V are kept).  The pools are token-major, so a
// token's K (or V) for one kv head is one row of head_dim values; one thread
// moves one 8-element run (16 bytes) of K and of V.  The op moves a few
// hundred KB per step and is bound by launch latency, not bandwidth.
#include "common.h"
#include "kernels.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int runs = p.head_dim >> 3;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * runs;
  if (i >= total) return;
  const int c = static_cast<int>(i % runs);
  const int64_t th = i / runs;  // token * Hkv + head
  const int h = static_cast<int>(th % p.num_kv_heads);
  const int64_t t = th / p.num_kv_heads;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= static_cast<int64_t>(p.num_blocks) * p.block_size) return;
  const int64_t n = slot / p.block_size;
  const int off = static_cast<int>(slot - n * p.block_size);
  const size_t row = ((static_cast<size_t>(n) * p.num_kv_heads + h) * p.block_size + off) * p.head_dim + c * 8;
  *reinterpret_cast<uint4*>(p.k_cache + row) = *reinterpret_cast<const uint4*>(p.k + th * p.head_dim + c * 8);
  *reinterpret_cast<uint4*>(p.v_cache + row) = *reinterpret_cast<const uint4*>(p.v + th * p.head_dim + c * 8);
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

template <typename T>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(AppendFp8Params p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int runs = p.head_dim >> 3;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * runs;
  if (i >= total) return;
  const int c = static_cast<int>(i % runs);
  const int64_t th = i / runs;  // token * Hkv + head
  const int h = static_cast<int>(th % p.num_kv_heads);
  const int64_t t = th / p.num_kv_heads;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= static_cast<int64_t>(p.num_blocks) * p.block_size) return;
  const int64_t n = slot / p.block_size;
  const int off = static_cast<int>(slot - n * p.block_size);
  const size_t row = ((static_cast<size_t>(n) * p.num_kv_heads + h) * p.block_size + off) * p.head_dim + c * 8;
  *reinterpret_cast<uint2*>(p.k_cache + row) =
      to_e4m3<T>(*reinterpret_cast<const uint4*>(p.k + th * p.head_dim + c * 8), p.k_inv_scale);
  *reinterpret_cast<uint2*>(p.v_cache + row) =
      to_e4m3<T>(*reinterpret_cast<const uint4*>(p.v + th * p.head_dim + c * 8), p.v_inv_scale);
}

hipError_t launch_kv_append_fp8(const AppendFp8Params& p, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * (p.head_dim >> 3);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (p.src_fp16) {
    hipLaunchKernelGGL(kv_append_fp8_kernel<Fp16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(kv_append_fp8_kernel<Bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * (p.head_dim >> 3);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kv_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
