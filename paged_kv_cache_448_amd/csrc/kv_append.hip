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
