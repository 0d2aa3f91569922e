// KV append: copy the K/V of new tokens into their cache slots.
//
// New K/V go only into the blocks a sequence already holds, one slot per
// token ("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린 서빙 엔진",
// section "PagedAttention -- OS 가상 메모리에서 영감"; section "KV Cache가 왜
// 병목인가" for why past K/V are kept).  One thread moves one 8-element run
// (16 bytes) of one (token, kv head): the K run lands as one 16-byte store (the
// K sub-tile keeps 8 dims of a token together); the V run is spread over 8
// rows of the V sub-tile (the V sub-tile keeps a dim's 16 tokens together), so
// it is 8 two-byte stores.  The op moves a few hundred KB per step and is bound
// by launch latency, not bandwidth.
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
  const int64_t sub = (n * p.num_kv_heads + h) * (p.block_size >> 4) + (off >> 4);
  const int r = off & 15;

  const uint4 kk = *reinterpret_cast<const uint4*>(p.k + th * p.head_dim + c * 8);
  const uint4 vv = *reinterpret_cast<const uint4*>(p.v + th * p.head_dim + c * 8);
  *reinterpret_cast<uint4*>(p.k_cache + ((sub * runs + c) * 16 + r) * 8) = kk;
  uint16_t* vb = p.v_cache + (sub * p.head_dim + c * 8) * 16 + r;
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vb[(2 * e) * 16] = static_cast<uint16_t>(w[e] & 0xffffu);
    vb[(2 * e + 1) * 16] = static_cast<uint16_t>(w[e] >> 16);
  }
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads * (p.head_dim >> 3);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kv_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
