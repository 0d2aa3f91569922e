// Paged decode attention, vector-ALU ("SIMT") kernel.
//
// Computes softmax(scale q K^T) V over each sequence's paged context with GQA
// ("[Hacker News 요약] C++와 CUDA로 vLLM의 경량 고성능 LLM 추론 엔진 'Tiny-vLLM'
// 직접 구축하기", section "고성능 추론을 위한 고급 최적화 기법"), reading K/V block
// by block through the block table ("vLLM -- PagedAttention으로 LLM 추론 성능을
// 2~4배 끌어올린 서빙 엔진", section "PagedAttention -- OS 가상 메모리에서 영감").
//
// One workgroup = one (sequence, kv head, partition of the context), NW waves.
// The waves take the partition's 16-token sub-tiles round robin (the pools are
// token-major, so a sub-tile is 16 rows of D values).  Per sub-tile a wave
// holds, lane l = 16*kg + tt:
//   * K: token tt, dims of 8-dim runs kg, kg+4, ... (D/32 runs of 16 bytes);
//     the partial dot products with the G queries are summed over kg by two
//     cross-row shuffles, so every lane ends with the score of token tt;
//   * V: dim l (and l+64 for D=128) of all 16 tokens (16 two-byte loads, each
//     instruction one row); the probabilities of the 16 tokens are broadcast
//     with readlane.
// Softmax is online in fp32 (log2 domain, scale folded into the score).
// Tokens past the context are masked by select: their score becomes -inf and
// their V values 0, so NaN in tail slots never reaches the output.
#include "decode_common.h"

namespace pkv {

namespace {

template <typename T>
__device__ __forceinline__ void unpack8(const uint4& r, float* f) {
  f[0] = lo_f32<T>(r.x); f[1] = hi_f32<T>(r.x);
  f[2] = lo_f32<T>(r.y); f[3] = hi_f32<T>(r.y);
  f[4] = lo_f32<T>(r.z); f[5] = hi_f32<T>(r.z);
  f[6] = lo_f32<T>(r.w); f[7] = hi_f32<T>(r.w);
}

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_simt_kernel(DecodeParams p) {
  constexpr int J = D / 32;   // 8-dim K runs per lane
  constexpr int DV = D / 64;  // V dims per lane
  __shared__ float sm_m[NW][G], sm_l[NW][G], sm_o[NW][G][D];

  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int tt = lane & 15, kg = lane >> 4;
  const WorkItem w = decode_item(p, blockIdx.x, gridDim.x);
  if (w.seq < 0) return;
  const int L = p.context_lens[w.seq];
  const bool bad_len = bad_length(L, p);
  if (bad_len || L == 0) {
    write_degenerate<T, G, NW * kWave>(p, w, bad_len);
    return;
  }
  const int start = w.part * p.part_tokens;
  if (start >= L) return;
  const int end = min(L, start + p.part_tokens);
  const int nsub = (end - start + 15) >> 4;
  const bool single = L <= p.part_tokens;

  float qf[G][J][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint4 r = *reinterpret_cast<const uint4*>(
          p.q + (static_cast<size_t>(w.seq) * p.num_q_heads + w.kvh * G + h) * D + (kg + 4 * j) * 8);
      unpack8<T>(r, qf[h][j]);
    }

  float m[G], ls[G], acc[G][DV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[h][e] = 0.f;
  }
  bool bad = false;
  const int spb = p.block_size >> 4;
  const int* table = p.block_tables + static_cast<size_t>(w.seq) * p.max_blocks_per_seq;

  for (int s = wv; s < nsub; s += NW) {
    const int tok0 = start + (s << 4);
    const int blk = tok0 / p.block_size;
    const int phys = table[blk];
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(p.num_blocks)) {
      bad = true;
      continue;
    }
    const size_t tile = (static_cast<size_t>(phys) * p.num_kv_heads + w.kvh) * spb + ((tok0 - blk * p.block_size) >> 4);
    const uint16_t* kt = p.k_cache + tile * (16 * D);
    const uint16_t* vt = p.v_cache + tile * (16 * D);
    uint4 kr[J];
#pragma unroll
    for (int j = 0; j < J; ++j) kr[j] = *reinterpret_cast<const uint4*>(kt + tt * D + (kg + 4 * j) * 8);
    // V: lane l holds dim l (and l + 64) of the 16 tokens; each load is one row
    uint16_t vr[DV][16];
#pragma unroll
    for (int e = 0; e < DV; ++e)
#pragma unroll
      for (int t = 0; t < 16; ++t) vr[e][t] = vt[t * D + lane + 64 * e];
    const int nvalid = min(16, end - tok0);
    const bool valid = tt < nvalid;

    float pr[G], al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float kf[8];
        unpack8<T>(kr[j], kf);
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qf[h][j][e], kf[e], a);
      }
      a += shfl_xor(a, 16);
      a += shfl_xor(a, 32);
      const float x = valid ? a * p.scale_log2 : -INFINITY;
      float bm = x;
      bm = fmaxf(bm, shfl_xor(bm, 1));
      bm = fmaxf(bm, shfl_xor(bm, 2));
      bm = fmaxf(bm, shfl_xor(bm, 4));
      bm = fmaxf(bm, shfl_xor(bm, 8));
      const float mn = fmaxf(m[h], bm);
      al[h] = fast_exp2(m[h] - mn);
      pr[h] = fast_exp2(x - mn);
      ls[h] = fmaf(ls[h], al[h], pr[h]);
      m[h] = mn;
    }

    float vv[DV][16];
#pragma unroll
    for (int e = 0; e < DV; ++e)
#pragma unroll
      for (int t = 0; t < 16; ++t) vv[e][t] = lo_f32<T>(vr[e][t]);
    if (nvalid < 16) {
#pragma unroll
      for (int e = 0; e < DV; ++e)
#pragma unroll
        for (int t = 0; t < 16; ++t) vv[e][t] = t < nvalid ? vv[e][t] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DV; ++e) {
        float a = acc[h][e] * al[h];
#pragma unroll
        for (int t = 0; t < 16; ++t) a = fmaf(readlane(pr[h], t), vv[e][t], a);
        acc[h][e] = a;
      }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = ls[h];  // per token slot; identical in the four kg rows
    l += shfl_xor(l, 1);
    l += shfl_xor(l, 2);
    l += shfl_xor(l, 4);
    l += shfl_xor(l, 8);
    if (bad) l = __int_as_float(0x7fc00000);
    if (lane == 0) {
      sm_m[wv][h] = m[h];
      sm_l[wv][h] = l;
    }
#pragma unroll
    for (int e = 0; e < DV; ++e) sm_o[wv][h][lane + 64 * e] = acc[h][e];
  }
  __syncthreads();
  combine_and_store<T, D, G, NW>(sm_m, sm_l, sm_o, p, w, single, p.num_parts);
}

constexpr int kSimtWaves = 4;

template <typename T, int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(p.num_seqs) * p.num_parts * p.num_kv_heads;
  hipLaunchKernelGGL((decode_simt_kernel<T, D, G, kSimtWaves>), dim3(static_cast<unsigned>(items)),
                     dim3(kSimtWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DecodeParams& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(p, stream);
    case 2: return launch_t<T, D, 2>(p, stream);
    case 4: return launch_t<T, D, 4>(p, stream);
    case 8:
      if constexpr (D * 8 <= 512) return launch_t<T, D, 8>(p, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_d(const DecodeParams& p, int group, hipStream_t stream) {
  return p.head_dim == 64 ? launch_g<T, 64>(p, group, stream) : launch_g<T, 128>(p, group, stream);
}

}  // namespace

bool simt_supported(int dtype, int head_dim, int group) {
  (void)dtype;
  if (head_dim != 64 && head_dim != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8) return false;
  return group * head_dim <= 512;
}

hipError_t launch_decode_simt(const DecodeParams& p, int dtype, hipStream_t stream) {
  const int group = p.num_q_heads / p.num_kv_heads;
  return dtype == 0 ? launch_d<Bf16>(p, group, stream) : launch_d<Fp16>(p, group, stream);
}

}  // namespace pkv
