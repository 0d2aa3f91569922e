// Paged decode attention on the matrix cores (MFMA) of gfx950.
//
// Same result as the vector-ALU kernel -- softmax(scale q K^T) V over each
// sequence's paged context with GQA ("[Hacker News 요약] C++와 CUDA로 vLLM의 경량
// 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을 위한 고급
// 최적화 기법"; paging per "vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배
// 끌어올린 서빙 엔진", section "PagedAttention -- OS 가상 메모리에서 영감") -- but the
// two contractions of a 16-token sub-tile run as MFMA tiles, so the vector ALU
// only does the softmax:
//
//   S^T[16 tok x 16 cols] = K[16 tok x D] . Q^T[D x 16 cols]   (D/32 x mfma 16x16x32)
//   O^T[D x 16 cols]     += V^T[D x 16 tok] . P^T[16 tok x 16 cols] (D/16 x mfma 16x16x16)
//
// The 16 columns are the G q heads that share the kv head (G <= 16; unused
// columns hold zero queries).  The cache layout makes every operand a plain
// coalesced load: lane l = 16*kg + r reads the 16-byte K run kg (+4j) of token
// r -- for fixed j the wave reads one contiguous KB -- and the 8-byte V piece
// (dim 16j + r, tokens 4kg..4kg+3) -- 512 contiguous bytes per j.  The S tile
// comes back with lane l holding tokens 4kg..4kg+3 of column r, which is
// exactly the P^T operand layout of the PV product, so probabilities never
// leave registers.
//
// Softmax is online in fp32 (log2 domain).  P enters the PV product rounded to
// the cache's 16-bit type (round to nearest even); the denominator sums the same
// rounded values, so the output is an exact convex combination of V rows up to
// fp32 rounding.  Tokens past the context are masked by select (score -inf, V
// 0), so NaN in tail slots never reaches the output.
//
// Work split: one workgroup per (sequence, kv head, partition); each of its NW
// waves takes a contiguous run of the partition's sub-tiles and keeps the next
// sub-tile's loads in flight while it computes the current one.
#include "decode_common.h"

namespace pkv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;

template <> struct Mma<Bf16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef short x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0,
                                                     0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2));
  }
};

template <> struct Mma<Fp16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x4 __attribute__((ext_vector_type(4)));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2));
  }
};

// The registers one sub-tile needs: K operands (one per 32 dims) and V
// operands (one per 16 dims).
template <int D> struct Tile {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_mfma_kernel(DecodeParams p) {
  constexpr int JK = D / 32, JV = D / 16;
  __shared__ float sm_m[NW][G], sm_l[NW][G], sm_o[NW][G][D];

  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int r = lane & 15, kg = lane >> 4;
  const WorkItem w = decode_item(p);
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

  // this wave's contiguous run of sub-tiles
  const int per = (nsub + NW - 1) / NW;
  const int s_begin = min(nsub, wv * per), s_end = min(nsub, s_begin + per);

  // Q^T operand: column r = q head kvh*G + r (zero for r >= G), dims of run kg + 4j
  u32x4 qop[JK];
#pragma unroll
  for (int j = 0; j < JK; ++j) {
    if (r < G) {
      qop[j] = *reinterpret_cast<const u32x4*>(
          p.q + (static_cast<size_t>(w.seq) * p.num_q_heads + w.kvh * G + r) * D + (kg + 4 * j) * 8);
    } else {
      qop[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int bs = p.block_size, spb = bs >> 4;
  const int nblk_seq = (L + bs - 1) / bs;
  const int* table = p.block_tables + static_cast<size_t>(w.seq) * p.max_blocks_per_seq;
  // window of 64 block ids, one per lane, refreshed when a sub-tile leaves it
  int win0 = -(1 << 30), ids = 0;
  bool bad = false;

  auto load = [&](int s, Tile<D>& t) {
    const int tok0 = start + (s << 4);
    const int blk = tok0 / bs;
    if (blk >= win0 + kWave || blk < win0) {
      win0 = blk;
      ids = win0 + lane < nblk_seq ? table[win0 + lane] : 0;
    }
    const int phys = __builtin_amdgcn_readlane(ids, blk - win0);
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(p.num_blocks)) {
      bad = true;
#pragma unroll
      for (int j = 0; j < JK; ++j) t.k[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < JV; ++j) t.v[j] = u32x2{0u, 0u};
      return;
    }
    const size_t tile = (static_cast<size_t>(phys) * p.num_kv_heads + w.kvh) * spb + ((tok0 - blk * bs) >> 4);
    const uint16_t* kt = p.k_cache + tile * (16 * D);
    const uint16_t* vt = p.v_cache + tile * (16 * D);
#pragma unroll
    for (int j = 0; j < JK; ++j) t.k[j] = *reinterpret_cast<const u32x4*>(kt + ((4 * j + kg) * 16 + r) * 8);
#pragma unroll
    for (int j = 0; j < JV; ++j) t.v[j] = *reinterpret_cast<const u32x2*>(vt + (16 * j + r) * 16 + 4 * kg);
  };

  float m = -INFINITY, l = 0.f;
  f32x4 o[JV];
#pragma unroll
  for (int j = 0; j < JV; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int s, Tile<D>& t) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < JK; ++j) sc = Mma<T>::qk(t.k[j], qop[j], sc);
    const int nvalid = min(16, end - (start + (s << 4)));
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 4 * kg + i < nvalid ? sc[i] * p.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, shfl_xor(bm, 16));
    bm = fmaxf(bm, shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const float al = fast_exp2(m - mn);
    m = mn;
    const uint32_t p01 = Mma<T>::pack(fast_exp2(x[0] - mn), fast_exp2(x[1] - mn));
    const uint32_t p23 = Mma<T>::pack(fast_exp2(x[2] - mn), fast_exp2(x[3] - mn));
    l = l * al + ((lo_f32<T>(p01) + hi_f32<T>(p01)) + (lo_f32<T>(p23) + hi_f32<T>(p23)));
    if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
      for (int j = 0; j < JV; ++j) o[j] *= al;
    }
    if (nvalid < 16) {
      const uint32_t m0 = (4 * kg < nvalid ? 0xffffu : 0u) | (4 * kg + 1 < nvalid ? 0xffff0000u : 0u);
      const uint32_t m1 = (4 * kg + 2 < nvalid ? 0xffffu : 0u) | (4 * kg + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        t.v[j].x &= m0;
        t.v[j].y &= m1;
      }
    }
    const u32x2 pop = {p01, p23};
#pragma unroll
    for (int j = 0; j < JV; ++j) o[j] = Mma<T>::pv(t.v[j], pop, o[j]);
  };

  // two register sets: the next sub-tile's loads are in flight during compute
  Tile<D> ta, tb;
  int s = s_begin;
  if (s < s_end) load(s, ta);
  while (s < s_end) {
    if (s + 1 < s_end) load(s + 1, tb);
    compute(s, ta);
    if (++s >= s_end) break;
    if (s + 1 < s_end) load(s + 1, ta);
    compute(s, tb);
    ++s;
  }

  // fold the four token rows (kg) of the denominator
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (bad) l = __int_as_float(0x7fc00000);
  if (r < G) {
    if (kg == 0) {
      sm_m[wv][r] = m;
      sm_l[wv][r] = l;
    }
#pragma unroll
    for (int j = 0; j < JV; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wv][r][16 * j + 4 * kg + i] = o[j][i];
  }
  __syncthreads();
  combine_and_store<T, D, G, NW>(sm_m, sm_l, sm_o, p, w, single);
}

constexpr int kMfmaWaves = 4;

template <typename T, int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(p.num_seqs) * p.num_parts * p.num_kv_heads;
  hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, kMfmaWaves>), dim3(static_cast<unsigned>(items)),
                     dim3(kMfmaWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DecodeParams& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(p, stream);
    case 2: return launch_t<T, D, 2>(p, stream);
    case 4: return launch_t<T, D, 4>(p, stream);
    case 8: return launch_t<T, D, 8>(p, stream);
    case 16: return launch_t<T, D, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_d(const DecodeParams& p, int group, hipStream_t stream) {
  return p.head_dim == 64 ? launch_g<T, 64>(p, group, stream) : launch_g<T, 128>(p, group, stream);
}

}  // namespace

bool mfma_supported(int dtype, int head_dim, int group) {
  (void)dtype;
  if (head_dim != 64 && head_dim != 128) return false;
  return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, hipStream_t stream) {
  const int group = p.num_q_heads / p.num_kv_heads;
  return dtype == 0 ? launch_d<Bf16>(p, group, stream) : launch_d<Fp16>(p, group, stream);
}

}  // namespace pkv
