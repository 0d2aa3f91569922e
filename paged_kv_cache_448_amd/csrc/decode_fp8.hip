// Paged decode attention over FP8 (E4M3) K/V pools on the matrix cores.
//
// Same computation and work split as decode_mfma_kernel (decode_mfma_kernel.h),
// over pools that hold one byte per element: a stored code c of the K (V) pool
// stands for e4m3(c) * k_scale (v_scale).  The pages name FP8 only as a future
// direction ("[Hacker News 요약] C++와 CUDA로 vLLM의 경량 고성능 LLM 추론 엔진
// 'Tiny-vLLM' 직접 구축하기", section "향후 전망"); the decode reads half the bytes of
// the 16-bit pools, which is the point of it, as decode is bound by reading the
// cache ("vLLM -- PagedAttention으로 ...", section "Prefill vs Decode").
//
// E4M3 values are exact in bf16 and in fp16, so each loaded code is widened
// (two per conversion instruction) to q's 16-bit type without rounding and
// the 16-bit MFMA tiles run unchanged; the scales never touch an element:
// k_scale is folded into the softmax scale (the launcher's scale_log2) and
// v_scale into the output (out_scale, applied when the waves' states are
// folded).  Per 16-token sub-tile a lane loads 8 bytes per K operand (8 dims of
// one token) and JV bytes per token for V (4 row slices; the codes of one dim
// from the 4 tokens are gathered with byte permutes first, then widened, so
// the regrouping costs one instruction per two operand words).
//
// Optionally the launch also performs the step's FP8 append, as the 16-bit
// kernel does: leading workgroups store each new token's codes (the bytes
// kv_append_fp8 writes, from the same encoder), and the wave that reads the
// sub-tile holding position L-1 puts the same codes into its registers from LDS.
#include "decode_mfma_kernel.h"

namespace pkv {

namespace {

// Two E4M3 codes (bytes 2*hi, 2*hi+1 of w) widened to one word of two 16-bit
// values of type T, with the gfx950 scaled conversion at scale 1 (exact: every
// E4M3 value is a bf16 and an fp16 value).
template <typename T> struct Widen;
template <> struct Widen<Bf16> {
  static __device__ __forceinline__ uint32_t pair(uint32_t w, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
};
template <> struct Widen<Fp16> {
  static __device__ __forceinline__ uint32_t pair(uint32_t w, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
};

// 8 codes (two words) to the 8 16-bit values of one K operand.
template <typename T>
__device__ __forceinline__ u32x4 widen8(u32x2 c) {
  return u32x4{Widen<T>::pair(c.x, false), Widen<T>::pair(c.x, true), Widen<T>::pair(c.y, false),
               Widen<T>::pair(c.y, true)};
}

// One token's V row slice: JV = D/16 codes (dims JV*r .. JV*r + JV-1).
template <int D> struct VCodes;
template <> struct VCodes<64> {
  uint32_t w[1];
  static __device__ __forceinline__ VCodes load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return VCodes{{static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0))}};
  }
};
template <> struct VCodes<128> {
  uint32_t w[2];
  static __device__ __forceinline__ VCodes load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
    return VCodes{{x.x, x.y}};
  }
};

// The JV PV operands of a sub-tile from the 4 tokens' row slices: operand j is
// dim JV*r + j of tokens 0..3, {t0 t1 | t2 t3}.  Bytes are regrouped first (one
// byte permute gives dims 4c+2h, 4c+2h+1 of two tokens), then each pair of
// codes is widened once.
template <typename T, int D>
__device__ __forceinline__ void v_operands(const VCodes<D> (&v)[4], u32x2 (&op)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {   // 32-bit word c of each slice: dims 4c .. 4c+3 of the slice
#pragma unroll
    for (int h = 0; h < 2; ++h) {      // dims 4c+2h, 4c+2h+1
      const uint32_t sel = h ? 0x07030602u : 0x05010400u;
      const uint32_t t01 = __builtin_amdgcn_perm(v[1].w[c], v[0].w[c], sel);
      const uint32_t t23 = __builtin_amdgcn_perm(v[3].w[c], v[2].w[c], sel);
      op[4 * c + 2 * h] = u32x2{Widen<T>::pair(t01, false), Widen<T>::pair(t23, false)};
      op[4 * c + 2 * h + 1] = u32x2{Widen<T>::pair(t01, true), Widen<T>::pair(t23, true)};
    }
  }
}

// Fused FP8 append, store side: the codes kv_append_fp8 writes for token i =
// sequence i, after the checks the decode side makes (a valid length, and the
// slot is the slot of position L_i - 1); thread per (token, kv head, 8-dim
// run), grid-strided over the append workgroups.
template <typename T, int D, int NT>
__device__ __forceinline__ void append_tokens_fp8(const DecodeParams& p) {
  constexpr int runs = D / 8;
  uint8_t* kc = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.k_cache));
  uint8_t* vc = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.v_cache));
  const int64_t total = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * runs;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < total;
       i += static_cast<int64_t>(p.append_wgs) * NT) {
    const int c = static_cast<int>(i % runs);
    const int64_t th = i / runs;  // sequence * Hkv + kv head
    const int h = static_cast<int>(th % p.num_kv_heads);
    const int t = static_cast<int>(th / p.num_kv_heads);
    const int64_t slot = p.slot_mapping[t];
    const int L = p.context_lens[t];
    if (slot < 0 || L <= 0 || bad_length(L, p)) continue;
    const int pos = L - 1;
    const int blk = pos / p.block_size;
    const int phys = p.block_tables[static_cast<size_t>(t) * p.max_blocks_per_seq + blk];
    const int off = pos - blk * p.block_size;
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(p.num_blocks) ||
        slot != static_cast<int64_t>(phys) * p.block_size + off)
      continue;
    const size_t row = ((static_cast<size_t>(phys) * p.num_kv_heads + h) * p.block_size + off) * D + c * 8;
    *reinterpret_cast<uint2*>(kc + row) =
        to_e4m3<T>(*reinterpret_cast<const uint4*>(p.k_new + th * D + c * 8), p.k_inv_scale);
    *reinterpret_cast<uint2*>(vc + row) =
        to_e4m3<T>(*reinterpret_cast<const uint4*>(p.v_new + th * D + c * 8), p.v_inv_scale);
  }
}

// Headroom of each wave's lazily moved softmax reference, log2 units: the
// reference moves only when a score exceeds it by more than this, so the
// probabilities stay below 2^8 (within range of both 16-bit types) and most
// steps need neither the column maximum across lanes nor a rescale (softmax
// does not depend on the reference).  Measured on the Llama-3.2-1B batch over
// FP8 pools: 18.6-18.7 us per step against 19.0 with the exact running
// maximum.
constexpr float kLazySlack = 8.f;

template <int D> struct Fp8Tile {
  u32x2 k[D / 32];
  VCodes<D> v[4];
};

template <typename T, int D, int G, int NW, int S, int MINW>
__global__ __launch_bounds__(NW * kWave, MINW) void decode_fp8_kernel(DecodeParams p) {
  constexpr int JK = D / 32, JV = D / 16;
  __shared__ float sm_m[NW][G], sm_l[NW][G], sm_o[NW][G][D];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int r = lane & 15, kg = lane >> 4;
  if (static_cast<int>(blockIdx.x) < p.append_wgs) {
    append_tokens_fp8<T, D, NW * kWave>(p);
    return;
  }
  const WorkItem w = decode_item(p, blockIdx.x - p.append_wgs, gridDim.x - p.append_wgs);
  if (w.seq < 0) return;
  const int L = p.context_lens[w.seq];
  const bool bad_len = bad_length(L, p);
  if (bad_len || L == 0) {
    // an appended token needs a position: L = 0 with a slot is a caller error
    const bool orphan = p.slot_mapping != nullptr && p.slot_mapping[w.seq] >= 0;
    write_degenerate<T, G, NW * kWave>(p, w, bad_len || orphan);
    return;
  }
  const int start = w.part * p.part_tokens;
  if (start >= L) return;
  const int end = min(L, start + p.part_tokens);
  const int nsub = (end - start + 15) >> 4;
  const int nparts = (L + p.part_tokens - 1) / p.part_tokens;
  const int n_w = wv < nsub ? (nsub - wv + NW - 1) / NW : 0;

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

  // K and V of the token appended this step (fused append), read together
  // with the block-table window below, with the slot and the block that holds
  // position L-1, so the check costs no round trip of its own.
  uint4 krun = {0u, 0u, 0u, 0u}, vrun = {0u, 0u, 0u, 0u};
  int64_t app_slot = -1;
  int app_phys = 0;
  if (p.slot_mapping != nullptr) {
    const size_t row = static_cast<size_t>(w.seq) * p.num_kv_heads + w.kvh;
    const int c = min(lane, D / 8 - 1);
    krun = *reinterpret_cast<const uint4*>(p.k_new + row * D + 8 * c);
    vrun = *reinterpret_cast<const uint4*>(p.v_new + row * D + 8 * c);
    app_slot = p.slot_mapping[w.seq];
    app_phys = p.block_tables[static_cast<size_t>(w.seq) * p.max_blocks_per_seq + (L - 1) / p.block_size];
  }

  // lane k: pool index of this wave's k-th sub-tile (16*D codes), or -1 for a
  // block id outside the pool
  int tid = 0;
  if (lane < n_w) {
    const int tok0 = start + 16 * (wv + lane * NW);
    const int blk = tok0 / p.block_size;
    const int phys = p.block_tables[static_cast<size_t>(w.seq) * p.max_blocks_per_seq + blk];
    tid = static_cast<unsigned>(phys) < static_cast<unsigned>(p.num_blocks)
              ? (phys * p.num_kv_heads + w.kvh) * (p.block_size >> 4) + ((tok0 - blk * p.block_size) >> 4)
              : -1;
  }
  bool bad = false;

  // Fused append of the token at position L-1: in the workgroup whose
  // partition holds it, the wave that reads that sub-tile encodes the token
  // into LDS of its own (no workgroup barrier) and puts the codes into its
  // registers in place of whatever the load returned (the pool stores are the
  // leading workgroups' job).  The slot is checked after the sub-tile loop; a
  // slot that is not the slot of L-1 is not written and makes the sequence's
  // output NaN (every workgroup of the sequence checks).
  __shared__ __align__(16) uint8_t sm_new[2][D];  // the appended token's K and V codes
  int app_w = -1, app_k = -1, app_r = 0;          // wave, step and token row that hold it
  if (p.slot_mapping != nullptr && app_slot >= 0) {
    const int app_pos = L - 1;
    if (app_pos >= start && app_pos < end) {
      app_r = app_pos & 15;  // the block size is a multiple of 16
      const int s_tok = (app_pos - start) >> 4;
      app_w = s_tok % NW;
      app_k = s_tok / NW;
      if (wv == app_w) {
        if (lane < D / 8) {
          *reinterpret_cast<uint2*>(&sm_new[0][8 * lane]) = to_e4m3<T>(krun, p.k_inv_scale);
          *reinterpret_cast<uint2*>(&sm_new[1][8 * lane]) = to_e4m3<T>(vrun, p.v_inv_scale);
        }
        // the same wave reads the codes back in its compute step
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }

  // byte offsets: K token r, dims 8kg.. (+32 B per operand j); V token 4kg, dims JV*r.. (+ one row per token)
  const int koff = r * D + kg * 8;
  const int voff = 4 * kg * D + r * JV;
  const uint8_t* kpool = reinterpret_cast<const uint8_t*>(p.k_cache);
  const uint8_t* vpool = reinterpret_cast<const uint8_t*>(p.v_cache);
  auto load = [&](int k, Fp8Tile<D>& t) {
    int sub = __builtin_amdgcn_readlane(tid, k);
    bad |= sub < 0;
    sub = max(sub, 0);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kpool + static_cast<size_t>(sub) * (16 * D)), 0, -1, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(vpool + static_cast<size_t>(sub) * (16 * D)), 0, -1, kBufferConfig);
#pragma unroll
    for (int j = 0; j < JK; ++j)
      t.k[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, koff, 32 * j, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = VCodes<D>::load(rv, voff, i * D);
  };

  float m = -INFINITY, l = 0.f;
  f32x4 o[JV];
#pragma unroll
  for (int j = 0; j < JV; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int k, Fp8Tile<D>& t) {
    if (k == app_k && wv == app_w) {
      // token row app_r of this sub-tile is the appended token
      if (r == app_r) {
#pragma unroll
        for (int j = 0; j < JK; ++j) t.k[j] = *reinterpret_cast<const u32x2*>(&sm_new[0][kg * 8 + 32 * j]);
      }
      if ((app_r >> 2) == kg) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((app_r & 3) == i) t.v[i] = *reinterpret_cast<const VCodes<D>*>(&sm_new[1][r * JV]);
      }
    }
    u32x2 vop[JV];
    v_operands<T, D>(t.v, vop);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < JK; ++j) sc = Mma<T>::qk(widen8<T>(t.k[j]), qop[j], sc);
    const int nvalid = k < n_w ? min(16, end - (start + 16 * (wv + k * NW))) : 0;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 4 * kg + i < nvalid ? sc[i] * p.scale_log2 : -INFINITY;
    const float lm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__builtin_amdgcn_ballot_w64(lm > m + kLazySlack)) {
      const float mn = fmaxf(m, max_xor32(max_xor16(lm)));
      const float al = fast_exp2(m - mn);
      m = mn;
      l *= al;
#pragma unroll
      for (int j = 0; j < JV; ++j) o[j] *= al;
    }
    const uint32_t p01 = Mma<T>::pack(fast_exp2(x[0] - m), fast_exp2(x[1] - m));
    const uint32_t p23 = Mma<T>::pack(fast_exp2(x[2] - m), fast_exp2(x[3] - m));
    l = Mma<T>::sum2(p23, Mma<T>::sum2(p01, l));
    if (nvalid < 16) {
      const uint32_t m0 = (4 * kg < nvalid ? 0xffffu : 0u) | (4 * kg + 1 < nvalid ? 0xffff0000u : 0u);
      const uint32_t m1 = (4 * kg + 2 < nvalid ? 0xffffu : 0u) | (4 * kg + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        vop[j].x &= m0;
        vop[j].y &= m1;
      }
    }
    const u32x2 pop = {p01, p23};
#pragma unroll
    for (int j = 0; j < JV; ++j) o[j] = Mma<T>::pv(vop[j], pop, o[j]);
  };

  // S register slots, rolling; past the wave's last sub-tile, empty pad steps
  // re-load it (a cache hit) so the loop body is the same every time
  if (n_w > 0) {
    Fp8Tile<D> t[S];
    const int last = n_w - 1;
#pragma unroll
    for (int i = 0; i < S; ++i) load(min(i, last), t[i]);
    const int n_pad = (n_w + S - 1) / S * S;
    int kb = 0;
    for (; kb + S < n_pad; kb += S) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        compute(kb + i, t[i]);
        load(min(kb + i + S, last), t[i]);
      }
    }
    // final round: pad steps leave the state unchanged and are skipped
#pragma unroll
    for (int i = 0; i < S; ++i)
      if (kb + i < n_w) compute(kb + i, t[i]);
  }

  if (p.slot_mapping != nullptr && app_slot >= 0) {
    const int app_pos = L - 1;
    const int off = app_pos - (app_pos / p.block_size) * p.block_size;
    if (static_cast<unsigned>(app_phys) >= static_cast<unsigned>(p.num_blocks) ||
        app_slot != static_cast<int64_t>(app_phys) * p.block_size + off)
      bad = true;
  }

  l = add_xor32(add_xor16(l));
  if (bad) l = __int_as_float(0x7fc00000);
  if (r < G) {
    if (kg == 0) {
      sm_m[wv][r] = m;
      sm_l[wv][r] = l;
    }
#pragma unroll
    for (int j = 0; j < JV; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wv][r][(4 * kg + i) * JV + j] = o[j][i];  // row 4kg+i of O^T is that dim
  }
  __syncthreads();
  combine_and_store<T, D, G, NW, true>(sm_m, sm_l, sm_o, p, w, nparts == 1, p.num_parts);
}

// Sub-tiles in flight per wave, measured on the Llama-3.2-1B batch and the
// LLaMA-2-70B layer: two (4 KB) at head_dim 64 and four (16 KB) at head_dim
// 128; deeper rings measured slower at head_dim 64 (2: 20.4 us, 4: 20.7 us,
// 8: 26.5 us per call on the batch), the register allocation is free (no cap).
template <int D> struct Fp8Shape;
template <> struct Fp8Shape<64> { static constexpr int kDepth = 2, kMinWaves = 2; };
template <> struct Fp8Shape<128> { static constexpr int kDepth = 4, kMinWaves = 2; };

template <typename T, int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int S = Fp8Shape<D>::kDepth, MW = Fp8Shape<D>::kMinWaves;
  int64_t items = static_cast<int64_t>(p.num_seqs) * p.num_parts * p.num_kv_heads;
  if (p.part_tokens > kMaxPartitionTokens) return hipErrorInvalidValue;
  const int nw = (p.num_parts == 1 || p.part_tokens > kFourWaveMaxTokens) ? 8 : 4;
  DecodeParams q = p;
  q.append_wgs = 0;
  if (p.slot_mapping != nullptr) {
    // leading append workgroups, as in the 16-bit launcher: at most 256, a
    // multiple of 8 so that the decode workgroups keep their XCD placement
    const int64_t threads = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * (D / 8);
    int64_t wgs = (threads + nw * kWave - 1) / (nw * kWave);
    wgs = ((wgs < 256 ? wgs : 256) + 7) / 8 * 8;
    q.append_wgs = static_cast<int32_t>(wgs);
    items += wgs;
  }
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  if (nw == 8) {
    hipLaunchKernelGGL((decode_fp8_kernel<T, D, G, 8, S, MW>), dim3(static_cast<unsigned>(items)), dim3(8 * kWave), 0,
                       stream, q);
  } else {
    hipLaunchKernelGGL((decode_fp8_kernel<T, D, G, 4, S, MW>), dim3(static_cast<unsigned>(items)), dim3(4 * kWave), 0,
                       stream, q);
  }
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

hipError_t launch_decode_fp8(const DecodeParams& p, int dtype, hipStream_t stream) {
  const int group = p.num_q_heads / p.num_kv_heads;
  return dtype == 0 ? launch_d<Bf16>(p, group, stream) : launch_d<Fp16>(p, group, stream);
}

}  // namespace pkv
