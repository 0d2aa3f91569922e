// Launchers of the MFMA paged decode kernel (decode_mfma_kernel.h).
#include "decode_mfma_kernel.h"

namespace pkv {

namespace {

// Sub-tiles each wave keeps in flight, and the waves per SIMD the register
// allocation must leave room for (measured on the Llama-3.2-1B batch and the
// LLaMA-2-70B layer): four sub-tiles (16 KB) at head_dim 64, two sub-tiles
// (16 KB) at head_dim 128; both at three waves per SIMD (the kernel caps it
// there: four measured slower at head_dim 64; at head_dim 128 three is the
// most that does not spill).
template <int D> struct MfmaShape;
template <> struct MfmaShape<64> { static constexpr int kDepth = 4, kMinWaves = 2; };
template <> struct MfmaShape<128> { static constexpr int kDepth = 2, kMinWaves = 3; };

// Whole contexts and partitions above kFourWaveMaxTokens run with 8 waves per
// workgroup, shorter partitions with 4 (each wave may own at most 64
// sub-tiles of a partition).
template <typename T, int D, int G>
hipError_t launch_t(const DecodeParams& p, const DecodeExt& x, hipStream_t stream) {
  constexpr int S = MfmaShape<D>::kDepth, W = MfmaShape<D>::kMinWaves;
  int64_t items = x.work != nullptr ? static_cast<int64_t>(x.num_work)
                                     : static_cast<int64_t>(p.num_seqs) * p.num_parts * p.num_kv_heads;
  if (p.part_tokens > kMaxPartitionTokens) return hipErrorInvalidValue;
  const int nw = decode_workgroup_waves(p.num_parts, p.part_tokens);
  DecodeParams q = p;
  q.append_wgs = 0;
  if (p.slot_mapping != nullptr) {
    // leading append workgroups: one thread per (token, kv head, 8-dim run),
    // at most 256 workgroups, a multiple of 8 so the decode workgroups keep
    // their XCD placement
    const int64_t threads = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * (D / 8);
    int64_t wgs = (threads + nw * kWave - 1) / (nw * kWave);
    wgs = ((wgs < 256 ? wgs : 256) + 7) / 8 * 8;
    q.append_wgs = static_cast<int32_t>(wgs);
    items += wgs;
  }
  DecodeExt xq = x;
  xq.prefix_wgs = 0;
  if (x.prefix_len != nullptr) {
    // shared-prefix units, one per wave, in a multiple of 8 workgroups (as the
    // append ones) right after the append workgroups
    const int64_t units = static_cast<int64_t>(x.num_prefix_items) * p.num_kv_heads * x.prefix_chunks;
    const int64_t wgs = ((units + nw - 1) / nw + 7) / 8 * 8;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    xq.prefix_wgs = static_cast<int32_t>(wgs);
    items += wgs;
  }
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(items));
  if (x.prefix_len != nullptr || x.work != nullptr) {
    if (nw == 8) {
      hipLaunchKernelGGL((decode_mfma_ext_kernel<T, D, G, 8, S, W>), grid, dim3(8 * kWave), 0, stream, q, xq);
    } else {
      hipLaunchKernelGGL((decode_mfma_ext_kernel<T, D, G, 4, S, W>), grid, dim3(4 * kWave), 0, stream, q, xq);
    }
  } else if (nw == 8) {
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, 8, S, W>), grid, dim3(8 * kWave), 0, stream, q);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, 4, S, W>), grid, dim3(4 * kWave), 0, stream, q);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DecodeParams& p, const DecodeExt& x, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(p, x, stream);
    case 2: return launch_t<T, D, 2>(p, x, stream);
    case 4: return launch_t<T, D, 4>(p, x, stream);
    case 8: return launch_t<T, D, 8>(p, x, stream);
    case 16: return launch_t<T, D, 16>(p, x, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_d(const DecodeParams& p, const DecodeExt& x, int group, hipStream_t stream) {
  return p.head_dim == 64 ? launch_g<T, 64>(p, x, group, stream) : launch_g<T, 128>(p, x, group, stream);
}

}  // namespace

bool mfma_supported(int dtype, int head_dim, int group) {
  (void)dtype;
  if (head_dim != 64 && head_dim != 128) return false;
  return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
}

hipError_t launch_decode_mfma(const DecodeParams& p, const DecodeExt& x, int dtype, hipStream_t stream) {
  const int group = p.num_q_heads / p.num_kv_heads;
  return dtype == 0 ? launch_d<Bf16>(p, x, group, stream) : launch_d<Fp16>(p, x, group, stream);
}

}  // namespace pkv
