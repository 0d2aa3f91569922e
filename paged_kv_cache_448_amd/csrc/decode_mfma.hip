// Launchers of the MFMA paged decode kernel (decode_mfma_kernel.h).
#include "decode_mfma_kernel.h"

namespace pkv {

namespace {

// Sub-tiles each wave keeps in flight.
constexpr int kMfmaDepth = 4;

// Whole contexts and partitions above kFourWaveMaxTokens run with 8 waves per
// workgroup, shorter partitions with 4 (each wave may own at most 64
// sub-tiles of a partition).
template <typename T, int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(p.num_seqs) * p.num_parts * p.num_kv_heads;
  if (p.part_tokens > kMaxPartitionTokens) return hipErrorInvalidValue;
  if (p.num_parts == 1 || p.part_tokens > kFourWaveMaxTokens) {
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, 8, kMfmaDepth>), dim3(static_cast<unsigned>(items)),
                       dim3(8 * kWave), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, 4, kMfmaDepth>), dim3(static_cast<unsigned>(items)),
                       dim3(4 * kWave), 0, stream, p);
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
