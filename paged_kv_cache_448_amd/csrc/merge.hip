// Merge pass of split-context decode: combine the per-partition softmax
// states of a sequence into its output with the log-sum-exp identity
// (see decode_common.h), together with the states of its shared-prefix chunks
// when it has one.  One wave per (sequence, q head); lane l owns dims l and
// l+64.  States are folded in slot order, so the result does not depend on
// which workgroup finished first.
//
// The pages never split a context; this pass exists because on one GPU a few
// long sequences alone cannot fill 256 compute units.
#include "decode_common.h"

namespace pkv {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p, DecodeExt x) {
  constexpr int DV = D / 64;
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;  // seq * Hq + q head
  if (row >= p.num_seqs * p.num_q_heads) return;
  const int seq = row / p.num_q_heads;
  const int L = p.context_lens[seq];
  if (bad_length(L, p) || L == 0) return;  // written by the partition kernel
  const int pl = seq_prefix(x, seq, L);
  if (pl < 0) return;                      // unusable prefix length: NaN written by the partition kernel
  const int np = (L - pl + p.part_tokens - 1) / p.part_tokens;
  const int npre = pl > 0 ? (pl + x.prefix_chunk - 1) / x.prefix_chunk : 0;
  if (np + npre <= 1) return;              // one pass over the whole context wrote the output
#pragma unroll
  for (int e = 0; e < DV; ++e)
    p.out[static_cast<size_t>(row) * D + lane + 64 * e] =
        to_bits<T>(merge_row_elem<D>(p, x, row, lane + 64 * e, np, npre));
}

template <typename T, int D>
hipError_t launch_t(const DecodeParams& p, const DecodeExt& x, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(p.num_seqs) * p.num_q_heads;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, p, x);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeParams& p, const DecodeExt& x, int dtype, hipStream_t stream) {
  if (dtype == 0) return p.head_dim == 64 ? launch_t<Bf16, 64>(p, x, stream) : launch_t<Bf16, 128>(p, x, stream);
  return p.head_dim == 64 ? launch_t<Fp16, 64>(p, x, stream) : launch_t<Fp16, 128>(p, x, stream);
}

}  // namespace pkv
