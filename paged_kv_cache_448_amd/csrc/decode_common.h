// Pieces shared by the decode kernels: work-item decoding, sequence checks and
// the workgroup epilogue that folds the waves' partial softmax states together.
//
// Every wave keeps an online-softmax state over the tokens it saw: a running
// maximum m (log2 units, scale folded in), a denominator l and an unnormalised
// accumulator o = sum_t 2^(s_t - m) v_t.  States combine exactly by the
// log-sum-exp identity: with M = max_w m_w,
//   l = sum_w 2^(m_w - M) l_w,   o = sum_w 2^(m_w - M) o_w,   out = o / l.
// The same identity merges the partitions of a long context in merge.hip.
#pragma once

#include "common.h"
#include "kernels.h"

namespace pkv {

struct WorkItem {
  int seq, kvh, part;
  bool wave;  // wave mode (work lists only): wave w takes kv head kvh + w alone
};

// Items are ordered (work slot, partition, kv head), or one work-list entry
// per workgroup; see xcd_remap for the workgroup -> item order.  Work slot s is sequence s, or seq_order[s] when
// the caller passes a dispatch order (a host schedule that balances the XCDs'
// work and starts long contexts first).  bid / n: this workgroup's index among
// the n decode workgroups of the launch.  An order entry outside
// [0, num_seqs) gives seq = -1: the workgroup does nothing.
// LIST: the kernel takes work lists (p.work); without, p.work is not read.
template <bool LIST = false>
__device__ __forceinline__ WorkItem decode_item(const DecodeParams& p, int bid, int n,
                                                const DecodeExt& x = DecodeExt{}) {
  WorkItem w;
  w.wave = false;
  if (LIST && x.work != nullptr) {
    // entry bid of the work list: one per workgroup; an entry outside the
    // grid is skipped
    const int e = xcd_remap(bid, n);
    const int s = x.work[2 * e];
    const uint32_t y = static_cast<uint32_t>(x.work[2 * e + 1]);
    const int part = static_cast<int>(y & 0xffffu), kvh = static_cast<int>((y >> 16) & 0x7fffu);
    const bool ok = static_cast<unsigned>(s) < static_cast<unsigned>(p.num_seqs) && part < p.num_parts &&
                    kvh < p.num_kv_heads;
    w.seq = ok ? s : -1;
    w.part = ok ? part : 0;
    w.kvh = ok ? kvh : 0;
    w.wave = (y >> 31) != 0;
    return w;
  }
  int it = xcd_remap(bid, n);
  w.kvh = it % p.num_kv_heads;
  it /= p.num_kv_heads;
  w.part = it % p.num_parts;
  w.seq = it / p.num_parts;
  if (p.seq_order != nullptr) {
    const int s = p.seq_order[w.seq];
    w.seq = static_cast<unsigned>(s) < static_cast<unsigned>(p.num_seqs) ? s : -1;
  }
  return w;
}

// A context length the kernel must not trust: outside [0, max_context_len] or
// beyond what the block table can hold.
__device__ __forceinline__ bool bad_length(int L, const DecodeParams& p) {
  return L < 0 || L > p.max_context_len ||
         static_cast<int64_t>(L) > static_cast<int64_t>(p.max_blocks_per_seq) * p.block_size;
}

// The shared-prefix length pl of a sequence of length L is usable when it is
// 0, or a positive multiple of 16 before the sequence's last position (so the
// token appended this step is never in it) and within the launch's bound.
__device__ __forceinline__ bool prefix_ok(int pl, int L, const DecodeExt& x) {
  return pl == 0 || (pl > 0 && (pl & 15) == 0 && pl <= L - 1 && pl <= x.max_prefix_len);
}

// Prefix length of sequence seq (0 without prefixes); -1 when unusable.
__device__ __forceinline__ int seq_prefix(const DecodeExt& x, int seq, int L) {
  if (x.prefix_len == nullptr) return 0;
  const int pl = x.prefix_len[seq];
  return prefix_ok(pl, L, x) ? pl : -1;
}

// For an empty or invalid sequence the workgroup of partition 0 writes the
// G heads' output (zeros or NaN); the others do nothing.
// tid / nt: this thread's index among the nt threads that share the writing.
template <typename T, int G, int NT>
__device__ __forceinline__ void write_degenerate(const DecodeParams& p, const WorkItem& w, bool bad,
                                                 int tid = threadIdx.x, int nt = NT) {
  if (w.part != 0) return;
  const int D = p.head_dim;
  const uint16_t v = bad ? kNanBits<T> : 0;
  uint16_t* o = p.out + (static_cast<size_t>(w.seq) * p.num_q_heads + w.kvh * G) * D;
  for (int i = tid; i < G * D; i += nt) o[i] = v;
}

// Fold NW waves' states (in LDS) and store either the final output (the whole
// context was one partition) or this partition's partial state (slots per row
// of the partial arrays).  kScaleOut:
// the accumulator is multiplied by p.out_scale first (partials carry it, so
// the merge needs nothing).
template <typename T, int D, int G, int NW, bool kScaleOut = false>
__device__ __forceinline__ void combine_and_store(const float (*sm_m)[G], const float (*sm_l)[G],
                                                  const float (*sm_o)[G][D], const DecodeParams& p,
                                                  const WorkItem& w, bool single,
                                                  int slots) {
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
    float lt = 0.f, o = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float c = fast_exp2(sm_m[k][h] - M);
      lt = fmaf(c, sm_l[k][h], lt);
      o = fmaf(c, sm_o[k][h][d], o);
    }
    if (kScaleOut) o *= p.out_scale;
    const size_t row = static_cast<size_t>(w.seq) * p.num_q_heads + w.kvh * G + h;
    if (single) {
      p.out[row * D + d] = to_bits<T>(o / lt);
    } else {
      const size_t pr = row * slots + w.part;
      p.part_o[pr * D + d] = o;
      if (d == 0) {
        p.part_m[pr] = M;
        p.part_l[pr] = lt;
      }
    }
  }
}

// Output element (row = sequence * Hq + q head, dim d) of a split context,
// folded from the row's partial states in slot order -- the first nparts
// partition slots, then nprefix prefix slots from slot num_parts on -- with
// the log-sum-exp identity, as a running (M, l, o) so that all loads of a row
// can be in flight together.
template <int D>
__device__ __forceinline__ float merge_row_elem(const DecodeParams& p, const DecodeExt& x, size_t row, int d,
                                                int nparts, int nprefix) {
  const size_t base = row * x.num_slots;
  float M = -INFINITY, lt = 0.f, o = 0.f;
  const int n = nparts + nprefix;
#pragma unroll 4
  for (int i = 0; i < n; ++i) {
    const size_t k = base + (i < nparts ? i : p.num_parts + (i - nparts));
    const float mk = p.part_m[k], lk = p.part_l[k], ok = p.part_o[k * D + d];
    const float mn = fmaxf(M, mk);
    const float a = fast_exp2(M - mn), b = fast_exp2(mk - mn);
    lt = fmaf(lt, a, lk * b);
    o = fmaf(o, a, ok * b);
    M = mn;
  }
  return o / lt;
}

}  // namespace pkv
