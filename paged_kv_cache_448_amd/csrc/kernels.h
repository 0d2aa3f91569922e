// Kernel parameter blocks and launchers (internal to the library; the public
// interface is include/pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct AppendParams {
  const uint16_t* k;            // [T, Hkv, D]
  const uint16_t* v;            // [T, Hkv, D]
  const int64_t* slot_mapping;  // [T]
  uint16_t* k_cache;
  uint16_t* v_cache;
  int32_t num_tokens, num_blocks, block_size, num_kv_heads, head_dim;
};

// FP8 (E4M3) append: 16-bit rows in, one byte per element out, each element
// rounded to the nearest code of x * inv_scale (saturating, NaN -> 0x7F).
struct AppendFp8Params {
  const uint16_t* k;            // [T, Hkv, D], 16-bit (src_fp16 selects fp16, else bf16)
  const uint16_t* v;
  const int64_t* slot_mapping;  // [T]
  uint8_t* k_cache;             // [N, Hkv, bs, D] codes
  uint8_t* v_cache;
  float k_inv_scale, v_inv_scale;
  int32_t num_tokens, num_blocks, block_size, num_kv_heads, head_dim, src_fp16;
};

struct DecodeParams {
  const uint16_t* q;             // [B, Hq, D]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;   // [B, max_blocks_per_seq]
  const int32_t* context_lens;   // [B]
  uint16_t* out;                 // [B, Hq, D]
  float* part_o;                 // [B, Hq, slots, D]  (only when slots > 1): slots = num_parts,
  float* part_m;                 // [B, Hq, slots]     or DecodeExt::num_slots; running max (log2 units)
  float* part_l;                 // [B, Hq, slots]     softmax denominator
  // Fused append (MFMA kernel only): token i of this step, k_new[i] / v_new[i]
  // ([B, Hkv, D]), goes into slot slot_mapping[i], which must be the slot of
  // position L_i - 1 of sequence i; slot_mapping == nullptr: no append.
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* slot_mapping;   // (the append writes through k_cache and v_cache)
  int32_t append_wgs;            // leading workgroups that store the appended tokens (fused append), else 0
  // Fused append into FP8 pools: the reciprocals of the pool scales, as
  // kv_append_fp8 multiplies by them (unused otherwise).
  float k_inv_scale, v_inv_scale;
  // Dispatch order (optional): work slot s decodes sequence seq_order[s], a
  // permutation of [0, num_seqs); nullptr = slot s is sequence s.
  const int32_t* seq_order;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
  int32_t max_blocks_per_seq, max_context_len;
  int32_t part_tokens;           // tokens per partition, a multiple of 16
  int32_t num_parts;             // ceil(max_context_len / part_tokens), >= 1
  float scale_log2;              // softmax scale * log2(e) (FP8 pools: times the K scale)
  float out_scale;               // factor on every output (FP8 pools: the V scale; else 1)
};

// Extensions of the MFMA decode launch (shared prefixes, work lists), a
// second kernel argument of the kernel that takes them: the plain decode's
// argument block stays as small as it is (a larger one measured 0.3 us slower
// per launch on the Llama-3.2-1B batch).  Zero-initialised: none.
struct DecodeExt {
  // Shared prefixes (MFMA kernel, 16-bit pools; prefix_len == nullptr: none).
  // Sequence i's first prefix_len[i] tokens are blocks it shares with the
  // other members of one prefix item; prefix work units read them once per
  // item, the regular work items take positions prefix_len[i] .. L_i - 1.
  // Item k's members are prefix_items[16k .. 16k+15] (-1: unused), member 0
  // the reference whose block-table row the units read.
  const int32_t* prefix_len;     // [B]
  const int32_t* prefix_items;   // [num_prefix_items][16]
  int32_t num_prefix_items;
  int32_t max_prefix_len;        // host bound of every prefix_len[i]
  int32_t prefix_chunk;          // prefix tokens per unit (one wave), multiple of 16, <= 1024
  int32_t prefix_chunks;         // ceil(max_prefix_len / prefix_chunk), 0 without prefixes
  int32_t prefix_wgs;            // workgroups of prefix units (after the append ones)
  // Partial-state slots per (sequence, q head): partitions 0 .. num_parts-1 of
  // the regular items, then prefix chunk c at slot num_parts + c.
  int32_t num_slots;
  // Work list (optional, MFMA kernel): one entry per workgroup, replacing the
  // (slot, partition, kv head) grid, so partitions past a sequence's end are
  // never launched.  Entry e: work[2e] = sequence (-1: skip), work[2e+1] =
  // partition | kv head << 16 | wave mode << 31.  In wave mode wave w takes
  // kv head + w of the partition alone (at most 64 sub-tiles), with no
  // workgroup barrier.  nullptr: the full grid.
  const int32_t* work;
  int32_t num_work;
};

// Paged prefill: the new tokens of every sequence, packed (sequence i's at rows
// query_start[i] .. query_start[i+1]-1), attend causally over the paged context.
struct PrefillParams {
  const uint16_t* q;             // [T, Hq, D]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;   // [B, max_blocks_per_seq]
  const int32_t* context_lens;   // [B]
  const int32_t* query_start;    // [B + 1]
  uint16_t* out;                 // [T, Hq, D]
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
  int32_t max_blocks_per_seq, max_context_len, max_query_len;
  int32_t chunks;                // work chunks per (sequence, kv head); set by the launcher
  float scale_log2;              // softmax scale * log2(e)
};

// Most tokens one decode workgroup takes (both kernels); longer contexts are
// always split.  The MFMA kernel's waves hold the pool index of each of their
// 16-token sub-tiles in one lane each: 8 waves x 64 lanes x 16 tokens.
constexpr int32_t kMaxPartitionTokens = 8192;
// Partitions longer than this run with 8 waves per workgroup, shorter ones with 4.
constexpr int32_t kFourWaveMaxTokens = 4096;
// Waves per workgroup of the MFMA decode launch: eight for a single pass or
// partitions above kFourWaveMaxTokens, four for shorter partitions.
constexpr int decode_workgroup_waves(int32_t num_parts, int32_t part_tokens) {
  return (num_parts == 1 || part_tokens > kFourWaveMaxTokens) ? 8 : 4;
}
// Partitions of at most this many tokens go to wave mode in a work list
// (at most 64 sub-tiles: a wave holds one sub-tile id per lane).  On the
// 16-layer step 256 measured best (128: +0.4 us, 512: +4.6, 1024: +9.3 per layer).
constexpr int32_t kWaveModeMaxTokens = 256;

// Column groups of a shared-prefix unit (two at head_dim 64, one at 128, at
// most G), and so the members of a prefix item: column groups * 16/G <= 16.
constexpr int prefix_column_groups(int head_dim, int group) {
  return (head_dim == 64 ? 2 : 1) < group ? (head_dim == 64 ? 2 : 1) : group;
}
constexpr int prefix_members_per_item(int head_dim, int group) {
  return prefix_column_groups(head_dim, group) * (16 / group);
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_kv_append_fp8(const AppendFp8Params& p, hipStream_t stream);

bool simt_supported(int dtype, int head_dim, int group);
hipError_t launch_decode_simt(const DecodeParams& p, int dtype, hipStream_t stream);

bool mfma_supported(int dtype, int head_dim, int group);
hipError_t launch_decode_mfma(const DecodeParams& p, const DecodeExt& x, int dtype, hipStream_t stream);

// FP8 (E4M3) pools (k_cache / v_cache hold one code per element); no fused append.
hipError_t launch_decode_fp8(const DecodeParams& p, int dtype, hipStream_t stream);

hipError_t launch_prefill_mfma(const PrefillParams& p, int dtype, hipStream_t stream);

// x: the extensions of the decode launch before it (shared prefixes; its
// partial-state slots per row)
hipError_t launch_merge(const DecodeParams& p, const DecodeExt& x, int dtype, hipStream_t stream);

// Size of the device scratch of the allocation-free decode entry point
// (split-context partial states): 16 MiB per GPU.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
// That scratch's device address on the current device (looked up once per
// device); hipError on failure.
hipError_t noalloc_scratch(void** ptr);

}  // namespace pkv
