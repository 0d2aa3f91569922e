/*
 * pkv.h -- C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * Device operations:
 *
 *   pkv_kv_append          writes the K/V of new tokens into their cache slots;
 *   pkv_paged_attn_decode  single-token attention of every sequence over its
 *                          cached context, read block by block through a
 *                          per-sequence block table, with GQA head sharing
 *                          (_ex: tuning knobs; pkv_append_paged_attn_decode:
 *                          both in one launch);
 *   pkv_paged_prefill      causal attention of many new tokens per sequence
 *                          over the same paged context;
 *   pkv_kv_append_fp8, pkv_paged_attn_decode_fp8
 *                          the append and the decode over FP8 (E4M3) pools.
 *
 * What they compute follows the pages this library was written from:
 * the KV cache is cut into fixed-size blocks, logical blocks of a sequence map
 * to physical blocks anywhere in a pool, blocks are handed out as tokens arrive
 * ("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린 서빙 엔진", section
 * "PagedAttention -- OS 가상 메모리에서 영감"); K and V of past tokens are kept
 * per layer and head so decode only reads them (same page, sections "KV Cache가
 * 왜 병목인가" and "Prefill vs Decode"); attention is softmax(scale q K^T) V with
 * several q heads sharing one kv head ("[Hacker News 요약] C++와 CUDA로 vLLM의
 * 경량 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을 위한
 * 고급 최적화 기법").  Block metadata (the host allocator, pkv_alloc.h) lives on
 * the CPU and the KV tensors on the GPU ("Nano-vLLM로 배우는 vLLM 추론 엔진 작동
 * 원리 한눈에 정리", section "KV 캐시와 Block Manager").
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are device pointers to contiguous row-major memory,
 *   16-byte aligned, owned by the caller.  The library never allocates or frees
 *   device memory, never synchronises, and never reads device memory on the
 *   host: it validates its scalar arguments, then enqueues kernels on `stream`
 *   (NULL = the default stream) and returns.  Calls on different streams may
 *   run concurrently; calls are stateless.
 * - Element type `dtype` is PKV_BF16 or PKV_FP16 and is the same for q, the
 *   new k/v, both caches and out.  Arithmetic is fp32.
 * - Status: PKV_OK or a negative code (see pkv_status_str).  Argument errors
 *   are reported before anything is enqueued; PKV_E_HIP means a launch failed.
 *
 * Cache layout (both caches hold N blocks of bs tokens, bs a multiple of 16;
 * the block is the outermost index, so block n is one contiguous range):
 *
 *   k_cache, v_cache: [N][Hkv][bs][D]   K[n,h,t,d] and V[n,h,t,d] at
 *            ((n*Hkv + h)*bs + t)*D + d
 *
 * i.e. one token's K (or V) for one kv head is one contiguous row of D
 * elements, so appending a token writes two rows.  A slot is
 * n*bs + t (block n, token t of the block).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "pkv_status.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { PKV_BF16 = 0, PKV_FP16 = 1 };

/* Decode kernel selection for pkv_paged_attn_decode_ex. */
enum { PKV_IMPL_AUTO = 0, PKV_IMPL_SIMT = 1, PKV_IMPL_MFMA = 2 };

/* Human-readable name of a status code (static string). */
const char* pkv_status_str(int status);

/*
 * pkv_kv_append -- store the K and V of num_tokens new tokens.
 *
 * Each generated token's K and V are kept for every later step, in the block
 * and offset its slot names ("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배
 * 끌어올린 서빙 엔진", sections "KV Cache가 왜 병목인가" (K and V kept per layer
 * and head for all past tokens) and "PagedAttention -- OS 가상 메모리에서 영감"
 * (tokens go into fixed-size blocks taken as they arrive)).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  [num_tokens] int64: slot of each token; a negative slot means
 *                 "padding token, write nothing"; a slot >= num_blocks*block_size
 *                 is ignored as well (never written).  Non-negative slots must be
 *                 distinct (caller precondition; with duplicates the surviving
 *                 value is unspecified).
 *   k_cache, v_cache  the pools described above, updated in place.  Only the
 *                 bytes of the written slots change.
 *
 * Supported: head_dim a multiple of 8 up to 512, block_size a multiple of 16
 * up to 1024, any number of kv heads.  The copy is bit-exact.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (negative sizes, misaligned pointers),
 * PKV_E_UNSUPPORTED, PKV_E_HIP.
 */
int pkv_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                  void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size,
                  int32_t num_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream);

/*
 * pkv_decode_workspace_bytes -- device workspace that pkv_paged_attn_decode
 * needs for these sizes (0 when no context is split).  With the automatic
 * plan the result covers every call with the same sizes and a max_context_len
 * up to this one (the plan of a shorter bound may use more partitions), so a
 * workspace sized once for the largest bound serves a whole decode loop.  The
 * _ex form takes the same partition_tokens as pkv_paged_attn_decode_ex.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_context_len);
size_t pkv_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                     int32_t partition_tokens);

/*
 * pkv_paged_attn_decode -- out = softmax(scale * q K^T) V for each sequence.
 *
 * Decode: the one new token of each sequence attends to every cached token of
 * its context, read from the KV cache rather than recomputed ("vLLM --
 * PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린 서빙 엔진", section "Prefill vs
 * Decode"); the context is found block by block through the sequence's block
 * table (same page, section "PagedAttention -- OS 가상 메모리에서 영감"); the
 * formula, the causal mask (for the last position: every cached token) and GQA
 * head sharing are those of "[Hacker News 요약] C++와 CUDA로 vLLM의 경량 고성능
 * LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을 위한 고급 최적화
 * 기법".
 *
 *   q             [num_seqs][num_q_heads][head_dim]: the query of the token
 *                 being decoded.  q head h reads kv head h / G, G = Hq / Hkv.
 *   k_cache, v_cache  pools of num_blocks blocks (layout above).
 *   block_tables  [num_seqs][max_blocks_per_seq] int32: physical block of each
 *                 logical block.  Entries at or past ceil(L_i / block_size) are
 *                 never read.
 *   context_lens  [num_seqs] int32: L_i, the number of cached tokens attended
 *                 to (positions 0 .. L_i-1; includes the token appended this
 *                 step).  Tail slots of a last block and unused blocks may hold
 *                 anything, NaN included: they never reach the output.
 *   max_context_len  host-side upper bound of every L_i; must not exceed
 *                 max_blocks_per_seq * block_size.  Sizes the partitioning.
 *   scale         softmax scale (typically 1/sqrt(head_dim)).
 *   out           [num_seqs][num_q_heads][head_dim], written in `dtype`
 *                 (fp32 result rounded to nearest even).
 *   workspace     device scratch of at least pkv_decode_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0).  Contents on entry do
 *                 not matter; it holds per-partition partial results.
 *
 * Result for a sequence with L_i = 0: zeros.  A sequence whose L_i is
 * negative, above max_context_len or above max_blocks_per_seq * block_size,
 * or whose table names a block outside [0, num_blocks), gets NaN in the
 * affected heads instead of a memory access outside the pool.
 *
 * Supported: head_dim 64 or 128; block_size a multiple of 16 up to 1024;
 * G in {1, 2, 4, 8, 16} (the SIMT kernel: G * head_dim <= 512).
 * Errors: PKV_E_NULL, PKV_E_SHAPE, PKV_E_UNSUPPORTED, PKV_E_WORKSPACE, PKV_E_HIP.
 */
int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float scale,
                          void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_paged_attn_decode_noalloc -- pkv_paged_attn_decode with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The
 * split-context partial states live in a library-owned device array of 16 MiB
 * per GPU (allocated when the library's code is loaded on that GPU, held until
 * the process ends); the call itself allocates and frees nothing.  Results
 * are bit-identical to pkv_paged_attn_decode with the automatic plan.
 *
 *   arguments as pkv_paged_attn_decode, without workspace / workspace_bytes.
 *
 * Every call on one GPU uses that GPU's one array, so calls that overlap on
 * one GPU (concurrent streams, or host threads) race and give undefined
 * results: serialise them (one stream, or events).  Nothing in the array needs
 * to start at zero.  PKV_E_WORKSPACE when the plan's partial states
 * (num_seqs * num_q_heads * partitions * (head_dim + 2) * 4 bytes, rounded up)
 * exceed 16 MiB.  Other errors as pkv_paged_attn_decode.
 */
int pkv_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t dtype, hipStream_t stream);

/*
 * pkv_paged_attn_decode_ex -- as above, with two tuning knobs:
 *   partition_tokens  0 = automatic; otherwise a multiple of 16: the context of
 *                     each sequence is cut into partitions of this many tokens,
 *                     each processed by its own workgroup, and the partial
 *                     results are combined by a log-sum-exp merge pass.  A value
 *                     >= max_context_len means a single pass without merge.
 *                     Partitions are at most 8192 tokens: larger values (and a
 *                     single pass over longer contexts) are cut to 8192.
 *   impl              PKV_IMPL_AUTO, PKV_IMPL_SIMT (vector-ALU dot products) or
 *                     PKV_IMPL_MFMA (matrix-core tiles).
 *   seq_order         NULL, or a device array [num_seqs] int32: the dispatch
 *                     order, a permutation of 0 .. num_seqs-1 (work slot s
 *                     decodes sequence seq_order[s]); pkv_decode_schedule makes
 *                     one from the host's copy of the context lengths.  It
 *                     changes only which workgroup decodes which sequence:
 *                     outputs stay indexed by sequence and are bit-identical to
 *                     those without an order.  Not a permutation: the output
 *                     rows of sequences no slot names are unspecified (entries
 *                     outside [0, num_seqs) are skipped; a repeated entry
 *                     decodes its sequence twice); nothing is read or written
 *                     outside the caller's buffers.
 * Results of all choices agree to fp32 rounding.
 */
int pkv_paged_attn_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len, float scale,
                             void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                             void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                             int32_t impl, const int32_t* seq_order, hipStream_t stream);

/*
 * pkv_append_paged_attn_decode -- one decode step of one layer in a single
 * launch: pkv_kv_append of one new token per sequence, then
 * pkv_paged_attn_decode over contexts that include it.
 *
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim]: K and V of the token
 *                 being decoded by each sequence.
 *   slot_mapping  [num_seqs] int64: slot_mapping[i] is the slot of position
 *                 context_lens[i] - 1 of sequence i (its last block-table
 *                 block, offset (L_i - 1) % block_size), where the token is
 *                 written; a negative slot means "append nothing for this
 *                 sequence".  That slot must lie in no other sequence's
 *                 context (a block manager guarantees it for the block a
 *                 sequence is still filling).
 *   the other arguments are those of pkv_paged_attn_decode_ex (MFMA kernel),
 *   seq_order included.
 *
 * Results, when the preconditions hold: the pools and out are bit-identical
 * to pkv_kv_append(k_new, v_new, slot_mapping, B, ...) followed by
 * pkv_paged_attn_decode_ex(..., impl = PKV_IMPL_MFMA).  A non-negative slot
 * that is not the slot of position L_i - 1 (or a sequence with L_i = 0 and a
 * slot) writes nothing and makes sequence i's output NaN; the kernel cannot
 * report it otherwise.
 * Supported: as the MFMA kernel (pkv_decode_supported(PKV_IMPL_MFMA, ...)).
 * Errors: PKV_E_NULL, PKV_E_SHAPE, PKV_E_UNSUPPORTED, PKV_E_WORKSPACE, PKV_E_HIP.
 */
int pkv_append_paged_attn_decode(const void* q, const void* k_new, const void* v_new,
                                 const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t dtype, void* workspace,
                                 size_t workspace_bytes, int32_t partition_tokens, const int32_t* seq_order,
                                 hipStream_t stream);

/*
 * pkv_decode_plan_partition -- the partition size (tokens) the automatic choice
 * would use for these sizes; 0 means a single pass.
 */
int32_t pkv_decode_plan_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                  int32_t max_context_len);

/*
 * pkv_decode_schedule -- a dispatch order for the decode calls' seq_order,
 * computed on the host from the host's copy of the context lengths (a block
 * manager keeps them: it hands out the block tables).  Host memory only; no
 * device call.
 *
 * The pages fix what decode computes, not how work is spread over the GPU;
 * this is a scheduling aid that leaves every output bit unchanged.  A launch
 * gives each of the MI355X's 8 XCDs a contiguous range of work slots; the
 * order deals the sequences, longest first, each to the XCD group with the
 * fewest tokens so far that has room (group x holds ceil(B/8) slots for
 * x < B % 8, floor(B/8) otherwise), and keeps each group longest first, so the
 * XCDs get about equal work and each starts its long contexts first.
 *
 *   context_lens  [num_seqs] int32, host memory (negative values count as 0)
 *   seq_order     [num_seqs] int32, host memory, written: a permutation of
 *                 0 .. num_seqs-1.
 * Errors: PKV_E_SHAPE (num_seqs < 0), PKV_E_NULL.
 */
int pkv_decode_schedule(const int32_t* context_lens, int32_t num_seqs, int32_t* seq_order);

/*
 * Shared prefixes read once.  Sequences that share prompt-prefix blocks by
 * reference ("Nano-vLLM로 배우는 vLLM 추론 엔진 작동 원리 한눈에 정리", section
 * "KV 캐시와 Block Manager": identical prefix blocks are reused instead of
 * stored again; a block manager hands out such tables) hold the same K/V in
 * those blocks.  The decode below reads such a prefix once for a whole
 * prefix item of up to 16 sequences instead of once per sequence; results
 * equal those of pkv_paged_attn_decode up to fp32 rounding order.
 *
 * pkv_decode_prefix_plan -- find the items from the host's copy of the block
 * tables and context lengths (host memory only; no device call).
 *
 *   block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
 *   num_kv_heads, head_dim, block_size: as the decode call takes them (the
 *                 lengths include the token appended this step).
 *   prefix_len    [num_seqs] int32, written: shared tokens of each sequence
 *                 (0: none), a multiple of block_size; only blocks that are
 *                 full before the sequence's last position are shared.
 *   prefix_items  [max_items][16] int32, written: the members of each item
 *                 (-1 pads), member 0 the reference whose table row the
 *                 kernel reads; every sequence with prefix_len > 0 is in
 *                 exactly one item, and its first prefix_len / block_size
 *                 table entries equal the reference's.  num_seqs / 2 items
 *                 always suffice.  Members per item: 16/G column slots per
 *                 column group, two column groups at head_dim 64 and one at
 *                 128 (at most G).
 *   num_items, max_prefix_len  written: items found, longest prefix_len.
 * Rows sharing their first block are grouped (rows sorted block by block);
 * an item ends at the member limit or at a row that does not share its
 * reference's first block.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (max_items too small, bad sizes),
 * PKV_E_UNSUPPORTED (as the MFMA kernel).
 */
int pkv_decode_prefix_plan(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t* prefix_len, int32_t* prefix_items, int32_t max_items,
                           int32_t* num_items, int32_t* max_prefix_len);

/*
 * pkv_decode_prefix_workspace_bytes -- workspace of pkv_paged_attn_decode_prefix
 * (the partition states plus one state per prefix chunk per sequence and q
 * head); max_prefix_len 0 gives pkv_decode_workspace_bytes_ex.
 */
size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                         int32_t max_prefix_len, int32_t partition_tokens);

/*
 * pkv_paged_attn_decode_prefix -- pkv_paged_attn_decode (MFMA kernel, 16-bit
 * pools) with shared prefixes read once per item, optionally with the step's
 * append fused in as pkv_append_paged_attn_decode (slot_mapping NULL: no
 * append; k_new / v_new unused then).
 *
 *   prefix_len, prefix_items  device copies of pkv_decode_prefix_plan's
 *                 output (or arrays with the same properties);
 *   num_prefix_items, max_prefix_len  its counts (host values).  Either 0:
 *                 the plain decode (prefix_len is not read).
 *   workspace     at least pkv_decode_prefix_workspace_bytes(...) bytes.
 *   work, num_work  NULL / 0, or a device copy of pkv_decode_work_list's
 *                 output for the same lengths, prefix lengths, max_context_len
 *                 and partition_tokens: only the partitions listed are
 *                 launched (in that order; seq_order is then not used).
 *   the other arguments as pkv_append_paged_attn_decode.
 *
 * Sequence i's positions 0 .. prefix_len[i]-1 are read from its item's
 * reference row, the rest from its own.  The kernel checks each member's
 * table against the reference row over the blocks it reads for it; a
 * sequence whose table differs there, whose prefix_len is not a multiple of
 * 16, not below L_i or above max_prefix_len or the reference's own, gets NaN
 * instead.  A sequence with prefix_len > 0 that is in no item, or in two,
 * gets an unspecified output (the item list is the caller's to keep).
 * Positions a member masks are still multiplied by probability 0 in P.V, so
 * cached values must be finite.
 * Errors: as pkv_append_paged_attn_decode; PKV_E_UNSUPPORTED for shapes the
 * MFMA kernel does not take; PKV_E_SHAPE for negative counts or
 * max_prefix_len above max_context_len.
 */
int pkv_paged_attn_decode_prefix(const void* q, const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                                 float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                                 const int32_t* prefix_len, const int32_t* prefix_items, int32_t num_prefix_items,
                                 int32_t max_prefix_len, void* workspace, size_t workspace_bytes,
                                 int32_t partition_tokens, const int32_t* seq_order, const int32_t* work,
                                 int32_t num_work, hipStream_t stream);

/*
 * pkv_decode_work_list -- the live work of a split decode, one entry per
 * workgroup, from the host's copy of the lengths, for the work argument of
 * pkv_paged_attn_decode_prefix.  Host memory only; no device call.
 *
 * The split plan gives every sequence as many partitions as the longest
 * context needs; a launch over that grid also starts the partitions past each
 * shorter context's end, which find nothing to do but still take a dispatch
 * slot each.  The list names only the partitions that hold tokens (partition
 * 0 of every sequence, so empty and invalid sequences still get their zeros
 * or NaN).  A partition of at most 256 tokens gets one workgroup per 4 or 8
 * kv heads (the launch's waves per workgroup), each wave taking one kv head
 * alone; a longer one a workgroup per kv head, its waves sharing the tokens.
 * Whole sequences are dealt, longest first, to the 8 XCDs' ranges of the
 * launch so that each gets about equal tokens, and each range is padded to
 * the same length with entries (-1, 0), which the kernel skips.  Which
 * workgroup does what changes, not what is computed: each (sequence, kv head,
 * partition) state is the same arithmetic, and outputs agree with those
 * without a list to fp32 rounding (identical when no partition is that short).
 *
 *   context_lens  [num_seqs] int32, host (the lengths of the decode call)
 *   prefix_len    NULL, or [num_seqs] int32 host, as pkv_decode_prefix_plan
 *                 wrote it (partitions then cover only the positions after it)
 *   num_kv_heads, max_context_len, partition_tokens  as the decode call takes them
 *   work          [max_work][2] int32, written: (sequence, partition | kv head
 *                 << 16 | one-wave-per-head << 31)
 *   num_work      written: entries used, padding included; with PKV_E_SHAPE
 *                 because max_work is too small, the number needed.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (max_work too small, bad sizes).
 */
int pkv_decode_work_list(const int32_t* context_lens, const int32_t* prefix_len, int32_t num_seqs,
                         int32_t num_kv_heads, int32_t max_context_len, int32_t partition_tokens, int32_t* work,
                         int32_t max_work, int32_t* num_work);

/*
 * pkv_decode_supported -- 1 if the decode kernel `impl` (PKV_IMPL_*) is built for
 * this dtype, head_dim and GQA group size G = Hq / Hkv, else 0.
 */
int pkv_decode_supported(int32_t impl, int32_t dtype, int32_t head_dim, int32_t group);

/*
 * pkv_paged_prefill -- causal attention of many new tokens per sequence over
 * the paged cache (prompt prefill, or a chunk of one).
 *
 * Prefill takes all prompt tokens at once ("vLLM -- PagedAttention으로 LLM
 * 추론 성능을 2~4배 끌어올린 서빙 엔진", section "Prefill vs Decode"); each token
 * attends to itself and to earlier positions only ("[Hacker News 요약] C++와
 * CUDA로 vLLM의 경량 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section
 * "고성능 추론을 위한 고급 최적화 기법", causal mask; same formula and GQA as
 * decode).
 *
 *   q             [num_tokens][num_q_heads][head_dim]: the new tokens of all
 *                 sequences, packed; sequence i's are rows
 *                 query_start[i] .. query_start[i+1]-1.
 *   query_start   [num_seqs + 1] int32, device: non-decreasing, query_start[0] = 0,
 *                 query_start[num_seqs] = num_tokens.  n_i = query_start[i+1] -
 *                 query_start[i] may be 0.
 *   context_lens  [num_seqs] int32, device: L_i >= n_i, the context including the
 *                 new tokens.  New token j of sequence i is position L_i - n_i + j
 *                 and attends to positions 0 .. L_i - n_i + j; positions before
 *                 L_i - n_i are a prefix already in the pool (a cached prompt
 *                 prefix or an earlier chunk).  The K/V of all L_i positions must
 *                 be in the pools (pkv_kv_append of the new tokens first).
 *   max_query_len host bound of every n_i (sizes the grid); max_context_len host
 *                 bound of every L_i, at most max_blocks_per_seq * block_size.
 *   out           [num_tokens][num_q_heads][head_dim] in dtype.
 *   scale         softmax scale, positive and finite.
 *   the pools and block_tables as in pkv_paged_attn_decode.
 *
 * A sequence with n_i > max_query_len, L_i < n_i or L_i above the bounds gets NaN
 * in its rows (rows past the first max_query_len are not written); a block id
 * outside the pool makes the heads that read it NaN.  Inconsistent query_start
 * entries (negative, decreasing, or past num_tokens): that sequence's rows are
 * not written.  No workspace.
 * Supported: as the MFMA decode kernel (head_dim 64 or 128, G in {1, 2, 4, 8, 16}).
 * Errors: PKV_E_NULL, PKV_E_SHAPE, PKV_E_UNSUPPORTED, PKV_E_HIP.
 */
int pkv_paged_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* query_start,
                      int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale, void* out,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t dtype, hipStream_t stream);

/*
 * FP8 KV cache.  The Tiny-vLLM summary ("[Hacker News 요약] C++와 CUDA로 vLLM의
 * 경량 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section "향후 전망") names
 * an FP8 datatype as a next step and fixes nothing more; this library takes
 * the E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, no infinities, S.1111.111 = NaN, largest finite 448) with one
 * fp32 scale per pool: a stored code c stands for e4m3(c) * scale.  The pools
 * have the 16-bit layout above with one byte per element:
 *
 *   k_cache, v_cache: uint8 [N][Hkv][bs][D], code of (n,h,t,d) at byte
 *            ((n*Hkv + h)*bs + t)*D + d
 *
 * Decode reads half the bytes of a 16-bit cache, and decode time is the time
 * to read the cache ("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린
 * 서빙 엔진", section "Prefill vs Decode").
 */

/*
 * pkv_kv_append_fp8 -- pkv_kv_append into FP8 pools.
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] in src_dtype (PKV_BF16 or
 *                 PKV_FP16).
 *   k_scale, v_scale  the pools' scales, positive and finite.
 * Each element x is stored as the code nearest to fp32(x * fp32(1 / scale))
 * (ties to the even code), with magnitudes above 448 (infinities included)
 * saturating to +-448 (0x7E / 0xFE) and NaN stored as 0x7F.  Slots as in
 * pkv_kv_append (negative or >= num_blocks*block_size: nothing written;
 * distinct otherwise).  Only the bytes of the written slots change.
 * Supported: as pkv_kv_append.  Errors: PKV_E_NULL, PKV_E_SHAPE (also a scale
 * that is not positive and finite), PKV_E_UNSUPPORTED, PKV_E_HIP.
 */
int pkv_kv_append_fp8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                      void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_dim, int32_t src_dtype, float k_scale, float v_scale, hipStream_t stream);

/*
 * pkv_paged_attn_decode_fp8 -- pkv_paged_attn_decode_ex over FP8 pools:
 * out = softmax(scale * q K^T) V with K = e4m3(k_cache) * k_scale and
 * V = e4m3(v_cache) * v_scale.
 *
 *   q, out        [num_seqs][num_q_heads][head_dim] in dtype (PKV_BF16 / PKV_FP16).
 *   k_scale, v_scale  positive and finite.
 *   the other arguments are those of pkv_paged_attn_decode_ex (seq_order
 *   included); the workspace is sized by the same pkv_decode_workspace_bytes_ex
 *   query.
 * Every code is exact in dtype, so the kernel runs the 16-bit MFMA tiles on
 * the widened codes; k_scale is folded into the softmax scale and v_scale
 * into the output (not into any element).  Tails, empty and invalid
 * sequences as in pkv_paged_attn_decode.  A NaN code inside a context makes
 * the heads that read it NaN.
 * Supported: as the MFMA kernel (pkv_decode_supported(PKV_IMPL_MFMA, ...)).
 * Errors: PKV_E_NULL, PKV_E_SHAPE, PKV_E_UNSUPPORTED, PKV_E_WORKSPACE, PKV_E_HIP.
 */
int pkv_paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t max_context_len, float scale, float k_scale,
                              float v_scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t dtype, void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                              const int32_t* seq_order, hipStream_t stream);

/*
 * pkv_append_paged_attn_decode_fp8 -- one decode step of one layer over FP8
 * pools in a single launch: pkv_kv_append_fp8 of one new token per sequence
 * (k_new, v_new [num_seqs][num_kv_heads][head_dim] in dtype, encoded with the
 * same rule and scales), then pkv_paged_attn_decode_fp8 over contexts that
 * include it; the slot_mapping contract is that of
 * pkv_append_paged_attn_decode.  The same one-launch step the 16-bit pools
 * have; the pages describe the append and the attention as separate steps and
 * name FP8 only as a future direction ("[Hacker News 요약] C++와 CUDA로 vLLM의
 * 경량 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section "향후 전망").
 *
 * Results, when the preconditions hold: pools and out bit-identical to
 * pkv_kv_append_fp8(k_new, v_new, slot_mapping, B, ..., k_scale, v_scale)
 * followed by pkv_paged_attn_decode_fp8(...).  A non-negative slot that is not
 * the slot of position L_i - 1 (or a sequence with L_i = 0 and a slot) writes
 * nothing and makes sequence i's output NaN.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (also a scale that is not positive and
 * finite), PKV_E_UNSUPPORTED, PKV_E_WORKSPACE, PKV_E_HIP.
 */
int pkv_append_paged_attn_decode_fp8(const void* q, const void* k_new, const void* v_new,
                                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len, float scale,
                                     float k_scale, float v_scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t dtype, void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                                     const int32_t* seq_order, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
