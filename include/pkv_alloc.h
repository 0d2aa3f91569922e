/*
 * pkv_alloc.h -- host-side block allocator of the paged KV-cache library (C ABI).
 *
 * It manages only block ids, in host memory: which physical blocks of a pool of
 * num_blocks are free, which belong to which sequence, and how many tokens each
 * sequence has.  From that it produces the int arrays the device calls consume
 * -- block tables, context lengths and the slot of every appended token -- and
 * never touches device memory.
 *
 * Semantics follow the pages: a sequence holds just the blocks its tokens need,
 * taken one at a time as tokens arrive, anywhere in the pool; a freed block
 * goes back to the pool for other requests ("vLLM -- PagedAttention으로 LLM 추론
 * 성능을 2~4배 끌어올린 서빙 엔진", section "PagedAttention -- OS 가상 메모리에서
 * 영감", and section "프로젝트 구조" for the block manager's logical/physical
 * mapping); block metadata stays on the CPU while the KV tensors stay on the GPU,
 * and sequences with the same prompt prefix can reuse its blocks ("Nano-vLLM로
 * 배우는 vLLM 추론 엔진 작동 원리 한눈에 정리", section "KV 캐시와 Block Manager").
 *
 * Sharing is by reference count and only of full blocks that lie before every
 * sharer's next token, so an append never writes into a shared block and no
 * copy-on-write is needed.
 *
 * A handle is not thread-safe: serialise calls on one handle.  Every function
 * returns PKV_OK (0) or a negative status from pkv_status.h; on error nothing
 * changes.
 */
#ifndef PKV_ALLOC_H_
#define PKV_ALLOC_H_

#include <stdint.h>

#include "pkv_status.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_alloc pkv_alloc;

/* New pool of num_blocks blocks of block_size tokens.  shuffle_seed 0 hands out
 * blocks in ascending id order; any other seed hands them out in a seeded
 * pseudo-random order (SplitMix64 + Fisher-Yates).  Returns NULL on bad sizes or
 * out of host memory. */
pkv_alloc* pkv_alloc_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed);
void pkv_alloc_destroy(pkv_alloc* a);

/* Register sequence seq_id holding num_tokens (>= 0) tokens: takes
 * ceil(num_tokens / block_size) free blocks.  PKV_E_EXISTS, PKV_E_NOMEM, PKV_E_SHAPE. */
int pkv_alloc_add_seq(pkv_alloc* a, int64_t seq_id, int32_t num_tokens);

/* Register seq_id with num_tokens tokens whose first num_shared_blocks logical
 * blocks are src_seq's (reference counted).  Needs num_shared_blocks*block_size
 * <= num_tokens and <= src's token count (the shared blocks are full).  The
 * remaining blocks are fresh.  PKV_E_NOSEQ, PKV_E_EXISTS, PKV_E_NOMEM, PKV_E_SHAPE. */
int pkv_alloc_add_seq_shared(pkv_alloc* a, int64_t seq_id, int32_t num_tokens, int64_t src_seq,
                             int32_t num_shared_blocks);

/* Make the first num_full_blocks logical blocks of the live sequence dst_seq
 * the same physical blocks as src_seq's (reference counted); dst_seq's own
 * blocks at those indices are released (returned to the pool when nobody else
 * holds them).  Used when the caller knows that dst_seq's leading tokens equal
 * src_seq's, so their K/V need to live in the pool once ("Nano-vLLM로 배우는
 * vLLM 추론 엔진 작동 원리 한눈에 정리", section "KV 캐시와 Block Manager":
 * sequences with the same prompt prefix reuse its blocks).  The shared blocks
 * must be full in both sequences and lie before both sequences' next write:
 * num_full_blocks * block_size <= min(len(src_seq), len(dst_seq)), so no later
 * append writes into a shared block.  dst_seq keeps its length and its blocks
 * past num_full_blocks.  num_full_blocks = 0 changes nothing.  PKV_E_NULL,
 * PKV_E_NOSEQ (either sequence missing), PKV_E_SHAPE (negative count, dst_seq
 * == src_seq, or blocks not full before the next write); on error nothing
 * changes. */
int pkv_alloc_share_prefix(pkv_alloc* a, int64_t dst_seq, int64_t src_seq, int32_t num_full_blocks);

/* Register seq_id with a num_tokens-token prompt given by its token ids, and
 * share the longest run of leading full blocks that a live sequence already
 * holds for the same tokens (prefix caching, "Nano-vLLM로 배우는 vLLM 추론 엔진
 * 작동 원리 한눈에 정리", section "KV 캐시와 Block Manager": a full block is
 * identified by a hash chained over its tokens and all earlier blocks' tokens;
 * a match is confirmed token by token and parent block by parent block).
 * *cached_tokens_out receives the number of leading tokens (a multiple of
 * block_size) whose K/V those shared blocks already hold: the caller writes K/V
 * only for the tokens after them.  The new sequence's own full blocks are
 * registered for later prompts.  A registered block outlives its holders: when
 * the last one frees it, it keeps its K/V and stays findable (the page's case
 * is a long system prompt that later requests repeat, so the cache should not
 * depend on the requests overlapping in time) until the pool needs it -- free
 * blocks holding nothing registered are handed out first, registered free
 * blocks only when no other block is free, least recently freed first, and
 * such a block leaves the registry when it is handed out.  So a match may
 * also take free blocks out of the pool.  Only prompt blocks are registered
 * (tokens appended later are not known here).  PKV_E_NULL, PKV_E_EXISTS,
 * PKV_E_NOMEM, PKV_E_SHAPE. */
int pkv_alloc_add_seq_prefix(pkv_alloc* a, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                             int32_t* cached_tokens_out);

/* Grow seq_id by one token; *slot_out receives that token's slot
 * (block * block_size + offset).  Takes a fresh block when the last one is full.
 * PKV_E_NOSEQ, PKV_E_NOMEM (the caller's cue to preempt or wait). */
int pkv_alloc_append_slot(pkv_alloc* a, int64_t seq_id, int64_t* slot_out);

/* pkv_alloc_append_slot for n sequences at once (one decode step); all or
 * nothing: on PKV_E_NOMEM / PKV_E_NOSEQ no sequence grows. */
int pkv_alloc_append_slots(pkv_alloc* a, const int64_t* seq_ids, int32_t n, int64_t* slots_out);

/* Release seq_id's blocks (a shared block returns to the pool when its last
 * holder is freed).  PKV_E_NOSEQ. */
int pkv_alloc_free_seq(pkv_alloc* a, int64_t seq_id);

/* Fill tables_out [n][max_blocks] (int32, row-major; entries past a sequence's
 * block count set to pad_value) and context_lens_out [n] for the listed
 * sequences.  PKV_E_NOSEQ, PKV_E_SHAPE (a sequence needs more than max_blocks). */
int pkv_alloc_block_tables(const pkv_alloc* a, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                           int32_t pad_value, int32_t* tables_out, int32_t* context_lens_out);

/* Number of free blocks (including the registered ones below); number of free
 * blocks that still hold a registered prompt block (prefix cache entries no
 * live sequence holds); number of live sequences; a sequence's token count. */
int32_t pkv_alloc_num_free(const pkv_alloc* a);
int32_t pkv_alloc_num_cached(const pkv_alloc* a);
int32_t pkv_alloc_num_seqs(const pkv_alloc* a);
int pkv_alloc_context_len(const pkv_alloc* a, int64_t seq_id, int32_t* len_out);
/* Reference count of a physical block (0 = free); -1 for an id outside the pool. */
int32_t pkv_alloc_refcount(const pkv_alloc* a, int32_t block);

#ifdef __cplusplus
}
#endif

#endif /* PKV_ALLOC_H_ */
