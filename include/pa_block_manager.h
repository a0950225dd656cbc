/*
 * pa_block_manager.h -- host-side allocator of the paged KV pool.
 *
 * The block manager decides which physical block (16 or 8 tokens) holds which tokens
 * of which sequence; the kernels of pa.h only read and write the blocks it
 * hands out.  What it implements is the block scheduling of the pages
 *   "LLM 推理优化：KV Cache、PagedAttention 与量化" (blog.tanteng.space),
 *     §2.2 (fixed 16-token blocks, a logical -> physical block table per
 *     sequence) and §2.3: (1) blocks are taken from a fixed-capacity pool when a
 *     sequence writes into them and returned at once when it ends, the pool
 *     keeps unreferenced blocks in LRU order, a full pool makes the scheduler
 *     preempt (swap a request out to the host); (2) copy-on-write: a fork
 *     copies the block table only and a shared block is copied when a sequence
 *     writes into it; (3) prefix sharing: identical prefixes are found by
 *     hashing block contents and tables then point at the same blocks;
 *   "大模型推理加速与显存黑科技 (Inference Acceleration & KV Cache)"
 *     (ialgorithm.me), §3.2: memory is taken on demand.
 *
 * Policy (fixed so that every result is unique and testable):
 *  - Free blocks form a stack: a fresh pool hands out 0, 1, 2, ...; a released
 *    block is pushed and handed out next.
 *  - A full block whose content is registered (prefix sharing) is not pushed
 *    when its last reference goes: it stays valid as a *cached* block at the
 *    most-recent end of an LRU list.  With the stack empty, the least recently
 *    released cached block is evicted (registration dropped) and handed out.
 *  - Releasing a sequence walks its table from its last block to its first.
 *  - A full block's content key is the whole token prefix up to its end, held
 *    as a chained 64-bit FNV-1a hash: chain(prev, block) = FNV-1a over the 8
 *    little-endian bytes of prev followed by the block's token ids as 4-byte
 *    little-endian integers; the empty prefix has chain 0.  The map key is
 *    (chain of the previous block, the block's token ids), compared exactly.
 *  - A prefix lookup matches at most (n - 1) / bs full blocks of an n-token
 *    prompt (bs = tokens per block), so the last prompt token is always left
 *    for the model.
 *  - Only the first token of an append can land in a partially filled block
 *    shared with another table; that block is copied (at most one copy per
 *    append) and the copy is reported for the caller to perform with
 *    pa_copy_blocks before it writes the new K/V.
 *  - An append that needs more blocks than are free plus cached returns
 *    PA_ERR_NO_SPACE and changes nothing.
 *
 * Ownership and threading: a manager is a host object owned by the caller
 * (create / destroy); it touches no device memory and is not thread-safe (one
 * scheduler thread per manager).  Sequence ids are any int64 chosen by the
 * caller.  All output arrays are host memory provided by the caller.
 * Unknown or duplicate sequence ids, null pointers and negative counts give
 * PA_ERR_INVALID_ARG with no change of state.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

typedef struct pa_bm_stats {
  int32_t num_blocks;
  int32_t free_blocks;      /* on the free stack */
  int32_t cached_blocks;    /* unreferenced, content registered, evictable */
  int32_t used_blocks;      /* referenced by at least one block table */
  int32_t num_seqs;         /* live sequences (swapped-out ones not counted) */
  int32_t swapped_seqs;     /* sequences swapped out */
  int64_t prefix_hit_blocks;/* blocks shared by pa_bm_match_prefix so far */
  int64_t cow_copies;       /* copy-on-write copies reported so far */
  int64_t evictions;        /* cached blocks evicted so far */
} pa_bm_stats;

/* A manager for a pool of num_blocks physical blocks (num_blocks > 0) of
 * block_size tokens: 16 (the pages' default) or 8 (the smaller blocks §2.2
 * of the blog.tanteng.space page mentions for 70B models); other sizes give
 * PA_ERR_UNSUPPORTED.  Slots are physical * block_size + offset. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new empty sequence.  hashing != 0: the full blocks it writes are registered
 * for prefix sharing (its appends must then pass token ids). */
pa_status pa_bm_add_seq(pa_block_manager* bm, int64_t seq_id, int32_t hashing);

/* Prefix sharing (§2.3 (3)): for an empty hashing sequence, share the
 * registered blocks that begin prompt[0 .. n); *cached_tokens = tokens now in
 * its table (a multiple of the block size bs, at most bs * ((n - 1) / bs)).  The caller then
 * appends the remaining prompt tokens. */
pa_status pa_bm_match_prefix(pa_block_manager* bm, int64_t seq_id, const int32_t* prompt,
                             int32_t n, int32_t* cached_tokens);

/* Slots for n new tokens of a sequence: slots[i] = physical * bs + offset of
 * token len + i (int64, the slot_mapping of pa_write_kv).  token_ids: the n
 * token ids (required for registration; NULL stops hashing for this sequence
 * from here on).  copy_src_dst[0..1] = (source, destination) block of a
 * copy-on-write the caller must perform before writing, or (-1, -1). */
pa_status pa_bm_append(pa_block_manager* bm, int64_t seq_id, const int32_t* token_ids, int32_t n,
                       int64_t* slots, int32_t* copy_src_dst);

/* One decode step: one token for each of n distinct sequences, all or nothing.
 * The blocks needed are counted before any change (every copy-on-write a
 * sequence would need on its own counts), then the sequences are appended in
 * order.  slots[i] is the slot of seq_ids[i]; copies = num_copies (source,
 * destination) pairs, room for n pairs.  token_ids may be NULL. */
pa_status pa_bm_append_step(pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                            const int32_t* token_ids, int64_t* slots, int32_t* copies,
                            int32_t* num_copies);

/* Copy-on-write fork (§2.3 (2)): child gets a copy of parent's table, length
 * and hashing state; every block's reference count goes up by one. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* End of a sequence: its references are released, last block first. */
pa_status pa_bm_free_seq(pa_block_manager* bm, int64_t seq_id);

/* Preemption (§2.3 (1)).  swap_out: copies the table (up to capacity entries)
 * into `table` (*num_blocks = its length, *context_len = the length) and then
 * releases it as pa_bm_free_seq does; the sequence keeps its length and hashing
 * state.  The caller saves the listed blocks' contents (pa_gather_blocks)
 * before anything else writes to the pool.  swap_in: ceil(len / bs) fresh
 * blocks, all or nothing (PA_ERR_NO_SPACE), written to `table`; the caller
 * restores the contents there (pa_scatter_blocks).  PA_ERR_INVALID_ARG when
 * capacity is too small (nothing changes). */
pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* table, int32_t capacity,
                         int32_t* num_blocks, int32_t* context_len);
pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* table, int32_t capacity,
                        int32_t* num_blocks);

/* The block table of a live sequence: row[0 .. *num_blocks) (capacity entries
 * at most; PA_ERR_INVALID_ARG if it does not fit) and its context length. */
pa_status pa_bm_get_table(const pa_block_manager* bm, int64_t seq_id, int32_t* row,
                          int32_t capacity, int32_t* num_blocks, int32_t* context_len);

/* Block tables of a batch, in the layout pa_decode reads: tables is int32
 * [n][max_blocks_per_seq], entries past a sequence's blocks set to -1;
 * context_lens is int32 [n]. */
pa_status pa_bm_fill_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                            int32_t* tables, int32_t max_blocks_per_seq, int32_t* context_lens);

/* A decode batch in dispatch-friendly order: out_ids = seq_ids sorted by
 * context length, longest first (equal lengths keep their input order).  The
 * decode kernel hands out its work in batch order, so a ragged batch whose
 * long sequences come first finishes its tail with short ones (measured on
 * MI355X, 32 sequences of U[512, 4096] tokens: 201.5 us in drawn order, 174.4
 * us longest first).  The caller builds q and reads out in this order.
 * out_ids may alias seq_ids. */
pa_status pa_bm_sort_longest_first(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                   int64_t* out_ids);

/* The shared prefix of a decode batch: *prefix_blocks = the number of leading
 * block-table entries that every sequence of seq_ids has in common (the same
 * physical blocks, e.g. a system prompt matched by pa_bm_match_prefix or
 * blocks inherited by pa_bm_fork), capped at the full blocks every context
 * covers (floor(min context length / block_size)).  Such a batch satisfies the
 * contract of pa_decode_shared_prefix with prefix_tokens = *prefix_blocks *
 * block_size (or any multiple of the partition size below it).  n = 0 gives 0. */
pa_status pa_bm_common_prefix(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                              int32_t* prefix_blocks);

pa_status pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* stats);

/* Reference count of a physical block (-1 when out of range). */
int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block);

/* Blocks a pa_bm_append of n tokens to seq_id would take now (-1 for an
 * unknown sequence). */
int32_t pa_bm_blocks_needed(const pa_block_manager* bm, int64_t seq_id, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
