/* libpmattn: host radix-tree KV cache manager for the paged block pool.
 *
 * The step before the plan: it turns token streams into block tables whose
 * shared prefixes name the same physical blocks. Defined by:
 *  - SGLang review ("Core claim", "What carries the argument"): RadixAttention
 *    keeps the KV of finished and running requests in a radix tree keyed by
 *    token ids, reuses the longest cached prefix for a new request, and evicts
 *    least-recently-used leaves when memory runs out.
 *  - XY-Serve review ("Assumptions & free parameters"; Figure 7, token-wise K/V
 *    reuse): matching is token-wise; block-table management with copy-on-write
 *    keeps K/V semantics when a match ends inside a block.
 *
 * Model. The pool holds num_blocks blocks of 16 token slots (the same pool
 * pmattn_forward reads). Position p of a sequence lives in slot p % 16 of the
 * sequence's block p / 16. Every block carries a reference count: one per
 * live sequence whose table names it and one per tree node that names it; a
 * block with no reference is free. A live sequence can therefore never lose a
 * block it uses, whatever the tree evicts.
 *
 * Life of a request:
 *   admit    match the longest cached prefix of its tokens; fully matched
 *            blocks are shared; if the match ends inside a block, that block
 *            is copied (copy-on-write: the caller copies the first `slots`
 *            slots of src into dst, e.g. with pmattn_copy_blocks, before
 *            writing); the rest of the table is fresh blocks.
 *   extend   add tokens (decode steps, next prefill chunk); new blocks as
 *            needed. Writing into the sequence's own partly filled last block
 *            is always safe: any other request that matched it got a copy.
 *   publish  insert the sequence's tokens so far into the tree (their K/V
 *            must be written by then), so later requests can reuse them.
 *   release  the request ends; its references go. Blocks still named by the
 *            tree stay cached until evicted.
 * Copy orders of a batch of admits must run before any K/V of that batch is
 * written, and before the admitted sequence's next extend, publish or
 * release: until then the sequence holds a reference on its copy's source
 * block, so no admit can hand that block out (as a fresh block or a copy
 * destination) while the copy may still read it, even when an eviction has
 * dropped the tree entry that held it.
 * When a block is needed and none is free, whole least-recently-used leaves
 * of the tree are evicted until one is. If nothing evictable remains the call
 * fails with PMATTN_E_CAPACITY and changes nothing.
 *
 * Host only: no function here touches the GPU. Not thread-safe: one cache per
 * thread, or external locking. */
#ifndef PMATTN_RADIX_H
#define PMATTN_RADIX_H

#include <stdint.h>

#include "pmattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pmattn_radix_s* pmattn_radix_t;

/* One copy-on-write order: copy slots [0, slots) of block src into block dst
 * (every kv head, K and V) before the new sequence writes into dst. */
typedef struct pmattn_block_copy {
  int32_t src;
  int32_t dst;
  int32_t slots;
} pmattn_block_copy;

typedef struct pmattn_radix_stats {
  int32_t num_blocks;      /* pool size */
  int32_t free_blocks;     /* blocks with no reference */
  int32_t tree_nodes;      /* radix nodes (root excluded) */
  int32_t tree_tokens;     /* tokens stored in the tree */
  int32_t live_seqs;       /* admitted, not yet released */
  int64_t evicted_nodes;   /* leaves evicted since creation */
} pmattn_radix_stats;

/* A cache over a pool of num_blocks blocks (ids 0 .. num_blocks-1).
 * Errors: PMATTN_E_INVALID (num_blocks < 1, out NULL), PMATTN_E_NOMEM. */
pmattn_status pmattn_radix_create(int32_t num_blocks, pmattn_radix_t* out);
void pmattn_radix_destroy(pmattn_radix_t cache);

/* Admit a request of n >= 0 tokens (host int32 token ids). Outputs: *seq_id
 * (a handle for the other calls), *cached_len (tokens whose K/V are reused:
 * positions [0, cached_len) need no write; the caller writes the rest), the
 * block table (ceil(n/16) entries into block_table, which holds `capacity`
 * int32), and at most one copy-on-write order (*num_copies is 0 or 1, written
 * to *copy). The tree entries used are marked recently used.
 * Errors: PMATTN_E_INVALID (NULL pointers, n < 0, capacity < ceil(n/16)),
 * PMATTN_E_CAPACITY (pool exhausted; nothing changes), PMATTN_E_NOMEM. */
pmattn_status pmattn_radix_admit(pmattn_radix_t cache, const int32_t* tokens, int32_t n,
                                 int32_t* seq_id, int32_t* cached_len, int32_t* block_table,
                                 int32_t capacity, pmattn_block_copy* copy, int32_t* num_copies);

/* Append n >= 0 tokens to live sequence seq_id; block_table receives the
 * sequence's whole table (ceil(total/16) entries, at most `capacity`).
 * Errors: PMATTN_E_INVALID (unknown seq_id, NULL pointers, capacity too small),
 * PMATTN_E_CAPACITY (nothing changes), PMATTN_E_NOMEM. */
pmattn_status pmattn_radix_extend(pmattn_radix_t cache, int32_t seq_id, const int32_t* tokens,
                                  int32_t n, int32_t* block_table, int32_t capacity);

/* Insert live sequence seq_id's tokens so far into the tree (their K/V must
 * be written). Errors: PMATTN_E_INVALID (unknown seq_id), PMATTN_E_NOMEM. */
pmattn_status pmattn_radix_publish(pmattn_radix_t cache, int32_t seq_id);

/* End live sequence seq_id. Errors: PMATTN_E_INVALID (unknown seq_id). */
pmattn_status pmattn_radix_release(pmattn_radix_t cache, int32_t seq_id);

/* Length of the longest cached prefix of tokens[0, n) (no side effects). */
pmattn_status pmattn_radix_match(pmattn_radix_t cache, const int32_t* tokens, int32_t n,
                                 int32_t* matched);

pmattn_status pmattn_radix_stats_get(pmattn_radix_t cache, pmattn_radix_stats* out);

/* Reference count of one block (for checks). Errors: PMATTN_E_INVALID. */
pmattn_status pmattn_radix_block_refs(pmattn_radix_t cache, int32_t block, int32_t* refs);

/* Device side of copy-on-write: for each order, copy slots [0, slots) of block
 * src into block dst, for every kv head, in both pools (layouts as for
 * pmattn_forward). copies_dev: device array of num_copies orders, with every
 * src != dst and no dst used twice. Asynchronous on `stream`.
 * Errors: PMATTN_E_INVALID (NULL pointers, num_copies < 0, num_kv_heads < 1),
 * PMATTN_E_UNSUPPORTED (head_dim, dtype), PMATTN_E_HIP. */
pmattn_status pmattn_copy_blocks(const pmattn_block_copy* copies_dev, int32_t num_copies,
                                 void* k_pool, void* v_pool, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PMATTN_RADIX_H */
