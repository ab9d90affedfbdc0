/*
 * pmattn.h - C ABI of libpmattn: attention over a paged KV block pool whose
 * prefix blocks may be shared by several requests, for one mixed batch of
 * prefill-chunk, decode and speculative-verify query rows, on AMD gfx950.
 *
 * What is computed (per query row r of sequence s at absolute position
 * pos = q_start[s] + (r - first row of s), per query head h with kv head
 * g = h / (Hq / Hkv)):
 *
 *     out[r][h] = sum_j softmax_j(scale * q[r][h] . K_s[j]) * V_s[j],   j = 0..pos
 *     lse[r][h] = ln sum_j exp(scale * q[r][h] . K_s[j])
 *
 * where K_s[j] / V_s[j] are logical key j of sequence s, found in physical
 * block block_table[s][j / 16] at slot j % 16.
 *
 * Sources (the pages this library implements):
 *  - XY-Serve pith review ("Tackling the Dynamicity in a Production LLM
 *    Serving System with SOTA Optimizations via Hybrid Prefill/Decode/Verify
 *    Scheduling on Efficient Meta-kernels"), "What carries the argument" and
 *    "Core claim": one matmul-softmax-matmul meta-kernel over tile tasks
 *    listed in tables, for prefill, decode and verify tokens alike, with
 *    PagedAttention-style block caches, chunked prefill and prefix caching;
 *    "Editorial extensions": row-wise mask control instead of separate code
 *    paths; "Assumptions & free parameters": online softmax equals softmax,
 *    padded entries do not affect the output, block-table/radix-tree reuse
 *    keeps K/V semantics; Figure 3: the QK and SV GEMM shapes; Figure 8:
 *    linear speculative drafts; Figure 11: masked tiles are skipped and decode
 *    is matrix-vector work.
 *  - SGLang pith review ("SGLang: Efficient Execution of Structured Language
 *    Model Programs"), "Core claim": RadixAttention reuses KV caches across
 *    requests, so block tables of different requests name the same blocks.
 *  - XY-Serve review reference list: "Flash-Decoding for long-context
 *    inference" (split the KV range, merge partial results by log-sum-exp).
 *
 * Memory layouts (all row-major, no padding between elements):
 *  - q, out     [R][Hq][d]         R = sum of q_len; rows of sequence s are
 *                                  contiguous, sequences in descriptor order.
 *  - k_pool     [num_blocks][Hkv][d/x][16][x]   grouped inside a block,
 *                                  x = 16 bytes / element size (8 for bf16, 4
 *                                  for float32): channel c of slot o sits at
 *                                  [c/x][o][c%x], so each 16-byte group holds
 *                                  x channels of one token and the 16 tokens
 *                                  of a group are 256 contiguous bytes (the
 *                                  grouped K cache of the PagedAttention
 *                                  kernel the pages build on).
 *  - v_pool     [num_blocks][Hkv][d][16]   channel-major inside a block, so
 *                                  that 16 consecutive tokens of one channel
 *                                  are one contiguous 32-byte (bf16) run.
 *  - lse        [R][Hq] float32, natural log of the scaled scores.
 *  - block_table int32 [B][bt_stride]; entries past ceil((q_start+q_len)/16)
 *                of a sequence are never read.
 * Element type of q, k_pool, v_pool and out: bf16 (PMATTN_BF16) or float32
 * (PMATTN_F32), all the same.
 *
 * Threading and errors: every function is safe to call from several threads
 * on distinct plans. No function throws across the ABI; failures return a
 * status and set a thread-local message (pmattn_last_error()).
 */
#ifndef PMATTN_H
#define PMATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pmattn_status {
  PMATTN_OK = 0,
  PMATTN_E_INVALID = 1,      /* malformed arguments (lengths, ids, pointers) */
  PMATTN_E_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, block size, dtype) */
  PMATTN_E_WORKSPACE = 3,    /* workspace too small */
  PMATTN_E_HIP = 4,          /* a HIP runtime call failed; see pmattn_last_error() */
  PMATTN_E_NOMEM = 5,        /* host allocation failed */
  PMATTN_E_CAPACITY = 6      /* the block pool is exhausted (pmattn_radix.h) */
} pmattn_status;

typedef enum pmattn_dtype { PMATTN_BF16 = 0, PMATTN_F32 = 1 } pmattn_dtype;

/* Batch description for pmattn_plan. All pointers are HOST pointers borrowed
 * for the duration of the call only.
 *  q_len[s]    query rows of sequence s this step (0 allowed: no rows).
 *  seq_len[s]  keys of s present in the pool, including this step's query
 *              tokens (their K/V are written before attention runs).
 *  q_start[s]  absolute position of the first query row; requires
 *              q_start + q_len <= seq_len. Decode: q_start = seq_len - 1,
 *              q_len = 1. Prefill chunk: q_len = chunk. Verify of k linear
 *              drafts: q_len = k (causal among the drafts).
 *  block_table [num_seqs][bt_stride] physical block ids; bt_stride must be
 *              >= ceil(seq_len/16) for every sequence with q_len > 0.
 *  num_kv_splits  0: the planner chooses KV partitions per sequence;
 *              n in 1..256: every sequence uses n block-aligned partitions
 *              (n_blk = ceil((q_start+q_len)/16), chunk = ceil(n_blk/n) blocks,
 *              partition p = [p*chunk*16, min((p+1)*chunk*16, q_start+q_len))).
 *  num_cus     compute units the plan balances for (0: 256, one MI355X).
 *  work_shuffle_seed  0: deterministic cost order; otherwise the work list is
 *              permuted by this seed (results must not change: a race check).
 *  tree_parent NULL (every row causal), or [R] int32, one entry per query row
 *              in row order: the row (0-based, within the same sequence) of its
 *              parent in a speculative token tree, or -1 for a node that hangs
 *              off the context. Requires -1 <= parent < row. The rows of a
 *              sequence are the tree's nodes in topological order, their K/V at
 *              positions q_start + row. Row r sees every key below q_start
 *              plus the keys of its ancestors and itself (tree-based
 *              speculative verification, XY-Serve review, Figure 8 caption and
 *              "Significance"; Medusa and SpecInfer by title). A chain (parent
 *              r - 1) is the causal rule. A sequence whose parents are not a
 *              chain holds at most 64 rows.
 *  cascade     0: off. 1 or 2: shared-prefix cascade (two-phase attention) for
 *              sequences whose rows fit one wave task (q_len * Hq/Hkv <= 64,
 *              i.e. decode and verify): runs of leading physical blocks that
 *              two or more of them share, and that lie wholly before each
 *              one's first query row, are attended once for all sharers (their
 *              rows gathered into one virtual sequence); each sharer then
 *              attends only to the keys after its deepest shared run, and the
 *              log-sum-exp merge joins the parts (SGLang review, "Core claim":
 *              shared prefixes computed once; XY-Serve review "Core claim":
 *              prefix reuse). The result is the same attention. 1 makes a
 *              group of every such run; 2 (automatic) only of runs shared by
 *              at least 8 sequences over at least 64 blocks since the group
 *              above (shorter or narrower sharing is served by the caches and
 *              measured slower with the extra merge); a run left out is folded
 *              into the groups below it. */
typedef struct pmattn_plan_desc {
  int32_t num_seqs;
  const int32_t* q_len;
  const int32_t* seq_len;
  const int32_t* q_start;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t num_pool_blocks;
  int32_t block_size;      /* must be 16 */
  int32_t num_q_heads;     /* Hq */
  int32_t num_kv_heads;    /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 64 */
  int32_t head_dim;        /* 64 or 128 */
  int32_t dtype;           /* pmattn_dtype */
  float scale;             /* softmax scale, finite and > 0 (usually 1/sqrt(d)) */
  int32_t num_kv_splits;
  int32_t num_cus;
  uint64_t work_shuffle_seed;
  const int32_t* tree_parent;
  int32_t cascade;
} pmattn_plan_desc;

typedef struct pmattn_plan_s* pmattn_plan_t;

/* One tile task of the work list (the Task-Table analogue): query tokens
 * [row_begin, row_begin + n_tok) of sequence `seq` (positions pos_begin..)
 * for the Hq/Hkv query heads of kv head `kv_head`, against keys
 * [kv_begin, kv_end). part < 0: the task covers the rows' whole key range and
 * writes out/lse directly; otherwise it writes partial results to records
 * part + t*G + i (t = token, i = head within the group) for the merge. */
typedef struct pmattn_work_item {
  int32_t seq;
  int32_t kv_head;
  int32_t row_begin;
  int32_t n_tok;
  int32_t pos_begin;
  int32_t kv_begin;
  int32_t kv_end;
  int32_t part;
} pmattn_work_item;

/* One output row (row, q_head) assembled from nparts partial records by the
 * log-sum-exp merge: records rec0, rec0 + rec_stride, ... when rec_stride > 0;
 * when rec_stride == -1 (rows of cascade sharers), the record ids are
 * rec_index[rec0 .. rec0 + nparts) of the plan tables. */
typedef struct pmattn_merge_row {
  int32_t rec0;
  int32_t rec_stride;
  int32_t nparts;
  int32_t row;
  int32_t q_head;
} pmattn_merge_row;

/* One unit of the KV append (pmattn_kv_append): query tokens
 * [row_begin, row_begin + n_tok) of sequence `seq` land in slots
 * slot_begin .. slot_begin + n_tok - 1 of the sequence's logical block
 * `block_index` (physical id block_table[seq][block_index]); n_tok <= 16. */
typedef struct pmattn_append_unit {
  int32_t seq;
  int32_t row_begin;
  int32_t n_tok;
  int32_t block_index;
  int32_t slot_begin;
} pmattn_append_unit;

/* Read-only views of a plan's canonical tables (owned by the plan, valid
 * until pmattn_plan_destroy). */
typedef struct pmattn_plan_tables {
  int32_t num_rows;                 /* R */
  const int32_t* row_seq;           /* [R] sequence of each query row */
  const int32_t* row_pos;           /* [R] absolute position of each query row */
  int32_t num_seqs;
  const int32_t* num_splits;        /* [B] KV partitions of each sequence (0 if q_len == 0) */
  const int32_t* split_offset;      /* [B+1] prefix sums of num_splits */
  const int32_t* split_begin;       /* [sum num_splits] first key of each partition */
  const int32_t* split_end;         /* [sum num_splits] one past its last key (may equal begin) */
  int32_t num_items;
  const pmattn_work_item* items;    /* [num_items] in launch order */
  int32_t num_classes;              /* tile-shape classes, each a contiguous item range */
  const int32_t* class_rows;        /* [num_classes] query rows (tokens x group) per task, max */
  const int32_t* class_begin;       /* [num_classes + 1] item ranges */
  int32_t num_merge_rows;
  const pmattn_merge_row* merge_rows;
  int32_t num_part_records;         /* partial (output, lse) records in the workspace */
  /* [R] or NULL when no sequence is a tree: visibility of the keys just
   * before each row. Bit d set: the key at position row_pos - d is visible
   * (as far as the tree is concerned; d >= 64 and keys below q_start always
   * are). Rows of causal sequences hold all ones. */
  const uint64_t* row_tree_mask;
  int32_t num_append_units;
  const pmattn_append_unit* append_units;  /* [num_append_units], sequence order */
  const int32_t* class_cascade;     /* [num_classes] 1: tasks of virtual (cascade) sequences */
  /* cascade virtual sequences: keys [cascade_lo, cascade_hi) of block-table
   * row cascade_seq, rows virtual_row_src[cascade_row_begin .. + cascade_rows),
   * cascade_splits KV partitions each. Tasks of cascade classes index rows in
   * this virtual row space (row_begin) and take positions past cascade_hi. */
  int32_t num_cascade;
  const int32_t* cascade_lo;
  const int32_t* cascade_hi;
  const int32_t* cascade_seq;
  const int32_t* cascade_row_begin;
  const int32_t* cascade_rows;
  const int32_t* cascade_splits;
  int32_t num_virtual_rows;
  const int32_t* virtual_row_src;   /* [num_virtual_rows] the real query row of each */
  int32_t num_rec_index;
  const int32_t* rec_index;         /* record ids of indirect merge rows */
  /* Equal-work decode plans (every task a decode wave task, automatic splits,
   * bf16, no cascade): the KV blocks of all sequences, laid end to end, are
   * cut into equal pieces; wave w of the single class runs tasks
   * [slot_begin[w], slot_begin[w + 1]) one after another. 0 / NULL otherwise
   * (one task per wave). */
  int32_t num_slots;
  const int32_t* slot_begin;        /* [num_slots + 1] */
  /* [num_classes] 1: every task of the class streams, 0: none, 2: some
   * (see item_stream). */
  const int32_t* class_stream;
  /* [num_items] 1: no KV block the task reads is also read by a task of
   * another row tile (readers: the tile's first row, real or for cascade
   * classes virtual). A one-wave task so marked loads its K/V with the
   * non-temporal hint; blocks read again stay cacheable for their other
   * readers. The workgroup kernel stages K/V through LDS with cacheable
   * loads whatever the flag. */
  const int32_t* item_stream;
  /* 1: pmattn_forward runs the whole batch as one kernel (bf16 plans without
   * token trees that hold both 16-row tasks and larger ones). Workgroup i of
   * that launch runs mix_table[i]: 4 * item + 2 * c (one task on the whole
   * workgroup; c = 1 for items of cascade classes) or 4 * b + 1 (bundle b: wave
   * w runs mix_bundles[4 * b + w] = item * 2 + c, or nothing for -1). Every
   * item appears exactly once. */
  int32_t mixed_kernel;
  int32_t num_mix_entries;
  const int32_t* mix_table;         /* [num_mix_entries] */
  int32_t num_mix_bundles;
  const int32_t* mix_bundles;       /* [4 * num_mix_bundles] */
} pmattn_plan_tables;

/* Build a plan on the host: the Token-Table / Task-Table step of the
 * XY-Serve design (XY-Serve review, "Core claim": each step's attention work
 * is cut into tile-level tasks recorded in tables; "What carries the
 * argument": tiles are reordered across cores by computational area at run
 * time). Validates the batch (see pmattn_plan_desc), splits the work into tile
 * tasks (automatic splits: balanced cost quanta; pure decode batches in bf16:
 * equal KV pieces, one per wave, see pmattn_plan_tables.slot_begin; the KV
 * partitions are Flash-Decoding's split-KV, reference list of the same page),
 * orders them by estimated cost (largest first) with every kv head's tasks on
 * one XCD of the GPU, and prepares the merge list. Makes no HIP call and
 * touches no GPU.
 * Errors: PMATTN_E_INVALID for null pointers, negative lengths,
 * q_start + q_len > seq_len, a block id outside [0, num_pool_blocks) among the
 * blocks a row can see, bt_stride too small, Hq % Hkv != 0, scale not finite
 * or <= 0, num_kv_splits outside 0..256, a tree_parent entry outside
 * [-1, row); PMATTN_E_UNSUPPORTED for block_size != 16, head_dim not in
 * {64, 128}, an unknown dtype, Hq / Hkv > 64, or a tree of more than 64
 * rows. On success *out owns host memory until pmattn_plan_destroy. */
pmattn_status pmattn_plan(const pmattn_plan_desc* desc, pmattn_plan_t* out);

void pmattn_plan_destroy(pmattn_plan_t plan);

/* Device workspace bytes pmattn_forward needs for this plan (work list,
 * merge list, partial records), >= 256. */
pmattn_status pmattn_plan_workspace_bytes(pmattn_plan_t plan, size_t* bytes);

pmattn_status pmattn_plan_export(pmattn_plan_t plan, pmattn_plan_tables* tables);

/* Copy the plan's tables (work list, merge list, row tables) into
 * `workspace`, device memory of at least pmattn_plan_workspace_bytes, with an
 * asynchronous host-to-device copy on `stream` (a hipStream_t; NULL = the
 * default stream). The tables then live in the caller's memory: call this
 * after pmattn_plan and before the first pmattn_forward, pmattn_forward_tasks
 * or pmattn_kv_append of the plan on that workspace, and again whenever the
 * workspace memory has been freed, handed to another plan or written by
 * anything other than those calls. They never upload by themselves and never
 * check what the workspace holds (a plan's tables are reused as they are, as a
 * serving loop runs one plan for every layer of a step). Errors:
 * PMATTN_E_INVALID, PMATTN_E_WORKSPACE, PMATTN_E_HIP. */
pmattn_status pmattn_plan_upload(pmattn_plan_t plan, void* workspace, size_t ws_bytes,
                                 void* stream);

/* Run the attention of `plan` on the GPU, asynchronously on `stream`: every
 * tile task of the work list (matmul-softmax-matmul under each row's own mask,
 * XY-Serve review, "What carries the argument" and "Editorial extensions"),
 * then the log-sum-exp merge of split partials (Flash-Decoding, reference list
 * of the same page). Device pointers (caller-owned): q [R][Hq][d], k_pool,
 * v_pool (layouts above, at least num_pool_blocks blocks), block_table_dev
 * int32 [B][bt_stride] holding the same ids as the host table given to
 * pmattn_plan, out [R][Hq][d] (same element type as q), lse [R][Hq] float32
 * or NULL, workspace of ws_bytes >= pmattn_plan_workspace_bytes into which
 * pmattn_plan_upload has copied this plan's tables (the passes also write
 * partial records into it). The kernels read only keys a row can see; pool
 * slots no row can see may hold anything (NaN included) without affecting the
 * result. Errors: PMATTN_E_INVALID (null pointer), PMATTN_E_WORKSPACE,
 * PMATTN_E_HIP (launch failure). */
pmattn_status pmattn_forward(pmattn_plan_t plan, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table_dev, void* out,
                             float* lse, void* workspace, size_t ws_bytes, void* stream);

/* The two passes pmattn_forward runs, exported separately so that a caller
 * can interleave other work or time them apart (same arguments and errors as
 * pmattn_forward). Pass 1, pmattn_forward_tasks, runs every tile task: tasks
 * that cover their rows' whole key range write out/lse, the others write
 * partial (output, lse) records into the workspace. Pass 2,
 * pmattn_forward_merge, merges those records into out/lse (a no-op when the
 * plan split nothing). pass 2 must follow pass 1 on the same stream, with the
 * same workspace (which holds the plan's tables, see pmattn_plan_upload). This is the split-KV scheme of "Flash-Decoding for
 * long-context inference" (XY-Serve pith review, reference list). */
pmattn_status pmattn_forward_tasks(pmattn_plan_t plan, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table_dev, void* out,
                                   float* lse, void* workspace, size_t ws_bytes, void* stream);
pmattn_status pmattn_forward_merge(pmattn_plan_t plan, void* out, float* lse, void* workspace,
                                   size_t ws_bytes, void* stream);

/* pmattn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments as pmattn_forward minus the workspace, same kernels and the
 * same result: the plan's tables and partial records go into a static device
 * array of the library (64 MiB, held by every GPU the library runs on until
 * the process ends), which each call first fills with this plan's tables on
 * `stream`. Calls no hipMalloc, hipFree or other allocating routine, and runs
 * every task class on `stream`. Every call on one GPU shares that array and
 * leaves its contents to the next: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialized by the caller,
 * e.g. all on one stream. Errors: PMATTN_E_WORKSPACE when the plan needs more
 * than the array holds (pmattn_plan_workspace_bytes > 64 MiB), otherwise as
 * pmattn_forward. */
pmattn_status pmattn_forward_noalloc(pmattn_plan_t plan, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table_dev, void* out,
                                     float* lse, void* stream);

/* Merge P partial attention results over disjoint key sets into the full
 * result (the Flash-Decoding merge): with L = ln sum_p exp(part_lse[p]),
 * out = sum_p exp(part_lse[p] - L) * part_o[p], lse = L. Partitions with
 * lse = -inf weigh 0; if all are -inf the output is 0 and lse -inf.
 * Device pointers: part_o float32 [P][rows][H][d], part_lse float32
 * [P][rows][H], out [rows][H][d] of out_dtype (pmattn_dtype), lse float32
 * [rows][H] or NULL. Asynchronous on `stream`. Errors: PMATTN_E_INVALID
 * (P < 1, rows < 0, H < 1, null pointers), PMATTN_E_UNSUPPORTED (d not in
 * {64, 128}), PMATTN_E_HIP. */
pmattn_status pmattn_merge_lse(int32_t num_parts, int32_t num_rows, int32_t num_heads,
                               int32_t head_dim, const float* part_o, const float* part_lse,
                               void* out, int32_t out_dtype, float* lse, void* stream);

/* Write this step's keys and values into their pool slots: the step before
 * attention (XY-Serve review, "Core claim" and Figure 7: new tokens' K/V go
 * into paged blocks named by the block table; PagedAttention by title).
 * Query row r of sequence s, at position pos = q_start[s] + r, goes to slot
 * pos % 16 of physical block block_table[s][pos / 16], for every kv head:
 * k_pool[blk][h][c / x][pos % 16][c % x] = k_new[row][h][c] and
 * v_pool[blk][h][c][pos % 16] = v_new[row][h][c] (layouts above).
 * Device pointers (caller-owned): k_new, v_new [R][Hkv][d] of the plan's
 * element type; block_table_dev as for pmattn_forward; k_pool, v_pool are
 * written in place (only the slots of this step's rows); workspace as for
 * pmattn_forward (the work units travel in it: pmattn_plan_upload first).
 * Asynchronous on `stream`.
 * A slot written here must belong to its sequence alone: if another sequence
 * of the plan can see it, or two rows write it, the call fails with
 * PMATTN_E_INVALID (copy such blocks first: copy-on-write). Errors:
 * PMATTN_E_INVALID (null pointer, shared target slot), PMATTN_E_WORKSPACE,
 * PMATTN_E_HIP. */
pmattn_status pmattn_kv_append(pmattn_plan_t plan, const void* k_new, const void* v_new,
                               const int32_t* block_table_dev, void* k_pool, void* v_pool,
                               void* workspace, size_t ws_bytes, void* stream);

/* Thread-local message describing the last failure on this thread ("" if none). */
const char* pmattn_last_error(void);
const char* pmattn_status_str(pmattn_status status);
/* Library version as "major.minor.patch". */
const char* pmattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PMATTN_H */
