/* libpmattn: token-budget batch builder (host only).
 *
 * Builds one step's mixed batch of prefill chunks, decode rows and
 * speculative-verify rows under a token budget, the step before the plan.
 * Defined by the XY-Serve review, Figure 6 caption (a scheduled chunk stays
 * within the token budget, long prefills are cut into smaller parts, and some
 * slots are reserved for decode and speculative tokens so that prefill does
 * not disturb the time between tokens) and "Core claim" (one mixed batch of
 * prefill, decode and verify work per step).
 *
 * Policy (the reading taken where the pages give no detail):
 *  1. Decode and verify requests come first, in request order, each whole (a
 *     verify request's drafts are never split); one that does not fit in what
 *     is left of token_budget waits for a later step.
 *  2. Prefill requests then share at most token_budget - reserved rows, and at
 *     most what is left of token_budget, in request order: each takes
 *     min(pending, max_chunk, rows left); a request cut short is the step's
 *     last prefill (later prefills wait, so prompts complete in order).
 * A request's rows this step are its next q tokens: q_start = context,
 * seq_len = context + q.
 */
#ifndef PMATTN_BATCH_H
#define PMATTN_BATCH_H

#include <stdint.h>

#include "pmattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pmattn_request_kind {
  PMATTN_REQ_PREFILL = 0,  /* prompt tokens not computed yet */
  PMATTN_REQ_DECODE = 1,   /* one new token */
  PMATTN_REQ_VERIFY = 2    /* speculative drafts to verify */
} pmattn_request_kind;

typedef struct pmattn_request {
  int32_t kind;      /* pmattn_request_kind */
  int32_t context;   /* tokens already in the KV cache */
  int32_t pending;   /* prefill: prompt tokens left; decode: 1; verify: drafts (>= 1) */
} pmattn_request;

typedef struct pmattn_budget {
  int32_t token_budget;  /* query rows per step, >= 1 */
  int32_t reserved;      /* rows prefill may not use, 0 <= reserved <= token_budget */
  int32_t max_chunk;     /* prefill rows per request per step, >= 1 */
} pmattn_budget;

/* Schedule one step. q_len[i] receives request i's rows this step (0: not
 * scheduled); *total_rows their sum. q_start/seq_len for the plan follow as
 * context and context + q_len. Errors: PMATTN_E_INVALID (NULL pointers,
 * n < 0, bad budget, a request with negative context, unknown kind, decode
 * pending != 1, pending < 1 for verify, pending < 0 for prefill). */
pmattn_status pmattn_build_batch(const pmattn_request* requests, int32_t n,
                                 const pmattn_budget* budget, int32_t* q_len, int32_t* total_rows);

#ifdef __cplusplus
}
#endif

#endif /* PMATTN_BATCH_H */
