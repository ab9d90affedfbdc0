// Token-budget batch builder (declared in pmattn_batch.h): decode and verify
// rows first, whole; prefill chunks in request order within the budget minus
// the reserved slots (XY-Serve review, Figure 6 caption).
#include <algorithm>
#include <string>

#include "pmattn_batch.h"
#include "plan_internal.h"

using namespace pmattn;

extern "C" pmattn_status pmattn_build_batch(const pmattn_request* requests, int32_t n,
                                            const pmattn_budget* budget, int32_t* q_len,
                                            int32_t* total_rows) {
  clear_error();
  if (!budget || !total_rows || n < 0 || (n > 0 && (!requests || !q_len)))
    return fail(PMATTN_E_INVALID, "NULL argument or n < 0");
  const int64_t cap = budget->token_budget;
  if (cap < 1 || budget->reserved < 0 || budget->reserved > cap || budget->max_chunk < 1)
    return fail(PMATTN_E_INVALID, "budget needs token_budget >= 1, 0 <= reserved <= token_budget, max_chunk >= 1");
  for (int32_t i = 0; i < n; ++i) {
    const pmattn_request& r = requests[i];
    const bool ok = r.context >= 0 &&
                    ((r.kind == PMATTN_REQ_PREFILL && r.pending >= 0) ||
                     (r.kind == PMATTN_REQ_DECODE && r.pending == 1) ||
                     (r.kind == PMATTN_REQ_VERIFY && r.pending >= 1));
    if (!ok) return fail(PMATTN_E_INVALID, "malformed request " + std::to_string(i));
    q_len[i] = 0;
  }
  int64_t used = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pmattn_request& r = requests[i];
    if (r.kind == PMATTN_REQ_PREFILL) continue;
    if (used + r.pending <= cap) {
      q_len[i] = r.pending;
      used += r.pending;
    }
  }
  int64_t prefill_left = std::min<int64_t>(cap - budget->reserved, cap - used);
  for (int32_t i = 0; i < n && prefill_left > 0; ++i) {
    const pmattn_request& r = requests[i];
    if (r.kind != PMATTN_REQ_PREFILL || r.pending == 0) continue;
    const int64_t want = std::min<int64_t>(r.pending, budget->max_chunk);
    const int64_t take = std::min(want, prefill_left);
    q_len[i] = (int32_t)take;
    used += take;
    prefill_left -= take;
    if (take < want) break;  // cut short: later prompts wait
  }
  *total_rows = (int32_t)used;
  return PMATTN_OK;
}
