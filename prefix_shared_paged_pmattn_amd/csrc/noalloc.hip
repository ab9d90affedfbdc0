// pmattn_forward_noalloc: pmattn_forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). The work list, merge list and partial records live
// in a static device array instead of a caller workspace; the passes and
// kernels are pmattn_forward's.
#include <mutex>
#include <string>
#include <unordered_map>

#include "attn_kernels.h"
#include "plan_internal.h"

namespace pmattn {
namespace {

// Every GPU the library runs on holds its own copy of this array until the
// process ends. On the host `scratch` is only a stand-in for the symbol, never
// a device address: host code uses the address hipGetSymbolAddress returns for
// the current device, looked up once per device with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;

pmattn_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(PMATTN_E_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return PMATTN_OK;
}

}  // namespace
}  // namespace pmattn

using namespace pmattn;

extern "C" {

pmattn_status pmattn_forward_noalloc(pmattn_plan_t plan, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table_dev, void* out,
                                     float* lse, void* stream) {
  clear_error();
  if (!plan) return fail(PMATTN_E_INVALID, "plan is NULL");
  const Plan& P = plan->p;
  if (P.ws_bytes > kScratchBytes)
    return fail(PMATTN_E_WORKSPACE, "the plan needs " + std::to_string(P.ws_bytes) +
                                        " bytes of scratch, more than the " + std::to_string(kScratchBytes) +
                                        " pmattn_forward_noalloc holds; use pmattn_forward with a workspace");
  if (P.items.empty()) return PMATTN_OK;
  if (!q || !k_pool || !v_pool || !block_table_dev || !out)
    return fail(PMATTN_E_INVALID, "q, k_pool, v_pool, block_table and out must be non-NULL");
  void* ws = nullptr;
  pmattn_status s = scratch_ptr(&ws);
  if (s != PMATTN_OK) return s;
  // The scratch holds whatever the last call on this device left there: this
  // plan's tables go in first, on the stream of the passes that read them. No
  // kernel needs any part of it cleared.
  if ((s = upload(P, ws, static_cast<hipStream_t>(stream))) != PMATTN_OK) return s;
  // every class on the caller's stream: the auxiliary streams would be created
  // on first use
  if ((s = run_tasks(plan, q, k_pool, v_pool, block_table_dev, out, lse, ws, kScratchBytes, stream,
                     false)) != PMATTN_OK)
    return s;
  return run_merge(plan, out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
