// Launcher half of the C ABI: uploads a plan's work list into the caller's
// workspace and launches the tile-task kernels and the merge on the caller's
// stream. All device memory is the caller's; nothing here allocates it.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <unordered_map>

#include "attn_kernels.h"
#include "plan_internal.h"

namespace pmattn {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// Per-device auxiliary streams (default priority) and fork/join events: a plan
// that mixes wave tasks (decode/verify, KV-stream bound) and workgroup tasks
// (prefill, MFMA bound) runs the two kinds concurrently, the wave-task classes
// on the auxiliary streams, joined back into the caller's stream before the
// merge.
// The record/wait sequence is enqueued under a mutex, so concurrent callers
// never interleave the shared events (a wait binds to the latest record at
// enqueue time).
constexpr int kAux = 2;
struct DeviceAux {
  hipStream_t stream[kAux] = {};
  hipEvent_t fork = nullptr, join[kAux] = {};
};
std::mutex g_aux_mu;
std::unordered_map<int, DeviceAux> g_aux;

}  // namespace

pmattn_status hip_fail(hipError_t e, const char* what) {
  return fail(PMATTN_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

pmattn_status upload(const Plan& P, void* ws, hipStream_t st) {
  if (P.off_upload_end > 0) {
    hipError_t e = hipMemcpyAsync(ws, P.blob.get(), P.off_upload_end, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list)");
  }
  return PMATTN_OK;
}

// use_aux: the wave-task classes of a plan that also holds workgroup tasks may run
// on the per-device auxiliary streams (created on first use); without it every
// class runs in turn on the caller's stream.
pmattn_status run_tasks(pmattn_plan_t plan, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table_dev, void* out,
                        float* lse, void* workspace, size_t ws_bytes, void* stream, bool use_aux) {
  if (!plan) return fail(PMATTN_E_INVALID, "plan is NULL");
  const Plan& P = plan->p;
  if (P.items.empty()) return PMATTN_OK;
  if (!q || !k_pool || !v_pool || !block_table_dev || !out || !workspace)
    return fail(PMATTN_E_INVALID, "q, k_pool, v_pool, block_table, out and workspace must be non-NULL");
  if (ws_bytes < P.ws_bytes) return fail(PMATTN_E_WORKSPACE, "workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  AttnArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table_dev;
  a.out = out;
  a.lse = lse;
  a.row_mask = P.row_mask.empty() ? nullptr : reinterpret_cast<const uint64_t*>(ws + P.off_row_mask);
  a.part_o = reinterpret_cast<float*>(ws + P.off_part_o);
  a.part_lse = reinterpret_cast<float*>(ws + P.off_part_lse);
  a.slot_begin = nullptr;
  a.q_row = nullptr;
  a.item_stream = nullptr;
  a.slot_count = 0;
  a.bt_stride = P.bt_stride;
  a.hq = P.hq;
  a.hkv = P.hkv;
  a.group = P.group;
  a.scale = P.scale;
  a.scale_log2 = P.scale * kLog2e;
  const pmattn_work_item* items = reinterpret_cast<const pmattn_work_item*>(ws + P.off_items);
  if (P.mixed) {
    // one kernel for the whole mixed batch, on the caller's stream
    MixedArgs m;
    m.a = a;
    m.a.items = items;
    m.a.item_stream = reinterpret_cast<const int32_t*>(ws + P.off_istream);
    m.a.q_row = P.vrow_src.empty() ? nullptr : reinterpret_cast<const int32_t*>(ws + P.off_vrow);
    m.a.item_count = (int32_t)P.items.size();
    m.table = reinterpret_cast<const int32_t*>(ws + P.off_mix_table);
    m.bundles = reinterpret_cast<const int32_t*>(ws + P.off_mix_bundles);
    m.entries = (int32_t)P.mix_table.size();
    hipError_t e = launch_attn_mixed(P.head_dim, m, st);
    if (e != hipSuccess) return hip_fail(e, "mixed-batch kernel launch");
    return PMATTN_OK;
  }
  bool has_wg = false, has_wave = false;
  for (int32_t rows : P.class_rows) (rows > kMaxWaveRows ? has_wg : has_wave) = true;
  const bool concurrent = P.dtype == PMATTN_BF16 && has_wg && has_wave;
  auto launch_class = [&](size_t c, hipStream_t s) -> hipError_t {
    AttnArgs ac = a;
    ac.items = items + P.class_begin[c];
    ac.item_stream = reinterpret_cast<const int32_t*>(ws + P.off_istream) + P.class_begin[c];
    ac.item_count = P.class_begin[c + 1] - P.class_begin[c];
    if ((int)c == P.slot_class) {
      // equal-work decode tasks: one slot per wave
      ac.slot_begin = reinterpret_cast<const int32_t*>(ws + P.off_slot);
      ac.slot_count = (int32_t)P.slot_begin.size() - 1;
    }
    if (P.class_cascade[c]) {
      // virtual rows read their member's query row through the uploaded row
      // table; their keys all lie below every member's first row, so no tree
      // mask applies
      ac.q_row = reinterpret_cast<const int32_t*>(ws + P.off_vrow);
      ac.row_mask = nullptr;
    }
    if (P.dtype != PMATTN_BF16) return launch_attn_f32(P.head_dim, ac, s);
    if (P.class_rows[c] > kMaxWaveRows) return launch_attn_prefill(P.head_dim, ac, s);
    return launch_attn_bf16(P.head_dim, P.class_rows[c], ac, concurrent, P.class_stream[c], s);
  };
  if (!concurrent || !use_aux) {
    for (size_t c = 0; c < P.class_rows.size(); ++c) {
      hipError_t e = launch_class(c, st);
      if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    }
    return PMATTN_OK;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_aux_mu);
  DeviceAux& aux = g_aux[dev];
  if (!aux.fork) {
    e = hipEventCreateWithFlags(&aux.fork, hipEventDisableTiming);
    for (int i = 0; i < kAux && e == hipSuccess; ++i)
      if ((e = hipStreamCreateWithFlags(&aux.stream[i], hipStreamNonBlocking)) == hipSuccess)
        e = hipEventCreateWithFlags(&aux.join[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      g_aux.erase(dev);
      return hip_fail(e, "auxiliary stream setup");
    }
  }
  // wave-task classes in turn on the auxiliary streams (decode beside verify
  // beside the workgroup tasks), forking no more streams than there are such
  // classes: an idle fork and join measured 10 us on a 0.12 ms step
  int n_wave = 0;
  for (int32_t rows : P.class_rows) n_wave += rows <= kMaxWaveRows;
  const int na = std::min(kAux, n_wave);
  if ((e = hipEventRecord(aux.fork, st)) != hipSuccess) return hip_fail(e, "stream fork");
  for (int i = 0; i < na; ++i)
    if ((e = hipStreamWaitEvent(aux.stream[i], aux.fork, 0)) != hipSuccess) return hip_fail(e, "stream fork");
  int k = 0;
  for (size_t c = 0; c < P.class_rows.size(); ++c)
    if (P.class_rows[c] <= kMaxWaveRows && (e = launch_class(c, aux.stream[k++ % na])) != hipSuccess)
      return hip_fail(e, "attention kernel launch (wave tasks)");
  for (size_t c = 0; c < P.class_rows.size(); ++c)
    if (P.class_rows[c] > kMaxWaveRows && (e = launch_class(c, st)) != hipSuccess)
      return hip_fail(e, "attention kernel launch (workgroup tasks)");
  for (int i = 0; i < na; ++i)
    if ((e = hipEventRecord(aux.join[i], aux.stream[i])) != hipSuccess ||
        (e = hipStreamWaitEvent(st, aux.join[i], 0)) != hipSuccess)
      return hip_fail(e, "stream join");
  return PMATTN_OK;
}

pmattn_status run_merge(pmattn_plan_t plan, void* out, float* lse, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (!plan) return fail(PMATTN_E_INVALID, "plan is NULL");
  const Plan& P = plan->p;
  if (P.merge_rows.empty()) return PMATTN_OK;
  if (!out || !workspace) return fail(PMATTN_E_INVALID, "out and workspace must be non-NULL");
  if (ws_bytes < P.ws_bytes) return fail(PMATTN_E_WORKSPACE, "workspace too small");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  MergeArgs m;
  m.part_o = reinterpret_cast<const float*>(ws + P.off_part_o);
  m.part_lse = reinterpret_cast<const float*>(ws + P.off_part_lse);
  m.rows = reinterpret_cast<const pmattn_merge_row*>(ws + P.off_merge);
  m.rec_index = reinterpret_cast<const int32_t*>(ws + P.off_rec_index);
  m.out = out;
  m.lse = lse;
  m.count = (int32_t)P.merge_rows.size();
  m.hq = P.hq;
  m.implicit_parts = 0;
  m.implicit_rows = 0;
  m.max_parts = P.merge_max_parts;
  m.total_parts = P.merge_total_parts;
  hipError_t e = launch_merge(P.head_dim, P.dtype, m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return PMATTN_OK;
}

}  // namespace pmattn

using namespace pmattn;

extern "C" {

void pmattn_plan_destroy(pmattn_plan_t plan) { delete plan; }

pmattn_status pmattn_plan_upload(pmattn_plan_t plan, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!plan || !workspace) return fail(PMATTN_E_INVALID, "NULL plan or workspace");
  if (ws_bytes < plan->p.ws_bytes) return fail(PMATTN_E_WORKSPACE, "workspace too small");
  return upload(plan->p, workspace, static_cast<hipStream_t>(stream));
}

pmattn_status pmattn_forward_tasks(pmattn_plan_t plan, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table_dev, void* out,
                                   float* lse, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  return run_tasks(plan, q, k_pool, v_pool, block_table_dev, out, lse, workspace, ws_bytes, stream, true);
}

pmattn_status pmattn_forward_merge(pmattn_plan_t plan, void* out, float* lse, void* workspace,
                                   size_t ws_bytes, void* stream) {
  clear_error();
  return run_merge(plan, out, lse, workspace, ws_bytes, stream);
}

pmattn_status pmattn_kv_append(pmattn_plan_t plan, const void* k_new, const void* v_new,
                               const int32_t* block_table_dev, void* k_pool, void* v_pool,
                               void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!plan) return fail(PMATTN_E_INVALID, "plan is NULL");
  const Plan& P = plan->p;
  if (!P.append_conflict.empty()) return fail(PMATTN_E_INVALID, P.append_conflict);
  if (P.append_units.empty()) return PMATTN_OK;
  if (!k_new || !v_new || !block_table_dev || !k_pool || !v_pool || !workspace)
    return fail(PMATTN_E_INVALID, "k_new, v_new, block_table, k_pool, v_pool and workspace must be non-NULL");
  if (ws_bytes < P.ws_bytes) return fail(PMATTN_E_WORKSPACE, "workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table_dev;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.units = reinterpret_cast<const pmattn_append_unit*>(static_cast<unsigned char*>(workspace) + P.off_append);
  a.unit_count = (int32_t)P.append_units.size();
  a.bt_stride = P.bt_stride;
  a.hkv = P.hkv;
  hipError_t e = launch_kv_append(P.head_dim, P.dtype, a, st);
  if (e != hipSuccess) return hip_fail(e, "kv append kernel launch");
  return PMATTN_OK;
}

pmattn_status pmattn_copy_blocks(const pmattn_block_copy* copies_dev, int32_t num_copies,
                                 void* k_pool, void* v_pool, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, void* stream) {
  clear_error();
  if (num_copies < 0 || num_kv_heads < 1) return fail(PMATTN_E_INVALID, "num_copies < 0 or num_kv_heads < 1");
  if (head_dim != 64 && head_dim != 128) return fail(PMATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != PMATTN_BF16 && dtype != PMATTN_F32) return fail(PMATTN_E_UNSUPPORTED, "unknown dtype");
  if (num_copies == 0) return PMATTN_OK;
  if (!copies_dev || !k_pool || !v_pool) return fail(PMATTN_E_INVALID, "NULL pointer");
  hipError_t e = launch_copy_blocks(head_dim, dtype, copies_dev, num_copies, k_pool, v_pool, num_kv_heads,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block copy kernel launch");
  return PMATTN_OK;
}

pmattn_status pmattn_forward(pmattn_plan_t plan, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table_dev, void* out,
                             float* lse, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  pmattn_status s = run_tasks(plan, q, k_pool, v_pool, block_table_dev, out, lse, workspace,
                              ws_bytes, stream, true);
  if (s != PMATTN_OK) return s;
  return run_merge(plan, out, lse, workspace, ws_bytes, stream);
}

pmattn_status pmattn_merge_lse(int32_t num_parts, int32_t num_rows, int32_t num_heads,
                               int32_t head_dim, const float* part_o, const float* part_lse,
                               void* out, int32_t out_dtype, float* lse, void* stream) {
  clear_error();
  if (num_parts < 1 || num_rows < 0 || num_heads < 1)
    return fail(PMATTN_E_INVALID, "need num_parts >= 1, num_rows >= 0, num_heads >= 1");
  if (head_dim != 64 && head_dim != 128) return fail(PMATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (out_dtype != PMATTN_BF16 && out_dtype != PMATTN_F32)
    return fail(PMATTN_E_UNSUPPORTED, "out_dtype must be PMATTN_BF16 or PMATTN_F32");
  if ((int64_t)num_parts * num_rows * num_heads > INT32_MAX / 2)
    return fail(PMATTN_E_INVALID, "too many partial records");
  if (num_rows == 0) return PMATTN_OK;
  if (!part_o || !part_lse || !out) return fail(PMATTN_E_INVALID, "part_o, part_lse and out must be non-NULL");
  MergeArgs m;
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.rows = nullptr;
  m.rec_index = nullptr;
  m.out = out;
  m.lse = lse;
  m.count = num_rows * num_heads;
  m.hq = num_heads;
  m.implicit_parts = num_parts;
  m.implicit_rows = num_rows;
  m.max_parts = num_parts;
  m.total_parts = (int64_t)num_parts * m.count;
  hipError_t e = launch_merge(head_dim, out_dtype, m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return PMATTN_OK;
}

}  // extern "C"
