// Internal plan representation shared by the host planner (plan.cpp) and the
// launcher (forward.hip). Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "pmattn.h"

namespace pmattn {

constexpr int kBlock = 16;
// Query rows (tokens x heads of one GQA group) a task may hold. Tasks of at
// most 64 rows run one per wave (classes 16, 32, 64: one, two or four 16-row
// MFMA column tiles); sequences with more rows than that are cut into
// 128-row tasks that run one per workgroup (4 waves x 32 rows, K/V staged in
// LDS).
constexpr int kMaxWaveRows = 64;
constexpr int kMaxTaskRows = 128;
constexpr int kNumClasses = 4;
constexpr int kClassRows[kNumClasses] = {16, 32, 64, 128};
// One-wave tasks run kWaveTasksPerWg to a workgroup (attn_bf16.hip).
constexpr int kWaveTasksPerWg = 4;
// Workgroups are dealt to the XCDs (accelerator dies, each with its own L2)
// round-robin in workgroup order: workgroup i runs on XCD i % kXcds.
constexpr int kXcds = 8;
constexpr int kMaxSplits = 256;
constexpr int kMaxTreeRows = 64;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Read-only view of one table inside the plan's upload image.
template <typename T>
struct Table {
  const T* ptr = nullptr;
  size_t n = 0;
  const T* data() const { return n ? ptr : nullptr; }
  size_t size() const { return n; }
  bool empty() const { return n == 0; }
  const T& operator[](size_t i) const { return ptr[i]; }
  const T* begin() const { return ptr; }
  const T* end() const { return ptr + n; }
};

struct Plan {
  uint64_t id = 0;
  // batch shape
  int32_t num_seqs = 0, num_rows = 0, bt_stride = 0, num_pool_blocks = 0;
  int32_t hq = 0, hkv = 0, group = 0, head_dim = 0, dtype = 0;
  float scale = 0.f;
  // canonical tables
  std::vector<int32_t> num_splits, split_offset, split_begin, split_end;
  std::vector<int32_t> class_rows, class_begin, class_cascade;
  // per class: 1 when all its tasks stream their K/V with non-temporal loads
  // (no block they read is read by another row tile), 0 none, 2 some (the
  // kernel reads the per-task flags, item_stream)
  std::vector<int32_t> class_stream;
  int32_t merge_max_parts = 0;  // largest nparts of any merge row
  int64_t merge_total_parts = 0;  // sum of nparts over the merge rows
  int32_t slot_class = -1;      // the class slot_begin belongs to
  int32_t num_records = 0;
  // Mixed-batch kernel (bf16 plans without token trees holding both 16-row
  // wave tasks and larger tasks): one workgroup per table entry, either one
  // workgroup task (entry 4 * item + 2 * cascade) or a bundle of four wave
  // tasks, one per wave (entry 4 * bundle + 1; bundle slots item * 2 +
  // cascade, or -1 for none).
  bool mixed = false;
  // cascade (shared-prefix) virtual sequences
  std::vector<int32_t> cascade_lo, cascade_hi, cascade_seq, cascade_row_begin, cascade_rows, cascade_splits;

  // Upload image: bytes [0, off_upload_end) of the workspace, laid out as
  // [items | merge rows | row masks | append units | record index | virtual
  // row sources | wave slots | task stream flags | mixed table | mixed
  // bundles]; the partial records follow it in the workspace (off_part_o,
  // off_part_lse). The tables below are views into it.
  std::unique_ptr<unsigned char[]> blob;
  Table<pmattn_work_item> items;
  Table<pmattn_merge_row> merge_rows;
  Table<uint64_t> row_mask;  // tree masks, one per row; empty unless some sequence is a tree
  Table<pmattn_append_unit> append_units;
  Table<int32_t> rec_index, vrow_src;
  // equal-work decode plans: wave w runs tasks [slot_begin[w], slot_begin[w + 1])
  // of class slot_class; empty when every task is its own wave
  Table<int32_t> slot_begin;
  Table<int32_t> item_stream;
  Table<int32_t> mix_table, mix_bundles;
  size_t off_items = 0, off_merge = 0, off_row_mask = 0, off_append = 0, off_rec_index = 0,
         off_vrow = 0, off_slot = 0, off_istream = 0, off_mix_table = 0, off_mix_bundles = 0,
         off_upload_end = 0, off_part_o = 0, off_part_lse = 0, ws_bytes = 0;

  // KV append check: empty, or why pmattn_kv_append must refuse this plan (a
  // target slot that another sequence can see, or that two rows write)
  std::string append_conflict;

  // Row tables (row_seq, row_pos): built on first export from the per-sequence
  // query starts and row offsets; nothing on the launch path reads them.
  std::vector<int32_t> seq_q_start, seq_row_off;
  std::once_flag rows_once;
  std::vector<int32_t> row_seq, row_pos;
};

// thread-local error message helpers (plan.cpp)
pmattn_status fail(pmattn_status st, const std::string& msg);
void clear_error();

}  // namespace pmattn

struct pmattn_plan_s {
  pmattn::Plan p;
};
