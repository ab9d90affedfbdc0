// Internal plan representation shared by the host planner (plan.cpp) and the
// launcher (forward.hip). Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
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

struct Plan {
  uint64_t id = 0;
  // batch shape
  int32_t num_seqs = 0, num_rows = 0, bt_stride = 0, num_pool_blocks = 0;
  int32_t hq = 0, hkv = 0, group = 0, head_dim = 0, dtype = 0;
  float scale = 0.f;
  // canonical tables
  std::vector<int32_t> row_seq, row_pos;
  std::vector<int32_t> num_splits, split_offset, split_begin, split_end;
  std::vector<pmattn_work_item> items;
  std::vector<int32_t> class_rows, class_begin, class_cascade;
  // per task: 1 when no block it reads is read by another sequence's tasks
  // (the kernel then streams its K/V with non-temporal loads); per class: 1
  // all tasks, 0 none, 2 some
  std::vector<int32_t> item_stream, class_stream;
  std::vector<pmattn_merge_row> merge_rows;
  int32_t merge_max_parts = 0;  // largest nparts of any merge row
  // equal-work decode plans: wave w runs tasks [slot_begin[w], slot_begin[w + 1])
  // of the plan's single class; empty when every task is its own wave
  std::vector<int32_t> slot_begin;
  int32_t slot_class = -1;  // the class slot_begin belongs to
  int32_t num_records = 0;
  // Mixed-batch kernel (bf16 plans without token trees holding both 16-row
  // wave tasks and larger tasks): one workgroup per table entry, either one
  // workgroup task (entry 4 * item + 2 * cascade) or a bundle of four wave
  // tasks, one per wave (entry 4 * bundle + 1; bundle slots item * 2 +
  // cascade, or -1 for none).
  bool mixed = false;
  std::vector<int32_t> mix_table, mix_bundles;
  // tree masks, one per row, present only when some sequence is a tree
  std::vector<uint64_t> row_mask;
  // cascade (shared-prefix) virtual sequences, their rows, and the record
  // lists of the rows they merge into
  std::vector<int32_t> cascade_lo, cascade_hi, cascade_seq, cascade_row_begin, cascade_rows,
      cascade_splits, vrow_src, rec_index;
  // KV append units; a non-empty message marks a target slot that another
  // sequence can see (or two rows write): the append refuses such a plan
  std::vector<pmattn_append_unit> append_units;
  std::string append_conflict;
  // workspace layout (bytes): [items | merge rows | row masks | append units |
  // record index | virtual row sources | wave slots | task stream flags |
  // mixed table | mixed bundles | partial O | partial lse]; everything before
  // the partials is uploaded
  size_t off_items = 0, off_merge = 0, off_row_mask = 0, off_append = 0, off_rec_index = 0,
         off_vrow = 0, off_slot = 0, off_istream = 0, off_mix_table = 0, off_mix_bundles = 0,
         off_upload_end = 0, off_part_o = 0, off_part_lse = 0, ws_bytes = 0;
  std::vector<unsigned char> upload_blob;  // bytes [0, off_part_o) of the workspace
};

// thread-local error message helpers (plan.cpp)
pmattn_status fail(pmattn_status st, const std::string& msg);
void clear_error();

}  // namespace pmattn

struct pmattn_plan_s {
  pmattn::Plan p;
};
