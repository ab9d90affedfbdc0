// Device-side definitions shared by the attention and merge kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmattn.h"
#include "pmattn_radix.h"

namespace pmattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  void* out;
  float* lse;                    // may be null
  const pmattn_work_item* items; // this launch's first task
  const int32_t* q_row;          // null: a task's query row r is row r of q; else row q_row[r]
                                 // (cascade classes: virtual rows name their member's row)
  const uint64_t* row_mask;      // [R] token-tree masks, or null: every row causal
  float* part_o;                 // [records][d]
  float* part_lse;               // [records]
  const int32_t* slot_begin;     // one-wave kernel: wave w runs tasks [slot_begin[w], slot_begin[w+1]);
                                 // null: wave w runs task w
  const int32_t* item_stream;    // per task of this launch: 1 = non-temporal K/V loads (one-wave
                                 // kernel, classes whose tasks differ)
  int32_t slot_count;
  int32_t item_count;
  int32_t bt_stride;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  float scale;                   // softmax scale
  float scale_log2;              // scale * log2(e)
};

// The mixed-batch kernel (attn_mixed.hip): workgroup i runs table[i], a
// workgroup task (4 * item + 2 * cascade) or a bundle of four wave tasks
// (4 * bundle + 1; bundles[4 * bundle + wave] = item * 2 + cascade, or -1).
struct MixedArgs {
  AttnArgs a;                    // a.items: the whole work list; a.q_row: the virtual
                                 // row table (cascade entries); a.item_stream per item
  const int32_t* table;
  const int32_t* bundles;
  int32_t entries;
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const pmattn_merge_row* rows;  // null: implicit [P][rows][H] layout
  const int32_t* rec_index;      // record ids of listed merge rows (rec_stride < 0)
  void* out;
  float* lse;
  int32_t count;                 // output (row, head) pairs
  int32_t hq;                    // heads per output row
  int32_t implicit_parts;        // implicit layout: P
  int32_t implicit_rows;         // implicit layout: rows
  int32_t max_parts;             // largest partial count of any output (kernel choice)
  int64_t total_parts;           // partials over all outputs (kernel choice)
};

struct AppendArgs {
  const void* k_new;               // [R][Hkv][d]
  const void* v_new;               // [R][Hkv][d]
  const int32_t* block_table;
  void* k_pool;
  void* v_pool;
  const pmattn_append_unit* units;
  int32_t unit_count;
  int32_t bt_stride;
  int32_t hkv;
};

// Launcher internals (forward.hip), shared with the allocation-free entry
// point (noalloc.hip). upload: the plan's tables into ws (async on st).
// run_tasks / run_merge: the two passes of pmattn_forward over the workspace
// ws; use_aux lets the wave-task classes of a plan that also holds workgroup
// tasks run on per-device auxiliary streams.
struct Plan;
pmattn_status hip_fail(hipError_t e, const char* what);
pmattn_status upload(const Plan& P, void* ws, hipStream_t st);
pmattn_status run_tasks(pmattn_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table_dev, void* out, float* lse, void* workspace,
                        size_t ws_bytes, void* stream, bool use_aux);
pmattn_status run_merge(pmattn_plan_t plan, void* out, float* lse, void* workspace, size_t ws_bytes,
                        void* stream);

// Kernel launchers.
// concurrent: workgroup tasks of the same plan run beside these waves (on a
// second stream); 16-row tasks then take the 3-waves-per-SIMD variant.
// stream: 1 no other sequence reads the class's KV blocks (non-temporal
// loads), 0 some do (cached loads), 2 per task (a.item_stream).
hipError_t launch_attn_bf16(int head_dim, int class_rows, const AttnArgs& a, bool concurrent, int stream,
                            hipStream_t st);
hipError_t launch_attn_prefill(int head_dim, const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_mixed(int head_dim, const MixedArgs& m, hipStream_t st);
hipError_t launch_attn_f32(int head_dim, const AttnArgs& a, hipStream_t st);
hipError_t launch_merge(int head_dim, int out_dtype, const MergeArgs& a, hipStream_t st);
hipError_t launch_kv_append(int head_dim, int dtype, const AppendArgs& a, hipStream_t st);
// Copy the query rows src_rows[0..n) of q ([R][row_elems]) into dst ([n][row_elems]).
hipError_t launch_copy_blocks(int head_dim, int dtype, const pmattn_block_copy* copies, int n,
                              void* k_pool, void* v_pool, int hkv, hipStream_t st);

}  // namespace pmattn
