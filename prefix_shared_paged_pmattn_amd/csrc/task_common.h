// Device helpers shared by the tile-task bodies (task_wave.h, task_wg.h).
#pragma once

#include "attn_kernels.h"

namespace pmattn {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Read-only tables are read through the constant address space so that
// wave-uniform indices turn into scalar loads: their waits count on lgkmcnt and
// never drain the vector loads of the KV stream.
typedef const int32_t __attribute__((address_space(4)))* cint_p;

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// A compiler memory barrier plus a scheduling barrier: pins loads to the
// point where they are issued, so that the optimizer can neither sink them
// next to their first use nor hoist other math above them.
__device__ __forceinline__ void issue_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ pmattn_work_item load_item(const pmattn_work_item* items, int idx) {
  const cint_p p = (cint_p)(items + idx);
  pmattn_work_item it;
  it.seq = p[0];
  it.kv_head = p[1];
  it.row_begin = p[2];
  it.n_tok = p[3];
  it.pos_begin = p[4];
  it.kv_begin = p[5];
  it.kv_end = p[6];
  it.part = p[7];
  return it;
}

}  // namespace
}  // namespace pmattn
