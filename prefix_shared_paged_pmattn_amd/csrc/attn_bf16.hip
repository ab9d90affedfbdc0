// bf16 one-wave kernel for gfx950: every wave runs its own tile task
// (decode, verify and other tasks of at most 64 rows). The task body, its KV
// streaming and its MFMA tiling are in task_wave.h.
#include "plan_internal.h"
#include "task_wave.h"

namespace pmattn {
namespace {

// Tasks are independent; a workgroup holds four of them, one per wave (1- and
// 2-wave workgroups measured the same or slower on the decode workloads). The
// planner's dispatch order groups tasks by this count.
constexpr int kWavesPerWg = kWaveTasksPerWg;

// Wave w of the launch runs task w, or, with a slot table (equal-work plans
// of 16- or 32-row tasks), its tasks [slot_begin[w], slot_begin[w + 1]) one
// after another. (The loop stays out of the 64-row tiles, which it pushes
// into spilling.)
// SMODE 0: cached K/V loads, 1: non-temporal, 2: the task's item_stream flag
// decides (a uniform branch between the two bodies).
template <int D, int NT, bool TREE, bool CONC, int SMODE>
__device__ __forceinline__ void run_one(const AttnArgs& a, int idx, int lane) {
  if constexpr (SMODE == 2) {
    if (((cint_p)a.item_stream)[idx]) run_task<D, NT, TREE, CONC, true>(a, load_item(a.items, idx), a.q_row, lane);
    else run_task<D, NT, TREE, CONC, false>(a, load_item(a.items, idx), a.q_row, lane);
  } else {
    run_task<D, NT, TREE, CONC, SMODE == 1>(a, load_item(a.items, idx), a.q_row, lane);
  }
}

template <int D, int NT, bool TREE, bool CONC, int SMODE>
__global__ __launch_bounds__(64 * kWavesPerWg) __attribute__((amdgpu_waves_per_eu(WavesPerEu<NT, CONC>::value, 8)))
void attn_bf16_kernel(AttnArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kWavesPerWg + wave;
  if constexpr (NT > 2) {
    if (w < a.item_count) run_one<D, NT, TREE, CONC, SMODE>(a, w, lane);
    return;
  }
  int first, last;
  if (a.slot_begin) {
    if (w >= a.slot_count) return;
    const cint_p sb = (cint_p)a.slot_begin;
    first = sb[w];
    last = sb[w + 1];
  } else {
    if (w >= a.item_count) return;
    first = w;
    last = w + 1;
  }
  for (int idx = first; idx < last; ++idx) run_one<D, NT, TREE, CONC, SMODE>(a, idx, lane);
}

}  // namespace

hipError_t launch_attn_bf16(int head_dim, int class_rows, const AttnArgs& a, bool concurrent, int stream,
                            hipStream_t st) {
  if (a.item_count <= 0) return hipSuccess;
  const int waves = a.slot_begin && class_rows <= 32 ? a.slot_count : a.item_count;
  const dim3 grid((waves + kWavesPerWg - 1) / kWavesPerWg), block(64 * kWavesPerWg);
#define PMATTN_LAUNCH(D, NT, CONC, SMODE)                                                            \
  do {                                                                                              \
    if (a.row_mask) hipLaunchKernelGGL((attn_bf16_kernel<D, NT, true, CONC, SMODE>), grid, block, 0, st, a); \
    else hipLaunchKernelGGL((attn_bf16_kernel<D, NT, false, CONC, SMODE>), grid, block, 0, st, a);  \
  } while (0)
#define PMATTN_LAUNCH_S(D, NT, CONC)                          \
  do {                                                       \
    if (stream == 1) PMATTN_LAUNCH(D, NT, CONC, 1);          \
    else if (stream == 2) PMATTN_LAUNCH(D, NT, CONC, 2);     \
    else PMATTN_LAUNCH(D, NT, CONC, 0);                      \
  } while (0)
  // 16- and 32-row tasks stream unshared KV; 64-row tasks always cache it
#define PMATTN_LAUNCH_D(D)                                             \
  do {                                                                \
    if (class_rows <= 16) {                                           \
      if (concurrent) PMATTN_LAUNCH_S(D, 1, true);                    \
      else PMATTN_LAUNCH_S(D, 1, false);                              \
    } else if (class_rows <= 32) PMATTN_LAUNCH_S(D, 2, false);        \
    else PMATTN_LAUNCH(D, 4, false, 0);                               \
  } while (0)
  if (head_dim == 128) PMATTN_LAUNCH_D(128);
  else PMATTN_LAUNCH_D(64);
#undef PMATTN_LAUNCH_D
#undef PMATTN_LAUNCH_S
#undef PMATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace pmattn
