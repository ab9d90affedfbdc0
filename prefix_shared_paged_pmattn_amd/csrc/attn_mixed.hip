// One kernel for a mixed batch: the prefill-chunk, verify and decode tasks of
// one plan in a single launch (XY-Serve review, "Core claim": attention
// becomes a single meta-kernel whose tile tasks, listed in a table, are
// reordered across cores; "Editorial extensions": one kernel with row-wise
// masks serves the three kinds of rows).
//
// Workgroup i (4 waves) runs entry i of the plan's mixed table:
// * a workgroup task (more than 32 rows: prefill tiles): the four waves share
//   each K/V chunk through LDS (task_wg.h);
// * or a bundle of four wave tasks of up to 32 rows (decode rows, verify
//   drafts): each wave streams its own task's K/V into registers
//   (task_wave.h; 32-row tasks in 16-key chunks to fit the registers).
// Both bodies fit the same budget, 168 registers and 48 KiB of LDS, so three
// workgroups of either kind share a CU. The planner interleaves the two kinds
// in cost proportion within each XCD's share of the table; the dispatcher
// hands entries to CUs in table order, so every CU holds both kinds while
// they run: decode waves stream HBM beside MFMA-bound prefill tiles instead of
// the two kinds taking whole CUs in turn (POD-Attention, XY-Serve review
// reference list, overlaps the two in one kernel the same way).
#include "plan_internal.h"
#include "task_wave.h"
#include "task_wg.h"

namespace pmattn {
namespace {

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_mixed_kernel(MixedArgs m) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[Cfg<D>::LDS_ELEMS];
  const AttnArgs& a = m.a;
  if ((int)blockIdx.x >= m.entries) return;  // uniform over the workgroup
  const int entry = ((cint_p)m.table)[blockIdx.x];
  if (!(entry & 1)) {
    const pmattn_work_item it = load_item(a.items, entry >> 2);
    wg_task<D, false>(a, it, (entry & 2) ? a.q_row : nullptr, lds);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = ((cint_p)m.bundles)[(entry >> 2) * 4 + wave];
  if (e < 0) return;
  const int idx = e >> 1, lane = threadIdx.x & 63;
  const pmattn_work_item it = load_item(a.items, idx);
  const int32_t* qr = (e & 1) ? a.q_row : nullptr;
  const bool stream = ((cint_p)a.item_stream)[idx];
  if (it.n_tok * a.group <= 16) {
    if (stream) run_task<D, 1, false, true, true>(a, it, qr, lane);
    else run_task<D, 1, false, true, false>(a, it, qr, lane);
  } else {
    // 17..32 rows (verify drafts): two 16-row tiles against 16-key chunks,
    // which keeps the wave within the kernel's 168 registers
    if (stream) run_task<D, 2, false, true, true, 1>(a, it, qr, lane);
    else run_task<D, 2, false, true, false, 1>(a, it, qr, lane);
  }
}

}  // namespace

hipError_t launch_attn_mixed(int head_dim, const MixedArgs& m, hipStream_t st) {
  if (m.entries <= 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((attn_mixed_kernel<128>), dim3(m.entries), dim3(256), 0, st, m);
  else hipLaunchKernelGGL((attn_mixed_kernel<64>), dim3(m.entries), dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace pmattn
