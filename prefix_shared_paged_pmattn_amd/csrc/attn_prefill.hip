// bf16 workgroup kernel for gfx950: one workgroup per task of up to 128 rows
// (prefill chunks, long verify runs). The task body, its LDS staging and its
// MFMA tiling are in task_wg.h.
#include "task_wg.h"

namespace pmattn {
namespace {

template <int D, bool TREE, int WAVES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
void attn_prefill_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[Cfg<D>::LDS_ELEMS];
  if ((int)blockIdx.x >= a.item_count) return;  // uniform over the workgroup
  const pmattn_work_item it = load_item(a.items, blockIdx.x);
  wg_task<D, TREE>(a, it, a.q_row, lds);
}

}  // namespace

namespace {
template <int D>
void launch_d(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.item_count), block(256);
  if (a.row_mask) hipLaunchKernelGGL((attn_prefill_kernel<D, true, 3>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_prefill_kernel<D, false, 3>), grid, block, 0, st, a);
}
}  // namespace

hipError_t launch_attn_prefill(int head_dim, const AttnArgs& a, hipStream_t st) {
  if (a.item_count <= 0) return hipSuccess;
  if (head_dim == 128) launch_d<128>(a, st);
  else launch_d<64>(a, st);
  return hipGetLastError();
}

}  // namespace pmattn
