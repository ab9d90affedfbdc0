// Paged KV append for gfx950: the step before attention writes this step's
// keys and values into the pool slots that the block table names (XY-Serve
// pith review, "Core claim" and Figure 7, token-wise K/V reuse in paged
// blocks; PagedAttention by title).
//
// One 128-thread workgroup per (append unit, kv head): a unit is the (up to
// 16) new tokens of one sequence that fall into one block. Both pool layouts
// keep a block's tokens together per channel group, so a unit that fills a
// whole block writes whole cache lines:
//   K [blk][h][d/x][16][x]: one 16-byte piece per (head, group, token), with
//     tokens the fastest index, so a full block's group is 256 contiguous
//     bytes;
//   V [blk][h][d][16]: one thread per (head, channel) writes the unit's slots
//     of that channel, as 16-byte stores when the unit covers the block.
// Pure data movement: HBM bound, 2 x (K + V) bytes of the new rows.
#include "attn_kernels.h"
#include "pmattn_radix.h"

namespace pmattn {
namespace {

typedef const int32_t __attribute__((address_space(4)))* cint_p;

template <typename T, int D>
__global__ __launch_bounds__(128) void kv_append_kernel(AppendArgs a) {
  constexpr int X = 16 / sizeof(T);  // channels per 16-byte group
  constexpr int NG = D / X;          // groups per token and head
  const cint_p up = (cint_p)(a.units + blockIdx.x);
  const int seq = up[0], row_begin = up[1], n_tok = up[2], block_index = up[3], slot0 = up[4];
  const int h = blockIdx.y, hkv = a.hkv;
  const int64_t blk = ((cint_p)a.block_table)[(int64_t)seq * a.bt_stride + block_index];
  const int64_t row_stride = (int64_t)hkv * D;
  const T* __restrict__ kn = static_cast<const T*>(a.k_new) + ((int64_t)row_begin * hkv + h) * D;
  const T* __restrict__ vn = static_cast<const T*>(a.v_new) + ((int64_t)row_begin * hkv + h) * D;
  T* __restrict__ kp = static_cast<T*>(a.k_pool) + (blk * hkv + h) * (int64_t)(16 * D);
  T* __restrict__ vp = static_cast<T*>(a.v_pool) + (blk * hkv + h) * (int64_t)(16 * D);

  for (int idx = threadIdx.x; idx < n_tok * NG; idx += 128) {
    const int t = idx % n_tok, g = idx / n_tok;
    const uint4 v = *reinterpret_cast<const uint4*>(kn + t * row_stride + g * X);
    *reinterpret_cast<uint4*>(kp + g * (16 * X) + (slot0 + t) * X) = v;
  }
  for (int c = threadIdx.x; c < D; c += 128) {
    const T* src = vn + c;
    T* dst = vp + c * 16;
    if (n_tok == 16) {
      // whole block: the channel's 16 slots are 32 (bf16) or 64 (fp32) bytes
      T buf[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) buf[t] = src[t * row_stride];
#pragma unroll
      for (int w = 0; w < (int)(16 * sizeof(T) / 16); ++w)
        reinterpret_cast<uint4*>(dst)[w] = reinterpret_cast<const uint4*>(buf)[w];
    } else {
      for (int t = 0; t < n_tok; ++t) dst[slot0 + t] = src[t * row_stride];
    }
  }
}

// Copy-on-write of pool blocks: one 128-thread workgroup per (order, kv head)
// copies slots [0, slots) of block src into block dst, K and V.
template <typename T, int D>
__global__ __launch_bounds__(128) void copy_blocks_kernel(const pmattn_block_copy* copies, void* k_pool,
                                                          void* v_pool, int hkv) {
  constexpr int X = 16 / sizeof(T), NG = D / X;
  const cint_p cp = (cint_p)(copies + blockIdx.x);
  const int64_t src = cp[0], dst = cp[1];
  const int slots = cp[2];
  const int h = blockIdx.y;
  const int64_t so = (src * hkv + h) * (int64_t)(16 * D), dso = (dst * hkv + h) * (int64_t)(16 * D);
  const T* ks = static_cast<const T*>(k_pool) + so;
  T* kd = static_cast<T*>(k_pool) + dso;
  for (int idx = threadIdx.x; idx < NG * slots; idx += 128) {
    const int g = idx / slots, o = idx - g * slots;
    *reinterpret_cast<uint4*>(kd + g * (16 * X) + o * X) =
        *reinterpret_cast<const uint4*>(ks + g * (16 * X) + o * X);
  }
  const T* vs = static_cast<const T*>(v_pool) + so;
  T* vd = static_cast<T*>(v_pool) + dso;
  for (int idx = threadIdx.x; idx < D * slots; idx += 128) {
    const int c = idx / slots, o = idx - c * slots;
    vd[c * 16 + o] = vs[c * 16 + o];
  }
}

}  // namespace

hipError_t launch_copy_blocks(int head_dim, int dtype, const pmattn_block_copy* copies, int n,
                              void* k_pool, void* v_pool, int hkv, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const dim3 grid(n, hkv), block(128);
  if (dtype == PMATTN_BF16) {
    if (head_dim == 128) hipLaunchKernelGGL((copy_blocks_kernel<uint16_t, 128>), grid, block, 0, st, copies, k_pool, v_pool, hkv);
    else hipLaunchKernelGGL((copy_blocks_kernel<uint16_t, 64>), grid, block, 0, st, copies, k_pool, v_pool, hkv);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((copy_blocks_kernel<float, 128>), grid, block, 0, st, copies, k_pool, v_pool, hkv);
    else hipLaunchKernelGGL((copy_blocks_kernel<float, 64>), grid, block, 0, st, copies, k_pool, v_pool, hkv);
  }
  return hipGetLastError();
}

hipError_t launch_kv_append(int head_dim, int dtype, const AppendArgs& a, hipStream_t st) {
  if (a.unit_count <= 0) return hipSuccess;
  const dim3 grid(a.unit_count, a.hkv), block(128);
  if (dtype == PMATTN_BF16) {
    if (head_dim == 128) hipLaunchKernelGGL((kv_append_kernel<uint16_t, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kv_append_kernel<uint16_t, 64>), grid, block, 0, st, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((kv_append_kernel<float, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kv_append_kernel<float, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace pmattn
