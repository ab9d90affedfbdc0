// float32 attention (the plumbing path) and the log-sum-exp merge kernel.
#include "attn_kernels.h"

namespace pmattn {
namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave per tile task, one query row at a time: lanes score 64 keys in
// parallel (serial dot products), then accumulate P.V with lane = channel.
// Plain online softmax in fp32 with expf/logf. Correct for any task shape;
// used for PMATTN_F32 batches, whose sizes are small.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int V = D / 64;  // channels per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= a.item_count) return;
  const pmattn_work_item it = a.items[idx];
  const int G = a.group, hq = a.hq, hkv = a.hkv, kvh = it.kv_head;
  const float* __restrict__ qp = static_cast<const float*>(a.q);
  const float* __restrict__ kpool = static_cast<const float*>(a.k_pool);
  const float* __restrict__ vpool = static_cast<const float*>(a.v_pool);
  const int32_t* bt_row = a.block_table + (int64_t)it.seq * a.bt_stride;
  const int M = it.n_tok * G;
  for (int m = 0; m < M; ++m) {
    const int t = m / G;
    const int qh = kvh * G + (m - t * G);
    const int64_t row = it.row_begin + t;
    const int kend = min(it.kv_end, it.pos_begin + t + 1);
    const int rpos = it.pos_begin + t;
    const uint64_t rel = a.row_mask ? a.row_mask[row] : ~0ull;  // token tree
    const float* qrow = qp + ((a.q_row ? (int64_t)a.q_row[row] : row) * hq + qh) * D;
    float m_run = kNegInf, l_run = 0.f, acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    for (int kb = it.kv_begin; kb < kend; kb += 64) {
      const int j = kb + lane;
      const int dd = rpos - j;
      const bool valid = j < kend && !((unsigned)dd < 64u && !((rel >> dd) & 1ull));
      const int blk = valid ? bt_row[j >> 4] : 0;
      float s = kNegInf;
      if (valid) {
        // grouped K block [D/4][16][4]: channel c of slot o at (c/4)*64 + 4o + c%4
        const float* kr = kpool + ((int64_t)blk * hkv + kvh) * 16 * D + 4 * (j & 15);
        float dot = 0.f;
        for (int c = 0; c < D; ++c) dot = fmaf(qrow[c], kr[(c >> 2) * 64 + (c & 3)], dot);
        s = dot * a.scale;
      }
      // a window can hide every key (a token tree over a KV partition)
      const float m_new = fmaxf(m_run, wave_max(s));
      const float alpha = m_new == kNegInf ? 1.f : expf(m_run - m_new);
      const float p = valid ? expf(s - m_new) : 0.f;
      l_run = l_run * alpha + wave_sum(p);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] *= alpha;
      const int nk = min(64, kend - kb);
      for (int jj = 0; jj < nk; ++jj) {
        const float pj = __shfl(p, jj);
        const int bj = __shfl(blk, jj);
        const float* vr = vpool + ((int64_t)bj * hkv + kvh) * D * 16 + ((kb + jj) & 15);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = fmaf(pj, vr[(lane + 64 * v) * 16], acc[v]);
      }
      m_run = m_new;
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse = l_run > 0.f ? m_run + logf(l_run) : kNegInf;
    if (it.part < 0) {
      float* dst = static_cast<float*>(a.out) + (row * hq + qh) * D;
#pragma unroll
      for (int v = 0; v < V; ++v) dst[lane + 64 * v] = acc[v] * inv;
      if (a.lse && lane == 0) a.lse[row * hq + qh] = lse;
    } else {
      const int64_t rec = (int64_t)it.part + m;
#pragma unroll
      for (int v = 0; v < V; ++v) a.part_o[rec * D + lane + 64 * v] = acc[v] * inv;
      if (lane == 0) a.part_lse[rec] = lse;
    }
  }
}

// The group kernel (below) takes its partials kGroupBatch at a time; the
// launcher gives it every merge of at most kGroupBatch partials per output,
// and any merge whose outputs average at most kGroupMeanParts.
constexpr int kGroupBatch = 8;
constexpr int kGroupMeanParts = 12;

// Log-sum-exp merge of partial results (Flash-Decoding, reference list of the
// XY-Serve pith review): out = sum_p w_p O_p / sum_p w_p with
// w_p = exp(lse_p - max lse); lse = max + ln sum w_p. Partials of weight 0
// (empty, lse -inf) are left out of the sum, so their output slots may hold
// anything; if all are empty the output is 0 and lse is -inf.
//
// Group variant, for merges of a few partials: a group of 16 lanes merges one
// output (row, head); lane j owns channels
// [D/16 j, D/16 (j + 1)), read as 16-byte pieces. Every lane walks the
// partials itself (no cross-lane reductions), kGroupBatch (8) at a time: the
// batch's record ids, lse values and output pieces are independent loads
// issued together, then folded in with an online max (running max m, sums
// rescaled by exp(m_old - m_new) when it grows). A merge of up to eight
// partials costs one memory round trip after its row record.
template <int D, bool BF16_OUT>
__global__ __launch_bounds__(256) void merge_group_kernel(MergeArgs a) {
  constexpr int C = D / 16;   // channels per lane (8 or 4)
  constexpr int Q = C / 4;    // 16-byte pieces per lane and partial
  constexpr int B = kGroupBatch;  // partials per batch
  constexpr float kLog2e = 1.44269504088896340736f;
  const int w = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (w >= a.count) return;
  int64_t rec0, stride, row;
  int np, qh;
  if (a.rows) {
    const pmattn_merge_row mr = a.rows[w];
    rec0 = mr.rec0;
    stride = mr.rec_stride;
    np = mr.nparts;
    row = mr.row;
    qh = mr.q_head;
  } else {
    rec0 = w;
    stride = (int64_t)a.implicit_rows * a.hq;
    np = a.implicit_parts;
    row = w / a.hq;
    qh = w - (int)row * a.hq;
  }
  // record id of partial p: strided (rec0 + p * stride) or listed
  // (rec_index[rec0 + p], rows of cascade sharers)
  const bool listed = stride < 0;
  float m = kNegInf, tot = 0.f;
  f32x4 acc[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) acc[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < np; p0 += B) {
    int64_t rid[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int p = p0 + u;
      rid[u] = p >= np ? -1 : listed ? (int64_t)a.rec_index[rec0 + p] : rec0 + (int64_t)p * stride;
    }
    float l[B];
    f32x4 x[B][Q];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      l[u] = rid[u] >= 0 ? a.part_lse[rid[u]] : kNegInf;
      const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + (rid[u] >= 0 ? rid[u] : 0) * D + C * j);
#pragma unroll
      for (int q = 0; q < Q; ++q) x[u][q] = src[q];
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (l[u] == kNegInf) continue;  // empty partition: its loaded slot (maybe never written) is unused
      const float m_new = fmaxf(m, l[u]);
      const float alpha = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * kLog2e);
      const float wt = __builtin_amdgcn_exp2f((l[u] - m_new) * kLog2e);
      tot = tot * alpha + wt;
#pragma unroll
      for (int q = 0; q < Q; ++q) acc[q] = acc[q] * alpha + wt * x[u][q];
      m = m_new;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int64_t o = (row * a.hq + qh) * D + C * j;
  if (BF16_OUT) {
    typedef __bf16 bf16xC __attribute__((ext_vector_type(C)));
    typedef float f32xC __attribute__((ext_vector_type(C)));
    f32xC v;
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = acc[c / 4][c % 4] * inv;
    *reinterpret_cast<bf16xC*>(static_cast<__bf16*>(a.out) + o) = __builtin_convertvector(v, bf16xC);
  } else {
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o);
#pragma unroll
    for (int q = 0; q < Q; ++q) dst[q] = acc[q] * inv;
  }
  if (a.lse && j == 0) a.lse[row * a.hq + qh] = tot > 0.f ? m + logf(tot) : kNegInf;
}

// Wave variant, for merges with many partials: one wave per output (row,
// head); lane owns D/64 consecutive channels. Latency-lean: lane p loads lse_p (64 partials per round) and the max and the
// weight sum are wave reductions. The partial outputs of the first kPre
// partials do not depend on the weights, so their loads are issued together
// with the lse loads; a merge of up to kPre partials costs one memory round
// trip after its row record. Further partials are loaded in unrolled groups.
template <int D, bool BF16_OUT>
__global__ __launch_bounds__(256) void merge_wave_kernel(MergeArgs a) {
  constexpr int V = D / 64;
  constexpr int kPre = 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + wave;
  if (w >= a.count) return;
  int64_t rec0, stride;
  int np, qh;
  int64_t row;
  if (a.rows) {
    const pmattn_merge_row mr = a.rows[w];
    rec0 = mr.rec0;
    stride = mr.rec_stride;
    np = mr.nparts;
    row = mr.row;
    qh = mr.q_head;
  } else {
    rec0 = w;
    stride = (int64_t)a.implicit_rows * a.hq;
    np = a.implicit_parts;
    row = w / a.hq;
    qh = w - (int)row * a.hq;
  }
  // record id of partial p0 + lane: strided (rec0 + p * stride) or listed
  // (rec_index[rec0 + p], rows of cascade sharers); partial u's id reaches
  // every lane by a broadcast
  const bool listed = stride < 0;
  auto rec_of = [&](int p0) -> int64_t {
    const int p = p0 + lane;
    if (p >= np) return 0;
    return listed ? (int64_t)a.rec_index[rec0 + p] : rec0 + (int64_t)p * stride;
  };
  const int64_t rid0 = rec_of(0);
  const float* po = a.part_o + lane * V;
  float pre[kPre][V];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int64_t ru = __shfl(rid0, u);
#pragma unroll
    for (int v = 0; v < V; ++v) pre[u][v] = u < np ? po[ru * D + v] : 0.f;
  }
  const float l0 = lane < np ? a.part_lse[rid0] : kNegInf;
  float mx = l0;
  for (int p0 = 64; p0 < np; p0 += 64) {
    const int64_t r = rec_of(p0);
    if (p0 + lane < np) mx = fmaxf(mx, a.part_lse[r]);
  }
  mx = wave_max(mx);
  float acc[V], tot = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  if (mx != kNegInf) {
    for (int p0 = 0; p0 < np; p0 += 64) {
      const int pn = min(64, np - p0);
      const int64_t rid = p0 == 0 ? rid0 : rec_of(p0);
      float l = l0;
      if (p0 > 0) l = lane < pn ? a.part_lse[rid] : kNegInf;
      const float wt = (l == kNegInf) ? 0.f : expf(l - mx);
      tot += wave_sum(wt);
      int q = 0;
      if (p0 == 0) {
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          const float wu = __shfl(wt, u);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] = fmaf(wu, wu != 0.f ? pre[u][v] : 0.f, acc[v]);
        }
        q = min(kPre, pn);
      }
      for (; q + 8 <= pn; q += 8) {
        float src[8][V];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t ru = __shfl(rid, q + u);
#pragma unroll
          for (int v = 0; v < V; ++v) src[u][v] = po[ru * D + v];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wu = __shfl(wt, q + u);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] = fmaf(wu, wu != 0.f ? src[u][v] : 0.f, acc[v]);
        }
      }
      for (; q < pn; ++q) {
        const float wu = __shfl(wt, q);
        const int64_t ru = __shfl(rid, q);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const float x = po[ru * D + v];
          acc[v] = fmaf(wu, wu != 0.f ? x : 0.f, acc[v]);
        }
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int64_t o = (row * a.hq + qh) * D + lane * V;
  if (BF16_OUT) {
    __bf16* dst = static_cast<__bf16*>(a.out) + o;
#pragma unroll
    for (int v = 0; v < V; ++v) dst[v] = (__bf16)(acc[v] * inv);
  } else {
    float* dst = static_cast<float*>(a.out) + o;
#pragma unroll
    for (int v = 0; v < V; ++v) dst[v] = acc[v] * inv;
  }
  if (a.lse && lane == 0) a.lse[row * a.hq + qh] = tot > 0.f ? mx + logf(tot) : kNegInf;
}

}  // namespace

hipError_t launch_attn_f32(int head_dim, const AttnArgs& a, hipStream_t st) {
  if (a.item_count <= 0) return hipSuccess;
  const dim3 grid((a.item_count + 3) / 4), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, int out_dtype, const MergeArgs& a, hipStream_t st) {
  if (a.count <= 0) return hipSuccess;
  const bool bf = out_dtype == PMATTN_BF16;
  // Measured on MI355X: the group kernel takes 20 us where the wave kernel
  // takes 47 (54k outputs of 1-3 partials); with tens of partials per output
  // the wave kernel's lane-parallel lse loads win (25 vs 22 us). In between,
  // the mean count decides: 8,192 outputs of 2-17 partials (mean 9.1) merge
  // in 14.5-14.8 us by groups against 16.5 by waves; 4,096 of 13-16 listed
  // partials (mean 14.8) in 12.1-12.3 against 11.2-11.9, and 512 of 16 in 8.2
  // against 7.4.
  if (a.max_parts <= kGroupBatch || a.total_parts <= (int64_t)kGroupMeanParts * a.count) {
    const dim3 grid((a.count + 15) / 16), block(256);
    if (head_dim == 128) {
      if (bf) hipLaunchKernelGGL((merge_group_kernel<128, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((merge_group_kernel<128, false>), grid, block, 0, st, a);
    } else {
      if (bf) hipLaunchKernelGGL((merge_group_kernel<64, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((merge_group_kernel<64, false>), grid, block, 0, st, a);
    }
  } else {
    const dim3 grid((a.count + 3) / 4), block(256);
    if (head_dim == 128) {
      if (bf) hipLaunchKernelGGL((merge_wave_kernel<128, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((merge_wave_kernel<128, false>), grid, block, 0, st, a);
    } else {
      if (bf) hipLaunchKernelGGL((merge_wave_kernel<64, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((merge_wave_kernel<64, false>), grid, block, 0, st, a);
    }
  }
  return hipGetLastError();
}

}  // namespace pmattn
