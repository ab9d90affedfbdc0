// bf16 tile-task attention kernel for gfx950 (CDNA4).
//
// One wave64 runs one tile task (see pmattn_work_item): the query rows of one
// GQA group for up to 64/G tokens of one sequence, against one KV partition.
// This is the matmul-softmax-matmul tile of the XY-Serve meta-kernel
// (XY-Serve pith review, "What carries the argument"), re-planned for MFMA:
//
//   S^T = K . Q^T     v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 channels,
//                     B = 32 channels x 16 query rows  (Figure 3's QK shape,
//                     transposed so that each lane ends up owning one query
//                     row and 8 keys of it)
//   online softmax    fp32, exp2 with scale*log2(e) folded in; the row max is
//                     reduced over the 4 lanes that share a row
//   O^T += V^T . P^T  v_mfma_f32_16x16x32_bf16: A = 16 channels x 32 keys,
//                     B = P^T taken straight from the S^T accumulator lanes
//
// Keys are consumed 32 at a time (two 16-token blocks). The channel order
// inside the QK contraction and the key order inside the PV contraction are
// permuted (identically on both operands, so the sums are unchanged) so that
// every operand a lane needs is one contiguous 16-byte run in memory:
//   K operand, lane (i, g): key 8*(i/4) + 4c + i%4 of the chunk, channels
//     [g*d/4, (g+1)*d/4)  -> d/32 consecutive 16-byte loads;
//   V operand, lane (i, g): channel 16t + i, keys 8g..8g+7 of the chunk,
//     which the channel-major V block stores contiguously -> one 16-byte load.
// K and V tiles are gathered through the block table (physical ids read once
// per 64 blocks into a VGPR and broadcast with readlane); no contiguous copy
// of the KV is ever formed (the K/V concatenation the XY-Serve referee report
// blames for the baseline's losses).
//
// Masks are row-wise (XY-Serve review, "Editorial extensions": one kernel for
// prefill, decode and verify rows): key j is visible to a row at position pos
// iff j <= pos; chunks that lie wholly below the task's first position skip
// the mask (Figure 11, mask-aware computation). Keys at or past the task's end
// are never used: their scores become -inf and their V lanes are zeroed before
// the PV product, so pool slots no row can see may hold NaN (virtual padding,
// "Assumptions & free parameters").
#include "attn_kernels.h"

namespace pmattn {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

template <int D>
struct Chunk {
  static constexpr int KS = D / 32;   // QK k-steps of 32 channels
  static constexpr int DT = D / 16;   // 16-channel output tiles
  bf16x8 k[2][KS];
  bf16x8 v[DT];
};

// Issue the loads of the 32-key chunk made of physical blocks blk0, blk1.
template <int D>
__device__ __forceinline__ void load_chunk(Chunk<D>& ch, const uint16_t* __restrict__ kpool,
                                           const uint16_t* __restrict__ vpool, int blk0, int blk1,
                                           int kvh, int hkv, int i, int g) {
  constexpr int KS = Chunk<D>::KS, DT = Chunk<D>::DT;
  const int64_t blk_k = (i >> 3) ? blk1 : blk0;
  const uint16_t* kp = kpool + ((blk_k * hkv + kvh) * 16 + 8 * ((i >> 2) & 1) + (i & 3)) * D + g * 8 * KS;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int s = 0; s < KS; ++s) ch.k[c][s] = ld16(kp + 4 * c * D + 8 * s);
  const int64_t blk_v = (g >> 1) ? blk1 : blk0;
  const uint16_t* vp = vpool + ((blk_v * hkv + kvh) * D + i) * 16 + 8 * (g & 1);
#pragma unroll
  for (int t = 0; t < DT; ++t) ch.v[t] = ld16(vp + 16 * 16 * t);
}

template <int D, int NT, bool MASK>
__device__ __forceinline__ void compute_chunk(Chunk<D>& ch, const bf16x8 (&qop)[NT][D / 32],
                                              f32x4 (&o)[NT][D / 16], float (&m_run)[NT],
                                              float (&l_run)[NT], const int (&pos)[NT], int c0,
                                              int kv_end, float sl2, int g) {
  constexpr int KS = D / 32, DT = D / 16;
  const int kbase = c0 + 8 * g;  // key of this lane's first score slot
  if (MASK) {
    const int nv = kv_end - kbase;  // V lanes past the task's end must be zero
    if (nv < 8) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= nv) ch.v[t][j] = (__bf16)0.0f;
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.k[0][s], qop[n][s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.k[1][s], qop[n][s], s1, 0, 0, 0);
    }
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    if (MASK) {
      const int lim = min(pos[n] + 1, kv_end) - kbase;  // slots j < lim are visible
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = (j < lim) ? sv[j] : kNegInf;
    }
    float mx = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run[n], mx);
    const float ms = (m_new == kNegInf) ? 0.f : m_new * sl2;
    const float alpha = __builtin_amdgcn_exp2f(m_run[n] * sl2 - ms);
    m_run[n] = m_new;
    f32x8 p;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(sv[j] * sl2 - ms);
      psum += p[j];
    }
    l_run[n] = l_run[n] * alpha + psum;
    const bf16x8 pb = __builtin_convertvector(p, bf16x8);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      o[n][t] *= alpha;
      o[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.v[t], pb, o[n][t], 0, 0, 0);
    }
  }
}

template <int D, int NT>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 32, DT = D / 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= a.item_count) return;
  const pmattn_work_item it = a.items[idx];
  const int i = lane & 15, g = lane >> 4;
  const int G = a.group, hq = a.hq, hkv = a.hkv, kvh = it.kv_head;
  const int M = it.n_tok * G;
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* __restrict__ vpool = static_cast<const uint16_t*>(a.v_pool);

  // Q operand (B of the QK product): lane (i, g) holds query row 16n+i,
  // channels [g*D/4, (g+1)*D/4), in k-step slices of 8.
  bf16x8 qop[NT][KS];
  int pos[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int m = 16 * n + i;
    pos[n] = -1;
    if (m < M) {
      const int t = m / G;
      pos[n] = it.pos_begin + t;
      const uint16_t* src = qp + ((int64_t)(it.row_begin + t) * hq + kvh * G + (m - t * G)) * D + g * 8 * KS;
#pragma unroll
      for (int s = 0; s < KS; ++s) qop[n][s] = ld16(src + 8 * s);
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qop[n][s] = (bf16x8)(__bf16)0.0f;
    }
  }

  f32x4 o[NT][DT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    m_run[n] = kNegInf;
    l_run[n] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) o[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // Physical block ids of up to 64 consecutive logical blocks, one per lane.
  const int32_t* bt_row = a.block_table + (int64_t)it.seq * a.bt_stride;
  const int nblk_end = (it.kv_end + 15) >> 4;
  int ids_base = it.kv_begin >> 4;
  int ids = (ids_base + lane < nblk_end) ? bt_row[ids_base + lane] : 0;
  auto block_id = [&](int bi) -> int {
    if (bi - ids_base >= 64) {
      ids_base = bi;
      ids = (ids_base + lane < nblk_end) ? bt_row[ids_base + lane] : 0;
    }
    return __builtin_amdgcn_readlane(ids, bi - ids_base);
  };
  auto chunk_blocks = [&](int c, int& b0, int& b1) {
    const int bi = c >> 4;
    b0 = block_id(bi);
    b1 = (bi + 1 < nblk_end) ? block_id(bi + 1) : b0;
  };

  const float sl2 = a.scale_log2;
  const int kv_end = it.kv_end;
  const int first_pos = it.pos_begin;
  Chunk<D> A, B;
  int c0 = it.kv_begin, b0, b1;
  chunk_blocks(c0, b0, b1);
  load_chunk<D>(A, kpool, vpool, b0, b1, kvh, hkv, i, g);
  // Two named buffers: while one chunk is computed the next one is in flight.
  // The prefetch is unconditional; past the last chunk it re-reads the current
  // one (an L2 hit, same block ids) so that the wait counts stay static.
  for (;;) {
    int cn = c0 + 32;
    bool more = cn < kv_end;
    if (more) chunk_blocks(cn, b0, b1);
    load_chunk<D>(B, kpool, vpool, b0, b1, kvh, hkv, i, g);
    if (c0 + 31 > first_pos || c0 + 32 > kv_end)
      compute_chunk<D, NT, true>(A, qop, o, m_run, l_run, pos, c0, kv_end, sl2, g);
    else
      compute_chunk<D, NT, false>(A, qop, o, m_run, l_run, pos, c0, kv_end, sl2, g);
    if (!more) break;
    c0 = cn;
    cn = c0 + 32;
    more = cn < kv_end;
    if (more) chunk_blocks(cn, b0, b1);
    load_chunk<D>(A, kpool, vpool, b0, b1, kvh, hkv, i, g);
    if (c0 + 31 > first_pos || c0 + 32 > kv_end)
      compute_chunk<D, NT, true>(B, qop, o, m_run, l_run, pos, c0, kv_end, sl2, g);
    else
      compute_chunk<D, NT, false>(B, qop, o, m_run, l_run, pos, c0, kv_end, sl2, g);
    if (!more) break;
    c0 = cn;
  }

  // Epilogue: lane (i, g) owns channels 16t + 4g + r of row 16n + i.
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int m = 16 * n + i;
    float l = l_run[n];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (m >= M) continue;
    const int t = m / G;
    const int64_t row = it.row_begin + t;
    const int qh = kvh * G + (m - t * G);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? m_run[n] * a.scale + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
    if (it.part < 0) {
      uint16_t* dst = static_cast<uint16_t*>(a.out) + (row * hq + qh) * D + 4 * g;
#pragma unroll
      for (int tt = 0; tt < DT; ++tt) {
        f32x4 v = o[n][tt] * inv;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 b = __builtin_convertvector(v, bf16x4);
        *reinterpret_cast<uint2*>(dst + 16 * tt) = __builtin_bit_cast(uint2, b);
      }
      if (a.lse && g == 0) a.lse[row * hq + qh] = lse;
    } else {
      const int64_t rec = (int64_t)it.part + m;
      float* dst = a.part_o + rec * D + 4 * g;
#pragma unroll
      for (int tt = 0; tt < DT; ++tt) *reinterpret_cast<f32x4*>(dst + 16 * tt) = o[n][tt] * inv;
      if (g == 0) a.part_lse[rec] = lse;
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(int head_dim, int class_rows, const AttnArgs& a, hipStream_t st) {
  if (a.item_count <= 0) return hipSuccess;
  const dim3 grid((a.item_count + 3) / 4), block(256);
#define PMATTN_LAUNCH(D, NT) hipLaunchKernelGGL((attn_bf16_kernel<D, NT>), grid, block, 0, st, a)
  if (head_dim == 128) {
    if (class_rows <= 16) PMATTN_LAUNCH(128, 1);
    else if (class_rows <= 32) PMATTN_LAUNCH(128, 2);
    else PMATTN_LAUNCH(128, 4);
  } else {
    if (class_rows <= 16) PMATTN_LAUNCH(64, 1);
    else if (class_rows <= 32) PMATTN_LAUNCH(64, 2);
    else PMATTN_LAUNCH(64, 4);
  }
#undef PMATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace pmattn
