// Wave tile task: one wave64 runs one task (see pmattn_work_item), the query
// rows of one GQA group for up to 64/G tokens of one sequence against one KV
// partition. Used by the one-wave kernel (attn_bf16.hip) and by the
// mixed-batch kernel (attn_mixed.hip).
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
// every operand a lane needs is a contiguous run in memory and every load
// instruction covers whole cache lines:
//   K operand, tile c = block c, lane (i, g): slot i, channel group 4s + g
//     of the grouped K block [d/8][16][8] -> d/32 16-byte loads per tile;
//   V operand, lane (i, g): channel 16t + i, slots 4g..4g+3 of each block,
//     which the channel-major V block stores contiguously -> two 8-byte loads.
// K and V tiles are gathered through the block table (physical ids fetched
// with scalar loads a chunk ahead); no contiguous copy of the KV is ever
// formed (the K/V concatenation the XY-Serve referee report blames for the
// baseline's losses).
//
// Masks are row-wise (XY-Serve review, "Editorial extensions": one kernel for
// prefill, decode and verify rows): key j is visible to a row at position pos
// iff j <= pos. The mask costs a few selects per 32 keys and is applied to
// every chunk, so the streaming loop has no data-dependent branch. Keys at or
// past the task's end are never used: their scores become -inf and their V
// lanes are zeroed before the PV product, so pool slots no row can see may
// hold NaN (virtual padding, "Assumptions & free parameters").
//
// Instances: head dim D; NT 16-row tiles per task (1 decode, 2 verify, 4);
// TREE token-tree masks; CONC the launch runs beside workgroup tasks of the
// same plan (16-row tasks then keep one chunk buffer at 3 waves per SIMD
// instead of two at 2, so that they pack with the 3-wave workgroup kernel);
// SMODE how K/V are loaded: 0 cacheable, 1 non-temporal, 2 per the task's
// flag from the planner (non-temporal when no other row tile reads its
// blocks, so shared prefix blocks stay in the caches for their other readers).
#pragma once

#include <type_traits>

#include "task_common.h"

namespace pmattn {
namespace {

// A chunk is NB blocks: 32 keys (NB = 2), or 16 (NB = 1: half the registers
// in flight, for tasks whose other state fills the register budget).
template <int D, int NB = 2>
struct Chunk {
  static constexpr int KS = D / 32;   // QK k-steps of 32 channels
  static constexpr int DT = D / 16;   // 16-channel output tiles
  bf16x8 k[NB][KS];
  // V operand of output tile t: slots 4g..4g+3 of both blocks (NB = 2), or
  // of the one block (NB = 1; the operand's upper half, the absent block, is
  // zero)
  typename std::conditional<NB == 2, bf16x8, u32x2>::type v[DT];
};

// Issue the loads of the 32-key chunk made of physical blocks blk0, blk1.
// Key tile c of the QK product is block c: lane (i, g) holds slot i, and for
// k-step s the 8 channels of group 4s + g, i.e. one 16-byte piece of the
// grouped K block [D/8][16][8]; a load instruction covers 1 KiB of one block.
// Contraction position 8g + 4c + r of the PV product is slot 4g + r of block
// c, so lane (channel, g) of V^T takes 4 slots of each block: two 8-byte
// pieces of the channel-major V blocks (512 contiguous bytes per instruction
// and block).

// STREAM: no other sequence's task reads these blocks, so the loads carry
// the non-temporal hint and leave the caches to data that is read again.
template <bool STREAM, typename T>
__device__ __forceinline__ T ld_kv(const uint16_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}

template <int D, bool STREAM, int NB>
__device__ __forceinline__ void load_chunk(Chunk<D, NB>& ch, const uint16_t* __restrict__ kpool,
                                           const uint16_t* __restrict__ vpool, int blk0, int blk1,
                                           int kvh, int hkv, int i, int g) {
  constexpr int KS = Chunk<D, NB>::KS, DT = Chunk<D, NB>::DT;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int64_t bk = c ? blk1 : blk0;
    const uint16_t* kp = kpool + ((bk * hkv + kvh) * (D / 8) + g) * 128 + 8 * i;
#pragma unroll
    for (int s = 0; s < KS; ++s) ch.k[c][s] = __builtin_bit_cast(bf16x8, ld_kv<STREAM, u32x4>(kp + 512 * s));
  }
  const uint16_t* vp0 = vpool + (((int64_t)blk0 * hkv + kvh) * D + i) * 16 + 4 * g;
  if constexpr (NB == 1) {
#pragma unroll
    for (int t = 0; t < DT; ++t) ch.v[t] = ld_kv<STREAM, u32x2>(vp0 + 256 * t);
  } else {
    const uint16_t* vp1 = vpool + (((int64_t)blk1 * hkv + kvh) * D + i) * 16 + 4 * g;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const u32x2 x0 = ld_kv<STREAM, u32x2>(vp0 + 256 * t);
      const u32x2 x1 = ld_kv<STREAM, u32x2>(vp1 + 256 * t);
      ch.v[t] = __builtin_bit_cast(bf16x8, (u32x4){x0.x, x0.y, x1.x, x1.y});
    }
  }
}

// The V operand of output tile t as the MFMA takes it.
template <int D, int NB>
__device__ __forceinline__ bf16x8 v_operand(const Chunk<D, NB>& ch, int t) {
  if constexpr (NB == 1) return __builtin_bit_cast(bf16x8, (u32x4){ch.v[t].x, ch.v[t].y, 0u, 0u});
  else return ch.v[t];
}

// Zero the V lanes of keys at or past the task's end (only the last, partial
// chunk has any; the masks are all-ones elsewhere): a masked key has weight
// exactly 0, but 0 * NaN would still poison the PV product if the slot holds
// garbage.
// Element e of a lane's V operand is key c0 + 4g + slot_off(e).
__device__ __forceinline__ constexpr int slot_off(int e) { return 16 * (e >> 2) + (e & 3); }

template <int D, int NB>
__device__ __forceinline__ void zero_tail_v(Chunk<D, NB>& ch, int c0, int kv_end, int g) {
  const int nv = kv_end - (c0 + 4 * g);
  uint32_t keep[4];
#pragma unroll
  for (int w = 0; w < 4; ++w)
    keep[w] = (slot_off(2 * w + 1) < nv ? 0xFFFF0000u : 0u) | (slot_off(2 * w) < nv ? 0x0000FFFFu : 0u);
#pragma unroll
  for (int t = 0; t < Chunk<D, NB>::DT; ++t) {
    if constexpr (NB == 1) {
      ch.v[t].x &= keep[0];
      ch.v[t].y &= keep[1];
    } else {
      uint4 u = __builtin_bit_cast(uint4, ch.v[t]);
      u.x &= keep[0];
      u.y &= keep[1];
      u.z &= keep[2];
      u.w &= keep[3];
      ch.v[t] = __builtin_bit_cast(bf16x8, u);
    }
  }
}

// One 32-key chunk: scores, row-wise causal mask, online softmax, PV.
// The mask is applied unconditionally (a handful of selects per 32 keys) so
// that the streaming loop has no data-dependent branches.
// Token trees: rel[n] bit k set = the key k positions before row n's own is
// visible; dbase[n] = that row's position - 4g. Chunks starting above tree_from
// hold keys within 64 positions of some row of the task; only they are tested.
template <int NT>
struct TreeRows {
  uint64_t rel[NT];
  int dbase[NT];
  int tree_from;
};

template <int D, int NT, bool TREE, int NB>
__device__ __forceinline__ void wave_chunk(const Chunk<D, NB>& ch, const bf16x8 (&qop)[NT][D / 32],
                                              f32x4 (&o)[NT][D / 16], float (&m_run)[NT],
                                              float (&l_run)[NT], const int (&lim_base)[NT], int c0,
                                              float sl2, int g, const TreeRows<NT>& tr) {
  constexpr int KS = D / 32, DT = D / 16, NS = 4 * NB;  // scores per lane
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.k[0][s], qop[n][s], s0, 0, 0, 0);
      if constexpr (NB == 2) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.k[1][s], qop[n][s], s1, 0, 0, 0);
    }
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    // score j holds key c0 + 4g + slot_off(j) (tile j/4, accumulator row
    // 4g + j%4); visible iff key < min(pos + 1, kv_end)
    const int lim = lim_base[n] - c0;
#pragma unroll
    for (int j = 0; j < NS; ++j) sv[j] = (slot_off(j) < lim) ? sv[j] : kNegInf;
    if constexpr (TREE) {
      if (c0 > tr.tree_from) {
        const int db = tr.dbase[n] - c0;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int dd = db - slot_off(j);  // how far before the row's position
          const bool hide = (unsigned)dd < 64u && !((tr.rel[n] >> dd) & 1ull);
          sv[j] = hide ? kNegInf : sv[j];
        }
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int j = 1; j < NS; ++j) mx = fmaxf(mx, sv[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run[n], mx);
    const float ms = (m_new == kNegInf) ? 0.f : m_new * sl2;
    const float alpha = __builtin_amdgcn_exp2f(m_run[n] * sl2 - ms);
    m_run[n] = m_new;
    f32x8 p = {};
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      p[j] = __builtin_amdgcn_exp2f(sv[j] * sl2 - ms);
      psum += p[j];
    }
    l_run[n] = l_run[n] * alpha + psum;
    const bf16x8 pb = __builtin_convertvector(p, bf16x8);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      o[n][t] *= alpha;
      o[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_operand(ch, t), pb, o[n][t], 0, 0, 0);
    }
  }
}

// Occupancy and chunk buffers per wave, by tile count NT and whether the
// launch shares the chip with workgroup tasks of the same plan (CONC).
// 16-row (decode) tasks double-buffer at 2 waves/SIMD (253 VGPRs): two chunks
// in flight per wave, eight waves per CU. Beside workgroup tasks they keep one
// buffer at 3 waves/SIMD (166 VGPRs): three of them, or any mix with the
// 3-wave workgroup kernel's 168, fill a SIMD's 512 registers, where a
// 253-register double-buffered wave left a third of them idle (measured on
// MI355X: shared-prompt cascade 0.116 against 0.124 ms, mixed batch 0.733
// against 0.752-0.765 ms). 32-row (verify) tasks keep one buffer at 2
// waves/SIMD (213 VGPRs; their two-buffer variant measured the same); 64-row
// tasks double-buffer and need the whole register file.
template <int NT, bool CONC>
struct WavesPerEu {
  static constexpr int value = NT == 1 ? (CONC ? 3 : 2) : (NT == 2 ? 2 : 1);
};
template <int NT, bool CONC>
struct Depth {
  static constexpr int value = NT == 1 ? (CONC ? 1 : 2) : (NT == 2 ? 1 : 2);
};

// One task on one wave. q_row: null, or the table naming each of the task's
// rows' query row (virtual rows of cascade tasks).
template <int D, int NT, bool TREE, bool CONC, bool STREAM, int NB = 2>
__device__ __forceinline__ void run_task(const AttnArgs& a, const pmattn_work_item& it, const int32_t* q_row,
                                         int lane) {
  static_assert(NB == 2 || Depth<NT, CONC>::value == 1, "16-key chunks run one buffer deep");
  constexpr int KS = D / 32, DT = D / 16;
  const int i = lane & 15, g = lane >> 4;
  const int G = a.group, hq = a.hq, hkv = a.hkv, kvh = it.kv_head;
  const int M = it.n_tok * G;
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* __restrict__ vpool = static_cast<const uint16_t*>(a.v_pool);

  // Q operand (B of the QK product): lane (i, g) holds query row 16n+i; k-step
  // s takes channels [32s + 8g, 32s + 8g + 8), the channel group K's lanes
  // hold for the same step.
  bf16x8 qop[NT][KS];
  int pos[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int m = 16 * n + i;
    pos[n] = -1;
    if (m < M) {
      const int t = m / G;
      pos[n] = it.pos_begin + t;
      const int64_t qr = q_row ? q_row[it.row_begin + t] : it.row_begin + t;
      const uint16_t* src = qp + (qr * hq + kvh * G + (m - t * G)) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < KS; ++s) qop[n][s] = ld16(src + 32 * s);
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

  // Physical block ids, fetched with scalar loads one chunk ahead of use.
  const cint_p bt_row = (cint_p)(a.block_table + (int64_t)it.seq * a.bt_stride);
  const int last_blk = ((it.kv_end + 15) >> 4) - 1;
  auto chunk_ids = [&](int c, int& b0, int& b1) {
    const int bi = c >> 4;
    b0 = bt_row[min(bi, last_blk)];
    b1 = NB == 2 ? bt_row[min(bi + 1, last_blk)] : b0;
  };

  const float sl2 = a.scale_log2;
  const int kv_end = it.kv_end;
  // per row: keys below min(pos + 1, kv_end) are visible; lanes of group g see
  // keys c0 + 4g + slot_off(j), so fold 4g in once
  int lim_base[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) lim_base[n] = min(pos[n] + 1, kv_end) - 4 * g;
  TreeRows<NT> tr;
  if constexpr (TREE) {
    tr.tree_from = it.pos_begin - 95;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int m = 16 * n + i;
      tr.rel[n] = m < M ? a.row_mask[it.row_begin + m / G] : ~0ull;
      tr.dbase[n] = pos[n] - 4 * g;
    }
  }
  if constexpr (Depth<NT, CONC>::value == 1) {
    // One buffer per wave; latency is hidden by the other waves on the SIMD.
    constexpr int CK = 16 * NB;  // keys per chunk
    const int nch = (kv_end - it.kv_begin + CK - 1) / CK;
    Chunk<D, NB> A;
    int c0 = it.kv_begin, b0, b1;
    chunk_ids(c0, b0, b1);
    for (int k = 0; k < nch; ++k) {
      load_chunk<D, STREAM>(A, kpool, vpool, b0, b1, kvh, hkv, i, g);
      chunk_ids(c0 + CK, b0, b1);
      zero_tail_v<D>(A, c0, kv_end, g);
      wave_chunk<D, NT, TREE>(A, qop, o, m_run, l_run, lim_base, c0, sl2, g, tr);
      c0 += CK;
    }
  } else {
    // Software pipeline over pairs of 32-key chunks with two register buffers:
    // while one buffer is consumed the other one's loads are in flight. The
    // body has no data-dependent branch. An odd chunk count leaves one
    // trailing compute on a chunk past kv_end: every score there is masked and
    // every V lane zeroed, so it adds exactly nothing. Loads past the last
    // chunk re-read the last chunk's blocks (cache hits), never memory
    // outside them.
    const int nch = (kv_end - it.kv_begin + 31) >> 5;
    const int npairs = (nch + 1) >> 1;
    Chunk<D> A, B;
    int c0 = it.kv_begin, b0, b1;
    chunk_ids(c0, b0, b1);
    load_chunk<D, STREAM>(A, kpool, vpool, b0, b1, kvh, hkv, i, g);
    chunk_ids(c0 + 32, b0, b1);
    load_chunk<D, STREAM>(B, kpool, vpool, b0, b1, kvh, hkv, i, g);
    // issue_barrier() pins each chunk's loads to the point where they are
    // issued (a compiler memory barrier plus a scheduling barrier), so that the
    // optimizer can neither sink them next to their first use nor hoist the
    // other buffer's math above them (either would undo the prefetch).
    issue_barrier();
    for (int k = 0; k < npairs; ++k) {
      chunk_ids(c0 + 64, b0, b1);
      zero_tail_v<D>(A, c0, kv_end, g);
      wave_chunk<D, NT, TREE>(A, qop, o, m_run, l_run, lim_base, c0, sl2, g, tr);
      load_chunk<D, STREAM>(A, kpool, vpool, b0, b1, kvh, hkv, i, g);
      issue_barrier();
      chunk_ids(c0 + 96, b0, b1);
      zero_tail_v<D>(B, c0 + 32, kv_end, g);
      wave_chunk<D, NT, TREE>(B, qop, o, m_run, l_run, lim_base, c0 + 32, sl2, g, tr);
      load_chunk<D, STREAM>(B, kpool, vpool, b0, b1, kvh, hkv, i, g);
      issue_barrier();
      c0 += 64;
    }
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
}  // namespace pmattn
