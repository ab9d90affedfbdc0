// Workgroup tile task: one workgroup of 4 waves runs one task of up to 128
// query rows. Used by the workgroup kernel (attn_prefill.hip) and by the
// mixed-batch kernel (attn_mixed.hip).
//
// A task here is up to 128 query rows of one sequence and one kv head (128/G
// tokens x the G query heads of the group) against one KV partition: the
// matmul-softmax-matmul tile of the XY-Serve meta-kernel (XY-Serve pith
// review, "What carries the argument"), laid out for CDNA4:
//
// * 4 waves x 32 rows. All four share the kv head, so each 32-key chunk of
//   K and V is gathered through the block table once per workgroup into LDS
//   and read by every wave from there: the K/V concatenation the XY-Serve
//   referee report blames for the baseline's prefix-reuse losses never
//   happens. The gather is a three-stage ring of LDS-destination buffer
//   loads: chunk c + 2 is in flight while chunk c is computed, one barrier per
//   chunk, and no register or LDS-store instruction carries the data.
// * S^T = K . Q^T and O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16. Each lane
//   owns one query row (l % 32) and 16 keys of every 32-key score tile. The
//   keys are permuted inside a tile (bits 2 and 3 of the slot swapped) so that
//   the P operand of the PV product is read straight from the S accumulator
//   registers and every V operand is one 16-byte LDS read of 8 consecutive
//   keys of one channel (V blocks are channel-major).
// * Online softmax in fp32 with exp2 (scale*log2e folded in). The O rescale
//   is lazy: a row's reference max moves only when the row's max passes it by
//   more than 2^8 (one compare against a per-row threshold per tile), which
//   after the first chunks almost never happens; P stays below 2^8 and the
//   final O/l is exact either way (online softmax equals softmax:
//   "Assumptions & free parameters"). The half-row max is one
//   v_permlane32_swap, the 16-score max eight v_maximum3.
// * Row-wise causal masks ("Editorial extensions"): chunks wholly visible to
//   every row of the task take an unmasked path (Figure 11, mask-aware
//   computation); V slots of keys past the task's end are zeroed in LDS once
//   that chunk has landed, so pool slots no row can see may hold NaN.
// * Occupancy is a template parameter: three waves per SIMD (168 VGPRs, 48
//   KiB of LDS per workgroup), so that LDS latency and one wave's softmax
//   VALU hide behind the other waves' MFMA. Beside one-wave tasks of the
//   same plan the kernel keeps three, and those tasks are built to fit the
//   same register share. Measured: few-shot prefill 907 vs 813 TFLOP/s (3 vs
//   2). Token trees run at three as well: with the LDS ring their mask code
//   fits 168 registers but for one value parked in scratch across the chunk
//   loop (one store before it, one load after), and run as fast as at two
//   waves with the same plan and 3.5% faster with more, shorter tasks (with
//   register staging, before the ring, their masks spilled inside the loop
//   and two waves were 19% faster). 64-key
//   chunks at 2 waves were 3% slower than 32-key ones.
// * Staging measured on MI355X (one session, few-shot prefill): the earlier
//   register staging (global -> registers -> LDS, one chunk ahead) took 20%
//   of the kernel's time (1.156 ms against 0.937 ms in a timing copy that
//   skipped it; 1.022 ms skipping only its global loads). The LDS ring made
//   the kernel 1.037 ms and the mixed batch 0.571 ms instead of 0.593-0.613.
#pragma once

#include <type_traits>

#include "task_common.h"

namespace pmattn {
namespace {

// lazy rescale threshold, in log2 units of the scaled scores
constexpr float kRescaleLog2 = 8.0f;
// LDS operand read-ahead of the QK (K) and PV (V) MFMA runs. Measured on
// MI355X, few-shot prefill: 962-965 TFLOP/s with the compiler's one-deep
// schedule, 982 with V two deep, 1,001-1,009 with K four deep as well (3
// waves/SIMD, no spills); V four deep spilled (851-861).
constexpr int kKAhead = 4;
constexpr int kVAhead = 2;


template <int D>
struct Cfg {
  static constexpr int CHUNK = 32;            // keys per iteration (two blocks)
  static constexpr int NBLK = CHUNK / 16;
  static constexpr int KSTEPS = D / 16;       // QK k-steps of 16 channels
  static constexpr int DT = D / 32;           // 32-channel output tiles
  static constexpr int BLK = 16 * D;          // elements of one (block, kv head) slice
  static constexpr int K_ELEMS = NBLK * BLK;  // K of one chunk; V follows
  static constexpr int STAGE = 2 * K_ELEMS;
  static constexpr int NSTAGE = 3;            // chunks c, c + 1 and c + 2 in flight
  static constexpr int LDS_ELEMS = NSTAGE * STAGE;
  static constexpr int PB = 2 * BLK / 1024;   // 1 KiB pieces per slice
  static constexpr int LOADS = NBLK * PB / 4; // 1 KiB loads of K (and of V) per wave and chunk
  static constexpr int VMEM_PER_CHUNK = 2 * LOADS;
};

// Buffer resource over one (block, kv head) slice of a pool: 16 tokens x D
// channels of bf16; reads past its end return 0.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* slice) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(slice), (short)0, 32 * D, 0x00020000);
}

// One wave load of 16 bytes per lane from a buffer into LDS: lane i's bytes
// land at dst + 16 i (dst wave-uniform).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint16_t* dst, uint32_t voff) {
  typedef __attribute__((address_space(3))) void* lds_t;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t)dst, 16, voff, 0, 0, 0);
}

// Issues the loads of one chunk (two blocks of K and of V) straight into an
// LDS stage (buffer loads with the LDS flag: no registers, no LDS stores).
// A wave load moves 1 KiB of one slice and writes it to 1 KiB of LDS in lane
// order, so the stage keeps the pool's block layouts: K grouped
// [D/8][16][8] (the QK operand of 16 consecutive keys is 256 contiguous
// bytes: no bank conflicts), V channel-major [D][16] with the two 16-byte
// halves of a channel's 32 bytes swapped on odd groups of eight channels
// (the lane filling LDS slot L reads global slot L ^ ((L >> 4) & 1)), so
// that the PV operand reads of 16 channels fall on distinct banks.
template <int D>
__device__ __forceinline__ void stage_issue(uint16_t* stage, const uint16_t* __restrict__ kpool,
                                            const uint16_t* __restrict__ vpool, const int (&blk)[Cfg<D>::NBLK],
                                            int kvh, int hkv, int wave, int lane) {
  constexpr int PB = Cfg<D>::PB, BLK = Cfg<D>::BLK;
  static_assert(Cfg<D>::NBLK == 2 && PB * 2 % 4 == 0, "whole wave loads per chunk");
#pragma unroll
  for (int u = 0; u < Cfg<D>::LOADS; ++u) {
    const int gp = wave + 4 * u;  // wave-uniform
    const int b = gp / PB, p = gp % PB;
    const int64_t base = ((int64_t)(b ? blk[1] : blk[0]) * hkv + kvh) * 16 * D;
    const uint32_t koff = 1024u * p + 16u * lane;
    const uint32_t voff = 1024u * p + 16u * (lane ^ ((lane >> 4) & 1));
    lds_load16(block_rsrc<D>(kpool + base), stage + b * BLK + 512 * p, koff);
    lds_load16(block_rsrc<D>(vpool + base), stage + Cfg<D>::K_ELEMS + b * BLK + 512 * p, voff);
  }
}

// Waits until at most N of this wave's vector memory operations are in
// flight (vmcnt; expcnt and lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses in the compiler but, unlike
// __syncthreads, does not wait for the LDS loads still in flight.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keeps the enclosing uniform branch a real branch: the compiler may not
// if-convert (speculate) a block containing it, so the rarely needed masking
// code runs only when its condition holds.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// In the chunk that holds the task's end, zeroes the V slots of keys >=
// kv_end in the landed stage (chunks past the last block re-read the last
// block; their keys are >= kv_end as well), so that pool slots no row can
// see may hold NaN: their weights are 0, and 0 * NaN would still be NaN.
template <int D>
__device__ __forceinline__ void zero_tail_v(uint16_t* stage, int c0, int kv_end, int tid) {
  constexpr int SLOTS = 2 * Cfg<D>::BLK / 8, PER_BLK = Cfg<D>::BLK / 8;
  uint16_t* vl = stage + Cfg<D>::K_ELEMS;
#pragma unroll
  for (int s0 = 0; s0 < SLOTS; s0 += 256) {
    const int sl = s0 + tid;
    const int b = sl / PER_BLK, ws = sl % PER_BLK, ch = ws >> 1;
    const int half = (ws & 1) ^ ((ch >> 3) & 1);
    const int nv = kv_end - (c0 + 16 * b + 8 * half);  // keys of this slot below kv_end
    if (nv < 8) {
      u32x4 v = *reinterpret_cast<const u32x4*>(vl + 8 * sl);
      v.x &= (0 < nv ? 0xFFFFu : 0u) | (1 < nv ? 0xFFFF0000u : 0u);
      v.y &= (2 < nv ? 0xFFFFu : 0u) | (3 < nv ? 0xFFFF0000u : 0u);
      v.z &= (4 < nv ? 0xFFFFu : 0u) | (5 < nv ? 0xFFFF0000u : 0u);
      v.w &= (6 < nv ? 0xFFFFu : 0u) | (7 < nv ? 0xFFFF0000u : 0u);
      *reinterpret_cast<u32x4*>(vl + 8 * sl) = v;
    }
  }
}

// Key offset (within a 64-key chunk) of score register r of tile kt held by
// lane half h: slot 8*(r/4) + 4h + r%4 of the 32x32 accumulator, with slot
// bits 2 and 3 swapped.
__device__ __forceinline__ int key_off(int kt, int r, int h) {
  return 32 * kt + 16 * (r >> 3) + 8 * h + 4 * ((r >> 2) & 1) + (r & 3);
}

// max without the sNaN quieting that fmaxf needs (scores are never
// signalling NaNs)
__device__ __forceinline__ float fmax_nq(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// max over lanes l and l ^ 32 (the two halves of a query row's keys)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nq(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Softmax state of a lane's row: the reference ref2 (in scaled log2 units)
// subtracted before exp2, and the raw score above which the reference must
// move (about ref2 / sl2 + kRescaleLog2 / sl2; -inf while the row has seen
// no visible key, when ref2 is 0).
struct RowRef {
  float ref2;
  float thr;
};

// One 32-key score tile: S^T = K.Q^T, mask, online softmax with lazy
// rescale, then O^T += V^T.P^T.
template <int D, bool TREE>
__device__ __forceinline__ void compute_tile(const uint16_t* lds, int kt, const bf16x8 (&qop)[D / 16],
                                             f32x16 (&o)[D / 32], RowRef& rr, float& l_part,
                                             bool mask, int lim, float sl2, int i32, int h,
                                             uint64_t rel, int dpos) {
  constexpr int KSTEPS = D / 16, DT = D / 32;
  constexpr int BLK = Cfg<D>::BLK;
  const uint16_t* kl = lds;
  const uint16_t* vl = lds + Cfg<D>::K_ELEMS;
  // A-operand row i32 holds key kappa(i32): slot bits 2 and 3 swapped. Its
  // channels (D/2)h + 8st .. + 7 are channel group (D/16)h + st of the key's
  // grouped K block: 16 bytes at group * 256 + token * 16.
  const int kap = (i32 & ~12) | ((i32 & 4) << 1) | ((i32 & 8) >> 1);
  f32x16 s = {};
  const uint16_t* kr = kl + (kap >> 4) * BLK + (kap & 15) * 8 + (D / 16) * h * 128;
  // K operands rotate through kKAhead registers, each read that many MFMAs
  // before its use; the scheduling barriers pin the order (left alone, the
  // scheduler sinks every read next to its MFMA and waits out the LDS
  // latency each time)
  bf16x8 kq[kKAhead];
#pragma unroll
  for (int st = 0; st < kKAhead && st < KSTEPS; ++st) kq[st] = ld16(kr + 128 * st);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[st % kKAhead], qop[st], s, 0, 0, 0);
    if (st + kKAhead < KSTEPS) kq[st % kKAhead] = ld16(kr + 128 * (st + kKAhead));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (mask) {
    // visible iff key < lim (lim = min(pos + 1, kv_end) - c0 for this lane's row)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = key_off(kt, r, h) < lim ? s[r] : kNegInf;
    if constexpr (TREE) {
      // token tree: bit k of rel = the key k positions before the row's own
      // position is visible (dpos = that position - c0)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dd = dpos - key_off(kt, r, h);
        s[r] = ((unsigned)dd < 64u && !((rel >> dd) & 1ull)) ? kNegInf : s[r];
      }
    }
  }
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmax_nq(mx, s[r]);
  mx = max_halves(mx);
  // the reference moves only for rows whose max passed the threshold (a row
  // with no visible key so far has threshold -inf: its first one moves it)
  const bool grow = mx > rr.thr;
  if (__any(grow)) {
    const float r2 = mx * sl2;
    const float alpha = !grow ? 1.f : rr.thr == kNegInf ? 0.f : __builtin_amdgcn_exp2f(rr.ref2 - r2);
    l_part *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] *= alpha;
    if (grow) {
      rr.ref2 = r2;
      rr.thr = mx + kRescaleLog2 * __builtin_amdgcn_rcpf(sl2);
    }
  }
  const float ms = rr.ref2;
  f32x8 p0, p1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p0[e] = __builtin_amdgcn_exp2f(s[e] * sl2 - ms);
    p1[e] = __builtin_amdgcn_exp2f(s[8 + e] * sl2 - ms);
  }
  float ps = p0[0] + p1[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) ps += p0[e] + p1[e];
  l_part += ps;
  const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
  const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
  // V operands likewise, kVAhead deep: operand j is keys 16 (j % 2) + 8h ..
  // + 7 (block j % 2, tokens 8h ..) of channel 32 (j / 2) + i32, the 16-byte
  // half h of the channel's 32 bytes, stored swapped on odd groups of eight
  // channels; read kVAhead MFMAs before its use
  const uint16_t* vb = vl + i32 * 16 + 8 * (h ^ ((i32 >> 3) & 1));
  constexpr int NV = 2 * DT;
  auto vaddr = [&](int j) { return vb + (j & 1) * BLK + (j >> 1) * 512; };
  bf16x8 vq[kVAhead];
#pragma unroll
  for (int j = 0; j < kVAhead && j < NV; ++j) vq[j] = ld16(vaddr(j));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    o[j >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[j % kVAhead], (j & 1) ? pb1 : pb0, o[j >> 1], 0, 0, 0);
    if (j + kVAhead < NV) vq[j % kVAhead] = ld16(vaddr(j + kVAhead));
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool TREE>
__device__ __forceinline__ void wg_chunk(const uint16_t* lds, const bf16x8 (&qop)[D / 16],
                                              f32x16 (&o)[D / 32], RowRef& rr, float& l_part,
                                              bool mask, int lim, float sl2, int i32, int h,
                                              uint64_t rel, int dpos) {
  compute_tile<D, TREE>(lds, 0, qop, o, rr, l_part, mask, lim, sl2, i32, h, rel, dpos);
}

// One task on the calling workgroup (all 256 threads call it, with the same
// item). lds: Cfg<D>::LDS_ELEMS elements of LDS, 16-byte aligned. q_row: null,
// or the table naming each task row's query row (virtual rows of cascade
// tasks). Waves may still read the LDS when they return: a caller reusing it
// must meet at a barrier first.
template <int D, bool TREE>
__device__ __forceinline__ void wg_task(const AttnArgs& a, const pmattn_work_item& it, const int32_t* q_row,
                                        uint16_t* lds) {
  constexpr int KSTEPS = D / 16, DT = D / 32, CHUNK = Cfg<D>::CHUNK;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63;
  const int i32 = lane & 31, h = lane >> 5;
  const int G = a.group, hq = a.hq, hkv = a.hkv, kvh = it.kv_head;
  const int M = it.n_tok * G;
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* __restrict__ vpool = static_cast<const uint16_t*>(a.v_pool);

  // this lane's query row and its Q operand (B of QK): channels (D/2)h + 8s
  const int m = 32 * wave + i32;
  const bool row_valid = m < M;
  // a wave holding none of the task's rows only helps stage K/V (tasks of
  // fewer than 128 rows: verify drafts, the last run of a prefill chunk)
  const bool wave_rows = 32 * wave < M;
  const int t = row_valid ? m / G : 0;
  const int pos = row_valid ? it.pos_begin + t : -1;
  bf16x8 qop[KSTEPS];
  if (row_valid) {
    const int64_t qr = q_row ? q_row[it.row_begin + t] : it.row_begin + t;
    const uint16_t* src = qp + (qr * hq + kvh * G + (m - t * G)) * D + (D / 2) * h;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qop[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + 8 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qop[s] = (bf16x8)(__bf16)0.0f;
  }
  f32x16 o[DT];
#pragma unroll
  for (int tt = 0; tt < DT; ++tt) o[tt] = (f32x16){};
  RowRef rr = {0.f, kNegInf};
  float l_part = 0.f;

  const cint_p bt_row = (cint_p)(a.block_table + (int64_t)it.seq * a.bt_stride);
  const int kv_end = it.kv_end;
  const int last_blk = ((kv_end + 15) >> 4) - 1;
  const int nch = (kv_end - it.kv_begin + CHUNK - 1) / CHUNK;
  const int min_pos = it.pos_begin;  // first token of the task
  const int row_lim = min(pos + 1, kv_end);
  uint64_t rel = ~0ull;
  if constexpr (TREE)
    if (row_valid) rel = a.row_mask[it.row_begin + t];
  const float sl2 = a.scale_log2;

  // physical ids of the chunk's blocks; blocks past the last one repeat it
  constexpr int NBLK = Cfg<D>::NBLK;
  auto chunk_blocks = [&](int c0, int (&blk)[NBLK]) {
    const int bi = c0 >> 4;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) blk[b] = bt_row[min(bi + b, last_blk)];
  };

  // Chunk c lands in LDS stage c % 3. Step c waits for its own loads (chunk
  // c + 1's may still be in flight), meets the other waves at a barrier
  // (chunk c is then complete, and every wave is done with chunk c - 1), and
  // issues chunk c + 2 into the stage chunk c - 1 left before computing.
  constexpr int STAGE = Cfg<D>::STAGE;
  int blk[NBLK];
  int c0 = it.kv_begin;
  if (nch > 0) {
    chunk_blocks(c0, blk);
    stage_issue<D>(lds, kpool, vpool, blk, kvh, hkv, wave, lane);
  }
  if (nch > 1) {
    chunk_blocks(c0 + CHUNK, blk);
    stage_issue<D>(lds + STAGE, kpool, vpool, blk, kvh, hkv, wave, lane);
  }
  // the loop runs the three stages in turn, so every LDS address takes its
  // stage as an immediate offset
  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    if (c + 1 < nch) vm_wait<Cfg<D>::VMEM_PER_CHUNK>();
    else vm_wait<0>();
    stage_barrier();
    if (c + 2 < nch) {
      chunk_blocks(c0 + 2 * CHUNK, blk);
      stage_issue<D>(lds + ((B + 2) % 3) * STAGE, kpool, vpool, blk, kvh, hkv, wave, lane);
    }
    issue_barrier();
    if (c0 + CHUNK > kv_end) {
      keep_branch();
      zero_tail_v<D>(lds + B * STAGE, c0, kv_end, tid);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the zeroes are written
      stage_barrier();
    }
    // a chunk every row of the task sees whole needs no mask; in a token tree
    // that excludes the 64 keys before the task's first row
    const bool mask = c0 + CHUNK - 1 > min_pos - (TREE ? 64 : 0) || c0 + CHUNK > kv_end;
    if (wave_rows)
      wg_chunk<D, TREE>(lds + B * STAGE, qop, o, rr, l_part, mask, row_lim - c0, sl2, i32, h, rel, pos - c0);
    c0 += CHUNK;
  };
  for (int c = 0; c < nch; c += 3) {
    step(std::integral_constant<int, 0>{}, c);
    if (c + 1 < nch) step(std::integral_constant<int, 1>{}, c + 1);
    if (c + 2 < nch) step(std::integral_constant<int, 2>{}, c + 2);
  }

  // epilogue: lane (i32, h) owns channels 32t + 8q + 4h + (0..3) of its row
  const float l = l_part + __shfl_xor(l_part, 32);
  if (!row_valid) return;
  const int64_t row = it.row_begin + t;
  const int qh = kvh * G + (m - t * G);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? (rr.ref2 + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
  if (it.part < 0) {
    uint16_t* dst = static_cast<uint16_t*>(a.out) + (row * hq + qh) * D + 4 * h;
#pragma unroll
    for (int tt = 0; tt < DT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[tt][4 * q] * inv, o[tt][4 * q + 1] * inv, o[tt][4 * q + 2] * inv, o[tt][4 * q + 3] * inv};
        *reinterpret_cast<uint2*>(dst + 32 * tt + 8 * q) = __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
      }
    if (a.lse && h == 0) a.lse[row * hq + qh] = lse;
  } else {
    const int64_t rec = (int64_t)it.part + m;
    float* dst = a.part_o + rec * D + 4 * h;
#pragma unroll
    for (int tt = 0; tt < DT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[tt][4 * q] * inv, o[tt][4 * q + 1] * inv, o[tt][4 * q + 2] * inv, o[tt][4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(dst + 32 * tt + 8 * q) = v;
      }
    if (h == 0) a.part_lse[rec] = lse;
  }
}

}  // namespace
}  // namespace pmattn
