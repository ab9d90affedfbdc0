// Host planner: validates a batch and turns it into a list of tile tasks.
//
// This is the Token-Table / Task-Table step of the XY-Serve design (XY-Serve
// pith review, "Core claim": each stage's attention work is decomposed into
// tile-level tasks recorded in tables; "What carries the argument": tiles are
// ordered by computational area at run time). Here a task is
// (sequence, kv head, a run of query tokens, a KV partition). The query heads
// of one GQA group ride together in the MFMA column dimension, so a task holds
// tokens x (Hq/Hkv) query rows. KV partitions are the split-KV of
// Flash-Decoding (reference list of the same page); partial results are
// merged by log-sum-exp afterwards.
//
// Pure host code: no HIP call, so every rule here is testable on a CPU.
//
// The planner runs once per batch on the host, so it is written to stay in
// the tens of microseconds for batches of ten thousand tasks: every ordering
// is a counting sort over small integer keys, the block table is walked once
// per row, the tables are written straight into the upload image, and the
// working buffers belong to the calling thread and are reused by its next
// plan (for the per-block marks, 16 bytes per pool block).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <new>
#include <numeric>

#include "plan_internal.h"

namespace pmattn {

namespace {
thread_local std::string g_last_error;
std::atomic<uint64_t> g_next_plan_id{1};

// Cost model for ordering and automatic splitting, in "block units": a task
// over n KV blocks costs n * (2 + rows/16). The constant 2 stands for the
// K/V stream of each block, the rows/16 term for its MFMA column tiles.
int64_t unit_cost(int cls) { return 2 + kClassRows[cls] / 16; }
// Automatic splitting aims at this many wave tasks per compute unit, and at
// 1.5 workgroup tasks per compute unit: fewer, longer workgroup tasks write
// fewer partials, more of them shorten the tail. Measured on MI355X, step
// time at 1 / 1.5 / 2 per CU: shared-prompt cascade (one kernel for its
// virtual tiles and member decode tasks) 0.0983 / 0.0935 / 0.0959 ms, mixed
// chunk batch 0.600 / 0.600 / 0.600 ms.
constexpr int64_t kTasksPerCu = 32;
constexpr int64_t kWgTasksPer2Cu = 3;
// Token trees (no one-wave tasks beside them, and more rows visible per key
// than a prefill tile's diagonal) take 2 per CU: measured on MI355X, token-tree
// verify at 3 waves per SIMD, step ms at 1.5 / 2 / 3 per CU: 0.1497-0.1563 / 0.1489-0.1516 /
// 0.1622-0.1633 (three sessions; the tasks pass 0.1358-0.1386 ms at 2 against
// 0.1418-0.1466 at 1.5, the merge 3 us longer).
constexpr int64_t kWgTasksPer2CuTree = 4;
// Equal-work decode: a plan whose tasks are all 16-row wave tasks (decode
// rows) with automatic splits gives each of kStreamWavesPerCu waves per CU an
// equal run of KV blocks of one kv head, never shorter than kStreamMinBlocks.
// (Measured on MI355X, 64-sequence decode, % of HBM peak: 2 waves per CU 61,
// 3: 69.4, 4: 68.6, 6: 62, 8: 66.8; 3 and 4 tie on other context mixes.)
// Plans with other tasks beside the decode ones keep one task per wave: there
// the decode waves share the chip with workgroup tasks, and fewer, longer
// decode waves were slower (mixed batch: 1, 2, 3 waves per CU gave 1.32,
// 0.92, 0.79 ms against 0.78; shared-prompt cascade 0.173, 0.130, 0.127
// against 0.125 ms).
constexpr int64_t kStreamWavesPerCu = 3;
// The same plan serves a batch whose tasks are all 17..32-row wave tasks
// (verify drafts), with kStreamWavesPerCu32 waves per CU (measured on
// MI355X, the 32 verify drafts of the mixed-chunk batch alone, % of HBM
// peak over the step: one task per wave 50.3; equal work at 3 waves per CU
// 59.5, 4: 61.7-61.9, 6: 53.7, 8: 58.3; double-buffered at one wave per
// SIMD 58.3).
constexpr int64_t kStreamWavesPerCu32 = 4;
constexpr int64_t kStreamMinBlocks = 16;
// ... but never cuts a task below this many block units.
constexpr int64_t kMinQuantum = 48;
constexpr int kMaxAutoSplits = 64;
// Mixed-batch kernel: each stream of the table is consumed in proportion to
// its own total of KV blocks (a bundle counts its longest task), so that the
// streams end together. The stream of 17..32-row wave bundles runs this much
// ahead (percent of its total): its smallest entries still last longer than
// the other streams' last ones (16-key chunks; measured on MI355X per table
// entry, mixed-chunk batch: about 3.9 us per block against 1.55 for 16-row
// tasks and 0.67 for prefill tiles).
constexpr int64_t kMixVerifyLead = 110;
// (Measured on MI355X, mixed-chunk batch, one session, three runs each: lead
// 100: 0.575 ms per step, 110: 0.568, 120: 0.569, 130: 0.571; leading the
// 16-row bundles as well, 104 or 108, or letting them lag, 96 or 92: slower.)
// Shader engines per XCD, which receive an XCD's workgroups in turn.
constexpr int kSeRoundRobin = 4;
// Automatic cascade: a shared run becomes a group only with this many members
// and this many blocks (measured on the pages' workloads).
constexpr int kCascadeAutoMembers = 8;
constexpr int kCascadeAutoBlocks = 64;
// ... and the automatic mode keeps its groups only when they spare at least
// 1/kCascadeAutoSaveDiv of the batch's logical keys (the repeated reads of the
// shared runs: (members - 1) x run length). Below that the caches serve the
// repeats, and the groups' extra tasks and merges cost more than they save:
// measured on MI355X, the 96 decode rows of the mixed batch (5% spared) took
// 0.363 ms with their two groups against 0.289 ms without; the shared-prompt
// decode batch spares 92%.
constexpr int64_t kCascadeAutoSaveDiv = 4;


int class_of_rows(int rows) {
  for (int c = 0; c < kNumClasses; ++c)
    if (rows <= kClassRows[c]) return c;
  return -1;
}

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Shuffles idx[0, n) in place (the work_shuffle_seed option).
template <typename T>
void shuffle(T* idx, size_t n, uint64_t& rng) {
  for (size_t i = n; i > 1; --i) std::swap(idx[i - 1], idx[splitmix64(rng) % i]);
}

// XCD of a task. K/V of (block, kv head) is read only by tasks of that kv
// head, so all tasks of one kv head go to one XCD (kv heads spread over
// several XCDs when there are fewer than kXcds, by sequence): every task that
// reads a shared block finds it in the same L2.
inline int xcd_of(int kv_head, int seq, int hkv) {
  const int rep = hkv >= kXcds ? 1 : (kXcds + hkv - 1) / hkv;  // XCDs per kv head
  return (hkv >= kXcds ? kv_head : kv_head * rep + seq % rep) % kXcds;
}

// Stable counting sort: out[0, n) = the indices 0..n-1 ordered by key
// ascending (keys in [0, nkeys)), equal keys in index order.
void counting_order(const uint32_t* key, uint32_t n, size_t nkeys, std::vector<uint32_t>& cnt, uint32_t* out) {
  cnt.assign(nkeys + 1, 0);
  for (uint32_t i = 0; i < n; ++i) ++cnt[key[i] + 1];
  for (size_t k = 0; k < nkeys; ++k) cnt[k + 1] += cnt[k];
  for (uint32_t i = 0; i < n; ++i) out[cnt[key[i]]++] = i;
}

// Deals the entries of kXcds queues (queue x: entries [beg[x], end[x]) of a
// common array) to workgroup slots: slot i, which the hardware gives to XCD
// i % kXcds, takes the next `per_wg` entries of that XCD's queue, topped up
// from the queue with the most entries left once that one runs out (so that
// every slot but the last holds exactly per_wg entries). emit(x, e) receives
// each entry's queue and its index in the common array, in dispatch order.
template <typename Emit>
void deal(const size_t* beg, const size_t* end, int per_wg, Emit&& emit) {
  size_t head[kXcds], total = 0, done = 0, least = std::numeric_limits<size_t>::max();
  for (int x = 0; x < kXcds; ++x) {
    head[x] = beg[x];
    total += end[x] - beg[x];
    least = std::min(least, end[x] - beg[x]);
  }
  // rounds in which every XCD still has a whole workgroup of tasks: slot s
  // takes per_wg tasks of XCD s % kXcds, no top-up (the general loop below
  // does the same, one slot at a time)
  const size_t rounds = least / (size_t)per_wg;
  for (size_t r = 0; r < rounds; ++r)
    for (int x = 0; x < kXcds; ++x)
      for (int k = 0; k < per_wg; ++k) emit(x, head[x]++);
  done = rounds * (size_t)per_wg * kXcds;
  for (size_t slot = rounds * kXcds; done < total; ++slot) {
    int x = (int)(slot % kXcds);
    for (size_t take = std::min<size_t>(per_wg, total - done); take > 0;) {
      if (head[x] == end[x]) {
        size_t best = 0;
        for (int y = 0; y < kXcds; ++y)
          if (end[y] - head[y] > best) best = end[y] - head[y], x = y;
      }
      const size_t m = std::min(take, end[x] - head[x]);
      for (size_t e = head[x]; e < head[x] + m; ++e) emit(x, e);
      head[x] += m;
      take -= m;
      done += m;
    }
  }
}

struct Tile {
  int32_t seq;  // unit: a real sequence (< B) or a virtual cascade sequence
  int32_t tok_begin, n_tok, cls;
  int32_t kv_end;  // one past the tile's last visible key
  int32_t range0;  // its first KV range (ranges [range0, range0 + k))
  int32_t k;       // its non-empty KV partitions
  int64_t rec0;    // its first partial record (kv head g: rec0 + g * k * rows), or -1
  int32_t row, row0, pos0;  // its block-table row, first query row (real or virtual), first position
};

// One KV partition of one tile, clipped to the tile's keys: the tasks of the
// tile's kv heads over these keys.
struct Range {
  int32_t tile, lo, hi;
  int32_t nblk;  // blocks' worth of keys, ceil((hi - lo) / 16)
  int32_t step;  // record offset between its kv heads' tasks (k * rows), if it has records
  int32_t row;   // its block-table row
  uint32_t seq;  // the sequence that sees its keys (kSeqMulti for a virtual tile)
};

// A task of a class before ordering: a range, a kv head and its XCD.
struct Cand {
  uint32_t range;
  uint16_t g, x;
};

// A task in its class's XCD queue: its item index and KV blocks.
struct QItem {
  int32_t item, nblk;
};

// Per pool block, valid while gen is the current plan's. state, bit 31
// clear: the block's one reader is range `state` (so its one reader tile is
// that range's tile, and the sequence that sees it is that tile's, unless
// the tile is virtual); bit 31 set: several tiles read it, and the low bits
// name the one sequence that sees it, or kSeqMulti.
constexpr uint32_t kMultiBit = 0x80000000u, kSeqMulti = 0x7FFFFFFFu;
struct Mark {
  uint32_t gen, state;
};

// A range's first block (start) or one past its last, along its table row.
struct Event {
  int32_t pos;
  uint32_t range;
  int32_t start;
  bool operator<(const Event& o) const { return pos != o.pos ? pos < o.pos : start < o.start; }
};

struct Target {
  int32_t blk, seq;
  uint32_t slots;  // bit o: slot o is written
};

struct VSeq {
  int32_t lo, hi, table_seq, row_begin, rows;
};

// A mixed-table stream entry: its weight (KV blocks; a bundle's longest task)
// and table code.
struct MixEntry {
  int64_t cost;
  int32_t e;
};

struct Listed {
  int64_t rec_base;
  int32_t parts, trows, row0, g;
  bool virt;
};

// Working buffers of one planning thread, reused by its next plan.
struct Scratch {
  std::vector<int32_t> row_off, own_lo, usplits, uoff, ubeg, uend, member_slot, vrow, cands;
  std::vector<int64_t> stream_start;
  std::vector<char> member, sunit;
  std::vector<VSeq> vseqs;
  std::vector<std::vector<int32_t>> members;
  std::vector<Tile> tiles;
  std::vector<Range> ranges;
  std::vector<Target> targets;
  std::vector<pmattn_append_unit> units;
  std::vector<uint64_t> row_mask, anc;
  std::vector<Listed> listed;
  std::vector<uint32_t> key, order, cnt, row_list, tile_first, tile_list;
  std::vector<Cand> cand, queue, outc;
  std::vector<pmattn_work_item> rtask;
  std::vector<QItem> qitem;
  std::vector<uint32_t> rlist;
  std::vector<char> rstream;
  std::vector<int32_t> rec_start, rec_fill, slot_first;
  std::vector<uint64_t> pairs;
  std::vector<int32_t> mix_cat;
  std::vector<QItem> mix_order, gtmp;
  std::vector<int32_t> group_of;
  std::vector<uint32_t> gkey, gorder;
  std::vector<MixEntry> mix_streams[4];
  std::vector<uint32_t> slot_key, slot_order;
  std::vector<int64_t> last_cost;
  std::vector<int32_t> unit_kind;
  std::vector<Event> events;
  std::vector<uint32_t> active, active_slot;
  std::vector<Mark> marks;
  std::vector<uint32_t> tstamp;  // per pool block: the last plan that appends to it
  uint32_t gen = 0;
};
thread_local Scratch g_scratch;
// The calling thread's buffers, as a plain pointer: taken once per plan, so
// that the compiler does not recompute the thread-local address at every use.
__attribute__((noinline)) Scratch* thread_scratch() { return &g_scratch; }

}  // namespace

pmattn_status fail(pmattn_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }

namespace {

// The exact copy-on-write check: two rows writing one pool slot, or a written
// slot that another sequence can see. Run only when the per-block marks of
// the plan's row walk cannot rule a conflict out (a block written by one
// sequence and seen, or also written, by another).
std::string exact_append_check(const pmattn_plan_desc* d, std::vector<Target>& targets) {
  std::sort(targets.begin(), targets.end(), [](const Target& a, const Target& b) { return a.blk < b.blk; });
  for (size_t i = 1; i < targets.size(); ++i)
    if (targets[i].blk == targets[i - 1].blk && (targets[i].slots & targets[i - 1].slots))
      return "two query rows write the same pool slot (block " + std::to_string(targets[i].blk) + ")";
  for (int s = 0; s < d->num_seqs && !targets.empty(); ++s) {
    if (d->q_len[s] == 0) continue;
    const int64_t kv = (int64_t)d->q_start[s] + d->q_len[s];
    const int32_t* bt = d->block_table + (int64_t)s * d->bt_stride;
    const int64_t nb = (kv + kBlock - 1) / kBlock;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t blk = bt[j];
      const uint32_t seen = j + 1 < nb ? 0xFFFFu : (1u << (kv - j * kBlock)) - 1u;
      auto it = std::lower_bound(targets.begin(), targets.end(), blk,
                                 [](const Target& a, int32_t b) { return a.blk < b; });
      for (; it != targets.end() && it->blk == blk; ++it)
        if (it->seq != s && (it->slots & seen))
          return "sequence " + std::to_string(s) + " can see pool slots that sequence " + std::to_string(it->seq) +
                 " appends to (block " + std::to_string(blk) + "): copy the block first";
    }
  }
  return std::string();
}

}  // namespace

static pmattn_status build_plan(const pmattn_plan_desc* d, Plan& P) {
  if (!d) return fail(PMATTN_E_INVALID, "desc is NULL");
  const int B = d->num_seqs;
  if (B < 0) return fail(PMATTN_E_INVALID, "num_seqs < 0");
  if (B > 0 && (!d->q_len || !d->seq_len || !d->q_start || !d->block_table))
    return fail(PMATTN_E_INVALID, "q_len, seq_len, q_start and block_table must be non-NULL");
  if (d->block_size != kBlock) return fail(PMATTN_E_UNSUPPORTED, "block_size must be 16");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PMATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->dtype != PMATTN_BF16 && d->dtype != PMATTN_F32)
    return fail(PMATTN_E_UNSUPPORTED, "dtype must be PMATTN_BF16 or PMATTN_F32");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(PMATTN_E_INVALID, "num_q_heads and num_kv_heads must be >= 1");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(PMATTN_E_INVALID, "num_q_heads must be a multiple of num_kv_heads");
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G > kMaxWaveRows) return fail(PMATTN_E_UNSUPPORTED, "num_q_heads / num_kv_heads must be <= 64");
  if (!std::isfinite(d->scale) || !(d->scale > 0.f))
    return fail(PMATTN_E_INVALID, "scale must be finite and > 0");
  if (d->num_kv_splits < 0 || d->num_kv_splits > kMaxSplits)
    return fail(PMATTN_E_INVALID, "num_kv_splits must be in 0..256");
  if (d->num_cus < 0) return fail(PMATTN_E_INVALID, "num_cus must be >= 0");
  if (d->cascade < 0 || d->cascade > 2) return fail(PMATTN_E_INVALID, "cascade must be 0, 1 or 2");
  if (d->num_pool_blocks < 0) return fail(PMATTN_E_INVALID, "num_pool_blocks < 0");
  if (B > 0 && d->bt_stride < 1) return fail(PMATTN_E_INVALID, "bt_stride must be >= 1");

  P.num_seqs = B;
  P.bt_stride = d->bt_stride;
  P.num_pool_blocks = d->num_pool_blocks;
  P.hq = d->num_q_heads;
  P.hkv = d->num_kv_heads;
  P.group = G;
  P.head_dim = d->head_dim;
  P.dtype = d->dtype;
  P.scale = d->scale;
  const int hkv = d->num_kv_heads;
  Scratch& S = *thread_scratch();
  auto bt_row = [&](int s) { return d->block_table + (int64_t)s * d->bt_stride; };

  // ---- validate sequences ---------------------------------------------------
  int64_t rows = 0;
  for (int s = 0; s < B; ++s) {
    const int64_t ql = d->q_len[s], sl = d->seq_len[s], qs = d->q_start[s];
    if (ql < 0 || sl < 0 || qs < 0)
      return fail(PMATTN_E_INVALID, "negative q_len/seq_len/q_start at sequence " + std::to_string(s));
    if (qs + ql > sl)
      return fail(PMATTN_E_INVALID, "q_start + q_len > seq_len at sequence " + std::to_string(s));
    if (ql == 0) continue;
    const int64_t need_blocks = (sl + kBlock - 1) / kBlock;
    if (need_blocks > d->bt_stride)
      return fail(PMATTN_E_INVALID, "bt_stride < ceil(seq_len/16) at sequence " + std::to_string(s));
    const int64_t vis_blocks = (qs + ql + kBlock - 1) / kBlock;
    const int32_t* row = bt_row(s);
    int32_t bad = 0;  // (a branch-free pass the compiler vectorizes)
    for (int64_t j = 0; j < vis_blocks; ++j) bad |= (row[j] < 0) | (row[j] >= d->num_pool_blocks);
    if (bad)
      for (int64_t j = 0; j < vis_blocks; ++j)
        if (row[j] < 0 || row[j] >= d->num_pool_blocks)
          return fail(PMATTN_E_INVALID, "block id out of [0, num_pool_blocks) at sequence " +
                                            std::to_string(s) + " block " + std::to_string(j));
    rows += ql;
  }
  if (rows > INT32_MAX / std::max(1, d->num_q_heads))
    return fail(PMATTN_E_INVALID, "too many query rows");
  P.num_rows = (int32_t)rows;
  std::vector<int32_t>& row_off = S.row_off;
  row_off.assign(B + 1, 0);
  for (int s = 0; s < B; ++s) row_off[s + 1] = row_off[s] + d->q_len[s];
  P.seq_row_off.assign(row_off.begin(), row_off.end());
  P.seq_q_start.assign(d->q_start, d->q_start + B);

  // ---- speculative token trees: per-row visibility of the 64 keys before it --
  // Bit k of a row's mask stands for the key k positions back. Ancestors (and
  // the row itself) set their bits; keys below q_start are context and always
  // visible, so every bit past the row's own index is set too. Chains (parent
  // r - 1) give all ones, the causal rule.
  bool tree = false;
  S.row_mask.clear();
  if (d->tree_parent && rows > 0) {
    for (int s = 0; s < B; ++s) {
      const int ql = d->q_len[s];
      const int32_t* par = d->tree_parent + row_off[s];
      bool chain = true;
      for (int r = 0; r < ql; ++r) {
        if (par[r] < -1 || par[r] >= r)
          return fail(PMATTN_E_INVALID, "tree_parent must lie in [-1, row) at sequence " +
                                            std::to_string(s) + " row " + std::to_string(r));
        chain = chain && par[r] == r - 1;
      }
      if (!chain && ql > kMaxTreeRows)
        return fail(PMATTN_E_UNSUPPORTED, "a token tree holds at most 64 rows (sequence " +
                                              std::to_string(s) + ")");
      tree = tree || !chain;
    }
    if (tree) {
      S.row_mask.assign(rows, ~0ull);
      std::vector<uint64_t>& anc = S.anc;  // bit a: row a of the sequence is an ancestor-or-self
      for (int s = 0; s < B; ++s) {
        const int ql = d->q_len[s];
        const int32_t* par = d->tree_parent + row_off[s];
        bool chain = true;
        for (int r = 0; r < ql; ++r) chain = chain && par[r] == r - 1;
        if (chain) continue;
        anc.assign(ql, 0);
        for (int r = 0; r < ql; ++r) {
          anc[r] = (par[r] < 0 ? 0ull : anc[par[r]]) | (1ull << r);
          uint64_t m = r < 63 ? ~0ull << (r + 1) : 0ull;
          for (int a = 0; a <= r; ++a)
            if (anc[r] >> a & 1ull) m |= 1ull << (r - a);
          S.row_mask[row_off[s] + r] = m;
        }
      }
    }
  }

  // ---- KV append units ------------------------------------------------------
  // A unit is the run of a sequence's new tokens that falls into one block.
  // Every slot written must be visible to its own sequence alone: checked
  // after the row walk below.
  S.units.clear();
  S.targets.clear();
  for (int s = 0; s < B; ++s) {
    const int ql = d->q_len[s], qs = d->q_start[s];
    const int32_t* bt = bt_row(s);
    for (int t = 0; t < ql;) {
      const int pos = qs + t, j = pos / kBlock, o = pos % kBlock;
      const int n = std::min(ql - t, kBlock - o);
      S.units.push_back(pmattn_append_unit{s, row_off[s] + t, n, j, o});
      S.targets.push_back(Target{bt[j], s, ((1u << n) - 1u) << o});
      t += n;
    }
  }

  // ---- cascade: shared prefix runs of decode/verify sequences -----------------
  // Sequences whose rows fit one wave task and whose leading physical blocks
  // coincide are grouped like a radix tree over block ids. Each run of blocks
  // shared by two or more of them, lying wholly before every member's first
  // query row, becomes a virtual sequence: its rows are all members' rows, its
  // keys the run. The members then attend only to the keys after their
  // deepest run, and the log-sum-exp merge joins the parts.
  std::vector<int32_t>& own_lo = S.own_lo;  // first key of each sequence's own range
  std::vector<char>& member = S.member;
  std::vector<VSeq>& vseqs = S.vseqs;
  std::vector<int32_t>& vrow = S.vrow;  // source row of each virtual row
  own_lo.assign(B, 0);
  member.assign(B, 0);
  vseqs.clear();
  vrow.clear();
  size_t nvm = 0;  // member lists in use (S.members[0, nvm))
  if (d->cascade) {
    auto bt = [&](int s, int j) { return d->block_table[(int64_t)s * d->bt_stride + j]; };
    auto shareable = [&](int s) { return d->q_start[s] / kBlock; };  // blocks before the first row
    std::vector<int32_t>& cands = S.cands;
    cands.clear();
    for (int s = 0; s < B; ++s)
      if (d->q_len[s] > 0 && (int64_t)d->q_len[s] * G <= kMaxWaveRows && shareable(s) >= 1) cands.push_back(s);
    // automatic mode: only runs that enough sequences share over enough
    // blocks become groups (measured: pairs, and runs of a few hundred
    // tokens, are already served by the caches and lose to the extra merge);
    // a run left out is folded into its descendants' ranges (cover_lo)
    const int min_members = d->cascade == 2 ? kCascadeAutoMembers : 2;
    const int min_blocks = d->cascade == 2 ? kCascadeAutoBlocks : 1;
    struct Node {
      std::vector<int32_t> mem;
      int32_t depth, cover_lo;
    };
    std::vector<Node> stack;
    if (cands.size() >= 2) stack.push_back(Node{cands, 0, 0});
    while (!stack.empty()) {
      Node node = std::move(stack.back());
      stack.pop_back();
      const int32_t depth = node.depth;
      // buckets: members by their block at `depth`, in ascending block id,
      // each bucket in node order
      std::vector<uint64_t>& pairs = S.pairs;
      pairs.clear();
      for (size_t i = 0; i < node.mem.size(); ++i)
        if (shareable(node.mem[i]) > depth) pairs.push_back((uint64_t)(uint32_t)bt(node.mem[i], depth) << 32 | i);
      std::sort(pairs.begin(), pairs.end());
      std::vector<Node> kids;
      for (size_t a = 0, e; a < pairs.size(); a = e) {
        for (e = a + 1; e < pairs.size() && pairs[e] >> 32 == pairs[a] >> 32;) ++e;
        if (e - a < 2) continue;
        std::vector<int32_t> bm(e - a);
        for (size_t i = a; i < e; ++i) bm[i - a] = node.mem[(uint32_t)pairs[i]];
        // the run all members share from here: up to the first block that
        // some member lacks or holds differently
        int32_t L = INT32_MAX;
        for (int32_t m : bm) L = std::min(L, shareable(m));
        const int32_t* first = bt_row(bm[0]);
        for (size_t i = 1; i < bm.size(); ++i) {
          const int32_t* row = bt_row(bm[i]);
          int32_t j = depth + 1;
          while (j < L && row[j] == first[j]) ++j;
          L = j;
        }
        int32_t cover = node.cover_lo;
        if ((int)bm.size() >= min_members && L - node.cover_lo >= min_blocks) {
          vseqs.push_back(VSeq{node.cover_lo * kBlock, L * kBlock, bm[0], 0, 0});
          if (S.members.size() <= nvm) S.members.resize(nvm + 1);
          S.members[nvm++] = bm;
          for (int32_t m : bm) {
            own_lo[m] = L * kBlock;
            member[m] = 1;
          }
          cover = L;
        }
        kids.push_back(Node{std::move(bm), L, cover});
      }
      for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(std::move(*it));
    }
    if (d->cascade == 2 && !vseqs.empty()) {
      int64_t spared = 0, logical = 0;
      for (size_t v = 0; v < vseqs.size(); ++v)
        spared += (int64_t)(S.members[v].size() - 1) * (vseqs[v].hi - vseqs[v].lo);
      for (int s = 0; s < B; ++s)
        if (d->q_len[s] > 0) logical += (int64_t)d->q_start[s] + d->q_len[s];
      if (spared * kCascadeAutoSaveDiv < logical) {
        vseqs.clear();
        nvm = 0;
        std::fill(own_lo.begin(), own_lo.end(), 0);
        std::fill(member.begin(), member.end(), 0);
      }
    }
    P.cascade_lo.clear();
    P.cascade_hi.clear();
    P.cascade_seq.clear();
    P.cascade_row_begin.clear();
    P.cascade_rows.clear();
    for (size_t v = 0; v < vseqs.size(); ++v) {
      vseqs[v].row_begin = (int32_t)vrow.size();
      for (int32_t m : S.members[v])
        for (int32_t r = 0; r < d->q_len[m]; ++r) vrow.push_back(row_off[m] + r);
      vseqs[v].rows = (int32_t)vrow.size() - vseqs[v].row_begin;
      P.cascade_lo.push_back(vseqs[v].lo);
      P.cascade_hi.push_back(vseqs[v].hi);
      P.cascade_seq.push_back(vseqs[v].table_seq);
      P.cascade_row_begin.push_back(vseqs[v].row_begin);
      P.cascade_rows.push_back(vseqs[v].rows);
    }
  }
  const int V = (int)vseqs.size();
  const int U = B + V;  // units: the real sequences, then the virtual ones
  auto unit_rows = [&](int u) { return u < B ? d->q_len[u] : vseqs[u - B].rows; };
  auto unit_lo = [&](int u) { return u < B ? own_lo[u] : vseqs[u - B].lo; };
  auto unit_hi = [&](int u) { return u < B ? d->q_start[u] + d->q_len[u] : vseqs[u - B].hi; };
  auto unit_row = [&](int u) { return u < B ? u : vseqs[u - B].table_seq; };  // its block-table row

  // ---- tiles: runs of query tokens whose G heads fit one task --------------
  // A unit whose rows fit one wave task (rows * G <= 64) is one tile; longer
  // ones are cut into runs of 128/G tokens for the workgroup kernel.
  const int tok_per_wg = std::max(1, kMaxTaskRows / G);
  std::vector<Tile>& tiles = S.tiles;
  tiles.clear();
  for (int u = 0; u < U; ++u) {
    const int ql = unit_rows(u);
    if (ql == 0) continue;
    auto kv_end = [&](int t0, int nt) { return u < B ? d->q_start[u] + t0 + nt : vseqs[u - B].hi; };
    if ((int64_t)ql * G <= kMaxWaveRows) {
      tiles.push_back(Tile{u, 0, ql, class_of_rows(ql * G), kv_end(0, ql), 0, 0, -1, 0, 0, 0});
      continue;
    }
    for (int t0 = 0; t0 < ql; t0 += tok_per_wg) {
      const int nt = std::min(tok_per_wg, ql - t0);
      tiles.push_back(Tile{u, t0, nt, kNumClasses - 1, kv_end(t0, nt), 0, 0, -1, 0, 0, 0});
    }
  }

  // ---- KV partitions per unit ------------------------------------------------
  std::vector<int32_t>& usplits = S.usplits;
  usplits.assign(U, 0);
  if (d->num_kv_splits > 0) {
    for (int u = 0; u < U; ++u) usplits[u] = unit_rows(u) > 0 ? d->num_kv_splits : 0;
  } else {
    // Two resource classes are balanced separately: wave tasks (<= 64 rows,
    // KV-stream bound) and workgroup tasks (128 rows, MFMA bound). A unit's
    // partition count is ceil(cost of its largest tile / quantum of its class).
    int64_t total[2] = {0, 0};
    std::vector<int64_t>& last_cost = S.last_cost;
    std::vector<int32_t>& unit_kind = S.unit_kind;
    last_cost.assign(U, 0);
    unit_kind.assign(U, 0);
    for (const Tile& t : tiles) {
      const int kind = kClassRows[t.cls] > kMaxWaveRows ? 1 : 0;
      const int64_t c = (int64_t)((t.kv_end - unit_lo(t.seq) + kBlock - 1) / kBlock) * unit_cost(t.cls);
      total[kind] += c * hkv;
      last_cost[t.seq] = std::max(last_cost[t.seq], c);
      unit_kind[t.seq] = kind;
    }
    const int64_t cus = d->num_cus > 0 ? d->num_cus : 256;
    const int64_t target[2] = {cus * kTasksPerCu, cus * (tree ? kWgTasksPer2CuTree : kWgTasksPer2Cu) / 2};
    int64_t quantum[2];
    for (int k = 0; k < 2; ++k)
      quantum[k] = std::max(kMinQuantum, (total[k] + target[k] - 1) / target[k]);
    for (int u = 0; u < U; ++u) {
      if (unit_rows(u) == 0) continue;
      const int64_t nblk = (unit_hi(u) - unit_lo(u) + kBlock - 1) / kBlock;
      const int64_t q = quantum[unit_kind[u]];
      int64_t p = (last_cost[u] + q - 1) / q;
      p = std::min<int64_t>(std::min<int64_t>(p, kMaxAutoSplits), nblk);
      usplits[u] = (int32_t)std::max<int64_t>(1, p);
    }
  }
  // Equal-work (stream) partitions when every unit is a real sequence whose
  // rows make one wave task of the same class, 16 rows (decode) or 32 rows
  // (verify). Laid end to end in unit order, unit u holds blocks
  // [S_u, S_u + n_u) of the concatenation; cut it into pieces of L blocks; a
  // unit's partitions are its parts of the pieces it meets, and piece j of kv
  // head g is the work of one wave.
  std::vector<char>& sunit = S.sunit;
  sunit.assign(U, 0);
  int stream_cls = -1;
  bool uniform = V == 0 && !tiles.empty();
  for (const Tile& t : tiles) {
    if (t.seq >= B || t.cls > 1 || (stream_cls >= 0 && t.cls != stream_cls)) uniform = false;
    if (stream_cls < 0) stream_cls = t.cls;
    sunit[t.seq] = 1;
  }
  const bool stream = d->dtype == PMATTN_BF16 && d->num_kv_splits == 0 && uniform;
  if (!stream) std::fill(sunit.begin(), sunit.end(), 0);
  std::vector<int64_t>& stream_start = S.stream_start;
  stream_start.assign(U, 0);
  int64_t stream_len = 0, stream_pieces = 0;
  if (stream) {
    int64_t total = 0;
    for (int u = 0; u < U; ++u) {
      stream_start[u] = total;
      if (sunit[u]) total += (unit_hi(u) - unit_lo(u) + kBlock - 1) / kBlock;
    }
    const int64_t cus = d->num_cus > 0 ? d->num_cus : 256;
    const int64_t per_head = std::max<int64_t>(1, cus * (stream_cls == 0 ? kStreamWavesPerCu : kStreamWavesPerCu32) / hkv);
    stream_len = std::max(kStreamMinBlocks, (total + per_head - 1) / per_head);
    stream_pieces = (total + stream_len - 1) / stream_len;
    for (int u = 0; u < U; ++u) {
      if (!sunit[u]) continue;
      const int64_t n = (unit_hi(u) - unit_lo(u) + kBlock - 1) / kBlock;
      usplits[u] = (int32_t)((stream_start[u] + n - 1) / stream_len - stream_start[u] / stream_len + 1);
    }
  }
  std::vector<int32_t>& uoff = S.uoff;
  std::vector<int32_t>& ubeg = S.ubeg;
  std::vector<int32_t>& uend = S.uend;
  uoff.assign(U + 1, 0);
  for (int u = 0; u < U; ++u) uoff[u + 1] = uoff[u] + usplits[u];
  ubeg.resize(uoff[U]);
  uend.resize(uoff[U]);
  for (int u = 0; u < U; ++u) {
    const int np = usplits[u];
    if (!np) continue;
    const int64_t lo = unit_lo(u), kv = unit_hi(u);
    if (stream && sunit[u]) {
      // partition p starts at the p-th piece boundary met (block offsets from
      // the unit's start)
      const int64_t s0 = stream_start[u], j0 = s0 / stream_len;
      for (int p = 0; p < np; ++p) {
        const int64_t b = p == 0 ? 0 : (j0 + p) * stream_len - s0;
        const int64_t e = (j0 + p + 1) * stream_len - s0;
        ubeg[uoff[u] + p] = (int32_t)std::min<int64_t>(lo + b * kBlock, kv);
        uend[uoff[u] + p] = (int32_t)std::min<int64_t>(lo + e * kBlock, kv);
      }
      continue;
    }
    const int64_t nblk = (kv - lo + kBlock - 1) / kBlock;
    const int64_t chunk = std::max<int64_t>(1, (nblk + np - 1) / np);
    for (int p = 0; p < np; ++p) {
      ubeg[uoff[u] + p] = (int32_t)std::min<int64_t>(lo + p * chunk * kBlock, kv);
      uend[uoff[u] + p] = (int32_t)std::min<int64_t>(lo + (p + 1) * chunk * kBlock, kv);
    }
  }
  P.num_splits.assign(usplits.begin(), usplits.begin() + B);
  P.split_offset.assign(uoff.begin(), uoff.begin() + B + 1);
  P.split_begin.assign(ubeg.begin(), ubeg.begin() + uoff[B]);
  P.split_end.assign(uend.begin(), uend.begin() + uoff[B]);
  P.cascade_splits.assign(usplits.begin() + B, usplits.end());

  // ---- KV ranges of the tiles, partial records and table sizes -------------
  // A tile's tasks are its kv heads times its non-empty partitions (clipped
  // to the tile's keys). Partial records are numbered tile by tile, kv head
  // by kv head: tile t, kv head g, its i-th partition, token row m write
  // record rec0 + (g * k + i) * rows + m. Rows of cascade members collect
  // their records from several tasks: their merge rows list record ids
  // (rec_stride -1) instead of a stride.
  std::vector<Range>& ranges = S.ranges;
  ranges.clear();
  int64_t records = 0, n_items = 0, n_merge = 0, n_rec_index = 0;
  int64_t cls_items[2 * kNumClasses] = {};
  for (size_t ti = 0; ti < tiles.size(); ++ti) {
    Tile& t = tiles[ti];
    const int u = t.seq;
    t.range0 = (int32_t)ranges.size();
    for (int p = 0; p < usplits[u]; ++p) {
      const int32_t lo = ubeg[uoff[u] + p], hi = std::min(uend[uoff[u] + p], t.kv_end);
      if (lo < hi) ranges.push_back(Range{(int32_t)ti, lo, hi, (hi - lo + kBlock - 1) / kBlock, 0, 0, 0});
    }
    t.k = (int32_t)ranges.size() - t.range0;
    for (int32_t r = t.range0; r < t.range0 + t.k; ++r) {
      ranges[r].step = t.k * t.n_tok * G;
      ranges[r].row = unit_row(u);
      ranges[r].seq = u < B ? (uint32_t)u : kSeqMulti;
    }
    const bool virt = u >= B, listed = virt || member[u];
    t.row = unit_row(u);
    t.row0 = virt ? vseqs[u - B].row_begin + t.tok_begin : row_off[u] + t.tok_begin;
    t.pos0 = virt ? vseqs[u - B].hi + t.tok_begin : d->q_start[u] + t.tok_begin;
    const int64_t trows = (int64_t)t.n_tok * G;
    if (t.k > 1 || listed) {
      t.rec0 = records;
      records += hkv * t.k * trows;
    }
    n_items += (int64_t)t.k * hkv;
    cls_items[t.cls + (virt ? kNumClasses : 0)] += (int64_t)t.k * hkv;
    if (t.k > 1 && !listed) n_merge += hkv * trows;
    if (listed) n_rec_index += hkv * trows * t.k;
  }
  // each range's task, less its kv head: kv head g takes part + g * k * rows
  std::vector<pmattn_work_item>& rtask = S.rtask;
  rtask.resize(ranges.size());
  for (size_t r = 0; r < ranges.size(); ++r) {
    const Range& rg = ranges[r];
    const Tile& t = tiles[rg.tile];
    rtask[r] = pmattn_work_item{t.row, 0, t.row0, t.n_tok, t.pos0, rg.lo, rg.hi,
                                t.rec0 < 0 ? -1 : (int32_t)(t.rec0 + (int64_t)(r - t.range0) * t.n_tok * G)};
  }
  std::vector<int32_t>& member_slot = S.member_slot;
  int32_t n_member_rows = 0;
  member_slot.assign(rows, -1);
  for (int s = 0; s < B; ++s)
    if (member[s])
      for (int r = 0; r < d->q_len[s]; ++r) member_slot[row_off[s] + r] = n_member_rows++;
  n_merge += (int64_t)n_member_rows * d->num_q_heads;
  if (records > INT32_MAX / 2 || n_items > INT32_MAX / 2 || n_merge > INT32_MAX / 2)
    return fail(PMATTN_E_INVALID, "too many tasks or partial records");
  P.num_records = (int32_t)records;

  // classes in use, and the kernel that serves the plan
  P.class_rows.clear();
  P.class_cascade.clear();
  P.class_begin.assign(1, 0);
  bool has_wave = false, has_wg = false;
  for (int c = 0; c < 2 * kNumClasses; ++c) {
    if (!cls_items[c]) continue;
    P.class_rows.push_back(kClassRows[c % kNumClasses]);
    P.class_cascade.push_back(c >= kNumClasses ? 1 : 0);
    P.class_begin.push_back(P.class_begin.back() + (int32_t)cls_items[c]);
    (kClassRows[c % kNumClasses] <= kClassRows[0] ? has_wave : has_wg) = true;
  }
  // Mixed-batch kernel: a bf16 batch without token trees that mixes 16-row
  // wave tasks with larger ones (a plan of 16- and 32-row tasks only is mixed
  // too: its 32-row tasks run as wave tasks beside the 16-row ones)
  P.mixed = d->dtype == PMATTN_BF16 && !tree && has_wave && has_wg;
  // the mixed table's streams per XCD: [0] workgroup tiles of more than 64
  // rows, [1] other workgroup tasks, [2] 16-row wave tasks, [3] 17..32-row
  // wave tasks
  auto mix_kind = [](int rows) { return rows <= kClassRows[0] ? 2 : rows <= kClassRows[1] ? 3 : rows > kMaxWaveRows ? 0 : 1; };
  int64_t mix_n[4][kXcds] = {};
  int64_t n_mix_entries = 0, n_bundles = 0;
  if (P.mixed) {
    for (const Tile& t : tiles)
      for (int g = 0; g < hkv; ++g) mix_n[mix_kind(kClassRows[t.cls])][xcd_of(g, unit_row(t.seq), hkv)] += t.k;
    for (int x = 0; x < kXcds; ++x) {
      const int64_t nb = (mix_n[2][x] + kWaveTasksPerWg - 1) / kWaveTasksPerWg +
                         (mix_n[3][x] + kWaveTasksPerWg - 1) / kWaveTasksPerWg;
      n_bundles += nb;
      n_mix_entries += mix_n[0][x] + mix_n[1][x] + nb;
    }
  }
  const int64_t n_slots = stream ? hkv * stream_pieces : 0;

  // ---- workspace layout and the upload image --------------------------------
  const size_t sz_items = n_items * sizeof(pmattn_work_item), sz_merge = n_merge * sizeof(pmattn_merge_row),
               sz_mask = S.row_mask.size() * sizeof(uint64_t), sz_append = S.units.size() * sizeof(pmattn_append_unit),
               sz_rec = n_rec_index * sizeof(int32_t), sz_vrow = vrow.size() * sizeof(int32_t),
               sz_slot = (stream ? n_slots + 1 : 0) * sizeof(int32_t), sz_istream = n_items * sizeof(int32_t),
               sz_mix = n_mix_entries * sizeof(int32_t), sz_bundles = n_bundles * kWaveTasksPerWg * sizeof(int32_t);
  P.off_items = 0;
  P.off_merge = align_up(P.off_items + sz_items, kAlign);
  P.off_row_mask = align_up(P.off_merge + sz_merge, kAlign);
  P.off_append = align_up(P.off_row_mask + sz_mask, kAlign);
  P.off_rec_index = align_up(P.off_append + sz_append, kAlign);
  P.off_vrow = align_up(P.off_rec_index + sz_rec, kAlign);
  P.off_slot = align_up(P.off_vrow + sz_vrow, kAlign);
  P.off_istream = align_up(P.off_slot + sz_slot, kAlign);
  P.off_mix_table = align_up(P.off_istream + sz_istream, kAlign);
  P.off_mix_bundles = align_up(P.off_mix_table + sz_mix, kAlign);
  P.off_upload_end = align_up(P.off_mix_bundles + sz_bundles, kAlign);
  P.off_part_o = P.off_upload_end;
  P.off_part_lse = align_up(P.off_part_o + (size_t)records * P.head_dim * sizeof(float), kAlign);
  P.ws_bytes = std::max(kAlign, align_up(P.off_part_lse + (size_t)records * sizeof(float), kAlign));
  P.blob.reset(P.off_upload_end ? new unsigned char[P.off_upload_end] : nullptr);
  unsigned char* blob = P.blob.get();
  {
    // zero the alignment gaps, so that the image is a function of the plan
    const size_t off[] = {P.off_items, P.off_merge, P.off_row_mask, P.off_append, P.off_rec_index, P.off_vrow,
                          P.off_slot, P.off_istream, P.off_mix_table, P.off_mix_bundles, P.off_upload_end};
    const size_t sz[] = {sz_items, sz_merge, sz_mask, sz_append, sz_rec, sz_vrow, sz_slot, sz_istream, sz_mix, sz_bundles};
    for (int i = 0; i < 10; ++i)
      if (off[i + 1] > off[i] + sz[i]) std::memset(blob + off[i] + sz[i], 0, off[i + 1] - off[i] - sz[i]);
  }
  auto* items = reinterpret_cast<pmattn_work_item*>(blob + P.off_items);
  auto* merge = reinterpret_cast<pmattn_merge_row*>(blob + P.off_merge);
  auto* rec_index = reinterpret_cast<int32_t*>(blob + P.off_rec_index);
  auto* slot_begin = reinterpret_cast<int32_t*>(blob + P.off_slot);
  auto* item_stream = reinterpret_cast<int32_t*>(blob + P.off_istream);
  auto* mix_table = reinterpret_cast<int32_t*>(blob + P.off_mix_table);
  auto* mix_bundles = reinterpret_cast<int32_t*>(blob + P.off_mix_bundles);
  if (sz_mask) std::memcpy(blob + P.off_row_mask, S.row_mask.data(), sz_mask);
  if (sz_append) std::memcpy(blob + P.off_append, S.units.data(), sz_append);
  if (sz_vrow) std::memcpy(blob + P.off_vrow, vrow.data(), sz_vrow);
  P.items = {items, (size_t)n_items};
  P.merge_rows = {merge, (size_t)n_merge};
  P.row_mask = {reinterpret_cast<const uint64_t*>(blob + P.off_row_mask), S.row_mask.size()};
  P.append_units = {reinterpret_cast<const pmattn_append_unit*>(blob + P.off_append), S.units.size()};
  P.rec_index = {rec_index, (size_t)n_rec_index};
  P.vrow_src = {reinterpret_cast<const int32_t*>(blob + P.off_vrow), vrow.size()};
  P.slot_begin = {slot_begin, stream ? (size_t)n_slots + 1 : 0};
  P.item_stream = {item_stream, (size_t)n_items};
  P.mix_table = {mix_table, (size_t)n_mix_entries};
  P.mix_bundles = {mix_bundles, (size_t)(n_bundles * kWaveTasksPerWg)};

  // ---- merge rows -------------------------------------------------------------
  // Rows split over several partitions of one tile: nparts records at a
  // stride; rows of cascade sharers: their record lists (rec_index), one entry
  // per (tile, kv head) collected below.
  {
    std::vector<Listed>& listed = S.listed;
    listed.clear();
    int64_t nm = 0;
    P.merge_max_parts = 0;
    P.merge_total_parts = 0;
    for (const Tile& t : tiles) {
      if (!t.k) continue;
      const int u = t.seq;
      const bool virt = u >= B, lst = virt || member[u];
      const int32_t trows = t.n_tok * G;
      for (int g = 0; g < hkv; ++g) {
        const int64_t rec_base = t.rec0 + (int64_t)g * t.k * trows;
        if (lst) listed.push_back(Listed{rec_base, t.k, trows, t.row0, g, virt});
        else if (t.k > 1)
          for (int tok = 0, m = 0; tok < t.n_tok; ++tok)
            for (int i = 0; i < G; ++i, ++m)
              merge[nm++] = pmattn_merge_row{(int32_t)(rec_base + m), trows, t.k, t.row0 + tok, g * G + i};
      }
      if (!lst && t.k > 1) {
        P.merge_max_parts = std::max(P.merge_max_parts, t.k);
        P.merge_total_parts += (int64_t)t.k * trows * hkv;
      }
    }
    if (n_member_rows > 0) {
      // key of (member row, q head): member_slot * Hq + head; each listed
      // block adds its `parts` records to the keys of its rows
      const size_t keys = (size_t)n_member_rows * d->num_q_heads;
      auto row_key = [&](const Listed& lb, int tok) {  // key of the block's token row, head g * G
        const int32_t row = lb.virt ? vrow[lb.row0 + tok] : lb.row0 + tok;
        return (size_t)member_slot[row] * d->num_q_heads + (size_t)lb.g * G;
      };
      std::vector<int32_t>& start = S.rec_start;
      start.assign(keys + 1, 0);
      for (const Listed& lb : listed)
        for (int tok = 0, ntok = lb.trows / G; tok < ntok; ++tok) {
          int32_t* c = start.data() + row_key(lb, tok) + 1;
          for (int i = 0; i < G; ++i) c[i] += lb.parts;
        }
      for (size_t k = 0; k < keys; ++k) start[k + 1] += start[k];
      P.merge_total_parts += start[keys];
      std::vector<int32_t>& fill = S.rec_fill;
      fill.assign(start.begin(), start.end() - 1);
      for (const Listed& lb : listed)
        for (int tok = 0, ntok = lb.trows / G; tok < ntok; ++tok) {
          int32_t* at = fill.data() + row_key(lb, tok);
          const int64_t rec = lb.rec_base + (int64_t)tok * G;  // record of (part 0, token tok, head 0)
          for (int i = 0; i < G; ++i) {
            int32_t* out = rec_index + at[i];
            for (int p = 0; p < lb.parts; ++p) out[p] = (int32_t)(rec + (int64_t)p * lb.trows + i);
            at[i] += lb.parts;
          }
        }
      for (int s = 0; s < B; ++s)
        if (member[s])
          for (int r = 0; r < d->q_len[s]; ++r)
            for (int h = 0; h < d->num_q_heads; ++h) {
              const size_t k = (size_t)member_slot[row_off[s] + r] * d->num_q_heads + h;
              const int32_t np = start[k + 1] - start[k];
              merge[nm++] = pmattn_merge_row{start[k], -1, np, row_off[s] + r, h};
              P.merge_max_parts = std::max(P.merge_max_parts, np);
            }
    }
  }

  // ---- row walk: who reads each pool block --------------------------------
  // Readers are row tiles. A table row's blocks are read by the ranges of its
  // own tiles, and by those of the virtual tiles whose keys it holds. Each
  // row is swept once, segment by segment (runs of block positions under the
  // same ranges; a tile's ranges never share a block, since partitions start
  // on block boundaries). A block is marked with its one reading tile (and
  // that tile's range) and with the one sequence that sees it; it becomes
  // shared when a segment under two ranges covers it, or when another
  // reader (or sequence) marks it later.
  //
  // Streaming tasks: KV no other tile reads. A block read by two row tiles (a
  // shared prefix, or the tiles of one long prefill chunk) is worth keeping
  // in the caches: the second reader often finds it there. A task none of
  // whose blocks is read that way streams its K/V with non-temporal loads
  // (a range loses its flag when one of its blocks becomes shared). A class
  // is 1 when all its tasks stream, 0 when none does, 2 when the kernel must
  // look up each task's flag. (Measured on MI355X: the 64-sequence decode
  // batch 69% -> 77% of HBM peak with non-temporal K/V; the long-decode batch,
  // whose blocks are shared in pairs, 69.5% -> 63.4% had all of it streamed.)
  std::vector<Mark>& marks = S.marks;
  if (marks.size() < (size_t)d->num_pool_blocks) {
    marks.resize(d->num_pool_blocks, Mark{0, 0});
    S.tstamp.resize(d->num_pool_blocks, 0);
  }
  if (++S.gen == 0) {
    std::fill(marks.begin(), marks.end(), Mark{0, 0});
    std::fill(S.tstamp.begin(), S.tstamp.end(), 0u);
    S.gen = 1;
  }
  const uint32_t gen = S.gen;
  const uint32_t nranges = (uint32_t)ranges.size();
  std::vector<char>& rstream = S.rstream;
  rstream.assign(nranges, 1);
  auto seq_of_range = [&](uint32_t r) { return ranges[r].seq; };
  {
    std::vector<uint32_t>& rkey = S.key;
    std::vector<uint32_t>& rorder = S.row_list;
    rkey.resize(nranges);
    rorder.resize(nranges);
    for (uint32_t r = 0; r < nranges; ++r) rkey[r] = (uint32_t)ranges[r].row;
    counting_order(rkey.data(), nranges, (size_t)B, S.cnt, rorder.data());
    std::vector<Event>& ev = S.events;
    std::vector<uint32_t>& active = S.active;  // the ranges over the current position
    std::vector<uint32_t>& slot_of = S.active_slot;  // a range's index in active
    slot_of.resize(nranges);
    for (uint32_t a = 0, e; a < nranges; a = e) {
      const int s = (int)rkey[rorder[a]];
      ev.clear();
      for (e = a; e < nranges && (int)rkey[rorder[e]] == s; ++e) {
        const uint32_t id = rorder[e];
        const Range& r = ranges[id];
        ev.push_back(Event{r.lo / kBlock, id, 1});
        ev.push_back(Event{(r.hi + kBlock - 1) / kBlock, id, 0});
      }
      // by position, ends before starts
      if (ev.size() <= 32) {
        for (size_t i = 1; i < ev.size(); ++i)
          for (size_t j = i; j > 0 && ev[j] < ev[j - 1]; --j) std::swap(ev[j], ev[j - 1]);
      } else {
        std::sort(ev.begin(), ev.end());
      }
      const int32_t* row = bt_row(s);
      active.clear();
      int32_t nvirt = 0;
      for (size_t i = 0; i < ev.size();) {
        const int32_t p = ev[i].pos;
        for (; i < ev.size() && ev[i].pos == p; ++i) {
          const Event& x = ev[i];
          const bool virt = ranges[x.range].seq == kSeqMulti;
          if (x.start) {
            // every range under a segment of two or more reads shared blocks
            // (the ranges that end here have left already)
            slot_of[x.range] = (uint32_t)active.size();
            active.push_back(x.range);
            if (active.size() >= 2) {
              rstream[x.range] = 0;
              rstream[active[0]] = 0;
            }
            nvirt += virt;
          } else {
            const uint32_t at = slot_of[x.range], last = active.back();
            active[at] = last;
            slot_of[last] = at;
            active.pop_back();
            nvirt -= virt;
          }
        }
        if (active.empty() || i == ev.size()) continue;
        const int32_t q = ev[i].pos;  // the segment is [p, q)
        const uint32_t who = nvirt ? kSeqMulti : (uint32_t)s;
        // a block read so far by range `st` alone: it is shared now
        auto to_multi = [&](Mark& m, uint32_t st) {
          rstream[st] = 0;
          m.state = kMultiBit | (seq_of_range(st) == who ? who : kSeqMulti);
        };
        Mark* __restrict__ mk = marks.data();
        if (active.size() == 1) {
          const uint32_t rid = active[0];
          const int32_t tile = ranges[rid].tile;
          bool shared = false;
          for (int32_t j = p; j < q; ++j) {
            Mark& m = mk[row[j]];
            if (m.gen != gen) {
              m = Mark{gen, rid};
              continue;
            }
            const uint32_t st = m.state;
            if (!(st & kMultiBit)) {
              if (ranges[st].tile == tile) continue;  // the same reader
              to_multi(m, st);
            } else if ((st & kSeqMulti) != who) {
              m.state = kMultiBit | kSeqMulti;
            }
            shared = true;
          }
          if (shared) rstream[rid] = 0;
        } else {
          for (int32_t j = p; j < q; ++j) {
            Mark& m = mk[row[j]];
            if (m.gen != gen) {
              m = Mark{gen, kMultiBit | who};
              continue;
            }
            const uint32_t st = m.state;
            if (!(st & kMultiBit)) to_multi(m, st);
            else if ((st & kSeqMulti) != who) m.state = kMultiBit | kSeqMulti;
          }
        }
      }
    }
  }
  // The append check: a block that one sequence writes and no other sequence
  // sees, and that no other unit writes, cannot conflict; otherwise the exact
  // check decides.
  {
    bool exact = false;
    for (const Target& t : S.targets) {
      const Mark& m = marks[t.blk];
      exact = exact || S.tstamp[t.blk] == gen || m.gen != gen ||
              (m.state & kMultiBit ? m.state & kSeqMulti : seq_of_range(m.state)) != (uint32_t)t.seq;
      S.tstamp[t.blk] = gen;
    }
    P.append_conflict = exact ? exact_append_check(d, S.targets) : std::string();
  }

  // ---- order: largest estimated cost first within each class (LPT) --------
  // Within a class, tasks are ordered by XCD and, per XCD, by estimated cost
  // descending (KV blocks: the class fixes the cost per block), ties in
  // generation order (tile, kv head, partition); workgroup slots then take
  // them per XCD (deal). Equal-work decode plans deal wave slots instead.
  uint64_t rng = d->work_shuffle_seed;
  const int rep = hkv >= kXcds ? 1 : (kXcds + hkv - 1) / hkv;  // XCDs per kv head
  std::vector<uint32_t>& tile_first = S.tile_first;
  std::vector<uint32_t>& tile_list = S.tile_list;
  {
    std::vector<uint32_t>& tkey = S.key;
    tkey.resize(tiles.size());
    tile_list.resize(tiles.size());
    for (size_t i = 0; i < tiles.size(); ++i) tkey[i] = tiles[i].cls + (tiles[i].seq >= B ? kNumClasses : 0);
    counting_order(tkey.data(), (uint32_t)tiles.size(), 2 * kNumClasses, S.cnt, tile_list.data());
    tile_first.assign(2 * kNumClasses + 1, 0);
    for (size_t i = 0; i < tiles.size(); ++i) ++tile_first[tkey[i] + 1];
    for (int c = 0; c < 2 * kNumClasses; ++c) tile_first[c + 1] += tile_first[c];
  }
  std::vector<Cand>& cand = S.cand;  // (equal-work decode) the class's tasks in generation order
  std::vector<Cand>& queue = S.queue;  // the class's tasks, per XCD, in queue order
  std::vector<Cand>& outc = S.outc;    // ... and in dispatch order (when shuffled)
  std::vector<uint32_t>& key = S.key;
  std::vector<uint32_t>& order = S.order;
  // per class and XCD, the class's tasks in queue order (largest first), as
  // item indices and KV blocks: qitem[class_begin + [qseg[c][x], qseg[c][x + 1]) )
  std::vector<QItem>& qitem = S.qitem;
  qitem.resize(n_items);
  size_t qseg[2 * kNumClasses][kXcds + 1] = {};
  int64_t pos = 0;
  P.slot_class = -1;
  P.class_stream.clear();
  for (int c = 0, ci = 0; c < 2 * kNumClasses; ++c) {
    if (!cls_items[c]) continue;
    const uint32_t n = (uint32_t)cls_items[c];
    outc.resize(n);
    // writes a task at item index `at` (in dispatch order directly, or after
    // the shuffle)
    int32_t nstream = 0;
    const bool direct = !d->work_shuffle_seed;
    auto emit = [&](int64_t at, const Cand& cd) {
      pmattn_work_item it = rtask[cd.range];
      it.kv_head = cd.g;
      if (it.part >= 0) it.part += cd.g * ranges[cd.range].step;
      items[at] = it;
      nstream += item_stream[at] = rstream[cd.range];
    };
    uint32_t nout = 0;
    if (stream && c == stream_cls) {
      // Slot (g, j) is the run of tasks of kv head g inside piece j, in unit
      // order (each unit's partition p lies in piece start_u / len + p;
      // partitions start at piece boundaries or at the unit's first key, so
      // the first block tells the piece). Slots go to XCDs like tasks (kv head
      // g on XCD g; with fewer than kXcds heads, piece j of head g on XCD
      // g * rep + j % rep), four per workgroup.
      cand.resize(n);
      key.resize(n);
      order.resize(n);
      uint32_t i = 0;
      for (uint32_t k = tile_first[c]; k < tile_first[c + 1]; ++k) {
        const Tile& t = tiles[tile_list[k]];
        for (int g = 0; g < hkv; ++g)
          for (int32_t r = t.range0; r < t.range0 + t.k; ++r) cand[i++] = Cand{(uint32_t)r, (uint16_t)g, 0};
      }
      for (uint32_t k = 0; k < n; ++k) {
        const Range& r = ranges[cand[k].range];
        const int u = tiles[r.tile].seq;
        key[k] = (uint32_t)(cand[k].g * stream_pieces + (stream_start[u] + (r.lo - unit_lo(u)) / kBlock) / stream_len);
      }
      uint32_t* byslot = order.data();
      counting_order(key.data(), n, (size_t)n_slots, S.cnt, byslot);
      std::vector<int32_t>& sfirst = S.slot_first;  // tasks of slot q: byslot[sfirst[q], sfirst[q + 1])
      sfirst.assign(n_slots + 1, 0);
      for (uint32_t k = 0; k < n; ++k) ++sfirst[key[k] + 1];
      for (int64_t q = 0; q < n_slots; ++q) sfirst[q + 1] += sfirst[q];
      // queues of slots per XCD, each in slot order
      std::vector<uint32_t>& qkey = S.slot_key;
      std::vector<uint32_t>& qorder = S.slot_order;
      qkey.resize(n_slots);
      qorder.resize(n_slots);
      size_t qb[kXcds], qe[kXcds] = {};
      for (int g = 0; g < hkv; ++g)
        for (int64_t j = 0; j < stream_pieces; ++j)
          ++qe[qkey[g * stream_pieces + j] = (uint32_t)((g * rep + (int)(j % rep)) % kXcds)];
      counting_order(qkey.data(), (uint32_t)n_slots, kXcds, S.cnt, qorder.data());
      for (size_t x = 0, acc = 0; x < kXcds; ++x) {
        qb[x] = acc;
        qe[x] = acc += qe[x];
      }
      slot_begin[0] = 0;
      int64_t w = 0;
      deal(qb, qe, kWaveTasksPerWg, [&](int, size_t e) {
        const uint32_t q = qorder[e];
        for (int32_t k = sfirst[q]; k < sfirst[q + 1]; ++k) {
          if (direct) emit(pos + nout, cand[byslot[k]]);
          else outc[nout] = cand[byslot[k]];
          ++nout;
        }
        slot_begin[++w] = (int32_t)nout;
      });
      P.slot_class = ci;
    } else {
      // The class's ranges largest first, ties in generation order; each
      // kv head's tasks then follow that order on their XCD. Within a run of
      // one tile's ranges of equal size, heads come before partitions, as in
      // generation order (tile, kv head, partition).
      const uint32_t nr = (uint32_t)(n / hkv);
      uint32_t maxb = 0;
      std::vector<uint32_t>& rlist = S.rlist;
      rlist.resize(nr);
      key.resize(nr);
      order.resize(nr);
      size_t qb[kXcds], qe[kXcds] = {};
      uint32_t i = 0;
      for (uint32_t k = tile_first[c]; k < tile_first[c + 1]; ++k) {
        const Tile& t = tiles[tile_list[k]];
        for (int32_t r = t.range0; r < t.range0 + t.k; ++r) {
          rlist[i++] = (uint32_t)r;
          maxb = std::max(maxb, (uint32_t)ranges[r].nblk);
        }
        const uint32_t xo = (uint32_t)(t.row % rep);
        for (int g = 0; g < hkv; ++g) qe[((uint32_t)g * rep + xo) % kXcds] += t.k;
      }
      for (uint32_t k = 0; k < nr; ++k) key[k] = maxb - (uint32_t)ranges[rlist[k]].nblk;
      counting_order(key.data(), nr, (size_t)maxb + 1, S.cnt, order.data());
      size_t* qs = qseg[c];
      size_t fillp[kXcds];
      for (size_t x = 0, acc = 0; x < kXcds; ++x) {
        qs[x] = qb[x] = fillp[x] = acc;
        qs[x + 1] = qe[x] = acc += qe[x];
      }
      const int per_wg = kClassRows[c % kNumClasses] <= kMaxWaveRows ? kWaveTasksPerWg : 1;
      QItem* qi = qitem.data() + pos;
      if (hkv == kXcds) {
        // one kv head per XCD: every queue is the sorted range list
        std::vector<uint32_t>& srt = S.slot_key;
        srt.resize(nr);
        for (uint32_t k = 0; k < nr; ++k) srt[k] = rlist[order[k]];
        if (direct) {
          // (emit, with the tables it reads held in locals: the stores into
          // the image cannot alias them)
          const pmattn_work_item* __restrict__ rt = rtask.data();
          const Range* __restrict__ rg = ranges.data();
          const char* __restrict__ rs = rstream.data();
          const uint32_t* __restrict__ sr = srt.data();
          pmattn_work_item* __restrict__ out = items + pos;
          int32_t* __restrict__ ost = item_stream + pos;
          const bool mixed = P.mixed;
          auto put = [&](int x, size_t e, uint32_t r) {
            pmattn_work_item it = rt[r];
            it.kv_head = x;
            if (it.part >= 0) it.part += x * rg[r].step;
            out[nout] = it;
            const int32_t st = rs[r];
            ost[nout] = st;
            nstream += st;
            if (mixed) qi[e] = QItem{(int32_t)(pos + nout), rg[r].nblk};
            ++nout;
          };
          deal(qb, qe, per_wg, [&](int x, size_t e) { put(x, e, sr[e - qb[x]]); });
        } else {
          deal(qb, qe, per_wg, [&](int x, size_t e) {
            const uint32_t r = srt[e - qb[x]];
            if (P.mixed) qi[e] = QItem{(int32_t)(pos + nout), ranges[r].nblk};
            outc[nout] = Cand{r, (uint16_t)x, (uint16_t)x};
            ++nout;
          });
        }
      } else {
        queue.resize(n);
        for (uint32_t a = 0, e; a < nr; a = e) {
          const Range& ra = ranges[rlist[order[a]]];
          for (e = a + 1; e < nr; ++e) {
            const Range& rb = ranges[rlist[order[e]]];
            if (rb.tile != ra.tile || rb.nblk != ra.nblk) break;
          }
          const uint32_t xo = (uint32_t)(tiles[ra.tile].row % rep);
          for (int g = 0; g < hkv; ++g) {
            const uint32_t x = ((uint32_t)g * rep + xo) % kXcds;
            for (uint32_t k = a; k < e; ++k) queue[fillp[x]++] = Cand{rlist[order[k]], (uint16_t)g, (uint16_t)x};
          }
        }
        deal(qb, qe, per_wg, [&](int, size_t e) {
          const Cand& cd = queue[e];
          if (P.mixed) qi[e] = QItem{(int32_t)(pos + nout), ranges[cd.range].nblk};
          if (direct) emit(pos + nout, cd);
          else outc[nout] = cd;
          ++nout;
        });
      }
    }
    if (!direct) {
      shuffle(outc.data(), n, rng);
      for (uint32_t k = 0; k < n; ++k) emit(pos + k, outc[k]);
    }
    P.class_stream.push_back(nstream == (int32_t)n ? 1 : nstream == 0 ? 0 : 2);
    pos += n;
    ++ci;
  }

  // ---- mixed-batch kernel table ----------------------------------------------
  // One kernel serves a bf16 batch that mixes 16-row wave tasks (decode rows)
  // with larger tasks (prefill chunks, verify drafts), without token trees
  // (XY-Serve review, "Core claim": one meta-kernel runs every stage's tile
  // tasks from one table, ordered by cost across cores). Each workgroup runs
  // one table entry: a workgroup task (K/V staged once in LDS for its four
  // waves) or a bundle of four wave tasks (one per wave, each streaming its
  // own K/V). Per XCD (kv head g on XCD g, as for the class order, so that
  // readers of a block meet in one L2), both kinds are taken largest first and
  // interleaved in proportion to their KV blocks, so that every CU holds
  // some of each while they run (decode streams HBM beside MFMA-bound prefill
  // tiles; POD-Attention, XY-Serve review reference list) and both kinds end
  // together. Bundles hold four wave tasks of neighbouring cost.
  if (P.mixed) {
    auto nblk_of = [&](uint32_t i) { return (items[i].kv_end - items[i].kv_begin + kBlock - 1) / kBlock; };
    int64_t casc_from = 0;  // cascade classes come after the plain ones
    for (int c = 0; c < kNumClasses; ++c) casc_from += cls_items[c];
    auto is_cascade = [&](int32_t i) { return i >= casc_from ? 1 : 0; };
    // Per stream k and XCD x, the tasks largest first, ties in plan order:
    // mord[seg[k * kXcds + x], seg[k * kXcds + x + 1]).
    const uint32_t n = (uint32_t)n_items;
    std::vector<QItem>& mord = S.mix_order;
    mord.resize(n);
    size_t seg[4 * kXcds + 1] = {};
    int cls_of_kind[4][2] = {{-1, -1}, {-1, -1}, {-1, -1}, {-1, -1}};  // (plain, cascade) class index
    for (int c = 0; c < 2 * kNumClasses; ++c)
      if (cls_items[c]) cls_of_kind[mix_kind(kClassRows[c % kNumClasses])][c >= kNumClasses] = c;
    if (!d->work_shuffle_seed) {
      // each class's XCD queues are in that order already: merge the plain
      // and the cascade class of each stream (plain first on ties, as in plan
      // order)
      size_t w = 0;
      for (int k = 0; k < 4; ++k)
        for (int x = 0; x < kXcds; ++x) {
          seg[k * kXcds + x] = w;
          const QItem *a = nullptr, *ae = nullptr, *b = nullptr, *be = nullptr;
          for (int h = 0; h < 2; ++h) {
            const int c = cls_of_kind[k][h];
            if (c < 0) continue;
            int64_t base = 0;
            for (int cc = 0; cc < c; ++cc) base += cls_items[cc];
            const QItem* lo = qitem.data() + base + qseg[c][x];
            const QItem* hi = qitem.data() + base + qseg[c][x + 1];
            if (h == 0) a = lo, ae = hi;
            else b = lo, be = hi;
          }
          while (a != ae && b != be) mord[w++] = b->nblk > a->nblk ? *b++ : *a++;
          while (a != ae) mord[w++] = *a++;
          while (b != be) mord[w++] = *b++;
        }
      seg[4 * kXcds] = w;
    } else {
      // shuffled class order: sort again (stable counting sort)
      uint32_t maxb = 0;
      for (uint32_t i = 0; i < n; ++i) maxb = std::max(maxb, (uint32_t)nblk_of(i));
      const uint32_t nb = maxb + 1;
      key.resize(n);
      order.resize(n);
      for (size_t c = 0; c + 1 < P.class_begin.size(); ++c) {
        const int kd = mix_kind(P.class_rows[c]);
        for (int32_t i = P.class_begin[c]; i < P.class_begin[c + 1]; ++i) {
          const uint32_t bucket = kd * kXcds + xcd_of(items[i].kv_head, items[i].seq, hkv);
          key[i] = bucket * nb + (maxb - (uint32_t)nblk_of(i));
          ++seg[bucket + 1];
        }
      }
      counting_order(key.data(), n, (size_t)4 * kXcds * nb, S.cnt, order.data());
      for (int k = 0; k < 4 * kXcds; ++k) seg[k + 1] += seg[k];
      for (uint32_t i = 0; i < n; ++i) mord[i] = QItem{(int32_t)order[i], nblk_of(order[i])};
    }
    std::vector<MixEntry>* streams = S.mix_streams;
    std::vector<int32_t>& cat = S.mix_cat;  // the XCDs' lists, end to end
    cat.clear();
    size_t lb[kXcds], le[kXcds];
    int32_t nbund = 0;
    for (int x = 0; x < kXcds; ++x) {
      for (int k = 0; k < 4; ++k) {
        QItem* v = mord.data() + seg[k * kXcds + x];
        const size_t m = seg[k * kXcds + x + 1] - seg[k * kXcds + x];
        if (d->work_shuffle_seed) shuffle(v, m, rng);
        if (k == 0 && m > 1) {
          // The tiles of one sequence side by side (its kv head's tiles are
          // all on this XCD), so that they run at the same time and read its
          // keys once into the L2; sequences in the order of their largest
          // tile. (Measured on MI355X, mixed-chunk batch: in cost order the
          // tiles of one prompt spread over a third of the XCD's entries,
          // and the kernel fetched 3.34 GB beyond the L2 for 2.16 GB of
          // distinct keys.)
          std::vector<int32_t>& gid = S.group_of;  // -1 outside this block
          if (gid.size() < (size_t)B) gid.resize(B, -1);
          std::vector<uint32_t>& gkey = S.gkey;
          std::vector<uint32_t>& gord = S.gorder;
          std::vector<QItem>& tmp = S.gtmp;
          gkey.resize(m);
          gord.resize(m);
          uint32_t ng = 0;
          for (size_t j = 0; j < m; ++j) {
            int32_t& g = gid[items[v[j].item].seq];
            if (g < 0) g = (int32_t)ng++;
            gkey[j] = (uint32_t)g;
          }
          counting_order(gkey.data(), (uint32_t)m, ng, S.cnt, gord.data());
          tmp.assign(v, v + m);
          for (size_t j = 0; j < m; ++j) v[j] = tmp[gord[j]];
          for (size_t j = 0; j < m; ++j) gid[items[v[j].item].seq] = -1;
          // Within a sequence, tiles of equal cost by first key: the row tiles
          // of one KV partition (a cascade prompt's virtual tiles, the tiles of
          // one prefill chunk) start together and share its keys in the L2.
          for (size_t j = 0, e; j < m; j = e) {
            const int32_t s = items[v[j].item].seq;
            for (e = j + 1; e < m && items[v[e].item].seq == s && v[e].nblk == v[j].nblk; ++e) {
            }
            if (e - j > 2)
              std::stable_sort(v + j, v + e, [&](const QItem& x, const QItem& y) {
                return items[x.item].kv_begin < items[y.item].kv_begin;
              });
          }
        }
        streams[k].resize(k < 2 ? m : (m + kWaveTasksPerWg - 1) / kWaveTasksPerWg);
        MixEntry* st = streams[k].data();
        if (k < 2) {
          for (size_t j = 0; j < m; ++j)
            st[j] = MixEntry{v[j].nblk, 4 * v[j].item + 2 * is_cascade(v[j].item)};
          continue;
        }
        // bundles of four wave tasks of neighbouring cost
        for (size_t j = 0; j < m; j += kWaveTasksPerWg) {
          int32_t* slot = mix_bundles + (size_t)nbund * kWaveTasksPerWg;
          for (size_t q = j; q < j + kWaveTasksPerWg; ++q)
            slot[q - j] = q < m ? 2 * v[q].item + is_cascade(v[q].item) : -1;
          st[j / kWaveTasksPerWg] = MixEntry{v[j].nblk, 4 * nbund + 1};  // the bundle's longest task
          ++nbund;
        }
      }
      // Interleave in proportion to KV blocks (next comes the
      // stream that has used the smallest share of its own total), in
      // groups of kSeRoundRobin entries of one stream and neighbouring cost.
      // Within an XCD the hardware deals workgroups to its shader engines
      // round-robin and in order (measured on MI355X: entry k of an XCD
      // always lands on engine k % 4 of a fixed per-XCD order), so a group
      // puts one entry of the same kind on every engine: the engines free
      // their slots at the same pace (one full engine blocks dispatch to
      // the others) and each engine's CUs see every kind in turn.
      lb[x] = cat.size();
      int64_t tot[4] = {0, 0, 0, 0}, used[4] = {0, 0, 0, 0};
      size_t h[4] = {0, 0, 0, 0};
      for (int k = 0; k < 4; ++k) {
        for (const MixEntry& en : streams[k]) tot[k] += en.cost;
        tot[k] *= k == 3 ? kMixVerifyLead : 100;
        for (MixEntry& en : streams[k]) en.cost *= 100;
      }
      // the share a stream has used, as a double: exact for the comparisons
      // while every total stays below 2^26 (two different shares then differ
      // by more than the rounding of either); larger totals compare exactly
      const bool exact = std::max(std::max(tot[0], tot[1]), std::max(tot[2], tot[3])) >= (int64_t)1 << 26;
      const double inf = std::numeric_limits<double>::infinity();
      double share[4];
      for (int k = 0; k < 4; ++k) share[k] = streams[k].empty() ? inf : 0.0;
      for (;;) {
        int k = 0;
        if (!exact) {
          double best = share[0];
          for (int j = 1; j < 4; ++j) {
            const bool lt = share[j] < best;
            best = lt ? share[j] : best;
            k = lt ? j : k;
          }
          if (best == inf) break;
        } else {
          k = -1;
          for (int j = 0; j < 4; ++j) {
            if (h[j] == streams[j].size()) continue;
            if (k < 0 || (__int128)used[j] * tot[k] < (__int128)used[k] * tot[j]) k = j;
          }
          if (k < 0) break;
        }
        const size_t m = std::min<size_t>(kSeRoundRobin, streams[k].size() - h[k]);
        const MixEntry* en = streams[k].data() + h[k];
        for (size_t g = 0; g < m; ++g) {
          used[k] += en[g].cost;
          cat.push_back(en[g].e);
        }
        h[k] += m;
        share[k] = h[k] == streams[k].size() ? inf : (double)used[k] / (double)tot[k];
      }
      le[x] = cat.size();
    }
    // workgroup i runs on XCD i % kXcds; an XCD whose list ran out is
    // topped up from the one with the most entries left
    int64_t nt = 0;
    deal(lb, le, 1, [&](int, size_t e) { mix_table[nt++] = cat[e]; });
  }

  P.id = g_next_plan_id.fetch_add(1);
  return PMATTN_OK;
}

}  // namespace pmattn

using namespace pmattn;

extern "C" {

pmattn_status pmattn_plan(const pmattn_plan_desc* desc, pmattn_plan_t* out) {
  clear_error();
  if (!out) return fail(PMATTN_E_INVALID, "out is NULL");
  *out = nullptr;
  pmattn_plan_s* h = new (std::nothrow) pmattn_plan_s();
  if (!h) return fail(PMATTN_E_NOMEM, "plan allocation failed");
  pmattn_status st;
  try {
    st = build_plan(desc, h->p);
  } catch (const std::bad_alloc&) {
    st = fail(PMATTN_E_NOMEM, "host allocation failed while planning");
  } catch (...) {
    st = fail(PMATTN_E_INVALID, "unexpected error while planning");
  }
  if (st != PMATTN_OK) {
    delete h;
    return st;
  }
  *out = h;
  return PMATTN_OK;
}

pmattn_status pmattn_plan_workspace_bytes(pmattn_plan_t plan, size_t* bytes) {
  clear_error();
  if (!plan || !bytes) return fail(PMATTN_E_INVALID, "NULL argument");
  *bytes = plan->p.ws_bytes;
  return PMATTN_OK;
}

pmattn_status pmattn_plan_export(pmattn_plan_t plan, pmattn_plan_tables* t) {
  clear_error();
  if (!plan || !t) return fail(PMATTN_E_INVALID, "NULL argument");
  Plan& P = plan->p;
  try {
    // the row tables are built on first export (nothing on the launch path
    // reads them)
    std::call_once(P.rows_once, [&P] {
      P.row_seq.resize(P.num_rows);
      P.row_pos.resize(P.num_rows);
      for (int s = 0; s < P.num_seqs; ++s)
        for (int32_t r = P.seq_row_off[s]; r < P.seq_row_off[s + 1]; ++r) {
          P.row_seq[r] = s;
          P.row_pos[r] = P.seq_q_start[s] + (r - P.seq_row_off[s]);
        }
    });
  } catch (const std::bad_alloc&) {
    return fail(PMATTN_E_NOMEM, "host allocation failed while exporting");
  } catch (...) {
    return fail(PMATTN_E_INVALID, "unexpected error while exporting");
  }
  t->num_rows = P.num_rows;
  t->row_seq = P.row_seq.data();
  t->row_pos = P.row_pos.data();
  t->num_seqs = P.num_seqs;
  t->num_splits = P.num_splits.data();
  t->split_offset = P.split_offset.data();
  t->split_begin = P.split_begin.data();
  t->split_end = P.split_end.data();
  t->num_items = (int32_t)P.items.size();
  t->items = P.items.data();
  t->num_classes = (int32_t)P.class_rows.size();
  t->class_rows = P.class_rows.data();
  t->class_begin = P.class_begin.data();
  t->num_merge_rows = (int32_t)P.merge_rows.size();
  t->merge_rows = P.merge_rows.data();
  t->num_part_records = P.num_records;
  t->row_tree_mask = P.row_mask.empty() ? nullptr : P.row_mask.data();
  t->num_append_units = (int32_t)P.append_units.size();
  t->append_units = P.append_units.data();
  t->class_cascade = P.class_cascade.data();
  t->num_cascade = (int32_t)P.cascade_lo.size();
  t->cascade_lo = P.cascade_lo.data();
  t->cascade_hi = P.cascade_hi.data();
  t->cascade_seq = P.cascade_seq.data();
  t->cascade_row_begin = P.cascade_row_begin.data();
  t->cascade_rows = P.cascade_rows.data();
  t->cascade_splits = P.cascade_splits.data();
  t->num_virtual_rows = (int32_t)P.vrow_src.size();
  t->virtual_row_src = P.vrow_src.data();
  t->num_rec_index = (int32_t)P.rec_index.size();
  t->rec_index = P.rec_index.data();
  t->num_slots = P.slot_begin.empty() ? 0 : (int32_t)P.slot_begin.size() - 1;
  t->slot_begin = P.slot_begin.data();
  t->class_stream = P.class_stream.data();
  t->item_stream = P.item_stream.data();
  t->mixed_kernel = P.mixed ? 1 : 0;
  t->num_mix_entries = (int32_t)P.mix_table.size();
  t->mix_table = P.mix_table.data();
  t->num_mix_bundles = (int32_t)(P.mix_bundles.size() / kWaveTasksPerWg);
  t->mix_bundles = P.mix_bundles.data();
  return PMATTN_OK;
}

const char* pmattn_last_error(void) { return g_last_error.c_str(); }

const char* pmattn_status_str(pmattn_status s) {
  switch (s) {
    case PMATTN_OK: return "PMATTN_OK";
    case PMATTN_E_INVALID: return "PMATTN_E_INVALID";
    case PMATTN_E_UNSUPPORTED: return "PMATTN_E_UNSUPPORTED";
    case PMATTN_E_WORKSPACE: return "PMATTN_E_WORKSPACE";
    case PMATTN_E_HIP: return "PMATTN_E_HIP";
    case PMATTN_E_NOMEM: return "PMATTN_E_NOMEM";
    case PMATTN_E_CAPACITY: return "PMATTN_E_CAPACITY";
  }
  return "PMATTN_E_UNKNOWN";
}

const char* pmattn_version(void) { return "0.1.0"; }

}  // extern "C"
