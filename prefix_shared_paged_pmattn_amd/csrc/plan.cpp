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
#include <algorithm>
#include <map>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <numeric>

#include "plan_internal.h"

namespace pmattn {

namespace {
thread_local std::string g_last_error;
std::atomic<uint64_t> g_next_plan_id{1};

// XCD-aware dispatch order. K/V of (block, kv head) is read only by tasks of
// that kv head, so all tasks of one kv head go to one XCD (kv heads spread
// over several XCDs when there are fewer than kXcds, by sequence): every task
// that reads a shared block finds it in the same L2. Each XCD keeps its tasks
// in the given (cost-descending) order; workgroup slot i, which the hardware
// gives to XCD i % kXcds, takes the next `per_wg` tasks of that XCD, topped up
// from the XCD with the most tasks left once that one runs out (so that every
// slot but the last holds exactly per_wg tasks).
std::vector<size_t> xcd_order(const std::vector<pmattn_work_item>& v, const std::vector<size_t>& order,
                              int per_wg, int hkv) {
  const int rep = hkv >= kXcds ? 1 : (kXcds + hkv - 1) / hkv;  // XCDs per kv head
  std::vector<std::vector<size_t>> q(kXcds);
  for (size_t i : order) {
    const pmattn_work_item& it = v[i];
    const int x = (hkv >= kXcds ? it.kv_head : it.kv_head * rep + it.seq % rep) % kXcds;
    q[x].push_back(i);
  }
  std::vector<size_t> head(kXcds, 0), out;
  out.reserve(order.size());
  for (size_t slot = 0; out.size() < order.size(); ++slot) {
    int x = (int)(slot % kXcds);
    for (int k = 0; k < per_wg && out.size() < order.size(); ++k) {
      if (head[x] == q[x].size()) {
        size_t best = 0;
        for (int y = 0; y < kXcds; ++y)
          if (q[y].size() - head[y] > best) best = q[y].size() - head[y], x = y;
      }
      out.push_back(q[x][head[x]++]);
    }
  }
  return out;
}

// Dispatch order of an equal-work decode plan. Slot (g, j) is the run of tasks
// of kv head g inside piece j, in unit order (each unit's partition p lies in
// piece start_u / len + p). Slots go to XCDs like tasks in xcd_order (kv head
// g on XCD g; with fewer than kXcds heads, piece j of head g on XCD
// g * rep + j % rep), four slots per workgroup, topped up from the XCD with
// the most slots left. Returns the task order and fills slot_begin.
std::vector<size_t> stream_order(const std::vector<pmattn_work_item>& v, const std::vector<int64_t>& start,
                                 const std::vector<int64_t>& lo, int64_t len, int64_t pieces, int hkv,
                                 std::vector<int32_t>& slot_begin) {
  const int64_t nslot = (int64_t)hkv * pieces;
  std::vector<std::vector<size_t>> slot(nslot);
  for (size_t i = 0; i < v.size(); ++i) {
    const pmattn_work_item& it = v[i];
    // partitions of a stream plan start at piece boundaries or at the unit's
    // first key, so the first block tells the piece
    const int64_t j = (start[it.seq] + (it.kv_begin - lo[it.seq]) / kBlock) / len;
    slot[(int64_t)it.kv_head * pieces + j].push_back(i);
  }
  const int rep = hkv >= kXcds ? 1 : (kXcds + hkv - 1) / hkv;
  std::vector<std::vector<int64_t>> q(kXcds);
  for (int g = 0; g < hkv; ++g)
    for (int64_t j = 0; j < pieces; ++j)
      q[(hkv >= kXcds ? g : g * rep + (int)(j % rep)) % kXcds].push_back((int64_t)g * pieces + j);
  std::vector<size_t> head(kXcds, 0), out;
  out.reserve(v.size());
  slot_begin.assign(1, 0);
  for (int64_t taken = 0, wg = 0; taken < nslot; ++wg) {
    int x = (int)(wg % kXcds);
    for (int k = 0; k < kWaveTasksPerWg && taken < nslot; ++k, ++taken) {
      if (head[x] == q[x].size()) {
        size_t best = 0;
        for (int y = 0; y < kXcds; ++y)
          if (q[y].size() - head[y] > best) best = q[y].size() - head[y], x = y;
      }
      for (size_t i : slot[q[x][head[x]++]]) out.push_back(i);
      slot_begin.push_back((int32_t)out.size());
    }
  }
  return out;
}

// Cost model for ordering and automatic splitting, in "block units": a task
// over n KV blocks costs n * (2 + rows/16). The constant 2 stands for the
// K/V stream of each block, the rows/16 term for its MFMA column tiles.
int64_t unit_cost(int cls) { return 2 + kClassRows[cls] / 16; }
// Automatic splitting aims at this many wave tasks per compute unit, and at
// 1.5 workgroup tasks per compute unit (measured on MI355X against 1, 2 and 4:
// fewer, longer workgroup tasks write fewer partials; 1.5 was 14% faster
// than 4 on the shared-prompt cascade and 5% on tree verify, 1.5% slower on
// the mixed batch) ...
constexpr int64_t kTasksPerCu = 32;
constexpr int64_t kWgTasksPer2Cu = 2;
// ... and 1.5 per CU when the plan holds token trees: their workgroup kernel
// runs at 2 waves per SIMD instead of 3, and measured on MI355X the
// token-tree workload took 0.161-0.163 ms at 1.5 per CU against 0.170-0.172
// at 1, while the shared-prompt cascade took 0.1035-0.1038 ms at 1 against
// 0.1084-0.1089 at 1.5 (mixed batch equal).
constexpr int64_t kWgTasksPer2CuTree = 3;
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
constexpr int64_t kStreamMinBlocks = 16;
// ... but never cuts a task below this many block units.
constexpr int64_t kMinQuantum = 48;
constexpr int kMaxAutoSplits = 64;
// Mixed-batch kernel: estimated duration per KV block (1/100 us) of a tile
// of more than 64 rows, of a smaller workgroup task and of a 16-row wave task,
// measured per table entry on MI355X (mixed-chunk workload, one session:
// 0.72, 0.98 and 1.45 us)
constexpr int64_t kMixTileBlockCost = 72;
constexpr int64_t kMixSmallTaskBlockCost = 98;
constexpr int64_t kMixWaveBlockCost = 145;
// ... and of a 17..32-row wave task (16-key chunks: twice the round trips
// per key of a 16-row task; measured 3.36 us)
constexpr int64_t kMixWave32BlockCost = 336;
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

struct Tile {
  int32_t seq;  // unit: a real sequence (< B) or a virtual cascade sequence
  int32_t tok_begin, n_tok, cls;
  int32_t kv_end;  // one past the tile's last visible key
};
}  // namespace

pmattn_status fail(pmattn_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }

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

  // ---- validate sequences, row tables -------------------------------------
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
    const int32_t* row = d->block_table + (int64_t)s * d->bt_stride;
    for (int64_t j = 0; j < vis_blocks; ++j)
      if (row[j] < 0 || row[j] >= d->num_pool_blocks)
        return fail(PMATTN_E_INVALID, "block id out of [0, num_pool_blocks) at sequence " +
                                          std::to_string(s) + " block " + std::to_string(j));
    rows += ql;
  }
  if (rows > INT32_MAX / std::max(1, d->num_q_heads))
    return fail(PMATTN_E_INVALID, "too many query rows");
  P.num_rows = (int32_t)rows;
  P.row_seq.resize(rows);
  P.row_pos.resize(rows);
  {
    int64_t r = 0;
    for (int s = 0; s < B; ++s)
      for (int t = 0; t < d->q_len[s]; ++t, ++r) {
        P.row_seq[r] = s;
        P.row_pos[r] = d->q_start[s] + t;
      }
  }

  // ---- speculative token trees: per-row visibility of the 64 keys before it --
  // Bit k of a row's mask stands for the key k positions back. Ancestors (and
  // the row itself) set their bits; keys below q_start are context and always
  // visible, so every bit past the row's own index is set too. Chains (parent
  // r - 1) give all ones, the causal rule.
  if (d->tree_parent && rows > 0) {
    bool any_tree = false;
    int64_t r0 = 0;
    for (int s = 0; s < B; ++s) {
      const int ql = d->q_len[s];
      bool chain = true;
      for (int r = 0; r < ql; ++r) {
        const int32_t par = d->tree_parent[r0 + r];
        if (par < -1 || par >= r)
          return fail(PMATTN_E_INVALID, "tree_parent must lie in [-1, row) at sequence " +
                                            std::to_string(s) + " row " + std::to_string(r));
        chain = chain && par == r - 1;
      }
      if (!chain && ql > kMaxTreeRows)
        return fail(PMATTN_E_UNSUPPORTED, "a token tree holds at most 64 rows (sequence " +
                                              std::to_string(s) + ")");
      any_tree = any_tree || !chain;
      r0 += ql;
    }
    if (any_tree) {
      P.row_mask.assign(rows, ~0ull);
      std::vector<uint64_t> anc;  // bit a: row a of the sequence is an ancestor-or-self
      r0 = 0;
      for (int s = 0; s < B; ++s) {
        const int ql = d->q_len[s];
        bool chain = true;
        for (int r = 0; r < ql; ++r) chain = chain && d->tree_parent[r0 + r] == r - 1;
        if (!chain) {
          anc.assign(ql, 0);
          for (int r = 0; r < ql; ++r) {
            const int32_t par = d->tree_parent[r0 + r];
            anc[r] = (par < 0 ? 0ull : anc[par]) | (1ull << r);
            uint64_t m = r < 63 ? ~0ull << (r + 1) : 0ull;
            for (int a = 0; a <= r; ++a)
              if (anc[r] >> a & 1ull) m |= 1ull << (r - a);
            P.row_mask[r0 + r] = m;
          }
        }
        r0 += ql;
      }
    }
  }

  // ---- KV append units and their copy-on-write check ------------------------
  // A unit is the run of a sequence's new tokens that falls into one block.
  // Every slot written must be visible to its own sequence alone.
  {
    struct Target {
      int32_t blk, seq;
      uint32_t slots;  // bit o: slot o is written
    };
    std::vector<Target> targets;
    int64_t r0 = 0;
    for (int s = 0; s < B; ++s) {
      const int ql = d->q_len[s], qs = d->q_start[s];
      const int32_t* bt = d->block_table + (int64_t)s * d->bt_stride;
      for (int t = 0; t < ql;) {
        const int pos = qs + t, j = pos / kBlock, o = pos % kBlock;
        const int n = std::min(ql - t, kBlock - o);
        P.append_units.push_back(pmattn_append_unit{s, (int32_t)(r0 + t), n, j, o});
        targets.push_back(Target{bt[j], s, ((1u << n) - 1u) << o});
        t += n;
      }
      r0 += ql;
    }
    std::sort(targets.begin(), targets.end(),
              [](const Target& a, const Target& b) { return a.blk < b.blk; });
    std::vector<uint64_t> filter(1024, 0);  // 65536-bit filter on the low id bits
    for (const Target& x : targets) filter[(x.blk & 0xFFFF) >> 6] |= 1ull << (x.blk & 63);
    for (size_t i = 1; i < targets.size() && P.append_conflict.empty(); ++i)
      if (targets[i].blk == targets[i - 1].blk && (targets[i].slots & targets[i - 1].slots))
        P.append_conflict = "two query rows write the same pool slot (block " +
                            std::to_string(targets[i].blk) + ")";
    for (int s = 0; s < B && P.append_conflict.empty() && !targets.empty(); ++s) {
      const int64_t kv = (int64_t)d->q_start[s] + d->q_len[s];
      if (d->q_len[s] == 0) continue;
      const int32_t* bt = d->block_table + (int64_t)s * d->bt_stride;
      const int64_t nb = (kv + kBlock - 1) / kBlock;
      for (int64_t j = 0; j < nb; ++j) {
        const int32_t blk = bt[j];
        if (!(filter[(blk & 0xFFFF) >> 6] >> (blk & 63) & 1ull)) continue;
        const uint32_t seen = j + 1 < nb ? 0xFFFFu : (1u << (kv - j * kBlock)) - 1u;
        auto it = std::lower_bound(targets.begin(), targets.end(), blk,
                                   [](const Target& a, int32_t b) { return a.blk < b; });
        for (; it != targets.end() && it->blk == blk; ++it)
          if (it->seq != s && (it->slots & seen)) {
            P.append_conflict = "sequence " + std::to_string(s) + " can see pool slots that sequence " +
                                std::to_string(it->seq) + " appends to (block " +
                                std::to_string(blk) + "): copy the block first";
            break;
          }
        if (!P.append_conflict.empty()) break;
      }
    }
  }

  // ---- cascade: shared prefix runs of decode/verify sequences -----------------
  // Sequences whose rows fit one wave task and whose leading physical blocks
  // coincide are grouped like a radix tree over block ids. Each run of blocks
  // shared by two or more of them, lying wholly before every member's first
  // query row, becomes a virtual sequence: its rows are all members' rows, its
  // keys the run. The members then attend only to the keys after their
  // deepest run, and the log-sum-exp merge joins the parts.
  std::vector<int32_t> row_off(B + 1, 0);
  for (int s = 0; s < B; ++s) row_off[s + 1] = row_off[s] + d->q_len[s];
  std::vector<int32_t> own_lo(B, 0);  // first key of each sequence's own range
  std::vector<char> member(B, 0);
  struct VSeq {
    int32_t lo, hi, table_seq, row_begin, rows;
  };
  std::vector<VSeq> vseqs;
  if (d->cascade) {
    auto bt = [&](int s, int j) { return d->block_table[(int64_t)s * d->bt_stride + j]; };
    auto shareable = [&](int s) { return d->q_start[s] / kBlock; };  // blocks before the first row
    std::vector<int32_t> cands;
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
    stack.push_back(Node{cands, 0, 0});
    std::vector<std::vector<int32_t>> members;
    while (!stack.empty()) {
      Node node = std::move(stack.back());
      stack.pop_back();
      const int32_t depth = node.depth;
      std::map<int32_t, std::vector<int32_t>> buckets;
      for (int32_t m : node.mem)
        if (shareable(m) > depth) buckets[bt(m, depth)].push_back(m);
      std::vector<Node> kids;
      for (auto& kv : buckets) {
        const std::vector<int32_t>& bm = kv.second;
        if (bm.size() < 2) continue;
        int32_t L = depth + 1;
        for (;;) {
          bool same = true;
          for (int32_t m : bm) same = same && shareable(m) > L && bt(m, L) == bt(bm[0], L);
          if (!same) break;
          ++L;
        }
        int32_t cover = node.cover_lo;
        if ((int)bm.size() >= min_members && L - node.cover_lo >= min_blocks) {
          vseqs.push_back(VSeq{node.cover_lo * kBlock, L * kBlock, bm[0], 0, 0});
          members.push_back(bm);
          for (int32_t m : bm) {
            own_lo[m] = L * kBlock;
            member[m] = 1;
          }
          cover = L;
        }
        kids.push_back(Node{bm, L, cover});
      }
      for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(std::move(*it));
    }
    if (d->cascade == 2 && !vseqs.empty()) {
      int64_t spared = 0, logical = 0;
      for (size_t v = 0; v < vseqs.size(); ++v)
        spared += (int64_t)(members[v].size() - 1) * (vseqs[v].hi - vseqs[v].lo);
      for (int s = 0; s < B; ++s)
        if (d->q_len[s] > 0) logical += (int64_t)d->q_start[s] + d->q_len[s];
      if (spared * kCascadeAutoSaveDiv < logical) {
        vseqs.clear();
        members.clear();
        std::fill(own_lo.begin(), own_lo.end(), 0);
        std::fill(member.begin(), member.end(), 0);
      }
    }
    for (size_t v = 0; v < vseqs.size(); ++v) {
      vseqs[v].row_begin = (int32_t)P.vrow_src.size();
      for (int32_t m : members[v])
        for (int32_t r = 0; r < d->q_len[m]; ++r) P.vrow_src.push_back(row_off[m] + r);
      vseqs[v].rows = (int32_t)P.vrow_src.size() - vseqs[v].row_begin;
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

  // ---- tiles: runs of query tokens whose G heads fit one task --------------
  // A unit whose rows fit one wave task (rows * G <= 64) is one tile; longer
  // ones are cut into runs of 128/G tokens for the workgroup kernel.
  const int tok_per_wg = std::max(1, kMaxTaskRows / G);
  std::vector<Tile> tiles;
  for (int u = 0; u < U; ++u) {
    const int ql = unit_rows(u);
    if (ql == 0) continue;
    auto kv_end = [&](int t0, int nt) { return u < B ? d->q_start[u] + t0 + nt : vseqs[u - B].hi; };
    if ((int64_t)ql * G <= kMaxWaveRows) {
      tiles.push_back(Tile{u, 0, ql, class_of_rows(ql * G), kv_end(0, ql)});
      continue;
    }
    for (int t0 = 0; t0 < ql; t0 += tok_per_wg) {
      const int nt = std::min(tok_per_wg, ql - t0);
      tiles.push_back(Tile{u, t0, nt, kNumClasses - 1, kv_end(t0, nt)});
    }
  }

  // ---- KV partitions per unit ------------------------------------------------
  std::vector<int32_t> usplits(U, 0);
  if (d->num_kv_splits > 0) {
    for (int u = 0; u < U; ++u) usplits[u] = unit_rows(u) > 0 ? d->num_kv_splits : 0;
  } else {
    // Two resource classes are balanced separately: wave tasks (<= 64 rows,
    // KV-stream bound) and workgroup tasks (128 rows, MFMA bound). A unit's
    // partition count is ceil(cost of its largest tile / quantum of its class).
    int64_t total[2] = {0, 0};
    std::vector<int64_t> last_cost(U, 0);
    std::vector<int> unit_kind(U, 0);
    for (const Tile& t : tiles) {
      const int kind = kClassRows[t.cls] > kMaxWaveRows ? 1 : 0;
      const int64_t c = (int64_t)((t.kv_end - unit_lo(t.seq) + kBlock - 1) / kBlock) * unit_cost(t.cls);
      total[kind] += c * d->num_kv_heads;
      last_cost[t.seq] = std::max(last_cost[t.seq], c);
      unit_kind[t.seq] = kind;
    }
    const int64_t cus = d->num_cus > 0 ? d->num_cus : 256;
    const int64_t target[2] = {cus * kTasksPerCu, cus * (P.row_mask.empty() ? kWgTasksPer2Cu : kWgTasksPer2CuTree) / 2};
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
  // Equal-work decode (stream) partitions of the decode units: real sequences
  // whose rows make one 16-row wave task. Laid end to end in unit order, unit
  // u holds blocks [S_u, S_u + n_u) of the concatenation; cut it into pieces of
  // L blocks; a unit's partitions are its parts of the pieces it meets, and
  // piece j of kv head g is the work of one wave.
  std::vector<char> sunit(U, 0);
  bool any_stream = false, any_other = V > 0;
  for (const Tile& t : tiles) {
    const bool dec = t.seq < B && t.cls == 0;
    sunit[t.seq] = dec;
    any_stream = any_stream || dec;
    any_other = any_other || !dec;
  }
  const bool stream = d->dtype == PMATTN_BF16 && d->num_kv_splits == 0 && any_stream && !any_other;
  std::vector<int64_t> stream_start(U, 0);
  int64_t stream_len = 0, stream_pieces = 0;
  if (stream) {
    int64_t total = 0;
    for (int u = 0; u < U; ++u) {
      stream_start[u] = total;
      if (sunit[u]) total += (unit_hi(u) - unit_lo(u) + kBlock - 1) / kBlock;
    }
    const int64_t cus = d->num_cus > 0 ? d->num_cus : 256;
    const int64_t per_head = std::max<int64_t>(1, cus * kStreamWavesPerCu / d->num_kv_heads);
    stream_len = std::max(kStreamMinBlocks, (total + per_head - 1) / per_head);
    stream_pieces = (total + stream_len - 1) / stream_len;
    for (int u = 0; u < U; ++u) {
      if (!sunit[u]) continue;
      const int64_t n = (unit_hi(u) - unit_lo(u) + kBlock - 1) / kBlock;
      usplits[u] = (int32_t)((stream_start[u] + n - 1) / stream_len - stream_start[u] / stream_len + 1);
    }
  }
  std::vector<int32_t> uoff(U + 1, 0), ubeg, uend;
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

  // ---- tasks, partial records and merge rows --------------------------------
  // Rows of cascade members collect their records from several tasks: their
  // merge rows list record ids (rec_stride -1) instead of a stride.
  std::vector<std::vector<pmattn_work_item>> by_class(2 * kNumClasses);
  std::vector<int32_t> member_slot(P.num_rows, -1);
  int32_t n_member_rows = 0;
  for (int s = 0; s < B; ++s)
    if (member[s])
      for (int r = 0; r < d->q_len[s]; ++r) member_slot[row_off[s] + r] = n_member_rows++;
  // records of cascade sharers' rows: one entry per (tile, kv head), expanded
  // into rec_index below (count per (row, head), then fill)
  struct Listed {
    int64_t rec_base;
    int32_t parts, trows, row0, g;
    bool virt;
  };
  std::vector<Listed> listed_blocks;
  int64_t records = 0;
  for (const Tile& t : tiles) {
    const int u = t.seq;
    const bool virt = u >= B;
    const int trows = t.n_tok * G;
    const int base = uoff[u];
    int k = 0;
    for (int p = 0; p < usplits[u]; ++p)
      if (ubeg[base + p] < std::min(uend[base + p], t.kv_end)) ++k;
    const bool listed = virt || member[u];
    const bool recs = k > 1 || listed;
    const int32_t row0 = virt ? vseqs[u - B].row_begin + t.tok_begin : row_off[u] + t.tok_begin;
    for (int g = 0; g < d->num_kv_heads; ++g) {
      const int64_t rec_base = records;
      if (recs) records += (int64_t)k * trows;
      int made = 0;
      for (int p = 0; p < usplits[u]; ++p) {
        const int32_t lo = ubeg[base + p];
        const int32_t hi = std::min(uend[base + p], t.kv_end);
        if (lo >= hi) continue;
        pmattn_work_item it;
        it.seq = virt ? vseqs[u - B].table_seq : u;
        it.kv_head = g;
        it.row_begin = row0;
        it.n_tok = t.n_tok;
        it.pos_begin = virt ? vseqs[u - B].hi + t.tok_begin : d->q_start[u] + t.tok_begin;
        it.kv_begin = lo;
        it.kv_end = hi;
        it.part = recs ? (int32_t)(rec_base + (int64_t)made * trows) : -1;
        by_class[t.cls + (virt ? kNumClasses : 0)].push_back(it);
        ++made;
      }
      if (listed && made) listed_blocks.push_back(Listed{rec_base, made, trows, row0, g, virt});
      if (k > 1 && !listed)
        for (int m = 0; m < trows; ++m)
          P.merge_rows.push_back(pmattn_merge_row{(int32_t)(rec_base + m), trows, k, row0 + m / G, g * G + m % G});
    }
  }
  if (n_member_rows > 0) {
    const size_t keys = (size_t)n_member_rows * d->num_q_heads;
    auto key_of = [&](const Listed& lb, int m) {
      const int32_t row = lb.virt ? P.vrow_src[lb.row0 + m / G] : lb.row0 + m / G;
      return (size_t)member_slot[row] * d->num_q_heads + lb.g * G + m % G;
    };
    std::vector<int32_t> start(keys + 1, 0);
    for (const Listed& lb : listed_blocks)
      for (int m = 0; m < lb.trows; ++m) start[key_of(lb, m) + 1] += lb.parts;
    for (size_t k = 0; k < keys; ++k) start[k + 1] += start[k];
    P.rec_index.resize(start[keys]);
    std::vector<int32_t> fill(start.begin(), start.end() - 1);
    for (const Listed& lb : listed_blocks)
      for (int m = 0; m < lb.trows; ++m) {
        int32_t& at = fill[key_of(lb, m)];
        for (int p = 0; p < lb.parts; ++p) P.rec_index[at++] = (int32_t)(lb.rec_base + (int64_t)p * lb.trows + m);
      }
    for (int s = 0; s < B; ++s)
      if (member[s])
        for (int r = 0; r < d->q_len[s]; ++r)
          for (int h = 0; h < d->num_q_heads; ++h) {
            const size_t k = (size_t)member_slot[row_off[s] + r] * d->num_q_heads + h;
            P.merge_rows.push_back(pmattn_merge_row{start[k], -1, start[k + 1] - start[k], row_off[s] + r, h});
          }
  }
  if (records > INT32_MAX / 2) return fail(PMATTN_E_INVALID, "too many partial records");
  P.num_records = (int32_t)records;

  // ---- order: largest estimated cost first within each class (LPT) --------
  uint64_t rng = d->work_shuffle_seed;
  P.class_begin.push_back(0);
  for (int c = 0; c < 2 * kNumClasses; ++c) {
    auto& v = by_class[c];
    if (v.empty()) continue;
    std::vector<int64_t> cost(v.size());
    for (size_t i = 0; i < v.size(); ++i)
      cost[i] = (int64_t)((v[i].kv_end - v[i].kv_begin + kBlock - 1) / kBlock) * unit_cost(c % kNumClasses);
    std::vector<size_t> idx(v.size());
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return cost[a] > cost[b]; });
    if (stream && c == 0) {
      std::vector<int64_t> ulo(B);
      for (int u = 0; u < B; ++u) ulo[u] = unit_lo(u);
      idx = stream_order(v, stream_start, ulo, stream_len, stream_pieces, d->num_kv_heads, P.slot_begin);
      P.slot_class = (int32_t)P.class_rows.size();
    } else
      idx = xcd_order(v, idx, kClassRows[c % kNumClasses] <= kMaxWaveRows ? kWaveTasksPerWg : 1,
                      d->num_kv_heads);
    if (d->work_shuffle_seed)
      for (size_t i = idx.size(); i > 1; --i) std::swap(idx[i - 1], idx[splitmix64(rng) % i]);
    for (size_t i : idx) P.items.push_back(v[i]);
    P.class_rows.push_back(kClassRows[c % kNumClasses]);
    P.class_cascade.push_back(c >= kNumClasses ? 1 : 0);
    P.class_begin.push_back((int32_t)P.items.size());
  }

  // ---- streaming tasks: KV no other tile reads --------------------------------
  // A block read by two row tiles (a shared prefix, or the tiles of one long
  // prefill chunk) is worth keeping in the caches: the second reader often
  // finds it there. A task none of whose blocks is read that way streams its
  // K/V with non-temporal loads. Readers are row tiles, named by their first
  // row (real or virtual); the split and kv-head tasks of one tile read
  // disjoint bytes. A class is 1 when all its tasks stream, 0 when none does,
  // 2 when the kernel must look up each task's flag. (Measured on MI355X: the 64-sequence decode batch 69% -> 77%
  // of HBM peak with non-temporal K/V; the long-decode batch, whose blocks
  // are shared in pairs, 69.5% -> 63.4% had all of it streamed.)
  {
    // Tasks of one tile and partition differ only in their kv head, so each
    // distinct (reader, key range) is walked once.
    // per block: -1 unread, its only reader so far (>= 0), or kMulti
    constexpr int32_t kMulti = -2;
    std::vector<int32_t> reader_of(d->num_pool_blocks, -1);
    auto for_blocks = [&](const pmattn_work_item& it, auto&& fn) {
      const int32_t* row = d->block_table + (int64_t)it.seq * d->bt_stride;
      for (int32_t j = it.kv_begin / kBlock; j * kBlock < it.kv_end; ++j) fn(row[j]);
    };
    // distinct ranges per reader as linked lists (a reader has one range per
    // KV partition of its tile); readers are row indices, real rows first
    std::vector<int32_t> head(row_off[B] + P.vrow_src.size(), -1), next;
    std::vector<size_t> reps;        // one task per distinct (reader, range)
    std::vector<int32_t> item_range(P.items.size());
    for (size_t c = 0; c + 1 < P.class_begin.size(); ++c)
      for (int32_t i = P.class_begin[c]; i < P.class_begin[c + 1]; ++i) {
        const pmattn_work_item& it = P.items[i];
        const int32_t reader = P.class_cascade[c] ? row_off[B] + it.row_begin : it.row_begin;
        int32_t r = head[reader];
        while (r >= 0 && (P.items[reps[r]].kv_begin != it.kv_begin || P.items[reps[r]].kv_end != it.kv_end)) r = next[r];
        if (r >= 0) {
          item_range[i] = r;
          continue;
        }
        item_range[i] = (int32_t)reps.size();
        next.push_back(head[reader]);
        head[reader] = (int32_t)reps.size();
        reps.push_back(i);
        for_blocks(it, [&](int32_t b) {
          const int32_t rd = reader_of[b];
          if (rd != reader && rd != kMulti) reader_of[b] = rd == -1 ? reader : kMulti;
        });
      }
    std::vector<int32_t> rep_stream(reps.size());
    for (size_t r = 0; r < reps.size(); ++r) {
      const pmattn_work_item& it = P.items[reps[r]];
      const int32_t* row = d->block_table + (int64_t)it.seq * d->bt_stride;
      int32_t j = it.kv_begin / kBlock;
      while (j * kBlock < it.kv_end && reader_of[row[j]] != kMulti) ++j;
      rep_stream[r] = j * kBlock >= it.kv_end ? 1 : 0;
    }
    P.item_stream.assign(P.items.size(), 0);
    for (size_t c = 0; c + 1 < P.class_begin.size(); ++c) {
      int32_t n = 0;
      for (int32_t i = P.class_begin[c]; i < P.class_begin[c + 1]; ++i) n += P.item_stream[i] = rep_stream[item_range[i]];
      const int32_t total = P.class_begin[c + 1] - P.class_begin[c];
      P.class_stream.push_back(n == total ? 1 : n == 0 ? 0 : 2);
    }
  }

  // ---- mixed-batch kernel table ----------------------------------------------
  // One kernel serves a bf16 batch that mixes 16-row wave tasks (decode rows)
  // with larger tasks (prefill chunks, verify drafts), without token trees
  // (XY-Serve review, "Core claim": one meta-kernel runs every stage's tile
  // tasks from one table, ordered by cost across cores). Each workgroup runs
  // one table entry: a workgroup task (K/V staged once in LDS for its four
  // waves) or a bundle of four wave tasks (one per wave, each streaming its
  // own K/V). Per XCD (kv head g on XCD g, as in xcd_order, so that readers
  // of a block meet in one L2), both kinds are taken largest first and
  // interleaved in proportion to their estimated cost, so that every CU holds
  // some of each while they run (decode streams HBM beside MFMA-bound prefill
  // tiles; POD-Attention, XY-Serve review reference list) and both kinds end
  // together. Bundles hold four wave tasks of neighbouring cost.
  {
    bool has_wave = false, has_wg = false;
    for (int32_t rows : P.class_rows) (rows <= kClassRows[0] ? has_wave : has_wg) = true;
    P.mixed = d->dtype == PMATTN_BF16 && P.row_mask.empty() && has_wave && has_wg;
    // (a plan of 16- and 32-row tasks only is mixed too: its 32-row tasks run
    // as wave tasks beside the 16-row ones)
    if (P.mixed) {
      const int rep = d->num_kv_heads >= kXcds ? 1 : (kXcds + d->num_kv_heads - 1) / d->num_kv_heads;
      struct Entry {
        int64_t cost;
        int32_t e;
      };
      // streams: [0] workgroup tiles of more than 64 rows, [1] other workgroup
      // tasks, [2] 16-row wave tasks, [3] 17..32-row wave tasks
      std::vector<Entry> parts[4][kXcds];
      for (size_t c = 0; c + 1 < P.class_begin.size(); ++c) {
        const int rows = P.class_rows[c];
        const int k = rows <= kClassRows[0] ? 2 : rows <= kClassRows[1] ? 3 : rows > kMaxWaveRows ? 0 : 1;
        for (int32_t i = P.class_begin[c]; i < P.class_begin[c + 1]; ++i) {
          const pmattn_work_item& it = P.items[i];
          const int x = (d->num_kv_heads >= kXcds ? it.kv_head : it.kv_head * rep + it.seq % rep) % kXcds;
          const int64_t nblk = (it.kv_end - it.kv_begin + kBlock - 1) / kBlock;
          // estimated duration (1/100 us) in this kernel, per KV block: see
          // kMix*BlockCost (a bundle lasts as long as its longest task)
          static constexpr int64_t per_block[4] = {kMixTileBlockCost, kMixSmallTaskBlockCost, kMixWaveBlockCost,
                                                   kMixWave32BlockCost};
          parts[k][x].push_back(Entry{nblk * per_block[k], i * 2 + P.class_cascade[c]});
        }
      }
      std::vector<std::vector<int32_t>> lists(kXcds);
      for (int x = 0; x < kXcds; ++x) {
        std::vector<Entry> streams[4];
        for (int k = 0; k < 4; ++k) {
          auto& v = parts[k][x];
          std::stable_sort(v.begin(), v.end(), [](const Entry& a, const Entry& b) { return a.cost > b.cost; });
          if (d->work_shuffle_seed)
            for (size_t i = v.size(); i > 1; --i) std::swap(v[i - 1], v[splitmix64(rng) % i]);
          if (k < 2) {
            for (const Entry& en : v) streams[k].push_back(Entry{en.cost, 4 * (en.e >> 1) + 2 * (en.e & 1)});
            continue;
          }
          // bundles of four wave tasks of neighbouring cost
          for (size_t i = 0; i < v.size(); i += kWaveTasksPerWg) {
            const int32_t b = (int32_t)(P.mix_bundles.size() / kWaveTasksPerWg);
            for (size_t j = i; j < i + kWaveTasksPerWg; ++j) P.mix_bundles.push_back(j < v.size() ? v[j].e : -1);
            streams[k].push_back(Entry{v[i].cost, 4 * b + 1});  // the bundle's longest task
          }
        }
        // Interleave in proportion to estimated duration (next comes the
        // stream that has used the smallest share of its own total), in
        // groups of kSeRoundRobin entries of one stream and neighbouring cost.
        // Within an XCD the hardware deals workgroups to its shader engines
        // round-robin and in order (measured on MI355X: entry k of an XCD
        // always lands on engine k % 4 of a fixed per-XCD order), so a group
        // puts one entry of the same kind on every engine: the engines free
        // their slots at the same pace (one full engine blocks dispatch to
        // the others) and each engine's CUs see every kind in turn.
        int64_t tot[4] = {0, 0, 0, 0}, used[4] = {0, 0, 0, 0};
        size_t h[4] = {0, 0, 0, 0};
        for (int k = 0; k < 4; ++k)
          for (const Entry& en : streams[k]) tot[k] += en.cost;
        for (;;) {
          int k = -1;
          for (int j = 0; j < 4; ++j) {
            if (h[j] == streams[j].size()) continue;
            if (k < 0 || (__int128)used[j] * tot[k] < (__int128)used[k] * tot[j]) k = j;
          }
          if (k < 0) break;
          for (int g = 0; g < kSeRoundRobin && h[k] < streams[k].size(); ++g) {
            const Entry& en = streams[k][h[k]++];
            used[k] += en.cost;
            lists[x].push_back(en.e);
          }
        }
      }
      // workgroup i runs on XCD i % kXcds; an XCD whose list ran out is
      // topped up from the one with the most entries left
      size_t total = 0;
      for (const auto& l : lists) total += l.size();
      std::vector<size_t> head(kXcds, 0);
      for (size_t slot = 0; P.mix_table.size() < total; ++slot) {
        int x = (int)(slot % kXcds);
        if (head[x] == lists[x].size()) {
          size_t best = 0;
          for (int y = 0; y < kXcds; ++y)
            if (lists[y].size() - head[y] > best) best = lists[y].size() - head[y], x = y;
        }
        P.mix_table.push_back(lists[x][head[x]++]);
      }
    }
  }

  for (const pmattn_merge_row& mr : P.merge_rows) P.merge_max_parts = std::max(P.merge_max_parts, mr.nparts);

  // ---- workspace layout and the upload image --------------------------------
  P.off_items = 0;
  P.off_merge = align_up(P.off_items + P.items.size() * sizeof(pmattn_work_item), kAlign);
  P.off_row_mask = align_up(P.off_merge + P.merge_rows.size() * sizeof(pmattn_merge_row), kAlign);
  P.off_append = align_up(P.off_row_mask + P.row_mask.size() * sizeof(uint64_t), kAlign);
  P.off_rec_index = align_up(P.off_append + P.append_units.size() * sizeof(pmattn_append_unit), kAlign);
  P.off_vrow = align_up(P.off_rec_index + P.rec_index.size() * sizeof(int32_t), kAlign);
  P.off_slot = align_up(P.off_vrow + P.vrow_src.size() * sizeof(int32_t), kAlign);
  P.off_istream = align_up(P.off_slot + P.slot_begin.size() * sizeof(int32_t), kAlign);
  P.off_mix_table = align_up(P.off_istream + P.item_stream.size() * sizeof(int32_t), kAlign);
  P.off_mix_bundles = align_up(P.off_mix_table + P.mix_table.size() * sizeof(int32_t), kAlign);
  P.off_upload_end = align_up(P.off_mix_bundles + P.mix_bundles.size() * sizeof(int32_t), kAlign);
  P.off_part_o = P.off_upload_end;
  P.off_part_lse = align_up(P.off_part_o + (size_t)records * P.head_dim * sizeof(float), kAlign);
  P.ws_bytes = std::max(kAlign, align_up(P.off_part_lse + (size_t)records * sizeof(float), kAlign));
  P.upload_blob.assign(P.off_upload_end, 0);
  if (!P.items.empty())
    std::memcpy(P.upload_blob.data() + P.off_items, P.items.data(),
                P.items.size() * sizeof(pmattn_work_item));
  if (!P.merge_rows.empty())
    std::memcpy(P.upload_blob.data() + P.off_merge, P.merge_rows.data(),
                P.merge_rows.size() * sizeof(pmattn_merge_row));
  if (!P.row_mask.empty())
    std::memcpy(P.upload_blob.data() + P.off_row_mask, P.row_mask.data(),
                P.row_mask.size() * sizeof(uint64_t));
  if (!P.append_units.empty())
    std::memcpy(P.upload_blob.data() + P.off_append, P.append_units.data(),
                P.append_units.size() * sizeof(pmattn_append_unit));
  if (!P.rec_index.empty())
    std::memcpy(P.upload_blob.data() + P.off_rec_index, P.rec_index.data(), P.rec_index.size() * sizeof(int32_t));
  if (!P.vrow_src.empty())
    std::memcpy(P.upload_blob.data() + P.off_vrow, P.vrow_src.data(), P.vrow_src.size() * sizeof(int32_t));
  if (!P.slot_begin.empty())
    std::memcpy(P.upload_blob.data() + P.off_slot, P.slot_begin.data(), P.slot_begin.size() * sizeof(int32_t));
  if (!P.item_stream.empty())
    std::memcpy(P.upload_blob.data() + P.off_istream, P.item_stream.data(), P.item_stream.size() * sizeof(int32_t));
  if (!P.mix_table.empty())
    std::memcpy(P.upload_blob.data() + P.off_mix_table, P.mix_table.data(), P.mix_table.size() * sizeof(int32_t));
  if (!P.mix_bundles.empty())
    std::memcpy(P.upload_blob.data() + P.off_mix_bundles, P.mix_bundles.data(),
                P.mix_bundles.size() * sizeof(int32_t));
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
  const Plan& P = plan->p;
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
  t->slot_begin = P.slot_begin.empty() ? nullptr : P.slot_begin.data();
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
