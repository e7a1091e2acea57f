// Work plan of a decode step over a pool whose sequences share blocks (prefix sharing).
//
// Prefix caching reuses the same physical blocks for several requests ("Dynamic HBM
// Repartitioning for Multi-Turn MoE Serving", §II-A), and the paged interface makes them
// plain table entries ("CrossPool", §3.1).  When two sequences have the same token range in
// the same blocks, the keys and values of that range are the same, so one pass over it can
// serve the query heads of every sequence that holds it; each sequence still gets its own
// partial (o, lse) of the range, which its LSE merge takes like any other ("Physically
// Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference", §5.1: partials
// of a partition of the tokens merge exactly).
//
// The plan is host bookkeeping (C++17, no HIP).  Built from the host copy of the block
// table, it is uploaded by the caller and read by kvattn_decode_partial_plan.

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <string>
#include <unordered_map>
#include <vector>

#include "plan_layout.h"
#include "pool_internal.h"

namespace kvattn {

namespace {

struct Item {
  int32_t seq, lo, hi, shared;
  std::vector<int32_t> members;
};

uint64_t mix(uint64_t h, uint64_t v) {
  h ^= v + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
  return h;
}

}  // namespace

}  // namespace kvattn

using namespace kvattn;

extern "C" kvattn_status kvattn_decode_plan(const kvattn_pool* pool, int32_t batch,
                                            int32_t num_q_heads, const int32_t* table,
                                            int32_t max_blocks, const int32_t* ctx_lens,
                                            const int32_t* tok_begin, const int32_t* part_tokens,
                                            int32_t span_parts, int32_t* plan, int64_t plan_cap,
                                            int64_t* plan_len, int32_t* n_groups,
                                            int32_t* max_parts) {
  clear_error();
  if (!pool || !table || !ctx_lens || !part_tokens || !plan_len || !n_groups || !max_parts)
    return set_error(KVATTN_E_INVAL, "decode_plan: null argument");
  const kvattn_layout& L = pool->layout;
  if (batch < 1 || max_blocks < 1 || num_q_heads < 1 || num_q_heads % L.num_kv_heads != 0)
    return set_error(KVATTN_E_INVAL, "decode_plan: bad batch, max_blocks or head count");
  if (L.latent || L.kv_dtype != KVATTN_BF16 || L.block_size < 16 || L.head_dim_k != L.head_dim_v ||
      (L.head_dim_k != 64 && L.head_dim_k != 128 && L.head_dim_k != 256))
    return set_error(KVATTN_E_UNSUPPORTED,
                     "decode_plan: needs a bf16 per-head cache with block size >= 16 and head dim "
                     "64, 128 or 256");
  const int group = num_q_heads / L.num_kv_heads;
  if (group > 16) return set_error(KVATTN_E_UNSUPPORTED, "decode_plan: at most 16 query heads per KV head");
  if (span_parts < 0) return set_error(KVATTN_E_INVAL, "decode_plan: span_parts must be >= 0");
  const int bs = L.block_size;
  const int mpw = 16 / group;  // sequences whose query heads fill one wave's 16 columns

  // per sequence and block position i of its range: the token extent [lo_i, hi_i) and the
  // key (i, block id, extent); sequences with the same key hold the same tokens in the same
  // block.  A position with an invalid id stays private (the kernel flags it).  A block id's
  // first key is found by direct lookup; a block id seen again at another position or with
  // another extent is looked up by its whole key.
  struct Key {
    int64_t a, b;
    bool operator==(const Key& o) const { return a == o.a && b == o.b; }
  };
  struct KeyHash {
    size_t operator()(const Key& k) const { return (size_t)mix(mix(0, (uint64_t)k.a), (uint64_t)k.b); }
  };
  struct KeyRec {
    int32_t i, lo, hi;
  };
  for (int b = 0; b < batch; ++b) {
    const int beg = tok_begin ? tok_begin[b] : 0;
    const int len = ctx_lens[b];
    const int P = part_tokens[b];
    if (beg < 0 || beg > len || (int64_t)len > (int64_t)max_blocks * bs || P <= 0 || P % bs != 0)
      return set_error(KVATTN_E_INVAL, "decode_plan: sequence " + std::to_string(b) +
                                           " needs 0 <= tok_begin <= ctx_len <= max_blocks * "
                                           "block_size and part_tokens a positive multiple of block_size");
    if (span_parts > 0 && (int64_t)span_parts * P / bs >= kPlanWindow)
      return set_error(KVATTN_E_UNSUPPORTED,
                       "decode_plan: span_parts * part_tokens spans more than 127 blocks");
  }
  std::vector<int64_t> pos_off(batch + 1, 0);  // positions of sequence b: [pos_off[b], pos_off[b + 1])
  for (int b = 0; b < batch; ++b) {
    const int beg = tok_begin ? tok_begin[b] : 0;
    const int len = ctx_lens[b];
    pos_off[b + 1] = pos_off[b] + (beg == len ? 0 : (len - 1) / bs - beg / bs + 1);
  }
  std::vector<int32_t> pos_key(pos_off[batch]);  // key of each position, or -1
  std::vector<KeyRec> key_rec;
  std::vector<int32_t> key_count;
  // a block id's first key: an array over the pool's ids where the pool is not much larger
  // than the plan, else a hash map (the cost then follows the plan's positions, not the pool)
  const bool direct = (int64_t)pool->total_blocks <= 16 * pos_off[batch] + 4096;
  std::vector<int32_t> first_key(direct ? pool->total_blocks : 0, -1);
  std::unordered_map<int32_t, int32_t> first_key_map;
  if (!direct) first_key_map.reserve((size_t)pos_off[batch]);
  std::unordered_map<Key, int32_t, KeyHash> key_index;
  for (int b = 0; b < batch; ++b) {
    const int beg = tok_begin ? tok_begin[b] : 0;
    const int len = ctx_lens[b];
    const int32_t* row = table + (int64_t)b * max_blocks;
    int64_t x = pos_off[b];
    if (beg == len) continue;
    for (int i = beg / bs; i <= (len - 1) / bs; ++i, ++x) {
      const int32_t pid = row[i];
      if (pid < 0 || pid >= pool->total_blocks) {
        pos_key[x] = -1;
        continue;
      }
      const int lo = std::max(beg, i * bs), hi = std::min(len, (i + 1) * bs);
      int32_t* slot = direct ? &first_key[pid] : &first_key_map.emplace(pid, -1).first->second;
      int32_t ki = *slot;
      if (ki < 0) {
        ki = *slot = (int32_t)key_rec.size();
        key_rec.push_back({i, lo, hi});
        key_count.push_back(0);
      } else if (key_rec[ki].i != i || key_rec[ki].lo != lo || key_rec[ki].hi != hi) {
        const Key k{((int64_t)i << 32) | (uint32_t)pid, ((int64_t)lo << 32) | (uint32_t)hi};
        auto it = key_index.find(k);
        if (it == key_index.end()) {
          ki = (int32_t)key_rec.size();
          key_index.emplace(k, ki);
          key_rec.push_back({i, lo, hi});
          key_count.push_back(0);
        } else {
          ki = it->second;
        }
      }
      ++key_count[ki];
      pos_key[x] = ki;
    }
  }
  // each key's sequences, ascending, in one flat array
  std::vector<int64_t> key_off(key_count.size() + 1, 0);
  for (size_t k = 0; k < key_count.size(); ++k) key_off[k + 1] = key_off[k] + key_count[k];
  std::vector<int32_t> key_seqs(key_off.back());
  {
    std::vector<int64_t> fill(key_off.begin(), key_off.end() - 1);
    for (int b = 0; b < batch; ++b)
      for (int64_t x = pos_off[b]; x < pos_off[b + 1]; ++x)
        if (pos_key[x] >= 0) key_seqs[fill[pos_key[x]]++] = b;
  }

  // items: maximal runs of positions of a sequence with the same sharers, taken from their
  // lowest sequence, cut into pieces of at most span_parts * part_tokens tokens (span_parts
  // 0: the most whole partitions a wave's window of 127 block ids holds), each split into
  // wave items of up to mpw sequences
  std::vector<Item> items;
  std::vector<int64_t> item_work;  // tokens
  for (int b = 0; b < batch; ++b) {
    const int beg = tok_begin ? tok_begin[b] : 0;
    const int len = ctx_lens[b];
    const int P = part_tokens[b];
    const int span = span_parts > 0 ? span_parts : std::max(1, (kPlanWindow - 1) / (P / bs));
    const int piece_blocks = std::min<int64_t>(kPlanWindow - 1, (int64_t)span * P / bs);
    const int32_t* keys = pos_key.data() + pos_off[b];
    const size_t nkeys = (size_t)(pos_off[b + 1] - pos_off[b]);
    const int i0 = beg / bs;
    const int32_t alone = b;
    // the sharers of a position (an invalid id: its own sequence alone)
    auto sharers = [&](size_t x, const int32_t*& p) -> size_t {
      if (keys[x] < 0) {
        p = &alone;
        return 1;
      }
      p = key_seqs.data() + key_off[keys[x]];
      return (size_t)key_count[keys[x]];
    };
    size_t x = 0;
    while (x < nkeys) {
      const int32_t* S;
      const size_t ns = sharers(x, S);
      size_t y = x + 1;
      for (; y < nkeys; ++y) {
        const int32_t* T;
        const size_t nt = sharers(y, T);
        if (nt != ns || !std::equal(S, S + ns, T)) break;
      }
      if (S[0] == b) {  // the run belongs to its lowest sequence
        for (size_t c = x; c < y; c += piece_blocks) {
          const size_t e = std::min(y, c + (size_t)piece_blocks);
          const int lo = std::max(beg, (int)(i0 + c) * bs);
          const int hi = std::min(len, (int)(i0 + e) * bs);
          for (size_t k = 0; k < ns; k += mpw) {
            Item it{b, lo, hi, ns > 1 ? 1 : 0, {}};
            it.members.assign(S + k, S + std::min(ns, k + (size_t)mpw));
            items.push_back(std::move(it));
            item_work.push_back(hi - lo);
          }
        }
      }
      x = y;
    }
  }

  // wave items of each item's range: a range that several waves read is mode 1 (or staged),
  // one a single wave reads, for however many sharers, is streamed like a private one
  std::vector<int32_t> run_items(items.size(), 1);
  for (size_t k = 0; k < items.size();) {
    size_t e = k + 1;
    while (items[k].shared && e < items.size() && items[e].shared && items[e].seq == items[k].seq &&
           items[e].lo == items[k].lo)
      ++e;
    for (size_t u = k; u < e; ++u) run_items[u] = (int32_t)(e - k);
    k = e;
  }

  // slots: every member's items in order of their first token
  std::vector<std::vector<std::pair<int32_t, int32_t>>> per_seq(batch);  // (lo, item)
  for (size_t k = 0; k < items.size(); ++k)
    for (int32_t m : items[k].members) per_seq[m].push_back({items[k].lo, (int32_t)k});
  std::vector<std::vector<int32_t>> slot_of(items.size());
  for (size_t k = 0; k < items.size(); ++k) slot_of[k].assign(items[k].members.size(), -1);
  int32_t most = 0;
  for (int b = 0; b < batch; ++b) {
    std::sort(per_seq[b].begin(), per_seq[b].end());
    for (size_t s = 0; s < per_seq[b].size(); ++s) {
      const Item& it = items[per_seq[b][s].second];
      const size_t u = std::find(it.members.begin(), it.members.end(), b) - it.members.begin();
      slot_of[per_seq[b][s].second][u] = (int32_t)s;
    }
    most = std::max<int32_t>(most, (int32_t)per_seq[b].size());
  }

  // workgroups of four waves.  A shared range cut into k >= 3 wave items (more sharers than
  // one wave's columns hold) is read by whole workgroups together: its items are split as
  // evenly as possible over ceil(k / 4) workgroups of their own, staged (item mode 2: the four
  // waves load the range once into LDS and each computes its sharers' partials from it; a
  // workgroup of fewer than four items is padded with items of no sequence).  A range of two
  // items goes to one workgroup as two independent waves that read it through L2 (mode 1).
  // Single items, shared (one wave reads the range for all its sharers) or private, fill the
  // free waves, longest work first.  Tuning only: KVATTN_PLAN_STAGE_MIN sets the k from which
  // ranges are staged, KVATTN_PLAN_LAYOUT=same stages none.
  const char* lay_env = std::getenv("KVATTN_PLAN_LAYOUT");
  const std::string layout = lay_env ? lay_env : "stage";
  const char* smin_env = std::getenv("KVATTN_PLAN_STAGE_MIN");
  const size_t stage_min = layout == "stage" ? (smin_env ? (size_t)std::atoi(smin_env) : 3) : SIZE_MAX;
  std::vector<std::vector<int32_t>> groups;       // item indices
  std::vector<char> staged;                       // per group
  std::vector<int32_t> open;                      // groups with free waves
  std::vector<int32_t> order(items.size());
  for (size_t k = 0; k < items.size(); ++k) order[k] = (int32_t)k;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return item_work[x] > item_work[y];
  });
  // a shared range's items are consecutive in `items`; place each run of them as a unit
  std::vector<char> placed(items.size(), 0);
  for (int32_t k : order) {
    if (placed[k] || !items[k].shared) continue;
    auto same = [&](size_t x) {
      return items[x].shared && items[x].seq == items[k].seq && items[x].lo == items[k].lo;
    };
    size_t s = k, e = k;  // the run [s, e]; equal-work sorting may have put k inside it
    while (s > 0 && same(s - 1)) --s;
    while (e + 1 < items.size() && same(e + 1)) ++e;
    const size_t n = e - s + 1;
    if (n == 1) continue;  // a single item: placed with the private ones
    if (n >= stage_min) {
      const size_t ngr = (n + kWavesPerGroup - 1) / kWavesPerGroup;
      size_t at = s;
      for (size_t q = 0; q < ngr; ++q) {
        const size_t take = n / ngr + (q < n % ngr ? 1 : 0);
        groups.push_back({});
        staged.push_back(1);
        for (size_t w = 0; w < take; ++w) {
          groups.back().push_back((int32_t)at);
          placed[at++] = 1;
        }
      }
      continue;
    }
    size_t left = n, at = s;
    while (left >= (size_t)kWavesPerGroup) {
      groups.push_back({});
      staged.push_back(0);
      for (int w = 0; w < kWavesPerGroup; ++w) {
        groups.back().push_back((int32_t)at);
        placed[at++] = 1;
      }
      left -= kWavesPerGroup;
    }
    if (left > 0) {
      int32_t g = -1;
      for (int32_t o : open)
        if (kWavesPerGroup - (int)groups[o].size() >= (int)left) {
          g = o;
          break;
        }
      if (g < 0) {
        g = (int32_t)groups.size();
        groups.push_back({});
        staged.push_back(0);
        open.push_back(g);
      }
      for (size_t w = 0; w < left; ++w) {
        groups[g].push_back((int32_t)at);
        placed[at++] = 1;
      }
      if ((int)groups[g].size() == kWavesPerGroup) open.erase(std::find(open.begin(), open.end(), g));
    }
  }
  size_t oi = 0;
  for (int32_t k : order) {
    if (placed[k]) continue;
    while (oi < open.size() && (int)groups[open[oi]].size() == kWavesPerGroup) ++oi;
    if (oi == open.size()) {
      open.push_back((int32_t)groups.size());
      groups.push_back({});
      staged.push_back(0);
    }
    groups[open[oi]].push_back(k);
    placed[k] = 1;
  }
  // Order of the workgroups in the launch: longest wave item first.  Measured on MI355X on
  // the 64-sequence shared pool, no other order was faster: most HBM bytes first, alternating
  // staged and other workgroups, staged first, staged last.  KVATTN_PLAN_ORDER=bytes (tuning
  // only) orders by HBM bytes: the sum over the distinct ranges of a workgroup's waves.
  std::vector<int64_t> gwork(groups.size(), 0), glong(groups.size(), 0);
  for (size_t g = 0; g < groups.size(); ++g)
    for (size_t u = 0; u < groups[g].size(); ++u) {
      const Item& it = items[groups[g][u]];
      glong[g] = std::max(glong[g], item_work[groups[g][u]]);
      bool seen = false;
      for (size_t v = 0; v < u; ++v) {
        const Item& o = items[groups[g][v]];
        seen |= o.seq == it.seq && o.lo == it.lo && o.hi == it.hi;
      }
      if (!seen) gwork[g] += item_work[groups[g][u]];
    }
  std::vector<int32_t> gorder(groups.size());
  for (size_t g = 0; g < groups.size(); ++g) gorder[g] = (int32_t)g;
  const char* ord = std::getenv("KVATTN_PLAN_ORDER");
  const std::vector<int64_t>& key = (ord && std::string(ord) == "bytes") ? gwork : glong;
  std::stable_sort(gorder.begin(), gorder.end(),
                   [&](int32_t x, int32_t y) { return key[x] > key[y]; });

  // the workgroups in launch order
  std::vector<std::vector<int32_t>> fin;
  std::vector<char> fin_staged;
  for (int32_t g : gorder) {
    fin.push_back(groups[g]);
    fin_staged.push_back(staged[g]);
  }

  int64_t n_members = 0;
  for (const Item& it : items) n_members += (int64_t)it.members.size();
  const int64_t ng = (int64_t)fin.size();
  const int64_t n_item_slots = ng * kWavesPerGroup;
  const int64_t need = kPlanHeader + batch + kItemInts * n_item_slots + 2 * n_members;
  if (need > INT32_MAX || ng > INT32_MAX / 64)
    return set_error(KVATTN_E_INVAL, "decode_plan: plan too large");
  *plan_len = need;
  *n_groups = (int32_t)ng;
  *max_parts = std::max<int32_t>(1, most);
  if (!plan) return KVATTN_OK;  // size query
  if (plan_cap < need) return set_error(KVATTN_E_INVAL, "decode_plan: plan_cap too small");

  int32_t* hdr = plan;
  int32_t* np_out = plan + kPlanHeader;
  int32_t* it_out = np_out + batch;
  int32_t* mem_out = it_out + kItemInts * n_item_slots;
  hdr[0] = kPlanMagic;
  hdr[1] = batch;
  hdr[2] = (int32_t)ng;
  hdr[3] = (int32_t)n_item_slots;
  hdr[4] = (int32_t)n_members;
  hdr[5] = *max_parts;
  hdr[6] = group;
  hdr[7] = mpw;
  for (int b = 0; b < batch; ++b) np_out[b] = (int32_t)per_seq[b].size();
  int32_t moff = 0;
  for (int64_t g = 0; g < ng; ++g) {
    const std::vector<int32_t>& gi = fin[g];
    for (int w = 0; w < kWavesPerGroup; ++w) {
      int32_t* o = it_out + kItemInts * (g * kWavesPerGroup + w);
      const bool st = fin_staged[g];
      if (w >= (int)gi.size()) {  // an idle wave, or a staged wave of no sequence
        for (int i = 0; i < kItemInts; ++i) o[i] = 0;
        if (st) {  // a staged workgroup's first item is a real one
          const Item& f = items[gi[0]];
          o[0] = f.seq; o[1] = f.lo; o[2] = f.hi; o[5] = 2;
        }
        continue;
      }
      const Item& it = items[gi[w]];
      o[0] = it.seq;
      o[1] = it.lo;
      o[2] = it.hi;
      o[3] = (int32_t)it.members.size();
      o[4] = moff;
      o[5] = st ? 2 : (run_items[gi[w]] > 1 ? 1 : 0);
      for (size_t u = 0; u < it.members.size(); ++u) {
        mem_out[2 * moff] = it.members[u];
        mem_out[2 * moff + 1] = slot_of[gi[w]][u];
        ++moff;
      }
    }
  }
  return KVATTN_OK;
}
