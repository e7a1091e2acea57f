// Block pool host bookkeeping: regions, free list, reference counts, block tables.
//
// Follows the admission and placement semantics of the pages, restated:
//   - reclaimed HBM joins the same free-block pool as the base KV region and is
//     allocatable at once ("Dynamic HBM Repartitioning for Multi-Turn MoE Serving", §IV-C,
//     §V-A); here every region's blocks share one id space and one free list;
//   - physical placement is the allocator's business, kernels only see block tables, and a
//     request that does not fit is refused without touching running state ("CrossPool",
//     §3.1); here every table call is all-or-nothing;
//   - blocks are the unit of placement ("Physically Partitioned KVCache Format for CPU-GPU
//     Load Balancing in MoE Inference", §4.1).
// Pure C++17 with no HIP dependency, so it is exercised by CPU-only tests.

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "pool_internal.h"

namespace kvattn {

static thread_local std::string g_last_error;

void pool_borrow(kvattn_pool* p) { ++p->borrowers; }

void pool_unborrow(kvattn_pool* p) {
  if (--p->borrowers == 0 && p->free_requested) delete p;
}

kvattn_status set_error(kvattn_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

std::string layout_problem(const kvattn_layout& l) {
  const int bs = l.block_size;
  if (bs < 1 || bs > 256 || (bs & (bs - 1)) != 0) return "block_size must be a power of two in [1, 256]";
  if (l.kv_dtype != KVATTN_F32 && l.kv_dtype != KVATTN_BF16) return "kv_dtype must be KVATTN_F32 or KVATTN_BF16";
  if (l.latent != 0 && l.latent != 1) return "latent must be 0 or 1";
  const int x = 16 / elem_bytes(l.kv_dtype);
  if (l.num_kv_heads < 1) return "num_kv_heads must be >= 1";
  if (l.head_dim_k < 1 || l.head_dim_k % x != 0) return "head_dim_k must be a positive multiple of 16 bytes";
  if (l.head_dim_v < 1 || l.head_dim_v % x != 0) return "head_dim_v must be a positive multiple of 16 bytes";
  if (l.latent) {
    if (l.num_kv_heads != 1) return "a latent cache has num_kv_heads == 1";
    if (l.head_dim_v > l.head_dim_k) return "latent head_dim_v must not exceed head_dim_k";
  }
  return "";
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): golden-ratio increment, then a mix.
static uint64_t splitmix64_next(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace kvattn

using namespace kvattn;

extern "C" {

const char* kvattn_last_error(void) { return g_last_error.c_str(); }

const char* kvattn_version(void) { return "kvattn 0.1.0 (gfx950)"; }

int64_t kvattn_block_bytes(const kvattn_layout* layout) {
  if (!layout || !layout_problem(*layout).empty()) return -1;
  const int64_t e = elem_bytes(layout->kv_dtype);
  if (layout->latent) return (int64_t)layout->block_size * layout->head_dim_k * e;
  return (int64_t)layout->num_kv_heads * layout->block_size *
         (layout->head_dim_k + layout->head_dim_v) * e;
}

kvattn_status kvattn_pool_alloc(const kvattn_layout* layout, const kvattn_region* regions,
                                int32_t n_regions, uint64_t seed, kvattn_pool** out) {
  clear_error();
  if (!layout || !regions || !out) return set_error(KVATTN_E_INVAL, "pool_alloc: null argument");
  std::string why = layout_problem(*layout);
  if (!why.empty()) return set_error(KVATTN_E_INVAL, "pool_alloc: " + why);
  if (n_regions < 1 || n_regions > KVATTN_MAX_REGIONS)
    return set_error(KVATTN_E_INVAL, "pool_alloc: n_regions must be in [1, KVATTN_MAX_REGIONS]");
  int64_t total = 0;
  for (int r = 0; r < n_regions; ++r) {
    if (!regions[r].base || (reinterpret_cast<uintptr_t>(regions[r].base) & 15u) != 0)
      return set_error(KVATTN_E_INVAL, "pool_alloc: region base must be non-null and 16-byte aligned");
    if (regions[r].num_blocks < 0) return set_error(KVATTN_E_INVAL, "pool_alloc: negative num_blocks");
    total += regions[r].num_blocks;
    if (total > INT32_MAX) return set_error(KVATTN_E_INVAL, "pool_alloc: more than 2^31-1 blocks");
  }
  kvattn_pool* p = new kvattn_pool();
  p->layout = *layout;
  p->block_bytes = kvattn_block_bytes(layout);
  p->n_regions = n_regions;
  int64_t first = 0;
  for (int r = 0; r < n_regions; ++r) {
    p->base[r] = regions[r].base;
    p->first_id[r] = first;
    first += regions[r].num_blocks;
  }
  for (int r = n_regions; r <= KVATTN_MAX_REGIONS; ++r) p->first_id[r] = first;
  p->total_blocks = total;
  // Durstenfeld's Fisher-Yates shuffle of 0..N-1; ids[0] is handed out first, so the
  // stack holds the shuffled order reversed (top = back()).
  std::vector<int32_t> ids((size_t)total);
  for (int64_t i = 0; i < total; ++i) ids[(size_t)i] = (int32_t)i;
  uint64_t state = seed;
  for (int64_t i = total - 1; i >= 1; --i) {
    const uint64_t j = splitmix64_next(&state) % (uint64_t)(i + 1);
    std::swap(ids[(size_t)i], ids[(size_t)j]);
  }
  p->free_stack.assign(ids.rbegin(), ids.rend());
  p->refcount.assign((size_t)total, 0);
  *out = p;
  return KVATTN_OK;
}

int32_t kvattn_pool_num_regions(const kvattn_pool* pool) { return pool ? pool->n_regions : -1; }

// New ids [first, first + n) go on top of the free stack so that they are handed out first and
// in ascending order.
static void push_new_ids(kvattn_pool* p, int64_t first, int64_t n) {
  for (int64_t i = first + n - 1; i >= first; --i) p->free_stack.push_back((int32_t)i);
  p->refcount.resize((size_t)(first + n), 0);
}

kvattn_status kvattn_pool_add_region(kvattn_pool* pool, void* base, int64_t num_blocks,
                                     int64_t* first_id) {
  clear_error();
  if (!pool || !base || !first_id) return set_error(KVATTN_E_INVAL, "pool_add_region: null argument");
  if ((reinterpret_cast<uintptr_t>(base) & 15u) != 0 || num_blocks < 1)
    return set_error(KVATTN_E_INVAL, "pool_add_region: base must be 16-byte aligned, num_blocks >= 1");
  if (pool->n_regions >= KVATTN_MAX_REGIONS)
    return set_error(KVATTN_E_INVAL, "pool_add_region: the pool already has KVATTN_MAX_REGIONS regions");
  if (pool->total_blocks + num_blocks > INT32_MAX)
    return set_error(KVATTN_E_INVAL, "pool_add_region: more than 2^31-1 blocks");
  const int r = pool->n_regions;
  const int64_t first = pool->total_blocks;
  pool->base[r] = base;
  pool->first_id[r] = first;
  pool->n_regions = r + 1;
  pool->total_blocks = first + num_blocks;
  for (int i = r + 1; i <= KVATTN_MAX_REGIONS; ++i) pool->first_id[i] = pool->total_blocks;
  push_new_ids(pool, first, num_blocks);
  *first_id = first;
  return KVATTN_OK;
}

kvattn_status kvattn_pool_resize_last_region(kvattn_pool* pool, int64_t num_blocks) {
  clear_error();
  if (!pool) return set_error(KVATTN_E_INVAL, "pool_resize_last_region: null pool");
  const int r = pool->n_regions - 1;
  const int64_t first = pool->first_id[r];
  const int64_t cur = pool->total_blocks - first;
  if (num_blocks < 0 || (num_blocks == 0 && pool->n_regions == 1))
    return set_error(KVATTN_E_INVAL, "pool_resize_last_region: negative size, or removal of the only region");
  if (first + num_blocks > INT32_MAX)
    return set_error(KVATTN_E_INVAL, "pool_resize_last_region: more than 2^31-1 blocks");
  if (num_blocks > cur) {
    pool->total_blocks = first + num_blocks;
    for (int i = r + 1; i <= KVATTN_MAX_REGIONS; ++i) pool->first_id[i] = pool->total_blocks;
    push_new_ids(pool, first + cur, num_blocks - cur);
    return KVATTN_OK;
  }
  if (num_blocks == cur) return KVATTN_OK;
  // shrinking: every removed block must be free
  const int64_t cut = first + num_blocks;
  for (int64_t i = cut; i < pool->total_blocks; ++i)
    if (pool->refcount[(size_t)i] != 0)
      return set_error(KVATTN_E_STATE, "pool_resize_last_region: block " + std::to_string(i) +
                                           " is in use");
  std::vector<int32_t> kept;
  kept.reserve(pool->free_stack.size());
  for (const int32_t id : pool->free_stack)
    if (id < cut) kept.push_back(id);
  pool->free_stack.swap(kept);
  pool->refcount.resize((size_t)cut);
  pool->total_blocks = cut;
  if (num_blocks == 0) {  // the region goes away
    pool->base[r] = nullptr;
    pool->n_regions = r;
  }
  for (int i = pool->n_regions; i <= KVATTN_MAX_REGIONS; ++i) pool->first_id[i] = pool->total_blocks;
  return KVATTN_OK;
}

void kvattn_pool_free(kvattn_pool* pool) {
  if (!pool) return;
  if (pool->borrowers > 0) {  // a store still holds it: deleted when the last one is freed
    pool->free_requested = true;
    return;
  }
  delete pool;
}

int64_t kvattn_pool_num_free(const kvattn_pool* pool) {
  return pool ? (int64_t)pool->free_stack.size() : -1;
}

int64_t kvattn_pool_shared_blocks(const kvattn_pool* pool) {
  return pool ? pool->shared_blocks : -1;
}

int32_t kvattn_pool_refcount(const kvattn_pool* pool, int32_t id) {
  if (!pool || id < 0 || id >= pool->total_blocks) return -1;
  return pool->refcount[(size_t)id];
}

int32_t kvattn_partition_count(int32_t ctx_len, int32_t tok_begin, int32_t part_tokens) {
  if (ctx_len < 0 || tok_begin < 0 || tok_begin > ctx_len || part_tokens <= 0) return -1;
  return (int32_t)ceil_div((int64_t)ctx_len - tok_begin, part_tokens);
}

static kvattn_status explicit_claim(kvattn_pool* p, int32_t batch, const int32_t* ctx_lens,
                                    const int32_t* tab, int32_t max_blocks, int32_t* table_out) {
  const int32_t bs = p->layout.block_size;
  std::unordered_map<int32_t, int32_t> counts;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t nb = ceil_div(ctx_lens[b], bs);
    if (ctx_lens[b] < 0 || nb > max_blocks)
      return set_error(KVATTN_E_INVAL, "block_table: sequence " + std::to_string(b) +
                                           " has a bad length for max_blocks");
    for (int32_t i = 0; i < max_blocks; ++i) {
      const int32_t pid = tab[(size_t)b * max_blocks + i];
      if (pid == KVATTN_BLOCK_ABSENT) continue;
      if (pid < 0 || pid >= p->total_blocks)
        return set_error(KVATTN_E_RANGE, "block_table: id " + std::to_string(pid) + " out of range");
      if (i >= nb)
        return set_error(KVATTN_E_INVAL, "block_table: entry past the sequence end must be ABSENT");
      ++counts[pid];
    }
  }
  for (const auto& kv : counts)
    if (p->refcount[(size_t)kv.first] != 0)
      return set_error(KVATTN_E_STATE, "block_table: block " + std::to_string(kv.first) + " is not free");
  for (const auto& kv : counts) {
    p->refcount[(size_t)kv.first] = kv.second;
    if (kv.second >= 2) ++p->shared_blocks;
  }
  std::vector<int32_t> kept;
  kept.reserve(p->free_stack.size());
  for (int32_t id : p->free_stack)
    if (!counts.count(id)) kept.push_back(id);
  p->free_stack.swap(kept);
  std::memcpy(table_out, tab, sizeof(int32_t) * (size_t)batch * max_blocks);
  return KVATTN_OK;
}

kvattn_status kvattn_block_table(kvattn_pool* pool, int32_t batch, const int32_t* ctx_lens,
                                 const int32_t* first_tok, const int32_t* share_src,
                                 const int32_t* share_nblocks, const int32_t* explicit_table,
                                 int32_t max_blocks, int32_t* table_out, int64_t* shortfall_out) {
  clear_error();
  if (shortfall_out) *shortfall_out = 0;
  if (!pool || !ctx_lens || !table_out) return set_error(KVATTN_E_INVAL, "block_table: null argument");
  if (batch < 1 || max_blocks < 1) return set_error(KVATTN_E_INVAL, "block_table: batch and max_blocks must be >= 1");
  if (explicit_table) return explicit_claim(pool, batch, ctx_lens, explicit_table, max_blocks, table_out);
  if (share_src && !share_nblocks) return set_error(KVATTN_E_INVAL, "block_table: share_src without share_nblocks");

  const int32_t bs = pool->layout.block_size;
  struct Plan { int64_t nb, nabs, nsh; int32_t src; };
  std::vector<Plan> plan((size_t)batch);
  int64_t need = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = ctx_lens[b];
    if (L < 0) return set_error(KVATTN_E_INVAL, "block_table: negative length");
    const int64_t nb = ceil_div(L, bs);
    if (nb > max_blocks) return set_error(KVATTN_E_INVAL, "block_table: sequence needs more than max_blocks blocks");
    const int64_t nabs = first_tok ? first_tok[b] / bs : 0;
    if (first_tok && (first_tok[b] < 0 || first_tok[b] > L))
      return set_error(KVATTN_E_INVAL, "block_table: first_tok must be in [0, ctx_len]");
    const int32_t src = share_src ? share_src[b] : -1;
    int64_t nsh = 0;
    if (src >= 0) {
      nsh = share_nblocks[b];
      if (src >= b || nabs > 0 || nsh < 0)
        return set_error(KVATTN_E_INVAL, "block_table: share_src must name an earlier sequence without ABSENT entries");
      const int64_t src_nb = ceil_div(ctx_lens[src], bs);
      const int64_t src_nabs = first_tok ? first_tok[src] / bs : 0;
      if (nsh > nb || nsh > src_nb || src_nabs > 0)
        return set_error(KVATTN_E_INVAL, "block_table: shared prefix longer than a sequence or not resident");
    }
    const int64_t fresh = nb - std::max(nabs, nsh);
    need += fresh > 0 ? fresh : 0;
    plan[(size_t)b] = Plan{nb, nabs, nsh, src};
  }
  const int64_t avail = (int64_t)pool->free_stack.size();
  if (need > avail) {
    if (shortfall_out) *shortfall_out = need - avail;
    return set_error(KVATTN_E_POOL_EXHAUSTED, "block_table: need " + std::to_string(need) +
                                                  " free blocks, pool has " + std::to_string(avail));
  }
  for (size_t i = 0; i < (size_t)batch * max_blocks; ++i) table_out[i] = KVATTN_BLOCK_ABSENT;
  for (int32_t b = 0; b < batch; ++b) {
    const Plan& pl = plan[(size_t)b];
    int32_t* row = table_out + (size_t)b * max_blocks;
    for (int64_t i = 0; i < pl.nb; ++i) {
      if (i < pl.nabs) continue;
      if (i < pl.nsh) {
        const int32_t pid = table_out[(size_t)pl.src * max_blocks + i];
        if (++pool->refcount[(size_t)pid] == 2) ++pool->shared_blocks;
        row[i] = pid;
      } else {
        const int32_t pid = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->refcount[(size_t)pid] = 1;
        row[i] = pid;
      }
    }
  }
  return KVATTN_OK;
}

kvattn_status kvattn_block_release(kvattn_pool* pool, const int32_t* table, int32_t batch,
                                   int32_t max_blocks) {
  clear_error();
  if (!pool || !table) return set_error(KVATTN_E_INVAL, "block_release: null argument");
  if (batch < 1 || max_blocks < 1) return set_error(KVATTN_E_INVAL, "block_release: batch and max_blocks must be >= 1");
  const size_t n = (size_t)batch * max_blocks;
  std::unordered_map<int32_t, int32_t> counts;
  for (size_t i = 0; i < n; ++i) {
    const int32_t pid = table[i];
    if (pid == KVATTN_BLOCK_ABSENT) continue;
    if (pid < 0 || pid >= pool->total_blocks)
      return set_error(KVATTN_E_RANGE, "block_release: id " + std::to_string(pid) + " out of range");
    ++counts[pid];
  }
  for (const auto& kv : counts)
    if (kv.second > pool->refcount[(size_t)kv.first])
      return set_error(KVATTN_E_STATE, "block_release: block " + std::to_string(kv.first) +
                                           " has fewer references than the table drops");
  for (size_t i = 0; i < n; ++i) {
    const int32_t pid = table[i];
    if (pid == KVATTN_BLOCK_ABSENT) continue;
    const int32_t left = --pool->refcount[(size_t)pid];
    if (left == 1) --pool->shared_blocks;
    if (left == 0) pool->free_stack.push_back(pid);
  }
  return KVATTN_OK;
}

}  // extern "C"
