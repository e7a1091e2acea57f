// Write-time placement of each sequence's KV across the two engines.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference":
//   §4.1  every region is made of fixed-size blocks, and the block is the unit of placement;
//   §4.2  new decode entries are staged in the GPU's window and take part in GPU attention at
//         once; when D of them have accumulated the batch is evicted whole, to the side the
//         share policy picks, and placed entries never move again; prefill is placed in one
//         shot at write time;
//   §5.3  the batches are routed so that the CPU's cumulative share follows r(L).
// Restated for one MI355X: the GPU share stays in HBM where it was written, so a batch routed
// to the GPU moves no data (its blocks change list); a batch routed to the CPU is copied block
// by block into host blocks and its device blocks return to the pool.  Each engine then reads
// its own blocks through a sub-table (its view).  Host bookkeeping; the only device work is
// the copies, enqueued on the caller's stream: one kernel writing straight into the host
// blocks when the host regions are mapped pinned memory, else one hipMemcpyAsync per block.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "pool_internal.h"

struct kvattn_kvstore {
  struct Seq {
    std::vector<int32_t> cpu, gpu, win;
    int64_t w = 0;  // tokens in the window
  };
  kvattn_pool* dev = nullptr;
  kvattn_pool* host = nullptr;
  int32_t batch = 0, D = 0, max_blocks = 0, bs = 0;
  std::vector<kvattn_share_ctl*> ctl;
  std::vector<Seq> seq;
  bool prefill_done = false, flushed = false;
  // device addresses of the host pool's regions when they are mapped pinned memory: copies
  // then run as one kernel writing over the host link.  Queried at the first enqueued copy
  // and again whenever the host pool's regions have changed since (a region added, say).
  int mapped = -1;  // -1 unknown, 0 no, 1 yes
  int mapped_regions = 0;                           // regions the query covered
  void* mapped_host[KVATTN_MAX_REGIONS] = {};       // their host addresses
  void* host_dev_base[KVATTN_MAX_REGIONS] = {};
};

namespace kvattn {

hipError_t launch_copy_blocks(const kvattn_pool* dev, const kvattn_pool* host,
                              void* const* host_bases, const int32_t* pairs, int n, hipStream_t st);

namespace {

// n fresh blocks of pool p appended to out (allocate mode of kvattn_block_table, one sequence)
kvattn_status claim(kvattn_pool* p, int32_t bs, int32_t n, std::vector<int32_t>& out) {
  if (n == 0) return KVATTN_OK;
  std::vector<int32_t> row((size_t)n);
  const int32_t ctx = n * bs;
  int64_t shortfall = 0;
  const kvattn_status st = kvattn_block_table(p, 1, &ctx, nullptr, nullptr, nullptr, nullptr, n,
                                              row.data(), &shortfall);
  if (st != KVATTN_OK) return st;
  out.insert(out.end(), row.begin(), row.end());
  return KVATTN_OK;
}

kvattn_status release(kvattn_pool* p, const int32_t* ids, int32_t n) {
  if (n == 0) return KVATTN_OK;
  return kvattn_block_release(p, ids, 1, n);
}

bool same_layout(const kvattn_layout& a, const kvattn_layout& b) {
  return a.block_size == b.block_size && a.num_kv_heads == b.num_kv_heads &&
         a.head_dim_k == b.head_dim_k && a.head_dim_v == b.head_dim_v &&
         a.kv_dtype == b.kv_dtype && a.latent == b.latent;
}

char* block_address(const kvattn_pool* p, int32_t id) {
  int r = 0;
  while (r + 1 < p->n_regions && id >= p->first_id[r + 1]) ++r;
  return static_cast<char*>(p->base[r]) + (int64_t)(id - p->first_id[r]) * p->block_bytes;
}

// Shared checks of the placement steps: the copy list has room and the host pool has the
// blocks for the worst case (every candidate block to the CPU).
// `per_seq_blocks(q)` is the most blocks sequence q may send to the CPU in this step; its CPU
// view must still fit in max_blocks.
template <class F>
kvattn_status check_worst(const kvattn_kvstore* s, F per_seq_blocks, const int32_t* copies,
                          int32_t max_copies, const char* what) {
  int64_t worst = 0;
  for (const auto& q : s->seq) {
    const int64_t n = per_seq_blocks(q);
    if ((int64_t)q.cpu.size() + n > s->max_blocks)
      return set_error(KVATTN_E_INVAL, std::string(what) + ": a CPU view could exceed max_blocks");
    worst += n;
  }
  if (worst > 0 && (!copies || max_copies < worst))
    return set_error(KVATTN_E_INVAL, std::string(what) + ": the copy list needs room for " +
                                         std::to_string(worst) + " pairs");
  if (worst > kvattn_pool_num_free(s->host))
    return set_error(KVATTN_E_POOL_EXHAUSTED, std::string(what) + ": the host pool has fewer than " +
                                                  std::to_string(worst) + " free blocks");
  return KVATTN_OK;
}

// Moves the first n window blocks of sequence q to the CPU share (claim host blocks, record
// the copies, release the device blocks) or to the GPU share.
kvattn_status place(kvattn_kvstore* s, kvattn_kvstore::Seq& q, int32_t n, bool to_cpu,
                    int32_t* copies, int32_t* n_copies) {
  if (to_cpu) {
    const size_t first = q.cpu.size();
    kvattn_status st = claim(s->host, s->bs, n, q.cpu);
    if (st != KVATTN_OK) return st;
    for (int32_t i = 0; i < n; ++i) {
      copies[2 * (*n_copies)] = q.win[(size_t)i];
      copies[2 * (*n_copies) + 1] = q.cpu[first + (size_t)i];
      ++*n_copies;
    }
    st = release(s->dev, q.win.data(), n);
    if (st != KVATTN_OK) return st;
  } else {
    q.gpu.insert(q.gpu.end(), q.win.begin(), q.win.begin() + n);
  }
  q.win.erase(q.win.begin(), q.win.begin() + n);
  return KVATTN_OK;
}

kvattn_status enqueue_copies(kvattn_kvstore* s, const std::vector<int32_t>& copies, int32_t n,
                             void* hip_stream) {
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (n == 0) return KVATTN_OK;
  bool stale = s->mapped < 0 || s->mapped_regions != s->host->n_regions;
  for (int r = 0; r < s->host->n_regions && !stale; ++r)
    stale = s->mapped_host[r] != s->host->base[r];
  if (stale) {
    s->mapped = 1;
    for (int r = 0; r < KVATTN_MAX_REGIONS; ++r) {
      s->host_dev_base[r] = nullptr;
      s->mapped_host[r] = r < s->host->n_regions ? s->host->base[r] : nullptr;
    }
    s->mapped_regions = s->host->n_regions;
    for (int r = 0; r < s->host->n_regions; ++r) {
      void* d = nullptr;
      if (hipHostGetDevicePointer(&d, s->host->base[r], 0) != hipSuccess || !d) {
        (void)hipGetLastError();  // clear the sticky error of the failed query
        s->mapped = 0;
        break;
      }
      s->host_dev_base[r] = d;
    }
  }
  if (s->mapped == 1) {
    const hipError_t e = launch_copy_blocks(s->dev, s->host, s->host_dev_base, copies.data(), n, st);
    if (e != hipSuccess)
      return set_error(KVATTN_E_HIP, std::string("kvstore copy kernel: ") + hipGetErrorString(e));
    return KVATTN_OK;
  }
  for (int32_t i = 0; i < n; ++i) {
    const hipError_t e = hipMemcpyAsync(block_address(s->host, copies[2 * i + 1]),
                                        block_address(s->dev, copies[2 * i]),
                                        (size_t)s->dev->block_bytes, hipMemcpyDeviceToHost, st);
    if (e != hipSuccess)
      return set_error(KVATTN_E_HIP, std::string("kvstore copy: ") + hipGetErrorString(e));
  }
  return KVATTN_OK;
}

}  // namespace
}  // namespace kvattn

using kvattn::set_error;

extern "C" {

kvattn_status kvattn_kvstore_create(kvattn_pool* dev_pool, kvattn_pool* host_pool, int32_t batch,
                                    int32_t window_tokens, int32_t max_blocks,
                                    kvattn_share_ctl* const* ctls, kvattn_kvstore** out) {
  kvattn::clear_error();
  if (!out) return set_error(KVATTN_E_INVAL, "kvstore_create: null output");
  *out = nullptr;
  if (!dev_pool || !host_pool) return set_error(KVATTN_E_INVAL, "kvstore_create: null pool");
  if (!kvattn::same_layout(dev_pool->layout, host_pool->layout))
    return set_error(KVATTN_E_INVAL, "kvstore_create: the two pools' layouts differ");
  const int32_t bs = dev_pool->layout.block_size;
  if (batch < 1 || max_blocks < 1 || window_tokens < bs || window_tokens % bs != 0)
    return set_error(KVATTN_E_INVAL,
                     "kvstore_create: batch, max_blocks >= 1 and window_tokens a positive "
                     "multiple of the block size required");
  if ((int64_t)max_blocks * bs > 0x7fffffff)
    return set_error(KVATTN_E_INVAL, "kvstore_create: max_blocks * block size exceeds int32");
  kvattn_kvstore* s = new (std::nothrow) kvattn_kvstore();
  if (!s) return set_error(KVATTN_E_INVAL, "kvstore_create: out of host memory");
  s->dev = dev_pool;
  s->host = host_pool;
  s->batch = batch;
  s->D = window_tokens;
  s->max_blocks = max_blocks;
  s->bs = bs;
  s->ctl.assign((size_t)batch, nullptr);
  if (ctls)
    for (int32_t b = 0; b < batch; ++b) s->ctl[(size_t)b] = ctls[b];
  s->seq.resize((size_t)batch);
  kvattn::pool_borrow(dev_pool);
  kvattn::pool_borrow(host_pool);
  *out = s;
  return KVATTN_OK;
}

void kvattn_kvstore_free(kvattn_kvstore* s) {
  if (!s) return;
  for (auto& q : s->seq) {
    kvattn::release(s->host, q.cpu.data(), (int32_t)q.cpu.size());
    kvattn::release(s->dev, q.gpu.data(), (int32_t)q.gpu.size());
    kvattn::release(s->dev, q.win.data(), (int32_t)q.win.size());
  }
  kvattn::pool_unborrow(s->dev);
  kvattn::pool_unborrow(s->host);
  delete s;
}

kvattn_status kvattn_kvstore_reserve(kvattn_kvstore* s, const int32_t* n_new, int32_t* changed) {
  kvattn::clear_error();
  if (!s || !n_new || !changed) return set_error(KVATTN_E_INVAL, "kvstore_reserve: null argument");
  for (int32_t b = 0; b < s->batch; ++b)
    if (n_new[b] < 0) return set_error(KVATTN_E_INVAL, "kvstore_reserve: n_new < 0");
  std::vector<int32_t> need((size_t)s->batch);
  int64_t total = 0;
  for (int32_t b = 0; b < s->batch; ++b) {
    const auto& q = s->seq[(size_t)b];
    const int64_t want = (q.w + n_new[b] + s->bs - 1) / s->bs;
    const int64_t add = std::max<int64_t>(0, want - (int64_t)q.win.size());
    if ((int64_t)q.gpu.size() + (int64_t)q.win.size() + add > s->max_blocks)
      return set_error(KVATTN_E_INVAL, "kvstore_reserve: sequence " + std::to_string(b) +
                                           " would exceed max_blocks in the GPU view");
    need[(size_t)b] = (int32_t)add;
    total += add;
  }
  if (total > kvattn_pool_num_free(s->dev))
    return set_error(KVATTN_E_POOL_EXHAUSTED, "kvstore_reserve: the device pool has fewer than " +
                                                  std::to_string(total) + " free blocks");
  for (int32_t b = 0; b < s->batch; ++b) {
    const kvattn_status st = kvattn::claim(s->dev, s->bs, need[(size_t)b], s->seq[(size_t)b].win);
    if (st != KVATTN_OK) return st;
  }
  *changed = total > 0 ? 1 : 0;
  return KVATTN_OK;
}

kvattn_status kvattn_kvstore_commit(kvattn_kvstore* s, const int32_t* n_new) {
  kvattn::clear_error();
  if (!s || !n_new) return set_error(KVATTN_E_INVAL, "kvstore_commit: null argument");
  for (int32_t b = 0; b < s->batch; ++b) {
    const auto& q = s->seq[(size_t)b];
    if (n_new[b] < 0) return set_error(KVATTN_E_INVAL, "kvstore_commit: n_new < 0");
    if ((q.w + n_new[b] + s->bs - 1) / s->bs > (int64_t)q.win.size())
      return set_error(KVATTN_E_STATE, "kvstore_commit: beyond the reserved window blocks");
  }
  for (int32_t b = 0; b < s->batch; ++b) s->seq[(size_t)b].w += n_new[b];
  return KVATTN_OK;
}

kvattn_status kvattn_kvstore_place_prefill_plan(kvattn_kvstore* s, int32_t* copies,
                                                int32_t max_copies, int32_t* n_copies,
                                                int32_t* changed) {
  kvattn::clear_error();
  if (!s || !n_copies || !changed)
    return set_error(KVATTN_E_INVAL, "kvstore_place_prefill: null argument");
  if (s->prefill_done || s->flushed)
    return set_error(KVATTN_E_STATE, "kvstore_place_prefill: only once, before any flush");
  // the admissions are known before anything changes, so the check is exact
  std::vector<int64_t> ncpu_of((size_t)s->batch, 0);
  for (int32_t b = 0; b < s->batch; ++b) {
    const kvattn_share_ctl* c = s->ctl[(size_t)b];
    if (!c) continue;
    const int64_t full_tokens = (s->seq[(size_t)b].w / s->bs) * s->bs;
    const int64_t t = kvattn::share_admit_tokens(c, full_tokens, s->bs);
    if (t < 0)
      return set_error(KVATTN_E_STATE, "kvstore_place_prefill: controller of sequence " +
                                           std::to_string(b) + " already admitted");
    ncpu_of[(size_t)b] = t / s->bs;
  }
  size_t idx = 0;
  kvattn_status st = kvattn::check_worst(
      s, [&](const kvattn_kvstore::Seq&) { return ncpu_of[idx++]; }, copies, max_copies,
      "kvstore_place_prefill");
  if (st != KVATTN_OK) return st;
  *n_copies = 0;
  *changed = 0;
  for (int32_t b = 0; b < s->batch; ++b) {
    auto& q = s->seq[(size_t)b];
    const int32_t full = (int32_t)(q.w / s->bs);
    int64_t cpu_tokens = 0;
    if (s->ctl[(size_t)b]) {
      st = kvattn_share_admit(s->ctl[(size_t)b], (int64_t)full * s->bs, s->bs, &cpu_tokens);
      if (st != KVATTN_OK) return st;
    }
    const int32_t ncpu = (int32_t)(cpu_tokens / s->bs);
    st = kvattn::place(s, q, ncpu, true, copies, n_copies);
    if (st == KVATTN_OK) st = kvattn::place(s, q, full - ncpu, false, copies, n_copies);
    if (st != KVATTN_OK) return st;
    q.w -= (int64_t)full * s->bs;
    if (ncpu > 0) *changed = 1;
  }
  s->prefill_done = true;
  return KVATTN_OK;
}

kvattn_status kvattn_kvstore_flush_plan(kvattn_kvstore* s, int32_t* copies, int32_t max_copies,
                                        int32_t* n_copies, int32_t* changed) {
  kvattn::clear_error();
  if (!s || !n_copies || !changed) return set_error(KVATTN_E_INVAL, "kvstore_flush: null argument");
  const int32_t nb = s->D / s->bs;
  kvattn_status st = kvattn::check_worst(
      s, [&](const kvattn_kvstore::Seq& q) { return (q.w / s->D) * nb; }, copies, max_copies,
      "kvstore_flush");
  if (st != KVATTN_OK) return st;
  *n_copies = 0;
  *changed = 0;
  for (int32_t b = 0; b < s->batch; ++b) {
    auto& q = s->seq[(size_t)b];
    while (q.w >= s->D) {
      int32_t to_cpu = 0;
      if (s->ctl[(size_t)b]) {
        st = kvattn_share_route(s->ctl[(size_t)b], s->D, &to_cpu);
        if (st != KVATTN_OK) return st;
      }
      st = kvattn::place(s, q, nb, to_cpu != 0, copies, n_copies);
      if (st != KVATTN_OK) return st;
      q.w -= s->D;
      if (to_cpu) *changed = 1;
    }
  }
  s->flushed = true;
  return KVATTN_OK;
}

kvattn_status kvattn_kvstore_place_prefill(kvattn_kvstore* s, void* hip_stream, int32_t* changed) {
  if (!s) return set_error(KVATTN_E_INVAL, "kvstore_place_prefill: null store");
  int64_t worst = 0;
  for (const auto& q : s->seq) worst += q.w / s->bs;
  std::vector<int32_t> copies((size_t)std::max<int64_t>(1, 2 * worst));
  int32_t n = 0;
  const kvattn_status st = kvattn_kvstore_place_prefill_plan(s, copies.data(), (int32_t)worst, &n,
                                                             changed);
  if (st != KVATTN_OK) return st;
  return kvattn::enqueue_copies(s, copies, n, hip_stream);
}

kvattn_status kvattn_kvstore_flush(kvattn_kvstore* s, void* hip_stream, int32_t* changed) {
  if (!s) return set_error(KVATTN_E_INVAL, "kvstore_flush: null store");
  int64_t worst = 0;
  for (const auto& q : s->seq) worst += (q.w / s->D) * (s->D / s->bs);
  std::vector<int32_t> copies((size_t)std::max<int64_t>(1, 2 * worst));
  int32_t n = 0;
  const kvattn_status st = kvattn_kvstore_flush_plan(s, copies.data(), (int32_t)worst, &n, changed);
  if (st != KVATTN_OK) return st;
  return kvattn::enqueue_copies(s, copies, n, hip_stream);
}

kvattn_status kvattn_kvstore_views(const kvattn_kvstore* s, int32_t* gpu_table, int32_t* gpu_len,
                                   int32_t* cpu_table, int32_t* cpu_len) {
  kvattn::clear_error();
  if (!s || !gpu_table || !gpu_len || !cpu_table || !cpu_len)
    return set_error(KVATTN_E_INVAL, "kvstore_views: null argument");
  for (int32_t b = 0; b < s->batch; ++b) {
    const auto& q = s->seq[(size_t)b];
    int32_t* g = gpu_table + (int64_t)b * s->max_blocks;
    int32_t* c = cpu_table + (int64_t)b * s->max_blocks;
    std::fill(g, g + s->max_blocks, KVATTN_BLOCK_ABSENT);
    std::fill(c, c + s->max_blocks, KVATTN_BLOCK_ABSENT);
    std::copy(q.gpu.begin(), q.gpu.end(), g);
    std::copy(q.win.begin(), q.win.end(), g + q.gpu.size());
    std::copy(q.cpu.begin(), q.cpu.end(), c);  // both views fit: checked when they grow
    gpu_len[b] = (int32_t)((int64_t)q.gpu.size() * s->bs + q.w);
    cpu_len[b] = (int32_t)((int64_t)q.cpu.size() * s->bs);
  }
  return KVATTN_OK;
}

}  // extern "C"
