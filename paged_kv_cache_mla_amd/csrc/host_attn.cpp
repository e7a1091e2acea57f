// CPU share of a decode step: the partial (o, lse) of each sequence's leading tokens, computed
// on the host from blocks in host memory laid out like the device pool.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference":
//   §5.1  the two engines split each sequence along its tokens, both over all heads, and the
//         partials merge exactly by LSE rescaling (here: kvattn_merge_lse on the GPU);
//   §4.2  the CPU returns only its partial output and normaliser, orders of magnitude smaller
//         than the KV it read;
//   §6.1  the CPU kernel reads the blocks in place (no contiguous copies), keeps scores in
//         registers / L1 with an online softmax (running max and normaliser), accumulates in
//         fp32, and for MLA reads each latent once for all heads.
// Restated for this library: work items are (sequence, KV head, chunk of whole blocks); each
// block of an item is widened to fp32 into small tiles laid out so that both products run
// over contiguous memory with AVX2 (plain loops for partial blocks and fp32 caches), then
// folded into a per-head online softmax.  Items are taken by persistent worker threads from a
// shared counter; each item's partial is merged into the sequence's result in chunk order, so
// the output does not depend on the thread count or timing.
// Pure C++17 with no HIP dependency.

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include <immintrin.h>
#include <sched.h>

#include "pool_internal.h"

namespace kvattn {
namespace {

constexpr int kMaxGroup = 16;        // query heads per KV head
constexpr int kChunkTokens = 1024;   // tokens per work item (rounded to whole blocks)

// Persistent workers: the per-step fixed cost of the CPU share (thread start-up, first touch of
// the partial workspace) is paid once per process, not once per decode step.  After a call a
// worker that took part spins on the job word for kSpinNs before sleeping on a condition
// variable, so calls that follow each other within a decode loop wake it without a system
// call; workers a call did not need go straight back to sleep.  One call runs at
// a time (call_mu); the workspace vectors are reused across calls under that lock.  The pool is
// never destroyed (its threads sleep until the process ends).
class WorkerPool {
 public:
  static WorkerPool& get() {
    static WorkerPool* p = new WorkerPool();
    return *p;
  }

  // Runs fn(i) for i in [0, n) on n workers, the calling thread being worker 0; returns when all
  // have finished.  The caller holds call_mu.
  void run(int n, const std::function<void(int)>& fn) {
    if (n <= 1) {  // nothing to hand out: no worker is woken
      fn(0);
      return;
    }
    while ((int)threads_.size() < n - 1) {
      const int idx = (int)threads_.size() + 1;
      threads_.emplace_back([this, idx] { loop(idx); });
      threads_.back().detach();
    }
    job_ = &fn;
    pending_.store(n - 1, std::memory_order_relaxed);
    // generation and worker count change together, so a worker never pairs one call's count
    // with another call's generation; the release publishes job_ and pending_
    const uint64_t gen = (state_.load(std::memory_order_relaxed) >> 8) + 1;
    state_.store(gen << 8 | (uint64_t)n, std::memory_order_release);
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (sleeping_ > 0) cv_.notify_all();
    }
    fn(0);
    while (pending_.load(std::memory_order_acquire) != 0) _mm_pause();
  }

  std::mutex call_mu;
  std::vector<float> ws_o, ws_m, ws_l;

 private:
  static constexpr int64_t kSpinNs = 2000000;  // 2 ms

  // state_ = generation << 8 | workers of that generation's call
  void loop(int idx) {
    uint64_t seen = 0;     // generation last handled
    bool worked = false;   // took part in that generation's call: spin before sleeping
    for (;;) {
      uint64_t w = state_.load(std::memory_order_acquire);
      if (w >> 8 == seen) {
        const auto t0 = std::chrono::steady_clock::now();
        int polls = 0;
        while (worked && (w = state_.load(std::memory_order_acquire)) >> 8 == seen) {
          _mm_pause();
          if (++polls == 256) {
            polls = 0;
            if (std::chrono::duration_cast<std::chrono::nanoseconds>(
                    std::chrono::steady_clock::now() - t0).count() > kSpinNs)
              break;
          }
        }
        if (w >> 8 == seen) {
          std::unique_lock<std::mutex> lk(mu_);
          ++sleeping_;
          cv_.wait(lk, [&] { return (w = state_.load(std::memory_order_acquire)) >> 8 != seen; });
          --sleeping_;
        }
      }
      seen = w >> 8;
      // a worker of this generation's call: the caller waits for it before the next call, so
      // job_ is still this call's job
      worked = (uint64_t)idx < (w & 255);
      if (worked) {
        (*job_)(idx);
        pending_.fetch_sub(1, std::memory_order_acq_rel);
      }
    }
  }

  std::mutex mu_;
  std::condition_variable cv_;
  int sleeping_ = 0;  // guarded by mu_
  std::vector<std::thread> threads_;
  const std::function<void(int)>* job_ = nullptr;
  std::atomic<uint64_t> state_{0};
  std::atomic<int> pending_{0};
};

struct HostCtx {
  kvattn_layout L;
  int64_t block_elems;
  int n_regions;
  const void* base[KVATTN_MAX_REGIONS];
  int64_t first[KVATTN_MAX_REGIONS + 1];
  const void* q;
  bool q_f32;
  int batch, hq, hkv, group;
  float scale;
  const int32_t* table;
  int max_blocks;
  const int32_t* tok_end;
};

inline float bf16_f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Element e of a block as fp32 (T = float for fp32 caches, uint16_t for bf16 bit patterns).
template <typename T>
inline float elem(const T* blk, int64_t e) {
  if constexpr (sizeof(T) == 4) {
    return blk[e];
  } else {
    return bf16_f(blk[e]);
  }
}

const void* block_base(const HostCtx& c, int32_t pid) {
  int r = 0;
  while (r + 1 < c.n_regions && pid >= c.first[r + 1]) ++r;
  const int64_t eb = c.L.kv_dtype == KVATTN_F32 ? 4 : 2;
  return static_cast<const char*>(c.base[r]) + (pid - c.first[r]) * c.block_elems * eb;
}

// Online-softmax state of the heads of one KV head over some tokens (natural-log domain).
struct State {
  float m[kMaxGroup], l[kMaxGroup];
  std::vector<float> acc;  // [group][Dv]
};

// Online-softmax update of head h with the scores s[0..n) of one block; returns the weights
// p[t] (relative to the new running max) in s and the factor the accumulator must be scaled by.
inline float softmax_update(State& st, int h, float* s, int n, float scale) {
  float mx = -INFINITY;
  for (int t = 0; t < n; ++t) {
    s[t] *= scale;
    mx = std::max(mx, s[t]);
  }
  const float mnew = std::max(st.m[h], mx);
  const float alpha = std::exp(st.m[h] - mnew);  // 0 when the state was empty
  float lsum = st.l[h] * alpha;
  for (int t = 0; t < n; ++t) {
    s[t] = std::exp(s[t] - mnew);
    lsum += s[t];
  }
  st.l[h] = lsum;
  st.m[h] = mnew;
  return alpha;
}

// Plain version, any block size and dtype: tokens [t0, t1) of logical block `blk_idx` of
// sequence b folded into `st` for KV head kvh.  Keys and values are widened into transposed
// fp32 tiles kt[dim][token] and vt[token][dim] first.
template <typename T>
void fold_block(const HostCtx& c, int b, int kvh, int blk_idx, int t0, int t1, const float* qf,
                State& st, std::vector<float>& kt, std::vector<float>& vt) {
  const int bs = c.L.block_size, dk = c.L.head_dim_k, dv = c.L.head_dim_v;
  constexpr int x = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  const int32_t pid = c.table[(int64_t)b * c.max_blocks + blk_idx];
  const T* blk = static_cast<const T*>(block_base(c, pid));
  const int lo = t0 - blk_idx * bs, hi = t1 - blk_idx * bs;  // token slots of the block used
  const int n = hi - lo;
  if (c.L.latent) {
    for (int ch = 0; ch < dk / x; ++ch)
      for (int t = 0; t < n; ++t)
        for (int u = 0; u < x; ++u) {
          const float v = elem(blk, ((int64_t)ch * bs + lo + t) * x + u);
          const int i = ch * x + u;
          kt[(size_t)i * bs + t] = v;
          if (i < dv) vt[(size_t)t * dv + i] = v;
        }
  } else {
    const int64_t kbase = (int64_t)kvh * (dk / x) * bs * x;
    for (int ch = 0; ch < dk / x; ++ch)
      for (int t = 0; t < n; ++t)
        for (int u = 0; u < x; ++u)
          kt[(size_t)(ch * x + u) * bs + t] = elem(blk, kbase + ((int64_t)ch * bs + lo + t) * x + u);
    const int64_t vbase = (int64_t)c.hkv * bs * dk + (int64_t)kvh * dv * bs;
    for (int j = 0; j < dv; ++j)
      for (int t = 0; t < n; ++t) vt[(size_t)t * dv + j] = elem(blk, vbase + (int64_t)j * bs + lo + t);
  }
  float s[256];
  for (int h = 0; h < c.group; ++h) {
    const float* qh = qf + (size_t)h * dk;
    for (int t = 0; t < n; ++t) s[t] = 0.f;
    for (int i = 0; i < dk; ++i) {
      const float qi = qh[i];
      const float* row = &kt[(size_t)i * bs];
      for (int t = 0; t < n; ++t) s[t] += qi * row[t];
    }
    const float alpha = softmax_update(st, h, s, n, c.scale);
    float* acc = &st.acc[(size_t)h * dv];
    for (int j = 0; j < dv; ++j) acc[j] *= alpha;
    for (int t = 0; t < n; ++t) {
      const float* vrow = &vt[(size_t)t * dv];
      for (int j = 0; j < dv; ++j) acc[j] += s[t] * vrow[j];
    }
  }
}

// 8 bf16 -> 8 fp32 (exact: the bits move to the high half of each word)
inline __m256 cvt8(const uint16_t* p) {
  const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i*>(p));
  return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
}

inline float hsum8(__m256 v) {
  __m128 x = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  x = _mm_add_ps(x, _mm_movehl_ps(x, x));
  x = _mm_add_ss(x, _mm_shuffle_ps(x, x, 1));
  return _mm_cvtss_f32(x);
}

// r[k] = sum of the 8 lanes of v[k], k = 0..7
inline __m256 hsum8x8(const __m256* v) {
  const __m256 a0 = _mm256_hadd_ps(v[0], v[1]), a1 = _mm256_hadd_ps(v[2], v[3]);
  const __m256 a2 = _mm256_hadd_ps(v[4], v[5]), a3 = _mm256_hadd_ps(v[6], v[7]);
  const __m256 b0 = _mm256_hadd_ps(a0, a1), b1 = _mm256_hadd_ps(a2, a3);
  return _mm256_add_ps(_mm256_permute2f128_ps(b0, b1, 0x20), _mm256_permute2f128_ps(b0, b1, 0x31));
}

// e^x for 8 lanes, x <= 0 finite (softmax weights relative to the running max): write
// x = n ln2 + r with n = round(x / ln2) and |r| <= ln2 / 2 (ln2 split in a high part exact in
// fp32 and a low correction, Cody and Waite's reduction), e^r by its Taylor series to degree 7
// (truncation below 6e-9 relative), and 2^n by adding n to the exponent field.  Below -87
// the result is flushed to 0.
inline __m256 exp8(__m256 x) {
  const __m256 lo_lim = _mm256_set1_ps(-87.0f);
  const __m256 under = _mm256_cmp_ps(x, lo_lim, _CMP_LT_OQ);
  x = _mm256_max_ps(x, lo_lim);
  const __m256 n = _mm256_round_ps(_mm256_mul_ps(x, _mm256_set1_ps(1.44269504088896341f)),
                                   _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
  __m256 r = _mm256_fnmadd_ps(n, _mm256_set1_ps(0.693145751953125f), x);   // ln2 high part
  r = _mm256_fnmadd_ps(n, _mm256_set1_ps(1.42860682030941723e-6f), r);      // ln2 - high part
  __m256 y = _mm256_set1_ps(1.f / 5040.f);
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(1.f / 720.f));
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(1.f / 120.f));
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(1.f / 24.f));
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(1.f / 6.f));
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(0.5f));
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(1.f));
  y = _mm256_fmadd_ps(y, r, _mm256_set1_ps(1.f));
  const __m256i e = _mm256_slli_epi32(_mm256_cvtps_epi32(n), 23);
  y = _mm256_castsi256_ps(_mm256_add_epi32(_mm256_castps_si256(y), e));
  return _mm256_andnot_ps(under, y);
}

// Online-softmax update of head h with the scores s[0..n) (n % 8 == 0) of one block: the
// 8-wide version of softmax_update.
inline float softmax_update8(State& st, int h, float* s, int n, float scale) {
  const __m256 sc = _mm256_set1_ps(scale);
  __m256 mx8 = _mm256_set1_ps(-INFINITY);
  for (int t = 0; t < n; t += 8) {
    const __m256 v = _mm256_mul_ps(_mm256_loadu_ps(s + t), sc);
    _mm256_storeu_ps(s + t, v);
    mx8 = _mm256_max_ps(mx8, v);
  }
  __m128 m4 = _mm_max_ps(_mm256_castps256_ps128(mx8), _mm256_extractf128_ps(mx8, 1));
  m4 = _mm_max_ps(m4, _mm_movehl_ps(m4, m4));
  m4 = _mm_max_ss(m4, _mm_shuffle_ps(m4, m4, 1));
  const float mnew = std::max(st.m[h], _mm_cvtss_f32(m4));
  const float alpha = std::exp(st.m[h] - mnew);  // 0 when the state was empty
  const __m256 mn = _mm256_set1_ps(mnew);
  __m256 l8 = _mm256_setzero_ps();
  for (int t = 0; t < n; t += 8) {
    const __m256 p = exp8(_mm256_sub_ps(_mm256_loadu_ps(s + t), mn));
    _mm256_storeu_ps(s + t, p);
    l8 = _mm256_add_ps(l8, p);
  }
  __m128 l4 = _mm_add_ps(_mm256_castps256_ps128(l8), _mm256_extractf128_ps(l8, 1));
  l4 = _mm_add_ps(l4, _mm_movehl_ps(l4, l4));
  l4 = _mm_add_ss(l4, _mm_shuffle_ps(l4, l4, 1));
  st.l[h] = st.l[h] * alpha + _mm_cvtss_f32(l4);
  st.m[h] = mnew;
  return alpha;
}

// AVX2 version for whole bf16 blocks with bs % 8 == 0: keys widened once into a token-major
// tile kf[token][dim] (8 dims per 16-byte chunk), scores as 8-wide dot products; GQA values
// widened into vf[dim][token] and accumulated 8 output dims at a time; MLA values are the
// leading dims of kf, read once for all heads.
void fold_block_bf16(const HostCtx& c, const uint16_t* blk, int kvh, const float* qf, State& st,
                     float* kf, float* vf, float* s) {
  const int bs = c.L.block_size, dk = c.L.head_dim_k, dv = c.L.head_dim_v, g = c.group;
  const int kc = dk / 8;
  const uint16_t* kb = c.L.latent ? blk : blk + (int64_t)kvh * dk * bs;
  for (int ch = 0; ch < kc; ++ch)
    for (int t = 0; t < bs; ++t) _mm256_storeu_ps(kf + (size_t)t * dk + ch * 8, cvt8(kb + ((size_t)ch * bs + t) * 8));
  for (int h = 0; h < g; ++h) {
    const float* qh = qf + (size_t)h * dk;
    float* sh = s + (size_t)h * bs;
    for (int t = 0; t < bs; ++t) {
      const float* kt = kf + (size_t)t * dk;
      __m256 a = _mm256_setzero_ps(), b2 = _mm256_setzero_ps();
      int ch = 0;
      for (; ch + 1 < kc; ch += 2) {
        a = _mm256_fmadd_ps(_mm256_loadu_ps(qh + ch * 8), _mm256_loadu_ps(kt + ch * 8), a);
        b2 = _mm256_fmadd_ps(_mm256_loadu_ps(qh + ch * 8 + 8), _mm256_loadu_ps(kt + ch * 8 + 8), b2);
      }
      if (ch < kc) a = _mm256_fmadd_ps(_mm256_loadu_ps(qh + ch * 8), _mm256_loadu_ps(kt + ch * 8), a);
      sh[t] = hsum8(_mm256_add_ps(a, b2));
    }
    const float alpha = softmax_update8(st, h, sh, bs, c.scale);
    float* acc = &st.acc[(size_t)h * dv];
    const __m256 al = _mm256_set1_ps(alpha);
    for (int j = 0; j < dv; j += 8) _mm256_storeu_ps(acc + j, _mm256_mul_ps(_mm256_loadu_ps(acc + j), al));
  }
  if (c.L.latent) {
    for (int t = 0; t < bs; ++t) {
      const float* vt = kf + (size_t)t * dk;
      for (int h = 0; h < g; ++h) {
        const __m256 p = _mm256_set1_ps(s[(size_t)h * bs + t]);
        float* acc = &st.acc[(size_t)h * dv];
        for (int j = 0; j < dv; j += 8)
          _mm256_storeu_ps(acc + j, _mm256_fmadd_ps(p, _mm256_loadu_ps(vt + j), _mm256_loadu_ps(acc + j)));
      }
    }
    return;
  }
  const uint16_t* vb = blk + (int64_t)c.hkv * bs * dk + (int64_t)kvh * dv * bs;
  const int tv = bs / 8;  // 8-token vectors per value row
  for (int j = 0; j < dv; ++j)
    for (int k = 0; k < tv; ++k) _mm256_storeu_ps(vf + (size_t)j * bs + k * 8, cvt8(vb + (size_t)j * bs + k * 8));
  for (int h = 0; h < g; ++h) {
    const float* sh = s + (size_t)h * bs;
    float* acc = &st.acc[(size_t)h * dv];
    for (int j = 0; j < dv; j += 8) {
      __m256 part[8];
      for (int jj = 0; jj < 8; ++jj) {
        const float* row = vf + (size_t)(j + jj) * bs;
        __m256 a = _mm256_mul_ps(_mm256_loadu_ps(sh), _mm256_loadu_ps(row));
        for (int k = 1; k < tv; ++k) a = _mm256_fmadd_ps(_mm256_loadu_ps(sh + k * 8), _mm256_loadu_ps(row + k * 8), a);
        part[jj] = a;
      }
      _mm256_storeu_ps(acc + j, _mm256_add_ps(_mm256_loadu_ps(acc + j), hsum8x8(part)));
    }
  }
}

}  // namespace
}  // namespace kvattn

using namespace kvattn;

extern "C" kvattn_status kvattn_host_partial(const kvattn_layout* layout,
                                             const kvattn_region* host_regions, int32_t n_regions,
                                             const void* q, int32_t q_dtype, int32_t batch,
                                             int32_t num_q_heads, float scale,
                                             const int32_t* table, int32_t max_blocks,
                                             const int32_t* tok_end, float* o_out, float* lse_out,
                                             int32_t n_threads) {
  clear_error();
  if (!layout || !host_regions || !q || !table || !tok_end || !o_out || !lse_out)
    return set_error(KVATTN_E_INVAL, "host_partial: null argument");
  const std::string why = layout_problem(*layout);
  if (!why.empty()) return set_error(KVATTN_E_INVAL, "host_partial: " + why);
  if (n_regions < 1 || n_regions > KVATTN_MAX_REGIONS || batch < 1 || num_q_heads < 1 || max_blocks < 1)
    return set_error(KVATTN_E_INVAL, "host_partial: bad sizes");
  if (q_dtype != layout->kv_dtype)
    return set_error(KVATTN_E_UNSUPPORTED, "host_partial: q_dtype must equal the cache dtype");
  if (num_q_heads % layout->num_kv_heads != 0 || num_q_heads / layout->num_kv_heads > kMaxGroup)
    return set_error(KVATTN_E_UNSUPPORTED, "host_partial: heads per KV head must divide and be <= 16");
  if (layout->block_size > 256 || !std::isfinite(scale))
    return set_error(KVATTN_E_INVAL, "host_partial: block size above 256 or non-finite scale");
  HostCtx c{};
  c.L = *layout;
  c.block_elems = kvattn_block_bytes(layout) / (layout->kv_dtype == KVATTN_F32 ? 4 : 2);
  c.n_regions = n_regions;
  int64_t total = 0;
  for (int r = 0; r < n_regions; ++r) {
    if (!host_regions[r].base || host_regions[r].num_blocks < 0)
      return set_error(KVATTN_E_INVAL, "host_partial: bad region");
    c.base[r] = host_regions[r].base;
    c.first[r] = total;
    total += host_regions[r].num_blocks;
  }
  c.first[n_regions] = total;
  c.q = q;
  c.q_f32 = q_dtype == KVATTN_F32;
  c.batch = batch;
  c.hq = num_q_heads;
  c.hkv = layout->latent ? 1 : layout->num_kv_heads;
  c.group = num_q_heads / c.hkv;
  c.scale = scale;
  c.table = table;
  c.max_blocks = max_blocks;
  c.tok_end = tok_end;
  const int bs = layout->block_size;
  // validate every table entry that will be read
  for (int b = 0; b < batch; ++b) {
    if (tok_end[b] < 0 || (int64_t)tok_end[b] > (int64_t)max_blocks * bs)
      return set_error(KVATTN_E_INVAL, "host_partial: tok_end outside [0, max_blocks * block_size]");
    for (int i = 0; i < (tok_end[b] + bs - 1) / bs; ++i) {
      const int32_t pid = table[(int64_t)b * max_blocks + i];
      if (pid < 0 || pid >= total)
        return set_error(KVATTN_E_RANGE, "host_partial: block id out of range in sequence " +
                                             std::to_string(b));
    }
  }

  // work items: (b, kvh, chunk of whole blocks)
  const int chunk_blocks = std::max(1, kChunkTokens / bs);
  std::vector<int> item_b, item_h, item_c;
  std::vector<int> first_item((size_t)batch * c.hkv + 1, 0);
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < c.hkv; ++h) {
      first_item[(size_t)b * c.hkv + h] = (int)item_b.size();
      const int nblk = (tok_end[b] + bs - 1) / bs;
      for (int k = 0; k * chunk_blocks < nblk; ++k) {
        item_b.push_back(b);
        item_h.push_back(h);
        item_c.push_back(k);
      }
    }
  first_item[(size_t)batch * c.hkv] = (int)item_b.size();
  const int nitems = (int)item_b.size();
  const int dk = layout->head_dim_k, dv = layout->head_dim_v, g = c.group;
  WorkerPool& wp = WorkerPool::get();
  std::lock_guard<std::mutex> call_lock(wp.call_mu);
  if (wp.ws_o.size() < (size_t)nitems * g * dv) wp.ws_o.resize((size_t)nitems * g * dv);
  if (wp.ws_m.size() < (size_t)nitems * g) {
    wp.ws_m.resize((size_t)nitems * g);
    wp.ws_l.resize((size_t)nitems * g);
  }
  float* part_o = wp.ws_o.data();
  float* part_m = wp.ws_m.data();
  float* part_l = wp.ws_l.data();

  std::atomic<int> next{0};
  const bool fast = layout->kv_dtype == KVATTN_BF16 && bs % 8 == 0;
  const std::function<void(int)> worker = [&](int) {
    std::vector<float> kt((size_t)dk * bs), vt((size_t)bs * dv), qf((size_t)g * dk);
    std::vector<float> sbuf((size_t)g * bs);
    State st;
    st.acc.resize((size_t)g * dv);
    for (int it = next.fetch_add(1); it < nitems; it = next.fetch_add(1)) {
      const int b = item_b[it], h = item_h[it], k = item_c[it];
      for (int hh = 0; hh < g; ++hh)
        for (int i = 0; i < dk; ++i) {
          const int64_t e = ((int64_t)b * c.hq + h * g + hh) * dk + i;
          qf[(size_t)hh * dk + i] = c.q_f32 ? static_cast<const float*>(q)[e]
                                            : bf16_f(static_cast<const uint16_t*>(q)[e]);
        }
      for (int hh = 0; hh < g; ++hh) {
        st.m[hh] = -INFINITY;
        st.l[hh] = 0.f;
      }
      std::fill(st.acc.begin(), st.acc.end(), 0.f);
      const int t_lo = k * chunk_blocks * bs;
      const int t_hi = std::min(tok_end[b], t_lo + chunk_blocks * bs);
      for (int t = t_lo; t < t_hi; t += bs) {
        const int t_end = std::min(t_hi, t + bs);
        if (fast && t_end - t == bs) {  // a whole block
          const int32_t pid = table[(int64_t)b * max_blocks + t / bs];
          fold_block_bf16(c, static_cast<const uint16_t*>(block_base(c, pid)), h, qf.data(), st,
                          kt.data(), vt.data(), sbuf.data());
        } else if (layout->kv_dtype == KVATTN_F32) {
          fold_block<float>(c, b, h, t / bs, t, t_end, qf.data(), st, kt, vt);
        } else {
          fold_block<uint16_t>(c, b, h, t / bs, t, t_end, qf.data(), st, kt, vt);
        }
      }
      for (int hh = 0; hh < g; ++hh) {
        part_m[(size_t)it * g + hh] = st.m[hh];
        part_l[(size_t)it * g + hh] = st.l[hh];
        std::memcpy(&part_o[((size_t)it * g + hh) * dv], &st.acc[(size_t)hh * dv], sizeof(float) * dv);
      }
    }
  };
  int want = n_threads;
  if (want <= 0) {
    cpu_set_t set;
    want = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : 1;
    want = std::min(want, 64);
  }
  const int nt = std::max(1, std::min({want, nitems, 255}));
  wp.run(nt, worker);

  // exact merge of each (sequence, head)'s chunk partials, in chunk order
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < c.hkv; ++h)
      for (int hh = 0; hh < g; ++hh) {
        const int qh = h * g + hh;
        float* o = o_out + ((int64_t)b * c.hq + qh) * dv;
        const int i0 = first_item[(size_t)b * c.hkv + h], i1 = first_item[(size_t)b * c.hkv + h + 1];
        float M = -INFINITY;
        for (int it = i0; it < i1; ++it) M = std::max(M, part_m[(size_t)it * g + hh]);
        std::fill(o, o + dv, 0.f);
        if (M == -INFINITY) {
          lse_out[(int64_t)b * c.hq + qh] = -INFINITY;
          continue;
        }
        double tot = 0.0;
        for (int it = i0; it < i1; ++it) {
          const float w = std::exp(part_m[(size_t)it * g + hh] - M);  // unnormalised weights
          tot += (double)w * part_l[(size_t)it * g + hh];
          const float* po = &part_o[((size_t)it * g + hh) * dv];
          for (int j = 0; j < dv; ++j) o[j] += w * po[j];
        }
        const float inv = (float)(1.0 / tot);
        for (int j = 0; j < dv; ++j) o[j] *= inv;
        lse_out[(int64_t)b * c.hq + qh] = M + (float)std::log(tot);
      }
  return KVATTN_OK;
}
