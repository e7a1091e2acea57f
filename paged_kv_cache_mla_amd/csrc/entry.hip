// C-ABI entry points of the device path: argument validation, kernel choice, launch.

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <string>

#include "device_common.h"
#include "launch_common.h"
#include "pool_internal.h"

namespace kvattn {

hipError_t launch_gqa_mfma(const DecodeArgs& a, int d, bool stream, dim3 grid, hipStream_t st);
int gqa_mfma_max_group(int d);
size_t gqa_mfma_lds_bytes(int group_parts, int group, int d);
hipError_t launch_gqa_generic(const DecodeArgs& a, int d, bool f32, dim3 grid, hipStream_t st);
hipError_t launch_gqa_plan(const DecodeArgs& a, int d, const int32_t* plan, int32_t n_groups,
                           uint32_t* work, int cus, hipStream_t st);
hipError_t launch_mla(const DecodeArgs& a, dim3 grid, hipStream_t st);
hipError_t launch_gqa_probe(const DecodeArgs& a, int d, bool stream, dim3 grid, uint32_t* xsum,
                            hipStream_t st);
hipError_t launch_mla_probe(const DecodeArgs& a, dim3 grid, uint32_t* xsum, hipStream_t st);

hipError_t launch_merge(const MergeArgs& a, hipStream_t st);
hipError_t launch_append(const RegionTable& rt, const kvattn_layout& L, const void* k_new,
                         const void* v_new, const int32_t* table, const int32_t* pos,
                         int32_t* err, int32_t batch, int32_t n_new, int32_t max_blocks,
                         int bs_shift, hipStream_t st);

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// Tuning override of the partitions per wave of the matrix-core kernel (1 or 2; 0 = auto).
static int wave_parts_override() {
  const char* e = std::getenv("KVATTN_WAVE_PARTS");
  if (!e) return 0;
  const int v = std::atoi(e);
  return (v == 1 || v == 2) ? v : 0;
}

static bool force_generic() {
  const char* e = std::getenv("KVATTN_FORCE_GENERIC");
  return e && e[0] == '1';
}

static kvattn_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return KVATTN_OK;
  return set_error(KVATTN_E_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

enum Kind { K_MFMA, K_GENERIC, K_MLA };

// Compute units of the current device (cached per device); 0 if there is no device.
static int current_device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The kernel for a layout and head count, before any group_parts is known; E_UNSUPPORTED
// (with the message set) if there is none.
static kvattn_status choose_kind(const char* what, const kvattn_layout& L, int32_t batch,
                                 int32_t num_q_heads, const int32_t* part_tokens, Kind* out) {
  const int hkv = L.num_kv_heads;
  const int group = num_q_heads / hkv;
  const int bs = L.block_size;
  if (L.latent) {
    if (L.kv_dtype != KVATTN_BF16 || L.head_dim_k != 576 || L.head_dim_v != 512 || bs != 64 ||
        num_q_heads > 16)
      return set_error(KVATTN_E_UNSUPPORTED,
                       std::string(what) + ": latent caches need bf16, Dk 576, Dv 512, block 64, <= 16 heads");
    *out = K_MLA;
    return KVATTN_OK;
  }
  const int d = L.head_dim_k;
  if (L.head_dim_v != d || (d != 64 && d != 128 && d != 256))
    return set_error(KVATTN_E_UNSUPPORTED, std::string(what) + ": GQA needs Dk == Dv in {64, 128, 256}");
  if (group > 16)
    return set_error(KVATTN_E_UNSUPPORTED, std::string(what) + ": at most 16 query heads per KV head");
  Kind kind = (L.kv_dtype == KVATTN_BF16 && bs >= 16 && !force_generic()) ? K_MFMA : K_GENERIC;
  // the matrix-core kernel keeps a wave's block ids in two 64-lane registers
  for (int b = 0; b < batch && kind == K_MFMA; ++b)
    if (part_tokens[b] > 0 && part_tokens[b] / bs + 1 > 128) kind = K_GENERIC;
  *out = kind;
  return KVATTN_OK;
}

// Partitions per wave of the matrix-core kernel for a group size: two when the group splits
// evenly, so that a long batch needs half the waves (at its register use a CU holds 8 waves of
// head dim 128 or 256, and a second round of waves restarts the load pipeline), unless two
// partitions would overflow the wave's 128-entry window of block ids.
static int mfma_wave_parts(int group_parts, int32_t batch, const int32_t* part_tokens, int bs) {
  int wave_parts = wave_parts_override();
  if (wave_parts == 0) wave_parts = (group_parts >= 4 && group_parts % 2 == 0) ? 2 : 1;
  if (group_parts % wave_parts != 0) wave_parts = 1;
  for (int b = 0; b < batch; ++b)
    if (part_tokens[b] > 0 && (int64_t)wave_parts * part_tokens[b] / bs + 1 > 128) wave_parts = 1;
  return wave_parts;
}

// Whether a group of group_parts partitions fits the matrix-core kernel: its waves on one CU
// and their LDS merge area within 64 KiB.
static bool mfma_group_fits(int group_parts, int wave_parts, int group, int d) {
  const int waves = group_parts / wave_parts;
  if (waves <= 1) return true;
  return waves <= gqa_mfma_max_group(d) && gqa_mfma_lds_bytes(waves, group, d) <= 65536;
}

// Work items (workgroups) of a launch at group size g: (sequences x KV heads) x partials.
static int64_t launch_items(Kind kind, int hkv, int32_t batch, const int32_t* ctx_lens,
                            const int32_t* tok_begin, const int32_t* part_tokens, int g) {
  int64_t w = 0;
  for (int b = 0; b < batch; ++b) {
    const int np = kvattn_partition_count(ctx_lens[b], tok_begin ? tok_begin[b] : 0, part_tokens[b]);
    w += np > 0 ? (np + g - 1) / g : 0;
  }
  return w * (kind == K_MLA ? 1 : hkv);
}

// group_parts = 0: the library's choice, a rule fitted to sweeps on MI355X (decode_partial
// plus merge, several batch x context shapes; cus = compute units).  W(g) is the launch's
// work items at group size g.
//  - latent (MLA) kernel, one workgroup of eight waves per CU: the largest g in {16, 8, 4, 2}
//    with W(g) >= cus, else 1: enough groups to cover the CUs, as few partials as that allows.
//  - matrix-core GQA kernel: 1 while W(1) < 8 cus (small launches want one-wave groups, as many
//    as there are); otherwise the largest g in {16, 8, 4, 2} that fits the kernel with W(g) a
//    positive multiple of cus (every round of workgroups fills the chip), else the largest
//    with W(g) >= cus.  A pool holding shared blocks (cache-retaining loads, sequences sharing a
//    prefix) is fastest at g <= 2.
//  - VALU kernel (fp32 caches, small blocks): 2 once W(1) >= 4 cus, else 1.
static int auto_group_parts(Kind kind, const kvattn_pool* pool, int32_t batch, int32_t num_q_heads,
                            const int32_t* ctx_lens, const int32_t* tok_begin,
                            const int32_t* part_tokens, int cus) {
  const kvattn_layout& L = pool->layout;
  const int hkv = L.num_kv_heads;
  const int group = num_q_heads / hkv;
  if (cus <= 0) cus = 256;
  auto W = [&](int g) { return launch_items(kind, hkv, batch, ctx_lens, tok_begin, part_tokens, g); };
  static const int cand[4] = {16, 8, 4, 2};
  if (kind == K_MLA) {
    for (int g : cand)
      if (W(g) >= cus) return g;
    return 1;
  }
  if (kind == K_GENERIC) return W(1) >= 4 * (int64_t)cus ? 2 : 1;
  if (W(1) < 8 * (int64_t)cus) return 1;
  const int cap = pool->shared_blocks > 0 ? 2 : 16;
  auto fits = [&](int g) {
    return g <= cap &&
           mfma_group_fits(g, mfma_wave_parts(g, batch, part_tokens, L.block_size), group, L.head_dim_k);
  };
  for (int g : cand)
    if (fits(g) && W(g) >= cus && W(g) % cus == 0) return g;
  for (int g : cand)
    if (fits(g) && W(g) >= cus) return g;
  return 1;
}

// Validation, kernel choice and kernel arguments shared by kvattn_decode_partial and
// kvattn_gather_probe (which checks its own pointers and passes no q or partials).
// group_parts = 0 is replaced by the library's choice for the current device.
static kvattn_status decode_prepare(const char* what, const kvattn_pool* pool, int32_t q_dtype,
                                    int32_t batch, int32_t num_q_heads, float scale,
                                    const int32_t* table_dev, int32_t max_blocks,
                                    const int32_t* ctx_lens, const int32_t* tok_begin,
                                    const int32_t* part_tokens, const int32_t* seq_dev,
                                    int32_t max_parts, int32_t group_parts, DecodeArgs* out,
                                    Kind* kind_out, dim3* grid_out) {
  if (!pool || !table_dev || !ctx_lens || !part_tokens || !seq_dev)
    return set_error(KVATTN_E_INVAL, std::string(what) + ": null argument");
  if (batch < 1 || num_q_heads < 1 || max_blocks < 1 || max_parts < 1)
    return set_error(KVATTN_E_INVAL,
                     std::string(what) + ": batch, heads, max_blocks and max_parts must be >= 1");
  if (group_parts < 0 || group_parts > KVATTN_MAX_GROUP_PARTS)
    return set_error(KVATTN_E_INVAL,
                     std::string(what) + ": group_parts must be in [0, KVATTN_MAX_GROUP_PARTS]");
  if (!std::isfinite(scale)) return set_error(KVATTN_E_INVAL,
                                              std::string(what) + ": scale must be finite");
  const kvattn_layout& L = pool->layout;
  if (q_dtype != L.kv_dtype)
    return set_error(KVATTN_E_UNSUPPORTED,
                     std::string(what) + ": q_dtype must equal the cache dtype");
  const int hkv = L.num_kv_heads;
  if (num_q_heads % hkv != 0)
    return set_error(KVATTN_E_INVAL,
                     std::string(what) + ": num_q_heads must be a multiple of num_kv_heads");
  const int group = num_q_heads / hkv;
  const int bs = L.block_size;
  for (int b = 0; b < batch; ++b)
    if (part_tokens[b] <= 0 || part_tokens[b] % bs != 0)
      return set_error(KVATTN_E_INVAL,
                       std::string(what) + ": part_tokens must be a positive multiple of block_size");

  // kernel choice
  Kind kind;
  const kvattn_status ks = choose_kind(what, L, batch, num_q_heads, part_tokens, &kind);
  if (ks != KVATTN_OK) return ks;
  if (group_parts == 0) {
    for (int b = 0; b < batch; ++b) {
      const int beg = tok_begin ? tok_begin[b] : 0;
      if (beg < 0 || beg > ctx_lens[b])
        return set_error(KVATTN_E_INVAL, std::string(what) + ": sequence " + std::to_string(b) +
                                             " needs 0 <= tok_begin <= ctx_len");
    }
    group_parts = auto_group_parts(kind, pool, batch, num_q_heads, ctx_lens, tok_begin,
                                   part_tokens, current_device_cus());
  }
  int wave_parts = 1;
  if (kind == K_MFMA) {
    wave_parts = mfma_wave_parts(group_parts, batch, part_tokens, bs);
    if (!mfma_group_fits(group_parts, wave_parts, group, L.head_dim_k)) {
      // waves of a group merge their partials in LDS
      const int d = L.head_dim_k;
      if (group_parts / wave_parts > gqa_mfma_max_group(d))
        return set_error(KVATTN_E_UNSUPPORTED, std::string(what) + ": group_parts above " +
                                                   std::to_string(gqa_mfma_max_group(d)) +
                                                   " for head dim " + std::to_string(d));
      return set_error(KVATTN_E_UNSUPPORTED,
                       std::string(what) + ": group_parts x heads per KV head x (head dim + 1) x 4 "
                       "bytes exceeds 64 KiB");
    }
  }

  // per-sequence checks and grid size
  int max_ng = 0;  // most partials any sequence writes
  for (int b = 0; b < batch; ++b) {
    const int len = ctx_lens[b];
    const int beg = tok_begin ? tok_begin[b] : 0;
    const int P = part_tokens[b];
    if (beg < 0 || beg > len || (int64_t)len > (int64_t)max_blocks * bs)
      return set_error(KVATTN_E_INVAL, std::string(what) + ": sequence " + std::to_string(b) +
                                           " needs 0 <= tok_begin <= ctx_len <= max_blocks * block_size");
    if (P <= 0 || P % bs != 0)
      return set_error(KVATTN_E_INVAL,
                       std::string(what) + ": part_tokens must be a positive multiple of block_size");
    const int np = kvattn_partition_count(len, beg, P);
    const int ng = (np + group_parts - 1) / group_parts;
    if (ng > max_parts)
      return set_error(KVATTN_E_INVAL, std::string(what) + ": sequence " + std::to_string(b) +
                                           " writes more partials than max_parts");
    if (ng > max_ng) max_ng = ng;
  }
  if (max_ng > 0 && pool->total_blocks == 0)
    return set_error(KVATTN_E_INVAL, std::string(what) + ": the pool holds no blocks");
  const int grid_ng = max_ng > 0 ? max_ng : 1;
  const int64_t items = (int64_t)batch * (kind == K_MLA ? 1 : hkv) * grid_ng;
  if (items > INT32_MAX) return set_error(KVATTN_E_INVAL, std::string(what) + ": launch too large");

  DecodeArgs& a = *out;
  a = DecodeArgs{};
  a.rt = region_table(pool);
  a.table = table_dev;
  a.seq = seq_dev;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = hkv;
  a.group = group;
  a.max_blocks = max_blocks;
  a.max_parts = max_parts;
  a.grid_ng = grid_ng;
  a.group_parts = group_parts;
  a.wave_parts = wave_parts;
  a.bs = bs;
  a.bs_shift = log2_exact(bs);
  a.scale = scale;
  a.scale_log2 = scale * 1.44269504088896340736f;
  *kind_out = kind;
  *grid_out = dim3((unsigned)items);
  return KVATTN_OK;
}

// Work counters of kvattn_decode_partial_plan_noalloc: a file-scope device array, one copy on
// every GPU the library runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up once per device
// (scratch_on_current_device) and only that address is passed to kernels.  The plan kernel
// uses two words; every launch that completes leaves them zero, as the module load does.
constexpr int kScratchWords = 64;  // 256 bytes per GPU
constexpr int kPlanWorkWords = 2;  // what any call needs, whatever its sizes
static_assert(kPlanWorkWords <= kScratchWords, "the plan kernel's counters fit the scratch array");
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static uint32_t* g_scratch_ptr[kMaxDevices];  // device address per device, once looked up

static kvattn_status scratch_on_current_device(uint32_t** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return set_error(KVATTN_E_HIP, std::string("scratch: hipGetDevice: ") + hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(KVATTN_E_UNSUPPORTED, "scratch: device index beyond " + std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(KVATTN_E_HIP, std::string("scratch: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return KVATTN_OK;
}

}  // namespace kvattn

using namespace kvattn;

extern "C" {

kvattn_status kvattn_decode_partial(const kvattn_pool* pool, const void* q, int32_t q_dtype,
                                    int32_t batch, int32_t num_q_heads, float scale,
                                    const int32_t* table_dev, int32_t max_blocks,
                                    const int32_t* ctx_lens, const int32_t* tok_begin,
                                    const int32_t* part_tokens, const int32_t* seq_dev,
                                    int32_t max_parts, int32_t group_parts, float* o_part,
                                    float* lse_part, int32_t* nparts_dev, int32_t* err_dev,
                                    void* hip_stream) {
  clear_error();
  if (!pool || !q || !table_dev || !ctx_lens || !part_tokens || !seq_dev || !o_part ||
      !lse_part || !nparts_dev)
    return set_error(KVATTN_E_INVAL, "decode_partial: null argument");
  if (!aligned16(q) || !aligned16(o_part))
    return set_error(KVATTN_E_INVAL, "decode_partial: q and o_part must be 16-byte aligned");
  DecodeArgs a;
  Kind kind;
  dim3 grid;
  const kvattn_status v =
      decode_prepare("decode_partial", pool, q_dtype, batch, num_q_heads, scale, table_dev,
                     max_blocks, ctx_lens, tok_begin, part_tokens, seq_dev, max_parts,
                     group_parts, &a, &kind, &grid);
  if (v != KVATTN_OK) return v;
  a.q = q;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.nparts = nparts_dev;
  a.err = err_dev;
  const kvattn_layout& L = pool->layout;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  switch (kind) {
    case K_MLA: e = launch_mla(a, grid, st); break;
    case K_MFMA: e = launch_gqa_mfma(a, L.head_dim_k, pool->shared_blocks == 0, grid, st); break;
    default: e = launch_gqa_generic(a, L.head_dim_k, L.kv_dtype == KVATTN_F32, grid, st); break;
  }
  return hip_status(e, "decode_partial launch");
}

int32_t kvattn_choose_group_parts(const kvattn_pool* pool, int32_t batch, int32_t num_q_heads,
                                  const int32_t* ctx_lens, const int32_t* tok_begin,
                                  const int32_t* part_tokens, int32_t num_cus) {
  clear_error();
  if (!pool || !ctx_lens || !part_tokens)
    return set_error(KVATTN_E_INVAL, "choose_group_parts: null argument");
  if (batch < 1 || num_q_heads < 1 || num_q_heads % pool->layout.num_kv_heads != 0)
    return set_error(KVATTN_E_INVAL, "choose_group_parts: bad batch or head count");
  for (int b = 0; b < batch; ++b) {
    const int beg = tok_begin ? tok_begin[b] : 0;
    if (kvattn_partition_count(ctx_lens[b], beg, part_tokens[b]) < 0 ||
        part_tokens[b] % pool->layout.block_size != 0)
      return set_error(KVATTN_E_INVAL, "choose_group_parts: sequence " + std::to_string(b) +
                                           " has invalid partition arguments");
  }
  Kind kind;
  const kvattn_status ks =
      choose_kind("choose_group_parts", pool->layout, batch, num_q_heads, part_tokens, &kind);
  if (ks != KVATTN_OK) return ks;
  return auto_group_parts(kind, pool, batch, num_q_heads, ctx_lens, tok_begin, part_tokens,
                          num_cus > 0 ? num_cus : current_device_cus());
}

kvattn_status kvattn_gather_probe(const kvattn_pool* pool, int32_t batch, int32_t num_q_heads,
                                  const int32_t* table_dev, int32_t max_blocks,
                                  const int32_t* ctx_lens, const int32_t* tok_begin,
                                  const int32_t* part_tokens, const int32_t* seq_dev,
                                  int32_t group_parts, uint32_t* xsum_dev, int32_t* err_dev,
                                  void* hip_stream) {
  clear_error();
  if (!pool || !xsum_dev) return set_error(KVATTN_E_INVAL, "gather_probe: null argument");
  DecodeArgs a;
  Kind kind;
  dim3 grid;
  const kvattn_status v =
      decode_prepare("gather_probe", pool, pool->layout.kv_dtype, batch, num_q_heads, 1.f,
                     table_dev, max_blocks, ctx_lens, tok_begin, part_tokens, seq_dev,
                     INT32_MAX, group_parts, &a, &kind, &grid);
  if (v != KVATTN_OK) return v;
  a.err = err_dev;
  const kvattn_layout& L = pool->layout;
  if (kind == K_GENERIC || (kind == K_MFMA && L.block_size != 16))
    return set_error(KVATTN_E_UNSUPPORTED,
                     "gather_probe: needs the matrix-core GQA kernel with block size 16, or MLA");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = kind == K_MLA ? launch_mla_probe(a, grid, xsum_dev, st)
                                     : launch_gqa_probe(a, L.head_dim_k, pool->shared_blocks == 0,
                                                        grid, xsum_dev, st);
  return hip_status(e, "gather_probe launch");
}

kvattn_status kvattn_decode_partial_plan(const kvattn_pool* pool, const void* q, int32_t q_dtype,
                                         int32_t batch, int32_t num_q_heads, float scale,
                                         const int32_t* table_dev, int32_t max_blocks,
                                         const int32_t* plan_dev, int32_t n_groups,
                                         uint32_t* work_dev, int32_t max_parts, float* o_part,
                                         float* lse_part, int32_t* nparts_dev, int32_t* err_dev,
                                         void* hip_stream) {
  clear_error();
  if (!pool || !q || !table_dev || !plan_dev || !o_part || !lse_part || !nparts_dev)
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: null argument");
  if (!aligned16(q) || !aligned16(o_part))
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: q and o_part must be 16-byte aligned");
  if (batch < 1 || num_q_heads < 1 || max_blocks < 1 || max_parts < 1 || n_groups < 0)
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: bad sizes");
  if (!std::isfinite(scale)) return set_error(KVATTN_E_INVAL, "decode_partial_plan: scale must be finite");
  const kvattn_layout& L = pool->layout;
  if (q_dtype != L.kv_dtype)
    return set_error(KVATTN_E_UNSUPPORTED, "decode_partial_plan: q_dtype must equal the cache dtype");
  if (num_q_heads % L.num_kv_heads != 0)
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: num_q_heads must be a multiple of num_kv_heads");
  const int group = num_q_heads / L.num_kv_heads;
  const int d = L.head_dim_k;
  if (L.latent || L.kv_dtype != KVATTN_BF16 || L.block_size < 16 || L.head_dim_v != d ||
      (d != 64 && d != 128 && d != 256) || group > 16)
    return set_error(KVATTN_E_UNSUPPORTED,
                     "decode_partial_plan: needs a bf16 per-head cache with block size >= 16, head "
                     "dim 64, 128 or 256 and at most 16 query heads per KV head");
  if (n_groups > 0 && pool->total_blocks == 0)
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: the pool holds no blocks");
  if ((int64_t)n_groups * L.num_kv_heads > INT32_MAX)  // one workgroup per (group, KV head)
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: n_groups x num_kv_heads above 2^31 - 1");
  DecodeArgs a{};
  a.rt = region_table(pool);
  a.q = q;
  a.table = table_dev;
  a.seq = nullptr;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.nparts = nparts_dev;
  a.err = err_dev;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = L.num_kv_heads;
  a.group = group;
  a.max_blocks = max_blocks;
  a.max_parts = max_parts;
  a.grid_ng = 1;
  a.group_parts = 1;
  a.wave_parts = 1;
  a.bs = L.block_size;
  a.bs_shift = log2_exact(L.block_size);
  a.scale = scale;
  a.scale_log2 = scale * 1.44269504088896340736f;
  if (work_dev && (reinterpret_cast<uintptr_t>(work_dev) & 7u) != 0)
    return set_error(KVATTN_E_INVAL, "decode_partial_plan: work_dev must be 8-byte aligned");
  return hip_status(launch_gqa_plan(a, d, plan_dev, n_groups, work_dev, current_device_cus(),
                                    static_cast<hipStream_t>(hip_stream)),
                    "decode_partial_plan launch");
}

kvattn_status kvattn_decode_partial_plan_noalloc(const kvattn_pool* pool, const void* q,
                                                 int32_t q_dtype, int32_t batch,
                                                 int32_t num_q_heads, float scale,
                                                 const int32_t* table_dev, int32_t max_blocks,
                                                 const int32_t* plan_dev, int32_t n_groups,
                                                 int32_t max_parts, float* o_part,
                                                 float* lse_part, int32_t* nparts_dev,
                                                 int32_t* err_dev, void* hip_stream) {
  clear_error();
  uint32_t* work = nullptr;
  const kvattn_status s = scratch_on_current_device(&work);
  if (s != KVATTN_OK) return s;
  return kvattn_decode_partial_plan(pool, q, q_dtype, batch, num_q_heads, scale, table_dev,
                                    max_blocks, plan_dev, n_groups, work, max_parts, o_part,
                                    lse_part, nparts_dev, err_dev, hip_stream);
}

kvattn_status kvattn_merge_lse(const float* o_part, const float* lse_part,
                               const int32_t* nparts_dev, int32_t batch, int32_t num_q_heads,
                               int32_t max_parts, int32_t dv, const float* o_ext,
                               const float* lse_ext, float* o_out, float* lse_out,
                               void* hip_stream) {
  clear_error();
  if (!o_part || !lse_part || !nparts_dev || !o_out)
    return set_error(KVATTN_E_INVAL, "merge_lse: null argument");
  if ((o_ext == nullptr) != (lse_ext == nullptr))
    return set_error(KVATTN_E_INVAL, "merge_lse: o_ext and lse_ext must both be given or both NULL");
  if (batch < 1 || num_q_heads < 1 || max_parts < 1)
    return set_error(KVATTN_E_INVAL, "merge_lse: batch, heads and max_parts must be >= 1");
  if (dv < 1 || dv > 1024 || dv % 4 != 0)
    return set_error(KVATTN_E_UNSUPPORTED, "merge_lse: dv must be a multiple of 4 in [4, 1024]");
  if (!aligned16(o_part) || !aligned16(o_out) || (o_ext && !aligned16(o_ext)))
    return set_error(KVATTN_E_INVAL, "merge_lse: o_part, o_ext and o_out must be 16-byte aligned");
  MergeArgs a{o_part, lse_part, nparts_dev, o_ext, lse_ext, o_out, lse_out,
              batch, num_q_heads, max_parts, dv};
  return hip_status(launch_merge(a, static_cast<hipStream_t>(hip_stream)), "merge_lse launch");
}

}  // extern "C"

namespace kvattn {

__global__ void resolve_offsets_kernel(RegionTable rt, const int32_t* table, int32_t batch,
                                       int32_t max_blocks, const int32_t* ctx_lens,
                                       int32_t max_tokens, int32_t bs_shift, int32_t* region_out,
                                       int64_t* offset_out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)batch * max_tokens) return;
  const int b = (int)(gid / max_tokens);
  const int t = (int)(gid - (int64_t)b * max_tokens);
  int32_t r_out = -1;
  int64_t off = -1;
  if (t < ctx_lens[b] && (t >> bs_shift) < max_blocks) {
    const int32_t pid = table[(int64_t)b * max_blocks + (t >> bs_shift)];
    if (valid_block(rt, pid)) {
      const int r = region_of(rt, pid);
      r_out = r;
      // same address arithmetic as the decode kernels: block start + 16 bytes per token slot
      off = (block_ptr(rt, pid) - rt.base[r]) + ((int64_t)(t & ((1 << bs_shift) - 1)) << 4);
    }
  }
  region_out[gid] = r_out;
  offset_out[gid] = off;
}

}  // namespace kvattn

extern "C" kvattn_status kvattn_resolve_offsets(const kvattn_pool* pool, const int32_t* table_dev,
                                                int32_t batch, int32_t max_blocks,
                                                const int32_t* ctx_lens_dev, int32_t max_tokens,
                                                int32_t* region_out, int64_t* offset_out,
                                                void* hip_stream) {
  clear_error();
  if (!pool || !table_dev || !ctx_lens_dev || !region_out || !offset_out)
    return set_error(KVATTN_E_INVAL, "resolve_offsets: null argument");
  if (batch < 1 || max_blocks < 1 || max_tokens < 1 ||
      (int64_t)max_tokens > (int64_t)max_blocks * pool->layout.block_size)
    return set_error(KVATTN_E_INVAL, "resolve_offsets: bad sizes");
  const int64_t n = (int64_t)batch * max_tokens;
  const RegionTable rt = region_table(pool);
  hipLaunchKernelGGL(resolve_offsets_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), rt, table_dev, batch, max_blocks,
                     ctx_lens_dev, max_tokens, log2_exact(pool->layout.block_size), region_out,
                     offset_out);
  return hip_status(hipGetLastError(), "resolve_offsets launch");
}

extern "C" kvattn_status kvattn_append_kv(const kvattn_pool* pool, const void* k_new,
                                          const void* v_new, int32_t kv_dtype, int32_t batch,
                                          int32_t n_new, const int32_t* table_dev,
                                          int32_t max_blocks, const int32_t* pos_dev,
                                          int32_t* err_dev, void* hip_stream) {
  using namespace kvattn;
  clear_error();
  if (!pool || !k_new || !table_dev || !pos_dev)
    return set_error(KVATTN_E_INVAL, "append_kv: null argument");
  const kvattn_layout& L = pool->layout;
  if (L.latent ? v_new != nullptr : v_new == nullptr)
    return set_error(KVATTN_E_INVAL, "append_kv: v_new must be NULL exactly for a latent cache");
  if (batch < 1 || n_new < 1 || max_blocks < 1 || (int64_t)batch * n_new > 0x7fffffff)
    return set_error(KVATTN_E_INVAL, "append_kv: bad sizes");
  if (kv_dtype != L.kv_dtype)
    return set_error(KVATTN_E_UNSUPPORTED, "append_kv: kv_dtype must equal the cache dtype");
  const uintptr_t esize = L.kv_dtype == KVATTN_F32 ? 4 : 2;
  if (!aligned16(k_new) || (v_new && (reinterpret_cast<uintptr_t>(v_new) % esize) != 0))
    return set_error(KVATTN_E_INVAL, "append_kv: k_new must be 16-byte aligned, v_new element-aligned");
  return hip_status(launch_append(region_table(pool), L, k_new, v_new, table_dev, pos_dev, err_dev,
                                  batch, n_new, max_blocks, log2_exact(L.block_size),
                                  static_cast<hipStream_t>(hip_stream)),
                    "append_kv launch");
}
