// Paged KV append: write the key/value entries of new tokens into their blocks through a
// block table ([InplaceKVCache] §4.1: the block is the unit of write-time placement; §4.2:
// new decode entries are first written into the GPU's staging window, from which they take
// part in attention at once).
//
// One workgroup per (sequence, new token).  Its threads copy the K part as 16-byte chunks
// (the block stores K chunk-major, so each chunk of one token is one aligned 16-byte slot)
// and the V part element by element (V is stored token-fastest, so one token's values are
// scattered with a stride of the block size).  A token of a latent (MLA) cache is one row of
// 16-byte chunks.  The volume is tiny (one token is 2 KiB for 4 KV heads of 128 bf16
// dimensions); the kernel is bound by launch and store latency.

#include "device_common.h"
#include "launch_common.h"

namespace kvattn {

struct AppendArgs {
  RegionTable rt;
  const char* k_new;     // [B][n_new][Hkv][Dk] (latent: [B][n_new][Dk])
  const char* v_new;     // [B][n_new][Hkv][Dv] or null (latent)
  const int32_t* table;  // [B][max_blocks]
  const int32_t* pos;    // [B]: logical index of each sequence's first new token
  int32_t* err;
  int32_t batch, n_new, max_blocks;
  int32_t hkv, dk, dv, bs, bs_shift, esize, latent;
};

constexpr int kAppendThreads = 256;
constexpr int kKPer = 4;  // K chunks per thread held in registers (heads * Dk / x <= 1024)
constexpr int kVPer = 8;  // V elements per thread held in registers (Hkv * Dv <= 2048)

__global__ void __launch_bounds__(kAppendThreads) append_kernel(AppendArgs a) {
  const int b = blockIdx.x / a.n_new;
  const int j = blockIdx.x - b * a.n_new;
  const int tid = threadIdx.x;
  const int x = 16 / a.esize;          // elements per 16-byte chunk
  const int kchunks = a.dk / x;        // chunks of one head's key
  const int heads = a.latent ? 1 : a.hkv;
  const int nk = heads * kchunks;
  const int nv = a.latent ? 0 : a.hkv * a.dv;
  const int64_t row = (int64_t)b * a.n_new + j;
  const char* ksrc = a.k_new + row * heads * a.dk * a.esize;
  const char* vsrc = a.latent ? nullptr : a.v_new + row * a.hkv * a.dv * a.esize;
  // The source values do not depend on where they go: their loads are issued first, so their
  // latency overlaps the dependent position -> table-entry lookups below.
  const bool in_regs = nk <= kAppendThreads * kKPer && nv <= kAppendThreads * kVPer;
  uint4 kreg[kKPer];
  uint32_t vreg[kVPer];
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kKPer; ++r) {
      const int i = tid + r * kAppendThreads;
      kreg[r] = i < nk ? *reinterpret_cast<const uint4*>(ksrc + (int64_t)i * 16) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < kVPer; ++r) {
      const int i = tid + r * kAppendThreads;
      vreg[r] = i >= nv ? 0u
                : a.esize == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(vsrc)[i]
                               : reinterpret_cast<const uint32_t*>(vsrc)[i];
    }
  }
  const int64_t t = (int64_t)a.pos[b] + j;
  if (t < 0 || (t >> a.bs_shift) >= a.max_blocks) {
    if (tid == 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
    return;
  }
  const int32_t pid = a.table[(int64_t)b * a.max_blocks + (t >> a.bs_shift)];
  if (!valid_block(a.rt, pid)) {
    if (tid == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);
    return;
  }
  char* blk = const_cast<char*>(block_ptr(a.rt, pid));
  const int ts = (int)(t & (a.bs - 1));
  // K (or the latent): chunk c of head h goes to chunk slot ((h * kchunks + c) * bs + ts);
  // V: element (h, d) goes to element hkv * bs * dk + (h * dv + d) * bs + ts
  char* vdst = blk + (int64_t)a.hkv * a.bs * a.dk * a.esize;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kKPer; ++r) {
      const int i = tid + r * kAppendThreads;
      if (i < nk) *reinterpret_cast<uint4*>(blk + (((int64_t)i * a.bs + ts) << 4)) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < kVPer; ++r) {
      const int i = tid + r * kAppendThreads;
      if (i >= nv) continue;
      const int64_t off = ((int64_t)i * a.bs + ts) * a.esize;
      if (a.esize == 2)
        *reinterpret_cast<uint16_t*>(vdst + off) = (uint16_t)vreg[r];
      else
        *reinterpret_cast<uint32_t*>(vdst + off) = vreg[r];
    }
    return;
  }
  for (int i = tid; i < nk; i += kAppendThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(ksrc + (int64_t)i * 16);
    *reinterpret_cast<uint4*>(blk + (((int64_t)i * a.bs + ts) << 4)) = v;
  }
  for (int i = tid; i < nv; i += kAppendThreads) {
    const int64_t off = ((int64_t)i * a.bs + ts) * a.esize;
    if (a.esize == 2)
      *reinterpret_cast<uint16_t*>(vdst + off) = reinterpret_cast<const uint16_t*>(vsrc)[i];
    else
      *reinterpret_cast<uint32_t*>(vdst + off) = reinterpret_cast<const uint32_t*>(vsrc)[i];
  }
}

// Appends of a tile or more per sequence (prefill): one workgroup per (sequence, touched tile
// of T tokens, T a power of two dividing the block size, the largest whose K/V fit 64 KiB of
// LDS).  The tokens of the tile are read from the source rows, which are contiguous, into
// LDS, then written with consecutive lanes on consecutive token slots: K chunk slots of one
// (head, chunk) are consecutive 16-byte slots, and V values of one (head, dim) are consecutive
// elements, so both the reads and the writes coalesce (the per-token kernel writes V as
// scattered 2-byte stores).  Tokens with an index below 0 or past the table, or in a block
// whose entry is not a valid id, are flagged exactly as the per-token kernel flags them and
// are not written: the two kernels leave the same bytes.
__global__ void __launch_bounds__(kAppendThreads) append_blocks_kernel(AppendArgs a, int nt_max,
                                                                       int tshift) {
  extern __shared__ uint4 stage[];  // [T tokens][heads * Dk + Hkv * Dv] elements
  const int b = blockIdx.x / nt_max;
  const int i = blockIdx.x - b * nt_max;
  const int tid = threadIdx.x;
  const int64_t pos = a.pos[b];
  // tile of T = 2^tshift tokens (T divides bs): [ti * T, (ti + 1) * T)
  const int64_t ti = (pos >> tshift) + i;  // floor for negative positions too
  const int64_t lo = max(pos, ti << tshift);
  const int64_t hi = min(pos + a.n_new, (ti + 1) << tshift);
  if (lo >= hi) return;  // past the appended range
  const int64_t bi = ti >> (a.bs_shift - tshift);
  if (bi < 0 || bi >= a.max_blocks) {
    if (tid == 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
    return;
  }
  const int32_t pid = a.table[(int64_t)b * a.max_blocks + bi];
  if (!valid_block(a.rt, pid)) {
    if (tid == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);
    return;
  }
  char* blk = const_cast<char*>(block_ptr(a.rt, pid));
  const int x = 16 / a.esize;
  const int kchunks = a.dk / x;
  const int heads = a.latent ? 1 : a.hkv;
  const int nk = heads * kchunks;                        // K chunks of one token
  const int nvb = a.latent ? 0 : a.hkv * a.dv * a.esize; // V bytes of one token
  const int ntok = (int)(hi - lo);
  const int ts0 = (int)(lo - (bi << a.bs_shift));
  const int64_t j0 = lo - pos;                           // first source row
  // 1. source rows -> LDS, 16 bytes per lane, contiguous
  const int kbytes = nk * 16;
  char* sk = reinterpret_cast<char*>(stage);
  char* sv = sk + (int64_t)ntok * kbytes;
  const int64_t krow = (int64_t)heads * a.dk * a.esize;
  const char* ksrc = a.k_new + ((int64_t)b * a.n_new + j0) * krow;
  for (int q = tid; q < ntok * nk; q += kAppendThreads)
    reinterpret_cast<uint4*>(sk)[q] = reinterpret_cast<const uint4*>(ksrc)[q];
  if (nvb) {
    const char* vsrc = a.v_new + ((int64_t)b * a.n_new + j0) * nvb;
    if ((nvb & 15) == 0 && (reinterpret_cast<uintptr_t>(vsrc) & 15) == 0) {
      for (int q = tid; q < ntok * nvb / 16; q += kAppendThreads)
        reinterpret_cast<uint4*>(sv)[q] = reinterpret_cast<const uint4*>(vsrc)[q];
    } else {
      for (int q = tid; q < ntok * nvb / a.esize; q += kAppendThreads) {
        if (a.esize == 2)
          reinterpret_cast<uint16_t*>(sv)[q] = reinterpret_cast<const uint16_t*>(vsrc)[q];
        else
          reinterpret_cast<uint32_t*>(sv)[q] = reinterpret_cast<const uint32_t*>(vsrc)[q];
      }
    }
  }
  __syncthreads();
  // 2. K: slot ((h * kchunks + c) * bs + ts) <- chunk c of head h of token ts; the token index
  //    runs fastest over the lanes
  for (int q = tid; q < nk * ntok; q += kAppendThreads) {
    const int hc = q / ntok, tt = q - hc * ntok;
    *reinterpret_cast<uint4*>(blk + (((int64_t)hc * a.bs + ts0 + tt) << 4)) =
        *reinterpret_cast<const uint4*>(sk + (int64_t)tt * kbytes + hc * 16);
  }
  if (!nvb) return;
  // 3. V: element hkv * bs * dk + (h * dv + d) * bs + ts, token index fastest
  char* vdst = blk + (int64_t)a.hkv * a.bs * a.dk * a.esize;
  const int nve = a.hkv * a.dv;
  for (int q = tid; q < nve * ntok; q += kAppendThreads) {
    const int e = q / ntok, tt = q - e * ntok;
    const int64_t off = ((int64_t)e * a.bs + ts0 + tt) * a.esize;
    if (a.esize == 2)
      *reinterpret_cast<uint16_t*>(vdst + off) =
          reinterpret_cast<const uint16_t*>(sv + (int64_t)tt * nvb)[e];
    else
      *reinterpret_cast<uint32_t*>(vdst + off) =
          reinterpret_cast<const uint32_t*>(sv + (int64_t)tt * nvb)[e];
  }
}

// Bytes of one token's K and V as the block kernel stages them
static size_t append_token_bytes(const kvattn_layout& L) {
  const int e = L.kv_dtype == KVATTN_F32 ? 4 : 2;
  const int heads = L.latent ? 1 : L.num_kv_heads;
  return ((size_t)heads * L.head_dim_k + (L.latent ? 0 : (size_t)L.num_kv_heads * L.head_dim_v)) * e;
}

hipError_t launch_append(const RegionTable& rt, const kvattn_layout& L, const void* k_new,
                         const void* v_new, const int32_t* table, const int32_t* pos,
                         int32_t* err, int32_t batch, int32_t n_new, int32_t max_blocks,
                         int bs_shift, hipStream_t st) {
  AppendArgs a{};
  a.rt = rt;
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.table = table;
  a.pos = pos;
  a.err = err;
  a.batch = batch;
  a.n_new = n_new;
  a.max_blocks = max_blocks;
  a.hkv = L.num_kv_heads;
  a.dk = L.head_dim_k;
  a.dv = L.head_dim_v;
  a.bs = L.block_size;
  a.bs_shift = bs_shift;
  a.esize = L.kv_dtype == KVATTN_F32 ? 4 : 2;
  a.latent = L.latent;
  // tile: the largest power of two dividing bs whose tokens fit 64 KiB of LDS
  const size_t tok = append_token_bytes(L);
  int tshift = bs_shift;
  while (tshift > 0 && ((size_t)1 << tshift) * tok > 64 * 1024) --tshift;
  const int T = 1 << tshift;
  if (n_new >= T && (size_t)T * tok <= 64 * 1024 && T >= 8) {
    // tiles touched by n_new tokens from any position: at most ceil(n_new / T) + 1
    const int nt_max = (n_new + T - 1) / T + 1;
    hipLaunchKernelGGL(append_blocks_kernel, dim3((unsigned)((int64_t)batch * nt_max)),
                       dim3(kAppendThreads), (size_t)T * tok, st, a, nt_max, tshift);
  } else {
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)((int64_t)batch * n_new)),
                       dim3(kAppendThreads), 0, st, a);
  }
  return hipGetLastError();
}

// Eviction of staging blocks to host blocks: workgroup i copies device block src[i] of the
// device pool to block dst[i] of the host pool, whose region table holds the device-mapped
// addresses of pinned host regions; 16 bytes per lane, written over the host link.  The
// list travels by value in the kernel arguments.
constexpr int kMaxCopies = 240;

struct CopyList {
  int32_t n;
  int32_t src[kMaxCopies];
  int32_t dst[kMaxCopies];
};

__global__ void __launch_bounds__(256) copy_blocks_kernel(RegionTable src_rt, RegionTable dst_rt,
                                                          CopyList list) {
  const int i = blockIdx.x;
  if (i >= list.n) return;
  const uint4* s = reinterpret_cast<const uint4*>(block_ptr(src_rt, list.src[i]));
  uint4* d = reinterpret_cast<uint4*>(const_cast<char*>(block_ptr(dst_rt, list.dst[i])));
  for (int64_t j = threadIdx.x; j < src_rt.block_bytes / 16; j += blockDim.x) d[j] = s[j];
}

// pairs: [n][2] = (device id, host id); host_bases: device addresses of the host pool's regions
hipError_t launch_copy_blocks(const kvattn_pool* dev, const kvattn_pool* host,
                              void* const* host_bases, const int32_t* pairs, int n,
                              hipStream_t st) {
  const RegionTable src_rt = region_table(dev);
  const RegionTable dst_rt = region_table(host, host_bases);
  for (int first = 0; first < n; first += kMaxCopies) {
    CopyList list{};
    list.n = n - first < kMaxCopies ? n - first : kMaxCopies;
    for (int i = 0; i < list.n; ++i) {
      list.src[i] = pairs[2 * (first + i)];
      list.dst[i] = pairs[2 * (first + i) + 1];
    }
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)list.n), dim3(256), 0, st, src_rt, dst_rt,
                       list);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvattn
