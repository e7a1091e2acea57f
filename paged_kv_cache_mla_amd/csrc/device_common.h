// Device-side helpers shared by the decode kernels, the merge and the resolution probe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvattn.h"

namespace kvattn {

// Region table passed by value in the kernel arguments (it lives in the kernarg segment and
// is read with scalar loads).  Block id `pid` belongs to the last region r with
// first[r] <= pid and starts at base[r] + (pid - first[r]) * block_bytes.
struct RegionTable {
  const char* base[KVATTN_MAX_REGIONS];
  int64_t first[KVATTN_MAX_REGIONS + 1];
  int64_t block_bytes;
  int32_t n;
  int32_t total;  // number of valid ids
};

// Per-launch arguments of the decode kernels.
struct DecodeArgs {
  RegionTable rt;
  const void* q;           // [B][Hq][Dk]
  const int32_t* table;    // [B][max_blocks]
  const int32_t* seq;      // [3][B]: ctx_len, tok_begin, part_tokens
  float* o_part;           // [B][Hq][max_parts][Dv]
  float* lse_part;         // [B][Hq][max_parts]
  int32_t* nparts;         // [B]
  int32_t* err;            // nullable
  int32_t batch, hq, hkv, group;
  int32_t max_blocks, max_parts, grid_np;
  int32_t bs, bs_shift;
  float scale;             // softmax scale
  float scale_log2;        // scale * log2(e)
};

// Arguments of the merge kernel.
struct MergeArgs {
  const float* o_part;     // [B][Hq][max_parts][dv]
  const float* lse_part;   // [B][Hq][max_parts]
  const int32_t* nparts;   // [B]
  const float* o_ext;      // [B][Hq][dv] or null
  const float* lse_ext;    // [B][Hq] or null
  float* o_out;            // [B][Hq][dv]
  float* lse_out;          // [B][Hq] or null
  int32_t batch, hq, max_parts, dv;
};

// Region index of a valid id (ids are < rt.total; the caller checked).
__device__ __forceinline__ int region_of(const RegionTable& rt, int32_t pid) {
  int r = 0;
#pragma unroll
  for (int i = 1; i < KVATTN_MAX_REGIONS; ++i)
    if (i < rt.n && (int64_t)pid >= rt.first[i]) r = i;
  return r;
}

__device__ __forceinline__ bool valid_block(const RegionTable& rt, int32_t pid) {
  return pid >= 0 && pid < rt.total;
}

// Start of block `pid`; for an invalid id, the start of block 0 (a harmless, in-bounds
// address whose data the caller masks out).
__device__ __forceinline__ const char* block_ptr(const RegionTable& rt, int32_t pid) {
  if (!valid_block(rt, pid)) return rt.base[0];
  const int r = region_of(rt, pid);
  return rt.base[r] + ((int64_t)pid - rt.first[r]) * rt.block_bytes;
}

__device__ __forceinline__ void flag_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Partition count of sequence b from the device copy of the per-sequence values; returns
// 0 (and flags KVATTN_ERR_BAD_SEQ) if they are inconsistent with the launch.
__device__ __forceinline__ int seq_partitions(const DecodeArgs& a, int b, int* lo_tok,
                                              int* part) {
  const int L = a.seq[b];
  const int beg = a.seq[a.batch + b];
  const int P = a.seq[2 * a.batch + b];
  *lo_tok = beg;
  *part = P;
  const bool ok = beg >= 0 && beg <= L && (int64_t)L <= ((int64_t)a.max_blocks << a.bs_shift) &&
                  P > 0 && (P & (a.bs - 1)) == 0;
  if (!ok) return -1;
  const int np = (int)(((int64_t)L - beg + P - 1) / P);
  if (np > a.max_parts || np > a.grid_np) return -1;
  return np;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// float -> bfloat16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(uint2 v) { return __builtin_bit_cast(i16x4, v); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace kvattn
