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
  uint64_t adj[KVATTN_MAX_REGIONS];  // (uint64)base[r] - first[r] * block_bytes (mod 2^64)
  int32_t first32[KVATTN_MAX_REGIONS];  // first[r] (ids fit in int32)
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
  int32_t max_blocks, max_parts;
  int32_t group_parts;     // consecutive partitions merged on chip into one written partial
  int32_t wave_parts;      // matrix-core GQA kernel: consecutive partitions per wave
  int32_t grid_ng;         // work items per (sequence, KV head): the largest group count
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

// Pointers into device memory in the global address space, so that loads through them are
// global (not flat) loads: flat loads also count against the LDS wait counter, which would
// make every LDS wait drain the outstanding HBM loads.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const char gchar;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;

// Start of block `pid`, which must be a valid id, with selects only (no dynamic indexing of
// the kernarg table, no branches): the last region whose first id is <= pid owns it.
__device__ __forceinline__ gchar* block_addr(const RegionTable& rt, int32_t pid) {
  uint64_t a = rt.adj[0];
#pragma unroll
  for (int i = 1; i < KVATTN_MAX_REGIONS; ++i)
    a = (i < rt.n && pid >= rt.first32[i]) ? rt.adj[i] : a;
  return reinterpret_cast<gchar*>(a + (uint64_t)(int64_t)pid * (uint64_t)rt.block_bytes);
}

__device__ __forceinline__ void flag_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Partition count of sequence b from the device copy of the per-sequence values, and in *ng
// the number of partials written for it, ceil(np / group_parts).  Returns -1 (and *ng = -1)
// if the values are inconsistent with the launch.
// Row stride, in floats, of the partial outputs a matrix-core GQA workgroup merges in LDS:
// padded by 4 so that the 16 rows one quarter of a wave writes at once start on different LDS
// banks (an unpadded power-of-two stride puts them all on the same ones), unless the padding
// would take the merge area (rows plus one lse per row) past 64 KiB.
__host__ __device__ inline int gqa_merge_row(int waves, int group, int d) {
  return (int64_t)waves * group * (d + 5) * 4 <= 65536 ? d + 4 : d;
}

__device__ __forceinline__ int seq_partitions(const DecodeArgs& a, int b, int* lo_tok, int* part,
                                              int* ng) {
  const int L = a.seq[b];
  const int beg = a.seq[a.batch + b];
  const int P = a.seq[2 * a.batch + b];
  *lo_tok = beg;
  *part = P;
  *ng = -1;
  const bool ok = beg >= 0 && beg <= L && (int64_t)L <= ((int64_t)a.max_blocks << a.bs_shift) &&
                  P > 0 && (P & (a.bs - 1)) == 0;
  if (!ok) return -1;
  const int np = (int)(((int64_t)L - beg + P - 1) / P);
  const int groups = (np + a.group_parts - 1) / a.group_parts;
  if (groups > a.max_parts || groups > a.grid_ng) return -1;
  *ng = groups;
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
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(u32x2 v) { return __builtin_bit_cast(i16x4, v); }

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with the
// gfx950 lane-swap instructions (VALU only, no LDS round trip): v_permlane32_swap with both
// operands = v yields v[l mod 32] and v[l mod 32 + 32]; v_permlane16_swap likewise pairs
// rows 0/1 and 2/3.  Every lane ends with the same value, summed in the same order.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Wave-wide max / sum on the VALU (no LDS round trips), for a wave with every lane active.
// Within each row of 16 lanes, DPP moves pair lane l with l^1 and l^2 (quad_perm), then with
// its mirror in the half row (l^7: the other quad, whose lanes agree by then) and in the row
// (l^15: the other half); the rows are then combined by rows_max / rows_sum.  Every lane
// combines the same two values at every step, so all lanes end with the same bits.
__device__ __forceinline__ float dpp_move(float v, int ctrl_sel) {
  const int x = __float_as_int(v);
  int y;
  switch (ctrl_sel) {  // the control must be a constant
    case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return __int_as_float(y);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = fmaxf(v, dpp_move(v, c));
  return rows_max(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = v + dpp_move(v, c);
  return rows_sum(v);
}

}  // namespace kvattn
