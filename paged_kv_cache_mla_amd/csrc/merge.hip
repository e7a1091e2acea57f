// Exact LSE merge of per-partition partials, plus an optional external partial.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference",
// §4.2 and §5.1-5.2: the engines' partial outputs merge exactly by log-sum-exp rescaling,
// one join per step, performed on the GPU; the other engine ships only its partial output
// and normaliser.  For each (sequence, head):
//     M = max_p lse_p,  T = sum_p exp(lse_p - M),  lse = M + ln T,
//     o = sum_p exp(lse_p - M) o_p / T        (= sum_p exp(lse_p - lse) o_p).
// A partial of zero weight (lse = -inf, or a weight that underflows) is left out of the sum
// by a select, never multiplied by 0: its o may be anything, NaN included.
//
// Three kernels.  The workgroup kernel: one 256-thread workgroup per (sequence, head); thread
// (g, c) of a [groups x dv/4] arrangement owns 16-byte column c of partitions g, g + groups,
// ...  The merge is bound by the latency of a few dependent steps, not by bandwidth, so the
// order is: issue the loads of
// the thread's first kSpec partial columns and of the first lse values at once, before the
// partition count is known (bounded by max_parts), then its next kR - kSpec columns bounded
// by the count, then take the block max, write the weights to LDS while summing them, and
// only then consume the partial columns already in registers.
// Partitions beyond kR * groups (long sequences, wide heads) follow in further chunks of
// kR * groups.  Every sum runs in a fixed order, so the result is bitwise reproducible.
// The two wave kernels below take one wave per (sequence, head) with every partial in
// registers: narrow heads (up to 128 values), and wide heads (256 or 512) with few partials.

#include <cstdlib>
#include <cstring>

#include "device_common.h"

namespace kvattn {

static constexpr float kNegInfG = -__builtin_huge_valf();
static constexpr int kThreads = 256;
static constexpr int kWts = 2048;  // partitions whose weights are kept in LDS
static constexpr int kR = 16;      // partial columns per thread held in registers
static constexpr int kSpec = 4;    // of which loaded before the partition count is known

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(kThreads) void merge_lse_kernel(MergeArgs a) {
  __shared__ float wts[kWts];
  __shared__ f32x4 part[kThreads];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;  // b * Hq + h
  const int b = (int)(row / a.hq);
  const int np_raw = a.nparts[b];
  const float* lrow = a.lse_part + row * a.max_parts;
  const bool ext = a.o_ext != nullptr;
  const float lx = ext ? a.lse_ext[row] : kNegInfG;

  const int cols = a.dv >> 2;
  const int groups = kThreads / cols;  // >= 1 since dv <= 1024
  const int g = tid / cols;
  const int c = tid - g * cols;
  const bool active = g < groups;
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.o_part + row * a.max_parts * a.dv);

  // 1. loads issued before the partition count arrives: the partial columns of the first
  //    kSpec * groups partition slots and the first 256 lse slots, bounded by max_parts
  //    (slots past the sequence's count hold stale data and are discarded by selection
  //    below); the rest of the first chunk follows as soon as the count is known, bounded by
  //    it, so a short sequence in a call sized for long ones reads only its own partials
  f32x4 ov[kR];
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    const int p = g + k * groups;
    ov[k] = (active && k < kSpec && p < a.max_parts) ? orow[(int64_t)p * cols + c]
                                                      : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float l0 = tid < a.max_parts ? lrow[tid] : kNegInfG;
  const int np = np_raw < 0 ? 0 : (np_raw > a.max_parts ? a.max_parts : np_raw);
#pragma unroll
  for (int k = kSpec; k < kR; ++k) {
    const int p = g + k * groups;
    if (active && p < np) ov[k] = orow[(int64_t)p * cols + c];
  }

  // 2. M = max over partitions (and the external partial)
  float mx = lx;
  if (tid < np) mx = fmaxf(mx, l0);
  for (int p = tid + kThreads; p < np; p += kThreads) mx = fmaxf(mx, lrow[p]);
  const float big = block_max(mx, red);
  f32x4* orow_out = reinterpret_cast<f32x4*>(a.o_out + row * a.dv);
  if (big == kNegInfG) {  // nothing of positive weight (uniform across the block)
    if (tid < cols) orow_out[tid] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.lse_out && tid == 0) a.lse_out[row] = kNegInfG;
    return;
  }

  // 3. weights exp(lse_p - M) into LDS, T = their sum (+ the external weight)
  const float wx = ext ? expf(lx - big) : 0.f;
  float sm = tid == 0 ? wx : 0.f;
  for (int p = tid; p < np; p += kThreads) {
    const float w = expf((p == tid ? l0 : lrow[p]) - big);
    sm += w;
    if (p < kWts) wts[p] = w;
  }
  const float tot = block_sum(sm, red);  // its barriers also publish wts

  // 4. weighted sum of the partial columns, chunk by chunk of kR * groups partitions; the
  //    loads of a chunk are all issued before any is used, so kR are in flight per thread
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int p0 = 0; p0 < np; p0 += kR * groups) {
      if (p0 > 0) {
#pragma unroll
        for (int k = 0; k < kR; ++k) {
          const int p = p0 + g + k * groups;
          ov[k] = p < np ? orow[(int64_t)p * cols + c] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int k = 0; k < kR; ++k) {
        const int p = p0 + g + k * groups;
        const float w = p < np ? (p < kWts ? wts[p] : expf(lrow[p] - big)) : 0.f;
        if (w != 0.f) acc += ov[k] * w;  // a select: stale slots and weightless partials
                                         // (o may be anything there, NaN included) never enter
      }
    }
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < cols) {
    f32x4 o = part[tid];
    for (int k = 1; k < groups; ++k) o += part[k * cols + tid];
    if (wx != 0.f) o += reinterpret_cast<const f32x4*>(a.o_ext + row * a.dv)[tid] * wx;
    orow_out[tid] = o * (1.f / tot);
  }
  if (a.lse_out && tid == 0) a.lse_out[row] = big + logf(tot);
}

// One wave per (sequence, head) for narrow heads and few partials, the common case once the
// decode kernels merge groups of partitions on chip: no barrier at all.  Lane (s, c) of a
// [64 / cols x cols] arrangement owns 16-byte column c of partitions s, s + S, s + 2S, ...
// (S = 64 / cols); lane p also holds lse_p.  The maximum and the sum of the weights are wave
// reductions, each lane fetches the weight of its partitions from the lane holding them, and
// the column sums are folded across the S lanes of a column with lane swaps.  All loads are
// issued before the partition count is used.  Fixed order everywhere: bitwise reproducible.
static constexpr int kWaveParts = 16;   // partitions per lane held in registers

__global__ __launch_bounds__(kThreads) void merge_lse_wave_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.batch * a.hq) return;  // uniform per wave
  const int b = (int)(row / a.hq);
  const int cols = a.dv >> 2;
  const int S = 64 / cols;
  const int s = lane / cols;
  const int c = lane - s * cols;
  const float* lrow = a.lse_part + row * a.max_parts;
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.o_part + row * a.max_parts * a.dv);
  const bool ext = a.o_ext != nullptr;
  f32x4 ov[kWaveParts];
#pragma unroll
  for (int k = 0; k < kWaveParts; ++k) {
    const int p = s + k * S;
    ov[k] = p < a.max_parts ? orow[(int64_t)p * cols + c] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float l0 = lane < a.max_parts ? lrow[lane] : kNegInfG;
  const float lx = ext ? a.lse_ext[row] : kNegInfG;
  const int np_raw = a.nparts[b];
  const int np = np_raw < 0 ? 0 : (np_raw > a.max_parts ? a.max_parts : np_raw);
  const float big = fmaxf(wave_max(lane < np ? l0 : kNegInfG), lx);
  f32x4* orow_out = reinterpret_cast<f32x4*>(a.o_out + row * a.dv);
  if (big == kNegInfG) {
    if (lane < cols) orow_out[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.lse_out && lane == 0) a.lse_out[row] = kNegInfG;
    return;
  }
  const float wl = lane < np ? expf(l0 - big) : 0.f;
  const float wx = ext ? expf(lx - big) : 0.f;
  const float tot = wave_sum(wl) + wx;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kWaveParts; ++k) {
    const int p = s + k * S;
    const float w = __shfl(wl, p < 64 ? p : 0);
    if (p < np && w != 0.f) acc += ov[k] * w;  // a select: stale slots and weightless
                                               // partials (o may be NaN there) never enter
  }
  for (int o = cols; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o);
    acc.y += __shfl_xor(acc.y, o);
    acc.z += __shfl_xor(acc.z, o);
    acc.w += __shfl_xor(acc.w, o);
  }
  if (lane < cols) {
    f32x4 o = acc;
    if (wx != 0.f) o += reinterpret_cast<const f32x4*>(a.o_ext + row * a.dv)[lane] * wx;
    orow_out[lane] = o * (1.f / tot);
  }
  if (a.lse_out && lane == 0) a.lse_out[row] = big + logf(tot);
}

// One wave per (sequence, head) for wide heads of 256 * C values (MLA's 512: C = 2) with at
// most kWideParts partials: lane l owns 16-byte columns l, l + 64, ..., l + 64 (C - 1) of
// every partition, and lane p holds lse_p.  The order of operations is the narrow wave
// kernel's: all loads before the partition count is used, wave reductions for the maximum and
// the weight sum, weights fetched from the lanes holding them, fixed summation order.
static constexpr int kWideParts = 16;

template <int C>
__global__ __launch_bounds__(kThreads) void merge_lse_wide_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.batch * a.hq) return;  // uniform per wave
  const int b = (int)(row / a.hq);
  constexpr int cols = 64 * C;
  const float* lrow = a.lse_part + row * a.max_parts;
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.o_part + row * a.max_parts * a.dv);
  const bool ext = a.o_ext != nullptr;
  f32x4 ov[kWideParts][C];
#pragma unroll
  for (int k = 0; k < kWideParts; ++k)
#pragma unroll
    for (int u = 0; u < C; ++u)
      ov[k][u] = k < a.max_parts ? orow[(int64_t)k * cols + lane + 64 * u] : f32x4{0.f, 0.f, 0.f, 0.f};
  const float l0 = lane < a.max_parts ? lrow[lane] : kNegInfG;
  const float lx = ext ? a.lse_ext[row] : kNegInfG;
  const int np_raw = a.nparts[b];
  const int np = np_raw < 0 ? 0 : (np_raw > a.max_parts ? a.max_parts : np_raw);
  const float big = fmaxf(wave_max(lane < np ? l0 : kNegInfG), lx);
  f32x4* orow_out = reinterpret_cast<f32x4*>(a.o_out + row * a.dv);
  if (big == kNegInfG) {
#pragma unroll
    for (int u = 0; u < C; ++u) orow_out[lane + 64 * u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.lse_out && lane == 0) a.lse_out[row] = kNegInfG;
    return;
  }
  const float wl = lane < np ? expf(l0 - big) : 0.f;
  const float wx = ext ? expf(lx - big) : 0.f;
  const float tot = wave_sum(wl) + wx;
  f32x4 acc[C];
#pragma unroll
  for (int u = 0; u < C; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kWideParts; ++k) {
    const float w = __shfl(wl, k);
    if (k < np && w != 0.f) {  // a select: stale slots and weightless partials never enter
#pragma unroll
      for (int u = 0; u < C; ++u) acc[u] += ov[k][u] * w;
    }
  }
  const float inv = 1.f / tot;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    f32x4 o = acc[u];
    if (wx != 0.f) o += reinterpret_cast<const f32x4*>(a.o_ext + row * a.dv)[lane + 64 * u] * wx;
    orow_out[lane + 64 * u] = o * inv;
  }
  if (a.lse_out && lane == 0) a.lse_out[row] = big + logf(tot);
}

enum MergeKind { kMergeBlock, kMergeWave, kMergeWide };

// The narrow wave kernel takes heads of 4 .. 128 values (a power-of-two number of 16-byte
// columns) with every partition slot in its registers, the wide one heads of 256 or 512
// values with at most 16 partials; anything else goes to the workgroup kernel.
// KVATTN_MERGE_KERNEL=block overrides the choice (tuning and tests).
static MergeKind merge_kind(const MergeArgs& a) {
  const char* e = std::getenv("KVATTN_MERGE_KERNEL");
  if (e && std::strcmp(e, "block") == 0) return kMergeBlock;
  const int cols = a.dv >> 2;
  if ((a.dv & 3) == 0 && cols >= 1 && cols <= 32 && (64 % cols) == 0 &&
      a.max_parts <= (64 / cols) * kWaveParts && a.max_parts <= 64)
    return kMergeWave;
  if ((a.dv == 256 || a.dv == 512) && a.max_parts <= kWideParts) return kMergeWide;
  return kMergeBlock;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.batch * a.hq;
  const int64_t per = kThreads / 64;
  const dim3 waves((unsigned)((rows + per - 1) / per));
  switch (merge_kind(a)) {
    case kMergeWave:
      hipLaunchKernelGGL(merge_lse_wave_kernel, waves, dim3(kThreads), 0, st, a);
      break;
    case kMergeWide:
      if (a.dv == 256)
        hipLaunchKernelGGL(merge_lse_wide_kernel<1>, waves, dim3(kThreads), 0, st, a);
      else
        hipLaunchKernelGGL(merge_lse_wide_kernel<2>, waves, dim3(kThreads), 0, st, a);
      break;
    default:
      hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace kvattn
