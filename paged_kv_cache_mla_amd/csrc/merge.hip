// Exact LSE merge of per-partition partials, plus an optional external partial.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference",
// §4.2 and §5.1-5.2: the engines' partial outputs merge exactly by log-sum-exp rescaling,
// one join per step, performed on the GPU; the other engine ships only its partial output
// and normaliser.  For each (sequence, head):
//     M = max_p lse_p,  lse = M + ln sum_p exp(lse_p - M),  o = sum_p exp(lse_p - lse) o_p.
//
// One 256-thread workgroup per (sequence, head).  The partition weights exp(lse_p - lse)
// are computed once (block-wide max and sum) into LDS; then thread (g, c) of a
// [groups x dv/4] arrangement sums 16-byte columns c of partitions p = g, g + groups, ...,
// and the groups are reduced through LDS.  Partitions are processed in chunks of kChunk so
// any partition count works with a fixed LDS footprint.

#include "device_common.h"

namespace kvattn {

static constexpr float kNegInfG = -__builtin_huge_valf();
static constexpr int kThreads = 256;
static constexpr int kChunk = 1024;

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
  __shared__ float wts[kChunk];
  __shared__ f32x4 part[kThreads];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;  // b * Hq + h
  const int b = (int)(row / a.hq);
  int np = a.nparts[b];
  np = np < 0 ? 0 : (np > a.max_parts ? a.max_parts : np);
  const float* lrow = a.lse_part + row * a.max_parts;
  const bool ext = a.o_ext != nullptr;
  const float lx = ext ? a.lse_ext[row] : kNegInfG;

  // M = max over partitions (and the external partial)
  float mx = lx;
  for (int p = tid; p < np; p += kThreads) mx = fmaxf(mx, lrow[p]);
  const float big = block_max(mx, red);
  const int cols = a.dv >> 2;
  const int groups = kThreads / cols;       // >= 1 since dv <= 1024
  const int g = tid / cols;
  const int c = tid - g * cols;
  const bool active = g < groups;
  f32x4* orow_out = reinterpret_cast<f32x4*>(a.o_out + row * a.dv);
  if (big == kNegInfG) {  // nothing of positive weight
    if (tid < cols) orow_out[tid] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.lse_out && tid == 0) a.lse_out[row] = kNegInfG;
    return;
  }
  float sm = (ext && tid == 0) ? expf(lx - big) : 0.f;
  for (int p = tid; p < np; p += kThreads) sm += expf(lrow[p] - big);
  const float tot = block_sum(sm, red);
  const float lse = big + logf(tot);

  const f32x4* orow = reinterpret_cast<const f32x4*>(a.o_part + row * a.max_parts * a.dv);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < np; p0 += kChunk) {
    const int n = min(kChunk, np - p0);
    __syncthreads();  // previous chunk's weights consumed
    for (int p = tid; p < n; p += kThreads) wts[p] = expf(lrow[p0 + p] - lse);
    __syncthreads();
    if (active) {
      int p = g;
      for (; p + 3 * groups < n; p += 4 * groups) {
        const f32x4 v0 = orow[(int64_t)(p0 + p) * cols + c];
        const f32x4 v1 = orow[(int64_t)(p0 + p + groups) * cols + c];
        const f32x4 v2 = orow[(int64_t)(p0 + p + 2 * groups) * cols + c];
        const f32x4 v3 = orow[(int64_t)(p0 + p + 3 * groups) * cols + c];
        acc += v0 * wts[p] + v1 * wts[p + groups] + v2 * wts[p + 2 * groups] + v3 * wts[p + 3 * groups];
      }
      for (; p < n; p += groups) acc += orow[(int64_t)(p0 + p) * cols + c] * wts[p];
    }
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < cols) {
    f32x4 o = part[tid];
    for (int k = 1; k < groups; ++k) o += part[k * cols + tid];
    if (ext) o += reinterpret_cast<const f32x4*>(a.o_ext + row * a.dv)[tid] * expf(lx - lse);
    orow_out[tid] = o;
  }
  if (a.lse_out && tid == 0) a.lse_out[row] = lse;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.batch * a.hq;
  hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvattn
