// Exact LSE merge of per-partition partials, plus an optional external partial.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference",
// §4.2 and §5.1-5.2: the engines' partial outputs merge exactly by log-sum-exp rescaling,
// one join per step, performed on the GPU; the other engine ships only its partial output
// and normaliser.  For each (sequence, head):
//     M = max_p lse_p,  lse = M + ln sum_p exp(lse_p - M),  o = sum_p exp(lse_p - lse) o_p.
// One thread per (sequence, head, 4 output dims); the weights are recomputed per thread from
// the lse row (broadcast reads), and the partial rows are read with 16-byte loads, eight
// partitions in flight at a time.

#include "device_common.h"

namespace kvattn {

static constexpr float kNegInfG = -__builtin_huge_valf();

__global__ __launch_bounds__(256) void merge_lse_kernel(MergeArgs a) {
  const int cols = a.dv >> 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)a.batch * a.hq;
  if (gid >= rows * cols) return;
  const int64_t row = gid / cols;  // b * Hq + h
  const int col = (int)(gid - row * cols);
  const int b = (int)(row / a.hq);
  int np = a.nparts[b];
  np = np < 0 ? 0 : (np > a.max_parts ? a.max_parts : np);
  const float* lrow = a.lse_part + row * a.max_parts;
  const bool ext = a.o_ext != nullptr;
  const float lx = ext ? a.lse_ext[row] : kNegInfG;

  float big = lx;
  for (int p = 0; p < np; ++p) big = fmaxf(big, lrow[p]);
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  float lse = kNegInfG;
  if (big != kNegInfG) {
    float tot = ext ? expf(lx - big) : 0.f;
    for (int p = 0; p < np; ++p) tot += expf(lrow[p] - big);
    lse = big + logf(tot);
    const f32x4* orow = reinterpret_cast<const f32x4*>(a.o_part + row * a.max_parts * a.dv) + col;
    const int stride = cols;  // f32x4 per partition row
    int p = 0;
    for (; p + 8 <= np; p += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = orow[(int64_t)(p + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) o += v[u] * expf(lrow[p + u] - lse);
    }
    for (; p < np; ++p) o += orow[(int64_t)p * stride] * expf(lrow[p] - lse);
    if (ext) {
      const f32x4 vx = reinterpret_cast<const f32x4*>(a.o_ext + row * a.dv)[col];
      o += vx * expf(lx - lse);
    }
  }
  reinterpret_cast<f32x4*>(a.o_out + row * a.dv)[col] = o;
  if (a.lse_out && col == 0) a.lse_out[row] = lse;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int64_t threads = (int64_t)a.batch * a.hq * (a.dv >> 2);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvattn
