// Block-level sparse selection: the sub-table of a per-sequence set of selected blocks.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference", §4.2
// (sparse-selection compatibility): a block-level top-k selection is a set of whole blocks, so
// the block format serves sparse attention unchanged.  Here the set becomes a sub-table on the
// device, with no host round trip, and the decode kernels run on it as they are.
//
// One workgroup per sequence: the selected logical indices are marked in an LDS bitmap (a
// repeated or out-of-range index is flagged and ignored), the partial last block is set aside,
// and the full blocks are written in ascending order through a prefix sum of per-thread
// popcounts; the partial block, if selected, goes last.

#include <string>

#include "device_common.h"
#include "pool_internal.h"

namespace kvattn {

constexpr int kSelThreads = 256;

__global__ void __launch_bounds__(kSelThreads)
select_blocks_kernel(const int32_t* table, int32_t max_blocks, const int32_t* ctx_lens, int bs,
                     int bs_shift, const int32_t* sel, int32_t k, int32_t* sub_table,
                     int32_t max_sub, int32_t* sub_len, int32_t* err) {
  extern __shared__ uint32_t bm[];          // ceil(max_blocks / 32) words
  __shared__ int32_t offs[kSelThreads + 1];
  __shared__ int32_t n_full_s;
  __shared__ int32_t last_sel_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int words = (max_blocks + 31) >> 5;
  const int32_t L = ctx_lens[b];
  const int64_t nb64 = L < 0 ? -1 : (((int64_t)L + bs - 1) >> bs_shift);
  int32_t* out = sub_table + (int64_t)b * max_sub;
  if (nb64 < 0 || nb64 > max_blocks) {
    if (tid == 0) {
      flag_error(err, KVATTN_ERR_BAD_SEQ);
      sub_len[b] = 0;
    }
    for (int i = tid; i < max_sub; i += kSelThreads) out[i] = KVATTN_BLOCK_ABSENT;
    return;
  }
  const int nb = (int)nb64;
  for (int w = tid; w < words; w += kSelThreads) bm[w] = 0u;
  __syncthreads();
  bool bad = false;
  for (int i = tid; i < k; i += kSelThreads) {
    const int32_t s = sel[(int64_t)b * k + i];
    if (s < 0) continue;
    if (s >= nb) {
      bad = true;
      continue;
    }
    const uint32_t bit = 1u << (s & 31);
    if (atomicOr(&bm[s >> 5], bit) & bit) bad = true;  // repeated
  }
  if (bad) flag_error(err, KVATTN_ERR_BAD_SELECT);
  __syncthreads();
  // the partial last block is placed after the full ones
  const int last = (L & (bs - 1)) ? nb - 1 : -1;
  if (tid == 0) {
    last_sel_s = 0;
    if (last >= 0 && (bm[last >> 5] >> (last & 31)) & 1u) {
      last_sel_s = 1;
      bm[last >> 5] &= ~(1u << (last & 31));
    }
  }
  __syncthreads();
  // per-thread contiguous word ranges, counted, then an exclusive scan over the threads
  const int per = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = tid * per, w1 = min(words, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  offs[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < kSelThreads; ++t) {
      const int c = offs[t];
      offs[t] = run;
      run += c;
    }
    n_full_s = run;
  }
  __syncthreads();
  int o = offs[tid];
  const int32_t* row = table + (int64_t)b * max_blocks;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      const int j = (w << 5) + __builtin_ctz(bits);
      out[o++] = row[j];
      bits &= bits - 1;
    }
  }
  const int n_full = n_full_s;
  const int n_out = n_full + last_sel_s;
  if (tid == 0) {
    if (last_sel_s) out[n_full] = row[last];
    sub_len[b] = n_full * bs + (last_sel_s ? L - last * bs : 0);
  }
  for (int i = n_out + tid; i < max_sub; i += kSelThreads) out[i] = KVATTN_BLOCK_ABSENT;
}

}  // namespace kvattn

extern "C" kvattn_status kvattn_select_blocks(const int32_t* table_dev, int32_t max_blocks,
                                              const int32_t* ctx_lens_dev, int32_t block_size,
                                              const int32_t* sel_dev, int32_t batch, int32_t k,
                                              int32_t* sub_table_dev, int32_t max_sub,
                                              int32_t* sub_len_dev, int32_t* err_dev,
                                              void* hip_stream) {
  using namespace kvattn;
  clear_error();
  if (!table_dev || !ctx_lens_dev || !sel_dev || !sub_table_dev || !sub_len_dev)
    return set_error(KVATTN_E_INVAL, "select_blocks: null argument");
  if (batch < 1 || k < 1 || max_sub < k || max_blocks < 1 || max_blocks > 65536)
    return set_error(KVATTN_E_INVAL,
                     "select_blocks: batch, k >= 1, max_sub >= k and max_blocks in [1, 65536] required");
  if (block_size < 1 || block_size > 256 || (block_size & (block_size - 1)) != 0)
    return set_error(KVATTN_E_INVAL, "select_blocks: block_size must be a power of two <= 256");
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const size_t lds = (size_t)((max_blocks + 31) / 32) * 4;
  hipLaunchKernelGGL(select_blocks_kernel, dim3((unsigned)batch), dim3(kSelThreads), lds,
                     static_cast<hipStream_t>(hip_stream), table_dev, max_blocks, ctx_lens_dev,
                     block_size, shift, sel_dev, k, sub_table_dev, max_sub, sub_len_dev, err_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(KVATTN_E_HIP, std::string("select_blocks launch: ") + hipGetErrorString(e));
  return KVATTN_OK;
}
