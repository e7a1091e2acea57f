// Decode-attention partials for per-head K/V caches (GQA), gfx950.
//
// Computes, for one (sequence, KV head, partition), the partial attention of the query heads
// sharing that KV head over the partition's tokens, with an online softmax (running max and
// normaliser, fp32 accumulation) -- "Physically Partitioned KVCache Format for CPU-GPU Load
// Balancing in MoE Inference", §6.1 -- and emits (o normalised by its own sum, lse) so that
// partials of disjoint token ranges merge exactly (same page, §5.1).
//
// Two kernels:
//  * gqa_decode_mfma_kernel (bf16, block size >= 16): one wave per work item.  Each 16-token
//    tile is a dense contraction on the matrix cores: S^T[16 tok x 16 heads] = K Q^T with
//    v_mfma_f32_16x16x32_bf16 (query heads of the group in the N columns, padded to 16),
//    then O^T[D x 16 heads] += V^T P^T with v_mfma_f32_16x16x16_bf16.  The block layout makes
//    both operands plain 16-byte / 8-byte per-lane loads straight from HBM: K is stored in
//    16-byte chunks with the chunks of consecutive tokens side by side (one k-step of one tile
//    is 1 KiB contiguous), V is stored transposed (one 16-dim slice of a tile is 512 B
//    contiguous).  The MFMA output layout of S^T (lane = head column, 4 consecutive tokens per
//    lane) is exactly the B-operand layout the PV product needs, so no data moves between
//    lanes except two shuffles for the per-head max.  Tiles are prefetched NBUF deep in
//    registers.
//  * gqa_decode_generic_kernel (fp32 or bf16, any block size): a plain VALU version, one token
//    per lane, used for fp32 caches and as an independent cross-check of the MFMA kernel.

#include "device_common.h"

namespace kvattn {

static constexpr float kNegInf = -__builtin_huge_valf();
static constexpr float kLn2 = 0.693147180559945309f;

template <int D, int NBUF>
__global__ __launch_bounds__(64) void gqa_decode_mfma_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;  // k-steps of the QK product (32 dims each)
  constexpr int VT = D / 16;  // 16-dim output tiles of the PV product
  const int lane = threadIdx.x;
  const int n = lane & 15;  // MFMA row / column index
  const int g4 = lane >> 4; // lane group: k-slot of the operands, row group of the output

  int w = blockIdx.x;
  const int p = w % a.grid_np;
  w /= a.grid_np;
  const int kvh = w % a.hkv;
  const int b = w / a.hkv;

  int beg, P;
  const int np = seq_partitions(a, b, &beg, &P);
  if (p == 0 && kvh == 0 && lane == 0) {
    a.nparts[b] = np < 0 ? 0 : np;
    if (np < 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
  }
  if (p >= np) return;  // also covers np < 0
  const int L = a.seq[b];
  const int lo = beg + p * P;
  const int hi = min(L, lo + P);
  const int t_lo = lo >> 4;
  const int ntiles = ((hi + 15) >> 4) - t_lo;

  // B operand of the QK product: Q^T, lane (n, g4) holds head n, dims 8*(g4+4j) .. +7.
  bf16x8 qop[KS];
  {
    const bool hv = n < a.group;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + kvh * a.group + (hv ? n : 0)) * D);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      uint4 v = qrow[g4 + 4 * j];
      if (!hv) v = make_uint4(0u, 0u, 0u, 0u);
      qop[j] = as_bf16x8(v);
    }
  }

  const int64_t kchunk0 = (int64_t)kvh * (D / 8);
  const int64_t vrow0 = (int64_t)kvh * D;
  const int64_t kpart_bytes = (int64_t)a.hkv * a.bs * D * 2;
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;

  uint4 kb[NBUF][KS];
  uint2 vb[NBUF][VT];
  bool vld[NBUF];

  auto issue = [&](int slot, int tile_rel) {
    const int tok0 = (t_lo + tile_rel) << 4;
    const int blk = tok0 >> a.bs_shift;
    const int sub = tok0 & (a.bs - 1);
    const int32_t pid = trow[blk];
    vld[slot] = valid_block(a.rt, pid);
    const char* base = block_ptr(a.rt, pid);
#pragma unroll
    for (int j = 0; j < KS; ++j)
      kb[slot][j] = *reinterpret_cast<const uint4*>(
          base + ((((kchunk0 + g4 + 4 * j) << a.bs_shift) + sub + n) << 4));
#pragma unroll
    for (int t = 0; t < VT; ++t)
      vb[slot][t] = *reinterpret_cast<const uint2*>(
          base + kpart_bytes + ((((vrow0 + 16 * t + n) << a.bs_shift) + sub + 4 * g4) << 1));
  };

  f32x4 acc[VT];
#pragma unroll
  for (int t = 0; t < VT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;  // running max of this lane's head, log2 domain
  float lsum = 0.f;   // this lane's share of the running normaliser
  bool bad = false;

#pragma unroll
  for (int s = 0; s < NBUF - 1; ++s) issue(s, min(s, ntiles - 1));

  for (int it = 0; it < ntiles; it += NBUF) {
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      issue((s + NBUF - 1) % NBUF, min(it + s + NBUF - 1, ntiles - 1));
      if (it + s < ntiles) {
        const int tile = t_lo + it + s;
        bad |= !vld[s];
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[s][j]), qop[j], sacc, 0, 0, 0);
        // lane (n, g4), register i: token 16*tile + 4*g4 + i, head n
        const int tb = (tile << 4) + 4 * g4;
        float sv[4];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb + i;
          const bool ok = vld[s] && t >= lo && t < hi;
          sv[i] = ok ? sacc[i] * a.scale_log2 : kNegInf;
          mx = fmaxf(mx, sv[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float mref = mnew == kNegInf ? 0.f : mnew;
        const float alpha = exp2f(m - mref);
        const uint32_t p01 = pack_bf16x2(exp2f(sv[0] - mref), exp2f(sv[1] - mref));
        const uint32_t p23 = pack_bf16x2(exp2f(sv[2] - mref), exp2f(sv[3] - mref));
        // normalise with the same bf16-rounded weights the PV product uses
        lsum = lsum * alpha + ((bf16_to_f32(p01 & 0xffffu) + bf16_to_f32(p01 >> 16)) +
                               (bf16_to_f32(p23 & 0xffffu) + bf16_to_f32(p23 >> 16)));
        m = mnew;
        const i16x4 pop = as_i16x4(make_uint2(p01, p23));
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          acc[t] *= alpha;
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(vb[s][t]), pop, acc[t], 0, 0, 0);
        }
      }
    }
  }
  if (bad && lane == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (n < a.group) {
    const int h = kvh * a.group + n;
    const int64_t row = ((int64_t)b * a.hq + h) * a.max_parts + p;
    const float inv = 1.f / lsum;
    float* op = a.o_part + row * D;
#pragma unroll
    for (int t = 0; t < VT; ++t)
      *reinterpret_cast<f32x4*>(op + 16 * t + 4 * g4) = acc[t] * inv;
    if (g4 == 0) a.lse_part[row] = (m + log2f(lsum)) * kLn2;
  }
}

template <typename T>
__device__ __forceinline__ float load_elem(const char* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const float*>(p);
  } else {
    return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  }
}

// Plain VALU version: one token per lane for the scores, lanes over dims for P V.
template <typename T, int D>
__global__ __launch_bounds__(64) void gqa_decode_generic_kernel(DecodeArgs a) {
  constexpr int R = D / 64;                // dims per lane in the output
  constexpr int X = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  __shared__ float qs[16][D];
  const int lane = threadIdx.x;

  int w = blockIdx.x;
  const int p = w % a.grid_np;
  w /= a.grid_np;
  const int kvh = w % a.hkv;
  const int b = w / a.hkv;

  int beg, P;
  const int np = seq_partitions(a, b, &beg, &P);
  if (p == 0 && kvh == 0 && lane == 0) {
    a.nparts[b] = np < 0 ? 0 : np;
    if (np < 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
  }
  if (p >= np) return;
  const int L = a.seq[b];
  const int lo = beg + p * P;
  const int hi = min(L, lo + P);
  const int G = a.group;

  for (int h = 0; h < G; ++h) {
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.hq + kvh * G + h) * D;
    for (int d = lane; d < D; d += 64)
      qs[h][d] = load_elem<T>(reinterpret_cast<const char*>(qrow + d));
  }
  __syncthreads();

  const int64_t kpart_bytes = (int64_t)a.hkv * a.bs * D * (int64_t)sizeof(T);
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
  float m[16], l[16], acc[16][R], pr[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[h][r] = 0.f;
  }
  bool bad = false;

  for (int c0 = lo; c0 < hi; c0 += 64) {
    const int t = c0 + lane;
    const bool in = t < hi;
    const int32_t pid = in ? trow[t >> a.bs_shift] : 0;
    const bool ok = in && valid_block(a.rt, pid);
    bad |= in && !ok;
    const char* base = block_ptr(a.rt, pid);
    const int tt = t & (a.bs - 1);
    float s[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) s[h] = 0.f;
    if (ok) {
      for (int c = 0; c < D / X; ++c) {
        const char* kp = base + ((((int64_t)kvh * (D / X) + c) << a.bs_shift) + tt) * 16;
        for (int u = 0; u < X; ++u) {
          const float kv = load_elem<T>(kp + u * (int)sizeof(T));
#pragma unroll
          for (int h = 0; h < 16; ++h)
            if (h < G) s[h] += qs[h][c * X + u] * kv;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      if (h >= G) continue;
      const float sc = ok ? s[h] * a.scale : kNegInf;
      const float mnew = fmaxf(m[h], wave_max(sc));
      const float mref = mnew == kNegInf ? 0.f : mnew;
      const float alpha = expf(m[h] - mref);
      pr[h] = expf(sc - mref);
      l[h] = l[h] * alpha + wave_sum(pr[h]);
      m[h] = mnew;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[h][r] *= alpha;
    }
    const int cnt = min(64, hi - c0);
    for (int j = 0; j < cnt; ++j) {
      const bool okj = __shfl(ok ? 1 : 0, j) != 0;
      if (!okj) continue;
      const int32_t pidj = __shfl(pid, j);
      const int ttj = __shfl(tt, j);
      const char* vbase = block_ptr(a.rt, pidj) + kpart_bytes;
      float vv[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        vv[r] = load_elem<T>(vbase + ((((int64_t)kvh * D + lane + 64 * r) << a.bs_shift) + ttj) * (int64_t)sizeof(T));
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h >= G) continue;
        const float pj = __shfl(pr[h], j);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[h][r] += pj * vv[r];
      }
    }
  }
  if (__any(bad) && lane == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);

#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h >= G) continue;
    const int64_t row = ((int64_t)b * a.hq + kvh * G + h) * a.max_parts + p;
    float* op = a.o_part + row * D;
#pragma unroll
    for (int r = 0; r < R; ++r) op[lane + 64 * r] = acc[h][r] / l[h];
    if (lane == 0) a.lse_part[row] = m[h] + logf(l[h]);
  }
}

// ------------------------------------------------------------------ launchers
template <int D>
static hipError_t launch_mfma_d(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  constexpr int NBUF = D <= 128 ? 3 : 2;
  hipLaunchKernelGGL((gqa_decode_mfma_kernel<D, NBUF>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gqa_mfma(const DecodeArgs& a, int d, dim3 grid, hipStream_t st) {
  switch (d) {
    case 64: return launch_mfma_d<64>(a, grid, st);
    case 128: return launch_mfma_d<128>(a, grid, st);
    case 256: return launch_mfma_d<256>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_generic_t(const DecodeArgs& a, int d, dim3 grid, hipStream_t st) {
  switch (d) {
    case 64: hipLaunchKernelGGL((gqa_decode_generic_kernel<T, 64>), grid, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((gqa_decode_generic_kernel<T, 128>), grid, dim3(64), 0, st, a); break;
    case 256: hipLaunchKernelGGL((gqa_decode_generic_kernel<T, 256>), grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gqa_generic(const DecodeArgs& a, int d, bool f32, dim3 grid, hipStream_t st) {
  return f32 ? launch_generic_t<float>(a, d, grid, st) : launch_generic_t<uint16_t>(a, d, grid, st);
}

}  // namespace kvattn
