// Decode-attention partials for a shared latent cache (MLA), gfx950.
//
// With multi-head latent attention every head attends to the same compressed per-token
// latent: the absorbed query q_h (576 wide) is scored against the latent and the value is
// the latent's leading 512 columns, so decode reduces to a query-side projection and an
// output-side expansion around one shared latent, and each latent need be read from DRAM
// only once for all heads ("Physically Partitioned KVCache Format for CPU-GPU Load Balancing
// in MoE Inference", §6.1, compressed-MLA variant).  Here that reuse is staged in LDS:
//
//   one workgroup of 4 waves per (sequence, partition); per 64-token block
//   1. the block's 72 KiB latent is fetched with fully coalesced 16-byte non-temporal loads
//      (read once per step; prefetched one block ahead in registers) and written to LDS with
//      an XOR swizzle
//      (slot(c, t) = c*64 + (t ^ (c & 15)) for 16-byte chunk c of token t);
//   2. wave w scores tokens 16w..16w+15 against all 16 heads on the matrix cores,
//      S^T = C Q^T with v_mfma_f32_16x16x32_bf16 (18 k-steps over 576 dims), and posts the
//      scores to LDS;
//   3. every wave reads all 64 x 16 scores, updates the running max / normaliser and forms
//      the bf16 P^T operands itself (one barrier, no second exchange);
//   4. wave w accumulates O^T for its 128 output dims, V^T P^T with
//      v_mfma_f32_16x16x16_bf16, reading 4-token x 8-dim patches of the latent from LDS and
//      regrouping them in registers with byte permutes.
// The swizzle makes both LDS read patterns (token-major for QK, chunk-major for PV) and the
// write pattern free of bank conflicts.

#include "device_common.h"

namespace kvattn {

static constexpr float kNegInfM = -__builtin_huge_valf();
static constexpr float kLn2M = 0.693147180559945309f;

static constexpr int kMlaDk = 576;
static constexpr int kMlaDv = 512;
static constexpr int kMlaChunks = kMlaDk / 8;  // 72 chunks of 8 bf16
static constexpr int kMlaBs = 64;
static constexpr int kMlaLoads = kMlaChunks * kMlaBs / 256;  // 16-byte loads per thread: 18

__device__ __forceinline__ int lat_slot(int c, int t) { return c * kMlaBs + (t ^ (c & 15)); }

__global__ __launch_bounds__(256, 2) void mla_decode_kernel(DecodeArgs a) {
  __shared__ uint4 lat[kMlaChunks * kMlaBs];  // 73,728 B
  __shared__ float sx[kMlaBs][16];            // scores of the stage, [token][head]
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g4 = lane >> 4;

  // one workgroup per (sequence, group of group_parts partitions); the group's partitions
  // are walked in order, the online softmax continuing across their boundaries
  const int k = blockIdx.x % a.grid_ng;
  const int b = blockIdx.x / a.grid_ng;
  int beg, P, ng;
  const int np = seq_partitions(a, b, &beg, &P, &ng);
  if (k == 0 && tid == 0) {
    a.nparts[b] = ng < 0 ? 0 : ng;
    if (np < 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
  }
  if (k >= ng) return;
  const int L = a.seq[b];
  const int64_t span = (int64_t)P * a.group_parts;
  const int lo = (int)(beg + k * span);
  const int hi = (int)min((int64_t)L, lo + span);
  const int st_lo = lo >> 6;
  const int nst = ((hi + kMlaBs - 1) >> 6) - st_lo;
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;

  // Q^T operand (B of the QK product): head n, dims 8*(g4+4j) .. +7.
  bf16x8 qop[kMlaChunks / 4];
  {
    const bool hv = n < a.hq;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + (hv ? n : 0)) * kMlaDk);
#pragma unroll
    for (int j = 0; j < kMlaChunks / 4; ++j) {
      uint4 v = qrow[g4 + 4 * j];
      if (!hv) v = make_uint4(0u, 0u, 0u, 0u);
      qop[j] = as_bf16x8(v);
    }
  }

  uint4 stage[kMlaLoads];
  bool vld_next = true;
  auto fetch = [&](int st_rel) {
    const int32_t pid = trow[st_lo + st_rel];
    vld_next = valid_block(a.rt, pid);
    gu32x4* src = reinterpret_cast<gu32x4*>(block_addr(a.rt, vld_next ? pid : 0));
#pragma unroll
    for (int r = 0; r < kMlaLoads; ++r)
      stage[r] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(src + r * 256 + tid));
  };

  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInfM, lsum = 0.f;
  bool bad = false;

  fetch(0);
  for (int s = 0; s < nst; ++s) {
    const bool vld = vld_next;
    bad |= !vld;
    __syncthreads();  // previous stage's LDS reads are done
#pragma unroll
    for (int r = 0; r < kMlaLoads; ++r) {
      const int q = r * 256 + tid;  // chunk q / 64, token q % 64
      lat[lat_slot(q >> 6, q & 63)] = stage[r];
    }
    if (s + 1 < nst) fetch(s + 1);  // nothing is fetched past the partition
    __syncthreads();  // latent of this stage visible

    // 2. scores of tokens 16*wv .. +15
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tok = 16 * wv + n;
#pragma unroll
    for (int j = 0; j < kMlaChunks / 4; ++j) {
      const int c = g4 + 4 * j;
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lat[lat_slot(c, tok)]), qop[j], sacc, 0, 0, 0);
    }
    const int tbase = ((st_lo + s) << 6);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = 16 * wv + 4 * g4 + i;
      const int t = tbase + tl;
      const bool ok = vld && t >= lo && t < hi;
      sx[tl][n] = ok ? sacc[i] * a.scale_log2 : kNegInfM;
    }
    __syncthreads();

    // 3. softmax update over the 64 tokens, all waves alike
    float sv[4][4];
    float mx = kNegInfM;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[ks][i] = sx[16 * ks + 4 * g4 + i][n];
        mx = fmaxf(mx, sv[ks][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float mref = mnew == kNegInfM ? 0.f : mnew;
    const float alpha = exp2f(m - mref);
    m = mnew;
    i16x4 pop[4];
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t p01 = pack_bf16x2(exp2f(sv[ks][0] - mref), exp2f(sv[ks][1] - mref));
      const uint32_t p23 = pack_bf16x2(exp2f(sv[ks][2] - mref), exp2f(sv[ks][3] - mref));
      part += (bf16_to_f32(p01 & 0xffffu) + bf16_to_f32(p01 >> 16)) +
              (bf16_to_f32(p23 & 0xffffu) + bf16_to_f32(p23 >> 16));
      pop[ks] = as_i16x4(make_uint2(p01, p23));
    }
    lsum = lsum * alpha + part;

    // 4. O^T for dims 8*c + e, c = 16*wv + row (row = MFMA row), e = 0..7
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    const int c = 16 * wv + n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 r4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r4[i] = lat[lat_slot(c, 16 * ks + 4 * g4 + i)];
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r4[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r4[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r4[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r4[3]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // dims 8c + 2k (low halves) and 8c + 2k + 1 (high halves) of the 4 tokens
        const uint2 lo_op = make_uint2((w0[k] & 0xffffu) | (w1[k] << 16), (w2[k] & 0xffffu) | (w3[k] << 16));
        const uint2 hi_op = make_uint2((w0[k] >> 16) | (w1[k] & 0xffff0000u), (w2[k] >> 16) | (w3[k] & 0xffff0000u));
        acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(lo_op), pop[ks], acc[2 * k], 0, 0, 0);
        acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(hi_op), pop[ks], acc[2 * k + 1], 0, 0, 0);
      }
    }
  }
  if (bad && tid == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (n < a.hq) {
    const int64_t row = ((int64_t)b * a.hq + n) * a.max_parts + k;
    const float inv = 1.f / lsum;
    float* op = a.o_part + row * kMlaDv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // output row 4*g4 + i of every tile e is chunk 16*wv + 4*g4 + i, dim offset e
      const int cc = 16 * wv + 4 * g4 + i;
      const f32x4 v0 = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]} * inv;
      const f32x4 v1 = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]} * inv;
      *reinterpret_cast<f32x4*>(op + 8 * cc) = v0;
      *reinterpret_cast<f32x4*>(op + 8 * cc + 4) = v1;
    }
    if (wv == 0 && g4 == 0) a.lse_part[row] = (m + log2f(lsum)) * kLn2M;
  }
}

hipError_t launch_mla(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(mla_decode_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvattn
