// Decode-attention partials for a shared latent cache (MLA), gfx950.
//
// With multi-head latent attention every head attends to the same compressed per-token
// latent: the absorbed query q_h (576 wide) is scored against the latent and the value is
// the latent's leading 512 columns, so decode reduces to a query-side projection and an
// output-side expansion around one shared latent, and each latent need be read from DRAM
// only once for all heads ("Physically Partitioned KVCache Format for CPU-GPU Load Balancing
// in MoE Inference", §6.1, compressed-MLA variant).
//
// One workgroup of 4 waves (one per SIMD, so each wave may hold up to 512 registers) per
// (sequence, group of partitions), walking the group's 64-token blocks ("stages") in order:
//   1. wave w loads the latent rows of tokens 16w .. 16w+15 of a stage straight into
//      registers with 16-byte non-temporal loads (the latent is read once per step) -- lane
//      (n, g4) holds token n, 16-byte chunks g4 + 4j -- into a ring of kRing stages; a slot
//      is refilled as soon as its stage's rows are in LDS (step 3), so kRing stages
//      (3 x 72 KiB per CU) are in flight through the softmax and PV of the current one;
//   2. the same registers are the A operand of the scores S^T = C Q^T on the matrix cores
//      (v_mfma_f32_16x16x32_bf16, 18 k-steps over the 576 dims, heads in the N columns; the
//      Q^T operand is read from LDS, leaving the registers to the ring);
//   3. the value part (chunks 0..63) is written to LDS with an XOR swizzle
//      (slot(c, t) = c*64 + (t ^ (c & 15)) for chunk c of token t, conflict-free for this
//      write and for the transposed read below), and the scores to LDS;
//   4. after one barrier every wave reads all 64 x 16 scores, updates the running max /
//      normaliser and forms the bf16 P^T operands, then accumulates O^T for its 128 output
//      dims, V^T P^T with v_mfma_f32_16x16x32_bf16 (two 32-token k-steps per stage), reading
//      8-token x 8-dim patches of the value part from LDS and regrouping them in registers
//      with byte permutes.
// The swizzle only touches the low 4 token bits, so all LDS addresses are a few per-lane bases
// plus immediate offsets; computing those bases once keeps ~100 registers free for the ring.
// LDS (values and scores) is double-buffered by stage parity, so one barrier per stage
// orders both the writes of a stage before its reads and the reads of the previous use of
// a buffer before its next writes.

#include "device_common.h"

namespace kvattn {

static constexpr float kNegInfM = -__builtin_huge_valf();
static constexpr float kLn2M = 0.693147180559945309f;

static constexpr int kMlaDk = 576;
static constexpr int kMlaDv = 512;
static constexpr int kMlaChunks = kMlaDk / 8;   // 72 chunks of 8 bf16
static constexpr int kMlaVChunks = kMlaDv / 8;  // 64 chunks hold the value part
static constexpr int kMlaKs = kMlaChunks / 4;   // 18 k-steps of the score product
static constexpr int kMlaBs = 64;
static constexpr int kRing = 3;                 // stages held in registers per wave
static constexpr int kWin = 128;                // stages whose block ids a window holds

__device__ __forceinline__ int lat_slot(int c, int t) { return c * kMlaBs + (t ^ (c & 15)); }

__global__ __launch_bounds__(256, 1) void mla_decode_kernel(DecodeArgs a) {
  __shared__ uint4 vlat[2][kMlaVChunks * kMlaBs];  // value part of a stage: 2 x 64 KiB
  __shared__ float sx[2][kMlaBs][16];             // scores of a stage, [token][head]
  __shared__ uint4 qs[kMlaKs * 64];                // Q^T operand, [k-step][lane]
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
  if (wv == 0) {
    const bool hv = n < a.hq;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + (hv ? n : 0)) * kMlaDk);
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j) {
      uint4 v = qrow[g4 + 4 * j];
      if (!hv) v = make_uint4(0u, 0u, 0u, 0u);
      qs[j * 64 + lane] = v;
    }
  }
  __syncthreads();

  // Register ring of latent rows: stage s lives in slot s % kRing.  It starts zeroed, so a
  // slot never loaded (short groups) is finite; its scores are masked anyway.
  u32x4 kb[kRing][kMlaKs];
  bool vld[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    vld[r] = false;
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j) kb[r][j] = u32x4{0u, 0u, 0u, 0u};
  }
  // lane (n, g4) of wave w: token 16w + n, chunk g4 + 4j at byte ((g4 + 4j) * 64 + token) * 16.
  // Stage s is loaded into slot s % kRing.  The main loop passes only stages of the group
  // (guard = false), so every stage issues the same loads and the compiler's wait counts stay
  // exact (a conditional load anywhere in the loop would make it wait for all outstanding
  // loads, the prefetch included); the prologue's loads past a short group re-read its last
  // block (clamped, harmless), the last round skips them.
  const uint32_t loff = (uint32_t)((g4 * kMlaBs + 16 * wv + n) * 16);
  // The stages are walked in windows of up to kWin; the window's block ids are read once into
  // two registers per lane (lane i: stages i and 64 + i of the window) and picked out with
  // lane reads.  A table load per stage would make every stage wait for all outstanding
  // loads (the load counter drains in order), prefetch included.
  int w0 = 0, wn = 0, pid0 = 0, pid1 = 0;
  auto issue = [&](int slot, int s, bool guard) {
    if (guard && s >= wn) return;
    const int r = min(s, wn - 1);
    const int32_t pa = __builtin_amdgcn_readlane(pid0, r & 63);
    const int32_t pb = __builtin_amdgcn_readlane(pid1, r & 63);
    const int32_t pid = r < 64 ? pa : pb;
    const bool ok = valid_block(a.rt, pid);
    vld[slot] = ok;
    gchar* base = block_addr(a.rt, ok ? pid : 0) + loff;
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j)
      kb[slot][j] = __builtin_nontemporal_load(reinterpret_cast<gu32x4*>(base + j * (4 * kMlaBs * 16)));
  };

  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInfM, lsum = 0.f;
  bool bad = false;
  // LDS slots (16-byte units within a value buffer): the value-part write of chunk g4 + 4j
  // is wslot[j % 4] + (j / 4) * 1024, the transposed read of chunk 16 wv + n, token
  // 32 kk + 8 g4 + i is rslot[i] + 32 kk (the swizzle only touches the low 4 token bits)
  int wslot[4], rslot[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) wslot[q] = lat_slot(g4 + 4 * q, 16 * wv + n);
#pragma unroll
  for (int i = 0; i < 8; ++i) rslot[i] = lat_slot(16 * wv + n, 8 * g4 + i);

  // One stage: compute stage s from slot r; the slot is refilled with stage s + kRing as soon
  // as its rows are in LDS, so kRing stages stay in flight through the softmax and PV.
  auto stage = [&](int r, int s, bool guard) {
    const int buf = s & 1;
    uint4* vbuf = vlat[buf];
    bad |= !vld[r];

    // 2. scores of tokens 16*wv .. +15 from the registers
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[r][j]), as_bf16x8(qs[j * 64 + lane]), sacc, 0, 0, 0);

    // 3. value part and scores to LDS.  In a stage not wholly inside the range (or of an
    //    invalid block) the outside token slots may hold anything, NaN bit patterns included,
    //    and a zero weight does not cancel a NaN in the PV product: their values are zeroed.
    //    The zeros overwrite the lane's own slots just before the barrier, later in its
    //    program order; in most stages no lane needs them and the branch skips them.
#pragma unroll
    for (int j = 0; j < kMlaVChunks / 4; ++j)
      vbuf[(j >> 2) * 1024 + wslot[j & 3]] = __builtin_bit_cast(uint4, kb[r][j]);
    const int tbase = (st_lo + w0 + s) << 6;
    const int tok = tbase + 16 * wv + n;
    const bool zero_tok = !(vld[r] & (tok >= lo) & (tok < hi));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = 16 * wv + 4 * g4 + i;
      const int t = tbase + tl;
      const bool ok = vld[r] & (t >= lo) & (t < hi);
      sx[buf][tl][n] = ok ? sacc[i] * a.scale_log2 : kNegInfM;
    }
    issue(r, s + kRing, guard);
    if (zero_tok) {
#pragma unroll
      for (int j = 0; j < kMlaVChunks / 4; ++j)
        vbuf[(j >> 2) * 1024 + wslot[j & 3]] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    // 4a. softmax update over the 64 tokens, all waves alike; lane (n, g4) takes head n's
    //     scores of tokens 32*kk + 8*g4 + i (i < 8), the k-slots of the PV product below
    float sv[2][8];
    float mx = kNegInfM;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[kk][i] = sx[buf][32 * kk + 8 * g4 + i][n];
        mx = fmaxf(mx, sv[kk][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float mref = mnew == kNegInfM ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    m = mnew;
    u32x4 pop[2];
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t p = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kk][2 * j] - mref),
                                       __builtin_amdgcn_exp2f(sv[kk][2 * j + 1] - mref));
        // the normaliser sums the bf16 weights the PV product uses
        part += bf16_to_f32(p & 0xffffu) + bf16_to_f32(p >> 16);
        pop[kk][j] = p;
      }
    lsum = lsum * alpha + part;

    // 4b. O^T for dims 8*c + e, c = 16*wv + row (row = MFMA row), e = 0..7: per 32-token
    //     k-step, lane (row, g4) reads chunk c of its 8 tokens and regroups the 8 x 8 bf16
    //     values dim-major with byte permutes, one v_mfma_f32_16x16x32_bf16 per e
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 r8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r8[i] = vbuf[32 * kk + rslot[i]];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // dims 8c + 2q (low halves) and 8c + 2q + 1 (high halves) of the 8 tokens
        u32x4 lo_op, hi_op;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = reinterpret_cast<const uint32_t*>(&r8[2 * j])[q];
          const uint32_t y = reinterpret_cast<const uint32_t*>(&r8[2 * j + 1])[q];
          lo_op[j] = (x & 0xffffu) | (y << 16);
          hi_op[j] = (x >> 16) | (y & 0xffff0000u);
        }
        acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo_op), as_bf16x8(pop[kk]), acc[2 * q], 0, 0, 0);
        acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi_op), as_bf16x8(pop[kk]), acc[2 * q + 1], 0, 0, 0);
      }
    }
  };

  // Each window fills the ring, runs, and drains it; kWin is even, so the LDS buffer parity
  // s & 1 of a window's stage s is that of the group's stage w0 + s.
  for (; w0 < nst; w0 += kWin) {
    wn = min(kWin, nst - w0);
    pid0 = trow[st_lo + w0 + min(lane, wn - 1)];
    pid1 = trow[st_lo + w0 + min(64 + lane, wn - 1)];
#pragma unroll
    for (int r = 0; r < kRing; ++r) issue(r, r, false);
    int it = 0;
    for (; it + 2 * kRing <= wn; it += kRing) {  // every refill inside the window
#pragma unroll
      for (int r = 0; r < kRing; ++r) stage(r, it + r, false);
    }
    for (; it < wn; it += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r)
        if (it + r < wn) stage(r, it + r, true);  // uniform over the workgroup
    }
  }
  if (bad && lane == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);

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
