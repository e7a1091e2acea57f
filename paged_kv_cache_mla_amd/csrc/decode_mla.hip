// Decode-attention partials for a shared latent cache (MLA), gfx950.
//
// With multi-head latent attention every head attends to the same compressed per-token
// latent: the absorbed query q_h (576 wide) is scored against the latent and the value is
// the latent's leading 512 columns, so decode reduces to a query-side projection and an
// output-side expansion around one shared latent, and each latent need be read from DRAM
// only once for all heads ("Physically Partitioned KVCache Format for CPU-GPU Load Balancing
// in MoE Inference", §6.1, compressed-MLA variant).
//
// One workgroup of 8 waves per (sequence, group of partitions), in two teams of 4 waves, walks
// the group's 64-token blocks ("stages"): team 0 takes the even stages, team 1 the odd ones,
// each with its own online softmax, and the two teams' states are merged exactly at the end.
// Each team has its own LDS tile; the teams run half a stage apart, so that on every SIMD one
// wave scores and stages its rows while the other runs its softmax and PV product (two waves
// per SIMD hide each other's MFMA and LDS latencies).  Per stage, in a team:
//   1. wave w of the team loads the latent rows of tokens 16w .. 16w+15 of its next stage
//      straight into registers with 16-byte non-temporal loads (the latent is read once per
//      step) -- lane (n, g4) holds token n, 16-byte chunks g4 + 4j -- issued as soon as the
//      current stage's rows are in LDS, so each load has two steps to land;
//   2. the same registers are the A operand of the scores S^T = C Q^T on the matrix cores
//      (v_mfma_f32_16x16x32_bf16, 18 k-steps over the 576 dims, heads in the N columns; the
//      Q^T operand is read from LDS, leaving the registers to the loads);
//   3. the value part (chunks 0..63) is written to the team's LDS tile with an XOR swizzle
//      (slot(c, t) = c*64 + (t ^ (c & 15)) for chunk c of token t, conflict-free for this
//      write and for the transposed read below), and the scores to LDS;
//   4. after a barrier every wave of the team reads all 64 x 16 scores, updates its running
//      max / normaliser and forms the bf16 P^T operands, then accumulates O^T for its 128
//      output dims, V^T P^T with v_mfma_f32_16x16x32_bf16 (two 32-token k-steps per stage),
//      reading 8-token x 8-dim patches of the value part from LDS and regrouping them in
//      registers with byte permutes.
// Steps are separated by one workgroup barrier: at step t team 0 runs phase 1-3 of its
// stage t/2 (t even) or phase 4 (t odd), team 1 the same one step later.  A team writes its
// tile in one step and reads it in the next, and the barrier between orders both the writes
// before the reads and the reads before the team's next writes.
// The swizzle only touches the low 4 token bits, so all LDS addresses are a few per-lane bases
// plus immediate offsets.

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
static constexpr int kTeams = 2;
static constexpr int kWin = 128;                // stages whose block ids a window holds (even)

__device__ __forceinline__ int lat_slot(int c, int t) { return c * kMlaBs + (t ^ (c & 15)); }

// PROBE: the same grid, waves and loads with no arithmetic, LDS traffic or barriers: each wave
// XORs the in-range 16-bit latent elements it loads and folds them into xsum[b] (the gather's
// own bandwidth ceiling, and a checksum).
template <bool PROBE>
__global__ __launch_bounds__(512, 1) void mla_decode_kernel(DecodeArgs a, uint32_t* xsum) {
  __shared__ uint4 vlat[kTeams][kMlaVChunks * kMlaBs];  // value part of a team's stage: 2 x 64 KiB
  __shared__ float sx[kTeams][kMlaBs][16];              // scores of a team's stage, [token][head]
  __shared__ uint4 qs[kMlaKs * 64];                     // Q^T operand, [k-step][lane]
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int team = wv >> 2;
  const int ww = wv & 3;  // place in the team: tokens 16 ww .. +15, output chunks 16 ww .. +15
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g4 = lane >> 4;

  // one workgroup per (sequence, group of group_parts partitions); each team walks its
  // blocks of the group in order, its online softmax continuing across partition boundaries
  const int k = blockIdx.x % a.grid_ng;
  const int b = blockIdx.x / a.grid_ng;
  int beg, P, ng;
  const int np = seq_partitions(a, b, &beg, &P, &ng);
  if (k == 0 && tid == 0) {
    if (!PROBE) a.nparts[b] = ng < 0 ? 0 : ng;
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

  // The wave's latent rows of the team's next stage.  They start zeroed, so a stage never
  // loaded is finite; its scores are masked anyway.
  u32x4 kb[kMlaKs];
  bool vld = false;
#pragma unroll
  for (int j = 0; j < kMlaKs; ++j) kb[j] = u32x4{0u, 0u, 0u, 0u};
  // lane (n, g4) of team wave ww: token 16ww + n, chunk g4 + 4j at byte ((g4 + 4j) * 64 +
  // token) * 16.  The stages are walked in windows of up to kWin; the window's block ids are
  // read once into two registers per lane (lane i: stages i and 64 + i of the window) and
  // picked out with lane reads, so no table load waits inside the loop.
  const uint32_t loff = (uint32_t)((g4 * kMlaBs + 16 * ww + n) * 16);
  int w0 = 0, wn = 0, pid0 = 0, pid1 = 0;
  auto issue = [&](int s) {  // window-relative stage s < wn (uniform over the wave)
    const int32_t pa = __builtin_amdgcn_readlane(pid0, s & 63);
    const int32_t pb = __builtin_amdgcn_readlane(pid1, s & 63);
    const int32_t pid = s < 64 ? pa : pb;
    const bool ok = valid_block(a.rt, pid);
    vld = ok;
    gchar* base = block_addr(a.rt, ok ? pid : 0) + loff;
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j)
      kb[j] = __builtin_nontemporal_load(reinterpret_cast<gu32x4*>(base + j * (4 * kMlaBs * 16)));
  };

  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInfM, lsum = 0.f;
  bool bad = false;
  uint4* vbuf = vlat[team];
  float (*sxt)[16] = sx[team];
  // LDS slots (16-byte units within a value tile): the value-part write of chunk g4 + 4j is
  // wslot[j % 4] + (j / 4) * 1024, the transposed read of chunk 16 ww + n, token
  // 32 kk + 8 g4 + i is rslot[i] + 32 kk (the swizzle only touches the low 4 token bits)
  int wslot[4], rslot[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) wslot[q] = lat_slot(g4 + 4 * q, 16 * ww + n);
#pragma unroll
  for (int i = 0; i < 8; ++i) rslot[i] = lat_slot(16 * ww + n, 8 * g4 + i);

  // Phases 1-3 of window-relative stage s: scores from the registers, value part and scores
  // to the team's tile, then the registers are refilled with the team's next stage.
  uint32_t xs = 0u;
  auto score_stage = [&](int s) {
    bad |= !vld;
    if constexpr (PROBE) {
      const int tok = ((st_lo + w0 + s) << 6) + 16 * ww + n;
      const bool ok = vld & (tok >= lo) & (tok < hi);
#pragma unroll
      for (int j = 0; j < kMlaKs; ++j) xs ^= ok ? (kb[j][0] ^ kb[j][1] ^ kb[j][2] ^ kb[j][3]) : 0u;
      if (s + kTeams < wn) issue(s + kTeams);
      return;
    }
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[j]), as_bf16x8(qs[j * 64 + lane]), sacc, 0, 0, 0);

    // In a stage not wholly inside the range (or of an invalid block) the outside token slots
    // may hold anything, NaN bit patterns included, and a zero weight does not cancel a NaN in
    // the PV product: their values are zeroed.  The zeros overwrite the lane's own slots later
    // in its program order; in most stages no lane needs them and the branch skips them.
#pragma unroll
    for (int j = 0; j < kMlaVChunks / 4; ++j)
      vbuf[(j >> 2) * 1024 + wslot[j & 3]] = __builtin_bit_cast(uint4, kb[j]);
    const int tbase = (st_lo + w0 + s) << 6;
    const int tok = tbase + 16 * ww + n;
    const bool cur = vld;
    const bool zero_tok = !(cur & (tok >= lo) & (tok < hi));
    if (s + kTeams < wn) issue(s + kTeams);  // the registers are free once the rows are in LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = 16 * ww + 4 * g4 + i;
      const int t = tbase + tl;
      const bool ok = cur & (t >= lo) & (t < hi);
      sxt[tl][n] = ok ? sacc[i] * a.scale_log2 : kNegInfM;
    }
    if (zero_tok) {
#pragma unroll
      for (int j = 0; j < kMlaVChunks / 4; ++j)
        vbuf[(j >> 2) * 1024 + wslot[j & 3]] = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  // Phase 4: softmax update over the stage's 64 tokens and the PV product, from the team's tile.
  auto attend_stage = [&]() {
    if constexpr (PROBE) return;
    // lane (n, g4) takes head n's scores of tokens 32*kk + 8*g4 + i (i < 8), the k-slots of
    // the PV product below
    float sv[2][8];
    float mx = kNegInfM;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[kk][i] = sxt[32 * kk + 8 * g4 + i][n];
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

    // O^T for dims 8*c + e, c = 16*ww + row (row = MFMA row), e = 0..7: per 32-token k-step,
    // lane (row, g4) reads chunk c of its 8 tokens and regroups the 8 x 8 bf16 values
    // dim-major with byte permutes, one v_mfma_f32_16x16x32_bf16 per e
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

  // Step t of a window: team 0 runs phases 1-3 of its stage t/2 (t even) or phase 4 (t odd);
  // team 1 does the same one step later.  Every wave passes every barrier (the step count is
  // uniform over the workgroup).
  // The first window's block ids and loads are issued before the barrier that publishes Q^T,
  // so their latency overlaps the Q load.
  auto open_window = [&]() {
    wn = min(kWin, nst - w0);
    pid0 = trow[st_lo + w0 + min(lane, wn - 1)];
    pid1 = trow[st_lo + w0 + min(64 + lane, wn - 1)];
    if (team < wn) issue(team);
  };
  // Q^T operand (B of the QK product): head n, dims 8*(g4+4j) .. +7.  The first wave of team 1
  // loads it (team 1 scores its first stage one step after team 0, so the later start of its
  // own loads costs nothing), into registers before its loads of the latent rows.
  constexpr int kQWave = 4;
  const bool hv = n < a.hq;
  uint4 qv[kMlaKs];
  if (wv == kQWave && !PROBE) {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + (hv ? n : 0)) * kMlaDk);
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j) qv[j] = qrow[g4 + 4 * j];
  }
  open_window();
  if (wv == kQWave && !PROBE) {
#pragma unroll
    for (int j = 0; j < kMlaKs; ++j) qs[j * 64 + lane] = hv ? qv[j] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (!PROBE) __syncthreads();

  for (; w0 < nst; w0 += kWin) {
    if (w0 > 0) open_window();
    const int n0 = (wn + 1) >> 1, n1 = wn >> 1;  // stages of teams 0 and 1 in the window
    const int steps = max(2 * n0, 2 * n1 + 1);
    for (int t = 0; t < steps; ++t) {
      const int rel = t - team;
      const int s = 2 * (rel >> 1) + team;
      if (rel >= 0 && s < wn) {  // uniform over the wave
        if ((rel & 1) == 0)
          score_stage(s);
        else
          attend_stage();
      }
      if (!PROBE) __syncthreads();
    }
  }
  if (bad && lane == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);
  if constexpr (PROBE) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) xs ^= __shfl_xor(xs, o);
    if (lane == 0) atomicXor(xsum + b, (xs ^ (xs >> 16)) & 0xffffu);
    return;
  }

  // Exact merge of the two teams' states (log2 domain): team 1 hands its running max, sum and
  // unnormalised output through LDS (the value tiles are free after the last barrier); wave
  // ww of team 0 holds the same heads and output dims in the same lanes.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  float* tb = reinterpret_cast<float*>(vlat[0]) + ww * 34 * 64 + lane;  // [ww][34][lane]
  if (team == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) tb[(4 * e + i) * 64] = acc[e][i];
    tb[32 * 64] = m;
    tb[33 * 64] = lsum;
  }
  __syncthreads();
  if (team == 1) return;
  {
    const float mb = tb[32 * 64];
    const float lb = tb[33 * 64];
    const float mnew = fmaxf(m, mb);
    const float mref = mnew == kNegInfM ? 0.f : mnew;
    const float ca = __builtin_amdgcn_exp2f(m - mref);
    const float cb = __builtin_amdgcn_exp2f(mb - mref);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[e][i] = acc[e][i] * ca + tb[(4 * e + i) * 64] * cb;
    lsum = lsum * ca + lb * cb;
    m = mnew;
  }
  if (n < a.hq) {
    const int64_t row = ((int64_t)b * a.hq + n) * a.max_parts + k;
    // a group with no weight (every block invalid) writes o = 0 beside lse = -inf
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* op = a.o_part + row * kMlaDv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // output row 4*g4 + i of every tile e is chunk 16*ww + 4*g4 + i, dim offset e
      const int cc = 16 * ww + 4 * g4 + i;
      const f32x4 v0 = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]} * inv;
      const f32x4 v1 = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]} * inv;
      *reinterpret_cast<f32x4*>(op + 8 * cc) = v0;
      *reinterpret_cast<f32x4*>(op + 8 * cc + 4) = v1;
    }
    if (ww == 0 && g4 == 0) a.lse_part[row] = (m + log2f(lsum)) * kLn2M;
  }
}

hipError_t launch_mla(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(mla_decode_kernel<false>, grid, dim3(512), 0, st, a, nullptr);
  return hipGetLastError();
}

hipError_t launch_mla_probe(const DecodeArgs& a, dim3 grid, uint32_t* xsum, hipStream_t st) {
  hipLaunchKernelGGL(mla_decode_kernel<true>, grid, dim3(512), 0, st, a, xsum);
  return hipGetLastError();
}

}  // namespace kvattn
