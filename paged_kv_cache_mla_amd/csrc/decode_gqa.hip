// Decode-attention partials for per-head K/V caches (GQA), gfx950.
//
// Computes, for one (sequence, KV head, partition), the partial attention of the query heads
// sharing that KV head over the partition's tokens, with an online softmax (running max and
// normaliser, fp32 accumulation) -- "Physically Partitioned KVCache Format for CPU-GPU Load
// Balancing in MoE Inference", §6.1 -- and emits (o normalised by its own sum, lse) so that
// partials of disjoint token ranges merge exactly (same page, §5.1).
//
// Work items are groups of `group_parts` consecutive partitions of one (sequence, KV head);
// one partial is written per group (with group_parts = 1, one per partition).
//
// Two kernels:
//  * gqa_decode_mfma_kernel (bf16, block size >= 16): one workgroup per group, one or two
//    consecutive partitions per wave.  Each 16-token tile is a dense contraction on the matrix cores:
//    S^T[16 tok x 16 heads] = K Q^T with v_mfma_f32_16x16x32_bf16 (query heads of the group
//    in the N columns, padded to 16), then, per pair of tiles, O^T[D x 16 heads] += V^T P^T,
//    also 16x16x32.  The block layout makes both operands plain 16-byte / 8-byte per-lane
//    loads straight from HBM: K is stored in 16-byte chunks with the chunks of consecutive
//    tokens side by side (one k-step of one tile is 1 KiB contiguous), V is stored transposed
//    (one 16-dim slice of a tile is 512 B contiguous).  The MFMA output layout of S^T (lane =
//    head column, 4 consecutive tokens per lane) is exactly the B-operand layout the PV
//    product needs, so no data moves between lanes except two lane swaps for the per-head
//    max.  The next pair of tiles is prefetched into registers while the current pair is
//    computed.  K and V are read once per step, so their loads carry the non-temporal hint,
//    unless the pool holds blocks shared by several sequences (prefix sharing): then plain,
//    cache-retaining loads let the sharing sequences reuse those blocks from L2 / MALL.
//    The waves' partials (o, lse) go to LDS and are merged there exactly, by the same LSE
//    rescaling as the merge kernel, before one partial per group is written: writes of
//    partial outputs are expensive while the read stream is running (on MI355X, 16.9 MB of
//    partials written next to the 1 GiB of 16 x 32K K/V cost ~16 us, ~8% of the step), and
//    the group merge divides them by group_parts.
//  * gqa_decode_generic_kernel (fp32 or bf16, any block size): a plain VALU version, four
//    waves per group taking its 64-token chunks in turn, merged exactly at the end; used for
//    fp32 caches and block sizes below 16, and as an independent cross-check of the MFMA
//    kernel.

#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "plan_layout.h"

namespace kvattn {

static constexpr float kNegInf = -__builtin_huge_valf();
static constexpr float kLn2 = 0.693147180559945309f;

// Growth of a head's running max (log2 domain) tolerated before the accumulators are
// rescaled: the unnormalised weights then stay below 2^8, well inside fp32 / bf16 range, and
// the rescale (a pass over every accumulator) happens only a few times per partition.
static constexpr float kRescaleSlack = 8.f;

// Largest workgroup (waves = partitions merged on chip) of the matrix-core kernel for head
// dim D: the waves of one group must fit on one CU at the kernel's register use.
template <int D>
constexpr int mfma_max_group() { return D <= 64 ? 16 : 8; }

// Partial of the token range [lo, hi) of table row `trow` (one or more consecutive
// partitions, spanning at most 64 * NWIN blocks: the wave keeps their ids in NWIN 64-lane
// registers) for the query heads of KV head kvh, on the calling wave.  MFMA column n (lane
// n, n + 16, ...) takes the query row `qrow` if `qvalid`, else zeros: the heads of one
// sequence's group, or the heads of several sequences holding the same blocks.  On return
// lane (n, g4) holds, for column n: acc[t] = unnormalised output dims 16t + 4*g4 .. +3,
// m = reference max (log2 domain), lsum = its share of the normaliser (to be summed over the
// four lane rows).
//
// Tiles are consumed in pairs.  For a pair (A, B) the PV product is one
// v_mfma_f32_16x16x32_bf16 per 16-dim output tile with k-slot (g4, i) = token 4*g4 + i of A
// for i < 4 and of B for i >= 4: the A operand is then just the two tiles' 8-byte V^T slices
// side by side, and the B operand the two tiles' score-layout weights side by side.  The
// weights enter as a bf16 pair hi + lo (hi = bf16(p), lo = bf16(p - hi)), two MFMAs per
// output tile, so P V is accurate to ~2^-16 relative rather than bf16's 2^-9.
// PROBE: the same loads in the same order, with no arithmetic: the in-range 16-bit elements
// of K and V are XOR-ed into `xs` (the gather's own bandwidth ceiling, and a checksum).
// QLDS: the Q^T operand lives in LDS at byte address `qlds` (D / 32 KiB, private to the wave)
// and is read back for every tile, instead of taking D / 8 registers for the whole range: at
// head dim 256 the ring, the accumulators and Q together would not fit the 256 registers a
// wave has at two waves per SIMD, and the spills cost HBM traffic.
template <int D, int BSL, int PAIRS, bool NT, bool PROBE = false, int NWIN = 2, bool QLDS = false>
__device__ __forceinline__ void gqa_range_mfma(const DecodeArgs& a, const int32_t* trow,
                                               const uint16_t* qrow, bool qvalid, int kvh, int lo,
                                               int hi, int lane, f32x4 (&acc)[D / 16], float& m,
                                               float& lsum, uint32_t& xs, uint32_t qlds = 0u) {
  typedef __attribute__((address_space(3))) u32x4 qlw32x4;
  constexpr int BS = 1 << BSL;
  constexpr int KS = D / 32;       // k-steps of the QK product (32 dims each)
  constexpr int VT = D / 16;       // 16-dim output tiles of the PV product
  constexpr int RING = 2 * PAIRS;  // tiles held in registers
  const int n = lane & 15;   // MFMA row / column index
  const int g4 = lane >> 4;  // lane group: k-slot of the operands, row group of the output
  const int t_lo = lo >> 4;
  const int ntiles = ((hi + 15) >> 4) - t_lo;

  // Block ids of the range (at most 64 * NWIN blocks; the launcher checks), NWIN per lane:
  // pidw[w] lane i = block wbase + 64 w + i.
  const int blk_last = ((t_lo + ntiles - 1) << 4) >> BSL;
  const int wbase = (t_lo << 4) >> BSL;
  int pidw[NWIN];
#pragma unroll
  for (int w = 0; w < NWIN; ++w) pidw[w] = trow[min(wbase + 64 * w + lane, blk_last)];

  // B operand of the QK product: Q^T, lane (n, g4) holds column n, dims 8*(g4+4j) .. +7.
  bf16x8 qop[QLDS ? 1 : KS];
  if constexpr (!PROBE) {
    const uint4* q4 = reinterpret_cast<const uint4*>(qrow);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      uint4 v = q4[g4 + 4 * j];
      if (!qvalid) v = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (QLDS)
        *reinterpret_cast<qlw32x4*>((uintptr_t)(qlds + (uint32_t)((j * 64 + lane) * 16))) =
            u32x4{v.x, v.y, v.z, v.w};
      else
        qop[j] = as_bf16x8(v);
    }
  }

  // Per-lane byte offsets inside a block (tile start folded into the uniform base):
  //   K chunk kvh*D/8 + g4 + 4j of token slot n:  koff + j * 4*BS*16
  //   V^T row kvh*D + n + 16t, token slots 4*g4..: voff + t * 16*BS*2
  const uint32_t koff = (uint32_t)((((kvh * (D / 8) + g4) << BSL) + n) * 16);
  const uint32_t voff = (uint32_t)((((kvh * D + n) << BSL) + 4 * g4) * 2);
  const int64_t kpart_bytes = (int64_t)a.hkv * BS * D * 2;

  // The ring starts zeroed: a slot that is never loaded (partitions shorter than the
  // prologue) enters the masked PV product as finite zeros, never as stale register bits.
  u32x4 kb[RING][KS];
  u32x2 vb[RING][VT];
  bool vld[RING];
#pragma unroll
  for (int s = 0; s < RING; ++s) {
    vld[s] = false;
#pragma unroll
    for (int j = 0; j < KS; ++j) kb[s][j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < VT; ++t) vb[s][t] = u32x2{0u, 0u};
  }

  // Loads of tile `rel` into ring slot `slot`.  Callers in the main loop pass only tiles of
  // the range (GUARD = false), so every round issues the same loads and the compiler's wait
  // counts stay exact (a conditional load anywhere in the loop would make it wait for all
  // outstanding loads, the prefetch included); the last round skips tiles past the end.
  auto issue = [&](int slot, int rel, bool guard) {
    if (guard && rel >= ntiles) return;
    const int tok0 = (t_lo + rel) << 4;
    const int blk = tok0 >> BSL;
    const int sub = tok0 & (BS - 1);
    const int rb = blk - wbase;
    int32_t pid = __builtin_amdgcn_readlane(pidw[0], rb & 63);
#pragma unroll
    for (int w = 1; w < NWIN; ++w) {
      const int32_t pw = __builtin_amdgcn_readlane(pidw[w], rb & 63);
      pid = (rb >> 6) == w ? pw : pid;
    }
    const bool ok = valid_block(a.rt, pid);
    vld[slot] = ok;
    gchar* base = block_addr(a.rt, ok ? pid : 0);
    gchar* kbase = base + sub * 16;
    gchar* vbase = base + kpart_bytes + sub * 2;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      gu32x4* pk = reinterpret_cast<gu32x4*>(kbase + koff + j * (4 * BS * 16));
      kb[slot][j] = NT ? __builtin_nontemporal_load(pk) : *pk;
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      gu32x2* pv = reinterpret_cast<gu32x2*>(vbase + voff + t * (16 * BS * 2));
      vb[slot][t] = NT ? __builtin_nontemporal_load(pv) : *pv;
    }
  };

#pragma unroll
  for (int t = 0; t < VT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  m = kNegInf;
  lsum = 0.f;
  bool bad = false;
  const float scale_log2 = a.scale_log2;

  // scores of one tile, masked: lane (n, g4), register i = token 16*tile + 4*g4 + i, head n;
  // bit i of the result is set when token i of the lane is inside the range
  auto scores = [&](int slot, int rel, float* sv) -> uint32_t {
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    // an opaque copy of the address, so that the compiler cannot hoist these loop-invariant
    // reads out of the loop and back into registers
    uint32_t qa = qlds + (uint32_t)(lane * 16);
    if constexpr (QLDS) asm volatile("" : "+v"(qa));
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      bf16x8 qj;
      if constexpr (QLDS)
        qj = as_bf16x8(*reinterpret_cast<const qlw32x4*>((uintptr_t)(qa + (uint32_t)(j * 1024))));
      else
        qj = qop[j];
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[slot][j]), qj, sacc, 0, 0, 0);
    }
    const int tb = ((t_lo + rel) << 4) + 4 * g4;
    uint32_t okbits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tb + i;
      const bool ok = vld[slot] & (t >= lo) & (t < hi);  // bitwise: no short-circuit branches
      sv[i] = ok ? sacc[i] * scale_log2 : kNegInf;
      okbits |= (uint32_t)ok << i;
    }
    bad |= !vld[slot] & (rel < ntiles);
    return okbits;
  };

  // A tile not wholly inside the range (the range's first and last, the fully masked tiles of
  // the last round, a tile of an invalid block) may hold anything in its outside token slots,
  // NaN bit patterns included: a slot no token was ever written to, for instance.  A zero
  // weight does not cancel a NaN in the PV product, so those V values are zeroed first.
  auto edge_tile = [&](int slot, int rel) {
    const int t0 = (t_lo + rel) << 4;
    return !vld[slot] | (t0 < lo) | (t0 + 16 > hi);  // uniform
  };
  auto mask_v = [&](int slot, uint32_t okbits) {
    const uint32_t m0 = ((okbits & 1u) ? 0xffffu : 0u) | ((okbits & 2u) ? 0xffff0000u : 0u);
    const uint32_t m1 = ((okbits & 4u) ? 0xffffu : 0u) | ((okbits & 8u) ? 0xffff0000u : 0u);
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      vb[slot][t][0] &= m0;
      vb[slot][t][1] &= m1;
    }
  };

  // One ring round: RING tiles starting at `it`, each pair's refill issued RING - 2 tiles
  // ahead.  Tiles past the end of the range (the tail of the last round) are computed fully
  // masked: zero weight, max unchanged.
  // PROBE: XOR of the tile's in-range elements (lane: token n's K chunks; V slices of tokens
  // 4*g4 .. 4*g4+3, two per 32-bit word)
  auto probe_tile = [&](int slot, int rel) -> uint32_t {
    if (rel >= ntiles) return 0u;  // uniform
    const int t0 = (t_lo + rel) << 4;
    bad |= !vld[slot];
    const bool okk = vld[slot] & (t0 + n >= lo) & (t0 + n < hi);
    uint32_t x = 0u;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      x ^= okk ? (kb[slot][j][0] ^ kb[slot][j][1] ^ kb[slot][j][2] ^ kb[slot][j][3]) : 0u;
    uint32_t mk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g4 + i;
      mk[i] = (vld[slot] & (t >= lo) & (t < hi)) ? 0xffffu : 0u;
    }
    const uint32_t m0 = mk[0] | (mk[1] << 16), m1 = mk[2] | (mk[3] << 16);
#pragma unroll
    for (int t = 0; t < VT; ++t) x ^= (vb[slot][t][0] & m0) ^ (vb[slot][t][1] & m1);
    return x;
  };

  auto round = [&](int it, bool guard) {
#pragma unroll
    for (int ps = 0; ps < PAIRS; ++ps) {
      const int sa = 2 * ps, sb = 2 * ps + 1;
      const int ra = it + 2 * ps, rb = ra + 1;
      // refill the pair slot consumed last round with the pair RING - 2 tiles ahead
      const int fs = (sa + RING - 2) % RING;
      issue(fs, ra + RING - 2, guard);
      issue(fs + 1, ra + RING - 1, guard);
      if constexpr (PROBE) {
        xs ^= probe_tile(sa, ra) ^ probe_tile(sb, rb);
        continue;
      }
      float sva[4], svb[4];
      const uint32_t oka = scores(sa, ra, sva);
      const uint32_t okb = scores(sb, rb, svb);
      if (edge_tile(sa, ra)) mask_v(sa, oka);
      if (edge_tile(sb, rb)) mask_v(sb, okb);
      const float mx = rows_max(fmaxf(fmaxf(fmaxf(sva[0], sva[1]), fmaxf(sva[2], sva[3])),
                                      fmaxf(fmaxf(svb[0], svb[1]), fmaxf(svb[2], svb[3]))));
      if (__any(mx > m + kRescaleSlack)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 when m = -inf
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[t] *= alpha;
        lsum *= alpha;
        m = mnew;
      }
      const float mref = m == kNegInf ? 0.f : m;
      float pw[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[i] = __builtin_amdgcn_exp2f(sva[i] - mref);
        pw[4 + i] = __builtin_amdgcn_exp2f(svb[i] - mref);
      }
      u32x4 phi, plo;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h = cvt_pk_bf16(pw[2 * k], pw[2 * k + 1]);
        phi[k] = h;
        plo[k] = cvt_pk_bf16(pw[2 * k] - __uint_as_float(h << 16),
                             pw[2 * k + 1] - __uint_as_float(h & 0xffff0000u));
      }
      lsum += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
      const bf16x8 bhi = as_bf16x8(phi), blo = as_bf16x8(plo);
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const bf16x8 vop = as_bf16x8(u32x4{vb[sa][t][0], vb[sa][t][1], vb[sb][t][0], vb[sb][t][1]});
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, bhi, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, blo, acc[t], 0, 0, 0);
      }
    }
  };

  // prologue: the first PAIRS - 1 pairs, unguarded so the wait counts stay exact (in a range
  // shorter than the prologue the extra tile reads a clamped, valid block id: a harmless
  // redundant load)
#pragma unroll
  for (int s = 0; s < RING - 2; ++s) issue(s, s, false);
  // rounds whose refills all fall inside the range, then the last round(s)
  int it = 0;
  for (; it + 2 * RING - 2 <= ntiles; it += RING) round(it, false);
  for (; it < ntiles; it += RING) round(it, true);
  if (bad) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);
}

// The range [lo, hi) of sequence b for the query heads of KV head kvh (column n = head n of
// the group; columns past the group get zero queries).
template <int D, int BSL, int PAIRS, bool NT, bool PROBE = false>
__device__ __forceinline__ void gqa_partition_mfma(const DecodeArgs& a, int b, int kvh, int lo,
                                                   int hi, int lane, f32x4 (&acc)[D / 16],
                                                   float& m, float& lsum, uint32_t& xs) {
  const int n = lane & 15;
  const bool hv = n < a.group;
  const uint16_t* qrow =
      PROBE ? nullptr
            : static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + kvh * a.group + (hv ? n : 0)) * D;
  gqa_range_mfma<D, BSL, PAIRS, NT, PROBE>(a, a.table + (int64_t)b * a.max_blocks, qrow, hv, kvh,
                                           lo, hi, lane, acc, m, lsum, xs);
}

// The range [lo, hi) of table row `trow` read by the four waves of a workgroup together
// (staged wave items of a plan: one range, up to 4 x 16 / group sequences), so that it crosses
// HBM once.  A stage is a pair of 16-token tiles (32 tokens), 2 * D / 32 K lines and D / 16 V
// lines of 1 KiB.  Within a pair, row r = 4 a + b of score tile u stands for token
// 8 a + 4 u + b, so that the eight tokens 8 g4 .. 8 g4 + 7 whose weights lane group g4 holds
// in the PV product are contiguous: the V operand of lane (n, g4) is row n of its 16-row
// group, tokens 8 g4 .. + 7, one 16-byte piece of the cache.  K line (u, j) holds at lane
// (n, g4) the 16-byte chunk 4 j + g4 of the token of row n of tile u; V line h holds at lane
// (n, g4) row 16 h + n, tokens 8 g4 .. + 7.  Every wave loads a quarter of each stage's lines
// (lane i: the line's bytes 16 i .. 16 i + 15, read back by the same lane position, so LDS
// reads and writes are 16-byte, bank-conflict free) into a register ring AHEAD stages deep,
// and writes a stage into one half of `lds` (two stages) when its turn comes, so that the
// four waves keep AHEAD stages of distinct bytes in flight between them.  Per stage p: write
// the wave's lines of stage p into half p % 2 (every wave finished reading stage p - 2 there
// before the previous barrier), refill that ring slot with stage p + AHEAD, barrier, then
// score both tiles with K read from LDS, the online softmax, and the PV product with V read
// from LDS: the arithmetic of the per-wave ring loop of gqa_range_mfma, tokens taken in
// another order.  A wave with no sequence (`active` false: padding) loads and writes its
// lines but computes nothing.  A tile past the range loads the range's last tile again and a
// stage past the last loads one line for all lanes (every load unconditional, so that the
// wait before a stage's LDS write leaves the later stages' loads in flight); such slots are
// fully masked.  The trip count depends on the range only, so all four waves meet every
// barrier.
template <int D, int BSL, int AHEAD>
__device__ __forceinline__ void gqa_range_staged(const DecodeArgs& a, const int32_t* trow,
                                                 const uint16_t* qrow, bool qvalid, bool active,
                                                 int kvh, int lo, int hi, int wv, int lane,
                                                 uint32_t lds, f32x4 (&acc)[D / 16], float& m,
                                                 float& lsum) {
  wv = __builtin_amdgcn_readfirstlane(wv);  // uniform: the line offsets stay scalar
  typedef __attribute__((address_space(3))) u32x4 lw32x4;
  typedef __attribute__((address_space(3))) const u32x4 lu32x4;
  constexpr int BS = 1 << BSL;
  constexpr int KS = D / 32;
  constexpr int VT = D / 16;
  constexpr int KLINES = 2 * KS;
  constexpr int LINES = KLINES + VT;
  constexpr int LPW = LINES / kWavesPerGroup;  // lines per wave and stage
  constexpr int KPW = KLINES / kWavesPerGroup;
  static_assert(KLINES % kWavesPerGroup == 0 && LINES % kWavesPerGroup == 0, "line split");
  constexpr uint32_t STAGE = LINES * 1024;
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int t_lo = lo >> 4;
  const int ntiles = ((hi + 15) >> 4) - t_lo;
  const int npairs = (ntiles + 1) >> 1;

  const int blk_last = ((t_lo + ntiles - 1) << 4) >> BSL;
  const int wbase = (t_lo << 4) >> BSL;
  const int pid0 = trow[min(wbase + lane, blk_last)];
  const int pid1 = trow[min(wbase + 64 + lane, blk_last)];
  auto tile_pid = [&](int rel) -> int32_t {  // uniform
    const int rb = ((((t_lo + rel) << 4) >> BSL) - wbase);
    const int32_t pa = __builtin_amdgcn_readlane(pid0, rb & 63);
    const int32_t pb = __builtin_amdgcn_readlane(pid1, rb & 63);
    return rb < 64 ? pa : pb;
  };

  bf16x8 qop[KS];
  {
    const uint4* q4 = reinterpret_cast<const uint4*>(qrow);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      uint4 v = q4[g4 + 4 * j];
      if (!qvalid) v = make_uint4(0u, 0u, 0u, 0u);
      qop[j] = as_bf16x8(v);
    }
  }

  // lane parts of the addresses: K, the token of row n of tile 0 (8 (n / 4) + n % 4, in pair
  // tile n / 8) and chunk g4; V, row n and tokens 8 g4 .. (pair tile g4 / 2)
  const int ktile = n >> 3;
  const uint32_t kpart = (uint32_t)((((kvh * (D / 8) + g4) << BSL) + (8 * ((n >> 2) & 1) + (n & 3))) * 16);
  const int vtile = g4 >> 1;
  const uint64_t vpart = (uint64_t)a.hkv * BS * D * 2 +
                         (uint64_t)((((kvh * D + n) << BSL) + 8 * (g4 & 1)) * 2);
  // Line i of this wave in a stage: its place in the stage (LDS line) and its byte offset
  // from the lane's base address.  Where a kind of line numbers at least four, each wave
  // takes a fixed share of both tiles' (K) or row groups' (V) lines.
  auto line_of = [&](int i, uint32_t& off) -> int {
    if (i < KPW) {  // K line (u, j): score tile u, k-step j
      int u, j;
      if (KS >= kWavesPerGroup) {
        u = i / (KS / kWavesPerGroup);
        j = wv + kWavesPerGroup * (i % (KS / kWavesPerGroup));
      } else {
        u = wv / KS;
        j = wv % KS;
      }
      off = (uint32_t)(u * 4 * 16 + j * (4 * BS * 16));
      return u * KS + j;
    }
    const int h = wv + kWavesPerGroup * (i - KPW);  // V line h: rows 16 h .. 16 h + 15
    off = (uint32_t)((16 * h) << BSL) * 2u;
    return KLINES + h;
  };
  const uint64_t dummy =
      (uint64_t)(uintptr_t)block_addr(a.rt, valid_block(a.rt, tile_pid(0)) ? tile_pid(0) : 0);
  auto load_stage = [&](int p, u32x4 (&r)[LPW]) {
    uint64_t tb[2];
    int sub[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int rel = min(2 * p + w, ntiles - 1);  // past the range: the last tile again
      const int32_t pid = tile_pid(rel);
      tb[w] = (uint64_t)(uintptr_t)block_addr(a.rt, valid_block(a.rt, pid) ? pid : 0);
      sub[w] = ((t_lo + rel) << 4) & (BS - 1);
    }
    const bool past = p >= npairs;  // uniform
    const uint64_t kb = past ? dummy : (ktile ? tb[1] : tb[0]) + kpart + (uint32_t)((ktile ? sub[1] : sub[0]) * 16);
    const uint64_t vb = past ? dummy : (vtile ? tb[1] : tb[0]) + vpart + (uint32_t)((vtile ? sub[1] : sub[0]) * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      uint32_t off;
      line_of(i, off);
      const uint64_t src = (i < KPW ? kb : vb) + (past ? 0u : off);
      r[i] = __builtin_nontemporal_load(reinterpret_cast<gu32x4*>((uintptr_t)src));
    }
  };

#pragma unroll
  for (int t = 0; t < VT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  m = kNegInf;
  lsum = 0.f;
  bool bad = false;
  const float scale_log2 = a.scale_log2;

  u32x4 ring[AHEAD][LPW];
  // stage by stage, in order (no scheduling across): the wait before stage p's LDS write
  // then counts only the loads of the stages after it
#pragma unroll
  for (int u = 0; u < AHEAD; ++u) {
    load_stage(u, ring[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int p0 = 0; p0 < npairs; p0 += AHEAD) {
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) {
      // a stage past the last (npairs not a multiple of AHEAD) runs fully masked: no weight,
      // no rescale; the loop body has no exit, so the loads stay in one order
      const int p = p0 + u;
      const uint32_t sb = lds + (uint32_t)(p & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        uint32_t off;
        const int line = line_of(i, off);
        *(lw32x4*)(uintptr_t)(sb + line * 1024u + lane * 16u) = ring[u][i];
      }
      load_stage(p + AHEAD, ring[u]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // stage p is in LDS for every wave
      if (!active) continue;
      const int ra = 2 * p;
      const bool vldA = valid_block(a.rt, tile_pid(min(ra, ntiles - 1)));
      const bool vldB = ra + 1 < ntiles && valid_block(a.rt, tile_pid(ra + 1));
      bad |= (!vldA & (ra < ntiles)) | (!vldB & (ra + 1 < ntiles));
      const bool vld = vtile ? vldB : vldA;  // tokens 8 g4 .. lie in pair tile g4 / 2
      const int pbase = (t_lo + ra) << 4;
      // scores S^T = K Q^T of both tiles, K operands read from LDS, masked to the range
      float sv[2][4];
      uint32_t okbits[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          const u32x4 kv = *(lu32x4*)(uintptr_t)(sb + (w * KS + j) * 1024u + lane * 16u);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), qop[j], sacc, 0, 0, 0);
        }
        const int tb = pbase + 8 * g4 + 4 * w;
        okbits[w] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb + i;
          const bool ok = vld & (t >= lo) & (t < hi);  // bitwise: no short-circuit branches
          sv[w][i] = ok ? sacc[i] * scale_log2 : kNegInf;
          okbits[w] |= (uint32_t)ok << i;
        }
      }
      // online softmax in the log2 domain with the lazy rescale of the per-wave ring loop
      const float mx = rows_max(fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                                      fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3]))));
      if (__any(mx > m + kRescaleSlack)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 when m = -inf
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[t] *= alpha;
        lsum *= alpha;
        m = mnew;
      }
      const float mref = m == kNegInf ? 0.f : m;
      float pw[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[i] = __builtin_amdgcn_exp2f(sv[0][i] - mref);
        pw[4 + i] = __builtin_amdgcn_exp2f(sv[1][i] - mref);
      }
      u32x4 phi, plo;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h = cvt_pk_bf16(pw[2 * k], pw[2 * k + 1]);
        phi[k] = h;
        plo[k] = cvt_pk_bf16(pw[2 * k] - __uint_as_float(h << 16),
                             pw[2 * k + 1] - __uint_as_float(h & 0xffff0000u));
      }
      lsum += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
      const bf16x8 bhi = as_bf16x8(phi), blo = as_bf16x8(plo);
      // V^T P^T with the V operands read from LDS.  In a pair not wholly inside the range and
      // valid (its first or last, past the end: stale LDS, an invalid block) the other token
      // slots may hold anything, NaN bit patterns included, and a zero weight does not cancel
      // a NaN, so those slots are zeroed as they are read (the token validity of lane group
      // g4 is the same in the score and V layouts).
      const bool edge = !vldA | (!vldB & (ra + 1 < ntiles)) | (pbase < lo) | (pbase + 32 > hi);
      if (edge) {  // uniform
        uint32_t vm[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t ob = okbits[w >> 1] >> (2 * (w & 1));
          vm[w] = ((ob & 1u) ? 0xffffu : 0u) | ((ob & 2u) ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const u32x4 v = *(lu32x4*)(uintptr_t)(sb + (KLINES + t) * 1024u + lane * 16u);
          const bf16x8 vop = as_bf16x8(u32x4{v[0] & vm[0], v[1] & vm[1], v[2] & vm[2], v[3] & vm[3]});
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, bhi, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, blo, acc[t], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const bf16x8 vop =
              as_bf16x8(*(lu32x4*)(uintptr_t)(sb + (KLINES + t) * 1024u + lane * 16u));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, bhi, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, blo, acc[t], 0, 0, 0);
        }
      }
    }
  }
  if (bad) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);
}

// Stages a staged workgroup's waves keep in flight (register ring depth) per head dim.
template <int D>
__host__ __device__ constexpr int staged_ahead() { return D == 256 ? 2 : 4; }

// One workgroup of W = group_parts / wave_parts waves per (sequence, KV head, group of
// partitions); wave w takes the group's partitions [w * wave_parts, (w + 1) * wave_parts),
// its online softmax continuing across their boundary.  Dynamic LDS (W > 1 only):
// [W][group][row] partial outputs (row = gqa_merge_row(W, group, D), D padded), then
// [W][group] lse values (log2 domain).
template <int D, int BSL, int PAIRS, bool NT>
__global__ __launch_bounds__(64 * mfma_max_group<D>()) void gqa_decode_mfma_kernel(DecodeArgs a) {
  constexpr int VT = D / 16;
  extern __shared__ float smem[];
  const int S = a.wave_parts;
  const int G = a.group_parts / S;  // waves of the workgroup
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g4 = lane >> 4;

  int w = blockIdx.x;
  const int k = w % a.grid_ng;
  w /= a.grid_ng;
  const int kvh = w % a.hkv;
  const int b = w / a.hkv;

  int beg, P, ng;
  const int np = seq_partitions(a, b, &beg, &P, &ng);
  if (k == 0 && kvh == 0 && threadIdx.x == 0) {
    a.nparts[b] = ng < 0 ? 0 : ng;
    if (np < 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
  }
  if (k >= ng) return;  // uniform over the workgroup; also covers ng < 0
  const int p = k * a.group_parts + wv * S;  // the wave's first partition
  const int L = a.seq[b];

  f32x4 acc[VT];
  float m = kNegInf, lsum = 0.f;
  if (p < np) {  // uniform over the wave: waves past the sequence's last partition idle
    const int lo = beg + p * P;
    uint32_t unused = 0u;
    gqa_partition_mfma<D, BSL, PAIRS, NT>(a, b, kvh, lo, (int)min((int64_t)L, (int64_t)lo + S * P),
                                      lane, acc, m, lsum, unused);
  }
  lsum = rows_sum(lsum);
  const int grp = a.group;

  if (G == 1) {  // the wave's partial is the group's partial
    if (n < grp) {
      const int64_t row = ((int64_t)b * a.hq + kvh * grp + n) * a.max_parts + k;
      // no weight (every block invalid): o = 0 beside lse = -inf, never 0 / 0
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float* op = a.o_part + row * D;
#pragma unroll
      for (int t = 0; t < VT; ++t)
        *reinterpret_cast<f32x4*>(op + 16 * t + 4 * g4) = acc[t] * inv;
      if (g4 == 0) a.lse_part[row] = (m + log2f(lsum)) * kLn2;
    }
    return;
  }

  // Exact LSE merge of the group's partials in LDS:
  //   M = max_w lse_w, s = sum_w 2^(lse_w - M), o = sum_w 2^(lse_w - M) o_w / s.
  const int rs = gqa_merge_row(G, grp, D);  // row stride
  float* so = smem;                  // [G][grp][rs]
  float* sl = smem + G * grp * rs;   // [G][grp]
  if (n < grp) {
    if (p < np) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float* op = so + (wv * grp + n) * rs;
#pragma unroll
      for (int t = 0; t < VT; ++t)
        *reinterpret_cast<f32x4*>(op + 16 * t + 4 * g4) = acc[t] * inv;
    }
    if (g4 == 0) sl[wv * grp + n] = p < np ? m + log2f(lsum) : kNegInf;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < grp * D; idx += 64 * G) {
    const int h = idx / D;
    const int d = idx % D;
    float mx = kNegInf;
    for (int u = 0; u < G; ++u) mx = fmaxf(mx, sl[u * grp + h]);
    float s = 0.f, o = 0.f;
    for (int u = 0; u < G; ++u) {
      const float l = sl[u * grp + h];
      if (l != kNegInf) {  // idle waves wrote no output
        const float e = exp2f(l - mx);
        s += e;
        o += e * so[(u * grp + h) * rs + d];
      }
    }
    const int64_t row = ((int64_t)b * a.hq + kvh * grp + h) * a.max_parts + k;
    a.o_part[row * D + d] = s > 0.f ? o / s : 0.f;
    if (d == 0) a.lse_part[row] = (mx + log2f(s)) * kLn2;
  }
}

// Gather probe of the matrix-core kernel's access pattern: the same grid, waves and loads,
// no arithmetic.  Each wave folds the XOR of its in-range 16-bit K/V elements into one 16-bit
// value and XORs it into xsum[b][kvh] (zeroed by the caller).
template <int D, int BSL, int PAIRS, bool NT>
__global__ __launch_bounds__(64 * mfma_max_group<D>()) void gqa_probe_kernel(DecodeArgs a,
                                                                            uint32_t* xsum) {
  const int S = a.wave_parts;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  int w = blockIdx.x;
  const int k = w % a.grid_ng;
  w /= a.grid_ng;
  const int kvh = w % a.hkv;
  const int b = w / a.hkv;
  int beg, P, ng;
  const int np = seq_partitions(a, b, &beg, &P, &ng);
  if (k == 0 && kvh == 0 && threadIdx.x == 0 && np < 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
  if (k >= ng) return;
  const int p = k * a.group_parts + wv * S;
  if (p >= np) return;  // uniform over the wave; no barrier follows
  const int L = a.seq[b];
  const int lo = beg + p * P;
  f32x4 acc[D / 16];
  float m = 0.f, lsum = 0.f;
  uint32_t xs = 0u;
  gqa_partition_mfma<D, BSL, PAIRS, NT, true>(a, b, kvh, lo,
                                                (int)min((int64_t)L, (int64_t)lo + S * P), lane,
                                                acc, m, lsum, xs);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) xs ^= __shfl_xor(xs, o);
  if (lane == 0) atomicXor(xsum + (int64_t)b * a.hkv + kvh, (xs ^ (xs >> 16)) & 0xffffu);
}

// LDS the plan kernel reserves per workgroup: two stages of gqa_range_staged (a quarter of it
// holds a ring wave's Q^T at head dim 256: D / 32 KiB).
__host__ __device__ constexpr uint32_t plan_lds_bytes(int d) { return 2u * (2 * (d / 32) + d / 16) * 1024u; }

// One wave item of a plan (kvattn_decode_plan): wave `wv` of workgroup `grp` for KV head kvh.
// An item is a token range of one table row and up to 16 / group sequences that hold that
// range in the same blocks: column n of the MFMA tiles is head n % group of member n / group,
// so one pass over the range's keys and values serves every member, and each member's
// partial of the range goes to its own slot.  Item modes: 0, a range this wave alone reads
// (private, or one wave for all its sharers), streamed with non-temporal loads; 1, a range
// another wave of the workgroup reads too (its other sharers), read with cache-retaining
// loads so that the second read hits in L2; 2, staged: the workgroup's four waves share one
// range (their sharers split between them) and read it once through LDS (gqa_range_staged;
// padding waves with no sequence still load their share).
// Every wave of a workgroup reads all four of its items, so the staged decision, and the
// range a staged workgroup loops over, are the same for all of them.  An idle wave returns at
// once; an item outside the call's arguments sets KVATTN_ERR_BAD_SEQ.
template <int D, int BSL, int PAIRS>
__device__ __forceinline__ void gqa_plan_item(const DecodeArgs& a, const int32_t* plan, int grp,
                                              int kvh, int wv, int lane, uint32_t lds) {
  constexpr int VT = D / 16;
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int32_t* np = plan + kPlanHeader;
  const int32_t* items0 = np + a.batch + kItemInts * ((int64_t)grp * kWavesPerGroup);
  const int32_t* item = items0 + kItemInts * wv;
  const int seq = item[0], lo = item[1], hi = item[2], nmem = item[3], moff = item[4];
  bool staged = true, any_staged = false;
#pragma unroll
  for (int w = 0; w < kWavesPerGroup; ++w) {
    const int32_t* it = items0 + kItemInts * w;
    staged &= it[5] == 2 && it[0] == items0[0] && it[1] == items0[1] && it[2] == items0[2];
    any_staged |= it[5] == 2;
  }
  if (any_staged && !staged) {  // uniform over the workgroup: nobody reaches a barrier
    if (wv == 0 && lane == 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
    return;
  }
  if (!staged && nmem <= 0) return;  // an idle wave (uniform)
  const bool range_ok = seq >= 0 && seq < a.batch && lo >= 0 && lo < hi &&
                        (int64_t)hi <= ((int64_t)a.max_blocks << BSL) &&
                        ((hi - 1) >> BSL) - (lo >> BSL) < kPlanWindow;
  if (!range_ok) {  // uniform over the workgroup when staged (one range)
    if (lane == 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
    return;
  }
  const int32_t* members = np + a.batch + kItemInts * plan[3];  // [M][2]
  bool ok = nmem >= 0 && nmem <= plan[7] && moff >= 0 && (int64_t)moff + nmem <= plan[4];
  const int32_t* mem = members + 2 * (int64_t)(ok ? moff : 0);  // this item's entries
  // column n: head h of member j
  const int j = n / a.group;
  const int h = n - j * a.group;
  bool col = ok && j < nmem;
  const int m = col ? mem[2 * j] : seq;
  const int slot = col ? mem[2 * j + 1] : 0;
  ok = ok && !__any(col && (m < 0 || m >= a.batch || slot < 0 || slot >= a.max_parts));
  if (!ok) {  // uniform over the wave
    if (lane == 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
    if (!staged) return;
    col = false;  // a staged wave keeps loading its share of the range for the others
  }
  const uint16_t* qrow =
      static_cast<const uint16_t*>(a.q) +
      ((int64_t)(col ? m : seq) * a.hq + kvh * a.group + (col ? h : 0)) * D;
  const int32_t* trow = a.table + (int64_t)seq * a.max_blocks;
  f32x4 acc[VT];
  float mx, lsum;
  uint32_t unused = 0u;
  // At head dim 256 a ring wave keeps Q^T in its quarter of the workgroup's LDS, which only
  // staged workgroups use otherwise.
  if (staged)
    gqa_range_staged<D, BSL, staged_ahead<D>()>(a, trow, qrow, col, __any(col), kvh, lo, hi, wv,
                                                lane, lds, acc, mx, lsum);
  else if (item[5] == 1)  // other waves of the workgroup read the same range: keep it in L2
    gqa_range_mfma<D, BSL, PAIRS, false, false, kPlanWindow / 64, D == 256>(
        a, trow, qrow, col, kvh, lo, hi, lane, acc, mx, lsum, unused, lds + wv * (D / 32) * 1024);
  else  // one wave reads the range, once, whatever its sharers: stream it
    gqa_range_mfma<D, BSL, PAIRS, true, false, kPlanWindow / 64, D == 256>(
        a, trow, qrow, col, kvh, lo, hi, lane, acc, mx, lsum, unused, lds + wv * (D / 32) * 1024);
  lsum = rows_sum(lsum);
  if (col) {
    // the member and slot are read again here rather than held in registers across the loop
    const int64_t row =
        ((int64_t)mem[2 * j] * a.hq + kvh * a.group + h) * a.max_parts + mem[2 * j + 1];
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // no weight: o = 0 beside lse = -inf
    float* op = a.o_part + row * D;
#pragma unroll
    for (int t = 0; t < VT; ++t) *reinterpret_cast<f32x4*>(op + 16 * t + 4 * g4) = acc[t] * inv;
    if (g4 == 0) a.lse_part[row] = (mx + log2f(lsum)) * kLn2;
  }
}

// Decode over a plan: workgroups of four independent waves.  The plan's units are its
// (workgroup, KV head) pairs, unit u = group u / Hkv, KV head u % Hkv, in the plan's order
// (longest wave item first).  Without a work counter (work == NULL) workgroup x runs unit x.  With
// one, the grid is the workgroups the device holds at once: workgroup x runs unit x, then
// claims unit gridDim.x + work[0]++ until none are left, so the CUs (and XCDs) that finish
// first take the rest; a unit's partials do not depend on which workgroup ran it.  The last
// workgroup to leave sets work[0] = work[1] = 0 again for the next launch.  Workgroup 0 also
// writes every sequence's partial count.  CLAIM selects the claiming form at compile time:
// the one-unit form then holds no claim loop, whose state would add to the register pressure
// (and spill stores) of the item path.
template <int D, int BSL, int PAIRS, bool CLAIM>
__global__ __launch_bounds__(64 * kWavesPerGroup, 2) void gqa_decode_plan_kernel(DecodeArgs a,
                                                                               const int32_t* plan,
                                                                               int32_t n_groups,
                                                                               uint32_t* work) {
  __shared__ int s_unit;
  extern __shared__ __attribute__((aligned(16))) char plan_lds[];  // plan_lds_bytes(D)
  const uint32_t lds = (uint32_t)(uintptr_t)plan_lds;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int32_t* np = plan + kPlanHeader;
  const bool hdr_ok = plan[0] == kPlanMagic && plan[1] == a.batch && plan[2] == n_groups &&
                      plan[3] == kWavesPerGroup * n_groups && plan[5] >= 1 &&
                      plan[5] <= a.max_parts && plan[6] == a.group && plan[7] >= 1 &&
                      plan[7] * a.group <= 16;
  if (!hdr_ok) {  // every workgroup returns here (the counters are left as they are)
    if (blockIdx.x == 0 && threadIdx.x == 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
    return;
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.batch; i += 64 * kWavesPerGroup)
      a.nparts[i] = min(max(np[i], 0), a.max_parts);
  if constexpr (!CLAIM) {  // one unit per workgroup (an empty plan: none)
    if ((int64_t)blockIdx.x < (int64_t)n_groups * a.hkv)
      gqa_plan_item<D, BSL, PAIRS>(a, plan, (int)blockIdx.x / a.hkv, (int)blockIdx.x % a.hkv, wv,
                                   lane, lds);
    return;
  }
  const int units = n_groups * a.hkv;
  int u = blockIdx.x;
  while (u < units) {  // uniform over the workgroup
    gqa_plan_item<D, BSL, PAIRS>(a, plan, u / a.hkv, u % a.hkv, wv, lane, lds);
    __syncthreads();  // every wave is done with s_unit's last value
    if (threadIdx.x == 0) s_unit = (int)gridDim.x + (int)atomicAdd(&work[0], 1u);
    __syncthreads();
    u = s_unit;
  }
  if (threadIdx.x == 0) {
    __threadfence();  // this workgroup's claims are done before it counts itself out
    if (atomicAdd(&work[1], 1u) == gridDim.x - 1) {
      atomicExch(&work[0], 0u);
      atomicExch(&work[1], 0u);
    }
  }
}

template <typename T>
__device__ __forceinline__ float load_elem_g(gchar* p) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(*reinterpret_cast<__attribute__((address_space(1))) const uint32_t*>(p));
  } else {
    return bf16_to_f32(*reinterpret_cast<__attribute__((address_space(1))) const uint16_t*>(p));
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

// Plain VALU version: one token per lane for the scores, lanes over dims for P V (the chunk's
// V values transposed through LDS, so that both the loads and the P V reads are coalesced).
// One workgroup of kGW waves per (sequence, KV head, group of partitions): wave w takes the
// group's 64-token chunks w, w + kGW, ..., each wave with its own online softmax and its own
// LDS staging area, and the waves' states are merged exactly at the end (the LSE rescaling of
// the merge kernel), so a group's chunks are read in parallel.
static constexpr int kCB = 16;  // at most this many K chunks per lane in flight (scores)
static constexpr int kVB = 32;  // V loads per lane in flight (P V, dims 64 and up)
static constexpr int kGW = 4;   // waves per workgroup

// Orders a wave's LDS writes before its own later reads by other lanes (and its reads before
// later writes): a wave's LDS operations complete in order, this keeps the compiler's too.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// GP: the query heads per KV head rounded up to a power of two, a compile-time bound (the
// head loops then carry no per-head branches, which keeps the code small enough for the
// instruction cache); heads G .. GP-1 get zero queries, are computed and never written.
template <typename T, int D, int GP>
__global__ __launch_bounds__(64 * kGW) void gqa_decode_generic_kernel(DecodeArgs a) {
  constexpr int R = D / 64;                // dims per lane in the output
  constexpr int X = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int CB = (D / X) < kCB ? (D / X) : kCB;  // K chunks in flight
  static_assert((D / X) % CB == 0, "K chunks per token must be a multiple of CB");
  static_assert(GP * D <= 64 * 65, "the wave merge reuses a wave's V staging area");
  __shared__ float qs[GP][D];
  // P V operands of each wave, staged through LDS: the chunk's weights [head][token], and 64
  // dims of its V values transposed, [dim][token] (row padded by one word: conflict-free both
  // ways).  V is stored token-fastest, so loads with lane = token coalesce (16 consecutive
  // slots of a block), where lane = dim would touch a cache line per lane and token.  At the
  // end the V areas hold the waves' unnormalised outputs for the merge.
  __shared__ float sp[kGW][GP][64];
  __shared__ float sv[kGW][64][65];
  __shared__ float sml[kGW][2][GP];  // each wave's running max and sum per head
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  int w = blockIdx.x;
  const int k = w % a.grid_ng;
  w /= a.grid_ng;
  const int kvh = w % a.hkv;
  const int b = w / a.hkv;

  int beg, P, ng;
  const int np = seq_partitions(a, b, &beg, &P, &ng);
  if (k == 0 && kvh == 0 && threadIdx.x == 0) {
    a.nparts[b] = ng < 0 ? 0 : ng;
    if (np < 0) flag_error(a.err, KVATTN_ERR_BAD_SEQ);
  }
  if (k >= ng) return;  // uniform over the workgroup
  const int L = a.seq[b];
  const int64_t span = (int64_t)P * a.group_parts;
  const int lo = (int)(beg + k * span);
  const int hi = (int)min((int64_t)L, lo + span);
  const int G = a.group;
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
  // block ids are read one chunk ahead (the first chunk's before q), so that a chunk's K / V
  // loads need not wait for a table read of their own
  const int first = lo + 64 * wv;
  int32_t pid_next = first + lane < hi ? trow[(first + lane) >> a.bs_shift] : 0;

  for (int i = threadIdx.x; i < GP * D; i += 64 * kGW) {
    const int h = i / D, d = i - (i / D) * D;
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.hq + kvh * G + min(h, G - 1)) * D;
    qs[h][d] = h < G ? load_elem<T>(reinterpret_cast<const char*>(qrow + d)) : 0.f;
  }
  __syncthreads();

  const int64_t kpart_bytes = (int64_t)a.hkv * a.bs * D * (int64_t)sizeof(T);
  float m[GP], l[GP], acc[GP][R], pr[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[h][r] = 0.f;
  }
  bool bad = false;
  float (*spw)[64] = sp[wv];
  float (*svw)[65] = sv[wv];

  for (int c0 = first; c0 < hi; c0 += 64 * kGW) {  // uniform over the wave
    const int t = c0 + lane;
    const bool in = t < hi;
    const int32_t pid = pid_next;
    const int tn = t + 64 * kGW;
    pid_next = tn < hi ? trow[tn >> a.bs_shift] : 0;
    const bool ok = in && valid_block(a.rt, pid);
    bad |= in && !ok;
    // global-address-space pointers: global loads count against the vector-memory counter
    // only, so the shuffles and LDS accesses below do not wait for them (flat loads would)
    const int32_t vpid = ok ? pid : 0;  // id 0 exists: the launcher checked the pool
    gchar* base = block_addr(a.rt, vpid);
    const int tt = t & (a.bs - 1);
    // the token's V values of output dims 0..63, loaded now, with the K chunks, since they
    // depend only on the block id (zeros for a token that takes no part)
    gchar* vtok = base + kpart_bytes + (int64_t)tt * (int64_t)sizeof(T);
    float v0[64];
#pragma unroll
    for (int j = 0; j < 64; ++j)
      v0[j] = ok ? load_elem_g<T>(vtok + ((((int64_t)kvh * D + j) << a.bs_shift) * (int64_t)sizeof(T)))
                 : 0.f;
    float s[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) s[h] = 0.f;
    if (ok) {
      // the token's K chunks, CB 16-byte loads in flight at a time
      for (int k0 = 0; k0 < D / X; k0 += CB) {
        uint4 kc[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          const u32x4 v = *reinterpret_cast<gu32x4*>(
              base + ((((int64_t)kvh * (D / X) + k0 + u) << a.bs_shift) + tt) * 16);
          kc[u] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          const uint32_t wd[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
#pragma unroll
          for (int e = 0; e < X; ++e) {
            const float kv = sizeof(T) == 4 ? __uint_as_float(wd[e])
                                            : bf16_to_f32((uint16_t)(wd[e >> 1] >> (16 * (e & 1))));
#pragma unroll
            for (int h = 0; h < GP; ++h) s[h] += qs[h][(k0 + u) * X + e] * kv;
          }
          // keeps the next chunk's q reads from LDS below this point: hoisting all of them
          // (a fully unrolled 64-dim bf16 token) would exhaust the registers
          asm volatile("" ::: "memory");
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
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
    // P V over the chunk's tokens, 64 output dims at a time.  A token outside the range or in
    // an invalid block stages zeros (its slots may hold NaN bit patterns, which a zero weight
    // would not cancel) and has weight zero.
    const int cnt = min(64, hi - c0);
    wave_lds_sync();  // the previous chunk's reads of sp are done
#pragma unroll
    for (int h = 0; h < GP; ++h) spw[h][lane] = pr[h];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wave_lds_sync();  // the previous slice's reads of sv are done
      if (r == 0) {
#pragma unroll
        for (int j = 0; j < 64; ++j) svw[j][lane] = v0[j];
      } else {
        for (int j0 = 0; j0 < 64; j0 += kVB) {
          float v[kVB];
#pragma unroll
          for (int u = 0; u < kVB; ++u)
            v[u] = ok ? load_elem_g<T>(vtok + ((((int64_t)kvh * D + 64 * r + j0 + u) << a.bs_shift) *
                                               (int64_t)sizeof(T)))
                      : 0.f;
#pragma unroll
          for (int u = 0; u < kVB; ++u) svw[j0 + u][lane] = v[u];
        }
      }
      wave_lds_sync();
      for (int j = 0; j < cnt; ++j) {
        const float vj = svw[lane][j];
#pragma unroll
        for (int h = 0; h < GP; ++h) acc[h][r] += spw[h][j] * vj;
      }
    }
  }
  if (__any(bad) && lane == 0) flag_error(a.err, KVATTN_ERR_BAD_BLOCK);

  // Exact merge of the waves' states: M = max_w m_w, l = sum_w l_w e^(m_w - M),
  // o = sum_w acc_w e^(m_w - M) / l, lse = M + ln l (waves without a chunk: m = -inf, weight 0).
  __syncthreads();  // every wave's staging reads are done: the V areas take the outputs
  float* so = &sv[wv][0][0];  // [GP][D] unnormalised output of this wave
#pragma unroll
  for (int h = 0; h < GP; ++h) {
#pragma unroll
    for (int r = 0; r < R; ++r) so[h * D + lane + 64 * r] = acc[h][r];
    if (lane == 0) {
      sml[wv][0][h] = m[h];
      sml[wv][1][h] = l[h];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += 64 * kGW) {
    const int h = i / D, d = i - (i / D) * D;
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kGW; ++u) mx = fmaxf(mx, sml[u][0][h]);
    const float mref = mx == kNegInf ? 0.f : mx;
    float ls = 0.f, o = 0.f;
#pragma unroll
    for (int u = 0; u < kGW; ++u) {
      const float e = expf(sml[u][0][h] - mref);  // 0 for a wave without tokens
      ls += sml[u][1][h] * e;
      o += (&sv[u][0][0])[h * D + d] * e;
    }
    const int64_t row = ((int64_t)b * a.hq + kvh * G + h) * a.max_parts + k;
    a.o_part[row * D + d] = ls > 0.f ? o / ls : 0.f;
    if (d == 0) a.lse_part[row] = mx + logf(ls);
  }
}

// ------------------------------------------------------------------ launchers
int gqa_mfma_max_group(int d) {
  switch (d) {
    case 64: return mfma_max_group<64>();
    case 128: return mfma_max_group<128>();
    case 256: return mfma_max_group<256>();
    default: return 0;
  }
}

template <int D, int BSL>
static hipError_t launch_mfma_db(const DecodeArgs& a, dim3 grid, size_t lds, bool stream,
                                 hipStream_t st) {
  constexpr int PAIRS = D <= 128 ? 2 : 1;  // tile pairs held in registers
  const dim3 block(64 * (a.group_parts / a.wave_parts));
  if (stream)
    hipLaunchKernelGGL((gqa_decode_mfma_kernel<D, BSL, PAIRS, true>), grid, block, lds, st, a);
  else
    hipLaunchKernelGGL((gqa_decode_mfma_kernel<D, BSL, PAIRS, false>), grid, block, lds, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_d(const DecodeArgs& a, dim3 grid, size_t lds, bool stream,
                                hipStream_t st) {
  switch (a.bs_shift) {
    case 4: return launch_mfma_db<D, 4>(a, grid, lds, stream, st);
    case 5: return launch_mfma_db<D, 5>(a, grid, lds, stream, st);
    case 6: return launch_mfma_db<D, 6>(a, grid, lds, stream, st);
    case 7: return launch_mfma_db<D, 7>(a, grid, lds, stream, st);
    case 8: return launch_mfma_db<D, 8>(a, grid, lds, stream, st);
    default: return hipErrorInvalidValue;
  }
}

size_t gqa_mfma_lds_bytes(int waves, int group, int d) {
  return waves > 1 ? (size_t)waves * group * (gqa_merge_row(waves, group, d) + 1) * sizeof(float) : 0;
}

// `stream`: non-temporal K/V loads (every block read once per step); otherwise
// cache-retaining loads, for pools whose blocks are shared by several sequences.
hipError_t launch_gqa_mfma(const DecodeArgs& a, int d, bool stream, dim3 grid, hipStream_t st) {
  const size_t lds = gqa_mfma_lds_bytes(a.group_parts / a.wave_parts, a.group, d);
  switch (d) {
    case 64: return launch_mfma_d<64>(a, grid, lds, stream, st);
    case 128: return launch_mfma_d<128>(a, grid, lds, stream, st);
    case 256: return launch_mfma_d<256>(a, grid, lds, stream, st);
    default: return hipErrorInvalidValue;
  }
}

// Workgroups of the plan kernel one CU holds at once (its register use and four-wave
// workgroups), per instantiation; 2 if the runtime does not say.
template <int D, int BSL, int PAIRS>
static int plan_groups_per_cu() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_decode_plan_kernel<D, BSL, PAIRS, true>,
                                                   64 * kWavesPerGroup, plan_lds_bytes(D)) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    n = 2;
  }
  cached.store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int BSL>
static hipError_t launch_plan_db(const DecodeArgs& a, const int32_t* plan, int32_t n_groups,
                                 uint32_t* work, int cus, hipStream_t st) {
  constexpr int PAIRS = D <= 128 ? 2 : 1;
  // one workgroup per unit, the KV heads of a plan workgroup next to each other: the launch
  // then dispatches the plan's order (longest wave item first) for every head, rather than
  // the first head's whole plan before the second's
  const int64_t units = (int64_t)n_groups * a.hkv;
  dim3 grid((unsigned)std::max<int64_t>(1, units), 1);
  if (work) {
    const int64_t resident = (int64_t)(cus > 0 ? cus : 256) * plan_groups_per_cu<D, BSL, PAIRS>();
    grid = dim3((unsigned)std::max<int64_t>(1, std::min(units, resident)), 1);
  }
  if (work)
    hipLaunchKernelGGL((gqa_decode_plan_kernel<D, BSL, PAIRS, true>), grid,
                       dim3(64 * kWavesPerGroup), plan_lds_bytes(D), st, a, plan, n_groups, work);
  else
    hipLaunchKernelGGL((gqa_decode_plan_kernel<D, BSL, PAIRS, false>), grid,
                       dim3(64 * kWavesPerGroup), plan_lds_bytes(D), st, a, plan, n_groups, work);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_plan_d(const DecodeArgs& a, const int32_t* plan, int32_t n_groups,
                                uint32_t* work, int cus, hipStream_t st) {
  switch (a.bs_shift) {
    case 4: return launch_plan_db<D, 4>(a, plan, n_groups, work, cus, st);
    case 5: return launch_plan_db<D, 5>(a, plan, n_groups, work, cus, st);
    case 6: return launch_plan_db<D, 6>(a, plan, n_groups, work, cus, st);
    case 7: return launch_plan_db<D, 7>(a, plan, n_groups, work, cus, st);
    case 8: return launch_plan_db<D, 8>(a, plan, n_groups, work, cus, st);
    default: return hipErrorInvalidValue;
  }
}

// The plan kernel; with an empty plan (n_groups = 0) one workgroup only writes the partial
// counts (all zero).  work: the two-counter workspace (NULL: one unit per workgroup).
hipError_t launch_gqa_plan(const DecodeArgs& a, int d, const int32_t* plan, int32_t n_groups,
                           uint32_t* work, int cus, hipStream_t st) {
  switch (d) {
    case 64: return launch_plan_d<64>(a, plan, n_groups, work, cus, st);
    case 128: return launch_plan_d<128>(a, plan, n_groups, work, cus, st);
    case 256: return launch_plan_d<256>(a, plan, n_groups, work, cus, st);
    default: return hipErrorInvalidValue;
  }
}

// The probe is built for the block size of 16 (the benchmark layers); other geometries
// return hipErrorInvalidValue.  `stream` selects the decode kernel's cache hint.
template <bool NT>
static hipError_t launch_gqa_probe_nt(const DecodeArgs& a, int d, dim3 grid, uint32_t* xsum,
                                      hipStream_t st) {
  const dim3 block(64 * (a.group_parts / a.wave_parts));
  switch (d) {
    case 64: hipLaunchKernelGGL((gqa_probe_kernel<64, 4, 2, NT>), grid, block, 0, st, a, xsum); break;
    case 128: hipLaunchKernelGGL((gqa_probe_kernel<128, 4, 2, NT>), grid, block, 0, st, a, xsum); break;
    case 256: hipLaunchKernelGGL((gqa_probe_kernel<256, 4, 1, NT>), grid, block, 0, st, a, xsum); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gqa_probe(const DecodeArgs& a, int d, bool stream, dim3 grid, uint32_t* xsum,
                            hipStream_t st) {
  if (a.bs_shift != 4) return hipErrorInvalidValue;
  return stream ? launch_gqa_probe_nt<true>(a, d, grid, xsum, st)
                : launch_gqa_probe_nt<false>(a, d, grid, xsum, st);
}

template <typename T, int GP>
static hipError_t launch_generic_tg(const DecodeArgs& a, int d, dim3 grid, hipStream_t st) {
  switch (d) {
    case 64: hipLaunchKernelGGL((gqa_decode_generic_kernel<T, 64, GP>), grid, dim3(64 * kGW), 0, st, a); break;
    case 128: hipLaunchKernelGGL((gqa_decode_generic_kernel<T, 128, GP>), grid, dim3(64 * kGW), 0, st, a); break;
    case 256: hipLaunchKernelGGL((gqa_decode_generic_kernel<T, 256, GP>), grid, dim3(64 * kGW), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_generic_t(const DecodeArgs& a, int d, dim3 grid, hipStream_t st) {
  if (a.group <= 1) return launch_generic_tg<T, 1>(a, d, grid, st);
  if (a.group <= 2) return launch_generic_tg<T, 2>(a, d, grid, st);
  if (a.group <= 4) return launch_generic_tg<T, 4>(a, d, grid, st);
  if (a.group <= 8) return launch_generic_tg<T, 8>(a, d, grid, st);
  return launch_generic_tg<T, 16>(a, d, grid, st);
}

hipError_t launch_gqa_generic(const DecodeArgs& a, int d, bool f32, dim3 grid, hipStream_t st) {
  return f32 ? launch_generic_t<float>(a, d, grid, st) : launch_generic_t<uint16_t>(a, d, grid, st);
}

}  // namespace kvattn
