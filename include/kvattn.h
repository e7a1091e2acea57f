/*
 * kvattn.h -- C ABI of a paged-KV decode-attention library for AMD MI355X (gfx950).
 *
 * Sources this interface follows (cited below by the tag in brackets):
 *   [InplaceKVCache] "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in
 *                    MoE Inference" (Yu, Dong, Liao)
 *   [CrossPool]      "CrossPool: Efficient Multi-LLM Serving for Cold MoE Models through
 *                    KV-Cache and Weight Disaggregation"
 *   [VAMP]           "Dynamic HBM Repartitioning for Multi-Turn MoE Serving"
 *
 * What it computes.  One decode step of exact attention for one new query token per
 * sequence, o = softmax(scale * q K^T) V, over a KV cache held in fixed-size blocks
 * ([InplaceKVCache] §4.1: every region is organised in fixed-size blocks; [CrossPool] §3.1:
 * kernels address a logical KV space through a paged interface while physical pages are
 * placed elsewhere).  A per-sequence block table maps logical block i to a physical block
 * id; physical ids index the union of several caller-owned device regions, e.g. the base KV
 * region plus HBM reclaimed from expert weights ([VAMP] §IV-C, §V-A: reclaimed pages join
 * the free-block pool).  Each sequence's token range is cut into partitions that each emit a
 * partial (o, lse) pair; an exact log-sum-exp merge folds them together, optionally with one
 * more partial computed elsewhere, e.g. a CPU share of the context ([InplaceKVCache] §4.2
 * and §5.1: the two engines cover disjoint sequence ranges over all heads and their partial
 * outputs merge exactly by LSE rescaling, one join per step, on the GPU).
 *
 * Conventions shared by every call:
 *   - Every function returns kvattn_status (0 = OK, < 0 = error) unless stated otherwise;
 *     kvattn_last_error() returns a message for the last failure on the calling thread.
 *   - "host" pointers are ordinary CPU memory read synchronously; "device" pointers are
 *     HIP device memory owned by the caller.  The library never allocates device memory.
 *   - Device work is enqueued asynchronously on the caller's HIP stream (hipStream_t passed
 *     as void*; NULL = the null stream).  Argument validation is synchronous: a call that
 *     returns an error has enqueued nothing.  Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - lse is the natural logarithm of the sum of exp(scaled score) over the partial's tokens.
 *     An empty partial has lse = -INFINITY and o = 0 and carries no weight in a merge.
 *
 * KV block layout in a region (element type e = 4 bytes for F32, 2 for BF16; x = 16 / e
 * elements per 16-byte chunk; bs = block_size; Hkv = num_kv_heads; Dk, Dv head dims):
 *   GQA (latent = 0):  block = [ K part | V part ], Hkv * bs * (Dk + Dv) elements.
 *       K(h, t, i) at element  ((h * (Dk / x) + i / x) * bs + t) * x + i % x
 *       V(h, t, j) at element  Hkv * bs * Dk + (h * Dv + j) * bs + t
 *     i.e. K is stored in 16-byte chunks of one token, the chunks of bs consecutive tokens
 *     side by side; V is stored transposed (token index fastest).
 *   MLA (latent = 1):  block = bs * Dk elements, Hkv must be 1, Dv <= Dk, Dv % x == 0.
 *       C(t, i) at element  ((i / x) * bs + t) * x + i % x     (K(t, i) = C(t, i),
 *       V(t, j) = C(t, j) for j < Dv: the value is the leading Dv columns of the latent).
 *   Block id n of region r (regions numbered in the order passed to kvattn_pool_alloc, ids
 *   consecutive across regions) starts at byte (n - first_id(r)) * block_bytes of region r.
 *   The layout is this library's choice: the pages fix only that blocks have a fixed size.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvattn_status;

enum {
  KVATTN_OK = 0,
  KVATTN_E_INVAL = -1,          /* bad argument: null pointer, size, alignment, inconsistency */
  KVATTN_E_POOL_EXHAUSTED = -2, /* not enough free blocks; pool and outputs left unchanged */
  KVATTN_E_RANGE = -3,          /* a block id outside [0, pool blocks) */
  KVATTN_E_STATE = -4,          /* block in the wrong state: claim of a used block, double release */
  KVATTN_E_UNSUPPORTED = -5,    /* shape / dtype combination without a kernel */
  KVATTN_E_HIP = -6             /* HIP runtime error while enqueueing */
};

enum { KVATTN_F32 = 0, KVATTN_BF16 = 1 };

#define KVATTN_BLOCK_ABSENT (-1) /* table entry with no block on this device */
#define KVATTN_MAX_REGIONS 8
#define KVATTN_MAX_GROUP_PARTS 16 /* largest group_parts of kvattn_decode_partial */

/* Error bits a decode kernel may set in *err_dev (see kvattn_decode_partial). */
#define KVATTN_ERR_BAD_BLOCK 1   /* a table entry inside a sequence's range is not a valid id */
#define KVATTN_ERR_BAD_SEQ 2     /* device per-sequence values disagree with the host ones */
#define KVATTN_ERR_BAD_SELECT 4  /* a selected block index outside the context, or repeated */

typedef struct {
  int32_t block_size;   /* tokens per block bs; power of two in [1, 256] */
  int32_t num_kv_heads; /* Hkv; 1 for a latent cache */
  int32_t head_dim_k;   /* Dk: key (latent) dimension; multiple of x */
  int32_t head_dim_v;   /* Dv: value dimension; multiple of x */
  int32_t kv_dtype;     /* KVATTN_F32 or KVATTN_BF16 */
  int32_t latent;       /* 0 = per-head K and V (GQA); 1 = shared latent (MLA) */
} kvattn_layout;

typedef struct {
  void* base;         /* device address of the region, 16-byte aligned; caller-owned */
  int64_t num_blocks; /* number of whole blocks the region holds */
} kvattn_region;

typedef struct kvattn_pool kvattn_pool; /* opaque host metadata: regions, free list, refcounts */

/* Bytes of one block under `layout`, or -1 if the layout is invalid. */
int64_t kvattn_block_bytes(const kvattn_layout* layout);

/*
 * Create a block pool over 1..KVATTN_MAX_REGIONS caller-owned device regions
 * ([VAMP] §IV-C and §V-A: HBM reclaimed from expert weights is inserted into the free-block
 * pool beside the base KV region; [InplaceKVCache] §4.1: fixed-size blocks are the unit).
 * Block ids are consecutive over the regions in the order given.  The free list starts as
 * a Fisher-Yates shuffle of all ids driven by SplitMix64 seeded with `seed`: with
 * state = seed, for i = N-1 down to 1: j = splitmix64_next(&state) % (i + 1), swap(ids[i],
 * ids[j]); blocks are then handed out in the order ids[0], ids[1], ...  (A released block
 * is handed out before any block never used: the free list is a stack.)
 * `out` receives a pool the caller frees with kvattn_pool_free.  Only host memory is used.
 * Errors: E_INVAL (null pointers, bad layout, zero regions, misaligned or null base,
 * a region with num_blocks < 0, more than 2^31-1 blocks in total).
 */
kvattn_status kvattn_pool_alloc(const kvattn_layout* layout, const kvattn_region* regions,
                                int32_t n_regions, uint64_t seed, kvattn_pool** out);

/*
 * Growth and shrinking of a pool at run time ([VAMP] §IV-C: physical HBM pages move between the
 * expert weights and the KV pool; §V-A: reclaimed pages join the free-block pool at once, and
 * the remapping primitive also runs in reverse; it moves a contiguous high-index region).
 *  - kvattn_pool_add_region: appends a region (device address, 16-byte aligned, caller-owned)
 *    of num_blocks blocks as region n_regions; its ids are [total, total + num_blocks), written
 *    to *first_id, and go on top of the free list so that they are handed out first, in
 *    ascending order.  E_INVAL: null pointers, misalignment, num_blocks < 1, already
 *    KVATTN_MAX_REGIONS regions, more than 2^31-1 blocks.
 *  - kvattn_pool_resize_last_region: sets the block count of the last region.  Growing appends
 *    ids as above: the caller guarantees that the memory after the region's current end is
 *    valid device memory (e.g. newly mapped pages of a reserved range).  Shrinking removes the
 *    highest ids, which must all be free (E_STATE otherwise); 0 removes the region (E_INVAL if
 *    it is the only one).  The removed ids leave the free list; other ids keep their order.
 * Tables and kernels refer to blocks by id and each launch carries the region table it was
 * given, so decodes enqueued before a change are unaffected; a shrink must not remove memory
 * that work still in flight reads (the removed blocks are free, but synchronise before
 * unmapping their pages).
 */
kvattn_status kvattn_pool_add_region(kvattn_pool* pool, void* base, int64_t num_blocks,
                                     int64_t* first_id);
kvattn_status kvattn_pool_resize_last_region(kvattn_pool* pool, int64_t num_blocks);
/* Number of regions (-1 for NULL). */
int32_t kvattn_pool_num_regions(const kvattn_pool* pool);

/*
 * Reserved device address ranges with movable physical pages ([VAMP] §IV-C: the physical pages
 * behind expert weights are unmapped and remapped into the KV pool while the experts' address
 * ranges stay reserved; §V-A: the remap unit is a multiple of the allocation granularity and the
 * primitive also runs in reverse).
 *  - create: reserves va_bytes (rounded up to the chunk size) of address space on `device`;
 *    nothing is mapped.  Pages are created, mapped and moved in chunks of chunk_bytes (a
 *    multiple of the device's minimum allocation granularity; 0 = the runtime's recommended
 *    granularity), reported by kvattn_vmm_granularity.  E_UNSUPPORTED if the device has no
 *    virtual memory management.
 *  - map_new: backs [offset, offset + bytes) with new physical memory, granule by granule,
 *    read-write for the device (E_STATE if part of it is mapped).  Contents are undefined.
 *  - move: takes the physical granules behind src[src_offset, + bytes) and maps them at
 *    dst[dst_offset, + bytes): the contents move with them, nothing is copied; the source
 *    range stays reserved and becomes unmapped.  The source must be fully mapped and the
 *    destination fully unmapped (E_STATE otherwise); both ranges on one device.  With
 *    sync_device != 0 the device is synchronised first, so no work in flight can still read
 *    the source; with 0 the caller guarantees that none does.
 *  - free: synchronises the device, unmaps and releases every granule, frees the range.
 * Offsets and sizes are multiples of the chunk size (E_INVAL otherwise).  Mapping new
 * pages never disturbs work in flight; a pool grows over a moved or mapped range with
 * kvattn_pool_add_region / kvattn_pool_resize_last_region.  Not thread-safe.
 * Errors also: E_INVAL for null pointers or a zero size, E_HIP (the range may then be partly
 * updated; kvattn_vmm_mapped_bytes tells how much is mapped).
 */
typedef struct kvattn_vmm kvattn_vmm;

kvattn_status kvattn_vmm_create(int32_t device, uint64_t va_bytes, uint64_t chunk_bytes,
                                kvattn_vmm** out);
void kvattn_vmm_free(kvattn_vmm* vmm);
uint64_t kvattn_vmm_granularity(const kvattn_vmm* vmm);
void* kvattn_vmm_base(const kvattn_vmm* vmm);
uint64_t kvattn_vmm_mapped_bytes(const kvattn_vmm* vmm);
kvattn_status kvattn_vmm_map_new(kvattn_vmm* vmm, uint64_t offset, uint64_t bytes);
kvattn_status kvattn_vmm_move(kvattn_vmm* src, uint64_t src_offset, kvattn_vmm* dst,
                              uint64_t dst_offset, uint64_t bytes, int32_t sync_device);

/* Release the pool's host metadata; the regions stay the caller's.  NULL is ignored.  While a
 * kvattn_kvstore still holds the pool, the release is deferred until the last such store is
 * freed (the pool must not be used by the caller after this call either way). */
void kvattn_pool_free(kvattn_pool* pool);

/*
 * Fill a block table for `batch` sequences ([CrossPool] §3.1: the virtualiser, not the
 * kernel, chooses physical pages; when the page budget runs out the request is queued or
 * rejected and running decodes are left alone).  All host memory.  Row b of table_out
 * (max_blocks entries) maps logical block i of sequence b to a physical id, or to
 * KVATTN_BLOCK_ABSENT.  Sequence b needs nb = ceil(ctx_lens[b] / bs) entries; entries
 * from nb on are ABSENT.  Two modes:
 *
 * Allocate (explicit_table == NULL), sequences processed in order b = 0, 1, ...:
 *   - entries i < first_tok[b] / bs (integer division) are ABSENT: the tokens before
 *     first_tok[b] live elsewhere (e.g. the CPU share); NULL means 0 for every sequence.
 *   - if share_src != NULL and share_src[b] >= 0, entries i < share_nblocks[b] are copied
 *     from row share_src[b] (which must be < b, resident there, and i < nb of both rows)
 *     and each shared block's reference count rises by one (prefix sharing);
 *     a sequence cannot both share and have ABSENT entries.
 *   - every remaining entry below nb takes the next block of the free list, refcount 1.
 *   All or nothing: if the free list is short, returns E_POOL_EXHAUSTED, writes the
 *   number of missing blocks to *shortfall_out (if non-NULL) and changes nothing.
 *
 * Explicit (explicit_table != NULL, [batch][max_blocks]): the caller chose the ids.  Each
 *   entry must be ABSENT or an id in range (else E_RANGE); entries from nb on must be
 *   ABSENT (else E_INVAL); every referenced id must be free (else E_STATE).  A block named
 *   k times gets refcount k and leaves the free list; table_out receives a copy.
 *
 * first_tok, share_src and share_nblocks are ignored in explicit mode.
 * Errors: E_INVAL, E_RANGE, E_STATE, E_POOL_EXHAUSTED, each leaving the pool unchanged.
 */
kvattn_status kvattn_block_table(kvattn_pool* pool, int32_t batch, const int32_t* ctx_lens,
                                 const int32_t* first_tok, const int32_t* share_src,
                                 const int32_t* share_nblocks, const int32_t* explicit_table,
                                 int32_t max_blocks, int32_t* table_out, int64_t* shortfall_out);

/*
 * Drop one reference for every non-ABSENT entry of a [batch][max_blocks] host table; a
 * block whose count reaches zero returns to the top of the free list (in table order).
 * All or nothing: E_RANGE for an id out of range, E_STATE if some block would drop below
 * zero references (e.g. a second release of the same table); then nothing changes.
 */
kvattn_status kvattn_block_release(kvattn_pool* pool, const int32_t* table, int32_t batch,
                                   int32_t max_blocks);

/* Free blocks left in the pool, or -1 for NULL. */
int64_t kvattn_pool_num_free(const kvattn_pool* pool);

/* Blocks referenced by two or more table entries (shared prefixes), or -1 for NULL.  While
 * the pool holds shared blocks, the bf16 GQA decode kernel reads K/V with cache-retaining
 * loads so that sequences sharing a prefix can reuse its blocks from the caches; otherwise
 * it streams them with non-temporal loads (every block is read once per step). */
int64_t kvattn_pool_shared_blocks(const kvattn_pool* pool);

/* Reference count of block `id`, or -1 if out of range. */
int32_t kvattn_pool_refcount(const kvattn_pool* pool, int32_t id);

/*
 * Number of partitions of a sequence whose device-resident range is [tok_begin, ctx_len),
 * cut into pieces of part_tokens tokens: ceil((ctx_len - tok_begin) / part_tokens), and 0
 * for an empty range.  Partition p covers [tok_begin + p * part_tokens,
 * min(ctx_len, tok_begin + (p + 1) * part_tokens)).  Returns -1 for invalid arguments
 * (negative values, tok_begin > ctx_len, part_tokens <= 0).  ([InplaceKVCache] §5.1: the
 * split is along the sequence, each engine over all heads.)
 */
int32_t kvattn_partition_count(int32_t ctx_len, int32_t tok_begin, int32_t part_tokens);

/*
 * One decode step's partial attention ([InplaceKVCache] §5.1 and §6.1: exact attention,
 * online softmax with a running max and normaliser, fp32 accumulation; sequence-dimension
 * split).  The device-resident range [tok_begin[b], ctx_lens[b]) of every sequence b is cut
 * into partitions of part_tokens[b] tokens (geometry as in kvattn_partition_count), and
 * consecutive partitions are taken group_parts at a time: group k of sequence b covers
 * partitions [k * group_parts, min(np_b, (k + 1) * group_parts)), i.e. the tokens
 *     [tok_begin + k * group_parts * part_tokens, min(ctx_len, tok_begin + (k+1) * ...)).
 * For every group and query head h (KV head h / (Hq / Hkv): consecutive query heads share a
 * KV head; MLA: all heads share the latent) one partial is written:
 *     o_part[b][h][k][:] = sum_t w_t V(t) / sum_t w_t,  w_t = exp(s_t - max s),
 *     s_t = scale * q[b][h] . K(t),      lse_part[b][h][k] = max s + ln(sum_t w_t)
 * over the group's tokens t.  The matrix-core GQA kernel spreads a group's partitions over
 * the waves of one workgroup (two consecutive partitions per wave when group_parts is even
 * and at least 4 and two partitions span at most 127 blocks, else one) and merges the waves'
 * partials on chip, exactly, by the LSE rescaling of kvattn_merge_lse; the latent (MLA)
 * kernel gives the group's even and odd blocks to two teams of waves and merges the two the
 * same way; the VALU kernel gives the group's 64-token chunks to four waves in turn and merges
 * them the same way.  group_parts = 1
 * writes one partial per partition; larger groups write fewer partials, which is faster on
 * long contexts (partial writes compete with the K/V read stream).  Logical token t of
 * sequence b lives at offset t % bs of physical block table_dev[b][t / bs].
 *
 *   q            device [batch][num_q_heads][Dk], element type q_dtype (must equal kv_dtype)
 *   table_dev    device [batch][max_blocks] int32 (entries of the range must be valid ids)
 *   ctx_lens, tok_begin (NULL = 0), part_tokens: host [batch] int32 used for validation and
 *                grid sizing; seq_dev: device int32 [3][batch] holding the same three arrays
 *                (row 1 all zeros if tok_begin is NULL), read by the kernels.
 *   max_parts    partials per sequence the o_part / lse_part arrays have room for
 *   group_parts  partitions per written partial, 1 .. KVATTN_MAX_GROUP_PARTS, or 0: the
 *                library's choice for the current device, kvattn_choose_group_parts(..., 0)
 *   o_part       device fp32 [batch][num_q_heads][max_parts][Dv]
 *   lse_part     device fp32 [batch][num_q_heads][max_parts]
 *   nparts_dev   device int32 [batch]: receives the number of partials written for each
 *                sequence, ceil(np_b / group_parts)
 *   err_dev      device int32 or NULL: KVATTN_ERR_* bits are OR-ed in (never cleared) if a
 *                kernel meets an invalid block id or device lengths that disagree with the
 *                host ones; the offending block contributes nothing / the sequence gets no
 *                partials, and no memory outside the arguments is touched.
 * Entries of o_part / lse_part for k >= nparts[b] are not written.
 * Validation (E_INVAL): null pointers, batch < 1, num_q_heads % Hkv != 0, per sequence
 * 0 <= tok_begin <= ctx_len <= max_blocks * bs, part_tokens > 0 and part_tokens % bs == 0,
 * partials per sequence <= max_parts, group_parts outside [0, KVATTN_MAX_GROUP_PARTS].
 * E_UNSUPPORTED: q_dtype != kv_dtype, or a head / dim combination without a kernel (GQA:
 * Dk = Dv in {64, 128, 256}, Hq / Hkv <= 16; MLA: BF16, Dk = 576, Dv = 512, Hq <= 16,
 * bs = 64); for the bf16 GQA kernel (block size >= 16) also a group needing more than 16
 * waves (Dk 64) or 8 waves (Dk 128, 256), or waves * (Hq / Hkv) * (Dk + 1) * 4 > 65536 bytes
 * of LDS.  E_HIP: launch failure.
 */
kvattn_status kvattn_decode_partial(const kvattn_pool* pool, const void* q, int32_t q_dtype,
                                    int32_t batch, int32_t num_q_heads, float scale,
                                    const int32_t* table_dev, int32_t max_blocks,
                                    const int32_t* ctx_lens, const int32_t* tok_begin,
                                    const int32_t* part_tokens, const int32_t* seq_dev,
                                    int32_t max_parts, int32_t group_parts, float* o_part,
                                    float* lse_part, int32_t* nparts_dev, int32_t* err_dev,
                                    void* hip_stream);

/*
 * The group_parts kvattn_decode_partial uses when passed 0, so that a caller can size
 * max_parts (ceil(partitions / group_parts) per sequence) for it.  A host-only rule over the
 * launch's work items W(g) = sum over sequences (x KV heads for GQA) of ceil(np_b / g), fitted
 * to decode-step sweeps on MI355X ([InplaceKVCache] §5.1: any grouping of the partitions of a
 * sequence merges to the same result, so the choice is free):
 *   latent (MLA) kernel: the largest g in {16, 8, 4, 2} with W(g) >= num_cus, else 1;
 *   matrix-core GQA kernel: 1 while W(1) < 8 num_cus; else the largest g in {16, 8, 4, 2}
 *     that the kernel allows (waves per CU, LDS) with W(g) a positive multiple of num_cus, else
 *     the largest with W(g) >= num_cus, else 1; at most 2 while the pool holds shared blocks;
 *   VALU kernel (fp32 caches, block size < 16): 2 once W(1) >= 4 num_cus, else 1.
 * num_cus: compute units to plan for; <= 0 = those of the current HIP device (256 if there is
 * none).  Arguments as for kvattn_decode_partial (host arrays).  Returns g >= 1, or a negative
 * status (E_INVAL for invalid arguments, E_UNSUPPORTED for a shape without a kernel).
 */
int32_t kvattn_choose_group_parts(const kvattn_pool* pool, int32_t batch, int32_t num_q_heads,
                                  const int32_t* ctx_lens, const int32_t* tok_begin,
                                  const int32_t* part_tokens, int32_t num_cus);

/*
 * ---- Decode over a work plan: sequences holding the same blocks share one pass ----
 *
 * Prefix caching hands the same physical blocks to several sequences ([VAMP] §II-A: cached
 * prefixes are reused across turns and requests; [CrossPool] §3.1: the paged interface makes
 * them ordinary table entries).  Where two sequences have the same token range in the same
 * blocks, the range's keys and values are the same, so one pass over them serves both; each
 * sequence still gets its own partial of the range, merged like any other ([InplaceKVCache]
 * §5.1: partials over a partition of the tokens merge exactly).
 *
 * kvattn_decode_plan (host only) reads the host copy of the tables.  Block position i of
 * sequence b (its tokens [max(tok_begin, i bs), min(ctx_len, (i + 1) bs))) is shared with
 * every sequence whose position i holds the same block id with the same token extent; the
 * sharers of a position form its set.  Each maximal run of positions of a sequence with the
 * same set (an invalid id: a set of its own sequence) is taken once, from the set's lowest
 * sequence, and cut into pieces of at most span_parts * part_tokens tokens (span_parts 0: as
 * many whole partitions as a wave's window of 127 block ids holds); a piece becomes wave
 * items of up to 16 / (Hq / Hkv) of its sequences each.  A piece of k >= 3 items runs in
 * ceil(k / 4) workgroups of its own whose four waves stage the range through LDS together
 * (mode 2: it crosses HBM once per such workgroup; a workgroup of fewer items is padded with
 * items of no sequence); the two items of a piece of k = 2 run as two waves of one workgroup
 * (mode 1); single items, shared or private, are streamed by one wave (mode 0).  Workgroups
 * other than staged ones hold four independent waves.  Every sequence's range [tok_begin, ctx_len) is
 * thus covered exactly once by the items it belongs to; its partials are written in the
 * order of their first tokens, slots 0 .. nparts[b] - 1.  The plan is an int32 array:
 *   header[8] = {magic, batch, n_groups, 4 n_groups, member entries M, max_parts,
 *                Hq / Hkv, sequences per wave item}, nparts[batch],
 *   items[4 n_groups][6] = {table row, first token, end token, sequences (0: idle wave),
 *                           first member entry, mode 0 / 1 / 2},
 *   members[M][2] = {sequence, partial slot}.
 *   table        host [batch][max_blocks] int32 (the device copy's contents)
 *   plan         host int32 [plan_cap], or NULL to query the size only.  plan_len never
 *                exceeds 8 + batch + 26 P, P the block positions of all ranges (sequence b:
 *                (ctx_len - 1) / bs - tok_begin / bs + 1 when ctx_len > tok_begin), so a
 *                buffer of that size needs one call
 *   plan_len     receives the plan's length in int32 entries
 *   n_groups     receives the workgroups of the plan (the grid of kvattn_decode_partial_plan)
 *   max_parts    receives the most partials any sequence gets (size o_part / lse_part for it)
 * Errors: E_INVAL (null pointers, sizes, per-sequence values as for kvattn_decode_partial,
 * plan_cap < plan_len), E_UNSUPPORTED (not a bf16 per-head cache with block size >= 16 and
 * head dim 64, 128 or 256; more than 16 query heads per KV head; span_parts * part_tokens
 * spanning more than 127 blocks).
 *
 * kvattn_decode_partial_plan runs a plan (uploaded by the caller to plan_dev) on the
 * device: for every item and KV head, the attention of its sequences' query heads over its
 * token range, read once through the table row it names; sequence b's partial of item k goes
 * to o_part[b][h][slot] / lse_part[b][h][slot] (same formulas as kvattn_decode_partial) and
 * nparts_dev[b] receives the plan's count, so kvattn_merge_lse completes the step.  Mode 0
 * streams its range with non-temporal loads, mode 1 reads it with cache-retaining loads (the
 * other waves of its range hit in L2), and a mode-2 workgroup (all four items mode 2 with one
 * range, else KVATTN_ERR_BAD_SEQ) loads it into LDS once for its four waves.
 *   q, q_dtype, batch, num_q_heads, scale, table_dev, max_blocks, o_part, lse_part, err_dev:
 *                as for kvattn_decode_partial (max_parts >= the plan's max_parts)
 *   plan_dev     device int32 copy of the plan (all plan_len entries); n_groups its workgroups
 *   work_dev     device uint32 [2] work counters, or NULL.  NULL: one workgroup per (plan
 *                workgroup, KV head) unit, unit u = plan workgroup u / Hkv, KV head u % Hkv,
 *                launched in that order (n_groups x Hkv at most 2^31 - 1).  Given: as many
 *                workgroups as the device holds at once, each running units in that order and
 *                taking the next one from the counters when it is done, so that the
 *                CUs and XCDs that finish first take more (the partials do not depend on which
 *                workgroup ran a unit: the result is the same bit for bit).  The counters must
 *                be zero before the first call (e.g. zero-filled once); every call that
 *                completes leaves them zero again.  Calls that overlap on one work_dev race.
 * A plan whose header disagrees with the arguments (its max_parts above the call's included),
 * or an item outside them, sets KVATTN_ERR_BAD_SEQ in *err_dev and is not run (the counters
 * are then left as they are);
 * invalid block ids set KVATTN_ERR_BAD_BLOCK and contribute nothing.  Errors: E_INVAL (null
 * pointers, misalignment (work_dev: 8 bytes), sizes), E_UNSUPPORTED
 * (as for kvattn_decode_plan, or q_dtype != kv_dtype), E_HIP.
 */
kvattn_status kvattn_decode_plan(const kvattn_pool* pool, int32_t batch, int32_t num_q_heads,
                                 const int32_t* table, int32_t max_blocks,
                                 const int32_t* ctx_lens, const int32_t* tok_begin,
                                 const int32_t* part_tokens, int32_t span_parts, int32_t* plan,
                                 int64_t plan_cap, int64_t* plan_len, int32_t* n_groups,
                                 int32_t* max_parts);
kvattn_status kvattn_decode_partial_plan(const kvattn_pool* pool, const void* q, int32_t q_dtype,
                                         int32_t batch, int32_t num_q_heads, float scale,
                                         const int32_t* table_dev, int32_t max_blocks,
                                         const int32_t* plan_dev, int32_t n_groups,
                                         uint32_t* work_dev, int32_t max_parts, float* o_part,
                                         float* lse_part, int32_t* nparts_dev, int32_t* err_dev,
                                         void* hip_stream);

/*
 * kvattn_decode_partial_plan for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same call with the
 * work counters in a library-owned device array instead of work_dev.  The array is a
 * file-scope device variable of 64 uint32 (256 bytes) on every GPU the library runs on, held
 * until the process ends, and looked up once per device on the first call with that device
 * current; the call itself allocates nothing.  The plan kernel needs two of its words for any
 * sizes, so no call is refused for its size.  Every call on a GPU shares that GPU's array:
 * each completed call leaves the counters zero for the next, and calls that overlap on one
 * GPU (several streams at once) race.  Arguments, results and errors as for
 * kvattn_decode_partial_plan (results equal bit for bit); also E_HIP if the array's address
 * cannot be looked up, E_UNSUPPORTED for a device index of 64 or more.
 */
kvattn_status kvattn_decode_partial_plan_noalloc(const kvattn_pool* pool, const void* q,
                                                 int32_t q_dtype, int32_t batch,
                                                 int32_t num_q_heads, float scale,
                                                 const int32_t* table_dev, int32_t max_blocks,
                                                 const int32_t* plan_dev, int32_t n_groups,
                                                 int32_t max_parts, float* o_part,
                                                 float* lse_part, int32_t* nparts_dev,
                                                 int32_t* err_dev, void* hip_stream);

/*
 * Gather probe: the loads of kvattn_decode_partial's kernel for the same arguments -- the same
 * grid, waves, block-table lookups, load widths, cache hints and order -- with no arithmetic.
 * It measures the access pattern's own bandwidth ceiling on this device, which bounds what
 * the decode kernel can reach. It also returns a checksum of exactly what the kernel reads:
 *     xsum_dev[b][h] ^= XOR over the 16-bit elements of K(h, t, :) and V(h, t, :) of
 *                       every token t in [tok_begin_b, ctx_len_b)
 * (MLA: h = 0 and the 576-wide latent rows C(t, :), each element once).  The XOR is
 * order-free, so the checksum is exact and reproducible, and it pins the block-table
 * resolution bit for bit.
 *   Arguments as for kvattn_decode_partial (no q, scale or partials).
 *   xsum_dev  device uint32 [batch][num_kv_heads] (MLA: [batch]); the probe XORs into it, so
 *             the caller zeroes it first; only the low 16 bits are used.
 * Errors: those of kvattn_decode_partial's validation; E_INVAL for xsum_dev NULL;
 * E_UNSUPPORTED unless the cache is bf16 GQA with block size 16 (matrix-core kernel), or MLA.
 */
kvattn_status kvattn_gather_probe(const kvattn_pool* pool, int32_t batch, int32_t num_q_heads,
                                  const int32_t* table_dev, int32_t max_blocks,
                                  const int32_t* ctx_lens, const int32_t* tok_begin,
                                  const int32_t* part_tokens, const int32_t* seq_dev,
                                  int32_t group_parts, uint32_t* xsum_dev, int32_t* err_dev,
                                  void* hip_stream);

/*
 * Exact LSE merge of each (sequence, head)'s partials ([InplaceKVCache] §4.2, §5.1, §5.2:
 * the partial outputs and their normalisers are folded on the GPU, one join per step):
 *     M = max_p lse_p,  lse = M + ln sum_p exp(lse_p - M),  o = sum_p exp(lse_p - lse) o_p
 * over p < nparts_dev[b], plus, when o_ext != NULL, one external partial (o_ext[b][h],
 * lse_ext[b][h]) computed elsewhere (e.g. the CPU share of the context).  With no partial
 * of positive weight the result is o = 0, lse = -INFINITY.
 *   o_part, lse_part, nparts_dev  as written by kvattn_decode_partial (device)
 *   o_ext, lse_ext   device fp32 [batch][num_q_heads][dv] and [batch][num_q_heads], or both
 *                    NULL.  They may be the device addresses of mapped, coherent pinned host
 *                    memory (hipHostMalloc with hipHostMallocMapped | hipHostMallocCoherent):
 *                    the merge then reads a host-computed partial over the host link with no
 *                    copy; the caller must have finished writing it before this call.
 *   o_out            device fp32 [batch][num_q_heads][dv]
 *   lse_out          device fp32 [batch][num_q_heads] or NULL
 * Errors: E_INVAL (null required pointers, one of o_ext/lse_ext NULL but not the other,
 * batch/heads/max_parts < 1, dv not in [1, 1024] or not a multiple of 4 is E_UNSUPPORTED),
 * E_HIP.  The output may not alias the inputs.
 */
kvattn_status kvattn_merge_lse(const float* o_part, const float* lse_part,
                               const int32_t* nparts_dev, int32_t batch, int32_t num_q_heads,
                               int32_t max_parts, int32_t dv, const float* o_ext,
                               const float* lse_ext, float* o_out, float* lse_out,
                               void* hip_stream);

/*
 * Paged KV append ([InplaceKVCache] §4.1: the block is the unit of write-time placement;
 * §4.2: new decode entries are written first into the GPU's staging window and take part in
 * attention from the next step).  For every sequence b and j < n_new, writes the new token
 * j at logical index t = pos_dev[b] + j into block table_dev[b][t / bs], slot t % bs, in the
 * pool's block layout (header comment above): K(h, t, :) and V(h, t, :) for every KV head,
 * or the latent row C(t, :) of an MLA cache.
 *   k_new     device [batch][n_new][Hkv][Dk] (latent: [batch][n_new][Dk]), element type
 *             kv_dtype, 16-byte aligned
 *   v_new     device [batch][n_new][Hkv][Dv]; NULL exactly for a latent cache
 *   table_dev device [batch][max_blocks] int32; pos_dev device [batch] int32
 *   err_dev   device int32 or NULL: KVATTN_ERR_BAD_SEQ is OR-ed in for a token whose index
 *             is negative or beyond max_blocks * bs, KVATTN_ERR_BAD_BLOCK for a token whose
 *             table entry is not a valid id; such tokens are not written.
 * Blocks must have been claimed (kvattn_block_table, or a kvattn_kvstore reservation); the
 * kernel does not allocate.  Appends to distinct slots may share a launch; two writes to one
 * slot in one launch leave either value.  Errors: E_INVAL (null pointers, v_new present for a
 * latent cache or missing otherwise, sizes < 1, batch * n_new >= 2^31, misalignment),
 * E_UNSUPPORTED (kv_dtype != the pool's), E_HIP.
 */
kvattn_status kvattn_append_kv(const kvattn_pool* pool, const void* k_new, const void* v_new,
                               int32_t kv_dtype, int32_t batch, int32_t n_new,
                               const int32_t* table_dev, int32_t max_blocks,
                               const int32_t* pos_dev, int32_t* err_dev, void* hip_stream);

/*
 * Block-level sparse selection ([InplaceKVCache] §4.2, sparse-selection compatibility: a
 * block-level top-k selection yields a set of whole blocks, so sparsity needs no change to the
 * block format).  For every sequence b, builds on the device the sub-table of the blocks whose
 * logical indices sel_dev[b][0..k) name, so that the decode kernels attend exactly the tokens
 * of those blocks:
 *   sub_table_dev[b] = table[b][j] for the selected full blocks j in ascending order, then the
 *                      partial last block (if ctx_len % bs != 0 and it is selected), then
 *                      KVATTN_BLOCK_ABSENT up to max_sub;
 *   sub_len_dev[b]   = bs * (selected full blocks) + (ctx_len - bs * (nb - 1) if the partial
 *                      block is selected), nb = ceil(ctx_len / bs).
 * Attention does not depend on the order of the cached tokens, so the order is a choice: the
 * ascending one makes the result independent of the order of the selection.
 *   table_dev [batch][max_blocks], ctx_lens_dev [batch], sel_dev [batch][k]: device int32;
 *   negative entries of sel_dev are padding.  sub_table_dev [batch][max_sub], sub_len_dev
 *   [batch]: device int32 (sub_len_dev may be row 0 of a decode's seq_dev).
 *   err_dev (nullable): KVATTN_ERR_BAD_SELECT for an index >= nb or repeated (ignored),
 *   KVATTN_ERR_BAD_SEQ for ctx_len < 0 or nb > max_blocks (the sequence gets length 0).
 * To decode the selection, pass host upper bounds (k * bs per sequence) as ctx_lens of
 * kvattn_decode_partial with table_dev = sub_table_dev and max_blocks = max_sub: the grid is
 * sized by the bounds and the kernels use the device lengths.
 * Errors: E_INVAL (null pointers, batch < 1, k < 1, max_sub < k, max_blocks outside
 * [1, 65536], block_size not a power of two in [1, 256]), E_HIP.
 */
kvattn_status kvattn_select_blocks(const int32_t* table_dev, int32_t max_blocks,
                                   const int32_t* ctx_lens_dev, int32_t block_size,
                                   const int32_t* sel_dev, int32_t batch, int32_t k,
                                   int32_t* sub_table_dev, int32_t max_sub, int32_t* sub_len_dev,
                                   int32_t* err_dev, void* hip_stream);

/*
 * CPU share of a decode step, computed on the host ([InplaceKVCache] §5.1: the engines take
 * disjoint token ranges of every sequence over all heads; §4.2: the CPU returns only its
 * partial output and normaliser, which the GPU merges; §6.1: the CPU kernel reads the blocks
 * in place with an online softmax and fp32 accumulation, and for MLA reads each latent once
 * for all heads).  For every sequence b and query head h it writes the partial over tokens
 * [0, tok_end[b]):
 *     o_out[b][h][:] = sum_t w_t V(t) / sum_t w_t,   lse_out[b][h] = max s + ln(sum_t w_t)
 * (natural log; tok_end[b] = 0 gives o = 0, lse = -INFINITY), ready to be passed to
 * kvattn_merge_lse as the external partial once copied to the device.
 *   layout         block layout, exactly as for the device pool (header comment above)
 *   host_regions   1..KVATTN_MAX_REGIONS regions of host memory holding whole blocks; block ids
 *                  run consecutively over them in order (like kvattn_pool_alloc)
 *   q              host [batch][num_q_heads][Dk], element type q_dtype (= kv_dtype)
 *   table          host [batch][max_blocks] int32; entries below ceil(tok_end[b] / bs) must be
 *                  valid ids of the host regions (E_RANGE otherwise)
 *   tok_end        host [batch] int32, 0 <= tok_end[b] <= max_blocks * bs
 *   o_out, lse_out host fp32 [batch][num_q_heads][Dv] and [batch][num_q_heads]
 *   n_threads      threads working on the call, the caller's included, at most 255 (<= 0: the
 *                  CPUs the process may run on, at most 64)
 * Work items are (sequence, KV head, 1024-token chunk of whole blocks) taken by the threads
 * from a shared counter; the chunk partials are merged in chunk order, so the result does not
 * depend on n_threads.  The worker threads persist between calls (they spin for about 2 ms
 * after a call, then sleep), and calls from several threads run one after another.
 * Synchronous; all memory is the caller's.  Errors: E_INVAL, E_RANGE, E_UNSUPPORTED (q_dtype
 * != kv_dtype, more than 16 query heads per KV head).
 */
kvattn_status kvattn_host_partial(const kvattn_layout* layout, const kvattn_region* host_regions,
                                  int32_t n_regions, const void* q, int32_t q_dtype,
                                  int32_t batch, int32_t num_q_heads, float scale,
                                  const int32_t* table, int32_t max_blocks,
                                  const int32_t* tok_end, float* o_out, float* lse_out,
                                  int32_t n_threads);

/*
 * ---- CPU / GPU share policy ([InplaceKVCache] §5.2 Eq. 1, §5.3 Eq. 2) ----
 *
 * Cost model of one decode step whose sequence of already-placed length L is split with the
 * CPU taking the oldest r * L tokens and the GPU the rest (§5.1):
 *     T_CPU(r) = r * A * L + C_CPU,     T_GPU(r) = (1 - r) * B * L + C_GPU          (Eq. 1)
 * A: CPU cost per KV token it reads; B: GPU cost per KV token routed to it (on the pages, the
 * host-to-device transfer; here whatever the caller measures for its GPU side); C_CPU, C_GPU:
 * fixed per-step overheads.  Any time unit, the same for all four.  Balancing the two gives
 *     r(L) = min(1, max(0, B / (A + B) + (C_GPU - C_CPU) / ((A + B) * L)))          (Eq. 2)
 * which tends to p = B / (A + B) for long sequences.
 */
typedef struct {
  double cpu_cost;  /* A  >= 0 */
  double gpu_cost;  /* B  >= 0, A + B > 0 */
  double cpu_fixed; /* C_CPU (any sign) */
  double gpu_fixed; /* C_GPU (any sign) */
} kvattn_share_model;

/*
 * Eq. 2 for one length.  r_out (host) receives r(L) in [0, 1].
 * E_INVAL: null pointers, a non-finite field, A < 0, B < 0, A + B == 0, or L not finite and > 0.
 */
kvattn_status kvattn_share_optimum(const kvattn_share_model* model, double placed_len,
                                   double* r_out);

/*
 * Offline calibration ([InplaceKVCache] §5.3: the parameters are scanned at several data
 * volumes for the target model): ordinary least-squares line through the points
 * (tokens[i], seconds[i]), i < count, so that seconds ~ slope * tokens + intercept -- A and
 * C_CPU from CPU timings, B and C_GPU from GPU ones.  Host arrays of doubles.
 * E_INVAL: null pointers, count < 2, non-finite values, or all tokens[i] equal.
 */
kvattn_status kvattn_share_fit(const double* tokens, const double* seconds, int32_t count,
                               double* slope, double* intercept);

/*
 * Share controller of one sequence (or of a batch whose sequences grow in step): where each
 * batch of tokens leaving the GPU's staging window (the D-window of [InplaceKVCache] §4.2)
 * is stored, so that the CPU's cumulative share R(L) follows r(L) (§5.3).
 *  - kvattn_share_admit(L0, block_tokens): the prefill of L0 tokens is placed with the CPU
 *    taking the oldest round(r(L0) * L0 / block_tokens) whole blocks (at most the whole blocks
 *    of L0), so R(L0) = r(L0) up to one block; returns that token count.
 *  - kvattn_share_observe(t, n): one measured CPU component latency t of a decode step that
 *    read n CPU tokens.  The last `window` samples are kept; their sliding average gives A back
 *    as (sum t - k * C_CPU) / sum n over the k samples held.
 *  - kvattn_share_route(D): a batch of D tokens leaves the window.  If the window of samples is
 *    full, A is first replaced by the back-computed value (kept unchanged when sum n == 0 or
 *    the value is not > 0).  Then, with L the placed length and c the CPU tokens so far, the
 *    target is r(L + D) * (L + D) (Eq. 2 with the current A); the batch goes to the CPU iff
 *    c + D / 2 < target, i.e. iff that leaves c nearer the target (ties stay on the GPU).
 *    While A, B and the overheads hold still the target grows by p * D per batch, so the CPU
 *    takes a fraction p of the batches and R(L) stays within D / (2 L) of r(L); the pages'
 *    R(L) = p + (R(L0) - p) * L0 / L is that with R(L0) = r(L0).  Already placed tokens never
 *    move.
 * Not thread-safe; one controller per caller thread or an external lock.
 * Errors: E_INVAL for null pointers, an invalid model (as kvattn_share_optimum), window < 1 or
 * > 65536, L0 < 0, block_tokens < 1, batch_tokens < 1, t or n non-finite or negative;
 * E_STATE for route / observe before admit, or admit twice.
 */
typedef struct kvattn_share_ctl kvattn_share_ctl;

typedef struct {
  int64_t placed_tokens; /* L: tokens placed so far (prefill + routed batches) */
  int64_t cpu_tokens;    /* c: of which on the CPU side */
  int64_t cpu_batches;   /* routed batches sent to the CPU */
  int64_t batches;       /* routed batches */
  double cpu_cost;       /* A currently used */
  double converged;      /* p = B / (A + B) with that A */
  double target_share;   /* r(L) with that A (0 when L == 0) */
  int32_t samples;       /* samples held in the window */
} kvattn_share_state;

kvattn_status kvattn_share_ctl_create(const kvattn_share_model* model, int32_t window,
                                      kvattn_share_ctl** out);
void kvattn_share_ctl_free(kvattn_share_ctl* ctl);
kvattn_status kvattn_share_admit(kvattn_share_ctl* ctl, int64_t prefill_tokens,
                                 int64_t block_tokens, int64_t* cpu_tokens);
kvattn_status kvattn_share_observe(kvattn_share_ctl* ctl, double cpu_seconds, double cpu_tokens);
kvattn_status kvattn_share_route(kvattn_share_ctl* ctl, int64_t batch_tokens, int32_t* to_cpu);
kvattn_status kvattn_share_get_state(const kvattn_share_ctl* ctl, kvattn_share_state* out);

/*
 * ---- Write-time placement across the two engines ([InplaceKVCache] §4.1, §4.2, §5.3) ----
 *
 * A kvattn_kvstore tracks, for each of `batch` sequences, three lists of whole blocks:
 *   cpu  blocks of the host pool holding the CPU share (read by kvattn_host_partial);
 *   gpu  blocks of the device pool holding the GPU share;
 *   win  blocks of the device pool forming the staging window (the D-window), which receives
 *        every new token; its tokens start at slot 0 of its first block, so only its last
 *        filled block may be partial.
 * Every placed block holds bs tokens.  Tokens are never moved once placed (§4.2).  Decode
 * attention is the same for any order of the tokens (keys carry their position already), so
 * each engine reads its own tokens through its own view:
 *   GPU view  table = gpu ++ win (the partial block last), length = bs * |gpu| + w
 *   CPU view  table = cpu, length = bs * |cpu|
 * where w is the number of tokens in the window.  A new token goes to logical index
 * bs * |gpu| + w of the GPU view, i.e. into the window (kvattn_append_kv with the GPU view).
 *
 * Operations (host bookkeeping; only kvattn_kvstore_place_prefill and kvattn_kvstore_flush
 * enqueue device work):
 *  - reserve(n_new): n_new host [batch], each >= 0.  Claims device blocks so that window b
 *    has room for n_new[b] more tokens (ceil((w + n_new[b]) / bs) window blocks), sequences
 *    in order, all or nothing
 *    (E_POOL_EXHAUSTED leaves everything unchanged; E_INVAL if a GPU view would exceed
 *    max_blocks).  Claims come from kvattn_block_table in allocate mode, one sequence at a
 *    time.  *changed = 1 if the GPU view tables changed.
 *  - commit(n_new): records n_new[b] appended tokens for each sequence b (E_STATE without
 *    room; nothing changes then).
 *  - place_prefill: once, before any flush.  For each sequence with a controller, the
 *    controller admits the w_full = bs * floor(w / bs) tokens of the window's full blocks
 *    (kvattn_share_admit with block_tokens = bs); that many of the oldest blocks go to the
 *    CPU share and the other full blocks to the GPU share; a partial block stays in the
 *    window.  Without a controller every full block goes to the GPU share.
 *  - flush: while a window holds at least D = window_tokens tokens, its first D / bs blocks
 *    form a batch; the controller routes it (kvattn_share_route(D); no controller: GPU).  A
 *    GPU batch moves to the GPU share in place (no copy); a CPU batch is copied block by
 *    block into newly claimed host blocks and its device blocks are released.
 *  - The _plan forms do the bookkeeping only and return the copies as pairs (device id,
 *    host id) in copy order; the others then enqueue the copies on hip_stream: one kernel that
 *    writes the blocks into the host regions over the host link when every host region is
 *    pinned memory mapped for the device (hipHostGetDevicePointer succeeds), else one
 *    hipMemcpyAsync (device to host) per pair.  A released device block may be claimed again by the next reserve:
 *    its copy must be enqueued (plan callers: performed) before any later write to it, which
 *    holds when appends go to the same stream.  The host must not read a CPU block before its
 *    copy has completed (synchronise the stream).
 *  - Before anything changes, place_prefill checks that the host pool has free blocks for
 *    what the controllers will admit (known in advance), and flush that it has them for the
 *    worst case (every pending batch to the CPU); otherwise E_POOL_EXHAUSTED, changing
 *    nothing.  Likewise E_INVAL if a CPU view would then exceed max_blocks, or if `copies`
 *    (host int32 [max_copies][2]) has fewer pairs than that count; E_STATE if a controller
 *    has already been admitted.
 *  - views: host arrays gpu_table / cpu_table [batch][max_blocks] (ABSENT after the list),
 *    gpu_len / cpu_len [batch].
 *  - free: returns every block the store holds to its pool; a pool whose kvattn_pool_free
 *    came first is deleted then (the store holds both pools until it is freed).
 * The controllers (ctls[b], NULL for none; the array may be NULL; one distinct, not yet
 * admitted controller per sequence) and pools are borrowed and must outlive the store.  Not thread-safe.  Both pools must have the same layout.
 * Errors: E_INVAL (null pointers, batch < 1, max_blocks < 1, window_tokens not a positive
 * multiple of bs, an n_new entry < 0, layouts differ), E_STATE (commit beyond the reservation,
 * place_prefill twice or after a flush), E_POOL_EXHAUSTED, E_HIP (copy enqueue failed; the
 * store is then unspecified).
 */
typedef struct kvattn_kvstore kvattn_kvstore;

kvattn_status kvattn_kvstore_create(kvattn_pool* dev_pool, kvattn_pool* host_pool, int32_t batch,
                                    int32_t window_tokens, int32_t max_blocks,
                                    kvattn_share_ctl* const* ctls, kvattn_kvstore** out);
void kvattn_kvstore_free(kvattn_kvstore* store);
kvattn_status kvattn_kvstore_reserve(kvattn_kvstore* store, const int32_t* n_new,
                                     int32_t* changed);
kvattn_status kvattn_kvstore_commit(kvattn_kvstore* store, const int32_t* n_new);
kvattn_status kvattn_kvstore_place_prefill_plan(kvattn_kvstore* store, int32_t* copies,
                                                int32_t max_copies, int32_t* n_copies,
                                                int32_t* changed);
kvattn_status kvattn_kvstore_place_prefill(kvattn_kvstore* store, void* hip_stream,
                                           int32_t* changed);
kvattn_status kvattn_kvstore_flush_plan(kvattn_kvstore* store, int32_t* copies,
                                        int32_t max_copies, int32_t* n_copies, int32_t* changed);
kvattn_status kvattn_kvstore_flush(kvattn_kvstore* store, void* hip_stream, int32_t* changed);
kvattn_status kvattn_kvstore_views(const kvattn_kvstore* store, int32_t* gpu_table,
                                   int32_t* gpu_len, int32_t* cpu_table, int32_t* cpu_len);

/*
 * Address-resolution probe (for tests): runs the same device resolution code as the decode
 * kernels ([CrossPool] §3.1: logical KV address -> physical page) and writes, for every
 * sequence b and token t < ctx_lens[b] with a resident block, the region index and the byte
 * offset (within that region) of element K(h = 0, t, 0) -- or C(t, 0) for MLA -- and -1 / -1
 * for t >= ctx_lens[b] or an ABSENT or invalid entry.
 *   table_dev  device [batch][max_blocks]; ctx_lens_dev device [batch]
 *   region_out device int32 [batch][max_tokens]; offset_out device int64 [batch][max_tokens]
 * Errors: E_INVAL (null pointers, max_tokens > max_blocks * bs), E_HIP.
 */
kvattn_status kvattn_resolve_offsets(const kvattn_pool* pool, const int32_t* table_dev,
                                     int32_t batch, int32_t max_blocks,
                                     const int32_t* ctx_lens_dev, int32_t max_tokens,
                                     int32_t* region_out, int64_t* offset_out, void* hip_stream);

/* Message of the last error on the calling thread ("" if none).  Never NULL. */
const char* kvattn_last_error(void);

/* Library version string.  Never NULL. */
const char* kvattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
