"""Thin Python binding over the kvattn C ABI.

Only argument marshalling lives here: torch supplies device memory and the current HIP
stream, numpy holds host tables; every step of the decode path runs in the library's
kernels.  Functions mirror the C names without the ``kvattn_`` prefix.
"""

import ctypes

import numpy as np

from . import _lib
from ._lib import BF16, F32, KvattnError, check

__all__ = ["Pool", "DecodeStep", "choose_group_parts", "decode_plan", "decode_partial_plan", "decode_partial_plan_noalloc", "plan_supported", "decode_partial", "merge_lse", "resolve_offsets", "append_kv", "select_blocks",
           "partition_count", "block_bytes", "host_partial", "HostShare", "share_optimum", "share_fit",
           "ShareController", "KVStore", "VMMRange", "KvattnError", "BF16", "F32"]


def _i32p(arr):
    if arr is None:
        return None
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _host_i32(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _dptr(t):
    """Device address of a torch tensor, or an int address passed through (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _layout(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent):
    return _lib.Layout(block_size, num_kv_heads, head_dim_k, head_dim_v,
                       F32 if dtype in ("f32", F32) else BF16, 1 if latent else 0)


def block_bytes(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent=False):
    lib = _lib.load()
    lay = _layout(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent)
    return int(lib.kvattn_block_bytes(ctypes.byref(lay)))


def partition_count(ctx_len, tok_begin, part_tokens):
    return int(_lib.load().kvattn_partition_count(ctx_len, tok_begin, part_tokens))


class Pool:
    """Host metadata of a block pool over caller-owned device regions.

    `regions` is a list of (device address, number of blocks) pairs -- typically
    ``(tensor.data_ptr(), n)`` of torch tensors the caller keeps alive.
    """

    def __init__(self, block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent,
                 regions, seed=0):
        self._lib = _lib.load()
        self.layout = _layout(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent)
        arr = (_lib.Region * len(regions))()
        for i, (addr, nblk) in enumerate(regions):
            arr[i].base = ctypes.c_void_p(int(addr))
            arr[i].num_blocks = int(nblk)
        out = ctypes.c_void_p()
        check(self._lib.kvattn_pool_alloc(ctypes.byref(self.layout), arr, len(regions),
                                          ctypes.c_uint64(seed & (2 ** 64 - 1)),
                                          ctypes.byref(out)), "pool_alloc")
        self.handle = out
        self.block_size = block_size

    def close(self):
        if self.handle:
            self._lib.kvattn_pool_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self):
        return int(self._lib.kvattn_pool_num_free(self.handle))

    @property
    def shared_blocks(self):
        return int(self._lib.kvattn_pool_shared_blocks(self.handle))

    @property
    def num_regions(self):
        return int(self._lib.kvattn_pool_num_regions(self.handle))

    def add_region(self, addr, num_blocks):
        """Append a region at run time; returns the first id of its blocks."""
        first = ctypes.c_int64()
        check(self._lib.kvattn_pool_add_region(self.handle, ctypes.c_void_p(int(addr)),
                                               int(num_blocks), ctypes.byref(first)),
              "pool_add_region")
        return first.value

    def resize_last_region(self, num_blocks):
        check(self._lib.kvattn_pool_resize_last_region(self.handle, int(num_blocks)),
              "pool_resize_last_region")

    def refcount(self, block_id):
        return int(self._lib.kvattn_pool_refcount(self.handle, int(block_id)))

    def block_table(self, ctx_lens, max_blocks, first_tok=None, share_src=None,
                    share_nblocks=None, explicit=None):
        """Returns (status, table [B, max_blocks] int32, shortfall); raises only on misuse
        of this wrapper -- the status codes of the C call are returned as they are."""
        ctx = _host_i32(ctx_lens)
        bsz = int(ctx.shape[0])
        ft, ss, sn = _host_i32(first_tok), _host_i32(share_src), _host_i32(share_nblocks)
        ex = None if explicit is None else np.ascontiguousarray(np.asarray(explicit, np.int32))
        out = np.full((bsz, max_blocks), -7, np.int32)
        short = ctypes.c_int64(-1)
        st = self._lib.kvattn_block_table(self.handle, bsz, _i32p(ctx), _i32p(ft), _i32p(ss),
                                          _i32p(sn), _i32p(ex), int(max_blocks), _i32p(out),
                                          ctypes.byref(short))
        return int(st), out, int(short.value)

    def release(self, table):
        t = np.ascontiguousarray(np.asarray(table, np.int32))
        return int(self._lib.kvattn_block_release(self.handle, _i32p(t), t.shape[0], t.shape[1]))


def choose_group_parts(pool, num_q_heads, ctx_lens, tok_begin, part_tokens, num_cus=0):
    """The group_parts decode_partial uses when passed 0 (num_cus 0: the current device's)."""
    lib = _lib.load()
    ctx, beg, part = _host_i32(ctx_lens), _host_i32(tok_begin), _host_i32(part_tokens)
    g = lib.kvattn_choose_group_parts(pool.handle, int(ctx.shape[0]), int(num_q_heads),
                                      _i32p(ctx), _i32p(beg), _i32p(part), int(num_cus))
    check(g if g < 0 else 0, "choose_group_parts")
    return int(g)


def plan_supported(pool, num_q_heads):
    """Whether kvattn_decode_plan serves this pool and head count (bf16 per-head cache, block
    size >= 16, head dim 64 / 128 / 256, at most 16 query heads per KV head)."""
    L = pool.layout
    return (not L.latent and L.kv_dtype == BF16 and L.block_size >= 16 and
            L.head_dim_k == L.head_dim_v and L.head_dim_k in (64, 128, 256) and
            num_q_heads % L.num_kv_heads == 0 and num_q_heads // L.num_kv_heads <= 16)


def decode_plan(pool, num_q_heads, table, ctx_lens, tok_begin, part_tokens, span_parts=0):
    """kvattn_decode_plan on host arrays: (plan int32 array, n_groups, max_parts)."""
    lib = _lib.load()
    t = np.ascontiguousarray(np.asarray(table, np.int32))
    ctx, beg, part = _host_i32(ctx_lens), _host_i32(tok_begin), _host_i32(part_tokens)
    n = ctypes.c_int64()
    ng, mp = ctypes.c_int32(), ctypes.c_int32()
    args = (pool.handle, int(ctx.shape[0]), int(num_q_heads), _i32p(t), int(t.shape[1]), _i32p(ctx),
            _i32p(beg), _i32p(part), int(span_parts))
    # one call into a buffer of the largest length a plan can have: with P block positions,
    # at most P member entries (each covers a position of its sequence), as many items, and
    # four wave slots of six ints per item; the planner writes every entry it reports
    bs = int(pool.block_size)
    b0 = np.zeros_like(ctx) if tok_begin is None else beg
    live = ctx > b0
    positions = int(np.sum((ctx[live] - 1) // bs - b0[live] // bs + 1))
    plan = np.empty(8 + int(ctx.shape[0]) + 26 * positions, np.int32)
    st = lib.kvattn_decode_plan(*args, _i32p(plan), plan.size, ctypes.byref(n), ctypes.byref(ng),
                                ctypes.byref(mp))
    if st == _lib.E_INVAL and n.value > plan.size:  # the bound cannot be short; kept as a guard
        plan = np.empty(n.value, np.int32)
        st = lib.kvattn_decode_plan(*args, _i32p(plan), plan.size, ctypes.byref(n),
                                    ctypes.byref(ng), ctypes.byref(mp))
    check(st, "decode_plan")
    return plan[:n.value].copy(), int(ng.value), int(mp.value)


def decode_partial_plan(pool, q, q_dtype, num_q_heads, scale, table_dev, max_blocks, plan_dev,
                        n_groups, max_parts, o_part, lse_part, nparts, err=None, stream=None,
                        work=None):
    """work: a zeroed device uint32 [2] (torch int32 tensor) for the claiming launch, or None."""
    lib = _lib.load()
    bsz = int(o_part.shape[0])
    check(lib.kvattn_decode_partial_plan(pool.handle, _dptr(q), int(q_dtype), bsz,
                                         int(num_q_heads), ctypes.c_float(scale), _dptr(table_dev),
                                         int(max_blocks), _dptr(plan_dev), int(n_groups),
                                         _dptr(work), int(max_parts), _dptr(o_part),
                                         _dptr(lse_part), _dptr(nparts), _dptr(err),
                                         _stream(stream)),
          "decode_partial_plan")


def decode_partial_plan_noalloc(pool, q, q_dtype, num_q_heads, scale, table_dev, max_blocks,
                                plan_dev, n_groups, max_parts, o_part, lse_part, nparts, err=None,
                                stream=None):
    """kvattn_decode_partial_plan with the library's own per-GPU work counters (no work_dev)."""
    lib = _lib.load()
    bsz = int(o_part.shape[0])
    check(lib.kvattn_decode_partial_plan_noalloc(pool.handle, _dptr(q), int(q_dtype), bsz,
                                                 int(num_q_heads), ctypes.c_float(scale),
                                                 _dptr(table_dev), int(max_blocks), _dptr(plan_dev),
                                                 int(n_groups), int(max_parts), _dptr(o_part),
                                                 _dptr(lse_part), _dptr(nparts), _dptr(err),
                                                 _stream(stream)),
          "decode_partial_plan_noalloc")


def decode_partial(pool, q, q_dtype, num_q_heads, scale, table_dev, max_blocks, ctx_lens,
                   tok_begin, part_tokens, seq_dev, max_parts, o_part, lse_part, nparts,
                   err=None, stream=None, group_parts=1):
    lib = _lib.load()
    ctx, beg, part = _host_i32(ctx_lens), _host_i32(tok_begin), _host_i32(part_tokens)
    st = lib.kvattn_decode_partial(pool.handle, _dptr(q), int(q_dtype), int(ctx.shape[0]),
                                   int(num_q_heads), ctypes.c_float(scale), _dptr(table_dev),
                                   int(max_blocks), _i32p(ctx), _i32p(beg), _i32p(part),
                                   _dptr(seq_dev), int(max_parts), int(group_parts),
                                   _dptr(o_part), _dptr(lse_part), _dptr(nparts), _dptr(err),
                                   _stream(stream))
    check(st, "decode_partial")


def gather_probe(pool, num_q_heads, table_dev, max_blocks, ctx_lens, tok_begin, part_tokens,
                 seq_dev, xsum, err=None, stream=None, group_parts=1):
    """kvattn_gather_probe: the decode kernel's loads without arithmetic; XORs a checksum of
    the read K/V elements into `xsum` (int32 [batch][num_kv_heads], zeroed by the caller)."""
    lib = _lib.load()
    ctx, beg, part = _host_i32(ctx_lens), _host_i32(tok_begin), _host_i32(part_tokens)
    st = lib.kvattn_gather_probe(pool.handle, int(ctx.shape[0]), int(num_q_heads),
                                 _dptr(table_dev), int(max_blocks), _i32p(ctx), _i32p(beg),
                                 _i32p(part), _dptr(seq_dev), int(group_parts), _dptr(xsum),
                                 _dptr(err), _stream(stream))
    check(st, "gather_probe")


def merge_lse(o_part, lse_part, nparts, batch, num_q_heads, max_parts, dv, o_out,
              o_ext=None, lse_ext=None, lse_out=None, stream=None):
    lib = _lib.load()
    st = lib.kvattn_merge_lse(_dptr(o_part), _dptr(lse_part), _dptr(nparts), int(batch),
                              int(num_q_heads), int(max_parts), int(dv), _dptr(o_ext),
                              _dptr(lse_ext), _dptr(o_out), _dptr(lse_out), _stream(stream))
    check(st, "merge_lse")


def select_blocks(table_dev, max_blocks, ctx_lens_dev, block_size, sel_dev, sub_table_dev,
                  sub_len_dev, err=None, stream=None):
    """Sub-table of the selected logical blocks of each sequence (kvattn_select_blocks):
    sel_dev [B][k] device int32 (negative = padding), sub_table_dev [B][max_sub], sub_len_dev
    [B] (may be row 0 of a decode step's seq_dev)."""
    lib = _lib.load()
    batch, k = int(sel_dev.shape[0]), int(sel_dev.shape[1])
    st = lib.kvattn_select_blocks(_dptr(table_dev), int(max_blocks), _dptr(ctx_lens_dev),
                                  int(block_size), _dptr(sel_dev), batch, k, _dptr(sub_table_dev),
                                  int(sub_table_dev.shape[1]), _dptr(sub_len_dev), _dptr(err),
                                  _stream(stream))
    check(st, "select_blocks")


def append_kv(pool, k_new, v_new, kv_dtype, table_dev, max_blocks, pos_dev, err=None,
              stream=None):
    """Write new tokens' K/V (device tensors [B][n_new][Hkv][D], v_new None for a latent
    cache) at logical positions pos_dev[b] + j through table_dev (kvattn_append_kv)."""
    lib = _lib.load()
    batch, n_new = int(k_new.shape[0]), int(k_new.shape[1])
    st = lib.kvattn_append_kv(pool.handle, _dptr(k_new), _dptr(v_new), int(kv_dtype), batch, n_new,
                              _dptr(table_dev), int(max_blocks), _dptr(pos_dev), _dptr(err),
                              _stream(stream))
    check(st, "append_kv")


def resolve_offsets(pool, table_dev, max_blocks, ctx_lens_dev, max_tokens, region_out,
                    offset_out, stream=None):
    lib = _lib.load()
    st = lib.kvattn_resolve_offsets(pool.handle, _dptr(table_dev), int(table_dev.shape[0]),
                                    int(max_blocks), _dptr(ctx_lens_dev), int(max_tokens),
                                    _dptr(region_out), _dptr(offset_out), _stream(stream))
    check(st, "resolve_offsets")


def host_partial(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent, regions, q,
                 num_q_heads, scale, table, tok_end, n_threads=0):
    """CPU share of a decode step over host-resident blocks (numpy arrays): returns
    (o [B, Hq, Dv] float32, lse [B, Hq] float32) over tokens [0, tok_end[b]) of each sequence.

    `regions` are numpy arrays holding whole blocks (uint16 bf16 bit patterns or float32), in
    the device pool's block layout; block ids run over them in order."""
    lib = _lib.load()
    lay = _layout(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent)
    nbytes = block_bytes(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent)
    arr = (_lib.Region * len(regions))()
    keep = []
    for i, r in enumerate(regions):
        r = np.ascontiguousarray(r)
        keep.append(r)
        arr[i].base = ctypes.c_void_p(r.ctypes.data)
        arr[i].num_blocks = int(r.nbytes // nbytes)
    qh = np.ascontiguousarray(q)
    tab = np.ascontiguousarray(np.asarray(table, np.int32))
    te = _host_i32(tok_end)
    bsz = int(te.shape[0])
    dv = head_dim_v
    o = np.empty((bsz, num_q_heads, dv), np.float32)
    lse = np.empty((bsz, num_q_heads), np.float32)
    st = lib.kvattn_host_partial(ctypes.byref(lay), arr, len(regions),
                                 ctypes.c_void_p(qh.ctypes.data), F32 if dtype in ("f32", F32) else BF16,
                                 bsz, int(num_q_heads), ctypes.c_float(scale), _i32p(tab),
                                 int(tab.shape[1]), _i32p(te), ctypes.c_void_p(o.ctypes.data),
                                 ctypes.c_void_p(lse.ctypes.data), int(n_threads))
    check(st, "host_partial")
    return o, lse


class HostShare:
    """kvattn_host_partial with its arguments marshalled once, for repeated decode steps over
    the same host blocks: `compute(q, o_out, lse_out)` fills caller-owned float32 arrays (for
    instance views of pinned host tensors) with the partial over tokens [0, tok_end[b])."""

    def __init__(self, block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent, regions,
                 num_q_heads, scale, table, tok_end, n_threads=0):
        self._lib = _lib.load()
        self._lay = _layout(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent)
        nbytes = block_bytes(block_size, num_kv_heads, head_dim_k, head_dim_v, dtype, latent)
        self._regions = [np.ascontiguousarray(r) for r in regions]
        self._arr = (_lib.Region * len(self._regions))()
        for i, r in enumerate(self._regions):
            self._arr[i].base = ctypes.c_void_p(r.ctypes.data)
            self._arr[i].num_blocks = int(r.nbytes // nbytes)
        self._table = np.ascontiguousarray(np.asarray(table, np.int32))
        self.tok_end = _host_i32(tok_end)
        self.batch = int(self.tok_end.shape[0])
        self.hq = int(num_q_heads)
        self.dv = int(head_dim_v)
        self._qdt = F32 if dtype in ("f32", F32) else BF16
        self._scale = ctypes.c_float(scale)
        self._n_threads = int(n_threads)

    def compute(self, q, o_out, lse_out):
        for a, shape in ((o_out, (self.batch, self.hq, self.dv)), (lse_out, (self.batch, self.hq))):
            if a.dtype != np.float32 or a.shape != shape or not a.flags.c_contiguous:
                raise ValueError(f"output must be a C-contiguous float32 array of shape {shape}")
        st = self._lib.kvattn_host_partial(
            ctypes.byref(self._lay), self._arr, len(self._regions), ctypes.c_void_p(q.ctypes.data),
            self._qdt, self.batch, self.hq, self._scale, _i32p(self._table),
            int(self._table.shape[1]), _i32p(self.tok_end), ctypes.c_void_p(o_out.ctypes.data),
            ctypes.c_void_p(lse_out.ctypes.data), self._n_threads)
        check(st, "host_partial")


def _share_model(cpu_cost, gpu_cost, cpu_fixed=0.0, gpu_fixed=0.0):
    return _lib.ShareModel(float(cpu_cost), float(gpu_cost), float(cpu_fixed), float(gpu_fixed))


def share_optimum(cpu_cost, gpu_cost, cpu_fixed, gpu_fixed, placed_len):
    """r(L) of the balance of the two engines' step latencies (kvattn_share_optimum)."""
    m = _share_model(cpu_cost, gpu_cost, cpu_fixed, gpu_fixed)
    r = ctypes.c_double()
    check(_lib.load().kvattn_share_optimum(ctypes.byref(m), float(placed_len), ctypes.byref(r)),
          "share_optimum")
    return r.value


def share_fit(tokens, seconds):
    """Least-squares (slope, intercept) of seconds ~ slope * tokens + intercept."""
    x = np.ascontiguousarray(tokens, np.float64)
    y = np.ascontiguousarray(seconds, np.float64)
    if x.shape != y.shape or x.ndim != 1:
        raise ValueError("tokens and seconds must be 1-D arrays of one length")
    a, b = ctypes.c_double(), ctypes.c_double()
    check(_lib.load().kvattn_share_fit(ctypes.c_void_p(x.ctypes.data), ctypes.c_void_p(y.ctypes.data),
                                       int(x.shape[0]), ctypes.byref(a), ctypes.byref(b)), "share_fit")
    return a.value, b.value


class ShareController:
    """Routing of tokens leaving the GPU staging window (kvattn_share_ctl_*)."""

    def __init__(self, cpu_cost, gpu_cost, cpu_fixed=0.0, gpu_fixed=0.0, window=256):
        self._lib = _lib.load()
        m = _share_model(cpu_cost, gpu_cost, cpu_fixed, gpu_fixed)
        h = ctypes.c_void_p()
        check(self._lib.kvattn_share_ctl_create(ctypes.byref(m), int(window), ctypes.byref(h)),
              "share_ctl_create")
        self._h = h

    def close(self):
        h = getattr(self, "_h", None)  # absent if the constructor raised
        if h:
            self._lib.kvattn_share_ctl_free(h)
            self._h = None

    def __del__(self):
        self.close()

    def admit(self, prefill_tokens, block_tokens):
        c = ctypes.c_int64()
        check(self._lib.kvattn_share_admit(self._h, int(prefill_tokens), int(block_tokens),
                                           ctypes.byref(c)), "share_admit")
        return c.value

    def observe(self, cpu_seconds, cpu_tokens):
        check(self._lib.kvattn_share_observe(self._h, float(cpu_seconds), float(cpu_tokens)),
              "share_observe")

    def route(self, batch_tokens):
        to_cpu = ctypes.c_int32()
        check(self._lib.kvattn_share_route(self._h, int(batch_tokens), ctypes.byref(to_cpu)),
              "share_route")
        return bool(to_cpu.value)

    def state(self):
        s = _lib.ShareState()
        check(self._lib.kvattn_share_get_state(self._h, ctypes.byref(s)), "share_get_state")
        return {f: getattr(s, f) for f, _ in _lib.ShareState._fields_}


class VMMRange:
    """A reserved device address range with movable physical pages (kvattn_vmm_*)."""

    def __init__(self, va_bytes, chunk_bytes=0, device=0):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        check(self._lib.kvattn_vmm_create(int(device), int(va_bytes), int(chunk_bytes),
                                          ctypes.byref(h)), "vmm_create")
        self._h = h

    def close(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.kvattn_vmm_free(h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def granularity(self):
        return int(self._lib.kvattn_vmm_granularity(self._h))

    @property
    def base(self):
        return int(self._lib.kvattn_vmm_base(self._h))

    @property
    def mapped_bytes(self):
        return int(self._lib.kvattn_vmm_mapped_bytes(self._h))

    def map_new(self, offset, nbytes):
        check(self._lib.kvattn_vmm_map_new(self._h, int(offset), int(nbytes)), "vmm_map_new")

    def move_to(self, offset, dst, dst_offset, nbytes, sync_device=True):
        """Move the pages behind [offset, offset + nbytes) of this range to `dst`."""
        check(self._lib.kvattn_vmm_move(self._h, int(offset), dst._h, int(dst_offset), int(nbytes),
                                        1 if sync_device else 0), "vmm_move")


class KVStore:
    """Write-time placement of each sequence's KV across a device pool (GPU share and the
    staging window) and a host pool (CPU share), routed by one share controller per sequence
    (kvattn_kvstore_*).  `controllers` is a list of ShareController or None per sequence."""

    def __init__(self, dev_pool, host_pool, batch, window_tokens, max_blocks, controllers=None):
        self._lib = _lib.load()
        self.batch, self.max_blocks = int(batch), int(max_blocks)
        self._ctls = list(controllers) if controllers is not None else [None] * self.batch
        if len(self._ctls) != self.batch:
            raise ValueError("one controller (or None) per sequence")
        arr = (ctypes.c_void_p * self.batch)(*[None if c is None else c._h.value for c in self._ctls])
        h = ctypes.c_void_p()
        check(self._lib.kvattn_kvstore_create(dev_pool.handle, host_pool.handle, self.batch,
                                              int(window_tokens), self.max_blocks, arr,
                                              ctypes.byref(h)), "kvstore_create")
        self._pools = (dev_pool, host_pool)  # keep the pools alive as long as the store
        self._h = h

    def close(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.kvattn_kvstore_free(h)
            self._h = None

    def __del__(self):
        self.close()

    def _counts(self, n_new):
        n = np.full(self.batch, n_new, np.int32) if np.isscalar(n_new) else _host_i32(n_new)
        if n.shape != (self.batch,):
            raise ValueError("n_new: a scalar or one count per sequence")
        return n

    def reserve(self, n_new):
        n = self._counts(n_new)
        changed = ctypes.c_int32()
        check(self._lib.kvattn_kvstore_reserve(self._h, _i32p(n), ctypes.byref(changed)),
              "kvstore_reserve")
        return bool(changed.value)

    def commit(self, n_new):
        n = self._counts(n_new)
        check(self._lib.kvattn_kvstore_commit(self._h, _i32p(n)), "kvstore_commit")

    def _plan(self, fn, what):
        cap = self.batch * self.max_blocks
        copies = np.empty((cap, 2), np.int32)
        n, changed = ctypes.c_int32(), ctypes.c_int32()
        check(fn(self._h, _i32p(copies), cap, ctypes.byref(n), ctypes.byref(changed)), what)
        return bool(changed.value), copies[:n.value].copy()

    def place_prefill_plan(self):
        """Bookkeeping only: returns (changed, copies [n, 2] of (device id, host id))."""
        return self._plan(self._lib.kvattn_kvstore_place_prefill_plan, "kvstore_place_prefill")

    def flush_plan(self):
        return self._plan(self._lib.kvattn_kvstore_flush_plan, "kvstore_flush")

    def place_prefill(self, stream=None):
        changed = ctypes.c_int32()
        check(self._lib.kvattn_kvstore_place_prefill(self._h, _stream(stream), ctypes.byref(changed)),
              "kvstore_place_prefill")
        return bool(changed.value)

    def flush(self, stream=None):
        changed = ctypes.c_int32()
        check(self._lib.kvattn_kvstore_flush(self._h, _stream(stream), ctypes.byref(changed)),
              "kvstore_flush")
        return bool(changed.value)

    def views(self):
        """(gpu_table [B, max_blocks], gpu_len [B], cpu_table [B, max_blocks], cpu_len [B])."""
        shape = (self.batch, self.max_blocks)
        gt, ct = np.empty(shape, np.int32), np.empty(shape, np.int32)
        gl, cl = np.empty(self.batch, np.int32), np.empty(self.batch, np.int32)
        check(self._lib.kvattn_kvstore_views(self._h, _i32p(gt), _i32p(gl), _i32p(ct), _i32p(cl)),
              "kvstore_views")
        return gt, gl, ct, cl


class DecodeStep:
    """Device-resident metadata and buffers for repeated decode steps over one batch.

    Holds the block table, the per-sequence [ctx_len, tok_begin, part_tokens] rows and the
    partial / output buffers on the device; `run` enqueues decode_partial then merge_lse on
    the current stream.  `group_parts` consecutive partitions are merged on chip into each
    written partial (1: one partial per partition; 0, the default: the library's choice,
    `self.group_parts` after construction, and decode_partial is called with 0).

    `plan`: run the step from a work plan (kvattn_decode_plan / kvattn_decode_partial_plan), so
    that sequences holding the same blocks share one pass over them.  None (the default) takes
    the plan when group_parts is the library's choice, the pool holds shared blocks and the
    layout has a plan kernel.  `span_parts` is the plan's partitions per wave item (0: auto);
    `claim` runs the plan with work counters (workgroups take the next unit when done).
    """

    def __init__(self, pool, table, ctx_lens, part_tokens, num_q_heads, head_dim_v,
                 tok_begin=None, device="cuda", group_parts=0, plan=None, span_parts=0,
                 claim=False):
        import torch
        self.pool = pool
        self.ctx = _host_i32(ctx_lens)
        self.part = _host_i32(part_tokens)
        self.beg = _host_i32(tok_begin)
        self.batch = int(self.ctx.shape[0])
        self.hq = int(num_q_heads)
        self.dv = int(head_dim_v)
        table = np.ascontiguousarray(np.asarray(table, np.int32))
        self.max_blocks = int(table.shape[1])
        begs = self.beg if self.beg is not None else np.zeros_like(self.ctx)
        counts = [partition_count(int(c), int(b), int(p)) for c, b, p in zip(self.ctx, begs, self.part)]
        if min(counts) < 0:
            raise ValueError("invalid partition arguments")
        self.auto = int(group_parts) == 0
        self.group_parts = (choose_group_parts(pool, num_q_heads, self.ctx, self.beg, self.part)
                            if self.auto else int(group_parts))
        self.max_parts = max(1, max(-(-c // self.group_parts) for c in counts))
        if plan is None:
            plan = self.auto and pool.shared_blocks > 0 and plan_supported(pool, num_q_heads)
        self.plan = None
        if plan:
            self.plan, self.n_groups, self.max_parts = decode_plan(
                pool, num_q_heads, table, self.ctx, self.beg, self.part, span_parts)
            self.plan_dev = torch.from_numpy(self.plan).to(device)
            # the work counters: zero once; every completed launch leaves them zero
            self.work = torch.zeros(2, dtype=torch.int32, device=device) if claim else None
        self.table_dev = torch.from_numpy(table).to(device)
        self.seq_dev = torch.from_numpy(np.stack([self.ctx, begs, self.part]).astype(np.int32)).to(device)
        f32 = torch.float32
        self.o_part = torch.empty((self.batch, self.hq, self.max_parts, self.dv), dtype=f32, device=device)
        self.lse_part = torch.empty((self.batch, self.hq, self.max_parts), dtype=f32, device=device)
        self.nparts = torch.empty(self.batch, dtype=torch.int32, device=device)
        self.o_out = torch.empty((self.batch, self.hq, self.dv), dtype=f32, device=device)
        self.lse_out = torch.empty((self.batch, self.hq), dtype=f32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self._fixed = None

    def _marshal(self):
        """The arguments of the two calls that do not change between steps, converted once
        (the per-call conversions are most of a small step's host time).  The tensors and host
        rows they point to stay referenced here, so the addresses stay valid while this object
        lives."""
        self._lib = _lib.load()
        part = (_dptr(self.table_dev), self.max_blocks, _i32p(self.ctx), _i32p(self.beg),
                _i32p(self.part), _dptr(self.seq_dev), self.max_parts,
                0 if self.auto else self.group_parts,
                _dptr(self.o_part), _dptr(self.lse_part), _dptr(self.nparts), _dptr(self.err))
        merge = (_dptr(self.o_part), _dptr(self.lse_part), _dptr(self.nparts), self.batch,
                 self.hq, self.max_parts, self.dv)
        out = (_dptr(self.o_out), _dptr(self.lse_out))
        if self.plan is not None:
            part = (_dptr(self.table_dev), self.max_blocks, _dptr(self.plan_dev), self.n_groups,
                    _dptr(self.work), self.max_parts, _dptr(self.o_part), _dptr(self.lse_part),
                    _dptr(self.nparts), _dptr(self.err))
        keep = (self.table_dev, self.seq_dev, self.o_part, self.lse_part, self.nparts, self.err,
                self.o_out, self.lse_out, self.ctx, self.beg, self.part,
                getattr(self, "plan_dev", None), getattr(self, "work", None))
        self._fixed = (part, merge, out, keep)

    def partial(self, q, q_dtype, scale, stream=None):
        if self._fixed is None:
            self._marshal()
        fn = (self._lib.kvattn_decode_partial if self.plan is None
              else self._lib.kvattn_decode_partial_plan)
        st = fn(self.pool.handle, _dptr(q), int(q_dtype), self.batch, self.hq,
                ctypes.c_float(scale), *self._fixed[0], _stream(stream))
        check(st, "decode_partial" if self.plan is None else "decode_partial_plan")

    def probe(self, xsum, stream=None):
        """The gather probe over this step's ranges, in its launch configuration."""
        gather_probe(self.pool, self.hq, self.table_dev, self.max_blocks, self.ctx, self.beg,
                     self.part, self.seq_dev, xsum, self.err, stream, self.group_parts)

    def merge(self, o_ext=None, lse_ext=None, stream=None):
        if self._fixed is None:
            self._marshal()
        st = self._lib.kvattn_merge_lse(*self._fixed[1], _dptr(o_ext), _dptr(lse_ext),
                                        *self._fixed[2], _stream(stream))
        check(st, "merge_lse")

    def run(self, q, q_dtype, scale, o_ext=None, lse_ext=None, stream=None):
        self.partial(q, q_dtype, scale, stream)
        self.merge(o_ext, lse_ext, stream)
        return self.o_out, self.lse_out
