"""Write-time placement across the two engines (oracle; test infrastructure only).

[InplaceKVCache]:
  §4.1  the block is the unit of placement;
  §4.2  new decode entries are staged in the GPU's window (the D-window), where the GPU
        attends them at once; every D entries the batch is evicted whole to the side the
        policy picks, and placed entries never move; prefill is placed at write time;
  §5.3  batches are routed so that the CPU's cumulative share follows r(L).

Readings (the pages leave these open):
  * The GPU share stays in HBM where it was written: a batch routed to the GPU changes list,
    a batch routed to the CPU is copied into newly claimed host blocks and its device blocks
    return to the device pool.
  * Decode attention does not depend on the order of the cached tokens (each key already
    carries its position), so each engine reads its own tokens through its own sub-table:
    GPU view = GPU-share blocks then window blocks (the partial block last), CPU view =
    CPU-share blocks.
  * Prefill: the controller admits the window's whole blocks; the oldest admitted blocks go
    to the CPU, the other whole blocks to the GPU share; a partial block stays in the window.
  * Blocks are claimed sequence by sequence from the allocator model (``oracle.alloc``), so
    every physical id is predictable; steps that could exhaust a pool or overflow a view fail
    before changing anything (prefill: for what the controllers will admit; flush: for every
    pending batch going to the CPU).

Steps follow the definitions in the order given, one sequence at a time.
"""

import copy

import numpy as np

from .alloc import ABSENT, PoolError


class StoreModel:
    def __init__(self, dev_pool, host_pool, batch, window_tokens, max_blocks, controllers=None):
        self.dev, self.host = dev_pool, host_pool
        self.bs = dev_pool.bs
        self.batch, self.D, self.max_blocks = batch, window_tokens, max_blocks
        self.ctl = list(controllers) if controllers is not None else [None] * batch
        self.cpu = [[] for _ in range(batch)]
        self.gpu = [[] for _ in range(batch)]
        self.win = [[] for _ in range(batch)]
        self.w = [0] * batch
        self.prefill_done = False
        self.flushed = False

    def _claim(self, pool, n):
        if n == 0:
            return []
        return [int(x) for x in pool.alloc([n * self.bs], n)[0]]

    def _release(self, pool, ids):
        if ids:
            pool.release(np.array([ids], np.int32))

    def reserve(self, n_new):
        need = []
        for b in range(self.batch):
            want = -(-(self.w[b] + int(n_new[b])) // self.bs)
            add = max(0, want - len(self.win[b]))
            if len(self.gpu[b]) + len(self.win[b]) + add > self.max_blocks:
                raise PoolError("inval")
            need.append(add)
        if sum(need) > len(self.dev.free):
            raise PoolError("exhausted")
        for b in range(self.batch):
            self.win[b] += self._claim(self.dev, need[b])
        return sum(need) > 0

    def commit(self, n_new):
        for b in range(self.batch):
            if -(-(self.w[b] + int(n_new[b])) // self.bs) > len(self.win[b]):
                raise PoolError("state")
        for b in range(self.batch):
            self.w[b] += int(n_new[b])

    def _check_worst(self, per_seq):
        for b in range(self.batch):
            if len(self.cpu[b]) + per_seq[b] > self.max_blocks:
                raise PoolError("inval")
        if sum(per_seq) > len(self.host.free):
            raise PoolError("exhausted")

    def _move(self, b, n, to_cpu, copies):
        batch_blocks = self.win[b][:n]
        self.win[b] = self.win[b][n:]
        if to_cpu:
            host_ids = self._claim(self.host, n)
            copies += list(zip(batch_blocks, host_ids))
            self.cpu[b] += host_ids
            self._release(self.dev, batch_blocks)
        else:
            self.gpu[b] += batch_blocks

    def place_prefill(self):
        if self.prefill_done or self.flushed:
            raise PoolError("state")
        # what each controller will admit is known beforehand (a copy of it admits)
        need = []
        for b in range(self.batch):
            full = self.w[b] // self.bs
            if self.ctl[b] is None:
                need.append(0)
                continue
            if self.ctl[b].admitted:
                raise PoolError("state")
            need.append(copy.deepcopy(self.ctl[b]).admit(full * self.bs, self.bs) // self.bs)
        self._check_worst(need)
        copies, changed = [], False
        for b in range(self.batch):
            full = self.w[b] // self.bs
            cpu_tokens = 0 if self.ctl[b] is None else self.ctl[b].admit(full * self.bs, self.bs)
            ncpu = cpu_tokens // self.bs
            self._move(b, ncpu, True, copies)
            self._move(b, full - ncpu, False, copies)
            self.w[b] -= full * self.bs
            changed |= ncpu > 0
        self.prefill_done = True
        return changed, copies

    def flush(self):
        nb = self.D // self.bs
        self._check_worst([(w // self.D) * nb for w in self.w])
        copies, changed = [], False
        for b in range(self.batch):
            while self.w[b] >= self.D:
                to_cpu = False if self.ctl[b] is None else self.ctl[b].route(self.D)
                self._move(b, nb, to_cpu, copies)
                self.w[b] -= self.D
                changed |= to_cpu
        self.flushed = True
        return changed, copies

    def views(self):
        gt = np.full((self.batch, self.max_blocks), ABSENT, np.int32)
        ct = np.full((self.batch, self.max_blocks), ABSENT, np.int32)
        gl = np.zeros(self.batch, np.int32)
        cl = np.zeros(self.batch, np.int32)
        for b in range(self.batch):
            row = self.gpu[b] + self.win[b]
            gt[b, :len(row)] = row
            ct[b, :len(self.cpu[b])] = self.cpu[b]
            gl[b] = len(self.gpu[b]) * self.bs + self.w[b]
            cl[b] = len(self.cpu[b]) * self.bs
        return gt, gl, ct, cl
