"""Model of the block pool's host bookkeeping (oracle; test infrastructure only).

Written from the library's documented contract, independently of its C++ source, so
tables produced by the library can be compared entry by entry:
  - free-block pool over all regions ([VAMP] §IV-C, §V-A: reclaimed pages are inserted
    into the free-block pool and are immediately allocatable);
  - all-or-nothing admission: when the budget cannot cover a request it is refused and
    running state is untouched ([CrossPool] §3.1);
  - shared prefix blocks are reference counted (prefix caching reuses blocks across turns
    and requests: [VAMP] §II-A; counting references is this library's reading).
The initial free-list order is a Fisher-Yates (Durstenfeld) shuffle of 0..N-1 driven by
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014), both implemented below from their published definitions.
"""

import numpy as np

MASK64 = (1 << 64) - 1
ABSENT = -1


class SplitMix64:
    """SplitMix64: add the golden-ratio increment to the state, then mix it."""

    GAMMA = 0x9E3779B97F4A7C15

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + self.GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def shuffled_ids(n: int, seed: int, draw=None):
    """Durstenfeld's Fisher-Yates shuffle of [0, n): for i = n-1 .. 1 swap i with a uniform
    j in [0, i].  `draw(i)` returns that j; by default j = splitmix64 % (i + 1)."""
    ids = list(range(n))
    if draw is None:
        gen = SplitMix64(seed)
        draw = lambda i: gen.next() % (i + 1)  # noqa: E731
    for i in range(n - 1, 0, -1):
        j = draw(i)
        ids[i], ids[j] = ids[j], ids[i]
    return ids


class PoolError(Exception):
    def __init__(self, kind: str, shortfall: int = 0):
        super().__init__(kind)
        self.kind = kind            # "inval", "exhausted", "range", "state"
        self.shortfall = shortfall


class PoolModel:
    """Free list as a stack (next block handed out = top); refcount per block."""

    def __init__(self, total_blocks: int, seed: int, block_size: int):
        order = shuffled_ids(total_blocks, seed)
        self.total = total_blocks
        self.bs = block_size
        self.free = list(reversed(order))   # top of stack = order[0]
        self.ref = [0] * total_blocks

    def _pop(self) -> int:
        return self.free.pop()

    def alloc(self, ctx_lens, max_blocks, first_tok=None, share_src=None, share_nblocks=None):
        """Allocate-mode table; raises PoolError and leaves the model unchanged on failure."""
        bsz = len(ctx_lens)
        plan = []
        need = 0
        for b in range(bsz):
            L = int(ctx_lens[b])
            if L < 0:
                raise PoolError("inval")
            nb = -(-L // self.bs)
            if nb > max_blocks:
                raise PoolError("inval")
            nabs = 0 if first_tok is None else int(first_tok[b]) // self.bs
            if first_tok is not None and not (0 <= int(first_tok[b]) <= L):
                raise PoolError("inval")
            src = -1 if share_src is None else int(share_src[b])
            nsh = 0
            if src >= 0:
                nsh = int(share_nblocks[b])
                if src >= b or nabs > 0 or nsh < 0:
                    raise PoolError("inval")
                src_nb = -(-int(ctx_lens[src]) // self.bs)
                src_nabs = 0 if first_tok is None else int(first_tok[src]) // self.bs
                if nsh > nb or nsh > src_nb or src_nabs > 0:
                    raise PoolError("inval")
            fresh = nb - max(nabs, nsh)
            need += max(fresh, 0)
            plan.append((nb, nabs, src, nsh))
        if need > len(self.free):
            raise PoolError("exhausted", need - len(self.free))
        table = np.full((bsz, max_blocks), ABSENT, np.int32)
        for b, (nb, nabs, src, nsh) in enumerate(plan):
            for i in range(nb):
                if i < nabs:
                    continue
                if i < nsh:
                    pid = int(table[src, i])
                    self.ref[pid] += 1
                    table[b, i] = pid
                else:
                    pid = self._pop()
                    self.ref[pid] = 1
                    table[b, i] = pid
        return table

    def claim_explicit(self, ctx_lens, table):
        """Explicit-mode claim of a caller-chosen table."""
        table = np.asarray(table, np.int32)
        counts = {}
        for b in range(table.shape[0]):
            nb = -(-int(ctx_lens[b]) // self.bs)
            if int(ctx_lens[b]) < 0 or nb > table.shape[1]:
                raise PoolError("inval")
            for i in range(table.shape[1]):
                pid = int(table[b, i])
                if pid == ABSENT:
                    continue
                if pid < 0 or pid >= self.total:
                    raise PoolError("range")
                if i >= nb:
                    raise PoolError("inval")
                counts[pid] = counts.get(pid, 0) + 1
        for pid in counts:
            if self.ref[pid] != 0:
                raise PoolError("state")
        for pid, c in counts.items():
            self.ref[pid] = c
        self.free = [pid for pid in self.free if pid not in counts]
        return table.copy()

    def release(self, table):
        table = np.asarray(table, np.int32)
        counts = {}
        for pid in table.reshape(-1):
            pid = int(pid)
            if pid == ABSENT:
                continue
            if pid < 0 or pid >= self.total:
                raise PoolError("range")
            counts[pid] = counts.get(pid, 0) + 1
        for pid, c in counts.items():
            if c > self.ref[pid]:
                raise PoolError("state")
        for pid in table.reshape(-1):
            pid = int(pid)
            if pid == ABSENT:
                continue
            self.ref[pid] -= 1
            if self.ref[pid] == 0:
                self.free.append(pid)


def _push_new(model, first, n):
    """New ids on top of the stack, handed out first and in ascending order."""
    model.free += list(range(first + n - 1, first - 1, -1))
    model.ref += [0] * n


def add_region(model, n):
    """Append n blocks as a new region ([VAMP] §V-A: reclaimed pages join the free-block pool
    and are allocatable at once); returns their first id."""
    first = model.total
    model.total += n
    _push_new(model, first, n)
    model.region_sizes = getattr(model, "region_sizes", [first]) + [n]
    return first


def resize_last_region(model, n):
    """Grow or shrink the last region ([VAMP] §V-A: the remap runs in reverse too); shrinking
    needs the removed (highest) ids free."""
    sizes = getattr(model, "region_sizes", [model.total])
    cur = sizes[-1]
    first = model.total - cur
    if n < 0 or (n == 0 and len(sizes) == 1):
        raise PoolError("inval")
    if n >= cur:
        _push_new(model, model.total, n - cur)
        model.total = first + n
    else:
        cut = first + n
        if any(model.ref[i] for i in range(cut, model.total)):
            raise PoolError("state")
        model.free = [i for i in model.free if i < cut]
        model.ref = model.ref[:cut]
        model.total = cut
    sizes = sizes[:-1] + ([n] if n else [])
    model.region_sizes = sizes
