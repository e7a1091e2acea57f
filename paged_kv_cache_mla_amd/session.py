"""Upload a host-side workload description to the device and set up a decode step.

A "case" is any object with the attributes of ``synth.Case`` (layout fields, flat region
arrays, block table, lengths, partition sizes, q, scale).  Region arrays and q are copied
to HBM byte for byte (bf16 bit patterns travel as int16); the block table is claimed in
the pool through the explicit-table mode of kvattn_block_table, then the decode runs
through ``DecodeStep``.  Torch is used for device memory only.
"""

import numpy as np

from ._lib import BF16, F32, OK, KvattnError
from .api import DecodeStep, Pool


def _to_device(arr, device):
    import torch
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


class DeviceCase:
    def __init__(self, case, device="cuda", seed=0, group_parts=1):
        self.case = case
        self.regions = [_to_device(r, device) for r in case.regions]
        self.pool = Pool(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                         case.dtype, case.latent,
                         [(t.data_ptr(), n) for t, n in zip(self.regions, case.region_blocks)],
                         seed=seed)
        st, table, _ = self.pool.block_table(case.ctx_lens, case.max_blocks, explicit=case.table)
        if st != OK:
            raise KvattnError(st, "block_table (explicit)")
        self.table = table
        self.step = DecodeStep(self.pool, table, case.ctx_lens, case.part_tokens,
                               case.num_q_heads, case.head_dim_v, tok_begin=case.tok_begin,
                               device=device, group_parts=group_parts)
        self.q = _to_device(case.q, device)
        self.q_dtype = F32 if case.dtype == "f32" else BF16

    def run(self, o_ext=None, lse_ext=None, stream=None):
        return self.step.run(self.q, self.q_dtype, self.case.scale, o_ext, lse_ext, stream)

    def partial(self, stream=None):
        self.step.partial(self.q, self.q_dtype, self.case.scale, stream)

    def merge(self, o_ext=None, lse_ext=None, stream=None):
        self.step.merge(o_ext, lse_ext, stream)
