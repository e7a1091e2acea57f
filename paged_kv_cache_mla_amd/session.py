"""Upload a host-side workload description to the device and set up a decode step; run a
decode step whose oldest tokens are attended on the host while the device takes the rest.

A "case" is any object with the attributes of ``synth.Case`` (layout fields, flat region
arrays, block table, lengths, partition sizes, q, scale).  Region arrays and q are copied
to HBM byte for byte (bf16 bit patterns travel as int16); the block table is claimed in
the pool through the explicit-table mode of kvattn_block_table, then the decode runs
through ``DecodeStep``.  Torch is used for device memory only.
"""

import numpy as np

from ._lib import BF16, F32, OK, KvattnError
from .api import DecodeStep, HostShare, Pool


def _to_device(arr, device):
    import torch
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


class DeviceCase:
    def __init__(self, case, device="cuda", seed=0, group_parts=0, plan=None, span_parts=0,
                 claim=False):
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
                               device=device, group_parts=group_parts, plan=plan,
                               span_parts=span_parts, claim=claim)
        self.q = _to_device(case.q, device)
        self.q_dtype = F32 if case.dtype == "f32" else BF16

    def run(self, o_ext=None, lse_ext=None, stream=None):
        return self.step.run(self.q, self.q_dtype, self.case.scale, o_ext, lse_ext, stream)

    def partial(self, stream=None):
        self.step.partial(self.q, self.q_dtype, self.case.scale, stream)

    def merge(self, o_ext=None, lse_ext=None, stream=None):
        self.step.merge(o_ext, lse_ext, stream)


def _hip_runtime():
    """The HIP runtime library torch has loaded (for host-memory calls torch does not expose)."""
    import ctypes
    import os
    with open("/proc/self/maps") as fh:
        for line in fh:
            f = line.split()[-1]
            if os.path.basename(f).startswith("libamdhip64"):
                hip = ctypes.CDLL(f)
                vp = ctypes.c_void_p
                hip.hipHostMalloc.argtypes = [ctypes.POINTER(vp), ctypes.c_size_t, ctypes.c_uint]
                hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(vp), vp, ctypes.c_uint]
                hip.hipHostFree.argtypes = [vp]
                return hip
    raise RuntimeError("the HIP runtime is not loaded (initialise torch.cuda first)")


class MappedHostArray:
    """float32 host array in pinned, device-mapped, coherent memory (hipHostMalloc with the
    Mapped and Coherent flags): the host writes it through `array`, kernels read it at `dev`
    over the host link, with no copy and no stale cached lines between uses."""

    MAPPED, COHERENT = 0x2, 0x40000000

    def __init__(self, shape):
        import ctypes
        self._hip = _hip_runtime()
        nbytes = int(np.prod(shape)) * 4
        host = ctypes.c_void_p()
        if self._hip.hipHostMalloc(ctypes.byref(host), nbytes, self.MAPPED | self.COHERENT) != 0:
            raise RuntimeError("hipHostMalloc failed")
        self._host = host
        dev = ctypes.c_void_p()
        if self._hip.hipHostGetDevicePointer(ctypes.byref(dev), host, 0) != 0:
            self.free()
            raise RuntimeError("hipHostGetDevicePointer failed")
        self.dev = int(dev.value)
        self.array = np.ctypeslib.as_array((ctypes.c_float * int(np.prod(shape))).from_address(
            host.value)).reshape(shape)

    def free(self):
        if getattr(self, "_host", None) is not None and self._host.value:
            self.array = None
            self._hip.hipHostFree(self._host)
            self._host = None

    def __del__(self):
        self.free()


class SplitStep:
    """One decode step split along the sequence ([InplaceKVCache] §5.1): the device computes
    [tok_begin, L) of every sequence with kvattn_decode_partial while the host computes
    [0, tok_begin) with kvattn_host_partial; kvattn_merge_lse joins the two on the device
    (§4.2: only the small (o, lse) crosses the link).

    Per step: the device partial is enqueued on the current stream; on a side stream, after
    the work already queued on the current stream (where q would come from), q is copied to
    pinned host memory; the host waits for that copy only and computes its share into one of
    two mapped host buffers (each reused only after the merge that last read it has run); the
    merge, enqueued on the current stream behind the device partial, reads that buffer over
    the host link directly.

    With q_first=True the device partial waits for the copy of q to the host: the host can then
    start at once instead of behind a device busy with the partial, at the price of the copy's
    latency on the device side.

    With timing=True each step also records the two component latencies of the step-time
    model ([InplaceKVCache] §5.2 Eq. 1), both from the moment the device partial is enqueued:
    `t_gpu` until the device partial ends (device events), `t_cpu` until the merge of the host
    partial has been enqueued (host clock: q transfer, host compute, launch).  The two clocks
    start within a launch latency of each other when the device is idle at the step's start,
    as in synchronised calibration steps.  Read them after synchronising.
    """

    def __init__(self, step, q_dev, q_dtype, scale, host_share, timing=False, q_first=False):
        import torch
        if host_share.batch != step.batch or host_share.hq != step.hq or host_share.dv != step.dv:
            raise ValueError("host share and device step disagree on batch / heads / Dv")
        self.step, self.q_dev, self.q_dtype, self.scale = step, q_dev, q_dtype, scale
        self.host = host_share
        dev = q_dev.device
        self.q_pin = torch.empty(q_dev.shape, dtype=q_dev.dtype, pin_memory=True)
        self.q_np = self.q_pin.numpy()
        self.o_buf = [MappedHostArray((step.batch, step.hq, step.dv)) for _ in range(2)]
        self.l_buf = [MappedHostArray((step.batch, step.hq)) for _ in range(2)]
        self.merged = [torch.cuda.Event(), torch.cuda.Event()]
        self.side = torch.cuda.Stream(device=dev)
        self.q_ready = torch.cuda.Event()
        self.timing = timing
        self.q_first = q_first
        if timing:
            self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        self.k = 0
        self.host_ms = 0.0  # host compute time of the last step
        self.t_cpu_ms = 0.0

    def run(self):
        import time
        import torch
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            self.q_pin.copy_(self.q_dev, non_blocking=True)
            self.q_ready.record(self.side)
        if self.q_first:
            main.wait_event(self.q_ready)
        if self.timing:
            t_start = time.perf_counter()
            self.ev[0].record(main)
        self.step.partial(self.q_dev, self.q_dtype, self.scale)
        if self.timing:
            self.ev[1].record(main)
        k = self.k
        self.k ^= 1
        self.merged[k].synchronize()   # the merge that last read buffer k has run
        while not self.q_ready.query():  # poll: a sleeping wait adds an interrupt's wake-up
            pass
        t0 = time.perf_counter()
        self.host.compute(self.q_np, self.o_buf[k].array, self.l_buf[k].array)
        self.host_ms = (time.perf_counter() - t0) * 1e3
        self.step.merge(self.o_buf[k].dev, self.l_buf[k].dev)
        if self.timing:
            self.t_cpu_ms = (time.perf_counter() - t_start) * 1e3
        self.merged[k].record(main)
        return self.step.o_out, self.step.lse_out

    def component_ms(self):
        """(t_gpu_ms, t_cpu_ms) of the last step (timing=True; call after synchronising)."""
        return self.ev[0].elapsed_time(self.ev[1]), self.t_cpu_ms
