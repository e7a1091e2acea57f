"""GPU test: one decode step (kvattn_decode_partial + kvattn_merge_lse) captured in a HIP graph
and replayed.

Neither entry point allocates device memory, records a memset or synchronises, so a step can be
captured once and replayed at every decode step.  Kernel arguments are frozen at capture, while
the kernels read q, the block table and the per-sequence rows from device memory: updates made
to those buffers in place between replays are seen by the replays.  Each replay runs after
eager work of the program's own and a synchronisation, and must equal the eager step bit for
bit (the decode is deterministic).
"""

import sys

import numpy as np
import pytest

from tests import oracle_cases as oc
from synth import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU-only hosts)")
    from paged_kv_cache_mla_amd import _lib
    _lib.load()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name,group_parts", [("gqa_32k", 4), ("gqa_32k", 16), ("mla_16k", 2),
                                              ("split_128k", 4), ("tiny_fp32", 1)])
def test_captured_step_replays_match_eager(name, group_parts):
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = make_case(name, "small")
    _say(f"[graph] {name} group_parts={group_parts}")
    dc = DeviceCase(case, group_parts=group_parts)
    o_ext = lse_ext = None
    if case.ext_regions is not None:
        e = oc.external_partial(case)
        o_ext = torch.from_numpy(e[0].astype(np.float32)).cuda()
        lse_ext = torch.from_numpy(e[1].astype(np.float32)).cuda()

    # eager references: the case's q, and the same queries in reverse sequence order
    q0 = dc.q.clone()
    q1 = dc.q.flip(0).contiguous()
    o, lse = dc.run(o_ext, lse_ext)
    torch.cuda.synchronize()
    ref0 = (o.clone(), lse.clone())
    dc.q.copy_(q1)
    o, lse = dc.run(o_ext, lse_ext)
    torch.cuda.synchronize()
    ref1 = (o.clone(), lse.clone())
    dc.q.copy_(q0)
    # the eager result is the oracle's
    o_ref, lse_ref = oc.full_reference(case)
    assert oc.out_error(case, ref0[0].cpu().numpy(), o_ref) <= oc.out_tol(case)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dc.run(o_ext, lse_ext)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dc.run(o_ext, lse_ext)
    torch.cuda.synchronize()

    for i, (q, ref) in enumerate([(q0, ref0), (q0, ref0), (q1, ref1), (q0, ref0), (q1, ref1)]):
        dc.step.o_out.fill_(float("nan"))      # eager work between replays
        dc.step.lse_out.fill_(float("nan"))
        dc.q.copy_(q)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.step.o_out, ref[0]), (name, i)
        assert torch.equal(dc.step.lse_out, ref[1]), (name, i)
    assert int(dc.step.err.item()) == 0
    del graph
