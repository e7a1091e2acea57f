"""kvattn_decode_partial_plan_noalloc (through the C ABI) against kvattn_decode_partial_plan with
a caller-owned work_dev: the same plan kernel with its work counters in the library's per-GPU
array.  Two calls in a row, the second with a smaller input (fewer sequences, another plan);
each must equal the workspace call bit for bit (partials, counts and merged output) and the
merged output must match the float64 oracle within the bf16 tolerance."""

import copy

import numpy as np
import pytest

from synth import make_case
from tests import oracle_cases as oc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU-only hosts)")
    from paged_kv_cache_mla_amd import _lib
    _lib.load()
    torch.cuda.set_device(0)


def _sub_batch(case, n):
    c = copy.copy(case)
    c.table = case.table[:n].copy()
    c.ctx_lens = case.ctx_lens[:n].copy()
    c.part_tokens = case.part_tokens[:n].copy()
    c.q = case.q[:n].copy()
    return c


def _both(case):
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import decode_partial_plan_noalloc, merge_lse
    from paged_kv_cache_mla_amd.session import DeviceCase
    dc = DeviceCase(case, plan=True, claim=True)       # the workspace entry point
    o_ws, l_ws = (t.clone() for t in dc.run())
    p_ws = (dc.step.o_part.clone(), dc.step.lse_part.clone(), dc.step.nparts.clone())
    st = dc.step
    st.o_part.fill_(float("nan"))
    st.lse_part.fill_(float("nan"))
    st.nparts.fill_(-1)
    decode_partial_plan_noalloc(dc.pool, dc.q, dc.q_dtype, case.num_q_heads, case.scale,
                                st.table_dev, st.max_blocks, st.plan_dev, st.n_groups,
                                st.max_parts, st.o_part, st.lse_part, st.nparts, st.err)
    o = torch.empty_like(o_ws)
    lse = torch.empty_like(l_ws)
    merge_lse(st.o_part, st.lse_part, st.nparts, case.batch, case.num_q_heads, st.max_parts,
              case.head_dim_v, o, None, None, lse)
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0
    assert torch.equal(st.nparts, p_ws[2])
    for b in range(case.batch):                       # the slots each sequence owns
        n = int(p_ws[2][b])
        assert torch.equal(st.o_part[b, :, :n], p_ws[0][b, :, :n])
        assert torch.equal(st.lse_part[b, :, :n], p_ws[1][b, :, :n])
    assert torch.equal(o, o_ws) and torch.equal(lse, l_ws)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o.cpu().numpy(), o_ref)
    print(f"[no-alloc] batch {case.batch}: out error {err:.3e}", flush=True)
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse.cpu().numpy() - lse_ref))) <= oc.lse_tol(case)


def test_no_alloc_plan_decode_equals_the_workspace_call_twice():
    case = make_case("prefix_shared", "small")
    _both(case)                       # 16 sequences
    _both(_sub_batch(case, 8))        # then a smaller input: one group, another plan
    _both(case)                       # and the first again: the counters were left at zero
