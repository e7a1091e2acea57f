"""GPU parity of block-level sparse decode through the C ABI: kvattn_select_blocks builds the
sub-table on the device (compared bit for bit with the oracle's, flags included), and the
decode kernels run on it unchanged (compared with the oracle's masked attention, which never
builds a sub-table).  Tolerances as for dense decode."""

import sys

import numpy as np
import pytest

import oracle
from oracle.sparse import masked_reference, select_blocks
from synth import make_case
from tests import oracle_cases as oc

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


def _selection(rng, case, density, extras=True):
    bs = case.block_size
    nbs = [-(-int(L) // bs) for L in case.ctx_lens]
    k = max(1, max(int(np.ceil(n * density)) for n in nbs) + (3 if extras else 0))
    sel = np.full((case.batch, k), -1, np.int32)
    for b, n in enumerate(nbs):
        m = min(n, int(np.ceil(n * density)))
        if m:
            sel[b, :m] = rng.choice(n, m, replace=False)
        if extras and b == 0 and n:
            sel[b, -1] = sel[b, 0] if m else 0          # a repeat
            sel[b, -2] = n + 3                          # beyond the context
        rng.shuffle(sel[b])
    return sel


def _run_sparse(case, dc, sel, group_parts=1):
    from paged_kv_cache_mla_amd.api import decode_partial, merge_lse, select_blocks as sel_blocks
    B, bs, k = case.batch, case.block_size, sel.shape[1]
    dev = "cuda"
    sel_dev = torch.from_numpy(sel).to(dev)
    sub_table = torch.full((B, k), -9, dtype=torch.int32, device=dev)
    seq_sub = torch.zeros((3, B), dtype=torch.int32, device=dev)
    seq_sub[2] = torch.from_numpy(case.part_tokens.astype(np.int32)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    sel_blocks(dc.step.table_dev, case.max_blocks, dc.step.seq_dev[0], bs, sel_dev, sub_table,
               seq_sub[0], err)
    bound = np.full(B, k * bs, np.int32)
    counts = [-(-(k * bs) // int(p)) for p in case.part_tokens]
    max_parts = max(1, max(-(-c // group_parts) for c in counts))
    o_part = torch.empty((B, case.num_q_heads, max_parts, case.head_dim_v), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, case.num_q_heads, max_parts), dtype=torch.float32, device=dev)
    nparts = torch.empty(B, dtype=torch.int32, device=dev)
    o = torch.empty((B, case.num_q_heads, case.head_dim_v), dtype=torch.float32, device=dev)
    lse = torch.empty((B, case.num_q_heads), dtype=torch.float32, device=dev)
    decode_partial(dc.pool, dc.q, dc.q_dtype, case.num_q_heads, case.scale, sub_table, k, bound,
                   None, case.part_tokens, seq_sub, max_parts, o_part, lse_part, nparts, err, None,
                   group_parts)
    merge_lse(o_part, lse_part, nparts, B, case.num_q_heads, max_parts, case.head_dim_v, o, None,
              None, lse)
    torch.cuda.synchronize()
    return (sub_table.cpu().numpy(), seq_sub[0].cpu().numpy(), int(err.item()),
            o.cpu().numpy(), lse.cpu().numpy())


def _check(case, sel, sub_table, sub_len, err, o, lse, seqs):
    flags = 0
    for b in range(case.batch):
        row, slen, f = select_blocks(case.table[b], case.ctx_lens[b], case.block_size, sel[b],
                                     case.max_blocks)
        flags |= f
        exp = np.full(sel.shape[1], -1, np.int32)
        exp[:len(row)] = row
        assert np.array_equal(sub_table[b], exp), b
        assert sub_len[b] == slen, b
    assert err == flags
    for b in seqs:
        o_ref, lse_ref = masked_reference(oc.layout_of(case), case.regions, case.region_blocks,
                                          case.table[b], case.ctx_lens[b], sel[b],
                                          oc.q_f64(case)[b], case.scale)
        if np.all(np.isneginf(lse_ref)):
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        if case.dtype == "bf16":
            e = np.max(np.abs(o[b] - o_ref)) / np.max(np.abs(o_ref))
            assert e <= 2e-3, (b, e)
            assert np.max(np.abs(lse[b] - lse_ref)) <= 2e-3
        else:
            assert np.max(np.abs(o[b] - o_ref)) <= 1e-5
            assert np.max(np.abs(lse[b] - lse_ref)) <= 1e-5


@pytest.mark.parametrize("name,density", [("gqa_32k", 0.3), ("mla_16k", 0.25),
                                          ("tiny_fp32", 0.5), ("gqa_32k", 1.0)])
def test_sparse_selection_matches_oracle(name, density):
    from paged_kv_cache_mla_amd.session import DeviceCase
    _say(f"[sparse] {name} density {density}")
    case = make_case(name, "small")
    dc = DeviceCase(case)
    rng = np.random.default_rng(int(density * 100) + len(name))
    sel = _selection(rng, case, density)
    res = _run_sparse(case, dc, sel)
    _check(case, sel, *res, range(case.batch))


@pytest.mark.parametrize("name,density,group_parts,seqs", [
    ("gqa_32k", 1 / 8, 4, [0, 9]), ("mla_16k", 1 / 4, 2, [0, 31])])
def test_sparse_selection_full_size_sampled(name, density, group_parts, seqs):
    """Full-size layers at a fraction of their blocks, grouped (the 16 x 32K GQA layer at 1/8,
    the 32 x 16K MLA layer at 1/4)."""
    from paged_kv_cache_mla_amd.session import DeviceCase
    _say(f"[sparse] {name} full, density {density}")
    case = make_case(name, "full")
    dc = DeviceCase(case)
    rng = np.random.default_rng(8)
    sel = _selection(rng, case, density, extras=False)
    res = _run_sparse(case, dc, sel, group_parts=group_parts)
    _check(case, sel, *res, seqs)
