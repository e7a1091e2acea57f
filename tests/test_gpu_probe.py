"""GPU test of the gather probe (kvattn_gather_probe): the decode kernel's loads with no
arithmetic, returning the XOR of the 16-bit K/V elements it read for each (sequence, KV head).

The expected checksum comes from the oracle's reader of the block layout (oracle.gather_sequence,
which decodes bf16 exactly, so the bit patterns are recovered from its values). The probe must
match it bit for bit: every in-range element read once, none outside the range. This pins the
block-table resolution of the kernels' own access path, independently of the attention
arithmetic.
"""

import sys

import numpy as np
import pytest

import oracle
from synth import make_case, mla_case
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


def _bits(x):
    """bf16 bit patterns of exactly representable float64 values."""
    return (np.asarray(x, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _expected(case, seqs):
    lay = oc.layout_of(case)
    out = {}
    for b in seqs:
        lo = 0 if case.tok_begin is None else int(case.tok_begin[b])
        hi = int(case.ctx_lens[b])
        k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[b], lo, hi)
        for h in range(case.num_kv_heads):
            x = np.bitwise_xor.reduce(_bits(k[:, h, :]).ravel(), initial=np.uint16(0))
            if not case.latent:   # MLA: the value is part of the latent, read once
                x ^= np.bitwise_xor.reduce(_bits(v[:, h, :]).ravel(), initial=np.uint16(0))
            out[(b, h)] = int(x)
    return out


def _probe(case, group_parts):
    from paged_kv_cache_mla_amd.session import DeviceCase
    dc = DeviceCase(case, group_parts=group_parts)
    xsum = torch.zeros(case.batch * case.num_kv_heads, dtype=torch.int32, device="cuda")
    dc.step.probe(xsum)
    torch.cuda.synchronize()
    assert int(dc.step.err.item()) == 0
    return xsum.cpu().numpy().view(np.uint32).reshape(case.batch, case.num_kv_heads)


SMALL = [("gqa_32k", 1), ("gqa_32k", 3), ("gqa_32k", 16), ("split_128k", 4),
         ("prefix_shared", 2), ("prefix_shared", 7), ("mla_16k", 1), ("mla_16k", 3)]


@pytest.mark.parametrize("name,group_parts", SMALL, ids=[f"{n}-g{g}" for n, g in SMALL])
def test_probe_checksum_matches_oracle_reader(name, group_parts):
    case = make_case(name, "small")
    _say(f"[probe] {name} small group_parts={group_parts}")
    got = _probe(case, group_parts)
    want = _expected(case, range(case.batch))
    for (b, h), x in want.items():
        assert int(got[b, h]) == x, (b, h, hex(int(got[b, h])), hex(x))


def test_probe_checksum_mla_ragged_stage_counts():
    """MLA groups of 1 to 10 blocks starting inside blocks: the two teams' halves of each group
    are read exactly once between them."""
    lens = [1, 67, 191, 256, 300, 400, 448, 512, 542, 640]
    begin = [0, 3, 63, 10, 20, 100, 0, 0, 30, 0]
    case = mla_case(lens, [192] * len(lens), tok_begin=begin)
    got = _probe(case, 2)
    want = _expected(case, range(case.batch))
    for (b, h), x in want.items():
        assert int(got[b, h]) == x, (b, h)


@pytest.mark.parametrize("name,group_parts,seqs", [("gqa_32k", 16, [0, 15]), ("mla_16k", 4, [3])])
def test_probe_checksum_full_size(name, group_parts, seqs):
    """Full-size layers in the launch configuration bench.py times, sampled sequences."""
    case = make_case(name, "full")
    _say(f"[probe-full] {name} group_parts={group_parts}")
    got = _probe(case, group_parts)
    want = _expected(case, seqs)
    for (b, h), x in want.items():
        assert int(got[b, h]) == x, (b, h)
