"""Oracle-side evaluation of synthetic workloads (test helper; calls only `oracle`)."""

import numpy as np

import oracle
from oracle.layout import gather_sequence

BF16_REL_TOL = 2e-3   # max |o_gpu - o_ref| / max |o_ref| for bf16 caches with fp32 accumulation
F32_ABS_TOL = 1e-5    # max |o_gpu - o_ref| for fp32 caches
LSE_ABS_TOL = 2e-3    # lse of bf16 caches (natural log); fp32 caches use F32_ABS_TOL


def layout_of(case):
    return oracle.Layout(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                         case.dtype, case.latent)


def q_f64(case):
    return (oracle.bf16_bits_to_f64(case.q) if case.dtype == "bf16"
            else case.q.astype(np.float64))


def full_reference(case, seqs=None):
    """Unsplit attention of each sequence over its whole context [0, L): the device share
    [tok_begin, L) and, for split workloads, the host-side share [0, tok_begin)."""
    lay = layout_of(case)
    if case.ext_regions is None:
        return oracle.decode_reference(lay, case.regions, case.region_blocks, case.table,
                                       case.ctx_lens, case.q, case.scale, tok_begin=case.tok_begin,
                                       seqs=seqs)
    qf = q_f64(case)
    o = np.zeros((case.batch, case.num_q_heads, case.head_dim_v))
    lse = np.full((case.batch, case.num_q_heads), -np.inf)
    for b in (range(case.batch) if seqs is None else seqs):
        beg, L = int(case.tok_begin[b]), int(case.ctx_lens[b])
        k1, v1 = gather_sequence(lay, case.ext_regions, case.ext_region_blocks, case.ext_table[b], 0, beg)
        k2, v2 = gather_sequence(lay, case.regions, case.region_blocks, case.table[b], beg, L)
        o[b], lse[b] = oracle.attend(qf[b], np.concatenate([k1, k2]), np.concatenate([v1, v2]), case.scale)
    return o, lse


def external_partial(case, seqs=None, seed=0):
    """The host-side share's partial (o, lse) over [0, tok_begin), from the oracle, for the
    sequences in `seqs`; other sequences get an arbitrary but valid random partial."""
    lay = layout_of(case)
    qf = q_f64(case)
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((case.batch, case.num_q_heads, case.head_dim_v)) * 0.05
    lse = rng.standard_normal((case.batch, case.num_q_heads)) + 5.0
    for b in (range(case.batch) if seqs is None else seqs):
        k, v = gather_sequence(lay, case.ext_regions, case.ext_region_blocks, case.ext_table[b],
                               0, int(case.tok_begin[b]))
        o[b], lse[b] = oracle.attend(qf[b], k, v, case.scale)
    return o, lse


def device_partials(case, seqs=None):
    lay = layout_of(case)
    return oracle.decode_partials_reference(lay, case.regions, case.region_blocks, case.table,
                                            case.ctx_lens, case.q, case.scale, case.part_tokens,
                                            tok_begin=case.tok_begin, seqs=seqs)


def out_error(case, o_gpu, o_ref):
    """The figure the tolerance applies to: relative-to-scale for bf16, absolute for fp32."""
    diff = float(np.max(np.abs(np.asarray(o_gpu, np.float64) - o_ref)))
    if case.dtype == "f32":
        return diff
    return diff / float(np.max(np.abs(o_ref)))


def out_tol(case):
    return F32_ABS_TOL if case.dtype == "f32" else BF16_REL_TOL


def lse_tol(case):
    return F32_ABS_TOL if case.dtype == "f32" else LSE_ABS_TOL


def grouped_partials(case, group_parts, seqs=None):
    """The partials a decode step writes when `group_parts` consecutive partitions are merged
    into one: the oracle's merge of each group's per-partition partials.  List over the
    sequences of (o [ngroups, Hq, Dv], lse [ngroups, Hq])."""
    out = []
    for po, pl in device_partials(case, seqs):
        n = po.shape[0]
        os_, ls_ = [], []
        for g0 in range(0, n, group_parts):
            o, l = oracle.merge(list(po[g0:g0 + group_parts]), list(pl[g0:g0 + group_parts]))
            os_.append(o)
            ls_.append(l)
        hq, dv = po.shape[1], po.shape[2]
        out.append((np.array(os_).reshape(len(os_), hq, dv), np.array(ls_).reshape(len(ls_), hq)))
    return out
