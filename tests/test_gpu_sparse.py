"""GPU parity of the block-sparse edge forward (pa_sparse_forward) and its merge against the CPU
oracle: tiny edge lists compared partial by partial, and the full-size workload (Tq 4096, hkv 8,
qhead 4, D 128, block 64, page 16) compared on every partial of a seeded sample of (q, h)
groups and on their merged rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_gqa_paged_amd as pa  # noqa: E402
import oracle  # noqa: E402
from block_sparse_gqa_paged_amd import device as dev  # noqa: E402
from block_sparse_gqa_paged_amd import workloads as W  # noqa: E402
from parity import assert_sparse_out_close, assert_sparse_partials_close  # noqa: E402

pytestmark = pytest.mark.gpu


def _tiny(seed, **kw):
    args = dict(Tq=24, hkv=2, qhead=4, head_dim=128, block_size=64, page_size=16, batch=2,
                key_capacity=512, window=2, p_random=0.3, unmapped_frac=0.15, name="tiny")
    args.update(kw)
    return W.sparse_workload(seed, **args)


TINY = [
    dict(seed=200),
    dict(seed=201, head_dim=64, block_size=32, page_size=8, qhead=2),
    dict(seed=202, qhead=1, hkv=3, block_size=16, page_size=16, unmapped_frac=0.0),
    dict(seed=203, qhead=8, block_size=128, page_size=32, head_dim=64, key_capacity=1024),
    dict(seed=204, qhead=3, block_size=48, page_size=16, key_capacity=480, all_blocks=True),
    # 128-key blocks at D = 128: the largest LDS footprint
    dict(seed=205, block_size=128, page_size=16, key_capacity=1024),
    # many edges per key block: several work items share one block
    dict(seed=206, Tq=600, hkv=1, qhead=2, key_capacity=256, window=3, p_random=0.5),
    # one edge per 16-row group
    dict(seed=207, qhead=16, hkv=1, head_dim=64, block_size=32, page_size=8),
]


@pytest.mark.parametrize("case", TINY, ids=lambda c: str(c["seed"]))
def test_tiny_partials_and_merge(case):
    case = dict(case)
    sw = _tiny(case.pop("seed"), **case)
    ref = oracle.sparse_forward(sw)
    c = dev.SparseCase(sw)
    got = c.forward()
    out = c.combine()
    torch.cuda.synchronize()
    assert_sparse_partials_close(got, ref, "partials")
    merged = oracle.split_combine(*ref, lanes=sw["qhead"], head_dim=sw["D"],
                                  group_ptr=sw["group_ptr"], out_dtype=np.float32)
    assert_sparse_out_close(out, merged, "merged")


@pytest.mark.parametrize("case", TINY[:4] + TINY[5:], ids=lambda c: str(c["seed"]))
def test_tiny_causal_partials_and_merge(case):
    """Right-aligned causal mask: partials and merged rows against the oracle with q_pos."""
    case = dict(case)
    sw = _tiny(case.pop("seed"), **case)
    ref = oracle.sparse_forward(sw, q_pos=sw["q_pos"])
    c = dev.SparseCase(sw)
    got = c.forward(causal=True)
    out = c.combine()
    torch.cuda.synchronize()
    assert_sparse_partials_close(got, ref, "causal partials")
    merged = oracle.split_combine(*ref, lanes=sw["qhead"], head_dim=sw["D"],
                                  group_ptr=sw["group_ptr"], out_dtype=np.float32)
    assert_sparse_out_close(out, merged, "causal merged")


def test_sentinels_and_out_of_range_edges():
    sw = _tiny(210)
    em = sw["edge_meta"].copy()
    em[0, 4] = 0                       # empty block
    em[1, 4] = -5
    bt = sw["block_tables"].copy()
    b, blk = em[2, 3], em[2, 2]
    bt[b, blk * 4:(blk + 1) * 4] = -1  # every page of edge 2's block unmapped
    sw = dict(sw, edge_meta=em, block_tables=bt)
    ref = oracle.sparse_forward(sw)
    c = dev.SparseCase(sw)
    o, m, l = c.forward()
    torch.cuda.synchronize()
    assert_sparse_partials_close((o, m, l), ref)
    for e in (0, 1, 2):
        p = slice(4 * e, 4 * e + 4)
        assert np.all(m[p].cpu().numpy() == np.float32(-1e30))
        assert np.all(l[p].cpu().numpy() == 0) and np.all(o[p].cpu().numpy() == 0)


def test_edge_order_does_not_change_results():
    sw = _tiny(211)
    c = dev.SparseCase(sw)
    a = [x.cpu().numpy().copy() for x in c.forward()]
    perm = np.random.default_rng(2).permutation(sw["E"])
    sw2 = dict(sw, edge_meta=sw["edge_meta"][perm])
    c2 = dev.SparseCase(sw2)
    b = [x.cpu().numpy() for x in c2.forward()]
    q = sw["qhead"]
    rows = (perm[:, None] * q + np.arange(q)[None, :]).reshape(-1)
    for x, y in zip(a, b):
        assert np.array_equal(x[rows], y)


@pytest.fixture(scope="module")
def full():
    sw = W.block_sparse_forward()
    c = dev.SparseCase(sw)
    o, m, l = c.forward()
    out = c.combine()
    torch.cuda.synchronize()
    return sw, o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), out.cpu().numpy()


def _check_sampled_groups(sw, o, m, l, out, q_pos=None):
    G = sw["Tq"] * sw["hkv"]
    groups = np.random.default_rng(7).choice(G, size=96, replace=False)
    groups.sort()
    gp = sw["group_ptr"]
    edges = np.concatenate([np.arange(gp[g], gp[g + 1]) for g in groups])
    sub_gp = np.concatenate([[0], np.cumsum(gp[groups + 1] - gp[groups])]).astype(np.int32)
    ro, rm, rl = oracle.sparse_forward(sw, edge_meta=sw["edge_meta"][edges], q_pos=q_pos)
    q = sw["qhead"]
    prow = (edges[:, None] * q + np.arange(q)[None, :]).reshape(-1)
    assert_sparse_partials_close((o[prow], m[prow], l[prow]), (ro, rm, rl), "sampled partials")
    merged = oracle.split_combine(ro, rm, rl, lanes=q, head_dim=sw["D"], group_ptr=sub_gp,
                                  out_dtype=np.float32)
    orow = (groups[:, None] * q + np.arange(q)[None, :]).reshape(-1)
    assert_sparse_out_close(out[orow], merged, "sampled merged rows")


def test_full_size_sampled_groups(full):
    _check_sampled_groups(*full)


def test_full_size_causal_sampled_groups(full):
    """The same workload under the right-aligned causal mask (its random blocks past a row's
    position become sentinels, the row's own block is cut at the position)."""
    sw = full[0]
    c = dev.SparseCase(sw)
    o, m, l = c.forward(causal=True)
    out = c.combine()
    torch.cuda.synchronize()
    _check_sampled_groups(sw, o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(),
                          out.cpu().numpy(), q_pos=sw["q_pos"])


def test_full_size_invariants(full):
    sw, o, m, l, out = full
    assert np.isfinite(out).all() and np.isfinite(o).all()
    # every mapped edge has l >= 1 (its max key contributes exp(0)); unmapped blocks l == 0
    assert (l >= 0).all()
    pos = l > 0
    assert (l[pos] >= 1.0 - 1e-6).all()
    assert np.all(m[~pos] == np.float32(-1e30))
